"""GPU test of kda_chunk_fwd_noalloc, the prefill entry point whose workspace
is the library's fixed device array instead of a caller's buffer.

Each call is checked against kda_chunk_fwd on the same inputs (outputs, final
states and, with the prologue, the convolution state): the two run the same
kernels on the same data, so they must agree bit for bit.  Calls follow one
another on one device, largest first, so every call after the first runs on
an array that still holds the previous call's workspace: packed sequences over
128 (sequence, head) pairs at bf16 (pair mode: the chain inside the
intra-chunk kernel, the array holding only the chunk table), then a smaller
batched call with the layer prologue and epilogue fused (split design, its
convolution state written by the intra-chunk stage), then a smaller float32
call that runs on the blocks the second call left.  A shape beyond the array is rejected and leaves the
output untouched."""
import dataclasses

import numpy as np
import pytest
import torch

import workloads as W
from kda_testutil import gpu_prefill

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gated_delta_rule_20_amd as kda
    kda.load_library()


def _same(name, got, ref):
    assert got.shape == ref.shape and got.dtype == ref.dtype, name
    bad = (got.view(torch.uint8) != ref.view(torch.uint8)).sum().item() if got.numel() else 0
    assert bad == 0, f"{name}: {bad} bytes differ from kda_chunk_fwd"


def _noalloc(inp, out, final_state, **kw):
    import gated_delta_rule_20_amd as kda
    return kda.chunk_fwd_noalloc(inp["q"], inp["k"], inp["v"], inp["z"], inp["beta"], out=out,
                                 final_state=final_state, A_log=inp["A_log"], g_min=inp["g_min"],
                                 cu_seqlens=inp.get("cu_seqlens"), initial_state=inp.get("h0"), **kw)


def _packed_128_pairs():
    w = dataclasses.replace(W.WORKLOADS["varlen_64"], seed=90)
    gen = torch.Generator().manual_seed(91)
    lens = torch.randint(0, 300, (64,), generator=gen)
    lens[:4] = torch.tensor([0, 1, 64, 65])
    return W.make_prefill(w, "cuda", H=2, lengths=lens)


def _check_pair(inp, **kw):
    import gated_delta_rule_20_amd as kda
    need = kda.chunk_fwd_workspace_size(inp["q"], inp["v"], cu_seqlens=inp.get("cu_seqlens"),
                                        N=None if inp.get("cu_seqlens") is None else inp["cu_seqlens"].numel() - 1)
    assert 0 < need <= kda.NOALLOC_WORKSPACE_BYTES
    o_ref, h_ref = gpu_prefill(inp, **kw)
    o = torch.full_like(o_ref, float("nan"))
    h = torch.full_like(h_ref, float("nan"))
    _noalloc(inp, o, h, **kw)
    torch.cuda.synchronize()
    _same("o", o, o_ref)
    _same("final_state", h, h_ref)
    return need


def test_noalloc_matches_chunk_fwd_on_calls_in_a_row():
    import gated_delta_rule_20_amd as kda
    # 1: packed sequences, 64 sequences x 2 heads (lengths 0..299, a chunk
    #    boundary and a one-token sequence among them).
    inp1 = _packed_128_pairs()
    print("noalloc call 1: packed, 64 sequences x 2 heads, bf16 128/128", flush=True)
    need1 = _check_pair(inp1)

    # 2: smaller, batched, with the layer prologue (width-4 convolution) and
    #    epilogue fused.
    w = dataclasses.replace(W.WORKLOADS["prefill_8k"], seed=92)
    d = W.make_layer(w, "cuda", N=2, T=150, H=3, conv_width=4)
    need2 = kda.chunk_fwd_workspace_size(d["q_pre"], d["v_pre"], prologue=True)
    assert 0 < need2 <= kda.NOALLOC_WORKSPACE_BYTES
    assert d["q_pre"].numel() < inp1["q"].numel()  # a smaller input than call 1
    print("noalloc call 2: batched B=2 T=150 H=3 with prologue + epilogue", flush=True)
    outs = []
    for noalloc in (False, True):
        cs_out = torch.full_like(d["conv_state"], float("nan"))
        fus = kda.Fusion(conv_weight=d["conv_weight"], conv_state=d["conv_state"], conv_state_out=cs_out,
                         qk_eps=1e-6, gate=d["gate"], o_norm_weight=d["o_norm_weight"], o_eps=1e-6)
        o = torch.full_like(d["v_pre"], float("nan"))
        h = torch.full_like(d["state"], float("nan"))
        args = (d["q_pre"], d["k_pre"], d["v_pre"], d["z"], d["beta_logit"])
        kw = dict(A_log=d["A_log"], g_min=d["g_min"], initial_state=d["state"], fusion=fus)
        if noalloc:
            kda.chunk_fwd_noalloc(*args, out=o, final_state=h, **kw)
        else:
            kda.chunk_fwd(*args, out=o, final_state=h, **kw)
        outs.append((o, h, cs_out))
    torch.cuda.synchronize()
    for name, ref, got in zip(("y", "final_state", "conv_state_out"), outs[0], outs[1]):
        _same(name, got, ref)

    # 3: smaller still, float32 inputs, Dk = Dv = 64.
    inp3 = W.make_prefill(dataclasses.replace(W.WORKLOADS["tiny_fp32"], seed=93), "cuda", T=130)
    print("noalloc call 3: float32 64/64", flush=True)
    assert inp3["q"].numel() < d["q_pre"].numel()
    _check_pair(inp3)


def test_noalloc_rejects_shapes_beyond_its_array():
    import gated_delta_rule_20_amd as kda
    inp = W.make_prefill(dataclasses.replace(W.WORKLOADS["prefill_8k"], seed=94), "cuda", T=7232, H=8)
    assert kda.chunk_fwd_workspace_size(inp["q"], inp["v"]) > kda.NOALLOC_WORKSPACE_BYTES
    o = torch.full(inp["v"].shape, 7.0, dtype=inp["v"].dtype, device="cuda")
    with pytest.raises(kda.KDAError) as e:
        _noalloc(inp, o, None)
    assert e.value.status == 3 and "at most" in str(e.value)
    torch.cuda.synchronize()
    assert bool((o == 7.0).all())
    # the largest dense bf16 call at H = 8 that fits: 112 chunks of 64 tokens
    inp = W.make_prefill(dataclasses.replace(W.WORKLOADS["prefill_8k"], seed=95), "cuda", T=7168, H=8)
    print("noalloc: largest fitting call, B=1 T=7168 H=8", flush=True)
    _check_pair(inp)
