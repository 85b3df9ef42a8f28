"""GPU parity of the prefix-state checkpoints ("Kimi K3 Technical Report",
§5.4.1, KDA-aware prefix cache: the recurrent state is persisted at
hash-block-aligned positions and a later request resumes from it).

Slot j of sequence s must hold the state after the first (j + 1) * every * 64
tokens of s.  Its reference is the fp64 oracle's final state over exactly
that prefix (eq. (1) run token by token); resuming from a slot must reproduce
the one-pass outputs of the remaining tokens."""
import numpy as np
import pytest
import torch

import workloads as W
from kda_testutil import TOL, gpu_prefill, np64, oracle_prefill, rel_err

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gated_delta_rule_20_amd as kda
    kda.load_library()


def _prefix_state(inp, s, ntok):
    """Oracle state of packed sequence s after its first ntok tokens."""
    cu = inp["cu_seqlens"].to("cpu", torch.int64)
    t0 = int(cu[s])
    sub = {k: v for k, v in inp.items()}
    for key in ("q", "k", "v", "z", "beta"):
        sub[key] = inp[key][t0:t0 + ntok]
    sub["cu_seqlens"] = torch.tensor([0, ntok], dtype=torch.int32, device=inp["q"].device)
    sub["h0"] = None if inp.get("h0") is None else inp["h0"][s:s + 1]
    _, hT, _ = oracle_prefill(sub)
    return hT[0]


def _packed(w, lengths, H, seed):
    import dataclasses
    w = dataclasses.replace(w, seed=seed)
    return W.make_prefill(w, device="cuda", H=H, lengths=lengths)


def _run_with_checkpoints(inp, every, slots):
    N = inp["cu_seqlens"].numel() - 1 if inp.get("cu_seqlens") is not None else inp["q"].shape[0]
    H, Dk = inp["q"].shape[-2:]
    Dv = inp["v"].shape[-1]
    ck = torch.full((N, slots, H, Dk, Dv), float("nan"), device="cuda")
    o, hT = gpu_prefill(inp, checkpoints=ck, checkpoint_every=every)
    torch.cuda.synchronize()
    return o, hT, ck


def _check_slots(inp, ck, every, lengths):
    tol = TOL[inp["q"].dtype]
    worst = 0.0
    for s, L in enumerate(lengths):
        for j in range(ck.shape[1]):
            pos = (j + 1) * every * 64
            got = ck[s, j]
            if pos < L:
                e = rel_err(np64(got), _prefix_state(inp, s, pos))
                worst = max(worst, e)
                assert e <= tol, (s, j, e)
            else:
                assert torch.isnan(got).all(), (s, j)  # slot past the sequence is not written
    print(f"worst checkpoint rel err {worst:.3e}")


def test_checkpoints_fp32_every_chunk():
    """Tiny fp32 workload (one 256-token sequence): slots after 64, 128 and 192
    tokens; the fourth slot (256 = the end) is not written."""
    w = W.WORKLOADS["tiny_fp32"]
    inp = _packed(w, [256], H=2, seed=0)
    o, hT, ck = _run_with_checkpoints(inp, every=1, slots=4)
    _check_slots(inp, ck, 1, [256])


def test_checkpoints_packed_bf16():
    """Packed bf16 sequences of ragged lengths, a checkpoint every 2 chunks
    (128 tokens); the 64-token sequence has none, capacity cuts the longest."""
    lengths = [700, 64, 1100, 129]
    inp = _packed(W.WORKLOADS["varlen_64"], lengths, H=3, seed=31)
    o, hT, ck = _run_with_checkpoints(inp, every=2, slots=6)
    _check_slots(inp, ck, 2, lengths)


def test_checkpoints_leave_outputs_unchanged():
    lengths = [300, 900]
    inp = _packed(W.WORKLOADS["varlen_64"], lengths, H=2, seed=32)
    o1, h1 = gpu_prefill(inp)
    o2, h2, _ = _run_with_checkpoints(inp, every=1, slots=16)
    assert torch.equal(o1, o2) and torch.equal(h1, h2)


def test_resume_from_checkpoint():
    """Resuming the second part of a sequence from its 512-token checkpoint
    reproduces the one-pass outputs and final state."""
    import gated_delta_rule_20_amd as kda
    L = 1000
    inp = _packed(W.WORKLOADS["varlen_64"], [L], H=4, seed=33)
    o, hT, ck = _run_with_checkpoints(inp, every=8, slots=1)  # state after 512 tokens
    rest = {key: inp[key][512:].contiguous() for key in ("q", "k", "v", "z", "beta")}
    cu = torch.tensor([0, L - 512], dtype=torch.int32, device="cuda")
    o2, h2 = kda.chunk_fwd(rest["q"], rest["k"], rest["v"], rest["z"], rest["beta"], A_log=inp["A_log"],
                           g_min=inp["g_min"], cu_seqlens=cu, initial_state=ck[:, 0].contiguous())
    torch.cuda.synchronize()
    tol = TOL[torch.bfloat16]
    assert rel_err(np64(o2), np64(o[512:])) <= tol
    assert rel_err(np64(h2), np64(hT)) <= tol


def test_checkpoints_prefill_8k_sampled_heads():
    """prefill_8k at full size with a checkpoint every 8 chunks (512 tokens), the
    configuration the benchmark times: outputs and final state bit-identical to the
    call without checkpoints; slots 0, 7 and 14 (after 512, 4096 and 7680 tokens) of
    three heads against the oracle over that prefix; slot 15 (the sequence end) not
    written."""
    inp = W.make_prefill(W.WORKLOADS["prefill_8k"], device="cuda")
    o1, h1 = gpu_prefill(inp)
    o2, h2, ck = _run_with_checkpoints(inp, every=8, slots=16)
    assert torch.equal(o1, o2) and torch.equal(h1, h2)
    assert torch.isnan(ck[:, 15]).all()
    heads = [0, 17, 31]
    tol = TOL[inp["q"].dtype]
    for j in (0, 7, 14):
        pos = (j + 1) * 8 * 64
        sub = dict(inp)
        for key in ("q", "k", "v", "z", "beta"):
            sub[key] = inp[key][:, :pos]
        _, ref, _ = oracle_prefill(sub, heads=heads, nthreads=16)
        e = rel_err(np64(ck[:, j][:, heads]), ref)
        print(f"slot {j} (after {pos} tokens): rel err {e:.3e}")
        assert e <= tol, (j, e)


def test_checkpoint_shape_rejected():
    inp = _packed(W.WORKLOADS["varlen_64"], [200, 100], H=2, seed=34)
    bad = torch.zeros((2, 2, 3, 128, 128), device="cuda")  # H = 3, inputs have 2
    with pytest.raises(ValueError, match="checkpoints must be"):
        gpu_prefill(inp, checkpoints=bad, checkpoint_every=1)
    with pytest.raises(ValueError, match="checkpoints must be"):
        gpu_prefill(inp, checkpoints=bad[:, :, :2].contiguous(), checkpoint_every=0)
