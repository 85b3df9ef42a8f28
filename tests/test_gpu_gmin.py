"""GPU parity at lower bounds g_min other than the pages' -5 (the gate of
eq. (5) scales with it, and in log-decay mode the kernels clamp g into
[g_min, 0]): prefill on the split design and in pair mode (with a query
scale), fp32 and bf16, and decode steps, each against the fp64 oracle."""
import dataclasses

import numpy as np
import pytest
import torch

import workloads as W
from kda_testutil import TOL, gpu_prefill, host64, np64, oracle_prefill, rel_err

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gated_delta_rule_20_amd as kda
    kda.load_library()


def _check(inp, z_mode=True, oracle_inp=None):
    dt = inp["q"].dtype
    o, hT = gpu_prefill(inp, z_mode=z_mode)
    torch.cuda.synchronize()
    ro, rh, _ = oracle_prefill(oracle_inp or inp, z_mode=z_mode)
    go = np64(o)
    if inp.get("cu_seqlens") is None:
        go = go.reshape((-1,) + go.shape[2:])
    e_o, e_s = rel_err(go, ro), rel_err(np64(hT), rh)
    print(f"g_min={inp['g_min']} rel err o={e_o:.3e} state={e_s:.3e}")
    assert e_o <= TOL[dt] and e_s <= TOL[dt], (e_o, e_s)


@pytest.mark.parametrize("g_min", [-1.5, -0.25])
def test_prefill_split_zmode(g_min):
    """4 (sequence, head) pairs, bf16, d = 128: intra-chunk and chain kernels."""
    w = dataclasses.replace(W.WORKLOADS["prefill_8k"], seed=50)
    inp = W.make_prefill(w, "cuda", T=300, H=4)
    inp["g_min"] = g_min
    _check(inp)


def test_prefill_fp32_zmode():
    w = dataclasses.replace(W.WORKLOADS["tiny_fp32"], zero_h0=False, A_uniform=1.0, seed=51)
    inp = W.make_prefill(w, "cuda", T=200, H=2)
    inp["g_min"] = -3.0
    _check(inp)


def test_prefill_pair_mode_zmode_with_scale():
    """64 packed sequences x 2 heads = 128 pairs (pair mode), g_min = -2, query scale 1/8."""
    w = dataclasses.replace(W.WORKLOADS["varlen_64"], seed=52)
    lens = torch.randint(0, 200, (64,), generator=torch.Generator().manual_seed(52))
    lens[:3] = torch.tensor([0, 1, 65])
    inp = W.make_prefill(w, "cuda", H=2, lengths=lens)
    inp["g_min"] = -2.0
    inp["scale"] = 0.125
    _check(inp)


def test_prefill_logdecay_clamped_into_range():
    """Log-decays drawn from U(-3, 0.5) with g_min = -2: the kernels clamp them
    into [-2, 0] (the documented handling of out-of-range g), so the oracle is
    given the clamped values."""
    w = dataclasses.replace(W.WORKLOADS["prefill_8k"], seed=53)
    inp = W.make_prefill(w, "cuda", T=260, H=3)
    gen = torch.Generator(device="cuda").manual_seed(53)
    inp["z"] = (torch.rand(inp["z"].shape, generator=gen, device="cuda") * 3.5 - 3.0).to(inp["q"].dtype)
    inp["g_min"] = -2.0
    ref = dict(inp)
    ref["z"] = inp["z"].float().clamp(-2.0, 0.0).to(inp["q"].dtype)  # exact: both ends are bf16 values
    _check(inp, z_mode=False, oracle_inp=ref)


def test_decode_steps_gmin():
    """8 sequences x 4 heads, four decode steps at g_min = -0.7, state in place."""
    import gated_delta_rule_20_amd as kda
    import oracle
    w = dataclasses.replace(W.WORKLOADS["decode_512"], seed=54)
    d = W.make_decode(w, device="cuda", N=8, H=4, steps=4)
    g_min = -0.7
    state = d["state"].clone()
    S = host64(d["state"])
    cu = np.arange(9, dtype=np.int64)
    for i, st in enumerate(d["steps"]):
        o = kda.recurrent_step(st["q"], st["k"], st["v"], st["z"], st["beta"], state, A_log=d["A_log"], g_min=g_min)
        ro, S = oracle.forward(*(host64(st[x]) for x in ("q", "k", "v", "z", "beta")), cu_seqlens=cu, h0=S,
                               A_log=np64(d["A_log"]), g_min=g_min)
        torch.cuda.synchronize()
        e_o = rel_err(host64(o), ro)
        print(f"step {i}: rel err o={e_o:.3e}")
        assert e_o <= TOL[torch.bfloat16]
    e_s = rel_err(host64(state), S)
    print(f"state after 4 steps: rel err {e_s:.3e}")
    assert e_s <= TOL[torch.bfloat16]
