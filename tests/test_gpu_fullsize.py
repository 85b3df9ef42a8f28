"""Parity at the workloads' full sizes, in the launch configuration the
benchmark times.  The oracle recomputes selected (sequence, head) pairs in
full: every output token and the final state of each selected pair."""
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


def _compare(inp, heads=None, seqs=None):
    o, hT = gpu_prefill(inp)
    torch.cuda.synchronize()
    ro, rh, tok = oracle_prefill(inp, heads=heads, seqs=seqs, nthreads=16)
    hs = slice(None) if heads is None else list(heads)
    go = o.reshape((-1,) + tuple(o.shape[-2:])) if o.dim() == 4 else o
    go = np64(go.index_select(0, tok.to(go.device))[:, hs])
    s_idx = list(range(hT.shape[0])) if seqs is None else list(seqs)
    gs = np64(hT[s_idx][:, hs])
    e_o, e_s = rel_err(go, ro), rel_err(gs, rh)
    print(f"rel err o={e_o:.3e} state={e_s:.3e}")
    tol = TOL[inp["q"].dtype]
    assert e_o <= tol and e_s <= tol, (e_o, e_s)
    return o, hT


def test_prefill_8k_all_heads():
    """B=1, T=8192, H=32, d=128: every head against the oracle."""
    inp = W.make_prefill(W.WORKLOADS["prefill_8k"], device="cuda")
    _compare(inp)


def test_prefill_128k_sampled_heads():
    """T=131072 with forced hard-forgetting / near-unit channels: two heads,
    chosen to include forced channels of both kinds, recomputed in full."""
    w = W.WORKLOADS["prefill_128k"]
    inp = W.make_prefill(w, device="cuda")
    hard, soft = inp["forced"]
    heads = sorted({int(hard[0]) // w.Dk, int(soft[0]) // w.Dk})
    _compare(inp, heads=heads)


def test_varlen_64_sampled_sequences():
    """64 packed sequences (~530K tokens): the two longest, the shortest and
    one more sequence, on two heads."""
    w = W.WORKLOADS["varlen_64"]
    inp = W.make_prefill(w, device="cuda")
    lens = (inp["cu_seqlens"][1:] - inp["cu_seqlens"][:-1]).cpu().numpy()
    order = np.argsort(-lens, kind="stable")
    seqs = sorted({int(order[0]), int(order[1]), int(order[-1]), 17})
    print("tokens", int(lens.sum()), "selected lengths", [int(lens[s]) for s in seqs])
    _compare(inp, heads=[0, 31], seqs=seqs)


def test_decode_512_sampled_pairs_all_steps():
    """512 x 32 heads, 64 steps with fresh inputs, state updated in place:
    8 sequences x 32 heads followed through all 64 steps (outputs of every
    step and the state after step 1 and step 64)."""
    import gated_delta_rule_20_amd as kda
    import oracle
    w = W.WORKLOADS["decode_512"]
    d = W.make_decode(w, device="cuda")
    seqs = [0, 1, 77, 200, 255, 256, 400, 511]
    S = np64(d["state"][seqs])
    A = np64(d["A_log"])
    state = d["state"]
    cu = np.arange(len(seqs) + 1, dtype=np.int64)
    worst = 0.0
    for i, st in enumerate(d["steps"]):
        o = kda.recurrent_step(st["q"], st["k"], st["v"], st["z"], st["beta"], state, A_log=d["A_log"])
        sel = lambda x: np64(x[seqs])
        ro, S = oracle.forward(sel(st["q"]), sel(st["k"]), sel(st["v"]), sel(st["z"]), sel(st["beta"]),
                               cu_seqlens=cu, h0=S, A_log=A)
        torch.cuda.synchronize()
        worst = max(worst, rel_err(np64(o[seqs]), ro))
        if i in (0, len(d["steps"]) - 1):
            e_s = rel_err(np64(state[seqs]), S)
            print(f"step {i}: state rel err {e_s:.3e}")
            assert e_s <= TOL[torch.bfloat16]
    print(f"worst per-step o rel err {worst:.3e}")
    assert worst <= TOL[torch.bfloat16]
