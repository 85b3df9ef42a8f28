"""Parity at the workloads' full sizes, in the launch configuration the
benchmark times.  Every output element and every final state of each
configuration is compared with the oracle; the comparison is streamed over
groups of heads (or steps) with running maxima, so no fp64 copy of a whole
configuration is held, and the measure is the whole-tensor
max|gpu - oracle| / max|oracle|."""
import numpy as np
import pytest
import torch

import workloads as W
from kda_testutil import TOL, RunningErr, gpu_prefill, host64, np64, oracle_prefill, rel_err, \
    stream_prefill_parity

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


def test_prefill_128k_all_heads():
    """T=131072 with forced hard-forgetting / near-unit channels: every head
    and every token against the oracle, streamed four heads at a time."""
    w = W.WORKLOADS["prefill_128k"]
    inp = W.make_prefill(w, device="cuda")
    o, hT = gpu_prefill(inp)
    torch.cuda.synchronize()
    e_o, e_s = stream_prefill_parity(inp, o, hT, heads_per_call=8)
    print(f"prefill_128k whole-tensor rel err o={e_o:.3e} state={e_s:.3e}")
    assert e_o <= TOL[torch.bfloat16] and e_s <= TOL[torch.bfloat16], (e_o, e_s)


def test_varlen_64_all_sequences_all_heads():
    """64 packed sequences (530,033 tokens), every sequence on every head
    against the oracle, streamed two heads at a time."""
    w = W.WORKLOADS["varlen_64"]
    inp = W.make_prefill(w, device="cuda")
    print("tokens", W.n_tokens(inp), "sequences", inp["cu_seqlens"].numel() - 1, flush=True)
    o, hT = gpu_prefill(inp)
    torch.cuda.synchronize()
    e_o, e_s = stream_prefill_parity(inp, o, hT, heads_per_call=2)
    print(f"varlen_64 whole-tensor rel err o={e_o:.3e} state={e_s:.3e}")
    assert e_o <= TOL[torch.bfloat16] and e_s <= TOL[torch.bfloat16], (e_o, e_s)


def test_decode_512_all_pairs_all_steps():
    """512 x 32 heads, 64 steps with fresh inputs, state updated in place:
    every sequence and head through all 64 steps (outputs of every step, the
    whole state after step 1 and after step 64)."""
    import gated_delta_rule_20_amd as kda
    import oracle
    w = W.WORKLOADS["decode_512"]
    d = W.make_decode(w, device="cuda")
    S = host64(d["state"])
    A = np64(d["A_log"])
    state = d["state"]
    N = state.shape[0]
    cu = np.arange(N + 1, dtype=np.int64)
    eo = RunningErr()
    for i, st in enumerate(d["steps"]):
        o = kda.recurrent_step(st["q"], st["k"], st["v"], st["z"], st["beta"], state, A_log=d["A_log"])
        ro, S = oracle.forward(*(host64(st[x]) for x in ("q", "k", "v", "z", "beta")),
                               cu_seqlens=cu, h0=S, A_log=A, nthreads=16)
        torch.cuda.synchronize()
        eo.add(host64(o), ro)
        if i in (0, len(d["steps"]) - 1):
            es = RunningErr()
            es.add(host64(state), S)
            print(f"step {i}: whole-state rel err {es.rel:.3e}", flush=True)
            assert es.rel <= TOL[torch.bfloat16]
        if i % 16 == 15:
            print(f"step {i}: running o rel err {eo.rel:.3e}", flush=True)
    print(f"decode_512 all steps o rel err {eo.rel:.3e}")
    assert eo.rel <= TOL[torch.bfloat16]
