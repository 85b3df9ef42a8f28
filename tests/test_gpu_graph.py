"""GPU tests of the entry points under HIP graph capture, for callers that
record their serving loop once and replay it (the audience of
kda_chunk_fwd_noalloc: no allocation inside the captured region).

The library enqueues only kernels (no memset or copy nodes), so a captured
call is a plain kernel graph.  Each test captures one call on static buffers,
then replays it several times with fresh inputs copied in eagerly between the
replays, and checks every replay bit for bit against an eager call of the
same entry point on the same inputs (the eager calls are the program's own
work between replays)."""
import dataclasses

import pytest
import torch

import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gated_delta_rule_20_amd as kda
    kda.load_library()


def _same(name, got, ref):
    assert got.shape == ref.shape and got.dtype == ref.dtype, name
    bad = (got.contiguous().view(torch.uint8) != ref.contiguous().view(torch.uint8)).sum().item()
    assert bad == 0, f"{name}: {bad} bytes differ from the eager call"


def _capture(fn):
    """Run fn once eagerly on a side stream (first-call set-up), then capture it."""
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def _inputs(kind, seed):
    if kind == "batch":  # 4 (sequence, head) pairs: intra-chunk + chain kernels, blocks in the fixed array
        w = dataclasses.replace(W.WORKLOADS["prefill_8k"], seed=seed)
        return W.make_prefill(w, "cuda", T=1000, H=4)
    # packed sequences over 128 pairs: pair mode, the chunk table in the fixed array
    # (the same lengths for every seed: the captured call's shapes are fixed)
    w = dataclasses.replace(W.WORKLOADS["varlen_64"], seed=seed)
    gen = torch.Generator().manual_seed(299)
    lens = torch.randint(0, 200, (64,), generator=gen)
    lens[:3] = torch.tensor([0, 1, 65])
    return W.make_prefill(w, "cuda", H=2, lengths=lens)


@pytest.mark.parametrize("kind", ["batch", "packed"])
def test_prefill_noalloc_graph_replays(kind):
    """kda_chunk_fwd_noalloc captured once, replayed on four input sets."""
    import gated_delta_rule_20_amd as kda
    names = ("q", "k", "v", "z", "beta", "h0")
    static = {n: t.clone() for n, t in _inputs(kind, 300).items() if isinstance(t, torch.Tensor)}
    cu = static.get("cu_seqlens")
    o = torch.empty_like(static["v"])
    hT = torch.empty_like(static["h0"])
    a_log, g_min = static["A_log"], -5.0

    def call():
        kda.chunk_fwd_noalloc(static["q"], static["k"], static["v"], static["z"], static["beta"], out=o,
                              final_state=hT, A_log=a_log, g_min=g_min, cu_seqlens=cu, initial_state=static["h0"])

    g = _capture(call)
    for rep in range(4):
        inp = _inputs(kind, 301 + rep)
        for n in names:
            static[n].copy_(inp[n])
        g.replay()
        o_ref, h_ref = kda.chunk_fwd(inp["q"], inp["k"], inp["v"], inp["z"], inp["beta"], A_log=a_log,
                                     g_min=g_min, cu_seqlens=cu, initial_state=inp["h0"])
        torch.cuda.synchronize()
        _same(f"o (replay {rep})", o, o_ref)
        _same(f"final state (replay {rep})", hT, h_ref)


def test_decode_step_graph_replays():
    """kda_recurrent_step captured once; eight replays advance the in-place
    state step by step, each with fresh token inputs, against eager steps on a
    copy of the state."""
    import gated_delta_rule_20_amd as kda
    w = dataclasses.replace(W.WORKLOADS["decode_512"], seed=310)
    d = W.make_decode(w, device="cuda", N=8, H=4, steps=8)
    names = ("q", "k", "v", "z", "beta")
    static = {n: d["steps"][0][n].clone() for n in names}
    state = d["state"].clone()
    o = torch.empty_like(static["v"])

    def call():
        kda.recurrent_step(static["q"], static["k"], static["v"], static["z"], static["beta"], state,
                           A_log=d["A_log"], out=o)

    g = _capture(call)  # the set-up run advanced `state`: restart from the initial state
    state.copy_(d["state"])
    ref_state = d["state"].clone()
    for i, st in enumerate(d["steps"]):
        for n in names:
            static[n].copy_(st[n])
        g.replay()
        o_ref = kda.recurrent_step(st["q"], st["k"], st["v"], st["z"], st["beta"], ref_state, A_log=d["A_log"])
        torch.cuda.synchronize()
        _same(f"o (step {i})", o, o_ref)
        _same(f"state (step {i})", state, ref_state)


def test_speculative_window_graph_replays():
    """kda_recurrent_replay (replayed drafts of a cached window, then a new
    window, bonus committed) captured once; four replays on fresh windows and
    accepted counts, against eager calls on a copy of the state."""
    import gated_delta_rule_20_amd as kda
    w = dataclasses.replace(W.WORKLOADS["decode_512_spec"], seed=320)
    d = W.make_spec_decode(w, device="cuda", N=8, H=4, calls=4)
    names = ("k_r", "v_r", "z_r", "beta_r", "n_replay", "q", "k", "v", "z", "beta")
    static = {n: d["calls"][0][n].clone() for n in names}
    state = d["state"].clone()
    o = torch.empty_like(static["v"])

    def call():
        kda.recurrent_replay(static["q"], static["k"], static["v"], static["z"], static["beta"], state,
                             replay=(static["k_r"], static["v_r"], static["z_r"], static["beta_r"]),
                             n_replay=static["n_replay"], n_commit=1, A_log=d["A_log"], g_min=d["g_min"], out=o)

    g = _capture(call)  # the set-up run advanced `state`: restart from the initial state
    state.copy_(d["state"])
    ref_state = d["state"].clone()
    for i, c in enumerate(d["calls"]):
        for n in names:
            static[n].copy_(c[n])
        g.replay()
        o_ref = kda.recurrent_replay(c["q"], c["k"], c["v"], c["z"], c["beta"], ref_state,
                                     replay=(c["k_r"], c["v_r"], c["z_r"], c["beta_r"]), n_replay=c["n_replay"],
                                     n_commit=1, A_log=d["A_log"], g_min=d["g_min"])
        torch.cuda.synchronize()
        _same(f"o (call {i})", o, o_ref)
        _same(f"state (call {i})", state, ref_state)
