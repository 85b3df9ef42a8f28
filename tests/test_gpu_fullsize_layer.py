"""The fused layer (eq. (2) prologue, eq. (6) epilogue) at the full workload
sizes, in the configuration the benchmark times: prefill_8k shapes (one call
over B=1, T=8192, H=32, d=128 from pre-convolution projections) and decode_512
shapes (512 sequences x 32 heads, consecutive steps, states in place).  The
layer oracle recomputes sampled heads / sequences in full.

The bf16 prefill output is checked as in test_gpu_fusion_prefill: the fused
output y end to end against the oracle's y within the per-element bound derived
from the core's bound (every head, streamed), and in addition o~ (the same call
without the epilogue) against the oracle and y against the fp64 epilogue of
that o~."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle.layer as L
import workloads as W
from kda_testutil import TOL, RunningErr, check_epilogue_end_to_end, np64, rel_err

pytestmark = pytest.mark.gpu

QK_EPS, O_EPS, EPI_TOL = 1e-6, 1e-6, 1e-2


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gated_delta_rule_20_amd as kda
    kda.load_library()


def test_layer_prefill_8k_all_heads():
    """prefill_8k shapes through the fused layer: every head against the layer
    oracle, streamed eight heads at a time.  y end to end within the derived
    bound; o~ and the final state within the core bound; the convolution
    state bit for bit."""
    import gated_delta_rule_20_amd as kda
    w = W.WORKLOADS["prefill_8k"]
    d = W.make_layer(w, "cuda", N=w.B, T=w.T, H=w.H)

    def run(epi):
        cs_out = torch.empty_like(d["conv_state"])
        f = kda.Fusion(conv_weight=d["conv_weight"], conv_state=d["conv_state"], conv_state_out=cs_out,
                       qk_eps=QK_EPS, gate=d["gate"] if epi else None,
                       o_norm_weight=d["o_norm_weight"] if epi else None, o_eps=O_EPS)
        o, hT = kda.chunk_fwd(d["q_pre"], d["k_pre"], d["v_pre"], d["z"], d["beta_logit"], A_log=d["A_log"],
                              g_min=d["g_min"], initial_state=d["state"], fusion=f)
        torch.cuda.synchronize()
        return o, hT, cs_out

    y, hT, cs = run(True)
    o_plain, _, _ = run(False)
    tol = TOL[torch.bfloat16]
    e_o, e_s, e_y, e_epi = RunningErr(), RunningErr(), RunningErr(), RunningErr()
    worst = 0.0
    for h0 in range(0, w.H, 8):
        heads = list(range(h0, min(w.H, h0 + 8)))
        sel = lambda t: np64(t[:, :, heads])                     # [B, T, H, .] -> these heads
        o_ref, h_ref, cs_ref = L.layer_forward(
            sel(d["q_pre"]), sel(d["k_pre"]), sel(d["v_pre"]), sel(d["z"]), sel(d["beta_logit"]),
            conv_weight=np64(d["conv_weight"])[heads], conv_state=np64(d["conv_state"])[:, heads],
            h0=np64(d["state"])[:, heads], A_log=np64(d["A_log"])[heads], g_min=d["g_min"], qk_eps=QK_EPS,
            nthreads=16)
        g_sel, w_sel = sel(d["gate"]), np64(d["o_norm_weight"])[heads]
        ratio, _ = check_epilogue_end_to_end(sel(y), o_ref, g_sel, w_sel, O_EPS, tol)
        worst = max(worst, ratio)
        e_y.add(sel(y), L.epilogue(o_ref, g_sel, w_sel, O_EPS))
        e_o.add(sel(o_plain), o_ref)
        e_s.add(np64(hT)[:, heads], h_ref)
        e_epi.add(sel(y), L.epilogue(sel(o_plain), g_sel, w_sel, O_EPS))
        assert np.array_equal(np64(cs)[:, heads], cs_ref)
        print(f"heads {heads[0]}..{heads[-1]}: worst |dy|/bound {worst:.3f}", flush=True)
    print(f"y end to end: worst |dy|/bound {worst:.3f}, whole-tensor rel err {e_y.rel:.3e}; "
          f"o~ {e_o.rel:.3e}  state {e_s.rel:.3e}  epilogue of o~ {e_epi.rel:.3e}")
    assert worst <= 1.0
    assert e_o.rel <= tol and e_s.rel <= tol and e_epi.rel <= EPI_TOL


def test_layer_decode_512_sampled_sequences():
    import gated_delta_rule_20_amd as kda
    w = W.WORKLOADS["decode_512"]
    K = 4
    d = W.make_layer(dataclasses.replace(w, A_uniform=1.0), "cuda", N=w.B, T=K, H=w.H)
    h0, cs0 = d["state"].clone(), d["conv_state"].clone()
    state, cs = d["state"], d["conv_state"]
    ys = []
    for t in range(K):
        sl = lambda n: d[n][:, t].contiguous()
        f = kda.Fusion(conv_weight=d["conv_weight"], conv_state=cs, qk_eps=QK_EPS, gate=sl("gate"),
                       o_norm_weight=d["o_norm_weight"], o_eps=O_EPS)
        ys.append(kda.recurrent_step(sl("q_pre"), sl("k_pre"), sl("v_pre"), sl("z"), sl("beta_logit"), state,
                                     A_log=d["A_log"], g_min=d["g_min"], fusion=f))
    torch.cuda.synchronize()
    seqs = [0, 1, 255, 511]
    sel = lambda n: np64(d[n][seqs])
    o_ref, h_ref, cs_ref = L.layer_forward(
        sel("q_pre"), sel("k_pre"), sel("v_pre"), sel("z"), sel("beta_logit"),
        conv_weight=np64(d["conv_weight"]), conv_state=np64(cs0[seqs]), h0=np64(h0[seqs]),
        A_log=np64(d["A_log"]), g_min=d["g_min"], qk_eps=QK_EPS, gate=np64(d["gate"][seqs]),
        o_weight=np64(d["o_norm_weight"]), o_eps=O_EPS, nthreads=16)
    e_o = rel_err(np64(torch.stack(ys, 1)[seqs]), o_ref)
    e_s = rel_err(np64(state[seqs]), h_ref)
    print(f"y {e_o:.3e}  state {e_s:.3e}")
    assert e_o <= TOL[torch.bfloat16] and e_s <= TOL[torch.bfloat16]
    assert np.array_equal(np64(cs[seqs]), cs_ref)


def test_layer_spec_512_sampled_sequences():
    """decode_512_spec shapes through the fused layer, as the benchmark times them:
    512 sequences x 32 heads, a cached 3-token window of which 0..3 drafts were
    accepted and are replayed, then 4 new tokens, the bonus token committed.
    Sampled sequences are recomputed by the layer oracle over (accepted drafts ++
    new tokens); the committed states against its state after the bonus token."""
    import gated_delta_rule_20_amd as kda
    w = W.WORKLOADS["decode_512_spec"]
    Tr, Tn = w.T - 1, 4
    d = W.make_layer(dataclasses.replace(w, A_uniform=1.0), "cuda", N=w.B, T=Tr + Tn, H=w.H)
    g = torch.Generator().manual_seed(77)
    n_rep = torch.randint(0, Tr + 1, (w.B,), generator=g, dtype=torch.int32)
    h0, cs0 = d["state"].clone(), d["conv_state"].clone()
    state, cs = d["state"], d["conv_state"]
    names = ("q_pre", "k_pre", "v_pre", "z", "beta_logit")
    part = lambda n, a, b: d[n][:, a:b].contiguous()
    q, k, v, z, b = (part(n, Tr, Tr + Tn) for n in names)
    rq, rk, rv, rz, rb = (part(n, 0, Tr) for n in names)
    f = kda.Fusion(conv_weight=d["conv_weight"], conv_state=cs, qk_eps=QK_EPS, gate=part("gate", Tr, Tr + Tn),
                   o_norm_weight=d["o_norm_weight"], o_eps=O_EPS)
    o = kda.recurrent_replay(q, k, v, z, b, state, replay=(rk, rv, rz, rb), n_replay=n_rep.cuda(), n_commit=1,
                             A_log=d["A_log"], g_min=d["g_min"], q_r=rq, fusion=f)
    torch.cuda.synchronize()
    seqs = [0, 1, 300, 511]
    for s in seqs:
        nr = int(n_rep[s])
        idx = list(range(nr)) + list(range(Tr, Tr + Tn))
        ref = lambda toks: L.layer_forward(
            *(np64(d[n][s:s + 1, toks]) for n in names), conv_weight=np64(d["conv_weight"]),
            conv_state=np64(cs0[s:s + 1]), h0=np64(h0[s:s + 1]), A_log=np64(d["A_log"]), g_min=d["g_min"],
            qk_eps=QK_EPS, gate=np64(d["gate"][s:s + 1, toks]), o_weight=np64(d["o_norm_weight"]), o_eps=O_EPS,
            nthreads=16)
        o_ref, _, _ = ref(idx)
        _, h_ref, cs_ref = ref(list(range(nr)) + [Tr])       # committed: the accepted drafts and the bonus
        e_o = rel_err(np64(o[s]), o_ref[0, nr:])
        e_s = rel_err(np64(state[s]), h_ref[0])
        print(f"seq {s} (replayed {nr}): y {e_o:.3e}  state {e_s:.3e}")
        assert e_o <= TOL[torch.bfloat16] and e_s <= TOL[torch.bfloat16], (s, nr, e_o, e_s)
        assert np.array_equal(np64(cs[s]), cs_ref[0]), s
