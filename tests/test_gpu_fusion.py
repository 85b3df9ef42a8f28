"""GPU parity of the layer prologue (eq. (2)) and epilogue (eq. (6)) fused into
the decode entry points ("Kimi K3 Technical Report", §2.1.1; §5.4.2 runs short
convolution, input normalisation, gating, the recurrence and output
normalisation in one decode kernel).

Reference: oracle.layer (fp64) over each sequence's token stream: the carried
convolution state, then the replayed tokens, then the new ones.  Outputs and
recurrent states within the dtype's bound; the convolution state holds copies
of input values and must match bit for bit."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle.layer as L
import workloads as W
from kda_testutil import TOL, np64, rel_err

pytestmark = pytest.mark.gpu

QK_EPS, O_EPS = 1e-6, 1e-6


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gated_delta_rule_20_amd as kda
    kda.load_library()


def _wl(dtype=torch.bfloat16, Dk=128, Dv=128, seed=60):
    return dataclasses.replace(W.WORKLOADS["decode_512"], dtype=dtype, Dk=Dk, Dv=Dv, seed=seed, A_uniform=1.0)


def _fusion(d, pro, epi, conv_state=None, gate=None):
    import gated_delta_rule_20_amd as kda
    return kda.Fusion(conv_weight=d["conv_weight"] if pro else None, conv_state=conv_state if pro else None,
                      qk_eps=QK_EPS, gate=gate if epi else None,
                      o_norm_weight=d["o_norm_weight"] if epi else None, o_eps=O_EPS)


def _plain_inputs(d):
    """Inputs of the core without the prologue: unit q, k, beta in (0, 1)."""
    unit = lambda x: (x.float() / x.float().norm(dim=-1, keepdim=True)).to(x.dtype)
    return dict(q=unit(d["q_pre"]), k=unit(d["k_pre"]), v=d["v_pre"], beta=torch.sigmoid(d["beta_logit"].float())
                .to(d["beta_logit"].dtype))


def _oracle(d, pro, epi, seq_tokens, n_out, h0, cs0):
    """Per sequence s, the token indices seq_tokens[s] (into the [N, T] axes of
    d) run through the layer from (h0[s], cs0[s]); returns the outputs of the
    last n_out[s] tokens of each stream, the final states and conv states."""
    N = len(seq_tokens)
    names = ("q_pre", "k_pre", "v_pre", "z", "beta_logit", "gate")
    src = {n: np64(d[n]) for n in names}
    if not pro:
        p = _plain_inputs(d)
        src.update(q_pre=np64(p["q"]), k_pre=np64(p["k"]), v_pre=np64(p["v"]), beta_logit=np64(p["beta"]))
    parts = {n: [src[n][s, idx] for s, idx in enumerate(seq_tokens)] for n in names}
    lens = [len(idx) for idx in seq_tokens]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    cat = {n: np.concatenate(parts[n]) for n in names}
    A = np64(d["A_log"])
    if pro:
        o, hT, cs = L.layer_forward(cat["q_pre"], cat["k_pre"], cat["v_pre"], cat["z"], cat["beta_logit"],
                                    conv_weight=np64(d["conv_weight"]), conv_state=np64(cs0), cu_seqlens=cu,
                                    h0=np64(h0), A_log=A, g_min=d["g_min"], qk_eps=QK_EPS,
                                    gate=cat["gate"] if epi else None, o_weight=np64(d["o_norm_weight"]),
                                    o_eps=O_EPS)
    else:
        import oracle
        o, hT = oracle.forward(cat["q_pre"], cat["k_pre"], cat["v_pre"], cat["z"], cat["beta_logit"], cu_seqlens=cu,
                               h0=np64(h0), A_log=A, g_min=d["g_min"])
        if epi:
            o = L.epilogue(o, cat["gate"], np64(d["o_norm_weight"]), O_EPS)
        cs = None
    outs = [o[cu[s + 1] - n_out[s]:cu[s + 1]] for s in range(N)]
    return outs, hT, cs


def _inputs_at(d, pro, sl):
    """(q, k, v, z, beta, gate) device tensors for token slice sl of every sequence."""
    if pro:
        q, k, v, b = d["q_pre"], d["k_pre"], d["v_pre"], d["beta_logit"]
    else:
        p = _plain_inputs(d)
        q, k, v, b = p["q"], p["k"], p["v"], p["beta"]
    c = lambda x: x[:, sl].contiguous()
    return c(q), c(k), c(v), c(d["z"]), c(b), c(d["gate"])


@pytest.mark.parametrize("pro,epi", [(True, True), (True, False), (False, True)])
@pytest.mark.parametrize("dtype,Dk,Dv,cw", [(torch.bfloat16, 128, 128, 4), (torch.bfloat16, 64, 128, 3),
                                            (torch.bfloat16, 128, 64, 2), (torch.float32, 64, 64, 4)])
def test_fused_decode_steps(pro, epi, dtype, Dk, Dv, cw):
    """Three consecutive kda_recurrent_step calls, state and conv state carried."""
    import gated_delta_rule_20_amd as kda
    N, H, K = 5, 3, 3
    d = W.make_layer(_wl(dtype, Dk, Dv), "cuda", N=N, T=K, H=H, conv_width=cw)
    h0, cs0 = d["state"].clone(), d["conv_state"].clone()
    state, cs = d["state"].clone(), d["conv_state"].clone()
    ys = []
    for t in range(K):
        q, k, v, z, b, gate = _inputs_at(d, pro, t)
        ys.append(kda.recurrent_step(q, k, v, z, b, state, A_log=d["A_log"],
                                     fusion=_fusion(d, pro, epi, cs, gate)))
    torch.cuda.synchronize()
    outs, hT, cs_ref = _oracle(d, pro, epi, [list(range(K))] * N, [K] * N, h0, cs0)
    tol = TOL[dtype]
    assert rel_err(np64(torch.stack(ys, 1)), np.stack(outs)) <= tol
    assert rel_err(np64(state), hT) <= tol
    if pro:
        assert np.array_equal(np64(cs), cs_ref)
    else:
        assert torch.equal(cs, cs0)


@pytest.mark.parametrize("cw", [1, 2, 3])
def test_fused_decode_conv_widths(cw):
    """Narrower convolutions (W = 1 carries no state)."""
    import gated_delta_rule_20_amd as kda
    N, H, K = 3, 2, 2
    d = W.make_layer(_wl(seed=61), "cuda", N=N, T=K, H=H, conv_width=cw)
    h0, cs0 = d["state"].clone(), d["conv_state"].clone()
    state, cs = d["state"].clone(), d["conv_state"].clone()
    ys = []
    for t in range(K):
        q, k, v, z, b, gate = _inputs_at(d, True, t)
        ys.append(kda.recurrent_step(q, k, v, z, b, state, A_log=d["A_log"],
                                     fusion=_fusion(d, True, True, cs if cw > 1 else None, gate)))
    torch.cuda.synchronize()
    outs, hT, cs_ref = _oracle(d, True, True, [list(range(K))] * N, [K] * N, h0, cs0)
    assert rel_err(np64(torch.stack(ys, 1)), np.stack(outs)) <= TOL[torch.bfloat16]
    assert rel_err(np64(state), hT) <= TOL[torch.bfloat16]
    if cw > 1:
        assert np.array_equal(np64(cs), cs_ref)


@pytest.mark.parametrize("pro,epi", [(True, True), (True, False), (False, True)])
@pytest.mark.parametrize("Tr,Tn,n_commit", [(3, 4, 1), (7, 5, 2), (0, 6, 6), (9, 2, 0)])
def test_fused_replay(pro, epi, Tr, Tn, n_commit):
    """Speculative step with the fused layer: per sequence the conv history runs
    through the replayed drafts into the new window; state and conv state are
    written back at the commit point (untouched when nothing is committed).
    Windows past 8 tokens cross the kernel's staging block."""
    import gated_delta_rule_20_amd as kda
    N, H = 6, 2
    d = W.make_layer(_wl(seed=62 + Tr), "cuda", N=N, T=Tr + Tn, H=H, conv_width=4)
    gen = torch.Generator().manual_seed(70 + Tr)
    n_rep = torch.randint(0, Tr + 1, (N,), generator=gen, dtype=torch.int32)
    if Tr:
        n_rep[0], n_rep[-1] = 0, Tr                    # both extremes present
    h0, cs0 = d["state"].clone(), d["conv_state"].clone()
    state, cs = d["state"].clone(), d["conv_state"].clone()
    qr, kr, vr, zr, br, _ = _inputs_at(d, pro, slice(0, Tr))
    q, k, v, z, b, gate = _inputs_at(d, pro, slice(Tr, Tr + Tn))
    o = kda.recurrent_replay(q, k, v, z, b, state, replay=(kr, vr, zr, br) if Tr else None,
                             n_replay=n_rep.cuda() if Tr else None, n_commit=n_commit, A_log=d["A_log"],
                             q_r=qr if (Tr and pro) else None, fusion=_fusion(d, pro, epi, cs, gate))
    torch.cuda.synchronize()
    nr = [int(x) for x in n_rep] if Tr else [0] * N
    streams = [list(range(r)) + list(range(Tr, Tr + Tn)) for r in nr]
    outs, _, _ = _oracle(d, pro, epi, streams, [Tn] * N, h0, cs0)
    tol = TOL[torch.bfloat16]
    assert rel_err(np64(o), np.stack(outs)) <= tol
    commit = [list(range(r)) + list(range(Tr, Tr + n_commit)) for r in nr]
    if any(commit):
        _, hT, cs_ref = _oracle(d, pro, epi, commit, [0] * N, h0, cs0)
    for s in range(N):
        if not commit[s]:                              # nothing committed: both states untouched
            assert torch.equal(state[s], h0[s]) and torch.equal(cs[s], cs0[s])
            continue
        assert rel_err(np64(state[s]), hT[s]) <= tol, s
        if pro:
            assert np.array_equal(np64(cs[s]), cs_ref[s]), s
