"""Seeded random configurations of kda_chunk_fwd and kda_recurrent_replay against
the oracles, mixing what the targeted tests cover one at a time: head dims,
packed lengths (including 0, 1 and lengths around the chunk size), initial
states, checkpoints, the layer prologue / epilogue and convolution widths, and
replay windows with ragged accepted counts.  Each configuration is small; the
seeds are fixed, so a failure names a reproducible case."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import oracle.layer as L
import workloads as W
from kda_testutil import TOL, np64, rel_err

pytestmark = pytest.mark.gpu

EPS = 1e-6


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gated_delta_rule_20_amd as kda
    kda.load_library()


def _draw(seed):
    r = np.random.default_rng(seed)
    Dk, Dv = (int(x) for x in r.choice([64, 128], size=2))
    H = int(r.integers(1, 4))
    n = int(r.integers(1, 6))
    pool = [0, 1, 2, 3, 63, 64, 65, 127, 128, 129, 200]
    lens = [int(r.choice(pool)) if r.random() < 0.6 else int(r.integers(1, 260)) for _ in range(n)]
    return dict(Dk=Dk, Dv=Dv, H=H, lens=lens, pro=bool(r.random() < 0.6), epi=bool(r.random() < 0.5),
                cw=int(r.integers(1, 5)), ckpt=bool(r.random() < 0.5), zmode=bool(r.random() < 0.7))


@pytest.mark.parametrize("seed", range(1000, 1012))
def test_random_prefill(seed):
    import gated_delta_rule_20_amd as kda
    c = _draw(seed)
    Dk, Dv, H, lens = c["Dk"], c["Dv"], c["H"], c["lens"]
    N = len(lens)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    T = int(cu[-1])
    w = dataclasses.replace(W.WORKLOADS["prefill_8k"], Dk=Dk, Dv=Dv, seed=seed)
    d = W.make_layer(w, "cuda", N=1, T=max(T, 1), H=H, conv_width=c["cw"])
    s = W.make_layer(w, "cuda", N=N, T=1, H=H, conv_width=c["cw"], seed_offset=7)
    x = {n: d[n][0, :T].contiguous() for n in ("q_pre", "k_pre", "v_pre", "z", "beta_logit", "gate")}
    if not c["pro"]:   # core inputs: unit q, k and beta in (0, 1)
        unit = lambda t: (t.float() / t.float().norm(dim=-1, keepdim=True).clamp_min(1e-6)).to(t.dtype)
        x["q_pre"], x["k_pre"] = unit(x["q_pre"]), unit(x["k_pre"])
        x["beta_logit"] = torch.sigmoid(x["beta_logit"].float()).to(x["beta_logit"].dtype)
    if not c["zmode"]:
        x["z"] = (-5.0 * torch.rand(x["z"].shape, device="cuda")).to(torch.bfloat16)
    A = d["A_log"] if c["zmode"] else None
    slots = 3
    ck = torch.full((N, slots, H, Dk, Dv), float("nan"), device="cuda") if c["ckpt"] else None
    cs_out = torch.full_like(s["conv_state"], float("nan")) if c["pro"] else None
    f = kda.Fusion(conv_weight=d["conv_weight"] if c["pro"] else None,
                   conv_state=s["conv_state"] if (c["pro"] and c["cw"] > 1) else None,
                   conv_state_out=cs_out if (c["pro"] and c["cw"] > 1) else None, qk_eps=EPS,
                   gate=x["gate"] if c["epi"] else None, o_norm_weight=d["o_norm_weight"] if c["epi"] else None,
                   o_eps=EPS)
    cu_t = torch.tensor(cu, dtype=torch.int32, device="cuda")
    run = lambda fu: kda.chunk_fwd(x["q_pre"], x["k_pre"], x["v_pre"], x["z"], x["beta_logit"], A_log=A,
                                   cu_seqlens=cu_t, initial_state=s["state"], checkpoints=ck,
                                   checkpoint_every=1, fusion=fu)
    y, hT = run(f)
    o_plain = y
    if c["epi"]:      # o~ of the same call without the epilogue (the bf16 epilogue is checked in two parts)
        f2 = kda.Fusion(conv_weight=f.conv_weight, conv_state=f.conv_state, qk_eps=EPS)
        o_plain, _ = run(f2 if c["pro"] else None)
    torch.cuda.synchronize()
    args = [np64(x[n]) for n in ("q_pre", "k_pre", "v_pre", "z", "beta_logit")]
    Ar = np64(A)
    if c["pro"]:
        o_ref, h_ref, cs_ref = L.layer_forward(*args, conv_weight=np64(d["conv_weight"]),
                                               conv_state=np64(s["conv_state"]) if c["cw"] > 1 else None,
                                               cu_seqlens=cu, h0=np64(s["state"]), A_log=Ar, g_min=-5.0, qk_eps=EPS)
    else:
        o_ref, h_ref = oracle.forward(*args, cu_seqlens=cu, h0=np64(s["state"]), A_log=Ar, g_min=-5.0)
    tol = TOL[torch.bfloat16]
    msg = f"seed {seed}: {c}"
    if T:
        assert rel_err(np64(o_plain), o_ref) <= tol, msg
        if c["epi"]:
            assert rel_err(np64(y), L.epilogue(np64(o_plain), np64(x["gate"]), np64(d["o_norm_weight"]), EPS)) \
                <= 1e-2, msg
    assert rel_err(np64(hT), h_ref) <= tol, msg
    if c["pro"] and c["cw"] > 1:
        assert np.array_equal(np64(cs_out), cs_ref), msg
    if c["ckpt"]:
        for sq in range(N):
            for j in range(slots):
                P = (j + 1) * 64
                if P >= lens[sq]:
                    assert torch.isnan(ck[sq, j]).all(), msg
                    continue
                a = int(cu[sq])
                pa = [v[a:a + P] for v in args]
                if c["pro"]:
                    _, hr, _ = L.layer_forward(*pa, conv_weight=np64(d["conv_weight"]),
                                               conv_state=np64(s["conv_state"][sq:sq + 1]) if c["cw"] > 1 else None,
                                               h0=np64(s["state"][sq:sq + 1]), A_log=Ar, g_min=-5.0, qk_eps=EPS)
                else:
                    _, hr = oracle.forward(*pa, h0=np64(s["state"][sq:sq + 1]), A_log=Ar, g_min=-5.0)
                assert rel_err(np64(ck[sq, j]), hr[0]) <= tol, (msg, sq, j)


@pytest.mark.parametrize("seed", range(2000, 2008))
def test_random_replay(seed):
    """Random windows through the plain or fused replay kernel, per sequence
    against the layer oracle over (replayed accepted drafts ++ new tokens)."""
    import gated_delta_rule_20_amd as kda
    r = np.random.default_rng(seed)
    Dk, Dv = (int(x) for x in r.choice([64, 128], size=2))
    N, H = int(r.integers(1, 6)), int(r.integers(1, 4))
    Tr, Tn = int(r.integers(0, 10)), int(r.integers(0, 10))
    if Tr + Tn == 0:
        Tn = 1
    n_commit = int(r.integers(0, Tn + 1))
    pro, epi = bool(r.random() < 0.5), bool(r.random() < 0.5) and Tn > 0
    w = dataclasses.replace(W.WORKLOADS["decode_512"], Dk=Dk, Dv=Dv, seed=seed, A_uniform=1.0)
    d = W.make_layer(w, "cuda", N=N, T=Tr + Tn, H=H, conv_width=4)
    if not pro:
        unit = lambda t: (t.float() / t.float().norm(dim=-1, keepdim=True).clamp_min(1e-6)).to(t.dtype)
        d["q_pre"], d["k_pre"] = unit(d["q_pre"]), unit(d["k_pre"])
        d["beta_logit"] = torch.sigmoid(d["beta_logit"].float()).to(d["beta_logit"].dtype)
    n_rep = torch.tensor(r.integers(0, Tr + 1, size=N), dtype=torch.int32)
    h0, cs0 = d["state"].clone(), d["conv_state"].clone()
    state, cs = d["state"], d["conv_state"]
    part = lambda n, a, b: d[n][:, a:b].contiguous()
    names = ("q_pre", "k_pre", "v_pre", "z", "beta_logit")
    rq, rk, rv, rz, rb = (part(n, 0, Tr) for n in names)
    q, k, v, z, b = (part(n, Tr, Tr + Tn) for n in names)
    gate = part("gate", Tr, Tr + Tn)
    f = kda.Fusion(conv_weight=d["conv_weight"] if pro else None, conv_state=cs if pro else None, qk_eps=EPS,
                   gate=gate if epi else None, o_norm_weight=d["o_norm_weight"] if epi else None, o_eps=EPS)
    o = kda.recurrent_replay(q if Tn else None, k if Tn else None, v if Tn else None, z if Tn else None,
                             b if Tn else None, state, replay=(rk, rv, rz, rb) if Tr else None,
                             n_replay=n_rep.cuda() if Tr else None, n_commit=n_commit, A_log=d["A_log"],
                             q_r=rq if (Tr and pro) else None, fusion=f)
    torch.cuda.synchronize()
    nr = [int(x) for x in n_rep] if Tr else [0] * N
    msg = f"seed {seed}: Dk={Dk} Dv={Dv} N={N} H={H} Tr={Tr} Tn={Tn} commit={n_commit} pro={pro} epi={epi} {nr}"

    def ref(tokens, seqs_out):
        lens = [len(t) for t in tokens]
        cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
        cat = lambda n: np.concatenate([np64(d[n][sq, idx]) for sq, idx in enumerate(tokens)])
        args = [cat(n) for n in names]
        if pro:
            return L.layer_forward(*args, conv_weight=np64(d["conv_weight"]), conv_state=np64(cs0), cu_seqlens=cu,
                                   h0=np64(h0), A_log=np64(d["A_log"]), g_min=-5.0, qk_eps=EPS,
                                   gate=cat("gate") if epi else None, o_weight=np64(d["o_norm_weight"]),
                                   o_eps=EPS) + (cu,)
        oo, hh = oracle.forward(*args, cu_seqlens=cu, h0=np64(h0), A_log=np64(d["A_log"]), g_min=-5.0)
        if epi:
            oo = L.epilogue(oo, cat("gate"), np64(d["o_norm_weight"]), EPS)
        return oo, hh, None, cu

    if Tn:
        oo, _, _, cu = ref([list(range(x)) + list(range(Tr, Tr + Tn)) for x in nr], None)
        o_ref = np.stack([oo[cu[s_] + nr[s_]:cu[s_ + 1]] for s_ in range(N)])
        assert rel_err(np64(o), o_ref) <= TOL[torch.bfloat16], msg
    commit = [list(range(x)) + list(range(Tr, Tr + n_commit)) for x in nr]
    _, h_ref, cs_ref, _ = ref(commit, None)
    for s_ in range(N):
        if not commit[s_]:
            assert torch.equal(state[s_], h0[s_]) and torch.equal(cs[s_], cs0[s_]), msg
            continue
        assert rel_err(np64(state[s_]), h_ref[s_]) <= TOL[torch.bfloat16], (msg, s_)
        if pro:
            assert np.array_equal(np64(cs[s_]), cs_ref[s_]), (msg, s_)
