"""Pins for the fp64 oracle: checks against what the pages and the mathematics
fix, independent of the oracle's own code.

Each ``pin_*`` function takes an oracle library handle (so the mutation test
can run the same pins against deliberately broken builds) and raises
AssertionError on failure.  Sources cited per pin refer to
"Kimi K3 Technical Report: Open Frontier Intelligence" §2.1.1 unless noted.
"""
from __future__ import annotations

import json
import os

import numpy as np
from scipy.special import expit

import oracle
from oracle.chunked import chunked_sequence

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _rng(seed):
    return np.random.default_rng(seed)


def _unit(x):
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def _rand_inputs(seed, T, H, Dk, Dv, g_floor=-5.0):
    r = _rng(seed)
    q = _unit(r.standard_normal((T, H, Dk)))
    k = _unit(r.standard_normal((T, H, Dk)))
    v = r.standard_normal((T, H, Dv))
    g = g_floor * r.random((T, H, Dk))
    beta = expit(r.standard_normal((T, H)))
    return q, k, v, g, beta


def _close(a, b, rtol, what):
    a, b = np.asarray(a), np.asarray(b)
    den = max(np.max(np.abs(b)), 1e-300)
    err = np.max(np.abs(a - b)) / den if a.size else 0.0
    assert err <= rtol, f"{what}: rel err {err:.3e} > {rtol:.1e}"


# --- hand-worked examples (tests/golden) --------------------------------------

def pin_golden_logdecay(lib):
    """eq. (1) on a two-token example worked by hand (d_k=2, d_v=1)."""
    f = json.load(open(os.path.join(GOLDEN, "hand_eq1_dk2_dv1.json")))
    sh = lambda x: np.array(x, dtype=np.float64)[:, None, :]
    o, hT = oracle.forward(sh(f["q"]), sh(f["k"]), sh(f["v"]), sh(f["g"]),
                           np.array(f["beta"])[:, None], h0=np.array(f["h0"])[None, None],
                           lib=lib)
    _close(o[:, 0, :], f["o"], 1e-14, "hand example o")
    _close(hT[0, 0], f["hT"], 1e-14, "hand example final state")


def pin_golden_gate(lib):
    """eq. (1) with the eq. (5) gate on a one-token example worked by hand."""
    f = json.load(open(os.path.join(GOLDEN, "hand_eq1_eq5_dk1_dv2.json")))
    sh = lambda x: np.array(x, dtype=np.float64)[:, None, :]
    o, hT = oracle.forward(sh(f["q"]), sh(f["k"]), sh(f["v"]), sh(f["z"]),
                           np.array(f["beta"])[:, None], h0=np.array(f["h0"])[None, None],
                           A_log=np.array([f["A_h"]]), g_min=f["g_min"], lib=lib)
    _close(o[:, 0, :], f["o"], 1e-14, "hand gate example o")
    _close(hT[0, 0], f["hT"], 1e-14, "hand gate example final state")


def pin_gate_page_bounds(lib):
    """eq. (5) and the numbers printed after it: alpha > e^-5 ~ 6.7e-3, a
    16-token tile's log-decay in (-80, 0), e^80 inside bf16; z = 0 gives
    g_min/2 for any A_h; agreement with scipy's logistic function."""
    f = json.load(open(os.path.join(GOLDEN, "page_gate_bounds.json")))
    gmin = f["g_min"]
    g_sat = oracle.gate(np.array([1e4, 1e6]), 0.7, gmin, lib=lib)
    assert np.all(g_sat == gmin), g_sat
    floor = np.exp(g_sat[0])
    assert abs(floor - f["alpha_floor_printed"]) / f["alpha_floor_printed"] < f["alpha_floor_rel_tol"]
    for A in (-1.0, 0.0, 0.37, 1.0):
        assert oracle.gate(np.zeros(3), A, gmin, lib=lib).tolist() == [gmin / 2] * 3
    r = _rng(11)
    z = r.standard_normal(4096) * 4
    for A in (-0.8, 0.0, 0.9):
        g = oracle.gate(z, A, gmin, lib=lib)
        assert np.all(g < 0) and np.all(g > gmin)
        _close(g, gmin * expit(np.exp(A) * z), 1e-14, "gate vs scipy expit")
        # monotone decreasing in z
        order = np.argsort(z)
        assert np.all(np.diff(g[order]) <= 0)
    g16 = np.full(f["tile_tokens"], gmin)
    assert g16.sum() >= f["tile_logdecay_floor"]
    assert np.exp(-g16.sum()) < f["bf16_max"]


# --- closed forms and invariants of eq. (1) -----------------------------------

def pin_beta_zero_pure_decay(lib):
    """beta = 0: eq. (1) reduces to S_t = Diag(prod alpha) S_0, o_t = S_t^T q_t."""
    T, H, Dk, Dv = 23, 2, 5, 3
    q, k, v, g, _ = _rand_inputs(1, T, H, Dk, Dv)
    h0 = _rng(2).standard_normal((1, H, Dk, Dv))
    o, hT = oracle.forward(q, k, v, g, np.zeros((T, H)), h0=h0, lib=lib)
    lam = np.cumsum(g, axis=0)                       # [T, H, Dk]
    for h in range(H):
        St = np.exp(lam[:, h, :])[:, :, None] * h0[0, h][None]   # [T, Dk, Dv]
        _close(o[:, h], np.einsum("tjc,tj->tc", St, q[:, h]), 1e-13, "beta=0 outputs")
        _close(hT[0, h], St[-1], 1e-13, "beta=0 final state")


def pin_orthonormal_retrieval(lib):
    """alpha = 1, beta = 1, orthonormal keys, S_0 = 0: the state stores each
    association exactly, S_n^T k_i = v_i; querying with k_t right after its
    write returns v_t (output read after the update)."""
    Dk, Dv, n = 6, 4, 5
    r = _rng(3)
    Qm, _ = np.linalg.qr(r.standard_normal((Dk, Dk)))
    k = Qm[:, :n].T[:, None, :]                       # [n, 1, Dk]
    v = r.standard_normal((n, 1, Dv))
    o, hT = oracle.forward(k.copy(), k, v, np.zeros((n, 1, Dk)), np.ones((n, 1)), lib=lib)
    _close(hT[0, 0].T @ k[:, 0, :].T, v[:, 0, :].T, 1e-13, "retrieval S^T k_i = v_i")
    _close(o[:, 0], v[:, 0], 1e-13, "read-after-write o_t = v_t")


def pin_overwrite(lib):
    """alpha = beta = 1: writing the same unit key twice leaves S^T k equal to
    the latest value, whatever the entering state."""
    Dk, Dv = 4, 3
    r = _rng(4)
    kk = _unit(r.standard_normal(Dk))
    v1, v2 = r.standard_normal(Dv), r.standard_normal(Dv)
    k = np.stack([kk, kk])[:, None]
    v = np.stack([v1, v2])[:, None]
    h0 = r.standard_normal((1, 1, Dk, Dv))
    _, hT = oracle.forward(k.copy(), k, v, np.zeros((2, 1, Dk)), np.ones((2, 1)), h0=h0, lib=lib)
    _close(hT[0, 0].T @ kk, v2, 1e-13, "overwrite")


def pin_scalar_case(lib):
    """d_k = d_v = 1: eq. (1) is the scalar recurrence
    s_t = alpha_t (1 - beta_t k_t^2) s_{t-1} + beta_t k_t v_t, o_t = s_t q_t."""
    T = 40
    r = _rng(5)
    q, k, v = r.standard_normal((3, T))
    g = -5 * r.random(T)
    b = expit(r.standard_normal(T))
    s, ref = 0.3, []
    for t in range(T):
        s = np.exp(g[t]) * (1 - b[t] * k[t] ** 2) * s + b[t] * k[t] * v[t]
        ref.append(s * q[t])
    o, hT = oracle.forward(q[:, None, None], k[:, None, None], v[:, None, None],
                           g[:, None, None], b[:, None], h0=np.full((1, 1, 1, 1), 0.3), lib=lib)
    _close(o[:, 0, 0], ref, 1e-13, "scalar outputs")
    _close(hT[0, 0, 0, 0], s, 1e-13, "scalar final state")


def pin_affine_transition(lib):
    """The final state is affine in the entering state with the transition
    M = M_T ... M_1, M_t = (I - beta_t k_t k_t^T) Diag(alpha_t)
    (§5.1.2, eq. (17)): S_T(S_0) = S_T(0) + M S_0, with M formed from dense
    matrices."""
    T, H, Dk, Dv = 17, 1, 5, 7
    q, k, v, g, b = _rand_inputs(6, T, H, Dk, Dv)
    h0 = _rng(7).standard_normal((1, H, Dk, Dv))
    _, hs = oracle.forward(q, k, v, g, b, h0=h0, lib=lib)
    _, hz = oracle.forward(q, k, v, g, b, lib=lib)
    M = np.eye(Dk)
    for t in range(T):
        kt = k[t, 0][:, None]
        Mt = (np.eye(Dk) - b[t, 0] * kt @ kt.T) @ np.diag(np.exp(g[t, 0]))
        M = Mt @ M
    _close(hs[0, 0], hz[0, 0] + M @ h0[0, 0], 1e-13, "eq. (17) affine structure")


def pin_split(lib):
    """One pass equals two passes, the second entered with the first's final
    state (state hand-off, as prefix-cache resume and KCP rely on)."""
    T, H, Dk, Dv = 61, 3, 8, 6
    q, k, v, g, b = _rand_inputs(8, T, H, Dk, Dv)
    h0 = _rng(9).standard_normal((1, H, Dk, Dv))
    o, hT = oracle.forward(q, k, v, g, b, h0=h0, lib=lib)
    for cut in (1, 29, 60):
        o1, h1 = oracle.forward(q[:cut], k[:cut], v[:cut], g[:cut], b[:cut], h0=h0, lib=lib)
        o2, h2 = oracle.forward(q[cut:], k[cut:], v[cut:], g[cut:], b[cut:], h0=h1, lib=lib)
        assert np.array_equal(np.concatenate([o1, o2]), o) and np.array_equal(h2, hT)


def pin_varlen_packing(lib):
    """Packed sequences behave exactly as separate runs (chunks and states
    restart at each sequence start)."""
    H, Dk, Dv = 2, 4, 5
    lens = [7, 0, 13, 1]
    cu = np.concatenate([[0], np.cumsum(lens)])
    q, k, v, g, b = _rand_inputs(10, int(cu[-1]), H, Dk, Dv)
    h0 = _rng(11).standard_normal((len(lens), H, Dk, Dv))
    o, hT = oracle.forward(q, k, v, g, b, cu_seqlens=cu, h0=h0, lib=lib)
    for s, (a, e) in enumerate(zip(cu[:-1], cu[1:])):
        os_, hs = oracle.forward(q[a:e], k[a:e], v[a:e], g[a:e], b[a:e], h0=h0[s:s + 1], lib=lib)
        assert np.array_equal(o[a:e], os_) and np.array_equal(hT[s], hs[0])
    assert np.array_equal(hT[1], h0[1])  # empty sequence: state passes through


def pin_heads_independent(lib):
    """Heads never interact: each head of a multi-head run equals a one-head
    run on that head's slice (catches per-head stride and index mistakes)."""
    T, H, Dk, Dv = 11, 3, 4, 6
    q, k, v, g, b = _rand_inputs(18, T, H, Dk, Dv)
    z = _rng(19).standard_normal((T, H, Dk))
    A = np.array([-0.5, 0.1, 0.6])
    h0 = _rng(20).standard_normal((1, H, Dk, Dv))
    for gz, Al in ((g, None), (z, A)):
        o, hT = oracle.forward(q, k, v, gz, b, h0=h0, A_log=Al, lib=lib)
        for h in range(H):
            s = slice(h, h + 1)
            oh, hh = oracle.forward(q[:, s], k[:, s], v[:, s], gz[:, s], b[:, s], h0=h0[:, s],
                                    A_log=None if Al is None else Al[s], lib=lib)
            assert np.array_equal(o[:, s], oh) and np.array_equal(hT[:, s], hh)


def pin_causal_and_diagonal(lib):
    """o_t depends on no later token, and does depend on token t's own
    (k_t, v_t, beta_t): Tril in eq. (4) keeps the diagonal."""
    T, H, Dk, Dv = 12, 1, 4, 4
    q, k, v, g, b = _rand_inputs(12, T, H, Dk, Dv)
    o, _ = oracle.forward(q, k, v, g, b, lib=lib)
    v2 = v.copy(); v2[7:] += 1.0
    o2, _ = oracle.forward(q, k, v2, g, b, lib=lib)
    assert np.array_equal(o[:7], o2[:7])
    assert np.all(np.abs(o[7] - o2[7]) > 1e-6)


def pin_scale(lib):
    """scale multiplies the outputs only."""
    T, H, Dk, Dv = 9, 2, 3, 5
    q, k, v, g, b = _rand_inputs(13, T, H, Dk, Dv)
    o1, h1 = oracle.forward(q, k, v, g, b, lib=lib)
    o2, h2 = oracle.forward(q, k, v, g, b, scale=0.125, lib=lib)
    _close(o2, 0.125 * o1, 1e-14, "scale")
    assert np.array_equal(h1, h2)


def pin_per_head_gate(lib):
    """Decay-logit mode applies eq. (5) with each head's own A_h: equal to
    log-decay mode fed g = g_min * expit(exp(A_h) z) from scipy."""
    T, H, Dk, Dv = 10, 3, 4, 4
    q, k, v, _, b = _rand_inputs(14, T, H, Dk, Dv)
    z = _rng(15).standard_normal((T, H, Dk))
    A = np.array([-0.9, 0.2, 0.8])
    g = -5.0 * expit(np.exp(A)[None, :, None] * z)
    o1, h1 = oracle.forward(q, k, v, z, b, A_log=A, lib=lib)
    o2, h2 = oracle.forward(q, k, v, g, b, lib=lib)
    _close(o1, o2, 1e-13, "z-mode vs g-mode o")
    _close(h1, h2, 1e-13, "z-mode vs g-mode state")


def pin_chunked_form(lib):
    """The chunk-parallel form (eqs. (3)-(4), explicit UT transform) matches
    the token recurrence for chunk sizes 1, 7, 16 and 64, including ragged last
    chunks, d_k != d_v and a non-zero entering state."""
    T, Dk, Dv = 150, 8, 5
    q, k, v, g, b = _rand_inputs(16, T, 1, Dk, Dv)
    h0 = _rng(17).standard_normal((1, 1, Dk, Dv))
    o, hT = oracle.forward(q, k, v, g, b, h0=h0, scale=0.5, lib=lib)
    for C in (1, 7, 16, 64):
        oc, Sc = chunked_sequence(q[:, 0], k[:, 0], v[:, 0], g[:, 0], b[:, 0], h0[0, 0], C, scale=0.5)
        _close(oc, o[:, 0], 1e-11, f"chunked C={C} outputs")
        _close(Sc, hT[0, 0], 1e-11, f"chunked C={C} state")


ALL_PINS = [v for k_, v in sorted(globals().items()) if k_.startswith("pin_")]
