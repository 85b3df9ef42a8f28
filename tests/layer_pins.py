"""Pins of the layer prologue/epilogue oracle (oracle/layer.py), each against
something other than the oracle itself: numpy's convolution, closed forms of
Swish, L2Norm and RMSNorm, cases of eq. (1) where the recurrence passes the
prologue's q (or k v^T) straight through, and the split and packing
invariants of a causal layer.

"Kimi K3 Technical Report: Open Frontier Intelligence", §2.1.1 eqs. (1), (2),
(6); Swish as defined in §2.3.2.  Every pin takes the layer module, so the
mutation test can run the suite on a planted mistake.
"""
import math

import numpy as np


def _rng(seed):
    return np.random.default_rng(seed)


def _close(a, b, tol, what):
    a, b = np.asarray(a, dtype=np.float64), np.asarray(b, dtype=np.float64)
    err = np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300)
    assert err <= tol, f"{what}: rel err {err:.3e} > {tol:.1e}"


def _ref_swish(x):
    return x / (1.0 + np.exp(-x))


def pin_conv_numpy(L):
    """Per channel the convolution is numpy.convolve over [state; x] with the
    taps reversed (numpy's convolution flips its kernel), 'valid' part."""
    r = _rng(1)
    T, C, W = 9, 5, 4
    x, w, st = r.normal(size=(T, C)), r.normal(size=(C, W)), r.normal(size=(W - 1, C))
    y, _ = L.short_conv(x, w, st)
    for c in range(C):
        ref = np.convolve(np.concatenate([st[:, c], x[:, c]]), w[c, ::-1], mode="valid")
        _close(y[:, c], ref, 1e-14, f"conv channel {c}")


def pin_conv_impulse(L):
    """A unit impulse at t = 0 from a zero state returns the taps newest-first:
    y_t = w[W-1-t] for t < W, then 0."""
    W, T = 4, 7
    w = np.array([[0.5, -2.0, 3.0, 7.0]])
    x = np.zeros((T, 1))
    x[0, 0] = 1.0
    y, _ = L.short_conv(x, w, None)
    assert np.array_equal(y[:, 0], [7.0, 3.0, -2.0, 0.5, 0.0, 0.0, 0.0]), y[:, 0]


def pin_conv_split(L):
    """Convolving [a; b] equals convolving a, then b from a's carried state;
    the carried state is the last W-1 inputs."""
    r = _rng(2)
    W, C = 4, 3
    a, b, w, s0 = r.normal(size=(5, C)), r.normal(size=(2, C)), r.normal(size=(C, W)), r.normal(size=(W - 1, C))
    y, s = L.short_conv(np.concatenate([a, b]), w, s0)
    ya, sa = L.short_conv(a, w, s0)
    yb, sb = L.short_conv(b, w, sa)
    assert np.array_equal(y, np.concatenate([ya, yb]))
    assert np.array_equal(s, sb)
    assert np.array_equal(sa, a[-(W - 1):])
    assert np.array_equal(sb, np.concatenate([a[-1:], b]))   # shorter than W-1: part of the old state stays


def pin_swish(L):
    """Swish(x) = x Sigmoid(x): Swish(0) = 0, Swish(x) - Swish(-x) = x,
    Sigmoid(ln 3) = 3/4; no overflow at large |x|."""
    assert L.swish(0.0) == 0.0
    x = np.linspace(-30, 30, 61)
    _close(L.swish(x) - L.swish(-x), x, 1e-14, "odd part of swish")
    _close(L.sigmoid(math.log(3.0)), 0.75, 1e-15, "sigmoid(ln 3)")
    _close(L.swish(math.log(3.0)), 0.75 * math.log(3.0), 1e-15, "swish(ln 3)")
    assert L.sigmoid(-800.0) == 0.0 and L.sigmoid(800.0) == 1.0


def pin_l2norm(L):
    """L2Norm: (3, 4) -> (0.6, 0.8); unit length and unchanged direction at
    eps = 0; eps enters under the root: (1e-4, 0) at eps 1e-8 -> 1/sqrt(2)."""
    _close(L.l2norm(np.array([3.0, 4.0]), 0.0), [0.6, 0.8], 1e-15, "(3,4)")
    _close(L.l2norm(np.array([1e-4, 0.0]), 1e-8), [1 / math.sqrt(2), 0.0], 1e-12, "eps")
    y = _rng(3).normal(size=(6, 16))
    n = L.l2norm(y, 0.0)
    _close(np.linalg.norm(n, axis=-1), np.ones(6), 1e-14, "unit norm")
    _close(n * np.linalg.norm(y, axis=-1, keepdims=True), y, 1e-14, "direction")


def pin_epilogue(L):
    """Sigmoid(gate) * RMSNorm(o): a constant row c maps to w sign(c) at
    eps = 0; the mean square of RMSNorm(o) / w is 1; gate ln 3 scales by 3/4;
    a positive rescaling of o changes nothing."""
    H, Dv = 2, 8
    w = np.arange(1, H * Dv + 1, dtype=np.float64).reshape(H, Dv)
    o = np.stack([np.full(Dv, -2.5), np.full(Dv, 0.3)])[None]          # [1, H, Dv]
    _close(L.epilogue(o, np.zeros_like(o), w, 0.0), 0.5 * w * np.sign(o), 1e-15, "constant row")
    _close(L.epilogue(o, np.full_like(o, math.log(3.0)), w, 0.0), 0.75 * w * np.sign(o), 1e-15, "gate")
    r = _rng(4)
    o = r.normal(size=(5, H, Dv))
    y = L.epilogue(o, np.zeros_like(o), np.ones((H, Dv)), 0.0)
    _close(np.mean((2 * y) ** 2, axis=-1), np.ones((5, H)), 1e-14, "unit mean square")
    _close(L.epilogue(7.0 * o, np.zeros_like(o), w, 0.0), y * w, 1e-14, "scale invariance and weight")


def _layer_inputs(seed, T, H, Dk, Dv, W=4):
    r = _rng(seed)
    return dict(q_pre=r.normal(size=(T, H, Dk)), k_pre=r.normal(size=(T, H, Dk)), v_pre=r.normal(size=(T, H, Dv)),
                gz=r.normal(size=(T, H, Dk)), beta_logit=r.normal(size=(T, H)),
                conv_weight=r.normal(scale=0.5, size=(H, 2 * Dk + Dv, W)))


def _conv_channel(x_seq, w_c, state_c):
    """Independent evaluation of one channel with numpy's convolution."""
    return np.convolve(np.concatenate([state_c, x_seq]), w_c[::-1], mode="valid")


def pin_layer_query_path(L):
    """With beta = 0 (logit -800), g = 0 and h0 = I, eq. (1) keeps S = I and
    o_t = q_t: the layer's output is the prologue's query,
    L2Norm(Swish(ShortConv(q_pre))), here built from numpy's convolution."""
    T, H, D, W = 6, 2, 8, 4
    x = _layer_inputs(5, T, H, D, D, W)
    st = _rng(6).normal(size=(1, H, W - 1, 3 * D))
    h0 = np.broadcast_to(np.eye(D), (1, H, D, D)).copy()
    o, hT, _ = L.layer_forward(x["q_pre"], x["k_pre"], x["v_pre"], np.zeros((T, H, D)), np.full((T, H), -800.0),
                               conv_weight=x["conv_weight"], conv_state=st, h0=h0, qk_eps=0.0)
    for h in range(H):
        c = np.stack([_conv_channel(x["q_pre"][:, h, j], x["conv_weight"][h, j], st[0, h, :, j]) for j in range(D)], 1)
        a = _ref_swish(c)
        _close(o[:, h], a / np.linalg.norm(a, axis=1, keepdims=True), 1e-13, f"query path head {h}")
    _close(hT, h0, 1e-15, "state unchanged")


def pin_layer_key_value_path(L):
    """One token from S_0 = 0 with g = 0: S_1 = Sigmoid(b) k v^T with
    k = L2Norm(Swish(conv(k_pre))) and v = Swish(conv(v_pre)), the
    convolution reading the carried state (channels Dk.. and 2Dk.. of it)."""
    H, Dk, Dv, W = 2, 4, 6, 3
    x = _layer_inputs(7, 1, H, Dk, Dv, W)
    st = _rng(8).normal(size=(1, H, W - 1, 2 * Dk + Dv))
    _, hT, _ = L.layer_forward(x["q_pre"], x["k_pre"], x["v_pre"], np.zeros((1, H, Dk)), x["beta_logit"],
                               conv_weight=x["conv_weight"], conv_state=st, qk_eps=0.0)
    for h in range(H):
        w = x["conv_weight"][h]
        ck = np.array([_conv_channel(x["k_pre"][:, h, j], w[Dk + j], st[0, h, :, Dk + j])[0] for j in range(Dk)])
        cv = np.array([_conv_channel(x["v_pre"][:, h, j], w[2 * Dk + j], st[0, h, :, 2 * Dk + j])[0]
                       for j in range(Dv)])
        k = _ref_swish(ck)
        k = k / np.linalg.norm(k)
        b = 1.0 / (1.0 + math.exp(-x["beta_logit"][0, h]))
        _close(hT[0, h], b * np.outer(k, _ref_swish(cv)), 1e-13, f"k v^T head {h}")


def pin_layer_split(L):
    """A causal layer: one pass over T tokens equals a pass over the first T1
    and a second one resumed from its final state and carried conv state
    (eq. (5) gate and eq. (6) epilogue on)."""
    T, T1, H, Dk, Dv = 11, 4, 2, 8, 4
    x = _layer_inputs(9, T, H, Dk, Dv)
    r = _rng(10)
    kw = dict(A_log=r.normal(size=H), gate=r.normal(size=(T, H, Dv)), o_weight=r.normal(size=(H, Dv)))
    st = r.normal(size=(1, H, 3, 2 * Dk + Dv))
    h0 = r.normal(scale=0.1, size=(1, H, Dk, Dv))
    args = lambda a, b: [x[n][a:b] for n in ("q_pre", "k_pre", "v_pre", "gz", "beta_logit")]
    sub = lambda a, b: dict(kw, gate=kw["gate"][a:b])
    o, hT, s = L.layer_forward(*args(0, T), conv_weight=x["conv_weight"], conv_state=st, h0=h0, **sub(0, T))
    o1, h1, s1 = L.layer_forward(*args(0, T1), conv_weight=x["conv_weight"], conv_state=st, h0=h0, **sub(0, T1))
    o2, h2, s2 = L.layer_forward(*args(T1, T), conv_weight=x["conv_weight"], conv_state=s1, h0=h1, **sub(T1, T))
    _close(np.concatenate([o1, o2]), o, 1e-12, "split outputs")
    _close(h2, hT, 1e-12, "split state")
    assert np.array_equal(s2, s)


def pin_layer_packing(L):
    """Packed sequences (cu_seqlens) with their own states equal separate runs."""
    H, Dk, Dv = 2, 4, 8
    lens = [3, 1, 6]
    cu = np.concatenate([[0], np.cumsum(lens)])
    x = _layer_inputs(11, cu[-1], H, Dk, Dv)
    r = _rng(12)
    st = r.normal(size=(3, H, 3, 2 * Dk + Dv))
    h0 = r.normal(scale=0.1, size=(3, H, Dk, Dv))
    gate, ow = r.normal(size=(cu[-1], H, Dv)), r.normal(size=(H, Dv))
    names = ("q_pre", "k_pre", "v_pre", "gz", "beta_logit")
    o, hT, s = L.layer_forward(*[x[n] for n in names], conv_weight=x["conv_weight"], conv_state=st,
                               cu_seqlens=cu, h0=h0, gate=gate, o_weight=ow)
    for i in range(3):
        a, b = cu[i], cu[i + 1]
        oi, hi, si = L.layer_forward(*[x[n][a:b] for n in names], conv_weight=x["conv_weight"],
                                     conv_state=st[i:i + 1], h0=h0[i:i + 1], gate=gate[a:b], o_weight=ow)
        _close(oi, o[a:b], 1e-14, f"sequence {i} outputs")
        _close(hi[0], hT[i], 1e-14, f"sequence {i} state")
        assert np.array_equal(si[0], s[i])


def pin_layer_gate_normalises(L):
    """With the epilogue on (weight 2, gate logit 0, eps 0) every output row has
    mean square 1 and the signs of the ungated output."""
    T, H, Dk, Dv = 5, 2, 8, 8
    x = _layer_inputs(13, T, H, Dk, Dv)
    names = ("q_pre", "k_pre", "v_pre", "gz", "beta_logit")
    h0 = _rng(14).normal(size=(1, H, Dk, Dv))
    o, _, _ = L.layer_forward(*[x[n] for n in names], conv_weight=x["conv_weight"], h0=h0)
    y, _, _ = L.layer_forward(*[x[n] for n in names], conv_weight=x["conv_weight"], h0=h0,
                              gate=np.zeros((T, H, Dv)), o_weight=np.full((H, Dv), 2.0), o_eps=0.0)
    _close(np.mean(y * y, axis=-1), np.ones((T, H)), 1e-13, "mean square")
    assert np.array_equal(np.sign(y), np.sign(o))


LAYER_PINS = [pin_conv_numpy, pin_conv_impulse, pin_conv_split, pin_swish, pin_l2norm, pin_epilogue,
              pin_layer_query_path, pin_layer_key_value_path, pin_layer_split, pin_layer_packing,
              pin_layer_gate_normalises]
