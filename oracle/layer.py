"""fp64 oracle of the KDA layer's input prologue and output epilogue.

TEST INFRASTRUCTURE ONLY (as the rest of ``oracle/``): nothing on the product
path imports it.

"Kimi K3 Technical Report: Open Frontier Intelligence", §2.1.1:

* eq. (2): per head, q = L2Norm(Swish(ShortConv(W_q x))), k likewise with W_k,
  v = Swish(ShortConv(W_v x)) (no normalisation), beta = Sigmoid(W_beta x),
  z = low-rank projection of x plus a per-head bias;
* eq. (6): y = W_o [Sigmoid(W_g x) * RMSNorm(o~)], with RMSNorm applied per head
  to the recurrence output o~;
* §2.3.2 states Swish(x) = x Sigmoid(x).

The dense projections (W_q x, W_k x, W_v x, W_beta x, the low-rank z, W_g x and
W_o) are matrix products outside this layer core; here they are inputs
("pre-activations").  Readings where the pages are silent:

* ShortConv is a causal depthwise convolution over time, one filter of width W
  per channel and no bias; ``conv_weight[c, W-1]`` multiplies the current
  token, ``conv_weight[c, W-1-j]`` the token j steps back.  The W - 1
  pre-activations before a sequence's first token come from a carried
  ``conv_state`` (zeros for a fresh sequence), and the state after a sequence
  is its last W - 1 pre-activations.
* L2Norm(y) = y / sqrt(sum(y^2) + eps) over the head's d_k channels.
* RMSNorm(o) = w * o / sqrt(mean(o^2) + eps) over the head's d_v channels, with a
  per-head weight w.

Channels of the convolution: per head, the d_k query channels, then the d_k key
channels, then the d_v value channels (one row of ``conv_weight`` each).
Every function here is pinned in tests/test_layer_oracle.py.
"""
from __future__ import annotations

import numpy as np

import oracle


def _f64(a):
    return np.asarray(a, dtype=np.float64)


def sigmoid(x):
    """Logistic function, elementwise (exp of a non-positive argument only)."""
    x = _f64(x)
    e = np.exp(-np.abs(x))
    return np.where(x >= 0, 1.0 / (1.0 + e), e / (1.0 + e))


def swish(x):
    """Swish(x) = x * Sigmoid(x) (§2.3.2)."""
    x = _f64(x)
    return x * sigmoid(x)


def l2norm(y, eps: float):
    """y / sqrt(sum(y^2) + eps) over the last axis."""
    y = _f64(y)
    return y / np.sqrt(np.sum(y * y, axis=-1, keepdims=True) + eps)


def rmsnorm(o, weight, eps: float):
    """weight * o / sqrt(mean(o^2) + eps) over the last axis."""
    o = _f64(o)
    return _f64(weight) * o / np.sqrt(np.mean(o * o, axis=-1, keepdims=True) + eps)


def short_conv(x, weight, state=None):
    """Causal depthwise convolution over time of one sequence.

    x: [T, ..., C] pre-activations; weight: [..., C, W]; state: [W-1, ..., C]
    (the pre-activations before token 0) or None for zeros.  Token t's output
    is sum_i weight[..., c, i] * x[t - (W-1) + i] with negative positions read
    from ``state``.  Returns (y [T, ..., C], state after the last token).
    """
    x = _f64(x)
    weight = _f64(weight)
    W = weight.shape[-1]
    T = x.shape[0]
    if state is None:
        state = np.zeros((W - 1,) + x.shape[1:])
    state = _f64(state)
    xt = np.concatenate([state, x], axis=0)        # position p at row p + W - 1
    y = np.zeros_like(x)
    for i in range(W):
        y += weight[..., i] * xt[i:i + T]
    return y, xt[T:T + W - 1].copy()


def prologue(q_pre, k_pre, v_pre, beta_logit, conv_weight, conv_state=None, qk_eps: float = 1e-6):
    """eq. (2) for one sequence, all heads.

    q_pre, k_pre: [T, H, Dk]; v_pre: [T, H, Dv]; beta_logit: [T, H];
    conv_weight: [H, 2*Dk + Dv, W]; conv_state: [H, W-1, 2*Dk + Dv] or None.
    Returns (q, k, v, beta, conv_state_out [H, W-1, 2*Dk + Dv]).
    """
    q_pre, k_pre, v_pre = _f64(q_pre), _f64(k_pre), _f64(v_pre)
    T, H, Dk = q_pre.shape
    W = conv_weight.shape[-1]
    x = np.concatenate([q_pre, k_pre, v_pre], axis=-1)           # [T, H, C]
    st = None if conv_state is None else np.transpose(_f64(conv_state), (1, 0, 2))
    c, st_out = short_conv(x, conv_weight, st)
    a = swish(c)
    q = l2norm(a[..., :Dk], qk_eps)
    k = l2norm(a[..., Dk:2 * Dk], qk_eps)
    v = a[..., 2 * Dk:]
    return q, k, v, sigmoid(beta_logit), np.transpose(st_out, (1, 0, 2)).reshape(H, W - 1, x.shape[-1])


def epilogue(o, gate_logit, o_weight, o_eps: float = 1e-6):
    """eq. (6) without W_o: Sigmoid(gate) * RMSNorm(o) per head.

    o, gate_logit: [..., H, Dv]; o_weight: [H, Dv]."""
    return sigmoid(gate_logit) * rmsnorm(o, o_weight, o_eps)


def layer_forward(q_pre, k_pre, v_pre, gz, beta_logit, *, conv_weight, conv_state=None,
                  cu_seqlens=None, h0=None, A_log=None, g_min: float = -5.0, scale: float = 1.0,
                  qk_eps: float = 1e-6, gate=None, o_weight=None, o_eps: float = 1e-6, nthreads: int = 0):
    """Prologue (eq. (2)), the recurrence (eq. (1), :func:`oracle.forward`) and,
    when ``gate`` is given, the epilogue (eq. (6)) over packed sequences.

    Token-major inputs [T, H, .] (a leading batch axis is flattened into B
    sequences of equal length); ``gz`` is as for :func:`oracle.forward`.
    conv_state: [N, H, W-1, 2*Dk + Dv] or None.
    Returns (y or o~ [T, H, Dv], hT [N, H, Dk, Dv], conv_state_out [N, H, W-1, 2*Dk + Dv]).
    """
    q_pre = _f64(q_pre)
    batched = q_pre.ndim == 4
    lead = q_pre.shape[:2]
    flat = lambda a: None if a is None else _f64(a).reshape((-1,) + _f64(a).shape[2:]) if batched else _f64(a)
    q_pre, k_pre, v_pre, gz, beta_logit = (flat(a) for a in (q_pre, k_pre, v_pre, gz, beta_logit))
    gate = flat(gate)
    Ttot, H, Dk = q_pre.shape
    Dv = v_pre.shape[-1]
    W = conv_weight.shape[-1]
    if cu_seqlens is None:
        cu_seqlens = np.arange(lead[0] + 1) * lead[1] if batched else np.array([0, Ttot])
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    N = cu.size - 1
    q = np.empty_like(q_pre)
    k = np.empty_like(k_pre)
    v = np.empty_like(v_pre)
    beta = np.empty_like(beta_logit)
    st_out = np.empty((N, H, W - 1, 2 * Dk + Dv))
    for s in range(N):
        a, b = cu[s], cu[s + 1]
        cs = None if conv_state is None else _f64(conv_state)[s]
        q[a:b], k[a:b], v[a:b], beta[a:b], st_out[s] = prologue(
            q_pre[a:b], k_pre[a:b], v_pre[a:b], beta_logit[a:b], conv_weight, cs, qk_eps)
    o, hT = oracle.forward(q, k, v, gz, beta, cu_seqlens=cu, h0=h0, A_log=A_log, g_min=g_min,
                           scale=scale, nthreads=nthreads)
    if gate is not None:
        o = epilogue(o, gate, o_weight, o_eps)
    if batched:
        o = o.reshape(lead + o.shape[1:])
    return o, hT, st_out
