"""Helpers shared by the GPU parity tests: tensor conversion, oracle calls on
the exact inputs the GPU received, and the relative error measure.

The error measure is max|gpu - oracle| / max|oracle| over the compared
elements; bounds are 1e-4 for fp32 inputs and 2e-2 for bf16 inputs with fp32
state and accumulation."""
import numpy as np
import torch

import oracle

TOL = {torch.float32: 1e-4, torch.bfloat16: 2e-2}


def np64(t):
    return None if t is None else t.detach().to("cpu", torch.float64).numpy()


def rel_err(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.max(np.abs(ref)) if ref.size else 0.0
    if den == 0.0:
        return float(np.max(np.abs(got))) if got.size else 0.0
    return float(np.max(np.abs(got - ref)) / den)


def oracle_prefill(inp, heads=None, seqs=None, z_mode=True, nthreads=0):
    """Oracle on the inputs dict of workloads.make_prefill (device or host
    tensors).  heads: optional list of head indices; seqs: optional list of
    sequence indices (packed layout).  Returns (o, hT) as numpy arrays laid
    out like the selection ([T_sel, H_sel, Dv], [N_sel, H_sel, Dk, Dv])."""
    q, k, v, z, b = (inp[x] for x in ("q", "k", "v", "z", "beta"))
    cu = inp.get("cu_seqlens")
    h0 = inp.get("h0")
    A = inp["A_log"] if z_mode else None
    if cu is None:  # [B, T, H, D] -> packed
        B, T = q.shape[:2]
        flat = lambda x: x.reshape((B * T,) + tuple(x.shape[2:]))
        q, k, v, z, b = (flat(x) for x in (q, k, v, z, b))
        cu = torch.arange(B + 1, dtype=torch.int64) * T
    cu = cu.to("cpu", torch.int64)
    hsel = slice(None) if heads is None else list(heads)
    if seqs is None:
        seqs = list(range(cu.numel() - 1))
    tok = torch.cat([torch.arange(int(cu[s]), int(cu[s + 1])) for s in seqs]) if seqs else torch.zeros(0, dtype=torch.int64)
    lens = [int(cu[s + 1] - cu[s]) for s in seqs]
    cu_sel = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    pick = lambda x: np64(x.index_select(0, tok.to(x.device))[:, hsel])
    qs, ks, vs, zs, bs = (pick(x) for x in (q, k, v, z, b))
    h0s = None if h0 is None else np64(h0[seqs][:, hsel])
    As = None if A is None else np64(A[hsel])
    o, hT = oracle.forward(qs, ks, vs, zs, bs, cu_seqlens=cu_sel, h0=h0s, A_log=As,
                           g_min=inp["g_min"], scale=inp.get("scale", 1.0), nthreads=nthreads)
    return o, hT, tok


def gpu_prefill(inp, z_mode=True, **kw):
    import gated_delta_rule_20_amd as kda
    return kda.chunk_fwd(inp["q"], inp["k"], inp["v"], inp["z"], inp["beta"],
                         A_log=inp["A_log"] if z_mode else None, g_min=inp["g_min"],
                         scale=inp.get("scale", 1.0), cu_seqlens=inp.get("cu_seqlens"),
                         initial_state=inp.get("h0"), **kw)


def to_device(inp, device="cuda"):
    out = {}
    for key, val in inp.items():
        out[key] = val.to(device) if isinstance(val, torch.Tensor) else val
    return out


class RunningErr:
    """max|got - ref| and max|ref| accumulated over pieces of a tensor, so the
    whole-tensor measure max|Δ| / max|ref| is formed without holding it."""

    def __init__(self):
        self.num = 0.0
        self.den = 0.0

    def add(self, got, ref):
        got = np.asarray(got, dtype=np.float64)
        ref = np.asarray(ref, dtype=np.float64)
        if ref.size:
            self.num = max(self.num, float(np.max(np.abs(got - ref))))
            self.den = max(self.den, float(np.max(np.abs(ref))))

    @property
    def rel(self):
        return self.num / self.den if self.den > 0 else self.num


def host64(t):
    """Device tensor -> contiguous fp64 numpy array (widened on the device, so
    only one copy crosses to the host)."""
    return t.contiguous().to(torch.float64).cpu().numpy()


def stream_prefill_parity(inp, o, hT, heads_per_call=4, nthreads=16, z_mode=True, log=print):
    """Whole-tensor parity of a prefill call against the oracle, streamed over
    groups of heads: every output token and every final state is compared, and
    only one group's fp64 copies are held at a time.  Returns
    (rel err of o, rel err of final state)."""
    q, k, v, z, b = (inp[x] for x in ("q", "k", "v", "z", "beta"))
    cu = inp.get("cu_seqlens")
    H = q.shape[-2]
    flat = lambda t: t.reshape((-1,) + tuple(t.shape[-2:]))
    q, k, v, z, o_f = (flat(x) for x in (q, k, v, z, o))
    b = b.reshape(-1, H)
    if cu is None:
        B, T = inp["q"].shape[:2]
        cu_np = np.arange(B + 1, dtype=np.int64) * T
    else:
        cu_np = cu.to("cpu", torch.int64).numpy()
    eo, es = RunningErr(), RunningErr()
    for h0_ in range(0, H, heads_per_call):
        sl = slice(h0_, min(H, h0_ + heads_per_call))
        ro, rh = oracle.forward(host64(q[:, sl]), host64(k[:, sl]), host64(v[:, sl]), host64(z[:, sl]),
                                host64(b[:, sl]), cu_seqlens=cu_np,
                                h0=None if inp.get("h0") is None else host64(inp["h0"][:, sl]),
                                A_log=host64(inp["A_log"][sl]) if z_mode else None, g_min=inp["g_min"],
                                scale=inp.get("scale", 1.0), nthreads=nthreads)
        eo.add(host64(o_f[:, sl]), ro)
        es.add(host64(hT[:, sl]), rh)
        del ro, rh
        log(f"heads {sl.start}..{sl.stop - 1}: running rel err o={eo.rel:.3e} state={es.rel:.3e}", flush=True)
    return eo.rel, es.rel


def epilogue_bound(o_ref, gate, o_weight, eps, core_tol):
    """Per-element bound on |y_gpu - y_ref| for the eq. (6) epilogue
    y = Sigmoid(gate) * w * o~ / sqrt(mean(o~^2) + eps) (per (token, head) row
    of d_v values), when the kernel's o~ may differ from the oracle's o~_ref by
    up to e = core_tol * max|o~_ref| (the core's whole-tensor bound).

    Derivation, per row with r = sqrt(mean(o~_ref^2) + eps), n = o~_ref / r and
    s = Sigmoid(gate) * w:  write o~ = o~_ref + d with |d|_inf <= e and
    r' = sqrt(mean(o~^2) + eps).  r and r' are Euclidean norms of
    (o~ / sqrt(d_v), sqrt(eps)), so |r - r'| <= rms(d) <= e (triangle
    inequality), hence r' >= r - e and
      |o~ / r' - o~_ref / r|_inf <= |d|_inf / r' + |o~_ref|_inf |r - r'| / (r r')
                                <= e (1 + |n|_inf) / (r - e)           (e < r).
    Both normalised rows have |.|_inf <= sqrt(d_v), so 2 sqrt(d_v) bounds the
    difference whatever e is.  Element j of y moves by at most |s_j| times
    that.  Returns (that deviation bound, |s|), shaped like o_ref; the caller
    adds the bf16 rounding of the output (2^-9 relative, taken as 2^-8 to
    cover the fp32 sigmoid and reciprocal square root)."""
    o_ref = np.asarray(o_ref, dtype=np.float64)
    s = np.abs(0.5 * (1.0 + np.tanh(0.5 * np.asarray(gate, dtype=np.float64))) * np.asarray(o_weight, dtype=np.float64))
    dv = o_ref.shape[-1]
    e = core_tol * float(np.max(np.abs(o_ref)))
    r = np.sqrt(np.mean(o_ref * o_ref, axis=-1, keepdims=True) + eps)
    n_inf = np.max(np.abs(o_ref), axis=-1, keepdims=True) / r
    bn = np.where(e < r, e * (1.0 + n_inf) / np.maximum(r - e, 1e-300), np.inf)
    bn = np.minimum(bn, 2.0 * np.sqrt(dv))
    return s * bn, s


def check_epilogue_end_to_end(y_gpu, o_ref, gate, o_weight, eps, core_tol):
    """y of the fused call against the oracle's y (its own epilogue of its own
    o~, no kernel intermediate), element by element within epilogue_bound.
    Returns (worst |Δy| / bound, whole-tensor max|Δy| / max|y_ref|)."""
    import oracle.layer as L
    y_ref = L.epilogue(o_ref, gate, o_weight, eps)
    dev, _ = epilogue_bound(o_ref, gate, o_weight, eps, core_tol)
    bound = dev + 2.0 ** -8 * (np.abs(y_ref) + dev)
    diff = np.abs(np.asarray(y_gpu, dtype=np.float64) - y_ref)
    ratio = float(np.max(diff / bound)) if diff.size else 0.0
    return ratio, rel_err(y_gpu, y_ref)
