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
