"""Seeded synthetic inputs for the KDA core (shared by tests, smoke and bench).

This module only draws random numbers and shapes them.  It contains none of
the method's arithmetic: no gate, no decay, no recurrence.  Decay logits z are
handed to the kernel (and to the oracle) as they are; both sides apply the
eq. (5) gate themselves.

Workloads (names state the shapes; all sizes per "Kimi K3 Technical Report:
Open Frontier Intelligence" §2.1.1 notation, d_k = d_v = d):

* ``tiny_fp32``      fp32, B=1, T=256, H=2, d=64, zero initial state, A_h = 0.
* ``prefill_8k``     bf16 q/k/v/z/beta, fp32 state, B=1, T=8192, H=32, d=128,
                     A_h ~ U(-1, 1) per head, initial state ~ N(0, 0.02^2).
* ``prefill_128k``   as prefill_8k with T=131072, plus 5% of (head, channel)
                     decay channels driven to hard forgetting and 5% to
                     near-unit retention (see ``_force_channels``).
* ``varlen_64``      64 packed sequences, lengths ~ U{128..16384} (the
                     length seed is picked so the total is ~530K tokens:
                     530,033), H=32, d=128, per-sequence initial states.
* ``decode_512``     512 sequences x 1 token per step, H=32, d=128, 64 steps
                     with fresh inputs, fp32 state [512, 32, 128, 128].
* ``decode_512_spec`` speculative decoding on the decode_512 shapes, 3 drafts
                     per step: per call, the cached window holds the previous
                     step's 3 drafts, of which 0..3 (uniform per sequence) were
                     accepted and are replayed; the new window holds 4 tokens
                     (the bonus token, which is certain and committed, and 3 new
                     drafts).  16 calls with fresh inputs.

Common distributions: q, k ~ N(0, 1) then L2-normalised over d_k per (token,
head) in fp32 (eq. (2) applies L2Norm before the core); v ~ N(0, 1);
beta = sigmoid(N(0, 1)); z ~ N(0, 1).  Values are drawn in fp32 with a torch
Generator on the requested device and then rounded to the workload dtype, so
a workload is reproducible per (seed, device type).
"""
from __future__ import annotations

import dataclasses
import math

import torch

G_MIN = -5.0


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    dtype: torch.dtype
    H: int
    Dk: int
    Dv: int
    seed: int
    B: int = 1
    T: int = 0                        # tokens per batch row (fixed-length)
    n_seqs: int = 0                   # varlen: number of packed sequences
    len_range: tuple = (0, 0)         # varlen: inclusive length range
    len_seed: int = 0                 # varlen: seed of the length draw
    zero_h0: bool = False
    A_uniform: float = 0.0            # A_h ~ U(-a, a); 0 -> A_h = 0
    h0_std: float = 0.02
    force_frac: float = 0.0           # fraction of channels forced each way
    decode_steps: int = 0             # decode: steps with fresh inputs
    chunk: int = 64

    @property
    def varlen(self) -> bool:
        return self.n_seqs > 0


WORKLOADS = {
    "tiny_fp32": Workload("tiny_fp32", torch.float32, H=2, Dk=64, Dv=64, seed=0,
                          B=1, T=256, zero_h0=True),
    "prefill_8k": Workload("prefill_8k", torch.bfloat16, H=32, Dk=128, Dv=128, seed=1,
                           B=1, T=8192, A_uniform=1.0),
    "prefill_128k": Workload("prefill_128k", torch.bfloat16, H=32, Dk=128, Dv=128, seed=2,
                             B=1, T=131072, A_uniform=1.0, force_frac=0.05),
    "varlen_64": Workload("varlen_64", torch.bfloat16, H=32, Dk=128, Dv=128, seed=3,
                          n_seqs=64, len_range=(128, 16384), len_seed=247, A_uniform=1.0),
    "decode_512": Workload("decode_512", torch.bfloat16, H=32, Dk=128, Dv=128, seed=4,
                           B=512, T=1, decode_steps=64),
    "decode_512_spec": Workload("decode_512_spec", torch.bfloat16, H=32, Dk=128, Dv=128, seed=5,
                                B=512, T=4, len_range=(0, 3), decode_steps=16),
}

# Decay logit that saturates the gate's sigmoid (hard forgetting, g = g_min),
# exactly representable in bf16.
Z_SATURATE = 30720.0
# Gate pre-activation whose sigmoid is ~2e-4, i.e. g ~ -1e-3 at g_min = -5
# (near-unit retention).  Solved once by hand: ln(2e-4 / (1 - 2e-4)).
X_NEAR_UNIT = -8.5170


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def _normal(shape, gen, device):
    return torch.randn(shape, generator=gen, device=device, dtype=torch.float32)


def _unit_rows(x):
    return x / x.norm(dim=-1, keepdim=True).clamp_min(1e-12)


def _force_channels(z, A, frac, gen, device):
    """Force two disjoint sets of (head, channel) decay channels, each a
    fraction ``frac`` of all H*Dk channels, for every token: one to hard
    forgetting (z saturating the sigmoid), one to near-unit retention (the
    logit chosen so that exp(A_h) * z = X_NEAR_UNIT)."""
    T, H, Dk = z.shape[-3:]
    n = int(round(frac * H * Dk))
    perm = torch.randperm(H * Dk, generator=gen, device=device)
    hard, soft = perm[:n], perm[n:2 * n]
    zf = z.reshape(-1, H * Dk)
    zf[:, hard] = Z_SATURATE
    heads = soft // Dk
    zf[:, soft] = X_NEAR_UNIT * torch.exp(-A[heads])
    return z, hard, soft


def varlen_lengths(w: Workload, device="cpu") -> torch.Tensor:
    """Sequence lengths ~ U{lo..hi}, drawn on the CPU so they do not depend
    on the device; the seed is the workload's ``len_seed``."""
    gen = _gen(w.len_seed, "cpu")
    lo, hi = w.len_range
    return torch.randint(lo, hi + 1, (w.n_seqs,), generator=gen).to(device)


def make_prefill(w: Workload, device="cpu", T: int | None = None, H: int | None = None,
                 n_seqs: int | None = None, lengths=None):
    """Inputs of one prefill call.  Optional overrides shrink a workload for
    fast tests while keeping its distributions (T: tokens per row, H: heads,
    n_seqs / lengths: packed sequences)."""
    H = H or w.H
    gen = _gen(w.seed, device)
    if w.varlen or lengths is not None:
        if lengths is None:
            lengths = varlen_lengths(w, device)
            if n_seqs is not None:
                lengths = lengths[:n_seqs]
        lengths = torch.as_tensor(lengths, dtype=torch.int64, device=device)
        cu = torch.zeros(lengths.numel() + 1, dtype=torch.int64, device=device)
        cu[1:] = torch.cumsum(lengths, 0)
        Btot, Ttok, N = 1, int(cu[-1].item()), lengths.numel()
        gen.manual_seed(w.seed + 1000003)
    else:
        cu = None
        Btot, Ttok = w.B, (T or w.T)
        N = Btot
    shp_k = (Btot, Ttok, H, w.Dk)
    shp_v = (Btot, Ttok, H, w.Dv)
    q = _unit_rows(_normal(shp_k, gen, device))
    k = _unit_rows(_normal(shp_k, gen, device))
    v = _normal(shp_v, gen, device)
    beta = torch.sigmoid(_normal((Btot, Ttok, H), gen, device))
    z = _normal(shp_k, gen, device)
    if w.A_uniform > 0:
        A = (torch.rand((H,), generator=gen, device=device) * 2 - 1) * w.A_uniform
    else:
        A = torch.zeros((H,), device=device)
    forced = None
    if w.force_frac > 0:
        z, hard, soft = _force_channels(z, A, w.force_frac, gen, device)
        forced = (hard, soft)
    h0 = None
    if not w.zero_h0:
        h0 = _normal((N, H, w.Dk, w.Dv), gen, device) * w.h0_std
    dt = w.dtype
    out = dict(q=q.to(dt), k=k.to(dt), v=v.to(dt), z=z.to(dt), beta=beta.to(dt),
               A_log=A.float(), h0=h0, cu_seqlens=None if cu is None else cu.to(torch.int32),
               forced=forced, g_min=G_MIN)
    if cu is not None:  # packed layout: batch axis of 1
        for key in ("q", "k", "v", "z", "beta"):
            out[key] = out[key].reshape(out[key].shape[1:])
    return out


def make_decode(w: Workload, device="cpu", N: int | None = None, H: int | None = None,
                steps: int | None = None):
    """State and per-step inputs of the decode workload.  Returns dict with
    ``state`` [N, H, Dk, Dv] fp32 and ``steps``: a list of per-step dicts with
    q, k, z [N, H, Dk], v [N, H, Dv], beta [N, H] in the workload dtype."""
    N = N or w.B
    H = H or w.H
    steps = steps or w.decode_steps
    gen = _gen(w.seed, device)
    state = _normal((N, H, w.Dk, w.Dv), gen, device) * w.h0_std
    A = torch.zeros((H,), device=device)
    per = []
    dt = w.dtype
    for _ in range(steps):
        q = _unit_rows(_normal((N, H, w.Dk), gen, device))
        k = _unit_rows(_normal((N, H, w.Dk), gen, device))
        v = _normal((N, H, w.Dv), gen, device)
        beta = torch.sigmoid(_normal((N, H), gen, device))
        z = _normal((N, H, w.Dk), gen, device)
        per.append(dict(q=q.to(dt), k=k.to(dt), v=v.to(dt), z=z.to(dt), beta=beta.to(dt)))
    return dict(state=state, A_log=A, steps=per, g_min=G_MIN)


def n_tokens(inp) -> int:
    q = inp["q"]
    return int(math.prod(q.shape[:-2]))



def make_spec_decode(w: Workload, device="cpu", N: int | None = None, H: int | None = None,
                     T_replay: int | None = None, T_new: int | None = None, calls: int | None = None,
                     accept_range=None):
    """State and per-call inputs of a speculative-decoding workload.  Returns
    dict with ``state`` [N, H, Dk, Dv] fp32 and ``calls``: a list of dicts,
    each with the cached window (k_r, z_r [N, Tr, H, Dk], v_r [N, Tr, H, Dv],
    beta_r [N, Tr, H]; Tr defaults to the workload's window minus the bonus
    token), ``n_replay`` [N] int32 (accepted drafts, drawn on the CPU from
    ``accept_range``, inclusive) and the new window (q, k, z, v, beta shaped
    like the cached window with T_new tokens)."""
    N = N or w.B
    H = H or w.H
    T_new = w.T if T_new is None else T_new
    T_replay = w.T - 1 if T_replay is None else T_replay
    calls = calls or w.decode_steps
    lo, hi = accept_range or w.len_range
    gen = _gen(w.seed, device)
    cpu = _gen(w.seed + 7, "cpu")
    state = _normal((N, H, w.Dk, w.Dv), gen, device) * w.h0_std
    A = (torch.rand((H,), generator=gen, device=device) * 2 - 1) * w.A_uniform if w.A_uniform > 0 \
        else torch.zeros((H,), device=device)
    dt = w.dtype

    def window(T):
        q = _unit_rows(_normal((N, T, H, w.Dk), gen, device))
        k = _unit_rows(_normal((N, T, H, w.Dk), gen, device))
        v = _normal((N, T, H, w.Dv), gen, device)
        beta = torch.sigmoid(_normal((N, T, H), gen, device))
        z = _normal((N, T, H, w.Dk), gen, device)
        return dict(q=q.to(dt), k=k.to(dt), v=v.to(dt), z=z.to(dt), beta=beta.to(dt))

    out = []
    for _ in range(calls):
        old, new = window(T_replay), window(T_new)
        n_rep = torch.randint(lo, hi + 1, (N,), generator=cpu, dtype=torch.int32)
        out.append(dict(k_r=old["k"], v_r=old["v"], z_r=old["z"], beta_r=old["beta"],
                        n_replay=n_rep.to(device), q=new["q"], k=new["k"], v=new["v"], z=new["z"],
                        beta=new["beta"]))
    return dict(state=state, A_log=A.float(), calls=out, g_min=G_MIN)


def make_layer(w: Workload, device="cpu", N: int | None = None, T: int | None = None, H: int | None = None,
               conv_width: int = 4, seed_offset: int = 0):
    """Inputs of the layer around the core (eq. (2) prologue, eq. (6) epilogue)
    on the workload's shapes: token-major [N, T, H, .] tensors in the workload
    dtype.  The dense projections are not modelled: their outputs are drawn
    directly.  Returns dict with
      q_pre, k_pre, z [N, T, H, Dk]; v_pre, gate [N, T, H, Dv]; beta_logit [N, T, H]
          (projections W x ~ N(0, 1), decay logits z ~ N(0, 1), gate logits ~ N(0, 1));
      conv_weight [H, 2*Dk + Dv, W] fp32 (taps ~ N(0, 0.5^2));
      conv_state [N, H, W-1, 2*Dk + Dv] (pre-activations ~ N(0, 1));
      o_norm_weight [H, Dv] fp32 (1 + N(0, 0.1^2));
      state [N, H, Dk, Dv] fp32 (N(0, h0_std^2)); A_log [H] (U(-a, a)); g_min.
    """
    N = N or w.B
    T = w.T if T is None else T
    H = H or w.H
    gen = _gen(w.seed + 1000 + seed_offset, device)
    dt = w.dtype
    C = 2 * w.Dk + w.Dv
    nrm = lambda *shape: _normal(shape, gen, device)
    out = dict(
        q_pre=nrm(N, T, H, w.Dk).to(dt), k_pre=nrm(N, T, H, w.Dk).to(dt), v_pre=nrm(N, T, H, w.Dv).to(dt),
        z=nrm(N, T, H, w.Dk).to(dt), beta_logit=nrm(N, T, H).to(dt), gate=nrm(N, T, H, w.Dv).to(dt),
        conv_weight=nrm(H, C, conv_width) * 0.5,
        conv_state=nrm(N, H, conv_width - 1, C).to(dt),
        o_norm_weight=1.0 + 0.1 * nrm(H, w.Dv),
        state=nrm(N, H, w.Dk, w.Dv) * w.h0_std,
        A_log=(torch.rand((H,), generator=gen, device=device) * 2 - 1) * w.A_uniform if w.A_uniform > 0
        else torch.zeros((H,), device=device),
        g_min=G_MIN)
    return out
