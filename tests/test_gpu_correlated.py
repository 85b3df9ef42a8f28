"""GPU parity with strongly correlated keys, where the chunk's triangular
system (I + L) is far from the identity: within a 16-token tile the strictly
lower part of L approaches the all-ones matrix, whose powers grow binomially
(the finite product for the diagonal inverses then cancels large terms), and
the inverse of the whole chunk couples every token.  Runs of one repeated key
are what a repeated token gives.  Checked against the fp64 oracle on the
split design and in pair mode.

A whole 64-token chunk on one key, with beta = 1 and no decay, is held to a
looser bound than the 2e-2 of the workloads.  There T' = (I + L)^-1 Diag(beta)
is close to the difference operator, the pseudo-values are differences of
consecutive values (V~_r ~ v_r - v_(r-1)), and the output of token r sums them
over the chunk's first r + 1 tokens (A_ri = q.k).  Each V~_r carries bf16
roundings of relative size 2^-9: T''s subdiagonal -beta |k|^2 as an MFMA
operand (so the difference no longer cancels exactly), U, and V~ as an
operand.  The sum then carries about sqrt(r + 1) independent roundings: for
r = 63 about 8 * 2 * 2^-9 * sqrt(2) ~ 0.044 of max|v|, which is what the
kernels measure (2e-2 to 5e-2).  The test bounds it at 0.1, which guards
against a blow-up, not against this accumulation."""
import dataclasses

import pytest
import torch

import workloads as W
from kda_testutil import TOL, gpu_prefill, np64, oracle_prefill, rel_err

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gated_delta_rule_20_amd as kda
    kda.load_library()


def _check(inp, z_mode, tol=None):
    dt = inp["q"].dtype
    tol = TOL[dt] if tol is None else tol
    o, hT = gpu_prefill(inp, z_mode=z_mode)
    torch.cuda.synchronize()
    ro, rh, _ = oracle_prefill(inp, z_mode=z_mode)
    go = np64(o)
    if inp.get("cu_seqlens") is None:
        go = go.reshape((-1,) + go.shape[2:])
    e_o, e_s = rel_err(go, ro), rel_err(np64(hT), rh)
    print(f"rel err o={e_o:.3e} state={e_s:.3e}")
    assert e_o <= tol and e_s <= tol, (e_o, e_s)


def _unit(x):
    return x / x.norm(dim=-1, keepdim=True)


def _inputs(kind, seed):
    if kind == "split":
        w = dataclasses.replace(W.WORKLOADS["prefill_8k"], seed=seed)
        return W.make_prefill(w, "cuda", T=520, H=2)
    w = dataclasses.replace(W.WORKLOADS["varlen_64"], seed=seed)
    lens = torch.randint(60, 260, (64,), generator=torch.Generator().manual_seed(seed))
    return W.make_prefill(w, "cuda", H=2, lengths=lens)


def _runs_of_one_key(k, run):
    """Tokens in runs of `run` share one key (per head): [.., T, H, D] -> same shape."""
    T = k.shape[-3]
    idx = (torch.arange(T, device=k.device) // run) * run
    return k.index_select(-3, idx).contiguous()


@pytest.mark.parametrize("kind", ["split", "pair"])
@pytest.mark.parametrize("run", [16, 64])
def test_repeated_keys_full_retention(kind, run):
    """Runs of 16 or 64 tokens with one key, beta = 1 and no decay (log-decay
    input g = 0): every tile's L is the all-ones strict lower triangle.  Runs
    of a whole chunk get the looser bound of the module docstring."""
    inp = _inputs(kind, 60 + run)
    inp["k"] = _runs_of_one_key(inp["k"], run)
    inp["beta"] = torch.ones_like(inp["beta"])
    inp["z"] = torch.zeros_like(inp["z"])
    _check(inp, z_mode=False, tol=0.1 if run == 64 else None)


@pytest.mark.parametrize("kind", ["split", "pair"])
def test_correlated_keys_workload_gates(kind):
    """Keys of one head within 0.05 of a common direction, beta in [0.5, 1], the
    workloads' own eq. (5) gates."""
    inp = _inputs(kind, 70)
    gen = torch.Generator(device="cuda").manual_seed(71)
    k = inp["k"].float()
    base = _unit(torch.randn(k.shape[-2:], generator=gen, device="cuda"))  # [H, D]
    noise = torch.randn(k.shape, generator=gen, device="cuda")
    inp["k"] = _unit(base + 0.05 * noise).to(inp["q"].dtype)
    inp["beta"] = (0.5 + 0.5 * torch.rand(inp["beta"].shape, generator=gen, device="cuda")).to(inp["q"].dtype)
    _check(inp, z_mode=True)
