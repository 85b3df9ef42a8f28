"""GPU parity of pair mode: from 128 (sequence, head) pairs at bf16 with
d_k = 128 (and no layer prologue) the inter-chunk recurrence and the output
("Kimi K3 Technical Report", §2.1.1, eqs. (1), (3)-(4)) run inside the
intra-chunk kernel, one workgroup walking whole pairs chunk by chunk.  These
cases hold that path against the fp64 oracle where the workloads do not reach:
d_v = 64, a carried initial state with sequences of 0, 1, 63-65 tokens and a
ragged tail, the log-decay gate input, and prefix-state checkpoints written by
the pair-mode chain step (§5.4.1)."""
import dataclasses

import numpy as np
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


def _lengths(n, seed, hi=300):
    """n packed lengths: the edge cases first, the rest uniform below hi."""
    r = np.random.default_rng(seed)
    lens = r.integers(0, hi, size=n)
    lens[:6] = [0, 1, 63, 64, 65, 129]
    return lens.tolist()


def _packed(lengths, H, seed, Dv=128):
    w = dataclasses.replace(W.WORKLOADS["varlen_64"], seed=seed, Dv=Dv)
    return W.make_prefill(w, device="cuda", H=H, lengths=lengths)


def _check(inp, z_mode=True):
    N = inp["cu_seqlens"].numel() - 1
    assert N * inp["q"].shape[-2] >= 128, "fewer pairs than pair mode needs"
    dt = inp["q"].dtype
    o, hT = gpu_prefill(inp, z_mode=z_mode)
    torch.cuda.synchronize()
    ro, rh, tok = oracle_prefill(inp, z_mode=z_mode)
    e_o = rel_err(np64(o)[tok.numpy()], ro)
    e_s = rel_err(np64(hT), rh)
    print(f"rel err o={e_o:.3e} state={e_s:.3e}")
    assert e_o <= TOL[dt] and e_s <= TOL[dt], (e_o, e_s)


@pytest.mark.parametrize("Dv", [128, 64])
def test_pair_mode_head_dims(Dv):
    """130 pairs (65 sequences x 2 heads), lengths 0..299 with the edge cases,
    initial state N(0, 0.02^2)."""
    inp = _packed(_lengths(65, 7 + Dv), H=2, seed=41 + Dv, Dv=Dv)
    _check(inp)


def test_pair_mode_logdecay_input():
    """The same path with g holding log-decays (no A_log), drawn in their range
    [g_min, 0] as -5 * U(0, 1)."""
    inp = _packed(_lengths(64, 9), H=2, seed=43)
    gen = torch.Generator(device="cuda").manual_seed(6)
    inp["z"] = (-5.0 * torch.rand(inp["z"].shape, generator=gen, device="cuda")).to(inp["q"].dtype)
    _check(inp, z_mode=False)


def test_pair_mode_long_pairs():
    """128 pairs of 1-10 chunks each (many chunk hand-offs inside a workgroup)."""
    inp = _packed(_lengths(32, 11, hi=640), H=4, seed=44)
    _check(inp)


def _prefix_state(inp, s, ntok):
    """Oracle state of packed sequence s after its first ntok tokens."""
    cu = inp["cu_seqlens"].to("cpu", torch.int64)
    t0 = int(cu[s])
    sub = dict(inp)
    for key in ("q", "k", "v", "z", "beta"):
        sub[key] = inp[key][t0:t0 + ntok]
    sub["cu_seqlens"] = torch.tensor([0, ntok], dtype=torch.int32, device=inp["q"].device)
    sub["h0"] = None if inp.get("h0") is None else inp["h0"][s:s + 1]
    _, hT, _ = oracle_prefill(sub)
    return hT[0]


def test_pair_mode_checkpoints():
    """Checkpoints every 2 chunks (128 tokens) from the pair-mode chain step:
    each written slot against the oracle's state over exactly that prefix,
    every slot past its sequence left untouched, and the outputs unchanged by
    writing them."""
    lengths = _lengths(64, 13, hi=600)
    inp = _packed(lengths, H=2, seed=45)
    N, H, Dk, Dv, every, slots = 64, 2, 128, 128, 2, 5
    o1, h1 = gpu_prefill(inp)
    ck = torch.full((N, slots, H, Dk, Dv), float("nan"), device="cuda")
    o2, h2 = gpu_prefill(inp, checkpoints=ck, checkpoint_every=every)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(h1, h2)
    tol = TOL[inp["q"].dtype]
    worst, checked = 0.0, 0
    for s, L in enumerate(lengths):
        for j in range(slots):
            pos = (j + 1) * every * 64
            if pos < L:
                e = rel_err(np64(ck[s, j]), _prefix_state(inp, s, pos))
                worst, checked = max(worst, e), checked + 1
                assert e <= tol, (s, j, e)
            else:
                assert torch.isnan(ck[s, j]).all(), (s, j)
    print(f"{checked} slots, worst checkpoint rel err {worst:.3e}")
    assert checked > 20


def test_pair_mode_partial_odd_round():
    """868 pairs (217 sequences x 4 heads): the workgroups take their pairs in
    rounds of 256, forwards on even rounds and backwards on odd ones, and the
    fourth round (odd) holds only 100 pairs, all on the high-numbered
    workgroups.  Every pair's output and final state against the oracle."""
    inp = _packed(_lengths(217, 17, hi=160), H=4, seed=46)
    _check(inp)
