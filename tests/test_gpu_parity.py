"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Small cases span several chunks, ragged tails, every head-dim combination,
both gate modes, packed sequences, split/resume and decode-vs-prefill; the
full-size workloads are compared on sampled (sequence, head) pairs."""
import numpy as np
import pytest
import torch

import workloads as W
from kda_testutil import TOL, gpu_prefill, np64, oracle_prefill, rel_err, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gated_delta_rule_20_amd as kda
    kda.load_library()


def _small(name, T=None, H=None, seed=None, device="cuda", **kw):
    w = W.WORKLOADS[name]
    if seed is not None:
        import dataclasses
        w = dataclasses.replace(w, seed=seed)
    return W.make_prefill(w, device=device, T=T, H=H, **kw)


def _check(inp, z_mode=True, heads=None):
    dt = inp["q"].dtype
    o, hT = gpu_prefill(inp, z_mode=z_mode)
    torch.cuda.synchronize()
    ro, rh, tok = oracle_prefill(inp, heads=heads, z_mode=z_mode)
    go = np64(o)
    if inp.get("cu_seqlens") is None:
        go = go.reshape((-1,) + go.shape[2:])
    hs = slice(None) if heads is None else list(heads)
    e_o = rel_err(go[tok.numpy()][:, hs], ro)
    e_s = rel_err(np64(hT)[:, hs], rh)
    print(f"rel err o={e_o:.3e} state={e_s:.3e}")
    assert e_o <= TOL[dt] and e_s <= TOL[dt], (e_o, e_s)
    return o, hT


def test_tiny_fp32_prefill():
    """Tiny fp32 workload (T=256, H=2, d=64), zero initial state, A_h = 0."""
    _check(_small("tiny_fp32"))


@pytest.mark.parametrize("T", [1, 17, 64, 65, 200, 1000])
def test_bf16_prefill_ragged(T):
    _check(_small("prefill_8k", T=T, H=4, seed=100 + T))


@pytest.mark.parametrize("Dk,Dv", [(64, 64), (64, 128), (128, 64)])
def test_bf16_head_dims(Dk, Dv):
    import dataclasses
    w = dataclasses.replace(W.WORKLOADS["prefill_8k"], Dk=Dk, Dv=Dv, seed=7)
    _check(W.make_prefill(w, device="cuda", T=333, H=3))


def test_fp32_prefill_ragged_with_state():
    import dataclasses
    w = dataclasses.replace(W.WORKLOADS["tiny_fp32"], zero_h0=False, A_uniform=1.0, seed=9)
    _check(W.make_prefill(w, device="cuda", T=301, H=3))


def test_logdecay_mode():
    """g given directly (A_log = NULL), drawn as -5 * U(0, 1)."""
    inp = _small("prefill_8k", T=300, H=4, seed=11)
    gen = torch.Generator(device="cuda").manual_seed(5)
    inp["z"] = (-5.0 * torch.rand(inp["z"].shape, generator=gen, device="cuda")).to(inp["q"].dtype)
    _check(inp, z_mode=False)


@pytest.mark.parametrize("dt", ["prefill_8k", "tiny_fp32"])
def test_weak_decay_long_memory(dt):
    """Log-decays g ~ -U(0, 0.002) and beta / 10: the state carries information over
    hundreds of tokens, so every chunk-to-chunk hand-off of the chain shows in the
    output (with the workloads' own gates the state forgets within ~10 tokens)."""
    inp = _small(dt, T=1000, H=3, seed=13)
    gen = torch.Generator(device="cuda").manual_seed(6)
    inp["z"] = (-0.002 * torch.rand(inp["z"].shape, generator=gen, device="cuda")).to(inp["q"].dtype)
    inp["beta"] = (inp["beta"].float() * 0.1).to(inp["q"].dtype)
    _check(inp, z_mode=False)


def test_forced_channels_short():
    """Hard-forgetting (g = -5) and near-unit (g ~ -1e-3) channels stress the
    range of the cumulative decay."""
    _check(_small("prefill_128k", T=700, H=4))


def test_varlen_small():
    lengths = [1, 64, 130, 0, 257, 5, 63, 64]
    inp = _small("varlen_64", H=3, lengths=lengths)
    _check(inp)


def test_varlen_many_sequences():
    """2100 packed sequences, past the 2048 up to which the chunk table sorts
    sequences longest first (beyond it they keep their given order): lengths
    0..39 with 40 at or around one and two chunks."""
    r = np.random.default_rng(31)
    lengths = r.integers(0, 40, size=2100)
    lengths[r.choice(2100, 40, replace=False)] = r.choice([63, 64, 65, 128, 129], 40)
    inp = _small("varlen_64", H=2, seed=31, lengths=lengths.tolist())
    _check(inp)


def test_query_scale():
    inp = _small("prefill_8k", T=150, H=2, seed=12)
    inp["scale"] = 0.0883883476
    _check(inp)


def test_zero_length_passes_state():
    inp = _small("prefill_8k", T=64, H=2, seed=13)
    for key in ("q", "k", "v", "z", "beta"):
        inp[key] = inp[key][:, :0].contiguous()
    o, hT = gpu_prefill(inp)
    torch.cuda.synchronize()
    assert o.numel() == 0 and torch.equal(hT, inp["h0"])


def test_split_resume_equals_one_pass():
    """Two calls split at a chunk boundary, the second resuming (in place) from
    the first's final state, match one call."""
    inp = _small("prefill_8k", T=512, H=4, seed=14)
    o, hT = gpu_prefill(inp)
    first = {k_: (v_[:, :192].contiguous() if k_ in ("q", "k", "v", "z", "beta") else v_) for k_, v_ in inp.items()}
    second = {k_: (v_[:, 192:].contiguous() if k_ in ("q", "k", "v", "z", "beta") else v_) for k_, v_ in inp.items()}
    o1, h1 = gpu_prefill(first)
    second["h0"] = h1
    import gated_delta_rule_20_amd as kda
    o2, h2 = kda.chunk_fwd(second["q"], second["k"], second["v"], second["z"], second["beta"],
                           A_log=second["A_log"], initial_state=h1, final_state=h1)
    torch.cuda.synchronize()
    tol = TOL[torch.bfloat16]
    assert rel_err(np64(torch.cat([o1, o2], 1)), np64(o)) <= tol
    assert rel_err(np64(h2), np64(hT)) <= tol


def test_deterministic_and_fully_written():
    inp = _small("prefill_8k", T=333, H=4, seed=15)
    out = torch.full(inp["v"].shape, float("nan"), dtype=inp["v"].dtype, device="cuda")
    fin = torch.full(inp["h0"].shape, float("nan"), device="cuda")
    o1, h1 = gpu_prefill(inp, out=out, final_state=fin)
    o2, h2 = gpu_prefill(inp)
    torch.cuda.synchronize()
    assert not torch.isnan(o1).any() and not torch.isnan(h1).any()
    assert torch.equal(o1, o2) and torch.equal(h1, h2)


# --- decode -------------------------------------------------------------------

def _decode_oracle(state0, steps, A, heads=None, seqs=None):
    """Run the oracle over the decode steps for selected (sequence, head)s."""
    import oracle
    hs = slice(None) if heads is None else list(heads)
    ss = slice(None) if seqs is None else list(seqs)
    S = np64(state0[ss][:, hs])
    outs = []
    for st in steps:
        sel = lambda x: np64(x[ss][:, hs])
        q, k, v, z, b = (sel(st[x]) for x in ("q", "k", "v", "z", "beta"))
        N = q.shape[0]
        cu = np.arange(N + 1, dtype=np.int64)
        o, S = oracle.forward(q, k, v, z, b, cu_seqlens=cu, h0=S, A_log=np64(A[hs]))
        outs.append(o)
    return outs, S


@pytest.mark.parametrize("dtype,Dk,Dv", [(torch.bfloat16, 128, 128), (torch.float32, 64, 64),
                                          (torch.bfloat16, 64, 128), (torch.float32, 128, 64)])
def test_decode_small(dtype, Dk, Dv):
    import dataclasses
    import gated_delta_rule_20_amd as kda
    w = dataclasses.replace(W.WORKLOADS["decode_512"], dtype=dtype, Dk=Dk, Dv=Dv)
    d = W.make_decode(w, device="cuda", N=5, H=3, steps=4)
    state = d["state"].clone()
    ref_o, ref_S = _decode_oracle(d["state"], d["steps"], d["A_log"])
    for i, st in enumerate(d["steps"]):
        o = kda.recurrent_step(st["q"], st["k"], st["v"], st["z"], st["beta"], state, A_log=d["A_log"])
        torch.cuda.synchronize()
        assert rel_err(np64(o), ref_o[i]) <= TOL[dtype]
    assert rel_err(np64(state), ref_S) <= TOL[dtype]


def test_tiny_fp32_as_decode_steps():
    """The tiny fp32 workload run as 256 single-token steps matches the oracle
    and the chunked prefill of the same tokens."""
    import gated_delta_rule_20_amd as kda
    inp = _small("tiny_fp32")
    o_pre, h_pre = gpu_prefill(inp)
    T, H = inp["q"].shape[1], inp["q"].shape[2]
    state = torch.zeros(1, H, 64, 64, device="cuda")
    outs = []
    for t in range(T):
        sl = lambda x: x[:, t].contiguous()
        outs.append(kda.recurrent_step(sl(inp["q"]), sl(inp["k"]), sl(inp["v"]), sl(inp["z"]),
                                       sl(inp["beta"]), state, A_log=inp["A_log"]))
    torch.cuda.synchronize()
    o_dec = torch.stack(outs, 1)
    ro, rh, _ = oracle_prefill(inp)
    assert rel_err(np64(o_dec)[0], ro) <= 1e-4
    assert rel_err(np64(state), rh) <= 1e-4
    assert rel_err(np64(o_dec), np64(o_pre)) <= 1e-4
    assert rel_err(np64(state), np64(h_pre)) <= 1e-4
