"""GPU parity at the extremes of the gates ("Kimi K3 Technical Report", §2.1.1,
eqs. (1), (3)-(5) and the lower-bounded decay paragraph), each on the split
design (a few (sequence, head) pairs) and in pair mode (128 pairs or more):

* every channel of every token at the decay bound g = g_min, so that each
  16-token sub-tile spans the whole e^-80 range its reference allows;
* no decay at all (g = 0);
* no writes (beta = 0): the state only decays, S_t = Diag(exp(sum g)) S_0 and
  o_t = S_t^T q_t, a closed form;
* exact retrieval: alpha = beta = 1, S_0 = 0, and keys that are distinct signed
  unit vectors of the standard basis (orthonormal, and exact in bf16) with
  q_t = k_t, so that every product in the chunked form is exact and
  o_t = v_t, the final state holds v_i in row i's axis and zeros elsewhere:
  compared bit for bit; the same conditions also for 64 decode steps and for
  speculative windows (replayed tokens, then new tokens with any commit count).

Log-decay mode throughout (g is given, A_log = NULL), except for the in-place
resume check at the end (final state written over the initial one)."""
import dataclasses

import numpy as np
import pytest
import torch

import workloads as W
from kda_testutil import TOL, gpu_prefill, np64, oracle_prefill, rel_err

pytestmark = pytest.mark.gpu

MODES = ["split", "pair"]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gated_delta_rule_20_amd as kda
    kda.load_library()


def _inputs(mode, seed, max_len=300):
    """bf16, d_k = d_v = 128.  split: 3 sequences (0, 1 and a ragged length of
    several chunks) x 2 heads; pair: 65 sequences x 2 heads = 130 pairs with
    lengths 0, 1, 63, 64, 65, 129 and the rest uniform below max_len."""
    r = np.random.default_rng(seed)
    if mode == "split":
        lengths = [0, 1, int(min(max_len, 1000))]
    else:
        lengths = r.integers(0, max_len, size=65)
        lengths[:6] = [0, 1, 63, 64, 65, 129]
        lengths = np.minimum(lengths, max_len).tolist()
    w = dataclasses.replace(W.WORKLOADS["varlen_64"], seed=seed)
    return W.make_prefill(w, device="cuda", H=2, lengths=lengths)


def _check_oracle(inp):
    o, hT = gpu_prefill(inp, z_mode=False)
    torch.cuda.synchronize()
    ro, rh, tok = oracle_prefill(inp, z_mode=False)
    e_o = rel_err(np64(o)[tok.numpy()], ro)
    e_s = rel_err(np64(hT), rh)
    print(f"rel err o={e_o:.3e} state={e_s:.3e}")
    assert e_o <= TOL[torch.bfloat16] and e_s <= TOL[torch.bfloat16], (e_o, e_s)
    return o, hT


def _full(inp, value):
    return torch.full_like(inp["z"], value)


@pytest.mark.parametrize("mode", MODES)
def test_decay_at_the_bound_everywhere(mode):
    inp = _inputs(mode, 80)
    inp["z"] = _full(inp, inp["g_min"])
    _check_oracle(inp)


@pytest.mark.parametrize("mode", MODES)
def test_no_decay(mode):
    inp = _inputs(mode, 81)
    inp["z"] = _full(inp, 0.0)
    _check_oracle(inp)


@pytest.mark.parametrize("mode", MODES)
def test_no_writes_closed_form(mode):
    """beta = 0 with weak decay g = -U(0, 0.02): the entering state decays
    channel by channel and is read, never written."""
    inp = _inputs(mode, 82)
    gen = torch.Generator(device="cuda").manual_seed(82)
    inp["z"] = (-0.02 * torch.rand(inp["z"].shape, generator=gen, device="cuda")).to(torch.bfloat16)
    inp["beta"] = torch.zeros_like(inp["beta"])
    o, hT = _check_oracle(inp)
    # closed form in fp64 on the host, from the bf16 values the kernel read
    cu = inp["cu_seqlens"].to("cpu", torch.int64)
    q, g = np64(inp["q"]), np64(inp["z"])  # packed: [T, H, Dk]
    S0 = np64(inp["h0"])  # [N, H, Dk, Dv]
    o_ref = np.zeros(np64(o).shape)
    hT_ref = np.zeros(S0.shape)
    for s in range(cu.numel() - 1):
        a, b = int(cu[s]), int(cu[s + 1])
        G = np.cumsum(g[a:b], axis=0)  # [L, H, Dk]
        for h in range(S0.shape[1]):
            o_ref[a:b, h] = (q[a:b, h] * np.exp(G[:, h])) @ S0[s, h]
            hT_ref[s, h] = (np.exp(G[-1, h]) if b > a else np.ones(S0.shape[2]))[:, None] * S0[s, h]
    e_o = rel_err(np64(o), o_ref)
    e_s = rel_err(np64(hT), hT_ref)
    print(f"closed form: rel err o={e_o:.3e} state={e_s:.3e}")
    assert e_o <= TOL[torch.bfloat16] and e_s <= TOL[torch.bfloat16]


@pytest.mark.parametrize("mode", MODES)
def test_exact_retrieval_bitwise(mode):
    """alpha = beta = 1, S_0 = 0, q_t = k_t = +-e_{pi(t)} (a random permutation of
    the axes per (sequence, head), sequences of at most d_k = 128 tokens): the
    keys are orthonormal and exact in bf16, so L = 0, (I + L)^-1 = I, A = I,
    W S reads only unwritten rows, and o_t = v_t and the final state (row
    pi(i) = +-v_i) come out exactly."""
    inp = _inputs(mode, 83, max_len=128)
    cu = inp["cu_seqlens"].to("cpu", torch.int64)
    T, H, Dk = inp["k"].shape  # packed: [T, H, Dk]
    Dv = inp["v"].shape[-1]
    r = np.random.default_rng(83)
    keys = np.zeros((T, H, Dk), dtype=np.float32)
    S_ref = np.zeros((cu.numel() - 1, H, Dk, Dv), dtype=np.float32)
    v = inp["v"].float().cpu().numpy()
    for s in range(cu.numel() - 1):
        a, b = int(cu[s]), int(cu[s + 1])
        assert b - a <= Dk
        for h in range(H):
            axes = r.permutation(Dk)[: b - a]
            signs = r.choice([-1.0, 1.0], size=b - a)
            keys[np.arange(a, b), h, axes] = signs
            S_ref[s, h, axes] = signs[:, None] * v[a:b, h]
    k = torch.from_numpy(keys).to("cuda", torch.bfloat16)
    inp["k"] = k
    inp["q"] = k.clone()
    inp["z"] = _full(inp, 0.0)
    inp["beta"] = torch.ones_like(inp["beta"])
    inp["h0"] = torch.zeros_like(inp["h0"])
    o, hT = gpu_prefill(inp, z_mode=False)
    torch.cuda.synchronize()
    assert torch.equal(o, inp["v"]), float((o.float() - inp["v"].float()).abs().max())
    assert torch.equal(hT.cpu(), torch.from_numpy(S_ref))
    _check_oracle(inp)


def _basis_keys(r, N, T, H, Dk):
    """[N, T, H, Dk] keys: for each (sequence, head), T distinct signed basis
    vectors (a random permutation of the axes); also their axes and signs."""
    axes = np.stack([np.stack([r.permutation(Dk)[:T] for _ in range(H)], 1) for _ in range(N)])  # [N, T, H]
    signs = r.choice([-1.0, 1.0], size=(N, T, H))
    keys = np.zeros((N, T, H, Dk), np.float32)
    n, t, h = np.meshgrid(np.arange(N), np.arange(T), np.arange(H), indexing="ij")
    keys[n, t, h, axes] = signs
    return keys, axes, signs


def _write_rows(S, axes, signs, v):
    """S[n, h, axes[n, t, h]] = signs * v[n, t, h] for every t (host arrays)."""
    N, T, H = axes.shape
    for t in range(T):
        n, h = np.meshgrid(np.arange(N), np.arange(H), indexing="ij")
        S[n, h, axes[:, t, :]] = signs[:, t, :, None] * v[:, t, :]


def test_decode_exact_retrieval_bitwise():
    """The decode step under the same exact conditions (alpha = beta = 1, S_0 = 0,
    q = k = distinct signed basis vectors): 64 steps over 8 sequences x 4 heads,
    every step returns o = v and the state ends with +-v in the written rows and
    zeros elsewhere, bit for bit."""
    import gated_delta_rule_20_amd as kda
    N, H, Dk, Dv, steps = 8, 4, 128, 128, 64
    r = np.random.default_rng(84)
    gen = torch.Generator(device="cuda").manual_seed(84)
    keys, axes, signs = _basis_keys(r, N, steps, H, Dk)
    v = torch.randn(N, steps, H, Dv, generator=gen, device="cuda").to(torch.bfloat16)
    state = torch.zeros(N, H, Dk, Dv, device="cuda")
    g = torch.zeros(N, H, Dk, dtype=torch.bfloat16, device="cuda")   # log-decay 0: alpha = 1
    beta = torch.ones(N, H, dtype=torch.bfloat16, device="cuda")
    kk = torch.from_numpy(keys).to("cuda", torch.bfloat16)
    for t in range(steps):
        k = kk[:, t].contiguous()
        o = kda.recurrent_step(k, k, v[:, t].contiguous(), g, beta, state)
        torch.cuda.synchronize()
        assert torch.equal(o, v[:, t]), (t, float((o.float() - v[:, t].float()).abs().max()))
    S_ref = np.zeros((N, H, Dk, Dv), np.float32)
    _write_rows(S_ref, axes, signs, v.float().cpu().numpy())
    assert torch.equal(state.cpu(), torch.from_numpy(S_ref))


@pytest.mark.parametrize("n_commit", [0, 5, 8])
def test_replay_exact_retrieval_bitwise(n_commit):
    """The speculative window under the same exact conditions: 6 cached tokens
    replayed, then 8 new tokens with outputs, n_commit of them committed: every
    new token's output is its v, and the state written back holds the replayed
    and committed tokens' rows only, bit for bit."""
    import gated_delta_rule_20_amd as kda
    N, H, Dk, Dv, Tr, Tn = 8, 4, 128, 128, 6, 8
    r = np.random.default_rng(85 + n_commit)
    gen = torch.Generator(device="cuda").manual_seed(85 + n_commit)
    keys, axes, signs = _basis_keys(r, N, Tr + Tn, H, Dk)
    kk = torch.from_numpy(keys).to("cuda", torch.bfloat16)
    v = torch.randn(N, Tr + Tn, H, Dv, generator=gen, device="cuda").to(torch.bfloat16)
    g = torch.zeros(N, Tr + Tn, H, Dk, dtype=torch.bfloat16, device="cuda")
    beta = torch.ones(N, Tr + Tn, H, dtype=torch.bfloat16, device="cuda")
    new = lambda x: x[:, Tr:].contiguous()
    old = lambda x: x[:, :Tr].contiguous()
    state = torch.zeros(N, H, Dk, Dv, device="cuda")
    o = kda.recurrent_replay(new(kk), new(kk), new(v), new(g), new(beta), state,
                             replay=(old(kk), old(v), old(g), old(beta)), n_commit=n_commit)
    torch.cuda.synchronize()
    assert torch.equal(o, new(v)), float((o.float() - new(v).float()).abs().max())
    S_ref = np.zeros((N, H, Dk, Dv), np.float32)
    kept = Tr + n_commit
    _write_rows(S_ref, axes[:, :kept], signs[:, :kept], v[:, :kept].float().cpu().numpy())
    assert torch.equal(state.cpu(), torch.from_numpy(S_ref))


@pytest.mark.parametrize("mode,Dk", [("split", 128), ("pair", 128), ("pair", 64)])
def test_in_place_resume(mode, Dk):
    """final_state given as the very tensor of initial_state (in-place resume, as
    the header allows): outputs and state bit for bit equal to the call with a
    separate final state.  ("pair", 64): 130 pairs at d_k = 64 take the wide
    chain (pair mode needs d_k = 128)."""
    import gated_delta_rule_20_amd as kda
    inp = _inputs(mode, 86)
    if Dk != 128:
        inp["q"], inp["k"], inp["z"] = (inp[n][..., :Dk].contiguous() for n in ("q", "k", "z"))
        inp["h0"] = inp["h0"][:, :, :Dk].contiguous()
    o1, h1 = gpu_prefill(inp, z_mode=True)
    S = inp["h0"].clone()
    o2, h2 = kda.chunk_fwd(inp["q"], inp["k"], inp["v"], inp["z"], inp["beta"], A_log=inp["A_log"],
                           g_min=inp["g_min"], cu_seqlens=inp["cu_seqlens"], initial_state=S, final_state=S)
    torch.cuda.synchronize()
    assert h2.data_ptr() == S.data_ptr()
    assert torch.equal(o1, o2) and torch.equal(h1, S)
