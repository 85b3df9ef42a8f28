"""The per-GPU share of KDA context parallelism at the real head size
("Kimi K3 Technical Report", §5.1.2, KCP, eq. (17)): a segment's effect on the
state is affine, S_out = M S_in + S~, with M the product of the per-token
transitions (I - beta k k^T) Diag(alpha) and S~ the state the segment produces
from zero.  Both are computed with the prefill path itself:
  S~ = final state from S_in = 0 with the segment's real v,
  M  = final state from S_in = I with v = 0 (d_v = d_k),
and segments merged in order then re-run from their true entering state must
reproduce the single pass.  The merge is done here in fp32 with torch on the
device: on several GPUs it is the all-gather plus prefix merge of eq. (17),
which is not implemented here (one GPU)."""
import dataclasses

import pytest
import torch

import workloads as W
from kda_testutil import TOL, np64, oracle_prefill, rel_err

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gated_delta_rule_20_amd as kda
    kda.load_library()


def _seg(inp, t0, t1):
    return {k: (v[:, t0:t1].contiguous() if k in ("q", "k", "v", "z", "beta") else v) for k, v in inp.items()}


def _run(inp, h0, v=None):
    import gated_delta_rule_20_amd as kda
    o, hT = kda.chunk_fwd(inp["q"], inp["k"], inp["v"] if v is None else v, inp["z"], inp["beta"],
                          A_log=None, g_min=inp["g_min"], initial_state=h0)
    return o, hT


def _affine_map(inp):
    """(M, S~) of a whole input window."""
    B, T, H, Dk = inp["q"].shape
    eye = torch.eye(Dk, device="cuda").expand(B, H, Dk, Dk).contiguous()
    _, M = _run(inp, eye, v=torch.zeros_like(inp["v"]))
    _, St = _run(inp, torch.zeros_like(inp["h0"]))
    return M, St


def _inputs(T=2048, H=4, seed=70):
    """prefill_8k-shaped inputs with weak forgetting, so that the state entering a
    segment still matters at its end (with the workload's own gates and betas a
    512-token segment forgets its incoming state completely, M = 0, and the merge
    would be untested): log-decays g ~ -U(0, 0.002) (log-decay mode), beta / 10."""
    w = dataclasses.replace(W.WORKLOADS["prefill_8k"], seed=seed)
    inp = W.make_prefill(w, device="cuda", T=T, H=H)
    gen = torch.Generator(device="cuda").manual_seed(seed)
    inp["z"] = (-0.002 * torch.rand(inp["z"].shape, generator=gen, device="cuda")).to(inp["z"].dtype)
    inp["beta"] = (inp["beta"].float() * 0.1).to(inp["beta"].dtype)
    return inp


def test_segment_map_is_affine():
    """Final state from a random S_in equals M S_in + S~ (d = 128, 4 heads, 512 tokens)."""
    inp = _inputs(T=512)
    M, St = _affine_map(inp)
    print(f"max|M| = {float(M.abs().max()):.3f}")
    assert float(M.abs().max()) > 0.1  # the incoming state survives the segment
    gen = torch.Generator(device="cuda").manual_seed(3)
    S_in = 0.02 * torch.randn(inp["h0"].shape, generator=gen, device="cuda")
    _, hT = _run(inp, S_in)
    pred = torch.matmul(M, S_in) + St
    torch.cuda.synchronize()
    e = rel_err(np64(pred), np64(hT))
    print(f"affine rel err {e:.3e}")
    assert e <= TOL[torch.bfloat16]


def test_segments_merged_in_order_reproduce_one_pass():
    """d = 128, 4 heads, 2048 tokens split into 4 segments of 512: local (M, S~) per
    segment, prefix merge, re-run from the merged entering states; outputs and
    final state match the single pass and the fp64 oracle's single pass."""
    inp = _inputs()
    T = inp["q"].shape[1]
    P = 4
    bounds = [(j * T // P, (j + 1) * T // P) for j in range(P)]
    o_ref, h_ref = _run(inp, inp["h0"])
    maps = [_affine_map(_seg(inp, a, b)) for a, b in bounds]   # independent: one per rank
    assert min(float(M.abs().max()) for M, _ in maps) > 0.1
    S_in, outs = inp["h0"], []
    for (a, b), (M, St) in zip(bounds, maps):
        o, _ = _run(_seg(inp, a, b), S_in)                       # re-run from the true entering state
        outs.append(o)
        S_in = torch.matmul(M, S_in) + St                        # eq. (17) merge
    torch.cuda.synchronize()
    e_o = rel_err(np64(torch.cat(outs, 1)), np64(o_ref))
    e_s = rel_err(np64(S_in), np64(h_ref))
    print(f"KCP rel err o={e_o:.3e} state={e_s:.3e}")
    assert e_o <= TOL[torch.bfloat16] and e_s <= TOL[torch.bfloat16]
    ro, rh, _ = oracle_prefill(inp, z_mode=False)  # log-decay mode, as the calls above
    H, Dv = inp["q"].shape[2], inp["v"].shape[-1]
    e_oo = rel_err(np64(torch.cat(outs, 1)).reshape(-1, H, Dv), ro)
    e_os = rel_err(np64(S_in), rh)
    print(f"KCP against the oracle: rel err o={e_oo:.3e} state={e_os:.3e}")
    assert e_oo <= TOL[torch.bfloat16] and e_os <= TOL[torch.bfloat16]
