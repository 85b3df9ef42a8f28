"""The C-ABI library loads and exports every symbol include/kda.h declares, and
rejects bad arguments with a status before touching the device (CPU only:
no call here reaches a kernel launch)."""
import ctypes
import os
import re
import subprocess

import pytest
import torch

import gated_delta_rule_20_amd as kda

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kda.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(kda.LIB_PATH):
        from gated_delta_rule_20_amd import build
        build.build()
    return kda.load_library()


def _declared():
    src = open(HEADER).read()
    return set(re.findall(r"KDA_API\s+[\w\s\*]+?\b(kda_\w+)\s*\(", src))


def test_header_declarations_match_binding():
    assert _declared() == set(kda.EXPORTED_SYMBOLS)


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", kda.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    exported = {ln.split()[-1] for ln in out.splitlines() if " T " in ln}
    for name in _declared():
        assert name in exported, name
        assert hasattr(lib, name)


def test_status_strings(lib):
    for s, text in [(0, "success"), (1, "invalid value"), (2, "not supported"), (3, "workspace"), (4, "HIP")]:
        assert text in lib.kda_status_string(s).decode()


def _args(**over):
    a = kda.ChunkFwdArgs()
    a.B, a.T, a.H, a.Dk, a.Dv, a.dtype = 1, 128, 2, 128, 128, kda.KDA_BF16
    for f in ("q", "k", "v", "g", "beta", "o"):
        setattr(a, f, 0x10000)
    a.g_min, a.scale = -5.0, 1.0
    for key, val in over.items():
        setattr(a, key, val)
    return a


def _ws(lib, a):
    out = ctypes.c_size_t(0)
    st = lib.kda_chunk_fwd_workspace_size(ctypes.byref(a), ctypes.byref(out))
    return st, out.value


def test_workspace_size_formula(lib):
    st, n = _ws(lib, _args())
    assert st == 0
    block = 74752  # bf16, d=128: 3*64*128 + 64*64 elements, 128 fp32 gammas, 64*128 elements of U, to a 1 KiB multiple
    assert n == 2 * 2 * block
    st, n2 = _ws(lib, _args(T=129))
    assert st == 0 and n2 == 2 * 3 * block
    cu = 0x20000
    st, n3 = _ws(lib, _args(T=1000, cu_seqlens=cu, N=5))
    assert st == 0 and n3 == 256 + 2 * (1000 // 64 + 5) * block


@pytest.mark.parametrize("over,status,msg", [
    (dict(Dk=96), 2, "head dims"),
    (dict(Dv=32), 2, "head dims"),
    (dict(dtype=7), 1, "dtype"),
    (dict(g_min=-6.0), 2, "g_min"),
    (dict(g_min=0.0), 2, "g_min"),
    (dict(H=0), 1, "H >= 1"),
    (dict(T=-1), 1, "T >= 0"),
    (dict(dtype=kda.KDA_F32), 2, "float32"),
    (dict(cu_seqlens=0x20000, B=2, N=2), 1, "B == 1"),
    (dict(cu_seqlens=0x20000, N=0), 1, "N >= 1"),
])
def test_workspace_size_rejects(lib, over, status, msg):
    st, _ = _ws(lib, _args(**over))
    assert st == status
    assert msg in lib.kda_last_error_message().decode()


@pytest.mark.parametrize("over,status,msg", [
    (dict(q=None), 1, "q is NULL"),
    (dict(o=None), 1, "o is NULL"),
    (dict(k=0x10008), 1, "k is not 16-byte aligned"),
    (dict(beta=0x10001), 1, "beta is not aligned"),
    (dict(initial_state=0x10004), 1, "initial_state"),
    (dict(workspace=None, workspace_bytes=0), 3, "workspace is NULL"),
    (dict(workspace=0x100000, workspace_bytes=1024), 3, "needs"),
    (dict(workspace=0x100010, workspace_bytes=1 << 30), 3, "256-byte"),
    (dict(checkpoints=0x100008), 1, "checkpoints is not 16-byte aligned"),
    (dict(checkpoints=0x100000, checkpoint_every=0, checkpoint_slots=4), 1, "checkpoint_every >= 1"),
    (dict(checkpoints=0x100000, checkpoint_every=8, checkpoint_slots=0), 1, "checkpoint_slots >= 1"),
])
def test_chunk_fwd_rejects_before_launch(lib, over, status, msg):
    a = _args(**over)
    st = lib.kda_chunk_fwd(ctypes.byref(a), None)
    assert st == status, lib.kda_last_error_message()
    assert msg in lib.kda_last_error_message().decode()


def test_chunk_fwd_rejects_null_args(lib):
    assert lib.kda_chunk_fwd(None, None) == 1
    out = ctypes.c_size_t(0)
    assert lib.kda_chunk_fwd_workspace_size(ctypes.byref(_args()), None) == 1


@pytest.mark.parametrize("over,status,msg", [
    (dict(Dk=32), 2, "head dims"),
    (dict(state=None), 1, "state is NULL"),
    (dict(v=0x10002), 1, "v is not 16-byte aligned"),
    (dict(H=0), 1, "H >= 1"),
    (dict(g_min=-7.0), 2, "g_min"),
])
def test_recurrent_step_rejects_before_launch(lib, over, status, msg):
    a = kda.StepArgs()
    a.N, a.H, a.Dk, a.Dv, a.dtype = 4, 2, 128, 128, kda.KDA_BF16
    for f in ("q", "k", "v", "g", "beta", "state", "o"):
        setattr(a, f, 0x10000)
    a.g_min, a.scale = -5.0, 1.0
    for key, val in over.items():
        setattr(a, key, val)
    assert lib.kda_recurrent_step(ctypes.byref(a), None) == status
    assert msg in lib.kda_last_error_message().decode()


def test_recurrent_step_zero_sequences_is_a_noop(lib):
    a = kda.StepArgs()
    a.N, a.H, a.Dk, a.Dv, a.dtype, a.g_min = 0, 2, 128, 128, kda.KDA_BF16, -5.0
    assert lib.kda_recurrent_step(ctypes.byref(a), None) == 0


def _replay_args(**over):
    a = kda.ReplayArgs()
    a.N, a.H, a.Dk, a.Dv, a.dtype = 4, 2, 128, 128, kda.KDA_BF16
    a.T_replay, a.T_new, a.n_commit = 3, 4, 1
    for f in ("k_r", "v_r", "g_r", "beta_r", "n_replay", "q", "k", "v", "g", "beta", "state", "o"):
        setattr(a, f, 0x10000)
    a.g_min, a.scale = -5.0, 1.0
    for key, val in over.items():
        setattr(a, key, val)
    return a


@pytest.mark.parametrize("over,status,msg", [
    (dict(Dk=96), 2, "head dims"),
    (dict(state=None), 1, "state is NULL"),
    (dict(state=0x10008), 1, "state is not 16-byte aligned"),
    (dict(n_commit=5), 1, "n_commit"),
    (dict(n_commit=-1), 1, "n_commit"),
    (dict(T_new=-1), 1, "T_new >= 0"),
    (dict(T_replay=-2), 1, "T_replay >= 0"),
    (dict(q=None), 1, "q is NULL"),
    (dict(o=None), 1, "o is NULL"),
    (dict(k_r=None), 1, "k_r is NULL"),
    (dict(beta_r=0x10001), 1, "beta_r is not aligned"),
    (dict(n_replay=0x10002), 1, "n_replay is not 4-byte aligned"),
    (dict(H=0), 1, "H >= 1"),
    (dict(dtype=7), 1, "dtype"),
])
def test_recurrent_replay_rejects_before_launch(lib, over, status, msg):
    a = _replay_args(**over)
    assert lib.kda_recurrent_replay(ctypes.byref(a), None) == status
    assert msg in lib.kda_last_error_message().decode()


@pytest.mark.parametrize("over", [
    dict(N=0),                                                    # no sequences
    dict(T_replay=0, T_new=0, n_commit=0, k_r=None, q=None, o=None),  # empty window
])
def test_recurrent_replay_noops(lib, over):
    a = _replay_args(**over)
    assert lib.kda_recurrent_replay(ctypes.byref(a), None) == 0


def test_recurrent_replay_window_pointers_only_when_used(lib):
    """Replay tensors may be NULL with T_replay = 0, new-window tensors with T_new = 0
    (checked on N = 0 so that nothing is launched)."""
    a = _replay_args(N=0, T_replay=0, k_r=None, v_r=None, g_r=None, beta_r=None, n_replay=None)
    assert lib.kda_recurrent_replay(ctypes.byref(a), None) == 0
    a = _replay_args(N=0, T_new=0, n_commit=0, q=None, k=None, v=None, g=None, beta=None, o=None)
    assert lib.kda_recurrent_replay(ctypes.byref(a), None) == 0


def test_python_binding_requires_device_tensors(lib):
    x = torch.zeros(1, 8, 2, 64)
    with pytest.raises(ValueError, match="device tensor"):
        kda.chunk_fwd(x, x, x, x, torch.zeros(1, 8, 2))


def test_product_path_does_not_import_oracle():
    pkg = os.path.join(ROOT, "gated_delta_rule_20_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                src = open(os.path.join(dirpath, f)).read()
                assert "oracle" not in src.replace("oracle/", ""), f


def test_bench_traffic_records_parse():
    """bench.py's profiled-traffic lookup returns an int (digest matches) or
    None (kernel changed since profiling) and never raises."""
    import bench
    for name in ("prefill", "decode"):
        t = bench.profiled_traffic(name)
        assert t is None or (isinstance(t, int) and t > 0)
    assert bench.profiled_traffic("no-such-kernel") is None


def test_bench_source_digest_ignores_comments_only():
    """The digest that keys the traffic records sees code, not comments or layout."""
    import bench
    a = 'int f(int x) { // scale\n  return 2 * x; /* twice */ }\nconst char *s = "a // b /* c */";'
    assert bench.code_tokens(a) == 'int f(int x) { return 2 * x; }\nconst char *s = "a // b /* c */";'.replace("\n", " ")
    assert bench.code_tokens("/* one // two */ x;\n// y */\nz;") == "x; z;"
    assert bench.code_tokens(a) != bench.code_tokens(a.replace("2 * x", "3 * x"))
    assert bench.source_digest(["no_such_file.hip"]) is None


def test_binding_shape_checks():
    """The binding rejects mismatched operand shapes before any launch."""
    import torch
    from gated_delta_rule_20_amd import _same_lead
    q = torch.zeros(1, 8, 2, 64)
    v = torch.zeros(1, 8, 2, 32)
    b = torch.zeros(1, 8, 2)
    _same_lead(q, q, v, q, b, torch.zeros(2), 2)
    with pytest.raises(ValueError, match="k and g"):
        _same_lead(q, q[:, :4], v, q, b, None, 2)
    with pytest.raises(ValueError, match="beta"):
        _same_lead(q, q, v, q, b[:, :4], None, 2)
    with pytest.raises(ValueError, match="A_log"):
        _same_lead(q, q, v, q, b, torch.zeros(3), 2)


def _fusion(**over):
    f = kda.LayerFusion()
    f.conv_width, f.conv_weight, f.conv_state, f.qk_norm_eps = 4, 0x30000, 0x40000, 1e-6
    for key, val in over.items():
        setattr(f, key, val)
    return f


@pytest.mark.parametrize("over,status,msg", [
    (dict(conv_width=5), 2, "conv_width=5"),
    (dict(conv_width=-1), 2, "conv_width=-1"),
    (dict(conv_weight=None), 1, "conv_weight is NULL"),
    (dict(conv_weight=0x30004), 1, "conv_weight is not 16-byte aligned"),
    (dict(conv_state=None), 1, "conv_state is NULL"),
    (dict(conv_state_out=0x50000), 1, "kda_chunk_fwd only"),
    (dict(conv_checkpoints=0x50000), 1, "kda_chunk_fwd only"),
    (dict(qk_norm_eps=-1.0), 1, "qk_norm_eps"),
    (dict(conv_width=0), 1, "conv_width = 0"),
    (dict(gate=0x60000, o_norm_weight=None), 1, "o_norm_weight is NULL"),
    (dict(gate=0x60008, o_norm_weight=0x70000), 1, "gate is not 16-byte aligned"),
    (dict(gate=0x60000, o_norm_weight=0x70000, o_norm_eps=-2.0), 1, "o_norm_eps"),
])
def test_decode_fusion_rejects_before_launch(lib, over, status, msg):
    f = _fusion(**over)
    a = kda.StepArgs()
    a.N, a.H, a.Dk, a.Dv, a.dtype = 4, 2, 128, 128, kda.KDA_BF16
    for name in ("q", "k", "v", "g", "beta", "state", "o"):
        setattr(a, name, 0x10000)
    a.g_min, a.scale = -5.0, 1.0
    a.fusion = ctypes.pointer(f)
    assert lib.kda_recurrent_step(ctypes.byref(a), None) == status
    assert msg in lib.kda_last_error_message().decode()
    r = _replay_args()
    r.fusion = ctypes.pointer(f)
    r.q_r = 0x10000
    assert lib.kda_recurrent_replay(ctypes.byref(r), None) == status
    assert msg in lib.kda_last_error_message().decode()


def test_replay_fusion_needs_query_projections(lib):
    f = _fusion()
    r = _replay_args()
    r.fusion = ctypes.pointer(f)
    assert lib.kda_recurrent_replay(ctypes.byref(r), None) == 1
    assert "q_r is NULL" in lib.kda_last_error_message().decode()
    r = _replay_args(T_replay=0, k_r=None, v_r=None, g_r=None, beta_r=None, n_replay=None, N=0)
    r.fusion = ctypes.pointer(f)                     # no replayed tokens: q_r not needed
    assert lib.kda_recurrent_replay(ctypes.byref(r), None) == 0


def test_decode_fusion_width_one_needs_no_state(lib):
    """W = 1 carries no convolution state (checked on N = 0: nothing launched)."""
    f = _fusion(conv_width=1, conv_state=None)
    a = kda.StepArgs()
    a.N, a.H, a.Dk, a.Dv, a.dtype, a.g_min = 0, 2, 128, 128, kda.KDA_BF16, -5.0
    a.fusion = ctypes.pointer(f)
    assert lib.kda_recurrent_step(ctypes.byref(a), None) == 0


def test_prefill_fusion_rejects_before_launch(lib):
    """kda_chunk_fwd's fusion checks: overlapping convolution states, convolution
    checkpoints without state checkpoints, a missing norm weight."""
    ws = 1 << 20
    for over, msg in [(dict(conv_state_out=0x40000), "overlaps"),
                      (dict(conv_checkpoints=0x50000), "needs checkpoints"),
                      (dict(gate=0x60000, o_norm_weight=None), "o_norm_weight is NULL"),
                      (dict(conv_width=9), "conv_width=9")]:
        f = _fusion(**over)
        a = _args(workspace=0x1000000, workspace_bytes=1 << 34)
        a.fusion = ctypes.pointer(f)
        st = lib.kda_chunk_fwd(ctypes.byref(a), None)
        assert st in (1, 2), (over, st)
        assert msg in lib.kda_last_error_message().decode(), (over, lib.kda_last_error_message())
    del ws


def test_prologue_needs_no_workspace(lib):
    """The layer prologue runs in the intra-chunk stage's registers: a fusion
    struct with conv_width > 0 leaves the workspace size unchanged."""
    st, base = _ws(lib, _args())
    f = _fusion()
    a = _args()
    a.fusion = ctypes.pointer(f)
    out = ctypes.c_size_t(0)
    assert st == 0 and lib.kda_chunk_fwd_workspace_size(ctypes.byref(a), ctypes.byref(out)) == 0
    assert out.value == base


def test_noalloc_limit_matches_header():
    m = re.search(r"#define\s+KDA_NOALLOC_WORKSPACE_BYTES\s+\((\d+)u\s*<<\s*(\d+)\)", open(HEADER).read())
    assert m and int(m.group(1)) << int(m.group(2)) == kda.NOALLOC_WORKSPACE_BYTES


@pytest.mark.parametrize("over,status,msg", [
    (dict(workspace=0x100000, workspace_bytes=1 << 30), 1, "takes no workspace"),
    (dict(workspace_bytes=4096), 1, "takes no workspace"),
    (dict(T=8192, H=32), 3, "holds at most"),
    (dict(T=7232, H=8), 3, "holds at most"),               # 113 chunks x 8 heads: one chunk over
    (dict(T=7000, H=8, cu_seqlens=0x20000, N=8), 3, "holds at most"),  # 64 pairs: chunk blocks in the workspace
    (dict(Dk=96), 2, "head dims"),
])
def test_chunk_fwd_noalloc_rejects_before_device_work(lib, over, status, msg):
    """Rejections the no-allocation entry point makes on the host, before it
    touches a device (so they hold on a machine without one)."""
    a = _args(**over)
    st = lib.kda_chunk_fwd_noalloc(ctypes.byref(a), None)
    assert st == status, lib.kda_last_error_message()
    assert msg in lib.kda_last_error_message().decode()
    assert lib.kda_chunk_fwd_noalloc(None, None) == 1


def test_noalloc_array_holds_the_documented_largest_call(lib):
    """The header's example: B = 1, T = 7168 at H = 8 (bf16, 128/128) fits,
    one more chunk does not."""
    st, n = _ws(lib, _args(T=7168, H=8))
    assert st == 0 and n <= kda.NOALLOC_WORKSPACE_BYTES
    st, n = _ws(lib, _args(T=7169, H=8))
    assert st == 0 and n > kda.NOALLOC_WORKSPACE_BYTES


def test_pair_mode_workspace_is_the_table(lib):
    """From 128 (sequence, head) pairs on (bf16, Dk = 128, no prologue) the chunk
    blocks stay on chip: the workspace is the chunk table (packed input) or
    nothing (a batch); with the prologue, float32, Dk = 64 or fewer pairs the
    blocks are there."""
    st, n = _ws(lib, _args(T=1000, cu_seqlens=0x20000, N=64, H=2))  # 128 pairs
    assert st == 0 and n == 1280                                        # (4 N + 1) int32, to 256 B
    st, n = _ws(lib, _args(B=128, T=100, H=1))
    assert st == 0 and n == 0
    block = 74752
    st, n = _ws(lib, _args(B=127, T=100, H=1))                          # 127 pairs
    assert st == 0 and n == 127 * 2 * block
    st, n = _ws(lib, _args(B=128, T=100, H=1, Dk=64))
    assert st == 0 and n > 0
    a = _args(B=128, T=100, H=1)
    f = _fusion()
    a.fusion = ctypes.pointer(f)
    out = ctypes.c_size_t(0)
    assert lib.kda_chunk_fwd_workspace_size(ctypes.byref(a), ctypes.byref(out)) == 0 and out.value == 128 * 2 * block
