// kda_abi.hip -- the C ABI declared in include/kda.h: argument validation,
// workspace planning and kernel dispatch.  Every check runs before anything
// is enqueued; nothing here allocates device memory or synchronises.
#include <stdarg.h>
#include <stdio.h>

#include <mutex>

#include "kda.h"
#include "kda_prefill.h"

// Workspace of kda_chunk_fwd_noalloc: one copy of this array lives on every
// device that loads the library, for the life of the process.  In host code
// its name is only a stand-in; the device address comes from
// hipGetSymbolAddress (once per device, below).
static __device__ __align__(256) char scratch[KDA_NOALLOC_WORKSPACE_BYTES];

namespace {

thread_local char g_err[512] = "";

kda_status_t fail(kda_status_t st, const char *fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return st;
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }
bool head_dim_ok(int d) { return d == 64 || d == 128; }

kda_status_t check_common(int dtype, int Dk, int Dv, const float *A_log, float g_min)
{
    if (dtype != KDA_F32 && dtype != KDA_BF16) return fail(KDA_ERROR_INVALID_VALUE, "dtype %d is not a kda_dtype_t", dtype);
    if (!head_dim_ok(Dk) || !head_dim_ok(Dv))
        return fail(KDA_ERROR_NOT_SUPPORTED, "head dims Dk=%d Dv=%d: each must be 64 or 128", Dk, Dv);
    if (!(g_min >= -5.0f && g_min < 0.0f))
        return fail(KDA_ERROR_NOT_SUPPORTED, "g_min=%g: must lie in [-5, 0) for the sub-tile range bound", (double)g_min);
    if (A_log && ((uintptr_t)A_log & 3u)) return fail(KDA_ERROR_INVALID_VALUE, "A_log is not 4-byte aligned");
    return KDA_SUCCESS;
}

bool overlap(const void *a, const void *b, size_t bytes)
{
    const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
    return x < y + bytes && y < x + bytes;
}

// Validates a kda_layer_fusion_t and fills the kernels' view of it.
// prefill: kda_chunk_fwd (read-only conv_state, optional conv_state_out and
// conv_checkpoints) vs the decode entry points (conv_state in place).
kda_status_t check_fusion(const kda_layer_fusion_t *f, bool prefill, bool has_ckpt, int dtype, int N, int H,
                          int Dk, int Dv, kda::FusionParams *out)
{
    *out = kda::FusionParams{};
    if (!f) return KDA_SUCCESS;
    if (f->conv_width < 0 || f->conv_width > 4)
        return fail(KDA_ERROR_NOT_SUPPORTED, "conv_width=%d: must be 0 (no prologue) or 1..4", f->conv_width);
    const size_t el = dtype == KDA_BF16 ? 2 : 4;
    if (f->conv_width > 0) {
        if (!f->conv_weight) return fail(KDA_ERROR_INVALID_VALUE, "conv_weight is NULL");
        if (!aligned16(f->conv_weight)) return fail(KDA_ERROR_INVALID_VALUE, "conv_weight is not 16-byte aligned");
        if (!(f->qk_norm_eps >= 0.0f)) return fail(KDA_ERROR_INVALID_VALUE, "qk_norm_eps must be >= 0");
        const size_t cs_bytes = (size_t)N * H * (f->conv_width - 1) * (2 * Dk + Dv) * el;
        const void *bufs[] = {f->conv_state, f->conv_state_out, f->conv_checkpoints};
        const char *nm[] = {"conv_state", "conv_state_out", "conv_checkpoints"};
        for (int i = 0; i < 3; ++i)
            if (bufs[i] && !aligned16(bufs[i])) return fail(KDA_ERROR_INVALID_VALUE, "%s is not 16-byte aligned", nm[i]);
        if (prefill) {
            if (f->conv_state && f->conv_state_out && cs_bytes > 0 && overlap(f->conv_state, f->conv_state_out, cs_bytes))
                return fail(KDA_ERROR_INVALID_VALUE, "conv_state_out overlaps conv_state");
            if (f->conv_checkpoints && !has_ckpt)
                return fail(KDA_ERROR_INVALID_VALUE, "conv_checkpoints needs checkpoints");
        } else {
            if (f->conv_state_out || f->conv_checkpoints)
                return fail(KDA_ERROR_INVALID_VALUE, "conv_state_out / conv_checkpoints are for kda_chunk_fwd only "
                            "(decode updates conv_state in place)");
            if (f->conv_width > 1 && !f->conv_state && N > 0)
                return fail(KDA_ERROR_INVALID_VALUE, "conv_state is NULL (decode carries the convolution state)");
        }
    } else if (f->conv_weight || f->conv_state || f->conv_state_out || f->conv_checkpoints) {
        return fail(KDA_ERROR_INVALID_VALUE, "convolution buffers given with conv_width = 0");
    }
    if (f->gate) {
        if (!aligned16(f->gate)) return fail(KDA_ERROR_INVALID_VALUE, "gate is not 16-byte aligned");
        if (!f->o_norm_weight) return fail(KDA_ERROR_INVALID_VALUE, "o_norm_weight is NULL");
        if (!aligned16(f->o_norm_weight)) return fail(KDA_ERROR_INVALID_VALUE, "o_norm_weight is not 16-byte aligned");
        if (!(f->o_norm_eps >= 0.0f)) return fail(KDA_ERROR_INVALID_VALUE, "o_norm_eps must be >= 0");
    }
    out->conv_w = f->conv_width;
    out->conv_weight = f->conv_weight;
    out->conv_state = f->conv_width > 1 ? f->conv_state : nullptr;
    out->conv_state_out = f->conv_width > 1 ? f->conv_state_out : nullptr;
    out->conv_ckpt = f->conv_width > 1 ? f->conv_checkpoints : nullptr;
    out->qk_eps = f->qk_norm_eps;
    out->gate = f->gate;
    out->o_weight = f->o_norm_weight;
    out->o_eps = f->o_norm_eps;
    return KDA_SUCCESS;
}

struct ChunkPlan {
    int varlen, N, rows;
    int n_chunks_cap;
    size_t table, block, blocks, total;
};

kda_status_t plan_chunk(const kda_chunk_fwd_args_t *a, ChunkPlan *pl)
{
    if (!a) return fail(KDA_ERROR_INVALID_VALUE, "args is NULL");
    kda_status_t st = check_common(a->dtype, a->Dk, a->Dv, a->A_log, a->g_min);
    if (st != KDA_SUCCESS) return st;
    if (a->B < 1 || a->T < 0 || a->H < 1)
        return fail(KDA_ERROR_INVALID_VALUE, "need B >= 1, T >= 0, H >= 1 (got B=%d T=%d H=%d)", a->B, a->T, a->H);
    const size_t block = kda::block_bytes(a->dtype == KDA_BF16, a->Dk, a->Dv);
    if (block == 0)
        return fail(KDA_ERROR_NOT_SUPPORTED, "prefill with float32 inputs supports Dk=Dv=64 only (got Dk=%d Dv=%d)",
                    a->Dk, a->Dv);
    pl->varlen = a->cu_seqlens != nullptr;
    if (pl->varlen) {
        if (a->B != 1) return fail(KDA_ERROR_INVALID_VALUE, "cu_seqlens requires B == 1 (got B=%d)", a->B);
        if (a->N < 1) return fail(KDA_ERROR_INVALID_VALUE, "cu_seqlens requires N >= 1 (got N=%d)", a->N);
        if ((uintptr_t)a->cu_seqlens & 3u) return fail(KDA_ERROR_INVALID_VALUE, "cu_seqlens is not 4-byte aligned");
        pl->N = a->N;
    } else {
        pl->N = a->B;
    }
    const long long rows = (long long)a->B * a->T;
    if (rows > 0x7fffffffLL || (long long)pl->N * a->H > 0x0fffffffLL)
        return fail(KDA_ERROR_NOT_SUPPORTED, "problem too large for 32-bit token/pair indices");
    pl->rows = (int)rows;
    const long long cap = pl->varlen ? (long long)a->T / KDA_CHUNK + pl->N
                                     : (long long)a->B * ((a->T + KDA_CHUNK - 1) / KDA_CHUNK);
    if (cap > 0x7fffffffLL) return fail(KDA_ERROR_NOT_SUPPORTED, "too many chunks");
    pl->n_chunks_cap = (int)cap;
    pl->table = kda::table_bytes(pl->varlen, pl->N);
    pl->block = block;
    // pair mode keeps every chunk block in LDS; the layer prologue runs in registers
    const int pro = a->fusion && a->fusion->conv_width > 0;
    const bool pairs = kda::pair_mode(a->dtype == KDA_BF16, a->Dk, (long)pl->N * a->H, pro);
    pl->blocks = pairs ? 0 : (size_t)a->H * (size_t)cap * block;
    pl->total = pl->table + pl->blocks;
    return KDA_SUCCESS;
}

kda_status_t hip_fail(hipError_t e, const char *what)
{
    return fail(KDA_ERROR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// Device address of `scratch` on the current device, looked up once per device.
constexpr int MAX_DEVICES = 64;
std::mutex g_scratch_mu;
void *g_scratch[MAX_DEVICES];

kda_status_t scratch_on_current_device(void **out)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (dev < 0 || dev >= MAX_DEVICES) return fail(KDA_ERROR_NOT_SUPPORTED, "device %d beyond %d", dev, MAX_DEVICES);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch[dev]) {
        void *ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !ptr) return hip_fail(e, "hipGetSymbolAddress(scratch)");
        g_scratch[dev] = ptr;
    }
    *out = g_scratch[dev];
    return KDA_SUCCESS;
}

}  // namespace

extern "C" {

const char *kda_status_string(kda_status_t s)
{
    switch (s) {
    case KDA_SUCCESS: return "success";
    case KDA_ERROR_INVALID_VALUE: return "invalid value";
    case KDA_ERROR_NOT_SUPPORTED: return "not supported";
    case KDA_ERROR_WORKSPACE: return "workspace missing or too small";
    case KDA_ERROR_HIP: return "HIP runtime error";
    }
    return "unknown status";
}

const char *kda_last_error_message(void) { return g_err; }

kda_status_t kda_chunk_fwd_workspace_size(const kda_chunk_fwd_args_t *a, size_t *bytes)
{
    if (!bytes) return fail(KDA_ERROR_INVALID_VALUE, "bytes is NULL");
    ChunkPlan pl;
    const kda_status_t st = plan_chunk(a, &pl);
    if (st != KDA_SUCCESS) return st;
    *bytes = pl.total;
    g_err[0] = 0;
    return KDA_SUCCESS;
}

kda_status_t kda_chunk_fwd(const kda_chunk_fwd_args_t *a, void *stream)
{
    ChunkPlan pl;
    kda_status_t st = plan_chunk(a, &pl);
    if (st != KDA_SUCCESS) return st;
    const bool has_tokens = pl.rows > 0;
    if (has_tokens) {
        const void *req[] = {a->q, a->k, a->v, a->g, a->beta, a->o};
        const char *nm[] = {"q", "k", "v", "g", "beta", "o"};
        for (int i = 0; i < 6; ++i) {
            if (!req[i]) return fail(KDA_ERROR_INVALID_VALUE, "%s is NULL", nm[i]);
            if (i != 4 && !aligned16(req[i])) return fail(KDA_ERROR_INVALID_VALUE, "%s is not 16-byte aligned", nm[i]);
        }
        if ((uintptr_t)a->beta & (a->dtype == KDA_BF16 ? 1u : 3u))
            return fail(KDA_ERROR_INVALID_VALUE, "beta is not aligned to its element size");
    }
    if (a->initial_state && !aligned16(a->initial_state))
        return fail(KDA_ERROR_INVALID_VALUE, "initial_state is not 16-byte aligned");
    if (a->final_state && !aligned16(a->final_state))
        return fail(KDA_ERROR_INVALID_VALUE, "final_state is not 16-byte aligned");
    if (a->checkpoints) {
        if (!aligned16(a->checkpoints)) return fail(KDA_ERROR_INVALID_VALUE, "checkpoints is not 16-byte aligned");
        if (a->checkpoint_every < 1 || a->checkpoint_slots < 1)
            return fail(KDA_ERROR_INVALID_VALUE, "need checkpoint_every >= 1 and checkpoint_slots >= 1 (got %d, %d)",
                        a->checkpoint_every, a->checkpoint_slots);
    }
    kda::FusionParams fp;
    st = check_fusion(a->fusion, true, a->checkpoints != nullptr, a->dtype, pl.N, a->H, a->Dk, a->Dv, &fp);
    if (st != KDA_SUCCESS) return st;
    if (pl.total > 0) {
        if (!a->workspace) return fail(KDA_ERROR_WORKSPACE, "workspace is NULL but %zu bytes are needed", pl.total);
        if (a->workspace_bytes < pl.total)
            return fail(KDA_ERROR_WORKSPACE, "workspace has %zu bytes, needs %zu", a->workspace_bytes, pl.total);
        if ((uintptr_t)a->workspace & 255u) return fail(KDA_ERROR_WORKSPACE, "workspace is not 256-byte aligned");
    }
    if (!has_tokens && !a->final_state && !fp.conv_state_out) {  // nothing observable to compute
        g_err[0] = 0;
        return KDA_SUCCESS;
    }

    kda::PrefillParams p;
    p.q = a->q; p.k = a->k; p.v = a->v; p.g = a->g; p.beta = a->beta;
    p.A_log = a->A_log; p.g_min = a->g_min; p.scale = a->scale;
    p.cu = a->cu_seqlens; p.N = pl.N; p.T = a->T; p.H = a->H; p.varlen = pl.varlen;
    p.h0 = a->initial_state; p.hT = a->final_state; p.o = a->o;
    char *ws = (char *)a->workspace;
    p.chunk_off = pl.varlen ? (int32_t *)ws : nullptr;
    p.order = pl.varlen ? (int32_t *)ws + (pl.N + 1) : nullptr;
    p.span = pl.varlen ? (int32_t *)ws + (2 * pl.N + 1) : nullptr;
    p.blocks = ws ? ws + pl.table : nullptr;
    p.n_chunks_cap = has_tokens ? pl.n_chunks_cap : 0;
    p.ckpt = a->checkpoints;
    p.ckpt_every = a->checkpoints ? a->checkpoint_every : 0;
    p.ckpt_slots = a->checkpoints ? a->checkpoint_slots : 0;
    p.f = fp;
    const hipError_t e = kda::launch_chunk_fwd(a->dtype == KDA_BF16, a->Dk, a->Dv, p, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "kda_chunk_fwd launch");
    g_err[0] = 0;
    return KDA_SUCCESS;
}

kda_status_t kda_chunk_fwd_noalloc(const kda_chunk_fwd_args_t *a, void *stream)
{
    if (!a) return fail(KDA_ERROR_INVALID_VALUE, "args is NULL");
    if (a->workspace || a->workspace_bytes)
        return fail(KDA_ERROR_INVALID_VALUE, "kda_chunk_fwd_noalloc takes no workspace (set workspace = NULL, "
                    "workspace_bytes = 0)");
    ChunkPlan pl;
    kda_status_t st = plan_chunk(a, &pl);
    if (st != KDA_SUCCESS) return st;
    if (pl.total > (size_t)KDA_NOALLOC_WORKSPACE_BYTES)
        return fail(KDA_ERROR_WORKSPACE, "these shapes need %zu workspace bytes; kda_chunk_fwd_noalloc holds at most "
                    "%zu (KDA_NOALLOC_WORKSPACE_BYTES): use kda_chunk_fwd with a workspace", pl.total,
                    (size_t)KDA_NOALLOC_WORKSPACE_BYTES);
    void *ws = nullptr;
    st = scratch_on_current_device(&ws);
    if (st != KDA_SUCCESS) return st;
    kda_chunk_fwd_args_t b = *a;
    b.workspace = ws;
    b.workspace_bytes = (size_t)KDA_NOALLOC_WORKSPACE_BYTES;
    return kda_chunk_fwd(&b, stream);
}

kda_status_t kda_recurrent_step(const kda_step_args_t *a, void *stream)
{
    if (!a) return fail(KDA_ERROR_INVALID_VALUE, "args is NULL");
    kda_status_t st = check_common(a->dtype, a->Dk, a->Dv, a->A_log, a->g_min);
    if (st != KDA_SUCCESS) return st;
    if (a->N < 0 || a->H < 1) return fail(KDA_ERROR_INVALID_VALUE, "need N >= 0, H >= 1 (got N=%d H=%d)", a->N, a->H);
    // one workgroup per (sequence, head) must fit the launch grid
    if ((long long)a->N * a->H > 0x3fffffffLL) return fail(KDA_ERROR_NOT_SUPPORTED, "N*H too large");
    kda::FusionParams fp;
    st = check_fusion(a->fusion, false, false, a->dtype, a->N, a->H, a->Dk, a->Dv, &fp);
    if (st != KDA_SUCCESS) return st;
    if (a->N == 0) { g_err[0] = 0; return KDA_SUCCESS; }
    const void *req[] = {a->q, a->k, a->v, a->g, a->beta, a->state, a->o};
    const char *nm[] = {"q", "k", "v", "g", "beta", "state", "o"};
    for (int i = 0; i < 7; ++i) {
        if (!req[i]) return fail(KDA_ERROR_INVALID_VALUE, "%s is NULL", nm[i]);
        if (i != 4 && !aligned16(req[i])) return fail(KDA_ERROR_INVALID_VALUE, "%s is not 16-byte aligned", nm[i]);
    }
    if ((uintptr_t)a->beta & (a->dtype == KDA_BF16 ? 1u : 3u))
        return fail(KDA_ERROR_INVALID_VALUE, "beta is not aligned to its element size");
    // One decode step is a one-token window of the replay kernel: no cached
    // tokens, one new token, committed.  [N, H, D] tensors are [N, 1, H, D].
    kda::ReplayParams p;
    p.N = a->N; p.H = a->H;
    p.T_replay = 0; p.T_new = 1; p.n_commit = 1;
    p.k_r = p.v_r = p.g_r = p.beta_r = nullptr;
    p.n_replay = nullptr;
    p.q = a->q; p.k = a->k; p.v = a->v; p.g = a->g; p.beta = a->beta;
    p.A_log = a->A_log; p.g_min = a->g_min; p.scale = a->scale;
    p.state = a->state; p.o = a->o;
    p.q_r = nullptr;
    p.f = fp;
    const hipError_t e = kda::launch_recurrent_replay(a->dtype == KDA_BF16, a->Dk, a->Dv, p, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "kda_recurrent_step launch");
    g_err[0] = 0;
    return KDA_SUCCESS;
}

kda_status_t kda_recurrent_replay(const kda_replay_args_t *a, void *stream)
{
    if (!a) return fail(KDA_ERROR_INVALID_VALUE, "args is NULL");
    kda_status_t st = check_common(a->dtype, a->Dk, a->Dv, a->A_log, a->g_min);
    if (st != KDA_SUCCESS) return st;
    if (a->N < 0 || a->H < 1) return fail(KDA_ERROR_INVALID_VALUE, "need N >= 0, H >= 1 (got N=%d H=%d)", a->N, a->H);
    if (a->T_replay < 0 || a->T_new < 0)
        return fail(KDA_ERROR_INVALID_VALUE, "need T_replay >= 0, T_new >= 0 (got %d, %d)", a->T_replay, a->T_new);
    if (a->n_commit < 0 || a->n_commit > a->T_new)
        return fail(KDA_ERROR_INVALID_VALUE, "need 0 <= n_commit <= T_new (got n_commit=%d T_new=%d)", a->n_commit, a->T_new);
    // one workgroup per (sequence, head) must fit the launch grid
    if ((long long)a->N * a->H > 0x3fffffffLL) return fail(KDA_ERROR_NOT_SUPPORTED, "N*H too large");
    if (!a->state) return fail(KDA_ERROR_INVALID_VALUE, "state is NULL");
    if (!aligned16(a->state)) return fail(KDA_ERROR_INVALID_VALUE, "state is not 16-byte aligned");
    const unsigned el = a->dtype == KDA_BF16 ? 1u : 3u;
    if (a->T_new > 0) {
        const void *req[] = {a->q, a->k, a->v, a->g, a->beta, a->o};
        const char *nm[] = {"q", "k", "v", "g", "beta", "o"};
        for (int i = 0; i < 6; ++i) {
            if (!req[i]) return fail(KDA_ERROR_INVALID_VALUE, "%s is NULL", nm[i]);
            if (i != 4 && !aligned16(req[i])) return fail(KDA_ERROR_INVALID_VALUE, "%s is not 16-byte aligned", nm[i]);
        }
        if ((uintptr_t)a->beta & el) return fail(KDA_ERROR_INVALID_VALUE, "beta is not aligned to its element size");
    }
    if (a->T_replay > 0) {
        const void *req[] = {a->k_r, a->v_r, a->g_r, a->beta_r};
        const char *nm[] = {"k_r", "v_r", "g_r", "beta_r"};
        for (int i = 0; i < 4; ++i) {
            if (!req[i]) return fail(KDA_ERROR_INVALID_VALUE, "%s is NULL", nm[i]);
            if (i != 3 && !aligned16(req[i])) return fail(KDA_ERROR_INVALID_VALUE, "%s is not 16-byte aligned", nm[i]);
        }
        if ((uintptr_t)a->beta_r & el) return fail(KDA_ERROR_INVALID_VALUE, "beta_r is not aligned to its element size");
        if (a->n_replay && ((uintptr_t)a->n_replay & 3u)) return fail(KDA_ERROR_INVALID_VALUE, "n_replay is not 4-byte aligned");
    }
    kda::FusionParams fp;
    st = check_fusion(a->fusion, false, false, a->dtype, a->N, a->H, a->Dk, a->Dv, &fp);
    if (st != KDA_SUCCESS) return st;
    if (fp.conv_w > 0 && a->T_replay > 0) {
        if (!a->q_r) return fail(KDA_ERROR_INVALID_VALUE, "q_r is NULL (the fused prologue replays the query convolution)");
        if (!aligned16(a->q_r)) return fail(KDA_ERROR_INVALID_VALUE, "q_r is not 16-byte aligned");
    }
    if (a->N == 0 || a->T_replay + a->T_new == 0) { g_err[0] = 0; return KDA_SUCCESS; }
    kda::ReplayParams p;
    p.N = a->N; p.H = a->H;
    p.T_replay = a->T_replay; p.T_new = a->T_new; p.n_commit = a->n_commit;
    p.k_r = a->k_r; p.v_r = a->v_r; p.g_r = a->g_r; p.beta_r = a->beta_r;
    p.n_replay = a->T_replay > 0 ? a->n_replay : nullptr;
    p.q = a->q; p.k = a->k; p.v = a->v; p.g = a->g; p.beta = a->beta;
    p.A_log = a->A_log; p.g_min = a->g_min; p.scale = a->scale;
    p.state = a->state; p.o = a->o;
    p.q_r = (fp.conv_w > 0 && a->T_replay > 0) ? a->q_r : nullptr;
    p.f = fp;
    const hipError_t e = kda::launch_recurrent_replay(a->dtype == KDA_BF16, a->Dk, a->Dv, p, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "kda_recurrent_replay launch");
    g_err[0] = 0;
    return KDA_SUCCESS;
}

}  // extern "C"
