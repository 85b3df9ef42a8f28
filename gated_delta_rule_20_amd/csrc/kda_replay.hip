// kda_replay.hip -- decode-side recurrence with the state updated in place:
// the single decode step and the speculative-decoding step with replay.
//
// "Kimi K3 Technical Report: Open Frontier Intelligence", §5.4.2 ("KDA"): decode
// is bound by moving the in-place state; under speculative decoding the
// accepted part of a draft window is rebuilt on chip from the drafts' cached
// projected inputs, and the replayed tokens, the certain (bonus) token and the
// next draft window run through one recurrence loop that reads the state once
// and writes it back once, after the last token whose state is kept.  A single
// decode step is the window with no cached tokens and one new token.
//
// Per token the update is eq. (1) with the eq. (5) gate, arranged as in the
// single-step kernel (D := Diag(alpha)):
//   p = (D S)^T k,  r = (D S)^T q,  delta = beta (v - p),
//   S <- D S + k delta^T,  o = scale * (r + delta * (k . q)).
// Replayed tokens skip q, r and o.
//
// Layout: see replay_kernel.  The state is read once at the start and written
// once, at the commit point, each access a row of d_v consecutive floats across
// the workgroup.
#include "kda_common.h"
#include "kda_prefill.h"

namespace kda {

// One element loaded or stored through a buffer descriptor (bf16: 2 bytes, fp32: 4 bytes).
template <typename T> __device__ __forceinline__ T elem_load(__amdgpu_buffer_rsrc_t rs, int off_bytes)
{
    if constexpr (sizeof(T) == 2)
        return __builtin_bit_cast(T, __builtin_amdgcn_raw_buffer_load_b16(rs, off_bytes, 0, 0));
    else
        return __builtin_bit_cast(T, __builtin_amdgcn_raw_buffer_load_b32(rs, off_bytes, 0, 0));
}
template <typename T> __device__ __forceinline__ void elem_store(__amdgpu_buffer_rsrc_t rs, int off_bytes, T v)
{
    if constexpr (sizeof(T) == 2)
        __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(uint16_t, v), rs, off_bytes, 0, 0);
    else
        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), rs, off_bytes, 0, 0);
}

// Row-broadcast FMAs.  Lane l holds row 16 V + (l % 16) of a per-row operand
// in kr; DPP row_newbcast:n hands every lane of a 16-lane row the value of
// its lane n, so 16 FMAs cover 16 rows with no further LDS reads and in the
// same order, with the same roundings, as the broadcast-read loop.  A DPP
// read of a VGPR needs two wait states after a VALU write of it and five after
// a VALU write of EXEC, which the compiler does not insert around inline
// assembly: each group starts with s_nop W (W + 1 wait states), W = 4 where
// EXEC may just have changed.
//   dot16: acc += sum over n of kr[row 16 V + n] * x[16 V + n]
//   upd16: x[16 V + n] += kr[row 16 V + n] * d
template <int V, int W = 1> __device__ __forceinline__ void dot16(float &acc, float kr, const float *x)
{
    asm("s_nop %c18\n"
        "v_fmac_f32_dpp %0, %1, %2 row_newbcast:0 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %0, %1, %3 row_newbcast:1 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %0, %1, %4 row_newbcast:2 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %0, %1, %5 row_newbcast:3 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %0, %1, %6 row_newbcast:4 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %0, %1, %7 row_newbcast:5 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %0, %1, %8 row_newbcast:6 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %0, %1, %9 row_newbcast:7 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %0, %1, %10 row_newbcast:8 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %0, %1, %11 row_newbcast:9 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %0, %1, %12 row_newbcast:10 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %0, %1, %13 row_newbcast:11 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %0, %1, %14 row_newbcast:12 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %0, %1, %15 row_newbcast:13 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %0, %1, %16 row_newbcast:14 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %0, %1, %17 row_newbcast:15 row_mask:0xf bank_mask:0xf\n"
        : "+v"(acc)
        : "v"(kr),
          "v"(x[16 * V + 0]), "v"(x[16 * V + 1]), "v"(x[16 * V + 2]), "v"(x[16 * V + 3]),
          "v"(x[16 * V + 4]), "v"(x[16 * V + 5]), "v"(x[16 * V + 6]), "v"(x[16 * V + 7]),
          "v"(x[16 * V + 8]), "v"(x[16 * V + 9]), "v"(x[16 * V + 10]), "v"(x[16 * V + 11]),
          "v"(x[16 * V + 12]), "v"(x[16 * V + 13]), "v"(x[16 * V + 14]), "v"(x[16 * V + 15]),
          "i"(W));
}
template <int V, int W = 1> __device__ __forceinline__ void upd16(float *x, float kr, float d)
{
    asm("s_nop %c18\n"
        "v_fmac_f32_dpp %0, %16, %17 row_newbcast:0 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %1, %16, %17 row_newbcast:1 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %2, %16, %17 row_newbcast:2 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %3, %16, %17 row_newbcast:3 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %4, %16, %17 row_newbcast:4 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %5, %16, %17 row_newbcast:5 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %6, %16, %17 row_newbcast:6 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %7, %16, %17 row_newbcast:7 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %8, %16, %17 row_newbcast:8 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %9, %16, %17 row_newbcast:9 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %10, %16, %17 row_newbcast:10 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %11, %16, %17 row_newbcast:11 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %12, %16, %17 row_newbcast:12 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %13, %16, %17 row_newbcast:13 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %14, %16, %17 row_newbcast:14 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %15, %16, %17 row_newbcast:15 row_mask:0xf bank_mask:0xf\n"
        : "+v"(x[16 * V + 0]), "+v"(x[16 * V + 1]), "+v"(x[16 * V + 2]), "+v"(x[16 * V + 3]),
          "+v"(x[16 * V + 4]), "+v"(x[16 * V + 5]), "+v"(x[16 * V + 6]), "+v"(x[16 * V + 7]),
          "+v"(x[16 * V + 8]), "+v"(x[16 * V + 9]), "+v"(x[16 * V + 10]), "+v"(x[16 * V + 11]),
          "+v"(x[16 * V + 12]), "+v"(x[16 * V + 13]), "+v"(x[16 * V + 14]), "+v"(x[16 * V + 15])
        : "v"(kr), "v"(d), "i"(W));
}

// pair_sum32: v[l] + v[l ^ 32] in every lane (wave_sum is in kda_common.h).
__device__ __forceinline__ float pair_sum32(float v)
{
    return v + __shfl_xor(v, 32);
}

// One workgroup per (sequence, head).  Each state column is held by NH = d_k/64
// lanes of one wave (lanes l and l + 32 when NH = 2), each with 64 rows of it
// in registers.  A token's two reductions over the rows, p = (D S)^T k and
// r = (D S)^T q, are then sums inside each lane plus one lane swap, so the
// token loop needs no barrier.  The per-row operands of a token come from LDS,
// in one of two loops (RB below):
//  * broadcast reads, four rows per read: the plain single step, which is
//    HBM-bound and runs best with few workgroups in flight;
//  * row broadcast, everywhere else: each lane reads a 16-row slice of each
//    operand once per token and every FMA takes its row from the lane that
//    holds it (DPP, see dot16 / upd16).  It frees registers: the plain window
//    and the fused single step fit in 128 VGPRs and run four workgroups per CU,
//    which their extra VALU work per state element needs to overlap the state
//    traffic (the fused window would spill there and stays at three).
// Both loops run the same FMAs in the same order.  Token inputs are staged TB
// tokens at a time (all loads in flight together); TB = 1 is the single decode
// step.
//
// Decay folding.  Inside a block the registers hold the state in a scaled
// frame, X = S / P_j with P_j the per-row product of alpha over the block's
// first j tokens (P <= 1, and P >= e^{-5 TB} by the gate's lower bound, so
// 1/P stays far inside fp32).  In that frame one token is
//   p = X^T (P_j k),  r = X^T (P_j q),  X <- X + (k / P_j) delta^T,
// with P_j k, P_j q and k / P_j formed once per row during staging, so the
// per-element decay multiply disappears; the true state X * P is formed only
// for the write-back and at the end of a block.
//
// FU: the layer's prologue (eq. (2)) and epilogue (eq. (6)) run in the same
// pass, each switched on at run time.  Prologue: during staging the thread of
// row r keeps the last three pre-activations of query and key channel r (and
// the thread of column c those of value channel c) in registers, convolves,
// applies Swish and stages the UNnormalised a_k, a_q with per-wave partial
// sums of a_k^2 and a_q^2; L2Norm is a per-token scalar, so the token loop
// multiplies the two reductions and the update by 1/|a_k| and 1/|a_q| instead
// of a second staging pass.  The convolution state is written back with the
// recurrent state's commit.  Epilogue: the block's outputs go to LDS; after
// the block, each wave sums o~^2 over the head's d_v columns for each token and
// the thread of column c writes Sigmoid(gate) * w_c * o~_c / rms.
template <typename T, int DK, int DV, int TB, bool FU>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(
    (TB == 1 && !FU) ? 3 : ((!FU || TB == 1 || DV * (DK / 64) >= DK + DV) ? 4 : 3)))) void replay_kernel(ReplayParams p)
{
    constexpr int NH = DK / 64;         // lanes per column
    constexpr int RH = 64;              // rows per lane
    constexpr int CPW = 64 / NH;        // columns per wave
    constexpr int NT = DV * NH;         // threads
    constexpr int NW = NT / 64;         // waves
    constexpr int CC = 2 * DK + DV;     // convolution channels per head
    constexpr bool RB = TB > 1 || FU;  // row-broadcast token loop (all but the plain single step)
    // Fused staging split by role when the workgroup has a thread per channel of
    // each kind: waves 0 .. DK/64 - 1 take the query / key / decay channels, the
    // other waves the value / output-gate channels.
    constexpr bool SPLIT = FU && NT >= DK + DV;
    static_assert(NH * RH == DK && NT % 64 == 0 && NT <= 256 && NT >= DK && NT >= DV, "shape");
    __shared__ __align__(16) float s_kd[TB][DK], s_qd[TB][DK], s_ki[TB][DK];  // P_j k, P_j q, k / P_j
    __shared__ __align__(16) float s_pc[DK], s_pe[DK];    // P at the commit token, P at the block end
    __shared__ float s_v[TB][DV], s_b[TB], s_kqw[NW][TB];
    constexpr int FT = FU ? TB : 1, FV = FU ? DV : 1, FW = FU ? NW : 1;
    __shared__ float s_sk[FW][FT], s_sq[FW][FT];          // partial sums of a_k^2, a_q^2 (prologue)
    __shared__ float s_o[FT][FV], s_gt[FT][FV];           // o~ and Sigmoid(gate) of the block (epilogue)
    constexpr bool GH = FU && !(NT >= DK + DV);           // generic fused staging
    __shared__ float s_hist[GH ? 3 : 1][GH ? CC : 1];     // conv history between blocks (prologue, generic staging)

    // (the fused variant keeps the wave index in a scalar: its per-wave LDS slots
    // then need no per-lane address registers)
    const int t = threadIdx.x, l = t & 63, w = FU ? __builtin_amdgcn_readfirstlane(t >> 6) : t >> 6;
    const int hf = l / CPW;                       // which 64 rows of the column
    const int col = w * CPW + (l % CPW);          // this lane's column
    const size_t nh = blockIdx.x;                 // sequence * H + head
    const int h = (int)(nh % p.H);
    const size_t sq = nh / p.H;                   // sequence
    // State of this (sequence, head) through a buffer descriptor: the lane's
    // offset in a VGPR, the row offset as a scalar, so the 64 row accesses need
    // no per-row 64-bit address registers.  Non-temporal: streamed once.
    const __amdgpu_buffer_rsrc_t srs = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(p.state + nh * (size_t)(DK * DV)), 0, (int)(DK * DV * sizeof(float)), 0x00020000);
    const int lane_off = ((hf * RH) * DV + col) * (int)sizeof(float);
    constexpr int ROW = DV * (int)sizeof(float), NT_AUX = 2;

    float st[RH];
#pragma unroll
    for (int r = 0; r < RH; ++r)
        st[r] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(srs, lane_off, r * ROW, NT_AUX));

    int n_rep = p.T_replay;
    if (p.n_replay) n_rep = min(max(p.n_replay[sq], 0), p.T_replay);
    const int n_tok = n_rep + p.T_new;
    const int commit_at = n_rep + p.n_commit;     // tokens applied before the write-back (0: none)
    const float eA = p.A_log ? __expf(p.A_log[h]) : 0.f;
    auto row_of = [&](int it) {                   // (s, t, h) row of token `it` of replay-then-new
        return it < n_rep ? (sq * (size_t)p.T_replay + it) * p.H + h
                          : (sq * (size_t)p.T_new + (it - n_rep)) * p.H + h;
    };
    const int r0h = hf * RH;                      // first row of this lane

    // Prologue state: pre-activations 3, 2, 1 tokens back (slot 2 newest) of
    // query / key channel t and value channel t, zero-padded below width 4,
    // kept in LDS between blocks by the thread that owns the channels.
    const bool pro = FU && p.f.conv_w > 0, epi = FU && p.f.gate != nullptr;
    const int cw = pro ? p.f.conv_w : 1;
    T *const cstate = (FU && cw > 1) ? (T *)p.f.conv_state + nh * (size_t)((cw - 1) * CC) : nullptr;
    // Split staging: the history of this thread's channels stays in registers
    // (h0: query or value channel, h1: key channel), the carried state's rows
    // loaded in the first block's staging right after its first token group's
    // inputs, so that waiting for them holds back nothing and they are not live
    // (nor spilled) before.
    float h0[3] = {0.f, 0.f, 0.f}, h1[3] = {0.f, 0.f, 0.f};
    if constexpr (!SPLIT && FU) {
        if (pro) {
#pragma unroll
            for (int i = 0; i < 3; ++i) {     // slot i holds state row i - 4 + cw (if any)
                const int j = i - 4 + cw;
                const bool in = cstate && j >= 0;
                if (t < DK) {
                    s_hist[i][t] = in ? to_f<T>(cstate[j * CC + t]) : 0.f;
                    s_hist[i][DK + t] = in ? to_f<T>(cstate[j * CC + DK + t]) : 0.f;
                }
                if (t < DV) s_hist[i][2 * DK + t] = in ? to_f<T>(cstate[j * CC + 2 * DK + t]) : 0.f;
            }
        }
    }

    for (int base = 0; base < n_tok; base += TB) {
        const int nb = min(TB, n_tok - base);
        const int jc = commit_at - 1 - base;      // commit token inside this block, if 0 <= jc < nb
        // ---- stage the block's inputs: all loads first (one latency per block),
        // then the per-row products into LDS ----
        if constexpr (SPLIT) {
            int tl = t;
            asm volatile("" : "+v"(tl));  // addresses formed here, not kept from before the block loop
            const bool kr = tl < DK;      // wave-uniform role
            const int ch = kr ? tl : tl - DK;
            // Per-lane offsets are unsigned 32-bit so that every global access is a
            // uniform base plus a zero-extended lane offset (no 64-bit lane addresses).
            const unsigned uch = (unsigned)ch;
            const unsigned c0 = kr ? uch : 2u * DK + uch, c1 = DK + uch;  // conv channels: q and k, or v
            float w0[4] = {0.f, 0.f, 0.f, 0.f}, w1[4] = {0.f, 0.f, 0.f, 0.f};
            if (pro) {
                const float *wb = p.f.conv_weight + (size_t)h * CC * cw;
#pragma unroll
                for (int i = 0; i < 4; ++i) {  // tap i holds weight i - 4 + cw (if any)
                    const int x = i - 4 + cw;
                    if (x >= 0) {
                        const float *wx = wb + x;
                        w0[i] = wx[c0 * (unsigned)cw];
                        if (kr) w1[i] = wx[c1 * (unsigned)cw];
                    }
                }
            }
            float pr = 1.f;                      // running product of alpha (query / key role)
            // SB tokens at a time: their loads together, then their products.  Sigmoids
            // and 1 / P use the hardware reciprocal (about 1 ulp).
            constexpr int SB = TB < 4 ? TB : 4;
            for (int j0 = 0; j0 < nb; j0 += SB) {
                // query / key role: decay logit, key, query; value role: value, output gate
                T a0[SB], a1[SB], a2[SB];
                float bt[SB];
#pragma unroll
                for (int jj = 0; jj < SB; ++jj) {
                    const int j = j0 + jj, it = base + j;
                    const bool ok = j < nb, rep = it < n_rep;
                    const size_t row = ok ? row_of(it) : 0;
                    if (kr) {
                        const T *gb = (const T *)(rep ? p.g_r : p.g) + row * DK;
                        const T *kb = (const T *)(rep ? p.k_r : p.k) + row * DK;
                        const T *qb = (const T *)(rep ? p.q_r : p.q) + row * DK;
                        a0[jj] = ok ? gb[uch] : from_f<T>(0.f);
                        a1[jj] = ok ? kb[uch] : from_f<T>(0.f);
                        // with the prologue the replayed queries feed the convolution
                        a2[jj] = (ok && (pro || !rep)) ? qb[uch] : from_f<T>(0.f);
                    } else {
                        const T *vb = (const T *)(rep ? p.v_r : p.v) + row * DV;
                        const T *eb = (const T *)p.f.gate + row * DV;
                        a0[jj] = ok ? vb[uch] : from_f<T>(0.f);
                        a1[jj] = (epi && ok && !rep) ? eb[uch] : from_f<T>(0.f);
                        a2[jj] = from_f<T>(0.f);
                    }
                    bt[jj] = ok ? to_f<T>(((const T *)(rep ? p.beta_r : p.beta))[row]) : 0.f;
                }
                if (pro && base == 0 && j0 == 0 && cstate) {  // the carried convolution state
                    const __amdgpu_buffer_rsrc_t crs = __builtin_amdgcn_make_buffer_rsrc(
                        cstate, 0, (cw - 1) * CC * (int)sizeof(T), 0x00020000);
#pragma unroll
                    for (int i = 0; i < 3; ++i) {
                        const int r = i - 4 + cw;  // slot i holds state row r (if any)
                        if (r >= 0) {
                            h0[i] = to_f<T>(elem_load<T>(crs, (r * CC + (int)c0) * (int)sizeof(T)));
                            if (kr) h1[i] = to_f<T>(elem_load<T>(crs, (r * CC + (int)c1) * (int)sizeof(T)));
                        }
                    }
                }
#pragma unroll
                for (int jj = 0; jj < SB; ++jj) {
                    const int j = j0 + jj;
                    if (j >= nb) break;
                    float kq = 0.f, ssk = 0.f, ssq = 0.f;
                    // ShortConv + Swish (eq. (2)) of channel c0 (and c1); the history advances
                    const float x0 = to_f<T>(kr ? a2[jj] : a0[jj]), x1 = to_f<T>(a1[jj]);
                    float y0 = x0, y1 = x1;
                    if (pro) {
                        float c0v = w0[3] * x0, c1v = w1[3] * x1;
#pragma unroll
                        for (int i = 0; i < 3; ++i) {
                            c0v += w0[i] * h0[i];
                            c1v += w1[i] * h1[i];
                        }
                        h0[0] = h0[1]; h0[1] = h0[2]; h0[2] = x0;
                        h1[0] = h1[1]; h1[1] = h1[2]; h1[2] = x1;
                        y0 = c0v * __builtin_amdgcn_rcpf(1.f + __expf(-c0v));
                        y1 = c1v * __builtin_amdgcn_rcpf(1.f + __expf(-c1v));
                        if (j == jc && cstate) {  // committed: carry the last cw - 1 pre-activations
                            // through a descriptor over this (sequence, head)'s rows: the base stays
                            // uniform and each store takes one 32-bit lane offset, so no per-lane
                            // 64-bit address is kept live across the token loop
                            const __amdgpu_buffer_rsrc_t crs = __builtin_amdgcn_make_buffer_rsrc(
                                cstate, 0, (cw - 1) * CC * (int)sizeof(T), 0x00020000);
#pragma unroll
                            for (int i = 0; i < 3; ++i) {
                                const int r = i - 4 + cw;
                                if (r >= 0) {
                                    elem_store<T>(crs, (r * CC + (int)c0) * (int)sizeof(T), from_f<T>(h0[i]));
                                    if (kr) elem_store<T>(crs, (r * CC + (int)c1) * (int)sizeof(T), from_f<T>(h1[i]));
                                }
                            }
                        }
                    }
                    if (kr) {  // y0 = a_q, y1 = a_k
                        float g = to_f<T>(a0[jj]);
                        g = p.A_log ? gate_from_logit(g, eA, p.g_min) : clamp_logdecay(g, p.g_min);
                        pr *= __expf(g);
                        s_kd[j][ch] = pr * y1;
                        s_qd[j][ch] = pr * y0;
                        s_ki[j][ch] = y1 * __builtin_amdgcn_rcpf(pr);
                        if (j == jc) s_pc[ch] = pr;
                        if (j == nb - 1) s_pe[ch] = pr;
                        kq = y1 * y0;
                        ssk = y1 * y1;
                        ssq = y0 * y0;
                    } else {   // y0 = value after the prologue
                        s_v[j][ch] = y0;
                        if (epi) s_gt[j][ch] = __builtin_amdgcn_rcpf(1.f + __expf(-x1));
                    }
                    kq = wave_sum(kq);
                    if (l == 0) s_kqw[w][j] = kq;
                    if (pro) {
                        ssk = wave_sum(ssk);
                        ssq = wave_sum(ssq);
                        if (l == 0) {
                            s_sk[FU ? w : 0][FU ? j : 0] = ssk;
                            s_sq[FU ? w : 0][FU ? j : 0] = ssq;
                        }
                    }
                    if (tl == 0) s_b[j] = pro ? __builtin_amdgcn_rcpf(1.f + __expf(-bt[jj])) : bt[jj];
                }
            }
        } else {
            constexpr int RPT = (DK + NT - 1) / NT;  // staged rows per thread
            constexpr int CPT = (DV + NT - 1) / NT;  // staged value columns per thread
            static_assert(!FU || (RPT == 1 && CPT == 1), "prologue staging assumes one row and one column per thread");
            T gz[TB][RPT], kk[TB][RPT], qq[TB][RPT], vr[TB][CPT], bt[TB], gl[FT][CPT];
            // The thread index, opaque to the compiler inside this block: the
            // per-thread addresses are recomputed here instead of being hoisted out
            // of the block loop and kept live beside the state.
            int tl = t;
            if constexpr (FU) asm volatile("" : "+v"(tl));
#pragma unroll
            for (int j = 0; j < TB; ++j) {
                const int it = base + j;
                const bool ok = j < nb, rep = it < n_rep;
                const size_t row = ok ? row_of(it) : 0;
#pragma unroll
                for (int i = 0; i < RPT; ++i) {
                    const int r = tl + i * NT;
                    const bool rk = ok && r < DK;
                    gz[j][i] = rk ? ((const T *)(rep ? p.g_r : p.g))[row * DK + r] : from_f<T>(0.f);
                    kk[j][i] = rk ? ((const T *)(rep ? p.k_r : p.k))[row * DK + r] : from_f<T>(0.f);
                    if constexpr (FU)  // with the prologue the replayed queries feed the convolution
                        qq[j][i] = (rk && (pro || !rep)) ? ((const T *)(rep ? p.q_r : p.q))[row * DK + r] : from_f<T>(0.f);
                    else
                        qq[j][i] = (rk && !rep) ? ((const T *)p.q)[row * DK + r] : from_f<T>(0.f);
                }
#pragma unroll
                for (int i = 0; i < CPT; ++i) {
                    const int cc = tl + i * NT;
                    vr[j][i] = (ok && cc < DV) ? ((const T *)(rep ? p.v_r : p.v))[row * DV + cc] : from_f<T>(0.f);
                    if constexpr (FU)
                        gl[j][i] = (epi && ok && !rep && cc < DV) ? ((const T *)p.f.gate)[row * DV + cc] : from_f<T>(0.f);
                }
                bt[j] = (ok && tl == 0) ? ((const T *)(rep ? p.beta_r : p.beta))[row] : from_f<T>(0.f);
            }
            float wq[4] = {0.f, 0.f, 0.f, 0.f}, wk[4] = {0.f, 0.f, 0.f, 0.f}, wv[4] = {0.f, 0.f, 0.f, 0.f};
            float hq[3] = {0.f, 0.f, 0.f}, hk[3] = {0.f, 0.f, 0.f}, hv[3] = {0.f, 0.f, 0.f};
            if constexpr (FU) {
                if (pro) {
#pragma unroll
                    for (int i = 0; i < 3; ++i) {
                        if (tl < DK) {
                            hq[i] = s_hist[i][tl];
                            hk[i] = s_hist[i][DK + tl];
                        }
                        if (tl < DV) hv[i] = s_hist[i][2 * DK + tl];
                    }
                    // taps, newest last, zero-padded at the old end
                    const float *wb = p.f.conv_weight + (size_t)h * CC * cw;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {  // tap i holds weight i - 4 + cw (if any)
                        const int x = i - 4 + cw;
                        if (x >= 0) {
                            if (tl < DK) {
                                wq[i] = wb[tl * cw + x];
                                wk[i] = wb[(DK + tl) * cw + x];
                            }
                            if (tl < DV) wv[i] = wb[(2 * DK + tl) * cw + x];
                        }
                    }
                }
            }
            float pr[RPT];                        // running product of alpha for this thread's rows
#pragma unroll
            for (int i = 0; i < RPT; ++i) pr[i] = 1.f;
#pragma unroll
            for (int j = 0; j < TB; ++j) {
                if (j >= nb) break;
                float kq = 0.f, ssk = 0.f, ssq = 0.f;
                float av = 0.f;
                if constexpr (FU) {
                    if (pro) {  // ShortConv + Swish (eq. (2)); conv history advances
                        const float xq = to_f<T>(qq[j][0]), xk = to_f<T>(kk[j][0]), xv = to_f<T>(vr[j][0]);
                        float cq = wq[3] * xq, ck = wk[3] * xk, cv = wv[3] * xv;
#pragma unroll
                        for (int i = 0; i < 3; ++i) {
                            cq += wq[i] * hq[i];
                            ck += wk[i] * hk[i];
                            cv += wv[i] * hv[i];
                        }
                        hq[0] = hq[1]; hq[1] = hq[2]; hq[2] = xq;
                        hk[0] = hk[1]; hk[1] = hk[2]; hk[2] = xk;
                        hv[0] = hv[1]; hv[1] = hv[2]; hv[2] = xv;
                        const float aq = cq / (1.f + __expf(-cq)), ak = ck / (1.f + __expf(-ck));
                        av = cv / (1.f + __expf(-cv));
                        if (j == jc && cstate) {  // committed: carry the last cw - 1 pre-activations
#pragma unroll
                            for (int i = 0; i < 3; ++i) {
                                const int r = i - 4 + cw;
                                if (r >= 0) {
                                    if (tl < DK) {
                                        cstate[r * CC + tl] = from_f<T>(hq[i]);
                                        cstate[r * CC + DK + tl] = from_f<T>(hk[i]);
                                    }
                                    if (tl < DV) cstate[r * CC + 2 * DK + tl] = from_f<T>(hv[i]);
                                }
                            }
                        }
                        if (tl < DK) {
                            float g = to_f<T>(gz[j][0]);
                            g = p.A_log ? gate_from_logit(g, eA, p.g_min) : clamp_logdecay(g, p.g_min);
                            pr[0] *= __expf(g);
                            s_kd[j][tl] = pr[0] * ak;
                            s_qd[j][tl] = pr[0] * aq;
                            s_ki[j][tl] = ak / pr[0];
                            if (j == jc) s_pc[tl] = pr[0];
                            if (j == nb - 1) s_pe[tl] = pr[0];
                            kq = ak * aq;
                            ssk = ak * ak;
                            ssq = aq * aq;
                        }
                    }
                }
                if (!pro) {
#pragma unroll
                    for (int i = 0; i < RPT; ++i) {
                        const int r = tl + i * NT;
                        if (r < DK) {
                            float g = to_f<T>(gz[j][i]);
                            g = p.A_log ? gate_from_logit(g, eA, p.g_min) : clamp_logdecay(g, p.g_min);
                            const float kr = to_f<T>(kk[j][i]), qr = to_f<T>(qq[j][i]);
                            pr[i] *= __expf(g);
                            s_kd[j][r] = pr[i] * kr;
                            s_qd[j][r] = pr[i] * qr;
                            s_ki[j][r] = kr / pr[i];
                            if (j == jc) s_pc[r] = pr[i];
                            if (j == nb - 1) s_pe[r] = pr[i];
                            kq += kr * qr;
                        }
                    }
                }
                kq = wave_sum(kq);
                if (l == 0) s_kqw[w][j] = kq;
                if constexpr (FU) {
                    if (pro) {
                        ssk = wave_sum(ssk);
                        ssq = wave_sum(ssq);
                        if (l == 0) {
                            s_sk[w][j] = ssk;
                            s_sq[w][j] = ssq;
                        }
                    }
                    if (epi && tl < DV) s_gt[j][tl] = 1.f / (1.f + __expf(-to_f<T>(gl[j][0])));
                }
#pragma unroll
                for (int i = 0; i < CPT; ++i) {
                    const int cc = tl + i * NT;
                    if (cc < DV) s_v[j][cc] = pro ? av : to_f<T>(vr[j][i]);
                }
                if (t == 0) {
                    const float b = to_f<T>(bt[j]);
                    s_b[j] = pro ? 1.f / (1.f + __expf(-b)) : b;
                }
            }
            if constexpr (FU) {
                if (pro) {
#pragma unroll
                    for (int i = 0; i < 3; ++i) {
                        if (t < DK) {
                            s_hist[i][tl] = hq[i];
                            s_hist[i][DK + tl] = hk[i];
                        }
                        if (tl < DV) s_hist[i][2 * DK + tl] = hv[i];
                    }
                }
            }
        }
        __syncthreads();
        // Rows in groups of GR; the scheduling barriers keep the compiler from
        // hoisting every group's LDS reads (which would need ~3 x 64 registers).
        constexpr int GR = 16;
        for (int j = 0; j < nb; ++j) {
            const int it = base + j;
            const bool rep = it < n_rep;          // uniform across the workgroup
            const float *kd = &s_kd[j][r0h], *qd = &s_qd[j][r0h], *ki = &s_ki[j][r0h];
            float nk = 1.f, nq = 1.f;             // 1 / |a_k|, 1 / |a_q| (prologue)
            if constexpr (FU) {
                if (pro) {
                    float a = 0.f, b = 0.f;
#pragma unroll
                    for (int x = 0; x < NW; ++x) {
                        a += s_sk[x][j];
                        b += s_sq[x][j];
                    }
                    nk = rsq_norm(a + p.f.qk_eps);
                    nq = rsq_norm(b + p.f.qk_eps);
                }
            }
            float pp = 0.f, rr = 0.f;
            if constexpr (RB) {
                float kv[4], qv[4];           // rows r0h + 16 v + (l % 16)
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    kv[v] = kd[16 * v + (l & 15)];
                    qv[v] = rep ? 0.f : qd[16 * v + (l & 15)];
                }
                dot16<0, 4>(pp, kv[0], st); dot16<1>(pp, kv[1], st); dot16<2>(pp, kv[2], st); dot16<3>(pp, kv[3], st);
                if (!rep) {
                    dot16<0, 4>(rr, qv[0], st); dot16<1>(rr, qv[1], st); dot16<2>(rr, qv[2], st);
                    dot16<3>(rr, qv[3], st);
                }
            } else {
#pragma unroll
                for (int g0 = 0; g0 < RH; g0 += GR) {
#pragma unroll
                    for (int r = g0; r < g0 + GR; r += 4) {
                        const f32x4 k4 = *reinterpret_cast<const f32x4 *>(kd + r);
#pragma unroll
                        for (int e = 0; e < 4; ++e) pp += st[r + e] * k4[e];
                    }
                    if (!rep) {
#pragma unroll
                        for (int r = g0; r < g0 + GR; r += 4) {
                            const f32x4 q4 = *reinterpret_cast<const f32x4 *>(qd + r);
#pragma unroll
                            for (int e = 0; e < 4; ++e) rr += st[r + e] * q4[e];
                        }
                    }
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
            if (NH == 2) {                        // the other 64 rows of the column
                pp = pair_sum32(pp);
                if (!rep) rr = pair_sum32(rr);
            }
            if constexpr (FU) {
                pp *= nk;
                rr *= nq;
            }
            const float d = s_b[j] * (s_v[j][col] - pp);
            if (!rep && hf == 0) {
                float kq = 0.f;
#pragma unroll
                for (int x = 0; x < NW; ++x) kq += s_kqw[x][j];
                if constexpr (FU) kq *= nk * nq;
                const float ot = p.scale * (rr + d * kq);
                if (FU && epi) {
                    int cl = col;
                    asm volatile("" : "+v"(cl));  // the address is formed here, not kept from before the loop
                    s_o[FU ? j : 0][FU ? cl : 0] = ot;
                } else {
                    ((T *)p.o)[row_of(it) * DV + col] = from_f<T>(ot);
                }
            }
            const float du = FU ? d * nk : d;     // k = a_k / |a_k| in the update
            if constexpr (RB) {
                float iv[4];
#pragma unroll
                for (int v = 0; v < 4; ++v) iv[v] = ki[16 * v + (l & 15)];
                // EXEC may have changed for the output store just above
                upd16<0, 4>(st, iv[0], du); upd16<1>(st, iv[1], du); upd16<2>(st, iv[2], du); upd16<3>(st, iv[3], du);
            } else {
#pragma unroll
                for (int g0 = 0; g0 < RH; g0 += GR) {
#pragma unroll
                    for (int r = g0; r < g0 + GR; r += 4) {
                        const f32x4 i4 = *reinterpret_cast<const f32x4 *>(ki + r);
#pragma unroll
                        for (int e = 0; e < 4; ++e) st[r + e] += i4[e] * du;
                    }
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
            if (j == jc) {                        // write back the true state X * P
#pragma unroll
                for (int r = 0; r < RH; r += 4) {
                    const f32x4 p4 = *reinterpret_cast<const f32x4 *>(&s_pc[r0h + r]);
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, st[r + e] * p4[e]), srs,
                                                              lane_off, (r + e) * ROW, NT_AUX);
                }
            }
        }
        if constexpr (FU) {
            if (epi && base + nb > n_rep) {       // eq. (6) over the block's new tokens
                __syncthreads();                  // every column's o~ is in LDS
                int te = t;
                asm volatile("" : "+v"(te));      // as in staging: no hoisted addresses
                const int le = te & 63;
                const float wo = (te < DV) ? p.f.o_weight[(size_t)h * DV + te] : 0.f;
                for (int j = max(n_rep - base, 0); j < nb; ++j) {
                    float ss = 0.f;
#pragma unroll
                    for (int c = 0; c < DV; c += 64) ss += s_o[j][c + le] * s_o[j][c + le];
                    ss = wave_sum(ss);
                    if (te < DV) {
                        const float y = s_gt[j][te] * wo * s_o[j][te] * rsq_norm(ss * (1.f / DV) + p.f.o_eps);
                        ((T *)p.o)[row_of(base + j) * DV + te] = from_f<T>(y);
                    }
                }
            }
        }
        if (base + TB < n_tok) {
            // Leave the scaled frame before the next block restarts the products.
#pragma unroll
            for (int r = 0; r < RH; r += 4) {
                const f32x4 p4 = *reinterpret_cast<const f32x4 *>(&s_pe[r0h + r]);
#pragma unroll
                for (int e = 0; e < 4; ++e) st[r + e] *= p4[e];
            }
            __syncthreads();  // the block is read to the end before the next is staged
        }
    }
}

// The plain single decode step is bound by HBM.  Its registers allow three
// resident workgroups per CU; two keep fewer state streams in flight at once,
// which the HBM serves faster (about 1% per step at 512 x 32 heads of
// 128 x 128; one per CU is far slower).  An unused dynamic LDS allocation caps
// residency at two: with the kernel's static LDS (1.5 to 3 KiB) each workgroup
// holds 57.5 to 59 KiB, more than a third of the CU's 160 KiB and less than
// the 64 KiB a launch may take without raising its limit.  The fused single
// step and the windows do more VALU work per state element: they need more
// workgroups in flight, not fewer, and launch without the pad.
constexpr size_t kDecodeOccupancyPad = 56 * 1024;

template <typename T, int DK, int DV, bool FU>
static void launch_replay_tb(const ReplayParams &p, hipStream_t stream)
{
    const unsigned grid = (unsigned)((size_t)p.N * p.H);
    const dim3 block(DV * (DK / 64));
    if (p.T_replay + p.T_new == 1)  // one token per sequence: the single decode step
        hipLaunchKernelGGL((replay_kernel<T, DK, DV, 1, FU>), dim3(grid), block, FU ? 0 : kDecodeOccupancyPad,
                           stream, p);
    else
        hipLaunchKernelGGL((replay_kernel<T, DK, DV, 8, FU>), dim3(grid), block, 0, stream, p);
}

template <typename T, int DK, int DV>
static hipError_t launch_replay_t(const ReplayParams &p, hipStream_t stream)
{
    if (p.f.conv_w > 0 || p.f.gate)
        launch_replay_tb<T, DK, DV, true>(p, stream);
    else
        launch_replay_tb<T, DK, DV, false>(p, stream);
    return hipGetLastError();
}

hipError_t launch_recurrent_replay(int dtype_bf16, int Dk, int Dv, const ReplayParams &p, hipStream_t stream)
{
#define KDA_REPLAY_CASE(TT, DKV, DVV) \
    if (Dk == DKV && Dv == DVV) return launch_replay_t<TT, DKV, DVV>(p, stream);
    if (dtype_bf16) {
        KDA_REPLAY_CASE(bf16, 64, 64)
        KDA_REPLAY_CASE(bf16, 64, 128)
        KDA_REPLAY_CASE(bf16, 128, 64)
        KDA_REPLAY_CASE(bf16, 128, 128)
    } else {
        KDA_REPLAY_CASE(float, 64, 64)
        KDA_REPLAY_CASE(float, 64, 128)
        KDA_REPLAY_CASE(float, 128, 64)
        KDA_REPLAY_CASE(float, 128, 128)
    }
#undef KDA_REPLAY_CASE
    return hipErrorInvalidValue;
}

}  // namespace kda
