// kda_prefill.hip -- chunkwise-parallel KDA forward over whole sequences.
//
// "Kimi K3 Technical Report: Open Frontier Intelligence", §2.1.1:
//   eq. (3)  per-channel cumulative decay inside a chunk, kept in log space:
//            lam_r = sum_{s<=r} g_s, so gamma^r = exp(lam_r);
//   eq. (4)  A = Tril[(Q*Gamma)(K/Gamma)^T] (diagonal kept) and
//            O = (Gamma*Q) S + A V~;
//   "UT transform"  U, W with pseudo-values V~ = U - W S;
//   eq. (5)  lower-bounded gate: g > g_min = -5, so the log-decay summed over
//            a 16-token sub-tile lies in (-80, 0] and its reciprocal rescale
//            factors stay below e^80, inside the bf16/fp32 range
//            ("lower-bounded decay" paragraph and Fig. 3).
// U, W and the hand-off between chunks are not printed on the page; unrolling
// eq. (1) over one chunk entered with state S gives
//   L     = StrictTril(Diag(beta) K+ K-^T),   K+ = K*Gamma, K- = K/Gamma
//   T'    = (I + L)^-1 Diag(beta)
//   U     = T' V,   W = T' K+,   V~ = U - W S
//   S_out = Diag(gamma^C) S + (K * gamma^C / Gamma)^T V~.
// §5.1.1 describes the production kernel as token-parallel stages plus a
// head-parallel recurrence; the same split is used here, laid out for gfx950:
//
//   chunk_table_kernel   (packed sequences only) clamped spans, chunk offsets
//                        per sequence and a longest-first sequence order.
//   intra_chunk_kernel   persistent over (chunk, head) items: gate, cumsum,
//                        sub-tile Gram products on MFMA, blocked triangular
//                        inverse in fp32, U / W / A on MFMA; with the layer
//                        prologue (eq. (2)) the inputs are first convolved,
//                        passed through Swish, L2-normalised (q, k) and Sigmoid
//                        (beta) in registers.  In the split design it writes
//                        every operand of the chain as a ready-to-issue MFMA
//                        fragment (layout in Block below).  In pair mode (128
//                        or more (sequence, head) pairs at bf16, d_k = 128, no
//                        prologue) each workgroup walks whole pairs chunk by
//                        chunk and runs the chain step itself from the chunk's
//                        block in LDS: no chain kernel, no block in HBM.
//   chain_kernel         split design, fewer than 128 pairs: one workgroup per
//                        (sequence, head, 16-column slice of d_v), walking the
//                        chunks in order with its slice of S in fp32 registers;
//                        per chunk two dependent MFMA products (W S, then
//                        K~^T V~) sit on the serial path and the output products
//                        (Q+ S, A V~) beside them.  Columns of S evolve
//                        independently (V~ = U - W S acts column by column),
//                        which licenses the split.
//   chain_wide_kernel    split design from 128 pairs (when pair mode does not
//                        apply): one workgroup per (sequence, head), all d_v
//                        columns, each chunk's block copied whole into LDS.
//   gate_norm_kernel     the layer epilogue (eq. (6)) in place on o.
//
// Sub-tile references.  Let B_m be lam just before 16-token tile m (B_0 = 0).
// For rows r in tile m and columns i in tile n <= m, exp(lam_r - lam_i) is
// factored at B_m: the row operand exp(lam_r - B_m) in [e^-80, 1] times the
// column operand exp(B_m - lam_i), which lies in [1, e^80] for n = m and is
// <= 1 for n < m.  No factor overflows; a column factor that underflows
// belongs to a product exp(lam_r - lam_i) below the smallest normal float.
#include "kda_common.h"
#include "kda_prefill.h"
#include "kda_table.h"

namespace kda {

// -----------------------------------------------------------------------------
// Per (head, chunk) workspace block written by intra_chunk_kernel and read by
// the chain kernels.  Element type T except gamma (fp32).  "wave w" is the
// slice chain's wave index: token rows 16w..16w+15 of the chunk, and state rows
// 16*RT*w .. 16*RT*(w+1)-1.  All fragments use kmap() along k.
//   Wn  [4 waves][KS][64 lanes][8]  A-operand fragments of -W    (rows tokens, k channels)
//   Qp  [4 waves][KS][64][8]        operand fragments of scale*Q*Gamma (rows tokens, k channels)
//   Kt  [4 waves][RT][2][64][8]     A-operand fragments of (K*gamma^C/Gamma)^T (rows channels, k tokens)
//   A   [4 waves][2][64][8]         A-operand fragments of A     (rows tokens, k tokens)
//   gamma [DK] float                gamma^C = exp(lam at the chunk's last token)
//   U   [NS][4 waves][64][4]        accumulator quads of U
// Everything up to U is what every wave of the wide chain reads; with U right
// behind it the block is one contiguous run that the wide chain copies into
// LDS in 1 KiB pieces (the block is a whole number of them).
// -----------------------------------------------------------------------------
template <typename T, int DK, int DV> struct Block {
    static constexpr int KS = DK / 32;
    static constexpr int RT = DK / 64;
    static constexpr int NS = DV / 16;
    static constexpr size_t W_OFF = 0;
    static constexpr size_t Q_OFF = W_OFF + (size_t)4 * KS * 512;
    static constexpr size_t KT_OFF = Q_OFF + (size_t)4 * KS * 512;
    static constexpr size_t A_OFF = KT_OFF + (size_t)4 * RT * 2 * 512;
    static constexpr size_t GAMMA_BYTE = (A_OFF + (size_t)4 * 2 * 512) * sizeof(T);
    static constexpr size_t STAGE_BYTES = GAMMA_BYTE + DK * sizeof(float);
    static constexpr size_t U_BYTE = STAGE_BYTES;
    static constexpr size_t U_OFF = U_BYTE / sizeof(T);
    static constexpr size_t U_BYTES = (size_t)NS * 4 * 256 * sizeof(T);
    static constexpr size_t BYTES = (U_BYTE + U_BYTES + 1023) / 1024 * 1024;
    static_assert(U_BYTE % 16 == 0, "U quads must stay 16-byte aligned");
};

size_t block_bytes(int bf16_, int Dk, int Dv)
{
#define KDA_BB(TT, A, B) \
    if (Dk == A && Dv == B) return Block<TT, A, B>::BYTES;
    if (bf16_) {
        KDA_BB(bf16, 64, 64) KDA_BB(bf16, 64, 128) KDA_BB(bf16, 128, 64) KDA_BB(bf16, 128, 128)
    } else {
        KDA_BB(float, 64, 64)
    }
#undef KDA_BB
    return 0;
}

// -----------------------------------------------------------------------------
// Packed sequences: the chunk table (layout and clamping in kda_table.h).  One
// workgroup of table::THREADS threads; the chunk counts are scanned in LDS in
// 64-bit, so no sum overflows before it saturates at the capacity.
// -----------------------------------------------------------------------------
__global__ __launch_bounds__(table::THREADS) void chunk_table_kernel(const int32_t *__restrict__ cu, int N, int T,
                                                                    int cap, int32_t *__restrict__ chunk_off,
                                                                    int32_t *__restrict__ order,
                                                                    int32_t *__restrict__ span)
{
    __shared__ long long part[table::THREADS];
    const int t = threadIdx.x;
    const long long local = table::count(cu, N, T, t, span);
    part[t] = local;
    __syncthreads();
    for (int d = 1; d < table::THREADS; d <<= 1) {  // inclusive scan
        const long long add = (t >= d) ? part[t - d] : 0;
        __syncthreads();
        part[t] += add;
        __syncthreads();
    }
    table::offsets(cu, N, T, cap, t, part[t] - local, chunk_off);
    if (t == table::THREADS - 1) chunk_off[N] = part[t] < cap ? (int)part[t] : cap;
    for (int s = t; s < N; s += table::THREADS) order[table::rank(cu, N, T, s)] = s;
}

// -----------------------------------------------------------------------------
// Intra-chunk stage.  512 threads = 8 waves.  The grid is persistent: each
// workgroup walks (chunk, head) items with a stride of gridDim.x, from the
// last chunk to the first (the blocks the chain kernel reads first are
// written last and are the likeliest to still sit in the last-level cache),
// and the raw inputs of its next item are loaded into registers while the
// current item is computed.
//
// Elementwise layout: wave w owns 8 tokens of a 16-token sub-tile (the first
// or second half, w / 4; see seg_tile) and lane l owns the CPT channels CPT*l..
// (CPT = d_k/64) across those 8 tokens, so the chunk-local cumsum runs inside
// each thread and only the eight half-tile totals are exchanged.  Log-decays
// are kept in log2 units (one exp2 per factor).
//
// Sub-tile references.  Let B_m be lam just before tile m (B_0 = 0) and
// T_m = B_{m+1} - B_m <= 0 the tile's total.  Row operands carry
// exp(lam_r - B_m) in [e^-80, 1]; the column operand met by row tile m
// carries exp(B_m - lam_i): for i in tile m (diagonal pair) that lies in
// [1, e^80] (inside the bf16 and fp32 range, the "lower-bounded decay"
// argument of §2.1.1), for i in an earlier tile it is <= 1.  The column
// operands of all ten (m, n) pairs are formed here, so the Gram products need
// no rescaling.
// -----------------------------------------------------------------------------
template <typename T, int N> struct Vec { typedef T type __attribute__((ext_vector_type(N))); };

constexpr float LOG2E = 1.4426950408889634f;

// LDS layouts.  The pitches and the XOR swizzles below keep every access of the
// kernel free of LDS bank conflicts on gfx950, whose LDS serves a 16-byte read
// for lanes {0-3, 20-23}, {4-7, 16-19}, {8-11, 28-31}, {12-15, 24-27} (and the
// same +32) on 32 four-byte banks, an 8-byte read for 32 lanes on 64 banks, and
// each address of a two-address 8-byte read for 16 consecutive lanes on 32 banks
// (measured with the bank-conflict counter).  Swizzles permute 8-element blocks
// within a row, so 16-byte fragments stay contiguous.
//
// Token-major operand rows (KR, QR, KC) hold each 32-channel k-step in the
// fragment order of the chain's products (channels 4j..4j+3 and 16+4j..16+4j+3
// at 8j..8j+7): the Q+ fragments are then plain 16-byte reads, and the Gram
// products, which read the same positions from the rows they pair, are
// unchanged (kpos gives the position of a channel).
// KpT, VT (row = channel): 8-token block b of row r sits at b ^ swz_kv(r).
__device__ __forceinline__ int swz_kv(int r) { return ((r >> 1) & 1) | (((r >> 2) & 1) << 1) | (((r ^ (r >> 3)) & 1) << 2); }
// Tp (row = token): 8-column block b of row r sits at b ^ swz_tp(r).
__device__ __forceinline__ int swz_tp(int r) { return (r >> 2) & 1; }
// L and the D blocks inside it (fp32): column c of row r sits at c ^ swz_l(r),
// which moves 4-column groups within 8-column groups.
__device__ __forceinline__ int swz_l(int r) { return 4 * ((r >> 2) & 1); }

template <typename T, int DK, int DV> struct IntraSmem {
    static constexpr int PR = DK + 16;    // row of the token-major operand arrays
    static constexpr int PT = CHUNK + 8;  // row of Tp
    static constexpr int PV = CHUNK;      // row of KpT and VT (swizzled)
    static constexpr int PK = CHUNK + 4;  // row of KtT: its 16-byte writes and two-address 8-byte reads stay conflict-free
    static constexpr int LP = CHUNK + 4;  // fp32 row pitch of L and its inverse
    // Column-operand rows: [0,64) exp(B_n - lam) for tile n (diagonal pairs);
    // [64,112) exp(B_{n+1} - lam) for tiles 0..2 (pairs (n+1, n)); [112,128)
    // tile 0 at B_2; [128,144) tile 0 at B_3; [144,160) tile 1 at B_3.
    static constexpr int NCOL = 160;
    struct {
        T KR[CHUNK][PR];   // k * exp(lam - B_m): row operand of L (P1 -> P2)
        T QR[CHUNK][PR];   // scale * q * exp(lam - B_m): row operand of A (P1 -> P3)
    } ops;
    // Lower 16x16 blocks: Diag(beta) StrictTril(K+ K-^T) (P2 -> P3); four of the
    // unused upper blocks hold the diagonal inverses D_m (P3), see dblk().
    float L[CHUNK][LP];
    union {
        T KC[NCOL][PR];    // column operands (P1 -> P2)
        struct {
            T keep[CHUNK][PR];  // diagonal column operands (not reused)
            T Tp[CHUNK][PT];    // (I + L)^-1 Diag(beta) (P3 -> P4)
        } t;
    } y;
    T KpT[DK][PV];         // (k * exp(lam))^T, A operand of W^T
    T KtT[DK][PK];         // (k * exp(lam_C - lam))^T, copied out as the chain's K~^T fragments (P1 -> P3)
    T VT[DV][PV];          // v^T, B operand of U
    float tot[8][DK];      // half-tile (8-token segment) totals (log2 units)
    float eB[4][DK];       // exp(B_m) per tile and channel (P1 -> P3)
    float beta[CHUNK];
    float gam[DK];         // gamma^C of the chunk (pair mode: P1 -> chain step)
};

// Upper block of L that holds D_m = (I + L_mm)^-1: (0,1), (0,2), (0,3), (1,2).
template <typename SM> __device__ __forceinline__ float *dblk(SM &sm, int m)
{
    return &sm.L[m == 3 ? 16 : 0][m == 3 ? 32 : 16 * (m + 1)];
}

__device__ __forceinline__ int colop_row(int m, int n)
{
    if (m == n) return 16 * n;
    if (m == n + 1) return 64 + 16 * n;
    return (n == 0) ? (m == 2 ? 112 : 128) : 144;
}

// Eight waves; wave w owns the first (w < 4) or second half of sub-tile
// seg_tile(w), i.e. tokens seg_base(w) .. +7.  Waves 4-7 take the sub-tiles in
// reverse order: the elementwise pass forms four column-operand rows per token
// of tile 0, three of tile 1, two of tile 2 and one of tile 3, and waves w and
// w + 4 usually share a SIMD, which then holds five either way.
constexpr int IWAVES = 8, HT = SUB / 2;
__device__ __forceinline__ int seg_tile(int w) { return w < 4 ? w : 7 - w; }
__device__ __forceinline__ int seg_base(int w) { return SUB * seg_tile(w) + HT * (w >> 2); }

// Raw inputs of one (chunk, head) in registers, unconverted (converting at
// load time would make the wave wait for the loads): lane l of wave w holds
// channels CPT*l.. of the wave's 8 tokens of g, k, q, value columns CPV*l..
// of the same tokens, and (lanes 0..7) beta of token seg_base(w) + l.
template <typename T, int DK, int DV> struct RawIn {
    static constexpr int CPT = DK / 64, CPV = DV / 64;
    typedef typename Vec<T, CPT>::type ku;
    typedef typename Vec<T, CPV>::type vu;
    ku g[HT], k[HT], q[HT];
    vu v[HT];
    T beta;
    float alog;
};

template <typename T, int DK, int DV>
__device__ __forceinline__ void load_raw(RawIn<T, DK, DV> &in, const PrefillParams &p, int tok0, int len,
                                         int h, int w, int l)
{
    using R = RawIn<T, DK, DV>;
    typedef typename R::ku ku;
    typedef typename R::vu vu;
    const T *gg = (const T *)p.g, *kg = (const T *)p.k, *qg = (const T *)p.q, *vg = (const T *)p.v;
    ku zk;
    vu zv;
#pragma unroll
    for (int c = 0; c < R::CPT; ++c) zk[c] = from_f<T>(0.f);
#pragma unroll
    for (int c = 0; c < R::CPV; ++c) zv[c] = from_f<T>(0.f);
    const int tb = seg_base(w);
#pragma unroll
    for (int r = 0; r < HT; ++r) {
        const int tok = tb + r;
        const bool ok = tok < len;
        const size_t row = (size_t)(tok0 + tok) * p.H + h;
        in.g[r] = ok ? *reinterpret_cast<const ku *>(gg + row * DK + R::CPT * l) : zk;
        in.k[r] = ok ? *reinterpret_cast<const ku *>(kg + row * DK + R::CPT * l) : zk;
        in.q[r] = ok ? *reinterpret_cast<const ku *>(qg + row * DK + R::CPT * l) : zk;
        in.v[r] = ok ? *reinterpret_cast<const vu *>(vg + row * DV + R::CPV * l) : zv;
    }
    const int bt = tb + l;
    in.beta = (l < HT && bt < len) ? ((const T *)p.beta)[(size_t)(tok0 + bt) * p.H + h] : from_f<T>(0.f);
    in.alog = p.A_log ? p.A_log[h] : 0.f;
}

// Uniform read of a table the kernel never writes, through the scalar cache:
// its completion is counted apart from the vector loads and stores, so the
// waits it needs do not also wait for outstanding result stores.
__device__ __forceinline__ int ld_uniform(const int32_t *ptr, int i)
{
    return ((const __attribute__((address_space(4))) int32_t *)ptr)[i];
}

// Raw buffer load of a 2-, 4- or 8-byte vector; offsets at or past the
// descriptor's record count read as zero.
template <typename V> __device__ __forceinline__ V buf_load(__amdgpu_buffer_rsrc_t rs, int voff)
{
    if constexpr (sizeof(V) == 2)
        return __builtin_bit_cast(V, __builtin_amdgcn_raw_buffer_load_b16(rs, voff, 0, 0));
    else if constexpr (sizeof(V) == 4)
        return __builtin_bit_cast(V, __builtin_amdgcn_raw_buffer_load_b32(rs, voff, 0, 0));
    else
        return __builtin_bit_cast(V, __builtin_amdgcn_raw_buffer_load_b64(rs, voff, 0, 0));
}

// Raw buffer store of a 2-, 4-, 8- or 16-byte vector; offsets at or past the
// descriptor's record count are dropped.
template <typename V> __device__ __forceinline__ void buf_store(__amdgpu_buffer_rsrc_t rs, int voff, V v)
{
    if constexpr (sizeof(V) == 2)
        __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(uint16_t, v), rs, voff, 0, 0);
    else if constexpr (sizeof(V) == 4)
        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), rs, voff, 0, 0);
    else if constexpr (sizeof(V) == 8)
    {
        typedef unsigned u32x2 __attribute__((vector_size(8)));
        __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, v), rs, voff, 0, 0);
    }
    else
    {
        static_assert(sizeof(V) == 16, "2, 4, 8 or 16 bytes");
        typedef unsigned u32x4 __attribute__((vector_size(16)));
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), rs, voff, 0, 0);
    }
}

// With the layer prologue folded into the intra-chunk stage: the 3 projection
// rows before the wave's 8 tokens (for its convolution) and the filter taps of
// this lane's query, key and value channels, loaded one item ahead like RawIn.
template <typename T, int DK, int DV> struct ProIn {
    static constexpr int CPT = DK / 64, CPV = DV / 64;
    typedef typename Vec<T, CPT>::type ku;
    typedef typename Vec<T, CPV>::type vu;
    ku hq[3], hk[3];
    vu hv[3];
    float wq[CPT][4], wk[CPT][4], wv[CPV][4];  // taps newest last, zero-padded at the old end
};

// History rows of tokens tb - 3 .. tb - 1 of a chunk: the tokens before (same
// sequence), or at a sequence start the carried convolution state's rows
// (slot i = state row i - 4 + W; older slots, or no state, read as zeros past
// the descriptors' record counts).  lc: chunk index in its sequence, sq: the
// sequence.
template <typename T, int DK, int DV>
__device__ __forceinline__ void load_hist(ProIn<T, DK, DV> &pr, const PrefillParams &p, int tok0, int len, int sq,
                                          int lc, int h, int tb, int l)
{
    using P = ProIn<T, DK, DV>;
    constexpr int C = 2 * DK + DV, EL = (int)sizeof(T), CPT = P::CPT, CPV = P::CPV;
    const int W = p.f.conv_w, rowk = p.H * DK * EL, rowv = p.H * DV * EL;
    const bool tok_hist = tb > 0 || lc > 0;
    // token rows tb - 3 + i exist for tb - 3 + i < len (rows before the chunk
    // belong to the previous chunk of the sequence); the record counts end at
    // the last of them, so a wave past the chunk's tokens reads nothing
    const int nh = tok_hist ? min(max(len - (tb - 3), 0), 3) : 0;
    const T *cs = (const T *)p.f.conv_state;
    const bool st = !tok_hist && cs && W > 1;
    const size_t rh = tok_hist ? (size_t)(tok0 + tb - 3) * p.H + h : 0;
    const T *sb = st ? cs + ((size_t)sq * p.H + h) * (W - 1) * C : nullptr;
    const int rk = nh ? (nh - 1) * rowk + DK * EL : 0, rv = nh ? (nh - 1) * rowv + DV * EL : 0;
    const __amdgpu_buffer_rsrc_t dq = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(st ? sb : (const T *)p.q + rh * DK), 0, st ? (W - 1) * C * EL : rk, 0x00020000);
    const __amdgpu_buffer_rsrc_t dk = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(st ? sb + DK : (const T *)p.k + rh * DK), 0, st ? (W - 1) * C * EL - DK * EL : rk, 0x00020000);
    const __amdgpu_buffer_rsrc_t dv = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(st ? sb + 2 * DK : (const T *)p.v + rh * DV), 0, st ? (W - 1) * C * EL - 2 * DK * EL : rv, 0x00020000);
#pragma unroll
    for (int i = 0; i < 3; ++i) {
        const int j = i - 4 + W;
        const int sk = st ? (j >= 0 ? j * C * EL : 0x40000000) : i * rowk;  // row offset, per descriptor
        const int sv = st ? (j >= 0 ? j * C * EL : 0x40000000) : i * rowv;
        pr.hq[i] = buf_load<typename P::ku>(dq, sk + CPT * l * EL);
        pr.hk[i] = buf_load<typename P::ku>(dk, sk + CPT * l * EL);
        pr.hv[i] = buf_load<typename P::vu>(dv, sv + CPV * l * EL);
    }
}

template <typename T, int DK, int DV>
__device__ __forceinline__ void load_taps(ProIn<T, DK, DV> &pr, const PrefillParams &p, int h, int l)
{
    using P = ProIn<T, DK, DV>;
    constexpr int C = 2 * DK + DV;
    const int W = p.f.conv_w;
    const float *wb = p.f.conv_weight + (size_t)h * C * W;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int xw = e - 4 + W;
#pragma unroll
        for (int cc = 0; cc < P::CPT; ++cc) {
            pr.wq[cc][e] = xw >= 0 ? wb[(P::CPT * l + cc) * W + xw] : 0.f;
            pr.wk[cc][e] = xw >= 0 ? wb[(DK + P::CPT * l + cc) * W + xw] : 0.f;
        }
#pragma unroll
        for (int cv = 0; cv < P::CPV; ++cv) pr.wv[cv][e] = xw >= 0 ? wb[(2 * DK + P::CPV * l + cv) * W + xw] : 0.f;
    }
}

// Token range of chunk c; false if c is past the last chunk (packed tail).
__device__ __forceinline__ bool locate_chunk(const PrefillParams &p, int c, int &tok0, int &len)
{
    if (p.varlen) {
        if (c >= ld_uniform(p.chunk_off, p.N)) return false;
        int lo = 0, hi = p.N - 1;  // largest s with chunk_off[s] <= c
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (ld_uniform(p.chunk_off, mid) <= c) lo = mid; else hi = mid - 1;
        }
        const int start = ld_uniform(p.span, 2 * lo);
        tok0 = start + (c - ld_uniform(p.chunk_off, lo)) * CHUNK;
        len = min(CHUNK, start + ld_uniform(p.span, 2 * lo + 1) - tok0);
    } else {
        const int cps = (p.T + CHUNK - 1) / CHUNK;
        const int s = c / cps, lc = c - s * cps;
        tok0 = s * p.T + lc * CHUNK;
        len = min(CHUNK, p.T - lc * CHUNK);
    }
    return true;
}

// Sequence of chunk c, its index inside the sequence and the sequence's length
// (besides the token range); false if c is past the last chunk.
__device__ __forceinline__ bool locate_seq(const PrefillParams &p, int c, int &tok0, int &len, int &sq, int &lc,
                                           int &slen)
{
    if (p.varlen) {
        if (c >= ld_uniform(p.chunk_off, p.N)) return false;
        int lo = 0, hi = p.N - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (ld_uniform(p.chunk_off, mid) <= c) lo = mid; else hi = mid - 1;
        }
        sq = lo;
        lc = c - ld_uniform(p.chunk_off, lo);
        slen = ld_uniform(p.span, 2 * lo + 1);
    } else {
        const int cps = (p.T + CHUNK - 1) / CHUNK;
        sq = c / cps;
        lc = c - sq * cps;
        slen = p.T;
    }
    tok0 = (p.varlen ? ld_uniform(p.span, 2 * sq) : sq * p.T) + lc * CHUNK;
    len = min(CHUNK, slen - lc * CHUNK);
    return true;
}

// Next valid item at or after i (stride gridDim.x); items run chunk-major
// from the last chunk down.  Returns false when the walk is done.
__device__ __forceinline__ bool next_item(const PrefillParams &p, int &i, int &c, int &h, int &tok0, int &len)
{
    const int n_items = p.n_chunks_cap * p.H;
    for (; i < n_items; i += gridDim.x) {
        const int ci = i / p.H;
        h = i - ci * p.H;
        c = p.n_chunks_cap - 1 - ci;
        if (locate_chunk(p, c, tok0, len)) return true;
    }
    return false;
}

// Pair mode: workgroup b walks one (sequence, head) pair per round k, of rank
// pair_rank(k) in the chunk table's longest-first order, and each pair's chunks
// in order.  Round k deals ranks kG .. kG + G - 1 (G = gridDim.x) to the
// workgroups forwards when k is even and backwards when k is odd, so that the
// longest pairs of one round and the shortest of the next meet on one
// workgroup; on the packed 64-sequence workload the busiest workgroup then
// carries 2% more chunks than the mean instead of 11% with a plain stride.
// Ranks grow with k for every workgroup.  pair_of: the pair of rank r; false
// past the last.
__device__ __forceinline__ int pair_rank(int k)
{
    const int G = (int)gridDim.x, b = (int)blockIdx.x;
    return k * G + ((k & 1) ? G - 1 - b : b);
}
__device__ __forceinline__ bool pair_of(const PrefillParams &p, int r, int &s, int &h, int &start, int &slen, int &nch)
{
    if (r >= p.N * p.H) return false;
    const int srank = r / p.H;
    h = r - srank * p.H;
    if (p.varlen) {
        s = ld_uniform(p.order, srank);
        start = ld_uniform(p.span, 2 * s);
        slen = ld_uniform(p.span, 2 * s + 1);
        nch = ld_uniform(p.chunk_off, s + 1) - ld_uniform(p.chunk_off, s);
    } else {
        s = srank;
        start = s * p.T;
        slen = p.T;
        nch = (p.T + CHUNK - 1) / CHUNK;
    }
    return true;
}

// The chunk after (round k, lc): the pair's next chunk, else chunk 0 of this
// workgroup's next pair that has chunks; its token range.  False when done.
__device__ __forceinline__ bool pair_next(const PrefillParams &p, int &k, int &lc, int &s, int &h, int &start,
                                          int &slen, int &nch, int &tok0, int &len)
{
    if (lc + 1 < nch) {
        ++lc;
    } else {
        lc = 0;
        for (++k;; ++k) {
            if (!pair_of(p, pair_rank(k), s, h, start, slen, nch)) return false;
            if (nch > 0) break;
        }
    }
    tok0 = start + lc * CHUNK;
    len = min(CHUNK, slen - lc * CHUNK);
    return true;
}

// As next_item, with the item's sequence, its chunk index in the sequence and
// the sequence length (the folded prologue needs them).
__device__ __forceinline__ bool next_item_seq(const PrefillParams &p, int &i, int &c, int &h, int &tok0, int &len,
                                              int &sq, int &lc, int &slen)
{
    const int n_items = p.n_chunks_cap * p.H;
    for (; i < n_items; i += gridDim.x) {
        const int ci = i / p.H;
        h = i - ci * p.H;
        c = p.n_chunks_cap - 1 - ci;
        if (locate_seq(p, c, tok0, len, sq, lc, slen)) return true;
    }
    return false;
}

// ZM: decay logits z with the eq. (5) gate (A_log given), else log-decays g;
// a template parameter so the elementwise pass carries no per-element branch.
// PRO: the layer prologue (eq. (2)) folded in: q, k, v and beta hold the
// projections before the convolution and the beta logits; P1a convolves,
// applies Swish, L2Norm (q, k) and Sigmoid (beta) in registers, and writes the
// convolution state and its checkpoints from the chunks that hold them.
// PAIR: the chain runs in the same workgroup (pair mode, above): each chunk's
// block goes to LDS regions the intra-chunk work no longer needs (Q+ over the
// row operand KR, U over QR, W over L, A behind Tp, gamma^C in gam; K~^T is
// read from KtT in place), and after P4 each wave advances one 16-column tile
// of the pair's state by the chunk as the wide chain does (state columns in
// MFMA accumulators).  No block crosses HBM.
template <typename T, int DK, int DV, bool ZM, bool PRO = false, bool PAIR = false>
__global__ __launch_bounds__(512) void intra_chunk_kernel(PrefillParams p)
{
    using BL = Block<T, DK, DV>;
    using SM = IntraSmem<T, DK, DV>;
    using R = RawIn<T, DK, DV>;
    constexpr int KS = DK / 32, RT = DK / 64, CPT = R::CPT, CPV = R::CPV;
    typedef typename R::ku ku;
    typedef typename Vec<T, HT>::type tok8;
    typedef typename Vec<T, 4>::type tok4;
    extern __shared__ __align__(16) char smem_raw[];
    SM &sm = *reinterpret_cast<SM *>(smem_raw);

    const int t = threadIdx.x, w = __builtin_amdgcn_readfirstlane(t >> 6), l = t & 63, g = l >> 4, x = l & 15;
    const int ch0 = CPT * l;  // first channel of this lane in the elementwise phase
    const int m0 = seg_tile(w), hf = w >> 2, tb = seg_base(w);  // elementwise: tile, half, first token

    using PI = ProIn<T, DK, DV>;
    typedef typename PI::vu vu;
    static_assert(!PAIR || (sizeof(T) == 2 && DK == 128 && !PRO), "pair mode: bf16, d_k = 128, no prologue");
    // pair mode: wave w < NCW holds state column tile w (CT = 1), all NR row tiles
    constexpr int CT = 1, NR = DK / 16, NCW = DV / 16;
    static_assert(NCW <= IWAVES, "a chain wave per column tile");
    int i = blockIdx.x, c = 0, h = 0, tok0 = 0, len = 0, sq = 0, lc = 0, slen = 0, pst = 0, nch = 0;
    bool have;
    f32x4 S[NR][CT];  // pair mode, waves w < NCW: the pair's state, columns 16 w + x
    if constexpr (PAIR) {
        // pairs without tokens: the final state is the initial one
        for (int k = 0;; ++k) {
            int s_, h_, st_, sl_, n_;
            if (!pair_of(p, pair_rank(k), s_, h_, st_, sl_, n_)) break;
            if (n_ == 0 && p.hT) {
                const size_t sb = ((size_t)s_ * p.H + h_) * DK * DV;
                for (int e = t; e < DK * DV; e += 64 * IWAVES) p.hT[sb + e] = p.h0 ? p.h0[sb + e] : 0.f;
            }
        }
        i = -1;  // pair mode: i counts the workgroup's rounds
        have = pair_next(p, i, lc, sq, h, pst, slen, nch, tok0, len);
    } else {
        have = PRO ? next_item_seq(p, i, c, h, tok0, len, sq, lc, slen) : next_item(p, i, c, h, tok0, len);
    }
    R raw;
    PI pro;
    if (have) load_raw(raw, p, tok0, len, h, w, l);
    if constexpr (PRO) {
        if (have) {
            load_hist(pro, p, tok0, len, sq, lc, h, tb, l);
            load_taps(pro, p, h, l);
        }
    }
    __builtin_amdgcn_s_waitcnt(0);
    // The layer prologue of one item in registers (PRO): its convolution state and
    // checkpoint rows from the pre-activations, then ShortConv, Swish and L2Norm
    // into raw.q / raw.k / raw.v.  It runs for the first item before the loop and
    // for each next item in the current item's P3, once the next item's loads
    // have been waited for, where its VALU work fills the substitution's MFMA
    // latency.
    auto prologue_regs = [&](int len, int sq, int lc, int slen, int h) {
            constexpr int C = 2 * DK + DV;
            const int W = p.f.conv_w;
            // Convolution state: the pre-activations of chunk positions q0 .. q0 + W - 2,
            // written by the wave whose rows hold them (row e holds position tb - 3 + e).
            auto put_rows = [&](T *dst, int q0) {
#pragma unroll
                for (int e = 0; e < 3 + HT; ++e) {
                    const int j = tb - 3 + e - q0;  // its state row
                    if (j < 0 || j >= W - 1 || (e < 3 && tb - 3 + e >= 0)) continue;  // not kept, or another wave's token
                    *reinterpret_cast<ku *>(dst + (size_t)j * C + CPT * l) = e < 3 ? pro.hq[e] : raw.q[e - 3];
                    *reinterpret_cast<ku *>(dst + (size_t)j * C + DK + CPT * l) = e < 3 ? pro.hk[e] : raw.k[e - 3];
                    *reinterpret_cast<vu *>(dst + (size_t)j * C + 2 * DK + CPV * l) = e < 3 ? pro.hv[e] : raw.v[e - 3];
                }
            };
            if (W > 1 && p.f.conv_state_out && lc * CHUNK + len == slen)
                put_rows((T *)p.f.conv_state_out + ((size_t)sq * p.H + h) * (W - 1) * C, len - (W - 1));
            if (W > 1 && p.f.conv_ckpt && p.ckpt_every > 0 && (lc + 1) % p.ckpt_every == 0) {
                const int slot = (lc + 1) / p.ckpt_every - 1;
                if (slot < p.ckpt_slots && (lc + 1) * CHUNK < slen)
                    put_rows((T *)p.f.conv_ckpt + (((size_t)sq * p.ckpt_slots + slot) * p.H + h) * (W - 1) * C,
                             CHUNK - (W - 1));
            }
            // ShortConv (taps zero-padded to width 4), Swish, and for q and k L2Norm
            // over the head's channels (this wave holds all of them for its tokens).
            // Tokens run last to first, so each token's own row is replaced by its
            // result only after the later tokens that read it as history.
            auto swish = [](float u) { return u * __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-LOG2E * u)); };
#pragma unroll
            for (int r = HT - 1; r >= 0; --r) {
                float aq[CPT], ak[CPT], sq2_ = 0.f, sk2_ = 0.f;
#pragma unroll
                for (int cc = 0; cc < CPT; ++cc) {
                    float cq = 0.f, ck = 0.f;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int row = r + e;  // 0..2: history, 3..: tokens
                        cq += pro.wq[cc][e] * to_f<T>((row < 3 ? pro.hq[row] : raw.q[row - 3])[cc]);
                        ck += pro.wk[cc][e] * to_f<T>((row < 3 ? pro.hk[row] : raw.k[row - 3])[cc]);
                    }
                    aq[cc] = swish(cq);
                    ak[cc] = swish(ck);
                    sq2_ += aq[cc] * aq[cc];
                    sk2_ += ak[cc] * ak[cc];
                }
                float av[CPV];
#pragma unroll
                for (int cv = 0; cv < CPV; ++cv) {
                    float cx = 0.f;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int row = r + e;
                        cx += pro.wv[cv][e] * to_f<T>((row < 3 ? pro.hv[row] : raw.v[row - 3])[cv]);
                    }
                    av[cv] = swish(cx);
                }
                const bool ok = tb + r < len;  // padded tokens carry q = k = v = 0
                const float nq = rsq_norm(wave_sum(sq2_) + p.f.qk_eps);
                const float nk = rsq_norm(wave_sum(sk2_) + p.f.qk_eps);
#pragma unroll
                for (int cc = 0; cc < CPT; ++cc) {
                    raw.q[r][cc] = from_f<T>(ok ? aq[cc] * nq : 0.f);
                    raw.k[r][cc] = from_f<T>(ok ? ak[cc] * nk : 0.f);
                }
#pragma unroll
                for (int cv = 0; cv < CPV; ++cv) raw.v[r][cv] = from_f<T>(ok ? av[cv] : 0.f);
            }
    };
    if constexpr (PRO) {
        if (have) prologue_regs(len, sq, lc, slen, h);
    }

    while (have) {
        char *blkb = p.blocks + ((size_t)h * p.n_chunks_cap + c) * BL::BYTES;
        T *blk = reinterpret_cast<T *>(blkb);
        // where this chunk's block goes: the workspace, or (pair mode) LDS
        T *bW, *bQ, *bA, *bU;
        float *bG;
        if constexpr (PAIR) {
            bW = reinterpret_cast<T *>(&sm.L[0][0]);
            bQ = &sm.ops.KR[0][0];
            bU = &sm.ops.QR[0][0];
            bA = reinterpret_cast<T *>(reinterpret_cast<char *>(&sm.y.t.Tp[0][0]) + sizeof(sm.y.t.Tp));
            bG = sm.gam;
            static_assert(!PAIR || (sizeof(sm.L) >= 16 * 1024 && sizeof(sm.ops.KR) >= 16 * 1024 &&
                                    sizeof(sm.ops.QR) >= 16 * 1024 &&
                                    offsetof(SM, y.t.Tp) + sizeof(sm.y.t.Tp) + 8 * 1024 <= offsetof(SM, y) + sizeof(sm.y)),
                          "pair mode: LDS regions for the block");
            if (lc == 0 && w < NCW) {  // the pair's entering state (waited for in P3)
                const size_t sb = ((size_t)sq * p.H + h) * DK * DV;
#pragma unroll
                for (int R = 0; R < NR; ++R)
#pragma unroll
                    for (int cc = 0; cc < CT; ++cc)
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            S[R][cc][e] = p.h0 ? p.h0[sb + (size_t)(16 * R + 4 * g + e) * DV + 16 * (CT * w + cc) + x] : 0.f;
            }
        } else {
            bW = blk + BL::W_OFF;
            bQ = blk + BL::Q_OFF;
            bU = blk + BL::U_OFF;
            bA = blk + BL::A_OFF;
            bG = reinterpret_cast<float *>(blkb + BL::GAMMA_BYTE);
        }

        // ---- P1: gate (eq. 5), in-tile cumsum, elementwise operands ----------
        // The raw registers were loaded during the previous item (or before the
        // loop) and have been waited for in that item's P3 (see there), so no
        // wait here holds back on the previous item's result stores.
        // The next item's raw inputs are loaded into each raw register right after
        // its last use below, so the loads issue between this item's VALU work.
        int i2 = i + gridDim.x, c2 = 0, h2 = 0, tok2 = 0, len2 = 0, sq2 = 0, lc2 = 0, slen2 = 0, pst2 = 0, nch2 = 0;
        bool have2;
        if constexpr (PAIR) {
            i2 = i; lc2 = lc; sq2 = sq; h2 = h; pst2 = pst; slen2 = slen; nch2 = nch;
            have2 = pair_next(p, i2, lc2, sq2, h2, pst2, slen2, nch2, tok2, len2);
        } else {
            have2 = PRO ? next_item_seq(p, i2, c2, h2, tok2, len2, sq2, lc2, slen2) : next_item(p, i2, c2, h2, tok2, len2);
        }
        // The next item's rows of this wave through buffer descriptors: base at its
        // first token (uniform), lane offset plus token offset in one VGPR shared by
        // g, k and q, and a record count that ends at the last valid token, so tokens
        // past the chunk read as zero without a mask.
        const int nvalid = have2 ? min(max(len2 - tb, 0), HT) : 0;
        const size_t row0 = ((size_t)(tok2 + tb) * p.H + h2);
        const int rowk = p.H * DK * (int)sizeof(T), rowv = p.H * DV * (int)sizeof(T);
        const int reck = nvalid ? (nvalid - 1) * rowk + DK * (int)sizeof(T) : 0;
        const int recv = nvalid ? (nvalid - 1) * rowv + DV * (int)sizeof(T) : 0;
        const __amdgpu_buffer_rsrc_t rsg = __builtin_amdgcn_make_buffer_rsrc((void *)((const T *)p.g + row0 * DK), 0, reck, 0x00020000);
        const __amdgpu_buffer_rsrc_t rsk = __builtin_amdgcn_make_buffer_rsrc((void *)((const T *)p.k + row0 * DK), 0, reck, 0x00020000);
        const __amdgpu_buffer_rsrc_t rsq = __builtin_amdgcn_make_buffer_rsrc((void *)((const T *)p.q + row0 * DK), 0, reck, 0x00020000);
        const __amdgpu_buffer_rsrc_t rsv = __builtin_amdgcn_make_buffer_rsrc((void *)((const T *)p.v + row0 * DV), 0, recv, 0x00020000);
        const int offk = ch0 * (int)sizeof(T), offv = CPV * l * (int)sizeof(T);
        float lam2[HT][CPT];  // (lam_r - B_m) log2(e) for this wave's tokens (tile m = m0)
        {
            const float cz = -__expf(raw.alog) * LOG2E;  // exp(-e^A z) = exp2(cz z)
            const float gm2 = p.g_min * LOG2E;
            float run[CPT];
#pragma unroll
            for (int cc = 0; cc < CPT; ++cc) run[cc] = 0.f;
#pragma unroll
            for (int r = 0; r < HT; ++r) {
#pragma unroll
                for (int cc = 0; cc < CPT; ++cc) {
                    const float z = to_f<T>(raw.g[r][cc]);
                    float g2 = ZM ? gm2 * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(cz * z))
                                       : clamp_logdecay(z, p.g_min) * LOG2E;
                    g2 = (tb + r < len) ? g2 : 0.f;  // tokens past the end keep S unchanged
                    run[cc] += g2;
                    lam2[r][cc] = run[cc];
                }
            }
#pragma unroll
            for (int cc = 0; cc < CPT; ++cc) sm.tot[2 * m0 + hf][ch0 + cc] = run[cc];
            if constexpr (PRO) {  // Sigmoid of the logit; padded tokens keep beta = 0
                if (l < HT) sm.beta[tb + l] = (tb + l < len) ? __builtin_amdgcn_rcpf(1.f + __expf(-to_f<T>(raw.beta))) : 0.f;
            } else {
                if (l < HT) sm.beta[tb + l] = to_f<T>(raw.beta);
            }
        }
        if constexpr (PRO) {
            // the next item's history rows and (for another head) taps, after their
            // last use (the next item's prologue ran in the previous item's P3)
            if (have2) {
                load_hist(pro, p, tok2, len2, sq2, lc2, h2, tb, l);
                if (h2 != h) load_taps(pro, p, h2, l);
            }
        }
        {
            const int bt = tb + l;
            raw.beta = (have2 && l < HT && bt < len2) ? ((const T *)p.beta)[(size_t)(tok2 + bt) * p.H + h2] : from_f<T>(0.f);
            raw.alog = (have2 && ZM) ? p.A_log[h2] : 0.f;
        }
        lds_barrier();
        {
            float eBm[CPT], eCB[CPT], eT[CPT], eX1[CPT], eX2[CPT], gC[CPT];
            // a lane's CPT channels of each half-tile total in one read (single
            // 4-byte reads at an 8-byte lane stride would meet in the LDS banks)
            typedef typename Vec<float, CPT>::type fc;
            fc sgv[8];
#pragma unroll
            for (int q2 = 0; q2 < 8; ++q2) sgv[q2] = *reinterpret_cast<const fc *>(&sm.tot[q2][ch0]);
            const fc hofv = *reinterpret_cast<const fc *>(&sm.tot[2 * m0][ch0]);
#pragma unroll
            for (int cc = 0; cc < CPT; ++cc) {
                float sg[8];
#pragma unroll
                for (int q2 = 0; q2 < 8; ++q2) sg[q2] = sgv[q2][cc];
                const float t0 = sg[0] + sg[1], t1 = sg[2] + sg[3], t2 = sg[4] + sg[5], t3 = sg[6] + sg[7];
                const float Bm = (m0 > 0 ? t0 : 0.f) + (m0 > 1 ? t1 : 0.f) + (m0 > 2 ? t2 : 0.f);
                const float C2 = t0 + t1 + t2 + t3;
                // first half of the tile, for the second half (read from LDS: a
                // register array indexed by the wave's tile would go to scratch)
                const float hoff = hf ? hofv[cc] : 0.f;
#pragma unroll
                for (int r = 0; r < HT; ++r) lam2[r][cc] += hoff;
                eBm[cc] = __builtin_amdgcn_exp2f(Bm);              // exp(B_m)            <= 1
                eCB[cc] = __builtin_amdgcn_exp2f(C2 - Bm);         // exp(lam_C - B_m)    <= 1
                const float Tw = (m0 == 0) ? t0 : (m0 == 1 ? t1 : (m0 == 2 ? t2 : t3));
                eT[cc] = __builtin_amdgcn_exp2f(Tw);               // exp(T_m): reference moved to the tile end
                eX1[cc] = __builtin_amdgcn_exp2f(m0 == 0 ? t1 : t2);  // tile 0 -> B_2, tile 1 -> B_3
                eX2[cc] = __builtin_amdgcn_exp2f(t1 + t2);            // tile 0 -> B_3
                gC[cc] = __builtin_amdgcn_exp2f(C2);
            }
            if (hf == 0) {
#pragma unroll
                for (int cc = 0; cc < CPT; ++cc) sm.eB[m0][ch0 + cc] = eBm[cc];
            }
            tok8 kpv[CPT], ktv[CPT];
#pragma unroll
            for (int r0 = 0; r0 < HT; ++r0) {
                const int r = HT * hf + r0, tok = tb + r0;  // r: token within the tile
                ku kr_, qr_, kc_;
                float kce[CPT];
#pragma unroll
                for (int cc = 0; cc < CPT; ++cc) {
                    const float kv = to_f<T>(raw.k[r0][cc]);
                    const float qv = p.scale * to_f<T>(raw.q[r0][cc]);
                    const float eR = __builtin_amdgcn_exp2f(lam2[r0][cc]);        // exp(lam_r - B_w) <= 1
                    const float eC = __builtin_amdgcn_rcpf(eR);  // exp(B_w - lam_r) <= e^80
                    const float kr = kv * eR, qr = qv * eR, kcs = kv * eC;
                    kce[cc] = kcs * eT[cc];
                    kr_[cc] = from_f<T>(kr);
                    qr_[cc] = from_f<T>(qr);
                    kc_[cc] = from_f<T>(kcs);
                    kpv[cc][r0] = from_f<T>(kr * eBm[cc]);
                    ktv[cc][r0] = from_f<T>(kcs * eCB[cc]);
                }
                const int cp = kpos(ch0);  // CPT <= 2 channels stay adjacent
                *reinterpret_cast<ku *>(&sm.ops.KR[tok][cp]) = kr_;
                *reinterpret_cast<ku *>(&sm.ops.QR[tok][cp]) = qr_;
                *reinterpret_cast<ku *>(&sm.y.KC[tok][cp]) = kc_;
                // the off-diagonal column operands, formed only by the tiles that have
                // them (wave-uniform branches)
                auto put_col = [&](int row, const float *fac) {
                    ku v_;
#pragma unroll
                    for (int cc = 0; cc < CPT; ++cc) v_[cc] = from_f<T>(fac ? kce[cc] * fac[cc] : kce[cc]);
                    *reinterpret_cast<ku *>(&sm.y.KC[row][cp]) = v_;
                };
                if (m0 < 3) put_col(64 + tok, nullptr);
                if (m0 == 0) {
                    put_col(112 + r, eX1);
                    put_col(128 + r, eX2);
                }
                if (m0 == 1) put_col(144 + r, eX1);
                raw.g[r0] = buf_load<ku>(rsg, offk + r0 * rowk);
                raw.k[r0] = buf_load<ku>(rsk, offk + r0 * rowk);
                raw.q[r0] = buf_load<ku>(rsq, offk + r0 * rowk);
            }
#pragma unroll
            for (int cc = 0; cc < CPT; ++cc) {
                const int ch = ch0 + cc;
                *reinterpret_cast<tok8 *>(&sm.KpT[ch][tb ^ (8 * swz_kv(ch))]) = kpv[cc];
                *reinterpret_cast<tok8 *>(&sm.KtT[ch][tb]) = ktv[cc];
            }
            if (w == 0) {  // gamma^C, stored after the last use of the raw registers
#pragma unroll
                for (int cc = 0; cc < CPT; ++cc) bG[ch0 + cc] = gC[cc];
            }
#pragma unroll
            for (int cv = 0; cv < CPV; ++cv) {
                tok8 col;
#pragma unroll
                for (int r = 0; r < HT; ++r) col[r] = raw.v[r][cv];
                *reinterpret_cast<tok8 *>(&sm.VT[CPV * l + cv][tb ^ (8 * swz_kv(CPV * l + cv))]) = col;
            }
#pragma unroll
            for (int r = 0; r < HT; ++r) raw.v[r] = buf_load<typename R::vu>(rsv, offv + r * rowv);
        }
        lds_barrier();

        // Q+ = scale Q Gamma as the chain's operand fragments (rows tokens, k
        // channels in kmap order), from the row operand and exp(B_m); fragment f
        // is token tile f / KS, k-step f % KS.
        auto qp_frag = [&](int f) {
            const int m = f / KS, ks = f % KS;
            const frag_t<T> qr = load_frag_lin<T>(&sm.ops.QR[16 * m + x][32 * ks], g);
            const f32x4 e0 = *reinterpret_cast<const f32x4 *>(&sm.eB[m][32 * ks + 4 * g]);
            const f32x4 e1 = *reinterpret_cast<const f32x4 *>(&sm.eB[m][32 * ks + 16 + 4 * g]);
            frag_t<T> qp;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                qp[e] = from_f<T>(to_f<T>(qr[e]) * e0[e]);
                qp[4 + e] = from_f<T>(to_f<T>(qr[4 + e]) * e1[e]);
            }
            store8(bQ + ((m * KS + ks) * 64 + l) * 8, qp);
        };

        // ---- P2: L and A sub-tiles on MFMA; diagonal inverses ----------------
        // Ten (m, n) tile pairs, each an L product (rows r of tile m, columns i
        // of tile n) and an A^T product.  Waves 0-3 take the diagonal pair
        // (m, m) = (w, w) and invert their block at once (below); waves 4-7
        // take the six off-diagonal pairs: one whole each, and (3,1), (3,2)
        // split by product (waves 4, 5 the L products, waves 6, 7 the A^T
        // products), then the first half of Q+.  All fragments of a pair are
        // read from LDS before its first product is issued.
        //
        // T' = (I + L)^-1 Diag(beta) by 16x16 blocks: the diagonal blocks
        // D_m = (I + N)^-1, N = L_mm strictly lower (N^16 = 0), as the finite
        // product (I - N)(I + N^2)(I + N^4)(I + N^8) on fp32 MFMA (a product X Y
        // takes Y in accumulator layout and X in row layout, which is X^T in
        // accumulator layout, so each factor is also kept transposed); then in
        // P3 wave n < 3 walks block column n downwards,
        //   T_mn = -D_m sum_{q=n}^{m-1} L_mq T_qn,   T_nn = D_n,
        // keeping T_qn in fp32 MFMA accumulators: with k = 4g + i at step i a
        // lane's accumulator element i is exactly its B operand, so no block
        // goes back through LDS.  Every block is written once, scaled by beta of
        // its column and rounded, into the MFMA operand array Tp.
        float(*L)[SM::LP] = sm.L;
        constexpr int LP = SM::LP;
        f32x4 dmv = {0.f, 0.f, 0.f, 0.f};  // waves 0-3: D_w in accumulator layout, D[4g+i][x]
        f32x4 apend0 = {0.f, 0.f, 0.f, 0.f}, apend1 = {0.f, 0.f, 0.f, 0.f};  // pair mode: A tiles for P3
        {
            auto pair_products = [&](int m, int n, bool doL, bool doA, f32x4 &aL, f32x4 &aA) {
                const int cr = colop_row(m, n);
                frag_t<T> kc[KS], kr[KS], qr[KS];
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) kc[ks] = load_frag_lin<T>(&sm.y.KC[cr + x][32 * ks], g);
                if (doL) {
#pragma unroll
                    for (int ks = 0; ks < KS; ++ks) kr[ks] = load_frag_lin<T>(&sm.ops.KR[16 * m + x][32 * ks], g);
                }
                if (doA) {
#pragma unroll
                    for (int ks = 0; ks < KS; ++ks) qr[ks] = load_frag_lin<T>(&sm.ops.QR[16 * m + x][32 * ks], g);
                }
                aL = f32x4{0.f, 0.f, 0.f, 0.f};
                aA = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    if (doL) aL = mma(kr[ks], kc[ks], aL);  // rows r (tile m), cols i (tile n)
                    if (doA) aA = mma(kc[ks], qr[ks], aA);  // rows i (tile n), cols r (tile m): A^T
                }
            };
            // beta of the row, strictly lower part only (all of an off-diagonal block)
            auto l_block = [&](int m, int n, const f32x4 &aL) {
                const f32x4 bt = *reinterpret_cast<const f32x4 *>(&sm.beta[16 * m + 4 * g]);
                f32x4 v;
#pragma unroll
                for (int ii = 0; ii < 4; ++ii) v[ii] = (m != n || x < 4 * g + ii) ? bt[ii] * aL[ii] : 0.f;
                return v;
            };
            // A tiles go to the workspace at once; in pair mode their LDS region is
            // still being read here, so they wait in registers for P3 (slot 0: the
            // wave's first pair, slot 1: the A half of (3,1) or (3,2)).
            auto store_a = [&](int m, int n, const f32x4 &aA, int slot) {
                f32x4 a4;
#pragma unroll
                for (int ii = 0; ii < 4; ++ii) a4[ii] = (m != n || 4 * g + ii <= x) ? aA[ii] : 0.f;
                if constexpr (PAIR) {
                    (slot == 0 ? apend0 : apend1) = a4;
                } else {
                    *reinterpret_cast<quad_t<T> *>(bA + ((m * 2 + n / 2) * 64 + l) * 8 + 4 * (n % 2)) = make_quad<T>(a4);
                }
            };
            f32x4 aL, aA;
            if (w < 4) {
                const int m = w, o0 = 16 * w;
                pair_products(m, m, true, true, aL, aA);
                store_a(m, m, aA, 0);
                const f32x4 na = l_block(m, m, aL);  // N in accumulator layout (lane (x,g): N[4g+i][x])
#pragma unroll
                for (int i = 0; i < 4; ++i) L[o0 + 4 * g + i][(o0 + x) ^ swz_l(4 * g + i)] = na[i];
                // N in row layout (lane (x,g): N[x][4g+i]), read back transposed by this wave
                const f32x4 nr = *reinterpret_cast<const f32x4 *>(&L[o0 + x][(o0 + 4 * g) ^ swz_l(x)]);
                auto mm = [](const f32x4 &a, const f32x4 &b) {
                    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int i = 0; i < 4; ++i) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[i], b[i], acc, 0, 0, 0);
                    return acc;
                };
                f32x4 a1r, a1a;  // A1 = I - N
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    a1r[i] = (x == 4 * g + i ? 1.f : 0.f) - nr[i];
                    a1a[i] = (x == 4 * g + i ? 1.f : 0.f) - na[i];
                }
                const f32x4 n2 = mm(nr, na), n2t = mm(na, nr);
                const f32x4 a2 = a1a + mm(a1r, n2), a2t = a1r + mm(n2, a1r);
                const f32x4 n4 = mm(n2t, n2), n4t = mm(n2, n2t);
                const f32x4 a3 = a2 + mm(a2t, n4), a3t = a2t + mm(n4, a2t);
                const f32x4 n8 = mm(n4t, n4);
                dmv = a3 + mm(a3t, n8);
                float *Dm = dblk(sm, w);
#pragma unroll
                for (int i = 0; i < 4; ++i) Dm[(4 * g + i) * LP + (x ^ swz_l(4 * g + i))] = dmv[i];
            } else {
                const int j = w - 4;
                {  // (1,0), (2,0), (2,1), (3,0)
                    const int m = j == 0 ? 1 : (j == 3 ? 3 : 2), n = j == 2 ? 1 : 0;
                    pair_products(m, n, true, true, aL, aA);
                    const f32x4 v = l_block(m, n, aL);
#pragma unroll
                    for (int ii = 0; ii < 4; ++ii) L[16 * m + 4 * g + ii][(16 * n + x) ^ swz_l(4 * g + ii)] = v[ii];
                    store_a(m, n, aA, 0);
                }
                {
                    const int m = 3, n = 1 + (j & 1);
                    const bool doL = j < 2;
                    pair_products(m, n, doL, !doL, aL, aA);
                    if (doL) {
                        const f32x4 v = l_block(m, n, aL);
#pragma unroll
                        for (int ii = 0; ii < 4; ++ii) L[16 * m + 4 * g + ii][(16 * n + x) ^ swz_l(4 * g + ii)] = v[ii];
                    } else {
                        store_a(m, n, aA, 1);
                    }
                }
                if (!PAIR && j < 2) {  // the all-zero upper A tiles inside used k-steps: (0,1) and (2,3)
                    const int m = 2 * j, n = m + 1;
                    const f32x4 z = {0.f, 0.f, 0.f, 0.f};
                    *reinterpret_cast<quad_t<T> *>(bA + ((m * 2 + n / 2) * 64 + l) * 8 + 4 * (n % 2)) = make_quad<T>(z);
                }
                if constexpr (!PAIR) {  // first half of Q+ (pair mode: all of it in P3, KR is still being read)
                    for (int f = j; f < 2 * KS; f += IWAVES - 4) qp_frag(f);
                }
            }
        }
        lds_barrier();  // L and D complete; KR / KC fully read (Tp may overwrite the off-diagonal column operands)

        // ---- P3: off-diagonal blocks of T'; K~^T and the rest of Q+ ----------
        {
            // The next item's raw inputs were loaded during P1, two phases ago; wait
            // for them here, where the only younger memory operations are this
            // item's early result stores.  Loads and stores share one counter, so
            // a wait at the top of the next item would also wait for every P3/P4
            // store.
            __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0), other counters untouched
            if constexpr (PAIR) {  // the A tiles held since P2, and the two zero tiles
                auto put_a = [&](int m, int n, const f32x4 &a4) {
                    *reinterpret_cast<quad_t<T> *>(bA + ((m * 2 + n / 2) * 64 + l) * 8 + 4 * (n % 2)) = make_quad<T>(a4);
                };
                if (w < 4) {
                    put_a(w, w, apend0);
                } else {
                    const int j = w - 4;
                    put_a(j == 0 ? 1 : (j == 3 ? 3 : 2), j == 2 ? 1 : 0, apend0);
                    if (j >= 2) put_a(3, 1 + (j & 1), apend1);
                    if (j < 2) put_a(2 * j, 2 * j + 1, f32x4{0.f, 0.f, 0.f, 0.f});
                }
            }
            if (w < 4) {  // diagonal block of Tp
                const float bc = sm.beta[16 * w + x];
#pragma unroll
                for (int i = 0; i < 4; ++i) sm.y.t.Tp[16 * w + 4 * g + i][(16 * w + x) ^ (8 * swz_tp(4 * g + i))] = from_f<T>(dmv[i] * bc);
            }
            if (w < 3) {
                const int n = w;
                const float bc = sm.beta[16 * n + x];
                f32x4 Tr[4];  // Tr[d] = T_{n+d, n}: rows 4g + i, column x
                Tr[0] = dmv;
#pragma unroll
                for (int d = 1; d < 4; ++d) {
                    if (n + d > 3) break;
                    const int m = n + d;
                    // the step's L blocks and D_m, read together before its products (the
                    // previous step's stores to Tp keep the compiler from reading earlier)
                    f32x4 La[3];
#pragma unroll
                    for (int qd = 0; qd < d; ++qd)
                        La[qd] = *reinterpret_cast<const f32x4 *>(&L[16 * m + x][(16 * (n + qd) + 4 * g) ^ swz_l(x)]);
                    f32x4 dm = *reinterpret_cast<const f32x4 *>(dblk(sm, m) + x * LP + ((4 * g) ^ swz_l(x)));
                    // (held in place: the compiler would otherwise sink each read to its
                    // product and wait for it there)
#pragma unroll
                    for (int qd = 0; qd < d; ++qd) asm volatile("" : "+v"(La[qd]));
                    asm volatile("" : "+v"(dm));
                    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int qd = 0; qd < d; ++qd) {
#pragma unroll
                        for (int i = 0; i < 4; ++i) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(La[qd][i], Tr[qd][i], acc, 0, 0, 0);
                    }
                    f32x4 tm = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int i = 0; i < 4; ++i) tm = __builtin_amdgcn_mfma_f32_16x16x4f32(dm[i], acc[i], tm, 0, 0, 0);
                    Tr[d] = -tm;
#pragma unroll
                    for (int i = 0; i < 4; ++i) sm.y.t.Tp[16 * m + 4 * g + i][(16 * n + x) ^ (8 * swz_tp(4 * g + i))] = from_f<T>(Tr[d][i] * bc);
                }
            } else {
                // Of the zero upper blocks of Tp, P4 reads only (0,1) and (2,3)
                // (inside its 32-wide k-steps of row tiles 0 and 2).
                if (w == 4 || w == 5) {
                    const int mb = (w == 4) ? 0 : 2, r = l >> 2, cq = 4 * (l & 3);
                    tok4 z;
#pragma unroll
                    for (int e = 0; e < 4; ++e) z[e] = from_f<T>(0.f);
                    *reinterpret_cast<tok4 *>(&sm.y.t.Tp[16 * mb + r][(16 * (mb + 1) + cq) ^ (8 * swz_tp(r))]) = z;
                }
                if constexpr (PAIR) {  // K~^T stays in KtT; all of Q+ here
                    for (int f = w - 3; f < 4 * KS; f += IWAVES - 3) qp_frag(f);
                } else {
                    // (K gamma^C / Gamma)^T as the chain's A-operand fragments (rows
                    // channels, k tokens in kmap order), copied from LDS.
                    for (int f = w - 3; f < 2 * (DK / 16); f += IWAVES - 3) {
                        const int R = f / 2, ks = f % 2;
                        store8(blk + BL::KT_OFF + (f * 64 + l) * 8, load_frag_kmap<T>(&sm.KtT[16 * R + x][32 * ks], g));
                    }
                    for (int f = 2 * KS + w - 3; f < 4 * KS; f += IWAVES - 3) qp_frag(f);  // second half of Q+
                }
            }
            if constexpr (PRO) {
                if (have2) prologue_regs(len2, sq2, lc2, slen2, h2);
            }
        }
        lds_barrier();

        // ---- P4: U = T' V and W^T = K+^T T'^T on MFMA -------------------------
        // The Tp fragments (row tile m, k-step ks <= m / 2) are the A operands of
        // U and the B operands of W^T: read once per wave.
        if (w < (DV > DK ? DV : DK) / 16) {
            frag_t<T> tpf[4][2];
#pragma unroll
            for (int m = 0; m < 4; ++m)
#pragma unroll
                for (int ks = 0; ks <= m / 2; ++ks) tpf[m][ks] = load8(&sm.y.t.Tp[16 * m + x][32 * ks + 8 * (g ^ swz_tp(x))]);
            for (int ct = w; ct < DV / 16; ct += IWAVES) {
                frag_t<T> vt[2];
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) vt[ks] = load8(&sm.VT[16 * ct + x][8 * ((4 * ks + g) ^ swz_kv(16 * ct + x))]);
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int ks = 0; ks <= m / 2; ++ks) acc = mma(tpf[m][ks], vt[ks], acc);
                    *reinterpret_cast<quad_t<T> *>(bU + ((ct * 4 + m) * 64 + l) * 4) = make_quad<T>(acc);
                }
            }
            for (int ct = w; ct < DK / 16; ct += IWAVES) {
                frag_t<T> kp[2];
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) kp[ks] = load8(&sm.KpT[16 * ct + x][8 * ((4 * ks + g) ^ swz_kv(16 * ct + x))]);
#pragma unroll
                for (int tt = 0; tt < 4; ++tt) {
                    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int ks = 0; ks <= tt / 2; ++ks) acc = mma(kp[ks], tpf[tt][ks], acc);
                    *reinterpret_cast<quad_t<T> *>(bW + ((tt * KS + ct / 2) * 64 + l) * 8 + 4 * (ct % 2)) = make_quad<T>(-acc);
                }
            }
        }
        lds_barrier();  // LDS is reused by the next item (pair mode: the block is complete)

        // ---- pair mode: the chain step of this chunk, a column tile per wave --
        // As in chain_wide_kernel, from the LDS block: V~ = U - W S, O^T = S^T (Q+)^T
        // + V~^T A^T, S <- Diag(gamma^C) S + K~^T V~; o and checkpoints out; the
        // final state after the pair's last chunk.  The next chunk's P1b writes
        // these regions only after its first barrier, which every wave reaches
        // after its share of this step.
        if constexpr (PAIR) {
            if (w < NCW) {
                constexpr int FB = (int)sizeof(frag_t<T>), QB = (int)sizeof(quad_t<T>), EL = (int)sizeof(T);
                const int ct0 = CT * w;
                auto frag = [&](const T *base, int piece) {
                    return *reinterpret_cast<const frag_t<T> *>(reinterpret_cast<const char *>(base) + piece * 64 * FB + l * FB);
                };
                static_assert(CT == 1 && KS == 4, "pair mode chain step: one column tile, d_k = 128");
                frag_t<T> Sf[KS];
#pragma unroll
                for (int ks = 0; ks < KS; ++ks)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        Sf[ks][e] = from_f<T>(S[2 * ks][0][e]);
                        Sf[ks][4 + e] = from_f<T>(S[2 * ks + 1][0][e]);
                    }
                f32x4 V[4], O[4];
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    V[m] = quad_to_f<T>(*reinterpret_cast<const quad_t<T> *>(
                        reinterpret_cast<const char *>(bU) + ((ct0 * 4 + m) * 64 + l) * QB));
                    O[m] = f32x4{0.f, 0.f, 0.f, 0.f};
                }
                frag_t<T> Vf[2];
                // The step's 54 products, in order: V~ = U - W S (W pieces 0-15, piece
                // m KS + ks), O^T = S^T (Q+)^T (Q+ pieces 0-15), S <- Diag(gamma^C) S +
                // K~^T V~ (K~^T row tile q / 2, k-step q % 2, from KtT), O^T += V~^T A^T
                // (A pieces 0, 2, 4, 5, 6, 7: A is lower triangular, so token tiles 0 and 1
                // have one k-step).  Operands are read from LDS four at a time, one group
                // ahead of the products, so that LDS latency overlaps MFMA work.
                constexpr int NP = 54, GP = 4;
                auto fetch = [&](int i) -> frag_t<T> {
                    if (i < 16) return frag(bW, i);
                    if (i < 32) return frag(bQ, i - 16);
                    if (i < 48) return load_frag_kmap<T>(&sm.KtT[16 * ((i - 32) / 2) + x][32 * ((i - 32) % 2)], g);
                    const int j = i - 48;
                    return frag(bA, j < 2 ? 2 * j : j + 2);
                };
                auto apply = [&](int i, const frag_t<T> &f) {
                    if (i < 16) {
                        V[i / KS] = mma(f, Sf[i % KS], V[i / KS]);
                    } else if (i < 32) {
                        O[(i - 16) / KS] = mma(Sf[(i - 16) % KS], f, O[(i - 16) / KS]);
                    } else if (i < 48) {
                        S[(i - 32) / 2][0] = mma(f, Vf[(i - 32) % 2], S[(i - 32) / 2][0]);
                    } else {
                        const int j = i - 48, m = j < 2 ? j : 2 + (j - 2) / 2;
                        O[m] = mma(Vf[j < 2 ? 0 : (j - 2) % 2], f, O[m]);
                    }
                };
                frag_t<T> cur[GP], nxt[GP];
#pragma unroll
                for (int q = 0; q < GP; ++q) cur[q] = fetch(q);
#pragma unroll
                for (int i0 = 0; i0 < NP; i0 += GP) {
#pragma unroll
                    for (int q = 0; q < GP; ++q)
                        if (i0 + GP + q < NP) nxt[q] = fetch(i0 + GP + q);
                    // Diag(gamma^C) S, one row tile per group while the fragments above
                    // (which hold S) feed the first products
                    if (i0 < 4 * NR) S[i0 / 4][0] *= *reinterpret_cast<const f32x4 *>(&bG[16 * (i0 / 4) + 4 * g]);
                    if (i0 == 32)  // V~ complete: its B fragments
#pragma unroll
                        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
                            for (int e = 0; e < 4; ++e) {
                                Vf[ks][e] = from_f<T>(V[2 * ks][e]);
                                Vf[ks][4 + e] = from_f<T>(V[2 * ks + 1][e]);
                            }
#pragma unroll
                    for (int q = 0; q < GP; ++q)
                        if (i0 + q < NP) apply(i0 + q, cur[q]);
#pragma unroll
                    for (int q = 0; q < GP; ++q) cur[q] = nxt[q];
                }
                // o through a descriptor whose record count ends at the chunk's last token
                const int rowb = p.H * DV * EL;
                const __amdgpu_buffer_rsrc_t ro = __builtin_amdgcn_make_buffer_rsrc(
                    (void *)((T *)p.o + ((size_t)tok0 * p.H + h) * DV), 0, (len - 1) * rowb + DV * EL, 0x00020000);
#pragma unroll
                for (int m = 0; m < 4; ++m)
                    buf_store<quad_t<T>>(ro, (16 * m + x) * rowb + (16 * ct0 + 4 * g) * EL, make_quad<T>(O[m]));
                const size_t sb = ((size_t)sq * p.H + h) * DK * DV;
                // prefix-state checkpoint after every ckpt_every-th chunk strictly inside the sequence
                if (p.ckpt_every > 0 && (lc + 1) % p.ckpt_every == 0) {
                    const int jk = (lc + 1) / p.ckpt_every - 1;
                    if (jk < p.ckpt_slots && (lc + 1) * CHUNK < slen) {
                        float *cp = p.ckpt + (((size_t)sq * p.ckpt_slots + jk) * p.H + h) * DK * DV;
#pragma unroll
                        for (int R = 0; R < NR; ++R)
#pragma unroll
                            for (int cc = 0; cc < CT; ++cc)
#pragma unroll
                                for (int e = 0; e < 4; ++e)
                                    cp[(size_t)(16 * R + 4 * g + e) * DV + 16 * (ct0 + cc) + x] = S[R][cc][e];
                    }
                }
                if (lc == nch - 1 && p.hT) {
#pragma unroll
                    for (int R = 0; R < NR; ++R)
#pragma unroll
                        for (int cc = 0; cc < CT; ++cc)
#pragma unroll
                            for (int e = 0; e < 4; ++e)
                                p.hT[sb + (size_t)(16 * R + 4 * g + e) * DV + 16 * (ct0 + cc) + x] = S[R][cc][e];
                }
            }
        }
        i = i2; c = c2; h = h2; tok0 = tok2; len = len2;
        sq = sq2; lc = lc2; slen = slen2;
        pst = pst2; nch = nch2;
        have = have2;
    }
}

// -----------------------------------------------------------------------------
// Chain stage: one workgroup per (sequence, head, 16-column slice of d_v);
// columns of S evolve independently (V~ = U - W S acts column by column).
// Workgroup ids are dispatched round-robin over the 8 XCDs (id % 8), so the NS
// slices of one (sequence, head) are given ids congruent mod 8: they share an
// XCD and read the chunk blocks through one L2.
//
// Eight waves in two roles over the same four token tiles (wave w, tile
// w % 4): waves 0-3 carry the recurrence (S in fp32 registers, rows
// 16*RT*w .. 16*RT*(w+1)-1; V~ = U - W S and S <- gamma^C S + K~^T V~), waves
// 4-7 form the output (O^T = S^T (Q+)^T + V~^T A^T) from the S^T and V~^T
// that the recurrence waves exchange through LDS.  Each role loads only its
// own operands, straight into registers, one chunk ahead, spread between its
// MFMA groups: a wave whose vector load is not accepted stalls in order, and
// the two roles sharing a SIMD keep it busy while the other waits.
// -----------------------------------------------------------------------------
template <typename T, int DK> struct ChainRec {   // recurrence operands of one chunk
    static constexpr int KS = DK / 32, RT = DK / 64;
    frag_t<T> Wn[KS], Kt[RT][2];
    quad_t<T> U;
    f32x4 gam[RT];
};
template <typename T, int DK> struct ChainOut {   // output operands of one chunk
    static constexpr int KS = DK / 32;
    frag_t<T> Qp[KS], Af[2];
};

// Fragment with every bit ANDed with m (m = 0 or ~0): a branch-free zeroing.
template <typename T> __device__ __forceinline__ frag_t<T> mask_frag(frag_t<T> f, uint32_t m)
{
    typedef uint32_t u32v __attribute__((ext_vector_type(sizeof(frag_t<T>) / 4)));
    u32v u = __builtin_bit_cast(u32v, f);
    u &= m;
    return __builtin_bit_cast(frag_t<T>, u);
}

// Loads of one chunk's operands for tile wv.  `b` is the block (uniform);
// each access is scalar base + lane offset + immediate.
template <typename V> __device__ __forceinline__ V ldg(const char *b, size_t off, uint32_t lane_off)
{
    return *reinterpret_cast<const V *>(b + off + lane_off);
}

template <typename T, int DK, int DV> struct ChainLoad {
    using BL = Block<T, DK, DV>;
    static constexpr int KS = DK / 32, RT = DK / 64;
    static constexpr size_t FB = sizeof(frag_t<T>), QB = sizeof(quad_t<T>);
    __device__ static __forceinline__ void uw(ChainRec<T, DK> &f, const char *b, int wv, int l, int sl) {
        f.U = ldg<quad_t<T>>(b, BL::U_OFF * sizeof(T) + (size_t)(sl * 4 + wv) * 64 * QB, (uint32_t)l * QB);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            f.Wn[ks] = ldg<frag_t<T>>(b, BL::W_OFF * sizeof(T) + (size_t)(wv * KS + ks) * 64 * FB, (uint32_t)l * FB);
    }
    __device__ static __forceinline__ void kt(ChainRec<T, DK> &f, const char *b, int wv, int l, int g) {
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
#pragma unroll
            for (int ks = 0; ks < 2; ++ks)
                f.Kt[rt][ks] = ldg<frag_t<T>>(b, BL::KT_OFF * sizeof(T) + (size_t)((wv * RT + rt) * 2 + ks) * 64 * FB,
                                              (uint32_t)l * FB);
            f.gam[rt] = ldg<f32x4>(b, BL::GAMMA_BYTE + (size_t)(wv * RT + rt) * 64, (uint32_t)g * 16u);
        }
    }
    __device__ static __forceinline__ void q(ChainOut<T, DK> &f, const char *b, int wv, int l) {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            f.Qp[ks] = ldg<frag_t<T>>(b, BL::Q_OFF * sizeof(T) + (size_t)(wv * KS + ks) * 64 * FB, (uint32_t)l * FB);
    }
    __device__ static __forceinline__ void a(ChainOut<T, DK> &f, const char *b, int wv, int l) {
        // Tiles 0, 1 have no second k-step of A (all zero, not stored): they load
        // the first one again and the step masks it to zero.
        f.Af[0] = ldg<frag_t<T>>(b, BL::A_OFF * sizeof(T) + (size_t)(wv * 2) * 64 * FB, (uint32_t)l * FB);
        f.Af[1] = ldg<frag_t<T>>(b, BL::A_OFF * sizeof(T) + (size_t)(wv * 2 + (wv >= 2)) * 64 * FB, (uint32_t)l * FB);
    }
};

// Runs step(cur, lc, next, lc + 1) over lc = 0 .. nch-1 with two alternating
// operand buffers.  The first one or two chunks are peeled so that the loop
// body holds exactly two steps with no branch between them (which keeps the
// compiler's load waits one chunk deep).
template <typename F, typename Step>
__device__ __forceinline__ void run_chunks(int nch, F &fa, F &fb, Step &&step)
{
    if (nch <= 0) return;
    step(fa, 0, fb, 1);
    if (nch & 1) {
        for (int lc = 1; lc < nch; lc += 2) {
            step(fb, lc, fa, lc + 1);
            step(fa, lc + 1, fb, lc + 2);
        }
    } else {
        step(fb, 1, fa, 2);
        for (int lc = 2; lc < nch; lc += 2) {
            step(fa, lc, fb, lc + 1);
            step(fb, lc + 1, fa, lc + 2);
        }
    }
}

template <typename T, int DK, int DV>
__global__ __launch_bounds__(512) void chain_kernel(PrefillParams p)
{
    using BL = Block<T, DK, DV>;
    using LD = ChainLoad<T, DK, DV>;
    constexpr int KS = DK / 32, RT = DK / 64, NS = DV / 16;
    // S^T and V~^T slices, [column][k], with k stored in kmap order inside each
    // block of 32 (position 8g + e holds k = kmap(g, e)), so an operand fragment
    // is one contiguous 16-byte read and an accumulator quad one 8-byte write.
    // Unpadded rows; 8-element block b of row x sits at b ^ (x & 7), which keeps
    // the fragment reads free of LDS bank conflicts (the quad writes, 16 lanes
    // at one 8-byte offset of a 16-byte block, cannot avoid a two-way conflict).
    __shared__ __align__(16) T sST[16][DK];
    __shared__ __align__(16) T sVT[16][CHUNK];

    const int npairs = p.N * p.H;
    const int bid = blockIdx.x, xcd = bid & 7, jj = bid >> 3;
    const int sl = jj % NS, pair = (jj / NS) * 8 + xcd;
    if (pair >= npairs) return;
    const int srank = pair / p.H, h = pair - srank * p.H;
    int s, tok0, len, chunk0, nch;
    if (p.varlen) {
        s = p.order[srank];
        tok0 = p.span[2 * s];
        len = p.span[2 * s + 1];
        chunk0 = p.chunk_off[s];
        nch = p.chunk_off[s + 1] - chunk0;
    } else {
        s = srank;
        tok0 = s * p.T;
        len = p.T;
        nch = (p.T + CHUNK - 1) / CHUNK;
        chunk0 = s * nch;
    }
    const int t = threadIdx.x, wr = __builtin_amdgcn_readfirstlane(t >> 6), w = wr & 3;
    const int l = t & 63, g = l >> 4, x = l & 15;
    const int col = 16 * sl + x, xsw = 8 * (x & 7);  // the row's block swizzle, in elements
    const size_t sbase = ((size_t)s * p.H + h) * DK * DV;
    const char *blk0 = p.blocks + ((size_t)h * p.n_chunks_cap + chunk0) * BL::BYTES;
    auto blk = [&](int lc) { return blk0 + (size_t)min(lc, nch - 1) * BL::BYTES; };  // last block again at the end

    if (wr < 4) {
        // ---- recurrence waves ------------------------------------------------
        // state slice in accumulator layout: rows 16*(w*RT+rt) + 4g + i, column col
        f32x4 S[RT];
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = 16 * (w * RT + rt) + 4 * g + i;
                S[rt][i] = p.h0 ? p.h0[sbase + (size_t)row * DV + col] : 0.f;
            }
            *reinterpret_cast<quad_t<T> *>(&sST[x][kpos(16 * (w * RT + rt) + 4 * g) ^ xsw]) = make_quad<T>(S[rt]);
        }
        auto step = [&](const ChainRec<T, DK> &f, int lc, ChainRec<T, DK> &nx, int nlc) {
            const char *nb = blk(nlc);
            lds_barrier();  // S^T of this chunk's entering state is in LDS
            frag_t<T> Sk[KS];
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) Sk[ks] = load8(&sST[x][(32 * ks + 8 * g) ^ xsw]);
            f32x4 accV = quad_to_f<T>(f.U);
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) accV = mma(f.Wn[ks], Sk[ks], accV);  // V~ = U - W S
            __builtin_amdgcn_sched_barrier(0);
            LD::uw(nx, nb, w, l, sl);
            __builtin_amdgcn_sched_barrier(0);
            *reinterpret_cast<quad_t<T> *>(&sVT[x][kpos(16 * w + 4 * g) ^ xsw]) = make_quad<T>(accV);
            lds_barrier();  // V~ of the whole chunk is in LDS; S^T fully read
            frag_t<T> Vf[2];
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) Vf[ks] = load8(&sVT[x][(32 * ks + 8 * g) ^ xsw]);
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
                S[rt] *= f.gam[rt];                       // Diag(gamma^C) S
                S[rt] = mma(f.Kt[rt][0], Vf[0], S[rt]);   // + (K gamma^C / Gamma)^T V~
                S[rt] = mma(f.Kt[rt][1], Vf[1], S[rt]);
            }
            __builtin_amdgcn_sched_barrier(0);
            LD::kt(nx, nb, w, l, g);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
                *reinterpret_cast<quad_t<T> *>(&sST[x][kpos(16 * (w * RT + rt) + 4 * g) ^ xsw]) = make_quad<T>(S[rt]);
            // Prefix-state checkpoint after every ckpt_every-th chunk strictly inside the sequence.
            if (p.ckpt_every > 0 && (lc + 1) % p.ckpt_every == 0) {
                const int j = (lc + 1) / p.ckpt_every - 1;
                if (j < p.ckpt_slots && (lc + 1) * CHUNK < len) {
                    float *cp = p.ckpt + (((size_t)s * p.ckpt_slots + j) * p.H + h) * DK * DV;
#pragma unroll
                    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                        for (int i = 0; i < 4; ++i) cp[(size_t)(16 * (w * RT + rt) + 4 * g + i) * DV + col] = S[rt][i];
                }
            }
        };
        ChainRec<T, DK> fa, fb;
        if (nch > 0) {
            LD::uw(fa, blk0, w, l, sl);
            LD::kt(fa, blk0, w, l, g);
        }
        run_chunks(nch, fa, fb, step);
        if (p.hT) {
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int row = 16 * (w * RT + rt) + 4 * g + i;
                    p.hT[sbase + (size_t)row * DV + col] = S[rt][i];
                }
        }
    } else {
        // ---- output waves ------------------------------------------------------
        const uint32_t amask = (w >= 2) ? ~0u : 0u;
        T *o = (T *)p.o;
        auto step = [&](const ChainOut<T, DK> &f, int lc, ChainOut<T, DK> &nx, int nlc) {
            const char *nb = blk(nlc);
            lds_barrier();  // S^T of this chunk's entering state is in LDS
            frag_t<T> Sk[KS];
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) Sk[ks] = load8(&sST[x][(32 * ks + 8 * g) ^ xsw]);
            // The output is formed transposed, O^T = S^T (Gamma Q)^T + V~^T A^T: the same
            // fragments with the operand roles swapped, so each lane ends with four
            // consecutive columns of one token (one 8-byte store).
            f32x4 accO = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) accO = mma(Sk[ks], f.Qp[ks], accO);
            __builtin_amdgcn_sched_barrier(0);
            LD::q(nx, nb, w, l);
            __builtin_amdgcn_sched_barrier(0);
            lds_barrier();  // V~ of the whole chunk is in LDS
            frag_t<T> Vf[2];
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) Vf[ks] = load8(&sVT[x][(32 * ks + 8 * g) ^ xsw]);
            accO = mma(Vf[0], f.Af[0], accO);             // + (A V~)^T
            accO = mma(Vf[1], mask_frag<T>(f.Af[1], amask), accO);
            __builtin_amdgcn_sched_barrier(0);
            LD::a(nx, nb, w, l);
            __builtin_amdgcn_sched_barrier(0);
            const int clen = min(CHUNK, len - lc * CHUNK), r = 16 * w + x;
            if (r < clen)
                *reinterpret_cast<quad_t<T> *>(o + ((size_t)(tok0 + lc * CHUNK + r) * p.H + h) * DV + 16 * sl + 4 * g) =
                    make_quad<T>(accO);
        };
        ChainOut<T, DK> fa, fb;
        if (nch > 0) {
            LD::q(fa, blk0, w, l);
            LD::a(fa, blk0, w, l);
        }
        run_chunks(nch, fa, fb, step);
    }
}

// -----------------------------------------------------------------------------
// Wide chain: one workgroup of four waves per (sequence, head), for inputs with
// many (sequence, head) pairs, where throughput, not the length of one chain,
// sets the time.  Wave w owns CT = d_v / 64 column tiles (16 columns each) of S
// with all d_k rows, as fp32 MFMA accumulators: lane (x, g) of tile (R, c)
// holds S[16R + 4g + i][col(c) + x].  With the shared k-map those registers,
// rounded to T, are exactly the operand fragments of the products that
// contract over d_k (B of W S, A of S^T (Q+)^T), and the accumulators of
// V~ = U - W S are exactly those of the products that contract over tokens
// (B of K~^T V~, A of V~^T A^T): the recurrence runs inside each wave, with no
// exchange.  The chunk's whole block (operands every wave reads, then U) is
// copied into LDS by direct global->LDS loads, one chunk ahead into the other
// of two buffers (two LDS arrays, so the compiler can tell a copy in flight
// into one from the reads of the other); each wave issues its share of the
// copies in four parts spread over the chunk's products, so that no wave
// stalls on a burst of memory requests.  Per (chunk, head) one compute unit
// does the work that the slice chain spreads over eight, at about three times
// the time per chunk: the slice chain is for long chains with few pairs.
// -----------------------------------------------------------------------------
template <typename T, int DK, int DV> struct WideShape {
    using BL = Block<T, DK, DV>;
    static constexpr int NLD = (int)((BL::STAGE_BYTES + 1023) / 1024);  // pieces of the shared operands
    // U goes through LDS with the operands when both buffers fit (every bf16
    // shape); otherwise (fp32) the waves read it from the block.
    static constexpr bool ULDS = 2 * BL::BYTES <= 160 * 1024;
    static constexpr int NPC = ULDS ? (int)(BL::BYTES / 1024) : NLD;   // pieces copied per chunk
};

template <typename T, int DK, int DV>
__global__ __launch_bounds__(256) void chain_wide_kernel(PrefillParams p)
{
    using BL = Block<T, DK, DV>;
    using WS = WideShape<T, DK, DV>;
    constexpr int KS = DK / 32, NR = DK / 16, CT = DV / 64;
    constexpr int FB = (int)sizeof(frag_t<T>), QB = (int)sizeof(quad_t<T>), EL = (int)sizeof(T);
    constexpr int NPC = WS::NPC;
    constexpr bool ULDS = WS::ULDS;
    constexpr int PER = (NPC + 3) / 4, PART = (PER + 3) / 4;  // pieces per wave, per part
    __shared__ __align__(16) char sA[NPC * 1024];
    __shared__ __align__(16) char sB[NPC * 1024];

    const int pair = blockIdx.x;
    if (pair >= p.N * p.H) return;
    const int srank = pair / p.H, h = pair - srank * p.H;
    int s, tok0, len, chunk0, nch;
    if (p.varlen) {
        s = p.order[srank];
        tok0 = p.span[2 * s];
        len = p.span[2 * s + 1];
        chunk0 = p.chunk_off[s];
        nch = p.chunk_off[s + 1] - chunk0;
    } else {
        s = srank;
        tok0 = s * p.T;
        len = p.T;
        nch = (p.T + CHUNK - 1) / CHUNK;
        chunk0 = s * nch;
    }
    const int t = threadIdx.x, w = __builtin_amdgcn_readfirstlane(t >> 6);
    const int l = t & 63, g = l >> 4, x = l & 15;
    const int ct0 = w * CT;  // first column tile of this wave
    const size_t sbase = ((size_t)s * p.H + h) * DK * DV;
    const char *blk0 = p.blocks + ((size_t)h * p.n_chunks_cap + chunk0) * BL::BYTES;

    f32x4 S[NR][CT];
#pragma unroll
    for (int R = 0; R < NR; ++R)
#pragma unroll
        for (int c = 0; c < CT; ++c) S[R][c] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (p.h0) {
#pragma unroll
        for (int R = 0; R < NR; ++R)
#pragma unroll
            for (int c = 0; c < CT; ++c)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    S[R][c][i] = p.h0[sbase + (size_t)(16 * R + 4 * g + i) * DV + 16 * (ct0 + c) + x];
    }

    // Part `part` of this wave's copies of chunk lc into buf: pieces w + 4 i for
    // i in [PART part, PART (part + 1)).
    auto stage = [&](char *buf, int lc, int part) {
        const char *b = blk0 + (size_t)lc * BL::BYTES + l * 16;
#pragma unroll
        for (int i = PART * part; i < PART * (part + 1); ++i) {
            const int j = w + 4 * i;
            if (j < NPC)
                __builtin_amdgcn_global_load_lds((const void *)(b + j * 1024),
                                                 (__attribute__((address_space(3))) void *)(buf + j * 1024), 16, 0, 0);
        }
    };
    auto frag = [&](const char *buf, size_t off_elems, int piece) {
        return *reinterpret_cast<const frag_t<T> *>(buf + off_elems * sizeof(T) + (size_t)piece * 64 * FB + l * FB);
    };
    const int rowb = p.H * DV * EL;  // bytes between consecutive tokens of o
    T *o = (T *)p.o;

    auto step = [&](const char *buf, char *nbuf, int lc) {
        const bool more = lc + 1 < nch;
        if (more) stage(nbuf, lc + 1, 0);
        frag_t<T> Sf[KS][CT];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
            for (int c = 0; c < CT; ++c)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    Sf[ks][c][e] = from_f<T>(S[2 * ks][c][e]);
                    Sf[ks][c][4 + e] = from_f<T>(S[2 * ks + 1][c][e]);
                }
        // V~ = U + (-W) S
        f32x4 V[4][CT];
#pragma unroll
        for (int m = 0; m < 4; ++m)
#pragma unroll
            for (int c = 0; c < CT; ++c) {
                const size_t uo = BL::U_BYTE + (size_t)((ct0 + c) * 4 + m) * 64 * QB + l * QB;
                V[m][c] = quad_to_f<T>(*reinterpret_cast<const quad_t<T> *>(ULDS ? buf + uo : blk0 + (size_t)lc * BL::BYTES + uo));
            }
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const frag_t<T> wf = frag(buf, BL::W_OFF, m * KS + ks);
#pragma unroll
                for (int c = 0; c < CT; ++c) V[m][c] = mma(wf, Sf[ks][c], V[m][c]);
            }
        if (more) stage(nbuf, lc + 1, 1);
        // O^T = S^T (Q+)^T + V~^T A^T (rows columns, columns tokens)
        f32x4 O[CT][4];
#pragma unroll
        for (int c = 0; c < CT; ++c)
#pragma unroll
            for (int m = 0; m < 4; ++m) O[c][m] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const frag_t<T> qf = frag(buf, BL::Q_OFF, m * KS + ks);
#pragma unroll
                for (int c = 0; c < CT; ++c) O[c][m] = mma(Sf[ks][c], qf, O[c][m]);
            }
        if (more) stage(nbuf, lc + 1, 2);
        frag_t<T> Vf[2][CT];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
            for (int c = 0; c < CT; ++c)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    Vf[ks][c][e] = from_f<T>(V[2 * ks][c][e]);
                    Vf[ks][c][4 + e] = from_f<T>(V[2 * ks + 1][c][e]);
                }
        // S <- Diag(gamma^C) S + (K gamma^C / Gamma)^T V~
#pragma unroll
        for (int R = 0; R < NR; ++R) {
            const f32x4 gam = *reinterpret_cast<const f32x4 *>(buf + BL::GAMMA_BYTE + (16 * R + 4 * g) * 4);
#pragma unroll
            for (int c = 0; c < CT; ++c) S[R][c] *= gam;
        }
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
            for (int R = 0; R < NR; ++R) {
                const frag_t<T> kf = frag(buf, BL::KT_OFF, R * 2 + ks);
#pragma unroll
                for (int c = 0; c < CT; ++c) S[R][c] = mma(kf, Vf[ks][c], S[R][c]);
            }
        if (more) stage(nbuf, lc + 1, 3);
        // + (A V~)^T; A is lower triangular, so token tiles 0 and 1 have one k-step
#pragma unroll
        for (int m = 0; m < 4; ++m)
#pragma unroll
            for (int ks = 0; ks <= m / 2; ++ks) {
                const frag_t<T> af = frag(buf, BL::A_OFF, m * 2 + ks);
#pragma unroll
                for (int c = 0; c < CT; ++c) O[c][m] = mma(Vf[ks][c], af, O[c][m]);
            }
        // The next chunk's block has landed (this wave's copies; the barrier below
        // covers the others'), then this chunk's outputs go out, so the wait does
        // not include their stores.  o goes through a buffer descriptor whose
        // record count ends at the chunk's last token (no branch per row).
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
        const int clen = min(CHUNK, len - lc * CHUNK);
        const __amdgpu_buffer_rsrc_t ro = __builtin_amdgcn_make_buffer_rsrc(
            (void *)(o + ((size_t)(tok0 + lc * CHUNK) * p.H + h) * DV), 0, (clen - 1) * rowb + DV * EL, 0x00020000);
#pragma unroll
        for (int c = 0; c < CT; ++c)
#pragma unroll
            for (int m = 0; m < 4; ++m)
                buf_store<quad_t<T>>(ro, (16 * m + x) * rowb + (16 * (ct0 + c) + 4 * g) * EL, make_quad<T>(O[c][m]));
        // Prefix-state checkpoint after every ckpt_every-th chunk strictly inside the sequence.
        if (p.ckpt_every > 0 && (lc + 1) % p.ckpt_every == 0) {
            const int j = (lc + 1) / p.ckpt_every - 1;
            if (j < p.ckpt_slots && (lc + 1) * CHUNK < len) {
                float *cp = p.ckpt + (((size_t)s * p.ckpt_slots + j) * p.H + h) * DK * DV;
#pragma unroll
                for (int R = 0; R < NR; ++R)
#pragma unroll
                    for (int c = 0; c < CT; ++c)
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            cp[(size_t)(16 * R + 4 * g + i) * DV + 16 * (ct0 + c) + x] = S[R][c][i];
            }
        }
        __builtin_amdgcn_s_barrier();
    };

    if (nch > 0) {
#pragma unroll
        for (int part = 0; part < 4; ++part) stage(sA, 0, part);
    }
    // Nothing loaded before the chunk loop stays in flight into it (the first
    // chunk's copies included), so no wait merged into the loop reaches back.
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    __builtin_amdgcn_s_barrier();
    for (int lc = 0; lc < nch; lc += 2) {
        step(sA, sB, lc);
        if (lc + 1 < nch) step(sB, sA, lc + 1);
    }
    if (p.hT) {
#pragma unroll
        for (int R = 0; R < NR; ++R)
#pragma unroll
            for (int c = 0; c < CT; ++c)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    p.hT[sbase + (size_t)(16 * R + 4 * g + i) * DV + 16 * (ct0 + c) + x] = S[R][c][i];
    }
}

// -----------------------------------------------------------------------------
// Output epilogue (eq. (6) without W_o), in place on o after the chain:
// o <- Sigmoid(gate) * w_h * o / sqrt(mean(o^2) + eps) per (token, head) row.
// The chain holds 16 of a head's d_v columns per workgroup, so the per-row
// mean square needs this separate, bandwidth-bound pass: each lane moves 16
// bytes of o and of the gate, a row spans DV / VPL lanes and is reduced with
// lane swaps inside that group.
template <typename T, int DV>
__global__ __launch_bounds__(256) void gate_norm_kernel(T *o, const T *gate, const float *wgt, int H, long rows,
                                                        float eps)
{
    constexpr int VPL = 16 / (int)sizeof(T), LPR = DV / VPL, RPW = 64 / LPR;
    typedef typename Vec<T, VPL>::type vec;
    const int l = threadIdx.x & 63, w = threadIdx.x >> 6;
    const long row = ((long)blockIdx.x * 4 + w) * RPW + l / LPR;
    const int c0 = (l % LPR) * VPL;
    const bool ok = row < rows;                    // uniform within a row's lane group
    const size_t off = (size_t)(ok ? row : 0) * DV + c0;
    vec ov = *reinterpret_cast<const vec *>(o + off), gv = *reinterpret_cast<const vec *>(gate + off);
    const int h = (int)((ok ? row : 0) % H);
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < VPL; ++e) ss += to_f<T>(ov[e]) * to_f<T>(ov[e]);
#pragma unroll
    for (int m = 1; m < LPR; m <<= 1) ss += __shfl_xor(ss, m);
    const float r = rsq_norm(ss * (1.f / DV) + eps);
    const float *wr = wgt + (size_t)h * DV + c0;
#pragma unroll
    for (int e = 0; e < VPL; ++e)
        ov[e] = from_f<T>(to_f<T>(ov[e]) * r * wr[e] / (1.f + __expf(-to_f<T>(gv[e]))));
    if (ok) *reinterpret_cast<vec *>(o + off) = ov;
}

// Convolution state of sequences with no tokens: the carried state (or zeros).
template <typename T>
__global__ __launch_bounds__(256) void empty_conv_state_kernel(const PrefillParams p, int C)
{
    const int s = blockIdx.x / p.H, h = blockIdx.x % p.H;
    const int slen = p.varlen ? p.span[2 * s + 1] : p.T;
    if (slen != 0) return;
    const size_t n = (size_t)(p.f.conv_w - 1) * C, base = ((size_t)s * p.H + h) * n;
    for (size_t e = threadIdx.x; e < n; e += blockDim.x)
        ((T *)p.f.conv_state_out)[base + e] = p.f.conv_state ? ((const T *)p.f.conv_state)[base + e] : from_f<T>(0.f);
}

// From MANY_PAIRS (sequence, head) pairs on, the chain runs per pair: in pair
// mode inside the intra-chunk kernel, else on the wide kernel (one compute unit
// per pair, about 2.7 times less work per chunk than the slice kernel's eight,
// each chunk about 3 times slower); below it the slice kernel's shorter time
// per chunk wins.
constexpr long WIDE_CHAIN_PAIRS = MANY_PAIRS;

// -----------------------------------------------------------------------------
// Persistent grid of the intra-chunk stage: one workgroup per compute unit
// (its LDS footprint allows one), queried once from the device.
static long intra_grid()
{
    static const long n = [] {
        int dev = 0, cus = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
            cus = 256;
        return (long)cus;
    }();
    return n;
}

template <typename T, int DK, int DV>
static hipError_t launch_t(const PrefillParams &p, hipStream_t st)
{
    if (p.varlen)
        hipLaunchKernelGGL(chunk_table_kernel, dim3(1), dim3(table::THREADS), 0, st, p.cu, p.N, p.T, p.n_chunks_cap,
                           p.chunk_off, p.order, p.span);
    const bool pro = p.f.conv_w > 0;  // the prologue runs inside the intra-chunk stage
    const long npairs = (long)p.N * p.H;
    // Many pairs (bf16, d_k = 128, no prologue): the chain runs inside the
    // intra-chunk kernel (pair mode), one workgroup per compute unit.
    constexpr bool PAIR_OK = sizeof(T) == 2 && DK == 128;
    if (pair_mode(sizeof(T) == 2, DK, npairs, pro) && p.n_chunks_cap > 0) {
        const size_t smem = sizeof(IntraSmem<T, DK, DV>);
        static const hipError_t attr[2] = {
            hipFuncSetAttribute((const void *)intra_chunk_kernel<T, DK, DV, true, false, PAIR_OK>,
                                hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem),
            hipFuncSetAttribute((const void *)intra_chunk_kernel<T, DK, DV, false, false, PAIR_OK>,
                                hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem)};
        for (hipError_t e : attr)
            if (e != hipSuccess) return e;
        const unsigned grid = (unsigned)(npairs < intra_grid() ? npairs : intra_grid());
        if (p.A_log)
            hipLaunchKernelGGL((intra_chunk_kernel<T, DK, DV, true, false, PAIR_OK>), dim3(grid), dim3(64 * IWAVES), smem, st, p);
        else
            hipLaunchKernelGGL((intra_chunk_kernel<T, DK, DV, false, false, PAIR_OK>), dim3(grid), dim3(64 * IWAVES), smem, st, p);
        const long rows = (long)(p.varlen ? p.T : (long)p.N * p.T) * p.H;
        if (p.f.gate && rows > 0) {
            constexpr int RPB = 4 * (64 / (DV / (16 / (int)sizeof(T))));  // rows per 256-thread workgroup
            hipLaunchKernelGGL((gate_norm_kernel<T, DV>), dim3((unsigned)((rows + RPB - 1) / RPB)), dim3(256), 0, st,
                               (T *)p.o, (const T *)p.f.gate, p.f.o_weight, p.H, rows, p.f.o_eps);
        }
        return hipGetLastError();
    }
    if (p.n_chunks_cap > 0) {
        const size_t smem = sizeof(IntraSmem<T, DK, DV>);
        static_assert(sizeof(IntraSmem<T, DK, DV>) <= 160 * 1024, "intra-chunk LDS exceeds 160 KiB");
        static const hipError_t attr[4] = {
            hipFuncSetAttribute((const void *)intra_chunk_kernel<T, DK, DV, true, false>,
                                hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem),
            hipFuncSetAttribute((const void *)intra_chunk_kernel<T, DK, DV, false, false>,
                                hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem),
            hipFuncSetAttribute((const void *)intra_chunk_kernel<T, DK, DV, true, true>,
                                hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem),
            hipFuncSetAttribute((const void *)intra_chunk_kernel<T, DK, DV, false, true>,
                                hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem)};
        for (hipError_t e : attr)
            if (e != hipSuccess) return e;
        const long items = (long)p.n_chunks_cap * p.H;
        const unsigned grid = (unsigned)(items < intra_grid() ? items : intra_grid());
        const dim3 gd(grid), bd(64 * IWAVES);
        if (p.A_log) {
            if (pro) hipLaunchKernelGGL((intra_chunk_kernel<T, DK, DV, true, true>), gd, bd, smem, st, p);
            else hipLaunchKernelGGL((intra_chunk_kernel<T, DK, DV, true, false>), gd, bd, smem, st, p);
        } else {
            if (pro) hipLaunchKernelGGL((intra_chunk_kernel<T, DK, DV, false, true>), gd, bd, smem, st, p);
            else hipLaunchKernelGGL((intra_chunk_kernel<T, DK, DV, false, false>), gd, bd, smem, st, p);
        }
    }
    if (npairs >= WIDE_CHAIN_PAIRS) {
        hipLaunchKernelGGL((chain_wide_kernel<T, DK, DV>), dim3((unsigned)npairs), dim3(256), 0, st, p);
    } else {
        const unsigned grid = (unsigned)(((npairs + 7) / 8) * 8 * (DV / 16));
        if (grid > 0) hipLaunchKernelGGL((chain_kernel<T, DK, DV>), dim3(grid), dim3(512), 0, st, p);
    }
    const long rows = (long)(p.varlen ? p.T : (long)p.N * p.T) * p.H;
    if (p.f.gate && rows > 0) {
        constexpr int RPB = 4 * (64 / (DV / (16 / (int)sizeof(T))));  // rows per 256-thread workgroup
        hipLaunchKernelGGL((gate_norm_kernel<T, DV>), dim3((unsigned)((rows + RPB - 1) / RPB)), dim3(256), 0, st,
                           (T *)p.o, (const T *)p.f.gate, p.f.o_weight, p.H, rows, p.f.o_eps);
    }
    // sequences without tokens (packed, or T = 0) get the carried convolution state
    if (pro && p.f.conv_state_out && p.f.conv_w > 1 && npairs > 0 && (p.varlen || p.T == 0))
        hipLaunchKernelGGL(empty_conv_state_kernel<T>, dim3((unsigned)npairs), dim3(256), 0, st, p, 2 * DK + DV);
    return hipGetLastError();
}

hipError_t launch_chunk_fwd(int bf16_, int Dk, int Dv, const PrefillParams &p, hipStream_t st)
{
#define KDA_CASE(TT, A, B) \
    if (Dk == A && Dv == B) return launch_t<TT, A, B>(p, st);
    if (bf16_) {
        KDA_CASE(bf16, 64, 64) KDA_CASE(bf16, 64, 128) KDA_CASE(bf16, 128, 64) KDA_CASE(bf16, 128, 128)
    } else {
        KDA_CASE(float, 64, 64)
    }
#undef KDA_CASE
    return hipErrorInvalidValue;
}

}  // namespace kda
