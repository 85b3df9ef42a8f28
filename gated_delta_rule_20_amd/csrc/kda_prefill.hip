// kda_prefill.hip -- chunkwise-parallel KDA forward over whole sequences.
//
// "Kimi K3 Technical Report: Open Frontier Intelligence", §2.1.1:
//   eq. (3)  per-channel cumulative decay inside a chunk, kept in log space:
//            lam_r = sum_{s<=r} g_s, so gamma^r = exp(lam_r);
//   eq. (4)  A = Tril[(Q*Gamma)(K/Gamma)^T] (diagonal kept) and
//            O = (Gamma*Q) S + A V~;
//   "UT transform"  U, W with pseudo-values V~ = U - W S;
//   eq. (5)  lower-bounded gate: a 16-token sub-tile spans a log-decay of at
//            most 15*|g_min| <= 75, so its rescale factors stay inside the
//            bf16/fp32 range ("lower-bounded decay" paragraph and Fig. 3).
// U, W and the hand-off between chunks are not printed on the page; unrolling
// eq. (1) over one chunk entered with state S gives
//   L     = StrictTril(Diag(beta) K+ K-^T),   K+ = K*Gamma, K- = K/Gamma
//   T'    = (I + L)^-1 Diag(beta)
//   U     = T' V,   W = T' K+,   V~ = U - W S
//   S_out = Diag(gamma^C) S + (K * gamma^C / Gamma)^T V~.
// §5.1.1 describes the production kernel as token-parallel stages plus a
// head-parallel recurrence; the same split is used here, laid out for gfx950:
//
//   chunk_table_kernel   (packed sequences only) chunk offsets per sequence
//                        and a longest-first sequence order.
//   intra_chunk_kernel   one workgroup per (chunk, head): gate, cumsum,
//                        sub-tile Gram products on MFMA, blocked triangular
//                        inverse in fp32, U / W / A on MFMA.  It writes every
//                        operand of the chain as a ready-to-issue MFMA
//                        fragment (layout in Block below).
//   chain_kernel         one workgroup per (sequence, head, 16-column slice of
//                        d_v): walks the chunks in order with its slice of S
//                        in fp32 registers; per chunk two dependent MFMA
//                        products (W S, then K~^T V~) sit on the serial path
//                        and the output products (Q+ S, A V~) beside them.
//                        Columns of S evolve independently (V~ = U - W S acts
//                        column by column), which licenses the split.
//
// Sub-tile references.  For rows r in 16-token tile m and columns i in tile
// n <= m, exp(lam_r - lam_i) is factored at b = 16n (first token of tile n):
// exp(lam_r - lam_b) <= 1 times exp(lam_b - lam_i) in [1, e^75].  Row
// operands are stored relative to their own tile start, exp(lam_r - lam_16m),
// and multiplied by the per-channel factor exp(lam_16m - lam_16n) <= 1 for
// off-diagonal tiles, so no factor overflows; a factor that underflows
// belongs to a product below e^-12 times its operands.
#include "kda_common.h"
#include "kda_prefill.h"

namespace kda {

// -----------------------------------------------------------------------------
// Per (head, chunk) workspace block written by intra_chunk_kernel and read by
// chain_kernel.  Element type T except gamma (fp32).  "wave w" is the chain
// kernel's wave index: token rows 16w..16w+15 of the chunk, and state rows
// 16*RT*w .. 16*RT*(w+1)-1.  All fragments use kmap() along k.
//   Wn  [4 waves][KS][64 lanes][8]  A-operand fragments of -W    (rows tokens, k channels)
//   Qp  [4 waves][KS][64][8]        A-operand fragments of scale*Q*Gamma
//   Kt  [4 waves][RT][2][64][8]     A-operand fragments of (K*gamma^C/Gamma)^T (rows channels, k tokens)
//   A   [4 waves][2][64][8]         A-operand fragments of A     (rows tokens, k tokens)
//   U   [NS][4 waves][64][4]        accumulator quads of U
//   gamma [DK] float                gamma^C = exp(lam at the chunk's last token)
// -----------------------------------------------------------------------------
template <typename T, int DK, int DV> struct Block {
    static constexpr int KS = DK / 32;
    static constexpr int RT = DK / 64;
    static constexpr int NS = DV / 16;
    static constexpr size_t W_OFF = 0;
    static constexpr size_t Q_OFF = W_OFF + (size_t)4 * KS * 512;
    static constexpr size_t KT_OFF = Q_OFF + (size_t)4 * KS * 512;
    static constexpr size_t A_OFF = KT_OFF + (size_t)4 * RT * 2 * 512;
    static constexpr size_t U_OFF = A_OFF + (size_t)4 * 2 * 512;
    static constexpr size_t T_ELEMS = U_OFF + (size_t)NS * 4 * 256;
    static constexpr size_t GAMMA_BYTE = T_ELEMS * sizeof(T);
    static constexpr size_t BYTES = (GAMMA_BYTE + DK * sizeof(float) + 255) / 256 * 256;
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
// Packed sequences: chunk_off[s] = sum_{s' < s} ceil(len_s' / 64); order =
// sequences by decreasing length (ties by index) when N <= 2048, else
// identity.  One workgroup of 1024 threads.
// -----------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void chunk_table_kernel(const int32_t *__restrict__ cu, int N,
                                                           int32_t *__restrict__ chunk_off,
                                                           int32_t *__restrict__ order)
{
    __shared__ int part[1024];
    const int t = threadIdx.x;
    const int per = (N + 1023) / 1024;
    const int s0 = min(N, t * per), s1 = min(N, s0 + per);
    int local = 0;
    for (int s = s0; s < s1; ++s) local += (cu[s + 1] - cu[s] + CHUNK - 1) / CHUNK;
    part[t] = local;
    __syncthreads();
    for (int d = 1; d < 1024; d <<= 1) {  // inclusive scan
        const int add = (t >= d) ? part[t - d] : 0;
        __syncthreads();
        part[t] += add;
        __syncthreads();
    }
    int run = part[t] - local;
    for (int s = s0; s < s1; ++s) {
        chunk_off[s] = run;
        run += (cu[s + 1] - cu[s] + CHUNK - 1) / CHUNK;
    }
    if (t == 1023) chunk_off[N] = part[1023];
    for (int s = t; s < N; s += 1024) {
        int rank = s;
        if (N <= 2048) {
            const int ls = cu[s + 1] - cu[s];
            rank = 0;
            for (int y = 0; y < N; ++y) {
                const int ly = cu[y + 1] - cu[y];
                rank += (ly > ls) || (ly == ls && y < s);
            }
        }
        order[rank] = s;
    }
}

// -----------------------------------------------------------------------------
// Intra-chunk stage: 256 threads = 4 waves, one (chunk, head) per workgroup.
// -----------------------------------------------------------------------------
template <typename T, int DK, int DV> struct IntraSmem {
    static constexpr int PR = DK + 8;     // padded row of token-major arrays
    static constexpr int PT = CHUNK + 8;  // padded row of channel-major arrays
    union {
        struct {
            T KR[CHUNK][PR];   // k * exp(lam - lam_16m): row operand of L (tile-start reference)
            T QR[CHUNK][PR];   // scale * q * exp(lam - lam_16m): row operand of A
        } ops;
        struct {
            float Ti[CHUNK][CHUNK + 1];  // (I + L)^-1
            T Tp[CHUNK][PT];             // (I + L)^-1 Diag(beta)
        } inv;
    } x;
    T Kc[CHUNK][PR];    // k * exp(lam_16n - lam): column operand (tile-start reference)
    T Qp[CHUNK][PR];    // scale * q * exp(lam), staged for the fragment copy
    T KpT[DK][PT];      // (k * exp(lam))^T, A operand of W^T
    T KtT[DK][PT];      // (k * exp(lam_C - lam))^T, staged for the fragment copy
    T VT[DV][PT];       // v^T, B operand of U
    float L[CHUNK][CHUNK + 1];  // strictly lower part used; upper blocks serve as scratch
    float F[6][DK];     // exp(lam_16m - lam_16n) for n < m, index m(m-1)/2 + n
    float E[4][DK];     // lam at the first token of each 16-token tile
    float beta[CHUNK];
};

// (m, n) sub-tile pairs (n <= m) handled by wave w in step s, as the index
// m(m+1)/2 + n; -1 = none.  Balances the 10 pairs over 4 waves as 3/3/2/2.
__device__ __forceinline__ int pair_of(int w, int s)
{
    switch (w * 3 + s) {
    case 0: return 0; case 1: return 2; case 2: return 5;
    case 3: return 9; case 4: return 1; case 5: return 4;
    case 6: return 8; case 7: return 3;
    case 9: return 7; case 10: return 6;
    default: return -1;
    }
}

template <typename T, int DK, int DV>
__global__ __launch_bounds__(256) void intra_chunk_kernel(PrefillParams p)
{
    using BL = Block<T, DK, DV>;
    using SM = IntraSmem<T, DK, DV>;
    constexpr int KS = DK / 32, RT = DK / 64;
    extern __shared__ __align__(16) char smem_raw[];
    SM &sm = *reinterpret_cast<SM *>(smem_raw);

    const int c = blockIdx.x, h = blockIdx.y;
    const int t = threadIdx.x, w = t >> 6, l = t & 63, g = l >> 4, x = l & 15;

    // ---- locate the chunk ----------------------------------------------------
    int tok0, len;
    if (p.varlen) {
        if (c >= p.chunk_off[p.N]) return;
        int lo = 0, hi = p.N - 1;  // largest s with chunk_off[s] <= c
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (p.chunk_off[mid] <= c) lo = mid; else hi = mid - 1;
        }
        tok0 = p.cu[lo] + (c - p.chunk_off[lo]) * CHUNK;
        len = min(CHUNK, p.cu[lo + 1] - tok0);
    } else {
        const int cps = (p.T + CHUNK - 1) / CHUNK;
        const int s = c / cps, lc = c - s * cps;
        tok0 = s * p.T + lc * CHUNK;
        len = min(CHUNK, p.T - lc * CHUNK);
    }
    char *blkb = p.blocks + ((size_t)h * p.n_chunks_cap + c) * BL::BYTES;
    T *blk = reinterpret_cast<T *>(blkb);
    float *gamma_out = reinterpret_cast<float *>(blkb + BL::GAMMA_BYTE);
    const T *qg = (const T *)p.q, *kg = (const T *)p.k, *vg = (const T *)p.v, *gg = (const T *)p.g;
    const T *bg = (const T *)p.beta;

    // ---- P1: gate, chunk-local cumsum, elementwise operands ------------------
    // Thread = 8 consecutive channels x TPP consecutive tokens (16-byte loads).
    constexpr int CG8 = DK / 8, NPT = 256 / CG8, TPP = CHUNK / NPT;
    const int cg = t % CG8, pp = t / CG8, j0 = cg * 8, r0 = pp * TPP, m0 = r0 / SUB;
    float lam[TPP][8];
    float lamC[8];
    {
        const float eA = p.A_log ? __expf(p.A_log[h]) : 0.f;
        float run[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
        for (int a = 0; a < TPP; ++a) {
            const int r = r0 + a;
            float gv[8] = {0, 0, 0, 0, 0, 0, 0, 0};  // tokens past the end: g = 0
            if (r < len) {
                const frag_t<T> raw = load8(gg + ((size_t)(tok0 + r) * p.H + h) * DK + j0);
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float z = to_f<T>(raw[e]);
                    gv[e] = p.A_log ? gate_from_logit(z, eA, p.g_min) : clamp_logdecay(z, p.g_min);
                }
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) { run[e] += gv[e]; lam[a][e] = run[e]; }
        }
        float *tot = &sm.L[0][0];  // [NPT][DK] part totals (L is free until P2)
#pragma unroll
        for (int e = 0; e < 8; ++e) tot[pp * DK + j0 + e] = run[e];
        __syncthreads();
        float carry[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
        for (int e = 0; e < 8; ++e) lamC[e] = 0.f;
        for (int q2 = 0; q2 < NPT; ++q2) {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float v2 = tot[q2 * DK + j0 + e];
                if (q2 < pp) carry[e] += v2;
                lamC[e] += v2;
            }
        }
#pragma unroll
        for (int a = 0; a < TPP; ++a)
#pragma unroll
            for (int e = 0; e < 8; ++e) lam[a][e] += carry[e];
        if (r0 % SUB == 0) {
#pragma unroll
            for (int e = 0; e < 8; ++e) sm.E[m0][j0 + e] = lam[0][e];
        }
        if (pp == 0) {
#pragma unroll
            for (int e = 0; e < 8; ++e) gamma_out[j0 + e] = __expf(lamC[e]);
        }
        if (t < CHUNK) sm.beta[t] = (t < len) ? to_f<T>(bg[(size_t)(tok0 + t) * p.H + h]) : 0.f;
    }
    __syncthreads();
    {
        float Em[8], eEm[8], eCm[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            Em[e] = sm.E[m0][j0 + e];
            eEm[e] = __expf(Em[e]);             // exp(lam_16m)            (<= 1)
            eCm[e] = __expf(lamC[e] - Em[e]);   // exp(lam_C - lam_16m)    (<= 1)
        }
#pragma unroll
        for (int a = 0; a < TPP; ++a) {
            const int r = r0 + a;
            float kv[8] = {0, 0, 0, 0, 0, 0, 0, 0}, qv[8] = {0, 0, 0, 0, 0, 0, 0, 0};
            if (r < len) {
                const size_t off = ((size_t)(tok0 + r) * p.H + h) * DK + j0;
                const frag_t<T> kr = load8(kg + off);
                const frag_t<T> qr = load8(qg + off);
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    kv[e] = to_f<T>(kr[e]);
                    qv[e] = p.scale * to_f<T>(qr[e]);
                }
            }
            float kr_[8], qr_[8], kc_[8], qp_[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float d = lam[a][e] - Em[e];  // lam_r - lam_16m in [-75, 0]
                const float eR = __expf(d);
                const float eC = __expf(-d);
                kr_[e] = kv[e] * eR;
                qr_[e] = qv[e] * eR;
                kc_[e] = kv[e] * eC;
                qp_[e] = qr_[e] * eEm[e];
                sm.KpT[j0 + e][r] = from_f<T>(kr_[e] * eEm[e]);
                sm.KtT[j0 + e][r] = from_f<T>(kc_[e] * eCm[e]);
            }
            store8(&sm.x.ops.KR[r][j0], make_frag<T>(kr_));
            store8(&sm.x.ops.QR[r][j0], make_frag<T>(qr_));
            store8(&sm.Kc[r][j0], make_frag<T>(kc_));
            store8(&sm.Qp[r][j0], make_frag<T>(qp_));
        }
        // per-channel tile-pair factors
        for (int idx = t; idx < 6 * DK; idx += 256) {
            const int pi = idx / DK, j = idx % DK;
            const int m = (pi == 0) ? 1 : (pi < 3 ? 2 : 3);
            const int n = pi - m * (m - 1) / 2;
            sm.F[pi][j] = __expf(sm.E[m][j] - sm.E[n][j]);
        }
        // v^T
        constexpr int VG8 = DV / 8, VNP = 256 / VG8, VTP = CHUNK / VNP;
        const int vc = t % VG8, vp = t / VG8;
#pragma unroll
        for (int a = 0; a < VTP; ++a) {
            const int r = vp * VTP + a;
            frag_t<T> vr;
            if (r < len) {
                vr = load8(vg + ((size_t)(tok0 + r) * p.H + h) * DV + vc * 8);
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) vr[e] = from_f<T>(0.f);
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) sm.VT[vc * 8 + e][r] = vr[e];
        }
    }
    __syncthreads();

    // ---- P2: L and A tiles on MFMA; Q+ and K~^T fragments out ----------------
    {
        // (m, n) pairs, n <= m, balanced over the 4 waves; index m(m+1)/2 + n.
        for (int s = 0; s < 3; ++s) {
            const int pi = pair_of(w, s);
            if (pi < 0) break;
            const int m = (pi == 0) ? 0 : (pi < 3 ? 1 : (pi < 6 ? 2 : 3));
            const int n = pi - m * (m + 1) / 2;
            const float *Fr = (n < m) ? sm.F[m * (m - 1) / 2 + n] : nullptr;
            f32x4 accL = {0.f, 0.f, 0.f, 0.f}, accA = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const int kb = 32 * ks + 8 * g;
                float kr8[8], qr8[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float f = Fr ? Fr[kb + e] : 1.f;
                    kr8[e] = to_f<T>(sm.x.ops.KR[16 * m + x][kb + e]) * f;
                    qr8[e] = to_f<T>(sm.x.ops.QR[16 * m + x][kb + e]) * f;
                }
                const frag_t<T> kc = load_frag_lin<T>(&sm.Kc[16 * n + x][32 * ks], g);
                accL = mma(make_frag<T>(kr8), kc, accL);   // rows r (tile m), cols i (tile n)
                accA = mma(kc, make_frag<T>(qr8), accA);   // rows i (tile n), cols r (tile m): A^T
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = 16 * m + 4 * g + i, col = 16 * n + x;
                sm.L[row][col] = (col < row) ? sm.beta[row] * accL[i] : 0.f;
            }
            f32x4 a4;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = 16 * m + x, col = 16 * n + 4 * g + i;
                a4[i] = (col <= r) ? accA[i] : 0.f;
            }
            *reinterpret_cast<quad_t<T> *>(blk + BL::A_OFF + ((m * 2 + n / 2) * 64 + l) * 8 + 4 * (n % 2)) =
                make_quad<T>(a4);
        }
        if (w >= 2) {  // the two all-zero upper tiles of A inside used k-steps: (0,1) and (2,3)
            const int m = (w == 2) ? 0 : 2, n = m + 1;
            const f32x4 z = {0.f, 0.f, 0.f, 0.f};
            *reinterpret_cast<quad_t<T> *>(blk + BL::A_OFF + ((m * 2 + n / 2) * 64 + l) * 8 + 4 * (n % 2)) =
                make_quad<T>(z);
        }
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            store8(blk + BL::Q_OFF + ((w * KS + ks) * 64 + l) * 8, load_frag_kmap<T>(&sm.Qp[16 * w + x][32 * ks], g));
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int ks = 0; ks < 2; ++ks)
                store8(blk + BL::KT_OFF + (((w * RT + rt) * 2 + ks) * 64 + l) * 8,
                       load_frag_kmap<T>(&sm.KtT[16 * (w * RT + rt) + x][32 * ks], g));
    }
    __syncthreads();

    // ---- P3: T' = (I + L)^-1 Diag(beta), blocked, fp32 ------------------------
    {
        float(*Ti)[CHUNK + 1] = sm.x.inv.Ti;
        if (t < 64) {
            // column cc of the inverse of the unit lower 16x16 diagonal block mb
            const int mb = t >> 4, cc = t & 15, o0 = 16 * mb;
            float xv[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                float acc = (r == cc) ? 1.f : 0.f;
#pragma unroll
                for (int i = 0; i < r; ++i) acc -= sm.L[o0 + r][o0 + i] * xv[i];
                xv[r] = acc;
            }
#pragma unroll
            for (int r = 0; r < 16; ++r) Ti[o0 + r][o0 + cc] = xv[r];
        } else {
            for (int e = t - 64; e < 6 * 256; e += 192) {  // upper off-diagonal blocks are zero
                const int bi = e / 256, a = (e / 16) % 16, b = e % 16;
                const int mb = (bi < 3) ? 0 : (bi < 5 ? 1 : 2);
                const int nb = (bi < 3) ? bi + 1 : (bi < 5 ? bi - 1 : 3);
                Ti[16 * mb + a][16 * nb + b] = 0.f;
            }
        }
        __syncthreads();
        for (int m = 1; m < 4; ++m) {
            // X_n = sum_{p=n}^{m-1} L_mp Ti_pn, parked in the unused upper block (n, m) of L
            for (int e = t; e < m * 256; e += 256) {
                const int n = e / 256, a = (e / 16) % 16, b = e % 16;
                float acc = 0.f;
                for (int pb = n; pb < m; ++pb)
#pragma unroll
                    for (int cc = 0; cc < 16; ++cc)
                        acc += sm.L[16 * m + a][16 * pb + cc] * Ti[16 * pb + cc][16 * n + b];
                sm.L[16 * n + a][16 * m + b] = acc;
            }
            __syncthreads();
            for (int e = t; e < m * 256; e += 256) {
                const int n = e / 256, a = (e / 16) % 16, b = e % 16;
                float acc = 0.f;
#pragma unroll
                for (int cc = 0; cc < 16; ++cc) acc += Ti[16 * m + a][16 * m + cc] * sm.L[16 * n + cc][16 * m + b];
                Ti[16 * m + a][16 * n + b] = -acc;
            }
            __syncthreads();
        }
        for (int e = t; e < CHUNK * CHUNK; e += 256) {
            const int r = e / CHUNK, i = e % CHUNK;
            sm.x.inv.Tp[r][i] = from_f<T>(Ti[r][i] * sm.beta[i]);
        }
    }
    __syncthreads();

    // ---- P4: U = T' V and W^T = K+^T T'^T on MFMA ----------------------------
    for (int ct = w; ct < DV / 16; ct += 4) {
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            for (int ks = 0; ks <= m / 2; ++ks)
                acc = mma(load_frag_lin<T>(&sm.x.inv.Tp[16 * m + x][32 * ks], g),
                          load_frag_lin<T>(&sm.VT[16 * ct + x][32 * ks], g), acc);
            *reinterpret_cast<quad_t<T> *>(blk + BL::U_OFF + ((ct * 4 + m) * 64 + l) * 4) = make_quad<T>(acc);
        }
    }
    for (int ct = w; ct < DK / 16; ct += 4) {
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            for (int ks = 0; ks <= tt / 2; ++ks)
                acc = mma(load_frag_lin<T>(&sm.KpT[16 * ct + x][32 * ks], g),
                          load_frag_lin<T>(&sm.x.inv.Tp[16 * tt + x][32 * ks], g), acc);
            *reinterpret_cast<quad_t<T> *>(blk + BL::W_OFF + ((tt * KS + ct / 2) * 64 + l) * 8 + 4 * (ct % 2)) =
                make_quad<T>(-acc);
        }
    }
}

// -----------------------------------------------------------------------------
// Chain stage: one workgroup (4 waves) per (sequence, head, 16-column slice).
// Workgroup ids are dispatched round-robin over the 8 XCDs (id % 8), so the NS
// slices of one (sequence, head) are given ids congruent mod 8: they share an
// XCD and read the chunk blocks through one L2.
// -----------------------------------------------------------------------------
template <typename T, int DK, int DV>
__global__ __launch_bounds__(256) void chain_kernel(PrefillParams p)
{
    using BL = Block<T, DK, DV>;
    constexpr int KS = DK / 32, RT = DK / 64, NS = DV / 16;
    constexpr int PS = DK + 8, PV = CHUNK + 8;
    __shared__ __align__(16) T sST[16][PS];  // S^T slice: [column][state row]
    __shared__ __align__(16) T sVT[16][PV];  // V~^T slice: [column][token]

    const int npairs = p.N * p.H;
    const int bid = blockIdx.x, xcd = bid & 7, jj = bid >> 3;
    const int sl = jj % NS, pair = (jj / NS) * 8 + xcd;
    if (pair >= npairs) return;
    const int srank = pair / p.H, h = pair - srank * p.H;
    int s, tok0, len, chunk0, nch;
    if (p.varlen) {
        s = p.order[srank];
        tok0 = p.cu[s];
        len = p.cu[s + 1] - tok0;
        chunk0 = p.chunk_off[s];
        nch = p.chunk_off[s + 1] - chunk0;
    } else {
        s = srank;
        tok0 = s * p.T;
        len = p.T;
        nch = (p.T + CHUNK - 1) / CHUNK;
        chunk0 = s * nch;
    }
    const int t = threadIdx.x, w = t >> 6, l = t & 63, g = l >> 4, x = l & 15;
    const int col = 16 * sl + x;

    // state slice in accumulator layout: rows 16*(w*RT+rt) + 4g + i, column col
    f32x4 S[RT];
    const size_t sbase = ((size_t)s * p.H + h) * DK * DV;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = 16 * (w * RT + rt) + 4 * g + i;
            S[rt][i] = p.h0 ? p.h0[sbase + (size_t)row * DV + col] : 0.f;
        }
        *reinterpret_cast<quad_t<T> *>(&sST[x][16 * (w * RT + rt) + 4 * g]) = make_quad<T>(S[rt]);
    }

    T *o = (T *)p.o;
    for (int lc = 0; lc < nch; ++lc) {
        const char *blkb = p.blocks + ((size_t)h * p.n_chunks_cap + chunk0 + lc) * BL::BYTES;
        const T *blk = reinterpret_cast<const T *>(blkb);
        frag_t<T> Wn[KS], Qp[KS], Af[2], Kt[RT][2];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            Wn[ks] = load8(blk + BL::W_OFF + ((w * KS + ks) * 64 + l) * 8);
            Qp[ks] = load8(blk + BL::Q_OFF + ((w * KS + ks) * 64 + l) * 8);
        }
        Af[0] = load8(blk + BL::A_OFF + ((w * 2) * 64 + l) * 8);
        if (w >= 2) Af[1] = load8(blk + BL::A_OFF + ((w * 2 + 1) * 64 + l) * 8);
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int ks = 0; ks < 2; ++ks)
                Kt[rt][ks] = load8(blk + BL::KT_OFF + (((w * RT + rt) * 2 + ks) * 64 + l) * 8);
        const quad_t<T> Uq = *reinterpret_cast<const quad_t<T> *>(blk + BL::U_OFF + ((sl * 4 + w) * 64 + l) * 4);
        f32x4 gam[RT];
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
            gam[rt] = *reinterpret_cast<const f32x4 *>(blkb + BL::GAMMA_BYTE +
                                                       (16 * (w * RT + rt) + 4 * g) * sizeof(float));
        __syncthreads();  // S^T of this chunk's entering state is in LDS
        frag_t<T> Sf[KS];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) Sf[ks] = load_frag_kmap<T>(&sST[x][32 * ks], g);
        f32x4 accV = quad_to_f<T>(Uq), accO = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) accV = mma(Wn[ks], Sf[ks], accV);  // V~ = U - W S
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) accO = mma(Qp[ks], Sf[ks], accO);  // (Gamma Q) S
        *reinterpret_cast<quad_t<T> *>(&sVT[x][16 * w + 4 * g]) = make_quad<T>(accV);
        __syncthreads();  // V~ of the whole chunk is in LDS
        frag_t<T> Vf[2];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) Vf[ks] = load_frag_kmap<T>(&sVT[x][32 * ks], g);
        accO = mma(Af[0], Vf[0], accO);             // + A V~ (causal: k-step 1 only for waves 2, 3)
        if (w >= 2) accO = mma(Af[1], Vf[1], accO);
        const int clen = min(CHUNK, len - lc * CHUNK), ctok = tok0 + lc * CHUNK;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = 16 * w + 4 * g + i;
            if (r < clen) o[((size_t)(ctok + r) * p.H + h) * DV + col] = from_f<T>(accO[i]);
        }
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            S[rt] *= gam[rt];                       // Diag(gamma^C) S
            S[rt] = mma(Kt[rt][0], Vf[0], S[rt]);   // + (K gamma^C / Gamma)^T V~
            S[rt] = mma(Kt[rt][1], Vf[1], S[rt]);
            *reinterpret_cast<quad_t<T> *>(&sST[x][16 * (w * RT + rt) + 4 * g]) = make_quad<T>(S[rt]);
        }
    }
    if (p.hT) {
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = 16 * (w * RT + rt) + 4 * g + i;
                p.hT[sbase + (size_t)row * DV + col] = S[rt][i];
            }
    }
}

// -----------------------------------------------------------------------------
template <typename T, int DK, int DV>
static hipError_t launch_t(const PrefillParams &p, hipStream_t st)
{
    if (p.varlen)
        hipLaunchKernelGGL(chunk_table_kernel, dim3(1), dim3(1024), 0, st, p.cu, p.N, p.chunk_off, p.order);
    if (p.n_chunks_cap > 0) {
        const size_t smem = sizeof(IntraSmem<T, DK, DV>);
        static const hipError_t attr = hipFuncSetAttribute((const void *)intra_chunk_kernel<T, DK, DV>,
                                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
        if (attr != hipSuccess) return attr;
        hipLaunchKernelGGL((intra_chunk_kernel<T, DK, DV>), dim3(p.n_chunks_cap, p.H), dim3(256), smem, st, p);
    }
    const long npairs = (long)p.N * p.H;
    const unsigned grid = (unsigned)(((npairs + 7) / 8) * 8 * (DV / 16));
    if (grid > 0) hipLaunchKernelGGL((chain_kernel<T, DK, DV>), dim3(grid), dim3(256), 0, st, p);
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
