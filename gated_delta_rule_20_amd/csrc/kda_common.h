// kda_common.h -- device-side building blocks shared by the KDA kernels (gfx950).
//
// Matrix-core convention used throughout.  Every contraction is a 16x16 output
// tile reduced over k in steps of 32:
//   * lane l (0..63) of a wave has row/col index  l % 16  and lane group
//     g = l / 16 (0..3);
//   * an operand fragment holds 8 values per lane; value e of lane (x, g) is
//     X[x][kmap(g, e)] for the A operand (x = output row) and X[kmap(g, e)][x]
//     for the B operand (x = output column);
//   * the accumulator (4 floats per lane) holds D[4g + i][l % 16], i = 0..3.
// The hardware contracts A and B over the same (g, e) pairs, so any kmap that
// both operands share is valid.  The kernels use
//     kmap(g, e) = 4g + e          (e < 4)
//                  16 + 4g + e - 4 (e >= 4),
// which is what a pair of adjacent accumulator tiles of a transposed product
// naturally holds; it lets one kernel's accumulators become the next kernel's
// operand fragments without shuffles.
//
// bf16 operands use v_mfma_f32_16x16x32_bf16 (one instruction per k-step);
// fp32 operands use eight v_mfma_f32_16x16x4_f32 (value e in step e).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

typedef __bf16 bf16;
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));

constexpr int CHUNK = 64;     // tokens per chunk
constexpr int SUB = 16;       // sub-tile (and MFMA tile) edge
constexpr int WAVE = 64;

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

__device__ __forceinline__ int kmap(int g, int e) { return (e < 4) ? 4 * g + e : 12 + 4 * g + e; }

// Storage position of index k when a k-axis is kept in kmap order (inverse of
// kmap inside each block of 32): position 8g + e holds k = kmap(g, e).  Four
// consecutive k starting at a multiple of 4 stay contiguous.
__device__ __forceinline__ int kpos(int k)
{
    const int b = k & ~31, kk = k & 31;
    return b + 8 * ((kk & 15) >> 2) + 4 * (kk >> 4) + (kk & 3);
}

// ---- element type traits ---------------------------------------------------
template <typename T> struct Elem;

template <> struct Elem<float> {
    typedef f32x8 frag;   // 8 operand values
    typedef f32x4 quad;   // 4 stored values (accumulator quad)
    __device__ static __forceinline__ float to_f(float x) { return x; }
    __device__ static __forceinline__ float from_f(float x) { return x; }
};

template <> struct Elem<bf16> {
    typedef bf16x8 frag;
    typedef bf16x4 quad;
    __device__ static __forceinline__ float to_f(bf16 x) { return (float)x; }
    __device__ static __forceinline__ bf16 from_f(float x) { return (bf16)x; }
};

template <typename T> using frag_t = typename Elem<T>::frag;
template <typename T> using quad_t = typename Elem<T>::quad;

template <typename T> __device__ __forceinline__ float to_f(T x) { return Elem<T>::to_f(x); }
template <typename T> __device__ __forceinline__ T from_f(float x) { return Elem<T>::from_f(x); }

// acc += A x B over one k-step of 32.
__device__ __forceinline__ f32x4 mma(const bf16x8 &a, const bf16x8 &b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma(const f32x8 &a, const f32x8 &b, f32x4 c) {
#pragma unroll
    for (int e = 0; e < 8; ++e) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[e], b[e], c, 0, 0, 0);
    return c;
}

// Fragment built from 8 floats (rounded to T).
template <typename T> __device__ __forceinline__ frag_t<T> make_frag(const float *x) {
    frag_t<T> f;
#pragma unroll
    for (int e = 0; e < 8; ++e) f[e] = from_f<T>(x[e]);
    return f;
}

template <typename T> __device__ __forceinline__ quad_t<T> make_quad(f32x4 x) {
    quad_t<T> q;
#pragma unroll
    for (int i = 0; i < 4; ++i) q[i] = from_f<T>(x[i]);
    return q;
}

template <typename T> __device__ __forceinline__ f32x4 quad_to_f(const quad_t<T> &q) {
    f32x4 x;
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] = to_f<T>(q[i]);
    return x;
}

// 8 contiguous elements, moved as 16-byte accesses (rows are 16-byte aligned).
__device__ __forceinline__ bf16x8 load8(const bf16 *p) { return *reinterpret_cast<const bf16x8 *>(p); }
__device__ __forceinline__ f32x8 load8(const float *p) {
    const f32x4 a = *reinterpret_cast<const f32x4 *>(p), b = *reinterpret_cast<const f32x4 *>(p + 4);
    f32x8 f;
#pragma unroll
    for (int i = 0; i < 4; ++i) { f[i] = a[i]; f[4 + i] = b[i]; }
    return f;
}
__device__ __forceinline__ void store8(bf16 *p, const bf16x8 &f) { *reinterpret_cast<bf16x8 *>(p) = f; }
__device__ __forceinline__ void store8(float *p, const f32x8 &f) {
    f32x4 a, b;
#pragma unroll
    for (int i = 0; i < 4; ++i) { a[i] = f[i]; b[i] = f[4 + i]; }
    *reinterpret_cast<f32x4 *>(p) = a;
    *reinterpret_cast<f32x4 *>(p + 4) = b;
}

// Fragment whose k-values sit in a row at positions kmap(g, 0..7) relative to
// `row` (two runs of 4 contiguous elements).
template <typename T> __device__ __forceinline__ frag_t<T> load_frag_kmap(const T *row, int g) {
    const quad_t<T> lo = *reinterpret_cast<const quad_t<T> *>(row + 4 * g);
    const quad_t<T> hi = *reinterpret_cast<const quad_t<T> *>(row + 16 + 4 * g);
    frag_t<T> f;
#pragma unroll
    for (int i = 0; i < 4; ++i) { f[i] = lo[i]; f[4 + i] = hi[i]; }
    return f;
}

// Fragment whose k-values are 8 contiguous elements at row + 8g.
template <typename T> __device__ __forceinline__ frag_t<T> load_frag_lin(const T *row, int g) {
    return load8(row + 8 * g);
}

// Workgroup barrier for LDS hand-offs only.  __syncthreads() also waits for
// every outstanding global load and store of the wave (vmcnt(0)), which would
// drain register prefetches and in-flight result stores at each barrier; the
// kernels never pass data between threads through global memory within a
// launch, so waiting for this wave's LDS operations is sufficient.  The
// "memory" clobber keeps the compiler from moving memory accesses across it.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

__device__ __forceinline__ float fast_exp(float x) { return __expf(x); }

// eq. (5) gate in fp32: g = g_min * sigmoid(exp(A_h) * z), with eA = exp(A_h);
// the sigmoid's reciprocal on the hardware reciprocal (about 1 ulp).
__device__ __forceinline__ float gate_from_logit(float z, float eA, float g_min) {
    const float x = eA * z;
    return g_min * __builtin_amdgcn_rcpf(1.0f + __expf(-x));
}

// 1 / sqrt(x) for the L2Norm / RMSNorm denominators (x = sum or mean of squares
// plus a non-negative epsilon) on the hardware reciprocal square root; x is
// raised to the smallest normal float first, so a zero vector with epsilon 0
// gives 0 instead of 0 * inf.
__device__ __forceinline__ float rsq_norm(float x) {
    return __builtin_amdgcn_rsqf(fmaxf(x, 1.17549435e-38f));
}

// The sum over the 64 lanes of a wave, returned uniform, from DPP steps
// (pairs, quads, 8- and 16-lane rows, then row broadcasts into rows 1-3; lane
// 63 ends with the total) instead of LDS permutes.  All 64 lanes must be active.
template <int CTRL, int ROWS> __device__ __forceinline__ float dpp_add(float v)
{
    return v + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, ROWS, 0xF, false));
}
__device__ __forceinline__ float wave_sum(float v)
{
    v = dpp_add<0xB1, 0xF>(v);   // quad_perm [1, 0, 3, 2]
    v = dpp_add<0x4E, 0xF>(v);   // quad_perm [2, 3, 0, 1]
    v = dpp_add<0x141, 0xF>(v);  // row_half_mirror
    v = dpp_add<0x140, 0xF>(v);  // row_mirror: every lane holds its 16-lane row's sum
    v = dpp_add<0x142, 0xA>(v);  // row_bcast:15 into rows 1 and 3
    v = dpp_add<0x143, 0xC>(v);  // row_bcast:31 into rows 2 and 3
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}
__device__ __forceinline__ float clamp_logdecay(float g, float g_min) {
    return fminf(fmaxf(g, g_min), 0.0f);
}

}  // namespace kda
