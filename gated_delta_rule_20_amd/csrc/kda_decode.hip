// kda_decode.hip -- single-token recurrent step, state updated in place.
//
// "Kimi K3 Technical Report: Open Frontier Intelligence", §2.1.1 eq. (1) for
// one token, with the eq. (5) gate; §5.4.2 ("KDA") notes that decode is bound
// by moving the in-place state, so this kernel reads and writes every state
// byte exactly once.
//
// Per (sequence, head), with D := Diag(alpha):
//   p = (D S)^T k,   r = (D S)^T q,   kq = k . q
//   delta = beta (v - p)
//   S <- D S + k delta^T                      (eq. (1), rearranged)
//   o = scale * S_new^T q = scale * (r + delta * kq)
// so one pass over S yields both reductions, and the update is applied while
// the rows are still in registers.
//
// Launch: two 128-thread workgroups per (sequence, head), each owning half of
// the d_v columns (columns evolve independently; small workgroups balance the
// 1 GiB stream better over the compute units).  Thread t owns the 4 columns
// c0 + 4*(t % CG) .. +3 (CG = column groups of the half) and rows
// (t / CG) + RG*i (RG = 128 / CG row groups), so each load instruction of a
// wave covers whole rows of the half (coalesced 16-byte accesses).  The two
// column reductions go through LDS once.  The state is read and written with
// non-temporal hints: it is streamed once per step and never re-read soon.
#include "kda_common.h"

namespace kda {

template <typename T, int DK, int DV>
__global__ __launch_bounds__(128) void recurrent_step_kernel(
    const T *__restrict__ q, const T *__restrict__ k, const T *__restrict__ v,
    const T *__restrict__ gz, const T *__restrict__ beta, const float *__restrict__ A_log,
    float g_min, float scale, int H, float *__restrict__ state, T *__restrict__ o)
{
    constexpr int WC = DV / 2;          // columns handled by this workgroup
    constexpr int CG = WC / 4;          // column groups of 4
    constexpr int RG = 128 / CG;        // row groups
    constexpr int RPT = DK / RG;        // rows per thread
    static_assert(RPT * RG == DK && DK <= 128, "row split; threads 0..DK-1 stage k, q, alpha");

    __shared__ float s_k[DK], s_q[DK], s_a[DK];
    __shared__ float s_red[2][RG][WC];
    __shared__ float s_delta[WC];
    __shared__ float s_kq;

    const int t = threadIdx.x;
    const int cg = t % CG, rg = t / CG;
    const size_t nh = blockIdx.x / 2;             // sequence * H + head
    const int c0 = (blockIdx.x % 2) * WC;         // first column of this half
    const int h = (int)(nh % H);
    float *S = state + nh * (size_t)(DK * DV);

    // Issue the state loads first: they are the whole cost of the kernel.
    f32x4 s[RPT];
#pragma unroll
    for (int i = 0; i < RPT; ++i)
        s[i] = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(S + (size_t)(rg + RG * i) * DV + c0 + 4 * cg));

    if (t < DK) {
        const size_t off = nh * DK + t;
        const float kv = to_f<T>(k[off]);
        const float qv = to_f<T>(q[off]);
        float g = to_f<T>(gz[off]);
        g = A_log ? gate_from_logit(g, __expf(A_log[h]), g_min) : clamp_logdecay(g, g_min);
        s_k[t] = kv;
        s_q[t] = qv;
        s_a[t] = __expf(g);
    }
    if (t < 64) {
        // k . q with one wave: lane t sums channels t, t + 64 (DK <= 128).
        float part = 0.f;
        for (int j = t; j < DK; j += 64) part += to_f<T>(k[nh * DK + j]) * to_f<T>(q[nh * DK + j]);
#pragma unroll
        for (int m = 32; m >= 1; m >>= 1) part += __shfl_xor(part, m);
        if (t == 0) s_kq = part;
    }
    __syncthreads();

    f32x4 p = {0.f, 0.f, 0.f, 0.f}, r = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        const int j = rg + RG * i;
        s[i] *= s_a[j];                 // row j of Diag(alpha) S
        p += s[i] * s_k[j];
        r += s[i] * s_q[j];
    }
    *reinterpret_cast<f32x4 *>(&s_red[0][rg][4 * cg]) = p;
    *reinterpret_cast<f32x4 *>(&s_red[1][rg][4 * cg]) = r;
    __syncthreads();

    if (t < WC) {
        float pc = 0.f, rc = 0.f;
#pragma unroll
        for (int x = 0; x < RG; ++x) { pc += s_red[0][x][t]; rc += s_red[1][x][t]; }
        const float b = to_f<T>(beta[nh]);
        const float d = b * (to_f<T>(v[nh * DV + c0 + t]) - pc);
        s_delta[t] = d;
        o[nh * DV + c0 + t] = from_f<T>(scale * (rc + d * s_kq));
    }
    __syncthreads();

    const f32x4 d4 = *reinterpret_cast<const f32x4 *>(&s_delta[4 * cg]);
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        const int j = rg + RG * i;
        __builtin_nontemporal_store(s[i] + s_k[j] * d4, reinterpret_cast<f32x4 *>(S + (size_t)j * DV + c0 + 4 * cg));
    }
}

template <typename T, int DK, int DV>
hipError_t launch_step_t(int N, int H, const void *q, const void *k, const void *v, const void *g,
                         const void *beta, const float *A_log, float g_min, float scale,
                         float *state, void *o, hipStream_t stream)
{
    const unsigned grid = (unsigned)((size_t)N * H * 2);
    hipLaunchKernelGGL((recurrent_step_kernel<T, DK, DV>), dim3(grid), dim3(128), 0, stream,
                       (const T *)q, (const T *)k, (const T *)v, (const T *)g, (const T *)beta,
                       A_log, g_min, scale, H, state, (T *)o);
    return hipGetLastError();
}

hipError_t launch_recurrent_step(int dtype_bf16, int N, int H, int Dk, int Dv, const void *q,
                                 const void *k, const void *v, const void *g, const void *beta,
                                 const float *A_log, float g_min, float scale, float *state,
                                 void *o, hipStream_t stream)
{
#define KDA_STEP_CASE(TT, DKV, DVV)                                                              \
    if (Dk == DKV && Dv == DVV)                                                                  \
        return launch_step_t<TT, DKV, DVV>(N, H, q, k, v, g, beta, A_log, g_min, scale, state, o, \
                                           stream);
    if (dtype_bf16) {
        KDA_STEP_CASE(bf16, 64, 64)
        KDA_STEP_CASE(bf16, 64, 128)
        KDA_STEP_CASE(bf16, 128, 64)
        KDA_STEP_CASE(bf16, 128, 128)
    } else {
        KDA_STEP_CASE(float, 64, 64)
        KDA_STEP_CASE(float, 64, 128)
        KDA_STEP_CASE(float, 128, 64)
        KDA_STEP_CASE(float, 128, 128)
    }
#undef KDA_STEP_CASE
    return hipErrorInvalidValue;
}

}  // namespace kda
