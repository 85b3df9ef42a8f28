// kda_table.h -- chunk table of packed sequences: the per-sequence arithmetic
// of chunk_table_kernel, written so that it also compiles for the host (a
// host build defines KDA_HD as empty before including this file).
//
// Chunks restart at every sequence start ("Kimi K3 Technical Report", §2.1.1,
// chunkwise form of eqs. (3)-(4), applied per packed sequence).  cu_seqlens is
// trusted to be non-decreasing from 0 to T, but not relied on for memory
// safety: each sequence's span is clamped into [0, T] (a decreasing pair gives
// an empty sequence) and the chunk offsets saturate at the workspace's chunk
// capacity, so bad offsets give wrong results, never accesses outside the
// caller's tensors or the workspace.
//
// Table (int32, in the workspace):
//   chunk_off [N + 1]  chunk_off[s] = min(cap, sum_{s' < s} chunks(len_s')),
//                      chunk_off[N] the number of chunks with a block
//   order     [N]      sequences by decreasing length, ties by index
//                      (N <= ORDER_MAX_N), else the identity
//   span      [2 N]    clamped (first token, length) of each sequence
#pragma once

#include <stdint.h>

#ifndef KDA_HD
#define KDA_HD __host__ __device__
#endif

namespace kda {
namespace table {

constexpr int THREADS = 1024;        // one workgroup builds the table
constexpr int ORDER_MAX_N = 2048;    // longest-first order up to this many sequences

// Clamped span of sequence s.
KDA_HD inline void seq_span(const int32_t *cu, int s, int T, int &start, int &len)
{
    const int a = cu[s] < 0 ? 0 : (cu[s] > T ? T : cu[s]);
    const int b = cu[s + 1] < 0 ? 0 : (cu[s + 1] > T ? T : cu[s + 1]);
    start = a;
    len = b > a ? b - a : 0;
}

// Chunks of a sequence of len >= 0 tokens (no overflow near INT_MAX).
KDA_HD inline int chunks_of(int len) { return (len >> 6) + ((len & 63) != 0); }

// Sequences [s0, s1) handled by thread t.
KDA_HD inline void thread_range(int N, int t, int &s0, int &s1)
{
    const int per = (N + THREADS - 1) / THREADS;
    const long long a = (long long)t * per;
    s0 = a < N ? (int)a : N;
    s1 = s0 + per < N ? s0 + per : N;
}

// First pass of thread t: chunks of its sequences; records their spans.
KDA_HD inline long long count(const int32_t *cu, int N, int T, int t, int32_t *span)
{
    int s0, s1;
    thread_range(N, t, s0, s1);
    long long n = 0;
    for (int s = s0; s < s1; ++s) {
        int a, l;
        seq_span(cu, s, T, a, l);
        span[2 * s] = a;
        span[2 * s + 1] = l;
        n += chunks_of(l);
    }
    return n;
}

// Second pass of thread t, given the chunks of all sequences before its own.
KDA_HD inline void offsets(const int32_t *cu, int N, int T, int cap, int t, long long before, int32_t *chunk_off)
{
    int s0, s1;
    thread_range(N, t, s0, s1);
    for (int s = s0; s < s1; ++s) {
        chunk_off[s] = before < cap ? (int)before : cap;
        int a, l;
        seq_span(cu, s, T, a, l);
        before += chunks_of(l);
    }
}

// Position of sequence s in the longest-first order (ties by index).
KDA_HD inline int rank(const int32_t *cu, int N, int T, int s)
{
    if (N > ORDER_MAX_N) return s;
    int a, ls;
    seq_span(cu, s, T, a, ls);
    int r = 0;
    for (int y = 0; y < N; ++y) {
        int b, ly;
        seq_span(cu, y, T, b, ly);
        r += (ly > ls) || (ly == ls && y < s);
    }
    return r;
}

}  // namespace table
}  // namespace kda
