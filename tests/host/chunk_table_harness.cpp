// Host build of the packed-sequence chunk table: runs the per-thread passes of
// chunk_table_kernel (gated_delta_rule_20_amd/csrc/kda_table.h) for every one
// of its threads in order, with the workgroup's scan done serially, and
// prints the table.  Input on stdin: N T cap, then the N + 1 entries of
// cu_seqlens.  Output: three lines (chunk_off, order, span).
#define KDA_HD
#include "kda_table.h"

#include <cstdio>
#include <vector>

int main()
{
    int N, T, cap;
    if (std::scanf("%d %d %d", &N, &T, &cap) != 3 || N < 1) return 2;
    std::vector<int32_t> cu(N + 1), chunk_off(N + 1, -1), order(N, -1), span(2 * N, -1);
    for (int s = 0; s <= N; ++s)
        if (std::scanf("%d", &cu[s]) != 1) return 2;
    using namespace kda::table;
    std::vector<long long> local(THREADS);
    for (int t = 0; t < THREADS; ++t) local[t] = count(cu.data(), N, T, t, span.data());
    long long before = 0;
    for (int t = 0; t < THREADS; ++t) {
        offsets(cu.data(), N, T, cap, t, before, chunk_off.data());
        before += local[t];
    }
    chunk_off[N] = before < cap ? (int)before : cap;
    for (int t = 0; t < THREADS; ++t)
        for (int s = t; s < N; s += THREADS) order[rank(cu.data(), N, T, s)] = s;
    for (auto *v : {&chunk_off, &order, &span}) {
        for (size_t i = 0; i < v->size(); ++i) std::printf(i ? " %d" : "%d", (*v)[i]);
        std::printf("\n");
    }
    return 0;
}
