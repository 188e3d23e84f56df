// Rank loads under an earlier plan: the periodic, historical-load
// balancing that the UltraEP abstract (arXiv 2606.04101) and the news
// write-up (section on the problem UltraEP solves) contrast with exact-load
// balancing, evaluated on a layer's new counts.
//
// The old plan keeps its replicas and their proportions. Of expert e's n
// new assignments, with old capacities c_1..c_m (master first, then the
// replicas in table order) summing to C, replica i takes those j with
// floor(n * c_<i / C) <= j < floor(n * c_<=i / C): the capacity prefix
// scaled from C to n, the same covering rule as the reroute. An expert the
// old plan saw no tokens of (C = 0) stays whole on its master.
//
// One workgroup per layer; one thread per expert walks its replicas and
// adds into per-rank LDS counters. Integer adds: the result does not depend
// on the order.
#include "ue_internal.h"

namespace ue {
namespace {

__global__ __launch_bounds__(kBlock) void k_stale(
    const int32_t *__restrict__ placement, const int32_t *__restrict__ counts,
    int E, int R, int NS, int P, ue_placement_layout lay,
    int32_t *__restrict__ rank_loads) {
    extern __shared__ __align__(16) int32_t lds[];
    unsigned long long *load = reinterpret_cast<unsigned long long *>(lds);
    const int layer = blockIdx.x;
    const int tid = threadIdx.x;
    const int32_t *pl = placement + static_cast<int64_t>(layer) * lay.words;
    const int32_t *cnt = counts + static_cast<int64_t>(layer) * E;
    for (int r = tid; r < R; r += kBlock) load[r] = 0ull;
    __syncthreads();
    for (int e = tid; e < E; e += kBlock) {
        const int64_t n = cnt[e] > 0 ? cnt[e] : 0;
        // the table as the planner wrote it, indices clamped: a corrupt
        // block cannot send a load outside [0, R)
        int lo = pl[lay.rep_off + e], hi = pl[lay.rep_off + e + 1];
        lo = lo < 0 ? 0 : (lo > P ? P : lo);
        hi = hi < lo ? lo : (hi > P ? P : hi);
        if (hi == lo) continue;
        int64_t C = 0;
        for (int i = lo; i < hi; ++i) {
            const int c = pl[lay.rep_cap + i];
            C += c > 0 ? c : 0;
        }
        if (C == 0) {                       // stays whole on its master
            const int s = pl[lay.rep_slot + lo];
            if (n > 0 && s >= 0 && s < P)
                atomicAdd(&load[s / NS], static_cast<unsigned long long>(n));
            continue;
        }
        int64_t before = 0, acc = 0;
        for (int i = lo; i < hi; ++i) {
            const int c = pl[lay.rep_cap + i];
            acc += c > 0 ? c : 0;
            const int64_t upto = (n * acc) / C;
            const int64_t take = upto - before;
            before = upto;
            const int s = pl[lay.rep_slot + i];
            if (take > 0 && s >= 0 && s < P)
                atomicAdd(&load[s / NS], static_cast<unsigned long long>(take));
        }
    }
    __syncthreads();
    for (int r = tid; r < R; r += kBlock)
        rank_loads[static_cast<int64_t>(layer) * R + r] =
            static_cast<int32_t>(load[r]);
}

}  // namespace

hipError_t launch_stale(const ue_ctx &c, const int32_t *placement,
                        const int32_t *counts, int L, int32_t *rank_loads,
                        hipStream_t s) {
    hipLaunchKernelGGL(k_stale, dim3(L), dim3(kBlock),
                       sizeof(unsigned long long) * c.R, s, placement, counts,
                       c.E, c.R, c.NS, c.P, c.lay, rank_loads);
    return hipGetLastError();
}

}  // namespace ue
