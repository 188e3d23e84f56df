// Exact per-expert load of the post-gating routing.
//
// The balancer is exact-load (UltraEP abstract, arXiv 2606.04101): it works
// from the true token count of each expert in the current microbatch, the
// "Load computation" component of "How dots-infra/ultraep works".
//
// One workgroup counts one tile of one layer into an LDS histogram (LDS
// atomics; integer adds commute, so the result is exact and independent of
// order), then adds its non-zero bins into a per-layer accumulator in the
// workspace with device-scope atomics. The last workgroup of the layer (by a
// completion counter) moves the accumulator into `counts` and leaves it at
// zero for the next call, so no separate clearing launch is needed.
#include "ue_internal.h"

namespace ue {
namespace {

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(kBlock) void k_load(
    const int32_t *__restrict__ routing, int64_t A, int E, int tiles,
    bool vec4, int32_t *__restrict__ acc, int32_t *__restrict__ inv_acc,
    uint32_t *__restrict__ done, int32_t *__restrict__ counts,
    int32_t *__restrict__ invalid_out) {
    extern __shared__ int32_t hist[];  // [E]
    __shared__ int wsum[kWaves];
    __shared__ int s_last;

    const int layer = blockIdx.y;
    const int tile = blockIdx.x;
    const int tid = threadIdx.x;
    for (int e = tid; e < E; e += kBlock) hist[e] = 0;
    __syncthreads();

    const int32_t *src = routing + static_cast<int64_t>(layer) * A;
    const int64_t t0 = static_cast<int64_t>(tile) * kLoadTile;
    const int64_t t1 = (t0 + kLoadTile < A) ? t0 + kLoadTile : A;
    int bad = 0;
    if (vec4 && t1 - t0 == kLoadTile) {
        // full tile: kLoadItems/4 coalesced 16-byte loads per thread
        const i32x4 *v = reinterpret_cast<const i32x4 *>(src + t0);
        i32x4 r[kLoadItems / 4];
#pragma unroll
        for (int i = 0; i < kLoadItems / 4; ++i)
            r[i] = __builtin_nontemporal_load(v + i * kBlock + tid);
#pragma unroll
        for (int i = 0; i < kLoadItems / 4; ++i) {
            const int32_t ids[4] = {r[i].x, r[i].y, r[i].z, r[i].w};
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                if (static_cast<uint32_t>(ids[q]) < static_cast<uint32_t>(E))
                    atomicAdd(&hist[ids[q]], 1);
                else
                    ++bad;
            }
        }
    } else {
        for (int64_t a = t0 + tid; a < t1; a += kBlock) {
            const int32_t id = src[a];
            if (static_cast<uint32_t>(id) < static_cast<uint32_t>(E))
                atomicAdd(&hist[id], 1);
            else
                ++bad;
        }
    }
    int bad_total;
    block_exclusive_sum(bad, wsum, bad_total);   // also a barrier for hist

    int32_t *lacc = acc + static_cast<int64_t>(layer) * E;
    for (int e = tid; e < E; e += kBlock) {
        const int c = hist[e];
        if (c) atomicAdd(&lacc[e], c);
    }
    if (tid == 0 && bad_total) atomicAdd(&inv_acc[layer], bad_total);
    __threadfence();
    __syncthreads();
    if (tid == 0) {
        const uint32_t prev = atomicAdd(&done[layer], 1u);
        s_last = (prev == static_cast<uint32_t>(tiles - 1));
    }
    __syncthreads();
    if (!s_last) return;
    __threadfence();
    int32_t *out = counts + static_cast<int64_t>(layer) * E;
    for (int e = tid; e < E; e += kBlock) out[e] = atomicExch(&lacc[e], 0);
    if (tid == 0) {
        const int inv = atomicExch(&inv_acc[layer], 0);
        if (invalid_out) invalid_out[layer] = inv;
        atomicExch(&done[layer], 0u);
    }
}

}  // namespace

hipError_t launch_load(const ue_ctx &c, const int32_t *routing, int L,
                       int64_t A, int32_t *counts, int32_t *invalid,
                       hipStream_t s) {
    int tiles = static_cast<int>((A + kLoadTile - 1) / kLoadTile);
    if (tiles < 1) tiles = 1;
    const bool vec4 = (A % 4 == 0) &&
                      (reinterpret_cast<uintptr_t>(routing) % 16 == 0);
    dim3 grid(tiles, L);
    hipLaunchKernelGGL(k_load, grid, dim3(kBlock), c.E * sizeof(int32_t), s,
                       routing, A, c.E, tiles, vec4, c.load_acc, c.load_inv,
                       c.load_done, counts, invalid);
    return hipGetLastError();
}

}  // namespace ue
