// Exact per-expert load of the post-gating routing.
//
// The balancer is exact-load (UltraEP abstract, arXiv 2606.04101): it works
// from the true token count of each expert in the current microbatch, the
// "Load computation" component of "How dots-infra/ultraep works".
//
// One workgroup counts one tile of one layer into LDS. Routing is skewed
// (a hot expert shows up in nearly every token), so the tile histogram is
// kept as kSub interleaved copies, bin e of copy c at e * kSub + c, and lane
// l adds into copy l mod kSub: lanes of a wave that hold the same id hit
// kSub different banks, which bounds the serialisation of an LDS atomic at
// 64 / kSub lanes. Tiles then combine their histograms with the decoupled
// lookback of ue_internal.h; the tile with the last ticket ends with the
// inclusive prefix over the whole layer, which is the layer's counts. No
// fence, no global atomics on data, no clearing launch; integer sums make
// the result exact and order-independent.
#include "ue_internal.h"

namespace ue {
namespace {

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

constexpr int kSub = 8;   // interleaved histogram copies

struct LoadArgs {
    const int32_t *routing;
    int64_t A;                 // assignments per layer
    int E, ebits, tiles, max_tiles;
    bool vec4;
    uint32_t spin_limit;
    uint64_t *state;           // [max_layers][max_tiles][E]
    uint64_t *tick;            // [max_layers]
    int32_t *counts, *invalid;
};

__device__ __forceinline__ void count_one(int id, int E, int sub,
                                          int32_t *hist) {
    if (static_cast<uint32_t>(id) < static_cast<uint32_t>(E))
        atomicAdd(&hist[id * kSub + sub], 1);
}

__global__ __launch_bounds__(kBlock) void k_load(LoadArgs g) {
    extern __shared__ int32_t lds[];
    int32_t *hist = lds;               // [E][kSub] this tile's counts
    int32_t *cnt = lds + kSub * g.E;   // [E] summed over the copies
    int32_t *excl = cnt + g.E;         // [E] counts of earlier tiles
    __shared__ uint32_t s_ticket, s_epoch;
    __shared__ int wsum[kWaves];

    const int E = g.E;
    const int layer = blockIdx.y;
    const int tid = threadIdx.x;
    const int sub = tid & (kSub - 1);
    if (tid == 0) take_ticket(g.tick + layer, g.tiles, s_ticket, s_epoch);
    for (int i = tid; i < kSub * E; i += kBlock) hist[i] = 0;
    __syncthreads();
    const int tile = static_cast<int>(s_ticket);
    if (tile >= g.tiles) return;    // only after a corrupted earlier launch

    const int32_t *src = g.routing + static_cast<int64_t>(layer) * g.A;
    const int64_t t0 = static_cast<int64_t>(tile) * kLoadTile;
    const int64_t t1 = (t0 + kLoadTile < g.A) ? t0 + kLoadTile : g.A;
    if (g.vec4 && t1 - t0 == kLoadTile) {
        const i32x4 *v = reinterpret_cast<const i32x4 *>(src + t0);
        i32x4 r[kLoadItems / 4];
#pragma unroll
        for (int i = 0; i < kLoadItems / 4; ++i)
            r[i] = __builtin_nontemporal_load(v + i * kBlock + tid);
#pragma unroll
        for (int i = 0; i < kLoadItems / 4; ++i) {
            count_one(r[i].x, E, sub, hist);
            count_one(r[i].y, E, sub, hist);
            count_one(r[i].z, E, sub, hist);
            count_one(r[i].w, E, sub, hist);
        }
    } else {
        for (int64_t a = t0 + tid; a < t1; a += kBlock)
            count_one(src[a], E, sub, hist);
    }
    __syncthreads();
    for (int e = tid; e < E; e += kBlock) {
        int c = 0;
#pragma unroll
        for (int k = 0; k < kSub; ++k) c += hist[e * kSub + k];
        cnt[e] = c;
    }
    __syncthreads();

    uint64_t *st = g.state + static_cast<int64_t>(layer) * g.max_tiles * E;
    const bool bad = tile_lookback(st, tile, E, s_epoch, cnt, excl,
                                   g.spin_limit);
    const int poisoned = __syncthreads_or(bad);
    if (tile != g.tiles - 1) return;

    // last tile: inclusive prefix over all tiles = the layer's counts
    int32_t *out = g.counts + static_cast<int64_t>(layer) * E;
    int part = 0;
    for (int e = tid; e < E; e += kBlock) {
        const int c = excl[e] + cnt[e];
        out[e] = c;
        part += c;
    }
    int total;
    block_exclusive_sum(part, wsum, total);
    if (tid == 0 && g.invalid)
        g.invalid[layer] = static_cast<int32_t>(g.A - total) |
                           (poisoned ? kPoisonBit : 0);
}

}  // namespace

size_t load_lds_bytes(int E) { return sizeof(int32_t) * (kSub + 2) * E; }

hipError_t launch_load(const ue_ctx &c, const int32_t *routing, int L,
                       int64_t A, int32_t *counts, int32_t *invalid,
                       hipStream_t s) {
    int tiles = static_cast<int>((A + kLoadTile - 1) / kLoadTile);
    if (tiles < 1) tiles = 1;
    LoadArgs g;
    g.routing = routing;
    g.A = A;
    g.E = c.E;
    g.ebits = c.ebits;
    g.tiles = tiles;
    g.max_tiles = c.max_load_tiles;
    g.vec4 = (A % 4 == 0) && (reinterpret_cast<uintptr_t>(routing) % 16 == 0);
    g.spin_limit = 1u << 22;
    g.state = c.load_state;
    g.tick = c.load_tick;
    g.counts = counts;
    g.invalid = invalid;
    hipLaunchKernelGGL(k_load, dim3(tiles, L), dim3(kBlock),
                       load_lds_bytes(c.E), s, g);
    return hipGetLastError();
}

}  // namespace ue
