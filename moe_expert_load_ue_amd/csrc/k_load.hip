// Exact per-expert load of the post-gating routing.
//
// The balancer is exact-load (UltraEP abstract, arXiv 2606.04101): it works
// from the true token count of each expert in the current microbatch, the
// "Load computation" component of "How dots-infra/ultraep works".
//
// One workgroup counts one tile of one layer. Routing is skewed (a hot
// expert shows up in nearly every token), so lanes first find the other
// lanes holding the same id (one ballot per id bit) and only one lane per
// distinct id adds the group's size to the LDS histogram: no LDS atomic
// ever sees two lanes of a wave on one address. Tiles then combine their
// histograms with the decoupled lookback of ue_internal.h; the tile with the
// last ticket ends with the inclusive prefix over the whole layer, which is
// the layer's counts. No fence, no global atomics on data, no clearing
// launch; integer sums make the result exact and order-independent.
#include "ue_internal.h"

namespace ue {
namespace {

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

struct LoadArgs {
    const int32_t *routing;
    int64_t A;                 // assignments per layer
    int E, ebits, tiles, max_tiles;
    bool vec4;
    uint32_t spin_limit;
    uint64_t *state;           // [max_layers][max_tiles][E]
    uint32_t *ticket, *epoch;  // [max_layers]
    int32_t *counts, *invalid;
};

__device__ __forceinline__ void count_one(int id, int E, int ebits,
                                          int32_t *hist) {
    const bool valid = static_cast<uint32_t>(id) < static_cast<uint32_t>(E);
    const uint64_t peers = match_peers(id, valid, ebits);
    if (valid && mask_rank(peers) == 0)
        atomicAdd(&hist[id], __builtin_popcountll(peers));
}

__global__ __launch_bounds__(kBlock) void k_load(LoadArgs g) {
    extern __shared__ int32_t lds[];
    int32_t *hist = lds;            // [E] this tile's counts
    int32_t *excl = lds + g.E;      // [E] counts of earlier tiles
    __shared__ uint32_t s_ticket, s_epoch;
    __shared__ int wsum[kWaves];

    const int E = g.E;
    const int layer = blockIdx.y;
    const int tid = threadIdx.x;
    if (tid == 0) take_ticket(g.ticket + layer, g.epoch + layer, g.tiles,
                              s_ticket, s_epoch);
    for (int e = tid; e < E; e += kBlock) hist[e] = 0;
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
            count_one(r[i].x, E, g.ebits, hist);
            count_one(r[i].y, E, g.ebits, hist);
            count_one(r[i].z, E, g.ebits, hist);
            count_one(r[i].w, E, g.ebits, hist);
        }
    } else {
        // ragged tile: whole waves step together so the ballots see all lanes
        for (int64_t a0 = t0; a0 < t1; a0 += kBlock) {
            const int64_t a = a0 + tid;
            count_one(a < t1 ? src[a] : -1, E, g.ebits, hist);
        }
    }
    __syncthreads();

    uint64_t *st = g.state + static_cast<int64_t>(layer) * g.max_tiles * E;
    const bool bad = tile_lookback(st, tile, E, s_epoch, hist, excl,
                                   g.spin_limit);
    const int poisoned = __syncthreads_or(bad);
    if (tile != g.tiles - 1) return;

    // last tile: inclusive prefix over all tiles = the layer's counts
    int32_t *out = g.counts + static_cast<int64_t>(layer) * E;
    int part = 0;
    for (int e = tid; e < E; e += kBlock) {
        const int c = excl[e] + hist[e];
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

size_t load_lds_bytes(int E) { return sizeof(int32_t) * 2 * E; }

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
    g.ticket = c.load_ticket;
    g.epoch = c.load_epoch;
    g.counts = counts;
    g.invalid = invalid;
    hipLaunchKernelGGL(k_load, dim3(tiles, L), dim3(kBlock),
                       load_lds_bytes(c.E), s, g);
    return hipGetLastError();
}

}  // namespace ue
