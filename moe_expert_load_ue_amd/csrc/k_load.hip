// Exact per-expert load of the post-gating routing.
//
// The balancer is exact-load (UltraEP abstract, arXiv 2606.04101): it works
// from the true token count of each expert in the current microbatch, the
// "Load computation" component of "How dots-infra/ultraep works".
//
// One workgroup counts a group of consecutive routing tiles of one layer
// into LDS: 8 tiles, or 16 when that still leaves two workgroups per CU
// (fewer groups per layer shorten the lookback). Routing is skewed (a hot
// expert shows up in nearly every token), so a tile's histogram is kept as
// kSub interleaved copies, and lane l adds into copy l mod kSub: lanes of a
// wave that hold the same id hit kSub different banks, which bounds the
// serialisation of an LDS atomic at 64 / kSub lanes. Two experts share a
// word (16 bits each): expert e of copy c is half e mod 2 of word
// (e / 2) * kSub + c. Tiles alternate between two such histograms, so one
// tile is counted while the previous one is summed and cleared, with one
// barrier per tile. Groups then combine their histograms with the
// decoupled lookback of ue_internal.h; the group with the last ticket ends
// with the inclusive prefix over the whole layer, which is the layer's
// counts. Every group also writes, for each of its tiles, the count of each
// expert in all earlier tiles of the layer (and the last group the layer's
// totals after the last tile): the fused reroute reads those instead of
// scanning again. No fence, no global atomics on data, no clearing launch;
// integer sums make the result exact and order-independent.
#include "ue_internal.h"

namespace ue {
namespace {

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

constexpr int kSub = 8;   // interleaved histogram copies (two 16-byte reads)

struct LoadArgs {
    const int32_t *routing;
    int64_t A;                 // assignments per layer
    int E, groups, tiles, max_groups, max_tiles;
    bool vec4;
    uint32_t spin_limit;
    uint64_t *state;           // [max_layers][max_groups][E]
    uint64_t *tick;            // [max_layers]
    int32_t *group_base;       // [max_layers][max_groups][E]
    uint16_t *tile_off;        // [max_layers][max_tiles + max_groups][E]
    int32_t *status;           // [max_layers] poisoned flag of the call
    int32_t *counts, *invalid;
};

// Two experts share a histogram word, 16 bits each: a copy of one tile
// takes at most kLoadTile / kSub ids, far below 2^16, so neither half
// carries into the other, and the eight copies of a word still sum
// without carrying (kLoadTile < 2^16).
static_assert(kLoadTile < 65536, "16-bit tile counters");
__device__ __forceinline__ void count_one(int id, int E, int sub,
                                          uint32_t *hist) {
    if (static_cast<uint32_t>(id) < static_cast<uint32_t>(E))
        atomicAdd(&hist[(id >> 1) * kSub + sub], 1u << ((id & 1) << 4));
}

// G tiles per workgroup: kLoadGroup, or kLoadGroupWide when there are
// enough groups to fill the device (fewer groups per layer shorten the
// lookback walks).
template <int G>
__global__ __launch_bounds__(kBlock) void k_load(LoadArgs g) {
    extern __shared__ __align__(16) int32_t lds[];
    const int EH = (g.E + 1) >> 1;         // expert pairs
    // [2][EH][kSub] alternating tiles, two 16-bit counters per word
    uint32_t *hist = reinterpret_cast<uint32_t *>(lds);
    // [G][E] per-tile counts, 16 bits each
    uint16_t *cnt = reinterpret_cast<uint16_t *>(lds + 2 * kSub * EH);
    int32_t *gcnt = lds + 2 * kSub * EH + (G * g.E + 1) / 2;  // [E]
    int32_t *excl = gcnt + g.E;            // [E] counts of earlier groups
    __shared__ uint32_t s_ticket, s_epoch;
    __shared__ int wsum[kWaves], wany[kWaves];

    const int E = g.E;
    const int layer = blockIdx.y;
    const int tid = threadIdx.x;
    const int sub = tid & (kSub - 1);
    if (tid == 0) take_ticket(g.tick + layer, g.groups, s_ticket, s_epoch);
    for (int i = tid; i < 2 * kSub * EH; i += kBlock) hist[i] = 0u;
    __syncthreads();
    const int grp = static_cast<int>(s_ticket);
    if (grp >= g.groups) return;    // only after a corrupted earlier launch

    const int32_t *src = g.routing + static_cast<int64_t>(layer) * g.A;
    const int tile_first = grp * G;
    // The loads of a full tile are issued kAhead tiles before it is
    // counted (a rolling set of registers). Plain (temporal) loads: the
    // fused reroute reads the same routing right after, and finds it in the
    // device-wide cache.
    constexpr int kAhead = 4;
    i32x4 r[kAhead][kLoadItems / 4];
    auto full = [&](int s) {
        const int64_t t0 = static_cast<int64_t>(tile_first + s) * kLoadTile;
        return g.vec4 && t0 + kLoadTile <= g.A;
    };
    auto issue = [&](int s) {
        if (full(s)) {
            const i32x4 *v = reinterpret_cast<const i32x4 *>(
                src + static_cast<int64_t>(tile_first + s) * kLoadTile);
#pragma unroll
            for (int i = 0; i < kLoadItems / 4; ++i)
                r[s % kAhead][i] = v[i * kBlock + tid];
        }
    };
#pragma unroll
    for (int s = 0; s < kAhead && s < G; ++s) issue(s);
#pragma unroll
    for (int s = 0; s < G; ++s) {
        uint32_t *h = hist + (s & 1) * kSub * EH;
        if (full(s)) {
#pragma unroll
            for (int i = 0; i < kLoadItems / 4; ++i) {
                const i32x4 v = r[s % kAhead][i];
                count_one(v.x, E, sub, h);
                count_one(v.y, E, sub, h);
                count_one(v.z, E, sub, h);
                count_one(v.w, E, sub, h);
            }
            if (s + kAhead < G) issue(s + kAhead);
        } else {
            const int64_t t0 = static_cast<int64_t>(tile_first + s) * kLoadTile;
            const int64_t t1 = (t0 + kLoadTile < g.A) ? t0 + kLoadTile : g.A;
            for (int64_t a = t0 + tid; a < t1; a += kBlock)
                count_one(src[a], E, sub, h);
        }
        __syncthreads();
        // sum and clear this tile's copies while the next tile is counted
        // into the other histogram; the barrier after that count orders
        // the clearing before this histogram's next use
        for (int ep = tid; ep < EH; ep += kBlock) {
            i32x4 *b = reinterpret_cast<i32x4 *>(h + ep * kSub);
            const i32x4 u = b[0], v = b[1];
            const uint32_t t = static_cast<uint32_t>(u.x + u.y + u.z + u.w +
                                                     v.x + v.y + v.z + v.w);
            cnt[s * E + 2 * ep] = static_cast<uint16_t>(t & 0xFFFFu);
            if (2 * ep + 1 < E)
                cnt[s * E + 2 * ep + 1] = static_cast<uint16_t>(t >> 16);
            b[0] = i32x4{0, 0, 0, 0};
            b[1] = i32x4{0, 0, 0, 0};
        }
    }
    __syncthreads();
    for (int e = tid; e < E; e += kBlock) {
        int c = 0;
        for (int s = 0; s < G; ++s) c += cnt[s * E + e];
        gcnt[e] = c;
    }
    __syncthreads();

    uint64_t *st = g.state + static_cast<int64_t>(layer) * g.max_groups * E;
    const bool bad = tile_lookback(
        st, grp, E, s_epoch, [&](int e) { return gcnt[e]; },
        [&](int e, int v) { excl[e] = v; }, g.spin_limit);
    const int poisoned = block_any(bad, wany);

    // the group's count of each expert in all earlier groups; per tile of
    // the group, the count in the group's earlier tiles (16 bits: a group
    // holds at most G * kLoadTile assignments), then the group's own count
    // in the row after its last tile
    static_assert(kLoadGroupWide * kLoadTile <= 65535, "16-bit tile offsets");
    int32_t *gb = g.group_base +
                  (static_cast<int64_t>(layer) * g.max_groups + grp) * E;
    uint16_t *to = g.tile_off +
                   (static_cast<int64_t>(layer) * (g.max_tiles + g.max_groups) +
                    tile_first + grp) * E;
    const int ntiles = g.tiles - tile_first < G ? g.tiles - tile_first : G;
    for (int e = tid; e < E; e += kBlock) {
        gb[e] = excl[e];
        int run = 0;
        for (int s = 0; s < ntiles; ++s) {
            to[s * E + e] = static_cast<uint16_t>(run);
            run += cnt[s * E + e];
        }
        to[ntiles * E + e] = static_cast<uint16_t>(run);
    }
    if (grp != g.groups - 1) return;

    // last group: inclusive prefix over all groups = the layer's counts
    int32_t *out = g.counts + static_cast<int64_t>(layer) * E;
    int part = 0;
    for (int e = tid; e < E; e += kBlock) {
        const int c = excl[e] + gcnt[e];
        out[e] = c;
        part += c;
    }
    int total;
    block_exclusive_sum(part, wsum, total);
    if (tid == 0) {
        // the last group's lookback saw every group's words, so it is
        // poisoned exactly when some wait of the layer gave up
        g.status[layer] = poisoned;
        if (g.invalid)
            g.invalid[layer] = static_cast<int32_t>(g.A - total) |
                               (poisoned ? kPoisonBit : 0);
    }
}

}  // namespace

static size_t load_lds_bytes_for(int E, int G) {
    const size_t EH = (static_cast<size_t>(E) + 1) / 2;
    return sizeof(int32_t) * (2 * kSub * EH +
                              (static_cast<size_t>(G) * E + 1) / 2 +
                              2 * static_cast<size_t>(E));
}

size_t load_lds_bytes(int E) { return load_lds_bytes_for(E, kLoadGroupWide); }

int load_group_tiles(const ue_ctx &c, int tiles, int L) {
    // wide groups once they still give two workgroups per CU
    const int wide_groups = (tiles + kLoadGroupWide - 1) / kLoadGroupWide;
    return static_cast<int64_t>(wide_groups) * L >= 2 * c.num_cu
               ? kLoadGroupWide
               : kLoadGroup;
}

hipError_t launch_load(const ue_ctx &c, const int32_t *routing, int L,
                       int64_t A, int32_t *counts, int32_t *invalid,
                       hipStream_t s) {
    int tiles = static_cast<int>((A + kLoadTile - 1) / kLoadTile);
    if (tiles < 1) tiles = 1;
    const int G = load_group_tiles(c, tiles, L);
    const bool wide = G == kLoadGroupWide;
    const int groups = (tiles + G - 1) / G;
    LoadArgs g;
    g.routing = routing;
    g.A = A;
    g.E = c.E;
    g.groups = groups;
    g.tiles = tiles;
    g.max_groups = c.max_load_groups;
    g.max_tiles = c.max_rr_tiles;
    g.vec4 = (A % 4 == 0) && (reinterpret_cast<uintptr_t>(routing) % 16 == 0);
    g.spin_limit = c.wait_limit;
    g.state = c.load_state;
    g.tick = c.load_tick;
    g.group_base = c.group_base;
    g.tile_off = c.tile_off;
    g.status = c.load_status;
    g.counts = counts;
    g.invalid = invalid;
    if (wide)
        hipLaunchKernelGGL(k_load<kLoadGroupWide>, dim3(groups, L),
                           dim3(kBlock), load_lds_bytes_for(c.E, G), s, g);
    else
        hipLaunchKernelGGL(k_load<kLoadGroup>, dim3(groups, L), dim3(kBlock),
                           load_lds_bytes_for(c.E, G), s, g);
    return hipGetLastError();
}

}  // namespace ue
