// Exact per-expert load of the post-gating routing: the counting half.
//
// The balancer is exact-load (UltraEP abstract, arXiv 2606.04101): it works
// from the true token count of each expert in the current microbatch, the
// "Load computation" component of "How dots-infra/ultraep works".
//
// One workgroup counts one group of G consecutive routing tiles of one
// layer and ends; the grid is launched once over every group of every
// layer, so no workgroup waits on another and the loads in flight stay in
// a narrow, advancing window of the routing. Routing is skewed (a hot
// expert shows up in nearly every token), so a tile's histogram is kept as
// kSub interleaved copies, and lane l adds into copy l mod kSub: lanes of a
// wave that hold the same id hit kSub different banks, which bounds the
// serialisation of an LDS atomic at 64 / kSub lanes. Two experts share a
// word (16 bits each): expert e of copy c is half e mod 2 of word
// (e / 2) * kSub + c. Tiles alternate between two such histograms, so one
// tile is counted while the previous one is summed and cleared, with one
// barrier per tile. The workgroup then writes, 16 bits per expert, each
// tile's count of every expert in the group's earlier tiles (tile t of
// group g at row t + g of the per-tile table) and the group's own counts
// (the row after its last tile); the planner's launch scans the groups'
// rows into each group's base and the layer's counts. Ids outside [0, E)
// are not counted. Integer sums: exact and order-independent.
#include "ue_internal.h"

namespace ue {
namespace {

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

constexpr int kSub = 8;   // interleaved histogram copies (two 16-byte reads)

struct CountArgs {
    const int32_t *routing;
    int64_t A;                 // assignments per layer
    int E, tiles, group, row_stride;
    bool vec4;
    uint16_t *rows;            // [L][row_stride = tiles + groups][E]
};

// Two experts share a histogram word, 16 bits each: a copy takes at most
// kLoadTile / kSub ids, far below 2^16, so neither half carries into the
// other, and the eight copies of a word still sum without carrying
// (kLoadTile < 2^16).
// Branch-free: an id out of range adds 0 to its lane's copy of the first
// word, so every lane issues the same instructions.
static_assert(kLoadTile < 65536, "16-bit tile counters");
__device__ __forceinline__ void count_one(int id, int E, int sub,
                                          uint32_t *hist) {
    const bool ok = static_cast<uint32_t>(id) < static_cast<uint32_t>(E);
    atomicAdd(&hist[(ok ? (id >> 1) * kSub : 0) + sub],
              ok ? 1u << ((id & 1) << 4) : 0u);
}

template <int G>
__global__ __launch_bounds__(kBlock) void k_count(CountArgs g) {
    extern __shared__ __align__(16) int32_t lds[];
    const int E = g.E;
    const int EH = (E + 1) >> 1;                     // expert pairs
    // [2][EH][kSub] alternating tiles, two 16-bit counters per word
    uint32_t *hist = reinterpret_cast<uint32_t *>(lds);
    // [G][E] per-tile counts, 16 bits each
    uint16_t *cnt = reinterpret_cast<uint16_t *>(lds + 2 * kSub * EH);
    const int tid = threadIdx.x;
    const int sub = tid & (kSub - 1);
    const int grp = blockIdx.x;
    const int layer = blockIdx.y;
    const int32_t *src = g.routing + static_cast<int64_t>(layer) * g.A;
    const int tile_first = grp * G;
    const int ntiles = g.tiles - tile_first < G ? g.tiles - tile_first : G;
    // The loads of a full tile are issued kAhead tiles before it is
    // counted (a rolling set of registers), the first ones before the
    // histograms are cleared. One tile ahead is the fastest: with every
    // workgroup of the launch resident at once, more loads in flight only
    // crowd the memory system (58 dsv3 layers: 24.9 us at one tile ahead,
    // 26.1 at two, 27.0 at three or four, 27.5 at eight, same box).
    // Plain (temporal) loads: the fused reroute reads the same routing
    // right after and finds it in the device-wide cache (nontemporal loads
    // here cost the reroute 20 us).
    constexpr int kAhead = 1;
    i32x4 r[kAhead][kLoadItems / 4];
    auto full = [&](int s) {
        const int64_t t0 = static_cast<int64_t>(tile_first + s) * kLoadTile;
        return g.vec4 && s < ntiles && t0 + kLoadTile <= g.A;
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
    for (int i = tid; i < 2 * kSub * EH; i += kBlock) hist[i] = 0u;
    __syncthreads();
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
        } else if (s < ntiles) {
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
    // the group's rows: each tile's count in the group's earlier tiles
    // (below G * kLoadTile, so 16 bits), then the group's own counts
    static_assert(kLoadGroup * kLoadTile <= 65535, "16-bit tile offsets");
    uint16_t *rows = g.rows + (static_cast<int64_t>(layer) * g.row_stride +
                               tile_first + grp) * E;
    for (int e = tid; e < E; e += kBlock) {
        int run = 0;
        for (int s = 0; s < ntiles; ++s) {
            rows[static_cast<int64_t>(s) * E + e] = static_cast<uint16_t>(run);
            run += cnt[s * E + e];
        }
        rows[static_cast<int64_t>(ntiles) * E + e] = static_cast<uint16_t>(run);
    }
}

}  // namespace

static size_t load_lds_bytes_for(int E, int G) {
    const size_t EH = (static_cast<size_t>(E) + 1) / 2;
    return sizeof(int32_t) * (2 * kSub * EH) +
           sizeof(uint16_t) * static_cast<size_t>(G) * E;
}

size_t load_lds_bytes(int E) { return load_lds_bytes_for(E, kLoadGroup); }

// Every workgroup of the count launch can be resident at once (eight per
// CU at dsv3 size), and then they crowd the memory system: at most four per
// CU, held there by the LDS each asks for, count 58 dsv3 layers in 23.6
// instead of 25.2 us (three per CU: 27.5 us; same box). The request stays
// within the 64 KiB a launch gets without raising the kernel's limit.
size_t quarter_cu_lds(size_t lds_per_cu, size_t lds_cap) {
    const size_t share = lds_per_cu / 4;
    return (share <= 65536 && share <= lds_cap) ? share : 0;
}
size_t count_lds_bytes(int E, size_t lds_per_cu, size_t lds_cap) {
    const size_t need = load_lds_bytes(E);
    const size_t share = quarter_cu_lds(lds_per_cu, lds_cap);
    return share > need ? share : need;
}

LoadShape load_shape(int64_t A, int L) {
    (void)L;
    LoadShape sh;
    int64_t tiles = (A + kLoadTile - 1) / kLoadTile;
    if (tiles < 1) tiles = 1;
    sh.tiles = static_cast<int>(tiles);
    sh.group = kLoadGroup;
    sh.groups = static_cast<int>((tiles + kLoadGroup - 1) / kLoadGroup);
    return sh;
}

int64_t load_group_rows_cap(int64_t A, int L) {
    return static_cast<int64_t>(L) * load_shape(A, L).groups;
}

hipError_t launch_count(const ue_ctx &c, const int32_t *routing, int L,
                        int64_t A, hipStream_t s) {
    const LoadShape sh = load_shape(A, L);
    CountArgs g;
    g.routing = routing;
    g.A = A;
    g.E = c.E;
    g.tiles = sh.tiles;
    g.group = sh.group;
    g.row_stride = sh.tiles + sh.groups;
    g.vec4 = (A % 4 == 0) && (reinterpret_cast<uintptr_t>(routing) % 16 == 0);
    g.rows = c.tile_off;
    const dim3 grid(sh.groups, L);
    const size_t need = load_lds_bytes_for(c.E, sh.group);
    const size_t lds = c.count_lds > need ? c.count_lds : need;
    hipLaunchKernelGGL(k_count<kLoadGroup>, grid, dim3(kBlock), lds, s, g);
    return hipGetLastError();
}

}  // namespace ue
