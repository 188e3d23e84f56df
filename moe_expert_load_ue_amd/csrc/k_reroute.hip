// Routing expansion and dispatch layout in one pass over the routing.
//
// "How dots-infra/ultraep works" (connection list): routing expansion turns
// logical routing into physical routing for token dispatch. The j-th
// assignment of expert e in flat (token, slot) order goes to the replica of
// e whose capacity prefix (master first, then replicas in creation order)
// covers j; its dispatch position is slot_off[p] + (j - prefix), which is
// the stable sort of assignments by physical slot.
//
// j needs, for every assignment, the number of earlier assignments of the
// same expert in the whole layer. Each workgroup takes a tile by an atomic
// ticket (so it only ever waits on tiles that have already started), and:
//   1. each wave ranks its ids in rounds of 64 consecutive assignments:
//      lanes with equal ids are found with one ballot per id bit, a lane's
//      rank among its peers is the popcount of peers below it, and a
//      per-wave LDS counter per expert carries the count across rounds;
//   2. per expert, the per-wave counts are scanned across the 4 waves;
//   3. decoupled lookback over earlier tiles, one expert per thread: the
//      tile publishes its per-expert count, then walks back over the tiles
//      before it, adding their published counts until it meets a published
//      inclusive prefix, then publishes its own inclusive prefix. Each
//      64-bit status word holds {call epoch, flag, value}, so stale words of
//      earlier calls are never mistaken for current ones and nothing has to
//      be cleared between calls;
//   4. j = tile prefix + wave prefix + rank; the replica is found by a short
//      scan of the expert's capacity prefixes held in LDS.
// The last workgroup of a layer publishes rank counts and fault counts and
// returns the ticket and completion counters to zero.
#include "ue_internal.h"

namespace ue {
namespace {

constexpr uint64_t kFlagAgg = 1;
constexpr uint64_t kFlagPrefix = 2;

__device__ __forceinline__ uint64_t pack_state(uint32_t epoch, uint64_t flag,
                                               uint32_t value) {
    return (static_cast<uint64_t>(epoch) << 32) | (flag << 30) | value;
}

struct RerouteArgs {
    const int32_t *routing;
    const int32_t *placement;
    int64_t A;                 // assignments per layer
    int E, R, NS, P, ebits, tiles, max_tiles;
    uint32_t spin_limit;       // bound on one lookback wait
    ue_placement_layout lay;
    int32_t *phys, *perm, *inv_perm;
    uint64_t *state;
    uint32_t *ticket, *done, *epoch;
    int32_t *rank_acc, *fault_acc, *rank_counts, *faults;
};

__global__ __launch_bounds__(kBlock) void k_reroute(RerouteArgs g) {
    extern __shared__ int32_t lds[];
    __shared__ int wsum[kWaves];
    __shared__ uint32_t s_ticket, s_epoch;
    __shared__ int s_last;

    const int E = g.E, P = g.P, R = g.R;
    const int layer = blockIdx.y;
    const int tid = threadIdx.x;
    const int w = tid >> 6;
    const int lane = tid & 63;

    // LDS: per-wave counters [kWaves][E], tile prefix [E], replica table
    // (rep_off [E+1], rep_slot [P], rep_lo [P] prefix start, rep_hi [P]
    // prefix end), slot_off [P], rank histogram [R].
    int32_t *whist = lds;
    int32_t *tile_base = whist + kWaves * E;
    int32_t *rep_off = tile_base + E;
    int32_t *rep_slot = rep_off + E + 1;
    int32_t *rep_lo = rep_slot + P;
    int32_t *rep_hi = rep_lo + P;
    int32_t *slot_off = rep_hi + P;
    int32_t *rank_hist = slot_off + P;

    if (tid == 0) {
        s_ticket = atomicAdd(&g.ticket[layer], 1u);
        s_epoch = atomic_load_agent(&g.epoch[layer]) + 1u;
    }
    const int32_t *pl = g.placement + static_cast<int64_t>(layer) * g.lay.words;
    for (int i = tid; i < kWaves * E; i += kBlock) whist[i] = 0;
    for (int r = tid; r < R; r += kBlock) rank_hist[r] = 0;
    // The table is read as written by the planner, but every index is
    // clamped so that a corrupt block can only produce faults.
    for (int e = tid; e <= E; e += kBlock) {
        const int v = pl[g.lay.rep_off + e];
        rep_off[e] = v < 0 ? 0 : (v > P ? P : v);
    }
    for (int p = tid; p < P; p += kBlock) {
        const int q = pl[g.lay.rep_slot + p];
        rep_slot[p] = (q >= 0 && q < P) ? q : -1;
        slot_off[p] = pl[g.lay.slot_off + p];
    }
    __syncthreads();
    // capacity prefix of each replica within its expert
    for (int e = tid; e < E; e += kBlock) {
        int run = 0;
        const int hi = rep_off[e + 1];
        for (int i = rep_off[e]; i < hi; ++i) {
            rep_lo[i] = run;
            const int cap = pl[g.lay.rep_cap + i];
            run += cap > 0 ? cap : 0;
            rep_hi[i] = run;
        }
    }
    __syncthreads();

    // Tickets run 0..tiles-1 within a launch; anything else means the
    // workspace counters were left inconsistent by an earlier failed launch.
    if (s_ticket >= static_cast<uint32_t>(g.tiles)) {
        if (tid == 0) atomicOr(&g.fault_acc[layer], 0x40000000);
        return;
    }
    const int tile = static_cast<int>(s_ticket);
    const uint32_t epoch = s_epoch;
    const int64_t base = static_cast<int64_t>(layer) * g.A;
    const int64_t a0 = static_cast<int64_t>(tile) * kRerouteTile +
                       static_cast<int64_t>(w) * 64 * kRerouteItems + lane;

    // ---- 1. per-wave stable ranks ----------------------------------------
    int32_t ids[kRerouteItems];
#pragma unroll
    for (int i = 0; i < kRerouteItems; ++i) {
        const int64_t a = a0 + 64 * i;
        ids[i] = (a < g.A) ? __builtin_nontemporal_load(g.routing + base + a)
                           : -1;
    }
    int32_t rank[kRerouteItems];
    int32_t *my_hist = whist + w * E;
#pragma unroll
    for (int i = 0; i < kRerouteItems; ++i) {
        const int id = ids[i];
        const bool valid = static_cast<uint32_t>(id) < static_cast<uint32_t>(E);
        uint64_t peers = __ballot(valid);
        for (int b = 0; b < g.ebits; ++b) {
            const bool bit = (id >> b) & 1;
            const uint64_t ones = __ballot(bit);
            peers &= bit ? ones : ~ones;
        }
        const uint32_t below = mask_rank(peers);
        int before = 0;
        if (valid) before = my_hist[id];
        if (valid && below == 0)
            my_hist[id] = before + __builtin_popcountll(peers);
        rank[i] = before + static_cast<int>(below);
    }
    __syncthreads();

    // ---- 2. scan the per-wave counts, publish the tile's counts ------------
    uint64_t *st = g.state +
                   (static_cast<int64_t>(layer) * g.max_tiles) * E;
    uint64_t *mine = st + static_cast<int64_t>(tile) * E;
    for (int e = tid; e < E; e += kBlock) {
        int run = 0;
#pragma unroll
        for (int v = 0; v < kWaves; ++v) {
            const int c = whist[v * E + e];
            whist[v * E + e] = run;
            run += c;
        }
        tile_base[e] = run;   // this tile's count until the lookback ends
        atomic_store_agent(mine + e,
                           pack_state(epoch, tile == 0 ? kFlagPrefix : kFlagAgg,
                                      static_cast<uint32_t>(run)));
    }
    // ---- 3. lookback over earlier tiles, one expert per thread -------------
    // Every tile before this one was taken by a workgroup that has started,
    // and each publishes all its counts before it waits on anything, so the
    // walk always ends at tile 0 at the latest. The wait is still bounded;
    // running out of patience is reported as a fault (bit 30 of the count).
    for (int e = tid; e < E; e += kBlock) {
        if (tile == 0) {
            tile_base[e] = 0;
            continue;
        }
        const int run = tile_base[e];
        uint32_t excl = 0;
        int t = tile - 1;
        uint32_t spins = 0;
        while (true) {
            const uint64_t v =
                atomic_load_agent(st + static_cast<int64_t>(t) * E + e);
            if (static_cast<uint32_t>(v >> 32) != epoch ||
                ((v >> 30) & 3u) == 0) {
                if (++spins > g.spin_limit) {
                    atomicOr(&g.fault_acc[layer], 0x40000000);
                    break;
                }
                __builtin_amdgcn_s_sleep(2);
                continue;
            }
            excl += static_cast<uint32_t>(v & 0x3FFFFFFFu);
            if (((v >> 30) & 3u) == kFlagPrefix || t == 0) break;
            --t;
        }
        atomic_store_agent(mine + e, pack_state(epoch, kFlagPrefix,
                                                excl + static_cast<uint32_t>(run)));
        tile_base[e] = static_cast<int32_t>(excl);
    }
    __syncthreads();

    // ---- 4. outputs ---------------------------------------------------------
    int nfault = 0;
#pragma unroll
    for (int i = 0; i < kRerouteItems; ++i) {
        const int64_t a = a0 + 64 * i;
        if (a >= g.A) continue;
        const int id = ids[i];
        int p = -1, pos = -1;
        if (static_cast<uint32_t>(id) < static_cast<uint32_t>(E)) {
            const int j = tile_base[id] + my_hist[id] + rank[i];
            for (int r = rep_off[id]; r < rep_off[id + 1]; ++r) {
                if (j < rep_hi[r]) {
                    if (j >= rep_lo[r] && rep_slot[r] >= 0) {
                        p = rep_slot[r];
                        pos = slot_off[p] + (j - rep_lo[r]);
                    }
                    break;
                }
            }
        }
        if (p >= 0 && pos >= 0 && pos < g.A) {
            __builtin_nontemporal_store(static_cast<int32_t>(a),
                                        g.perm + base + pos);
            atomicAdd(&rank_hist[p / g.NS], 1);
        } else {
            p = -1;
            pos = -1;
            ++nfault;
        }
        __builtin_nontemporal_store(p, g.phys + base + a);
        if (g.inv_perm) __builtin_nontemporal_store(pos, g.inv_perm + base + a);
    }
    int fault_total;
    block_exclusive_sum(nfault, wsum, fault_total);   // barrier: rank_hist
    for (int r = tid; r < R; r += kBlock) {
        const int c = rank_hist[r];
        if (c) atomicAdd(&g.rank_acc[static_cast<int64_t>(layer) * R + r], c);
    }
    if (tid == 0 && fault_total) atomicAdd(&g.fault_acc[layer], fault_total);
    __threadfence();
    __syncthreads();
    if (tid == 0) {
        const uint32_t prev = atomicAdd(&g.done[layer], 1u);
        s_last = (prev == static_cast<uint32_t>(g.tiles - 1));
    }
    __syncthreads();
    if (!s_last) return;
    __threadfence();
    for (int r = tid; r < R; r += kBlock)
        g.rank_counts[static_cast<int64_t>(layer) * R + r] =
            atomicExch(&g.rank_acc[static_cast<int64_t>(layer) * R + r], 0);
    if (tid == 0) {
        const int f = atomicExch(&g.fault_acc[layer], 0);
        if (g.faults) g.faults[layer] = f;
        atomic_store_agent(&g.ticket[layer], 0u);
        atomic_store_agent(&g.done[layer], 0u);
        atomic_store_agent(&g.epoch[layer], epoch);
    }
}

}  // namespace

size_t reroute_lds_bytes(int E, int R, int P) {
    return sizeof(int32_t) *
           (static_cast<size_t>(kWaves + 2) * E + 1 + 4 * P + R);
}

hipError_t launch_reroute(const ue_ctx &c, const int32_t *routing,
                          const int32_t *placement, int L, int64_t A,
                          int32_t *phys, int32_t *rank_counts, int32_t *perm,
                          int32_t *inv_perm, int32_t *faults, hipStream_t s) {
    int tiles = static_cast<int>((A + kRerouteTile - 1) / kRerouteTile);
    if (tiles < 1) tiles = 1;
    RerouteArgs g;
    g.routing = routing;
    g.placement = placement;
    g.A = A;
    g.E = c.E;
    g.R = c.R;
    g.NS = c.NS;
    g.P = c.P;
    g.ebits = c.ebits;
    g.tiles = tiles;
    g.max_tiles = c.max_rr_tiles;
    g.spin_limit = 1u << 22;
    g.lay = c.lay;
    g.phys = phys;
    g.perm = perm;
    g.inv_perm = inv_perm;
    g.state = c.scan_state;
    g.ticket = c.rr_ticket;
    g.done = c.rr_done;
    g.epoch = c.rr_epoch;
    g.rank_acc = c.rr_rank_acc;
    g.fault_acc = c.rr_fault_acc;
    g.rank_counts = rank_counts;
    g.faults = faults;
    hipLaunchKernelGGL(k_reroute, dim3(tiles, L), dim3(kBlock), c.reroute_lds,
                       s, g);
    return hipGetLastError();
}

}  // namespace ue
