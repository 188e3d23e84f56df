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
// same expert in the whole layer. Each workgroup takes a tile by ticket (so
// it only ever waits on tiles that have already started) and:
//   1. each wave ranks its ids in rounds of 64 consecutive assignments:
//      lanes with equal ids are found with one ballot per id bit, a lane's
//      rank among its peers is the popcount of peers below it, and a
//      per-wave LDS counter per expert carries the count across rounds;
//   2. per expert, the per-wave counts are scanned across the 4 waves, and
//      the tile counts across experts (the tile's own sorted order);
//   3. decoupled lookback over earlier tiles (ue_internal.h) gives the count
//      of each expert before this tile;
//   4. j = tile prefix + wave prefix + rank; the replica is found by a short
//      scan of the expert's capacity prefixes held in LDS; phys and inv_perm
//      are written straight out (coalesced); perm entries are first placed
//      in LDS in the tile's (expert, j) order, where neighbours have
//      consecutive dispatch positions, then written out in that order so
//      that stores land in contiguous runs;
//   5. the tile with the last ticket knows every expert's total; per-rank
//      counts are the overlaps of [0, total) with the replicas' capacity
//      intervals, and faults are the ids out of range plus the assignments
//      beyond an expert's capacity.
// No fences and no global atomics on data.
#include "ue_internal.h"

namespace ue {
namespace {

struct RerouteArgs {
    const int32_t *routing;
    const int32_t *placement;
    int64_t A;                 // assignments per layer
    int E, R, NS, P, ebits, tiles, max_tiles;
    uint32_t spin_limit;       // bound on one lookback wait
    uint32_t lds_bytes;        // dynamic LDS the launch provides
    ue_placement_layout lay;
    int32_t *phys, *perm, *inv_perm;
    uint64_t *state;           // [max_layers][max_tiles][E]
    uint32_t *ticket, *epoch;  // [max_layers]
    int32_t *rank_counts, *faults;
};

__global__ __launch_bounds__(kBlock) void k_reroute(RerouteArgs g) {
    extern __shared__ int32_t lds[];
    __shared__ int wsum[kWaves];
    __shared__ uint32_t s_ticket, s_epoch;

    const int E = g.E, P = g.P, R = g.R;
    const int layer = blockIdx.y;
    const int tid = threadIdx.x;
    const int w = tid >> 6;
    const int lane = tid & 63;

    // LDS: per-wave counters [kWaves][E] (then wave prefixes), tile counts
    // [E], tile order offsets [E], earlier-tile prefix [E], replica table
    // (rep_off [E+1], rep_slot [P], rep_lo [P], rep_hi [P]), slot_off [P],
    // rank histogram [R], staged perm (assignment, position) [2][tile].
    int32_t *whist = lds;
    int32_t *tcount = whist + kWaves * E;
    int32_t *torder = tcount + E;
    int32_t *tbase = torder + E;
    int32_t *rep_off = tbase + E;
    int32_t *rep_slot = rep_off + E + 1;
    int32_t *rep_lo = rep_slot + P;
    int32_t *rep_hi = rep_lo + P;
    int32_t *slot_off = rep_hi + P;
    int32_t *rank_hist = slot_off + P;
    int32_t *stage_a = rank_hist + R;
    int32_t *stage_pos = stage_a + kRerouteTile;
    // the carve-up must fit the launch's LDS (checked, not assumed)
    if (static_cast<size_t>(stage_pos + kRerouteTile - lds) * 4 > g.lds_bytes)
        return;

    if (tid == 0) take_ticket(g.ticket + layer, g.epoch + layer, g.tiles,
                              s_ticket, s_epoch);
    const int32_t *pl = g.placement + static_cast<int64_t>(layer) * g.lay.words;
    for (int i = tid; i < kWaves * E; i += kBlock) whist[i] = 0;
    for (int r = tid; r < R; r += kBlock) rank_hist[r] = 0;
    // The table is read as the planner wrote it, with every index clamped,
    // so a corrupt block can only produce faults.
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
    const int tile = static_cast<int>(s_ticket);
    if (tile >= g.tiles) return;    // only after a corrupted earlier launch
    const uint32_t epoch = s_epoch;
    const int64_t base = static_cast<int64_t>(layer) * g.A;
    const int64_t tile0 = static_cast<int64_t>(tile) * kRerouteTile;
    const int64_t a0 = tile0 + static_cast<int64_t>(w) * 64 * kRerouteItems +
                       lane;

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
        const uint64_t peers = match_peers(id, valid, g.ebits);
        const uint32_t below = mask_rank(peers);
        int before = 0;
        if (valid) before = my_hist[id];
        if (valid && below == 0)
            my_hist[id] = before + __builtin_popcountll(peers);
        rank[i] = before + static_cast<int>(below);
    }
    __syncthreads();

    // ---- 2. wave prefixes and tile counts per expert ------------------------
    for (int e = tid; e < E; e += kBlock) {
        int run = 0;
#pragma unroll
        for (int v = 0; v < kWaves; ++v) {
            const int c = whist[v * E + e];
            whist[v * E + e] = run;
            run += c;
        }
        tcount[e] = run;
        torder[e] = run;
    }
    __syncthreads();
    {
        // exclusive scan of the tile counts over experts (the tile order)
        const int per = (E + kBlock - 1) / kBlock;
        const int b = tid * per;
        const int eend = (b + per < E) ? b + per : E;
        int local = 0;
        for (int e = b; e < eend; ++e) local += torder[e];
        int total;
        int run = block_exclusive_sum(local, wsum, total);
        for (int e = b; e < eend; ++e) {
            const int c = torder[e];
            torder[e] = run;
            run += c;
        }
    }

    // ---- 3. lookback: count of each expert in earlier tiles -----------------
    uint64_t *st = g.state + static_cast<int64_t>(layer) * g.max_tiles * E;
    const bool bad = tile_lookback(st, tile, E, epoch, tcount, tbase,
                                   g.spin_limit);
    const int poisoned = __syncthreads_or(bad);

    // ---- 4. outputs ---------------------------------------------------------
#pragma unroll
    for (int i = 0; i < kRerouteItems; ++i) {
        const int64_t a = a0 + 64 * i;
        if (a >= g.A) continue;
        const int id = ids[i];
        int p = -1, pos = -1;
        if (static_cast<uint32_t>(id) < static_cast<uint32_t>(E)) {
            const int jt = my_hist[id] + rank[i];      // j within the tile
            const int j = tbase[id] + jt;
            for (int r = rep_off[id]; r < rep_off[id + 1]; ++r) {
                if (j < rep_hi[r]) {
                    if (j >= rep_lo[r] && rep_slot[r] >= 0) {
                        const int q = rep_slot[r];
                        const int at = slot_off[q] + (j - rep_lo[r]);
                        if (at >= 0 && at < g.A) {
                            p = q;
                            pos = at;
                        }
                    }
                    break;
                }
            }
            const int s = torder[id] + jt;             // tile (expert, j) order
            stage_a[s] = static_cast<int32_t>(a);
            stage_pos[s] = pos;
        }
        __builtin_nontemporal_store(p, g.phys + base + a);
        if (g.inv_perm) __builtin_nontemporal_store(pos, g.inv_perm + base + a);
    }
    __syncthreads();
    const int n_valid = torder[E - 1] + tcount[E - 1];
    for (int s = tid; s < n_valid; s += kBlock) {
        const int pos = stage_pos[s];
        if (pos >= 0) g.perm[base + pos] = stage_a[s];
    }

    // ---- 5. last tile: per-rank counts and faults ----------------------------
    if (tile != g.tiles - 1) return;
    // Assignments j in [lo, top) of a replica land at slot_off + (j - lo);
    // those whose position falls outside [0, A) (a plan made for other
    // counts) are faults like those beyond the expert's capacity.
    int part_valid = 0, part_over = 0;
    for (int e = tid; e < E; e += kBlock) {
        const int total = tbase[e] + tcount[e];
        part_valid += total;
        int placed = 0;
        for (int r = rep_off[e]; r < rep_off[e + 1]; ++r) {
            const int lo = rep_lo[r], hi = rep_hi[r];
            const int top = total < hi ? total : hi;
            if (top <= lo || rep_slot[r] < 0) continue;
            const int64_t first = slot_off[rep_slot[r]];
            const int64_t n = top - lo;
            int64_t lo_ok = first < 0 ? -first : 0;
            int64_t hi_ok = g.A - first < n ? g.A - first : n;
            const int in_range = hi_ok > lo_ok ? static_cast<int>(hi_ok - lo_ok) : 0;
            if (in_range) atomicAdd(&rank_hist[rep_slot[r] / g.NS], in_range);
            placed += in_range;
        }
        part_over += total - placed;
    }
    int tot_valid, tot_over;
    block_exclusive_sum(part_valid, wsum, tot_valid);
    block_exclusive_sum(part_over, wsum, tot_over);
    for (int r = tid; r < R; r += kBlock)
        g.rank_counts[static_cast<int64_t>(layer) * R + r] = rank_hist[r];
    if (tid == 0 && g.faults)
        g.faults[layer] = static_cast<int32_t>(g.A - tot_valid + tot_over) |
                          (poisoned ? kPoisonBit : 0);
}

}  // namespace

size_t reroute_lds_bytes(int E, int R, int P) {
    // whist, tcount, torder, tbase, rep_off (+1), four P-sized tables,
    // the rank histogram and the two staging arrays
    return sizeof(int32_t) * (static_cast<size_t>(kWaves + 4) * E + 1 + 4 * P +
                              R + 2 * kRerouteTile);
}

hipError_t reroute_prepare(size_t lds_bytes) {
    return hipFuncSetAttribute(reinterpret_cast<const void *>(&k_reroute),
                               hipFuncAttributeMaxDynamicSharedMemorySize,
                               static_cast<int>(lds_bytes));
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
    g.lds_bytes = static_cast<uint32_t>(c.reroute_lds);
    g.lay = c.lay;
    g.phys = phys;
    g.perm = perm;
    g.inv_perm = inv_perm;
    g.state = c.scan_state;
    g.ticket = c.rr_ticket;
    g.epoch = c.rr_epoch;
    g.rank_counts = rank_counts;
    g.faults = faults;
    hipLaunchKernelGGL(k_reroute, dim3(tiles, L), dim3(kBlock), c.reroute_lds,
                       s, g);
    return hipGetLastError();
}

}  // namespace ue
