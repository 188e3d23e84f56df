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
//   1. ranks its items within the tile. A token routes to distinct experts,
//      so the rank of item (token t, expert e) is the number of earlier
//      tokens of the tile that route to e: the tile builds one bitmap of
//      tokens per expert in LDS (one LDS OR per item), takes a prefix of
//      popcounts over each bitmap's words, and reads every rank back as
//      prefix + popcount of the bits below the token. A token that names
//      the same expert twice is seen when its second OR finds the bit set;
//      such a tile (and any configuration whose bitmaps do not fit) ranks by
//      matching lanes with equal ids instead: one ballot per id bit within
//      rounds of 64 consecutive items, and a per-wave counter per expert;
//   2. scans the tile counts across experts (the tile's own sorted order);
//   3. decoupled lookback over earlier tiles (ue_internal.h) gives the count
//      of each expert before this tile; when the load kernel has just
//      counted the same routing with the same tiles, the prefix it published
//      for the previous tile is read instead (no ticket, no waiting);
//   4. j = tile prefix + rank; the replica is found through a per-expert
//      fast path (the replica covering the tile's first assignment of e and
//      how many of the tile's assignments it still takes) or, for items that
//      cross into a later replica, a scan of the expert's capacity prefixes;
//      phys and inv_perm are written straight out (coalesced); perm entries
//      are placed in LDS in the tile's (expert, j) order, where neighbours
//      have consecutive dispatch positions, and written out in that order so
//      that stores land in contiguous runs;
//   5. the tile with the last ticket knows every expert's total; per-rank
//      counts are the overlaps of [0, total) with the replicas' capacity
//      intervals, and faults are the ids out of range plus the assignments
//      beyond an expert's capacity or outside [0, T*k).
// No fences and no global atomics on data.
#include <algorithm>

#include "ue_internal.h"

namespace ue {
namespace {

struct RerouteArgs {
    const int32_t *routing;
    const int32_t *placement;
    int64_t A;                 // assignments per layer
    int E, R, NS, P, k, ebits, tiles, max_tiles;
    int bm_words;              // words per expert bitmap (0: no bitmap path)
    uint32_t spin_limit;       // bound on one lookback wait
    uint32_t lds_bytes;        // dynamic LDS the launch provides
    ue_placement_layout lay;
    int32_t *phys, *perm, *inv_perm;
    uint64_t *state;           // [max_layers][max_tiles][E] own lookback
    uint64_t *tick;            // [max_layers] own ticket and epoch
    const int32_t *tile_prefix;// [max_layers][max_tiles][E] from the load
    int32_t *rank_counts, *faults;
};

// Bitmap path: bits of expert e live in words [e*Wp, e*Wp + W), with an odd
// stride Wp so that neighbouring experts fall in other banks.
__host__ __device__ __forceinline__ int bm_stride(int W) { return W | 1; }

// Largest region A (ints) the bitmap path may take; beyond it, the
// configuration ranks by matching.
constexpr int kBitmapBudget = 12288;

// Size in ints of region A, shared in turn by the rank bitmaps and their
// word prefixes (or the per-wave counters of the matching path) and by the
// staged perm entries.
__host__ __device__ __forceinline__ int region_a_ints(int E, int W) {
    int a = 2 * E * bm_stride(W);
    a = a > kWaves * E ? a : kWaves * E;
    return a > 2 * kRerouteTile ? a : 2 * kRerouteTile;
}

// kAfterLoad: the count of each expert in earlier tiles is the per-tile
// prefix the load kernel just wrote, tiles do not depend on each other and
// workgroup blockIdx.x takes tile blockIdx.x. Otherwise the workgroup takes
// one tile by ticket and finds the prefix by lookback.
template <bool kAfterLoad>
__global__ __launch_bounds__(kBlock) void k_reroute(RerouteArgs g) {
    extern __shared__ int32_t lds[];
    __shared__ int wsum[kWaves];
    __shared__ uint32_t s_ticket, s_epoch;

    const int E = g.E, P = g.P, R = g.R;
    const int layer = blockIdx.y;
    const int tid = threadIdx.x;
    const int w = tid >> 6;
    const int lane = tid & 63;
    const int W = g.bm_words;
    const int Wp = bm_stride(W);

    int32_t *area = lds;
    int32_t *tcount = area + region_a_ints(E, W);
    int32_t *torder = tcount + E;
    int32_t *tbase = torder + E;
    int32_t *fslot = tbase + E;
    int32_t *flim = fslot + E;
    int32_t *fpos = flim + E;
    int32_t *rep_off = fpos + E;
    int32_t *rep_slot = rep_off + E + 1;
    int32_t *rep_lo = rep_slot + P;
    int32_t *rep_hi = rep_lo + P;
    int32_t *slot_off = rep_hi + P;
    int32_t *rank_hist = slot_off + P;
    // the carve-up must fit the launch's LDS (checked, not assumed)
    if (static_cast<size_t>(rank_hist + R - lds) * 4 > g.lds_bytes) return;

    if (kAfterLoad) {
        if (tid == 0) {
            s_ticket = blockIdx.x;
            s_epoch = 0;
        }
    } else if (tid == 0) {
        take_ticket(g.tick + layer, g.tiles, s_ticket, s_epoch);
    }
    const int32_t *pl = g.placement + static_cast<int64_t>(layer) * g.lay.words;
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
        const int cap = pl[g.lay.rep_cap + p];
        rep_hi[p] = cap > 0 ? cap : 0;     // capacity, until the prefix below
    }
    const bool bitmap = W > 0;
    int32_t *bm = area;                    // [E][Wp] token bitmaps
    int32_t *bpre = area + E * Wp;         // [E][Wp] popcount prefixes
    __syncthreads();
    if (static_cast<int>(s_ticket) >= g.tiles)
        return;    // only after a corrupted earlier launch
    // capacity prefix of each replica within its expert, from LDS
    for (int e = tid; e < E; e += kBlock) {
        int run = 0;
        const int hi = rep_off[e + 1];
        for (int i = rep_off[e]; i < hi; ++i) {
            rep_lo[i] = run;
            run += rep_hi[i];
            rep_hi[i] = run;
        }
    }
    const uint32_t epoch = s_epoch;
    const int tile = static_cast<int>(s_ticket);
    const int64_t base = static_cast<int64_t>(layer) * g.A;
    const int64_t tile0 = static_cast<int64_t>(tile) * kRerouteTile;
    const int64_t a0 = tile0 + static_cast<int64_t>(w) * 64 * kRerouteItems +
                       lane;

    // global reads first: the tile's ids and, after a load, its prefixes
    int32_t ids[kRerouteItems];
#pragma unroll
    for (int i = 0; i < kRerouteItems; ++i) {
        const int64_t a = a0 + 64 * i;
        ids[i] = (a < g.A) ? __builtin_nontemporal_load(g.routing + base + a)
                           : -1;
    }
    constexpr int kPerThread = kMaxExperts / kBlock;
    int32_t pre_reg[kPerThread];
    if (kAfterLoad) {
        const int32_t *tp = g.tile_prefix +
                            (static_cast<int64_t>(layer) * g.max_tiles + tile) * E;
#pragma unroll
        for (int q = 0; q < kPerThread; ++q) {
            const int e = tid + q * kBlock;
            pre_reg[q] = e < E ? tp[e] : 0;
        }
    }
    if (bitmap)
        for (int i = tid; i < E * Wp; i += kBlock) bm[i] = 0;
#pragma unroll
    for (int i = 0; i < kRerouteItems; ++i)
        ids[i] = static_cast<uint32_t>(ids[i]) < static_cast<uint32_t>(E) ? ids[i]
                                                                          : -1;
    __syncthreads();

    // ---- 1. ranks within the tile ------------------------------------------
    int32_t rank[kRerouteItems];
    int dup = 0;
    if (bitmap) {
        // token of item a0 + 64 i relative to the tile's first token,
        // stepped without a division per item
        const int k = g.k;
        const int t_first = static_cast<int>(tile0 / k);
        int tl = static_cast<int>(a0 / k) - t_first;
        int rm = static_cast<int>(a0 % k);
        const int q64 = 64 / k, r64 = 64 % k;
#pragma unroll
        for (int i = 0; i < kRerouteItems; ++i) {
            const int id = ids[i];
            rank[i] = tl;                  // the token, until the read-back
            if (id >= 0) {
                const uint32_t bit = 1u << (tl & 31);
                const uint32_t old = atomicOr(
                    reinterpret_cast<uint32_t *>(&bm[id * Wp + (tl >> 5)]), bit);
                dup |= (old & bit) != 0;
            }
            tl += q64;
            rm += r64;
            if (rm >= k) {
                rm -= k;
                ++tl;
            }
        }
    }
    const int use_match = !bitmap || __syncthreads_or(dup);
    if (!use_match) {
        // prefix of popcounts over each expert's words; tile counts
        for (int e = tid; e < E; e += kBlock) {
            int run = 0;
            for (int i = 0; i < W; ++i) {
                bpre[e * Wp + i] = run;
                run += __builtin_popcount(static_cast<uint32_t>(bm[e * Wp + i]));
            }
            tcount[e] = run;
            torder[e] = run;
        }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < kRerouteItems; ++i) {
            const int id = ids[i];
            const int tl = rank[i];
            if (id >= 0) {
                const int word = id * Wp + (tl >> 5);
                const uint32_t below = (1u << (tl & 31)) - 1u;
                rank[i] = bpre[word] + __builtin_popcount(
                                           static_cast<uint32_t>(bm[word]) & below);
            }
        }
    } else {
        // matching path: ranks within rounds of 64 consecutive items
        int32_t *whist = area;              // [kWaves][E]
        __syncthreads();
        for (int i = tid; i < kWaves * E; i += kBlock) whist[i] = 0;
        __syncthreads();
        int32_t *my_hist = whist + w * E;
        // rank[i] packs the leader's count before the round (13 bits, a
        // tile holds at most 4096 items), the rank below (6 bits) and the
        // leader lane (6 bits) until the leaders' counts are fetched
#pragma unroll
        for (int i = 0; i < kRerouteItems; ++i) {
            const int id = ids[i];
            const bool valid = id >= 0;
            const uint64_t peers = match_peers(id, valid, g.ebits);
            const uint32_t below = mask_rank(peers);
            int old = 0;
            if (valid && below == 0)
                old = atomicAdd(&my_hist[id], __builtin_popcountll(peers));
            const int leader = peers ? __builtin_ctzll(peers) : lane;
            rank[i] = (old & 0x1FFF) | static_cast<int>(below << 13) |
                      (leader << 19);
        }
#pragma unroll
        for (int i = 0; i < kRerouteItems; ++i) {
            const int pk = rank[i];
            const int before = __shfl(pk, (pk >> 19) & 63, 64) & 0x1FFF;
            rank[i] = before + ((pk >> 13) & 63);
        }
        __syncthreads();
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
#pragma unroll
        for (int i = 0; i < kRerouteItems; ++i)
            if (ids[i] >= 0) rank[i] += my_hist[ids[i]];
    }

    // ---- 2. the tile's own (expert, j) order --------------------------------
    __syncthreads();
    {
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

    // ---- 3. count of each expert in earlier tiles ---------------------------
    bool bad = false;
    if (kAfterLoad) {
#pragma unroll
        for (int q = 0; q < kPerThread; ++q) {
            const int e = tid + q * kBlock;
            if (e < E) tbase[e] = pre_reg[q];
        }
    } else {
        uint64_t *st = g.state + static_cast<int64_t>(layer) * g.max_tiles * E;
        bad = tile_lookback(st, tile, E, epoch, tcount, tbase, g.spin_limit);
    }
    const int poisoned = __syncthreads_or(bad);

    // ---- 4. outputs ---------------------------------------------------------
    // Per expert: the replica covering the tile's first assignment j0, the
    // dispatch position of j0 and how many of the tile's assignments stay in
    // that replica.
    for (int e = tid; e < E; e += kBlock) {
        const int j0 = tbase[e];
        int q = -1, lim = 0, pos0 = 0;
        for (int r = rep_off[e]; r < rep_off[e + 1]; ++r) {
            if (j0 < rep_hi[r]) {
                if (j0 >= rep_lo[r] && rep_slot[r] >= 0) {
                    q = rep_slot[r];
                    lim = rep_hi[r] - j0;
                    pos0 = slot_off[q] + (j0 - rep_lo[r]);
                }
                break;
            }
        }
        fslot[e] = q;
        flim[e] = q >= 0 ? lim : 0;
        fpos[e] = pos0;
    }
    __syncthreads();
    int32_t *stage_a = area;
    int32_t *stage_pos = area + kRerouteTile;
    // partly unrolled: fully unrolled, the sixteen items' addresses and
    // stores keep too many registers live and halve the waves per SIMD
#pragma unroll 4
    for (int i = 0; i < kRerouteItems; ++i) {
        const int64_t a = a0 + 64 * i;
        if (a >= g.A) continue;
        const int id = ids[i];
        int p = -1, pos = -1;
        if (id >= 0) {
            const int jt = rank[i];                    // j within the tile
            const int s = torder[id] + jt;             // tile (expert, j) order
            if (jt < flim[id]) {
                p = fslot[id];
                pos = fpos[id] + jt;
            } else {
                const int j = tbase[id] + jt;
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
            if (p < 0 || pos < 0 || pos >= g.A) {
                p = -1;
                pos = -1;
            }
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
    if (tile == g.tiles - 1) {
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
            const int64_t lo_ok = first < 0 ? -first : 0;
            const int64_t hi_ok = g.A - first < n ? g.A - first : n;
            const int in_range =
                hi_ok > lo_ok ? static_cast<int>(hi_ok - lo_ok) : 0;
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
}

// Largest number of tokens that kRerouteTile consecutive assignments touch.
int tile_tokens(int k) { return (kRerouteTile - 1) / k + 2; }

}  // namespace

int reroute_bitmap_words(int E, int k) {
    const int W = (tile_tokens(k) + 31) / 32;
    // the bitmaps and their prefixes share region A with the staged perm
    return 2 * E * bm_stride(W) <= kBitmapBudget ? W : 0;
}

size_t reroute_lds_bytes(int E, int R, int P, int k) {
    const int W = reroute_bitmap_words(E, k);
    // region A; tcount, torder, tbase, fslot, flim, fpos; rep_off (+1);
    // four P-sized tables; the rank histogram
    return sizeof(int32_t) * (static_cast<size_t>(region_a_ints(E, W)) +
                              static_cast<size_t>(7) * E + 1 + 4 * P + R);
}

hipError_t reroute_prepare(size_t lds_bytes) {
    hipError_t e = hipFuncSetAttribute(
        reinterpret_cast<const void *>(&k_reroute<false>),
        hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds_bytes));
    if (e != hipSuccess) return e;
    return hipFuncSetAttribute(reinterpret_cast<const void *>(&k_reroute<true>),
                               hipFuncAttributeMaxDynamicSharedMemorySize,
                               static_cast<int>(lds_bytes));
}

static hipError_t launch(const ue_ctx &c, bool after_load,
                         const int32_t *routing, const int32_t *placement,
                         int L, int64_t A, int32_t *phys,
                         int32_t *rank_counts, int32_t *perm,
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
    g.k = c.k;
    g.ebits = c.ebits;
    g.tiles = tiles;
    g.max_tiles = c.max_rr_tiles;
    g.bm_words = reroute_bitmap_words(c.E, c.k);
    g.spin_limit = 1u << 22;
    g.lds_bytes = static_cast<uint32_t>(c.reroute_lds);
    g.lay = c.lay;
    g.phys = phys;
    g.perm = perm;
    g.inv_perm = inv_perm;
    g.state = c.scan_state;
    g.tick = c.rr_tick;
    g.tile_prefix = c.tile_prefix;
    g.rank_counts = rank_counts;
    g.faults = faults;
    if (after_load) {
        // one tile per workgroup: the hardware then overlaps one tile's
        // tail with the next tile's loads on the same CU, which a
        // persistent workgroup looping over tiles cannot
        hipLaunchKernelGGL(k_reroute<true>, dim3(tiles, L), dim3(kBlock),
                           c.reroute_lds, s, g);
    }
    else
        hipLaunchKernelGGL(k_reroute<false>, dim3(tiles, L), dim3(kBlock),
                           c.reroute_lds, s, g);
    return hipGetLastError();
}

hipError_t launch_reroute(const ue_ctx &c, const int32_t *routing,
                          const int32_t *placement, int L, int64_t A,
                          int32_t *phys, int32_t *rank_counts, int32_t *perm,
                          int32_t *inv_perm, int32_t *faults, hipStream_t s) {
    return launch(c, false, routing, placement, L, A, phys, rank_counts, perm,
                  inv_perm, faults, s);
}

hipError_t launch_reroute_after_load(const ue_ctx &c, const int32_t *routing,
                                     const int32_t *placement, int L,
                                     int64_t A, int32_t *phys,
                                     int32_t *rank_counts, int32_t *perm,
                                     int32_t *inv_perm, int32_t *faults,
                                     hipStream_t s) {
    return launch(c, true, routing, placement, L, A, phys, rank_counts, perm,
                  inv_perm, faults, s);
}

}  // namespace ue
