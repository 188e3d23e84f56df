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
#include <type_traits>

#include "ue_internal.h"

namespace ue {
namespace {

struct RerouteArgs {
    const int32_t *routing;
    const int32_t *placement;
    int32_t A;                 // assignments per layer (< 2^30)
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

// Element i of a per-layer array, with the byte offset formed in 32 bits
// (every offset here is below 2^32 since T*k < 2^30): the address is then
// a uniform 64-bit base plus one 32-bit register.
template <typename T>
__device__ __forceinline__ T *at(T *p, int i) {
    using B = typename std::conditional<std::is_const<T>::value, const char,
                                        char>::type;
    return reinterpret_cast<T *>(reinterpret_cast<B *>(p) +
                                 static_cast<uint32_t>(i) * sizeof(T));
}

// Bitmap path: expert e's token bitmap is words [e*Wp, e*Wp + W) of an
// array of int2 {bits, popcount prefix}, with an odd stride Wp so that
// neighbouring experts fall in other banks; one 8-byte read gives an item
// both the word and the count of the bits before it.
__host__ __device__ __forceinline__ int bm_stride(int W) { return W | 1; }

// Largest region A (ints) the bitmap path may take; beyond it, the
// configuration ranks by matching.
constexpr int kBitmapBudget = 12288;

// Size in ints of region A, shared in turn by the rank bitmaps (or the
// per-wave counters of the matching path) and by the staged perm entries
// (plus one dummy entry per thread); a multiple of 4 so that what follows
// stays 16-byte aligned.
static_assert(kRerouteTile <= 4096, "matching ranks are packed in 13 bits");

__host__ __device__ __forceinline__ int region_a_ints(int E, int W) {
    int a = 2 * E * bm_stride(W);
    a = a > kWaves * E ? a : kWaves * E;
    a = a > 2 * (kRerouteTile + kBlock) ? a : 2 * (kRerouteTile + kBlock);
    return (a + 3) & ~3;
}

// kAfterLoad: the count of each expert in earlier tiles is the per-tile
// prefix the load kernel just wrote, tiles do not depend on each other and
// workgroup blockIdx.x takes tile blockIdx.x. Otherwise the workgroup takes
// one tile by ticket and finds the prefix by lookback. (A persistent grid
// that loads the replica table once and loops over tiles measured no
// faster: the hardware already overlaps one workgroup's table reads with
// others' work.)
template <bool kAfterLoad>
__global__ __launch_bounds__(kBlock) void k_reroute(RerouteArgs g) {
    extern __shared__ __align__(16) int32_t lds[];
    __shared__ int wsum[kWaves];
    __shared__ uint32_t s_ticket, s_epoch;

    const int E = g.E, P = g.P, R = g.R;
    // after a load: launch order -> (layer, tile), contiguous per XCD, so
    // that a tile's perm runs and its neighbour's share one L2
    const int item = kAfterLoad
        ? xcd_order(blockIdx.y * gridDim.x + blockIdx.x, gridDim.x * gridDim.y)
        : 0;
    const int layer = kAfterLoad ? item / static_cast<int>(gridDim.x)
                                 : static_cast<int>(blockIdx.y);
    const int tid = threadIdx.x;
    const int w = tid >> 6;
    const int lane = tid & 63;
    const int W = g.bm_words;
    const int Wp = bm_stride(W);

    int32_t *area = lds;
    int4 *einfo = reinterpret_cast<int4 *>(area + region_a_ints(E, W));
    int32_t *tcount = reinterpret_cast<int32_t *>(einfo + E);
    int32_t *torder = tcount + E;
    int32_t *tbase = torder + E;
    int32_t *rep_off = tbase + E;
    int32_t *rep_slot = rep_off + E + 1;
    int32_t *rep_lo = rep_slot + P;
    int32_t *rep_hi = rep_lo + P;
    int32_t *slot_off = rep_hi + P;
    int32_t *rank_hist = slot_off + P;
    // the carve-up must fit the launch's LDS (checked, not assumed); a
    // mismatch poisons the layer's fault count rather than pass silently
    if (static_cast<size_t>(rank_hist + R - lds) * 4 > g.lds_bytes) {
        if (tid == 0 && blockIdx.x == 0 && g.faults) g.faults[layer] = kPoisonBit;
        return;
    }

    // per-layer bases, uniform across the workgroup; items are then
    // addressed by 32-bit offsets (A < 2^30)
    const int64_t base = static_cast<int64_t>(layer) * g.A;
    const int32_t *__restrict__ routing_l = g.routing + base;
    int32_t *__restrict__ phys_l = g.phys + base;
    int32_t *__restrict__ perm_l = g.perm + base;
    int32_t *__restrict__ inv_l = g.inv_perm ? g.inv_perm + base : nullptr;
    const int A = g.A;
    constexpr int kPerThread = kMaxExperts / kBlock;
    int32_t ids[kRerouteItems];
    int32_t pre_reg[kPerThread];
    int tile = 0;
    int tile0 = 0, a0 = 0;
    // the tile's ids (and, after a load, its prefixes): issued first so
    // that their latency overlaps the placement table reads
    // (a full tile loads unconditionally at immediate offsets; the ragged
    // last tile clamps its reads into the layer and drops what lies beyond)
    auto load_ids = [&](int t, int32_t *dst) {
        const int first = t * kRerouteTile + w * 64 * kRerouteItems + lane;
        if ((t + 1) * kRerouteTile <= A) {
            const int32_t *src = at(routing_l, first);
#pragma unroll
            for (int i = 0; i < kRerouteItems; ++i)
                dst[i] = __builtin_nontemporal_load(src + 64 * i);
        } else {
#pragma unroll
            for (int i = 0; i < kRerouteItems; ++i) {
                const int a = first + 64 * i;
                const int v = A > 0 ? __builtin_nontemporal_load(
                                          at(routing_l, a < A ? a : A - 1))
                                    : -1;
                dst[i] = a < A ? v : -1;
            }
        }
    };
    auto load_prefix = [&](int t, int32_t *dst) {
        const int32_t *tp = g.tile_prefix +
                            (static_cast<int64_t>(layer) * g.max_tiles + t) * E;
#pragma unroll
        for (int q = 0; q < kPerThread; ++q) {
            const int e = tid + q * kBlock;
            dst[q] = e < E ? tp[e] : 0;
        }
    };
    if (kAfterLoad) {
        tile = item % static_cast<int>(gridDim.x);
        if (tile >= g.tiles) return;
        load_ids(tile, ids);
        load_prefix(tile, pre_reg);
        if (tid == 0) s_epoch = 0;
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
    int2 *bm = reinterpret_cast<int2 *>(area);   // [E][Wp] {bits, prefix}
    if (bitmap)
        for (int i = tid; i < E * Wp; i += kBlock) bm[i] = int2{0, 0};
    __syncthreads();
    if (!kAfterLoad) {
        tile = static_cast<int>(s_ticket);
        if (tile >= g.tiles) return;   // only after a corrupted earlier launch
        load_ids(tile, ids);
    }
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
    tile0 = tile * kRerouteTile;
    a0 = tile0 + w * 64 * kRerouteItems + lane;
#pragma unroll
    for (int i = 0; i < kRerouteItems; ++i)
        ids[i] = static_cast<uint32_t>(ids[i]) < static_cast<uint32_t>(E) ? ids[i]
                                                                          : -1;

    // ---- 1. ranks within the tile ------------------------------------------
    int32_t rank[kRerouteItems];
    int dup = 0;
    if (bitmap) {
        // token of item a0 + 64 i relative to the tile's first token,
        // stepped without a division per item
        const int k = g.k;
        const uint32_t uk = static_cast<uint32_t>(k);
        const int t_first = static_cast<int>(static_cast<uint32_t>(tile0) / uk);
        const uint32_t qa = static_cast<uint32_t>(a0) / uk;
        int tl = static_cast<int>(qa) - t_first;
        int rm = static_cast<int>(static_cast<uint32_t>(a0) - qa * uk);
        const int q64 = 64 / k, r64 = 64 % k;
        // Branch-free: an id out of range ORs nothing into expert 0's
        // word, so every lane issues the same instructions.
#pragma unroll
        for (int i = 0; i < kRerouteItems; ++i) {
            const int id = ids[i];
            rank[i] = tl;                  // the token, until the read-back
            const uint32_t bit = id >= 0 ? 1u << (tl & 31) : 0u;
            const uint32_t old = atomicOr(
                reinterpret_cast<uint32_t *>(area) +
                    2 * ((id >= 0 ? id : 0) * Wp + (tl >> 5)),
                bit);
            dup |= (old & bit) != 0;
            rm += r64;
            const int carry = rm >= k;
            rm -= carry ? k : 0;
            tl += q64 + carry;
        }
    }
    const int use_match = !bitmap || __syncthreads_or(dup);
    if (!use_match) {
        // prefix of popcounts over each expert's words (read in batches so
        // the reads overlap); tile counts
        for (int e = tid; e < E; e += kBlock) {
            int2 *row = bm + e * Wp;
            int run = 0;
            for (int i0 = 0; i0 < W; i0 += 8) {
                uint32_t bits[8];
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    bits[j] = i0 + j < W ? static_cast<uint32_t>(row[i0 + j].x) : 0u;
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    if (i0 + j < W) row[i0 + j].y = run;
                    run += __builtin_popcount(bits[j]);
                }
            }
            tcount[e] = run;
            torder[e] = run;
        }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < kRerouteItems; ++i) {
            const int id = ids[i];
            const int tl = rank[i];
            const int2 v = bm[(id >= 0 ? id : 0) * Wp + (tl >> 5)];
            const uint32_t below = (1u << (tl & 31)) - 1u;
            rank[i] = v.y + __builtin_popcount(static_cast<uint32_t>(v.x) & below);
        }
    } else {
        // matching path: ranks within rounds of 64 consecutive items
        int32_t *whist = area;              // [kWaves][E]
        __syncthreads();
        for (int i = tid; i < kWaves * E; i += kBlock) whist[i] = 0;
        __syncthreads();
        int32_t *my_hist = whist + w * E;
        // rank[i] packs the leader's count before the round (13 bits; a
        // tile holds kRerouteTile <= 4096 items), the rank below (6 bits)
        // and the leader lane (6 bits) until the leaders' counts are fetched
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
    // Per expert, in one 16-byte word: the tile's first position in its
    // (expert, j) order, how many of the tile's assignments stay in the
    // replica covering the tile's first j, that replica's slot and the
    // dispatch position of that first j.
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
        einfo[e] = int4{torder[e], q >= 0 ? lim : 0, q, pos0};
    }
    __syncthreads();
    // [tile] {a, pos} in (expert, j) order, then one dummy entry per thread
    // that items without a valid id write to, so the stores need no branch
    int2 *stage = reinterpret_cast<int2 *>(area);
    const bool full_tile = tile0 + kRerouteTile <= A;
    int32_t *phys_t = at(phys_l, a0);
    int32_t *inv_t = inv_l ? at(inv_l, a0) : nullptr;
    int p_out[kRerouteItems], pos_out[kRerouteItems], s_out[kRerouteItems];
    bool slow = false;
#pragma unroll
    for (int i = 0; i < kRerouteItems; ++i) {
        const int id = ids[i];
        const int4 f = einfo[id >= 0 ? id : 0];
        const int jt = rank[i];                        // j within the tile
        const bool fast = id >= 0 && jt < f.y;
        slow |= id >= 0 && !fast;
        p_out[i] = fast ? f.z : -1;
        pos_out[i] = fast ? f.w + jt : -1;
        s_out[i] = id >= 0 ? f.x + jt : kRerouteTile + tid;
    }
    // Items past the replica covering the tile's first j (or faults) walk
    // the expert's capacity prefixes; rare, so skipped per wave.
    if (__ballot(slow) != 0) {
#pragma unroll
        for (int i = 0; i < kRerouteItems; ++i) {
            const int id = ids[i];
            if (id < 0 || p_out[i] >= 0) continue;
            const int j = tbase[id] + rank[i];
            for (int r = rep_off[id]; r < rep_off[id + 1]; ++r) {
                if (j < rep_hi[r]) {
                    if (j >= rep_lo[r] && rep_slot[r] >= 0) {
                        p_out[i] = rep_slot[r];
                        pos_out[i] = slot_off[p_out[i]] + (j - rep_lo[r]);
                    }
                    break;
                }
            }
        }
    }
#pragma unroll
    for (int i = 0; i < kRerouteItems; ++i) {
        int p = p_out[i], pos = pos_out[i];
        const bool ok = p >= 0 && pos >= 0 && pos < A;
        p = ok ? p : -1;
        pos = ok ? pos : -1;
        stage[s_out[i]] = int2{a0 + 64 * i, pos};
        p_out[i] = p;
        pos_out[i] = pos;
    }
    if (full_tile) {
#pragma unroll
        for (int i = 0; i < kRerouteItems; ++i) {
            __builtin_nontemporal_store(p_out[i], phys_t + 64 * i);
            if (inv_t) __builtin_nontemporal_store(pos_out[i], inv_t + 64 * i);
        }
    } else {
#pragma unroll
        for (int i = 0; i < kRerouteItems; ++i) {
            if (a0 + 64 * i >= A) continue;
            __builtin_nontemporal_store(p_out[i], phys_t + 64 * i);
            if (inv_t) __builtin_nontemporal_store(pos_out[i], inv_t + 64 * i);
        }
    }
    __syncthreads();
    const int n_valid = torder[E - 1] + tcount[E - 1];
    for (int s = tid; s < n_valid; s += kBlock) {
        const int2 v = stage[s];
        if (v.y >= 0) *at(perm_l, v.y) = v.x;
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
    // region A; einfo (4 words per expert), tcount, torder, tbase;
    // rep_off (+1); four P-sized tables; the rank histogram
    return sizeof(int32_t) * (static_cast<size_t>(region_a_ints(E, W)) +
                              static_cast<size_t>(8) * E + 1 + 4 * P + R);
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
    g.A = static_cast<int32_t>(A);   // the context bounds T*k below 2^30
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
