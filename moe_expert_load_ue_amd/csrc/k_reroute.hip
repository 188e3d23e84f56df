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
//      the same expert twice is seen when its second OR finds the bit set
//      (after a load: when the popcounts fall short of the tile's count);
//      such a tile (and any configuration whose bitmaps do not fit) ranks by
//      matching lanes with equal ids instead: one ballot per id bit within
//      rounds of 64 consecutive items, and a per-wave counter per expert;
//   2. scans the tile counts across experts (the tile's own sorted order);
//   3. decoupled lookback over earlier tiles (ue_internal.h) gives the count
//      of each expert before this tile; when the load kernel has just
//      counted the same routing with the same tiles, the counts it published
//      (its group's base plus the tile's offset in the group) are read
//      instead (no ticket, no waiting);
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
//      beyond an expert's capacity or outside [0, T*k). (After a load the
//      plan was made from the same counts, so these follow from the plan:
//      the planner's launch writes them and no tile does this step.)
// No fences and no global atomics on data.
#include <algorithm>
#include <mutex>
#include <type_traits>

#include "ue_internal.h"

namespace ue {
namespace {

struct RerouteArgs {
    const int32_t *routing;
    const int32_t *placement;
    int32_t A;                 // assignments per layer (< 2^30)
    int E, R, NS, P, k, ebits, tiles, max_tiles;
    int load_groups;           // the load's groups (of kLoadGroup tiles)
    int bm_words;              // words per expert bitmap (0: no bitmap path)
    uint32_t spin_limit;       // bound on one lookback wait
    uint32_t lds_bytes;        // dynamic LDS the launch provides
    ue_placement_layout lay;
    int32_t *phys, *perm, *inv_perm;
    uint64_t *state;           // [max_layers][max_tiles][E] own lookback
    uint64_t *tick;            // [max_layers] own ticket and epoch
    const int32_t *group_base; // [L][load_groups][E] from the load
    const uint16_t *tile_off;  // [L][tiles + load_groups][E]
    int32_t *rank_counts, *faults;
};

// Element i of a per-layer array, with the byte offset formed in 32 bits
// (every offset here is below 2^32 since T*k < 2^30): the address is then
// a uniform 64-bit base plus one 32-bit register, which the loads and
// stores take as it is (a product formed in 64 bits would need a 64-bit
// add per access).
template <typename T>
__device__ __forceinline__ T *at(T *p, int i) {
    using B = typename std::conditional<std::is_const<T>::value, const char,
                                        char>::type;
    const uint32_t off = static_cast<uint32_t>(i) * static_cast<uint32_t>(sizeof(T));
    return reinterpret_cast<T *>(reinterpret_cast<B *>(p) + off);
}

// Largest number of tokens that kRerouteTile consecutive assignments touch.
// (a tile of whole tokens when k divides the tile size, since tiles start
// at multiples of it)
__host__ __device__ constexpr int tile_tokens(int k) {
    return kRerouteTile % k == 0 ? kRerouteTile / k
                                 : (kRerouteTile - 1) / k + 2;
}

// The common shape (top-8 routing, at most one expert per thread) has its
// own instance: k, the bitmap's words per expert and the per-expert loops
// are then constants, and the token arithmetic of every item folds.
constexpr int kFastK = 8;
constexpr int kFastWords = (tile_tokens(kFastK) + 31) / 32;

// Bitmap path: expert e's token bitmap is words [e*Wp, e*Wp + W), with an
// odd stride Wp so that neighbouring experts fall in other banks; the
// popcount prefix of each word follows in a second array: one byte per
// word (rows of W) when at most 8 words per expert keep every prefix below
// 256, else 16 bits per word at the words' own indices.
__host__ __device__ __forceinline__ int bm_stride(int W) { return W | 1; }
__host__ __device__ __forceinline__ bool bm_pre8(int W) { return W <= 8; }

// Ints of the bitmap region (words, then the prefixes).
__host__ __device__ __forceinline__ int bitmap_ints(int E, int W) {
    const int n = E * bm_stride(W);
    return n + (bm_pre8(W) ? (E * W + 3) / 4 : (n + 1) / 2);
}

// How many of the n consecutive dispatch positions from pos0 the fast path
// of an expert's record may take: the run stops before the first position
// outside [0, A) (only a plan made for other counts has such positions),
// so that every position the fast path gives is valid and the permutation
// pass needs no check for it; the rest go through the replica walk, which
// checks each one.
__device__ __forceinline__ int in_range_run(int pos0, int n, int A) {
    if (pos0 < 0) return 0;
    const int room = A - pos0;
    return n < room ? n : (room > 0 ? room : 0);
}

// Largest bitmap region (ints); beyond it, the configuration ranks by
// matching.
constexpr int kBitmapBudget = 9216;

// Staged perm entries: (assignment - tile start) | expert << 11, one per
// item in the tile's (expert, j) order, then one dummy per thread.
static_assert(kRerouteTile <= 2048, "staged entries keep 11 bits of position");
static_assert(kMaxExperts <= (1 << 20), "staged entries keep the expert above");

// Size in ints of region A, shared in turn by the rank bitmaps (or the
// per-wave counters of the matching path), the staged perm entries and, in
// the last tile, the per-rank histogram;
// a multiple of 4 so that what follows stays 16-byte aligned. The rest of
// the LDS (per-expert arrays and the replica table) follows it.
__host__ __device__ __forceinline__ int region_a_ints(int E, int W) {
    int a = W > 0 ? bitmap_ints(E, W) : 0;
    a = a > kWaves * E ? a : kWaves * E;
    a = a > kRerouteTile + kBlock ? a : kRerouteTile + kBlock;
    return (a + 3) & ~3;
}

// kAfterLoad: the count of each expert in earlier tiles is the per-tile
// prefix the load kernel just wrote, tiles do not depend on each other and
// workgroup blockIdx.x takes tile blockIdx.x. Otherwise the workgroup takes
// one tile by ticket and finds the prefix by lookback. (A persistent grid
// that loads the replica table once and loops over tiles measured no
// faster: the hardware already overlaps one workgroup's table reads with
// others' work, while the LDS per workgroup sets how many share a CU.)
// After a load the kernel is held to 8 waves per SIMD (at most 64 VGPRs;
// it uses 60, the top-8 instance 64), which it meets without spilling:
// left to itself the compiler took 68 and 7 waves, 5% slower at dsv3 size.
// The standalone instances would spill at 64 and are left free.
template <bool kAfterLoad, bool kFast>
__global__ __launch_bounds__(kBlock)
__attribute__((amdgpu_waves_per_eu(kAfterLoad ? 8 : 1, 8))) void k_reroute(RerouteArgs g) {
    extern __shared__ __align__(16) int32_t lds[];
    __shared__ int wsum[kWaves], wany[kWaves];
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
    const int W = kFast ? kFastWords : g.bm_words;
    const int Wp = bm_stride(W);

    int32_t *area = lds;
    // Per expert, in one 16-byte record: {the tile's own count, then its
    // first position in the tile's (expert, j) order : 16 | how many of the
    // tile's assignments stay in the replica covering the tile's first j,
    // at most a tile : 16; that replica's slot; the dispatch position of
    // that first j; the expert's assignments in earlier tiles (that j)}.
    int4 *einfo = reinterpret_cast<int4 *>(area + region_a_ints(E, W));
    uint16_t *ehalf = reinterpret_cast<uint16_t *>(einfo);   // [E][8]
    int32_t *rep_off = reinterpret_cast<int32_t *>(einfo + E);
    int32_t *rep_slot = rep_off + E + 1;
    int32_t *rep_hi = rep_slot + P;   // capacity prefix: end of each replica
    int32_t *slot_off = rep_hi + P;
    // the carve-up must fit the launch's LDS (checked, not assumed); a
    // mismatch poisons the layer's fault count rather than pass silently
    if (static_cast<size_t>(slot_off + P - lds) * 4 > g.lds_bytes) {
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
    constexpr int kPerThread = kFast ? 1 : kMaxExperts / kBlock;
    int32_t ids[kRerouteItems];
    int32_t pre_reg[kPerThread], cnt_reg[kPerThread];
    int tile = 0;
    // Item i of a lane is assignment aL + 64 i: each step of a wave covers
    // 64 consecutive assignments, so global reads and writes coalesce.
    // (Spreading a step's tokens 32 apart, to keep a hot expert's bitmap
    // ORs off one LDS word, measured slower: the accesses no longer
    // coalesce.)
    const int k = kFast ? kFastK : g.k;
    auto lane_base = [&](int t) {
        return t * kRerouteTile + w * 64 * kRerouteItems + lane;
    };
    int tile0 = 0, aL = 0;
    // the tile's ids (and, after a load, its prefixes): issued first so
    // that their latency overlaps the placement table reads
    // (a full tile loads unconditionally at immediate offsets; the ragged
    // last tile clamps its reads into the layer and drops what lies beyond;
    // plain loads, since after the load kernel the routing sits in the
    // device-wide cache)
    auto load_ids = [&](int t, int32_t *dst) {
        const int first = lane_base(t);
        if ((t + 1) * kRerouteTile <= A) {
            const int32_t *src = at(routing_l, first);
#pragma unroll
            for (int i = 0; i < kRerouteItems; ++i)
                dst[i] = src[64 * i];
        } else {
#pragma unroll
            for (int i = 0; i < kRerouteItems; ++i) {
                const int a = first + 64 * i;
                const int v = A > 0 ? *at(routing_l, a < A ? a : A - 1) : -1;
                dst[i] = a < A ? v : -1;
            }
        }
    };
    // tile t's count of each expert in all earlier tiles, and in t itself:
    // its group's base plus the tile's 16-bit offset in the group, and the
    // next row's offset (the next tile's, or the group's own count)
    auto load_prefix = [&](int t, int32_t *pre, int32_t *cnt) {
        const int grp = t / kLoadGroup;    // the load's split (load_shape)
        const int32_t *gb = g.group_base +
                            (static_cast<int64_t>(layer) * g.load_groups + grp) * E;
        const uint16_t *to = g.tile_off +
                             (static_cast<int64_t>(layer) * (g.tiles + g.load_groups) +
                              t + grp) * E;
#pragma unroll
        for (int q = 0; q < kPerThread; ++q) {
            const int e = tid + q * kBlock;
            const int b = e < E ? *at(gb, e) : 0;
            const int o0 = e < E ? *at(to, e) : 0;
            const int o1 = e < E ? *at(to, E + e) : 0;
            pre[q] = b + o0;
            cnt[q] = o1 - o0;
        }
    };
    const int32_t *pl = g.placement + static_cast<int64_t>(layer) * g.lay.words;
    // The table is read as the planner wrote it, with every index clamped,
    // so a corrupt block can only produce faults. Two rounds of both tables
    // at a time, every read of a round pair issued before the first write.
    // The first pair is read before the tile's ids and prefixes: loads
    // complete in order, so the table's writes then wait for the table
    // alone, and the ids arrive while the capacity prefixes are formed.
    // (The reads are unconditional, at indices clamped into each table,
    // and the writes drop what lies beyond: a conditional read lets the
    // compiler wait on it inside its own branch.)
    int vo[2], vq[2], vs[2], vc[2];
    auto table_read = [&](int i0) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int i = i0 + u * kBlock + tid;
            const int ie = i <= E ? i : E, ip = i < P ? i : P - 1;
            vo[u] = *at(pl, g.lay.rep_off + ie);
            vq[u] = *at(pl, g.lay.rep_slot + ip);
            vs[u] = *at(pl, g.lay.slot_off + ip);
            vc[u] = *at(pl, g.lay.rep_cap + ip);
        }
    };
    auto table_write = [&](int i0) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int i = i0 + u * kBlock + tid;
            if (i <= E) rep_off[i] = vo[u] < 0 ? 0 : (vo[u] > P ? P : vo[u]);
            if (i < P) {
                rep_slot[i] = (vq[u] >= 0 && vq[u] < P) ? vq[u] : -1;
                slot_off[i] = vs[u];
                rep_hi[i] = vc[u] > 0 ? vc[u] : 0;  // capacity, until the prefix below
            }
        }
    };
    table_read(0);
    if (kAfterLoad) {
        tile = item % static_cast<int>(gridDim.x);
        if (tile >= g.tiles) return;
        load_prefix(tile, pre_reg, cnt_reg);
        load_ids(tile, ids);
        if (tid == 0) s_epoch = 0;
    } else if (tid == 0) {
        take_ticket(g.tick + layer, g.tiles, s_ticket, s_epoch);
    }
    table_write(0);
    const int tab_n = E + 1 > P ? E + 1 : P;
    for (int i0 = 2 * kBlock; i0 < tab_n; i0 += 2 * kBlock) {
        table_read(i0);
        table_write(i0);
    }
    const bool bitmap = W > 0;
    // first word of expert e's bitmap: in the fast instance a 24-bit
    // multiply (e < 2^10, the stride a small constant), which issues at the
    // full rate where a 32-bit one takes four cycles (1 us off the 58-layer
    // dsv3 launch)
    auto bm_row = [](int e, int stride) {
        return kFast ? static_cast<int>(__umul24(static_cast<uint32_t>(e),
                                                 static_cast<uint32_t>(stride)))
                     : e * stride;
    };
    uint32_t *bm = reinterpret_cast<uint32_t *>(area);          // [E][Wp]
    const bool pre8 = bm_pre8(W);
    uint8_t *bpre8 = reinterpret_cast<uint8_t *>(area + E * Wp);    // [E][W]
    uint16_t *bpre16 = reinterpret_cast<uint16_t *>(area + E * Wp); // [E][Wp]
    if (bitmap) {
        // cleared 16 bytes at a time (the region starts 16-byte aligned):
        // a quarter of the LDS stores, and the compiler then holds 59 VGPRs
        // after a load instead of 64 (the launch 1.3 us faster at dsv3)
        const int nw = E * Wp, n4 = nw >> 2;
        uint4 *bm4 = reinterpret_cast<uint4 *>(bm);
        for (int i = tid; i < n4; i += kBlock) bm4[i] = uint4{0u, 0u, 0u, 0u};
        for (int i = 4 * n4 + tid; i < nw; i += kBlock) bm[i] = 0u;
    }
    __syncthreads();
    if (!kAfterLoad) {
        tile = static_cast<int>(s_ticket);
        if (tile >= g.tiles) return;   // only after a corrupted earlier launch
        load_ids(tile, ids);
    }
    // capacity prefix of each replica within its expert, from LDS; replica
    // r of expert e then covers j in [r == rep_off[e] ? 0 : rep_hi[r-1],
    // rep_hi[r]). The prefix saturates at A: every j is below A, so a
    // larger end covers the same j, and the prefix stays non-decreasing
    // (searchable by bisection) whatever the capacities. After a load the
    // tile's first j of each expert (its prefix) is already known, so the
    // same pass finds the replica that covers it: how many of the tile's
    // assignments it still takes, its slot and the dispatch position of
    // that first j (fields y, z, w of the expert's record; x, the tile's
    // own order, follows the scan).
#pragma unroll
    for (int q = 0; q < kPerThread; ++q) {
        const int e = tid + q * kBlock;
        if (e >= E) break;
        const int j0 = kAfterLoad ? pre_reg[q] : 0;
        int run = 0, lim = 0, slot = -1, pos0 = -1;
        bool found = false;
        const int hi = rep_off[e + 1];
        for (int i = rep_off[e]; i < hi; ++i) {
            const int lo = run;
            const int cap = rep_hi[i];
            run = cap < A - run ? run + cap : A;
            rep_hi[i] = run;
            if (kAfterLoad && !found && j0 < run) {
                found = true;
                const int sl = rep_slot[i];
                if (sl >= 0) {
                    slot = sl;
                    pos0 = slot_off[sl] + (j0 - lo);
                    lim = in_range_run(pos0, run - j0, A);
                }
            }
        }
        if (kAfterLoad)
            einfo[e] = int4{(lim < kRerouteTile ? lim : kRerouteTile) << 16,
                            slot, pos0, j0};
    }
    // Physical slot and dispatch position of assignment j of expert e, or
    // -1 for both if no replica covers j (only a plan made for other counts
    // leaves such assignments); end is set to the covering replica's
    // capacity prefix. The replica is the first of the expert's whose
    // prefix exceeds j, found by bisection: an expert split into many
    // pieces costs a few steps, not one per piece.
    auto locate = [&](int e, int j, int &p, int &pos, int &end) {
        p = -1;
        pos = -1;
        end = 0;
        const int first = rep_off[e], last = rep_off[e + 1];
        int lo = first, hi = last;
        while (lo < hi) {
            const int mid = (lo + hi) >> 1;
            if (rep_hi[mid] > j) hi = mid;
            else lo = mid + 1;
        }
        if (lo < last) {
            end = rep_hi[lo];
            if (rep_slot[lo] >= 0) {
                p = rep_slot[lo];
                pos = slot_off[p] + (j - (lo > first ? rep_hi[lo - 1] : 0));
            }
        }
    };
    const uint32_t epoch = s_epoch;
    tile0 = tile * kRerouteTile;
    aL = lane_base(tile);
#pragma unroll
    for (int i = 0; i < kRerouteItems; ++i)
        ids[i] = static_cast<uint32_t>(ids[i]) < static_cast<uint32_t>(E) ? ids[i]
                                                                          : -1;

    // ---- 1. ranks within the tile ------------------------------------------
    int32_t rank[kRerouteItems];
    int dup = 0;
    // the lane's first token in the tile; in the fast instance the token of
    // item i is tl_lane + i * 64 / k, found again at the read-back instead
    // of being held in rank[] across the popcount pass
    int tl_lane = 0;
    if (bitmap) {
        // token of item i relative to the tile's first token, stepped
        // without a division per item
        const uint32_t uk = static_cast<uint32_t>(k);
        const int t_first = static_cast<int>(static_cast<uint32_t>(tile0) / uk);
        const uint32_t qa = static_cast<uint32_t>(aL) / uk;
        int tl = static_cast<int>(qa) - t_first;
        int rm = static_cast<int>(static_cast<uint32_t>(aL) - qa * uk);
        const int q64 = 64 / k, r64 = 64 % k;
        tl_lane = tl;
        // Branch-free: an id out of range ORs nothing into expert 0's
        // word, so every lane issues the same instructions. After a load
        // the OR returns nothing (a repeated expert shows up below as a
        // popcount short of the load's count); otherwise the returned word
        // shows a bit already set.
#pragma unroll
        for (int i = 0; i < kRerouteItems; ++i) {
            const int id = ids[i];
            if (!kFast) rank[i] = tl;      // the token, until the read-back
            const uint32_t bit = id >= 0 ? 1u << (tl & 31) : 0u;
            uint32_t *word = bm + bm_row(id >= 0 ? id : 0, Wp) + (tl >> 5);
            if (kAfterLoad) {
                __hip_atomic_fetch_or(word, bit, __ATOMIC_RELAXED,
                                      __HIP_MEMORY_SCOPE_WORKGROUP);
            } else {
                const uint32_t old = atomicOr(word, bit);
                dup |= (old & bit) != 0;
            }
            rm += r64;
            const int carry = rm >= k;
            rm -= carry ? k : 0;
            tl += q64 + carry;
        }
    }
    if (kAfterLoad && bitmap) __syncthreads();
    int use_match = !bitmap || (!kAfterLoad && block_any(dup, wany));
    if (!use_match) {
        // prefix of popcounts over each expert's words (read in batches so
        // the reads overlap); tile counts, checked against the load's
        for (int q = 0; q < kPerThread; ++q) {
            const int e = tid + q * kBlock;
            if (e >= E) break;
            const uint32_t *row = bm + e * Wp;
            uint16_t *prow = bpre16 + e * Wp;
            uint8_t *prow8 = bpre8 + e * W;
            int run = 0;
            for (int i0 = 0; i0 < W; i0 += 8) {
                // eight words loaded unconditionally (four paired reads,
                // one wait), then the ones past the row masked: a
                // conditional load per word made the compiler wait on each
                // before the next. The over-read (at most 7 words past the
                // last expert's row, none at W = 8) stays in region A,
                // whose prefix arrays follow the words.
                uint32_t bits[8];
#pragma unroll
                for (int j = 0; j < 8; ++j) bits[j] = row[i0 + j];
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    if (i0 + j >= W) bits[j] = 0u;
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    if (i0 + j < W) {
                        if (pre8) prow8[i0 + j] = static_cast<uint8_t>(run);
                        else prow[i0 + j] = static_cast<uint16_t>(run);
                    }
                    run += __builtin_popcount(bits[j]);
                }
            }
            ehalf[8 * e] = static_cast<uint16_t>(run);
            if (kAfterLoad) dup |= run != cnt_reg[q];
        }
        if (kAfterLoad) use_match = block_any(dup, wany);
        else __syncthreads();
    }
    if (!use_match) {
        // (the fast instance forms each word's address again here: held
        // from the ORs across the popcount pass, the eight addresses
        // pushed it past 64 VGPRs; the empty asm hides that they equal
        // the ORs' addresses)
        if (kFast) {
#pragma unroll
            for (int i = 0; i < kRerouteItems; ++i) asm volatile("" : "+v"(ids[i]));
        }
#pragma unroll
        for (int i = 0; i < kRerouteItems; ++i) {
            const int id = ids[i];
            const int tl = kFast ? tl_lane + i * (64 / kFastK) : rank[i];
            const int e = id >= 0 ? id : 0;
            const int word = bm_row(e, Wp) + (tl >> 5);
            const uint32_t below = (1u << (tl & 31)) - 1u;
            const int pre = pre8 ? static_cast<int>(bpre8[e * W + (tl >> 5)])
                                 : static_cast<int>(bpre16[word]);
            rank[i] = pre + __builtin_popcount(bm[word] & below);
        }
    } else {
        // matching path: ranks within rounds of 64 consecutive items
        int32_t *whist = area;              // [kWaves][E]
        __syncthreads();
        for (int i = tid; i < kWaves * E; i += kBlock) whist[i] = 0;
        __syncthreads();
        int32_t *my_hist = whist + w * E;
        // rank[i] is the leader's count before the round (fetched from the
        // leader lane right after its add) plus the rank below
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
            rank[i] = __shfl(old, leader, 64) + static_cast<int>(below);
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
            ehalf[8 * e] = static_cast<uint16_t>(run);
        }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < kRerouteItems; ++i)
            if (ids[i] >= 0) rank[i] += my_hist[ids[i]];
    }

    // ---- 2. the tile's own (expert, j) order --------------------------------
    __syncthreads();
    // (the first field of each expert's record; the total is the number
    // of valid items in the tile)
    int n_valid;
    {
        const int per = kFast ? 1 : (E + kBlock - 1) / kBlock;   // experts per thread
        const int b = tid * per;
        const int eend = (b + per < E) ? b + per : E;
        int local = 0;
        for (int e = b; e < eend; ++e) local += ehalf[8 * e];
        int run = block_exclusive_sum(local, wsum, n_valid);
        for (int e = b; e < eend; ++e) {
            const int c = ehalf[8 * e];
            ehalf[8 * e] = static_cast<uint16_t>(run);
            run += c;
        }
    }
    // the tile's count of expert e, from the order's starts
    auto tile_count = [&](int e) {
        const int next = e + 1 < E ? static_cast<int>(ehalf[8 * (e + 1)]) : n_valid;
        return next - static_cast<int>(ehalf[8 * e]);
    };

    // ---- 3. count of each expert in earlier tiles ---------------------------
    // (after a load it came with the prefixes, and the expert records are
    // complete once the scan has written their first field)
    // (after a load nothing waited: the prefixes are the scan's)
    int poisoned = 0;
    if (kAfterLoad) {
        __syncthreads();
    } else {
        uint64_t *st = g.state + static_cast<int64_t>(layer) * g.max_tiles * E;
        __syncthreads();   // every start written
        const bool bad = tile_lookback(
            st, tile, E, epoch, tile_count,
            [&](int e, int v) { einfo[e].w = v; }, g.spin_limit);
        poisoned = block_any(bad, wany);
    }

    // ---- 4. outputs ---------------------------------------------------------
    // (after a load the expert records were completed with the prefixes)
    if (!kAfterLoad) {
        for (int e = tid; e < E; e += kBlock) {
            const int j0 = einfo[e].w;
            int q, pos0, end;
            locate(e, j0, q, pos0, end);
            const int lim = q >= 0 ? in_range_run(pos0, end - j0, A) : 0;
            ehalf[8 * e + 1] =
                static_cast<uint16_t>(lim < kRerouteTile ? lim : kRerouteTile);
            einfo[e].y = q;
            einfo[e].z = pos0;
        }
        __syncthreads();
    }
    uint32_t *stage = reinterpret_cast<uint32_t *>(area);
    const bool full_tile = tile0 + kRerouteTile <= A;
    int32_t *phys_t = at(phys_l, aL);
    int32_t *inv_t = inv_l ? at(inv_l, aL) : nullptr;
    // Each item is finished in turn (its outputs stored at once) so that
    // no per-item output array stays live across the tile. Items past the
    // replica covering the tile's first j (or faults) walk the expert's
    // capacity prefixes: rare, and skipped by every wave none of whose
    // lanes needs it. Whether the tile is full and whether inv_perm is
    // wanted are the same for every item, so the loop is instantiated for
    // each case (no per-item test of either; 1.5% off the launch).
    auto outputs = [&](auto full_c, auto inv_c) {
#pragma unroll
    for (int i = 0; i < kRerouteItems; ++i) {
        const int id = ids[i];
        const int4 f = einfo[id >= 0 ? id : 0];
        const int jt = rank[i];                        // j within the tile
        int p = -1, pos = -1;
        if (id >= 0) {
            if (jt < (f.x >> 16)) {
                p = f.y;
                pos = f.z + jt;
            } else {
                int end;
                locate(id, f.w + jt, p, pos, end);
            }
        }
        const bool ok = p >= 0 && pos >= 0 && pos < A;
        if (decltype(full_c)::value || aL + 64 * i < A) {
            __builtin_nontemporal_store(ok ? p : -1, phys_t + 64 * i);
            if (decltype(inv_c)::value) __builtin_nontemporal_store(ok ? pos : -1, inv_t + 64 * i);
        }
        stage[id >= 0 ? (f.x & 0xFFFF) + jt : kRerouteTile + tid] =
            static_cast<uint32_t>(64 * i + aL - tile0) |
            (static_cast<uint32_t>(id >= 0 ? id : 0) << 11);
    }
    };
    if (full_tile && inv_t) outputs(std::true_type{}, std::true_type{});
    else if (full_tile) outputs(std::true_type{}, std::false_type{});
    else if (inv_t) outputs(std::false_type{}, std::true_type{});
    else outputs(std::false_type{}, std::false_type{});
    __syncthreads();
    // perm in the tile's (expert, j) order: each entry's dispatch position
    // again from its expert's fast path (or the replica walk)
    // (kPermBatch entries per thread at a time, their LDS reads in flight
    // together: four were 2.5 us off the 58-layer dsv3 launch against one
    // at a time; the top-8 instance takes eight within its 64 VGPRs, and
    // with the scan below at one expert per thread the launch measured
    // 80.1 against 81.0-81.4 us; the general instance would spill at eight)
    constexpr int kPermBatch = kFast ? 8 : 4;
    for (int s0 = tid; s0 < n_valid; s0 += kPermBatch * kBlock) {
        uint32_t v[kPermBatch];
        int4 f[kPermBatch];
#pragma unroll
        for (int u = 0; u < kPermBatch; ++u) {
            const int s2 = s0 + u * kBlock;
            v[u] = s2 < n_valid ? stage[s2] : 0u;
        }
#pragma unroll
        for (int u = 0; u < kPermBatch; ++u) f[u] = einfo[v[u] >> 11];
#pragma unroll
        for (int u = 0; u < kPermBatch; ++u) {
            const int s2 = s0 + u * kBlock;
            if (s2 >= n_valid) break;
            const int e = static_cast<int>(v[u] >> 11);
            const int jt = s2 - (f[u].x & 0xFFFF);
            int p = f[u].y, pos = f[u].z + jt;
            bool ok = true;
            if (jt >= (f[u].x >> 16)) {
                int end;
                locate(e, f[u].w + jt, p, pos, end);
                ok = p >= 0 && pos >= 0 && pos < A;
            }
            if (ok) *at(perm_l, pos) = tile0 + static_cast<int>(v[u] & 2047u);
        }
    }

    // ---- 5. last tile: per-rank counts and faults ----------------------------
    // (after a load the planner's launch wrote them from the same counts)
    if (kAfterLoad || tile != g.tiles - 1) return;
    // the per-rank histogram takes region A once the staged entries are read
    __syncthreads();
    int32_t *rank_hist = area;
    for (int r = tid; r < R; r += kBlock) rank_hist[r] = 0;
    __syncthreads();
    // Assignments j in [lo, top) of a replica land at slot_off + (j - lo);
    // those whose position falls outside [0, A) (a plan made for other
    // counts) are faults like those beyond the expert's capacity.
    int part_valid = 0, part_over = 0;
    for (int e = tid; e < E; e += kBlock) {
        const int total = einfo[e].w + tile_count(e);
        part_valid += total;
        int placed = 0, lo = 0;
        for (int r = rep_off[e]; r < rep_off[e + 1]; ++r) {
            const int hi = rep_hi[r];
            const int top = total < hi ? total : hi;
            if (top > lo && rep_slot[r] >= 0) {
                const int64_t first = slot_off[rep_slot[r]];
                const int64_t n = top - lo;
                const int64_t lo_ok = first < 0 ? -first : 0;
                const int64_t hi_ok = g.A - first < n ? g.A - first : n;
                const int in_range =
                    hi_ok > lo_ok ? static_cast<int>(hi_ok - lo_ok) : 0;
                if (in_range) atomicAdd(&rank_hist[rep_slot[r] / g.NS], in_range);
                placed += in_range;
            }
            lo = hi;
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

int reroute_bitmap_words(int E, int k) {
    const int W = (tile_tokens(k) + 31) / 32;
    // the bitmaps and their prefixes share region A with the staged perm
    return bitmap_ints(E, W) <= kBitmapBudget ? W : 0;
}

size_t reroute_lds_bytes(int E, int R, int P, int k) {
    const int W = reroute_bitmap_words(E, k);
    // region A (which also takes the last tile's rank histogram); the
    // expert records (4 words each); rep_off (+1); three P-sized tables
    return sizeof(int32_t) * (static_cast<size_t>(region_a_ints(E, W)) +
                              static_cast<size_t>(5) * E + 1 + 3 * P);
}

// The limit only rises (the largest need so far), so a context or call
// with a smaller need never lowers what another one relies on.
hipError_t reroute_prepare(size_t lds_bytes) {
    static std::mutex mu;
    static size_t granted = 0;
    std::lock_guard<std::mutex> lock(mu);
    if (lds_bytes <= granted) return hipSuccess;
    const void *fns[] = {reinterpret_cast<const void *>(&k_reroute<false, false>),
                         reinterpret_cast<const void *>(&k_reroute<true, false>),
                         reinterpret_cast<const void *>(&k_reroute<false, true>),
                         reinterpret_cast<const void *>(&k_reroute<true, true>)};
    hipError_t e = hipSuccess;
    for (const void *f : fns)
        if (e == hipSuccess)
            e = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize,
                                    static_cast<int>(lds_bytes));
    if (e == hipSuccess) granted = lds_bytes;
    return e;
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
    g.spin_limit = c.wait_limit;
    g.lds_bytes = static_cast<uint32_t>(c.reroute_lds);
    g.lay = c.lay;
    g.phys = phys;
    g.perm = perm;
    g.inv_perm = inv_perm;
    g.state = c.scan_state;
    g.tick = c.rr_tick;
    g.group_base = c.group_base;
    g.tile_off = c.tile_off;
    const LoadShape sh = load_shape(A, L);
    if (sh.group != kLoadGroup) return hipErrorInvalidValue;   // never: one split
    g.load_groups = sh.groups;
    g.rank_counts = rank_counts;
    g.faults = faults;
    // the fast instance: top-8 routing, every expert's bitmap at its full
    // size, at most one expert per thread
    const bool fast = c.k == kFastK && g.bm_words == kFastWords && c.E <= kBlock;
    const dim3 grid(tiles, L);
    if (after_load && fast)
        hipLaunchKernelGGL((k_reroute<true, true>), grid, dim3(kBlock), c.reroute_lds, s, g);
    else if (after_load)
        hipLaunchKernelGGL((k_reroute<true, false>), grid, dim3(kBlock), c.reroute_lds, s, g);
    else if (fast)
        hipLaunchKernelGGL((k_reroute<false, true>), grid, dim3(kBlock), c.reroute_lds, s, g);
    else
        hipLaunchKernelGGL((k_reroute<false, false>), grid, dim3(kBlock), c.reroute_lds, s, g);
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
