// Quota replica planner: one workgroup per layer, all state in LDS.
//
// The UltraEP news write-up (section on how balancing in 300 microseconds
// works) describes a quota-driven scheduler that reacts to each
// microbatch's load right after gating; "How dots-infra/ultraep works"
// (summary) says it plans replicas that receive synchronised weights. The
// pages give no formula; the rule implemented here is the plainest reading:
//   Q = ceil(sum(counts) / R); expert e lives on rank e / N (slot e mod N);
//   experts of ranks loaded above Q are visited heaviest first (count desc,
//   id asc); each spills its rank's excess, chunk by chunk, into the lowest
//   free spare slot of the least-loaded rank (ties: lowest id) that has a
//   free spare slot and load < Q; chunk = min(source excess, expert
//   remainder, destination headroom); no such rank stops the plan.
//   A second rule (best fit, chosen per context) differs in one step: when
//   the amount left (min of source excess and expert remainder) is below
//   the least-loaded rank's headroom, it goes whole to the eligible rank
//   with the smallest headroom that still holds it (ties: lowest id), so
//   partly filled ranks close up instead of many ranks each taking a bit.
//   A third rule (best fit in covering order) keeps best fit's destinations
//   and changes the order of the candidates: with one spare slot per rank
//   each destination takes one chunk, so the destinations are pieces the
//   sources' excesses must cover, and a small excess left for last finds
//   only big pieces, or none. The amounts one rank can take at Q0 (at most
//   the largest headroom there) go first, smallest first, then the others,
//   largest first; the order is fixed once, at Q0. A fourth rule (best fit
//   in ascending order) takes every amount at Q0 smallest first, so that
//   of the amounts too large for one rank the largest, which needs the
//   most pieces, is placed last.
//   The quota search (also per context) makes the same plan at the quotas
//   Q0 + j * ceil(Q0 / 256), j = 0..63, in order, and keeps the first that
//   leaves nothing over (with none, Q0 stands): the pages call the
//   scheduler quota-driven without saying how the quota is set, and one
//   spare slot per rank leaves too little room at Q0 itself.
//
// Layout of the work (1024 threads):
//   A. all threads: counts and rank loads into LDS, Q0, the candidate list
//      and the list of ranks that can receive (compacted together by one
//      scan, then each ranked by comparison counting, four threads per
//      item: exact, and no sort network; the covering order ranks the
//      candidates a second time, by their amounts at Q0);
//   B. one wave per greedy pass, with the pass's state in registers. The
//      least-loaded eligible rank is the smaller of two minima: the next
//      entry of the receiving list, sorted once by (load, id) in part A
//      (such a rank has received nothing yet, so its key is unchanged), and
//      the smallest key among ranks that received a chunk and are still
//      eligible, held by their owner lanes and reduced with DPP only while
//      that set is non-empty (never with one spare slot per rank, where a
//      destination fills its only slot). The fixed quota takes one pass on
//      wave 0; the search runs 16 quotas at a time, one per wave;
//   C. all threads: replica table (CSR) and slot tables by one three-way
//      scan.
// Everything is integer and deterministic; the result does not depend on
// scheduling.
#include <climits>
#include <mutex>

#include "ue_internal.h"

namespace ue {
namespace {

struct PlanLds {
    int32_t *cnt, *rem, *load, *cand, *sorted, *first_rec, *nrec_e;
    int32_t *dkey, *dsorted, *scount, *slimit;
    int32_t *camt, *clim;       // covering order: amount at Q0, limit
    int32_t *rec_e, *rec_p, *rec_m, *slot_cap, *slot_exp, *rep_off;
};

__device__ __forceinline__ int32_t *carve_end(const PlanLds &s, int P) {
    return s.slot_exp + P;
}

// Chunk records: `regions` regions of 3 * R*S ints (expert, slot, amount),
// one per wave when the quota search keeps every pass's chunks.
__device__ __forceinline__ PlanLds carve(int32_t *base, int E, int R, int S,
                                         int P, int regions) {
    PlanLds s;
    int32_t *p = base;
    s.cnt = p; p += E;
    s.rem = p; p += E;
    s.cand = p; p += 2 * E;          // {rank << 16 | expert, count}
    s.sorted = p; p += E;
    s.first_rec = p; p += E;
    s.nrec_e = p; p += E;
    s.rep_off = p; p += E + 1;
    s.load = p; p += R;
    s.dkey = p; p += R;
    s.dsorted = p; p += R;
    s.scount = p; p += E;
    s.slimit = p; p += E;
    s.camt = p; p += E;
    s.clim = p; p += E;
    s.rec_e = p;
    s.rec_p = p + R * S;
    s.rec_m = p + 2 * R * S;
    p += regions * 3 * R * S;
    s.slot_cap = p; p += P;
    s.slot_exp = p; p += P;
    return s;
}

// The planner runs 16 waves per layer: phases A and C use them all, and
// the quota search runs one greedy pass per wave.
constexpr int kPlanBlock = 1024;
constexpr int kPlanWaves = kPlanBlock / 64;
// Quota search: quotas Q0 + j * ceil(Q0 / kQuotaGrain), j < kQuotaSteps.
constexpr int kQuotaSteps = 64;
constexpr int kQuotaGrain = 256;
static_assert(kQuotaSteps % kPlanWaves == 0, "whole rounds of passes");

// Exclusive prefix sum of one value per thread over the planner's block;
// the block total goes to `total`. Contains barriers: every thread calls it.
__device__ __forceinline__ int plan_block_sum(int v, int *wsum, int &total) {
    const int w = threadIdx.x >> 6;
    const int x = wave_inclusive_sum(v);
    if (lane_id() == 63) wsum[w] = x;
    __syncthreads();
    int before = 0;
    total = 0;
#pragma unroll
    for (int i = 0; i < kPlanWaves; ++i) {
        const int t = wsum[i];
        before += (i < w) ? t : 0;
        total += t;
    }
    __syncthreads();
    return before + x - v;
}

// Exclusive prefix sums of three values per thread at once; `wsum3` is
// 3 * kPlanWaves ints of LDS. Contains one barrier: every thread calls it,
// and a barrier must follow before `wsum3` is used again.
__device__ __forceinline__ void plan_block_sum3(int v[3], int *wsum3,
                                                int pre[3], int tot[3]) {
    const int w = threadIdx.x >> 6;
    int x[3];
#pragma unroll
    for (int i = 0; i < 3; ++i) {
        x[i] = wave_inclusive_sum(v[i]);
        if (lane_id() == 63) wsum3[i * kPlanWaves + w] = x[i];
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 3; ++i) {
        int before = 0, total = 0;
#pragma unroll
        for (int j = 0; j < kPlanWaves; ++j) {
            const int t = wsum3[i * kPlanWaves + j];
            before += (j < w) ? t : 0;
            total += t;
        }
        pre[i] = before + x[i] - v[i];
        tot[i] = total;
    }
}

// Sum over the four lanes of a quad (lanes 4q .. 4q + 3), in every one of
// them: DPP quad permutations swapping neighbours, then pairs.
__device__ __forceinline__ int quad_sum(int x) {
    x += __builtin_amdgcn_update_dpp(0, x, 0xB1, 0xF, 0xF, false);  // [1,0,3,2]
    x += __builtin_amdgcn_update_dpp(0, x, 0x4E, 0xF, 0xF, false);  // [2,3,0,1]
    return x;
}

// Entry c of an LDS list through a 64-entry window held one per lane:
// readlane with a uniform index, one LDS read per 64 entries.
struct ListWindow {
    const int32_t *list;
    int n, base, reg;
    __device__ __forceinline__ void init(const int32_t *l, int count) {
        list = l;
        n = count;
        base = 0;
        const int lane = threadIdx.x & 63;
        reg = lane < n ? list[lane] : -1;
    }
    __device__ __forceinline__ int get(int c) {
        if (c - base >= 64) {
            base = c & ~63;
            const int i = base + (threadIdx.x & 63);
            reg = i < n ? list[i] : -1;
        }
        return __builtin_amdgcn_readlane(reg, c - base);
    }
};

// Inclusive prefix sum over the wave with DPP (row shifts, then the row
// broadcasts), saturating at 2^30: values are non-negative and below
// 2^30, so no sum overflows and the saturating add stays associative.
__device__ __forceinline__ uint32_t wave_sat_inclusive_sum(uint32_t x) {
    constexpr uint32_t kCap = 1u << 30;
    auto step = [&](uint32_t t) {
        x = x + t;
        x = x < kCap ? x : kCap;
    };
    step(__builtin_amdgcn_update_dpp(0u, x, 0x111, 0xF, 0xF, false));  // row_shr:1
    step(__builtin_amdgcn_update_dpp(0u, x, 0x112, 0xF, 0xF, false));  // row_shr:2
    step(__builtin_amdgcn_update_dpp(0u, x, 0x114, 0xF, 0xF, false));  // row_shr:4
    step(__builtin_amdgcn_update_dpp(0u, x, 0x118, 0xF, 0xF, false));  // row_shr:8
    step(__builtin_amdgcn_update_dpp(0u, x, 0x142, 0xA, 0xF, false));  // row_bcast:15
    step(__builtin_amdgcn_update_dpp(0u, x, 0x143, 0xC, 0xF, false));  // row_bcast:31
    return x;
}

// Number of entries of the ascending key list `list[0, n)` below `bound`,
// found by one wave with two LDS reads: 64 samples at stride ceil(n / 64)
// bracket the boundary, then the entries strictly inside the bracket are
// compared (n up to 4096).
__device__ __forceinline__ int count_below(const int32_t *list, int n,
                                           uint32_t bound) {
    const int lane = threadIdx.x & 63;
    if (n <= 64) {
        const bool below = lane < n &&
                           static_cast<uint32_t>(list[lane]) < bound;
        return __builtin_popcountll(__ballot(below));
    }
    const int st = (n + 63) / 64;
    const int si = lane * st;
    const bool sb = si < n && static_cast<uint32_t>(list[si]) < bound;
    const int nb = __builtin_popcountll(__ballot(sb));
    if (nb == 0) return 0;
    const int b0 = (nb - 1) * st + 1;
    const int idx = b0 + lane;
    const bool in = lane < st - 1 && idx < n;
    const bool below = in && static_cast<uint32_t>(list[idx]) < bound;
    return b0 + __builtin_popcountll(__ballot(below));
}

// The spill loop at quota Q, run by one wave. With `write` it records the
// chunks in LDS (a search pass into a region of its own, when LDS allows
// one per wave); without, it only finds whether the plan runs out.
//  - Candidate c (in order) moves A_c = min(count, its home rank's excess
//    over Q left by the rank's earlier candidates) = clamp(limit_c - Q, 0,
//    count_c), where limit_c = rank load - counts of the rank's earlier
//    candidates (part A); the loop only places those amounts, chunk by
//    chunk, and stops the plan when no destination is left (exhausted).
//  - dsorted holds ranks with a spare slot as keys (load << rbits | rank),
//    ascending; the nd of them below Q are eligible at the start. Such a
//    rank has all S spare slots free until it is first chosen, and the
//    chunks of a run of such ranks are computed 64 at
//    a time: lane j takes the j-th next rank, a saturating prefix sum of
//    their headrooms (Q - load) finds the rank where the amount runs out,
//    every rank before it is filled to Q and that rank takes the rest.
//  - A rank left below Q with spare slots (only after taking the rest, and
//    only with S > 1) is held by its owner lane (rank mod 64) as a key plus
//    its free-slot count. Ranks of the list beyond the smallest held key
//    wait while that rank takes one chunk on its own.
//  - Best fit: when the rest is below the headroom of the rank that would
//    take it (always the least-loaded eligible one), it goes instead to the
//    eligible rank with the smallest headroom that holds it, ties to the
//    lowest id: a forward search of the list (from where the run stopped)
//    and a reduction over held ranks. A list entry taken this way is marked
//    gone (bit b of lane l: entry 64 b + l) and skipped when the run gets
//    there.
template <int RPL>
__device__ void spill_loop(PlanLds &s, int ncand, int nd_all, int R, int S,
                           int N, int NS, int Q, int rbits, bool best_fit,
                           bool write, int &nrec_out, int &exhausted_out) {
    const int lane = threadIdx.x & 63;
    // list entries below Q (a prefix: the list is ascending)
    const int nd = count_below(s.dsorted, nd_all,
                               static_cast<uint32_t>(Q) << rbits);
    uint32_t hkey[RPL];
    int hfree[RPL];
#pragma unroll
    for (int i = 0; i < RPL; ++i) {
        hkey[i] = 0xFFFFFFFFu;
        hfree[i] = 0;
    }
    uint32_t my_min = 0xFFFFFFFFu;
    uint32_t dgone = 0;
    int h_count = 0;
    // hold rank d (key k, f free slots) in its owner lane, or release it
    auto hold = [&](int d, uint32_t k, int f) {
        if (lane == (d & 63)) {
            const int dk = d >> 6;
            uint32_t b = 0xFFFFFFFFu;
#pragma unroll
            for (int i = 0; i < RPL; ++i) {
                if (i == dk) {
                    hkey[i] = k;
                    hfree[i] = f;
                }
                b = hkey[i] < b ? hkey[i] : b;
            }
            my_min = b;
        }
    };
    auto held_free = [&](int d) {
        const int dk = d >> 6;
        int f = 0;
#pragma unroll
        for (int i = 0; i < RPL; ++i) f = (i == dk) ? hfree[i] : f;
        return __builtin_amdgcn_readlane(f, d & 63);
    };
    const uint32_t rmask = (1u << rbits) - 1u;
    const int max_rec = R * S;
    int di = 0, nrec = 0, exhausted = 0;
    // whether list entry idx (any idx, per lane) was taken out of order
    auto is_gone = [&](int idx, bool in) {
        const uint32_t w = static_cast<uint32_t>(
            __shfl(static_cast<int>(dgone), idx & 63, 64));
        return in && ((w >> ((idx >> 6) & 31)) & 1u) != 0;
    };
    auto record = [&](int e, int d, int fr, int m) {
        if (write && lane == 0) {
            s.rec_e[nrec] = e;
            s.rec_p[nrec] = d * NS + N + (S - fr);
            s.rec_m[nrec] = m;
        }
        ++nrec;
    };
    // Place `need` whole on the eligible rank with the smallest headroom
    // >= need (the most loaded one with load <= Q - need; ties: lowest id),
    // among list entries from `from` on and held ranks.
    auto place_best_fit = [&](int e, int need, int from) {
        const int thr = Q - need;
        int bestL = -1, bestIdx = -1;
        for (int x0 = from; x0 < nd; x0 += 64) {
            const int idx = x0 + lane;
            const bool in = idx < nd;
            const uint32_t key = in ? static_cast<uint32_t>(s.dsorted[idx])
                                    : 0xFFFFFFFFu;
            const bool g = is_gone(idx, in);
            const int L = static_cast<int>(key >> rbits);
            const bool q = in && !g && L <= thr;
            const uint64_t bq = __ballot(q);
            if (bq) {
                const int last = 63 - __builtin_clzll(bq);
                const int Lw = __builtin_amdgcn_readlane(L, last);
                const uint64_t eq = __ballot(q && L == Lw);
                if (Lw > bestL) {
                    bestL = Lw;
                    bestIdx = x0 + __builtin_ctzll(eq);
                }
            }
            if (__ballot(in && !g && L > thr)) break;   // sorted: no more
        }
        // held ranks: (load + 1) << rbits | (rmask - id), largest wins
        uint32_t hb = 0;
#pragma unroll
        for (int i = 0; i < RPL; ++i) {
            if (hkey[i] == 0xFFFFFFFFu) continue;
            const uint32_t L = hkey[i] >> rbits;
            const uint32_t id = hkey[i] & rmask;
            const uint32_t enc = ((L + 1u) << rbits) | (rmask - id);
            if (static_cast<int>(L) <= thr && enc > hb) hb = enc;
        }
        const uint32_t hbest = h_count > 0 ? ~wave_min_u32(~hb) : 0u;
        const int Lh = static_cast<int>(hbest >> rbits) - 1;
        const int idh = static_cast<int>(rmask - (hbest & rmask));
        const int idd = bestIdx >= 0
            ? static_cast<int>(static_cast<uint32_t>(s.dsorted[bestIdx]) & rmask)
            : 0;
        const bool from_held = hbest != 0u &&
            (bestIdx < 0 || Lh > bestL || (Lh == bestL && idh < idd));
        if ((!from_held && bestIdx < 0) || nrec >= max_rec) {
            exhausted = 1;           // cannot happen with a consistent state
            return;
        }
        int d, Ld, fr;
        if (from_held) {
            d = idh;
            Ld = Lh;
            fr = held_free(d);
            hold(d, 0xFFFFFFFFu, 0);
            --h_count;
        } else {
            d = idd;
            Ld = bestL;
            fr = S;
            if (lane == (bestIdx & 63)) dgone |= 1u << (bestIdx >> 6);
        }
        record(e, d, fr, need);
        if (fr > 1 && Ld + need < Q) {
            hold(d, (static_cast<uint32_t>(Ld + need) << rbits) |
                        static_cast<uint32_t>(d), fr - 1);
            ++h_count;
        }
    };
    ListWindow cand, ccount, climit;
    cand.init(s.sorted, ncand);
    ccount.init(s.scount, ncand);
    climit.init(s.slimit, ncand);
    for (int c = 0; c < ncand && !exhausted; ++c) {
        const int e = cand.get(c);
        const int cnt = ccount.get(c);
        const int over = climit.get(c) - Q;
        int rem = over <= 0 ? 0 : (cnt < over ? cnt : over);
        while (rem > 0 && !exhausted) {
            const uint32_t kh = h_count > 0 ? wave_min_u32(my_min) : 0xFFFFFFFFu;
            // the next list ranks below the smallest held key, within the
            // spare slots left; entries taken out of order are skipped
            const int idx = di + lane;
            const bool in = idx < nd;
            const uint32_t key = in ? static_cast<uint32_t>(s.dsorted[idx])
                                    : 0xFFFFFFFFu;
            const bool g = is_gone(idx, in);
            const bool ok = in && !g && key < kh;
            const int cr = static_cast<int>(mask_rank(__ballot(ok)));
            const bool valid = ok && nrec + cr < max_rec;
            const uint64_t stops = __ballot(!valid && !g);
            const int stop = stops ? __builtin_ctzll(stops) : 64;
            const bool run = valid && lane < stop;
            const int Ld = static_cast<int>(key >> rbits);
            const int h = run ? Q - Ld : 0;
            const int pre = static_cast<int>(
                wave_sat_inclusive_sum(static_cast<uint32_t>(h)));
            const uint64_t hit = __ballot(run && pre >= rem);
            const int hl = hit ? __builtin_ctzll(hit) : stop;
            // the sum before the hit lane is below rem, hence exact
            const int before =
                hl >= 1 ? __builtin_amdgcn_readlane(pre, hl - 1) : 0;
            const int need = rem - before;
            const bool bf = hit && best_fit &&
                            need < __builtin_amdgcn_readlane(h, hl);
            // lanes placed now: full headroom before the hit lane, the rest
            // on the hit lane (unless best fit sends it elsewhere)
            const bool put = run && (lane < hl || (hit && lane == hl && !bf));
            const uint64_t puts = __ballot(put);
            if (write && put) {
                const int m = lane == hl ? need : h;
                const int d = static_cast<int>(key & rmask);
                const int at = nrec + static_cast<int>(mask_rank(puts));
                s.rec_e[at] = e;
                s.rec_p[at] = d * NS + N;      // its first spare
                s.rec_m[at] = m;
            }
            nrec += __builtin_popcountll(puts);
            if (hit) {
                di += hl + (bf ? 0 : 1);
                if (bf) {
                    place_best_fit(e, need, di);
                } else {
                    const uint32_t lk = static_cast<uint32_t>(
                        __builtin_amdgcn_readlane(static_cast<int>(key), hl));
                    const int Ld2 = static_cast<int>(lk >> rbits) + need;
                    if (S > 1 && Ld2 < Q) {
                        const int d = static_cast<int>(lk & rmask);
                        hold(d, (static_cast<uint32_t>(Ld2) << rbits) |
                                    static_cast<uint32_t>(d), S - 1);
                        ++h_count;
                    }
                }
                rem = 0;
                continue;
            }
            rem = need;                    // what the full chunks left
            di += stop;
            if (stop == 64) continue;
            // the run stopped before the amount: the smallest held rank is
            // now the least-loaded eligible one, or nothing is left
            if (kh == 0xFFFFFFFFu || nrec >= max_rec) {
                exhausted = 1;
                break;
            }
            const int d = static_cast<int>(kh & rmask);
            const int Lh = static_cast<int>(kh >> rbits);
            if (best_fit && rem < Q - Lh) {
                place_best_fit(e, rem, di);
                rem = 0;
                continue;
            }
            const int fr = held_free(d);
            const int m = rem < Q - Lh ? rem : Q - Lh;
            record(e, d, fr, m);
            rem -= m;
            const bool again = fr > 1 && Lh + m < Q;
            hold(d, again ? (static_cast<uint32_t>(Lh + m) << rbits) |
                                static_cast<uint32_t>(d)
                          : 0xFFFFFFFFu,
                 fr - 1);
            h_count -= again ? 0 : 1;
        }
    }
    nrec_out = nrec;
    exhausted_out = exhausted;
}

// The spill loop at quota Q for one spare slot per rank and at most 64 RPL
// ranks, run by one wave with the receiving list held in registers: entry
// x = 64 i + lane in slot i of every lane. A rank that takes a chunk has no
// slot left, so nothing is held and an entry leaves the list once used. Each
// entry keeps the prefix sum of the headrooms (Q - load) of the entries up
// to it that were not taken out of order (below 2^31: at most R * Q). An
// amount is placed with one ballot per slot: the run from di ends at the
// first entry whose headroom sum since di reaches it; the entries before it
// fill to Q and that entry takes the rest, or under best fit, when the rest
// is below its headroom, the rest goes to the most loaded entry from there
// on that holds it (lowest id among equal loads), which leaves the list and
// the sums. No entry reaching it means the list runs out. Candidates are
// read 64 at a time and those with nothing to move are skipped with a
// ballot. The same placements as spill_loop with S = 1, without LDS reads
// inside the loop.
template <int RPL>
__device__ __forceinline__ void spill_one_slot(PlanLds &s, int ncand, int nd_all,
                                               int N, int NS, int Q, int rbits,
                                               bool best_fit, bool write,
                                               int &nrec_out, int &exhausted_out) {
    const int lane = threadIdx.x & 63;
    const int nd = count_below(s.dsorted, nd_all,
                               static_cast<uint32_t>(Q) << rbits);
    const uint32_t rmask = (1u << rbits) - 1u;
    constexpr int kNone = 64 * RPL;
    // per slot: key, load, headroom and headroom prefix of the lane's entry;
    // avail (wave-uniform): bit l of slot i set while entry 64 i + l is in
    // the list and was not taken out of order
    int keyi[RPL], L[RPL], h[RPL], hsum[RPL];
    uint64_t avail[RPL];
    {
        int carry = 0;
#pragma unroll
        for (int i = 0; i < RPL; ++i) {
            const int x = 64 * i + lane;
            const bool in = x < nd;
            keyi[i] = in ? s.dsorted[x] : 0;
            L[i] = static_cast<int>(static_cast<uint32_t>(keyi[i]) >> rbits);
            h[i] = in ? Q - L[i] : 0;
            hsum[i] = wave_inclusive_sum(h[i]) + carry;
            carry = __builtin_amdgcn_readlane(hsum[i], 63);
            avail[i] = __ballot(in);
        }
    }
    // lanes below t of a slot (t may fall outside [0, 64))
    auto below = [](int t) -> uint64_t {
        return t <= 0 ? 0ull : (t >= 64 ? ~0ull : ((1ull << t) - 1ull));
    };
    // passing entry di: entries before it leave avail
    auto pass_to = [&](int d) {
#pragma unroll
        for (int i = 0; i < RPL; ++i) avail[i] &= ~below(d - 64 * i);
    };
    // di: first entry not yet passed; base: the headroom prefix before it
    int di = 0, base = 0, nrec = 0, exhausted = 0;
    for (int c0 = 0; c0 < ncand && !exhausted; c0 += 64) {
        const int ci = c0 + lane;
        const bool cv = ci < ncand;
        const int over_l = cv ? s.slimit[ci] - Q : 0;
        const int cnt_l = cv ? s.scount[ci] : 0;
        const int rem_l = over_l <= 0 ? 0 : (cnt_l < over_l ? cnt_l : over_l);
        const int e_l = cv ? s.sorted[ci] : 0;
        uint64_t todo = __ballot(rem_l > 0);
        while (todo) {
            const int j = __builtin_ctzll(todo);
            todo &= todo - 1;
            const int rem = __builtin_amdgcn_readlane(rem_l, j);
            const int e = __builtin_amdgcn_readlane(e_l, j);
            // the hit entry: the first live one whose sum since di reaches
            // rem; hh its headroom, hs its prefix
            int hl = kNone, hh = 0, hs = 0;
#pragma unroll
            for (int i = 0; i < RPL; ++i) {
                const uint64_t b = __ballot(hsum[i] - base >= rem) & avail[i];
                if (hl == kNone && b != 0) {
                    const int l = __builtin_ctzll(b);
                    hl = 64 * i + l;
                    hh = __builtin_amdgcn_readlane(h[i], l);
                    hs = __builtin_amdgcn_readlane(hsum[i], l);
                }
            }
            const bool hit = hl != kNone;
            const int need = hit ? rem - (hs - hh - base) : 0;
            const bool bf = hit && best_fit && need < hh;
            // entries placed now: full headroom before the hit entry, the
            // rest on the hit entry (unless best fit sends it elsewhere)
            const int end = bf ? hl : hl + 1;
            int placed = 0;
#pragma unroll
            for (int i = 0; i < RPL; ++i) {
                const int hi = hl - 64 * i;
                const uint64_t puts = avail[i] & below(end - 64 * i);
                if (write && ((puts >> lane) & 1ull)) {
                    const int at = nrec + placed + static_cast<int>(mask_rank(puts));
                    s.rec_e[at] = e;
                    s.rec_p[at] = static_cast<int>(static_cast<uint32_t>(keyi[i]) & rmask) * NS + N;
                    s.rec_m[at] = lane == hi ? need : h[i];
                }
                placed += __builtin_popcountll(puts);
            }
            nrec += placed;
            if (!hit) {
                exhausted = 1;
                break;
            }
            di = end;
            base = bf ? hs - hh : hs;
            pass_to(di);
            if (!bf) continue;
            // the list ascends, so the largest fitting load is the last
            // fitting entry's; the hit entry fits, so one exists
            const int thr = Q - need;
            int Lw = -1;
#pragma unroll
            for (int i = 0; i < RPL; ++i) {
                const uint64_t b = __ballot(L[i] <= thr) & avail[i];
                if (b != 0) Lw = __builtin_amdgcn_readlane(L[i], 63 - __builtin_clzll(b));
            }
            int bi = kNone, kb = 0, hb = 0;
#pragma unroll
            for (int i = 0; i < RPL; ++i) {
                const uint64_t b = __ballot(L[i] == Lw) & avail[i];
                if (bi == kNone && b != 0) {
                    const int l = __builtin_ctzll(b);
                    bi = 64 * i + l;
                    kb = __builtin_amdgcn_readlane(keyi[i], l);
                    hb = __builtin_amdgcn_readlane(h[i], l);
                    avail[i] &= ~(1ull << l);
                }
            }
            if (write && lane == 0) {
                s.rec_e[nrec] = e;
                s.rec_p[nrec] = static_cast<int>(static_cast<uint32_t>(kb) & rmask) * NS + N;
                s.rec_m[nrec] = need;
            }
            ++nrec;
#pragma unroll
            for (int i = 0; i < RPL; ++i)
                hsum[i] -= 64 * i + lane >= bi ? hb : 0;
        }
    }
    nrec_out = nrec;
    exhausted_out = exhausted;
}

// One greedy pass at quota Q by the calling wave, dispatched on the number
// of ranks each lane may hold.
__device__ __forceinline__ void spill_pass(PlanLds &s, int ncand, int nd_all, int R, int S,
                           int N, int NS, int Q, int rbits, bool best_fit,
                           bool write, int &nrec, int &exhausted) {
    nrec = 0;
    exhausted = 0;
    if (S == 1 && R <= 256) {
        switch ((R + 63) / 64) {
            case 1: spill_one_slot<1>(s, ncand, nd_all, N, NS, Q, rbits, best_fit, write, nrec, exhausted); break;
            case 2: spill_one_slot<2>(s, ncand, nd_all, N, NS, Q, rbits, best_fit, write, nrec, exhausted); break;
            default: spill_one_slot<4>(s, ncand, nd_all, N, NS, Q, rbits, best_fit, write, nrec, exhausted); break;
        }
        return;
    }
    switch ((R + 63) / 64) {
        case 1: spill_loop<1>(s, ncand, nd_all, R, S, N, NS, Q, rbits, best_fit, write, nrec, exhausted); break;
        case 2: spill_loop<2>(s, ncand, nd_all, R, S, N, NS, Q, rbits, best_fit, write, nrec, exhausted); break;
        case 3:
        case 4: spill_loop<4>(s, ncand, nd_all, R, S, N, NS, Q, rbits, best_fit, write, nrec, exhausted); break;
        case 5: case 6: case 7:
        case 8: spill_loop<8>(s, ncand, nd_all, R, S, N, NS, Q, rbits, best_fit, write, nrec, exhausted); break;
        default: spill_loop<16>(s, ncand, nd_all, R, S, N, NS, Q, rbits, best_fit, write, nrec, exhausted); break;
    }
}

// The scan that finishes the load: the count kernel left, per group of
// tiles, each tile's count of every expert in the group's earlier tiles
// (tile t of group g at row t + g of the per-tile table) and the group's
// own counts in the row after its last tile; the scan writes each group's
// base row (the count in all earlier groups) and the layer's counts (and
// the ids out of range: assignments minus counted ones). Those rows are
// what the fused reroute reads.
struct ScanArgs {
    uint16_t *rows;            // [L][row_stride = tiles + groups][E]
    int32_t *group_base;       // [L][groups][E]
    int64_t A;                 // assignments per layer
    int tiles, group, row_stride, groups;
    int32_t *counts;           // [L][E] out
    int32_t *invalid;          // [L] out, may be null
    // When the plan is made in the same launch from these counts, the
    // dispatch totals the reroute would find follow from the plan alone:
    // every assignment of a valid id falls in a replica's capacity (the
    // capacities of an expert's replicas add up to its count), so a rank
    // receives what the plan's slots on it hold (its load after the plan)
    // and the faults are the ids out of range. Written here when not null.
    int32_t *rank_counts;      // [L][R] out, may be null
    int32_t *faults;           // [L] out, may be null
};
constexpr int kModeScan = 1;   // finish the load (ScanArgs)
constexpr int kModePlan = 2;   // make the plan

// The quota search spread over `split` workgroups per layer (1: not
// spread). Each runs part A and then kSplitWaves passes, one per SIMD, at
// quotas j = p * kSplitWaves + wave (p: its place among the layer's): with 16 waves on four SIMDs the
// passes of one workgroup contend for issue, one per SIMD they do not.
// Each publishes, per pass, the number of chunks (or -1 when the pass ran
// out) and a successful pass's chunks; the last workgroup of the layer to
// finish (a counter per layer, reset by that workgroup) keeps the first
// quota that works and goes on alone: with the plan from there, or with
// the remaining quotas in rounds as above. No workgroup waits on another.
constexpr int kSplitWaves = 4;
struct SplitArgs {
    int split;
    int32_t *rec;      // [slots][3][R*S] chunks (expert, slot, amount)
    int32_t *flag;     // [slots] chunks of a pass that works, else -1
    uint32_t *cnt;     // [layers] workgroups done; 0 between calls
};

// kSpread: the quota search may be spread (sp.split > 1); the other
// instance is the plain one-workgroup-per-layer planner, compiled without
// any of it.
template <bool kSpread>
__global__ __launch_bounds__(kPlanBlock) void k_plan(
    const int32_t *__restrict__ counts, int E, int R, int S, int N, int NS,
    int P, int rbits, int policy, int quota_mode, int per_wave,
    uint32_t lds_bytes, ue_placement_layout lay,
    int32_t *__restrict__ placement, int mode, ScanArgs sc, SplitArgs sp) {
    extern __shared__ __align__(16) int32_t lds[];
    __shared__ int wsum[kPlanWaves];
    __shared__ int wsum3[3 * kPlanWaves];
    __shared__ int s_works[kPlanWaves];
    __shared__ int s_nrecw[kPlanWaves];
    __shared__ int s_nrec, s_exhausted, s_quota, s_region;
    __shared__ uint32_t wsat[kPlanWaves];
    __shared__ int scan_tot[kMaxExperts];   // scan: the layer's counts
    __shared__ int s_last, s_first;

    // workgroups of one layer: the first writes everything before the
    // plan (the others compute the same values), the last to finish makes
    // the plan itself
    const int split = kSpread ? sp.split : 1;
    const int layer = kSpread ? static_cast<int>(blockIdx.x) / split
                              : static_cast<int>(blockIdx.x);
    const int wg_part = kSpread ? static_cast<int>(blockIdx.x) - layer * split : 0;
    const int tid = threadIdx.x;

    if (mode & kModeScan) {
        // Group g's own counts are in the row after its last tile (row
        // min(tiles, (g + 1) * group) + g); each group's base is the
        // exclusive prefix of those over earlier groups, and the layer's
        // counts their sum.
        const int G = sc.group;
        const int ng = (sc.tiles + G - 1) / G;
        const uint16_t *rows =
            sc.rows + static_cast<int64_t>(layer) * sc.row_stride * E;
        int32_t *gb = sc.group_base + static_cast<int64_t>(layer) * sc.groups * E;
        auto total_row = [&](int g) {
            const int tend = (g + 1) * G < sc.tiles ? (g + 1) * G : sc.tiles;
            return static_cast<int64_t>(tend + g) * E;
        };
        // (one expert per thread below needs a second round of loads, and
        // reads its rows again, once a thread's chunk exceeds 8 groups)
        const int pt1 = kPlanBlock / E;
        if ((E & 1) == 0 && (ng + pt1 - 1) / pt1 > 8 &&
            lds_bytes >= 2 * kPlanBlock * sizeof(int32_t)) {
            // Two experts per thread (E even, so every row is 4-byte
            // aligned): one 32-bit load reads a pair's counts in a group's
            // row. PT2 threads per pair (at least 2, since E <= 1024), each
            // summing a chunk of consecutive groups, up to kScanY groups
            // in flight in registers; a chunk of at most kScanY groups is
            // then written out without reading its rows again (large EP:
            // 128 groups, 16 per thread, one round of loads: its plan
            // 34.8 -> 31.6 us; with 32 groups, as at dsv3, the pairs
            // measured 1.3 us slower than one expert per thread).
            constexpr int kScanY = 16;
            const int EP = E >> 1;
            const int PT2 = kPlanBlock / EP;
            const int j = tid / EP, ep = tid - j * EP;
            const int cs = (ng + PT2 - 1) / PT2;
            const int g0 = j < PT2 ? j * cs : ng;
            const int g1 = g0 + cs < ng ? g0 + cs : ng;
            uint32_t y[kScanY];
            auto load_y = [&](int b) {
#pragma unroll
                for (int q = 0; q < kScanY; ++q)
                    y[q] = b + q < g1
                        ? *reinterpret_cast<const uint32_t *>(rows + total_row(b + q) + 2 * ep)
                        : 0u;
            };
            int lo = 0, hi = 0;
            for (int b = g0; b < g1; b += kScanY) {
                load_y(b);
#pragma unroll
                for (int q = 0; q < kScanY; ++q) {
                    lo += static_cast<int>(y[q] & 0xFFFFu);
                    hi += static_cast<int>(y[q] >> 16);
                }
            }
            // thread (j, pair) at lds[j * E + 2 * pair + half]
            if (j < PT2) {
                lds[2 * tid] = lo;
                lds[2 * tid + 1] = hi;
            }
            __syncthreads();
            if (j < PT2) {
                int rlo = 0, rhi = 0;
                for (int jj = 0; jj < j; ++jj) {
                    rlo += lds[jj * E + 2 * ep];
                    rhi += lds[jj * E + 2 * ep + 1];
                }
                if (j == 0) {
                    int alo = 0, ahi = 0;
                    for (int jj = 0; jj < PT2; ++jj) {
                        alo += lds[jj * E + 2 * ep];
                        ahi += lds[jj * E + 2 * ep + 1];
                    }
                    scan_tot[2 * ep] = alo;
                    scan_tot[2 * ep + 1] = ahi;
                    if (wg_part == 0) {
                        int32_t *cl = sc.counts + static_cast<int64_t>(layer) * E;
                        cl[2 * ep] = alo;
                        cl[2 * ep + 1] = ahi;
                    }
                }
                for (int b = g0; b < g1; b += kScanY) {
                    if (cs > kScanY) load_y(b);
#pragma unroll
                    for (int q = 0; q < kScanY; ++q) {
                        if (b + q < g1 && wg_part == 0)
                            *reinterpret_cast<int2 *>(gb + static_cast<int64_t>(b + q) * E +
                                                      2 * ep) = int2{rlo, rhi};
                        rlo += static_cast<int>(y[q] & 0xFFFFu);
                        rhi += static_cast<int>(y[q] >> 16);
                    }
                }
            }
        } else {
            // PT threads per expert (E <= kPlanBlock): thread (j, e) sums its
            // chunk of consecutive groups, the chunks' sums meet in LDS, and
            // each thread then writes the running base of its own groups. A
            // thread holds up to 8 group counts in registers; longer chunks
            // read their counts a second time (from cache).
            const int PT = kPlanBlock / E;
            const int j = tid / E, e = tid - j * E;
            const int cs = (ng + PT - 1) / PT;
            const int g0 = j < PT ? j * cs : ng;
            const int g1 = g0 + cs < ng ? g0 + cs : ng;
            int y[8];
            auto load8 = [&](int b) {
#pragma unroll
                for (int q = 0; q < 8; ++q)
                    y[q] = b + q < g1 ? static_cast<int>(rows[total_row(b + q) + e]) : 0;
            };
            int tot = 0;
            for (int b = g0; b < g1; b += 8) {
                load8(b);
#pragma unroll
                for (int q = 0; q < 8; ++q) tot += y[q];
            }
            if (j < PT) lds[tid] = tot;
            __syncthreads();
            if (j < PT) {
                int run = 0;
                for (int jj = 0; jj < j; ++jj) run += lds[jj * E + e];
                if (j == 0) {
                    int all = 0;
                    for (int jj = 0; jj < PT; ++jj) all += lds[jj * E + e];
                    scan_tot[e] = all;
                    if (wg_part == 0) sc.counts[static_cast<int64_t>(layer) * E + e] = all;
                }
                for (int b = g0; b < g1; b += 8) {
                    if (cs > 8) load8(b);
#pragma unroll
                    for (int q = 0; q < 8; ++q) {
                        if (b + q < g1 && wg_part == 0)
                            gb[static_cast<int64_t>(b + q) * E + e] = run;
                        run += y[q];
                    }
                }
            }
        }
        __syncthreads();
    }
    if (mode & kModeScan) {
        int part = 0;
        for (int x = tid; x < E; x += kPlanBlock) part += scan_tot[x];
        int total;
        plan_block_sum(part, wsum, total);
        if (tid == 0 && sc.invalid && wg_part == 0)
            sc.invalid[layer] = static_cast<int32_t>(sc.A - total);
        if (!(mode & kModePlan)) return;
    }
    const bool scanned = (mode & kModeScan) != 0;
    const int32_t *cin = counts + static_cast<int64_t>(layer) * E;
    int32_t *out = placement + static_cast<int64_t>(layer) * lay.words;
    PlanLds s = carve(lds, E, R, S, P, per_wave ? kPlanWaves : 1);
    // the carve-up must fit the launch's LDS (checked, not assumed); a
    // mismatch marks the block (exhausted = -1) rather than pass silently
    if (static_cast<size_t>(carve_end(s, P) - lds) * 4 > lds_bytes) {
        if (wg_part != 0) return;
        if (tid == 0) out[lay.exhausted] = -1;
        // the table is not written: every assignment is marked a fault
        for (int r = tid; r < R && sc.rank_counts; r += kPlanBlock)
            sc.rank_counts[static_cast<int64_t>(layer) * R + r] = 0;
        if (tid == 0 && sc.faults)
            sc.faults[layer] = static_cast<int32_t>(sc.A) | kPoisonBit;
        return;
    }

    // ---- A. loads, quota, candidates ----------------------------------
    // (E <= kPlanBlock: one count per thread)
    int part = 0;
    uint32_t sat = 0;    // the count, a negative one as 2^30
    for (int e = tid; e < E; e += kPlanBlock) {
        const int c = scanned ? scan_tot[e] : cin[e];
        s.cnt[e] = c;
        s.rem[e] = c;
        s.nrec_e[e] = 0;
        s.first_rec[e] = 0;
        part += c;
        sat = c < 0 ? (1u << 30) : static_cast<uint32_t>(c);
    }
    for (int p = tid; p < P; p += kPlanBlock) {
        s.slot_cap[p] = 0;
        s.slot_exp[p] = -1;
    }
    // counts must be >= 0 and sum below 2^30 (the int32 loads, the packed
    // rank keys and the headroom sums rely on it; ue_load's counts always
    // do): a saturating sum per wave, joined after the barrier below
    sat = wave_sat_inclusive_sum(sat);
    if ((tid & 63) == 63) wsat[tid >> 6] = sat;
    int total;
    plan_block_sum(part, wsum, total);   // barrier: cnt and wsat visible
    {
        uint64_t all = 0;
#pragma unroll
        for (int w = 0; w < kPlanWaves; ++w) all += wsat[w];
        if (all >= (1u << 30)) {
            // not planned: an empty table (no replica, every later reroute
            // assignment a fault), marked exhausted = -1; uniform across
            // the block, so every thread leaves here
            if (wg_part != 0) return;
            for (int i = tid; i < lay.words; i += kPlanBlock) {
                const bool neg1 =
                    i == lay.exhausted ||
                    (i >= lay.rep_slot && i < lay.rep_slot + P) ||
                    (i >= lay.slot_expert && i < lay.slot_expert + P);
                out[i] = neg1 ? -1 : 0;
            }
            // no replica at all: every assignment is a fault
            for (int r = tid; r < R && sc.rank_counts; r += kPlanBlock)
                sc.rank_counts[static_cast<int64_t>(layer) * R + r] = 0;
            if (tid == 0 && sc.faults) sc.faults[layer] = static_cast<int32_t>(sc.A);
            return;
        }
    }
    const int Q0 = (total + R - 1) / R;
    const bool search = quota_mode == UE_QUOTA_SEARCH;
    const int step = (Q0 + kQuotaGrain - 1) / kQuotaGrain;
    // highest quota any pass may use: ranks below it can be destinations
    const int Qmax = search ? Q0 + (kQuotaSteps - 1) * step : Q0;
    for (int r = tid; r < R; r += kPlanBlock) {
        int l = 0;
        for (int i = 0; i < N; ++i) l += s.cnt[r * N + i];
        s.load[r] = l;
        if (wg_part == 0) out[lay.load_before + r] = l;
    }
    __syncthreads();

    // Two lists compacted with one scan: the candidates in id order
    // (experts whose home rank is above Q0, so above any quota tried: a
    // superset of each pass's candidates), packed as (home rank << 16 |
    // expert) with the count beside it (E and R below 2^16); and the ranks
    // that can receive at some quota tried (a spare slot, load below Qmax),
    // as keys (load << rbits | rank), in rank order.
    int ncand, nd;
    {
        const int pe = (E + kPlanBlock - 1) / kPlanBlock;
        const int e0 = tid * pe, e1 = (e0 + pe < E) ? e0 + pe : E;
        const int pr = (R + kPlanBlock - 1) / kPlanBlock;
        const int r0 = tid * pr, r1 = (r0 + pr < R) ? r0 + pr : R;
        int v[3] = {0, 0, 0}, pre[3], tot[3];
        for (int e = e0; e < e1; ++e) v[0] += (s.load[e / N] > Q0);
        for (int r = r0; r < r1; ++r) v[1] += (S > 0 && s.load[r] < Qmax);
        plan_block_sum3(v, wsum3, pre, tot);
        int2 *cand2 = reinterpret_cast<int2 *>(s.cand);
        for (int e = e0; e < e1; ++e)
            if (s.load[e / N] > Q0)
                cand2[pre[0]++] = int2{((e / N) << 16) | e, s.cnt[e]};
        for (int r = r0; r < r1; ++r)
            if (S > 0 && s.load[r] < Qmax)
                s.dkey[pre[1]++] = static_cast<int32_t>(
                    (static_cast<uint32_t>(s.load[r]) << rbits) |
                    static_cast<uint32_t>(r));
        ncand = tot[0];
        nd = tot[1];
    }
    __syncthreads();
    // rank each candidate by (count desc, id asc); at quota Q it moves its
    // count capped by the excess its home rank still has after the rank's
    // earlier candidates (each of those moved min(count, excess)), i.e.
    // clamp(limit - Q, 0, count) with limit = rank load - their counts
    // (kSplit adjacent threads share a candidate, each comparing against
    // every kSplit-th other one; their sums meet through lane swaps)
    constexpr int kSplit = 4;
    static_assert(kSplit == 4, "quad_sum joins the four threads of a candidate");
    const bool cover = policy == UE_PLAN_BEST_FIT_COVER ||
                       policy == UE_PLAN_BEST_FIT_ASCENDING;
    const int2 *cand2 = reinterpret_cast<const int2 *>(s.cand);
    for (int i0 = 0; i0 < ncand; i0 += kPlanBlock / kSplit) {
        const int i = i0 + tid / kSplit;
        const int q = tid % kSplit;
        const bool act = i < ncand;
        const int2 me = act ? cand2[i] : int2{0, 0};
        const int e = me.x & 0xFFFF;
        const int r = me.x >> 16;
        const int c = me.y;
        int pos = 0, before = 0;
        if (act) {
#pragma unroll 4
            for (int j = q; j < ncand; j += kSplit) {
                const int2 o = cand2[j];
                const int f = o.x & 0xFFFF;
                const bool earlier = (o.y > c) || (o.y == c && f < e);
                pos += earlier;
                before += (earlier && (o.x >> 16) == r) ? o.y : 0;
            }
        }
        pos = quad_sum(pos);
        before = quad_sum(before);
        if (act && q == 0) {
            if (cover) {
                // placed below, by its amount at Q0 instead
                const int lim = s.load[r] - before;
                const int a = lim - Q0;
                s.camt[i] = a <= 0 ? 0 : (a < c ? a : c);
                s.clim[i] = lim;
            } else {
                s.sorted[pos] = e;
                s.scount[pos] = c;
                s.slimit[pos] = s.load[r] - before;
            }
        }
    }
    // the receiving ranks placed by their rank among the keys (distinct,
    // so the order is strict)
    for (int i0 = 0; i0 < nd; i0 += kPlanBlock / kSplit) {
        const int i = i0 + tid / kSplit;
        const int q = tid % kSplit;
        const bool act = i < nd;
        const uint32_t k = act ? static_cast<uint32_t>(s.dkey[i]) : 0u;
        int pos = 0;
        if (act) {
#pragma unroll 4
            for (int j = q; j < nd; j += kSplit)
                pos += static_cast<uint32_t>(s.dkey[j]) < k;
        }
        pos = quad_sum(pos);
        if (act && q == 0) s.dsorted[pos] = static_cast<int32_t>(k);
    }
    __syncthreads();
    if (cover) {
        // Covering order. H0, the largest headroom at Q0 among ranks with
        // a spare slot, comes from the smallest receiving key (the list
        // holds every rank with a spare slot and load below the highest
        // quota tried, sorted); amounts at Q0 up to H0 go first, smallest
        // first, then the larger ones, largest first (ties: lowest id).
        // The ascending order is the same with no amount counted as large
        const int minload = nd > 0
            ? static_cast<int>(static_cast<uint32_t>(s.dsorted[0]) >> rbits)
            : Q0;
        const int H0 = policy == UE_PLAN_BEST_FIT_ASCENDING
            ? INT_MAX : (minload < Q0 ? Q0 - minload : 0);
        // one key per candidate orders all three levels at once: the
        // group (the amounts one rank can take first), the amount within
        // it (ascending, or descending among the large ones; amounts are
        // below 2^30), then the id (below 2^16); a branch-free compare
        // keeps both reads of each step in flight together
        auto ckey = [&](int a_, int f_) -> uint64_t {
            const uint32_t k_ = a_ > H0
                ? 0x80000000u | static_cast<uint32_t>(0x3FFFFFFF - a_)
                : static_cast<uint32_t>(a_);
            return (static_cast<uint64_t>(k_) << 16) | static_cast<uint32_t>(f_);
        };
        for (int i0 = 0; i0 < ncand; i0 += kPlanBlock / kSplit) {
            const int i = i0 + tid / kSplit;
            const int q = tid % kSplit;
            const bool act = i < ncand;
            const int2 me = act ? cand2[i] : int2{0, 0};
            const int e = me.x & 0xFFFF;
            const uint64_t mk = ckey(act ? s.camt[i] : 0, e);
            int pos = 0;
            if (act) {
#pragma unroll 4
                for (int j = q; j < ncand; j += kSplit)
                    pos += ckey(s.camt[j], cand2[j].x & 0xFFFF) < mk;
            }
            pos = quad_sum(pos);
            if (act && q == 0) {
                s.sorted[pos] = e;
                s.scount[pos] = me.y;
                s.slimit[pos] = s.clim[i];
            }
        }
        __syncthreads();
    }

    const bool best_fit = policy != UE_PLAN_LEAST_LOADED;
    const int wave = tid >> 6;
    // ---- B. greedy passes. Quota search: rounds of one pass per wave over
    // the quotas in order; the first round with a quota that leaves nothing
    // over ends the search, and the lowest such quota of that round is kept
    // (every lower one was tried); with none, Q0 stands. With a record
    // region per wave the chosen pass's chunks are kept as they are;
    // otherwise (and for the fixed quota) wave 0 makes the plan at the
    // chosen quota and records it. One call site keeps the pass inlined
    // once.
    const int RS = R * S;
    int Q = Q0;
    int j0 = 0;
    bool rec = !search;
    bool chosen = false;
    if (kSpread && search && split > 1) {
        // the first kSplitWaves * split quotas, spread over the layer's
        // workgroups (records per wave: the host spreads only then)
        int nrec_w = 0, exh_w = 1;
        if (wave < kSplitWaves) {
            PlanLds sw = s;
            sw.rec_e = s.rec_e + wave * 3 * RS;
            sw.rec_p = sw.rec_e + RS;
            sw.rec_m = sw.rec_e + 2 * RS;
            spill_pass(sw, ncand, nd, R, S, N, NS,
                       Q0 + (wg_part * kSplitWaves + wave) * step, rbits,
                       best_fit, true, nrec_w, exh_w);
        }
        if ((tid & 63) == 0 && wave < kSplitWaves) {
            s_works[wave] = !exh_w;
            s_nrecw[wave] = nrec_w;
        }
        __syncthreads();
        // publish: chunk counts, and the chunks of the passes that work
        const int64_t slot0 = static_cast<int64_t>(blockIdx.x) * kSplitWaves;
        for (int w = 0; w < kSplitWaves; ++w) {
            if (!s_works[w]) continue;
            const int n = s_nrecw[w];
            const int32_t *src = s.rec_e + w * 3 * RS;
            int32_t *dst = sp.rec + (slot0 + w) * 3 * RS;
            for (int i = tid; i < n; i += kPlanBlock) {
                dst[i] = src[i];
                dst[RS + i] = src[RS + i];
                dst[2 * RS + i] = src[2 * RS + i];
            }
        }
        if (tid < kSplitWaves)
            sp.flag[slot0 + tid] = s_works[tid] ? s_nrecw[tid] : -1;
        // one device-scope fence per workgroup on each side, after the
        // barrier that orders the workgroup's own stores and loads: each
        // such fence writes back or invalidates a whole L2, so one per
        // wave would cost a multiple of the plan
        __syncthreads();
        if (tid == 0) {
            __threadfence();
            s_last = atomicAdd(sp.cnt + layer, 1u) == static_cast<uint32_t>(split - 1);
            if (s_last) __threadfence();
        }
        __syncthreads();
        if (!s_last) return;
        const int nq = kSplitWaves * split;
        const int64_t lslot0 = static_cast<int64_t>(layer) * nq;
        static_assert(kSplitWaves * 16 <= 64, "one wave reads every flag");
        if (tid < 64) {
            // the flags read at once, one per lane; the first that works
            const bool works = tid < nq && sp.flag[lslot0 + tid] >= 0;
            const uint64_t b = __ballot(works);
            if (tid == 0) {
                sp.cnt[layer] = 0;
                s_first = b ? __builtin_ctzll(b) : -1;
            }
        }
        __syncthreads();
        const int first = s_first;
        if (first >= 0) {
            const int n = sp.flag[lslot0 + first];
            const int32_t *src = sp.rec + (lslot0 + first) * 3 * RS;
            for (int i = tid; i < n; i += kPlanBlock) {
                s.rec_e[i] = src[i];
                s.rec_p[i] = src[RS + i];
                s.rec_m[i] = src[2 * RS + i];
            }
            if (tid == 0) {
                s_nrec = n;
                s_exhausted = 0;
                s_quota = Q0 + first * step;
                s_region = 0;
            }
            Q = Q0 + first * step;
            chosen = true;
        } else {
            j0 = nq;
            rec = j0 >= kQuotaSteps;
        }
        __syncthreads();
    }
#pragma unroll 1
    while (!chosen) {
        int nrec_w = 0, exh_w = 0;
        PlanLds sw = s;
        if (!rec && per_wave) {
            sw.rec_e = s.rec_e + wave * 3 * RS;
            sw.rec_p = sw.rec_e + RS;
            sw.rec_m = sw.rec_e + 2 * RS;
        }
        if (!rec || wave == 0)
            spill_pass(sw, ncand, nd, R, S, N, NS,
                       rec ? Q : Q0 + (j0 + wave) * step, rbits, best_fit,
                       rec || per_wave, nrec_w, exh_w);
        if (rec) {
            if (tid == 0) {
                s_nrec = nrec_w;
                s_exhausted = exh_w;
                s_quota = Q;
                s_region = 0;
            }
            break;
        }
        if ((tid & 63) == 0) {
            s_works[wave] = !exh_w;
            s_nrecw[wave] = nrec_w;
        }
        __syncthreads();
        int first = -1;
        for (int w = kPlanWaves - 1; w >= 0; --w)
            if (s_works[w]) first = w;
        if (first >= 0) {
            Q = Q0 + (j0 + first) * step;
            if (per_wave) {
                if (tid == 0) {
                    s_nrec = s_nrecw[first];
                    s_exhausted = 0;
                    s_quota = Q;
                    s_region = first;
                }
                break;
            }
        }
        __syncthreads();
        j0 += kPlanWaves;
        rec = first >= 0 || j0 >= kQuotaSteps;
    }
    __syncthreads();
    s.rec_e += s_region * 3 * RS;
    s.rec_p += s_region * 3 * RS;
    s.rec_m += s_region * 3 * RS;

    // per expert: chunks placed (records of one expert are consecutive),
    // the first of them and the remainder kept by the master; per rank: the
    // loads after the plan; each used spare slot takes its chunk (the slot
    // tables were cleared in part A). Integer adds: order does not matter.
    const int nrec = s_nrec;
    for (int i = tid; i < nrec; i += kPlanBlock) {
        const int e = s.rec_e[i];
        const int m = s.rec_m[i];
        const int p = s.rec_p[i];
        if (i == 0 || s.rec_e[i - 1] != e) s.first_rec[e] = i;
        atomicAdd(&s.nrec_e[e], 1);
        atomicSub(&s.rem[e], m);
        atomicSub(&s.load[e / N], m);
        atomicAdd(&s.load[p / NS], m);
        s.slot_exp[p] = e;
        s.slot_cap[p] = m;
    }
    __syncthreads();

    // ---- C. replica table and slot tables --------------------------------
    // native slots hold what their masters keep
    for (int e = tid; e < E; e += kPlanBlock) {
        const int p = (e / N) * NS + (e % N);
        s.slot_exp[p] = e;
        s.slot_cap[p] = s.rem[e];
    }
    __syncthreads();
    // one scan for three sums: replica offsets (1 + chunks per expert),
    // slot offsets (slot capacities) and the residual (excess over the
    // quota used, per rank); each thread takes a contiguous run of experts
    // and of slots
    const int pe = (E + kPlanBlock - 1) / kPlanBlock;
    const int pp = (P + kPlanBlock - 1) / kPlanBlock;
    const int e0 = tid * pe, e1 = (e0 + pe < E) ? e0 + pe : E;
    const int p0 = tid * pp, p1 = (p0 + pp < P) ? p0 + pp : P;
    int v[3] = {0, 0, 0}, pre[3], tot[3];
    for (int e = e0; e < e1; ++e) v[0] += 1 + s.nrec_e[e];
    for (int p = p0; p < p1; ++p) v[1] += s.slot_cap[p];
    for (int r = tid; r < R; r += kPlanBlock) {
        const int l = s.load[r];
        out[lay.load_after + r] = l;
        if (sc.rank_counts) sc.rank_counts[static_cast<int64_t>(layer) * R + r] = l;
        v[2] += (l > Q) ? (l - Q) : 0;   // Q: the quota used
    }
    plan_block_sum3(v, wsum3, pre, tot);
    const int n_rep = tot[0];
    {
        int run = pre[0];
        for (int e = e0; e < e1; ++e) {
            s.rep_off[e] = run;
            out[lay.rep_off + e] = run;
            run += 1 + s.nrec_e[e];
        }
        run = pre[1];
        for (int p = p0; p < p1; ++p) {
            const int c = s.slot_cap[p];
            out[lay.slot_expert + p] = s.slot_exp[p];
            out[lay.slot_cap + p] = c;
            out[lay.slot_off + p] = run;
            run += c;
        }
    }
    __syncthreads();   // replica offsets visible
    for (int e = tid; e < E; e += kPlanBlock) {
        const int base = s.rep_off[e];
        out[lay.rep_slot + base] = (e / N) * NS + (e % N);
        out[lay.rep_cap + base] = s.rem[e];
        const int f = s.first_rec[e];
        const int n = s.nrec_e[e];
        for (int i = 0; i < n; ++i) {
            out[lay.rep_slot + base + 1 + i] = s.rec_p[f + i];
            out[lay.rep_cap + base + 1 + i] = s.rec_m[f + i];
        }
    }
    for (int i = n_rep + tid; i < P; i += kPlanBlock) {
        out[lay.rep_slot + i] = -1;
        out[lay.rep_cap + i] = 0;
    }
    // the block's alignment padding is written too, so a block is fully
    // defined by its counts
    for (int i = lay.load_after + R + tid; i < lay.words; i += kPlanBlock) out[i] = 0;
    if (tid == 0 && sc.faults)
        sc.faults[layer] = static_cast<int32_t>(sc.A - total);
    if (tid == 0) {
        out[lay.rep_off + E] = n_rep;
        out[lay.slot_off + P] = tot[1];
        out[lay.quota] = s_quota;
        out[lay.exhausted] = s_exhausted;
        out[lay.residual] = tot[2];
        out[lay.n_rep] = n_rep;
    }
}

}  // namespace

size_t plan_lds_bytes(int E, int R, int S, int P, bool per_wave) {
    const size_t regions = per_wave ? kPlanWaves : 1;
    const size_t plan = sizeof(int32_t) * (static_cast<size_t>(12) * E + 1 +
                                           3 * R + regions * 3 * R * S + 2 * P);
    // the load's scan first uses the same LDS for its partial sums (two
    // per thread when experts are taken in pairs)
    const size_t scan = static_cast<size_t>(2 * kPlanBlock) * sizeof(int32_t);
    return plan > scan ? plan : scan;
}

// The limit only rises (the largest need so far), so a context or call
// with a smaller need never lowers what another one relies on.
hipError_t plan_prepare(size_t lds_bytes) {
    static std::mutex mu;
    static size_t granted = 0;
    std::lock_guard<std::mutex> lock(mu);
    if (lds_bytes <= granted) return hipSuccess;
    hipError_t e = hipFuncSetAttribute(
        reinterpret_cast<const void *>(&k_plan<false>),
        hipFuncAttributeMaxDynamicSharedMemorySize,
        static_cast<int>(lds_bytes));
    if (e == hipSuccess)
        e = hipFuncSetAttribute(
            reinterpret_cast<const void *>(&k_plan<true>),
            hipFuncAttributeMaxDynamicSharedMemorySize,
            static_cast<int>(lds_bytes));
    if (e == hipSuccess) granted = lds_bytes;
    return e;
}

static hipError_t launch(const ue_ctx &c, const int32_t *counts, int L,
                         int32_t *placement, int mode, const ScanArgs &sc,
                         hipStream_t s) {
    // spread the quota search when its passes are long (more than 64
    // receiving ranks: at 64 or fewer a pass takes a few microseconds, and
    // the exchange costs what the spread saves) and the layers' workgroups
    // then fit the device one per CU, with pass slots for all of them
    SplitArgs sp{1, c.plan_xrec, c.plan_xflag, c.plan_xcnt};
    if ((mode & kModePlan) && c.plan_xrec && c.R > 64 &&
        c.cfg.quota_mode == UE_QUOTA_SEARCH) {
        for (const int cand : {16, 4}) {
            if (static_cast<int64_t>(L) * cand <= c.num_cu &&
                static_cast<int64_t>(L) * cand * kSplitWaves <= c.plan_xslots) {
                sp.split = cand;
                break;
            }
        }
    }
    auto kernel = sp.split > 1 ? k_plan<true> : k_plan<false>;
    hipLaunchKernelGGL(kernel, dim3(L * sp.split), dim3(kPlanBlock), c.plan_lds, s,
                       counts, c.E, c.R, c.S, c.N, c.NS, c.P, c.rbits,
                       static_cast<int>(c.cfg.plan_policy),
                       static_cast<int>(c.cfg.quota_mode),
                       c.plan_per_wave ? 1 : 0,
                       static_cast<uint32_t>(c.plan_lds), c.lay, placement,
                       mode, sc, sp);
    return hipGetLastError();
}

hipError_t launch_plan(const ue_ctx &c, const int32_t *counts, int L,
                       int32_t *placement, hipStream_t s) {
    return launch(c, counts, L, placement, kModePlan, ScanArgs{}, s);
}

hipError_t launch_scan(const ue_ctx &c, int L, int64_t A, int32_t *counts,
                       int32_t *invalid, int32_t *placement,
                       int32_t *rank_counts, int32_t *faults, hipStream_t s) {
    const LoadShape sh = load_shape(A, L);
    ScanArgs sc;
    sc.rows = c.tile_off;
    sc.group_base = c.group_base;
    sc.A = A;
    sc.tiles = sh.tiles;
    sc.group = sh.group;
    sc.row_stride = sh.tiles + sh.groups;
    sc.groups = sh.groups;
    sc.counts = counts;
    sc.invalid = invalid;
    sc.rank_counts = placement ? rank_counts : nullptr;
    sc.faults = placement ? faults : nullptr;
    return launch(c, counts, L, placement,
                  kModeScan | (placement ? kModePlan : 0), sc, s);
}

}  // namespace ue
