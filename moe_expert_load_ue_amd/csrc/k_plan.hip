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
//
// Layout of the work:
//   A. all 256 threads: counts and rank loads into LDS, the quota, the
//      candidate list (compacted in id order, then ranked by comparison
//      counting, which is exact and needs no sort network);
//   B. wave 0 alone: the sequential spill loop. Each lane owns ranks
//      lane, lane+64, ... and caches the smallest key (load << rbits | rank)
//      among its eligible ranks; one DPP min-reduction per chunk picks the
//      destination, and only the owner lane of that rank refreshes its key;
//   C. all threads: replica table (CSR) and slot tables by prefix sums.
// Everything is integer and deterministic; the result does not depend on
// scheduling.
#include "ue_internal.h"

namespace ue {
namespace {

struct PlanLds {
    int32_t *cnt, *rem, *load, *nfree, *cand, *sorted, *first_rec, *nrec_e;
    int32_t *rec_e, *rec_p, *rec_m, *slot_cap, *slot_exp, *rep_off;
};

__device__ __forceinline__ int32_t *carve_end(const PlanLds &s, int P) {
    return s.slot_exp + P;
}

__device__ __forceinline__ PlanLds carve(int32_t *base, int E, int R, int P) {
    PlanLds s;
    int32_t *p = base;
    s.cnt = p; p += E;
    s.rem = p; p += E;
    s.cand = p; p += E;
    s.sorted = p; p += E;
    s.first_rec = p; p += E;
    s.nrec_e = p; p += E;
    s.rep_off = p; p += E + 1;
    s.load = p; p += R;
    s.nfree = p; p += R;
    s.rec_e = p; p += P;
    s.rec_p = p; p += P;
    s.rec_m = p; p += P;
    s.slot_cap = p; p += P;
    s.slot_exp = p; p += P;
    return s;
}

// Exclusive scan of `n` ints in place in LDS (n up to a few thousand);
// returns the total. Every thread must call it.
__device__ int block_scan_inplace(int32_t *data, int n, int *wsum) {
    const int tid = threadIdx.x;
    const int per = (n + kBlock - 1) / kBlock;
    const int b = tid * per;
    const int e = (b + per < n) ? b + per : n;
    int local = 0;
    for (int i = b; i < e; ++i) local += data[i];
    int total;
    int run = block_exclusive_sum(local, wsum, total);
    for (int i = b; i < e; ++i) {
        const int v = data[i];
        data[i] = run;
        run += v;
    }
    __syncthreads();
    return total;
}

// Per-lane register state of the ranks a lane owns (lane, lane+64, ...),
// read and written with a wave-uniform slot index through unrolled selects.
template <int RPL>
struct RankRegs {
    int load[RPL];
    int nfree[RPL];

    __device__ __forceinline__ int get_load(int k) const {
        int v = 0;
#pragma unroll
        for (int i = 0; i < RPL; ++i) v = (i == k) ? load[i] : v;
        return v;
    }
    __device__ __forceinline__ int get_free(int k) const {
        int v = 0;
#pragma unroll
        for (int i = 0; i < RPL; ++i) v = (i == k) ? nfree[i] : v;
        return v;
    }
    // smallest key (load << rbits | rank) among this lane's eligible ranks
    __device__ __forceinline__ uint32_t key(int lane, int R, int Q,
                                            int rbits) const {
        uint32_t best = 0xFFFFFFFFu;
#pragma unroll
        for (int i = 0; i < RPL; ++i) {
            const int r = lane + 64 * i;
            const uint32_t k = (static_cast<uint32_t>(load[i]) << rbits) |
                               static_cast<uint32_t>(r);
            const bool ok = r < R && nfree[i] > 0 && load[i] < Q;
            best = (ok && k < best) ? k : best;
        }
        return best;
    }
};

// The spill loop, run by wave 0 alone. Everything that decides the next
// step is wave-uniform: the candidate, its rank's load, the expert's
// remainder and the reduced minimum key. Only the lane owning the chosen
// destination changes its registers and refreshes its cached key.
template <int RPL>
__device__ void spill_loop(PlanLds &s, int ncand, int R, int S, int N, int NS,
                           int Q, int rbits, int &nrec_out,
                           int &exhausted_out) {
    const int lane = threadIdx.x & 63;
    RankRegs<RPL> st;
#pragma unroll
    for (int i = 0; i < RPL; ++i) {
        const int r = lane + 64 * i;
        st.load[i] = r < R ? s.load[r] : 0;
        st.nfree[i] = r < R ? S : 0;
    }
    uint32_t my_key = st.key(lane, R, Q, rbits);
    const uint32_t rmask = (1u << rbits) - 1u;
    const int max_rec = R * S;
    int nrec = 0;
    int exhausted = 0;
    for (int c = 0; c < ncand && !exhausted; ++c) {
        const int e = __builtin_amdgcn_readfirstlane(s.sorted[c]);
        const int r = e / N;
        int Lr = __builtin_amdgcn_readlane(st.get_load(r >> 6), r & 63);
        int rem_e = __builtin_amdgcn_readfirstlane(s.rem[e]);
        const int first = nrec;
        while (Lr > Q && rem_e > 0) {
            // each chunk takes one spare slot: with all R*S taken no rank
            // is eligible (this also bounds the loop whatever the keys hold)
            const uint32_t best =
                nrec < max_rec ? wave_min_u32(my_key) : 0xFFFFFFFFu;
            if (best == 0xFFFFFFFFu) {
                exhausted = 1;
                break;
            }
            const int d = static_cast<int>(best & rmask);
            const int Ld = static_cast<int>(best >> rbits);
            int m = Lr - Q;
            m = rem_e < m ? rem_e : m;
            m = (Q - Ld) < m ? (Q - Ld) : m;
            const int dk = d >> 6;
            const int fr = __builtin_amdgcn_readlane(st.get_free(dk), d & 63);
            const int p = d * NS + N + (S - fr);
            if (lane == 0) {
                s.rec_e[nrec] = e;
                s.rec_p[nrec] = p;
                s.rec_m[nrec] = m;
            }
            ++nrec;
            rem_e -= m;
            Lr -= m;
            if (lane == (d & 63)) {
#pragma unroll
                for (int i = 0; i < RPL; ++i) {
                    if (i == dk) {
                        st.load[i] = Ld + m;
                        st.nfree[i] -= 1;
                    }
                }
                my_key = st.key(lane, R, Q, rbits);
            }
        }
        if (lane == (r & 63)) {
#pragma unroll
            for (int i = 0; i < RPL; ++i)
                if (i == (r >> 6)) st.load[i] = Lr;
        }
        if (lane == 0) {
            s.rem[e] = rem_e;
            s.first_rec[e] = first;
            s.nrec_e[e] = nrec - first;
        }
    }
#pragma unroll
    for (int i = 0; i < RPL; ++i) {
        const int r = lane + 64 * i;
        if (r < R) s.load[r] = st.load[i];
    }
    nrec_out = nrec;
    exhausted_out = exhausted;
}

__global__ __launch_bounds__(kBlock) void k_plan(
    const int32_t *__restrict__ counts, int E, int R, int S, int N, int NS,
    int P, int rbits, uint32_t lds_bytes, ue_placement_layout lay,
    int32_t *__restrict__ placement) {
    extern __shared__ int32_t lds[];
    __shared__ int wsum[kWaves];
    __shared__ int s_ncand, s_nrec, s_exhausted, s_quota;

    const int layer = blockIdx.x;
    const int tid = threadIdx.x;
    const int32_t *cin = counts + static_cast<int64_t>(layer) * E;
    int32_t *out = placement + static_cast<int64_t>(layer) * lay.words;
    PlanLds s = carve(lds, E, R, P);
    // the carve-up must fit the launch's LDS (checked, not assumed); a
    // mismatch marks the block (exhausted = -1) rather than pass silently
    if (static_cast<size_t>(carve_end(s, P) - lds) * 4 > lds_bytes) {
        if (tid == 0) out[lay.exhausted] = -1;
        return;
    }

    // ---- A. loads, quota, candidates ----------------------------------
    int part = 0;
    for (int e = tid; e < E; e += kBlock) {
        const int c = cin[e];
        s.cnt[e] = c;
        s.rem[e] = c;
        s.nrec_e[e] = 0;
        s.first_rec[e] = 0;
        part += c;
    }
    int total;
    block_exclusive_sum(part, wsum, total);   // barrier: cnt visible
    const int Q = (total + R - 1) / R;
    for (int r = tid; r < R; r += kBlock) {
        int l = 0;
        for (int i = 0; i < N; ++i) l += s.cnt[r * N + i];
        s.load[r] = l;
        s.nfree[r] = S;
        out[lay.load_before + r] = l;
    }
    __syncthreads();

    // candidates in id order: experts whose home rank is above quota
    {
        const int per = (E + kBlock - 1) / kBlock;
        const int b = tid * per;
        const int e_end = (b + per < E) ? b + per : E;
        int local = 0;
        for (int e = b; e < e_end; ++e) local += (s.load[e / N] > Q);
        int n;
        int pos = block_exclusive_sum(local, wsum, n);
        for (int e = b; e < e_end; ++e)
            if (s.load[e / N] > Q) s.cand[pos++] = e;
        if (tid == 0) s_ncand = n;
    }
    __syncthreads();
    const int ncand = s_ncand;
    // rank each candidate by (count desc, id asc)
    for (int i = tid; i < ncand; i += kBlock) {
        const int e = s.cand[i];
        const int c = s.cnt[e];
        int pos = 0;
        for (int j = 0; j < ncand; ++j) {
            const int f = s.cand[j];
            const int cf = s.cnt[f];
            pos += (cf > c) || (cf == c && f < e);
        }
        s.sorted[pos] = e;
    }
    __syncthreads();

    // ---- B. sequential spill loop on wave 0 ------------------------------
    if (tid < 64) {
        int nrec = 0, exhausted = 0;
        switch ((R + 63) / 64) {
            case 1: spill_loop<1>(s, ncand, R, S, N, NS, Q, rbits, nrec, exhausted); break;
            case 2: spill_loop<2>(s, ncand, R, S, N, NS, Q, rbits, nrec, exhausted); break;
            case 3:
            case 4: spill_loop<4>(s, ncand, R, S, N, NS, Q, rbits, nrec, exhausted); break;
            case 5: case 6: case 7:
            case 8: spill_loop<8>(s, ncand, R, S, N, NS, Q, rbits, nrec, exhausted); break;
            default: spill_loop<16>(s, ncand, R, S, N, NS, Q, rbits, nrec, exhausted); break;
        }
        if (tid == 0) {
            s_nrec = nrec;
            s_exhausted = exhausted;
            s_quota = Q;
        }
    }
    __syncthreads();

    // ---- C. replica table and slot tables --------------------------------
    const int nrec = s_nrec;
    for (int e = tid; e < E; e += kBlock) s.rep_off[e] = 1 + s.nrec_e[e];
    __syncthreads();
    const int n_rep = block_scan_inplace(s.rep_off, E, wsum);
    for (int e = tid; e < E; e += kBlock) {
        const int base = s.rep_off[e];
        out[lay.rep_off + e] = base;
        out[lay.rep_slot + base] = (e / N) * NS + (e % N);
        out[lay.rep_cap + base] = s.rem[e];
        const int f = s.first_rec[e];
        const int n = s.nrec_e[e];
        for (int i = 0; i < n; ++i) {
            out[lay.rep_slot + base + 1 + i] = s.rec_p[f + i];
            out[lay.rep_cap + base + 1 + i] = s.rec_m[f + i];
        }
    }
    if (tid == 0) out[lay.rep_off + E] = n_rep;
    for (int i = n_rep + tid; i < P; i += kBlock) {
        out[lay.rep_slot + i] = -1;
        out[lay.rep_cap + i] = 0;
    }
    for (int p = tid; p < P; p += kBlock) {
        s.slot_cap[p] = 0;
        s.slot_exp[p] = -1;
    }
    __syncthreads();
    for (int e = tid; e < E; e += kBlock) {
        const int p = (e / N) * NS + (e % N);
        s.slot_exp[p] = e;
        s.slot_cap[p] = s.rem[e];
    }
    for (int i = tid; i < nrec; i += kBlock) {
        s.slot_exp[s.rec_p[i]] = s.rec_e[i];
        s.slot_cap[s.rec_p[i]] = s.rec_m[i];
    }
    __syncthreads();
    for (int p = tid; p < P; p += kBlock) {
        out[lay.slot_expert + p] = s.slot_exp[p];
        out[lay.slot_cap + p] = s.slot_cap[p];
    }
    __syncthreads();
    const int slot_total = block_scan_inplace(s.slot_cap, P, wsum);
    for (int p = tid; p < P; p += kBlock) out[lay.slot_off + p] = s.slot_cap[p];
    int resid = 0;
    for (int r = tid; r < R; r += kBlock) {
        const int l = s.load[r];
        out[lay.load_after + r] = l;
        resid += (l > Q) ? (l - Q) : 0;
    }
    int resid_total;
    block_exclusive_sum(resid, wsum, resid_total);
    // the block's alignment padding is written too, so a block is fully
    // defined by its counts
    for (int i = lay.load_after + R + tid; i < lay.words; i += kBlock) out[i] = 0;
    if (tid == 0) {
        out[lay.slot_off + P] = slot_total;
        out[lay.quota] = s_quota;
        out[lay.exhausted] = s_exhausted;
        out[lay.residual] = resid_total;
        out[lay.n_rep] = n_rep;
    }
}

}  // namespace

size_t plan_lds_bytes(int E, int R, int P) {
    return sizeof(int32_t) * (static_cast<size_t>(7) * E + 1 + 2 * R + 5 * P);
}

hipError_t plan_prepare(size_t lds_bytes) {
    return hipFuncSetAttribute(reinterpret_cast<const void *>(&k_plan),
                               hipFuncAttributeMaxDynamicSharedMemorySize,
                               static_cast<int>(lds_bytes));
}

hipError_t launch_plan(const ue_ctx &c, const int32_t *counts, int L,
                       int32_t *placement, hipStream_t s) {
    hipLaunchKernelGGL(k_plan, dim3(L), dim3(kBlock), c.plan_lds, s, counts,
                       c.E, c.R, c.S, c.N, c.NS, c.P, c.rbits,
                       static_cast<uint32_t>(c.plan_lds), c.lay, placement);
    return hipGetLastError();
}

}  // namespace ue
