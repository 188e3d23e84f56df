/*
 * ue_oracle.c -- plain, sequential CPU reference for the per-layer MoE
 * expert-rebalancing path: exact expert load, quota replica planning,
 * logical -> physical reroute, and the stable dispatch layout.
 *
 * TEST INFRASTRUCTURE. Only the test suite, the smoke check and the CPU
 * baseline leg of the benchmark load this file's library. The product
 * library (the HIP path) never links, loads or calls it, and the two share
 * no source, header, table or helper.
 *
 * What is computed, and where it comes from:
 *  - UltraEP (arXiv 2606.04101) abstract: the balancer is "exact-load",
 *    i.e. it works from the true per-expert token count of the current
 *    routing, not from history.
 *  - "How dots-infra/ultraep works" (gitdiagram), summary and connection
 *    list: the framework passes post-gating routing; the manager profiles
 *    loads, updates placement (plans replicas), syncs weights, then expands
 *    routing to physical routing for token dispatch.
 *  - UltraEP news write-up ("balansirovka MoE-ekspertov za 300 mks"),
 *    section on how the 300 us balancing works: a quota-driven scheduler
 *    rebalances every microbatch and every layer right after gating.
 *  The pages give no quota formula, tie-break or slot model. The rule here
 *  is the plainest reading consistent with them:
 *    quota Q = ceil(sum(counts) / R);
 *    expert e lives natively on rank e*R/E (= e / N with N = E/R experts
 *    per rank), in slot e mod N; each rank also owns S empty spare slots;
 *    physical slot id p = r*(N+S) + s (natives 0..N-1, spares N..N+S-1);
 *    experts of overloaded ranks (load > Q) are visited heaviest first
 *    (count desc, id asc); each spills its rank's excess, chunk by chunk,
 *    into a spare slot of the least-loaded rank (ties: lowest rank id) that
 *    has a free spare slot and load < Q; a chunk is the smallest of the
 *    source's excess, the expert's remaining tokens and the destination's
 *    headroom; if no destination exists the plan stops ("exhausted");
 *    the j-th assignment of expert e, in flat (token, slot) order, goes to
 *    the replica whose capacity prefix covers j (master first, then replicas
 *    in creation order);
 *    the dispatch permutation is the stable counting sort by physical slot.
 *  Four variants, each one step different (see Step 2): best fit for a
 *  remainder the least-loaded rank would not fill; best fit with the
 *  candidates visited in covering order (amounts one rank can take first,
 *  smallest first, then the rest, largest first); best fit with the
 *  candidates visited by ascending amount; and a quota search that raises
 *  Q in small steps until the plan is no longer exhausted.
 *
 * Everything is integer; there is nothing to round.
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ---------------------------------------------------------------------- */
/* Step 1. Exact per-expert load: counts[e] = number of assignments whose
 * logical expert id is e. Ids outside [0, E) are not counted; the number
 * of such ids is returned. */
int64_t orc_load(const int32_t *routing, int64_t n_assign, int32_t n_experts,
                 int32_t *counts)
{
    int64_t invalid = 0;
    for (int32_t e = 0; e < n_experts; ++e)
        counts[e] = 0;
    for (int64_t a = 0; a < n_assign; ++a) {
        int32_t e = routing[a];
        if (e < 0 || e >= n_experts) {
            ++invalid;
            continue;
        }
        counts[e] += 1;
    }
    return invalid;
}

/* ---------------------------------------------------------------------- */
/* Step 2. Quota plan for one layer.
 *
 * policy 0: every chunk goes to the least-loaded eligible rank (the rule
 * stated above). policy 1 (best fit): when that rank would be left with
 * room to spare, the chunk goes to the eligible rank with the smallest
 * headroom that still takes all of it, ties to the lowest id. policy 2:
 * policy 1's destinations, candidates in covering order (greedy_cover_at).
 * policy 3: policy 1's destinations, candidates by ascending amount
 * (greedy_cover_at with `ascending`).
 *
 * quota_mode 0: Q = ceil(sum(counts) / R). quota_mode 1 (quota search):
 * with one spare slot a rank takes one chunk, so a chunk that leaves a
 * destination part full wastes the rest of its headroom, while the ranks
 * below Q0 = ceil(sum / R) hold, together, only the sources' excess plus
 * less than R of slack; the plan at Q0 then almost always stops with
 * excess left. The search raises the quota in steps of ceil(Q0 / 256) and
 * keeps the lowest of Q0, Q0 + step, ..., Q0 + 63 step at which nothing is
 * left (the scheduler is quota-driven; the pages do not say how the quota
 * is set). With none, Q0 stands.
 *
 * scalars[0] = quota Q (the one used)
 * scalars[1] = exhausted (1 if an overloaded rank still had excess but no
 *              rank was left with a free spare slot and load < Q)
 * scalars[2] = residual = sum over ranks of max(0, load_after - Q)
 * scalars[3] = n_rep, number of replica-table entries (masters included)
 *
 * Replica table (CSR by expert): entries rep_off[e] .. rep_off[e+1]-1 of
 * rep_slot / rep_cap are the replicas of e; the first is always the native
 * (master) slot, the rest follow in creation order. Entries at and after
 * n_rep (the table has room for P = R*(N+S) entries) hold slot -1, cap 0.
 *
 * Slot tables over the P physical slots: slot_expert[p] is the expert held
 * by p (-1 for an unused spare), slot_cap[p] its capacity (0 if unused),
 * slot_off the exclusive prefix sum of slot_cap (P+1 entries).
 *
 * Returns 0, or -1 if the shape is not one the slot model covers. */
/* Native placement: every rank's load is the sum of its N native experts'
 * counts; every expert still holds all its tokens; every rank has all S
 * spare slots free. */
static void native_state(const int32_t *counts, int32_t E, int32_t R,
                         int32_t S, int64_t *load, int64_t *rem,
                         int32_t *nfree)
{
    const int32_t N = E / R;
    for (int32_t r = 0; r < R; ++r) {
        load[r] = 0;
        nfree[r] = S;
    }
    for (int32_t e = 0; e < E; ++e) {
        load[e / N] += counts[e];
        rem[e] = counts[e];
    }
}

/* Destination of an amount m: the least-loaded rank with a free spare slot
 * and load below Q (ties: lowest id), or -1 if there is none. With best
 * fit, when that rank could take the whole amount with room to spare, the
 * eligible rank whose headroom is the smallest that still holds it (the
 * most loaded such rank; ties: lowest id). */
static int32_t pick_destination(const int64_t *load, const int32_t *nfree,
                                int32_t R, int64_t Q, int64_t m, int best_fit)
{
    /* ascending scan with a strict comparison keeps the lowest rank id
     * among ties */
    int32_t d = -1;
    for (int32_t x = 0; x < R; ++x) {
        if (nfree[x] <= 0 || load[x] >= Q)
            continue;
        if (d < 0 || load[x] < load[d])
            d = x;
    }
    if (d >= 0 && best_fit && m < Q - load[d]) {
        int32_t b = d;
        for (int32_t x = 0; x < R; ++x) {
            if (nfree[x] > 0 && load[x] < Q && Q - load[x] >= m &&
                load[x] > load[b])
                b = x;
        }
        d = b;
    }
    return d;
}

/* Moves a chunk of expert e (home rank r) into d's lowest free spare slot:
 * the amount m capped by d's headroom. Records (expert, slot, chunk) and
 * returns the chunk. */
static int64_t place_chunk(int32_t e, int32_t r, int32_t d, int64_t m,
                           int64_t Q, int32_t N, int32_t S, int64_t *load,
                           int64_t *rem, int32_t *nfree, int32_t *rec_e,
                           int32_t *rec_p, int64_t *rec_m, int32_t *nrec)
{
    if (Q - load[d] < m)
        m = Q - load[d];
    rec_e[*nrec] = e;
    rec_p[*nrec] = d * (N + S) + N + (S - nfree[d]);
    rec_m[*nrec] = m;
    ++*nrec;
    rem[e] -= m;
    load[r] -= m;
    load[d] += m;
    nfree[d] -= 1;
    return m;
}

/* One greedy pass at quota Q for policies 0 and 1: native loads,
 * candidates, spill loop. Fills load, rem, nfree and the spill records;
 * returns 1 if the plan stopped with excess left (exhausted), else 0. */
static int greedy_at(const int32_t *counts, int32_t E, int32_t R, int32_t S,
                     int32_t policy, int64_t Q, int64_t *load, int64_t *rem,
                     int32_t *nfree, int32_t *cand, int32_t *rec_e,
                     int32_t *rec_p, int64_t *rec_m, int32_t *nrec_out)
{
    const int32_t N = E / R;
    native_state(counts, E, R, S, load, rem, nfree);

    /* Candidates: experts of overloaded ranks, heaviest first (count desc,
     * id asc). Plain insertion sort. */
    int32_t ncand = 0;
    for (int32_t e = 0; e < E; ++e) {
        if (load[e / N] <= Q)
            continue;
        int32_t i = ncand++;
        while (i > 0) {
            int32_t prev = cand[i - 1];
            int before = counts[prev] > counts[e] ||
                         (counts[prev] == counts[e] && prev < e);
            if (before)
                break;
            cand[i] = prev;
            --i;
        }
        cand[i] = e;
    }

    /* Spill loop: the amount is the smallest of the source's excess and
     * the expert's remaining tokens. */
    int exhausted = 0;
    int32_t nrec = 0;
    for (int32_t c = 0; c < ncand && !exhausted; ++c) {
        const int32_t e = cand[c];
        const int32_t r = e / N;
        while (load[r] > Q && rem[e] > 0) {
            int64_t m = load[r] - Q;
            if (rem[e] < m)
                m = rem[e];
            const int32_t d = pick_destination(load, nfree, R, Q, m,
                                               policy == 1);
            if (d < 0) {
                exhausted = 1;
                break;
            }
            place_chunk(e, r, d, m, Q, N, S, load, rem, nfree, rec_e, rec_p,
                        rec_m, &nrec);
        }
    }
    *nrec_out = nrec;
    return exhausted;
}

/* Each expert's amount at quota M: a rank above M sheds its excess from
 * its experts heaviest first (count desc, id asc), each giving what it has
 * of what is still left (0 for experts of other ranks). The next expert is
 * the heaviest of those after the previous one in that order. */
static void amounts_at(const int32_t *counts, int32_t E, int32_t R,
                       const int64_t *load, int64_t M, int64_t *amt)
{
    const int32_t N = E / R;
    for (int32_t r = 0; r < R; ++r) {
        int64_t left = load[r] - M;
        int32_t prev = -1;
        for (int32_t k = 0; k < N; ++k) {
            int32_t best = -1;
            for (int32_t i = 0; i < N; ++i) {
                const int32_t e = r * N + i;
                const int after = prev < 0 || counts[e] < counts[prev] ||
                                  (counts[e] == counts[prev] && e > prev);
                if (!after)
                    continue;
                if (best < 0 || counts[e] > counts[best])
                    best = e;
            }
            prev = best;
            amt[best] = left > 0 ? (counts[best] < left ? counts[best] : left)
                                 : 0;
            left -= amt[best];
        }
    }
}

/* Policy 2 (best fit in covering order): the destination rule of policy 1,
 * with the candidates visited in another order. With one spare slot per
 * rank a destination takes one chunk, so the destinations are pieces that
 * the sources' excesses must cover; a large excess spends the big pieces,
 * and a small excess that comes last finds only big pieces, or none. So
 * the amounts that one rank can take are placed first, smallest first,
 * then the others, largest first. The order is fixed once, from the plain
 * quota Q0:
 *   - every expert of a rank whose load exceeds Q0 is a candidate;
 *   - its amount at a quota M is given by amounts_at;
 *   - H0 is the largest headroom Q0 - load among ranks with a spare slot
 *     and load below Q0 (0 if there is none);
 *   - candidates with amount at Q0 at most H0 come first, by (amount asc,
 *     id asc); then the others, by (amount desc, id asc).
 * At the pass's quota Q each candidate in that order places its amount at
 * Q, chunk by chunk, into the destination policy 1 would choose.
 *
 * Policy 3 (best fit, ascending amounts; `ascending` set): the same, with
 * every candidate in one order, (amount at Q0 asc, id asc). The large
 * amounts then also go smallest first: each takes the big pieces that
 * remain after the smaller ones, and the largest amounts, which need many
 * pieces in any order, come last and split over what is left. */
static int greedy_cover_at(const int32_t *counts, int32_t E, int32_t R,
                           int32_t S, int ascending, int64_t Q0, int64_t Q,
                           int64_t *load,
                           int64_t *rem, int32_t *nfree, int32_t *cand,
                           int32_t *rec_e, int32_t *rec_p, int64_t *rec_m,
                           int32_t *nrec_out, int64_t *amt0, int64_t *amt)
{
    const int32_t N = E / R;
    native_state(counts, E, R, S, load, rem, nfree);
    amounts_at(counts, E, R, load, Q0, amt0);
    amounts_at(counts, E, R, load, Q, amt);
    int64_t H0 = 0;
    for (int32_t r = 0; r < R; ++r)
        if (S > 0 && load[r] < Q0 && Q0 - load[r] > H0)
            H0 = Q0 - load[r];

    /* candidates in covering order (insertion sort on the key above) */
    int32_t ncand = 0;
    for (int32_t e = 0; e < E; ++e) {
        if (load[e / N] <= Q0)
            continue;
        int32_t i = ncand++;
        while (i > 0) {
            const int32_t p = cand[i - 1];
            const int gp = amt0[p] > H0, ge = amt0[e] > H0;
            int before;
            if (ascending)
                before = amt0[p] != amt0[e] ? amt0[e] > amt0[p] : p < e;
            else if (gp != ge)
                before = gp < ge;
            else if (amt0[p] != amt0[e])
                before = ge ? amt0[p] > amt0[e] : amt0[p] < amt0[e];
            else
                before = p < e;
            if (before)
                break;
            cand[i] = p;
            --i;
        }
        cand[i] = e;
    }

    int exhausted = 0;
    int32_t nrec = 0;
    for (int32_t c = 0; c < ncand && !exhausted; ++c) {
        const int32_t e = cand[c];
        int64_t need = amt[e];
        while (need > 0) {
            const int32_t d = pick_destination(load, nfree, R, Q, need, 1);
            if (d < 0) {
                exhausted = 1;
                break;
            }
            need -= place_chunk(e, e / N, d, need, Q, N, S, load, rem, nfree,
                                rec_e, rec_p, rec_m, &nrec);
        }
    }
    *nrec_out = nrec;
    return exhausted;
}

/* One pass of the policy's rule at quota M (Q0: the plain quota). */
static int pass_at(int32_t policy, const int32_t *counts, int32_t E,
                   int32_t R, int32_t S, int64_t Q0, int64_t M, int64_t *load,
                   int64_t *rem, int32_t *nfree, int32_t *cand,
                   int32_t *rec_e, int32_t *rec_p, int64_t *rec_m,
                   int32_t *nrec, int64_t *amt0, int64_t *amt)
{
    if (policy >= 2)
        return greedy_cover_at(counts, E, R, S, policy == 3, Q0, M, load,
                               rem, nfree, cand, rec_e, rec_p, rec_m, nrec,
                               amt0, amt);
    return greedy_at(counts, E, R, S, policy, M, load, rem, nfree, cand,
                     rec_e, rec_p, rec_m, nrec);
}

int orc_plan(const int32_t *counts, int32_t E, int32_t R, int32_t S,
             int32_t policy, int32_t quota_mode, int32_t *scalars,
             int32_t *rep_off, int32_t *rep_slot, int32_t *rep_cap,
             int32_t *slot_expert, int32_t *slot_cap, int32_t *slot_off,
             int32_t *load_before, int32_t *load_after)
{
    if (E <= 0 || R <= 0 || S < 0 || E % R != 0 || policy < 0 || policy > 3)
        return -1;
    const int32_t N = E / R;       /* native experts per rank */
    const int32_t NS = N + S;      /* physical slots per rank */
    const int32_t P = R * NS;      /* physical slots in total */

    int64_t *load = calloc((size_t)R, sizeof(int64_t));
    int64_t *rem = calloc((size_t)E, sizeof(int64_t));
    int32_t *nfree = calloc((size_t)R, sizeof(int32_t));
    int32_t *cand = calloc((size_t)E, sizeof(int32_t));
    /* spill records in creation order: expert, slot, amount */
    int32_t *rec_e = calloc((size_t)(R * S + 1), sizeof(int32_t));
    int32_t *rec_p = calloc((size_t)(R * S + 1), sizeof(int32_t));
    int64_t *rec_m = calloc((size_t)(R * S + 1), sizeof(int64_t));
    /* policies 2, 3: each candidate's amount at Q0 and at the pass's quota */
    int64_t *amt0 = calloc((size_t)E, sizeof(int64_t));
    int64_t *amt = calloc((size_t)E, sizeof(int64_t));
    if (!load || !rem || !nfree || !cand || !rec_e || !rec_p || !rec_m ||
        !amt0 || !amt) {
        free(load); free(rem); free(nfree); free(cand);
        free(rec_e); free(rec_p); free(rec_m); free(amt0); free(amt);
        return -1;
    }

    /* Plain quota and the native rank loads. */
    int64_t total = 0;
    for (int32_t e = 0; e < E; ++e)
        total += counts[e];
    const int64_t Q0 = (total + R - 1) / R;
    for (int32_t r = 0; r < R; ++r) {
        int64_t l = 0;
        for (int32_t i = 0; i < N; ++i)
            l += counts[r * N + i];
        load_before[r] = (int32_t)l;
    }

    /* Quota search (quota_mode 1): the quotas Q0 + j * ceil(Q0 / 256),
     * j = 0 .. 63, are tried in increasing order, and the first at which
     * the greedy pass places every excess is kept; if none does, the plain
     * quota Q0 stands. */
    int64_t Q = Q0;
    int32_t nrec = 0;
    if (quota_mode == 1) {
        const int64_t step = (Q0 + 255) / 256;
        for (int32_t j = 0; j < 64; ++j) {
            const int64_t M = Q0 + j * step;
            if (!pass_at(policy, counts, E, R, S, Q0, M, load, rem, nfree,
                         cand, rec_e, rec_p, rec_m, &nrec, amt0, amt)) {
                Q = M;
                break;
            }
        }
    }
    const int exhausted = pass_at(policy, counts, E, R, S, Q0, Q, load, rem,
                                  nfree, cand, rec_e, rec_p, rec_m, &nrec,
                                  amt0, amt);

    /* Replica table: master first (keeps what was not spilled), then the
     * spilled replicas in creation order. */
    int32_t n = 0;
    for (int32_t e = 0; e < E; ++e) {
        rep_off[e] = n;
        rep_slot[n] = (e / N) * NS + (e % N);
        rep_cap[n] = (int32_t)rem[e];
        ++n;
        for (int32_t i = 0; i < nrec; ++i) {
            if (rec_e[i] != e)
                continue;
            rep_slot[n] = rec_p[i];
            rep_cap[n] = (int32_t)rec_m[i];
            ++n;
        }
    }
    rep_off[E] = n;
    for (int32_t i = n; i < P; ++i) {
        rep_slot[i] = -1;
        rep_cap[i] = 0;
    }

    /* Slot tables. */
    for (int32_t p = 0; p < P; ++p) {
        slot_expert[p] = -1;
        slot_cap[p] = 0;
    }
    for (int32_t e = 0; e < E; ++e) {
        for (int32_t i = rep_off[e]; i < rep_off[e + 1]; ++i) {
            slot_expert[rep_slot[i]] = e;
            slot_cap[rep_slot[i]] = rep_cap[i];
        }
    }
    slot_off[0] = 0;
    for (int32_t p = 0; p < P; ++p)
        slot_off[p + 1] = slot_off[p] + slot_cap[p];

    int64_t residual = 0;
    for (int32_t r = 0; r < R; ++r) {
        load_after[r] = (int32_t)load[r];
        if (load[r] > Q)
            residual += load[r] - Q;
    }
    scalars[0] = (int32_t)Q;
    scalars[1] = exhausted;
    scalars[2] = (int32_t)residual;
    scalars[3] = n;

    free(load); free(rem); free(nfree); free(cand);
    free(rec_e); free(rec_p); free(rec_m); free(amt0); free(amt);
    return 0;
}

/* ---------------------------------------------------------------------- */
/* Step 3. Reroute and dispatch layout for one layer.
 *
 * For every assignment a in flat (token, slot) order with logical expert
 * e = routing[a]: j = number of earlier assignments of e; the replica i of
 * e whose capacity prefix covers j receives it:
 *     phys[a]     = rep_slot[i]
 *     pos         = slot_off[phys[a]] + (j - prefix_i)
 *     perm[pos]   = a,  inv_perm[a] = pos
 * rank_counts[r] counts the assignments whose physical slot is on rank r.
 *
 * Assignments with an id outside [0, E), beyond the plan's capacity for
 * their expert, or whose position would fall outside [0, n_assign) (a plan
 * made for other counts), get phys = -1 and inv_perm = -1, and are counted
 * in the return value; perm entries nobody fills keep whatever the caller put
 * there. */
int64_t orc_reroute(const int32_t *routing, int64_t n_assign, int32_t E,
                    int32_t R, int32_t S, const int32_t *rep_off,
                    const int32_t *rep_slot, const int32_t *rep_cap,
                    const int32_t *slot_off, int32_t *phys, int32_t *perm,
                    int32_t *inv_perm, int32_t *rank_counts)
{
    const int32_t N = E / R;
    const int32_t NS = N + S;
    int64_t *seen = calloc((size_t)E, sizeof(int64_t));
    if (!seen)
        return -1;
    int64_t faults = 0;
    for (int32_t r = 0; r < R; ++r)
        rank_counts[r] = 0;

    for (int64_t a = 0; a < n_assign; ++a) {
        const int32_t e = routing[a];
        phys[a] = -1;
        inv_perm[a] = -1;
        if (e < 0 || e >= E) {
            ++faults;
            continue;
        }
        const int64_t j = seen[e]++;
        int64_t prefix = 0;
        int32_t hit = -1;
        for (int32_t i = rep_off[e]; i < rep_off[e + 1]; ++i) {
            if (j < prefix + rep_cap[i]) {
                hit = i;
                break;
            }
            prefix += rep_cap[i];
        }
        if (hit < 0) {
            ++faults;
            continue;
        }
        const int32_t p = rep_slot[hit];
        const int64_t pos = slot_off[p] + (j - prefix);
        if (pos < 0 || pos >= n_assign) {
            ++faults;
            continue;
        }
        phys[a] = p;
        perm[pos] = (int32_t)a;
        inv_perm[a] = (int32_t)pos;
        rank_counts[p / NS] += 1;
    }
    free(seen);
    return faults;
}
