"""Checks that pin the CPU oracle to facts other than itself.

Every check raises AssertionError on failure. They are used twice: against
the oracle as built (``test_oracle_pins.py``) and against copies of the
oracle with a planted mistake (``test_oracle_mutants.py``), which must each
fail at least one check.

Sources of truth, none of them the oracle's own code:
  * hand-worked golden cases under ``tests/golden`` (planning rule read from
    the pages: "quota-driven scheduler", UltraEP news write-up; "plans
    replicas ... expands routing", gitdiagram summary; "exact-load", UltraEP
    abstract);
  * closed forms of degenerate cases (no spare slots, one rank, balanced
    routing, a single hot expert);
  * library routines: ``np.bincount`` for loads, ``np.argsort(kind="stable")``
    for the dispatch permutation, ``np.searchsorted`` for the capacity-prefix
    lookup, ``scipy.sparse.csgraph.maximum_flow`` for optimal placements;
  * invariants any correct plan satisfies (conservation, one replica per
    spare slot, quota respected whenever slots suffice, ...).
"""
from __future__ import annotations

import glob
import itertools
import json
import math
import os

import numpy as np

import oracle

GOLDEN_DIR = os.path.join(os.path.dirname(os.path.abspath(__file__)),
                          "golden")


# --------------------------------------------------------------------------
# golden cases

def golden_cases():
    return [json.load(open(p)) for p in
            sorted(glob.glob(os.path.join(GOLDEN_DIR, "*.json")))]


def _eq(name, got, want):
    got = [int(v) for v in np.asarray(got).reshape(-1)]
    want = [int(v) for v in want]
    assert got == want, f"{name}: got {got}, want {want}"


def check_golden(g):
    if g.get("kind") == "faults":
        check_golden_faults(g)
        return
    pl = oracle.plan(np.asarray(g["counts"], np.int32), g["R"], g["S"],
                     g.get("policy", 0), g.get("quota_mode", 0))
    for key in ("quota", "exhausted", "residual", "n_rep"):
        assert pl[key] == g[key], f"{g['name']}: {key} {pl[key]} != {g[key]}"
    for key in ("load_before", "load_after", "rep_off", "slot_expert",
                "slot_cap", "slot_off"):
        _eq(f"{g['name']}: {key}", pl[key], g[key])
    n = g["n_rep"]
    _eq(f"{g['name']}: rep_slot", pl["rep_slot"][:n], g["rep_slot"])
    _eq(f"{g['name']}: rep_cap", pl["rep_cap"][:n], g["rep_cap"])
    assert np.all(pl["rep_slot"][n:] == -1) and np.all(pl["rep_cap"][n:] == 0)
    if "routing" in g:
        routing = np.asarray(g["routing"], np.int32)
        counts, invalid = oracle.load(routing[None], g["E"])
        _eq(f"{g['name']}: counts", counts[0], g["counts"])
        assert invalid[0] == 0
        rr = oracle.reroute(routing.reshape(-1), pl)
        assert rr["faults"] == 0
        for key in ("phys", "perm", "inv_perm", "rank_counts"):
            _eq(f"{g['name']}: {key}", rr[key], g[key])


PERM_FILL = -777


def check_golden_faults(g):
    """A plan made from other counts applied to routing with ids out of
    range: faulted assignments get phys = inv_perm = -1, take no position,
    and are left out of rank_counts; perm positions nothing fills keep the
    caller's value."""
    pl = oracle.plan(np.asarray(g["plan_counts"], np.int32), g["R"], g["S"],
                     g.get("policy", 0), g.get("quota_mode", 0))
    for key in ("rep_off", "slot_off"):
        _eq(f"{g['name']}: {key}", pl[key], g[key])
    n = pl["n_rep"]
    _eq(f"{g['name']}: rep_slot", pl["rep_slot"][:n], g["rep_slot"])
    _eq(f"{g['name']}: rep_cap", pl["rep_cap"][:n], g["rep_cap"])
    routing = np.asarray(g["routing"], np.int32)
    counts, invalid = oracle.load(routing[None], g["E"])
    _eq(f"{g['name']}: routing counts", counts[0], g["routing_counts"])
    assert invalid[0] == g["invalid"], f"{g['name']}: invalid"
    rr = oracle.reroute(routing.reshape(-1), pl, perm_fill=PERM_FILL)
    assert rr["faults"] == g["faults"], \
        f"{g['name']}: faults {rr['faults']} != {g['faults']}"
    for key in ("phys", "inv_perm", "rank_counts"):
        _eq(f"{g['name']}: {key}", rr[key], g[key])
    want_perm = [PERM_FILL if v is None else v for v in g["perm"]]
    _eq(f"{g['name']}: perm", rr["perm"], want_perm)


# --------------------------------------------------------------------------
# invariants on arbitrary instances

def random_routing(rng, T, E, k, skew):
    """T tokens with k distinct experts each, Zipf-like weights."""
    if T == 0:
        return np.zeros((0, k), np.int32)
    w = np.arange(1, E + 1, dtype=np.float64) ** (-skew)
    w = w[rng.permutation(E)]
    p = w / w.sum()
    # successive sampling without replacement via Gumbel keys
    keys = np.log(p)[None, :] + rng.gumbel(size=(T, E))
    return np.argsort(-keys, axis=1, kind="stable")[:, :k].astype(np.int32)


def random_instance(rng, max_ranks=8, max_native=4, max_spare=3,
                    max_tokens=64, max_k=4):
    R = int(rng.integers(1, max_ranks + 1))
    N = int(rng.integers(1, max_native + 1))
    E = R * N
    S = int(rng.integers(0, max_spare + 1))
    k = int(rng.integers(1, min(E, max_k) + 1))
    T = int(rng.integers(0, max_tokens + 1))
    skew = float(rng.uniform(0.0, 3.0))
    return random_routing(rng, T, E, k, skew), E, R, S


def check_load(routing, E):
    flat = np.asarray(routing, np.int32).reshape(-1)
    counts, invalid = oracle.load(flat[None, None, :], E)
    valid = flat[(flat >= 0) & (flat < E)]
    want = np.bincount(valid, minlength=E)
    assert np.array_equal(counts[0], want), "counts differ from bincount"
    assert invalid[0] == flat.size - valid.size, "invalid id count"
    return counts[0]


def rank_amounts(counts, R, Q):
    """Each expert's amount at quota Q: a rank above Q sheds its excess
    from its experts heaviest first (count desc, id asc), each giving what
    it has of what is still left."""
    counts = np.asarray(counts, np.int64)
    E = counts.size
    N = E // R
    amt = np.zeros(E, np.int64)
    for r in range(R):
        left = int(counts[r * N:(r + 1) * N].sum()) - Q
        for e in sorted(range(r * N, (r + 1) * N),
                        key=lambda e: (-counts[e], e)):
            take = max(0, min(int(counts[e]), left))
            amt[e] = take
            left -= take
    return amt


def visit_order(counts, R, S, policy, Q):
    """Candidates (experts of ranks above the quota that fixes the order)
    in the order the rule visits them, and the amount each must place at
    Q. Policies 0 and 1: experts of ranks above Q, count desc, id asc.
    Policy 2: experts of ranks above Q0 = ceil(total / R); first those
    whose amount at Q0 is at most H0 (the largest headroom at Q0 among
    ranks with a spare slot), by amount asc, id asc; then the others by
    amount desc, id asc. Policy 3: experts of ranks above Q0 by amount at
    Q0 asc, id asc."""
    counts = np.asarray(counts, np.int64)
    E = counts.size
    N = E // R
    L = counts.reshape(R, N).sum(axis=1)
    if policy not in (2, 3):
        cands = sorted((e for e in range(E) if L[e // N] > Q),
                       key=lambda e: (-counts[e], e))
        return cands, rank_amounts(counts, R, Q)
    Q0 = -(-int(counts.sum()) // R)
    a0 = rank_amounts(counts, R, Q0)
    if policy == 3:
        cands = sorted((e for e in range(E) if L[e // N] > Q0),
                       key=lambda e: (a0[e], e))
        return cands, rank_amounts(counts, R, Q)
    H0 = max([Q0 - int(L[r]) for r in range(R) if S > 0 and L[r] < Q0],
             default=0)
    cands = [e for e in range(E) if L[e // N] > Q0]
    small = sorted((e for e in cands if a0[e] <= H0), key=lambda e: (a0[e], e))
    big = sorted((e for e in cands if a0[e] > H0), key=lambda e: (-a0[e], e))
    return small + big, rank_amounts(counts, R, Q)


def exhausts_at(counts, R, S, policy, Q):
    """Runs the planning rule at quota Q from scratch and says whether it
    stops with excess left: candidates by count desc, id asc; each chunk to
    the least-loaded rank with a free spare and load below Q (lowest id on
    ties), or under policy 1 to the eligible rank with the smallest headroom
    that holds a remainder the least-loaded rank would not fill."""
    counts = np.asarray(counts, np.int64)
    E = counts.size
    N = E // R
    L = counts.reshape(R, N).sum(axis=1).astype(np.int64)
    free = np.full(R, S)
    order, amt = visit_order(counts, R, S, policy, Q)
    for e in order:
        r, rem = e // N, int(amt[e])
        while L[r] > Q and rem > 0:
            elig = [x for x in range(R) if free[x] > 0 and L[x] < Q]
            if not elig:
                return True
            need = min(int(L[r] - Q), rem)
            d = min(elig, key=lambda x: (L[x], x))
            if policy >= 1 and need < Q - L[d]:
                d = min((x for x in elig if Q - L[x] >= need),
                        key=lambda x: (Q - L[x], x))
            m = min(need, int(Q - L[d]))
            L[r] -= m
            L[d] += m
            free[d] -= 1
            rem -= m
    return False


# The two checks below re-run the planning rule in Python (the quota
# search's steps, each chunk's destination). They are a second statement of
# the rule, not a fact independent of it, so the mutant tests also require
# every planted mistake to be caught with both switched off.
REPLAYS = True


def check_quota(counts, R, S, policy, quota_mode, pl):
    """Quota 0: ceil(total / R). Quota search: one of Q0 + j ceil(Q0/256),
    j < 64; every lower one exhausts when the rule is run on its own; the
    kept one does not, unless none of the 64 works, and then Q0 stands."""
    total = int(np.asarray(counts, np.int64).sum())
    Q0 = -(-total // R)
    Q = pl["quota"]
    if quota_mode == 0:
        assert Q == Q0, "quota is ceil(total / ranks)"
        return
    if not REPLAYS:
        return
    step = -(-Q0 // 256)
    grid = [Q0 + j * step for j in range(64)]
    assert Q in grid, "the quota is one of the searched steps"
    for M in grid[:grid.index(Q)]:
        assert exhausts_at(counts, R, S, policy, M), \
            f"quota {M} below the kept {Q} would place everything"
    if pl["exhausted"]:
        assert Q == Q0, "with no step that places everything, Q0 stands"
        assert all(exhausts_at(counts, R, S, policy, M) for M in grid)
    else:
        assert not exhausts_at(counts, R, S, policy, Q)


def check_plan(counts, R, S, A=None, policy=0, quota_mode=0):
    counts = np.asarray(counts, np.int64)
    E = counts.size
    N, NS = E // R, E // R + S
    P = R * NS
    pl = oracle.plan(counts.astype(np.int32), R, S, policy, quota_mode)
    Q = pl["quota"]
    total = int(counts.sum())
    A = total if A is None else A
    check_quota(counts, R, S, policy, quota_mode, pl)
    assert pl["P"] == P and pl["N"] == N

    rep_off, rep_slot, rep_cap = pl["rep_off"], pl["rep_slot"], pl["rep_cap"]
    n = pl["n_rep"]
    assert rep_off[0] == 0 and rep_off[E] == n and n <= P
    assert np.all(np.diff(rep_off) >= 1), "every expert keeps its master"
    assert np.all(rep_slot[n:] == -1) and np.all(rep_cap[n:] == 0)
    assert np.all(rep_cap[:n] >= 0)

    seen_slots = set()
    ranks_used_spares = {r: [] for r in range(R)}
    for e in range(E):
        ents = range(rep_off[e], rep_off[e + 1])
        first = rep_off[e]
        home = e // N
        assert rep_slot[first] == home * NS + e % N, "master is native slot"
        assert sum(int(rep_cap[i]) for i in ents) == counts[e], \
            "replica capacities sum to the expert's load"
        hosts = set()
        for i in ents:
            p = int(rep_slot[i])
            assert 0 <= p < P and p not in seen_slots, "one entry per slot"
            seen_slots.add(p)
            r = p // NS
            assert r not in hosts, "one replica per rank per expert"
            hosts.add(r)
            if i != first:
                assert p % NS >= N, "replicas live in spare slots"
                assert r != home, "never a replica on the home rank"
                assert rep_cap[i] > 0, "a created replica carries tokens"
                ranks_used_spares[r].append(p % NS - N)
    for r, used in ranks_used_spares.items():
        assert sorted(used) == list(range(len(used))), \
            "spare slots are taken lowest first"

    slot_expert, slot_cap = pl["slot_expert"], pl["slot_cap"]
    want_exp = np.full(P, -1)
    want_cap = np.zeros(P, np.int64)
    for p in range(P):
        if p % NS < N:
            want_exp[p] = (p // NS) * N + p % NS
    for e in range(E):
        for i in range(rep_off[e], rep_off[e + 1]):
            want_exp[rep_slot[i]] = e
            want_cap[rep_slot[i]] = rep_cap[i]
    assert np.array_equal(slot_expert, want_exp), "slot owner table"
    assert np.array_equal(slot_cap, want_cap), "slot capacity table"
    assert np.array_equal(pl["slot_off"],
                          np.concatenate([[0], np.cumsum(want_cap)])), \
        "slot offsets are the exclusive prefix of capacities"

    before = counts.reshape(R, N).sum(axis=1)
    after = np.asarray(slot_cap, np.int64).reshape(R, NS).sum(axis=1)
    assert np.array_equal(pl["load_before"], before), "native rank loads"
    assert np.array_equal(pl["load_after"], after), "rank loads after plan"
    assert after.sum() == total, "assignments are conserved"
    residual = int(np.maximum(after - Q, 0).sum())
    assert pl["residual"] == residual
    for r in range(R):
        if before[r] > Q:
            assert Q <= after[r] <= before[r], "sources shed down to Q only"
        else:
            assert before[r] <= after[r] <= Q, "destinations fill up to Q"
    if pl["exhausted"]:
        assert residual > 0
        free = np.array([S - len(ranks_used_spares[r]) for r in range(R)])
        assert np.all((free == 0) | (after >= Q)), \
            "exhausted only when no rank has room and a free spare"
    else:
        assert residual == 0 and after.max(initial=0) <= Q, \
            "every rank within quota whenever slots suffice"
    check_choices(counts, R, S, policy, pl)
    return pl


def check_choices(counts, R, S, policy, pl):
    """Replays the plan's chunks in creation order (candidates by count
    desc, id asc; each expert's replicas in table order) from the native
    loads and checks every step against the rule: the destination is
    eligible (a free spare slot, load below Q); under policy 0 it is the
    least-loaded such rank (lowest id on ties); under policy 1 too, unless
    the amount is below that rank's headroom, when it is the eligible rank
    with the smallest headroom that holds the amount (lowest id on ties);
    the chunk is min(source excess, expert remainder, headroom) and takes
    the lowest free spare slot; an expert stops short only when no rank is
    eligible, and then nothing moves after it."""
    if not REPLAYS:
        return
    counts = np.asarray(counts, np.int64)
    E = counts.size
    N, NS = E // R, E // R + S
    Q = pl["quota"]
    L = counts.reshape(R, N).sum(axis=1).astype(np.int64)
    free = np.full(R, S)
    cands, amt = visit_order(counts, R, S, policy, Q)
    stopped = False
    for e in cands:
        chunks = [(int(pl["rep_slot"][i]), int(pl["rep_cap"][i]))
                  for i in range(pl["rep_off"][e] + 1, pl["rep_off"][e + 1])]
        if stopped:
            assert not chunks, "nothing moves after the plan stops"
            continue
        r, rem = e // N, int(amt[e])
        while L[r] > Q and rem > 0:
            elig = [x for x in range(R) if free[x] > 0 and L[x] < Q]
            if not elig:
                assert not chunks, "a chunk placed with no eligible rank"
                stopped = True
                break
            assert chunks, "an expert stopped while a rank was eligible"
            p, m = chunks.pop(0)
            d = p // NS
            need = min(int(L[r] - Q), rem)
            least = min(elig, key=lambda x: (L[x], x))
            want = least
            if policy >= 1 and need < Q - L[least]:
                fits = [x for x in elig if Q - L[x] >= need]
                want = min(fits, key=lambda x: (Q - L[x], x))
            assert d == want, f"expert {e}: chunk to rank {d}, rule says {want}"
            assert m == min(need, int(Q - L[d])), "chunk size"
            assert p == d * NS + N + (S - free[d]), "lowest free spare slot"
            L[r] -= m
            L[d] += m
            free[d] -= 1
            rem -= m
        assert not chunks, f"expert {e}: more chunks than the rule places"
    assert bool(pl["exhausted"]) == stopped, "exhausted flag"


def check_reroute(routing, pl):
    flat = np.asarray(routing, np.int32).reshape(-1)
    A = flat.size
    E, R, S = pl["E"], pl["R"], pl["S"]
    NS = pl["N"] + S
    rr = oracle.reroute(flat, pl)
    phys, perm, inv = rr["phys"], rr["perm"], rr["inv_perm"]
    assert rr["faults"] == 0
    # stable dispatch order == library stable sort by physical slot
    assert np.array_equal(perm, np.argsort(phys, kind="stable")), \
        "perm is the stable sort of assignments by physical slot"
    assert np.array_equal(inv[perm], np.arange(A)), "inverse permutation"
    assert np.array_equal(pl["slot_expert"][phys], flat), \
        "physical slot holds the logical expert"
    assert np.array_equal(np.bincount(phys, minlength=pl["P"]),
                          pl["slot_cap"]), "slot hit counts equal capacities"
    assert np.array_equal(rr["rank_counts"],
                          np.bincount(phys // NS, minlength=R))
    assert np.array_equal(rr["rank_counts"], pl["load_after"])
    # j-th assignment of e (flat order) -> replica whose prefix covers j
    order = np.argsort(flat, kind="stable")
    j = np.empty(A, np.int64)
    sorted_e = flat[order]
    starts = np.searchsorted(sorted_e, sorted_e, side="left")
    j[order] = np.arange(A) - starts
    for a in range(A):
        e = flat[a]
        lo, hi = pl["rep_off"][e], pl["rep_off"][e + 1]
        cum = np.cumsum(pl["rep_cap"][lo:hi])
        idx = int(np.searchsorted(cum, j[a], side="right"))
        assert phys[a] == pl["rep_slot"][lo + idx], \
            "j-th assignment goes to the replica covering j"
    return rr


def check_instance(routing, E, R, S, policy=0, quota_mode=0):
    counts = check_load(routing, E)
    pl = check_plan(counts, R, S, policy=policy, quota_mode=quota_mode)
    check_reroute(routing, pl)
    return pl


# --------------------------------------------------------------------------
# closed forms

def check_no_spares(rng):
    """S = 0: nothing can move, so physical ids equal logical ids
    (p = r*N + s = e) and the plan is exhausted iff a rank is over quota."""
    for _ in range(20):
        routing, E, R, _ = random_instance(rng)
        counts = check_load(routing, E)
        pl = oracle.plan(counts, R, 0)
        rr = oracle.reroute(routing.reshape(-1), pl)
        assert np.array_equal(rr["phys"], routing.reshape(-1))
        assert pl["n_rep"] == E
        over = counts.reshape(R, -1).sum(axis=1) > pl["quota"]
        assert pl["exhausted"] == int(over.any())


def check_one_rank(rng):
    """R = 1: the only rank carries everything and is never over quota."""
    for _ in range(20):
        E = int(rng.integers(1, 9))
        k = int(rng.integers(1, E + 1))
        routing = random_routing(rng, int(rng.integers(0, 40)), E, k, 1.0)
        counts = check_load(routing, E)
        S = int(rng.integers(0, 3))
        pl = oracle.plan(counts, 1, S)
        assert pl["quota"] == routing.size and pl["n_rep"] == E
        assert pl["exhausted"] == 0
        rr = oracle.reroute(routing.reshape(-1), pl)
        assert np.array_equal(rr["phys"], routing.reshape(-1))


def check_balanced():
    """Round-robin routing loads every rank equally: no replicas."""
    for R, N, S, k in ((4, 2, 1, 2), (8, 8, 2, 8), (16, 1, 1, 4)):
        E = R * N
        T = 3 * E
        routing = (np.arange(T * k) % E).astype(np.int32).reshape(T, k)
        counts = check_load(routing, E)
        pl = oracle.plan(counts, R, S)
        assert pl["n_rep"] == E and pl["exhausted"] == 0
        assert np.all(pl["load_after"] == T * k // R)


def check_single_hot(max_ranks=12):
    """N = 1, k = 1, every token on expert 0: Q = ceil(L/R); the master keeps
    Q and ranks 1, 2, ... receive one replica each, all of Q tokens except
    the last, which takes what is left."""
    for R in range(2, max_ranks + 1):
        for L in range(1, 5 * R + 3):
            counts = np.zeros(R, np.int32)
            counts[0] = L
            pl = oracle.plan(counts, R, 1)
            Q = -(-L // R)
            assert pl["quota"] == Q
            n_extra = -(-L // Q) - 1
            lo, hi = pl["rep_off"][0], pl["rep_off"][1]
            slots = list(pl["rep_slot"][lo:hi])
            caps = list(pl["rep_cap"][lo:hi])
            assert slots == [0] + [2 * r + 1 for r in range(1, n_extra + 1)]
            last = (L - Q) - Q * (n_extra - 1) if n_extra else None
            want = [Q] + [Q] * (n_extra - 1) + ([last] if n_extra else [])
            assert caps == want, (R, L, caps, want)
            assert pl["exhausted"] == 0


def check_invalid_ids():
    """Ids outside [0, E) are not counted, and are reported."""
    routing = np.array([[0, 5], [-1, 2], [4, 1], [7, 3]], np.int32)
    counts, invalid = oracle.load(routing[None], 5)
    assert list(counts[0]) == [1, 1, 1, 1, 1] and invalid[0] == 3
    counts, invalid = oracle.load(routing[None], 8)
    assert invalid[0] == 1 and counts[0].sum() == 7


# --------------------------------------------------------------------------
# brute force: optimal placement over every choice of spare-slot contents

def _min_max_load(counts, hosts, R):
    """Smallest M such that every expert's tokens can be spread over the
    ranks hosting it with no rank above M (integral max-flow)."""
    from scipy.sparse import csr_matrix
    from scipy.sparse.csgraph import maximum_flow

    E = len(counts)
    total = int(sum(counts))
    if total == 0:
        return 0
    src, sink = 0, E + R + 1

    def feasible(M):
        rows, cols, caps = [], [], []
        for e in range(E):
            rows.append(src), cols.append(1 + e), caps.append(int(counts[e]))
            for r in hosts[e]:
                rows.append(1 + e), cols.append(1 + E + r)
                caps.append(int(counts[e]))
        for r in range(R):
            rows.append(1 + E + r), cols.append(sink), caps.append(int(M))
        g = csr_matrix((np.array(caps, np.int32), (rows, cols)),
                       shape=(E + R + 2, E + R + 2))
        return maximum_flow(g, src, sink).flow_value == total

    lo = -(-total // R)
    hi = max(sum(int(counts[e]) for e in range(E) if e // (E // R) == r)
             for r in range(R))
    while lo < hi:
        mid = (lo + hi) // 2
        if feasible(mid):
            hi = mid
        else:
            lo = mid + 1
    return lo


def optimum_max_load(counts, R, S):
    E = len(counts)
    N = E // R
    slots = [(r, i) for r in range(R) for i in range(S)]
    options = [[-1] + [e for e in range(E) if e // N != r and counts[e] > 0]
               for (r, _) in slots]
    best = math.inf
    for combo in itertools.product(*options):
        hosts = [{e // N} for e in range(E)]
        for (r, _), e in zip(slots, combo):
            if e >= 0:
                hosts[e].add(r)
        best = min(best, _min_max_load(counts, hosts, R))
    return best


def check_against_optimum(counts, R, S, policy=0, quota_mode=0):
    """Returns greedy / optimum. The greedy plan is one of the placements
    enumerated, so the optimum can never exceed it; every placement has a
    rank at or above ceil(total / R) = Q0, so when slots suffice at Q0 the
    greedy (which then ends with every rank <= Q0) is optimal; a raised
    quota that places everything bounds the greedy's maximum."""
    pl = check_plan(counts, R, S, policy=policy, quota_mode=quota_mode)
    greedy = int(pl["load_after"].max(initial=0))
    opt = optimum_max_load(list(counts), R, S)
    Q0 = -(-int(np.sum(counts)) // R)
    assert opt <= greedy, "greedy beats the exhaustive optimum"
    assert opt >= Q0, "no placement beats the quota"
    if not pl["exhausted"]:
        assert greedy <= pl["quota"]
        if pl["quota"] == Q0:
            assert greedy == opt == Q0
    return greedy / opt if opt else 1.0
