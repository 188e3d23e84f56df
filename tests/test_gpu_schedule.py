"""The per-layer schedule around the rebalance, on the device: the plan's
own replica table drives the replica weight sync, the restore before
backward (the same sync from the saved plan) and the gradient reduction;
and the whole sequence replays from a captured graph with fresh routing
each time. Results against the oracle: bitwise for the routing outputs and
the copies, within the fp32 summation bound for the gradient sums."""
import numpy as np
import pytest
import torch

import moe_expert_load_ue_amd as ue
import oracle
import pins
from gpu_helpers import compare_with_oracle, say

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
U = 2.0 ** -24
MATS = (1000, 4099)          # odd matrix sizes: vector tails


def slot_state(ctx, gen):
    """Masters (bf16 weights, fp32 gradients) and one buffer per physical
    slot: a native slot's buffer is its expert's master, a spare slot's is
    its own (weights filled with a sentinel, gradients random)."""
    E, N, NS, P = ctx.E, ctx.N, ctx.N + ctx.S, ctx.P

    def rnd(n, dtype):
        return (torch.randn(n, generator=gen, device=DEV) * 0.02).to(dtype)

    mw = [[rnd(n, torch.bfloat16) for n in MATS] for _ in range(E)]
    mg = [[rnd(n, torch.float32) for n in MATS] for _ in range(E)]
    sw, sg = [], []
    for p in range(P):
        if p % NS < N:
            e = (p // NS) * N + p % NS
            sw.append(mw[e])
            sg.append(mg[e])
        else:
            sw.append([torch.full((n,), -1, dtype=torch.int16,
                                  device=DEV).view(torch.bfloat16)
                       for n in MATS])
            sg.append([rnd(n, torch.float32) for n in MATS])
    ctx.register_experts(list(MATS), mw, mg, sw, sg)
    return mw, mg, sw, sg


def bits(t):
    return t.view(torch.int16).cpu().numpy()


def check_replicas(pl, mw, sw, NS, N):
    """Every replica slot of the plan holds its master bitwise; spare slots
    the plan leaves unused still hold the sentinel."""
    named = set()
    for e in range(len(mw)):
        for i in range(pl["rep_off"][e] + 1, pl["rep_off"][e + 1]):
            p = int(pl["rep_slot"][i])
            named.add(p)
            for m in range(len(MATS)):
                assert np.array_equal(bits(sw[p][m]), bits(mw[e][m])), \
                    f"slot {p} expert {e} matrix {m}"
    for p in range(len(sw)):
        if p % NS >= N and p not in named:
            for m in range(len(MATS)):
                assert np.all(bits(sw[p][m]) == -1), f"unused slot {p}"


def routing_outputs(ctx, L, T):
    i32 = dict(dtype=torch.int32, device=DEV)
    A = T * ctx.k
    return dict(counts=torch.empty((L, ctx.E), **i32),
                invalid=torch.empty((L,), **i32),
                placement=ctx.new_placement(L),
                phys=torch.empty((L, T, ctx.k), **i32),
                rank_counts=torch.empty((L, ctx.R), **i32),
                perm=torch.empty((L, A), **i32),
                inv_perm=torch.empty((L, A), **i32),
                faults=torch.empty((L,), **i32))


def as_result(ctx, outs):
    f = ctx.placement_fields(outs["placement"])
    res = {k: v.cpu().numpy() for k, v in outs.items()}
    res["plan"] = {k: v.cpu().numpy() for k, v in f.items()}
    res["policy"], res["quota_mode"] = ctx.plan_policy, ctx.quota_mode
    return res


@pytest.mark.parametrize("policy,quota_mode",
                         [(0, 0), (1, 1), (2, 1), (3, 1)],
                         ids=["least_loaded", "best_fit_search",
                              "cover_search", "ascending_search"])
def test_plan_driven_sync_restore_reduce(policy, quota_mode):
    E, R, S, k, T = 32, 8, 2, 4, 3000
    rng = np.random.default_rng(5 + policy)
    routing = pins.random_routing(rng, T, E, k, 1.8)[None]
    say("schedule", policy, quota_mode)
    ctx = ue.Context(E, R, S, k, T, 1, device=DEV, plan_policy=policy,
                     quota_mode=quota_mode)
    gen = torch.Generator(device=DEV)
    gen.manual_seed(77)
    mw, mg, sw, sg = slot_state(ctx, gen)
    outs = routing_outputs(ctx, 1, T)
    ue.ue_rebalance(ctx, torch.from_numpy(routing).to(DEV), **outs)
    torch.cuda.synchronize()
    compare_with_oracle(as_result(ctx, outs), routing, E, R, S)
    counts, _ = oracle.load(routing, E)
    pl = oracle.plan(counts[0], R, S, policy, quota_mode)
    assert pl["n_rep"] > E, "the case must create replicas"
    N, NS = ctx.N, ctx.N + ctx.S
    masters_w = [[bits(t) for t in row] for row in mw]

    rep_off, rep_slot = ue.replica_table(ctx, outs["placement"], 0)
    ctx.weight_sync(rep_off, rep_slot)
    torch.cuda.synchronize()
    check_replicas(pl, mw, sw, NS, N)
    for e in range(E):                       # masters untouched
        for m in range(len(MATS)):
            assert np.array_equal(bits(mw[e][m]), masters_w[e][m])

    # the forward pass may overwrite replica buffers; the restore before
    # backward is the same sync from the saved plan
    for e in range(E):
        for i in range(pl["rep_off"][e] + 1, pl["rep_off"][e + 1]):
            for t in sw[int(pl["rep_slot"][i])]:
                t.view(torch.int16).fill_(0x1234)
    ctx.weight_sync(rep_off, rep_slot)
    torch.cuda.synchronize()
    check_replicas(pl, mw, sw, NS, N)

    before = [[t.cpu().numpy() for t in row] for row in mg]
    reps = [[t.cpu().numpy() for t in row] for row in sg]
    ctx.grad_reduce(rep_off, rep_slot)
    torch.cuda.synchronize()
    for e in range(E):
        slots = [int(pl["rep_slot"][i])
                 for i in range(pl["rep_off"][e] + 1, pl["rep_off"][e + 1])]
        for m in range(len(MATS)):
            terms = [before[e][m]] + [reps[p][m] for p in slots]
            want = oracle.grad_reduce(terms[0], terms[1:])
            got = mg[e][m].cpu().numpy().astype(np.float64)
            n = len(slots)
            g = n * U / (1 - n * U)
            bound = g * np.sum(np.abs(np.stack(terms).astype(np.float64)),
                               axis=0)
            assert np.all(np.abs(got - want) <= bound), f"expert {e} m {m}"
            if n == 0:
                assert np.array_equal(got, before[e][m])


def test_graph_replay_rebalance_and_sync():
    """ue_rebalance and the plan-driven sync captured once, replayed with
    new routing copied into the captured input between replays (eager work
    in between); every replay matches the oracle."""
    E, R, S, k, T = 64, 8, 2, 8, 4096
    ctx = ue.Context(E, R, S, k, T, 1, device=DEV,
                     plan_policy=ue.PLAN_BEST_FIT, quota_mode=ue.QUOTA_SEARCH)
    gen = torch.Generator(device=DEV)
    gen.manual_seed(78)
    mw, mg, sw, sg = slot_state(ctx, gen)
    outs = routing_outputs(ctx, 1, T)
    rng = np.random.default_rng(8)
    cases = [pins.random_routing(rng, T, E, k, s)[None]
             for s in (1.2, 0.3, 2.2, 1.6)]
    static = torch.from_numpy(cases[0]).to(DEV)
    rep_off, rep_slot = ue.replica_table(ctx, outs["placement"], 0)
    ue.ue_rebalance(ctx, static, **outs)          # eager warm-up
    ctx.weight_sync(rep_off, rep_slot)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        ue.ue_rebalance(ctx, static, **outs)
        ctx.weight_sync(rep_off, rep_slot)
    N, NS = ctx.N, ctx.N + ctx.S
    for i, routing in enumerate(cases[1:] + cases[:1]):
        say("graph replay", i)
        static.copy_(torch.from_numpy(routing))
        for p in range(ctx.P):                     # reset the spare slots
            if p % NS >= N:
                for t in sw[p]:
                    t.view(torch.int16).fill_(-1)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        compare_with_oracle(as_result(ctx, outs), routing, E, R, S)
        counts, _ = oracle.load(routing, E)
        pl = oracle.plan(counts[0], R, S, ue.PLAN_BEST_FIT, ue.QUOTA_SEARCH)
        check_replicas(pl, mw, sw, NS, N)


def test_graph_replay_batched_layers():
    """ue_rebalance over nine layers (three launches on the caller's
    stream) captured once and replayed on fresh routing, every layer
    against the oracle."""
    E, R, S, k, T, L = 64, 8, 2, 8, 3001, 9
    ctx = ue.Context(E, R, S, k, T, L, device=DEV)
    outs = routing_outputs(ctx, L, T)
    rng = np.random.default_rng(9)
    cases = [np.stack([pins.random_routing(rng, T, E, k, s)
                       for s in rng.uniform(0.3, 2.2, L)]) for _ in range(3)]
    static = torch.from_numpy(cases[0]).to(DEV)
    ue.ue_rebalance(ctx, static, **outs)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        ue.ue_rebalance(ctx, static, **outs)
    for i, routing in enumerate(cases[1:] + cases[:1]):
        say("batched graph replay", i)
        static.copy_(torch.from_numpy(routing))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        compare_with_oracle(as_result(ctx, outs), routing, E, R, S)


def test_two_stream_schedule():
    """The overlapped forward schedule: every layer's rebalance on one
    stream, each layer's plan-driven weight sync and dispatch gather on a
    second stream once that layer's rebalance has finished (an event), so
    the next layers' rebalances run beside this layer's copies. Every
    layer's routing outputs and gather against the oracle; the replica
    buffers, shared by all layers and written in layer order, end as the
    last layer naming each slot left them."""
    E, R, S, k, T, H, L = 64, 8, 2, 8, 4096, 64, 4
    ctx = ue.Context(E, R, S, k, T, 1, device=DEV,
                     plan_policy=ue.PLAN_BEST_FIT, quota_mode=ue.QUOTA_SEARCH)
    gen = torch.Generator(device=DEV)
    gen.manual_seed(79)
    mw, mg, sw, sg = slot_state(ctx, gen)
    rng = np.random.default_rng(10)
    routings = [pins.random_routing(rng, T, E, k, s)[None]
                for s in (1.4, 0.6, 2.0, 1.1)]
    rin = [torch.from_numpy(r).to(DEV) for r in routings]
    outs = [routing_outputs(ctx, 1, T) for _ in range(L)]
    tables = [ue.replica_table(ctx, o["placement"], 0) for o in outs]
    x = (torch.randn((T, H), generator=gen, device=DEV)).to(torch.bfloat16)
    xo = [torch.empty((T * k, H), dtype=torch.bfloat16, device=DEV)
          for _ in range(L)]
    a, b = torch.cuda.Stream(device=DEV), torch.cuda.Stream(device=DEV)
    ev = [torch.cuda.Event() for _ in range(L)]
    torch.cuda.synchronize()
    say("two-stream schedule")
    for l in range(L):
        ue.ue_rebalance(ctx, rin[l], **outs[l], stream=a)
        ev[l].record(a)
    for l in range(L):
        b.wait_event(ev[l])
        ctx.weight_sync(*tables[l], stream=b)
        ue.ue_gather_rows(ctx, x, outs[l]["inv_perm"][0], xo[l], stream=b)
    torch.cuda.synchronize()

    xs = bits(x).reshape(T, H)
    N, NS = ctx.N, ctx.N + ctx.S
    last = {}                                   # slot -> expert, layer order
    for l in range(L):
        compare_with_oracle(as_result(ctx, outs[l]), routings[l], E, R, S)
        counts, _ = oracle.load(routings[l], E)
        pl = oracle.plan(counts[0], R, S, ue.PLAN_BEST_FIT, ue.QUOTA_SEARCH)
        rr = oracle.reroute(routings[l].reshape(-1), pl)
        want = oracle.gather(xs, rr["perm"], k)
        assert np.array_equal(bits(xo[l]).reshape(T * k, H), want), \
            f"layer {l} gather"
        for e in range(E):
            for i in range(pl["rep_off"][e] + 1, pl["rep_off"][e + 1]):
                last[int(pl["rep_slot"][i])] = e
    for p in range(ctx.P):
        if p % NS < N:
            continue
        for m in range(len(MATS)):
            got = bits(sw[p][m])
            if p in last:
                assert np.array_equal(got, bits(mw[last[p]][m])), f"slot {p}"
            else:
                assert np.all(got == -1), f"unused slot {p}"
