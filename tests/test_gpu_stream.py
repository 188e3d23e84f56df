"""Replica weight sync, replica gradient reduction and the dispatch gather
on the device, against the oracle (numpy): bitwise for the copies, within
the fp32 summation bound for the gradient sums."""
import numpy as np
import pytest
import torch

import moe_expert_load_ue_amd as ue
import oracle
from gpu_helpers import gpu_rebalance, say
from moe_expert_load_ue_amd import workloads as W

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
U = 2.0 ** -24          # unit roundoff of fp32


def sum_bound(terms_abs_sum, n_adds):
    """|fl(sum) - sum| <= gamma_n * sum |terms| for n left-to-right adds."""
    g = n_adds * U / (1 - n_adds * U)
    return g * terms_abs_sum


def register(ctx, sb):
    M = sb.master_w.shape[1]
    ctx.register_experts([sb.elems] * M, sb.tables("master_w"),
                         sb.tables("master_g"), sb.tables("spare_w"),
                         sb.tables("spare_g"))


def csr_tensors(sb):
    return (torch.tensor(sb.rep_off, dtype=torch.int32, device=DEV),
            torch.tensor(sb.rep_buf, dtype=torch.int32, device=DEV))


@pytest.mark.parametrize("elems", [8, 1000, 4099, 70001, 262144])
def test_sync_and_reduce_small(elems):
    """Odd sizes: partial last chunks and tails not a multiple of a vector."""
    say("stream small", elems)
    fan = (3, 0, 1, 2, 4)
    sb = W.make_stream_buffers(elems=elems, n_mats=3, fanout=fan, device=DEV)
    sb.spare_w.view(torch.int16).fill_(-1)
    ctx = ue.Context(8, 1, 0, 1, 1, device=DEV)
    register(ctx, sb)
    rep_off, rep_buf = csr_tensors(sb)
    n = sb.elems
    master_w = sb.master_w[..., :n].view(torch.int16).cpu().numpy().view(
        np.uint16)
    master_g = sb.master_g[..., :n].cpu().numpy().astype(np.float64)
    spare_g = sb.spare_g[..., :n].cpu().numpy()
    ctx.weight_sync(rep_off, rep_buf)
    ctx.grad_reduce(rep_off, rep_buf)
    torch.cuda.synchronize()
    got_w = sb.spare_w[..., :n].view(torch.int16).cpu().numpy().view(
        np.uint16)
    got_g = sb.master_g[..., :n].cpu().numpy()
    for e, f in enumerate(fan):
        bufs = sb.rep_buf[sb.rep_off[e] + 1: sb.rep_off[e + 1]]
        want = oracle.weight_sync(master_w[e], len(bufs))
        for b, w in zip(bufs, want):
            assert np.array_equal(got_w[b], w), (e, b)
        ref = oracle.grad_reduce(master_g[e], [spare_g[b] for b in bufs])
        terms = np.abs(master_g[e]) + sum(np.abs(spare_g[b]) for b in bufs)
        err = np.abs(got_g[e].astype(np.float64) - ref)
        assert np.all(err <= sum_bound(terms, len(bufs)) + 1e-45), e
        want_g = oracle.grad_reduce_rounded(master_g[e].astype(np.float32),
                                            [spare_g[b] for b in bufs])
        assert np.array_equal(got_g[e].view(np.int32),
                              want_g.view(np.int32)), e
        if not bufs:
            assert np.array_equal(got_g[e], master_g[e].astype(np.float32))
    # replicas' gradients are left unchanged
    assert np.array_equal(sb.spare_g[..., :n].cpu().numpy(), spare_g)
    # nothing beyond the matrices was written
    assert bool((sb.spare_w[..., n:].view(torch.int16) == -1).all())


def test_reduce_order_is_left_to_right():
    """The sum is carried in binary64, left to right, and rounded once:
    1 + 2^-24 + 2^-24 gives 1 + 2^-23 (a binary32 running sum would give 1),
    and 1 + 2^-60 - 1 gives 0 (the exact sum, or the order 1 - 1 + 2^-60,
    gives 2^-60). Both equal the oracle's rounded sum bitwise."""
    say("reduce order")
    n = 4096
    cases = {"carried wide": (1.0, 2.0 ** -24, 2.0 ** -24, 1.0 + 2.0 ** -23),
             "left to right": (1.0, 2.0 ** -60, -1.0, 0.0)}
    for name, (m0, r1, r2, want) in cases.items():
        mg = torch.full((2, 1, n), m0, dtype=torch.float32, device=DEV)
        sg = torch.empty((2, 1, n), dtype=torch.float32, device=DEV)
        sg[0].fill_(r1)
        sg[1].fill_(r2)
        mw = torch.zeros((2, 1, n), dtype=torch.bfloat16, device=DEV)
        sw = torch.zeros((2, 1, n), dtype=torch.bfloat16, device=DEV)
        ctx = ue.Context(2, 1, 0, 1, 1, device=DEV)
        ctx.register_experts([n], [[mw[0, 0]], [mw[1, 0]]],
                             [[mg[0, 0]], [mg[1, 0]]], [[sw[0, 0]], [sw[1, 0]]],
                             [[sg[0, 0]], [sg[1, 0]]])
        rep_off = torch.tensor([0, 3, 4], dtype=torch.int32, device=DEV)
        rep_buf = torch.tensor([-1, 0, 1, -1], dtype=torch.int32, device=DEV)
        ctx.grad_reduce(rep_off, rep_buf)
        torch.cuda.synchronize()
        assert bool((mg[0] == want).all()), name
        assert bool((mg[1] == m0).all()), name      # no replica: unchanged
        ref = oracle.grad_reduce_rounded(np.full(1, m0, np.float32),
                                         [np.full(1, r1, np.float32),
                                          np.full(1, r2, np.float32)])
        assert ref[0] == np.float32(want), name
        ctx.close()


def test_sync_reduce_full_size():
    """32 experts x 3 DeepSeek-V3 expert matrices (14,680,064 elements
    each), 64 replica buffers, every element compared: every replica equals
    its master bitwise (on the device), and every master gradient equals
    the oracle's rounded binary64 left-to-right sum bitwise, matrix by
    matrix on the host. Against the exact sum (the float64 sum: the
    partial sums of these terms are exact in float64) every element's
    relative error is at most 1e-6 (one binary32 rounding is 2^-24)."""
    say("stream full size")
    sb = W.make_stream_buffers(device=DEV)
    ctx = ue.Context(32, 1, 0, 1, 1, device=DEV)
    register(ctx, sb)
    rep_off, rep_buf = csr_tensors(sb)
    n = sb.elems
    before = sb.master_g[:, :, :n].clone()      # on the device (5.6 GB)
    ctx.weight_sync(rep_off, rep_buf)
    ctx.grad_reduce(rep_off, rep_buf)
    torch.cuda.synchronize()
    worst_rel, worst_terms, above = 0.0, 0.0, 0
    for e in range(32):
        bufs = sb.rep_buf[sb.rep_off[e] + 1: sb.rep_off[e + 1]]
        say("stream full size: expert", e, "replicas", len(bufs))
        for b in bufs:
            assert torch.equal(sb.spare_w[b, :, :n].view(torch.int16),
                               sb.master_w[e, :, :n].view(torch.int16)), (e, b)
        for m in range(sb.master_g.shape[1]):
            m0 = before[e, m].cpu().numpy()
            reps = [sb.spare_g[b, m, :n].cpu().numpy() for b in bufs]
            got = sb.master_g[e, m, :n].cpu().numpy()
            want = oracle.grad_reduce_rounded(m0, reps)
            assert np.array_equal(got.view(np.int32), want.view(np.int32)), \
                (e, m, int(np.sum(got != want)))
            exact = oracle.grad_reduce(m0, reps)
            err = np.abs(got.astype(np.float64) - exact)
            terms = np.abs(m0).astype(np.float64)
            for r in reps:
                terms += np.abs(r)
            assert np.all(err <= sum_bound(terms, len(bufs))), (e, m)
            nz = exact != 0
            rel = err[nz] / np.abs(exact[nz])
            worst_rel = max(worst_rel, float(rel.max(initial=0.0)))
            above += int(np.sum(rel > 1e-6))
            worst_terms = max(worst_terms, float(
                (err[terms > 0] / terms[terms > 0]).max(initial=0.0)))
    say("stream full size: largest error / |float64 sum|", worst_rel,
        "elements above 1e-6:", above, "of", 32 * 3 * n,
        "largest error / sum|terms|", worst_terms)
    assert worst_rel <= 1e-6 and above == 0


def test_gather_small():
    rng = np.random.default_rng(8)
    for T, k, H in ((1, 1, 8), (37, 3, 24), (300, 8, 1032), (1000, 2, 4096)):
        say("gather", T, k, H)
        x = torch.from_numpy(rng.standard_normal((T, H)).astype(np.float32)
                             ).to(torch.bfloat16).to(DEV)
        perm = rng.permutation(T * k).astype(np.int32)
        inv = np.empty_like(perm)
        inv[perm] = np.arange(T * k, dtype=np.int32)
        ctx = ue.Context(8, 1, 0, k, T, device=DEV)
        out = torch.full((T * k, H), -1, dtype=torch.int16, device=DEV
                         ).view(torch.bfloat16)
        ctx.gather_rows(x, torch.from_numpy(inv).to(DEV), out=out)
        torch.cuda.synchronize()
        want = oracle.gather(x.view(torch.int16).cpu().numpy(), perm, k)
        assert np.array_equal(out.view(torch.int16).cpu().numpy(), want)


def test_gather_pipeline_microbatch_full():
    """One microbatch of the pipeline workload at full size: rebalance,
    then gather [131072, 4096] bf16 into [1048576, 4096] physical-expert
    order; every row checked against the oracle's permutation, in blocks
    of rows on the host."""
    cfg = W.CONFIGS["pipeline"]
    say("gather pipeline full size")
    routing = W.make_routing(cfg, device=DEV, layers=1)
    ctx = ue.Context(cfg.experts, cfg.ranks, cfg.spare, cfg.topk, cfg.tokens,
                     1, device=DEV)
    res = gpu_rebalance(ctx, routing)
    pl = oracle.plan(oracle.load(routing.cpu().numpy(), cfg.experts)[0][0],
                     cfg.ranks, cfg.spare)
    rr = oracle.reroute(routing.cpu().numpy().reshape(-1), pl)
    assert rr["faults"] == 0
    x = W.make_activations(cfg.tokens, cfg.hidden, 0, device=DEV)
    inv = torch.from_numpy(res["inv_perm"][0]).to(DEV)
    out = torch.full((cfg.assignments, cfg.hidden), -1, dtype=torch.int16,
                     device=DEV).view(torch.bfloat16)
    ctx.gather_rows(x, inv, out=out)
    torch.cuda.synchronize()
    x_host = x.view(torch.int16).cpu().numpy()
    block = 1 << 16
    for r0 in range(0, cfg.assignments, block):
        r1 = min(r0 + block, cfg.assignments)
        got = out[r0:r1].view(torch.int16).cpu().numpy()
        want = oracle.gather(x_host, rr["perm"][r0:r1], cfg.topk)
        assert np.array_equal(got, want), f"rows {r0}..{r1}"
