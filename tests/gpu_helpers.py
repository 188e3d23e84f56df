"""Shared pieces of the GPU tests: run the HIP path through the C ABI and
compare its outputs with the oracle's, field by field."""
from __future__ import annotations

import sys

import numpy as np
import torch

import moe_expert_load_ue_amd as ue
import oracle

PLAN_ARRAYS = ("rep_off", "slot_expert", "slot_cap", "slot_off",
               "load_before", "load_after", "rep_slot", "rep_cap")
PLAN_SCALARS = ("quota", "exhausted", "residual", "n_rep")


def say(*a):
    """Names the case before a GPU step, flushed (the box may not return
    later output if a step faults)."""
    print(*a, flush=True)
    sys.stdout.flush()


def gpu_rebalance(ctx, routing, with_inv=True, fused=False):
    """load -> plan -> reroute on the device, as three calls or as one
    ue_rebalance call; returns numpy copies."""
    dev = ctx.device
    r = routing.to(dev)
    L = r.shape[0]
    invalid = torch.full((L,), -7, dtype=torch.int32, device=dev)
    if fused:
        out = ue.ue_rebalance(ctx, r, invalid=invalid, with_inv=with_inv)
        counts, placement = out.pop("counts"), out.pop("placement")
        out.pop("invalid")
    else:
        counts = ue.ue_load(ctx, r, invalid=invalid)
        placement = ue.ue_plan(ctx, counts)
        out = ue.ue_reroute(ctx, r, placement, with_inv=with_inv)
    torch.cuda.synchronize(dev)
    f = ctx.placement_fields(placement)
    res = dict(counts=counts.cpu().numpy(), invalid=invalid.cpu().numpy(),
               placement=placement.cpu().numpy(), policy=ctx.plan_policy,
               quota_mode=ctx.quota_mode)
    res["plan"] = {k: v.cpu().numpy() for k, v in f.items()}
    for k, v in out.items():
        res[k] = None if v is None else v.cpu().numpy()
    return res


def compare_with_oracle(res, routing_np, E, R, S, layers=None):
    """Bit-exact comparison of every output with the oracle, per layer."""
    L = routing_np.shape[0]
    layers = range(L) if layers is None else layers
    counts, invalid = oracle.load(routing_np, E)
    assert np.array_equal(res["counts"], counts), "counts"
    assert np.array_equal(res["invalid"], invalid.astype(np.int32)), "invalid"
    flat = routing_np.reshape(L, -1)
    for layer in layers:
        pl = oracle.plan(counts[layer], R, S, res.get("policy", 0),
                         res.get("quota_mode", 0))
        for key in PLAN_SCALARS:
            got = int(res["plan"][key][layer])
            assert got == pl[key], f"layer {layer} {key}: {got} != {pl[key]}"
        for key in PLAN_ARRAYS:
            got = res["plan"][key][layer]
            assert np.array_equal(got, pl[key]), f"layer {layer} {key}"
        rr = oracle.reroute(flat[layer], pl)
        assert np.array_equal(res["phys"][layer].reshape(-1), rr["phys"]), \
            f"layer {layer} phys"
        assert np.array_equal(res["rank_counts"][layer], rr["rank_counts"]), \
            f"layer {layer} rank_counts"
        assert int(res["faults"][layer]) == rr["faults"], f"layer {layer} faults"
        if rr["faults"] == 0:
            assert np.array_equal(res["perm"][layer], rr["perm"]), \
                f"layer {layer} perm"
        if res["inv_perm"] is not None:
            assert np.array_equal(res["inv_perm"][layer], rr["inv_perm"]), \
                f"layer {layer} inv_perm"
    return counts
