"""One layer of about 537 million assignments (T*k just above 2^29, with a
ragged last tile): byte offsets past 2^31 in every per-layer array, 262,145
routing tiles and 16,385 load groups, against the oracle bit-exact (fused
call), and the three separate calls against the fused one."""
import numpy as np
import pytest
import torch

import moe_expert_load_ue_amd as ue
from gpu_helpers import compare_with_oracle, gpu_rebalance, say
from moe_expert_load_ue_amd import workloads as W

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def test_layer_past_2_31_bytes():
    E, R, S, k = 256, 64, 1, 8
    T = (1 << 26) + 123
    say(f"large layer: E={E} R={R} S={S} k={k} T={T}")
    g = torch.Generator(device=DEV)
    g.manual_seed(20261203)
    order = torch.randperm(E, generator=g, device=DEV)
    routing = torch.empty((1, T, k), dtype=torch.int32, device=DEV)
    step = 1 << 20
    for t0 in range(0, T, step):
        n = min(step, T - t0)
        routing[0, t0:t0 + n] = W.zipf_layer(n, E, k, 1.1, order, g)
    ctx = ue.Context(E, R, S, k, T, 1, device=DEV)
    res = gpu_rebalance(ctx, routing, fused=True)
    compare_with_oracle(res, routing.cpu().numpy(), E, R, S)
    say("large layer: separate calls")
    calls = gpu_rebalance(ctx, routing, fused=False)
    for key in ("counts", "placement", "phys", "perm", "inv_perm",
                "rank_counts", "faults"):
        assert np.array_equal(calls[key], res[key]), key
