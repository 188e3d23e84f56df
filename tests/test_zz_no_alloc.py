"""ue_rebalance_static (no context, no allocation: scratch in a static
device array) against ue_rebalance on the same routing, every output
bit-exact, over calls in a row on one device: the 58-layer dsv3 rebalance,
then a smaller ragged input under another rule, then dsv3 again (each call
reads only scratch it wrote itself). A call whose scratch would exceed the
array is refused before anything is written."""
import numpy as np
import pytest
import torch

import moe_expert_load_ue_amd as ue
from gpu_helpers import say
from moe_expert_load_ue_amd import workloads as W

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
KEYS = ("counts", "invalid", "placement", "phys", "rank_counts", "perm",
        "inv_perm", "faults")


def outputs(cfg, L, T, fill=-5):
    words = ue.placement_words(cfg.num_experts, cfg.num_ranks,
                               cfg.spare_per_rank)
    A = T * cfg.topk
    shapes = dict(counts=(L, cfg.num_experts), invalid=(L,),
                  placement=(L, words), phys=(L, T, cfg.topk),
                  rank_counts=(L, cfg.num_ranks), perm=(L, A),
                  inv_perm=(L, A), faults=(L,))
    return {k: torch.full(v, fill, dtype=torch.int32, device=DEV)
            for k, v in shapes.items()}


def run_both(E, R, S, k, T, L, routing, policy=0, quota_mode=0):
    cfg = ue.ue_config(E, R, S, k, T, L, policy, quota_mode)
    ctx = ue.Context(E, R, S, k, T, L, device=DEV, plan_policy=policy,
                     quota_mode=quota_mode)
    assert ctx.placement_words == ue.placement_words(E, R, S)
    want = ue.ue_rebalance(ctx, routing)
    got = outputs(cfg, L, T)
    ue.ue_rebalance_static(cfg, routing, **got)
    torch.cuda.synchronize()
    for key in KEYS:
        assert torch.equal(got[key].reshape(-1), want[key].reshape(-1)), key
    assert int(got["faults"].sum()) == 0
    ctx.close()


def test_static_rebalance_matches_context_calls():
    d = W.CONFIGS["dsv3"]
    dsv3 = W.make_routing(d, device=DEV)
    say("static rebalance: dsv3, 58 layers")
    run_both(d.experts, d.ranks, d.spare, d.topk, d.tokens, d.layers, dsv3)

    say("static rebalance: smaller ragged input, best fit + quota search")
    rng = np.random.default_rng(21)
    E, R, S, k, T, L = 64, 8, 2, 6, 5001, 3
    w = np.arange(1, E + 1, dtype=np.float64) ** -1.3
    keys = np.log(w)[None, None, :] + rng.gumbel(size=(L, T, E))
    small = torch.from_numpy(
        np.argsort(-keys, axis=2)[:, :, :k].astype(np.int32)).to(DEV)
    run_both(E, R, S, k, T, L, small, ue.PLAN_BEST_FIT, ue.QUOTA_SEARCH)

    say("static rebalance: dsv3 again")
    run_both(d.experts, d.ranks, d.spare, d.topk, d.tokens, d.layers, dsv3)


def test_static_rebalance_refuses_oversized_calls():
    """128 layers of dsv3 size need about 23 MB of scratch: refused with
    UE_ESHAPE, every output left as it was."""
    d = W.CONFIGS["dsv3"]
    L, T = 128, d.tokens
    cfg = ue.ue_config(d.experts, d.ranks, d.spare, d.topk, T, L, 0, 0)
    routing = torch.zeros((L, T, d.topk), dtype=torch.int32, device=DEV)
    out = outputs(cfg, L, T, fill=-9)
    say("static rebalance: oversized call")
    with pytest.raises(ue.UEError) as err:
        ue.ue_rebalance_static(cfg, routing, **out)
    assert err.value.code == -2 and "scratch" in str(err.value)
    torch.cuda.synchronize()
    for key in KEYS:
        assert bool((out[key] == -9).all()), key
