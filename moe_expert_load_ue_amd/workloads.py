"""Seeded synthetic workloads shaped like the UltraEP pages' workloads.

The pages measure on production routing of 106B-671B MoE models, which is
not available; these generators stand in for it. They hold none of the
rebalancing arithmetic (no counting, planning or rerouting): they only draw
routing tensors, weights, gradients and activations from fixed seeds. Both
the HIP path and the CPU oracle consume what they produce.

Routing recipe (all configurations): Zipf rank i = 1..M has weight i^-s; a
seeded permutation maps Zipf ranks to expert ids. Each token draws its k
distinct experts by sampling without replacement in proportion to the
weights, done as Gumbel-top-k (argtopk of log w + Gumbel noise), and lists
them by descending key, the order a router's top-k returns. Every stream has
its own torch generator seeded with ``seed_of(config, stream)``; the same
device type and seed give the same tensor.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import torch


@dataclass(frozen=True)
class RoutingConfig:
    name: str
    layers: int          # layers (or microbatches) planned independently
    tokens: int          # T
    topk: int            # k
    experts: int         # E
    ranks: int           # R simulated expert-parallel ranks
    spare: int           # S spare slots per rank
    kind: str            # zipf | zipf_layers | hot | drift
    params: dict = field(default_factory=dict)
    hidden: int = 0      # activation width for the dispatch gather (0: none)

    @property
    def native(self) -> int:
        return self.experts // self.ranks

    @property
    def assignments(self) -> int:
        return self.tokens * self.topk


# The four routing workloads (E=64..256, k=8) and the streaming workload.
CONFIGS = {
    "tiny": RoutingConfig("tiny", 1, 4096, 8, 64, 8, 2, "zipf",
                          dict(s=1.2, seed=1)),
    "dsv3": RoutingConfig("dsv3", 58, 65536, 8, 256, 64, 1, "zipf_layers",
                          dict(s_lo=0.6, s_hi=1.4, seed=2)),
    "large_ep": RoutingConfig("large_ep", 1, 262144, 8, 256, 256, 1, "hot",
                              dict(s=1.0, n_hot=4, p_hot=0.4, seed=3)),
    "pipeline": RoutingConfig("pipeline", 16, 131072, 8, 128, 32, 2, "drift",
                              dict(s_first=0.5, s_last=1.5, seed=5),
                              hidden=4096),
}

# Replica weight sync / gradient reduction: 32 experts, three DeepSeek-V3
# sized expert matrices each (gate and up 7168x2048, down 2048x7168), bf16
# weights and fp32 gradients drawn N(0, 0.02), 64 replica buffers. Fan-out
# per expert: 4 replicas for 4 experts, 3 for 8, 2 for 4, 1 for 16.
STREAM_MATS = (7168 * 2048, 7168 * 2048, 2048 * 7168)
STREAM_FANOUT = (4,) * 4 + (3,) * 8 + (2,) * 4 + (1,) * 16
STREAM_SEED = 4


def seed_of(base: int, stream: int) -> int:
    return int(base) * 1_000_003 + int(stream)


def _gen(device, seed: int) -> torch.Generator:
    g = torch.Generator(device=torch.device(device))
    g.manual_seed(seed)
    return g


def _zipf_logw(m: int, s: float, device) -> torch.Tensor:
    """log of the Zipf weight of ranks 1..m (float32)."""
    ranks = torch.arange(1, m + 1, dtype=torch.float64, device=device)
    return (-s * torch.log(ranks)).to(torch.float32)


def _gumbel_topk(logw_by_id: torch.Tensor, tokens: int, k: int,
                 g: torch.Generator) -> torch.Tensor:
    """k distinct ids per token, sampled without replacement in proportion
    to exp(logw_by_id), listed by descending Gumbel key."""
    m = logw_by_id.numel()
    u = torch.rand((tokens, m), generator=g, device=logw_by_id.device)
    keys = logw_by_id[None, :] - torch.log(-torch.log(u))
    _, idx = torch.topk(keys, k, dim=1, largest=True, sorted=True)
    return idx


def zipf_layer(tokens: int, experts: int, k: int, s: float,
               perm: torch.Tensor, g: torch.Generator) -> torch.Tensor:
    """One layer of Zipf(s) top-k routing; ``perm[i]`` is the expert id of
    Zipf rank i+1."""
    device = perm.device
    logw = torch.empty(experts, dtype=torch.float32, device=device)
    logw[perm] = _zipf_logw(experts, s, device)
    return _gumbel_topk(logw, tokens, k, g).to(torch.int32)


def hot_layer(tokens: int, k: int, s: float, hot: torch.Tensor,
              others: torch.Tensor, p_hot: float,
              g: torch.Generator) -> torch.Tensor:
    """Zipf(s) routing over ``others`` plus the ``hot`` experts: each token
    includes each hot id independently with probability ``p_hot``; its
    remaining slots are Zipf picks without replacement over the others
    (``others[i]`` has Zipf rank i+1); hot ids sit at seeded random
    positions of the row."""
    device = g.device
    n_hot = hot.numel()
    include = torch.rand((tokens, n_hot), generator=g, device=device) < p_hot
    logw = _zipf_logw(others.numel(), s, device)
    picks = others[_gumbel_topk(logw, tokens, k, g)]          # [T, k]
    # Keep the included hot ids, then the first k - (#hot) Zipf picks.
    big = n_hot + k + 1
    prio_hot = torch.where(include,
                           torch.arange(n_hot, device=device)[None, :],
                           torch.full((1, n_hot), big, device=device))
    prio_pick = (n_hot + torch.arange(k, device=device))[None, :].expand(
        tokens, k)
    cand = torch.cat([hot[None, :].expand(tokens, n_hot), picks], dim=1)
    prio = torch.cat([prio_hot.expand(tokens, n_hot), prio_pick], dim=1)
    sel = torch.argsort(prio, dim=1, stable=True)[:, :k]
    row = torch.gather(cand, 1, sel)
    shuffle = torch.argsort(torch.rand((tokens, k), generator=g,
                                       device=device), dim=1)
    return torch.gather(row, 1, shuffle).to(torch.int32)


def layer_setup(cfg: RoutingConfig | str, layer: int, device="cpu"):
    """Seeded per-layer draws: ``(generator, exponent, zipf_order, hot)``.

    ``zipf_order[i]`` is the expert id of Zipf rank i+1; ``hot`` holds the
    hot expert ids (empty unless the configuration has hot experts). The
    returned generator continues the layer's stream."""
    if isinstance(cfg, str):
        cfg = CONFIGS[cfg]
    E, p = cfg.experts, cfg.params
    empty = torch.empty(0, dtype=torch.int64, device=device)
    if cfg.kind == "zipf":
        # one stream and one permutation shared by all layers
        g = _gen(device, seed_of(p["seed"], 0))
        perm = torch.randperm(E, generator=g, device=device)
        for _ in range(layer):
            _gumbel_topk(torch.zeros(E, device=device), cfg.tokens,
                         cfg.topk, g)
        return g, p["s"], perm, empty
    if cfg.kind == "zipf_layers":
        g = _gen(device, seed_of(p["seed"], layer))
        u = torch.rand((1,), generator=g, device=device, dtype=torch.float64)
        s = p["s_lo"] + (p["s_hi"] - p["s_lo"]) * float(u.item())
        perm = torch.randperm(E, generator=g, device=device)
        return g, s, perm, empty
    if cfg.kind == "hot":
        g = _gen(device, seed_of(p["seed"], layer))
        order = torch.randperm(E, generator=g, device=device)
        return g, p["s"], order[p["n_hot"]:], order[:p["n_hot"]]
    if cfg.kind == "drift":
        g0 = _gen(device, seed_of(p["seed"], 0))
        perm = torch.randperm(E, generator=g0, device=device)
        n = cfg.layers
        s = p["s_first"] + (p["s_last"] - p["s_first"]) * (
            layer / max(n - 1, 1))
        return _gen(device, seed_of(p["seed"], 1 + layer)), s, perm, empty
    raise ValueError(f"unknown routing kind {cfg.kind}")


def make_routing(cfg: RoutingConfig | str, device="cpu",
                 layers: int | None = None,
                 tokens: int | None = None, step: int = 0) -> torch.Tensor:
    """Routing tensor int32 ``[L, T, k]`` for a named configuration.

    ``layers``/``tokens`` may shrink the workload (same recipe, fewer layers
    or tokens) for fast tests. ``step`` > 0 gives the same layers at a later
    training step: the same exponent, expert order and hot set per layer
    (the same distribution), with fresh token draws."""
    if isinstance(cfg, str):
        cfg = CONFIGS[cfg]
    L = cfg.layers if layers is None else int(layers)
    T = cfg.tokens if tokens is None else int(tokens)
    E, k, p = cfg.experts, cfg.topk, cfg.params
    out = torch.empty((L, T, k), dtype=torch.int32, device=device)
    g = None
    for layer in range(L):
        if cfg.kind == "zipf" and g is not None:
            pass                    # one stream continues across layers
        else:
            g, s, order, hot = layer_setup(cfg, layer, device)
            if step:
                g = _gen(device, seed_of(p["seed"], (int(step) << 20) + layer))
        if cfg.kind == "hot":
            out[layer] = hot_layer(T, k, s, hot, order, p["p_hot"], g)
        else:
            out[layer] = zipf_layer(T, E, k, s, order, g)
    return out


def layer_exponents(cfg: RoutingConfig | str, device="cpu") -> list:
    """Zipf exponent used for each layer (for reports)."""
    if isinstance(cfg, str):
        cfg = CONFIGS[cfg]
    return [layer_setup(cfg, layer, device)[1] if cfg.kind != "zipf"
            else cfg.params["s"] for layer in range(cfg.layers)]


def make_activations(tokens: int, hidden: int, microbatch: int,
                     device="cpu", seed: int = 5) -> torch.Tensor:
    """bf16 activations ``[T, H]`` drawn N(0, 1), one seed per microbatch."""
    g = _gen(device, seed_of(seed * 100 + 7, microbatch))
    x = torch.randn((tokens, hidden), generator=g, device=device,
                    dtype=torch.float32)
    return x.to(torch.bfloat16)


@dataclass
class StreamBuffers:
    """Expert state for replica weight sync / gradient reduction.

    Each set is one dense tensor ``[experts or buffers, matrices, stride]``
    whose rows are padded to a multiple of 64 elements so every matrix starts
    16-byte aligned; ``elems`` is the matrix size and :meth:`mat` gives the
    exact view of one matrix."""
    master_w: torch.Tensor   # bf16 [E, M, stride]
    master_g: torch.Tensor   # fp32 [E, M, stride]
    spare_w: torch.Tensor    # bf16 [B, M, stride]
    spare_g: torch.Tensor    # fp32 [B, M, stride]
    rep_off: list            # CSR offsets per expert (entry 0 = master)
    rep_buf: list            # CSR entries: -1 for the master, else buffer id
    elems: int = 0

    def mat(self, name: str, i: int, m: int) -> torch.Tensor:
        return getattr(self, name)[i, m, :self.elems]

    def tables(self, name: str) -> list:
        t = getattr(self, name)
        return [[t[i, m, :self.elems] for m in range(t.shape[1])]
                for i in range(t.shape[0])]


def stream_csr(fanout=STREAM_FANOUT):
    """Replica table with ``fanout[e]`` replicas for expert e, buffers
    handed out in expert order."""
    rep_off, rep_buf, b = [0], [], 0
    for f in fanout:
        rep_buf.append(-1)
        for _ in range(f):
            rep_buf.append(b)
            b += 1
        rep_off.append(len(rep_buf))
    return rep_off, rep_buf, b


def make_stream_buffers(elems: int = STREAM_MATS[0], n_mats: int = 3,
                        fanout=STREAM_FANOUT, device="cpu",
                        seed: int = STREAM_SEED) -> StreamBuffers:
    rep_off, rep_buf, n_buf = stream_csr(fanout)
    E = len(fanout)
    stride = (elems + 63) // 64 * 64
    g = _gen(device, seed_of(seed, 0))
    mw = torch.zeros((E, n_mats, stride), dtype=torch.bfloat16, device=device)
    mg = torch.zeros((E, n_mats, stride), dtype=torch.float32, device=device)
    sg = torch.zeros((n_buf, n_mats, stride), dtype=torch.float32,
                     device=device)
    for t in (mw, mg, sg):
        for i in range(t.shape[0]):
            chunk = torch.randn((n_mats, elems), generator=g, device=device,
                                dtype=torch.float32) * 0.02
            t[i, :, :elems].copy_(chunk)
    sw = torch.empty((n_buf, n_mats, stride), dtype=torch.bfloat16,
                     device=device)
    sw.view(torch.int16).fill_(-1)      # 0xFFFF sentinel: a bf16 NaN
    return StreamBuffers(mw, mg, sw, sg, rep_off, rep_buf, elems)
