"""Python binding of libue, the MI355X (gfx950) per-layer MoE expert
rebalancing library (C ABI in ``include/ue.h``).

Argument marshalling only: every step of the path runs in the HIP kernels
behind the C ABI. PyTorch provides device memory and streams. The binding
raises at import of the first call if ``libue.so`` is not built; there is no
fallback implementation.

Functions carry the C names (``ue_load``, ``ue_plan``, ``ue_reroute``,
``ue_rebalance``,
``ue_weight_sync``, ``ue_grad_reduce``, ``ue_gather_rows``, ...) and take a
:class:`Context` plus torch tensors; :class:`Context` also exposes them as
methods without the prefix.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libue.so")

UE_OK = 0
STATUS = {0: "UE_OK", -1: "UE_EINVAL", -2: "UE_ESHAPE", -3: "UE_ENOMEM",
          -4: "UE_EHIP", -5: "UE_EUNSUPPORTED", -6: "UE_ESTATE"}


class UEError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"{STATUS.get(code, code)}: {msg}")
        self.code = code


class ue_config(ctypes.Structure):
    _fields_ = [("num_experts", ctypes.c_int32),
                ("num_ranks", ctypes.c_int32),
                ("spare_per_rank", ctypes.c_int32),
                ("topk", ctypes.c_int32),
                ("max_tokens", ctypes.c_int32),
                ("max_layers", ctypes.c_int32),
                ("plan_policy", ctypes.c_int32),
                ("quota_mode", ctypes.c_int32)]

PLAN_LEAST_LOADED, PLAN_BEST_FIT, PLAN_BEST_FIT_COVER, PLAN_BEST_FIT_ASCENDING = \
    0, 1, 2, 3
QUOTA_FIXED, QUOTA_SEARCH = 0, 1


PLACEMENT_FIELDS = ("words", "quota", "exhausted", "residual", "n_rep",
                    "rep_off", "rep_slot", "rep_cap", "slot_expert",
                    "slot_cap", "slot_off", "load_before", "load_after")


class ue_placement_layout(ctypes.Structure):
    _fields_ = [(f, ctypes.c_int32) for f in PLACEMENT_FIELDS]


# Every symbol the header declares, with its ctypes signature.
_vp, _i32, _i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
SIGNATURES = {
    "ue_create": (ctypes.c_int, [ctypes.POINTER(ue_config),
                                 ctypes.POINTER(_vp)]),
    "ue_destroy": (None, [_vp]),
    "ue_last_error": (ctypes.c_char_p, [_vp]),
    "ue_status_name": (ctypes.c_char_p, [ctypes.c_int]),
    "ue_get_placement_layout": (ctypes.c_int,
                                [_vp, ctypes.POINTER(ue_placement_layout)]),
    "ue_placement_bytes": (ctypes.c_size_t, [_vp]),
    "ue_load": (ctypes.c_int, [_vp, _vp, _i32, _i32, _vp, _vp, _vp]),
    "ue_plan": (ctypes.c_int, [_vp, _vp, _i32, _vp, _vp]),
    "ue_reroute": (ctypes.c_int, [_vp, _vp, _vp, _i32, _i32, _vp, _vp, _vp,
                                  _vp, _vp, _vp]),
    "ue_rebalance": (ctypes.c_int, [_vp, _vp, _i32, _i32, _vp, _vp, _vp, _vp,
                                    _vp, _vp, _vp, _vp, _vp]),
    "ue_set_timing": (ctypes.c_int, [_vp, ctypes.c_int]),
    "ue_kernel_times": (ctypes.c_int, [_vp, ctypes.POINTER(ctypes.c_float),
                                       _i32, ctypes.POINTER(_i32)]),
    "ue_register_experts": (ctypes.c_int, [_vp, _i32, _i32,
                                           ctypes.POINTER(_i64),
                                           ctypes.POINTER(_vp),
                                           ctypes.POINTER(_vp), _i32,
                                           ctypes.POINTER(_vp),
                                           ctypes.POINTER(_vp)]),
    "ue_weight_sync": (ctypes.c_int, [_vp, _vp, _vp, _i32, _vp]),
    "ue_grad_reduce": (ctypes.c_int, [_vp, _vp, _vp, _i32, _vp]),
    "ue_gather_rows": (ctypes.c_int, [_vp, _vp, _vp, _i32, _i32, _i32, _vp,
                                      _vp]),
    "ue_stale_loads": (ctypes.c_int, [_vp, _vp, _vp, _i32, _vp, _vp]),
    "ue_set_wait_limit": (ctypes.c_int, [_vp, ctypes.c_uint32]),
    "ue_rebalance_static": (ctypes.c_int, [ctypes.POINTER(ue_config), _vp,
                                           _i32, _i32, _vp, _vp, _vp, _vp,
                                           _vp, _vp, _vp, _vp, _vp]),
}

_lib = None


def library():
    """The loaded libue.so (raises if it is not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is not built; run "
                "`python -m moe_expert_load_ue_amd.build` (hipcc, gfx950)")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream, device):
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(stream.cuda_stream)


def _need(t, name, dtype, device, numel=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.device != device:
        raise ValueError(f"{name} must be on {device}, got {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if numel is not None and t.numel() != numel:
        raise ValueError(f"{name} must hold {numel} elements, has {t.numel()}")
    return t


class Context:
    """One ``ue_ctx`` on one device (see ``ue_create`` in ``ue.h``)."""

    def __init__(self, num_experts: int, num_ranks: int, spare_per_rank: int,
                 topk: int, max_tokens: int, max_layers: int = 1,
                 device=None, plan_policy: int = PLAN_LEAST_LOADED,
                 quota_mode: int = QUOTA_FIXED):
        self.device = torch.device(device if device is not None else
                                   f"cuda:{torch.cuda.current_device()}")
        self.E, self.R, self.S = int(num_experts), int(num_ranks), int(
            spare_per_rank)
        self.k, self.max_tokens = int(topk), int(max_tokens)
        self.max_layers = int(max_layers)
        self.plan_policy = int(plan_policy)
        self.quota_mode = int(quota_mode)
        self.N = self.E // self.R if self.R else 0
        self.P = self.R * (self.N + self.S)
        cfg = ue_config(self.E, self.R, self.S, self.k, self.max_tokens,
                        self.max_layers, self.plan_policy, self.quota_mode)
        h = ctypes.c_void_p()
        with torch.cuda.device(self.device):
            rc = library().ue_create(ctypes.byref(cfg), ctypes.byref(h))
        if rc != UE_OK:
            raise UEError(rc, "ue_create refused the configuration")
        self._h = h
        lay = ue_placement_layout()
        library().ue_get_placement_layout(self._h, ctypes.byref(lay))
        self.layout = {f: getattr(lay, f) for f in PLACEMENT_FIELDS}
        self.placement_words = lay.words
        self._registered = None

    # -- lifetime ----------------------------------------------------------
    def close(self):
        if getattr(self, "_h", None):
            library().ue_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def _check(self, rc, what):
        if rc != UE_OK:
            msg = library().ue_last_error(self._h).decode()
            raise UEError(rc, f"{what}: {msg}")

    # -- placement helpers --------------------------------------------------
    def new_placement(self, L: int) -> torch.Tensor:
        return torch.empty((L, self.placement_words), dtype=torch.int32,
                           device=self.device)

    def placement_fields(self, placement: torch.Tensor) -> dict:
        """Views of one or more placement blocks by field name."""
        pl = placement.reshape(-1, self.placement_words)
        lay, E, P, R = self.layout, self.E, self.P, self.R
        sizes = dict(rep_off=E + 1, rep_slot=P, rep_cap=P, slot_expert=P,
                     slot_cap=P, slot_off=P + 1, load_before=R, load_after=R)
        out = {k: pl[:, lay[k]] for k in ("quota", "exhausted", "residual",
                                          "n_rep")}
        for k, n in sizes.items():
            out[k] = pl[:, lay[k]:lay[k] + n]
        return out

    # -- steps (methods mirror the module-level functions) ------------------
    def load(self, routing, counts=None, invalid=None, stream=None):
        return ue_load(self, routing, counts, invalid, stream)

    def plan(self, counts, placement=None, stream=None):
        return ue_plan(self, counts, placement, stream)

    def reroute(self, routing, placement, **kw):
        return ue_reroute(self, routing, placement, **kw)

    def rebalance(self, routing, **kw):
        return ue_rebalance(self, routing, **kw)

    def register_experts(self, *a, **kw):
        return ue_register_experts(self, *a, **kw)

    def weight_sync(self, rep_off, rep_buf, n_experts=None, stream=None):
        return ue_weight_sync(self, rep_off, rep_buf, n_experts, stream)

    def grad_reduce(self, rep_off, rep_buf, n_experts=None, stream=None):
        return ue_grad_reduce(self, rep_off, rep_buf, n_experts, stream)

    def gather_rows(self, x, inv_perm, out=None, stream=None):
        return ue_gather_rows(self, x, inv_perm, out, stream)


def ue_create(num_experts, num_ranks, spare_per_rank, topk, max_tokens,
              max_layers=1, device=None, plan_policy=PLAN_LEAST_LOADED,
              quota_mode=QUOTA_FIXED) -> Context:
    return Context(num_experts, num_ranks, spare_per_rank, topk, max_tokens,
                   max_layers, device, plan_policy, quota_mode)


def ue_destroy(ctx: Context):
    ctx.close()


def ue_placement_bytes(ctx: Context) -> int:
    return int(library().ue_placement_bytes(ctx._h))


def ue_get_placement_layout(ctx: Context) -> dict:
    return dict(ctx.layout)


def ue_last_error(ctx: Context) -> str:
    return library().ue_last_error(ctx._h).decode()


def _routing_shape(ctx, routing):
    if routing.dim() == 2:
        routing = routing.unsqueeze(0)
    if routing.dim() != 3 or routing.shape[2] != ctx.k:
        raise ValueError(f"routing must be [L, T, {ctx.k}]")
    return routing, routing.shape[0], routing.shape[1]


def ue_load(ctx: Context, routing, counts=None, invalid=None, stream=None):
    """counts int32 [L, E] of routing int32 [L, T, k]."""
    routing, L, T = _routing_shape(ctx, routing)
    _need(routing, "routing", torch.int32, ctx.device)
    if counts is None:
        counts = torch.empty((L, ctx.E), dtype=torch.int32, device=ctx.device)
    _need(counts, "counts", torch.int32, ctx.device, L * ctx.E)
    if invalid is not None:
        _need(invalid, "invalid", torch.int32, ctx.device, L)
    rc = library().ue_load(ctx._h, _ptr(routing), L, T, _ptr(counts),
                           _ptr(invalid), _stream(stream, ctx.device))
    ctx._check(rc, "ue_load")
    return counts


def ue_plan(ctx: Context, counts, placement=None, stream=None):
    """Placement blocks int32 [L, words] from counts int32 [L, E]."""
    counts = counts.reshape(-1, ctx.E)
    L = counts.shape[0]
    _need(counts, "counts", torch.int32, ctx.device)
    if placement is None:
        placement = ctx.new_placement(L)
    _need(placement, "placement", torch.int32, ctx.device,
          L * ctx.placement_words)
    rc = library().ue_plan(ctx._h, _ptr(counts), L, _ptr(placement),
                           _stream(stream, ctx.device))
    ctx._check(rc, "ue_plan")
    return placement


def ue_stale_loads(ctx: Context, placement, counts, rank_loads=None,
                   stream=None):
    """Rank loads int32 [L, R] when placement blocks made from earlier counts
    are applied to new counts int32 [L, E]."""
    counts = counts.reshape(-1, ctx.E)
    L = counts.shape[0]
    _need(counts, "counts", torch.int32, ctx.device)
    _need(placement, "placement", torch.int32, ctx.device,
          L * ctx.placement_words)
    if rank_loads is None:
        rank_loads = torch.empty((L, ctx.R), dtype=torch.int32,
                                 device=ctx.device)
    _need(rank_loads, "rank_loads", torch.int32, ctx.device, L * ctx.R)
    rc = library().ue_stale_loads(ctx._h, _ptr(placement), _ptr(counts), L,
                                  _ptr(rank_loads),
                                  _stream(stream, ctx.device))
    ctx._check(rc, "ue_stale_loads")
    return rank_loads


def ue_reroute(ctx: Context, routing, placement, phys=None, rank_counts=None,
               perm=None, inv_perm=None, faults=None, with_inv=True,
               stream=None):
    """Physical routing, per-rank counts, dispatch permutation (and its
    inverse) for every layer. Returns a dict of the output tensors."""
    routing, L, T = _routing_shape(ctx, routing)
    _need(routing, "routing", torch.int32, ctx.device)
    _need(placement, "placement", torch.int32, ctx.device,
          L * ctx.placement_words)
    A = T * ctx.k
    dev = ctx.device

    def mk(t, shape, name, need=True):
        if t is None and need:
            t = torch.empty(shape, dtype=torch.int32, device=dev)
        if t is not None:
            n = 1
            for s in shape:
                n *= s
            _need(t, name, torch.int32, dev, n)
        return t

    phys = mk(phys, (L, T, ctx.k), "phys")
    rank_counts = mk(rank_counts, (L, ctx.R), "rank_counts")
    perm = mk(perm, (L, A), "perm")
    inv_perm = mk(inv_perm, (L, A), "inv_perm", with_inv)
    faults = mk(faults, (L,), "faults")
    rc = library().ue_reroute(ctx._h, _ptr(routing), _ptr(placement), L, T,
                              _ptr(phys), _ptr(rank_counts), _ptr(perm),
                              _ptr(inv_perm), _ptr(faults),
                              _stream(stream, dev))
    ctx._check(rc, "ue_reroute")
    return dict(phys=phys, rank_counts=rank_counts, perm=perm,
                inv_perm=inv_perm, faults=faults)


POISONED = 0x40000000   # bit of invalid / faults: a wait gave up


def ue_set_wait_limit(ctx: Context, polls: int):
    """Polls one cross-workgroup wait may take before it gives up (0: at
    once, marking every multi-group layer poisoned)."""
    ctx._check(library().ue_set_wait_limit(ctx._h, int(polls)),
               "ue_set_wait_limit")


def ue_set_timing(ctx: Context, enable: bool = True):
    ctx._check(library().ue_set_timing(ctx._h, int(bool(enable))),
               "ue_set_timing")


def ue_kernel_times(ctx: Context) -> list:
    """Durations (ms) of the kernels of the latest timed call."""
    ms = (ctypes.c_float * 8)()
    n = ctypes.c_int32()
    ctx._check(library().ue_kernel_times(ctx._h, ms, 8, ctypes.byref(n)),
               "ue_kernel_times")
    return [ms[i] for i in range(n.value)]


def ue_rebalance(ctx: Context, routing, counts=None, invalid=None,
                 placement=None, phys=None, rank_counts=None, perm=None,
                 inv_perm=None, faults=None, with_inv=True, stream=None):
    """load -> plan -> reroute in one call (see ``ue_rebalance`` in ue.h).
    Returns a dict with every output tensor."""
    routing, L, T = _routing_shape(ctx, routing)
    _need(routing, "routing", torch.int32, ctx.device)
    A = T * ctx.k
    dev = ctx.device

    def mk(t, shape, name, need=True):
        if t is None and need:
            t = torch.empty(shape, dtype=torch.int32, device=dev)
        if t is not None:
            n = 1
            for s in shape:
                n *= s
            _need(t, name, torch.int32, dev, n)
        return t

    counts = mk(counts, (L, ctx.E), "counts")
    invalid = mk(invalid, (L,), "invalid")
    placement = mk(placement, (L, ctx.placement_words), "placement")
    phys = mk(phys, (L, T, ctx.k), "phys")
    rank_counts = mk(rank_counts, (L, ctx.R), "rank_counts")
    perm = mk(perm, (L, A), "perm")
    inv_perm = mk(inv_perm, (L, A), "inv_perm", with_inv)
    faults = mk(faults, (L,), "faults")
    rc = library().ue_rebalance(ctx._h, _ptr(routing), L, T, _ptr(counts),
                                _ptr(invalid), _ptr(placement), _ptr(phys),
                                _ptr(rank_counts), _ptr(perm), _ptr(inv_perm),
                                _ptr(faults), _stream(stream, dev))
    ctx._check(rc, "ue_rebalance")
    return dict(counts=counts, invalid=invalid, placement=placement,
                phys=phys, rank_counts=rank_counts, perm=perm,
                inv_perm=inv_perm, faults=faults)


STATIC_SCRATCH_BYTES = 16 << 20


def placement_words(num_experts, num_ranks, spare_per_rank):
    """int32 words of one layer's placement block for a configuration (the
    layout ue_get_placement_layout reports, padded to 64 words)."""
    E, R = int(num_experts), int(num_ranks)
    P = R * (E // R + int(spare_per_rank))
    return (6 + E + 5 * P + 2 * R + 63) // 64 * 64


def ue_rebalance_static(cfg: ue_config, routing, counts, invalid, placement,
                        phys, rank_counts, perm, inv_perm, faults,
                        stream=None):
    """ue_rebalance with no context and no allocation (see
    ``ue_rebalance_static`` in ue.h): every output is the caller's
    preallocated tensor (invalid and inv_perm may be None)."""
    if not isinstance(cfg, ue_config):
        raise TypeError("cfg must be a ue_config")
    if routing.dim() == 2:
        routing = routing.unsqueeze(0)
    L, T, k = routing.shape
    if k != cfg.topk:
        raise ValueError(f"routing has {k} experts per token, cfg {cfg.topk}")
    dev = routing.device
    _need(routing, "routing", torch.int32, dev)
    A = T * k
    words = placement_words(cfg.num_experts, cfg.num_ranks,
                            cfg.spare_per_rank)
    for t, name, n in ((counts, "counts", L * cfg.num_experts),
                       (invalid, "invalid", L),
                       (placement, "placement", L * words),
                       (phys, "phys", L * A),
                       (rank_counts, "rank_counts", L * cfg.num_ranks),
                       (perm, "perm", L * A), (inv_perm, "inv_perm", L * A),
                       (faults, "faults", L)):
        if t is not None or name not in ("invalid", "inv_perm"):
            _need(t, name, torch.int32, dev, n)
    rc = library().ue_rebalance_static(
        ctypes.byref(cfg), _ptr(routing), L, T, _ptr(counts), _ptr(invalid),
        _ptr(placement), _ptr(phys), _ptr(rank_counts), _ptr(perm),
        _ptr(inv_perm), _ptr(faults), _stream(stream, dev))
    if rc != UE_OK:
        raise UEError(rc, library().ue_last_error(None).decode())


def ue_register_experts(ctx: Context, mat_elems, master_w=None, master_g=None,
                        spare_w=None, spare_g=None):
    """Registers expert state. ``master_w[e][m]`` etc. are tensors (bf16
    weights, fp32 gradients), or None for the kind not registered.
    ``mat_elems[m]`` is the element count of matrix m."""
    n_mats = len(mat_elems)
    n_exp = len(master_w if master_w is not None else master_g)
    sp = spare_w if spare_w is not None else spare_g
    n_buf = len(sp) if sp is not None else 0

    def table(rows, dtype):
        if rows is None:
            return None
        arr = (ctypes.c_void_p * (len(rows) * n_mats))()
        for i, row in enumerate(rows):
            if len(row) != n_mats:
                raise ValueError("every expert needs one tensor per matrix")
            for m, t in enumerate(row):
                _need(t, "expert tensor", dtype, ctx.device, mat_elems[m])
                arr[i * n_mats + m] = t.data_ptr()
        return arr

    tw, tg = table(master_w, torch.bfloat16), table(master_g, torch.float32)
    sw, sg = table(spare_w, torch.bfloat16), table(spare_g, torch.float32)
    elems = (ctypes.c_int64 * n_mats)(*[int(v) for v in mat_elems])
    rc = library().ue_register_experts(ctx._h, n_exp, n_mats, elems, tw, tg,
                                       n_buf, sw, sg)
    ctx._check(rc, "ue_register_experts")
    # keep the tensors alive while the library holds their pointers
    ctx._registered = (master_w, master_g, spare_w, spare_g)


def _csr(ctx, rep_off, rep_buf, n_experts):
    _need(rep_off, "rep_off", torch.int32, ctx.device)
    _need(rep_buf, "rep_buf", torch.int32, ctx.device)
    n = rep_off.numel() - 1 if n_experts is None else int(n_experts)
    return n


def ue_weight_sync(ctx: Context, rep_off, rep_buf, n_experts=None,
                   stream=None):
    n = _csr(ctx, rep_off, rep_buf, n_experts)
    rc = library().ue_weight_sync(ctx._h, _ptr(rep_off), _ptr(rep_buf), n,
                                  _stream(stream, ctx.device))
    ctx._check(rc, "ue_weight_sync")


def ue_grad_reduce(ctx: Context, rep_off, rep_buf, n_experts=None,
                   stream=None):
    n = _csr(ctx, rep_off, rep_buf, n_experts)
    rc = library().ue_grad_reduce(ctx._h, _ptr(rep_off), _ptr(rep_buf), n,
                                  _stream(stream, ctx.device))
    ctx._check(rc, "ue_grad_reduce")


def replica_table(ctx: Context, placement, layer: int = 0):
    """The replica table of one layer's placement block as the (rep_off,
    rep_buf) pair that ue_weight_sync and ue_grad_reduce take: views of the
    block's rep_off and rep_slot fields, on the device. With one buffer
    registered per physical slot (buffer p for slot p), the plan drives the
    sync and the reduction directly."""
    blk = placement.reshape(-1, ctx.placement_words)[layer]
    lay = ctx.layout
    return (blk[lay["rep_off"]:lay["rep_off"] + ctx.E + 1],
            blk[lay["rep_slot"]:lay["rep_slot"] + ctx.P])


def ue_gather_rows(ctx: Context, x, inv_perm, out=None, stream=None):
    """out[pos] = x[perm[pos] // k] for one layer's inverse permutation."""
    if x.dim() != 2:
        raise ValueError("x must be [T, H]")
    T, H = x.shape
    _need(x, "x", torch.bfloat16, ctx.device)
    _need(inv_perm, "inv_perm", torch.int32, ctx.device, T * ctx.k)
    if out is None:
        out = torch.empty((T * ctx.k, H), dtype=torch.bfloat16,
                          device=ctx.device)
    _need(out, "out", torch.bfloat16, ctx.device, T * ctx.k * H)
    rc = library().ue_gather_rows(ctx._h, _ptr(x), _ptr(inv_perm), T, ctx.k,
                                  H, _ptr(out), _stream(stream, ctx.device))
    ctx._check(rc, "ue_gather_rows")
    return out
