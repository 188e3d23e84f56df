"""CPU oracle for the per-layer MoE expert-rebalancing path.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` import this package. The product
library never imports, links or calls it, and it shares no code with the
HIP path: the integer steps (load, plan, reroute/layout) are the plain C in
``ue_oracle.c`` driven through ctypes, the streaming steps are numpy.

Steps and the passages they follow (page titles as they appear on the web):

* ``load`` -- exact per-expert load, the "exact-load" property stated in the
  UltraEP abstract (arXiv 2606.04101) and the "Load computation" component of
  "How dots-infra/ultraep works" (gitdiagram, component list).
* ``plan`` -- the quota-driven scheduler of the UltraEP news write-up
  (section on how balancing in 300 microseconds works); "Placement planning"
  on the gitdiagram page. The concrete rule is spelled out in ``ue_oracle.c``.
* ``reroute`` -- "Routing expansion": logical routing becomes physical
  routing for token dispatch (gitdiagram connection list), plus the stable
  dispatch permutation that orders assignments by physical slot.
* ``weight_sync`` -- "Replica weight sync": every replica receives the master
  weights (gitdiagram summary: replicas are synchronised before expert
  execution).
* ``grad_reduce`` -- "Replica gradient reduction": master gradient plus the
  sum of its replicas' gradients (gitdiagram summary: replica gradients are
  reduced during backward). Computed in float64.
* ``gather`` -- token dispatch into physical-expert order (gitdiagram: token
  dispatch consumes the physical routing).
* ``stale_loads`` -- rank loads when a plan made from earlier counts is
  applied to new ones: the periodic, history-driven balancing the pages
  contrast with exact-load balancing (UltraEP abstract; news write-up,
  section on the problem UltraEP solves).
"""
from __future__ import annotations

import contextlib
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ue_oracle.c")
_LIB = os.path.join(_HERE, "libue_oracle.so")
_lib = None


def build(out: str | None = None, src: str | None = None,
          strict: bool = True) -> str:
    """Compile the oracle C source (default ``ue_oracle.c``) into a shared
    library (default ``libue_oracle.so`` next to it) with gcc; ``strict``
    turns warnings into errors."""
    out = out or _LIB
    cmd = ["gcc", "-O2", "-std=c11", "-Wall", "-Wextra"]
    cmd += ["-Werror"] if strict else ["-w"]
    cmd += ["-fPIC", "-shared", "-o", out, src or _SRC]
    subprocess.run(cmd, check=True)
    return out


def load_library(path: str):
    """Open a compiled oracle library and declare its signatures."""
    lib = ctypes.CDLL(path)
    i32p = np.ctypeslib.ndpointer(dtype=np.int32, flags="C_CONTIGUOUS")
    lib.orc_load.restype = ctypes.c_int64
    lib.orc_load.argtypes = [i32p, ctypes.c_int64, ctypes.c_int32, i32p]
    lib.orc_plan.restype = ctypes.c_int
    lib.orc_plan.argtypes = [i32p, ctypes.c_int32, ctypes.c_int32,
                             ctypes.c_int32, ctypes.c_int32,
                             ctypes.c_int32] + [i32p] * 9
    lib.orc_reroute.restype = ctypes.c_int64
    lib.orc_reroute.argtypes = [i32p, ctypes.c_int64, ctypes.c_int32,
                                ctypes.c_int32, ctypes.c_int32] + [i32p] * 8
    return lib


def _get():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        _lib = load_library(_LIB)
    return _lib


@contextlib.contextmanager
def library(path: str):
    """Run the oracle functions against another compiled copy of the C
    source (used by the tests that plant mistakes in the oracle)."""
    global _lib
    saved = _get()
    _lib = load_library(path)
    try:
        yield _lib
    finally:
        _lib = saved


def load(routing: np.ndarray, n_experts: int):
    """Per-layer expert counts.

    ``routing`` is int32 ``[L, T, k]`` (or ``[T, k]``, or flat ``[T*k]`` for
    one layer). Returns ``(counts int32 [L, E], invalid int64 [L])`` where
    ``invalid`` counts ids outside ``[0, E)``."""
    r = np.ascontiguousarray(routing, dtype=np.int32)
    if r.ndim <= 2:
        r = r.reshape(1, -1)
    r = r.reshape(r.shape[0], -1)
    lib = _get()
    counts = np.zeros((r.shape[0], n_experts), dtype=np.int32)
    invalid = np.zeros(r.shape[0], dtype=np.int64)
    for layer in range(r.shape[0]):
        row = np.ascontiguousarray(r[layer])
        out = np.zeros(n_experts, dtype=np.int32)
        invalid[layer] = lib.orc_load(row, row.size, n_experts, out)
        counts[layer] = out
    return counts, invalid


def plan(counts: np.ndarray, n_ranks: int, n_spare: int,
         policy: int = 0, quota_mode: int = 0) -> dict:
    """Quota plan for one layer from its ``counts`` (int32 ``[E]``).
    ``policy`` 0: least-loaded destination; 1: best fit for a chunk the
    least-loaded rank would not fill; 2: best fit with the candidates in
    covering order (amounts one rank can take first, smallest first, then
    the rest, largest first; fixed at the plain quota); 3: best fit with
    the candidates by ascending amount at the plain quota. ``quota_mode`` 0:
    Q = ceil(total / R); 1: the lowest of 64 raised quotas at which
    nothing is left."""
    c = np.ascontiguousarray(counts, dtype=np.int32).reshape(-1)
    E, R, S = c.size, int(n_ranks), int(n_spare)
    if E % R != 0:
        raise ValueError("number of experts must be a multiple of ranks")
    P = R * (E // R + S)
    out = dict(
        scalars=np.zeros(4, np.int32),
        rep_off=np.zeros(E + 1, np.int32),
        rep_slot=np.zeros(P, np.int32),
        rep_cap=np.zeros(P, np.int32),
        slot_expert=np.zeros(P, np.int32),
        slot_cap=np.zeros(P, np.int32),
        slot_off=np.zeros(P + 1, np.int32),
        load_before=np.zeros(R, np.int32),
        load_after=np.zeros(R, np.int32),
    )
    rc = _get().orc_plan(c, E, R, S, int(policy), int(quota_mode),
                         out["scalars"],
                         out["rep_off"],
                         out["rep_slot"], out["rep_cap"], out["slot_expert"],
                         out["slot_cap"], out["slot_off"], out["load_before"],
                         out["load_after"])
    if rc != 0:
        raise ValueError("oracle plan refused the shape")
    q, exhausted, residual, n_rep = (int(v) for v in out["scalars"])
    out.update(quota=q, exhausted=exhausted, residual=residual, n_rep=n_rep,
               E=E, R=R, S=S, N=E // R, P=P, policy=int(policy),
               quota_mode=int(quota_mode))
    return out


def reroute(routing: np.ndarray, pl: dict, perm_fill: int = -1) -> dict:
    """Physical routing, dispatch permutation, its inverse and per-rank
    counts for one layer. ``routing`` is the layer's flat assignments."""
    r = np.ascontiguousarray(routing, dtype=np.int32).reshape(-1)
    A = r.size
    phys = np.empty(A, np.int32)
    perm = np.full(A, perm_fill, np.int32)
    inv = np.empty(A, np.int32)
    rank_counts = np.zeros(pl["R"], np.int32)
    faults = _get().orc_reroute(r, A, pl["E"], pl["R"], pl["S"],
                                pl["rep_off"], pl["rep_slot"], pl["rep_cap"],
                                pl["slot_off"], phys, perm, inv, rank_counts)
    return dict(phys=phys, perm=perm, inv_perm=inv, rank_counts=rank_counts,
                faults=int(faults))


def rebalance(routing: np.ndarray, n_experts: int, n_ranks: int,
              n_spare: int, policy: int = 0, quota_mode: int = 0) -> list:
    """load -> plan -> reroute for every layer of ``routing [L, T, k]``."""
    r = np.ascontiguousarray(routing, dtype=np.int32)
    if r.ndim <= 2:
        r = r.reshape(1, -1)
    r = r.reshape(r.shape[0], 1, -1)
    counts, invalid = load(r, n_experts)
    r = r.reshape(r.shape[0], -1)
    res = []
    for layer in range(r.shape[0]):
        pl = plan(counts[layer], n_ranks, n_spare, policy, quota_mode)
        rr = reroute(r[layer], pl)
        pl.update(rr)
        pl["counts"] = counts[layer]
        pl["invalid"] = int(invalid[layer])
        res.append(pl)
    return res


def stale_loads(pl: dict, counts_new: np.ndarray) -> np.ndarray:
    """Rank loads when the plan ``pl`` (made from earlier counts) is applied
    to one layer's new counts (int ``[E]``): the periodic, historical-load
    balancing that the UltraEP abstract (arXiv 2606.04101) and the news
    write-up (section on the problem UltraEP solves) contrast with exact-load
    balancing. The plan keeps its replicas and their proportions: of expert
    e's n new assignments, with old capacities c_1..c_m (master first, then
    replicas in table order) summing to C, replica i takes those j with
    floor(n * c_<i / C) <= j < floor(n * c_<=i / C) -- the capacity prefix
    scaled from C to n. An expert the plan saw no tokens of (C = 0) stays
    whole on its master. Returns int64 ``[R]``."""
    n_new = np.asarray(counts_new, dtype=np.int64).reshape(-1)
    E, R = pl["E"], pl["R"]
    NS = pl["N"] + pl["S"]
    loads = np.zeros(R, dtype=np.int64)
    for e in range(E):
        n = int(n_new[e])
        lo, hi = int(pl["rep_off"][e]), int(pl["rep_off"][e + 1])
        caps = [int(c) for c in pl["rep_cap"][lo:hi]]
        slots = [int(p) for p in pl["rep_slot"][lo:hi]]
        C = sum(caps)
        if C == 0:
            loads[slots[0] // NS] += n
            continue
        before = 0
        acc = 0
        for slot, cap in zip(slots, caps):
            acc += cap
            upto = (n * acc) // C
            loads[slot // NS] += upto - before
            before = upto
    return loads


def weight_sync(master: np.ndarray, n_replicas: int) -> list:
    """Every replica receives a bitwise copy of the master weights."""
    return [np.array(master, copy=True) for _ in range(n_replicas)]


def grad_reduce(master: np.ndarray, replicas: list) -> np.ndarray:
    """Master gradient plus every replica's gradient, in float64."""
    acc = np.asarray(master, dtype=np.float64).copy()
    for rep in replicas:
        acc = acc + np.asarray(rep, dtype=np.float64)
    return acc


def grad_reduce_rounded(master: np.ndarray, replicas: list) -> np.ndarray:
    """The same sum as the fp32 gradient it becomes: one binary64 add at a
    time from the master through the replicas in table order (no fused or
    reassociated adds), then one rounding to binary32, nearest even."""
    acc = np.array(master, dtype=np.float64, copy=True)
    for rep in replicas:
        acc = np.add(acc, np.asarray(rep, dtype=np.float64), dtype=np.float64)
    return acc.astype(np.float32)


def gather(x: np.ndarray, perm: np.ndarray, k: int) -> np.ndarray:
    """Row ``pos`` of the output is the token row that assignment
    ``perm[pos]`` came from (token = assignment div k)."""
    return np.asarray(x)[np.asarray(perm, dtype=np.int64) // int(k)]
