/*
 * ue.h -- C ABI of the MI355X (gfx950) per-layer MoE expert-rebalancing
 * library (libue.so).
 *
 * The library implements the data-parallel hot path of an exact-load,
 * real-time expert balancer: count each expert's load from the post-gating
 * routing, plan replicas of hot experts onto spare slots of expert-parallel
 * ranks under a quota, expand logical expert ids to physical replica ids
 * with the stable dispatch permutation, copy master weights into replicas,
 * and sum replica gradients into the masters.
 *
 * Sources: the gitdiagram page "How dots-infra/ultraep works" (summary and
 * connection list: the framework registers expert pointers and passes
 * routing; the manager profiles loads, updates placement, syncs weights,
 * reroutes tokens and reduces gradients); the UltraEP news write-up
 * ("UltraEP ot Xiaohongshu: balansirovka MoE-ekspertov za 300 mks"), section
 * on how balancing in 300 microseconds works (quota-driven scheduler, every
 * microbatch and layer, right after gating; persistent tile streaming of
 * expert state); the UltraEP abstract, arXiv 2606.04101 ("exact-load,
 * real-time balancer").
 *
 * Conventions for every call:
 *  - Pointers named as device pointers must point to device memory of the
 *    current HIP device (e.g. torch CUDA tensors on ROCm). Host pointers are
 *    read before the call returns and not kept, unless stated.
 *  - `stream` is a hipStream_t passed as void*; NULL means the null stream.
 *    Every call is asynchronous and stream-ordered; results are valid once
 *    the stream reaches that point. No call synchronises with the host.
 *  - The return value is UE_OK (0) or a negative ue_status. Every argument
 *    is validated before anything is launched or written: a refused call
 *    leaves all outputs untouched. The reason is in ue_last_error().
 *  - A context is not thread-safe: one host thread at a time. Its routing
 *    calls (ue_load, ue_plan, ue_reroute, ue_rebalance) use the context's
 *    workspace and must not overlap one another in time on different
 *    streams. ue_weight_sync, ue_grad_reduce and ue_gather_rows use no
 *    workspace and may run on another stream beside them (the next layer's
 *    rebalance beside this layer's sync), while kernel timing is off and
 *    the registered tables are not replaced meanwhile.
 *  - All shapes are int32; the number of assignments per layer, T*k, must
 *    stay below 2^30.
 *  - The workgroups of ue_reroute combine per-tile counts through bounded
 *    waits on each other (decoupled lookback); no other call waits across
 *    workgroups (ue_load and ue_rebalance count every tile on its own and
 *    scan the counts in the planner's launch). A wait that outlasts the
 *    context's wait limit (ue_set_wait_limit) gives up, and every kernel
 *    still runs to its end; the layer is then marked poisoned: bit 30
 *    (0x40000000, UE_POISONED) is set in that layer's `faults` word, the
 *    other bits keep their counts, and the layer's other outputs are
 *    unspecified.
 */
#ifndef UE_H
#define UE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum ue_status {
    UE_OK = 0,
    UE_EINVAL = -1,       /* null pointer, bad alignment, bad value       */
    UE_ESHAPE = -2,       /* dimensions outside what the context allows   */
    UE_ENOMEM = -3,       /* device allocation failed                     */
    UE_EHIP = -4,         /* a HIP runtime call failed                    */
    UE_EUNSUPPORTED = -5, /* configuration outside what the kernels cover */
    UE_ESTATE = -6        /* call made in the wrong state (e.g. unregistered) */
} ue_status;

/* Shape of the simulated expert-parallel machine and the size limits of
 * one context.
 *   num_experts E      logical experts, 1..1024
 *   num_ranks R        expert-parallel ranks, divides E; N = E / R experts
 *                      live natively on each rank (expert e on rank e / N,
 *                      native slot e mod N)
 *   spare_per_rank S   empty replica slots per rank, 0..64; physical slot id
 *                      p = r*(N+S) + s, natives s < N, spares N <= s < N+S;
 *                      P = R*(N+S) <= 4096
 *   topk k             experts per token, 1..E
 *   max_tokens         largest T of any call (T*k < 2^30)
 *   max_layers         largest L (layers or microbatches) of any call
 *   plan_policy        rule of the planner (see ue_plan):
 *                      UE_PLAN_LEAST_LOADED (0), UE_PLAN_BEST_FIT (1),
 *                      UE_PLAN_BEST_FIT_COVER (2) or
 *                      UE_PLAN_BEST_FIT_ASCENDING (3)
 *   quota_mode         how the planner sets the quota (see ue_plan):
 *                      UE_QUOTA_FIXED (0) or UE_QUOTA_SEARCH (1)           */
typedef struct ue_config {
    int32_t num_experts;
    int32_t num_ranks;
    int32_t spare_per_rank;
    int32_t topk;
    int32_t max_tokens;
    int32_t max_layers;
    int32_t plan_policy;
    int32_t quota_mode;
} ue_config;

enum {
    UE_PLAN_LEAST_LOADED = 0,  /* every chunk to the least-loaded rank     */
    UE_PLAN_BEST_FIT = 1,      /* a chunk the least-loaded rank would not
                                  fill goes to the eligible rank with the
                                  smallest headroom that holds it          */
    UE_PLAN_BEST_FIT_COVER = 2, /* best fit, candidates in covering order:
                                  amounts one rank can take first, smallest
                                  first, then the rest, largest first      */
    UE_PLAN_BEST_FIT_ASCENDING = 3 /* best fit, candidates by their amount
                                  at Q0, smallest first                   */
};

enum {
    UE_QUOTA_FIXED = 0,        /* Q = ceil(sum(counts) / R)                 */
    UE_QUOTA_SEARCH = 1        /* the lowest of Q0 + j*ceil(Q0/256), j < 64,
                                  at which nothing is left over (else Q0)   */
};

/* Bit of a layer's invalid / faults word marking a wait that gave up. */
#define UE_POISONED 0x40000000

typedef struct ue_ctx ue_ctx;

/* Creates a context on the current HIP device and allocates its device
 * workspace once (per-tile scan state and counters, sized from the
 * limits). *out is set only on success. Errors: UE_EINVAL (null),
 * UE_EUNSUPPORTED (limits above), UE_ENOMEM, UE_EHIP. */
int ue_create(const ue_config *cfg, ue_ctx **out);

/* Frees the workspace and the context. Registered expert memory is the
 * caller's and is not freed. Waits for the device to finish pending work
 * of the context. NULL is accepted. */
void ue_destroy(ue_ctx *ctx);

/* Last error message of the context ("" if none); valid until the next
 * call on the context. With ctx NULL: the message of the calling thread's
 * last ue_rebalance_static call. */
const char *ue_last_error(const ue_ctx *ctx);

/* Short name of a status code. */
const char *ue_status_name(int status);

/* ---------------------------------------------------------------------
 * Placement block: one per layer, int32 words at fixed offsets.
 * ue_get_placement_layout() reports the offsets (in int32 words from the start
 * of a layer's block) and the block size. Fields:
 *   quota        Q = ceil(sum(counts) / R)
 *   exhausted    1 if overloaded ranks kept excess because no rank had a
 *                free spare slot and load < Q, else 0
 *   residual     sum over ranks of max(0, load_after - Q)
 *   n_rep        entries used in the replica table (masters included)
 *   rep_off[E+1] replica table offsets per expert (CSR)
 *   rep_slot[P]  physical slot of each replica; per expert the master
 *                (native slot) first, then replicas in creation order;
 *                entries >= n_rep hold -1
 *   rep_cap[P]   assignments routed to each replica (0 beyond n_rep)
 *   slot_expert[P] logical expert held by each slot, -1 for an unused spare
 *   slot_cap[P]  assignments routed to each slot (0 if unused)
 *   slot_off[P+1] exclusive prefix sum of slot_cap: where each slot's
 *                assignments start in the dispatch permutation
 *   load_before[R], load_after[R]  rank loads under the native placement
 *                and after the plan                                        */
typedef struct ue_placement_layout {
    int32_t words;          /* int32 words per layer block */
    int32_t quota, exhausted, residual, n_rep;
    int32_t rep_off, rep_slot, rep_cap;
    int32_t slot_expert, slot_cap, slot_off;
    int32_t load_before, load_after;
} ue_placement_layout;

int ue_get_placement_layout(const ue_ctx *ctx, ue_placement_layout *out);

/* Bytes of one layer's placement block (words * 4). 0 for a NULL ctx. */
size_t ue_placement_bytes(const ue_ctx *ctx);

/* ---------------------------------------------------------------------
 * Exact per-expert load ("Load computation"; the balancer is exact-load).
 *   routing  device, int32 [L, T, k], logical expert ids, flat assignment
 *            order a = t*k + j within a layer
 *   counts   device, int32 [L, E] out: counts[l][e] = #{a : routing = e}
 *   invalid  device, int32 [L] out, may be NULL: ids outside [0, E) per
 *            layer (such ids are not counted)
 * L in 1..max_layers, T in 0..max_tokens. */
int ue_load(ue_ctx *ctx, const int32_t *routing, int32_t L, int32_t T,
            int32_t *counts, int32_t *invalid, void *stream);

/* Quota replica plan ("Placement planning", the quota-driven scheduler),
 * per layer, from counts alone:
 *   Q = ceil(sum(counts)/R); experts of ranks whose load exceeds Q are
 *   visited heaviest first (count desc, id asc); each spills its rank's
 *   excess, chunk by chunk, into the lowest free spare slot of the
 *   least-loaded rank (ties: lowest id) that has a free spare slot and load
 *   < Q; chunk = min(source excess, expert remainder, destination
 *   headroom); with no such rank the plan stops (exhausted = 1).
 *   Under UE_PLAN_BEST_FIT, when the amount left (min of source excess and
 *   expert remainder) is below the least-loaded rank's headroom, it goes
 *   whole to the eligible rank with the smallest headroom >= the amount
 *   (ties: lowest id) instead.
 *   UE_PLAN_BEST_FIT_COVER places chunks as UE_PLAN_BEST_FIT does but
 *   visits the candidates in covering order, fixed at Q0: a candidate's
 *   amount at a quota is what its rank must shed below it that the rank's
 *   heavier experts (count desc, id asc) do not; H0 is the largest
 *   headroom Q0 - load among ranks with a spare slot; candidates whose
 *   amount at Q0 is at most H0 come first (amount asc, id asc), then the
 *   others (amount desc, id asc); each places its amount at the pass's
 *   quota. With one spare slot per rank every destination takes one
 *   chunk, and this order keeps the small pieces for the small amounts.
 *   UE_PLAN_BEST_FIT_ASCENDING is the same with every candidate in the
 *   first group: all amounts at Q0 ascending (ties: lowest id), so the
 *   large amounts too go smallest first and the largest, which needs the
 *   most pieces, is placed last, into what the others left.
 *   Under UE_QUOTA_SEARCH the plan above is made at the quotas
 *   Q0 + j*ceil(Q0/256), j = 0..63 (Q0 = ceil(sum(counts)/R)), in order,
 *   and the first that leaves nothing over is kept; with none, Q0 stands.
 *   The placement's quota field holds the quota used.
 *   counts     device, int32 [L, E] (e.g. from ue_load); every count >= 0
 *              and each layer's sum below 2^30 (ue_load's counts always
 *              are). A layer that breaks this is not planned: its block
 *              gets exhausted = -1 and an empty replica table (rep_off all
 *              0, n_rep 0), so every assignment of a later ue_reroute with
 *              it is a fault.
 *   placement  device, L blocks of ue_placement_bytes() bytes, out
 * Fully on the device; nothing returns to the host. */
int ue_plan(ue_ctx *ctx, const int32_t *counts, int32_t L, void *placement,
            void *stream);

/* Routing expansion and dispatch layout ("Routing expansion": physical
 * routing for token dispatch). For every assignment a of layer l with
 * logical expert e, j = number of earlier assignments of e in flat order;
 * the replica of e whose capacity prefix (master first) covers j gets it:
 *   phys        device, int32 [L, T, k] out: physical slot id
 *   rank_counts device, int32 [L, R] out: assignments per rank, counted
 *               from phys
 *   perm        device, int32 [L, T*k] out: perm[pos] = a, the stable sort
 *               of assignments by physical slot (pos = slot_off[p] + j -
 *               prefix)
 *   inv_perm    device, int32 [L, T*k] out, may be NULL: inv_perm[a] = pos
 *   faults      device, int32 [L] out, may be NULL: assignments that could
 *               not be placed (id outside [0, E), or beyond the plan's
 *               capacity for its expert); their phys and inv_perm are -1
 * The placement must come from ue_plan on the counts of this routing; with
 * faults > 0 perm is unspecified. */
int ue_reroute(ue_ctx *ctx, const int32_t *routing, const void *placement,
               int32_t L, int32_t T, int32_t *phys, int32_t *rank_counts,
               int32_t *perm, int32_t *inv_perm, int32_t *faults,
               void *stream);

/* One rebalance of L layers in one call: ue_load, ue_plan and ue_reroute
 * with the same arguments and results as those three calls in a row (every
 * output of each is an output here; invalid and inv_perm may be NULL). The
 * pages rebalance right after gating, on the critical path, for every
 * microbatch and layer; this entry point is that path as three launches
 * with no host work between them. The reroute reuses the per-tile expert
 * prefixes the load kernel publishes, so it reads the routing once more but
 * never waits on another workgroup; and since the plan is made from these
 * very counts, rank_counts and faults follow from it (the plan's loads
 * after, and the ids out of range) and the planner's launch writes them.
 * Arguments are validated before the first launch; a refusal leaves every
 * output untouched. */
int ue_rebalance(ue_ctx *ctx, const int32_t *routing, int32_t L, int32_t T,
                 int32_t *counts, int32_t *invalid, void *placement,
                 int32_t *phys, int32_t *rank_counts, int32_t *perm,
                 int32_t *inv_perm, int32_t *faults, void *stream);

/* Rank loads under an earlier plan: the periodic, historical-load
 * balancing that the UltraEP abstract (arXiv 2606.04101) and the news
 * write-up (section on the problem UltraEP solves) contrast with exact-load
 * balancing. Each layer's placement block (from ue_plan on earlier counts)
 * is applied to that layer's new counts: the plan keeps its replicas and
 * their proportions, so of expert e's n new assignments, with old
 * capacities c_1..c_m (master first, then replicas in table order) summing
 * to C, replica i takes floor(n * c_<=i / C) - floor(n * c_<i / C); an
 * expert the plan saw no tokens of (C = 0) stays whole on its master.
 *   placement   device, L blocks from ue_plan (on other counts)
 *   counts      device, int32 [L, E], the new counts (each >= 0, the sum of
 *               a layer below 2^30)
 *   rank_loads  device, int32 [L, R] out: assignments per rank
 * Exact integer arithmetic; the same covering rule as ue_reroute with the
 * capacities rescaled. Errors: UE_EINVAL (null or misaligned pointers),
 * UE_ESHAPE (L outside 1..max_layers). */
int ue_stale_loads(ue_ctx *ctx, const void *placement, const int32_t *counts,
                   int32_t L, int32_t *rank_loads, void *stream);

/* Polls one cross-workgroup wait of ue_reroute may take before it gives up
 * and marks its layer poisoned (see the conventions above); default
 * 4,194,304, far beyond any wait of a healthy device. 0 makes every wait
 * give up without polling, so every layer of more than one routing tile is
 * marked: a way to exercise the error path with every kernel still ending
 * normally. Applies to later calls on the context. */
int ue_set_wait_limit(ue_ctx *ctx, uint32_t polls);

/* ue_rebalance without a context and without allocating: for callers
 * that cannot allocate device memory where they rebalance (code under
 * stream capture, tight serving loops, harnesses that forbid allocation).
 * Same arguments, outputs and results as ue_rebalance, with the context
 * replaced by its configuration (validated as ue_create does: the same
 * UE_EUNSUPPORTED cases; L <= max_layers and T <= max_tokens).
 * Its scratch is one device array of UE_STATIC_SCRATCH_BYTES (16 MiB) in
 * the library, which every device the library runs on holds until the
 * process ends. A call needs, with tiles = max(1, ceil(T*k / 2048)) and
 * groups = ceil(tiles / 8), each term rounded up to 256 bytes:
 *   4 L groups E + 2 L (tiles + groups) E
 * bytes (the 58-layer dsv3 rebalance, E=256, T=65536, k=8: 10.5 MB). A call
 * needing more is refused with UE_ESHAPE before anything is launched.
 * Every scratch word a call reads it has written itself, so nothing is
 * cleared between calls (and the call may be captured in a graph). Calls
 * share the array: calls that overlap in time on one device race and give
 * wrong results; order them on one stream. The first call on a device
 * looks up the array's address there (hipGetSymbolAddress).
 * Calls no allocation routine. Error text: ue_last_error(NULL). */
#define UE_STATIC_SCRATCH_BYTES (16u << 20)
int ue_rebalance_static(const ue_config *cfg, const int32_t *routing,
                        int32_t L, int32_t T, int32_t *counts,
                        int32_t *invalid, void *placement, int32_t *phys,
                        int32_t *rank_counts, int32_t *perm,
                        int32_t *inv_perm, int32_t *faults, void *stream);

/* Kernel timing. With timing enabled, every call records a HIP event on its
 * stream before its first kernel and after each kernel it launches.
 * ue_kernel_times waits for the latest call's last event and writes the
 * duration in milliseconds of each of its kernels, in launch order, to
 * ms[0 .. *n-1] (at most max_n values; *n is the number that call launched).
 * Off by default; enabling it costs one event per kernel. Errors:
 * UE_ESTATE if timing is off or no call has run since it was enabled. */
int ue_set_timing(ue_ctx *ctx, int enable);
int ue_kernel_times(ue_ctx *ctx, float *ms, int32_t max_n, int32_t *n);

/* ---------------------------------------------------------------------
 * Expert state ("registers expert pointers"). Stores device pointers to
 * n_experts master experts and n_buffers replica buffers, each made of
 * n_mats matrices; matrix m has mat_elems[m] elements in every expert and
 * buffer. Weights are bf16 (2 bytes per element), gradients fp32.
 *   mat_elems  host, int64 [n_mats]
 *   master_w   host array of device pointers [n_experts * n_mats], index
 *              e*n_mats + m; master_g likewise (float*)
 *   spare_w    host array of device pointers [n_buffers * n_mats];
 *              spare_g likewise
 * Every pointer must be 16-byte aligned. The memory stays the caller's;
 * the context keeps the pointers (copied to the device) until the next
 * registration or ue_destroy. n_mats in 1..16. Any of master_g/spare_g
 * may be NULL (then ue_grad_reduce is refused), any of master_w/spare_w
 * may be NULL (then ue_weight_sync is refused). */
int ue_register_experts(ue_ctx *ctx, int32_t n_experts, int32_t n_mats,
                        const int64_t *mat_elems, void *const *master_w,
                        float *const *master_g, int32_t n_buffers,
                        void *const *spare_w, float *const *spare_g);

/* Replica weight sync ("Replica weight sync": replicas receive the master
 * weights before expert compute). Replica table as device CSR:
 *   rep_off  device, int32 [n_experts + 1]
 *   rep_buf  device, int32 [rep_off[n_experts]]; for expert e the entries
 *            rep_off[e] .. rep_off[e+1]-1: the first stands for the master
 *            and is ignored, the others are replica buffer indices
 * Every matrix of every replica becomes a bitwise copy of its master's.
 * The master is read once per tile and written to all its replicas.
 * n_experts must not exceed the registered count; buffer indices must be
 * < n_buffers (entries outside are skipped). Replica buffers that the table
 * names must not alias masters or each other.
 * A placement block's rep_off and rep_slot fields (ue_plan) form such a
 * table when buffer p is registered for physical slot p (n_buffers = P):
 * its first entry per expert is the native slot, the others are spare
 * slots. Buffers of native slots are never named as replicas, so they may
 * be the masters themselves. The plan then drives the sync (and, before
 * backward, the restore: the same call with the saved plan) and the
 * gradient reduction without leaving the device. */
int ue_weight_sync(ue_ctx *ctx, const int32_t *rep_off, const int32_t *rep_buf,
                   int32_t n_experts, void *stream);

/* Replica gradient reduction ("Replica gradient reduction": replica
 * gradients are summed into master gradients during backward). Same CSR as
 * ue_weight_sync. Per element, with the running sum in binary64 and no
 * reassociation: g = master; g += replica_1; g += replica_2; ...; then
 * master = g rounded once to binary32 (nearest even). The fp32 gradient is
 * thus within one rounding of the exact sum (unless the binary64 partial
 * sums themselves round, which takes terms some 2^29 apart in magnitude),
 * also where replicas cancel the master. Replica gradients are left
 * unchanged. */
int ue_grad_reduce(ue_ctx *ctx, const int32_t *rep_off, const int32_t *rep_buf,
                   int32_t n_experts, void *stream);

/* Token dispatch into physical-expert order on one device: out[pos, :] =
 * x[perm[pos] div k, :], done source-major through the inverse
 * permutation (every token row is read once and written to its k
 * positions).
 *   x        device, bf16 [T, H], 16-byte aligned rows (H % 8 == 0)
 *   inv_perm device, int32 [T*k] (from ue_reroute, one layer)
 *   out      device, bf16 [T*k, H]
 * Positions outside [0, T*k) are skipped. */
int ue_gather_rows(ue_ctx *ctx, const void *x, const int32_t *inv_perm,
                   int32_t T, int32_t k, int32_t H, void *out, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* UE_H */
