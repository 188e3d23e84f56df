// C ABI of libue: context, argument validation and kernel launches.
//
// Every entry point validates all of its host-visible arguments before it
// launches or writes anything, so a refused call leaves every output as it
// was; the reason goes to ue_last_error(). Device-side conditions (an
// exhausted plan, ids out of range, assignments beyond a plan's capacity)
// are results, reported in the outputs, not errors.
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <new>

#include "ue_internal.h"

namespace {

int fail(ue_ctx *c, int code, const char *fmt, ...)
    __attribute__((format(printf, 3, 4)));

int fail(ue_ctx *c, int code, const char *fmt, ...) {
    if (c) {
        char buf[512];
        va_list ap;
        va_start(ap, fmt);
        vsnprintf(buf, sizeof(buf), fmt, ap);
        va_end(ap);
        c->err = buf;
    }
    return code;
}

int hip_fail(ue_ctx *c, hipError_t e, const char *what) {
    return fail(c, UE_EHIP, "%s: %s", what, hipGetErrorString(e));
}

int bits_for(int n) {   // smallest b with (1 << b) >= n
    int b = 0;
    while ((1 << b) < n) ++b;
    return b;
}

bool aligned(const void *p, size_t a) {
    return (reinterpret_cast<uintptr_t>(p) % a) == 0;
}

size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// Kernel timing: tbegin() before a call's first launch, tmark() after each.
void tbegin(ue_ctx *c, hipStream_t s) {
    if (!c->timing) return;
    c->n_ev = 0;
    if (hipEventRecord(c->ev[c->n_ev], s) == hipSuccess) ++c->n_ev;
}
void tmark(ue_ctx *c, hipStream_t s) {
    if (!c->timing || c->n_ev == 0 || c->n_ev >= ue_ctx::kMaxEvents) return;
    if (hipEventRecord(c->ev[c->n_ev], s) == hipSuccess) ++c->n_ev;
}

}  // namespace

namespace ue {

hipError_t device_info(int dev, DeviceInfo &out) {
    hipDeviceProp_t prop;
    hipError_t he = hipGetDeviceProperties(&prop, dev);
    if (he != hipSuccess) return he;
    out.num_cu = prop.multiProcessorCount;
    out.lds_cap = prop.sharedMemPerBlock;
    if (prop.sharedMemPerBlockOptin > out.lds_cap)
        out.lds_cap = prop.sharedMemPerBlockOptin;
    out.lds_per_cu = prop.maxSharedMemoryPerMultiProcessor;
    return hipSuccess;
}

int init_shape(const ue_config &cfg, int dev, const DeviceInfo &info,
               ue_ctx &c) {
    const int E = cfg.num_experts, R = cfg.num_ranks,
              S = cfg.spare_per_rank, k = cfg.topk;
    if (E < 1 || E > kMaxExperts || R < 1 || E % R != 0 || S < 0 ||
        S > kMaxSpare || k < 1 || k > E || cfg.max_tokens < 0 ||
        cfg.max_layers < 1 ||
        (cfg.plan_policy != UE_PLAN_LEAST_LOADED &&
         cfg.plan_policy != UE_PLAN_BEST_FIT &&
         cfg.plan_policy != UE_PLAN_BEST_FIT_COVER &&
         cfg.plan_policy != UE_PLAN_BEST_FIT_ASCENDING) ||
        (cfg.quota_mode != UE_QUOTA_FIXED &&
         cfg.quota_mode != UE_QUOTA_SEARCH))
        return UE_EUNSUPPORTED;
    const int N = E / R, NS = N + S;
    const int64_t P = static_cast<int64_t>(R) * NS;
    const int64_t A = static_cast<int64_t>(cfg.max_tokens) * k;
    if (P > kMaxSlots || A >= (int64_t(1) << 30)) return UE_EUNSUPPORTED;
    c.cfg = cfg;
    c.E = E;
    c.R = R;
    c.S = S;
    c.N = N;
    c.NS = NS;
    c.P = static_cast<int>(P);
    c.k = k;
    c.ebits = bits_for(E);
    c.rbits = bits_for(R);
    c.device = dev;
    c.num_cu = info.num_cu;

    // Placement block layout (int32 words).
    ue_placement_layout &l = c.lay;
    int w = 0;
    l.quota = w++;
    l.exhausted = w++;
    l.residual = w++;
    l.n_rep = w++;
    l.rep_off = w; w += E + 1;
    l.rep_slot = w; w += c.P;
    l.rep_cap = w; w += c.P;
    l.slot_expert = w; w += c.P;
    l.slot_cap = w; w += c.P;
    l.slot_off = w; w += c.P + 1;
    l.load_before = w; w += R;
    l.load_after = w; w += R;
    l.words = static_cast<int>(round_up(w, 64));   // 256-byte blocks

    c.reroute_lds = reroute_lds_bytes(E, R, c.P, k);
    c.count_lds = count_lds_bytes(E, info.lds_per_cu, info.lds_cap);
    c.stream_lds = quarter_cu_lds(info.lds_per_cu, info.lds_cap);
    // the quota search keeps each pass's chunks when they fit in LDS
    c.plan_per_wave = cfg.quota_mode == UE_QUOTA_SEARCH &&
                      plan_lds_bytes(E, R, S, c.P, true) + kPlanStaticLds <=
                          info.lds_cap;
    c.plan_lds = plan_lds_bytes(E, R, S, c.P, c.plan_per_wave);
    if (c.plan_lds + kPlanStaticLds > info.lds_cap ||
        c.reroute_lds + 256 > info.lds_cap ||
        load_lds_bytes(E) + 256 > info.lds_cap)
        return UE_EUNSUPPORTED;
    // kernels that need more than 64 KiB of dynamic LDS have their limit
    // raised to the need (it only ever rises)
    if ((c.plan_lds > 65536 && plan_prepare(c.plan_lds) != hipSuccess) ||
        (c.reroute_lds > 65536 && reroute_prepare(c.reroute_lds) != hipSuccess))
        return UE_EUNSUPPORTED;
    return UE_OK;
}

}  // namespace ue

extern "C" {

const char *ue_status_name(int status) {
    switch (status) {
        case UE_OK: return "UE_OK";
        case UE_EINVAL: return "UE_EINVAL";
        case UE_ESHAPE: return "UE_ESHAPE";
        case UE_ENOMEM: return "UE_ENOMEM";
        case UE_EHIP: return "UE_EHIP";
        case UE_EUNSUPPORTED: return "UE_EUNSUPPORTED";
        case UE_ESTATE: return "UE_ESTATE";
        default: return "UE_UNKNOWN";
    }
}

const char *ue_last_error(const ue_ctx *ctx) {
    // no context: the calling thread's last ue_rebalance_static error
    return ctx ? ctx->err.c_str() : ue::static_last_error();
}

int ue_create(const ue_config *cfg, ue_ctx **out) {
    if (!cfg || !out) return UE_EINVAL;
    ue_ctx *c = new (std::nothrow) ue_ctx();
    if (!c) return UE_ENOMEM;
    int dev = 0;
    ue::DeviceInfo info;
    hipError_t he = hipGetDevice(&dev);
    if (he == hipSuccess) he = ue::device_info(dev, info);
    if (he != hipSuccess) {
        delete c;
        return UE_EHIP;
    }
    if (int rc = ue::init_shape(*cfg, dev, info, *c)) {
        delete c;
        return rc;
    }
    const int E = c->E, k = c->k;
    const int64_t A = static_cast<int64_t>(cfg->max_tokens) * k;
    const int Lmax = cfg->max_layers;
    int64_t rr_tiles = (A + ue::kRerouteTile - 1) / ue::kRerouteTile;
    if (rr_tiles < 1) rr_tiles = 1;
    const int64_t ld_rows = ue::load_group_rows_cap(A, Lmax);
    c->max_rr_tiles = static_cast<int>(rr_tiles);
    c->load_group_rows = static_cast<int>(ld_rows);

    // Workspace carve-up, each piece 256-byte aligned.
    size_t off = 0;
    auto take = [&](size_t bytes) {
        size_t o = off;
        off = round_up(off + bytes, 256);
        return o;
    };
    // the load's prefixes: a base row per group of tiles and a 16-bit row
    // per tile plus one per group (row t + g for tile t of group g, and row
    // t + g + 1 after the group's last tile t), so tiles + groups per layer
    const size_t o_gbase = take(sizeof(int32_t) * ld_rows * E);
    const size_t o_toff =
        take(sizeof(uint16_t) * (Lmax * rr_tiles + ld_rows) * E);
    const size_t o_state = take(sizeof(uint64_t) * Lmax * rr_tiles * E);
    const size_t o_tick = take(sizeof(uint64_t) * Lmax);
    // the spread quota search's exchange (only with the search and the
    // chunks of every pass kept)
    const bool spread = c->plan_per_wave && c->R > 64;
    const int xslots = spread ? 4 * c->num_cu : 0;
    const size_t o_xrec =
        take(sizeof(int32_t) * 3 * static_cast<size_t>(xslots) * c->R * c->S);
    const size_t o_xflag = take(sizeof(int32_t) * xslots);
    const size_t o_xcnt = take(spread ? sizeof(uint32_t) * Lmax : 0);
    c->ws_bytes = off;
    he = hipMalloc(&c->ws, c->ws_bytes);
    if (he != hipSuccess) {
        delete c;
        return UE_ENOMEM;
    }
    he = hipMemset(c->ws, 0, c->ws_bytes);
    if (he == hipSuccess) he = hipDeviceSynchronize();
    if (he != hipSuccess) {
        (void)hipFree(c->ws);
        delete c;
        return UE_EHIP;
    }
    char *b = static_cast<char *>(c->ws);
    c->group_base = reinterpret_cast<int32_t *>(b + o_gbase);
    c->tile_off = reinterpret_cast<uint16_t *>(b + o_toff);
    c->scan_state = reinterpret_cast<uint64_t *>(b + o_state);
    c->rr_tick = reinterpret_cast<uint64_t *>(b + o_tick);
    if (spread) {
        c->plan_xrec = reinterpret_cast<int32_t *>(b + o_xrec);
        c->plan_xflag = reinterpret_cast<int32_t *>(b + o_xflag);
        c->plan_xcnt = reinterpret_cast<uint32_t *>(b + o_xcnt);
        c->plan_xslots = xslots;
    }
    *out = c;
    return UE_OK;
}

void ue_destroy(ue_ctx *ctx) {
    if (!ctx) return;
    (void)hipDeviceSynchronize();
    if (ctx->ws) (void)hipFree(ctx->ws);
    if (ctx->reg_tables) (void)hipFree(ctx->reg_tables);
    for (auto &e : ctx->ev)
        if (e) (void)hipEventDestroy(e);
    delete ctx;
}

int ue_get_placement_layout(const ue_ctx *ctx, ue_placement_layout *out) {
    if (!ctx || !out) return UE_EINVAL;
    *out = ctx->lay;
    return UE_OK;
}

size_t ue_placement_bytes(const ue_ctx *ctx) {
    return ctx ? static_cast<size_t>(ctx->lay.words) * sizeof(int32_t) : 0;
}

int ue_set_timing(ue_ctx *ctx, int enable) {
    if (!ctx) return UE_EINVAL;
    ctx->err.clear();
    if (enable && !ctx->ev[0]) {
        for (auto &e : ctx->ev) {
            hipError_t he = hipEventCreate(&e);
            if (he != hipSuccess) return hip_fail(ctx, he, "hipEventCreate");
        }
    }
    ctx->timing = enable != 0;
    ctx->n_ev = 0;
    return UE_OK;
}

int ue_set_wait_limit(ue_ctx *ctx, uint32_t polls) {
    if (!ctx) return UE_EINVAL;
    ctx->err.clear();
    ctx->wait_limit = polls;
    return UE_OK;
}

int ue_kernel_times(ue_ctx *ctx, float *ms, int32_t max_n, int32_t *n) {
    if (!ctx || !ms || !n || max_n < 0) return UE_EINVAL;
    ctx->err.clear();
    if (!ctx->timing || ctx->n_ev < 2)
        return fail(ctx, UE_ESTATE, "no timed call");
    hipError_t he = hipEventSynchronize(ctx->ev[ctx->n_ev - 1]);
    if (he != hipSuccess) return hip_fail(ctx, he, "hipEventSynchronize");
    const int k = ctx->n_ev - 1;
    for (int i = 0; i < k && i < max_n; ++i) {
        float t = 0.f;
        he = hipEventElapsedTime(&t, ctx->ev[i], ctx->ev[i + 1]);
        if (he != hipSuccess) return hip_fail(ctx, he, "hipEventElapsedTime");
        ms[i] = t;
    }
    *n = k;
    return UE_OK;
}

static int check_LT(ue_ctx *c, int32_t L, int32_t T) {
    if (L < 1 || L > c->cfg.max_layers)
        return fail(c, UE_ESHAPE, "L=%d outside 1..%d", L, c->cfg.max_layers);
    if (T < 0 || T > c->cfg.max_tokens)
        return fail(c, UE_ESHAPE, "T=%d outside 0..%d", T, c->cfg.max_tokens);
    return UE_OK;
}

int ue_load(ue_ctx *ctx, const int32_t *routing, int32_t L, int32_t T,
            int32_t *counts, int32_t *invalid, void *stream) {
    if (!ctx) return UE_EINVAL;
    ctx->err.clear();
    if (int rc = check_LT(ctx, L, T)) return rc;
    if ((!routing && T > 0) || !counts)
        return fail(ctx, UE_EINVAL, "ue_load: null routing or counts");
    if (!aligned(routing, 4) || !aligned(counts, 4) || !aligned(invalid, 4))
        return fail(ctx, UE_EINVAL, "ue_load: int32 arrays must be 4-byte aligned");
    const int64_t A = static_cast<int64_t>(T) * ctx->k;
    hipStream_t s = static_cast<hipStream_t>(stream);
    tbegin(ctx, s);
    hipError_t he = ue::launch_count(*ctx, routing, L, A, s);
    if (he != hipSuccess) return hip_fail(ctx, he, "k_count launch");
    tmark(ctx, s);
    he = ue::launch_scan(*ctx, L, A, counts, invalid, nullptr, nullptr,
                         nullptr, s);
    tmark(ctx, s);
    return he == hipSuccess ? UE_OK : hip_fail(ctx, he, "k_plan (scan) launch");
}

int ue_plan(ue_ctx *ctx, const int32_t *counts, int32_t L, void *placement,
            void *stream) {
    if (!ctx) return UE_EINVAL;
    ctx->err.clear();
    if (L < 1 || L > ctx->cfg.max_layers)
        return fail(ctx, UE_ESHAPE, "L=%d outside 1..%d", L, ctx->cfg.max_layers);
    if (!counts || !placement)
        return fail(ctx, UE_EINVAL, "ue_plan: null counts or placement");
    if (!aligned(counts, 4) || !aligned(placement, 4))
        return fail(ctx, UE_EINVAL, "ue_plan: arrays must be 4-byte aligned");
    hipStream_t s = static_cast<hipStream_t>(stream);
    tbegin(ctx, s);
    hipError_t he = ue::launch_plan(*ctx, counts, L,
                                    static_cast<int32_t *>(placement), s);
    tmark(ctx, s);
    return he == hipSuccess ? UE_OK : hip_fail(ctx, he, "k_plan launch");
}

int ue_reroute(ue_ctx *ctx, const int32_t *routing, const void *placement,
               int32_t L, int32_t T, int32_t *phys, int32_t *rank_counts,
               int32_t *perm, int32_t *inv_perm, int32_t *faults,
               void *stream) {
    if (!ctx) return UE_EINVAL;
    ctx->err.clear();
    if (int rc = check_LT(ctx, L, T)) return rc;
    if (!placement || !rank_counts || (T > 0 && (!routing || !phys || !perm)))
        return fail(ctx, UE_EINVAL, "ue_reroute: null required pointer");
    if (!aligned(routing, 4) || !aligned(placement, 4) || !aligned(phys, 4) ||
        !aligned(rank_counts, 4) || !aligned(perm, 4) ||
        !aligned(inv_perm, 4) || !aligned(faults, 4))
        return fail(ctx, UE_EINVAL, "ue_reroute: arrays must be 4-byte aligned");
    const int64_t A = static_cast<int64_t>(T) * ctx->k;
    hipStream_t s = static_cast<hipStream_t>(stream);
    tbegin(ctx, s);
    hipError_t he = ue::launch_reroute(
        *ctx, routing, static_cast<const int32_t *>(placement), L, A, phys,
        rank_counts, perm, inv_perm, faults, s);
    tmark(ctx, s);
    return he == hipSuccess ? UE_OK : hip_fail(ctx, he, "k_reroute launch");
}

int ue_rebalance(ue_ctx *ctx, const int32_t *routing, int32_t L, int32_t T,
                 int32_t *counts, int32_t *invalid, void *placement,
                 int32_t *phys, int32_t *rank_counts, int32_t *perm,
                 int32_t *inv_perm, int32_t *faults, void *stream) {
    if (!ctx) return UE_EINVAL;
    ctx->err.clear();
    if (int rc = check_LT(ctx, L, T)) return rc;
    if (!counts || !placement || !rank_counts ||
        (T > 0 && (!routing || !phys || !perm)))
        return fail(ctx, UE_EINVAL, "ue_rebalance: null required pointer");
    if (!aligned(routing, 4) || !aligned(counts, 4) || !aligned(invalid, 4) ||
        !aligned(placement, 4) || !aligned(phys, 4) ||
        !aligned(rank_counts, 4) || !aligned(perm, 4) ||
        !aligned(inv_perm, 4) || !aligned(faults, 4))
        return fail(ctx, UE_EINVAL,
                    "ue_rebalance: arrays must be 4-byte aligned");
    const int64_t A = static_cast<int64_t>(T) * ctx->k;
    hipStream_t s = static_cast<hipStream_t>(stream);
    tbegin(ctx, s);
    hipError_t he = ue::launch_count(*ctx, routing, L, A, s);
    if (he != hipSuccess) return hip_fail(ctx, he, "k_count launch");
    tmark(ctx, s);
    he = ue::launch_scan(*ctx, L, A, counts, invalid,
                         static_cast<int32_t *>(placement), rank_counts,
                         faults, s);
    if (he != hipSuccess) return hip_fail(ctx, he, "k_plan launch");
    tmark(ctx, s);
    he = ue::launch_reroute_after_load(
        *ctx, routing, static_cast<const int32_t *>(placement), L, A, phys,
        rank_counts, perm, inv_perm, faults, s);
    tmark(ctx, s);
    return he == hipSuccess ? UE_OK : hip_fail(ctx, he, "k_reroute launch");
}

int ue_stale_loads(ue_ctx *ctx, const void *placement, const int32_t *counts,
                   int32_t L, int32_t *rank_loads, void *stream) {
    if (!ctx) return UE_EINVAL;
    ctx->err.clear();
    if (L < 1 || L > ctx->cfg.max_layers)
        return fail(ctx, UE_ESHAPE, "L=%d outside 1..%d", L, ctx->cfg.max_layers);
    if (!placement || !counts || !rank_loads)
        return fail(ctx, UE_EINVAL, "ue_stale_loads: null pointer");
    if (!aligned(placement, 4) || !aligned(counts, 4) || !aligned(rank_loads, 4))
        return fail(ctx, UE_EINVAL,
                    "ue_stale_loads: arrays must be 4-byte aligned");
    hipStream_t s = static_cast<hipStream_t>(stream);
    tbegin(ctx, s);
    hipError_t he = ue::launch_stale(*ctx, static_cast<const int32_t *>(placement),
                                     counts, L, rank_loads, s);
    tmark(ctx, s);
    return he == hipSuccess ? UE_OK : hip_fail(ctx, he, "k_stale launch");
}

int ue_register_experts(ue_ctx *ctx, int32_t n_experts, int32_t n_mats,
                        const int64_t *mat_elems, void *const *master_w,
                        float *const *master_g, int32_t n_buffers,
                        void *const *spare_w, float *const *spare_g) {
    if (!ctx) return UE_EINVAL;
    ctx->err.clear();
    if (n_experts < 1 || n_mats < 1 || n_mats > ue::kMaxMats ||
        n_buffers < 0 || !mat_elems)
        return fail(ctx, UE_ESHAPE, "ue_register_experts: bad counts");
    const bool has_w = master_w && (spare_w || n_buffers == 0);
    const bool has_g = master_g && (spare_g || n_buffers == 0);
    if (!has_w && !has_g)
        return fail(ctx, UE_EINVAL, "ue_register_experts: no weights or gradients");
    for (int m = 0; m < n_mats; ++m)
        if (mat_elems[m] < 0)
            return fail(ctx, UE_EINVAL, "ue_register_experts: negative size");
    const int64_t nm = static_cast<int64_t>(n_experts) * n_mats;
    const int64_t nb = static_cast<int64_t>(n_buffers) * n_mats;
    for (int64_t i = 0; i < nm; ++i) {
        if (has_w && (!master_w[i] || !aligned(master_w[i], 16)))
            return fail(ctx, UE_EINVAL, "master weight %lld null or unaligned",
                        static_cast<long long>(i));
        if (has_g && (!master_g[i] || !aligned(master_g[i], 16)))
            return fail(ctx, UE_EINVAL, "master grad %lld null or unaligned",
                        static_cast<long long>(i));
    }
    for (int64_t i = 0; i < nb; ++i) {
        if (has_w && (!spare_w[i] || !aligned(spare_w[i], 16)))
            return fail(ctx, UE_EINVAL, "replica weight %lld null or unaligned",
                        static_cast<long long>(i));
        if (has_g && (!spare_g[i] || !aligned(spare_g[i], 16)))
            return fail(ctx, UE_EINVAL, "replica grad %lld null or unaligned",
                        static_cast<long long>(i));
    }
    const size_t bytes = sizeof(void *) * static_cast<size_t>(2 * nm + 2 * nb + 4);
    void *tables = nullptr;
    hipError_t he = hipMalloc(&tables, bytes);
    if (he != hipSuccess) return fail(ctx, UE_ENOMEM, "pointer tables");
    void **host = new (std::nothrow) void *[2 * nm + 2 * nb + 4];
    if (!host) {
        (void)hipFree(tables);
        return fail(ctx, UE_ENOMEM, "pointer tables (host)");
    }
    for (int64_t i = 0; i < nm; ++i) {
        host[i] = has_w ? master_w[i] : nullptr;
        host[nm + i] = has_g ? static_cast<void *>(master_g[i]) : nullptr;
    }
    for (int64_t i = 0; i < nb; ++i) {
        host[2 * nm + i] = has_w ? spare_w[i] : nullptr;
        host[2 * nm + nb + i] = has_g ? static_cast<void *>(spare_g[i]) : nullptr;
    }
    he = hipMemcpy(tables, host, sizeof(void *) * (2 * nm + 2 * nb),
                   hipMemcpyHostToDevice);
    delete[] host;
    if (he != hipSuccess) {
        (void)hipFree(tables);
        return hip_fail(ctx, he, "pointer table upload");
    }
    if (ctx->reg_tables) {
        (void)hipDeviceSynchronize();
        (void)hipFree(ctx->reg_tables);
    }
    ctx->reg_tables = tables;
    void **t = static_cast<void **>(tables);
    ctx->d_master_w = t;
    ctx->d_master_g = reinterpret_cast<float **>(t + nm);
    ctx->d_spare_w = t + 2 * nm;
    ctx->d_spare_g = reinterpret_cast<float **>(t + 2 * nm + nb);
    ctx->reg_experts = n_experts;
    ctx->reg_mats = n_mats;
    ctx->reg_buffers = n_buffers;
    for (int m = 0; m < n_mats; ++m) ctx->mat_elems[m] = mat_elems[m];
    ctx->has_w = has_w;
    ctx->has_g = has_g;
    return UE_OK;
}

static int check_stream_call(ue_ctx *ctx, const int32_t *rep_off,
                             const int32_t *rep_buf, int32_t n_experts,
                             bool weights) {
    if (ctx->reg_mats == 0)
        return fail(ctx, UE_ESTATE, "no experts registered");
    if (weights ? !ctx->has_w : !ctx->has_g)
        return fail(ctx, UE_ESTATE, "%s not registered",
                    weights ? "weights" : "gradients");
    if (n_experts < 0 || n_experts > ctx->reg_experts)
        return fail(ctx, UE_ESHAPE, "n_experts=%d outside 0..%d", n_experts,
                    ctx->reg_experts);
    if (n_experts > 0 && (!rep_off || !rep_buf))
        return fail(ctx, UE_EINVAL, "null replica table");
    if (!aligned(rep_off, 4) || !aligned(rep_buf, 4))
        return fail(ctx, UE_EINVAL, "replica table must be 4-byte aligned");
    return UE_OK;
}

int ue_weight_sync(ue_ctx *ctx, const int32_t *rep_off, const int32_t *rep_buf,
                   int32_t n_experts, void *stream) {
    if (!ctx) return UE_EINVAL;
    ctx->err.clear();
    if (int rc = check_stream_call(ctx, rep_off, rep_buf, n_experts, true))
        return rc;
    if (n_experts == 0) return UE_OK;
    hipStream_t s = static_cast<hipStream_t>(stream);
    tbegin(ctx, s);
    hipError_t he = ue::launch_weight_sync(*ctx, rep_off, rep_buf, n_experts, s);
    tmark(ctx, s);
    return he == hipSuccess ? UE_OK : hip_fail(ctx, he, "k_weight_sync launch");
}

int ue_grad_reduce(ue_ctx *ctx, const int32_t *rep_off, const int32_t *rep_buf,
                   int32_t n_experts, void *stream) {
    if (!ctx) return UE_EINVAL;
    ctx->err.clear();
    if (int rc = check_stream_call(ctx, rep_off, rep_buf, n_experts, false))
        return rc;
    if (n_experts == 0) return UE_OK;
    hipStream_t s = static_cast<hipStream_t>(stream);
    tbegin(ctx, s);
    hipError_t he = ue::launch_grad_reduce(*ctx, rep_off, rep_buf, n_experts, s);
    tmark(ctx, s);
    return he == hipSuccess ? UE_OK : hip_fail(ctx, he, "k_grad_reduce launch");
}

int ue_gather_rows(ue_ctx *ctx, const void *x, const int32_t *inv_perm,
                   int32_t T, int32_t k, int32_t H, void *out, void *stream) {
    if (!ctx) return UE_EINVAL;
    ctx->err.clear();
    if (T < 0 || k < 1 || H < 0 || H % 8 != 0)
        return fail(ctx, UE_ESHAPE, "ue_gather_rows: T=%d k=%d H=%d", T, k, H);
    if (static_cast<int64_t>(T) * k >= (int64_t(1) << 31))
        return fail(ctx, UE_ESHAPE, "ue_gather_rows: T*k too large");
    if (T > 0 && (!x || !inv_perm || !out))
        return fail(ctx, UE_EINVAL, "ue_gather_rows: null pointer");
    if (!aligned(x, 16) || !aligned(out, 16) || !aligned(inv_perm, 4))
        return fail(ctx, UE_EINVAL, "ue_gather_rows: x/out need 16-byte alignment");
    if (H == 0) return UE_OK;
    hipStream_t s = static_cast<hipStream_t>(stream);
    tbegin(ctx, s);
    hipError_t he = ue::launch_gather_rows(*ctx, x, inv_perm, T, k, H, out, s);
    tmark(ctx, s);
    return he == hipSuccess ? UE_OK : hip_fail(ctx, he, "k_gather_rows launch");
}

}  // extern "C"
