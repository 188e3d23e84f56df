// The rebalance without allocation: ue_rebalance_static.
//
// Some callers cannot allocate device memory where they rebalance (code
// under stream capture, tight serving loops, harnesses that forbid it).
// This entry point runs the same three kernels as ue_rebalance with the
// same results, but needs no context: its scratch (the load's per-tile
// table: group bases and per-tile offsets) lives in one file-scope device
// array of kStaticScratch bytes, which every device the library runs on
// holds until the process ends. Its device address is taken once per
// device, on the first call there, and only that address is handed to
// kernels.
//
// Calls of any shape share the array. Every word a call reads was written
// earlier in the same call (the count kernel writes each tile's row, the
// scan the rest), so nothing is cleared between calls. Calls that overlap
// in time on one device race on the array.
#include <cstdarg>
#include <cstdio>
#include <mutex>

#include "ue_internal.h"

namespace {

constexpr size_t kStaticScratch = UE_STATIC_SCRATCH_BYTES;
static_assert(kStaticScratch % 256 == 0, "whole 256-byte blocks");

// The scratch array. In host code `scratch` names a host-side stand-in, not
// device memory: kernels and copies get the address that
// hipGetSymbolAddress returns for the current device instead.
static __device__ __align__(256) unsigned char scratch[kStaticScratch];

constexpr int kMaxDevices = 64;
struct DeviceSlot {
    bool ready = false;
    int status = UE_OK;         // of the one-time set-up
    unsigned char *ptr = nullptr;
    ue::DeviceInfo info;
};
DeviceSlot g_devices[kMaxDevices];
std::mutex g_devices_mu;
thread_local char g_err[256];

int set_err(int code, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
int set_err(int code, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return code;
}

// One-time set-up of the current device: the scratch array's address on
// it and what the kernels need to know of it.
int device_slot(int dev, const DeviceSlot *&out) {
    if (dev < 0 || dev >= kMaxDevices)
        return set_err(UE_EUNSUPPORTED, "device %d beyond %d", dev, kMaxDevices);
    std::lock_guard<std::mutex> lock(g_devices_mu);
    DeviceSlot &d = g_devices[dev];
    if (!d.ready) {
        void *p = nullptr;
        hipError_t he = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (he == hipSuccess) he = ue::device_info(dev, d.info);
        d.status = he == hipSuccess ? UE_OK : UE_EHIP;
        d.ptr = static_cast<unsigned char *>(p);
        d.ready = true;
        if (he != hipSuccess) {
            out = &d;
            return set_err(UE_EHIP, "scratch set-up on device %d: %s", dev,
                           hipGetErrorString(he));
        }
    }
    out = &d;
    return d.status == UE_OK
               ? UE_OK
               : set_err(d.status, "scratch set-up on device %d failed", dev);
}

bool aligned4(const void *p) {
    return (reinterpret_cast<uintptr_t>(p) & 3u) == 0;
}

size_t up256(size_t v) { return (v + 255) / 256 * 256; }

// Scratch bytes of one call (the formula stated beside the entry point).
size_t scratch_need(const ue_config *cfg, int32_t L, int32_t T) {
    const int64_t A = static_cast<int64_t>(T) * cfg->topk;
    const ue::LoadShape sh = ue::load_shape(A, L);
    const size_t E = static_cast<size_t>(cfg->num_experts);
    // group bases, then the 16-bit per-tile rows
    return up256(sizeof(int32_t) * L * sh.groups * E) +
           up256(sizeof(uint16_t) * L * (sh.tiles + sh.groups) * E);
}

}  // namespace

namespace ue {
const char *static_last_error() { return g_err; }
}  // namespace ue

extern "C" {

int ue_rebalance_static(const ue_config *cfg, const int32_t *routing,
                        int32_t L, int32_t T, int32_t *counts,
                        int32_t *invalid, void *placement, int32_t *phys,
                        int32_t *rank_counts, int32_t *perm,
                        int32_t *inv_perm, int32_t *faults, void *stream) {
    g_err[0] = '\0';
    if (!cfg) return set_err(UE_EINVAL, "ue_rebalance_static: null config");
    int dev = 0;
    hipError_t he = hipGetDevice(&dev);
    if (he != hipSuccess)
        return set_err(UE_EHIP, "hipGetDevice: %s", hipGetErrorString(he));
    const DeviceSlot *d = nullptr;
    if (int rc = device_slot(dev, d)) return rc;
    ue_ctx c;
    if (int rc = ue::init_shape(*cfg, dev, d->info, c))
        return set_err(rc, "ue_rebalance_static: configuration not supported");
    if (L < 1 || L > cfg->max_layers)
        return set_err(UE_ESHAPE, "L=%d outside 1..%d", L, cfg->max_layers);
    if (T < 0 || T > cfg->max_tokens)
        return set_err(UE_ESHAPE, "T=%d outside 0..%d", T, cfg->max_tokens);
    if (!counts || !placement || !rank_counts ||
        (T > 0 && (!routing || !phys || !perm)))
        return set_err(UE_EINVAL, "ue_rebalance_static: null required pointer");
    if (!aligned4(routing) || !aligned4(counts) || !aligned4(invalid) ||
        !aligned4(placement) || !aligned4(phys) || !aligned4(rank_counts) ||
        !aligned4(perm) || !aligned4(inv_perm) || !aligned4(faults))
        return set_err(UE_EINVAL,
                       "ue_rebalance_static: arrays must be 4-byte aligned");
    const size_t need = scratch_need(cfg, L, T);
    if (need > kStaticScratch)
        return set_err(UE_ESHAPE,
                       "ue_rebalance_static: L=%d, T=%d needs %zu bytes of "
                       "scratch, above the %zu the library holds",
                       L, T, need, kStaticScratch);

    const int64_t A = static_cast<int64_t>(T) * c.k;
    const ue::LoadShape sh = ue::load_shape(A, L);
    const int64_t tiles = sh.tiles, groups = sh.groups;
    c.max_rr_tiles = static_cast<int>(tiles);
    c.load_group_rows = static_cast<int>(L * groups);
    const size_t E = static_cast<size_t>(c.E);
    unsigned char *b = d->ptr;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        unsigned char *p = b + off;
        off += up256(bytes);
        return p;
    };
    c.group_base = reinterpret_cast<int32_t *>(
        take(sizeof(int32_t) * L * groups * E));
    c.tile_off = reinterpret_cast<uint16_t *>(
        take(sizeof(uint16_t) * L * (tiles + groups) * E));
    c.scan_state = nullptr;        // the fused reroute does not scan
    c.rr_tick = nullptr;

    hipStream_t s = static_cast<hipStream_t>(stream);
    he = ue::launch_count(c, routing, L, A, s);
    if (he == hipSuccess)
        he = ue::launch_scan(c, L, A, counts, invalid,
                             static_cast<int32_t *>(placement), rank_counts,
                             faults, s);
    if (he == hipSuccess)
        he = ue::launch_reroute_after_load(
            c, routing, static_cast<const int32_t *>(placement), L, A, phys,
            rank_counts, perm, inv_perm, faults, s);
    if (he != hipSuccess)
        return set_err(UE_EHIP, "ue_rebalance_static launch: %s",
                       hipGetErrorString(he));
    return UE_OK;
}

}  // extern "C"
