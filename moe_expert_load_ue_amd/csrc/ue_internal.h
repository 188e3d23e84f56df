// Internal declarations of libue: the context, workspace layout, kernel
// launchers and small wave-level helpers for gfx950 (wave64).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>
#include <string>

#include "../../include/ue.h"

namespace ue {

constexpr int kMaxExperts = 1024;
constexpr int kMaxSlots = 4096;      // P = R * (N + S)
constexpr int kMaxSpare = 64;
constexpr int kMaxMats = 16;
constexpr int kBlock = 256;          // threads per workgroup (4 waves)
constexpr int kWaves = kBlock / 64;

// Routing tiles: kRerouteItems assignments per thread, processed as rounds
// of 64 consecutive assignments per wave. The load kernel uses the same
// tiles, so the per-tile prefixes it publishes serve the fused reroute.
constexpr int kRerouteItems = 8;
constexpr int kRerouteTile = kBlock * kRerouteItems;
constexpr int kLoadItems = kRerouteItems;
constexpr int kLoadTile = kRerouteTile;
constexpr int kLoadGroup = 16384 / kLoadTile;   // tiles per load workgroup

}  // namespace ue

struct ue_ctx {
    ue_config cfg{};
    int E = 0, R = 0, S = 0, N = 0, NS = 0, P = 0, k = 0;
    int ebits = 0;          // bits to hold an expert id (ceil(log2 E))
    int rbits = 0;          // bits to hold a rank id (ceil(log2 R))
    int device = 0;
    int num_cu = 0;
    ue_placement_layout lay{};
    int max_rr_tiles = 0;   // reroute tiles of the largest layer

    // One device allocation holds the whole workspace: the per-tile table
    // the load fills and the fused reroute reads, and the standalone
    // reroute's lookback words with, per layer, a tile ticket and a call
    // epoch. Tickets return to zero at the end of every launch and epochs
    // only grow, so nothing is cleared between calls.
    void *ws = nullptr;
    size_t ws_bytes = 0;
    int load_group_rows = 0;       // group rows of the load's tables, all layers
    // the load's per-tile prefixes, in two parts: per group of tiles, the
    // count of each expert in all earlier groups, and per tile the count
    // in the group's earlier tiles (16 bits; each group also has a row
    // after its last tile: the group's own counts). Tile t of group g has
    // row t + g. The count kernel first writes each tile's own counts
    // there; the scan rewrites them in place.
    // the load's tables of one call (LoadShape): per layer, `groups` base
    // rows and `tiles + groups` 16-bit rows, layers one after another
    int32_t *group_base = nullptr; // [load_group_rows][E]
    uint16_t *tile_off = nullptr;  // [max_layers * max_rr_tiles + load_group_rows][E]
    uint64_t *scan_state = nullptr;// [max_layers][max_rr_tiles][E]
    uint64_t *rr_tick = nullptr;   // [max_layers] {epoch:32 | ticket:32}
    // polls of one cross-workgroup wait before it gives up
    uint32_t wait_limit = 1u << 22;

    size_t plan_lds = 0;
    bool plan_per_wave = false;   // planner keeps every pass's chunks
    size_t count_lds = 0;         // LDS the count asks for (see k_load)
    size_t stream_lds = 0;        // LDS the sync and reduction ask for (k_stream)
    // the quota search spread over several workgroups per layer: per pass
    // slot (4 per workgroup, at most 4 * num_cu) its chunks and their
    // number, and per layer a count of workgroups done (zero between
    // calls); null when the search is not spread (then one per layer)
    int32_t *plan_xrec = nullptr;    // [plan_xslots][3][R*S]
    int32_t *plan_xflag = nullptr;   // [plan_xslots]
    uint32_t *plan_xcnt = nullptr;   // [max_layers]
    int plan_xslots = 0;
    size_t reroute_lds = 0;

    // Registered expert state (device pointer tables).
    int reg_experts = 0, reg_mats = 0, reg_buffers = 0;
    int64_t mat_elems[ue::kMaxMats] = {};
    bool has_w = false, has_g = false;
    void *reg_tables = nullptr;    // device: master_w, master_g, spare_w, spare_g
    void **d_master_w = nullptr;
    float **d_master_g = nullptr;
    void **d_spare_w = nullptr;
    float **d_spare_g = nullptr;

    // Kernel timing (off unless ue_set_timing enabled it).
    static constexpr int kMaxEvents = 8;
    bool timing = false;
    hipEvent_t ev[kMaxEvents] = {};
    int n_ev = 0;

    std::string err;
};

namespace ue {

// Launchers (each returns a hipError_t from the launch).
// The load is two launches: launch_count writes every tile's counts into
// the per-tile table, launch_scan finishes it (group bases, in-group
// offsets, counts, invalid) and, with a placement, plans in the same
// launch and writes the rank counts and faults of the reroute that
// follows (launch_reroute_after_load then leaves them alone).
hipError_t launch_count(const ue_ctx &c, const int32_t *routing, int L,
                        int64_t A, hipStream_t s);
hipError_t launch_scan(const ue_ctx &c, int L, int64_t A, int32_t *counts,
                       int32_t *invalid, int32_t *placement,
                       int32_t *rank_counts, int32_t *faults, hipStream_t s);
hipError_t launch_plan(const ue_ctx &c, const int32_t *counts, int L,
                       int32_t *placement, hipStream_t s);
hipError_t launch_reroute(const ue_ctx &c, const int32_t *routing,
                          const int32_t *placement, int L, int64_t A,
                          int32_t *phys, int32_t *rank_counts, int32_t *perm,
                          int32_t *inv_perm, int32_t *faults, hipStream_t s);
// Reroute that takes each tile's expert prefix from the rows the load's
// scan just wrote instead of its own lookback (the routing must be the one
// the immediately preceding launch_count / launch_scan counted).
hipError_t launch_reroute_after_load(const ue_ctx &c, const int32_t *routing,
                                     const int32_t *placement, int L,
                                     int64_t A, int32_t *phys,
                                     int32_t *rank_counts, int32_t *perm,
                                     int32_t *inv_perm, int32_t *faults,
                                     hipStream_t s);
hipError_t launch_weight_sync(const ue_ctx &c, const int32_t *rep_off,
                              const int32_t *rep_buf, int n_experts,
                              hipStream_t s);
hipError_t launch_grad_reduce(const ue_ctx &c, const int32_t *rep_off,
                              const int32_t *rep_buf, int n_experts,
                              hipStream_t s);
hipError_t launch_stale(const ue_ctx &c, const int32_t *placement,
                        const int32_t *counts, int L, int32_t *rank_loads,
                        hipStream_t s);
hipError_t launch_gather_rows(const ue_ctx &c, const void *x,
                              const int32_t *inv_perm, int T, int k, int H,
                              void *out, hipStream_t s);

// What the kernels need to know of a device.
struct DeviceInfo {
    int num_cu = 0;
    size_t lds_cap = 0;      // dynamic LDS one workgroup may have
    size_t lds_per_cu = 0;   // LDS of one CU
};
hipError_t device_info(int dev, DeviceInfo &out);
// Validates a configuration and fills the shape fields of `c` (sizes,
// placement layout, LDS needs) for device `dev`, raising kernels' LDS
// limits where needed; allocates nothing. UE_OK or UE_EUNSUPPORTED.
int init_shape(const ue_config &cfg, int dev, const DeviceInfo &info,
               ue_ctx &c);

// Error text of the calling thread's last ue_rebalance_static call.
const char *static_last_error();
// Static LDS of the planner kernel (dynamic LDS comes on top of it).
constexpr size_t kPlanStaticLds = 5120;

size_t load_lds_bytes(int E);
// A quarter of a CU's LDS when a launch may ask for it without raising a
// kernel's limit (at most 64 KiB and within the per-workgroup cap), else
// 0: asked for by a streaming launch, it holds at most four of its
// workgroups on a CU
size_t quarter_cu_lds(size_t lds_per_cu, size_t lds_cap);
// LDS the count kernel asks for: its need, or the quarter share when that
// is more
size_t count_lds_bytes(int E, size_t lds_per_cu, size_t lds_cap);
// The load's split of one call over L layers of A assignments: tiles of
// kLoadTile assignments, groups of `group` consecutive tiles (one counting
// workgroup each). The count, the scan and the fused reroute all take it
// from here. (Fewer tiles per group when layers are few gives the count
// more workgroups, but the planner's scan then reads and writes more
// group rows in its one workgroup per layer, which costs more than the
// count gains.)
struct LoadShape {
    int tiles, group, groups;
};
LoadShape load_shape(int64_t A, int L);
// Group rows (over all layers) that any call of up to L layers of up to A
// assignments needs.
int64_t load_group_rows_cap(int64_t A, int L);
// per_wave: one chunk-record region per wave (the quota search keeps each
// pass's chunks, so the chosen one needs no second pass).
size_t plan_lds_bytes(int E, int R, int S, int P, bool per_wave);
size_t reroute_lds_bytes(int E, int R, int P, int k);
// Words per expert bitmap of the reroute's ranking (0: ranks by matching).
int reroute_bitmap_words(int E, int k);
// Raise the dynamic LDS limit of a kernel that needs more than 64 KiB.
hipError_t plan_prepare(size_t lds_bytes);
hipError_t reroute_prepare(size_t lds_bytes);
// Reroute workgroups that can be resident on one CU with this much LDS.

// ---------------------------------------------------------------------
// wave64 helpers

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

// Number of set bits of `mask` below this lane.
// Workgroups are handed to the 8 XCDs round robin in launch order, and
// each XCD has its own L2. Work item xcd_order(i, n) of n gives XCD i mod 8
// one contiguous run of items, so neighbouring items (whose outputs share
// cache lines) meet in the same L2. A bijection of [0, n) for any n.
constexpr int kXcds = 8;
__device__ __forceinline__ int xcd_order(int i, int n) {
    const int x = i % kXcds, k = i / kXcds;
    const int q = n / kXcds, r = n % kXcds;
    // XCD x receives q + (x < r) items; those of XCDs below x come first
    return x * q + (x < r ? x : r) + k;
}

__device__ __forceinline__ uint32_t mask_rank(uint64_t mask) {
    return __builtin_amdgcn_mbcnt_hi(
        static_cast<uint32_t>(mask >> 32),
        __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(mask), 0u));
}

// Minimum of v over the 64 lanes, returned wave-uniform. Row reduction with
// DPP (quad swaps, half-row and row mirrors), then the four row minima are
// read from lanes 0, 16, 32, 48.
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
    auto dpp_min = [](uint32_t x, int ctrl) -> uint32_t {
        uint32_t y;
        switch (ctrl) {
            case 0: y = __builtin_amdgcn_update_dpp(x, x, 0xB1, 0xF, 0xF, false); break;
            case 1: y = __builtin_amdgcn_update_dpp(x, x, 0x4E, 0xF, 0xF, false); break;
            case 2: y = __builtin_amdgcn_update_dpp(x, x, 0x141, 0xF, 0xF, false); break;
            default: y = __builtin_amdgcn_update_dpp(x, x, 0x140, 0xF, 0xF, false); break;
        }
        return x < y ? x : y;
    };
    v = dpp_min(v, 0);
    v = dpp_min(v, 1);
    v = dpp_min(v, 2);
    v = dpp_min(v, 3);
    uint32_t a = __builtin_amdgcn_readlane(v, 0);
    uint32_t b = __builtin_amdgcn_readlane(v, 16);
    uint32_t c = __builtin_amdgcn_readlane(v, 32);
    uint32_t d = __builtin_amdgcn_readlane(v, 48);
    a = a < b ? a : b;
    c = c < d ? c : d;
    return a < c ? a : c;
}

// Inclusive sum over lanes below and including this one, by DPP lane
// moves (no LDS round trip): shifts by 1, 2, 4 and 8 within each row of 16
// lanes (a lane with no source adds 0), then the last lane of row 0 into
// rows 1 and 3 and the last lane of row 1 into rows 2 and 3.
__device__ __forceinline__ int wave_inclusive_sum(int x) {
    x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, false);  // row_shr:1
    x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, false);  // row_shr:2
    x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, false);  // row_shr:4
    x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, false);  // row_shr:8
    x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xA, 0xF, false);  // row_bcast:15
    x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xC, 0xF, false);  // row_bcast:31
    return x;
}

// Exclusive prefix sum of one value per thread over a kBlock-thread
// workgroup. `wsum` is kWaves ints of LDS. Returns the prefix; the block
// total goes to `total`. Contains barriers: every thread must call it.
__device__ __forceinline__ int block_exclusive_sum(int v, int *wsum,
                                                   int &total) {
    const int w = threadIdx.x >> 6;
    int x = wave_inclusive_sum(v);
    if (lane_id() == 63) wsum[w] = x;
    __syncthreads();
    int before = 0;
    total = 0;
#pragma unroll
    for (int i = 0; i < kWaves; ++i) {
        int s = wsum[i];
        before += (i < w) ? s : 0;
        total += s;
    }
    __syncthreads();
    return before + x - v;
}

// Whether `pred` holds on any thread of the workgroup; `wany` holds one
// int per wave. (The same as __syncthreads_or, without the 256 bytes of
// static LDS that the library's version claims, which can cost a
// workgroup per CU.)
__device__ __forceinline__ bool block_any(bool pred, int *wany) {
    const int w = threadIdx.x >> 6;
    const bool mine = __ballot(pred) != 0;
    if (lane_id() == 0) wany[w] = mine;
    __syncthreads();
    int any = 0;
#pragma unroll
    for (int i = 0; i < kWaves; ++i) any |= wany[i];
    __syncthreads();
    return any != 0;
}

// Set of lanes holding the same value as this lane, among lanes where
// `valid`: one ballot per bit of the value (values < 2^bits).
__device__ __forceinline__ uint64_t match_peers(int v, bool valid, int bits) {
    uint64_t peers = __ballot(valid);
    for (int b = 0; b < bits; ++b) {
        const bool bit = (v >> b) & 1;
        const uint64_t ones = __ballot(bit);
        peers &= bit ? ones : ~ones;
    }
    return peers;
}

__device__ __forceinline__ uint64_t atomic_load_agent(const uint64_t *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void atomic_store_agent(uint64_t *p, uint64_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t atomic_load_agent(const uint32_t *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void atomic_store_agent(uint32_t *p, uint32_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---------------------------------------------------------------------
// Decoupled lookback across the tiles of one layer.
//
// A tile publishes, per bin, a 64-bit word {epoch:32 | flag:2 | value:30}:
// first its own count (flag AGG, or PREFIX for tile 0), then, after walking
// back over earlier tiles until it meets a PREFIX, its inclusive prefix.
// Words of earlier calls carry an older epoch and are never taken for
// current ones, so nothing is cleared between calls. A wait that outlasts
// `spin_limit` polls gives up and publishes POISON instead, which every
// later tile propagates; callers report it. A limit of 0 gives up at once,
// without polling (every tile but the first is then poisoned).
constexpr uint32_t kFlagAgg = 1;
constexpr uint32_t kFlagPrefix = 2;
constexpr uint32_t kFlagPoison = 3;
constexpr uint32_t kValueMask = 0x3FFFFFFFu;
constexpr int32_t kPoisonBit = 0x40000000;   // reported in fault counts
constexpr int kLookbackWindow = 8;           // predecessors polled at once

__device__ __forceinline__ uint64_t pack_state(uint32_t epoch, uint32_t flag,
                                               uint32_t value) {
    return (static_cast<uint64_t>(epoch) << 32) |
           (static_cast<uint64_t>(flag) << 30) | (value & kValueMask);
}

// Every thread calls it. `st` points at the layer's words [tiles][nbins];
// `cnt(b)` gives this tile's count of bin b (from LDS); `set_excl(b, v)`
// stores the count of bin b in all earlier tiles (in LDS, visible after the
// caller's barrier); each thread passes only the bins b = tid + i * kBlock
// to both. Returns true in a thread that saw a poisoned or timed-out wait.
template <class Count, class SetExcl>
__device__ __forceinline__ bool tile_lookback(uint64_t *st, int tile,
                                              int nbins, uint32_t epoch,
                                              Count cnt, SetExcl set_excl,
                                              uint32_t spin_limit) {
    const int tid = threadIdx.x;
    uint64_t *mine = st + static_cast<int64_t>(tile) * nbins;
    for (int b = tid; b < nbins; b += kBlock)
        atomic_store_agent(mine + b,
                           pack_state(epoch, tile == 0 ? kFlagPrefix : kFlagAgg,
                                      static_cast<uint32_t>(cnt(b))));
    bool poisoned = false;
    for (int b = tid; b < nbins; b += kBlock) {
        if (tile == 0) {
            set_excl(b, 0);
            continue;
        }
        // Poll a window of kLookbackWindow predecessors per round trip (the
        // loads are independent), then fold them in from the nearest one:
        // add AGG values until a PREFIX; a word not yet published restarts
        // the next window at that tile.
        uint32_t acc = 0;
        bool bad = spin_limit == 0, done = bad;
        int t = tile - 1;
        uint32_t spins = 0;
        while (!done) {
            uint64_t v[kLookbackWindow];
#pragma unroll
            for (int i = 0; i < kLookbackWindow; ++i)
                v[i] = (t - i >= 0) ? atomic_load_agent(
                                          st + static_cast<int64_t>(t - i) * nbins + b)
                                    : 0;
            bool stalled = false;
#pragma unroll
            for (int i = 0; i < kLookbackWindow; ++i) {
                if (done || stalled) continue;
                const uint32_t flag = static_cast<uint32_t>(v[i] >> 30) & 3u;
                if (static_cast<uint32_t>(v[i] >> 32) != epoch || flag == 0) {
                    stalled = true;          // resume at tile t (not consumed)
                    continue;
                }
                acc += static_cast<uint32_t>(v[i]) & kValueMask;
                if (flag == kFlagPoison) {
                    bad = true;
                    done = true;
                } else if (flag == kFlagPrefix || t == 0) {
                    done = true;
                } else {
                    --t;
                }
            }
            if (done) break;
            if (stalled) {
                if (++spins > spin_limit) {
                    bad = true;
                    break;
                }
                __builtin_amdgcn_s_sleep(1);
            } else {
                spins = 0;
            }
        }
        atomic_store_agent(mine + b,
                           pack_state(epoch, bad ? kFlagPoison : kFlagPrefix,
                                      acc + static_cast<uint32_t>(cnt(b))));
        set_excl(b, static_cast<int32_t>(acc));
        poisoned |= bad;
    }
    return poisoned;
}

// Tile ticket and call epoch of one launch over one layer, from one 64-bit
// word {epoch:32 | ticket:32} with one atomic: the old value gives this
// workgroup's ticket and the epoch of the previous call. The holder of the
// last ticket adds 2^32 - tiles, which carries the ticket count (then equal
// to tiles) into the epoch: the word returns to {epoch + 1 | 0} after every
// other workgroup of the launch has taken its ticket and so read the old
// epoch. The call's own epoch is the old one plus one.
__device__ __forceinline__ void take_ticket(uint64_t *tick, int tiles,
                                            uint32_t &my_ticket,
                                            uint32_t &my_epoch) {
    const uint64_t v = atomicAdd(reinterpret_cast<unsigned long long *>(tick),
                                 1ull);
    const uint32_t t = static_cast<uint32_t>(v);
    if (t == static_cast<uint32_t>(tiles - 1))
        atomicAdd(reinterpret_cast<unsigned long long *>(tick),
                  (1ull << 32) - static_cast<uint64_t>(tiles));
    my_ticket = t;
    my_epoch = static_cast<uint32_t>(v >> 32) + 1u;
}

// Epoch of the latest completed launch over a layer (read by a later
// kernel, after that launch finished).
__device__ __forceinline__ uint32_t last_epoch(const uint64_t *tick) {
    return static_cast<uint32_t>(atomic_load_agent(tick) >> 32);
}

}  // namespace ue
