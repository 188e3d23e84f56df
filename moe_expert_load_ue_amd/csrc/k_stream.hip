// HBM-streaming steps: replica weight sync, replica gradient reduction and
// the dispatch gather.
//
// "How dots-infra/ultraep works" (summary and connection list): replicas
// receive synchronised master weights before expert compute, and replica
// gradients are reduced into the master gradients during backward. The
// UltraEP news write-up (section on how balancing in 300 microseconds
// works) moves expert state by persistent tile streaming; on one device
// that becomes persistent workgroups streaming 16-byte vectors through
// registers.
//
// Work items are (expert, matrix, chunk) triples taken grid-stride by a
// persistent grid sized to the device. Weight sync loads each master chunk
// once and stores it to every replica (read-once fan-out). Gradient
// reduction loads the master chunk and each replica chunk in table order
// and adds them left to right in fp32 (round to nearest even, no
// reassociation, no packed fp32 instructions). The gather reads each token
// row once and writes it to the k dispatch positions of that token. Loads
// are nontemporal; so are the stores of the reduction, while those of the
// sync and the gather are plain (measured 1.3% and 2.5% faster for their
// 1 : 2 and 1 : 8 mixes).
#include "ue_internal.h"

namespace ue {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kSyncVec = 8;     // 16-byte vectors per thread per chunk
constexpr int kSyncChunk = kBlock * kSyncVec * 16;       // bytes
constexpr int kReduceVec = 4;
constexpr int kReduceChunk = kBlock * kReduceVec * 16;   // bytes

struct StreamArgs {
    const int32_t *rep_off;
    const int32_t *rep_buf;
    int n_experts, n_mats, n_buffers;
    void *const *master;       // [n_experts_registered * n_mats]
    void *const *spare;        // [n_buffers * n_mats]
    int64_t mat_bytes[kMaxMats];
    int64_t mat_chunks[kMaxMats];
    int64_t chunks_per_expert;
    int64_t total;
};

__device__ __forceinline__ void locate(const StreamArgs &g, int64_t wi,
                                       int &e, int &m, int64_t &chunk) {
    e = static_cast<int>(wi / g.chunks_per_expert);
    int64_t c = wi - static_cast<int64_t>(e) * g.chunks_per_expert;
    m = 0;
    while (c >= g.mat_chunks[m]) {
        c -= g.mat_chunks[m];
        ++m;
    }
    chunk = c;
}

__global__ __launch_bounds__(kBlock) void k_weight_sync(StreamArgs g) {
    const int tid = threadIdx.x;
    for (int64_t wi = blockIdx.x; wi < g.total; wi += gridDim.x) {
        int e, m;
        int64_t chunk;
        locate(g, wi, e, m, chunk);
        const int lo = g.rep_off[e] + 1;
        const int hi = g.rep_off[e + 1];
        if (hi <= lo) continue;
        const char *src = static_cast<const char *>(g.master[e * g.n_mats + m]);
        const int64_t off = chunk * kSyncChunk;
        const int64_t end = (off + kSyncChunk < g.mat_bytes[m])
                                ? off + kSyncChunk : g.mat_bytes[m];
        if (end - off == kSyncChunk) {
            u32x4 v[kSyncVec];
            const u32x4 *s = reinterpret_cast<const u32x4 *>(src + off);
#pragma unroll
            for (int i = 0; i < kSyncVec; ++i)
                v[i] = __builtin_nontemporal_load(s + i * kBlock + tid);
            for (int r = lo; r < hi; ++r) {
                const int b = g.rep_buf[r];
                if (static_cast<uint32_t>(b) >= static_cast<uint32_t>(g.n_buffers))
                    continue;
                u32x4 *d = reinterpret_cast<u32x4 *>(
                    static_cast<char *>(g.spare[b * g.n_mats + m]) + off);
#pragma unroll
                for (int i = 0; i < kSyncVec; ++i)
                    d[i * kBlock + tid] = v[i];
            }
        } else {
            // last, partial chunk: whole vectors, then 2-byte elements
            const int64_t nvec = (end - off) / 16;
            for (int r = lo; r < hi; ++r) {
                const int b = g.rep_buf[r];
                if (static_cast<uint32_t>(b) >= static_cast<uint32_t>(g.n_buffers))
                    continue;
                char *dst = static_cast<char *>(g.spare[b * g.n_mats + m]);
                const u32x4 *s = reinterpret_cast<const u32x4 *>(src + off);
                u32x4 *d = reinterpret_cast<u32x4 *>(dst + off);
                for (int64_t i = tid; i < nvec; i += kBlock) d[i] = s[i];
                const int64_t t0 = off + nvec * 16;
                for (int64_t i = t0 + 2 * tid; i < end; i += 2 * kBlock)
                    *reinterpret_cast<uint16_t *>(dst + i) =
                        *reinterpret_cast<const uint16_t *>(src + i);
            }
        }
    }
}

__global__ __launch_bounds__(kBlock) void k_grad_reduce(StreamArgs g) {
    const int tid = threadIdx.x;
    for (int64_t wi = blockIdx.x; wi < g.total; wi += gridDim.x) {
        int e, m;
        int64_t chunk;
        locate(g, wi, e, m, chunk);
        const int lo = g.rep_off[e] + 1;
        const int hi = g.rep_off[e + 1];
        if (hi <= lo) continue;
        char *mst = static_cast<char *>(g.master[e * g.n_mats + m]);
        const int64_t off = chunk * kReduceChunk;
        const int64_t end = (off + kReduceChunk < g.mat_bytes[m])
                                ? off + kReduceChunk : g.mat_bytes[m];
        if (end - off == kReduceChunk) {
            f32x4 acc[kReduceVec];
            f32x4 *ms = reinterpret_cast<f32x4 *>(mst + off);
#pragma unroll
            for (int i = 0; i < kReduceVec; ++i)
                acc[i] = __builtin_nontemporal_load(ms + i * kBlock + tid);
            for (int r = lo; r < hi; ++r) {
                const int b = g.rep_buf[r];
                if (static_cast<uint32_t>(b) >= static_cast<uint32_t>(g.n_buffers))
                    continue;
                const f32x4 *rs = reinterpret_cast<const f32x4 *>(
                    static_cast<const char *>(g.spare[b * g.n_mats + m]) + off);
                f32x4 v[kReduceVec];
#pragma unroll
                for (int i = 0; i < kReduceVec; ++i)
                    v[i] = __builtin_nontemporal_load(rs + i * kBlock + tid);
#pragma unroll
                for (int i = 0; i < kReduceVec; ++i) {
                    acc[i].x = acc[i].x + v[i].x;
                    acc[i].y = acc[i].y + v[i].y;
                    acc[i].z = acc[i].z + v[i].z;
                    acc[i].w = acc[i].w + v[i].w;
                }
            }
#pragma unroll
            for (int i = 0; i < kReduceVec; ++i)
                __builtin_nontemporal_store(acc[i], ms + i * kBlock + tid);
        } else {
            float *mf = reinterpret_cast<float *>(mst + off);
            const int64_t n = (end - off) / 4;
            for (int64_t i = tid; i < n; i += kBlock) {
                float acc = mf[i];
                for (int r = lo; r < hi; ++r) {
                    const int b = g.rep_buf[r];
                    if (static_cast<uint32_t>(b) >=
                        static_cast<uint32_t>(g.n_buffers))
                        continue;
                    const float *rf = reinterpret_cast<const float *>(
                        static_cast<const char *>(g.spare[b * g.n_mats + m]) +
                        off);
                    acc = acc + rf[i];
                }
                mf[i] = acc;
            }
        }
    }
}

// One wave per token row; kGatherVec 16-byte vectors per lane per pass.
constexpr int kGatherVec = 8;

__global__ __launch_bounds__(kBlock) void k_gather_rows(
    const char *__restrict__ x, const int32_t *__restrict__ inv_perm, int T,
    int k, int64_t row_bytes, int64_t n_pos, char *__restrict__ out) {
    const int lane = threadIdx.x & 63;
    const int wave = (blockIdx.x * kBlock + threadIdx.x) >> 6;
    const int nwaves = (gridDim.x * kBlock) >> 6;
    const int64_t nvec = row_bytes / 16;
    for (int t = wave; t < T; t += nwaves) {
        const u32x4 *src = reinterpret_cast<const u32x4 *>(
            x + static_cast<int64_t>(t) * row_bytes);
        for (int64_t v0 = 0; v0 < nvec; v0 += 64 * kGatherVec) {
            u32x4 v[kGatherVec];
#pragma unroll
            for (int i = 0; i < kGatherVec; ++i) {
                const int64_t idx = v0 + i * 64 + lane;
                if (idx < nvec) v[i] = __builtin_nontemporal_load(src + idx);
            }
            // the token's destinations, 64 at a time: one load per lane,
            // then each broadcast from its lane, so that the row's stores
            // do not wait on one position load after another
            for (int j0 = 0; j0 < k; j0 += 64) {
                const int nj = k - j0 < 64 ? k - j0 : 64;
                const int my_pos =
                    lane < nj ? inv_perm[static_cast<int64_t>(t) * k + j0 + lane] : -1;
                for (int j = 0; j < nj; ++j) {
                    const int pos = __builtin_amdgcn_readlane(my_pos, j);
                    if (static_cast<uint64_t>(pos) >= static_cast<uint64_t>(n_pos))
                        continue;
                    u32x4 *dst = reinterpret_cast<u32x4 *>(
                        out + static_cast<int64_t>(pos) * row_bytes);
#pragma unroll
                    for (int i = 0; i < kGatherVec; ++i) {
                        const int64_t idx = v0 + i * 64 + lane;
                        if (idx < nvec) dst[idx] = v[i];
                    }
                }
            }
        }
    }
}

StreamArgs make_args(const ue_ctx &c, const int32_t *rep_off,
                     const int32_t *rep_buf, int n_experts, bool weights,
                     int64_t chunk_bytes) {
    StreamArgs g{};
    g.rep_off = rep_off;
    g.rep_buf = rep_buf;
    g.n_experts = n_experts;
    g.n_mats = c.reg_mats;
    g.n_buffers = c.reg_buffers;
    g.master = weights ? c.d_master_w : reinterpret_cast<void *const *>(c.d_master_g);
    g.spare = weights ? c.d_spare_w : reinterpret_cast<void *const *>(c.d_spare_g);
    g.chunks_per_expert = 0;
    const int64_t esize = weights ? 2 : 4;
    for (int m = 0; m < c.reg_mats; ++m) {
        g.mat_bytes[m] = c.mat_elems[m] * esize;
        g.mat_chunks[m] = (g.mat_bytes[m] + chunk_bytes - 1) / chunk_bytes;
        g.chunks_per_expert += g.mat_chunks[m];
    }
    g.total = g.chunks_per_expert * n_experts;
    return g;
}

int persistent_grid(const ue_ctx &c, int64_t work, int per_cu) {
    int64_t n = static_cast<int64_t>(c.num_cu) * per_cu;
    if (work < n) n = work;
    return n < 1 ? 1 : static_cast<int>(n);
}

}  // namespace

hipError_t launch_weight_sync(const ue_ctx &c, const int32_t *rep_off,
                              const int32_t *rep_buf, int n_experts,
                              hipStream_t s) {
    StreamArgs g = make_args(c, rep_off, rep_buf, n_experts, true, kSyncChunk);
    if (g.total == 0) return hipSuccess;
    // 16 workgroups per CU with plain stores: measured 1.3% faster than 8
    // with nontemporal stores
    hipLaunchKernelGGL(k_weight_sync, dim3(persistent_grid(c, g.total, 16)),
                       dim3(kBlock), 0, s, g);
    return hipGetLastError();
}

hipError_t launch_grad_reduce(const ue_ctx &c, const int32_t *rep_off,
                              const int32_t *rep_buf, int n_experts,
                              hipStream_t s) {
    StreamArgs g = make_args(c, rep_off, rep_buf, n_experts, false,
                             kReduceChunk);
    if (g.total == 0) return hipSuccess;
    // 4 workgroups per CU: measured faster than 8 for this read-heavy mix
    hipLaunchKernelGGL(k_grad_reduce, dim3(persistent_grid(c, g.total, 4)),
                       dim3(kBlock), 0, s, g);
    return hipGetLastError();
}

hipError_t launch_gather_rows(const ue_ctx &c, const void *x,
                              const int32_t *inv_perm, int T, int k, int H,
                              void *out, hipStream_t s) {
    if (T == 0) return hipSuccess;
    const int64_t row_bytes = static_cast<int64_t>(H) * 2;
    const int waves_per_block = kBlock / 64;
    int64_t blocks = (static_cast<int64_t>(T) + waves_per_block - 1) /
                     waves_per_block;
    const int64_t cap = static_cast<int64_t>(c.num_cu) * 16;
    if (blocks > cap) blocks = cap;
    hipLaunchKernelGGL(k_gather_rows, dim3(static_cast<int>(blocks)),
                       dim3(kBlock), 0, s, static_cast<const char *>(x),
                       inv_perm, T, k, row_bytes,
                       static_cast<int64_t>(T) * k, static_cast<char *>(out));
    return hipGetLastError();
}

}  // namespace ue
