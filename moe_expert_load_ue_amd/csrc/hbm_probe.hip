// Standalone HBM probe (not part of libue.so): what plain streaming kernels
// reach on this device with buffers far larger than the device-wide cache,
// for the traffic mixes of the streaming steps. Weight sync reads a chunk
// once and writes it to each replica (one read, f writes); gradient
// reduction reads the master and each replica and writes the master; the
// gather reads a row once and writes it k times. The probe times a 1:1 copy,
// a 1:2 fan-out, a 3:1 sum, read-only and write-only streams, each with
// 16-byte vectors over a persistent grid, and prints GB/s per pattern; then
// the rate of non-returning LDS atomic adds per cycle per CU.
//
// Build: hipcc --offload-arch=gfx950 -O3 -std=c++17 hbm_probe.hip -o hbm_probe
// Every index stays below the buffer's vector count (chunk loops are bounded
// by the whole chunks that fit).
#include <hip/hip_runtime.h>

#include <cstdio>

#define CHECK(x)                                                         \
    do {                                                                 \
        hipError_t err_ = (x);                                           \
        if (err_ != hipSuccess) {                                        \
            std::printf("HIP error %s at line %d\n",                     \
                        hipGetErrorString(err_), __LINE__);              \
            return 1;                                                    \
        }                                                                \
    } while (0)

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
constexpr int kV = 8;                       // vectors per thread per chunk
constexpr long kChunk = 256L * kV;          // vectors per chunk

// n_in inputs summed (xor) into n_out outputs, chunk by chunk
template <int NIN, int NOUT>
__global__ __launch_bounds__(256) void k_stream(const u32x4 *const *in,
                                                u32x4 *const *out, long n16) {
    const long nchunks = n16 / kChunk;
    for (long c = blockIdx.x; c < nchunks; c += gridDim.x) {
        const long base = c * kChunk + threadIdx.x;
        u32x4 v[kV];
#pragma unroll
        for (int i = 0; i < kV; ++i)
            v[i] = __builtin_nontemporal_load(in[0] + base + 256L * i);
#pragma unroll
        for (int j = 1; j < NIN; ++j)
#pragma unroll
            for (int i = 0; i < kV; ++i)
                v[i] ^= __builtin_nontemporal_load(in[j] + base + 256L * i);
#pragma unroll
        for (int j = 0; j < NOUT; ++j)
#pragma unroll
            for (int i = 0; i < kV; ++i)
                __builtin_nontemporal_store(v[i], out[j] + base + 256L * i);
    }
}

// read-only: one store per thread at the end keeps the loads
__global__ __launch_bounds__(256) void k_read(const u32x4 *in, u32x4 *sink,
                                              long n16) {
    const long nchunks = n16 / kChunk;
    u32x4 acc = {0, 0, 0, 0};
    for (long c = blockIdx.x; c < nchunks; c += gridDim.x) {
        const long base = c * kChunk + threadIdx.x;
#pragma unroll
        for (int i = 0; i < kV; ++i)
            acc ^= __builtin_nontemporal_load(in + base + 256L * i);
    }
    sink[blockIdx.x * 256L + threadIdx.x] = acc;
}

__global__ __launch_bounds__(256) void k_write(u32x4 *out, long n16) {
    const long nchunks = n16 / kChunk;
    const u32x4 v = {1u, 2u, 3u, static_cast<unsigned>(threadIdx.x)};
    for (long c = blockIdx.x; c < nchunks; c += gridDim.x) {
        const long base = c * kChunk + threadIdx.x;
#pragma unroll
        for (int i = 0; i < kV; ++i)
            __builtin_nontemporal_store(v, out + base + 256L * i);
    }
}

// LDS atomic throughput: each thread issues kLdsIters non-returning adds
// into a 2048-word LDS array, at hashed (random) or lane-linear addresses;
// every address is masked into the array.
constexpr int kLdsIters = 2048;
template <bool kRandom>
__global__ __launch_bounds__(256) void k_lds_add(unsigned *out) {
    __shared__ unsigned a[2048];
    for (int i = threadIdx.x; i < 2048; i += 256) a[i] = 0;
    __syncthreads();
    unsigned x = threadIdx.x * 2654435761u + blockIdx.x;
    const int lane = threadIdx.x & 63;
    for (int i = 0; i < kLdsIters; ++i) {
        unsigned addr;
        if (kRandom) {
            x = x * 1664525u + 1013904223u;
            addr = (x >> 8) & 2047u;
        } else {
            addr = static_cast<unsigned>(lane + 64 * (i & 31)) & 2047u;
        }
        __hip_atomic_fetch_add(&a[addr], 1u, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_WORKGROUP);
    }
    __syncthreads();
    if (threadIdx.x == 0) out[blockIdx.x] = a[5];
}

int main() {
    const long bytes = 1L << 30;            // per buffer, 4x the cache
    const long n16 = bytes / 16;
    int dev = 0, ncu = 0;
    CHECK(hipGetDevice(&dev));
    CHECK(hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev));
    u32x4 *buf[4];
    for (auto &b : buf) {
        CHECK(hipMalloc(&b, bytes));
        CHECK(hipMemset(b, 1, bytes));
    }
    u32x4 **ptrs;
    CHECK(hipMalloc(&ptrs, sizeof(u32x4 *) * 8));
    hipEvent_t e0, e1;
    CHECK(hipEventCreate(&e0));
    CHECK(hipEventCreate(&e1));
    const int grid = ncu * 4;
    auto timed = [&](const char *name, double moved, auto launch) -> int {
        for (int w = 0; w < 2; ++w) launch();
        CHECK(hipDeviceSynchronize());
        CHECK(hipEventRecord(e0, 0));
        for (int r = 0; r < 10; ++r) launch();
        CHECK(hipEventRecord(e1, 0));
        CHECK(hipEventSynchronize(e1));
        float ms = 0;
        CHECK(hipEventElapsedTime(&ms, e0, e1));
        std::printf("%-34s %9.1f GB/s\n", name, moved / (ms / 10 * 1e-3) / 1e9);
        return 0;
    };
    const u32x4 *const *cin = ptrs;
    u32x4 *const *cout4 = ptrs + 4;
    u32x4 *host[8] = {buf[0], buf[1], buf[2], buf[3], buf[3], buf[2], buf[1], buf[0]};
    // inputs buf0..; outputs from buf3 down: never an input of the same run
    CHECK(hipMemcpy(ptrs, host, sizeof(host), hipMemcpyHostToDevice));
    if (timed("copy 1 read : 1 write", 2.0 * bytes, [&] {
            hipLaunchKernelGGL((k_stream<1, 1>), dim3(grid), dim3(256), 0, 0, cin, cout4, n16);
        })) return 1;
    if (timed("fan-out 1 read : 2 writes", 3.0 * bytes, [&] {
            hipLaunchKernelGGL((k_stream<1, 2>), dim3(grid), dim3(256), 0, 0, cin, cout4, n16);
        })) return 1;
    if (timed("sum 3 reads : 1 write", 4.0 * bytes, [&] {
            hipLaunchKernelGGL((k_stream<3, 1>), dim3(grid), dim3(256), 0, 0, cin, cout4, n16);
        })) return 1;
    if (timed("read only", 1.0 * bytes, [&] {
            hipLaunchKernelGGL(k_read, dim3(grid), dim3(256), 0, 0, buf[0], buf[3], n16);
        })) return 1;
    if (timed("write only", 1.0 * bytes, [&] {
            hipLaunchKernelGGL(k_write, dim3(grid), dim3(256), 0, 0, buf[3], n16);
        })) return 1;
    if (timed("hipMemcpyAsync device to device", 2.0 * bytes, [&] {
            (void)hipMemcpyAsync(buf[3], buf[0], bytes, hipMemcpyDeviceToDevice, 0);
        })) return 1;
    // what the device reports of its memory (the transfers per clock are
    // not reported, so no peak is derived here)
    int mem_khz = 0, bus_bits = 0;
    CHECK(hipDeviceGetAttribute(&mem_khz, hipDeviceAttributeMemoryClockRate, dev));
    CHECK(hipDeviceGetAttribute(&bus_bits, hipDeviceAttributeMemoryBusWidth, dev));
    std::printf("%-34s memory clock %d kHz, bus %d bits\n",
                "device-reported memory", mem_khz, bus_bits);
    // LDS atomics: adds per cycle per CU at the device clock
    int clock_khz = 0;
    CHECK(hipDeviceGetAttribute(&clock_khz, hipDeviceAttributeClockRate, dev));
    const int lgrid = ncu * 8;
    auto lds = [&](const char *name, auto launch) -> int {
        launch();
        CHECK(hipDeviceSynchronize());
        CHECK(hipEventRecord(e0, 0));
        for (int r = 0; r < 5; ++r) launch();
        CHECK(hipEventRecord(e1, 0));
        CHECK(hipEventSynchronize(e1));
        float ms = 0;
        CHECK(hipEventElapsedTime(&ms, e0, e1));
        const double adds = double(lgrid) * 256 * kLdsIters;
        const double per_s = adds / (ms / 5 * 1e-3);
        std::printf("%-34s %9.2f adds/cycle/CU (%d CUs, %d MHz)\n", name,
                    per_s / (clock_khz * 1e3) / ncu, ncu, clock_khz / 1000);
        return 0;
    };
    unsigned *sink = reinterpret_cast<unsigned *>(buf[3]);
    if (lds("LDS atomic add, random addresses", [&] {
            hipLaunchKernelGGL(k_lds_add<true>, dim3(lgrid), dim3(256), 0, 0, sink);
        })) return 1;
    if (lds("LDS atomic add, lane-linear", [&] {
            hipLaunchKernelGGL(k_lds_add<false>, dim3(lgrid), dim3(256), 0, 0, sink);
        })) return 1;
    return 0;
}
