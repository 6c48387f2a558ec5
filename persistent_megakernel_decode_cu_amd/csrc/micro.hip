// Microbenchmarks of the costs the megakernel design trades against each other:
// an empty kernel launch from a stream and from a HIP graph (the per-kernel cost
// that a one-kernel-per-op step pays hundreds of times; Hazy Research megakernel
// news page, section 3), a flag handed back and forth between two workgroups
// through device memory with the same device-scope stores and loads the
// megakernel's events use (the cost of one dependency hop; section 4 gives about
// 500 ns for its GPU), a workgroup barrier, the rate at which one CU or all CUs
// fill LDS straight from HBM (the loader's page stream), and a plain streaming
// read of device memory (the practical bandwidth ceiling).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <vector>

#include "../../include/mk.h"

namespace mkm {

__device__ __forceinline__ uint64_t rtc() { return __builtin_amdgcn_s_memrealtime(); }
__device__ __forceinline__ uint32_t xcc_id() { return __builtin_amdgcn_s_getreg(20 | (3 << 11)) & 7u; }
__device__ __forceinline__ uint32_t uni(uint32_t v) { return __builtin_amdgcn_readfirstlane(v); }

typedef __attribute__((address_space(1))) uint32_t g_u32;
// device-scope store and load (bypassing the per-XCD non-coherent cache path)
__device__ __forceinline__ void st_dev(uint32_t* p, uint32_t v) {
    __hip_atomic_store((g_u32*)p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t ld_dev(const uint32_t* p) {
    return __hip_atomic_load((g_u32*)p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__global__ void k_empty() {}

// Blocks `a` and `b` pass a counter back and forth `rounds` times: a writes 2r + 1 to
// flag[0] and waits for 2r + 2 in flag[32]; b waits for 2r + 1 and answers 2r + 2.
// Every wait gives up after `limit` ticks of the 100 MHz clock (err = 1).  out: ticks
// of block a for all rounds, and the XCD of each block.
__global__ void k_pingpong(uint32_t* flag, int rounds, int a, int b, uint64_t limit, unsigned long long* ticks,
                           uint32_t* xcc, uint32_t* err) {
    const int me = blockIdx.x;
    if ((me != a && me != b) || threadIdx.x != 0) return;
    xcc[me == a ? 0 : 1] = xcc_id();
    const uint64_t t0 = rtc();
    for (int r = 0; r < rounds; ++r) {
        if (me == a) {
            st_dev(&flag[0], 2u * r + 1u);
            while (ld_dev(&flag[32]) != 2u * r + 2u)
                if (rtc() - t0 > limit || ld_dev(&flag[64])) {
                    st_dev(&flag[64], 1u);
                    *err = 1u;
                    return;
                }
        } else {
            while (ld_dev(&flag[0]) != 2u * r + 1u)
                if (rtc() - t0 > limit || ld_dev(&flag[64])) {
                    st_dev(&flag[64], 1u);
                    *err = 1u;
                    return;
                }
            st_dev(&flag[32], 2u * r + 2u);
        }
    }
    if (me == a) *ticks = rtc() - t0;
}

// n workgroup barriers of 384 threads (the megakernel's workgroup size)
__global__ void __launch_bounds__(384) k_barrier(int n, unsigned long long* ticks) {
    const uint64_t t0 = rtc();
    for (int i = 0; i < n; ++i) __syncthreads();
    if (threadIdx.x == 0) *ticks = rtc() - t0;
}

// Each workgroup streams its own `bytes` of src into a 64 KiB LDS ring with direct
// global-to-LDS 16-byte loads (4 waves, 1 KiB per load instruction, `depth` loads in
// flight per wave), as the megakernel's loader does.
template <int DEPTH>
__global__ void __launch_bounds__(256) k_lds_fill(const uint8_t* src, uint64_t bytes, uint32_t* sink) {
    __shared__ __attribute__((aligned(16))) uint8_t ring[65536];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const uint8_t* base = src + (uint64_t)blockIdx.x * bytes;
    const uint64_t nload = bytes / 1024;
    uint32_t j = 0;
    for (uint64_t i = (uint64_t)wave; i < nload; i += 4, ++j) {
        __builtin_amdgcn_global_load_lds((__attribute__((address_space(1))) void*)(base + i * 1024 + lane * 16),
                                         (__attribute__((address_space(3))) void*)&ring[(i % 64) * 1024], 16, 0, 2);
        if (j % DEPTH == DEPTH - 1) __builtin_amdgcn_s_waitcnt(0);  // all loads of this wave landed
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (threadIdx.x == 0) sink[blockIdx.x] = *(volatile uint32_t*)&ring[(blockIdx.x * 16) % 65536];
}

// Plain streaming read: every thread folds its 16-byte elements into one word.
typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));
__global__ void __launch_bounds__(256) k_stream_read(const u32x4v* src, uint64_t n16, uint32_t* sink) {
    uint32_t acc = 0;
    const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
    for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride) {
        const u32x4v v = __builtin_nontemporal_load(&src[i]);
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    sink[(uint64_t)blockIdx.x * blockDim.x + threadIdx.x] = acc;
}

struct Timer {
    hipEvent_t a = nullptr, b = nullptr;
    Timer() {
        (void)hipEventCreate(&a);
        (void)hipEventCreate(&b);
    }
    ~Timer() {
        (void)hipEventDestroy(a);
        (void)hipEventDestroy(b);
    }
};

int device_cus() {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    return n;
}

}  // namespace mkm

using namespace mkm;

#define MKM_CHECK(x)                    \
    do {                                \
        if ((x) != hipSuccess) {        \
            st = MK_E_HIP;              \
            goto done;                  \
        }                               \
    } while (0)

extern "C" {

mk_status mkm_launch_latency(int32_t n, float* us_stream, float* us_graph) {
    if (n < 1 || n > 100000 || !us_stream || !us_graph) return MK_E_INVALID;
    mk_status st = MK_OK;
    hipStream_t s = nullptr;
    hipGraph_t g = nullptr;
    hipGraphExec_t ge = nullptr;
    Timer t;
    float ms = 0.f;
    MKM_CHECK(hipStreamCreate(&s));
    for (int i = 0; i < 100; ++i) hipLaunchKernelGGL(k_empty, dim3(1), dim3(64), 0, s);
    MKM_CHECK(hipStreamSynchronize(s));
    MKM_CHECK(hipEventRecord(t.a, s));
    for (int i = 0; i < n; ++i) hipLaunchKernelGGL(k_empty, dim3(1), dim3(64), 0, s);
    MKM_CHECK(hipEventRecord(t.b, s));
    MKM_CHECK(hipEventSynchronize(t.b));
    MKM_CHECK(hipEventElapsedTime(&ms, t.a, t.b));
    *us_stream = ms * 1000.f / (float)n;
    MKM_CHECK(hipStreamBeginCapture(s, hipStreamCaptureModeThreadLocal));
    for (int i = 0; i < n; ++i) hipLaunchKernelGGL(k_empty, dim3(1), dim3(64), 0, s);
    MKM_CHECK(hipStreamEndCapture(s, &g));
    MKM_CHECK(hipGraphInstantiate(&ge, g, nullptr, nullptr, 0));
    MKM_CHECK(hipGraphLaunch(ge, s));
    MKM_CHECK(hipStreamSynchronize(s));
    MKM_CHECK(hipEventRecord(t.a, s));
    MKM_CHECK(hipGraphLaunch(ge, s));
    MKM_CHECK(hipEventRecord(t.b, s));
    MKM_CHECK(hipEventSynchronize(t.b));
    MKM_CHECK(hipEventElapsedTime(&ms, t.a, t.b));
    *us_graph = ms * 1000.f / (float)n;
done:
    if (ge) (void)hipGraphExecDestroy(ge);
    if (g) (void)hipGraphDestroy(g);
    if (s) (void)hipStreamDestroy(s);
    return st;
}

mk_status mkm_pingpong(int32_t rounds, int32_t same_xcd, float* ns_per_hop, int32_t* xcd_a, int32_t* xcd_b) {
    if (rounds < 1 || rounds > 1000000 || !ns_per_hop || !xcd_a || !xcd_b) return MK_E_INVALID;
    mk_status st = MK_OK;
    uint32_t* buf = nullptr;
    // workgroups are dealt to the 8 XCDs in turn: blocks 0 and 1 sit on different
    // XCDs, blocks 0 and 8 on the same one (the XCD ids read in the kernel say which)
    const int a = 0, b = same_xcd ? 8 : 1, grid = b + 1;
    uint32_t host[4] = {0, 0, 0, 0};
    unsigned long long ticks = 0;
    MKM_CHECK(hipMalloc(&buf, 4096));
    MKM_CHECK(hipMemset(buf, 0, 4096));
    hipLaunchKernelGGL(k_pingpong, dim3(grid), dim3(64), 0, nullptr, buf, rounds, a, b, (uint64_t)100000000ull,
                       (unsigned long long*)(buf + 256), buf + 300, buf + 310);
    MKM_CHECK(hipDeviceSynchronize());
    MKM_CHECK(hipMemcpy(&ticks, buf + 256, 8, hipMemcpyDeviceToHost));
    MKM_CHECK(hipMemcpy(host, buf + 300, 8, hipMemcpyDeviceToHost));
    MKM_CHECK(hipMemcpy(&host[2], buf + 310, 4, hipMemcpyDeviceToHost));
    if (host[2]) {
        st = MK_E_DEVICE;
        goto done;
    }
    *ns_per_hop = (float)ticks * 10.f / (2.f * (float)rounds);
    *xcd_a = (int32_t)host[0];
    *xcd_b = (int32_t)host[1];
done:
    if (buf) (void)hipFree(buf);
    return st;
}

mk_status mkm_barrier(int32_t n, float* ns_per_barrier) {
    if (n < 1 || n > 10000000 || !ns_per_barrier) return MK_E_INVALID;
    mk_status st = MK_OK;
    unsigned long long* d = nullptr;
    unsigned long long ticks = 0;
    MKM_CHECK(hipMalloc(&d, 8));
    hipLaunchKernelGGL(k_barrier, dim3(1), dim3(384), 0, nullptr, n, d);
    MKM_CHECK(hipDeviceSynchronize());
    MKM_CHECK(hipMemcpy(&ticks, d, 8, hipMemcpyDeviceToHost));
    *ns_per_barrier = (float)ticks * 10.f / (float)n;
done:
    if (d) (void)hipFree(d);
    return st;
}

mk_status mkm_lds_fill(uint64_t bytes_per_wg, int32_t n_wg, int32_t depth, float* gbps) {
    if (bytes_per_wg < 65536 || bytes_per_wg % 4096 || n_wg < 1 || n_wg > 4096 || !gbps ||
        (depth != 4 && depth != 8 && depth != 16))
        return MK_E_INVALID;
    mk_status st = MK_OK;
    uint8_t* src = nullptr;
    uint32_t* sink = nullptr;
    Timer t;
    float ms = 0.f;
    const uint64_t total = bytes_per_wg * (uint64_t)n_wg;
    auto launch = [&]() {
        if (depth == 4) hipLaunchKernelGGL(k_lds_fill<4>, dim3(n_wg), dim3(256), 0, nullptr, src, bytes_per_wg, sink);
        else if (depth == 8) hipLaunchKernelGGL(k_lds_fill<8>, dim3(n_wg), dim3(256), 0, nullptr, src, bytes_per_wg, sink);
        else hipLaunchKernelGGL(k_lds_fill<16>, dim3(n_wg), dim3(256), 0, nullptr, src, bytes_per_wg, sink);
    };
    MKM_CHECK(hipMalloc(&src, total));
    MKM_CHECK(hipMalloc(&sink, (size_t)n_wg * 4));
    MKM_CHECK(hipMemset(src, 1, total));
    launch();
    MKM_CHECK(hipDeviceSynchronize());
    MKM_CHECK(hipEventRecord(t.a, nullptr));
    for (int i = 0; i < 3; ++i) launch();
    MKM_CHECK(hipEventRecord(t.b, nullptr));
    MKM_CHECK(hipEventSynchronize(t.b));
    MKM_CHECK(hipEventElapsedTime(&ms, t.a, t.b));
    *gbps = (float)(3.0 * (double)total / ((double)ms * 1e-3) / 1e9);
done:
    if (src) (void)hipFree(src);
    if (sink) (void)hipFree(sink);
    return st;
}

mk_status mkm_stream_read(uint64_t bytes, float* gbps) {
    if (bytes < (1u << 20) || bytes % 16 || !gbps) return MK_E_INVALID;
    mk_status st = MK_OK;
    u32x4v* src = nullptr;
    uint32_t* sink = nullptr;
    Timer t;
    float ms = 0.f;
    const int cus = device_cus() > 0 ? device_cus() : 256;
    const int grid = cus * 8;
    MKM_CHECK(hipMalloc(&src, bytes));
    MKM_CHECK(hipMalloc(&sink, (size_t)grid * 256 * 4));
    MKM_CHECK(hipMemset(src, 1, bytes));
    hipLaunchKernelGGL(k_stream_read, dim3(grid), dim3(256), 0, nullptr, src, bytes / 16, sink);
    MKM_CHECK(hipDeviceSynchronize());
    MKM_CHECK(hipEventRecord(t.a, nullptr));
    for (int i = 0; i < 3; ++i) hipLaunchKernelGGL(k_stream_read, dim3(grid), dim3(256), 0, nullptr, src, bytes / 16, sink);
    MKM_CHECK(hipEventRecord(t.b, nullptr));
    MKM_CHECK(hipEventSynchronize(t.b));
    MKM_CHECK(hipEventElapsedTime(&ms, t.a, t.b));
    *gbps = (float)(3.0 * (double)bytes / ((double)ms * 1e-3) / 1e9);
done:
    if (src) (void)hipFree(src);
    if (sink) (void)hipFree(sink);
    return st;
}

}  // extern "C"
