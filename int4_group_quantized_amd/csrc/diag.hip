// Benchmark diagnostics (a library of their own, libq4g128_diag.so): kernels
// that give the batch-1 GEMV's ceilings on the device it runs on.  None of
// them is part of the product; bench.py times them beside the GEMV.
//
//   * a read-only twin of the batch-1 GEMV kernel for K = 3,072 (32 lanes per
//     row, 3 chunks per lane): the same grid, pass walk and pass schedule,
//     weight, scale, minimum and activation loads with the same addresses,
//     and no arithmetic: every loaded word is XOR-folded into one
//     value per wave.  The rumik write-up ("Step 7: why the GEMV was stuck, and
//     a CUDA kernel") builds exactly such a twin to separate the memory time of
//     a GEMV from its arithmetic;
//   * a plain streaming read of a byte range with 16-byte non-temporal loads
//     (the achievable read rate for one launch of that size);
//   * an empty kernel on the same grid (the back-to-back launch floor).
#include <hip/hip_runtime.h>

#include <atomic>

#include "q4g128_diag.h"
#include "q4_device.hpp"
#include "gemv_pass.hpp"

namespace q4 {

constexpr int kOutWords = 4096;  // checksum words: at least the waves of the GEMV grid on 256 CUs

__device__ __forceinline__ uint32_t fold_wave(uint32_t v) {
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) v ^= (uint32_t)__shfl_xor((int)v, o, 64);
    return v;
}

template <int LPR, int CPL>
__device__ __forceinline__ uint32_t fold_pass(const PassLoad<CPL>& L) {
    uint32_t v = 0;
#pragma unroll
    for (int t = 0; t < CPL; ++t) v ^= L.q[t].x ^ L.q[t].y ^ L.q[t].z ^ L.q[t].w ^ ((uint32_t)L.s[t] << 16) ^ L.m[t];
    return v;
}

template <int LPR, int CPL>
__global__ void __launch_bounds__(kGemvThreads)
gemv_read_twin_kernel(const uint8_t* __restrict__ packed, const uint16_t* __restrict__ scales,
                      const uint16_t* __restrict__ mins, const uint16_t* __restrict__ x,
                      uint32_t* __restrict__ out, int n, int k) {
    constexpr int RPW = 64 / LPR;
    extern __shared__ u4 x_lds[];
    const int C = k >> 5;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int j = lane % LPR;
    const int rsub = lane / LPR;
    const long passes = ((long)n + RPW - 1) / RPW;
    const long W = (long)gridDim.x * (blockDim.x >> 6);
    long p = (long)wave * gridDim.x + xcd_block_order(blockIdx.x, gridDim.x);
    auto row_of = [&](long pp) { return (int)(pp * RPW) + rsub; };
    auto clamp = [&](int r) { return r < n ? r : n - 1; };

    // The GEMV's schedule at this K: the next pass is requested before the
    // current one is consumed.
    static_assert(pass_schedule(LPR, CPL, false) == kPassNextFirst, "twin follows the GEMV's schedule");
    PassLoad<CPL> A, B;
    if (p < passes) load_pass<LPR, CPL>(A, packed, scales, mins, clamp(row_of(p)), k, j);
    stage_x<LPR, CPL>(x, x_lds, k);
    __syncthreads();
    h2 xp[CPL][16];
    float xs[CPL];
    lane_activations<LPR, CPL, false>(x_lds, C, j, xp, xs);
    uint32_t acc = 0;
#pragma unroll
    for (int t = 0; t < CPL; ++t) {
        acc ^= __builtin_bit_cast(uint32_t, xs[t]);
#pragma unroll
        for (int i = 0; i < 16; ++i) acc ^= as_u32(xp[t][i]);
    }

    while (p < passes) {
        if (p + W < passes) load_pass<LPR, CPL>(B, packed, scales, mins, clamp(row_of(p + W)), k, j);
        acc ^= fold_pass<LPR, CPL>(A);
        p += W;
        if (p >= passes) break;
        if (p + W < passes) load_pass<LPR, CPL>(A, packed, scales, mins, clamp(row_of(p + W)), k, j);
        acc ^= fold_pass<LPR, CPL>(B);
        p += W;
    }
    acc = fold_wave(acc);
    if (lane == 0) out[(long)blockIdx.x * (blockDim.x >> 6) + wave] = acc;
}

// One-shot read: block b reads U * blockDim.x consecutive 16-byte words,
// thread t words t, t + blockDim.x, ...; the grid covers the range once, so
// the hardware dispatcher hands blocks to whichever CU frees up first.  Of
// the grids measured for a 41 MB read (persistent 512 x 512 threads with 1 to
// 16 loads in flight, one-shot blocks of 256 to 1,024 threads with 1 to 16
// words each) this one was the fastest.
constexpr int kStreamThreads = 1024;
constexpr int kStreamWords = 2;

__global__ void __launch_bounds__(kStreamThreads)
stream_read_kernel(const u4* __restrict__ src, long nvec, uint32_t* __restrict__ out) {
    const long base = (long)blockIdx.x * kStreamThreads * kStreamWords + threadIdx.x;
    uint32_t acc = 0;
    u4 v[kStreamWords];
#pragma unroll
    for (int u = 0; u < kStreamWords; ++u) {
        const long i = base + (long)u * kStreamThreads;
        v[u] = i < nvec ? __builtin_nontemporal_load(src + i) : u4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < kStreamWords; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    // The loads must not be optimised away: a thread stores its checksum only
    // when it equals a fixed value, which leaves the stores out in practice.
    if (acc == 0x9E3779B9u) out[(((long)blockIdx.x * kStreamThreads + threadIdx.x) >> 6) % kOutWords] = acc;
}

__global__ void __launch_bounds__(kGemvThreads) empty_kernel() {}

constexpr int kBlocksPerCu = 2;  // the GEMV's grid for K = 3,072: two 8-wave workgroups per CU
constexpr int kMaxDev = 64;
static std::atomic<int> g_cu[kMaxDev];

// The GEMV's grid on the current device (CU count queried once per device, so
// that the launch costs of these diagnostics match the library's).
static int grid_blocks() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDev) return -1;
    int cu = g_cu[dev].load(std::memory_order_relaxed);
    if (cu == 0) {
        if (hipDeviceGetAttribute(&cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return -1;
        g_cu[dev].store(cu, std::memory_order_relaxed);
    }
    return cu * kBlocksPerCu;
}

}  // namespace q4

extern "C" {

int32_t q4diag_out_words(void) { return q4::kOutWords; }

int32_t q4diag_gemv_read_twin(const uint8_t* packed, const uint16_t* scales, const uint16_t* mins,
                              const uint16_t* x, uint32_t* out, int64_t n, int64_t k, void* stream) {
    if (!packed || !scales || !mins || !x || !out || n <= 0 || n > 0x7FFFFF00LL) return -1;
    if (k != 3072) return -2;
    constexpr int LPR = 32, CPL = 3, RPW = 64 / LPR;
    const int blocks = q4::grid_blocks();
    if (blocks < 0) return -4;
    if ((long)blocks * (q4::kGemvThreads / 64) > q4::kOutWords) return -1;
    const long passes = (n + RPW - 1) / RPW;
    long grid = blocks;
    const long need = (passes + 7) / 8;
    if (grid > need) grid = need;
    hipLaunchKernelGGL((q4::gemv_read_twin_kernel<LPR, CPL>), dim3((unsigned)grid), dim3(q4::kGemvThreads),
                       (size_t)k * 2, (hipStream_t)stream, packed, scales, mins, x, out, (int)n, (int)k);
    return hipGetLastError() == hipSuccess ? 0 : -4;
}

int32_t q4diag_stream_read(const void* src, int64_t bytes, uint32_t* out, void* stream) {
    if (!src || !out || bytes <= 0 || bytes % 16 != 0 || ((uintptr_t)src & 15) != 0) return -1;
    const long nvec = bytes / 16;
    const long per = (long)q4::kStreamThreads * q4::kStreamWords;
    const long blocks = (nvec + per - 1) / per;
    if (blocks > 0x7FFFFFFFL) return -1;
    hipLaunchKernelGGL(q4::stream_read_kernel, dim3((unsigned)blocks), dim3(q4::kStreamThreads), 0,
                       (hipStream_t)stream, reinterpret_cast<const q4::u4*>(src), nvec, out);
    return hipGetLastError() == hipSuccess ? 0 : -4;
}

int32_t q4diag_empty(void* stream) {
    const int blocks = q4::grid_blocks();
    if (blocks < 0) return -4;
    hipLaunchKernelGGL(q4::empty_kernel, dim3((unsigned)blocks), dim3(q4::kGemvThreads), 0, (hipStream_t)stream);
    return hipGetLastError() == hipSuccess ? 0 : -4;
}

}  // extern "C"
