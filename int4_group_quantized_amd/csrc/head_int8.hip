// int8 output-head matrix-vector product for gfx950:
//   y[n] = scale[n] * sum_k q[n][k] * x[k]
// q int8 [N][K] (one signed code per byte, row-major), scale one fp16 per
// row, x fp16 [K], y fp32.  The rumik-oss-1 int4 write-up moved the audio
// output head to int8 with a kernel of its own because int4 group-128 was
// too lossy there (the section on the per-token time after the 36 layers);
// the per-row symmetric layout is the plain reading of "int8 weights".
//
// Work mapping (K only): a chunk is 16 codes (16 bytes); C8 = K / 16 chunks
// per row; 64 lanes per row, so one wave covers one row per pass; lane j owns
// chunks j + 64t, t < CPL = ceil(C8 / 64).  Rows whose C8 is not a multiple
// of 64 are ragged: a missing chunk loads the row's last chunk (in range)
// and meets zero activations, adding exactly zero.
//
// Exact codes without a convert: for a dword of four signed codes,
// t = q ^ 0x80808080 holds q + 128 in each byte; OR-ing bytes 0 and 2 (or
// 1 and 3) into the mantissa of fp16 1024.0 gives 1152 + q exactly, and one
// packed fp16 subtraction of 1152 leaves q (|q| <= 128 is exact in fp16).
// v_dot2_f32_f16 then multiplies codes and activations exactly and adds in
// fp32: two chains per lane (even and odd code pairs), joined once, summed
// over the 64 lanes by a fixed butterfly and scaled by the row's fp16 scale.
//
// Persistent grid as in the int4 GEMV: every wave walks rows p, p + W, ...
// with one or two rows of codes in flight (per chunk count, below),
// workgroups renumbered XCD by XCD.
#include "q4_device.hpp"
#include "launch.hpp"

namespace q4 {

constexpr int kHeadThreads = 512;

template <int CPL>
struct HeadRow {
    u4 q[CPL];
    uint16_t s;
};

template <int CPL, bool RAGGED>
__device__ __forceinline__ void head_load(HeadRow<CPL>& R, const int8_t* __restrict__ q,
                                          const uint16_t* __restrict__ scales, int rowc, int k, int j) {
    const int C8 = k >> 4;
    const u4* rp = reinterpret_cast<const u4*>(q + (size_t)rowc * (size_t)k);
#pragma unroll
    for (int t = 0; t < CPL; ++t) {
        int c = j + 64 * t;
        if (RAGGED) c = c < C8 ? c : C8 - 1;
        R.q[t] = __builtin_nontemporal_load(rp + c);
    }
    R.s = scales[rowc];
}

// Four signed codes -> (q0, q2) and (q1, q3) as exact fp16 pairs.
__device__ __forceinline__ void int8_pairs(uint32_t w, uint32_t magic, h2& even, h2& odd) {
    const uint32_t t = w ^ 0x80808080u;
    const h2 bias = {(_Float16)1152.0f, (_Float16)1152.0f};
    even = as_h2((t & 0x00FF00FFu) | magic) - bias;
    odd = as_h2(((t >> 8) & 0x00FF00FFu) | magic) - bias;
}

template <int CPL>
__device__ __forceinline__ void head_compute(const HeadRow<CPL>& R, const u4 (&xr)[CPL][2], uint32_t magic,
                                             float* __restrict__ y, int row, int n, int j) {
    float ev = 0.0f, od = 0.0f;
#pragma unroll
    for (int t = 0; t < CPL; ++t) {
        const uint32_t w[4] = {R.q[t].x, R.q[t].y, R.q[t].z, R.q[t].w};
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            h2 ce, co;
            int8_pairs(w[d], magic, ce, co);
            const u4 xv = xr[t][d >> 1];
            const uint32_t xe = (d & 1) ? xv.z : xv.x;
            const uint32_t xo = (d & 1) ? xv.w : xv.y;
            ev = __builtin_amdgcn_fdot2(ce, as_h2(xe), ev, false);
            od = __builtin_amdgcn_fdot2(co, as_h2(xo), od, false);
        }
    }
    const float v = reduce_lanes<64>(ev + od) * f16_bits_to_f32(R.s);
    if (j == 0 && row < n) y[row] = v;
}

// D = rows of codes a wave keeps in flight: 2 (the next requested two rows
// ahead, after a row is computed) or 1 (the next requested after the
// current row is computed).  One row measured faster at 2, 3 and 8 chunks
// per lane (16,384 x 3,072: 9.34 against 10.22 us; 16,384 x 2,048: 7.62
// against 7.89; 4,096 x 8,192: 9.31 against 9.74; same bits) and slower at 4
// (8,192 x 4,096: 9.08 against 8.11), so the choice is per chunk count.
// XF: x is staged before the first rows are requested (otherwise after), so
// that the staging's wait does not also wait for those rows (loads complete
// in order) and the barrier does not hold the workgroup for its slowest
// wave's rows; the host picks it for short grids (launch_head).
template <int CPL, bool RAGGED, int D, bool XF>
__global__ void __launch_bounds__(kHeadThreads)
head_int8_kernel(const int8_t* __restrict__ q, const uint16_t* __restrict__ scales,
                 const uint16_t* __restrict__ x, float* __restrict__ y, int n, int k) {
    extern __shared__ u4 xl[];  // [C8][2]: window h of chunk c, pairs (e0, o0, e1, o1)
    const int C8 = k >> 4;
    const int tid = threadIdx.x;
    const int j = tid & 63;
    const int wave = tid >> 6;
    const long W = (long)gridDim.x * (blockDim.x >> 6);
    long p = (long)wave * gridDim.x + xcd_block_order(blockIdx.x, gridDim.x);
    auto clamp = [&](long r) { return (int)(r < n ? r : n - 1); };

    HeadRow<CPL> A, B;
    if constexpr (!XF) {
        if (p < n) head_load<CPL, RAGGED>(A, q, scales, clamp(p), k, j);
        if (D == 2 && p + W < n) head_load<CPL, RAGGED>(B, q, scales, clamp(p + W), k, j);
    }

    // Window w = 8 activations x0..x7 -> (x0, x2), (x1, x3), (x4, x6), (x5, x7),
    // the pair order of int8_pairs for the window's two code dwords.
    const u4* xv = reinterpret_cast<const u4*>(x);
    for (int w = tid; w < (k >> 3); w += blockDim.x) {
        const u4 v = xv[w];
        xl[w] = (u4){__builtin_amdgcn_perm(v.y, v.x, 0x05040100u), __builtin_amdgcn_perm(v.y, v.x, 0x07060302u),
                     __builtin_amdgcn_perm(v.w, v.z, 0x05040100u), __builtin_amdgcn_perm(v.w, v.z, 0x07060302u)};
    }
    __syncthreads();
    if constexpr (XF) {
        if (p < n) head_load<CPL, RAGGED>(A, q, scales, clamp(p), k, j);
        if (D == 2 && p + W < n) head_load<CPL, RAGGED>(B, q, scales, clamp(p + W), k, j);
    }
    u4 xr[CPL][2];
#pragma unroll
    for (int t = 0; t < CPL; ++t) {
        const int c = j + 64 * t;
        const bool valid = !RAGGED || c < C8;
        const uint32_t keep = valid ? 0xFFFFFFFFu : 0u;
        const int cc = valid ? c : C8 - 1;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const u4 v = xl[2 * cc + h];
            xr[t][h] = (u4){v.x & keep, v.y & keep, v.z & keep, v.w & keep};
        }
    }
    uint32_t magic;
    asm volatile("v_mov_b32 %0, 0x64006400" : "=v"(magic));

    if constexpr (D == 1) {
        while (p < n) {
            head_compute<CPL>(A, xr, magic, y, (int)p, n, j);
            p += W;
            if (p < n) head_load<CPL, RAGGED>(A, q, scales, clamp(p), k, j);
        }
        return;
    }
    while (p < n) {
        head_compute<CPL>(A, xr, magic, y, (int)p, n, j);
        if (p + 2 * W < n) head_load<CPL, RAGGED>(A, q, scales, clamp(p + 2 * W), k, j);
        p += W;
        if (p >= n) break;
        head_compute<CPL>(B, xr, magic, y, (int)p, n, j);
        if (p + 2 * W < n) head_load<CPL, RAGGED>(B, q, scales, clamp(p + 2 * W), k, j);
        p += W;
    }
}

template <int CPL, bool RAGGED, int D = (CPL == 2 || CPL == 3 || CPL == 8) ? 1 : 2>
static hipError_t launch_head(const int8_t* q, const uint16_t* scales, const uint16_t* x, float* y, int n, int k,
                              const DeviceInfo& dev, hipStream_t st) {
    const size_t lds = (size_t)k * 2;
    std::atomic<int>& cached = PerDevice<&head_int8_kernel<CPL, RAGGED, D, false>>::value[dev.device];
    int per_cu = cached.load(std::memory_order_relaxed);  // once per device; both forms have the same registers
    if (per_cu == 0) {
        int nb = 0;
        hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &nb, reinterpret_cast<const void*>(&head_int8_kernel<CPL, RAGGED, D, false>), kHeadThreads, 8192 * 2);
        if (e != hipSuccess) return e;
        per_cu = nb > 0 ? nb : 1;
        cached.store(per_cu, std::memory_order_relaxed);
    }
    long grid = (long)dev.num_cu * per_cu;
    const long need = ((long)n + (kHeadThreads / 64) - 1) / (kHeadThreads / 64);
    if (grid > need) grid = need;
    // x staged before the first row is requested when every wave has one row,
    // or two with two rows ahead (as for the int4 GEMV; measured, same bits:
    // 4,096 x 8,192 7.67 against 9.29 us, 4,096 x 3,072 4.21 against 4.62,
    // 8,192 x 4,096 7.58 against 8.17; 16,384 x 3,072, two rows per wave with
    // one ahead, 9.58 against 9.37, keeps the default order).
    const long waves = grid * (kHeadThreads / 64);
    if ((long)n <= waves || (D == 2 && (long)n <= 2 * waves)) {
        hipLaunchKernelGGL((head_int8_kernel<CPL, RAGGED, D, true>), dim3((unsigned)grid), dim3(kHeadThreads), lds,
                           st, q, scales, x, y, n, k);
    } else {
        hipLaunchKernelGGL((head_int8_kernel<CPL, RAGGED, D, false>), dim3((unsigned)grid), dim3(kHeadThreads), lds,
                           st, q, scales, x, y, n, k);
    }
    return hipGetLastError();
}

hipError_t launch_head_int8(const int8_t* q, const uint16_t* scales, const uint16_t* x, float* y, int64_t n,
                            int64_t k, const DeviceInfo& dev, hipStream_t st) {
    const int C8 = (int)(k >> 4);
    const int cpl = (C8 + 63) / 64;
    const bool ragged = C8 % 64 != 0;
#define Q4_HEAD(P)                                                                          \
    if (cpl == P)                                                                           \
        return ragged ? launch_head<P, true>(q, scales, x, y, (int)n, (int)k, dev, st)      \
                      : launch_head<P, false>(q, scales, x, y, (int)n, (int)k, dev, st);
    Q4_HEAD(1) Q4_HEAD(2) Q4_HEAD(3) Q4_HEAD(4) Q4_HEAD(5) Q4_HEAD(6) Q4_HEAD(7) Q4_HEAD(8)
#undef Q4_HEAD
    return hipErrorInvalidValue;  // K above the validated limit
}

}  // namespace q4
