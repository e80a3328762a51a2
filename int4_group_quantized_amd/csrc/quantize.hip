// Export of float32 weights to the int4 group-128 format (the short CPU job of
// the rumik-oss-1 int4 write-up, "Step 3: an int4 file and a first kernel on
// the laptop", which quantised every projection in groups of 128 columns with
// an fp16 scale and minimum per group), as a streaming GPU kernel.
//
// Per group: lo = min, hi = max of its 128 values; min = fp16(lo + 0);
// scale = fp16(fl32(hi - lo) / 15); code = clamp(rne((w - min) / scale), 0, 15)
// against the stored fp16 values, and code 0 everywhere when the stored scale
// is 0.  Every step is one IEEE fp32 operation, correctly rounded (hipcc's
// default division is the correctly rounded one, and contraction is off), so
// the codes, scales and minimums are fully determined by the input.  The
// per-value division is replaced by a reciprocal wherever that provably
// gives the same code (code_from and near_half below).
//
// Mapping: the groups of all rows are one flat array (row n, group g is group
// n*G + g; its 128 floats are contiguous, and so are its 64 packed bytes).
// 32 lanes own one group, 4 consecutive floats per lane (one 16-byte load);
// a half-wave handles kGroupsPerHalf consecutive groups with all its loads
// issued first.  The group minimum and maximum are reduced across the 32
// lanes with DPP row operations and one swizzle.
#include "q4_device.hpp"
#include "launch.hpp"

namespace q4 {

constexpr int kQuantThreads = 256;
constexpr int kGroupsPerHalf = 4;
constexpr int kGroupsPerBlock = (kQuantThreads / 32) * kGroupsPerHalf;

// Minimum and maximum over the 32 lanes of a half-wave; every lane gets both.
__device__ __forceinline__ void minmax32(float& lo, float& hi) {
    lo = fminf(lo, dpp_move<0xB1>(lo));   // quad_perm [1,0,3,2]
    hi = fmaxf(hi, dpp_move<0xB1>(hi));
    lo = fminf(lo, dpp_move<0x4E>(lo));   // quad_perm [2,3,0,1]
    hi = fmaxf(hi, dpp_move<0x4E>(hi));
    lo = fminf(lo, dpp_move<0x141>(lo));  // row_half_mirror
    hi = fmaxf(hi, dpp_move<0x141>(hi));
    lo = fminf(lo, dpp_move<0x140>(lo));  // row_mirror
    hi = fmaxf(hi, dpp_move<0x140>(hi));
    lo = fminf(lo, lane_swap16(lo));
    hi = fmaxf(hi, lane_swap16(hi));
}

// The code of one value: clamp(rne(RN(RN(w - min) / scale)), 0, 15), 0 when
// the scale is 0.  The quotient is first formed with the hardware reciprocal,
// q' = RN(RN(w - min) * rcp(scale)), within 2^-22 * |q| of the correctly
// rounded q.  Only the half-integers 0.5 .. 14.5 separate different codes
// (rne, then the clamp), and below 16 that error is under 2^-18; so when q'
// lies more than 2^-16 from every half-integer, rne(q') = rne(q).  Lanes
// where it does not are redone with the correctly rounded division (the
// caller's `near` test), which keeps every code equal to the definition.
__device__ __forceinline__ float quotient_fast(float w, float mf, float rs) { return (w - mf) * rs; }

__device__ __forceinline__ int near_half(float q) {
    const float e = __builtin_fabsf(q - __builtin_rintf(q));  // exact
    return e > 0.5f - 1.52587890625e-05f;                     // 2^-16
}

__device__ __forceinline__ uint32_t code_from(float q, float sf) {
    const float c = fminf(fmaxf(__builtin_rintf(q), 0.0f), 15.0f);
    return sf != 0.0f ? (uint32_t)c : 0u;
}

typedef float f4v __attribute__((ext_vector_type(4)));

__global__ void __launch_bounds__(kQuantThreads)
quantize_kernel(const f4v* __restrict__ W, uint16_t* __restrict__ packed, uint16_t* __restrict__ scales,
                uint16_t* __restrict__ mins, long ngroups) {
    const int lane = threadIdx.x & 31;
    const long g0 = ((long)blockIdx.x * (kQuantThreads / 32) + (threadIdx.x >> 5)) * kGroupsPerHalf;
    f4v v[kGroupsPerHalf];
#pragma unroll
    for (int u = 0; u < kGroupsPerHalf; ++u) {
        const long g = g0 + u < ngroups ? g0 + u : ngroups - 1;  // clamped, every load in range
        v[u] = __builtin_nontemporal_load(W + g * 32 + lane);
    }
#pragma unroll
    for (int u = 0; u < kGroupsPerHalf; ++u) {
        float lo = fminf(fminf(v[u].x, v[u].y), fminf(v[u].z, v[u].w));
        float hi = fmaxf(fmaxf(v[u].x, v[u].y), fmaxf(v[u].z, v[u].w));
        minmax32(lo, hi);
        const _Float16 s16 = (_Float16)((hi - lo) / 15.0f);
        const _Float16 m16 = (_Float16)(lo + 0.0f);
        const float sf = (float)s16, mf = (float)m16;
        const float rs = __builtin_amdgcn_rcpf(sf);
        float q0 = quotient_fast(v[u].x, mf, rs), q1 = quotient_fast(v[u].y, mf, rs);
        float q2 = quotient_fast(v[u].z, mf, rs), q3 = quotient_fast(v[u].w, mf, rs);
        const int near = near_half(q0) | near_half(q1) | near_half(q2) | near_half(q3);
        if (__ballot(near) != 0 && near) {  // rare: the correctly rounded quotients
            const float d = sf != 0.0f ? sf : 1.0f;
            q0 = (v[u].x - mf) / d;
            q1 = (v[u].y - mf) / d;
            q2 = (v[u].z - mf) / d;
            q3 = (v[u].w - mf) / d;
        }
        const uint32_t c0 = code_from(q0, sf), c1 = code_from(q1, sf);
        const uint32_t c2 = code_from(q2, sf), c3 = code_from(q3, sf);
        const long g = g0 + u;
        if (g < ngroups) {
            packed[g * 32 + lane] = (uint16_t)(c0 | (c1 << 4) | (c2 << 8) | (c3 << 12));
            if (lane == 0) {
                scales[g] = __builtin_bit_cast(uint16_t, s16);
                mins[g] = __builtin_bit_cast(uint16_t, m16);
            }
        }
    }
}

hipError_t launch_quantize(const float* W, uint8_t* packed, uint16_t* scales, uint16_t* mins, int64_t n,
                           int64_t k, hipStream_t st) {
    const long ngroups = (long)n * (long)(k / 128);
    const long grid = (ngroups + kGroupsPerBlock - 1) / kGroupsPerBlock;
    hipLaunchKernelGGL(quantize_kernel, dim3((unsigned)grid), dim3(kQuantThreads), 0, st,
                       reinterpret_cast<const f4v*>(W), reinterpret_cast<uint16_t*>(packed), scales, mins,
                       ngroups);
    return hipGetLastError();
}

}  // namespace q4
