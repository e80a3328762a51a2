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
// gives the same code (near_half below).
//
// Mapping: the groups of all rows are one flat array (row n, group g is group
// n*G + g; its 128 floats are contiguous, and so are its 64 packed bytes).
// 32 lanes own one group, 4 consecutive floats per lane (one 16-byte load);
// a half-wave handles kGroupsPerHalf consecutive groups with all its loads
// issued first, and a workgroup of two waves covers 4 KB of input.  The group
// minimum and maximum are reduced across the 32 lanes with DPP row operations
// (folded into the min/max instructions) and one swizzle.
//
// This file is built with -fno-honor-nans: the inputs are finite by contract,
// and every intermediate of a finite input is finite (the reciprocal is taken
// only of a non-zero scale).  Without NaNs the min/max need no quieting of
// their operands, which lets each DPP move fold into its min or max.
#include "q4_device.hpp"
#include "launch.hpp"

namespace q4 {

constexpr int kQuantThreads = 128;
constexpr int kGroupsPerHalf = 2;
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

// The code of one value is clamp(rne(RN(RN(w - min) / scale)), 0, 15), 0
// when the scale is 0.  The quotient is first formed with the hardware
// reciprocal, q' = RN(RN(w - min) * rcp(scale)), within 2^-22 * |q| of the
// correctly rounded q.  Only the half-integers 0.5 .. 14.5 separate different
// codes (rne, then the clamp), and below 16 that error is under 2^-18; so when
// q' lies more than 2^-16 from every half-integer, rne(q') = rne(q).  Lanes
// where it does not are redone with the correctly rounded division, which
// keeps every code equal to the definition.  A zero scale gets a zero
// reciprocal: every q' is then +-0, never near a half-integer, and every code
// is 0 as defined.
__device__ __forceinline__ int near_half(float q) {
    const float e = __builtin_fabsf(q - __builtin_rintf(q));  // exact
    return e > 0.5f - 1.52587890625e-05f;                     // 2^-16
}

typedef float f4v __attribute__((ext_vector_type(4)));

__global__ void __launch_bounds__(kQuantThreads)
quantize_kernel(const f4v* __restrict__ W, uint16_t* __restrict__ packed, uint16_t* __restrict__ scales,
                uint16_t* __restrict__ mins, long ngroups) {
    // Workgroup index over a two-dimensional grid (one dimension cannot hold
    // the largest exports); workgroups past the last group have nothing to do.
    const long block = (long)blockIdx.y * (long)gridDim.x + (long)blockIdx.x;
    if (block * kGroupsPerBlock >= ngroups) return;
    const int lane = threadIdx.x & 31;
    const long g0 = (block * (kQuantThreads / 32) + (threadIdx.x >> 5)) * kGroupsPerHalf;
    f4v v[kGroupsPerHalf];
    if ((block + 1) * kGroupsPerBlock <= ngroups) {
        // Every group of the workgroup exists: one base address, constant offsets.
        const f4v* wp = W + g0 * 32 + lane;
#pragma unroll
        for (int u = 0; u < kGroupsPerHalf; ++u) v[u] = __builtin_nontemporal_load(wp + u * 32);
    } else {
#pragma unroll
        for (int u = 0; u < kGroupsPerHalf; ++u) {
            const long g = g0 + u < ngroups ? g0 + u : ngroups - 1;  // clamped, every load in range
            v[u] = __builtin_nontemporal_load(W + g * 32 + lane);
        }
    }
    float sf[kGroupsPerHalf], mf[kGroupsPerHalf], q[kGroupsPerHalf][4];
    _Float16 s16[kGroupsPerHalf], m16[kGroupsPerHalf];
    int near = 0;  // bit u: a quotient of group u lies near a half-integer
#pragma unroll
    for (int u = 0; u < kGroupsPerHalf; ++u) {
        float lo = fminf(fminf(v[u].x, v[u].y), fminf(v[u].z, v[u].w));
        float hi = fmaxf(fmaxf(v[u].x, v[u].y), fmaxf(v[u].z, v[u].w));
        minmax32(lo, hi);
        s16[u] = (_Float16)((hi - lo) / 15.0f);
        m16[u] = (_Float16)(lo + 0.0f);
        sf[u] = (float)s16[u];
        mf[u] = (float)m16[u];
        const float rs = sf[u] != 0.0f ? __builtin_amdgcn_rcpf(sf[u]) : 0.0f;
        q[u][0] = (v[u].x - mf[u]) * rs;
        q[u][1] = (v[u].y - mf[u]) * rs;
        q[u][2] = (v[u].z - mf[u]) * rs;
        q[u][3] = (v[u].w - mf[u]) * rs;
        near |= (near_half(q[u][0]) | near_half(q[u][1]) | near_half(q[u][2]) | near_half(q[u][3])) << u;
    }
    if (__ballot(near != 0) != 0) {  // rare: the correctly rounded quotients
#pragma unroll
        for (int u = 0; u < kGroupsPerHalf; ++u)
            if ((near >> u) & 1) {
                const float d = sf[u] != 0.0f ? sf[u] : 1.0f;
                q[u][0] = (v[u].x - mf[u]) / d;
                q[u][1] = (v[u].y - mf[u]) / d;
                q[u][2] = (v[u].z - mf[u]) / d;
                q[u][3] = (v[u].w - mf[u]) / d;
            }
    }
#pragma unroll
    for (int u = 0; u < kGroupsPerHalf; ++u) {
        // Codes as exact small integers in fp32, clamped by one median each,
        // packed as c0 + 16 c1 + 256 c2 + 4096 c3 (exact) and converted once.
        const float c0 = __builtin_amdgcn_fmed3f(__builtin_rintf(q[u][0]), 0.0f, 15.0f);
        const float c1 = __builtin_amdgcn_fmed3f(__builtin_rintf(q[u][1]), 0.0f, 15.0f);
        const float c2 = __builtin_amdgcn_fmed3f(__builtin_rintf(q[u][2]), 0.0f, 15.0f);
        const float c3 = __builtin_amdgcn_fmed3f(__builtin_rintf(q[u][3]), 0.0f, 15.0f);
        const float word = __builtin_fmaf(c3, 4096.0f, __builtin_fmaf(c2, 256.0f, __builtin_fmaf(c1, 16.0f, c0)));
        const long g = g0 + u;
        if (g < ngroups) {
            packed[g * 32 + lane] = (uint16_t)(uint32_t)word;
            if (lane == 0) {
                scales[g] = __builtin_bit_cast(uint16_t, s16[u]);
                mins[g] = __builtin_bit_cast(uint16_t, m16[u]);
            }
        }
    }
}

hipError_t launch_quantize(const float* W, uint8_t* packed, uint16_t* scales, uint16_t* mins, int64_t n,
                           int64_t k, hipStream_t st) {
    const long ngroups = (long)n * (long)(k / 128);
    const long blocks = (ngroups + kGroupsPerBlock - 1) / kGroupsPerBlock;
    constexpr long kMaxX = 1L << 30;
    const long gx = blocks < kMaxX ? blocks : kMaxX;
    const long gy = (blocks + gx - 1) / gx;  // at most 8 for kQuantizeMaxGroups
    hipLaunchKernelGGL(quantize_kernel, dim3((unsigned)gx, (unsigned)gy), dim3(kQuantThreads), 0, st,
                       reinterpret_cast<const f4v*>(W), reinterpret_cast<uint16_t*>(packed), scales, mins,
                       ngroups);
    return hipGetLastError();
}

}  // namespace q4
