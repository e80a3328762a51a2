// One "pass" of the batch-1 GEMV mapping: the loads and the per-lane
// arithmetic of RPW = 64 / LPR rows of one wave, shared by every kernel that
// must reproduce the batch-1 result bit for bit (the GEMV itself and the
// grouped GEMV), and the activation staging helper they use.
//
// Mapping (depends on K only): C = K / 32 chunks per row, LPR lanes per row,
// CPL chunks per lane; lane j of a row owns chunks j + t*LPR below C.
#pragma once

#include "q4_device.hpp"

namespace q4 {

// Schedules of the batch-1 pass loop (passes of weights a wave keeps in
// flight): two, the next requested after a pass is computed; or next-first,
// the next requested before the current pass is computed.  The mapping's
// choice is shared by the batch-1 and the grouped kernels.
constexpr int kPassAhead2 = 2;
constexpr int kPassNextFirst = 3;
constexpr int pass_schedule(int lpr, int cpl, bool ragged) {
    return !ragged && ((lpr == 32 && (cpl == 2 || cpl == 3)) || (lpr == 64 && cpl == 4)) ? kPassNextFirst
                                                                                          : kPassAhead2;
}

template <int CPL>
struct PassLoad {
    u4 q[CPL];
    uint16_t s[CPL];
    uint16_t m[CPL];
};

// Chunks past C (ragged rows only) load the row's last chunk instead: every
// load stays in range, and the chunk's activations are zero.
template <int LPR, int CPL, bool RAGGED = false>
__device__ __forceinline__ void load_pass(PassLoad<CPL>& L, const uint8_t* __restrict__ packed,
                                          const uint16_t* __restrict__ scales,
                                          const uint16_t* __restrict__ mins, int rowc, int k, int j) {
    const int G = k >> 7;
    if constexpr (!RAGGED) {
        const u4* rp = reinterpret_cast<const u4*>(packed + (size_t)rowc * (size_t)(k >> 1)) + j;
        const size_t g0 = (size_t)rowc * (size_t)G + (size_t)(j >> 2);
#pragma unroll
        for (int t = 0; t < CPL; ++t) {
            L.q[t] = __builtin_nontemporal_load(rp + t * LPR);
            L.s[t] = scales[g0 + t * (LPR / 4)];
            L.m[t] = mins[g0 + t * (LPR / 4)];
        }
    } else {
        const int C = k >> 5;
        const u4* rp = reinterpret_cast<const u4*>(packed + (size_t)rowc * (size_t)(k >> 1));
        const uint16_t* sp = scales + (size_t)rowc * (size_t)G;
        const uint16_t* mp = mins + (size_t)rowc * (size_t)G;
#pragma unroll
        for (int t = 0; t < CPL; ++t) {
            const int c = j + t * LPR < C ? j + t * LPR : C - 1;
            L.q[t] = __builtin_nontemporal_load(rp + c);
            L.s[t] = sp[c >> 2];
            L.m[t] = mp[c >> 2];
        }
    }
}

// Activation staging: nw 16-byte windows, window w read by load(w) and written
// by store(w, v), U windows per thread per batch.  A thread issues a batch's
// loads before its first wait: a wait on the vector-memory counter also
// covers the weight loads already in flight, and a wait per window would cost
// one L2 round trip each (three at K = 11,008).  A slot past nw loads and
// stores the thread's first window of the batch again (the same value to the
// same place, at a distinct address per lane), so a batch has no branch for
// the compiler to sink a load into.
template <int U, typename Load, typename Store>
__device__ __forceinline__ void stage_windows(int nw, Load load, Store store) {
    const int step = (int)blockDim.x;
    for (int w0 = (int)threadIdx.x; w0 < nw; w0 += U * step) {
        u4 v[U];
        int w[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            w[u] = w0 + u * step < nw ? w0 + u * step : w0;
            v[u] = load(w[u]);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) store(w[u], v[u]);
    }
}

template <int LPR, int CPL>
__device__ __forceinline__ void compute_pass(const PassLoad<CPL>& L, const h2 (&xp)[CPL][16],
                                             const float (&xs)[CPL], float* __restrict__ y, int row,
                                             int n, int j) {
    float yl = 0.0f;
#pragma unroll
    for (int t = 0; t < CPL; ++t) {
        h2 codes[16];
        chunk_codes(L.q[t], codes);
        const float dot = chunk_dot(codes, xp[t]);
        yl = group_update(yl, L.s[t], L.m[t], dot, xs[t]);
    }
    yl = reduce_lanes<LPR>(yl) * kInvUnit;
    if (j == 0 && row < n) y[row] = yl;
}

constexpr int kGemvThreads = 512;  // 8 waves: two workgroups fill a CU at four waves per SIMD

// Stage x [K] in LDS for the lanes' chunks: window w (8 halves) = quad
// (w & 3) of chunk (w >> 2), stored permuted into the code-pair order at
// x_lds[(w & 3) * C + (w >> 2)].  The caller synchronises the workgroup.
template <int LPR, int CPL>
__device__ __forceinline__ void stage_x(const uint16_t* __restrict__ x, u4* x_lds, int k) {
    const int C = k >> 5;
    const u4* xv = reinterpret_cast<const u4*>(x);
    // The longest row of an instantiation, K = 32 * LPR * CPL, has
    // 4 * LPR * CPL windows: one batch covers them.
    constexpr int kStage = (4 * LPR * CPL + kGemvThreads - 1) / kGemvThreads;
    stage_windows<kStage>(
        k >> 3, [&](int w) { return xv[w]; },
        [&](int w, u4 v) { x_lds[(w & 3) * C + (w >> 2)] = permute_window(v); });
}

// A lane's activation pairs and per-chunk sums, read from the staged x for
// its chunks j + t*LPR; a ragged lane's missing chunk gets zeros.
template <int LPR, int CPL, bool RAGGED>
__device__ __forceinline__ void lane_activations(const u4* x_lds, int C, int j, h2 (&xp)[CPL][16],
                                                 float (&xs)[CPL]) {
#pragma unroll
    for (int t = 0; t < CPL; ++t) {
        const int c = j + t * LPR;
        const bool valid = !RAGGED || c < C;
        const uint32_t keep = valid ? 0xFFFFFFFFu : 0u;
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            u4 v = x_lds[d * C + (valid ? c : C - 1)];
            v.x &= keep;
            v.y &= keep;
            v.z &= keep;
            v.w &= keep;
            xp[t][4 * d + 0] = as_h2(v.x);
            xp[t][4 * d + 1] = as_h2(v.y);
            xp[t][4 * d + 2] = as_h2(v.z);
            xp[t][4 * d + 3] = as_h2(v.w);
        }
        xs[t] = chunk_xsum(xp[t]);
    }
}

}  // namespace q4
