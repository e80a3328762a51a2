// Prompt processing for up to 48 tokens with the activations held in
// registers (the dense M-token contraction of the rumik-oss-1 write-up,
// "Step 8: a prefill that stays int4"), in both forms of the library:
//   fp16 weights (as prefill.hip):
//     Y[m][n] = sum_k fp16(code*scale + min)[n][k] * X[m][k],  fp32 accumulate;
//   EPI, scale and minimum on the result (as prefill_epilogue.hip):
//     Y[m][n] = sum_g scale[n][g] * C_g[m][n] + min[n][g] * S_g[m],
//     C_g = sum over the group of code * x on the matrix cores, S_g = sum of x.
//
// Work split: one workgroup of NW waves per slice of at most 128 rows (the N
// rows cut into gridDim.x contiguous ranges, as for the other prefill
// kernels).  The waves split K instead of the rows: in round rd, wave w owns
// the GR groups starting at rd*NW*GR + w*GR and every 16-row tile of the
// slice.  So:
//  * each wave loads the activation fragments of its groups once per round
//    and keeps them in registers (16*GR*TT VGPRs); the matrix instructions
//    read both operands from registers, with no LDS tile and no barrier per
//    group;
//  * each weight byte of the slice is read and dequantised by exactly one
//    wave; a lane (r = lane & 15, q = lane >> 4) holds chunk q (32 codes) of
//    row r of a tile, requested two tiles ahead;
//  * after each tile the waves' partial sums meet in LDS (double-buffered by
//    tile parity, one barrier per tile) and wave t adds the NW partials of
//    token tile t in wave order, a fixed order, into the tile's total in LDS
//    (later rounds add to it); the workgroup stores Y from the totals at the
//    end.
// Groups past K get zero scale and minimum (their weights are +0); rows and
// tokens past the ends are clamped copies whose results are not stored.
//
// v_mfma_f32_16x16x32_f16 step s (0..3) contracts dword s of every lane's
// chunk: B = the lane's 8 fp16 weights (EPI: the 8 exact codes as fp16
// denormals c * 2^-20) in the pair order of dequant_dword, A = the same 8
// columns of token r of a token tile, permuted alike.  Output lane layout:
// lane l holds tokens 4*(l/16)+i of weight row l%16.  In the EPI form each
// group starts from a zero accumulator and y += (scale * 2^20) * C_g follows
// in fp32; the minimum term of the wave's (at most three) groups goes to the
// matrix cores as one v_mfma_f32_16x16x4_f32 per token tile, A = S_g of the
// tokens (computed once per round from the activation fragments, lane (r, q)
// holding token r and group q), B = the row's minimums.
#include "q4_device.hpp"
#include "launch.hpp"

namespace q4 {

constexpr int kSplitWaves = 8;
constexpr int kSplitMaxTiles = 8;  // 16-row tiles per workgroup (128 rows)

template <int TT, int GR, int NW, bool EPI>
__global__ void __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(NW / 4, NW / 4)))
prefill_split_kernel(const uint8_t* __restrict__ packed, const uint16_t* __restrict__ scales,
                     const uint16_t* __restrict__ mins, const uint16_t* __restrict__ X,
                     float* __restrict__ Y, int n, int k, int m) {
    extern __shared__ f4 lds_f4[];
    f4* part = lds_f4;                         // [2][NW][TT][64] partial sums per tile parity
    f4* tot = lds_f4 + 2 * NW * TT * 64;       // [kSplitMaxTiles][TT][64] totals of the slice
    constexpr int PER_ROUND = NW * GR;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r = lane & 15;
    const int q = lane >> 4;
    const int G = k >> 7;
    const int row_lo = (int)((long)blockIdx.x * n / gridDim.x);
    const int row_hi = (int)((long)(blockIdx.x + 1) * n / gridDim.x);
    const int RT = (row_hi - row_lo + 15) >> 4;
    const int R = (G + PER_ROUND - 1) / PER_ROUND;
    const size_t row_bytes = (size_t)(k >> 1);
    const DequantConsts kc = make_dequant_consts();

    for (int rd = 0; rd < R; ++rd) {
        const int gw = rd * PER_ROUND + wave * GR;  // first group of this wave (uniform)

        // Weight ring: slot [tile parity][group of the wave].
        u4 wq[2][GR];
        uint16_t ws[2][GR], wm[2][GR];
        auto load_w = [&](int p, int gi, int rt) {
            int row = row_lo + 16 * rt + r;
            row = row < row_hi ? row : row_hi - 1;
            int g = gw + gi;
            g = g < G ? g : G - 1;
            wq[p][gi] = __builtin_nontemporal_load(
                reinterpret_cast<const u4*>(packed + (size_t)row * row_bytes) + g * 4 + q);
            ws[p][gi] = scales[(size_t)row * G + g];
            wm[p][gi] = mins[(size_t)row * G + g];
        };
        // With one or three token tiles the activations are requested before
        // the first two tiles' weights (loads complete in order, so staging
        // them then waits for them alone); measured on the fused matrix (same
        // bits): M = 34 21.31 against 21.87 us, epilogue form 23.12 against
        // 24.10; M = 1 to 16 0.7-2.6% faster; but with two tiles (M = 24, 32)
        // 1.0-2.5% slower, so those keep the weights first.
        constexpr bool kActFirst = TT != 2;
        if constexpr (!kActFirst) {
#pragma unroll
            for (int p = 0; p < 2; ++p)
#pragma unroll
                for (int gi = 0; gi < GR; ++gi) load_w(p, gi, p);
        }

        // Activation fragments of this wave's groups: [group][k-step][token tile].
        u4 xa[GR][4][TT];
#pragma unroll
        for (int gi = 0; gi < GR; ++gi) {
            int g = gw + gi;
            g = g < G ? g : G - 1;
#pragma unroll
            for (int t = 0; t < TT; ++t) {
                int tok = 16 * t + r;
                tok = tok < m ? tok : m - 1;
                const u4* xp = reinterpret_cast<const u4*>(X + (size_t)tok * (size_t)k + (size_t)g * 128 + 32 * q);
#pragma unroll
                for (int s = 0; s < 4; ++s) xa[gi][s][t] = kActFirst ? xp[s] : permute_window(xp[s]);
            }
        }
        if constexpr (kActFirst) {
#pragma unroll
            for (int p = 0; p < 2; ++p)
#pragma unroll
                for (int gi = 0; gi < GR; ++gi) load_w(p, gi, p);
#pragma unroll
            for (int gi = 0; gi < GR; ++gi)
#pragma unroll
                for (int t = 0; t < TT; ++t)
#pragma unroll
                    for (int s = 0; s < 4; ++s) xa[gi][s][t] = permute_window(xa[gi][s][t]);
        }
        // EPI: the A operand of the minimum term, S_g of token r of each
        // token tile for the wave's group q (zero for q >= GR): the lane's 32
        // columns of token r, then the other three k-slots of the token
        // (lanes r + 16j).
        float sa[TT];
        if constexpr (EPI) {
            const h2 ones = {(_Float16)1.0f, (_Float16)1.0f};
#pragma unroll
            for (int t = 0; t < TT; ++t) sa[t] = 0.0f;
#pragma unroll
            for (int gi = 0; gi < GR; ++gi)
#pragma unroll
                for (int t = 0; t < TT; ++t) {
                    float v = 0.0f;
#pragma unroll
                    for (int s = 0; s < 4; ++s) {
                        const u4 w = xa[gi][s][t];
                        v = __builtin_amdgcn_fdot2(as_h2(w.x), ones, v, false);
                        v = __builtin_amdgcn_fdot2(as_h2(w.y), ones, v, false);
                        v = __builtin_amdgcn_fdot2(as_h2(w.z), ones, v, false);
                        v = __builtin_amdgcn_fdot2(as_h2(w.w), ones, v, false);
                    }
                    v = v + lane_swap16(v);
                    v = v + __shfl_xor(v, 32, 64);
                    sa[t] = q == gi ? v : sa[t];
                }
        }

        auto tile = [&](int rt, int p) {
            const f4 zero = {0.0f, 0.0f, 0.0f, 0.0f};
            f4 acc[TT];
#pragma unroll
            for (int t = 0; t < TT; ++t) acc[t] = zero;
            float bm = 0.0f;  // EPI: min of this lane's row for the wave's group q
#pragma unroll
            for (int gi = 0; gi < GR; ++gi) {
                const uint32_t keep = (uint32_t)__builtin_amdgcn_readfirstlane(-(int)(gw + gi < G));
                if constexpr (EPI) {
                    // Exact codes as fp16 denormals c * 2^-20 (each nibble moved
                    // to mantissa bits 4..7), in the pair order of dequant_dword.
                    const float sf = f16_bits_to_f32((uint16_t)(ws[p][gi] & keep)) * kInvUnit;
                    bm = q == gi ? f16_bits_to_f32((uint16_t)(wm[p][gi] & keep)) : bm;
                    const u4 cw = wq[p][gi];
                    load_w(p, gi, rt + 2);
                    f4 cg[TT];
#pragma unroll
                    for (int s = 0; s < 4; ++s) {
                        const uint32_t d = s == 0 ? cw.x : s == 1 ? cw.y : s == 2 ? cw.z : cw.w;
                        const u4 bw = {(d << 4) & 0x00F000F0u, d & 0x00F000F0u, (d >> 4) & 0x00F000F0u,
                                       (d >> 8) & 0x00F000F0u};
                        const h8 b = __builtin_bit_cast(h8, bw);
#pragma unroll
                        for (int t = 0; t < TT; ++t)
                            cg[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(h8, xa[gi][s][t]), b,
                                                                           s == 0 ? zero : cg[t], 0, 0, 0);
                    }
#pragma unroll
                    for (int t = 0; t < TT; ++t)
#pragma unroll
                        for (int i = 0; i < 4; ++i) acc[t][i] = __builtin_fmaf(sf, cg[t][i], acc[t][i]);
                } else {
                    uint32_t wv[16];
                    weights_fp16(wq[p][gi], (uint16_t)(ws[p][gi] & keep), (uint16_t)(wm[p][gi] & keep), kc, wv);
                    load_w(p, gi, rt + 2);
#pragma unroll
                    for (int s = 0; s < 4; ++s) {
                        const u4 bw = {wv[4 * s + 0], wv[4 * s + 1], wv[4 * s + 2], wv[4 * s + 3]};
                        const h8 b = __builtin_bit_cast(h8, bw);
#pragma unroll
                        for (int t = 0; t < TT; ++t)
                            acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(h8, xa[gi][s][t]), b,
                                                                            acc[t], 0, 0, 0);
                    }
                }
            }
            if constexpr (EPI) {
                // The minimum term of the wave's groups, sum over q of
                // S_q[tok] * min_q[row], on the matrix cores (fp32 operands).
#pragma unroll
                for (int t = 0; t < TT; ++t) acc[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(sa[t], bm, acc[t], 0, 0, 0);
            }
#pragma unroll
            for (int t = 0; t < TT; ++t) part[((p * NW + wave) * TT + t) * 64 + lane] = acc[t];
            lds_barrier();
            if (wave < TT) {
                f4 sum = part[(p * NW * TT + wave) * 64 + lane];
#pragma unroll
                for (int w2 = 1; w2 < NW; ++w2) sum += part[((p * NW + w2) * TT + wave) * 64 + lane];
                f4* tp = tot + (rt * TT + wave) * 64 + lane;
                *tp = rd > 0 ? *tp + sum : sum;
            }
        };

        // Pairs of tiles, then an odd last tile outside the loop (a break in
        // the middle of the pair would merge into the loop head and make the
        // compiler wait for every prefetched load there).
        int rt = 0;
        for (; rt + 1 < RT; rt += 2) {
            tile(rt, 0);
            tile(rt + 1, 1);
        }
        if (rt < RT) tile(rt, 0);
        lds_barrier();  // the next round reuses the partial buffers; the totals are complete
    }

    // Y from the totals, consecutive threads on consecutive rows of a token.
    // (Stores stay out of the tile loop: on this target a pending store in
    // the loop makes the compiler wait for every prefetched load.)
    const int nrows = row_hi - row_lo;
    const float* tf = reinterpret_cast<const float*>(tot);
    for (int idx = tid; idx < nrows * m; idx += 64 * NW) {
        const int tok = idx / nrows;
        const int rr = idx - tok * nrows;
        const int src = (((rr >> 4) * TT + (tok >> 4)) * 64 + ((tok & 15) >> 2) * 16 + (rr & 15)) * 4 + (tok & 3);
        Y[(size_t)tok * (size_t)n + row_lo + rr] = tf[src];
    }
}

template <int TT, int GR, bool EPI>
static hipError_t launch_split(const GemvArgs& a, const uint16_t* X, float* Y, int m,
                               const DeviceInfo& dev, hipStream_t st) {
    constexpr int NW = kSplitWaves;
    const size_t lds = ((size_t)2 * NW * TT + (size_t)kSplitMaxTiles * TT) * 64 *
                       sizeof(f4);
    std::atomic<int>& attr_set = PerDevice<&prefill_split_kernel<TT, GR, NW, EPI>>::value[dev.device];
    if (attr_set.load(std::memory_order_acquire) == 0) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&prefill_split_kernel<TT, GR, NW, EPI>),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)dev.max_lds);
        if (e != hipSuccess) return e;
        attr_set.store(1, std::memory_order_release);
    }
    // One workgroup per CU when the rows allow it; never more than
    // kSplitMaxTiles tiles per workgroup, never fewer than one row.
    long grid = dev.num_cu > 0 ? dev.num_cu : 1;
    const long need = ((long)a.n + 16 * kSplitMaxTiles - 1) / (16 * kSplitMaxTiles);
    if (grid < need) grid = need;
    const long tiles = ((long)a.n + 15) / 16;
    if (grid > tiles) grid = tiles;
    hipLaunchKernelGGL((prefill_split_kernel<TT, GR, NW, EPI>), dim3((unsigned)grid), dim3(64 * NW), lds, st,
                       a.packed, a.scales, a.mins, X, Y, a.n, a.k, m);
    return hipGetLastError();
}

template <int TT, bool EPI>
static hipError_t dispatch_split(const GemvArgs& a, const uint16_t* X, float* Y, int m, const DeviceInfo& dev,
                                 hipStream_t st) {
    // The fewest rounds at up to three groups per wave, then the fewest
    // groups per wave that cover K in that many rounds.
    constexpr int kMaxGroupsPerWave = 3;
    const int G = a.k >> 7;
    const int rounds = (G + kSplitWaves * kMaxGroupsPerWave - 1) / (kSplitWaves * kMaxGroupsPerWave);
    const int gr = (G + kSplitWaves * rounds - 1) / (kSplitWaves * rounds);
    if (gr <= 1) return launch_split<TT, 1, EPI>(a, X, Y, m, dev, st);
    if (gr <= 2) return launch_split<TT, 2, EPI>(a, X, Y, m, dev, st);
    return launch_split<TT, 3, EPI>(a, X, Y, m, dev, st);
}

template <bool EPI>
static hipError_t split_by_tokens(const GemvArgs& a, const uint16_t* X, float* Y, int m, const DeviceInfo& dev,
                                  hipStream_t st) {
    // At most three token tiles: the activation fragments of three groups of
    // 48 tokens take 144 of the 256 registers a wave has at two waves per SIMD.
    const int tiles = (m + 15) / 16;
    if (tiles <= 1) return dispatch_split<1, EPI>(a, X, Y, m, dev, st);
    if (tiles <= 2) return dispatch_split<2, EPI>(a, X, Y, m, dev, st);
    if (tiles <= 3) return dispatch_split<3, EPI>(a, X, Y, m, dev, st);
    return hipErrorInvalidValue;  // more than 48 tokens go to the other prefill kernels
}

hipError_t launch_prefill_split(const GemvArgs& a, const uint16_t* X, float* Y, int m, const DeviceInfo& dev,
                                hipStream_t st) {
    return split_by_tokens<false>(a, X, Y, m, dev, st);
}

hipError_t launch_prefill_split_epilogue(const GemvArgs& a, const uint16_t* X, float* Y, int m,
                                         const DeviceInfo& dev, hipStream_t st) {
    return split_by_tokens<true>(a, X, Y, m, dev, st);
}

}  // namespace q4
