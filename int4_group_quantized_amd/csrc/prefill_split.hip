// Prompt processing for up to 64 tokens with the activations held in
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
//    wave; at the matrix instructions a lane (r = lane & 15, q = lane >> 4)
//    holds chunk q (32 codes) of row r of a tile; the next tile is requested
//    when a tile starts;
//  * after each tile the waves' partial sums meet in LDS (double-buffered by
//    tile parity, one barrier per tile) and wave t adds the NW partials of
//    token tile t in wave order, a fixed order, into the tile's total in LDS
//    (later rounds add to it); the workgroup stores Y from the totals at the
//    end.
// Groups past K get zero scale and minimum (their weights are +0); rows and
// tokens past the ends are clamped copies whose results are not stored.
// Up to three token tiles take up to three groups per wave and round, four
// tiles one; more than 64 tokens (up to 96, or more on matrices of few rows,
// where the other prefill kernels leave CUs idle) run as launches over blocks
// of up to four token tiles.
//
// Load patterns.  Requested in the matrix-core layout, one 16-byte-per-lane
// load touches 16 rows (or tokens) at 64 bytes each.  Instead consecutive
// lanes request consecutive 16-byte words of a row, and each wave hands the
// words to the matrix-core layout through an LDS block of its own (one
// write and one read per word; padded rows, so the reads are conflict-free):
//  * activations, once per round: the 16 tokens x 16 words of a (group,
//    token tile) per four loads;
//  * codes, per tile, with one or two token tiles: the wave's 16 rows x 4*GR
//    words (with three they fit only in the fp16 form and measured 1-5%
//    slower on the fused matrix, 1-1.6% faster on 2,048 and 8,192 rows;
//    with four 3.6% slower; both keep the matrix-core layout);
//  * scales and minimums, per tile: one 2-byte load each by lane
//    row * GR + group, handed out with ds_bpermute.
// Measured on the fused matrix (same bits, fp16-weight form), all three and
// one tile ahead against the matrix-core layout two tiles ahead: M = 1 14.48
// -> 12.05 us, 16: 16.94 -> 13.22, 32: 20.97 -> 16.80; with three token
// tiles (activations, scales and minimums only) M = 34 22.09 -> 18.16, 48:
// 24.93 -> 19.76.  Two tiles ahead with the new patterns: 1 to 6% slower
// with one or two token tiles; with three the codes' pattern then spills
// (M = 34 26.1 us).  A twin of the loads alone (no arithmetic) gave the
// activations 3.8 against 7.4 us and the codes 10.2 against 12.0 us.
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
constexpr int kSplitStageWords = 16 * 17;  // 16-byte words of a wave's staging block

template <int TT, int GR, int NW, bool EPI>
__global__ void __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(NW / 4, NW / 4)))
prefill_split_kernel(const uint8_t* __restrict__ packed, const uint16_t* __restrict__ scales,
                     const uint16_t* __restrict__ mins, const uint16_t* __restrict__ X,
                     float* __restrict__ Y, int n, int k, int m) {
    extern __shared__ f4 lds_f4[];
    f4* part = lds_f4;                         // [2][NW][TT][64] partial sums per tile parity
    f4* tot = lds_f4 + 2 * NW * TT * 64;       // [kSplitMaxTiles][TT][64] totals of the slice
    constexpr int PER_ROUND = NW * GR;
    constexpr int W = 4 * GR;                  // words of a row in the wave's part of a tile
    constexpr bool kRowCodes = TT <= 2;        // codes requested in row order (3.6% slower at four tiles)

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    // The wave's staging block: 16 rows of up to 16 words, padded to 17.
    u4* stg = reinterpret_cast<u4*>(tot + kSplitMaxTiles * TT * 64) + wave * kSplitStageWords;
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

        // The tile in flight: codes (word gi*64 + lane of the tile's 16 x W
        // in row order, or chunk q of row r of group gi), and the scale and
        // minimum of (row lane / GR, group lane % GR).
        u4 wq[GR];
        uint16_t ws, wm;
        auto load_codes = [&](int gi, int rt) {
            int row, g, c;
            if constexpr (kRowCodes) {
                const int w = gi * 64 + lane;
                row = w / W;
                g = gw + (w % W) / 4;
                c = w & 3;
            } else {
                row = r;
                g = gw + gi;
                c = q;
            }
            row = row_lo + 16 * rt + row;
            row = row < row_hi ? row : row_hi - 1;
            g = g < G ? g : G - 1;
            wq[gi] = __builtin_nontemporal_load(
                reinterpret_cast<const u4*>(packed + (size_t)row * row_bytes) + g * 4 + c);
        };
        auto load_sm = [&](int rt) {
            const int l2 = lane < 16 * GR ? lane : 0;
            int row = row_lo + 16 * rt + l2 / GR;
            row = row < row_hi ? row : row_hi - 1;
            int g = gw + l2 % GR;
            g = g < G ? g : G - 1;
            ws = scales[(size_t)row * G + g];
            wm = mins[(size_t)row * G + g];
        };
        auto load_w = [&](int rt) {
#pragma unroll
            for (int gi = 0; gi < GR; ++gi) load_codes(gi, rt);
            load_sm(rt);
        };
        // With one or three token tiles the activations are requested before
        // the first tile's weights (loads complete in order, so staging them
        // then waits for them alone); with two, after (measured 1.0-2.5%
        // faster with the earlier patterns at M = 24 and 32).
        constexpr bool kActFirst = TT != 2;
        if constexpr (!kActFirst) load_w(0);

        // Activation fragments of this wave's groups: [group][k-step][token tile].
        // Requested as word s*64 + lane of the (group, token tile)'s 16 tokens
        // x 16 words, then moved to lane (r, q): words 4q + s of token r.
        u4 xa[GR][4][TT];
        // With three token tiles the token rows' offsets are computed here,
        // per round: an opaque zero keeps the compiler from hoisting them out
        // of the round loop (12 64-bit values held through every tile
        // otherwise).  This took the epilogue form from 256 registers and a
        // 24-byte spill to 254 and none (M = 33 to 48 1-5% faster, same
        // bits) and the fp16 form from 248 to 227 registers.  With one or two
        // tiles the hoisted offsets fit, and recomputing them measured 3-6%
        // slower on long rows (K = 11,008).
        int fresh = 0;
        if constexpr (TT == 3) asm volatile("v_mov_b32 %0, 0" : "=v"(fresh));
#pragma unroll
        for (int gi = 0; gi < GR; ++gi) {
            int g = gw + gi;
            g = g < G ? g : G - 1;
#pragma unroll
            for (int t = 0; t < TT; ++t)
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    const int w = s * 64 + lane;
                    int tok = 16 * t + (w >> 4) + fresh;
                    tok = tok < m ? tok : m - 1;
                    xa[gi][s][t] = reinterpret_cast<const u4*>(X + (size_t)tok * (size_t)k + (size_t)g * 128)[w & 15];
                }
        }
#pragma unroll
        for (int gi = 0; gi < GR; ++gi)
#pragma unroll
            for (int t = 0; t < TT; ++t) {
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    const int w = s * 64 + lane;
                    stg[(w >> 4) * 17 + (w & 15)] = xa[gi][s][t];
                }
#pragma unroll
                for (int s = 0; s < 4; ++s) xa[gi][s][t] = permute_window(stg[r * 17 + 4 * q + s]);
            }
        if constexpr (kActFirst) load_w(0);

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
            // Take the tile's codes (in row order: all, through the staging
            // block; otherwise each group's when it is used), scales and
            // minimums out of the registers, requesting the next tile's in
            // their place.
            if constexpr (kRowCodes) {
#pragma unroll
                for (int gi = 0; gi < GR; ++gi) {
                    const int w = gi * 64 + lane;
                    stg[(w / W) * (W + 1) + w % W] = wq[gi];
                    load_codes(gi, rt + 1);
                }
            }
            const uint32_t sm = (uint32_t)ws | ((uint32_t)wm << 16);
            load_sm(rt + 1);
            float bm = 0.0f;  // EPI: min of this lane's row for the wave's group q
#pragma unroll
            for (int gi = 0; gi < GR; ++gi) {
                const uint32_t keep = (uint32_t)__builtin_amdgcn_readfirstlane(-(int)(gw + gi < G));
                const uint32_t smg = (uint32_t)__builtin_amdgcn_ds_bpermute((r * GR + gi) * 4, (int)sm) & keep;
                const uint16_t sb = (uint16_t)smg;
                const uint16_t mb = (uint16_t)(smg >> 16);
                u4 cw;
                if constexpr (kRowCodes) {
                    cw = stg[r * (W + 1) + 4 * gi + q];
                } else {
                    cw = wq[gi];
                    load_codes(gi, rt + 1);
                }
                if constexpr (EPI) {
                    // Exact codes as fp16 denormals c * 2^-20 (each nibble moved
                    // to mantissa bits 4..7), in the pair order of dequant_dword.
                    const float sf = f16_bits_to_f32(sb) * kInvUnit;
                    bm = q == gi ? f16_bits_to_f32(mb) : bm;
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
                    weights_fp16(cw, sb, mb, kc, wv);
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
    const size_t lds = ((size_t)2 * NW * TT + (size_t)kSplitMaxTiles * TT) * 64 * sizeof(f4) +
                       (size_t)NW * kSplitStageWords * sizeof(u4);
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
    // Four token tiles: one group per wave and round (their activation
    // fragments take 64 registers; two groups measured 2-3% slower at
    // K = 3,072).  This replaced a kernel with one 16-row tile per wave for
    // 49 to 64 tokens (M = 49, same tolerance, another summation order):
    // fp16 weights 25,088 x 3,072 30.8 -> 26.8 us, 2,048 x 11,008 112.6 ->
    // 31.3, 8,192 x 2,048 24.1 -> 10.6; epilogue form 28.8 -> 30.3 (5%
    // slower), 92.0 -> 34.1, 21.4 -> 11.6.  Otherwise the fewest rounds at up
    // to three groups per wave, then the fewest groups per wave that cover K
    // in that many rounds.
    if constexpr (TT == 4) {
        return launch_split<4, 1, EPI>(a, X, Y, m, dev, st);
    } else {
        constexpr int kMaxGroupsPerWave = 3;
        const int G = a.k >> 7;
        const int rounds = (G + kSplitWaves * kMaxGroupsPerWave - 1) / (kSplitWaves * kMaxGroupsPerWave);
        const int gr = (G + kSplitWaves * rounds - 1) / (kSplitWaves * rounds);
        if (gr <= 1) return launch_split<TT, 1, EPI>(a, X, Y, m, dev, st);
        if (gr <= 2) return launch_split<TT, 2, EPI>(a, X, Y, m, dev, st);
        return launch_split<TT, 3, EPI>(a, X, Y, m, dev, st);
    }
}

template <bool EPI>
static hipError_t split_by_tokens(const GemvArgs& a, const uint16_t* X, float* Y, int m, const DeviceInfo& dev,
                                  hipStream_t st) {
    // At most four token tiles (the activation fragments of three groups of
    // 48 tokens take 144 of the 256 registers a wave has at two waves per
    // SIMD; with four tiles, one group per wave and round).
    const int tiles = (m + 15) / 16;
    if (tiles <= 1) return dispatch_split<1, EPI>(a, X, Y, m, dev, st);
    if (tiles <= 2) return dispatch_split<2, EPI>(a, X, Y, m, dev, st);
    if (tiles <= 3) return dispatch_split<3, EPI>(a, X, Y, m, dev, st);
    if (tiles <= 4) return dispatch_split<4, EPI>(a, X, Y, m, dev, st);
    return hipErrorInvalidValue;  // more than 64 tokens go to the other prefill kernels
}

// More than 64 tokens: the prompt in blocks of up to four token tiles, one
// launch each, the tiles spread evenly over the blocks (larger blocks
// first).  Every block reads the weights again (from L2 or the Infinity
// Cache on the matrices where this is chosen).
template <bool EPI>
static hipError_t split_token_blocks(const GemvArgs& a, const uint16_t* X, float* Y, int m, const DeviceInfo& dev,
                                     hipStream_t st) {
    const int tiles = (m + 15) / 16;
    const int blocks = (tiles + 3) / 4;
    int t0 = 0;
    for (int b = 0; b < blocks; ++b) {
        const int tb = tiles / blocks + (b < tiles % blocks ? 1 : 0);
        const int mb = 16 * tb < m - t0 ? 16 * tb : m - t0;
        const hipError_t e =
            split_by_tokens<EPI>(a, X + (size_t)t0 * (size_t)a.k, Y + (size_t)t0 * (size_t)a.n, mb, dev, st);
        if (e != hipSuccess) return e;
        t0 += mb;
    }
    return hipSuccess;
}

bool prefill_token_blocks_pay(long n, long m, const DeviceInfo& dev) {
    // The kernels for more than 64 tokens give each workgroup a slice of at
    // most 128 rows (or 256), so on few rows most CUs idle, while the split
    // kernel's grid has one workgroup per 16 rows.  Measured (one launch ->
    // blocks, fp16 weights / epilogue form): 2,048 x 11,008 at M = 65 80.8 ->
    // 43.4 / 127.4 -> 46.4 us, at 256 134.6 -> 131.4 / 183.4 -> 140.6;
    // 8,192 x 2,048 at 128 25.0 -> 22.3 / 28.7 -> 24.7, at 192 33.0 -> 33.2 /
    // 39.1 -> 36.8, at 256 30.3 -> 43.6 (slower); 16,384 x 3,072 at 65 37.3
    // -> 25.6 / 39.8 -> 25.8, at 128 37.5 -> 39.1 / 44.0 -> 43.0, at 192
    // 49.9 -> 58.1 (slower); 25,088 x 3,072 at 128 42.8 -> 55.4 (slower).
    // On many rows two blocks of at most three token tiles still beat one
    // launch (25,088 x 3,072, fp16 weights / epilogue form): at 65 38.2 /
    // 40.6 -> 34.2 / 33.6, at 81 40.0 / 42.7 -> 37.9 / 38.1, at 96 40.6 /
    // 43.7 -> 40.1 / 40.2; at 104 (four and three tiles) 41.5 / 44.3 -> 46.5
    // / 49.7.  So: up to 96 tokens, up to 256 tokens when the slices of 128
    // rows number at most 1/16 of the CUs, or up to 192 tokens when slices x
    // blocks is at most the number of CUs.
    const long cu = dev.num_cu > 0 ? dev.num_cu : 1;
    const long slices = (n + 127) / 128;
    const long blocks = ((m + 15) / 16 + 3) / 4;
    return m <= 96 || (m <= 256 && 16 * slices <= cu) || (m <= 192 && slices * blocks <= cu);
}

hipError_t launch_prefill_split(const GemvArgs& a, const uint16_t* X, float* Y, int m, const DeviceInfo& dev,
                                hipStream_t st) {
    if (m > 64) return split_token_blocks<false>(a, X, Y, m, dev, st);
    return split_by_tokens<false>(a, X, Y, m, dev, st);
}

hipError_t launch_prefill_split_epilogue(const GemvArgs& a, const uint16_t* X, float* Y, int m,
                                         const DeviceInfo& dev, hipStream_t st) {
    if (m > 64) return split_token_blocks<true>(a, X, Y, m, dev, st);
    return split_by_tokens<true>(a, X, Y, m, dev, st);
}

}  // namespace q4
