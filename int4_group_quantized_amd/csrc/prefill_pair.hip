// Prompt processing for many tokens (the dense M-token contraction of the
// rumik-oss-1 write-up, "Step 8: a prefill that stays int4"), in both forms
// of the library (above 192 tokens for fp16 weights, above 64 for EPI):
//   fp16 weights (as prefill.hip):
//     Y[m][n] = sum_k fp16(code*scale + min)[n][k] * X[m][k],  fp32 accumulate;
//   EPI, scale and minimum on the result (as prefill_epilogue.hip):
//     Y[m][n] = sum_g scale[n][g] * C_g[m][n] + min[n][g] * S_g[m].
//
// What bounds this shape is not the matrix cores but the activations: every
// workgroup that covers all of K for its rows reads all of its tokens' X
// from L2 (about 10 TB/s in aggregate measured with loads in the matrix-core
// operand layout).  So a
// workgroup takes a block of 128 tokens and twice the rows of the
// one-block-per-CU cut: the blocks of one row slice are placed on one XCD
// (workgroups are dealt to the 8 XCDs round-robin), where the second read
// of the slice's weights is served by the shared L2.
//
// Work split inside a workgroup of 8 waves (rows [row_lo, row_hi), at most
// 16 row tiles of 16, 8 in the EPI form; tokens [tb*128, tb*128 + 128)):
//  * wave w owns row tiles w and w + 8 (EPI: row tile w) for all 8 token
//    tiles of the block: 16 accumulator tiles, 64 VGPRs;
//  * it streams its tiles' packed codes, scales and mins a window of four
//    groups ahead (RC, below) or four groups ahead in the operand layout,
//    and dequantises one dword (8 weights) per tile and k-step in registers,
//    w = fma(code, scale, min) rounded once to fp16;
//  * the activations of one 128-column group sit in a double-buffered LDS
//    tile of matrix-instruction fragments, [token tile][k-step][lane], each
//    16 bytes in the pair order of dequant_dword; wave w stages token tile w
//    of the next group (loaded two groups ahead, permuted, written), so one
//    barrier per group hands the tile over.  Row-order loads (kRowAct):
//    load s, lane L requests word L & 15 of token 4s + L / 16, and the
//    fragment slots are XOR-swizzled within a k-step so that both those
//    writes and the lanes' reads are free of bank conflicts.  Measured on
//    the fused matrix (same bits): fp16 weights M = 128 45.1 -> 40.9 us,
//    256 60.7 -> 58.7, 512 118.5 -> 113.3; the epilogue form with two row
//    tiles per wave 2-3% faster, with one (M = 65 to 128) up to 5% slower,
//    so that one keeps the matrix-core layout;
//  * v_mfma_f32_16x16x32_f16 step s (0..3) contracts dword s of every lane's
//    chunk: B = the lane's 8 weights, A = the same 8 columns of token r of a
//    token tile.  One LDS read of an A fragment serves the wave's row tiles.
// EPI: B = the 8 exact codes as fp16 denormals c * 2^-20; each group's four
// k-steps start from zero (two token tiles at a time) and are followed by
// y += (scale * 2^20) * C_g in fp32.  The minimum term, sum over g of
// min_g * S_g, is a product of rank G: every four groups it goes to the matrix
// cores as one v_mfma_f32_16x16x4_f32 per tile (A = the tokens' group sums
// S_g, summed by the wave that stages the token and kept in an LDS ring of
// eight groups; B = the rows' minimums), accumulated into the same tile.
// Groups past K are zero weights against clamped activations; rows and
// tokens past the ends are clamped copies whose results are not stored.
// Output lane layout: lane l holds tokens 4*(l/16)+i of weight row l%16.
#include "q4_device.hpp"
#include "launch.hpp"

namespace q4 {

constexpr int kPairWaves = 8;
constexpr int kPairTokTiles = 8;  // token tiles per block (128 tokens)
constexpr int kPairDW = 4;        // weight groups in flight
constexpr int kPairDX = 2;        // activation groups in flight

// RW row tiles per wave (16 * 8 * RW rows per workgroup).  Two when a row
// slice has several token blocks: one LDS read of an activation fragment then
// serves two row tiles.  With a single block (up to 128 tokens) one, so that
// every CU has a slice; a wave without a second tile in range still computes
// it on clamped rows (results not stored), which costs nothing when another
// wave of its SIMD has two (the busiest SIMD sets the time) and is
// cheaper than a branch inside the group loop (measured: the epilogue form
// then spills).
template <bool EPI, int RW, bool RC>
__global__ void __launch_bounds__(64 * kPairWaves) __attribute__((amdgpu_waves_per_eu(2, 2)))
prefill_pair_kernel(const uint8_t* __restrict__ packed, const uint16_t* __restrict__ scales,
                    const uint16_t* __restrict__ mins, const uint16_t* __restrict__ X,
                    float* __restrict__ Y, int n, int k, int m, int blocks) {
    constexpr int TB = kPairTokTiles, DW = kPairDW, DX = kPairDX;
    constexpr int U = 4;  // group loop unroll: a multiple of DW, DX and 2
    static_assert(U % DW == 0 && U % DX == 0 && U % 2 == 0, "ring depths");
    static_assert(TB == kPairWaves, "wave w stages token tile w");
    static_assert(RW == 1 || RW == 2, "row tiles per wave");
    __shared__ u4 xs[2][TB][4][64];
    constexpr bool kRowAct = !EPI || RW == 2;
    // RC: each wave's codes of a window of U groups requested in row order
    // (16 rows x 16 words per row tile, four rows x 256 B per load) and moved
    // to the operand layout through this staging block (rows padded to 17
    // words); the window's scales and minimums one 2-byte load each per row
    // tile, by lane row * U + group, handed out with ds_bpermute.  The next
    // window is requested when a window starts.  Measured against the
    // operand layout four groups ahead (same bits, fused matrix): fp16
    // weights M = 193 59.0 -> 53.1 us, 256 59.0 -> 54.6, 512 113.1 -> 109.7;
    // epilogue form with one row tile per wave (65 to 128 tokens) 1-6%
    // faster, with two 1-4% slower (M = 256 1.1% faster), so that one keeps
    // the operand layout.
    __shared__ u4 cstage[RC ? kPairWaves * RW * 16 * 17 : 1];
    __shared__ float xsum[8][TB][16];  // EPI: S_g of every token of the block, groups g mod 8

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r = lane & 15;
    const int q = lane >> 4;
    const int G = k >> 7;
    const int Gp = ((G + U - 1) / U) * U;

    // Workgroup -> (row slice, token block): the `blocks` token blocks of a
    // slice are consecutive workgroups of one XCD.
    const int xcd = blockIdx.x & 7;
    const int within = blockIdx.x >> 3;
    const int slices = (int)gridDim.x / blocks;
    const int slice = (within / blocks) * 8 + xcd;
    const int tb = within % blocks;
    const int row_lo = (int)((long)slice * n / slices);
    const int row_hi = (int)((long)(slice + 1) * n / slices);
    const int RT = (row_hi - row_lo + 15) >> 4;
    const int tok0 = tb * 16 * TB;
    if (RT == 0 || tok0 >= m) return;  // uniform: an empty slice or block
    const bool two = RW == 2 && wave + kPairWaves < RT;  // uniform: this wave has a second row tile

    const size_t row_bytes = (size_t)(k >> 1);
    const u4* cp[RW];
    const uint16_t* sp[RW];
    const uint16_t* mp[RW];
#pragma unroll
    for (int j = 0; j < RW; ++j) {
        int row = row_lo + 16 * (wave + kPairWaves * j) + r;
        row = row < row_hi ? row : row_hi - 1;
        cp[j] = reinterpret_cast<const u4*>(packed + (size_t)row * row_bytes) + q;
        sp[j] = scales + (size_t)row * G;
        mp[j] = mins + (size_t)row * G;
    }
    // The words this lane requests for its wave's token tile: in row order,
    // word L & 15 of token 4s + L / 16 per load s; otherwise words 4q .. 4q+3
    // of token r.
    const u4* xp[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        int xt = tok0 + 16 * wave + (kRowAct ? 4 * s + (lane >> 4) : r);
        xt = xt < m ? xt : m - 1;
        xp[s] = reinterpret_cast<const u4*>(X + (size_t)xt * (size_t)k) + (kRowAct ? (lane & 15) : 4 * q + s);
    }
    // Fragment slot of lane l = r + 16q at k-step s (kRowAct): r XOR (4q + s).
    auto slot_of = [](int l, int s) { return kRowAct ? (l & 48) | ((l & 15) ^ ((4 * (l >> 4) + s) & 15)) : l; };
    const DequantConsts kc = make_dequant_consts();

    u4* cst = cstage + (RC ? wave * RW * 16 * 17 : 0);
    u4 wr[RW][4];          // RC: the next window's codes, word 64 i + lane of a row tile's 16 x 16
    uint16_t wsr[RW], wmr[RW];  // RC: the next window's scale and minimum of (row lane / U, group lane % U)
    auto load_window = [&](int g0) {
#pragma unroll
        for (int j = 0; j < RW; ++j) {
            const int rb = row_lo + 16 * (wave + kPairWaves * j);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int w = 64 * i + lane;
                int row = rb + (w >> 4);
                row = row < row_hi ? row : row_hi - 1;
                int g = g0 + ((w & 15) >> 2);
                g = g < G ? g : G - 1;
                wr[j][i] = __builtin_nontemporal_load(reinterpret_cast<const u4*>(packed + (size_t)row * row_bytes) +
                                                      g * 4 + (w & 3));
            }
            const int l2 = lane < 16 * U ? lane : 0;
            int row = rb + l2 / U;
            row = row < row_hi ? row : row_hi - 1;
            int g = g0 + l2 % U;
            g = g < G ? g : G - 1;
            wsr[j] = scales[(size_t)row * G + g];
            wmr[j] = mins[(size_t)row * G + g];
        }
    };

    u4 wq[DW][RW];
    uint16_t ws[DW][RW], wm[DW][RW];
    auto load_w = [&](int slot, int g) {
        const int gc = g < G ? g : G - 1;
#pragma unroll
        for (int j = 0; j < RW; ++j) {
            wq[slot][j] = __builtin_nontemporal_load(cp[j] + gc * 4);
            ws[slot][j] = sp[j][gc];
            wm[slot][j] = mp[j][gc];
        }
    };
    u4 xq[DX][4];
    auto load_x = [&](int slot, int g) {
        const int gc = g < G ? g : G - 1;
#pragma unroll
        for (int s = 0; s < 4; ++s) xq[slot][s] = xp[s][gc * 16];
    };
    auto stage_x = [&](int slot, int buf, int sg) {
        float v = 0.0f;
        const h2 ones = {(_Float16)1.0f, (_Float16)1.0f};
        if constexpr (kRowAct) {
            // word c = lane & 15 of token 4s + lane / 16 is k-step c & 3 of
            // lane (token) + 16 (c >> 2)
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const int c = lane & 15;
                xs[buf][wave][c & 3][slot_of(4 * s + (lane >> 4) + 16 * (c >> 2), c & 3)] =
                    permute_window(xq[slot][s]);
            }
        }
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            // the lane's own fragment (read back from LDS in row order)
            const u4 w = kRowAct ? xs[buf][wave][s][slot_of(lane, s)] : permute_window(xq[slot][s]);
            if constexpr (!kRowAct) xs[buf][wave][s][lane] = w;
            if constexpr (EPI) {
                v = __builtin_amdgcn_fdot2(as_h2(w.x), ones, v, false);
                v = __builtin_amdgcn_fdot2(as_h2(w.y), ones, v, false);
                v = __builtin_amdgcn_fdot2(as_h2(w.z), ones, v, false);
                v = __builtin_amdgcn_fdot2(as_h2(w.w), ones, v, false);
            }
        }
        if constexpr (EPI) {
            // the token's four k-slots are lanes r, r + 16, r + 32, r + 48
            v = v + lane_swap16(v);
            v = v + __shfl_xor(v, 32, 64);
            xsum[sg][wave][r] = v;  // the four lanes of the token write the same value
        }
    };

    if constexpr (RC) {
        load_window(0);
    } else {
#pragma unroll
        for (int d = 0; d < DW; ++d) load_w(d, d);
    }
#pragma unroll
    for (int d = 0; d < DX; ++d) load_x(d, d);
    stage_x(0, 0, 0);
    load_x(0, DX);
    lds_barrier();

    const f4 zero = {0.0f, 0.0f, 0.0f, 0.0f};
    f4 acc[RW][TB];
#pragma unroll
    for (int j = 0; j < RW; ++j)
#pragma unroll
        for (int t = 0; t < TB; ++t) acc[j][t] = zero;

    for (int g0 = 0; g0 < Gp; g0 += U) {
        uint32_t smw[RW];
        if constexpr (RC) {
            // this window's codes into the staging block, its scales and
            // minimums packed; then the next window requested in their place
#pragma unroll
            for (int j = 0; j < RW; ++j) {
#pragma unroll
                for (int i = 0; i < 4; ++i) cst[j * 272 + (4 * i + (lane >> 4)) * 17 + (lane & 15)] = wr[j][i];
                smw[j] = (uint32_t)wsr[j] | ((uint32_t)wmr[j] << 16);
            }
            load_window(g0 + U);
        }
        // EPI: this window's minimums, min[row][g0 + q] for lane (r, q) and
        // each row tile (zero past G), requested four groups before use.
        float mwin[RW];
        if constexpr (EPI && RC) {
            const uint32_t live = (uint32_t)(-(int)(g0 + q < G));
#pragma unroll
            for (int j = 0; j < RW; ++j) {
                const uint32_t v = (uint32_t)__builtin_amdgcn_ds_bpermute((r * U + q) * 4, (int)smw[j]);
                mwin[j] = (float)__builtin_bit_cast(_Float16, (uint16_t)((v >> 16) & live));
            }
        } else if constexpr (EPI) {
            const int gq = g0 + q;
            const uint32_t live = (uint32_t)(-(int)(gq < G));
#pragma unroll
            for (int j = 0; j < RW; ++j)
                mwin[j] = (float)__builtin_bit_cast(_Float16, (uint16_t)(mp[j][gq < G ? gq : G - 1] & live));
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int g = g0 + u;
            const int buf = u & 1;
            const int slot = u % DW;
            const uint32_t keep = (uint32_t)__builtin_amdgcn_readfirstlane(-(int)(g < G));
            u4 cq[RW];
            h2 sv[RW], mv[RW];
            float sf[RW];
#pragma unroll
            for (int j = 0; j < RW; ++j) {
                uint16_t sb, mb;
                if constexpr (RC) {
                    cq[j] = cst[j * 272 + r * 17 + 4 * u + q];
                    const uint32_t v = (uint32_t)__builtin_amdgcn_ds_bpermute((r * U + u) * 4, (int)smw[j]) & keep;
                    sb = (uint16_t)v;
                    mb = (uint16_t)(v >> 16);
                } else {
                    cq[j] = wq[slot][j];
                    sb = (uint16_t)(ws[slot][j] & keep);
                    mb = (uint16_t)(wm[slot][j] & keep);
                }
                const _Float16 sh = __builtin_bit_cast(_Float16, sb);
                const _Float16 mh = __builtin_bit_cast(_Float16, mb);
                sv[j] = (h2){sh, sh};
                mv[j] = (h2){mh, mh};
                sf[j] = (float)sh * kInvUnit;  // EPI: codes enter as c * 2^-20
            }
            if constexpr (!RC) load_w(slot, g + DW);
            if constexpr (EPI) {
                // Exact codes as fp16 denormals c * 2^-20 (pair order of
                // dequant_dword), then per pair of token tiles: the group's
                // four k-steps from a zero accumulator for each row tile and
                // y += scale * C_g + min * S_g for the tokens 4q + i.
                h8 b[RW][4];
#pragma unroll
                for (int j = 0; j < RW; ++j)
#pragma unroll
                    for (int s = 0; s < 4; ++s) {
                        const uint32_t dw = s == 0 ? cq[j].x : s == 1 ? cq[j].y : s == 2 ? cq[j].z : cq[j].w;
                        const u4 bw = {(dw << 4) & 0x00F000F0u, dw & 0x00F000F0u, (dw >> 4) & 0x00F000F0u,
                                       (dw >> 8) & 0x00F000F0u};
                        b[j][s] = __builtin_bit_cast(h8, bw);
                    }
#pragma unroll
                for (int t = 0; t < TB; t += 2) {
                    f4 c[RW][2];
#pragma unroll
                    for (int s = 0; s < 4; ++s) {
                        const h8 a0 = __builtin_bit_cast(h8, xs[buf][t][s][slot_of(lane, s)]);
                        const h8 a1 = __builtin_bit_cast(h8, xs[buf][t + 1][s][slot_of(lane, s)]);
#pragma unroll
                        for (int j = 0; j < RW; ++j) {
                            c[j][0] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a0, b[j][s], s == 0 ? zero : c[j][0],
                                                                             0, 0, 0);
                            c[j][1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a1, b[j][s], s == 0 ? zero : c[j][1],
                                                                             0, 0, 0);
                        }
                    }
#pragma unroll
                    for (int j = 0; j < RW; ++j)
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            acc[j][t][i] = __builtin_fmaf(sf[j], c[j][0][i], acc[j][t][i]);
                            acc[j][t + 1][i] = __builtin_fmaf(sf[j], c[j][1][i], acc[j][t + 1][i]);
                        }
                }
            } else {
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    h8 a[TB];
#pragma unroll
                    for (int t = 0; t < TB; ++t) a[t] = __builtin_bit_cast(h8, xs[buf][t][s][slot_of(lane, s)]);
#pragma unroll
                    for (int j = 0; j < RW; ++j) {
                        if (j == 1 && !two) break;
                        const uint32_t dw = s == 0 ? cq[j].x : s == 1 ? cq[j].y : s == 2 ? cq[j].z : cq[j].w;
                        h2 c[4];
                        dequant_dword(dw, kc, c);
                        const u4 bw = {as_u32(__builtin_elementwise_fma(c[0], sv[j], mv[j])),
                                       as_u32(__builtin_elementwise_fma(c[1], sv[j], mv[j])),
                                       as_u32(__builtin_elementwise_fma(c[2], sv[j], mv[j])),
                                       as_u32(__builtin_elementwise_fma(c[3], sv[j], mv[j]))};
                        const h8 b = __builtin_bit_cast(h8, bw);
#pragma unroll
                        for (int t = 0; t < TB; ++t)
                            acc[j][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[t], b, acc[j][t], 0, 0, 0);
                    }
                }
            }
            // the next group's activations: staged now, read after the barrier
            stage_x((u + 1) % DX, buf ^ 1, (g + 1) & 7);
            load_x((u + 1) % DX, g + 1 + DX);
            lds_barrier();
        }
        if constexpr (EPI) {
            // The minimum term of the window's four groups on the matrix
            // cores: y[tok][row] += sum over q of S_(g0+q)[tok] * min[row][g0+q],
            // A = the tokens' group sums (token r, group q), B = the rows'
            // minimums (group q, row r), fp32 operands.
#pragma unroll
            for (int t = 0; t < TB; ++t) {
                const float a = xsum[(g0 + q) & 7][t][r];
#pragma unroll
                for (int j = 0; j < RW; ++j)
                    acc[j][t] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, mwin[j], acc[j][t], 0, 0, 0);
            }
        }
    }

#pragma unroll
    for (int j = 0; j < RW; ++j) {
        const int row = row_lo + 16 * (wave + kPairWaves * j) + r;
        if (row < row_hi) {
#pragma unroll
            for (int t = 0; t < TB; ++t)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int tok = tok0 + 16 * t + 4 * q + i;
                    if (tok < m) Y[(size_t)tok * (size_t)n + row] = acc[j][t][i];
                }
        }
    }
}

template <bool EPI, int RW, bool RC>
static hipError_t launch_pair(const GemvArgs& a, const uint16_t* X, float* Y, int m, long blocks,
                              const DeviceInfo& dev, hipStream_t st) {
    // Row slices in multiples of 8 (one set per XCD): as many as give every
    // CU at most one workgroup, unless a slice would then exceed the rows of
    // its waves' tiles.  Rounding up instead left a few workgroups for a
    // second wave whenever the CU count is not a multiple of 8 x blocks
    // (3, 5, 6 or 7 blocks), which doubled the call.
    const long rows_max = 16L * kPairWaves * RW;
    const long cu = dev.num_cu > 0 ? dev.num_cu : 1;
    const long need = ((long)a.n + rows_max - 1) / rows_max;
    long slices = (cu / blocks) / 8 * 8;
    if (slices < need) slices = ((need + 7) / 8) * 8;
    if (slices < 8) slices = 8;
    const long grid = slices * blocks;
    if (grid > 0x7FFFFFFFL) return hipErrorInvalidValue;
    hipLaunchKernelGGL((prefill_pair_kernel<EPI, RW, RC>), dim3((unsigned)grid), dim3(64 * kPairWaves), 0, st,
                       a.packed, a.scales, a.mins, X, Y, a.n, a.k, m, (int)blocks);
    return hipGetLastError();
}

template <bool EPI>
static hipError_t launch_pair_blocks(const GemvArgs& a, const uint16_t* X, float* Y, int m, const DeviceInfo& dev,
                                     hipStream_t st) {
    const long blocks = ((long)m + 16 * kPairTokTiles - 1) / (16 * kPairTokTiles);  // of 128 tokens
    // Codes in row order (RC) everywhere but the epilogue form with two row
    // tiles per wave, where it measured 1-4% slower (same bits).
    if (blocks == 1) return launch_pair<EPI, 1, true>(a, X, Y, m, blocks, dev, st);
    return launch_pair<EPI, 2, !EPI>(a, X, Y, m, blocks, dev, st);
}

long prefill_pair_head_tokens(long n, long m, const DeviceInfo& dev) {
    // With two row tiles per wave a slice holds at most 256 rows; on many
    // rows the slices, in multiples of 8, leave room for `fit` blocks of 128
    // tokens in one wave of workgroups (one per CU).  One block more puts
    // most of a second wave behind them: on 25,088 rows 300 tokens took
    // 105.6 us against 57.5 for 256.  Then the first fit * 128 tokens run as
    // one launch and the rest (at most 128 tokens) on their own.
    const long cu = dev.num_cu > 0 ? dev.num_cu : 1;
    const long rows_max = 16L * kPairWaves * 2;
    const long slices = ((n + rows_max - 1) / rows_max + 7) / 8 * 8;
    const long fit = cu / slices;
    const long blocks = (m + 16 * kPairTokTiles - 1) / (16 * kPairTokTiles);
    return fit >= 2 && blocks == fit + 1 ? fit * 16 * kPairTokTiles : 0;
}

hipError_t launch_prefill_pair(const GemvArgs& a, const uint16_t* X, float* Y, int m, const DeviceInfo& dev,
                               hipStream_t st) {
    return launch_pair_blocks<false>(a, X, Y, m, dev, st);
}

hipError_t launch_prefill_pair_epilogue(const GemvArgs& a, const uint16_t* X, float* Y, int m,
                                        const DeviceInfo& dev, hipStream_t st) {
    return launch_pair_blocks<true>(a, X, Y, m, dev, st);
}

}  // namespace q4
