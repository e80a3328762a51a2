// Prompt-processing contraction on the gfx950 matrix cores:
//   Y[m][n] = sum_k fp16(code*scale + min)[n][k] * X[m][k],  fp32 accumulate.
// Three kernels: prefill_split_kernel (prefill_split.hip) for up to 64
// tokens (and in blocks of up to 64 for up to 96 tokens, or more on matrices
// of few rows), prefill_wide_kernel for the rest up to 192 (below) and
// prefill_pair_kernel (prefill_pair.hip) above.
//
// In every kernel v_mfma_f32_16x16x32_f16 step s (0..3) contracts dword s of
// every lane's 32-code chunk: B operand = the lane's 8 weights, A operand =
// the same 8 columns of token r of each token tile.  A and B hold the same
// column in the same operand slot, so the hardware's numbering of k inside
// one instruction does not matter.  Output lane layout of the 16x16
// instruction: lane l holds rows 4*(l/16)+i (tokens) of column l%16 (weight
// row).
#include "q4_device.hpp"
#include "launch.hpp"

namespace q4 {

// ---------------------------------------------------------------------------
// Wide prompt-processing kernel (97 to 192 tokens on matrices of many rows).
//
// Workgroup of 8 waves on a slice of at most 128 rows (8 row tiles) and a
// block of 64*TM tokens:
//  * waves 4..7 ("helpers") stream the slice's packed codes, scales and mins
//    from HBM in bursts of BG groups (each lane one 16-byte chunk of one row
//    per group) and write each group once to LDS as fp16 weights,
//    w = fma(code, scale, min) rounded once, in natural column order and in
//    the operand layout of the matrix instruction: [row tile][k-step][lane];
//  * waves 0..3 own TM token tiles each and read every row tile's weight
//    fragment from LDS (one read serves TM instructions); their activation
//    fragments come straight from global memory (L2), DA k-steps ahead.
// A helper wave issues only HBM loads and an MFMA wave only activation loads:
// vector loads of one wave complete in order, so mixing the two would make
// every activation wait for the weight stream.  One barrier per group hands
// the double-buffered weight tile over.  Groups past K (the loop runs in
// trips of 2*BG groups) have zero weights and zero activations.
// ---------------------------------------------------------------------------

constexpr int kWideRowTiles = 8;  // 128 rows per workgroup
constexpr int kWideDA = 2;        // activation k-steps in flight
constexpr int kWideBG = 4;        // groups per helper load burst

template <int TM>
__global__ void __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
prefill_wide_kernel(const uint8_t* __restrict__ packed, const uint16_t* __restrict__ scales,
                    const uint16_t* __restrict__ mins, const uint16_t* __restrict__ X,
                    float* __restrict__ Y, int n, int k, int m) {
    constexpr int TN = kWideRowTiles, DA = kWideDA, BG = kWideBG;
    __shared__ u4 wl[2][TN][4][64];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int G = k >> 7;
    const int Gp = ((G + 2 * BG - 1) / (2 * BG)) * (2 * BG);
    const int row_lo = (int)((long)blockIdx.x * n / gridDim.x);
    const int row_hi = (int)((long)(blockIdx.x + 1) * n / gridDim.x);

    if (wave >= 4) {
        // ---------------------------------------------------------- helpers
        const int hw = wave - 4, ht = tid - 256;
        const int r16 = ht & 15, sq = (ht >> 4) & 3;  // row within a tile, 16-byte chunk of the group
        const DequantConsts kc = make_dequant_consts();
        const u4* cp[2];
        const uint16_t* sp[2];
        const uint16_t* mp[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            int r = row_lo + 16 * (hw + 4 * h) + r16;
            r = r < row_hi ? r : row_hi - 1;
            cp[h] = reinterpret_cast<const u4*>(packed + (size_t)r * (size_t)(k >> 1)) + sq;
            sp[h] = scales + (size_t)r * G;
            mp[h] = mins + (size_t)r * G;
        }
        u4 cq[2][BG][2];
        uint16_t cs[2][BG][2], cm[2][BG][2];
        auto load_burst = [&](int slot, int b) {
#pragma unroll
            for (int j = 0; j < BG; ++j) {
                int g = b * BG + j;
                g = g < G ? g : G - 1;
#pragma unroll
                for (int h = 0; h < 2; ++h) cq[slot][j][h] = __builtin_nontemporal_load(cp[h] + g * 4);
            }
#pragma unroll
            for (int j = 0; j < BG; ++j) {
                int g = b * BG + j;
                g = g < G ? g : G - 1;
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    cs[slot][j][h] = sp[h][g];
                    cm[slot][j][h] = mp[h][g];
                }
            }
        };
        auto dequant = [&](int slot, int j, int buf, int g) {
            const uint32_t keep = (uint32_t)__builtin_amdgcn_readfirstlane(-(int)(g < G));
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                uint32_t wv[16];
                weights_fp16(cq[slot][j][h], (uint16_t)(cs[slot][j][h] & keep), (uint16_t)(cm[slot][j][h] & keep),
                             kc, wv);
#pragma unroll
                for (int d = 0; d < 4; ++d) {
                    // pairs (w0,w4) (w1,w5) (w2,w6) (w3,w7) -> (w0,w1) (w2,w3) (w4,w5) (w6,w7)
                    const uint32_t p0 = wv[4 * d], p1 = wv[4 * d + 1], p2 = wv[4 * d + 2], p3 = wv[4 * d + 3];
                    wl[buf][hw + 4 * h][sq][r16 + 16 * d] =
                        (u4){__builtin_amdgcn_perm(p1, p0, 0x05040100u), __builtin_amdgcn_perm(p3, p2, 0x05040100u),
                             __builtin_amdgcn_perm(p1, p0, 0x07060302u), __builtin_amdgcn_perm(p3, p2, 0x07060302u)};
                }
            }
        };
        for (int tb = 0; tb < m; tb += 64 * TM) {
            load_burst(0, 0);
            load_burst(1, 1);
            dequant(0, 0, 0, 0);
            lds_barrier();
            for (int g0 = 0; g0 < Gp; g0 += 2 * BG) {
#pragma unroll
                for (int u = 0; u < 2 * BG; ++u) {
                    const int un = u + 1;  // group g0 + un is written while group g0 + u is consumed
                    dequant((un / BG) & 1, un % BG, un & 1, g0 + un);
                    if (u % BG == BG - 1) load_burst((u / BG) & 1, (g0 + u + 1) / BG + 1);
                    lds_barrier();
                }
            }
        }
        return;
    }

    // -------------------------------------------------------------- MFMA waves
    for (int tb = 0; tb < m; tb += 64 * TM) {
        const uint16_t* xr[TM];
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            int t = tb + 16 * (wave * TM + i) + (lane & 15);
            t = t < m ? t : m - 1;
            xr[i] = X + (size_t)t * (size_t)k + 8 * (lane >> 4);
        }
        // activation window of k-step kk (32 columns; lane holds 8 of them) in slot kk % DA
        u4 ar[DA][TM];
        auto load_a = [&](int kk) {
            const int gc = (kk >> 2) < G ? (kk >> 2) : G - 1;
#pragma unroll
            for (int i = 0; i < TM; ++i)
                ar[kk % DA][i] = *reinterpret_cast<const u4*>(xr[i] + gc * 128 + 32 * (kk & 3));
        };
        u4 bf[2][TN];
        auto load_b = [&](int slot, int buf, int s) {
#pragma unroll
            for (int r = 0; r < TN; ++r) bf[slot][r] = wl[buf][r][s][lane];
        };
#pragma unroll
        for (int d = 0; d < DA; ++d) load_a(d);
        lds_barrier();
        load_b(0, 0, 0);
        f4 acc[TM][TN];
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int r = 0; r < TN; ++r) acc[i][r] = (f4){0.0f, 0.0f, 0.0f, 0.0f};
        for (int g0 = 0; g0 < Gp; g0 += 2 * BG) {
#pragma unroll
            for (int u = 0; u < 2 * BG; ++u) {
                const int g = g0 + u;
                const uint32_t gmask = (uint32_t)__builtin_amdgcn_readfirstlane(-(int)(g < G));
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    if (s == 3) lds_barrier();  // group g+1 is in LDS; group g-1's buffer is free
                    if (s < 3) load_b((s + 1) & 1, u & 1, s + 1);
                    else load_b(0, (u + 1) & 1, 0);
                    h8 a[TM];
#pragma unroll
                    for (int i = 0; i < TM; ++i) a[i] = __builtin_bit_cast(h8, ar[(4 * u + s) % DA][i] & gmask);
                    load_a(4 * g + s + DA);
#pragma unroll
                    for (int r = 0; r < TN; ++r) {
                        const h8 b = __builtin_bit_cast(h8, bf[s & 1][r]);
#pragma unroll
                        for (int i = 0; i < TM; ++i)
                            acc[i][r] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[i], b, acc[i][r], 0, 0, 0);
                    }
                    // keep each k-step's activation use after its loads were issued two steps earlier
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
        }
        // lane l holds tokens 4*(l/16)+e of a token tile, row l%16 of a row tile
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int r = 0; r < TN; ++r) {
                const int row = row_lo + 16 * r + (lane & 15);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int tok = tb + 16 * (wave * TM + i) + 4 * (lane >> 4) + e;
                    if (tok < m && row < row_hi) Y[(size_t)tok * n + row] = acc[i][r][e];
                }
            }
    }
}

template <int TM>
static hipError_t launch_wide(const GemvArgs& a, const uint16_t* X, float* Y, int m, const DeviceInfo& dev,
                              hipStream_t st) {
    // One workgroup per CU when the rows allow it; at most 128 rows per workgroup.
    long grid = dev.num_cu > 0 ? dev.num_cu : 1;
    const long need = ((long)a.n + 16 * kWideRowTiles - 1) / (16 * kWideRowTiles);
    if (grid < need) grid = need;
    const long tiles = ((long)a.n + 15) / 16;
    if (grid > tiles) grid = tiles;
    hipLaunchKernelGGL((prefill_wide_kernel<TM>), dim3((unsigned)grid), dim3(512), 0, st, a.packed, a.scales,
                       a.mins, X, Y, a.n, a.k, m);
    return hipGetLastError();
}

hipError_t launch_prefill(const GemvArgs& a, const uint16_t* X, float* Y, int m, const DeviceInfo& dev,
                          hipStream_t st) {
    // Up to 96 tokens, and more on matrices of few rows: the waves of a
    // workgroup split K, activations in registers (prefill_split.hip; above
    // 64 tokens in blocks of up to 64).
    if (m <= 64 || prefill_token_blocks_pay(a.n, m, dev)) return launch_prefill_split(a, X, Y, m, dev, st);
    // More than 192 tokens: blocks of 128 tokens, the blocks of a row slice on
    // one XCD (prefill_pair.hip); on many rows one block past a full wave of
    // workgroups runs on its own, after the others.
    if (m > 192) {
        const long head = prefill_pair_head_tokens(a.n, m, dev);
        if (head > 0) {
            const hipError_t e = launch_prefill_pair(a, X, Y, (int)head, dev, st);
            if (e != hipSuccess) return e;
            return launch_prefill(a, X + head * (long)a.k, Y + head * (long)a.n, m - (int)head, dev, st);
        }
        return launch_prefill_pair(a, X, Y, m, dev, st);
    }
    // 97 to 192 tokens: weights dequantised once per workgroup into LDS.
    if (m > 128) return launch_wide<3>(a, X, Y, m, dev, st);
    return launch_wide<2>(a, X, Y, m, dev, st);
}

}  // namespace q4
