// Prompt-processing contraction on the gfx950 matrix cores:
//   Y[m][n] = sum_k fp16(code*scale + min)[n][k] * X[m][k],  fp32 accumulate.
// Four kernels: prefill_split_kernel (prefill_split.hip) for up to 48
// tokens, prefill_kernel for 49 to 64 tokens (below), prefill_wide_kernel
// for 65 to 192 (further down) and prefill_pair_kernel (prefill_pair.hip)
// above.
//
// prefill_kernel work split: one workgroup of 8 waves per CU-sized slice of rows.  The N
// rows are cut into gridDim.x contiguous ranges of at most 128 rows (the
// same number of rows, hence bytes, per workgroup up to one row); wave w
// owns the 16-row tile starting at row_lo + 16w (the last tile of a range
// may be partial, and waves past the range compute on clamped rows and
// store nothing).  Tokens are processed in blocks of 16*TT.
//
// Per 128-column group g (software pipelined):
//  * the activation tile X[block][g*128 .. +128] is requested into registers
//    three groups ahead and written to a double-buffered LDS tile as
//    permuted 8-element windows (pair order of dequant_dword), rows padded
//    by 16 bytes, then one barrier;
//  * each lane (r = lane & 15, q = lane >> 4) holds chunk q (16 bytes =
//    columns 32q .. 32q+31 of the group) of row r of its tile, requested six
//    groups ahead; the codes become exact fp16 values and then fp16 weights
//    with one rounding, w = fma(code, scale, min);
//  * v_mfma_f32_16x16x32_f16 step s (0..3) contracts dword s of every lane's
//    chunk: B operand = the lane's 8 weights, A operand = the same 8 columns
//    of token r of each token tile.  A and B hold the same column in the
//    same operand slot, so the hardware's numbering of k inside one
//    instruction does not matter.
// Output lane layout of the 16x16 instruction: lane l holds rows 4*(l/16)+i
// (tokens) of column l%16 (weight row).
#include "q4_device.hpp"
#include "launch.hpp"

namespace q4 {

constexpr int kPrefillWaves = 8;
constexpr int kPrefillRowsPerBlock = 16 * kPrefillWaves;

template <int TT>
__global__ void __launch_bounds__(64 * kPrefillWaves) __attribute__((amdgpu_waves_per_eu(2, 2)))
prefill_kernel(const uint8_t* __restrict__ packed, const uint16_t* __restrict__ scales,
               const uint16_t* __restrict__ mins, const uint16_t* __restrict__ X,
               float* __restrict__ Y, int n, int k, int m) {
    constexpr int TOK = 16 * TT;           // tokens per block
    constexpr int WIN = TOK * 16;          // 16-byte windows per staged group
    constexpr int THREADS = 64 * kPrefillWaves;
    constexpr int WPT = (WIN + THREADS - 1) / THREADS;  // windows per thread
    constexpr int DX = 3;                  // activation groups in flight
    constexpr int DW = 6;                  // weight groups in flight (multiple of DX and 2)
    static_assert(DW % DX == 0 && DW % 2 == 0, "ring depths");
    __shared__ u4 xt[2][TOK][17];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r = lane & 15;
    const int q = lane >> 4;
    const int G = k >> 7;
    const int row_lo = (int)((long)blockIdx.x * n / gridDim.x);
    const int row_hi = (int)((long)(blockIdx.x + 1) * n / gridDim.x);
    const int tile0 = row_lo + 16 * wave;
    const int row = tile0 + r;
    const bool store_row = row < row_hi;
    const int rowc = row < n ? row : n - 1;
    const u4* rp = reinterpret_cast<const u4*>(packed + (size_t)rowc * (size_t)(k >> 1));
    const uint16_t* srow = scales + (size_t)rowc * G;
    const uint16_t* mrow = mins + (size_t)rowc * G;
    const DequantConsts kc = make_dequant_consts();

    // Every global load below is issued unconditionally with clamped, in-range
    // addresses; out-of-range groups and tokens are zeroed where the data is
    // used.  A uniform stream of loads lets the compiler wait for exactly the
    // load it needs instead of draining the prefetch rings.
    const int Gp = ((G + DW - 1) / DW) * DW;  // group loop padded with zero-weight groups
    for (int tb = 0; tb < m; tb += TOK) {
        // Activation windows owned by this thread, DX groups ahead: X(j) in slot j % DX.
        u4 xr[DX][WPT];
        auto load_x = [&](u4 (&dst)[WPT], int g) {
            const int gc = g < G ? g : G - 1;
#pragma unroll
            for (int i = 0; i < WPT; ++i) {
                int w = tid + i * THREADS;
                w = w < WIN ? w : WIN - 1;
                int t = tb + (w >> 4);
                t = t < m ? t : m - 1;
                dst[i] = reinterpret_cast<const u4*>(X + (size_t)t * (size_t)k + (size_t)gc * 128)[w & 15];
            }
        };
        auto store_x = [&](const u4 (&src)[WPT], int buf, int g) {
#pragma unroll
            for (int i = 0; i < WPT; ++i) {
                const int w = tid + i * THREADS;
                if (w < WIN) {
                    const bool valid = g < G && tb + (w >> 4) < m;
                    const u4 zero = {0u, 0u, 0u, 0u};
                    xt[buf][w >> 4][w & 15] = valid ? permute_window(src[i]) : zero;
                }
            }
        };
        // Weight chunks of this lane, DW groups ahead: W(j) in slot j % DW.
        u4 wq[DW];
        uint16_t ws[DW], wm[DW];
        auto load_w = [&](int slot, int g) {
            const int gc = g < G ? g : G - 1;
            wq[slot] = __builtin_nontemporal_load(rp + gc * 4 + q);
            ws[slot] = srow[gc];
            wm[slot] = mrow[gc];
        };
#pragma unroll
        for (int d = 0; d < DW; ++d) load_w(d, d);
#pragma unroll
        for (int d = 0; d < DX; ++d) load_x(xr[d], d);
        store_x(xr[0], 0, 0);
        lds_barrier();

        f4 acc[TT];
#pragma unroll
        for (int t = 0; t < TT; ++t) acc[t] = (f4){0.0f, 0.0f, 0.0f, 0.0f};

        // The loop is unrolled by DW (a multiple of DX and of 2), so every ring
        // slot is a fixed register set and nothing is copied while in flight.
        for (int g0 = 0; g0 < Gp; g0 += DW) {
#pragma unroll
            for (int u = 0; u < DW; ++u) {
                const int g = g0 + u;
                const int buf = u & 1;
                const bool gv = g < G;  // padded groups contribute zero weights
                uint32_t wv[16];
                weights_fp16(wq[u], gv ? ws[u] : (uint16_t)0, gv ? wm[u] : (uint16_t)0, kc, wv);
                load_w(u, g + DW);
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    const u4 bw = {wv[4 * s + 0], wv[4 * s + 1], wv[4 * s + 2], wv[4 * s + 3]};
                    const h8 b = __builtin_bit_cast(h8, bw);
#pragma unroll
                    for (int t = 0; t < TT; ++t) {
                        const h8 a = __builtin_bit_cast(h8, xt[buf][t * 16 + r][4 * q + s]);
                        acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, acc[t], 0, 0, 0);
                    }
                }
                store_x(xr[(u + 1) % DX], buf ^ 1, g + 1);
                load_x(xr[u % DX], g + DX);
                lds_barrier();
            }
        }

        if (store_row) {
#pragma unroll
            for (int t = 0; t < TT; ++t) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int tok = tb + t * 16 + 4 * q + i;
                    if (tok < m) Y[(size_t)tok * (size_t)n + row] = acc[t][i];
                }
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Wide prompt-processing kernel (65 to 192 tokens).
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

template <int TT>
static hipError_t launch_tt(const GemvArgs& a, const uint16_t* X, float* Y, int m, const DeviceInfo& dev,
                            hipStream_t st) {
    // One workgroup per CU when the rows allow it; never more than 128 rows
    // (8 tiles) per workgroup, never fewer than one row.
    long grid = dev.num_cu > 0 ? dev.num_cu : 1;
    const long need = ((long)a.n + kPrefillRowsPerBlock - 1) / kPrefillRowsPerBlock;
    if (grid < need) grid = need;
    const long tiles = ((long)a.n + 15) / 16;
    if (grid > tiles) grid = tiles;
    hipLaunchKernelGGL((prefill_kernel<TT>), dim3((unsigned)grid), dim3(64 * kPrefillWaves), 0, st,
                       a.packed, a.scales, a.mins, X, Y, a.n, a.k, m);
    return hipGetLastError();
}

hipError_t launch_prefill(const GemvArgs& a, const uint16_t* X, float* Y, int m, const DeviceInfo& dev,
                          hipStream_t st) {
    // More than 192 tokens: blocks of 128 tokens, the blocks of a row slice on
    // one XCD (prefill_pair.hip).
    if (m > 192) return launch_prefill_pair(a, X, Y, m, dev, st);
    // 65 to 192 tokens: weights dequantised once per workgroup into LDS.
    if (m > 128) return launch_wide<3>(a, X, Y, m, dev, st);
    if (m > 64) return launch_wide<2>(a, X, Y, m, dev, st);
    // 49 to 64 tokens: every wave dequantises its own 16 rows for four token tiles.
    if (m > 48) return launch_tt<4>(a, X, Y, m, dev, st);
    // Up to 48 tokens: the waves of a workgroup split K, activations in registers
    // (prefill_split.hip).
    return launch_prefill_split(a, X, Y, m, dev, st);
}

}  // namespace q4
