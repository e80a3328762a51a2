// Prompt-processing contraction in the form of the rumik-oss-1 write-up
// ("Step 8: a prefill that stays int4"): the weights stay int4, each group
// of 128 columns is unpacked on chip and contracted on the matrix cores, and
// the group's scale and minimum are applied to the result:
//
//   Y[t][n] = sum_g  scale[n][g] * C_g[t][n]  +  min[n][g] * S_g[t],
//   C_g[t][n] = sum_{k in g} code[n][k] * X[t][k]   (matrix cores, fp32),
//   S_g[t]    = sum_{k in g} X[t][k]                (fp32).
//
// This is exactly sum_k (code*scale + min) * x regrouped; no weight is ever
// rounded to fp16, so the result keeps the accuracy of the matrix-vector
// kernels (every product code*x is exact; only fp32 sums round).
//
// This kernel serves 49 to 64 tokens; fewer go to prefill_split.hip and more
// to prefill_pair.hip, in the same form.
//
// Work mapping (as the fp16-weight kernel for up to 64 tokens): one
// workgroup of 8 waves per slice of at most 128 rows; wave w owns the 16-row
// tile starting at row_lo + 16w; tokens are processed in blocks of 16*TT
// (blocks of 64 re-stream the weights when M > 64).  Per group:
//  * lane (r = lane & 15, q = lane >> 4) holds chunk q (32 codes) of row r
//    and turns it into 16 exact integer fp16 code pairs (dequant_dword),
//    in the pair order (c0,c4) (c1,c5) (c2,c6) (c3,c7) of each dword;
//  * the group's activations sit in a double-buffered LDS tile as permuted
//    8-element windows (same pair order), and their per-token sums S_g in
//    an LDS ring of eight groups, both written one group ahead; one barrier
//    per group;
//  * v_mfma_f32_16x16x32_f16 step s (0..3) contracts dword s of every
//    lane's chunk; the first step of a group starts from a zero accumulator;
//  * then y = fma(scale, C_g, y) per output, fp32; every four groups the
//    minimum term, sum over the four of min_g * S_g, is one
//    v_mfma_f32_16x16x4_f32 per token tile (A = the tokens' sums S_g,
//    B = the row's minimums).
// Output lane layout of the 16x16 instruction: lane l holds rows 4*(l/16)+i
// (tokens) of column l%16 (weight row).
#include "q4_device.hpp"
#include "launch.hpp"

namespace q4 {

constexpr int kEpiWaves = 8;
constexpr int kEpiRowsPerBlock = 16 * kEpiWaves;

template <int TT>
__global__ void __launch_bounds__(64 * kEpiWaves) __attribute__((amdgpu_waves_per_eu(2, 2)))
prefill_epilogue_kernel(const uint8_t* __restrict__ packed, const uint16_t* __restrict__ scales,
                        const uint16_t* __restrict__ mins, const uint16_t* __restrict__ X,
                        float* __restrict__ Y, int n, int k, int m) {
    constexpr int TOK = 16 * TT;           // tokens per block
    constexpr int WIN = TOK * 16;          // 16-byte windows per staged group
    constexpr int THREADS = 64 * kEpiWaves;
    constexpr int WPT = (WIN + THREADS - 1) / THREADS;  // windows per thread
    // Groups in flight (weights, activations); shallower rings where the
    // per-group accumulators of 3 or 4 token tiles need the registers.
    constexpr int DX = TT <= 2 ? 3 : 2;
    constexpr int DW = TT <= 2 ? 6 : 4;    // a multiple of DX and of 2
    static_assert(DW % DX == 0 && DW % 2 == 0, "ring depths");
    static_assert(DW == 4, "the minimum term runs on windows of four groups");
    static_assert(THREADS % 16 == 0, "the 16 windows of a token are one DPP row");
    __shared__ u4 xt[2][TOK][17];
    __shared__ float xsr[8][TOK];          // S_g per token, groups g mod 8

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r = lane & 15;
    const int q = lane >> 4;
    const int G = k >> 7;
    const int row_lo = (int)((long)blockIdx.x * n / gridDim.x);
    const int row_hi = (int)((long)(blockIdx.x + 1) * n / gridDim.x);
    const int row = row_lo + 16 * wave + r;
    const bool store_row = row < row_hi;
    const int rowc = row < n ? row : n - 1;
    const u4* rp = reinterpret_cast<const u4*>(packed + (size_t)rowc * (size_t)(k >> 1));
    const uint16_t* srow = scales + (size_t)rowc * G;
    const uint16_t* mrow = mins + (size_t)rowc * G;
    const DequantConsts kc = make_dequant_consts();
    const h2 ones = {(_Float16)1.0f, (_Float16)1.0f};
    const f4 zero = {0.0f, 0.0f, 0.0f, 0.0f};

    // Every global load is issued unconditionally with clamped, in-range
    // addresses; groups past K and tokens past m are zeroed where used.
    const int Gp = ((G + DW - 1) / DW) * DW;  // group loop padded with zero groups
    for (int tb = 0; tb < m; tb += TOK) {
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
        // Windows and per-token sums of one group.  Masks rather than
        // selects keep the loads out of branches; all lanes run the row sum.
        auto store_x = [&](const u4 (&src)[WPT], int buf, int g) {
#pragma unroll
            for (int i = 0; i < WPT; ++i) {
                const int w = tid + i * THREADS;
                const uint32_t keep = -(uint32_t)(w < WIN && g < G && tb + (w >> 4) < m);
                const u4 p = permute_window(src[i]);
                const u4 v = {p.x & keep, p.y & keep, p.z & keep, p.w & keep};
                float part = __builtin_amdgcn_fdot2(as_h2(v.x), ones, 0.0f, false);
                part = __builtin_amdgcn_fdot2(as_h2(v.y), ones, part, false);
                part = __builtin_amdgcn_fdot2(as_h2(v.z), ones, part, false);
                part = __builtin_amdgcn_fdot2(as_h2(v.w), ones, part, false);
                const float tot = reduce_lanes<16>(part);  // every lane of the DPP row gets the token's sum
                if (w < WIN) {
                    xt[buf][w >> 4][w & 15] = v;
                    if ((w & 15) == 0) xsr[g & 7][w >> 4] = tot;
                }
            }
        };
        u4 wq[DW];
        uint16_t ws[DW];
        auto load_w = [&](int slot, int g) {
            const int gc = g < G ? g : G - 1;
            wq[slot] = __builtin_nontemporal_load(rp + gc * 4 + q);
            ws[slot] = srow[gc];
        };
#pragma unroll
        for (int d = 0; d < DW; ++d) load_w(d, d);
#pragma unroll
        for (int d = 0; d < DX; ++d) load_x(xr[d], d);
        store_x(xr[0], 0, 0);
        lds_barrier();

        f4 y[TT];
#pragma unroll
        for (int t = 0; t < TT; ++t) y[t] = zero;

        for (int g0 = 0; g0 < Gp; g0 += DW) {
            // This window's minimums, min[row][g0 + q] for lane (r, q) (zero
            // past G), requested four groups before use.
            const int gq = g0 + q;
            const float mwin = f16_bits_to_f32((uint16_t)(mrow[gq < G ? gq : G - 1] & (uint32_t)(-(int)(gq < G))));
#pragma unroll
            for (int u = 0; u < DW; ++u) {
                const int g = g0 + u;
                const int buf = u & 1;
                // padded groups: zero scale and minimum (their activations are zero too)
                const uint32_t keep = (uint32_t)__builtin_amdgcn_readfirstlane(-(int)(g < G));
                const float sf = f16_bits_to_f32((uint16_t)(ws[u] & keep));
                h2 codes[16];
                dequant_dword(wq[u].x, kc, codes + 0);
                dequant_dword(wq[u].y, kc, codes + 4);
                dequant_dword(wq[u].z, kc, codes + 8);
                dequant_dword(wq[u].w, kc, codes + 12);
                load_w(u, g + DW);
                f4 acc[TT];
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    const h8 b = {codes[4 * s].x, codes[4 * s].y, codes[4 * s + 1].x, codes[4 * s + 1].y,
                                  codes[4 * s + 2].x, codes[4 * s + 2].y, codes[4 * s + 3].x, codes[4 * s + 3].y};
#pragma unroll
                    for (int t = 0; t < TT; ++t) {
                        const h8 a = __builtin_bit_cast(h8, xt[buf][t * 16 + r][4 * q + s]);
                        acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, s == 0 ? zero : acc[t], 0, 0, 0);
                    }
                }
#pragma unroll
                for (int t = 0; t < TT; ++t)
#pragma unroll
                    for (int i = 0; i < 4; ++i) y[t][i] = __builtin_fmaf(sf, acc[t][i], y[t][i]);
                store_x(xr[(u + 1) % DX], buf ^ 1, g + 1);
                load_x(xr[u % DX], g + DX);
                lds_barrier();
            }
            // The minimum term of the window on the matrix cores:
            // y[tok][row] += sum over q of S_(g0+q)[tok] * min[row][g0+q].
#pragma unroll
            for (int t = 0; t < TT; ++t)
                y[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(xsr[(g0 + q) & 7][t * 16 + r], mwin, y[t], 0, 0, 0);
        }

        if (store_row) {
#pragma unroll
            for (int t = 0; t < TT; ++t) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int tok = tb + t * 16 + 4 * q + i;
                    if (tok < m) Y[(size_t)tok * (size_t)n + row] = y[t][i];
                }
            }
        }
    }
}

template <int TT>
static hipError_t launch_epi(const GemvArgs& a, const uint16_t* X, float* Y, int m, const DeviceInfo& dev,
                             hipStream_t st) {
    // One workgroup per CU when the rows allow it; never more than 128 rows
    // (8 tiles) per workgroup, never fewer than one row.
    long grid = dev.num_cu > 0 ? dev.num_cu : 1;
    const long need = ((long)a.n + kEpiRowsPerBlock - 1) / kEpiRowsPerBlock;
    if (grid < need) grid = need;
    const long tiles = ((long)a.n + 15) / 16;
    if (grid > tiles) grid = tiles;
    hipLaunchKernelGGL((prefill_epilogue_kernel<TT>), dim3((unsigned)grid), dim3(64 * kEpiWaves), 0, st,
                       a.packed, a.scales, a.mins, X, Y, a.n, a.k, m);
    return hipGetLastError();
}

hipError_t launch_prefill_epilogue(const GemvArgs& a, const uint16_t* X, float* Y, int m, const DeviceInfo& dev,
                                   hipStream_t st) {
    // Up to 48 tokens: the waves of a workgroup split K (prefill_split.hip).
    if (m <= 48) return launch_prefill_split_epilogue(a, X, Y, m, dev, st);
    // More than 64: blocks of 128 tokens per workgroup, the blocks of a row
    // slice on one XCD (prefill_pair.hip).
    if (m > 64) return launch_prefill_pair_epilogue(a, X, Y, m, dev, st);
    // 49 to 64 tokens: four token tiles per wave (below).
    return launch_epi<4>(a, X, Y, m, dev, st);
}

}  // namespace q4
