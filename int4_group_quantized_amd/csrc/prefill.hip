// Prompt-processing contraction on the gfx950 matrix cores:
//   Y[m][n] = sum_k fp16(code*scale + min)[n][k] * X[m][k],  fp32 accumulate.
//
// Work split: one workgroup of 8 waves per CU-sized slice of rows.  The N
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

// Workgroup barrier for LDS hand-offs only.  It waits for this wave's LDS
// operations and does not drain outstanding global loads (unlike
// __syncthreads, whose fence would empty the prefetch rings).
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt and expcnt untouched
    __builtin_amdgcn_s_barrier();
}

// fp16 weights of one chunk (packed codes q, scale and minimum of its
// group), 16 pairs in the permuted pair order.
__device__ __forceinline__ void weights_fp16(const u4 q, uint16_t sb, uint16_t mb, const DequantConsts& kc,
                                             uint32_t wv[16]) {
    h2 codes[16];
    dequant_dword(q.x, kc, codes + 0);
    dequant_dword(q.y, kc, codes + 4);
    dequant_dword(q.z, kc, codes + 8);
    dequant_dword(q.w, kc, codes + 12);
    const _Float16 sh = __builtin_bit_cast(_Float16, sb);
    const _Float16 mh = __builtin_bit_cast(_Float16, mb);
    const h2 s2 = {sh, sh};
    const h2 m2 = {mh, mh};
#pragma unroll
    for (int i = 0; i < 16; ++i) wv[i] = as_u32(__builtin_elementwise_fma(codes[i], s2, m2));
}

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
    const int tiles = (m + 15) / 16;
    if (tiles <= 1) return launch_tt<1>(a, X, Y, m, dev, st);
    if (tiles <= 2) return launch_tt<2>(a, X, Y, m, dev, st);
    if (tiles <= 3) return launch_tt<3>(a, X, Y, m, dev, st);
    if (tiles <= 4) return launch_tt<4>(a, X, Y, m, dev, st);
    return launch_tt<8>(a, X, Y, m, dev, st);
}

}  // namespace q4
