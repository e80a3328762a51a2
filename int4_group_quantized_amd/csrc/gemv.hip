// int4 group-128 GEMV and small-batch matmat kernels for gfx950.
//
// Work mapping (depends on K only, never on the batch size, so that every
// batched output column repeats the batch-1 arithmetic bit for bit):
//   C   = K / 32 chunks per row (a chunk = 16 packed bytes = 32 codes);
//   LPR = lanes per row: 32 if C = 64 (K = 2,048), else the largest of 64,
//         32, 16 dividing C; otherwise 64 if C > 64 ("ragged": the last
//         chunk column of a row is partial), else the largest of 8, 4
//         dividing C;
//   CPL = ceil(C / LPR) chunks per lane; lane j of a row owns chunks
//         j + t*LPR that are below C.  A ragged lane's missing chunk is
//         either skipped or fed zero activations, which leaves its sum
//         unchanged bit for bit (fma(s, +0, y) and fma(m, +0, y) return y
//         for any y other than -0, and a lane sum starting at +0 never
//         becomes -0), so every kernel computes the same bits.
// A wave therefore covers RPW = 64 / LPR rows per "pass"; one load
// instruction of a wave reads RPW contiguous segments of LPR * 16 bytes.
// Per lane and chunk: codes as exact fp16 denormals (chunk_codes), exact
// products with the activations accumulated in fp32 (chunk_dot), then
//   y += scale * dot + min * sum(x)   (group_update),
// all carried in units of 2^-20.  The LPR lane partials of a row are summed
// by a fixed butterfly and the row sum is rescaled by 2^20 (exact).
#include "q4_device.hpp"
#include "gemv_pass.hpp"
#include "launch.hpp"

namespace q4 {

// ---------------------------------------------------------------------------
// Batch-1 kernel: the activation slice of each lane lives in registers for
// the whole kernel (CPL <= 4), staged once per workgroup through LDS.
// Persistent grid: every wave walks passes p, p + W, p + 2W, ... (W = waves
// in the grid).  How many passes of weights a wave keeps in flight is the
// schedule D (kPassAhead2, the default: two, the next one requested after a
// pass is computed; kPassNextFirst: the next pass requested before the
// current one is computed, so one or two in flight).  In the default form
// the first passes are requested before the activations are staged (XF
// below is the other order).  Next-first keeps about half
// the bytes in flight at the start of a call; measured (back-to-back calls,
// same bits): 25,088 x 3,072 8.53 against 9.01 us, 3,072 x 8,192 5.53
// against 5.61, 25,088 x 2,048 6.56 against 6.68; ragged rows at
// K = 11,008 6.77 against 6.01 (kept at two).
//
// XF (x first): the workgroup stages x before any wave requests weights.
// In the default order a wave's first wait, for its x window, also waits for
// the weights it requested before (loads complete in order), and the barrier
// then holds the workgroup until its slowest wave's first pass has arrived.
// Measured (same bits; passes per wave in brackets), x first against the
// default order:
//   one workgroup per CU (K = 8,192; ragged K = 11,008), at every length:
//     3,072 x 8,192 [1.5] 4.85 / 5.56 us, 6,144 x 8,192 [3] 6.65 / 7.49,
//     2,048 x 11,008 [1] 5.13 / 6.02, 8,192 x 11,008 [4] 10.86 / 12.32;
//   two passes ahead (K = 4,096), up to three: 8,192 x 4,096 [2] 5.37 /
//     5.98, 12,288 x 4,096 [3] 6.63 / 7.10, 16,384 x 4,096 [4] 8.19 / 7.98;
//   next-first at two workgroups per CU, up to 1.5: 3,072 x 3,072 [1] 3.30
//     / 3.80, 12,288 x 3,072 [1.5] 5.68 / 5.96, 14,336 x 3,072 [1.75] 6.83 /
//     6.59, 25,088 x 3,072 [3.06] 9.05 / 8.56, 16,384 x 2,048 [2] 5.52 /
//     5.37.
// The host picks the form from the grid (launch_reg).
// ---------------------------------------------------------------------------

template <int LPR, int CPL, bool RAGGED, int D, bool XF>
__global__ void __launch_bounds__(kGemvThreads)
gemv_reg_kernel(const uint8_t* __restrict__ packed, const uint16_t* __restrict__ scales,
                const uint16_t* __restrict__ mins, const uint16_t* __restrict__ x,
                float* __restrict__ y, int n, int k) {
    constexpr int RPW = 64 / LPR;
    extern __shared__ u4 x_lds[];  // [4][C]: quad d of chunk c at d*C + c, permuted pairs
    const int C = k >> 5;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int j = lane % LPR;
    const int rsub = lane / LPR;
    const long passes = ((long)n + RPW - 1) / RPW;
    const long W = (long)gridDim.x * (blockDim.x >> 6);
    // Workgroups are dealt to the 8 XCDs round-robin (block b on XCD b % 8).
    // Renumber them so that consecutive numbers share an XCD: adjacent rows,
    // whose scale/min bytes share cache lines, then meet in one L2.  Passes
    // are numbered wave-major, so the last, partial round lands on one wave
    // of many workgroups rather than on a few workgroups.
    long p = (long)wave * gridDim.x + xcd_block_order(blockIdx.x, gridDim.x);
    auto row_of = [&](long pp) { return (int)(pp * RPW) + rsub; };
    auto clamp = [&](int r) { return r < n ? r : n - 1; };

    PassLoad<CPL> A, B;
    if constexpr (XF) {
        stage_x<LPR, CPL>(x, x_lds, k);
        __syncthreads();
    }
    if (p < passes) load_pass<LPR, CPL, RAGGED>(A, packed, scales, mins, clamp(row_of(p)), k, j);
    if (D == kPassAhead2 && p + W < passes)
        load_pass<LPR, CPL, RAGGED>(B, packed, scales, mins, clamp(row_of(p + W)), k, j);
    if constexpr (!XF) {
        stage_x<LPR, CPL>(x, x_lds, k);
        __syncthreads();
    }

    h2 xp[CPL][16];
    float xs[CPL];
    lane_activations<LPR, CPL, RAGGED>(x_lds, C, j, xp, xs);

    if constexpr (D == kPassNextFirst) {
        while (p < passes) {
            if (p + W < passes) load_pass<LPR, CPL, RAGGED>(B, packed, scales, mins, clamp(row_of(p + W)), k, j);
            compute_pass<LPR, CPL>(A, xp, xs, y, row_of(p), n, j);
            p += W;
            if (p >= passes) break;
            if (p + W < passes) load_pass<LPR, CPL, RAGGED>(A, packed, scales, mins, clamp(row_of(p + W)), k, j);
            compute_pass<LPR, CPL>(B, xp, xs, y, row_of(p), n, j);
            p += W;
        }
        return;
    }
    while (p < passes) {
        compute_pass<LPR, CPL>(A, xp, xs, y, row_of(p), n, j);
        if (p + 2 * W < passes)
            load_pass<LPR, CPL, RAGGED>(A, packed, scales, mins, clamp(row_of(p + 2 * W)), k, j);
        p += W;
        if (p >= passes) break;
        compute_pass<LPR, CPL>(B, xp, xs, y, row_of(p), n, j);
        if (p + 2 * W < passes)
            load_pass<LPR, CPL, RAGGED>(B, packed, scales, mins, clamp(row_of(p + 2 * W)), k, j);
        p += W;
    }
}

// ---------------------------------------------------------------------------
// Small-batch kernel with the batch-1 work mapping: the persistent pass walk
// of gemv_reg_kernel with one pass of weights in flight per wave, and BT
// activation columns staged in LDS (permuted windows and per-chunk sums).  For every
// column the per-lane arithmetic is compute_pass's, in the same order, and the
// same butterfly finishes each row, so column b equals the batch-1 result for
// X[b] bit for bit.  Columns b >= nb are zero and never stored.
//
// LDS layout, chunk c = j + t*LPR (lane j, slot t):
//   windows  xq  [t][b][quad d][j]  (16 bytes each)
//   sums     xsm [t][b][j]          (fp32)
// so a lane's reads for slot t are one base address plus compile-time offsets
// in (b, d), and the LPR lanes of a row read consecutive 16-byte words.
// ---------------------------------------------------------------------------

template <int LPR, int BT>
__device__ __forceinline__ int cols_win_index(int c, int b, int d) {
    return (((c / LPR) * BT + b) * 4 + d) * LPR + (c % LPR);
}

template <int LPR, int BT>
__device__ __forceinline__ int cols_sum_index(int c, int b) {
    return ((c / LPR) * BT + b) * LPR + (c % LPR);
}

// Lane sums through LDS for 32 lanes per row and 8 or more columns.  The
// butterfly of reduce_lanes costs each lane 5 vector adds (and one swizzle)
// per column, and every lane gets every sum.  Here the lanes instead write
// their partial sums to a per-wave LDS area, a round of CR columns at a time,
// and each of the 2 * CR outputs of the round (2 rows x CR columns) is summed
// by 32 / PPL lanes: PPL partials in registers, then DPP adds across those
// lanes.  The additions pair the same partial sums as reduce_lanes<32> does
// (lanes j and j^1, then j^2, j^4, j^8, j^16), and fp32 addition is
// commutative, so each sum has the same bits.
template <int LPR, int BT>
constexpr bool cols_lds_reduce() { return LPR == 32 && BT >= 8; }
constexpr int kColsRedFloats = 512;  // per wave: 2 rows x 8 columns x 32 lanes

template <int BT>
__device__ __forceinline__ void reduce_store_cols(const float (&y)[BT], float* red, float* __restrict__ Y,
                                                  int row0, int n, int lane, int nb) {
    constexpr int CR = BT % 8 == 0 ? 8 : 4;  // columns per round
    constexpr int LPO = 64 / (2 * CR);       // lanes per output
    constexpr int PPL = 32 / LPO;            // partial sums per lane
    const int j = lane & 31;
    const int rsub = lane >> 5;
    const int o = lane / LPO;                // output (row o / CR, column o % CR) of the round
    const int e = lane % LPO;                // its lanes: e = 0 .. LPO-1, partials j = PPL*e ..
    const float* src = red + (o * 32 + PPL * e);
#pragma unroll
    for (int r = 0; r < BT / CR; ++r) {
#pragma unroll
        for (int c = 0; c < CR; ++c) red[(rsub * CR + c) * 32 + j] = y[CR * r + c];
        const f4 a = *reinterpret_cast<const f4*>(src);
        float v = (a.x + a.y) + (a.z + a.w);                                    // j^1, j^2
        if constexpr (PPL == 8) {
            const f4 b = *reinterpret_cast<const f4*>(src + 4);
            v = v + ((b.x + b.y) + (b.z + b.w));                                // j^4
            v = v + dpp_move<0xB1>(v);                                          // j^8
            v = v + dpp_move<0x4E>(v);                                          // j^16
        } else {
            v = v + dpp_move<0xB1>(v);                                          // j^4
            v = v + dpp_move<0x4E>(v);                                          // j^8
            v = v + dpp_move<0x141>(v);                                         // j^16 (quads uniform)
        }
        const int col = CR * r + o % CR;
        const int row = row0 + o / CR;
        if (e == 0 && row < n && col < nb) Y[(size_t)col * (size_t)n + row] = v * kInvUnit;
    }
}

template <int LPR, int CPL, int BT>
__device__ __forceinline__ void compute_pass_cols(const PassLoad<CPL>& L, const u4* __restrict__ xq,
                                                  const float* __restrict__ xsm, float* red,
                                                  float* __restrict__ Y, int row, int n, int j, int lane,
                                                  int nb) {
    float y[BT];
#pragma unroll
    for (int b = 0; b < BT; ++b) y[b] = 0.0f;
    // One column's windows and chunk sum are read from LDS one column ahead of
    // their use; the scheduling barrier keeps the compiler from hoisting every
    // column's reads, which would exhaust the registers.
#pragma unroll
    for (int t = 0; t < CPL; ++t) {
        const u4* wt = xq + (size_t)t * BT * 4 * LPR + j;
        const float* st = xsm + (size_t)t * BT * LPR + j;
        h2 codes[16];
        chunk_codes(L.q[t], codes);
        u4 w[2][4];
        float xs[2];
        auto load_col = [&](int slot, int b) {
#pragma unroll
            for (int d = 0; d < 4; ++d) w[slot][d] = wt[(b * 4 + d) * LPR];
            xs[slot] = st[b * LPR];
        };
        load_col(0, 0);
#pragma unroll
        for (int b = 0; b < BT; ++b) {
            if (b + 1 < BT) load_col((b + 1) & 1, b + 1);
            h2 xp[16];
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                xp[4 * d + 0] = as_h2(w[b & 1][d].x);
                xp[4 * d + 1] = as_h2(w[b & 1][d].y);
                xp[4 * d + 2] = as_h2(w[b & 1][d].z);
                xp[4 * d + 3] = as_h2(w[b & 1][d].w);
            }
            y[b] = group_update(y[b], L.s[t], L.m[t], chunk_dot(codes, xp), xs[b & 1]);
            // Pin the column's result here: without it the compiler sinks the
            // dot chains below later columns and keeps every window live.
            asm volatile("" : "+v"(y[b]));
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    if constexpr (cols_lds_reduce<LPR, BT>()) {
        reduce_store_cols<BT>(y, red, Y, row - (lane >> 5), n, lane, nb);
        return;
    }
#pragma unroll
    for (int b = 0; b < BT; ++b) {
        const float v = reduce_lanes<LPR>(y[b]) * kInvUnit;
        if (j == 0 && row < n && b < nb) Y[(size_t)b * (size_t)n + row] = v;
    }
}

// Stage BT columns of X (zero past nb) in the layout above.
template <int LPR, int BT>
__device__ __forceinline__ void stage_columns(const uint16_t* __restrict__ X, u4* xq, float* xsm, int k, int nb) {
    const int C = k >> 5;
    const int wpc = k >> 3;  // windows per column
    for (int w = threadIdx.x; w < BT * wpc; w += blockDim.x) {
        const int b = w / wpc;
        const int win = w - b * wpc;
        u4 v = {0u, 0u, 0u, 0u};
        if (b < nb) v = reinterpret_cast<const u4*>(X + (size_t)b * (size_t)k)[win];
        xq[cols_win_index<LPR, BT>(win >> 2, b, win & 3)] = permute_window(v);
    }
    __syncthreads();
    for (int w = threadIdx.x; w < BT * C; w += blockDim.x) {
        const int b = w / C;
        const int c = w - b * C;
        h2 xp[16];
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            const u4 v = xq[cols_win_index<LPR, BT>(c, b, d)];
            xp[4 * d + 0] = as_h2(v.x);
            xp[4 * d + 1] = as_h2(v.y);
            xp[4 * d + 2] = as_h2(v.z);
            xp[4 * d + 3] = as_h2(v.w);
        }
        xsm[cols_sum_index<LPR, BT>(c, b)] = chunk_xsum(xp);
    }
    __syncthreads();
}

// 16 waves where the kernel fits in 128 registers (LPR <= 32, CPL <= 3): one
// workgroup holds the columns in LDS and four waves per SIMD hide the LDS
// latency of the column loop; 8 waves otherwise.
template <int LPR, int CPL>
constexpr int cols_threads() { return (LPR <= 32 && CPL <= 3) ? 1024 : 512; }

template <int LPR, int CPL, int BT, bool XF>
__global__ void __launch_bounds__((cols_threads<LPR, CPL>()))
gemm_cols_kernel(const uint8_t* __restrict__ packed, const uint16_t* __restrict__ scales,
                 const uint16_t* __restrict__ mins, const uint16_t* __restrict__ X,
                 float* __restrict__ Y, int n, int k, int nb) {
    constexpr int RPW = 64 / LPR;
    extern __shared__ u4 lds[];
    const int C = k >> 5;
    u4* xq = lds;                                                       // [CPL][BT][4][LPR]
    float* xsm = reinterpret_cast<float*>(lds + (size_t)BT * 4 * C);   // [CPL][BT][LPR]
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    float* red = xsm + (size_t)BT * C + (size_t)wave * kColsRedFloats;  // lane sums (LDS reduction only)
    const int j = lane % LPR;
    const int rsub = lane / LPR;
    const long passes = ((long)n + RPW - 1) / RPW;
    const long W = (long)gridDim.x * (blockDim.x >> 6);
    long p = (long)wave * gridDim.x + xcd_block_order(blockIdx.x, gridDim.x);
    auto row_of = [&](long pp) { return (int)(pp * RPW) + rsub; };
    auto clamp = [&](int r) { return r < n ? r : n - 1; };

    // One pass of weights in flight per wave: the next pass is requested after
    // the current one is computed.  Against two passes ahead this measured
    // 5-7% faster at B = 2 and 4, 1-3% at B = 8 to 16 (25,088 x 3,072 and
    // 25,088 x 2,048, same bits); the next pass requested before the current
    // one is computed measured 5-12% slower.  XF: the columns are staged
    // before the first pass is requested, chosen with one workgroup per CU
    // and at most 4 column slots.  Measured on two boxes (same bits), x first
    // against the default order: 25,088 x 3,072 at B = 2 2.5% and 4.8%
    // faster, B = 4 2.0% and 1.6%; 25,088 x 2,048 at B = 4 3.4% and 5.4%;
    // but at B = 8 and 16 from 4.9% faster to 4.4% slower, box by box.
    PassLoad<CPL> A;
    if constexpr (!XF) {
        if (p < passes) load_pass<LPR, CPL>(A, packed, scales, mins, clamp(row_of(p)), k, j);
    }
    stage_columns<LPR, BT>(X, xq, xsm, k, nb);
    if constexpr (XF) {
        if (p < passes) load_pass<LPR, CPL>(A, packed, scales, mins, clamp(row_of(p)), k, j);
    }

    while (p < passes) {
        compute_pass_cols<LPR, CPL, BT>(A, xq, xsm, red, Y, row_of(p), n, j, lane, nb);
        p += W;
        if (p < passes) load_pass<LPR, CPL>(A, packed, scales, mins, clamp(row_of(p)), k, j);
    }
}

// ---------------------------------------------------------------------------
// Batched kernel (also the batch-1 path when CPL > 4): BT activation columns
// staged in LDS in permuted order with their per-chunk sums; the chunk loop
// runs over t at run time.  Columns b >= nb are zero and never stored.
// ---------------------------------------------------------------------------

template <int LPR, int BT>
__global__ void __launch_bounds__(512)
gemm_batched_kernel(const uint8_t* __restrict__ packed, const uint16_t* __restrict__ scales,
                    const uint16_t* __restrict__ mins, const uint16_t* __restrict__ X,
                    float* __restrict__ Y, int n, int k, int nb, int ppw) {
    constexpr int RPW = 64 / LPR;
    extern __shared__ u4 lds[];
    const int C = k >> 5;
    const int G = k >> 7;
    u4* xq = lds;                                           // [BT][4][C]
    float* xsum = reinterpret_cast<float*>(lds + (size_t)BT * 4 * C);  // [BT][C]
    const int tid = threadIdx.x;

    const int wpc = k >> 3;  // windows per column
    for (int w = tid; w < BT * wpc; w += blockDim.x) {
        const int b = w / wpc;
        const int win = w - b * wpc;
        u4 v = {0u, 0u, 0u, 0u};
        if (b < nb) v = reinterpret_cast<const u4*>(X + (size_t)b * (size_t)k)[win];
        xq[((size_t)b * 4 + (win & 3)) * C + (win >> 2)] = permute_window(v);
    }
    __syncthreads();
    for (int w = tid; w < BT * C; w += blockDim.x) {
        const int b = w / C;
        const int c = w - b * C;
        h2 xp[16];
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            const u4 v = xq[((size_t)b * 4 + d) * C + c];
            xp[4 * d + 0] = as_h2(v.x);
            xp[4 * d + 1] = as_h2(v.y);
            xp[4 * d + 2] = as_h2(v.z);
            xp[4 * d + 3] = as_h2(v.w);
        }
        xsum[w] = chunk_xsum(xp);
    }
    __syncthreads();

    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int j = lane % LPR;
    const int rsub = lane / LPR;
    // Ragged rows: a lane's chunk past C loads the row's last chunk (in range)
    // and meets zero activations and a zero chunk sum, as in gemv_reg_kernel,
    // so that every lane applies the same group updates in the same order.
    const int CPL = (C + LPR - 1) / LPR;
    const long passes = ((long)n + RPW - 1) / RPW;
    const long p0 = ((long)blockIdx.x * (blockDim.x >> 6) + wave) * (long)ppw;

    for (int i = 0; i < ppw; ++i) {
        const long p = p0 + i;
        if (p >= passes) break;
        const int row = (int)(p * RPW) + rsub;
        const int rowc = row < n ? row : n - 1;
        const u4* rp = reinterpret_cast<const u4*>(packed + (size_t)rowc * (size_t)(k >> 1));
        const size_t gbase = (size_t)rowc * (size_t)G;
        float yl[BT];
#pragma unroll
        for (int b = 0; b < BT; ++b) yl[b] = 0.0f;
        for (int t = 0; t < CPL; ++t) {
            const int c0 = j + t * LPR;
            const bool valid = c0 < C;
            const int c = valid ? c0 : C - 1;
            const uint32_t keep = valid ? 0xFFFFFFFFu : 0u;
            const u4 q = __builtin_nontemporal_load(rp + c);
            const uint16_t s = scales[gbase + (c >> 2)];
            const uint16_t m = mins[gbase + (c >> 2)];
            h2 codes[16];
            chunk_codes(q, codes);
#pragma unroll
            for (int b = 0; b < BT; ++b) {
                h2 xp[16];
#pragma unroll
                for (int d = 0; d < 4; ++d) {
                    const u4 v = xq[((size_t)b * 4 + d) * C + c];
                    xp[4 * d + 0] = as_h2(v.x & keep);
                    xp[4 * d + 1] = as_h2(v.y & keep);
                    xp[4 * d + 2] = as_h2(v.z & keep);
                    xp[4 * d + 3] = as_h2(v.w & keep);
                }
                const float dot = chunk_dot(codes, xp);
                yl[b] = group_update(yl[b], s, m, dot, valid ? xsum[b * C + c] : 0.0f);
            }
        }
#pragma unroll
        for (int b = 0; b < BT; ++b) {
            const float v = reduce_lanes<LPR>(yl[b]) * kInvUnit;
            if (j == 0 && row < n && b < nb) Y[(size_t)b * (size_t)n + row] = v;
        }
    }
}

// ---------------------------------------------------------------------------
// Host-side launchers
// ---------------------------------------------------------------------------

int lanes_per_row(int k) {
    const int C = k >> 5;
    // K = 2,048: one chunk per lane at 64 lanes would spend a full-wave
    // butterfly per row (and per batch column) on 64 chunks; 32 lanes of two
    // chunks measured faster at every batch size.
    if (C == 64) return 32;
    if (C % 64 == 0) return 64;
    if (C % 32 == 0) return 32;
    if (C % 16 == 0) return 16;
    if (C > 64) return 64;  // ragged: 8 or 4 lanes per row would leave most CUs idle
    if (C % 8 == 0) return 8;
    return 4;  // C = 4 * (K / 128) is always a multiple of 4
}

// Resident workgroups per CU of one instantiation (registers bound it; the
// LDS footprint is at most 16 KB), queried once per device.
template <int LPR, int CPL, bool RAGGED, int D, bool XF>
static hipError_t reg_per_cu(const DeviceInfo& dev, int* per_cu) {
    std::atomic<int>& cached = PerDevice<&gemv_reg_kernel<LPR, CPL, RAGGED, D, XF>>::value[dev.device];
    int v = cached.load(std::memory_order_relaxed);
    if (v == 0) {
        int nb = 0;
        hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &nb, reinterpret_cast<const void*>(&gemv_reg_kernel<LPR, CPL, RAGGED, D, XF>), kGemvThreads, 8192 * 2);
        if (e != hipSuccess) return e;
        v = nb > 0 ? nb : 1;
        cached.store(v, std::memory_order_relaxed);
    }
    *per_cu = v;
    return hipSuccess;
}

template <int LPR, int CPL, bool RAGGED, int D = kPassAhead2>
static hipError_t launch_reg(const GemvArgs& a, const DeviceInfo& dev, hipStream_t st) {
    constexpr int RPW = 64 / LPR;
    constexpr int kThreads = kGemvThreads;
    constexpr int kWaves = kThreads / 64;
    const size_t lds = (size_t)a.k * 2;
    const long passes = ((long)a.n + RPW - 1) / RPW;
    const long need = (passes + kWaves - 1) / kWaves;
    // Both forms have the same register count, hence the same grid.
    int per_cu = 0;
    hipError_t e = reg_per_cu<LPR, CPL, RAGGED, D, false>(dev, &per_cu);
    if (e != hipSuccess) return e;
    long grid = (long)dev.num_cu * per_cu;
    if (grid > need) grid = need;
    // x first (measured per mapping; see the kernel): with one workgroup per
    // CU always, else up to 1.5 passes per wave, or 3 with two passes ahead.
    const long waves = grid * kWaves;
    const bool xf = per_cu == 1 || 2 * passes <= 3 * waves || (D == kPassAhead2 && passes <= 3 * waves);
    if (xf) {
        hipLaunchKernelGGL((gemv_reg_kernel<LPR, CPL, RAGGED, D, true>), dim3((unsigned)grid), dim3(kThreads), lds,
                           st, a.packed, a.scales, a.mins, a.x, a.y, a.n, a.k);
    } else {
        hipLaunchKernelGGL((gemv_reg_kernel<LPR, CPL, RAGGED, D, false>), dim3((unsigned)grid), dim3(kThreads), lds,
                           st, a.packed, a.scales, a.mins, a.x, a.y, a.n, a.k);
    }
    return hipGetLastError();
}

// Returns hipErrorNotSupported when (LPR, CPL) has no register-resident
// instantiation; the caller then uses the batched kernel with one column.
static hipError_t dispatch_reg(int lpr, int cpl, bool ragged, const GemvArgs& a, const DeviceInfo& dev,
                               hipStream_t st) {
#define Q4_REG(L, P) \
    if (!ragged && lpr == L && cpl == P) return launch_reg<L, P, false>(a, dev, st);
#define Q4_REG_R(L, P) \
    if (ragged && lpr == L && cpl == P) return launch_reg<L, P, true>(a, dev, st);
#define Q4_REG_NF(L, P) \
    if (!ragged && lpr == L && cpl == P) return launch_reg<L, P, false, pass_schedule(L, P, false)>(a, dev, st);
    Q4_REG(64, 1) Q4_REG(64, 2) Q4_REG(64, 3) Q4_REG_NF(64, 4)
    Q4_REG(32, 1) Q4_REG_NF(32, 2) Q4_REG_NF(32, 3)
    Q4_REG(16, 1) Q4_REG(16, 3)
    Q4_REG(8, 1) Q4_REG(8, 3)
    Q4_REG(4, 1) Q4_REG(4, 3)
    Q4_REG_R(64, 2) Q4_REG_R(64, 3) Q4_REG_R(64, 4) Q4_REG_R(64, 5) Q4_REG_R(64, 6)
#undef Q4_REG
#undef Q4_REG_NF
#undef Q4_REG_R
    return hipErrorNotSupported;
}

template <int LPR, int BT>
static hipError_t launch_batched(const GemvArgs& a, const uint16_t* X, float* Y, int nb,
                                 const DeviceInfo& dev, hipStream_t st) {
    constexpr int RPW = 64 / LPR;
    const int C = a.k >> 5;
    const size_t lds = (size_t)BT * 4 * C * 16 + (size_t)BT * C * 4;
    // The dynamic-LDS limit is a function attribute, set once per device.
    std::atomic<int>& attr_set = PerDevice<&gemm_batched_kernel<LPR, BT>>::value[dev.device];
    if (attr_set.load(std::memory_order_acquire) == 0) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&gemm_batched_kernel<LPR, BT>),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)dev.max_lds);
        if (e != hipSuccess) return e;
        attr_set.store(1, std::memory_order_release);
    }
    const long passes = ((long)a.n + RPW - 1) / RPW;
    const int waves = 8;
    const long per_cu = lds <= dev.max_lds / 2 ? 2 : 1;
    long grid = (long)dev.num_cu * per_cu;
    const long need = (passes + waves - 1) / waves;
    if (grid > need) grid = need;
    const long ppw = (passes + grid * waves - 1) / (grid * waves);
    grid = (passes + waves * ppw - 1) / (waves * ppw);
    hipLaunchKernelGGL((gemm_batched_kernel<LPR, BT>), dim3((unsigned)grid), dim3(64 * waves), lds, st,
                       a.packed, a.scales, a.mins, X, Y, a.n, a.k, nb, (int)ppw);
    return hipGetLastError();
}

template <int LPR>
static hipError_t dispatch_bt(int bt, const GemvArgs& a, const uint16_t* X, float* Y, int nb,
                              const DeviceInfo& dev, hipStream_t st) {
    switch (bt) {
        case 1: return launch_batched<LPR, 1>(a, X, Y, nb, dev, st);
        case 2: return launch_batched<LPR, 2>(a, X, Y, nb, dev, st);
        case 4: return launch_batched<LPR, 4>(a, X, Y, nb, dev, st);
        case 8: return launch_batched<LPR, 8>(a, X, Y, nb, dev, st);
        case 16: return launch_batched<LPR, 16>(a, X, Y, nb, dev, st);
    }
    return hipErrorInvalidValue;
}

static hipError_t dispatch_batched(int lpr, int bt, const GemvArgs& a, const uint16_t* X, float* Y,
                                   int nb, const DeviceInfo& dev, hipStream_t st) {
    switch (lpr) {
        case 64: return dispatch_bt<64>(bt, a, X, Y, nb, dev, st);
        case 32: return dispatch_bt<32>(bt, a, X, Y, nb, dev, st);
        case 16: return dispatch_bt<16>(bt, a, X, Y, nb, dev, st);
        case 8: return dispatch_bt<8>(bt, a, X, Y, nb, dev, st);
        case 4: return dispatch_bt<4>(bt, a, X, Y, nb, dev, st);
    }
    return hipErrorInvalidValue;
}

template <int LPR, int CPL, int BT>
static hipError_t launch_cols(const GemvArgs& a, const uint16_t* X, float* Y, int nb, const DeviceInfo& dev,
                              hipStream_t st) {
    constexpr int RPW = 64 / LPR;
    constexpr int kThreads = cols_threads<LPR, CPL>();
    const int C = a.k >> 5;
    const size_t red = cols_lds_reduce<LPR, BT>() ? (size_t)(kThreads / 64) * kColsRedFloats * 4 : 0;
    const size_t lds = (size_t)BT * 4 * C * 16 + (size_t)BT * C * 4 + red;
    if (lds > dev.max_lds) return hipErrorNotSupported;  // the caller falls back to the batched kernel
    // Once per device: the dynamic-LDS attribute of both forms, then the
    // occupancy (the same for both: same registers).
    std::atomic<int>& cached = PerDevice<&gemm_cols_kernel<LPR, CPL, BT, false>>::value[dev.device];
    int per_cu = cached.load(std::memory_order_acquire);
    if (per_cu == 0) {
        const void* fn = reinterpret_cast<const void*>(&gemm_cols_kernel<LPR, CPL, BT, false>);
        const void* fx = reinterpret_cast<const void*>(&gemm_cols_kernel<LPR, CPL, BT, true>);
        hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)dev.max_lds);
        if (e != hipSuccess) return e;
        e = hipFuncSetAttribute(fx, hipFuncAttributeMaxDynamicSharedMemorySize, (int)dev.max_lds);
        if (e != hipSuccess) return e;
        int nb_cu = 0;
        e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb_cu, fn, kThreads, lds);
        if (e != hipSuccess) return e;
        per_cu = nb_cu > 0 ? nb_cu : 1;
        cached.store(per_cu, std::memory_order_release);
    }
    const long passes = ((long)a.n + RPW - 1) / RPW;
    long grid = (long)dev.num_cu * per_cu;
    const long need = (passes + (kThreads / 64) - 1) / (kThreads / 64);
    if (grid > need) grid = need;
    if (per_cu == 1 && BT <= 4)
        hipLaunchKernelGGL((gemm_cols_kernel<LPR, CPL, BT, true>), dim3((unsigned)grid), dim3(kThreads), lds, st,
                           a.packed, a.scales, a.mins, X, Y, a.n, a.k, nb);
    else
        hipLaunchKernelGGL((gemm_cols_kernel<LPR, CPL, BT, false>), dim3((unsigned)grid), dim3(kThreads), lds, st,
                           a.packed, a.scales, a.mins, X, Y, a.n, a.k, nb);
    return hipGetLastError();
}

// Register-resident small-batch path for the (LPR, CPL) shapes that have one;
// hipErrorNotSupported sends the caller to the generic batched kernel.
static hipError_t dispatch_cols(int lpr, int cpl, int bt, const GemvArgs& a, const uint16_t* X, float* Y, int nb,
                                const DeviceInfo& dev, hipStream_t st) {
#define Q4_COLS(L, P)                                                          \
    if (lpr == L && cpl == P) {                                                \
        switch (bt) {                                                          \
            case 2: return launch_cols<L, P, 2>(a, X, Y, nb, dev, st);         \
            case 4: return launch_cols<L, P, 4>(a, X, Y, nb, dev, st);         \
            case 8: return launch_cols<L, P, 8>(a, X, Y, nb, dev, st);         \
            case 12: return launch_cols<L, P, 12>(a, X, Y, nb, dev, st);       \
            case 16: return launch_cols<L, P, 16>(a, X, Y, nb, dev, st);       \
        }                                                                      \
    }
    Q4_COLS(32, 3) Q4_COLS(32, 2) Q4_COLS(64, 4) Q4_COLS(16, 1) Q4_COLS(64, 1) Q4_COLS(64, 2)
#undef Q4_COLS
    return hipErrorNotSupported;
}

static int round_up_pow2_batch(int b) {
    int bt = 1;
    while (bt < b) bt <<= 1;
    return bt;
}

// Largest column count per launch whose staged activations fit in LDS.
static int max_cols_per_launch(int k, const DeviceInfo& dev) {
    const size_t per_col = (size_t)k * 2 + (size_t)(k >> 5) * 4;
    int cols = 16;
    while (cols > 1 && (size_t)cols * per_col > dev.max_lds) cols >>= 1;
    return cols;
}

hipError_t launch_gemv(const GemvArgs& a, const DeviceInfo& dev, hipStream_t st) {
    const int lpr = lanes_per_row(a.k);
    const int C = a.k >> 5;
    const int cpl = (C + lpr - 1) / lpr;
    hipError_t e = dispatch_reg(lpr, cpl, C % lpr != 0, a, dev, st);
    if (e != hipErrorNotSupported) return e;
    return dispatch_batched(lpr, 1, a, a.x, a.y, 1, dev, st);
}

hipError_t launch_small_batch(const GemvArgs& a, const uint16_t* X, float* Y, int b,
                              const DeviceInfo& dev, hipStream_t st) {
    if (b == 1) {
        GemvArgs one = a;
        one.x = X;
        one.y = Y;
        return launch_gemv(one, dev, st);
    }
    const int lpr = lanes_per_row(a.k);
    const int C = a.k >> 5;
    const bool ragged = C % lpr != 0;
    const int cap = max_cols_per_launch(a.k, dev);
    // The slot-by-slot kernel (gemv_seg.hip) when the columns do not all fit
    // in LDS (instead of one launch, and one weight read, per LDS-full), and
    // whenever its one-workgroup-per-CU grid covers every row in one round
    // (at most two passes per wave): measured faster there for every shape
    // tried but 3,072 x 8,192 at B = 2 (0.2 us).  Taller matrices keep the
    // column kernel (25,088 x 3,072 at B = 16: 39 against 55 us).
    const long passes = ((long)a.n * lpr + 63) / 64;
    const bool one_round = passes <= 16L * dev.num_cu;
    if (b > cap || one_round) {
        hipError_t e = launch_small_batch_segmented(a, X, Y, b, dev, st);
        if (e != hipErrorNotSupported) return e;
    }
    for (int b0 = 0; b0 < b; b0 += cap) {
        const int nb = (b - b0) < cap ? (b - b0) : cap;
        const int bt = round_up_pow2_batch(nb);
        // The column kernel also has a 12-column form (9 to 12 columns).
        const int bt_cols = nb > 8 && nb <= 12 && 12 <= cap ? 12 : bt;
        const uint16_t* Xc = X + (size_t)b0 * (size_t)a.k;
        float* Yc = Y + (size_t)b0 * (size_t)a.n;
        // The columns kernel has no ragged rows; those go to the batched kernel.
        hipError_t e = ragged ? hipErrorNotSupported : dispatch_cols(lpr, C / lpr, bt_cols, a, Xc, Yc, nb, dev, st);
        if (e == hipErrorNotSupported) e = dispatch_batched(lpr, bt, a, Xc, Yc, nb, dev, st);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace q4
