// Prompt processing for more than 192 tokens (the dense M-token contraction
// of the rumik-oss-1 write-up, "Step 8: a prefill that stays int4"; fp16
// weights as in prefill.hip):
//   Y[m][n] = sum_k fp16(code*scale + min)[n][k] * X[m][k],  fp32 accumulate.
//
// What bounds this shape is not the matrix cores but the activations: every
// workgroup that covers all of K for its rows reads all of its tokens' X
// from L2, and the L2 delivers about 10 TB/s to the CUs in aggregate.  So a
// workgroup takes a block of 128 tokens and twice the rows of the
// one-block-per-CU cut: the blocks of one row slice are placed on one XCD
// (workgroups are dealt to the 8 XCDs round-robin), where the second read
// of the slice's weights is served by the shared L2.
//
// Work split inside a workgroup of 8 waves (rows [row_lo, row_hi), at most
// 16 row tiles of 16; tokens [tb*128, tb*128 + 128)):
//  * wave w owns row tiles w and w + 8 (when they exist) for all 8 token
//    tiles of the block: 16 accumulator tiles, 64 VGPRs;
//  * it streams its tiles' packed codes, scales and mins four groups ahead
//    and dequantises one dword (8 weights) per tile and k-step in registers,
//    w = fma(code, scale, min) rounded once to fp16;
//  * the activations of one 128-column group sit in a double-buffered LDS
//    tile of matrix-instruction fragments, [token tile][k-step][lane], each
//    16 bytes in the pair order of dequant_dword; wave w stages token tile w
//    of the next group (loaded two groups ahead, permuted, written), so one
//    barrier per group hands the tile over;
//  * v_mfma_f32_16x16x32_f16 step s (0..3) contracts dword s of every lane's
//    chunk: B = the lane's 8 weights, A = the same 8 columns of token r of a
//    token tile.  One LDS read of an A fragment serves the wave's row tiles.
// Groups past K are zero weights against clamped activations; rows and
// tokens past the ends are clamped copies whose results are not stored.
// Output lane layout: lane l holds tokens 4*(l/16)+i of weight row l%16.
#include "q4_device.hpp"
#include "launch.hpp"

namespace q4 {

constexpr int kPairWaves = 8;
constexpr int kPairTokTiles = 8;              // token tiles per block (128 tokens)
constexpr int kPairMaxRowTiles = 2 * kPairWaves;  // 256 rows per workgroup
constexpr int kPairDW = 4;                    // weight groups in flight
constexpr int kPairDX = 2;                    // activation groups in flight

__global__ void __launch_bounds__(64 * kPairWaves) __attribute__((amdgpu_waves_per_eu(2, 2)))
prefill_pair_kernel(const uint8_t* __restrict__ packed, const uint16_t* __restrict__ scales,
                    const uint16_t* __restrict__ mins, const uint16_t* __restrict__ X,
                    float* __restrict__ Y, int n, int k, int m, int blocks) {
    constexpr int TB = kPairTokTiles, DW = kPairDW, DX = kPairDX;
    constexpr int U = 4;  // group loop unroll: a multiple of DW, DX and 2
    static_assert(U % DW == 0 && U % DX == 0 && U % 2 == 0, "ring depths");
    static_assert(TB == kPairWaves, "wave w stages token tile w");
    __shared__ u4 xs[2][TB][4][64];

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
    const bool two = wave + kPairWaves < RT;  // uniform: this wave has a second row tile

    const size_t row_bytes = (size_t)(k >> 1);
    const u4* cp[2];
    const uint16_t* sp[2];
    const uint16_t* mp[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        int row = row_lo + 16 * (wave + kPairWaves * j) + r;
        row = row < row_hi ? row : row_hi - 1;
        cp[j] = reinterpret_cast<const u4*>(packed + (size_t)row * row_bytes) + q;
        sp[j] = scales + (size_t)row * G;
        mp[j] = mins + (size_t)row * G;
    }
    int xt = tok0 + 16 * wave + r;  // the token this lane stages
    xt = xt < m ? xt : m - 1;
    const u4* xp = reinterpret_cast<const u4*>(X + (size_t)xt * (size_t)k) + 4 * q;
    const DequantConsts kc = make_dequant_consts();

    u4 wq[DW][2];
    uint16_t ws[DW][2], wm[DW][2];
    auto load_w = [&](int slot, int g) {
        const int gc = g < G ? g : G - 1;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            wq[slot][j] = __builtin_nontemporal_load(cp[j] + gc * 4);
            ws[slot][j] = sp[j][gc];
            wm[slot][j] = mp[j][gc];
        }
    };
    u4 xq[DX][4];
    auto load_x = [&](int slot, int g) {
        const int gc = g < G ? g : G - 1;
#pragma unroll
        for (int s = 0; s < 4; ++s) xq[slot][s] = xp[gc * 16 + s];
    };
    auto stage_x = [&](int slot, int buf) {
#pragma unroll
        for (int s = 0; s < 4; ++s) xs[buf][wave][s][lane] = permute_window(xq[slot][s]);
    };

#pragma unroll
    for (int d = 0; d < DW; ++d) load_w(d, d);
#pragma unroll
    for (int d = 0; d < DX; ++d) load_x(d, d);
    stage_x(0, 0);
    load_x(0, DX);
    lds_barrier();

    const f4 zero = {0.0f, 0.0f, 0.0f, 0.0f};
    f4 acc[2][TB];
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int t = 0; t < TB; ++t) acc[j][t] = zero;

    for (int g0 = 0; g0 < Gp; g0 += U) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int g = g0 + u;
            const int buf = u & 1;
            const int ws_slot = u % DW;
            const uint32_t keep = (uint32_t)__builtin_amdgcn_readfirstlane(-(int)(g < G));
            const _Float16 s0 = __builtin_bit_cast(_Float16, (uint16_t)(ws[ws_slot][0] & keep));
            const _Float16 m0 = __builtin_bit_cast(_Float16, (uint16_t)(wm[ws_slot][0] & keep));
            const _Float16 s1 = __builtin_bit_cast(_Float16, (uint16_t)(ws[ws_slot][1] & keep));
            const _Float16 m1 = __builtin_bit_cast(_Float16, (uint16_t)(wm[ws_slot][1] & keep));
            const h2 sv[2] = {{s0, s0}, {s1, s1}};
            const h2 mv[2] = {{m0, m0}, {m1, m1}};
            const u4 cq[2] = {wq[ws_slot][0], wq[ws_slot][1]};
            load_w(ws_slot, g + DW);
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                h8 a[TB];
#pragma unroll
                for (int t = 0; t < TB; ++t) a[t] = __builtin_bit_cast(h8, xs[buf][t][s][lane]);
#pragma unroll
                for (int j = 0; j < 2; ++j) {
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
            // the next group's activations: staged now, read after the barrier
            stage_x((u + 1) % DX, buf ^ 1);
            load_x((u + 1) % DX, g + 1 + DX);
            lds_barrier();
        }
    }

#pragma unroll
    for (int j = 0; j < 2; ++j) {
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

hipError_t launch_prefill_pair(const GemvArgs& a, const uint16_t* X, float* Y, int m, const DeviceInfo& dev,
                               hipStream_t st) {
    // Token blocks of 128; row slices in multiples of 8 (one set per XCD),
    // enough that every CU has a workgroup and no slice exceeds 256 rows.
    const long blocks = ((long)m + 16 * kPairTokTiles - 1) / (16 * kPairTokTiles);
    const long cu = dev.num_cu > 0 ? dev.num_cu : 1;
    long slices = (cu + blocks - 1) / blocks;
    const long need = ((long)a.n + 16 * kPairMaxRowTiles - 1) / (16 * kPairMaxRowTiles);
    if (slices < need) slices = need;
    slices = ((slices + 7) / 8) * 8;
    const long grid = slices * blocks;
    if (grid > 0x7FFFFFFFL) return hipErrorInvalidValue;
    hipLaunchKernelGGL(prefill_pair_kernel, dim3((unsigned)grid), dim3(64 * kPairWaves), 0, st, a.packed, a.scales,
                       a.mins, X, Y, a.n, a.k, m, (int)blocks);
    return hipGetLastError();
}

}  // namespace q4
