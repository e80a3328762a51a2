// Prompt-processing contraction on the gfx950 matrix cores:
//   Y[m][n] = sum_k fp16(code*scale + min)[n][k] * X[m][k],  fp32 accumulate.
//
// Workgroup = 4 waves; its tile is 64 weight rows (16 per wave) by 16*TM
// tokens (a one-dimensional grid, row tiles fastest).  The K loop walks the 128-column groups.  Per group:
//  * the activation tile [16*TM tokens][128] is staged in LDS as permuted
//    8-element windows (pair order of dequant_dword), rows padded by 16 bytes;
//  * lane (r = lane & 15, q = lane >> 4) loads chunk q (16 bytes = columns
//    32q .. 32q+31 of the group) of its weight row, turns the codes into
//    exact fp16 values and then into fp16 weights with one rounding,
//    w = fma(code, scale, min);
//  * v_mfma_f32_16x16x32_f16 step s (0..3) contracts dword s of every
//    lane's chunk: B operand = the lane's 8 weights, A operand = the same 8
//    columns of token r of each token tile.  A and B hold the same column in
//    the same operand slot, so the hardware's numbering of k inside one
//    instruction does not matter.
// Output lane layout of the 16x16 instruction: lane l holds rows 4*(l/16)+i
// (tokens) of column l%16 (weight row).
#include "q4_device.hpp"
#include "launch.hpp"

namespace q4 {

template <int TM>
__global__ void __launch_bounds__(256)
prefill_kernel(const uint8_t* __restrict__ packed, const uint16_t* __restrict__ scales,
               const uint16_t* __restrict__ mins, const uint16_t* __restrict__ X,
               float* __restrict__ Y, int n, int k, int m, int row_tiles) {
    __shared__ u4 xt[16 * TM][17];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int r = lane & 15;
    const int q = lane >> 4;
    const int G = k >> 7;
    const int tok_tile = (int)(blockIdx.x / (unsigned)row_tiles);
    const int row_tile = (int)(blockIdx.x - (unsigned)tok_tile * (unsigned)row_tiles);
    const int row = row_tile * 64 + wave * 16 + r;
    const int rowc = row < n ? row : n - 1;
    const int tok0 = tok_tile * 16 * TM;
    const u4* rp = reinterpret_cast<const u4*>(packed + (size_t)rowc * (size_t)(k >> 1));
    const size_t gbase = (size_t)rowc * (size_t)G;
    const DequantConsts kc = make_dequant_consts();

    f4 acc[TM];
#pragma unroll
    for (int t = 0; t < TM; ++t) acc[t] = (f4){0.0f, 0.0f, 0.0f, 0.0f};

    for (int g = 0; g < G; ++g) {
        for (int w = tid; w < 16 * TM * 16; w += 256) {
            const int tl = w >> 4;
            const int win = w & 15;
            const int t = tok0 + tl;
            u4 v = {0u, 0u, 0u, 0u};
            if (t < m) v = reinterpret_cast<const u4*>(X + (size_t)t * (size_t)k + (size_t)g * 128)[win];
            xt[tl][win] = permute_window(v);
        }
        const u4 qv = __builtin_nontemporal_load(rp + g * 4 + q);
        const uint16_t sb = scales[gbase + g];
        const uint16_t mb = mins[gbase + g];
        h2 codes[16];
        dequant_dword(qv.x, kc, codes + 0);
        dequant_dword(qv.y, kc, codes + 4);
        dequant_dword(qv.z, kc, codes + 8);
        dequant_dword(qv.w, kc, codes + 12);
        const _Float16 sh = __builtin_bit_cast(_Float16, sb);
        const _Float16 mh = __builtin_bit_cast(_Float16, mb);
        const h2 s2 = {sh, sh};
        const h2 m2 = {mh, mh};
        uint32_t wv[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) wv[i] = as_u32(__builtin_elementwise_fma(codes[i], s2, m2));
        __syncthreads();
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const u4 bw = {wv[4 * s + 0], wv[4 * s + 1], wv[4 * s + 2], wv[4 * s + 3]};
            const h8 b = __builtin_bit_cast(h8, bw);
#pragma unroll
            for (int t = 0; t < TM; ++t) {
                const h8 a = __builtin_bit_cast(h8, xt[t * 16 + r][4 * q + s]);
                acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, acc[t], 0, 0, 0);
            }
        }
        __syncthreads();
    }

    if (row < n) {
#pragma unroll
        for (int t = 0; t < TM; ++t) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int tok = tok0 + t * 16 + 4 * q + i;
                if (tok < m) Y[(size_t)tok * (size_t)n + row] = acc[t][i];
            }
        }
    }
}

template <int TM>
static hipError_t launch_tm(const GemvArgs& a, const uint16_t* X, float* Y, int m, hipStream_t st) {
    // One-dimensional grid, row tiles fastest: workgroups launched together
    // share the token tile and stream different weight rows.
    const long row_tiles = ((long)a.n + 63) / 64;
    const long tok_tiles = ((long)m + 16 * TM - 1) / (16 * TM);
    const long blocks = row_tiles * tok_tiles;
    if (blocks > 0x7FFFFFFFL) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((prefill_kernel<TM>), dim3((unsigned)blocks), dim3(256), 0, st,
                       a.packed, a.scales, a.mins, X, Y, a.n, a.k, m, (int)row_tiles);
    return hipGetLastError();
}

hipError_t launch_prefill(const GemvArgs& a, const uint16_t* X, float* Y, int m,
                          const DeviceInfo&, hipStream_t st) {
    const int tiles = (m + 15) / 16;
    if (tiles <= 1) return launch_tm<1>(a, X, Y, m, st);
    if (tiles <= 2) return launch_tm<2>(a, X, Y, m, st);
    if (tiles <= 3) return launch_tm<3>(a, X, Y, m, st);
    if (tiles <= 4) return launch_tm<4>(a, X, Y, m, st);
    if (tiles <= 8) return launch_tm<8>(a, X, Y, m, st);
    return launch_tm<16>(a, X, Y, m, st);
}

}  // namespace q4
