// Device-side building blocks shared by the gfx950 kernels of the int4
// group-128 library.  Everything here is per-lane arithmetic whose order is
// fixed, so that every kernel that calls it produces the same bits for the
// same (row, column) pair.
//
// Unit of work: a "chunk" is 16 bytes of one packed row = 32 consecutive
// codes = a quarter of a 128-column group.  A chunk is consumed as four
// dwords of eight codes each.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace q4 {

typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef uint32_t u4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ h2 as_h2(uint32_t v) { return __builtin_bit_cast(h2, v); }
__device__ __forceinline__ uint32_t as_u32(h2 v) { return __builtin_bit_cast(uint32_t, v); }

__device__ __forceinline__ float f16_bits_to_f32(uint16_t b) {
    return (float)__builtin_bit_cast(_Float16, b);
}

// ---------------------------------------------------------------------------
// Matrix-vector path: codes as fp16 denormals.
//
// An fp16 whose exponent field is zero is a denormal worth mantissa * 2^-24,
// with no implicit leading one.  Masking a dword of packed codes therefore
// yields exact, bias-free fp16 pairs in one AND each:
//   q        & 0x000F000F -> (c0, c4) * 2^-24     (nibbles in bits 0..3)
//   q        & 0x00F000F0 -> (c1, c5) * 2^-20     (nibbles in bits 4..7)
//   (q >> 8) & 0x000F000F -> (c2, c6) * 2^-24
//   (q >> 8) & 0x00F000F0 -> (c3, c7) * 2^-20
// (byte b of the dword holds columns 2b and 2b+1 in its low and high
// nibble).  v_dot2_f32_f16 multiplies these by the fp16 activations
// exactly, so the products carry the scale 2^-24 or 2^-20; the two scales
// are summed in separate fp32 chains (lo = L * 2^-24, hi = H * 2^-20) and
// joined exactly as lo * 16 + hi = (L + H) * 2^-20.  One chunk costs 1 shift + 4 ANDs + 4 dot2 per 8 codes.
// ---------------------------------------------------------------------------

constexpr float kLoScale = 16.0f;          // (L * 2^-24) * 16 = L * 2^-20
constexpr float kUnit = 9.5367431640625e-07f;  // 2^-20: scale of chunk dots and sums
constexpr float kInvUnit = 1048576.0f;    // 2^20

// 32 codes of a chunk -> 16 fp16 pairs (see above) in pair order
//   [4d + 0] = (c0, c4), [4d + 1] = (c1, c5), [4d + 2] = (c2, c6), [4d + 3] = (c3, c7)
// for dword d of the chunk (columns 8d .. 8d+7).
__device__ __forceinline__ void chunk_codes(const u4 q, h2 codes[16]) {
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        const uint32_t q8 = w[d] >> 8;
        codes[4 * d + 0] = as_h2(w[d] & 0x000F000Fu);
        codes[4 * d + 1] = as_h2(w[d] & 0x00F000F0u);
        codes[4 * d + 2] = as_h2(q8 & 0x000F000Fu);
        codes[4 * d + 3] = as_h2(q8 & 0x00F000F0u);
    }
}

// a.x * b.x + a.y * b.y + 0 in one instruction.  Equal to fdot2(a, b, 0.0f);
// spelled out because the compiler otherwise zeroes a register and uses the
// accumulating two-address form, one extra instruction per chain.
__device__ __forceinline__ float dot2_first(h2 a, h2 b) {
    float r;
    asm("v_dot2_f32_f16 %0, %1, %2, 0" : "=v"(r) : "v"(a), "v"(b));
    return r;
}

// sum(code * x) * 2^-20 over one chunk, from chunk_codes() and the 16
// activation pairs in the same order.  Exact products; two fp32 chains
// starting from 0 (pairs 0, 2, 4, ... and 1, 3, 5, ...), then
// lo * 16 + hi in one fused multiply-add (the multiply is exact).  Every kernel that needs a chunk dot calls this.
__device__ __forceinline__ float chunk_dot(const h2 codes[16], const h2 xp[16]) {
    float lo = dot2_first(codes[0], xp[0]);
    float hi = dot2_first(codes[1], xp[1]);
#pragma unroll
    for (int i = 2; i < 16; i += 2) {
        lo = __builtin_amdgcn_fdot2(codes[i], xp[i], lo, false);
        hi = __builtin_amdgcn_fdot2(codes[i + 1], xp[i + 1], hi, false);
    }
    return __builtin_fmaf(lo, kLoScale, hi);
}

// Eight consecutive fp16 activations (one 16-byte window, natural order
// x0..x7) -> the pair order of the code pairs:
//   (x0, x4), (x1, x5), (x2, x6), (x3, x7).
__device__ __forceinline__ u4 permute_window(u4 v) {
    u4 r;
    r.x = (v.x & 0xFFFFu) | (v.z << 16);
    r.y = (v.x >> 16) | (v.z & 0xFFFF0000u);
    r.z = (v.y & 0xFFFFu) | (v.w << 16);
    r.w = (v.y >> 16) | (v.w & 0xFFFF0000u);
    return r;
}

// sum(x) * 2^-20 over the 32 activations of a chunk, from its 16 permuted
// pairs, in fp32 with a fixed order (pair 0 first).
__device__ __forceinline__ float chunk_xsum(const h2 xp[16]) {
    const h2 one = {(_Float16)1.0f, (_Float16)1.0f};
    float acc = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) acc = __builtin_amdgcn_fdot2(xp[i], one, acc, false);
    return acc * kUnit;
}

// ---------------------------------------------------------------------------
// Prompt-processing path: exact integer-valued fp16 codes.
//
// OR-ing a nibble into the mantissa of fp16 1024.0 (exponent 10, so the
// mantissa's unit is 1) gives 1024 + c with no integer-to-float convert; a
// nibble in mantissa bits 4..7 gives 1024 + 16c.  The bias is removed
// exactly: (1024 + c) - 1024 = c and (1024 + 16c) * (1/16) - 64 = c.  The
// result feeds fp16 arithmetic (w = fma(c, scale, min)), which needs the
// code itself rather than a scaled denormal.
// ---------------------------------------------------------------------------

// Constants of that conversion, materialised once per kernel.  gfx950 VOP3
// instructions cannot encode literals and read at most one scalar register,
// so the masks live in SGPRs and the exponent pattern in a VGPR; each
// nibble pair then costs a single v_and_or_b32.
struct DequantConsts {
    uint32_t mask_lo;  // 0x000F000F: nibbles 0 and 4 of a dword
    uint32_t mask_hi;  // 0x00F000F0: nibbles 1 and 5 of a dword
    uint32_t magic;    // 0x64006400: fp16 1024.0 in both halves
};

__device__ __forceinline__ DequantConsts make_dequant_consts() {
    DequantConsts c;
    asm volatile("s_mov_b32 %0, 0x000F000F" : "=s"(c.mask_lo));
    asm volatile("s_mov_b32 %0, 0x00F000F0" : "=s"(c.mask_hi));
    uint32_t m;
    asm volatile("s_mov_b32 %0, 0x64006400" : "=s"(m));
    asm volatile("v_mov_b32 %0, %1" : "=v"(c.magic) : "s"(m));
    return c;
}

// Eight codes of one dword -> four fp16 pairs holding the exact codes, in
// the pair order (c0, c4), (c1, c5), (c2, c6), (c3, c7).
__device__ __forceinline__ void dequant_dword(uint32_t q, const DequantConsts& k, h2 out[4]) {
    const uint32_t q8 = q >> 8;
    const uint32_t a = (q & k.mask_lo) | k.magic;
    const uint32_t b = (q & k.mask_hi) | k.magic;
    const uint32_t c = (q8 & k.mask_lo) | k.magic;
    const uint32_t d = (q8 & k.mask_hi) | k.magic;
    const h2 bias = {(_Float16)1024.0f, (_Float16)1024.0f};
    const h2 sixteenth = {(_Float16)0.0625f, (_Float16)0.0625f};
    const h2 neg64 = {(_Float16)-64.0f, (_Float16)-64.0f};
    out[0] = as_h2(a) - bias;
    out[1] = __builtin_elementwise_fma(as_h2(b), sixteenth, neg64);
    out[2] = as_h2(c) - bias;
    out[3] = __builtin_elementwise_fma(as_h2(d), sixteenth, neg64);
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

// Rank of workgroup b among the workgroups of its XCD, laid out XCD by XCD
// (the dispatcher deals workgroups to the 8 XCDs round-robin, block b on
// XCD b % 8): consecutive ranks then share one L2.
__device__ __forceinline__ int xcd_block_order(int b, int grid) {
    constexpr int kXcd = 8;
    const int per = grid / kXcd, rem = grid % kXcd, x = b % kXcd;
    return x * per + (x < rem ? x : rem) + b / kXcd;
}

// Workgroup barrier for LDS hand-offs only.  It waits for this wave's LDS
// operations and does not drain outstanding global loads (unlike
// __syncthreads, whose fence would empty the prefetch rings).
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt and expcnt untouched
    __builtin_amdgcn_s_barrier();
}

// One group-slice update of a lane's running row sum (all in 2^-20 units):
//   y += scale * sum(code*x) ; y += min * sum(x)
// i.e. sum((code*scale + min) * x) over the slice, with each term once.
__device__ __forceinline__ float group_update(float y, uint16_t s_bits, uint16_t m_bits, float dot, float xsum) {
    y = __builtin_fmaf(f16_bits_to_f32(s_bits), dot, y);
    y = __builtin_fmaf(f16_bits_to_f32(m_bits), xsum, y);
    return y;
}

// Butterfly sum over aligned groups of LPR lanes (LPR a power of two <= 64).
// Pairing per level: lane i with i^1, then i^2, then the other half of its
// 8-lane group (row_half_mirror), the other half of its 16-lane row
// (row_mirror), the other row of its 32-lane half (ds_swizzle xor 16) and the
// other half of the wave.  Each level pairs the same partial sums as an xor
// butterfly, and every lane of a group ends with the same bits.
template <int CTRL>
__device__ __forceinline__ float dpp_move(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

// The value of lane ^ 16 within each 32-lane half.
__device__ __forceinline__ float lane_swap16(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, v), 0x401F));
}

template <int LPR>
__device__ __forceinline__ float reduce_lanes(float v) {
    if constexpr (LPR >= 2) v = v + dpp_move<0xB1>(v);    // quad_perm [1,0,3,2]
    if constexpr (LPR >= 4) v = v + dpp_move<0x4E>(v);    // quad_perm [2,3,0,1]
    if constexpr (LPR >= 8) v = v + dpp_move<0x141>(v);   // row_half_mirror
    if constexpr (LPR >= 16) v = v + dpp_move<0x140>(v);  // row_mirror
    if constexpr (LPR >= 32) v = v + lane_swap16(v);
    if constexpr (LPR >= 64) v = v + __shfl_xor(v, 32, 64);
    return v;
}

}  // namespace q4
