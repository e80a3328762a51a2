// Pack unpacked 4-bit codes two per byte: byte j of a row holds column 2j in
// bits 0..3 and column 2j+1 in bits 4..7.
#include "q4_device.hpp"
#include "launch.hpp"

namespace q4 {

// Per dword of four codes c0..c3 (one per byte): v | (v >> 4) puts
// c0 | c1 << 4 in byte 0 and c2 | c3 << 4 in byte 2; keep those two bytes.
__device__ __forceinline__ uint32_t pack_dword(uint32_t w) {
    const uint32_t v = w & 0x0F0F0F0Fu;
    const uint32_t t = v | (v >> 4);
    return (t & 0xFFu) | ((t >> 8) & 0xFF00u);
}

// Each thread turns 32 codes (two 16-byte loads) into 16 packed bytes.
__global__ void __launch_bounds__(256)
pack_kernel(const u4* __restrict__ codes, u4* __restrict__ packed, size_t units) {
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < units;
         i += (size_t)gridDim.x * blockDim.x) {
        const u4 a = codes[2 * i];
        const u4 b = codes[2 * i + 1];
        u4 r;
        r.x = pack_dword(a.x) | (pack_dword(a.y) << 16);
        r.y = pack_dword(a.z) | (pack_dword(a.w) << 16);
        r.z = pack_dword(b.x) | (pack_dword(b.y) << 16);
        r.w = pack_dword(b.z) | (pack_dword(b.w) << 16);
        packed[i] = r;
    }
}

hipError_t launch_pack(const uint8_t* codes, uint8_t* packed, int64_t n, int64_t k, hipStream_t st) {
    const size_t units = (size_t)n * (size_t)k / 32;  // K is a multiple of 128
    const unsigned block = 256;
    size_t grid = (units + block - 1) / block;
    if (grid > 65536) grid = 65536;  // grid-stride loop covers the rest
    hipLaunchKernelGGL(pack_kernel, dim3((unsigned)grid), dim3(block), 0, st,
                       reinterpret_cast<const u4*>(codes), reinterpret_cast<u4*>(packed), units);
    return hipGetLastError();
}

}  // namespace q4
