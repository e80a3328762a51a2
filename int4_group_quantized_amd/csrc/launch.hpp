// Internal host-side interface between the C-ABI layer (api.cpp) and the
// kernel translation units.  Arguments reaching these launchers have already
// been validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <atomic>

namespace q4 {

constexpr int kMaxDevices = 64;  // device ordinals the library serves (checked by the C ABI)

// A launch property computed once per device and kernel instantiation
// (occupancy, a function attribute): 0 until set.  Racing first calls
// compute the same value; release/acquire order makes a set attribute
// visible to any thread that reads the flag.
template <auto Kernel>
struct PerDevice {
    static std::atomic<int> value[kMaxDevices];
};
template <auto Kernel>
std::atomic<int> PerDevice<Kernel>::value[kMaxDevices];

struct DeviceInfo {
    int device = -1;
    int num_cu = 0;
    size_t max_lds = 0;  // usable dynamic LDS bytes per workgroup
};

struct GemvArgs {
    const uint8_t* packed;
    const uint16_t* scales;
    const uint16_t* mins;
    const uint16_t* x;
    float* y;
    int n;
    int k;
};

int lanes_per_row(int k);

// Projections of one grouped-GEMV launch (passed by value as the kernel
// argument).  Projection i owns the global passes first[i] .. first[i+1]-1.
// 64 projections make a 3,596-byte table (3,856 bytes of kernel arguments
// with the implicit ones), inside the 4 KB that a kernel's arguments may
// take; 64 per launch against 32 measured 2.8% faster on the 36-layer step
// at K = 3,072 and 3.7% on the pages' step (same bits).
constexpr int kGroupMax = 64;
static_assert(sizeof(void*) == 8, "table size above assumes 64-bit pointers");
struct GroupTable {
    const uint8_t* packed[kGroupMax];
    const uint16_t* scales[kGroupMax];
    const uint16_t* mins[kGroupMax];
    const uint16_t* x[kGroupMax];
    float* y[kGroupMax];
    int n[kGroupMax];
    int k[kGroupMax];
    long first[kGroupMax + 1];
    int count;
};
static_assert(sizeof(GroupTable) <= 3840, "the grouped table must fit in the kernel argument space");

hipError_t launch_pack(const uint8_t* codes, uint8_t* packed, int64_t n, int64_t k, hipStream_t st);
hipError_t launch_quantize(const float* W, uint8_t* packed, uint16_t* scales, uint16_t* mins, int64_t n,
                           int64_t k, hipStream_t st);
constexpr long kQuantizeMaxGroups = 1L << 36;  // largest export (groups of 128 values)
hipError_t launch_head_int8(const int8_t* q, const uint16_t* scales, const uint16_t* x, float* y, int64_t n,
                            int64_t k, const DeviceInfo& dev, hipStream_t st);
hipError_t launch_gemv(const GemvArgs& a, const DeviceInfo& dev, hipStream_t st);
// Independent projections (no output overlaps any input or other output):
// one launch per kGroupMax projections of the same pass mapping; shapes the
// batch-1 GEMV runs on its batched kernel are launched one by one.
hipError_t launch_gemv_group(const GemvArgs* list, int count, const DeviceInfo& dev, hipStream_t st);
hipError_t launch_small_batch(const GemvArgs& a, const uint16_t* X, float* Y, int b,
                              const DeviceInfo& dev, hipStream_t st);
// hipErrorNotSupported when the shape has no segmented form (LPR below 16, or
// the two staging buffers exceed the LDS).
hipError_t launch_small_batch_segmented(const GemvArgs& a, const uint16_t* X, float* Y, int b,
                                        const DeviceInfo& dev, hipStream_t st);
hipError_t launch_prefill(const GemvArgs& a, const uint16_t* X, float* Y, int m,
                          const DeviceInfo& dev, hipStream_t st);
// Whether a prompt of more than 64 tokens runs faster as blocks of the split
// kernel (launch_prefill_split takes any m; above 64 it launches blocks).
bool prefill_token_blocks_pay(long n, long m, const DeviceInfo& dev);
// Tokens of a prompt that the prompt calls run first as one paired-block
// launch (the rest routed on its own), or 0 for one launch.
long prefill_pair_head_tokens(long n, long m, const DeviceInfo& dev);
hipError_t launch_prefill_split(const GemvArgs& a, const uint16_t* X, float* Y, int m,
                                const DeviceInfo& dev, hipStream_t st);
hipError_t launch_prefill_split_epilogue(const GemvArgs& a, const uint16_t* X, float* Y, int m,
                                         const DeviceInfo& dev, hipStream_t st);
hipError_t launch_prefill_pair(const GemvArgs& a, const uint16_t* X, float* Y, int m,
                               const DeviceInfo& dev, hipStream_t st);
hipError_t launch_prefill_pair_epilogue(const GemvArgs& a, const uint16_t* X, float* Y, int m,
                                        const DeviceInfo& dev, hipStream_t st);
hipError_t launch_prefill_epilogue(const GemvArgs& a, const uint16_t* X, float* Y, int m,
                                   const DeviceInfo& dev, hipStream_t st);

}  // namespace q4
