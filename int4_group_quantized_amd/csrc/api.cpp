// C ABI of the int4 group-128 library: argument validation (host only, no
// HIP call before it passes), per-device properties, dispatch to the kernel
// launchers and status reporting.
#include "q4g128.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <mutex>
#include <utility>
#include <vector>

#include "launch.hpp"

namespace {

thread_local int32_t g_last_hip_error = 0;

constexpr int kMaxDevices = q4::kMaxDevices;
q4::DeviceInfo g_dev[kMaxDevices];
std::mutex g_dev_mu;

q4_status device_error(hipError_t e) {
    g_last_hip_error = (int32_t)e;
    (void)hipGetLastError();  // clear the sticky per-thread error for the caller
    return Q4_EDEVICE;
}

// Properties of the current device, queried once per device.
q4_status current_device(q4::DeviceInfo* out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return device_error(e);
    if (dev < 0 || dev >= kMaxDevices) return device_error(hipErrorInvalidDevice);
    std::lock_guard<std::mutex> lock(g_dev_mu);
    q4::DeviceInfo& d = g_dev[dev];
    if (d.device != dev) {
        int cu = 0, lds = 0, lds_optin = 0;
        e = hipDeviceGetAttribute(&cu, hipDeviceAttributeMultiprocessorCount, dev);
        if (e != hipSuccess) return device_error(e);
        e = hipDeviceGetAttribute(&lds, hipDeviceAttributeMaxSharedMemoryPerBlock, dev);
        if (e != hipSuccess) return device_error(e);
        if (hipDeviceGetAttribute(&lds_optin, hipDeviceAttributeSharedMemPerBlockOptin, dev) != hipSuccess) {
            (void)hipGetLastError();
            lds_optin = 0;
        }
        d.num_cu = cu;
        d.max_lds = (size_t)(lds_optin > lds ? lds_optin : lds);
        d.device = dev;
    }
    *out = d;
    return Q4_OK;
}

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

// End of [p, p + bytes), saturated at the top of the address space.
uintptr_t end_of(const void* p, size_t bytes) {
    const uintptr_t a = (uintptr_t)p;
    return bytes > UINTPTR_MAX - a ? UINTPTR_MAX : a + bytes;
}

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
    return (uintptr_t)a < end_of(b, nb) && (uintptr_t)b < end_of(a, na);
}

q4_status check_nk(int64_t n, int64_t k) {
    if (n <= 0) return Q4_EINVAL;
    if (k < Q4G128_GROUP || k % Q4G128_GROUP != 0 || k > Q4G128_MAX_K) return Q4_ESHAPE;
    if (n > Q4G128_MAX_N) return Q4_ESHAPE;
    return Q4_OK;
}

// Shared checks of the three product entry points; `rows` = B or M.
q4_status check_product(const uint8_t* packed, const uint16_t* scales, const uint16_t* mins,
                        const uint16_t* X, const float* Y, int64_t n, int64_t k, int64_t rows) {
    if (!packed || !scales || !mins || !X || !Y) return Q4_EINVAL;
    q4_status s = check_nk(n, k);
    if (s != Q4_OK) return s;
    if (rows > Q4G128_MAX_N) return Q4_ESHAPE;
    if (!aligned(packed, 16) || !aligned(X, 16) || !aligned(scales, 2) || !aligned(mins, 2) ||
        !aligned(Y, 4))
        return Q4_EALIGN;
    const size_t g = (size_t)(k / Q4G128_GROUP);
    // rows and n are below 2^31, so their product fits; its byte count may not.
    const uint64_t yelems = (uint64_t)rows * (uint64_t)n;
    if (yelems > UINT64_MAX / sizeof(float)) return Q4_ESHAPE;
    const size_t ybytes = (size_t)yelems * sizeof(float);
    if (overlaps(Y, ybytes, packed, (size_t)n * (size_t)k / 2) ||
        overlaps(Y, ybytes, scales, (size_t)n * g * 2) || overlaps(Y, ybytes, mins, (size_t)n * g * 2) ||
        overlaps(Y, ybytes, X, (size_t)rows * (size_t)k * 2))
        return Q4_EINVAL;
    return Q4_OK;
}

q4::GemvArgs make_args(const uint8_t* packed, const uint16_t* scales, const uint16_t* mins,
                       const uint16_t* x, float* y, int64_t n, int64_t k) {
    q4::GemvArgs a;
    a.packed = packed;
    a.scales = scales;
    a.mins = mins;
    a.x = x;
    a.y = y;
    a.n = (int)n;
    a.k = (int)k;
    return a;
}

}  // namespace

extern "C" {

q4_status q4g128_pack(const uint8_t* codes, uint8_t* packed, int64_t n, int64_t k, void* stream) {
    if (!codes || !packed) return Q4_EINVAL;
    q4_status s = check_nk(n, k);
    if (s != Q4_OK) return s;
    if (!aligned(codes, 16) || !aligned(packed, 16)) return Q4_EALIGN;
    if (overlaps(packed, (size_t)n * (size_t)k / 2, codes, (size_t)n * (size_t)k)) return Q4_EINVAL;
    hipError_t e = q4::launch_pack(codes, packed, n, k, (hipStream_t)stream);
    return e == hipSuccess ? Q4_OK : device_error(e);
}

q4_status q4g128_quantize(const float* W, uint8_t* packed, uint16_t* scales, uint16_t* mins, int64_t n,
                          int64_t k, void* stream) {
    if (!W || !packed || !scales || !mins) return Q4_EINVAL;
    q4_status s = check_nk(n, k);
    if (s != Q4_OK) return s;
    const size_t groups = (size_t)n * (size_t)(k / Q4G128_GROUP);
    if (groups > (size_t)q4::kQuantizeMaxGroups) return Q4_ESHAPE;
    if (!aligned(W, 16) || !aligned(packed, 16) || !aligned(scales, 2) || !aligned(mins, 2)) return Q4_EALIGN;
    const size_t wbytes = (size_t)n * (size_t)k * 4, pbytes = (size_t)n * (size_t)k / 2, gbytes = groups * 2;
    if (overlaps(packed, pbytes, W, wbytes) || overlaps(scales, gbytes, W, wbytes) ||
        overlaps(mins, gbytes, W, wbytes) || overlaps(packed, pbytes, scales, gbytes) ||
        overlaps(packed, pbytes, mins, gbytes) || overlaps(scales, gbytes, mins, gbytes))
        return Q4_EINVAL;
    hipError_t e = q4::launch_quantize(W, packed, scales, mins, n, k, (hipStream_t)stream);
    return e == hipSuccess ? Q4_OK : device_error(e);
}

q4_status q4g128_gemv(const uint8_t* packed, const uint16_t* scales, const uint16_t* mins,
                      const uint16_t* x, float* y, int64_t n, int64_t k, void* stream) {
    q4_status s = check_product(packed, scales, mins, x, y, n, k, 1);
    if (s != Q4_OK) return s;
    q4::DeviceInfo dev;
    s = current_device(&dev);
    if (s != Q4_OK) return s;
    hipError_t e = q4::launch_gemv(make_args(packed, scales, mins, x, y, n, k), dev, (hipStream_t)stream);
    return e == hipSuccess ? Q4_OK : device_error(e);
}

q4_status q4g128_gemv_grouped(const q4g128_gemv_desc* descs, int64_t count, void* stream) {
    if (!descs || count < 1 || count > Q4G128_MAX_GROUPED) return Q4_EINVAL;
    std::vector<q4::GemvArgs> list((size_t)count);
    // Outputs must be pairwise disjoint and disjoint from every input.
    std::vector<std::pair<uintptr_t, uintptr_t>> outs((size_t)count);
    for (int64_t i = 0; i < count; ++i) {
        const q4g128_gemv_desc& d = descs[i];
        q4_status s = check_product(d.packed, d.scales, d.mins, d.x, d.y, d.n, d.k, 1);
        if (s != Q4_OK) return s;
        list[(size_t)i] = make_args(d.packed, d.scales, d.mins, d.x, d.y, d.n, d.k);
        outs[(size_t)i] = {(uintptr_t)d.y, end_of(d.y, (size_t)d.n * sizeof(float))};
    }
    std::sort(outs.begin(), outs.end());
    for (size_t i = 1; i < outs.size(); ++i)
        if (outs[i - 1].second > outs[i].first) return Q4_EINVAL;
    // The only output that can overlap [lo, hi) is the last one starting below hi.
    auto hits_output = [&](const void* p, size_t bytes) {
        const uintptr_t lo = (uintptr_t)p, hi = end_of(p, bytes);
        auto it = std::lower_bound(outs.begin(), outs.end(), std::make_pair(hi, (uintptr_t)0));
        if (it == outs.begin()) return false;
        --it;
        return it->second > lo;
    };
    for (int64_t i = 0; i < count; ++i) {
        const q4g128_gemv_desc& d = descs[i];
        const size_t g = (size_t)(d.k / Q4G128_GROUP);
        if (hits_output(d.packed, (size_t)d.n * (size_t)d.k / 2) || hits_output(d.scales, (size_t)d.n * g * 2) ||
            hits_output(d.mins, (size_t)d.n * g * 2) || hits_output(d.x, (size_t)d.k * 2))
            return Q4_EINVAL;
    }
    q4::DeviceInfo dev;
    q4_status s = current_device(&dev);
    if (s != Q4_OK) return s;
    hipError_t e = q4::launch_gemv_group(list.data(), (int)count, dev, (hipStream_t)stream);
    return e == hipSuccess ? Q4_OK : device_error(e);
}

q4_status q4g128_gemm_small_batch(const uint8_t* packed, const uint16_t* scales, const uint16_t* mins,
                                  const uint16_t* X, float* Y, int64_t n, int64_t k, int64_t b,
                                  void* stream) {
    if (b < 1 || b > Q4G128_MAX_BATCH) return Q4_EINVAL;
    q4_status s = check_product(packed, scales, mins, X, Y, n, k, b);
    if (s != Q4_OK) return s;
    q4::DeviceInfo dev;
    s = current_device(&dev);
    if (s != Q4_OK) return s;
    hipError_t e = q4::launch_small_batch(make_args(packed, scales, mins, X, Y, n, k), X, Y, (int)b, dev,
                                          (hipStream_t)stream);
    return e == hipSuccess ? Q4_OK : device_error(e);
}

q4_status q4g128_gemm_prefill(const uint8_t* packed, const uint16_t* scales, const uint16_t* mins,
                              const uint16_t* X, float* Y, int64_t n, int64_t k, int64_t m,
                              void* stream) {
    if (m < 1) return Q4_EINVAL;
    q4_status s = check_product(packed, scales, mins, X, Y, n, k, m);
    if (s != Q4_OK) return s;
    if (((n + 63) / 64) * ((m + 15) / 16) > 0x7FFFFFFFLL) return Q4_ESHAPE;
    q4::DeviceInfo dev;
    s = current_device(&dev);
    if (s != Q4_OK) return s;
    hipError_t e = q4::launch_prefill(make_args(packed, scales, mins, X, Y, n, k), X, Y, (int)m, dev,
                                      (hipStream_t)stream);
    return e == hipSuccess ? Q4_OK : device_error(e);
}

q4_status q4g128_gemm_prefill_epilogue(const uint8_t* packed, const uint16_t* scales, const uint16_t* mins,
                                       const uint16_t* X, float* Y, int64_t n, int64_t k, int64_t m,
                                       void* stream) {
    if (m < 1) return Q4_EINVAL;
    q4_status s = check_product(packed, scales, mins, X, Y, n, k, m);
    if (s != Q4_OK) return s;
    if ((size_t)m * (size_t)n > (size_t)0x7FFFFFFFFFFFLL) return Q4_ESHAPE;
    q4::DeviceInfo dev;
    s = current_device(&dev);
    if (s != Q4_OK) return s;
    hipError_t e = q4::launch_prefill_epilogue(make_args(packed, scales, mins, X, Y, n, k), X, Y, (int)m, dev,
                                               (hipStream_t)stream);
    return e == hipSuccess ? Q4_OK : device_error(e);
}

q4_status q4g128_gemv_int8(const int8_t* q, const uint16_t* scales, const uint16_t* x, float* y, int64_t n,
                           int64_t k, void* stream) {
    if (!q || !scales || !x || !y) return Q4_EINVAL;
    if (n <= 0) return Q4_EINVAL;
    if (k < Q4G128_GROUP || k % Q4G128_GROUP != 0 || k > Q4G128_INT8_MAX_K || n > Q4G128_MAX_N) return Q4_ESHAPE;
    if (!aligned(q, 16) || !aligned(x, 16) || !aligned(scales, 2) || !aligned(y, 4)) return Q4_EALIGN;
    const size_t ybytes = (size_t)n * sizeof(float);
    if (overlaps(y, ybytes, q, (size_t)n * (size_t)k) || overlaps(y, ybytes, scales, (size_t)n * 2) ||
        overlaps(y, ybytes, x, (size_t)k * 2))
        return Q4_EINVAL;
    q4::DeviceInfo dev;
    q4_status s = current_device(&dev);
    if (s != Q4_OK) return s;
    hipError_t e = q4::launch_head_int8(q, scales, x, y, n, k, dev, (hipStream_t)stream);
    return e == hipSuccess ? Q4_OK : device_error(e);
}

const char* q4g128_status_string(q4_status status) {
    switch (status) {
        case Q4_OK: return "Q4_OK: success";
        case Q4_EINVAL: return "Q4_EINVAL: null pointer, non-positive size, batch outside 1..16 or overlapping output";
        case Q4_ESHAPE: return "Q4_ESHAPE: K must be a multiple of 128 in [128, 32768]; sizes must fit the kernels' index range";
        case Q4_EALIGN: return "Q4_EALIGN: packed/codes/activations/float weights need 16-byte, scales/mins 2-byte, outputs 4-byte alignment";
        case Q4_EDEVICE: return "Q4_EDEVICE: the HIP runtime reported an error (see q4g128_last_hip_error)";
    }
    return "unknown q4g128 status";
}

int32_t q4g128_last_hip_error(void) { return g_last_hip_error; }

}  // extern "C"
