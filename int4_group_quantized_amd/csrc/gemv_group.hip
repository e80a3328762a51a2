// Grouped batch-1 GEMV: many independent int4 group-128 projections in one
// launch.
//
// The rumik write-up ("A detour: the laptop engine on an H100") finds that
// on a fast GPU a small projection costs about one launch latency and that a
// decode step of ~230 launches is bound by launch count, not bytes; its
// advice is to count launches and issue far fewer kernels per layer.  This
// kernel takes up to kGroupMax projections that share one pass mapping
// (lanes per row LPR, chunks per lane CPL, ragged or not: a function of K)
// and streams all of them in one persistent launch.
//
// Work split.  The passes of the projections are numbered one after another
// (projection i owns global passes first[i] .. first[i+1]-1).  Workgroup r,
// in XCD-major order, takes the contiguous range [r*T/G, (r+1)*T/G) of the T
// passes; its 8 waves walk that range wave-major.  A range crosses one or a
// few projections; for each "segment" (the part of the range inside one
// projection) the workgroup stages that projection's x once in LDS, every
// lane copies its slice into registers, and the waves run the batch-1 pass
// loop with the batch-1 kernel's pass schedule for the mapping.
//
// Every row goes through compute_pass<LPR, CPL> with the same lanes, chunk
// order, group updates and butterfly as gemv_reg_kernel for its K, so every
// output is bit-identical to q4g128_gemv on that projection.
#include "q4_device.hpp"
#include "gemv_pass.hpp"
#include "launch.hpp"

namespace q4 {

template <int LPR, int CPL, bool RAGGED, int D, bool XF>
__global__ void __launch_bounds__(kGemvThreads)
gemv_group_kernel(const GroupTable tab) {
    constexpr int RPW = 64 / LPR;
    constexpr int NW = kGemvThreads / 64;
    extern __shared__ u4 x_lds[];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int j = lane % LPR;
    const int rsub = lane / LPR;
    const long total = tab.first[tab.count];
    const long r = xcd_block_order(blockIdx.x, gridDim.x);
    const long a = r * total / gridDim.x;
    const long e = (r + 1) * total / gridDim.x;

    // The projection holding pass a: first[i] <= a < first[i + 1] (every
    // projection has at least one pass, so first[] is strictly increasing),
    // found by bisection over the table in the kernel arguments.
    int i = 0;
    for (int hi = tab.count; hi - i > 1;) {
        const int mid = (i + hi) >> 1;
        if (tab.first[mid] <= a) i = mid; else hi = mid;
    }
    bool staged = false;
    for (; i < tab.count && tab.first[i] < e; ++i) {
        const long f0 = tab.first[i];
        const long s0 = a > f0 ? a : f0;
        const long s1 = e < tab.first[i + 1] ? e : tab.first[i + 1];
        const uint8_t* __restrict__ packed = tab.packed[i];
        const uint16_t* __restrict__ scales = tab.scales[i];
        const uint16_t* __restrict__ mins = tab.mins[i];
        float* __restrict__ y = tab.y[i];
        const int n = tab.n[i];
        const int k = tab.k[i];
        const int C = k >> 5;
        // Local pass numbers within projection i.
        long p = s0 - f0 + wave;
        const long pend = s1 - f0;
        auto row_of = [&](long pp) { return (int)(pp * RPW) + rsub; };
        auto clamp = [&](int rr) { return rr < n ? rr : n - 1; };

        // XF: x is staged before the segment's first weights are requested
        // (as the batch-1 kernel does for short grids), else after.
        PassLoad<CPL> A, B;
        if constexpr (!XF) {
            if (p < pend) load_pass<LPR, CPL, RAGGED>(A, packed, scales, mins, clamp(row_of(p)), k, j);
            if (D == kPassAhead2 && p + NW < pend)
                load_pass<LPR, CPL, RAGGED>(B, packed, scales, mins, clamp(row_of(p + NW)), k, j);
        }

        // Every wave has copied the previous segment's x into registers.
        if (staged) lds_barrier();
        stage_x<LPR, CPL>(tab.x[i], x_lds, k);
        __syncthreads();
        staged = true;
        if constexpr (XF) {
            if (p < pend) load_pass<LPR, CPL, RAGGED>(A, packed, scales, mins, clamp(row_of(p)), k, j);
            if (D == kPassAhead2 && p + NW < pend)
                load_pass<LPR, CPL, RAGGED>(B, packed, scales, mins, clamp(row_of(p + NW)), k, j);
        }

        h2 xp[CPL][16];
        float xs[CPL];
        lane_activations<LPR, CPL, RAGGED>(x_lds, C, j, xp, xs);

        if constexpr (D == kPassNextFirst) {
            while (p < pend) {
                if (p + NW < pend) load_pass<LPR, CPL, RAGGED>(B, packed, scales, mins, clamp(row_of(p + NW)), k, j);
                compute_pass<LPR, CPL>(A, xp, xs, y, row_of(p), n, j);
                p += NW;
                if (p >= pend) break;
                if (p + NW < pend) load_pass<LPR, CPL, RAGGED>(A, packed, scales, mins, clamp(row_of(p + NW)), k, j);
                compute_pass<LPR, CPL>(B, xp, xs, y, row_of(p), n, j);
                p += NW;
            }
            continue;
        }
        while (p < pend) {
            compute_pass<LPR, CPL>(A, xp, xs, y, row_of(p), n, j);
            if (p + 2 * NW < pend)
                load_pass<LPR, CPL, RAGGED>(A, packed, scales, mins, clamp(row_of(p + 2 * NW)), k, j);
            p += NW;
            if (p >= pend) break;
            compute_pass<LPR, CPL>(B, xp, xs, y, row_of(p), n, j);
            if (p + 2 * NW < pend)
                load_pass<LPR, CPL, RAGGED>(B, packed, scales, mins, clamp(row_of(p + 2 * NW)), k, j);
            p += NW;
        }
    }
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------

template <int LPR, int CPL, bool RAGGED, int D>
static hipError_t launch_group_table(const GroupTable& tab, int max_k, const DeviceInfo& dev, hipStream_t st) {
    constexpr int kThreads = kGemvThreads;
    const size_t lds = (size_t)max_k * 2;
    // Both forms have the same registers, hence the same occupancy.
    std::atomic<int>& cached = PerDevice<&gemv_group_kernel<LPR, CPL, RAGGED, D, false>>::value[dev.device];
    int per_cu = cached.load(std::memory_order_relaxed);
    if (per_cu == 0) {
        int nb = 0;
        // The largest x this instantiation stages: K = 32 * LPR * CPL.
        hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &nb, reinterpret_cast<const void*>(&gemv_group_kernel<LPR, CPL, RAGGED, D, false>), kThreads,
            (size_t)64 * LPR * CPL);
        if (e != hipSuccess) return e;
        per_cu = nb > 0 ? nb : 1;
        cached.store(per_cu, std::memory_order_relaxed);
    }
    const long total = tab.first[tab.count];
    long grid = (long)dev.num_cu * per_cu;
    const long need = (total + (kThreads / 64) - 1) / (kThreads / 64);
    if (grid > need) grid = need;
    // x first with one workgroup per CU (measured on the pages' step, whose
    // K = 11,008 projections run at one workgroup per CU: 238.2-238.6 against
    // 241.0-241.3 us, same bits; the 36-layer step's K = 8,192 launch, also
    // one per CU, is unchanged; at two per CU it is not faster either).
    if (per_cu == 1)
        hipLaunchKernelGGL((gemv_group_kernel<LPR, CPL, RAGGED, D, true>), dim3((unsigned)grid), dim3(kThreads), lds,
                           st, tab);
    else
        hipLaunchKernelGGL((gemv_group_kernel<LPR, CPL, RAGGED, D, false>), dim3((unsigned)grid), dim3(kThreads), lds,
                           st, tab);
    return hipGetLastError();
}

// Variant index of a K: the (LPR, CPL, ragged) instantiations that the
// batch-1 GEMV runs in registers; -1 for shapes it runs on the batched
// kernel (those are launched one by one as q4g128_gemv calls).
struct GroupVariant {
    int lpr, cpl;
    bool ragged;
};
static constexpr GroupVariant kVariants[] = {
    {64, 1, false}, {64, 2, false}, {64, 3, false}, {64, 4, false}, {32, 1, false}, {32, 2, false},
    {32, 3, false}, {16, 1, false}, {16, 3, false}, {8, 1, false},  {8, 3, false},  {4, 1, false},
    {4, 3, false},  {64, 2, true},  {64, 3, true},  {64, 4, true},  {64, 5, true},  {64, 6, true},
};
static constexpr int kNumVariants = sizeof(kVariants) / sizeof(kVariants[0]);

int group_variant(int k) {
    const int lpr = lanes_per_row(k);
    const int C = k >> 5;
    const int cpl = (C + lpr - 1) / lpr;
    const bool ragged = C % lpr != 0;
    for (int v = 0; v < kNumVariants; ++v)
        if (kVariants[v].lpr == lpr && kVariants[v].cpl == cpl && kVariants[v].ragged == ragged) return v;
    return -1;
}

static hipError_t dispatch_group(int v, const GroupTable& tab, int max_k, const DeviceInfo& dev, hipStream_t st) {
    switch (v) {
// The pass schedule follows the batch-1 GEMV's choice for the mapping.
#define Q4_GRP(I, L, P, R) \
    case I: return launch_group_table<L, P, R, pass_schedule(L, P, R)>(tab, max_k, dev, st);
        Q4_GRP(0, 64, 1, false) Q4_GRP(1, 64, 2, false) Q4_GRP(2, 64, 3, false) Q4_GRP(3, 64, 4, false)
        Q4_GRP(4, 32, 1, false) Q4_GRP(5, 32, 2, false) Q4_GRP(6, 32, 3, false) Q4_GRP(7, 16, 1, false)
        Q4_GRP(8, 16, 3, false) Q4_GRP(9, 8, 1, false) Q4_GRP(10, 8, 3, false) Q4_GRP(11, 4, 1, false)
        Q4_GRP(12, 4, 3, false) Q4_GRP(13, 64, 2, true) Q4_GRP(14, 64, 3, true) Q4_GRP(15, 64, 4, true)
        Q4_GRP(16, 64, 5, true) Q4_GRP(17, 64, 6, true)
#undef Q4_GRP
    }
    return hipErrorInvalidValue;
}

hipError_t launch_gemv_group(const GemvArgs* list, int count, const DeviceInfo& dev, hipStream_t st) {
    // Projections of one variant, in call order, kGroupMax per launch.
    for (int v = -1; v < kNumVariants; ++v) {
        GroupTable tab;
        tab.count = 0;
        tab.first[0] = 0;
        int max_k = 0;
        for (int q = 0; q <= count; ++q) {
            const bool flush = q == count || tab.count == kGroupMax;
            if (flush && tab.count > 0) {
                hipError_t e = dispatch_group(v, tab, max_k, dev, st);
                if (e != hipSuccess) return e;
                tab.count = 0;
                max_k = 0;
            }
            if (q == count) break;
            const GemvArgs& a = list[q];
            if (group_variant(a.k) != v) continue;
            if (v < 0) {
                hipError_t e = launch_gemv(a, dev, st);
                if (e != hipSuccess) return e;
                continue;
            }
            const int rpw = 64 / kVariants[v].lpr;
            const int c = tab.count;
            tab.packed[c] = a.packed;
            tab.scales[c] = a.scales;
            tab.mins[c] = a.mins;
            tab.x[c] = a.x;
            tab.y[c] = a.y;
            tab.n[c] = a.n;
            tab.k[c] = a.k;
            tab.first[c + 1] = tab.first[c] + ((long)a.n + rpw - 1) / rpw;
            tab.count = c + 1;
            if (a.k > max_k) max_k = a.k;
        }
    }
    return hipSuccess;
}

}  // namespace q4
