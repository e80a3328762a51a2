// Small-batch matmat, slot by slot: for rows too long for all B activation
// columns to sit in LDS at once (16 columns of K = 11,008 would need 374 KB),
// and for matrices whose rows this grid covers in one round (at most
// 4,096 passes on 256 CUs).
//
// The work mapping is the batch-1 one (lanes per row LPR, lane j of a row
// owns chunks j + t*LPR), walked one chunk slot t at a time: slot t covers
// chunks [t*LPR, (t+1)*LPR) of every row, and the workgroup stages exactly
// those chunks of all BT columns.  Two LDS buffers alternate, so slot t + 1
// is staged while slot t is consumed, with one barrier per slot.  Each wave
// owns R passes (64 / LPR rows each) for the whole kernel and keeps their
// R x BT running lane sums in registers across the slots (R = 2 once the rows
// exceed one pass per wave of a workgroup per CU: every column read from LDS
// then serves two rows, and no second round of workgroups is needed).  Every
// lane applies
// group_update in ascending t exactly as the batch-1 kernel does, and the
// same butterfly finishes each row: column b equals q4g128_gemv(X[b]) bit for
// bit.  Chunks past C (ragged rows) get zero activations and a zero chunk sum
// against the row's last chunk of codes, which leaves a lane sum unchanged
// (the argument of the batch-1 kernel).  Columns b >= nb are zero and never
// stored.
#include "q4_device.hpp"
#include "launch.hpp"

namespace q4 {

// Waves per workgroup: 8, or 4 for matrices of at most 4 passes per CU.
constexpr int kSegWaves = 8;

// Staging unit: chunk jj of slot t for column b = 64 bytes of X (4 windows).
// One thread permutes the unit's windows and sums its 32 activations in the
// fixed chunk_xsum order.
template <int LPR, int BT, int NW>
struct SegStage {
    static constexpr int kThreads = 64 * NW;
    static constexpr int kUnits = BT * LPR;
    static constexpr int kPerThread = (kUnits + kThreads - 1) / kThreads;
    u4 v[kPerThread][4];
};

template <int LPR, int BT, int NW>
__device__ __forceinline__ void seg_issue(SegStage<LPR, BT, NW>& S, const uint16_t* __restrict__ X, int k, int nb,
                                          int t, bool live) {
    using St = SegStage<LPR, BT, NW>;
    const int C = k >> 5;
    const u4* xv = reinterpret_cast<const u4*>(X);
#pragma unroll
    for (int i = 0; i < St::kPerThread; ++i) {
        const int u = (int)threadIdx.x + i * St::kThreads;
        const int b = u / LPR;
        const int c = t * LPR + (u % LPR);
        // Chunks past C load the last chunk (in range) and are zeroed when
        // stored.  Units that are not stored (columns past nb, unit numbers
        // past the slot, slots past the row) all load window 0 of column 0:
        // one cache line per instruction, and no branch, so that every slot
        // issues the same loads and the compiler can count them.
        const int cc = c < C ? c : C - 1;
        const bool real = live && u < St::kUnits && b < nb;
        const size_t off = real ? (size_t)b * (size_t)(k >> 3) + (size_t)cc * 4 : 0;
#pragma unroll
        for (int d = 0; d < 4; ++d) S.v[i][d] = xv[off + (real ? d : 0)];
    }
}

// LDS buffer: windows [BT][4][LPR] (16 bytes each), then sums [BT][LPR].
template <int LPR, int BT, int NW>
__device__ __forceinline__ void seg_store(const SegStage<LPR, BT, NW>& S, u4* __restrict__ xq,
                                          float* __restrict__ xsm, int k, int nb, int t) {
    using St = SegStage<LPR, BT, NW>;
    const int C = k >> 5;
#pragma unroll
    for (int i = 0; i < St::kPerThread; ++i) {
        const int u = (int)threadIdx.x + i * St::kThreads;
        if (u < St::kUnits) {
            const int b = u / LPR;
            const int jj = u % LPR;
            const uint32_t keep = (b < nb && t * LPR + jj < C) ? 0xFFFFFFFFu : 0u;
            h2 xp[16];
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                u4 w = S.v[i][d];
                w.x &= keep;
                w.y &= keep;
                w.z &= keep;
                w.w &= keep;
                w = permute_window(w);
                xq[(b * 4 + d) * LPR + jj] = w;
                xp[4 * d + 0] = as_h2(w.x);
                xp[4 * d + 1] = as_h2(w.y);
                xp[4 * d + 2] = as_h2(w.z);
                xp[4 * d + 3] = as_h2(w.w);
            }
            xsm[b * LPR + jj] = chunk_xsum(xp);
        }
    }
}

struct SegWeights {
    u4 q;
    uint16_t s;
    uint16_t m;
};

// A slot past the row (live = false) loads chunk 0 of row 0 on every lane.
__device__ __forceinline__ void seg_weights(SegWeights& W, const uint8_t* __restrict__ packed,
                                            const uint16_t* __restrict__ scales,
                                            const uint16_t* __restrict__ mins, int rowc, int k, int c,
                                            bool live) {
    const int C = k >> 5;
    const int cc = c < C ? c : C - 1;
    const size_t q = live ? (size_t)rowc * (size_t)(k >> 5) + (size_t)cc : 0;
    const size_t g = live ? (size_t)rowc * (size_t)(k >> 7) + (size_t)(cc >> 2) : 0;
    W.q = __builtin_nontemporal_load(reinterpret_cast<const u4*>(packed) + q);
    W.s = scales[g];
    W.m = mins[g];
}

template <int LPR, int BT, int R, int NW>
__global__ void __launch_bounds__(64 * NW)
gemm_seg_kernel(const uint8_t* __restrict__ packed, const uint16_t* __restrict__ scales,
                const uint16_t* __restrict__ mins, const uint16_t* __restrict__ X, float* __restrict__ Y,
                int n, int k, int nb) {
    constexpr int RPW = 64 / LPR;
    constexpr int kBufU4 = BT * 4 * LPR + BT * LPR / 4;  // windows, then fp32 sums
    extern __shared__ u4 lds[];
    const int C = k >> 5;
    const int slots = (C + LPR - 1) / LPR;
    const int lane = (int)threadIdx.x & 63;
    const int wave = (int)threadIdx.x >> 6;
    const int j = lane % LPR;
    int row[R], rowc[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        row[r] = (((int)blockIdx.x * NW + wave) * R + r) * RPW + lane / LPR;
        rowc[r] = row[r] < n ? row[r] : n - 1;
    }

    float y[R][BT];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int b = 0; b < BT; ++b) y[r][b] = 0.0f;

    // D slots in flight (D = 2 for slots of at most 512 units, 32 KB of
    // activations per workgroup; 1 above, where twice the staging in flight
    // measured slower: 64 lanes x 16 columns, 22.6 against 20.9 us at
    // 2,048 x 11,008).  Ring entry `par` holds the weights and staged
    // activations of the slots congruent to par mod 2.  Step t requests slot
    // t + D, consumes slot t, then stores slot t + 1 (requested D - 1 steps
    // earlier) to LDS, so each load has D steps of arithmetic to arrive.
    constexpr int D = BT * LPR <= 512 ? 2 : 1;
    SegWeights W[2][R];
    SegStage<LPR, BT, NW> S[2];
    auto issue_slot = [&](int par, int sl) {
        const bool live = sl < slots;
#pragma unroll
        for (int r = 0; r < R; ++r) seg_weights(W[par][r], packed, scales, mins, rowc[r], k, sl * LPR + j, live);
        seg_issue<LPR, BT, NW>(S[par], X, k, nb, sl, live);
    };
    auto store_slot = [&](int par, int sl) {
        u4* q = lds + par * kBufU4;
        seg_store<LPR, BT, NW>(S[par], q, reinterpret_cast<float*>(q + BT * 4 * LPR), k, nb, sl);
    };
    auto step = [&](int par, int t) {
        h2 codes[R][16];
        uint16_t sc[R], mc[R];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            chunk_codes(W[par][r].q, codes[r]);
            sc[r] = W[par][r].s;
            mc[r] = W[par][r].m;
        }
        issue_slot(D == 2 ? par : par ^ 1, t + D);
        const u4* xq = lds + par * kBufU4 + j;
        const float* xsm = reinterpret_cast<const float*>(lds + par * kBufU4 + BT * 4 * LPR) + j;
        // One column's windows and sum are read one column ahead of their
        // use, and each column's results are pinned before the next column:
        // otherwise the compiler hoists every column's reads and runs out of
        // registers.
        u4 w[2][4];
        float xs[2];
        auto read_col = [&](int slot, int b) {
#pragma unroll
            for (int d = 0; d < 4; ++d) w[slot][d] = xq[(b * 4 + d) * LPR];
            xs[slot] = xsm[b * LPR];
        };
        read_col(0, 0);
#pragma unroll
        for (int b = 0; b < BT; ++b) {
            if (b + 1 < BT) read_col((b + 1) & 1, b + 1);
            h2 xp[16];
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                xp[4 * d + 0] = as_h2(w[b & 1][d].x);
                xp[4 * d + 1] = as_h2(w[b & 1][d].y);
                xp[4 * d + 2] = as_h2(w[b & 1][d].z);
                xp[4 * d + 3] = as_h2(w[b & 1][d].w);
            }
#pragma unroll
            for (int r = 0; r < R; ++r) {
                y[r][b] = group_update(y[r][b], sc[r], mc[r], chunk_dot(codes[r], xp), xs[b & 1]);
                asm volatile("" : "+v"(y[r][b]));
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        if (t + 1 < slots) store_slot(par ^ 1, t + 1);
        lds_barrier();
    };

    issue_slot(0, 0);
    if (D == 2) issue_slot(1, 1);
    store_slot(0, 0);
    lds_barrier();
    // The odd last slot is peeled: a conditional second step would join two
    // paths at the loop head, where the compiler then waits for every load.
    int t = 0;
    for (; t + 1 < slots; t += 2) {
        step(0, t);
        step(1, t + 1);
    }
    if (t < slots) step(0, t);

#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int b = 0; b < BT; ++b) {
            const float v = reduce_lanes<LPR>(y[r][b]) * kInvUnit;
            if (j == 0 && row[r] < n && b < nb) Y[(size_t)b * (size_t)n + row[r]] = v;
        }
}

template <int LPR, int BT, int R, int NW>
static hipError_t launch_seg(const GemvArgs& a, const uint16_t* X, float* Y, int nb, const DeviceInfo& dev,
                             hipStream_t st) {
    constexpr int RPW = 64 / LPR;
    const size_t lds = 2 * ((size_t)BT * 4 * LPR * 16 + (size_t)BT * LPR * 4);
    if (lds > dev.max_lds) return hipErrorNotSupported;
    std::atomic<int>& attr_set = PerDevice<&gemm_seg_kernel<LPR, BT, R, NW>>::value[dev.device];
    if (attr_set.load(std::memory_order_acquire) == 0) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&gemm_seg_kernel<LPR, BT, R, NW>),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)dev.max_lds);
        if (e != hipSuccess) return e;
        attr_set.store(1, std::memory_order_release);
    }
    const long passes = ((long)a.n + RPW - 1) / RPW;
    const long per_block = (long)NW * R;
    const long grid = (passes + per_block - 1) / per_block;
    hipLaunchKernelGGL((gemm_seg_kernel<LPR, BT, R, NW>), dim3((unsigned)grid), dim3(64 * NW), lds, st, a.packed,
                       a.scales, a.mins, X, Y, a.n, a.k, nb);
    return hipGetLastError();
}

// One workgroup per CU (the staging buffers allow one at 16 columns) and one
// pass per wave where possible: 4 waves per workgroup up to 4 passes per CU,
// 8 up to 8, 12 up to 12; beyond, two passes per wave in 8-wave workgroups,
// where each column read from LDS serves two rows.  At 8 to 12 passes per CU,
// 12 waves of one pass measured 15-20% faster than 8 waves of two (3,072 x
// 8,192 at B = 16: 17.3 against 20.8 us); at 16 passes per CU, 16 waves of one
// were slower than 8 of two (4,096 x 11,008: 30.2 against 28.6 us).
template <int LPR, int BT>
static hipError_t launch_seg_rows(const GemvArgs& a, const uint16_t* X, float* Y, int nb, const DeviceInfo& dev,
                                  hipStream_t st) {
    constexpr int RPW = 64 / LPR;
    const long passes = ((long)a.n + RPW - 1) / RPW;
    if (passes > (long)kSegWaves * dev.num_cu && passes <= 12L * dev.num_cu)
        return launch_seg<LPR, BT, 1, 12>(a, X, Y, nb, dev, st);
    if (passes > (long)kSegWaves * dev.num_cu) return launch_seg<LPR, BT, 2, kSegWaves>(a, X, Y, nb, dev, st);
    if (passes <= (long)(kSegWaves / 2) * dev.num_cu) return launch_seg<LPR, BT, 1, kSegWaves / 2>(a, X, Y, nb, dev, st);
    return launch_seg<LPR, BT, 1, kSegWaves>(a, X, Y, nb, dev, st);
}

template <int LPR>
static hipError_t dispatch_seg_bt(int bt, const GemvArgs& a, const uint16_t* X, float* Y, int nb,
                                  const DeviceInfo& dev, hipStream_t st) {
    switch (bt) {
        case 2: return launch_seg_rows<LPR, 2>(a, X, Y, nb, dev, st);
        case 4: return launch_seg_rows<LPR, 4>(a, X, Y, nb, dev, st);
        case 8: return launch_seg_rows<LPR, 8>(a, X, Y, nb, dev, st);
        case 12: return launch_seg_rows<LPR, 12>(a, X, Y, nb, dev, st);
        case 16: return launch_seg_rows<LPR, 16>(a, X, Y, nb, dev, st);
    }
    return hipErrorNotSupported;
}

hipError_t launch_small_batch_segmented(const GemvArgs& a, const uint16_t* X, float* Y, int b,
                                        const DeviceInfo& dev, hipStream_t st) {
    // Column slots: 2, 4, 8, 12 or 16 (columns past b are zero and not stored).
    int bt = 2;
    while (bt < b) bt <<= 1;
    if (b > 8 && b <= 12) bt = 12;
    switch (lanes_per_row(a.k)) {
        case 64: return dispatch_seg_bt<64>(bt, a, X, Y, b, dev, st);
        case 32: return dispatch_seg_bt<32>(bt, a, X, Y, b, dev, st);
        case 16: return dispatch_seg_bt<16>(bt, a, X, Y, b, dev, st);
    }
    return hipErrorNotSupported;
}

}  // namespace q4
