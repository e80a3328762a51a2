// Prompt-processing contraction in the form of the rumik-oss-1 write-up
// ("Step 8: a prefill that stays int4"): the weights stay int4, each group
// of 128 columns is unpacked on chip and contracted on the matrix cores, and
// the group's scale and minimum are applied to the result:
//
//   Y[t][n] = sum_g  scale[n][g] * C_g[t][n]  +  min[n][g] * S_g[t],
//   C_g[t][n] = sum_{k in g} code[n][k] * X[t][k]   (matrix cores, fp32),
//   S_g[t]    = sum_{k in g} X[t][k]                (fp32).
//
// This is exactly sum_k (code*scale + min) * x regrouped; no weight is ever
// rounded to fp16, so the result keeps the accuracy of the matrix-vector
// kernels (every product code*x is exact; only fp32 sums round).
//
// Routing of the form: up to 64 tokens prefill_split.hip (the waves of a
// workgroup split K; its epilogue instantiation), and in blocks of up to 64
// tokens up to 96 tokens, or more on matrices of few rows; otherwise
// prefill_pair.hip (blocks of 128 tokens, the blocks of a row slice on one
// XCD).
#include "launch.hpp"

namespace q4 {

hipError_t launch_prefill_epilogue(const GemvArgs& a, const uint16_t* X, float* Y, int m, const DeviceInfo& dev,
                                   hipStream_t st) {
    if (m <= 64 || prefill_token_blocks_pay(a.n, m, dev)) return launch_prefill_split_epilogue(a, X, Y, m, dev, st);
    // On many rows one block past a full wave of workgroups runs on its own.
    const long head = prefill_pair_head_tokens(a.n, m, dev);
    if (head > 0) {
        const hipError_t e = launch_prefill_pair_epilogue(a, X, Y, (int)head, dev, st);
        if (e != hipSuccess) return e;
        return launch_prefill_epilogue(a, X + head * (long)a.k, Y + head * (long)a.n, m - (int)head, dev, st);
    }
    return launch_prefill_pair_epilogue(a, X, Y, m, dev, st);
}

}  // namespace q4
