// Kernels of stages 2-5 (vLLM blog "Adaptive Verification in vLLM", sections
// "Scheduling the budget" and "The cost model"): the fused pass and the stage-wise
// entry points, each ONE workgroup of 1024 threads out of LDS (n = R*K <= 16384
// slots).  The pages keep this work on the GPU with no host read-back, and at these
// sizes a single CU with 160 KB of LDS avoids every grid-wide synchronisation.  The
// device code (sched_dev.h) also runs inside the single-launch step kernel.
#include "kernels.h"
#include "sched_dev.h"

namespace dspark {

namespace {

constexpr int kST = 1024;  // scheduler threads

__global__ __launch_bounds__(kST, 1) void sched_fused_kernel(
    const float* __restrict__ conf, int R, int K, int n_sampling, int T, int num_reqs,
    const float* __restrict__ vc, const float* __restrict__ dc, int bmax, SizingArgs sizing, float* __restrict__ surv_out,
    int32_t* __restrict__ order, float* __restrict__ sorted_surv, int32_t* __restrict__ b_star,
    double* __restrict__ best_obj, int32_t* __restrict__ prefix_len, int32_t* __restrict__ offsets,
    int32_t* __restrict__ ver_idx, uint32_t* status, uint64_t* __restrict__ ws, int ws_words,
    const int32_t* __restrict__ tokens, int32_t* __restrict__ ver_tokens) {
    __shared__ SchedShared<kST> sh;
    // The chain's workspace (argmax keys, barrier counters) starts from zero; this launch
    // precedes the chain kernels on the stream.
    for (int j = threadIdx.x; j < ws_words; j += kST) ws[j] = 0ull;
    const Sizing sz{sizing.separate, sizing.conf, sizing.R, sizing.bmax, sizing.rule};
    sched_pass<kST>(sh, conf, R, K, n_sampling, T, num_reqs, vc, dc, bmax, sz, surv_out, order, sorted_surv, b_star,
                    best_obj, prefix_len, offsets, ver_idx, status, nullptr, tokens, ver_tokens);
}

__global__ __launch_bounds__(256) void survival_kernel(const float* __restrict__ conf, int R, int K,
                                                        float* __restrict__ surv, uint32_t* status) {
    const int r = blockIdx.x * blockDim.x + threadIdx.x;
    bool bad = false;
    if (r < R) {
        float s = 0.f;
        for (int i = 0; i < K; ++i) {
            const float c = sanitize_conf(conf[(size_t)r * K + i], bad);
            s = (i == 0) ? c : s * c;
            surv[(size_t)r * K + i] = s;
        }
    }
    if (bad) raise_status(status, kStatusConfSanitized);
}

__global__ __launch_bounds__(kST, 1) void topb_kernel(const float* __restrict__ surv, int R, int K,
                                                     int32_t* __restrict__ order, float* __restrict__ sorted_surv,
                                                     int32_t* __restrict__ rank) {
    __shared__ SchedShared<kST> sh;
    const int n = R * K;
    surv_global_to_lds<kST>(sh, surv, n);
    const uint64_t* rk = rank_slots<kST>(sh, n, 1);  // the survivals may come in any order
    write_ranking<kST>(rk, n, order, sorted_surv, rank);
}

__global__ __launch_bounds__(kST, 1) void budget_kernel(const float* __restrict__ sorted_surv, int n, int n_sampling,
                                                       int T, int num_reqs, const float* __restrict__ vc,
                                                       const float* __restrict__ dc, int bmax, int rule,
                                                       int32_t* __restrict__ b_star, double* __restrict__ best_obj,
                                                       double* __restrict__ obj, uint32_t* status) {
    __shared__ SchedShared<kST> sh;
    const int n_pad = pad_slots<kST>(n);
    CostPrefetch cp;
    prefetch_costs<kST>(cp, vc, dc, T, num_reqs, bmax, n_pad);
    for (int j = threadIdx.x; j < n; j += kST) {
        bool bad = false;
        sh.item[j] = slot_word(kOne - __float_as_uint(sanitize_conf(sorted_surv[j], bad)), 0);
    }
    __syncthreads();
    choose_budget_lds<kST>(sh, sh.item, cp, vc + T, n, n_pad, n_sampling, bmax, rule, b_star, best_obj, obj, status);
}

__global__ __launch_bounds__(kST, 1) void allocate_kernel(const int32_t* __restrict__ order,
                                                         const int32_t* __restrict__ b_star, int R, int K,
                                                         const int32_t* __restrict__ tokens,
                                                         int32_t* __restrict__ prefix_len,
                                                         int32_t* __restrict__ offsets, int32_t* __restrict__ ver_idx,
                                                         int32_t* __restrict__ ver_tokens) {
    __shared__ SchedShared<kST> sh;
    const int n = R * K;
    int B = *b_star;
    B = B < 0 ? 0 : (B > n ? n : B);
    uint8_t* sel = selection_map<kST>(sh);
    for (int f = threadIdx.x; f < n; f += kST) sel[f] = 0;
    __syncthreads();
    for (int j = threadIdx.x; j < B; j += kST) {
        const int f = order[j];
        if (f >= 0 && f < n) sel[f] = 1;
    }
    __syncthreads();
    allocate_lds<kST>(sh, sel, R, K, B, tokens, prefix_len, offsets, ver_idx, ver_tokens);
}

}  // namespace

hipError_t launch_survival(const float* conf, int R, int K, float* surv, uint32_t* status, hipStream_t s) {
    hipLaunchKernelGGL(survival_kernel, dim3((R + 255) / 256), dim3(256), 0, s, conf, R, K, surv, status);
    return hipGetLastError();
}

hipError_t launch_topb(const float* surv, int R, int K, int32_t* order, float* sorted_surv, int32_t* rank,
                       hipStream_t s) {
    hipLaunchKernelGGL(topb_kernel, dim3(1), dim3(kST), 0, s, surv, R, K, order, sorted_surv, rank);
    return hipGetLastError();
}

hipError_t launch_budget(const BudgetArgs& a, hipStream_t s) {
    hipLaunchKernelGGL(budget_kernel, dim3(1), dim3(kST), 0, s, a.sorted_surv, a.n, a.n_sampling, a.T, a.num_reqs,
                       a.vc, a.dc, a.bmax, a.rule, a.b_star, a.best_obj, a.obj, a.status);
    return hipGetLastError();
}

hipError_t launch_allocate(const int32_t* order, const int32_t* b_star, int R, int K, const int32_t* tokens,
                           int32_t* prefix_len, int32_t* offsets, int32_t* ver_idx, int32_t* ver_tokens,
                           hipStream_t s) {
    hipLaunchKernelGGL(allocate_kernel, dim3(1), dim3(kST), 0, s, order, b_star, R, K, tokens, prefix_len, offsets,
                       ver_idx, ver_tokens);
    return hipGetLastError();
}

hipError_t launch_sched_fused(const FusedSchedArgs& a, hipStream_t s) {
    hipLaunchKernelGGL(sched_fused_kernel, dim3(1), dim3(kST), 0, s, a.conf, a.R, a.K, a.n_sampling, a.T,
                       a.num_reqs, a.vc, a.dc, a.bmax, a.sizing, a.surv, a.order, a.sorted_surv, a.b_star, a.best_obj,
                       a.prefix_len, a.offsets, a.ver_idx, a.status, a.ws, a.ws_words, a.tokens, a.ver_tokens);
    return hipGetLastError();
}

}  // namespace dspark
