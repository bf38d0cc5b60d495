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

// ---------------------------------------------------------------------------------
// Stages 2-5 over many workgroups, for steps of up to kWideMaxN slots sized from their
// own confidences.  One workgroup alone is bound by its CU's vector ALU (the ranking and
// the exact scan); here the work that grows with n^2 is spread over the device, in two
// launches (the boundary between them is cheaper than a device-wide fence and counter):
//   sched_rank_kernel, workgroup g: survival of all n slots into LDS (their words and
//     exact values); for slots [8g, 8g+8) the rank (the number of smaller words) and the
//     exact sum of the survivals ranked before (32 thread groups per slot count over a
//     share of the words each), so S_rank needs no scan; then f(rank) and f(rank+1),
//     i.e. every B the argmax and the first-drop rule look at, order / sorted_surv and
//     the workgroup's best candidates into the workspace;
//   sched_finish_kernel, one workgroup: the budget from every workgroup's candidates,
//     then the allocation.
// f(B) is computed from the same exact integer S_B and the same rounding as in the
// one-workgroup kernel, so B* and f(B*) are the same doubles.

constexpr int kWT = 256;                     // threads per workgroup

__global__ __launch_bounds__(kWT) void sched_rank_kernel(RankArgs a) {
    __shared__ RankShared<kWT> sh;
    rank_prepare<kWT>(sh, a);
    rank_share<kWT>(sh, a, (int)blockIdx.x);
}

__global__ __launch_bounds__(kWT) void sched_finish_kernel(
    int R, int K, int G, int bmax, int rule, int32_t* __restrict__ b_star, double* __restrict__ best_obj,
    int32_t* __restrict__ prefix_len, int32_t* __restrict__ offsets, int32_t* __restrict__ ver_idx,
    const unsigned char* __restrict__ ws, const int32_t* __restrict__ tokens, int32_t* __restrict__ ver_tokens) {
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int n = R * K;
    const WidePartial* parts = reinterpret_cast<const WidePartial*>(ws);
    const int32_t* rank_of = reinterpret_cast<const int32_t*>(ws + (size_t)kWideMaxGroups * kWidePartialBytes);
    __shared__ double s_f[kWT / 64];
    __shared__ int s_b[kWT / 64], s_d[kWT / 64];
    __shared__ double s_fdrop, s_fbmax;
    __shared__ uint32_t s_wsum[kWT / 64];
    const int CR = (R + kWT - 1) / kWT;
    const int r0 = tid * CR;
    // With one request per thread and K <= 8, its ranks and draft tokens are requested
    // with the workgroups' candidates, in the same memory round trip.
    const bool pre = CR == 1 && K <= 8 && r0 < R;
    int32_t rk8[8], tk8[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
        rk8[u] = pre && u < K ? rank_of[r0 * K + u] : kNone;
        tk8[u] = pre && u < K && ver_tokens ? tokens[r0 * K + u] : 0;
    }
    // the budget from every workgroup's candidates
    WidePartial q = tid < G ? parts[tid] : no_partial();
    const double Fw = wave_max_f64(q.f);
    const int Bw = wave_min_i32(q.f == Fw ? q.B : kNone);
    const int Dw = wave_min_i32(q.drop);
    if (lane == 0) {
        s_f[w] = Fw;
        s_b[w] = Bw;
        s_d[w] = Dw;
    }
    if (q.has_fbmax) s_fbmax = q.fbmax;  // exactly one workgroup evaluated f(bmax)
    __syncthreads();
    double F = s_f[0];
    int Bx = s_b[0], D = s_d[0];
    for (int e = 1; e < kWT / 64; ++e) {
        if (s_f[e] > F || (s_f[e] == F && s_b[e] < Bx)) {
            F = s_f[e];
            Bx = s_b[e];
        }
        D = min(D, s_d[e]);
    }
    if (tid < G && q.drop == D && D != kNone) s_fdrop = q.fdrop;  // a drop belongs to one slot
    __syncthreads();
    int B;
    double obj;
    if (rule == kRuleFirstDrop) {
        B = D != kNone ? D : bmax;
        obj = D != kNone ? s_fdrop : s_fbmax;
    } else {
        B = Bx;
        obj = F;
    }
    if (tid == 0) {
        if (b_star) *b_star = B;
        if (best_obj) *best_obj = obj;
    }
    // the allocation: a request's selected slots are its first ones (its ranks rise
    // along its positions), so its prefix length counts its ranks below B
    uint32_t cnt = 0u;
    if (pre) {
#pragma unroll
        for (int u = 0; u < 8; ++u) cnt += rk8[u] < B ? 1u : 0u;
    } else {
        for (int e = 0; e < CR; ++e) {
            const int r = r0 + e;
            if (r < R)
                for (int i = 0; i < K; ++i) cnt += rank_of[r * K + i] < B ? 1u : 0u;
        }
    }
    const uint32_t x = wave_incl_scan_u32(cnt);
    if (lane == 63) s_wsum[w] = x;
    __syncthreads();
    uint32_t o = x - cnt, total = 0;
    for (int e = 0; e < kWT / 64; ++e) {
        if (e < w) o += s_wsum[e];
        total += s_wsum[e];
    }
    if (pre) {
        offsets[r0] = (int32_t)o;
        prefix_len[r0] = (int32_t)cnt;
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            if ((uint32_t)u < cnt) {
                ver_idx[o + u] = r0 * K + u;
                if (ver_tokens) ver_tokens[o + u] = tk8[u];
            }
        }
    } else {
        for (int e = 0; e < CR; ++e) {
            const int r = r0 + e;
            if (r >= R) break;
            uint32_t L = 0;
            for (int i = 0; i < K; ++i) L += rank_of[r * K + i] < B ? 1u : 0u;
            offsets[r] = (int32_t)o;
            prefix_len[r] = (int32_t)L;
            for (uint32_t i = 0; i < L; ++i) {
                ver_idx[o + i] = r * K + (int)i;
                if (ver_tokens) ver_tokens[o + i] = tokens[r * K + (int)i];
            }
            o += L;
        }
    }
    if (tid == 0) offsets[R] = (int32_t)total;
    for (int j = B + tid; j < n; j += kWT) {
        ver_idx[j] = -1;
        if (ver_tokens) ver_tokens[j] = -1;
    }
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

hipError_t launch_sched_wide(const FusedSchedArgs& a, hipStream_t s) {
    const int n = a.R * a.K;
    if (n <= 0 || n > kWideMaxN || a.sizing.separate || !a.ws) return hipErrorInvalidValue;
    const int G = (n + kWideSlots - 1) / kWideSlots;
    unsigned char* ws = reinterpret_cast<unsigned char*>(a.ws);
    hipLaunchKernelGGL(sched_rank_kernel, dim3(G), dim3(kWT), 0, s, rank_args(a, nullptr));
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(sched_finish_kernel, dim3(1), dim3(kWT), 0, s, a.R, a.K, G, a.bmax, a.sizing.rule, a.b_star,
                       a.best_obj, a.prefix_len, a.offsets, a.ver_idx, ws, a.tokens, a.ver_tokens);
    return hipGetLastError();
}

RankArgs rank_args(const FusedSchedArgs& a, uint32_t* claim) {
    const int n = a.R * a.K;
    return RankArgs{a.conf,  a.R,     a.K,     a.n_sampling, a.T,  a.num_reqs, a.vc,
                    a.dc,    a.bmax,  a.surv,  a.order,      a.sorted_surv, a.status,
                    reinterpret_cast<unsigned char*>(a.ws), (n + kWideSlots - 1) / kWideSlots, claim};
}

hipError_t launch_sched_finish(const FusedSchedArgs& a, hipStream_t s) {
    const int n = a.R * a.K;
    if (n <= 0 || n > kWideMaxN || a.sizing.separate || !a.ws) return hipErrorInvalidValue;
    const int G = (n + kWideSlots - 1) / kWideSlots;
    hipLaunchKernelGGL(sched_finish_kernel, dim3(1), dim3(kWT), 0, s, a.R, a.K, G, a.bmax, a.sizing.rule, a.b_star,
                       a.best_obj, a.prefix_len, a.offsets, a.ver_idx, reinterpret_cast<unsigned char*>(a.ws),
                       a.tokens, a.ver_tokens);
    return hipGetLastError();
}

}  // namespace dspark
