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
//     exact sum of the survivals ranked before (64 thread groups per slot count over a
//     share of the words each), so S_rank needs no scan; then f(rank) and f(rank+1),
//     i.e. every B the argmax and the first-drop rule look at, order / sorted_surv and
//     the workgroup's best candidates into the workspace;
//   sched_finish_kernel, one workgroup: the budget from every workgroup's candidates,
//     then the allocation.
// f(B) is computed from the same exact integer S_B and the same rounding as in the
// one-workgroup kernel, so B* and f(B*) are the same doubles.

constexpr int kWT = 256;                     // threads of the finish workgroup
constexpr int kWR = 512;                     // threads of a ranking workgroup
constexpr int kWRParts = kWR / kWideSlots;   // thread groups counting for one slot
constexpr int kNone = 0x7FFFFFFF;

struct WidePartial {  // kWidePartialBytes
    double f;      // largest f(B) among this workgroup's B
    double fdrop;  // f at the drop below
    double fbmax;  // f(bmax), if this workgroup evaluated it
    int32_t B;     // the smallest B reaching f
    int32_t drop;  // the smallest B with f(B+1) <= f(B) among this workgroup's slots, or kNone
    int32_t has_fbmax;
    int32_t pad[3];
};
static_assert(sizeof(WidePartial) == kWidePartialBytes, "the workspace holds kWidePartialBytes per workgroup");

__device__ __forceinline__ WidePartial no_partial() {
    WidePartial p;
    p.f = -INFINITY;
    p.fdrop = 0.0;
    p.fbmax = 0.0;
    p.B = kNone;
    p.drop = kNone;
    p.has_fbmax = 0;
    p.pad[0] = p.pad[1] = p.pad[2] = 0;
    return p;
}

// a takes over b's candidates where they are better (argmax: larger f, then smaller B;
// first drop: smaller B; f(bmax) from whichever has it)
__device__ __forceinline__ void merge_partial(WidePartial& a, const WidePartial& b) {
    if (b.f > a.f || (b.f == a.f && b.B < a.B)) {
        a.f = b.f;
        a.B = b.B;
    }
    if (b.drop < a.drop) {
        a.drop = b.drop;
        a.fdrop = b.fdrop;
    }
    if (b.has_fbmax) {
        a.fbmax = b.fbmax;
        a.has_fbmax = 1;
    }
}

struct RankShared {
    uint64_t word[kWideMaxN];    // slot words in flat order
    uint64_t fa[kWideMaxN], fb[kWideMaxN], fc[kWideMaxN];  // each slot's survival, exact (units of 2^-149)
    float vc[kWideMaxN + 1];     // vc[T + B], B = 0 .. bmax
    uint32_t wcnt[kWR / 64][kWideSlots];
    U192 wsum[kWR / 64][kWideSlots];
    WidePartial part[kWideSlots];
};

__device__ __forceinline__ U192 shfl_xor_192(const U192& x, int m) {
    return U192{shfl_xor_u64(x.a, m), shfl_xor_u64(x.b, m), shfl_xor_u64(x.c, m)};
}

__global__ __launch_bounds__(kWR) void sched_rank_kernel(
    const float* __restrict__ conf, int R, int K, int n_sampling, int T, int num_reqs, const float* __restrict__ vc,
    const float* __restrict__ dc, int bmax, float* __restrict__ surv_out, int32_t* __restrict__ order,
    float* __restrict__ sorted_surv, uint32_t* status, unsigned char* __restrict__ ws) {
    __shared__ RankShared sh;
    const int tid = threadIdx.x, g = blockIdx.x;
    const int n = R * K;
    WidePartial* parts = reinterpret_cast<WidePartial*>(ws);
    int32_t* rank_of = reinterpret_cast<int32_t*>(ws + (size_t)kWideMaxGroups * kWidePartialBytes);

    // survival of every slot (each thread one request at a time, eight confidences per
    // memory round trip), and the cost-table entries B = 0 .. bmax, all requested before
    // the first is used
    constexpr int kVq = kWideMaxN / kWR + 1;
    float vq[kVq];
#pragma unroll
    for (int u = 0; u < kVq; ++u) vq[u] = tid + u * kWR <= bmax ? vc[T + tid + u * kWR] : 0.f;
    const float dcost_f = dc[num_reqs];
    bool bad = false;
    for (int r = tid; r < R; r += kWR) {
        const int f0 = r * K;
        float s = 0.f;
        for (int i0 = 0; i0 < K; i0 += 8) {
            float c[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) c[u] = i0 + u < K ? conf[f0 + i0 + u] : 0.f;
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int i = i0 + u;
                if (i < K) {
                    const float cu = sanitize_conf(c[u], bad);
                    s = (i == 0) ? cu : s * cu;
                    sh.word[f0 + i] = slot_word(kOne - __float_as_uint(s), f0 + i);
                    const U192 fs = fixed_from_bits(__float_as_uint(s));
                    sh.fa[f0 + i] = fs.a;
                    sh.fb[f0 + i] = fs.b;
                    sh.fc[f0 + i] = fs.c;
                    if (g == 0 && surv_out) surv_out[f0 + i] = s;
                }
            }
        }
    }
    if (bad && g == 0) raise_status(status, kStatusConfSanitized);
#pragma unroll
    for (int u = 0; u < kVq; ++u)
        if (tid + u * kWR <= bmax) sh.vc[tid + u * kWR] = vq[u];
    __syncthreads();

    // this workgroup's slots: thread (el, pt) counts slot 8g + el over words [y0, y1)
    const int el = tid % kWideSlots, pt = tid / kWideSlots;
    const int x = g * kWideSlots + el;
    const int lane = tid & 63, w = tid >> 6;
    uint32_t cnt = 0u;
    U192 S = {0ull, 0ull, 0ull};
    if (x < n) {
        const uint64_t wx = sh.word[x];
        const int y0 = (int)(((long)pt * n) / kWRParts), y1 = (int)(((long)(pt + 1) * n) / kWRParts);
        int y = y0;
        for (; y + 4 <= y1; y += 4) {  // four words' reads in flight together
            uint64_t wy[4], a[4], b[4], c[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                wy[u] = sh.word[y + u];
                a[u] = sh.fa[y + u];
                b[u] = sh.fb[y + u];
                c[u] = sh.fc[y + u];
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const bool lt = wy[u] < wx;
                cnt += lt ? 1u : 0u;
                S = add192(S, lt ? U192{a[u], b[u], c[u]} : U192{0ull, 0ull, 0ull});
            }
        }
        for (; y < y1; ++y) {
            const bool lt = sh.word[y] < wx;
            cnt += lt ? 1u : 0u;
            S = add192(S, lt ? U192{sh.fa[y], sh.fb[y], sh.fc[y]} : U192{0ull, 0ull, 0ull});
        }
    }
    // the wave's eight groups of each slot (lanes el, el + 8, ..., el + 56), then the waves
#pragma unroll
    for (int m = 8; m < 64; m <<= 1) {
        cnt += (uint32_t)__shfl_xor((int)cnt, m, 64);
        S = add192(S, shfl_xor_192(S, m));
    }
    if (lane < kWideSlots) {
        sh.wcnt[w][lane] = cnt;
        sh.wsum[w][lane] = S;
    }
    __syncthreads();
    if (tid < kWideSlots) {
        WidePartial p = no_partial();
        if (x < n) {
            uint32_t rk = 0u;
            U192 Sx = {0ull, 0ull, 0ull};
#pragma unroll
            for (int q = 0; q < kWR / 64; ++q) {
                rk += sh.wcnt[q][tid];
                Sx = add192(Sx, sh.wsum[q][tid]);
            }
            const int r = (int)rk;
            const uint64_t wx = sh.word[x];
            if (order) order[r] = x;
            if (sorted_surv) sorted_surv[r] = __uint_as_float(kOne - word_key(wx));
            rank_of[x] = r;
            const double dcost = (double)dcost_f;
            const uint64_t ns_hi = (uint64_t)(uint32_t)n_sampling << 21;  // n_sampling * 2^149
            bool badc = false;
            auto eval = [&](const U192& s_excl, float vcost) -> double {
                U192 X = s_excl;
                X.c += ns_hi;
                const double num = fixed_to_double(X);
                const double den = (double)vcost + dcost;
                if (den > 0.0 && den <= 1.7976931348623157e308) return num / den;
                badc = true;
                return -INFINITY;
            };
            // f(r) and f(r+1): the argmax candidate B = r + 1 (and B = 0 from rank 0), the
            // first-drop test at B = r, and f(bmax) from whichever slot evaluates it
            if (r <= bmax) {
                const double fr = eval(Sx, sh.vc[r]);
                if (r == 0) {
                    p.f = fr;
                    p.B = 0;
                    if (bmax == 0) {
                        p.fbmax = fr;
                        p.has_fbmax = 1;
                    }
                }
                if (r + 1 <= bmax) {
                    const double f1 = eval(add192(Sx, U192{sh.fa[x], sh.fb[x], sh.fc[x]}), sh.vc[r + 1]);
                    if (f1 > p.f || (f1 == p.f && r + 1 < p.B)) {
                        p.f = f1;
                        p.B = r + 1;
                    }
                    if (!(f1 > fr)) {
                        p.drop = r;
                        p.fdrop = fr;
                    }
                    if (r + 1 == bmax) {
                        p.fbmax = f1;
                        p.has_fbmax = 1;
                    }
                }
            }
            if (badc) raise_status(status, kStatusCostInvalid);
        }
        sh.part[tid] = p;
    }
    __syncthreads();
    if (tid == 0) {
        WidePartial q = sh.part[0];
        for (int e = 1; e < kWideSlots; ++e) merge_partial(q, sh.part[e]);
        parts[g] = q;
    }
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
    hipLaunchKernelGGL(sched_rank_kernel, dim3(G), dim3(kWR), 0, s, a.conf, a.R, a.K, a.n_sampling, a.T, a.num_reqs,
                       a.vc, a.dc, a.bmax, a.surv, a.order, a.sorted_surv, a.status, ws);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(sched_finish_kernel, dim3(1), dim3(kWT), 0, s, a.R, a.K, G, a.bmax, a.sizing.rule, a.b_star,
                       a.best_obj, a.prefix_len, a.offsets, a.ver_idx, ws, a.tokens, a.ver_tokens);
    return hipGetLastError();
}

}  // namespace dspark
