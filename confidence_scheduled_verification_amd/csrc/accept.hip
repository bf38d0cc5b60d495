// Greedy verification of the allocated drafts: the accepted run, the bonus token
// and the next step's prev0 (MAX worklog "DSpark on MAX", section "The kernel pass",
// item 2: under greedy decoding acceptance is a compare with the target's best
// token; DSpark summary "How DSpark Speeds Up LLM Inference", section "Context": the
// longest matching run is kept; vLLM blog "Adaptive Verification in vLLM", section
// "Scheduling the budget": one bonus token per request).
//
// One wavefront per request: lane j compares draft j with the target's entry j, a
// ballot marks the mismatches and the lowest set bit is the accepted length, so a
// request costs one load round trip for its row and one for its data, whatever its
// length.  Rows longer than 64 are walked in chunks of 64.  Four requests per
// 256-thread workgroup.
#include "common.h"
#include "kernels.h"

namespace dspark {

namespace {

constexpr int kAcceptThreads = 256;
constexpr int kReqPerBlock = kAcceptThreads / 64;

__global__ __launch_bounds__(kAcceptThreads) void accept_greedy_kernel(
    const int32_t* __restrict__ ver_tokens, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ target, int R, int K, int32_t* __restrict__ accept_len,
    int32_t* __restrict__ next_prev0, int32_t* __restrict__ out_tokens, uint32_t* status) {
    const int lane = threadIdx.x & 63;
    const int r = blockIdx.x * kReqPerBlock + (threadIdx.x >> 6);
    if (r >= R) return;
    const int o = offsets[r];
    const int L = offsets[r + 1] - o;
    const bool ok = o >= 0 && L >= 0 && L <= K && (long long)o + L <= (long long)R * K;
    int a = 0;
    int32_t bonus = -1;
    if (ok) {
        const int32_t* d = ver_tokens + o;
        const int32_t* t = target + (size_t)o + r;
        a = L;
        for (int c0 = 0; c0 < L; c0 += 64) {
            const int j = c0 + lane;
            const bool miss = j < L && d[j] != t[j];
            const uint64_t m = __ballot(miss);
            if (m) {
                a = c0 + (int)__ffsll((unsigned long long)m) - 1;
                break;
            }
        }
        bonus = t[a];
    } else if (lane == 0) {
        raise_status(status, kStatusBadAllocation);
    }
    if (lane == 0) {
        accept_len[r] = a;
        next_prev0[r] = bonus;
    }
    if (out_tokens) {
        int32_t* row = out_tokens + (size_t)r * (K + 1);
        for (int j = lane; j <= K; j += 64) row[j] = (ok && j < a) ? ver_tokens[o + j] : (j == a && ok ? bonus : -1);
    }
}

}  // namespace

hipError_t launch_accept_greedy(const int32_t* ver_tokens, const int32_t* offsets, const int32_t* target, int R,
                                int K, int32_t* accept_len, int32_t* next_prev0, int32_t* out_tokens,
                                uint32_t* status, hipStream_t s) {
    const int blocks = (R + kReqPerBlock - 1) / kReqPerBlock;
    hipLaunchKernelGGL(accept_greedy_kernel, dim3(blocks), dim3(kAcceptThreads), 0, s, ver_tokens, offsets, target,
                       R, K, accept_len, next_prev0, out_tokens, status);
    return hipGetLastError();
}

}  // namespace dspark
