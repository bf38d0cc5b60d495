// The whole chain-and-schedule step in ONE launch of a resident grid.
//
// Stages 2-5 (survival, ranking, budget, allocation; vLLM blog "Adaptive
// Verification in vLLM", sections "Scheduling the budget" and "The cost model")
// depend only on the confidences, stage 1 (the chain; DSpark summary "How DSpark
// Speeds Up LLM Inference", section "Draft better") only on the drafter outputs, so
// they run side by side: the grid is one workgroup per vocabulary tile for the
// chain plus one more workgroup that schedules.  The vocabulary tiles leave a few
// CUs free, so the schedule costs no chain time, and the step pays for one launch
// instead of three.
//
// The extra workgroup also
//   * zeroes the argmax keys first and then raises a ready flag, which the chain
//     workgroups wait for before their first key atomics;
//   * waits for the chain's last barrier, puts the step counters and the flag back to
//     zero (no chain workgroup reads them any more: every one has passed its last wait
//     once the last barrier is full), so the next launch starts from zero, and writes
//     tokens [R, K] and the verified tokens ver_tokens[j] = tokens[ver_idx[j]] (j < B*,
//     -1 after) in one pass over the keys (agent-scope loads).
// Like the chain's own exchanges, these go through agent-scope atomics that return
// a value, completed before the flag or counter that publishes them.
#include "chain_dev.h"
#include "sched_dev.h"

namespace dspark {

namespace {

template <int KS>
struct StepLds {
    static constexpr size_t kChain = sizeof(ChainLds<KS>);
    static constexpr size_t kSched = sizeof(SchedShared<kNT>);
    static constexpr size_t kBytes = kChain > kSched ? kChain : kSched;
};

__device__ __forceinline__ void zero_agent_u64(uint64_t* p) {
    const uint64_t old = __hip_atomic_exchange(p, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    asm volatile("" ::"v"(old));
}

__device__ __forceinline__ void set_agent_u32(uint32_t* p, uint32_t v) {
    const uint32_t old = __hip_atomic_exchange(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    asm volatile("" ::"v"(old));
}

__device__ __forceinline__ int32_t token_of(const uint64_t* keys, int R, int K, int f) {
    const int r = f / K, i = f - r * K;
    return key_index(load_agent_u64(&keys[(size_t)i * R + r]));
}

template <int KS, bool VEC>
__global__ __launch_bounds__(kNT, 1) void step_single_bf16_kernel(StepArgs a) {
    __shared__ __attribute__((aligned(16))) unsigned char smem[StepLds<KS>::kBytes];
    const int G = (int)gridDim.x - 1;  // chain workgroups
    uint32_t* bar = a.sync;            // bar[p] counts the chain workgroups done with position p
    uint32_t* ready = a.sync + a.K * kMaxGroups;
    if ((int)blockIdx.x < G) {
        chain_persist_body<KS, VEC>(*reinterpret_cast<ChainLds<KS>*>(smem), (const uint16_t*)a.base,
                                    (const uint16_t*)a.A, (const uint16_t*)a.Bt, a.prev0, a.keys, bar, nullptr,
                                    a.status, a.R, a.K, a.V, a.rank, G, ready);
        return;
    }
    SchedShared<kNT>& sh = *reinterpret_cast<SchedShared<kNT>*>(smem);
    const int n = a.R * a.K;
    for (int j = threadIdx.x; j < n; j += kNT) zero_agent_u64(&a.keys[j]);
    __builtin_amdgcn_s_waitcnt(0);  // every exchange has returned
    __syncthreads();
    if (threadIdx.x == 0) set_agent_u32(ready, 1u);
    int32_t* lds_rows = reinterpret_cast<int32_t*>(sh.key);  // per request: offset, prefix length
    const Sizing sz{a.sizing.separate, a.sizing.conf, a.sizing.R, a.sizing.bmax, a.sizing.rule};
    sched_pass<kNT>(sh, a.conf, a.R, a.K, a.n_sampling, a.T, a.num_reqs, a.vc, a.dc, a.bmax, sz, a.surv, a.order,
                    a.sorted_surv, a.b_star, a.best_obj, a.prefix_len, a.offsets, a.ver_idx, a.status, lds_rows);
    __syncthreads();
    // each chain workgroup arrives for the groups of a position in order
    grid_wait(&bar[(a.K - 1) * kMaxGroups + group_count(a.R) - 1], (uint32_t)G, a.status);
    // Every chain workgroup has passed its last wait: the counters and the flag go back
    // to zero for the next launch, while the tokens are decoded.
    for (int p = threadIdx.x; p < a.K * kMaxGroups; p += kNT) set_agent_u32(&bar[p], 0u);
    if (threadIdx.x == 0) set_agent_u32(ready, 0u);
    // One pass over the keys: tokens[r, i], and ver_tokens[offset_r + i] for the i below
    // request r's prefix length (the verified slots are each request's first ones).
    const int B = sh.b_star;
    for (int f = threadIdx.x; f < n; f += kNT) {
        const int r = f / a.K, i = f - r * a.K;
        const int32_t tok = token_of(a.keys, a.R, a.K, f);
        a.tokens[f] = tok;
        if (a.ver_tokens != nullptr && i < lds_rows[2 * r + 1]) a.ver_tokens[lds_rows[2 * r] + i] = tok;
    }
    if (a.ver_tokens != nullptr)
        for (int j = B + threadIdx.x; j < n; j += kNT) a.ver_tokens[j] = -1;
}

template <int KS, bool VEC>
hipError_t launch_single(const StepArgs& a, int grid, hipStream_t s) {
    const void* fn = (const void*)step_single_bf16_kernel<KS, VEC>;
    static int resident[64] = {0};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= 64) return hipErrorCooperativeLaunchTooLarge;
    if (resident[dev] == 0) {
        int per_cu = 0, cus = 0;
        if ((e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, kNT, 0)) != hipSuccess) return e;
        if ((e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess) return e;
        resident[dev] = per_cu * cus > 0 ? per_cu * cus : -1;
    }
    if (grid > resident[dev]) return hipErrorCooperativeLaunchTooLarge;
    if (!a.coop) {
        hipLaunchKernelGGL((step_single_bf16_kernel<KS, VEC>), dim3(grid), dim3(kNT), 0, s, a);
        return hipGetLastError();
    }
    StepArgs arg = a;
    void* args[] = {&arg};
    return hipLaunchCooperativeKernel(fn, dim3(grid), dim3(kNT), args, 0, s);
}

template <int KS>
hipError_t launch_single_ks(const StepArgs& a, int grid, hipStream_t s) {
    if (a.V % 8 == 0) return launch_single<KS, true>(a, grid, s);
    return launch_single<KS, false>(a, grid, s);
}

}  // namespace

hipError_t launch_step_single(const StepArgs& a, hipStream_t s) {
    if (a.R < 1 || a.R > kReqChunk || a.K < 1) return hipErrorCooperativeLaunchTooLarge;
    const int grid = (a.V + kTileV - 1) / kTileV + 1;  // vocabulary tiles + the scheduling workgroup
    const int ks = (a.rank + 31) / 32;
    if (ks <= 1) return launch_single_ks<1>(a, grid, s);
    if (ks <= 2) return launch_single_ks<2>(a, grid, s);
    if (ks <= 4) return launch_single_ks<4>(a, grid, s);
    return launch_single_ks<8>(a, grid, s);
}

}  // namespace dspark
