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

// The scheduling workgroup of a single-launch step: G chain workgroups precede it in
// the grid; the chain's last barrier counter is bar[last_bar].  pos_bar >= 0: every
// position's barriers are passed in order, position p's last one at
// bar[p * kMaxGroups + pos_bar], so the tokens of each position are written as soon as
// it is final, while the chain runs on, and only the last position's wait for the end.
__device__ __forceinline__ void step_schedule_wg(const StepArgs& a, unsigned char* smem, int G, int last_bar,
                                                 int pos_bar = -1) {
    uint32_t* bar = a.sync;
    uint32_t* ready = a.sync + a.K * kMaxGroups;
    SchedShared<kNT>& sh = *reinterpret_cast<SchedShared<kNT>*>(smem);
    const int n = a.R * a.K;
    for (int j = threadIdx.x; j < n; j += kNT) zero_agent_u64(&a.keys[j]);
    __builtin_amdgcn_s_waitcnt(0);  // every exchange has returned
    __syncthreads();
    if (threadIdx.x == 0) set_agent_u32(ready, 1u);
    int32_t* lds_rows = reinterpret_cast<int32_t*>(sh.item);  // per request: offset, prefix length
    const Sizing sz{a.sizing.separate, a.sizing.conf, a.sizing.R, a.sizing.bmax, a.sizing.rule};
    sched_pass<kNT>(sh, a.conf, a.R, a.K, a.n_sampling, a.T, a.num_reqs, a.vc, a.dc, a.bmax, sz, a.surv, a.order,
                    a.sorted_surv, a.b_star, a.best_obj, a.prefix_len, a.offsets, a.ver_idx, a.status, lds_rows);
    __syncthreads();
    // tokens[r, i], and ver_tokens[offset_r + i] for the i below request r's prefix length
    // (the verified slots are each request's first ones), for positions [p0, p1)
    auto write_tokens = [&](int p0, int p1) {
        const int np = p1 - p0;
        for (int q = threadIdx.x; q < a.R * np; q += kNT) {
            const int r = q / np, i = p0 + (q - r * np);
            const int32_t tok = key_index(load_agent_u64(&a.keys[(size_t)i * a.R + r]));
            a.tokens[r * a.K + i] = tok;
            if (a.ver_tokens != nullptr && i < lds_rows[2 * r + 1]) a.ver_tokens[lds_rows[2 * r] + i] = tok;
        }
    };
    const int B = sh.b_star;
    if (a.ver_tokens != nullptr)
        for (int j = B + threadIdx.x; j < n; j += kNT) a.ver_tokens[j] = -1;
    int p0 = 0;
    if (pos_bar >= 0) {
        for (; p0 + 1 < a.K; ++p0) {
            grid_wait(&bar[p0 * kMaxGroups + pos_bar], (uint32_t)G, a.status);
            write_tokens(p0, p0 + 1);
        }
    }
    // each chain workgroup arrives for the groups of a position in order
    grid_wait(&bar[last_bar], (uint32_t)G, a.status);
    // Every chain workgroup has passed its last wait: the counters and the flag go back
    // to zero for the next launch, while the remaining tokens are decoded.
    for (int p = threadIdx.x; p < a.K * kMaxGroups; p += kNT) set_agent_u32(&bar[p], 0u);
    if (threadIdx.x == 0) set_agent_u32(ready, 0u);
    write_tokens(p0, a.K);
}

template <int KS, bool VEC, int PF>
__global__ __launch_bounds__(kNT, 1) void step_single_bf16_kernel(StepArgs a) {
    __shared__ __attribute__((aligned(16))) unsigned char smem[StepLds<KS>::kBytes];
    const int G = (int)gridDim.x - 1;  // chain workgroups
    if ((int)blockIdx.x < G) {
        chain_persist_body<KS, VEC, false, PF>(*reinterpret_cast<ChainLds<KS>*>(smem), (const uint16_t*)a.base,
                                    (const uint16_t*)a.A, (const uint16_t*)a.Bt, a.prev0, a.keys, a.sync, nullptr,
                                    a.status, a.R, a.K, a.V, a.rank, G, a.sync + a.K * kMaxGroups);
        return;
    }
    step_schedule_wg(a, smem, G, (a.K - 1) * kMaxGroups + group_count(a.R) - 1, group_count(a.R) - 1);
}

// fp32 factors, small batches (R <= kF32StepRows, rank <= kF32StepRank): each chain
// workgroup takes NV * kNT vocabulary entries, NV per thread (kNT apart, so a wave's loads
// stay contiguous), for every request and position, with the arithmetic of
// chain_pos_f32_kernel (fp32 fused multiply-adds in increasing k from zero, then the base
// logit added), so its tokens equal the per-position launches'.  A thread keeps its
// entries' second-factor rows in registers for the whole step; the key rows are
// wave-uniform; requests go in batches of kF32Batch so their loads overlap.  Per position
// every request's key is reduced over the workgroup and raised into the device-wide key.
// With several chain workgroups they then meet at one barrier (bar[pos * kMaxGroups]) and
// decode the next position's previous tokens from the device-wide keys; a lone chain
// workgroup (the whole vocabulary in one) takes them from its own reduction instead, so
// no position waits on device memory, and counts itself in once, at the last barrier,
// when every key has landed.  One launch replaces K chain launches, the schedule launch
// and the finalize launch.
constexpr int kF32StepRows = 64;
constexpr int kF32StepRank = 64;
constexpr int kF32Batch = 8;

struct StepF32Chain {
    int32_t prev[kF32StepRows];
    uint64_t wkey[kNT / 64][kF32StepRows];
};

template <int RK, int NV>
__device__ __forceinline__ void chain_f32_step_body(StepF32Chain& L, const StepArgs& a, int G) {
    const float* base = (const float*)a.base;
    const float* A = (const float*)a.A;
    const float* Bt = (const float*)a.Bt;
    uint32_t* bar = a.sync;
    const uint32_t* ready = a.sync + a.K * kMaxGroups;
    const int R = a.R, K = a.K, V = a.V, rank = a.rank;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const bool alone = G == 1;
    int v[NV];
    float b[NV][RK];
#pragma unroll
    for (int t = 0; t < NV; ++t) {
        v[t] = (blockIdx.x * NV + t) * kNT + tid;
#pragma unroll
        for (int k = 0; k < RK; ++k) b[t][k] = (v[t] < V && k < rank) ? Bt[(size_t)v[t] * rank + k] : 0.f;
    }
    for (int j = tid; j < R; j += kNT) L.prev[j] = decode_prev(a.prev0, a.keys, a.status, R, V, 0, j, blockIdx.x == 0);
    __syncthreads();
    uint64_t token = 0;
    for (int pos = 0; pos < K; ++pos) {
        for (int r0 = 0; r0 < R; r0 += kF32Batch) {
            float x[kF32Batch][NV];
#pragma unroll
            for (int q = 0; q < kF32Batch; ++q) {
                const int r = r0 + q < R ? r0 + q : R - 1;
#pragma unroll
                for (int t = 0; t < NV; ++t) x[q][t] = v[t] < V ? base[((size_t)r * K + pos) * V + v[t]] : 0.f;
            }
#pragma unroll
            for (int q = 0; q < kF32Batch; ++q) {
                if (r0 + q >= R) break;
                const int r = r0 + q;
                const float* ar = A + (size_t)__builtin_amdgcn_readfirstlane(L.prev[r]) * rank;
                // The key row, zero past rank.  The padded steps add +0 * +0: the sum starts
                // at +0 and can never become -0 (a sum is -0 only if both terms are), so
                // they leave every value as the rank-long loop leaves it.
                float arow[RK];
#pragma unroll
                for (int k = 0; k < RK; ++k) arow[k] = k < rank ? ar[k] : 0.f;
                uint64_t key = 0ull;
#pragma unroll
                for (int t = 0; t < NV; ++t) {
                    float acc = 0.f;
#pragma unroll
                    for (int k = 0; k < RK; ++k) acc = fmaf(arow[k], b[t][k], acc);
                    if (v[t] < V) key = umax64(key, argmax_key(x[q][t] + acc, (uint32_t)v[t]));
                }
#pragma unroll
                for (int m = 1; m < 64; m <<= 1) key = umax64(key, shfl_xor_u64(key, m));
                if (lane == 0) L.wkey[w][r] = key;
            }
        }
        __syncthreads();
        if (pos == 0) grid_wait(ready, 1u, a.status);
        for (int j = tid; j < R; j += kNT) {
            uint64_t bk = L.wkey[0][j];
            for (int q = 1; q < kNT / 64; ++q) bk = umax64(bk, L.wkey[q][j]);
            if (alone) {
                // The only contributor, onto a zeroed key: an atomic max that returns nothing
                // (performed where every workgroup sees it, like all key updates), and
                // nothing to wait for until the final count, whose memory-counter wait
                // covers it.
                __hip_atomic_fetch_max(&a.keys[(size_t)pos * R + j], bk, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                L.prev[j] = key_index(bk);  // every row has a key, so the index is in [0, V)
            } else if (bk) {
                token ^= __hip_atomic_fetch_max(&a.keys[(size_t)pos * R + j], bk, __ATOMIC_RELAXED,
                                                __HIP_MEMORY_SCOPE_AGENT);
            }
        }
        if (alone) {
            if (pos + 1 == K) grid_arrive(&bar[pos * kMaxGroups], token);
            else __syncthreads();
            continue;
        }
        grid_arrive(&bar[pos * kMaxGroups], token);
        token = 0;
        if (pos + 1 < K) {
            grid_wait(&bar[pos * kMaxGroups], (uint32_t)G, a.status);
            for (int j = tid; j < R; j += kNT)
                L.prev[j] = decode_prev(a.prev0, a.keys, a.status, R, V, pos + 1, j, false);
            __syncthreads();
        }
    }
}

template <int RK, int NV>
__global__ __launch_bounds__(kNT, 1) void step_single_f32_kernel(StepArgs a) {
    constexpr size_t kBytes =
        sizeof(StepF32Chain) > sizeof(SchedShared<kNT>) ? sizeof(StepF32Chain) : sizeof(SchedShared<kNT>);
    __shared__ __attribute__((aligned(16))) unsigned char smem[kBytes];
    const int G = (int)gridDim.x - 1;  // chain workgroups
    if ((int)blockIdx.x < G) {
        chain_f32_step_body<RK, NV>(*reinterpret_cast<StepF32Chain*>(smem), a, G);
        return;
    }
    step_schedule_wg(a, smem, G, (a.K - 1) * kMaxGroups);
}

// Launches `fn` (a single-launch step kernel) when its grid fits on the device at once.
hipError_t launch_resident(const void* fn, int* resident, const StepArgs& a, int grid, hipStream_t s) {
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
    StepArgs arg = a;
    void* args[] = {&arg};
    if (!a.coop) return hipLaunchKernel(fn, dim3(grid), dim3(kNT), args, 0, s);
    return hipLaunchCooperativeKernel(fn, dim3(grid), dim3(kNT), args, 0, s);
}

template <int KS, bool VEC>
hipError_t launch_single(const StepArgs& a, int grid, hipStream_t s) {
    // A single group of at most 64 requests sweeps whole 2-block ring cycles (the full
    // rank only; other ranks keep the 4-block ring).
    if (KS == 8 && a.R <= 64) {
        static int resident[64] = {0};
        return launch_resident((const void*)step_single_bf16_kernel<KS, VEC, 2>, resident, a, grid, s);
    }
    static int resident[64] = {0};
    return launch_resident((const void*)step_single_bf16_kernel<KS, VEC, kPF>, resident, a, grid, s);
}

template <int KS>
hipError_t launch_single_ks(const StepArgs& a, int grid, hipStream_t s) {
    if (a.V % 8 == 0) return launch_single<KS, true>(a, grid, s);
    return launch_single<KS, false>(a, grid, s);
}

}  // namespace

hipError_t launch_step_single_f32(const StepArgs& a, hipStream_t s) {
    if (a.R < 1 || a.R > kF32StepRows || a.K < 1 || a.rank < 1 || a.rank > kF32StepRank)
        return hipErrorCooperativeLaunchTooLarge;
    if (a.rank <= 16 && a.V <= 4 * kNT) {  // the whole vocabulary in one chain workgroup
        static int resident[64] = {0};
        return launch_resident((const void*)step_single_f32_kernel<16, 4>, resident, a, 2, s);
    }
    const int grid = (a.V + kNT - 1) / kNT + 1;  // vocabulary tiles + the scheduling workgroup
    if (a.rank <= 16) {
        static int resident[64] = {0};
        return launch_resident((const void*)step_single_f32_kernel<16, 1>, resident, a, grid, s);
    }
    static int resident[64] = {0};
    return launch_resident((const void*)step_single_f32_kernel<kF32StepRank, 1>, resident, a, grid, s);
}

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
