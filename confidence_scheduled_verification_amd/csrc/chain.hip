// Stage 1 of the chain-and-schedule pass: semi-autoregressive chaining of a
// K-token draft block (DSpark summary "How DSpark Speeds Up LLM Inference",
// section "Draft better"; MAX worklog "DSpark on MAX", section "What DSpark is",
// item 3).  Position i of request r scores every vocabulary entry v as
//     x[r,i,v] = base[r,i,v] + <A[prev_r,:], Bt[v,:]>
// and takes the argmax; the winner keys position i+1.
//
// gfx950 design:
//   * The low-rank bias is the contraction (R x rank) . (rank x V).  It runs on
//     the bf16 matrix cores (v_mfma_f32_16x16x32_bf16, fp32 accumulation) in the
//     transposed form D[v, r] = Bt[v,:] . A[prev_r,:]: vocabulary rows are the
//     MFMA M dimension, requests the N dimension.  The accumulator starts at the
//     base logits, so the matrix cores also add them.
//   * A workgroup of 8 waves owns one vocabulary tile of 512 entries; each wave
//     keeps the Bt fragments of its 64 rows in registers and sweeps the requests
//     in blocks of 16.  The key rows A[prev_r,:] of up to 256 requests are
//     gathered into LDS and shared by the waves.
//   * Each lane's accumulators hold 8 consecutive vocabulary entries of one
//     request per pair of M blocks (the M-row -> vocabulary mapping is permuted
//     to make that so), so base logits stream in as 16-byte coalesced loads,
//     prefetched a few request blocks ahead.
//   * The argmax is fused: per lane a NaN-propagating maximum3 tree and the first
//     index holding the maximum, then 64-bit keys (ordered value, ~index) raised by
//     LDS atomic max over the lanes and waves of the workgroup, and across
//     workgroups by one 64-bit atomic max per request per workgroup.
//   * Persistent form (the default when the tiles fit on the CUs at once): ONE
//     launch of a resident grid runs all K positions.  Bt stays in registers for the
//     whole step (read from memory once instead of K times), and positions are
//     separated by grid barriers on counters in the workspace.  Requests are
//     split into two groups whose phases alternate, so a group's barrier wait
//     falls behind the other group's work.  Every wait is bounded; a timeout
//     sets DSPARK_STATUS_SYNC_TIMEOUT and the kernel still exits.
//   * Per-position form (larger vocabularies, more than 256 requests): one launch
//     per position; kernel boundaries order the positions.
//   * Grids hold one 512-thread workgroup per 512 vocabulary entries (about 250
//     for a 129280-entry vocabulary) instead of ~10^5 tiny blocks, which the MAX
//     worklog found dispatch-bound ("Correctness, then 1.3x").
#include "chain_dev.h"

namespace dspark {

namespace {

// One launch per position, one vocabulary tile per workgroup, requests in chunks of
// kReqChunk.  KS = padded rank / 32, VEC = V % 8 == 0 (16-byte base loads), LOGITS =
// the general scorer (chained logits written when `logits` is given, tokens sampled
// when SAMPLE).
template <int KS, bool VEC, bool LOGITS, bool SAMPLE = false>
__global__ __launch_bounds__(kNT, 1) void chain_pos_bf16_kernel(
    const uint16_t* __restrict__ base, const uint16_t* __restrict__ A, const uint16_t* __restrict__ Bt,
    const int32_t* __restrict__ prev0, uint64_t* __restrict__ keys, int32_t* __restrict__ tokens,
    float* __restrict__ logits, uint32_t* __restrict__ status, int R, int K, int V, int rank, int pos,
    SampleArgs smp) {
    static_assert(LOGITS || !SAMPLE, "sampling runs in the general scorer");
    __shared__ __attribute__((aligned(16))) ChainLds<KS> L;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int vb = blockIdx.x * kTileV + w * kWV;
    bf16x8 bt[kMB][KS];
    load_bt<KS>(bt, Bt, V, rank, vb, lane & 15, lane >> 4);
    BaseFrag pre[kPF];
    if (!LOGITS) prefetch_rows<VEC>(pre, base, R, K, V, pos, 0, vb);
    for (int c0 = 0; c0 < R; c0 += kReqChunk) {
        const int RC = min(kReqChunk, R - c0);
        const int rows = LOGITS ? (RC + 15) & ~15 : fast_rows(RC);
        if (LOGITS) prefetch_rows<VEC>(pre, base, R, K, V, pos, c0, vb);
        if (c0 > 0) __syncthreads();  // the previous chunk is done with the LDS
        decode_rows(L.prev, L.best, prev0, keys, tokens, status, R, K, V, pos, c0, RC, 0, rows);
        __syncthreads();
        gather_rows<KS>(L, A, V, rank, RC, 0, rows);
        __syncthreads();
        if (LOGITS) {
            score_generic<KS, VEC, SAMPLE>(L, bt, pre, base, logits, R, K, V, pos, c0, RC, 0, vb, smp);
        } else {
            const int nc0 = c0 + kReqChunk < R ? c0 + kReqChunk : c0;
            score_rows<KS, VEC>(L, bt, pre, base, R, K, V, pos, c0, RC, 0, vb, pos, nc0);
        }
        __syncthreads();
        uint64_t token = 0;  // kernel end orders the key atomics before the next launch
        publish_rows<KS>(L, keys, R, pos, c0, RC, 0, token);
    }
}

// All K positions in one launch of a resident grid (R <= kReqChunk, gridDim.x <= resident
// workgroups).  SAMPLE: tokens drawn by Gumbel-max (probabilistic drafting).
template <int KS, bool VEC, bool SAMPLE, int PF>
__global__ __launch_bounds__(kNT, 1) void chain_persist_bf16_kernel(
    const uint16_t* __restrict__ base, const uint16_t* __restrict__ A, const uint16_t* __restrict__ Bt,
    const int32_t* __restrict__ prev0, uint64_t* __restrict__ keys, uint32_t* __restrict__ bar,
    int32_t* __restrict__ tokens, uint32_t* __restrict__ status, int R, int K, int V, int rank, SampleArgs smp) {
    __shared__ __attribute__((aligned(16))) ChainLds<KS> L;
    chain_persist_body<KS, VEC, SAMPLE, PF>(L, base, A, Bt, prev0, keys, bar, tokens, status, R, K, V, rank,
                                            (int)gridDim.x, nullptr, smp);
}

// Second-factor fragments of one wave's vocabulary slice kept in LDS, lane-linear:
// fragment (mb, ks) of lane l at byte ((mb * KS + ks) * 64 + l) * 16 of the slice, the
// layout load_bt gives in registers.  kLdsWaves waves of a two-tile workgroup keep their
// second tile there (in the key-row rows that at most 64 requests leave free), so they
// never reload it.
template <int KS>
constexpr int lds_waves() {
    constexpr int free_bytes = (kReqChunk - 64) * ChainLds<KS>::LROW * 2;
    constexpr int slice = kMB * KS * 64 * 16;
    return free_bytes / slice < kWaves ? free_bytes / slice : kWaves;
}

template <int KS>
__device__ __forceinline__ char* lds_slice(ChainLds<KS>& L, int s) {
    return reinterpret_cast<char*>(L.a + 64 * ChainLds<KS>::LROW) + s * (kMB * KS * 64 * 16);
}

// The wave slice starting at vocabulary vb into LDS by direct-to-LDS loads (rows past V
// and k past rank land as zeros).
template <int KS>
__device__ __forceinline__ void load_slice_lds(char* slice, const uint16_t* __restrict__ Bt, int V, int rank, int vb) {
    const int lane = threadIdx.x & 63, n16 = lane & 15, g = lane >> 4;
    const u32x4 rs = buffer_rsrc(Bt, (uint32_t)V * (uint32_t)rank * 2u);
#pragma unroll
    for (int mb = 0; mb < kMB; ++mb) {
        const int v = vb + 32 * (mb >> 1) + 8 * (n16 >> 2) + 4 * (mb & 1) + (n16 & 3);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const int k0 = ks * 32 + g * 8;
            const uint32_t voff = (v < V && k0 < rank) ? ((uint32_t)v * (uint32_t)rank + (uint32_t)k0) * 2u : 0xFFFFFFF0u;
            dma16_to_lds(rs, lds_addr(slice + (mb * KS + ks) * 1024), voff);
        }
    }
}

// Score the (at most 4) request blocks of requests [0, RC) against the wave slice held in
// LDS at `slice` (vocabulary vb).  EXACT: the ordered-key scan of every element (for a
// wave whose fast pass met a NaN); otherwise the fused argmax, returning the NaN mask.
// Base blocks are all requested first.
template <int KS, bool VEC, bool EXACT>
__device__ __forceinline__ uint64_t score_slice_lds(ChainLds<KS>& L, const char* slice,
                                                    const uint16_t* __restrict__ base, int R, int K, int V, int pos,
                                                    int RC, int vb) {
    constexpr int LROW = ChainLds<KS>::LROW;
    const int lane = threadIdx.x & 63, n16 = lane & 15, g = lane >> 4;
    const int vlane = vb + 8 * g;
    const int nB = (RC + 15) >> 4;
    const BaseSrc src = base_src(base, R, K, V, n16, vlane);
    const __amdgpu_buffer_rsrc_t rs = seg_rsrc(src, 0, pos, K, V);
    BaseFrag f[4];
#pragma unroll
    for (int b = 0; b < 4; ++b)
        if (b < nB) load_block<VEC>(f[b], src, rs, b, 0, pos, R, K, V, n16, vlane);
    uint64_t nan_mask = 0ull;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        if (b < nB) {
            f32x4 acc[kMB];
            if (EXACT || vb + kWV > V) init_acc<true, VEC>(acc, f[b], vlane, V);
            else init_acc<false, VEC>(acc, f[b], vlane, V);
            const uint16_t* arow = L.a + (b * 16 + n16) * LROW + g * 8;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const bf16x8 bfr = *(const bf16x8*)(arow + ks * 32);
#pragma unroll
                for (int mb = 0; mb < kMB; ++mb) {
                    const bf16x8 afr = *(const bf16x8*)(slice + ((mb * KS + ks) * 64 + lane) * 16);
                    acc[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(afr, bfr, acc[mb], 0, 0, 0);
                }
            }
            uint64_t* best = L.best + b * 16 + n16;
            if (!EXACT) {
                block_argmax<false>(acc, best, vlane, nan_mask, SampleArgs{}, pos, 0);
            } else {
                uint32_t bu = 0u, bv = 0u;
#pragma unroll
                for (int e = 0; e < 4 * kMB; ++e) {
                    const uint32_t v = (uint32_t)(vlane + 32 * (e >> 3) + (e & 7));
                    const uint32_t u = ordered_u32(acc[2 * (e >> 3) + ((e & 7) >> 2)][e & 3]);
                    if (v < (uint32_t)V && u > bu) {
                        bu = u;
                        bv = v;
                    }
                }
                const uint64_t key = bu ? (((uint64_t)bu << 32) | (uint64_t)(~bv)) : 0ull;
                atomicMax((unsigned long long*)best, (unsigned long long)key);
            }
        }
    }
    return nan_mask;
}

// Two vocabulary tiles per workgroup, for vocabularies with more tiles than the CUs
// hold at once (up to twice as many): workgroup b owns tiles b and b + G.  The
// registers hold one tile's second-factor rows, so each position scores the tile
// already held, then loads the other tile's rows and scores it, and the order flips
// every position (b, b+G | b+G, b | b, b+G ...): the tile scored last at one position
// is scored first at the next.  A position then reads half of the second factor from
// memory instead of all of it, and the K positions are one launch with grid barriers
// instead of K launches.  At the full rank with 16-byte base loads, the last
// lds_waves<KS>() waves keep their second tile's slice in LDS instead (loaded once) and
// score it from there at every position, so they never reload.  One request group (R <= 64): the key rows are gathered once per
// position for both tiles, and each request's key goes out once per workgroup.
template <int KS, bool VEC, int PF>
__global__ __launch_bounds__(kNT, 1) void chain_persist2_bf16_kernel(
    const uint16_t* __restrict__ base, const uint16_t* __restrict__ A, const uint16_t* __restrict__ Bt,
    const int32_t* __restrict__ prev0, uint64_t* __restrict__ keys, uint32_t* __restrict__ bar,
    int32_t* __restrict__ tokens, uint32_t* __restrict__ status, int R, int K, int V, int rank) {
    __shared__ __attribute__((aligned(16))) ChainLds<KS> L;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int G = (int)gridDim.x;
    const int vb0 = (int)blockIdx.x * kTileV + w * kWV, vb1 = ((int)blockIdx.x + G) * kTileV + w * kWV;
    const int rows = fast_rows<PF>(R);
    decode_rows(L.prev, L.best, prev0, keys, tokens, status, R, K, V, 0, 0, R, 0, rows);
    __syncthreads();
    gather_rows<KS, false>(L, A, V, rank, R, 0, rows);
    // LDS slices only with 16-byte base loads at the full rank (the other forms would
    // run out of registers beside them)
    constexpr int NL = (VEC && KS == 8) ? lds_waves<KS>() : 0;
    const bool in_lds = NL > 0 && w >= kWaves - NL;  // this wave's second tile lives in LDS
    char* slice = lds_slice(L, in_lds ? w - (kWaves - NL) : 0);
    bf16x8 bt[kMB][KS];
    load_bt<KS>(bt, Bt, V, rank, vb0, lane & 15, lane >> 4);
    if (in_lds) load_slice_lds<KS>(slice, Bt, V, rank, vb1);
    BaseFrag pre[PF];
    prefetch_rows<VEC, PF>(pre, base, R, K, V, 0, 0, vb0);
    int ring_pos = 0, ring_vb = vb0;  // the ring holds the first blocks of (position, wave slice)
    __builtin_amdgcn_s_waitcnt(0);    // this wave's gather and LDS slots have landed
    __syncthreads();
    for (int pos = 0; pos < K; ++pos) {
        if (in_lds) {
            // the first tile from registers (its ring runs on to the next position), the
            // second from LDS
            if (vb0 < V)
                score_rows<KS, VEC, false, PF>(L, bt, pre, base, R, K, V, pos, 0, R, 0, vb0,
                                               pos + 1 < K ? pos + 1 : pos, 0);
            if (vb1 < V && score_slice_lds<KS, VEC, false>(L, slice, base, R, K, V, pos, R, vb1) != 0ull)
                score_slice_lds<KS, VEC, true>(L, slice, base, R, K, V, pos, R, vb1);
        } else {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const bool second = ((pos + h) & 1) != 0;
            const int vb = second ? vb1 : vb0;
            if (h == 1) load_bt<KS>(bt, Bt, V, rank, vb, lane & 15, lane >> 4);
            // the next slice this wave scores: the other tile at this position, else this
            // tile at the next position
            const int npos = h == 0 ? pos : (pos + 1 < K ? pos + 1 : pos);
            const int nvb = h == 0 ? (second ? vb0 : vb1) : vb;
            if (vb < V) {
                if (ring_pos != pos || ring_vb != vb) prefetch_rows<VEC, PF>(pre, base, R, K, V, pos, 0, vb);
                score_rows<KS, VEC, false, PF, true>(L, bt, pre, base, R, K, V, pos, 0, R, 0, vb, npos, 0,
                                                     SampleArgs{}, nvb);
                ring_pos = npos;
                ring_vb = nvb;
            }
        }
        }
        __syncthreads();
        uint64_t token = 0;
        publish_rows<KS>(L, keys, R, pos, 0, R, 0, token);
        grid_arrive(&bar[pos * kMaxGroups], token);
        if (pos + 1 < K) {
            grid_wait(&bar[pos * kMaxGroups], (uint32_t)G, status);
            decode_rows(L.prev, L.best, prev0, keys, tokens, status, R, K, V, pos + 1, 0, R, 0, rows);
            __syncthreads();
            gather_rows<KS>(L, A, V, rank, R, 0, rows);
            __syncthreads();
        }
    }
}

// fp32 factors: one thread per vocabulary entry, fused multiply-add in increasing k.
__global__ __launch_bounds__(kF32Threads) void chain_pos_f32_kernel(
    const float* __restrict__ base, const float* __restrict__ A, const float* __restrict__ Bt,
    const int32_t* __restrict__ prev0, uint64_t* __restrict__ keys, int32_t* __restrict__ tokens,
    float* __restrict__ logits, uint32_t* __restrict__ status, int R, int K, int V, int rank, int pos,
    SampleArgs smp) {
    __shared__ uint64_t s_wbest[kF32Threads / 64];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int v = blockIdx.x * kF32Threads + tid;
    for (int r = 0; r < R; ++r) {
        const int p = decode_prev(prev0, keys, status, R, V, pos, r, blockIdx.x == 0 && tid == 0);
        if (pos > 0 && blockIdx.x == 0 && tid == 0) tokens[(size_t)r * K + (pos - 1)] = p;
        uint64_t key = 0ull;
        if (v < V) {
            const float* a = A + (size_t)p * rank;
            const float* b = Bt + (size_t)v * rank;
            float acc = 0.f;
            for (int k = 0; k < rank; ++k) acc = fmaf(a[k], b[k], acc);
            float x = base[((size_t)r * K + pos) * V + v] + acc;
            if (logits != nullptr) logits[((size_t)r * K + pos) * V + v] = x;
            if (smp.on) {  // Gumbel-max sample of softmax(x / temperature)
                uint32_t wd[4];
                philox4x32_10((uint32_t)v >> 2, (uint32_t)pos, (uint32_t)r, 0u, smp.k0, smp.k1, wd);
                x = sampled_value(x, smp.scale, wd[v & 3]);
            }
            key = argmax_key(x, (uint32_t)v);
        }
#pragma unroll
        for (int m = 1; m < 64; m <<= 1) key = umax64(key, shfl_xor_u64(key, m));
        if (lane == 0) s_wbest[w] = key;
        __syncthreads();
        if (tid == 0) {
            uint64_t b = s_wbest[0];
            for (int q = 1; q < kF32Threads / 64; ++q) b = umax64(b, s_wbest[q]);
            if (b) publish_key(&keys[(size_t)pos * R + r], b);
        }
        __syncthreads();
    }
}

__global__ void fill_u64_kernel(uint64_t* __restrict__ p, size_t n) {
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
        p[i] = 0ull;
}

// Last position's tokens, and (when ver_idx is given) the verified tokens
// ver_tokens[j] = tokens[ver_idx[j]] for j < *b_star, -1 after.  A slot of the last
// position is decoded from its key directly, so no workgroup reads a token another
// workgroup of this launch writes.
__global__ void chain_finalize_kernel(const uint64_t* __restrict__ keys, int32_t* __restrict__ tokens, int R,
                                      int K, const int32_t* __restrict__ ver_idx,
                                      const int32_t* __restrict__ b_star, int32_t* __restrict__ ver_tokens) {
    const int stride = gridDim.x * blockDim.x;
    const int i0 = blockIdx.x * blockDim.x + threadIdx.x;
    for (int r = i0; r < R; r += stride)
        tokens[(size_t)r * K + (K - 1)] = key_index(load_agent_u64(&keys[(size_t)(K - 1) * R + r]));
    if (ver_tokens != nullptr) {
        const int n = R * K;
        const int B = *b_star;
        for (int j = i0; j < n; j += stride) {
            int32_t tok = -1;
            const int f = j < B ? ver_idx[j] : -1;
            if (f >= 0 && f < n) {
                const int r = f / K, i = f - r * K;
                tok = (i == K - 1) ? key_index(load_agent_u64(&keys[(size_t)(K - 1) * R + r])) : tokens[f];
            }
            ver_tokens[j] = tok;
        }
    }
}

// Bt[v, k] = Bmat[k, v] through 32x32 LDS tiles (start-up layout change).
template <typename T>
__global__ void transpose_kernel(const T* __restrict__ src, int rows, int cols, T* __restrict__ dst) {
    __shared__ T tile[32][33];
    const int c0 = blockIdx.x * 32, r0 = blockIdx.y * 32;
    for (int y = threadIdx.y; y < 32; y += blockDim.y) {
        const int r = r0 + y, c = c0 + threadIdx.x;
        if (r < rows && c < cols) tile[y][threadIdx.x] = src[(size_t)r * cols + c];
    }
    __syncthreads();
    for (int y = threadIdx.y; y < 32; y += blockDim.y) {
        const int c = c0 + y, r = r0 + threadIdx.x;
        if (r < rows && c < cols) dst[(size_t)c * rows + r] = tile[threadIdx.x][y];
    }
}

// Persistent launch when every tile's workgroup can be resident at once: one
// workgroup per CU (the LDS footprint allows no more), so the grid must not exceed
// the CUs reported by the occupancy query.  Returns hipErrorCooperativeLaunchTooLarge
// when it does not fit; the caller then launches per position.
// hipSuccess when a grid of `grid` workgroups of `fn` fits on the current device at
// once (cached per device and kernel instantiation through `resident`).
hipError_t check_resident(const void* fn, int (&resident)[64], int grid) {
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
    return grid > resident[dev] ? hipErrorCooperativeLaunchTooLarge : hipSuccess;
}

template <int KS, bool VEC, bool SAMPLE, int PF>
hipError_t launch_persist(const ChainArgs& a, int grid, hipStream_t s) {
    const void* fn = (const void*)chain_persist_bf16_kernel<KS, VEC, SAMPLE, PF>;
    static int resident[64] = {0};
    hipError_t e = check_resident(fn, resident, grid);
    if (e != hipSuccess) return e;
    const uint16_t* base = (const uint16_t*)a.base;
    const uint16_t* A = (const uint16_t*)a.A;
    const uint16_t* Bt = (const uint16_t*)a.Bt;
    const int32_t* prev0 = a.prev0;
    uint64_t* keys = a.keys;
    uint32_t* bar = a.bar;
    int32_t* tokens = a.tokens;
    uint32_t* status = a.status;
    int R = a.R, K = a.K, V = a.V, rank = a.rank;
    SampleArgs smp = a.smp;
    if (!a.coop) {
        hipLaunchKernelGGL((chain_persist_bf16_kernel<KS, VEC, SAMPLE, PF>), dim3(grid), dim3(kNT), 0, s, base, A, Bt,
                           prev0, keys, bar, tokens, status, R, K, V, rank, smp);
        return hipGetLastError();
    }
    void* args[] = {&base, &A, &Bt, &prev0, &keys, &bar, &tokens, &status, &R, &K, &V, &rank, &smp};
    return hipLaunchCooperativeKernel(fn, dim3(grid), dim3(kNT), args, 0, s);
}

template <int KS, bool VEC, int PF>
hipError_t launch_persist2(const ChainArgs& a, int grid, hipStream_t s) {
    const void* fn = (const void*)chain_persist2_bf16_kernel<KS, VEC, PF>;
    static int resident[64] = {0};
    hipError_t e = check_resident(fn, resident, grid);
    if (e != hipSuccess) return e;
    const uint16_t* base = (const uint16_t*)a.base;
    const uint16_t* A = (const uint16_t*)a.A;
    const uint16_t* Bt = (const uint16_t*)a.Bt;
    const int32_t* prev0 = a.prev0;
    uint64_t* keys = a.keys;
    uint32_t* bar = a.bar;
    int32_t* tokens = a.tokens;
    uint32_t* status = a.status;
    int R = a.R, K = a.K, V = a.V, rank = a.rank;
    if (!a.coop) {
        hipLaunchKernelGGL((chain_persist2_bf16_kernel<KS, VEC, PF>), dim3(grid), dim3(kNT), 0, s, base, A, Bt, prev0,
                           keys, bar, tokens, status, R, K, V, rank);
        return hipGetLastError();
    }
    void* args[] = {&base, &A, &Bt, &prev0, &keys, &bar, &tokens, &status, &R, &K, &V, &rank};
    return hipLaunchCooperativeKernel(fn, dim3(grid), dim3(kNT), args, 0, s);
}

template <int KS, bool VEC>
hipError_t launch_bf16(const ChainArgs& a, int grid, hipStream_t s) {
    if (a.R <= kReqChunk && a.logits == nullptr) {
        // A single group of at most 64 requests sweeps whole 2-block ring cycles (the full
        // rank only; other ranks keep the 4-block ring).
        hipError_t e;
        if (KS == 8 && a.R <= 64)
            e = a.smp.on ? launch_persist<KS, VEC, true, 2>(a, grid, s) : launch_persist<KS, VEC, false, 2>(a, grid, s);
        else
            e = a.smp.on ? launch_persist<KS, VEC, true, kPF>(a, grid, s) : launch_persist<KS, VEC, false, kPF>(a, grid, s);
        if (e != hipErrorCooperativeLaunchTooLarge) return e;
        (void)hipGetLastError();  // clear the sticky launch error before falling back
        if (a.R <= 64 && !a.smp.on) {  // one request group, greedy: two tiles per workgroup
            e = KS == 8 ? launch_persist2<KS, VEC, 2>(a, (grid + 1) / 2, s)
                        : launch_persist2<KS, VEC, kPF>(a, (grid + 1) / 2, s);
            if (e != hipErrorCooperativeLaunchTooLarge) return e;
            (void)hipGetLastError();
        }
    }
    for (int pos = 0; pos < a.K; ++pos) {
        if (a.smp.on)
            hipLaunchKernelGGL((chain_pos_bf16_kernel<KS, VEC, true, true>), dim3(grid), dim3(kNT), 0, s,
                               (const uint16_t*)a.base, (const uint16_t*)a.A, (const uint16_t*)a.Bt, a.prev0, a.keys,
                               a.tokens, a.logits, a.status, a.R, a.K, a.V, a.rank, pos, a.smp);
        else if (a.logits != nullptr)
            hipLaunchKernelGGL((chain_pos_bf16_kernel<KS, VEC, true>), dim3(grid), dim3(kNT), 0, s,
                               (const uint16_t*)a.base, (const uint16_t*)a.A, (const uint16_t*)a.Bt, a.prev0, a.keys,
                               a.tokens, a.logits, a.status, a.R, a.K, a.V, a.rank, pos, a.smp);
        else
            hipLaunchKernelGGL((chain_pos_bf16_kernel<KS, VEC, false>), dim3(grid), dim3(kNT), 0, s,
                               (const uint16_t*)a.base, (const uint16_t*)a.A, (const uint16_t*)a.Bt, a.prev0, a.keys,
                               a.tokens, nullptr, a.status, a.R, a.K, a.V, a.rank, pos, a.smp);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

template <int KS>
hipError_t launch_bf16_ks(const ChainArgs& a, int grid, hipStream_t s) {
    if (a.V % 8 == 0) return launch_bf16<KS, true>(a, grid, s);
    return launch_bf16<KS, false>(a, grid, s);
}

}  // namespace

int chain_tile_vocab() { return kTileV; }

hipError_t launch_zero_keys(uint64_t* keys, size_t n, hipStream_t s) {
    if (n == 0) return hipSuccess;
    const int grid = (int)std::min<size_t>((n + 255) / 256, 1024);
    hipLaunchKernelGGL(fill_u64_kernel, dim3(grid), dim3(256), 0, s, keys, n);
    return hipGetLastError();
}

hipError_t launch_chain_positions(const ChainArgs& a, int num_cu, hipStream_t s) {
    (void)num_cu;
    if (a.dtype == 1) {
        const int grid = (a.V + kTileV - 1) / kTileV;  // one vocabulary tile per workgroup
        const int ks = (a.rank + 31) / 32;
        if (ks <= 1) return launch_bf16_ks<1>(a, grid, s);
        if (ks <= 2) return launch_bf16_ks<2>(a, grid, s);
        if (ks <= 4) return launch_bf16_ks<4>(a, grid, s);
        return launch_bf16_ks<8>(a, grid, s);
    }
    const int grid = (a.V + kF32Threads - 1) / kF32Threads;
    for (int pos = 0; pos < a.K; ++pos) {
        hipLaunchKernelGGL(chain_pos_f32_kernel, dim3(grid), dim3(kF32Threads), 0, s, (const float*)a.base,
                           (const float*)a.A, (const float*)a.Bt, a.prev0, a.keys, a.tokens, a.logits, a.status,
                           a.R, a.K, a.V, a.rank, pos, a.smp);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

hipError_t launch_chain_finalize(const uint64_t* keys, int32_t* tokens, int R, int K, const int32_t* ver_idx,
                                 const int32_t* b_star, int32_t* ver_tokens, hipStream_t s) {
    const int n = ver_tokens ? R * K : R;
    const int grid = std::max(1, std::min((n + 255) / 256, 256));
    hipLaunchKernelGGL(chain_finalize_kernel, dim3(grid), dim3(256), 0, s, keys, tokens, R, K, ver_idx, b_star,
                       ver_tokens);
    return hipGetLastError();
}

hipError_t launch_transpose(const void* src, int rows, int cols, int elem_bytes, void* dst, hipStream_t s) {
    const dim3 grid((cols + 31) / 32, (rows + 31) / 32), block(32, 8);
    if (elem_bytes == 2)
        hipLaunchKernelGGL(transpose_kernel<uint16_t>, grid, block, 0, s, (const uint16_t*)src, rows, cols,
                           (uint16_t*)dst);
    else
        hipLaunchKernelGGL(transpose_kernel<float>, grid, block, 0, s, (const float*)src, rows, cols, (float*)dst);
    return hipGetLastError();
}

}  // namespace dspark
