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
//     index holding the maximum, then 64-bit keys (ordered value, ~index)
//     reduced by cross-lane shuffles, across waves in LDS, and across workgroups
//     by one 64-bit atomicMax per request per workgroup (skipped when the stored
//     key is already larger).
//   * Persistent form (the default when the tiles fit on the CUs at once): ONE
//     cooperative launch runs all K positions.  Bt stays in registers for the
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
#include "common.h"
#include "kernels.h"

namespace dspark {

namespace {

constexpr int kReqChunk = 256;   // requests whose key rows fit in LDS at once
#ifndef DSPARK_CHAIN_WAVES
#define DSPARK_CHAIN_WAVES 8
#endif
#ifndef DSPARK_CHAIN_MB
#define DSPARK_CHAIN_MB 4
#endif
#ifndef DSPARK_CHAIN_LDS_PAD
#define DSPARK_CHAIN_LDS_PAD 8
#endif
constexpr int kWaves = DSPARK_CHAIN_WAVES;  // waves per workgroup of the bf16 kernels
constexpr int kNT = kWaves * 64;
constexpr int kMB = DSPARK_CHAIN_MB;        // 16-row M blocks per wave (even)
#ifndef DSPARK_CHAIN_PF
#define DSPARK_CHAIN_PF 3
#endif
#ifndef DSPARK_CHAIN_GATHER_BATCH
#define DSPARK_CHAIN_GATHER_BATCH 4
#endif
constexpr int kPF = DSPARK_CHAIN_PF;        // request blocks of base prefetched ahead
constexpr int kWV = 16 * kMB;    // vocabulary entries per wave
constexpr int kTileV = kWaves * kWV;
constexpr int kF32Threads = 256;
constexpr long kSpinLimit = 1L << 22;  // barrier polls (with a short sleep each) before giving up

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ int decode_prev(const int32_t* prev0, const uint64_t* keys, uint32_t* status, int R,
                                           int V, int pos, int r, bool report) {
    if (pos == 0) {
        int p = prev0[r];
        if (p < 0 || p >= V) {
            if (report) raise_status(status, kStatusPrevClamped);
            p = p < 0 ? 0 : V - 1;
        }
        return p;
    }
    // Every row receives at least one key per position, so the decoded index is in
    // range; the clamp only guarantees that the gather can never leave A.
    const int p = key_index(load_agent_u64(&keys[(size_t)(pos - 1) * R + r]));
    return p < 0 ? 0 : (p >= V ? V - 1 : p);
}

// Order-preserving image of a float in the unsigned integers: NaN above every
// number, -0 equal to +0.  Never 0, so 0 marks "no candidate".
__device__ __forceinline__ uint32_t ordered_u32(float x) {
    uint32_t b = __float_as_uint(x);
    if (x != x) return 0xFFFFFFFFu;
    if (b == 0x80000000u) b = 0u;
    return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// Base logits of one request block for one wave: 2 groups of 8 consecutive
// vocabulary entries per lane (16 bytes each).
struct BaseFrag {
    u32x4 q[kMB / 2];
};

template <bool VEC>
__device__ __forceinline__ void load_base(BaseFrag& f, const uint16_t* __restrict__ base, int r, int R, int K, int V,
                                          int pos, int vlane) {
    const bool row_ok = r < R;
    const uint16_t* row = base + ((size_t)(row_ok ? r : 0) * K + pos) * (size_t)V;
#pragma unroll
    for (int p = 0; p < kMB / 2; ++p) {
        const int v0 = vlane + 32 * p;
        if (VEC) {
            if (row_ok && v0 < V)
                f.q[p] = __builtin_nontemporal_load((const u32x4*)(row + v0));
            else
                f.q[p] = u32x4{0u, 0u, 0u, 0u};
        } else {
            uint32_t h[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) h[e] = (row_ok && v0 + e < V) ? (uint32_t)row[v0 + e] : 0u;
            f.q[p] = u32x4{h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16)};
        }
    }
}

// LDS of one bf16 chain workgroup.
template <int KS>
struct ChainLds {
    static constexpr int RP = 32 * KS;   // padded rank
    static constexpr int LROW = RP + DSPARK_CHAIN_LDS_PAD;  // row stride in bf16 elements (pad spreads banks)
    static constexpr int SEGS = RP / 8;  // 16-byte segments per key row
    uint16_t a[kReqChunk * LROW];        // gathered key rows
    uint64_t best[kReqChunk];            // workgroup argmax key per request (LDS atomic max)
    int32_t prev[kReqChunk];             // previous tokens
};

// Bt fragments of this wave's 64 vocabulary rows.  M row m of block mb is
// vocabulary vb + 32*(mb/2) + 8*(m/4) + 4*(mb%2) + m%4, which puts 8 consecutive
// entries in each lane's accumulator pair.
template <int KS>
__device__ __forceinline__ void load_bt(bf16x8 (&bt)[kMB][KS], const uint16_t* __restrict__ Bt, int V, int rank,
                                        int vb, int n16, int g) {
#pragma unroll
    for (int mb = 0; mb < kMB; ++mb) {
        const int v = vb + 32 * (mb >> 1) + 8 * (n16 >> 2) + 4 * (mb & 1) + (n16 & 3);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const int k0 = ks * 32 + g * 8;
            if (v < V && k0 < rank)
                bt[mb][ks] = *(const bf16x8*)(Bt + (size_t)v * rank + k0);
            else
                bt[mb][ks] = bf16x8{};
        }
    }
}

// Requests [c0, c0+RC) use LDS rows l0 .. l0+RC (rounded up to 16 with zero rows).

__device__ __forceinline__ void decode_rows(int32_t* s_prev, uint64_t* s_best, const int32_t* prev0,
                                            const uint64_t* keys, int32_t* tokens, uint32_t* status, int R, int K,
                                            int V, int pos, int c0, int RC, int l0) {
    const int tid = threadIdx.x;
    for (int j = tid; j < RC; j += kNT) {
        const int p = decode_prev(prev0, keys, status, R, V, pos, c0 + j, blockIdx.x == 0);
        s_prev[l0 + j] = p;
        if (pos > 0 && blockIdx.x == 0) tokens[(size_t)(c0 + j) * K + (pos - 1)] = p;
    }
    const int rows = ((RC + 15) >> 4) << 4;
    for (int j = tid; j < rows; j += kNT) s_best[l0 + j] = 0ull;
}

// Key rows A[prev_r, :] into LDS (zero past rank and past RC), a batch of independent
// loads in flight per thread before their stores.
template <int KS>
__device__ __forceinline__ void gather_rows(ChainLds<KS>& L, const uint16_t* __restrict__ A, int rank, int RC,
                                            int l0) {
    constexpr int SEGS = ChainLds<KS>::SEGS, LROW = ChainLds<KS>::LROW;
    constexpr int GB = DSPARK_CHAIN_GATHER_BATCH;
    const int tid = threadIdx.x;
    const int total = ((RC + 15) >> 4) * 16 * SEGS;
    for (int q0 = 0; q0 < total; q0 += GB * kNT) {
        u32x4 seg[GB];
#pragma unroll
        for (int q = 0; q < GB; ++q) {
            const int idx = q0 + tid + q * kNT;
            const int j = idx / SEGS, s = idx - j * SEGS;
            seg[q] = u32x4{0u, 0u, 0u, 0u};
            if (idx < total && j < RC && s * 8 < rank)
                seg[q] = *(const u32x4*)(A + (size_t)L.prev[l0 + j] * rank + s * 8);
        }
#pragma unroll
        for (int q = 0; q < GB; ++q) {
            const int idx = q0 + tid + q * kNT;
            const int j = idx / SEGS, s = idx - j * SEGS;
            if (idx < total) *(u32x4*)(L.a + (l0 + j) * LROW + s * 8) = seg[q];
        }
    }
}

// Score the wave's 64 vocabulary rows against requests [c0, c0+RC) and leave each
// request's best key of this wave in L.best[w][l0 + j].  pre[] holds the first kPF
// base blocks of the range, already requested.
template <int KS, bool VEC>
__device__ __forceinline__ void score_rows(ChainLds<KS>& L, const bf16x8 (&bt)[kMB][KS], BaseFrag (&pre)[kPF],
                                           const uint16_t* __restrict__ base, float* __restrict__ logits, int R,
                                           int K, int V, int pos, int c0, int RC, int l0, int vb) {
    constexpr int LROW = ChainLds<KS>::LROW, MB = kMB, PF = kPF;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int n16 = lane & 15, g = lane >> 4;
    const int vlane = vb + 8 * g;
    const int nRB = (RC + 15) >> 4;
    for (int rb0 = 0; rb0 < nRB; rb0 += PF) {
#pragma unroll
        for (int q = 0; q < PF; ++q) {
            const int rb = rb0 + q;
            if (rb < nRB) {
                // Accumulators start at the base logits (bf16 -> fp32 is exact).  Lane
                // element e (0..15) is vocabulary vlane + 32*(e/8) + e%8, held in
                // acc[2*(e/8) + (e%8)/4][e%4].
                f32x4 acc[MB];
#pragma unroll
                for (int p = 0; p < MB / 2; ++p) {
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        const uint32_t w0 = pre[q].q[p][2 * h], w1 = pre[q].q[p][2 * h + 1];
                        acc[2 * p + h] = f32x4{__uint_as_float(w0 << 16), __uint_as_float(w0 & 0xFFFF0000u),
                                               __uint_as_float(w1 << 16), __uint_as_float(w1 & 0xFFFF0000u)};
                    }
                }
                // refill this slot with the block PF ahead (its base is in acc now)
                if (rb + PF < nRB) load_base<VEC>(pre[q], base, c0 + (rb + PF) * 16 + n16, R, K, V, pos, vlane);
                const uint16_t* arow = L.a + (l0 + rb * 16 + n16) * LROW + g * 8;
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    const bf16x8 bfr = *(const bf16x8*)(arow + ks * 32);
#pragma unroll
                    for (int mb = 0; mb < MB; ++mb)
                        acc[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bt[mb][ks], bfr, acc[mb], 0, 0, 0);
                }

                const int r = c0 + rb * 16 + n16;
                float x[4 * MB];
#pragma unroll
                for (int e = 0; e < 4 * MB; ++e) x[e] = acc[2 * (e >> 3) + ((e & 7) >> 2)][e & 3];
                if (logits != nullptr && r < R) {
#pragma unroll
                    for (int e = 0; e < 4 * MB; ++e) {
                        const int v = vlane + 32 * (e >> 3) + (e & 7);
                        if (v < V) logits[((size_t)r * K + pos) * V + v] = x[e];
                    }
                }
                if (vb + kWV > V) {  // ragged last tile: entries past V cannot win
#pragma unroll
                    for (int e = 0; e < 4 * MB; ++e)
                        if (vlane + 32 * (e >> 3) + (e & 7) >= V) x[e] = -__builtin_huge_valf();
                }
                // Largest x of this lane (NaN-propagating; -0 below +0), then the first
                // element equal to it (== treats -0 and +0 as equal).
                float m = x[0];
#pragma unroll
                for (int e = 1; e + 1 < 4 * MB; e += 2)
                    m = __builtin_elementwise_maximum(__builtin_elementwise_maximum(m, x[e]), x[e + 1]);
                m = __builtin_elementwise_maximum(m, x[4 * MB - 1]);
                uint32_t bu, bv;
                if (__ballot(m != m) == 0ull) {
                    int idx = 4 * MB - 1;
#pragma unroll
                    for (int e = 4 * MB - 1; e >= 0; --e) idx = (x[e] == m) ? e : idx;
                    bv = (uint32_t)(vlane + 32 * (idx >> 3) + (idx & 7));
                    bu = ordered_u32(m);
                } else {  // a NaN in this wave's block: the general ordered-key scan
                    bu = 0u;
                    bv = 0u;
#pragma unroll
                    for (int e = 0; e < 4 * MB; ++e) {
                        const uint32_t u = ordered_u32(x[e]);
                        if (u > bu) {
                            bu = u;
                            bv = (uint32_t)(vlane + 32 * (e >> 3) + (e & 7));
                        }
                    }
                }
                uint64_t best = (bv < (uint32_t)V) ? (((uint64_t)bu << 32) | (uint64_t)(~bv)) : 0ull;
                best = umax64(best, shfl_xor_u64(best, 16));
                best = umax64(best, shfl_xor_u64(best, 32));
                if (g == 0) {
                    const int j = rb * 16 + n16;
                    if (j < RC) atomicMax((unsigned long long*)&L.best[l0 + j], (unsigned long long)best);
                }
            }
        }
    }
}

// Best key over the waves, raised into the device-wide key of each request by an
// atomic max that returns the old value (so a later s_waitcnt covers its completion).
// Every workgroup raises every request's key: measured cheaper than reading the key
// first to skip atomics that cannot win.
template <int KS>
__device__ __forceinline__ void publish_rows(const ChainLds<KS>& L, uint64_t* keys, int R, int pos, int c0, int RC,
                                             int l0) {
    for (int j = threadIdx.x; j < RC; j += kNT) {
        const uint64_t b = L.best[l0 + j];
        if (b) {
            const uint64_t old =
                __hip_atomic_fetch_max(&keys[(size_t)pos * R + c0 + j], b, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            asm volatile("" ::"v"(old));
        }
    }
}

template <bool VEC>
__device__ __forceinline__ void prefetch_rows(BaseFrag (&pre)[kPF], const uint16_t* __restrict__ base, int R, int K,
                                              int V, int pos, int c0, int RC, int vb) {
    const int lane = threadIdx.x & 63;
    const int nRB = (RC + 15) >> 4;
#pragma unroll
    for (int q = 0; q < kPF; ++q)
        if (q < nRB) load_base<VEC>(pre[q], base, c0 + q * 16 + (lane & 15), R, K, V, pos, vb + 8 * (lane >> 4));
}

// One launch per position, one vocabulary tile per workgroup.  KS = padded rank / 32,
// VEC = V % 8 == 0 (16-byte base loads).
template <int KS, bool VEC>
__global__ __launch_bounds__(kNT, 1) void chain_pos_bf16_kernel(
    const uint16_t* __restrict__ base, const uint16_t* __restrict__ A, const uint16_t* __restrict__ Bt,
    const int32_t* __restrict__ prev0, uint64_t* __restrict__ keys, int32_t* __restrict__ tokens,
    float* __restrict__ logits, uint32_t* __restrict__ status, int R, int K, int V, int rank, int pos) {
    __shared__ __attribute__((aligned(16))) ChainLds<KS> L;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int vb = blockIdx.x * kTileV + w * kWV;
    bf16x8 bt[kMB][KS];
    load_bt<KS>(bt, Bt, V, rank, vb, lane & 15, lane >> 4);
    for (int c0 = 0; c0 < R; c0 += kReqChunk) {
        const int RC = min(kReqChunk, R - c0);
        BaseFrag pre[kPF];
        prefetch_rows<VEC>(pre, base, R, K, V, pos, c0, RC, vb);
        if (c0 > 0) __syncthreads();  // the previous chunk is done with the LDS
        decode_rows(L.prev, L.best, prev0, keys, tokens, status, R, K, V, pos, c0, RC, 0);
        __syncthreads();
        gather_rows<KS>(L, A, rank, RC, 0);
        __syncthreads();
        score_rows<KS, VEC>(L, bt, pre, base, logits, R, K, V, pos, c0, RC, 0, vb);
        __syncthreads();
        publish_rows<KS>(L, keys, R, pos, c0, RC, 0);
    }
}

// Grid barrier.  Everything workgroups exchange inside the launch -- the argmax keys
// and these counters -- moves only through agent-scope atomics: read-modify-writes
// that return their old value, and loads that bypass the per-XCD L2 caches.  No
// agent-scope fence is used (on this part such a fence writes back or invalidates
// whole L2 caches): a workgroup counts itself in only after each of its threads has
// received the results of its own key atomics, and a waiting workgroup reads keys
// only after thread 0 has seen the full count.  A poll budget bounds the wait.
__device__ __forceinline__ void grid_wait(const uint32_t* ctr, uint32_t target, uint32_t* status) {
    if (threadIdx.x == 0) {
        long n = 0;
        while (__hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < target) {
            if (++n > kSpinLimit) {
                raise_status(status, kStatusSyncTimeout);
                break;
            }
            __builtin_amdgcn_s_sleep(1);
        }
    }
    __syncthreads();
}

__device__ __forceinline__ void grid_arrive(uint32_t* ctr) {
    __builtin_amdgcn_s_waitcnt(0);  // this thread's key atomics have returned
    __syncthreads();
    if (threadIdx.x == 0) __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// All K positions in one cooperative launch (R <= 256, gridDim.x <= resident
// workgroups).  Requests are split into ng groups; phase (pos, g) scores group g
// at position pos and waits only for group g of position pos-1.
template <int KS, bool VEC>
__global__ __launch_bounds__(kNT, 1) void chain_persist_bf16_kernel(
    const uint16_t* __restrict__ base, const uint16_t* __restrict__ A, const uint16_t* __restrict__ Bt,
    const int32_t* __restrict__ prev0, uint64_t* __restrict__ keys, uint32_t* __restrict__ bar,
    int32_t* __restrict__ tokens, float* __restrict__ logits, uint32_t* __restrict__ status, int R, int K, int V,
    int rank, int ng) {
    __shared__ __attribute__((aligned(16))) ChainLds<KS> L;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int vb = blockIdx.x * kTileV + w * kWV;
    const int RG = (((R + ng - 1) / ng) + 15) & ~15;  // requests per group (multiple of 16)
    bf16x8 bt[kMB][KS];
    load_bt<KS>(bt, Bt, V, rank, vb, lane & 15, lane >> 4);
    for (int pos = 0; pos < K; ++pos) {
        for (int g = 0; g < ng; ++g) {
            const int c0 = g * RG;
            if (c0 >= R) break;
            const int RC = min(RG, R - c0);
            BaseFrag pre[kPF];
            prefetch_rows<VEC>(pre, base, R, K, V, pos, c0, RC, vb);
            if (pos > 0) grid_wait(&bar[(pos - 1) * kMaxGroups + g], gridDim.x, status);
            decode_rows(L.prev, L.best, prev0, keys, tokens, status, R, K, V, pos, c0, RC, c0);
            __syncthreads();
            gather_rows<KS>(L, A, rank, RC, c0);
            __syncthreads();
            score_rows<KS, VEC>(L, bt, pre, base, logits, R, K, V, pos, c0, RC, c0, vb);
            __syncthreads();
            publish_rows<KS>(L, keys, R, pos, c0, RC, c0);
            grid_arrive(&bar[pos * kMaxGroups + g]);
        }
    }
}

// fp32 factors: one thread per vocabulary entry, fused multiply-add in increasing k.
__global__ __launch_bounds__(kF32Threads) void chain_pos_f32_kernel(
    const float* __restrict__ base, const float* __restrict__ A, const float* __restrict__ Bt,
    const int32_t* __restrict__ prev0, uint64_t* __restrict__ keys, int32_t* __restrict__ tokens,
    float* __restrict__ logits, uint32_t* __restrict__ status, int R, int K, int V, int rank, int pos) {
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
            const float x = base[((size_t)r * K + pos) * V + v] + acc;
            if (logits != nullptr) logits[((size_t)r * K + pos) * V + v] = x;
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
template <int KS, bool VEC>
hipError_t launch_persist(const ChainArgs& a, int grid, int ng, hipStream_t s) {
    const void* fn = (const void*)chain_persist_bf16_kernel<KS, VEC>;
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
    const uint16_t* base = (const uint16_t*)a.base;
    const uint16_t* A = (const uint16_t*)a.A;
    const uint16_t* Bt = (const uint16_t*)a.Bt;
    const int32_t* prev0 = a.prev0;
    uint64_t* keys = a.keys;
    uint32_t* bar = a.bar;
    int32_t* tokens = a.tokens;
    float* logits = a.logits;
    uint32_t* status = a.status;
    int R = a.R, K = a.K, V = a.V, rank = a.rank;
    void* args[] = {&base, &A, &Bt, &prev0, &keys, &bar, &tokens, &logits, &status, &R, &K, &V, &rank, &ng};
    return hipLaunchCooperativeKernel(fn, dim3(grid), dim3(kNT), args, 0, s);
}

template <int KS, bool VEC>
hipError_t launch_bf16(const ChainArgs& a, int grid, hipStream_t s) {
    if (a.R <= kReqChunk) {
        const int ng = 1;  // two alternating groups only pay off once their sync work overlaps
        const hipError_t e = launch_persist<KS, VEC>(a, grid, ng, s);
        if (e != hipErrorCooperativeLaunchTooLarge) return e;
        (void)hipGetLastError();  // clear the sticky launch error before falling back
    }
    for (int pos = 0; pos < a.K; ++pos) {
        hipLaunchKernelGGL((chain_pos_bf16_kernel<KS, VEC>), dim3(grid), dim3(kNT), 0, s, (const uint16_t*)a.base,
                           (const uint16_t*)a.A, (const uint16_t*)a.Bt, a.prev0, a.keys, a.tokens, a.logits,
                           a.status, a.R, a.K, a.V, a.rank, pos);
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
                           a.R, a.K, a.V, a.rank, pos);
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
