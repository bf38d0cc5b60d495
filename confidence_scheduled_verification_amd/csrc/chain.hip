// Stage 1 of the chain-and-schedule pass: semi-autoregressive chaining of a
// K-token draft block (DSpark summary "How DSpark Speeds Up LLM Inference",
// section "Draft better"; MAX worklog "DSpark on MAX", section "What DSpark is",
// item 3).  Position i of request r scores every vocabulary entry v as
//     x[r,i,v] = base[r,i,v] + <A[prev_r,:], Bt[v,:]>
// and takes the argmax; the winner keys position i+1.
//
// gfx950 design (one launch per position, positions are serially dependent):
//   * The low-rank bias is the contraction (R x rank) . (rank x V).  It runs on
//     the bf16 matrix cores (v_mfma_f32_16x16x32_bf16, fp32 accumulation) in the
//     transposed form D[v, r] = Bt[v,:] . A[prev_r,:]: vocabulary rows are the
//     MFMA M dimension, requests the N dimension.
//   * A workgroup of WAVES waves owns one vocabulary tile of WAVES*16*MB
//     entries; each wave keeps its rows' Bt fragments in registers and sweeps
//     all requests in blocks of 16.  The gathered key rows A[prev_r,:] of up to
//     256 requests are staged once per launch in LDS and shared by the waves.
//   * Everything that does not depend on the previous position -- the Bt
//     fragments and the first base blocks -- is requested before the previous
//     position's winners are decoded, so those loads overlap the key-row gather,
//     and the gather itself keeps all of a thread's loads in flight at once.
//   * Each lane's accumulator holds 8 consecutive vocabulary entries of one
//     request per pair of M blocks (the M-row -> vocabulary mapping is permuted
//     to make that so), so base logits stream in as 16-byte coalesced loads,
//     prefetched PF request blocks ahead.
//   * The argmax is fused: per lane an ordered 32-bit key and the first index of
//     its maximum, then 64-bit keys (value, ~index) reduced by cross-lane
//     shuffles, across waves in LDS, and across workgroups by one 64-bit
//     atomicMax per request per workgroup (skipped when the stored key is
//     already larger).  The next position's launch decodes the winners.
//   * About 250 workgroups of 512 threads per launch for a 129280-entry
//     vocabulary: enough to fill the CUs without ~10^5 tiny blocks, which the MAX
//     worklog found dispatch-bound ("Correctness, then 1.3x").
#include "common.h"
#include "kernels.h"

namespace dspark {

namespace {

constexpr int kReqChunk = 256;   // requests whose key rows are staged in LDS at once
constexpr int kWaves = 8;        // waves per workgroup of the bf16 kernel
constexpr int kMB = 4;           // 16-row M blocks per wave
constexpr int kPF = 3;           // request blocks of base prefetched ahead
constexpr int kTileV = kWaves * 16 * kMB;
constexpr int kF32Threads = 256;

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
    // range; the clamp only guarantees that the gather below can never leave A.
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

// Base logits of one request block for one wave: MB/2 groups of 8 consecutive
// vocabulary entries per lane (16 bytes each).
template <int MB>
struct BaseFrag {
    u32x4 q[MB / 2];
};

template <int MB, bool VEC>
__device__ __forceinline__ void load_base(BaseFrag<MB>& f, const uint16_t* __restrict__ base, int r, int R, int K,
                                          int V, int pos, int vlane) {
    const bool row_ok = r < R;
    const uint16_t* row = base + ((size_t)(row_ok ? r : 0) * K + pos) * (size_t)V;
#pragma unroll
    for (int p = 0; p < MB / 2; ++p) {
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

// One launch per position, one vocabulary tile per workgroup.  KS = padded rank / 32,
// VEC = V % 8 == 0 (16-byte base loads).
template <int KS, bool VEC>
__global__ __launch_bounds__(kWaves * 64, 1) void chain_pos_bf16_kernel(
    const uint16_t* __restrict__ base, const uint16_t* __restrict__ A, const uint16_t* __restrict__ Bt,
    const int32_t* __restrict__ prev0, uint64_t* __restrict__ keys, int32_t* __restrict__ tokens,
    float* __restrict__ logits, uint32_t* __restrict__ status, int R, int K, int V, int rank, int pos) {
    constexpr int MB = kMB, PF = kPF, NT = kWaves * 64;
    constexpr int RP = 32 * KS;     // padded rank
    constexpr int LROW = RP + 8;    // LDS row stride in bf16 elements (16-byte pad spreads banks)
    constexpr int SEGS = RP / 8;    // 16-byte segments per key row
    constexpr int WV = 16 * MB;     // vocabulary entries per wave
    constexpr int GATHER = (kReqChunk * SEGS + NT - 1) / NT;  // key-row segments per thread
    constexpr int GB = GATHER < 8 ? GATHER : 8;                 // of which in flight at once
    __shared__ __attribute__((aligned(16))) uint16_t s_a[kReqChunk * LROW];
    __shared__ uint64_t s_best[kWaves][kReqChunk];
    __shared__ int32_t s_prev[kReqChunk];

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int n16 = lane & 15, g = lane >> 4;
    const int vb = blockIdx.x * kTileV + w * WV;
    const int vlane = vb + 8 * g;  // first vocabulary entry of this lane's first group

    // Bt fragments of this wave's vocabulary rows (independent of the previous
    // position).  M row m of block mb is vocabulary vb + 32*(mb/2) + 8*(m/4) +
    // 4*(mb%2) + m%4, which puts 8 consecutive entries in each lane's accumulator pair.
    bf16x8 bt[MB][KS];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
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

    for (int c0 = 0; c0 < R; c0 += kReqChunk) {
        const int RC = min(kReqChunk, R - c0);
        const int nRB = (RC + 15) >> 4;

        // First base blocks of this chunk (independent of the previous position).
        BaseFrag<MB> pre[PF];
#pragma unroll
        for (int q = 0; q < PF; ++q)
            if (q < nRB) load_base<MB, VEC>(pre[q], base, c0 + q * 16 + n16, R, K, V, pos, vlane);

        if (c0 > 0) __syncthreads();  // the previous chunk is done with s_a / s_best / s_prev
        for (int j = tid; j < RC; j += NT) {
            const int p = decode_prev(prev0, keys, status, R, V, pos, c0 + j, blockIdx.x == 0);
            s_prev[j] = p;
            if (pos > 0 && blockIdx.x == 0) tokens[(size_t)(c0 + j) * K + (pos - 1)] = p;
        }
        for (int j = tid; j < kWaves * kReqChunk; j += NT) (&s_best[0][0])[j] = 0ull;
        __syncthreads();

        // Gather the key rows A[prev_r, :] of this chunk into LDS (zero past rank and
        // R), GB independent loads in flight per thread before their stores.
#pragma unroll
        for (int q0 = 0; q0 < GATHER; q0 += GB) {
            u32x4 seg[GB];
#pragma unroll
            for (int q = 0; q < GB; ++q) {
                const int idx = tid + (q0 + q) * NT;
                const int j = idx / SEGS, s = idx - j * SEGS;
                seg[q] = u32x4{0u, 0u, 0u, 0u};
                if (q0 + q < GATHER && j < RC && s * 8 < rank)
                    seg[q] = *(const u32x4*)(A + (size_t)s_prev[j] * rank + s * 8);
            }
#pragma unroll
            for (int q = 0; q < GB; ++q) {
                const int idx = tid + (q0 + q) * NT;
                const int j = idx / SEGS, s = idx - j * SEGS;
                if (q0 + q < GATHER && j < nRB * 16) *(u32x4*)(s_a + j * LROW + s * 8) = seg[q];
            }
        }
        __syncthreads();

        for (int rb0 = 0; rb0 < nRB; rb0 += PF) {
#pragma unroll
            for (int q = 0; q < PF; ++q) {
                const int rb = rb0 + q;
                if (rb < nRB) {
                    // The accumulator starts at the base logits (bf16 -> fp32 is exact), so the
                    // matrix cores add the bias.  Lane element e (0..15) is vocabulary
                    // vlane + 32*(e/8) + e%8, held in acc[2*(e/8) + (e%8)/4][e%4].
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
                    if (rb + PF < nRB)
                        load_base<MB, VEC>(pre[q], base, c0 + (rb + PF) * 16 + n16, R, K, V, pos, vlane);
                    const uint16_t* arow = s_a + (rb * 16 + n16) * LROW + g * 8;
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
                    if (vb + WV > V) {  // ragged last tile: entries past V cannot win
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
                        if (j < RC) s_best[w][j] = best;
                    }
                }
            }
        }
        __syncthreads();
        for (int j = tid; j < RC; j += NT) {
            uint64_t b = s_best[0][j];
#pragma unroll
            for (int q = 1; q < kWaves; ++q) b = umax64(b, s_best[q][j]);
            if (b) publish_key(&keys[(size_t)pos * R + c0 + j], b);
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

template <int KS, bool VEC>
hipError_t launch_bf16(const ChainArgs& a, int pos, int grid, hipStream_t s) {
    hipLaunchKernelGGL((chain_pos_bf16_kernel<KS, VEC>), dim3(grid), dim3(kWaves * 64), 0, s,
                       (const uint16_t*)a.base, (const uint16_t*)a.A, (const uint16_t*)a.Bt, a.prev0, a.keys,
                       a.tokens, a.logits, a.status, a.R, a.K, a.V, a.rank, pos);
    return hipGetLastError();
}

template <int KS>
hipError_t launch_bf16_ks(const ChainArgs& a, int pos, int grid, hipStream_t s) {
    if (a.V % 8 == 0) return launch_bf16<KS, true>(a, pos, grid, s);
    return launch_bf16<KS, false>(a, pos, grid, s);
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
        for (int pos = 0; pos < a.K; ++pos) {
            hipError_t e;
            if (ks <= 1) e = launch_bf16_ks<1>(a, pos, grid, s);
            else if (ks <= 2) e = launch_bf16_ks<2>(a, pos, grid, s);
            else if (ks <= 4) e = launch_bf16_ks<4>(a, pos, grid, s);
            else e = launch_bf16_ks<8>(a, pos, grid, s);
            if (e != hipSuccess) return e;
        }
    } else {
        const int grid = (a.V + kF32Threads - 1) / kF32Threads;
        for (int pos = 0; pos < a.K; ++pos) {
            hipLaunchKernelGGL(chain_pos_f32_kernel, dim3(grid), dim3(kF32Threads), 0, s, (const float*)a.base,
                               (const float*)a.A, (const float*)a.Bt, a.prev0, a.keys, a.tokens, a.logits,
                               a.status, a.R, a.K, a.V, a.rank, pos);
            const hipError_t e = hipGetLastError();
            if (e != hipSuccess) return e;
        }
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
