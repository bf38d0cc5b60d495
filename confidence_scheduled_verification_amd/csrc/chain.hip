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
//   * A workgroup (4 waves) owns vocabulary tiles of 4*16*MB entries; each wave
//     keeps its tile's Bt fragments in registers and sweeps all requests in
//     blocks of 16.  The gathered key rows A[prev_r,:] of up to 256 requests are
//     staged once per launch in LDS and shared by the 4 waves.
//   * Each lane's accumulator holds 8 consecutive vocabulary entries of one
//     request per pair of M blocks (the M-row -> vocabulary mapping is permuted
//     to make that so), so base logits stream in as 16-byte coalesced loads,
//     prefetched PF request blocks ahead.
//   * The argmax is fused: 64-bit keys (value, ~index) reduced in registers, by
//     cross-lane shuffles, across the 4 waves in LDS, and across workgroups by
//     one 64-bit atomicMax per request per workgroup (skipped when the stored
//     key is already larger).  The next position's launch decodes the winners.
//   * Grids are capped at the CU count (the 141 KB of LDS allows one workgroup
//     per CU); workgroups loop over tiles rather than launching ~10^5 tiny
//     blocks, which the MAX worklog found dispatch-bound ("Correctness, then
//     1.3x").
#include "common.h"
#include "kernels.h"

namespace dspark {

namespace {

constexpr int kChainThreads = 256;
constexpr int kReqChunk = 256;  // requests whose key rows are staged in LDS at once

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

// One launch per position.  KS = padded rank / 32, MB = 16-row M blocks per wave,
// PF = request blocks of base prefetched ahead, VEC = V % 8 == 0 (16-byte loads).
template <int KS, int MB, int PF, bool VEC>
__global__ __launch_bounds__(kChainThreads, 1) void chain_pos_bf16_kernel(
    const uint16_t* __restrict__ base, const uint16_t* __restrict__ A, const uint16_t* __restrict__ Bt,
    const int32_t* __restrict__ prev0, uint64_t* __restrict__ keys, int32_t* __restrict__ tokens,
    float* __restrict__ logits, uint32_t* __restrict__ status, int R, int K, int V, int rank, int pos) {
    constexpr int RP = 32 * KS;     // padded rank
    constexpr int LROW = RP + 8;    // LDS row stride in bf16 elements (16-byte pad spreads banks)
    constexpr int SEGS = RP / 8;    // 16-byte segments per key row
    constexpr int WV = 16 * MB;     // vocabulary entries per wave
    constexpr int TV = 4 * WV;      // vocabulary entries per workgroup tile
    __shared__ __attribute__((aligned(16))) uint16_t s_a[kReqChunk * LROW];
    __shared__ uint64_t s_best[4][kReqChunk];
    __shared__ int32_t s_prev[kReqChunk];

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int n16 = lane & 15, g = lane >> 4;
    const int ntiles = (V + TV - 1) / TV;

    for (int c0 = 0; c0 < R; c0 += kReqChunk) {
        const int RC = min(kReqChunk, R - c0);
        const int nRB = (RC + 15) >> 4;
        for (int j = tid; j < RC; j += kChainThreads) {
            const int p = decode_prev(prev0, keys, status, R, V, pos, c0 + j, blockIdx.x == 0);
            s_prev[j] = p;
            if (pos > 0 && blockIdx.x == 0) tokens[(size_t)(c0 + j) * K + (pos - 1)] = p;
        }
        for (int j = tid; j < 4 * kReqChunk; j += kChainThreads) (&s_best[0][0])[j] = 0ull;
        __syncthreads();

        // Gather the key rows A[prev_r, :] of this chunk into LDS (zero past rank and R).
        for (int idx = tid; idx < nRB * 16 * SEGS; idx += kChainThreads) {
            const int j = idx / SEGS, s = idx - j * SEGS;
            u32x4 val = {0u, 0u, 0u, 0u};
            if (j < RC && s * 8 < rank) val = *(const u32x4*)(A + (size_t)s_prev[j] * rank + s * 8);
            *(u32x4*)(s_a + j * LROW + s * 8) = val;
        }
        __syncthreads();

        for (int t = blockIdx.x; t < ntiles; t += gridDim.x) {
            const int vb = t * TV + w * WV;
            // Bt fragments of this wave's vocabulary rows.  M row m of block mb is
            // vocabulary vb + 32*(mb/2) + 8*(m/4) + 4*(mb%2) + m%4, which puts 8
            // consecutive entries in each lane's accumulator pair.
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
            const int vlane = vb + 8 * g;  // first vocabulary entry of this lane's first group

            BaseFrag<MB> pre[PF];
#pragma unroll
            for (int q = 0; q < PF; ++q)
                if (q < nRB) load_base<MB, VEC>(pre[q], base, c0 + q * 16 + n16, R, K, V, pos, vlane);

            for (int rb0 = 0; rb0 < nRB; rb0 += PF) {
#pragma unroll
                for (int q = 0; q < PF; ++q) {
                    const int rb = rb0 + q;
                    if (rb < nRB) {
                        const BaseFrag<MB> cur = pre[q];
                        if (rb + PF < nRB)
                            load_base<MB, VEC>(pre[q], base, c0 + (rb + PF) * 16 + n16, R, K, V, pos, vlane);

                        f32x4 acc[MB];
#pragma unroll
                        for (int mb = 0; mb < MB; ++mb) acc[mb] = f32x4{0.f, 0.f, 0.f, 0.f};
                        const uint16_t* arow = s_a + (rb * 16 + n16) * LROW + g * 8;
#pragma unroll
                        for (int ks = 0; ks < KS; ++ks) {
                            const bf16x8 bfr = *(const bf16x8*)(arow + ks * 32);
#pragma unroll
                            for (int mb = 0; mb < MB; ++mb)
                                acc[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bt[mb][ks], bfr, acc[mb], 0, 0, 0);
                        }

                        const int r = c0 + rb * 16 + n16;
                        uint64_t best = 0ull;
#pragma unroll
                        for (int p = 0; p < MB / 2; ++p) {
                            const int v0 = vlane + 32 * p;
#pragma unroll
                            for (int e = 0; e < 8; ++e) {
                                const uint32_t h = (cur.q[p][e >> 1] >> (16 * (e & 1))) & 0xFFFFu;
                                const float x = acc[2 * p + (e >> 2)][e & 3] + bf16_bits_to_f32(h);
                                const int v = v0 + e;
                                if (v < V) {
                                    best = umax64(best, argmax_key(x, (uint32_t)v));
                                    if (logits != nullptr && r < R) logits[((size_t)r * K + pos) * V + v] = x;
                                }
                            }
                        }
                        best = umax64(best, shfl_xor_u64(best, 16));
                        best = umax64(best, shfl_xor_u64(best, 32));
                        if (g == 0) {
                            const int j = rb * 16 + n16;
                            if (j < RC) s_best[w][j] = umax64(s_best[w][j], best);
                        }
                    }
                }
            }
        }
        __syncthreads();
        for (int j = tid; j < RC; j += kChainThreads) {
            const uint64_t b = umax64(umax64(s_best[0][j], s_best[1][j]), umax64(s_best[2][j], s_best[3][j]));
            if (b) publish_key(&keys[(size_t)pos * R + c0 + j], b);
        }
        __syncthreads();
    }
}

// fp32 factors: one thread per vocabulary entry, fused multiply-add in increasing k.
__global__ __launch_bounds__(kChainThreads) void chain_pos_f32_kernel(
    const float* __restrict__ base, const float* __restrict__ A, const float* __restrict__ Bt,
    const int32_t* __restrict__ prev0, uint64_t* __restrict__ keys, int32_t* __restrict__ tokens,
    float* __restrict__ logits, uint32_t* __restrict__ status, int R, int K, int V, int rank, int pos) {
    __shared__ uint64_t s_wbest[kChainThreads / 64];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int v = blockIdx.x * kChainThreads + tid;
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
            for (int q = 1; q < kChainThreads / 64; ++q) b = umax64(b, s_wbest[q]);
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

template <int KS, int MB, int PF, bool VEC>
hipError_t launch_bf16(const ChainArgs& a, int pos, int grid, hipStream_t s) {
    hipLaunchKernelGGL((chain_pos_bf16_kernel<KS, MB, PF, VEC>), dim3(grid), dim3(kChainThreads), 0, s,
                       (const uint16_t*)a.base, (const uint16_t*)a.A, (const uint16_t*)a.Bt, a.prev0, a.keys,
                       a.tokens, a.logits, a.status, a.R, a.K, a.V, a.rank, pos);
    return hipGetLastError();
}

template <int KS>
hipError_t launch_bf16_ks(const ChainArgs& a, int pos, int grid, hipStream_t s) {
    constexpr int MB = 4, PF = 4;
    if (a.V % 8 == 0) return launch_bf16<KS, MB, PF, true>(a, pos, grid, s);
    return launch_bf16<KS, MB, PF, false>(a, pos, grid, s);
}

}  // namespace

int chain_tile_vocab() { return 4 * 16 * 4; }

hipError_t launch_zero_keys(uint64_t* keys, size_t n, hipStream_t s) {
    if (n == 0) return hipSuccess;
    const int grid = (int)std::min<size_t>((n + 255) / 256, 1024);
    hipLaunchKernelGGL(fill_u64_kernel, dim3(grid), dim3(256), 0, s, keys, n);
    return hipGetLastError();
}

hipError_t launch_chain_positions(const ChainArgs& a, int num_cu, hipStream_t s) {
    if (a.dtype == 1) {
        const int ntiles = (a.V + chain_tile_vocab() - 1) / chain_tile_vocab();
        const int grid = std::max(1, std::min(ntiles, num_cu));
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
        const int grid = (a.V + kChainThreads - 1) / kChainThreads;
        for (int pos = 0; pos < a.K; ++pos) {
            hipLaunchKernelGGL(chain_pos_f32_kernel, dim3(grid), dim3(kChainThreads), 0, s, (const float*)a.base,
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
