// Device code of stage 1 (the chain), shared by the chain kernels and the
// single-launch step kernel.  Design notes at the top of chain.hip.
#pragma once

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
#define DSPARK_CHAIN_PF 4
#endif
#ifndef DSPARK_BASE_AUX
#define DSPARK_BASE_AUX 0
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

// Rows past R and entries past V load in-range data that no caller uses (rows past
// R are never published; entries past V are masked before the argmax), so the
// loads need no lane masks.
template <bool VEC>
__device__ __forceinline__ void load_base(BaseFrag& f, const uint16_t* __restrict__ base, int r, int R, int K, int V,
                                          int pos, int vlane) {
    const uint16_t* row = base + ((size_t)(r < R ? r : 0) * K + pos) * (size_t)V;
#pragma unroll
    for (int p = 0; p < kMB / 2; ++p) {
        const int v0 = vlane + 32 * p;
        if (VEC) {
            f.q[p] = __builtin_nontemporal_load((const u32x4*)(row + min(v0, V - 8)));
        } else {
            uint32_t h[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) h[e] = (uint32_t)row[min(v0 + e, V - 1)];
            f.q[p] = u32x4{h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16)};
        }
    }
}

// Base blocks for the pipelined scorer.  With 8 | V each lane's 16-byte groups are
// aligned, and the blocks of one segment (requests c0.. at one position) are read
// through a buffer resource whose base is the segment's first row at that position
// and whose size ends at the end of the base tensor: rows past R read as zero
// (hardware range check), entries past V read in-range data that the scorer masks.
// A lane's offset is its loop-invariant (n16*K*V + vlane)*2 plus t blocks of
// 16*K*V*2 bytes, all in 32 bits (K*V <= DSPARK_MAX_KV_BF16).  The resource is built
// once per segment, so a block costs one vector add.  Without 8 | V the
// element-wise clamped form is used.
struct BaseSrc {
    const uint16_t* base;
    uint64_t bytes;    // R*K*V*2
    uint32_t voff;     // (n16*K*V + vlane) * 2
    uint32_t bstride;  // 16*K*V*2: one block of 16 rows
};

__device__ __forceinline__ BaseSrc base_src(const uint16_t* base, int R, int K, int V, int n16, int vlane) {
    return BaseSrc{base, (uint64_t)R * K * V * 2, (uint32_t)(((uint64_t)n16 * K * V + vlane) * 2),
                   (uint32_t)(16u * (uint32_t)K * (uint32_t)V * 2u)};
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t seg_rsrc(const BaseSrc& src, int c0, int pos, int K, int V) {
    const uint64_t o = ((uint64_t)c0 * K + pos) * (uint64_t)V * 2;
    const uint64_t rem = o < src.bytes ? src.bytes - o : 0;
    return __builtin_amdgcn_make_buffer_rsrc((void*)((const char*)src.base + o), 0,
                                             (int)(uint32_t)(rem < 0xFFFFFFFFull ? rem : 0xFFFFFFFFull), 0x00020000);
}

// Block t of the segment whose resource is rs (VEC), or of segment (c0, pos).
template <bool VEC>
__device__ __forceinline__ void load_block(BaseFrag& f, const BaseSrc& src, __amdgpu_buffer_rsrc_t rs, int t, int c0,
                                           int pos, int R, int K, int V, int n16, int vlane) {
    if (VEC) {
        const uint32_t off = src.voff + (uint32_t)t * src.bstride;
#pragma unroll
        for (int p = 0; p < kMB / 2; ++p)
            f.q[p] = __builtin_amdgcn_raw_buffer_load_b128(rs, (int)(off + 64 * p), 0, DSPARK_BASE_AUX);
    } else {
        load_base<false>(f, src.base, c0 + t * 16 + n16, R, K, V, pos, vlane);
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

// Thread index the compiler cannot treat as loop-invariant: per-phase index math is
// then recomputed inside the position loop instead of being held in registers
// across the scoring sweep, which needs nearly all of them.
__device__ __forceinline__ int phase_tid() {
    int t = threadIdx.x;
    asm volatile("" : "+v"(t));
    return t;
}

// Requests [c0, c0+RC) use LDS rows l0 .. l0+RC; rows RC .. `rows` (the padded
// count the scoring form works on) hold zero key rows and are never published.

// Rows the pipelined scorer sweeps: whole ring cycles of PF blocks of 16 (PF base
// blocks in flight per wave: kPF, or 2 for a single group of at most 64 requests, where
// a 4-block ring would sweep padding rows -- 32 requests in a 64-row cycle).
static_assert(kPF % 2 == 0 && kReqChunk % (16 * kPF) == 0, "ring cycles must tile an LDS chunk of requests");
template <int PF = kPF>
__device__ __forceinline__ int fast_rows(int RC) {
    static_assert(PF % 2 == 0 && kReqChunk % (16 * PF) == 0, "ring cycles must tile an LDS chunk of requests");
    constexpr int C = 16 * PF;
    return (RC + C - 1) / C * C;
}

__device__ __forceinline__ void decode_rows(int32_t* s_prev, uint64_t* s_best, const int32_t* prev0,
                                            const uint64_t* keys, int32_t* tokens, uint32_t* status, int R, int K,
                                            int V, int pos, int c0, int RC, int l0, int rows) {
    const int tid = phase_tid();
    for (int j = tid; j < RC; j += kNT) {
        const int p = decode_prev(prev0, keys, status, R, V, pos, c0 + j, blockIdx.x == 0);
        s_prev[l0 + j] = p;
        if (pos > 0 && blockIdx.x == 0 && tokens != nullptr) tokens[(size_t)(c0 + j) * K + (pos - 1)] = p;
    }
    for (int j = tid; j < rows; j += kNT) s_best[l0 + j] = 0ull;
}

// A raw buffer resource (stride 0) over `bytes` bytes at p: loads at offsets past the
// end return zeros.
__device__ __forceinline__ u32x4 buffer_rsrc(const void* p, uint32_t bytes) {
    const uint64_t a = (uint64_t)(uintptr_t)p;
    return u32x4{(uint32_t)a, (uint32_t)(a >> 32) & 0xFFFFu, bytes, 0x00020000u};
}

// LDS byte address of a pointer into a __shared__ object.
__device__ __forceinline__ uint32_t lds_addr(const void* p) { return (uint32_t)(uintptr_t)p; }

// One wave instruction of a direct-to-LDS 16-byte buffer load: lane i's 16 bytes at
// buffer offset voff land at LDS byte address lds + 16*i.  Issued through inline
// assembly so that the compiler does not order every later LDS read after it (it
// cannot tell the target rows from the ones being read); callers wait for it with
// an explicit s_waitcnt before reading what it wrote.
__device__ __forceinline__ void dma16_to_lds(const u32x4& rsrc, uint32_t lds, uint32_t voff) {
    uint32_t saved;  // M0 is the compiler's too: restore it
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %1\n\t"
        "s_nop 0\n\t"
        "buffer_load_dwordx4 %2, %3, 0 offen lds\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "s"(__builtin_amdgcn_readfirstlane(lds)), "v"(voff), "s"(rsrc)
        : "memory");
}

// Key rows A[prev_r, :] into LDS by direct-to-LDS buffer loads: the rows region is
// a sequence of 16-byte slots, SEGS data slots and one pad slot per row, and each
// wave instruction fills 64 consecutive slots (lane i -> slot base + i), so no data
// passes through registers and all of a workgroup's loads are in flight at once.
// Slots past rank, the pad slots and rows RC .. `rows` read out of the buffer's
// range and land as zeros.  Needs V * rank * 2 < 2^32.  WAIT: return only once this
// wave's slots have landed (otherwise a later s_waitcnt covers them).
template <int KS, bool WAIT = true>
__device__ __forceinline__ void gather_rows(ChainLds<KS>& L, const uint16_t* __restrict__ A, int V, int rank, int RC,
                                            int l0, int rows) {
    constexpr int SEGS = ChainLds<KS>::SEGS, SP = ChainLds<KS>::LROW / 8;
    static_assert(ChainLds<KS>::LROW % 8 == 0 && SP > SEGS, "rows are whole 16-byte slots with a pad");
    const int tid = phase_tid();
    const int lane = tid & 63, w = tid >> 6;
    const u32x4 rs = buffer_rsrc(A, (uint32_t)V * (uint32_t)rank * 2u);
    const int total = rows * SP;
    for (int t0 = w * 64; t0 < total; t0 += kNT) {
        const int t = t0 + lane;
        const int j = t / SP, sg = t - j * SP;
        uint32_t voff = 0xFFFFFFF0u;  // out of range: zeros
        if (j < RC && sg < SEGS && sg * 8 < rank) voff = ((uint32_t)L.prev[l0 + j] * (uint32_t)rank + sg * 8) * 2u;
        dma16_to_lds(rs, lds_addr(L.a + (l0 * SP + t0) * 8), voff);
    }
    if (WAIT) __builtin_amdgcn_s_waitcnt(0);  // this wave's slots have landed (the caller then syncs the workgroup)
}

// Probabilistic drafting: lane element e (vocabulary vlane + 32*(e/8) + e%8) of request r
// becomes its sampled value (x / temperature + a Gumbel variate, in base 2) from
// Philox4x32-10 word v % 4 at counter (v / 4, pos, r, 0) under the seed (one call per 4
// consecutive entries).
template <int NE>
__device__ __forceinline__ void perturb(float (&x)[NE], const SampleArgs& smp, int vlane, int pos, int r) {
    static_assert(NE == 16, "2 x 8 consecutive entries per lane");
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            uint32_t wd[4];
            philox4x32_10((uint32_t)(vlane + 32 * h + 4 * q) >> 2, (uint32_t)pos, (uint32_t)r, 0u, smp.k0, smp.k1, wd);
#pragma unroll
            for (int j = 0; j < 4; ++j) x[8 * h + 4 * q + j] = sampled_value(x[8 * h + 4 * q + j], smp.scale, wd[j]);
        }
    }
}

// Score the wave's 64 vocabulary rows against requests [c0, c0+RC) and raise each
// request's key in L.best[l0 + j] to this wave's best.  pre[] holds the first kPF
// base blocks of the range, already requested.  General form: optional logits
// output, ragged tiles, and an exact ordered-key scan for blocks holding a NaN.
// SAMPLE: the key ranks the sampled value (see perturb) instead of x, so the winner is
// a sample of softmax(x / temperature) (Gumbel-max); the logits output stays x.
template <int KS, bool VEC, bool SAMPLE = false>
__device__ __forceinline__ void score_generic(ChainLds<KS>& L, const bf16x8 (&bt)[kMB][KS], BaseFrag (&pre)[kPF],
                                              const uint16_t* __restrict__ base, float* __restrict__ logits, int R,
                                              int K, int V, int pos, int c0, int RC, int l0, int vb,
                                              const SampleArgs& smp = SampleArgs{}) {
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
                if (SAMPLE) perturb(x, smp, vlane, pos, r);
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

// Accumulators of one request block start at its base logits (bf16 -> fp32 is
// exact).  Lane element e (0..15) is vocabulary vlane + 32*(e/8) + e%8, held in
// acc[2*(e/8) + (e%8)/4][e%4].  MASK (ragged last tile): entries past V start at
// -inf; their Bt rows are zero, so they stay -inf and never win.
template <bool MASK, bool VEC>
__device__ __forceinline__ void init_acc(f32x4 (&acc)[kMB], const BaseFrag& f, int vlane, int V) {
    constexpr float kNegInf = -__builtin_huge_valf();
#pragma unroll
    for (int p = 0; p < kMB / 2; ++p) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const uint32_t w0 = f.q[p][2 * h], w1 = f.q[p][2 * h + 1];
            float x[4] = {__uint_as_float(w0 << 16), __uint_as_float(w0 & 0xFFFF0000u), __uint_as_float(w1 << 16),
                          __uint_as_float(w1 & 0xFFFF0000u)};
            if (MASK) {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    // with 8 | V a group of 8 is wholly in or out
                    const bool ok = VEC ? (vlane + 32 * p < V) : (vlane + 32 * p + 4 * h + j < V);
                    x[j] = ok ? x[j] : kNegInf;
                }
            }
            acc[2 * p + h] = f32x4{x[0], x[1], x[2], x[3]};
        }
    }
}

// acc += Bt rows x the block's 16 key rows (arow: this lane's row and k-chunk in LDS).
template <int KS>
__device__ __forceinline__ void mfma_block(f32x4 (&acc)[kMB], const bf16x8 (&bt)[kMB][KS], const uint16_t* arow) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        const bf16x8 bfr = *(const bf16x8*)(arow + ks * 32);
#pragma unroll
        for (int mb = 0; mb < kMB; ++mb)
            acc[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bt[mb][ks], bfr, acc[mb], 0, 0, 0);
    }
}

// Argmax of one scored block, without branches, in 8 slices that a pipeline
// stage spreads between its matrix-core instructions (source order is what the
// compiler keeps when a reordered schedule would need more registers).  Per lane:
// NaN-propagating maximum3 tree, then the first element equal to it, then one LDS
// atomic max of the lane's 64-bit key (ordered value, ~index).  The 4 lanes of a
// request raise the same LDS word, so the atomic itself takes their maximum and, among
// equal values, the smallest index: no cross-lane exchange is needed.  Exact unless
// the block holds a NaN: then the lane's key is (NaN rank, index bits 0), never above
// the exact key, and the wave's NaN mask tells the caller to rescore with the exact
// scan.  Entries past V arrive as -inf and sit at larger indices than every real entry
// of the wave, so they cannot be chosen.
struct Argmax {
    static constexpr int NE = 4 * kMB;
    float x[NE];
    float m;
    uint32_t off, c;

    __device__ __forceinline__ explicit Argmax(const f32x4 (&acc)[kMB]) {
#pragma unroll
        for (int e = 0; e < NE; ++e) x[e] = acc[2 * (e >> 3) + ((e & 7) >> 2)][e & 3];
    }

    // slice s in 0..7
    __device__ __forceinline__ void slice(int s, uint64_t* best, int vlane, uint64_t& nan_mask) {
        constexpr int H = NE / 2, Q = NE / 4;
        if (s == 0) {
            m = x[0];
#pragma unroll
            for (int e = 1; e + 1 < H; e += 2)
                m = __builtin_elementwise_maximum(__builtin_elementwise_maximum(m, x[e]), x[e + 1]);
        } else if (s == 1) {
#pragma unroll
            for (int e = H - 1; e + 1 < NE; e += 2)
                m = __builtin_elementwise_maximum(__builtin_elementwise_maximum(m, x[e]), x[e + 1]);
            m = __builtin_elementwise_maximum(m, x[NE - 1]);
            nan_mask |= __ballot(m != m);
            off = 1u << 20;  // no element equal (m is NaN)
        } else if (s >= 2 && s <= 5) {
            const int e1 = NE - 1 - (s - 2) * Q;
#pragma unroll
            for (int e = e1; e > e1 - Q; --e) off = (x[e] == m) ? (uint32_t)(32 * (e >> 3) + (e & 7)) : off;
        } else if (s == 6) {
            c = (m == m) ? (uint32_t)vlane + off : 0xFFFFFFFFu;
        } else {
            const uint64_t key = ((uint64_t)ordered_u32(m) << 32) | (uint64_t)(~c);
            atomicMax((unsigned long long*)best, (unsigned long long)key);
        }
    }
};

// One pipeline stage: start block b+1 (accumulators from its ring slot, refill of
// the slot, then its matrix-core instructions one k-chunk at a time) and finish
// block b's argmax, a slice after each k-chunk.
template <int KS, bool TAIL, bool VEC, bool SAMPLE, typename Refill>
__device__ __forceinline__ void stage(f32x4 (&nxt)[kMB], BaseFrag& slot, Refill&& refill, int t,
                                      const bf16x8 (&bt)[kMB][KS], const uint16_t* arow, const f32x4 (&cur)[kMB],
                                      uint64_t* best, int vlane, int V, uint64_t& nan_mask, const SampleArgs& smp,
                                      int pos, int r) {
    init_acc<TAIL, VEC>(nxt, slot, vlane, V);
    refill(slot, t);
    Argmax am(cur);
    if (SAMPLE) perturb(am.x, smp, vlane, pos, r);
    // key-row fragments are read one k-chunk ahead of their matrix-core use
    bf16x8 bfr = *(const bf16x8*)arow;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        bf16x8 nfr = bfr;
        if (ks + 1 < KS) nfr = *(const bf16x8*)(arow + (ks + 1) * 32);
#pragma unroll
        for (int mb = 0; mb < kMB; ++mb)
            nxt[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bt[mb][ks], bfr, nxt[mb], 0, 0, 0);
#pragma unroll
        for (int s = ks * 8 / KS; s < (ks + 1) * 8 / KS; ++s) am.slice(s, best, vlane, nan_mask);
        bfr = nfr;
    }
}

template <bool SAMPLE>
__device__ __forceinline__ void block_argmax(const f32x4 (&acc)[kMB], uint64_t* best, int vlane, uint64_t& nan_mask,
                                             const SampleArgs& smp, int pos, int r) {
    Argmax am(acc);
    if (SAMPLE) perturb(am.x, smp, vlane, pos, r);
#pragma unroll
    for (int s = 0; s < 8; ++s) am.slice(s, best, vlane, nan_mask);
}

// Fast form of score_generic (no logits output), software-pipelined: the
// matrix-core work of block b+1 is interleaved with the argmax of block b (two
// accumulator sets), so one wave keeps both the matrix cores and the vector ALUs
// busy.  Base blocks stream through the
// kPF-slot register ring; slot b % kPF is refilled, unconditionally, right after
// block b is taken from it, with the block kPF further on -- past this segment's
// last block that is the next segment's (npos, nc0) first blocks, so the ring is
// full when the next call starts.  XT: the next segment belongs to another
// vocabulary tile, whose wave slice starts at nvb.  The sweep covers fast_rows(RC)
// rows (whole ring cycles); blocks past RC score zero key rows into keys never
// published.  Returns the wave's NaN mask (nonzero: rescore exactly).
template <int KS, bool VEC, bool TAIL, bool SAMPLE, int PF, bool XT = false>
__device__ __forceinline__ uint64_t score_fast(ChainLds<KS>& L, const bf16x8 (&bt)[kMB][KS], BaseFrag (&pre)[PF],
                                               const uint16_t* __restrict__ base, int R, int K, int V, int pos,
                                               int c0, int RC, int l0, int vb, int npos, int nc0,
                                               const SampleArgs& smp, int nvb = 0) {
    constexpr int LROW = ChainLds<KS>::LROW;
    static_assert(PF % 2 == 0, "the two accumulator sets alternate within a ring cycle");
    const int lane = threadIdx.x & 63;
    const int n16 = lane & 15, g = lane >> 4;
    const int vlane = vb + 8 * g;
    const int nB = fast_rows<PF>(RC) >> 4;  // a multiple of PF
    const uint16_t* arow = L.a + (l0 + n16) * LROW + g * 8;
    uint64_t* best = L.best + l0 + n16;
    uint64_t nan_mask = 0ull;
    const BaseSrc src = base_src(base, R, K, V, n16, vlane);
    const int nvlane = XT ? nvb + 8 * g : vlane;
    const BaseSrc src_n = XT ? base_src(base, R, K, V, n16, nvlane) : src;
    const __amdgpu_buffer_rsrc_t rs_cur = seg_rsrc(src, c0, pos, K, V), rs_nxt = seg_rsrc(src, nc0, npos, K, V);
    // refill of the slot just emptied with ring block t (t >= PF)
    auto refill = [&](BaseFrag& f, int t) {
        const bool next = t >= nB;
        load_block<VEC>(f, next ? src_n : src, next ? rs_nxt : rs_cur, next ? t - nB : t, next ? nc0 : c0,
                        next ? npos : pos, R, K, V, n16, next ? nvlane : vlane);
    };
    f32x4 acc[2][kMB];
    init_acc<TAIL, VEC>(acc[0], pre[0], vlane, V);
    refill(pre[0], PF);
    mfma_block<KS>(acc[0], bt, arow);
    // Stage q of a ring cycle: block rb0+q sits in acc[q&1] with its products
    // issued; start block rb0+q+1 in the other set, then take block rb0+q's argmax.
    int rb0 = 0;
    for (; rb0 + PF < nB; rb0 += PF) {
#pragma unroll
        for (int q = 0; q < PF; ++q) {
            const int rb = rb0 + q;
            stage<KS, TAIL, VEC, SAMPLE>(acc[(q + 1) & 1], pre[(q + 1) % PF], refill, rb + 1 + PF, bt,
                                         arow + (rb + 1) * 16 * LROW, acc[q & 1], best + rb * 16, vlane, V, nan_mask,
                                         smp, pos, c0 + rb * 16 + n16);
        }
    }
    // last ring cycle: its final stage has no next block
#pragma unroll
    for (int q = 0; q + 1 < PF; ++q) {
        const int rb = rb0 + q;
        stage<KS, TAIL, VEC, SAMPLE>(acc[(q + 1) & 1], pre[(q + 1) % PF], refill, rb + 1 + PF, bt,
                                     arow + (rb + 1) * 16 * LROW, acc[q & 1], best + rb * 16, vlane, V, nan_mask, smp,
                                     pos, c0 + rb * 16 + n16);
    }
    block_argmax<SAMPLE>(acc[(PF - 1) & 1], best + (rb0 + PF - 1) * 16, vlane, nan_mask, smp, pos,
                         c0 + (rb0 + PF - 1) * 16 + n16);
    return nan_mask;
}

// Exact rescore of the wave's blocks, one at a time (base loaded per block): the
// ordered-key scan of every element, for waves whose fast pass met a NaN.
template <int KS, bool VEC, bool SAMPLE = false>
__device__ __forceinline__ void score_exact(ChainLds<KS>& L, const bf16x8 (&bt)[kMB][KS],
                                            const uint16_t* __restrict__ base, int R, int K, int V, int pos, int c0,
                                            int RC, int l0, int vb, const SampleArgs& smp = SampleArgs{}) {
    constexpr int LROW = ChainLds<KS>::LROW;
    const int lane = threadIdx.x & 63;
    const int n16 = lane & 15, g = lane >> 4;
    const int vlane = vb + 8 * g;
    const int nRB = (RC + 15) >> 4;
    for (int rb = 0; rb < nRB; ++rb) {
        BaseFrag f;
        load_base<VEC>(f, base, c0 + rb * 16 + n16, R, K, V, pos, vlane);
        f32x4 acc[kMB];
        init_acc<true, VEC>(acc, f, vlane, V);
        mfma_block<KS>(acc, bt, L.a + (l0 + rb * 16 + n16) * LROW + g * 8);
        float x[4 * kMB];
#pragma unroll
        for (int e = 0; e < 4 * kMB; ++e) x[e] = acc[2 * (e >> 3) + ((e & 7) >> 2)][e & 3];
        if (SAMPLE) perturb(x, smp, vlane, pos, c0 + rb * 16 + n16);
        uint32_t bu = 0u, bv = 0u;
#pragma unroll
        for (int e = 0; e < 4 * kMB; ++e) {
            const uint32_t v = (uint32_t)(vlane + 32 * (e >> 3) + (e & 7));
            const uint32_t u = ordered_u32(x[e]);
            if (v < (uint32_t)V && u > bu) {
                bu = u;
                bv = v;
            }
        }
        uint64_t key = bu ? (((uint64_t)bu << 32) | (uint64_t)(~bv)) : 0ull;
        key = umax64(key, shfl_xor_u64(key, 16));
        key = umax64(key, shfl_xor_u64(key, 32));
        if (g == 0) atomicMax((unsigned long long*)&L.best[l0 + rb * 16 + n16], (unsigned long long)key);
    }
}

// Score dispatch without logits output: the pipelined form; waves wholly past V
// have nothing to score; a NaN seen by the fast form triggers an exact rescore of
// the wave (its keys only ever raise the stored ones).
template <int KS, bool VEC, bool SAMPLE = false, int PF = kPF, bool XT = false>
__device__ __forceinline__ void score_rows(ChainLds<KS>& L, const bf16x8 (&bt)[kMB][KS], BaseFrag (&pre)[PF],
                                           const uint16_t* __restrict__ base, int R, int K, int V, int pos, int c0,
                                           int RC, int l0, int vb, int npos, int nc0,
                                           const SampleArgs& smp = SampleArgs{}, int nvb = 0) {
    if (vb >= V) return;
    const uint64_t nan_mask =
        (vb + kWV > V)
            ? score_fast<KS, VEC, true, SAMPLE, PF, XT>(L, bt, pre, base, R, K, V, pos, c0, RC, l0, vb, npos, nc0,
                                                        smp, nvb)
            : score_fast<KS, VEC, false, SAMPLE, PF, XT>(L, bt, pre, base, R, K, V, pos, c0, RC, l0, vb, npos, nc0,
                                                         smp, nvb);
    if (nan_mask != 0ull) score_exact<KS, VEC, SAMPLE>(L, bt, base, R, K, V, pos, c0, RC, l0, vb, smp);
}

// Best key over the waves, raised into the device-wide key of each request by an
// atomic max that returns the old value.  The returned values are folded into
// `token` and consumed only by grid_arrive (through its s_waitcnt), so the round
// trip of the atomics overlaps whatever the caller does in between.  Every
// workgroup raises every request's key: measured cheaper than reading the key first
// to skip atomics that cannot win.
// Threads [t0, kNT) take part (waves whose memory-counter waits should not include
// the atomics' round trip stay out).
template <int KS>
__device__ __forceinline__ void publish_rows(const ChainLds<KS>& L, uint64_t* keys, int R, int pos, int c0, int RC,
                                             int l0, uint64_t& token, int t0 = 0) {
    for (int j = phase_tid() - t0; j >= 0 && j < RC; j += kNT - t0) {
        const uint64_t b = L.best[l0 + j];
        if (b) token ^= __hip_atomic_fetch_max(&keys[(size_t)pos * R + c0 + j], b, __ATOMIC_RELAXED,
                                               __HIP_MEMORY_SCOPE_AGENT);
    }
}

// First PF base blocks of segment (pos, c0) into the ring (rows past R clamp).
template <bool VEC, int PF = kPF>
__device__ __forceinline__ void prefetch_rows(BaseFrag (&pre)[PF], const uint16_t* __restrict__ base, int R, int K,
                                              int V, int pos, int c0, int vb) {
    const int lane = threadIdx.x & 63;
    const int n16 = lane & 15, vlane = vb + 8 * (lane >> 4);
    const BaseSrc src = base_src(base, R, K, V, n16, vlane);
    const __amdgpu_buffer_rsrc_t rs = seg_rsrc(src, c0, pos, K, V);
#pragma unroll
    for (int q = 0; q < PF; ++q) load_block<VEC>(pre[q], src, rs, q, c0, pos, R, K, V, n16, vlane);
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

__device__ __forceinline__ void grid_arrive(uint32_t* ctr, uint64_t token = 0) {
    asm volatile("" ::"v"(token));  // the key atomics folded into token have returned
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (threadIdx.x == 0) __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// All K positions in one launch of a resident grid (R <= kReqChunk, gridDim.x <= resident
// workgroups).  Position pos waits for every workgroup to have published position
// pos-1; the base ring already holds position pos's first blocks by then.
// Split of the requests for the persistent schedule into groups of Hg requests (whole
// ring cycles of 64), at most kMaxGroups of them; a single group when R <= 64.
__device__ __forceinline__ int group_rows(int R) {
    if (R <= 64) return R;
    const int want = (R + 63) / 64 < kMaxGroups ? (R + 63) / 64 : kMaxGroups;
    return ((R + want - 1) / want + 63) / 64 * 64;
}

__device__ __forceinline__ int group_count(int R) {
    const int Hg = group_rows(R);
    return Hg > 0 ? (R + Hg - 1) / Hg : 1;
}

// All K positions of the chain in one launch.  G = the workgroups taking part
// (blockIdx.x < G).  `ready` (may be null): a flag that must read nonzero before the
// first keys are published (the single-launch step kernel zeroes the keys in-launch
// first).  tokens may be null.
//
// The request groups run out of phase (two by default): while a workgroup scores one
// group, the next group's keys of the previous position finish arriving from every
// workgroup, so its barrier wait is (nearly) free; its key rows are gathered
// asynchronously and its publish atomics overlap that gather.  Per position, two groups:
//   score h0 | wait h1(p-1), decode h1(p), gather h1 (async), publish h0(p), arrive h0
//   score h1 | wait h0(p),   decode h0(p+1), gather h0 (async), publish h1(p), arrive h1
// More groups give the barriers more slack but add a decode-gather-arrive chain per
// group and position; on the headline shape four groups measured slower than two.
// Barrier counters: bar[p * kMaxGroups + h].
template <int KS, bool VEC, bool SAMPLE = false, int PF = kPF>
__device__ __forceinline__ void chain_persist_body(ChainLds<KS>& L, const uint16_t* __restrict__ base,
                                                   const uint16_t* __restrict__ A, const uint16_t* __restrict__ Bt,
                                                   const int32_t* __restrict__ prev0, uint64_t* __restrict__ keys,
                                                   uint32_t* __restrict__ bar, int32_t* __restrict__ tokens,
                                                   uint32_t* __restrict__ status, int R, int K, int V, int rank,
                                                   int G, const uint32_t* ready, const SampleArgs& smp = SampleArgs{}) {
    static_assert(kMaxGroups >= 2, "at least two request groups");
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int vb = blockIdx.x * kTileV + w * kWV;
    bf16x8 bt[kMB][KS];
    load_bt<KS>(bt, Bt, V, rank, vb, lane & 15, lane >> 4);
    BaseFrag pre[PF];
    prefetch_rows<VEC, PF>(pre, base, R, K, V, 0, 0, vb);
    // Segments in order: (pos, group) for pos = 0..K-1 and each group.
    const int Hg = group_rows(R), ng = group_count(R);
    const int nseg = ng * K;
    const int RC0 = Hg < R ? Hg : R;
    decode_rows(L.prev, L.best, prev0, keys, tokens, status, R, K, V, 0, 0, RC0, 0, fast_rows<PF>(RC0));
    __syncthreads();
    gather_rows<KS>(L, A, V, rank, RC0, 0, fast_rows<PF>(RC0));
    __syncthreads();
    for (int sg = 0; sg < nseg; ++sg) {
        const int pos = sg / ng, h = sg - pos * ng;
        const int c0 = h * Hg, RC = (R - c0) < Hg ? (R - c0) : Hg;
        const int ns = sg + 1;  // the next segment
        const bool more = ns < nseg;
        const int npos = ns / ng, nh = ns - npos * ng;
        const int nc0 = nh * Hg, nRC = (R - nc0) < Hg ? (R - nc0) : Hg, nrows = fast_rows<PF>(nRC);
        score_rows<KS, VEC, SAMPLE, PF>(L, bt, pre, base, R, K, V, pos, c0, RC, c0, vb, more ? npos : pos,
                                    more ? nc0 : c0, smp);
        __syncthreads();
        if (ng > 1) {
            // The key atomics go out first, from the upper half of the waves; their
            // round trip overlaps the next segment's barrier poll, decode and gather
            // (the next segment's barrier is its group's previous position, passed by
            // every workgroup ng - 1 segments ago), which run in waves 0-1 (at most 128
            // requests per group), whose in-order memory-counter waits then exclude the
            // atomics.
            if (sg == 0 && ready != nullptr) grid_wait(ready, 1u, status);
            uint64_t token = 0;
            publish_rows<KS>(L, keys, R, pos, c0, RC, c0, token, kNT / 2);
            if (more) {
                if (npos > 0) grid_wait(&bar[(npos - 1) * kMaxGroups + nh], (uint32_t)G, status);
                decode_rows(L.prev, L.best, prev0, keys, tokens, status, R, K, V, npos, nc0, nRC, nc0, nrows);
                __syncthreads();
                gather_rows<KS, false>(L, A, V, rank, nRC, nc0, nrows);
            }
            grid_arrive(&bar[pos * kMaxGroups + h], token);  // its wait covers the key atomics and the gather
        } else {
            if (sg == 0 && ready != nullptr) grid_wait(ready, 1u, status);
            uint64_t token = 0;
            publish_rows<KS>(L, keys, R, pos, 0, RC0, 0, token);
            grid_arrive(&bar[pos * kMaxGroups], token);
            if (more) {
                grid_wait(&bar[pos * kMaxGroups], (uint32_t)G, status);
                decode_rows(L.prev, L.best, prev0, keys, tokens, status, R, K, V, npos, 0, RC0, 0, fast_rows<PF>(RC0));
                __syncthreads();
                gather_rows<KS>(L, A, V, rank, RC0, 0, fast_rows<PF>(RC0));
                __syncthreads();
            }
        }
    }
}

}  // namespace

}  // namespace dspark
