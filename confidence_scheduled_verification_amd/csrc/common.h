// Internal helpers shared by the gfx950 kernels of libdspark (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dspark {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr uint32_t kStatusPrevClamped = 1u;
constexpr uint32_t kStatusConfSanitized = 2u;
constexpr uint32_t kStatusCostInvalid = 4u;
constexpr uint32_t kStatusSyncTimeout = 8u;
constexpr uint32_t kStatusBadAllocation = 16u;

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

// Argmax key.  A 64-bit value whose unsigned order is the argmax order: larger
// logit first, NaN above every number, and among equal logits the lower index
// (the low word holds the bitwise complement of the index).  -0 is read as +0 so
// that equal numbers compare equal.  Every key built here is non-zero, so 0 is
// the identity of the max-reduction and never decodes to an index.
__device__ __forceinline__ uint64_t argmax_key(float x, uint32_t v) {
    uint32_t b = __float_as_uint(x);
    uint32_t u;
    if (x != x) {
        u = 0xFFFFFFFFu;
    } else {
        if (b == 0x80000000u) b = 0u;
        u = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
    }
    return ((uint64_t)u << 32) | (uint64_t)(~v);
}

__device__ __forceinline__ int32_t key_index(uint64_t key) { return (int32_t)(~(uint32_t)key); }

__device__ __forceinline__ uint64_t umax64(uint64_t a, uint64_t b) { return a > b ? a : b; }

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t x, int mask) {
    uint32_t lo = (uint32_t)x, hi = (uint32_t)(x >> 32);
    lo = __shfl_xor(lo, mask, 64);
    hi = __shfl_xor(hi, mask, 64);
    return ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ uint64_t load_agent_u64(const uint64_t* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Raise the device-wide best key at *p to at least k.  A relaxed read first skips the
// atomic when the stored key is already larger (keys only grow within a launch).  The
// atomic returns its old value, so a later s_waitcnt covers its completion.
__device__ __forceinline__ void publish_key(uint64_t* p, uint64_t k) {
    if (k > load_agent_u64(p)) {
        const uint64_t old = __hip_atomic_fetch_max(p, k, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        asm volatile("" ::"v"(old));
    }
}

// a ^ b ^ c in one instruction: gfx950's three-input bitwise operation with the truth
// table of a three-way exclusive or (0x96); c is wave-uniform.
__device__ __forceinline__ uint32_t xor3(uint32_t a, uint32_t b, uint32_t c) {
    uint32_t r;
    asm("v_bitop3_b32 %0, %1, %2, %3 bitop3:0x96" : "=v"(r) : "v"(a), "v"(b), "s"(__builtin_amdgcn_readfirstlane(c)));
    return r;
}

// Philox4x32-10 (Salmon, Moraes, Dror and Shaw, "Parallel random numbers: as easy as
// 1, 2, 3", SC 2011): ten rounds of the Philox S-box over the counter (c0, c1, c2, c3)
// under the key (k0, k1), the key advanced by the two Weyl constants between rounds.
// Each round's two 32x32 -> 64-bit products are one multiply-add each and its two
// three-way exclusive ors one instruction each.
__device__ __forceinline__ void philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3, uint32_t k0,
                                              uint32_t k1, uint32_t (&out)[4]) {
#pragma unroll
    for (int round = 0; round < 10; ++round) {
        const uint64_t p0 = (uint64_t)0xD2511F53u * c0;
        const uint64_t p1 = (uint64_t)0xCD9E8D57u * c2;
        const uint32_t n0 = xor3((uint32_t)(p1 >> 32), c1, k0);
        const uint32_t n2 = xor3((uint32_t)(p0 >> 32), c3, k1);
        c1 = (uint32_t)p1;
        c3 = (uint32_t)p0;
        c0 = n0;
        c2 = n2;
        k0 += 0x9E3779B9u;
        k1 += 0xBB67AE85u;
    }
    out[0] = c0;
    out[1] = c1;
    out[2] = c2;
    out[3] = c3;
}

// The value a sampled entry is ranked by: x / T + g, g = -ln(-ln u) a standard Gumbel
// variate, u = (2b + 1) / 2^24 for the top 23 bits b of w (exact in float32, strictly
// inside (0, 1)) -- computed in base 2 as x * (log2(e) / T) - log2(-log2 u), which is
// log2(e) (x / T + g) + log2(ln 2): a positive affine image with the same argmax, at
// one fused multiply-add and two hardware base-2 logarithms.  scale = log2(e) / T.
__device__ __forceinline__ float sampled_value(float x, float scale, uint32_t w) {
    const float u = (float)((w >> 8) | 1u) * 0x1p-24f;
    const float l = __builtin_amdgcn_logf(-__builtin_amdgcn_logf(u));
    return __builtin_fmaf(x, scale, -l);
}

__device__ __forceinline__ void raise_status(uint32_t* status, uint32_t bits) {
    if (status) atomicOr(status, bits);
}

}  // namespace dspark
