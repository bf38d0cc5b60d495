// Stages 2-5 of the chain-and-schedule pass (vLLM blog "Adaptive Verification
// in vLLM", sections "Scheduling the budget" and "The cost model"):
//   survival      s[r,i] = c[r,0] * ... * c[r,i]        (float32, increasing i)
//   global top-B  slots ranked by (s desc, request asc, position asc)
//   budget        B* = smallest argmax_B fl64(N + S_B) / fl64(vc[T+B] + dc[num_reqs])
//   allocation    per-request prefix lengths, offsets and the compacted slot list
//
// Everything after survival runs in ONE workgroup of 1024 threads out of LDS
// (n = R*K <= 16384 slots): the pages keep this work on the GPU with no host
// read-back, and at these sizes a single CU with 160 KB of LDS avoids every
// grid-wide synchronisation.
//   * Ranking is a stable LSD radix sort of 32-bit keys (0x3F800000 - bits(s):
//     non-negative floats order like their bit patterns) over slots laid out in
//     flat-id order, so equal survivals keep (request, position) order.  Each
//     8-bit pass ranks a wave's 64 items per round by wavefront ballots (match of
//     the digit bits), keeps per-wave digit counters in LDS, and scatters through
//     one block-wide scan of the 16 x 256 counters.
//   * S_B is summed EXACTLY: each float32 survival is an integer multiple of
//     2^-149, held as a 192-bit integer, scanned in any order with the same
//     result; N + S_B is rounded to double once (round to nearest even) and the
//     division is IEEE double.  B* therefore does not depend on the summation
//     order and is reproducible bit for bit.
#include <math.h>

#include "common.h"
#include "kernels.h"

namespace dspark {

namespace {

constexpr int kST = 1024;              // scheduler threads
constexpr int kSW = kST / 64;          // scheduler waves
constexpr int kMaxN = 16384;           // slots
constexpr uint32_t kOne = 0x3F800000u; // bits of 1.0f
constexpr uint32_t kPadKey = 0xFFFFFFFFu;

struct U192 {
    uint64_t a, b, c;  // little-endian limbs
};

__device__ __forceinline__ U192 add192(U192 x, U192 y) {
    U192 r;
    r.a = x.a + y.a;
    const uint64_t c0 = r.a < x.a;
    const uint64_t t = x.b + y.b;
    uint64_t c1 = t < x.b;
    r.b = t + c0;
    c1 |= (r.b < t);
    r.c = x.c + y.c + c1;
    return r;
}

// An IEEE float32 in [0,1] as an integer count of 2^-149 (exact).
__device__ __forceinline__ U192 fixed_from_bits(uint32_t bits) {
    const uint32_t E = bits >> 23, M = bits & 0x7FFFFFu;
    const uint64_t m = E ? (uint64_t)(M | 0x800000u) : (uint64_t)M;
    const int sh = E ? (int)E - 1 : 0;  // 0 .. 126
    U192 r = {0ull, 0ull, 0ull};
    if (sh < 64) {
        r.a = m << sh;
        r.b = sh ? (m >> (64 - sh)) : 0ull;
    } else if (sh < 128) {
        const int s2 = sh - 64;
        r.b = m << s2;
        r.c = s2 ? (m >> (64 - s2)) : 0ull;
    } else {
        r.c = m << (sh - 128);
    }
    return r;
}

__device__ __forceinline__ bool bit192(const U192& x, int i) {
    const uint64_t w = i < 64 ? x.a : (i < 128 ? x.b : x.c);
    return (w >> (i & 63)) & 1ull;
}

// Any bit strictly below position i (0 <= i <= 191)?
__device__ __forceinline__ bool any_below192(const U192& x, int i) {
    if (i <= 0) return false;
    if (i < 64) return (x.a & ((1ull << i) - 1ull)) != 0ull;
    if (x.a) return true;
    if (i == 64) return false;
    if (i < 128) return (x.b & ((1ull << (i - 64)) - 1ull)) != 0ull;
    if (x.b) return true;
    if (i == 128) return false;
    return (x.c & ((1ull << (i - 128)) - 1ull)) != 0ull;
}

// Low 64 bits of x >> s, 1 <= s <= 191.
__device__ __forceinline__ uint64_t shr192_lo(const U192& x, int s) {
    if (s < 64) return (x.a >> s) | (x.b << (64 - s));
    if (s == 64) return x.b;
    if (s < 128) return (x.b >> (s - 64)) | (x.c << (128 - s));
    if (s == 128) return x.c;
    return x.c >> (s - 128);
}

// x * 2^-149 rounded to the nearest double, ties to even.
__device__ __forceinline__ double fixed_to_double(const U192& x) {
    int p;
    if (x.c) p = 128 + 63 - __clzll(x.c);
    else if (x.b) p = 64 + 63 - __clzll(x.b);
    else if (x.a) p = 63 - __clzll(x.a);
    else return 0.0;
    if (p <= 52) return ldexp((double)x.a, -149);
    int sh = p - 52;
    uint64_t mant = shr192_lo(x, sh);
    const bool guard = bit192(x, sh - 1);
    const bool sticky = any_below192(x, sh - 1);
    if (guard && (sticky || (mant & 1ull))) {
        mant += 1ull;
        if (mant == (1ull << 53)) {
            mant >>= 1;
            sh += 1;
        }
    }
    return ldexp((double)mant, sh - 149);
}

__device__ __forceinline__ uint64_t shfl_up_u64(uint64_t x, int d) {
    uint32_t lo = (uint32_t)x, hi = (uint32_t)(x >> 32);
    lo = __shfl_up(lo, d, 64);
    hi = __shfl_up(hi, d, 64);
    return ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ U192 shfl_up_192(U192 x, int d) {
    return U192{shfl_up_u64(x.a, d), shfl_up_u64(x.b, d), shfl_up_u64(x.c, d)};
}

__device__ __forceinline__ double shfl_xor_f64(double x, int m) {
    return __longlong_as_double((long long)shfl_xor_u64((uint64_t)__double_as_longlong(x), m));
}

// Digit counters are stored digit-major with a stride of 17 words, so that both
// the per-wave ranking (one digit per lane) and the block scan (consecutive
// (digit, wave) entries per thread) touch distinct LDS banks.
constexpr int kHistStride = kSW + 1;
__device__ __forceinline__ int hist_at(int d, int w) { return d * kHistStride + w; }

struct SchedShared {
    uint32_t key[kMaxN];                 // sort keys; after sorting: keys in rank order
    uint16_t id[kMaxN];                  // flat slot ids travelling with the keys
    uint32_t hist[256 * kHistStride];    // per-(digit, wave) counters / offsets
    U192 part[kST];                      // per-thread partial sums; reused as the selection map
    uint32_t wsum[kSW];
    U192 wsum192[kSW];
    double wbest_f[kSW];
    int32_t wbest_b[kSW];
    int32_t b_star;
};

// Exclusive scan of one uint32 per thread over the 1024-thread block.
__device__ __forceinline__ uint32_t block_excl_scan(SchedShared& sh, uint32_t v, uint32_t* total) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    uint32_t x = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const uint32_t y = __shfl_up(x, o, 64);
        if (lane >= o) x += y;
    }
    if (lane == 63) sh.wsum[w] = x;
    __syncthreads();
    uint32_t off = 0, tot = 0;
    for (int q = 0; q < kSW; ++q) {
        const uint32_t s = sh.wsum[q];
        if (q < w) off += s;
        tot += s;
    }
    __syncthreads();
    if (total) *total = tot;
    return off + x - v;
}

// Exclusive scan of one 192-bit integer per thread.
__device__ __forceinline__ U192 block_excl_scan192(SchedShared& sh, U192 v) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    U192 x = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const U192 y = shfl_up_192(x, o);
        if (lane >= o) x = add192(x, y);
    }
    U192 excl = shfl_up_192(x, 1);
    if (lane == 0) excl = U192{0ull, 0ull, 0ull};
    if (lane == 63) sh.wsum192[w] = x;
    __syncthreads();
    if (w == 0) {  // exclusive scan of the 16 wave totals, in lanes 0..15 of wave 0
        U192 t = lane < kSW ? sh.wsum192[lane] : U192{0ull, 0ull, 0ull};
#pragma unroll
        for (int o = 1; o < kSW; o <<= 1) {
            const U192 y = shfl_up_192(t, o);
            if (lane >= o) t = add192(t, y);
        }
        U192 te = shfl_up_192(t, 1);
        if (lane == 0) te = U192{0ull, 0ull, 0ull};
        if (lane < kSW) sh.part[lane] = te;
    }
    __syncthreads();
    const U192 off = sh.part[w];
    __syncthreads();
    return add192(off, excl);
}

__device__ __forceinline__ int pad_slots(int n) {
    int p = ((n + kST - 1) / kST) * kST;
    return p < kST ? kST : p;
}

__device__ __forceinline__ float sanitize_conf(float c, bool& bad) {
    if (!(c >= 0.f)) {  // NaN or negative
        bad = true;
        return 0.f;
    }
    if (c > 1.f) {
        bad = true;
        return 1.f;
    }
    return c == 0.f ? 0.f : c;  // -0 -> +0
}

// Stage 2 for all requests; keys/ids in flat order, pads after n.  The confidences
// are first read coalesced into LDS (one memory round trip for the whole block),
// then each thread runs the sequential product of its request from LDS.
__device__ __forceinline__ void survival_to_lds(SchedShared& sh, const float* __restrict__ conf, int R, int K, int n_pad,
                                                float* __restrict__ surv_out, uint32_t* status) {
    const int n = R * K;
    for (int f = threadIdx.x; f < n_pad; f += kST) {
        sh.key[f] = f < n ? __float_as_uint(conf[f]) : kPadKey;
        sh.id[f] = (uint16_t)f;
    }
    __syncthreads();
    bool bad = false;
    for (int r = threadIdx.x; r < R; r += kST) {
        float s = 0.f;
        for (int i = 0; i < K; ++i) {
            const int f = r * K + i;
            const float c = sanitize_conf(__uint_as_float(sh.key[f]), bad);
            s = (i == 0) ? c : s * c;
            sh.key[f] = kOne - __float_as_uint(s);
            if (surv_out) surv_out[f] = s;
        }
    }
    if (bad) raise_status(status, kStatusConfSanitized);
    __syncthreads();
}

// Survivals given in global memory (topb-only entry point); values outside [0,1] are clamped.
__device__ __forceinline__ void surv_global_to_lds(SchedShared& sh, const float* __restrict__ surv, int n, int n_pad) {
    for (int f = threadIdx.x; f < n_pad; f += kST) {
        if (f < n) {
            bool bad = false;
            const float s = sanitize_conf(surv[f], bad);
            sh.key[f] = kOne - __float_as_uint(s);
        } else {
            sh.key[f] = kPadKey;
        }
        sh.id[f] = (uint16_t)f;
    }
    __syncthreads();
}

// One stable counting pass over the 8-bit digit at `shift`.  Wave w owns items
// [w*S, (w+1)*S) of the current order, 64 per round; an item's rank among equal
// digits of its wave comes from a ballot match of the digit bits and a running
// per-(digit, wave) counter.
__device__ __forceinline__ void radix_pass(SchedShared& sh, int n_pad, int shift) {
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int S = n_pad / kSW;  // items per wave, a multiple of 64
    const int J = S / 64;       // rounds, <= 16
    uint32_t k[16];
    uint32_t il[16];  // flat id (low 16 bits) and rank among equal digits of the wave (high 16 bits)
    for (int d = lane; d < 256; d += 64) sh.hist[hist_at(d, w)] = 0u;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        if (j < J) {
            const int p = w * S + j * 64 + lane;
            k[j] = sh.key[p];
            il[j] = sh.id[p];
        }
    }
    __syncthreads();
    const uint64_t lt = (1ull << lane) - 1ull;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        if (j < J) {
            const uint32_t d = (k[j] >> shift) & 0xFFu;
            uint64_t peers = ~0ull;
#pragma unroll
            for (int b = 0; b < 8; ++b) {
                const bool on = (d >> b) & 1u;
                const uint64_t m = __ballot(on);
                peers &= on ? m : ~m;
            }
            const uint32_t before = (uint32_t)__popcll(peers & lt);
            const uint32_t h = sh.hist[hist_at(d, w)];
            il[j] |= (h + before) << 16;
            if (before == 0u) sh.hist[hist_at(d, w)] = h + (uint32_t)__popcll(peers);
        }
    }
    __syncthreads();
    // Offsets in (digit, wave) order: entries e = 4*tid .. 4*tid+3, digit e/16, wave e%16.
    uint32_t c[4], s = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int e = 4 * tid + q;
        c[q] = sh.hist[hist_at(e >> 4, e & 15)];
        s += c[q];
    }
    uint32_t ex = block_excl_scan(sh, s, nullptr);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int e = 4 * tid + q;
        sh.hist[hist_at(e >> 4, e & 15)] = ex;
        ex += c[q];
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        if (j < J) {
            const uint32_t d = (k[j] >> shift) & 0xFFu;
            const uint32_t dest = sh.hist[hist_at(d, w)] + (il[j] >> 16);
            sh.key[dest] = k[j];
            sh.id[dest] = (uint16_t)(il[j] & 0xFFFFu);
        }
    }
    __syncthreads();
}

__device__ __forceinline__ void sort_slots(SchedShared& sh, int n_pad) {
#pragma unroll 1
    for (int shift = 0; shift < 32; shift += 8) radix_pass(sh, n_pad, shift);
}

__device__ __forceinline__ void write_ranking(const SchedShared& sh, int n, int32_t* __restrict__ order,
                              float* __restrict__ sorted_surv, int32_t* __restrict__ rank) {
    for (int j = threadIdx.x; j < n; j += kST) {
        const int f = sh.id[j];
        if (order) order[j] = f;
        if (sorted_surv) sorted_surv[j] = __uint_as_float(kOne - sh.key[j]);
        if (rank) rank[f] = j;
    }
}

// The cost-table entries one thread evaluates in stage 4 (B = tid*C + q, and B = n_pad
// for the last thread), read at the start of the kernel so that their memory latency
// overlaps the earlier stages.
struct CostPrefetch {
    float vc[16];
    float vc_last;
    float dc;
};

__device__ __forceinline__ void prefetch_costs(CostPrefetch& cp, const float* __restrict__ vc,
                                               const float* __restrict__ dc, int T, int num_reqs, int bmax,
                                               int n_pad) {
    const int C = n_pad / kST;
    const int j0 = threadIdx.x * C;
#pragma unroll
    for (int q = 0; q < 16; ++q) cp.vc[q] = (q < C && j0 + q <= bmax) ? vc[T + j0 + q] : 0.f;
    cp.vc_last = (threadIdx.x == kST - 1 && bmax == n_pad) ? vc[T + n_pad] : 0.f;
    cp.dc = dc[num_reqs];
}

// Stage 4 over the keys in sh.key (rank order).  Leaves B* in sh.b_star.
__device__ __forceinline__ void choose_budget_lds(SchedShared& sh, const CostPrefetch& cp, int n, int n_pad,
                                                  int n_sampling, int bmax, int32_t* __restrict__ b_star,
                                                  double* __restrict__ best_obj, double* __restrict__ obj,
                                                  uint32_t* status) {
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int C = n_pad / kST;
    const int j0 = tid * C;
    U192 local = {0ull, 0ull, 0ull};
    for (int q = 0; q < C; ++q) {
        const int j = j0 + q;
        if (j < n) local = add192(local, fixed_from_bits(kOne - sh.key[j]));
    }
    U192 S = block_excl_scan192(sh, local);
    const double dcost = (double)cp.dc;
    const uint64_t ns_hi = (uint64_t)(uint32_t)n_sampling << 21;  // n_sampling * 2^149: bit 149 is bit 21 of limb 2
    double bf = -INFINITY;
    int bb = 0x7FFFFFFF;
    bool bad = false;
    auto eval = [&](int B, float vcost) {
        U192 X = S;
        X.c += ns_hi;
        const double num = fixed_to_double(X);
        const double den = (double)vcost + dcost;
        double f;
        if (den > 0.0 && den <= 1.7976931348623157e308) {
            f = num / den;
        } else {
            f = -INFINITY;
            bad = true;
        }
        if (obj) obj[B] = f;
        if (f > bf || (f == bf && B < bb)) {
            bf = f;
            bb = B;
        }
    };
#pragma unroll
    for (int q = 0; q < 16; ++q) {
        if (q < C) {
            const int B = j0 + q;
            if (B <= bmax) eval(B, cp.vc[q]);
            if (B < n) S = add192(S, fixed_from_bits(kOne - sh.key[B]));
        }
    }
    if (tid == kST - 1 && bmax == n_pad) eval(n_pad, cp.vc_last);
    if (bad) raise_status(status, kStatusCostInvalid);
    // Block argmax: larger f, then smaller B.
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) {
        const double of = shfl_xor_f64(bf, m);
        const int ob = __shfl_xor(bb, m, 64);
        if (of > bf || (of == bf && ob < bb)) {
            bf = of;
            bb = ob;
        }
    }
    if (lane == 0) {
        sh.wbest_f[w] = bf;
        sh.wbest_b[w] = bb;
    }
    __syncthreads();
    if (tid == 0) {
        double f = sh.wbest_f[0];
        int b = sh.wbest_b[0];
        for (int q = 1; q < kSW; ++q) {
            if (sh.wbest_f[q] > f || (sh.wbest_f[q] == f && sh.wbest_b[q] < b)) {
                f = sh.wbest_f[q];
                b = sh.wbest_b[q];
            }
        }
        sh.b_star = b;
        if (b_star) *b_star = b;
        if (best_obj) *best_obj = f;
    }
    __syncthreads();
}

// Stage 5.  sel must already mark the chosen slots (1 byte per flat id, n entries).
__device__ __forceinline__ void allocate_lds(SchedShared& sh, const uint8_t* sel, int R, int K, int B,
                             const int32_t* __restrict__ tokens, int32_t* __restrict__ prefix_len,
                             int32_t* __restrict__ offsets, int32_t* __restrict__ ver_idx,
                             int32_t* __restrict__ ver_tokens) {
    const int tid = threadIdx.x;
    const int n = R * K;
    const int CR = (R + kST - 1) / kST;
    const int r0 = tid * CR;
    uint32_t cnt = 0;
    for (int q = 0; q < CR; ++q) {
        const int r = r0 + q;
        if (r < R)
            for (int i = 0; i < K; ++i) cnt += sel[r * K + i];
    }
    uint32_t total = 0;
    uint32_t o = block_excl_scan(sh, cnt, &total);
    for (int q = 0; q < CR; ++q) {
        const int r = r0 + q;
        if (r >= R) break;
        uint32_t L = 0;
        offsets[r] = (int32_t)o;
        for (int i = 0; i < K; ++i) {
            const int f = r * K + i;
            if (sel[f]) {
                ver_idx[o + L] = f;
                if (ver_tokens) ver_tokens[o + L] = tokens[f];
                ++L;
            }
        }
        prefix_len[r] = (int32_t)L;
        o += L;
    }
    if (tid == 0) offsets[R] = (int32_t)total;
    for (int j = B + tid; j < n; j += kST) {
        ver_idx[j] = -1;
        if (ver_tokens) ver_tokens[j] = -1;
    }
}

__device__ __forceinline__ uint8_t* selection_map(SchedShared& sh) { return reinterpret_cast<uint8_t*>(&sh.part[0]); }

__global__ __launch_bounds__(kST, 1) void sched_fused_kernel(
    const float* __restrict__ conf, int R, int K, int n_sampling, int T, int num_reqs,
    const float* __restrict__ vc, const float* __restrict__ dc, int bmax, float* __restrict__ surv_out,
    int32_t* __restrict__ order, float* __restrict__ sorted_surv, int32_t* __restrict__ b_star,
    double* __restrict__ best_obj, int32_t* __restrict__ prefix_len, int32_t* __restrict__ offsets,
    int32_t* __restrict__ ver_idx, uint32_t* status, uint64_t* __restrict__ ws, int ws_words) {
    __shared__ SchedShared sh;
    const int n = R * K, n_pad = pad_slots(n);
    // The chain's workspace (argmax keys, barrier counters) starts from zero; this launch
    // precedes the chain kernels on the stream.
    for (int j = threadIdx.x; j < ws_words; j += kST) ws[j] = 0ull;
    survival_to_lds(sh, conf, R, K, n_pad, surv_out, status);
    sort_slots(sh, n_pad);
    CostPrefetch cp;  // requested here so the loads overlap the write-out and the exact scan
    prefetch_costs(cp, vc, dc, T, num_reqs, bmax, n_pad);
    write_ranking(sh, n, order, sorted_surv, nullptr);
    choose_budget_lds(sh, cp, n, n_pad, n_sampling, bmax, b_star, best_obj, nullptr, status);
    const int B = sh.b_star;
    uint8_t* sel = selection_map(sh);
    for (int j = threadIdx.x; j < n; j += kST) sel[sh.id[j]] = (uint8_t)(j < B);
    __syncthreads();
    allocate_lds(sh, sel, R, K, B, nullptr, prefix_len, offsets, ver_idx, nullptr);
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
    __shared__ SchedShared sh;
    const int n = R * K, n_pad = pad_slots(n);
    surv_global_to_lds(sh, surv, n, n_pad);
    sort_slots(sh, n_pad);
    write_ranking(sh, n, order, sorted_surv, rank);
}

__global__ __launch_bounds__(kST, 1) void budget_kernel(const float* __restrict__ sorted_surv, int n, int n_sampling,
                                                       int T, int num_reqs, const float* __restrict__ vc,
                                                       const float* __restrict__ dc, int bmax,
                                                       int32_t* __restrict__ b_star, double* __restrict__ best_obj,
                                                       double* __restrict__ obj, uint32_t* status) {
    __shared__ SchedShared sh;
    const int n_pad = pad_slots(n);
    CostPrefetch cp;
    prefetch_costs(cp, vc, dc, T, num_reqs, bmax, n_pad);
    for (int j = threadIdx.x; j < n_pad; j += kST) {
        uint32_t key = kOne;  // value 0 for pads (never summed: j >= n)
        if (j < n) {
            bool bad = false;
            key = kOne - __float_as_uint(sanitize_conf(sorted_surv[j], bad));
        }
        sh.key[j] = key;
    }
    __syncthreads();
    choose_budget_lds(sh, cp, n, n_pad, n_sampling, bmax, b_star, best_obj, obj, status);
}

__global__ __launch_bounds__(kST, 1) void allocate_kernel(const int32_t* __restrict__ order,
                                                         const int32_t* __restrict__ b_star, int R, int K,
                                                         const int32_t* __restrict__ tokens,
                                                         int32_t* __restrict__ prefix_len,
                                                         int32_t* __restrict__ offsets, int32_t* __restrict__ ver_idx,
                                                         int32_t* __restrict__ ver_tokens) {
    __shared__ SchedShared sh;
    const int n = R * K;
    int B = *b_star;
    B = B < 0 ? 0 : (B > n ? n : B);
    uint8_t* sel = selection_map(sh);
    for (int f = threadIdx.x; f < n; f += kST) sel[f] = 0;
    __syncthreads();
    for (int j = threadIdx.x; j < B; j += kST) {
        const int f = order[j];
        if (f >= 0 && f < n) sel[f] = 1;
    }
    __syncthreads();
    allocate_lds(sh, sel, R, K, B, tokens, prefix_len, offsets, ver_idx, ver_tokens);
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
                       a.vc, a.dc, a.bmax, a.b_star, a.best_obj, a.obj, a.status);
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
                       a.num_reqs, a.vc, a.dc, a.bmax, a.surv, a.order, a.sorted_surv, a.b_star, a.best_obj,
                       a.prefix_len, a.offsets, a.ver_idx, a.status, a.ws, a.ws_words);
    return hipGetLastError();
}

}  // namespace dspark
