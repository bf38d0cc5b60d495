// Device code of stages 2-5 of the chain-and-schedule pass (vLLM blog "Adaptive
// Verification in vLLM", sections "Scheduling the budget" and "The cost model"),
// for one workgroup of NT threads working out of LDS:
//   survival      s[r,i] = c[r,0] * ... * c[r,i]        (float32, increasing i)
//   global top-B  slots ranked by (s desc, request asc, position asc)
//   budget        B* = smallest argmax_B fl64(N + S_B) / fl64(vc[T+B] + dc[num_reqs]), or
//                 the first-drop rule: admit slots in rank order while that ratio
//                 strictly rises (DSpark summary "How DSpark Speeds Up LLM
//                 Inference", section "Verify smarter")
//   allocation    per-request prefix lengths, offsets and the compacted slot list
//
//   * Ranking is a stable LSD radix sort of 32-bit keys (0x3F800000 - bits(s):
//     non-negative floats order like their bit patterns) over slots laid out in
//     flat-id order, so equal survivals keep (request, position) order.  Each
//     8-bit pass ranks a wave's 64 items per round by wavefront ballots (match of
//     the digit bits), keeps per-wave digit counters in LDS, and scatters through
//     one block-wide scan of the 256 x waves counters.
//   * S_B is summed EXACTLY: each float32 survival is an integer multiple of
//     2^-149, held as a 192-bit integer, scanned in any order with the same
//     result; N + S_B is rounded to double once (round to nearest even) and the
//     division is IEEE double.  B* therefore does not depend on the summation
//     order or the thread count and is reproducible bit for bit.
#pragma once

#include <math.h>

#include "common.h"

namespace dspark {

namespace {

constexpr int kMaxN = 16384;           // slots
constexpr uint32_t kOne = 0x3F800000u; // bits of 1.0f
constexpr uint32_t kPadKey = 0xFFFFFFFFu;
constexpr int kRuleArgmax = 0;
constexpr int kRuleFirstDrop = 1;

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

// Digit counters are stored digit-major with a stride of (waves + 1) words, so that
// both the per-wave ranking (one digit per lane) and the block scan (consecutive
// (digit, wave) entries per thread) touch distinct LDS banks.
template <int NT>
__device__ __forceinline__ int hist_at(int d, int w) { return d * (NT / 64 + 1) + w; }

// LDS of the scheduling workgroup (NT threads).
template <int NT>
struct SchedShared {
    static constexpr int SW = NT / 64;
    uint32_t key[kMaxN];                 // sort keys; after sorting: keys in rank order
    uint16_t id[kMaxN];                  // flat slot ids travelling with the keys
    uint32_t hist[256 * (SW + 1)];       // per-(digit, wave) counters / offsets
    // per-thread partial sums; reused as the selection map (one byte per slot)
    static constexpr int kPart = NT > (kMaxN + 23) / 24 ? NT : (kMaxN + 23) / 24;
    U192 part[kPart];
    uint32_t wsum[SW];
    U192 wsum192[SW];
    double wbest_f[SW];
    double wbest_v[SW];
    int32_t wbest_b[SW];
    int32_t b_star;
};

// Exclusive scan of one uint32 per thread over the block.  TRAIL: end with a barrier so
// that the next call may reuse sh.wsum at once (callers with barriers of their own in
// between pass false).
template <int NT, bool TRAIL = true>
__device__ __forceinline__ uint32_t block_excl_scan(SchedShared<NT>& sh, uint32_t v, uint32_t* total) {
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
    for (int q = 0; q < NT / 64; ++q) {
        const uint32_t s = sh.wsum[q];
        if (q < w) off += s;
        tot += s;
    }
    if (TRAIL) __syncthreads();
    if (total) *total = tot;
    return off + x - v;
}

// Exclusive scan of one 192-bit integer per thread.
template <int NT>
__device__ __forceinline__ U192 block_excl_scan192(SchedShared<NT>& sh, U192 v) {
    constexpr int kSW = NT / 64;
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
    if (w == 0) {  // exclusive scan of the wave totals, in the first lanes of wave 0
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

template <int NT>
__device__ __forceinline__ int pad_slots(int n) {
    int p = ((n + NT - 1) / NT) * NT;
    return p < NT ? NT : p;
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
template <int NT>
__device__ __forceinline__ void survival_to_lds(SchedShared<NT>& sh, const float* __restrict__ conf, int R, int K, int n_pad,
                                                float* __restrict__ surv_out, uint32_t* status) {
    const int n = R * K;
    for (int f = threadIdx.x; f < n_pad; f += NT) {
        sh.key[f] = f < n ? __float_as_uint(conf[f]) : kPadKey;
        sh.id[f] = (uint16_t)f;
    }
    __syncthreads();
    bool bad = false;
    for (int r = threadIdx.x; r < R; r += NT) {
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
template <int NT>
__device__ __forceinline__ void surv_global_to_lds(SchedShared<NT>& sh, const float* __restrict__ surv, int n, int n_pad) {
    for (int f = threadIdx.x; f < n_pad; f += NT) {
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
// per-(digit, wave) counter.  Entered after a barrier that follows the last writes of
// the keys (the previous pass's scatter, or the survival stage).  A wave's counter
// column is written and read by that wave alone until the barrier before the offset
// scan, so clearing it needs no barrier of its own; the scan's scratch is not written
// again before this pass's later barriers, so it needs no trailing one either.
template <int NT>
__device__ __forceinline__ void radix_pass(SchedShared<NT>& sh, int n_pad, int shift) {
    constexpr int kSW = NT / 64, JM = kMaxN / NT;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int S = n_pad / kSW;  // items per wave, a multiple of 64
    const int J = S / 64;       // rounds, <= JM
    uint32_t k[JM];
    uint32_t il[JM];  // flat id (low 16 bits) and rank among equal digits of the wave (high 16 bits)
    for (int d = lane; d < 256; d += 64) sh.hist[hist_at<NT>(d, w)] = 0u;
#pragma unroll
    for (int j = 0; j < JM; ++j) {
        if (j < J) {
            const int p = w * S + j * 64 + lane;
            k[j] = sh.key[p];
            il[j] = sh.id[p];
        }
    }
    const uint64_t lt = (1ull << lane) - 1ull;
#pragma unroll
    for (int j = 0; j < JM; ++j) {
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
            const uint32_t h = sh.hist[hist_at<NT>(d, w)];
            il[j] |= (h + before) << 16;
            if (before == 0u) sh.hist[hist_at<NT>(d, w)] = h + (uint32_t)__popcll(peers);
        }
    }
    __syncthreads();
    // Offsets in (digit, wave) order: entries e = 4*tid .. 4*tid+3 (256 digits x kSW
    // waves = 4 per thread), digit e / kSW, wave e % kSW.
    uint32_t c[4], s = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int e = 4 * tid + q;
        c[q] = sh.hist[hist_at<NT>(e / kSW, e % kSW)];
        s += c[q];
    }
    uint32_t ex = block_excl_scan<NT, false>(sh, s, nullptr);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int e = 4 * tid + q;
        sh.hist[hist_at<NT>(e / kSW, e % kSW)] = ex;
        ex += c[q];
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < JM; ++j) {
        if (j < J) {
            const uint32_t d = (k[j] >> shift) & 0xFFu;
            const uint32_t dest = sh.hist[hist_at<NT>(d, w)] + (il[j] >> 16);
            sh.key[dest] = k[j];
            sh.id[dest] = (uint16_t)(il[j] & 0xFFFFu);
        }
    }
    __syncthreads();
}

template <int NT>
__device__ __forceinline__ void sort_slots(SchedShared<NT>& sh, int n_pad) {
#pragma unroll 1
    for (int shift = 0; shift < 32; shift += 8) radix_pass<NT>(sh, n_pad, shift);
}

template <int NT>
__device__ __forceinline__ void write_ranking(const SchedShared<NT>& sh, int n, int32_t* __restrict__ order,
                              float* __restrict__ sorted_surv, int32_t* __restrict__ rank) {
    for (int j = threadIdx.x; j < n; j += NT) {
        const int f = sh.id[j];
        if (order) order[j] = f;
        if (sorted_surv) sorted_surv[j] = __uint_as_float(kOne - sh.key[j]);
        if (rank) rank[f] = j;
    }
}

// The cost-table entries one thread evaluates in stage 4 (B = tid*C + q, and
// B = tid*C + C, the next thread's first candidate, which the first-drop rule compares
// against and which is n_pad for the last thread), read at the start of the kernel so
// that their memory latency overlaps the earlier stages.
template <int NT>
struct CostPrefetch {
    float vc[kMaxN / NT];
    float vc_next;
    float dc;
};

template <int NT>
__device__ __forceinline__ void prefetch_costs(CostPrefetch<NT>& cp, const float* __restrict__ vc,
                                               const float* __restrict__ dc, int T, int num_reqs, int bmax,
                                               int n_pad) {
    const int C = n_pad / NT;
    const int j0 = threadIdx.x * C;
#pragma unroll
    for (int q = 0; q < kMaxN / NT; ++q) cp.vc[q] = (q < C && j0 + q <= bmax) ? vc[T + j0 + q] : 0.f;
    cp.vc_next = (j0 + C <= bmax) ? vc[T + j0 + C] : 0.f;
    cp.dc = dc[num_reqs];
}

// Stage 4 over the keys in sh.key (rank order).  Leaves the budget in sh.b_star.
// rule kRuleArgmax: the smallest B with the largest f.  rule kRuleFirstDrop: the first
// B whose successor does not raise f (f(B+1) <= f(B)), else bmax.  Every f(B) is the
// same double in both rules, so where f rises to a single peak they agree.
template <int NT>
__device__ __forceinline__ void choose_budget_lds(SchedShared<NT>& sh, const CostPrefetch<NT>& cp, int n, int n_pad,
                                                  int n_sampling, int bmax, int rule, int32_t* __restrict__ b_star,
                                                  double* __restrict__ best_obj, double* __restrict__ obj,
                                                  uint32_t* status) {
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    constexpr int kSW = NT / 64;
    const int C = n_pad / NT;
    const int j0 = tid * C;
    U192 local = {0ull, 0ull, 0ull};
    for (int q = 0; q < C; ++q) {
        const int j = j0 + q;
        if (j < n) local = add192(local, fixed_from_bits(kOne - sh.key[j]));
    }
    U192 S = block_excl_scan192<NT>(sh, local);
    const double dcost = (double)cp.dc;
    const uint64_t ns_hi = (uint64_t)(uint32_t)n_sampling << 21;  // n_sampling * 2^149: bit 149 is bit 21 of limb 2
    bool bad = false;
    auto eval = [&](float vcost) -> double {
        U192 X = S;
        X.c += ns_hi;
        const double num = fixed_to_double(X);
        const double den = (double)vcost + dcost;
        if (den > 0.0 && den <= 1.7976931348623157e308) return num / den;
        bad = true;
        return -INFINITY;
    };
    double bf = -INFINITY;   // argmax candidate of this thread: f and B
    int bb = 0x7FFFFFFF;
    double fprev = 0.0;      // f(B-1) of the previous candidate of this thread
    int drop = 0x7FFFFFFF;   // first-drop candidate: B with f(B+1) <= f(B), and f(B)
    double fdrop = 0.0;
    auto take = [&](int B, double f, bool own) {
        if (own) {
            if (obj) obj[B] = f;
            if (f > bf || (f == bf && B < bb)) {
                bf = f;
                bb = B;
            }
            if (B == bmax && drop == 0x7FFFFFFF) {  // no drop before bmax: admission ends there
                drop = B;
                fdrop = f;
            }
        }
        if (B > j0 && !(f > fprev) && drop > B - 1) {
            drop = B - 1;
            fdrop = fprev;
        }
        fprev = f;
    };
#pragma unroll
    for (int q = 0; q < kMaxN / NT; ++q) {
        if (q < C) {
            const int B = j0 + q;
            if (B <= bmax) take(B, eval(cp.vc[q]), true);
            if (B < n) S = add192(S, fixed_from_bits(kOne - sh.key[B]));
        }
    }
    // B = j0 + C: the next thread's first candidate (compared against f(j0 + C - 1)), or
    // B = n_pad for the last thread.
    if (j0 + C <= bmax) take(j0 + C, eval(cp.vc_next), tid == NT - 1);
    if (bad) raise_status(status, kStatusCostInvalid);
    // Block reduction: argmax takes the larger f, then the smaller B; first drop takes
    // the smaller B.  (kf, kb) is the key, vf the objective carried along.
    double kf = bf, vf = bf;
    int kb = bb;
    if (rule == kRuleFirstDrop) {
        kf = drop == 0x7FFFFFFF ? -INFINITY : 0.0;
        kb = drop;
        vf = fdrop;
    }
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) {
        const double of = shfl_xor_f64(kf, m);
        const double ov = shfl_xor_f64(vf, m);
        const int ob = __shfl_xor(kb, m, 64);
        if (of > kf || (of == kf && ob < kb)) {
            kf = of;
            kb = ob;
            vf = ov;
        }
    }
    if (lane == 0) {
        sh.wbest_f[w] = kf;
        sh.wbest_v[w] = vf;
        sh.wbest_b[w] = kb;
    }
    __syncthreads();
    if (tid == 0) {
        double f = sh.wbest_f[0], v = sh.wbest_v[0];
        int b = sh.wbest_b[0];
        for (int q = 1; q < kSW; ++q) {
            if (sh.wbest_f[q] > f || (sh.wbest_f[q] == f && sh.wbest_b[q] < b)) {
                f = sh.wbest_f[q];
                v = sh.wbest_v[q];
                b = sh.wbest_b[q];
            }
        }
        sh.b_star = b;
        if (b_star) *b_star = b;
        if (best_obj) *best_obj = v;
    }
    __syncthreads();
}

// Stage 5.  sel must already mark the chosen slots (1 byte per flat id, n entries).
// lds_rows (may be null): per request r, lds_rows[2r] = its offset into ver_idx and
// lds_rows[2r + 1] = its prefix length.
template <int NT>
__device__ __forceinline__ void allocate_lds(SchedShared<NT>& sh, const uint8_t* sel, int R, int K, int B,
                             const int32_t* __restrict__ tokens, int32_t* __restrict__ prefix_len,
                             int32_t* __restrict__ offsets, int32_t* __restrict__ ver_idx,
                             int32_t* __restrict__ ver_tokens, int32_t* lds_rows = nullptr) {
    const int tid = threadIdx.x;
    const int n = R * K;
    const int CR = (R + NT - 1) / NT;
    const int r0 = tid * CR;
    uint32_t cnt = 0;
    for (int q = 0; q < CR; ++q) {
        const int r = r0 + q;
        if (r < R)
            for (int i = 0; i < K; ++i) cnt += sel[r * K + i];
    }
    uint32_t total = 0;
    uint32_t o = block_excl_scan<NT>(sh, cnt, &total);
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
        if (lds_rows) {
            lds_rows[2 * r] = (int32_t)o;
            lds_rows[2 * r + 1] = (int32_t)L;
        }
        prefix_len[r] = (int32_t)L;
        o += L;
    }
    if (tid == 0) offsets[R] = (int32_t)total;
    for (int j = B + tid; j < n; j += NT) {
        ver_idx[j] = -1;
        if (ver_tokens) ver_tokens[j] = -1;
    }
}

template <int NT>
__device__ __forceinline__ uint8_t* selection_map(SchedShared<NT>& sh) {
    static_assert(sizeof(sh.part) >= kMaxN, "the selection map needs one byte per slot");
    return reinterpret_cast<uint8_t*>(&sh.part[0]);
}


// Where the budget is sized from: the current confidences (separate == 0), or another
// array [R][K] such as the one of one or two steps earlier (vLLM blog, "Scheduling the
// budget": B is sized from a one-step-old confidence buffer while the slots are handed
// out with current values).  bmax is the largest B of that sizing, rule the admission
// rule.
struct Sizing {
    int separate;
    const float* conf;
    int R;
    int bmax;
    int rule;
};

// Stages 2-5 in sequence: survival (optionally written out), ranking (written out),
// budget, selection and allocation.  Leaves B* in sh.b_star and the selection map in
// LDS; every output pointer except the required ones may be null.  lds_rows (may be
// null, may alias sh.key, which is free by then): each request's offset and prefix
// length (see allocate_lds).  tokens and ver_tokens (may be null): the draft tokens and
// the verified-token output of allocate_lds.
// With a separate sizing array, B is chosen from its survivals first (same survival,
// ranking and budget code over its slots), capped at R*K, and best_obj is the sizing
// objective.
template <int NT>
__device__ __forceinline__ void sched_pass(SchedShared<NT>& sh, const float* __restrict__ conf, int R, int K,
                                           int n_sampling, int T, int num_reqs, const float* __restrict__ vc,
                                           const float* __restrict__ dc, int bmax, const Sizing& sz,
                                           float* __restrict__ surv_out, int32_t* __restrict__ order,
                                           float* __restrict__ sorted_surv, int32_t* __restrict__ b_star,
                                           double* __restrict__ best_obj, int32_t* __restrict__ prefix_len,
                                           int32_t* __restrict__ offsets, int32_t* __restrict__ ver_idx,
                                           uint32_t* status, int32_t* lds_rows = nullptr,
                                           const int32_t* __restrict__ tokens = nullptr,
                                           int32_t* __restrict__ ver_tokens = nullptr) {
    const int n = R * K;
    // One or two passes of the same code (a loop, so that the stage code exists once in
    // the kernel): with a separate sizing array, pass 0 sizes B from it and pass 1 ranks
    // the current slots; otherwise one pass does both.
    const int passes = sz.separate ? 2 : 1;
    int B = 0;
#pragma unroll 1
    for (int ps = 0; ps < passes; ++ps) {
        const bool sizing = ps == 0, last = ps == passes - 1;
        const float* src = sz.separate && sizing ? sz.conf : conf;
        const int rows = sz.separate && sizing ? sz.R : R;
        const int m = rows * K, m_pad = pad_slots<NT>(m);
        const int bm = sz.separate ? sz.bmax : bmax;
        // The cost-table entries are requested before the ranking where the registers
        // allow (up to 512 threads), so their memory round trip overlaps the confidences'
        // and the sort; with more threads, after the sort (overlapping the write-out and
        // the exact scan).
        constexpr bool kEarly = NT <= 512;
        CostPrefetch<NT> cp;
        if (kEarly && sizing) prefetch_costs<NT>(cp, vc, dc, T, num_reqs, bm, m_pad);
        survival_to_lds<NT>(sh, src, rows, K, m_pad, last ? surv_out : nullptr, status);
        sort_slots<NT>(sh, m_pad);
        if (sizing) {
            if (!kEarly) prefetch_costs<NT>(cp, vc, dc, T, num_reqs, bm, m_pad);
            if (last) write_ranking<NT>(sh, n, order, sorted_surv, nullptr);
            choose_budget_lds<NT>(sh, cp, m, m_pad, n_sampling, bm, sz.rule, last ? b_star : nullptr, best_obj,
                                  nullptr, status);
            B = sh.b_star;  // every thread reads it before the next barrier
        } else {
            write_ranking<NT>(sh, n, order, sorted_surv, nullptr);
        }
    }
    if (sz.separate) {
        B = B < n ? B : n;
        if (threadIdx.x == 0) {
            sh.b_star = B;
            if (b_star) *b_star = B;
        }
    }
    uint8_t* sel = selection_map<NT>(sh);
    for (int j = threadIdx.x; j < n; j += NT) sel[sh.id[j]] = (uint8_t)(j < B);
    __syncthreads();
    allocate_lds<NT>(sh, sel, R, K, B, tokens, prefix_len, offsets, ver_idx, ver_tokens, lds_rows);
}

}  // namespace

}  // namespace dspark
