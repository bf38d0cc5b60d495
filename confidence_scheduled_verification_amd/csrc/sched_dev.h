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
//   * Ranking sorts one 64-bit word per slot, (0x3F800000 - bits(s)) << 16 | flat id:
//     non-negative floats order like their bit patterns, so ascending words are
//     (s descending, request ascending, position ascending) and every word is
//     distinct.  Up to two slots per thread the sort is a bottom-up merge over runs
//     that are adjacent in flat order: each level moves a slot to its own index in its
//     run plus the number of smaller words in the partner run (a binary search in
//     LDS), so a level is one parallel step with no counters or scans.  A request's
//     survivals never rise along its positions (each factor is at most 1 and rounding
//     is monotone), so the first runs are whole requests and R requests take
//     ceil(log2 R) levels.  Past that size the merge's n log n searches cost more than
//     a stable LSD radix sort of the key bits (four 8-bit passes, each ranking a
//     wave's 64 words per round by wavefront ballots of the digit bits, with per-wave
//     digit counters and one block scan), which takes over.
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
constexpr int kRuleArgmax = 0;
constexpr int kRuleFirstDrop = 1;

struct U192 {
    uint64_t a, b, c;  // little-endian limbs
};

__device__ __forceinline__ U192 add192(U192 x, U192 y) {
    unsigned long long c0, c1, c2;
    U192 r;
    r.a = __builtin_addcll(x.a, y.a, 0ull, &c0);
    r.b = __builtin_addcll(x.b, y.b, c0, &c1);
    r.c = __builtin_addcll(x.c, y.c, c1, &c2);
    return r;
}

__device__ __forceinline__ U192 sub192(U192 x, U192 y) {
    unsigned long long b0, b1, b2;
    U192 r;
    r.a = __builtin_subcll(x.a, y.a, 0ull, &b0);
    r.b = __builtin_subcll(x.b, y.b, b0, &b1);
    r.c = __builtin_subcll(x.c, y.c, b1, &b2);
    return r;
}

// An IEEE float32 in [0,1] as an integer count of 2^-149 (exact).
__device__ __forceinline__ U192 fixed_from_bits(uint32_t bits) {
    const uint32_t E = bits >> 23, M = bits & 0x7FFFFFu;
    const uint64_t m = E ? (uint64_t)(M | 0x800000u) : (uint64_t)M;
    const int sh = E ? (int)E - 1 : 0;  // 0 .. 126
    const int li = sh >> 6, off = sh & 63;  // limb and offset of m's lowest bit
    const uint64_t lo = m << off;
    const uint64_t hi = off ? m >> (64 - off) : 0ull;
    U192 r;
    r.a = li == 0 ? lo : 0ull;
    r.b = li == 0 ? hi : (li == 1 ? lo : 0ull);
    r.c = li == 1 ? hi : (li == 2 ? lo : 0ull);
    return r;
}

// x * 2^-149 rounded to the nearest double, ties to even: the 64 bits from x's leading
// one down, with every lower bit ORed into their last bit (that bit lies below the
// rounding position of a 53-bit significand, so it only breaks ties the way the exact
// value does), converted once.
__device__ __forceinline__ double fixed_to_double(const U192& x) {
    const bool c_nz = x.c != 0ull, b_nz = x.b != 0ull;
    const uint64_t h = c_nz ? x.c : (b_nz ? x.b : x.a);      // limb of the leading one
    const uint64_t m = c_nz ? x.b : (b_nz ? x.a : 0ull);     // the limb below it
    const bool low = c_nz && x.a != 0ull;                    // anything further below
    const int base = c_nz ? 128 : (b_nz ? 64 : 0);
    if (h == 0ull) return 0.0;
    const int z = __clzll(h);
    const uint64_t top = z ? (h << z) | (m >> (64 - z)) : h;
    const uint64_t rest = z ? (m << z) : m;
    const double d = (double)(top | (uint64_t)(rest != 0ull || low));
    return ldexp(d, base - z - 149);
}

// Wavefront data movement (DPP) for the scans and reductions below: lanes whose source
// lies outside the pattern (or rows outside row_mask) receive 0.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t x) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, CTRL, ROW_MASK, 0xF, false);
}

template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t x) {
    return ((uint64_t)dpp_u32<CTRL, ROW_MASK>((uint32_t)(x >> 32)) << 32) | dpp_u32<CTRL, ROW_MASK>((uint32_t)x);
}

template <int CTRL, int ROW_MASK>
__device__ __forceinline__ U192 dpp192(const U192& x) {
    return U192{dpp_u64<CTRL, ROW_MASK>(x.a), dpp_u64<CTRL, ROW_MASK>(x.b), dpp_u64<CTRL, ROW_MASK>(x.c)};
}

// Inclusive wavefront scans: shifts by 1, 2, 4, 8 within each row of 16 lanes, then lane
// 15 into row 1, lane 47 into row 3, and lane 31 into rows 2 and 3.
constexpr int kDppShr1 = 0x111, kDppShr2 = 0x112, kDppShr4 = 0x114, kDppShr8 = 0x118;
constexpr int kDppBcast15 = 0x142, kDppBcast31 = 0x143;
// Reductions: partner lanes at xor 1 and xor 2 within quads, then the mirrored lane of the
// half row and of the row.
constexpr int kDppXor1 = 0xB1, kDppXor2 = 0x4E, kDppHalfMirror = 0x141, kDppMirror = 0x140;

__device__ __forceinline__ uint32_t wave_incl_scan_u32(uint32_t x) {
    x += dpp_u32<kDppShr1, 0xF>(x);
    x += dpp_u32<kDppShr2, 0xF>(x);
    x += dpp_u32<kDppShr4, 0xF>(x);
    x += dpp_u32<kDppShr8, 0xF>(x);
    x += dpp_u32<kDppBcast15, 0xA>(x);
    x += dpp_u32<kDppBcast31, 0xC>(x);
    return x;
}

__device__ __forceinline__ U192 wave_incl_scan192(U192 x) {
    x = add192(x, dpp192<kDppShr1, 0xF>(x));
    x = add192(x, dpp192<kDppShr2, 0xF>(x));
    x = add192(x, dpp192<kDppShr4, 0xF>(x));
    x = add192(x, dpp192<kDppShr8, 0xF>(x));
    x = add192(x, dpp192<kDppBcast15, 0xA>(x));
    x = add192(x, dpp192<kDppBcast31, 0xC>(x));
    return x;
}

template <int CTRL>
__device__ __forceinline__ double dpp_max_step_f64(double v) {
    const double w = __longlong_as_double((long long)dpp_u64<CTRL, 0xF>((uint64_t)__double_as_longlong(v)));
    return w > v ? w : v;
}

__device__ __forceinline__ double readlane_f64(double v, int l) {
    const uint64_t u = (uint64_t)__double_as_longlong(v);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)u, l);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(u >> 32), l);
    return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}

// Wavefront maximum of a double (no NaN) and minimum of an int, the same in every lane.
// The patterns have no lane outside them, so the 0 fill never enters.
__device__ __forceinline__ double wave_max_f64(double x) {
    x = dpp_max_step_f64<kDppXor1>(x);
    x = dpp_max_step_f64<kDppXor2>(x);
    x = dpp_max_step_f64<kDppHalfMirror>(x);
    x = dpp_max_step_f64<kDppMirror>(x);
    const double a = readlane_f64(x, 0), b = readlane_f64(x, 16), c = readlane_f64(x, 32), d = readlane_f64(x, 48);
    const double ab = a > b ? a : b, cd = c > d ? c : d;
    return ab > cd ? ab : cd;
}

template <int CTRL>
__device__ __forceinline__ int dpp_min_step_i32(int v) {
    const int w = (int)dpp_u32<CTRL, 0xF>((uint32_t)v);
    return w < v ? w : v;
}

__device__ __forceinline__ int wave_min_i32(int x) {
    x = dpp_min_step_i32<kDppXor1>(x);
    x = dpp_min_step_i32<kDppXor2>(x);
    x = dpp_min_step_i32<kDppHalfMirror>(x);
    x = dpp_min_step_i32<kDppMirror>(x);
    const int a = __builtin_amdgcn_readlane(x, 0), b = __builtin_amdgcn_readlane(x, 16);
    const int c = __builtin_amdgcn_readlane(x, 32), d = __builtin_amdgcn_readlane(x, 48);
    return min(min(a, b), min(c, d));
}

// LDS of the scheduling workgroup (NT threads).
template <int NT>
struct SchedShared {
    static constexpr int SW = NT / 64;
    // slot words (see slot_word); with n <= kMaxN / 2 the two halves are the merge's
    // source and destination in turn, above that it merges in place
    uint64_t item[kMaxN];
    // per-thread partial sums; reused as the selection map (one byte per slot)
    static constexpr int kPart = NT > (kMaxN + 23) / 24 ? NT : (kMaxN + 23) / 24;
    U192 part[kPart];
    uint32_t wsum[SW];
    U192 wsum192[SW];
    double wbest_f[SW];   // per wave: largest objective, the smallest B that reaches it, and
    int32_t wbest_b[SW];  // the smallest first-drop candidate
    int32_t wdrop[SW];
    int32_t b_star;
};

__device__ __forceinline__ uint64_t slot_word(uint32_t key, int f) { return ((uint64_t)key << 16) | (uint32_t)f; }
__device__ __forceinline__ uint32_t word_key(uint64_t x) { return (uint32_t)(x >> 16); }
__device__ __forceinline__ int word_slot(uint64_t x) { return (int)(x & 0xFFFFull); }

// Exclusive scan of one uint32 per thread over the block.  TRAIL: end with a barrier so
// that the next call may reuse sh.wsum at once (callers with barriers of their own in
// between pass false).
template <int NT, bool TRAIL = true>
__device__ __forceinline__ uint32_t block_excl_scan(SchedShared<NT>& sh, uint32_t v, uint32_t* total) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const uint32_t x = wave_incl_scan_u32(v);
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

// Exclusive scan of one 192-bit integer per thread.  sh.wsum192 may be written again
// once every thread has passed a later barrier.
template <int NT>
__device__ __forceinline__ U192 block_excl_scan192(SchedShared<NT>& sh, U192 v) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const U192 x = wave_incl_scan192(v);
    if (lane == 63) sh.wsum192[w] = x;
    __syncthreads();
    U192 off = {0ull, 0ull, 0ull};
    for (int q = 0; q < w; ++q) off = add192(off, sh.wsum192[q]);
    return sub192(add192(off, x), v);
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

// Stage 2 for all requests; slot words in flat order.  Each thread runs the sequential
// product of its request, its confidences requested eight at a time (one memory round
// trip for up to eight positions).  tok_lds (may be null): the request's draft tokens are
// copied there too, read in the same round trip.
template <int NT>
__device__ __forceinline__ void survival_to_lds(SchedShared<NT>& sh, const float* __restrict__ conf, int R, int K,
                                                float* __restrict__ surv_out, uint32_t* status,
                                                const int32_t* __restrict__ tokens = nullptr,
                                                int32_t* tok_lds = nullptr) {
    bool bad = false;
    for (int r = threadIdx.x; r < R; r += NT) {
        const int f0 = r * K;
        float s = 0.f;
        for (int i0 = 0; i0 < K; i0 += 8) {
            float c[8];
            int32_t tk[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) c[u] = i0 + u < K ? conf[f0 + i0 + u] : 0.f;
            if (tok_lds) {
#pragma unroll
                for (int u = 0; u < 8; ++u) tk[u] = i0 + u < K ? tokens[f0 + i0 + u] : 0;
            }
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int i = i0 + u;
                if (i < K) {
                    const float cu = sanitize_conf(c[u], bad);
                    s = (i == 0) ? cu : s * cu;
                    sh.item[f0 + i] = slot_word(kOne - __float_as_uint(s), f0 + i);
                    if (surv_out) surv_out[f0 + i] = s;
                    if (tok_lds) tok_lds[f0 + i] = tk[u];
                }
            }
        }
    }
    if (bad) raise_status(status, kStatusConfSanitized);
    __syncthreads();
}

// Survivals given in global memory (topb-only entry point); values outside [0,1] are clamped.
template <int NT>
__device__ __forceinline__ void surv_global_to_lds(SchedShared<NT>& sh, const float* __restrict__ surv, int n) {
    for (int f = threadIdx.x; f < n; f += NT) {
        bool bad = false;
        const float s = sanitize_conf(surv[f], bad);
        sh.item[f] = slot_word(kOne - __float_as_uint(s), f);
    }
    __syncthreads();
}

// One merge level for the word at index p of src (see merge_sort_slots), W = run0 << lvl:
// its partner run [plo, plo + len) and where it goes when c words of that run are below
// it (base + c).  With no partner run, len = 0 and plo = 1 (reads stay at src[0]).
struct MergeSlot {
    int plo, len, base;
};

// p / run0 for p, run0 <= 2^14 with magic = ceil(2^32 / run0) (run0 > 1): the product
// overshoots p / run0 by less than p / 2^32 <= 2^-18, while p / run0 stays at least
// 1 / run0 >= 2^-14 below the next integer, so the floor is exact.
__device__ __forceinline__ int run_index(int p, int run0, uint32_t magic) {
    return run0 == 1 ? p : (int)__umulhi((uint32_t)p, magic);
}

__device__ __forceinline__ MergeSlot merge_slot(int n, int p, int q, int lvl, int W) {
    const int j = q >> lvl;
    const int own = (int)__umul24((uint32_t)j, (uint32_t)W);  // < 2^24
    const bool odd = j & 1;
    MergeSlot m;
    m.plo = odd ? own - W : own + W;
    const int end = odd ? own : min(own + 2 * W, n);
    m.len = end - m.plo;
    m.base = odd ? p - W : p;  // the pair's start plus p's index in its own run
    if (m.len <= 0) {
        m.plo = 1;
        m.len = 0;
    }
    return m;
}

// Binary search step t (>= 1) reads the partner run's word t - 1, or its last word when
// t > len: the test "word < v" then answers as it does at t = len, so the predicate stays
// monotone in t and the count found, clamped to len at the end, is exact.  Every read is
// in [0, n).
__device__ __forceinline__ int merge_probe(const MergeSlot& m, int t) { return m.plo + (t < m.len ? t : m.len) - 1; }

// Where the word v at index p of src goes: words of the partner run below v counted by
// a binary search of top, top / 2, ..., 1 (top: the largest power of two <= W, so the
// steps reach any count up to W).
__device__ __forceinline__ int merge_dest(const uint64_t* src, int n, int p, uint64_t v, int run0, uint32_t magic,
                                          int lvl, int W, int top) {
    const MergeSlot m = merge_slot(n, p, run_index(p, run0, magic), lvl, W);
    int c = 0;
#pragma unroll 1
    for (int st = top; st > 0; st >>= 1) {
        const int t = c + st;
        c = src[merge_probe(m, t)] < v ? t : c;
    }
    return m.base + (c < m.len ? c : m.len);
}

// The same for two words at once (indices p0 and p1 of src), their searches interleaved
// so that each step's two LDS reads are in flight together.
__device__ __forceinline__ void merge_dest2(const uint64_t* src, int n, int p0, uint64_t v0, int p1, uint64_t v1,
                                            int run0, uint32_t magic, int lvl, int W, int top, int& d0, int& d1) {
    const MergeSlot m0 = merge_slot(n, p0, run_index(p0, run0, magic), lvl, W);
    const MergeSlot m1 = merge_slot(n, p1, run_index(p1, run0, magic), lvl, W);
    int c0 = 0, c1 = 0;
#pragma unroll 1
    for (int st = top; st > 0; st >>= 1) {
        const int t0 = c0 + st, t1 = c1 + st;
        const uint64_t x0 = src[merge_probe(m0, t0)];
        const uint64_t x1 = src[merge_probe(m1, t1)];
        c0 = x0 < v0 ? t0 : c0;
        c1 = x1 < v1 ? t1 : c1;
    }
    d0 = m0.base + (c0 < m0.len ? c0 : m0.len);
    d1 = m1.base + (c1 < m1.len ? c1 : m1.len);
}

// Sorts the n <= kMaxN / 2 slot words in sh.item, whose runs [j*run0, (j+1)*run0) are
// each ascending already (run0 = 1 for arbitrary words); returns where the sorted words
// are (sh.item or its upper half, the two halves serving as source and destination in
// turn).  Entered after a barrier that follows the last writes of the words.
// Level l merges run pairs of width W = run0 << l: the word at index p of run j moves to
// (start of the pair) + (p - j W) + (number of words of the partner run below it), so
// runs that are adjacent in flat order stay adjacent and no two words share a place.
template <int NT>
__device__ __forceinline__ const uint64_t* merge_sort_slots(SchedShared<NT>& sh, int n, int run0) {
    const int tid = threadIdx.x;
    uint64_t* src = sh.item;
    uint64_t* dst = sh.item + kMaxN / 2;
    const uint32_t magic = run0 > 1 ? (uint32_t)((0xFFFFFFFFull + (uint64_t)run0) / (uint64_t)run0) : 0u;
    int top = 1;  // largest power of two <= W
    while (2 * top <= run0) top *= 2;
    int lvl = 0;
#pragma unroll 1
    for (int W = run0; W < n; W *= 2, top *= 2, ++lvl) {
#pragma unroll 1
        for (int p0 = tid; p0 < n; p0 += 2 * NT) {
            const int p1 = p0 + NT;
            const uint64_t v0 = src[p0];
            if (p1 < n) {
                const uint64_t v1 = src[p1];
                int d0, d1;
                merge_dest2(src, n, p0, v0, p1, v1, run0, magic, lvl, W, top, d0, d1);
                dst[d0] = v0;
                dst[d1] = v1;
            } else {
                dst[merge_dest(src, n, p0, v0, run0, magic, lvl, W, top)] = v0;
            }
        }
        __syncthreads();
        uint64_t* t = src;
        src = dst;
        dst = t;
    }
    return src;
}

// Digit counters of the radix passes, digit-major with a stride of (waves + 1) words so
// that both the per-wave ranking (one digit per lane) and the block scan (consecutive
// (digit, wave) entries per thread) touch distinct LDS banks.  They live in the space of
// the per-thread partials (free until the selection map is built).
template <int NT>
__device__ __forceinline__ int hist_at(int d, int w) { return d * (NT / 64 + 1) + w; }

template <int NT>
__device__ __forceinline__ uint32_t* radix_hist(SchedShared<NT>& sh) {
    static_assert(sizeof(sh.part) >= 256 * (NT / 64 + 1) * sizeof(uint32_t), "the digit counters fit");
    return reinterpret_cast<uint32_t*>(&sh.part[0]);
}

// One stable counting pass over the 8-bit digit at key bit `shift` of the n_pad words in
// sh.item.  Wave w owns words [w*S, (w+1)*S) of the current order, 64 per round; a
// word's rank among equal digits of its wave comes from a ballot match of the digit
// bits and a running per-(digit, wave) counter.  Entered after a barrier that follows
// the last writes of the words.  A wave's counter column is written and read by that
// wave alone until the barrier before the offset scan, so clearing it needs no barrier
// of its own.
template <int NT>
__device__ __forceinline__ void radix_pass(SchedShared<NT>& sh, int n_pad, int shift) {
    constexpr int kSW = NT / 64, JM = kMaxN / NT;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int S = n_pad / kSW;  // words per wave, a multiple of 64
    const int J = S / 64;       // rounds, <= JM
    uint32_t* hist = radix_hist<NT>(sh);
    uint32_t k[JM];   // key bits of the word
    uint32_t il[JM];  // its flat id (low 16 bits) and rank among equal digits of the wave (high 16 bits)
    for (int d = lane; d < 256; d += 64) hist[hist_at<NT>(d, w)] = 0u;
#pragma unroll
    for (int j = 0; j < JM; ++j) {
        if (j < J) {
            const uint64_t x = sh.item[w * S + j * 64 + lane];
            k[j] = word_key(x);
            il[j] = (uint32_t)x & 0xFFFFu;
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
            const uint32_t h = hist[hist_at<NT>(d, w)];
            il[j] |= (h + before) << 16;
            if (before == 0u) hist[hist_at<NT>(d, w)] = h + (uint32_t)__popcll(peers);
        }
    }
    __syncthreads();
    // offsets in (digit, wave) order: entries e = 4*tid .. 4*tid+3 (256 digits x kSW
    // waves = 4 per thread), digit e / kSW, wave e % kSW
    uint32_t c[4], sum = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int e = 4 * tid + q;
        c[q] = hist[hist_at<NT>(e / kSW, e % kSW)];
        sum += c[q];
    }
    uint32_t ex = block_excl_scan<NT, false>(sh, sum, nullptr);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int e = 4 * tid + q;
        hist[hist_at<NT>(e / kSW, e % kSW)] = ex;
        ex += c[q];
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < JM; ++j) {
        if (j < J) {
            const uint32_t d = (k[j] >> shift) & 0xFFu;
            sh.item[hist[hist_at<NT>(d, w)] + (il[j] >> 16)] = slot_word(k[j], (int)(il[j] & 0xFFFFu));
        }
    }
    __syncthreads();
}

// The n slot words in sh.item sorted by four radix passes over their 32 key bits (the
// flat ids below them ride along; the passes are stable and the words start in flat
// order).  Pads up to a multiple of NT carry the largest key and sort last.
template <int NT>
__device__ __forceinline__ const uint64_t* radix_sort_words(SchedShared<NT>& sh, int n) {
    const int n_pad = pad_slots<NT>(n);
    for (int f = n + (int)threadIdx.x; f < n_pad; f += NT) sh.item[f] = ~0ull;
    __syncthreads();
#pragma unroll 1
    for (int shift = 0; shift < 32; shift += 8) radix_pass<NT>(sh, n_pad, shift);
    return sh.item;
}

// The n slot words ranked (see the file comment); run0 as in merge_sort_slots.
template <int NT>
__device__ __forceinline__ const uint64_t* rank_slots(SchedShared<NT>& sh, int n, int run0) {
    return n <= 2 * NT ? merge_sort_slots<NT>(sh, n, run0) : radix_sort_words<NT>(sh, n);
}

template <int NT>
__device__ __forceinline__ void write_ranking(const uint64_t* rk, int n, int32_t* __restrict__ order,
                                              float* __restrict__ sorted_surv, int32_t* __restrict__ rank) {
    for (int j = threadIdx.x; j < n; j += NT) {
        const uint64_t x = rk[j];
        const int f = word_slot(x);
        if (order) order[j] = f;
        if (sorted_surv) sorted_surv[j] = __uint_as_float(kOne - word_key(x));
        if (rank) rank[f] = j;
    }
}

// The cost-table entries of the first kCostPre candidates one thread evaluates in stage
// 4 (B = tid*C + q), of B = tid*C + C (the next thread's first candidate, which the
// first-drop rule compares against, n_pad for the last thread) and the draft cost, read
// at the start of the kernel so that their memory latency overlaps the earlier stages.
// With more than kCostPre * NT slots the later candidates read theirs in stage 4.
constexpr int kCostPre = 2;
struct CostPrefetch {
    float vc[kCostPre];
    float vc_next;
    float dc;
};

template <int NT>
__device__ __forceinline__ void prefetch_costs(CostPrefetch& cp, const float* __restrict__ vc,
                                               const float* __restrict__ dc, int T, int num_reqs, int bmax,
                                               int n_pad) {
    const int C = n_pad / NT;
    const int j0 = threadIdx.x * C;
#pragma unroll
    for (int q = 0; q < kCostPre; ++q) cp.vc[q] = (q < C && j0 + q <= bmax) ? vc[T + j0 + q] : 0.f;
    cp.vc_next = (j0 + C <= bmax) ? vc[T + j0 + C] : 0.f;
    cp.dc = dc[num_reqs];
}

// Stage 4 over the slot words rk (rank order); returns the budget (the same in every
// thread) and writes b_star and best_obj.  rule kRuleArgmax: the smallest B with the
// largest f.  rule kRuleFirstDrop: the first B whose successor does not raise f
// (f(B+1) <= f(B)), else bmax.  Every f(B) is the same double in both rules, so where f
// rises to a single peak they agree.  vcT is the verify-cost table from B = 0 (its
// entries beyond the prefetched ones are read here).
template <int NT>
__device__ __forceinline__ int choose_budget_lds(SchedShared<NT>& sh, const uint64_t* rk, const CostPrefetch& cp,
                                                 const float* __restrict__ vcT, int n, int n_pad, int n_sampling,
                                                 int bmax, int rule, int32_t* __restrict__ b_star,
                                                 double* __restrict__ best_obj, double* __restrict__ obj,
                                                 uint32_t* status) {
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    constexpr int kSW = NT / 64, QM = kMaxN / NT;
    constexpr int kNone = 0x7FFFFFFF;
    const int C = n_pad / NT;
    const int j0 = tid * C;
    // this thread's cost-table entries (those past the prefetched ones requested now, so
    // that their memory round trip overlaps the scan)
    float vq[QM];
#pragma unroll
    for (int q = 0; q < QM; ++q)
        vq[q] = (q < C && j0 + q <= bmax) ? (q < kCostPre ? cp.vc[q < kCostPre ? q : 0] : vcT[j0 + q]) : 0.f;
    U192 local = {0ull, 0ull, 0ull};
    for (int q = 0; q < C; ++q) {
        const int j = j0 + q;
        if (j < n) local = add192(local, fixed_from_bits(kOne - word_key(rk[j])));
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
    int bb = kNone;
    double fprev = 0.0;      // f(B-1) of the previous candidate of this thread
    int drop = kNone;        // first-drop candidate: B with f(B+1) <= f(B), and f(B)
    double fdrop = 0.0;
    auto take = [&](int B, double f, bool own) {
        if (own) {
            if (obj) obj[B] = f;
            if (f > bf || (f == bf && B < bb)) {
                bf = f;
                bb = B;
            }
            if (B == bmax && drop == kNone) {  // no drop before bmax: admission ends there
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
    for (int q = 0; q < QM; ++q) {
        if (q < C) {
            const int B = j0 + q;
            if (B <= bmax) take(B, eval(vq[q]), true);
            if (B < n) S = add192(S, fixed_from_bits(kOne - word_key(rk[B])));
        }
    }
    // B = j0 + C: the next thread's first candidate (compared against f(j0 + C - 1)), or
    // B = n_pad for the last thread.
    if (j0 + C <= bmax) take(j0 + C, eval(cp.vc_next), tid == NT - 1);
    if (bad) raise_status(status, kStatusCostInvalid);
    // Per wave: the largest f and the smallest B reaching it, and the smallest drop; then
    // every thread combines the waves' (a drop, once found, belongs to one thread only).
    const double fw = wave_max_f64(bf);
    const int bw = wave_min_i32(bf == fw ? bb : kNone);
    const int dw = wave_min_i32(drop);
    if (lane == 0) {
        sh.wbest_f[w] = fw;
        sh.wbest_b[w] = bw;
        sh.wdrop[w] = dw;
    }
    __syncthreads();
    static_assert(kSW <= 64, "one lane per wave's partials");
    const double fq = lane < kSW ? sh.wbest_f[lane] : -INFINITY;
    const int bq = lane < kSW ? sh.wbest_b[lane] : kNone;
    const double F = wave_max_f64(fq);
    const int Bx = wave_min_i32(fq == F ? bq : kNone);
    const int D = wave_min_i32(lane < kSW ? sh.wdrop[lane] : kNone);
    const int B = rule == kRuleFirstDrop ? D : Bx;
    if (tid == 0 && b_star) *b_star = B;
    if (best_obj) {
        if (rule == kRuleFirstDrop) {
            if (drop == D) *best_obj = fdrop;
        } else if (tid == 0) {
            *best_obj = F;
        }
    }
    __syncthreads();  // sh.wbest_* and sh.wdrop are read before they are written again
    return B;
}

// Stage 5.  sel must already mark the chosen slots (1 byte per flat id, n entries).
// lds_rows (may be null): per request r, lds_rows[2r] = its offset into ver_idx and
// lds_rows[2r + 1] = its prefix length.  tok_lds (may be null): the draft tokens, already
// in LDS.
template <int NT>
__device__ __forceinline__ void allocate_lds(SchedShared<NT>& sh, const uint8_t* sel, int R, int K, int B,
                             const int32_t* __restrict__ tokens, int32_t* __restrict__ prefix_len,
                             int32_t* __restrict__ offsets, int32_t* __restrict__ ver_idx,
                             int32_t* __restrict__ ver_tokens, int32_t* lds_rows = nullptr,
                             const int32_t* tok_lds = nullptr) {
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
                if (ver_tokens) ver_tokens[o + L] = tok_lds ? tok_lds[f] : tokens[f];
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
// budget": the size of B may come from confidences a step old, the slots themselves
// are then assigned by the current ones).  bmax is the largest B of that sizing, rule the admission
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
// null, may alias sh.item, which is free by then): each request's offset and prefix
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
    const uint64_t* rk = sh.item;
    // The draft tokens (for ver_tokens) go to LDS with the confidences when they fit past
    // the merge's upper half (n <= kMaxN / 3): words [kMaxN / 2 + n, kMaxN) are free.
    int32_t* tok_lds = (tokens && ver_tokens && 3 * n <= kMaxN)
                           ? reinterpret_cast<int32_t*>(sh.item + kMaxN / 2 + n) : nullptr;
#pragma unroll 1
    for (int ps = 0; ps < passes; ++ps) {
        const bool sizing = ps == 0, last = ps == passes - 1;
        const float* src = sz.separate && sizing ? sz.conf : conf;
        const int rows = sz.separate && sizing ? sz.R : R;
        const int m = rows * K, m_pad = pad_slots<NT>(m);
        const int bm = sz.separate ? sz.bmax : bmax;
        // the cost-table entries are requested before the confidences, so that both
        // memory round trips overlap (and the sort)
        CostPrefetch cp;
        if (sizing) prefetch_costs<NT>(cp, vc, dc, T, num_reqs, bm, m_pad);
        survival_to_lds<NT>(sh, src, rows, K, last ? surv_out : nullptr, status, tokens, last ? tok_lds : nullptr);
        rk = rank_slots<NT>(sh, m, K);  // each request's row is a sorted run
        if (sizing) {
            if (last) write_ranking<NT>(rk, n, order, sorted_surv, nullptr);
            B = choose_budget_lds<NT>(sh, rk, cp, vc + T, m, m_pad, n_sampling, bm, sz.rule, last ? b_star : nullptr,
                                      best_obj, nullptr, status);
        } else {
            write_ranking<NT>(rk, n, order, sorted_surv, nullptr);
        }
    }
    if (sz.separate) {
        B = B < n ? B : n;
        if (threadIdx.x == 0 && b_star) *b_star = B;
    }
    if (threadIdx.x == 0) sh.b_star = B;
    uint8_t* sel = selection_map<NT>(sh);
    for (int j = threadIdx.x; j < n; j += NT) sel[word_slot(rk[j])] = (uint8_t)(j < B);
    __syncthreads();
    allocate_lds<NT>(sh, sel, R, K, B, tokens, prefix_len, offsets, ver_idx, ver_tokens, lds_rows, tok_lds);
}

}  // namespace

}  // namespace dspark
