// Stage 1 (the chain) by candidate pruning.
//
// What is computed is the chain of the DSpark summary "How DSpark Speeds Up LLM
// Inference", section "Draft better" (a rank-r bias keyed on the previous token added to
// the backbone's logits, then an argmax; MAX worklog "DSpark on MAX", section "What
// DSpark is", item 3): for every request r and position i,
//     x[v] = base[r,i,v] + A[prev,:] . Bt[v,:],   tokens[r,i] = argmax_v x[v],  prev = tokens[r,i].
//
// The bias is bounded.  By the Cauchy-Schwarz inequality |A[u,:] . Bt[v,:]| <= a * b with
// a = max_u |A[u,:]| and b = max_v |Bt[v,:]| (Euclidean norms, weight properties measured
// once by dspark_markov_prepare).  With M = max_v base[v], the winner w has
// x[w] >= x[argmax base] >= M - a b, hence base[w] >= M - 2 a b.  Only the entries with
// base[v] >= M - 2ab (the candidates) can win, and which entries these are does not
// depend on the previous token.  So a row needs one streaming pass over its base logits
// (all of the stage's HBM traffic) that keeps its maximum and its candidates (index and
// value), and then the bias of a few tens of candidates instead of V entries.
// The bound is applied with a margin (2ab(1 + 2^-10), plus 2^-20 |M| for the rounding of
// the subtraction), so the candidate set always contains the exact (real-number, and
// hence the double-precision) argmax.  Among the candidates the kernel takes the float32
// argmax of fl32(base + fl32 dot).  Where the bound cannot prune, the row is scored over
// the whole vocabulary, so the result never depends on the data: a NaN in the row makes
// the first NaN the token (the bias is finite whenever the bound is, so x is NaN exactly
// where base is); a row of -inf gives 0; a row whose kept groups do not fit the LDS
// pool, or weights whose bound is not finite, are scored densely.
//
// One workgroup per compute unit takes requests g, g + G, ... whole, so a request's
// candidates never leave the compute unit's LDS (with fewer requests than compute units,
// helper workgroups stream shares of a request's rows and hand their kept groups over;
// see "One request over several workgroups" below).  Its eight waves (two per SIMD)
// split the work:
//
// Streaming (waves 0-6).  The request's K*V base entries are items of 4096 entries, 2048
// in rows of at most 32768 (a row is ceil(V/item) items); a wave takes the next item from an LDS counter whenever it
// starts a load, keeps the next item's loads in flight, and never waits for the other
// waves.  For each item it folds the item's maximum into the row's maximum in LDS
// and keeps, whole, every 8-entry group whose maximum clears the floor of the row's
// maximum seen so far (a lower bound of the final one, so nothing that can win is
// dropped): no entry is tested on its own here.  A row's kept groups are numbered by an
// LDS counter and stored in 64-group chunks of a per-request LDS pool, which the wave
// that claims a chunk's first place takes from the pool; then the item is counted into
// its row.
//
// Chain (wave 7), concurrently, at raised issue priority.  Position by position it waits
// for the row's count to reach its item count, lists the entries of the row's kept groups
// that clear the row's final floor, and scores them with the key row of the previous
// token, eight lanes per candidate (each load instruction reads whole 128-byte lines of
// eight Bt rows) with the Bt rows of up to 64 candidates in flight at once (x = value +
// the dot product: each lane's chunks by fused multiply-adds in increasing k, then the
// eight lanes' sums added as a tree).  The key row of the next position is prefetched
// for the row's largest entry -- the token unless the bias reorders the top -- while the
// row is scored, and loaded again only when that guess misses.  So the chain keeps up
// with the streaming, and only the last row's scoring is left once the last item arrives.
#include <hip/hip_ext.h>

#include "common.h"
#include "kernels.h"

namespace dspark {

namespace {

constexpr int kQS = 7;                   // streaming waves (with the chain wave, two waves per SIMD)
constexpr int kQT = (kQS + 1) * 64;      // threads per workgroup: the streaming waves and the chain wave
// Items are LOADS x 512 entries: 64 lanes x LOADS 16-byte loads x 8 entries (LOADS = 8 for
// items of kCandItemLong entries, 4 for kCandItemShort).
constexpr int kQChunk = 64;              // kept groups per chunk of the pool
constexpr int kQChunks = kCandGroups / kQChunk;  // chunks of the pool
constexpr uint8_t kQUnset = 0xFF;        // chunk table: not taken yet
constexpr uint8_t kQNone = 0xFE;         // chunk table: the pool was empty (the row is scored densely)
constexpr int kQList = 768;              // candidates the chain wave lists at once (256 + 64 groups' 512 at most)
constexpr int kQGList = 256;             // kept groups the chain wave lists at once
constexpr uint32_t kNegInfPair = 0xFF80FF80u;  // two bf16 -inf
constexpr long kQSpinLimit = 1L << 26;   // polls (with a short sleep each) before the chain wave gives up

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

static_assert(kQChunks <= 0xFE, "chunk numbers fit a byte beside the two marks");
static_assert((long)kCandMaxItems * kCandItemLong / 8 <= 65536, "group numbers within a row fit 16 bits");
static_assert(kCandItemLong == 8 * 512 && kCandItemShort == 4 * 512, "items are whole 512-entry loads");

// Order-preserving image of a float in the unsigned integers (NaN above every number,
// -0 equal to +0); never 0.
__device__ __forceinline__ uint32_t ord32(float x) {
    uint32_t b = __float_as_uint(x);
    if (x != x) return 0xFFFFFFFFu;
    if (b == 0x80000000u) b = 0u;
    return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

__device__ __forceinline__ float unord32(uint32_t u) {
    return __uint_as_float((u & 0x80000000u) ? (u & 0x7FFFFFFFu) : ~u);
}

// Lowest value a candidate of a row with maximum M may have: M - ab2 - |M| 2^-20, where
// ab2 >= 2 a b (1 + 2^-10) already carries the bound's margin; the |M| term covers the
// rounding of this subtraction.  An infinite maximum keeps the entries equal to it.
__device__ __forceinline__ float cand_floor(float M, float ab2) {
    if (M == __builtin_huge_valf()) return M;
    return (M - ab2) - __builtin_fabsf(M) * 0x1p-20f;
}

// DPP lane moves within rows of 16 lanes (no LDS round trip, unlike a shuffle).
constexpr int kDppXor1 = 0xB1;         // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;         // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;  // lane i <-> 7 - i within each 8
constexpr int kDppMirror = 0x140;      // lane i <-> 15 - i within each 16

__device__ __forceinline__ float dpp_f32(float x, int ctrl) {
    switch (ctrl) {  // the control must be a constant of the builtin
        case kDppXor1: return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), kDppXor1, 0xF, 0xF, false));
        case kDppXor2: return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), kDppXor2, 0xF, 0xF, false));
        case kDppHalfMirror:
            return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), kDppHalfMirror, 0xF, 0xF, false));
        default: return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), kDppMirror, 0xF, 0xF, false));
    }
}

__device__ __forceinline__ uint64_t dpp_u64(uint64_t x, int ctrl) {
    const uint32_t lo = __float_as_uint(dpp_f32(__uint_as_float((uint32_t)x), ctrl));
    const uint32_t hi = __float_as_uint(dpp_f32(__uint_as_float((uint32_t)(x >> 32)), ctrl));
    return ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ uint64_t pack_u64(int hi, int lo) { return ((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo; }

__device__ __forceinline__ uint64_t readlane_u64(uint64_t x, int lane) {
    const int hi = (int)(x >> 32), lo = (int)x;
    switch (lane) {  // the lane must be a constant of the builtin
        case 0: return pack_u64(__builtin_amdgcn_readlane(hi, 0), __builtin_amdgcn_readlane(lo, 0));
        case 16: return pack_u64(__builtin_amdgcn_readlane(hi, 16), __builtin_amdgcn_readlane(lo, 16));
        case 32: return pack_u64(__builtin_amdgcn_readlane(hi, 32), __builtin_amdgcn_readlane(lo, 32));
        default: return pack_u64(__builtin_amdgcn_readlane(hi, 48), __builtin_amdgcn_readlane(lo, 48));
    }
}

// The maximum over the wave (NaN if any lane holds one), the same in every lane: within
// rows of 16 by lane moves, then the four rows' values read out.
__device__ __forceinline__ float wave_max(float x) {
    x = __builtin_elementwise_maximum(x, dpp_f32(x, kDppXor1));
    x = __builtin_elementwise_maximum(x, dpp_f32(x, kDppXor2));
    x = __builtin_elementwise_maximum(x, dpp_f32(x, kDppHalfMirror));
    x = __builtin_elementwise_maximum(x, dpp_f32(x, kDppMirror));
    const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 0));
    const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 16));
    const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 32));
    const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 48));
    return __builtin_elementwise_maximum(__builtin_elementwise_maximum(r0, r1), __builtin_elementwise_maximum(r2, r3));
}

// Exclusive prefix sum over the wave of values below 128, from one ballot per bit (no
// LDS round trip); *total receives the sum.
__device__ __forceinline__ uint32_t wave_excl_scan_small(uint32_t v, uint32_t* total) {
    uint32_t pre = 0u, tot = 0u;
#pragma unroll
    for (int b = 0; b < 7; ++b) {
        const uint64_t m = __ballot((v >> b) & 1u);
        const uint32_t below =
            __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
        pre += below << b;
        tot += (uint32_t)__builtin_popcountll(m) << b;
    }
    *total = tot;
    return pre;
}

__device__ __forceinline__ uint32_t wave_min_u32(uint32_t x) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
        const uint32_t y = __shfl_xor(x, o, 64);
        x = y < x ? y : x;
    }
    return x;
}

// The largest key over the wave (every lane active), the same in every lane: as wave_max.
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t x) {
    x = umax64(x, dpp_u64(x, kDppXor1));
    x = umax64(x, dpp_u64(x, kDppXor2));
    x = umax64(x, dpp_u64(x, kDppHalfMirror));
    x = umax64(x, dpp_u64(x, kDppMirror));
    return umax64(umax64(readlane_u64(x, 0), readlane_u64(x, 16)), umax64(readlane_u64(x, 32), readlane_u64(x, 48)));
}

// LDS written by some lanes of a wave and read by others: the writes come first.
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// The prepared head's bound: ab2 = 2 a b (1 + 2^-10) rounded up, ok = it is finite, and
// b1 = b (1 + 2^-10) rounded up (a, b: the largest row norms of A and Bt).
struct HeaderView {
    float ab2;
    bool ok;
    float b1;
};

__device__ __forceinline__ HeaderView header_view(const void* hdr) {
    const uint32_t* h = (const uint32_t*)hdr;
    return HeaderView{__uint_as_float(h[4]), h[5] != 0u, __uint_as_float(h[6])};
}

// LDS of one request.
struct QLds {
    u32x4 grp[kCandGroups];                  // kept 8-entry groups (bf16), in chunks of kQChunk
    uint16_t gid[kCandGroups];               // their group numbers within the row (first entry / 8)
    uint8_t ctab[kCandMaxK][kQChunks];       // per row: pool chunk of each of its chunks (kQUnset, kQNone)
    uint32_t rowfill[kCandMaxK];             // groups each row has kept (places claimed)
    uint32_t rowover[kCandMaxK];             // 1: some of a row's groups found no chunk (the row is scored densely)
    uint32_t pool;                           // chunks taken from the pool
    uint64_t clist[kQList];                  // the chain wave's listed candidates
    uint16_t glist[kQGList];                 // the chain wave's listed groups (their places in the pool)
    uint16_t akey[256];                      // key row of a densely scored row
    uint32_t rowmax[kCandMaxK];              // the rows' maxima so far (order-preserving image; 0 = none yet)
    uint32_t rownan[kCandMaxK];              // ~(first NaN index), 0 = none
    uint32_t rowdone[kCandMaxK];             // items of the row kept so far
    uint32_t next;                           // the next item to hand to a streaming wave
};

// LDS writes of this wave complete, and not moved past this point by the compiler.  (A
// release fence at workgroup scope would also wait for the wave's global loads in
// flight.)
__device__ __forceinline__ void lds_writes_done() {
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt and expcnt not waited for
    asm volatile("" ::: "memory");
}

// ---------------------------------------------------------------------------------
// Streaming

// Entries [v0, v0 + 512 LOADS) of a row into buf (LOADS groups of 8 entries per lane;
// entries past V read as -inf).  VEC: 8 | V and an aligned base, so groups are 16-byte aligned and
// wholly in or out of the row.
template <bool VEC, int LOADS>
__device__ __forceinline__ void load_item(u32x4 (&buf)[LOADS], const uint16_t* __restrict__ p, int v0, int V) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int q = 0; q < LOADS; ++q) {
        const int e = v0 + q * 512 + lane * 8;
        if (VEC) {
            // every load is issued (past the row, at the row's start), so that the number of
            // loads in flight is the same on every path and the waits for one buffer never
            // wait for the buffers loaded after it
            const u32x4 x = __builtin_nontemporal_load((const u32x4*)(p + (e < V ? e : 0)));
            buf[q] = e < V ? x : u32x4{kNegInfPair, kNegInfPair, kNegInfPair, kNegInfPair};
        } else {
            uint32_t h[8];
#pragma unroll
            for (int t = 0; t < 8; ++t) h[t] = e + t < V ? (uint32_t)p[e + t] : 0xFF80u;
            buf[q] = u32x4{h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16)};
        }
    }
}

// The maxima of an item's LOADS 8-entry groups (per lane).
template <int LOADS>
__device__ __forceinline__ void group_maxima(const u32x4 (&cur)[LOADS], float (&gm)[LOADS]) {
#pragma unroll
    for (int q = 0; q < LOADS; ++q) {
        float g = -__builtin_huge_valf();
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            const uint32_t x = cur[q][d];
            g = __builtin_elementwise_maximum(
                g, __builtin_elementwise_maximum(__uint_as_float(x << 16), __uint_as_float(x & 0xFFFF0000u)));
        }
        gm[q] = g;
    }
}

// Entry t (0..7) of 16-byte group `word4` as a float.  The word goes through an empty asm
// statement first, so the compiler recomputes the unpacking where it is used instead of
// keeping all 64 unpacked entries of an item live across the passes over it.
__device__ __forceinline__ float entry_of(const u32x4& word4, int t) {
    uint32_t w = word4[t >> 1];
    asm volatile("" : "+v"(w));
    return __uint_as_float((t & 1) ? (w & 0xFFFF0000u) : (w << 16));
}

// Pool chunks for row i's kept-group places [at, at + n), just claimed by this wave.  The
// chunks whose first place lies in the range are this wave's to take (a lane each); the
// chunk holding `at`, when `at` is not its first place, is taken by the wave that claimed
// that first place -- an earlier claim, whose wave takes its chunks straight after it --
// and is waited for.  A chunk past the table, or not found, reads as none.
__device__ __forceinline__ void take_chunks(QLds& L, int i, uint32_t at, uint32_t n) {
    const int lane = threadIdx.x & 63;
    const uint32_t c0 = at / kQChunk, c1 = (at + n - 1u) / kQChunk;
    const uint32_t first = (at % kQChunk == 0u) ? c0 : c0 + 1u;
    const uint32_t c = first + (uint32_t)lane;  // n <= 512: at most 9 chunks
    if (c <= c1 && c < (uint32_t)kQChunks) {
        const uint32_t id = __hip_atomic_fetch_add(&L.pool, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        L.ctab[i][c] = id < (uint32_t)kQChunks ? (uint8_t)id : kQNone;
    }
    if (first != c0 && c0 < (uint32_t)kQChunks && lane == 0) {
        const volatile uint8_t* t = &L.ctab[i][c0];
        for (long n_polls = 0; *t == kQUnset && n_polls < kQSpinLimit; ++n_polls) __builtin_amdgcn_s_sleep(1);
    }
    wave_lds_sync();
}

// One item of a streaming wave (see the file comment): the item's maximum into its row's
// (or its first NaN into the row's mark), then every 8-entry group of the item whose
// maximum clears the floor of the row's maximum so far, kept whole with its group number
// at places claimed in row i's chunks; then the item is counted into its row (the count
// after it is returned).  A group of
// -inf entries never wins unless the whole row is -inf, which is handled apart, so it is
// never kept.
template <int LOADS>
__device__ __forceinline__ uint32_t keep_item(QLds& L, const u32x4 (&cur)[LOADS], int i, int v0, float ab2) {
    const int lane = threadIdx.x & 63;
    constexpr float kNegInf = -__builtin_huge_valf();
    float gm[LOADS];
    group_maxima<LOADS>(cur, gm);
    float m = gm[0];
#pragma unroll
    for (int q = 1; q < LOADS; ++q) m = __builtin_elementwise_maximum(m, gm[q]);
    const float mw = wave_max(m);
    if (mw != mw) {
        // the row's token is its first NaN, whatever the bias
        uint32_t first = 0xFFFFFFFFu;
#pragma unroll
        for (int q = LOADS - 1; q >= 0; --q) {
            if (gm[q] != gm[q]) {
#pragma unroll
                for (int s = 7; s >= 0; --s) {
                    const float x = entry_of(cur[q], s);
                    if (x != x) first = (uint32_t)(v0 + q * 512 + lane * 8 + s);
                }
            }
        }
        first = wave_min_u32(first);
        if (lane == 0) atomicMax(&L.rownan[i], ~first);
    } else {
        uint32_t seen = 0u;
        if (lane == 0) seen = atomicMax(&L.rowmax[i], ord32(mw));
        seen = __builtin_amdgcn_readfirstlane(seen);
        const uint32_t now = seen > ord32(mw) ? seen : ord32(mw);
        const float fl = cand_floor(unord32(now), ab2);
        uint32_t need = 0u;  // bit q: group q of this lane is kept
#pragma unroll
        for (int q = 0; q < LOADS; ++q) need |= (gm[q] >= fl && gm[q] > kNegInf) ? (1u << q) : 0u;
        uint32_t total = 0;
        const uint32_t before = wave_excl_scan_small((uint32_t)__builtin_popcount(need), &total);
        if (total != 0u) {
            uint32_t at = 0u;
            if (lane == 0)
                at = __hip_atomic_fetch_add(&L.rowfill[i], total, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
            at = __builtin_amdgcn_readfirstlane(at);
            take_chunks(L, i, at, total);
            // this lane's places [p, p + popcount(need)) lie in chunk ca or the next
            uint32_t p = at + before;
            const uint32_t ca = p / kQChunk;
            const uint32_t ida = ca < (uint32_t)kQChunks ? (uint32_t)L.ctab[i][ca] : (uint32_t)kQNone;
            const uint32_t idb = ca + 1u < (uint32_t)kQChunks ? (uint32_t)L.ctab[i][ca + 1u] : (uint32_t)kQNone;
            const uint32_t g0 = ((uint32_t)v0 >> 3) + (uint32_t)lane;
            bool lost = false;
#pragma unroll
            for (int q = 0; q < LOADS; ++q) {
                if (__ballot((need >> q) & 1u) == 0ull) continue;
                if ((need >> q) & 1u) {
                    const uint32_t id = p / kQChunk == ca ? ida : idb;
                    if (id < (uint32_t)kQChunks) {
                        const uint32_t slot = id * kQChunk + p % kQChunk;
                        L.grp[slot] = cur[q];
                        L.gid[slot] = (uint16_t)(g0 + (uint32_t)q * 64u);
                    } else {
                        lost = true;
                    }
                    ++p;
                }
            }
            if (__ballot(lost) != 0ull && lane == 0) L.rowover[i] = 1u;  // the row is scored densely
        }
    }
    lds_writes_done();
    uint32_t done = 0u;
    if (lane == 0) done = __hip_atomic_fetch_add(&L.rowdone[i], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    return __builtin_amdgcn_readfirstlane(done) + 1u;
}

// ---------------------------------------------------------------------------------
// One request over several workgroups (a.S > 1)

// Header of a helper's row in the workspace: the launch epoch it was written in (set
// last), the row's maximum over the helper's share (order-preserving image, 0 = none),
// its kept groups (kSplitNone: more than kSplitCap) and ~(first NaN index) (0 = none).
struct SplitHdr {
    uint32_t flag, max, count, nan;
};
constexpr uint32_t kSplitNone = 0xFFFFFFFFu;
static_assert(sizeof(SplitHdr) == kSplitHdrBytes, "header size");

// Helper h = r (S - 1) + s - 1 of request r (share s >= 1): header of its row i, and its
// groups for that row.
__device__ __forceinline__ SplitHdr* split_hdr(const CandArgs& a, int h, int i) {
    return reinterpret_cast<SplitHdr*>(reinterpret_cast<char*>(a.split_ctl) + 256) + (size_t)h * kCandMaxK + i;
}
__device__ __forceinline__ size_t split_row(const CandArgs& a, int h, int i) {
    return ((size_t)h * (size_t)a.K + (size_t)i) * kSplitCap;
}
__device__ __forceinline__ u32x4* split_grp(const CandArgs& a) { return reinterpret_cast<u32x4*>(a.split_grp); }
__device__ __forceinline__ uint32_t* split_gid(const CandArgs& a) { return a.split_gid; }

// A row's NC items split S ways (in the request's rotated order, below) are dealt in
// rounds of P = 2S - 1: the owner (share 0) takes the first of each round, helper s the
// (2s - 1)-th and 2s-th, so that the owner, which also imports the helpers' groups and
// runs the chain, streams half as much as a helper, and the workgroups of one request
// read neighbouring items at any time.  S = 1: every item, in order.
__device__ __forceinline__ int share_items(int s, int NC, int S) {
    const int P = 2 * S - 1, full = NC / P, rem = NC - full * P;
    if (s == 0) return full + (rem > 0 ? 1 : 0);
    const int extra = rem - (2 * s - 1);
    return 2 * full + (extra < 0 ? 0 : (extra > 2 ? 2 : extra));
}
// Position within the row's dealing of share s's t-th item.
__device__ __forceinline__ int share_item(int s, int t, int S) {
    const int P = 2 * S - 1;
    return s == 0 ? t * P : (t >> 1) * P + 2 * s - 1 + (t & 1);
}

// Words exchanged between workgroups, which may sit on different dies, are stored and
// loaded as relaxed device-scope atomics: each access is coherent by itself, without the
// whole-cache write-back or invalidation that a release or acquire fence would cost
// every other workgroup on the die.  Order comes from waiting: the writer's stores have
// all completed before it stores the epoch, and the reader loads nothing before it has
// seen the epoch.
__device__ __forceinline__ void put_u32(uint32_t* p, uint32_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t get_u32(uint32_t* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void put_grp(u32x4* p, const u32x4& g) {
    uint64_t* q = reinterpret_cast<uint64_t*>(p);
    __hip_atomic_store(q, ((uint64_t)g[1] << 32) | g[0], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(q + 1, ((uint64_t)g[3] << 32) | g[2], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ u32x4 get_grp(u32x4* p) {
    uint64_t* q = reinterpret_cast<uint64_t*>(p);
    const uint64_t lo = __hip_atomic_load(q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const uint64_t hi = __hip_atomic_load(q + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return u32x4{(uint32_t)lo, (uint32_t)(lo >> 32), (uint32_t)hi, (uint32_t)(hi >> 32)};
}
// Every memory access of this wave so far has completed (stores included).
__device__ __forceinline__ void wave_memory_done() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0);
    asm volatile("" ::: "memory");
}

// A helper's wave that has just completed row i: the row's kept groups (unless more than
// kSplitCap, or some found no chunk) and its header go to the workspace, the epoch last.
__device__ __forceinline__ void export_row(QLds& L, const CandArgs& a, int h, int i, uint32_t ep) {
    const int lane = threadIdx.x & 63;
    const uint32_t total = L.rowfill[i];
    const bool none = L.rowover[i] != 0u || total > (uint32_t)kSplitCap;
    if (!none) {
        u32x4* gd = split_grp(a) + split_row(a, h, i);
        uint32_t* gg = split_gid(a) + split_row(a, h, i);
        for (uint32_t e = (uint32_t)lane; e < total; e += 64u) {
            const uint32_t slot = (L.ctab[i][e / kQChunk] % (uint32_t)kQChunks) * kQChunk + e % kQChunk;
            put_grp(gd + e, L.grp[slot]);
            put_u32(gg + e, L.gid[slot]);
        }
    }
    SplitHdr* hd = split_hdr(a, h, i);
    if (lane == 0) {
        put_u32(&hd->max, L.rowmax[i]);
        put_u32(&hd->count, none ? kSplitNone : total);
        put_u32(&hd->nan, L.rownan[i]);
    }
    wave_memory_done();
    if (lane == 0) put_u32(&hd->flag, ep);
}

// The owner's import of share p >= 1 of row i: once the helper has written the row in this
// launch (its epoch), the row's maximum and first NaN join the owner's, and so do the
// helper's kept groups that clear the floor of the row's maximum as now known (the helper
// kept against its share's maximum alone); the share's items are counted into the row.  A
// helper not heard from within the poll limit, or with more groups than it could hand
// over, leaves the row to be scored densely.
__device__ __forceinline__ void import_row(QLds& L, const CandArgs& a, int r, int p, int i, uint32_t ep, float ab2) {
    const int lane = threadIdx.x & 63;
    const int h = r * (a.S - 1) + p - 1;
    SplitHdr* hd = split_hdr(a, h, i);
    uint32_t seen = 1u;
    if (lane == 0) {
        for (long n_polls = 0; get_u32(&hd->flag) != ep;) {
            if (++n_polls > kQSpinLimit) {
                seen = 0u;
                raise_status(a.status, kStatusSyncTimeout);
                break;
            }
            __builtin_amdgcn_s_sleep(2);
        }
    }
    seen = __builtin_amdgcn_readfirstlane(seen);
    asm volatile("" ::: "memory");
    if (seen == 0u) {
        if (lane == 0) L.rowover[i] = 1u;
    } else {
        const uint32_t hmax = get_u32(&hd->max), cnt = get_u32(&hd->count), hnan = get_u32(&hd->nan);
        if (lane == 0) {
            if (hnan != 0u) atomicMax(&L.rownan[i], hnan);
            if (hmax != 0u) atomicMax(&L.rowmax[i], hmax);
        }
        if (cnt > (uint32_t)kSplitCap) {
            if (lane == 0) L.rowover[i] = 1u;
        } else if (cnt != 0u) {
            constexpr float kNegInf = -__builtin_huge_valf();
            const uint32_t own = __hip_atomic_load(&L.rowmax[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
            const uint32_t now = own > hmax ? own : hmax;
            const float fl = now != 0u ? cand_floor(unord32(now), ab2) : kNegInf;
            u32x4* gd = split_grp(a) + split_row(a, h, i);
            uint32_t* gg = split_gid(a) + split_row(a, h, i);
            bool lost = false;
            // four lists of 64 groups at a time, their loads all in flight together
            for (uint32_t e0 = 0; e0 < cnt; e0 += 4u * 64u) {
                u32x4 gv[4];
                uint32_t iv[4];
#pragma unroll
                for (int b = 0; b < 4; ++b) {
                    const uint32_t e = e0 + (uint32_t)b * 64u + (uint32_t)lane;
                    if (e < cnt) {
                        gv[b] = get_grp(gd + e);
                        iv[b] = get_u32(gg + e);
                    }
                }
#pragma unroll
                for (int b = 0; b < 4; ++b) {
                    const uint32_t e = e0 + (uint32_t)b * 64u + (uint32_t)lane;
                    float gx = kNegInf;
                    if (e < cnt) {
#pragma unroll
                        for (int d = 0; d < 4; ++d)
                            gx = __builtin_elementwise_maximum(
                                gx, __builtin_elementwise_maximum(__uint_as_float(gv[b][d] << 16),
                                                                  __uint_as_float(gv[b][d] & 0xFFFF0000u)));
                    }
                    const bool keep = e < cnt && gx >= fl && gx > kNegInf;
                    const uint64_t bal = __ballot(keep);
                    const uint32_t nk = (uint32_t)__builtin_popcountll(bal);
                    if (nk == 0u) continue;
                    uint32_t at = 0u;
                    if (lane == 0)
                        at = __hip_atomic_fetch_add(&L.rowfill[i], nk, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
                    at = __builtin_amdgcn_readfirstlane(at);
                    take_chunks(L, i, at, nk);
                    if (keep) {
                        const uint32_t q = at + (uint32_t)__builtin_popcountll(bal & ((1ull << lane) - 1ull));
                        const uint32_t c = q / kQChunk;
                        const uint32_t id = c < (uint32_t)kQChunks ? (uint32_t)L.ctab[i][c] : (uint32_t)kQNone;
                        if (id < (uint32_t)kQChunks) {
                            L.grp[id * kQChunk + q % kQChunk] = gv[b];
                            L.gid[id * kQChunk + q % kQChunk] = (uint16_t)iv[b];
                        } else {
                            lost = true;
                        }
                    }
                }
            }
            if (__ballot(lost) != 0ull && lane == 0) L.rowover[i] = 1u;
        }
    }
    lds_writes_done();
    const uint32_t items = (uint32_t)share_items(p, a.NC, a.S);
    if (lane == 0) __hip_atomic_fetch_add(&L.rowdone[i], items, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

// ---------------------------------------------------------------------------------
// A streaming wave's tasks of one request.  Every row has T tasks: the workgroup's share
// of the row's items (all of them when S = 1) and, for the owner of a split request
// (MODE 2), one import per helper.  Request r visits a row's items from item r mod NC on,
// wrapping round, so that requests whose rows lie a power of two apart do not all read
// the same offset (and so the same memory channels) at once.
// MODE 0: whole requests; MODE 1: a helper (exports each row it completes); MODE 2: the
// owner.  A wave takes the next task from the workgroup's counter whenever it starts
// loading one, so that waves which happen to be served faster take more, and tasks are
// taken in order (rows complete in order).  Each item is loaded one item ahead (two
// buffers in turn); a task that is no item (an import, or past the request) loads nothing
// (v0 = V: every entry reads as -inf).  Items are 512 LOADS entries.
template <bool VEC, int MODE, int LOADS>
__device__ __forceinline__ void stream_tasks(QLds& L, const CandArgs& a, int r, int s, float ab2, uint32_t ep) {
    constexpr int kItem = LOADS * 512;
    const int K = a.K, NC = a.NC, V = a.V;
    const int S = MODE == 0 ? 1 : a.S;
    const int n_own = share_items(s, NC, S);
    const int T = n_own + (MODE == 2 ? S - 1 : 0);
    const int rot = r % NC;
    auto item_of = [&](int t) {  // item index within the row of the t-th own task
        const int u = rot + share_item(s, t, S);
        return u < NC ? u : u - NC;
    };
    const int per_req = K * T;
    const uint16_t* rbase = a.base + (size_t)r * (size_t)K * (size_t)V;
    auto claim = [&]() -> int {
        uint32_t j = 0u;
        if ((threadIdx.x & 63) == 0) j = atomicAdd(&L.next, 1u);
        return (int)__builtin_amdgcn_readfirstlane(j);
    };
    auto issue = [&](u32x4 (&buf)[LOADS], int j) {
        const int i = j / T, t = j - i * T;
        const bool ok = j < per_req && t < n_own;
        load_item<VEC, LOADS>(buf, rbase + (size_t)(ok ? i : 0) * V, ok ? item_of(t) * kItem : V, V);
    };
    auto take = [&](const u32x4 (&buf)[LOADS], int j) {
        if (j < per_req) {
            const int i = j / T, t = j - i * T;
            if (t < n_own) {
                const uint32_t done = keep_item<LOADS>(L, buf, i, item_of(t) * kItem, ab2);
                if constexpr (MODE == 1) {
                    if (done == (uint32_t)n_own) export_row(L, a, r * (a.S - 1) + s - 1, i, ep);
                }
            } else if constexpr (MODE == 2) {
                import_row(L, a, r, t - n_own + 1, i, ep, ab2);
            }
        }
    };
    // (one item ahead already reads at the device's rate, and the chain wave's own loads
    // then queue behind fewer of the streams' than with two)
    u32x4 b0[LOADS], b1[LOADS];
    int j0 = claim(), j1;
    issue(b0, j0);
    while (j0 < per_req) {
        j1 = claim();
        issue(b1, j1);
        take(b0, j0);
        j0 = claim();
        issue(b0, j0);
        take(b1, j1);
    }
}

// ---------------------------------------------------------------------------------
// Chain

// This lane's four entries of a key row (A row u) or of a Bt row: entries [4 lane, 4 lane + 4).
__device__ __forceinline__ u32x2 row_quad(const uint16_t* __restrict__ M, int u, int rank) {
    const int lane = threadIdx.x & 63;
    return 4 * lane < rank ? *(const u32x2*)(M + (size_t)u * rank + 4 * lane) : u32x2{0u, 0u};
}

// Candidates are scored eight lanes each: lanes 8c .. 8c+7 of the wave take candidate c of
// a pass (8 candidates per pass).  A Bt row of rank entries is rank/8 16-byte chunks;
// chunk j belongs to lane j mod 8, as its (j div 8)-th, so that each load instruction of
// the pass reads whole 128-byte lines of the 8 rows.  kQRounds = the chunks a lane holds
// per row (rank <= 256); kQPasses = the passes whose loads are in flight together.
constexpr int kQRounds = 4;
constexpr int kQPasses = 8;

// This lane's chunks of Bt row v.
__device__ __forceinline__ void load_bt_part(u32x4 (&bt)[kQRounds], const uint16_t* __restrict__ Bt, int v, int rank) {
    const int l = threadIdx.x & 7, nch = rank / 8;
    const u32x4* b = (const u32x4*)(Bt + (size_t)v * rank);
#pragma unroll
    for (int g = 0; g < kQRounds; ++g) bt[g] = g * 8 + l < nch ? b[g * 8 + l] : u32x4{0u, 0u, 0u, 0u};
}

// x for this lane group's entry: fl32(value + the dot product of the key row in L.akey and
// the Bt row).  Each lane sums its chunks' products by fused multiply-adds in increasing k;
// the eight lanes' sums are then added as a tree (neighbours, then pairs, then quads), the
// same way round in every lane, so that all eight end with the same value.
__device__ __forceinline__ float oct_x(const QLds& L, const u32x4 (&bt)[kQRounds], int rank, float value) {
    const int l = threadIdx.x & 7, nch = rank / 8;
    const u32x4* k = (const u32x4*)L.akey;
    float acc = 0.f;
#pragma unroll
    for (int g = 0; g < kQRounds; ++g) {
        if (g * 8 + l < nch) {
            const u32x4 kv = k[g * 8 + l], bv = bt[g];
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                acc = __builtin_fmaf(__uint_as_float(kv[d] << 16), __uint_as_float(bv[d] << 16), acc);
                acc = __builtin_fmaf(__uint_as_float(kv[d] & 0xFFFF0000u), __uint_as_float(bv[d] & 0xFFFF0000u), acc);
            }
        }
    }
    // lane pairs, then pairs of pairs, then the two quads (lane i <-> 7 - i); each sum is
    // formed with the lower lanes' part first, so both partners compute the same value
    float o = dpp_f32(acc, kDppXor1);
    acc = (l & 1) ? o + acc : acc + o;
    o = dpp_f32(acc, kDppXor2);
    acc = (l & 2) ? o + acc : acc + o;
    o = dpp_f32(acc, kDppHalfMirror);
    acc = (l & 4) ? o + acc : acc + o;
    return value + acc;
}

// Candidates c0 + 8p + (lane div 8), p < kQPasses, of a list of n scored into best: all
// their Bt loads in flight together.  at(c) gives candidate c's (index, value bits) key as
// the list stores it.
template <typename At>
__device__ __forceinline__ void score_passes(const QLds& L, uint32_t c0, uint32_t n, const uint16_t* __restrict__ Bt,
                                             int rank, At at, uint64_t& best) {
    const uint32_t grp = (threadIdx.x & 63) >> 3;
    u32x4 bt[kQPasses][kQRounds];
    uint64_t e[kQPasses];
#pragma unroll
    for (int p = 0; p < kQPasses; ++p) {
        const uint32_t c = c0 + 8u * (uint32_t)p + grp;
        e[p] = at(c < n ? c : c0);
        if (c0 + 8u * (uint32_t)p < n) load_bt_part(bt[p], Bt, (int)(e[p] >> 32), rank);
    }
#pragma unroll
    for (int p = 0; p < kQPasses; ++p) {
        if (c0 + 8u * (uint32_t)p < n) {
            const uint32_t c = c0 + 8u * (uint32_t)p + grp;
            const float x = oct_x(L, bt[p], rank, __uint_as_float((uint32_t)e[p]));
            if (c < n) best = umax64(best, argmax_key(x, (uint32_t)(e[p] >> 32)));
        }
    }
}

// Row `row` scored over the whole vocabulary with the key row in L.akey, 64 entries at a
// time.  Returns the argmax key (every lane alike).
__device__ __forceinline__ uint64_t dense_row(const QLds& L, const uint16_t* __restrict__ bp, int V,
                                              const uint16_t* __restrict__ Bt, int rank) {
    uint64_t best = 0ull;
    auto at = [&](uint32_t v) -> uint64_t { return ((uint64_t)v << 32) | ((uint32_t)bp[v] << 16); };
    for (uint32_t v0 = 0; v0 < (uint32_t)V; v0 += 8u * kQPasses) score_passes(L, v0, (uint32_t)V, Bt, rank, at, best);
    return wave_max_u64(best);
}

// Scores L.clist[0, n) with the key row in L.akey into best, 64 candidates at a time.
__device__ __forceinline__ void score_list(const QLds& L, uint32_t n, const uint16_t* __restrict__ Bt, int rank,
                                           uint64_t& best) {
    auto at = [&](uint32_t c) -> uint64_t { return L.clist[c]; };
    for (uint32_t c0 = 0; c0 < n; c0 += 8u * kQPasses) score_passes(L, c0, n, Bt, rank, at, best);
}

// Bound on the norm of the key row this wave holds (lane l: entries 4l .. 4l+3): the
// square root of the sum of squares, times 1 + 2^-12 for the sum's rounding; the same
// value in every lane.
__device__ __forceinline__ float key_norm_up(const u32x2& key) {
    float s = 0.f;
#pragma unroll
    for (int d = 0; d < 2; ++d) {
        const float lo = __uint_as_float(key[d] << 16), hi = __uint_as_float(key[d] & 0xFFFF0000u);
        s = __builtin_fmaf(lo, lo, s);
        s = __builtin_fmaf(hi, hi, s);
    }
    // the sum over the wave, within rows of 16 by lane moves and then over the four rows
    s += dpp_f32(s, kDppXor1);
    s += dpp_f32(s, kDppXor2);
    s += dpp_f32(s, kDppHalfMirror);
    s += dpp_f32(s, kDppMirror);
    s = (__int_as_float(__builtin_amdgcn_readlane(__float_as_int(s), 0)) +
         __int_as_float(__builtin_amdgcn_readlane(__float_as_int(s), 16))) +
        (__int_as_float(__builtin_amdgcn_readlane(__float_as_int(s), 32)) +
         __int_as_float(__builtin_amdgcn_readlane(__float_as_int(s), 48)));
    return __builtin_sqrtf(s) * (1.0f + 0x1p-12f);
}

// The chain wave's work on request r (see the file comment).
__device__ __forceinline__ void chain_wave(const CandArgs& a, QLds& L, int r, float ab2, float b1, bool bound_ok) {
    const int lane = threadIdx.x & 63;
    const int K = a.K, NC = a.NC, V = a.V, rank = a.rank;
    const long row0 = (long)r * K;
    constexpr float kNegInf = -__builtin_huge_valf();
    int prev = a.prev0[r];
    if (prev < 0 || prev >= V) {
        if (lane == 0) raise_status(a.status, kStatusPrevClamped);
        prev = prev < 0 ? 0 : V - 1;
    }
    u32x2 key = row_quad(a.A, prev, rank);  // key row of the current position
    for (int i = 0; i < K; ++i) {
        // the row's items are all kept
        long n_polls = 0;
        while (__hip_atomic_load(&L.rowdone[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) < (uint32_t)NC) {
            if (++n_polls > kQSpinLimit) {
                if (lane == 0) raise_status(a.status, kStatusSyncTimeout);
                return;  // the rest of the request's tokens are left unwritten (the status says so)
            }
            __builtin_amdgcn_s_sleep(1);
        }
        asm volatile("" ::: "memory");
        // the row's kept groups: places [0, total) of its chunks, unless some found no chunk
        const bool over = L.rowover[i] != 0u;
        const uint32_t total = over ? 0u : L.rowfill[i];
        if (4 * lane < rank) *(u32x2*)(L.akey + 4 * lane) = key;  // this position's key row, for every lane
        wave_lds_sync();
        const uint32_t nk = L.rownan[i];
        const float M = unord32(L.rowmax[i]);
        // (a row of candidates always keeps its maximum; an empty one is scored densely all the same)
        int kind = nk ? 1 : (M == kNegInf ? 2 : ((!bound_ok || over || total == 0) ? 3 : 0));
        int tok = 0;  // (kind 2)
        u32x2 next_key{0u, 0u};
        bool have_next = false;
        if (kind == 1) {
            tok = (int)~nk;
        } else if (kind == 0) {
            // list the kept entries that clear the final floor, score them in lists of
            // at most kQList; note the largest (the likely token)
            // Once the position's key row is known, every bias is at most |key| b in size, so
            // the floor may use 2 |key| b1 where the streams had to use 2 a b (the lower wins).
            const float ab2_key = 2.0f * key_norm_up(key) * b1 * (1.0f + 0x1p-20f);
            const float fl = cand_floor(M, ab2_key < ab2 ? ab2_key : ab2);
            uint64_t best = 0ull, top = 0ull;
            uint32_t n = 0, ng = 0;
            // The groups whose maximum clears the floor, a lane per kept group and a chunk at
            // a time, are listed; then, a lane per listed group, their entries that clear it,
            // which are scored once more than 256 are listed.
            for (uint32_t e0 = 0; e0 < total; e0 += kQChunk) {
                const uint32_t slot = (L.ctab[i][e0 / kQChunk] % (uint32_t)kQChunks) * kQChunk + (uint32_t)lane;
                float gmx = kNegInf;
                if (e0 + (uint32_t)lane < total) {
                    const u32x4 g = L.grp[slot];
#pragma unroll
                    for (int d = 0; d < 4; ++d)
                        gmx = __builtin_elementwise_maximum(
                            gmx, __builtin_elementwise_maximum(__uint_as_float(g[d] << 16),
                                                               __uint_as_float(g[d] & 0xFFFF0000u)));
                }
                const bool pass = gmx >= fl;
                const uint64_t bal = __ballot(pass);
                if (pass) L.glist[ng + (uint32_t)__builtin_popcountll(bal & ((1ull << lane) - 1ull))] = (uint16_t)slot;
                ng += (uint32_t)__builtin_popcountll(bal);
                if (ng > (uint32_t)(kQGList - 64) || (e0 + kQChunk >= total && ng != 0u)) {
                    wave_lds_sync();
                    for (uint32_t b0 = 0; b0 < ng; b0 += 64) {
                        uint32_t mk = 0u, v = 0u;
                        u32x4 g{kNegInfPair, kNegInfPair, kNegInfPair, kNegInfPair};
                        if (b0 + (uint32_t)lane < ng) {
                            const uint32_t gs = L.glist[b0 + (uint32_t)lane];
                            g = L.grp[gs];
                            v = (uint32_t)L.gid[gs] * 8u;
#pragma unroll
                            for (int t = 0; t < 8; ++t) {
                                const uint32_t w = g[t >> 1];
                                mk |= __uint_as_float((t & 1) ? (w & 0xFFFF0000u) : (w << 16)) >= fl ? (1u << t) : 0u;
                            }
                        }
                        uint32_t cnt = 0;
                        uint32_t at = n + wave_excl_scan_small((uint32_t)__builtin_popcount(mk), &cnt);
                        while (mk != 0u) {
                            const int t = __builtin_ctz(mk);
                            mk &= mk - 1u;
                            const uint32_t w = g[t >> 1];
                            const uint32_t bits = (t & 1) ? (w & 0xFFFF0000u) : (w << 16);
                            L.clist[at++] = ((uint64_t)(v + (uint32_t)t) << 32) | bits;
                            top = umax64(top, argmax_key(__uint_as_float(bits), v + (uint32_t)t));
                        }
                        n += cnt;
                        if (n > (uint32_t)(kQList - 8 * 64) && (b0 + 64 < ng || e0 + kQChunk < total)) {
                            wave_lds_sync();
                            score_list(L, n, a.Bt, rank, best);
                            wave_lds_sync();
                            n = 0;
                        }
                    }
                    wave_lds_sync();
                    ng = 0;
                }
            }
            top = wave_max_u64(top);
            if (i + 1 < K && top != 0ull) {
                // the next position's key row, for the likely token, while the rest is scored
                next_key = row_quad(a.A, key_index(top), rank);
                have_next = true;
            }
            if (n != 0u) {
                wave_lds_sync();
                score_list(L, n, a.Bt, rank, best);
                wave_lds_sync();
            }
            best = wave_max_u64(best);
            // (the group of the row's maximum is always kept and listed; scored densely otherwise)
            if (best != 0ull) tok = key_index(best);
            else kind = 3;
            have_next = have_next && best != 0ull && key_index(top) == tok;
        }
        if (kind == 3) tok = key_index(dense_row(L, a.base + (size_t)(row0 + i) * (size_t)V, V, a.Bt, rank));
        wave_lds_sync();  // L.akey is read before the next position's key row is written
        if (lane == 0) a.tokens[row0 + i] = tok;
        if (i + 1 < K) key = have_next ? next_key : row_quad(a.A, tok, rank);
    }
}

// The request's LDS state before its first item.
__device__ __forceinline__ void reset_request(QLds& L, int K) {
    if ((int)threadIdx.x < K) {
        L.rowmax[threadIdx.x] = 0u;
        L.rownan[threadIdx.x] = 0u;
        L.rowdone[threadIdx.x] = 0u;
        L.rowfill[threadIdx.x] = 0u;
        L.rowover[threadIdx.x] = 0u;
    }
    for (int t = (int)threadIdx.x; t < K * kQChunks / 4; t += kQT) reinterpret_cast<uint32_t*>(L.ctab)[t] = 0xFFFFFFFFu;
    if (threadIdx.x == 0) {
        L.next = 0u;
        L.pool = 0u;
    }
}

__device__ __forceinline__ void run_chain(const CandArgs& a, QLds& L, int r, const HeaderView& hv) {
    // the chain is the request's critical path: its wave goes first on its SIMD
    __builtin_amdgcn_s_setprio(3);
    chain_wave(a, L, r, hv.ab2, hv.b1, hv.ok);
    __builtin_amdgcn_s_setprio(0);
}

// Stage 1 in one launch.  S = 1: workgroup g takes requests g, g + G, ...  S > 1: the
// first R (S - 1) workgroups are the helpers (dispatched first, and they never wait for
// another workgroup), the last R the owners.  The launch's epoch is one more than the
// workspace's; the last workgroup to finish stores it there for the next launch.
template <bool VEC, int LOADS>
__global__ __launch_bounds__(kQT, 1) void cand_chain_kernel(CandArgs a) {
    __shared__ QLds S;
    const HeaderView hv = header_view(a.hdr);
    if (a.S > 1) {
        __shared__ uint32_t ep_lds;
        const int nh = a.R * (a.S - 1);
        const int b = (int)blockIdx.x;
        const bool helper = b < nh;
        const int r = helper ? b / (a.S - 1) : b - nh;
        const int s = helper ? 1 + b % (a.S - 1) : 0;
        if (threadIdx.x == 0)
            ep_lds = __hip_atomic_load(&a.split_ctl[0], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + 1u;
        reset_request(S, a.K);
        __syncthreads();
        const uint32_t ep = ep_lds;
        if (helper)
            stream_tasks<VEC, 1, LOADS>(S, a, r, s, hv.ab2, ep);
        else if ((int)(threadIdx.x >> 6) < kQS)
            stream_tasks<VEC, 2, LOADS>(S, a, r, 0, hv.ab2, ep);
        else
            run_chain(a, S, r, hv);
        __syncthreads();
        if (threadIdx.x == 0 && atomicInc(&a.split_ctl[1], gridDim.x - 1u) == gridDim.x - 1u)
            __hip_atomic_store(&a.split_ctl[0], ep, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        return;
    }
    for (int r = blockIdx.x; r < a.R; r += (int)gridDim.x) {
        reset_request(S, a.K);
        __syncthreads();
        if ((int)(threadIdx.x >> 6) < kQS)
            stream_tasks<VEC, 0, LOADS>(S, a, r, 0, hv.ab2, 0u);
        else
            run_chain(a, S, r, hv);
        __syncthreads();  // the request's LDS is read before the next one is streamed into it
    }
}

__global__ void markov_norms_kernel(const uint16_t* __restrict__ A, const uint16_t* __restrict__ Bt, int V, int rank,
                                    uint64_t* hdr) {
    const int v = blockIdx.x * blockDim.x + threadIdx.x;
    if (v >= V) return;
    double sa = 0.0, sb = 0.0;
    for (int k = 0; k < rank; ++k) {
        const double x = (double)bf16_bits_to_f32(A[(size_t)v * rank + k]);
        const double y = (double)bf16_bits_to_f32(Bt[(size_t)v * rank + k]);
        sa += x * x;
        sb += y * y;
    }
    // non-negative doubles (and NaN, above +inf) order as their bit patterns
    atomicMax((unsigned long long*)&hdr[0], (unsigned long long)__double_as_longlong(sa));
    atomicMax((unsigned long long*)&hdr[1], (unsigned long long)__double_as_longlong(sb));
}

__global__ void markov_bound_kernel(uint64_t* hdr) {
    const double a2 = __longlong_as_double((long long)hdr[0]), b2 = __longlong_as_double((long long)hdr[1]);
    const double ab2 = 2.0 * __builtin_sqrt(a2) * __builtin_sqrt(b2) * (1.0 + 0x1p-10);
    float* f = reinterpret_cast<float*>(&hdr[2]);
    const bool ok = ab2 == ab2 && ab2 < 1e30;
    f[0] = ok ? __double2float_ru(ab2) : 0.f;
    reinterpret_cast<uint32_t*>(&hdr[2])[1] = ok ? 1u : 0u;
    f[2] = ok ? __double2float_ru(__builtin_sqrt(b2) * (1.0 + 0x1p-10)) : 0.f;
}

__global__ void zero_u64_kernel(uint64_t* p, int n) {
    const int t = blockIdx.x * blockDim.x + threadIdx.x;
    if (t < n) p[t] = 0ull;
}

}  // namespace

hipError_t launch_markov_bound(const void* A, const void* Bt, int V, int rank, void* hdr, hipStream_t s) {
    zero_u64_kernel<<<1, 64, 0, s>>>((uint64_t*)hdr, 4);
    markov_norms_kernel<<<(V + 255) / 256, 256, 0, s>>>((const uint16_t*)A, (const uint16_t*)Bt, V, rank,
                                                       (uint64_t*)hdr);
    markov_bound_kernel<<<1, 1, 0, s>>>((uint64_t*)hdr);
    return hipGetLastError();
}

hipError_t launch_cand(const CandArgs& a, int num_cu, hipStream_t s, hipEvent_t start, hipEvent_t stop) {
    // one workgroup per compute unit, at most one per request, or S per request
    int grid = num_cu < kCandMaxGroups ? num_cu : kCandMaxGroups;
    if (grid > a.R) grid = a.R;
    if (a.S > 1) grid = a.R * a.S;
    CandArgs arg = a;
    void* args[] = {&arg};
    // 16-byte loads of the base logits need 8 | V and an aligned base
    const bool vec = a.V % 8 == 0 && ((uintptr_t)a.base & 15u) == 0;
    if (a.item != kCandItemLong && a.item != kCandItemShort) return hipErrorInvalidValue;
    const bool lng = a.item == kCandItemLong;
    const void* fn = vec ? (lng ? (const void*)cand_chain_kernel<true, 8> : (const void*)cand_chain_kernel<true, 4>)
                         : (lng ? (const void*)cand_chain_kernel<false, 8> : (const void*)cand_chain_kernel<false, 4>);
    if (start || stop) return hipExtLaunchKernel(fn, dim3(grid), dim3(kQT), args, 0, s, start, stop, 0);
    return hipLaunchKernel(fn, dim3(grid), dim3(kQT), args, 0, s);
}

}  // namespace dspark
