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
// depend on the previous token.  So a request splits into
//   1. one streaming pass over its base logits -- all of the stage's HBM traffic, with no
//      dependence between positions -- that keeps, per (request, position) row, its
//      maximum and its candidates (index and value), and
//   2. the chain over the candidates alone: the bias is evaluated for a few tens of
//      entries per position instead of V.
// The bound is applied with a margin (2ab(1 + 2^-10), plus 2^-20 |M| for the rounding of
// the subtraction), so the candidate set always contains the exact (real-number, and
// hence the double-precision) argmax.  Among the candidates the kernel takes the float32
// argmax of fl32(base + fl32 dot).  Where the bound cannot prune, the row is scored over
// the whole vocabulary, so the result never depends on the data: a NaN in the row makes
// the first NaN the token (the bias is finite whenever the bound is, so x is NaN exactly
// where base is); a row of -inf gives 0; a row whose candidates overflow a buffer, or
// weights whose bound is not finite, are scored densely.
//
// One workgroup per compute unit; workgroup g takes requests g, g + G, ... whole, so a
// request's candidates never leave the compute unit's LDS.
//
// Streaming.  A request's K*V base entries are items of 4096 entries (a row is
// ceil(V/4096) items), streamed in rounds: in round t wave w takes item 16t + w, with the
// next round's loads in flight.  Each wave folds its item's maximum into the row's
// maximum in LDS; after a barrier every wave keeps the entries of its item that clear
// the floor of the row's maximum so far (a lower bound of the final one, so nothing that
// can win is dropped; the 16 items of a round already give a floor close to the final).
// Candidates and one directory word per item stay in the wave's part of the LDS.
//
// Chain.  Once the request is streamed its 1024 threads (a) read the rows' maxima and
// NaN marks, (b) keep the candidates that clear each row's final floor, in one LDS list,
// (c) put each listed candidate's Bt row in registers or LDS (8 threads per candidate,
// 32 rank entries each) and the key rows each position most likely needs: prev0 for
// position 0 and, for position i > 0, row i-1's largest base entry (its token unless the
// bias reorders the top), (d) score every position with that key row, all at once, and
// (e) walk the positions: where the previous token is the one guessed, the scored token
// stands; otherwise that position is scored again with the right key row.
#include "common.h"
#include "kernels.h"

namespace dspark {

namespace {

constexpr int kQT = 1024;               // threads per workgroup
constexpr int kQW = kQT / 64;           // waves per workgroup
constexpr int kQItem = kCandItem;       // base entries per item: 64 lanes x 8 loads x 8 entries
constexpr int kQStage = kCandWaveStage; // candidates a wave keeps for its items of one request
constexpr int kQRegCands = kQT / 8;     // listed candidates whose Bt slices sit in registers (one per 8 threads)
constexpr int kQLdsCands = 128;         // the next ones, whose Bt rows are staged in LDS
constexpr uint32_t kQOverflow = 0xFFFFFFFFu;
constexpr uint32_t kNegInfPair = 0xFF80FF80u;  // two bf16 -inf

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

static_assert(kCandMaxK * kCandMaxItems <= 2048, "a request's directory fits the LDS array");
static_assert(kQW * kQStage < (1 << 16), "LDS slots fit the directory word");

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

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) x = __builtin_elementwise_maximum(x, __shfl_xor(x, o, 64));
    return x;
}

__device__ __forceinline__ uint32_t wave_min_u32(uint32_t x) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
        const uint32_t y = __shfl_xor(x, o, 64);
        x = y < x ? y : x;
    }
    return x;
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t x) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) x = umax64(x, shfl_xor_u64(x, o));
    return x;
}

// Exclusive prefix sum over the wave; *total receives the sum.
__device__ __forceinline__ uint32_t wave_excl_scan(uint32_t v, uint32_t* total) {
    const int lane = threadIdx.x & 63;
    uint32_t x = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const uint32_t y = __shfl_up(x, o, 64);
        if (lane >= o) x += y;
    }
    *total = __shfl(x, 63, 64);
    return x - v;
}

// LDS written by some lanes of a wave and read by others: the writes come first.
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// The prepared head's bound: ab2 = 2 a b (1 + 2^-10) rounded up, ok = it is finite.
struct HeaderView {
    float ab2;
    bool ok;
};

__device__ __forceinline__ HeaderView header_view(const void* hdr) {
    const uint32_t* h = (const uint32_t*)hdr;
    return HeaderView{__uint_as_float(h[4]), h[5] != 0u};
}

// LDS of one request.
struct QLds {
    uint64_t stage[kQW * kQStage];   // candidates, wave w's in [w kQStage, (w + 1) kQStage): (index << 32) | value bits
    uint64_t dir[kCandMaxK * kCandMaxItems];  // per item: (first slot << 32) | count (kQOverflow: no room);
                                     // from (b) on (first slot << 32) | the row's prefix
    uint64_t flat[kCandListCap];     // the rows' candidate lists, concatenated
    uint16_t btrow[kQLdsCands][256]; // Bt rows of listed candidates kQRegCands ..
    uint16_t arow[kCandMaxK][256];   // key rows (bf16): the one guessed for each position
    uint16_t fix[256];               // key row of a re-scored position
    uint64_t best[kCandMaxK];        // per-position argmax key (LDS atomic max)
    uint64_t dbest;                  // a whole-row scoring's key
    uint32_t rowmax[kCandMaxK];      // the rows' maxima so far (order-preserving image; 0 = none yet)
    uint32_t rownan[kCandMaxK];      // ~(first NaN index), 0 = none
    int32_t rowstart[kCandMaxK];     // listed candidates of row i: flat[rowstart[i] ..] (rowcnt[i] of them)
    int32_t rowcnt[kCandMaxK];
    int32_t npool[kCandMaxK];        // the row's kept entries before the final floor
    int32_t kind[kCandMaxK];         // 0 listed candidates, 1 first NaN, 2 all -inf, 3 dense, 4 candidates
                                     // scored from the kept entries (more than the list holds)
    int32_t nanidx[kCandMaxK];
    float floor_[kCandMaxK];
    int32_t top[kCandMaxK];          // the row's largest candidate (lowest index among equals)
    int32_t guess[kCandMaxK];        // key token row i was scored with
    int32_t tok[kCandMaxK];
    uint8_t frow[kCandListCap];      // row of each listed candidate
    int32_t ntot;
};

// ---------------------------------------------------------------------------------
// Streaming

// Entries [v0, v0 + 4096) of a row into buf (8 groups of 8 entries per lane; entries past
// V read as -inf).  VEC: 8 | V and an aligned base, so groups are 16-byte aligned and
// wholly in or out of the row.
template <bool VEC>
__device__ __forceinline__ void load_item(u32x4 (&buf)[8], const uint16_t* __restrict__ p, int v0, int V) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
        const int e = v0 + q * 512 + lane * 8;
        if (VEC) {
            buf[q] = e < V ? __builtin_nontemporal_load((const u32x4*)(p + e))
                           : u32x4{kNegInfPair, kNegInfPair, kNegInfPair, kNegInfPair};
        } else {
            uint32_t h[8];
#pragma unroll
            for (int t = 0; t < 8; ++t) h[t] = e + t < V ? (uint32_t)p[e + t] : 0xFF80u;
            buf[q] = u32x4{h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16)};
        }
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

// Streams request r (see the file comment): the rows' maxima and NaN marks, and each
// item's candidates with its directory word, into L.
template <bool VEC>
__device__ __forceinline__ void stream_request(const CandArgs& a, QLds& L, int r, float ab2) {
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
    const int K = a.K, NC = a.NC, V = a.V;
    const int per_req = K * NC;
    const int n_rounds = (per_req + kQW - 1) / kQW;
    const uint16_t* rbase = a.base + (size_t)r * (size_t)K * (size_t)V;
    constexpr float kNegInf = -__builtin_huge_valf();
    if (tid < K) {
        L.rowmax[tid] = 0u;
        L.rownan[tid] = 0u;
    }
    __syncthreads();
    uint32_t used = 0;  // candidates this wave keeps so far
    u32x4 cur[8], nxt[8];
    if (w < per_req) load_item<VEC>(nxt, rbase + (size_t)(w / NC) * V, (w % NC) * kQItem, V);
    for (int t = 0; t < n_rounds; ++t) {
        const int jl = t * kQW + w;  // the item of the request this wave takes
        const bool valid = jl < per_req;
        const int i = valid ? jl / NC : 0;
        const int v0 = valid ? (jl - i * NC) * kQItem : 0;
#pragma unroll
        for (int q = 0; q < 8; ++q) cur[q] = nxt[q];
        const int jn = jl + kQW;
        if (jn < per_req) load_item<VEC>(nxt, rbase + (size_t)(jn / NC) * V, (jn % NC) * kQItem, V);
        // the item's 8-entry group maxima and its maximum; a NaN marks the row at once
        float gm[8];
        bool nan_item = false;
        if (valid) {
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                float g = kNegInf;
#pragma unroll
                for (int d = 0; d < 4; ++d) {
                    const uint32_t x = cur[q][d];
                    g = __builtin_elementwise_maximum(
                        g, __builtin_elementwise_maximum(__uint_as_float(x << 16), __uint_as_float(x & 0xFFFF0000u)));
                }
                gm[q] = g;
            }
            float m = gm[0];
#pragma unroll
            for (int q = 1; q < 8; ++q) m = __builtin_elementwise_maximum(m, gm[q]);
            const float mw = wave_max(m);
            if (mw != mw) {
                // the row's token is its first NaN, whatever the bias
                nan_item = true;
                uint32_t first = 0xFFFFFFFFu;
#pragma unroll
                for (int q = 7; q >= 0; --q) {
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
            } else if (lane == 0) {
                atomicMax(&L.rowmax[i], ord32(mw));
            }
        }
        __syncthreads();  // the round's maxima are in
        if (valid) {
            uint32_t count = 0;
            const uint32_t first_slot = (uint32_t)(w * kQStage) + used;
            if (!nan_item) {
                const float fl = cand_floor(unord32(L.rowmax[i]), ab2);
                // -inf never wins unless the whole row is -inf, which the chain handles apart
                bool any = false;
#pragma unroll
                for (int q = 0; q < 8; ++q) any |= gm[q] >= fl && gm[q] > kNegInf;
                if (__ballot(any) != 0ull) {
                    uint32_t c = 0;
#pragma unroll
                    for (int q = 0; q < 8; ++q) {
                        if (gm[q] >= fl && gm[q] > kNegInf) {
#pragma unroll
                            for (int s = 0; s < 8; ++s) {
                                const float x = entry_of(cur[q], s);
                                c += (x >= fl && x > kNegInf) ? 1u : 0u;
                            }
                        }
                    }
                    uint32_t total = 0;
                    uint32_t slot = first_slot + wave_excl_scan(c, &total);
                    if (used + total <= (uint32_t)kQStage) {
#pragma unroll
                        for (int q = 0; q < 8; ++q) {
                            if (gm[q] >= fl && gm[q] > kNegInf) {
#pragma unroll
                                for (int s = 0; s < 8; ++s) {
                                    const float x = entry_of(cur[q], s);
                                    if (x >= fl && x > kNegInf) {
                                        const uint32_t v = (uint32_t)(v0 + q * 512 + lane * 8 + s);
                                        L.stage[slot++] = ((uint64_t)v << 32) | __float_as_uint(x);
                                    }
                                }
                            }
                        }
                        count = total;
                        used += total;
                    } else {
                        count = kQOverflow;  // no room: the row is scored densely
                    }
                }
            }
            if (lane == 0) L.dir[jl] = ((uint64_t)first_slot << 32) | count;
        }
    }
    __syncthreads();
}

// ---------------------------------------------------------------------------------
// Chain

// x for a candidate scored with key row `arow` (LDS, bf16): the 8 threads of a candidate
// each take 32 rank entries (slice s = lane % 8, held in `bt`), fused multiply-adds in
// increasing k, then a butterfly over the 8 threads (every one ends with the same sum);
// x = fl32(value + dot).
__device__ __forceinline__ float cand_x(const u32x4 (&bt)[4], const uint16_t* arow, int rank, float value) {
    const int s = threadIdx.x & 7;
    float acc = 0.f;
    if (32 * s < rank) {
        const u32x4* ap = (const u32x4*)(arow + 32 * s);
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const u32x4 av = ap[g];
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                acc = __builtin_fmaf(__uint_as_float(av[d] << 16), __uint_as_float(bt[g][d] << 16), acc);
                acc = __builtin_fmaf(__uint_as_float(av[d] & 0xFFFF0000u), __uint_as_float(bt[g][d] & 0xFFFF0000u),
                                     acc);
            }
        }
    }
    acc += __shfl_xor(acc, 1, 64);
    acc += __shfl_xor(acc, 2, 64);
    acc += __shfl_xor(acc, 4, 64);
    return value + acc;
}

__device__ __forceinline__ void load_bt_slice(u32x4 (&bt)[4], const uint16_t* __restrict__ Bt, int c, int rank) {
    const int s = threadIdx.x & 7;
    if (32 * s < rank) {
        const u32x4* p = (const u32x4*)(Bt + (size_t)c * rank + 32 * s);
#pragma unroll
        for (int g = 0; g < 4; ++g) bt[g] = p[g];
    } else {
#pragma unroll
        for (int g = 0; g < 4; ++g) bt[g] = u32x4{0u, 0u, 0u, 0u};
    }
}

// A key row into LDS (threads [t0, t0 + rank/8) load 16 bytes each).
__device__ __forceinline__ void key_row_to_lds(uint16_t* dst, const uint16_t* __restrict__ A, int u, int rank, int t0) {
    const int t = (int)threadIdx.x - t0;
    if (t >= 0 && t < rank / 8) ((u32x4*)dst)[t] = ((const u32x4*)(A + (size_t)u * rank))[t];
}

// Entry e of row i's kept entries, through the row's (first slot, prefix) directory: the
// item holding it is the last with prefix <= e.
__device__ __forceinline__ uint64_t kept_entry(const QLds& L, int i, int NC, uint32_t e) {
    int lo = 0, hi = NC - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if ((uint32_t)L.dir[i * NC + mid] <= e) lo = mid;
        else hi = mid - 1;
    }
    const uint64_t d = L.dir[i * NC + lo];
    return L.stage[(uint32_t)(d >> 32) + (e - (uint32_t)d)];
}

// Row `row` scored over the whole vocabulary with key row L.fix: the exact argmax (every
// entry) for rows the bound does not prune.
__device__ __forceinline__ int dense_row(const CandArgs& a, QLds& L, long row) {
    const uint16_t* bp = a.base + (size_t)row * (size_t)a.V;
    if (threadIdx.x == 0) L.dbest = 0ull;
    __syncthreads();
    uint64_t best = 0ull;
    for (int v0 = 0; v0 < a.V; v0 += kQT / 8) {
        const int v = v0 + (int)(threadIdx.x >> 3);
        u32x4 bt[4];
        load_bt_slice(bt, a.Bt, v < a.V ? v : 0, a.rank);
        const float value = __uint_as_float((uint32_t)bp[v < a.V ? v : 0] << 16);
        const float x = cand_x(bt, L.fix, a.rank, value);
        if (v < a.V && (threadIdx.x & 7) == 0) best = umax64(best, argmax_key(x, (uint32_t)v));
    }
    best = wave_max_u64(best);
    if ((threadIdx.x & 63) == 0) atomicMax((unsigned long long*)&L.dbest, (unsigned long long)best);
    __syncthreads();
    const int tok = key_index(L.dbest);
    __syncthreads();
    return tok;
}

// Row i's kept entries that clear its floor (rows with more candidates than the list
// holds), scored with key row `arow`, into L.best[i].
__device__ __forceinline__ void score_row_kept(const CandArgs& a, QLds& L, int i, int NC, const uint16_t* arow) {
    const int n = L.npool[i];
    const float fl = L.floor_[i];
    for (int j0 = 0; j0 < n; j0 += kQT / 8) {
        const int j = j0 + (int)(threadIdx.x >> 3);
        const uint64_t e = j < n ? kept_entry(L, i, NC, (uint32_t)j) : 0ull;
        const float value = __uint_as_float((uint32_t)e);
        u32x4 b[4];
        load_bt_slice(b, a.Bt, (int)(e >> 32), a.rank);
        const float x = cand_x(b, arow, a.rank, value);
        if (j < n && value >= fl && (threadIdx.x & 7) == 0)
            atomicMax((unsigned long long*)&L.best[i], (unsigned long long)argmax_key(x, (uint32_t)(e >> 32)));
    }
}

// Scores listed candidates with key rows from LDS and raises each row's key in L.best.
// only < 0: every listed candidate, with its own row's guessed key row; only = i: the
// candidates of row i alone, with L.fix.  Candidate j's Bt slice comes from this
// thread's registers (j < kQRegCands: `bt`), from LDS (the next kQLdsCands) or from
// global memory (the rest).
__device__ __forceinline__ void score_pass(const CandArgs& a, QLds& L, const u32x4 (&bt)[4], int N, int only) {
    const int tid = threadIdx.x, g = tid >> 3, s = tid & 7;
    auto score = [&](const u32x4 (&b)[4], int j) {
        const bool in = j < N;
        const int i = in ? L.frow[j] : 0;
        const uint64_t e = in ? L.flat[j] : 0ull;
        const bool live = in && (only < 0 || i == only);
        const float x = cand_x(b, only < 0 ? L.arow[i] : L.fix, a.rank, __uint_as_float((uint32_t)e));
        if (live && s == 0)
            atomicMax((unsigned long long*)&L.best[i], (unsigned long long)argmax_key(x, (uint32_t)(e >> 32)));
    };
    score(bt, g);
    if (kQRegCands < N) {
        const int j = kQRegCands + g;  // kQLdsCands == kQT / 8: one LDS candidate per 8 threads
        u32x4 b[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) b[q] = ((const u32x4*)(L.btrow[g] + 32 * s))[q];
        score(b, j);
    }
    for (int j0 = kQRegCands + kQLdsCands; j0 < N; j0 += kQT / 8) {
        const int j = j0 + g;
        u32x4 b[4];
        load_bt_slice(b, a.Bt, j < N ? (int)(L.flat[j] >> 32) : 0, a.rank);
        score(b, j);
    }
}

// The chain of request r, streamed into L (see the file comment).
__device__ __forceinline__ void chain_request(const CandArgs& a, QLds& L, int r, float ab2, bool bound_ok) {
    const int K = a.K, NC = a.NC, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const long row0 = (long)r * K;
    // (a) the rows' kinds and final floors
    if (tid < K) {
        const uint32_t nk = L.rownan[tid];
        const float M = unord32(L.rowmax[tid]);
        L.nanidx[tid] = (int)~nk;
        L.kind[tid] = nk ? 1 : (M == -__builtin_huge_valf() ? 2 : (bound_ok ? 0 : 3));
        L.floor_[tid] = cand_floor(M, ab2);
        L.best[tid] = 0ull;
    }
    if (tid == 0) {
        int p = a.prev0[r];
        if (p < 0 || p >= a.V) {
            raise_status(a.status, kStatusPrevClamped);
            p = p < 0 ? 0 : a.V - 1;
        }
        L.guess[0] = p;
    }
    __syncthreads();
    // (b) per row (one wave each): the items' counts and their prefix, then the kept
    // entries that clear the row's final floor: how many, and the largest (lowest index
    // among equals)
    for (int i = w; i < K; i += kQW) {
        uint32_t cnt = 0, start = 0;
        bool over = false;
        if (lane < NC) {
            const uint64_t d = L.dir[i * NC + lane];
            cnt = (uint32_t)d;
            start = (uint32_t)(d >> 32);
            over = cnt == kQOverflow;
        }
        const bool any_over = __ballot(over) != 0ull;
        if (any_over) cnt = 0;
        uint32_t total = 0;
        const uint32_t pre = wave_excl_scan(cnt, &total);
        if (lane < NC) L.dir[i * NC + lane] = ((uint64_t)start << 32) | pre;
        wave_lds_sync();
        const bool use = L.kind[i] == 0 && !any_over;
        const float fl = L.floor_[i];
        uint32_t kept = 0, best_u = 0, best_v = 0xFFFFFFFFu;
        for (uint32_t e0 = 0; use && e0 < total; e0 += 64) {
            const uint32_t e = e0 + lane;
            const uint64_t ent = e < total ? kept_entry(L, i, NC, e) : 0ull;
            const bool ok = e < total && __uint_as_float((uint32_t)ent) >= fl;
            if (ok) {
                const uint32_t u = ord32(__uint_as_float((uint32_t)ent)), v = (uint32_t)(ent >> 32);
                if (u > best_u || (u == best_u && v < best_v)) {
                    best_u = u;
                    best_v = v;
                }
            }
            kept += (uint32_t)__builtin_popcountll(__ballot(ok));
        }
        uint64_t k = best_u ? (((uint64_t)best_u << 32) | (uint64_t)(~best_v)) : 0ull;
        k = wave_max_u64(k);
        if (lane == 0) {
            // overflowed buffers mean lost candidates: the row is scored densely
            if (L.kind[i] == 0 && any_over) L.kind[i] = 3;
            if (L.kind[i] == 0 && kept == 0) L.kind[i] = 3;  // cannot occur: its maximum clears the floor
            L.rowcnt[i] = L.kind[i] == 0 ? (int)kept : 0;
            L.npool[i] = L.kind[i] == 0 ? (int)total : 0;
            // the token row i most likely gets: its largest candidate, its first NaN, or 0
            L.top[i] = L.kind[i] == 1 ? L.nanidx[i] : (L.kind[i] == 0 ? key_index(k) : 0);
        }
    }
    __syncthreads();
    // the rows' lists in one LDS list (a row that does not fit is scored from its kept
    // entries), and the key rows guessed for each position
    if (tid == 0) {
        int acc = 0;
        for (int i = 0; i < K; ++i) {
            if (L.kind[i] == 0 && acc + L.rowcnt[i] > kCandListCap) L.kind[i] = 4;
            L.rowstart[i] = acc;
            if (L.kind[i] == 0) acc += L.rowcnt[i];
        }
        L.ntot = acc;
    }
    if (tid > 0 && tid < K) L.guess[tid] = L.top[tid - 1];
    __syncthreads();
    for (int i = w; i < K; i += kQW) {
        if (L.kind[i] != 0) continue;
        const uint32_t n_kept = (uint32_t)L.npool[i];
        const float fl = L.floor_[i];
        uint32_t placed = (uint32_t)L.rowstart[i];
        for (uint32_t e0 = 0; e0 < n_kept; e0 += 64) {
            const uint32_t e = e0 + lane;
            const uint64_t ent = e < n_kept ? kept_entry(L, i, NC, e) : 0ull;
            const bool ok = e < n_kept && __uint_as_float((uint32_t)ent) >= fl;
            const uint64_t bal = __ballot(ok);
            if (ok) {
                const uint32_t at = placed + (uint32_t)__builtin_popcountll(bal & ((1ull << lane) - 1ull));
                L.flat[at] = ent;
                L.frow[at] = (uint8_t)i;
            }
            placed += (uint32_t)__builtin_popcountll(bal);
        }
    }
    __syncthreads();
    const int N = L.ntot;
    // (c) the listed candidates' Bt slices (registers, then LDS) and the guessed key rows
    u32x4 bt[4];
    load_bt_slice(bt, a.Bt, (tid >> 3) < N ? (int)(L.flat[tid >> 3] >> 32) : 0, a.rank);
    {
        const int j = kQRegCands + (tid >> 3);
        if (j < N && j < kQRegCands + kQLdsCands) {
            u32x4 b1[4];
            load_bt_slice(b1, a.Bt, (int)(L.flat[j] >> 32), a.rank);
#pragma unroll
            for (int q = 0; q < 4; ++q) ((u32x4*)(L.btrow[j - kQRegCands] + 32 * (tid & 7)))[q] = b1[q];
        }
    }
    for (int i = 0; i < K; ++i) key_row_to_lds(L.arow[i], a.A, L.guess[i], a.rank, i * 32);
    __syncthreads();
    // (d) every position scored with its guessed key row
    score_pass(a, L, bt, N, -1);
    for (int i = 0; i < K; ++i)
        if (L.kind[i] == 4) score_row_kept(a, L, i, NC, L.arow[i]);
    __syncthreads();
    // (e) the walk
    int prev = L.guess[0];
    for (int i = 0; i < K; ++i) {
        const int kind = L.kind[i];
        int tok;
        if (kind == 1) {
            tok = L.nanidx[i];
        } else if (kind == 2) {
            tok = 0;
        } else if ((kind == 0 || kind == 4) && prev == L.guess[i]) {
            tok = key_index(L.best[i]);
        } else {
            // the guess missed, or the row is scored densely: row i with prev's key row
            key_row_to_lds(L.fix, a.A, prev, a.rank, 0);
            if (tid == 0) L.best[i] = 0ull;
            __syncthreads();
            if (kind == 3) {
                tok = dense_row(a, L, row0 + i);
            } else {
                if (kind == 0) score_pass(a, L, bt, N, i);
                else score_row_kept(a, L, i, NC, L.fix);
                __syncthreads();
                tok = key_index(L.best[i]);
            }
            __syncthreads();  // L.fix and L.best[i] are read before the next re-score
        }
        if (tid == 0) L.tok[i] = tok;
        prev = tok;
    }
    __syncthreads();
    if (tid < K) a.tokens[row0 + tid] = L.tok[tid];
}

// Stage 1 in one launch: workgroup g streams and chains requests g, g + G, ...
template <bool VEC>
__global__ __launch_bounds__(kQT, 1) void cand_chain_kernel(CandArgs a) {
    __shared__ QLds S;
    const HeaderView hv = header_view(a.hdr);
    for (int r = blockIdx.x; r < a.R; r += (int)gridDim.x) {
        stream_request<VEC>(a, S, r, hv.ab2);
        chain_request(a, S, r, hv.ab2, hv.ok);
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

hipError_t launch_cand(const CandArgs& a, int num_cu, hipStream_t s) {
    // one workgroup per compute unit, at most one per request
    int grid = num_cu < kCandMaxGroups ? num_cu : kCandMaxGroups;
    if (grid > a.R) grid = a.R;
    CandArgs arg = a;
    void* args[] = {&arg};
    // 16-byte loads of the base logits need 8 | V and an aligned base
    const bool vec = a.V % 8 == 0 && ((uintptr_t)a.base & 15u) == 0;
    const void* fn = vec ? (const void*)cand_chain_kernel<true> : (const void*)cand_chain_kernel<false>;
    return hipLaunchKernel(fn, dim3(grid), dim3(kQT), args, 0, s);
}

}  // namespace dspark
