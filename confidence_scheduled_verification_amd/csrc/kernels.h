// Internal launchers of libdspark (not part of the C ABI).  Each enqueues on the
// given stream and returns the launch status; argument checks happen in api.hip.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

namespace dspark {

// Workspace layout, each region 256-byte aligned:
//   [0, ws_sync_bytes)   the single-launch step kernel's counters [K][kMaxGroups] and
//                        ready flag (uint32), sized for the largest K so that the region
//                        does not move with the shape;
//   then ws_wide_bytes   the many-workgroup schedule's per-workgroup results and the
//                        slots' ranks (fixed size, written before they are read);
//   then ws_split_ctl_bytes  the pruned chain's split of requests over workgroups: its
//                        launch epoch and finished-workgroup counter, then one 16-byte
//                        header per (helper workgroup, row) whose first word is an epoch
//                        (fixed size, so each word keeps its role whatever the shape);
//   then                 the per-position argmax keys [K][R] (uint64) and the
//                        persistent chain kernel's barrier counters [K][kMaxGroups];
//   then (optional)      the helpers' kept groups, ws_split_dat_bytes (cand.hip).
// The stage-wise paths zero the keys and counters they use first.  The step kernel
// zeroes its keys in-launch and puts its counters and flag back to zero when it ends,
// so once the workspace was zero-filled one time they are zero at every launch,
// whatever R and K the earlier calls had.
#ifndef DSPARK_GROUPS
#define DSPARK_GROUPS 2
#endif
constexpr int kMaxGroups = DSPARK_GROUPS;  // request groups of the persistent chain, out of phase
constexpr int kMaxSlotsWs = 16384;
inline size_t ws_round(size_t x) { return (x + 255) / 256 * 256; }
inline size_t ws_sync_bytes() { return ws_round((size_t)(kMaxSlotsWs * kMaxGroups + 1) * 4); }
inline size_t ws_keys_bytes(int R, int K) { return ws_round((size_t)R * (size_t)K * 8); }
inline size_t ws_bar_bytes(int K) { return ws_round((size_t)K * kMaxGroups * 4); }
// Keys and chain counters: what the stage-wise paths clear.
inline size_t ws_chain_bytes(int R, int K) { return ws_keys_bytes(R, K) + ws_bar_bytes(K); }
// The many-workgroup schedule (sched.hip): up to kWideMaxN slots, kWideSlots per workgroup.
constexpr int kWideMaxN = 2048;
constexpr int kWideSlots = 8;
constexpr int kWideMaxGroups = kWideMaxN / kWideSlots;
constexpr size_t kWidePartialBytes = 48;  // one workgroup's result
inline size_t ws_wide_off() { return ws_sync_bytes(); }
inline size_t ws_wide_bytes() { return ws_round((size_t)kWideMaxGroups * kWidePartialBytes + (size_t)kWideMaxN * 4); }
inline size_t ws_split_ctl_off() { return ws_sync_bytes() + ws_wide_bytes(); }
inline size_t ws_split_ctl_bytes();  // defined with the pruned chain's constants below
inline size_t ws_chain_off() { return ws_split_ctl_off() + ws_split_ctl_bytes(); }
inline size_t ws_total_bytes(int R, int K) { return ws_chain_off() + ws_chain_bytes(R, K); }

// Probabilistic drafting: Gumbel-max sampling of softmax(x / temperature) with
// Philox4x32-10 random numbers keyed on the 64-bit seed (k0 low word, k1 high word).
struct SampleArgs {
    int on;
    uint32_t k0, k1;
    float scale;  // log2(e) / temperature
};

struct ChainArgs {
    const void* base;
    const void* A;
    const void* Bt;
    int dtype;  // 0 fp32, 1 bf16
    const int32_t* prev0;
    int R, K, V, rank;
    int32_t* tokens;
    float* logits;
    uint32_t* status;
    uint64_t* keys;  // [K, R] per-position argmax keys, zeroed before the first position
    uint32_t* bar;   // [K, kMaxGroups] barrier counters, zeroed before the first position
    SampleArgs smp;  // off unless the tokens are sampled
    int coop;        // persistent kernel: cooperative launch (1) or plain launch of a resident grid (0)
};

// Budget sizing: from a separate confidence array [R][K] (separate != 0; conf may be
// null when R == 0) or from the current confidences, its largest B and the admission
// rule (0 argmax, 1 first drop).
struct SizingArgs {
    int separate;
    const float* conf;
    int R;
    int bmax;
    int rule;
};

struct BudgetArgs {
    const float* sorted_surv;
    int n, n_sampling, T, num_reqs;
    const float* vc;
    const float* dc;
    int bmax;
    int rule;
    int32_t* b_star;
    double* best_obj;
    double* obj;
    uint32_t* status;
};

struct FusedSchedArgs {
    const float* conf;
    int R, K, n_sampling, T, num_reqs;
    const float* vc;
    const float* dc;
    int bmax;
    SizingArgs sizing;
    float* surv;
    int32_t* order;
    float* sorted_surv;
    int32_t* b_star;
    double* best_obj;
    int32_t* prefix_len;
    int32_t* offsets;
    int32_t* ver_idx;
    uint32_t* status;
    uint64_t* ws;    // chain workspace to zero (keys and barrier counters), or null
    int ws_words;    // its size in uint64 words
    const int32_t* tokens = nullptr;  // draft tokens for ver_tokens, or null
    int32_t* ver_tokens = nullptr;    // verified tokens, or null
};

// Everything of one step in a single launch: the chain on one
// workgroup per vocabulary tile plus one workgroup that runs stages 2-5 and writes
// tokens and ver_tokens once the chain is done.
struct StepArgs {
    const void* base;
    const void* A;
    const void* Bt;
    const int32_t* prev0;
    int R, K, V, rank;
    int32_t* tokens;
    uint32_t* status;
    uint64_t* keys;     // [K, R]
    uint32_t* sync;     // [K][kMaxGroups] step barrier counters, then the ready flag; zero at launch
    const float* conf;
    int n_sampling, T, num_reqs;
    const float* vc;
    const float* dc;
    int bmax;
    SizingArgs sizing;
    float* surv;
    int32_t* order;
    float* sorted_surv;
    int32_t* b_star;
    double* best_obj;
    int32_t* prefix_len;
    int32_t* offsets;
    int32_t* ver_idx;
    int32_t* ver_tokens;
    int coop;  // cooperative launch (1) or plain launch of a resident grid (0)
};

// Candidate-pruned chain (cand.hip).  Limits of that path: K <= kCandMaxK positions and
// V <= kCandMaxItems * kCandItemLong entries per row.  Rows of at most kCandShortRowMaxV
// entries are streamed in items of kCandItemShort entries (a finer deal keeps more waves
// busy when a row has few items), longer rows in items of kCandItemLong.
constexpr int kCandMaxK = 32;
constexpr int kCandMaxItems = 64;
constexpr int kCandItemLong = 4096;       // base entries per streaming item
constexpr int kCandItemShort = 2048;
constexpr int kCandShortRowMaxV = 32768;
constexpr int kCandGroups = 8192;         // kept 8-entry groups a request's LDS pool holds
constexpr int kCandMaxGroups = 256;       // workgroups of one launch at most
constexpr size_t kMarkovHeaderBytes = 256;  // prepared state: bound scalars, then Bt

inline int cand_item(int V) { return V <= kCandShortRowMaxV ? kCandItemShort : kCandItemLong; }
inline int cand_items_per_row(int V) { return (V + cand_item(V) - 1) / cand_item(V); }

// With fewer requests than compute units a request is streamed by S <= kSplitMax
// workgroups: its owner (which also runs the chain) and S - 1 helpers, each taking a
// share of every row's items (dealt in rounds of 2S - 1, so NC >= 2S - 1).  A helper
// hands each row's kept groups (at most kSplitCap) and maximum over to the owner through
// the workspace.
constexpr int kSplitMax = 4;
constexpr int kSplitCap = 512;
constexpr size_t kSplitHdrBytes = 16;
inline size_t ws_split_ctl_bytes() { return 256 + (size_t)kCandMaxGroups * kCandMaxK * kSplitHdrBytes; }
inline int cand_split(int R, int NC, int num_cu) {
    const int cus = num_cu < kCandMaxGroups ? num_cu : kCandMaxGroups;
    int S = R > 0 ? cus / R : 1;
    S = S < kSplitMax ? S : kSplitMax;
    S = S < (NC + 1) / 2 ? S : (NC + 1) / 2;  // a round of 2S - 1 items per row at least
    return S > 1 ? S : 1;
}
inline size_t ws_split_dat_off(int R, int K) { return ws_total_bytes(R, K); }
// groups [R (S-1)][K][kSplitCap] as 16-byte data, then their group numbers (uint32)
inline size_t ws_split_grp_bytes(int R, int K, int S) {
    return S > 1 ? ws_round((size_t)R * (size_t)(S - 1) * (size_t)K * kSplitCap * 16) : 0;
}
inline size_t ws_split_dat_bytes(int R, int K, int S) {
    return S > 1 ? ws_split_grp_bytes(R, K, S) + ws_round((size_t)R * (size_t)(S - 1) * (size_t)K * kSplitCap * 4)
                 : 0;
}

struct CandArgs {
    const uint16_t* base;
    const uint16_t* A;
    const uint16_t* Bt;
    const void* hdr;   // prepared bound scalars (device)
    const int32_t* prev0;
    int R, K, V, rank, NC;
    int item;  // base entries per item (cand_item(V)); NC = items per row
    int32_t* tokens;
    uint32_t* status;
    int S;                // workgroups per request (1: one workgroup takes whole requests)
    uint32_t* split_ctl;  // S > 1: the workspace at ws_split_ctl_off
    void* split_grp;      // S > 1: the workspace at ws_split_dat_off: the helpers' groups
    uint32_t* split_gid;  // S > 1: then their group numbers
};

int chain_tile_vocab();
// Persistent kernels (the single-launch step, the single-launch chain) keep every
// workgroup resident and synchronise them through counters in the workspace.  They are
// launched either cooperatively (the runtime guarantees residency, at a cost of about
// 17 us per launch on this part) or as a plain launch of a grid that fits on the
// device at once (the caller keeps other kernels off the device meanwhile; every wait
// is bounded, so a workgroup held back longer than the bound ends the step with
// DSPARK_STATUS_SYNC_TIMEOUT instead of hanging).
// bf16 with 1 <= R <= 256 when the grid fits on the device at once; otherwise
// hipErrorCooperativeLaunchTooLarge (nothing enqueued) and the caller runs the
// stage-wise launches.
hipError_t launch_step_single(const StepArgs& a, hipStream_t s);
// fp32 factors, R <= 64 and rank <= 64: the same single launch (chain workgroups +
// scheduling workgroup).
hipError_t launch_step_single_f32(const StepArgs& a, hipStream_t s);
hipError_t launch_zero_keys(uint64_t* keys, size_t n, hipStream_t s);
hipError_t launch_chain_positions(const ChainArgs& a, int num_cu, hipStream_t s);
hipError_t launch_chain_finalize(const uint64_t* keys, int32_t* tokens, int R, int K, const int32_t* ver_idx,
                                 const int32_t* b_star, int32_t* ver_tokens, hipStream_t s);
hipError_t launch_transpose(const void* src, int rows, int cols, int elem_bytes, void* dst, hipStream_t s);
// Bound scalars of a prepared bf16 Markov head into hdr (kMarkovHeaderBytes): the largest
// squared row norms of A and Bt, then 2 max|A| max|Bt| (1 + 2^-10) rounded up and a flag
// that it is finite.
hipError_t launch_markov_bound(const void* A, const void* Bt, int V, int rank, void* hdr, hipStream_t s);
// The candidate-pruned chain: one 512-thread workgroup per compute unit (at most
// kCandMaxGroups of them), or R S workgroups when a request is split (a.S > 1).
// start / stop: when non-null, events that take the kernel's own start and stop time.
hipError_t launch_cand(const CandArgs& a, int num_cu, hipStream_t s, hipEvent_t start = nullptr,
                       hipEvent_t stop = nullptr);

hipError_t launch_survival(const float* conf, int R, int K, float* surv, uint32_t* status, hipStream_t s);
hipError_t launch_topb(const float* surv, int R, int K, int32_t* order, float* sorted_surv, int32_t* rank,
                       hipStream_t s);
hipError_t launch_budget(const BudgetArgs& a, hipStream_t s);
hipError_t launch_allocate(const int32_t* order, const int32_t* b_star, int R, int K, const int32_t* tokens,
                           int32_t* prefix_len, int32_t* offsets, int32_t* ver_idx, int32_t* ver_tokens,
                           hipStream_t s);
hipError_t launch_sched_fused(const FusedSchedArgs& a, hipStream_t s);
// Stages 2-5 over many workgroups, then one (sizing from the current confidences, R*K <=
// kWideMaxN): a.ws is the workspace region at ws_wide_off().
hipError_t launch_sched_wide(const FusedSchedArgs& a, hipStream_t s);
hipError_t launch_accept_greedy(const int32_t* ver_tokens, const int32_t* offsets, const int32_t* target, int R,
                                int K, int32_t* accept_len, int32_t* next_prev0, int32_t* out_tokens,
                                uint32_t* status, hipStream_t s);

}  // namespace dspark
