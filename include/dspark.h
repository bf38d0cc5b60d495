/*
 * dspark.h -- C ABI of libdspark.so, the MI355X (gfx950) implementation of the
 * per-step chain-and-schedule pass of DSpark confidence-scheduled verification.
 *
 * The pass, in the order one step runs it:
 *   1. chain     -- a K-token draft block is chained semi-autoregressively: each
 *                   position adds a rank-r bias keyed on the previously chosen
 *                   token to the backbone's logits and takes the argmax
 *                   (DSpark summary "How DSpark Speeds Up LLM Inference", section
 *                   "Draft better"; MAX worklog "DSpark on MAX", section "What
 *                   DSpark is", item 3);
 *   2. survival  -- running product of per-position confidences along each
 *                   request (vLLM blog "Adaptive Verification in vLLM", section
 *                   "Scheduling the budget");
 *   3. top-B     -- all request x position slots ranked globally by survival;
 *                   taking the ranking's first B slots takes, in each request,
 *                   its first positions only (same section);
 *   4. budget    -- B chosen to maximise expected tokens per microsecond,
 *                   (N_sampling + sum of the B best survivals) divided by
 *                   verify_cost[T + B] + draft_cost[num_reqs] (same section, and
 *                   section "The cost model" for the two summed tables);
 *   5. allocate  -- per-request prefix lengths and a compacted list of the
 *                   verified slots, computed on the GPU with no read-back
 *                   (same section, last paragraph).
 *
 * Conventions shared by every entry point below
 *   - Pointers are DEVICE pointers unless marked (host).  All arrays are
 *     row-major and densely packed.  bf16 data is passed as its 16-bit bit
 *     patterns.
 *   - `stream` is a hipStream_t.  Calls only enqueue work on it and return; they
 *     never synchronise, never copy to the host and never allocate device
 *     memory.  Work enqueued by one call completes in stream order.
 *   - The caller owns every buffer.  Outputs must not alias inputs.  A
 *     workspace is used by one call at a time (calls on different streams need
 *     different workspaces).
 *   - A negative return value means nothing was enqueued; the reason is in
 *     dspark_last_error().  DSPARK_EHIP means a HIP launch failed after host
 *     checks passed; work enqueued before the failure may already be running.
 *   - `status` (optional, may be NULL) is a device uint32 into which kernels OR
 *     the DSPARK_STATUS_* bits for conditions only the device can see.  It is
 *     never cleared by the library.
 */
#ifndef DSPARK_H
#define DSPARK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    DSPARK_OK = 0,
    DSPARK_EINVAL = -1,       /* null pointer, negative size, unknown dtype      */
    DSPARK_ERANGE = -2,       /* scalar outside its documented range              */
    DSPARK_EUNSUPPORTED = -3, /* shape the kernels do not implement (see limits)  */
    DSPARK_EWORKSPACE = -4,   /* workspace missing or smaller than required       */
    DSPARK_EHIP = -5          /* HIP runtime error (text in dspark_last_error)    */
} dspark_status_t;

typedef enum { DSPARK_F32 = 0, DSPARK_BF16 = 1 } dspark_dtype_t;

/* Device-side conditions, OR-ed into *status. */
#define DSPARK_STATUS_PREV_CLAMPED 1u   /* a prev0 entry was outside [0,V); it was clamped into range      */
#define DSPARK_STATUS_CONF_SANITIZED 2u /* a confidence was NaN or outside [0,1]; NaN and <0 became 0, >1 became 1 */
#define DSPARK_STATUS_COST_INVALID 4u   /* verify_cost[T+B] + draft_cost[num_reqs] was not a positive finite
                                           number for some B; that B's objective is -inf                    */
#define DSPARK_STATUS_SYNC_TIMEOUT 8u   /* a persistent kernel waited too long at a grid barrier (its
                                           workgroups were not all resident; see dspark_set_launch_mode);
                                           tokens are then unreliable                                       */
#define DSPARK_STATUS_BAD_ALLOCATION 16u /* dspark_accept_greedy met an inconsistent offsets row; that request
                                           accepted nothing and its next prev0 is -1                        */

/* Admission rules of stage 4. */
#define DSPARK_RULE_ARGMAX 0      /* the smallest B with the largest f(B) (vLLM blog, "Scheduling the budget")  */
#define DSPARK_RULE_FIRST_DROP 1  /* admit slots in rank order while f strictly rises; stop at the first B
                                     with f(B+1) <= f(B), else Bmax (DSpark summary "How DSpark Speeds Up
                                     LLM Inference", section "Verify smarter")                              */

/* Limits. */
#define DSPARK_MAX_SLOTS 16384          /* R*K handled by the single-workgroup scheduler                 */
#define DSPARK_MAX_RANK_BF16 256        /* bf16 chain: rank must be a multiple of 32 and at most this     */
#define DSPARK_MAX_RANK_F32 1024        /* fp32 chain: any rank up to this                                */
#define DSPARK_MAX_KV_BF16 (1 << 23)    /* bf16 chain: K*V at most this (32-bit offsets in 256 rows)      */
#define DSPARK_MAX_VR_BF16 0x7FFFFFFF   /* bf16 chain: V*rank at most this (32-bit key-row offsets)       */

/* Thread-local text describing the last non-OK return on this thread. */
const char* dspark_last_error(void);

/* Library version string. */
const char* dspark_version(void);

/* Bytes of device workspace for dspark_chain / dspark_chain_sample / dspark_step /
 * dspark_step_sized at this shape (0 when R*K == 0).  Zero-fill a workspace once, before
 * its first use: the kernels keep counters in it (grid-barrier counters and a ready flag
 * of the dense single-launch step, the pruned chain's launch epoch and finished-workgroup
 * counter) and leave them ready for the next call, so later calls need no clearing.  A
 * call that ends with DSPARK_STATUS_SYNC_TIMEOUT may leave counters set: zero-fill the
 * workspace again before its next use.  The size includes room for the pruned chain to
 * split each request over several workgroups when there are fewer requests than compute
 * units (the helpers hand their kept candidates over through it); the calls also accept a
 * smaller workspace, down to the size without that room (DSPARK_EINVAL below it), and then
 * stream each request with one workgroup.  So a workspace sized for one shape serves any
 * smaller R and K and any V, rank and dtype.  Calls that share a workspace must not
 * overlap (enqueue them on one stream, or order them with events). */
size_t dspark_workspace_bytes(int R, int K, int V, int rank, int dtype);

/*
 * Prepared state of the Markov head (start-up).  The head's bias for previous token u
 * and candidate v is W[u,v] = sum_k A[u,k] * Bmat[k,v] with A [V,rank] and Bmat
 * [rank,V], a rank-r factorisation (DSpark summary "How DSpark Speeds Up LLM
 * Inference", section "Draft better").  dspark_markov_prepare writes, into the caller's
 * device buffer `state`:
 *   - Bt [V,rank], Bmat transposed (Bt[v,k] = Bmat[k,v]), so that each candidate's
 *     rank-r vector is contiguous for the kernels;
 *   - for bf16, the bias bound of the pruned chain: 2 max_u |A[u,:]| max_v |Bmat[:,v]|
 *     (Euclidean norms, summed in double), times (1 + 2^-10) and rounded up, and
 *     whether it is finite;
 * and fills the host struct *m, which records the pointers it was prepared from.  The
 * chain and step calls take A and Bmat as the method states them plus `m`, and refuse
 * (DSPARK_EINVAL) a handle that was not prepared, or was prepared from other pointers,
 * sizes or dtype -- a transposed or stale factor cannot reach the kernels.  Run it once
 * when the weights are loaded (again if they change), not per step; it enqueues on
 * `stream` like every call.  The caller owns A, Bmat and state; they must stay valid
 * while m is used.  state_bytes must be at least dspark_markov_state_bytes(V, rank,
 * dtype); state must be 256-byte aligned.
 */
#define DSPARK_MARKOV_MAGIC 0x31766b6d6b707364ull /* set in m->magic once prepared */
typedef struct dspark_markov {
    uint64_t magic;
    const void* A;      /* [V,rank] device, as prepared                        */
    const void* Bmat;   /* [rank,V] device, as prepared                        */
    void* state;        /* device: bound scalars (256 bytes), then Bt [V,rank] */
    size_t state_bytes;
    int32_t V, rank, dtype, reserved;
} dspark_markov_t;

size_t dspark_markov_state_bytes(int V, int rank, int dtype);
int dspark_markov_prepare(dspark_markov_t* m, const void* A, const void* Bmat, int V, int rank, int dtype,
                          void* state, size_t state_bytes, void* stream);

/*
 * Stage 1, chain.  For every request r, with prev = prev0[r]:
 *   for i in 0..K-1:
 *     x[v] = base[r,i,v] + sum_k A[prev,k] * Bmat[k,v]    (fp32 accumulation)
 *     tokens[r,i] = argmax_v x[v];  prev = tokens[r,i]
 * (DSpark summary, "Draft better": a small Markov head corrects each position's scores
 * from the previous token alone; MAX worklog, "What DSpark is": a rank-r additive term
 * selected by the token chosen one position earlier, then an argmax.)
 *
 *   base            [R,K,V]   backbone logits (dtype)
 *   A               [V,rank]  first factor, row u = key vector of previous token u (dtype)
 *   Bmat            [rank,V]  second factor (dtype)
 *   markov          the head prepared from exactly this A and Bmat (dspark_markov_prepare)
 *   prev0           [R]       int32 token preceding position 0; values outside [0,V)
 *                             are clamped and flagged with DSPARK_STATUS_PREV_CLAMPED
 *   tokens          [R,K]     int32 output
 *   chained_logits  [R,K,V]   fp32 output x, or NULL (debug / parity use only)
 *   ws, ws_bytes              workspace of at least dspark_workspace_bytes(R,K,V,rank,dtype)
 *
 * argmax: the largest value wins; NaN counts as larger than every number; among
 * equal values the lowest index wins.  The returned index is always in [0,V).
 * How it is computed (dspark_set_chain_form): bf16 without chained_logits, K <=
 * DSPARK_PRUNED_MAX_K and V <= DSPARK_PRUNED_MAX_V runs the pruned chain by default:
 * one streaming pass over base keeps each row's entries within the bias bound of its
 * maximum (the only ones that can win), then every request's chain scores those
 * candidates alone (the rank split into 16-byte chunks dealt over eight lanes, chunk j
 * to lane j mod 8; each lane's products summed by fp32 fused multiply-adds in increasing
 * k, then the eight sums added as a tree: neighbours, pairs, quads, lower part first).
 * Rows the bound cannot prune (a non-finite bound, more
 * candidates than the buffers hold) are scored over the whole vocabulary, so the
 * tokens never depend on how well the bound prunes.  Otherwise (and in the dense form)
 * bf16 products are summed in fp32 by the matrix cores over the whole vocabulary;
 * fp32: fused multiply-add in increasing k.  Forms may differ only where two logits are
 * within float32 rounding of each other.  R == 0 or K == 0 enqueues nothing (data
 * pointers may then be NULL).
 * Limits: V >= 1; bf16 needs rank % 32 == 0, rank <= DSPARK_MAX_RANK_BF16 and
 * K*V <= DSPARK_MAX_KV_BF16 and V*rank <= DSPARK_MAX_VR_BF16;
 * fp32 needs 1 <= rank <= DSPARK_MAX_RANK_F32.
 */
int dspark_chain(const void* base, const void* A, const void* Bmat, int dtype, const int32_t* prev0,
                 int R, int K, int V, int rank, const dspark_markov_t* markov, int32_t* tokens,
                 float* chained_logits, uint32_t* status, void* ws, size_t ws_bytes, void* stream);

/*
 * Which form computes stage 1 (process-wide, for calls made after it):
 *   DSPARK_CHAIN_PRUNED (default): the pruned chain where it applies (see dspark_chain);
 *   DSPARK_CHAIN_DENSE: the matrix-core chain over the whole vocabulary everywhere.
 * Returns DSPARK_EINVAL for an unknown form.
 */
#define DSPARK_CHAIN_PRUNED 0
#define DSPARK_CHAIN_DENSE 1
#define DSPARK_PRUNED_MAX_K 32
#define DSPARK_PRUNED_MAX_V 262144
int dspark_set_chain_form(int form);
int dspark_get_chain_form(void);

/*
 * Stage 1 with probabilistic drafting: as dspark_chain, but each position's token is
 * a SAMPLE of softmax(x / temperature) over the chained logits x instead of their
 * argmax (the vLLM blog's benchmark drafts at temperature 1.0, "Results"), drawn by
 * the Gumbel-max rule (over the whole vocabulary, matrix-core form):
 *   tokens[r,i] = argmax_v  x[v] * (1 / temperature) + g(seed, r, i, v)
 *   g = -log(-log u),  u = (2 b + 1) / 2^24,  b = top 23 bits of word v % 4 of
 *       Philox4x32-10 (Salmon et al., SC 2011) at counter (v / 4, i, r, 0) under the
 *       key (seed & 0xFFFFFFFF, seed >> 32)
 * and the sampled token keys the next position, as in the greedy chain.  The same
 * (seed, inputs) always give the same tokens; use a new seed every step.  The kernels
 * rank the equivalent base-2 value x * (log2(e) / temperature) - log2(-log2 u), a
 * positive affine image of the one above (same argmax), with the hardware base-2
 * logarithm (about 1 ulp), so tokens match an exact evaluation except where two
 * perturbed values are within rounding of each other.  chained_logits (optional) receives x, unperturbed.  temperature must be
 * positive and finite with a finite reciprocal (DSPARK_ERANGE otherwise).  Other
 * arguments, limits and the workspace are those of dspark_chain.  The tokens can be
 * scheduled with the stage calls (survival, top-B, budget, allocate with tokens).
 */
int dspark_chain_sample(const void* base, const void* A, const void* Bmat, int dtype, const int32_t* prev0,
                        int R, int K, int V, int rank, const dspark_markov_t* markov, float temperature,
                        uint64_t seed, int32_t* tokens, float* chained_logits, uint32_t* status, void* ws,
                        size_t ws_bytes, void* stream);

/*
 * Stage 2, survival (vLLM blog, "Scheduling the budget"): for every request r,
 *   surv[r,0] = c[r,0];  surv[r,i] = fl32(surv[r,i-1] * c[r,i])   for i = 1..K-1,
 * i.e. the inclusive running product in float32, in increasing i.  A confidence
 * that is NaN or below 0 is read as 0 and one above 1 as 1
 * (DSPARK_STATUS_CONF_SANITIZED); -0.0 is read as +0.0.
 *   conf [R,K] fp32 input; surv [R,K] fp32 output.
 */
int dspark_survival(const float* conf, int R, int K, float* surv, uint32_t* status, void* stream);

/*
 * Stage 3, global top-B (vLLM blog, "Scheduling the budget"): all n = R*K slots
 * ranked by survival descending, then request ascending, then position
 * ascending.  The first B entries of `order` are the top-B slots for every B.
 *   surv        [R,K] fp32 input, entries in [0,1] (as produced by dspark_survival)
 *   order       [n]   int32 output, flat slot ids r*K+i in rank order
 *   sorted_surv [n]   fp32 output, surv at those slots
 *   rank        [R,K] int32 output (position of each slot in `order`), or NULL
 * Limit: n <= DSPARK_MAX_SLOTS.
 */
int dspark_topb_select(const float* surv, int R, int K, int32_t* order, float* sorted_surv, int32_t* rank,
                       void* stream);

/*
 * Stage 4, budget (vLLM blog, "Scheduling the budget" and "The cost model"):
 *   Bmax = min(n_slots, verify_len - 1 - T)
 *   f(B) = fl64(n_sampling + S_B) / fl64(verify_cost[T+B] + draft_cost[num_reqs]),  B = 0..Bmax
 * where S_B is the exact sum of sorted_surv[0..B) (rounded to double once, with
 * n_sampling) and the division is IEEE double.  A denominator that is not a positive
 * finite number gives f(B) = -inf and sets DSPARK_STATUS_COST_INVALID.
 *   rule DSPARK_RULE_ARGMAX:     b_star is the smallest B with the largest f;
 *   rule DSPARK_RULE_FIRST_DROP: slots are admitted one at a time in rank order while
 *        f strictly rises: b_star is the smallest B < Bmax with f(B+1) <= f(B), else
 *        Bmax (DSpark summary "How DSpark Speeds Up LLM Inference", section "Verify
 *        smarter": admission stops as soon as throughput would fall).
 * Both rules see the same f values; the first-drop b_star never exceeds the argmax
 * one, and they agree whenever f rises to a single peak (e.g. for a linear cost).
 * best_obj is f(b_star).  An unknown rule returns DSPARK_EINVAL.
 *   sorted_surv  [n_slots] fp32, non-increasing, entries in [0,1]
 *   n_sampling   requests that sample a bonus token this step (>= 0)
 *   T            non-draft tokens already in the step, 0 <= T < verify_len
 *   num_reqs     index into draft_cost (scheduled requests), 0 <= num_reqs < draft_len
 *   verify_cost  [verify_len] fp32 microseconds by step token count (forced monotone)
 *   draft_cost   [draft_len]  fp32 microseconds by request count (forced monotone)
 *   b_star [1] int32 output; best_obj [1] fp64 output; obj [Bmax+1] fp64 output or NULL
 * Limit: n_slots <= DSPARK_MAX_SLOTS.
 */
int dspark_choose_budget(const float* sorted_surv, int n_slots, int n_sampling, int T, int num_reqs,
                         const float* verify_cost, int verify_len, const float* draft_cost, int draft_len, int rule,
                         int32_t* b_star, double* best_obj, double* obj, uint32_t* status, void* stream);

/*
 * Stage 5, allocation (vLLM blog, "Scheduling the budget": the B slots are
 * handed to individual requests on the GPU, with no read-back to the host).
 * The selected slots are order[0 .. *b_star).
 *   order       [R*K] int32, a permutation of 0..R*K-1 (from dspark_topb_select)
 *   b_star      [1]   int32 device scalar, 0 <= *b_star <= R*K
 *   tokens      [R,K] int32 draft tokens, or NULL
 *   prefix_len  [R]   int32 output: selected slots of each request
 *   offsets     [R+1] int32 output: exclusive running sum of prefix_len
 *   ver_idx     [R*K] int32 output: selected flat ids r*K+i ordered by request
 *                     then position; entries from *b_star on are -1
 *   ver_tokens  [R*K] int32 output tokens[ver_idx[j]] (-1 past *b_star), or NULL;
 *                     requires tokens
 * Limit: R*K <= DSPARK_MAX_SLOTS.
 */
int dspark_allocate(const int32_t* order, const int32_t* b_star, int R, int K, const int32_t* tokens,
                    int32_t* prefix_len, int32_t* offsets, int32_t* ver_idx, int32_t* ver_tokens,
                    void* stream);

/*
 * The whole pass on one stream: stage 1 (chain) and stages 2-5 (survival, top-B,
 * budget, the allocation), then the verified tokens are gathered.  The stages share
 * no host round trip.  Arguments are those of the stage calls; `surv`, `order`,
 * `sorted_surv`, `prefix_len`, `offsets`, `ver_idx`, `ver_tokens` and `best_obj` are
 * outputs (surv, order, sorted_surv may be NULL).  conf holds R rows (the drafting
 * requests), R*K <= DSPARK_MAX_SLOTS.
 * Order.  Where the pruned chain applies (see dspark_chain), the chain runs first and
 * stages 2-5 start once it has ended, in launches of their own on the same stream (with
 * R*K <= 2048 and sizing from the current confidences, a ranking launch over many
 * workgroups and a one-workgroup finish; otherwise one workgroup): in the method the
 * confidences score the drafted tokens, so the schedule follows the chain (DSpark
 * summary, Figure 1).  Otherwise (and in the dense form) it is ONE launch when the grid
 * fits on the device at once -- one workgroup per 512 vocabulary entries plus one
 * scheduling workgroup that runs stages 2-5 beside the chain, bf16 with R <= 256, and
 * fp32 with R <= 64 and rank <= 64 (with the whole vocabulary in one workgroup, V <=
 * 2048 and rank <= 16, positions need no device-wide barrier) -- else the stage-wise
 * launches.  Results are the same in every form (tokens up to float32 near-ties, see
 * dspark_chain).
 */
int dspark_step(const void* base, const void* A, const void* Bmat, int dtype, const int32_t* prev0,
                int R, int K, int V, int rank, const dspark_markov_t* markov,
                const float* conf, int n_sampling, int T, int num_reqs,
                const float* verify_cost, int verify_len, const float* draft_cost, int draft_len,
                int32_t* tokens, float* surv, int32_t* order, float* sorted_surv,
                int32_t* b_star, double* best_obj,
                int32_t* prefix_len, int32_t* offsets, int32_t* ver_idx, int32_t* ver_tokens,
                uint32_t* status, void* ws, size_t ws_bytes, void* stream);

/*
 * dspark_step for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): the same arguments
 * and results without ws / ws_bytes.  The workspace is a static array of
 * DSPARK_STATIC_WS_BYTES in the library's device code, one per GPU (each GPU holds it
 * from the first call made on it until the process ends), which covers every shape
 * dspark_step accepts; a shape needing more returns DSPARK_ERANGE.  The call allocates
 * nothing and enqueues, before the step, one fill kernel that clears the array's
 * counters and keys when a dense form will run.  Every call on a GPU shares that GPU's
 * array: calls that overlap on one GPU (on different streams, or from different host
 * threads without ordering) race and must be serialised by the caller.
 */
#define DSPARK_STATIC_WS_BYTES (512 * 1024)
int dspark_step_static(const void* base, const void* A, const void* Bmat, int dtype, const int32_t* prev0,
                       int R, int K, int V, int rank, const dspark_markov_t* markov,
                       const float* conf, int n_sampling, int T, int num_reqs,
                       const float* verify_cost, int verify_len, const float* draft_cost, int draft_len,
                       int32_t* tokens, float* surv, int32_t* order, float* sorted_surv,
                       int32_t* b_star, double* best_obj,
                       int32_t* prefix_len, int32_t* offsets, int32_t* ver_idx, int32_t* ver_tokens,
                       uint32_t* status, void* stream);

/*
 * Stages 2-5 alone, in one kernel (one workgroup of 1024 threads working out of LDS):
 * survival, global top-B, the budget under `rule` (optionally sized from another
 * confidence array, as in dspark_step_sized) and the allocation, with no host
 * read-back (vLLM blog, "Scheduling the budget").  For a step whose drafts come from
 * elsewhere, and for scheduler-only batches (up to DSPARK_MAX_SLOTS slots, e.g.
 * 1024 requests x 15 positions).
 *   conf [R,K] fp32; size_conf / size_R / rule as in dspark_step_sized (size_R = -1:
 *   size from conf); scalars and tables as in dspark_choose_budget;
 *   tokens [R,K] int32 draft tokens or NULL; outputs as in dspark_step (surv, order,
 *   sorted_surv and ver_tokens may be NULL; ver_tokens needs tokens).
 */
int dspark_schedule(const float* conf, int R, int K, const float* size_conf, int size_R, int rule,
                    int n_sampling, int T, int num_reqs,
                    const float* verify_cost, int verify_len, const float* draft_cost, int draft_len,
                    const int32_t* tokens, float* surv, int32_t* order, float* sorted_surv,
                    int32_t* b_star, double* best_obj,
                    int32_t* prefix_len, int32_t* offsets, int32_t* ver_idx, int32_t* ver_tokens,
                    uint32_t* status, void* stream);

/*
 * dspark_step with the budget sized from a separate confidence array and a chosen
 * admission rule (vLLM blog, "Scheduling the budget": B is sized from a
 * double-buffered confidence array one step old, while the slots are handed to the
 * requests with current values; the DSpark summary's production notes size it from
 * confidences two steps earlier).
 *   size_conf  [size_R, K] fp32 confidences B is sized from (e.g. the previous step's
 *              conf buffer); may be NULL when size_R is 0 or -1
 *   size_R     rows of size_conf (may differ from R), size_R*K <= DSPARK_MAX_SLOTS;
 *              0 sizes from no slots at all (B = 0); -1 sizes from `conf` itself
 *   rule       DSPARK_RULE_ARGMAX or DSPARK_RULE_FIRST_DROP (see dspark_choose_budget)
 * Sizing: survival, ranking and budget (stages 2-4) over size_conf's slots with this
 * step's n_sampling, T, num_reqs and cost tables, Bmax = min(size_R*K, verify_len-1-T).
 * Allocation: the first min(B, R*K) slots of the ranking of the CURRENT conf; *b_star
 * receives that capped value and *best_obj the sizing objective f(B).  surv, order and
 * sorted_surv describe the current conf.  Everything else is as in dspark_step, and
 * dspark_step is this call with size_R = -1 and DSPARK_RULE_ARGMAX.  size_conf is
 * read before the chain finishes; it must not alias an output.
 */
int dspark_step_sized(const void* base, const void* A, const void* Bmat, int dtype, const int32_t* prev0,
                      int R, int K, int V, int rank, const dspark_markov_t* markov,
                      const float* conf, const float* size_conf, int size_R, int rule,
                      int n_sampling, int T, int num_reqs,
                      const float* verify_cost, int verify_len, const float* draft_cost, int draft_len,
                      int32_t* tokens, float* surv, int32_t* order, float* sorted_surv,
                      int32_t* b_star, double* best_obj,
                      int32_t* prefix_len, int32_t* offsets, int32_t* ver_idx, int32_t* ver_tokens,
                      uint32_t* status, void* ws, size_t ws_bytes, void* stream);

/*
 * Greedy verification of one step's allocated drafts (MAX worklog "DSpark on MAX",
 * section "The kernel pass", item 2: under greedy decoding a draft is accepted
 * exactly when it equals the target's best token; DSpark summary "How DSpark Speeds
 * Up LLM Inference", section "Context": the verifier keeps the longest matching
 * run; vLLM blog "Adaptive Verification in vLLM", section "Scheduling the budget":
 * each request also gains one bonus token).  For every request r, with
 * o = offsets[r] and L = offsets[r+1] - o:
 *   accept_len[r] = the number of leading j < L with ver_tokens[o+j] == target[o+r+j]
 *   next_prev0[r] = target[o + r + accept_len[r]]      (the bonus token)
 *   out_tokens[r] = ver_tokens[o .. o+accept_len[r]), then the bonus token, then -1
 *
 *   ver_tokens  [R*K]     int32 verified draft tokens by request then position (the
 *                         ver_tokens output of dspark_step); may be NULL when K == 0
 *   offsets     [R+1]     int32 exclusive running sum of the prefix lengths (dspark_step)
 *   target      [R*K + R] int32 the target model's greedy tokens: request r's 1 + L
 *                         entries start at o + r (the last accepted token and the L
 *                         drafts run through the target together; vLLM blog, section
 *                         "Varlen decode CUDA graphs"), entry j being its choice after
 *                         the request's first j drafts
 *   accept_len  [R]       int32 output
 *   next_prev0  [R]       int32 output: the token the next step's chain is keyed on
 *   out_tokens  [R, K+1]  int32 output: the tokens this step emits per request, or NULL
 * A row with o < 0, L < 0, L > K or o + L > R*K accepts nothing, gets next_prev0 = -1
 * and an all -1 out_tokens row, and sets DSPARK_STATUS_BAD_ALLOCATION.  R == 0
 * enqueues nothing.  Limit: R*K + R <= INT32_MAX.
 */
int dspark_accept_greedy(const int32_t* ver_tokens, const int32_t* offsets, const int32_t* target, int R, int K,
                         int32_t* accept_len, int32_t* next_prev0, int32_t* out_tokens, uint32_t* status,
                         void* stream);

/*
 * How the persistent kernels are launched.  The single-launch step (dspark_step,
 * dspark_step_sized), the single-launch bf16 chain (dspark_chain), and the bf16 chain
 * that takes two vocabulary tiles per workgroup (dspark_chain and the steps, when the
 * vocabulary has more 512-entry tiles than compute units, up to twice as many, with at
 * most 64 requests) keep every workgroup resident for the whole step and synchronise
 * them through counters in the workspace, which needs all of their workgroups on the
 * device at once (the grid is sized to fit: one workgroup per compute unit).
 *   DSPARK_LAUNCH_RESIDENT (default): a plain kernel launch.  The caller keeps other
 *       kernels off the device while a step runs (one engine stream, as a serving
 *       engine has).  Should another kernel hold compute units, the step waits for
 *       them; every wait is bounded, and a workgroup held back past the bound ends the
 *       step with DSPARK_STATUS_SYNC_TIMEOUT (tokens then unreliable) instead of hanging.
 *   DSPARK_LAUNCH_COOPERATIVE: hipLaunchCooperativeKernel, which guarantees residency
 *       on a shared device; on MI355X it costs about 17 us more per launch.
 * Process-wide; takes effect for calls made after it.  Returns DSPARK_EINVAL for an
 * unknown mode.
 */
#define DSPARK_LAUNCH_RESIDENT 0
#define DSPARK_LAUNCH_COOPERATIVE 1
int dspark_set_launch_mode(int mode);
int dspark_get_launch_mode(void);

/*
 * Measurement hook.  When set (non-NULL hipEvent_t handles, created before the call),
 * every later dspark_step call on this thread sets `before_chain` and `after_chain` on
 * its stream around the chain, so a caller can time the chain with
 * hipEventElapsedTime: for the pruned chain (one kernel) they take that kernel's own
 * start and stop time (hipExtLaunchKernel); otherwise they are markers recorded right
 * before the first chain kernel and right after the last (for a single-launch step,
 * around that launch).
 * Pass NULLs to turn it off (the default).  No synchronisation happens.
 */
int dspark_set_timing_events(void* before_chain, void* after_chain);

/*
 * Start-up forcing of a profiled cost table (host memory): each entry becomes
 * the running maximum of the entries up to it, so the table never decreases
 * (vLLM blog, "The cost model": profiling noise is smoothed by forcing the
 * curve monotonic).  Returns DSPARK_EINVAL for a NULL table, a negative length
 * or a non-finite entry (the table is then left unchanged).
 */
int dspark_force_monotone(float* table, int len);

/*
 * Start-up profiling of a step's cost over a set of shapes (vLLM blog "Adaptive
 * Verification in vLLM", section "The cost model": the engine times dummy steps over
 * the captured graph sizes plus a couple of sizes above the largest, five runs per
 * shape).  For every shape, `warmup` untimed calls and then `runs` timed calls of
 *   fn(shape, user, stream)
 * which must enqueue one step of that size on `stream` and return 0 (anything else
 * aborts with DSPARK_EINVAL).  Each timed call is bracketed by HIP events on `stream`
 * and waited for, so unlike the per-step calls above THIS CALL SYNCHRONISES (it is a
 * start-up routine).
 *   shapes      [n_shapes] (host) token or request counts
 *   samples_us  [n_shapes, runs] (host) output: microseconds of each timed call
 */
typedef int (*dspark_shape_fn)(int shape, void* user, void* stream);
int dspark_profile_shapes(dspark_shape_fn fn, void* user, const int32_t* shapes, int n_shapes, int runs, int warmup,
                          float* samples_us, void* stream);

/*
 * Start-up construction of a cost table from profiled runs (host memory; vLLM blog,
 * section "The cost model"):
 *   1. each shape's cost is the median of its runs (the mean of the two middle runs
 *      for an even count, in double);
 *   2. shapes <= graph_max are the captured graph sizes and must include graph_max;
 *      entry t <= graph_max is the cost of the smallest captured shape >= t (t = 0
 *      counts as 1): a step runs, and pays for, the padded graph, so the table is a
 *      staircase (121 tokens are charged what the 128-token graph costs);
 *   3. past the capture limit the cost is continuous: entry t > graph_max lies on
 *      the line through the two nearest measured shapes above graph_max (the first
 *      or last segment extended beyond them; a single such shape gives a constant),
 *      evaluated in double as c_a + ((c_b - c_a) * (t - s_a)) / (s_b - s_a);
 *   4. entries are rounded to float32 and the table is forced monotone, each entry
 *      the running maximum of the entries up to it.
 *   shapes      [n_shapes] (host) strictly increasing positive counts
 *   samples_us  [n_shapes, runs] (host) e.g. from dspark_profile_shapes; finite
 *   table       [table_len] (host) output, ready for dspark_choose_budget
 * Returns DSPARK_EINVAL for a NULL pointer, a bad count, unsorted shapes, a
 * non-finite run, graph_max missing from the shapes, or entries above graph_max
 * with no measured shape above it.
 */
int dspark_build_cost_table(const int32_t* shapes, int n_shapes, const float* samples_us, int runs, int graph_max,
                            float* table, int table_len);

#ifdef __cplusplus
}
#endif

#endif /* DSPARK_H */
