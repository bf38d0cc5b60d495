// C ABI of libdspark: argument checks, workspace layout and kernel launches.
// Semantics of every entry point are documented in include/dspark.h.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>

#include <algorithm>
#include <atomic>
#include <mutex>
#include <vector>

#include "dspark.h"
#include "kernels.h"

static_assert(dspark::kMaxSlotsWs == DSPARK_MAX_SLOTS, "the step counters are sized for the slot limit");

namespace {

thread_local char g_err[512] = "";
std::atomic<int> g_launch_mode{DSPARK_LAUNCH_RESIDENT};
std::atomic<int> g_chain_form{DSPARK_CHAIN_PRUNED};
thread_local hipEvent_t g_ev_before_chain = nullptr;
thread_local hipEvent_t g_ev_after_chain = nullptr;

int fail(int code, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return code;
}

int hip_fail(hipError_t e, const char* where) {
    return fail(DSPARK_EHIP, "%s: %s", where, hipGetErrorString(e));
}

// Compute units of the current device, cached per device ordinal.
int num_cu() {
    static int cache[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (cache[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        cache[dev] = n;
    }
    return cache[dev];
}

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

int coop_launch() { return g_launch_mode.load(std::memory_order_relaxed) == DSPARK_LAUNCH_COOPERATIVE ? 1 : 0; }

size_t keys_bytes(int R, int K) { return dspark::ws_total_bytes(R, K); }

// Workspace bytes a call of this shape needs: the dense paths' region, then for bf16 the
// pruned chain's candidate buffers.
size_t ws_need(int R, int K, int V, int dtype) {
    (void)V;
    (void)dtype;
    return keys_bytes(R, K);
}

int check_markov(const dspark_markov_t* m, const void* A, const void* Bmat, int V, int rank, int dtype) {
    if (!m) return fail(DSPARK_EINVAL, "markov: NULL handle (prepare the head with dspark_markov_prepare)");
    if (m->magic != DSPARK_MARKOV_MAGIC || !m->state)
        return fail(DSPARK_EINVAL, "markov: the handle was not prepared (dspark_markov_prepare)");
    if (m->A != A || m->Bmat != Bmat)
        return fail(DSPARK_EINVAL, "markov: the handle was prepared from other A / Bmat pointers");
    if (m->V != V || m->rank != rank || m->dtype != dtype)
        return fail(DSPARK_EINVAL, "markov: the handle was prepared for V=%d rank=%d dtype=%d, the call has V=%d "
                                   "rank=%d dtype=%d", m->V, m->rank, m->dtype, V, rank, dtype);
    return DSPARK_OK;
}

const void* markov_bt(const dspark_markov_t* m) { return (const char*)m->state + dspark::kMarkovHeaderBytes; }

// The pruned chain applies to bf16 with K <= DSPARK_PRUNED_MAX_K and V <= DSPARK_PRUNED_MAX_V
// when no chained logits are asked for and the pruned form is selected.
bool use_pruned(int dtype, int R, int K, int V, const void* A, const float* chained_logits) {
    // the per-row counters hold DSPARK_MAX_SLOTS rows; key rows are read 16 bytes at a time
    return g_chain_form.load(std::memory_order_relaxed) == DSPARK_CHAIN_PRUNED && dtype == DSPARK_BF16 &&
           chained_logits == nullptr && K <= DSPARK_PRUNED_MAX_K && V <= DSPARK_PRUNED_MAX_V &&
           (long long)R * K <= DSPARK_MAX_SLOTS && ((uintptr_t)A & 15u) == 0;
}

dspark::CandArgs cand_args(const void* base, const dspark_markov_t* m, const int32_t* prev0, int R, int K, int V,
                           int rank, int32_t* tokens, uint32_t* status, void* ws, size_t ws_bytes) {
    dspark::CandArgs a{};
    a.base = (const uint16_t*)base;
    a.A = (const uint16_t*)m->A;
    a.Bt = (const uint16_t*)markov_bt(m);
    a.hdr = m->state;
    a.prev0 = prev0;
    a.R = R;
    a.K = K;
    a.V = V;
    a.rank = rank;
    a.item = dspark::cand_item(V);
    a.NC = dspark::cand_items_per_row(V);
    a.tokens = tokens;
    a.status = status;
    // fewer requests than compute units: split each over several workgroups when the
    // workspace holds the helpers' groups (dspark_workspace_bytes sizes it so)
    a.S = 1;
    const int S = dspark::cand_split(R, a.NC, num_cu());
    if (S > 1 && ws_bytes >= dspark::ws_split_dat_off(R, K) + dspark::ws_split_dat_bytes(R, K, S)) {
        char* w = (char*)ws;
        a.S = S;
        a.split_ctl = (uint32_t*)(w + dspark::ws_split_ctl_off());
        a.split_grp = w + dspark::ws_split_dat_off(R, K);
        a.split_gid = (uint32_t*)(w + dspark::ws_split_dat_off(R, K) + dspark::ws_split_grp_bytes(R, K, S));
    }
    return a;
}

int check_chain(const void* base, const void* A, const void* Bt, int dtype, const int32_t* prev0, int R, int K,
                int V, int rank, const int32_t* tokens) {
    if (R < 0 || K < 0) return fail(DSPARK_EINVAL, "chain: negative R (%d) or K (%d)", R, K);
    if (R > 0 && K > 0 && (!base || !A || !Bt || !prev0 || !tokens))
        return fail(DSPARK_EINVAL, "chain: a required pointer is NULL");
    if (V < 1 || rank < 1) return fail(DSPARK_EINVAL, "chain: V (%d) and rank (%d) must be >= 1", V, rank);
    if (dtype != DSPARK_F32 && dtype != DSPARK_BF16) return fail(DSPARK_EINVAL, "chain: unknown dtype %d", dtype);
    if (dtype == DSPARK_BF16 && (rank % 32 != 0 || rank > DSPARK_MAX_RANK_BF16))
        return fail(DSPARK_EUNSUPPORTED, "chain: bf16 rank %d must be a multiple of 32 and <= %d", rank,
                    DSPARK_MAX_RANK_BF16);
    if (dtype == DSPARK_BF16 && (long long)K * V > DSPARK_MAX_KV_BF16)
        return fail(DSPARK_EUNSUPPORTED, "chain: bf16 K*V = %lld exceeds %d", (long long)K * V, DSPARK_MAX_KV_BF16);
    if (dtype == DSPARK_BF16 && (long long)V * rank > DSPARK_MAX_VR_BF16)
        return fail(DSPARK_EUNSUPPORTED, "chain: bf16 V*rank = %lld exceeds %d", (long long)V * rank, DSPARK_MAX_VR_BF16);
    if (dtype == DSPARK_F32 && rank > DSPARK_MAX_RANK_F32)
        return fail(DSPARK_EUNSUPPORTED, "chain: fp32 rank %d exceeds %d", rank, DSPARK_MAX_RANK_F32);
    if ((size_t)R * (size_t)K > (size_t)INT32_MAX) return fail(DSPARK_ERANGE, "chain: R*K overflows int32");
    return DSPARK_OK;
}

int check_ws(void* ws, size_t ws_bytes, int R, int K, int V, int dtype) {
    const size_t need = ws_need(R, K, V, dtype);
    if (!ws || ws_bytes < need)
        return fail(DSPARK_EWORKSPACE, "workspace of %zu bytes needed, %zu given%s", need, ws_bytes,
                    ws ? "" : " (NULL)");
    if (((uintptr_t)ws & 7u) != 0) return fail(DSPARK_EINVAL, "workspace must be 8-byte aligned");
    return DSPARK_OK;
}

int check_sched_scalars(int n, int n_sampling, int T, int num_reqs, const float* vc, int verify_len,
                        const float* dc, int draft_len) {
    if (n > DSPARK_MAX_SLOTS) return fail(DSPARK_EUNSUPPORTED, "schedule: %d slots exceed %d", n, DSPARK_MAX_SLOTS);
    if (!vc || !dc) return fail(DSPARK_EINVAL, "schedule: cost tables must not be NULL");
    if (verify_len < 1 || draft_len < 1) return fail(DSPARK_EINVAL, "schedule: empty cost table");
    if (n_sampling < 0) return fail(DSPARK_ERANGE, "schedule: n_sampling %d < 0", n_sampling);
    if (T < 0 || T >= verify_len) return fail(DSPARK_ERANGE, "schedule: T %d outside [0, %d)", T, verify_len);
    if (num_reqs < 0 || num_reqs >= draft_len)
        return fail(DSPARK_ERANGE, "schedule: num_reqs %d outside [0, %d)", num_reqs, draft_len);
    return DSPARK_OK;
}

}  // namespace

extern "C" {

const char* dspark_last_error(void) { return g_err; }

const char* dspark_version(void) { return "dspark-gfx950 0.1"; }

size_t dspark_workspace_bytes(int R, int K, int V, int rank, int dtype) {
    (void)rank;
    if (R <= 0 || K <= 0) return 0;
    // the minimum, and room for the pruned chain's split requests (on up to kCandMaxGroups
    // compute units)
    const int S = dspark::cand_split(R, dspark::cand_items_per_row(V < 1 ? 1 : V), dspark::kCandMaxGroups);
    return ws_need(R, K, V < 1 ? 1 : V, dtype) + dspark::ws_split_dat_bytes(R, K, S);
}

size_t dspark_markov_state_bytes(int V, int rank, int dtype) {
    if (V < 1 || rank < 1) return 0;
    return dspark::kMarkovHeaderBytes + (size_t)V * (size_t)rank * (dtype == DSPARK_BF16 ? 2 : 4);
}

int dspark_markov_prepare(dspark_markov_t* m, const void* A, const void* Bmat, int V, int rank, int dtype,
                          void* state, size_t state_bytes, void* stream) {
    if (!m || !A || !Bmat || !state) return fail(DSPARK_EINVAL, "markov_prepare: NULL pointer");
    m->magic = 0;
    if (rank < 1 || V < 1) return fail(DSPARK_EINVAL, "markov_prepare: rank %d and V %d must be >= 1", rank, V);
    if (dtype != DSPARK_F32 && dtype != DSPARK_BF16)
        return fail(DSPARK_EINVAL, "markov_prepare: unknown dtype %d", dtype);
    if (((uintptr_t)state & 255u) != 0) return fail(DSPARK_EINVAL, "markov_prepare: state must be 256-byte aligned");
    if (state_bytes < dspark_markov_state_bytes(V, rank, dtype))
        return fail(DSPARK_EWORKSPACE, "markov_prepare: state of %zu bytes needed, %zu given",
                    dspark_markov_state_bytes(V, rank, dtype), state_bytes);
    hipStream_t s = (hipStream_t)stream;
    void* Bt = (char*)state + dspark::kMarkovHeaderBytes;
    hipError_t e = dspark::launch_transpose(Bmat, rank, V, dtype == DSPARK_BF16 ? 2 : 4, Bt, s);
    if (e == hipSuccess && dtype == DSPARK_BF16) e = dspark::launch_markov_bound(A, Bt, V, rank, state, s);
    if (e != hipSuccess) return hip_fail(e, "markov_prepare");
    *m = dspark_markov_t{DSPARK_MARKOV_MAGIC, A, Bmat, state, state_bytes, V, rank, dtype, 0};
    return DSPARK_OK;
}

int dspark_set_chain_form(int form) {
    if (form != DSPARK_CHAIN_PRUNED && form != DSPARK_CHAIN_DENSE)
        return fail(DSPARK_EINVAL, "set_chain_form: unknown form %d", form);
    g_chain_form.store(form, std::memory_order_relaxed);
    return DSPARK_OK;
}

int dspark_get_chain_form(void) { return g_chain_form.load(std::memory_order_relaxed); }

int dspark_chain(const void* base, const void* A, const void* Bmat, int dtype, const int32_t* prev0, int R, int K,
                 int V, int rank, const dspark_markov_t* markov, int32_t* tokens, float* chained_logits,
                 uint32_t* status, void* ws, size_t ws_bytes, void* stream) {
    int rc = check_chain(base, A, Bmat, dtype, prev0, R, K, V, rank, tokens);
    if (rc != DSPARK_OK) return rc;
    if (R == 0 || K == 0) return DSPARK_OK;
    if ((rc = check_markov(markov, A, Bmat, V, rank, dtype)) != DSPARK_OK) return rc;
    if ((rc = check_ws(ws, ws_bytes, R, K, V, dtype)) != DSPARK_OK) return rc;
    hipStream_t s = (hipStream_t)stream;
    const void* Bt = markov_bt(markov);
    if (use_pruned(dtype, R, K, V, A, chained_logits)) {
        const dspark::CandArgs ca = cand_args(base, markov, prev0, R, K, V, rank, tokens, status, ws, ws_bytes);
        const hipError_t e = dspark::launch_cand(ca, num_cu(), s);
        return e == hipSuccess ? DSPARK_OK : hip_fail(e, "chain (pruned)");
    }
    char* chain_ws = (char*)ws + dspark::ws_chain_off();
    dspark::ChainArgs a{base,   A,  Bt,   dtype,          prev0,  R,           K,
                        V,      rank, tokens, chained_logits, status, (uint64_t*)chain_ws,
                        (uint32_t*)(chain_ws + dspark::ws_keys_bytes(R, K)), dspark::SampleArgs{},
                        coop_launch()};
    hipError_t e = dspark::launch_zero_keys(a.keys, dspark::ws_chain_bytes(R, K) / 8, s);
    if (e != hipSuccess) return hip_fail(e, "chain (zero keys)");
    e = dspark::launch_chain_positions(a, num_cu(), s);
    if (e != hipSuccess) return hip_fail(e, "chain");
    e = dspark::launch_chain_finalize(a.keys, tokens, R, K, nullptr, nullptr, nullptr, s);
    return e == hipSuccess ? DSPARK_OK : hip_fail(e, "chain (finalize)");
}

int dspark_chain_sample(const void* base, const void* A, const void* Bmat, int dtype, const int32_t* prev0, int R,
                        int K, int V, int rank, const dspark_markov_t* markov, float temperature, uint64_t seed,
                        int32_t* tokens, float* chained_logits, uint32_t* status, void* ws, size_t ws_bytes,
                        void* stream) {
    int rc = check_chain(base, A, Bmat, dtype, prev0, R, K, V, rank, tokens);
    if (rc != DSPARK_OK) return rc;
    const float scale = 1.4426950408889634f / temperature;  // log2(e) / temperature
    if (!(temperature > 0.f) || !isfinite(temperature) || !isfinite(scale))
        return fail(DSPARK_ERANGE, "chain_sample: temperature %g must be positive, finite and invertible",
                    (double)temperature);
    if (R == 0 || K == 0) return DSPARK_OK;
    if ((rc = check_markov(markov, A, Bmat, V, rank, dtype)) != DSPARK_OK) return rc;
    if ((rc = check_ws(ws, ws_bytes, R, K, V, dtype)) != DSPARK_OK) return rc;
    hipStream_t s = (hipStream_t)stream;
    const void* Bt = markov_bt(markov);
    char* chain_ws = (char*)ws + dspark::ws_chain_off();
    dspark::ChainArgs a{base,   A,  Bt,   dtype,          prev0,  R,           K,
                        V,      rank, tokens, chained_logits, status, (uint64_t*)chain_ws,
                        (uint32_t*)(chain_ws + dspark::ws_keys_bytes(R, K)),
                        dspark::SampleArgs{1, (uint32_t)seed, (uint32_t)(seed >> 32), scale},
                        coop_launch()};
    hipError_t e = dspark::launch_zero_keys(a.keys, dspark::ws_chain_bytes(R, K) / 8, s);
    if (e != hipSuccess) return hip_fail(e, "chain_sample (zero keys)");
    e = dspark::launch_chain_positions(a, num_cu(), s);
    if (e != hipSuccess) return hip_fail(e, "chain_sample");
    e = dspark::launch_chain_finalize(a.keys, tokens, R, K, nullptr, nullptr, nullptr, s);
    return e == hipSuccess ? DSPARK_OK : hip_fail(e, "chain_sample (finalize)");
}

int dspark_survival(const float* conf, int R, int K, float* surv, uint32_t* status, void* stream) {
    if (!conf || !surv) return fail(DSPARK_EINVAL, "survival: NULL pointer");
    if (R < 0 || K < 0) return fail(DSPARK_EINVAL, "survival: negative R (%d) or K (%d)", R, K);
    if (R == 0 || K == 0) return DSPARK_OK;
    const hipError_t e = dspark::launch_survival(conf, R, K, surv, status, (hipStream_t)stream);
    return e == hipSuccess ? DSPARK_OK : hip_fail(e, "survival");
}

int dspark_topb_select(const float* surv, int R, int K, int32_t* order, float* sorted_surv, int32_t* rank,
                       void* stream) {
    if (!surv || !order || !sorted_surv) return fail(DSPARK_EINVAL, "topb_select: NULL pointer");
    if (R < 0 || K < 0) return fail(DSPARK_EINVAL, "topb_select: negative R (%d) or K (%d)", R, K);
    if ((long long)R * K > DSPARK_MAX_SLOTS)
        return fail(DSPARK_EUNSUPPORTED, "topb_select: %lld slots exceed %d", (long long)R * K, DSPARK_MAX_SLOTS);
    if (R == 0 || K == 0) return DSPARK_OK;
    const hipError_t e = dspark::launch_topb(surv, R, K, order, sorted_surv, rank, (hipStream_t)stream);
    return e == hipSuccess ? DSPARK_OK : hip_fail(e, "topb_select");
}

int dspark_choose_budget(const float* sorted_surv, int n_slots, int n_sampling, int T, int num_reqs,
                         const float* verify_cost, int verify_len, const float* draft_cost, int draft_len, int rule,
                         int32_t* b_star, double* best_obj, double* obj, uint32_t* status, void* stream) {
    if (!b_star || !best_obj) return fail(DSPARK_EINVAL, "choose_budget: NULL output");
    if (rule != DSPARK_RULE_ARGMAX && rule != DSPARK_RULE_FIRST_DROP)
        return fail(DSPARK_EINVAL, "choose_budget: unknown admission rule %d", rule);
    if (n_slots < 0) return fail(DSPARK_EINVAL, "choose_budget: negative n_slots %d", n_slots);
    if (n_slots > 0 && !sorted_surv) return fail(DSPARK_EINVAL, "choose_budget: NULL sorted_surv");
    int rc = check_sched_scalars(n_slots, n_sampling, T, num_reqs, verify_cost, verify_len, draft_cost, draft_len);
    if (rc != DSPARK_OK) return rc;
    const int bmax = std::min(n_slots, verify_len - 1 - T);
    dspark::BudgetArgs a{sorted_surv, n_slots, n_sampling, T, num_reqs, verify_cost, draft_cost, bmax, rule,
                         b_star, best_obj, obj, status};
    const hipError_t e = dspark::launch_budget(a, (hipStream_t)stream);
    return e == hipSuccess ? DSPARK_OK : hip_fail(e, "choose_budget");
}

int dspark_allocate(const int32_t* order, const int32_t* b_star, int R, int K, const int32_t* tokens,
                    int32_t* prefix_len, int32_t* offsets, int32_t* ver_idx, int32_t* ver_tokens, void* stream) {
    if (!b_star || !offsets) return fail(DSPARK_EINVAL, "allocate: NULL pointer");
    if (R < 0 || K < 0) return fail(DSPARK_EINVAL, "allocate: negative R (%d) or K (%d)", R, K);
    if ((long long)R * K > DSPARK_MAX_SLOTS)
        return fail(DSPARK_EUNSUPPORTED, "allocate: %lld slots exceed %d", (long long)R * K, DSPARK_MAX_SLOTS);
    if (R > 0 && (!prefix_len || (K > 0 && (!order || !ver_idx))))
        return fail(DSPARK_EINVAL, "allocate: NULL pointer");
    if (ver_tokens && !tokens) return fail(DSPARK_EINVAL, "allocate: ver_tokens needs tokens");
    const hipError_t e = dspark::launch_allocate(order, b_star, R, K, tokens, prefix_len, offsets, ver_idx,
                                                 ver_tokens, (hipStream_t)stream);
    return e == hipSuccess ? DSPARK_OK : hip_fail(e, "allocate");
}

int dspark_step_sized(const void* base, const void* A, const void* Bmat, int dtype, const int32_t* prev0, int R,
                      int K, int V, int rank, const dspark_markov_t* markov, const float* conf,
                      const float* size_conf, int size_R, int rule,
                      int n_sampling, int T, int num_reqs, const float* verify_cost, int verify_len,
                      const float* draft_cost, int draft_len, int32_t* tokens, float* surv, int32_t* order,
                      float* sorted_surv, int32_t* b_star, double* best_obj, int32_t* prefix_len, int32_t* offsets,
                      int32_t* ver_idx, int32_t* ver_tokens, uint32_t* status, void* ws, size_t ws_bytes,
                      void* stream) {
    int rc = check_chain(base, A, Bmat, dtype, prev0, R, K, V, rank, tokens);
    if (rc != DSPARK_OK) return rc;
    const long long n = (long long)R * K;
    if (n > DSPARK_MAX_SLOTS) return fail(DSPARK_EUNSUPPORTED, "step: %lld slots exceed %d", n, DSPARK_MAX_SLOTS);
    if (!b_star || !best_obj || !offsets || (R > 0 && !prefix_len) || (n > 0 && (!ver_idx || !conf)))
        return fail(DSPARK_EINVAL, "step: a required schedule pointer is NULL");
    if (rule != DSPARK_RULE_ARGMAX && rule != DSPARK_RULE_FIRST_DROP)
        return fail(DSPARK_EINVAL, "step: unknown admission rule %d", rule);
    if (size_R < -1) return fail(DSPARK_EINVAL, "step: size_R %d < -1", size_R);
    const bool stale = size_R >= 0;  // -1: size from conf itself
    const long long ns = stale ? (long long)size_R * K : n;
    if (ns > DSPARK_MAX_SLOTS)
        return fail(DSPARK_EUNSUPPORTED, "step: %lld sizing slots exceed %d", ns, DSPARK_MAX_SLOTS);
    if (stale && ns > 0 && !size_conf) return fail(DSPARK_EINVAL, "step: NULL size_conf with %d rows", size_R);
    rc = check_sched_scalars((int)n, n_sampling, T, num_reqs, verify_cost, verify_len, draft_cost, draft_len);
    if (rc != DSPARK_OK) return rc;
    if (n > 0 && (rc = check_markov(markov, A, Bmat, V, rank, dtype)) != DSPARK_OK) return rc;
    if (n > 0 && (rc = check_ws(ws, ws_bytes, R, K, V, dtype)) != DSPARK_OK) return rc;
    hipStream_t s = (hipStream_t)stream;
    const void* Bt = n > 0 ? markov_bt(markov) : nullptr;
    const int bmax = std::min((int)n, verify_len - 1 - T);
    const dspark::SizingArgs sizing{stale ? 1 : 0, size_conf, stale ? size_R : R,
                                    std::min((int)ns, verify_len - 1 - T), rule};
    hipError_t e;
    if (n > 0 && use_pruned(dtype, R, K, V, A, nullptr)) {
        // the chain, then stages 2-5 over the confidences and the verified tokens (in the
        // method the confidences score the drafted tokens, so the schedule follows)
        // (timing events, when set, take the chain kernel's own start and stop time)
        const dspark::CandArgs ca = cand_args(base, markov, prev0, R, K, V, rank, tokens, status, ws, ws_bytes);
        e = dspark::launch_cand(ca, num_cu(), s, g_ev_before_chain, g_ev_after_chain);
        if (e != hipSuccess) return hip_fail(e, "step (pruned chain)");
        dspark::FusedSchedArgs sa{conf,   R,        K,          n_sampling, T,      num_reqs, verify_cost,
                                  draft_cost, bmax, sizing,    surv,       order,  sorted_surv, b_star,
                                  best_obj, prefix_len, offsets, ver_idx,   status, nullptr, 0,
                                  tokens,   ver_tokens};
        if (!stale && n <= dspark::kWideMaxN) {
            // stages 2-5 over many workgroups (their counter and results in the workspace)
            sa.ws = (uint64_t*)((char*)ws + dspark::ws_wide_off());
            e = dspark::launch_sched_wide(sa, s);
        } else {
            e = dspark::launch_sched_fused(sa, s);
        }
        return e == hipSuccess ? DSPARK_OK : hip_fail(e, "step (schedule)");
    }
    if (n > 0) {
        // One launch for the whole step when its grid fits on the device at once (fp32
        // factors: small batches only).
        char* w = (char*)ws;
        dspark::StepArgs st{base, A, Bt, prev0, R, K, V, rank, tokens, status,
                            (uint64_t*)(w + dspark::ws_chain_off()), (uint32_t*)w, conf,
                            n_sampling, T, num_reqs, verify_cost, draft_cost, bmax, sizing, surv, order,
                            sorted_surv, b_star, best_obj, prefix_len, offsets, ver_idx, ver_tokens,
                            coop_launch()};
        if (g_ev_before_chain && (e = hipEventRecord(g_ev_before_chain, s)) != hipSuccess)
            return hip_fail(e, "step (timing event)");
        e = dtype == DSPARK_BF16 ? dspark::launch_step_single(st, s) : dspark::launch_step_single_f32(st, s);
        if (e == hipSuccess) {
            if (g_ev_after_chain && (e = hipEventRecord(g_ev_after_chain, s)) != hipSuccess)
                return hip_fail(e, "step (timing event)");
            return DSPARK_OK;
        }
        if (e != hipErrorCooperativeLaunchTooLarge) return hip_fail(e, "step (single launch)");
        (void)hipGetLastError();  // nothing was enqueued; run the stage-wise launches
    }
    dspark::FusedSchedArgs sa{conf, R, K, n_sampling, T, num_reqs, verify_cost, draft_cost, bmax, sizing, surv, order,
                              sorted_surv, b_star, best_obj, prefix_len, offsets, ver_idx, status,
                              (uint64_t*)((char*)ws + dspark::ws_chain_off()),
                              n > 0 ? (int)(dspark::ws_chain_bytes(R, K) / 8) : 0};
    e = dspark::launch_sched_fused(sa, s);
    if (e != hipSuccess) return hip_fail(e, "step (schedule)");
    if (n == 0) return DSPARK_OK;
    char* chain_ws = (char*)ws + dspark::ws_chain_off();
    dspark::ChainArgs a{base,    A,      Bt,     dtype, prev0, R, K, V, rank, tokens, nullptr, status,
                        (uint64_t*)chain_ws, (uint32_t*)(chain_ws + dspark::ws_keys_bytes(R, K)),
                        dspark::SampleArgs{}, coop_launch()};
    if (g_ev_before_chain && (e = hipEventRecord(g_ev_before_chain, s)) != hipSuccess)
        return hip_fail(e, "step (timing event)");
    e = dspark::launch_chain_positions(a, num_cu(), s);
    if (e != hipSuccess) return hip_fail(e, "step (chain)");
    if (g_ev_after_chain && (e = hipEventRecord(g_ev_after_chain, s)) != hipSuccess)
        return hip_fail(e, "step (timing event)");
    e = dspark::launch_chain_finalize(a.keys, tokens, R, K, ver_idx, b_star, ver_tokens, s);
    return e == hipSuccess ? DSPARK_OK : hip_fail(e, "step (finalize)");
}

int dspark_step(const void* base, const void* A, const void* Bmat, int dtype, const int32_t* prev0, int R, int K,
                int V, int rank, const dspark_markov_t* markov, const float* conf, int n_sampling, int T,
                int num_reqs, const float* verify_cost,
                int verify_len, const float* draft_cost, int draft_len, int32_t* tokens, float* surv,
                int32_t* order, float* sorted_surv, int32_t* b_star, double* best_obj, int32_t* prefix_len,
                int32_t* offsets, int32_t* ver_idx, int32_t* ver_tokens, uint32_t* status, void* ws,
                size_t ws_bytes, void* stream) {
    return dspark_step_sized(base, A, Bmat, dtype, prev0, R, K, V, rank, markov, conf, nullptr, -1, DSPARK_RULE_ARGMAX,
                             n_sampling, T, num_reqs, verify_cost, verify_len, draft_cost, draft_len, tokens, surv,
                             order, sorted_surv, b_star, best_obj, prefix_len, offsets, ver_idx, ver_tokens, status,
                             ws, ws_bytes, stream);
}

}  // extern "C"

// The workspace of dspark_step_static: one array per GPU, in the library's device code,
// zero at load and held until the process ends.  Host code never uses its name as an
// address: each device's copy is found once with hipGetSymbolAddress and kept here.
static __device__ __align__(256) unsigned char scratch[DSPARK_STATIC_WS_BYTES];

namespace {

constexpr int kScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kScratchDevices] = {};

// The current device's copy of `scratch` (found on the first call made on that device).
int static_scratch(void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "step_static (current device)");
    if (dev < 0 || dev >= kScratchDevices)
        return fail(DSPARK_EUNSUPPORTED, "step_static: device %d beyond the %d this library tracks", dev,
                    kScratchDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch[dev]) {
        void* ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_fail(e, "step_static (address of the static workspace)");
        if (!ptr) return fail(DSPARK_EHIP, "step_static: no address for the static workspace");
        g_scratch[dev] = ptr;
    }
    *out = g_scratch[dev];
    return DSPARK_OK;
}

}  // namespace

extern "C" {

int dspark_step_static(const void* base, const void* A, const void* Bmat, int dtype, const int32_t* prev0, int R,
                       int K, int V, int rank, const dspark_markov_t* markov, const float* conf, int n_sampling,
                       int T, int num_reqs, const float* verify_cost, int verify_len, const float* draft_cost,
                       int draft_len, int32_t* tokens, float* surv, int32_t* order, float* sorted_surv,
                       int32_t* b_star, double* best_obj, int32_t* prefix_len, int32_t* offsets, int32_t* ver_idx,
                       int32_t* ver_tokens, uint32_t* status, void* stream) {
    int rc = check_chain(base, A, Bmat, dtype, prev0, R, K, V, rank, tokens);
    if (rc != DSPARK_OK) return rc;
    const size_t need = R > 0 && K > 0 ? ws_need(R, K, V, dtype) : 0;
    if (need > (size_t)DSPARK_STATIC_WS_BYTES)
        return fail(DSPARK_ERANGE, "step_static: R=%d, K=%d need %zu bytes of workspace, the static one holds %d", R,
                    K, need, DSPARK_STATIC_WS_BYTES);
    void* ws = nullptr;
    if ((rc = static_scratch(&ws)) != DSPARK_OK) return rc;
    // The dense forms need their counters and keys at zero; an earlier call may have left
    // them set (a DSPARK_STATUS_SYNC_TIMEOUT), so they are cleared by a fill kernel first.
    // The pruned chain and the schedule keep nothing in the workspace.
    if (need > 0 && !use_pruned(dtype, R, K, V, A, nullptr)) {
        const hipError_t e = dspark::launch_zero_keys((uint64_t*)ws, need / 8, (hipStream_t)stream);
        if (e != hipSuccess) return hip_fail(e, "step_static (clearing the static workspace)");
    }
    return dspark_step(base, A, Bmat, dtype, prev0, R, K, V, rank, markov, conf, n_sampling, T, num_reqs, verify_cost,
                       verify_len, draft_cost, draft_len, tokens, surv, order, sorted_surv, b_star, best_obj,
                       prefix_len, offsets, ver_idx, ver_tokens, status, ws, (size_t)DSPARK_STATIC_WS_BYTES, stream);
}

int dspark_accept_greedy(const int32_t* ver_tokens, const int32_t* offsets, const int32_t* target, int R, int K,
                         int32_t* accept_len, int32_t* next_prev0, int32_t* out_tokens, uint32_t* status,
                         void* stream) {
    if (R < 0 || K < 0) return fail(DSPARK_EINVAL, "accept_greedy: negative R (%d) or K (%d)", R, K);
    if (R == 0) return DSPARK_OK;
    if (!offsets || !target || !accept_len || !next_prev0 || (K > 0 && !ver_tokens))
        return fail(DSPARK_EINVAL, "accept_greedy: a required pointer is NULL");
    if ((long long)R * K + R > (long long)INT32_MAX) return fail(DSPARK_ERANGE, "accept_greedy: R*K + R overflows int32");
    const hipError_t e = dspark::launch_accept_greedy(ver_tokens, offsets, target, R, K, accept_len, next_prev0,
                                                      out_tokens, status, (hipStream_t)stream);
    return e == hipSuccess ? DSPARK_OK : hip_fail(e, "accept_greedy");
}

int dspark_schedule(const float* conf, int R, int K, const float* size_conf, int size_R, int rule, int n_sampling,
                    int T, int num_reqs, const float* verify_cost, int verify_len, const float* draft_cost,
                    int draft_len, const int32_t* tokens, float* surv, int32_t* order, float* sorted_surv,
                    int32_t* b_star, double* best_obj, int32_t* prefix_len, int32_t* offsets, int32_t* ver_idx,
                    int32_t* ver_tokens, uint32_t* status, void* stream) {
    if (R < 0 || K < 0) return fail(DSPARK_EINVAL, "schedule: negative R (%d) or K (%d)", R, K);
    const long long n = (long long)R * K;
    if (n > DSPARK_MAX_SLOTS) return fail(DSPARK_EUNSUPPORTED, "schedule: %lld slots exceed %d", n, DSPARK_MAX_SLOTS);
    if (!b_star || !best_obj || !offsets || (R > 0 && !prefix_len) || (n > 0 && (!ver_idx || !conf)))
        return fail(DSPARK_EINVAL, "schedule: a required pointer is NULL");
    if (ver_tokens && !tokens) return fail(DSPARK_EINVAL, "schedule: ver_tokens needs tokens");
    if (rule != DSPARK_RULE_ARGMAX && rule != DSPARK_RULE_FIRST_DROP)
        return fail(DSPARK_EINVAL, "schedule: unknown admission rule %d", rule);
    if (size_R < -1) return fail(DSPARK_EINVAL, "schedule: size_R %d < -1", size_R);
    const bool stale = size_R >= 0;
    const long long ns = stale ? (long long)size_R * K : n;
    if (ns > DSPARK_MAX_SLOTS)
        return fail(DSPARK_EUNSUPPORTED, "schedule: %lld sizing slots exceed %d", ns, DSPARK_MAX_SLOTS);
    if (stale && ns > 0 && !size_conf) return fail(DSPARK_EINVAL, "schedule: NULL size_conf with %d rows", size_R);
    int rc = check_sched_scalars((int)n, n_sampling, T, num_reqs, verify_cost, verify_len, draft_cost, draft_len);
    if (rc != DSPARK_OK) return rc;
    const int bmax = std::min((int)n, verify_len - 1 - T);
    const dspark::SizingArgs sizing{stale ? 1 : 0, size_conf, stale ? size_R : R,
                                    std::min((int)ns, verify_len - 1 - T), rule};
    dspark::FusedSchedArgs sa{conf,       R,     K,       n_sampling, T,          num_reqs, verify_cost, draft_cost,
                              bmax,       sizing, surv,   order,      sorted_surv, b_star,  best_obj,    prefix_len,
                              offsets,    ver_idx, status, nullptr,   0,           tokens,  ver_tokens};
    const hipError_t e = dspark::launch_sched_fused(sa, (hipStream_t)stream);
    return e == hipSuccess ? DSPARK_OK : hip_fail(e, "schedule");
}

int dspark_set_launch_mode(int mode) {
    if (mode != DSPARK_LAUNCH_RESIDENT && mode != DSPARK_LAUNCH_COOPERATIVE)
        return fail(DSPARK_EINVAL, "set_launch_mode: unknown mode %d", mode);
    g_launch_mode.store(mode, std::memory_order_relaxed);
    return DSPARK_OK;
}

int dspark_get_launch_mode(void) { return g_launch_mode.load(std::memory_order_relaxed); }

int dspark_set_timing_events(void* before_chain, void* after_chain) {
    g_ev_before_chain = (hipEvent_t)before_chain;
    g_ev_after_chain = (hipEvent_t)after_chain;
    return DSPARK_OK;
}

int dspark_profile_shapes(dspark_shape_fn fn, void* user, const int32_t* shapes, int n_shapes, int runs, int warmup,
                          float* samples_us, void* stream) {
    if (!fn || !shapes || !samples_us) return fail(DSPARK_EINVAL, "profile_shapes: NULL argument");
    if (n_shapes < 1 || runs < 1 || warmup < 0)
        return fail(DSPARK_EINVAL, "profile_shapes: n_shapes %d and runs %d must be >= 1, warmup %d >= 0", n_shapes,
                    runs, warmup);
    hipStream_t s = (hipStream_t)stream;
    hipEvent_t e0 = nullptr, e1 = nullptr;
    hipError_t e = hipEventCreate(&e0);
    if (e == hipSuccess) e = hipEventCreate(&e1);
    int rc = DSPARK_OK;
    for (int i = 0; i < n_shapes && rc == DSPARK_OK && e == hipSuccess; ++i) {
        for (int k = 0; k < warmup + runs && rc == DSPARK_OK; ++k) {
            const bool timed = k >= warmup;
            if (timed && (e = hipEventRecord(e0, s)) != hipSuccess) break;
            const int cb = fn(shapes[i], user, stream);
            if (cb != 0) {
                rc = fail(DSPARK_EINVAL, "profile_shapes: the step callback returned %d for shape %d", cb, shapes[i]);
                break;
            }
            if (!timed) continue;
            float ms = 0.f;
            if ((e = hipEventRecord(e1, s)) != hipSuccess || (e = hipEventSynchronize(e1)) != hipSuccess ||
                (e = hipEventElapsedTime(&ms, e0, e1)) != hipSuccess)
                break;
            samples_us[(size_t)i * runs + (k - warmup)] = ms * 1000.f;
        }
    }
    if (e != hipSuccess && rc == DSPARK_OK) rc = hip_fail(e, "profile_shapes");
    if (e0) (void)hipEventDestroy(e0);
    if (e1) (void)hipEventDestroy(e1);
    return rc;
}

int dspark_build_cost_table(const int32_t* shapes, int n_shapes, const float* samples_us, int runs, int graph_max,
                            float* table, int table_len) {
    if (!shapes || !samples_us || (table_len > 0 && !table)) return fail(DSPARK_EINVAL, "build_cost_table: NULL argument");
    if (n_shapes < 1 || runs < 1 || table_len < 0 || graph_max < 1)
        return fail(DSPARK_EINVAL, "build_cost_table: need n_shapes >= 1, runs >= 1, table_len >= 0, graph_max >= 1");
    for (int i = 0; i < n_shapes; ++i)
        if (shapes[i] < 1 || (i > 0 && shapes[i] <= shapes[i - 1]))
            return fail(DSPARK_EINVAL, "build_cost_table: shapes must be positive and strictly increasing");
    // Median of each shape's runs.
    std::vector<double> med(n_shapes), runs_of(runs);
    for (int i = 0; i < n_shapes; ++i) {
        for (int k = 0; k < runs; ++k) {
            runs_of[k] = (double)samples_us[(size_t)i * runs + k];
            if (!isfinite(runs_of[k]))
                return fail(DSPARK_EINVAL, "build_cost_table: shape %d has a non-finite run", shapes[i]);
        }
        std::sort(runs_of.begin(), runs_of.end());
        med[i] = (runs % 2) ? runs_of[runs / 2] : (runs_of[runs / 2 - 1] + runs_of[runs / 2]) / 2.0;
    }
    int n_cap = 0;  // shapes[0, n_cap) are captured graph sizes
    while (n_cap < n_shapes && shapes[n_cap] <= graph_max) ++n_cap;
    if (n_cap == 0 || shapes[n_cap - 1] != graph_max)
        return fail(DSPARK_EINVAL, "build_cost_table: the captured shapes must include graph_max %d", graph_max);
    const int n_eager = n_shapes - n_cap;
    if (table_len - 1 > graph_max && n_eager == 0)
        return fail(DSPARK_EINVAL, "build_cost_table: entries above graph_max need a measured shape above it");
    std::vector<float> out(table_len);
    int g = 0;  // smallest captured shape >= max(t, 1)
    for (int t = 0; t < table_len && t <= graph_max; ++t) {
        while (shapes[g] < std::max(t, 1)) ++g;
        out[t] = (float)med[g];
    }
    int a = n_cap;  // segment [a, a+1] of the measured shapes above graph_max
    for (int t = graph_max + 1; t < table_len; ++t) {
        if (n_eager == 1) {
            out[t] = (float)med[n_cap];
            continue;
        }
        while (a + 2 < n_shapes && shapes[a + 1] <= t) ++a;
        const double sa = shapes[a], sb = shapes[a + 1], ca = med[a], cb = med[a + 1];
        out[t] = (float)(ca + ((cb - ca) * ((double)t - sa)) / (sb - sa));
    }
    for (int t = 0; t < table_len; ++t) table[t] = (t > 0 && out[t] < table[t - 1]) ? table[t - 1] : out[t];
    return DSPARK_OK;
}

int dspark_force_monotone(float* table, int len) {
    if (!table || len < 0) return fail(DSPARK_EINVAL, "force_monotone: NULL table or negative length");
    for (int t = 0; t < len; ++t)
        if (!isfinite(table[t])) return fail(DSPARK_EINVAL, "force_monotone: entry %d is not finite", t);
    for (int t = 1; t < len; ++t)
        if (table[t] < table[t - 1]) table[t] = table[t - 1];
    return DSPARK_OK;
}

}  // extern "C"
