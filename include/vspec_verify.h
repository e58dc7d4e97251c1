/*
 * vspec_verify.h -- C ABI of the packed draft-token verification library
 * (MI355X / gfx950).
 *
 * One call verifies a whole ragged batch of speculative-decoding requests
 * whose target logits rows are packed into one matrix. Request i owns the
 * consecutive rows row_offsets[i] .. row_offsets[i+1]-1: its K_i draft-verify
 * rows first, then its bonus row (K_i = row_offsets[i+1] - row_offsets[i] - 1
 * may be 0). Per-request data is reached from a row through the row-owner
 * map, as the xLLM documentation describes its ragged verifier ("Adaptive
 * speculative inference", DSpark section "Launch example": per-request
 * sampling parameters are mapped through device-side packed-row owners, and
 * packing boundaries are never read back to the host).
 *
 * Conventions shared by every entry point:
 *  - Every data pointer is a caller-owned DEVICE pointer unless stated. The
 *    library allocates nothing. What carries over from one verify call to
 *    the next lives in the caller's workspace (see vsv_workspace_bytes): a
 *    call counter, the row queue of sampled verification, and tagged words
 *    through which workgroups hand results to the batch scan. The workspace
 *    is zero-filled once before its first use and every call leaves it
 *    ready for the next; one workspace serves one call at a time, so calls
 *    that may overlap in time (on different streams) need workspaces and
 *    outputs of their own. The host side keeps only a per-device cache of
 *    the CU count; vsv_verify_greedy_static alone uses library-owned device
 *    memory (its own comment states the contract).
 *  - All work is enqueued on `stream` (0 = the null stream). Nothing is
 *    synchronised and nothing is read back to the host; results are valid
 *    once the stream reaches them.
 *  - Host-side argument errors return a status before anything is enqueued.
 *    Conditions that only the device can see (layout, token range, logits,
 *    sampling parameters) set bits in the optional sticky `error_flag` word;
 *    outputs are then unspecified but every write stays inside the buffers.
 *  - bfloat16 logits are raw 16-bit patterns; float32 logits are IEEE single.
 *    Row r starts at element r * ld; only its first `vocab` entries are read.
 *    The logits pointer must be aligned to the element size.
 *  - Token ties are broken by lowest index; values compare as IEEE numbers
 *    (so -0 == +0).
 */
#ifndef VSPEC_VERIFY_H
#define VSPEC_VERIFY_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  VSV_OK = 0,
  VSV_EINVAL = 1,        /* NULL required pointer, bad size, dtype or option  */
  VSV_EUNSUPPORTED = 2,  /* option not built into this library                */
  VSV_EWORKSPACE = 3,    /* workspace NULL, misaligned or smaller than needed */
  VSV_EHIP = 4,          /* the HIP runtime refused the launch                */
  VSV_ELIMIT = 5         /* batch beyond the fixed capacity of an entry point */
                         /* that allocates nothing                            */
} vsv_status;

typedef enum { VSV_F32 = 0, VSV_BF16 = 1 } vsv_dtype;

/* Bits of the sticky device error word (OR-ed in, never cleared). */
#define VSV_FLAG_LAYOUT 1  /* offsets not 0 .. R strictly increasing, or owner map inconsistent */
#define VSV_FLAG_TOKEN 2   /* a draft / selected token outside [0, vocab): treated as a mismatch */
#define VSV_FLAG_LOGITS 4  /* NaN or +inf logit, or a row with no finite logit                  */
#define VSV_FLAG_PARAMS 8  /* temperature < 0, top_p outside (0, 1], min_p outside [0, 1]       */
#define VSV_FLAG_STALLED 16 /* a row's result did not reach the batch scan within the scan's    */
                            /* bounded wait (rows of one launch could not all be resident;   */
                            /* not expected on a dedicated GPU); outputs are unspecified     */

typedef struct {
  const void* logits;          /* [num_rows, ld] vocab-wide target logits             */
  int32_t dtype;               /* vsv_dtype                                           */
  int32_t vocab;               /* 1 <= V < 2^30, and a row of V logits < 2 GiB        */
  int64_t ld;                  /* row stride in elements, >= vocab                    */
  int32_t num_requests;        /* B >= 0                                              */
  int32_t num_rows;            /* R = sum_i (K_i + 1) >= B                            */
  const int32_t* row_offsets;  /* [B + 1]: 0 = off[0] < off[1] < ... < off[B] = R     */
  const int32_t* row_owner;    /* [R]: owner[r] = i for off[i] <= r < off[i+1]        */
  const int32_t* draft_tokens; /* [R - B]: draft j of request i at off[i] - i + j;     */
                               /* may be NULL when R == B                             */
} vsv_batch;

typedef struct {
  int32_t* accepted_len; /* [B] a_i = number of leading accepted drafts              */
  int32_t* next_token;   /* [B] replacement token (a_i < K_i) or bonus (a_i = K_i)   */
  int32_t* out_offsets;  /* [B + 1] exclusive scan of (a_i + 1); out_offsets[B] = total */
  int32_t* out_tokens;   /* [R] capacity; request i writes its a_i accepted drafts   */
                         /* and then next_token[i] at out_offsets[i]                 */
  int32_t* row_token;    /* [R] or NULL: the target token chosen for every row       */
  float* row_lse;        /* [R] or NULL: log-sum-exp of the logits the row uses:     */
                         /* x for greedy rows, x / T for sampled rows                */
  int32_t* error_flag;   /* [1] or NULL: sticky VSV_FLAG_* bits                      */
  int32_t* slow_rows;    /* [1] or NULL: incremented once per sampled row whose     */
                         /* draw needed the exact whole-row path (the row is read  */
                         /* again); diagnostics only, results are identical        */
} vsv_outputs;

/* Bytes of device workspace a verify call needs (B requests, R rows): the
 * words through which rows and workgroups hand their results to the
 * batch-wide scan, a call counter, and the row queue of sampled and
 * probabilistic verification. `sampled` is accepted for compatibility; the
 * size is the same for every entry point. The workspace
 * must be zero-filled before its first use (vsv_workspace_init or any
 * zeroed allocation); after that every call leaves it ready for the next
 * one, so one workspace serves any later call on the same stream. Two calls
 * that may overlap in time need two workspaces. */
size_t vsv_workspace_bytes(int32_t num_requests, int32_t num_rows, int32_t sampled);

/* Zero-fill `bytes` of workspace on `stream` with a kernel (no memset node,
 * so it can be captured into a HIP graph). */
vsv_status vsv_workspace_init(void* workspace, size_t bytes, hipStream_t stream);

/* Greedy target verification.
 * Every row's target token is its arg-max (vllm-hust-vspec 0.13.0 README,
 * "EAGLE features": strict greedy top-1 acceptance on a linear, D2H-free
 * acceptance path). relaxed_topk = 1 accepts a draft iff it equals that
 * token; relaxed_topk = K > 1 accepts a draft whose rank in the order
 * (value desc, index asc) is below K, and then emits the draft token itself
 * (same README, "Scope of support": relaxed top-K acceptance is an explicit
 * quality trade-off whose output may differ from strict greedy). The scan
 * accepts the longest run of leading accepted drafts; the next token is the
 * target token of the first rejected row, or of the bonus row if all pass.
 * Errors: VSV_EINVAL (NULL logits/offsets/owner/required output, vocab < 1,
 * ld < vocab, num_rows < num_requests, relaxed_topk outside [1, vocab],
 * misaligned logits, unknown dtype), VSV_EWORKSPACE, VSV_EHIP. */
vsv_status vsv_verify_greedy(const vsv_batch* batch, int32_t relaxed_topk,
                             const vsv_outputs* out, void* workspace,
                             size_t workspace_bytes, hipStream_t stream);

/* Relaxed greedy acceptance, as the serving switches name it without a
 * formula (vllm-hust-vspec 0.13.0 README: section "Launch" sets a
 * confidence-accept margin of 5.25 and says it relaxes greedy acceptance,
 * output no longer matching the target alone token for token; section
 * "General parameters" lists the margin, its from-position and after-tokens
 * gates and protected token ids; section "EAGLE features" lists top-K
 * relaxed acceptance with an after-tokens gate and the strict prefix).
 * A draft equal to the row's greedy token is always accepted. Any other
 * draft d at draft position j of request i is accepted only if
 * j >= from_position, generated[i] + j >= after_tokens, neither d nor the
 * greedy token is in protected_ids, and either top-K holds (topk > 1 and
 * rank(d) < topk, rank in the order value desc, index asc) or the margin
 * holds (margin > 0 and max - x[d] < margin, evaluated in double from the
 * float values: the draft's target log-probability lies within `margin` of
 * the greedy token's). An accepted draft is emitted as itself; replacement
 * and bonus are greedy tokens. topk = 1, margin = 0 is strict top-1. */
#define VSV_MAX_PROTECTED 256
typedef struct {
  int32_t topk;                 /* >= 1; 1: no top-K relaxation                     */
  float margin;                 /* >= 0, finite; 0: no margin relaxation            */
  int32_t from_position;        /* >= 0: first draft position that may relax        */
  int32_t after_tokens;         /* >= 0: generated[i] + j must reach it to relax    */
  const int32_t* generated;     /* [B] device: tokens request i has generated so    */
                                /* far; NULL counts 0 for every request             */
  const int32_t* protected_ids; /* [num_protected] device, any order; NULL if none  */
  int32_t num_protected;        /* 0 .. VSV_MAX_PROTECTED                           */
} vsv_relax;

/* Greedy verification with relaxed acceptance (vsv_relax above); the rest
 * as vsv_verify_greedy, with the same workspace. Errors: as
 * vsv_verify_greedy, plus VSV_EINVAL for a NULL relax, topk outside
 * [1, vocab], a negative or non-finite margin, negative gates,
 * num_protected outside [0, VSV_MAX_PROTECTED] or NULL protected_ids with
 * num_protected > 0. */
vsv_status vsv_verify_greedy_relaxed(const vsv_batch* batch, const vsv_relax* relax,
                                     const vsv_outputs* out, void* workspace,
                                     size_t workspace_bytes, hipStream_t stream);

/* Greedy verification that allocates nothing, for callers that cannot
 * allocate device memory or pass a workspace: code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation. Same arguments,
 * results and errors as vsv_verify_greedy without the workspace: the
 * library keeps one fixed scratch array per GPU for it, sized for
 * VSV_STATIC_MAX_ROWS packed rows (about 0.95 MiB, held until the process
 * ends), zero-filled on the first call on that GPU. Every call on a GPU
 * shares that GPU's array and leaves its contents for the next call, so
 * calls that may overlap in time on one GPU (different streams, threads)
 * race and must not be issued. No hipMalloc, hipFree or other allocation
 * happens in any call.
 * Errors: as vsv_verify_greedy, plus VSV_ELIMIT for num_rows above
 * VSV_STATIC_MAX_ROWS. */
#define VSV_STATIC_MAX_ROWS 16384
vsv_status vsv_verify_greedy_static(const vsv_batch* batch, int32_t relaxed_topk,
                                    const vsv_outputs* out, hipStream_t stream);

/* Sampled (or mixed) target verification with point-mass drafts.
 * Per-request device arrays [B]: temperature (0 = greedy arg-max for that
 * request), top_k (<= 0 or >= vocab: off), top_p (>= 1: off), min_p
 * (<= 0: off). For T > 0 every row draws its own token from the
 * temperature-scaled distribution filtered in this order: top-k, then top-p
 * renormalised over the top-k survivors (shortest prefix of the rank order
 * whose mass reaches top_p, crossing token kept), then min-p (keep
 * (x - max)/T >= ln(min_p)); the draw is the inverse CDF in rank order at
 * u = (w0 >> 8) * 2^-24, w0 = word 0 of Philox4x32-10 with counter
 * (local row j, request i, offset lo, offset hi) and key (seed lo, seed hi).
 * With deterministic drafts this equals rejection sampling against a point
 * mass: the leading matches are accepted, the first mismatching sample is
 * the replacement and the last row's sample is the bonus (xLLM docs,
 * "Adaptive speculative inference", DSpark section "Launch example").
 * Acceptance is strict (draft == sampled token).
 * Errors: as vsv_verify_greedy, plus VSV_EINVAL for NULL parameter arrays. */
vsv_status vsv_verify_sampled(const vsv_batch* batch, const float* temperature,
                              const int32_t* top_k, const float* top_p,
                              const float* min_p, uint64_t seed, uint64_t offset,
                              const vsv_outputs* out, void* workspace,
                              size_t workspace_bytes, hipStream_t stream);

/* Verification with probabilistic drafts: the rejection sampler of
 * speculative decoding. The pages support only the point-mass drafts of
 * vsv_verify_sampled and name this general case as unsupported (xLLM docs,
 * "Adaptive speculative inference", DSpark section "Launch example").
 * draft_logits: device [R - B, draft_ld] rows of the batch's dtype and
 * vocabulary; draft j of request i sits at row off[i] - i + j, like its
 * token. draft_temperature [B]: the temperature the draft was drawn at
 * (0: the draft row's lowest arg-max). With p the target row's law (as in
 * vsv_verify_sampled, or the arg-max's point mass when T = 0) and q the
 * draft row's softmax over its temperature: draft j passes iff
 * u_acc * q(d_j) < p(d_j), u_acc = (w1 >> 8) * 2^-24 from word 1 of the
 * same Philox block as u; the first rejected row emits the inverse-CDF draw
 * of max(0, p - q) in rank order at u (its own draw from p if that residual
 * has no mass); a request whose drafts all pass emits the bonus row's draw.
 * row_token holds each row's emitted-if-first-rejected token (the bonus
 * row's own draw); row_lse is not written; slow_rows counts sampled rows
 * whose survivor set reached below the captured head of the rank order and
 * took the exact whole-row path (several more passes over the row).
 * Workspace: vsv_workspace_bytes(B, R, 0) or more.
 * Errors: as vsv_verify_sampled, plus VSV_EINVAL for NULL draft rows (when
 * R > B) or draft temperatures, draft_ld < vocab or misaligned draft rows.
 * NaN in a draft row sets VSV_FLAG_LOGITS; a negative, NaN or infinite
 * draft temperature sets VSV_FLAG_PARAMS and counts as 0. */
vsv_status vsv_verify_probabilistic(const vsv_batch* batch, const void* draft_logits,
                                    int64_t draft_ld, const float* temperature,
                                    const int32_t* top_k, const float* top_p,
                                    const float* min_p, const float* draft_temperature,
                                    uint64_t seed, uint64_t offset, const vsv_outputs* out,
                                    void* workspace, size_t workspace_bytes,
                                    hipStream_t stream);

/* Draft confidence c_q = exp(y[s_q] - logsumexp(y)) for every draft row q of
 * raw draft logits y (no temperature): the draft probability of the selected
 * token, the score adaptive verification budgets consume (xLLM docs,
 * "Adaptive speculative inference", section "Adaptive target verification
 * from MTP logits"). selected = NULL uses each row's arg-max; an out-of-range
 * selected token gives c_q = 0 and sets VSV_FLAG_TOKEN. lse may be NULL.
 * Errors: VSV_EINVAL (NULL logits/confidence, vocab < 1, ld < vocab,
 * num_draft_rows < 0, misaligned logits, unknown dtype), VSV_EHIP. */
vsv_status vsv_draft_confidence(const void* draft_logits, int32_t dtype,
                                int32_t vocab, int64_t ld, int32_t num_draft_rows,
                                const int32_t* selected, float* confidence,
                                float* lse, int32_t* error_flag,
                                hipStream_t stream);

/* Adaptive target-verify allocation: how many leading drafts of each request
 * the target verifies under a padded row budget, and the packed layout of
 * those verify rows (xLLM docs, "Adaptive speculative inference": the
 * enable_adaptive_target_verify switch, and section "Adaptive target
 * verification from MTP logits": every draft step still runs, the host fixes
 * the padded target-row budget ahead of the round, and the round's draft
 * confidence scores stay on the device to decide the prefix allocation and
 * the packing).
 *
 * Inputs (device, request-major, B requests of K drafts each):
 *   confidence [B * K]  score of draft j of request i at i * K + j, e.g. the
 *                       output of vsv_draft_confidence; clamped to [0, 1],
 *                       NaN counts as 0; may be NULL when K == 0
 *   draft_tokens [B*K]  the drafts in the same layout, or NULL
 *   row_budget G        host value, B <= G <= B * (K + 1): packed target rows
 *                       including every request's bonus row
 * The predicted acceptance of draft j is the float32 running product of its
 * request's clamped scores through j (left to right). The G - B rows beyond
 * the bonus rows go to the positions with the largest products, ties broken
 * by request, then position, ascending; this maximises the expected number
 * of accepted drafts, and each request receives a prefix of its drafts.
 *
 * Outputs (device, caller-allocated):
 *   verify_len [B]      k_i, the number of drafts request i verifies
 *   row_offsets [B+1]   exclusive scan of (k_i + 1); row_offsets[B] = G
 *   row_owner [G]       request of every packed row
 *   row_source [G]      or NULL: full-width row i * (K + 1) + j that packed
 *                       row off[i] + j stands for (j = k_i is the bonus row)
 *   packed_drafts [G-B] or NULL (exactly when draft_tokens is NULL): draft j
 *                       of request i at off[i] - i + j, the layout that
 *                       vsv_verify_greedy / vsv_verify_sampled read
 *   prefix [B * K]      or NULL: the running products
 * The outputs feed vsv_batch directly (num_rows = G).
 * Errors: VSV_EINVAL (B < 0, K < 0, G outside [B, B * (K + 1)],
 * B > 8192 or B * K > 16384, NULL confidence with K > 0, NULL verify_len /
 * row_offsets / row_owner, exactly one of draft_tokens and packed_drafts
 * NULL), VSV_EHIP. B = 0 (with G = 0) is a no-op. */
vsv_status vsv_allocate_verify(const float* confidence, const int32_t* draft_tokens,
                               int32_t num_requests, int32_t num_drafts, int32_t row_budget,
                               int32_t* verify_len, int32_t* row_offsets, int32_t* row_owner,
                               int32_t* row_source, int32_t* packed_drafts, float* prefix,
                               hipStream_t stream);

/* Goodput step selection: the step count of the next decode batch from
 * completed verification results (xLLM docs, "Adaptive speculative
 * inference", section "Adaptive draft step (MTP)" and its policy options:
 * one step count s for the whole batch, the one maximising
 * B * (1 + sum(prefix_acceptance[:s])) / cost_ms(s); prefix acceptance
 * counted over a window of completed batches (default 20); candidates
 * re-scored every update_interval batches (default 5); the step changes only
 * when the predicted relative gain is strictly above switch_min_gain
 * (default 0.05)).
 * HOST code and HOST pointers: the caller reads accepted lengths back with
 * its normal results and passes the full-round cost of every candidate.
 * Rules the page leaves open: candidates are 1 .. max_steps and the
 * controller starts at max_steps; prefix acceptance j is the share, among
 * the window's requests that verified at least j + 1 drafts, of those that
 * accepted at least j + 1 (a position no request in the window verified
 * keeps its last estimate, 0 before any); equal scores go to the smaller
 * step count. The caller owns the state; one state per controller, not
 * thread-safe. */
#define VSV_GOODPUT_MAX_STEPS 32
#define VSV_GOODPUT_MAX_WINDOW 64
typedef struct {
  int32_t max_steps;        /* S: largest step count                           */
  int32_t window_size;      /* completed batches counted                       */
  int32_t update_interval;  /* batches between re-scorings                     */
  double switch_min_gain;   /* strict relative gain needed to switch           */
  int32_t current;          /* step count in force                             */
  int32_t since;            /* batches observed since the last re-scoring      */
  int32_t filled;           /* batches in the window                           */
  int32_t head;             /* window slot of the next batch                   */
  int32_t reached[VSV_GOODPUT_MAX_WINDOW][VSV_GOODPUT_MAX_STEPS];   /* per batch: */
  int32_t accepted[VSV_GOODPUT_MAX_WINDOW][VSV_GOODPUT_MAX_STEPS];  /* requests that verified / accepted > j drafts */
  double estimate[VSV_GOODPUT_MAX_STEPS];  /* prefix acceptance per position */
} vsv_goodput;

/* Reset `state`. Errors: VSV_EINVAL (NULL state, max_steps outside
 * [1, VSV_GOODPUT_MAX_STEPS], window_size outside [1, VSV_GOODPUT_MAX_WINDOW],
 * update_interval < 1, non-finite switch_min_gain). */
vsv_status vsv_goodput_init(vsv_goodput* state, int32_t max_steps, int32_t window_size,
                            int32_t update_interval, double switch_min_gain);

/* Record one completed batch: accepted_len[i] and verify_len[i] (drafts the
 * target verified) of its num_requests requests, host arrays. Positions at or
 * beyond max_steps are not counted. Errors: VSV_EINVAL (NULL state or arrays,
 * num_requests < 0, an entry with accepted_len < 0 or > verify_len); the batch
 * is then not recorded. */
vsv_status vsv_goodput_observe(vsv_goodput* state, const int32_t* accepted_len,
                               const int32_t* verify_len, int32_t num_requests);

/* The step count for the next batch of batch_size requests. cost_ms[s - 1] is
 * the full-round cost of s steps (host array of max_steps positive values);
 * re-scores when update_interval batches were observed since the last
 * re-scoring. Errors: VSV_EINVAL (NULL state, cost_ms or step, a cost that is
 * not positive and finite, batch_size < 0). */
vsv_status vsv_goodput_step(vsv_goodput* state, const double* cost_ms, int32_t batch_size,
                            int32_t* step);

/* One scoring without state: the step count among 1 .. max_steps that the
 * rule above picks from `current`, given prefix_acceptance[max_steps] and
 * cost_ms[max_steps] (host arrays). Returns -1 for invalid arguments. */
int32_t vsv_goodput_select(const double* prefix_acceptance, const double* cost_ms,
                           int32_t max_steps, int32_t batch_size, int32_t current,
                           double switch_min_gain);

/* Static description of a status code. */
const char* vsv_status_string(vsv_status status);

/* Test hook for the batch scan's bounded wait (VSV_FLAG_STALLED), which a
 * dedicated GPU never reaches. Until called again with -1, every later
 * verify launch (vsv_verify_greedy, _relaxed and _static,
 * vsv_verify_sampled and vsv_verify_probabilistic) computes row `row` as
 * usual but leaves its result word unpublished. The launch's scan then
 * spends its poll budget on that word (well under a second), sets
 * VSV_FLAG_STALLED, uses the stale word and completes: outputs stay inside
 * their buffers and the workspace serves the next call as usual.
 * Process-wide; read when a call is made.
 * Returns VSV_EINVAL for row < -1. */
vsv_status vsv_test_withhold_row_word(int32_t row);

/* Library ABI version (major * 100 + minor). */
int32_t vsv_version(void);

#ifdef __cplusplus
}
#endif

#endif /* VSPEC_VERIFY_H */
