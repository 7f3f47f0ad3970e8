/*
 * gdn.h -- C ABI of libgdn.so: the Gated DeltaNet verify / commit / rewind /
 * conv-step / chunked-prefill path of speculative multi-token-prediction
 * (MTP) decoding, with the commit folded into the next verify, device greedy
 * acceptance and the gated RMSNorm epilogue, as hand-written HIP kernels for
 * AMD Instinct MI355X (gfx950).
 *
 * Page sources (title, then section):
 *  [P1] "perf(qwen): full-context MTP draft prefill and replay-free rewind"
 *       (Whallm PR #14): Summary item 4 (replay-free rollback: rerun only the
 *       Gated DeltaNet mixer on the captured verification inputs from the
 *       pre-verification state); Measurements (1,024-token layer-major
 *       prefill calls); Tests (rewind equals a direct forward over the
 *       accepted prefix).
 *  [P2] "MTP inference: review and commit structure" (eole docs):
 *       Functional commits items 2 and 4 (verifier buffers, accepted-prefix
 *       state replay, grouped copies, short convolution with a mutated
 *       convolution cache); Review fixes (a grouped replay validates its
 *       layers' arguments before combining them); Verification and limits
 *       (chunked recurrence differs from the sequential one only in rounding).
 *  [P3] "Add request-owned eight-way MTP serving for Qwen 35B" (MTPLX PR
 *       #245): What was broken item 2 (a row commits two, one or no tokens;
 *       inactive rows use keep=0 and keep their pre-verification recurrent
 *       state), item 4 (keep=0 restores the snapshotted base state), item 6
 *       (a fixed B8/T2 cohort; the grid grows to 8 x 32 head rows; rows are
 *       separable); Clean-install verification (fail closed, no fallback).
 * The recurrence is the gated delta rule (Yang, Kautz, Hatamizadeh, "Gated
 * Delta Networks", ICLR 2025):
 *     S_t = a_t S_{t-1} (I - b_t k_t k_t^T) + b_t v_t k_t^T,  o_t = S_t q_t
 * stored transposed: h = S^T, h[i][j], i over d_k, j over d_v (contiguous).
 *
 * CONVENTIONS (every entry point)
 *  - Every array argument is a caller-owned DEVICE pointer, dense, row-major
 *    in the layout given below.  Tensors (x, y, conv_w, conv_b, conv_state,
 *    g, beta, state, o, workspace) must be 16-byte aligned; the int32 arrays
 *    cur, keep and err 4-byte aligned; active has no alignment rule.  The library never
 *    allocates, frees or synchronises inside a call; it launches on `stream`
 *    (a hipStream_t; NULL = the legacy default stream) and returns.
 *  - Host-side validation runs before anything is launched.  On any failure
 *    a status other than GDN_OK is returned and nothing is launched.
 *  - Data errors found on the device (keep or slot out of range, keep != 0
 *    on an inactive row) leave that (layer, row) untouched and OR a
 *    GDN_ERR_* bit into *err when err is not NULL.  The library never
 *    clears *err.
 *  - Outputs (o, y, workspace) must not alias any input, except where an
 *    entry point allows it (gdn_gated_rmsnorm: y may be o).
 *  - The library holds no per-call global state: calls on distinct streams
 *    over disjoint buffers are independent.
 *
 * SHAPES (C = 2*HK*DK + HV*DV conv channels ordered [q heads | k heads |
 * v heads]; value head h reads qk head h / (HV/HK))
 *   x, y        [L][B][T][C]          act dtype
 *   conv_w      [L][C][KCONV]         act dtype (tap KCONV-1 hits the newest token)
 *   conv_b      [L][C] or NULL        act dtype
 *   conv_state  [L][B][KCONV-1][C]    act dtype (row 0 is the oldest)
 *   g, beta     [L][B][T][HV]         act dtype; a = exp(g) (g <= 0), beta in [0,1]
 *   state       [L][B][S][HV][DK][DV] float32, S ring slots per (layer, row)
 *   cur         [L][B] int32          committed slot; NULL means slot 0
 *   o           [L][B][T][HV][DV]     out dtype
 *   active      [B] uint8             NULL means every row is active
 *   keep        [B] int32             tokens to commit per row, 0..T
 *   err         [1] int32 or NULL
 */
#ifndef GDN_H
#define GDN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    GDN_OK = 0,
    GDN_E_NULL = 1,        /* a required pointer is NULL */
    GDN_E_SHAPE = 2,       /* a size is out of the supported range */
    GDN_E_DTYPE = 3,       /* act/out is not GDN_F32 or GDN_BF16 */
    GDN_E_ALIGN = 4,       /* a pointer breaks the alignment rule above */
    GDN_E_UNSUPPORTED = 5, /* a valid request the library does not implement */
    GDN_E_WORKSPACE = 6,   /* workspace NULL or smaller than gdn_workspace_size */
    GDN_E_HIP = 7          /* the HIP runtime reported a launch failure */
} gdn_status;

typedef enum { GDN_F32 = 0, GDN_BF16 = 1 } gdn_dtype;

#define GDN_FLAG_CONV_SILU 1u /* SiLU after the conv */
#define GDN_FLAG_QK_L2NORM 2u /* q, k divided by sqrt(sum of squares + l2_eps) per qk head */

#define GDN_ERR_KEEP 1          /* keep[b] outside 0..T */
#define GDN_ERR_SLOT 2          /* cur[l][b] outside 0..S-1 */
#define GDN_ERR_INACTIVE_KEEP 4 /* keep[b] != 0 on an inactive row */
#define GDN_ERR_LENGTH 8        /* lengths[b] outside 0..T (ragged prefill) */

typedef struct {
    int32_t L, B, T;        /* layers, rows, tokens per call */
    int32_t HV, HK;         /* value heads, qk heads (HV % HK == 0) */
    int32_t DK, DV;         /* head dims, each one of 16, 32, 64, 128 */
    int32_t KCONV;          /* conv width; must be 4 */
    int32_t S;              /* state ring slots per (layer, row) */
    int32_t act, out;       /* gdn_dtype of activations / of o and y */
    float scale, l2_eps;    /* output scale; eps of the q/k L2 norm */
    uint32_t flags;         /* GDN_FLAG_* */
} gdn_dims;

/* Short causal depthwise conv (+ SiLU) over every token of every active row
 * ([P2] Functional commits 2 and 4): y[t][c] = act(sum_j w[c][j] W[t+j][c]
 * + b[c]) with the window W = [conv_state ; x].  If commit_state != 0 the
 * conv cache of each active row becomes the last KCONV-1 window rows.
 * Writes y (out dtype) and, if asked, conv_state; inactive rows are not
 * touched.  Used for decode (T=1) and for prompt prefill (e.g. T=1024). */
gdn_status gdn_conv_step(const gdn_dims* d, const void* x, const void* conv_w,
                         const void* conv_b, void* conv_state, void* y,
                         const uint8_t* active, int commit_state, int32_t* err,
                         void* stream);

/* Verify a window of T <= 4 tokens ([P3] What was broken items 2, 4, 6;
 * [P1] Summary item 4): for each active row, conv + SiLU + q/k L2 norm on
 * the window, then T steps of the gated delta rule from slot cur.  The state
 * after token t (t = 0..T-1) is written to slot (cur + t + 1) mod S and the
 * token's output to o[t].  Slot cur (the pre-verification snapshot),
 * conv_state and cur are never written, so any keep in 0..T can be
 * committed afterwards.  Requires S >= T + 1.  Inactive rows write nothing.
 * err: GDN_ERR_SLOT. */
gdn_status gdn_verify(const gdn_dims* d, const void* x, const void* conv_w,
                      const void* conv_b, const void* conv_state, const void* g,
                      const void* beta, float* state, const int32_t* cur, void* o,
                      const uint8_t* active, int32_t* err, void* stream);

/* Commit each row's accepted length after gdn_verify ([P3] What was broken
 * items 2 and 4): for active rows with keep >= 1, cur <- (cur + keep) mod S
 * (the candidate slot becomes the committed state, no copy) and conv_state
 * <- window rows keep .. keep+KCONV-2 of [conv_state ; x].  keep = 0 and
 * inactive rows write nothing, so the snapshot stays bit-identical.  x and
 * the dims must be those given to gdn_verify.  Requires S >= T + 1.
 * err: GDN_ERR_KEEP, GDN_ERR_SLOT, GDN_ERR_INACTIVE_KEEP. */
gdn_status gdn_commit(const gdn_dims* d, const void* x, void* conv_state, int32_t* cur,
                      const int32_t* keep, const uint8_t* active, int32_t* err,
                      void* stream);

/* Replay-free rewind ([P1] Summary item 4; [P2] Verification and limits:
 * partial commits replay only the accepted recurrent prefix; Review fixes:
 * grouped replay over layers): for each row with keep >= 1, rerun conv +
 * recurrence over the first keep captured window tokens (x, g, beta of the
 * verification, T <= 4) starting from slot cur, write the result back into
 * slot cur in place and commit the conv cache as gdn_commit does.  cur is
 * not changed.  keep = 0 touches nothing.  o may be NULL; when given, o[t]
 * is written for t < keep.  Bit-identical to gdn_verify's candidate keep.
 * err: GDN_ERR_KEEP, GDN_ERR_SLOT. */
gdn_status gdn_rewind(const gdn_dims* d, const void* x, const void* conv_w,
                      const void* conv_b, void* conv_state, const void* g,
                      const void* beta, float* state, const int32_t* cur,
                      const int32_t* keep, void* o, int32_t* err, void* stream);

/* One decode cycle with the commit of the previous cycle folded in ([P2]
 * Functional commits item 2: accepted-prefix state replay; Verification and
 * limits: partial commits replay only the accepted recurrent prefix).  For
 * each row with keep_prev >= 1 the first keep_prev tokens of the previous
 * window (x_prev, g_prev, beta_prev, same dims) are replayed from slot cur
 * and the result is written back into slot cur in place, and conv_state
 * becomes rows keep_prev .. keep_prev+KCONV-2 of [conv_state ; x_prev]; then
 * the new window (x, g, beta) runs on from that state and o[t] is written
 * for every active row, with no candidate states.  cur is never changed, so
 * S may be 1.  The result equals gdn_rewind(previous window, keep_prev)
 * followed by gdn_verify(new window) bit for bit, with one state read and at
 * most one state write per (row, head).  keep_prev may be NULL (no previous
 * window, x_prev/g_prev/beta_prev then unused); active governs only the new
 * window (inactive rows get no outputs; a nonzero keep_prev is still
 * committed).  The accepted length of this cycle's window is passed as
 * keep_prev of the next call; a final gdn_rewind flushes the last one.
 * err: GDN_ERR_KEEP, GDN_ERR_SLOT (the row is then left untouched). */
gdn_status gdn_verify_lazy(const gdn_dims* d, const void* x_prev, const void* g_prev,
                           const void* beta_prev, const int32_t* keep_prev, const void* x,
                           const void* conv_w, const void* conv_b, void* conv_state,
                           const void* g, const void* beta, float* state, const int32_t* cur,
                           void* o, const uint8_t* active, int32_t* err, void* stream);

/* Greedy acceptance of the verified window on the device ([P3] Follow-up:
 * the greedy cohort route keeps the draft IDs on the device and transfers only
 * token-ID arrays; What was broken item 2: keep in {0, 1, 2} at T = 2).
 * Window token 0 is the pending token, tokens 1..T-1 are the drafts
 * draft_ids [B][T-1] (may be NULL when T = 1); target_ids [B][T] holds the
 * target model's greedy token after each window position (its argmax, taken
 * by the caller).  For active rows keep[b] = 1 + the number of leading drafts
 * with draft_ids[b][j] == target_ids[b][j] (the first mismatch ends the
 * prefix), and next_ids[b] (optional) = target_ids[b][keep[b] - 1], the next
 * pending token; inactive rows get keep[b] = 0 and no next token.  All arrays
 * are device int32 (active uint8); keep can go straight into gdn_commit or
 * gdn_verify_lazy on the same stream.  Only d->B and d->T are used (the dims
 * are still validated as for gdn_verify). */
gdn_status gdn_accept_greedy(const gdn_dims* d, const int32_t* draft_ids, const int32_t* target_ids,
                             const uint8_t* active, int32_t* keep, int32_t* next_ids,
                             void* stream);

/* Gated RMSNorm epilogue of the mixer output ([P2] Functional commits item 4:
 * the gated RMSNorm of the FLA path): for every (layer, row, token, value
 * head), y[j] = o[j] / sqrt(mean_j(o^2) + eps) * w[l][j] * SiLU(z[j]).
 * o and y: [L][B][T][HV][DV] in the out dtype (y may alias o); z: same shape
 * in the act dtype; w: [L][DV] in the act dtype.  Inactive rows (active NULL
 * => all active) are not written.  Works after gdn_verify, gdn_verify_lazy,
 * gdn_rewind (T = keep window) and the prefills (T = prompt tokens). */
gdn_status gdn_gated_rmsnorm(const gdn_dims* d, const void* o, const void* z, const void* w,
                             float eps, void* y, const uint8_t* active, void* stream);

/* gdn_verify with the gated RMSNorm of gdn_gated_rmsnorm applied to every
 * output inside the same launch ([P2] Functional commits item 4), so the raw
 * mixer output never goes to memory: y[t] (out dtype, [L][B][T][HV][DV])
 * receives RMSNorm(o[t]) * w * SiLU(z[t]) for every active row; z (act dtype,
 * same shape as y) and norm_w (act dtype, [L][DV]) must be given, norm_eps
 * >= 0.  The mean square is taken over the fp32 outputs before any rounding.
 * Candidate states, slots and error bits are exactly those of gdn_verify
 * (bit for bit).  err: GDN_ERR_SLOT. */
gdn_status gdn_verify_gated_norm(const gdn_dims* d, const void* x, const void* conv_w,
                                 const void* conv_b, const void* conv_state, const void* g,
                                 const void* beta, float* state, const int32_t* cur,
                                 const void* z, const void* norm_w, float norm_eps, void* y,
                                 const uint8_t* active, int32_t* err, void* stream);

/* gdn_verify_lazy with the same fused gated RMSNorm on the new window's
 * outputs (y, z, norm_w, norm_eps as for gdn_verify_gated_norm).  The
 * committed state, conv cache and error bits are exactly those of
 * gdn_verify_lazy.  err: GDN_ERR_KEEP, GDN_ERR_SLOT. */
gdn_status gdn_verify_lazy_gated_norm(const gdn_dims* d, const void* x_prev, const void* g_prev,
                                      const void* beta_prev, const int32_t* keep_prev, const void* x,
                                      const void* conv_w, const void* conv_b, void* conv_state,
                                      const void* g, const void* beta, float* state,
                                      const int32_t* cur, const void* z, const void* norm_w,
                                      float norm_eps, void* y, const uint8_t* active, int32_t* err,
                                      void* stream);

/* Chunked prompt prefill of the same recurrence ([P1] Measurements:
 * 1,024-token layer-major prefill calls; [P2] Verification and limits: the
 * chunk recurrence equals the sequential one up to rounding).  y holds the
 * post-conv q|k|v channels (as written by gdn_conv_step); q and k are
 * L2-normalised here when GDN_FLAG_QK_L2NORM is set.  Every row's state in
 * slot cur is advanced over all T tokens in place, and o[t] is written for
 * every token.  chunk must be 64; chunks restart at each call's first token
 * and the last one may be short.  Every head shape (DK, DV in 16..128) and
 * both activation dtypes are served: bf16 activations with DK >= 32 run on
 * bf16 MFMA with fp32 accumulation (precision recovered by hi/lo splits),
 * fp32 activations and DK = 16 on fp32 MFMA.  workspace: device scratch of
 * at least gdn_workspace_size(d, chunk) bytes, owned by the caller,
 * clobbered; may be NULL when that size is 0 (the fp32 form needs none).
 * err: GDN_ERR_SLOT. */
gdn_status gdn_prefill_chunked(const gdn_dims* d, const void* y, const void* g,
                               const void* beta, float* state, const int32_t* cur, void* o,
                               int32_t chunk, void* workspace, size_t workspace_bytes,
                               int32_t* err, void* stream);

/* Ragged multi-prompt prefill ([P3] What was broken items 1 and 5: several
 * prompts of unequal length prefilled into the rows of one row-owned B8
 * state): gdn_prefill_chunked where row b holds a prompt of lengths[b]
 * tokens (device int32 [B], the same for every layer, 0 <= lengths[b] <= T).
 * y, g, beta and o keep the padded [L][B][T][...] layout with T the longest
 * prompt; the tokens of row b past lengths[b] are never read, their o rows
 * are never written, and the state of slot cur is advanced over exactly
 * lengths[b] tokens (a row of length 0 is left untouched).  Row b's result
 * equals gdn_prefill_chunked on that row alone with T = lengths[b] bit for
 * bit.  workspace: gdn_workspace_size(d, chunk) bytes as for the padded call.
 * err: GDN_ERR_SLOT, GDN_ERR_LENGTH (the row is then left untouched). */
gdn_status gdn_prefill_ragged(const gdn_dims* d, const void* y, const void* g, const void* beta,
                              float* state, const int32_t* cur, void* o, const int32_t* lengths,
                              int32_t chunk, void* workspace, size_t workspace_bytes,
                              int32_t* err, void* stream);

/* Prompt prefill from the raw projection ([P2] Functional commits items 2
 * and 4: the short conv with its cache mutated in place; [P1] Measurements:
 * prompts prefilled in 1,024-token calls): equals gdn_conv_step(d with
 * out = act, x, conv_w, conv_b, conv_state, y, active = NULL,
 * commit_state = 1) followed by gdn_prefill_chunked(d, y, g, beta, state,
 * cur, o, chunk, workspace) bit for bit, without writing y: the conv (+ SiLU
 * when GDN_FLAG_CONV_SILU is set) is computed inside the prefill and rounded to
 * the act dtype as the conv step would store it, and conv_state ends as the
 * last KCONV-1 window rows of [conv_state ; x].  bf16 activations with
 * DK >= 32 only; other shapes return GDN_E_UNSUPPORTED (use the two calls).
 * x: [L][B][T][C] act dtype; conv_w, conv_b, conv_state as for
 * gdn_conv_step; workspace as for gdn_prefill_chunked.  A row whose slot is
 * out of range gets GDN_ERR_SLOT and is left untouched, conv_state included
 * (the two-call sequence would have committed its conv cache). */
gdn_status gdn_prefill_conv_chunked(const gdn_dims* d, const void* x, const void* conv_w,
                                    const void* conv_b, void* conv_state, const void* g,
                                    const void* beta, float* state, const int32_t* cur, void* o,
                                    int32_t chunk, void* workspace, size_t workspace_bytes,
                                    int32_t* err, void* stream);

/* gdn_prefill_chunked without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): the chunk records go to a static device
 * array of the library, GDN_NOALLOC_SCRATCH_BYTES long, which every GPU the
 * library runs on holds (its own copy) until the process ends.  The call
 * allocates and frees nothing.  Dims whose records need more than that
 * (gdn_workspace_size(d, chunk) > GDN_NOALLOC_SCRATCH_BYTES; e.g. one row of
 * 1,024 tokens at 32 value heads and d = 128 needs 50,724,864 bytes) return
 * GDN_E_WORKSPACE before anything is launched.  Every call on one GPU uses
 * that GPU's one array: calls that overlap in time on the same GPU (other
 * streams or threads) race and give undefined results; calls in one stream
 * order are safe.  The records are written in full before they are read, so
 * nothing carries over between calls.  Results equal gdn_prefill_chunked's
 * bit for bit.  err: GDN_ERR_SLOT. */
#define GDN_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
gdn_status gdn_prefill_chunked_noalloc(const gdn_dims* d, const void* y, const void* g,
                                       const void* beta, float* state, const int32_t* cur, void* o,
                                       int32_t chunk, int32_t* err, void* stream);

/* Workspace bytes gdn_prefill_chunked and gdn_prefill_ragged need for these
 * dims: 0 on bad dims and for the fp32 form (fp32 activations or DK = 16),
 * which needs none. */
size_t gdn_workspace_size(const gdn_dims* d, int32_t chunk);

/* Static, human-readable name of a status. */
const char* gdn_status_string(gdn_status s);

/* Build identification: library version and target architecture. */
const char* gdn_version(void);

/* Text of the HIP runtime error behind this thread's most recent GDN_E_HIP
 * ("" if there was none).  Static storage; never NULL. */
const char* gdn_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* GDN_H */
