/*
 * gdn.h -- C ABI of the gated delta-rule recurrence library (libgdn.so, gfx950).
 *
 * The recurrence, per (sequence, head), with a d_v x d_k fp32 state S:
 *
 *     S_t = g_t S_{t-1} + beta_t (v_t - S_{t-1} k_t) k_t^T,      o_t = S_t q_t
 *
 * Source: "Qwen3.8-27B 架构深读: Gated DeltaNet 混合线性注意力与 262K 长上下文"
 * (feifeigd.github.io, 2026-08-17), section 三 (Gated DeltaNet): the gated
 * delta-rule equation, whose error term v_t - S_{t-1} k_t reads the state
 * before the gate.  The read-out o_t = S_t q_t is the page's linear-attention
 * read-out applied to the updated state.  The same section says training accumulates the state chunk
 * by chunk in parallel while inference does one fixed-size matrix update per
 * step: gdn_prefill and gdn_decode_step are those two modes.
 *
 * Conventions for every entry point:
 *   - Pointers are DEVICE pointers unless the name ends in _host.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Every call only
 *     enqueues work on it; nothing synchronises and nothing allocates.
 *   - The caller owns every buffer.  The library keeps no device memory; its
 *     only host state is per thread: the last error message and the events
 *     armed by gdn_prefill_set_marks.
 *   - Arguments are validated on the host before anything is enqueued.  On any
 *     error the call returns a non-zero gdn_status, enqueues nothing and leaves
 *     every output untouched; gdn_last_error() then describes the problem.
 *     A failing launch returns GDN_ERR_HIP (earlier launches of the same call
 *     may already be enqueued).
 *   - Device data is not inspected.  The documented domain is 0 < g <= 1 and
 *     finite q, k, v, beta and states; g <= 0 is treated as the smallest
 *     positive float by the chunked prefill.
 *   - Head dimensions: d_k == d_v, one of 16, 32, 64, 128.
 *   - One kernel launch covers at most 2^32 - 1 work-items (the dispatch
 *     packet's grid size is 32 bits); a call whose largest launch would
 *     exceed that returns GDN_ERR_SHAPE.  The limits: chunked prefill
 *     n_seq*H <= 2,097,144; token-serial prefill n_seq*H*tiles <= 67,108,863
 *     (tiles = 16 at d = 128, 2 at d = 64, else 1); decode B*H <= 16,777,215
 *     for d >= 64 and 67,108,863 below;
 *     pre-processing 3 * ceil(H / (2048/d)) * ceil(total_tokens / R) <=
 *     16,777,215 (R = 16 for bf16 and 8 for fp32 when the sequences average
 *     at least R tokens, else 1).
 */
#ifndef GDN_H
#define GDN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element type of q, k and v.  g, beta, states and o are always fp32.  The
 * type is a plain 32-bit integer (not an enum), so that any value a caller
 * passes is a valid argument: unknown values return GDN_ERR_DTYPE. */
typedef int32_t gdn_dtype;
enum { GDN_BF16 = 0, GDN_FP32 = 1 };

/* Status of every call: GDN_OK or one of the error codes below (a plain
 * 32-bit integer, for the same reason). */
typedef int32_t gdn_status;
enum {
    GDN_OK = 0,
    GDN_ERR_NULL = 1,        /* a required pointer is NULL */
    GDN_ERR_SHAPE = 2,       /* a size is out of range or sizes disagree */
    GDN_ERR_DTYPE = 3,       /* unknown gdn_dtype */
    GDN_ERR_ALIGN = 4,       /* q/k/v/o/state not 16-byte aligned, or g/beta not 4-byte aligned */
    GDN_ERR_SEQLENS = 5,     /* cu_seqlens_host not 0 = c[0] <= c[1] <= ... <= c[n] = total */
    GDN_ERR_WORKSPACE = 6,   /* workspace NULL or smaller than gdn_prefill_workspace_bytes() */
    GDN_ERR_UNSUPPORTED = 7, /* head dimension, dtype or chunk size not built */
    GDN_ERR_ALIAS = 8,       /* an output overlaps an input it must not overlap */
    GDN_ERR_HIP = 9,         /* the HIP runtime reported an error */
    GDN_ERR_SLOTS = 10       /* a state slot out of range, or one slot used twice in a batch */
};

/* Prefill algorithms (the `chunk` argument of gdn_prefill). */
#define GDN_CHUNK_AUTO 0     /* chunked (64) where built, else token-serial */
#define GDN_CHUNK_SERIAL 1   /* token-serial: one fixed-size update per token */
#define GDN_CHUNK_64 64      /* chunkwise-parallel, 64-token chunks, MFMA (bf16 q/k/v, d = 128);
                                the library picks one of the two forms below */
#define GDN_CHUNK_64_CHAIN 65 /* chunked; each (sequence, head) carries its state chunk to chunk */
#define GDN_CHUNK_64_SCAN 66  /* chunked; each sequence cut into segments whose affine state maps
                                 (S_out = S_in M + R) are formed in parallel and combined in order
                                 (the chunk-parallel state accumulation of "Qwen3.8-27B 架构深读",
                                 section 三); picked by GDN_CHUNK_64 for few (sequence, head) pairs
                                 when it is expected to be faster */
#define GDN_CHUNK_16 16       /* chunked with 16- or 32-token chunks: the same kernels with each     */
#define GDN_CHUNK_32 32       /* chunk's 64-row tiles part filled, one chain per (sequence, head).
                                 The chunk length changes no result beyond rounding; these exist to
                                 test that (more chunks, more records: slower than GDN_CHUNK_64) */

/* Variants of the recurrence (the `variant` argument of gdn_prefill,
 * gdn_decode_step and gdn_decode_step_slots), from the equations of the
 * Gated DeltaNet section (三) of "Qwen3.8-27B 架构深读":
 *   GDN_VARIANT_GATED_DELTA  the gated delta rule above
 *   GDN_VARIANT_NO_GATE      g = 1: the delta rule S_t = S_{t-1} + beta_t (v_t - S_{t-1} k_t) k_t^T;
 *                            g is ignored and may be NULL
 *   GDN_VARIANT_NO_ERASE     no recall term: S_t = g_t S_{t-1} + beta_t v_t k_t^T, the
 *                            linear-attention write (with both flags and beta = 1:
 *                            plain linear attention, S_t = S_{t-1} + v_t k_t^T)
 * Flags may be combined; any other bit is GDN_ERR_UNSUPPORTED. */
#define GDN_VARIANT_GATED_DELTA 0
#define GDN_VARIANT_NO_GATE 1
#define GDN_VARIANT_NO_ERASE 2
#define GDN_VARIANT_MASK 3

/* Bytes of fp32 state for n_seq sequences: n_seq * H * dv * dk * 4.
 * Returns 0 if a size is negative or zero (n_seq == 0 gives 0 as well).
 * The state is [n_seq][H][dv][dk]: row i of a head's state (its d_k entries)
 * is contiguous, so each row is one coalesced 4*dk-byte run. */
size_t gdn_state_bytes(int64_t n_seq, int32_t H, int32_t dk, int32_t dv);

/* Which algorithm gdn_prefill would run for these arguments:
 * GDN_CHUNK_SERIAL, GDN_CHUNK_64 (or the explicit GDN_CHUNK_64_CHAIN /
 * GDN_CHUNK_64_SCAN / GDN_CHUNK_32 / GDN_CHUNK_16 asked for), or 0 if the
 * combination is not supported. */
int32_t gdn_prefill_algorithm(gdn_dtype dtype, int32_t dk, int32_t dv, int32_t chunk);

/* Set a state before any token arrives ("attention and memory", stethem.com,
 * "Sources, assumptions & limits": the recurrent state exists before the first
 * token).  state [n_seq][H][dv][dk] fp32 is written: a copy of `init` (same
 * layout; may not partially overlap `state`), or zeros when init == NULL. */
gdn_status gdn_state_init(float *state, int64_t n_seq, int32_t H, int32_t dk, int32_t dv,
                          const float *init, void *stream);

/* Zero the states of the listed sequences (the batch/reset rule of
 * "Hybrid · kết hợp nhiều cơ chế..." (openarchlab.com), section 3: a runtime
 * needs state update and batch/reset rules).  slots: device int32 array of
 * n_slots sequence indices; entries outside [0, n_seq) are skipped; NULL zeroes
 * every sequence (n_slots is then ignored). */
gdn_status gdn_state_reset(float *state, int64_t n_seq, int32_t H, int32_t dk, int32_t dv,
                           const int32_t *slots, int32_t n_slots, void *stream);

/* Device workspace that gdn_prefill needs for these sizes (0 for the
 * token-serial algorithm).  Use the same arguments as the gdn_prefill call. */
size_t gdn_prefill_workspace_bytes(int64_t total_tokens, int64_t n_seq, int32_t H,
                                   int32_t dk, int32_t dv, gdn_dtype dtype, int32_t chunk);

/* Prefill a packed batch of n_seq sequences (total_tokens tokens in all).
 *
 *   q, k          [N][H][dk]  dtype, token-major, contiguous, 16-byte aligned
 *   v             [N][H][dv]  dtype
 *   g, beta       [N][H]      fp32 (gate and write strength per token and head);
 *                             g is ignored, and may be NULL, with GDN_VARIANT_NO_GATE
 *   cu_seqlens    [n_seq+1]   int32 device copy of the sequence offsets, and
 *   cu_seqlens_host           the same offsets in host memory (validated here);
 *                             both NULL means one sequence (n_seq must be 1)
 *   initial_state [n_seq][H][dv][dk] fp32, or NULL for zeros.  May be the same
 *                             pointer as final_state (updated in place), but may
 *                             not otherwise overlap it.
 *   o             [N][H][dv]  fp32 output (must not overlap any input)
 *   final_state   [n_seq][H][dv][dk] fp32 output
 *   chunk         GDN_CHUNK_AUTO, GDN_CHUNK_SERIAL, GDN_CHUNK_64, GDN_CHUNK_64_CHAIN,
 *                 GDN_CHUNK_64_SCAN (1 to 64 sequences and at least one token, else GDN_ERR_UNSUPPORTED),
 *                 GDN_CHUNK_32 or GDN_CHUNK_16
 *   workspace     device scratch of at least gdn_prefill_workspace_bytes();
 *                 may be NULL when that is 0.  Its contents on entry do not matter.
 *   variant       GDN_VARIANT_* flags (0: the gated delta rule)
 *
 * Each sequence starts from its own initial state and never sees another
 * sequence's tokens; a zero-length sequence copies its initial state to its
 * final state.  Running a sequence in segments, feeding each final state back
 * as the next initial state, gives the one-shot result up to rounding
 * ("Hybrid..." (openarchlab.com), section 4: segmented runs with carried state
 * must not change the result). */
gdn_status gdn_prefill(const void *q, const void *k, const void *v, gdn_dtype dtype,
                       const float *g, const float *beta,
                       const int32_t *cu_seqlens, const int32_t *cu_seqlens_host, int64_t n_seq,
                       int64_t total_tokens, int32_t H, int32_t dk, int32_t dv,
                       const float *initial_state, float *o, float *final_state,
                       int32_t chunk, void *workspace, size_t workspace_bytes, int32_t variant,
                       void *stream);

/* Allocation-free form of gdn_prefill, for callers that cannot allocate
 * device memory or pass a workspace: code recorded under HIP graph capture,
 * tight serving loops, and harnesses that forbid allocation.  Arguments,
 * semantics and errors are those of gdn_prefill without the workspace: the
 * kernels use a fixed scratch array of GDN_NOALLOC_SCRATCH_BYTES that the
 * library holds on each device it runs on until the process ends (the array
 * of the device current at the call; the stream must belong to that device).
 * Sizes whose gdn_prefill_workspace_bytes() exceeds that limit return
 * GDN_ERR_WORKSPACE and enqueue nothing (128 MiB covers, for example, one
 * sequence of up to 6,912 tokens at H = 48 with d = 128).
 * Nothing is allocated, freed or synchronised.  Every call on one device
 * shares that device's array and leaves its contents behind (nothing in it
 * needs to start at zero): calls that can overlap on one device, on any
 * streams, race and must be serialised by the caller. */
#define GDN_NOALLOC_SCRATCH_BYTES (128u << 20)
gdn_status gdn_prefill_noalloc(const void *q, const void *k, const void *v, gdn_dtype dtype,
                               const float *g, const float *beta,
                               const int32_t *cu_seqlens, const int32_t *cu_seqlens_host, int64_t n_seq,
                               int64_t total_tokens, int32_t H, int32_t dk, int32_t dv,
                               const float *initial_state, float *o, float *final_state,
                               int32_t chunk, int32_t variant, void *stream);

/* One token for each of B sequences, updating their states in place.
 *
 *   q, k    [B][H][dk] dtype;   v [B][H][dv] dtype;   g, beta [B][H] fp32
 *   state   [B][H][dv][dk] fp32, read once and written once (in place)
 *   o       [B][H][dv] fp32, o = S_t q_t from the updated state
 *   variant GDN_VARIANT_* flags (0: the gated delta rule)
 *
 * The per-token cost is fixed, whatever the position of the token ("Layouts
 * híbridos: três DeltaNet, uma attention" (llmdeepdive.com), section Conceito:
 * the state is a fixed set of matrices edited in place). */
gdn_status gdn_decode_step(const void *q, const void *k, const void *v, gdn_dtype dtype,
                           const float *g, const float *beta, float *state, float *o,
                           int64_t B, int32_t H, int32_t dk, int32_t dv, int32_t variant, void *stream);

/* One token for each of B requests whose states live in a pool of n_slots
 * states, the serving form of gdn_decode_step.  "Hybrid · kết hợp nhiều cơ
 * chế..." (openarchlab.com), section 3: a runtime needs state-update and
 * batch/reset rules, and its memory planning must count the recurrent state
 * (gdn_state_bytes(n_slots, ...) for the pool).  Row b of the batch reads and
 * updates state slot slots[b] in place; slots are assigned by the caller, and a
 * slot handed to a new request is cleared first with gdn_state_reset.
 *
 *   q, k, v, g, beta, o, variant   as for gdn_decode_step, with B rows
 *   state_pool   [n_slots][H][dv][dk] fp32, updated in place for the slots used
 *   slots        device int32 [B]: the slot of each row; -1 marks a padding row,
 *                whose o row is written as zeros and which touches no state
 *   slots_host   optional host copy of slots, checked before anything is
 *                enqueued: every entry in [-1, n_slots) and no slot twice
 *                (GDN_ERR_SLOTS otherwise).  Pass NULL when the device array
 *                changes after the call is recorded (a captured graph): the
 *                kernel then treats any entry outside [0, n_slots) as padding,
 *                and two rows naming one slot race, which the caller must avoid.
 * Nothing here allocates or synchronises, so the call can be captured in a
 * HIP graph together with gdn_state_reset. */
gdn_status gdn_decode_step_slots(const void *q, const void *k, const void *v, gdn_dtype dtype,
                                 const float *g, const float *beta, float *state_pool, int64_t n_slots,
                                 const int32_t *slots, const int32_t *slots_host, float *o,
                                 int64_t B, int32_t H, int32_t dk, int32_t dv, int32_t variant, void *stream);

/* Activation after the pre-processing convolution (the `activation` argument). */
enum { GDN_ACT_NONE = 0, GDN_ACT_SILU = 1 };

/* Pre-processing in front of the recurrence, for a packed batch laid out as
 * for gdn_prefill.  The DeltaNet layers of "Layouts híbridos: três DeltaNet,
 * uma attention" (llmdeepdive.com), section Conceito, carry a convolution of
 * kernel 4 beside their gated state; "Qwen3.8-27B 架构深读"
 * (feifeigd.github.io, 2026-08-17), section 三, gives one gate and one write
 * strength per token.  Per sequence, head and channel of each of q, k, v:
 *   y_t = w[0] x_{t-3} + w[1] x_{t-2} + w[2] x_{t-1} + w[3] x_t
 * (causal, depthwise; before a sequence's first token the window holds the
 * sequence's conv state), then SiLU when activation == GDN_ACT_SILU; q and k
 * are L2-normalised per (token, head) (a zero vector stays zero), v is not;
 *   beta = sigmoid(b_logit),  g = exp(-softplus(a_logit + gate_bias[h])).
 *
 *   xq, xk, xv       [N][H][d] dtype: raw (projected) q, k, v
 *   conv_w           [3][H][d][4] fp32: taps of tensor q, k, v (tap 3 = current token)
 *   conv_state_in    [n_seq][3][3][H][d] dtype: per sequence and tensor, the raw
 *                    inputs of the three tokens before this part (oldest first),
 *                    or NULL for zeros
 *   conv_state_out   [n_seq][3][3][H][d] dtype: the last three raw inputs of each
 *                    sequence (for a sequence shorter than three, shifted in from
 *                    its starting state).  May be the same pointer as
 *                    conv_state_in (updated in place), but may not otherwise
 *                    overlap it.  Feeding it back as the next part's
 *                    conv_state_in continues the sequence exactly.
 *   a_logit, b_logit [N][H] fp32;   gate_bias [H] fp32 or NULL (zeros)
 *   cu_seqlens, cu_seqlens_host, n_seq, total_tokens: as for gdn_prefill
 *   q, k, v          [N][H][d] dtype outputs (rounded to nearest even for bf16);
 *                    they may not overlap any input
 *   g, beta          [N][H] fp32 outputs
 * A decode step is a batch of n_seq one-token sequences.  Errors as for the
 * other calls; activation outside the enum is GDN_ERR_UNSUPPORTED. */
gdn_status gdn_preprocess(const void *xq, const void *xk, const void *xv, gdn_dtype dtype,
                          const float *conv_w, const void *conv_state_in, void *conv_state_out,
                          const float *a_logit, const float *b_logit, const float *gate_bias,
                          const int32_t *cu_seqlens, const int32_t *cu_seqlens_host, int64_t n_seq,
                          int64_t total_tokens, int32_t H, int32_t d, int32_t activation,
                          void *q, void *k, void *v, float *g, float *beta, void *stream);

/* The layer's recurrence from its raw projections: gdn_preprocess and
 * gdn_prefill in one pass over the raw inputs.  The DeltaNet layers of
 * "Layouts híbridos: três DeltaNet, uma attention" (llmdeepdive.com), section
 * Conceito, carry a convolution of kernel 4 beside their gated state; the
 * gated delta rule and its per-token gate and strength are those of
 * "Qwen3.8-27B 架构深读" (feifeigd.github.io, 2026-08-17), section 三.
 * The chunk preparation forms the convolution, activation, L2 norm of q and
 * k, and the gate maps exactly as gdn_preprocess does (the same bits), writes
 * the processed q, k, v once, and the state chain reads them back: the
 * outputs equal gdn_preprocess followed by gdn_prefill (chunked), bit for bit.
 *
 *   xq, xk, xv, conv_w, conv_state_in, conv_state_out, activation, a_logit,
 *   b_logit, gate_bias     as for gdn_preprocess (conv_state_out required;
 *                          a_logit ignored, and may be NULL, with GDN_VARIANT_NO_GATE)
 *   cu_seqlens, cu_seqlens_host, n_seq, total_tokens, H, initial_state, o,
 *   final_state, chunk, workspace, workspace_bytes, variant
 *                          as for gdn_prefill (chunk: GDN_CHUNK_AUTO, one of the
 *                          GDN_CHUNK_64 forms, GDN_CHUNK_32 or GDN_CHUNK_16; the workspace size is
 *                          gdn_prefill_workspace_bytes(..., GDN_BF16, chunk))
 *   q, k, v    [N][H][d] bf16 outputs: the processed inputs of the recurrence
 *              (caller-owned; the state chain reads them)
 *   g, beta    [N][H] fp32 outputs, or NULL when not wanted
 * Only bf16 with d = 128 (the chunked prefill) is built: anything else is
 * GDN_ERR_UNSUPPORTED (use gdn_preprocess, then gdn_prefill).  No output may
 * overlap an input or another output, except conv_state_out == conv_state_in
 * and final_state == initial_state (updated in place).  Errors as for the
 * other calls. */
gdn_status gdn_layer_prefill(const void *xq, const void *xk, const void *xv, gdn_dtype dtype,
                             const float *conv_w, const void *conv_state_in, void *conv_state_out,
                             int32_t activation, const float *a_logit, const float *b_logit,
                             const float *gate_bias, const int32_t *cu_seqlens, const int32_t *cu_seqlens_host,
                             int64_t n_seq, int64_t total_tokens, int32_t H, int32_t d,
                             const float *initial_state, float *o, float *final_state,
                             void *q, void *k, void *v, float *g, float *beta, int32_t chunk,
                             void *workspace, size_t workspace_bytes, int32_t variant, void *stream);

/* Profiling hook.  Arms up to three caller-owned hipEvent_t handles
 * (events[0..n_events-1]; NULL entries are skipped) for the NEXT gdn_prefill
 * call made by this host thread, which records them on its stream:
 *   events[0] before its first kernel,
 *   events[1] after the state-independent per-chunk kernels (planning and
 *             chunk preparation; nothing for the token-serial algorithm),
 *   events[2] after the state chain (its last kernel).
 * That call disarms the hook whether it succeeds or not; n_events = 0 disarms
 * it at once.  Returns GDN_ERR_SHAPE for n_events outside [0, 3] and
 * GDN_ERR_NULL for a NULL array with n_events > 0 (the hook is then disarmed). */
gdn_status gdn_prefill_set_marks(void *const *events, int32_t n_events);

/* Static description of a status code ("unknown status" for any other value). */
const char *gdn_status_string(gdn_status status);

/* Detail of the last failing call made by the calling thread ("" if none). */
const char *gdn_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* GDN_H */
