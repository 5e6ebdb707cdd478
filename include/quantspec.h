/*
 * quantspec.h -- C ABI of the hierarchical INT8 KV cache (QuantSpec) decode-attention library
 * for AMD Instinct MI355X (gfx950).
 *
 * What the library computes
 * -------------------------
 * A per-(layer, sequence, head) KV cache in two tiers:
 *
 *  - a quantized tier: every group of G tokens is quantized once to 8-bit codes with an
 *    asymmetric scale s and zero-point z per group (keys: one (s, z) per channel over the G
 *    tokens of the group; values: one (s, z) per token over its head_dim channels), and each
 *    8-bit code C8 is stored as two 4-bit planes, C8 = 16*C_U + C_L, with s and z shared by both
 *    planes.  [QuantSpec Guide (aifetchly), "1. Hierarchical Two-Level Quantization with
 *    Bit-Sharing" and the "Hierarchical Quantizer with Bit-Packing" listing; Pith review of
 *    arXiv:2502.10424, "What carries the argument" and Fig. 3; Fig. 7 and reference [128] for
 *    the channel-wise key / token-wise value axes.]
 *  - a full-precision fp16 tail: a ring of 2G slots made of two G-token halves that holds the
 *    most recent tokens unquantized until they are committed.  [Pith review, "What carries the
 *    argument" and "Core claim" (double full-precision buffer of size 2G); QuantSpec Guide,
 *    "3. Double Full-Precision Cache Buffer (CF1 and CF2)".]
 *
 * Two attention passes read the cache:
 *  - the draft pass reads only the upper plane C_U of the quantized tier (dequantized as
 *    ((16*C_U + draft_offset) - z) * s) plus the fp16 tail;  [QuantSpec Guide, "Upper 4-Bit
 *    Representation (Draft)" and unpack_for_draft in the quantizer listing.]
 *  - the verify pass reads both planes ((C8 - z) * s) plus the fp16 tail, for m = gamma+1 query
 *    tokens in one pass, causally masked inside the tail.  [QuantSpec Guide, "Lower 4-Bit
 *    Representation (Residual)" and the verification loop; Pith review, one-line read.]
 * Both passes split the context into chunks whose softmax partials are merged by their
 * log-sum-exp (Flash-Decoding style).  [Pith review, reference [128]: appendix E, compatibility of
 * the full-precision buffer with Flash Decoding.]
 *
 * Rejected speculative tokens are removed from the tail (qs_rollback) before they are ever
 * quantized; qs_flush quantizes the oldest G-token half of the tail once per G committed tokens.
 * [QuantSpec Guide, "Zero-Overhead Rollback" and "Periodic Group Quantization".]
 *
 * Conventions
 * -----------
 *  - Every call returns a qs_status.  Nothing throws across this boundary.
 *  - Every argument is validated before any state changes: on error the cache is unchanged and
 *    qs_last_error() describes the problem.
 *  - Pointers named d_* are device pointers (HBM of the current HIP device); pointers named h_*
 *    are host pointers.  The caller owns all device memory (the arena, q, k, v, out); the
 *    library owns only the host-side handle.  Device buffers must stay alive until the stream
 *    has executed the enqueued kernels.
 *  - `stream` is a hipStream_t passed as void* (NULL = the default stream).  Calls are
 *    asynchronous; all bookkeeping (lengths, ring head) lives on the host and is updated at
 *    enqueue time, so no call synchronizes with the device.  All calls on one cache must be
 *    ordered on one stream: they share the arena's split workspace.
 *  - A handle is not thread-safe; different handles may be used from different threads.
 *  - fp16 means IEEE binary16; fp32 means IEEE binary32.
 *
 * Supported shapes: group == 128, head_dim in {64, 128}, 1 <= gamma_max + 1 <= 16,
 * 1 <= batch <= QS_MAX_BATCH, max_ctx a positive multiple of group.
 */
#ifndef QUANTSPEC_H
#define QUANTSPEC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define QS_MAX_BATCH 64
#define QS_MAX_QUERIES 16

typedef enum {
  QS_OK = 0,
  QS_ERR_INVALID_ARG = 1, /* null pointer, out-of-range layer, unsupported shape, bad count  */
  QS_ERR_CAPACITY = 2,    /* append past the 2G-slot tail, or flush past max_ctx               */
  QS_ERR_STATE = 3,       /* rollback of more tokens than the tail holds, verify with m > nt,
                             attention over a sequence that holds no token                     */
  QS_ERR_BUFFER = 4,      /* arena null, misaligned or smaller than qs_arena_bytes()           */
  QS_ERR_DEVICE = 5       /* a HIP runtime call failed (message in qs_last_error)              */
} qs_status;

typedef struct qs_cache qs_cache; /* opaque host handle */

typedef struct {
  int32_t n_layers;     /* L >= 1                                                              */
  int32_t batch;        /* B, 1..QS_MAX_BATCH                                                  */
  int32_t n_heads;      /* H >= 1 (key/value heads; one query head per key/value head)         */
  int32_t head_dim;     /* D, 64 or 128                                                        */
  int32_t group;        /* G, must be 128; the tail ring holds 2G tokens                       */
  int32_t max_ctx;      /* quantized-token capacity per sequence, positive multiple of G       */
  int32_t gamma_max;    /* verify accepts m <= gamma_max + 1 queries; gamma_max + 1 <= 16      */
  int32_t draft_offset; /* constant added to 16*C_U by the draft dequantization: 8 or 0        */
  int32_t meta_fp16;    /* metadata format: 0 = fp32 (scale s, zero-point z), a code C stands
                           for s (C - z); 1 = fp16 (scale s, offset b = -s z), C stands for
                           s C + b (half the metadata bytes).  The codes are the same in both
                           formats (computed from the fp32 s and z); the fp16 pair is s and the
                           fp32 product -s z, each rounded to nearest-even fp16, an offset past
                           the fp16 range saturating at +-65504.  Storing b rather than z keeps
                           a degenerate group exact: its scale (clamped to 1e-8) rounds to 0
                           and b is the group's value.                                         */
  int32_t split_upper;  /* upper-plane layout: 0 = one 4-bit plane C_U; 1 = C_U = 4*C_T + C_M
                           stored as two 2-bit planes, the top bits C_T = C8 >> 6 and the
                           middle bits C_M = (C8 >> 4) & 3, so that a 2-bit draft
                           (qs_attend_draft_bits) reads C_T alone while the 4-bit draft and
                           verify read both (same bytes as layout 0).  Needs meta_fp16 = 0;
                           serves the host-mode and fused calls (not grouped queries or device
                           mode, which return QS_ERR_INVALID_ARG).                             */
} qs_config;

/* Byte offsets (from the arena base) and sizes of the arena sections.  Every section starts
 * on a 256-byte boundary.  The logical layout of each section, with T = max_ctx, NG = T / G:
 *
 *  uk, lk   u8  [L][B][H][T][D/2]      key planes, token-major rows.  Byte j of a token row
 *                                      holds channel 2j in bits 0-3 and channel 2j+1 in bits
 *                                      4-7 (uk: C_U = C8 >> 4, lk: C_L = C8 & 15).
 *  uv, lv   u8  [L][B][H][NG][2][D][G/4]  value planes: each group is stored as two halves
 *                                      of G/2 tokens, each channel-major.  Byte j of the row of
 *                                      channel d in half e holds token e*G/2 + 2j of the group
 *                                      in bits 0-3 and token e*G/2 + 2j + 1 in bits 4-7.
 *  split_upper = 1: within the (layer, sequence, head) stripe of uk (T*D/2 bytes) the first
 *                 half is the C_T plane and the second the C_M plane, each [T][D/4]; within
 *                 the stripe of uv (NG*D*G/2 bytes) likewise, each [NG][2][D][G/8].  A row of
 *                 either plane is made of 32-bit little-endian words, word w covering 16
 *                 entries 16w .. 16w+15 (channels of a key row, tokens of a value row): nibble
 *                 e of a C_T word holds C_T(16w + e) in bits 2-3 and C_T(16w + 8 + e) in bits
 *                 0-1; nibble e of a C_M word holds C_M(16w + e) in bits 0-1 and C_M(16w + 8 + e)
 *                 in bits 2-3.  lk, lv are as above.
 *  kmeta    f32 [L][B][H][NG][D][2]    key (scale, zero-point) per group and channel;
 *                                      meta_fp16: f16 [L][B][H][NG][D][2] (scale, offset).
 *  vmeta    f32 [L][B][H][T][2]        value (scale, zero-point) per token;
 *                                      meta_fp16: f16 [L][B][H][T][2] (scale, offset).
 *  tail_k,  f16 [L][B][H][2G][D]       fp16 tail ring.  Logical tail token i of a sequence
 *  tail_v                              lives in slot (head + i) mod 2G, head in {0, G}.
 *  work     --                         split-softmax workspace (library private).
 *  state    i32 [L][B][4] + 1          device-mode counters (nq, nt, head, unused) per layer
 *                                      and sequence, then the device-mode error word.
 */
typedef struct {
  size_t uk, lk, uv, lv, kmeta, vmeta, tail_k, tail_v, work, state;        /* offsets */
  size_t uk_bytes, uv_bytes, kmeta_bytes, vmeta_bytes, tail_bytes, work_bytes,
      state_bytes;                                                          /* per section */
  size_t total;                                                             /* = qs_arena_bytes */
} qs_layout;

/* Size in bytes of the device arena for `cfg` (0 if cfg is invalid). */
size_t qs_arena_bytes(const qs_config* cfg);

/* Fills *out with the arena's section offsets for `cfg`.  Host only. */
qs_status qs_arena_layout(const qs_config* cfg, qs_layout* out);

/* Creates a cache over the caller's arena (d_arena: device pointer, 256-byte aligned, at least
 * qs_arena_bytes(cfg) bytes).  Every sequence starts empty (nq = nt = 0, head = 0).  The arena
 * contents need not be initialised.  Host only: enqueues nothing. */
qs_status qs_cache_create(const qs_config* cfg, void* d_arena, size_t arena_bytes, qs_cache** out);

/* Frees the host handle (never the arena).  NULL is accepted. */
qs_status qs_cache_destroy(qs_cache* cache);

/* Appends n_b new tokens to the fp16 tail of every sequence b of `layer`:
 *   d_k, d_v : fp16 [B][n_max][H][D], row (b, i) is read for i < n_b.
 *   h_n      : host int32 [B] with 0 <= n_b <= n_max, or NULL for n_b = n_max.
 * Token i goes to logical tail position nt_b + i; then nt_b += n_b.
 * Errors: QS_ERR_CAPACITY if nt_b + n_b > 2G for any b.  [QuantSpec Guide,
 * append_speculative_token in the cache-manager listing; Pith review, "What carries the
 * argument": new tokens are absorbed by the full-precision buffer.] */
qs_status qs_append(qs_cache* cache, int32_t layer, const void* d_k, const void* d_v,
                    int32_t n_max, const int32_t* h_n, void* stream);

/* Bulk prefill ("quantize once"): appends a prompt of n_b tokens to every sequence b of
 * `layer`, with the result of append(G) + flush repeated floor(n_b / G) times followed by
 * append(n_b mod G), bit for bit (planes, metadata, tail slots and counters), in one launch:
 * the whole groups are quantized straight from the prompt, the rest goes to the tail.
 *   d_k, d_v : fp16 [B][n_max][H][D], rows (b, i) for i < n_b are read.
 *   h_n      : host int32 [B] with 0 <= n_b <= n_max, or NULL for n_b = n_max.
 * Then nq_b += G floor(n_b / G), head_b ^= G if floor(n_b / G) is odd, nt_b = n_b mod G.
 * Errors: QS_ERR_STATE if n_b > 0 and the tail of b is not empty (nt_b != 0);
 * QS_ERR_CAPACITY if nq_b + G floor(n_b / G) > max_ctx; QS_ERR_INVALID_ARG if n_max / G > 65534.
 * [QuantSpec Guide, "Core Architectural Blueprint" figure: the prefill context is quantized
 * once into the hierarchical cache; "Periodic Group Quantization" and the quantizer listing for
 * the per-group codes.] */
qs_status qs_prefill(qs_cache* cache, int32_t layer, const void* d_k, const void* d_v,
                     int32_t n_max, const int32_t* h_n, void* stream);

/* Drops the newest h_n_drop[b] tail tokens of every sequence b (nt_b -= h_n_drop[b]) of
 * `layer`, or of every layer when layer == -1.  h_n_drop: host int32 [B] (NULL drops nothing).
 * Quantized tokens are never rolled back: QS_ERR_STATE if h_n_drop[b] > nt_b.  Host only.
 * [QuantSpec Guide, "Zero-Overhead Rollback"; Pith review, "What carries the argument".] */
qs_status qs_rollback(qs_cache* cache, int32_t layer, const int32_t* h_n_drop);

/* Quantizes the oldest G tail tokens (one ring half) of every sequence b of `layer` (every
 * layer when layer == -1) whose nt_b >= max(G, min_tail): computes the key and value
 * (scale, zero-point) and 8-bit codes, splits each code into C_U and C_L, writes both planes
 * and the metadata (in the cache's format, see meta_fp16) at quantized position nq_b, then
 * nq_b += G, nt_b -= G, head_b ^= G.
 * Sequences below the threshold are left unchanged.  h_flushed: host int32 [B] (or NULL),
 * receives 1 for flushed sequences (of the last layer when layer == -1), else 0.
 * Must be called only when every tail token is committed.
 * Errors: QS_ERR_CAPACITY if a selected sequence has nq_b + G > max_ctx; QS_ERR_INVALID_ARG
 * if min_tail > 2G.  [QuantSpec Guide, "Periodic Group Quantization" and the quantizer
 * listing; Pith review, "What carries the argument" and Fig. 3.] */
qs_status qs_flush(qs_cache* cache, int32_t layer, int32_t min_tail, void* stream,
                   int32_t* h_flushed);

/* Speculative accept / correct (the step after the verify pass), for `batch` sequences:
 *   d_target_logits : fp32 [batch][gamma+1][vocab]  target scores at the gamma drafted
 *                     positions and one past them (p_i = softmax of row i)
 *   d_draft_logits  : fp32 [batch][gamma][vocab]    draft scores (q_i = softmax of row i)
 *   d_draft_tokens  : int32 [batch][gamma]          the drafted tokens x_i
 *   d_uniforms      : fp32 [batch][gamma+1]         u_0 .. u_{gamma-1} for the acceptance
 *                     tests, u_gamma for the sample; each in [0, 1)
 * Drafted token i is accepted iff u_i <= min(1, p_i(x_i) / (q_i(x_i) + 1e-8)), for i = 0, 1, ..
 * until the first rejection j (a token outside [0, vocab) is rejected); d_n_accepted[b]
 * receives j (gamma if all are accepted) and d_next_token[b] the token sampled with u_gamma by
 * inverse CDF in token order from (p_j - q_j)_+ normalised, or from p_gamma when all were
 * accepted (from p_j if the residual has vanished in rounding).  All arithmetic is fp32.
 * d_workspace: device memory of at least qs_spec_workspace_bytes(batch, gamma, vocab) bytes
 * (row statistics, the drafted tokens' logits and the rejection point's per-part sampling
 * totals; every value a call uses is written earlier in that call; calls that share one
 * workspace must be ordered on one stream); the outputs are device int32 [batch].  Asynchronous on `stream`; needs no
 * cache.  qs_spec_workspace_bytes returns 0 for arguments qs_spec_accept rejects.
 * Errors: QS_ERR_INVALID_ARG for a null pointer, batch outside 1..65535, gamma outside
 * 1..QS_MAX_QUERIES-1 or vocab outside 1..1048576; QS_ERR_BUFFER for a short workspace.
 * [QuantSpec Guide, "The Self-Speculative Verification Loop" listing: the acceptance test;
 * Pith review of arXiv:2502.10424, major comment 1 (VERIFY with min(1, p/q), CORRECT from the
 * normalised residual (p - q)_+) and minor comment 5 (the token after gamma acceptances from
 * p_{gamma+1}).] */
size_t qs_spec_workspace_bytes(int32_t batch, int32_t gamma, int32_t vocab);
qs_status qs_spec_accept(const float* d_target_logits, const float* d_draft_logits,
                         const int32_t* d_draft_tokens, const float* d_uniforms, int32_t batch,
                         int32_t gamma, int32_t vocab, void* d_workspace, size_t workspace_bytes,
                         int32_t* d_n_accepted, int32_t* d_next_token, void* stream);

/* qs_spec_accept for callers that cannot allocate (code under HIP graph capture, serving loops
 * or harnesses that forbid hipMalloc): the same step and arguments without the workspace,
 * which is instead a device array inside the library (one copy per GPU of 4 MiB = 4194304
 * bytes, held until the process ends; its device address is looked up once per GPU, with that
 * GPU current, on the first call there).  Allocates nothing, on the host or the device.  The
 * array is fully rewritten before it is read by every call, so nothing carries over between
 * calls; but all calls on one GPU share it, so calls whose kernels may overlap on one GPU (on
 * different streams, or from different threads without ordering) race: order them on one
 * stream.
 * Errors: as qs_spec_accept; QS_ERR_BUFFER if qs_spec_workspace_bytes(batch, gamma, vocab)
 * exceeds 4 MiB (e.g. batch 256, gamma 15, vocab 128256 fits: 3.2 MB); QS_ERR_DEVICE if the
 * array's address cannot be found. */
qs_status qs_spec_accept_static(const float* d_target_logits, const float* d_draft_logits,
                                const int32_t* d_draft_tokens, const float* d_uniforms,
                                int32_t batch, int32_t gamma, int32_t vocab, int32_t* d_n_accepted,
                                int32_t* d_next_token, void* stream);

/* Draft attention: one query per (sequence, head) over the upper plane of every quantized
 * token plus every tail token.
 *   d_q   : fp16 [B][H][D]      d_out : fp32 [B][H][D]
 *   out = softmax(sm_scale * q . k_j) weighted sum of v_j over all cached tokens j, with
 *   quantized k, v dequantized as ((16*C_U + draft_offset) - z) * s (fp16 metadata:
 *   s * (16*C_U + draft_offset) + b).
 * Errors: QS_ERR_STATE if a sequence holds no token.  [QuantSpec Guide, "Upper 4-Bit
 * Representation (Draft)"; Pith review, one-line read.] */
qs_status qs_attend_draft(qs_cache* cache, int32_t layer, const void* d_q, float sm_scale,
                          float* d_out, void* stream);

/* Verify attention: m queries per (sequence, head) over both planes of every quantized token
 * plus the tail, causally masked: query i sees every quantized token and tail positions
 * 0 .. nt_b - m + i (the last m tail tokens are the m verified tokens themselves).
 *   d_q   : fp16 [B][m][H][D]   d_out : fp32 [B][m][H][D]
 *   quantized k, v dequantized as (C8 - z) * s with C8 = 16*C_U + C_L (fp16 metadata:
 *   s * C8 + b).
 * Errors: QS_ERR_INVALID_ARG if m < 1 or m > gamma_max + 1; QS_ERR_STATE if m > nt_b.
 * [QuantSpec Guide, "Lower 4-Bit Representation (Residual)" and "3. The Self-Speculative
 * Verification Loop"; Pith review, one-line read.] */
qs_status qs_attend_verify(qs_cache* cache, int32_t layer, const void* d_q, int32_t m,
                           float sm_scale, float* d_out, void* stream);

/* Draft attention on the top `bits` bits of every code: the same call as qs_attend_draft with
 * quantized k, v dequantized as ((C8 with its low 8 - bits bits replaced by
 * draft_offset * 2^(4 - bits)) - z) * s.  bits = 4 is qs_attend_draft; bits = 2 reads only the
 * C_T plane of the split-upper layout: ((64*C_T + 4*draft_offset) - z) * s, 80 bytes per
 * quantized token-head at head_dim 128 against 144 for the 4-bit draft.
 *   d_q   : fp16 [B][H][D]      d_out : fp32 [B][H][D]
 * Errors: as qs_attend_draft; QS_ERR_INVALID_ARG if bits is not 2 or 4, or bits = 2 without
 * split_upper.  [Pith review of arXiv:2502.10424, "Editorial extensions" / "Reading between
 * the lines": the top k bits for the draft and all bits for the verifier, the paper using
 * k = 4; the replacement of the dropped bits carries the centring of QuantSpec Guide's
 * unpack_for_draft ("| 0x08" for k = 4) to every k.] */
qs_status qs_attend_draft_bits(qs_cache* cache, int32_t layer, const void* d_q, int32_t bits,
                               float sm_scale, float* d_out, void* stream);

/* Grouped queries: g query heads share each cached (key/value) head -- query head h*g + r
 * (r < g) attends over cached head h, so the cache holds H = n_heads heads and the queries
 * H*g.  The draft form takes one query per query head, d_q fp16 [B][H*g][D], d_out fp32
 * [B][H*g][D]; the verify form m per query head, d_q fp16 [B][m][H*g][D], d_out fp32
 * [B][m][H*g][D], with the causal tail mask of qs_attend_verify per query token.  The m*g query
 * columns of a (sequence, cached head) go through one pass over its planes (both passes use
 * MFMA; the draft reads only the upper planes, its lower nibbles being draft_offset), so the
 * cached bytes are read once per group of g query heads.
 * Errors: as qs_attend_draft / qs_attend_verify; QS_ERR_INVALID_ARG if g is outside 1..16 or
 * m*g > gamma_max + 1 (the split workspace holds gamma_max + 1 query columns per head).  A
 * wider verify splits into calls in token order, each after the append of its own tokens (the
 * causal mask then gives every token the same view of the tail as one call would).
 * [QuantSpec Guide, "Empirical Evaluation: QuantSpec Benchmark Results" (LLaMA-3.1-8B among the
 * evaluated models, whose key/value heads are shared by groups of query heads); the passes as
 * in qs_attend_draft / qs_attend_verify.] */
qs_status qs_attend_draft_gqa(qs_cache* cache, int32_t layer, const void* d_q, int32_t g,
                              float sm_scale, float* d_out, void* stream);
qs_status qs_attend_verify_gqa(qs_cache* cache, int32_t layer, const void* d_q, int32_t m,
                               int32_t g, float sm_scale, float* d_out, void* stream);

/* Append then attend, fused: the same result, ring contents and counters as qs_append(cache,
 * layer, d_k, d_v, n_max, h_n, stream) followed by qs_attend_draft(cache, layer, d_q, sm_scale,
 * d_out, stream), with no separate append launch -- the attention's tail work items read the
 * new tokens from d_k / d_v and write them to their ring slots as they attend over them.  The
 * verify form appends the m verified tokens themselves (d_k, d_v: fp16 [B][m][H][D]) and then
 * runs qs_attend_verify with m queries.  Validation (and errors) are those of the two verbs in
 * sequence, all made before anything changes.  [QuantSpec Guide, "3. Double Full-Precision
 * Cache Buffer (CF1 and CF2)" and the verification-loop listing: each drafted token's K/V
 * enters the buffer before the next draft step attends; Pith review, "What carries the
 * argument".] */
qs_status qs_append_attend_draft(qs_cache* cache, int32_t layer, const void* d_k,
                                 const void* d_v, int32_t n_max, const int32_t* h_n,
                                 const void* d_q, float sm_scale, float* d_out, void* stream);
qs_status qs_append_attend_verify(qs_cache* cache, int32_t layer, const void* d_k,
                                  const void* d_v, const void* d_q, int32_t m, float sm_scale,
                                  float* d_out, void* stream);

/* Host copies of the bookkeeping of `layer`: h_nq, h_nt, h_head are int32 [B] (any may be
 * NULL). */
qs_status qs_get_state(const qs_cache* cache, int32_t layer, int32_t* h_nq, int32_t* h_nt,
                       int32_t* h_head);

/* ---- Device mode: the bookkeeping in device memory -----------------------------------------
 * The same verbs with the counters (nq, nt, head) held in the arena's state section and
 * advanced by the device, so that their calls can be captured in a HIP graph and the graph
 * replayed round after round, with rollback counts that come from the device (the accept
 * step's d_n_accepted).  [QuantSpec Guide, "3. Double Full-Precision Cache Buffer (CF1 and
 * CF2)" and the verification-loop listing (commit, then roll back the speculative buffer);
 * Pith review, "What carries the argument".]
 *
 * qs_state_to_device copies the host counters into the state section, clears the error word
 * and switches the handle to device mode; qs_state_from_device copies the counters back,
 * writes the error word to *h_error (if not NULL) and switches back to host mode.  Both
 * synchronize with `stream` (the only calls that do).  In device mode the host verbs above
 * (and qs_get_state) return QS_ERR_STATE, and in host mode the _dev verbs do.
 *
 * The _dev verbs validate their arguments on the host (QS_ERR_INVALID_ARG) and enqueue kernels
 * only: no synchronization, no allocation, no memset.  Appends and rollbacks are applied to the
 * counters lazily: each is recorded on the handle as a pending operation of its layer (at most
 * 4; a fifth commits the list first), every later kernel of that layer applies the pending
 * ones, and they are committed to the state section by the next attention call on the layer
 * (its last kernel), qs_flush_dev, qs_commit_dev or qs_state_from_device.  A rollback's d_sub
 * must keep its values until then.  A sequence of calls captured in a graph for replay must
 * begin and end with nothing pending (end it with an attention call, qs_flush_dev or
 * qs_commit_dev for every layer it appended to or rolled back).
 * Conditions that depend on the counters are checked by the device: the affected sequence is
 * left unchanged and a bit is set in the error word at the commit (1: append past 2G;
 * 2: rollback count negative or past the tail; 4: flush past max_ctx; 8: attention over an
 * empty sequence, or verify with m > nt).  The outputs of a flagged attention call are
 * unspecified (finite or not).
 *
 * qs_append_dev: n tokens for every sequence (d_k, d_v fp16 [B][n][H][D]), 0 <= n <= 2G.
 * qs_rollback_dev: drops n - d_sub[b] tail tokens of sequence b (n tokens if d_sub is NULL) of
 *   `layer`, or of every layer when layer == -1; d_sub: device int32 [B].
 * qs_flush_dev: quantizes the oldest G tail tokens of every sequence with nt >= max(G,
 *   min_tail), as qs_flush.
 * qs_commit_dev: commits the pending operations of `layer` (every layer when layer == -1).
 * qs_attend_draft_dev / qs_attend_verify_dev: as the host verbs, over a fixed work plan sized
 *   for a full cache (every sequence at max_ctx), so that a captured call stays valid while
 *   the counters grow. */
qs_status qs_state_to_device(qs_cache* cache, void* stream);
qs_status qs_state_from_device(qs_cache* cache, void* stream, int32_t* h_error);
qs_status qs_append_dev(qs_cache* cache, int32_t layer, const void* d_k, const void* d_v,
                        int32_t n, void* stream);
qs_status qs_rollback_dev(qs_cache* cache, int32_t layer, int32_t n, const int32_t* d_sub,
                          void* stream);
qs_status qs_flush_dev(qs_cache* cache, int32_t layer, int32_t min_tail, void* stream);
qs_status qs_commit_dev(qs_cache* cache, int32_t layer, void* stream);
qs_status qs_attend_draft_dev(qs_cache* cache, int32_t layer, const void* d_q, float sm_scale,
                              float* d_out, void* stream);
qs_status qs_attend_verify_dev(qs_cache* cache, int32_t layer, const void* d_q, int32_t m,
                               float sm_scale, float* d_out, void* stream);

/* Message of the last error on this handle ("" if none).  Valid until the next call. */
const char* qs_last_error(const qs_cache* cache);

#ifdef __cplusplus
}
#endif

#endif /* QUANTSPEC_H */
