/*
 * gdn.h -- C ABI of libgdn, a Gated DeltaNet (GDN) state layer for AMD
 * Instinct MI355X (gfx950).
 *
 * The layer core is the gated delta rule over a depthwise causal
 * conv1d + SiLU front end:
 *     y      = silu(depthwise causal conv of the raw q|k|v channels)
 *     q^, k^ = per-head L2 normalisation of q, k (q^ also times q_scale)
 *     S_t    = a_t * S_{t-1} (I - b_t k^_t k^_t^T) + b_t v_t k^_t^T
 *     o_t    = S_t q^_t
 * with one fp32 [d_v, d_k] state per value head and request ("Plan
 * (research-based): Qwen3.6-35B-A3B", section "What the research found":
 * delta rule, full [V,K] state, chunked (I+A)^-1 UT-transform prefill).
 *
 * It runs over a pool of independent fixed-size request slots: an outer slot
 * dimension on the state cache and a slot index in every kernel (baseRT issue
 * #31, sections "Why this looks tractable" and "Scope note"); each slot holds
 * one conv window and one recurrent state per layer, a new request starts
 * from zero and chunked prefill carries the state from chunk to chunk
 * ("Project: adding the hybrid model Qwen3.5", table "What to do", row
 * "State").
 *
 * Conventions shared by every call
 * --------------------------------
 *  - Memory: the caller owns every device buffer (pool, inputs, outputs,
 *    workspace); the library never allocates device memory.  All pointers
 *    marked "device" are device pointers; index arrays (slot_ids, cu_seqlens,
 *    accept_len) are device arrays too, so calls never read them on the host
 *    (except in GDN_VALIDATE mode, below).
 *  - Streams: `stream` is a hipStream_t passed as void* (NULL = the null
 *    stream).  Every call only enqueues work on it and returns; nothing
 *    synchronises except gdn_pool_error and GDN_VALIDATE mode.  Calls are
 *    therefore safe to record into a HIP graph (no memset nodes are used).
 *  - Errors: a negative gdn_status means the call enqueued nothing and
 *    touched no memory.  Out-of-range slot ids found by a kernel (id >=
 *    n_slots) skip that entry and set a sticky device error word, read with
 *    gdn_pool_error.  A negative slot id marks a padding entry: skipped
 *    silently, its output rows are left unwritten.
 *  - Threads: a pool may be used from several host threads, but calls that
 *    touch the same slot must be ordered by the caller (same stream or
 *    events).  Slot ids within one call must be distinct; a duplicate is a
 *    data race (GDN_VALIDATE rejects it).
 *
 * Pool memory layout (part of the ABI: tests and checkpointing may read or
 * write a slot directly):
 *   state buffer, fp32, row-major
 *       [n_slots][n_layers][h_v][d_v][d_k]        (d_k contiguous)
 *   aux buffer:
 *       conv windows, io dtype, [n_slots][n_layers][conv_k-1][C_conv]
 *       (row 0 = oldest raw input; C_conv = 2*h_k*d_k + h_v*d_v channels in
 *       the order q heads | k heads | v heads, each head's d contiguous),
 *       then, at the next 256-byte boundary, a 256-byte meta block whose
 *       first int32 is the sticky device error word, then int32
 *       [n_slots][n_layers][h_k] counters of the low-batch decode path and
 *       the ring commit (zero between calls; zeroed by gdn_pool_create).
 *     With ring_len = L > 0 (see gdn_ring_verify), then, each at the next
 *     256-byte boundary: int32 [n_slots][n_layers] ring counts (tokens held,
 *     0..L), int32 [n_slots][n_layers] ring-commit counters (zero between
 *     calls), and fp32 ring records, one block per (slot, layer) of
 *     L*(h_k*d_k + h_v*d_v + 2*h_v) floats rounded up to a multiple of 64:
 *     k^ [L][h_k][d_k] (post conv, normalised), v [L][h_v][d_v] (post conv),
 *     a [L][h_v], b [L][h_v].
 *
 * Activations: per token, raw q, k are [h_k][d_k] and v is [h_v][d_v] in the
 * io dtype; a and b are [h_v] fp32, already activated (a in (0,1], b in
 * [0,1]).  Value head h reads q/k head h / (h_v/h_k).  Conv weights are fp32
 * [C_conv][conv_k]; tap conv_k-1 multiplies the current token.
 */
#ifndef GDN_H
#define GDN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct gdn_pool gdn_pool; /* opaque: host metadata + borrowed device pointers */

typedef int32_t gdn_status;
#define GDN_OK 0
#define GDN_ERR_INVALID_ARG (-1) /* null pointer, bad size or range */
#define GDN_ERR_UNSUPPORTED (-2) /* shape outside the compiled kernels */
#define GDN_ERR_BAD_INDEX (-3)   /* GDN_VALIDATE: slot id out of range or repeated */
#define GDN_ERR_WORKSPACE (-4)   /* prefill workspace too small */
#define GDN_ERR_HIP (-5)         /* a HIP runtime call failed */
#define GDN_ERR_RING (-6)        /* GDN_VALIDATE: a listed slot's verify ring is not empty */
#define GDN_ERR_HOST (-7)        /* host-side failure (e.g. GDN_VALIDATE cannot allocate its host copies) */

typedef int32_t gdn_dtype;
#define GDN_F32 0
#define GDN_BF16 1

/* flags */
#define GDN_VALIDATE 1u /* check device index arrays on the host (synchronises) */
/* Decode and verify always run the kernel with one workgroup per (entry,
 * q/k group) instead of the finer splits chosen by batch size and d_k.  The
 * results are bitwise the same; the flag exists so the kernels can be
 * checked against each other. */
#define GDN_GROUP_KERNEL 2u

typedef struct {
    int32_t n_slots;   /* >= 1 */
    int32_t n_layers;  /* >= 1 */
    int32_t h_k;       /* q/k heads, >= 1 */
    int32_t h_v;       /* value heads, a multiple of h_k */
    int32_t d_k;       /* head widths: d_k == d_v, one of 32, 64, 128 */
    int32_t d_v;
    int32_t conv_k;    /* conv taps, 2..8 */
    gdn_dtype io_dtype; /* GDN_F32 or GDN_BF16: q, k, v, outputs and windows */
    float q_scale;     /* multiplies the normalised q; 0 -> 1/sqrt(d_k) */
    float norm_eps;    /* eps in x/sqrt(|x|^2+eps); 0 -> 1e-6 */
    uint32_t flags;    /* GDN_VALIDATE | GDN_GROUP_KERNEL, or 0 */
    int32_t ring_len;  /* tokens of the verify ring per slot and layer, 0..24 (0: no ring) */
} gdn_pool_desc;

/* Bytes the caller must allocate for a pool with this descriptor: the fp32
 * state buffer and the aux buffer (conv windows + meta).  Both buffers must be
 * 256-byte aligned.  Returns INVALID_ARG / UNSUPPORTED for a bad descriptor.
 * The size is fixed by the slot count and the layer shapes alone, not by any
 * context length: a recurrent state does not grow with the sequence, and the
 * slot dimension is an outer dimension on it (baseRT issue #31, "Why this
 * looks tractable"). */
gdn_status gdn_pool_bytes(const gdn_pool_desc* desc, size_t* state_bytes, size_t* aux_bytes);

/* Create a pool over caller-owned device buffers sized by gdn_pool_bytes and
 * zero them on `stream`: every slot starts from zero state and window, as a
 * new request does ("Project: adding the hybrid model Qwen3.5", table "What
 * to do", row "State").  The buffers must outlive the pool.  *out receives a
 * host handle.  Returns INVALID_ARG for a null or misaligned buffer, HIP if
 * the zero fill cannot be enqueued (then no handle is returned). */
gdn_status gdn_pool_create(const gdn_pool_desc* desc, void* state_buf, void* aux_buf,
                           void* stream, gdn_pool** out);

/* Free the host handle (device buffers are the caller's). */
gdn_status gdn_pool_destroy(gdn_pool* pool);

/* Zero the state and conv window of every layer of the n listed slots, and
 * empty their verify rings (slot_ids: device int32[n]); a reused slot starts
 * from zero ("Project: adding the hybrid model Qwen3.5", table "What to do",
 * row "State"). */
gdn_status gdn_slot_reset(gdn_pool* pool, int32_t n, const int32_t* slot_ids, void* stream);

/* Copy the state, conv window and verify ring of every layer of slot
 * src_ids[i] to slot dst_ids[i] (device int32[n] each), bit for bit: a state is saved and
 * copied whole, e.g. from a prefill checkpoint into a new request's slot
 * ("Project: adding the hybrid model Qwen3.5", prefix-cache notes: cache hits
 * only where a state checkpoint was stored).  An entry with a negative id is
 * skipped.  Destinations must be distinct and must not be sources of the same
 * call (else the copies race; GDN_VALIDATE rejects it). */
gdn_status gdn_slot_copy(gdn_pool* pool, int32_t n, const int32_t* src_ids, const int32_t* dst_ids,
                         void* stream);

/* One decode token for each of n entries; entry i reads and writes slot
 * slot_ids[i] of layer `layer` (baseRT issue #31, "Why this looks tractable":
 * a slot index in the recurrence kernels).  With few entries the rows of each
 * state tile are spread over several workgroups; results are bitwise the
 * same either way.
 *   q, k    device io dtype [n][h_k][d_k]      raw (pre-conv) inputs
 *   v       device io dtype [n][h_v][d_v]
 *   a, b    device fp32 [n][h_v]
 *   conv_w  device fp32 [C_conv][conv_k]        this layer's conv weights
 *   out     device io dtype [n][h_v][d_v]       o = S q^ with the updated S
 *                                               (16-byte aligned)
 * The state and window of each listed slot advance by one token; every other
 * slot is left bitwise unchanged. */
gdn_status gdn_decode_step(gdn_pool* pool, int32_t layer, int32_t n, const int32_t* slot_ids,
                           const void* q, const void* k, const void* v, const float* a,
                           const float* b, const float* conv_w, void* out, void* stream);

/* Speculative verify: n_tok tokens (1..8) per entry run through the
 * recurrence in order, every position's output is written, and the slot keeps
 * the state and window reached after accept_len[i] tokens (0..n_tok; 0 leaves
 * the slot untouched).  No per-position state copies are stored ("Plan
 * (research-based)", sections "What the research found" and "Why >150 is
 * still reachable": the per-position state is the costly part of verify).
 * When acceptance is only known after sampling, call it twice: with
 * accept_len all 0 for the outputs (the slots stay as they are), then with the
 * sampled accept_len and out = NULL to commit (no outputs are written and
 * tokens past accept_len are not run); drafts never touch the slot until
 * they are accepted, as with the pages' output-only reconstruction.
 *   q, k       device io dtype [n][n_tok][h_k][d_k]
 *   v          device io dtype [n][n_tok][h_v][d_v]
 *   a, b       device fp32 [n][n_tok][h_v]
 *   accept_len device int32 [n]; values outside 0..n_tok are clamped
 *   out        device io dtype [n][n_tok][h_v][d_v] (16-byte aligned), or NULL
 * Each position's output is bitwise the output of the same number of
 * gdn_decode_step calls. */
gdn_status gdn_verify_step(gdn_pool* pool, int32_t layer, int32_t n, const int32_t* slot_ids,
                           int32_t n_tok, const void* q, const void* k, const void* v,
                           const float* a, const float* b, const float* conv_w,
                           const int32_t* accept_len, void* out, void* stream);

/* Workspace bytes for gdn_prefill_chunked with these sizes (an upper bound
 * that depends only on n_seq, total_tokens and chunk). */
gdn_status gdn_prefill_workspace_bytes(const gdn_pool* pool, int32_t n_seq, int64_t total_tokens,
                                       int32_t chunk, size_t* bytes);

/* Chunked prefill of n_seq packed sequences, sequence j = tokens
 * [cu_seqlens[j], cu_seqlens[j+1]) into slot slot_ids[j], starting from what
 * the slot holds (zero after reset, or an earlier chunk's state and window:
 * scheduler chunks carry over).  Inside a call each sequence is cut into
 * chunks of `chunk` tokens (16, 32 or 64) aligned to its start; each chunk is
 * solved in the (I+A)^-1 UT-transform form and the state is carried chunk to
 * chunk ("Plan (research-based)", "What the research found"; "Project: adding
 * the hybrid model Qwen3.5", "What to do", row "State").
 *   cu_seqlens device int32 [n_seq+1]: 0, non-decreasing, last = total_tokens
 *   slot_ids   device int32 [n_seq]
 *   q, k       device io dtype [total_tokens][h_k][d_k]
 *   v          device io dtype [total_tokens][h_v][d_v]
 *   a, b       device fp32 [total_tokens][h_v]
 *   out        device io dtype [total_tokens][h_v][d_v]
 *              (q, k, v and out must be 16-byte aligned: rows are read and
 *              written in 16-byte vectors)
 *   workspace  device, >= gdn_prefill_workspace_bytes, 256-byte aligned;
 *              scratch only, contents undefined afterwards
 * Zero-length sequences are no-ops.  A single sequence may be as long as
 * total_tokens allows (up to 2^31 - 1 tokens; output rows are addressed per
 * chunk with 64-bit bases).  Returns GDN_ERR_UNSUPPORTED for more than 4
 * value heads per q/k head (h_v/h_k > 4) or total_tokens >= 2^31. */
gdn_status gdn_prefill_chunked(gdn_pool* pool, int32_t layer, int32_t n_seq,
                               const int32_t* cu_seqlens, const int32_t* slot_ids,
                               int64_t total_tokens, int32_t chunk, const void* q, const void* k,
                               const void* v, const float* a, const float* b,
                               const float* conv_w, void* out, void* workspace,
                               size_t workspace_bytes, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc):
 * gdn_prefill_chunked with its workspace taken from a device array that the
 * library holds on every device it runs on, GDN_STATIC_SCRATCH_BYTES (64 MiB)
 * each, until the process ends.  The call itself allocates no device memory
 * (in GDN_VALIDATE mode the host-side index checks copy the index arrays to
 * host memory, as for every call).  Same arguments, layout and results as
 * gdn_prefill_chunked; returns GDN_ERR_WORKSPACE, enqueuing nothing, when
 * gdn_prefill_workspace_bytes(n_seq, total_tokens, chunk) exceeds
 * GDN_STATIC_SCRATCH_BYTES (e.g. about 1,900 tokens of one sequence with
 * h_k = 16, h_v = 32, d = 128, chunk 64).  All calls on one device share the
 * array, which keeps the last call's contents: calls that may overlap on one
 * device (different streams, no ordering between them) race and must be
 * serialised by the caller. */
#define GDN_STATIC_SCRATCH_BYTES ((size_t)64 << 20)
gdn_status gdn_prefill_chunked_static(gdn_pool* pool, int32_t layer, int32_t n_seq,
                                      const int32_t* cu_seqlens, const int32_t* slot_ids,
                                      int64_t total_tokens, int32_t chunk, const void* q,
                                      const void* k, const void* v, const float* a,
                                      const float* b, const float* conv_w, void* out,
                                      void* stream);

/* gdn_prefill_chunked that also stores state checkpoints inside the
 * sequences, for prefix caching (the pages: a cache hit is only possible
 * where a state checkpoint was stored, and a state is copied whole).
 *   ckpt_every    tokens between checkpoints, a positive multiple of `chunk`
 *                 (0: none; the call is then gdn_prefill_chunked)
 *   ckpt_offsets  device int32 [n_seq+1], from 0, non-decreasing: sequence j
 *                 owns checkpoint rows [ckpt_offsets[j], ckpt_offsets[j+1])
 *   ckpt_slots    device int32 [ckpt_offsets[n_seq]]: pool slots receiving them
 * Checkpoint m of sequence j is written to slot ckpt_slots[ckpt_offsets[j]+m]
 * for every m with (m+1)*ckpt_every <= its length and m below its row count:
 * layer `layer`'s state and conv window after its first (m+1)*ckpt_every
 * tokens, exactly what the sequence's own slot would hold had the sequence
 * ended there (within the prefill's tolerance).  A negative checkpoint slot
 * is skipped.  Checkpoint slots must differ from each other and from
 * slot_ids (GDN_VALIDATE checks).  GDN_VALIDATE also returns BAD_INDEX,
 * before reading ckpt_slots, when ckpt_offsets[n_seq] exceeds
 * total_tokens / ckpt_every + n_seq (more rows than any call can fill). */
gdn_status gdn_prefill_chunked_ckpt(gdn_pool* pool, int32_t layer, int32_t n_seq,
                                    const int32_t* cu_seqlens, const int32_t* slot_ids,
                                    int64_t total_tokens, int32_t chunk, const void* q,
                                    const void* k, const void* v, const float* a, const float* b,
                                    const float* conv_w, void* out, int32_t ckpt_every,
                                    const int32_t* ckpt_offsets, const int32_t* ckpt_slots,
                                    void* workspace, size_t workspace_bytes, void* stream);

/* Verify ring ("Plan (research-based): Qwen3.6-35B-A3B", section "What the
 * research found": an output-only reconstruction from a ring of recent
 * tokens with the chunked (I+A)^-1 form, the full state written only every
 * L tokens).  For pools created with ring_len = L > 0.  A slot's state tile
 * then holds the state as of its last flush, and the ring the post-conv
 * k^, v, a, b of the c <= L tokens committed since; the slot's logical state
 * is the tile advanced by those tokens (its conv window is always current).
 * The one-call path (gdn_decode_step, gdn_verify_step, gdn_prefill_*,
 * checkpoints) reads and writes the tile directly, so a slot must have an
 * empty ring when passed to it: call gdn_ring_flush first (GDN_VALIDATE
 * returns GDN_ERR_RING otherwise).  Reset empties a ring; copy copies it.
 *
 * gdn_ring_verify: outputs of n_tok draft tokens (1..8, ring_len + n_tok <=
 * 32) for each entry, as if they were decoded in order after the slot's
 * logical state; nothing in the pool is written, so it can be repeated.
 *   q, k     device io dtype [n][n_tok][h_k][d_k]   raw draft inputs
 *   v        device io dtype [n][n_tok][h_v][d_v]
 *   a, b     device fp32 [n][n_tok][h_v]
 *   out      device io dtype [n][n_tok][h_v][d_v]
 * Outputs match gdn_verify_step on the same logical state within the
 * chunked form's rounding (not bitwise). */
gdn_status gdn_ring_verify(gdn_pool* pool, int32_t layer, int32_t n, const int32_t* slot_ids,
                           int32_t n_tok, const void* q, const void* k, const void* v,
                           const float* a, const float* b, const float* conv_w, void* out,
                           void* stream);

/* gdn_ring_commit: after sampling, commit the first accept_len[i] (clamped to
 * 0..n_tok) of the same draft tokens (the same q, k, v, a, b as the verify
 * call).  The conv window advances by them and they join the ring; when the
 * ring would exceed ring_len, the ring and the accepted tokens are folded
 * into the state tile instead and the ring is emptied, so each fold covers
 * at least ring_len + 1 committed tokens.  An entry with accept_len 0 is left
 * untouched.  Slots whose ring holds tokens must not be given to the one-call
 * path before gdn_ring_flush. */
gdn_status gdn_ring_commit(gdn_pool* pool, int32_t layer, int32_t n, const int32_t* slot_ids,
                           int32_t n_tok, const void* q, const void* k, const void* v,
                           const float* a, const float* b, const float* conv_w,
                           const int32_t* accept_len, void* stream);

/* gdn_ring_flush: fold each listed slot's ring into its state tile and empty
 * it (no-op for empty rings); afterwards the tile is the logical state. */
gdn_status gdn_ring_flush(gdn_pool* pool, int32_t layer, int32_t n, const int32_t* slot_ids,
                          void* stream);

/* Input projection, the step in front of the conv ("baseRT issue #31",
 * section "Why this looks tractable": an input-projection kernel beside the
 * conv).  For n_tok tokens, y = x W^T over the hidden size (bf16 inputs, fp32
 * accumulation), written as the raw inputs of the other calls:
 *   x          device bf16 [n_tok][hidden] (16-byte aligned; hidden % 32 == 0)
 *   w          device bf16 [C_conv + 2*h_v][hidden] (16-byte aligned): rows
 *              are the output channels, q heads | k heads | v heads | h_v a
 *              logits | h_v b logits
 *   q, k       device io dtype [n_tok][h_k][d_k]   raw (pre-conv) inputs
 *   v          device io dtype [n_tok][h_v][d_v]
 *   a, b       device fp32 [n_tok][h_v]: a = exp(-softplus(y_a)),
 *              b = sigmoid(y_b)
 *   workspace  device, >= gdn_in_proj_workspace_bytes (0 for large n_tok),
 *              256-byte aligned; scratch only
 * The pool supplies the shapes only; no slot is read or written.  Returns
 * GDN_ERR_UNSUPPORTED when hidden is not a multiple of 32 or the operands
 * exceed 2 GiB. */
gdn_status gdn_in_proj_workspace_bytes(const gdn_pool* pool, int64_t n_tok, int32_t hidden,
                                       size_t* bytes);
gdn_status gdn_in_proj(gdn_pool* pool, int64_t n_tok, int32_t hidden, const void* x, const void* w,
                       void* q, void* k, void* v, float* a, float* b, void* workspace,
                       size_t workspace_bytes, void* stream);

/* Synchronise `stream`, then read and clear the sticky device error word
 * (0 = none; bit 0 = a slot id >= n_slots was skipped; bit 1 = a malformed
 * cu_seqlens was seen). */
gdn_status gdn_pool_error(gdn_pool* pool, void* stream, int32_t* device_error);

/* Static text for a status code. */
const char* gdn_status_string(gdn_status status);

#ifdef __cplusplus
}
#endif

#endif /* GDN_H */
