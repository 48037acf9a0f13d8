/*
 * gla.h -- C ABI of the gated linear-attention state recurrence on MI355X
 * (gfx950): GLA and Gated DeltaNet, chunked prefill and slot-indexed decode,
 * plus the short causal convolution that precedes the layer.
 *
 * Source of the computation: "Inference for linear attention and hybrid
 * architectures" (section "Two ways to write the same computation"):
 *
 *   GLA             S_t = a_t S_{t-1} + k_t^T v_t
 *   Gated DeltaNet  S_t = a_t (I - b_t k_t^T k_t) S_{t-1} + b_t k_t^T v_t
 *   output          o_t = q_t S_t            (state after the update)
 *
 * q_t, k_t are d_k row vectors, v_t is a d_v row vector, S is a d_k x d_v
 * fp32 state per head, a_t (alpha, the decay gate) and b_t (beta) are one
 * scalar per token per head.  There is no softmax, no normaliser and no
 * scale: callers pre-scale q.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Every pointer argument is a DEVICE pointer (hipMalloc'ed or a tensor's
 *    data) unless stated otherwise.  The library never allocates or frees
 *    device memory and keeps no pointer after a call returns.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *    Work is enqueued asynchronously; execution errors surface at the
 *    caller's next synchronisation, as for any HIP launch.
 *  - Arguments are validated on the host before anything is enqueued.  A
 *    negative return value means nothing was enqueued and no output, state
 *    slot or cache was touched.  GLA_EHIP reports a failed launch.
 *  - No global state: calls are re-entrant.  No C++ exception crosses the
 *    ABI.
 *  - Packed variable-length layout: token n of sequence b is row
 *    cu_seqlens[b] + n of the token-major arrays
 *        q, k   [n_tokens, n_heads, dk]    (in_dtype)
 *        v, o   [n_tokens, n_heads, dv]    (in_dtype / out_dtype)
 *        alpha, beta  [n_tokens, n_heads]  fp32
 *    cu_seqlens [n_seqs + 1] int32, non-decreasing, cu[0] = 0,
 *    cu[n_seqs] = n_tokens.  Empty sequences are allowed.
 *  - State pool [n_slots, n_heads, dk, dv] fp32, row-major (dv fastest).
 *    Sequence / request b reads its initial state from
 *    pool[slot_idx[b]] and writes its final state back to the same slot, in
 *    place.  Slots not named by slot_idx are never read or written.
 *    slot_idx entries must be distinct; an entry outside [0, n_slots)
 *    makes the kernels skip that sequence (its outputs are left as they
 *    were) instead of faulting.
 *  - Supported sizes: dk, dv in {16, 32, 64, 128}; chunk in {16, 32, 64}.
 *    dtypes: in_dtype, out_dtype in {GLA_F32, GLA_BF16}.  bf16 outputs are
 *    the fp32 result rounded to nearest even.
 *  - Parity contract: alpha in (0, 1] and finite, as the page states the
 *    gate ("Two ways to write the same computation"); results then match
 *    the fp64 recurrence within 1e-5 absolute for fp32 inputs and 3e-3 of
 *    the largest magnitude for bf16 inputs.  A gate below 2^-126, exactly 0
 *    (a complete reset) included, is accepted and taken as 2^-126: results
 *    stay finite, but the chunked form works with log2 alpha, and after such
 *    a gate inside a chunk fp32 keeps the running log decay (near -126) to
 *    about 2^-17, so fp32 results then carry up to ~5e-5 absolute error.
 *  - Preconditions (undefined results, not faults, if violated):
 *    alpha in [0, 1] and finite; beta >= 0 with beta |k|^2 <= 2; q/k/v/o
 *    do not overlap the pool.
 *    Token indices derived from cu_seqlens are clamped to [0, n_tokens),
 *    so a malformed cu_seqlens gives wrong results, never an out-of-bounds
 *    access.
 */
#ifndef GLA_MI355X_H
#define GLA_MI355X_H

#include <stddef.h>
#include <stdint.h>

#if defined(__GNUC__) || defined(__clang__)
#define GLA_API __attribute__((visibility("default")))
#else
#define GLA_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { GLA_F32 = 0, GLA_BF16 = 1 } gla_dtype;

enum {
    GLA_OK = 0,
    GLA_EPTR = -1,       /* a required pointer is NULL                        */
    GLA_ESHAPE = -2,     /* a size is negative, unsupported or inconsistent   */
    GLA_EDTYPE = -3,     /* unsupported dtype                                 */
    GLA_ECHUNK = -4,     /* unsupported chunk size                            */
    GLA_EWORKSPACE = -5, /* workspace missing or smaller than required        */
    GLA_EHIP = -6,       /* the HIP launch failed                             */
    GLA_ESCRATCH = -7    /* needs more than gla_chunk_fwd_noalloc's fixed scratch */
};

/* flags */
enum { GLA_ZERO_INIT = 1u };  /* ignore the pool's contents: S_0 = 0 */

/*
 * gla_chunk_fwd -- GLA prefill by the chunked algorithm ("Two ways to write
 * the same computation", the chunked form; chunks start at each sequence's
 * first token of this call and the last one may be partial).  Per chunk of
 * C tokens with g = running sum of log alpha inside the chunk:
 *   O = ((Q K^T) .* D) V + diag(exp g) Q S,   D_ij = exp(g_i - g_j) [j <= i]
 *   S <- exp(g_last) S + (diag(exp(g_last - g)) K)^T V
 * The initial state is pool[slot_idx[b]] (zeros with GLA_ZERO_INIT); the
 * final state is written back to that slot.  Splitting a prompt over
 * several calls that pass the state through the pool gives the same result
 * up to rounding ("Chunked prefill comes for free").
 * `o` is fully overwritten for tokens of sequences with a valid slot.
 * Requires workspace of gla_chunk_workspace_bytes() bytes (may be 0; NULL is
 * then accepted).  For bf16 inputs with d_k = d_v = 128 and C = 64 the
 * sequences are also cut into segments of whole chunks that run in
 * parallel: a first pass writes each segment's state contribution and total
 * decay to the workspace, and each segment folds its entry state from them
 * (the same hand-off of the state, inside one call; where sequences average
 * six or more segments, a scan forms the entry states once instead).
 * Contents of the workspace are scratch; it must not be shared by calls
 * that overlap.
 */
GLA_API int gla_chunk_fwd(const void* q, const void* k, const void* v, const float* alpha,
                  const int32_t* cu_seqlens, int32_t n_seqs, int32_t n_tokens,
                  int32_t n_heads, int32_t dk, int32_t dv, int32_t chunk,
                  gla_dtype in_dtype, gla_dtype out_dtype,
                  float* state_pool, int32_t n_slots, const int32_t* slot_idx,
                  uint32_t flags, void* o,
                  void* workspace, size_t workspace_bytes, void* stream);

/*
 * gla_chunk_fwd_noalloc -- gla_chunk_fwd for callers that cannot allocate
 * device memory (code being captured into a HIP graph, tight serving
 * loops, harnesses that forbid hipMalloc): the same arguments, results and
 * errors without the workspace.  The per-segment states go to a fixed
 * array of GLA_NOALLOC_SCRATCH_BYTES in each GPU's memory, owned by the
 * library and held until the process ends; the call allocates nothing.  A
 * call whose gla_chunk_workspace_bytes() exceeds that size returns
 * GLA_ESCRATCH with nothing enqueued (at 16 heads, d = 128, chunk 64 the
 * bound is 64 KiB + 516 B per (segment, head) with about n_tokens / 1024 +
 * n_seqs segments, so e.g. 40 sequences totalling 16384 tokens fit).  All
 * calls on one GPU share that array: calls that overlap in time on one
 * GPU (different streams, or host threads) race and give wrong results;
 * calls ordered on one stream do not.  The array's address on a device is
 * looked up the first time the call runs with that device current.
 */
#define GLA_NOALLOC_SCRATCH_BYTES (64u << 20)
GLA_API int gla_chunk_fwd_noalloc(const void* q, const void* k, const void* v,
                  const float* alpha, const int32_t* cu_seqlens, int32_t n_seqs,
                  int32_t n_tokens, int32_t n_heads, int32_t dk, int32_t dv, int32_t chunk,
                  gla_dtype in_dtype, gla_dtype out_dtype, float* state_pool,
                  int32_t n_slots, const int32_t* slot_idx, uint32_t flags, void* o,
                  void* stream);

/*
 * gdn_chunk_fwd -- Gated DeltaNet prefill, chunked.  Same contract as
 * gla_chunk_fwd plus beta [n_tokens, n_heads] fp32.  The page gives no
 * chunked form for DeltaNet (it only says the in-chunk corrections must be
 * written in matrix form); the one used is derived from the update: with
 * u_t = b_t (v_t - a_t k_t S_{t-1}) each step is a GLA step with value u_t,
 * and inside a chunk entered with state S
 *   (I + A) U = diag(b) V - diag(b exp g) K S,
 *   A_tj = b_t exp(g_t - g_j) (k_t . k_j) for j < t,
 * solved as U = T diag(b) V - (T diag(b exp g) K) S with T = (I + A)^-1,
 * followed by the GLA chunk formulas with U in place of V.
 * Requires workspace of gdn_chunk_workspace_bytes() bytes (may be 0).
 * For bf16 inputs with d_k = d_v = 128 and C = 64, each (sequence segment,
 * head) is one workgroup over all 128 state columns, and a sequence longer
 * than the segment length (about n_tokens * n_heads / 256 tokens, at least
 * 256) is cut into segments that run side by side: a first pass computes
 * each segment's state contribution and its d_k x d_k transition, a scan
 * over the segments forms every segment's entry state, and the second pass
 * produces the outputs (the state hand-off of "Chunked prefill comes for
 * free", used inside one call); in batches of at least 512 (sequence, head)
 * pairs the first segment of a cut sequence runs straight from the pool
 * state instead, next to the first pass.  That path multiplies fp16 operands with
 * fp32 accumulation, each fp32-derived operand scaled by a power of two
 * into fp16's range; it needs |q_i| |k_j| < 2^15 and |q|, |k| entries
 * below 2^15 (true for L2-normalised q and k) and gives results about 5e-4
 * (relative to the largest) from the exact ones on such inputs.
 */
GLA_API int gdn_chunk_fwd(const void* q, const void* k, const void* v, const float* alpha,
                  const float* beta,
                  const int32_t* cu_seqlens, int32_t n_seqs, int32_t n_tokens,
                  int32_t n_heads, int32_t dk, int32_t dv, int32_t chunk,
                  gla_dtype in_dtype, gla_dtype out_dtype,
                  float* state_pool, int32_t n_slots, const int32_t* slot_idx,
                  uint32_t flags, void* o,
                  void* workspace, size_t workspace_bytes, void* stream);

/*
 * gla_chunk_fwd_ckpt / gdn_chunk_fwd_ckpt -- the chunked prefills above,
 * also saving state checkpoints at block boundaries ("Prefix caching has to
 * be redone": a linear-attention state summarises its whole prefix, so a
 * prefix can be reused only at a position where a whole state was saved;
 * engines save one at every block boundary, or selectively).  Checkpoint j
 * of sequence b is the state after (j + 1) * ckpt_interval tokens of that
 * sequence in this call (counted from its first token in the call), written
 * to pool[ckpt_slots[b * ckpt_stride + j]] for every j < ckpt_stride with
 * (j + 1) * ckpt_interval <= its length.  ckpt_interval must be a positive
 * multiple of chunk (GLA_ECHUNK otherwise), so checkpoints fall on chunk
 * ends.  ckpt_slots [n_seqs, ckpt_stride] int32 in device memory; an entry
 * outside [0, n_slots) saves nothing.  Checkpoint slots must be distinct
 * and distinct from every slot_idx entry of the call.  ckpt_stride = 0
 * (ckpt_slots may then be NULL) is the plain call.  A saved state continues
 * exactly like the sequence it came from: a later call that starts from
 * it gives the results of the uncut prompt, up to rounding.
 */
GLA_API int gla_chunk_fwd_ckpt(const void* q, const void* k, const void* v, const float* alpha,
                  const int32_t* cu_seqlens, int32_t n_seqs, int32_t n_tokens,
                  int32_t n_heads, int32_t dk, int32_t dv, int32_t chunk,
                  gla_dtype in_dtype, gla_dtype out_dtype,
                  float* state_pool, int32_t n_slots, const int32_t* slot_idx,
                  uint32_t flags, int32_t ckpt_interval, const int32_t* ckpt_slots,
                  int32_t ckpt_stride, void* o,
                  void* workspace, size_t workspace_bytes, void* stream);
GLA_API int gdn_chunk_fwd_ckpt(const void* q, const void* k, const void* v, const float* alpha,
                  const float* beta,
                  const int32_t* cu_seqlens, int32_t n_seqs, int32_t n_tokens,
                  int32_t n_heads, int32_t dk, int32_t dv, int32_t chunk,
                  gla_dtype in_dtype, gla_dtype out_dtype,
                  float* state_pool, int32_t n_slots, const int32_t* slot_idx,
                  uint32_t flags, int32_t ckpt_interval, const int32_t* ckpt_slots,
                  int32_t ckpt_stride, void* o,
                  void* workspace, size_t workspace_bytes, void* stream);

/*
 * gdn_chunk_prep + gdn_chunk_run -- gdn_chunk_fwd in its two parts, for
 * callers that overlap the state-independent part with other work.
 * gdn_chunk_prep computes, into the workspace, what does not depend on the
 * state or on v: the per-sequence chunk offsets and order, and for every
 * (chunk, head) the inverse T = (I + A)^-1 (with diag(beta) and the decayed
 * scores P for bf16 inputs).  gdn_chunk_run then runs the serial chunk loop
 * and must get the same q, k, alpha, beta, cu_seqlens, sizes, in_dtype and
 * workspace, ordered after gdn_chunk_prep (same stream, or an event); v, the
 * pool and the outputs are only touched by gdn_chunk_run.  Together they give
 * exactly gdn_chunk_fwd's results.  Arguments as gdn_chunk_fwd.
 */
GLA_API int gdn_chunk_prep(const void* q, const void* k, const float* alpha, const float* beta,
                  const int32_t* cu_seqlens, int32_t n_seqs, int32_t n_tokens,
                  int32_t n_heads, int32_t dk, int32_t dv, int32_t chunk, gla_dtype in_dtype,
                  void* workspace, size_t workspace_bytes, void* stream);
GLA_API int gdn_chunk_run(const void* q, const void* k, const void* v, const float* alpha,
                  const float* beta,
                  const int32_t* cu_seqlens, int32_t n_seqs, int32_t n_tokens,
                  int32_t n_heads, int32_t dk, int32_t dv, int32_t chunk,
                  gla_dtype in_dtype, gla_dtype out_dtype,
                  float* state_pool, int32_t n_slots, const int32_t* slot_idx,
                  uint32_t flags, void* o,
                  void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes the chunked calls need for these sizes (an upper bound
 * that does not depend on the contents of cu_seqlens).  0 = none. */
GLA_API size_t gla_chunk_workspace_bytes(int32_t n_seqs, int32_t n_tokens, int32_t n_heads,
                                 int32_t dk, int32_t dv, int32_t chunk);
GLA_API size_t gdn_chunk_workspace_bytes(int32_t n_seqs, int32_t n_tokens, int32_t n_heads,
                                 int32_t dk, int32_t dv, int32_t chunk);

/*
 * gla_decode_step -- one GLA token per request, recurrent form ("Two ways
 * to write the same computation": the state is read once and updated by one
 * rank-one term; "Speculative decoding and PD disaggregation": batched
 * decode reads and writes each request's fixed pool slot).
 *   S = pool[slot_idx[r]];  S <- alpha_r S + k_r^T v_r;  o_r = q_r S;
 *   pool[slot_idx[r]] <- S          (in place)
 * q, k [n_req, n_heads, dk]; v, o [n_req, n_heads, dv]; alpha [n_req, n_heads].
 */
GLA_API int gla_decode_step(const void* q, const void* k, const void* v, const float* alpha,
                    int32_t n_req, int32_t n_heads, int32_t dk, int32_t dv,
                    gla_dtype in_dtype, gla_dtype out_dtype,
                    float* state_pool, int32_t n_slots, const int32_t* slot_idx,
                    void* o, void* stream);

/*
 * gdn_decode_step -- one Gated DeltaNet token per request, in place:
 *   p = k S;  u = beta (v - alpha p);  S <- alpha S + k^T u;  o = q S
 * (equal to alpha (I - beta k^T k) S + beta k^T v).  beta [n_req, n_heads].
 */
GLA_API int gdn_decode_step(const void* q, const void* k, const void* v, const float* alpha,
                    const float* beta,
                    int32_t n_req, int32_t n_heads, int32_t dk, int32_t dv,
                    gla_dtype in_dtype, gla_dtype out_dtype,
                    float* state_pool, int32_t n_slots, const int32_t* slot_idx,
                    void* o, void* stream);

/*
 * gla_decode_multi -- n_tok consecutive GLA tokens per request with the
 * state after every position kept, for speculative decoding ("Speculative
 * decoding and PD disaggregation": verifying draft tokens runs several
 * recurrence steps, and a rejected token's update must be undone, which for
 * a recurrent state means keeping the state of every position or replaying).
 * For request r, starting from S = pool[slot_idx[r]]:
 *   for j = 0 .. n_tok-1:
 *     S <- alpha[r,j] S + k[r,j]^T v[r,j];   o[r,j] = q[r,j] S;
 *     if 0 <= pos_slots[r*n_tok + j] < n_slots:  pool[pos_slots[r*n_tok + j]] <- S
 * pool[slot_idx[r]] is only read (unless pos_slots names it), so the
 * request's committed state survives a rejected draft.  After verifying
 * that a of the n_tok tokens are accepted, the caller makes
 * pos_slots[r*n_tok + a-1] the request's slot (or copies it back with
 * gla_state_copy); with a = 0 nothing changes.  A negative pos_slots entry
 * keeps no state for that position.
 * q, k [n_req, n_tok, n_heads, dk]; v, o [n_req, n_tok, n_heads, dv];
 * alpha [n_req, n_tok, n_heads] fp32; slot_idx [n_req]; pos_slots
 * [n_req, n_tok] int32 in device memory.  All slots named
 * by pos_slots must be distinct and distinct from the other requests'
 * slot_idx (a request may name its own slot).  With n_tok = 1 and
 * pos_slots = slot_idx this is gla_decode_step.
 *
 * The page's second way to roll back (replay the accepted updates instead
 * of keeping every position) is the same call twice: verify with every
 * pos_slots entry negative (the state is read once, nothing is written),
 * then, once a_r tokens are accepted, call again on those tokens with
 * pos_slots[r*n_tok + a_r - 1] = slot_idx[r] and every other entry
 * negative (the state after a_r tokens is written in place; a_r = 0 writes
 * nothing).  Per head that moves 64 KiB + 128 KiB of state instead of
 * 64 KiB + n_tok x 64 KiB, at the price of recomputing the accepted steps.
 */
GLA_API int gla_decode_multi(const void* q, const void* k, const void* v, const float* alpha,
                     int32_t n_req, int32_t n_tok, int32_t n_heads, int32_t dk, int32_t dv,
                     gla_dtype in_dtype, gla_dtype out_dtype,
                     float* state_pool, int32_t n_slots, const int32_t* slot_idx,
                     const int32_t* pos_slots, void* o, void* stream);

/*
 * gdn_decode_multi -- the Gated DeltaNet form of gla_decode_multi: per
 * position p = k S; u = beta (v - alpha p); S <- alpha S + k^T u; o = q S.
 * beta [n_req, n_tok, n_heads] fp32.
 */
GLA_API int gdn_decode_multi(const void* q, const void* k, const void* v, const float* alpha,
                     const float* beta,
                     int32_t n_req, int32_t n_tok, int32_t n_heads, int32_t dk, int32_t dv,
                     gla_dtype in_dtype, gla_dtype out_dtype,
                     float* state_pool, int32_t n_slots, const int32_t* slot_idx,
                     const int32_t* pos_slots, void* o, void* stream);

/*
 * gla_state_copy -- pool[dst_slots[i]] <- pool[src_slots[i]] (all heads) for
 * i < n_copy: commits an accepted speculative position into a fixed slot,
 * or gives a new request its own copy of a saved prefix state (section
 * "Prefix caching has to be redone": a state summarises the whole prefix,
 * so it is reused whole, at the position where it was saved, and each
 * request that continues from it needs a copy because decoding updates the
 * state in place).  src/dst_slots [n_copy]
 * int32, device memory.  A destination must not be the source of another
 * pair in the same call; pairs with a slot outside [0, n_slots) or with
 * src == dst are skipped.
 */
GLA_API int gla_state_copy(float* state_pool, int32_t n_slots, int32_t n_heads, int32_t dk,
                   int32_t dv, const int32_t* src_slots, const int32_t* dst_slots,
                   int32_t n_copy, void* stream);

/*
 * gla_slot_copy -- the same copy for any slot-strided buffer
 * [n_slots, slot_bytes] (16-byte aligned, slot_bytes a multiple of 16): the
 * normaliser pool of lin_attn_*, or the conv cache [n_slots, W-1, channels],
 * which a saved prefix needs together with its state (section "Prefix
 * caching has to be redone": the checkpoint there holds the states and the
 * conv cache).  gla_state_copy is gla_slot_copy with slot_bytes =
 * n_heads * dk * dv * 4.  Same skipping rules.
 */
GLA_API int gla_slot_copy(void* buf, size_t slot_bytes, int32_t n_slots,
                  const int32_t* src_slots, const int32_t* dst_slots, int32_t n_copy,
                  void* stream);

/*
 * lin_attn_chunk_fwd -- normalised kernelised linear attention, chunked
 * prefill (page "Long context, fast inference, smart decoding, and life
 * beyond attention", section "Linear attention: removing softmax entirely"
 * and its running-state listing).  With phi(x) = elu(x) + 1 elementwise:
 *   S_t = S_{t-1} + phi(k_t)^T v_t,   z_t = z_{t-1} + phi(k_t),
 *   o_t = phi(q_t) S_t / (phi(q_t) . z_t + eps)
 * (no gate; eps = 1e-6 on the page).  S starts from pool[slot_idx[b]] and
 * the normaliser z from norm_pool[slot_idx[b]] (both zero with
 * GLA_ZERO_INIT); both are written back in place.  norm_pool
 * [n_slots, n_heads, dk] fp32.  Other arguments and the layout as
 * gla_chunk_fwd (no alpha); eps >= 0 and finite (GLA_ESHAPE otherwise).
 * Requires workspace of lin_attn_chunk_workspace_bytes() bytes (may be 0):
 * for bf16 inputs with d_k = d_v = 128 and chunk 64 the sequences are cut
 * into segments as in gla_chunk_fwd, and each segment's sum of phi(k) is
 * handed on with its state; otherwise, for d_v > 32 (several 32-column
 * d_v tiles per head), it holds a copy of the entry normalisers taken
 * before the kernel runs, so that no tile reads a z another tile has
 * already replaced.  For bf16 inputs phi(q) and phi(k) are rounded to bf16
 * before the contractions.
 */
GLA_API int lin_attn_chunk_fwd(const void* q, const void* k, const void* v,
                  const int32_t* cu_seqlens, int32_t n_seqs, int32_t n_tokens,
                  int32_t n_heads, int32_t dk, int32_t dv, int32_t chunk,
                  gla_dtype in_dtype, gla_dtype out_dtype,
                  float* state_pool, float* norm_pool, int32_t n_slots,
                  const int32_t* slot_idx, uint32_t flags, float eps, void* o,
                  void* workspace, size_t workspace_bytes, void* stream);
GLA_API size_t lin_attn_chunk_workspace_bytes(int32_t n_seqs, int32_t n_tokens, int32_t n_heads,
                  int32_t dk, int32_t dv, int32_t chunk);

/*
 * lin_attn_decode_step -- one token per request of lin_attn_chunk_fwd's
 * recurrence, in place on pool[slot_idx[r]] and norm_pool[slot_idx[r]]:
 *   S <- S + phi(k)^T v;  z <- z + phi(k);  o = phi(q) S / (phi(q) . z + eps)
 * q, k [n_req, n_heads, dk]; v, o [n_req, n_heads, dv].
 */
GLA_API int lin_attn_decode_step(const void* q, const void* k, const void* v,
                  int32_t n_req, int32_t n_heads, int32_t dk, int32_t dv,
                  gla_dtype in_dtype, gla_dtype out_dtype,
                  float* state_pool, float* norm_pool, int32_t n_slots,
                  const int32_t* slot_idx, float eps, void* o, void* stream);

/*
 * causal_conv1d_fwd -- depthwise causal convolution of width W with a
 * per-request cache of the last W-1 inputs ("Two ways to write the same
 * computation", last paragraph; "The real model's ledger": an engine keeps
 * W-1 columns).  For sequence b with cache rows c = conv_cache[slot_idx[b]]
 * (zeros with GLA_ZERO_INIT) and xx = [c ; x_b]:
 *   y[t, ch] = sum_{i<W} w[ch, i] * xx[t + i, ch]     (w[:, W-1] = current token)
 * then conv_cache[slot_idx[b]] <- the last W-1 rows of xx.  No bias, no
 * activation.  x, y [n_tokens, channels] (dtype); w [channels, W] fp32;
 * conv_cache [n_slots, W-1, channels] (dtype).  W in {2, 3, 4}; channels a
 * multiple of 8.  x and y must not overlap.
 */
GLA_API int causal_conv1d_fwd(const void* x, const float* w, const int32_t* cu_seqlens,
                      int32_t n_seqs, int32_t n_tokens, int32_t channels, int32_t width,
                      void* conv_cache, int32_t n_slots, const int32_t* slot_idx,
                      uint32_t flags, void* y, gla_dtype dtype, void* stream);

/*
 * gla_hbm_probe -- measurement helper, not part of the recurrence: the HBM
 * traffic of one decode step (gla_decode_step / gdn_decode_step at d_k =
 * d_v = 128) without its arithmetic, to measure the read / write ceiling
 * that step runs against on the machine at hand.  Item (request r, head h)
 * is the 64 KiB block state_pool + (slot_idx[r] * n_heads + h) * 16384
 * floats, accessed with the decode kernel's pattern.  mode & 3 = 0: read
 * every block; 1: write zeros over every block (destroys those states); 2:
 * read each block and write the same bytes back in place (the pool is left
 * as it was); 3: as 2, with two items per workgroup and both blocks read
 * before either is written.  Loads and stores are nontemporal, unless bit 2
 * (loads) or bit 3 (stores) of mode asks for the default cache policy.
 * sink: 16 bytes of device memory that a read
 * may write (it never does for finite data).  Slots outside [0, n_slots)
 * are skipped.  dk = dv = 128 only (GLA_ESHAPE otherwise).
 */
GLA_API int gla_hbm_probe(int32_t mode, float* state_pool, int32_t n_req, int32_t n_heads,
                  int32_t dk, int32_t dv, int32_t n_slots, const int32_t* slot_idx,
                  void* sink, void* stream);

/* Static description of a status code. */
GLA_API const char* gla_status_string(int status);

/* Library version, "major.minor.patch". */
GLA_API const char* gla_version(void);

#ifdef __cplusplus
}
#endif

#endif /* GLA_MI355X_H */
