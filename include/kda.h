/*
 * kda.h - C ABI of the MI355X (gfx950) KDA state-recurrence library, libkda.so.
 *
 * The library implements the hot path of Kimi Delta Attention's recurrent
 * state as four GPU calls.  Per head the state S is a d_k x d_v fp32 matrix
 * and one token does
 *
 *     alpha = exp(g)      (g = log alpha, one value per key channel)
 *     beta  = sigmoid(b)  (b = beta logit, one value per head)
 *     u     = beta * (v - (Diag(alpha) S)^T k)
 *     S     = Diag(alpha) S + k u^T
 *     o     = S^T q
 *
 * Sources, by page title and section (the pages give structure, not code):
 *  [P1] "State semantics deep water: rollback, fork, replay consistency, TP
 *       state": sec. 1 (fixed-size per-head state), sec. 2 (rollback is an
 *       exact block copy), sec. 3 (fork copies the whole state, COW off),
 *       sec. 4 (sigmoid beta; chunk vs recurrent activation placement).
 *  [P2] SGLang PR #34820 summary: "Implementation breakdown" items 1-4 and the
 *       kda_backend.py / hybrid_linear_attn_backend.py / kda_prefill.py
 *       excerpts (fp32 track snapshot at a chunk index, one cast into the
 *       pool dtype, sync-free indexed copies, explicit error instead of a
 *       silently unwritten snapshot).
 *  [P3] vLLM PR #51855 summary: "Implementation breakdown" steps 1-5 (one
 *       checkpoint; fp32 correction u and key/raw-gate records; reverse-order
 *       non-recursive commit) and "Risks" item 1 (reject at call time what a
 *       kernel would otherwise trip over at run time).
 *
 * Conventions shared by every call
 *  - Every pointer except `stream` and the pool struct itself is a DEVICE
 *    pointer.  The caller owns all buffers; the library keeps no pointer
 *    after a call returns and holds no global mutable state (the one
 *    exception is kda_chunk_prefill_noalloc's static scratch, below).
 *  - Calls are asynchronous on `stream` (a hipStream_t; NULL = the default
 *    stream).  No call reads device memory back to the host, none allocates,
 *    and none synchronises, so all of them can be captured in a HIP graph.
 *  - Every condition checkable on the host (null pointers, negative counts,
 *    unsupported shapes or dtypes, a workspace that is too small) returns a
 *    non-zero kda_status before any launch and touches no device memory.
 *  - Conditions only the device can see (a slot index out of range, a
 *    snapshot chunk outside its sequence, accepted length outside [0, L],
 *    malformed cu_seqlens or track_ptr) set a bit in *dev_err (when dev_err
 *    is non-NULL, via atomic OR) and the offending item is skipped.  The
 *    caller clears *dev_err before the call if it wants a fresh word.
 *  - A dispatch holds at most 2^32 - 1 work-items, so each call bounds its
 *    launch grid on the host (KDA_ERR_UNSUPPORTED beyond it): prefill as
 *    stated there; verify n_req * H, rounded up to a multiple of 8,
 *    <= 8,388,607; commit and align commit n_req * H <= 16,777,215; copy
 *    ceil(slot bytes / 16 KiB) * n_pairs <= 16,777,215; conv update
 *    n_ops * n_tensors <= 16,777,215.
 *  - Every cast into a 16-bit output or pool is one round-to-nearest-even
 *    cast from an fp32 value held in registers.
 *  - Floating-point results are deterministic run to run.
 *
 * Layouts (row-major, innermost last):
 *  tokens (prefill):   q, k, g [T_total][H][d_k];  v, o [T_total][H][d_v];
 *                      b [T_total][H]
 *  speculative (verify): q, k, g [n_req][L][H][d_k]; v, o [n_req][L][H][d_v];
 *                      b [n_req][L][H]
 *  state pool:         [n_slots][H][d_v][d_k]  (per head, row v holds the
 *                      d_k entries S[0..d_k-1][v]; k is contiguous)
 *  records:            u_rec [n_req][H][L][d_v] fp32;
 *                      kg_rec [n_req][H][L][2*d_k]: key then raw gate g
 *
 * Built shapes: (d_k, d_v, chunk) = (128, 128, 64) with bf16 or fp16 inputs,
 * and (16, 16, 16) with fp32 inputs.  Pools may be fp32, fp16 or bf16.  The
 * verify and commit calls take d_k = d_v = 128 (other head sizes return
 * KDA_ERR_UNSUPPORTED); the copy call takes any shape whose slot is a
 * multiple of 16 bytes.
 */
#ifndef KDA_H
#define KDA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  KDA_OK = 0,
  KDA_ERR_INVALID_ARG = 1, /* null pointer, negative count, inconsistent sizes */
  KDA_ERR_UNSUPPORTED = 2, /* shape / dtype combination that is not built      */
  KDA_ERR_WORKSPACE = 3,   /* workspace missing or smaller than required       */
  KDA_ERR_LAUNCH = 4       /* the HIP runtime rejected a kernel launch         */
} kda_status;

typedef enum { KDA_F32 = 0, KDA_F16 = 1, KDA_BF16 = 2 } kda_dtype;

/* Bits of the `flags` argument of kda_chunk_prefill and kda_recurrent_verify.
 * KDA_QK_L2NORM: q and k arrive unnormalised and the kernel normalises each
 * (token, head) row over d_k, qhat = q / sqrt(sum q^2 + 1e-6) and likewise
 * k, computed in fp32 and rounded once (RNE) to in_dtype; the recurrence,
 * the outputs and verify's key record all use the rounded qhat, khat, so a
 * commit from the records replays exactly what verify computed.  This is
 * the per-head L2 normalisation of q and k that the single-layer and
 * varlen workloads specify, fused into the loads instead of a separate
 * pass.  Other bits are rejected with KDA_ERR_INVALID_ARG. */
#define KDA_QK_L2NORM 1u

/* Bits set in *dev_err by the kernels. */
#define KDA_DEV_ERR_SLOT 1u   /* a slot index outside [0, n_slots) (or -1 where not allowed) */
#define KDA_DEV_ERR_TRACK 2u  /* a snapshot chunk outside [0, floor(T_i / chunk)], or a bad track_ptr */
#define KDA_DEV_ERR_ACCEPT 4u /* an accepted length outside [0, L] */
#define KDA_DEV_ERR_SEQLEN 8u /* cu_seqlens decreasing, negative, or beyond total_tokens */
#define KDA_DEV_ERR_SHIFT 16u /* a conv-state shift outside [0, rows - keep] */
#define KDA_DEV_ERR_GATE 32u  /* a gate beyond the supported range (below): results not exact */

/* Supported gate range.  The chunked prefill scales keys by e^-Gamma, Gamma
 * being the cumulative log decay (sum of g) since the start of the chunk,
 * and rounds the result to the operand type: with |k| <= 1 elementwise that
 * stays finite while every chunk's cumulative log decay stays above about
 * -11 with fp16 inputs (65504 = e^11.09), about -88 with bf16 inputs, and
 * about -87 with fp32 inputs (chunk 16).  verify forms the same factor over
 * each block of 8 positions in fp32, finite while a block's summed gate stays
 * above about -88.  A chunk or block beyond that sets KDA_DEV_ERR_GATE in
 * *dev_err (its results are then not to be used); inside it the results meet
 * the usual bars.  The workloads' gates, g in [-0.1, -0.001], give at most
 * -6.4 per chunk. */

/* A slot-indexed state pool, passed by value.  base points to
 * n_slots * H * d_v * d_k elements of `dtype` (a kda_dtype value). */
typedef struct {
  void* base;
  int64_t n_slots;
  int32_t dtype;
  int32_t H;
  int32_t d_k;
  int32_t d_v;
} kda_pool;

/* Bytes of device workspace kda_chunk_prefill needs for these sizes
 * (an upper bound that depends only on the arguments).  *bytes is set on
 * KDA_OK.  Same shape checks as kda_chunk_prefill. */
kda_status kda_chunk_prefill_workspace(int32_t n_seqs, int64_t total_tokens, int32_t H,
                                       int32_t d_k, int32_t d_v, int32_t chunk,
                                       int32_t in_dtype, size_t* bytes);

/* Chunked prefill over packed variable-length sequences ([P2] items 1-2 and
 * the kda_prefill.py excerpt; serial steps = ceil(T_i / chunk), [P1] sec. 5).
 *
 * q, k, v, g, b   inputs in `in_dtype` (layouts above); o output, same dtype.
 * cu_seqlens      int32 [n_seqs + 1] token offsets, non-decreasing, last <= total_tokens.
 * sizes           total_tokens <= INT32_MAX, (total_tokens / chunk + n_seqs) * H
 *                 <= 16,777,215 and n_seqs * H, rounded up to a multiple of
 *                 8, <= 2,097,151 (the launch grids' work-item limit, see
 *                 the conventions), else KDA_ERR_UNSUPPORTED.
 * pool            state pool; pool.H, d_k, d_v must equal H, d_k, d_v.
 * init_slot       int32 [n_seqs]: slot holding the initial state of sequence
 *                 i (upcast exactly to fp32), or -1 for a zero state.
 * final_slot      int32 [n_seqs]: slot that receives the final state (one
 *                 RNE cast), or -1 for none.  It may equal the sequence's own
 *                 init_slot; every other written slot must be distinct from
 *                 every slot read or written in the call.
 * track_ptr       int32 [n_seqs + 1] CSR offsets into track_chunk/track_slot
 *                 (may be NULL when n_track == 0).  Entry e of sequence i asks
 *                 for the state after track_chunk[e] full chunks of that
 *                 sequence, 0 <= track_chunk[e] <= floor(T_i / chunk): taken
 *                 straight from the fp32 accumulator, written to
 *                 track_f32[e] (fp32 [n_track][H][d_v][d_k], optional) and,
 *                 unless track_slot[e] == -1, cast once into that pool slot.
 * flags           0 or KDA_QK_L2NORM (q and k normalised inside the kernel).
 * dev_err         optional device word for the KDA_DEV_ERR_* bits.
 * workspace       device scratch of at least kda_chunk_prefill_workspace()
 *                 bytes, 256-byte aligned; its contents need no initialisation.
 */
kda_status kda_chunk_prefill(const void* q, const void* k, const void* v, const void* g,
                             const void* b, int32_t in_dtype, void* o,
                             const int32_t* cu_seqlens, int32_t n_seqs, int64_t total_tokens,
                             int32_t H, int32_t d_k, int32_t d_v, int32_t chunk, kda_pool pool,
                             const int32_t* init_slot, const int32_t* final_slot,
                             const int32_t* track_ptr, const int32_t* track_chunk,
                             const int32_t* track_slot, int32_t n_track, float* track_f32,
                             uint32_t flags, int32_t* dev_err, void* workspace,
                             size_t workspace_bytes, void* stream);

/* Allocation-free variant of kda_chunk_prefill, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc.  Same arguments, layouts, checks
 * and results as kda_chunk_prefill, without the workspace: the chunk map and
 * records live in a static device array of the library,
 * KDA_NOALLOC_SCRATCH_BYTES (256 MiB) per GPU, held by every GPU the
 * library runs on until the process ends (the single-layer workload,
 * 8229 tokens x 32 heads, takes 230 MB of it).  A call whose workspace
 * (kda_chunk_prefill_workspace) exceeds that returns KDA_ERR_WORKSPACE
 * before any launch.  The call allocates nothing; its first call on a
 * device resolves the array's address there (no allocation), so a caller
 * that captures graphs makes one call before capturing.  Every call on a
 * GPU shares that GPU's array and leaves its last contents there (nothing in
 * it needs to start at zero): calls that overlap on one GPU, from different
 * streams or threads, race on it and must be serialised by the caller. */
#define KDA_NOALLOC_SCRATCH_BYTES ((size_t)256 << 20)
kda_status kda_chunk_prefill_noalloc(const void* q, const void* k, const void* v, const void* g,
                                     const void* b, int32_t in_dtype, void* o,
                                     const int32_t* cu_seqlens, int32_t n_seqs, int64_t total_tokens,
                                     int32_t H, int32_t d_k, int32_t d_v, int32_t chunk, kda_pool pool,
                                     const int32_t* init_slot, const int32_t* final_slot,
                                     const int32_t* track_ptr, const int32_t* track_chunk,
                                     const int32_t* track_slot, int32_t n_track, float* track_f32,
                                     uint32_t flags, int32_t* dev_err, void* stream);

/* Speculative-decode verify ([P3] step 3): per request, read the checkpoint
 * in pool slot ckpt_slot[r] (never written), run the token recurrence over
 * the L positions with the gate activations applied inside the kernel, and
 * write
 *   o       [n_req][L][H][d_v] in in_dtype,
 *   u_rec   [n_req][H][L][d_v] fp32 correction u_t (beta folded in),
 *   kg_rec  [n_req][H][L][2*d_k] in in_dtype: key k_t then raw gate g_t
 *           (with KDA_QK_L2NORM in flags, the normalised key).
 * flags is 0 or KDA_QK_L2NORM (q and k normalised inside the kernel).
 * 1 <= L <= 256.  q, k, v, g, o, u_rec and kg_rec must be 16-byte aligned
 * (KDA_ERR_INVALID_ARG otherwise).  The outputs are stored non-temporally
 * (they are read by other kernels, not by this one).  A request whose ckpt_slot is outside
 * [0, n_slots) sets KDA_DEV_ERR_SLOT in *dev_err and its outputs are left
 * unwritten; the other requests are computed as usual. */
kda_status kda_recurrent_verify(const void* q, const void* k, const void* v, const void* g,
                                const void* b, int32_t in_dtype, void* o, int32_t n_req,
                                int32_t L, int32_t H, int32_t d_k, int32_t d_v, kda_pool pool,
                                const int32_t* ckpt_slot, float* u_rec, void* kg_rec,
                                uint32_t flags, int32_t* dev_err, void* stream);

/* RecoverSSM commit ([P3] step 4): rebuild, without re-running the
 * recurrence, the state after accepted_len[r] = n positions,
 *   S_n = Diag(e^{sum_{t<=n} g_t}) S_0 + sum_{t<=n} Diag(e^{sum_{t<s<=n} g_s}) k_t u_t^T,
 * accumulated in reverse order t = n..1, from the checkpoint in
 * ckpt_slot[r] and the records of a verify call; write it (one RNE cast) to
 * dst_slot[r] (dst_slot == NULL means in place, dst_slot[r] == ckpt_slot[r]
 * is allowed).  An in-place request with n == 0 touches nothing.  rec_dtype
 * is the dtype of kg_rec.  0 <= accepted_len[r] <= L <= 256.  Requests run
 * concurrently: the destination slots must be distinct from each other and
 * from every other request's checkpoint slot (a request may write over its
 * own checkpoint); otherwise the result is a data race.  A request with n
 * outside [0, L] sets KDA_DEV_ERR_ACCEPT, one with a slot outside
 * [0, n_slots) KDA_DEV_ERR_SLOT; either is skipped. */
kda_status kda_commit(kda_pool pool, const int32_t* ckpt_slot, const int32_t* dst_slot,
                      const int32_t* accepted_len, const float* u_rec, const void* kg_rec,
                      int32_t rec_dtype, int32_t n_req, int32_t L, int32_t H, int32_t d_k,
                      int32_t d_v, int32_t* dev_err, void* stream);

/* Align-mode commit ([P3] steps 4-5: the commit plan finds the accepted
 * length and the block boundary, the running block index moves on; the
 * review's check that the block size exceeds the speculative window).  The
 * state is kept per block of block_size tokens: the state after p tokens
 * lives in the slot of the block holding token p (1-based),
 * block_table[r * blocks_per_req + (p - 1) / block_size], and a block's slot
 * ends up holding the state at its last token.  Request r holds
 * p = num_tokens[r] >= 1 tokens; with n = accepted_len[r] (0..L) accepted
 * positions, b0 = (p - 1) / block_size and b1 = (p + n - 1) / block_size:
 *   b1 == b0: the state after p + n tokens -> slot of b0, in place (n = 0
 *             touches nothing);
 *   b1 == b0 + 1: the state after the m = b1 * block_size - p accepted
 *             tokens that close block b0 -> slot of b0 (when m > 0), and the
 *             state after p + n tokens -> slot of b1.
 * Both are rebuilt, as in kda_commit, from the checkpoint in b0's slot and
 * the records of a verify call (one RNE cast each).  block_size > L is
 * required (KDA_ERR_INVALID_ARG otherwise), so a window closes at most one
 * block.  A request with n outside [0, L] sets KDA_DEV_ERR_ACCEPT; one with
 * p < 1, b1 beyond its table row or a slot outside [0, n_slots) sets
 * KDA_DEV_ERR_SLOT; either is skipped.  The slots of different requests
 * must be distinct.  block_table, num_tokens, accepted_len: device arrays.
 *
 * Post-processing for the next step ([P3] step 4: the align post-process
 * moves the running block index on and resets the next step's copy bias to
 * neutral), in the same launch, into the device arrays of `next` (each
 * [n_req] int32, each optional: NULL fields are not written; none may alias
 * an input):
 *   num_tokens  p + n, the tokens the request holds after the commit (the
 *               next call's num_tokens);
 *   block       b1, the running block, whose slot holds the current state;
 *   ckpt_slot   block_table[r][b1], the checkpoint the next verify reads;
 *   copy_bias   0: the current state sits at the running block itself, so
 *               the next step copies from no offset.
 * A skipped request gets num_tokens = p, block = ckpt_slot = -1 (so a verify
 * from that slot flags KDA_DEV_ERR_SLOT instead of reading a stale state)
 * and copy_bias = 0. */
typedef struct {
  int32_t* num_tokens;
  int32_t* block;
  int32_t* ckpt_slot;
  int32_t* copy_bias;
} kda_align_next;

kda_status kda_commit_align(kda_pool pool, const int32_t* block_table, int32_t blocks_per_req,
                            const int32_t* num_tokens, const int32_t* accepted_len,
                            int32_t block_size, const float* u_rec, const void* kg_rec,
                            int32_t rec_dtype, int32_t n_req, int32_t L, int32_t H, int32_t d_k,
                            int32_t d_v, kda_align_next next, int32_t* dev_err, void* stream);

/* Rollback / fork ([P1] secs. 2-3; one launch for many slots as in the
 * fused slot copy of sec. 2): for every pair i, pool slot dst_slot[i]
 * receives the bits of slot src_slot[i].  Destinations must be distinct and
 * disjoint from the sources; src == dst is a no-op. */
kda_status kda_state_copy(kda_pool pool, const int32_t* src_slot, const int32_t* dst_slot,
                          int32_t n_pairs, int32_t* dev_err, void* stream);

/* One conv tensor (a short-convolution window of the state tuple) for
 * kda_conv_state_update.  Slot s, row r, channel c is the element at byte
 * base + s * slot_stride + (r * dim + c) * elem_bytes: per slot, `rows`
 * positions of `dim` channels, position-major; the first `keep` rows are
 * the history carried between steps (the convolution width minus one), the
 * rest an extended window's speculative positions.  Requirements (checked
 * on the host): base 16-byte aligned; slot_stride a multiple of 16 and at
 * least rows * dim * elem_bytes; 1 <= keep <= rows; elem_bytes 2 or 4 and
 * dim * elem_bytes a multiple of 16 (KDA_ERR_UNSUPPORTED otherwise). */
#define KDA_MAX_CONV_TENSORS 8
typedef struct {
  void* base;
  int64_t slot_stride;
  int64_t n_slots;
  int32_t rows;
  int32_t keep;
  int32_t dim;
  int32_t elem_bytes;
} kda_conv_tensor;

/* Fused conv-state update ([P1] sec. 2: the conv-state slots of many
 * tensors cleared or copied in one launch, the conv window moved by an
 * offset copy; [P3] steps 2 and 4: the extended window kept under
 * speculation and compacted to the accepted length at commit).
 * tensors: host array of n_tensors (1..KDA_MAX_CONV_TENSORS) descriptors,
 * read during the call only.  dst_slot, src_slot, shift: device arrays of
 * n_ops.  Op i applies to every tensor:
 *   src_slot[i] == -1: every row of slot dst_slot[i] becomes zero;
 *   otherwise rows [0, keep) of dst_slot[i] become rows
 *   [shift[i], shift[i] + keep) of src_slot[i]; rows >= keep of the
 *   destination are left as they were.  shift 0 copies the history (fork);
 *   src == dst with shift n compacts the window after n accepted positions.
 * Bits are copied, never converted.  The ops run concurrently: destinations
 * must be distinct, and no op may read a slot another op writes (an op may
 * read its own destination).  An op with a slot outside [0, n_slots) of
 * any tensor (or src < -1) sets KDA_DEV_ERR_SLOT, one with a shift outside
 * [0, rows - keep] of any tensor sets KDA_DEV_ERR_SHIFT; either way the op
 * is skipped for every tensor.  n_ops == 0 launches nothing. */
kda_status kda_conv_state_update(const kda_conv_tensor* tensors, int32_t n_tensors,
                                 const int32_t* dst_slot, const int32_t* src_slot,
                                 const int32_t* shift, int32_t n_ops, int32_t* dev_err,
                                 void* stream);

/* Static, NUL-terminated name of a status code. */
const char* kda_status_string(kda_status status);

#ifdef __cplusplus
}
#endif

#endif /* KDA_H */
