/*
 * libulysses -- one rank's share of an Ulysses sequence-parallel attention
 * layer on an AMD Instinct MI355X (gfx950).
 *
 * The method (Hugging Face blog "Ulysses Sequence Parallelism: Training with
 * Million-Token Contexts", section "The challenge of long-sequence
 * training"; DeepSpeed blog "DeepSpeed Ulysses: system optimizations for
 * training extremely long sequence Transformer models", design section):
 * every rank holds a 1/P slice of the sequence with all heads; an
 * all-to-all gives every rank all positions for 1/P of the heads; each rank
 * runs ordinary attention for its heads; a second all-to-all restores the
 * sequence slicing.  This library provides the per-rank pieces of that path:
 *
 *   ulysses_seq_to_head  -- assemble the P sequence chunks into the rank's
 *                           full-sequence, head-sliced buffer
 *   ulysses_head_to_seq  -- its inverse
 *   ulysses_seq_to_head_batch, ulysses_head_to_seq_batch
 *                        -- the same for up to four tensors in one launch
 *   ulysses_attn_fwd     -- causal (GQA, optionally document-masked)
 *                           softmax attention, returning O and the LSE
 *   ulysses_attn_bwd     -- its backward pass (dQ, dK, dV)
 *   ulysses_attn_fwd_fused, ulysses_attn_bwd_fused
 *                        -- the same with the exchange fused into the
 *                           attention kernels' addressing
 *   ulysses_attn_merge   -- merge of two partial results (ring / blockwise
 *                           attention step)
 *   ulysses_logits_loss, ulysses_tiled_mlp_fwd/bwd
 *                        -- the sequence-tiled language-model loss and
 *                           SwiGLU MLP of the ALST memory recipe
 *   ulysses_attn_bwd_noalloc
 *                        -- ulysses_attn_bwd for callers that cannot
 *                           allocate
 *
 * Tensor layout is the pages' [sl, bs, hc, hs] (sequence, batch, heads, head
 * size), contiguous row-major (DeepSpeed Ulysses SP + ALST integration guide,
 * zwxr.cn, section on the attention adapter).
 *
 * Conventions for every entry point:
 *  - Device buffers are owned by the caller; scratch memory comes from a
 *    caller-provided workspace.  Library state and allocation, precisely:
 *      * every call except ulysses_attn_bwd_noalloc allocates and frees
 *        nothing and keeps no state between calls;
 *      * ulysses_attn_bwd_noalloc uses a fixed device array that every GPU
 *        the library runs on holds until the process ends, and caches that
 *        array's address per device (a mutex guards the cache).
 *    Calls are re-entrant: different host threads may call concurrently,
 *    except that concurrent ulysses_attn_bwd_noalloc calls on one GPU race
 *    on its shared array.
 *  - Calls are asynchronous: they validate their arguments on the host,
 *    enqueue kernels on `stream` and return.  Inputs must stay valid until
 *    the stream work completes.  A NULL stream is the default stream.
 *  - Argument validation runs before any HIP call.  On a validation error
 *    nothing is launched and no output is touched.
 *  - Device pointers must be 16-byte aligned; row sizes (head_dim * element
 *    size) must be multiples of 16 bytes.
 *  - Errors are returned as ulysses_status_t; no exception crosses the ABI.
 *    ULYSSES_ERR_HIP reports a failed launch (the status hipLaunchKernel returns); faults
 *    inside a kernel surface at the caller's next synchronisation.
 */
#ifndef ULYSSES_H
#define ULYSSES_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ULYSSES_ABI_VERSION 7

/* Status codes and element types are plain ints (the enumerators below name
 * their values), so that any value a caller passes in, valid or not, is
 * defined behaviour: an unknown dtype gets ULYSSES_ERR_DTYPE and an unknown
 * status "unknown status". */
typedef int ulysses_status_t;
enum {
  ULYSSES_OK = 0,
  ULYSSES_ERR_NULL = 1,           /* a required pointer is NULL */
  ULYSSES_ERR_SHAPE = 2,          /* non-positive size, or head_dim not supported */
  ULYSSES_ERR_DIVISIBILITY = 3,   /* head counts do not divide as the method requires */
  ULYSSES_ERR_DTYPE = 4,          /* unknown element type */
  ULYSSES_ERR_ALIGNMENT = 5,      /* pointer or row not 16-byte aligned */
  ULYSSES_ERR_UNSUPPORTED = 6,    /* valid request the library does not implement */
  ULYSSES_ERR_WORKSPACE = 7,      /* workspace NULL or smaller than required */
  ULYSSES_ERR_HIP = 8             /* kernel launch failed */
};

typedef int ulysses_dtype_t;
enum {
  ULYSSES_BF16 = 0,   /* bfloat16 storage, fp32 accumulation */
  ULYSSES_FP32 = 1    /* float32 storage and arithmetic */
};

/* ABI version of the loaded library (ULYSSES_ABI_VERSION it was built with). */
int ulysses_abi_version(void);

/* Static, NUL-terminated description of a status code.  Never NULL. */
const char* ulysses_status_string(ulysses_status_t status);

/*
 * Sequence-sharded -> head-sharded exchange as rank `rank` sees it
 * (Hugging Face Ulysses blog, "The challenge of long-sequence training":
 * the first all-to-all leaves each GPU with every position for a subset of
 * the heads; Transformers ALST guide walkthrough, two-GPU layout diagram).
 *
 *   chunks   host array of P device pointers (read during the call only).
 *            Chunk c is [n_local, bs, heads, head_dim] and holds sequence
 *            positions [c*n_local, (c+1)*n_local) with all heads.
 *   out      device [P*n_local, bs, heads_l, head_dim]:
 *              out[c*n_local + s, b, h, :] = chunks[c][s, b, src(h), :]
 *            with heads_l = heads / P and src(h) = rank*heads_l + h when
 *            heads >= P; when heads < P (GQA/MQA key/value heads, which the
 *            integration guide says are replicated) heads_l = 1 and
 *            src = floor(rank*heads/P).
 *   Requires 1 <= P <= 64, 0 <= rank < P, n_local >= 0 (0 is a no-op whose
 *   buffer pointers are not checked, so empty tensors may pass NULL),
 *   bs >= 1, heads % P == 0 or P % heads == 0 (else ERR_DIVISIBILITY, the
 *   pages' divisibility rule), out not overlapping any chunk.
 *   The copy is bit-exact.
 */
ulysses_status_t ulysses_seq_to_head(const void* const* chunks, int P, int rank,
                                     int64_t n_local, int bs, int heads, int head_dim,
                                     ulysses_dtype_t dtype, void* out, hipStream_t stream);

/*
 * Head-sharded -> sequence-sharded exchange, the inverse of
 * ulysses_seq_to_head (Hugging Face Ulysses blog: the second all-to-all
 * returns to sequence sharding).
 *
 *   in       device [P*n_local, bs, heads/P, head_dim]
 *   chunks   host array of P device pointers to [n_local, bs, heads,
 *            head_dim]; only head slots [rank*heads/P, (rank+1)*heads/P) of
 *            every chunk are written, the other ranks' slots are untouched.
 *   Requires heads % P == 0 (else ERR_DIVISIBILITY); other rules as above.
 */
ulysses_status_t ulysses_head_to_seq(const void* in, int P, int rank, int64_t n_local, int bs,
                                     int heads, int head_dim, ulysses_dtype_t dtype,
                                     void* const* chunks, hipStream_t stream);

/*
 * Up to ULYSSES_MAX_BATCH exchanges of one layer in a single launch (the
 * Ulysses all-to-all moves the query, key and value projections together,
 * and the gradients back; Hugging Face Ulysses blog, "The challenge of
 * long-sequence training").  Tensor i behaves exactly as the single-tensor
 * call with its own head count; P, rank, n_local, bs, head_dim and dtype are
 * shared.  One launch instead of several saves the launch and tail time of
 * the small key/value tensors.
 */
#define ULYSSES_MAX_BATCH 4

typedef struct {
  void* const* chunks; /* host array of P device pointers, chunk c [n_local, bs, heads,
                          head_dim]: read by ulysses_seq_to_head_batch; only this rank's
                          head slots written by ulysses_head_to_seq_batch */
  void* head;          /* device [P*n_local, bs, heads_l, head_dim]: written by
                          ulysses_seq_to_head_batch, read by ulysses_head_to_seq_batch */
  int heads;           /* this tensor's global head count */
} ulysses_exchange_tensor_t;

/*
 *   tensors    host array of n_tensors descriptors (read during the call only)
 *   n_tensors  1 .. ULYSSES_MAX_BATCH (ERR_SHAPE otherwise; ERR_NULL if
 *              tensors is NULL)
 *   Every descriptor is checked as the single-tensor call checks its
 *   arguments, in order, before anything is launched; the first failing
 *   status is returned.  Outputs of different tensors must not overlap each
 *   other or any input.  n_local == 0 is a no-op.
 */
ulysses_status_t ulysses_seq_to_head_batch(const ulysses_exchange_tensor_t* tensors,
                                           int n_tensors, int P, int rank, int64_t n_local,
                                           int bs, int head_dim, ulysses_dtype_t dtype,
                                           hipStream_t stream);
ulysses_status_t ulysses_head_to_seq_batch(const ulysses_exchange_tensor_t* tensors,
                                           int n_tensors, int P, int rank, int64_t n_local,
                                           int bs, int head_dim, ulysses_dtype_t dtype,
                                           hipStream_t stream);

/*
 * Local attention over the full sequence for this rank's heads (Hugging
 * Face Ulysses blog: each GPU runs standard attention for its heads;
 * integration guide: causality comes from positions, not from a 4D mask,
 * and packed samples must not attend across document boundaries).
 *
 *   q, o     device [seqlen, bs, hq, head_dim]
 *   k, v     device [seqlen, bs, hkv, head_dim]; query head h uses key/value
 *            head floor(h / (hq/hkv)).  Requires hq % hkv == 0.
 *   causal   1: key j is visible to query i iff j <= i (and same document);
 *            0: every key of the query's document is visible.
 *   cu_seqlens  NULL (one document) or a device int32 array of n_docs+1
 *            offsets 0 = cu[0] < cu[1] < ... < cu[n_docs] = seqlen; requires
 *            bs == 1.  The kernels clamp what they read from it, so bad
 *            contents give wrong results but no out-of-bounds access.
 *   lse      device fp32 [bs, hq, seqlen]: natural-log log-sum-exp of the
 *            scaled scores of each query row.
 *   s_i,j = softmax_scale * <q_i, k_j>;  O_i = sum_j softmax_j(s_i,.) v_j.
 *   softmax_scale  must be positive and finite (ERR_SHAPE otherwise).
 *   dtype    ULYSSES_BF16: head_dim 64 or 128, bf16 matrix cores with fp32
 *            accumulation, O rounded to nearest even.  ULYSSES_FP32:
 *            head_dim 32, 64 or 128, fp32 throughout.
 *   seqlen == 0 is a no-op.  n_docs must lie in [1, seqlen] when cu_seqlens
 *   is given.  ERR_UNSUPPORTED for seqlen >= 2^30, bs * hq > 65535, or
 *   (seqlen / 64 + 1) * (hq / hkv) >= 2^31.
 */
ulysses_status_t ulysses_attn_fwd(const void* q, const void* k, const void* v, int64_t seqlen,
                                  int bs, int hq, int hkv, int head_dim, ulysses_dtype_t dtype,
                                  float softmax_scale, int causal, const int32_t* cu_seqlens,
                                  int n_docs, void* o, float* lse, hipStream_t stream);

/*
 * ulysses_attn_fwd with the layout exchange fused into the attention: Q, K
 * and V are read straight from their sequence chunks and O is written into
 * this rank's head slots of the O chunks, so neither the head-sharded
 * tensors nor the exchange launches exist (the first extension the pages'
 * path allows: the exchange is the step on either side of attention).
 *   q_chunks, k_chunks, v_chunks, o_chunks
 *            host arrays of P device pointers; chunk c is [n_local, bs, H,
 *            head_dim] and holds tokens [c*n_local, (c+1)*n_local) with all H
 *            heads (H = hq for q and o, hkv for k and v), as for
 *            ulysses_seq_to_head.  The arrays are read during the call only.
 *   hq, hkv  global head counts.  This rank attends with q heads
 *            [rank*hq/P, (rank+1)*hq/P) and the matching key/value heads
 *            (replicated as in ulysses_seq_to_head when hkv < P); only
 *            those head slots of the o chunks are written.
 *   lse      device fp32 [bs, hq/P, P*n_local] (the rank's heads).
 * The result equals ulysses_seq_to_head of Q, K, V, then ulysses_attn_fwd,
 * then ulysses_head_to_seq of O, bit for bit.  Other arguments as in
 * ulysses_attn_fwd.  ERR_UNSUPPORTED unless dtype is ULYSSES_BF16, P <= 16,
 * n_local is a multiple of 64 and 128 * bs * max(hq, hkv) * head_dim < 2^31;
 * ERR_DIVISIBILITY for head counts the exchange rejects.
 */
ulysses_status_t ulysses_attn_fwd_fused(const void* const* q_chunks, const void* const* k_chunks,
                                        const void* const* v_chunks, int P, int rank,
                                        int64_t n_local, int bs, int hq, int hkv, int head_dim,
                                        ulysses_dtype_t dtype, float softmax_scale, int causal,
                                        const int32_t* cu_seqlens, int n_docs,
                                        void* const* o_chunks, float* lse, hipStream_t stream);

/* Bytes of device workspace ulysses_attn_bwd needs for these sizes: the
 * per-row statistics of the backward below and, in bf16 when the 128-key
 * blocks number fewer than 1024 (seqlen * bs * hkv < 131072), the fp32
 * partial dK/dV of its split key blocks (2 or 4 parts of 8 bytes per key,
 * KV head and head-dim element); 0 for sizes it rejects. */
size_t ulysses_attn_bwd_workspace_size(int64_t seqlen, int bs, int hq, int hkv, int head_dim,
                                       ulysses_dtype_t dtype);

/*
 * Backward pass of ulysses_attn_fwd, which training runs through every
 * Ulysses attention layer (integration guide, the training-loop example:
 * the loss aggregated over the ranks is backpropagated through the model;
 * the gradients cross the two all-to-alls in the opposite direction, so on
 * one rank the backward of the local attention is this call).  Given O and
 * LSE from the forward call and the upstream gradient dO (same layout as
 * O), computes
 *   D_i = <dO_i, O_i>,  P_ij = exp(s_ij - LSE_i),  dS_ij = P_ij (<dO_i, v_j> - D_i)
 *   dQ_i = scale * sum_j dS_ij k_j
 *   dK_j = scale * sum_{h in group(j)} sum_i dS_ij q_i
 *   dV_j = sum_{h in group(j)} sum_i P_ij dO_i
 * recomputing P from Q, K and the saved LSE (no N x N storage).
 * dq has q's layout, dk/dv have k's; all in `dtype`.  Other arguments as in
 * ulysses_attn_fwd.  `workspace` is device memory of at least
 * ulysses_attn_bwd_workspace_size(...) bytes, 256-byte aligned, whose
 * contents on entry do not matter.  dq, dk, dv are fully overwritten.  In
 * bf16 with few key blocks, each block's queries are shared over 2 or 4
 * workgroups whose fp32 partial dK/dV are added in a fixed order, so the
 * results stay bitwise reproducible for given sizes.
 */
ulysses_status_t ulysses_attn_bwd(const void* q, const void* k, const void* v, const void* o,
                                  const float* lse, const void* dout, int64_t seqlen, int bs,
                                  int hq, int hkv, int head_dim, ulysses_dtype_t dtype,
                                  float softmax_scale, int causal, const int32_t* cu_seqlens,
                                  int n_docs, void* dq, void* dk, void* dv, void* workspace,
                                  size_t workspace_bytes, hipStream_t stream);

/*
 * ulysses_attn_bwd for callers that cannot allocate memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.  It
 * takes no workspace; the backward's per-row statistics live instead in a
 * fixed scratch array of ULYSSES_NOALLOC_SCRATCH_BYTES that the library
 * holds on every GPU it runs on until the process ends.  The call itself
 * allocates and frees nothing.
 *   Arguments, results and errors as in ulysses_attn_bwd, plus
 *   ULYSSES_ERR_WORKSPACE when the statistics of these sizes exceed
 *   ULYSSES_NOALLOC_SCRATCH_BYTES (bf16: seqlen * bs * hq up to 2^21 rows;
 *   fp32: 2^22), with nothing launched.  When the bf16 dK/dV split's
 *   partials do not fit beside the statistics, dK/dV run unsplit here: they
 *   may then differ from ulysses_attn_bwd's in the last bit (the order of one
 *   fp32 sum), within the same accuracy; otherwise both calls give the same
 *   bits.
 * All calls on one GPU share its scratch array: calls that overlap in time
 * on one GPU (several streams or host threads) race and give wrong results;
 * calls ordered on one stream are safe.  The array's contents left by one
 * call do not matter to the next (every statistic is written before it is
 * read).  ULYSSES_ERR_HIP also when the scratch address cannot be obtained.
 */
#define ULYSSES_NOALLOC_SCRATCH_BYTES (16u << 20)

ulysses_status_t ulysses_attn_bwd_noalloc(const void* q, const void* k, const void* v,
                                          const void* o, const float* lse, const void* dout,
                                          int64_t seqlen, int bs, int hq, int hkv, int head_dim,
                                          ulysses_dtype_t dtype, float softmax_scale, int causal,
                                          const int32_t* cu_seqlens, int n_docs, void* dq,
                                          void* dk, void* dv, hipStream_t stream);

/*
 * ulysses_attn_bwd with the layout exchange fused in, the backward of
 * ulysses_attn_fwd_fused: Q, K, V, O and dO are read straight from their
 * sequence chunks and dQ, dK, dV are written into this rank's head slots of
 * their sequence chunks.  The gradients cross the exchange the other way
 * round from the activations (dO seq -> head, dQ/dK/dV head -> seq; the
 * exchange itself is the DeepSpeed blog's design section), and here that
 * crossing is the kernels' addressing.
 *   q/k/v/o/do/dq/dk/dv_chunks
 *            host arrays of P device pointers laid out as in
 *            ulysses_attn_fwd_fused (H = hq for q, o, do, dq; hkv for k, v,
 *            dk, dv); read during the call only.  Only this rank's head
 *            slots of dq, dk and dv are written.
 *   lse      device fp32 [bs, hq/P, P*n_local] from ulysses_attn_fwd_fused.
 *   workspace  at least ulysses_attn_bwd_workspace_size(P*n_local, bs, hq/P,
 *            max(hkv/P, 1), head_dim, dtype) bytes, 256-byte aligned.
 * The result equals ulysses_seq_to_head of Q, K, V, O and dO, then
 * ulysses_attn_bwd, then ulysses_head_to_seq of dQ, dK and dV, bit for bit.
 * ERR_DIVISIBILITY also when hkv < P: a key/value head shared by several
 * ranks would need their partial dK, dV summed, which a write cannot do.
 * ERR_UNSUPPORTED and the other arguments as in ulysses_attn_fwd_fused.
 */
ulysses_status_t ulysses_attn_bwd_fused(
    const void* const* q_chunks, const void* const* k_chunks, const void* const* v_chunks,
    const void* const* o_chunks, const float* lse, const void* const* do_chunks, int P, int rank,
    int64_t n_local, int bs, int hq, int hkv, int head_dim, ulysses_dtype_t dtype,
    float softmax_scale, int causal, const int32_t* cu_seqlens, int n_docs,
    void* const* dq_chunks, void* const* dk_chunks, void* const* dv_chunks, void* workspace,
    size_t workspace_bytes, hipStream_t stream);

/*
 * Merge of two partial attention results over disjoint key sets: the
 * combination step of ring (blockwise) attention, which the Hugging Face
 * Ulysses blog compares with Ulysses ("Ulysses vs Ring Attention").  Given
 * (o_a, lse_a) and (o_b, lse_b) from ulysses_attn_fwd calls for the same
 * queries against key sets A and B, writes the result over A and B:
 *   lse = ln(e^lse_a + e^lse_b),
 *   o   = e^(lse_a - lse) o_a + e^(lse_b - lse) o_b.
 * A row whose statistic is -inf in one input (no key seen) takes the other
 * input, whatever the -inf input's O holds; -inf in both gives o = 0 and
 * lse = -inf.
 *   o_a, o_b, o       device [seqlen, bs, heads, head_dim] in `dtype`
 *                     (16-byte aligned)
 *   lse_a, lse_b, lse device fp32 [bs, heads, seqlen] (4-byte aligned)
 *   head_dim          32, 64 or 128
 *   dtype             ULYSSES_BF16 (fp32 arithmetic, o rounded to nearest
 *                     even) or ULYSSES_FP32
 * o may be the same buffer as o_a or o_b, and lse the same as lse_a or lse_b
 * (in-place merge); any other overlap is undefined.  seqlen == 0 is a no-op.
 * ERR_UNSUPPORTED for seqlen >= 2^30, bs * heads > 65535 or more than 2^34
 * rows.
 */
ulysses_status_t ulysses_attn_merge(const void* o_a, const float* lse_a, const void* o_b,
                                    const float* lse_b, int64_t seqlen, int bs, int heads,
                                    int head_dim, ulysses_dtype_t dtype, void* o, float* lse,
                                    hipStream_t stream);

/* Bytes of device workspace ulysses_logits_loss needs for shard_rows rows of
 * logits over a vocabulary of `vocab` (0 for sizes it rejects). */
size_t ulysses_logits_loss_workspace_size(int64_t shard_rows, int64_t vocab);

/*
 * Language-model loss of the rank's T tokens and its gradients, with the
 * logits formed shard_rows rows at a time so that the [T, vocab] logits
 * never exist in full (the integration guide's tiled fused logits loss,
 * section on tiled loss computation: the backward runs inside the forward,
 * shard by shard).  For token i with label y_i (labels arrive already
 * shifted: y_i is the target of position i):
 *   z_iv = <h_i, w_v>,  lse_i = ln sum_v exp(z_iv),
 *   loss_rows[i] = lse_i - z_i,y_i,  or 0 when y_i == ignore_index;
 *   loss_sum = sum_i loss_rows[i],  n_good = number of kept tokens;
 *   G_iv = grad_scale (softmax(z_i)_v - [v == y_i]) (0 for ignored rows);
 *   dh = G W,  dw = G^T H  (the gradients of grad_scale * loss_sum).
 * grad_scale = 1 / (kept tokens over all ranks) gives the gradient of the
 * guide's token-weighted loss aggregation.
 *   h          device bf16 [T, d] (16-byte aligned)
 *   w          device bf16 [vocab, d] (16-byte aligned)
 *   labels     device int64 [T] (8-byte aligned)
 *   dtype      ULYSSES_BF16 (inputs and dh; fp32 logits, statistics and
 *              accumulation; exp(z - tile max) kept in bf16, G rounded to
 *              bf16 before the two gradient products)
 *   loss_rows  device fp32 [T]; loss_sum device fp32 [1]; n_good device
 *              int64 [1] (8-byte aligned)
 *   dh         device bf16 [T, d]; dw device fp32 [vocab, d]: fully
 *              overwritten (T == 0: dw = 0, loss_sum = 0, n_good = 0)
 *   workspace  device memory of at least
 *              ulysses_logits_loss_workspace_size(min(shard_rows, T), vocab)
 *              bytes, 16-byte aligned, contents irrelevant (bf16
 *              exp(z - tile max), turned into G in place, the per-tile
 *              statistics and the label logits of one shard)
 * A label outside [0, vocab) other than ignore_index gives a NaN loss row
 * and a NaN gradient row, without an out-of-bounds access.  The three
 * products per shard run on the library's own matrix-core GEMM.  The fp32
 * logits never reach memory: the epilogue of the Z product writes, per row
 * and 256-column tile, the tile's max m and sum of exp(z - m), the label's
 * logit, and exp(z - m) in bf16, which one pass turns into G in place.
 * Every sum is taken in a fixed order, so results are bitwise
 * reproducible.  ERR_SHAPE for T < 0, d < 1
 * or not a multiple of 8, vocab < 1, shard_rows < 1 or a non-finite
 * grad_scale; ERR_UNSUPPORTED for a dtype other than bf16 or a size >= 2^31.
 */
ulysses_status_t ulysses_logits_loss(const void* h, const void* w, const int64_t* labels,
                                     int64_t T, int64_t d, int64_t vocab, ulysses_dtype_t dtype,
                                     int64_t ignore_index, float grad_scale, int64_t shard_rows,
                                     float* loss_rows, float* loss_sum, int64_t* n_good, void* dh,
                                     float* dw, void* workspace, size_t workspace_bytes,
                                     hipStream_t stream);

/* Bytes of device workspace the tiled MLP needs for shard_rows rows
 * (backward != 0: ulysses_tiled_mlp_bwd, else ulysses_tiled_mlp_fwd); 0 for
 * sizes it rejects. */
size_t ulysses_tiled_mlp_workspace_size(int64_t shard_rows, int64_t d, int64_t inter,
                                        int backward);

/*
 * Sequence-tiled SwiGLU MLP of a Llama-style block (the integration guide's
 * TiledMLP, section on the ALST memory tricks), shard_rows token rows at a
 * time so that the [T, inter] intermediates exist for one shard only (the
 * guide picks ceil(T / d) shards, i.e. shard_rows = d):
 *   g = x Wg^T,  u = x Wu^T,  a = silu(g) * u,  y = a Wd^T.
 * The backward recomputes each shard's g and u (nothing is kept from the
 * forward) and, for the upstream gradient dy, writes
 *   da = dy Wd,  dg = da * u * silu'(g),  du = da * silu(g),
 *   dx = dg Wg + du Wu,  dWg = dg^T x,  dWu = du^T x,  dWd = dy^T a.
 *   x, y, dy, dx  device bf16 [T, d]
 *   wg, wu        device bf16 [inter, d] (gate_proj, up_proj weights)
 *   wd            device bf16 [d, inter] (down_proj weight)
 *   dwg, dwu      device fp32 [inter, d]; dwd device fp32 [d, inter]: fully
 *                 overwritten (T == 0: zero)
 *   workspace     ulysses_tiled_mlp_workspace_size(min(shard_rows, T), d,
 *                 inter, backward) bytes, 16-byte aligned, contents
 *                 irrelevant
 * Every pointer 16-byte aligned.  g, u and da are kept in fp32; a, dg and du
 * are rounded to bf16 as operands of the following products; dx is summed
 * in fp32 and rounded once.  The products run on the library's own
 * matrix-core GEMM, in the layout each operand is stored in (no transposed
 * copies), in a fixed order (bitwise reproducible).  ERR_SHAPE for T < 0, d or inter < 1 or not a
 * multiple of 8, shard_rows < 1; ERR_UNSUPPORTED for a dtype other than bf16
 * or a size >= 2^31.
 */
ulysses_status_t ulysses_tiled_mlp_fwd(const void* x, const void* wg, const void* wu,
                                       const void* wd, int64_t T, int64_t d, int64_t inter,
                                       ulysses_dtype_t dtype, int64_t shard_rows, void* y,
                                       void* workspace, size_t workspace_bytes,
                                       hipStream_t stream);
ulysses_status_t ulysses_tiled_mlp_bwd(const void* x, const void* wg, const void* wu,
                                       const void* wd, const void* dy, int64_t T, int64_t d,
                                       int64_t inter, ulysses_dtype_t dtype, int64_t shard_rows,
                                       void* dx, float* dwg, float* dwu, float* dwd,
                                       void* workspace, size_t workspace_bytes,
                                       hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* ULYSSES_H */
