// C-ABI of libulysses: argument validation and dispatch to the kernels.
// Every check runs before the first HIP call, so a rejected call launches
// nothing and leaves every output untouched.  Contracts are stated in
// include/ulysses.h.
#include <cmath>

#include "ulysses.h"

#include <math.h>
#include <stdint.h>

#include "launch.h"

namespace {

using ulysses::AttnShape;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

int elem_size(ulysses_dtype_t dt) {
  switch (dt) {
    case ULYSSES_BF16: return 2;
    case ULYSSES_FP32: return 4;
    default: return 0;
  }
}

ulysses_status_t from_hip(hipError_t e) { return e == hipSuccess ? ULYSSES_OK : ULYSSES_ERR_HIP; }

// Shared checks of the exchange calls; fills the launch geometry.
ulysses_status_t check_exchange(const void* const* chunks, int P, int rank, int64_t n_local, int bs,
                                int heads, int head_dim, ulysses_dtype_t dtype, const void* headbuf,
                                bool to_head, ulysses::ChunkTable* table, int64_t* chunk_row_bytes,
                                int64_t* slot_bytes, int64_t* head_row_bytes) {
  if (chunks == nullptr) return ULYSSES_ERR_NULL;
  const int es = elem_size(dtype);
  if (es == 0) return ULYSSES_ERR_DTYPE;
  if (P < 1 || P > ulysses::kMaxChunks || rank < 0 || rank >= P || n_local < 0 || bs < 1 ||
      heads < 1 || head_dim < 1)
    return ULYSSES_ERR_SHAPE;
  if (to_head ? (heads >= P ? heads % P != 0 : P % heads != 0) : heads % P != 0)
    return ULYSSES_ERR_DIVISIBILITY;
  if (n_local == 0) return ULYSSES_OK;   // nothing is read or written
  if (headbuf == nullptr) return ULYSSES_ERR_NULL;
  for (int c = 0; c < P; ++c)
    if (chunks[c] == nullptr) return ULYSSES_ERR_NULL;
  if (((int64_t)head_dim * es) % 16 != 0 || !aligned16(headbuf)) return ULYSSES_ERR_ALIGNMENT;
  for (int c = 0; c < P; ++c)
    if (!aligned16(chunks[c])) return ULYSSES_ERR_ALIGNMENT;
  const int hl = heads >= P ? heads / P : 1;
  const int src0 = heads >= P ? rank * hl : (int)(((int64_t)rank * heads) / P);
  const int64_t row = (int64_t)head_dim * es;
  *chunk_row_bytes = (int64_t)heads * row;
  *slot_bytes = (int64_t)src0 * row;
  *head_row_bytes = (int64_t)hl * row;
  if ((uint64_t)n_local * (uint64_t)bs * (uint64_t)(*head_row_bytes / 16) >= (1ull << 32))
    return ULYSSES_ERR_UNSUPPORTED;
  for (int c = 0; c < P; ++c) table->ptr[c] = reinterpret_cast<uintptr_t>(chunks[c]);
  return ULYSSES_OK;
}

// Shared checks of the attention calls.
ulysses_status_t check_attn(int64_t seqlen, int bs, int hq, int hkv, int head_dim,
                            ulysses_dtype_t dtype, float scale, int causal, const int32_t* cu,
                            int n_docs, AttnShape* s) {
  if (elem_size(dtype) == 0) return ULYSSES_ERR_DTYPE;
  if (seqlen < 0 || bs < 1 || hq < 1 || hkv < 1) return ULYSSES_ERR_SHAPE;
  if (dtype == ULYSSES_BF16 ? (head_dim != 64 && head_dim != 128)
                            : (head_dim != 32 && head_dim != 64 && head_dim != 128))
    return ULYSSES_ERR_SHAPE;
  if (!(scale > 0.f) || !isfinite(scale)) return ULYSSES_ERR_SHAPE;
  if (hq % hkv != 0) return ULYSSES_ERR_DIVISIBILITY;
  if (cu != nullptr) {
    if (bs != 1 || n_docs < 1 || n_docs > seqlen) return ULYSSES_ERR_SHAPE;
    if (!aligned4(cu)) return ULYSSES_ERR_ALIGNMENT;
  }
  if ((int64_t)bs * hq > 65535) return ULYSSES_ERR_UNSUPPORTED;   // grid.y of the launches
  // The kernels count positions and 64-row query steps (over the heads of a
  // GQA group) in 32 bits.
  if (seqlen >= (int64_t(1) << 30) || (seqlen / 64 + 1) * (hq / hkv) >= (int64_t(1) << 31))
    return ULYSSES_ERR_UNSUPPORTED;
  s->N = seqlen;
  s->bs = bs;
  s->hq = hq;
  s->hkv = hkv;
  s->hd = head_dim;
  s->scale = scale;
  s->causal = causal ? 1 : 0;
  s->cu = cu;
  s->n_docs = cu ? n_docs : 0;
  return ULYSSES_OK;
}

// Checks of the fused (exchange-in-attention) calls shared by forward and
// backward: the chunk tables, the rank's head slices and the rank's
// attention shape.  Fills one SeqChunks per global head count.
ulysses_status_t check_fused(int P, int rank, int64_t n_local, int bs, int hq, int hkv,
                             int head_dim, ulysses_dtype_t dtype, float scale, int causal,
                             const int32_t* cu, int n_docs, AttnShape* s, int* q_head0,
                             int* kv_head0) {
  if (elem_size(dtype) == 0) return ULYSSES_ERR_DTYPE;
  if (P < 1 || rank < 0 || rank >= P || n_local < 0 || bs < 1 || hq < 1 || hkv < 1)
    return ULYSSES_ERR_SHAPE;
  if (hq % P != 0) return ULYSSES_ERR_DIVISIBILITY;
  if (hkv >= P ? hkv % P != 0 : P % hkv != 0) return ULYSSES_ERR_DIVISIBILITY;
  const int hq_l = hq / P;
  const int hkv_l = hkv >= P ? hkv / P : 1;
  ulysses_status_t st = check_attn(n_local * P, bs, hq_l, hkv_l, head_dim, dtype, scale, causal,
                                   cu, n_docs, s);
  if (st != ULYSSES_OK) return st;
  // bf16 tensor-core kernels only; 64-row tiles never straddle two chunks;
  // a tile's row offsets (64 rows of all heads) fit the copies' 32 bits.
  if (dtype != ULYSSES_BF16 || P > ulysses::kMaxFusedChunks || n_local % 64 != 0 ||
      64 * (int64_t)bs * (hq > hkv ? hq : hkv) * head_dim * 2 >= (int64_t(1) << 31))
    return ULYSSES_ERR_UNSUPPORTED;
  *q_head0 = rank * hq_l;
  *kv_head0 = hkv >= P ? rank * hkv_l : (int)((int64_t)rank * hkv / P);
  return ULYSSES_OK;
}

// Chunk table of one operand for the fused calls (pointers already checked).
ulysses::SeqChunks seq_chunks(const void* const* chunks, int P, int64_t n_local, int row_heads,
                              int head0) {
  ulysses::SeqChunks c{};
  for (int i = 0; i < P; ++i) c.chunk[i] = reinterpret_cast<uintptr_t>(chunks[i]);
  c.n = n_local;
  c.row_heads = row_heads;
  c.head0 = head0;
  c.tiles_per_chunk = ulysses::make_fastdiv((uint32_t)(n_local / 64 > 0 ? n_local / 64 : 1));
  return c;
}

// NULL or misaligned (16 bytes) entry in a host table of P chunk pointers.
ulysses_status_t check_table(const void* const* chunks, int P) {
  if (chunks == nullptr) return ULYSSES_ERR_NULL;
  for (int i = 0; i < P; ++i)
    if (chunks[i] == nullptr) return ULYSSES_ERR_NULL;
  for (int i = 0; i < P; ++i)
    if (!aligned16(chunks[i])) return ULYSSES_ERR_ALIGNMENT;
  return ULYSSES_OK;
}

ulysses_status_t exchange_batch(bool to_head, const ulysses_exchange_tensor_t* tensors, int n,
                                int P, int rank, int64_t n_local, int bs, int head_dim,
                                ulysses_dtype_t dtype, hipStream_t stream) {
  if (tensors == nullptr) return ULYSSES_ERR_NULL;
  if (n < 1 || n > ULYSSES_MAX_BATCH) return ULYSSES_ERR_SHAPE;
  ulysses::ExchangeTensor t[ULYSSES_MAX_BATCH];
  for (int i = 0; i < n; ++i) {
    t[i] = ulysses::ExchangeTensor{};
    int64_t crb = 0, slot = 0, hrb = 0;
    const ulysses_status_t st =
        check_exchange(tensors[i].chunks, P, rank, n_local, bs, tensors[i].heads, head_dim, dtype,
                       tensors[i].head, to_head, &t[i].chunks, &crb, &slot, &hrb);
    if (st != ULYSSES_OK) return st;
    t[i].head_buf = static_cast<char*>(tensors[i].head);
    t[i].chunk_row_bytes = crb;
    t[i].slot_bytes = slot;
    t[i].head_row_bytes = hrb;
  }
  if (n_local == 0) return ULYSSES_OK;
  return from_hip(ulysses::launch_exchange_batch(to_head, t, n, P, n_local * bs, stream));
}

static_assert(ULYSSES_MAX_BATCH == ulysses::kMaxBatch, "batch limit");

}  // namespace

extern "C" {

int ulysses_abi_version(void) { return ULYSSES_ABI_VERSION; }

const char* ulysses_status_string(ulysses_status_t status) {
  switch (status) {
    case ULYSSES_OK: return "ok";
    case ULYSSES_ERR_NULL: return "required pointer is NULL";
    case ULYSSES_ERR_SHAPE: return "invalid or unsupported size";
    case ULYSSES_ERR_DIVISIBILITY: return "head counts not divisible as required";
    case ULYSSES_ERR_DTYPE: return "unknown element type";
    case ULYSSES_ERR_ALIGNMENT: return "pointer or row not 16-byte aligned";
    case ULYSSES_ERR_UNSUPPORTED: return "request not supported by the library";
    case ULYSSES_ERR_WORKSPACE: return "workspace missing or too small";
    case ULYSSES_ERR_HIP: return "HIP kernel launch failed";
  }
  return "unknown status";
}

ulysses_status_t ulysses_seq_to_head(const void* const* chunks, int P, int rank, int64_t n_local,
                                     int bs, int heads, int head_dim, ulysses_dtype_t dtype,
                                     void* out, hipStream_t stream) {
  ulysses::ChunkTable table{};
  int64_t crb, slot, hrb;
  ulysses_status_t st = check_exchange(chunks, P, rank, n_local, bs, heads, head_dim, dtype, out,
                                       true, &table, &crb, &slot, &hrb);
  if (st != ULYSSES_OK) return st;
  if (n_local == 0) return ULYSSES_OK;
  return from_hip(ulysses::launch_exchange(true, table, P, static_cast<char*>(out),
                                           n_local * bs, crb, slot, hrb, stream));
}

ulysses_status_t ulysses_head_to_seq(const void* in, int P, int rank, int64_t n_local, int bs,
                                     int heads, int head_dim, ulysses_dtype_t dtype,
                                     void* const* chunks, hipStream_t stream) {
  ulysses::ChunkTable table{};
  int64_t crb, slot, hrb;
  ulysses_status_t st = check_exchange(chunks, P, rank, n_local, bs, heads, head_dim, dtype, in,
                                       false, &table, &crb, &slot, &hrb);
  if (st != ULYSSES_OK) return st;
  if (n_local == 0) return ULYSSES_OK;
  return from_hip(ulysses::launch_exchange(false, table, P, const_cast<char*>(static_cast<const char*>(in)),
                                           n_local * bs, crb, slot, hrb, stream));
}

ulysses_status_t ulysses_seq_to_head_batch(const ulysses_exchange_tensor_t* tensors,
                                           int n_tensors, int P, int rank, int64_t n_local,
                                           int bs, int head_dim, ulysses_dtype_t dtype,
                                           hipStream_t stream) {
  return exchange_batch(true, tensors, n_tensors, P, rank, n_local, bs, head_dim, dtype, stream);
}

ulysses_status_t ulysses_head_to_seq_batch(const ulysses_exchange_tensor_t* tensors,
                                           int n_tensors, int P, int rank, int64_t n_local,
                                           int bs, int head_dim, ulysses_dtype_t dtype,
                                           hipStream_t stream) {
  return exchange_batch(false, tensors, n_tensors, P, rank, n_local, bs, head_dim, dtype, stream);
}

ulysses_status_t ulysses_attn_fwd(const void* q, const void* k, const void* v, int64_t seqlen,
                                  int bs, int hq, int hkv, int head_dim, ulysses_dtype_t dtype,
                                  float softmax_scale, int causal, const int32_t* cu_seqlens,
                                  int n_docs, void* o, float* lse, hipStream_t stream) {
  if (q == nullptr || k == nullptr || v == nullptr || o == nullptr || lse == nullptr)
    return ULYSSES_ERR_NULL;
  AttnShape s;
  ulysses_status_t st = check_attn(seqlen, bs, hq, hkv, head_dim, dtype, softmax_scale, causal,
                                   cu_seqlens, n_docs, &s);
  if (st != ULYSSES_OK) return st;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned4(lse))
    return ULYSSES_ERR_ALIGNMENT;
  if (seqlen == 0) return ULYSSES_OK;
  if (dtype == ULYSSES_BF16) return from_hip(ulysses::launch_attn_fwd_bf16(s, q, k, v, o, lse, stream));
  return from_hip(ulysses::launch_attn_fwd_f32(s, static_cast<const float*>(q),
                                               static_cast<const float*>(k),
                                               static_cast<const float*>(v), static_cast<float*>(o),
                                               lse, stream));
}

size_t ulysses_attn_bwd_workspace_size(int64_t seqlen, int bs, int hq, int hkv, int head_dim,
                                       ulysses_dtype_t dtype) {
  AttnShape s;
  if (check_attn(seqlen, bs, hq, hkv, head_dim, dtype, 1.0f, 1, nullptr, 0, &s) != ULYSSES_OK)
    return 0;
  return ulysses::attn_bwd_workspace_bytes(s, dtype == ULYSSES_BF16);
}

namespace {

// Argument checks shared by ulysses_attn_bwd and ulysses_attn_bwd_noalloc
// (everything but the workspace); fills *s.
ulysses_status_t check_attn_bwd(const void* q, const void* k, const void* v, const void* o,
                                const float* lse, const void* dout, int64_t seqlen, int bs, int hq,
                                int hkv, int head_dim, ulysses_dtype_t dtype, float softmax_scale,
                                int causal, const int32_t* cu_seqlens, int n_docs, const void* dq,
                                const void* dk, const void* dv, AttnShape* s) {
  if (q == nullptr || k == nullptr || v == nullptr || o == nullptr || lse == nullptr ||
      dout == nullptr || dq == nullptr || dk == nullptr || dv == nullptr)
    return ULYSSES_ERR_NULL;
  ulysses_status_t st = check_attn(seqlen, bs, hq, hkv, head_dim, dtype, softmax_scale, causal,
                                   cu_seqlens, n_docs, s);
  if (st != ULYSSES_OK) return st;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(dout) ||
      !aligned16(dq) || !aligned16(dk) || !aligned16(dv) || !aligned4(lse))
    return ULYSSES_ERR_ALIGNMENT;
  return ULYSSES_OK;
}

// The backward's launches, with a workspace that has passed its checks.
ulysses_status_t attn_bwd_launch(const AttnShape& s, ulysses_dtype_t dtype, const void* q,
                                 const void* k, const void* v, const void* o, const float* lse,
                                 const void* dout, void* dq, void* dk, void* dv, void* workspace,
                                 size_t workspace_bytes, hipStream_t stream) {
  if (dtype == ULYSSES_BF16)
    return from_hip(ulysses::launch_attn_bwd_bf16(s, q, k, v, o, lse, dout, dq, dk, dv, workspace,
                                                  workspace_bytes, stream));
  return from_hip(ulysses::launch_attn_bwd_f32(
      s, static_cast<const float*>(q), static_cast<const float*>(k), static_cast<const float*>(v),
      static_cast<const float*>(o), lse, static_cast<const float*>(dout), static_cast<float*>(dq),
      static_cast<float*>(dk), static_cast<float*>(dv), workspace, stream));
}

}  // namespace

ulysses_status_t ulysses_attn_bwd(const void* q, const void* k, const void* v, const void* o,
                                  const float* lse, const void* dout, int64_t seqlen, int bs,
                                  int hq, int hkv, int head_dim, ulysses_dtype_t dtype,
                                  float softmax_scale, int causal, const int32_t* cu_seqlens,
                                  int n_docs, void* dq, void* dk, void* dv, void* workspace,
                                  size_t workspace_bytes, hipStream_t stream) {
  AttnShape s;
  ulysses_status_t st = check_attn_bwd(q, k, v, o, lse, dout, seqlen, bs, hq, hkv, head_dim, dtype,
                                       softmax_scale, causal, cu_seqlens, n_docs, dq, dk, dv, &s);
  if (st != ULYSSES_OK) return st;
  const size_t need = ulysses::attn_bwd_workspace_bytes(s, dtype == ULYSSES_BF16);
  if (seqlen > 0 && (workspace == nullptr || workspace_bytes < need)) return ULYSSES_ERR_WORKSPACE;
  if (seqlen > 0 && !aligned16(workspace)) return ULYSSES_ERR_ALIGNMENT;
  if (seqlen == 0) return ULYSSES_OK;
  return attn_bwd_launch(s, dtype, q, k, v, o, lse, dout, dq, dk, dv, workspace, workspace_bytes,
                         stream);
}

ulysses_status_t ulysses_attn_bwd_noalloc(const void* q, const void* k, const void* v,
                                          const void* o, const float* lse, const void* dout,
                                          int64_t seqlen, int bs, int hq, int hkv, int head_dim,
                                          ulysses_dtype_t dtype, float softmax_scale, int causal,
                                          const int32_t* cu_seqlens, int n_docs, void* dq,
                                          void* dk, void* dv, hipStream_t stream) {
  AttnShape s;
  ulysses_status_t st = check_attn_bwd(q, k, v, o, lse, dout, seqlen, bs, hq, hkv, head_dim, dtype,
                                       softmax_scale, causal, cu_seqlens, n_docs, dq, dk, dv, &s);
  if (st != ULYSSES_OK) return st;
  // The statistics must fit the scratch; the dK/dV split's partials are
  // used only when they fit too.
  if (ulysses::attn_bwd_min_workspace_bytes(s, dtype == ULYSSES_BF16) >
      ulysses::noalloc_scratch_bytes())
    return ULYSSES_ERR_WORKSPACE;
  if (seqlen == 0) return ULYSSES_OK;
  void* scratch = nullptr;
  if (ulysses::noalloc_scratch(&scratch) != hipSuccess) return ULYSSES_ERR_HIP;
  return attn_bwd_launch(s, dtype, q, k, v, o, lse, dout, dq, dk, dv, scratch,
                         ulysses::noalloc_scratch_bytes(), stream);
}

ulysses_status_t ulysses_attn_merge(const void* o_a, const float* lse_a, const void* o_b,
                                    const float* lse_b, int64_t seqlen, int bs, int heads,
                                    int head_dim, ulysses_dtype_t dtype, void* o, float* lse,
                                    hipStream_t stream) {
  if (o_a == nullptr || lse_a == nullptr || o_b == nullptr || lse_b == nullptr || o == nullptr ||
      lse == nullptr)
    return ULYSSES_ERR_NULL;
  if (elem_size(dtype) == 0) return ULYSSES_ERR_DTYPE;
  if (seqlen < 0 || bs < 1 || heads < 1) return ULYSSES_ERR_SHAPE;
  if (head_dim != 32 && head_dim != 64 && head_dim != 128) return ULYSSES_ERR_SHAPE;
  if (seqlen >= (int64_t(1) << 30) || (int64_t)bs * heads > 65535 ||
      seqlen * bs * heads >= (int64_t(1) << 34))
    return ULYSSES_ERR_UNSUPPORTED;
  if (!aligned16(o_a) || !aligned16(o_b) || !aligned16(o) || !aligned4(lse_a) ||
      !aligned4(lse_b) || !aligned4(lse))
    return ULYSSES_ERR_ALIGNMENT;
  if (seqlen == 0) return ULYSSES_OK;
  return from_hip(ulysses::launch_attn_merge(dtype == ULYSSES_BF16, o_a, lse_a, o_b, lse_b, seqlen,
                                             bs, heads, head_dim, o, lse, stream));
}

ulysses_status_t ulysses_attn_fwd_fused(const void* const* q_chunks, const void* const* k_chunks,
                                        const void* const* v_chunks, int P, int rank,
                                        int64_t n_local, int bs, int hq, int hkv, int head_dim,
                                        ulysses_dtype_t dtype, float softmax_scale, int causal,
                                        const int32_t* cu_seqlens, int n_docs,
                                        void* const* o_chunks, float* lse, hipStream_t stream) {
  if (q_chunks == nullptr || k_chunks == nullptr || v_chunks == nullptr || o_chunks == nullptr ||
      lse == nullptr)
    return ULYSSES_ERR_NULL;
  AttnShape s;
  int q0 = 0, kv0 = 0;
  ulysses_status_t st = check_fused(P, rank, n_local, bs, hq, hkv, head_dim, dtype, softmax_scale,
                                    causal, cu_seqlens, n_docs, &s, &q0, &kv0);
  if (st != ULYSSES_OK) return st;
  for (const void* const* t : {q_chunks, k_chunks, v_chunks})
    if ((st = check_table(t, P)) != ULYSSES_OK) return st;
  if ((st = check_table(const_cast<const void* const*>(o_chunks), P)) != ULYSSES_OK) return st;
  if (!aligned4(lse)) return ULYSSES_ERR_ALIGNMENT;
  if (n_local == 0) return ULYSSES_OK;
  const ulysses::SeqChunks cq = seq_chunks(q_chunks, P, n_local, hq, q0);
  const ulysses::SeqChunks ck = seq_chunks(k_chunks, P, n_local, hkv, kv0);
  const ulysses::SeqChunks cv = seq_chunks(v_chunks, P, n_local, hkv, kv0);
  const ulysses::SeqChunks co =
      seq_chunks(const_cast<const void* const*>(o_chunks), P, n_local, hq, q0);
  return from_hip(ulysses::launch_attn_fwd_bf16_fused(s, cq, ck, cv, co, lse, stream));
}

ulysses_status_t ulysses_attn_bwd_fused(
    const void* const* q_chunks, const void* const* k_chunks, const void* const* v_chunks,
    const void* const* o_chunks, const float* lse, const void* const* do_chunks, int P, int rank,
    int64_t n_local, int bs, int hq, int hkv, int head_dim, ulysses_dtype_t dtype,
    float softmax_scale, int causal, const int32_t* cu_seqlens, int n_docs,
    void* const* dq_chunks, void* const* dk_chunks, void* const* dv_chunks, void* workspace,
    size_t workspace_bytes, hipStream_t stream) {
  if (q_chunks == nullptr || k_chunks == nullptr || v_chunks == nullptr || o_chunks == nullptr ||
      lse == nullptr || do_chunks == nullptr || dq_chunks == nullptr || dk_chunks == nullptr ||
      dv_chunks == nullptr)
    return ULYSSES_ERR_NULL;
  AttnShape s;
  int q0 = 0, kv0 = 0;
  ulysses_status_t st = check_fused(P, rank, n_local, bs, hq, hkv, head_dim, dtype, softmax_scale,
                                    causal, cu_seqlens, n_docs, &s, &q0, &kv0);
  if (st != ULYSSES_OK) return st;
  // A replicated KV head (hkv < P) would need its ranks' partial dK/dV summed
  // before it lands in the sequence chunks: not a plain write.
  if (hkv < P) return ULYSSES_ERR_DIVISIBILITY;
  for (const void* const* t : {q_chunks, k_chunks, v_chunks, o_chunks, do_chunks})
    if ((st = check_table(t, P)) != ULYSSES_OK) return st;
  for (void* const* t : {dq_chunks, dk_chunks, dv_chunks})
    if ((st = check_table(const_cast<const void* const*>(t), P)) != ULYSSES_OK) return st;
  if (!aligned4(lse)) return ULYSSES_ERR_ALIGNMENT;
  const size_t need = ulysses::attn_bwd_workspace_bytes(s, true);
  if (n_local > 0 && (workspace == nullptr || workspace_bytes < need)) return ULYSSES_ERR_WORKSPACE;
  if (n_local > 0 && !aligned16(workspace)) return ULYSSES_ERR_ALIGNMENT;
  if (n_local == 0) return ULYSSES_OK;
  auto table = [&](const void* const* t, int heads, int head0) {
    return seq_chunks(t, P, n_local, heads, head0);
  };
  auto out_table = [&](void* const* t, int heads, int head0) {
    return seq_chunks(const_cast<const void* const*>(t), P, n_local, heads, head0);
  };
  return from_hip(ulysses::launch_attn_bwd_bf16_fused(
      s, table(q_chunks, hq, q0), table(k_chunks, hkv, kv0), table(v_chunks, hkv, kv0),
      table(o_chunks, hq, q0), lse, table(do_chunks, hq, q0), out_table(dq_chunks, hq, q0),
      out_table(dk_chunks, hkv, kv0), out_table(dv_chunks, hkv, kv0), workspace,
      workspace_bytes, stream));
}

size_t ulysses_logits_loss_workspace_size(int64_t shard_rows, int64_t vocab) {
  if (shard_rows < 1 || vocab < 1 || shard_rows >= (int64_t(1) << 31) ||
      vocab >= (int64_t(1) << 31))
    return 0;
  return ulysses::logits_loss_workspace_bytes(shard_rows, vocab);
}

ulysses_status_t ulysses_logits_loss(const void* h, const void* w, const int64_t* labels,
                                     int64_t T, int64_t d, int64_t vocab, ulysses_dtype_t dtype,
                                     int64_t ignore_index, float grad_scale, int64_t shard_rows,
                                     float* loss_rows, float* loss_sum, int64_t* n_good, void* dh,
                                     float* dw, void* workspace, size_t workspace_bytes,
                                     hipStream_t stream) {
  if (w == nullptr || loss_sum == nullptr || n_good == nullptr || dw == nullptr)
    return ULYSSES_ERR_NULL;
  if (T > 0 && (h == nullptr || labels == nullptr || loss_rows == nullptr || dh == nullptr))
    return ULYSSES_ERR_NULL;
  if (elem_size(dtype) == 0) return ULYSSES_ERR_DTYPE;
  if (T < 0 || d < 1 || d % 8 != 0 || vocab < 1 || shard_rows < 1 || !std::isfinite(grad_scale))
    return ULYSSES_ERR_SHAPE;
  if (dtype != ULYSSES_BF16) return ULYSSES_ERR_UNSUPPORTED;
  // The GEMM counts rows, columns and the inner size in 32 bits.
  if (T >= (int64_t(1) << 31) || d >= (int64_t(1) << 31) || vocab >= (int64_t(1) << 31) ||
      shard_rows >= (int64_t(1) << 31))
    return ULYSSES_ERR_UNSUPPORTED;
  if (!aligned16(h) || !aligned16(w) || !aligned16(dh) || !aligned16(dw) ||
      reinterpret_cast<uintptr_t>(labels) % 8 != 0 || !aligned4(loss_rows) || !aligned4(loss_sum) ||
      reinterpret_cast<uintptr_t>(n_good) % 8 != 0)
    return ULYSSES_ERR_ALIGNMENT;
  if (T > 0) {
    const size_t need = ulysses::logits_loss_workspace_bytes(shard_rows < T ? shard_rows : T, vocab);
    if (workspace == nullptr || workspace_bytes < need) return ULYSSES_ERR_WORKSPACE;
    if (!aligned16(workspace)) return ULYSSES_ERR_ALIGNMENT;
  }
  ulysses::LogitsLossArgs a{};
  a.h = h;
  a.w = w;
  a.labels = labels;
  a.T = T;
  a.d = d;
  a.V = vocab;
  a.ignore_index = ignore_index;
  a.shard_rows = shard_rows < T ? shard_rows : (T > 0 ? T : 1);
  a.grad_scale = grad_scale;
  a.loss_rows = loss_rows;
  a.loss_sum = loss_sum;
  a.n_good = n_good;
  a.dh = dh;
  a.dw = dw;
  a.workspace = workspace;
  return from_hip(ulysses::launch_logits_loss(a, stream));
}

size_t ulysses_tiled_mlp_workspace_size(int64_t shard_rows, int64_t d, int64_t inter,
                                        int backward) {
  if (shard_rows < 1 || d < 1 || inter < 1 || shard_rows >= (int64_t(1) << 31) ||
      d >= (int64_t(1) << 31) || inter >= (int64_t(1) << 31))
    return 0;
  return ulysses::tiled_mlp_workspace_bytes(shard_rows, d, inter, backward != 0);
}

namespace {

ulysses_status_t tiled_mlp(ulysses::TiledMlpArgs& a, ulysses_dtype_t dtype, size_t ws_bytes,
                           hipStream_t stream) {
  if (a.wg == nullptr || a.wu == nullptr || a.wd == nullptr) return ULYSSES_ERR_NULL;
  if (a.T > 0 && (a.x == nullptr || (a.backward ? (a.dy == nullptr || a.dx == nullptr)
                                                : a.y == nullptr)))
    return ULYSSES_ERR_NULL;
  if (a.backward && (a.dwg == nullptr || a.dwu == nullptr || a.dwd == nullptr))
    return ULYSSES_ERR_NULL;
  if (elem_size(dtype) == 0) return ULYSSES_ERR_DTYPE;
  if (a.T < 0 || a.d < 1 || a.I < 1 || a.shard_rows < 1) return ULYSSES_ERR_SHAPE;
  // 16-byte rows for the vector loads and stores of the row kernels
  if (a.d % 8 != 0 || a.I % 8 != 0) return ULYSSES_ERR_SHAPE;
  if (dtype != ULYSSES_BF16) return ULYSSES_ERR_UNSUPPORTED;
  if (a.T >= (int64_t(1) << 31) || a.d >= (int64_t(1) << 31) || a.I >= (int64_t(1) << 31) ||
      a.shard_rows >= (int64_t(1) << 31))
    return ULYSSES_ERR_UNSUPPORTED;
  if (!aligned16(a.x) || !aligned16(a.wg) || !aligned16(a.wu) || !aligned16(a.wd) ||
      !aligned16(a.y) || !aligned16(a.dy) || !aligned16(a.dx) || !aligned16(a.dwg) ||
      !aligned16(a.dwu) || !aligned16(a.dwd))
    return ULYSSES_ERR_ALIGNMENT;
  if (a.shard_rows > a.T && a.T > 0) a.shard_rows = a.T;
  if (a.T > 0) {
    const size_t need = ulysses::tiled_mlp_workspace_bytes(a.shard_rows, a.d, a.I, a.backward);
    if (a.workspace == nullptr || ws_bytes < need) return ULYSSES_ERR_WORKSPACE;
    if (!aligned16(a.workspace)) return ULYSSES_ERR_ALIGNMENT;
  } else if (!a.backward) {
    return ULYSSES_OK;
  }
  return from_hip(ulysses::launch_tiled_mlp(a, stream));
}

}  // namespace

ulysses_status_t ulysses_tiled_mlp_fwd(const void* x, const void* wg, const void* wu,
                                       const void* wd, int64_t T, int64_t d, int64_t inter,
                                       ulysses_dtype_t dtype, int64_t shard_rows, void* y,
                                       void* workspace, size_t workspace_bytes,
                                       hipStream_t stream) {
  ulysses::TiledMlpArgs a{};
  a.x = x;
  a.wg = wg;
  a.wu = wu;
  a.wd = wd;
  a.T = T;
  a.d = d;
  a.I = inter;
  a.shard_rows = shard_rows;
  a.backward = false;
  a.y = y;
  a.workspace = workspace;
  return tiled_mlp(a, dtype, workspace_bytes, stream);
}

ulysses_status_t ulysses_tiled_mlp_bwd(const void* x, const void* wg, const void* wu,
                                       const void* wd, const void* dy, int64_t T, int64_t d,
                                       int64_t inter, ulysses_dtype_t dtype, int64_t shard_rows,
                                       void* dx, float* dwg, float* dwu, float* dwd,
                                       void* workspace, size_t workspace_bytes,
                                       hipStream_t stream) {
  ulysses::TiledMlpArgs a{};
  a.x = x;
  a.wg = wg;
  a.wu = wu;
  a.wd = wd;
  a.dy = dy;
  a.T = T;
  a.d = d;
  a.I = inter;
  a.shard_rows = shard_rows;
  a.backward = true;
  a.dx = dx;
  a.dwg = dwg;
  a.dwu = dwu;
  a.dwd = dwd;
  a.workspace = workspace;
  return tiled_mlp(a, dtype, workspace_bytes, stream);
}

}  // extern "C"
