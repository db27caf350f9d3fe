// Internal launcher interface between the C-ABI layer (api.cpp) and the
// kernels.  Arguments reaching these functions are already validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ulysses {

constexpr int kMaxChunks = 64;

struct ChunkTable {
  uintptr_t ptr[kMaxChunks];
};

// Layout exchange.  to_head: chunks -> head buffer; otherwise the reverse.
//   chunk_row_bytes : bytes between consecutive (position, batch) rows of a
//                     chunk (heads * head_dim * esize)
//   slot_bytes      : byte offset of the rank's head slice inside a row
//   head_row_bytes  : bytes of one (position, batch) row of the head buffer
//                     (heads_l * head_dim * esize), a multiple of 16
//   rows_per_chunk  : n_local * bs
constexpr int kMaxBatch = 4;

// One tensor of an exchange launch (see launch_exchange for the meaning).
struct ExchangeTensor {
  ChunkTable chunks;
  char* head_buf;
  int64_t chunk_row_bytes, slot_bytes, head_row_bytes;
};

// Moves n (1..kMaxBatch) tensors in one launch; every tensor has P chunks of
// rows_per_chunk rows.
hipError_t launch_exchange_batch(bool to_head, const ExchangeTensor* tensors, int n, int P,
                                 int64_t rows_per_chunk, hipStream_t stream);

hipError_t launch_exchange(bool to_head, const ChunkTable& chunks, int P, char* head_buf,
                           int64_t rows_per_chunk, int64_t chunk_row_bytes, int64_t slot_bytes,
                           int64_t head_row_bytes, hipStream_t stream);

// Unsigned 32-bit division by a run-time invariant divisor with one
// multiply-high and a shift (Granlund and Montgomery, "Division by invariant
// integers using multiplication", PLDI 1994; the round-up multiplier
// m = floor(2^32 (2^l - d) / d) + 1 with l = ceil(log2 d)); fast_div in
// device_common.h applies it.
struct FastDiv {
  uint32_t d, m, l;
};

inline FastDiv make_fastdiv(uint32_t d) {
  uint32_t l = 0;
  while ((1ull << l) < d) ++l;
  const uint64_t m = ((1ull << 32) * ((1ull << l) - d)) / d + 1;
  return FastDiv{d, (uint32_t)m, l};
}

// An attention operand still in its P sequence chunks (the layout on either
// side of the exchange; each chunk [n, bs, row_heads, hd] holds every head):
// row i, batch b, head h of this rank's slice is at
//   chunk[i / n] + ((i % n) * bs + b) * row_heads * hd + (head0 + h) * hd
// elements.  n is a multiple of 64, so a 64-row tile never straddles chunks;
// tiles_per_chunk divides a tile index by n / 64.
constexpr int kMaxFusedChunks = 16;
struct SeqChunks {
  uintptr_t chunk[kMaxFusedChunks];
  int64_t n;
  int row_heads;
  int head0;
  FastDiv tiles_per_chunk;
};

// Base address of this table's first head slot when its chunks are one
// buffer's consecutive slices (chunk c at chunk[0] + c * n rows of bs *
// row_heads * hd bf16 values), 0 otherwise.  Such a table is a strided view
// of one [N, bs, row_heads, hd] tensor.
inline uintptr_t contiguous_base(const SeqChunks& c, int64_t N, int bs, int hd) {
  const int64_t P = c.n > 0 ? N / c.n : 0;
  const uintptr_t step = (uintptr_t)c.n * bs * c.row_heads * hd * 2;
  for (int64_t i = 1; i < P; ++i)
    if (c.chunk[i] != c.chunk[0] + (uintptr_t)i * step) return 0;
  return c.chunk[0] + (uintptr_t)c.head0 * hd * 2;
}

struct AttnShape {
  int64_t N;
  int bs, hq, hkv, hd;
  float scale;
  int causal;
  const int32_t* cu;  // device, or nullptr
  int n_docs;
};

hipError_t launch_attn_fwd_bf16(const AttnShape& s, const void* q, const void* k, const void* v,
                                void* o, float* lse, hipStream_t stream);
// The forward reading Q, K, V from their sequence chunks and writing O into
// the rank's head slots of the O chunks (s.hq / s.hkv are the rank's heads).
hipError_t launch_attn_fwd_bf16_fused(const AttnShape& s, const SeqChunks& q, const SeqChunks& k,
                                      const SeqChunks& v, const SeqChunks& o, float* lse,
                                      hipStream_t stream);
hipError_t launch_attn_fwd_f32(const AttnShape& s, const float* q, const float* k, const float* v,
                               float* o, float* lse, hipStream_t stream);

size_t attn_bwd_workspace_bytes(const AttnShape& s, bool bf16);
// The statistics alone: a smaller workspace runs the bf16 dK/dV kernel
// without its split (same results up to the order of one fp32 sum).
size_t attn_bwd_min_workspace_bytes(const AttnShape& s, bool bf16);

// The fixed per-GPU scratch of ulysses_attn_bwd_noalloc (noalloc.hip): its
// size, and its device address on the current device (looked up once per
// device, then cached).
size_t noalloc_scratch_bytes();
hipError_t noalloc_scratch(void** out);
hipError_t launch_attn_bwd_bf16(const AttnShape& s, const void* q, const void* k, const void* v,
                                const void* o, const float* lse, const void* dout, void* dq,
                                void* dk, void* dv, void* workspace, size_t workspace_bytes,
                                hipStream_t stream);
// The backward with every operand in its sequence chunks (dq, dk, dv written
// into the rank's head slots).
hipError_t launch_attn_bwd_bf16_fused(const AttnShape& s, const SeqChunks& q, const SeqChunks& k,
                                      const SeqChunks& v, const SeqChunks& o, const float* lse,
                                      const SeqChunks& dout, const SeqChunks& dq,
                                      const SeqChunks& dk, const SeqChunks& dv, void* workspace,
                                      size_t workspace_bytes, hipStream_t stream);
hipError_t launch_attn_bwd_f32(const AttnShape& s, const float* q, const float* k, const float* v,
                               const float* o, const float* lse, const float* dout, float* dq,
                               float* dk, float* dv, void* workspace, hipStream_t stream);

// Merge of two partial attention results (O, LSE) over disjoint key sets;
// O is [N, bs, heads, hd] in bf16 or fp32, LSE [bs, heads, N] fp32.
hipError_t launch_attn_merge(bool bf16, const void* o_a, const float* lse_a, const void* o_b,
                             const float* lse_b, int64_t N, int bs, int heads, int hd, void* o,
                             float* lse, hipStream_t stream);

// Language-model loss (lm_head GEMM, cross-entropy over the vocabulary, the
// gradients of grad_scale * loss_sum) over T tokens, shard_rows rows of
// logits at a time.  h [T, d] and w [V, d] bf16; labels int64 [T];
// loss_rows fp32 [T]; loss_sum fp32 [1]; n_good int64 [1]; dh bf16 [T, d];
// dw fp32 [V, d]; workspace of logits_loss_workspace_bytes(shard_rows, V).
struct LogitsLossArgs {
  const void* h;
  const void* w;
  const int64_t* labels;
  int64_t T, d, V, ignore_index, shard_rows;
  float grad_scale;
  float* loss_rows;
  float* loss_sum;
  int64_t* n_good;
  void* dh;
  float* dw;
  void* workspace;
};
size_t logits_loss_workspace_bytes(int64_t shard_rows, int64_t V);
hipError_t launch_logits_loss(const LogitsLossArgs& a, hipStream_t stream);

// Dense bf16 product on the matrix cores (gemm.hip):
//   C[x][y] (+)= sum_k X(x, k) Y(y, k),   x < nx, y < ny, k < K,
// fp32 accumulation.  An operand is k-major (element (r, k) at p[r*ld + k],
// ld >= round_up(K, 8)) or row-major over k (element (r, k) at p[k*ld + r],
// ld >= round_up(rows, 8)); ld % 8 == 0 and p 16-byte aligned either way.
// C is fp32 (stored, or added to when accumulate) or bf16 (c_bf16), row
// stride ldc % 4 == 0.  stats (the loss's logits: both operands k-major,
// c_bf16, labels and label_logit set): for every row x and 256-column tile t
// of the product Z, m = the tile's row max goes to stats[(x *
// gemm_tiles_y(ny) + t) * 2], C receives exp(Z - m) instead of Z, their sum
// goes to stats[... + 1], and Z[x][labels[x]] to label_logit[x] (rows whose
// label is outside [0, ny) get no label_logit).
struct GemmOperand {
  const void* p;
  int64_t ld;
  bool kmajor;
};
struct GemmOp {
  GemmOperand x, y;
  int64_t nx, ny, K;
  void* c;
  int64_t ldc;
  bool c_bf16;
  bool accumulate;
  float* stats;
  const int64_t* labels;
  float* label_logit;
};
int gemm_tiles_y(int64_t ny);
hipError_t launch_gemm(const GemmOp& op, hipStream_t stream);
// Two products in one launch when they share every size, layout and output
// mode (and neither has stats), so their tiles fill one grid; two launches,
// a then b, otherwise or when both write the same output.  In one launch the
// products run concurrently: neither output may overlap the other product's
// operands.
hipError_t launch_gemm_pair(const GemmOp& a, const GemmOp& b, hipStream_t stream);

// Sequence-tiled SwiGLU MLP over T rows, shard_rows at a time.  x [T, d],
// wg and wu [I, d], wd [d, I], y/dy/dx [T, d] bf16; dwg, dwu [I, d] and dwd
// [d, I] fp32; workspace of tiled_mlp_workspace_bytes(shard_rows, d, I,
// backward).  backward == false: y only; true: dx, dwg, dwu, dwd from dy.
struct TiledMlpArgs {
  const void* x;
  const void* wg;
  const void* wu;
  const void* wd;
  const void* dy;
  int64_t T, d, I, shard_rows;
  bool backward;
  void* y;
  void* dx;
  float* dwg;
  float* dwu;
  float* dwd;
  void* workspace;
};
size_t tiled_mlp_workspace_bytes(int64_t shard_rows, int64_t d, int64_t I, bool backward);
hipError_t launch_tiled_mlp(const TiledMlpArgs& a, hipStream_t stream);

}  // namespace ulysses
