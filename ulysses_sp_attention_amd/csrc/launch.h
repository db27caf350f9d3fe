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
hipError_t launch_attn_fwd_f32(const AttnShape& s, const float* q, const float* k, const float* v,
                               float* o, float* lse, hipStream_t stream);

size_t attn_bwd_workspace_bytes(const AttnShape& s, bool bf16);
hipError_t launch_attn_bwd_bf16(const AttnShape& s, const void* q, const void* k, const void* v,
                                const void* o, const float* lse, const void* dout, void* dq,
                                void* dk, void* dv, void* workspace, hipStream_t stream);
hipError_t launch_attn_bwd_f32(const AttnShape& s, const float* q, const float* k, const float* v,
                               const float* o, const float* lse, const float* dout, float* dq,
                               float* dk, float* dv, void* workspace, hipStream_t stream);

// Merge of two partial attention results (O, LSE) over disjoint key sets;
// O is [N, bs, heads, hd] in bf16 or fp32, LSE [bs, heads, N] fp32.
hipError_t launch_attn_merge(bool bf16, const void* o_a, const float* lse_a, const void* o_b,
                             const float* lse_b, int64_t N, int bs, int heads, int hd, void* o,
                             float* lse, hipStream_t stream);

}  // namespace ulysses
