// Layout exchange kernels: the per-rank data movement of the two Ulysses
// all-to-alls (Hugging Face Ulysses blog, "The challenge of long-sequence
// training": seq-sharded -> head-sharded before attention, and back after).
//
// For every (position, batch) row the rank's head slice is one contiguous
// run of heads_l * head_dim elements on both sides, so the exchange is a
// gather of contiguous 16-byte vectors: no arithmetic, bit-exact.  Each
// thread moves kUnroll vectors (all loads issued before the stores), with
// consecutive lanes on consecutive 16-byte vectors of a row, so every wave
// reads and writes whole 64-byte segments.  One vector per thread and many
// small workgroups measured fastest on MI355X with the caches cold; loads and
// stores are non-temporal (each byte is moved once), which took the four
// exchanges of a training step, run back to back on cold buffers, from 5.1
// to 5.7 TB/s read+write, above the 5.4 TB/s of a device-to-device copy of
// the same bytes (4 or 8 vectors per thread measured slower).
#include "device_common.h"
#include "launch.h"

namespace ulysses {
namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 1;

// Per-tensor launch data: its chunk table is in ExchangeArgs::chunks.
struct SliceArgs {
  char* head_buf;
  int64_t chunk_row_bytes, slot_bytes, head_row_bytes;
  uint32_t vecs_per_chunk;   // rows_per_chunk * vectors per head row
  FastDiv vpr;               // vectors per head row
  uint32_t block_begin;      // first blockIdx.x of this tensor
};
struct ExchangeArgs {
  SliceArgs t[kMaxBatch];
  uintptr_t chunks[kMaxBatch][kMaxChunks];
  int n;
  int64_t rows_per_chunk;
};

// Blocks [t[i].block_begin, t[i+1].block_begin) of grid.x move tensor i;
// grid.y is the chunk.
template <bool kToHead>
__global__ __launch_bounds__(kThreads) void exchange_kernel(ExchangeArgs a) {
  int ti = 0;
#pragma unroll
  for (int i = 1; i < kMaxBatch; ++i)
    if (i < a.n && blockIdx.x >= a.t[i].block_begin) ti = i;
  const SliceArgs& s = a.t[ti];
  const int c = blockIdx.y;
  char* chunk = reinterpret_cast<char*>(a.chunks[ti][c]) + s.slot_bytes;
  char* head = s.head_buf + (int64_t)c * a.rows_per_chunk * s.head_row_bytes;
  const uint32_t base = (blockIdx.x - s.block_begin) * (kThreads * kUnroll) + threadIdx.x;
  u32x4_t val[kUnroll];
  char* dst[kUnroll];
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) {
    const uint32_t w = base + u * kThreads;
    dst[u] = nullptr;
    if (w < s.vecs_per_chunk) {
      const uint32_t row = fast_div(w, s.vpr);
      const uint32_t col = w - row * s.vpr.d;
      char* cp = chunk + (int64_t)row * s.chunk_row_bytes + (int64_t)col * 16;
      char* hp = head + (int64_t)row * s.head_row_bytes + (int64_t)col * 16;
      const char* src = kToHead ? cp : hp;
      dst[u] = kToHead ? hp : cp;
      val[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(src));
    }
  }
#pragma unroll
  for (int u = 0; u < kUnroll; ++u)
    if (dst[u]) __builtin_nontemporal_store(val[u], reinterpret_cast<u32x4_t*>(dst[u]));
}

}  // namespace

hipError_t launch_exchange_batch(bool to_head, const ExchangeTensor* tensors, int n, int P,
                                 int64_t rows_per_chunk, hipStream_t stream) {
  ExchangeArgs a{};
  a.n = n;
  a.rows_per_chunk = rows_per_chunk;
  const uint32_t per_block = kThreads * kUnroll;
  uint64_t blocks = 0;
  for (int i = 0; i < n; ++i) {
    const ExchangeTensor& t = tensors[i];
    const uint32_t vpr = (uint32_t)(t.head_row_bytes / 16);
    const uint64_t vecs = (uint64_t)rows_per_chunk * vpr;
    if (vecs + per_block > (1ull << 32)) return hipErrorInvalidValue;   // 32-bit vector index
    SliceArgs& s = a.t[i];
    s.head_buf = t.head_buf;
    s.chunk_row_bytes = t.chunk_row_bytes;
    s.slot_bytes = t.slot_bytes;
    s.head_row_bytes = t.head_row_bytes;
    s.vecs_per_chunk = (uint32_t)vecs;
    s.vpr = make_fastdiv(vpr);
    s.block_begin = (uint32_t)blocks;
    for (int c = 0; c < P; ++c) a.chunks[i][c] = t.chunks.ptr[c];
    blocks += (vecs + per_block - 1) / per_block;
  }
  if (blocks == 0) return hipSuccess;
  if (blocks >= (1ull << 31)) return hipErrorInvalidValue;
  dim3 grid((uint32_t)blocks, (uint32_t)P);
  auto kernel = to_head ? exchange_kernel<true> : exchange_kernel<false>;
  return launch_kernel(kernel, grid, dim3(kThreads), 0, stream, a);
}

hipError_t launch_exchange(bool to_head, const ChunkTable& chunks, int P, char* head_buf,
                           int64_t rows_per_chunk, int64_t chunk_row_bytes, int64_t slot_bytes,
                           int64_t head_row_bytes, hipStream_t stream) {
  ExchangeTensor t{chunks, head_buf, chunk_row_bytes, slot_bytes, head_row_bytes};
  return launch_exchange_batch(to_head, &t, 1, P, rows_per_chunk, stream);
}

}  // namespace ulysses
