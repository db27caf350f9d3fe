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
// small workgroups measured fastest on MI355X with the caches cold (5.4 TB/s
// read+write for the 128K query pack, against 5.3 TB/s for a device-to-device
// hipMemcpy of the same size; 4 or 8 vectors per thread: 4.6 and 3.5 TB/s).
#include "device_common.h"
#include "launch.h"

namespace ulysses {
namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 1;

// Unsigned 32-bit division by a run-time invariant divisor with one
// multiply-high and a shift (Granlund and Montgomery, "Division by invariant
// integers using multiplication", PLDI 1994; the round-up multiplier
// m = floor(2^32 (2^l - d) / d) + 1 with l = ceil(log2 d)).
struct FastDiv {
  uint32_t d, m, l;
};

FastDiv make_fastdiv(uint32_t d) {
  uint32_t l = 0;
  while ((1ull << l) < d) ++l;
  const uint64_t m = ((1ull << 32) * ((1ull << l) - d)) / d + 1;
  return FastDiv{d, (uint32_t)m, l};
}

__device__ __forceinline__ uint32_t fast_div(uint32_t n, FastDiv f) {
  const uint32_t t = __umulhi(n, f.m);
  return (uint32_t)(((uint64_t)t + n) >> f.l);
}

template <bool kToHead>
__global__ __launch_bounds__(kThreads) void exchange_kernel(ChunkTable chunks, char* head_buf,
                                                            uint32_t vecs_per_chunk, FastDiv vpr,
                                                            int64_t rows_per_chunk,
                                                            int64_t chunk_row_bytes,
                                                            int64_t slot_bytes,
                                                            int64_t head_row_bytes) {
  const int c = blockIdx.y;
  char* chunk = reinterpret_cast<char*>(chunks.ptr[c]) + slot_bytes;
  char* head = head_buf + (int64_t)c * rows_per_chunk * head_row_bytes;
  const uint32_t base = blockIdx.x * (kThreads * kUnroll) + threadIdx.x;
  u32x4_t val[kUnroll];
  char* dst[kUnroll];
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) {
    const uint32_t w = base + u * kThreads;
    dst[u] = nullptr;
    if (w < vecs_per_chunk) {
      const uint32_t row = fast_div(w, vpr);
      const uint32_t col = w - row * vpr.d;
      char* cp = chunk + (int64_t)row * chunk_row_bytes + (int64_t)col * 16;
      char* hp = head + (int64_t)row * head_row_bytes + (int64_t)col * 16;
      const char* src = kToHead ? cp : hp;
      dst[u] = kToHead ? hp : cp;
      val[u] = *reinterpret_cast<const u32x4_t*>(src);
    }
  }
#pragma unroll
  for (int u = 0; u < kUnroll; ++u)
    if (dst[u]) *reinterpret_cast<u32x4_t*>(dst[u]) = val[u];
}

}  // namespace

hipError_t launch_exchange(bool to_head, const ChunkTable& chunks, int P, char* head_buf,
                           int64_t rows_per_chunk, int64_t chunk_row_bytes, int64_t slot_bytes,
                           int64_t head_row_bytes, hipStream_t stream) {
  const uint32_t vpr = (uint32_t)(head_row_bytes / 16);
  const uint64_t vecs = (uint64_t)rows_per_chunk * vpr;
  if (vecs == 0) return hipSuccess;
  const FastDiv fd = make_fastdiv(vpr);
  const uint32_t per_block = kThreads * kUnroll;
  dim3 grid((uint32_t)((vecs + per_block - 1) / per_block), (uint32_t)P);
  auto kernel = to_head ? exchange_kernel<true> : exchange_kernel<false>;
  return launch_kernel(kernel, grid, dim3(kThreads), 0, stream, chunks, head_buf, (uint32_t)vecs, fd,
                       rows_per_chunk, chunk_row_bytes, slot_bytes, head_row_bytes);
}

}  // namespace ulysses
