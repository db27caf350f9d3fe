// Merge of two partial attention results over disjoint key sets: the
// combination step of ring (blockwise) attention, which the Hugging Face
// Ulysses blog compares with Ulysses ("Ulysses vs Ring Attention": key/value
// blocks travel around a ring and each block's result is folded into the
// running one).  With (O_a, LSE_a) and (O_b, LSE_b) the results of the same
// queries against key sets A and B, the result over A and B is
//   LSE = ln(e^LSE_a + e^LSE_b),  O = w_a O_a + w_b O_b,
//   w_a = e^LSE_a / (e^LSE_a + e^LSE_b),  w_b = e^LSE_b / (e^LSE_a + e^LSE_b),
// all evaluated relative to the larger statistic, so nothing overflows.  A
// partial with weight 0 (LSE = -inf: it saw no key) contributes nothing,
// whatever its O holds; two -inf partials give O = 0 and LSE = -inf.
//
// HBM-bound elementwise work: each O row is read once per partial and
// written once, in 16-byte vectors.  The kLanes consecutive lanes that own a
// row (row bytes / 16, a power of two up to 64) sit in one wave, so a wave
// reads whole 64-byte segments, and a row's statistics are read by the same
// instruction in every lane before its first lane writes the merged one;
// that keeps the in-place form (o the same buffer as o_a or o_b, lse as
// lse_a or lse_b) correct.
#include <math.h>

#include "device_common.h"
#include "launch.h"

namespace ulysses {
namespace {

constexpr int kMergeThreads = 256;

template <typename T, int HD>
__global__ __launch_bounds__(kMergeThreads) void attn_merge_kernel(
    const T* o_a, const float* lse_a, const T* o_b, const float* lse_b, T* o, float* lse,
    int64_t rows, int64_t N, int bs, int heads) {
  constexpr int kVec = 16 / (int)sizeof(T);   // elements per 16-byte vector
  constexpr int kLanes = HD / kVec;            // lanes per row
  constexpr int kRowsPerBlock = kMergeThreads / kLanes;
  static_assert(kLanes >= 1 && kLanes <= 64 && (64 % kLanes) == 0, "a row within one wave");
  const int64_t r = (int64_t)blockIdx.x * kRowsPerBlock + threadIdx.x / kLanes;
  const int sub = threadIdx.x % kLanes;
  if (r >= rows) return;
  // r enumerates (position, batch, head) in O's memory order; LSE is
  // [batch, head, position].
  const int h = (int)(r % heads);
  const int64_t ib = r / heads;
  const int b = (int)(ib % bs);
  const int64_t i = ib / bs;
  const int64_t si = ((int64_t)b * heads + h) * N + i;
  const float la = lse_a[si], lb = lse_b[si];
  // Streaming accesses (non-temporal): every O byte is touched once.
  const u32x4_t va = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(o_a + r * HD + sub * kVec));
  const u32x4_t vb = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(o_b + r * HD + sub * kVec));

  const float m = fmaxf(la, lb);
  float merged = -INFINITY, wa = 0.f, wb = 0.f;
  if (m != -INFINITY) {
    const float ea = expf(la - m), eb = expf(lb - m);   // the larger one is exactly 1
    const float s = ea + eb;
    merged = m + logf(s);
    wa = ea / s;
    wb = eb / s;
  }
  u32x4_t out;
  if constexpr (sizeof(T) == 2) {
    const bf16x8_t xa = __builtin_bit_cast(bf16x8_t, va), xb = __builtin_bit_cast(bf16x8_t, vb);
    bf16x8_t y;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float ta = wa != 0.f ? wa * (float)xa[e] : 0.f;
      const float tb = wb != 0.f ? wb * (float)xb[e] : 0.f;
      y[e] = (__bf16)(ta + tb);
    }
    out = __builtin_bit_cast(u32x4_t, y);
  } else {
    const f32x4_t xa = __builtin_bit_cast(f32x4_t, va), xb = __builtin_bit_cast(f32x4_t, vb);
    f32x4_t y;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float ta = wa != 0.f ? wa * xa[e] : 0.f;
      const float tb = wb != 0.f ? wb * xb[e] : 0.f;
      y[e] = ta + tb;
    }
    out = __builtin_bit_cast(u32x4_t, y);
  }
  __builtin_nontemporal_store(out, reinterpret_cast<u32x4_t*>(o + r * HD + sub * kVec));
  if (sub == 0) lse[si] = merged;
}

template <typename T, int HD>
hipError_t launch_merge(const void* o_a, const float* lse_a, const void* o_b, const float* lse_b,
                        int64_t N, int bs, int heads, void* o, float* lse, hipStream_t stream) {
  constexpr int kRowsPerBlock = kMergeThreads / (HD * (int)sizeof(T) / 16);
  const int64_t rows = N * bs * heads;
  const int64_t blocks = (rows + kRowsPerBlock - 1) / kRowsPerBlock;
  if (blocks >= (int64_t(1) << 31)) return hipErrorInvalidValue;
  return launch_kernel(attn_merge_kernel<T, HD>, dim3((uint32_t)blocks), dim3(kMergeThreads), 0,
                       stream, static_cast<const T*>(o_a), lse_a, static_cast<const T*>(o_b), lse_b,
                       static_cast<T*>(o), lse, rows, N, bs, heads);
}

}  // namespace

hipError_t launch_attn_merge(bool bf16, const void* o_a, const float* lse_a, const void* o_b,
                             const float* lse_b, int64_t N, int bs, int heads, int hd, void* o,
                             float* lse, hipStream_t stream) {
  if (N == 0) return hipSuccess;
  if (bf16) {
    if (hd == 32) return launch_merge<__bf16, 32>(o_a, lse_a, o_b, lse_b, N, bs, heads, o, lse, stream);
    if (hd == 64) return launch_merge<__bf16, 64>(o_a, lse_a, o_b, lse_b, N, bs, heads, o, lse, stream);
    return launch_merge<__bf16, 128>(o_a, lse_a, o_b, lse_b, N, bs, heads, o, lse, stream);
  }
  if (hd == 32) return launch_merge<float, 32>(o_a, lse_a, o_b, lse_b, N, bs, heads, o, lse, stream);
  if (hd == 64) return launch_merge<float, 64>(o_a, lse_a, o_b, lse_b, N, bs, heads, o, lse, stream);
  return launch_merge<float, 128>(o_a, lse_a, o_b, lse_b, N, bs, heads, o, lse, stream);
}

}  // namespace ulysses
