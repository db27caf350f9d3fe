// Language-model loss over a rank's tokens with the lm_head projection, the
// cross-entropy and both gradients done shard by shard, so that the
// [tokens, vocab] logits exist for one shard at a time only (the
// integration guide's tiled fused logits loss, section on tiled loss
// computation: the backward runs inside the forward, shard by shard, with
// no second forward and no full logits).
//
// Per shard of S token rows:
//   Z = H_s W^T            fp32 [S, V]      rocBLAS GEMM (bf16 in, fp32 out)
//   ce_grad_kernel         one pass per row: lse, the row loss and
//                          G = s (softmax(Z) - onehot(label)) as bf16 [S, V]
//   dH_s = G W             bf16 [S, d]      rocBLAS GEMM (fp32 accumulate)
//   dW (+)= G^T H_s        fp32 [V, d]      rocBLAS GEMM (beta 0, then 1)
// then one workgroup sums the row losses and counts the kept tokens in a
// fixed order (bitwise reproducible).  The GEMMs are plain dense products,
// left to the vendor library; the fused part is the row kernel.
#include "blas.h"
#include "device_common.h"
#include "launch.h"

namespace ulysses {
namespace {

constexpr int kCeThreads = 512;
constexpr int kCeWaves = kCeThreads / 64;

// Online (max, sum of 2^(x - max)) pair in the log2 domain.
struct MaxSum {
  float m, l;
};

__device__ __forceinline__ MaxSum merge(MaxSum a, MaxSum b) {
  if (a.m == -INFINITY) return b;
  if (b.m == -INFINITY) return a;
  const float m = fmaxf(a.m, b.m);
  return MaxSum{m, a.l * exp2f(a.m - m) + b.l * exp2f(b.m - m)};
}

__device__ __forceinline__ MaxSum add(MaxSum a, float x) {
  if (x <= a.m) return MaxSum{a.m, a.l + exp2f(x - a.m)};
  return MaxSum{x, a.l * exp2f(a.m - x) + 1.0f};   // exp2f(-inf) = 0 for the first value
}

// One workgroup per token row r of the shard.  Reads Z[r, :] twice (the
// second pass mostly from cache), writes G[r, :] once.  kVec4: V % 4 == 0,
// rows read as float4 and written as 4 bf16.
template <bool kVec4>
__global__ __launch_bounds__(kCeThreads) void ce_grad_kernel(const float* __restrict__ z,
                                                             __bf16* __restrict__ g,
                                                             const int64_t* __restrict__ labels,
                                                             float* __restrict__ loss_rows,
                                                             int64_t V, int64_t ignore, float s) {
  __shared__ MaxSum part[kCeWaves];
  __shared__ float row_stat[2];
  const int64_t r = blockIdx.x;
  const float* zr = z + r * V;
  __bf16* gr = g + r * V;
  const int64_t y = labels[r];
  const int tid = threadIdx.x;

  if (y == ignore) {   // kept out of the loss: zero gradient row
    if constexpr (kVec4) {
      for (int64_t v = 4 * (int64_t)tid; v < V; v += 4 * kCeThreads)
        *reinterpret_cast<bf16x4_t*>(gr + v) = bf16x4_t{};
    } else {
      for (int64_t v = tid; v < V; v += kCeThreads) gr[v] = (__bf16)0.0f;
    }
    if (tid == 0) loss_rows[r] = 0.0f;
    return;
  }

  MaxSum acc{-INFINITY, 0.0f};
  if constexpr (kVec4) {
    for (int64_t v = 4 * (int64_t)tid; v < V; v += 4 * kCeThreads) {
      const float4 x = *reinterpret_cast<const float4*>(zr + v);
      acc = add(add(add(add(acc, x.x * kLog2e), x.y * kLog2e), x.z * kLog2e), x.w * kLog2e);
    }
  } else {
    for (int64_t v = tid; v < V; v += kCeThreads) acc = add(acc, zr[v] * kLog2e);
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const MaxSum o{__shfl_xor(acc.m, off, 64), __shfl_xor(acc.l, off, 64)};
    acc = merge(acc, o);
  }
  if ((tid & 63) == 0) part[tid >> 6] = acc;
  __syncthreads();
  if (tid == 0) {
    MaxSum t = part[0];
    for (int w = 1; w < kCeWaves; ++w) t = merge(t, part[w]);
    const float lse2 = t.m + log2f(t.l);                   // log2-domain lse
    const bool valid = y >= 0 && y < V;
    row_stat[0] = valid ? lse2 : NAN;
    loss_rows[r] = valid ? lse2 * kLn2 - zr[y] : NAN;
  }
  __syncthreads();
  const float lse2 = row_stat[0];
  if constexpr (kVec4) {
    for (int64_t v = 4 * (int64_t)tid; v < V; v += 4 * kCeThreads) {
      const f32x4_t x = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(zr + v));   // last use
      bf16x4_t o;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        o[e] = (__bf16)(s * (exp2f(x[e] * kLog2e - lse2) - (v + e == y ? 1.0f : 0.0f)));
      *reinterpret_cast<bf16x4_t*>(gr + v) = o;
    }
  } else {
    for (int64_t v = tid; v < V; v += kCeThreads)
      gr[v] = (__bf16)(s * (exp2f(zr[v] * kLog2e - lse2) - (v == y ? 1.0f : 0.0f)));
  }
}

// Loss sum (in double, fixed order) and kept-token count over all T rows.
constexpr int kSumThreads = 1024;
__global__ __launch_bounds__(kSumThreads) void loss_sum_kernel(const float* __restrict__ loss_rows,
                                                               const int64_t* __restrict__ labels,
                                                               int64_t T, int64_t ignore,
                                                               float* __restrict__ loss_sum,
                                                               int64_t* __restrict__ n_good) {
  __shared__ double sums[kSumThreads];
  __shared__ int64_t counts[kSumThreads];
  const int tid = threadIdx.x;
  double acc = 0.0;
  int64_t cnt = 0;
  for (int64_t i = tid; i < T; i += kSumThreads) {
    acc += (double)loss_rows[i];
    cnt += labels[i] != ignore ? 1 : 0;
  }
  sums[tid] = acc;
  counts[tid] = cnt;
  __syncthreads();
  for (int half = kSumThreads / 2; half > 0; half >>= 1) {
    if (tid < half) {
      sums[tid] += sums[tid + half];
      counts[tid] += counts[tid + half];
    }
    __syncthreads();
  }
  if (tid == 0) {
    *loss_sum = (float)sums[0];
    *n_good = counts[0];
  }
}

// dW = 0 (the empty-input case: no shard writes it).
__global__ __launch_bounds__(256) void zero_f32_kernel(float* __restrict__ x, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) x[i] = 0.0f;
}

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

}  // namespace

size_t logits_loss_workspace_bytes(int64_t shard_rows, int64_t V) {
  return align256((size_t)shard_rows * V * sizeof(float)) +
         align256((size_t)shard_rows * V * sizeof(uint16_t));
}

hipError_t launch_logits_loss(const LogitsLossArgs& a, hipStream_t stream) {
  rocblas_handle hd = blas_handle();
  if (!hd) return hipErrorNotInitialized;
  if (rocblas_set_stream(hd, stream) != rocblas_status_success) return hipErrorUnknown;
  const int64_t T = a.T, d = a.d, V = a.V;
  float* z = static_cast<float*>(a.workspace);
  __bf16* g = reinterpret_cast<__bf16*>(static_cast<char*>(a.workspace) +
                                        align256((size_t)a.shard_rows * V * sizeof(float)));
  const __bf16* h = static_cast<const __bf16*>(a.h);
  __bf16* dh = static_cast<__bf16*>(a.dh);
  hipError_t e;
  if (T == 0) {
    const int64_t n = V * d;
    e = launch_kernel(zero_f32_kernel, dim3((uint32_t)((n + 255) / 256)), dim3(256), 0, stream,
                      a.dw, n);
    if (e != hipSuccess) return e;
  }
  for (int64_t r0 = 0; r0 < T; r0 += a.shard_rows) {
    const int64_t rows = T - r0 < a.shard_rows ? T - r0 : a.shard_rows;
    const __bf16* hs = h + r0 * d;
    // Z^T (col-major V x rows) = W (col-major d x V)^T . H_s^T (col-major d x rows)
    if (!gemm_bf16(hd, true, false, V, rows, d, a.w, d, hs, d, 0.0f, z, false, V))
      return hipErrorUnknown;
    e = launch_kernel(V % 4 == 0 ? ce_grad_kernel<true> : ce_grad_kernel<false>,
                      dim3((uint32_t)rows), dim3(kCeThreads), 0, stream, z, g, a.labels + r0,
                      a.loss_rows + r0, V, a.ignore_index, a.grad_scale);
    if (e != hipSuccess) return e;
    // dH_s^T (col-major d x rows) = W (col-major d x V) . G^T (col-major V x rows)
    if (!gemm_bf16(hd, false, false, d, rows, V, a.w, d, g, V, 0.0f, dh + r0 * d, true, d))
      return hipErrorUnknown;
    // dW^T (col-major d x V) (+)= H_s^T (col-major d x rows) . G (col-major V x rows)^T
    if (!gemm_bf16(hd, false, true, d, V, rows, hs, d, g, V, r0 == 0 ? 0.0f : 1.0f, a.dw, false, d))
      return hipErrorUnknown;
  }
  return launch_kernel(loss_sum_kernel, dim3(1), dim3(kSumThreads), 0, stream, a.loss_rows,
                       a.labels, T, a.ignore_index, a.loss_sum, a.n_good);
}

}  // namespace ulysses
