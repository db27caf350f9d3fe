// Language-model loss over a rank's tokens with the lm_head projection, the
// cross-entropy and both gradients done shard by shard, so that the
// [tokens, vocab] logits exist for one shard at a time only (the
// integration guide's tiled fused logits loss, section on tiled loss
// computation: the backward runs inside the forward, shard by shard, with
// no second forward and no full logits).
//
// Per shard of S token rows (every product on the library's matrix-core
// GEMM, gemm.hip):
//   Z = H_s W^T            never stored: the GEMM's epilogue writes, per row
//                          and 256-column tile t with row max m_t, the values
//                          E = exp(Z - m_t) as bf16 [S, V], the pair (m_t,
//                          sum of E over the tile), and the label's logit
//                          Z[s][label] in fp32
//   ce_grad_kernel         per row: lse from the tile pairs, the row loss
//                          lse - Z[s][label], and, in place of E, G = s
//                          (softmax(Z) - onehot(label)) = s (E exp(m_t - lse)
//                          - onehot): one bf16 read and one bf16 write per
//                          logit
//   dH_s = G W             bf16 [S, d]
//   dW (+)= G^T H_s        fp32 [V, d] (stored for the first shard, added to
//                          for the others)
// then one workgroup sums the row losses and counts the kept tokens in a
// fixed order (bitwise reproducible).  E/G rows are padded to a multiple of
// 8 columns (16-byte rows for the GEMM's copies).
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

// One workgroup per token row r of the shard.  The row's log-sum-exp comes
// from the Z GEMM's per-tile pairs (m_t, l_t) (natural-log max and sum of
// exp(z - m_t)); then the row's E values (bf16, padded to ld columns, 8 per
// lane and step) are turned into G in place, columns >= V set to zero.
__global__ __launch_bounds__(kCeThreads) void ce_grad_kernel(__bf16* __restrict__ g,
                                                             const float* __restrict__ stats,
                                                             int tiles,
                                                             const float* __restrict__ zlabel,
                                                             const int64_t* __restrict__ labels,
                                                             float* __restrict__ loss_rows,
                                                             int64_t V, int64_t ld,
                                                             int64_t ignore, float s) {
  __shared__ MaxSum part[kCeWaves];
  __shared__ float row_stat[2];
  const int64_t r = blockIdx.x;
  __bf16* gr = g + r * ld;
  const int64_t y = labels[r];
  const int tid = threadIdx.x;

  if (y == ignore) {   // kept out of the loss: zero gradient row
    for (int64_t v = 8 * (int64_t)tid; v < ld; v += 8 * kCeThreads)
      *reinterpret_cast<bf16x8_t*>(gr + v) = bf16x8_t{};
    if (tid == 0) loss_rows[r] = 0.0f;
    return;
  }

  // Merge the tile pairs (log2 domain: max * log2(e), same sums).
  MaxSum acc{-INFINITY, 0.0f};
  const float* st = stats + r * (int64_t)tiles * 2;
  for (int t = tid; t < tiles; t += kCeThreads)
    acc = merge(acc, MaxSum{st[2 * t] * kLog2e, st[2 * t + 1]});
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
    loss_rows[r] = valid ? lse2 * kLn2 - zlabel[r] : NAN;
  }
  __syncthreads();
  const float lse2 = row_stat[0];
  // 8 columns per lane and step never straddle a 256-column tile.
  for (int64_t v = 8 * (int64_t)tid; v < ld; v += 8 * kCeThreads) {
    const float f = s * exp2f(st[2 * (v >> 8)] * kLog2e - lse2);   // s exp(m_t - lse)
    const bf16x8_t ev = *reinterpret_cast<const bf16x8_t*>(gr + v);
    bf16x8_t o;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float gv = f * (float)ev[e] - (v + e == y ? s : 0.0f);
      o[e] = v + e < V ? (__bf16)gv : (__bf16)0.0f;
    }
    *reinterpret_cast<bf16x8_t*>(gr + v) = o;
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

int64_t pad8(int64_t v) { return (v + 7) / 8 * 8; }

}  // namespace

size_t logits_loss_workspace_bytes(int64_t shard_rows, int64_t V) {
  const size_t vp = (size_t)pad8(V);
  return align256((size_t)shard_rows * vp * sizeof(uint16_t)) +
         align256((size_t)shard_rows * gemm_tiles_y(V) * 2 * sizeof(float)) +
         align256((size_t)shard_rows * sizeof(float));
}

hipError_t launch_logits_loss(const LogitsLossArgs& a, hipStream_t stream) {
  const int64_t T = a.T, d = a.d, V = a.V, vp = pad8(V);
  const int tiles = gemm_tiles_y(V);
  char* ws = static_cast<char*>(a.workspace);
  __bf16* g = reinterpret_cast<__bf16*>(ws);   // E, then G in place
  ws += align256((size_t)a.shard_rows * vp * sizeof(uint16_t));
  float* stats = reinterpret_cast<float*>(ws);
  ws += align256((size_t)a.shard_rows * tiles * 2 * sizeof(float));
  float* zlabel = reinterpret_cast<float*>(ws);
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
    // Z[s][v] = sum_k H[s][k] W[v][k], kept as E = exp(Z - m_t), the tile
    // pairs and the label logits
    GemmOp op{};
    op.x = GemmOperand{hs, d, true};
    op.y = GemmOperand{a.w, d, true};
    op.nx = rows;
    op.ny = V;
    op.K = d;
    op.c = g;
    op.ldc = vp;
    op.c_bf16 = true;
    op.stats = stats;
    op.labels = a.labels + r0;
    op.label_logit = zlabel;
    if ((e = launch_gemm(op, stream)) != hipSuccess) return e;
    e = launch_kernel(ce_grad_kernel, dim3((uint32_t)rows), dim3(kCeThreads), 0, stream, g,
                      stats, tiles, zlabel, a.labels + r0, a.loss_rows + r0, V, vp,
                      a.ignore_index, a.grad_scale);
    if (e != hipSuccess) return e;
    // dH_s[s][j] = sum_v G[s][v] W[v][j]
    op = GemmOp{};
    op.x = GemmOperand{g, vp, true};
    op.y = GemmOperand{a.w, d, false};
    op.nx = rows;
    op.ny = d;
    op.K = V;
    op.c = dh + r0 * d;
    op.ldc = d;
    op.c_bf16 = true;
    if ((e = launch_gemm(op, stream)) != hipSuccess) return e;
    // dW[v][j] (+)= sum_s G[s][v] H_s[s][j]
    op = GemmOp{};
    op.x = GemmOperand{g, vp, false};
    op.y = GemmOperand{hs, d, false};
    op.nx = V;
    op.ny = d;
    op.K = rows;
    op.c = a.dw;
    op.ldc = d;
    op.accumulate = r0 > 0;
    if ((e = launch_gemm(op, stream)) != hipSuccess) return e;
  }
  return launch_kernel(loss_sum_kernel, dim3(1), dim3(kSumThreads), 0, stream, a.loss_rows,
                       a.labels, T, a.ignore_index, a.loss_sum, a.n_good);
}

}  // namespace ulysses
