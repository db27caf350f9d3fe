// Sequence-tiled SwiGLU MLP (the integration guide's TiledMLP, section on
// the ALST memory tricks): y = (silu(x Wg^T) * (x Wu^T)) Wd^T computed a
// shard of token rows at a time, so the [T, I] intermediates exist for one
// shard only; the backward recomputes each shard's intermediates instead of
// keeping them (the guide's tiled compute replays the forward in the
// backward).  Rows are independent, so sharding changes no result.
//
// Per shard of S rows (intermediates in the workspace; every product on the
// library's matrix-core GEMM, gemm.hip, with operands in whatever layout
// they are stored in):
//   forward : g = x_s Wg^T, u = x_s Wu^T (fp32)
//             a = bf16(silu(g) u)                  swiglu_fwd_kernel
//             y_s = a Wd^T (bf16)
//   backward: g, u as above; da = dy_s Wd (fp32)
//             a, dg = bf16(da u silu'(g)), du = bf16(da silu(g))
//                                                  swiglu_bwd_kernel
//             dWd (+)= dy_s^T a; dWg (+)= dg^T x_s; dWu (+)= du^T x_s (fp32)
//             dx_s = dg Wg + du Wu (fp32, then bf16 by f32_to_bf16_kernel)
// g, u and da stay fp32; only the operands of a GEMM are rounded to bf16.
#include "device_common.h"
#include "launch.h"

namespace ulysses {
namespace {

constexpr int kEwThreads = 256;

__device__ __forceinline__ float sigmoidf(float g) { return 1.0f / (1.0f + expf(-g)); }

// a = bf16(silu(g) u) for n elements.
__global__ __launch_bounds__(kEwThreads) void swiglu_fwd_kernel(const float* __restrict__ g,
                                                                const float* __restrict__ u,
                                                                __bf16* __restrict__ a, int64_t n) {
  const int64_t i = ((int64_t)blockIdx.x * kEwThreads + threadIdx.x) * 4;
  if (i + 4 <= n) {
    // g and u are read once: non-temporal
    const f32x4_t gv = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(g + i));
    const f32x4_t uv = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(u + i));
    bf16x4_t o;
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] = (__bf16)(gv[e] * sigmoidf(gv[e]) * uv[e]);
    *reinterpret_cast<bf16x4_t*>(a + i) = o;
  } else {
    for (int64_t j = i; j < n; ++j) a[j] = (__bf16)(g[j] * sigmoidf(g[j]) * u[j]);
  }
}

// a, dg = da u silu'(g), du = da silu(g) (each rounded to bf16 when stored)
// for n elements, with silu'(g) = s (1 + g (1 - s)) and s the logistic
// sigmoid of g.
struct SwigluGrad {
  float a, dg, du;
};

__device__ __forceinline__ SwigluGrad swiglu_bwd_one(float g, float u, float da) {
  const float s = sigmoidf(g);
  const float silu = g * s;
  return SwigluGrad{silu * u, da * u * (s * (1.0f + g * (1.0f - s))), da * silu};
}

__global__ __launch_bounds__(kEwThreads) void swiglu_bwd_kernel(const float* __restrict__ g,
                                                                const float* __restrict__ u,
                                                                const float* __restrict__ da,
                                                                __bf16* __restrict__ a,
                                                                __bf16* __restrict__ dg,
                                                                __bf16* __restrict__ du, int64_t n) {
  const int64_t i = ((int64_t)blockIdx.x * kEwThreads + threadIdx.x) * 4;
  if (i + 4 <= n) {
    // g, u and da are read once: non-temporal
    const f32x4_t gv = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(g + i));
    const f32x4_t uv = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(u + i));
    const f32x4_t dv = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(da + i));
    SwigluGrad r[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) r[e] = swiglu_bwd_one(gv[e], uv[e], dv[e]);
    bf16x4_t oa, og, ou;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      oa[e] = (__bf16)r[e].a;
      og[e] = (__bf16)r[e].dg;
      ou[e] = (__bf16)r[e].du;
    }
    *reinterpret_cast<bf16x4_t*>(a + i) = oa;
    *reinterpret_cast<bf16x4_t*>(dg + i) = og;
    *reinterpret_cast<bf16x4_t*>(du + i) = ou;
  } else {
    for (int64_t j = i; j < n; ++j) {
      const SwigluGrad r = swiglu_bwd_one(g[j], u[j], da[j]);
      a[j] = (__bf16)r.a;
      dg[j] = (__bf16)r.dg;
      du[j] = (__bf16)r.du;
    }
  }
}

__global__ __launch_bounds__(kEwThreads) void f32_to_bf16_kernel(const float* __restrict__ x,
                                                                 __bf16* __restrict__ y, int64_t n) {
  const int64_t i = ((int64_t)blockIdx.x * kEwThreads + threadIdx.x) * 4;
  if (i + 4 <= n) {
    const float4 v = *reinterpret_cast<const float4*>(x + i);
    bf16x4_t o;
    o[0] = (__bf16)v.x;
    o[1] = (__bf16)v.y;
    o[2] = (__bf16)v.z;
    o[3] = (__bf16)v.w;
    *reinterpret_cast<bf16x4_t*>(y + i) = o;
  } else {
    for (int64_t j = i; j < n; ++j) y[j] = (__bf16)x[j];
  }
}

__global__ __launch_bounds__(kEwThreads) void fill_zero_kernel(float* __restrict__ x, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * kEwThreads + threadIdx.x;
  if (i < n) x[i] = 0.0f;
}

dim3 ew_grid(int64_t n) { return dim3((uint32_t)((n + 4 * kEwThreads - 1) / (4 * kEwThreads))); }

size_t al(size_t x) { return (x + 255) / 256 * 256; }

// Workspace regions of one shard.
struct MlpWork {
  float* g;
  float* u;
  float* da;      // backward only
  __bf16* a;
  __bf16* dg;     // backward only
  __bf16* du;     // backward only
  float* dx;      // backward only, [S, d]
};

MlpWork carve(void* ws, int64_t S, int64_t d, int64_t I) {
  char* p = static_cast<char*>(ws);
  const size_t f = al((size_t)S * I * 4), h = al((size_t)S * I * 2);
  MlpWork w;
  w.g = reinterpret_cast<float*>(p);
  w.u = reinterpret_cast<float*>(p + f);
  w.a = reinterpret_cast<__bf16*>(p + 2 * f);
  w.da = reinterpret_cast<float*>(p + 2 * f + h);
  w.dg = reinterpret_cast<__bf16*>(p + 3 * f + h);
  w.du = reinterpret_cast<__bf16*>(p + 3 * f + 2 * h);
  w.dx = reinterpret_cast<float*>(p + 3 * f + 3 * h);
  (void)d;
  return w;
}

// C (+)= X Y^T on the matrix-core GEMM; each operand given as (pointer,
// leading dimension, k-major?).
GemmOp gemm_op(const void* x, int64_t ldx, bool xk, const void* y, int64_t ldy, bool yk,
               int64_t nx, int64_t ny, int64_t K, void* c, int64_t ldc, bool c_bf16,
               bool accumulate) {
  GemmOp op{};
  op.x = GemmOperand{x, ldx, xk};
  op.y = GemmOperand{y, ldy, yk};
  op.nx = nx;
  op.ny = ny;
  op.K = K;
  op.c = c;
  op.ldc = ldc;
  op.c_bf16 = c_bf16;
  op.accumulate = accumulate;
  return op;
}

hipError_t gemm(const void* x, int64_t ldx, bool xk, const void* y, int64_t ldy, bool yk,
                int64_t nx, int64_t ny, int64_t K, void* c, int64_t ldc, bool c_bf16,
                bool accumulate, hipStream_t stream) {
  return launch_gemm(gemm_op(x, ldx, xk, y, ldy, yk, nx, ny, K, c, ldc, c_bf16, accumulate), stream);
}

// g and u of rows [r0, r0 + rows): g[s][i] = sum_k x[s][k] Wg[i][k].
hipError_t gate_up(const TiledMlpArgs& a, const MlpWork& w, int64_t r0, int64_t rows,
                   hipStream_t stream) {
  const __bf16* xs = static_cast<const __bf16*>(a.x) + r0 * a.d;
  // both products in one launch: their tiles fill one grid
  return launch_gemm_pair(gemm_op(xs, a.d, true, a.wg, a.d, true, rows, a.I, a.d, w.g, a.I, false, false),
                          gemm_op(xs, a.d, true, a.wu, a.d, true, rows, a.I, a.d, w.u, a.I, false, false),
                          stream);
}

}  // namespace

size_t tiled_mlp_workspace_bytes(int64_t shard_rows, int64_t d, int64_t I, bool backward) {
  const size_t f = al((size_t)shard_rows * I * 4), h = al((size_t)shard_rows * I * 2);
  if (!backward) return 2 * f + h;
  return 3 * f + 3 * h + al((size_t)shard_rows * d * 4);
}

hipError_t launch_tiled_mlp(const TiledMlpArgs& a, hipStream_t stream) {
  const int64_t d = a.d, I = a.I;
  const MlpWork w = carve(a.workspace, a.shard_rows, d, I);
  hipError_t e;
  if (a.backward && a.T == 0) {
    for (float* t : {a.dwg, a.dwu, a.dwd}) {
      e = launch_kernel(fill_zero_kernel, dim3((uint32_t)((I * d + kEwThreads - 1) / kEwThreads)),
                        dim3(kEwThreads), 0, stream, t, I * d);
      if (e != hipSuccess) return e;
    }
  }
  for (int64_t r0 = 0; r0 < a.T; r0 += a.shard_rows) {
    const int64_t rows = a.T - r0 < a.shard_rows ? a.T - r0 : a.shard_rows;
    const int64_t n = rows * I;
    if ((e = gate_up(a, w, r0, rows, stream)) != hipSuccess) return e;
    if (!a.backward) {
      e = launch_kernel(swiglu_fwd_kernel, ew_grid(n), dim3(kEwThreads), 0, stream, w.g, w.u, w.a, n);
      if (e != hipSuccess) return e;
      // y_s[s][j] = sum_i a[s][i] Wd[j][i]
      e = gemm(w.a, I, true, a.wd, I, true, rows, d, I, static_cast<__bf16*>(a.y) + r0 * d, d,
               true, false, stream);
      if (e != hipSuccess) return e;
      continue;
    }
    const __bf16* xs = static_cast<const __bf16*>(a.x) + r0 * d;
    const __bf16* dys = static_cast<const __bf16*>(a.dy) + r0 * d;
    const bool acc = r0 > 0;   // weight gradients: stored by the first shard, added to after
    // da[s][i] = sum_j dy[s][j] Wd[j][i]
    if ((e = gemm(dys, d, true, a.wd, I, false, rows, I, d, w.da, I, false, false, stream)) !=
        hipSuccess)
      return e;
    e = launch_kernel(swiglu_bwd_kernel, ew_grid(n), dim3(kEwThreads), 0, stream, w.g, w.u, w.da,
                      w.a, w.dg, w.du, n);
    if (e != hipSuccess) return e;
    // dWd[j][i] (+)= sum_s dy[s][j] a[s][i]
    if ((e = gemm(dys, d, false, w.a, I, false, d, I, rows, a.dwd, I, false, acc, stream)) !=
        hipSuccess)
      return e;
    // dWg[i][j] (+)= sum_s dg[s][i] x[s][j]; dWu likewise with du (one launch)
    if ((e = launch_gemm_pair(gemm_op(w.dg, I, false, xs, d, false, I, d, rows, a.dwg, d, false, acc),
                              gemm_op(w.du, I, false, xs, d, false, I, d, rows, a.dwu, d, false, acc),
                              stream)) != hipSuccess)
      return e;
    // dx[s][j] = sum_i dg[s][i] Wg[i][j] + sum_i du[s][i] Wu[i][j]
    if ((e = gemm(w.dg, I, true, a.wg, d, false, rows, d, I, w.dx, d, false, false, stream)) !=
            hipSuccess ||
        (e = gemm(w.du, I, true, a.wu, d, false, rows, d, I, w.dx, d, false, true, stream)) !=
            hipSuccess)
      return e;
    e = launch_kernel(f32_to_bf16_kernel, ew_grid(rows * d), dim3(kEwThreads), 0, stream, w.dx,
                      static_cast<__bf16*>(a.dx) + r0 * d, rows * d);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace ulysses
