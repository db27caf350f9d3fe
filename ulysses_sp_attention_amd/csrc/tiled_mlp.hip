// Sequence-tiled SwiGLU MLP (the integration guide's TiledMLP, section on
// the ALST memory tricks): y = (silu(x Wg^T) * (x Wu^T)) Wd^T computed a
// shard of token rows at a time, so the [T, I] intermediates exist for one
// shard only; the backward recomputes each shard's intermediates instead of
// keeping them (the guide's tiled compute replays the forward in the
// backward).  Rows are independent, so sharding changes no result.
//
// Per shard of S rows (intermediates in the workspace):
//   forward : g = x_s Wg^T, u = x_s Wu^T (fp32)   rocBLAS
//             a = bf16(silu(g) u)                  swiglu_fwd_kernel
//             y_s = a Wd^T (bf16)                  rocBLAS
//   backward: g, u as above; da = dy_s Wd (fp32)   rocBLAS
//             a, dg = bf16(da u silu'(g)), du = bf16(da silu(g))
//                                                  swiglu_bwd_kernel
//             dWd (+)= dy_s^T a; dWg (+)= dg^T x_s; dWu (+)= du^T x_s (fp32)
//             dx_s = dg Wg + du Wu (fp32, then bf16) rocBLAS + cast
// g, u and da stay fp32; only the operands of a GEMM are rounded to bf16.
#include "blas.h"
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

// g and u of rows [r0, r0 + rows).
bool gate_up(rocblas_handle hd, const TiledMlpArgs& a, const MlpWork& w, int64_t r0, int64_t rows) {
  const __bf16* xs = static_cast<const __bf16*>(a.x) + r0 * a.d;
  // g^T (col-major I x rows) = Wg (col-major d x I)^T . x_s^T (col-major d x rows)
  return gemm_bf16(hd, true, false, a.I, rows, a.d, a.wg, a.d, xs, a.d, 0.0f, w.g, false, a.I) &&
         gemm_bf16(hd, true, false, a.I, rows, a.d, a.wu, a.d, xs, a.d, 0.0f, w.u, false, a.I);
}

}  // namespace

size_t tiled_mlp_workspace_bytes(int64_t shard_rows, int64_t d, int64_t I, bool backward) {
  const size_t f = al((size_t)shard_rows * I * 4), h = al((size_t)shard_rows * I * 2);
  if (!backward) return 2 * f + h;
  return 3 * f + 3 * h + al((size_t)shard_rows * d * 4);
}

hipError_t launch_tiled_mlp(const TiledMlpArgs& a, hipStream_t stream) {
  rocblas_handle hd = blas_handle();
  if (!hd) return hipErrorNotInitialized;
  if (rocblas_set_stream(hd, stream) != rocblas_status_success) return hipErrorUnknown;
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
    if (!gate_up(hd, a, w, r0, rows)) return hipErrorUnknown;
    if (!a.backward) {
      e = launch_kernel(swiglu_fwd_kernel, ew_grid(n), dim3(kEwThreads), 0, stream, w.g, w.u, w.a, n);
      if (e != hipSuccess) return e;
      // y_s^T (col-major d x rows) = Wd (col-major I x d)^T . a^T (col-major I x rows)
      if (!gemm_bf16(hd, true, false, d, rows, I, a.wd, I, w.a, I, 0.0f,
                     static_cast<__bf16*>(a.y) + r0 * d, true, d))
        return hipErrorUnknown;
      continue;
    }
    const __bf16* xs = static_cast<const __bf16*>(a.x) + r0 * d;
    const __bf16* dys = static_cast<const __bf16*>(a.dy) + r0 * d;
    const float beta = r0 == 0 ? 0.0f : 1.0f;
    // da^T (col-major I x rows) = Wd (col-major I x d) . dy_s^T (col-major d x rows)
    if (!gemm_bf16(hd, false, false, I, rows, d, a.wd, I, dys, d, 0.0f, w.da, false, I))
      return hipErrorUnknown;
    e = launch_kernel(swiglu_bwd_kernel, ew_grid(n), dim3(kEwThreads), 0, stream, w.g, w.u, w.da,
                      w.a, w.dg, w.du, n);
    if (e != hipSuccess) return e;
    // dWd^T (col-major I x d) (+)= a^T (col-major I x rows) . dy_s (col-major d x rows)^T
    if (!gemm_bf16(hd, false, true, I, d, rows, w.a, I, dys, d, beta, a.dwd, false, I))
      return hipErrorUnknown;
    // dWg^T (col-major d x I) (+)= x_s^T (col-major d x rows) . dg (col-major I x rows)^T
    if (!gemm_bf16(hd, false, true, d, I, rows, xs, d, w.dg, I, beta, a.dwg, false, d) ||
        !gemm_bf16(hd, false, true, d, I, rows, xs, d, w.du, I, beta, a.dwu, false, d))
      return hipErrorUnknown;
    // dx_s^T (col-major d x rows) = Wg (col-major d x I) . dg^T + Wu . du^T
    if (!gemm_bf16(hd, false, false, d, rows, I, a.wg, d, w.dg, I, 0.0f, w.dx, false, d) ||
        !gemm_bf16(hd, false, false, d, rows, I, a.wu, d, w.du, I, 1.0f, w.dx, false, d))
      return hipErrorUnknown;
    e = launch_kernel(f32_to_bf16_kernel, ew_grid(rows * d), dim3(kEwThreads), 0, stream, w.dx,
                      static_cast<__bf16*>(a.dx) + r0 * d, rows * d);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace ulysses
