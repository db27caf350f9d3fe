// fp32 attention, forward and backward, on the vector ALUs.
//
// Same operation as the bf16 matrix-core path (standard scaled-dot-product
// softmax attention per head with causal / document visibility, Hugging
// Face Ulysses blog and integration guide), for fp32 storage where the
// result must hold to fp32 accuracy.  One thread owns one query row (forward,
// dQ) or one key row (dK, dV) and walks the visible keys (queries) with an
// online softmax; the rows a block's threads read at the same time are the
// same, so K/V (Q/dO) reads are broadcasts served from cache.
//
// Also holds the row-dot preprocess D_i = <dO_i, O_i> of the backward pass,
// shared by the fp32 and bf16 paths.
#include <math.h>

#include "device_common.h"
#include "launch.h"

namespace ulysses {

// D[b, h, i] = sum_d dO[i, b, h, d] * O[i, b, h, d] in fp32.  Rows are read in
// memory order; 16 bytes per lane, the lanes of a row reduced by shuffles.
template <typename T, int HD>
__global__ __launch_bounds__(256) void row_dot_kernel(const T* __restrict__ o,
                                                      const T* __restrict__ dout,
                                                      float* __restrict__ D, int64_t rows,
                                                      int64_t N, int bs, int hq) {
  constexpr int kVec = 16 / sizeof(T);
  constexpr int kLanes = HD / kVec;   // lanes per row (power of two, <= 64)
  constexpr int kRowsPerBlock = 256 / kLanes;
  const int64_t r = (int64_t)blockIdx.x * kRowsPerBlock + threadIdx.x / kLanes;
  const int sub = threadIdx.x % kLanes;
  float acc = 0.f;
  if (r < rows) {
    const T* a = o + r * HD + sub * kVec;
    const T* c = dout + r * HD + sub * kVec;
#pragma unroll
    for (int e = 0; e < kVec; ++e) acc += (float)a[e] * (float)c[e];
  }
#pragma unroll
  for (int off = kLanes / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off, 64);
  if (r < rows && sub == 0) {
    // r enumerates (i, b, h) in memory order
    const int h = (int)(r % hq);
    const int64_t ib = r / hq;
    const int b = (int)(ib % bs);
    const int64_t i = ib / bs;
    D[((int64_t)b * hq + h) * N + i] = acc;
  }
}

template <typename T, int HD>
hipError_t launch_row_dot(const T* o, const T* dout, float* D, const AttnShape& s,
                          hipStream_t stream) {
  constexpr int kLanes = HD / (16 / sizeof(T));
  constexpr int kRowsPerBlock = 256 / kLanes;
  const int64_t rows = s.N * s.bs * s.hq;
  const int64_t blocks = (rows + kRowsPerBlock - 1) / kRowsPerBlock;
  return launch_kernel(row_dot_kernel<T, HD>, dim3((uint32_t)blocks), dim3(256), 0, stream, o, dout,
                       D, rows, s.N, s.bs, s.hq);
}


namespace {

struct F32Params {
  const float* q;
  const float* k;
  const float* v;
  const float* o;
  const float* lse;
  const float* dout;
  const float* D;
  float* out0;   // o (forward) or dq
  float* out1;   // lse (forward) or dk
  float* out2;   // dv
  int64_t N;
  int bs, hq, hkv, g;
  float scale;
  int causal;
  const int32_t* cu;
  int n_docs;
};

constexpr int kF32Threads = 64;

template <int HD>
__global__ __launch_bounds__(kF32Threads) void attn_fwd_f32_kernel(F32Params p) {
  const int64_t i = (int64_t)blockIdx.x * kF32Threads + threadIdx.x;
  const int h = blockIdx.y % p.hq;
  const int b = blockIdx.y / p.hq;
  if (i >= p.N) return;
  const int kh = h / p.g;
  const int64_t q_tok = (int64_t)p.bs * p.hq * HD;
  const int64_t kv_tok = (int64_t)p.bs * p.hkv * HD;
  const float* qrow = p.q + i * q_tok + ((int64_t)b * p.hq + h) * HD;
  const float* kb = p.k + ((int64_t)b * p.hkv + kh) * HD;
  const float* vb = p.v + ((int64_t)b * p.hkv + kh) * HD;
  float qr[HD], acc[HD];
#pragma unroll
  for (int e = 0; e < HD; ++e) {
    qr[e] = qrow[e];
    acc[e] = 0.f;
  }
  const int64_t lo = doc_start_of(p.cu, p.n_docs, i);
  const int64_t hi = p.causal ? i + 1 : doc_end_of(p.cu, p.n_docs, i, p.N);
  float m = -INFINITY, l = 0.f;
  for (int64_t j = lo; j < hi; ++j) {
    const float* kr = kb + j * kv_tok;
    const float* vr = vb + j * kv_tok;
    float s = 0.f;
#pragma unroll
    for (int e = 0; e < HD; ++e) s = fmaf(qr[e], kr[e], s);
    s *= p.scale;
    const float mn = fmaxf(m, s);
    const float corr = expf(m - mn);
    const float pj = expf(s - mn);
    l = l * corr + pj;
#pragma unroll
    for (int e = 0; e < HD; ++e) acc[e] = fmaf(pj, vr[e], acc[e] * corr);
    m = mn;
  }
  float* orow = p.out0 + i * q_tok + ((int64_t)b * p.hq + h) * HD;
  const float inv = 1.f / l;
#pragma unroll
  for (int e = 0; e < HD; ++e) orow[e] = acc[e] * inv;
  p.out1[((int64_t)b * p.hq + h) * p.N + i] = m + logf(l);
}

template <int HD>
__global__ __launch_bounds__(kF32Threads) void attn_bwd_dq_f32_kernel(F32Params p) {
  const int64_t i = (int64_t)blockIdx.x * kF32Threads + threadIdx.x;
  const int h = blockIdx.y % p.hq;
  const int b = blockIdx.y / p.hq;
  if (i >= p.N) return;
  const int kh = h / p.g;
  const int64_t q_tok = (int64_t)p.bs * p.hq * HD;
  const int64_t kv_tok = (int64_t)p.bs * p.hkv * HD;
  const int64_t row_off = i * q_tok + ((int64_t)b * p.hq + h) * HD;
  const float* kb = p.k + ((int64_t)b * p.hkv + kh) * HD;
  const float* vb = p.v + ((int64_t)b * p.hkv + kh) * HD;
  float qr[HD], dor[HD], acc[HD];
#pragma unroll
  for (int e = 0; e < HD; ++e) {
    qr[e] = p.q[row_off + e];
    dor[e] = p.dout[row_off + e];
    acc[e] = 0.f;
  }
  const int64_t stat = ((int64_t)b * p.hq + h) * p.N + i;
  const float lse = p.lse[stat];
  const float Di = p.D[stat];
  const int64_t lo = doc_start_of(p.cu, p.n_docs, i);
  const int64_t hi = p.causal ? i + 1 : doc_end_of(p.cu, p.n_docs, i, p.N);
  for (int64_t j = lo; j < hi; ++j) {
    const float* kr = kb + j * kv_tok;
    const float* vr = vb + j * kv_tok;
    float s = 0.f, dp = 0.f;
#pragma unroll
    for (int e = 0; e < HD; ++e) {
      s = fmaf(qr[e], kr[e], s);
      dp = fmaf(dor[e], vr[e], dp);
    }
    const float pij = expf(s * p.scale - lse);
    const float ds = pij * (dp - Di);
#pragma unroll
    for (int e = 0; e < HD; ++e) acc[e] = fmaf(ds, kr[e], acc[e]);
  }
#pragma unroll
  for (int e = 0; e < HD; ++e) p.out0[row_off + e] = acc[e] * p.scale;
}

template <int HD>
__global__ __launch_bounds__(kF32Threads) void attn_bwd_dkv_f32_kernel(F32Params p) {
  const int64_t j = (int64_t)blockIdx.x * kF32Threads + threadIdx.x;
  const int kh = blockIdx.y % p.hkv;
  const int b = blockIdx.y / p.hkv;
  if (j >= p.N) return;
  const int64_t q_tok = (int64_t)p.bs * p.hq * HD;
  const int64_t kv_tok = (int64_t)p.bs * p.hkv * HD;
  const int64_t kv_off = j * kv_tok + ((int64_t)b * p.hkv + kh) * HD;
  float kr[HD], vr[HD], dk[HD], dv[HD];
#pragma unroll
  for (int e = 0; e < HD; ++e) {
    kr[e] = p.k[kv_off + e];
    vr[e] = p.v[kv_off + e];
    dk[e] = 0.f;
    dv[e] = 0.f;
  }
  const int64_t lo = p.causal ? j : doc_start_of(p.cu, p.n_docs, j);
  const int64_t hi = doc_end_of(p.cu, p.n_docs, j, p.N);
  for (int hh = 0; hh < p.g; ++hh) {
    const int h = kh * p.g + hh;
    const float* qb = p.q + ((int64_t)b * p.hq + h) * HD;
    const float* db = p.dout + ((int64_t)b * p.hq + h) * HD;
    const float* lse = p.lse + ((int64_t)b * p.hq + h) * p.N;
    const float* Dr = p.D + ((int64_t)b * p.hq + h) * p.N;
    for (int64_t i = lo; i < hi; ++i) {
      const float* qr = qb + i * q_tok;
      const float* dr = db + i * q_tok;
      float s = 0.f, dp = 0.f;
#pragma unroll
      for (int e = 0; e < HD; ++e) {
        s = fmaf(qr[e], kr[e], s);
        dp = fmaf(dr[e], vr[e], dp);
      }
      const float pij = expf(s * p.scale - lse[i]);
      const float ds = pij * (dp - Dr[i]);
#pragma unroll
      for (int e = 0; e < HD; ++e) {
        dk[e] = fmaf(ds, qr[e], dk[e]);
        dv[e] = fmaf(pij, dr[e], dv[e]);
      }
    }
  }
#pragma unroll
  for (int e = 0; e < HD; ++e) {
    p.out1[kv_off + e] = dk[e] * p.scale;
    p.out2[kv_off + e] = dv[e];
  }
}

F32Params base_params(const AttnShape& s) {
  F32Params p{};
  p.N = s.N;
  p.bs = s.bs;
  p.hq = s.hq;
  p.hkv = s.hkv;
  p.g = s.hq / s.hkv;
  p.scale = s.scale;
  p.causal = s.causal;
  p.cu = s.cu;
  p.n_docs = s.n_docs;
  return p;
}

template <int HD>
hipError_t fwd_f32(const F32Params& p, hipStream_t stream) {
  dim3 grid((uint32_t)((p.N + kF32Threads - 1) / kF32Threads), (uint32_t)(p.bs * p.hq));
  return launch_kernel(attn_fwd_f32_kernel<HD>, grid, dim3(kF32Threads), 0, stream, p);
}

template <int HD>
hipError_t bwd_f32(const F32Params& p, const AttnShape& s, hipStream_t stream) {
  hipError_t e = launch_row_dot<float, HD>(p.o, p.dout, const_cast<float*>(p.D), s, stream);
  if (e != hipSuccess) return e;
  const uint32_t nb = (uint32_t)((p.N + kF32Threads - 1) / kF32Threads);
  e = launch_kernel(attn_bwd_dq_f32_kernel<HD>, dim3(nb, (uint32_t)(p.bs * p.hq)),
                    dim3(kF32Threads), 0, stream, p);
  if (e != hipSuccess) return e;
  return launch_kernel(attn_bwd_dkv_f32_kernel<HD>, dim3(nb, (uint32_t)(p.bs * p.hkv)),
                       dim3(kF32Threads), 0, stream, p);
}

}  // namespace

hipError_t launch_attn_fwd_f32(const AttnShape& s, const float* q, const float* k, const float* v,
                               float* o, float* lse, hipStream_t stream) {
  if (s.N == 0) return hipSuccess;
  F32Params p = base_params(s);
  p.q = q;
  p.k = k;
  p.v = v;
  p.out0 = o;
  p.out1 = lse;
  switch (s.hd) {
    case 32: return fwd_f32<32>(p, stream);
    case 64: return fwd_f32<64>(p, stream);
    case 128: return fwd_f32<128>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_attn_bwd_f32(const AttnShape& s, const float* q, const float* k, const float* v,
                               const float* o, const float* lse, const float* dout, float* dq,
                               float* dk, float* dv, void* workspace, hipStream_t stream) {
  if (s.N == 0) return hipSuccess;
  F32Params p = base_params(s);
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.lse = lse;
  p.dout = dout;
  p.D = static_cast<const float*>(workspace);
  p.out0 = dq;
  p.out1 = dk;
  p.out2 = dv;
  switch (s.hd) {
    case 32: return bwd_f32<32>(p, s, stream);
    case 64: return bwd_f32<64>(p, s, stream);
    case 128: return bwd_f32<128>(p, s, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace ulysses
