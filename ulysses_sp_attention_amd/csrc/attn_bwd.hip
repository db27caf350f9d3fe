// Backward pass of the bf16 attention on gfx950 matrix cores.
//
// Gradient of O_i = sum_j P_ij v_j, P_ij = exp(s_ij - LSE_i),
// s_ij = scale <q_i, k_j> (the attention each rank runs for its heads,
// Hugging Face Ulysses blog; training backpropagates through it):
//   D_i   = <dO_i, O_i>
//   dS_ij = P_ij (<dO_i, v_j> - D_i)
//   dQ_i  = scale sum_j dS_ij k_j
//   dK_j  = scale sum_{h in group} sum_i dS_ij q_i
//   dV_j  = sum_{h in group} sum_i P_ij dO_i
// P is recomputed from Q, K and the saved LSE; nothing of size N x N is
// stored.  Three launches on the caller's stream:
//   1. D for every query row (row_dot_kernel, in attn_f32.hip);
//   2. dQ: a workgroup owns query rows (as in the forward) and walks the
//      visible key tiles staged in LDS;
//   3. dK, dV: a workgroup owns 128 key rows of one key/value head and walks
//      the visible query tiles of every query head of its group, so the GQA
//      sum over heads happens in registers; no atomics anywhere, so results
//      are deterministic.
// Every product is a v_mfma_f32_32x32x16_bf16.  Operands whose contraction
// runs along the sequence (dV = P^T dO, dK = dS^T Q, dQ = dS K) come from
// LDS through the transposing read ds_read_b64_tr_b16, so all tiles keep
// their natural row layout in LDS.
#include <math.h>

#include <type_traits>

#include "device_common.h"
#include "launch.h"

namespace ulysses {

template <typename T, int HD>
hipError_t launch_row_dot(const T* o, const T* dout, float* D, const AttnShape& s,
                          hipStream_t stream);

namespace {

struct BwdParams {
  const __bf16* q;
  const __bf16* k;
  const __bf16* v;
  const __bf16* dout;
  const float* lse;
  const float* D;
  __bf16* dq;
  __bf16* dk;
  __bf16* dv;
  int64_t N;
  int bs, hq, hkv, g;
  float scale;
  float scale_log2;
  int causal;
  const int32_t* cu;
  int n_docs;
  int64_t num_blocks;
};

// A operand (rows = head dim, k = 16 sequence positions starting at row0)
// read transposed from a row-major swizzled LDS tile: lane l gets the
// values of column d = 32*db + l%32 at the 8 sequence rows matching the
// accumulator layout of the other operand.
template <int kChunks, int kRowBytes>
__device__ __forceinline__ bf16x8_t load_tr_operand(const char* tile, int row0, int db, int lane) {
  const int grp = lane >> 4;
  const int u = lane & 15;
  bf16x4_t part[2];
#pragma unroll
  for (int jh = 0; jh < 2; ++jh) {
    const int row = row0 + 8 * jh + 4 * (grp >> 1) + (u >> 2);
    const int col = db * 32 + 16 * (grp & 1) + 4 * (u & 3);
    const int off = swz<kChunks, kRowBytes>(row, col >> 3) + ((col >> 2) & 1) * 8;
    part[jh] = lds_read_tr16(tile + off);
  }
  return __builtin_shufflevector(part[0], part[1], 0, 1, 2, 3, 4, 5, 6, 7);
}

// ------------------------------------------------------------------------
// dQ
// ------------------------------------------------------------------------
template <int HD, int GPACK>
struct DqCfg {
  static constexpr int kWaves = 8;
  static constexpr int kThreads = 64 * kWaves;
  static constexpr int kBP = 32 * kWaves / GPACK;
  static constexpr int kBC = 64;
  static constexpr int kChunks = HD / 8;
  static constexpr int kRowBytes = HD * 2;
  static constexpr int kTileBytes = kBC * kRowBytes;
  static constexpr int kKS = HD / 16;
  static constexpr int kDB = HD / 32;
  static constexpr int kLoads = kBC * kChunks / kThreads;
};

template <int HD, int GPACK>
__global__ __launch_bounds__(512) void attn_bwd_dq_kernel(BwdParams p) {
  using C = DqCfg<HD, GPACK>;
  __shared__ __attribute__((aligned(16))) char smem[2 * C::kTileBytes];
  char* lds_k = smem;
  char* lds_v = smem + C::kTileBytes;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int half = lane >> 5;
  const int r32 = lane & 31;

  const int64_t N = p.N;
  const int64_t pb = p.num_blocks - 1 - (int64_t)blockIdx.x;
  const int ngroups = p.g / GPACK;
  int y = blockIdx.y;
  const int hg = y % ngroups;
  y /= ngroups;
  const int kh = y % p.hkv;
  const int b = y / p.hkv;
  const int h = kh * p.g + hg * GPACK + (wave % GPACK);

  const int64_t p0 = pb * C::kBP;
  const int64_t pw = p0 + (int64_t)(wave / GPACK) * 32;
  const int64_t qi = pw + r32;

  const int64_t q_tok = (int64_t)p.bs * p.hq * HD;
  const int64_t kv_tok = (int64_t)p.bs * p.hkv * HD;
  const int64_t qoff = ((int64_t)b * p.hq + h) * HD;
  const __bf16* kbase = p.k + ((int64_t)b * p.hkv + kh) * HD;
  const __bf16* vbase = p.v + ((int64_t)b * p.hkv + kh) * HD;

  bf16x8_t qf[C::kKS], df[C::kKS];
#pragma unroll
  for (int ks = 0; ks < C::kKS; ++ks) {
    if (qi < N) {
      qf[ks] = *reinterpret_cast<const bf16x8_t*>(p.q + qi * q_tok + qoff + 16 * ks + 8 * half);
      df[ks] = *reinterpret_cast<const bf16x8_t*>(p.dout + qi * q_tok + qoff + 16 * ks + 8 * half);
    } else {
      qf[ks] = bf16x8_t{};
      df[ks] = bf16x8_t{};
    }
  }
  const int64_t stat = ((int64_t)b * p.hq + h) * N + qi;
  const float lse2 = qi < N ? p.lse[stat] * kLog2e : 0.f;
  const float Di = qi < N ? p.D[stat] : 0.f;

  const int64_t blk_last = (p0 + C::kBP < N ? p0 + C::kBP : N) - 1;
  const int64_t kv_lo = doc_start_of(p.cu, p.n_docs, p0);
  const int64_t kv_hi = p.causal ? blk_last + 1 : doc_end_of(p.cu, p.n_docs, blk_last, N);
  const bool wave_active = pw < N;
  const int64_t w_last = wave_active ? (pw + 31 < N ? pw + 31 : N - 1) : 0;
  const int64_t w_lo = wave_active ? doc_start_of(p.cu, p.n_docs, pw) : 0;
  const int64_t w_hi = wave_active ? (p.causal ? w_last + 1 : doc_end_of(p.cu, p.n_docs, w_last, N)) : 0;
  const int64_t full_lo = wave_active ? doc_start_of(p.cu, p.n_docs, w_last) : 0;
  const int64_t full_hi = wave_active ? (p.causal ? pw + 1 : doc_end_of(p.cu, p.n_docs, pw, N)) : 0;
  const int64_t my_lo = qi < N ? doc_start_of(p.cu, p.n_docs, qi) : 0;
  const int64_t my_hi = qi < N ? (p.causal ? qi + 1 : doc_end_of(p.cu, p.n_docs, qi, N)) : 0;
  const int64_t t_begin = kv_lo / C::kBC;
  const int64_t t_end = (kv_hi + C::kBC - 1) / C::kBC;

  f32x16_t acc[C::kDB];
#pragma unroll
  for (int db = 0; db < C::kDB; ++db) acc[db] = f32x16_t{};

  u32x4_t kst[C::kLoads], vst[C::kLoads];
  auto load_tile = [&](int64_t t) {
#pragma unroll
    for (int i = 0; i < C::kLoads; ++i) {
      const int cid = tid + i * C::kThreads;
      const int64_t j = t * C::kBC + cid / C::kChunks;
      const int ch = cid % C::kChunks;
      if (j < N) {
        kst[i] = *reinterpret_cast<const u32x4_t*>(kbase + j * kv_tok + ch * 8);
        vst[i] = *reinterpret_cast<const u32x4_t*>(vbase + j * kv_tok + ch * 8);
      } else {
        kst[i] = u32x4_t{};
        vst[i] = u32x4_t{};
      }
    }
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int i = 0; i < C::kLoads; ++i) {
      const int cid = tid + i * C::kThreads;
      const int off = swz<C::kChunks, C::kRowBytes>(cid / C::kChunks, cid % C::kChunks);
      *reinterpret_cast<u32x4_t*>(lds_k + off) = kst[i];
      *reinterpret_cast<u32x4_t*>(lds_v + off) = vst[i];
    }
  };

  if (t_begin < t_end) load_tile(t_begin);
  for (int64_t t = t_begin; t < t_end; ++t) {
    __syncthreads();
    store_tile();
    __syncthreads();
    if (t + 1 < t_end) load_tile(t + 1);
    const int64_t j0 = t * C::kBC;
    if (!wave_active || j0 >= w_hi || j0 + C::kBC <= w_lo) continue;
    const bool need_mask = j0 < full_lo || j0 + C::kBC > full_hi;

#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      // S^T = K Q^T and dP^T = V dO^T for 32 keys; the K and V fragments of
      // each k-step are read from LDS two steps ahead of their products.
      f32x16_t s = f32x16_t{}, dp = f32x16_t{};
      {
        const int row = kb * 32 + r32;
        auto frags = [&](int ks, bf16x8_t& kfr, bf16x8_t& vfr) {
          const int off = swz<C::kChunks, C::kRowBytes>(row, 2 * ks + half);
          kfr = *reinterpret_cast<const bf16x8_t*>(lds_k + off);
          vfr = *reinterpret_cast<const bf16x8_t*>(lds_v + off);
        };
        bf16x8_t kb3[3], vb3[3];
        frags(0, kb3[0], vb3[0]);
        frags(1, kb3[1], vb3[1]);
#pragma unroll
        for (int ks = 0; ks < C::kKS; ++ks) {
          if (ks + 2 < C::kKS) frags(ks + 2, kb3[(ks + 2) % 3], vb3[(ks + 2) % 3]);
          s = mfma32(kb3[ks % 3], qf[ks], s);
          dp = mfma32(vb3[ks % 3], df[ks], dp);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      bf16x8_t dsf[2];
      if (need_mask) {
        // visible keys of this row as offsets into the 32-key block, clamped;
        // invisible scores become -inf so their P and dS are exactly 0
        const int64_t jb = j0 + kb * 32;
        const int lo = (int)(my_lo - jb < -1 ? -1 : (my_lo - jb > 33 ? 33 : my_lo - jb));
        const int hi = (int)(my_hi - jb < -1 ? -1 : (my_hi - jb > 33 ? 33 : my_hi - jb));
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int j = 8 * (i >> 2) + 4 * half + (i & 3);
          if (j < lo || j >= hi) s[i] = -INFINITY;
        }
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float pv = __builtin_amdgcn_exp2f(fmaf(s[i], p.scale_log2, -lse2));
        dsf[i >> 3][i & 7] = (__bf16)(pv * (dp[i] - Di));
      }
      // dQ^T += K^T dS^T; K^T fragments by transposing LDS reads, two
      // products ahead, four independent accumulator chains.
      {
        constexpr int kSteps = 2 * C::kDB;   // (ks2, db) pairs, db fastest
        auto ktfrag = [&](int idx) {
          return load_tr_operand<C::kChunks, C::kRowBytes>(lds_k, kb * 32 + 16 * (idx / C::kDB),
                                                           idx % C::kDB, lane);
        };
        bf16x8_t buf[3];
        buf[0] = ktfrag(0);
        buf[1] = ktfrag(1);
#pragma unroll
        for (int idx = 0; idx < kSteps; ++idx) {
          if (idx + 2 < kSteps) buf[(idx + 2) % 3] = ktfrag(idx + 2);
          acc[idx % C::kDB] = mfma32(buf[idx % 3], dsf[idx / C::kDB], acc[idx % C::kDB]);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
  }

  if (qi >= N) return;
  __bf16* orow = p.dq + qi * q_tok + qoff;
#pragma unroll
  for (int db = 0; db < C::kDB; ++db)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      bf16x4_t w;
#pragma unroll
      for (int e = 0; e < 4; ++e) w[e] = (__bf16)(acc[db][4 * r4 + e] * p.scale);
      *reinterpret_cast<bf16x4_t*>(orow + db * 32 + 8 * r4 + 4 * half) = w;
    }
}

// ------------------------------------------------------------------------
// dK, dV
// ------------------------------------------------------------------------
// A workgroup of WAVES waves owns WAVES * KB * 32 key rows of one key/value
// head; each wave owns KB blocks of 32 rows and keeps their K fragments and
// its dK^T, dV^T accumulators in registers.  V for the workgroup's rows stays
// in LDS (B operand of dP = dO V^T).  The workgroup walks the visible query
// positions in tiles of BQ, from the last tile down to the first, and within
// a tile every query head of the GQA group; each (tile, head) step stages Q,
// dO, LSE and D in LDS once for all its keys, and every Q or dO fragment a
// wave reads from LDS feeds all KB of its key blocks.  Walking queries from
// the end keeps the workgroups resident at the same time on the same query
// tiles, so those tiles are shared through L2.  The launch uses 4 waves of
// one 32-row block each (128 keys, one wave per SIMD): larger shapes do not
// fit the register file without spilling.
template <int HD, int WAVES = 4, int KB = 2, int BQ = 64>
struct DkvCfg {
  static constexpr int kWaves = WAVES;
  static constexpr int kThreads = 64 * kWaves;
  static constexpr int kKB = KB;              // 32-row key blocks per wave
  static constexpr int kBK = 32 * kKB * kWaves;   // key rows per workgroup
  static constexpr int kBQ = BQ;              // query rows per step
  static constexpr int kChunks = HD / 8;
  static constexpr int kRowBytes = HD * 2;
  static constexpr int kVBytes = kBK * kRowBytes;
  static constexpr int kTileBytes = kBQ * kRowBytes;
  static constexpr int kKS = HD / 16;
  static constexpr int kDB = HD / 32;
  static constexpr int kLoads = kBQ * kChunks / kThreads;   // per tensor per step
  static constexpr int kVLoads = kBK * kChunks / kThreads;
  static_assert(kLoads >= 1 && kBQ * kChunks % kThreads == 0, "tile loads");
};

template <int HD, int WAVES, int KB, int BQ, int PF>
__global__ __launch_bounds__(64 * WAVES) void attn_bwd_dkv_kernel(BwdParams p) {
  using C = DkvCfg<HD, WAVES, KB, BQ>;
  __shared__ __attribute__((aligned(16))) char smem[C::kVBytes + 2 * C::kTileBytes + 2 * C::kBQ * 4];
  char* lds_v = smem;
  char* lds_q = smem + C::kVBytes;
  char* lds_do = lds_q + C::kTileBytes;
  float* lds_lse = reinterpret_cast<float*>(lds_do + C::kTileBytes);
  float* lds_D = lds_lse + C::kBQ;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int half = lane >> 5;
  const int r32 = lane & 31;

  const int64_t N = p.N;
  const int kh = blockIdx.y % p.hkv;
  const int b = blockIdx.y / p.hkv;
  const int64_t k0 = (int64_t)blockIdx.x * C::kBK;   // heaviest (smallest keys) first
  const int64_t kw = k0 + 32 * C::kKB * wave;       // first key row of this wave

  const int64_t q_tok = (int64_t)p.bs * p.hq * HD;
  const int64_t kv_tok = (int64_t)p.bs * p.hkv * HD;
  const int64_t kvoff = ((int64_t)b * p.hkv + kh) * HD;

  // K rows of this lane (B operand of S = Q K^T), one per key block.
  bf16x8_t kf[C::kKB][C::kKS];
  int64_t my_lo[C::kKB], my_hi[C::kKB];
#pragma unroll
  for (int kb = 0; kb < C::kKB; ++kb) {
    const int64_t kj = kw + 32 * kb + r32;
#pragma unroll
    for (int ks = 0; ks < C::kKS; ++ks)
      kf[kb][ks] = kj < N ? *reinterpret_cast<const bf16x8_t*>(p.k + kj * kv_tok + kvoff + 16 * ks + 8 * half)
                          : bf16x8_t{};
    // queries that see key kj: [causal ? kj : doc_start(kj), doc_end(kj))
    my_lo[kb] = kj < N ? (p.causal ? kj : doc_start_of(p.cu, p.n_docs, kj)) : 0;
    my_hi[kb] = kj < N ? doc_end_of(p.cu, p.n_docs, kj, N) : 0;
  }
  // V rows of the whole workgroup into LDS.
#pragma unroll
  for (int i = 0; i < C::kVLoads; ++i) {
    const int cid = tid + i * C::kThreads;
    const int row = cid / C::kChunks;
    const int ch = cid % C::kChunks;
    const int64_t j = k0 + row;
    const u32x4_t val = j < N ? *reinterpret_cast<const u32x4_t*>(p.v + j * kv_tok + kvoff + ch * 8)
                              : u32x4_t{};
    *reinterpret_cast<u32x4_t*>(lds_v + swz<C::kChunks, C::kRowBytes>(row, ch)) = val;
  }

  const int64_t k_last = (k0 + C::kBK < N ? k0 + C::kBK : N) - 1;
  const int64_t q_lo = p.causal ? k0 : doc_start_of(p.cu, p.n_docs, k0);
  const int64_t q_hi = doc_end_of(p.cu, p.n_docs, k_last, N);
  const bool wave_active = kw < N;
  const int64_t w_last = wave_active ? (kw + 32 * C::kKB - 1 < N ? kw + 32 * C::kKB - 1 : N - 1) : 0;
  const int64_t w_lo = wave_active ? (p.causal ? kw : doc_start_of(p.cu, p.n_docs, kw)) : 0;
  const int64_t w_hi = wave_active ? doc_end_of(p.cu, p.n_docs, w_last, N) : 0;
  // Queries seen by every key of the wave: [full_lo, full_hi).
  const int64_t full_lo = wave_active ? (p.causal ? w_last : doc_start_of(p.cu, p.n_docs, w_last)) : 0;
  const int64_t full_hi = wave_active ? doc_end_of(p.cu, p.n_docs, kw, N) : 0;

  const int64_t qt_lo = q_lo / C::kBQ;
  const int64_t qt_hi = (q_hi + C::kBQ - 1) / C::kBQ;
  // Steps run from the last query tile down: step n is tile qt_hi-1-n/g, head n%g.
  const int64_t n_steps = (qt_hi - qt_lo) * p.g;

  f32x16_t acc_dk[C::kKB][C::kDB], acc_dv[C::kKB][C::kDB];
#pragma unroll
  for (int kb = 0; kb < C::kKB; ++kb)
#pragma unroll
    for (int db = 0; db < C::kDB; ++db) {
      acc_dk[kb][db] = f32x16_t{};
      acc_dv[kb][db] = f32x16_t{};
    }

  u32x4_t qst[C::kLoads], dst[C::kLoads];
  float sst = 0.f;
  auto load_step = [&](int64_t n) {
    const int64_t i0 = (qt_hi - 1 - n / p.g) * C::kBQ;
    const int h = kh * p.g + (int)(n % p.g);
    const int64_t qoff = ((int64_t)b * p.hq + h) * HD;
#pragma unroll
    for (int i = 0; i < C::kLoads; ++i) {
      const int cid = tid + i * C::kThreads;
      const int64_t qi = i0 + cid / C::kChunks;
      const int ch = cid % C::kChunks;
      if (qi < N) {
        qst[i] = *reinterpret_cast<const u32x4_t*>(p.q + qi * q_tok + qoff + ch * 8);
        dst[i] = *reinterpret_cast<const u32x4_t*>(p.dout + qi * q_tok + qoff + ch * 8);
      } else {
        qst[i] = u32x4_t{};
        dst[i] = u32x4_t{};
      }
    }
    if (tid < 2 * C::kBQ) {
      const int64_t qi = i0 + (tid % C::kBQ);
      const int64_t idx = ((int64_t)b * p.hq + h) * N + qi;
      sst = qi < N ? (tid < C::kBQ ? p.lse[idx] * kLog2e : p.D[idx]) : 0.f;
    }
  };
  auto store_step = [&]() {
#pragma unroll
    for (int i = 0; i < C::kLoads; ++i) {
      const int cid = tid + i * C::kThreads;
      const int off = swz<C::kChunks, C::kRowBytes>(cid / C::kChunks, cid % C::kChunks);
      *reinterpret_cast<u32x4_t*>(lds_q + off) = qst[i];
      *reinterpret_cast<u32x4_t*>(lds_do + off) = dst[i];
    }
    if (tid < 2 * C::kBQ) lds_lse[tid] = sst;   // lds_D follows lds_lse
  };

  if (n_steps > 0) load_step(0);
  for (int64_t n = 0; n < n_steps; ++n) {
    __syncthreads();
    store_step();
    __syncthreads();
    if (n + 1 < n_steps) load_step(n + 1);
    const int64_t i0 = (qt_hi - 1 - n / p.g) * C::kBQ;
    if (!wave_active || i0 >= w_hi || i0 + C::kBQ <= w_lo) continue;

#pragma unroll 1
    for (int sub = 0; sub < C::kBQ / 32; ++sub) {
      const int64_t s0 = i0 + 32 * sub;
      if (s0 >= w_hi || s0 + 32 <= w_lo) continue;
      const bool need_mask = s0 < full_lo || s0 + 32 > full_hi;
      // S = Q K^T and dP = dO V^T for every key block: lane holds key
      // kw + 32 kb + lane%32 and 16 query rows.  The Q, dO and V fragments of
      // each k-step are read from LDS PF steps ahead of their products.
      f32x16_t s[C::kKB], dp[C::kKB];
#pragma unroll
      for (int kb = 0; kb < C::kKB; ++kb) {
        s[kb] = f32x16_t{};
        dp[kb] = f32x16_t{};
      }
      {
        struct Frags {
          bf16x8_t qa, da, vb[C::kKB];
        };
        auto frags = [&](int ks) {
          Frags f;
          const int off = swz<C::kChunks, C::kRowBytes>(32 * sub + r32, 2 * ks + half);
          f.qa = *reinterpret_cast<const bf16x8_t*>(lds_q + off);
          f.da = *reinterpret_cast<const bf16x8_t*>(lds_do + off);
#pragma unroll
          for (int kb = 0; kb < C::kKB; ++kb)
            f.vb[kb] = *reinterpret_cast<const bf16x8_t*>(
                lds_v + swz<C::kChunks, C::kRowBytes>(32 * (C::kKB * wave + kb) + r32, 2 * ks + half));
          return f;
        };
        Frags buf[PF + 1];
#pragma unroll
        for (int i = 0; i < PF; ++i) buf[i] = frags(i);
#pragma unroll
        for (int ks = 0; ks < C::kKS; ++ks) {
          if (ks + PF < C::kKS) buf[(ks + PF) % (PF + 1)] = frags(ks + PF);
          const Frags& f = buf[ks % (PF + 1)];
#pragma unroll
          for (int kb = 0; kb < C::kKB; ++kb) {
            s[kb] = mfma32(f.qa, kf[kb][ks], s[kb]);
            dp[kb] = mfma32(f.da, f.vb[kb], dp[kb]);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      // On sub-tiles that cross a boundary, scores of invisible (query, key)
      // pairs become -inf, so their P and dS are exactly 0.
      if (need_mask) {
#pragma unroll
        for (int kb = 0; kb < C::kKB; ++kb) {
          // visible queries of this key as offsets into the 32-row sub-tile
          const int lo = (int)(my_lo[kb] - s0 < -1 ? -1 : (my_lo[kb] - s0 > 33 ? 33 : my_lo[kb] - s0));
          const int hi = (int)(my_hi[kb] - s0 < -1 ? -1 : (my_hi[kb] - s0 > 33 ? 33 : my_hi[kb] - s0));
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int qr = 8 * (i >> 2) + 4 * half + (i & 3);
            if (qr < lo || qr >= hi) s[kb][i] = -INFINITY;
          }
        }
      }
      // dO^T and Q^T fragments (transposing LDS reads) for the (16-row step,
      // head-dim block) products, read PF products ahead.
      struct TrFrags {
        bf16x8_t dot, qt;
      };
      constexpr int kTrSteps = 2 * C::kDB;
      auto trfrags = [&](int idx) {
        TrFrags f;
        const int ks2 = idx / C::kDB, db = idx % C::kDB;
        f.dot = load_tr_operand<C::kChunks, C::kRowBytes>(lds_do, 32 * sub + 16 * ks2, db, lane);
        f.qt = load_tr_operand<C::kChunks, C::kRowBytes>(lds_q, 32 * sub + 16 * ks2, db, lane);
        return f;
      };
      TrFrags tbuf[PF + 1];
#pragma unroll
      for (int i = 0; i < PF; ++i) tbuf[i] = trfrags(i);
      // P and dS for 16 query rows at a time (B operands), then
      // dV^T += dO^T P and dK^T += Q^T dS over those rows.
#pragma unroll
      for (int ks2 = 0; ks2 < 2; ++ks2) {
        bf16x8_t pf[C::kKB], dsf[C::kKB];
#pragma unroll
        for (int r2 = 0; r2 < 2; ++r2) {
          const int r4 = 2 * ks2 + r2;
          const int qr0 = 32 * sub + 8 * r4 + 4 * half;
          const f32x4_t l4 = *reinterpret_cast<const f32x4_t*>(lds_lse + qr0);
          const f32x4_t d4 = *reinterpret_cast<const f32x4_t*>(lds_D + qr0);
#pragma unroll
          for (int kb = 0; kb < C::kKB; ++kb)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int i = 4 * r4 + e;
              const float pv = __builtin_amdgcn_exp2f(fmaf(s[kb][i], p.scale_log2, -l4[e]));
              pf[kb][4 * r2 + e] = (__bf16)pv;
              dsf[kb][4 * r2 + e] = (__bf16)(pv * (dp[kb][i] - d4[e]));
            }
        }
#pragma unroll
        for (int db = 0; db < C::kDB; ++db) {
          const int idx = ks2 * C::kDB + db;
          if (idx + PF < kTrSteps) tbuf[(idx + PF) % (PF + 1)] = trfrags(idx + PF);
          const TrFrags& f = tbuf[idx % (PF + 1)];
#pragma unroll
          for (int kb = 0; kb < C::kKB; ++kb) {
            acc_dv[kb][db] = mfma32(f.dot, pf[kb], acc_dv[kb][db]);
            acc_dk[kb][db] = mfma32(f.qt, dsf[kb], acc_dk[kb][db]);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
  }

#pragma unroll
  for (int kb = 0; kb < C::kKB; ++kb) {
    const int64_t kj = kw + 32 * kb + r32;
    if (kj >= N) continue;
    __bf16* dkrow = p.dk + kj * kv_tok + kvoff;
    __bf16* dvrow = p.dv + kj * kv_tok + kvoff;
#pragma unroll
    for (int db = 0; db < C::kDB; ++db)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        bf16x4_t wk, wv;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          wk[e] = (__bf16)(acc_dk[kb][db][4 * r4 + e] * p.scale);
          wv[e] = (__bf16)acc_dv[kb][db][4 * r4 + e];
        }
        *reinterpret_cast<bf16x4_t*>(dkrow + db * 32 + 8 * r4 + 4 * half) = wk;
        *reinterpret_cast<bf16x4_t*>(dvrow + db * 32 + 8 * r4 + 4 * half) = wv;
      }
  }
}

template <int HD, int GPACK>
hipError_t launch_dq(BwdParams p, const AttnShape& s, hipStream_t stream) {
  using C = DqCfg<HD, GPACK>;
  p.num_blocks = (s.N + C::kBP - 1) / C::kBP;
  dim3 grid((uint32_t)p.num_blocks, (uint32_t)(s.bs * s.hkv * (p.g / GPACK)));
  return launch_kernel(attn_bwd_dq_kernel<HD, GPACK>, grid, dim3(C::kThreads), 0, stream, p);
}

}  // namespace

size_t attn_bwd_workspace_bytes(const AttnShape& s, bool /*bf16*/) {
  const size_t d = (size_t)s.N * s.bs * s.hq * sizeof(float);
  return (d + 255) / 256 * 256;
}

hipError_t launch_attn_bwd_bf16(const AttnShape& s, const void* q, const void* k, const void* v,
                                const void* o, const float* lse, const void* dout, void* dq,
                                void* dk, void* dv, void* workspace, hipStream_t stream) {
  if (s.N == 0) return hipSuccess;
  BwdParams p;
  p.q = static_cast<const __bf16*>(q);
  p.k = static_cast<const __bf16*>(k);
  p.v = static_cast<const __bf16*>(v);
  p.dout = static_cast<const __bf16*>(dout);
  p.lse = lse;
  p.D = static_cast<const float*>(workspace);
  p.dq = static_cast<__bf16*>(dq);
  p.dk = static_cast<__bf16*>(dk);
  p.dv = static_cast<__bf16*>(dv);
  p.N = s.N;
  p.bs = s.bs;
  p.hq = s.hq;
  p.hkv = s.hkv;
  p.g = s.hq / s.hkv;
  p.scale = s.scale;
  p.scale_log2 = s.scale * kLog2e;
  p.causal = s.causal;
  p.cu = s.cu;
  p.n_docs = s.n_docs;
  p.num_blocks = 0;

  float* D = static_cast<float*>(workspace);
  const __bf16* ob = static_cast<const __bf16*>(o);
  hipError_t e = s.hd == 128 ? launch_row_dot<__bf16, 128>(ob, p.dout, D, s, stream)
                             : launch_row_dot<__bf16, 64>(ob, p.dout, D, s, stream);
  if (e != hipSuccess) return e;

  auto dq_launch = [&](auto hd_tag) -> hipError_t {
    constexpr int HD = decltype(hd_tag)::value;
    if (p.g % 8 == 0) return launch_dq<HD, 8>(p, s, stream);
    if (p.g % 4 == 0) return launch_dq<HD, 4>(p, s, stream);
    if (p.g % 2 == 0) return launch_dq<HD, 2>(p, s, stream);
    return launch_dq<HD, 1>(p, s, stream);
  };
  auto dkv_launch = [&](auto hd_tag) -> hipError_t {
    constexpr int HD = decltype(hd_tag)::value;
    using C = DkvCfg<HD, 4, 1, 64>;
    dim3 grid((uint32_t)((s.N + C::kBK - 1) / C::kBK), (uint32_t)(s.bs * s.hkv));
    return launch_kernel(attn_bwd_dkv_kernel<HD, 4, 1, 64, 2>, grid, dim3(C::kThreads), 0, stream, p);
  };
  if (s.hd == 128) {
    if ((e = dq_launch(std::integral_constant<int, 128>{})) != hipSuccess) return e;
    return dkv_launch(std::integral_constant<int, 128>{});
  }
  if ((e = dq_launch(std::integral_constant<int, 64>{})) != hipSuccess) return e;
  return dkv_launch(std::integral_constant<int, 64>{});
}

}  // namespace ulysses
