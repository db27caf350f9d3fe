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
// dK, dV.  A workgroup of 8 waves owns 128 key rows of one key/value head as
// 4 blocks of 32.  Each block is worked by the two waves that share a SIMD
// (waves w and w + 4):
//   the P wave holds the block's K rows and, for every 64-query step,
//     computes S = Q K^T, P = exp(S - LSE) (handed over through LDS in fp32)
//     and dV^T += dO^T P;
//   the dS wave holds the V rows and, in the same phase, finishes the
//     previous step (dS = P (dP - D), dK^T += Q^T dS) before computing
//     dP = dO V^T of the current one.
// Running the dS wave one step behind its partner leaves independent matrix
// products in every phase for one wave while the other does exponentials or
// dS arithmetic; one barrier per step hands P over.  Each wave carries one
// accumulator set, so two waves fit per SIMD.
// Steps walk the visible queries from the last 64-row tile down, over every
// query head of the GQA group within a tile, so the GQA sum stays in
// registers; no atomics, deterministic.  Q and dO tiles arrive by direct
// global-to-LDS copies one step ahead; Q stays one step longer (the dS wave
// reads Q^T a phase late), so it rotates through three buffers, and dO, LSE
// and D through two.
template <int HD>
struct DkvCfg {
  static constexpr int kPairs = 4;
  static constexpr int kWaves = 2 * kPairs;
  static constexpr int kThreads = 64 * kWaves;
  static constexpr int kBK = 32 * kPairs;   // key rows per workgroup
  static constexpr int kBQ = 64;            // query rows per step
  static constexpr int kSubs = kBQ / 32;
  static_assert(kSubs == 2, "the interleaved schedules take two 32-row sub-tiles per step");
  static constexpr int kChunks = HD / 8;
  static constexpr int kRowBytes = HD * 2;
  static constexpr int kTileBytes = kBQ * kRowBytes;
  static constexpr int kQBufs = 3, kDoBufs = 2;
  static constexpr int kDoOff = kQBufs * kTileBytes;
  static constexpr int kLseOff = kDoOff + kDoBufs * kTileBytes;
  static constexpr int kDOff = kLseOff + kDoBufs * kBQ * 4;
  static constexpr int kPOff = kDOff + kDoBufs * kBQ * 4;
  static constexpr int kPSub = 16 * 64 * 4;          // a 32 x 32 fp32 P tile
  static constexpr int kPBytes = kSubs * kPSub;      // one step of one pair
  static constexpr int kSmem = kPOff + kPairs * 2 * kPBytes;
  static constexpr int kKS = HD / 16;
  static constexpr int kDB = HD / 32;
  // The dS waves issue the copies of the next step, one 1 KB copy per wave
  // per tensor and part, in kParts parts spread over their work.
  static constexpr int kParts = kTileBytes / (16 * 64 * kPairs);
  static_assert(kParts >= 1 && kParts <= 4 && kTileBytes % (16 * 64 * kPairs) == 0, "tile copies");
  static_assert(2 * kBQ <= 64 * kPairs, "LSE and D staging");
};

template <int HD, int PF>
__global__ __launch_bounds__(512) void attn_bwd_dkv_kernel(BwdParams p) {
  using C = DkvCfg<HD>;
  __shared__ __attribute__((aligned(16))) char smem[C::kSmem];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int pair = wave & (C::kPairs - 1);
  const bool p_wave = wave < C::kPairs;
  const int half = lane >> 5;
  const int r32 = lane & 31;

  const int64_t N = p.N;
  const int kh = blockIdx.y % p.hkv;
  const int b = blockIdx.y / p.hkv;
  const int64_t k0 = (int64_t)blockIdx.x * C::kBK;   // heaviest (smallest keys) first
  const int64_t kw = k0 + 32 * pair;                // first key row of this pair
  const int64_t kj = kw + r32;                      // this lane's key row

  const int64_t q_tok = (int64_t)p.bs * p.hq * HD;
  const int64_t kv_tok = (int64_t)p.bs * p.hkv * HD;
  const int64_t kvoff = ((int64_t)b * p.hkv + kh) * HD;

  // B operand rows of this lane: K (S = Q K^T) or V (dP = dO V^T).
  const __bf16* brows = p_wave ? p.k : p.v;
  bf16x8_t bfrag[C::kKS];
#pragma unroll
  for (int ks = 0; ks < C::kKS; ++ks)
    bfrag[ks] = kj < N ? *reinterpret_cast<const bf16x8_t*>(brows + kj * kv_tok + kvoff + 16 * ks + 8 * half)
                       : bf16x8_t{};
  // queries that see key kj: [causal ? kj : doc_start(kj), doc_end(kj))
  const int64_t my_lo = kj < N ? (p.causal ? kj : doc_start_of(p.cu, p.n_docs, kj)) : 0;
  const int64_t my_hi = kj < N ? doc_end_of(p.cu, p.n_docs, kj, N) : 0;

  // Workgroup- and pair-level bounds, held in scalar registers.
  const int64_t k_last = (k0 + C::kBK < N ? k0 + C::kBK : N) - 1;
  const int64_t q_lo = wave_uniform(p.causal ? k0 : doc_start_of(p.cu, p.n_docs, k0));
  const int64_t q_hi = wave_uniform(doc_end_of(p.cu, p.n_docs, k_last, N));
  const bool pair_active = kw < N;
  const int64_t w_last = pair_active ? (kw + 31 < N ? kw + 31 : N - 1) : 0;
  const int64_t w_lo = wave_uniform(pair_active ? (p.causal ? kw : doc_start_of(p.cu, p.n_docs, kw)) : 0);
  const int64_t w_hi = wave_uniform(pair_active ? doc_end_of(p.cu, p.n_docs, w_last, N) : 0);
  // Queries seen by every key of the pair: [full_lo, full_hi).
  const int64_t full_lo =
      wave_uniform(pair_active ? (p.causal ? w_last : doc_start_of(p.cu, p.n_docs, w_last)) : 0);
  const int64_t full_hi = wave_uniform(pair_active ? doc_end_of(p.cu, p.n_docs, kw, N) : 0);

  const int64_t qt_lo = q_lo / C::kBQ;
  const int64_t qt_hi = (q_hi + C::kBQ - 1) / C::kBQ;
  const int64_t n_steps = (qt_hi - qt_lo) * p.g;

  // Stages step (query tile t, head kh*g + hh): Q into Q buffer qb and dO
  // into dO buffer db by direct copies issued by the dS waves (rows past N
  // repeat row N-1; every pair that reads them is masked), in kParts parts
  // so that the copies interleave with matrix products instead of queueing
  // at once; LSE (log2 units) and D through registers of the dS waves,
  // published by publish_stats once the copies have landed.
  const int dtid = tid - 64 * C::kPairs;   // thread index among the dS waves
  // Tile row and source chunk of this lane's 16 bytes in each part, and
  // their element offset within the step's rows.
  int part_row[C::kParts];
  int64_t part_off[C::kParts];
#pragma unroll
  for (int j = 0; j < C::kParts; ++j) {
    const int piece = (j * C::kPairs + pair) * 64 + lane;
    part_row[j] = piece / C::kChunks;
    const int ch = (piece % C::kChunks) ^ swz_f<C::kChunks>(part_row[j]);
    part_off[j] = part_row[j] * q_tok + ch * 8;
  }
  float sst = 0.f;
  auto issue_part = [&](int j, int64_t t, int hh, int qb, int db) {
    const int h = kh * p.g + hh;
    const int64_t qoff = ((int64_t)b * p.hq + h) * HD;
    const int64_t i0 = t * C::kBQ;
    const int slot = (j * C::kPairs + pair) * 64;   // first 16-byte slot of this copy
    int64_t e = i0 * q_tok + qoff + part_off[j];
    if (i0 + C::kBQ > N && i0 + part_row[j] >= N)   // last tile: repeat row N-1
      e -= (i0 + part_row[j] - (N - 1)) * q_tok;
    load_lds16(p.q + e, smem + qb * C::kTileBytes + slot * 16);
    load_lds16(p.dout + e, smem + C::kDoOff + db * C::kTileBytes + slot * 16);
    if (j == 0 && dtid >= 0 && dtid < 2 * C::kBQ) {
      const int64_t qs = i0 + (dtid % C::kBQ);
      const int64_t idx = ((int64_t)b * p.hq + h) * N + qs;
      // LSE in log2 units; D negated (it seeds the dP accumulator)
      sst = qs < N ? (dtid < C::kBQ ? p.lse[idx] * kLog2e : -p.D[idx]) : 0.f;
    }
  };
  auto publish_stats = [&](int qb, int db) {
    if (dtid >= 0 && dtid < C::kBQ)
      reinterpret_cast<float*>(smem + C::kLseOff)[db * C::kBQ + dtid] = sst;
    else if (dtid >= C::kBQ && dtid < 2 * C::kBQ)
      reinterpret_cast<float*>(smem + C::kDOff)[db * C::kBQ + dtid - C::kBQ] = sst;
  };

  const TrReader<C::kChunks, C::kRowBytes, C::kDB> tr(lane);

  if (n_steps > 0 && !p_wave) {
#pragma unroll
    for (int j = 0; j < C::kParts; ++j) issue_part(j, qt_hi - 1, 0, 0, 0);
    wait_vmem();
    publish_stats(0, 0);
  }
  __syncthreads();

  // The step loop, instantiated once per role so that each role's
  // accumulators stay in place; both instances pass the same barriers.
  auto run = [&](auto role) {
    constexpr bool kP = decltype(role)::value;
    f32x16_t acc[C::kDB];   // dV^T (P waves) or dK^T (dS waves)
#pragma unroll
    for (int db = 0; db < C::kDB; ++db) acc[db] = f32x16_t{};
    f32x16_t dp_prev[C::kSubs];   // dS waves: dP - D of the previous step
#pragma unroll
    for (int sub = 0; sub < C::kSubs; ++sub) dp_prev[sub] = f32x16_t{};

    int64_t t = qt_hi - 1;
    int hh = 0, qb = 0, db = 0;
    bool prev_vis = false;
    int prev_qb = 0;
    for (int64_t n = 0; n <= n_steps; ++n) {
      const bool cur = n < n_steps;
      const bool has_next = n + 1 < n_steps;
      const int nqb = qb == C::kQBufs - 1 ? 0 : qb + 1;
      const int ndb = db ^ 1;
      const int64_t nt = hh + 1 < p.g ? t : t - 1;
      const int nhh = hh + 1 < p.g ? hh + 1 : 0;
      // dS waves: part i of the next step's copies goes out at point i.
      auto issue_at = [&](int i) {
        if (!kP && has_next && i < C::kParts) issue_part(i, nt, nhh, nqb, ndb);
      };
      const int64_t i0 = t * C::kBQ;
      const bool vis = cur && pair_active && i0 < w_hi && i0 + C::kBQ > w_lo;
      const char* tq = smem + qb * C::kTileBytes;
      const char* tdo = smem + C::kDoOff + db * C::kTileBytes;
      char* pbuf = smem + C::kPOff + (2 * pair + (int)(n & 1)) * C::kPBytes;

      if constexpr (kP) {
        if (vis) {
          const float* tlse = reinterpret_cast<const float*>(smem + C::kLseOff) + db * C::kBQ;
          // S = Q K^T for both 32-row sub-tiles: lane holds key kj and 16
          // query rows of each.
          f32x16_t s[C::kSubs];
#pragma unroll
          for (int sub = 0; sub < C::kSubs; ++sub) s[sub] = f32x16_t{};
          {
            // A fragments read PF products ahead, over both sub-tiles.
            constexpr int kN = C::kSubs * C::kKS;
            auto afrag = [&](int i) {
              return *reinterpret_cast<const bf16x8_t*>(
                  tq + swz<C::kChunks, C::kRowBytes>(32 * (i / C::kKS) + r32, 2 * (i % C::kKS) + half));
            };
            bf16x8_t buf[PF + 1];
#pragma unroll
            for (int i = 0; i < PF; ++i) buf[i] = afrag(i);
#pragma unroll
            for (int i = 0; i < kN; ++i) {
              if (i + PF < kN) buf[(i + PF) % (PF + 1)] = afrag(i + PF);
              s[i / C::kKS] = mfma32(buf[i % (PF + 1)], bfrag[i % C::kKS], s[i / C::kKS]);
              __builtin_amdgcn_sched_barrier(0);
            }
          }
          bf16x8_t pf[C::kSubs][2];
#pragma unroll
          for (int sub = 0; sub < C::kSubs; ++sub) {
            const int64_t s0 = i0 + 32 * sub;
            // On sub-tiles that cross a boundary (or that this pair does
            // not see at all), scores of invisible (query, key) pairs become
            // -inf, so their P is exactly 0.
            if (s0 < full_lo || s0 + 32 > full_hi) {
              const int lo = (int)(my_lo - s0 < -1 ? -1 : (my_lo - s0 > 33 ? 33 : my_lo - s0));
              const int hi = (int)(my_hi - s0 < -1 ? -1 : (my_hi - s0 > 33 ? 33 : my_hi - s0));
#pragma unroll
              for (int i = 0; i < 16; ++i) {
                const int qr = 8 * (i >> 2) + 4 * half + (i & 3);
                if (qr < lo || qr >= hi) s[sub][i] = -INFINITY;
              }
            }
            float* pt = reinterpret_cast<float*>(pbuf + sub * C::kPSub);
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
              const f32x4_t l4 = *reinterpret_cast<const f32x4_t*>(tlse + 32 * sub + 8 * r4 + 4 * half);
              f32x4_t p4;
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                p4[e] = __builtin_amdgcn_exp2f(fmaf(s[sub][4 * r4 + e], p.scale_log2, -l4[e]));
                pf[sub][r4 >> 1][4 * (r4 & 1) + e] = (__bf16)p4[e];
              }
              *reinterpret_cast<f32x4_t*>(pt + 4 * (64 * r4 + lane)) = p4;
            }
            // dV^T += dO^T P over the sub-tile's two 16-row steps, the
            // transposed A fragments read PF products ahead.
            {
              constexpr int kN = 2 * C::kDB;
              auto tfrag = [&](int i) { return tr.load(tdo, 32 * sub + 16 * (i / C::kDB), i % C::kDB); };
              bf16x8_t buf[PF + 1];
#pragma unroll
              for (int i = 0; i < PF; ++i) buf[i] = tfrag(i);
#pragma unroll
              for (int i = 0; i < kN; ++i) {
                if (i + PF < kN) buf[(i + PF) % (PF + 1)] = tfrag(i + PF);
                acc[i % C::kDB] = mfma32(buf[i % (PF + 1)], pf[sub][i / C::kDB], acc[i % C::kDB]);
                __builtin_amdgcn_sched_barrier(0);
              }
            }
          }
        }
      } else {
        // Finish the previous step, one sub-tile at a time:
        // dS = P (dP - D), dK^T += Q^T dS; the next step's copies go out
        // between the stages.
        issue_at(0);
        const char* pq = smem + prev_qb * C::kTileBytes;
        const char* ppbuf = smem + C::kPOff + (2 * pair + (int)((n - 1) & 1)) * C::kPBytes;
#pragma unroll
        for (int sub = 0; sub < C::kSubs; ++sub) {
          if (prev_vis) {
            const float* pt = reinterpret_cast<const float*>(ppbuf + sub * C::kPSub);
            bf16x8_t dsf[2];
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
              const f32x4_t p4 = *reinterpret_cast<const f32x4_t*>(pt + 4 * (64 * r4 + lane));
#pragma unroll
              for (int e = 0; e < 4; ++e)
                dsf[r4 >> 1][4 * (r4 & 1) + e] = (__bf16)(p4[e] * dp_prev[sub][4 * r4 + e]);
            }
            {
              constexpr int kN = 2 * C::kDB;
              auto tfrag = [&](int i) { return tr.load(pq, 32 * sub + 16 * (i / C::kDB), i % C::kDB); };
              bf16x8_t buf[PF + 1];
#pragma unroll
              for (int i = 0; i < PF; ++i) buf[i] = tfrag(i);
#pragma unroll
              for (int i = 0; i < kN; ++i) {
                if (i + PF < kN) buf[(i + PF) % (PF + 1)] = tfrag(i + PF);
                acc[i % C::kDB] = mfma32(buf[i % (PF + 1)], dsf[i / C::kDB], acc[i % C::kDB]);
                __builtin_amdgcn_sched_barrier(0);
              }
            }
          }
          issue_at(1 + sub);
        }
        issue_at(3);
        // dP - D = dO V^T - D for both sub-tiles (the accumulators start at
        // -D), finished in the next phase; A fragments read PF products
        // ahead.
        if (vis) {
          const float* tnd = reinterpret_cast<const float*>(smem + C::kDOff) + db * C::kBQ;
          constexpr int kN = C::kSubs * C::kKS;
          auto afrag = [&](int i) {
            return *reinterpret_cast<const bf16x8_t*>(
                tdo + swz<C::kChunks, C::kRowBytes>(32 * (i / C::kKS) + r32, 2 * (i % C::kKS) + half));
          };
#pragma unroll
          for (int sub = 0; sub < C::kSubs; ++sub)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
              const f32x4_t d4 = *reinterpret_cast<const f32x4_t*>(tnd + 32 * sub + 8 * r4 + 4 * half);
#pragma unroll
              for (int e = 0; e < 4; ++e) dp_prev[sub][4 * r4 + e] = d4[e];
            }
          bf16x8_t buf[PF + 1];
#pragma unroll
          for (int i = 0; i < PF; ++i) buf[i] = afrag(i);
#pragma unroll
          for (int i = 0; i < kN; ++i) {
            if (i + PF < kN) buf[(i + PF) % (PF + 1)] = afrag(i + PF);
            dp_prev[i / C::kKS] = mfma32(buf[i % (PF + 1)], bfrag[i % C::kKS], dp_prev[i / C::kKS]);
            __builtin_amdgcn_sched_barrier(0);
          }
        }
      }

      if (has_next && !kP) {
        wait_vmem();   // this wave's copies of the next step have landed
        publish_stats(nqb, ndb);
      }
      __syncthreads();

      prev_vis = vis;
      prev_qb = qb;
      qb = nqb;
      db = ndb;
      if (++hh == p.g) {
        hh = 0;
        --t;
      }
    }

    if (kj < N) {
      __bf16* row = (kP ? p.dv : p.dk) + kj * kv_tok + kvoff;
      const float mul = kP ? 1.f : p.scale;
#pragma unroll
      for (int d = 0; d < C::kDB; ++d)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          bf16x4_t w;
#pragma unroll
          for (int e = 0; e < 4; ++e) w[e] = (__bf16)(acc[d][4 * r4 + e] * mul);
          *reinterpret_cast<bf16x4_t*>(row + d * 32 + 8 * r4 + 4 * half) = w;
        }
    }
  };
  if (p_wave)
    run(std::true_type{});
  else
    run(std::false_type{});
}

// LDS fragments read this many products ahead in the dK/dV kernel.
constexpr int kDkvPrefetch = 3;

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
    using C = DkvCfg<HD>;
    dim3 grid((uint32_t)((s.N + C::kBK - 1) / C::kBK), (uint32_t)(s.bs * s.hkv));
    return launch_kernel(attn_bwd_dkv_kernel<HD, kDkvPrefetch>, grid, dim3(C::kThreads), 0, stream, p);
  };
  if (s.hd == 128) {
    if ((e = dq_launch(std::integral_constant<int, 128>{})) != hipSuccess) return e;
    return dkv_launch(std::integral_constant<int, 128>{});
  }
  if ((e = dq_launch(std::integral_constant<int, 64>{})) != hipSuccess) return e;
  return dkv_launch(std::integral_constant<int, 64>{});
}

}  // namespace ulysses
