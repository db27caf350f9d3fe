// Causal (GQA, optionally document-masked) softmax attention, forward, on
// gfx950 bf16 matrix cores.
//
// What is computed (Hugging Face Ulysses blog: each GPU runs standard
// attention over the full sequence for its heads; integration guide: the
// causal mask comes from positions, and packed documents must not attend
// across their boundaries):
//   s_ij = scale <q_i, k_j>,   O_i = sum_j exp(s_ij - LSE_i) v_j,
//   LSE_i = ln sum_j exp(s_ij)   over the keys j visible to query i.
//
// Design for CDNA4:
//  * A workgroup of 8 waves owns a block of query positions for GPACK query
//    heads that share one key/value head (GQA), so every K/V tile staged in
//    LDS serves 256 query rows.  Each wave owns 32 rows of one head.
//  * The scores are formed transposed, S^T = K Q^T, with
//    v_mfma_f32_32x32x16_bf16: K comes from LDS (one 16-byte read per lane
//    per MFMA), Q stays in registers.  In the accumulator every lane then
//    holds 32 scores of a single query row, so the row max and row sum need
//    one cross-lane exchange (lane l with l^32) per tile.
//  * The same accumulator, rounded to bf16, is directly the B operand of
//    O^T += V^T P^T; V^T comes from LDS through the gfx950 transposing read
//    (ds_read_b64_tr_b16), so V is stored in LDS in its natural row layout.
//  * Online softmax in the exp2 domain with scale*log2(e) folded into one
//    FMA per score.  The running max is only raised when a row's max grows by
//    more than 8 (a factor 256), so O and the row sum are rarely rescaled;
//    any reference max gives the same result in exact arithmetic.
//  * Key tiles entirely above the diagonal (or outside the documents of a
//    block) are never visited; per wave, tiles entirely masked for its rows
//    are skipped; only tiles crossing a boundary apply the element mask.
//  * LDS rows are swizzled in 16-byte chunks (swz in device_common.h) so both
//    the row reads of K and the transposing reads of V avoid bank conflicts;
//    every fragment is read two products ahead of the MFMA that uses it, and
//    consecutive MFMAs go to different accumulators, so LDS latency and MFMA
//    dependency latency overlap the matrix work.
//  * Blocks are launched heaviest (largest positions) first.
#include <math.h>

#include "device_common.h"
#include "launch.h"

namespace ulysses {
namespace {

struct FwdParams {
  const __bf16* q;
  const __bf16* k;
  const __bf16* v;
  __bf16* o;
  float* lse;
  int64_t N;
  int bs, hq, hkv, g;
  float scale_log2;   // softmax scale * log2(e)
  int causal;
  const int32_t* cu;
  int n_docs;
  int64_t num_pos_blocks;
};

template <int HD, int GPACK>
struct FwdCfg {
  static constexpr int kWaves = 8;
  static constexpr int kThreads = 64 * kWaves;
  static constexpr int kBP = 32 * kWaves / GPACK;   // query positions per block
  static constexpr int kBC = 64;                     // keys per tile
  static constexpr int kChunks = HD / 8;             // 16-byte chunks per row
  static constexpr int kRowBytes = HD * 2;
  static constexpr int kTileBytes = kBC * kRowBytes;
  static constexpr int kKS = HD / 16;                // k-steps of S^T = K Q^T
  static constexpr int kDB = HD / 32;                // 32-wide blocks of head dim
  static constexpr int kLoads = kBC * kChunks / kThreads;  // 16-byte loads per tensor per tile
  static_assert(kLoads >= 1 && kBC * kChunks % kThreads == 0, "tile loads");
};

template <int HD, int GPACK>
__global__ __launch_bounds__(512) void attn_fwd_bf16_kernel(FwdParams p) {
  using C = FwdCfg<HD, GPACK>;
  __shared__ __attribute__((aligned(16))) char smem[2 * C::kTileBytes];
  char* lds_k = smem;
  char* lds_v = smem + C::kTileBytes;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int half = lane >> 5;      // which k-half / row-quad of the MFMA layout
  const int r32 = lane & 31;

  const int64_t N = p.N;
  const int64_t pb = p.num_pos_blocks - 1 - (int64_t)blockIdx.x;   // heaviest first
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
  const __bf16* qbase = p.q + ((int64_t)b * p.hq + h) * HD;
  const __bf16* kbase = p.k + ((int64_t)b * p.hkv + kh) * HD;
  const __bf16* vbase = p.v + ((int64_t)b * p.hkv + kh) * HD;

  // Q fragments (B operand of S^T): lane holds Q[qi][16 ks + 8 half + 0..7].
  bf16x8_t qf[C::kKS];
#pragma unroll
  for (int ks = 0; ks < C::kKS; ++ks) {
    if (qi < N)
      qf[ks] = *reinterpret_cast<const bf16x8_t*>(qbase + qi * q_tok + 16 * ks + 8 * half);
    else
      qf[ks] = bf16x8_t{};
  }

  // Key range of the whole block, of this wave, and of this lane's row.
  const int64_t blk_last = (p0 + C::kBP < N ? p0 + C::kBP : N) - 1;
  const int64_t kv_lo = doc_start_of(p.cu, p.n_docs, p0);
  const int64_t kv_hi = p.causal ? blk_last + 1 : doc_end_of(p.cu, p.n_docs, blk_last, N);
  const bool wave_active = pw < N;
  const int64_t w_last = wave_active ? (pw + 31 < N ? pw + 31 : N - 1) : 0;
  const int64_t w_lo = wave_active ? doc_start_of(p.cu, p.n_docs, pw) : 0;
  const int64_t w_hi = wave_active ? (p.causal ? w_last + 1 : doc_end_of(p.cu, p.n_docs, w_last, N)) : 0;
  // Keys visible to every row of the wave: [full_lo, full_hi).
  const int64_t full_lo = wave_active ? doc_start_of(p.cu, p.n_docs, w_last) : 0;
  const int64_t full_hi = wave_active ? (p.causal ? pw + 1 : doc_end_of(p.cu, p.n_docs, pw, N)) : 0;
  const int64_t my_lo = qi < N ? doc_start_of(p.cu, p.n_docs, qi) : 0;
  const int64_t my_hi = qi < N ? (p.causal ? qi + 1 : doc_end_of(p.cu, p.n_docs, qi, N)) : 0;

  const int64_t t_begin = kv_lo / C::kBC;
  const int64_t t_end = (kv_hi + C::kBC - 1) / C::kBC;

  f32x16_t acc_o[C::kDB];
#pragma unroll
  for (int db = 0; db < C::kDB; ++db) acc_o[db] = f32x16_t{};
  float m_run = -INFINITY;   // reference max, log2 domain
  float l_run = 0.f;         // this lane's share of the row sum

  u32x4_t kst[C::kLoads], vst[C::kLoads];
  auto load_tile = [&](int64_t t) {
#pragma unroll
    for (int i = 0; i < C::kLoads; ++i) {
      const int cid = tid + i * C::kThreads;
      const int row = cid / C::kChunks;
      const int ch = cid % C::kChunks;
      const int64_t j = t * C::kBC + row;
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

    // S^T[kv][q] = K Q^T for the two 32-key halves of the tile: the two
    // accumulator chains alternate, and each K fragment is read from LDS two
    // products ahead of its use.
    f32x16_t s[2];
    s[0] = f32x16_t{};
    s[1] = f32x16_t{};
    {
      constexpr int kSteps = 2 * C::kKS;   // (ks, kb) pairs, kb fastest
      auto kfrag = [&](int idx) {
        const int ks = idx >> 1, kb = idx & 1;
        return *reinterpret_cast<const bf16x8_t*>(
            lds_k + swz<C::kChunks, C::kRowBytes>(kb * 32 + r32, 2 * ks + half));
      };
      bf16x8_t buf[3];
      buf[0] = kfrag(0);
      buf[1] = kfrag(1);
#pragma unroll
      for (int idx = 0; idx < kSteps; ++idx) {
        if (idx + 2 < kSteps) buf[(idx + 2) % 3] = kfrag(idx + 2);
        s[idx & 1] = mfma32(buf[idx % 3], qf[idx >> 1], s[idx & 1]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }

    // Element mask on tiles that cross a boundary of some row of the wave.
    const bool need_mask = j0 < full_lo || j0 + C::kBC > full_hi;
    if (need_mask) {
      // visible keys of this row as offsets into the tile, clamped to [-1, 65]
      const int lo = (int)(my_lo - j0 < -1 ? -1 : (my_lo - j0 > 65 ? 65 : my_lo - j0));
      const int hi = (int)(my_hi - j0 < -1 ? -1 : (my_hi - j0 > 65 ? 65 : my_hi - j0));
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int j = kb * 32 + 8 * (i >> 2) + 4 * half + (i & 3);
          if (j < lo || j >= hi) s[kb][i] = -INFINITY;
        }
    }

    // Row max over the tile (this lane's 32 keys, then the partner lane's).
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[kb][i]);
    mx = fmaxf(mx, wave_shfl_xor32(mx));
    const float mx2 = mx * p.scale_log2;
    const bool raise = mx2 > m_run + 8.0f;
    if (wave_any(raise)) {
      const float alpha = raise ? __builtin_amdgcn_exp2f(m_run - mx2) : 1.0f;
      if (raise) m_run = mx2;
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < C::kDB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc_o[db][i] *= alpha;
    }
    const float mb = m_run == -INFINITY ? 0.f : m_run;

    // P = exp2(s * scale*log2e - m), rounded to bf16 as the B operand of PV.
    bf16x8_t pf[4];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float e = __builtin_amdgcn_exp2f(fmaf(s[kb][i], p.scale_log2, -mb));
        l_run += e;
        pf[2 * kb + (i >> 3)][i & 7] = (__bf16)e;
      }

    // O^T[d][q] += V^T P^T; V^T fragments via the transposing LDS read, two
    // products ahead of their use, four independent accumulator chains.
    const int grp = lane >> 4;
    const int u = lane & 15;
    {
      constexpr int kSteps = 4 * C::kDB;   // (ks, db) pairs, db fastest
      auto vfrag = [&](int idx) {
        const int ks = idx / C::kDB, db = idx % C::kDB;
        bf16x4_t part[2];
#pragma unroll
        for (int jh = 0; jh < 2; ++jh) {
          const int row = 16 * ks + 8 * jh + 4 * (grp >> 1) + (u >> 2);
          const int col = db * 32 + 16 * (grp & 1) + 4 * (u & 3);
          const int off = swz<C::kChunks, C::kRowBytes>(row, col >> 3) + ((col >> 2) & 1) * 8;
          part[jh] = lds_read_tr16(lds_v + off);
        }
        return __builtin_shufflevector(part[0], part[1], 0, 1, 2, 3, 4, 5, 6, 7);
      };
      bf16x8_t buf[3];
      buf[0] = vfrag(0);
      buf[1] = vfrag(1);
#pragma unroll
      for (int idx = 0; idx < kSteps; ++idx) {
        if (idx + 2 < kSteps) buf[(idx + 2) % 3] = vfrag(idx + 2);
        acc_o[idx % C::kDB] = mfma32(buf[idx % 3], pf[idx / C::kDB], acc_o[idx % C::kDB]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }

  if (qi >= N) return;
  const float l = l_run + wave_shfl_xor32(l_run);
  const float inv = 1.0f / l;
  __bf16* orow = p.o + (qi * p.bs + b) * (int64_t)p.hq * HD + (int64_t)h * HD;
#pragma unroll
  for (int db = 0; db < C::kDB; ++db)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      bf16x4_t w;
#pragma unroll
      for (int e = 0; e < 4; ++e) w[e] = (__bf16)(acc_o[db][4 * r4 + e] * inv);
      *reinterpret_cast<bf16x4_t*>(orow + db * 32 + 8 * r4 + 4 * half) = w;
    }
  if (half == 0) p.lse[((int64_t)b * p.hq + h) * N + qi] = (m_run + __log2f(l)) * kLn2;
}

template <int HD, int GPACK>
hipError_t launch_fwd(const FwdParams& prm, const AttnShape& s, hipStream_t stream) {
  using C = FwdCfg<HD, GPACK>;
  FwdParams p = prm;
  p.num_pos_blocks = (s.N + C::kBP - 1) / C::kBP;
  dim3 grid((uint32_t)p.num_pos_blocks, (uint32_t)(s.bs * s.hkv * (p.g / GPACK)));
  return launch_kernel(attn_fwd_bf16_kernel<HD, GPACK>, grid, dim3(C::kThreads), 0, stream, p);
}

template <int HD>
hipError_t launch_fwd_hd(const FwdParams& p, const AttnShape& s, hipStream_t stream) {
  if (p.g % 8 == 0) return launch_fwd<HD, 8>(p, s, stream);
  if (p.g % 4 == 0) return launch_fwd<HD, 4>(p, s, stream);
  if (p.g % 2 == 0) return launch_fwd<HD, 2>(p, s, stream);
  return launch_fwd<HD, 1>(p, s, stream);
}

}  // namespace

hipError_t launch_attn_fwd_bf16(const AttnShape& s, const void* q, const void* k, const void* v,
                                void* o, float* lse, hipStream_t stream) {
  if (s.N == 0) return hipSuccess;
  FwdParams p;
  p.q = static_cast<const __bf16*>(q);
  p.k = static_cast<const __bf16*>(k);
  p.v = static_cast<const __bf16*>(v);
  p.o = static_cast<__bf16*>(o);
  p.lse = lse;
  p.N = s.N;
  p.bs = s.bs;
  p.hq = s.hq;
  p.hkv = s.hkv;
  p.g = s.hq / s.hkv;
  p.scale_log2 = s.scale * kLog2e;
  p.causal = s.causal;
  p.cu = s.cu;
  p.n_docs = s.n_docs;
  p.num_pos_blocks = 0;
  if (s.hd == 128) return launch_fwd_hd<128>(p, s, stream);
  return launch_fwd_hd<64>(p, s, stream);
}

}  // namespace ulysses
