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
//   1. bwd_stats_kernel: -D and -LSE / scale for every query row, into the
//      workspace;
//   2. dQ: a workgroup owns query rows (as in the forward) and walks the
//      visible key tiles staged in LDS;
//   3. dK, dV: a workgroup owns 128 key rows of one key/value head and walks
//      the visible query tiles of every query head of its group, so the GQA
//      sum over heads happens in registers; no atomics anywhere, so results
//      are deterministic.
// Q, K, V and dO enter the products exactly as given (bf16); the softmax
// scale and log2(e) are applied to the fp32 scores, so they add no bf16
// rounding.  Every product is a v_mfma_f32_32x32x16_bf16.  Operands whose contraction
// runs along the sequence (dV = P^T dO, dK = dS^T Q, dQ = dS K) come from
// LDS through the transposing read ds_read_b64_tr_b16, so all tiles keep
// their natural row layout in LDS.
#include <math.h>

#include <type_traits>

#include "device_common.h"
#include "launch.h"

namespace ulysses {

namespace {

// Workspace: one fp32 array per query row of [bs, hq, N], 256-byte aligned:
// D for the fp32 path; -D then -LSE / scale for the bf16 path.
size_t stat_array_bytes(const AttnShape& s) {
  return ((size_t)s.N * s.bs * s.hq * sizeof(float) + 255) / 256 * 256;
}

// dK/dV split.  With fewer than four workgroups of 128-key blocks per CU,
// the long early key blocks of a causal share (the first sees every query,
// the last only its own tile) set the kernel's time.  Each key block's
// query tiles are then shared out, in contiguous runs, over `split`
// workgroups, which write fp32 partial dK/dV to the workspace; a reduction
// adds the parts in a fixed order (bitwise reproducible) and rounds once.
int dkv_split(const AttnShape& s) {
  const int64_t blocks = (s.N + 127) / 128 * s.bs * s.hkv;
  return blocks >= 1024 ? 1 : (blocks >= 512 ? 2 : 4);
}
size_t dkv_part_bytes(const AttnShape& s, int split) {
  if (split <= 1) return 0;
  return ((size_t)split * 2 * s.bs * s.hkv * s.N * s.hd * sizeof(float) + 255) / 256 * 256;
}

struct BwdParams {
  const __bf16* q;
  const __bf16* k;
  const __bf16* v;
  const __bf16* dout;
  const float* nlse_r;  // -LSE / scale (raw score units), [batch][head][position]
  const float* nD;      // -<dO, O>, same layout
  __bf16* dq;
  __bf16* dk;
  __bf16* dv;
  int64_t N;
  int bs, hq, hkv, g;
  // Heads per token row in memory of q/o/dout/dq and of k/v/dk/dv: hq and
  // hkv for head-sharded tensors, the global counts for strided views of
  // the sequence chunks (the pointers then point at the rank's first head).
  int q_row_heads, kv_row_heads;
  float scale;
  float scale_log2;
  int causal;
  const int32_t* cu;
  int n_docs;
  int64_t num_blocks;
  // dK/dV split (dkv_split): parts per key block, and with split > 1 the
  // fp32 partials [part][dK, dV][batch][kv head][position][head dim].
  int split;
  float* dkv_part;
  // Fused form only: the operands in their sequence chunks (the pointers
  // above, except the statistics, are unused).
  SeqChunks cq, ck, cv, cdo, cdq, cdk, cdv;
};

// ------------------------------------------------------------------------
// dQ
// ------------------------------------------------------------------------
// A workgroup of 8 waves owns a block of query positions for GPACK query
// heads of one key/value head, as in the forward: each wave owns 32 query
// rows of one head and keeps Q and dO in registers.  For every 64-key tile t
// it forms, transposed so that each lane holds one query row,
//   S^T = K Q^T,  P = exp2(S scale log2(e) - LSE log2(e)),  dP^T = V dO^T,
//   dS = P (dP - D),  dQ^T += K^T dS^T
// (K^T by transposing LDS reads).  As in the forward, matrix and vector work
// alternate between the two waves of a SIMD: in every phase one wave issues
// only matrix products (dQ of tile t-1, then S^T and dP^T of tile t: 48
// products) while its partner forms dS of a tile; the second group of waves
// runs one phase behind the first.  K and V tiles arrive by direct
// global-to-LDS copies three tiles ahead.  A K tile is read for two tiles
// (S^T now, K^T for dQ next), so K rotates through five buffers (a
// run-time rotation) and V through four (unrolled, compile-time).
template <int HD, int GPACK>
struct DqCfg {
  static constexpr int kWaves = 8;
  static constexpr int kThreads = 64 * kWaves;
  static constexpr int kBP = 32 * kWaves / GPACK;   // query positions per block
  static constexpr int kBC = 64;                     // keys per tile
  static constexpr int kChunks = HD / 8;
  static constexpr int kRowBytes = HD * 2;
  static constexpr int kTileBytes = kBC * kRowBytes;
  static constexpr int kKS = HD / 16;
  static constexpr int kDB = HD / 32;
  static constexpr int kKBufs = 5, kVBufs = 4;
  static constexpr int kVOff = kKBufs * kTileBytes;
  static constexpr int kSmem = kVOff + kVBufs * kTileBytes;
  // One wave-wide direct copy moves 1 KiB.
  static constexpr int kRowsPerCopy = 1024 / kRowBytes;
  static constexpr int kCopiesPerWave = kTileBytes / 1024 / kWaves;   // per tensor and tile
  static constexpr int kPrefetch = 4;   // LDS fragments read ahead of their product
  static_assert(kCopiesPerWave >= 1 && kTileBytes % (1024 * kWaves) == 0, "tile copies");
  static_assert(kSmem <= 160 * 1024, "LDS");
};

template <int HD, int GPACK, bool kFused>
__global__ __launch_bounds__(512) void attn_bwd_dq_kernel(BwdParams p) {
  using C = DqCfg<HD, GPACK>;
  using std::false_type;
  using std::integral_constant;
  using std::true_type;
  __shared__ __attribute__((aligned(1024))) char smem[C::kSmem];
  char* const lds_k0 = smem;              // K buffers
  char* const lds_v0 = smem + C::kVOff;   // V buffers

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5;
  const int r32 = lane & 31;
  const int group = wave >> 2;   // waves w and w+4 share a SIMD

  const int64_t N = wave_uniform(p.N);
  // Dispatch order as in the forward: slices fastest, blocks heaviest first
  // (by position, or by work within documents).
  const uint64_t lin = (uint64_t)blockIdx.y * gridDim.x + blockIdx.x;
  const int64_t t = lin / gridDim.y;
  int64_t pb = p.num_blocks - 1 - t;
  if (p.cu != nullptr && p.causal) {
    const int64_t s = doc_sorted_block<false>(t, p.num_blocks, C::kBP, p.cu, p.n_docs, N);
    if (s >= 0) pb = s;
  }
  pb = wave_uniform(pb);
  const int ngroups = p.g / GPACK;
  int y = (int)(lin % gridDim.y);
  const int hg = y % ngroups;
  y /= ngroups;
  const int kh = y % p.hkv;
  const int b = y / p.hkv;
  const int h = kh * p.g + hg * GPACK + (wave % GPACK);

  const int64_t p0 = pb * C::kBP;
  const int64_t pw = p0 + (int64_t)(wave / GPACK) * 32;
  const int64_t qi = pw + r32;

  const int64_t q_tok = (int64_t)p.bs * p.q_row_heads * HD;
  const int64_t kv_tok = (int64_t)p.bs * p.kv_row_heads * HD;
  const int64_t qoff = ((int64_t)b * p.q_row_heads + h) * HD;
  // (Kept in scalar registers: the copies take their base from there.)
  const __bf16* kbase = reinterpret_cast<const __bf16*>(wave_uniform(
      kFused ? (int64_t)p.ck.chunk[0] : reinterpret_cast<int64_t>(p.k + ((int64_t)b * p.kv_row_heads + kh) * HD)));
  const __bf16* vbase = reinterpret_cast<const __bf16*>(wave_uniform(
      kFused ? (int64_t)p.cv.chunk[0] : reinterpret_cast<int64_t>(p.v + ((int64_t)b * p.kv_row_heads + kh) * HD)));

  // B operands of this lane's query row: Q and dO as stored.
  bf16x8_t qf[C::kKS], df[C::kKS];
#pragma unroll
  for (int ks = 0; ks < C::kKS; ++ks) {
    qf[ks] = bf16x8_t{};
    df[ks] = bf16x8_t{};
    if (qi < N) {
      const __bf16* qrow = kFused ? chunk_row(p.cq, (uint32_t)qi, p.bs, b, h, HD) : p.q + qi * q_tok + qoff;
      const __bf16* drow = kFused ? chunk_row(p.cdo, (uint32_t)qi, p.bs, b, h, HD) : p.dout + qi * q_tok + qoff;
      qf[ks] = *reinterpret_cast<const bf16x8_t*>(qrow + 16 * ks + 8 * half);
      df[ks] = *reinterpret_cast<const bf16x8_t*>(drow + 16 * ks + 8 * half);
    }
  }
  const float c2 = p.scale_log2;   // softmax scale * log2(e)
  const int64_t stat = ((int64_t)b * p.hq + h) * N + qi;
  const float nl = qi < N ? p.nlse_r[stat] * c2 : 0.f;   // -LSE log2(e)
  const float nd = qi < N ? p.nD[stat] : 0.f;           // -D

  // Key range of the block; every wave walks all its tiles (one schedule for
  // all waves), tiles a wave does not see being masked out entirely.
  const int64_t blk_last = (p0 + C::kBP < N ? p0 + C::kBP : N) - 1;
  const int64_t kv_lo = doc_start_of(p.cu, p.n_docs, p0);
  const int64_t kv_hi = p.causal ? blk_last + 1 : doc_end_of(p.cu, p.n_docs, blk_last, N);
  const bool wave_active = pw < N;
  const int64_t w_last = wave_active ? (pw + 31 < N ? pw + 31 : N - 1) : 0;
  // Keys visible to every row of the wave: [full_lo, full_hi).
  const int64_t full_lo = wave_uniform(wave_active ? doc_start_of(p.cu, p.n_docs, w_last) : 0);
  const int64_t full_hi = wave_uniform(
      wave_active ? (p.causal ? pw + 1 : doc_end_of(p.cu, p.n_docs, pw, N)) : 0);
  // Visible keys of this lane's row, relative to the block's first key.
  const int64_t key0 = wave_uniform((kv_lo / C::kBC) * C::kBC);
  const int my_lo = qi < N ? (int)(doc_start_of(p.cu, p.n_docs, qi) - key0) : 0;
  const int my_hi =
      qi < N ? (int)((p.causal ? qi + 1 : doc_end_of(p.cu, p.n_docs, qi, N)) - key0) : 0;
  const int64_t t_begin = wave_uniform(kv_lo / C::kBC);
  const int n_tiles = (int)wave_uniform((kv_hi + C::kBC - 1) / C::kBC - t_begin);
  const int keys_left = (int)wave_uniform(N - key0);   // keys from key0 to the end
  const int m_tail = keys_left / C::kBC;                // first tile running past N
  const int flo = (int)wave_uniform(full_lo - key0);
  const int fhi = (int)wave_uniform(full_hi - key0);

  // Direct copies: slice c of this wave lands at bytes [1024 cidx, 1024 cidx
  // + 1024) of a tile buffer, lane l at +16 l, so lane l fetches the source
  // chunk that the swizzle places there.  Rows past the sequence end repeat
  // row N-1 (masked for every query).
  const int64_t row_bytes = kFused ? (int64_t)p.bs * p.ck.row_heads * HD * 2 : kv_tok * 2;
  uint32_t slice_off[C::kCopiesPerWave];
#pragma unroll
  for (int c = 0; c < C::kCopiesPerWave; ++c) {
    const int cidx = wave * C::kCopiesPerWave + c;
    const int row0 = cidx * C::kRowsPerCopy + lane / C::kChunks;
    const int col_bytes = ((lane % C::kChunks) ^ swz_f<C::kChunks>(row0)) * 16;
    slice_off[c] = (uint32_t)(row0 * row_bytes) + (uint32_t)col_bytes;
  }
  auto copy_slice = [&](const __bf16* base, const SeqChunks& ch, char* buf, int m, int c)
      __attribute__((always_inline)) {
    const int64_t j0 = (t_begin + m) * C::kBC;
    const char* tile;
    if constexpr (kFused)
      tile = reinterpret_cast<const char*>(
          wave_uniform(chunk_tile_base(ch, (uint32_t)(t_begin + m), p.bs, b, kh, HD)));
    else
      tile = reinterpret_cast<const char*>(wave_uniform((int64_t)base + j0 * row_bytes));
    const int cidx = wave * C::kCopiesPerWave + c;
    uint32_t off = slice_off[c];
    if (m >= m_tail) {   // the tile runs past the sequence end
      const int last = keys_left - 1 - m * C::kBC;
      const int row0 = cidx * C::kRowsPerCopy + lane / C::kChunks;
      const int col_bytes = ((lane % C::kChunks) ^ swz_f<C::kChunks>(row0)) * 16;
      const int row = row0 < last ? row0 : last;
      off = (uint32_t)(row * row_bytes) + (uint32_t)col_bytes;
    }
    copy_lds16_async_sbase(tile, off, buf + cidx * 1024);
  };
  auto k_buf = [&](int slot) __attribute__((always_inline)) { return lds_k0 + slot * C::kTileBytes; };
  auto v_buf = [&](int slot) __attribute__((always_inline)) { return lds_v0 + slot * C::kTileBytes; };

  f32x16_t acc[C::kDB];   // dQ^T
#pragma unroll
  for (int db = 0; db < C::kDB; ++db) acc[db] = f32x16_t{};
  f32x16_t s[2], dp[2];   // S^T and dP^T of a tile (two 32-key halves)
  bf16x8_t dsf[4];        // bf16 dS^T of a tile, B operand of dQ^T

  // --- matrix phase: dQ^T += K^T dS^T of tile m-1 (DQ, K buffer lkp), then
  // S^T and dP^T of tile m (SP, K buffer lk, V buffer lv) ---------------------
  int koff[C::kKS];
#pragma unroll
  for (int ks = 0; ks < C::kKS; ++ks) koff[ks] = swz<C::kChunks, C::kRowBytes>(r32, 2 * ks + half);
  const TrReader<C::kChunks, C::kRowBytes, C::kDB> tr(lane);
  auto matrix_phase = [&](auto dq_tag, auto sp_tag, const char* lkp, const char* lk, const char* lv)
      __attribute__((always_inline)) {
    constexpr bool kDQ = decltype(dq_tag)::value;
    constexpr bool kSP = decltype(sp_tag)::value;
    constexpr int NQ = kDQ ? 4 * C::kDB : 0;       // (16-key step, db), db fastest
    constexpr int NS = kSP ? 4 * C::kKS : 0;       // (ks, kb, K or V), fastest last
    constexpr int NT = NQ + NS;
    constexpr int PF = C::kPrefetch < NT ? C::kPrefetch : NT;
    auto frag = [&](int idx) __attribute__((always_inline)) {
      if (idx < NQ) return tr.load(lkp, 16 * (idx / C::kDB), idx % C::kDB);
      const int j = idx - NQ, kb = (j >> 1) & 1, ks = j >> 2;
      return *reinterpret_cast<const bf16x8_t*>(((j & 1) ? lv : lk) + kb * 32 * C::kRowBytes + koff[ks]);
    };
    bf16x8_t buf[PF + 1];
#pragma unroll
    for (int i = 0; i < PF; ++i) buf[i] = frag(i);
#pragma unroll
    for (int idx = 0; idx < NT; ++idx) {
      if (idx + PF < NT) buf[(idx + PF) % (PF + 1)] = frag(idx + PF);
      if (idx < NQ) {
        acc[idx % C::kDB] = mfma32(buf[idx % (PF + 1)], dsf[idx / C::kDB], acc[idx % C::kDB]);
      } else {
        const int j = idx - NQ, kb = (j >> 1) & 1, ks = j >> 2;
        if (j & 1)
          dp[kb] = mfma32(buf[idx % (PF + 1)], df[ks], ks == 0 ? f32x16_t{} : dp[kb]);
        else
          s[kb] = mfma32(buf[idx % (PF + 1)], qf[ks], ks == 0 ? f32x16_t{} : s[kb]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // --- vector phase: dS of tile m; issue(k), k = 0..3, issues a quarter of
  // the wave's tile copies -----------------------------------------------------
  auto vector_phase = [&](int m, auto issue) __attribute__((always_inline)) {
    const int jr = m * C::kBC;   // first key of the tile, relative to key0
    issue(0);
    // Raw fp32 scores to the exp2 domain: S scale log2(e) - LSE log2(e).
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) s[kb][i] = fmaf(s[kb][i], c2, nl);
    // Element mask without compares (as in the forward): invisible scores
    // become exactly -2^100, whose probability is exactly 0.
    if (jr < flo || jr + C::kBC > fhi) {
      const float neg_lo = (float)(4 * half - min(max(my_lo - jr, -1), 65));
      const float hi_m1 = (float)(min(max(my_hi - jr, -1), 65) - 1 - 4 * half);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float j = (float)(kb * 32 + 8 * (i >> 2) + (i & 3));   // key offset minus 4*half
          const float d = __builtin_amdgcn_fmed3f(fminf(j + neg_lo, hi_m1 - j), -1.0f, 0.0f);
          s[kb][i] = fmaf(d, 0x1p100f, s[kb][i]);
        }
    }
    issue(1);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float pv = __builtin_amdgcn_exp2f(s[kb][i]);
        dsf[2 * kb + (i >> 3)][i & 7] = (__bf16)(pv * (dp[kb][i] + nd));
      }
      issue(2 + kb);
    }
  };

  // Global phases 2m and 2m+1 form pair m (m = 0 .. n_tiles).  Group 0 runs
  // the matrix work of pair m in phase 2m and dS of tile m in phase 2m+1;
  // group 1 runs one phase later.  In its vector phase of pair m every wave
  // copies its share of K and V of tile m+3 into K buffer (m+3)%5 and V
  // buffer (m+3)%4 (K of tile m-2, last read as K^T in pair m-1, and V of
  // tile m-1, last read in pair m-1); group 1 issues pair m+1's copies, one
  // pair ahead, so that by global phase both groups issue pair m's copies
  // before phase 2m+2.  At the end of phase 2m+1 every wave waits for its
  // copies of pair m-2, so the barrier publishes the tiles of pair m+1 while
  // two pairs of copies stay in flight.  Copies past the last tile are
  // clamped to it (the data lands in a buffer nobody reads again).
  constexpr int kPairCopies = 2 * C::kCopiesPerWave;
  // Part k of the copies of pair m: k = 0, 1 for K, k = 2, 3 for V (with one
  // slice per tensor, parts 1 and 3 are empty).  ks5 = (m+3) % 5.
  auto copy_part = [&](int m, auto r_tag, int ks5, int k) __attribute__((always_inline)) {
    constexpr int r = decltype(r_tag)::value;   // m % 4
    const int last = n_tiles - 1;
    const bool is_v = k >= 2;
    const int c = k & 1;
    if (c >= C::kCopiesPerWave) return;
    const int t = m + 3 < last ? m + 3 : last;
    char* buf = is_v ? v_buf((r + 3) & 3) : k_buf(ks5);
    copy_slice(is_v ? vbase : kbase, is_v ? p.cv : p.ck, buf, t, c);
    __builtin_amdgcn_sched_barrier(0);
  };
  auto copy_pair = [&](int m, auto r_tag, int ks5) __attribute__((always_inline)) {
#pragma unroll
    for (int k = 0; k < 4; ++k) copy_part(m, r_tag, ks5, k);
  };
  auto next5 = [](int x) __attribute__((always_inline)) { return x == 4 ? 0 : x + 1; };

  auto run = [&](auto g_tag) __attribute__((always_inline)) {
    constexpr int g = decltype(g_tag)::value;
    // K buffer of tile m (k_cur) and of its copy target, tile m+3 (k_cpy).
    int k_cur = 0, k_cpy = 3;
    // Pair m of the main run (1 <= m < n_tiles).
    auto mid_pair = [&](int m, auto r_tag) __attribute__((always_inline)) {
      constexpr int r = decltype(r_tag)::value;
      const int k_prev = k_cur == 0 ? 4 : k_cur - 1;
      matrix_phase(true_type{}, true_type{}, k_buf(k_prev), k_buf(k_cur), v_buf(r));
      if constexpr (g == 1) wait_vmem_n<2 * kPairCopies>();
      block_barrier();
      auto issue = [&](int k) __attribute__((always_inline)) {
        if constexpr (g == 0) copy_part(m, r_tag, k_cpy, k);
        else copy_part(m + 1, integral_constant<int, (r + 1) & 3>{}, next5(k_cpy), k);
      };
      vector_phase(m, issue);
      if constexpr (g == 0) wait_vmem_n<2 * kPairCopies>();
      block_barrier();
      k_cur = next5(k_cur);
      k_cpy = next5(k_cpy);
    };
    // Prologue: K and V of tiles 0..2.
    const int last = n_tiles - 1;
#pragma unroll
    for (int t = 0; t < 3; ++t)
#pragma unroll
      for (int c = 0; c < C::kCopiesPerWave; ++c) {
        copy_slice(kbase, p.ck, k_buf(t), t < last ? t : last, c);
        copy_slice(vbase, p.cv, v_buf(t), t < last ? t : last, c);
      }
    wait_vmem();
    block_barrier();
    if constexpr (g == 1) {   // phase 0: group 1 has no vector work yet, only copies
      copy_pair(0, integral_constant<int, 0>{}, 3);
      block_barrier();
    }

    // Pair 0: S^T and dP^T of tile 0 only.
    matrix_phase(false_type{}, true_type{}, k_buf(0), k_buf(0), v_buf(0));
    block_barrier();
    auto issue0 = [&](int k) __attribute__((always_inline)) {
      if constexpr (g == 0) copy_part(0, integral_constant<int, 0>{}, 3, k);
      else copy_part(1, integral_constant<int, 1>{}, 4, k);
    };
    vector_phase(0, issue0);
    block_barrier();
    k_cur = 1;
    k_cpy = 4;

    // Pairs 1 .. n_tiles-1, four per iteration so that the V rotation m % 4
    // is a compile-time constant.
    for (int m = 1; m < n_tiles; m += 4) {
      mid_pair(m, integral_constant<int, 1>{});
      if (m + 1 < n_tiles) mid_pair(m + 1, integral_constant<int, 2>{});
      if (m + 2 < n_tiles) mid_pair(m + 2, integral_constant<int, 3>{});
      if (m + 3 < n_tiles) mid_pair(m + 3, integral_constant<int, 0>{});
    }

    // Pair n_tiles: dQ of the last tile only.
    matrix_phase(true_type{}, false_type{}, k_buf(k_cur == 0 ? 4 : k_cur - 1), k_buf(0), v_buf(0));
    wait_vmem();
    block_barrier();
    block_barrier();
    if constexpr (g == 0) block_barrier();   // matches group 1's leading phase
  };
  if (group == 0) run(integral_constant<int, 0>{});
  else run(integral_constant<int, 1>{});

  if (qi >= N) return;
  __bf16* orow = kFused ? chunk_row(p.cdq, (uint32_t)qi, p.bs, b, h, HD) : p.dq + qi * q_tok + qoff;
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
// A workgroup of 8 waves owns 128 key rows of one key/value head as 4
// blocks of 32 keys; the two waves that share a SIMD (waves w and w + 4)
// work block w.  The block walks the 64-query steps its keys see, over every
// query head of the GQA group within a query tile, so the sum over the
// group's heads stays in registers (no atomics: results are deterministic).
// For step n:
//   the P wave holds K and forms S'_n = Q_n K^T - LSE / scale, whose
//     accumulator starts at the negated statistic, so that
//     P_n = exp2(S'_n scale log2(e)) needs one multiply per score (K stays
//     exact: the scale is applied to the fp32 scores; c = scale log2(e));
//     then dV^T += dO^T P;
//   the dS wave holds V and forms dP'_n = dO_n V^T - D (likewise seeded),
//     dS = P dP' and dK^T += Q^T dS.
// Each step is two phases separated by workgroup barriers.  In every phase
// one wave of each SIMD issues only matrix products while its partner does
// only vector work, which the SIMD executes alongside:
//   phase A(n): P wave  S'_n, dV^T += dO_{n-1}^T P_{n-1}        (matrix)
//               dS wave dS_{n-1} = P_{n-1} dP'_{n-1}, to bf16  (vector)
//   phase B(n): P wave  scale, mask, P_n = exp2(S'_n c)          (vector)
//               dS wave dK^T += Q_{n-1}^T dS_{n-1}, dP'_n       (matrix)
// P reaches the dS wave through LDS as the same bf16 values that form dV
// (one buffer per block; measured 4% faster than an fp32 hand-off).  Q and dO
// tiles and the per-row statistics arrive by direct global-to-LDS copies
// two steps ahead, issued in pieces through the vector phases (Q by the dS
// waves, dO by the P waves).  A Q tile is read until phase B of the next
// step, so Q rotates through four buffers (a compile-time rotation: the
// step loop is unrolled four times) and dO through three (a run-time
// rotation).  Every block computes every step, with an element mask where
// not all of its keys see the step's queries, so all waves share one
// schedule.  The statistics are produced by bwd_stats_kernel.
template <int HD>
struct DkvCfg {
  static constexpr int kPairs = 4;
  static constexpr int kWaves = 2 * kPairs;
  static constexpr int kThreads = 64 * kWaves;
  static constexpr int kBK = 32 * kPairs;   // key rows per workgroup
  static constexpr int kBQ = 64;            // query rows per step
  static constexpr int kChunks = HD / 8;
  static constexpr int kRowBytes = HD * 2;
  static constexpr int kTileBytes = kBQ * kRowBytes;
  static constexpr int kKS = HD / 16;
  static constexpr int kDB = HD / 32;
  static constexpr int kQBufs = 4, kDoBufs = 3;
  // LDS: the statistics of the steps in flight, then Q, dO and P.
  static constexpr int kStatBytes = kBQ * 4;
  static constexpr int kLseOff = 0;
  static constexpr int kDOff = kLseOff + kQBufs * kStatBytes;
  static constexpr int kQOff = 2048;
  static constexpr int kDoOff = kQOff + kQBufs * kTileBytes;
  static constexpr int kPOff = kDoOff + kDoBufs * kTileBytes;
  static constexpr int kPBytes = kBQ * 32 * 2;   // bf16 P of one block and step
  static constexpr int kSmem = kPOff + kPairs * kPBytes;
  // A wave-wide direct copy moves 1 KiB.  For each step a group of four
  // waves copies one tile (kCopies slices per wave) and one 256-byte
  // statistic (every wave of the group copies the same bytes).
  static constexpr int kRowsPerCopy = 1024 / kRowBytes;
  static constexpr int kCopies = kTileBytes / 1024 / kPairs;
  static constexpr int kPhaseCopies = kCopies + 1;
  static_assert(kDOff + kDoBufs * kStatBytes <= kQOff, "statistics region");
  static_assert(kCopies >= 1 && kTileBytes % (1024 * kPairs) == 0, "tile copies");
  static_assert(kSmem <= 160 * 1024, "LDS");
};

// Product order within a matrix phase: na products of the kind whose LDS
// operand is published before the phase (kind a: PV on the P wave, dK on the
// dS wave) and nb of the other kind (b).  ord 0: a then b; 1: b then a;
// 2: the first half of a, then b, then the rest of a.  Returns the product
// at position i, numbered a first.
__device__ constexpr int phase_order(int na, int nb, int ord, int i) {
  if (ord == 1) return i < nb ? na + i : i - nb;
  if (ord == 2) {
    const int h = na / 2;
    return i < h ? i : (i < h + nb ? na + (i - h) : i - nb);
  }
  return i;
}
// Position of the first kind-b product.
__device__ constexpr int phase_first_b(int na, int nb, int ord) {
  return ord == 1 ? 0 : (ord == 2 ? na / 2 : na);
}

// Matrix-phase schedule of the dK/dV kernel: fragments read ahead (PF),
// product order of the P and dS waves (phase_order), whether a wave reads
// the first fragments of its next matrix phase at the end of its vector
// phase (needs the order to start with kind a), and how many positions
// before the first kind-b product its accumulator seeds are read.
template <int PF_, int POrd_, int DOrd_, bool PPre_, bool DPre_, int SeedLead_>
struct DkvSched {
  static constexpr int PF = PF_, POrd = POrd_, DOrd = DOrd_, SeedLead = SeedLead_;
  static constexpr bool PPre = PPre_, DPre = DPre_;
  static_assert(!PPre || POrd != 1, "early reads need kind a first");
  static_assert(!DPre || DOrd != 1, "early reads need kind a first");
};
using DkvSchedDefault = DkvSched<3, 1, 0, false, false, 16>;

template <int HD, bool kFused, class SC = DkvSchedDefault>
__global__ __launch_bounds__(512) void attn_bwd_dkv_kernel(BwdParams p) {
  using C = DkvCfg<HD>;
  using std::false_type;
  using std::integral_constant;
  using std::true_type;
  __shared__ __attribute__((aligned(1024))) char smem[C::kSmem];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int pair = wave & (C::kPairs - 1);   // key block; also the wave's index in its group
  const bool p_wave = wave < C::kPairs;
  const int half = lane >> 5;
  const int r32 = lane & 31;

  const int64_t N = wave_uniform(p.N);
  // Dispatch rank u over (key block, part, slice), slices fastest: key blocks
  // heaviest first (smallest keys, or by work within documents), the parts
  // of a block next to each other.
  const uint64_t lin = (uint64_t)blockIdx.y * gridDim.x + blockIdx.x;
  const uint64_t u = lin / gridDim.y;
  const int ys = (int)(lin % gridDim.y);
  const int kh = ys % p.hkv;
  const int b = ys / p.hkv;
  const int split = p.split;
  const int part = (int)(u % (uint32_t)split);
  int64_t kb = (int64_t)(u / (uint32_t)split);
  if (p.cu != nullptr && p.causal) {
    const int64_t s = doc_sorted_block<true>(kb, gridDim.x / (uint32_t)split, C::kBK, p.cu, p.n_docs, N);
    if (s >= 0) kb = s;
  }
  const int64_t k0 = wave_uniform(kb) * C::kBK;
  const int64_t kw = k0 + 32 * pair;                // first key of the block
  const int64_t kj = kw + r32;                      // this lane's key

  const int64_t q_tok = (int64_t)p.bs * p.q_row_heads * HD;
  const int64_t kv_tok = (int64_t)p.bs * p.kv_row_heads * HD;
  const int64_t kvoff = ((int64_t)b * p.kv_row_heads + kh) * HD;

  // B operand rows of this lane, as stored: K (P wave) or V (dS wave).
  bf16x8_t bfrag[C::kKS];
  {
    const __bf16* rows = p_wave ? p.k : p.v;
    const __bf16* krow = nullptr;
    if (kj < N)
      krow = kFused ? chunk_row(p_wave ? p.ck : p.cv, (uint32_t)kj, p.bs, b, kh, HD)
                    : rows + kj * kv_tok + kvoff;
#pragma unroll
    for (int ks = 0; ks < C::kKS; ++ks) {
      bfrag[ks] = bf16x8_t{};
      if (kj < N) bfrag[ks] = *reinterpret_cast<const bf16x8_t*>(krow + 16 * ks + 8 * half);
    }
  }
  const float c2 = p.scale_log2;   // softmax scale * log2(e)

  // Queries seen by the workgroup's keys: [q_lo, q_hi).  Steps walk its
  // 64-row query tiles from the last one down (concurrent workgroups then
  // read the same tiles), every head of the group within a tile.
  const int64_t k_last = (k0 + C::kBK < N ? k0 + C::kBK : N) - 1;
  const int64_t q_lo = p.causal ? k0 : doc_start_of(p.cu, p.n_docs, k0);
  const int64_t q_hi = doc_end_of(p.cu, p.n_docs, k_last, N);
  const int qt_blo = (int)wave_uniform(q_lo / C::kBQ);
  const int qt_bhi = (int)wave_uniform((q_hi + C::kBQ - 1) / C::kBQ);
  // This part's contiguous run of the block's query tiles (all of them
  // without a split).
  const int64_t nt = qt_bhi - qt_blo;
  const int qt_lo = qt_blo + (int)(nt * part / split);
  const int qt_hi = qt_blo + (int)(nt * (part + 1) / split);
  const int n_steps = (qt_hi - qt_lo) * p.g;
  const int t_tail = (int)wave_uniform(N / C::kBQ);   // tiles from here on run past N
  // Query positions from here on are relative to the first query tile
  // (32-bit, so that tile-level tests are scalar compares).
  const int64_t q_base = (int64_t)qt_lo * C::kBQ;
  // Queries that see key kj: [my_lo, my_hi).
  const int my_lo = kj < N ? (int)((p.causal ? kj : doc_start_of(p.cu, p.n_docs, kj)) - q_base) : 0;
  const int my_hi = kj < N ? (int)(doc_end_of(p.cu, p.n_docs, kj, N) - q_base) : 0;
  // Queries seen by every key of the block: [flo, fhi).
  const bool blk_active = kw < N;
  const int64_t w_last = blk_active ? (kw + 31 < N ? kw + 31 : N - 1) : 0;
  const int flo = blk_active
      ? (int)wave_uniform((p.causal ? w_last : doc_start_of(p.cu, p.n_docs, w_last)) - q_base) : 0;
  const int fhi = blk_active ? (int)wave_uniform(doc_end_of(p.cu, p.n_docs, kw, N) - q_base) : 0;

  // --- direct copies -----------------------------------------------------
  // Slice c of this wave lands at bytes [1024 cidx, 1024 cidx + 1024) of a
  // tile buffer, lane l at +16 l, so lane l fetches the source chunk that
  // the swizzle places there.  Rows past N repeat row N-1 (the tail tile);
  // those queries are masked for every key, so only finiteness matters.
  const int64_t row_bytes = kFused ? (int64_t)p.bs * p.cq.row_heads * HD * 2 : q_tok * 2;
  uint32_t slice_off[C::kCopies];
#pragma unroll
  for (int c = 0; c < C::kCopies; ++c) {
    const int cidx = pair * C::kCopies + c;
    const int row0 = cidx * C::kRowsPerCopy + lane / C::kChunks;
    const int col = ((lane % C::kChunks) ^ swz_f<C::kChunks>(row0)) * 16;
    slice_off[c] = (uint32_t)(row0 * row_bytes) + (uint32_t)col;
  }
  // A step: its query tile t and head index hh within the group.
  struct Cursor {
    int t, hh, n;
  };
  // Next step, or the same one at the last step (copies past the end repeat
  // the last step's data into buffers nobody reads again).
  auto advance = [&](Cursor& c) __attribute__((always_inline)) {
    if (c.n + 1 < n_steps) {
      ++c.n;
      if (++c.hh == p.g) {
        c.hh = 0;
        --c.t;
      }
    }
  };
  // Part k of a group's copies for step c: tile slices k < kCopies of Q (or
  // dO) into tile buffer `tile`, then at k == kCopies its statistic
  // -LSE / scale (or -D) into `stat`.
  auto copy_part = [&](auto q_tag, const Cursor& c, int k, char* tile, char* stat)
      __attribute__((always_inline)) {
    constexpr bool kQ = decltype(q_tag)::value;
    const int h = kh * p.g + c.hh;
    const int64_t i0 = (int64_t)c.t * C::kBQ;
    if (k < C::kCopies) {
      const __bf16* src = kQ ? p.q : p.dout;
      const char* base;
      if constexpr (kFused)
        base = reinterpret_cast<const char*>(
            wave_uniform(chunk_tile_base(kQ ? p.cq : p.cdo, (uint32_t)c.t, p.bs, b, h, HD)));
      else
        base = reinterpret_cast<const char*>(
            wave_uniform(reinterpret_cast<int64_t>(src + i0 * q_tok + ((int64_t)b * p.q_row_heads + h) * HD)));
      const int cidx = pair * C::kCopies + k;
      uint32_t off = slice_off[k];
      if (c.t >= t_tail) {
        const int last = (int)(N - 1 - i0);
        const int row0 = cidx * C::kRowsPerCopy + lane / C::kChunks;
        const int col = ((lane % C::kChunks) ^ swz_f<C::kChunks>(row0)) * 16;
        off = (uint32_t)((row0 < last ? row0 : last) * row_bytes) + (uint32_t)col;
      }
      copy_lds16_async_sbase(base, off, tile + cidx * 1024);
    } else if (k == C::kCopies) {
      const float* src = kQ ? p.nlse_r : p.nD;
      const char* base = reinterpret_cast<const char*>(
          wave_uniform(reinterpret_cast<int64_t>(src + ((int64_t)b * p.hq + h) * N + i0)));
      int row = lane;
      if (c.t >= t_tail) {
        const int last = (int)(N - 1 - i0);
        row = lane < last ? lane : last;
      }
      copy_lds4_async_sbase(base, (uint32_t)row * 4u, stat);
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  auto q_tile = [&](int slot) __attribute__((always_inline)) { return smem + C::kQOff + slot * C::kTileBytes; };
  auto do_tile = [&](int slot) __attribute__((always_inline)) { return smem + C::kDoOff + slot * C::kTileBytes; };
  auto lse_stat = [&](int slot) __attribute__((always_inline)) { return smem + C::kLseOff + slot * C::kStatBytes; };
  auto d_stat = [&](int slot) __attribute__((always_inline)) { return smem + C::kDOff + slot * C::kStatBytes; };

  // --- LDS operands --------------------------------------------------------
  // Row reads (A rows = 32 queries from row0): the swizzle depends on the low
  // four row bits only, so the 32-row sub-tile adds a constant offset.
  int roff[C::kKS];
#pragma unroll
  for (int ks = 0; ks < C::kKS; ++ks) roff[ks] = swz<C::kChunks, C::kRowBytes>(r32, 2 * ks + half);
  const TrReader<C::kChunks, C::kRowBytes, C::kDB> tr(lane);
  auto row_frag = [&](const char* tile, int idx) __attribute__((always_inline)) {
    return *reinterpret_cast<const bf16x8_t*>(tile + (idx & 1) * 32 * C::kRowBytes + roff[idx >> 1]);
  };
  // Accumulator seed: the statistic of the 16 query rows this lane holds in
  // sub-tile `sub` (element 4 r4 + e is row 32 sub + 8 r4 + 4 half + e).
  auto load_seed = [&](const char* stat, int sub) __attribute__((always_inline)) {
    f32x16_t v;
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const f32x4_t x = *reinterpret_cast<const f32x4_t*>(stat + 4 * (32 * sub + 8 * r4 + 4 * half));
#pragma unroll
      for (int e = 0; e < 4; ++e) v[4 * r4 + e] = x[e];
    }
    return v;
  };
  // bf16 P of the block: [sub][16-query step][lane] x 8 values, the B
  // operand fragments of dV in accumulator order.
  char* const pbuf = smem + C::kPOff + pair * C::kPBytes;
  auto p_slot = [&](int sub, int j) __attribute__((always_inline)) {
    return reinterpret_cast<bf16x8_t*>(pbuf + ((sub * 2 + j) * 64 + lane) * 16);
  };

  f32x16_t acc[C::kDB];   // dV^T (P waves) or dK^T (dS waves)
#pragma unroll
  for (int db = 0; db < C::kDB; ++db) acc[db] = f32x16_t{};

  constexpr int PF = SC::PF;
  bf16x8_t fb[PF + 1];   // fragments in flight, slot position % (PF + 1)

  // ======================= P waves =======================================
  auto run_p = [&]() __attribute__((always_inline)) {
    f32x16_t s[2];        // S' of the current step, two 32-query sub-tiles
    bf16x8_t pf[2][2];    // bf16 P of the previous step, B operand of dV
    // Products of a matrix phase, kind a first: dV^T += dO^T P of the
    // previous step (PV, dO tile ldo), then S' of the current step (QK, Q
    // tile lq).  frag(pos) reads the fragment of the product at position pos.
    auto frag = [&](auto qk_tag, auto pv_tag, int pos, const char* lq, const char* ldo)
        __attribute__((always_inline)) {
      constexpr int NP = decltype(pv_tag)::value ? 4 * C::kDB : 0;
      constexpr int NQ = decltype(qk_tag)::value ? 2 * C::kKS : 0;
      const int idx = phase_order(NP, NQ, SC::POrd, pos);
      return idx < NP ? tr.load(ldo, 16 * (idx / C::kDB), idx % C::kDB) : row_frag(lq, idx - NP);
    };
    auto prefetch = [&](auto qk_tag, auto pv_tag, const char* lq, const char* ldo)
        __attribute__((always_inline)) {
      constexpr int NS = (decltype(qk_tag)::value ? 2 * C::kKS : 0) + (decltype(pv_tag)::value ? 4 * C::kDB : 0);
#pragma unroll
      for (int i = 0; i < (PF < NS ? PF : NS); ++i) fb[i] = frag(qk_tag, pv_tag, i, lq, ldo);
    };
    // QK seeds its accumulators from statistic lst.  With pre_tag false the
    // phase reads its own first fragments.
    auto matrix = [&](auto qk_tag, auto pv_tag, auto pre_tag, const char* lq, const char* lst,
                      const char* ldo) __attribute__((always_inline)) {
      constexpr bool kQK = decltype(qk_tag)::value;
      constexpr bool kPV = decltype(pv_tag)::value;
      constexpr int NP = kPV ? 4 * C::kDB : 0;   // (16-row step, db), db fastest
      constexpr int NQ = kQK ? 2 * C::kKS : 0;   // (ks, sub), sub fastest
      constexpr int NS = NQ + NP;
      constexpr int fb0 = phase_first_b(NP, NQ, SC::POrd);
      constexpr int seed_pos = fb0 > SC::SeedLead ? fb0 - SC::SeedLead : 0;
      if constexpr (!decltype(pre_tag)::value) prefetch(qk_tag, pv_tag, lq, ldo);
#pragma unroll
      for (int pos = 0; pos < NS; ++pos) {
        if (pos + PF < NS) fb[(pos + PF) % (PF + 1)] = frag(qk_tag, pv_tag, pos + PF, lq, ldo);
        if (kQK && pos == seed_pos) {
          s[0] = load_seed(lst, 0);
          s[1] = load_seed(lst, 1);
        }
        const int idx = phase_order(NP, NQ, SC::POrd, pos);
        if (idx < NP) {
          const int st = idx / C::kDB;
          acc[idx % C::kDB] = mfma32(fb[pos % (PF + 1)], pf[st >> 1][st & 1], acc[idx % C::kDB]);
        } else {
          const int j = idx - NP;
          s[j & 1] = mfma32(fb[pos % (PF + 1)], bfrag[j >> 1], s[j & 1]);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    // Vector phase of a step whose first query is i0r: scale, mask,
    // exponentials, P to LDS; issue(k), k = 0..4, issues part k of the dO
    // copies.
    auto vector = [&](int i0r, auto issue) __attribute__((always_inline)) {
      issue(0);
      // S' scale log2(e) = S scale log2(e) - LSE log2(e): the exp2 domain.
#pragma unroll
      for (int sub = 0; sub < 2; ++sub)
#pragma unroll
        for (int i = 0; i < 16; ++i) s[sub][i] *= c2;
      // Element mask without compares: with [lo, hi) the visible queries of
      // this lane's key as offsets into the sub-tile, each score gets
      // clamp(min(q - lo, hi - 1 - q), -1, 0) * 2^100 added: exactly 0 when
      // visible; otherwise the score becomes exactly -2^100 (the score itself
      // is absorbed) and its probability exactly 0.
#pragma unroll
      for (int sub = 0; sub < 2; ++sub) {
        const int s0 = i0r + 32 * sub;
        if (s0 < flo || s0 + 32 > fhi) {
          // Offsets clamped to [-1, 33], then shifted by this lane's 4*half
          // so that every element uses a constant query offset.
          const float neg_lo = (float)(4 * half - min(max(my_lo - s0, -1), 33));
          const float hi_m1 = (float)(min(max(my_hi - s0, -1), 33) - 1 - 4 * half);
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const float j = (float)(8 * (i >> 2) + (i & 3));   // query offset minus 4*half
            const float d = __builtin_amdgcn_fmed3f(fminf(j + neg_lo, hi_m1 - j), -1.0f, 0.0f);
            s[sub][i] = fmaf(d, 0x1p100f, s[sub][i]);
          }
        }
      }
      issue(1);
#pragma unroll
      for (int sub = 0; sub < 2; ++sub) {
#pragma unroll
        for (int i = 0; i < 16; ++i) pf[sub][i >> 3][i & 7] = (__bf16)__builtin_amdgcn_exp2f(s[sub][i]);
        *p_slot(sub, 0) = pf[sub][0];
        *p_slot(sub, 1) = pf[sub][1];
        issue(2 + sub);
      }
      issue(4);
    };

    constexpr std::integral_constant<bool, SC::PPre> p_pre{};
    Cursor cur{qt_hi - 1, 0, 0};   // step being computed
    Cursor cp = cur;               // step whose dO copies go out next
    auto issue_to = [&](int slot) __attribute__((always_inline)) {
      return [&, slot](int k) __attribute__((always_inline)) {
        copy_part(false_type{}, cp, k, do_tile(slot), d_stat(slot));
      };
    };
    // Prologue: dO and D of steps 0 and 1.
#pragma unroll
    for (int k = 0; k <= C::kCopies; ++k) copy_part(false_type{}, cp, k, do_tile(0), d_stat(0));
    advance(cp);
#pragma unroll
    for (int k = 0; k <= C::kCopies; ++k) copy_part(false_type{}, cp, k, do_tile(1), d_stat(1));
    advance(cp);
    block_barrier();
    // Step 0: scores only.
    matrix(true_type{}, false_type{}, false_type{}, q_tile(0), lse_stat(0), do_tile(0));
    wait_vmem_n<C::kPhaseCopies>();
    block_barrier();
    vector((cur.t - qt_lo) * C::kBQ, issue_to(2));
    if constexpr (SC::PPre) prefetch(true_type{}, true_type{}, q_tile(0), do_tile(0));   // dO of step 0, for A(1)
    advance(cp);
    block_barrier();
    advance(cur);
    int dslot = 1;   // dO buffer of the current step: n % 3
    auto step = [&](auto r_tag) __attribute__((always_inline)) {
      constexpr int r = decltype(r_tag)::value;   // n % 4
      const int prev = dslot == 0 ? 2 : dslot - 1;  // (n - 1) % 3 == (n + 2) % 3
      matrix(true_type{}, true_type{}, p_pre, q_tile(r), lse_stat(r), do_tile(prev));
      wait_vmem_n<C::kPhaseCopies>();
      block_barrier();
      vector((cur.t - qt_lo) * C::kBQ, issue_to(prev));
      if constexpr (SC::PPre) prefetch(true_type{}, true_type{}, q_tile(0), do_tile(dslot));   // dO of step n, for A(n+1)
      advance(cp);
      block_barrier();
      advance(cur);
      dslot = dslot == 2 ? 0 : dslot + 1;
    };
    for (int n = 1; n < n_steps; n += 4) {
      step(integral_constant<int, 1>{});
      if (n + 1 < n_steps) step(integral_constant<int, 2>{});
      if (n + 2 < n_steps) step(integral_constant<int, 3>{});
      if (n + 3 < n_steps) step(integral_constant<int, 0>{});
    }
    // Phase A after the last step: dV of the last step only (its first
    // fragments, from the same dO tile, were read above).
    matrix(false_type{}, true_type{}, p_pre, q_tile(0), lse_stat(0),
           do_tile(dslot == 0 ? 2 : dslot - 1));
    block_barrier();
  };

  // ======================= dS waves ======================================
  auto run_ds = [&]() __attribute__((always_inline)) {
    f32x16_t dp[2];       // dP' of the current step, two 32-query sub-tiles
    bf16x8_t dsf[2][2];   // bf16 dS of the previous step, B operand of dK
    // Products of a matrix phase, kind a first: dK^T += Q^T dS of the
    // previous step (DK, Q tile lq), then dP' of the current step (DP, dO
    // tile ldo).
    auto frag = [&](auto dk_tag, auto dp_tag, int pos, const char* lq, const char* ldo)
        __attribute__((always_inline)) {
      constexpr int NK = decltype(dk_tag)::value ? 4 * C::kDB : 0;
      constexpr int ND = decltype(dp_tag)::value ? 2 * C::kKS : 0;
      const int idx = phase_order(NK, ND, SC::DOrd, pos);
      return idx < NK ? tr.load(lq, 16 * (idx / C::kDB), idx % C::kDB) : row_frag(ldo, idx - NK);
    };
    auto prefetch = [&](auto dk_tag, auto dp_tag, const char* lq, const char* ldo)
        __attribute__((always_inline)) {
      constexpr int NS = (decltype(dk_tag)::value ? 4 * C::kDB : 0) + (decltype(dp_tag)::value ? 2 * C::kKS : 0);
#pragma unroll
      for (int i = 0; i < (PF < NS ? PF : NS); ++i) fb[i] = frag(dk_tag, dp_tag, i, lq, ldo);
    };
    // DP seeds its accumulators from statistic lst.
    auto matrix = [&](auto dk_tag, auto dp_tag, auto pre_tag, const char* lq, const char* ldo,
                      const char* lst) __attribute__((always_inline)) {
      constexpr bool kDK = decltype(dk_tag)::value;
      constexpr bool kDP = decltype(dp_tag)::value;
      constexpr int NK = kDK ? 4 * C::kDB : 0;   // (16-row step, db), db fastest
      constexpr int ND = kDP ? 2 * C::kKS : 0;   // (ks, sub), sub fastest
      constexpr int NS = NK + ND;
      constexpr int fb0 = phase_first_b(NK, ND, SC::DOrd);
      constexpr int seed_pos = fb0 > SC::SeedLead ? fb0 - SC::SeedLead : 0;
      if constexpr (!decltype(pre_tag)::value) prefetch(dk_tag, dp_tag, lq, ldo);
#pragma unroll
      for (int pos = 0; pos < NS; ++pos) {
        if (pos + PF < NS) fb[(pos + PF) % (PF + 1)] = frag(dk_tag, dp_tag, pos + PF, lq, ldo);
        if (kDP && pos == seed_pos) {
          dp[0] = load_seed(lst, 0);
          dp[1] = load_seed(lst, 1);
        }
        const int idx = phase_order(NK, ND, SC::DOrd, pos);
        if (idx < NK) {
          const int st = idx / C::kDB;
          acc[idx % C::kDB] = mfma32(fb[pos % (PF + 1)], dsf[st >> 1][st & 1], acc[idx % C::kDB]);
        } else {
          const int j = idx - NK;
          dp[j & 1] = mfma32(fb[pos % (PF + 1)], bfrag[j >> 1], dp[j & 1]);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    // Vector phase: dS = P dP' of the previous step, to bf16; issue(k),
    // k = 0..4, issues part k of the Q copies.
    auto vector = [&](auto issue) __attribute__((always_inline)) {
      bf16x8_t pb[2][2];
#pragma unroll
      for (int sub = 0; sub < 2; ++sub) {
        pb[sub][0] = *p_slot(sub, 0);
        pb[sub][1] = *p_slot(sub, 1);
      }
      issue(0);
      issue(1);
#pragma unroll
      for (int sub = 0; sub < 2; ++sub) {
#pragma unroll
        for (int i = 0; i < 16; ++i)
          dsf[sub][i >> 3][i & 7] = (__bf16)((float)pb[sub][i >> 3][i & 7] * dp[sub][i]);
        issue(2 + sub);
      }
      issue(4);
    };

    constexpr std::integral_constant<bool, SC::DPre> d_pre{};
    Cursor cq{qt_hi - 1, 0, 0};   // step whose Q copies go out next
    auto issue_to = [&](int slot) __attribute__((always_inline)) {
      return [&, slot](int k) __attribute__((always_inline)) {
        copy_part(true_type{}, cq, k, q_tile(slot), lse_stat(slot));
      };
    };
    auto no_issue = [](int) {};
    // Prologue: Q and LSE of steps 0 and 1; step 0's must land before A(0).
#pragma unroll
    for (int k = 0; k <= C::kCopies; ++k) copy_part(true_type{}, cq, k, q_tile(0), lse_stat(0));
    advance(cq);
#pragma unroll
    for (int k = 0; k <= C::kCopies; ++k) copy_part(true_type{}, cq, k, q_tile(1), lse_stat(1));
    advance(cq);
    wait_vmem_n<C::kPhaseCopies>();
    block_barrier();
    // Step 0: phase A only copies, phase B forms dP'.
    {
      auto issue = issue_to(2);
#pragma unroll
      for (int k = 0; k <= C::kCopies; ++k) issue(k);
    }
    advance(cq);
    block_barrier();
    matrix(false_type{}, true_type{}, false_type{}, q_tile(0), do_tile(0), d_stat(0));
    wait_vmem_n<C::kPhaseCopies>();
    block_barrier();
    int dslot = 1;   // dO buffer of the current step: n % 3
    auto step = [&](auto r_tag) __attribute__((always_inline)) {
      constexpr int r = decltype(r_tag)::value;   // n % 4
      vector(issue_to((r + 2) & 3));
      if constexpr (SC::DPre) prefetch(true_type{}, true_type{}, q_tile((r + 3) & 3), do_tile(0));   // Q of step n-1
      advance(cq);
      block_barrier();
      matrix(true_type{}, true_type{}, d_pre, q_tile((r + 3) & 3), do_tile(dslot), d_stat(dslot));
      wait_vmem_n<C::kPhaseCopies>();
      block_barrier();
      dslot = dslot == 2 ? 0 : dslot + 1;
    };
    for (int n = 1; n < n_steps; n += 4) {
      step(integral_constant<int, 1>{});
      if (n + 1 < n_steps) step(integral_constant<int, 2>{});
      if (n + 2 < n_steps) step(integral_constant<int, 3>{});
      if (n + 3 < n_steps) step(integral_constant<int, 0>{});
    }
    // After the last step: its dS (phase A), then its dK product (phase B).
    vector(no_issue);
    const char* q_last = q_tile((n_steps - 1) & 3);
    if constexpr (SC::DPre) prefetch(true_type{}, false_type{}, q_last, do_tile(0));
    block_barrier();
    matrix(true_type{}, false_type{}, d_pre, q_last, do_tile(0), d_stat(0));
  };

  if (n_steps > 0) {
    if (p_wave)
      run_p();
    else
      run_ds();
  }
  // No copy may still be writing LDS when the workgroup ends.
  wait_vmem();

  if (kj < N) {
    const float mul = p_wave ? 1.f : p.scale;
    if (split > 1) {   // fp32 partial of this part
      float* row = p.dkv_part +
                   ((((int64_t)part * 2 + (p_wave ? 1 : 0)) * p.bs + b) * p.hkv + kh) * N * HD +
                   kj * HD;
#pragma unroll
      for (int d = 0; d < C::kDB; ++d)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          f32x4_t w;
#pragma unroll
          for (int e = 0; e < 4; ++e) w[e] = acc[d][4 * r4 + e] * mul;
          *reinterpret_cast<f32x4_t*>(row + d * 32 + 8 * r4 + 4 * half) = w;
        }
    } else {
      __bf16* row = kFused ? chunk_row(p_wave ? p.cdv : p.cdk, (uint32_t)kj, p.bs, b, kh, HD)
                           : (p_wave ? p.dv : p.dk) + kj * kv_tok + kvoff;
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
  }
}

// dK and dV from the split's fp32 partials: parts added in order 0, 1, ...
// and rounded once to bf16.  One thread per 4 consecutive head-dim values
// of a (tensor, batch, kv head, key) row.
template <int HD, bool kFused>
__global__ __launch_bounds__(256) void dkv_reduce_kernel(BwdParams p) {
  constexpr int kQuads = HD / 4;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t N = p.N;
  const int64_t rows = 2 * (int64_t)p.bs * p.hkv * N;
  if (i >= rows * kQuads) return;
  const int qd = (int)(i % kQuads);
  int64_t r = i / kQuads;
  const int64_t kj = r % N;
  r /= N;
  const int kh = (int)(r % p.hkv);
  r /= p.hkv;
  const int b = (int)(r % p.bs);
  const int tensor = (int)(r / p.bs);   // 0: dK, 1: dV
  const int64_t plane = rows * HD;      // floats per part
  const float* src = p.dkv_part + (((int64_t)tensor * p.bs + b) * p.hkv + kh) * N * HD + kj * HD + 4 * qd;
  f32x4_t sum = *reinterpret_cast<const f32x4_t*>(src);
  for (int part = 1; part < p.split; ++part) {
    const f32x4_t x = *reinterpret_cast<const f32x4_t*>(src + part * plane);
#pragma unroll
    for (int e = 0; e < 4; ++e) sum[e] += x[e];
  }
  bf16x4_t w;
#pragma unroll
  for (int e = 0; e < 4; ++e) w[e] = (__bf16)sum[e];
  const int64_t kv_tok = (int64_t)p.bs * p.kv_row_heads * HD;
  const int64_t kvoff = ((int64_t)b * p.kv_row_heads + kh) * HD;
  __bf16* row = kFused ? chunk_row(tensor ? p.cdv : p.cdk, (uint32_t)kj, p.bs, b, kh, HD)
                       : (tensor ? p.dv : p.dk) + kj * kv_tok + kvoff;
  *reinterpret_cast<bf16x4_t*>(row + 4 * qd) = w;
}

// -D_i = -<dO_i, O_i> and -LSE_i / scale of every query row, stored
// [batch][head][position]: the dQ kernel reads them per row, the dK/dV
// kernel as 64-row runs.  kLanes lanes reduce one row.  In the fused form O
// and dO are read from their sequence chunks (co, cdo).
template <int HD, bool kFused>
__global__ __launch_bounds__(256) void bwd_stats_kernel(const __bf16* __restrict__ o,
                                                        const __bf16* __restrict__ dout,
                                                        const float* __restrict__ lse,
                                                        float* __restrict__ nD,
                                                        float* __restrict__ nlse_r, float scale,
                                                        int64_t rows, int64_t N, int bs, int hq,
                                                        SeqChunks co, SeqChunks cdo) {
  constexpr int kLanes = HD / 8;
  constexpr int kRowsPerBlock = 256 / kLanes;
  const int64_t r = (int64_t)blockIdx.x * kRowsPerBlock + threadIdx.x / kLanes;
  const int sub = threadIdx.x % kLanes;
  // r enumerates (i, b, h) in the memory order of a head-sharded tensor
  const int h = (int)(r % hq);
  const int64_t ib = r / hq;
  const int b = (int)(ib % bs);
  const int64_t i = ib / bs;
  float acc = 0.f;
  if (r < rows) {
    const __bf16* orow = kFused ? chunk_row(co, (uint32_t)i, bs, b, h, HD) : o + r * HD;
    const __bf16* drow = kFused ? chunk_row(cdo, (uint32_t)i, bs, b, h, HD) : dout + r * HD;
    const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(orow + sub * 8);
    const bf16x8_t c = *reinterpret_cast<const bf16x8_t*>(drow + sub * 8);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc += (float)a[e] * (float)c[e];
  }
#pragma unroll
  for (int off = kLanes / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off, 64);
  if (r < rows && sub == 0) {
    const int64_t idx = ((int64_t)b * hq + h) * N + i;
    nD[idx] = -acc;
    nlse_r[idx] = -lse[idx] / scale;
  }
}

template <int HD, int GPACK, bool kFused>
hipError_t launch_dq(BwdParams p, const AttnShape& s, hipStream_t stream) {
  using C = DqCfg<HD, GPACK>;
  p.num_blocks = (s.N + C::kBP - 1) / C::kBP;
  dim3 grid((uint32_t)p.num_blocks, (uint32_t)(s.bs * s.hkv * (p.g / GPACK)));
  return launch_kernel(attn_bwd_dq_kernel<HD, GPACK, kFused>, grid, dim3(C::kThreads), 0, stream, p);
}

// The three launches of the backward (statistics, dQ, dK/dV) for parameters
// p; o and p.dout (single-buffer statistics) or co and p.cdo (chunked
// statistics) feed the statistics.
template <bool kFused, bool kStatsFused = kFused>
hipError_t launch_bwd(BwdParams& p, const AttnShape& s, const __bf16* o, const SeqChunks& co,
                      const float* lse, void* workspace, size_t workspace_bytes,
                      hipStream_t stream) {
  float* nD = static_cast<float*>(workspace);
  float* nlse_r = reinterpret_cast<float*>(static_cast<char*>(workspace) + stat_array_bytes(s));
  p.nD = nD;
  p.nlse_r = nlse_r;
  // The split runs when the workspace holds its partials (always for a
  // workspace of attn_bwd_workspace_bytes; the fixed scratch of the
  // allocation-free entry point may not).
  p.split = dkv_split(s);
  if (2 * stat_array_bytes(s) + dkv_part_bytes(s, p.split) > workspace_bytes) p.split = 1;
  p.dkv_part = reinterpret_cast<float*>(static_cast<char*>(workspace) + 2 * stat_array_bytes(s));
  p.N = s.N;
  p.bs = s.bs;
  p.hq = s.hq;
  p.hkv = s.hkv;
  p.g = s.hq / s.hkv;
  if (!p.q_row_heads) p.q_row_heads = s.hq;
  if (!p.kv_row_heads) p.kv_row_heads = s.hkv;
  p.scale = s.scale;
  p.scale_log2 = s.scale * kLog2e;
  p.causal = s.causal;
  p.cu = s.cu;
  p.n_docs = s.n_docs;
  p.num_blocks = 0;

  const int64_t rows = s.N * s.bs * s.hq;
  const int64_t stat_blocks = (rows + (s.hd == 128 ? 15 : 31)) / (s.hd == 128 ? 16 : 32);
  hipError_t e = launch_kernel(s.hd == 128 ? bwd_stats_kernel<128, kStatsFused>
                                            : bwd_stats_kernel<64, kStatsFused>,
                               dim3((uint32_t)stat_blocks), dim3(256), 0, stream, o, p.dout, lse,
                               nD, nlse_r, s.scale, rows, s.N, s.bs, s.hq, co, p.cdo);
  if (e != hipSuccess) return e;

  auto dq_launch = [&](auto hd_tag) -> hipError_t {
    constexpr int HD = decltype(hd_tag)::value;
    if (p.g % 8 == 0) return launch_dq<HD, 8, kFused>(p, s, stream);
    if (p.g % 4 == 0) return launch_dq<HD, 4, kFused>(p, s, stream);
    if (p.g % 2 == 0) return launch_dq<HD, 2, kFused>(p, s, stream);
    return launch_dq<HD, 1, kFused>(p, s, stream);
  };
  auto dkv_launch = [&](auto hd_tag) -> hipError_t {
    constexpr int HD = decltype(hd_tag)::value;
    using C = DkvCfg<HD>;
    static_assert(C::kBK == 128, "dkv_split counts 128-key blocks");
    dim3 grid((uint32_t)((s.N + C::kBK - 1) / C::kBK * p.split), (uint32_t)(s.bs * s.hkv));
    hipError_t e2 = launch_kernel(attn_bwd_dkv_kernel<HD, kFused>, grid, dim3(C::kThreads), 0,
                                  stream, p);
    if (e2 != hipSuccess || p.split == 1) return e2;
    const int64_t quads = 2 * (int64_t)s.bs * s.hkv * s.N * (HD / 4);
    return launch_kernel(dkv_reduce_kernel<HD, kFused>, dim3((uint32_t)((quads + 255) / 256)),
                         dim3(256), 0, stream, p);
  };
  if (s.hd == 128) {
    if ((e = dq_launch(std::integral_constant<int, 128>{})) != hipSuccess) return e;
    return dkv_launch(std::integral_constant<int, 128>{});
  }
  if ((e = dq_launch(std::integral_constant<int, 64>{})) != hipSuccess) return e;
  return dkv_launch(std::integral_constant<int, 64>{});
}

}  // namespace


size_t attn_bwd_workspace_bytes(const AttnShape& s, bool bf16) {
  if (!bf16) return stat_array_bytes(s);
  return 2 * stat_array_bytes(s) + dkv_part_bytes(s, dkv_split(s));
}

size_t attn_bwd_min_workspace_bytes(const AttnShape& s, bool bf16) {
  return (bf16 ? 2 : 1) * stat_array_bytes(s);
}

hipError_t launch_attn_bwd_bf16(const AttnShape& s, const void* q, const void* k, const void* v,
                                const void* o, const float* lse, const void* dout, void* dq,
                                void* dk, void* dv, void* workspace, size_t workspace_bytes,
                                hipStream_t stream) {
  if (s.N == 0) return hipSuccess;
  BwdParams p{};
  p.q = static_cast<const __bf16*>(q);
  p.k = static_cast<const __bf16*>(k);
  p.v = static_cast<const __bf16*>(v);
  p.dout = static_cast<const __bf16*>(dout);
  p.dq = static_cast<__bf16*>(dq);
  p.dk = static_cast<__bf16*>(dk);
  p.dv = static_cast<__bf16*>(dv);
  return launch_bwd<false>(p, s, static_cast<const __bf16*>(o), p.cq, lse, workspace,
                           workspace_bytes, stream);
}

hipError_t launch_attn_bwd_bf16_fused(const AttnShape& s, const SeqChunks& q, const SeqChunks& k,
                                      const SeqChunks& v, const SeqChunks& o, const float* lse,
                                      const SeqChunks& dout, const SeqChunks& dq,
                                      const SeqChunks& dk, const SeqChunks& dv, void* workspace,
                                      size_t workspace_bytes, hipStream_t stream) {
  if (s.N == 0) return hipSuccess;
  BwdParams p{};
  p.cdo = dout;   // the statistics read O and dO from their chunks either way
  const uintptr_t base[7] = {
      contiguous_base(q, s.N, s.bs, s.hd),  contiguous_base(k, s.N, s.bs, s.hd),
      contiguous_base(v, s.N, s.bs, s.hd),  contiguous_base(dout, s.N, s.bs, s.hd),
      contiguous_base(dq, s.N, s.bs, s.hd), contiguous_base(dk, s.N, s.bs, s.hd),
      contiguous_base(dv, s.N, s.bs, s.hd)};
  bool strided = true;
  for (uintptr_t b : base) strided = strided && b != 0;
  if (strided) {
    // Every gradient-kernel table is a strided view of one tensor: the
    // single-buffer kernels with the global head counts as row strides.
    p.q = reinterpret_cast<const __bf16*>(base[0]);
    p.k = reinterpret_cast<const __bf16*>(base[1]);
    p.v = reinterpret_cast<const __bf16*>(base[2]);
    p.dout = reinterpret_cast<const __bf16*>(base[3]);
    p.dq = reinterpret_cast<__bf16*>(base[4]);
    p.dk = reinterpret_cast<__bf16*>(base[5]);
    p.dv = reinterpret_cast<__bf16*>(base[6]);
    p.q_row_heads = q.row_heads;
    p.kv_row_heads = k.row_heads;
    return launch_bwd<false, true>(p, s, nullptr, o, lse, workspace, workspace_bytes, stream);
  }
  p.cq = q;
  p.ck = k;
  p.cv = v;
  p.cdo = dout;
  p.cdq = dq;
  p.cdk = dk;
  p.cdv = dv;
  return launch_bwd<true>(p, s, nullptr, o, lse, workspace, workspace_bytes, stream);
}

}  // namespace ulysses
