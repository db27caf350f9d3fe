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
//  * Matrix and vector work alternate between the two waves that share a
//    SIMD (waves w and w+4).  Work is cut into phases separated by
//    workgroup barriers; in every phase one wave of each SIMD issues only
//    matrix products (the scores of key tile t and the PV product of tile
//    t-1, 32 MFMAs) while its partner runs only the softmax of a tile (mask,
//    row max, exponentials, row sum, bf16 rounding), which the SIMD executes
//    alongside the partner's MFMAs.  The second group of waves runs one
//    phase behind the first.  Each group has its own copy of the loop, and
//    every pair of phases has the same shape, so the compiler keeps the
//    loop free of spills and of conservative memory waits.
//  * K and V tiles reach LDS by direct global-to-LDS copies (no registers
//    spent on staging), issued by the waves in pieces spread through their
//    softmax phase, two pairs of phases ahead of use, into four rotating
//    buffers per tensor (128 KiB of LDS at head size 128).
//  * Online softmax in the exp2 domain.  Q enters the products exactly as
//    given (bf16); the fp32 score is taken to the exp2 domain by one FMA,
//    s * scale*log2(e) - m, so the softmax scale adds no bf16 rounding.  The
//    running max is only raised when a row's max grows by more than 8 (a
//    factor 256), so O and the row sum are rarely rescaled; any reference max
//    gives the same result in exact arithmetic.  The row max of a lane pair
//    uses v_permlane32_swap.
//  * Key tiles entirely above the diagonal (or outside the documents of a
//    block) are never visited.  Every wave walks all tiles of its block;
//    tiles crossing a boundary of some row of the wave (or not seen by it at
//    all) get an element mask that adds a penalty instead of comparing, so
//    the rarely taken mask code holds no compare masks in scalar registers.
//  * LDS rows are swizzled in 16-byte chunks (swz in device_common.h) so both
//    the row reads of K and the transposing reads of V avoid bank conflicts;
//    fragments are read several products ahead of the MFMA that uses them.
//  * Blocks are launched heaviest first: by position for one document, by
//    their work within documents for packed documents (doc_sorted_block).
#include <math.h>

#include <type_traits>

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
  // Heads per token row in memory of q/o and of k/v: hq and hkv for
  // head-sharded tensors, the global counts for strided views of the
  // sequence chunks (q, k, v, o then point at the rank's first head).
  int q_row_heads, kv_row_heads;
  float scale_log2;   // softmax scale * log2(e)
  int causal;
  const int32_t* cu;
  int n_docs;
  int64_t num_pos_blocks;
  // Fused form only: the operands in their sequence chunks (q, k, v, o
  // above are unused).
  SeqChunks cq, ck, cv, co;
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
  static constexpr int kBufs = 4;                    // rotating LDS buffers per tensor
  // One wave-wide direct copy moves 1 KiB (64 lanes x 16 bytes).
  static constexpr int kRowsPerCopy = 1024 / kRowBytes;
  static constexpr int kCopiesPerWave = kTileBytes / 1024 / kWaves;   // per tensor and tile
  static constexpr int kPrefetch = 4;                // fragments read ahead of their MFMA
  static_assert(kCopiesPerWave >= 1 && kTileBytes % (1024 * kWaves) == 0, "tile copies");
};

template <int HD, int GPACK, bool kFused>
__global__ __launch_bounds__(512) void attn_fwd_bf16_kernel(FwdParams p) {
  using C = FwdCfg<HD, GPACK>;
  __shared__ __attribute__((aligned(1024))) char smem[2 * C::kBufs * C::kTileBytes];
  char* const lds_k0 = smem;                               // K buffers
  char* const lds_v0 = smem + C::kBufs * C::kTileBytes;    // V buffers

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5;      // which k-half / row-quad of the MFMA layout
  const int r32 = lane & 31;
  const int group = wave >> 2;     // waves w and w+4 share a SIMD

  const int64_t N = wave_uniform(p.N);
  // Dispatch rank t of this workgroup over (block, slice) pairs, slices
  // fastest, so every slice's heavy blocks go first; blocks by position,
  // heaviest (largest positions) first, or by work within documents.
  const uint64_t lin = (uint64_t)blockIdx.y * gridDim.x + blockIdx.x;
  const int64_t t = lin / gridDim.y;
  int64_t pb = p.num_pos_blocks - 1 - t;
  if (p.cu != nullptr && p.causal) {
    const int64_t s = doc_sorted_block<false>(t, p.num_pos_blocks, C::kBP, p.cu, p.n_docs, N);
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
  const __bf16* qbase = p.q + ((int64_t)b * p.q_row_heads + h) * HD;
  // (Kept in scalar registers: the copies take their base from there.)  In
  // the fused form they are the chunk tables' first chunk, replaced per tile.
  const __bf16* kbase = reinterpret_cast<const __bf16*>(wave_uniform(
      kFused ? (int64_t)p.ck.chunk[0] : reinterpret_cast<int64_t>(p.k + ((int64_t)b * p.kv_row_heads + kh) * HD)));
  const __bf16* vbase = reinterpret_cast<const __bf16*>(wave_uniform(
      kFused ? (int64_t)p.cv.chunk[0] : reinterpret_cast<int64_t>(p.v + ((int64_t)b * p.kv_row_heads + kh) * HD)));
  // Address of row i of Q (or O) for this lane's head.
  auto q_row = [&](const SeqChunks& c, int64_t i) __attribute__((always_inline)) {
    return chunk_row(c, (uint32_t)i, p.bs, b, h, HD);
  };

  // Q fragments (B operand of S^T): lane holds Q[qi][16 ks + 8 half + 0..7]
  // as stored (the scale is applied to the fp32 scores).
  bf16x8_t qf[C::kKS];
#pragma unroll
  for (int ks = 0; ks < C::kKS; ++ks) {
    qf[ks] = bf16x8_t{};
    if (qi < N) {
      const __bf16* row = kFused ? q_row(p.cq, qi) : qbase + qi * q_tok;
      qf[ks] = *reinterpret_cast<const bf16x8_t*>(row + 16 * ks + 8 * half);
    }
  }
  const float c2 = p.scale_log2;   // softmax scale * log2(e)

  // Key range of the whole block, and the keys of this wave and lane.  Every
  // wave walks all key tiles of its block (so all waves share one schedule);
  // tiles a wave does not see are masked out entirely.
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

  // Key tiles of the block: t_begin .. t_begin + n_tiles - 1.
  const int64_t t_begin = wave_uniform(kv_lo / C::kBC);
  const int n_tiles = (int)wave_uniform((kv_hi + C::kBC - 1) / C::kBC - t_begin);

  // K and V tiles reach LDS by direct global-to-LDS copies: a wave moves its
  // share of a tile (kCopiesPerWave slices of 1 KiB, 16 bytes per lane).
  // Slice c of the tile lands at bytes [1024 c, 1024 c + 1024) of the
  // buffer, lane l at +16 l, so lane l fetches the source chunk that the
  // swizzle places there.  Rows past the sequence end re-read row N-1: those
  // keys are masked for every query, so only their finiteness matters.
  const int64_t row_bytes = kFused ? (int64_t)p.bs * p.ck.row_heads * HD * 2 : kv_tok * 2;
  // Lane byte offsets of this wave's slices within a tile that lies wholly
  // inside the sequence (the usual case; the last tile of a sequence whose
  // length is not a multiple of kBC clamps its rows instead).
  // Tile-level decisions use 32-bit offsets from the block's first key (the
  // scalar unit has no 64-bit ordered compare).
  const int keys_left = (int)wave_uniform(N - key0);      // keys from key0 to the end
  const int m_tail = keys_left / C::kBC;                   // first tile running past N
  const int flo = (int)wave_uniform(full_lo - key0);
  const int fhi = (int)wave_uniform(full_hi - key0);
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
    if constexpr (kFused) {
      tile = reinterpret_cast<const char*>(
          wave_uniform(chunk_tile_base(ch, (uint32_t)(t_begin + m), p.bs, b, kh, HD)));
    } else {
      tile = reinterpret_cast<const char*>(wave_uniform((int64_t)base + j0 * row_bytes));
    }
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
  auto copy_tile = [&](const __bf16* base, const SeqChunks& ch, char* buf, int m)
      __attribute__((always_inline)) {
#pragma unroll
    for (int c = 0; c < C::kCopiesPerWave; ++c) copy_slice(base, ch, buf, m, c);
  };

  f32x16_t acc_o[C::kDB];
#pragma unroll
  for (int db = 0; db < C::kDB; ++db) acc_o[db] = f32x16_t{};
  float m_run = -INFINITY;   // reference max, log2 domain
  float l_run = 0.f;         // this lane's share of the row sum
  // -m_run, or 0 while the row has no maximum yet: a raw score s becomes
  // s * scale*log2(e) - m_run.
  float nbias = 0.f;
  bool ref_ready = false;    // every row of the wave has a reference max
  f32x16_t s[2];             // scores of a tile, from its matrix to its vector phase
  bf16x8_t pf[4];            // bf16 probabilities of a tile, awaiting its PV product
#pragma unroll
  for (int i = 0; i < 4; ++i) pf[i] = bf16x8_t{};

  // --- matrix phase: S = scores of tile m (QK), O += P(m-1) V(m-1) (PV) ---
  // LDS byte offsets of this lane's fragments.  The swizzle depends on the
  // low four row bits only, so the 32-key half kb of a K read and the 16-key
  // step ks of a V read add constant offsets.
  int koff[C::kKS];
#pragma unroll
  for (int ks = 0; ks < C::kKS; ++ks) koff[ks] = swz<C::kChunks, C::kRowBytes>(r32, 2 * ks + half);
  // The V buffers start past a ds_read's 16-bit offset field (64 KiB at
  // head size 128).  Their start is folded into the transposing reader's
  // lane offsets, behind an empty asm so the compiler cannot split it back
  // out, and V tiles are addressed from the K region's start: every V read
  // is then a lane register plus an immediate, with no vector add per read.
  TrReader<C::kChunks, C::kRowBytes, C::kDB> vtr(lane);
  {
    int vregion = C::kBufs * C::kTileBytes;
    asm volatile("" : "+v"(vregion));
#pragma unroll
    for (int jh = 0; jh < 2; ++jh)
#pragma unroll
      for (int db = 0; db < C::kDB; ++db) vtr.off[jh][db] += vregion;
  }
  auto kfrag = [&](const char* lk, int idx) __attribute__((always_inline)) {
    const int ks = idx >> 1, kb = idx & 1;
    return *reinterpret_cast<const bf16x8_t*>(lk + kb * 32 * C::kRowBytes + koff[ks]);
  };
  auto vfrag = [&](const char* lv, int idx) __attribute__((always_inline)) {
    return vtr.load(lv - C::kBufs * C::kTileBytes, 16 * (idx / C::kDB), idx % C::kDB);
  };
  auto matrix_phase = [&](auto qk_tag, auto pv_tag, const char* lk, const char* lv) __attribute__((always_inline)) {
    constexpr bool kQK = decltype(qk_tag)::value;
    constexpr bool kPV = decltype(pv_tag)::value;
    constexpr int NQ = kQK ? 2 * C::kKS : 0;   // (ks, kb) pairs, kb fastest
    constexpr int NP = kPV ? 4 * C::kDB : 0;   // (ks, db) pairs, db fastest
    constexpr int NS = NQ + NP;
    constexpr int PF = C::kPrefetch < NS ? C::kPrefetch : NS;
    auto frag = [&](int idx) __attribute__((always_inline)) { return idx < NQ ? kfrag(lk, idx) : vfrag(lv, idx - NQ); };
    bf16x8_t buf[PF + 1];
#pragma unroll
    for (int i = 0; i < PF; ++i) buf[i] = frag(i);
#pragma unroll
    for (int idx = 0; idx < NS; ++idx) {
      if (idx + PF < NS) buf[(idx + PF) % (PF + 1)] = frag(idx + PF);
      if (idx < NQ) {
        s[idx & 1] = mfma32(buf[idx % (PF + 1)], qf[idx >> 1], idx < 2 ? f32x16_t{} : s[idx & 1]);
      } else {
        const int i = idx - NQ;
        acc_o[i % C::kDB] = mfma32(buf[idx % (PF + 1)], pf[i / C::kDB], acc_o[i % C::kDB]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // --- vector phase: softmax of tile m's scores into pf -------------------
  // `issue(k)`, k = 0..3, issues a quarter of the wave's tile copies; the
  // quarters are spread through the softmax so that the copies, which block
  // the wave while the address unit is busy, overlap its vector work.
  auto vector_phase = [&](int m, auto mask_tag, auto issue) __attribute__((always_inline)) {
    const int jr = m * C::kBC;   // first key of the tile, relative to key0
    issue(0);
    // Raw fp32 scores to the exp2 domain, relative to the reference max.
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) s[kb][i] = fmaf(s[kb][i], c2, nbias);
    // Element mask on tiles that cross a boundary of some row of the wave,
    // without compares: with lo <= key < hi the visible keys of this row as
    // offsets into the tile, each score gets clamp(min(key - lo,
    // hi - 1 - key), -1, 0) * 2^100 added: exactly 0 when visible, and when
    // not the score becomes exactly -2^100 (the score itself is absorbed),
    // whose probability is exactly 0.
    if (decltype(mask_tag)::value && (jr < flo || jr + C::kBC > fhi)) {
      // Offsets clamped to [-1, 65], then shifted by this lane's 4*half so
      // that every element uses a constant key offset.
      const float neg_lo = (float)(4 * half - min(max(my_lo - jr, -1), 65));
      const float hi_m1 = (float)(min(max(my_hi - jr, -1), 65) - 1 - 4 * half);
      const float big = 0x1p100f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float j = (float)(kb * 32 + 8 * (i >> 2) + (i & 3));   // key offset minus 4*half
          const float d = __builtin_amdgcn_fmed3f(fminf(j + neg_lo, hi_m1 - j), -1.0f, 0.0f);
          s[kb][i] = fmaf(d, big, s[kb][i]);
        }
    }

    issue(1);

    // P = exp2(s * scale*log2e - m_run) (s already in that form), rounded to
    // bf16 as the B operand of PV; returns this lane's share of the tile's
    // row sum.
    auto exps = [&](auto issue_tag) __attribute__((always_inline)) {
      float lt = 0.f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float e = __builtin_amdgcn_exp2f(s[kb][i]);
          lt += e;
          pf[2 * kb + (i >> 3)][i & 7] = (__bf16)e;
        }
        if constexpr (decltype(issue_tag)::value) issue(2 + kb);
      }
      return lt;
    };

    // Fast path: every row of the wave has a reference max, and no
    // probability of the tile exceeds 2^60 (its lane sum stays below that).
    // The reference may then lag the true running max: probabilities up to
    // 2^60 keep O and the row sum far inside fp32 range, and rounding to bf16
    // is relative, so the result is the same as with an exact max.
    bool issued = false;
    if (ref_ready) {
      const float lt = exps(std::true_type{});
      issued = true;
      if (!wave_any(!(lt <= 0x1p60f))) {
        l_run += lt;
        return;
      }
    }

    // Exact path (a row without a reference, or a tile that would overflow):
    // row max relative to m_run (this lane's 32 keys, then the partner
    // lane's).  A row takes the tile max as its reference when it has none
    // yet and sees a key here (max above -2^99), or when its max grew by
    // more than 8; a row that sees no key here keeps m_run = -inf.
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[kb][i]);
    mx = fmaxf(mx, wave_xor32_f(mx));
    const bool raise = mx > (m_run == -INFINITY ? -0x1p99f : 8.0f);
    if (wave_any(raise)) {
      const float mb = m_run == -INFINITY ? 0.f : m_run;
      const float m_new = raise ? mb + mx : m_run;
      const float alpha = raise ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.0f;
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < C::kDB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc_o[db][i] *= alpha;
      nbias = m_run == -INFINITY ? 0.f : -m_run;
      const float shift = raise ? mx : 0.0f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) s[kb][i] -= shift;
      ref_ready = !wave_any(m_run == -INFINITY);
    }
    l_run += issued ? exps(std::false_type{}) : exps(std::true_type{});
  };

  // Global phases 2m and 2m+1 form pair m (m = 0 .. n_tiles).  Group 0 runs
  // the matrix work of pair m in phase 2m and the softmax of tile m in phase
  // 2m+1; group 1 runs one phase later (its softmax of tile m falls in phase
  // 2m+2).  The matrix work of pair m reads K of tile m from K buffer m%4
  // and V of tile m-1 from V buffer (m+3)%4.  In its softmax phase within
  // pair m every wave copies its share of K of tile m+3 into K buffer
  // (m+3)%4 and of V of tile m+2 into V buffer (m+2)%4 (both last read in
  // pair m-1).  At the end of pair m every wave waits for its copies of pair
  // m-2, so the barrier publishes the tiles that pair m+1 reads while the
  // copies of two pairs stay in flight.  Copies past the last tile are
  // clamped to it (the data lands in a buffer nobody reads again).
  using std::integral_constant;
  using std::true_type;
  using std::false_type;
  constexpr int kPairCopies = 2 * C::kCopiesPerWave;
  // Copies of pair m, in four parts: k = 0, 1 for K of tile m+3 and k = 2, 3
  // for V of tile m+2 (with one slice per tensor, parts 1 and 3 are empty).
  auto copy_part = [&](int m, auto r_tag, int k) __attribute__((always_inline)) {
    constexpr int r = decltype(r_tag)::value;   // m % 4
    const int last = n_tiles - 1;
    const bool is_v = k >= 2;
    const int c = k & 1;
    if (c >= C::kCopiesPerWave) return;
    const int t = is_v ? (m + 2 < last ? m + 2 : last) : (m + 3 < last ? m + 3 : last);
    char* buf = is_v ? lds_v0 + ((r + 2) & 3) * C::kTileBytes : lds_k0 + ((r + 3) & 3) * C::kTileBytes;
    copy_slice(is_v ? vbase : kbase, is_v ? p.cv : p.ck, buf, t, c);
    __builtin_amdgcn_sched_barrier(0);
  };
  auto copy_pair = [&](int m, auto r_tag) __attribute__((always_inline)) {
#pragma unroll
    for (int k = 0; k < 4; ++k) copy_part(m, r_tag, k);
  };

  // Pair m of the main run (1 <= m < n_tiles): scores of tile m, PV of tile
  // m-1, softmax of tile m.  Tiles the wave does not see are computed and
  // masked out entirely (P = 0), which keeps every wave on the same code.
  auto mid_pair = [&](int m, auto r_tag, auto g_tag) __attribute__((always_inline)) {
    constexpr int r = decltype(r_tag)::value;
    constexpr int g = decltype(g_tag)::value;
    matrix_phase(true_type{}, true_type{}, lds_k0 + r * C::kTileBytes,
                 lds_v0 + ((r + 3) & 3) * C::kTileBytes);
    if constexpr (g == 1) wait_vmem_n<2 * kPairCopies>();
    block_barrier();
    auto issue = [&](int k) __attribute__((always_inline)) {
      if constexpr (g == 0) copy_part(m, r_tag, k);
      else copy_part(m + 1, integral_constant<int, (r + 1) & 3>{}, k);
    };
    vector_phase(m, true_type{}, issue);
    if constexpr (g == 0) wait_vmem_n<2 * kPairCopies>();
    block_barrier();
  };
  auto run = [&](auto g_tag) __attribute__((always_inline)) {
    constexpr int g = decltype(g_tag)::value;
    // Prologue: K of tiles 0..2 and V of tiles 0..1.
    const int last = n_tiles - 1;
    copy_tile(kbase, p.ck, lds_k0, 0);
    copy_tile(kbase, p.ck, lds_k0 + C::kTileBytes, 1 < last ? 1 : last);
    copy_tile(kbase, p.ck, lds_k0 + 2 * C::kTileBytes, 2 < last ? 2 : last);
    copy_tile(vbase, p.cv, lds_v0, 0);
    copy_tile(vbase, p.cv, lds_v0 + C::kTileBytes, 1 < last ? 1 : last);
    wait_vmem();
    block_barrier();
    if constexpr (g == 1) {   // phase 0: group 1 has no softmax yet, only copies
      copy_pair(0, integral_constant<int, 0>{});
      block_barrier();
    }

    // Pair 0: scores of tile 0 only.
    matrix_phase(true_type{}, false_type{}, lds_k0, lds_v0);
    block_barrier();
    auto issue0 = [&](int k) __attribute__((always_inline)) {
      if constexpr (g == 0) copy_part(0, integral_constant<int, 0>{}, k);
      else copy_part(1, integral_constant<int, 1>{}, k);
    };
    vector_phase(0, true_type{}, issue0);
    block_barrier();

    // Pairs 1 .. n_tiles-1, four per iteration so that the buffer rotation
    // m % 4 is a compile-time constant.
    for (int m = 1; m < n_tiles; m += 4) {
      mid_pair(m, integral_constant<int, 1>{}, g_tag);
      if (m + 1 < n_tiles) mid_pair(m + 1, integral_constant<int, 2>{}, g_tag);
      if (m + 2 < n_tiles) mid_pair(m + 2, integral_constant<int, 3>{}, g_tag);
      if (m + 3 < n_tiles) mid_pair(m + 3, integral_constant<int, 0>{}, g_tag);
    }

    // Pair n_tiles: PV of the last tile only.
    matrix_phase(false_type{}, true_type{}, lds_k0,
                 lds_v0 + ((n_tiles + 3) & 3) * C::kTileBytes);
    wait_vmem();
    block_barrier();
    block_barrier();
    if constexpr (g == 0) block_barrier();   // matches group 1's leading phase
  };
  if (group == 0) run(integral_constant<int, 0>{});
  else run(integral_constant<int, 1>{});

  if (qi >= N) return;
  const float l = l_run + wave_xor32_f(l_run);
  const float inv = 1.0f / l;
  __bf16* orow = kFused ? q_row(p.co, qi) : p.o + (qi * p.bs + b) * (int64_t)p.q_row_heads * HD + (int64_t)h * HD;
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

template <int HD, int GPACK, bool kFused>
hipError_t launch_fwd(const FwdParams& prm, const AttnShape& s, hipStream_t stream) {
  using C = FwdCfg<HD, GPACK>;
  FwdParams p = prm;
  p.num_pos_blocks = (s.N + C::kBP - 1) / C::kBP;
  dim3 grid((uint32_t)p.num_pos_blocks, (uint32_t)(s.bs * s.hkv * (p.g / GPACK)));
  return launch_kernel(attn_fwd_bf16_kernel<HD, GPACK, kFused>, grid, dim3(C::kThreads), 0, stream,
                       p);
}

template <int HD, bool kFused>
hipError_t launch_fwd_hd(const FwdParams& p, const AttnShape& s, hipStream_t stream) {
  if (p.g % 8 == 0) return launch_fwd<HD, 8, kFused>(p, s, stream);
  if (p.g % 4 == 0) return launch_fwd<HD, 4, kFused>(p, s, stream);
  if (p.g % 2 == 0) return launch_fwd<HD, 2, kFused>(p, s, stream);
  return launch_fwd<HD, 1, kFused>(p, s, stream);
}

FwdParams common_params(const AttnShape& s, float* lse) {
  FwdParams p{};
  p.lse = lse;
  p.N = s.N;
  p.bs = s.bs;
  p.hq = s.hq;
  p.hkv = s.hkv;
  p.g = s.hq / s.hkv;
  p.q_row_heads = s.hq;
  p.kv_row_heads = s.hkv;
  p.scale_log2 = s.scale * kLog2e;
  p.causal = s.causal;
  p.cu = s.cu;
  p.n_docs = s.n_docs;
  p.num_pos_blocks = 0;
  return p;
}

}  // namespace

hipError_t launch_attn_fwd_bf16_fused(const AttnShape& s, const SeqChunks& q, const SeqChunks& k,
                                      const SeqChunks& v, const SeqChunks& o, float* lse,
                                      hipStream_t stream) {
  if (s.N == 0) return hipSuccess;
  FwdParams p = common_params(s, lse);
  const uintptr_t qb = contiguous_base(q, s.N, s.bs, s.hd), kb = contiguous_base(k, s.N, s.bs, s.hd),
                  vb = contiguous_base(v, s.N, s.bs, s.hd), ob = contiguous_base(o, s.N, s.bs, s.hd);
  if (qb && kb && vb && ob) {
    // Every table is a strided view of one tensor: the single-buffer kernel
    // with the global head counts as row strides.
    p.q = reinterpret_cast<const __bf16*>(qb);
    p.k = reinterpret_cast<const __bf16*>(kb);
    p.v = reinterpret_cast<const __bf16*>(vb);
    p.o = reinterpret_cast<__bf16*>(ob);
    p.q_row_heads = q.row_heads;
    p.kv_row_heads = k.row_heads;
    if (s.hd == 128) return launch_fwd_hd<128, false>(p, s, stream);
    return launch_fwd_hd<64, false>(p, s, stream);
  }
  p.cq = q;
  p.ck = k;
  p.cv = v;
  p.co = o;
  if (s.hd == 128) return launch_fwd_hd<128, true>(p, s, stream);
  return launch_fwd_hd<64, true>(p, s, stream);
}

hipError_t launch_attn_fwd_bf16(const AttnShape& s, const void* q, const void* k, const void* v,
                                void* o, float* lse, hipStream_t stream) {
  if (s.N == 0) return hipSuccess;
  FwdParams p = common_params(s, lse);
  p.q = static_cast<const __bf16*>(q);
  p.k = static_cast<const __bf16*>(k);
  p.v = static_cast<const __bf16*>(v);
  p.o = static_cast<__bf16*>(o);
  if (s.hd == 128) return launch_fwd_hd<128, false>(p, s, stream);
  return launch_fwd_hd<64, false>(p, s, stream);
}

}  // namespace ulysses
