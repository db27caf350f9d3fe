// Dense bf16 products of the sequence-tiled language-model loss and SwiGLU
// MLP (the integration guide's TiledFusedLogitsLoss and TiledMLP, sections
// on tiled loss and MLP computation) on gfx950 matrix cores.
//
// One kernel computes
//   C[x][y] (+)= sum_k X(x, k) Y(y, k)        (fp32 accumulation)
// where each operand is stored either with k contiguous ("k-major": element
// (r, k) at p[r*ld + k]) or with its rows contiguous ("row-major over k":
// element (r, k) at p[k*ld + r]); with the two layouts of X and Y every
// product of the loss (Z = H W^T, dH = G W, dW = G^T H) and of the MLP (the
// gate, up and down projections and their gradients) is one launch, with no
// transposed copy of any operand.
//
// Design for CDNA4:
//  * A workgroup of 8 waves (two per SIMD) owns a 256 x 256 tile of C; wave
//    w owns X rows 128 (w % 2) .. + 128 and Y rows 64 (w / 2) .. + 64, as
//    4 x 2 tiles of v_mfma_f32_32x32x16_bf16: 128 accumulators, 8
//    independent products per 16-deep k step fed by 6 fragment reads.  Two
//    waves per SIMD keep its matrix pipe busy (one wave alone, measured,
//    issues at most ~870 TFLOP/s here, two ~1300), and the 256 x 256 tile
//    keeps 128 flop per byte moved from L2 (a 256 x 128 tile on two
//    workgroups per CU, measured, was bound by that traffic).  The Y fragment
//    is the MFMA's A operand and the X fragment its B operand, so every
//    lane's accumulators hold one row x of C: the loss's row statistics need
//    no cross-lane shuffles beyond one lane swap and one LDS merge.
//  * K advances 32 at a time through four LDS stages (4 x 32 KiB; the X
//    tiles of all stages first, then the Y tiles).  Operand tiles reach LDS
//    by direct global-to-LDS copies (no registers spent on staging), issued
//    three steps ahead of their products so that a fetch from L2 or the
//    Infinity Cache has one to two steps to land (measured: the copies, not
//    the LDS reads, are what keeps the matrix pipe from its peak).  The step
//    loop is unrolled by the stage count, so every LDS address is a
//    per-lane register plus a constant offset (X tiles within 0..64 KiB, Y
//    tiles within 64..128 KiB) and the 12 to 24 fragment reads of a step
//    cost no address arithmetic: ~10% faster with a row-major operand,
//    whose transposing reads are twice as many; a k-major tile
//    is stored as 256 rows of 4 16-byte chunks, the chunk index XORed with
//    bits 2-3 of the row, a row-major one as two halves of 32 k-rows x 16
//    chunks swizzled as in device_common.h (swz), so both the 16-byte row
//    reads and the transposing reads (ds_read_b64_tr_b16, for row-major
//    operands) of 16 lanes fall in 16 different bank groups.
//  * The transposing read (row-major operands) is addressed so that lane l
//    gets k = 8h .. 8h+7 (h = l / 32) in order, the order of one 16-byte
//    read of a k-major row, so both MFMA operands agree on which k each
//    element carries whatever the layouts.
//  * Edges: source rows and chunks are clamped into the operands' valid
//    memory, values with k >= K are zeroed in the last step, and stores are
//    bounds-checked, so any shape works (only the step loop is full speed).
//  * Workgroups are remapped so that each XCD works on a contiguous run of
//    tiles ordered in groups of four tile rows (x-tiles 0.. of y-tiles
//    4g..4g+3 together): the 32 tiles an XCD runs at once form a 4 x 8
//    block that reads 12 operand slabs per k step instead of the 18 of a
//    2 x 16 row-order block, and so hit its L2 more often.
#include <math.h>

#include <type_traits>

#include "device_common.h"
#include "launch.h"

namespace ulysses {
namespace {

constexpr int kBX = 256, kBY = 256, kBK = 32;
constexpr int kStages = 4;                          // copies run kStages - 1 steps ahead
constexpr int kTileBytes = 256 * kBK * 2;           // 16 KiB per operand and stage
constexpr int kStageBytes = 2 * kTileBytes;         // one X and one Y tile
constexpr int kSmem = kStages * kStageBytes;        // 128 KiB
constexpr int kGroupY = 4;                          // y-tiles per group of the tile order
constexpr int kWaves = 8;
constexpr int kCopies = kTileBytes / 1024 / kWaves; // wave copies per operand and step

// Chunk swizzle of a k-major tile row (4 chunks of 16 bytes): 16 consecutive
// rows read at one chunk position land in 16 different bank groups.
__device__ __forceinline__ int swz4(int row) { return (row >> 2) & 3; }

struct GemmParams {
  const __bf16* x;
  const __bf16* y;
  int64_t ldx, ldy;          // elements between rows (k-major) or k steps (row-major)
  int nx, ny, K;
  void* c;
  int64_t ldc;
  float* stats;              // loss epilogue: [nx][tiles_y] x (max, sum exp(z - max))
  const int64_t* labels;     // loss epilogue: label of row x; C[x][label] goes to zlabel[x]
  float* zlabel;
  // Second product of a pair launch (grid z = 1): same sizes, layouts and
  // output mode, its own operands and output.
  const __bf16* x2;
  const __bf16* y2;
  void* c2;
  int tiles_x, tiles_y;
};

enum OutMode { kStoreF32 = 0, kAccumF32 = 1, kStoreBF16 = 2 };

// Zero the elements of an 8-value fragment whose k is >= K (first four at
// k_lo.., last four at k_hi..).
__device__ __forceinline__ bf16x8_t mask_k(bf16x8_t f, int k_lo, int k_hi, int K) {
  u32x4_t u = __builtin_bit_cast(u32x4_t, f);
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int k = (p < 2 ? k_lo : k_hi) + 2 * (p & 1);
    const uint32_t lo = k < K ? 0xffffu : 0u;
    const uint32_t hi = k + 1 < K ? 0xffff0000u : 0u;
    u[p] &= lo | hi;
  }
  return __builtin_bit_cast(bf16x8_t, u);
}

template <bool kXK, bool kYK, int kOut, bool kStats>
__global__ __launch_bounds__(512) void gemm_bf16_kernel(GemmParams p) {
  __shared__ __attribute__((aligned(1024))) char smem[kSmem];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // Operands and output of this product (blockIdx.z of a pair launch).
  const __bf16* const gx = blockIdx.z ? p.x2 : p.x;
  const __bf16* const gy = blockIdx.z ? p.y2 : p.y;
  void* const gc = blockIdx.z ? p.c2 : p.c;
  const int half = lane >> 5;
  const int r32 = lane & 31;
  const int wx = wave & 1;    // X rows 128 wx ..
  const int wy = wave >> 1;   // Y rows 64 wy ..

  // Workgroup -> tile.  Workgroups reach the 8 XCDs round-robin; blocks
  // b, b + 8, b + 16, ... run on one XCD, and they take consecutive tiles
  // of the grouped order (groups of kGroupY y-tiles, x-tiles outer and y
  // inner within a group), so the tiles an XCD runs at once share slabs.
  const int nb = p.tiles_x * p.tiles_y;
  const int b = blockIdx.x;
  const int per_xcd = nb / 8, rem = nb % 8;
  const int xcd = b % 8, j = b / 8;
  const int lin = (xcd < rem ? xcd * (per_xcd + 1) : rem * (per_xcd + 1) + (xcd - rem) * per_xcd) + j;
  const int gsz = kGroupY * p.tiles_x, grp = lin / gsz, in_grp = lin % gsz;
  const int rows_g = min(kGroupY, p.tiles_y - grp * kGroupY);   // last group may be short
  const int ty = grp * kGroupY + in_grp % rows_g, tx = in_grp / rows_g;
  const int x0 = tx * kBX, y0 = ty * kBY;

  const int K = p.K;
  const int nk = (K + kBK - 1) / kBK;

  // ---- direct copies ------------------------------------------------------
  // k-major tile: 256 rows x 4 chunks; wave copy c moves rows 16c .. 16c+15,
  // lane l the chunk that the swizzle places at slot l % 4 of row 16c + l/4.
  // Row-major tile: halves hh of [32 k][128 rows] x 16 chunks; wave copy c
  // moves half c / 8, k-rows 4 (c % 8) .. + 3, lane l the chunk for slot
  // l % 16 of k-row 4 (c % 8) + l / 16.  Each wave issues copies
  // kCopies w .. kCopies w + kCopies - 1 of each operand.  A copy is a
  // wave-uniform base (the tile's corner, in scalar registers) plus a 32-bit
  // lane offset whose row and chunk are clamped into the operand (rows <
  // nrows, k < K), so a tile reaching past the operand reads valid memory
  // and needs no separate code path; its extra values are zeroed (k >= K) or
  // never stored.  The swizzle depends on the row's low bits only, so the
  // chunk is fixed per lane (k-major) or per lane and c % 4 (row-major).
  // only >= 0: issue just copy `only` of this wave (to spread the copies
  // between matrix products).
  auto copy_operand = [&](auto kmajor_tag, const __bf16* base, int64_t ld, int nrows, int r0,
                          int k0, char* tile, int only) __attribute__((always_inline)) {
    constexpr bool kKM = decltype(kmajor_tag)::value;
    const char* corner = reinterpret_cast<const char*>(wave_uniform(reinterpret_cast<int64_t>(
        base + (kKM ? (int64_t)r0 * ld + k0 : (int64_t)k0 * ld + r0))));
    const uint32_t ld2 = (uint32_t)(ld * 2);
#pragma unroll
    for (int i = 0; i < kCopies; ++i) {
      if (only >= 0 && i != only) continue;
      const int c = kCopies * wave + i;
      uint32_t off;
      if constexpr (kKM) {
        const int row = 16 * c + lane / 4;              // tile row
        const int chunk = (lane % 4) ^ swz4(lane / 4);  // swz4 of row
        const int r = min(row, nrows - 1 - r0);
        const int k = min(8 * chunk, ((K + 7) / 8 - 1) * 8 - k0);   // last valid chunk
        off = (uint32_t)r * ld2 + (uint32_t)k * 2u;
      } else {
        const int krow = 4 * (c % 8) + lane / 16;
        const int chunk = (lane % 16) ^ swz_f<16>(4 * (c % 4) + lane / 16);   // swz_f<16> of krow
        const int k = min(krow, K - 1 - k0);
        const int r = min(128 * (c / 8) + 8 * chunk, ((nrows + 7) / 8 - 1) * 8 - r0);
        off = (uint32_t)k * ld2 + (uint32_t)r * 2u;
      }
      copy_lds16_async_sbase(corner, off, tile + c * 1024);
    }
  };
  // Copies of step kt (clamped to the last step: such a copy refills a stage
  // nobody reads again, and keeps every step's count of pending copies the
  // same) into stage kt % kStages.
  auto xtile = [&](int st) __attribute__((always_inline)) { return smem + st * kTileBytes; };
  auto ytile = [&](int st) __attribute__((always_inline)) {
    return smem + (kStages + st) * kTileBytes;
  };
  auto copy_stage = [&](int kt) __attribute__((always_inline)) {
    const int kc = kt < nk ? kt : nk - 1;
    copy_operand(std::integral_constant<bool, kXK>{}, gx, p.ldx, p.nx, x0, kc * kBK,
                 xtile(kt % kStages), -1);
    copy_operand(std::integral_constant<bool, kYK>{}, gy, p.ldy, p.ny, y0, kc * kBK,
                 ytile(kt % kStages), -1);
  };

  // ---- fragment reads -----------------------------------------------------
  // Fragment of 32 operand rows starting at tile row `sub32 * 32`, k step
  // ks.  Row-major tiles are read through a transposing reader whose column
  // block (32 rows of the half) is a compile-time index: X rows 128 wx + 32 i
  // are block i of half wx, Y rows 64 wy + 32 jy block 2 (wy % 2) + jy of
  // half wy / 2.
  const TrReader<16, 256, 4, true> tr_x(lane);
  const TrReader<16, 256, 2, true> tr_y(lane, 2 * (wy & 1));
  auto read_kmajor = [&](const char* tile, int sub32, int ks) __attribute__((always_inline))
      -> bf16x8_t {
    const int row = 32 * sub32 + r32;
    const char* rb = tile + row * (kBK * 2);
    return *reinterpret_cast<const bf16x8_t*>(rb + (((2 * ks + half) ^ swz4(row)) << 4));
  };

  f32x16_t acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int jy = 0; jy < 2; ++jy) acc[i][jy] = f32x16_t{};

  // Fragments of 16-deep k step ks of stage `stage` into slot bsel.
  bf16x8_t xf[2][4], yf[2][2];
  auto load = [&](int stage, int ks, int bsel) __attribute__((always_inline)) {
    const char* tx_ = xtile(stage);
    const char* ty_ = ytile(stage);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if constexpr (kXK)
        xf[bsel][i] = read_kmajor(tx_, 4 * wx + i, ks);
      else
        xf[bsel][i] = tr_x.load(tx_ + wx * (kTileBytes / 2), 16 * ks, i);
    }
#pragma unroll
    for (int jy = 0; jy < 2; ++jy) {
      if constexpr (kYK)
        yf[bsel][jy] = read_kmajor(ty_, 2 * wy + jy, ks);
      else
        yf[bsel][jy] = tr_y.load(ty_ + (wy >> 1) * (kTileBytes / 2), 16 * ks, jy);
    }
  };
  // The 8 products of the fragments in slot bsel (k step starting at k16);
  // after the second and the fourth pair of products one copy of `copy_tag`
  // (0: X copies, 1: Y copies of step kc into `copy_tile`; 2: none) goes
  // out, so the copies' issue overlaps the matrix pipe.
  auto products = [&](int bsel, auto mask_tag, int k16, auto copy_tag, int kc, char* copy_tile)
      __attribute__((always_inline)) {
    constexpr bool kMask = decltype(mask_tag)::value;
    constexpr int kCopy = decltype(copy_tag)::value;
    if constexpr (kMask) {
      const int k_lo = k16 + 8 * half, k_hi = k_lo + 4;   // the fragment's two k quads
#pragma unroll
      for (int i = 0; i < 4; ++i) xf[bsel][i] = mask_k(xf[bsel][i], k_lo, k_hi, K);
#pragma unroll
      for (int jy = 0; jy < 2; ++jy) yf[bsel][jy] = mask_k(yf[bsel][jy], k_lo, k_hi, K);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int jy = 0; jy < 2; ++jy) acc[i][jy] = mfma32(yf[bsel][jy], xf[bsel][i], acc[i][jy]);
      if (i & 1) {
        if constexpr (kCopy == 0)
          copy_operand(std::integral_constant<bool, kXK>{}, gx, p.ldx, p.nx, x0, kc * kBK,
                       copy_tile, i >> 1);
        else if constexpr (kCopy == 1)
          copy_operand(std::integral_constant<bool, kYK>{}, gy, p.ldy, p.ny, y0, kc * kBK,
                       copy_tile, i >> 1);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  static_assert(kBK == 32 && kCopies == 2, "two k steps per stage, two copies per operand");

  // ---- main loop ----------------------------------------------------------
  // Step t reads stage t % 4.  Its copies went out during step t - 3; the
  // barrier after step t - 2 published them (each wave first waits until
  // only the copies of the step after are pending), so during step t - 1
  // every wave can already read the first fragments of step t: the barrier
  // after a step does not wait for fragment reads in flight, and no matrix
  // product waits for a barrier-to-read round trip.  The copies of step t + 3
  // go to the stage step t - 1 read, whose fragments every wave consumed
  // before that barrier.  Copies past the last step are clamped to it (they
  // refill a stage nobody reads again; each step keeps the same count of
  // pending copies).  The last step is peeled off and always zeroes k >= K
  // (a no-op when K is a multiple of 32), so the loop has one code path.
  constexpr int kStepCopies = 2 * kCopies;   // per wave and step
#pragma unroll
  for (int t = 0; t < kStages - 1; ++t) copy_stage(t);
  wait_vmem_n<(kStages - 3) * kStepCopies>();   // steps 0 and 1 landed (2 may be pending)
  block_barrier();
  load(0, 0, 0);
  // Step kt, reading stage st = kt % kStages.
  auto step = [&](int kt, int st) __attribute__((always_inline)) {
    const int cs = kt + kStages - 1;                      // step whose copies go out now
    const int kc = cs < nk ? cs : nk - 1;
    const int cst = (st + kStages - 1) % kStages;         // its stage
    load(st, 1, 1);
    products(0, std::false_type{}, kt * kBK, std::integral_constant<int, 0>{}, kc, xtile(cst));
    load((st + 1) % kStages, 0, 0);
    products(1, std::false_type{}, kt * kBK + 16, std::integral_constant<int, 1>{}, kc,
             ytile(cst));
    wait_vmem_n<(kStages - 3) * kStepCopies>();   // the copies of step kt + 2 landed
    asm volatile("s_barrier" ::: "memory");
  };
  // Whole rounds of kStages steps with the stage a constant, then the rest.
  int kt0 = 0;
  for (; kt0 + kStages < nk; kt0 += kStages) {
#pragma unroll
    for (int u = 0; u < kStages; ++u) step(kt0 + u, u);
  }
  for (int kt = kt0; kt + 1 < nk; ++kt) step(kt, kt % kStages);
  {
    const int kt = nk - 1;
    load(kt % kStages, 1, 1);
    products(0, std::true_type{}, kt * kBK, std::integral_constant<int, 2>{}, 0, smem);
    products(1, std::true_type{}, kt * kBK + 16, std::integral_constant<int, 2>{}, 0, smem);
  }
  wait_vmem();       // no copy may still be writing LDS ...
  block_barrier();   // ... nor any wave reading it when the epilogue reuses it

  // ---- epilogue -----------------------------------------------------------
  // Lane l holds C[x][y] for x = x0 + 128 wx + 32 i + l % 32 and
  // y = y0 + 64 wy + 32 jy + 8 q + 4 half + e (element 4 q + e of acc[i][jy]).
  if constexpr (kStats) {
    // Loss epilogue.  Per row x of the tile: the logit of x's label when it
    // falls in this tile (written to zlabel[x], fp32), the tile's row max m
    // over its columns < ny, and in place of C the values exp(C - m) (in
    // [0, 1], stored as bf16 below: a bf16 of a value in [0, 1] keeps 8
    // significant bits, where a bf16 logit of magnitude 16 would keep an
    // absolute error of 2^-4 in the exponent) with their sum l.  Partial
    // maxima and sums of the four waves that share rows meet in LDS.
    float* pmax = reinterpret_cast<float*>(smem);   // [4 wy][256 x]
    float* psum = pmax + 4 * 256;                   // [4 wy][256 x]
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int xr = 128 * wx + 32 * i + r32;
      const int x = x0 + xr;
      const int64_t lab = x < p.nx ? p.labels[x] : -1;
      float m = -INFINITY, zl = 0.f;
      bool found = false;
#pragma unroll
      for (int jy = 0; jy < 2; ++jy)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int y = y0 + 64 * wy + 32 * jy + 8 * (e / 4) + 4 * half + (e % 4);
          if (y < p.ny) m = fmaxf(m, acc[i][jy][e]);
          if (y == lab) {
            zl = acc[i][jy][e];
            found = true;
          }
        }
      if (found) p.zlabel[x] = zl;
      m = fmaxf(m, wave_xor32_f(m));
      if (half == 0) pmax[wy * 256 + xr] = m;
      __builtin_amdgcn_sched_barrier(0);   // one 32-row block's accumulators live at a time
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int xr = 128 * wx + 32 * i + r32;
      const float m = fmaxf(fmaxf(pmax[xr], pmax[256 + xr]), fmaxf(pmax[512 + xr], pmax[768 + xr]));
      const float mb = m == -INFINITY ? 0.f : m * kLog2e;   // rows past nx: every column < ny
      float l = 0.f;
#pragma unroll
      for (int jy = 0; jy < 2; ++jy)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int y = y0 + 64 * wy + 32 * jy + 8 * (e / 4) + 4 * half + (e % 4);
          const float v = y < p.ny ? __builtin_amdgcn_exp2f(fmaf(acc[i][jy][e], kLog2e, -mb)) : 0.f;
          acc[i][jy][e] = v;
          l += v;
        }
      l += wave_xor32_f(l);
      if (half == 0) psum[wy * 256 + xr] = l;
      __builtin_amdgcn_sched_barrier(0);
    }
    __syncthreads();
    if (tid < 256) {
      const int x = x0 + tid;
      if (x < p.nx) {
        float* sp = p.stats + ((int64_t)x * p.tiles_y + ty) * 2;
        sp[0] = fmaxf(fmaxf(pmax[tid], pmax[256 + tid]), fmaxf(pmax[512 + tid], pmax[768 + tid]));
        sp[1] = (psum[tid] + psum[256 + tid]) + (psum[512 + tid] + psum[768 + tid]);
      }
    }
  }
  if constexpr (kOut == kAccumF32) {
    // The wave's whole 128 x 64 block inside C: the old values of row block
    // i + 1 are loaded before block i is stored back, so each load's latency
    // overlaps the previous block's adds and stores.
    if (x0 + 128 * wx + 128 <= p.nx && y0 + 64 * wy + 64 <= p.ny) {
      float* cb = static_cast<float*>(gc) + (int64_t)(x0 + 128 * wx + r32) * p.ldc + y0 +
                  64 * wy + 4 * half;
      f32x4_t old[2][2][4];   // [row block % 2][jy][q]
      auto load_old = [&](int i) __attribute__((always_inline)) {
#pragma unroll
        for (int jy = 0; jy < 2; ++jy)
#pragma unroll
          for (int q = 0; q < 4; ++q)
            old[i & 1][jy][q] = *reinterpret_cast<const f32x4_t*>(cb + (int64_t)32 * i * p.ldc +
                                                                  32 * jy + 8 * q);
      };
      load_old(0);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (i < 3) load_old(i + 1);
#pragma unroll
        for (int jy = 0; jy < 2; ++jy)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const f32x4_t v = {acc[i][jy][4 * q], acc[i][jy][4 * q + 1], acc[i][jy][4 * q + 2],
                               acc[i][jy][4 * q + 3]};
            *reinterpret_cast<f32x4_t*>(cb + (int64_t)32 * i * p.ldc + 32 * jy + 8 * q) =
                old[i & 1][jy][q] + v;
          }
      }
      return;
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    __builtin_amdgcn_sched_barrier(0);   // one 32-row block's accumulators live at a time
    const int x = x0 + 128 * wx + 32 * i + r32;
    if (x >= p.nx) continue;
#pragma unroll
    for (int jy = 0; jy < 2; ++jy)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int y = y0 + 64 * wy + 32 * jy + 8 * q + 4 * half;
        const f32x4_t v = {acc[i][jy][4 * q], acc[i][jy][4 * q + 1], acc[i][jy][4 * q + 2],
                           acc[i][jy][4 * q + 3]};
        if constexpr (kOut == kStoreBF16) {
          __bf16* cp = static_cast<__bf16*>(gc) + (int64_t)x * p.ldc + y;
          if (y + 3 < p.ny) {
            bf16x4_t o;
#pragma unroll
            for (int e = 0; e < 4; ++e) o[e] = (__bf16)v[e];
            *reinterpret_cast<bf16x4_t*>(cp) = o;
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (y + e < p.ny) cp[e] = (__bf16)v[e];
          }
        } else {
          float* cp = static_cast<float*>(gc) + (int64_t)x * p.ldc + y;
          if (y + 3 < p.ny) {
            if constexpr (kOut == kAccumF32) {
              const f32x4_t old = *reinterpret_cast<const f32x4_t*>(cp);
              *reinterpret_cast<f32x4_t*>(cp) = old + v;
            } else {
              *reinterpret_cast<f32x4_t*>(cp) = v;
            }
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (y + e < p.ny) cp[e] = (kOut == kAccumF32 ? cp[e] : 0.0f) + v[e];
          }
        }
      }
  }
}

template <bool kXK, bool kYK>
hipError_t launch_layout(const GemmParams& p, int out, bool stats, int products,
                         hipStream_t stream) {
  const dim3 grid((uint32_t)(p.tiles_x * p.tiles_y), 1, (uint32_t)products), block(512);
  if (stats) {
    if constexpr (kXK && kYK)
      return launch_kernel(gemm_bf16_kernel<true, true, kStoreBF16, true>, grid, block, 0, stream, p);
    return hipErrorInvalidValue;
  }
  switch (out) {
    case kStoreF32:
      return launch_kernel(gemm_bf16_kernel<kXK, kYK, kStoreF32, false>, grid, block, 0, stream, p);
    case kAccumF32:
      return launch_kernel(gemm_bf16_kernel<kXK, kYK, kAccumF32, false>, grid, block, 0, stream, p);
    case kStoreBF16:
      return launch_kernel(gemm_bf16_kernel<kXK, kYK, kStoreBF16, false>, grid, block, 0, stream, p);
  }
  return hipErrorInvalidValue;
}

}  // namespace

int gemm_tiles_y(int64_t ny) { return (int)((ny + kBY - 1) / kBY); }

namespace {

GemmParams make_params(const GemmOp& op) {
  GemmParams p{};
  p.x = static_cast<const __bf16*>(op.x.p);
  p.y = static_cast<const __bf16*>(op.y.p);
  p.ldx = op.x.ld;
  p.ldy = op.y.ld;
  p.nx = (int)op.nx;
  p.ny = (int)op.ny;
  p.K = (int)op.K;
  p.c = op.c;
  p.ldc = op.ldc;
  p.stats = op.stats;
  p.labels = op.labels;
  p.zlabel = op.label_logit;
  p.tiles_x = (int)((op.nx + kBX - 1) / kBX);
  p.tiles_y = gemm_tiles_y(op.ny);
  return p;
}

hipError_t launch_params(const GemmOp& op, const GemmParams& p, int products, hipStream_t stream) {
  const int out = op.accumulate ? kAccumF32 : (op.c_bf16 ? kStoreBF16 : kStoreF32);
  if (op.stats != nullptr && (out != kStoreBF16 || op.labels == nullptr || op.label_logit == nullptr))
    return hipErrorInvalidValue;
  const bool st = op.stats != nullptr;
  if (op.x.kmajor && op.y.kmajor) return launch_layout<true, true>(p, out, st, products, stream);
  if (op.x.kmajor && !op.y.kmajor) return launch_layout<true, false>(p, out, false, products, stream);
  if (!op.x.kmajor && !op.y.kmajor) return launch_layout<false, false>(p, out, false, products, stream);
  return launch_layout<false, true>(p, out, false, products, stream);
}

}  // namespace

hipError_t launch_gemm(const GemmOp& op, hipStream_t stream) {
  if (op.nx <= 0 || op.ny <= 0) return hipSuccess;
  if (op.K <= 0) return hipErrorInvalidValue;   // callers never ask for an empty sum
  return launch_params(op, make_params(op), 1, stream);
}

hipError_t launch_gemm_pair(const GemmOp& a, const GemmOp& b, hipStream_t stream) {
  const bool same = a.nx == b.nx && a.ny == b.ny && a.K == b.K && a.x.ld == b.x.ld &&
                    a.y.ld == b.y.ld && a.x.kmajor == b.x.kmajor && a.y.kmajor == b.y.kmajor &&
                    a.ldc == b.ldc && a.c_bf16 == b.c_bf16 && a.accumulate == b.accumulate &&
                    a.stats == nullptr && b.stats == nullptr && a.c != b.c;
  if (!same) {
    const hipError_t e = launch_gemm(a, stream);
    return e != hipSuccess ? e : launch_gemm(b, stream);
  }
  if (a.nx <= 0 || a.ny <= 0) return hipSuccess;
  if (a.K <= 0) return hipErrorInvalidValue;
  GemmParams p = make_params(a);
  p.x2 = static_cast<const __bf16*>(b.x.p);
  p.y2 = static_cast<const __bf16*>(b.y.p);
  p.c2 = b.c;
  return launch_params(a, p, 2, stream);
}

}  // namespace ulysses
