// Device-side helpers shared by the gfx950 kernels of libulysses.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <tuple>
#include <utility>

namespace ulysses {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4_t;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2_t;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short i16x4_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4_t;
typedef __attribute__((__vector_size__(2 * sizeof(uint32_t)))) uint32_t u32x2_t;

#define ULY_LDS __attribute__((address_space(3)))

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// D(32x32) += A(32x16) * B(16x32), bf16 in, fp32 accumulate.
// Lane layout (measured on gfx950): A lane l holds row l%32, B lane l holds
// column l%32, each with 8 k-values; lanes l and l+32 carry the two k-halves
// (any k order works as long as A and B agree).  Accumulator element i of
// lane l is D[8*(i/4) + 4*(l/32) + i%4][l%32].
__device__ __forceinline__ f32x16_t mfma32(bf16x8_t a, bf16x8_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Transposing LDS read of four 16-bit values (ds_read_b64_tr_b16).  Within
// each group of 16 lanes, lane u supplies the address of 4 consecutive
// values (a row fragment); lane l of the group receives value (l % 4) of the
// fragments loaded by lanes 4*j + l/4, for j = 0..3.
__device__ __forceinline__ bf16x4_t lds_read_tr16(const void* p) {
  i16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((ULY_LDS i16x4_t*)(p));
  return __builtin_bit_cast(bf16x4_t, v);
}

// Lanes l and l^32 exchange values.
__device__ __forceinline__ float wave_shfl_xor32(float x) {
  return __shfl_xor(x, 32, 64);
}

// Lanes l and l^32 exchange values through v_permlane32_swap (a VALU
// operation, unlike the LDS-routed shuffle above): with both operands x, the
// swap leaves x of lanes 0..31 in both halves of one result and x of lanes
// 32..63 in both halves of the other.
__device__ __forceinline__ float wave_xor32_f(float x) {
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  const uint32_t lo_half = r[0], hi_half = r[1];   // x of lanes 0..31 and of 32..63
  const bool upper = (__lane_id() & 32) != 0;
  return __builtin_bit_cast(float, upper ? lo_half : hi_half);
}

// Byte offset of 16-byte chunk `ch` of row `row` in an LDS tile of rows of
// kChunks chunks.  The chunk index is XORed with a per-row value f(row) that
// takes all 16 values over any 16 consecutive rows (so 16 lanes reading one
// chunk column of 16 rows hit 16 different bank groups) and, over any 4
// consecutive rows starting at a multiple of 4, differs in its upper two bits
// (so the transposing reads, which take 4 rows x 4 chunks per 16 or 32
// lanes, also hit distinct bank groups).  For 8-chunk rows the same holds
// with 8 values.
template <int kChunks>
__device__ __forceinline__ int swz_f(int row) {
  if constexpr (kChunks == 16)
    return ((row & 3) << 2) | ((row >> 2) & 3);
  else
    return ((row & 1) << 2) | ((row >> 1) & 3);
}
template <int kChunks, int kRowBytes>
__device__ __forceinline__ int swz(int row, int ch) {
  return row * kRowBytes + ((ch ^ swz_f<kChunks>(row)) << 4);
}

// Direct global-to-LDS copy of 16 bytes per lane (global_load_lds_dwordx4):
// lane l's 16 bytes from `src` land at lds_dst + 16 l, where lds_dst must be
// the same for the whole wave.  Completion is tracked by the vector memory
// counter only, so the reader waits with wait_vmem() before a barrier.
__device__ __forceinline__ void load_lds16(const void* src, void* lds_dst) {
  __builtin_amdgcn_global_load_lds(src, (ULY_LDS void*)lds_dst, 16, 0, 0);
}
__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// The same copy issued from inline assembly, so the compiler does not treat
// it as a pending write to all of LDS (it would otherwise wait for it before
// every later LDS read); the caller orders it with wait_vmem / wait_vmem_n
// and a barrier.  lds_dst must be wave-uniform; M0 carries it.  The
// compiler's hazard checks do not look inside inline assembly, so the block
// starts with the 5 wait states that a vector memory instruction needs after
// a VALU write (v_readfirstlane) of an SGPR it reads, and that also cover the
// M0 write before an LDS-DMA load.
__device__ __forceinline__ void copy_lds16_async(const void* src, void* lds_dst) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)((ULY_LDS char*)(lds_dst)));
  asm volatile("s_nop 4\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "{m0}"(m0) : "memory");
}

// The same with a wave-uniform 64-bit base in scalar registers and a 32-bit
// per-lane byte offset (the saddr form of the instruction).
__device__ __forceinline__ void copy_lds16_async_sbase(const void* base, uint32_t offset,
                                                       void* lds_dst) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)((ULY_LDS char*)(lds_dst)));
  // readfirstlane yields a signed int: widen through uint32_t, never directly.
  const uint64_t b = (uint64_t)(uintptr_t)base;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)b);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(b >> 32));
  const uint64_t sb = ((uint64_t)hi << 32) | (uint64_t)lo;
  asm volatile("s_nop 4\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(offset), "s"(sb), "{m0}"(m0)
               : "memory");
}

// The 4-byte form (global_load_lds_dword): lane l's 4 bytes from base +
// offset land at lds_dst + 4 l, so one wave moves 256 contiguous LDS bytes.
__device__ __forceinline__ void copy_lds4_async_sbase(const void* base, uint32_t offset,
                                                      void* lds_dst) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)((ULY_LDS char*)(lds_dst)));
  const uint64_t b = (uint64_t)(uintptr_t)base;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)b);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(b >> 32));
  const uint64_t sb = ((uint64_t)hi << 32) | (uint64_t)lo;
  asm volatile("s_nop 4\n\tglobal_load_lds_dword %0, %1" ::"v"(offset), "s"(sb), "{m0}"(m0)
               : "memory");
}

// Waits until at most N vector-memory operations of this wave are pending
// (they complete in issue order).
template <int N>
__device__ __forceinline__ void wait_vmem_n() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Workgroup barrier for kernels that order their own global-to-LDS copies:
// waits for this wave's LDS reads, then s_barrier, with no release fence
// over vector memory (which would also wait for copies still in flight).
__device__ __forceinline__ void block_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// A operand of v_mfma_f32_32x32x16_bf16 (rows = head dim, k = 16 sequence
// positions from row0) read transposed, with ds_read_b64_tr_b16, from a
// row-major swizzled LDS tile: lane l gets column d = 32*db + l%32 at the 8
// sequence rows that match the accumulator layout of the other operand.  The
// swizzle depends on the low four row bits only, so for row0 a multiple of 16
// the address is tile + row0 * kRowBytes + a per-lane offset for each (8-row
// half, db), computed once.  db0 shifts the column blocks read to db0 ..
// db0 + kDB - 1 (db stays a compile-time index into off).  kNaturalK: the 8
// rows of lane l are instead 8 (l / 32) .. + 7 in order, the k order of a
// plain 16-byte read of a k-major operand.
template <int kChunks, int kRowBytes, int kDB, bool kNaturalK = false>
struct TrReader {
  int off[2][kDB];
  __device__ __forceinline__ explicit TrReader(int lane, int db0 = 0) {
    const int grp = lane >> 4;
    const int u = lane & 15;
#pragma unroll
    for (int jh = 0; jh < 2; ++jh)
#pragma unroll
      for (int db = 0; db < kDB; ++db) {
        const int row = kNaturalK ? 8 * (grp >> 1) + 4 * jh + (u >> 2)
                                  : 8 * jh + 4 * (grp >> 1) + (u >> 2);
        const int col = (db0 + db) * 32 + 16 * (grp & 1) + 4 * (u & 3);
        off[jh][db] = swz<kChunks, kRowBytes>(row, col >> 3) + ((col >> 2) & 1) * 8;
      }
  }
  __device__ __forceinline__ bf16x8_t load(const char* tile, int row0, int db) const {
    const char* base = tile + row0 * kRowBytes;
    const bf16x4_t a = lds_read_tr16(base + off[0][db]);
    const bf16x4_t b = lds_read_tr16(base + off[1][db]);
    return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
  }
};

// n / f.d for the divisor of make_fastdiv (launch.h), exact for every
// 32-bit n.
template <typename FD>
__device__ __forceinline__ uint32_t fast_div(uint32_t n, FD f) {
  const uint32_t t = __umulhi(n, f.m);
  return (uint32_t)(((uint64_t)t + n) >> f.l);
}

// Addresses in an operand held as sequence chunks (SeqChunks in launch.h):
// the element offset of row i (batch b, head h of the rank's slice) from the
// start of its chunk, whose index goes to *chunk ...
template <typename SC>
__device__ __forceinline__ int64_t chunk_row_offset(const SC& c, uint32_t i, int bs, int b, int h,
                                                    int hd, uint32_t* chunk) {
  const uint32_t ci = i / (uint32_t)c.n;
  *chunk = ci;
  return (((int64_t)(i - ci * (uint32_t)c.n) * bs + b) * c.row_heads + c.head0 + h) * hd;
}
// ... the address of that row ...
template <typename SC>
__device__ __forceinline__ __bf16* chunk_row(const SC& c, uint32_t i, int bs, int b, int h, int hd) {
  uint32_t ci;
  const int64_t off = chunk_row_offset(c, i, bs, b, h, hd, &ci);
  return reinterpret_cast<__bf16*>(c.chunk[ci]) + off;
}
// ... and the byte address of the first row of 64-row tile `tile` (tiles
// never straddle chunks).
template <typename SC>
__device__ __forceinline__ int64_t chunk_tile_base(const SC& c, uint32_t tile, int bs, int b, int h,
                                                   int hd) {
  const uint32_t ci = fast_div(tile, c.tiles_per_chunk);
  const int64_t s0 = (int64_t)(tile - ci * c.tiles_per_chunk.d) * 64;
  return (int64_t)c.chunk[ci] + ((s0 * bs + b) * c.row_heads + c.head0 + h) * hd * 2;
}

// A value the whole wave agrees on, moved to scalar registers so that
// branches on it stay scalar branches.
__device__ __forceinline__ int64_t wave_uniform(int64_t x) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)x);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)x >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

__device__ __forceinline__ bool wave_any(bool pred) {
  return __any(pred);
}

// Start offset of the document holding position i: the largest cu[d] <= i
// over d in [0, n_docs).  Values read from cu are clamped to [0, i].
__device__ __forceinline__ int64_t doc_start_of(const int32_t* cu, int n_docs, int64_t i) {
  if (cu == nullptr) return 0;
  int lo = 0, hi = n_docs - 1;  // invariant: answer index in [lo, hi]
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if ((int64_t)cu[mid] <= i) lo = mid; else hi = mid - 1;
  }
  int64_t s = cu[lo];
  if (s < 0) s = 0;
  if (s > i) s = i;
  return s;
}

// End offset (exclusive) of the document holding position i, clamped to
// [i + 1, N].
__device__ __forceinline__ int64_t doc_end_of(const int32_t* cu, int n_docs, int64_t i, int64_t N) {
  if (cu == nullptr) return N;
  int lo = 0, hi = n_docs - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if ((int64_t)cu[mid] <= i) lo = mid; else hi = mid - 1;
  }
  int64_t e = cu[lo + 1];
  if (e > N) e = N;
  if (e < i + 1) e = i + 1;
  return e;
}

// Dispatch order of the position blocks of a packed-document share, heaviest
// first.  Under the causal mask within documents, the work of a block of B
// query positions grows with its index inside its document, and that of a
// block of B keys with its distance to the document's end, so launching by
// position (right for one document) interleaves heavy and light blocks and
// leaves a long tail.  A block of query positions [kb B, kb B + B) belongs
// to the document holding its first position and its sort key is its index
// from the block holding the document's start (kKeyBlocks false); a block of
// keys belongs to the document holding its last key (whose end bounds the
// queries it sees) and its key is its distance to that document's last
// block (kKeyBlocks true).  Rank t of the order
// (largest key first, documents in order within a key) is found by a binary
// search over the key j of C(j), the number of blocks whose key is at least
// j, then a ballot over the documents with a block of that key.  The whole
// wave computes it, 64 documents per pass; the result is wave-uniform.  It
// returns -1, and the caller keeps its default order, without cu, with more
// than kOrderDocs documents, or when cu's contents (clamped to [0, N]) do not
// cover rank t.
constexpr int kOrderDocs = 256;

template <bool kKeyBlocks>
__device__ __forceinline__ int64_t doc_sorted_block(int64_t t, int64_t nblocks, int B,
                                                      const int32_t* cu, int n_docs,
                                                      int64_t N) {
  constexpr int kPer = kOrderDocs / 64;
  if (cu == nullptr || n_docs < 1 || n_docs > kOrderDocs) return -1;
  const int lane = threadIdx.x & 63;
  // Owned blocks [f, l] and start block a of this lane's documents.
  int f[kPer], l[kPer], a[kPer];
  int jmax = -1;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int d = lane + 64 * i;
    f[i] = 1;
    l[i] = 0;
    a[i] = 0;
    if (d < n_docs) {
      int64_t s = cu[d], e = cu[d + 1];
      s = s < 0 ? 0 : (s > N ? N : s);
      e = e < s ? s : (e > N ? N : e);
      if (kKeyBlocks) {   // blocks whose last key lies in [s, e)
        f[i] = (int)(s / B);
        l[i] = e <= s ? f[i] - 1 : (e >= N ? (int)(nblocks - 1) : (int)(e / B) - 1);
      } else {            // blocks whose first position lies in [s, e)
        f[i] = (int)((s + B - 1) / B);
        l[i] = (int)((e + B - 1) / B) - 1;
        a[i] = (int)(s / B);
      }
      if (l[i] > nblocks - 1) l[i] = (int)(nblocks - 1);
      if (l[i] >= f[i]) {
        const int top = kKeyBlocks ? l[i] - f[i] : l[i] - a[i];
        jmax = top > jmax ? top : jmax;
      }
    }
  }
  for (int off = 32; off > 0; off >>= 1) {
    const int o = __shfl_xor(jmax, off, 64);
    jmax = o > jmax ? o : jmax;
  }
  // C(j), summed over the wave.
  auto count_ge = [&](int j) __attribute__((always_inline)) {
    int c = 0;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int lo = kKeyBlocks ? f[i] : (f[i] > a[i] + j ? f[i] : a[i] + j);
      const int hi = kKeyBlocks ? l[i] - j : l[i];
      c += hi >= lo ? hi - lo + 1 : 0;
    }
    for (int off = 32; off > 0; off >>= 1) c += __shfl_xor(c, off, 64);
    return c;
  };
  if (jmax < 0 || count_ge(0) <= t) return -1;
  int lo = 0, hi = jmax;   // the largest j with C(j) > t lies in [lo, hi]
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (count_ge(mid) > t) lo = mid; else hi = mid - 1;
  }
  int r = (int)t - count_ge(lo + 1);   // rank among the blocks of key lo
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int kb = kKeyBlocks ? l[i] - lo : a[i] + lo;
    const bool member = l[i] >= f[i] && kb >= f[i] && kb <= l[i];
    const uint64_t m = __ballot(member);
    const int cnt = __popcll(m);
    if (r < cnt) {
      const int below = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                                   __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
      const uint64_t sel = __ballot(member && below == r);
      return wave_uniform(__shfl(kb, __ffsll((unsigned long long)sel) - 1, 64));
    }
    r -= cnt;
  }
  return -1;
}

template <typename Tuple, size_t... I>
inline void fill_argv(Tuple& t, void** argv, std::index_sequence<I...>) {
  ((argv[I] = static_cast<void*>(&std::get<I>(t))), ...);
}

// Launches `kernel` on `stream` and returns the launch status itself (not the
// thread's sticky last-error state, which other HIP users may have left set).
template <typename... KArgs, typename... Args>
inline hipError_t launch_kernel(void (*kernel)(KArgs...), dim3 grid, dim3 block, size_t shmem,
                                hipStream_t stream, Args... args) {
  static_assert(sizeof...(KArgs) == sizeof...(Args), "kernel argument count");
  struct Pack {
    std::tuple<KArgs...> v;
  } pack{std::tuple<KArgs...>(args...)};
  void* argv[sizeof...(KArgs) + 1];
  fill_argv(pack.v, argv, std::index_sequence_for<KArgs...>{});
  return hipLaunchKernel(reinterpret_cast<const void*>(kernel), grid, block, argv, shmem, stream);
}

}  // namespace ulysses
