// streamkl_device.h -- gfx950 building blocks shared by the StreamKL kernels.
//
// Matrix-core conventions (CDNA3/CDNA4 32x32 MFMA, wave64):
//   * A operand (M x K): lane L supplies row m = L % 32 and a run of K values
//     picked by its half h = L / 32; B operand (K x N): lane L supplies column
//     n = L % 32 and the same run of K values.
//   * C/D (32 x 32 fp32, 16 registers): lane L holds column n = L % 32 and rows
//     m(r, h) = (r / 4) * 8 + 4 h + (r % 4), r = 0..15.
// Scores are produced with the "stationary" operand (the tensor whose rows the
// workgroup owns: queries in the forward and dQ kernels, keys in the dK kernel)
// as the B operand, so that each lane owns one stationary row and 16 streamed
// rows of every 32 x 32 score block.  Row reductions are then in-lane, and the
// score block feeds the gradient product directly as a B operand.
//
// Element types: bf16 uses v_mfma_f32_32x32x16_bf16 (8 values per lane per
// product); fp32 uses v_mfma_f32_32x32x2_f32 (1 value per lane per product).
// A lane always holds half of a row (d/2 elements) as 16-byte chunks.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace streamkl {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Geometry of one row of d elements stored as 16-byte chunks.
template <bool BF16, int D>
struct RowGeom {
  static constexpr int kElemBytes = BF16 ? 2 : 4;
  static constexpr int kRowBytes = D * kElemBytes;
  static constexpr int kChunks = kRowBytes / 16;    // 16-byte chunks per row
  static constexpr int kLaneChunks = kChunks / 2;   // chunks one lane holds
  static constexpr int kElemsPerChunk = 16 / kElemBytes;
};

// Which logical chunk of a row lane-half h holds as its c-th fragment chunk.
// bf16: product c covers d = 16c..16c+15 and half h supplies d = 16c+8h..+7.
// fp32: half h supplies the contiguous half d in [h*D/2, (h+1)*D/2); chunk c
// carries 4 consecutive k values consumed by 4 successive 32x32x2 products.
template <bool BF16, int D>
__device__ __forceinline__ int frag_chunk(int h, int c) {
  if constexpr (BF16) return 2 * c + h;
  else return h * RowGeom<BF16, D>::kLaneChunks + c;
}

// XOR swizzle of the 16-byte chunks of an LDS row: chunk c of row r is stored
// at c ^ sigma(r).  sigma is a bijection on 16 consecutive rows, so 16 lanes
// reading one logical chunk of 16 consecutive rows hit 16 distinct bank
// groups; and for 8 consecutive rows x 4 consecutive chunks (the footprint of
// a transposing read, see read_tr below) every bank group is hit exactly twice.
template <int CPR>
__device__ __forceinline__ int swz(int row, int c) {
  if constexpr (CPR >= 16) return c ^ (4 * (row & 3) + ((row >> 2) & 3));
  else if constexpr (CPR == 8) return c ^ (4 * ((row >> 1) & 1) + ((row >> 2) & 3));
  else return c;
}

// Reinterpret a 32-bit word as fp32.  Always pass the word by value: clang
// mis-evaluates __builtin_bit_cast applied directly to an ext_vector element
// (it reads element 0), which is why the element is copied into `x` first.
__device__ __forceinline__ float u2f(uint32_t x) { return __builtin_bit_cast(float, x); }

// acc += A(chunk a) * B(chunk b) over the k values the chunks carry.
template <bool BF16>
__device__ __forceinline__ void mfma_chunk(const u32x4 &a, const u32x4 &b, f32x16 &acc) {
  if constexpr (BF16) {
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                  __builtin_bit_cast(bf16x8, b), acc, 0, 0, 0);
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      acc = __builtin_amdgcn_mfma_f32_32x32x2f32(u2f(a[i]), u2f(b[i]), acc, 0, 0, 0);
  }
}

// Row index (within a 32-row block) of accumulator register r for half h.
__host__ __device__ constexpr int c_row(int r, int h) { return (r >> 2) * 8 + 4 * h + (r & 3); }

// Position of streamed row o (0..15 inside a 16-row group) in the transposed
// LDS layout.  Lane-half h consumes positions 8h..8h+7 of a group as one run,
// which are the rows c_row(j, h) for j = 0..7 (the rows its score registers
// hold), so the gradient product reads one contiguous run per lane.
__device__ __forceinline__ int tpos(int o) { return 8 * ((o >> 2) & 1) + 4 * (o >> 3) + (o & 3); }

// Map the hardware workgroup id to a logical one so that consecutive logical
// ids run on the same XCD (workgroups are dealt round-robin over 8 XCDs):
// all query blocks of one head then share that XCD's L2.
__device__ __forceinline__ int xcd_remap(int b, int n) {
  const int per = n >> 3;
  const int full = per << 3;
  if (b >= full) return b;
  return (b & 7) * per + (b >> 3);
}

// Head and length rank (0 = the most work) of logical workgroup `bid` of a
// causal grid of n = heads * nblk workgroups, nblk per head, whose blocks of
// rank r all do about the same work and rank 0 the most.  The XCD that runs
// logical ids [x per, (x + 1) per), per = n / 8, holds whole heads when per
// is a multiple of nblk: there the ids take the ranks in order, each rank
// over the XCD's heads in turn, so the longest blocks of all its heads start
// first and the short ones fill the end.  Taking one head after the other,
// when a head has fewer blocks than an XCD has resident workgroups, starts
// the long blocks of its last heads late (32 blocks a head, 64 resident, 4
// heads per XCD: list scheduling finishes at 1.5x the ideal time).  The
// cost: more heads share each XCD's L2 at a time.  Otherwise: head-major,
// rank order within a head.
struct BlockPos {
  int bh, rank;
};
__device__ __forceinline__ BlockPos longest_first(int bid, int n, int nblk) {
  const int per = n >> 3;
  if (bid < (per << 3) && per % nblk == 0) {
    const int g = per / nblk;  // heads per XCD
    const int base = bid - bid % per;
    const int pos = bid - base;
    return {base / nblk + pos % g, pos / g};
  }
  return {bid / nblk, bid % nblk};
}

// Rank-major order over the whole grid, for causal grids of more than one
// round whose XCDs would otherwise hold parts of heads: hardware workgroup
// b takes rank b / nbh of head b % nbh (nbh heads).  The hardware deals
// consecutive ids to the eight XCDs in turn, so each XCD runs every eighth
// entry of the list sorted longest first: the same mix of long and short
// blocks on every XCD.  Taking the heads one after the other instead gives
// the XCD that holds a head's first half all of its long blocks (4 heads of
// 128 blocks at one workgroup per CU: list scheduling finishes at 1.5x the
// ideal time, against 1.01x in this order).  The heads' rows then spread
// over every XCD's L2.
__device__ __forceinline__ BlockPos rank_major(int b, int nbh) { return {b % nbh, b / nbh}; }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// NaN-propagating maximum (IEEE 754-2019 maximum).  gfx950 executes it
// natively (v_maximum3_f32), without the per-input NaN quieting that fmaxf
// (maxNum) needs in IEEE mode.
__device__ __forceinline__ float vmax(float a, float b) { return __builtin_elementwise_maximum(a, b); }
__device__ __forceinline__ float vmax3(float a, float b, float c) { return vmax(vmax(a, b), c); }

typedef short lds_v4s __attribute__((vector_size(8)));

// Transposing LDS read (ds_read_b64_tr_b16).  Within each group of 16 lanes,
// lane s supplies the address of 4 consecutive 16-bit values M[s][0..3]; lane
// i = 4a + b receives M[a][b], M[4+a][b], M[8+a][b], M[12+a][b].  With
// M[s] = row (base + s/4) of a row-major bf16 tile, columns d0(s%4)..+3, lane
// i gets column d0(a) + b of 4 consecutive rows: a K-major MFMA operand read
// straight from an N-major tile.
__device__ __forceinline__ u32x2 read_tr(const void *lds_byte_addr) {
  typedef __attribute__((address_space(3))) lds_v4s lds_v4s_ptr;
  const auto *p = (const lds_v4s_ptr *)(__attribute__((address_space(3))) char *)(lds_byte_addr);
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s_ptr *)p));
}

// Asynchronous 16-byte global -> LDS copy (global_load_lds_dwordx4): lane L
// of the wave writes its 16 bytes to lds_wave_base + 16 L.  `lds_wave_base`
// must be the same for the whole wave.  Completion is tracked by vmcnt, so a
// __syncthreads() (which waits for it) orders it before later LDS reads.
__device__ __forceinline__ void dma16(const void *gsrc, u32x4 *lds_wave_base) {
  __builtin_amdgcn_global_load_lds(gsrc, lds_wave_base, 16, 0, 0);
}

// The same copy, from a wave-uniform 64-bit base plus a 32-bit lane offset,
// issued as inline assembly so that the compiler does not see it.  The
// compiler then neither waits for it before LDS reads it cannot tell apart
// from its target (the transposing reads) nor treats LDS reads as unordered
// while it is in flight.  The caller owns its completion: s_waitcnt vmcnt(0)
// (vmcnt0_wait below) before the barrier that publishes the tile.  The copy
// writes no register; m0 is set and declared clobbered in the same statement
// (one wait state between the m0 write and the copy).
__device__ __forceinline__ void dma16_unseen(const void *sbase, uint32_t voff, u32x4 *lds_wave_base) {
  typedef __attribute__((address_space(3))) char lds_char;
  const uint32_t lds = uint32_t(reinterpret_cast<uintptr_t>((lds_char *)(reinterpret_cast<char *>(lds_wave_base))));
  asm volatile(
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %0, %1"
      :
      : "v"(voff), "s"(sbase), "s"(lds)
      : "memory", "m0");
}

// Wait for every vector-memory load of the wave, copies included.
__device__ __forceinline__ void vmcnt0_wait() { __builtin_amdgcn_s_waitcnt(0x0F70); }

__device__ __forceinline__ u32x4 zero4() { return u32x4{0u, 0u, 0u, 0u}; }

// Pack two fp32 values to bf16 (round to nearest even) in one dword.
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}

// ------------------------------------------------------------ debug build
// Built with -DSTREAMKL_DEBUG, every global-memory access of the kernels, and
// the LDS accesses of their tile loops, are checked against the extent of
// the buffer they belong to (the extents travel in the kernels' parameters).
// An access found outside its buffer is not made: a global load or copy
// reads a zeroed dummy line instead, an LDS access goes to the start of the
// workgroup's LDS, a store or atomic is dropped.  The site of the first such
// access, (file id << 16) | line, is kept in dbg_word -- one per translation
// unit -- for the host to collect (dbg_take).  Without the macro, SK_G and
// SK_L return their pointer and SK_OK is true, so a release build compiles
// to the same instructions as the code without the checks.
// File ids: 1 streamkl_fwd.hip, 2 streamkl_bwd.h, 3 streamkl_bwd_fused.hip.
__host__ __device__ inline bool dbg_in(uintptr_t a, size_t n, uintptr_t lo, size_t bytes) {
  return a >= lo && a - lo <= bytes && n <= bytes - (a - lo);
}
#ifdef STREAMKL_DEBUG
static __device__ unsigned int dbg_word;
static __device__ __align__(16) u32x4 dbg_dummy[4];
__device__ __forceinline__ bool dbg_ok(const void *p, size_t n, const void *lo, size_t bytes, unsigned site) {
  const bool ok = dbg_in(uintptr_t(p), n, uintptr_t(lo), bytes);
  if (!ok) atomicCAS(&dbg_word, 0u, site);
  return ok;
}
template <class T>
__device__ __forceinline__ T *dbg_global(T *p, size_t n, const void *lo, size_t bytes, unsigned site) {
  return dbg_ok(p, n, lo, bytes, site) ? p : reinterpret_cast<T *>(dbg_dummy);
}
template <class T>
__device__ __forceinline__ T *dbg_lds(T *p, size_t n, const void *lo, size_t bytes, unsigned site) {
  return dbg_ok(p, n, lo, bytes, site) ? p : (T *)(lo);
}
// The first violation recorded by this translation unit's kernels since the
// last call (0: none), then cleared.  Synchronises the device.
static inline unsigned dbg_take() {
  unsigned w = 0;
  if (hipDeviceSynchronize() != hipSuccess) return ~0u;
  if (hipMemcpyFromSymbol(&w, HIP_SYMBOL(dbg_word), sizeof(w)) != hipSuccess) return ~0u;
  const unsigned z = 0;
  if (hipMemcpyToSymbol(HIP_SYMBOL(dbg_word), &z, sizeof(z)) != hipSuccess) return ~0u;
  return w;
}
#define SK_SITE(file) ((unsigned(file) << 16) | unsigned(__LINE__))
#define SK_G(p, n, lo, bytes, file) ::streamkl::dbg_global((p), (n), (lo), (bytes), SK_SITE(file))
#define SK_L(p, n, lo, bytes, file) ::streamkl::dbg_lds((p), (n), (lo), (bytes), SK_SITE(file))
#define SK_OK(p, n, lo, bytes, file) ::streamkl::dbg_ok((p), (n), (lo), (bytes), SK_SITE(file))
#define SK_DBG_ARGS(...) , __VA_ARGS__
#else
#define SK_G(p, n, lo, bytes, file) (p)
#define SK_L(p, n, lo, bytes, file) (p)
#define SK_OK(p, n, lo, bytes, file) true
#define SK_DBG_ARGS(...)
#endif

}  // namespace streamkl
