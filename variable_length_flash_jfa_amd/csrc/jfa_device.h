// Device-side building blocks shared by the gfx950 JFA kernels.
//
// Matrix products use the CDNA4 bf16 MFMA v_mfma_f32_32x32x16_bf16 (one 64-lane
// wave computes a 32x32 fp32 tile from a 32x16 and a 16x32 bf16 operand).
// Operand/accumulator lane layouts (checked on the device):
//   A (M x K):  lane l holds A[m = l % 32][k = 8 * (l / 32) + e], e = 0..7
//   B (K x N):  lane l holds B[k = 8 * (l / 32) + e][n = l % 32]
//   C (M x N):  lane l, register r holds C[m = 8 * (r / 4) + 4 * (l / 32) + r % 4][n = l % 32]
// Only the pairing of k between A and B matters for the product, so an operand
// may carry any fixed permutation of k as long as the other carries the same.
//
// LDS tiles of bf16 rows (D elements) are stored row-major with 16-byte chunks
// XOR-swizzled by row, so that both 16-byte row reads of 32 consecutive rows and
// the gfx950 transposing read ds_read_b64_tr_b16 over groups of 4 rows are spread
// over the LDS banks.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace jfa {

typedef __bf16 bf16;
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegBig = -1.0e30f;   // finite "minus infinity" for running maxima

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.f;
  return z;
}

__device__ __forceinline__ bf16x8 zero_bf16x8() {
  bf16x8 z;
#pragma unroll
  for (int i = 0; i < 8; ++i) z[i] = (bf16)0.f;
  return z;
}

__device__ __forceinline__ bf16x8 cat(bf16x4 a, bf16x4 b) {
  return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Value of x held by lane (l ^ 32), combined with x by max / sum, via the gfx950
// cross-half swap (lanes < 32 see the upper half in element 1, lanes >= 32 see
// the lower half in element 0; the other element keeps the lane's own value).
__device__ __forceinline__ float max_across_halves(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_across_halves(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Sixteen dot products at once over the 32 lanes of each wave half: x[r] y[r] of
// every lane of a half is added up for each r.  Transpose-reduce: at each step a
// lane keeps half of its values and adds its partner's copy of them (partners
// differ in lane bit 4, then 3, 2, 1), so 16 shuffles do what 16 butterflies of 5
// steps would; the products are formed in the first step.  Lane l returns the sum
// for r = (l >> 1) & 15 (lanes l and l ^ 1 agree).
__device__ __forceinline__ float half_lane_dots16(const float (&x)[16], const f32x16& y, int lane) {
  float a[8], c[4], d[2];
  const bool b4 = (lane >> 4) & 1, b3 = (lane >> 3) & 1, b2 = (lane >> 2) & 1, b1 = (lane >> 1) & 1;
#pragma unroll
  for (int k = 0; k < 8; ++k) {   // a[k]: r = k + 8 b4
    const float lo = x[k] * y[k], hi = x[k + 8] * y[k + 8];
    a[k] = (b4 ? hi : lo) + __shfl_xor(b4 ? lo : hi, 16);
  }
#pragma unroll
  for (int k = 0; k < 4; ++k)   // c[k]: r = k + 4 b3 + 8 b4
    c[k] = (b3 ? a[k + 4] : a[k]) + __shfl_xor(b3 ? a[k] : a[k + 4], 8);
#pragma unroll
  for (int k = 0; k < 2; ++k)   // d[k]: r = k + 2 b2 + 4 b3 + 8 b4
    d[k] = (b2 ? c[k + 2] : c[k]) + __shfl_xor(b2 ? c[k] : c[k + 2], 4);
  float e = (b1 ? d[1] : d[0]) + __shfl_xor(b1 ? d[0] : d[1], 2);
  return e + __shfl_xor(e, 1);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// ---- swizzled LDS tiles -----------------------------------------------------

// XOR mask applied to the 16-byte chunk index of a row.  For D = 128 (16 chunks)
// rows 0..15 get 16 distinct masks; for D = 64 (8 chunks) rows 0..7 get 8.
template <int D>
__host__ __device__ __forceinline__ int swz_mask(int row) {
  if constexpr (D == 128) {
    return ((row & 3) << 2) | ((row >> 2) & 3);
  } else {
    return ((row & 3) << 1) | ((row >> 2) & 1);
  }
}

template <int D>
__host__ __device__ __forceinline__ int swz_chunk(int row, int chunk) {
  return chunk ^ swz_mask<D>(row);
}

// Byte offset of element (row, col) of a [rows][D] bf16 tile; col % 4 == 0.
template <int D>
__host__ __device__ __forceinline__ int tile_off(int row, int col) {
  return row * (D * 2) + (swz_chunk<D>(row, col >> 3) << 4) + ((col & 7) << 1);
}

// Fast per-lane addressing.  Every LDS operand read of the kernels is written as
// (lane_base ^ x) + y with compile-time (or wave-uniform) x and y, so that one
// VGPR per access pattern holds the lane's part and each read costs at most one
// XOR (y becomes the instruction's immediate offset).
//
// Row read (MFMA A operand, or B operand of a K^T product): lane l reads the 16
// bytes of logical chunk 2 * ks + l / 32 of row r0 + l % 32, r0 a multiple of 16:
//   tile_off(r0 + l % 32, 16 ks + 8 (l / 32)) == (row_base ^ (ks << 5)) + r0 * 2D.
template <int D>
__host__ __device__ __forceinline__ uint32_t row_read_base(int lane) {
  const int r = lane & 31, hf = lane >> 5;
  return (uint32_t)(r * (2 * D) + ((hf ^ swz_mask<D>(r)) << 4));
}
__host__ __device__ __forceinline__ uint32_t row_read_addr(uint32_t base, int ks) {
  return base ^ (uint32_t)(ks << 5);
}

// Transposing read (ds_read_b64_tr_b16): lane l supplies row kl + K + (t >> 2) and
// column 32 dt + 16 ((l >> 4) & 1) + 4 (t & 3), t = l % 16, where kl is the lane's
// k offset (4 (l / 32) or 8 (l / 32)) and K a compile-time multiple of 4 (0, 4, 8,
// 16 m, 32 m and their sums as used by the kernels: adding K then flips the row
// mask by a constant, see tr_mask_delta):
//   tile_off(kl + K + (t >> 2), col) == (tr_base ^ (((4 dt) ^ delta(K)) << 4)) + K * 2D.
template <int D>
__host__ __device__ __forceinline__ uint32_t tr_read_base(int lane, int kl) {
  const int t = lane & 15, g1 = (lane >> 4) & 1;
  const int r = kl + (t >> 2);
  const int cl = 16 * g1 + 4 * (t & 3);
  return (uint32_t)(r * (2 * D) + (((cl >> 3) ^ swz_mask<D>(r)) << 4) + ((cl & 7) << 1));
}
template <int D>
__host__ __device__ __forceinline__ int tr_mask_delta(int K) {
  return D == 128 ? ((K >> 2) & 3) : ((K >> 2) & 1);
}
template <int D>
__host__ __device__ __forceinline__ uint32_t tr_read_addr(uint32_t base, int K, int dt) {
  return (base ^ (uint32_t)(((4 * dt) ^ tr_mask_delta<D>(K)) << 4)) + (uint32_t)(K * 2 * D);
}

// Hides a value from the optimiser so that addresses derived from it are
// recomputed where they are used instead of being hoisted out of loops (which
// would keep dozens of loop-invariant addresses alive in VGPRs).
__device__ __forceinline__ uint32_t launder(uint32_t x) {
  asm volatile("" : "+v"(x));
  return x;
}

__device__ __forceinline__ bf16x8 lds_read8(const char* base, uint32_t off) {
  return *reinterpret_cast<const bf16x8*>(base + off);
}
__device__ __forceinline__ void lds_write8(char* base, uint32_t off, bf16x8 v) {
  *reinterpret_cast<bf16x8*>(base + off) = v;
}

// gfx950 transposing LDS read.  Within each group of 16 lanes, lane t supplies the
// address of 4 consecutive bf16 and receives element (t % 4) of the chunk read by
// lanes 4e + t / 4, e = 0..3.  With lane t pointing at row (k0 + t / 4), column
// (n0 + 4 * (t % 4)) of a row-major matrix M, lane t receives M[k0 + e][n0 + t].
__device__ __forceinline__ bf16x4 lds_read_tr(const char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
      (__attribute__((address_space(3))) bf16x4*)(p));
}

// MFMA operand (32 columns x 8 k) from a swizzled row-major [k][n] tile through two
// transposing reads: lane l gets M[kl + Klo + e][32 dt + l % 32] for e = 0..3 and
// M[kl + Khi + e][...] for e = 4..7 (kl is folded into tr_base).
template <int D>
__device__ __forceinline__ bf16x8 lds_operand_tr(const char* tile, uint32_t tr_base, int Klo, int Khi,
                                                 int dt) {
  const bf16x4 lo = lds_read_tr(tile + tr_read_addr<D>(tr_base, Klo, dt));
  const bf16x4 hi = lds_read_tr(tile + tr_read_addr<D>(tr_base, Khi, dt));
  return cat(lo, hi);
}

// ---- direct HBM -> LDS loads ------------------------------------------------------

// Raw buffer resource over `bytes` bytes from `base` (gfx9-family descriptor word 3).
// Buffer loads past `bytes` return zeros, which zero-fills rows past a sequence end.
// Both arguments must be wave-uniform; they are taken from the first lane so that
// the descriptor lives in SGPRs (a descriptor the compiler believes divergent is
// wrapped in a loop over its distinct values).
typedef __amdgpu_buffer_rsrc_t rsrc_t;
// 64-bit value from two 32-bit words; the words are unsigned so that a low word with
// bit 31 set does not sign-extend into the high word (readfirstlane returns int).
__host__ __device__ __forceinline__ uint64_t join_u32(uint32_t hi, uint32_t lo) {
  return ((uint64_t)hi << 32) | (uint64_t)lo;
}
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = (uint64_t)base;
  const uint64_t u = join_u32((uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(a >> 32)),
                              (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)a));
  return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>(u), (short)0,
                                           (int)__builtin_amdgcn_readfirstlane(bytes), 0x00020000);
}

// One 16-byte (or 4-byte) chunk per lane from the buffer straight into LDS (gfx950
// buffer_load_dwordx4 ... lds): the 64 lanes of a wave fill 64 consecutive chunks
// starting at the wave-uniform LDS address `lds`.  Completion is tracked by the
// vector-memory counter: call wait_lds_loads() before the barrier that publishes
// the data.
//
// The loads are issued through inline assembly on purpose: the compiler cannot
// tell which LDS bytes a DMA load writes, so for the builtin it inserts a full
// vmcnt(0) wait before the next LDS read, which would expose every prefetch (and
// every outstanding dQ reduce-add).  The kernels instead wait explicitly before the
// barrier that publishes a buffer.  The compiler does not count these loads, which
// can only make its own vmcnt waits more conservative (vector memory operations
// retire in issue order).
__device__ __forceinline__ uint32_t lds_addr(const char* p) {
  return __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)p);
}
// Buffer descriptor words forced into SGPRs (the same fields as make_rsrc).
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ u32x4 make_rsrc_sgpr(const void* base, uint32_t bytes) {
  const uint64_t a = (uint64_t)base;
  u32x4 r;
  r[0] = __builtin_amdgcn_readfirstlane((uint32_t)a);
  r[1] = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32) & 0xFFFFu);
  r[2] = __builtin_amdgcn_readfirstlane(bytes);
  r[3] = 0x00020000u;
  return r;
}
__device__ __forceinline__ void lds_load16(u32x4 r, uint32_t voff, char* lds) {
  asm volatile("s_mov_b32 m0, %2\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
               :
               : "v"(voff), "s"(r), "s"(lds_addr(lds))
               : "memory", "m0");
}
__device__ __forceinline__ void lds_load4(u32x4 r, uint32_t voff, char* lds) {
  asm volatile("s_mov_b32 m0, %2\n\tbuffer_load_dword %0, %1, 0 offen lds"
               :
               : "v"(voff), "s"(r), "s"(lds_addr(lds))
               : "memory", "m0");
}
// s_waitcnt vmcnt(0): all of this wave's vector memory operations are complete.
__device__ __forceinline__ void wait_lds_loads() { __builtin_amdgcn_s_waitcnt(0x0F70); }
// s_waitcnt vmcnt(N): all but the N most recently issued vector memory operations are
// complete (they retire in issue order).  gfx9 encoding: vmcnt in bits 3:0 and 15:14,
// expcnt (7) and lgkmcnt (15) left unconstrained.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Copies rows [0, nrows) of a [rows][D] bf16 tile (row r at byte r * row_bytes of
// the buffer, row_bytes a multiple of 2 D) into a swizzled LDS tile.  Each wave
// instruction covers 1024 bytes = RPI = 1024 / (2 D) rows; instruction u goes to
// wave u % NW.  Lane i of an instruction fills LDS chunk slot (i % CH) of row
// u RPI + i / CH, so it fetches logical chunk swz_chunk(row, slot) (the swizzle is
// an XOR involution).  The row mask splits as swz_mask(r0) ^ swz_mask(u RPI) for
// r0 < RPI, so the lane's offset is one base XOR a wave-uniform constant plus a
// wave-uniform row offset.
template <int D, int NW>
__device__ __forceinline__ void lds_load_tile(char* tile, int nrows, int wave, int lane, u32x4 r,
                                              uint32_t row_bytes) {
  constexpr int CH = D / 8;
  constexpr int RPI = 64 / CH;
  const int ninstr = nrows / RPI;
  const uint32_t l = launder((uint32_t)lane);
  const uint32_t r0 = l / CH;
  const uint32_t base = r0 * row_bytes + ((((uint32_t)l % CH) ^ (uint32_t)swz_mask<D>((int)r0)) << 4);
#pragma unroll
  for (int k = 0; k < (ninstr + NW - 1) / NW; ++k) {
    const int u = wave + k * NW;
    if (u < ninstr) {
      const uint32_t voff = (base ^ ((uint32_t)swz_mask<D>(u * RPI) << 4)) + (uint32_t)(u * RPI) * row_bytes;
      lds_load16(r, voff, tile + u * 1024);
    }
  }
}

// The same copy for a tile of NROWS rows with a fixed row pitch, with each wave's
// lane offsets computed once (one VGPR per instruction the wave issues, PER of
// them) instead of at every call, and the LDS destination given as a 32-bit LDS
// address.  Every wave issues exactly PER instructions (NROWS / RPI is a multiple
// of NW), so the calls need no per-instruction test either.
__device__ __forceinline__ void lds_load16_at(u32x4 r, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
               :
               : "v"(voff), "s"(r), "s"(lds)
               : "memory", "m0");
}
// Lane part of the global offset of copy instruction u (rows u RPI .. u RPI + RPI - 1).
template <int D>
__host__ __device__ __forceinline__ uint32_t tile_load_voff(int u, int lane, uint32_t row_bytes) {
  constexpr int CH = D / 8;
  constexpr int RPI = 64 / CH;
  const uint32_t r0 = (uint32_t)lane / CH;
  const uint32_t base = r0 * row_bytes + ((((uint32_t)lane % CH) ^ (uint32_t)swz_mask<D>((int)r0)) << 4);
  return (base ^ ((uint32_t)swz_mask<D>(u * RPI) << 4)) + (uint32_t)(u * RPI) * row_bytes;
}
template <int D, int NW, int NROWS>
struct TileLoader {
  static constexpr int CH = D / 8;
  static constexpr int RPI = 64 / CH;
  static constexpr int NI = NROWS / RPI;
  static constexpr int PER = NI / NW;
  static_assert(NI % NW == 0 && PER >= 1, "every wave issues the same number of instructions");
  uint32_t voff[PER];
  int wave;
  __device__ __forceinline__ void init(int wave_, int lane, uint32_t row_bytes) {
    wave = wave_;
#pragma unroll
    for (int k = 0; k < PER; ++k) voff[k] = tile_load_voff<D>(wave + k * NW, lane, row_bytes);
  }
  // Copies the tile whose first row `r` addresses into the LDS tile at `lds`.
  __device__ __forceinline__ void issue(u32x4 r, uint32_t lds) const {
#pragma unroll
    for (int k = 0; k < PER; ++k) lds_load16_at(r, voff[k], lds + (uint32_t)((wave + k * NW) * 1024));
  }
};

// ---- offsets -------------------------------------------------------------------

__device__ __forceinline__ int64_t load_offset(const void* offsets, int is64, int64_t i) {
  return is64 ? reinterpret_cast<const int64_t*>(offsets)[i]
              : (int64_t)reinterpret_cast<const int32_t*>(offsets)[i];
}

// ---- tile schedules ------------------------------------------------------------

enum Schedule : int { kSortedZigzag = 0, kIdentity = 1, kDynamic = 2 };

// Logical index of this persistent workgroup such that logical neighbours sit on
// the same XCD (workgroups are dispatched to the 8 XCDs round-robin by blockIdx).
__device__ __forceinline__ int xcd_logical_wg(int wg, int num_wg) {
  const int per = num_wg >> 3;            // num_wg is a multiple of 8
  return (wg & 7) * per + (wg >> 3);
}

// ---- transposed accumulator tiles -> bf16 rows ----------------------------------

// Writes a wave's 32 x D result, held as D / 32 MFMA accumulators with rows in the
// n index (acc[dt] register r = C[m = d - 32 dt][n = row]: lane l owns row l % 32
// and d = 32 dt + 8 (r / 4) + 4 (l / 32) + r % 4), to 32 consecutive rows of a bf16
// array with a row pitch of `ld` elements, times the lane's `scale`.  Straight from
// registers every store would cover 8 bytes of 32 different rows; instead the tile
// is staged through a private LDS slot of 64 D / PASSES bytes (16-byte chunks
// XOR-swizzled by row), 32 / PASSES rows per pass, and read back so that each store
// instruction writes whole rows in 16-byte pieces.  The stores go through a buffer
// descriptor spanning `nrows` rows, so rows past the end are dropped by the
// hardware range check; every call issues exactly D / 16 store instructions.
template <int D, int PASSES = 1>
__device__ __forceinline__ void store_acc_rows(const f32x16 (&acc)[D / 32], float scale, char* slot,
                                               bf16* dst, int64_t ld, int nrows, int lane) {
  constexpr int CH = D / 8;            // 16-byte chunks per row
  constexpr int RPI = 64 / CH;         // rows per read instruction
  constexpr int RPP = 32 / PASSES;     // rows per pass (the slot holds RPP rows)
  static_assert(RPP % RPI == 0, "a pass must cover whole read instructions");
  const int r = lane & 31, hf = lane >> 5;
  const uint32_t pitch = (uint32_t)(ld * 2);
  const rsrc_t out = make_rsrc(dst, (uint32_t)max(nrows, 0) * pitch);
  // lane-derived offsets are recomputed here rather than hoisted across tiles
  const uint32_t l = launder((uint32_t)lane);
  const uint32_t c = l % CH, r0 = l / CH;
  const uint32_t voff = r0 * pitch + 16u * c;
  const uint32_t loff = r0 * (2 * D) + ((c ^ r0) << 4);
#pragma unroll
  for (int p = 0; p < PASSES; ++p) {
    if (PASSES == 1 || r / RPP == p) {
      const int sr = r % RPP;   // slot row
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt) {
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          bf16x4 w;
#pragma unroll
          for (int e = 0; e < 4; ++e) w[e] = (bf16)(acc[dt][4 * q4 + e] * scale);
          const int ci = 4 * dt + q4;   // chunk of d = 32 dt + 8 q4 + 4 hf + e
          *reinterpret_cast<bf16x4*>(slot + sr * (2 * D) + ((ci ^ (sr & (CH - 1))) << 4) + 8 * hf) = w;
        }
      }
    }
    // LDS operations of a wave execute in order; the fences only keep the compiler
    // from moving the reads above the other lanes' writes (or a pass's writes above
    // the previous pass's reads).
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
    for (int i = 0; i < RPP / RPI; ++i) {
      // slot row RPI i + r0 with r0 < RPI: its swizzle mask is r0 ^ (RPI i mod CH)
      const uint32_t la = (loff ^ (uint32_t)(((RPI * i) & (CH - 1)) << 4)) + (uint32_t)(RPI * i * 2 * D);
      const bf16x8 v = *reinterpret_cast<const bf16x8*>(slot + la);
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), out,
                                             voff + (uint32_t)(RPP * p + RPI * i) * pitch, 0, 0);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }
}

}  // namespace jfa
