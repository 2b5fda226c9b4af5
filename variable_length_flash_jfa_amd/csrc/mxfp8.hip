// MXFP8 forward: E4M3 values with one E8M0 scale per block of 32 elements along
// each product's contraction axis ("Meta's TLX attention kernel outpaces
// FlashAttention-4 on B200", section on the kernel's variants; "Optimizing Jagged
// Flash Attention with TLX" reading note: the low-precision fork keeps the kernel's
// structure).
//
// Formats (the pages name E4M3 values and E8M0 block scales and nothing more):
//   * E4M3 is the OCP 8-bit float (bias 7, subnormals, max 448, no infinities);
//     E8M0 code c stands for 2^(c - 127).
//   * A block's scale is the smallest 2^e with max|x| <= 448 * 2^e (nothing
//     saturates); elements are x / 2^e rounded to nearest even E4M3.
//   * Q and K: blocks of 32 head-dimension columns of one row.
//   * V: blocks of 32 consecutive keys of one sequence and column.  Block j of
//     sequence b (first key kv0) is stored at block index g = b + floor(kv0 / 32) + j,
//     which is distinct for every (b, j) and below batch + ceil(total_kv / 32); its
//     32 bytes per (head, column) hold the keys in the order the matrix-core B/A
//     operand takes them (see v_pos).
//   * P: blocks of 32 consecutive keys of a row, aligned to the sequence start.
//
// Softmax runs in base 2 with the row maximum rounded up to an integer, so every
// rescale of the running sums is an exact power of two and the block quantization of
// P commutes with it: the result does not depend on the order of the key blocks.
//
// Matrix cores: v_mfma_scale_f32_32x32x64_f8f6f4.  Its 64-deep contraction is two
// 32-element scale blocks: block 0 is bytes 0..15 of lanes i and i + 32, block 1 is
// bytes 16..31 of the same lanes; lane i supplies block 0's E8M0 code for row i and
// lane i + 32 block 1's.  S^T = K Q^T takes two such products per 64 head-dimension
// columns; O^T = V^T P^T takes one per 64 keys and 32 columns, with P^T in exactly the
// register order the S^T accumulator leaves it.
#include "jfa_device.h"
#include "jfa_internal.h"

namespace jfa {
namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

// E8M0 code of the smallest 2^e with amax <= 448 * 2^e: with amax = (1 + f) 2^(E - 127),
// 448 * 2^e = 1.75 * 2^(e + 8), so e = E - 135 when f <= 0.75 and one more above.
__device__ __forceinline__ int mx_scale_code(float amax) {
  const uint32_t bits = __float_as_uint(amax);
  const int e = (int)((bits >> 23) & 0xff) - 8 + ((bits & 0x7fffff) > 0x600000u ? 1 : 0);
  return min(max(e, 0), 254);
}
// 2^-(code - 127) as a float (codes up to 253 stay normal; finite inputs give <= 248).
__device__ __forceinline__ float mx_inv_scale(int code) { return __uint_as_float((uint32_t)(254 - code) << 23); }

// Four floats (|y| <= 448) -> four E4M3 bytes, round to nearest even.
__device__ __forceinline__ int pack4_e4m3(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  return __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
}

// Byte position of key k (0 .. 31) inside a stored V block: the S^T accumulator of a
// 32-key tile gives lane half hh the keys 8 grp + 4 hh + e (grp, e = 0 .. 3) in
// register order 4 grp + e, and the same bytes of V^T must line up with them.
__device__ __forceinline__ int v_pos(int k) { return 16 * ((k >> 2) & 1) + 4 * (k >> 3) + (k & 3); }

// ----------------------------------------------------------------------------
// Quantizers
// ----------------------------------------------------------------------------

// One thread per 32-column block of a row: [rows * H, D] bf16 -> bytes + codes.
__global__ __launch_bounds__(256) void quantize_rows_kernel(const bf16* __restrict__ x, int64_t nblocks,
                                                            uint8_t* __restrict__ val, uint8_t* __restrict__ scl) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= nblocks) return;
  const bf16x8* src = reinterpret_cast<const bf16x8*>(x + i * 32);
  float f[32];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const bf16x8 v = src[c];
#pragma unroll
    for (int e = 0; e < 8; ++e) f[8 * c + e] = (float)v[e];
  }
  float amax = 0.f;
#pragma unroll
  for (int e = 0; e < 32; ++e) amax = fmaxf(amax, fabsf(f[e]));
  const int code = mx_scale_code(amax);
  const float inv = mx_inv_scale(code);
  i32x4 w0, w1;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    w0[e] = pack4_e4m3(f[4 * e] * inv, f[4 * e + 1] * inv, f[4 * e + 2] * inv, f[4 * e + 3] * inv);
    w1[e] = pack4_e4m3(f[16 + 4 * e] * inv, f[17 + 4 * e] * inv, f[18 + 4 * e] * inv, f[19 + 4 * e] * inv);
  }
  i32x4* dst = reinterpret_cast<i32x4*>(val + i * 32);
  dst[0] = w0;
  dst[1] = w1;
  scl[i] = (uint8_t)code;
}

struct QuantVArgs {
  const bf16* v;
  const void* offsets;
  int off64;
  int heads, hd;     // H, D
  uint8_t* val;      // [G, H, D, 32]
  uint8_t* scl;      // [G, H, D]
};

// Workgroup (b, y) takes the tasks y, y + gridDim.y, ... of sequence b, a task being
// one 32-key block j and a chunk of up to 256 of the H * D columns.  The block's rows
// are read with 16-byte loads into LDS, then each thread quantizes one column.
__global__ __launch_bounds__(256) void quantize_v_kernel(QuantVArgs a) {
  constexpr int CW = 256, PAD = 8;
  __shared__ __attribute__((aligned(16))) bf16 tile[32][CW + PAD];
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const int64_t kv0 = load_offset(a.offsets, a.off64, b);
  const int n = (int)(load_offset(a.offsets, a.off64, b + 1) - kv0);
  const int nblk = (n + 31) / 32;
  const int64_t g0 = (int64_t)b + kv0 / 32;
  const int width = a.heads * a.hd;           // elements between consecutive keys
  const int nch = (width + CW - 1) / CW;
  for (int task = blockIdx.y; task < nblk * nch; task += gridDim.y) {
    const int j = task / nch;
    const int c0 = (task - j * nch) * CW;
    const int cw = min(CW, width - c0);       // a multiple of 64
    const int kn = min(32, n - 32 * j);
    const int slots = cw / 8;                 // 16-byte slots per row
    __syncthreads();                          // the previous task's readers are done
    for (int idx = tid; idx < 32 * slots; idx += 256) {
      const int r = idx / slots, sl = idx - r * slots;
      bf16x8 v = bf16x8{};
      if (r < kn) v = *reinterpret_cast<const bf16x8*>(a.v + (kv0 + 32 * j + r) * width + c0 + 8 * sl);
      *reinterpret_cast<bf16x8*>(&tile[r][8 * sl]) = v;
    }
    __syncthreads();
    if (tid < cw) {
      float y[32];
      float amax = 0.f;
#pragma unroll
      for (int k = 0; k < 32; ++k) {
        y[v_pos(k)] = (float)tile[k][tid];
        amax = fmaxf(amax, fabsf(y[v_pos(k)]));
      }
      const int code = mx_scale_code(amax);
      const float inv = mx_inv_scale(code);
      i32x4 w0, w1;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        w0[e] = pack4_e4m3(y[4 * e] * inv, y[4 * e + 1] * inv, y[4 * e + 2] * inv, y[4 * e + 3] * inv);
        w1[e] = pack4_e4m3(y[16 + 4 * e] * inv, y[17 + 4 * e] * inv, y[18 + 4 * e] * inv, y[19 + 4 * e] * inv);
      }
      const int64_t blk = (g0 + j) * width + c0 + tid;
      i32x4* dst = reinterpret_cast<i32x4*>(a.val + blk * 32);
      dst[0] = w0;
      dst[1] = w1;
      a.scl[blk] = (uint8_t)code;
    }
  }
}

// ----------------------------------------------------------------------------
// Forward
// ----------------------------------------------------------------------------

struct MxArgs {
  const uint8_t* q8;   // [q rows, H, D]
  const uint8_t* qs;   // [q rows, H, D / 32]
  const uint8_t* k8;   // [total_kv, H, D]
  const uint8_t* ks;   // [total_kv, H, D / 32]
  const uint8_t* v8;   // [G, H, D, 32]
  const uint8_t* vs;   // [G, H, D]
  const int4* items;
  const int* meta;
  bf16* o;
  float* lse;
  int q_len, heads;
  int64_t rows;        // output rows
  float c2;            // softmax scale * log2(e)
};

__device__ __forceinline__ i32x8 load32(const uint8_t* p0, const uint8_t* p1) {
  const i32x4 lo = *reinterpret_cast<const i32x4*>(p0);
  const i32x4 hi = *reinterpret_cast<const i32x4*>(p1);
  return i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

// Workgroups of NW waves walk the planned tiles (descending cost) round-robin; a tile
// is BM = 32 NW query rows of one sequence and head, a wave owns 32 of them.  Each
// 64-key block of K and V (and their scales) is read once per workgroup with
// coalesced 16-byte loads, one block ahead into registers, and written to one of two
// LDS buffers; one barrier per block.  K rows sit in LDS padded to D + 16 bytes, so
// the fragment reads of 16 consecutive rows meet 16 distinct groups of 4 banks; V
// blocks sit in operand order, so a fragment read is one contiguous KiB.
template <int D, int NW, bool BCAST, bool CAUSAL>
__global__ __launch_bounds__(64 * NW) void fwd_mx_kernel(MxArgs a) {
  constexpr int BM = 32 * NW;
  constexpr int NT = 64 * NW;           // threads
  constexpr int KS = D / 64;            // 64-column contraction steps of S
  constexpr int DB = D / 32;            // 32-column blocks of O
  constexpr int NSB = D / 32;           // scale bytes per Q/K row
  constexpr int KROW = D + 16;          // LDS bytes per K row
  constexpr int KT = 64 * KROW;         // K tile
  constexpr int VT = 2 * D * 32;        // V tile: two 32-key blocks in operand order
  constexpr int KST = 64 * NSB;         // K scales [64 keys][NSB]
  constexpr int VST = 2 * D;            // V scales [2 blocks][D]
  constexpr int BUF = KT + VT + KST + VST;
  constexpr int KCH = 64 * D / 16;      // 16-byte chunks of a K tile
  constexpr int VCH = VT / 16;
  constexpr int KR = (KCH + NT - 1) / NT;
  constexpr int VR = (VCH + NT - 1) / NT;
  constexpr int VSCH = VST / 16;        // 16-byte chunks of the V scales
  static_assert(64 + VSCH <= NT, "scale staging needs 64 + 2D/16 threads");
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * BUF];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int li = lane & 31, hh = lane >> 5;
  const int ntiles = a.meta[2];
  const int per_item = BCAST ? ((a.q_len + BM - 1) / BM) * a.heads : a.heads;
  const int64_t vstride = (int64_t)a.heads * D;   // between consecutive V blocks (x 32 bytes)
  // tile geometry: sequence b (K/V rows kv0 .. kv0 + n), query block m, head h, and
  // the key blocks the workgroup visits (all of the sequence, or, causal, up to its
  // last query row)
  struct Geo {
    int64_t kv0, gbase;
    int b, n, m, h, nblk;
  };
  auto geo = [&](int t) {
    Geo g;
    const int4 it = a.items[t / per_item];
    const int rem = t % per_item;
    g.b = it.x;
    g.kv0 = it.z;
    g.n = it.w;
    g.m = BCAST ? rem / a.heads : it.y;
    g.h = BCAST ? rem % a.heads : rem;
    g.nblk = ((CAUSAL ? min(g.n, g.m * BM + BM) : g.n) + 63) / 64;
    g.gbase = (int64_t)g.b + g.kv0 / 32;
    return g;
  };
  // staging registers of the next block
  i32x4 kst[KR], vst_[VR];
  uint32_t kss = 0;
  i32x4 vss = i32x4{0, 0, 0, 0};
  auto fetch = [&](const Geo& g, int kb) {
    const int j0 = 64 * kb;
#pragma unroll
    for (int r = 0; r < KR; ++r) {
      const int c = tid + NT * r;
      if (KCH % NT == 0 || c < KCH) {
        const int row = c / (D / 16), col = c % (D / 16);
        const int key = min(j0 + row, g.n - 1);
        kst[r] = *reinterpret_cast<const i32x4*>(a.k8 + ((g.kv0 + key) * a.heads + g.h) * D + col * 16);
      }
    }
#pragma unroll
    for (int r = 0; r < VR; ++r) {
      const int c = tid + NT * r;
      if (VCH % NT == 0 || c < VCH) {
        const int blk = c / (2 * D), within = c % (2 * D);
        vst_[r] = i32x4{0, 0, 0, 0};
        if (j0 + 32 * blk < g.n)
          vst_[r] = *reinterpret_cast<const i32x4*>(a.v8 + ((g.gbase + j0 / 32 + blk) * vstride + g.h * D) * 32 +
                                                    within * 16);
      }
    }
    if (tid < 64) {
      const int key = min(j0 + tid, g.n - 1);
      const uint8_t* sp = a.ks + ((g.kv0 + key) * a.heads + g.h) * NSB;
      kss = NSB == 4 ? *reinterpret_cast<const uint32_t*>(sp) : *reinterpret_cast<const uint16_t*>(sp);
    } else if (tid < 64 + VSCH) {
      const int c = tid - 64;
      const int blk = c / (D / 16), within = c % (D / 16);
      vss = i32x4{0x7f7f7f7f, 0x7f7f7f7f, 0x7f7f7f7f, 0x7f7f7f7f};   // code 127 (1.0) for a missing block
      if (j0 + 32 * blk < g.n)
        vss = *reinterpret_cast<const i32x4*>(a.vs + (g.gbase + j0 / 32 + blk) * vstride + g.h * D + within * 16);
    }
  };
  auto stash = [&](int buf) {
    uint8_t* base = smem + buf * BUF;
#pragma unroll
    for (int r = 0; r < KR; ++r) {
      const int c = tid + NT * r;
      if (KCH % NT == 0 || c < KCH)
        *reinterpret_cast<i32x4*>(base + (c / (D / 16)) * KROW + (c % (D / 16)) * 16) = kst[r];
    }
#pragma unroll
    for (int r = 0; r < VR; ++r) {
      const int c = tid + NT * r;
      if (VCH % NT == 0 || c < VCH) *reinterpret_cast<i32x4*>(base + KT + c * 16) = vst_[r];
    }
    if (tid < 64) {
      if (NSB == 4)
        *reinterpret_cast<uint32_t*>(base + KT + VT + tid * 4) = kss;
      else
        *reinterpret_cast<uint16_t*>(base + KT + VT + tid * 2) = (uint16_t)kss;
    } else if (tid < 64 + VSCH) {
      *reinterpret_cast<i32x4*>(base + KT + VT + KST + (tid - 64) * 16) = vss;
    }
  };
  // Q^T fragment: lane (query li, half hh) holds columns 64 s + 16 hh .. + 15 and
  // 64 s + 32 + 16 hh .. + 15, and the code of column block 2 s + hh
  i32x8 qf[KS];
  int qsc[KS];
  auto load_q = [&](const Geo& g) {
    const int q_rows = BCAST ? a.q_len : g.n;
    const int i0 = g.m * BM + 32 * wave;
    if (i0 < q_rows) {
      const int64_t qrow = BCAST ? (int64_t)min(i0 + li, q_rows - 1) : g.kv0 + min(i0 + li, q_rows - 1);
      const uint8_t* qp = a.q8 + (qrow * a.heads + g.h) * D;
      const uint8_t* qsp = a.qs + (qrow * a.heads + g.h) * NSB;
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        qf[s] = load32(qp + 64 * s + 16 * hh, qp + 64 * s + 32 + 16 * hh);
        qsc[s] = qsp[2 * s + hh];
      }
    }
  };

  // XT: tile t + gridDim.x's first block is loaded during tile t's last block (into
  // the other LDS buffer) and its Q fragment after it; in broadcast mode a tile of
  // the same query block and head keeps the Q fragment (with a grid that is a
  // multiple of the tiles per sequence, every tile of a workgroup does).  Without
  // XT (self mode at two waves, chosen for short sequences: tiles of one or two
  // blocks) a tile loads its Q fragment and first block together at its start, so
  // that they land in one memory latency.  Block kb of a tile sits in buffer
  // (pb + kb) & 1.
  constexpr bool XT = BCAST || NW > 2;
  int t = blockIdx.x;
  if (t >= ntiles) return;
  Geo cur{};
  if constexpr (XT) {
    cur = geo(t);
    load_q(cur);
    if (cur.nblk > 0) {
      fetch(cur, 0);
      stash(0);
    }
    __syncthreads();
  }
  int pb = 0;
  for (;;) {
    if constexpr (!XT) {   // the previous tile's last barrier retired its readers
      cur = geo(t);
      load_q(cur);
      if (cur.nblk > 0) {
        fetch(cur, 0);
        stash(pb);
      }
      __syncthreads();
    }
    const int tn = t + (int)gridDim.x;
    const bool has_next = tn < ntiles;
    const Geo nxt = XT && has_next ? geo(tn) : cur;
    const int b = cur.b, n = cur.n, m = cur.m, h = cur.h, nblk = cur.nblk;
    const int64_t kv0 = cur.kv0;
    const int q_rows = BCAST ? a.q_len : n;
    const int i0 = m * BM + 32 * wave;
    const bool active = i0 < q_rows;
    const int wave_end = CAUSAL ? min(n, i0 + 32) : n;
    // The Q fragment may have been loaded at the end of the previous tile: consume it
    // here, so that the compiler's wait for it lands before the block loop and not at
    // every block's first product (where it would also wait for the next block's loads).
#pragma unroll
    for (int s = 0; s < KS; ++s) asm volatile("" : "+v"(qf[s]), "+v"(qsc[s]));
    f32x16 acc[DB];
#pragma unroll
    for (int d = 0; d < DB; ++d) acc[d] = f32x16{};
    float mrun = -INFINITY, lrun = 0.f;
    for (int kb = 0; kb < nblk; ++kb) {
      const int j0 = 64 * kb;
      const int buf = (pb + kb) & 1;
      // the next block of this tile, or else the next tile's first, goes into the
      // other buffer at the end of this one (one load site: with a load site per
      // case the compiler merges the staging registers with copies that wait for
      // the loads at once)
      const bool in_tile = kb + 1 < nblk;
      const bool pf = in_tile || (XT && has_next && nxt.nblk > 0);
      if (pf) fetch(in_tile ? cur : nxt, in_tile ? kb + 1 : 0);
      if (active && j0 < wave_end) {
        const uint8_t* base = smem + buf * BUF;
        // S^T for keys j0 + 32 rb + li (rows) x the wave's 32 queries (columns)
        f32x16 st[2];
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
          const uint8_t* krow = base + (32 * rb + li) * KROW;
          st[rb] = f32x16{};
#pragma unroll
          for (int s = 0; s < KS; ++s) {
            const i32x4 lo = *reinterpret_cast<const i32x4*>(krow + 64 * s + 16 * hh);
            const i32x4 hi = *reinterpret_cast<const i32x4*>(krow + 64 * s + 32 + 16 * hh);
            const int ksc = base[KT + VT + (32 * rb + li) * NSB + 2 * s + hh];
            st[rb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]}, qf[s], st[rb], 0, 0, 0, ksc, 0,
                qsc[s]);
          }
        }
        // masks (only blocks that reach past the sequence end or, causal, above the
        // diagonal of the wave's first query row need them)
        const int qcol = i0 + li;   // query index inside the sequence (self mode)
        if (j0 + 64 > n || (CAUSAL && j0 + 63 > i0)) {
#pragma unroll
          for (int rb = 0; rb < 2; ++rb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int key = j0 + 32 * rb + 8 * (r >> 2) + 4 * hh + (r & 3);
              const bool ok = key < n && (!CAUSAL || key <= qcol);
              st[rb][r] = ok ? st[rb][r] : -INFINITY;
            }
        }
        // raw-score maxima of the two 32-key halves of column li (c2 > 0 and rounding
        // are monotone, so the base-2 maximum is this maximum times c2)
        // (a tree, emitted as three-input maxima: a serial chain of 15 would stall the
        // wave on each step; with -fno-honor-nans the MFMA results are not first
        // quieted)
        float smax[2];
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
          float m[5];
#pragma unroll
          for (int k = 0; k < 5; ++k) m[k] = fmaxf(fmaxf(st[rb][3 * k], st[rb][3 * k + 1]), st[rb][3 * k + 2]);
          const float mx = fmaxf(fmaxf(fmaxf(m[0], m[1]), m[2]), fmaxf(fmaxf(m[3], m[4]), st[rb][15]));
          smax[rb] = fmaxf(mx, __shfl_xor(mx, 32));
        }
        // Lazy rescaling: the integer running max moves only when some row of the
        // wave would grow by more than 2^8 (a wave-uniform test); otherwise P is taken
        // against the stale max and may reach 2^8, which the block scale codes absorb
        // (with an integer max the scaled elements y, and so the quantized P, do not
        // depend on it) and O / l and the log-sum-exp divide out.
        const float mc = ceilf(fmaxf(smax[0], smax[1]) * a.c2);
        if (__ballot(mc > mrun + 8.f)) {
          const float mnew = fmaxf(mrun, mc);
          const float alpha = mrun == -INFINITY ? 0.f : ldexpf(1.f, (int)(mrun - mnew));
          lrun *= alpha;
#pragma unroll
          for (int d = 0; d < DB; ++d)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[d][r] *= alpha;
          mrun = mnew;
        }
        const float msub = mrun == -INFINITY ? 0.f : mrun;
        // P in 32-key blocks: the block maximum 2^(c2 smax - m) sets the E8M0 code e,
        // then y = 2^(c2 s - m - e) is the scaled element, and l gains 2^e sum(y)
        int pcode[2];
        i32x8 pf;
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
          pcode[rb] = mx_scale_code(fast_exp2(fmaf(smax[rb], a.c2, -msub)));
          const float off = msub + (float)(pcode[rb] - 127);
          float y[16];
          float ysum[4] = {0.f, 0.f, 0.f, 0.f};   // four short chains instead of one of 16 adds
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            y[r] = fast_exp2(fmaf(st[rb][r], a.c2, -off));
            ysum[r & 3] += y[r];
          }
          lrun += ldexpf((ysum[0] + ysum[1]) + (ysum[2] + ysum[3]), pcode[rb] - 127);
#pragma unroll
          for (int e = 0; e < 4; ++e)
            pf[4 * rb + e] = pack4_e4m3(y[4 * e], y[4 * e + 1], y[4 * e + 2], y[4 * e + 3]);
        }
        const int psc = hh == 0 ? pcode[0] : pcode[1];
        // O^T += V^T P^T: lane (column 32 d + li, half hh) reads bytes 16 hh .. of both
        // key blocks; its scale is that of key block hh
#pragma unroll
        for (int d = 0; d < DB; ++d) {
          const uint8_t* vp = base + KT + (32 * d + li) * 32 + 16 * hh;
          const i32x4 lo = *reinterpret_cast<const i32x4*>(vp);
          const i32x4 hi = *reinterpret_cast<const i32x4*>(vp + D * 32);
          const int vsc = base[KT + VT + KST + hh * D + 32 * d + li];
          acc[d] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
              i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]}, pf, acc[d], 0, 0, 0, vsc, 0, psc);
        }
      }
      if (pf) stash(buf ^ 1);
      __syncthreads();
    }
    if (XT && nblk == 0 && has_next && nxt.nblk > 0) {   // an empty sequence (broadcast mode)
      fetch(nxt, 0);
      stash(pb);
      __syncthreads();
    }
    // the tile is done with its Q fragment
    if (XT && has_next && !(BCAST && nxt.m == m && nxt.h == h)) load_q(nxt);
    // epilogue: O = acc / l (bf16), LSE = ln 2 (m + log2 l)
    if (active) {
      const float lt = lrun + __shfl_xor(lrun, 32);
      const float inv_l = lt > 0.f ? 1.f / lt : 0.f;
      if (i0 + li < q_rows) {
        const int64_t orow = (BCAST ? (int64_t)b * a.q_len : kv0) + i0 + li;
        bf16* op = a.o + (orow * a.heads + h) * D;
#pragma unroll
        for (int d = 0; d < DB; ++d)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            bf16x4 w;
#pragma unroll
            for (int e = 0; e < 4; ++e) w[e] = (bf16)(acc[d][4 * g + e] * inv_l);
            *reinterpret_cast<bf16x4*>(op + 32 * d + 8 * g + 4 * hh) = w;
          }
        if (hh == 0) a.lse[(int64_t)h * a.rows + orow] = lt > 0.f ? (mrun + __log2f(lt)) * kLn2 : -INFINITY;
      }
    }
    if (!has_next) break;
    pb = (pb + nblk) & 1;
    cur = nxt;
    t = tn;
  }
}

template <int D, int NW, bool BCAST, bool CAUSAL>
hipError_t launch_mx_one(const MxArgs& a, int64_t max_tiles, hipStream_t s) {
  const void* fn = reinterpret_cast<const void*>(&fwd_mx_kernel<D, NW, BCAST, CAUSAL>);
  const int grid = persistent_grid(fn, 64 * NW, max_tiles);
  hipLaunchKernelGGL((fwd_mx_kernel<D, NW, BCAST, CAUSAL>), dim3(grid), dim3(64 * NW), 0, s, a);
  return hipGetLastError();
}

template <int D, int NW>
hipError_t launch_mx_nw(const Problem& p, const MxArgs& a, int64_t max_tiles, hipStream_t s) {
  if (p.broadcast) return launch_mx_one<D, NW, true, false>(a, max_tiles, s);
  if (p.causal) return launch_mx_one<D, NW, false, true>(a, max_tiles, s);
  return launch_mx_one<D, NW, false, false>(a, max_tiles, s);
}

template <int D>
hipError_t launch_mx_d(const Problem& p, const MxArgs& a, int64_t max_tiles, hipStream_t s) {
  switch (fwd_waves(p)) {
    case 2: return launch_mx_nw<D, 2>(p, a, max_tiles, s);
    case 4: return launch_mx_nw<D, 4>(p, a, max_tiles, s);
    default: return launch_mx_nw<D, 8>(p, a, max_tiles, s);
  }
}

}  // namespace

int64_t mx_v_blocks(int64_t batch, int64_t total_kv) { return batch + (total_kv + 31) / 32; }

hipError_t launch_mx_quantize_rows(const void* x, int64_t rows, int heads, int head_dim, void* val, void* scl,
                                   hipStream_t s) {
  const int64_t nblocks = rows * heads * (head_dim / 32);
  if (nblocks == 0) return hipSuccess;
  hipLaunchKernelGGL(quantize_rows_kernel, dim3((unsigned)((nblocks + 255) / 256)), dim3(256), 0, s,
                     reinterpret_cast<const bf16*>(x), nblocks, reinterpret_cast<uint8_t*>(val),
                     reinterpret_cast<uint8_t*>(scl));
  return hipGetLastError();
}

hipError_t launch_mx_quantize_v(const Problem& p, const void* v, void* val, void* scl, hipStream_t s) {
  if (p.batch == 0) return hipSuccess;
  QuantVArgs a;
  a.v = reinterpret_cast<const bf16*>(v);
  a.offsets = p.offsets;
  a.off64 = p.off64;
  a.heads = p.heads;
  a.hd = p.head_dim;
  a.val = reinterpret_cast<uint8_t*>(val);
  a.scl = reinterpret_cast<uint8_t*>(scl);
  hipLaunchKernelGGL(quantize_v_kernel, dim3((unsigned)p.batch, 8), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_fwd_mx(const Problem& p, const Plan& plan, const MxOperands& x, void* o, float* lse,
                         hipStream_t s) {
  MxArgs a;
  a.q8 = reinterpret_cast<const uint8_t*>(x.q8);
  a.qs = reinterpret_cast<const uint8_t*>(x.qs);
  a.k8 = reinterpret_cast<const uint8_t*>(x.k8);
  a.ks = reinterpret_cast<const uint8_t*>(x.ks);
  a.v8 = reinterpret_cast<const uint8_t*>(x.v8);
  a.vs = reinterpret_cast<const uint8_t*>(x.vs);
  a.items = plan.items;
  a.meta = plan.meta;
  a.o = reinterpret_cast<bf16*>(o);
  a.lse = lse;
  a.q_len = p.q_len;
  a.heads = p.heads;
  a.rows = p.rows;
  a.c2 = p.scale * kLog2e;
  const int nw = fwd_waves(p);
  const int64_t max_tiles =
      p.broadcast ? (int64_t)p.batch * ((p.q_len + 32 * nw - 1) / (32 * nw)) * p.heads
                  : ((int64_t)p.total_kv / (32 * nw) + p.batch) * p.heads;
  return p.head_dim == 64 ? launch_mx_d<64>(p, a, max_tiles, s) : launch_mx_d<128>(p, a, max_tiles, s);
}

}  // namespace jfa
