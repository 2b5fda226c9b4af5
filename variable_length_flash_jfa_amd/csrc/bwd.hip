// Jagged Flash Attention backward for gfx950.
//
// Launch sequence of one backward call:
//   1. the backward tile planner (plan.hip).  In self mode, when the sequences may
//      fit one tile each, it splits the tiles in two lists: sequences within one
//      tile, whose tiles form delta themselves and store their final dQ (the
//      single-tile, DIRECT kernel), and the longer ones, which take the steps below;
//   2. bwd_pre_kernel: delta_i = sum_d dO_i . O_i per (row, head) -- the row-wise
//      sum the backward needs ("Meta's TLX Block Attention Beats Flash Attention
//      v2 by 2.3x on Blackwell GPUs", section "One Constraint, Five
//      Eliminations", the Di preprocessing) -- and zeroing of the fp32 dQ
//      accumulator (bwd_pre_split_kernel: the rows of the first list only);
//   3. bwd_kernel: persistent workgroups over valid (sequence, 256-key block, head)
//      tiles.  Eight waves own 32 keys each, hold dK^T / dV^T accumulators and
//      their V fragment in registers, and stream the tile's query rows in blocks
//      of 32 straight from HBM into double-buffered LDS (gfx950 direct LDS loads).
//      Per query block every wave recomputes P from the saved LSE and forms
//      dV^T += dO^T P, dP = dO V^T, dS = P (dP - delta), dK^T += Q^T dS on
//      v_mfma_f32_32x32x16_bf16.  Waves whose 32 keys all lie past the sequence
//      end skip their work;
//   4. the dQ contribution of the whole 256-key tile is reduced on chip first: the
//      waves publish dS^T to LDS and each computes one 32-column slice of dS K over
//      all keys of the tile (with eight waves and four slices, the waves take two
//      consecutive query blocks, one each, so no partial sums are exchanged), and a
//      tile adds one fp32 partial per query row into HBM.  In broadcast-Q mode every sequence
//      adds into the same dQ ("Meta's TLX attention kernel outpaces
//      FlashAttention-4 on B200", section "GEM's sequences do not fit a fixed
//      grid"), so the accumulator is striped per XCD (8 fp32 copies).  The
//      reduce-adds of a block are issued behind the loads of the next one and
//      stay in flight while it computes (the pages pipeline this reduction through
//      a double-buffered on-chip stage: section "Five changes unlocked the gains",
//      item 3);
//   5. dq_finalize_kernel: sum of the stripes, times the softmax scale -> bf16 (in a
//      split call, dq_finalize_split_kernel over the first list's rows).
#include "jfa_device.h"
#include "jfa_internal.h"

namespace jfa {
namespace {

// ---------------------------------------------------------------------------
// 1. per-row statistics (LSE log2e, delta = rowsum(dO * O)) and dQ accumulator
//    zeroing
// ---------------------------------------------------------------------------
// rowstat[(h rows + row) 2 + 0] = LSE[h][row] log2(e) (so that P = exp2(S c log2 e -
// that) needs no multiply per score), rowstat[... + 1] = delta[h][row]; one 8-byte
// pair per row lets a single direct load bring both values of 32 rows into LDS.
// Every (row, head) pair of the call: one group of D / 8 threads per pair, and a
// grid-stride zero fill of the whole accumulator.
template <int D>
__global__ __launch_bounds__(256) void bwd_pre_kernel(const bf16* __restrict__ o,
                                                       const bf16* __restrict__ d_o,
                                                       const float* __restrict__ lse,
                                                       float2* __restrict__ rowstat, int64_t rows,
                                                       int heads, float* __restrict__ dq_acc,
                                                       int64_t acc_vec4) {
  constexpr int TPR = D / 8;                 // threads per (row, head)
  const int part = threadIdx.x % TPR;
  const int64_t npairs = rows * heads;
  const int64_t pair = ((int64_t)blockIdx.x * 256 + threadIdx.x) / TPR;
  if (pair < npairs) {   // a pair's TPR lanes share the branch
    const bf16x8 x = *reinterpret_cast<const bf16x8*>(o + pair * D + part * 8);
    const bf16x8 y = *reinterpret_cast<const bf16x8*>(d_o + pair * D + part * 8);
    float s = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) s += (float)x[e] * (float)y[e];
#pragma unroll
    for (int m = TPR / 2; m >= 1; m >>= 1) s += __shfl_xor(s, m);
    if (part == 0) {
      const int64_t row = pair / heads;
      const int64_t i = (pair - row * heads) * rows + row;   // [head][row]
      rowstat[i] = make_float2(lse[i] * kLog2e, s);
    }
  }
  // grid-stride zero fill of the dQ accumulator
  const int64_t nthreads = (int64_t)gridDim.x * 256;
  float4* acc = reinterpret_cast<float4*>(dq_acc);
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < acc_vec4; i += nthreads)
    acc[i] = make_float4(0.f, 0.f, 0.f, 0.f);
}

// Rows of a split call's first list (self mode; see the backward plan): an item
// (b, j, kv0, n) of a sequence longer than one tile covers the rows [kv0 + j bn,
// kv0 + min(n, (j + 1) bn)), and together the items cover every row whose delta and
// dQ finalize the call needs; the single-tile kernel forms the others' itself.
// Each wave takes items in turn (units of 16 rows would leave most of a larger group
// idle) and walks the item's (row, head) pairs in memory order, a group of lanes per
// pair; the next item is loaded during the current one.
struct SplitWalk {
  int lane, nwaves, unit, units;
  __device__ SplitWalk(const int* __restrict__ meta, int heads) {
    lane = threadIdx.x & 63;
    nwaves = (int)gridDim.x * (int)(blockDim.x >> 6);
    unit = (int)blockIdx.x * (int)(blockDim.x >> 6) + (int)(threadIdx.x >> 6);
    units = meta[2] / heads;   // meta[2] counts the first list's (item, head) tiles
  }
};
__device__ __forceinline__ void split_pairs(const int4& it, int heads, int bn, int64_t& p0, int64_t& p1) {
  p0 = ((int64_t)it.z + (int64_t)it.y * bn) * heads;                 // first (row, head) pair
  p1 = ((int64_t)it.z + min(it.w, (it.y + 1) * bn)) * heads;          // one past the last
}

// The same statistics and zeroing for the rows of a split call's first list only
// (none when every sequence fits one tile).  NP passes of pairs have their loads
// issued before any of them is used.
template <int D>
__global__ __launch_bounds__(256) void bwd_pre_split_kernel(const bf16* __restrict__ o,
                                                             const bf16* __restrict__ d_o,
                                                             const float* __restrict__ lse,
                                                             float2* __restrict__ rowstat, int64_t rows,
                                                             int heads, float* __restrict__ dq_acc,
                                                             const int4* __restrict__ items,
                                                             const int* __restrict__ meta, int bn) {
  constexpr int TPR = D / 8, PPP = 64 / TPR, NP = 16;   // lanes per pair, pairs per wave pass, passes in flight
  SplitWalk w(meta, heads);
  const int part = w.lane % TPR, sub = w.lane / TPR;
  if (w.unit >= w.units) return;
  int4 it = items[w.unit];
  for (int u = w.unit; u < w.units; u += w.nwaves) {
    const int un = u + w.nwaves;
    const int4 itn = un < w.units ? items[un] : it;
    int64_t p0, p1;
    split_pairs(it, heads, bn, p0, p1);
    for (int64_t q0 = p0 + sub; q0 < p1; q0 += NP * PPP) {   // a pair's TPR lanes share it
      bf16x8 x[NP], y[NP];
#pragma unroll
      for (int k = 0; k < NP; ++k) {
        const int64_t pair = q0 + k * PPP;
        if (pair < p1) {
          x[k] = *reinterpret_cast<const bf16x8*>(o + pair * D + part * 8);
          y[k] = *reinterpret_cast<const bf16x8*>(d_o + pair * D + part * 8);
        }
      }
#pragma unroll
      for (int k = 0; k < NP; ++k) {
        const int64_t pair = q0 + k * PPP;
        if (pair < p1) {
          float s = 0.f;
#pragma unroll
          for (int e = 0; e < 8; ++e) s += (float)x[k][e] * (float)y[k][e];
#pragma unroll
          for (int m = TPR / 2; m >= 1; m >>= 1) s += __shfl_xor(s, m);
          if (part == 0) {
            const int64_t row = pair / heads;
            const int64_t i = (pair - row * heads) * rows + row;   // [head][row]
            rowstat[i] = make_float2(lse[i] * kLog2e, s);
          }
          float4* acc = reinterpret_cast<float4*>(dq_acc + pair * D + part * 8);
          acc[0] = make_float4(0.f, 0.f, 0.f, 0.f);
          acc[1] = make_float4(0.f, 0.f, 0.f, 0.f);
        }
      }
    }
    it = itn;
  }
}

// ---------------------------------------------------------------------------
// 3./4. tile kernel
// ---------------------------------------------------------------------------
struct BwdArgs {
  const bf16* q;
  const bf16* k;
  const bf16* v;
  const bf16* d_o;
  const float2* rowstat;
  const float* lse;   // [heads][rows], read directly when every tile holds a whole sequence
  const void* offsets;
  int off64;
  int heads;
  int q_len;
  int64_t rows;
  float scale_log2;
  float scale;
  float* dq_acc;
  bf16* dq;        // written directly when every tile holds a whole sequence
  bf16* dk;
  bf16* dv;
  const int4* items;
  int* meta;
  int sched;
  // rotary conjugate of dK (null cos: none); tables [max_pos][D/2], key positions [T]
  const float* rope_cos;
  const float* rope_sin;
  const int* rope_pos_k;
  const int* rope_pos_q;   // query positions (the single-tile path rotates dQ itself)
  int rope_max_pos;
};

// LDS offsets below are byte offsets from the start of the kernel's LDS block.  A
// lane's part of every access pattern lives in one VGPR; runtime tile offsets
// (buffer parity, wave, dS^T slot) are multiples of 256 (128 for D = 64) and are
// added to that VGPR once, which commutes with the per-read XOR of the swizzle
// (the XOR only touches the low 8 (7) bits).  Each read then costs at most one
// XOR and its constant part rides in the instruction's offset field.
// DIRECT: self-mode tiles that hold a whole sequence (the plan's second list);
// delta is formed inline and dQ is stored, not reduce-added.
// ROPE: the rotary conjugate is applied to dK in the epilogue (and to dQ where the
// tiles store it); without it none of that code is compiled in.
template <int D, int NW, bool BCAST, bool CAUSAL, bool DIRECT, bool ROPE>
struct BwdKernel {
  static constexpr int BN = 32 * NW;         // keys per tile (NW waves x 32)
  static constexpr int BQ = kBwdBQ;          // query rows per block
  static constexpr int NT = 64 * NW;
  static constexpr int DT = D / 32;          // 32-wide d tiles
  static constexpr int KS = D / 16;          // 16-deep k steps over d
  static constexpr int DTW = DT > NW ? DT / NW : 1;   // d tiles of the dQ product per wave
  // With more waves than d tiles the waves split the query blocks instead: G
  // consecutive query blocks form a group, and wave (d tile, g) computes the dQ of
  // block g of the group over all BN keys, once the whole group's dS^T is in LDS.
  static constexpr int G = DT > NW ? 1 : NW / DT;     // query blocks per dQ group
  static constexpr int NDS = G > 1 ? G + 1 : 1;      // dS^T slots (a ring when G > 1)
  static constexpr int KT_BYTES = BN * D * 2;
  static constexpr int QT_BYTES = BQ * D * 2;
  static constexpr int DS_BYTES = BN * BQ * 2;
  // per query row: (LSE log2 e, delta), or in DIRECT the forward's LSE alone
  static constexpr int ROW_BYTES = DIRECT ? BQ * 4 : BQ * 8;
  // LDS map
  static constexpr int OFF_K = 0;
  static constexpr int OFF_Q = OFF_K + KT_BYTES;              // 2 buffers
  static constexpr int OFF_DO = OFF_Q + 2 * QT_BYTES;         // 2 buffers
  static constexpr int OFF_DS = OFF_DO + 2 * QT_BYTES;        // NDS slots
  static constexpr int OFF_ROW = OFF_DS + NDS * DS_BYTES;     // 2 buffers
  static constexpr int OFF_DEL = OFF_ROW + 2 * ROW_BYTES;     // per-wave partial deltas (self mode)
  static constexpr int DEL_BYTES = DIRECT ? NW * BQ * 4 : 0;
  // The single-tile rotary path rotates dQ in its tiles: the positions of each query
  // block's rows come with the block (2 buffers of 64 dwords), and each wave copies
  // the (cos, sin) table rows of its 32 columns for the block's 32 rows into a region
  // of its own, one block ahead of the rotation.
  static constexpr bool RTAB = DIRECT && ROPE;
  static constexpr int OFF_RPOS = OFF_DEL + DEL_BYTES;
  static constexpr int RPOS_BYTES = RTAB ? 2 * 256 : 0;
  static constexpr int RTAB_WAVE = 2 * BQ * 32 * 4;            // cos, then sin: [32 rows][32 columns] fp32
  static constexpr int OFF_RTAB = OFF_RPOS + RPOS_BYTES;
  // The schedule's words: the claimed tile index and the static schedules' next plan
  // item (a 64-lane copy target).  DIRECT keeps neither here: its claimed index
  // borrows the partial-delta area, which is idle between a tile's last query block
  // and the next tile's first barrier, and its static schedules read the item from
  // memory.  That keeps the 2-wave D = 128 workgroup at 53,760 bytes, 42 of the
  // 1,280-byte LDS allocation units, so that three fit in a CU's 160 KB.
  static constexpr int OFF_ITEM = OFF_RTAB + (RTAB ? NW * RTAB_WAVE : 0);
  static constexpr int SMEM = OFF_ITEM + (DIRECT ? 0 : 256 + 4);
  static constexpr uint32_t GQ = OFF_DO - OFF_Q;              // dO tile minus Q tile, same buffer
  static constexpr int XB = D == 128 ? 256 : 128;             // the XOR-free granule
  static_assert(BN == 32 * NW && G * DT == NW * DTW && DTW <= 2, "tile shape");
  static_assert(!(DIRECT && ROPE) || (G == 1 && DTW == 2 && D == 128 && NW == 2),
                "the single-tile rotary path needs both halves of a dQ column pair in one wave");
  static_assert(OFF_Q % XB == 0 && QT_BYTES % XB == 0 && GQ % XB == 0 && (32 * 2 * D) % XB == 0 &&
                    OFF_DS % 64 == 0 && DS_BYTES % 64 == 0,
                "tile offsets must commute with the swizzle XOR");

  BwdArgs a;
  char* smem;
  int lane, wave, c32, hf;
  int64_t rs;
  int dq_dt, dq_qb;      // this wave's (first) d tile and query block of a group in the dQ product

  // per tile
  int64_t kv0;           // first K/V row of the sequence
  int64_t grow0;         // first dO / LSE row of the sequence
  int n, j0, h, q_rows;
  int nvalid;            // keys of this tile inside the sequence (1..BN)
  bool active;           // this wave owns at least one key inside the sequence
  int kpos;              // RTAB: position of this lane's key, loaded at the start of the tile
  bf16x8 vf[KS];
  f32x16 dvt[DT], dkt[DT];
  // lane parts of the LDS addresses (see row_read_base / tr_read_base)
  uint32_t row_base;     // Q / dO row reads (add the tile offset)
  uint32_t k_row_base;   // this wave's K rows
  uint32_t tr4_base;     // Q^T / dO^T transposing reads (add the tile offset)
  // One Q and one dO copy instruction per wave and query block: its lane offset is
  // computed once (QLD); other shapes compute it at each copy.
  static constexpr bool QLD = BQ / (64 / (D / 8)) == NW;
  uint32_t q_voff;
  uint32_t lds0;         // LDS address of smem

  __device__ BwdKernel(const BwdArgs& args, char* sm) : a(args), smem(sm) {
    lane = threadIdx.x & 63;
    wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform (SGPR)
    c32 = lane & 31;
    hf = lane >> 5;
    rs = (int64_t)a.heads * D;
    dq_dt = wave % (DT / DTW);   // with two d tiles a wave takes dq_dt and dq_dt + DT / 2
    dq_qb = wave / (DT / DTW);
    row_base = row_read_base<D>(lane);
    k_row_base = row_base + (uint32_t)(OFF_K + 32 * wave * 2 * D);
    tr4_base = tr_read_base<D>(lane, 4 * hf);
    if constexpr (QLD) q_voff = tile_load_voff<D>(wave, lane, (uint32_t)(rs * 2));
    lds0 = lds_addr(smem);
  }

  // Lane parts of the dQ-product, dS^T and reduce-add addresses.  They are formed
  // where they are used, from a laundered lane index, instead of being held in
  // VGPRs for the whole kernel.
  // K transposing reads of this wave's dQ slice (all BN keys):
  __device__ __forceinline__ uint32_t kq_base() const {
    const int l = (int)launder((uint32_t)lane);
    return (tr_read_base<D>(l, 8 * (l >> 5)) ^ (uint32_t)((4 * dq_dt) << 4)) + (uint32_t)OFF_K;
  }
  // dS^T tile [BN keys][BQ queries] bf16, 64-byte rows of eight 8-byte units; unit u
  // of row j is stored at u ^ ((j >> 2) & 7), which keeps both the 32-row writes
  // and the 4-row transposing reads free of bank conflicts.
  // dS^T transposing reads (all BN keys) of the block in dS^T slot `slot`:
  __device__ __forceinline__ uint32_t dsq_base(int slot) const {
    const int l = (int)launder((uint32_t)lane);
    const int t = l & 15, h2 = l >> 5;
    const int unit = 4 * ((l >> 4) & 1) + (t & 3);
    return (uint32_t)(OFF_DS + slot * DS_BYTES + (8 * h2 + (t >> 2)) * (BQ * 2) + ((unit ^ (2 * h2)) << 3));
  }
  // dS^T writes of this lane's key row into slot `slot`:
  __device__ __forceinline__ uint32_t dsw_base(int slot) const {
    const int l = (int)launder((uint32_t)lane);
    const int j = 32 * wave + (l & 31);
    return (uint32_t)(OFF_DS + slot * DS_BYTES + j * (BQ * 2) + (((l >> 5) ^ ((j >> 2) & 7)) << 3));
  }
  // dS^T slot of the query block starting at row qi0
  __device__ __forceinline__ static int ds_slot(int qi0) { return NDS > 1 ? (qi0 / BQ) % NDS : 0; }
  // byte offset of this lane's fp32 dQ element within a query block:
  __device__ __forceinline__ uint32_t dq_lane_off() const {
    const int l = (int)launder((uint32_t)lane);
    return (uint32_t)(((4 * (l >> 5)) * a.heads * D + 32 * dq_dt + (l & 31)) * 4);
  }

  __device__ __forceinline__ char* rowbuf(int b) { return smem + OFF_ROW + b * ROW_BYTES; }

  // Issues the direct LDS loads of query block [qi0, qi0 + BQ): Q and dO rows, and
  // the (LSE, delta) pairs of those rows.  Rows past the end read as zeros; the
  // masked path gives them zero weight.
  __device__ __forceinline__ void load_qblock(int qi0, int buf) { load_qblock(qi0, buf, kv0, grow0, h, q_rows); }
  __device__ __forceinline__ void load_qblock(int qi0, int buf, int64_t kv0_, int64_t grow0_, int h_, int q_rows_) {
    const int rows = min(q_rows_ - qi0, BQ);
    const uint32_t row_bytes = (uint32_t)(rs * 2);
    const uint32_t bytes = (uint32_t)rows * row_bytes;
    const bf16* qsrc = a.q + ((BCAST ? 0 : kv0_) + qi0) * rs + (int64_t)h_ * D;
    const bf16* gsrc = a.d_o + (grow0_ + qi0) * rs + (int64_t)h_ * D;
    if constexpr (QLD) {
      // (wave-uniform; stated, since the DIRECT row copy below is lane-masked)
      const uint32_t dst = __builtin_amdgcn_readfirstlane(lds0 + (uint32_t)(buf * QT_BYTES + wave * 1024));
      lds_load16_at(make_rsrc_sgpr(qsrc, bytes), q_voff, dst + (uint32_t)OFF_Q);
      lds_load16_at(make_rsrc_sgpr(gsrc, bytes), q_voff, dst + (uint32_t)OFF_DO);
    } else {
      lds_load_tile<D, NW>(smem + OFF_Q + buf * QT_BYTES, BQ, wave, lane, make_rsrc_sgpr(qsrc, bytes),
                           row_bytes);
      lds_load_tile<D, NW>(smem + OFF_DO + buf * QT_BYTES, BQ, wave, lane, make_rsrc_sgpr(gsrc, bytes),
                           row_bytes);
    }
    if constexpr (RTAB) {   // the rows' positions
      if (wave == 0) {
        const int* src = a.rope_pos_q + kv0_ + qi0;
        lds_load4(make_rsrc_sgpr(src, (uint32_t)rows * 4u), (uint32_t)lane * 4u, smem + OFF_RPOS + buf * 256);
      }
    }
    if (wave == NW - 1) {
      if constexpr (DIRECT) {   // the forward's LSE, one float per row, from BQ lanes
        const float* src = a.lse + (int64_t)h_ * a.rows + grow0_ + qi0;
        if (lane < BQ) lds_load4(make_rsrc_sgpr(src, (uint32_t)rows * 4u), (uint32_t)lane * 4u, rowbuf(buf));
      } else {                  // (LSE log2 e, delta) pairs
        const float2* src = a.rowstat + (int64_t)h_ * a.rows + grow0_ + qi0;
        lds_load4(make_rsrc_sgpr(src, (uint32_t)rows * 8u), (uint32_t)lane * 4u, rowbuf(buf));
      }
    }
  }

  // S, dP, P, dS for this wave's 32 keys, dS^T -> LDS and dV^T / dK^T accumulation.
  // With MID_BAR the barrier that retires the previous block's dS^T readers comes
  // last, right before the dS^T write (every wave reaches it, active or not);
  // otherwise the caller has passed it.
  //
  // DIRECT (every key of the sequence is in this tile): P comes from the forward's
  // LSE and delta_i = sum_j P_ij dP_ij is formed here, without a pass over O
  // ("Meta's TLX Block Attention Beats Flash Attention v2 by 2.3x on Blackwell
  // GPUs", section "One Constraint, Five Eliminations").  Each wave sums its 32 keys
  // (half_lane_sums16), the partial sums meet in LDS at a barrier (the MID_BAR one
  // when there is one), and every wave adds the NW partials of its rows.
  template <bool MASKED, bool MID_BAR>
  __device__ __forceinline__ void qblock(int buf, int qi0, int slot) {
    if (!active) {
      if constexpr (MID_BAR || DIRECT) __syncthreads();
      return;
    }
    const uint32_t boff = (uint32_t)(buf * QT_BYTES);
    bf16x8 pb[2], sb[2];
    {
      // S = Q K^T and dP = dO V^T for this wave's 32 keys (C: m = query i, n = key j).
      // Operands are read one step ahead of their MFMAs; the scheduling fences keep
      // the compiler from hoisting every read of the unrolled loop (which would push
      // the live registers past the 256 that two waves per SIMD allow).
      const uint32_t qb = launder(row_base + (uint32_t)OFF_Q + boff);
      const uint32_t kb = launder(k_row_base);
      f32x16 s = zero16(), dp = zero16();
      bf16x8 qa = lds_read8(smem, qb);
      bf16x8 kk = lds_read8(smem, kb);
      bf16x8 ga = lds_read8(smem + GQ, qb);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        bf16x8 qa_n = qa, kk_n = kk, ga_n = ga;
        if (ks + 1 < KS) {
          const uint32_t x = (uint32_t)((ks + 1) << 5);
          qa_n = lds_read8(smem, qb ^ x);
          kk_n = lds_read8(smem, kb ^ x);
          ga_n = lds_read8(smem + GQ, qb ^ x);
        }
        s = mfma32(qa, kk, s);
        dp = mfma32(ga, vf[ks], dp);
        qa = qa_n;
        kk = kk_n;
        ga = ga_n;
        __builtin_amdgcn_sched_barrier(0);
      }
      // rows past the query end, keys past the sequence end, and (causal) keys after
      // the query get zero probability
      auto visible = [&](int q4, int e) {
        const int ipos = qi0 + 8 * q4 + 4 * hf + e;
        const int jpos = j0 + 32 * wave + c32;
        bool vis = jpos < n && ipos < q_rows;
        if constexpr (CAUSAL) vis = vis && jpos <= ipos;
        return vis;
      };
      if constexpr (DIRECT) {
        const float* lsep = reinterpret_cast<const float*>(rowbuf(buf)) + 4 * hf;
        float pv[16];
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const f32x4 l4 = *reinterpret_cast<const f32x4*>(lsep + 8 * q4);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int r = 4 * q4 + e;
            float p = fast_exp2(fmaf(s[r], a.scale_log2, -(l4[e] * kLog2e)));
            if constexpr (MASKED) {
              if (!visible(q4, e)) p = 0.f;
            }
            pv[r] = p;
          }
        }
        const float part = half_lane_dots16(pv, dp, lane);
        float* del = reinterpret_cast<float*>(smem + OFF_DEL);
        if ((lane & 1) == 0) {
          const int r = (lane >> 1) & 15;
          del[wave * BQ + 8 * (r >> 2) + 4 * hf + (r & 3)] = part;
        }
        __syncthreads();   // partial deltas visible; the previous block's dS^T readers are done
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          f32x4 d4 = *reinterpret_cast<const f32x4*>(del + 8 * q4 + 4 * hf);
#pragma unroll
          for (int w = 1; w < NW; ++w) d4 += *reinterpret_cast<const f32x4*>(del + w * BQ + 8 * q4 + 4 * hf);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int r = 4 * q4 + e;
            pb[r >> 3][r & 7] = (bf16)pv[r];
            sb[r >> 3][r & 7] = (bf16)(pv[r] * (dp[r] - d4[e]));
          }
        }
      }
      // P = exp2(S c log2 e - LSE log2 e); dS = P (dP - delta) for query rows
      // 8 q4 + 4 hf + e (register r = 4 q4 + e); (rs01, rs23) hold the (LSE log2 e,
      // delta) pairs of rows e = 0, 1 and e = 2, 3
      auto softmax = [&](int q4, int e, const f32x4& rs01, const f32x4& rs23) {
        const int r = 4 * q4 + e;
        const float l2 = e < 2 ? rs01[2 * e] : rs23[2 * (e - 2)];
        const float dl = e < 2 ? rs01[2 * e + 1] : rs23[2 * (e - 2) + 1];
        float p = fast_exp2(fmaf(s[r], a.scale_log2, -l2));
        if constexpr (MASKED) {
          if (!visible(q4, e)) p = 0.f;
        }
        const float ds = p * (dp[r] - dl);
        pb[r >> 3][r & 7] = (bf16)p;
        sb[r >> 3][r & 7] = (bf16)ds;
      };
      const char* rowp = rowbuf(buf) + 32 * hf;
      f32x4 h01 = {}, h23 = {};
      if constexpr (!DIRECT) {
        // rows of query block half 0 (registers 0..7) now; those of half 1 are formed
        // between the dV / dK products of half 0, which do not depend on them
#pragma unroll
        for (int q4 = 0; q4 < 2; ++q4) {
          const f32x4 rs01 = *reinterpret_cast<const f32x4*>(rowp + 64 * q4);
          const f32x4 rs23 = *reinterpret_cast<const f32x4*>(rowp + 64 * q4 + 16);
#pragma unroll
          for (int e = 0; e < 4; ++e) softmax(q4, e, rs01, rs23);
        }
        // (LSE, delta) of q4 = 2 now, of q4 = 3 once q4 = 2 is done
        h01 = *reinterpret_cast<const f32x4*>(rowp + 128);
        h23 = *reinterpret_cast<const f32x4*>(rowp + 128 + 16);
      }
      // publish dS^T [key][query] (bf16)
      auto publish_ds = [&]() {
        const uint32_t wb = dsw_base(slot);
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          bf16x4 w;
#pragma unroll
          for (int e = 0; e < 4; ++e) w[e] = sb[q4 >> 1][4 * (q4 & 1) + e];
          *reinterpret_cast<bf16x4*>(smem + (wb ^ (uint32_t)(q4 << 4))) = w;
        }
      };
      // dV^T += dO^T P and dK^T += Q^T dS (C: m = d, n = key j); query rows
      // 16 kc + 4 (lane / 32) + e and + 8 pair with the P / dS registers
      constexpr int EPS = 8 / DT;   // half-1 softmax elements per half-0 step
      const uint32_t tb = launder(tr4_base + (uint32_t)OFF_Q + boff);
      bf16x8 g_op = lds_operand_tr<D>(smem + GQ, tb, 0, 8, 0);
      bf16x8 q_op = lds_operand_tr<D>(smem, tb, 0, 8, 0);
#pragma unroll
      for (int step = 0; step < 2 * DT; ++step) {
        const int kc = step / DT, dt = step % DT;
        bf16x8 g_n = g_op, q_n = q_op;
        if (step + 1 < 2 * DT) {
          const int kc1 = (step + 1) / DT, dt1 = (step + 1) % DT;
          g_n = lds_operand_tr<D>(smem + GQ, tb, 16 * kc1, 16 * kc1 + 8, dt1);
          q_n = lds_operand_tr<D>(smem, tb, 16 * kc1, 16 * kc1 + 8, dt1);
        }
        dvt[dt] = mfma32(g_op, pb[kc], dvt[dt]);
        if (!DIRECT && kc == 0) {
#pragma unroll
          for (int k = 0; k < EPS / 2; ++k) {
            const int el = EPS * step + k;   // 0..7 -> (q4 2 + el / 4, e el % 4)
            softmax(2 + el / 4, el % 4, h01, h23);
          }
        }
        dkt[dt] = mfma32(q_op, sb[kc], dkt[dt]);
        if (!DIRECT && kc == 0) {
#pragma unroll
          for (int k = EPS / 2; k < EPS; ++k) {
            const int el = EPS * step + k;
            softmax(2 + el / 4, el % 4, h01, h23);
          }
          if (EPS * (step + 1) == 4) {
            h01 = *reinterpret_cast<const f32x4*>(rowp + 192);
            h23 = *reinterpret_cast<const f32x4*>(rowp + 192 + 16);
          }
        }
        g_op = g_n;
        q_op = q_n;
        if constexpr (!MID_BAR || DIRECT) {   // (DIRECT: the barrier came with the deltas)
          if (step == DT - 1) publish_ds();
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      if constexpr (MID_BAR && !DIRECT) {
        __syncthreads();   // the previous block's dS^T readers are done
        publish_ds();
      }
    }
  }

  // dQ of the block whose dS^T is in slot `slot`: this wave's 32-column slice
  // (d tile dq_dt, and dq_dt + DT / 2 with two d tiles) over all BN keys.  The rows
  // of keys past the sequence end hold zeros (zero probability, or zeroed at the
  // start of the tile for waves with no key inside), so the loop needs no bounds.
  __device__ __forceinline__ void dq_compute(f32x16 (&out)[DTW], int slot) {
    const uint32_t dsb = dsq_base(slot);
    const uint32_t kb8 = kq_base();
    auto ds_op = [&](int jj) {   // dS[query l % 32][keys jj + 8 (l / 32) + e] of the part
      const uint32_t x = (uint32_t)(((jj >> 2) & 4) << 3);
      return cat(lds_read_tr(smem + ((dsb ^ x) + jj * (BQ * 2))),
                 lds_read_tr(smem + ((dsb ^ x ^ 8u) + (jj + 4) * (BQ * 2))));
    };
    if constexpr (DTW == 1) {
      // one chain: the other wave of the SIMD fills the MFMA pipe while a step waits
      // for the one before it (two chains cost 16 adds to merge)
      f32x16 acc = zero16();
      bf16x8 sa = ds_op(0);
      bf16x8 kb = lds_operand_tr<D>(smem, kb8, 0, 4, 0);
#pragma unroll
      for (int jj = 0; jj < BN; jj += 16) {
        bf16x8 sa_n = sa, kb_n = kb;
        if (jj + 16 < BN) {
          sa_n = ds_op(jj + 16);
          kb_n = lds_operand_tr<D>(smem, kb8, jj + 16, jj + 20, 0);
        }
        acc = mfma32(sa, kb, acc);
        sa = sa_n;
        kb = kb_n;
        __builtin_amdgcn_sched_barrier(0);
      }
      out[0] = acc;
    } else {
      // two d tiles, dq_dt and dq_dt + DT / 2 = dq_dt + 2 (an XOR of the chunk index
      // with 8, since dq_dt < 2), so that a lane holds columns d and d + D / 2 of its
      // rows (the pairs of the rotary conjugate): two independent chains sharing the
      // dS operand
      out[0] = zero16();
      out[DTW - 1] = zero16();
      bf16x8 sa = ds_op(0);
      bf16x8 k0 = lds_operand_tr<D>(smem, kb8, 0, 4, 0);
      bf16x8 k1 = lds_operand_tr<D>(smem, kb8, 0, 4, DT / 2);
#pragma unroll
      for (int jj = 0; jj < BN; jj += 16) {
        bf16x8 sa_n = sa, k0_n = k0, k1_n = k1;
        if (jj + 16 < BN) {
          sa_n = ds_op(jj + 16);
          k0_n = lds_operand_tr<D>(smem, kb8, jj + 16, jj + 20, 0);
          k1_n = lds_operand_tr<D>(smem, kb8, jj + 16, jj + 20, DT / 2);
        }
        out[0] = mfma32(sa, k0, out[0]);
        out[DTW - 1] = mfma32(sa, k1, out[DTW - 1]);
        sa = sa_n;
        k0 = k0_n;
        k1 = k1_n;
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }
  // Reduce-add of rows 8 g .. 8 g + 7 (g = g0 .. g0 + NG - 1) of a block's dQ slice
  // into the fp32 accumulator with buffer atomics; vals[k] holds registers 4 (g0 + k)
  // .. + 3, i.e. rows 8 g + 4 (lane / 32) + e.  One descriptor per group bounds the
  // group, so rows past the query end fall outside the buffer range and are dropped
  // by the hardware.
  template <int NG>
  __device__ __forceinline__ void dq_atomics(const f32x4 (&vals)[NG], int g0, int qi0, int dtk = 0) {
    const int rows = min(q_rows - qi0, BQ);
    if constexpr (DIRECT) {
      // the tile holds every key of these queries: dQ = c dS K is final, one bf16 per
      // (row, column) with the same row grouping and bounds
      const uint32_t row_bytes = (uint32_t)(a.heads * D * 2);
      bf16* base = a.dq + ((kv0 + qi0) * a.heads + h) * D;
      const uint32_t o0 = (dq_lane_off() >> 1) + (uint32_t)(D / 2 * 2) * dtk;   // fp32 -> bf16 offset
      const uint32_t o[4] = {o0, o0 + row_bytes, o0 + 2 * row_bytes, o0 + 3 * row_bytes};
#pragma unroll
      for (int k = 0; k < NG; ++k) {
        const int g = g0 + k;
        const int grow = max(rows - 8 * g, 0);
        const rsrc_t out = make_rsrc(base + (int64_t)(8 * g) * a.heads * D, (uint32_t)grow * row_bytes);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const bf16 v = (bf16)(vals[k][e] * a.scale);
          __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(unsigned short, v), out, o[e], 0, 0);
        }
      }
      return;
    }
    const int64_t qrow0 = BCAST ? (int64_t)(blockIdx.x & (kDqStripes - 1)) * a.q_len + qi0 : kv0 + qi0;
    const uint32_t row_bytes = (uint32_t)(a.heads * D * 4);
    float* base = a.dq_acc + (qrow0 * a.heads + h) * D;
    const uint32_t o0 = dq_lane_off() + (uint32_t)(D / 2 * 4) * dtk;   // second d tile: + D / 2 columns
    const uint32_t o[4] = {o0, o0 + row_bytes, o0 + 2 * row_bytes, o0 + 3 * row_bytes};
#pragma unroll
    for (int k = 0; k < NG; ++k) {
      const int g = g0 + k;
      const int grow = max(rows - 8 * g, 0);
      const rsrc_t acc = make_rsrc(base + (int64_t)(8 * g) * a.heads * D, (uint32_t)grow * row_bytes);
#pragma unroll
      for (int e = 0; e < 4; ++e)
        __builtin_amdgcn_raw_ptr_buffer_atomic_fadd_f32(vals[k][e], acc, o[e], 0, 0);
    }
  }
  // dQ of the query block starting at row qi0 (its dS^T in LDS): reduce-add (or
  // store) every row of this wave's d tile(s).
  __device__ __forceinline__ void dq_block(int qi0) {
    f32x16 dq[DTW];
    dq_compute(dq, ds_slot(qi0));
    if constexpr (RTAB) rope_conjugate_dq(dq);
#pragma unroll
    for (int k = 0; k < DTW; ++k) {
      const f32x4 v[4] = {{dq[k][0], dq[k][1], dq[k][2], dq[k][3]},
                          {dq[k][4], dq[k][5], dq[k][6], dq[k][7]},
                          {dq[k][8], dq[k][9], dq[k][10], dq[k][11]},
                          {dq[k][12], dq[k][13], dq[k][14], dq[k][15]}};
      dq_atomics<4>(v, 0, qi0, k);
    }
  }
  // The dQ of a group of `cnt` query blocks from row g0: wave (d tile, g) takes
  // block g.
  __device__ __forceinline__ void dq_group(int g0, int cnt) {
    if (dq_qb < cnt) dq_block(g0 + dq_qb * BQ);
  }
  // reduce-adds (or stores) one wave issues for one query block
  static constexpr int DQ_OPS = 16 * DTW;

  // Query-block loop.  Iteration t issues the LDS loads of block t + 1, runs the dQ
  // products of the pending group once it is complete (G blocks whose dS^T has been
  // in LDS since the previous closing barrier), then block t.  With G = 1 the
  // barrier that retires the readers of the one dS^T slot sits inside block t,
  // before its dS^T write; with G > 1 the blocks' dS^T go round a ring of G + 1
  // slots, so that block t never writes a slot the products of its iteration read,
  // and one barrier per block remains.  Vector memory operations retire in issue
  // order, so the wait before the closing barrier (for the loads) leaves the
  // reduce-adds issued after them in flight; the last block loads nothing and does
  // not wait.  (gfirst, npend): first row and count of the blocks whose dQ is
  // still to be formed.
  template <bool MASKED>
  __device__ __forceinline__ void run(int qs, int qe, int q_last, int& gfirst, int& npend) {
    for (int qi0 = qs; qi0 < qe; qi0 += BQ) {
      const int buf = (qi0 / BQ) & 1;
      const bool group = npend == G;   // wave-uniform
      // With the rotary conjugate in the single-tile path the dQ of the pending block
      // reads table entries: done before the next block's loads are issued, so that
      // waiting for those entries does not wait for the loads (vector memory
      // operations complete in order).
      constexpr bool kDqFirst = DIRECT && ROPE;
      if constexpr (kDqFirst) {
        if (group) dq_group(gfirst, G);
        // this block's table rows, for its rotation in the next iteration (the
        // rotation just done has read the region)
        issue_rope_tables(buf);
      }
      if (qi0 + BQ < q_last) load_qblock(qi0 + BQ, buf ^ 1);   // one block ahead
      if (!kDqFirst && group) dq_group(gfirst, G);
      qblock<MASKED, G == 1>(buf, qi0, ds_slot(qi0));
      if (group) npend = 0;
      if (npend == 0) gfirst = qi0;
      ++npend;
      if (qi0 + BQ < q_last) {   // the next block's loads must have landed
        if (!kDqFirst && group) {
          wait_vmcnt<DQ_OPS>();   // the reduce-adds issued after them stay in flight
        } else {
          wait_lds_loads();
        }
      }
      __syncthreads();
    }
  }

  // Geometry of a tile from its plan item (sequence, key block, first row, length).
  struct Geo {
    int64_t kv0;
    int b, n, j0, h;
  };
  __device__ __forceinline__ Geo geometry(int4 it, int head) const {
    Geo g;
    g.b = __builtin_amdgcn_readfirstlane(it.x);
    g.j0 = __builtin_amdgcn_readfirstlane(it.y) * BN;
    g.kv0 = __builtin_amdgcn_readfirstlane(it.z);
    g.n = __builtin_amdgcn_readfirstlane(it.w);
    g.h = head;
    return g;
  }

  // Issues the loads of a tile's K (direct to LDS; rows past the end read as zeros
  // and are masked) and of this wave's V fragment (to registers, zeros past the end).
  // The caller ensures that nobody reads the K region, or vf, meanwhile.
  __device__ __forceinline__ void issue_k(const Geo& g) {
    const int nv = min(g.n - g.j0, BN);
    lds_load_tile<D, NW>(smem + OFF_K, BN, wave, lane,
                         make_rsrc_sgpr(a.k + (g.kv0 + g.j0) * rs + (int64_t)g.h * D, (uint32_t)(nv * rs * 2)),
                         (uint32_t)(rs * 2));
  }
  __device__ __forceinline__ void issue_v(const Geo& g) {
    const int nv = min(g.n - g.j0, BN);
    const int nw = min(max(nv - 32 * wave, 0), 32);   // this wave's keys inside the sequence
    const rsrc_t vr = make_rsrc(a.v + (g.kv0 + g.j0 + 32 * wave) * rs + (int64_t)g.h * D,
                                (uint32_t)(nw * rs * 2));
    const uint32_t l = launder((uint32_t)lane);
    const uint32_t vo = (l & 31) * (uint32_t)(rs * 2) + 16u * (l >> 5);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      vf[ks] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(vr, vo + 32u * ks, 0, 0));
  }
  __device__ __forceinline__ void issue_kv(const Geo& g) {
    issue_k(g);
    issue_v(g);
  }
  // First query block that sees a tile's keys, and its buffer.
  __device__ __forceinline__ static int first_qblock(const Geo& g) {
    if constexpr (CAUSAL) return (g.j0 / BQ) * BQ;
    return 0;
  }
  __device__ __forceinline__ static int first_qbuf(const Geo& g) { return (first_qblock(g) / BQ) & 1; }
  // Issues the loads of a tile's first query block.
  __device__ __forceinline__ void issue_q0(const Geo& g) {
    const int qr = BCAST ? a.q_len : g.n;
    const int qs = first_qblock(g);
    if (qs < qr) load_qblock(qs, first_qbuf(g), g.kv0, BCAST ? (int64_t)g.b * a.q_len : g.kv0, g.h, qr);
  }

  // Epilogue slots: wave 0 stages through the query buffer that the next tile's
  // first block leaves free, wave 1 through the matching dO buffer, the others
  // through the dS^T slots; EPI_PASSES splits a slot's 32 rows so that they fit.
  static constexpr int EPI_PASSES =
      (NW - 2) * 32 * 2 * D <= NDS * DS_BYTES ? 1 : ((NW - 2) * 16 * 2 * D <= NDS * DS_BYTES ? 2 : 4);
  static constexpr int SLOT_BYTES = 32 * 2 * D / EPI_PASSES;
  static_assert((NW - 2) * SLOT_BYTES <= NDS * DS_BYTES && SLOT_BYTES <= QT_BYTES,
                "epilogue slots must fit in the free query buffers and the dS^T slots");
  static constexpr int EPI_STORES = 2 * (D / 16);   // store instructions of one epilogue
  static_assert(!RTAB || SLOT_BYTES >= 2 * 32 * 32 * 4, "the slot holds dK's second table rows");
  __device__ __forceinline__ char* epilogue_slot(int free_buf) const {
    if (wave == 0) return smem + OFF_Q + free_buf * QT_BYTES;
    if (wave == 1) return smem + OFF_DO + free_buf * QT_BYTES;
    return smem + OFF_DS + (wave - 2) * SLOT_BYTES;
  }

  // Copies the (cos, sin) table rows of the query block in buffer `buf` (its rows'
  // positions are in LDS since the barrier that published the block) for this wave's
  // 32 columns, 32 dq_dt .. 32 dq_dt + 31, into the wave's table region: copy i takes
  // rows 8 i .. 8 i + 7, lane l row 8 i + l / 8 and columns 4 (l % 8) .. + 3.  Only
  // this wave reads the region, after its own wait for these loads.
  __device__ __forceinline__ void issue_rope_tables(int buf) {
    if constexpr (RTAB) {
      const int* pos = reinterpret_cast<const int*>(smem + OFF_RPOS + buf * 256);
      const uint32_t l = launder((uint32_t)lane);
      const uint32_t col = (uint32_t)(32 * dq_dt) + 4u * (l & 7);
      const uint32_t bytes = (uint32_t)min((int64_t)a.rope_max_pos * (D / 2) * 4, (int64_t)0xFFFFFFFF);
      const u32x4 rc = make_rsrc_sgpr(a.rope_cos, bytes), rsn = make_rsrc_sgpr(a.rope_sin, bytes);
      const uint32_t dst = lds0 + (uint32_t)(OFF_RTAB + wave * RTAB_WAVE);
#pragma unroll
      for (int i = 0; i < BQ / 8; ++i) {
        const int p = min(max(pos[8 * i + (int)(l >> 3)], 0), a.rope_max_pos - 1);
        const uint32_t voff = ((uint32_t)p * (uint32_t)(D / 2) + col) * 4u;   // < 2^32 for max_pos <= 2^24
        lds_load16_at(rc, voff, dst + (uint32_t)(i * 1024));
        lds_load16_at(rsn, voff, dst + (uint32_t)(BQ * 32 * 4 + i * 1024));
      }
    }
  }

  // Rotary conjugate of a query block's dQ in the single-tile path, where the tile
  // stores dQ itself: with two d tiles per wave, register r of dq[0] and dq[1] holds
  // columns d = 32 dq_dt + lane % 32 and d + D / 2 of row
  // 8 (r / 4) + 4 (lane / 32) + r % 4 (the MFMA C layout), the rotated pair; the
  // (cos, sin) entries of (row, d) are in the wave's table region.
  __device__ __forceinline__ void rope_conjugate_dq(f32x16 (&dq)[DTW]) {
    const float* tc = reinterpret_cast<const float*>(smem + OFF_RTAB + wave * RTAB_WAVE) + c32;
    const float* ts = tc + BQ * 32;
#pragma unroll
    for (int r0 = 0; r0 < 16; r0 += 8) {
      float c[8], sn[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int r = r0 + i;
        const int row = 8 * (r >> 2) + 4 * hf + (r & 3);
        c[i] = tc[row * 32];
        sn[i] = ts[row * 32];
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int r = r0 + i;
        const float lo = dq[0][r], hi = dq[DTW - 1][r];
        dq[0][r] = lo * c[i] + hi * sn[i];
        dq[DTW - 1][r] = hi * c[i] - lo * sn[i];
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // Copies the (cos, sin) table rows of this wave's 32 keys (positions kpos; lane
  // c32 holds key c32), columns 32 cp .. 32 cp + 31, to the LDS address dst: cos, then
  // sin 4 KB further, each [32 keys][8 chunks of 4 columns] with chunk c of key r at
  // slot c ^ (r & 7), so that the rotation's reads of one chunk for 32 keys spread
  // over the banks.  Copy i takes keys 8 i .. 8 i + 7: lane l fills slot l % 8 of key
  // 8 i + l / 8.
  __device__ __forceinline__ void issue_rope_k_tables(uint32_t dst, int cp) {
    if constexpr (RTAB) {
      const uint32_t l = launder((uint32_t)lane);
      const uint32_t bytes = (uint32_t)min((int64_t)a.rope_max_pos * (D / 2) * 4, (int64_t)0xFFFFFFFF);
      const u32x4 rc = make_rsrc_sgpr(a.rope_cos, bytes), rsn = make_rsrc_sgpr(a.rope_sin, bytes);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 8 * i + (int)(l >> 3);
        const int p = min(max(__shfl(kpos, r), 0), a.rope_max_pos - 1);
        const uint32_t c = (l & 7) ^ (uint32_t)(r & 7);
        const uint32_t voff = ((uint32_t)p * (uint32_t)(D / 2) + 32u * (uint32_t)cp + 4u * c) * 4u;
        lds_load16_at(rc, voff, dst + (uint32_t)(i * 1024));
        lds_load16_at(rsn, voff, dst + (uint32_t)(4096 + i * 1024));
      }
    }
  }
  // The conjugate of dK^T (as rope_conjugate_dk) with the table rows of d tiles
  // (0, 2) at t0 and of d tiles (1, 3) at t1, laid out by issue_rope_k_tables.
  __device__ __forceinline__ void rope_conjugate_dk_lds(const char* t0, const char* t1) {
#pragma unroll
    for (int dt = 0; dt < DT / 2; ++dt) {
      const char* t = dt == 0 ? t0 : t1;
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int chunk = 2 * q4 + hf;   // columns 8 q4 + 4 hf .. + 3 of the pair's 32
        const int off = c32 * 128 + ((chunk ^ (c32 & 7)) << 4);
        const f32x4 c4 = *reinterpret_cast<const f32x4*>(t + off);
        const f32x4 s4 = *reinterpret_cast<const f32x4*>(t + 4096 + off);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 4 * q4 + e;
          const float lo = dkt[dt][r], hi = dkt[dt + DT / 2][r];
          dkt[dt][r] = lo * c4[e] + hi * s4[e];
          dkt[dt + DT / 2][r] = hi * c4[e] - lo * s4[e];
        }
      }
    }
  }

  // Rotary conjugate of this wave's dK^T accumulators, in fp32 before the bf16
  // rounding ("Meta's TLX Block Attention Beats Flash Attention v2 by 2.3x on
  // Blackwell GPUs", section "The Rotary Fusion Bonus").  The pair (d, d + D/2) of
  // the lane's key row sits in the same register of d tiles dt and dt + DT/2:
  //   dk[d] = g[d] cos + g[d + D/2] sin,  dk[d + D/2] = g[d + D/2] cos - g[d] sin
  // with (cos, sin) of the key's position; register r of d tile dt holds
  // d = 32 dt + 8 (r / 4) + 4 (lane / 32) + r % 4, so four consecutive table entries
  // serve four registers.
  __device__ __forceinline__ void rope_conjugate_dk() {
    int pos = kpos;
    if constexpr (!RTAB) {   // (the multi-tile variants have no register to hold it across the tile)
      const int j = j0 + 32 * wave + c32;
      pos = j < n ? a.rope_pos_k[kv0 + j] : 0;
    }
    pos = min(max(pos, 0), a.rope_max_pos - 1);
    const float* cr = a.rope_cos + (int64_t)pos * (D / 2);
    const float* sr = a.rope_sin + (int64_t)pos * (D / 2);
    // one d-tile pair at a time: its 32 table values are loaded together, then used
    // (the epilogue holds little register room)
#pragma unroll
    for (int dt = 0; dt < DT / 2; ++dt) {
      constexpr int QG = RTAB ? 4 : 2;   // table quads loaded together (fewer where registers are short)
#pragma unroll
      for (int qg = 0; qg < 4; qg += QG) {
        f32x4 c4[QG], s4[QG];
#pragma unroll
        for (int k = 0; k < QG; ++k) {
          const int d0 = 32 * dt + 8 * (qg + k) + 4 * hf;
          c4[k] = *reinterpret_cast<const f32x4*>(cr + d0);
          s4[k] = *reinterpret_cast<const f32x4*>(sr + d0);
        }
#pragma unroll
        for (int r = 4 * qg; r < 4 * (qg + QG); ++r) {
          const float c = c4[r / 4 - qg][r % 4], sn = s4[r / 4 - qg][r % 4];
          const float lo = dkt[dt][r], hi = dkt[dt + DT / 2][r];
          dkt[dt][r] = lo * c + hi * sn;
          dkt[dt + DT / 2][r] = hi * c - lo * sn;
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }

  // One tile whose K/V and first query block loads have been issued (`first`: by
  // the kernel prologue, so nothing else is in flight).  `pre` runs after the first
  // barrier.  After the query loop `next(ng)` names the following tile (or returns
  // false); its V fragment (vf is no longer read) is loaded during the last dQ
  // product, and its K tile and first query block once every wave is past that
  // product, before this tile's dK / dV leave.
  template <class Pre, class Next>
  __device__ __forceinline__ bool process(const Geo& g, bool first, Pre&& pre, Next&& next, Geo& ng) {
    h = g.h;
    kv0 = g.kv0;
    n = g.n;
    j0 = g.j0;
    nvalid = min(n - j0, BN);
    active = 32 * wave < nvalid;
    q_rows = BCAST ? a.q_len : n;
    grow0 = BCAST ? (int64_t)g.b * a.q_len : kv0;
    if constexpr (RTAB) {   // used by the epilogue: the load has the whole tile to land
      const int j = j0 + 32 * wave + c32;
      kpos = j < n ? a.rope_pos_k[kv0 + j] : 0;
    }

    __syncthreads();   // the previous tile's epilogue is done with its LDS slots
    pre();
    // a wave with no key inside the sequence never writes its dS^T rows in this
    // tile: zero them once for the dQ products
    if (!active) {
#pragma unroll
      for (int slot = 0; slot < NDS; ++slot) {
        const uint32_t wb = dsw_base(slot);
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4)
          *reinterpret_cast<bf16x4*>(smem + (wb ^ (uint32_t)(q4 << 4))) = bf16x4{};
      }
      // nor its partial deltas
      if (DIRECT && lane < BQ) reinterpret_cast<float*>(smem + OFF_DEL)[wave * BQ + lane] = 0.f;
    }
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      dvt[dt] = zero16();
      dkt[dt] = zero16();
    }
    // query rows that can see this tile's keys; their first block was issued with
    // the tile's K/V, before the previous tile's epilogue, whose row stores may stay
    // in flight
    const int qs = first_qblock(g);
    const int q_last = q_rows;
    if (first) {
      wait_lds_loads();
    } else {
      wait_vmcnt<EPI_STORES>();
    }
    __syncthreads();
    // Peeled loops: query blocks that need a mask (causal diagonal, a partial K/V
    // block at the sequence end, or a partial last query block) run apart from the
    // branch-free bulk.
    const bool kv_tail = j0 + BN > n;
    int qm = qs;
    if constexpr (CAUSAL) qm = min(q_last, ((j0 + BN - 1 + BQ - 1) / BQ) * BQ);
    if (kv_tail) qm = q_last;
    const int qfull = max(qm, (q_last / BQ) * BQ);
    int gfirst = 0, npend = 0;   // query blocks whose dQ is still to be formed
    run<true>(qs, qm, q_last, gfirst, npend);
    run<false>(qm, qfull, q_last, gfirst, npend);
    run<true>(qfull, q_last, q_last, gfirst, npend);
    const bool more = next(ng);
    char* slot = epilogue_slot(more ? first_qbuf(ng) ^ 1 : 0);
    constexpr bool kDqFirst = DIRECT && ROPE;   // as in run(): the table reads go first
    if (more && !kDqFirst) issue_v(ng);
    if constexpr (RTAB) {
      // dK's table rows of d tiles (1, 3) into the epilogue slot (free since the
      // closing barrier: the next tile's first query block goes to the other buffer),
      // then wait for everything before them, the last block's rows included
      issue_rope_k_tables(lds_addr(slot), 1);
      wait_vmcnt<8>();
    }
    if (npend > 0) dq_group(gfirst, npend);   // the closing barrier published their dS^T
    if constexpr (RTAB) issue_rope_k_tables(lds0 + (uint32_t)(OFF_RTAB + wave * RTAB_WAVE), 0);   // d tiles (0, 2)
    if (more && kDqFirst) issue_v(ng);
    if constexpr (RTAB) {   // both copies (only the next tile's V fragment may stay in flight)
      if (more) {
        wait_vmcnt<KS>();
      } else {
        wait_lds_loads();
      }
      rope_conjugate_dk_lds(smem + OFF_RTAB + wave * RTAB_WAVE, slot);
    }
    __syncthreads();   // every wave is past its last read of the K tile, dQ partials and query blocks
    if (more) {
      issue_k(ng);
      issue_q0(ng);
    }

    // dK = c dS^T Q and dV -> bf16 rows, staged through this wave's epilogue slot
    {
      const int nrows = min(max(n - (j0 + 32 * wave), 0), 32);
      const int64_t off = (kv0 + j0 + 32 * wave) * rs + (int64_t)h * D;
      if constexpr (ROPE && !RTAB) rope_conjugate_dk();
      store_acc_rows<D, EPI_PASSES>(dkt, a.scale, slot, a.dk + off, rs, nrows, lane);
      store_acc_rows<D, EPI_PASSES>(dvt, 1.f, slot, a.dv + off, rs, nrows, lane);
    }
    return more;
  }
};

template <int D, int NW, bool BCAST, bool CAUSAL, bool DIRECT, bool ROPE>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(2)))
void bwd_kernel(BwdArgs a) {
  // The plan's lists: a DIRECT kernel takes the tiles of sequences within one tile
  // (the second list), the other the rest (the first); either may be empty.
  using K = BwdKernel<D, NW, BCAST, CAUSAL, DIRECT, ROPE>;
  using Geo = typename K::Geo;
  __shared__ __attribute__((aligned(16))) char smem[K::SMEM];
  int* const next_item = reinterpret_cast<int*>(smem + K::OFF_ITEM);   // DMA target, 16 bytes used
  int* const claimed = reinterpret_cast<int*>(smem + (DIRECT ? K::OFF_DEL : K::OFF_ITEM + 256));
  K kern(a, smem);
  const int num_wg = gridDim.x;
  const int lwg = xcd_logical_wg(blockIdx.x, num_wg);
  const int ntiles = __builtin_amdgcn_readfirstlane(DIRECT ? a.meta[3] : a.meta[2]);
  const int4* const items = a.items + (DIRECT ? __builtin_amdgcn_readfirstlane(a.meta[5]) : 0);
  int* const counter = a.meta + (DIRECT ? 4 : 1);
  const bool dyn = a.sched == kDynamic;
  auto claim = [&]() {
    if (threadIdx.x == 0) *claimed = atomicAdd(counter, 1);
    __syncthreads();
    const int v = *claimed;
    __syncthreads();
    return v;
  };
  int idx = dyn ? claim() : lwg;
  if (idx >= ntiles) return;
  Geo g = kern.geometry(items[idx / a.heads], idx % a.heads);
  kern.issue_kv(g);
  kern.issue_q0(g);
  for (bool first = true;; first = false) {
    // static schedules know the next tile now: outside DIRECT its item is copied
    // into LDS while this tile runs (the copy completes at this tile's first load wait)
    int nidx = dyn ? -1 : idx + num_wg;
    auto pre = [&]() {
      if (!DIRECT && !dyn && nidx < ntiles && kern.wave == 0)
        lds_load4(make_rsrc_sgpr(items + nidx / a.heads, 16u), (uint32_t)kern.lane * 4u,
                  reinterpret_cast<char*>(next_item));
    };
    auto next = [&](Geo& out) -> bool {
      if (dyn) nidx = claim();
      if (nidx >= ntiles) return false;
      const int4 it = (dyn || DIRECT) ? items[nidx / a.heads] : *reinterpret_cast<const int4*>(next_item);
      out = kern.geometry(it, nidx % a.heads);
      return true;
    };
    Geo ng;
    if (!kern.process(g, first, pre, next, ng)) break;
    g = ng;
    idx = nidx;
  }
}

// ---------------------------------------------------------------------------
// 5. dQ finalize
// ---------------------------------------------------------------------------
// One thread per four accumulator elements of the call.
__global__ __launch_bounds__(256) void dq_finalize_kernel(const float* __restrict__ acc,
                                                          bf16* __restrict__ dq, int64_t n_vec4,
                                                          int64_t stripe_vec4, int stripes, float scale) {
  const float4* a4 = reinterpret_cast<const float4*>(acc);
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n_vec4) return;
  float4 s = a4[i];
  for (int k = 1; k < stripes; ++k) {
    const float4 t = a4[i + k * stripe_vec4];
    s.x += t.x;
    s.y += t.y;
    s.z += t.z;
    s.w += t.w;
  }
  bf16x4 o;
  o[0] = (bf16)(s.x * scale);
  o[1] = (bf16)(s.y * scale);
  o[2] = (bf16)(s.z * scale);
  o[3] = (bf16)(s.w * scale);
  reinterpret_cast<bf16x4*>(dq)[i] = o;
}

// The rows of a split call's first list only (self mode: one accumulator stripe);
// the single-tile kernel stored the others' dQ itself.  Walk as in
// bwd_pre_split_kernel.
template <int D>
__global__ __launch_bounds__(256) void dq_finalize_split_kernel(const float* __restrict__ acc,
                                                                bf16* __restrict__ dq, int heads, float scale,
                                                                const int4* __restrict__ items,
                                                                const int* __restrict__ meta, int bn) {
  constexpr int TPR = D / 4, PPP = 64 / TPR, NP = 16;   // lanes per pair (four columns each), pairs per pass
  SplitWalk w(meta, heads);
  const int part = w.lane % TPR, sub = w.lane / TPR;
  if (w.unit >= w.units) return;
  int4 it = items[w.unit];
  for (int u = w.unit; u < w.units; u += w.nwaves) {
    const int un = u + w.nwaves;
    const int4 itn = un < w.units ? items[un] : it;
    int64_t p0, p1;
    split_pairs(it, heads, bn, p0, p1);
    for (int64_t q0 = p0 + sub; q0 < p1; q0 += NP * PPP) {
      f32x4 v[NP];
#pragma unroll
      for (int k = 0; k < NP; ++k) {
        const int64_t pair = q0 + k * PPP;
        if (pair < p1) v[k] = *reinterpret_cast<const f32x4*>(acc + pair * D + part * 4);
      }
#pragma unroll
      for (int k = 0; k < NP; ++k) {
        const int64_t pair = q0 + k * PPP;
        if (pair < p1) {
          bf16x4 x;
#pragma unroll
          for (int e = 0; e < 4; ++e) x[e] = (bf16)(v[k][e] * scale);
          *reinterpret_cast<bf16x4*>(dq + pair * D + part * 4) = x;
        }
      }
    }
    it = itn;
  }
}

// dQ finalize with the rotary conjugate: sum of the stripes, times the softmax
// scale, rotated by the opposite angle of the query row's position, -> bf16.  One
// thread takes four columns d .. d + 3 (d = 4 g < D/2) of a (row, head) pair rh and
// their partners d + D/2 .. d + D/2 + 3.
template <int D>
__device__ __forceinline__ void finalize_rope_group(const float* __restrict__ acc, bf16* __restrict__ dq,
                                                    int64_t rh, int64_t row, int g, int64_t stripe_elems,
                                                    int stripes, float scale, const float* __restrict__ rcos,
                                                    const float* __restrict__ rsin,
                                                    const int* __restrict__ pos_q, int max_pos) {
  const int64_t e0 = rh * D + 4 * g;
  f32x4 lo = *reinterpret_cast<const f32x4*>(acc + e0);
  f32x4 hi = *reinterpret_cast<const f32x4*>(acc + e0 + D / 2);
  for (int k = 1; k < stripes; ++k) {
    lo += *reinterpret_cast<const f32x4*>(acc + e0 + k * stripe_elems);
    hi += *reinterpret_cast<const f32x4*>(acc + e0 + D / 2 + k * stripe_elems);
  }
  const int pos = min(max(pos_q[row], 0), max_pos - 1);
  const f32x4 c = *reinterpret_cast<const f32x4*>(rcos + (int64_t)pos * (D / 2) + 4 * g);
  const f32x4 sn = *reinterpret_cast<const f32x4*>(rsin + (int64_t)pos * (D / 2) + 4 * g);
  bf16x4 olo, ohi;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float a0 = lo[e] * scale, b0 = hi[e] * scale;
    olo[e] = (bf16)(a0 * c[e] + b0 * sn[e]);
    ohi[e] = (bf16)(b0 * c[e] - a0 * sn[e]);
  }
  *reinterpret_cast<bf16x4*>(dq + e0) = olo;
  *reinterpret_cast<bf16x4*>(dq + e0 + D / 2) = ohi;
}

// Every (row, head) pair of the call, one thread per four-column group.
template <int D>
__global__ __launch_bounds__(256) void dq_finalize_rope_kernel(const float* __restrict__ acc,
                                                               bf16* __restrict__ dq, int64_t rows,
                                                               int heads, int64_t stripe_elems,
                                                               int stripes, float scale,
                                                               const float* __restrict__ rcos,
                                                               const float* __restrict__ rsin,
                                                               const int* __restrict__ pos_q, int max_pos) {
  constexpr int G = D / 8;   // four-column groups in each half
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= rows * heads * G) return;
  const int64_t rh = t / G;   // row * heads + head
  finalize_rope_group<D>(acc, dq, rh, rh / heads, (int)(t - rh * G), stripe_elems, stripes, scale, rcos,
                         rsin, pos_q, max_pos);
}

// The rows of a split call's first list only, with the rotary conjugate.
template <int D>
__global__ __launch_bounds__(256) void dq_finalize_rope_split_kernel(const float* __restrict__ acc,
                                                                     bf16* __restrict__ dq, int heads,
                                                                     float scale,
                                                                     const float* __restrict__ rcos,
                                                                     const float* __restrict__ rsin,
                                                                     const int* __restrict__ pos_q,
                                                                     int max_pos, const int4* __restrict__ items,
                                                                     const int* __restrict__ meta, int bn) {
  constexpr int G = D / 8, PPP = 64 / G;   // lanes per pair, pairs per wave pass
  SplitWalk w(meta, heads);
  const int g = w.lane % G, sub = w.lane / G;
  if (w.unit >= w.units) return;
  int4 it = items[w.unit];
  for (int u = w.unit; u < w.units; u += w.nwaves) {
    const int un = u + w.nwaves;
    const int4 itn = un < w.units ? items[un] : it;   // the next item, during this one
    int64_t p0, p1;
    split_pairs(it, heads, bn, p0, p1);
    for (int64_t pair = p0 + sub; pair < p1; pair += PPP)
      finalize_rope_group<D>(acc, dq, pair, pair / heads, g, 0, 1, scale, rcos, rsin, pos_q, max_pos);
    it = itn;
  }
}

template <int D, int NW, bool BCAST, bool CAUSAL, bool DIRECT, bool ROPE>
hipError_t launch_bwd_one(const BwdArgs& a, hipStream_t s, int64_t max_tiles) {
  const void* fn = reinterpret_cast<const void*>(&bwd_kernel<D, NW, BCAST, CAUSAL, DIRECT, ROPE>);
  const int grid = persistent_grid(fn, 64 * NW, max_tiles);
  hipLaunchKernelGGL((bwd_kernel<D, NW, BCAST, CAUSAL, DIRECT, ROPE>), dim3(grid), dim3(64 * NW), 0, s, a);
  return hipGetLastError();
}
// Broadcast mode has one variant.  In a split self-mode call (maybe_single_tile)
// both are launched, each over its list of the plan (an empty list returns at once):
// which sequences fit one tile is known on the device only.  With the rotary
// conjugate the single-tile variant exists only for two d tiles per wave (D = 128,
// two waves), see single_tile_allowed.
template <int D, int NW, bool BCAST, bool CAUSAL, bool ROPE>
hipError_t launch_bwd_inst(const BwdArgs& a, hipStream_t s, int64_t max_tiles, bool maybe_single) {
  if constexpr (BCAST) {
    return launch_bwd_one<D, NW, true, false, false, ROPE>(a, s, max_tiles);
  } else {
    constexpr bool kDirect = !ROPE || (D == 128 && NW == 2);
    if constexpr (kDirect) {
      if (maybe_single) {
        const hipError_t e = launch_bwd_one<D, NW, false, CAUSAL, true, ROPE>(a, s, max_tiles);
        if (e != hipSuccess) return e;
      }
    }
    return launch_bwd_one<D, NW, false, CAUSAL, false, ROPE>(a, s, max_tiles);
  }
}

template <int D, int NW, bool ROPE>
hipError_t launch_bwd_dwr(const Problem& p, const BwdArgs& a, hipStream_t s) {
  const int64_t max_tiles = bwd_max_items(p) * p.heads;
  const bool ms = maybe_single_tile(p);
  if (p.broadcast) {
    if constexpr (NW == 8) return launch_bwd_inst<D, NW, true, false, ROPE>(a, s, max_tiles, ms);
    return hipErrorInvalidValue;   // broadcast mode always takes eight waves
  }
  if (p.causal) return launch_bwd_inst<D, NW, false, true, ROPE>(a, s, max_tiles, ms);
  return launch_bwd_inst<D, NW, false, false, ROPE>(a, s, max_tiles, ms);
}

template <int D, int NW>
hipError_t launch_bwd_dw(const Problem& p, const BwdArgs& a, hipStream_t s) {
  return p.rope ? launch_bwd_dwr<D, NW, true>(p, a, s) : launch_bwd_dwr<D, NW, false>(p, a, s);
}

template <int D>
hipError_t launch_bwd_d(const Problem& p, const BwdArgs& a, hipStream_t s) {
  const int nw = bwd_waves(p);
  if (nw == 8) return launch_bwd_dw<D, 8>(p, a, s);
  if (nw == 4) return launch_bwd_dw<D, 4>(p, a, s);
  return launch_bwd_dw<D, 2>(p, a, s);
}

}  // namespace

// Eight waves (256-key tiles) halve the dQ reduce-adds per key.  In broadcast mode
// every tile adds into the one shared dQ, so that always pays; in self mode it pays
// when a tile's query loop is long, and four waves (128-key tiles) waste less on
// short sequences.  Sequences of about 64 keys take two waves (64-key tiles, each
// wave computing two d tiles of dQ), so that no wave of a tile sits idle.
int bwd_waves(const Problem& p) {
  if (p.broadcast) return 8;
  const int64_t mean_len = p.batch > 0 ? p.total_kv / p.batch : 0;
  if (mean_len <= 96) return 2;   // 64-key tiles for short sequences
  return mean_len >= 512 ? 8 : 4;
}

// Whether the single-tile kernel may take the sequences that lie within one backward
// tile: self mode, and with the rotary conjugate only where its tiles can rotate dQ.
bool single_tile_allowed(const Problem& p) {
  // with the rotary conjugate the tiles can rotate dQ only when a lane holds both
  // halves of its columns: two d tiles per wave (D = 128, two waves)
  return !p.broadcast && (!p.rope || (p.head_dim == 128 && bwd_waves(p) == 2));
}

// Whether the plan splits the tiles between the single-tile kernel and the
// reduce-adding one: where the single-tile kernel may run and the mean length is at
// most 9/8 of a tile.  The split pays when most rows belong to sequences of one tile
// (its delta pass and dQ finalize walk the longer sequences' items, which is slower
// per row than the all-rows kernels); the mean is all the host knows, and up to 9/8
// of a tile it still admits a batch of one-tile sequences with a few longer ones.
bool maybe_single_tile(const Problem& p) {
  if (!single_tile_allowed(p)) return false;
  return p.total_kv * 8 <= (int64_t)p.batch * 32 * bwd_waves(p) * 9;
}

int64_t bwd_max_items(const Problem& p) {
  const int bn = 32 * bwd_waves(p);
  return (p.total_kv + bn - 1) / bn + p.batch;
}

// Grid of the split-mode row kernels: workgroups that take (item, head) units in turn.
static unsigned split_grid(const Problem& p) {
  const int64_t units = bwd_max_items(p) * p.heads;
  return (unsigned)std::max<int64_t>(1, std::min<int64_t>(units, (int64_t)device_cu_count() * 64));
}

hipError_t launch_bwd_pre(const Problem& p, const void* o, const void* d_o, const float* lse,
                          float* rowstat, float* dq_acc, int64_t dq_acc_elems, const Plan& plan,
                          hipStream_t s) {
  float2* rs2 = reinterpret_cast<float2*>(rowstat);
  const bf16* o16 = static_cast<const bf16*>(o);
  const bf16* g16 = static_cast<const bf16*>(d_o);
  if (maybe_single_tile(p)) {   // the plan split the tiles: rows of the first list only
    auto go = [&](auto kernel) {
      hipLaunchKernelGGL(kernel, dim3(split_grid(p)), dim3(256), 0, s, o16, g16, lse, rs2, p.rows, p.heads,
                         dq_acc, plan.items, plan.meta, 32 * bwd_waves(p));
    };
    p.head_dim == 128 ? go(bwd_pre_split_kernel<128>) : go(bwd_pre_split_kernel<64>);
    return hipGetLastError();
  }
  const int64_t pairs = p.rows * p.heads;
  const int tpr = p.head_dim / 8;
  int64_t blocks = (pairs * tpr + 255) / 256;
  if (blocks < 1) blocks = 1;
  const int64_t vec4 = dq_acc_elems / 4;
  auto go = [&](auto kernel) {
    hipLaunchKernelGGL(kernel, dim3((unsigned)blocks), dim3(256), 0, s, o16, g16, lse, rs2, p.rows, p.heads,
                       dq_acc, vec4);
  };
  p.head_dim == 128 ? go(bwd_pre_kernel<128>) : go(bwd_pre_kernel<64>);
  return hipGetLastError();
}

hipError_t launch_bwd(const Problem& p, const Plan& plan, int sched, const float* rowstat,
                      const float* lse, const void* d_o, float* dq_acc, void* dq, void* dk, void* dv,
                      const Rope& rope, hipStream_t s) {
  BwdArgs a;
  a.q = static_cast<const bf16*>(p.q);
  a.k = static_cast<const bf16*>(p.k);
  a.v = static_cast<const bf16*>(p.v);
  a.d_o = static_cast<const bf16*>(d_o);
  a.rowstat = reinterpret_cast<const float2*>(rowstat);
  a.lse = lse;
  a.offsets = p.offsets;
  a.off64 = p.off64;
  a.heads = p.heads;
  a.q_len = p.q_len;
  a.rows = p.rows;
  a.scale_log2 = p.scale * kLog2e;
  a.scale = p.scale;
  a.dq_acc = dq_acc;
  a.dq = static_cast<bf16*>(dq);
  a.dk = static_cast<bf16*>(dk);
  a.dv = static_cast<bf16*>(dv);
  a.rope_cos = rope.cos;
  a.rope_sin = rope.sin;
  a.rope_pos_k = rope.pos_k;
  a.rope_pos_q = rope.pos_q;
  a.rope_max_pos = rope.max_pos;
  a.items = plan.items;
  a.meta = plan.meta;
  a.sched = sched;
  return p.head_dim == 128 ? launch_bwd_d<128>(p, a, s) : launch_bwd_d<64>(p, a, s);
}

hipError_t launch_dq_finalize(const Problem& p, const float* dq_acc, void* dq, const Plan& plan,
                              const Rope& rope, hipStream_t s) {
  bf16* dq16 = static_cast<bf16*>(dq);
  if (maybe_single_tile(p)) {   // the plan split the tiles: rows of the first list only
    const int bn = 32 * bwd_waves(p);
    if (rope.cos != nullptr) {
      auto go = [&](auto kernel) {
        hipLaunchKernelGGL(kernel, dim3(split_grid(p)), dim3(256), 0, s, dq_acc, dq16, p.heads, p.scale,
                           rope.cos, rope.sin, rope.pos_q, rope.max_pos, plan.items, plan.meta, bn);
      };
      p.head_dim == 128 ? go(dq_finalize_rope_split_kernel<128>) : go(dq_finalize_rope_split_kernel<64>);
    } else {
      auto go = [&](auto kernel) {
        hipLaunchKernelGGL(kernel, dim3(split_grid(p)), dim3(256), 0, s, dq_acc, dq16, p.heads, p.scale,
                           plan.items, plan.meta, bn);
      };
      p.head_dim == 128 ? go(dq_finalize_split_kernel<128>) : go(dq_finalize_split_kernel<64>);
    }
    return hipGetLastError();
  }
  const int64_t q_rows = p.broadcast ? p.q_len : p.total_kv;
  const int64_t n = q_rows * p.heads * p.head_dim;
  const int stripes = p.broadcast ? kDqStripes : 1;
  if (rope.cos != nullptr) {
    const int64_t blocks = (q_rows * p.heads * (p.head_dim / 8) + 255) / 256;
    if (blocks == 0) return hipSuccess;
    auto go = [&](auto kernel) {
      hipLaunchKernelGGL(kernel, dim3((unsigned)blocks), dim3(256), 0, s, dq_acc, dq16, q_rows, p.heads, n,
                         stripes, p.scale, rope.cos, rope.sin, rope.pos_q, rope.max_pos);
    };
    p.head_dim == 128 ? go(dq_finalize_rope_kernel<128>) : go(dq_finalize_rope_kernel<64>);
    return hipGetLastError();
  }
  const int64_t vec4 = n / 4;
  const int64_t blocks = (vec4 + 255) / 256;
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL(dq_finalize_kernel, dim3((unsigned)blocks), dim3(256), 0, s, dq_acc, dq16, vec4, vec4,
                     stripes, p.scale);
  return hipGetLastError();
}

}  // namespace jfa
