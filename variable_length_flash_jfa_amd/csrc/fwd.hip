// Jagged Flash Attention forward for gfx950.
//
// Exact softmax attention on packed sequences addressed through offsets, with
// the broadcast-Q mode (one dense query sequence for every sequence) and jagged
// self-attention, optionally causal ("Meta's TLX attention kernel outpaces
// FlashAttention-4 on B200", section "GEM's sequences do not fit a fixed grid").
//
// Structure (MI355X design; the pages' Blackwell kernel is prior art only):
//  * persistent workgroups walk a device-built tile list (sorted by K/V work and
//    dealt boustrophedon, or round-robin, or claimed through an atomic counter;
//    section "Five changes unlocked the gains", items 1 and 2); in broadcast mode
//    the counter is split by (query block, head) class, one class per workgroup,
//    so that a workgroup's Q fragment stays in registers from tile to tile;
//  * a tile is (sequence, block of 32*NW query rows, head); each 64-lane wave owns
//    32 query rows, keeps its Q fragment in registers and computes
//    S^T = K Q^T and O^T += V^T P^T with v_mfma_f32_32x32x16_bf16, so that the
//    fp32 score accumulator is already laid out as the bf16 P operand;
//  * K/V blocks of 64 keys stream straight from HBM into swizzled LDS (gfx950
//    direct global->LDS loads, double buffered) one block ahead of the MFMA work,
//    across tile boundaries too: the next tile's first block and Q fragment load
//    during the current tile's last block and epilogue;
//    V^T operands come from the gfx950 transposing LDS read;
//  * online softmax in the exp2 domain with a running max and a lane-local running
//    sum (the two halves of a wave hold the two halves of a row's keys and are
//    combined once, at the end), one step per 32-key half block, each half's
//    softmax interleaved with the other half's MFMA chain; the max moves (and O is
//    rescaled) only when it would grow by more than a factor 2^8;
//  * the K/V loop is peeled: a branch-free bulk loop over fully visible blocks,
//    then a masked loop over the tail block and the causal diagonal (section
//    "Five changes unlocked the gains", item 5);
//  * epilogue O /= l -> bf16 and LSE = (m + log2 l) ln 2 -> fp32 ("Meta's TLX Block
//    Attention Beats Flash Attention v2 by 2.3x on Blackwell GPUs", section "One
//    Constraint, Five Eliminations", on the saved log-sum-exp).
#include "jfa_device.h"
#include "jfa_internal.h"

namespace jfa {
namespace {

struct FwdArgs {
  const bf16* q;
  const bf16* k;
  const bf16* v;
  const void* offsets;
  int off64;
  int heads;
  int q_len;
  int64_t rows;
  float scale_log2;
  bf16* o;
  float* lse;
  const int4* items;
  int* meta;
  int sched;
  // broadcast mode, dynamic schedule: tile classes (query block, head), each with a
  // counter of its own (0: one counter for all tiles)
  int classes;
  // block-sparse forward: [tiles][topk] selected key blocks (ascending) per tile
  const int* tile_blocks;
  int topk;
};

// SPARSE: the block-sparse forward (no causal mask); a tile visits only the key
// blocks its selection lists, read from a per-tile list in LDS (`lists`, two
// buffers of 64 entries: the current tile's and the next one's).
template <int D, int NW, bool BCAST, bool CAUSAL, bool SPARSE = false>
struct FwdKernel {
  static constexpr int BN = kFwdBN;
  static constexpr int BM = 32 * NW;
  static constexpr int NT = 64 * NW;
  static constexpr int CH = D / 8;               // 16-byte chunks per row
  static constexpr int TILE_BYTES = BN * D * 2;
  static constexpr int DT = D / 32;              // 32-wide d tiles of O
  static constexpr int KS = D / 16;              // 16-deep k steps of Q K^T
  static constexpr int PF_S = 2;                 // operand reads in flight ahead of the S MFMAs
  static constexpr int PF_V = 3;                 // ... and of the O MFMAs
  static_assert((BN * D * 2 / 1024) % NW == 0, "a K/V block must split evenly over the waves");
  // The epilogue stages O through one K/V buffer (K and V tiles) while the next
  // tile's first block lands in the other; with eight waves it takes two passes.
  static constexpr int EPI_PASSES = NW * 32 * 2 * D > 2 * TILE_BYTES ? 2 : 1;
  static constexpr int SLOT_BYTES = 32 * 2 * D / EPI_PASSES;
  static_assert(NW * SLOT_BYTES <= 2 * TILE_BYTES, "epilogue slots must fit in one K/V buffer");

  // Tile-invariant per-wave state.
  FwdArgs a;
  char* smem;          // [2 buffers][K, V][BN x D] swizzled
  int lane, wave, c32, hf;
  int64_t rs;          // row stride (elements) of q, k, v, o

  // Tile geometry: sequence b with K/V rows [kv0, kv0 + n), query block m, head h.
  struct Geo {
    int64_t kv0;
    int n, b, m, h;
  };

  // Per-tile state.
  const int* lists = nullptr;   // SPARSE: LDS list buffers
  int lb = 0;                   // SPARSE: the current tile's list buffer
  Geo g;               // the current tile
  int q_rows, m0, i0;
  int64_t out_row0;    // first output row of the sequence
  bf16x8 qf[KS];
  f32x16 acc[DT];
  float mrun, lsum, lsum2;   // row sums of even and odd P elements (two short chains)
  uint32_t k_row_base;   // lane part of K row reads (rows 32 c + lane % 32)
  uint32_t v_tr_base;    // lane part of V^T transposing reads (k offset 4 (lane / 32))
  TileLoader<D, NW, BN> ld;   // this wave's share of a K or V block copy
  uint32_t lds0;              // LDS address of smem

  __device__ FwdKernel(const FwdArgs& args, char* sm) : a(args), smem(sm) {
    lane = threadIdx.x & 63;
    wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform (SGPR)
    c32 = lane & 31;
    hf = lane >> 5;
    rs = (int64_t)a.heads * D;
    k_row_base = row_read_base<D>(lane);
    v_tr_base = tr_read_base<D>(lane, 4 * hf);
    ld.init(wave, lane, (uint32_t)(rs * 2));
    lds0 = lds_addr(smem);
  }


  // Tile idx of the list: item `it` = (sequence, query block, first row, length).
  __device__ __forceinline__ Geo geometry(int idx, int4 it, int per_item) const {
    Geo t;
    const int item = idx / per_item;
    const int rem = idx - item * per_item;
    t.b = __builtin_amdgcn_readfirstlane(it.x);
    t.kv0 = __builtin_amdgcn_readfirstlane(it.z);
    t.n = __builtin_amdgcn_readfirstlane(it.w);
    if (BCAST) {
      t.m = rem / a.heads;
      t.h = rem % a.heads;
    } else {
      t.m = __builtin_amdgcn_readfirstlane(it.y);
      t.h = rem;
    }
    return t;
  }

  // K/V blocks the tile visits.
  __device__ __forceinline__ int num_blocks(const Geo& t) const {
    const int64_t kv_end = CAUSAL ? min((int64_t)t.n, (int64_t)(t.m + 1) * BM) : (int64_t)t.n;
    const int nb = (int)((kv_end + BN - 1) / BN);
    if constexpr (SPARSE) return min(nb, min(a.topk, 64 * 64));
    return nb;
  }
  // Key block visited at position t of the current tile, and the first block of the
  // next tile.
  __device__ __forceinline__ int blk_of(int t) const {
    if constexpr (SPARSE) return __builtin_amdgcn_readfirstlane(lists[lb * 64 + t]);
    return t;
  }
  __device__ __forceinline__ int first_next() const {
    if constexpr (SPARSE) return __builtin_amdgcn_readfirstlane(lists[(lb ^ 1) * 64]);
    return 0;
  }

  // This wave's Q fragment of tile t (rows past the query end read as zeros).
  __device__ __forceinline__ void load_q(const Geo& t) {
    const int qr = BCAST ? a.q_len : t.n;
    const int qi = t.m * BM + 32 * wave + c32;
    const bool qvalid = qi < qr;
    const bf16* qp = a.q + ((BCAST ? (int64_t)qi : t.kv0 + qi) * rs + (int64_t)t.h * D);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      qf[ks] = qvalid ? *reinterpret_cast<const bf16x8*>(qp + 16 * ks + 8 * hf) : zero_bf16x8();
  }

  // Issues the direct LDS loads of K/V block `blk` of tile t into buffer `buf`; rows
  // past the sequence end read as zeros (and the masked tail gives them zero weight).
  __device__ __forceinline__ void load_block(const Geo& t, int blk, int buf) {
    const int64_t jb = (int64_t)blk * BN;
    const int64_t rows = max(min((int64_t)t.n - jb, (int64_t)BN), (int64_t)0);
    const uint32_t bytes = (uint32_t)(rows * rs * 2);
    const int64_t base = (t.kv0 + jb) * rs + (int64_t)t.h * D;
    ld.issue(make_rsrc_sgpr(a.k + base, bytes), lds0 + (uint32_t)((buf * 2 + 0) * TILE_BYTES));
    ld.issue(make_rsrc_sgpr(a.v + base, bytes), lds0 + (uint32_t)((buf * 2 + 1) * TILE_BYTES));
  }

  // One K/V block for this wave's 32 query rows, as two 32-key halves, each its
  // own online-softmax step.  A wave's vector work runs under its own MFMA chains
  // (the matrix cores execute an MFMA while the wave issues independent vector
  // instructions), so the softmax is spread over the block's four MFMA phases:
  //   S0 = K0 Q^T                  (MFMA only)
  //   S1 = K1 Q^T                  half 0: mask, maximum, rescale test, exp2 of
  //                                its first 12 keys
  //   O^T += V0^T P0^T             half 0: last 4 keys (their P is needed from the
  //                                second half of this phase on); half 1: mask,
  //                                maximum, rescale test, first 10 keys
  //   O^T += V1^T P1^T             half 1: last 6 keys (needed from the second
  //                                half of this phase on), after half 1's rescale
  //                                of O, if it made one
  // Each pair of keys takes two MFMA slots: its exponentials in one, their row sums
  // and bf16 P in the next, so that no instruction waits on the exponential just
  // issued (a wave issues in order, and a stalled vector instruction also holds
  // back the wave's next MFMA).
  // Lazy rescaling: the running max of a row moves only when some row of the wave
  // sees a score above its running max by more than 2^kLazyLog2 (a wave-uniform
  // test), so O and the row sums are rescaled rarely; otherwise P is taken against
  // the stale max and may reach 2^kLazyLog2, which O / l and the saved log-sum-exp
  // divide out exactly.
  static constexpr float kLazyLog2 = 8.f;

  template <bool MASKED>
  __device__ __forceinline__ void mask_half(f32x16& s, int blk, int c) const {
    if constexpr (MASKED) {
      // Element r of the lane holds key x = 8 (r / 4) + 4 (lane / 32) + r % 4 of the
      // half, visible when x < lim: keys before the sequence end and, causal, not
      // after the lane's row.  Compared as r's constant part against lim - 4 (lane / 32),
      // so that no per-element key index is kept in registers.
      const int jb = blk * BN + 32 * c;
      int lim = min(g.n - jb, 64);
      if constexpr (CAUSAL) lim = min(lim, i0 + c32 - jb + 1);
      const int L = max(lim, 0) - 4 * hf;
#pragma unroll
      for (int r = 0; r < 16; ++r) s[r] = 8 * (r >> 2) + (r & 3) < L ? s[r] : -INFINITY;
    }
  }
  // As a tree of depth three (a serial chain would hold the wave for its whole
  // latency while the MFMAs of the other half wait behind it), which the compiler
  // emits as eight three-input maxima.  This file is compiled with
  // -fno-honor-nans: otherwise every MFMA result is first quieted (a v_max of the
  // value with itself) in case it is a signalling NaN, which doubles the count.
  // Scores from finite inputs are never NaN, and a NaN input reaches O through the
  // products anyway.
  __device__ __forceinline__ static float half_max(const f32x16& s) {
    float m[5];
#pragma unroll
    for (int k = 0; k < 5; ++k) m[k] = fmaxf(fmaxf(s[3 * k], s[3 * k + 1]), s[3 * k + 2]);
    return fmaxf(fmaxf(fmaxf(m[0], m[1]), m[2]), fmaxf(fmaxf(m[3], m[4]), s[15]));
  }
  // Rescale test of a half whose lane maximum is mx; returns the factor O must be
  // multiplied by when `moved` (row sums are rescaled here).
  __device__ __forceinline__ float rescale_test(float mx, bool& moved) {
    const float mc = max_across_halves(mx) * a.scale_log2;
    float alpha = 1.f;
    moved = __builtin_amdgcn_ballot_w64(mc > mrun + kLazyLog2) != 0;
    if (moved) {
      const float mnew = fmaxf(mrun, mc);
      alpha = fast_exp2(mrun - mnew);
      mrun = mnew;
      lsum *= alpha;
      lsum2 *= alpha;
    }
    return alpha;
  }
  __device__ __forceinline__ void scale_acc(float alpha) {
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[dt][r] *= alpha;
  }
  // Elements 2q and 2q + 1 of a half (keys 16 kc + 8 (e / 4) + 4 (lane / 32) + e % 4
  // of the half for element 8 kc + e): first exp2 of the scaled, shifted score in
  // place, later the row sums and the bf16 P.  The empty asm keeps each stage in the
  // slot the schedule gives it: otherwise the compiler sinks the exponentials past
  // the rescale branches, behind the MFMAs they were meant to run beside.
  __device__ __forceinline__ void pair_exp(f32x16& s, int q) {
    float e0 = fast_exp2(fmaf(s[2 * q], a.scale_log2, -mrun));
    float e1 = fast_exp2(fmaf(s[2 * q + 1], a.scale_log2, -mrun));
    asm volatile("" : "+v"(e0), "+v"(e1));
    s[2 * q] = e0;
    s[2 * q + 1] = e1;
  }
  __device__ __forceinline__ void pair_sum(const f32x16& s, bf16x8 (&p)[2], int q) {
    lsum += s[2 * q];
    lsum2 += s[2 * q + 1];
    p[q >> 2][(2 * q) & 7] = (bf16)s[2 * q];
    p[q >> 2][(2 * q + 1) & 7] = (bf16)s[2 * q + 1];
    asm volatile("" : "+v"(p[q >> 2]), "+v"(lsum), "+v"(lsum2));
  }

  // Softmax work of MFMA slot s8 (0..7, eight per phase; with D = 64 a slot takes
  // two) of phase ph (0: S1, 1: O += P0 V0, 2: O += P1 V1), as bits: 0..7 exps of
  // half 0's pairs, 8..15 of half 1's, 16..23 sums of half 0's pairs, 24..31 of
  // half 1's, 32 / 33 mask and maximum / rescale test of half 0, 34 / 35 of half 1.
  // A pair's sums come one slot after its exps; a half's P is complete before the
  // first O product that reads it, and every sum of half 0 is in before half 1's
  // rescale test multiplies the row sums.
  static constexpr uint64_t slot_acts(int ph, int s8) {
    auto fe = [](int h, int q) { return uint64_t(1) << (8 * h + q); };
    auto cs = [](int h, int q) { return uint64_t(1) << (16 + 8 * h + q); };
    if (ph == 0) {
      if (s8 == 0) return uint64_t(1) << 32;
      if (s8 == 1) return uint64_t(1) << 33;
      return fe(0, s8 - 2) | (s8 >= 3 ? cs(0, s8 - 3) : 0);
    }
    if (ph == 1) {
      if (s8 == 0) return cs(0, 5) | fe(0, 6) | fe(0, 7);
      if (s8 == 1) return cs(0, 6) | cs(0, 7) | (uint64_t(1) << 34);
      if (s8 == 2) return uint64_t(1) << 35;
      return fe(1, s8 - 3) | (s8 >= 4 ? cs(1, s8 - 4) : 0);
    }
    if (s8 < 3) return cs(1, s8 + 4) | fe(1, s8 + 5);
    if (s8 == 3) return cs(1, 7);
    return 0;
  }

  template <bool MASKED>
  __device__ __forceinline__ void compute_block(int buf, int blk) {
    // The buffer's offset (a multiple of 16 KB) is added to the lane bases once: the
    // swizzle's XORs touch only bits below 9, so (base + offset) ^ x equals
    // (base ^ x) + offset, and each operand read costs one XOR.
    const uint32_t krb = launder(k_row_base + (uint32_t)(buf * 2 * TILE_BYTES));
    const uint32_t vtb = launder(v_tr_base + (uint32_t)((buf * 2 + 1) * TILE_BYTES));
    // K operand of half c, k step ks; V^T operand of O step i (keys 16 (i / DT), d
    // tile i % DT).  Operands are read PF_S (PF_V) MFMA steps ahead; the scheduling
    // fences keep that pipeline, and the interleaving, as written.
    auto kop = [&](int i) { return lds_read8(smem, row_read_addr(krb, i % KS) + 32 * (i / KS) * 2 * D); };
    auto vop = [&](int i) { return lds_operand_tr<D>(smem, vtb, 16 * (i / DT), 16 * (i / DT) + 8, i % DT); };
    // S1 is one chain: the other wave of the SIMD fills the MFMA pipe while a step
    // waits for the one before it.
    f32x16 s0 = zero16(), s1 = zero16();
    bf16x8 p[2][2];
    bf16x8 vr[PF_V + 1];
    float mx0 = 0.f, mx1 = 0.f, alpha1 = 1.f;
    bool moved1 = false;
    auto slot = [&](int ph, int s8) {
      const uint64_t A = slot_acts(ph, s8);
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        if ((A >> (16 + q)) & 1) pair_sum(s0, p[0], q);
        if ((A >> (24 + q)) & 1) pair_sum(s1, p[1], q);
      }
      if ((A >> 32) & 1) {
        mask_half<MASKED>(s0, blk, 0);
        mx0 = half_max(s0);
      }
      if ((A >> 33) & 1) {
        bool moved;
        const float alpha = rescale_test(mx0, moved);
        if (moved) scale_acc(alpha);
      }
      if ((A >> 34) & 1) {
        mask_half<MASKED>(s1, blk, 1);
        mx1 = half_max(s1);
      }
      if ((A >> 35) & 1) alpha1 = rescale_test(mx1, moved1);   // applied once O += P0 V0 is issued
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        if ((A >> q) & 1) pair_exp(s0, q);
        if ((A >> (8 + q)) & 1) pair_exp(s1, q);
      }
    };
    // MFMA step k of a phase with n steps covers slots [8 k / n, 8 (k + 1) / n)
    auto slots = [&](int ph, int k, int n) {
#pragma unroll
      for (int s8 = 8 * k / n; s8 < 8 * (k + 1) / n; ++s8) slot(ph, s8);
    };
    {
      bf16x8 kr[PF_S + 1];
#pragma unroll
      for (int i = 0; i < PF_S; ++i) kr[i] = kop(i);
      // S0, then S1 with phase B
#pragma unroll
      for (int i = 0; i < 2 * KS; ++i) {
        if (i + PF_S < 2 * KS) kr[(i + PF_S) % (PF_S + 1)] = kop(i + PF_S);
        if (i + PF_V >= 2 * KS) vr[i + PF_V - 2 * KS] = vop(i + PF_V - 2 * KS);
        if (i < KS) {
          s0 = mfma32(kr[i % (PF_S + 1)], qf[i], s0);
        } else {
          const int k = i - KS;
          s1 = mfma32(kr[i % (PF_S + 1)], qf[k], s1);
          slots(0, k, KS);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // O += P0 V0 with phase C, half 1's rescale of O, then O += P1 V1 with phase D
#pragma unroll
    for (int i = 0; i < 4 * DT; ++i) {
      if (i + PF_V < 4 * DT) vr[(i + PF_V) % (PF_V + 1)] = vop(i + PF_V);
      if (i == 2 * DT && moved1) scale_acc(alpha1);
      const int ckc = i / DT;
      acc[i % DT] = mfma32(vr[i % (PF_V + 1)], p[ckc / 2][ckc % 2], acc[i % DT]);
      if (i < 2 * DT) {
        slots(1, i, 2 * DT);
      } else {
        slots(2, i - 2 * DT, 2 * DT);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  __device__ __forceinline__ bool wave_needs(int blk) const {
    if (i0 >= q_rows) return false;
    if constexpr (CAUSAL) return (int64_t)blk * BN <= (int64_t)i0 + 31;
    return true;
  }

  // Blocks [t_begin, t_end) of the current tile; block t sits in buffer (pb + t) & 1.
  // Each iteration first issues the loads of the block after it: the tile's own, or,
  // after the last one, the first block of the next tile, which stays in flight
  // through the epilogue (the last iteration does not wait).
  template <bool MASKED>
  __device__ __forceinline__ void run_blocks(int t_begin, int t_end, int nblk, int pb, const Geo& nxt,
                                             bool has_next) {
    for (int t = t_begin; t < t_end; ++t) {
      const int buf = (pb + t) & 1;
      if (t + 1 < nblk) {
        load_block(g, blk_of(t + 1), buf ^ 1);
      } else if (has_next) {
        load_block(nxt, first_next(), buf ^ 1);
      }
      const int blk = blk_of(t);
      if (wave_needs(blk)) compute_block<MASKED>(buf, blk);
      if (t + 1 < nblk) wait_lds_loads();
      __syncthreads();
    }
  }

  // Runs tile g, whose first K/V block is in buffer pb and whose Q fragment is in
  // qf (both loaded or in flight, the block published by a barrier).  After the last
  // barrier over the K/V buffers it issues the next tile's Q fragment, runs
  // `between`, and writes O and LSE, staging O through the buffer of the last block
  // (the next tile's first block goes to the other).  Returns the next tile's pb.
  template <class Between>
  __device__ __forceinline__ int tile(int pb, const Geo& nxt, bool has_next, Between&& between) {
    q_rows = BCAST ? a.q_len : g.n;
    m0 = g.m * BM;
    i0 = m0 + 32 * wave;
    out_row0 = BCAST ? (int64_t)g.b * a.q_len : g.kv0;
    const int qi = i0 + c32;
    const bool qvalid = qi < q_rows;
    // The Q fragment was loaded during the previous tile: consume it here so that the
    // compiler's wait for it lands before the block loop, not inside it (where it
    // would also wait for the next block's loads).
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) asm volatile("" : "+v"(qf[ks]));
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) acc[dt] = zero16();
    mrun = kNegBig;
    lsum = 0.f;
    lsum2 = 0.f;

    const int nblk = num_blocks(g);
    int nfull = (int)(g.n / BN);
    if constexpr (CAUSAL) nfull = min(nfull, (m0 + 1) / BN);
    nfull = min(nfull, nblk);
    if constexpr (SPARSE) {   // ascending list: only its last block can be the partial one
      nfull = nblk;
      if (nblk > 0 && (int64_t)(blk_of(nblk - 1) + 1) * BN > g.n) nfull = nblk - 1;
    }
    run_blocks<false>(0, nfull, nblk, pb, nxt, has_next);
    run_blocks<true>(nfull, nblk, nblk, pb, nxt, has_next);
    if (nblk == 0) {   // an empty sequence (broadcast mode): no block barrier ran
      __syncthreads();
      if (has_next) load_block(nxt, first_next(), pb);
    }
    // this tile is done with its Q fragment; in broadcast mode the next tile keeps it
    // when it has the same query block and head
    if (has_next && !(BCAST && nxt.m == g.m && nxt.h == g.h)) load_q(nxt);
    between();

    // epilogue
    const float lt = sum_across_halves(lsum + lsum2);
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    char* slot = smem + ((pb + nblk + 1) & 1) * (2 * TILE_BYTES) + wave * SLOT_BYTES;
    store_acc_rows<D, EPI_PASSES>(acc, inv, slot, a.o + ((out_row0 + i0) * rs + (int64_t)g.h * D), rs,
                                  min(max(q_rows - i0, 0), 32), lane);
    if (qvalid && hf == 0)
      a.lse[(int64_t)g.h * a.rows + out_row0 + qi] = lt > 0.f ? (mrun + __log2f(lt)) * kLn2 : -INFINITY;
    return (pb + nblk) & 1;
  }
};

// Persistent tile loop.  A workgroup knows two tiles ahead: while tile r runs, the
// index of tile r + 2 is claimed (or computed, for the static schedules) and, after
// tile r's last block, its plan item is copied into LDS by a direct load, so that
// tile r + 1's first K/V block and Q fragment can be issued during tile r.
// Broadcast mode, dynamic schedule: the tiles of one (query block, head) class all
// read the same Q fragment, and every class has the same work (each sequence's
// tiles see all its keys).  With few classes, each workgroup serves one class,
// claiming that class's tiles in plan order from a counter of its own, so its Q
// fragment is loaded once and the tile boundaries load only K/V.
template <int D, int NW, bool BCAST, bool CAUSAL, bool SPARSE = false>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(2)))
void fwd_kernel(FwdArgs a) {
  using K = FwdKernel<D, NW, BCAST, CAUSAL, SPARSE>;
  using Geo = typename K::Geo;
  __shared__ __attribute__((aligned(16))) char smem[4 * K::TILE_BYTES];
  __shared__ __attribute__((aligned(16))) int next_item[64];   // one dword per lane of the copy
  __shared__ __attribute__((aligned(16))) int lists[SPARSE ? 2 * 64 : 1];
  __shared__ int next_idx;
  __shared__ int first_idx[2];
  K kern(a, smem);
  kern.lists = lists;
  const int num_wg = gridDim.x;
  const int lwg = xcd_logical_wg(blockIdx.x, num_wg);
  const int ntiles = a.meta[2];
  const int per_item = BCAST ? ((a.q_len + K::BM - 1) / K::BM) * a.heads : a.heads;
  const bool dyn = a.sched == kDynamic;
  const int cls = a.classes > 0 ? lwg % a.classes : 0;
  auto claim = [&]() {   // next tile of the dynamic schedule (one lane)
    if (a.classes > 0) return atomicAdd(a.meta + 4 + cls, 1) * a.classes + cls;
    return atomicAdd(a.meta + 1, 1);
  };
  auto sched_idx = [&](int r) {
    if (a.sched == kIdentity) return r * num_wg + lwg;
    return r * num_wg + ((r & 1) ? (num_wg - 1 - lwg) : lwg);
  };
  auto fetch_item = [&](int idx) {   // plan item of tile idx -> next_item[0 .. 3]
    lds_load4(make_rsrc_sgpr(a.items + idx / per_item, 16u), (uint32_t)kern.lane * 4u,
              reinterpret_cast<char*>(next_item));
  };
  // SPARSE: key-block list of tile idx -> list buffer `buf` (entries past topk read
  // as zeros and are never used)
  auto fetch_list = [&](int idx, int buf) {
    if constexpr (SPARSE)
      lds_load4(make_rsrc_sgpr(a.tile_blocks + (int64_t)idx * a.topk, (uint32_t)a.topk * 4u),
                (uint32_t)kern.lane * 4u, reinterpret_cast<char*>(lists + buf * 64));
  };

  int idx0, idx1;
  if (dyn) {
    if (threadIdx.x == 0) {
      first_idx[0] = claim();
      first_idx[1] = claim();
    }
    __syncthreads();
    idx0 = __builtin_amdgcn_readfirstlane(first_idx[0]);
    idx1 = __builtin_amdgcn_readfirstlane(first_idx[1]);
  } else {
    idx0 = sched_idx(0);
    idx1 = sched_idx(1);
  }
  if (idx0 >= ntiles) return;
  kern.g = kern.geometry(idx0, a.items[idx0 / per_item], per_item);
  if (kern.wave == 0) {
    if (idx1 < ntiles) fetch_item(idx1);
    if (threadIdx.x == 0) next_idx = idx1;
  }
  if constexpr (SPARSE) {   // the first two tiles' lists, before the first block's address
    if (kern.wave == 0) {
      fetch_list(idx0, 0);
      if (idx1 < ntiles) fetch_list(idx1, 1);
    }
    wait_lds_loads();
    __syncthreads();
  }
  kern.load_q(kern.g);
  if (kern.num_blocks(kern.g) > 0) kern.load_block(kern.g, kern.blk_of(0), 0);

  int pb = 0;
  for (int r = 0;; ++r) {
    // Everything but the previous epilogue's D / 16 stores has landed: this tile's
    // first block, its Q fragment and the next tile's item.
    if (r == 0) {
      wait_lds_loads();
    } else {
      wait_vmcnt<D / 16>();
    }
    __syncthreads();
    const int nidx = __builtin_amdgcn_readfirstlane(next_idx);
    const bool has_next = nidx < ntiles;
    Geo nxt = kern.g;
    if (has_next) nxt = kern.geometry(nidx, *reinterpret_cast<const int4*>(next_item), per_item);
    int pend = ntiles;   // index of tile r + 2 (lane 0 of wave 0 under the dynamic schedule)
    if (dyn) {
      if (threadIdx.x == 0) pend = claim();
    } else {
      pend = sched_idx(r + 2);
    }
    pb = kern.tile(pb, nxt, has_next, [&]() {
      if (has_next && kern.wave == 0) {
        const int i2 = __builtin_amdgcn_readfirstlane(pend);
        if (i2 < ntiles) {
          fetch_item(i2);
          fetch_list(i2, kern.lb);   // tile r + 2 takes this tile's (finished) list buffer
        }
        if (threadIdx.x == 0) next_idx = i2;
      }
    });
    if (!has_next) break;
    kern.g = nxt;
    kern.lb ^= 1;
  }
}

template <int D, int NW, bool BCAST, bool CAUSAL, bool SPARSE = false>
hipError_t launch_inst(const FwdArgs& args, hipStream_t s, int64_t max_tiles) {
  const void* fn = reinterpret_cast<const void*>(&fwd_kernel<D, NW, BCAST, CAUSAL, SPARSE>);
  const int grid = persistent_grid(fn, 64 * NW, max_tiles);
  FwdArgs a = args;
  a.classes = 0;
  if (BCAST && !CAUSAL && a.sched == kDynamic) {
    // one class per workgroup when there are at least four workgroups per class (the
    // block-sparse tiles of a sequence all visit min(k, its key blocks) blocks)
    const int per_item = ((a.q_len + 32 * NW - 1) / (32 * NW)) * a.heads;
    if (per_item <= kFwdClassMax && grid >= 4 * per_item) a.classes = per_item;
  }
  hipLaunchKernelGGL((fwd_kernel<D, NW, BCAST, CAUSAL, SPARSE>), dim3(grid), dim3(64 * NW), 0, s, a);
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const Problem& p, const FwdArgs& a, hipStream_t s) {
  const int nw = fwd_waves(p);
  if (p.broadcast) {
    const int64_t max_tiles = (int64_t)p.batch * ((p.q_len + 32 * nw - 1) / (32 * nw)) * p.heads;
    if (nw == 8) return launch_inst<D, 8, true, false>(a, s, max_tiles);
    if (nw == 4) return launch_inst<D, 4, true, false>(a, s, max_tiles);
    return launch_inst<D, 2, true, false>(a, s, max_tiles);
  }
  const int64_t max_tiles = fwd_max_items(p) * p.heads;
  if (nw == 8)
    return p.causal ? launch_inst<D, 8, false, true>(a, s, max_tiles) : launch_inst<D, 8, false, false>(a, s, max_tiles);
  if (p.causal) return launch_inst<D, 4, false, true>(a, s, max_tiles);
  return launch_inst<D, 4, false, false>(a, s, max_tiles);
}

}  // namespace

int fwd_waves(const Problem& p) {
  if (p.topk > 0) return sparse_qb(p) / 32;   // block-sparse: the tile is one query block
  if (p.mx && !p.broadcast) {                  // MXFP8 self mode: tiles near the mean length
    const int64_t mean = p.batch > 0 ? p.total_kv / p.batch : 0;
    return mean <= 96 ? 2 : (mean >= 384 ? 8 : 4);
  }
  // Self mode: 256-row tiles when sequences are long on average, so that the query
  // tiles of a sequence read its K/V half as often; 128-row tiles otherwise.
  if (!p.broadcast) return (p.batch > 0 && p.total_kv / p.batch >= 512) ? 8 : 4;
  if (p.q_len > 128) return 8;
  if (p.q_len > 64) return 4;
  return 2;
}

int64_t fwd_max_items(const Problem& p) {
  if (p.broadcast) return p.batch;
  const int bm = 32 * fwd_waves(p);
  return (p.total_kv + bm - 1) / bm + p.batch;
}

hipError_t launch_fwd(const Problem& p, const Plan& plan, int sched, void* o, float* lse,
                      hipStream_t s) {
  FwdArgs a;
  a.q = static_cast<const bf16*>(p.q);
  a.k = static_cast<const bf16*>(p.k);
  a.v = static_cast<const bf16*>(p.v);
  a.offsets = p.offsets;
  a.off64 = p.off64;
  a.heads = p.heads;
  a.q_len = p.q_len;
  a.rows = p.rows;
  a.scale_log2 = p.scale * kLog2e;
  a.o = static_cast<bf16*>(o);
  a.lse = lse;
  a.items = plan.items;
  a.meta = plan.meta;
  a.sched = sched;
  a.tile_blocks = nullptr;
  a.topk = 0;
  return p.head_dim == 128 ? launch_d<128>(p, a, s) : launch_d<64>(p, a, s);
}

hipError_t launch_fwd_sparse(const Problem& p, const Plan& plan, int sched, const Sparse& sp, void* o,
                             float* lse, hipStream_t s) {
  FwdArgs a;
  a.q = static_cast<const bf16*>(p.q);
  a.k = static_cast<const bf16*>(p.k);
  a.v = static_cast<const bf16*>(p.v);
  a.offsets = p.offsets;
  a.off64 = p.off64;
  a.heads = p.heads;
  a.q_len = p.q_len;
  a.rows = p.rows;
  a.scale_log2 = p.scale * kLog2e;
  a.o = static_cast<bf16*>(o);
  a.lse = lse;
  a.items = plan.items;
  a.meta = plan.meta;
  a.sched = sched;
  a.tile_blocks = sp.tile_blocks;
  a.topk = p.topk;
  constexpr int NWB = kSparseQBBroadcast / 32, NWS = kSparseQBSelf / 32;
  const int64_t per_item =
      p.broadcast ? ((p.q_len + kSparseQBBroadcast - 1) / kSparseQBBroadcast) * p.heads : p.heads;
  const int64_t max_tiles = fwd_max_items(p) * per_item;
  if (p.head_dim == 128) {
    return p.broadcast ? launch_inst<128, NWB, true, false, true>(a, s, max_tiles)
                       : launch_inst<128, NWS, false, false, true>(a, s, max_tiles);
  }
  return p.broadcast ? launch_inst<64, NWB, true, false, true>(a, s, max_tiles)
                     : launch_inst<64, NWS, false, false, true>(a, s, max_tiles);
}

}  // namespace jfa
