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
//    section "Five changes unlocked the gains", items 1 and 2);
//  * a tile is (sequence, block of 32*NW query rows, head); each 64-lane wave owns
//    32 query rows, keeps its Q fragment in registers and computes
//    S^T = K Q^T and O^T += V^T P^T with v_mfma_f32_32x32x16_bf16, so that the
//    fp32 score accumulator is already laid out as the bf16 P operand;
//  * K/V blocks of 64 keys stream straight from HBM into swizzled LDS (gfx950
//    direct global->LDS loads, double buffered) one block ahead of the MFMA work;
//    V^T operands come from the gfx950 transposing LDS read;
//  * online softmax in the exp2 domain with a running max and a lane-local running
//    sum (the two halves of a wave hold the two halves of a row's keys and are
//    combined once, at the end);
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
};

template <int D, int NW, bool BCAST, bool CAUSAL>
struct FwdKernel {
  static constexpr int BN = kFwdBN;
  static constexpr int BM = 32 * NW;
  static constexpr int NT = 64 * NW;
  static constexpr int CH = D / 8;               // 16-byte chunks per row
  static constexpr int TILE_BYTES = BN * D * 2;
  static constexpr int DT = D / 32;              // 32-wide d tiles of O
  static constexpr int KS = D / 16;              // 16-deep k steps of Q K^T
  static_assert((BN * D * 2 / 1024) % NW == 0, "a K/V block must split evenly over the waves");
  static_assert(NW * 32 * 2 * D <= 4 * TILE_BYTES, "epilogue slots must fit in the K/V buffers");

  // Tile-invariant per-wave state.
  FwdArgs a;
  char* smem;          // [2 buffers][K, V][BN x D] swizzled
  int lane, wave, c32, hf;
  int64_t rs;          // row stride (elements) of q, k, v, o

  // Per-tile state.
  int64_t kv0, n;
  int h, q_rows, m0, i0;
  int64_t out_row0;    // first output row of the sequence
  bf16x8 qf[KS];
  f32x16 acc[DT];
  float mrun, lsum;
  uint32_t k_row_base;   // lane part of K row reads (rows 32 c + lane % 32)
  uint32_t v_tr_base;    // lane part of V^T transposing reads (k offset 4 (lane / 32))

  __device__ FwdKernel(const FwdArgs& args, char* sm) : a(args), smem(sm) {
    lane = threadIdx.x & 63;
    wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform (SGPR)
    c32 = lane & 31;
    hf = lane >> 5;
    rs = (int64_t)a.heads * D;
    k_row_base = row_read_base<D>(lane);
    v_tr_base = tr_read_base<D>(lane, 4 * hf);
  }

  __device__ __forceinline__ char* kbuf(int buf) { return smem + (buf * 2 + 0) * TILE_BYTES; }
  __device__ __forceinline__ char* vbuf(int buf) { return smem + (buf * 2 + 1) * TILE_BYTES; }

  // Issues the direct LDS loads of K/V block `blk` into buffer `buf`; rows past the
  // sequence end read as zeros (and the masked tail gives them zero weight).
  __device__ __forceinline__ void load_block(int blk, int buf) {
    const int64_t jb = (int64_t)blk * BN;
    const int64_t rows = min(n - jb, (int64_t)BN);
    const uint32_t bytes = (uint32_t)(rows * rs * 2);
    const int64_t base = (kv0 + jb) * rs + (int64_t)h * D;
    const uint32_t row_bytes = (uint32_t)(rs * 2);
    lds_load_tile<D, NW>(kbuf(buf), BN, wave, lane, make_rsrc_sgpr(a.k + base, bytes), row_bytes);
    lds_load_tile<D, NW>(vbuf(buf), BN, wave, lane, make_rsrc_sgpr(a.v + base, bytes), row_bytes);
  }

  // One K/V block for this wave's 32 query rows.
  template <bool MASKED>
  __device__ __forceinline__ void compute_block(int buf, int blk) {
    const char* kb = kbuf(buf);
    const char* vb = vbuf(buf);
    const uint32_t krb = launder(k_row_base);
    const uint32_t vtb = launder(v_tr_base);
    f32x16 s[2];
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      s[c] = zero16();
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const bf16x8 kf = lds_read8(kb, row_read_addr(krb, ks) + 32 * c * 2 * D);
        s[c] = mfma32(kf, qf[ks], s[c]);
      }
    }
    if constexpr (MASKED) {
      const int64_t i = i0 + c32;
#pragma unroll
      for (int c = 0; c < 2; ++c) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int64_t j = (int64_t)blk * BN + 32 * c + 8 * (r >> 2) + 4 * hf + (r & 3);
          bool vis = j < n;
          if constexpr (CAUSAL) vis = vis && (j <= i);
          s[c][r] = vis ? s[c][r] : -INFINITY;
        }
      }
    }
    float mx = s[0][0];
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[c][r]);
    mx = max_across_halves(mx);
    const float mnew = fmaxf(mrun, mx * a.scale_log2);
    const float alpha = fast_exp2(mrun - mnew);
    mrun = mnew;
    lsum *= alpha;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[dt][r] *= alpha;

    bf16x8 p[2][2];
#pragma unroll
    for (int c = 0; c < 2; ++c) {
#pragma unroll
      for (int kc = 0; kc < 2; ++kc) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float pv = fast_exp2(fmaf(s[c][8 * kc + e], a.scale_log2, -mnew));
          lsum += pv;
          p[c][kc][e] = (bf16)pv;
        }
      }
    }
#pragma unroll
    for (int c = 0; c < 2; ++c) {
#pragma unroll
      for (int kc = 0; kc < 2; ++kc) {
        const int jb = 32 * c + 16 * kc;   // keys jb + 4 (lane / 32) + e, and + 8
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          const bf16x8 vt = lds_operand_tr<D>(vb, vtb, jb, jb + 8, dt);
          acc[dt] = mfma32(vt, p[c][kc], acc[dt]);
        }
      }
    }
  }

  __device__ __forceinline__ bool wave_needs(int blk) const {
    if (i0 >= q_rows) return false;
    if constexpr (CAUSAL) return (int64_t)blk * BN <= (int64_t)i0 + 31;
    return true;
  }

  template <bool MASKED>
  __device__ __forceinline__ void run_blocks(int t_begin, int t_end, int nblk) {
    for (int t = t_begin; t < t_end; ++t) {
      if (t + 1 < nblk) load_block(t + 1, (t + 1) & 1);   // one block ahead
      if (wave_needs(t)) compute_block<MASKED>(t & 1, t);
      wait_lds_loads();
      __syncthreads();
    }
  }

  // Tile (sequence b with rows [kv0, kv0 + len), query block m, head).
  __device__ __forceinline__ void tile(int b, int m, int head, int seq_kv0, int seq_len) {
    __syncthreads();   // the previous tile's epilogue is done with the K/V buffers
    h = head;
    kv0 = seq_kv0;
    n = seq_len;
    q_rows = BCAST ? a.q_len : (int)n;
    m0 = m * BM;
    i0 = m0 + 32 * wave;
    out_row0 = BCAST ? (int64_t)b * a.q_len : kv0;

    const int qi = i0 + c32;
    const bool qvalid = qi < q_rows;
    const bf16* qp = a.q + ((BCAST ? (int64_t)qi : kv0 + qi) * rs + (int64_t)h * D);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      qf[ks] = qvalid ? *reinterpret_cast<const bf16x8*>(qp + 16 * ks + 8 * hf) : zero_bf16x8();
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) acc[dt] = zero16();
    mrun = kNegBig;
    lsum = 0.f;

    const int64_t kv_end = CAUSAL ? min(n, (int64_t)m0 + BM) : n;
    const int nblk = (int)((kv_end + BN - 1) / BN);
    int nfull = (int)(n / BN);
    if constexpr (CAUSAL) nfull = min(nfull, (m0 + 1) / BN);
    nfull = min(nfull, nblk);

    if (nblk > 0) load_block(0, 0);
    wait_lds_loads();
    __syncthreads();
    run_blocks<false>(0, nfull, nblk);
    run_blocks<true>(nfull, nblk, nblk);

    // epilogue
    const float lt = sum_across_halves(lsum);
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    // O rows staged through this wave's slot of the (now idle) K/V buffers
    store_acc_rows<D>(acc, inv, smem + wave * (32 * 2 * D), a.o + ((out_row0 + i0) * rs + (int64_t)h * D), rs,
                      min(max(q_rows - i0, 0), 32), lane);
    if (qvalid && hf == 0)
      a.lse[(int64_t)h * a.rows + out_row0 + qi] = lt > 0.f ? (mrun + __log2f(lt)) * kLn2 : -INFINITY;
  }
};

template <int D, int NW, bool BCAST, bool CAUSAL>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(2)))
void fwd_kernel(FwdArgs a) {
  using K = FwdKernel<D, NW, BCAST, CAUSAL>;
  __shared__ __attribute__((aligned(16))) char smem[4 * K::TILE_BYTES];
  __shared__ int claimed;
  K kern(a, smem);
  const int num_wg = gridDim.x;
  const int lwg = xcd_logical_wg(blockIdx.x, num_wg);
  const int ntiles = a.meta[2];
  const int per_item = BCAST ? ((a.q_len + K::BM - 1) / K::BM) * a.heads : a.heads;
  for (int r = 0;; ++r) {
    int idx;
    if (a.sched == kDynamic) {
      if (threadIdx.x == 0) claimed = atomicAdd(a.meta + 1, 1);
      __syncthreads();
      idx = claimed;
      __syncthreads();
    } else if (a.sched == kIdentity) {
      idx = r * num_wg + lwg;
    } else {
      idx = r * num_wg + ((r & 1) ? (num_wg - 1 - lwg) : lwg);
    }
    if (idx >= ntiles) break;
    const int item = idx / per_item;
    const int rem = idx - item * per_item;
    const int4 it = a.items[item];
    const int b = __builtin_amdgcn_readfirstlane(it.x), blk = __builtin_amdgcn_readfirstlane(it.y);
    const int s0 = __builtin_amdgcn_readfirstlane(it.z), len = __builtin_amdgcn_readfirstlane(it.w);
    if (BCAST) {
      kern.tile(b, rem / a.heads, rem % a.heads, s0, len);
    } else {
      kern.tile(b, blk, rem, s0, len);
    }
  }
}

template <int D, int NW, bool BCAST, bool CAUSAL>
hipError_t launch_inst(const FwdArgs& a, hipStream_t s, int64_t max_tiles) {
  const void* fn = reinterpret_cast<const void*>(&fwd_kernel<D, NW, BCAST, CAUSAL>);
  const int grid = persistent_grid(fn, 64 * NW, max_tiles);
  hipLaunchKernelGGL((fwd_kernel<D, NW, BCAST, CAUSAL>), dim3(grid), dim3(64 * NW), 0, s, a);
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
  if (p.causal) return launch_inst<D, 4, false, true>(a, s, max_tiles);
  return launch_inst<D, 4, false, false>(a, s, max_tiles);
}

}  // namespace

int fwd_waves(const Problem& p) {
  if (!p.broadcast) return 4;
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
  return p.head_dim == 128 ? launch_d<128>(p, a, s) : launch_d<64>(p, a, s);
}

}  // namespace jfa
