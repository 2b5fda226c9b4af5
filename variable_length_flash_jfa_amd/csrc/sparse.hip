// Scoring and top-k selection of the block-sparse forward.
//
// "Optimizing Jagged Flash Attention with TLX" (reading note) and "Meta's TLX
// attention kernel outpaces FlashAttention-4 on B200" (the kernel's variants): a
// scoring step picks, for every query block, the top k key/value blocks, and the
// attention then runs only over the keys of those blocks.  The pages do not say
// how blocks are scored; here the score of (query block, key block) for a head is
// c * mean(query rows) . mean(key rows), the common pooled estimate of the block's
// scores, decided in fp32.
//
//  * pool_blocks_kernel: fp32 mean rows of every key block (64 keys of a
//    sequence) and query block (256 broadcast rows, or 128 rows of a sequence) for
//    every head, one workgroup per block;
//  * select_blocks_kernel: one wave per forward tile (query block, head): k rounds
//    of a wave-wide argmax over the sequence's key blocks in the order (score
//    descending, block index ascending), each round taking the best block after the
//    previous round's; the k blocks are then listed in ascending order, in forward
//    tile order for the kernel and in natural order for the caller.
#include <algorithm>

#include "jfa_device.h"
#include "jfa_internal.h"

namespace jfa {
namespace {

// Index b of the sequence that holds global block g, given first[0 .. batch]
// (exclusive prefix sums of the per-sequence block counts): the first b + 1 with
// first[b + 1] > g (sequences without blocks are skipped).
__device__ __forceinline__ int find_sequence(const int* first, int batch, int g) {
  int lo = 1, hi = batch;   // answer index i in [1, batch] with first[i] > g, minimal
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (first[mid] > g) {
      hi = mid;
    } else {
      lo = mid + 1;
    }
  }
  return lo - 1;
}

// One workgroup per block.  Jagged blocks (first != null): block g of the packed
// rows, block_rows rows of sequence b = find_sequence(g).  Shared blocks (first ==
// null): block g of one sequence of shared_rows rows (the broadcast query).
// out[(h * cap + g) * D + d] = mean over the block's rows of x[row][h][d].  A row of
// all heads is C = heads D / 8 chunks of 8 columns; thread t adds chunk t % C of rows
// t / C, t / C + 256 / C, ... (16-byte loads), and the 256 / C partial sums of a
// chunk meet in LDS.  Rows of more than 256 chunks (heads D / 8 > 256) take one
// thread per chunk over all rows instead.
template <int D>
__global__ __launch_bounds__(256) void pool_blocks_kernel(const bf16* __restrict__ x, int heads,
                                                          const void* offsets, int off64, int batch,
                                                          const int* __restrict__ first, int block_rows,
                                                          int64_t shared_rows, float* __restrict__ out,
                                                          int64_t cap) {
  __shared__ float part[256][9];   // 8 sums per thread (+1 against bank conflicts)
  const int g = blockIdx.x;
  int64_t r0, nr;
  if (first != nullptr) {
    if (g >= first[batch]) return;
    const int b = find_sequence(first, batch, g);
    const int64_t s0 = load_offset(offsets, off64, b);
    const int64_t n = load_offset(offsets, off64, b + 1) - s0;
    const int64_t j = g - first[b];
    r0 = s0 + j * block_rows;
    nr = min((int64_t)block_rows, n - j * block_rows);
  } else {
    r0 = (int64_t)g * block_rows;
    if (r0 >= shared_rows) return;
    nr = min((int64_t)block_rows, shared_rows - r0);
  }
  const int64_t rs = (int64_t)heads * D;
  const int C = heads * D / 8;        // chunks per row
  const float inv = 1.f / (float)nr;
  if (C > 256) {   // wide rows: a thread per chunk
    for (int c = threadIdx.x; c < C; c += 256) {
      float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
      for (int64_t row = 0; row < nr; ++row) {
        const bf16x8 v = *reinterpret_cast<const bf16x8*>(x + (r0 + row) * rs + 8 * c);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] += (float)v[e];
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int i = 8 * c + e;
        const int h = i / D, d = i - h * D;
        out[((int64_t)h * cap + g) * D + d] = acc[e] * inv;
      }
    }
    return;
  }
  const int R = 256 / C;              // rows per pass
  const int t = threadIdx.x;
  const int c = t % C, r = t / C;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  if (r < R) {
    // four rows' loads in flight at a time (the adds keep the row order)
    int64_t row = r;
    for (; row + 3 * R < nr; row += 4 * R) {
      bf16x8 v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) v[u] = *reinterpret_cast<const bf16x8*>(x + (r0 + row + u * R) * rs + 8 * c);
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] += (float)v[u][e];
    }
    for (; row < nr; row += R) {
      const bf16x8 v = *reinterpret_cast<const bf16x8*>(x + (r0 + row) * rs + 8 * c);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] += (float)v[e];
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) part[t][e] = acc[e];
  __syncthreads();
  if (t < C) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float sum = 0.f;
      for (int k = 0; k < R; ++k) sum += part[k * C + t][e];
      const int i = 8 * t + e;   // element (h, d) of a row
      const int h = i / D, d = i - h * D;
      out[((int64_t)h * cap + g) * D + d] = sum * inv;
    }
  }
}

struct SelectArgs {
  const int4* items;
  const int* meta;
  const int* kv_first;
  const int* q_first;
  const float* pooled_k;
  const float* pooled_q;
  int* tile_blocks;
  int* out_blocks;
  int64_t kv_cap, q_cap, out_cap;
  int heads;
  int q_len;
  int broadcast;
  int topk;
  float scale;
};

// (score, index) order of the selection: a before b if a's score is higher, or equal
// with the lower index.
__device__ __forceinline__ bool ranks_before(float sa, int ja, float sb, int jb) {
  return sa > sb || (sa == sb && ja < jb);
}

template <int D>
__global__ __launch_bounds__(256) void select_blocks_kernel(SelectArgs a) {
  __shared__ float pq_lds[4][D];
  // each candidate's score, computed once (the first kScoreCache candidates; the
  // rest, sequences past 65536 keys, are recomputed in every round): lane l writes
  // and later reads only the entries l + 64 u, so the wave needs no barrier
  constexpr int kScoreCache = 1024;
  __shared__ float sc_lds[4][kScoreCache];
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int ntiles = a.meta[2];
  const int nqb = (a.q_len + kSparseQBBroadcast - 1) / kSparseQBBroadcast;   // broadcast: query blocks
  const int per_item = a.broadcast ? nqb * a.heads : a.heads;
  for (int idx = blockIdx.x * 4 + w; idx < ntiles; idx += gridDim.x * 4) {
    const int item = idx / per_item;
    const int rem = idx - item * per_item;
    const int4 it = a.items[item];
    const int b = __builtin_amdgcn_readfirstlane(it.x);
    const int n = __builtin_amdgcn_readfirstlane(it.w);
    const int m = a.broadcast ? rem / a.heads : __builtin_amdgcn_readfirstlane(it.y);
    const int h = a.broadcast ? rem % a.heads : rem;
    // candidates: the sequence's key blocks, at most 64 x 64 of them (a lane's
    // selection bits are one 64-bit word; longer sequences keep their first 262144 keys
    // as candidates)
    const int nkv = min((n + kFwdBN - 1) / kFwdBN, 64 * 64);
    const int cnt = min(a.topk, nkv);
    const int qg = a.broadcast ? m : a.q_first[b] + m;   // pooled query block
    const int qnat = a.broadcast ? b * nqb + m : qg;      // natural query block index
    const float* pq = a.pooled_q + ((int64_t)h * a.q_cap + qg) * D;
    const float* pk = a.pooled_k + ((int64_t)h * a.kv_cap + a.kv_first[b]) * D;
    for (int d = lane; d < D; d += 64) pq_lds[w][d] = pq[d];
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    auto score = [&](int j) {
      const float* kr = pk + (int64_t)j * D;
      float s = 0.f;
#pragma unroll 8
      for (int d = 0; d < D; d += 4) {
        const f32x4 kv = *reinterpret_cast<const f32x4*>(kr + d);
        s = fmaf(pq_lds[w][d], kv[0], s);
        s = fmaf(pq_lds[w][d + 1], kv[1], s);
        s = fmaf(pq_lds[w][d + 2], kv[2], s);
        s = fmaf(pq_lds[w][d + 3], kv[3], s);
      }
      return s * a.scale;
    };
    for (int j = lane; j < min(nkv, kScoreCache); j += 64) sc_lds[w][j] = score(j);
    // k rounds; the blocks a lane owns are j = lane + 64 u, with their selection bits
    uint64_t mine = 0;   // bit u: block lane + 64 u selected (u < 64)
    float prev_s = INFINITY;
    int prev_j = -1;
    for (int t = 0; t < cnt; ++t) {
      float best_s = -INFINITY;
      int best_j = 0x7fffffff;
      for (int j = lane; j < nkv; j += 64) {
        const float s = j < kScoreCache ? sc_lds[w][j] : score(j);
        if (ranks_before(prev_s, prev_j, s, j) && ranks_before(s, j, best_s, best_j)) {
          best_s = s;
          best_j = j;
        }
      }
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) {
        const float os = __shfl_xor(best_s, off);
        const int oj = __shfl_xor(best_j, off);
        if (ranks_before(os, oj, best_s, best_j)) {
          best_s = os;
          best_j = oj;
        }
      }
      prev_s = best_s;
      prev_j = best_j;
      if ((best_j & 63) == lane) mine |= 1ull << (best_j >> 6);
    }
    // ascending list: chunk u of 64 blocks at a time, positions from a ballot count
    int* tb = a.tile_blocks + (int64_t)idx * a.topk;
    int* ob = a.out_blocks ? a.out_blocks + ((int64_t)h * a.out_cap + qnat) * a.topk : nullptr;
    int base = 0;
    for (int u = 0; u * 64 < nkv && base < cnt; ++u) {
      const bool sel = (mine >> u) & 1;
      const uint64_t bal = __ballot(sel);
      if (sel) {
        const int pos = base + __popcll(bal & ((1ull << lane) - 1ull));
        tb[pos] = 64 * u + lane;
        if (ob) ob[pos] = 64 * u + lane;
      }
      base += __popcll(bal);
    }
    if (ob)
      for (int t = cnt + lane; t < a.topk; t += 64) ob[t] = -1;
  }
}

}  // namespace

hipError_t launch_sparse_select(const Problem& p, const Plan& plan, const Sparse& sp, hipStream_t s) {
  const int D = p.head_dim;
  // pooled key blocks (jagged, 64 keys) and query blocks (broadcast: the shared query
  // sequence; self: jagged, 128 rows)
  auto pool = [&](auto kernel) {
    hipLaunchKernelGGL(kernel, dim3((unsigned)sp.kv_blocks_cap), dim3(256), 0, s,
                       static_cast<const bf16*>(p.k), p.heads, p.offsets, p.off64, p.batch, sp.kv_first,
                       kFwdBN, (int64_t)0, sp.pooled_k, sp.kv_blocks_cap);
    if (p.broadcast) {
      hipLaunchKernelGGL(kernel, dim3((unsigned)sp.q_blocks_cap), dim3(256), 0, s,
                         static_cast<const bf16*>(p.q), p.heads, p.offsets, p.off64, p.batch,
                         static_cast<const int*>(nullptr), kSparseQBBroadcast, (int64_t)p.q_len, sp.pooled_q,
                         sp.q_blocks_cap);
    } else {
      hipLaunchKernelGGL(kernel, dim3((unsigned)sp.q_blocks_cap), dim3(256), 0, s,
                         static_cast<const bf16*>(p.q), p.heads, p.offsets, p.off64, p.batch, sp.q_first,
                         kSparseQBSelf, (int64_t)0, sp.pooled_q, sp.q_blocks_cap);
    }
  };
  D == 128 ? pool(pool_blocks_kernel<128>) : pool(pool_blocks_kernel<64>);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;

  SelectArgs a;
  a.items = plan.items;
  a.meta = plan.meta;
  a.kv_first = sp.kv_first;
  a.q_first = sp.q_first;
  a.pooled_k = sp.pooled_k;
  a.pooled_q = sp.pooled_q;
  a.tile_blocks = sp.tile_blocks;
  a.out_blocks = sp.out_blocks;
  a.kv_cap = sp.kv_blocks_cap;
  a.q_cap = sp.q_blocks_cap;
  a.out_cap = p.broadcast ? (int64_t)p.batch * ((p.q_len + kSparseQBBroadcast - 1) / kSparseQBBroadcast)
                          : sp.q_blocks_cap;
  a.heads = p.heads;
  a.q_len = p.q_len;
  a.broadcast = p.broadcast;
  a.topk = p.topk;
  a.scale = p.scale;
  const int64_t tiles =
      fwd_max_items(p) *
      (p.broadcast ? ((p.q_len + kSparseQBBroadcast - 1) / kSparseQBBroadcast) * p.heads : p.heads);
  const int64_t wg = std::max<int64_t>(1, std::min<int64_t>((tiles + 3) / 4, (int64_t)device_cu_count() * 16));
  if (D == 128) {
    hipLaunchKernelGGL(select_blocks_kernel<128>, dim3((unsigned)wg), dim3(256), 0, s, a);
  } else {
    hipLaunchKernelGGL(select_blocks_kernel<64>, dim3((unsigned)wg), dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace jfa
