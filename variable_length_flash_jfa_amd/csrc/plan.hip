// Device-side tile planners.
//
// Forward: tiles are sorted by the number of K/V blocks they visit (descending)
// so that the persistent forward kernel can deal them boustrophedon across its
// workgroups ("Meta's TLX attention kernel outpaces FlashAttention-4 on B200",
// section "Five changes unlocked the gains", item 1; "Optimizing Jagged Flash
// Attention with TLX" reading note, section "Why both static and dynamic
// balancing help").  The pages sort on the host; here one workgroup does a
// counting sort on the device so that a call needs no device-to-host copy of the
// offsets and no synchronisation.
//
// Backward: the list of valid (sequence, K/V block) pairs is precomputed from a
// prefix sum of per-sequence block counts ("Optimizing Jagged Flash Attention with
// TLX", same section; "TLX JFA: Meta's Blackwell Attention Kernel", section
// "Structural changes and layered opts", item 1), and the kernel deals them
// round-robin.
#include "jfa_device.h"
#include "jfa_internal.h"

namespace jfa {
namespace {

constexpr int kPlanThreads = 1024;
constexpr int kKeys = 1024;   // sort buckets; larger costs share the last bucket

__device__ __forceinline__ int wave_max(int x) {
#pragma unroll
  for (int s = 32; s >= 1; s >>= 1) x = max(x, __shfl_xor(x, s));
  return x;
}

// Exclusive scan over the 1024 threads of the block; *total receives the sum.
__device__ int block_exclusive_scan(int x, int* wave_sums, int* total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int incl = x;
#pragma unroll
  for (int s = 1; s < 64; s <<= 1) {
    const int y = __shfl_up(incl, s);
    if (lane >= s) incl += y;
  }
  if (lane == 63) wave_sums[w] = incl;
  __syncthreads();
  if (w == 0) {
    int v = lane < kPlanThreads / 64 ? wave_sums[lane] : 0;
    int vi = v;
#pragma unroll
    for (int s = 1; s < 64; s <<= 1) {
      const int y = __shfl_up(vi, s);
      if (lane >= s) vi += y;
    }
    if (lane < kPlanThreads / 64) wave_sums[lane] = vi - v;
    if (lane == kPlanThreads / 64 - 1) wave_sums[kPlanThreads / 64] = vi;
  }
  __syncthreads();
  const int r = wave_sums[w] + incl - x;
  *total = wave_sums[kPlanThreads / 64];
  __syncthreads();
  return r;
}

// Wave-aggregated LDS atomic add of 1 to counters[key]: one atomic per distinct
// key among the active lanes.  Returns the old value plus the lane's rank.
__device__ __forceinline__ int aggregated_increment(int* counters, int key) {
  const int lane = threadIdx.x & 63;
  unsigned long long pending = __ballot(1);
  int result = 0;
  while (pending) {
    const int leader = __ffsll((long long)pending) - 1;
    const int lk = __shfl(key, leader);
    const unsigned long long same = __ballot(key == lk) & pending;
    if (key == lk) {
      const int rank = __popcll(same & ((1ull << lane) - 1ull));
      int base = 0;
      if (lane == leader) base = atomicAdd(&counters[lk], __popcll(same));
      base = __shfl(base, leader);
      result = base + rank;
    }
    pending &= ~same;
  }
  return result;
}

// The planners walk the batch in segments of kSeg sequences whose offsets are first
// copied into LDS with coalesced loads (offsets < 2^30 fit in int); each thread then
// takes a run of at most kSeg / kPlanThreads consecutive sequences of the segment.
constexpr int kSeg = 8192;
struct Segment {
  int b0;    // first sequence of the segment
  int len;   // sequences in it
  int bb, be;   // this thread's run [bb, be) (segment-relative)
};
// Copies offsets[b0 .. b0 + len] of segment s into offs; returns the thread's run.
__device__ Segment stage_segment(const void* offsets, int off64, int batch, int s, int* offs) {
  Segment g;
  g.b0 = s * kSeg;
  g.len = min(kSeg, batch - g.b0);
  __syncthreads();   // earlier readers of offs are done
  for (int i = threadIdx.x; i <= g.len; i += kPlanThreads) offs[i] = (int)load_offset(offsets, off64, g.b0 + i);
  __syncthreads();
  const int per = (g.len + kPlanThreads - 1) / kPlanThreads;
  g.bb = min(g.len, (int)threadIdx.x * per);
  g.be = min(g.len, g.bb + per);
  return g;
}

struct PlanFwdArgs {
  const void* offsets;
  int off64;
  int batch;
  int q_len;
  int bm;          // query rows per tile
  int broadcast;
  int causal;
  int heads;
  int sched;
  int topk;        // block-sparse forward: a tile visits at most topk key blocks (0: dense)
  int4* items;
  int* meta;
};

// Items: broadcast mode -> one item per sequence (its ceil(Lq / BM) x H tiles share
// the cost); self mode -> one item per (sequence, query block).  Cost = number of
// kFwdBN-key blocks the tile visits.
__device__ __forceinline__ int fwd_items_of(const PlanFwdArgs& a, int64_t n) {
  return a.broadcast ? 1 : (int)((n + a.bm - 1) / a.bm);
}
__device__ __forceinline__ int fwd_cost(const PlanFwdArgs& a, int64_t n, int m) {
  int64_t kv = n;
  if (a.causal) kv = min(n, (int64_t)(m + 1) * a.bm);
  int64_t c = (kv + kFwdBN - 1) / kFwdBN;
  if (a.topk > 0) c = min(c, (int64_t)a.topk);
  return (int)min(c, (int64_t)(kKeys - 1));
}

__global__ __launch_bounds__(kPlanThreads) void plan_fwd_kernel(PlanFwdArgs a) {
  static_assert(kKeys == kPlanThreads, "one sort bucket per thread");
  constexpr int kWaves = kPlanThreads / 64;
  __shared__ int wave_sums[kWaves + 1];
  __shared__ int hist[kKeys];
  __shared__ int offs[kSeg + 1];
  __shared__ int first_item[kPlanThreads];     // a segment's first item of each thread's run
  __shared__ int wave_hist[kWaves][kKeys];     // per-wave counts of a chunk's items by cost
  __shared__ int one_cost;
  const int tid = threadIdx.x;
  const int nseg = (a.batch + kSeg - 1) / kSeg;
  auto seq_len = [&](int b) { return (int64_t)(offs[b + 1] - offs[b]); };
  int total = 0;

  if (a.sched == kIdentity) {
    for (int sg = 0; sg < nseg; ++sg) {
      const Segment g = stage_segment(a.offsets, a.off64, a.batch, sg, offs);
      int count = 0;
      for (int b = g.bb; b < g.be; ++b) count += fwd_items_of(a, seq_len(b));
      int tot = 0;
      int pos = total + block_exclusive_scan(count, wave_sums, &tot);
      for (int b = g.bb; b < g.be; ++b) {
        const int mi = fwd_items_of(a, seq_len(b));
        for (int m = 0; m < mi; ++m) a.items[pos++] = make_int4(g.b0 + b, m, offs[b], (int)seq_len(b));
      }
      total += tot;
    }
  } else {
    for (int i = tid; i < kKeys; i += kPlanThreads) hist[i] = 0;
    // pass 1: histogram of costs (and the item count)
    for (int sg = 0; sg < nseg; ++sg) {
      const Segment g = stage_segment(a.offsets, a.off64, a.batch, sg, offs);
      int count = 0;
      for (int b = g.bb; b < g.be; ++b) count += fwd_items_of(a, seq_len(b));
      int tot = 0;
      block_exclusive_scan(count, wave_sums, &tot);
      total += tot;
      const int rounds = wave_max(count);
      int b = g.bb, m = 0, mi = 0;
      int64_t n = 0;
      for (int r = 0; r < rounds; ++r) {
        if (r < count) {
          while (m >= mi) {  // advance to the next sequence that has items
            n = seq_len(b);
            mi = fwd_items_of(a, n);
            m = 0;
            if (mi == 0) ++b;
          }
          aggregated_increment(hist, fwd_cost(a, n, m));
          if (++m >= mi) ++b;
        }
      }
    }
    __syncthreads();
    // when every item has the same cost the natural order is the sorted order
    if (tid == 0) one_cost = 0;
    __syncthreads();
    if (hist[tid] == total) one_cost = 1;
    __syncthreads();
    if (one_cost) {
      int base = 0;
      for (int sg = 0; sg < nseg; ++sg) {
        const Segment g = stage_segment(a.offsets, a.off64, a.batch, sg, offs);
        int count = 0;
        for (int b = g.bb; b < g.be; ++b) count += fwd_items_of(a, seq_len(b));
        int tot = 0;
        int pos = base + block_exclusive_scan(count, wave_sums, &tot);
        for (int b = g.bb; b < g.be; ++b) {
          const int mi = fwd_items_of(a, seq_len(b));
          for (int m = 0; m < mi; ++m) a.items[pos++] = make_int4(g.b0 + b, m, offs[b], (int)seq_len(b));
        }
        base += tot;
      }
    } else {
      // descending exclusive scan of the histogram: cursor[k] = #items with cost > k
      {
        const int k = kKeys - 1 - tid;
        int tot = 0;
        const int start = block_exclusive_scan(hist[k], wave_sums, &tot);
        __syncthreads();
        hist[k] = start;
      }
#pragma unroll
      for (int w = 0; w < kWaves; ++w) wave_hist[w][tid] = 0;
      __syncthreads();
      // pass 2: a stable counting sort.  Each segment's items are taken 1024 at a time
      // in (sequence, query block) order, one per thread; an item's place in its cost
      // bucket is the bucket's running cursor, plus the chunk's items of that cost in
      // lower waves, plus those in lower lanes of its own wave.  Equal costs thus keep
      // (sequence, query block) order, and the tile order does not depend on timing.
      const int lane = tid & 63, wv = tid >> 6;
      for (int sg = 0; sg < nseg; ++sg) {
        const Segment g = stage_segment(a.offsets, a.off64, a.batch, sg, offs);
        const int per = (g.len + kPlanThreads - 1) / kPlanThreads;   // as in stage_segment
        int count = 0;
        for (int b = g.bb; b < g.be; ++b) count += fwd_items_of(a, seq_len(b));
        int tot = 0;
        first_item[tid] = block_exclusive_scan(count, wave_sums, &tot);
        __syncthreads();
        for (int c0 = 0; c0 < tot; c0 += kPlanThreads) {
          const int i = c0 + tid;
          int key = -1;
          int4 item = make_int4(0, 0, 0, 0);
          if (i < tot) {
            // the thread whose run holds item i: the last one whose run starts at or before i
            int lo = 0, hi = kPlanThreads - 1;
            while (lo < hi) {
              const int mid = (lo + hi + 1) >> 1;
              if (first_item[mid] <= i) lo = mid; else hi = mid - 1;
            }
            int local = i - first_item[lo];
            const int bb = min(g.len, lo * per), be = min(g.len, bb + per);
            for (int b = bb; b < be; ++b) {
              const int64_t n = seq_len(b);
              const int mi = fwd_items_of(a, n);
              if (local < mi) {
                key = fwd_cost(a, n, local);
                item = make_int4(g.b0 + b, local, offs[b], (int)n);
                break;
              }
              local -= mi;
            }
          }
          // rank among the wave's items of the same cost, in lane order
          unsigned long long pending = __ballot(key >= 0);
          int rank = 0;
          while (pending) {
            const int leader = __ffsll((long long)pending) - 1;
            const int lk = __shfl(key, leader);
            const unsigned long long same = __ballot(key == lk) & pending;
            if (key == lk) rank = __popcll(same & ((1ull << lane) - 1ull));
            if (lane == leader) wave_hist[wv][lk] = __popcll(same);
            pending &= ~same;
          }
          __syncthreads();
          if (key >= 0) {
            int before = 0;
            for (int w = 0; w < wv; ++w) before += wave_hist[w][key];
            a.items[hist[key] + before + rank] = item;
          }
          __syncthreads();
          // advance the cursors past this chunk and clear its counts
          {
            int add = 0;
#pragma unroll
            for (int w = 0; w < kWaves; ++w) {
              add += wave_hist[w][tid];
              wave_hist[w][tid] = 0;
            }
            hist[tid] += add;
          }
          __syncthreads();
        }
      }
    }
  }
  if (tid == 0) {
    const int per_item = a.broadcast ? ((a.q_len + a.bm - 1) / a.bm) * a.heads : a.heads;
    a.meta[0] = total;
    a.meta[1] = 0;
    a.meta[2] = total * per_item;
  }
  if (tid < kFwdClassMax) a.meta[4 + tid] = 0;
}

struct PlanBwdArgs {
  const void* offsets;
  int off64;
  int batch;
  int heads;
  int bn;          // keys per backward tile
  int split;       // sequences of one tile get a list of their own (maybe_single_tile)
  int4* items;
  int* meta;
};

// Valid (sequence, K/V block) pairs in natural order, in up to two lists; tile t of
// a list = (list[t / H], t % H).  Each item also carries the sequence's first row and
// length (int32: the library rejects T >= 2^30), so a tile's geometry is one 16-byte
// load.
// Without split every tile reduce-adds its dQ partial: one list, meta[2] = its tiles,
// meta[3] = 0.
// With split (self mode, where the single-tile backward may run) a sequence of 1..bn
// keys goes to a second list, after the first.  Such a tile sees all keys of its
// queries, so its dQ is final and is written directly (with the rotary conjugate only
// where the tiles can rotate dQ, see single_tile_allowed); the tiles of longer
// sequences reduce-add.  meta[2] = tiles of the first list (M H), meta[3] = tiles of
// the second, meta[5] = M, the second list's first item; meta[1] and meta[4] are the
// lists' dynamic-schedule counters.  In self mode an item of the first list also names
// the rows whose delta and dQ finalize the call needs: [kv0 + j bn, kv0 + min(n,
// (j + 1) bn)).
__global__ __launch_bounds__(kPlanThreads) void plan_bwd_kernel(PlanBwdArgs a) {
  __shared__ int wave_sums[kPlanThreads / 64 + 1];
  __shared__ int offs[kSeg + 1];
  const int tid = threadIdx.x;
  const int nseg = (a.batch + kSeg - 1) / kSeg;
  auto first_items = [&](int n) { return a.split && n <= a.bn ? 0 : (n + a.bn - 1) / a.bn; };
  auto second_items = [&](int n) { return a.split && n >= 1 && n <= a.bn ? 1 : 0; };
  // with split, a first pass sizes the first list
  int first_total = 0;
  if (a.split) {
    for (int sg = 0; sg < nseg; ++sg) {
      const Segment g = stage_segment(a.offsets, a.off64, a.batch, sg, offs);
      int count = 0;
      for (int b = g.bb; b < g.be; ++b) count += first_items(offs[b + 1] - offs[b]);
      int tot = 0;
      block_exclusive_scan(count, wave_sums, &tot);
      first_total += tot;
    }
  }
  int total = 0, total2 = 0;
  for (int sg = 0; sg < nseg; ++sg) {
    const Segment g = stage_segment(a.offsets, a.off64, a.batch, sg, offs);
    int count = 0, count2 = 0;
    for (int b = g.bb; b < g.be; ++b) {
      const int n = offs[b + 1] - offs[b];
      count += first_items(n);
      count2 += second_items(n);
    }
    int tot = 0, tot2 = 0;
    int pos = total + block_exclusive_scan(count, wave_sums, &tot);
    int pos2 = first_total + total2 + block_exclusive_scan(count2, wave_sums, &tot2);
    for (int b = g.bb; b < g.be; ++b) {
      const int kv0 = offs[b], n = offs[b + 1] - kv0;
      if (second_items(n)) a.items[pos2++] = make_int4(g.b0 + b, 0, kv0, n);
      const int nb = first_items(n);
      for (int j = 0; j < nb; ++j) a.items[pos++] = make_int4(g.b0 + b, j, kv0, n);
    }
    total += tot;
    total2 += tot2;
  }
  if (tid == 0) {
    a.meta[0] = total + total2;
    a.meta[1] = 0;
    a.meta[2] = total * a.heads;
    a.meta[3] = total2 * a.heads;
    a.meta[4] = 0;
    a.meta[5] = total;
  }
}

// Block-sparse forward: first global key block (64 keys) and first query block
// (kSparseQBSelf rows; self mode) of every sequence, as exclusive prefix sums:
// kv_first[b] = sum over b' < b of ceil(n_b' / 64), q_first likewise (entry B holds
// the totals).
struct PlanSparseArgs {
  const void* offsets;
  int off64;
  int batch;
  int* kv_first;
  int* q_first;
};

__global__ __launch_bounds__(kPlanThreads) void plan_sparse_kernel(PlanSparseArgs a) {
  __shared__ int wave_sums[kPlanThreads / 64 + 1];
  __shared__ int offs[kSeg + 1];
  const int nseg = (a.batch + kSeg - 1) / kSeg;
  int base_kv = 0, base_q = 0;
  for (int sg = 0; sg < nseg; ++sg) {
    const Segment g = stage_segment(a.offsets, a.off64, a.batch, sg, offs);
    int ckv = 0, cq = 0;
    for (int b = g.bb; b < g.be; ++b) {
      const int n = offs[b + 1] - offs[b];
      ckv += (n + kFwdBN - 1) / kFwdBN;
      cq += (n + kSparseQBSelf - 1) / kSparseQBSelf;
    }
    int tkv = 0, tq = 0;
    int pkv = base_kv + block_exclusive_scan(ckv, wave_sums, &tkv);
    int pq = base_q + block_exclusive_scan(cq, wave_sums, &tq);
    for (int b = g.bb; b < g.be; ++b) {
      a.kv_first[g.b0 + b] = pkv;
      a.q_first[g.b0 + b] = pq;
      const int n = offs[b + 1] - offs[b];
      pkv += (n + kFwdBN - 1) / kFwdBN;
      pq += (n + kSparseQBSelf - 1) / kSparseQBSelf;
    }
    base_kv += tkv;
    base_q += tq;
  }
  if (threadIdx.x == 0) {
    a.kv_first[a.batch] = base_kv;
    a.q_first[a.batch] = base_q;
  }
}

}  // namespace

hipError_t launch_plan_sparse(const Problem& p, int* kv_first, int* q_first, hipStream_t s) {
  PlanSparseArgs a;
  a.offsets = p.offsets;
  a.off64 = p.off64;
  a.batch = p.batch;
  a.kv_first = kv_first;
  a.q_first = q_first;
  hipLaunchKernelGGL(plan_sparse_kernel, dim3(1), dim3(kPlanThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_plan_fwd(const Problem& p, const Plan& plan, int sched, hipStream_t s) {
  PlanFwdArgs a;
  a.offsets = p.offsets;
  a.off64 = p.off64;
  a.batch = p.batch;
  a.q_len = p.q_len;
  a.bm = 32 * fwd_waves(p);
  a.broadcast = p.broadcast;
  a.causal = p.causal;
  a.heads = p.heads;
  a.sched = sched;
  a.topk = p.topk;
  a.items = plan.items;
  a.meta = plan.meta;
  hipLaunchKernelGGL(plan_fwd_kernel, dim3(1), dim3(kPlanThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_plan_bwd(const Problem& p, const Plan& plan, int /*sched*/, hipStream_t s) {
  PlanBwdArgs a;
  a.offsets = p.offsets;
  a.off64 = p.off64;
  a.batch = p.batch;
  a.heads = p.heads;
  a.bn = 32 * bwd_waves(p);
  a.split = maybe_single_tile(p) ? 1 : 0;
  a.items = plan.items;
  a.meta = plan.meta;
  hipLaunchKernelGGL(plan_bwd_kernel, dim3(1), dim3(kPlanThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace jfa
