// Host-side interface between the C ABI layer and the kernel translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "jfa.h"

namespace jfa {

// Forward tile geometry.  A forward tile is (sequence, block of BM query rows, head);
// every wave owns 32 query rows and K/V stream through LDS in blocks of kFwdBN keys.
constexpr int kFwdBN = 64;
// Backward tile geometry: a tile is (sequence, block of 32 * bwd_waves(p) keys,
// head); every wave owns 32 keys and the query rows stream in blocks of kBwdBQ.
constexpr int kBwdBQ = 32;
// Broadcast-mode dQ accumulates into one fp32 stripe per XCD.
constexpr int kDqStripes = 8;

struct Problem {
  const void* q;
  const void* k;
  const void* v;
  const void* offsets;
  int off64;
  int batch;
  int heads;
  int head_dim;
  int q_len;          // Lq in broadcast mode, 0 in self mode
  int64_t total_kv;   // T
  int64_t rows;       // output rows: batch * Lq or T
  int broadcast;
  int causal;
  float scale;
  int rope = 0;       // the backward applies the rotary conjugate (no direct dQ store)
  int topk = 0;       // block-sparse forward: key blocks kept per query block (0: dense)
  int mx = 0;         // the MXFP8 forward (its own workgroup size in self mode)
};

// Block-sparse forward: the method's block sizes (include/jfa.h).  The sparse
// forward kernel takes one query block per workgroup (32 rows per wave), so these
// fix its wave counts, and its key blocks are the dense forward's K/V blocks.
constexpr int kSparseQBBroadcast = JFA_SPARSE_QUERY_BLOCK_BROADCAST;
constexpr int kSparseQBSelf = JFA_SPARSE_QUERY_BLOCK_SELF;
static_assert(JFA_SPARSE_KEY_BLOCK == kFwdBN, "sparse key blocks are the forward's K/V blocks");
static_assert(kSparseQBBroadcast % 32 == 0 && kSparseQBBroadcast / 32 <= 8 && kSparseQBSelf % 32 == 0 &&
                  kSparseQBSelf / 32 <= 8,
              "a sparse query block must be whole 32-row waves of one workgroup");
inline int sparse_qb(const Problem& p) { return p.broadcast ? kSparseQBBroadcast : kSparseQBSelf; }
constexpr int kSparseMaxTopk = 64;

// Workspace of the block-sparse forward (all device pointers).
struct Sparse {
  int* kv_first = nullptr;      // [B + 1] first global key block of each sequence
  int* q_first = nullptr;       // [B + 1] first global query block (self mode)
  float* pooled_k = nullptr;    // [H][key blocks][D] mean key rows
  float* pooled_q = nullptr;    // [H][query blocks][D] mean query rows
  int* tile_blocks = nullptr;   // [tiles][topk] selected key blocks, in forward tile order
  int* out_blocks = nullptr;    // optional [H][query blocks][topk], natural order, -1 padded
  int64_t kv_blocks_cap = 0;    // capacity of pooled_k's block dimension
  int64_t q_blocks_cap = 0;     // capacity of pooled_q's block dimension
};

// Rotary-embedding conjugate of the backward: fp32 tables [max_pos][D/2] and int32
// positions of the query rows ([q rows]) and key rows ([T]), clamped to
// [0, max_pos).  Inactive when cos is null.
struct Rope {
  const float* cos = nullptr;
  const float* sin = nullptr;
  const int* pos_q = nullptr;
  const int* pos_k = nullptr;
  int max_pos = 0;
};

// Plan written on the device: meta[0] = number of items, meta[1] = dynamic-schedule
// counter, meta[2] = number of tiles.  Forward: meta[4 .. 4 + kFwdClassMax) =
// per-class counters of the broadcast-mode dynamic schedule.  Backward of a split
// call (maybe_single_tile): meta[2] counts the tiles of the first list (sequences
// longer than one tile), meta[3] those of the second (sequences within one tile,
// which write their dQ directly), meta[4] is the second list's counter and meta[5]
// its first item; otherwise meta[3] = 0.
// items[i] = (sequence b, block, offsets[b], offsets[b + 1] - offsets[b]).
constexpr int kFwdClassMax = 12;
struct Plan {
  int* meta;
  int4* items;
  int64_t max_items;
};

int fwd_waves(const Problem& p);                 // waves per forward workgroup
int64_t fwd_max_items(const Problem& p);         // capacity of the forward item list
int64_t bwd_max_items(const Problem& p);         // capacity of the backward item list
int bwd_waves(const Problem& p);                 // waves per backward workgroup (2, 4 or 8)
bool single_tile_allowed(const Problem& p);      // the single-tile backward path may be used
bool maybe_single_tile(const Problem& p);        // ... and the plan splits the tiles for it

hipError_t launch_plan_fwd(const Problem& p, const Plan& plan, int sched, hipStream_t s);
hipError_t launch_plan_sparse(const Problem& p, int* kv_first, int* q_first, hipStream_t s);
// Pooling and top-k selection of the block-sparse forward (after the forward plan).
hipError_t launch_sparse_select(const Problem& p, const Plan& plan, const Sparse& sp, hipStream_t s);
hipError_t launch_fwd_sparse(const Problem& p, const Plan& plan, int sched, const Sparse& sp, void* o,
                             float* lse, hipStream_t s);
hipError_t launch_fwd(const Problem& p, const Plan& plan, int sched, void* o, float* lse,
                      hipStream_t s);

// MXFP8 forward operands (device pointers; layouts in the MXFP8 source).
struct MxOperands {
  const void* q8;   // E4M3 [q rows, H, D]
  const void* qs;   // E8M0 [q rows, H, D / 32]
  const void* k8;   // E4M3 [T, H, D]
  const void* ks;   // E8M0 [T, H, D / 32]
  const void* v8;   // E4M3 [G, H, D, 32], G = mx_v_blocks(B, T)
  const void* vs;   // E8M0 [G, H, D]
};
int64_t mx_v_blocks(int64_t batch, int64_t total_kv);
hipError_t launch_mx_quantize_rows(const void* x, int64_t rows, int heads, int head_dim, void* val, void* scl,
                                   hipStream_t s);
hipError_t launch_mx_quantize_v(const Problem& p, const void* v, void* val, void* scl, hipStream_t s);
// After the forward plan (launch_plan_fwd with the same problem).
hipError_t launch_fwd_mx(const Problem& p, const Plan& plan, const MxOperands& x, void* o, float* lse,
                         hipStream_t s);

// rowstat: [heads][rows] pairs (LSE log2 e, delta = rowsum(dO * O)), 2 floats each,
// and the zeroed dQ accumulator.  Runs after the backward plan; in a split call only
// for the rows of the plan's first list (the single-tile tiles form delta themselves
// and write dQ directly).
hipError_t launch_bwd_pre(const Problem& p, const void* o, const void* d_o, const float* lse,
                          float* rowstat, float* dq_acc, int64_t dq_acc_elems, const Plan& plan,
                          hipStream_t s);
hipError_t launch_plan_bwd(const Problem& p, const Plan& plan, int sched, hipStream_t s);
// lse: the forward's [heads][rows] LSE, read instead of rowstat by the tiles of a
// split call's second list (each holds a whole self-mode sequence).
hipError_t launch_bwd(const Problem& p, const Plan& plan, int sched, const float* rowstat,
                      const float* lse, const void* d_o, float* dq_acc, void* dq, void* dk, void* dv,
                      const Rope& rope, hipStream_t s);
// In a split call only the rows of the plan's first list (the others' tiles wrote dQ).
hipError_t launch_dq_finalize(const Problem& p, const float* dq_acc, void* dq, const Plan& plan,
                              const Rope& rope, hipStream_t s);

// Number of compute units of the current device (cached per device).
int device_cu_count();
// Persistent grid size for a kernel: CUs x resident workgroups, a multiple of 8.
int persistent_grid(const void* kernel, int block_threads, int64_t max_tiles);

}  // namespace jfa
