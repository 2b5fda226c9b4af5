// C ABI of libjfa.so: argument checks, workspace sizing and carving, launches.
// The declarations and their documentation are in include/jfa.h.
#include "jfa.h"

#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <utility>
#include <vector>

#include "jfa_internal.h"

namespace {

thread_local char g_error[512] = "";
std::atomic<int> g_schedule{JFA_SCHED_DYNAMIC};

jfa_status_t fail(jfa_status_t st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_error, sizeof(g_error), fmt, ap);
  va_end(ap);
  return st;
}

jfa_status_t hip_fail(hipError_t e, const char* what) {
  return fail(JFA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}
jfa_status_t hip_fail(hipError_t e, const char* fn, const char* what) {
  return fail(JFA_ERR_HIP, "%s: %s: %s", fn, what, hipGetErrorString(e));
}

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

struct Sizes {
  bool ok;
  const char* why;
  jfa_status_t st;
};

Sizes check_sizes(int64_t batch, int64_t heads, int64_t head_dim, int64_t q_len, int64_t total_kv,
                  int broadcast_q, int causal) {
  if (head_dim != 64 && head_dim != 128)
    return {false, "head_dim must be 64 or 128", JFA_ERR_UNSUPPORTED};
  if (broadcast_q && causal)
    return {false, "causal masking is defined for self-attention only (broadcast_q=1, causal=1)",
            JFA_ERR_UNSUPPORTED};
  if (batch < 0 || heads < 1 || q_len < 0 || total_kv < 0)
    return {false, "sizes must be non-negative and num_heads >= 1", JFA_ERR_INVALID_ARGUMENT};
  if (broadcast_q && q_len < 1)
    return {false, "broadcast mode needs q_len >= 1", JFA_ERR_INVALID_ARGUMENT};
  if (!broadcast_q && q_len != 0)
    return {false, "self mode needs q_len == 0 (queries come from the packed sequences)",
            JFA_ERR_INVALID_ARGUMENT};
  // 32-bit limits of the tile indices used on the device
  const int64_t lim = (int64_t)1 << 30;
  const int64_t rows = broadcast_q ? batch * q_len : total_kv;
  if (batch >= lim || total_kv >= lim || q_len >= lim || heads >= 4096 || rows >= ((int64_t)1 << 36))
    return {false, "problem too large for this library build", JFA_ERR_UNSUPPORTED};
  if ((total_kv / 128 + batch) * heads >= lim)
    return {false, "too many tiles for this library build", JFA_ERR_UNSUPPORTED};
  return {true, "", JFA_OK};
}

jfa::Problem make_problem(const void* q, const void* k, const void* v, const void* offsets,
                          int off64, int64_t batch, int64_t heads, int64_t head_dim, int64_t q_len,
                          int64_t total_kv, int broadcast_q, int causal, float scale) {
  jfa::Problem p;
  p.q = q;
  p.k = k;
  p.v = v;
  p.offsets = offsets;
  p.off64 = off64 ? 1 : 0;
  p.batch = (int)batch;
  p.heads = (int)heads;
  p.head_dim = (int)head_dim;
  p.q_len = (int)q_len;
  p.total_kv = total_kv;
  p.rows = broadcast_q ? batch * q_len : total_kv;
  p.broadcast = broadcast_q ? 1 : 0;
  p.causal = causal ? 1 : 0;
  p.scale = scale;
  return p;
}

size_t fwd_ws_bytes(const jfa::Problem& p) {
  return kAlign + align_up(64) + align_up((size_t)jfa::fwd_max_items(p) * sizeof(int4));
}

// Block-sparse forward: capacities of the pooled key / query blocks and of the
// natural-order selection output.
int64_t sparse_kv_cap(const jfa::Problem& p) { return p.total_kv / jfa::kFwdBN + p.batch + 1; }
int64_t sparse_bcast_qblocks(const jfa::Problem& p) {   // query blocks of the broadcast query
  return (p.q_len + jfa::kSparseQBBroadcast - 1) / jfa::kSparseQBBroadcast;
}
int64_t sparse_q_cap(const jfa::Problem& p) {
  return p.broadcast ? sparse_bcast_qblocks(p) : p.total_kv / jfa::kSparseQBSelf + p.batch + 1;
}
int64_t sparse_out_qblocks(const jfa::Problem& p) {
  return p.broadcast ? (int64_t)p.batch * sparse_bcast_qblocks(p) : sparse_q_cap(p);
}
int64_t sparse_tiles(const jfa::Problem& p) {
  return jfa::fwd_max_items(p) * (p.broadcast ? sparse_bcast_qblocks(p) * p.heads : p.heads);
}

size_t fwd_sparse_ws_bytes(const jfa::Problem& p) {
  return fwd_ws_bytes(p) + 2 * align_up((size_t)(p.batch + 1) * sizeof(int)) +
         align_up((size_t)p.heads * sparse_kv_cap(p) * p.head_dim * sizeof(float)) +
         align_up((size_t)p.heads * sparse_q_cap(p) * p.head_dim * sizeof(float)) +
         align_up((size_t)sparse_tiles(p) * p.topk * sizeof(int));
}

size_t bwd_ws_bytes(const jfa::Problem& p) {
  const int64_t q_rows = p.broadcast ? (int64_t)p.q_len * jfa::kDqStripes : p.total_kv;
  return kAlign + align_up(64) + align_up((size_t)jfa::bwd_max_items(p) * sizeof(int4)) +
         align_up((size_t)p.heads * p.rows * 2 * sizeof(float)) +
         align_up((size_t)q_rows * p.heads * p.head_dim * sizeof(float));
}

// ---- optional per-launch event timing (jfa_profile_*) ----------------------------
struct ProfRecord {
  const char* name;
  hipEvent_t start, stop;
};
thread_local bool g_prof = false;
thread_local std::vector<ProfRecord> g_prof_records;
thread_local std::vector<hipEvent_t> g_prof_pool;

hipEvent_t prof_event() {
  if (!g_prof_pool.empty()) {
    hipEvent_t e = g_prof_pool.back();
    g_prof_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

// Runs one launch; when profiling is on, brackets it with events on `s`.
template <typename F>
hipError_t timed_launch(const char* name, hipStream_t s, F&& launch) {
  if (!g_prof) return launch();
  hipEvent_t a = prof_event(), b = prof_event();
  if (a) (void)hipEventRecord(a, s);
  const hipError_t e = launch();
  if (b) (void)hipEventRecord(b, s);
  if (a && b) g_prof_records.push_back({name, a, b});
  return e;
}

bool misaligned(const void* ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15) != 0; }

char* carve(char*& cur, size_t bytes) {
  char* r = cur;
  cur += align_up(bytes);
  return r;
}

}  // namespace

namespace jfa {

int device_cu_count() {
  static std::mutex mu;
  static std::map<int, int> cache;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  std::lock_guard<std::mutex> lock(mu);
  auto it = cache.find(dev);
  if (it != cache.end()) return it->second;
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    cus = 256;
  cache[dev] = cus;
  return cus;
}

int persistent_grid(const void* kernel, int block_threads, int64_t max_tiles) {
  static std::mutex mu;
  static std::map<std::pair<const void*, int>, int> cache;
  int dev = 0;
  (void)hipGetDevice(&dev);
  int per_cu = 0;
  {
    std::lock_guard<std::mutex> lock(mu);
    auto key = std::make_pair(kernel, dev);
    auto it = cache.find(key);
    if (it != cache.end()) {
      per_cu = it->second;
    } else {
      if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, block_threads, 0) != hipSuccess ||
          per_cu < 1)
        per_cu = 1;
      cache[key] = per_cu;
    }
  }
  int64_t grid = (int64_t)device_cu_count() * per_cu;
  const int64_t cap = (max_tiles + 7) / 8 * 8;
  if (grid > cap) grid = cap;
  grid = grid / 8 * 8;
  if (grid < 8) grid = 8;
  return (int)grid;
}

}  // namespace jfa

extern "C" {

jfa_status_t jfa_set_schedule(int schedule) {
  if (schedule < JFA_SCHED_SORTED_ZIGZAG || schedule > JFA_SCHED_DYNAMIC)
    return fail(JFA_ERR_INVALID_ARGUMENT, "unknown schedule %d", schedule);
  g_schedule.store(schedule);
  return JFA_OK;
}

int jfa_get_schedule(void) { return g_schedule.load(); }

size_t jfa_fwd_workspace_size(int64_t batch, int64_t num_heads, int64_t head_dim, int64_t q_len,
                              int64_t total_kv, int broadcast_q, int causal) {
  if (!check_sizes(batch, num_heads, head_dim, q_len, total_kv, broadcast_q, causal).ok) return 0;
  jfa::Problem p = make_problem(nullptr, nullptr, nullptr, nullptr, 0, batch, num_heads, head_dim,
                                q_len, total_kv, broadcast_q, causal, 1.f);
  const size_t plain = fwd_ws_bytes(p);
  p.mx = 1;   // the MXFP8 forward takes the same workspace
  return std::max(plain, fwd_ws_bytes(p));
}

size_t jfa_bwd_workspace_size(int64_t batch, int64_t num_heads, int64_t head_dim, int64_t q_len,
                              int64_t total_kv, int broadcast_q, int causal) {
  if (!check_sizes(batch, num_heads, head_dim, q_len, total_kv, broadcast_q, causal).ok) return 0;
  const jfa::Problem p = make_problem(nullptr, nullptr, nullptr, nullptr, 0, batch, num_heads, head_dim,
                                      q_len, total_kv, broadcast_q, causal, 1.f);
  return bwd_ws_bytes(p);
}

}  // extern "C"

// Plan scratch of jfa_fwd_noalloc: one copy of this array per GPU, held until the
// process ends.  Host code never uses the array's name as an address (on the host it
// is only a stand-in): each device's copy is looked up once with
// hipGetSymbolAddress, with that device current, and only that pointer is passed on.
static __device__ __align__(256) char scratch[JFA_FWD_NOALLOC_SCRATCH_BYTES];

namespace {

std::mutex g_scratch_mu;
std::map<int, char*> g_scratch_ptr;   // device -> address of its copy of `scratch`

jfa_status_t scratch_address(const char* fn, char** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, fn, "hipGetDevice");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  auto it = g_scratch_ptr.find(dev);
  if (it == g_scratch_ptr.end()) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, fn, "hipGetSymbolAddress of the plan scratch");
    if (ptr == nullptr) return fail(JFA_ERR_HIP, "%s: hipGetSymbolAddress gave a null plan scratch", fn);
    it = g_scratch_ptr.emplace(dev, static_cast<char*>(ptr)).first;
  }
  *out = it->second;
  return JFA_OK;
}

// jfa_fwd (plan in the caller's workspace) and jfa_fwd_noalloc (plan in this
// device's copy of `scratch`; no event timing, so that nothing is created).
jfa_status_t fwd_impl(const char* fn, const void* q, const void* k, const void* v, const void* offsets,
                      int offsets_is_int64, int64_t batch, int64_t num_heads, int64_t head_dim,
                      int64_t q_len, int64_t total_kv, int broadcast_q, int causal, float softmax_scale,
                      void* o, float* lse, void* workspace, size_t workspace_bytes, bool noalloc,
                      void* stream) {
  g_error[0] = '\0';
  const Sizes sz = check_sizes(batch, num_heads, head_dim, q_len, total_kv, broadcast_q, causal);
  if (!sz.ok) return fail(sz.st, "%s: %s", fn, sz.why);
  if (!std::isfinite(softmax_scale) || softmax_scale <= 0.f)
    return fail(JFA_ERR_INVALID_ARGUMENT, "%s: softmax_scale must be finite and > 0", fn);
  const jfa::Problem p = make_problem(q, k, v, offsets, offsets_is_int64, batch, num_heads, head_dim,
                                      q_len, total_kv, broadcast_q, causal, softmax_scale);
  if (p.batch == 0 || p.rows == 0) return JFA_OK;
  if (!q || !offsets || !o || !lse || (!noalloc && !workspace) || (p.total_kv > 0 && (!k || !v)))
    return fail(JFA_ERR_INVALID_ARGUMENT, "%s: null pointer argument", fn);
  if (misaligned(q) || misaligned(k) || misaligned(v) || misaligned(o) || (!noalloc && misaligned(workspace)) ||
      (reinterpret_cast<uintptr_t>(lse) & 3) ||
      (reinterpret_cast<uintptr_t>(offsets) & (offsets_is_int64 ? 7 : 3)))
    return fail(JFA_ERR_INVALID_ARGUMENT, "%s: tensors must be 16-byte aligned", fn);
  const size_t need = fwd_ws_bytes(p);
  char* base = nullptr;
  if (noalloc) {
    if (need > (size_t)JFA_FWD_NOALLOC_SCRATCH_BYTES)
      return fail(JFA_ERR_WORKSPACE_TOO_SMALL,
                  "%s: the tile plan of this problem needs %zu bytes, more than the %zu bytes of plan "
                  "scratch the library holds; use jfa_fwd with a workspace",
                  fn, need, (size_t)JFA_FWD_NOALLOC_SCRATCH_BYTES);
    const jfa_status_t st = scratch_address(fn, &base);
    if (st != JFA_OK) return st;
  } else {
    if (workspace_bytes < need)
      return fail(JFA_ERR_WORKSPACE_TOO_SMALL, "%s: workspace of %zu bytes, need %zu", fn, workspace_bytes,
                  need);
    base = static_cast<char*>(workspace);
  }
  char* cur = reinterpret_cast<char*>(align_up(reinterpret_cast<uintptr_t>(base)));
  jfa::Plan plan;
  plan.meta = reinterpret_cast<int*>(carve(cur, 64));
  plan.max_items = jfa::fwd_max_items(p);
  plan.items = reinterpret_cast<int4*>(carve(cur, plan.max_items * sizeof(int4)));
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const int sched = g_schedule.load();
  // the plan kernel rewrites every word of the plan it uses, the work counter included
  hipError_t e = noalloc ? jfa::launch_plan_fwd(p, plan, sched, s)
                         : timed_launch("plan_fwd", s, [&] { return jfa::launch_plan_fwd(p, plan, sched, s); });
  if (e != hipSuccess) return hip_fail(e, fn, "plan launch");
  e = noalloc ? jfa::launch_fwd(p, plan, sched, o, lse, s)
              : timed_launch("fwd", s, [&] { return jfa::launch_fwd(p, plan, sched, o, lse, s); });
  if (e != hipSuccess) return hip_fail(e, fn, "kernel launch");
  return JFA_OK;
}

}  // namespace

extern "C" {

jfa_status_t jfa_fwd(const void* q, const void* k, const void* v, const void* offsets,
                     int offsets_is_int64, int64_t batch, int64_t num_heads, int64_t head_dim,
                     int64_t q_len, int64_t total_kv, int broadcast_q, int causal, float softmax_scale,
                     void* o, float* lse, void* workspace, size_t workspace_bytes, void* stream) {
  return fwd_impl("jfa_fwd", q, k, v, offsets, offsets_is_int64, batch, num_heads, head_dim, q_len, total_kv,
                  broadcast_q, causal, softmax_scale, o, lse, workspace, workspace_bytes, false, stream);
}

jfa_status_t jfa_fwd_noalloc(const void* q, const void* k, const void* v, const void* offsets,
                             int offsets_is_int64, int64_t batch, int64_t num_heads, int64_t head_dim,
                             int64_t q_len, int64_t total_kv, int broadcast_q, int causal,
                             float softmax_scale, void* o, float* lse, void* stream) {
  return fwd_impl("jfa_fwd_noalloc", q, k, v, offsets, offsets_is_int64, batch, num_heads, head_dim, q_len,
                  total_kv, broadcast_q, causal, softmax_scale, o, lse, nullptr, 0, true, stream);
}

namespace {

// jfa_bwd and jfa_bwd_rope; `fn` names the entry point in error messages.
jfa_status_t bwd_impl(const char* fn, const void* q, const void* k, const void* v, const void* offsets,
                      int offsets_is_int64, int64_t batch, int64_t num_heads, int64_t head_dim,
                      int64_t q_len, int64_t total_kv, int broadcast_q, int causal, float softmax_scale,
                      const void* o, const float* lse, const void* d_o, void* dq, void* dk, void* dv,
                      const jfa::Rope& rope, void* workspace, size_t workspace_bytes, void* stream) {
  g_error[0] = '\0';
  const Sizes sz = check_sizes(batch, num_heads, head_dim, q_len, total_kv, broadcast_q, causal);
  if (!sz.ok) return fail(sz.st, "%s: %s", fn, sz.why);
  if (!std::isfinite(softmax_scale) || softmax_scale <= 0.f)
    return fail(JFA_ERR_INVALID_ARGUMENT, "%s: softmax_scale must be finite and > 0", fn);
  jfa::Problem p = make_problem(q, k, v, offsets, offsets_is_int64, batch, num_heads, head_dim,
                                q_len, total_kv, broadcast_q, causal, softmax_scale);
  p.rope = rope.cos != nullptr ? 1 : 0;
  if (p.batch == 0 || p.rows == 0) return JFA_OK;
  if (!q || !offsets || !o || !lse || !d_o || !dq || !workspace ||
      (p.total_kv > 0 && (!k || !v || !dk || !dv)))
    return fail(JFA_ERR_INVALID_ARGUMENT, "%s: null pointer argument", fn);
  if (misaligned(q) || misaligned(k) || misaligned(v) || misaligned(o) || misaligned(d_o) ||
      misaligned(dq) || misaligned(dk) || misaligned(dv) || misaligned(workspace) ||
      (reinterpret_cast<uintptr_t>(lse) & 3) ||
      (reinterpret_cast<uintptr_t>(offsets) & (offsets_is_int64 ? 7 : 3)))
    return fail(JFA_ERR_INVALID_ARGUMENT, "%s: tensors must be 16-byte aligned", fn);
  const size_t need = bwd_ws_bytes(p);
  if (workspace_bytes < need)
    return fail(JFA_ERR_WORKSPACE_TOO_SMALL, "%s: workspace of %zu bytes, need %zu", fn,
                workspace_bytes, need);
  char* cur = reinterpret_cast<char*>(align_up(reinterpret_cast<uintptr_t>(workspace)));
  jfa::Plan plan;
  plan.meta = reinterpret_cast<int*>(carve(cur, 64));
  plan.max_items = jfa::bwd_max_items(p);
  plan.items = reinterpret_cast<int4*>(carve(cur, plan.max_items * sizeof(int4)));
  float* rowstat = reinterpret_cast<float*>(carve(cur, (size_t)p.heads * p.rows * 2 * sizeof(float)));
  const int64_t q_rows = p.broadcast ? (int64_t)p.q_len * jfa::kDqStripes : p.total_kv;
  const int64_t acc_elems = q_rows * p.heads * p.head_dim;
  float* dq_acc = reinterpret_cast<float*>(carve(cur, (size_t)acc_elems * sizeof(float)));
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const int sched = g_schedule.load();
  hipError_t e = timed_launch("plan_bwd", s, [&] { return jfa::launch_plan_bwd(p, plan, sched, s); });
  if (e != hipSuccess) return hip_fail(e, fn, "plan launch");
  e = timed_launch("bwd_pre", s, [&] {
    return jfa::launch_bwd_pre(p, o, d_o, lse, rowstat, dq_acc, acc_elems, plan, s);
  });
  if (e != hipSuccess) return hip_fail(e, fn, "delta launch");
  if (p.total_kv > 0) {
    e = timed_launch("bwd", s, [&] {
      return jfa::launch_bwd(p, plan, sched, rowstat, lse, d_o, dq_acc, dq, dk, dv, rope, s);
    });
    if (e != hipSuccess) return hip_fail(e, fn, "kernel launch");
  }
  e = timed_launch("dq_finalize", s,
                   [&] { return jfa::launch_dq_finalize(p, dq_acc, dq, plan, rope, s); });
  if (e != hipSuccess) return hip_fail(e, fn, "dq finalize launch");
  return JFA_OK;
}

}  // namespace

jfa_status_t jfa_bwd(const void* q, const void* k, const void* v, const void* offsets,
                     int offsets_is_int64, int64_t batch, int64_t num_heads, int64_t head_dim,
                     int64_t q_len, int64_t total_kv, int broadcast_q, int causal, float softmax_scale,
                     const void* o, const float* lse, const void* d_o, void* dq, void* dk, void* dv,
                     void* workspace, size_t workspace_bytes, void* stream) {
  return bwd_impl("jfa_bwd", q, k, v, offsets, offsets_is_int64, batch, num_heads, head_dim, q_len,
                  total_kv, broadcast_q, causal, softmax_scale, o, lse, d_o, dq, dk, dv, jfa::Rope{},
                  workspace, workspace_bytes, stream);
}

jfa_status_t jfa_bwd_rope(const void* q, const void* k, const void* v, const void* offsets,
                          int offsets_is_int64, int64_t batch, int64_t num_heads, int64_t head_dim,
                          int64_t q_len, int64_t total_kv, int broadcast_q, int causal,
                          float softmax_scale, const void* o, const float* lse, const void* d_o,
                          const float* rope_cos, const float* rope_sin, const int32_t* pos_q,
                          const int32_t* pos_k, int64_t max_pos, void* dq, void* dk, void* dv,
                          void* workspace, size_t workspace_bytes, void* stream) {
  g_error[0] = '\0';
  if (!rope_cos || !rope_sin || !pos_q || (total_kv > 0 && !pos_k))
    return fail(JFA_ERR_INVALID_ARGUMENT, "jfa_bwd_rope: null rotary table or position pointer");
  if (max_pos < 1 || max_pos > (int64_t)1 << 24)
    return fail(JFA_ERR_INVALID_ARGUMENT, "jfa_bwd_rope: max_pos must be in [1, 2^24]");
  if (misaligned(rope_cos) || misaligned(rope_sin) || (reinterpret_cast<uintptr_t>(pos_q) & 3) ||
      (reinterpret_cast<uintptr_t>(pos_k) & 3))
    return fail(JFA_ERR_INVALID_ARGUMENT,
                "jfa_bwd_rope: rotary tables must be 16-byte aligned, positions 4-byte aligned");
  jfa::Rope rope;
  rope.cos = rope_cos;
  rope.sin = rope_sin;
  rope.pos_q = pos_q;
  rope.pos_k = pos_k;
  rope.max_pos = (int)max_pos;
  return bwd_impl("jfa_bwd_rope", q, k, v, offsets, offsets_is_int64, batch, num_heads, head_dim, q_len,
                  total_kv, broadcast_q, causal, softmax_scale, o, lse, d_o, dq, dk, dv, rope, workspace,
                  workspace_bytes, stream);
}

size_t jfa_fwd_sparse_workspace_size(int64_t batch, int64_t num_heads, int64_t head_dim, int64_t q_len,
                                     int64_t total_kv, int broadcast_q, int topk) {
  if (!check_sizes(batch, num_heads, head_dim, q_len, total_kv, broadcast_q, 0).ok) return 0;
  if (topk < 1 || topk > jfa::kSparseMaxTopk) return 0;
  jfa::Problem p = make_problem(nullptr, nullptr, nullptr, nullptr, 0, batch, num_heads, head_dim, q_len,
                                total_kv, broadcast_q, 0, 1.f);
  p.topk = topk;
  return fwd_sparse_ws_bytes(p);
}

int64_t jfa_fwd_sparse_query_blocks(int64_t batch, int64_t q_len, int64_t total_kv, int broadcast_q) {
  jfa::Problem p = make_problem(nullptr, nullptr, nullptr, nullptr, 0, batch, 1, 128, q_len, total_kv,
                                broadcast_q, 0, 1.f);
  return sparse_out_qblocks(p);
}

jfa_status_t jfa_fwd_sparse(const void* q, const void* k, const void* v, const void* offsets,
                            int offsets_is_int64, int64_t batch, int64_t num_heads, int64_t head_dim,
                            int64_t q_len, int64_t total_kv, int broadcast_q, float softmax_scale, int topk,
                            void* o, float* lse, int32_t* blocks, void* workspace, size_t workspace_bytes,
                            void* stream) {
  g_error[0] = '\0';
  const Sizes sz = check_sizes(batch, num_heads, head_dim, q_len, total_kv, broadcast_q, 0);
  if (!sz.ok) return fail(sz.st, "jfa_fwd_sparse: %s", sz.why);
  if (topk < 1 || topk > jfa::kSparseMaxTopk)
    return fail(JFA_ERR_INVALID_ARGUMENT, "jfa_fwd_sparse: topk must be in [1, %d]", jfa::kSparseMaxTopk);
  if (!std::isfinite(softmax_scale) || softmax_scale <= 0.f)
    return fail(JFA_ERR_INVALID_ARGUMENT, "jfa_fwd_sparse: softmax_scale must be finite and > 0");
  jfa::Problem p = make_problem(q, k, v, offsets, offsets_is_int64, batch, num_heads, head_dim, q_len,
                                total_kv, broadcast_q, 0, softmax_scale);
  p.topk = topk;
  if (p.batch == 0 || p.rows == 0) return JFA_OK;
  if (!q || !offsets || !o || !lse || !workspace || (p.total_kv > 0 && (!k || !v)))
    return fail(JFA_ERR_INVALID_ARGUMENT, "jfa_fwd_sparse: null pointer argument");
  if (misaligned(q) || misaligned(k) || misaligned(v) || misaligned(o) || misaligned(workspace) ||
      (reinterpret_cast<uintptr_t>(lse) & 3) || (reinterpret_cast<uintptr_t>(blocks) & 3) ||
      (reinterpret_cast<uintptr_t>(offsets) & (offsets_is_int64 ? 7 : 3)))
    return fail(JFA_ERR_INVALID_ARGUMENT, "jfa_fwd_sparse: tensors must be 16-byte aligned");
  const size_t need = fwd_sparse_ws_bytes(p);
  if (workspace_bytes < need)
    return fail(JFA_ERR_WORKSPACE_TOO_SMALL, "jfa_fwd_sparse: workspace of %zu bytes, need %zu",
                workspace_bytes, need);
  char* cur = reinterpret_cast<char*>(align_up(reinterpret_cast<uintptr_t>(workspace)));
  jfa::Plan plan;
  plan.meta = reinterpret_cast<int*>(carve(cur, 64));
  plan.max_items = jfa::fwd_max_items(p);
  plan.items = reinterpret_cast<int4*>(carve(cur, plan.max_items * sizeof(int4)));
  jfa::Sparse sp;
  sp.kv_first = reinterpret_cast<int*>(carve(cur, (size_t)(p.batch + 1) * sizeof(int)));
  sp.q_first = reinterpret_cast<int*>(carve(cur, (size_t)(p.batch + 1) * sizeof(int)));
  sp.kv_blocks_cap = sparse_kv_cap(p);
  sp.q_blocks_cap = sparse_q_cap(p);
  sp.pooled_k = reinterpret_cast<float*>(carve(cur, (size_t)p.heads * sp.kv_blocks_cap * p.head_dim * sizeof(float)));
  sp.pooled_q = reinterpret_cast<float*>(carve(cur, (size_t)p.heads * sp.q_blocks_cap * p.head_dim * sizeof(float)));
  sp.tile_blocks = reinterpret_cast<int*>(carve(cur, (size_t)sparse_tiles(p) * p.topk * sizeof(int)));
  sp.out_blocks = blocks;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const int sched = g_schedule.load();
  hipError_t e = timed_launch("plan_sparse", s, [&] { return jfa::launch_plan_sparse(p, sp.kv_first, sp.q_first, s); });
  if (e != hipSuccess) return hip_fail(e, "jfa_fwd_sparse: plan launch");
  e = timed_launch("plan_fwd", s, [&] { return jfa::launch_plan_fwd(p, plan, sched, s); });
  if (e != hipSuccess) return hip_fail(e, "jfa_fwd_sparse: plan launch");
  e = timed_launch("sparse_select", s, [&] { return jfa::launch_sparse_select(p, plan, sp, s); });
  if (e != hipSuccess) return hip_fail(e, "jfa_fwd_sparse: selection launch");
  e = timed_launch("fwd_sparse", s, [&] { return jfa::launch_fwd_sparse(p, plan, sched, sp, o, lse, s); });
  if (e != hipSuccess) return hip_fail(e, "jfa_fwd_sparse: kernel launch");
  return JFA_OK;
}

int64_t jfa_mxfp8_v_blocks(int64_t batch, int64_t total_kv) {
  if (batch < 0 || total_kv < 0) return 0;
  return jfa::mx_v_blocks(batch, total_kv);
}

jfa_status_t jfa_mxfp8_quantize_rows(const void* x, int64_t rows, int64_t num_heads, int64_t head_dim,
                                     void* values, void* scales, void* stream) {
  g_error[0] = '\0';
  if (rows < 0 || num_heads < 1 || num_heads >= 4096)
    return fail(JFA_ERR_INVALID_ARGUMENT, "jfa_mxfp8_quantize_rows: rows must be >= 0, num_heads in [1, 4095]");
  if (head_dim != 64 && head_dim != 128)
    return fail(JFA_ERR_UNSUPPORTED, "jfa_mxfp8_quantize_rows: head_dim must be 64 or 128");
  if (rows >= ((int64_t)1 << 31) / num_heads)
    return fail(JFA_ERR_UNSUPPORTED, "jfa_mxfp8_quantize_rows: too many rows for this library build");
  if (rows == 0) return JFA_OK;
  if (!x || !values || !scales) return fail(JFA_ERR_INVALID_ARGUMENT, "jfa_mxfp8_quantize_rows: null pointer argument");
  if (misaligned(x) || misaligned(values))
    return fail(JFA_ERR_INVALID_ARGUMENT, "jfa_mxfp8_quantize_rows: x and values must be 16-byte aligned");
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const hipError_t e = timed_launch("mx_quantize_rows", s, [&] {
    return jfa::launch_mx_quantize_rows(x, rows, (int)num_heads, (int)head_dim, values, scales, s);
  });
  if (e != hipSuccess) return hip_fail(e, "jfa_mxfp8_quantize_rows: kernel launch");
  return JFA_OK;
}

jfa_status_t jfa_mxfp8_quantize_v(const void* v, const void* offsets, int offsets_is_int64, int64_t batch,
                                  int64_t num_heads, int64_t head_dim, int64_t total_kv, void* values,
                                  void* scales, void* stream) {
  g_error[0] = '\0';
  const Sizes sz = check_sizes(batch, num_heads, head_dim, 0, total_kv, 0, 0);
  if (!sz.ok) return fail(sz.st, "jfa_mxfp8_quantize_v: %s", sz.why);
  if (batch == 0) return JFA_OK;
  if (!offsets || !values || !scales || (total_kv > 0 && !v))
    return fail(JFA_ERR_INVALID_ARGUMENT, "jfa_mxfp8_quantize_v: null pointer argument");
  if (misaligned(v) || misaligned(values) || (reinterpret_cast<uintptr_t>(offsets) & (offsets_is_int64 ? 7 : 3)))
    return fail(JFA_ERR_INVALID_ARGUMENT, "jfa_mxfp8_quantize_v: v and values must be 16-byte aligned");
  const jfa::Problem p = make_problem(nullptr, nullptr, v, offsets, offsets_is_int64, batch, num_heads, head_dim,
                                      0, total_kv, 0, 0, 1.f);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const hipError_t e = timed_launch("mx_quantize_v", s, [&] { return jfa::launch_mx_quantize_v(p, v, values, scales, s); });
  if (e != hipSuccess) return hip_fail(e, "jfa_mxfp8_quantize_v: kernel launch");
  return JFA_OK;
}

jfa_status_t jfa_fwd_mxfp8(const void* q8, const void* q_scales, const void* k8, const void* k_scales,
                           const void* v8, const void* v_scales, const void* offsets, int offsets_is_int64,
                           int64_t batch, int64_t num_heads, int64_t head_dim, int64_t q_len, int64_t total_kv,
                           int broadcast_q, int causal, float softmax_scale, void* o, float* lse,
                           void* workspace, size_t workspace_bytes, void* stream) {
  g_error[0] = '\0';
  const Sizes sz = check_sizes(batch, num_heads, head_dim, q_len, total_kv, broadcast_q, causal);
  if (!sz.ok) return fail(sz.st, "jfa_fwd_mxfp8: %s", sz.why);
  if (!std::isfinite(softmax_scale) || softmax_scale <= 0.f)
    return fail(JFA_ERR_INVALID_ARGUMENT, "jfa_fwd_mxfp8: softmax_scale must be finite and > 0");
  jfa::Problem p = make_problem(q8, k8, v8, offsets, offsets_is_int64, batch, num_heads, head_dim, q_len,
                                total_kv, broadcast_q, causal, softmax_scale);
  p.mx = 1;
  if (p.batch == 0 || p.rows == 0) return JFA_OK;
  if (!q8 || !q_scales || !offsets || !o || !lse || !workspace ||
      (p.total_kv > 0 && (!k8 || !k_scales || !v8 || !v_scales)))
    return fail(JFA_ERR_INVALID_ARGUMENT, "jfa_fwd_mxfp8: null pointer argument");
  if (misaligned(q8) || misaligned(k8) || misaligned(v8) || misaligned(v_scales) || misaligned(o) ||
      misaligned(workspace) || (reinterpret_cast<uintptr_t>(lse) & 3) ||
      (reinterpret_cast<uintptr_t>(k_scales) & (head_dim / 32 - 1)) ||
      (reinterpret_cast<uintptr_t>(offsets) & (offsets_is_int64 ? 7 : 3)))
    return fail(JFA_ERR_INVALID_ARGUMENT, "jfa_fwd_mxfp8: tensors must be 16-byte aligned");
  const size_t need = fwd_ws_bytes(p);
  if (workspace_bytes < need)
    return fail(JFA_ERR_WORKSPACE_TOO_SMALL, "jfa_fwd_mxfp8: workspace of %zu bytes, need %zu",
                workspace_bytes, need);
  char* cur = reinterpret_cast<char*>(align_up(reinterpret_cast<uintptr_t>(workspace)));
  jfa::Plan plan;
  plan.meta = reinterpret_cast<int*>(carve(cur, 64));
  plan.max_items = jfa::fwd_max_items(p);
  plan.items = reinterpret_cast<int4*>(carve(cur, plan.max_items * sizeof(int4)));
  const jfa::MxOperands x{q8, q_scales, k8, k_scales, v8, v_scales};
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  hipError_t e = timed_launch("plan_fwd", s, [&] { return jfa::launch_plan_fwd(p, plan, JFA_SCHED_SORTED_ZIGZAG, s); });
  if (e != hipSuccess) return hip_fail(e, "jfa_fwd_mxfp8: plan launch");
  e = timed_launch("fwd_mxfp8", s, [&] { return jfa::launch_fwd_mx(p, plan, x, o, lse, s); });
  if (e != hipSuccess) return hip_fail(e, "jfa_fwd_mxfp8: kernel launch");
  return JFA_OK;
}

jfa_status_t jfa_profile_enable(int enable) {
  g_prof = enable != 0;
  return JFA_OK;
}

jfa_status_t jfa_profile_read(char* names, int name_len, double* total_ms, int64_t* launches,
                              int max_entries, int* count) {
  std::vector<std::string> keys;
  std::vector<double> ms;
  std::vector<int64_t> cnt;
  jfa_status_t st = JFA_OK;
  for (const ProfRecord& r : g_prof_records) {
    float t = 0.f;
    hipError_t e = hipEventSynchronize(r.stop);
    if (e == hipSuccess) e = hipEventElapsedTime(&t, r.start, r.stop);
    if (e != hipSuccess && st == JFA_OK) st = hip_fail(e, "jfa_profile_read");
    size_t i = 0;
    while (i < keys.size() && keys[i] != r.name) ++i;
    if (i == keys.size()) {
      keys.emplace_back(r.name);
      ms.push_back(0.0);
      cnt.push_back(0);
    }
    ms[i] += t;
    cnt[i] += 1;
    g_prof_pool.push_back(r.start);
    g_prof_pool.push_back(r.stop);
  }
  g_prof_records.clear();
  if (count) *count = (int)keys.size();
  for (int i = 0; i < (int)keys.size() && i < max_entries; ++i) {
    if (names && name_len > 0) {
      snprintf(names + (size_t)i * name_len, (size_t)name_len, "%s", keys[i].c_str());
    }
    if (total_ms) total_ms[i] = ms[i];
    if (launches) launches[i] = cnt[i];
  }
  return st;
}

const char* jfa_last_error(void) { return g_error; }

const char* jfa_version(void) { return "jfa 0.1 gfx950"; }

}  // extern "C"
