// C ABI of the MoE layer library: host-side argument checks, workspace sizing and dispatch to
// the gfx950 kernels.  Nothing is enqueued when a check fails; no call allocates or keeps state.
#include <stdint.h>
#include <string.h>

#include <mutex>

#include "moe_launch.h"
#include "moe_lora.h"

using namespace moe;

namespace {

constexpr size_t ALIGN = 256;
constexpr int GROUPED_MIN_T = 32;  // token count from which the grouped MFMA path runs

size_t align_up(size_t v) { return (v + ALIGN - 1) / ALIGN * ALIGN; }
bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
bool known_flags(uint32_t f) { return (f & ~(MOE_TOPK_RENORM | MOE_INPUT_RMSNORM)) == 0; }
moe_status from_hip(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

bool routing_dims_ok(int32_t T, int32_t E, int32_t K) {
  return T >= 1 && E >= 1 && E <= MOE_MAX_E && K >= 1 && K <= MOE_MAX_K && K <= E;
}

// workspace layout of moe_expert_ffn_q4
struct FfnWs {
  size_t act, u_gate, u_up, u_down, grouped, total;
};
// TS: pairs of a shared expert run with the routed ones (T, or 0); its expert-sorted activations
// [T*K + T][I] float16 fit the T*K*I float32 of the decode path's act for any K >= 1.
FfnWs ffn_ws(int32_t T, int32_t K, const moe_experts* ex, int32_t TS = 0) {
  FfnWs w{};
  w.act = 0;
  w.u_gate = w.act + align_up((size_t)T * K * ex->d_ff * sizeof(float));
  w.u_up = w.u_gate + align_up((size_t)T * LORA_MAX_RANK * sizeof(float));
  w.u_down = w.u_up + align_up((size_t)T * LORA_MAX_RANK * sizeof(float));
  // the grouped path's down adapter keeps grouped_lora_parts(I) partial products per token
  const size_t parts = T >= GROUPED_MIN_T ? (size_t)grouped_lora_parts(ex->d_ff) : 1;
  w.grouped = w.u_down + align_up((size_t)T * LORA_MAX_RANK * parts * sizeof(float));
  w.total = w.grouped + (T >= GROUPED_MIN_T ? grouped_layout(T, K, ex->n_experts, ex->d_model, TS).total : 0);
  return w;
}

// workspace layout of moe_expert_ffn_sparse
struct SparseWs {
  size_t act, o, cnt, total;
};
SparseWs sparse_ws(int32_t T, int32_t K, const moe_experts* ex) {
  SparseWs w{};
  const int ns = sparse_slabs(ex->bits, ex->d_model);
  w.act = 0;
  w.o = w.act + align_up((size_t)T * K * ex->d_ff * sizeof(float));
  w.cnt = w.o + align_up((size_t)T * K * ex->d_model * sizeof(float));
  w.total = w.cnt + align_up((size_t)T * (ns > 0 ? ns : 1) * sizeof(int32_t));
  return w;
}

moe_status check_qmat(const moe_qmat& m) {
  if (!m.q || !m.scales || !m.biases) return MOE_ERR_INVALID_ARG;
  if (!aligned16(m.q)) return MOE_ERR_INVALID_ARG;
  if (((uintptr_t)m.scales & 1u) || ((uintptr_t)m.biases & 1u)) return MOE_ERR_INVALID_ARG;
  return MOE_OK;
}

moe_status check_experts(const moe_experts* ex) {
  if (!ex) return MOE_ERR_INVALID_ARG;
  if (ex->n_experts < 1 || ex->n_experts > MOE_MAX_E) return MOE_ERR_INVALID_ARG;
  if (ex->bits != 4 && ex->bits != 2) return MOE_ERR_UNSUPPORTED;
  if (ex->group != 32 && ex->group != 64 && ex->group != 128) return MOE_ERR_UNSUPPORTED;
  const int d = ex->d_model, I = ex->d_ff;
  if (d < 1 || I < 1 || d > MOE_MAX_D || I > MOE_MAX_D) return MOE_ERR_INVALID_ARG;
  if (d % ex->group || I % ex->group) return MOE_ERR_INVALID_ARG;
  if ((d * ex->bits) % 128 || (I * ex->bits) % 128) return MOE_ERR_INVALID_ARG;
  if (!decode_shape_supported(ex->bits, ex->group, d, I)) return MOE_ERR_UNSUPPORTED;
  moe_status s;
  if ((s = check_qmat(ex->gate)) != MOE_OK) return s;
  if ((s = check_qmat(ex->up)) != MOE_OK) return s;
  if ((s = check_qmat(ex->down)) != MOE_OK) return s;
  return MOE_OK;
}

// Scratch of moe_expert_ffn_q4_noalloc: a file-scope device array, one copy on every GPU the library
// runs on, held until the process ends.  In host code its name is only a host-side stand-in: the
// device address of each GPU's copy is looked up once per device (with that device current) and
// kept; kernels only ever receive that address.
static __device__ __align__(256) unsigned char scratch[MOE_NOALLOC_SCRATCH_BYTES];

constexpr int NOALLOC_MAX_DEVICES = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[NOALLOC_MAX_DEVICES];  // device address of `scratch` per device, once looked up

moe_status scratch_on_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= NOALLOC_MAX_DEVICES) return MOE_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return MOE_ERR_HIP;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return MOE_OK;
}

}  // namespace

extern "C" {

const char* moe_status_string(moe_status s) {
  switch (s) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID_ARG: return "MOE_ERR_INVALID_ARG: invalid argument";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED: unsupported bits, group or shape";
    case MOE_ERR_HIP: return "MOE_ERR_HIP: the HIP runtime rejected a launch";
    case MOE_ERR_TOO_LARGE:
      return "MOE_ERR_TOO_LARGE: the call needs more scratch than the allocation-free entry point holds";
  }
  return "unknown moe_status";
}

int32_t moe_version(void) { return 100; }

moe_status moe_route_topk(void* stream, int32_t T, int32_t d, int32_t E, int32_t K, uint32_t flags,
                          const uint16_t* x, const uint16_t* w_router, float* logits, int32_t* idx, float* w) {
  if (!routing_dims_ok(T, E, K) || !known_flags(flags)) return MOE_ERR_INVALID_ARG;
  if (!logits || !idx || !w) return MOE_ERR_INVALID_ARG;
  hipStream_t s = (hipStream_t)stream;
  if (w_router) {
    if (!x || d < 8 || d % 8 || d > MOE_MAX_D) return MOE_ERR_INVALID_ARG;
    if (!aligned16(x) || !aligned16(w_router)) return MOE_ERR_INVALID_ARG;
    if (launch_router_gemv(s, T, d, E, flags, x, w_router, logits) != hipSuccess) return MOE_ERR_HIP;
  }
  return from_hip(launch_topk(s, T, E, K, flags, logits, idx, w));
}

size_t moe_prerouter_workspace_size(int32_t T, int32_t E, int32_t d_hidden) {
  if (T < 1 || E < 1 || d_hidden < 1) return 0;
  return align_up((size_t)T * d_hidden * sizeof(float)) + align_up((size_t)T * E * sizeof(float));
}

moe_status moe_prerouter(void* stream, int32_t T, int32_t d, int32_t E, int32_t K, uint32_t flags,
                         const uint16_t* x, const int32_t* idx_cur, const int32_t* idx_prev,
                         const moe_prerouter_w* pw, float* logits, void* workspace, size_t workspace_bytes) {
  if (!routing_dims_ok(T, E, K) || !known_flags(flags)) return MOE_ERR_INVALID_ARG;
  if (!x || !idx_cur || !pw || !logits || !workspace) return MOE_ERR_INVALID_ARG;
  if (d < 8 || d % 8 || d > MOE_MAX_D) return MOE_ERR_INVALID_ARG;
  const int H = pw->d_hidden;
  if (H < 8 || H % 8 || H > MOE_MAX_D) return MOE_ERR_INVALID_ARG;
  if (!pw->fc1_x || !pw->fc1_r || !pw->fc2 || !pw->lin_x || !pw->lin_r) return MOE_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(pw->fc1_x) || !aligned16(pw->fc2) || !aligned16(pw->lin_x) ||
      !aligned16(workspace))
    return MOE_ERR_INVALID_ARG;
  if (workspace_bytes < moe_prerouter_workspace_size(T, E, H)) return MOE_ERR_INVALID_ARG;
  float* g = (float*)workspace;
  float* lin = (float*)((char*)workspace + align_up((size_t)T * H * sizeof(float)));
  return from_hip(launch_prerouter((hipStream_t)stream, T, d, E, K, flags, x, idx_cur, idx_prev, *pw, logits, g, lin));
}

size_t moe_expert_ffn_workspace_size(int32_t T, int32_t K, const moe_experts* ex) {
  if (!ex || T < 1 || K < 1 || ex->d_ff < 1 || ex->d_model < 1) return 0;
  return ffn_ws(T, K, ex).total;
}

// Argument checks of moe_expert_ffn_q4 other than the workspace.
static moe_status check_expert_ffn(int32_t T, int32_t K, uint32_t flags, const uint16_t* x, const int32_t* idx,
                                   const moe_experts* ex, const moe_lora* lora3, float* out, const float* w_fuse,
                                   const uint16_t* r_fuse, uint16_t* y_fuse) {
  moe_status st = check_experts(ex);
  if (st != MOE_OK) return st;
  if (!routing_dims_ok(T, ex->n_experts, K) || !known_flags(flags)) return MOE_ERR_INVALID_ARG;
  if (!x || !idx || !aligned16(x)) return MOE_ERR_INVALID_ARG;
  const bool fuse = w_fuse || r_fuse || y_fuse;
  if (fuse && !(w_fuse && r_fuse && y_fuse)) return MOE_ERR_INVALID_ARG;
  if (!out && !fuse) return MOE_ERR_INVALID_ARG;
  if (lora3) {
    if (ex->n_experts != 1) return MOE_ERR_INVALID_ARG;
    for (int m = 0; m < 3; ++m) {
      if (!lora3[m].A || !lora3[m].B || lora3[m].rank < 1 || lora3[m].rank > LORA_MAX_RANK) return MOE_ERR_INVALID_ARG;
      if (!aligned16(lora3[m].A)) return MOE_ERR_INVALID_ARG;
    }
  }
  return MOE_OK;
}

// Enqueue the expert FFN on checked arguments with `workspace` (ffn_ws(T, K, ex).total bytes).
static moe_status run_expert_ffn(void* stream, int32_t T, int32_t K, uint32_t flags, const uint16_t* x,
                                 const int32_t* idx, const moe_experts* ex, const moe_lora* lora3, float* out,
                                 const float* w_fuse, const uint16_t* r_fuse, uint16_t* y_fuse, void* workspace,
                                 const moe_experts* shared = nullptr) {
  const int32_t TS = shared ? T : 0;
  const FfnWs ws = ffn_ws(T, K, ex, TS);
  char* base = (char*)workspace;
  DecodeArgs a{};
  a.T = T;
  a.K = K;
  a.E = ex->n_experts;
  a.d = ex->d_model;
  a.I = ex->d_ff;
  a.bits = ex->bits;
  a.group = ex->group;
  a.flags = flags;
  a.x = x;
  a.idx = idx;
  a.ex = *ex;
  a.lora3 = lora3;
  a.out = out;
  a.w_fuse = w_fuse;
  a.r_fuse = r_fuse;
  a.y_fuse = y_fuse;
  a.act = base + ws.act;
  a.u_gate = (float*)(base + ws.u_gate);
  a.u_up = (float*)(base + ws.u_up);
  a.u_down = (float*)(base + ws.u_down);
  a.shared = shared;
  hipStream_t s = (hipStream_t)stream;
  if (T >= GROUPED_MIN_T) {
    GroupedArgs g{};
    g.base = a;
    char* gb = base + ws.grouped;
    const GroupedLayout gl = grouped_layout(T, K, ex->n_experts, ex->d_model, TS);
    g.counts = (int32_t*)(gb + gl.counts);
    g.tiles = (int32_t*)(gb + gl.tiles);
    g.offsets = (int32_t*)(gb + gl.offsets);
    g.perm = (int32_t*)(gb + gl.perm);
    g.rowscale = (float*)(gb + gl.rowscale);
    g.o_sorted = (float*)(gb + gl.o_sorted);
    return from_hip(launch_expert_grouped(s, g));
  }
  return from_hip(launch_expert_decode(s, a));
}

moe_status moe_expert_ffn_q4(void* stream, int32_t T, int32_t K, uint32_t flags, const uint16_t* x,
                             const int32_t* idx, const moe_experts* ex, const moe_lora* lora3, float* out,
                             const float* w_fuse, const uint16_t* r_fuse, uint16_t* y_fuse, void* workspace,
                             size_t workspace_bytes) {
  const moe_status st = check_expert_ffn(T, K, flags, x, idx, ex, lora3, out, w_fuse, r_fuse, y_fuse);
  if (st != MOE_OK) return st;
  if (!workspace || !aligned16(workspace) || workspace_bytes < ffn_ws(T, K, ex).total) return MOE_ERR_INVALID_ARG;
  return run_expert_ffn(stream, T, K, flags, x, idx, ex, lora3, out, w_fuse, r_fuse, y_fuse, workspace);
}

moe_status moe_expert_ffn_q4_noalloc(void* stream, int32_t T, int32_t K, uint32_t flags, const uint16_t* x,
                                     const int32_t* idx, const moe_experts* ex, const moe_lora* lora3, float* out,
                                     const float* w_fuse, const uint16_t* r_fuse, uint16_t* y_fuse) {
  const moe_status st = check_expert_ffn(T, K, flags, x, idx, ex, lora3, out, w_fuse, r_fuse, y_fuse);
  if (st != MOE_OK) return st;
  if (ffn_ws(T, K, ex).total > MOE_NOALLOC_SCRATCH_BYTES) return MOE_ERR_TOO_LARGE;
  void* ptr = nullptr;
  const moe_status sp = scratch_on_current_device(&ptr);
  if (sp != MOE_OK) return sp;
  return run_expert_ffn(stream, T, K, flags, x, idx, ex, lora3, out, w_fuse, r_fuse, y_fuse, ptr);
}

size_t moe_expert_ffn_shared_workspace_size(int32_t T, int32_t K, const moe_experts* ex) {
  if (!ex || T < GROUPED_MIN_T || K < 1 || ex->d_ff < 1 || ex->d_model < 1) return 0;
  return ffn_ws(T, K, ex, T).total;
}

moe_status moe_expert_ffn_q4_shared(void* stream, int32_t T, int32_t K, uint32_t flags, const uint16_t* x,
                                    const int32_t* idx, const moe_experts* ex, const moe_experts* shared,
                                    const moe_lora* lora3, const float* w, const uint16_t* r, uint16_t* y,
                                    void* workspace, size_t workspace_bytes) {
  // the routed experts' checks (the LoRA is the shared expert's, checked against it below)
  moe_status st = check_expert_ffn(T, K, flags, x, idx, ex, nullptr, nullptr, w, r, y);
  if (st != MOE_OK) return st;
  if (!w || !r || !y) return MOE_ERR_INVALID_ARG;
  if (!shared) return MOE_ERR_INVALID_ARG;
  st = check_expert_ffn(T, 1, flags, x, idx, shared, lora3, nullptr, w, r, y);
  if (st != MOE_OK) return st;
  if (shared->n_experts != 1 || shared->d_model != ex->d_model || shared->d_ff != ex->d_ff ||
      shared->bits != ex->bits || shared->group != ex->group)
    return MOE_ERR_INVALID_ARG;
  if (T < GROUPED_MIN_T) return MOE_ERR_UNSUPPORTED;
  if (!workspace || !aligned16(workspace) || workspace_bytes < ffn_ws(T, K, ex, T).total) return MOE_ERR_INVALID_ARG;
  return run_expert_ffn(stream, T, K, flags, x, idx, ex, lora3, nullptr, w, r, y, workspace, shared);
}

size_t moe_expert_ffn_sparse_workspace_size(int32_t T, int32_t K, const moe_experts* ex) {
  if (!ex || T < 1 || K < 1 || ex->d_ff < 1 || ex->d_model < 1) return 0;
  return sparse_ws(T, K, ex).total;
}

moe_status moe_expert_ffn_sparse(void* stream, int32_t T, int32_t K, uint32_t flags, const uint16_t* x,
                                 const int32_t* idx, const moe_experts* ex, float* out, const float* w_fuse,
                                 const uint16_t* r_fuse, uint16_t* y_fuse, int32_t* n_active, void* workspace,
                                 size_t workspace_bytes) {
  moe_status st = check_experts(ex);
  if (st != MOE_OK) return st;
  if (!routing_dims_ok(T, ex->n_experts, K) || (flags & ~MOE_INPUT_RMSNORM)) return MOE_ERR_INVALID_ARG;
  if (!x || !idx || !workspace || !aligned16(x) || !aligned16(workspace)) return MOE_ERR_INVALID_ARG;
  const bool fuse = w_fuse || r_fuse || y_fuse;
  if (fuse && !(w_fuse && r_fuse && y_fuse)) return MOE_ERR_INVALID_ARG;
  if (!out && !fuse) return MOE_ERR_INVALID_ARG;
  const int nslab = sparse_slabs(ex->bits, ex->d_model);
  if (nslab < 1 || ex->d_ff > 4096 || sparse_lds(ex->bits, ex->d_ff) > 65536) return MOE_ERR_UNSUPPORTED;
  const SparseWs ws = sparse_ws(T, K, ex);
  if (workspace_bytes < ws.total) return MOE_ERR_INVALID_ARG;
  char* base = (char*)workspace;
  SparseArgs sp{};
  DecodeArgs& a = sp.base;
  a.T = T;
  a.K = K;
  a.E = ex->n_experts;
  a.d = ex->d_model;
  a.I = ex->d_ff;
  a.bits = ex->bits;
  a.group = ex->group;
  a.flags = flags;
  a.x = x;
  a.idx = idx;
  a.ex = *ex;
  a.out = out;
  a.w_fuse = w_fuse;
  a.r_fuse = r_fuse;
  a.y_fuse = y_fuse;
  a.act = base + ws.act;
  a.relu = true;
  sp.o = out ? out : (float*)(base + ws.o);
  sp.cnt = (int32_t*)(base + ws.cnt);
  sp.n_active = n_active;
  a.zero = sp.cnt;
  a.nzero = nslab;
  hipStream_t s = (hipStream_t)stream;
  hipError_t err = launch_gateup_decode(s, a);
  if (err == hipSuccess) err = launch_down_sparse(s, sp);
  return from_hip(err);
}

size_t moe_stream_workspace_size(int32_t K) {
  if (K < 1 || K > MOE_MAX_K) return 0;
  return align_up(pool_plan_bytes(K));
}

static moe_status check_stream_job(int32_t K, const moe_stream_job& j, const moe_experts* shape) {
  const moe_experts* src = j.src;
  const moe_experts* pool_experts = j.pool_experts;
  const moe_pool* pool = j.pool;
  if (!src || !pool_experts || !pool || !j.idx || !j.idx_slot) return MOE_ERR_INVALID_ARG;
  if (!pool->slot_expert || !pool->slot_stamp || !pool->clock) return MOE_ERR_INVALID_ARG;
  if (pool->n_slots < K || pool->n_slots > MOE_POOL_MAX_SLOTS || pool_experts->n_experts != pool->n_slots)
    return MOE_ERR_INVALID_ARG;
  if (src->n_experts < 1 || src->n_experts > (1 << 20)) return MOE_ERR_INVALID_ARG;
  if (src->d_model != pool_experts->d_model || src->d_ff != pool_experts->d_ff || src->bits != pool_experts->bits ||
      src->group != pool_experts->group)
    return MOE_ERR_INVALID_ARG;
  if (src->d_model != shape->d_model || src->d_ff != shape->d_ff || src->bits != shape->bits ||
      src->group != shape->group)
    return MOE_ERR_INVALID_ARG;
  if (src->bits != 4 && src->bits != 2) return MOE_ERR_UNSUPPORTED;
  if (src->group != 32 && src->group != 64 && src->group != 128) return MOE_ERR_UNSUPPORTED;
  const int d = src->d_model, I = src->d_ff;
  if (d < 1 || I < 1 || d > MOE_MAX_D || I > MOE_MAX_D || d % src->group || I % src->group) return MOE_ERR_INVALID_ARG;
  if ((d * src->bits) % 128 || (I * src->bits) % 128) return MOE_ERR_INVALID_ARG;
  for (const moe_qmat* m : {&src->gate, &src->up, &src->down, &pool_experts->gate, &pool_experts->up, &pool_experts->down}) {
    moe_status st = check_qmat(*m);
    if (st != MOE_OK) return st;
  }
  return MOE_OK;
}

moe_status moe_stream_in_many(void* stream, int32_t n, int32_t K, const moe_stream_job* jobs, void* workspace,
                              size_t workspace_bytes) {
  if (n < 1 || n > MOE_POOL_MAX_JOBS || !jobs || !workspace) return MOE_ERR_INVALID_ARG;
  if (K < 1 || K > MOE_MAX_K) return MOE_ERR_INVALID_ARG;
  if (!jobs[0].src) return MOE_ERR_INVALID_ARG;
  const size_t per = moe_stream_workspace_size(K);
  if (!aligned16(workspace) || workspace_bytes < per * (size_t)n) return MOE_ERR_INVALID_ARG;
  PoolArgs a[MOE_POOL_MAX_JOBS];
  const moe_experts* src[MOE_POOL_MAX_JOBS];
  const moe_experts* pex[MOE_POOL_MAX_JOBS];
  for (int j = 0; j < n; ++j) {
    moe_status st = check_stream_job(K, jobs[j], jobs[0].src);
    if (st != MOE_OK) return st;
    for (int i = 0; i < j; ++i)
      if (jobs[i].pool->slot_expert == jobs[j].pool->slot_expert) return MOE_ERR_INVALID_ARG;  // one pool twice
    a[j] = PoolArgs{};
    a[j].K = K;
    a[j].E = jobs[j].src->n_experts;
    a[j].n_slots = jobs[j].pool->n_slots;
    a[j].idx = jobs[j].idx;
    a[j].slot_expert = jobs[j].pool->slot_expert;
    a[j].slot_stamp = jobs[j].pool->slot_stamp;
    a[j].clock = jobs[j].pool->clock;
    a[j].idx_slot = jobs[j].idx_slot;
    a[j].counters = jobs[j].counters;
    a[j].plan = (int32_t*)((char*)workspace + per * j);
    src[j] = jobs[j].src;
    pex[j] = jobs[j].pool_experts;
  }
  return from_hip(launch_pool_stream_in((hipStream_t)stream, n, a, src, pex));
}

moe_status moe_stream_in(void* stream, int32_t K, const int32_t* idx, const moe_experts* src,
                         const moe_experts* pool_experts, const moe_pool* pool, int32_t* idx_slot, int32_t* counters,
                         void* workspace, size_t workspace_bytes) {
  if (!src) return MOE_ERR_INVALID_ARG;
  const moe_stream_job j{idx, src, pool_experts, pool, idx_slot, counters};
  return moe_stream_in_many(stream, 1, K, &j, workspace, workspace_bytes);
}

moe_status moe_read_probe(void* stream, const void* buf, size_t bytes, uint32_t* out) {
  if (!buf || !out || bytes < 16 || (bytes & 15) || !aligned16(buf)) return MOE_ERR_INVALID_ARG;
  return from_hip(launch_read_probe((hipStream_t)stream, buf, bytes, out));
}

static bool xchg_cfg_ok(const moe_xchg_cfg* c) {
  if (!c) return false;
  if (c->pattern != MOE_XCHG_ALL && c->pattern != MOE_XCHG_RING) return false;
  if (c->load_scope != MOE_XCHG_SCOPE_DEVICE && c->load_scope != MOE_XCHG_SCOPE_XCD) return false;
  if (c->store_scope != MOE_XCHG_SCOPE_DEVICE && c->store_scope != MOE_XCHG_SCOPE_XCD) return false;
  if (c->xcd_local != 0 && c->xcd_local != 1) return false;
  if (c->n_wg < 1 || c->group_size < 1 || c->n_wg % c->group_size) return false;
  if (c->iters < 1) return false;
  if (c->replicas < 1 || c->replicas > 8) return false;
  if (c->wide_loads < 0 || c->wide_loads > 2) return false;
  if (c->wide_loads == 2 && c->words > 1024) return false;
  if (c->pattern == MOE_XCHG_ALL) {
    if (c->words < c->group_size || c->words % c->group_size || c->words / c->group_size > 64 || c->words > 16384)
      return false;
    if (c->iters > 32767) return false;
  } else if ((int64_t)c->iters * c->group_size > 65535) {
    return false;
  }
  return true;
}

size_t moe_exchange_probe_workspace_size(const moe_xchg_cfg* cfg) {
  return xchg_cfg_ok(cfg) ? xchg_probe_workspace(*cfg) : 0;
}

moe_status moe_exchange_probe(void* stream, const moe_xchg_cfg* cfg, void* workspace, size_t workspace_bytes,
                              uint32_t* out) {
  if (!xchg_cfg_ok(cfg) || !workspace || !out || ((uintptr_t)workspace & 255)) return MOE_ERR_INVALID_ARG;
  if (workspace_bytes < xchg_probe_workspace(*cfg)) return MOE_ERR_INVALID_ARG;
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return MOE_ERR_HIP;
  if (cfg->n_wg > cus) return MOE_ERR_INVALID_ARG;  // every workgroup must be resident at once
  return from_hip(launch_xchg_probe((hipStream_t)stream, *cfg, workspace, out));
}

moe_status moe_sort_by_expert(void* stream, int32_t T, int32_t K, int32_t E, const int32_t* idx, int32_t* counts,
                              int32_t* offsets, int32_t* perm) {
  if (T < 1 || K < 1 || E < 1 || E > MOE_MAX_E || (int64_t)T * K > (1 << 24)) return MOE_ERR_INVALID_ARG;
  if (!idx || !counts || !offsets || !perm) return MOE_ERR_INVALID_ARG;
  return from_hip(launch_sort((hipStream_t)stream, T * K, E, idx, counts, offsets, perm, nullptr));
}

size_t moe_decode_workspace_size(const moe_decode_stack* st) {
  if (!st || st->L < 1 || st->E < 1 || st->K < 1 || st->d_model < 2 || st->d_ff < 1) return 0;
  return decode_step_workspace(*st);
}

static moe_status check_decode_step(const moe_decode_stack* st, int32_t token, uint32_t flags, const uint16_t* h_in,
                                    uint16_t* h_out, uint16_t* h_layers, void* workspace, size_t workspace_bytes) {
  if (!st || !h_in || !h_out || !workspace || token < 0) return MOE_ERR_INVALID_ARG;
  if (flags & ~(MOE_TOPK_RENORM | MOE_DECODE_GIVEN_ROUTING)) return MOE_ERR_INVALID_ARG;
  if (st->norm_gains != 0 && st->norm_gains != 1) return MOE_ERR_INVALID_ARG;
  if (st->L < 1 || st->L > 256 || !routing_dims_ok(1, st->E, st->K)) return MOE_ERR_INVALID_ARG;
  if (!st->layers || !st->route_idx || !st->route_w) return MOE_ERR_INVALID_ARG;
  if (st->bits != 4 && st->bits != 2) return MOE_ERR_UNSUPPORTED;
  if (st->group != 32 && st->group != 64 && st->group != 128) return MOE_ERR_UNSUPPORTED;
  if (st->d_model < 1 || st->d_model > MOE_MAX_D || st->d_ff < 1 || st->d_ff > MOE_MAX_D || st->d_hidden < 0)
    return MOE_ERR_INVALID_ARG;
  if (st->d_model % st->group || st->d_ff % st->group) return MOE_ERR_INVALID_ARG;
  if (((uintptr_t)h_in & 3u) || ((uintptr_t)h_out & 3u) || ((uintptr_t)h_layers & 3u) || ((uintptr_t)workspace & 255u))
    return MOE_ERR_INVALID_ARG;
  if (workspace_bytes < decode_step_workspace(*st)) return MOE_ERR_INVALID_ARG;
  if (!decode_step_supported(*st)) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

moe_status moe_decode_step(void* stream, const moe_decode_stack* st, int32_t token, uint32_t flags,
                           const uint16_t* h_in, uint16_t* h_out, uint16_t* h_layers, void* workspace,
                           size_t workspace_bytes) {
  const moe_status c = check_decode_step(st, token, flags, h_in, h_out, h_layers, workspace, workspace_bytes);
  if (c != MOE_OK) return c;
  return from_hip(launch_decode_step((hipStream_t)stream, *st, token, flags, h_in, h_out, h_layers, workspace));
}

static bool decode_stack_shape_ok(const moe_decode_stack* st) {
  if (!st || st->L < 1 || st->L > 256 || !routing_dims_ok(1, st->E, st->K)) return false;
  return (st->bits == 4 || st->bits == 2) && st->d_model >= 1 && st->d_ff >= 1 && st->d_hidden >= 0;
}

int32_t moe_decode_step_grid(const moe_decode_stack* st) {
  return decode_stack_shape_ok(st) ? decode_step_grid(*st) : 0;
}

int32_t moe_decode_step_grid_for(const moe_decode_stack* st, int32_t compute_units) {
  return decode_stack_shape_ok(st) && compute_units >= 1 ? decode_step_grid_for(*st, compute_units) : 0;
}

moe_status moe_decode_step_stamped(void* stream, const moe_decode_stack* st, int32_t token, uint32_t flags,
                                   const uint16_t* h_in, uint16_t* h_out, uint16_t* h_layers, uint64_t* stamps,
                                   size_t stamp_bytes, void* workspace, size_t workspace_bytes) {
  const moe_status c = check_decode_step(st, token, flags, h_in, h_out, h_layers, workspace, workspace_bytes);
  if (c != MOE_OK) return c;
  const int G = decode_step_grid(*st);
  if (!stamps || ((uintptr_t)stamps & 7u) || G < 1 || stamp_bytes < (size_t)G * st->L * 16 * sizeof(uint64_t))
    return MOE_ERR_INVALID_ARG;
  return from_hip(launch_decode_step((hipStream_t)stream, *st, token, flags, h_in, h_out, h_layers, workspace, stamps));
}

moe_status moe_rmsnorm(void* stream, int32_t T, int32_t d, const uint16_t* h, const uint16_t* gain, uint16_t* x) {
  if (T < 1 || d < 8 || d % 8 || d > MOE_MAX_D || !h || !x) return MOE_ERR_INVALID_ARG;
  if (!aligned16(h) || !aligned16(x) || (gain && !aligned16(gain))) return MOE_ERR_INVALID_ARG;
  return from_hip(launch_rmsnorm((hipStream_t)stream, T, d, h, gain, x));
}

moe_status moe_combine(void* stream, int32_t T, int32_t K, int32_t d, const float* o, const float* w,
                       const uint16_t* r, const float* shared, uint16_t* y) {
  if (T < 1 || K < 1 || K > MOE_MAX_K || d < 1 || d > MOE_MAX_D) return MOE_ERR_INVALID_ARG;
  if (!o || !w || !r || !y) return MOE_ERR_INVALID_ARG;
  return from_hip(launch_combine((hipStream_t)stream, T, K, d, o, w, r, shared, y));
}

}  // extern "C"
