// Exchange-latency probe: how long one hand-off of tagged 8-byte words between resident
// workgroups takes, the unit every grid-wide step of the persistent decode kernel pays.  Not a
// step of the method; a measurement aid in the library so that the latency figures the decode
// design rests on come from committed code.
//
// One workgroup of one wave per compute unit (a large static LDS allocation keeps two from
// sharing a CU).  Workgroups form groups; a group is either `group_size` consecutive workgroup
// numbers (which the dispatcher deals round robin over the XCDs, so a group spans them all) or the
// workgroups b with equal b % 8 (one XCD each under that dealing; every workgroup reports the XCD
// it ran on, read from the hardware register, so the caller can check).  Two patterns:
//   * ALL: in every phase each member publishes `words / group_size` words of a vector and then
//     polls the whole vector until every word carries the phase's tag: the exchange of h and of
//     the SwiGLU outputs in the decode kernel (two buffers by phase parity, so a member that runs
//     ahead never overwrites a word a slow member has yet to read);
//   * RING: one word is passed member to member, each hop one store and one poll: the latency of a
//     single hand-off.
// Loads are either agent-scope (device-coherent: what crosses XCDs needs) or XCD-scope (the L1 is
// bypassed and the XCD's L2 answers: enough inside one XCD); stores either device-coherent or plain
// (they end in the XCD's L2).  A mismatch (XCD-scope traffic across XCDs) shows up as a wait that
// runs out: every wait is bounded (0.1 s), raises the error count and lets the grid finish.
#include "moe_device.h"
#include "moe_launch.h"

namespace moe {
namespace {

constexpr int XP_LDS_WORDS = 22 * 1024;        // 88 KiB of LDS: more than half a CU's, one workgroup per CU
constexpr uint64_t XP_WAIT_TICKS = 10000000;   // 0.1 s at the 100 MHz real-time counter
constexpr int XP_POLL = 16;                    // words per lane per polling pass
constexpr uint32_t XP_SALT = 0x3C3C3C3Cu;
constexpr uint32_t XP_OFF_NONE = 0x80000000u;  // past the workspace: the hardware drops the access
constexpr int CPOL_SC0 = 1, CPOL_SC1 = 16;

struct XchgParams {
  int pattern, n_wg, gs, xcd_local, words, iters, replicas, wide;
  int load_aux, store_aux;  // cache-policy bits of the polling loads and of the stores
  uint32_t epoch;
  const void* ws;
  uint32_t ws_bytes;
  uint32_t start_off, groups_off, group_stride, copy_stride;  // byte offsets into the workspace
  uint32_t* out;
};

typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t xp_tag(uint32_t epoch, int phase) { return ((epoch << 16) | (uint32_t)phase) ^ XP_SALT; }

__device__ __forceinline__ uint64_t xp_load(__amdgpu_buffer_rsrc_t rs, uint32_t off, int aux) {
  // the cache policy must be a constant: two call sites
  const u32x2 v = aux == CPOL_SC1 ? __builtin_amdgcn_raw_buffer_load_b64(rs, off, 0, CPOL_SC1)
                                  : __builtin_amdgcn_raw_buffer_load_b64(rs, off, 0, CPOL_SC0);
  return (uint64_t)v.x | ((uint64_t)v.y << 32);
}
__device__ __forceinline__ void xp_store(__amdgpu_buffer_rsrc_t rs, uint32_t off, bool on, uint32_t payload, uint32_t tag,
                                         int aux) {
  u32x2 v;
  v.x = payload;
  v.y = tag;
  if (aux == CPOL_SC1)
    __builtin_amdgcn_raw_buffer_store_b64(v, rs, on ? off : XP_OFF_NONE, 0, CPOL_SC1);
  else
    __builtin_amdgcn_raw_buffer_store_b64(v, rs, on ? off : XP_OFF_NONE, 0, 0);
}

// Poll n words at byte offset `base` until each carries `tag` (whole wave, NP words per lane per
// pass, two passes in flight; NP = the fewest that cover n, at most 16, so that no lane loads a
// word twice in one pass).  Bounded: past XP_WAIT_TICKS it counts an error and sets `failed`.
template <int NP>
__device__ void xp_wait_np(__amdgpu_buffer_rsrc_t rs, uint32_t base, int n, uint32_t tag, int aux, uint32_t* err,
                           bool& failed) {
  const int lane = threadIdx.x % WAVE;
  const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
  for (int b0 = 0; b0 < n; b0 += NP * WAVE) {
    uint32_t done = 0;
#pragma unroll
    for (int j = 0; j < NP; ++j)
      if (b0 + lane + j * WAVE >= n) done |= 1u << j;
    uint64_t a[NP], b[NP];
    auto issue = [&](uint64_t (&v)[NP]) {
#pragma unroll
      for (int j = 0; j < NP; ++j) v[j] = xp_load(rs, base + 8u * (uint32_t)min(b0 + lane + j * WAVE, n - 1), aux);
    };
    auto check = [&](const uint64_t (&v)[NP]) {
#pragma unroll
      for (int j = 0; j < NP; ++j)
        if ((uint32_t)(v[j] >> 32) == tag) done |= 1u << j;
    };
    issue(a);
    while (true) {
      issue(b);
      check(a);
      if (__all(done == (1u << NP) - 1)) break;
      issue(a);
      check(b);
      if (__all(done == (1u << NP) - 1)) break;
      if (__builtin_amdgcn_s_memrealtime() - t0 > XP_WAIT_TICKS) {
        if (lane == 0) atomicAdd(err, 1u);
        failed = true;
        return;
      }
    }
  }
}
// The same with 16-byte loads: each lane reads two consecutive words per load (NI loads per lane
// per pass cover 128 NI words).
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ u32x4 xp_load16(__amdgpu_buffer_rsrc_t rs, uint32_t off, int aux) {
  return aux == CPOL_SC1 ? __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, CPOL_SC1)
                         : __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, CPOL_SC0);
}
template <int NI>
__device__ void xp_wait_wide(__amdgpu_buffer_rsrc_t rs, uint32_t base, int n, uint32_t tag, int aux, uint32_t* err,
                             bool& failed) {
  const int lane = threadIdx.x % WAVE;
  const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
  for (int b0 = 0; b0 < n; b0 += 2 * NI * WAVE) {
    uint32_t done = 0;
#pragma unroll
    for (int j = 0; j < NI; ++j)
      if (b0 + 2 * (lane + j * WAVE) >= n) done |= 3u << (2 * j);
    while (true) {
      u32x4 v[NI];
#pragma unroll
      for (int j = 0; j < NI; ++j) v[j] = xp_load16(rs, base + 8u * (uint32_t)min(b0 + 2 * (lane + j * WAVE), n - 2), aux);
#pragma unroll
      for (int j = 0; j < NI; ++j) {
        if (v[j].y == tag) done |= 1u << (2 * j);
        if (v[j].w == tag) done |= 2u << (2 * j);
      }
      if (__all(done == (1u << (2 * NI)) - 1)) break;
      if (__builtin_amdgcn_s_memrealtime() - t0 > XP_WAIT_TICKS) {
        if (lane == 0) atomicAdd(err, 1u);
        failed = true;
        return;
      }
    }
  }
}

// The same with agent-scope atomic 8-byte loads through the global (flat) path instead of buffer
// loads (NP words per lane per pass; the decode kernel's polling loads).
template <int NP>
__device__ void xp_wait_global(const uint64_t* src, int n, uint32_t tag, uint32_t* err, bool& failed) {
  const int lane = threadIdx.x % WAVE;
  const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
  for (int b0 = 0; b0 < n; b0 += NP * WAVE) {
    uint32_t done = 0;
#pragma unroll
    for (int j = 0; j < NP; ++j)
      if (b0 + lane + j * WAVE >= n) done |= 1u << j;
    uint64_t a[NP], b[NP];
    auto issue = [&](uint64_t (&v)[NP]) {
#pragma unroll
      for (int j = 0; j < NP; ++j)
        v[j] = __hip_atomic_load(src + min(b0 + lane + j * WAVE, n - 1), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    };
    auto check = [&](const uint64_t (&v)[NP]) {
#pragma unroll
      for (int j = 0; j < NP; ++j)
        if ((uint32_t)(v[j] >> 32) == tag) done |= 1u << j;
    };
    issue(a);
    while (true) {
      issue(b);
      check(a);
      if (__all(done == (1u << NP) - 1)) break;
      issue(a);
      check(b);
      if (__all(done == (1u << NP) - 1)) break;
      if (__builtin_amdgcn_s_memrealtime() - t0 > XP_WAIT_TICKS) {
        if (lane == 0) atomicAdd(err, 1u);
        failed = true;
        return;
      }
    }
  }
}

__device__ void xp_wait_all(__amdgpu_buffer_rsrc_t rs, uint32_t base, int n, uint32_t tag, int aux, uint32_t* err,
                            bool& failed, int wide = 0, const void* ws = nullptr) {
  if (failed) return;
  if (wide == 2) {  // global atomic loads, sixteen per lane per pass (n <= 1024)
    const uint64_t* src = (const uint64_t*)((const char*)ws + base);
    if (n <= 4 * WAVE) xp_wait_global<4>(src, n, tag, err, failed);
    else if (n <= 8 * WAVE) xp_wait_global<8>(src, n, tag, err, failed);
    else xp_wait_global<16>(src, n, tag, err, failed);
    return;
  }
  if (wide) {
    if (n <= 2 * WAVE) xp_wait_wide<1>(rs, base, n, tag, aux, err, failed);
    else if (n <= 4 * WAVE) xp_wait_wide<2>(rs, base, n, tag, aux, err, failed);
    else if (n <= 8 * WAVE) xp_wait_wide<4>(rs, base, n, tag, aux, err, failed);
    else xp_wait_wide<8>(rs, base, n, tag, aux, err, failed);
    return;
  }
  if (n <= WAVE) xp_wait_np<1>(rs, base, n, tag, aux, err, failed);
  else if (n <= 2 * WAVE) xp_wait_np<2>(rs, base, n, tag, aux, err, failed);
  else if (n <= 4 * WAVE) xp_wait_np<4>(rs, base, n, tag, aux, err, failed);
  else if (n <= 8 * WAVE) xp_wait_np<8>(rs, base, n, tag, aux, err, failed);
  else xp_wait_np<XP_POLL>(rs, base, n, tag, aux, err, failed);
}

// Single-word wait of the ring (lane 0 polls; the wave follows).
__device__ void xp_wait_one(__amdgpu_buffer_rsrc_t rs, uint32_t off, uint32_t tag, int aux, uint32_t* err, bool& failed) {
  if (failed) return;
  const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
  while (true) {
    const uint64_t v = xp_load(rs, off, aux);
    if (__builtin_amdgcn_readfirstlane((uint32_t)(v >> 32)) == tag) return;
    if (__builtin_amdgcn_s_memrealtime() - t0 > XP_WAIT_TICKS) {
      if (threadIdx.x == 0) atomicAdd(err, 1u);
      failed = true;
      return;
    }
  }
}

__device__ __forceinline__ uint32_t xcc_id() {
  uint32_t v;
  asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(v));
  return v & 0xFu;
}

__global__ void __launch_bounds__(WAVE) k_xchg_probe(XchgParams p) {
  __shared__ uint32_t pad[XP_LDS_WORDS];  // occupancy only
  const int b = blockIdx.x, lane = threadIdx.x;
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p.ws), 0, p.ws_bytes, 0x00020000);
  uint32_t* err = p.out;
  bool failed = false;
  // group and rank of this workgroup
  const int ngroups = p.n_wg / p.gs;
  const int g = p.xcd_local ? b % ngroups : b / p.gs;
  const int r = p.xcd_local ? b / ngroups : b % p.gs;
  pad[lane] = (uint32_t)r;  // keeps the allocation (read back only under a condition the host rules out)
  __syncthreads();
  if (p.iters < 0) p.out[0] = pad[(lane + 1) % WAVE];
  // start together: every workgroup publishes one word, then waits for all of them (device scope)
  xp_store(rs, p.start_off + 8u * (uint32_t)b, lane == 0, 0, xp_tag(p.epoch, 0), CPOL_SC1);
  xp_wait_all(rs, p.start_off, p.n_wg, xp_tag(p.epoch, 0), CPOL_SC1, err, failed);
  const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
  const uint32_t gbase = p.groups_off + (uint32_t)g * p.group_stride;
  if (p.pattern == MOE_XCHG_ALL) {
    // every word is stored in `replicas` copies; a member reads copy b % replicas (its XCD's when
    // replicas is 8), so the readers of one copy are fewer and its lines less contended
    const int per = p.words / p.gs;
    for (int ph = 1; ph <= p.iters; ++ph) {
      const uint32_t buf = gbase + (uint32_t)(ph & 1) * 8u * (uint32_t)p.words;
      const uint32_t tag = xp_tag(p.epoch, ph);
      for (int c = 0; c < p.replicas; ++c)
        xp_store(rs, buf + (uint32_t)c * p.copy_stride + 8u * (uint32_t)(r * per + min(lane, per - 1)), lane < per,
                 (uint32_t)ph, tag, p.store_aux);
      xp_wait_all(rs, buf + (uint32_t)(b % p.replicas) * p.copy_stride, p.words, tag, p.load_aux, err, failed,
                  p.wide, p.ws);
    }
  } else {  // RING: slot s of the group at gbase + 256 s; hop v lands in slot v % gs
    const uint32_t mine = gbase + 256u * (uint32_t)r, next = gbase + 256u * (uint32_t)((r + 1) % p.gs);
    for (int lap = 0; lap < p.iters; ++lap) {
      const int v = lap * p.gs + r;  // the hop that reaches this member
      if (v > 0) xp_wait_one(rs, mine, xp_tag(p.epoch, v), p.load_aux, err, failed);
      xp_store(rs, next, lane == 0, 0, xp_tag(p.epoch, v + 1), p.store_aux);
    }
    if (r == 0) xp_wait_one(rs, mine, xp_tag(p.epoch, p.iters * p.gs), p.load_aux, err, failed);
  }
  const uint64_t t1 = __builtin_amdgcn_s_memrealtime();
  if (lane == 0) {
    p.out[1 + 3 * b] = (uint32_t)(t1 - t0);
    p.out[2 + 3 * b] = (uint32_t)((t1 - t0) >> 32);
    p.out[3 + 3 * b] = xcc_id();
  }
}

}  // namespace

size_t xchg_probe_workspace(const moe_xchg_cfg& c) {
  const size_t start = ((size_t)c.n_wg * 8 + 255) / 256 * 256;
  const size_t per = c.pattern == MOE_XCHG_ALL ? (size_t)c.replicas * (((size_t)2 * c.words * 8 + 255) / 256 * 256)
                                              : (size_t)c.group_size * 256;
  return 256 + start + (size_t)(c.n_wg / c.group_size) * per;
}

hipError_t launch_xchg_probe(hipStream_t s, const moe_xchg_cfg& c, void* ws, uint32_t* out) {
  XchgParams p{};
  p.pattern = c.pattern;
  p.n_wg = c.n_wg;
  p.gs = c.group_size;
  p.xcd_local = c.xcd_local;
  p.words = c.words;
  p.iters = c.iters;
  p.load_aux = c.load_scope == MOE_XCHG_SCOPE_XCD ? CPOL_SC0 : CPOL_SC1;
  p.store_aux = c.store_scope == MOE_XCHG_SCOPE_XCD ? 0 : CPOL_SC1;
  p.epoch = c.epoch;
  p.ws = ws;
  const size_t total = xchg_probe_workspace(c);
  p.ws_bytes = (uint32_t)total;
  p.start_off = 256;
  p.groups_off = 256 + (uint32_t)(((size_t)c.n_wg * 8 + 255) / 256 * 256);
  p.copy_stride = (uint32_t)(((size_t)2 * c.words * 8 + 255) / 256 * 256);
  p.replicas = c.pattern == MOE_XCHG_ALL ? c.replicas : 1;
  p.wide = c.wide_loads;
  p.group_stride = c.pattern == MOE_XCHG_ALL ? (uint32_t)c.replicas * p.copy_stride : (uint32_t)c.group_size * 256u;
  p.out = out;
  return launch(k_xchg_probe, dim3(c.n_wg), dim3(WAVE), 0, s, p);
}

}  // namespace moe
