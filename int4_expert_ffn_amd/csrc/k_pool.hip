// Expert streaming into an HBM pool: placement of a token's selected experts in the pool's slots
// and the copy of the missing ones from a slower tier (pinned host memory the GPU reads over the
// host link).
//
// "Arquitecturas nativas para device: MoE de grano fino y pre-attention router", section "Las
// matemáticas que importan": only the active experts and a cache of recent ones stay resident; the
// rest is fetched when needed.  "La otra mitad del muro de la memoria ...", section "Ideas clave":
// experts stream into a compact pool, and the one-token-ahead prediction is the routing, so what
// was prepared is exactly what runs.
//
// Placement (one wave, k_pool_plan): an expert already in a slot is a hit and the slot takes the
// call's stamp (the pool's own call counter, kept on the device, so a replayed graph ages slots as
// a host-side token number baked into it could not); each missing expert, in slot-k order, takes the least recently used slot among
// those this call has not claimed (empty slots first, ties to the lowest slot).  The pool state
// (expert per slot, last-use stamp) lives in device memory, so routing never leaves the GPU.
//
// Copy (k_pool_copy): a few blocks walk (miss, array, chunk) units and move each missing expert's
// nine arrays (q, scales, biases of gate, up and down) with 16-byte loads where the layout allows.
#include "moe_device.h"
#include "moe_launch.h"

namespace moe {
namespace {

constexpr int COPY_THREADS = 256;
constexpr int COPY_UNITS = 8;                                  // 16-byte loads in flight per thread
constexpr int COPY_CHUNK = COPY_THREADS * 16 * COPY_UNITS;     // bytes per block step
constexpr int COPY_BLOCKS = 32;

// wave-wide minimum of a 64-bit key
__device__ __forceinline__ uint64_t wave_min_u64(uint64_t v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const uint32_t lo = __shfl_xor((uint32_t)v, off), hi = __shfl_xor((uint32_t)(v >> 32), off);
    const uint64_t o = ((uint64_t)hi << 32) | lo;
    v = o < v ? o : v;
  }
  return v;
}

__device__ __forceinline__ void pool_plan(const PoolArgs& a);

__global__ void __launch_bounds__(WAVE) k_pool_plan(PoolJobs jobs) { pool_plan(jobs.job[blockIdx.x]); }

__device__ __forceinline__ void pool_plan(const PoolArgs& a) {
  __shared__ int s_exp[MOE_POOL_MAX_SLOTS];
  __shared__ int s_stamp[MOE_POOL_MAX_SLOTS];
  __shared__ int s_slot[MOE_MAX_K];
  __shared__ int s_idx[MOE_MAX_K];
  const int lane = threadIdx.x, S = a.n_slots, K = a.K;
  const int now = *a.clock;   // this call's stamp: the pool's call count
  for (int s = lane; s < S; s += WAVE) {
    s_exp[s] = a.slot_expert[s];
    s_stamp[s] = a.slot_stamp[s];
  }
  if (lane < K) {
    s_slot[lane] = -1;
    s_idx[lane] = a.idx[lane];
  }
  __syncthreads();
  // hits: a slot holding a selected expert keeps it
  for (int s = lane; s < S; s += WAVE) {
    const int e = s_exp[s];
    if (e < 0) continue;
    for (int k = 0; k < K; ++k)
      if (s_idx[k] == e) {
        s_slot[k] = s;
        s_stamp[s] = now;
      }
  }
  __syncthreads();
  int n_hit = 0;
  for (int k = 0; k < K; ++k) n_hit += s_slot[k] >= 0;
  // misses, in slot-k order: the oldest slot this call has not claimed
  int n_copy = 0;
  for (int k = 0; k < K; ++k) {
    const int e = s_idx[k];
    if (s_slot[k] >= 0 || (unsigned)e >= (unsigned)a.E) continue;   // hit, or an index outside [0, E)
    uint64_t best = ~0ull;
    for (int s = lane; s < S; s += WAVE) {
      bool claimed = false;
      for (int j = 0; j < K; ++j) claimed |= s_slot[j] == s;
      if (!claimed) {
        const uint64_t key = ((uint64_t)(uint32_t)(s_stamp[s] + 1) << 32) | (uint32_t)s;
        best = key < best ? key : best;
      }
    }
    best = wave_min_u64(best);
    if (best == ~0ull) continue;   // no free slot (fewer slots than K, refused on the host)
    const int v = (int)(uint32_t)best;
    if (lane == 0) {
      s_slot[k] = v;
      s_exp[v] = e;
      s_stamp[v] = now;
      a.plan[1 + 2 * n_copy] = v;
      a.plan[2 + 2 * n_copy] = e;
    }
    __syncthreads();
    ++n_copy;
  }
  for (int s = lane; s < S; s += WAVE) {
    a.slot_expert[s] = s_exp[s];
    a.slot_stamp[s] = s_stamp[s];
  }
  if (lane < K) a.idx_slot[lane] = s_slot[lane];
  if (lane == 0) {
    *a.clock = now + 1;
    a.plan[0] = n_copy;
    if (a.counters) {   // calls on other streams may share them
      atomicAdd(&a.counters[0], n_hit);
      atomicAdd(&a.counters[1], n_copy);
    }
  }
}

// one of the nine per-expert arrays of a job: bytes per expert, source and pool bases, and the first
// work unit (chunk) of the array in the per-expert chunk list
struct CopyArr {
  const unsigned char* src;
  unsigned char* dst;
};
struct CopyJobs {
  CopyArr arr[MOE_POOL_MAX_JOBS][9];
  const int32_t* plan[MOE_POOL_MAX_JOBS];
  size_t bytes[9];   // per expert, the same for every job
  int chunk0[9];     // chunks of the arrays before this one
  int chunks;        // chunks per expert, all nine arrays
  int n;             // jobs
};

// A small grid that walks (job, copy, array, chunk) units: the copy reads host memory at the host
// link's pace whatever the grid size, and a few resident blocks leave the other CUs to the kernels
// that run beside it (a grid of thousands of short blocks kept them waiting for the dispatcher).
__global__ void __launch_bounds__(COPY_THREADS) k_pool_copy(CopyJobs c) {
  int first[MOE_POOL_MAX_JOBS + 1];   // first unit of each job
  first[0] = 0;
#pragma unroll
  for (int j = 0; j < MOE_POOL_MAX_JOBS; ++j) first[j + 1] = first[j] + (j < c.n ? c.plan[j][0] * c.chunks : 0);
  const int n_units = first[MOE_POOL_MAX_JOBS];
  for (int u = blockIdx.x; u < n_units; u += gridDim.x) {
    int j = 0;
#pragma unroll
    for (int i = 1; i < MOE_POOL_MAX_JOBS; ++i) j += u >= first[i];
    const int v = u - first[j];
    const int m = v / c.chunks, cu = v - m * c.chunks;
    int a = 0;
#pragma unroll
    for (int i = 1; i < 9; ++i) a += cu >= c.chunk0[i];
    const CopyArr& A = c.arr[j][a];
    const size_t bytes = c.bytes[a];
    const size_t begin = (size_t)(cu - c.chunk0[a]) * COPY_CHUNK;
    const int slot = c.plan[j][1 + 2 * m], e = c.plan[j][2 + 2 * m];
    const unsigned char* src = A.src + (size_t)e * bytes;
    unsigned char* dst = A.dst + (size_t)slot * bytes;
    const size_t end = min(bytes, begin + (size_t)COPY_CHUNK);
    if ((bytes & 15) == 0 && (((uintptr_t)A.src | (uintptr_t)A.dst) & 15) == 0) {
      uint4 v4[COPY_UNITS];
#pragma unroll
      for (int i = 0; i < COPY_UNITS; ++i) {
        const size_t o = begin + ((size_t)i * COPY_THREADS + threadIdx.x) * 16;
        if (o < end) v4[i] = *reinterpret_cast<const uint4*>(src + o);
      }
#pragma unroll
      for (int i = 0; i < COPY_UNITS; ++i) {
        const size_t o = begin + ((size_t)i * COPY_THREADS + threadIdx.x) * 16;
        if (o < end) *reinterpret_cast<uint4*>(dst + o) = v4[i];
      }
    } else {   // 2-byte units (every array holds whole float16 or uint32 elements)
      for (size_t o = begin + (size_t)threadIdx.x * 2; o < end; o += (size_t)COPY_THREADS * 2)
        *reinterpret_cast<uint16_t*>(dst + o) = *reinterpret_cast<const uint16_t*>(src + o);
    }
  }
}

}  // namespace

hipError_t launch_pool_stream_in(hipStream_t s, int n, const PoolArgs* jobs, const moe_experts* const* src,
                                 const moe_experts* const* pool) {
  PoolJobs pj{};
  for (int j = 0; j < n; ++j) pj.job[j] = jobs[j];
  hipError_t err = launch(k_pool_plan, dim3(n), dim3(WAVE), 0, s, pj);
  if (err != hipSuccess) return err;
  const moe_experts& s0 = *src[0];
  const size_t d = s0.d_model, I = s0.d_ff, bits = s0.bits, g = s0.group;
  const size_t qb = I * d * bits / 8;                  // codes of one matrix of one expert
  const size_t gu_sb = I * (d / g) * 2;                // gate / up scales (or biases) of one expert
  const size_t dn_sb = d * I / g * 2;                  // down scales (or biases): the same count either layout
  CopyJobs c{};
  int chunk0 = 0;
  for (int m = 0; m < 3; ++m) {
    const size_t sb = m < 2 ? gu_sb : dn_sb;
    const size_t b3[3] = {qb, sb, sb};
    for (int i = 0; i < 3; ++i) {
      c.bytes[3 * m + i] = b3[i];
      c.chunk0[3 * m + i] = chunk0;
      chunk0 += (int)((b3[i] + COPY_CHUNK - 1) / COPY_CHUNK);
    }
  }
  c.chunks = chunk0;
  c.n = n;
  for (int j = 0; j < n; ++j) {
    const moe_qmat* sm[3] = {&src[j]->gate, &src[j]->up, &src[j]->down};
    const moe_qmat* pm[3] = {&pool[j]->gate, &pool[j]->up, &pool[j]->down};
    for (int m = 0; m < 3; ++m) {
      c.arr[j][3 * m] = CopyArr{(const unsigned char*)sm[m]->q, (unsigned char*)pm[m]->q};
      c.arr[j][3 * m + 1] = CopyArr{(const unsigned char*)sm[m]->scales, (unsigned char*)pm[m]->scales};
      c.arr[j][3 * m + 2] = CopyArr{(const unsigned char*)sm[m]->biases, (unsigned char*)pm[m]->biases};
    }
    c.plan[j] = jobs[j].plan;
  }
  return launch(k_pool_copy, dim3(COPY_BLOCKS), dim3(COPY_THREADS), 0, s, c);
}

size_t pool_plan_bytes(int K) { return (size_t)(1 + 2 * K) * sizeof(int32_t); }

}  // namespace moe
