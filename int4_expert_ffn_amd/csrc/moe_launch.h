// Internal launchers: host-side C++ functions that enqueue the gfx950 kernels.  Arguments are
// already validated by the C ABI layer (moe_api.hip); every launcher returns hipGetLastError().
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/moe.h"

namespace moe {

// routing ---------------------------------------------------------------------------------
hipError_t launch_router_gemv(hipStream_t s, int T, int d, int E, uint32_t flags, const uint16_t* x,
                              const uint16_t* w, float* logits);
hipError_t launch_topk(hipStream_t s, int T, int E, int K, uint32_t flags, const float* logits,
                       int32_t* idx, float* w);

// prerouter head ----------------------------------------------------------------------------
hipError_t launch_prerouter(hipStream_t s, int T, int d, int E, int K, uint32_t flags,
                            const uint16_t* x, const int32_t* idx_cur, const int32_t* idx_prev,
                            const moe_prerouter_w& pw, float* logits, float* ws_g, float* ws_lin);

// decode expert FFN -------------------------------------------------------------------------
struct DecodeArgs {
  int T, K, E, d, I, bits, group;
  uint32_t flags;
  const uint16_t* x;
  const int32_t* idx;
  moe_experts ex;
  const moe_lora* lora3;   // nullptr or [3]
  float* out;              // [T][K][d] or nullptr
  const float* w_fuse;     // [T][K] or nullptr
  const uint16_t* r_fuse;  // [T][d] or nullptr
  uint16_t* y_fuse;        // [T][d] or nullptr
  void* act;               // workspace: decode [T][K][I] float32; batched [T*K][I] float16 (expert-sorted)
  float* u_gate;           // workspace [T][rank] (LoRA)
  float* u_up;
  float* u_down;
  bool relu;               // ReLU on the gate branch instead of SiLU (activation-sparse variant)
  int32_t* zero;           // [T][nzero] int32 cleared by the gate/up kernel, or nullptr
  int nzero;
  const moe_experts* shared;  // batched path only: a shared expert run with the routed ones (lora3 is
                              // its LoRA), whose output joins the fused combine; nullptr: none
};
hipError_t launch_expert_decode(hipStream_t s, const DecodeArgs& a);
// gate/up + activation only (act[T][K][I] float32), for the activation-sparse variant
hipError_t launch_gateup_decode(hipStream_t s, const DecodeArgs& a);

// ReLU activation-sparse down projection over neuron-major rows, then the combine
struct SparseArgs {
  DecodeArgs base;         // base.act: act[T][K][I] from launch_gateup_decode; base.ex.down neuron-major
  float* o;                // [T][K][d] float32: base.out, or workspace when only the fused output is wanted
  int32_t* cnt;            // workspace [T][nslab]: blocks done per (token, slab), cleared by the gate/up kernel
  int32_t* n_active;       // [T][K] or nullptr
};
int sparse_slabs(int bits, int d);  // column slabs of the down kernel (0: unsupported shape)
size_t sparse_lds(int bits, int I); // dynamic LDS bytes of the down kernel
hipError_t launch_down_sparse(hipStream_t s, const SparseArgs& a);
bool decode_shape_supported(int bits, int group, int d, int I);
// u[t][r] = s_t * A[r] . v_t for `waves` = T * rank waves (s_t = RMS-norm factor when rmsnorm)
// u[t][r] = A[r] . v_t (v_t optionally RMS-normed); with A2 also u2 = A2 . v_t in the same launch
// (the two ranks equal).  waves = T * rank.
hipError_t launch_lora_a(hipStream_t s, int waves, int T, int n_in, int rank, int rmsnorm, const uint16_t* v,
                         size_t v_stride, const uint16_t* A, float* u, const uint16_t* A2 = nullptr,
                         float* u2 = nullptr);

// batched (grouped GEMM) expert FFN ------------------------------------------------------------
// With a shared expert (base.shared), NB = E + 2 buckets and NP = T*K + T pairs (the shared
// expert's pair of token t is T*K + t, in bucket E + 1); else NB = E + 1 and NP = T*K.
struct GroupedArgs {
  DecodeArgs base;    // base.act holds the expert-sorted activations [NP][I]
  int32_t* counts;    // workspace [NB] (bucket E: indices outside [0, E))
  int32_t* offsets;   // workspace [NB+1]
  int32_t* perm;      // workspace [NP]
  float* rowscale;    // workspace [T]
  float* o_sorted;    // workspace [NP][d] float32 (used when out == nullptr or with a shared expert)
  int32_t* tiles;     // workspace: the grouped GEMMs' work list (count, then one record per tile)
};
hipError_t launch_expert_grouped(hipStream_t s, const GroupedArgs& a);
hipError_t launch_sort(hipStream_t s, int TK, int E, const int32_t* idx, int32_t* counts, int32_t* offsets,
                       int32_t* perm, int32_t* tiles, int TS = 0);
// byte offsets of GroupedArgs' workspace arrays (TS: the shared expert's pairs, T or 0)
struct GroupedLayout {
  size_t counts, offsets, perm, rowscale, o_sorted, tiles, total;
};
GroupedLayout grouped_layout(int T, int K, int E, int d, int TS);

// whole-token persistent decode -----------------------------------------------------------------
bool decode_step_supported(const moe_decode_stack& st);
size_t decode_step_workspace(const moe_decode_stack& st);
hipError_t launch_decode_step(hipStream_t s, const moe_decode_stack& st, int token, uint32_t flags,
                              const uint16_t* h_in, uint16_t* h_out, uint16_t* h_layers, void* ws,
                              uint64_t* stamps = nullptr);
int decode_step_grid(const moe_decode_stack& st);  // workgroups of one launch (0: unsupported)
int decode_step_grid_for(const moe_decode_stack& st, int cus);  // the same on a device with `cus` CUs

// expert streaming into an HBM pool --------------------------------------------------------------
struct PoolArgs {
  int K, E, n_slots;
  const int32_t* idx;      // [K] selected experts
  int32_t* slot_expert;    // [n_slots] pool state
  int32_t* slot_stamp;     // [n_slots]
  int32_t* clock;          // [1] calls so far (the stamp of this call)
  int32_t* idx_slot;       // [K] out
  int32_t* counters;       // [2] hits, misses (accumulated) or nullptr
  int32_t* plan;           // workspace: copy count, then (slot, expert) pairs
};
struct PoolJobs {
  PoolArgs job[MOE_POOL_MAX_JOBS];
};
// n <= MOE_POOL_MAX_JOBS pools of one shape: placement (one wave per pool), then one copy grid for all
hipError_t launch_pool_stream_in(hipStream_t s, int n, const PoolArgs* jobs, const moe_experts* const* src,
                                 const moe_experts* const* pool);
size_t pool_plan_bytes(int K);

// measurement aid: streaming read of a buffer (MOE_READ_PROBE_BLOCKS words out)
hipError_t launch_read_probe(hipStream_t s, const void* buf, size_t bytes, uint32_t* out);
// measurement aid: tagged-word hand-off latency between resident workgroups
size_t xchg_probe_workspace(const moe_xchg_cfg& c);
hipError_t launch_xchg_probe(hipStream_t s, const moe_xchg_cfg& c, void* ws, uint32_t* out);

// combine -------------------------------------------------------------------------------------
hipError_t launch_rmsnorm(hipStream_t s, int T, int d, const uint16_t* h, const uint16_t* gain, uint16_t* x);
hipError_t launch_combine(hipStream_t s, int T, int K, int d, const float* o, const float* w,
                          const uint16_t* r, const float* shared, uint16_t* y);

}  // namespace moe
