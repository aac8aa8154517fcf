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
  uint16_t* act;           // workspace [T][K][I] float16
  float* u_gate;           // workspace [T][rank] (LoRA)
  float* u_up;
  float* u_down;
};
hipError_t launch_expert_decode(hipStream_t s, const DecodeArgs& a);
bool decode_shape_supported(int bits, int group, int d, int I);

// batched (grouped GEMM) expert FFN ------------------------------------------------------------
struct GroupedArgs {
  DecodeArgs base;
  int32_t* counts;    // workspace [E]
  int32_t* offsets;   // workspace [E+1]
  int32_t* perm;      // workspace [T*K]
  float* o_sorted;    // workspace [T*K][d] float32 (used when out == nullptr)
};
hipError_t launch_expert_grouped(hipStream_t s, const GroupedArgs& a);
size_t grouped_workspace_extra(int T, int K, int E, int d);

// combine -------------------------------------------------------------------------------------
hipError_t launch_combine(hipStream_t s, int T, int K, int d, const float* o, const float* w,
                          const uint16_t* r, const float* shared, uint16_t* y);

}  // namespace moe
