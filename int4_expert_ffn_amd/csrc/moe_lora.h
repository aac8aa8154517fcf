// The first product of an unmerged LoRA adapter, u = A . v, on the batched and decode paths
// ("La otra mitad del muro de la memoria ...", section "Ejecucion del adaptador no fusionado":
// the adapter stays beside the base weights and its two thin products run at every call).
#pragma once
#include "moe_device.h"

namespace moe {

constexpr int LORA_MAX_RANK = 64;  // the largest adapter rank the entry points accept

// u[t][r] = s_t * sum_i A[r][i] v_t[i] for the T rows v_t (row stride v_stride halves) and, with
// A2, u2[t][r] = s_t * A2[r] . v_t in the same pass; s_t is the RMS-norm factor of v_t when
// `rmsnorm`, else 1.  One wave per (token, rank row): waves [0, T*rank) are A's, the next
// T*rank2 are A2's.
struct LoraAJob {
  int T, n_in, rmsnorm;
  const uint16_t* v;
  size_t v_stride;
  const uint16_t* A;
  float* u;
  int rank;
  const uint16_t* A2;  // null: one matrix
  float* u2;
  int rank2;
  __host__ __device__ int waves() const { return T * rank + (A2 ? T * rank2 : 0); }
};

// Wave `wave` of the job (waves past the end return at once).  The sums run in a fixed order, so
// the result does not depend on which kernel hosts the wave.
__device__ __forceinline__ void lora_a_wave(const LoraAJob& j, int wave, int lane) {
  const uint16_t* A = j.A;
  float* u = j.u;
  int rank = j.rank;
  if (wave >= j.T * j.rank) {  // the second matrix's waves (uniform over the wave)
    if (j.A2 == nullptr || wave >= j.waves()) return;
    wave -= j.T * j.rank;
    A = j.A2;
    u = j.u2;
    rank = j.rank2;
  }
  const int t = wave / rank, r = wave % rank;
  const uint16_t* vr = j.v + (size_t)t * j.v_stride;
  const uint16_t* ar = A + (size_t)r * j.n_in;
  float acc = 0.f, sq = 0.f;
  for (int c = lane * 8; c < j.n_in; c += WAVE * 8) {
    const uint4 va = *reinterpret_cast<const uint4*>(vr + c);
    const uint4 aa = *reinterpret_cast<const uint4*>(ar + c);
    const uint32_t vv[4] = {va.x, va.y, va.z, va.w}, av[4] = {aa.x, aa.y, aa.z, aa.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc = __builtin_amdgcn_fdot2(as_h2(vv[i]), as_h2(av[i]), acc, false);
      sq = __builtin_amdgcn_fdot2(as_h2(vv[i]), as_h2(vv[i]), sq, false);
    }
  }
  acc = group_sum(acc, WAVE);
  sq = group_sum(sq, WAVE);
  const float s = j.rmsnorm ? 1.f / sqrtf(sq / (float)j.n_in + RMS_EPS) : 1.f;
  if (lane == 0) u[(size_t)t * rank + r] = acc * s;
}

// The grouped path takes the down adapter's A . act in parts, one per block row of the gate/up
// launch: this many for I activation rows.  Its u_down buffer holds parts x T x rank floats.
int grouped_lora_parts(int I);

}  // namespace moe
