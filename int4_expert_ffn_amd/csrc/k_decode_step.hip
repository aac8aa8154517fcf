// One decode token through every layer of a resident prerouted stack, as ONE persistent kernel.
//
// The method is the per-layer one of the other kernels (router or prerouter routing, softmax
// top-K, dequantised gate/up + SwiGLU, down + weighted combine + residual; pages: "La otra mitad
// del muro de la memoria ..." sections "Ideas clave" and "Arquitectura del cabezal Prerouter",
// "Inferencia de LLM MoE en MacBook Pro ..." section "Arquitectura del Sistema"); what changes is
// the schedule.  At batch 1 every layer moves only ~13 MB, so a launch per step (a few us each)
// costs more than the bytes.  Here one workgroup per CU stays resident for the whole token:
//
//   * Work is split statically: every workgroup owns a slice of the gate/up row pairs, of the
//     head's fc1 / linear rows, of the down rows (all K experts of a row live in one workgroup,
//     so the weighted combine stays local and in fixed order) and of the fc2 rows.
//   * The SwiGLU output travels in float32 and meets the down weights as a float16 hi + lo pair.
//   * Data moves between workgroups as tagged 8-byte words (32-bit payload, 32-bit tag naming
//     the token epoch and the phase), written and read with agent-scope relaxed atomics; a
//     reader polls until every tag matches, so no flag/data ordering is needed.
//   * Per workgroup, wave 0 only waits for and unpacks the vector the next phase needs (into
//     LDS); waves 1..4 compute.  Their weight loads for a phase are issued one phase early, and
//     workgroup barriers fence LDS only, so those loads stay in flight while the phase waits.
//   * The heads (off the critical path: their output routes the next token) ride in the same
//     phases; their top-Ks run after the last layer, spread over the workgroups.
//   * The whole token's routing state is staged in LDS at the start, so issuing a phase's weight
//     loads never waits on a global read of the expert indices.
//
// Phases per layer l: [R_l: own router + top-K, only for layer 0, layers with no prediction and
// the first token] -> A_l: gate/up + SwiGLU, head fc1 (+GELU) and linear rows -> B_l: down +
// combine + residual, head fc2 rows.  Every wait is bounded in time: one that runs out sets the
// error word and lets the kernel finish (its results are then invalid).
#include "moe_device.h"
#include "moe_launch.h"

namespace moe {
namespace {

constexpr int MW = 4;                        // compute waves per workgroup
constexpr int NTHREADS = (MW + 1) * WAVE;
constexpr int GU_MAX = 4;                    // gate/up row pairs per compute wave
constexpr int NH_MAX = 2;                    // head fc1/linear rows per compute wave
constexpr int PD_MAX = 8;                    // (expert, row-group) down items per compute wave
constexpr int LDS_D = 4096, LDS_ACT = 4096, LDS_H = 2048, LDS_E = 1024, LDS_PART = 512, LDS_LK = 512;
constexpr int POLL_MAX = 16;                 // words per lane per polling pass (1024 per wave)
constexpr uint32_t TAG_SALT = 0x5A5A5A5Au;
constexpr uint64_t WAIT_TICKS = 20000000;       // 0.2 s of the 100 MHz real-time counter

struct StepParams {
  int L, E, K, d, I, H, lg2g;
  int G, GU, NH, NR, NO, DR, DI, PD, Ldn;
  const moe_decode_layer* layers;
  const uint16_t* h_in;
  uint16_t* h_out;
  int32_t* ridx;
  float* rw;
  int slot, bootstrap;
  uint32_t topk_flags;
  uint64_t *ll_logits, *ll_act, *ll_g, *ll_lin, *ll_hlog, *ll_h;
  uint32_t* epoch;
  int* err;
};

__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

__device__ __forceinline__ void ll_store(uint64_t* p, uint32_t payload, uint32_t tag) {
  __hip_atomic_store(p, ((uint64_t)tag << 32) | payload, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t ll_load(const uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Poll n tagged words until all carry `tag`; sink(i, payload) receives each word once.
// Whole wave, POLL_MAX words per lane per pass.  A wait is bounded in wall-clock time: past
// WAIT_TICKS it raises the error word, sets `failed`, and every later wait of this wave returns
// at once, so a grid that cannot make progress still finishes quickly (with invalid results).
template <class Sink>
__device__ __forceinline__ void ll_wait(const uint64_t* src, int n, uint32_t tag, int* err, bool& failed, Sink sink) {
  if (failed) return;
  const int lane = threadIdx.x % WAVE;
  const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
  for (int base = 0; base < n; base += POLL_MAX * WAVE) {
    uint32_t done = 0;
#pragma unroll
    for (int j = 0; j < POLL_MAX; ++j)
      if (base + lane + j * WAVE >= n) done |= 1u << j;
    while (true) {
      uint64_t v[POLL_MAX];
#pragma unroll
      for (int j = 0; j < POLL_MAX; ++j)
        if (!((done >> j) & 1u)) v[j] = ll_load(src + base + lane + j * WAVE);
#pragma unroll
      for (int j = 0; j < POLL_MAX; ++j)
        if (!((done >> j) & 1u) && (uint32_t)(v[j] >> 32) == tag) {
          sink(base + lane + j * WAVE, (uint32_t)v[j]);
          done |= 1u << j;
        }
      if (__all(done == (1u << POLL_MAX) - 1u)) break;
      if (__builtin_amdgcn_s_memrealtime() - t0 > WAIT_TICKS) {
        if (lane == 0) atomicAdd(err, 1);
        failed = true;
        return;
      }
    }
  }
}

// DPP sum inside aligned groups of G lanes (G a power of two <= 64); the sum lands in the last
// lane of each group.  Out-of-range DPP sources contribute zero.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_add(float x) {
  return x + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, ROW_MASK, 0xf, false));
}
__device__ __forceinline__ float group_sum_last(float v, int G) {
  if (G >= 2) v = dpp_add<0x111, 0xf>(v);
  if (G >= 4) v = dpp_add<0x112, 0xf>(v);
  if (G >= 8) v = dpp_add<0x114, 0xf>(v);
  if (G >= 16) v = dpp_add<0x118, 0xf>(v);
  if (G >= 32) v = dpp_add<0x142, 0xa>(v);
  if (G >= 64) v = dpp_add<0x143, 0xc>(v);
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(group_sum_last(v, 64)), 63));
}

__device__ __forceinline__ uint32_t order_bits(float v) {
  uint32_t u = __float_as_uint(v);
  if (u == 0x80000000u) u = 0;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Softmax top-K of E logits held in LDS (one wave); idx/w land in lanes 0..K-1.
__device__ __forceinline__ void wave_topk(const float* lt, int E, int K, uint32_t flags, int& out_e, float& out_w) {
  const int lane = threadIdx.x % WAVE;
  constexpr int VPL = MOE_MAX_E / WAVE;
  uint64_t key[VPL];
  float val[VPL];
#pragma unroll
  for (int j = 0; j < VPL; ++j) {
    const int e = lane + j * WAVE;
    val[j] = e < E ? lt[e] : 0.f;
    key[j] = e < E ? ((uint64_t)order_bits(val[j]) << 32) | (uint32_t)(0xFFFFFFFFu - (uint32_t)e) : 0ull;
  }
  float top = 0.f, den = 0.f, mine_v = 0.f;
  int mine_e = 0;
  for (int k = 0; k < K; ++k) {
    uint64_t best = 0;
#pragma unroll
    for (int j = 0; j < VPL; ++j) best = key[j] > best ? key[j] : best;
    const uint32_t hi = wave_max_u32((uint32_t)(best >> 32));
    const uint32_t lo = wave_max_u32((uint32_t)(best >> 32) == hi ? (uint32_t)best : 0u);
    const uint64_t t = ((uint64_t)hi << 32) | lo;
#pragma unroll
    for (int j = 0; j < VPL; ++j)
      if (key[j] == t) key[j] = 0;
    const float v = __uint_as_float((hi & 0x80000000u) ? (hi & 0x7FFFFFFFu) : ~hi);
    if (k == 0) top = v;
    if (flags & MOE_TOPK_RENORM) den += expf(v - top);
    if (lane == k) {
      mine_e = (int)(0xFFFFFFFFu - lo);
      mine_v = v;
    }
  }
  if (!(flags & MOE_TOPK_RENORM)) {
    float part = 0.f;
#pragma unroll
    for (int j = 0; j < VPL; ++j)
      if (lane + j * WAVE < E) part += expf(val[j] - top);
    den = wave_sum(part);
  }
  out_e = mine_e;
  out_w = expf(mine_v - top) / den;
}

__device__ __forceinline__ float gelu_erf(float a) { return 0.5f * a * (1.f + erff(a * 0.70710678118654752f)); }

// ------------------------------------------------------------------------------------------
// Per-layer weight loads held in registers between phases.
template <int BITS, int PG, int NSH, int GUM>
struct ABuf {  // gate/up row pairs + head fc1/linear rows (+ their K-hot gather terms)
  uint4 qg[GUM][PG], qu[GUM][PG];
  uint16_t sg[GUM][PG], bg[GUM][PG], su[GUM][PG], bu[GUM][PG];
  bool bad[GUM];
  uint4 hr[NH_MAX][NSH];
  float kh[NH_MAX];
};
template <int BITS, int NSF, int PDM>
struct BBuf {  // down (expert, row group) items + fc2 rows
  uint4 q[PDM];
  uint16_t s[PDM], b[PDM];
  int k[PDM];
  bool bad[PDM];
  uint4 fr[NSF];
};

__device__ __forceinline__ const moe_decode_layer& layer_desc(const StepParams& p, int l) { return p.layers[l]; }

template <int BITS, int PG, int NSH, int GUM>
__device__ __forceinline__ void issue_A(const StepParams& p, int l, const int* re, const int* prev, int gw, int lane,
                        ABuf<BITS, PG, NSH, GUM>& a) {
  const moe_decode_layer& D = layer_desc(p, l);
  const int wpr = p.d * BITS / 32, ngr = p.d >> p.lg2g;
  const int items = p.K * p.I;
#pragma unroll
  for (int u = 0; u < GUM; ++u) {
    const int item = gw * p.GU + u;
    a.bad[u] = false;
    if (u < p.GU && item < items) {
      const int k = item / p.I, i = item - k * p.I;
      int e = re[k];
      a.bad[u] = (unsigned)e >= (unsigned)p.E;
      if (a.bad[u]) e = 0;
      const size_t row = (size_t)e * p.I + i;
#pragma unroll
      for (int q = 0; q < PG; ++q) {
        const int seg = lane + q * WAVE;
        const size_t wo = row * wpr + (size_t)seg * 4;
        a.qg[u][q] = *reinterpret_cast<const uint4*>(D.experts.gate.q + wo);
        a.qu[u][q] = *reinterpret_cast<const uint4*>(D.experts.up.q + wo);
        const size_t go = row * ngr + ((seg * SegT<BITS>::COLS) >> p.lg2g);
        a.sg[u][q] = D.experts.gate.scales[go];
        a.bg[u][q] = D.experts.gate.biases[go];
        a.su[u][q] = D.experts.up.scales[go];
        a.bu[u][q] = D.experts.up.biases[go];
      }
    }
  }
  const bool head = l + 1 < p.L && D.head.fc1_x != nullptr;
#pragma unroll
  for (int r = 0; r < NH_MAX; ++r) {
    a.kh[r] = 0.f;
    const int row = gw * p.NH + r;
    if (head && r < p.NH && row < p.H + p.E) {
      const bool fc1 = row < p.H;
      const int c = fc1 ? row : row - p.H;
      const uint16_t* W = fc1 ? D.head.fc1_x + (size_t)c * p.d : D.head.lin_x + (size_t)c * p.d;
#pragma unroll
      for (int s = 0; s < NSH; ++s) a.hr[r][s] = *reinterpret_cast<const uint4*>(W + (size_t)(lane + s * WAVE) * 8);
      const uint16_t* rtab = fc1 ? D.head.fc1_r : D.head.lin_r;
      const int ncol = fc1 ? p.H : p.E;
      if (lane < p.K) {
        const int e = re[lane];
        a.kh[r] = (unsigned)e < (unsigned)p.E ? h2f(rtab[(size_t)e * ncol + c]) : quiet_nan();
      } else if (prev && lane < 2 * p.K) {
        const int e = prev[lane - p.K];
        a.kh[r] = (unsigned)e < (unsigned)p.E ? h2f(rtab[(size_t)(p.E + e) * ncol + c]) : quiet_nan();
      }
    }
  }
}

template <int BITS, int NSF, int PDM>
__device__ __forceinline__ void issue_B(const StepParams& p, int l, const int* re, int wg, int cw, int lane,
                        BBuf<BITS, NSF, PDM>& b) {
  const moe_decode_layer& D = layer_desc(p, l);
  const int wpr = p.I * BITS / 32, ngr = p.I >> p.lg2g;
  const int RPI = WAVE / p.Ldn, slot = lane / p.Ldn, ls = lane % p.Ldn;
  const int S = p.I * BITS / 128;
  const int npairs = p.K * p.DI;
#pragma unroll
  for (int u = 0; u < PDM; ++u) {
    const int pk = cw + u * MW;
    b.k[u] = 0;
    b.bad[u] = false;
    if (u < p.PD && pk < npairs) {
      const int k = pk / p.DI, q = pk - k * p.DI;
      int e = re[k];
      b.bad[u] = (unsigned)e >= (unsigned)p.E;
      if (b.bad[u]) e = 0;
      b.k[u] = k;
      int j = wg * p.DR + q * RPI + slot;
      if (j >= p.d) j = p.d - 1;
      const size_t row = (size_t)e * p.d + j;
      if (ls < S) {
        b.q[u] = *reinterpret_cast<const uint4*>(D.experts.down.q + row * wpr + (size_t)ls * 4);
        const size_t go = row * ngr + ((ls * SegT<BITS>::COLS) >> p.lg2g);
        b.s[u] = D.experts.down.scales[go];
        b.b[u] = D.experts.down.biases[go];
      }
    }
  }
  const bool head = l + 1 < p.L && D.head.fc1_x != nullptr;
  const int row = wg * MW + cw;  // one fc2 row per compute wave (NO == 1)
  if (head && row < p.E) {
#pragma unroll
    for (int s = 0; s < NSF; ++s)
      b.fr[s] = *reinterpret_cast<const uint4*>(D.head.fc2 + (size_t)row * p.H + (size_t)(lane + s * WAVE) * 8);
  }
}

struct StepShared {
  uint16_t h[2][LDS_D];
  float act[LDS_ACT];
  float g[LDS_H];
  float lin[LDS_E];
  float logit[LDS_E];
  float part[LDS_PART];
  float scale[2];
  int route_e[LDS_LK];  // this token's routing of every layer: [l * K + k]
  float route_w[LDS_LK];
  int prev_e[LDS_LK];   // the previous token's routing (K-hot "previous" input of the heads)
};

struct StepCtx {
  int wg, lane, cw, gw;
  uint32_t epoch;
  int32_t *cur_i, *nxt_i;
  float *cur_w, *nxt_w;
  const int32_t* prev_i;
  __device__ uint32_t tag(int ph) const { return ((epoch << 10) | (uint32_t)ph) ^ TAG_SALT; }
};

__device__ __forceinline__ bool self_routed(const StepParams& p, int l) {
  return p.bootstrap || l == 0 || p.layers[l - 1].head.fc1_x == nullptr;
}
__device__ __forceinline__ bool has_head(const StepParams& p, int l) {
  return l + 1 < p.L && p.layers[l].head.fc1_x != nullptr;
}

// Wave 0 of every workgroup: waits for the vectors each phase needs and unpacks them into LDS.
__device__ __forceinline__ void sync_role(const StepParams& p, const StepCtx& c, StepShared& sm) {
  const int lane = c.lane, dh = p.d / 2;
  bool failed = false;
  for (int l = 0; l < p.L; ++l) {
    const int hb = l & 1;
    uint32_t* hw = reinterpret_cast<uint32_t*>(sm.h[hb]);
    if (l == 0) {
      for (int m = lane; m < dh; m += WAVE) hw[m] = reinterpret_cast<const uint32_t*>(p.h_in)[m];
    } else {
      ll_wait(p.ll_h + (size_t)l * dh, dh, c.tag(3 * (l - 1) + 2), p.err, failed, [&](int i, uint32_t v) { hw[i] = v; });
    }
    float sq = 0.f;
    for (int m = lane; m < dh; m += WAVE) {
      const half2_t v = as_h2(hw[m]);
      sq = __builtin_amdgcn_fdot2(v, v, sq, false);
    }
    sq = wave_sum(sq);
    if (lane == 0) sm.scale[hb] = 1.f / sqrtf(sq / (float)p.d + RMS_EPS);
    lds_barrier();  // B1: h_l ready
    if (self_routed(p, l)) {
      ll_wait(p.ll_logits, p.E, c.tag(3 * l), p.err, failed, [&](int i, uint32_t v) { sm.logit[i] = __uint_as_float(v); });
      int e;
      float w;
      wave_topk(sm.logit, p.E, p.K, p.topk_flags, e, w);
      if (lane < p.K) {
        sm.route_e[l * p.K + lane] = e;
        sm.route_w[l * p.K + lane] = w;
        if (c.wg == 0) {
          c.cur_i[l * p.K + lane] = e;
          c.cur_w[l * p.K + lane] = w;
        }
      }
      lds_barrier();  // B2: routing of layer l ready
    }
    const uint32_t tA = c.tag(3 * l + 1);
    ll_wait(p.ll_act, p.K * p.I, tA, p.err, failed, [&](int i, uint32_t v) { sm.act[i] = __uint_as_float(v); });
    if (has_head(p, l)) {
      ll_wait(p.ll_g, p.H, tA, p.err, failed, [&](int i, uint32_t v) { sm.g[i] = __uint_as_float(v); });
      ll_wait(p.ll_lin, p.E, tA, p.err, failed, [&](int i, uint32_t v) { sm.lin[i] = __uint_as_float(v); });
    }
    lds_barrier();  // B3: act (and head fc1 / linear outputs) ready
    lds_barrier();  // B4: partial down sums ready (the combine runs in wave 1)
  }
  // Top-K of every head, off the token's critical path: head l predicts layer l+1's routing for
  // the next token; workgroup l % G handles head l.
  for (int l = c.wg; l + 1 < p.L; l += p.G) {
    if (!has_head(p, l)) continue;
    ll_wait(p.ll_hlog + (size_t)l * p.E, p.E, c.tag(3 * l + 2), p.err, failed,
            [&](int i, uint32_t v) { sm.logit[i] = __uint_as_float(v); });
    int e;
    float w;
    wave_topk(sm.logit, p.E, p.K, p.topk_flags, e, w);
    if (lane < p.K) {
      c.nxt_i[(l + 1) * p.K + lane] = e;
      c.nxt_w[(l + 1) * p.K + lane] = w;
    }
  }
}

// Waves 1..MW: the arithmetic, with each phase's weight loads issued one phase early.
template <int BITS, int PG, int NSH, int NSF, int GUM, int PDM>
__device__ __forceinline__ void compute_role(const StepParams& p, const StepCtx& c, StepShared& sm) {
  using GS = SegT<BITS>;
  const int lane = c.lane, cw = c.cw, gw = c.gw, wg = c.wg, dh = p.d / 2;
  ABuf<BITS, PG, NSH, GUM> A;
  BBuf<BITS, NSF, PDM> B;
  for (int l = 0; l < p.L; ++l) {
    const moe_decode_layer& D = p.layers[l];
    const bool self = self_routed(p, l);
    const bool head = has_head(p, l);
    const int hb = l & 1;
    const int* prev_l = c.prev_i ? sm.prev_e + l * p.K : nullptr;
    lds_barrier();  // B1
    const float scale = sm.scale[hb];
    const uint16_t* hl = sm.h[hb];
    if (self) {
      // R_l: this wave's router rows -> tagged logits
      for (int r = gw * p.NR; r < min(p.E, gw * p.NR + p.NR); ++r) {
        const uint16_t* W = D.router + (size_t)r * p.d;
        float acc = 0.f;
#pragma unroll
        for (int sg = 0; sg < NSH; ++sg) {
          const int g = lane + sg * WAVE;
          const uint4 wv = *reinterpret_cast<const uint4*>(W + (size_t)g * 8);
          const uint4 xv = *reinterpret_cast<const uint4*>(hl + (size_t)g * 8);
          acc = __builtin_amdgcn_fdot2(as_h2(wv.x), as_h2(xv.x), acc, false);
          acc = __builtin_amdgcn_fdot2(as_h2(wv.y), as_h2(xv.y), acc, false);
          acc = __builtin_amdgcn_fdot2(as_h2(wv.z), as_h2(xv.z), acc, false);
          acc = __builtin_amdgcn_fdot2(as_h2(wv.w), as_h2(xv.w), acc, false);
        }
        acc = wave_sum(acc) * scale;
        if (lane == 0) ll_store(p.ll_logits + r, __float_as_uint(acc), c.tag(3 * l));
      }
      lds_barrier();  // B2
      issue_A<BITS, PG, NSH, GUM>(p, l, sm.route_e + l * p.K, prev_l, gw, lane, A);
      issue_B<BITS, NSF, PDM>(p, l, sm.route_e + l * p.K, wg, cw, lane, B);
    }

    // ---- A_l: gate/up + SwiGLU, head fc1 (+GELU) and linear rows ----
    {
      const uint32_t tA = c.tag(3 * l + 1);
      uint32_t xp[PG][GS::PAIRS];
      float sx[PG][2], sq = 0.f;
#pragma unroll
      for (int q = 0; q < PG; ++q) load_xpairs<BITS>(hl + (size_t)(lane + q * WAVE) * GS::COLS, xp[q], sx[q], sq);
#pragma unroll
      for (int u = 0; u < GUM; ++u) {
        const int item = gw * p.GU + u;
        if (u < p.GU && item < p.K * p.I) {
          float pg = 0.f, pu = 0.f;
#pragma unroll
          for (int q = 0; q < PG; ++q) {
            float d0 = 0.f, d1 = 0.f;
            dot_segment<BITS>(A.qg[u][q], xp[q], d0, d1);
            pg += h2f(A.sg[u][q]) * (d0 + d1) + h2f(A.bg[u][q]) * (sx[q][0] + sx[q][1]);
            d0 = d1 = 0.f;
            dot_segment<BITS>(A.qu[u][q], xp[q], d0, d1);
            pu += h2f(A.su[u][q]) * (d0 + d1) + h2f(A.bu[u][q]) * (sx[q][0] + sx[q][1]);
          }
          pg = wave_sum(pg) * scale;
          pu = wave_sum(pu) * scale;
          float a = pg / (1.f + expf(-pg)) * pu;
          if (A.bad[u]) a = quiet_nan();
          if (lane == 0) ll_store(p.ll_act + item, __float_as_uint(a), tA);
        }
      }
      if (head) {
#pragma unroll
        for (int r = 0; r < NH_MAX; ++r) {
          const int row = gw * p.NH + r;
          if (r < p.NH && row < p.H + p.E) {
            float acc = 0.f;
#pragma unroll
            for (int sg = 0; sg < NSH; ++sg) {
              const uint4 xv = *reinterpret_cast<const uint4*>(hl + (size_t)(lane + sg * WAVE) * 8);
              acc = __builtin_amdgcn_fdot2(as_h2(A.hr[r][sg].x), as_h2(xv.x), acc, false);
              acc = __builtin_amdgcn_fdot2(as_h2(A.hr[r][sg].y), as_h2(xv.y), acc, false);
              acc = __builtin_amdgcn_fdot2(as_h2(A.hr[r][sg].z), as_h2(xv.z), acc, false);
              acc = __builtin_amdgcn_fdot2(as_h2(A.hr[r][sg].w), as_h2(xv.w), acc, false);
            }
            acc = wave_sum(acc) * scale;
            const float gsum = wave_sum(A.kh[r]);
            if (lane == 0) {
              if (row < p.H) {
                const float v = acc + gsum + (D.head.fc1_b ? h2f(D.head.fc1_b[row]) : 0.f);
                ll_store(p.ll_g + row, __float_as_uint(gelu_erf(v)), tA);
              } else {
                const int col = row - p.H;
                const float v = acc + gsum + (D.head.lin_b ? h2f(D.head.lin_b[col]) : 0.f);
                ll_store(p.ll_lin + col, __float_as_uint(v), tA);
              }
            }
          }
        }
      }
    }
    if (l + 1 < p.L && !self_routed(p, l + 1))  // weights of A_{l+1}, one phase early
      issue_A<BITS, PG, NSH, GUM>(p, l + 1, sm.route_e + (l + 1) * p.K,
                                  c.prev_i ? sm.prev_e + (l + 1) * p.K : nullptr, gw, lane, A);
    lds_barrier();  // B3

    // ---- B_l: down partials of this workgroup's rows, head fc2 rows ----
    {
      const int RPI = WAVE / p.Ldn, slot = lane / p.Ldn, ls = lane % p.Ldn;
      const int S = p.I * BITS / 128;
#pragma unroll
      for (int u = 0; u < PDM; ++u) {
        const int pk = cw + u * MW;
        if (u < p.PD && pk < p.K * p.DI) {
          const int k = B.k[u], q = pk - k * p.DI;
          float po = 0.f;
          if (ls < S) {
            uint32_t xh[GS::PAIRS], xl[GS::PAIRS];
            float sx[2];
            load_xpairs_f32<BITS>(sm.act + (size_t)k * p.I + (size_t)ls * GS::COLS, xh, xl, sx);
            float d0 = 0.f, d1 = 0.f;
            dot_segment_split<BITS>(B.q[u], xh, xl, d0, d1);
            po = h2f(B.s[u]) * (d0 + d1) + h2f(B.b[u]) * (sx[0] + sx[1]);
          }
          po = group_sum_last(po, p.Ldn);
          if (ls == p.Ldn - 1) sm.part[k * p.DR + q * RPI + slot] = B.bad[u] ? quiet_nan() : po;
        }
      }
      if (head) {
        const int row = wg * MW + cw;
        if (row < p.E) {
          float acc = 0.f;
#pragma unroll
          for (int sg = 0; sg < NSF; ++sg) {
            const float* gp = sm.g + (size_t)(lane + sg * WAVE) * 8;
            const half2_t w0 = as_h2(B.fr[sg].x), w1 = as_h2(B.fr[sg].y), w2 = as_h2(B.fr[sg].z),
                          w3 = as_h2(B.fr[sg].w);
            acc = fmaf((float)w0.x, gp[0], acc);
            acc = fmaf((float)w0.y, gp[1], acc);
            acc = fmaf((float)w1.x, gp[2], acc);
            acc = fmaf((float)w1.y, gp[3], acc);
            acc = fmaf((float)w2.x, gp[4], acc);
            acc = fmaf((float)w2.y, gp[5], acc);
            acc = fmaf((float)w3.x, gp[6], acc);
            acc = fmaf((float)w3.y, gp[7], acc);
          }
          acc = wave_sum(acc);
          if (lane == 0) {
            const float v = acc + sm.lin[row] + (D.head.fc2_b ? h2f(D.head.fc2_b[row]) : 0.f);
            ll_store(p.ll_hlog + (size_t)l * p.E + row, __float_as_uint(v), c.tag(3 * l + 2));
          }
        }
      }
    }
    if (l + 1 < p.L && !self_routed(p, l + 1))  // weights of B_{l+1}, one phase early
      issue_B<BITS, NSF, PDM>(p, l + 1, sm.route_e + (l + 1) * p.K, wg, cw, lane, B);
    lds_barrier();  // B4
    // ---- combine + residual of this workgroup's rows -> h_{l+1} ----
    if (cw == 0) {
      const int jr = lane, j = wg * p.DR + jr;
      float y = 0.f;
      if (jr < p.DR && j < p.d) {
        float acc = 0.f;
        for (int k = 0; k < p.K; ++k) acc = fmaf(sm.route_w[l * p.K + k], sm.part[k * p.DR + jr], acc);
        y = h2f(hl[j]) + acc;
      }
      const uint32_t yb = f2h(y);
      const uint32_t nb = __shfl_down(yb, 1, WAVE);
      if (jr < p.DR && j < p.d) {
        if (l + 1 == p.L)
          p.h_out[j] = (uint16_t)yb;
        else if ((jr & 1) == 0)
          ll_store(p.ll_h + (size_t)(l + 1) * dh + j / 2, yb | (nb << 16), c.tag(3 * l + 2));
      }
    }
  }
}

template <int BITS, int PG, int NSH, int NSF, int GUM, int PDM>
__global__ void __launch_bounds__(NTHREADS) k_decode_step(StepParams p) {
  __shared__ __attribute__((aligned(16))) StepShared sm;
  StepCtx c;
  c.wg = blockIdx.x;
  c.lane = threadIdx.x % WAVE;
  const int wave = threadIdx.x / WAVE;
  c.cw = wave - 1;
  c.gw = c.wg * MW + c.cw;
  c.epoch = *p.epoch;
  const int LK = p.L * p.K;
  c.cur_i = p.ridx + (size_t)p.slot * LK;
  c.cur_w = p.rw + (size_t)p.slot * LK;
  c.prev_i = p.bootstrap ? nullptr : p.ridx + (size_t)((p.slot + 2) % 3) * LK;
  c.nxt_i = p.ridx + (size_t)((p.slot + 1) % 3) * LK;
  c.nxt_w = p.rw + (size_t)((p.slot + 1) % 3) * LK;
  if (wave > 0) {  // routing state of the whole token into LDS (read before the first barrier's use)
    for (int i = threadIdx.x - WAVE; i < LK; i += MW * WAVE) {
      sm.route_e[i] = c.cur_i[i];
      sm.route_w[i] = c.cur_w[i];
      sm.prev_e[i] = c.prev_i ? c.prev_i[i] : 0;
    }
  }
  if (wave == 0)
    sync_role(p, c, sm);
  else
    compute_role<BITS, PG, NSH, NSF, GUM, PDM>(p, c, sm);
  if (c.wg == 0 && threadIdx.x == 0) *p.epoch = c.epoch + 1;
}

}  // namespace

// ------------------------------------------------------------------------------------------ host
struct StepPlan {
  bool ok;
  int G, GU, NH, NR, NO, DR, DI, PD, Ldn, PG, NSH, NSF;
};

static StepPlan plan_step(const moe_decode_stack& st, int G) {
  StepPlan pl{};
  const int d = st.d_model, I = st.d_ff, E = st.E, K = st.K, H = st.d_hidden, bits = st.bits;
  const int GW = G * MW;
  if (G < 1 || d % 512 || d > LDS_D || (d * bits / 128) % WAVE) return pl;
  pl.PG = d * bits / 128 / WAVE;
  pl.NSH = d / 512;
  if (pl.PG > 2 || (pl.NSH != 4 && pl.NSH != 8)) return pl;
  const int SI = I * bits / 128;
  if (SI < 1 || SI > WAVE || (I * bits) % 128) return pl;
  if (bits == 2 && st.group < 64) return pl;  // a 2-bit segment must sit inside one group
  pl.Ldn = 1;
  while (pl.Ldn < SI) pl.Ldn <<= 1;
  const int RPI = WAVE / pl.Ldn;
  if (K > 8 || K * I > LDS_ACT || E > LDS_E || st.L * K > LDS_LK) return pl;
  pl.GU = (K * I + GW - 1) / GW;
  if (pl.GU > GU_MAX) return pl;
  pl.NR = (E + GW - 1) / GW;
  if (pl.NR > 1) return pl;
  pl.NO = 1;
  if (E > GW) return pl;
  pl.DR = (d + G - 1) / G;
  pl.DR = (pl.DR + RPI - 1) / RPI * RPI;
  pl.DR += pl.DR & 1;
  if (pl.DR > WAVE || K * pl.DR > LDS_PART) return pl;
  pl.DI = (pl.DR + RPI - 1) / RPI;
  pl.PD = (K * pl.DI + MW - 1) / MW;
  if (pl.PD > PD_MAX) return pl;
  if (H > 0) {
    if (H % 512 || H > LDS_H) return pl;
    pl.NSF = H / 512;
    if (pl.NSF != 1 && pl.NSF != 2 && pl.NSF != 4) return pl;
    pl.NH = (H + E + GW - 1) / GW;
    if (pl.NH > NH_MAX) return pl;
  } else {
    pl.NSF = 1;
    pl.NH = 0;
  }
  pl.G = G;
  pl.ok = true;
  return pl;
}

struct StepWs {
  size_t epoch, err, logits, act, g, lin, hlog, h, total;
};
static StepWs step_ws(const moe_decode_stack& st) {
  auto al = [](size_t v) { return (v + 255) / 256 * 256; };
  StepWs w{};
  w.epoch = 0;
  w.err = 4;
  w.logits = 256;
  w.act = w.logits + al((size_t)st.E * 8);
  w.g = w.act + al((size_t)st.K * st.d_ff * 8);
  w.lin = w.g + al((size_t)(st.d_hidden > 0 ? st.d_hidden : 1) * 8);
  w.hlog = w.lin + al((size_t)st.E * 8);
  w.h = w.hlog + al((size_t)st.L * st.E * 8);
  w.total = w.h + al((size_t)(st.L + 1) * (st.d_model / 2) * 8);
  return w;
}

static int device_cus() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  return cus;
}

template <int BITS, int PG, int NSH, int NSF, int GUM, int PDM>
static hipError_t go(hipStream_t s, const StepParams& p) {
  int occ = 0;
  auto k = k_decode_step<BITS, PG, NSH, NSF, GUM, PDM>;
  hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, k, NTHREADS, 0);
  if (e != hipSuccess) return e;
  if (occ < 1) return hipErrorInvalidConfiguration;  // every workgroup must be resident at once
  return launch(k, dim3(p.G), dim3(NTHREADS), 0, s, p);
}

// Instantiated shapes (bits, gate/up segments per lane, fp16 segments per lane for d and H,
// gate/up pairs and down items per wave): the decode configurations, then general fallbacks.
static hipError_t dispatch(hipStream_t s, const StepParams& p, int bits, int PG, int NSH, int NSF) {
  const int gum = p.GU <= 2 ? 2 : 4, pdm = p.PD <= 2 ? 2 : (p.PD <= 4 ? 4 : 8);
#define MOE_STEP_CASE(B_, PG_, NSH_, NSF_, GUM_, PDM_)                                                  \
  if (bits == B_ && PG == PG_ && NSH == NSH_ && NSF <= NSF_ && gum <= GUM_ && pdm <= PDM_)           \
    return go<B_, PG_, NSH_, NSF_, GUM_, PDM_>(s, p);
  MOE_STEP_CASE(4, 1, 4, 2, 2, 2)   // d 2048, I 512, K 4, H 1024
  MOE_STEP_CASE(4, 1, 4, 2, 4, 4)   // d 2048, I 512, K 8
  MOE_STEP_CASE(4, 2, 8, 1, 4, 8)   // d 4096, I 1024, int4
  MOE_STEP_CASE(2, 1, 8, 1, 4, 4)   // d 4096, I 1024, int2
  MOE_STEP_CASE(4, 1, 4, 4, 4, 8)
  MOE_STEP_CASE(4, 2, 8, 4, 4, 8)
  MOE_STEP_CASE(2, 1, 8, 4, 4, 8)
  MOE_STEP_CASE(2, 2, 8, 4, 4, 8)
#undef MOE_STEP_CASE
  return hipErrorInvalidValue;
}

bool decode_step_supported(const moe_decode_stack& st) { return plan_step(st, 256).ok; }

size_t decode_step_workspace(const moe_decode_stack& st) { return step_ws(st).total; }

hipError_t launch_decode_step(hipStream_t s, const moe_decode_stack& st, int token, uint32_t flags,
                              const uint16_t* h_in, uint16_t* h_out, void* ws) {
  const int G = device_cus();
  const StepPlan pl = plan_step(st, G);
  if (!pl.ok) return hipErrorInvalidValue;
  const StepWs w = step_ws(st);
  char* b = (char*)ws;
  StepParams p{};
  p.L = st.L;
  p.E = st.E;
  p.K = st.K;
  p.d = st.d_model;
  p.I = st.d_ff;
  p.H = st.d_hidden;
  int lg = 0;
  while ((1 << lg) < st.group) ++lg;
  p.lg2g = lg;
  p.G = pl.G;
  p.GU = pl.GU;
  p.NH = pl.NH;
  p.NR = pl.NR;
  p.NO = pl.NO;
  p.DR = pl.DR;
  p.DI = pl.DI;
  p.PD = pl.PD;
  p.Ldn = pl.Ldn;
  p.layers = st.layers;
  p.h_in = h_in;
  p.h_out = h_out;
  p.ridx = st.route_idx;
  p.rw = st.route_w;
  p.slot = token % 3;
  p.bootstrap = token == 0;
  p.topk_flags = flags & MOE_TOPK_RENORM;
  p.ll_logits = (uint64_t*)(b + w.logits);
  p.ll_act = (uint64_t*)(b + w.act);
  p.ll_g = (uint64_t*)(b + w.g);
  p.ll_lin = (uint64_t*)(b + w.lin);
  p.ll_hlog = (uint64_t*)(b + w.hlog);
  p.ll_h = (uint64_t*)(b + w.h);
  p.epoch = (uint32_t*)(b + w.epoch);
  p.err = (int*)(b + w.err);
  return dispatch(s, p, st.bits, pl.PG, pl.NSH, pl.NSF);
}

}  // namespace moe
