// Routing on gfx950: float16 router / prerouter-head matvecs and the wave64 softmax top-K.
//
// Router logits and top-K: each token goes to the K experts with the largest router logits
// ("Arquitecturas nativas para device: MoE de grano fino y pre-attention router", section "Dos
// niveles de sparsity").  Prerouter head: head(z) = fc2(gelu_erf(fc1 z)) + l(z) over
// z = [x; K-hot of this layer's routing at t; K-hot at t-1], length d + 2E ("La otra mitad del
// muro de la memoria: Servir MoEs de 35B desde SSD ...", section "Arquitectura del cabezal
// Prerouter", both equations).  The K-hot columns of fc1 and l are stored as rows (split
// layout), so the head reads only the 2K selected rows instead of 2E dense columns.
//
// Matvecs: one wave per output row; the row is held in registers as 128-bit segments and reused
// across the wave's tokens; products of float16 pairs are exact in float32 (v_dot2_f32_f16).
// The RMS-norm option scales the finished dot product (linearity), so x is never rounded.
//
// Top-K: one wave per token, up to 16 logits per lane.  A logit becomes a 64-bit key
// (order-preserving bits of the float, then the complemented expert index), so one unsigned
// max picks the largest logit and, among equal logits, the lowest index.  K rounds of a
// wave-wide max pick the experts in order.
#include <math.h>

#include "moe_device.h"
#include "moe_launch.h"

namespace moe {
namespace {

// Dot products of one float16 row (held in registers) with TPW tokens' float16 activations.
template <int NSEG>
__device__ __forceinline__ void row_dot_tokens(const uint4* wr, int nseg, const uint16_t* __restrict__ x,
                                               int d, int t, int lane, float& acc, float& sq) {
  acc = 0.f;
  sq = 0.f;
  const uint16_t* xt = x + (size_t)t * d;
#pragma unroll
  for (int p = 0; p < NSEG; ++p) {
    const int sgi = lane + p * WAVE;
    if (sgi < nseg) {
      const uint4 xv = *reinterpret_cast<const uint4*>(xt + (size_t)sgi * 8);
      const uint32_t xa[4] = {xv.x, xv.y, xv.z, xv.w};
      const uint32_t wa[4] = {wr[p].x, wr[p].y, wr[p].z, wr[p].w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc = __builtin_amdgcn_fdot2(as_h2(wa[i]), as_h2(xa[i]), acc, false);
        sq = __builtin_amdgcn_fdot2(as_h2(xa[i]), as_h2(xa[i]), sq, false);
      }
    }
  }
  acc = group_sum(acc, WAVE);
  sq = group_sum(sq, WAVE);
}

template <int NSEG>
__device__ __forceinline__ void load_row(uint4* wr, const uint16_t* __restrict__ row, int nseg, int lane) {
#pragma unroll
  for (int p = 0; p < NSEG; ++p) {
    const int sgi = lane + p * WAVE;
    wr[p] = sgi < nseg ? *reinterpret_cast<const uint4*>(row + (size_t)sgi * 8) : make_uint4(0, 0, 0, 0);
  }
}

// logits[t][e] = s_t * W[e] . x_t ; grid (E, ceil(T / tpw)), one wave per block.
template <int NSEG>
__global__ void __launch_bounds__(64) k_router(int T, int d, int E, uint32_t flags, int tpw,
                                               const uint16_t* __restrict__ x,
                                               const uint16_t* __restrict__ W, float* __restrict__ logits) {
  const int e = blockIdx.x, lane = threadIdx.x;
  const int nseg = d / 8;
  uint4 wr[NSEG];
  load_row<NSEG>(wr, W + (size_t)e * d, nseg, lane);
  const int t1 = min(T, (int)(blockIdx.y + 1) * tpw);
  for (int t = blockIdx.y * tpw; t < t1; ++t) {
    float acc, sq;
    row_dot_tokens<NSEG>(wr, nseg, x, d, t, lane, acc, sq);
    const float s = (flags & MOE_INPUT_RMSNORM) ? 1.f / sqrtf(sq / (float)d + RMS_EPS) : 1.f;
    if (lane == 0) logits[(size_t)t * E + e] = acc * s;
  }
}

// The same logits for many tokens at once, on the matrix cores: logits = X W^T with X [T][d] and
// W [E][d] both K-contiguous.  A block computes one 16-token x 16-expert tile; its waves split the
// d columns (at most RK each) and each wave issues all of its loads at once, straight from memory
// (both operands stay in L2), before its MFMAs (gfx950's v_mfma_f32_16x16x32_f16; D lane (n, q)
// holds rows 4q..4q+3 of column n).  A lane reads 8 consecutive halves of its row per load and
// feeds them to one MFMA step; X and W use the same column order, which is all a dot product needs.  With
// MOE_INPUT_RMSNORM each token's sum of squares comes from the same X reads.  The partial tiles
// meet in LDS.  Needs T and E multiples of 16, d of 32 and 16-byte aligned rows (the host checks).
constexpr int R_MAXW = 16;  // waves per block at most

// RK: columns per wave (RK / 32 16-byte loads per lane and operand)
template <int RK>
__global__ void __launch_bounds__(R_MAXW * WAVE) k_router_mfma(int T, int d, int E, uint32_t flags,
                                                               const uint16_t* __restrict__ x,
                                                               const uint16_t* __restrict__ W,
                                                               float* __restrict__ logits) {
  constexpr int RK_LOADS = RK / 32;
  __shared__ float part[R_MAXW][WAVE][5];
  const int lane = threadIdx.x % WAVE, wave = threadIdx.x / WAVE, nw = blockDim.x / WAVE;
  const int m = lane % 16, q = lane / 16;
  const int t0 = blockIdx.x * 16, e0 = blockIdx.y * 16;
  const int c0 = wave * RK;
  const uint16_t* xr = x + (size_t)(t0 + m) * d + 8 * q;
  const uint16_t* wr = W + (size_t)(e0 + m) * d + 8 * q;
  uint4 a[RK_LOADS], b[RK_LOADS];
#pragma unroll
  for (int i = 0; i < RK_LOADS; ++i) {
    const int c = min(c0 + 32 * i, d - 32);  // clamped: every load valid, extra ones ignored below
    a[i] = *reinterpret_cast<const uint4*>(xr + c);
    b[i] = *reinterpret_cast<const uint4*>(wr + c);
  }
  __builtin_amdgcn_sched_barrier(0);  // keep every load ahead of the arithmetic: one memory latency in all
  float4_t acc = {0.f, 0.f, 0.f, 0.f};
  float sq = 0.f;
#pragma unroll
  for (int i = 0; i < RK_LOADS; ++i) {
    if (c0 + 32 * i >= d) break;  // uniform
    const half8_t a8 = __builtin_bit_cast(half8_t, a[i]);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(a8, __builtin_bit_cast(half8_t, b[i]), acc, 0, 0, 0);
#pragma unroll
    for (int j = 0; j < 4; ++j) sq = fmaf((float)a8[j], (float)a8[j], fmaf((float)a8[4 + j], (float)a8[4 + j], sq));
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) part[wave][lane][i] = acc[i];
  part[wave][lane][4] = sq;
  __syncthreads();
  if (wave != 0) return;
  for (int w = 1; w < nw; ++w) {
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i] += part[w][lane][i];
    sq += part[w][lane][4];
  }
  float s[4] = {1.f, 1.f, 1.f, 1.f};
  if (flags & MOE_INPUT_RMSNORM) {
    sq += __shfl_xor(sq, 16);
    sq += __shfl_xor(sq, 32);  // every lane of row m now holds the row's sum of squares
#pragma unroll
    for (int i = 0; i < 4; ++i) s[i] = 1.f / sqrtf(__shfl(sq, 4 * q + i) / (float)d + RMS_EPS);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) logits[(size_t)(t0 + 4 * q + i) * E + e0 + m] = acc[i] * s[i];
}

__device__ __forceinline__ uint32_t order_bits(float v) {
  uint32_t u = __float_as_uint(v);
  if (u == 0x80000000u) u = 0;  // -0 ranks as +0 (equal logits tie to the lower index)
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float from_order_bits(uint32_t o) {
  return __uint_as_float((o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o);
}

// TOPK_VPL logits per lane: the smallest power of two with 64 * TOPK_VPL >= E (up to MOE_MAX_E / 64),
// so a small E does not pay for the largest one's registers and compare rounds.
template <int TOPK_VPL>
__global__ void __launch_bounds__(64) k_topk(int T, int E, int K, uint32_t flags,
                                             const float* __restrict__ logits, int32_t* __restrict__ idx,
                                             float* __restrict__ w) {
  const int t = blockIdx.x, lane = threadIdx.x;
  const float* lt = logits + (size_t)t * E;
  uint64_t key[TOPK_VPL];
  float val[TOPK_VPL];
#pragma unroll
  for (int j = 0; j < TOPK_VPL; ++j) {
    const int e = lane + j * WAVE;
    val[j] = e < E ? lt[e] : 0.f;
    key[j] = e < E ? ((uint64_t)order_bits(val[j]) << 32) | (uint32_t)(0xFFFFFFFFu - (uint32_t)e) : 0ull;
  }
  int sel_e[MOE_MAX_K];
  float sel_v[MOE_MAX_K];
#pragma unroll
  for (int k = 0; k < MOE_MAX_K; ++k) {
    sel_e[k] = 0;
    sel_v[k] = 0.f;
    if (k < K) {
      uint64_t best = 0;
#pragma unroll
      for (int j = 0; j < TOPK_VPL; ++j) best = key[j] > best ? key[j] : best;
      // wave max of the 64-bit keys: largest order bits first, then among those lanes the
      // largest complemented index (= the lowest expert index)
      const uint32_t hi = wave_max_u32((uint32_t)(best >> 32));
      const uint32_t lo = wave_max_u32((uint32_t)(best >> 32) == hi ? (uint32_t)best : 0u);
      const uint64_t top = ((uint64_t)hi << 32) | lo;
#pragma unroll
      for (int j = 0; j < TOPK_VPL; ++j)
        if (key[j] == top) key[j] = 0;
      sel_e[k] = (int)(0xFFFFFFFFu - lo);
      sel_v[k] = from_order_bits(hi);
    }
  }
  // softmax weights, float32
  float den = 0.f;
  if (flags & MOE_TOPK_RENORM) {
#pragma unroll
    for (int k = 0; k < MOE_MAX_K; ++k)
      if (k < K) den += expf(sel_v[k] - sel_v[0]);
  } else {
    float part = 0.f;
#pragma unroll
    for (int j = 0; j < TOPK_VPL; ++j)
      if (lane + j * WAVE < E) part += expf(val[j] - sel_v[0]);
    den = group_sum(part, WAVE);
  }
  if (lane < K) {
    float v = 0.f;
    int e = 0;
#pragma unroll
    for (int k = 0; k < MOE_MAX_K; ++k)
      if (k == lane) {
        v = sel_v[k];
        e = sel_e[k];
      }
    idx[(size_t)t * K + lane] = e;
    w[(size_t)t * K + lane] = expf(v - sel_v[0]) / den;
  }
}

// ----------------------------------------------------------------------------------------------
// prerouter head
struct HeadArgs {
  int T, d, E, K, H;
  uint32_t flags;
  const uint16_t* x;
  const int32_t* cur;
  const int32_t* prev;
  moe_prerouter_w pw;
  float* g;    // [T][H] gelu(fc1 z + b1)
  float* lin;  // [T][E] l z + b_l
};

__device__ __forceinline__ float gelu_erf(float a) { return 0.5f * a * (1.f + erff(a * 0.70710678118654752f)); }

// One term of the K-hot gather, spread over lanes: lane j < K reads row cur[j] of `rtab`
// ([2E][ncol] float16), lane K <= j < 2K reads row E + prev[j - K]; other lanes give 0.  A row
// index outside [0, E) yields NaN.
__device__ __forceinline__ float khot_term(const uint16_t* __restrict__ rtab, int ncol, int c, int E, int K,
                                           const int32_t* cur, const int32_t* prev, int lane) {
  if (lane >= 2 * K || (lane >= K && !prev)) return 0.f;
  const int e = lane < K ? cur[lane] : prev[lane - K];
  if ((unsigned)e >= (unsigned)E) return quiet_nan();
  return h2f(rtab[(size_t)(lane < K ? e : E + e) * ncol + c]);
}

// fc1 rows (blockIdx.x < H) and l rows (blockIdx.x >= H) against x; grid (H + E, ceil(T / tpw)).
template <int NSEG>
__global__ void __launch_bounds__(64) k_head_in(HeadArgs a, int tpw) {
  const int r = blockIdx.x, lane = threadIdx.x;
  const bool is_fc1 = r < a.H;
  const int c = is_fc1 ? r : r - a.H;
  const uint16_t* W = is_fc1 ? a.pw.fc1_x + (size_t)c * a.d : a.pw.lin_x + (size_t)c * a.d;
  const uint16_t* rtab = is_fc1 ? a.pw.fc1_r : a.pw.lin_r;
  const int ncol = is_fc1 ? a.H : a.E;
  const uint16_t* bias = is_fc1 ? a.pw.fc1_b : a.pw.lin_b;
  const int nseg = a.d / 8;
  const int t0 = blockIdx.y * tpw, t1 = min(a.T, t0 + tpw);
  // the gather of the first token goes out before the row loads
  float kh = khot_term(rtab, ncol, c, a.E, a.K, a.cur + (size_t)t0 * a.K,
                       a.prev ? a.prev + (size_t)t0 * a.K : nullptr, lane);
  uint4 wr[NSEG];
  load_row<NSEG>(wr, W, nseg, lane);
  const float b = bias ? h2f(bias[c]) : 0.f;
  for (int t = t0; t < t1; ++t) {
    if (t > t0)
      kh = khot_term(rtab, ncol, c, a.E, a.K, a.cur + (size_t)t * a.K, a.prev ? a.prev + (size_t)t * a.K : nullptr,
                     lane);
    float acc, sq;
    row_dot_tokens<NSEG>(wr, nseg, a.x, a.d, t, lane, acc, sq);
    const float g = group_sum(kh, 32);   // at most 2K <= 32 lanes hold terms
    if (lane == 0) {
      const float s = (a.flags & MOE_INPUT_RMSNORM) ? 1.f / sqrtf(sq / (float)a.d + RMS_EPS) : 1.f;
      const float v = acc * s + g + b;
      if (is_fc1)
        a.g[(size_t)t * a.H + c] = gelu_erf(v);
      else
        a.lin[(size_t)t * a.E + c] = v;
    }
  }
}

// logits[t][e] = fc2[e] . g_t + fc2_b[e] + lin[t][e]; grid (E, ceil(T / tpw)).
template <int NSEG>
__global__ void __launch_bounds__(64) k_head_out(HeadArgs a, int tpw, float* __restrict__ logits) {
  const int e = blockIdx.x, lane = threadIdx.x;
  const int nseg = a.H / 8;
  uint4 wr[NSEG];
  load_row<NSEG>(wr, a.pw.fc2 + (size_t)e * a.H, nseg, lane);
  const int t1 = min(a.T, (int)(blockIdx.y + 1) * tpw);
  for (int t = blockIdx.y * tpw; t < t1; ++t) {
    const float* gt = a.g + (size_t)t * a.H;
    float acc = 0.f;
#pragma unroll
    for (int p = 0; p < NSEG; ++p) {
      const int sgi = lane + p * WAVE;
      if (sgi < nseg) {
        const float4 g0 = *reinterpret_cast<const float4*>(gt + (size_t)sgi * 8);
        const float4 g1 = *reinterpret_cast<const float4*>(gt + (size_t)sgi * 8 + 4);
        const half2_t w0 = as_h2(wr[p].x), w1 = as_h2(wr[p].y), w2 = as_h2(wr[p].z), w3 = as_h2(wr[p].w);
        acc = fmaf((float)w0.x, g0.x, acc);
        acc = fmaf((float)w0.y, g0.y, acc);
        acc = fmaf((float)w1.x, g0.z, acc);
        acc = fmaf((float)w1.y, g0.w, acc);
        acc = fmaf((float)w2.x, g1.x, acc);
        acc = fmaf((float)w2.y, g1.y, acc);
        acc = fmaf((float)w3.x, g1.z, acc);
        acc = fmaf((float)w3.y, g1.w, acc);
      }
    }
    acc = group_sum(acc, WAVE);
    if (lane == 0) {
      float v = acc + a.lin[(size_t)t * a.E + e];
      if (a.pw.fc2_b) v += h2f(a.pw.fc2_b[e]);
      logits[(size_t)t * a.E + e] = v;
    }
  }
}

int nseg_for(int cols) {  // 128-bit segments per lane, rounded up to a power of two
  const int per_lane = (cols / 8 + WAVE - 1) / WAVE;
  int n = 1;
  while (n < per_lane) n <<= 1;
  return n;
}

constexpr int TPW = 16;  // tokens per wave in the matvecs

}  // namespace

// x[t] = float16(g * h[t] / sqrt(mean(h[t]^2) + eps)); one wave per token, the sum of squares in a
// fixed order (each lane's 8-column slices, then a DPP reduction), so equal rows give equal x.
__global__ void __launch_bounds__(256) k_rmsnorm(int T, int d, const uint16_t* __restrict__ h,
                                                 const uint16_t* __restrict__ gain, uint16_t* __restrict__ x) {
  const int t = (int)((blockIdx.x * blockDim.x + threadIdx.x) / WAVE), lane = threadIdx.x % WAVE;
  if (t >= T) return;  // uniform over the wave
  const uint16_t* hr = h + (size_t)t * d;
  float sq = 0.f;
  for (int c = lane * 8; c < d; c += WAVE * 8) {
    const uint4 v = *reinterpret_cast<const uint4*>(hr + c);
    const uint32_t a[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) sq = __builtin_amdgcn_fdot2(as_h2(a[i]), as_h2(a[i]), sq, false);
  }
  const float s = 1.f / sqrtf(group_sum(sq, WAVE) / (float)d + RMS_EPS);
  for (int c = lane * 8; c < d; c += WAVE * 8) {
    const uint4 v = *reinterpret_cast<const uint4*>(hr + c);
    const uint4 g = gain ? *reinterpret_cast<const uint4*>(gain + c) : make_uint4(0x3C003C00u, 0x3C003C00u,
                                                                                   0x3C003C00u, 0x3C003C00u);
    const uint32_t a[4] = {v.x, v.y, v.z, v.w}, b[4] = {g.x, g.y, g.z, g.w};
    uint32_t o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const half2_t hv = as_h2(a[i]), gv = as_h2(b[i]);
      o[i] = f2h((float)hv[0] * (float)gv[0] * s) | ((uint32_t)f2h((float)hv[1] * (float)gv[1] * s) << 16);
    }
    *reinterpret_cast<uint4*>(x + (size_t)t * d + c) = make_uint4(o[0], o[1], o[2], o[3]);
  }
}

hipError_t launch_rmsnorm(hipStream_t s, int T, int d, const uint16_t* h, const uint16_t* gain, uint16_t* x) {
  return launch(k_rmsnorm, dim3((T + 3) / 4), dim3(256), 0, s, T, d, h, gain, x);
}

constexpr int RK_SMALL = 128;  // 16 waves at d = 2048: shorter load chains than 4 waves of 512 columns
hipError_t launch_router_gemv(hipStream_t s, int T, int d, int E, uint32_t flags, const uint16_t* x,
                              const uint16_t* w, float* logits) {
  if (T >= 32 && T % 16 == 0 && E % 16 == 0 && d % 32 == 0 && d <= MOE_MAX_D && (((uintptr_t)x | (uintptr_t)w) & 15) == 0) {
    // the fewest columns per wave that keep the block within R_MAXW waves
    const dim3 grid(T / 16, E / 16);
    if (d <= R_MAXW * RK_SMALL)
      return launch(k_router_mfma<RK_SMALL>, grid, dim3((d + RK_SMALL - 1) / RK_SMALL * WAVE), 0, s, T, d, E, flags,
                    x, w, logits);
    if (d <= R_MAXW * 256)
      return launch(k_router_mfma<256>, grid, dim3((d + 255) / 256 * WAVE), 0, s, T, d, E, flags, x, w, logits);
    return launch(k_router_mfma<512>, grid, dim3((d + 511) / 512 * WAVE), 0, s, T, d, E, flags, x, w, logits);
  }
  const dim3 grid(E, (T + TPW - 1) / TPW);
  switch (nseg_for(d)) {
    case 1: return launch(k_router<1>, grid, dim3(WAVE), 0, s, T, d, E, flags, TPW, x, w, logits);
    case 2: return launch(k_router<2>, grid, dim3(WAVE), 0, s, T, d, E, flags, TPW, x, w, logits);
    case 4: return launch(k_router<4>, grid, dim3(WAVE), 0, s, T, d, E, flags, TPW, x, w, logits);
    case 8: return launch(k_router<8>, grid, dim3(WAVE), 0, s, T, d, E, flags, TPW, x, w, logits);
    default: return launch(k_router<16>, grid, dim3(WAVE), 0, s, T, d, E, flags, TPW, x, w, logits);
  }
}

hipError_t launch_topk(hipStream_t s, int T, int E, int K, uint32_t flags, const float* logits, int32_t* idx,
                       float* w) {
  static_assert(MOE_MAX_E <= 16 * WAVE, "k_topk holds at most 16 logits per lane");
  if (E <= WAVE) return launch(k_topk<1>, dim3(T), dim3(WAVE), 0, s, T, E, K, flags, logits, idx, w);
  if (E <= 2 * WAVE) return launch(k_topk<2>, dim3(T), dim3(WAVE), 0, s, T, E, K, flags, logits, idx, w);
  if (E <= 4 * WAVE) return launch(k_topk<4>, dim3(T), dim3(WAVE), 0, s, T, E, K, flags, logits, idx, w);
  if (E <= 8 * WAVE) return launch(k_topk<8>, dim3(T), dim3(WAVE), 0, s, T, E, K, flags, logits, idx, w);
  return launch(k_topk<16>, dim3(T), dim3(WAVE), 0, s, T, E, K, flags, logits, idx, w);
}

hipError_t launch_prerouter(hipStream_t s, int T, int d, int E, int K, uint32_t flags, const uint16_t* x,
                            const int32_t* idx_cur, const int32_t* idx_prev, const moe_prerouter_w& pw,
                            float* logits, float* ws_g, float* ws_lin) {
  HeadArgs a{T, d, E, K, pw.d_hidden, flags, x, idx_cur, idx_prev, pw, ws_g, ws_lin};
  const int ty = (T + TPW - 1) / TPW;
  const dim3 g1(a.H + E, ty), g2(E, ty);
  hipError_t e1, e2;
  switch (nseg_for(d)) {
    case 1: e1 = launch(k_head_in<1>, g1, dim3(WAVE), 0, s, a, TPW); break;
    case 2: e1 = launch(k_head_in<2>, g1, dim3(WAVE), 0, s, a, TPW); break;
    case 4: e1 = launch(k_head_in<4>, g1, dim3(WAVE), 0, s, a, TPW); break;
    case 8: e1 = launch(k_head_in<8>, g1, dim3(WAVE), 0, s, a, TPW); break;
    default: e1 = launch(k_head_in<16>, g1, dim3(WAVE), 0, s, a, TPW); break;
  }
  if (e1 != hipSuccess) return e1;
  switch (nseg_for(a.H)) {
    case 1: e2 = launch(k_head_out<1>, g2, dim3(WAVE), 0, s, a, TPW, logits); break;
    case 2: e2 = launch(k_head_out<2>, g2, dim3(WAVE), 0, s, a, TPW, logits); break;
    case 4: e2 = launch(k_head_out<4>, g2, dim3(WAVE), 0, s, a, TPW, logits); break;
    case 8: e2 = launch(k_head_out<8>, g2, dim3(WAVE), 0, s, a, TPW, logits); break;
    default: e2 = launch(k_head_out<16>, g2, dim3(WAVE), 0, s, a, TPW, logits); break;
  }
  return e2;
}

}  // namespace moe
