// Batch-1 (small T) decode path of the expert FFN on gfx950: dequantise-and-matvec of the K
// selected experts' gate / up projections with SwiGLU in the epilogue, then the down projection
// with the weighted combine + residual in the epilogue.
//
// Steps follow "Inferencia de LLM MoE en MacBook Pro: Streaming de Expertos desde SSD con
// Metal", section "Arquitectura del Sistema" (4/2-bit dequantised matvec, fused SwiGLU, expert
// combine fused with the residual) and, for the shared-path adapter, the unmerged LoRA equation
// of the Edge0 reading guide ("Ejecucion del adaptador no fusionado").
//
// The SwiGLU output stays in float32 between the two kernels; the down projection meets it as a
// float16 hi + lo pair (two dot2 per code pair), so chained layers do not add a float16 rounding
// of the activation to the error they pass on.
//
// Mapping.  A packed row is S 16-byte segments.  A "row slot" of L lanes (the power of two at or
// above S, at most 64; lanes at or past S idle) owns one row; a lane owns P = ceil(S / L) <= 4
// segments and always the same columns, so it builds
// its permuted activation pairs once and reuses them for every row it visits.  A wave runs
// 64 / L row slots side by side and NB rows per slot, with all NB*P 128-bit weight loads issued
// before any arithmetic.  Row sums are xor-butterfly reductions inside the slot.  Every sum runs
// in a fixed order, so results are bit-reproducible run to run.
#include "moe_device.h"
#include "moe_launch.h"
#include "moe_lora.h"

namespace moe {
namespace {

struct LoraRef {
  const uint16_t* B;  // [rows][rank]
  const float* u;     // [T][rank]   (A v, already in float32)
  int rank;
  float scale;        // alpha / rank
};

__device__ __forceinline__ float lora_row(const LoraRef& lr, int t, int row) {
  const uint16_t* b = lr.B + (size_t)row * lr.rank;
  const float* u = lr.u + (size_t)t * lr.rank;
  float acc = 0.f;
  for (int r = 0; r < lr.rank; ++r) acc = fmaf(h2f(b[r]), u[r], acc);
  return lr.scale * acc;
}

// u = A . v (and u2 = A2 . v) for the adapter, one wave per (token, rank row).
__global__ void __launch_bounds__(256) k_lora_a(LoraAJob j) {
  lora_a_wave(j, (int)((blockIdx.x * blockDim.x + threadIdx.x) / WAVE), threadIdx.x % WAVE);
}

// scale and bias of the one or two groups a segment touches (SPLIT: a 2-bit segment spanning two
// 32-column groups)
template <int BITS, bool SPLIT>
struct SegSB {
  uint16_t sa, ba, sb, bb;
  __device__ __forceinline__ void load(const moe_qmat& m, size_t row, int ngr, int lg2g, int seg) {
    const int c0 = seg * SegT<BITS>::COLS;
    const size_t ga = row * ngr + (c0 >> lg2g);
    sa = m.scales[ga];
    ba = m.biases[ga];
    if (SPLIT) {
      const size_t gb = row * ngr + ((c0 + SegT<BITS>::COLS / 2) >> lg2g);
      sb = m.scales[gb];
      bb = m.biases[gb];
    }
  }
  // scale * sum(q x) + bias * sum(x) over the segment
  __device__ __forceinline__ float apply(float d0, float d1, const float* sx) const {
    if (SPLIT) return h2f(sa) * d0 + h2f(ba) * sx[0] + h2f(sb) * d1 + h2f(bb) * sx[1];
    return h2f(sa) * (d0 + d1) + h2f(ba) * (sx[0] + sx[1]);
  }
};

// u[t][r] = A[r] . v_t with float32 v (the SwiGLU output feeding the down projection's adapter).
__global__ void __launch_bounds__(256) k_lora_a_f32(int T, int n_in, int rank, const float* __restrict__ v,
                                                    size_t v_stride, const uint16_t* __restrict__ A,
                                                    float* __restrict__ u) {
  const int wave = (int)((blockIdx.x * blockDim.x + threadIdx.x) / WAVE);
  const int lane = threadIdx.x % WAVE;
  if (wave >= T * rank) return;
  const int t = wave / rank, r = wave % rank;
  const float* vr = v + (size_t)t * v_stride;
  const uint16_t* ar = A + (size_t)r * n_in;
  float acc = 0.f;
  for (int c = lane; c < n_in; c += WAVE) acc = fmaf(h2f(ar[c]), vr[c], acc);
  acc = group_sum(acc, WAVE);
  if (lane == 0) u[(size_t)t * rank + r] = acc;
}

// gate/up + SwiGLU.  Items are (k, i) pairs of token t = blockIdx.y, item = k * I + i.
// Loads go out in the order weights, scales/biases, activations, so one wait covers them all.
template <int BITS, int P, bool SPLIT, int NB>
__global__ void __launch_bounds__(64) k_gateup(int T, int K, int E, int d, int I, int lg2g, int L,
                                               uint32_t flags, const uint16_t* __restrict__ x,
                                               const int32_t* __restrict__ idx, moe_qmat gate,
                                               moe_qmat up, float* __restrict__ act, LoraRef lg,
                                               LoraRef lu, int relu, int32_t* __restrict__ zero, int nzero) {
  using G = SegT<BITS>;
  const int lane = threadIdx.x;
  const int t = blockIdx.y;
  // counters of the kernel that follows on the stream, cleared here so that it needs no launch of its own
  if (zero && blockIdx.x == 0)
    for (int i = lane; i < nzero; i += WAVE) zero[(size_t)t * nzero + i] = 0;
  const int RPI = WAVE / L;
  const int slot = lane / L, ls = lane % L;
  const int wpr = d * BITS / 32;
  const int ngr = d >> lg2g;
  const int S = d * BITS / 128;
  const int items = K * I;
  const int base = blockIdx.x * RPI * NB;
  if (base >= items) return;

  uint4 qg[NB][P], qu[NB][P];
  SegSB<BITS, SPLIT> sg[NB][P], su[NB][P];
  size_t row[NB];
  bool valid[NB], bad[NB];
  int kk[NB], ii[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int item = base + nb * RPI + slot;
    valid[nb] = item < items;
    const int k = valid[nb] ? item / I : 0;
    const int i = valid[nb] ? item - k * I : 0;
    int e = idx[(size_t)t * K + k];
    bad[nb] = (unsigned)e >= (unsigned)E;
    if (bad[nb]) e = 0;
    kk[nb] = k;
    ii[nb] = i;
    row[nb] = (size_t)e * I + i;
  }
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int p = 0; p < P; ++p)
      if (ls + p * L < S) {
        const size_t wo = row[nb] * wpr + (size_t)(ls + p * L) * 4;
        qg[nb][p] = *reinterpret_cast<const uint4*>(gate.q + wo);
        qu[nb][p] = *reinterpret_cast<const uint4*>(up.q + wo);
      }
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int p = 0; p < P; ++p)
      if (ls + p * L < S) {
        sg[nb][p].load(gate, row[nb], ngr, lg2g, ls + p * L);
        su[nb][p].load(up, row[nb], ngr, lg2g, ls + p * L);
      }

  uint32_t xp[P][G::PAIRS];
  float sx[P][2];
  float sq = 0.f;
  const uint16_t* xt = x + (size_t)t * d;
#pragma unroll
  for (int p = 0; p < P; ++p)
    if (ls + p * L < S) load_xpairs<BITS>(xt + (size_t)(ls + p * L) * G::COLS, xp[p], sx[p], sq);
  float scale = 1.f;
  if (flags & MOE_INPUT_RMSNORM) scale = 1.f / sqrtf(group_sum(sq, L) / (float)d + RMS_EPS);

#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    float pg = 0.f, pu = 0.f;
#pragma unroll
    for (int p = 0; p < P; ++p) {
      if (ls + p * L >= S) continue;
      float d0 = 0.f, d1 = 0.f;
      dot_segment<BITS>(qg[nb][p], xp[p], d0, d1);
      pg += sg[nb][p].apply(d0, d1, sx[p]);
      d0 = d1 = 0.f;
      dot_segment<BITS>(qu[nb][p], xp[p], d0, d1);
      pu += su[nb][p].apply(d0, d1, sx[p]);
    }
    pg = group_sum(pg, L) * scale;
    pu = group_sum(pu, L) * scale;
    if (ls == 0 && valid[nb]) {
      if (lg.B) pg += lora_row(lg, t, ii[nb]);
      if (lu.B) pu += lora_row(lu, t, ii[nb]);
      // SwiGLU: silu(gate) * up; the ReLU variant: relu(gate) * up, exactly zero for gate <= 0
      float a = relu ? (pg > 0.f ? pg * pu : 0.f) : pg / (1.f + expf(-pg)) * pu;
      if (bad[nb]) a = quiet_nan();
      act[((size_t)t * K + kk[nb]) * I + ii[nb]] = a;
    }
  }
}

// down projection (+ weighted combine + residual).  Items are output rows j of token t; the wave
// walks the token's K experts in chunks of KC, issuing every weight load of a chunk first.
template <int BITS, int P, bool SPLIT, int NB, int KC>
__global__ void __launch_bounds__(64) k_down(int T, int K, int E, int d, int I, int lg2g, int L,
                                             const float* __restrict__ act,
                                             const int32_t* __restrict__ idx, moe_qmat down,
                                             float* __restrict__ out, const float* __restrict__ wf,
                                             const uint16_t* __restrict__ rf, uint16_t* __restrict__ yf,
                                             LoraRef ldn) {
  using G = SegT<BITS>;
  const int lane = threadIdx.x;
  const int t = blockIdx.y;
  const int RPI = WAVE / L;
  const int slot = lane / L, ls = lane % L;
  const int wpr = I * BITS / 32;
  const int ngr = I >> lg2g;
  const int S = I * BITS / 128;
  const int base = blockIdx.x * RPI * NB;
  if (base >= d) return;

  int jj[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) jj[nb] = base + nb * RPI + slot;
  float acc[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) acc[nb] = 0.f;

  for (int k0 = 0; k0 < K; k0 += KC) {
    uint4 q[KC][NB][P];
    SegSB<BITS, SPLIT> sb[KC][NB][P];
    bool bad[KC];
    float wk[KC];
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
      const int k = k0 + kc;
      bad[kc] = true;
      wk[kc] = 0.f;
      if (k < K) {
        int e = idx[(size_t)t * K + k];
        bad[kc] = (unsigned)e >= (unsigned)E;
        if (bad[kc]) e = 0;
        wk[kc] = wf ? wf[(size_t)t * K + k] : 0.f;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          const size_t rw = (size_t)e * d + (jj[nb] < d ? jj[nb] : 0);
#pragma unroll
          for (int p = 0; p < P; ++p)
            if (ls + p * L < S) {
              q[kc][nb][p] = *reinterpret_cast<const uint4*>(down.q + rw * wpr + (size_t)(ls + p * L) * 4);
              sb[kc][nb][p].load(down, rw, ngr, lg2g, ls + p * L);
            }
        }
      }
    }
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
      const int k = k0 + kc;
      if (k >= K) break;
      uint32_t xh[P][G::PAIRS], xl[P][G::PAIRS];
      float sx[P][2];
      const float* at = act + ((size_t)t * K + k) * I;
#pragma unroll
      for (int p = 0; p < P; ++p)
        if (ls + p * L < S) load_xpairs_f32<BITS>(at + (size_t)(ls + p * L) * G::COLS, xh[p], xl[p], sx[p]);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        float po = 0.f;
#pragma unroll
        for (int p = 0; p < P; ++p) {
          if (ls + p * L >= S) continue;
          float d0 = 0.f, d1 = 0.f;
          dot_segment_split<BITS>(q[kc][nb][p], xh[p], xl[p], d0, d1);
          po += sb[kc][nb][p].apply(d0, d1, sx[p]);
        }
        po = group_sum(po, L);
        const int j = jj[nb];
        if (ls == 0 && j < d) {
          if (ldn.B) po += lora_row(ldn, t, j);
          if (bad[kc]) po = quiet_nan();
          if (out) out[((size_t)t * K + k) * d + j] = po;
          acc[nb] = fmaf(wk[kc], po, acc[nb]);
        }
      }
    }
  }
  if (yf) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int j = jj[nb];
      if (ls == 0 && j < d) yf[(size_t)t * d + j] = f2h(h2f(rf[(size_t)t * d + j]) + acc[nb]);
    }
  }
}

// Waves per block of the LDS-staged down kernel, and its segment layout in LDS.
constexpr int DN_WAVES = 4;
template <int BITS>
struct DnLds {
  static constexpr int PAIRS = SegT<BITS>::PAIRS;
  static constexpr int STRIDE = PAIRS + 4;   // words per segment: 16 lanes of a row slot hit distinct banks
};

// The down projection with the token's activations staged once per block.  The plain k_down has
// every row slot of every wave load and split the float32 activations of all K experts itself
// (4 row slots per wave x every wave: the 8 KB of a decode35b token was read from L2 some 2,000
// times); here DN_WAVES waves share one copy in LDS, held as the permuted float16 hi / lo pairs the
// dot products take.  One segment per lane (P = 1), K <= KMAX, all K experts' weights issued before
// the staging so that its latency hides under theirs.
template <int BITS>
size_t down_lds_bytes(int K, int I) {
  const int segs = K * (I * BITS / 128);
  return (size_t)segs * (2 * DnLds<BITS>::STRIDE * 4 + 8);
}

template <int BITS, bool SPLIT, int KMAX>
__global__ void __launch_bounds__(DN_WAVES * WAVE) k_down_lds(int T, int K, int E, int d, int I, int lg2g, int L,
                                                          const float* __restrict__ act,
                                                          const int32_t* __restrict__ idx, moe_qmat down,
                                                          float* __restrict__ out, const float* __restrict__ wf,
                                                          const uint16_t* __restrict__ rf,
                                                          uint16_t* __restrict__ yf, LoraRef ldn) {
  using G = SegT<BITS>;
  using D = DnLds<BITS>;
  extern __shared__ __align__(16) uint32_t dsm[];
  const int tid = threadIdx.x, lane = tid % WAVE, wv = tid / WAVE;
  const int t = blockIdx.y;
  const int RPI = WAVE / L;
  const int slot = lane / L, ls = lane % L;
  const int wpr = I * BITS / 32;
  const int ngr = I >> lg2g;
  const int S = I * BITS / 128;
  const int j = (blockIdx.x * DN_WAVES + wv) * RPI + slot;
  const bool jok = j < d;
  const bool seg = ls < S;
  const int lsc = seg ? ls : 0;
  uint32_t* hpL = dsm;                                   // [K * S][STRIDE]
  uint32_t* lpL = dsm + (size_t)K * S * D::STRIDE;       // [K * S][STRIDE]
  float* sxL = reinterpret_cast<float*>(lpL + (size_t)K * S * D::STRIDE);  // [K * S][2]

  // 1. this lane's weights of all K experts
  uint4 q[KMAX];
  SegSB<BITS, SPLIT> sb[KMAX];
  bool bad[KMAX];
  float wk[KMAX];
#pragma unroll
  for (int k = 0; k < KMAX; ++k) {
    bad[k] = true;
    wk[k] = 0.f;
    if (k < K) {
      int e = idx[(size_t)t * K + k];
      bad[k] = (unsigned)e >= (unsigned)E;
      if (bad[k]) e = 0;
      wk[k] = wf ? wf[(size_t)t * K + k] : 0.f;
      const size_t rw = (size_t)e * d + (jok ? j : 0);
      q[k] = *reinterpret_cast<const uint4*>(down.q + rw * wpr + (size_t)lsc * 4);
      sb[k].load(down, rw, ngr, lg2g, lsc);
    }
  }
  // 2. the token's activations, split and permuted once per block (one segment per thread step)
  for (int u = tid; u < K * S; u += DN_WAVES * WAVE) {
    const int k = u / S, sg = u - k * S;
    uint32_t hp[G::PAIRS], lp[G::PAIRS];
    float sx[2];
    load_xpairs_f32<BITS>(act + ((size_t)t * K + k) * I + (size_t)sg * G::COLS, hp, lp, sx);
    uint4* hd = reinterpret_cast<uint4*>(hpL + (size_t)u * D::STRIDE);
    uint4* ld = reinterpret_cast<uint4*>(lpL + (size_t)u * D::STRIDE);
#pragma unroll
    for (int w = 0; w < G::PAIRS / 4; ++w) {
      hd[w] = make_uint4(hp[4 * w], hp[4 * w + 1], hp[4 * w + 2], hp[4 * w + 3]);
      ld[w] = make_uint4(lp[4 * w], lp[4 * w + 1], lp[4 * w + 2], lp[4 * w + 3]);
    }
    sxL[2 * u] = sx[0];
    sxL[2 * u + 1] = sx[1];
  }
  __syncthreads();
  // 3. dot products, expert by expert, and the weighted combine in ascending k
  float acc = 0.f;
#pragma unroll
  for (int k = 0; k < KMAX; ++k) {
    if (k >= K) break;
    float po = 0.f;
    if (seg) {
      const int u = k * S + ls;
      uint32_t hp[G::PAIRS], lp[G::PAIRS];
      const uint4* hs = reinterpret_cast<const uint4*>(hpL + (size_t)u * D::STRIDE);
      const uint4* lsrc = reinterpret_cast<const uint4*>(lpL + (size_t)u * D::STRIDE);
#pragma unroll
      for (int w = 0; w < G::PAIRS / 4; ++w) {
        const uint4 a = hs[w], b = lsrc[w];
        hp[4 * w] = a.x, hp[4 * w + 1] = a.y, hp[4 * w + 2] = a.z, hp[4 * w + 3] = a.w;
        lp[4 * w] = b.x, lp[4 * w + 1] = b.y, lp[4 * w + 2] = b.z, lp[4 * w + 3] = b.w;
      }
      const float sx[2] = {sxL[2 * u], sxL[2 * u + 1]};
      float d0 = 0.f, d1 = 0.f;
      dot_segment_split<BITS>(q[k], hp, lp, d0, d1);
      po = sb[k].apply(d0, d1, sx);
    }
    po = group_sum(po, L);
    if (ls == 0 && jok) {
      if (ldn.B) po += lora_row(ldn, t, j);
      if (bad[k]) po = quiet_nan();
      if (out) out[((size_t)t * K + k) * d + j] = po;
      acc = fmaf(wk[k], po, acc);
    }
  }
  if (yf && ls == 0 && jok) yf[(size_t)t * d + j] = f2h(h2f(rf[(size_t)t * d + j]) + acc);
}

__global__ void __launch_bounds__(256) k_combine(int T, int K, int d, const float* __restrict__ o,
                                                 const float* __restrict__ w,
                                                 const uint16_t* __restrict__ r,
                                                 const float* __restrict__ shared,
                                                 uint16_t* __restrict__ y) {
  const size_t n = (size_t)T * d;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) {
    const size_t t = i / d, j = i - t * d;
    float acc = 0.f;
    for (int k = 0; k < K; ++k) acc = fmaf(w[t * K + k], o[(t * K + k) * d + j], acc);
    if (shared) acc += shared[i];
    y[i] = f2h(h2f(r[i]) + acc);
  }
}

// The same four columns at a time (d a multiple of 4, 16-byte aligned o and shared, 8-byte aligned r
// and y, T d < 2^31): 16-byte loads of o and 32-bit index arithmetic.  Each element's arithmetic
// is k_combine's, in the same order, so the two give the same bits.
__global__ void __launch_bounds__(256) k_combine4(int T, int K, int d, const float4* __restrict__ o,
                                                  const float* __restrict__ w, const uint2* __restrict__ r,
                                                  const float4* __restrict__ shared, uint2* __restrict__ y) {
  const int d4 = d / 4, n4 = T * d4;
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += gridDim.x * blockDim.x) {
    const int t = i / d4, j = i - t * d4;
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
    for (int k = 0; k < K; ++k) {
      const float wk = w[t * K + k];
      const float4 v = o[(size_t)(t * K + k) * d4 + j];
      acc[0] = fmaf(wk, v.x, acc[0]);
      acc[1] = fmaf(wk, v.y, acc[1]);
      acc[2] = fmaf(wk, v.z, acc[2]);
      acc[3] = fmaf(wk, v.w, acc[3]);
    }
    if (shared) {
      const float4 v = shared[i];
      acc[0] += v.x;
      acc[1] += v.y;
      acc[2] += v.z;
      acc[3] += v.w;
    }
    const uint2 rv = r[i];
    const uint32_t rw[2] = {rv.x, rv.y};
    uint32_t yw[2];
#pragma unroll
    for (int h = 0; h < 2; ++h)
      yw[h] = f2h(h2f((uint16_t)rw[h]) + acc[2 * h]) | (uint32_t)f2h(h2f((uint16_t)(rw[h] >> 16)) + acc[2 * h + 1]) << 16;
    y[i] = make_uint2(yw[0], yw[1]);
  }
}

// geometry of a packed row with `cols` columns: S segments, row slots of L lanes (a power of two,
// lanes at or past S idle), P segments per lane.
struct RowGeo {
  int S, L, P;
  bool ok;
};
RowGeo row_geo(int bits, int cols) {
  RowGeo g{};
  g.S = cols * bits / 128;
  if (g.S <= 0 || (cols * bits) % 128) return g;
  g.L = 1;
  while (g.L < g.S && g.L < WAVE) g.L <<= 1;
  g.P = (g.S + g.L - 1) / g.L;
  g.ok = g.P <= 4;
  return g;
}

int ilog2(int v) {
  int r = 0;
  while ((1 << r) < v) ++r;
  return r;
}

constexpr int NB_GATEUP = 2;
constexpr int NB_DOWN = 1;

template <int BITS, int P, bool SPLIT>
hipError_t launch_pair(hipStream_t s, const DecodeArgs& a, const RowGeo& gu, const RowGeo& gd, LoraRef lg,
                 LoraRef lu, LoraRef ldn, int which) {
  const int lg2g = ilog2(a.group);
  if (which == 0) {
    const int rpw = (WAVE / gu.L) * NB_GATEUP;
    dim3 grid((a.K * a.I + rpw - 1) / rpw, a.T);
    return launch(k_gateup<BITS, P, SPLIT, NB_GATEUP>, grid, dim3(WAVE), 0, s, a.T, a.K, a.E, a.d, a.I, lg2g,
                  gu.L, a.flags, a.x, a.idx, a.ex.gate, a.ex.up, (float*)a.act, lg, lu, a.relu ? 1 : 0, a.zero,
                  a.nzero);
  }
  if (P == 1 && a.K <= 8 && down_lds_bytes<BITS>(a.K, a.I) <= 48 * 1024) {
    const int rpb = (WAVE / gd.L) * DN_WAVES;
    dim3 grid((a.d + rpb - 1) / rpb, a.T);
    auto go_lds = [&](auto kern) {
      return launch(kern, grid, dim3(DN_WAVES * WAVE), down_lds_bytes<BITS>(a.K, a.I), s, a.T, a.K, a.E, a.d, a.I,
                    lg2g, gd.L, (const float*)a.act, a.idx, a.ex.down, a.out, a.w_fuse, a.r_fuse, a.y_fuse, ldn);
    };
    if (a.K <= 4) return go_lds(k_down_lds<BITS, SPLIT, 4>);
    return go_lds(k_down_lds<BITS, SPLIT, 8>);
  }
  const int rpw = (WAVE / gd.L) * NB_DOWN;
  dim3 grid((a.d + rpw - 1) / rpw, a.T);
  auto go = [&](auto kern) {
    return launch(kern, grid, dim3(WAVE), 0, s, a.T, a.K, a.E, a.d, a.I, lg2g, gd.L, (const float*)a.act,
                  a.idx, a.ex.down, a.out, a.w_fuse, a.r_fuse, a.y_fuse, ldn);
  };
  if (a.K <= 2) return go(k_down<BITS, P, SPLIT, NB_DOWN, 2>);
  if (a.K <= 4) return go(k_down<BITS, P, SPLIT, NB_DOWN, 4>);
  return go(k_down<BITS, P, SPLIT, NB_DOWN, 8>);
}

template <int BITS, bool SPLIT>
hipError_t launch_p(hipStream_t s, const DecodeArgs& a, const RowGeo& gu, const RowGeo& gd, LoraRef lg,
              LoraRef lu, LoraRef ldn, int which) {
  switch (which == 0 ? gu.P : gd.P) {
    case 1: return launch_pair<BITS, 1, SPLIT>(s, a, gu, gd, lg, lu, ldn, which);
    case 2: return launch_pair<BITS, 2, SPLIT>(s, a, gu, gd, lg, lu, ldn, which);
    case 3: return launch_pair<BITS, 3, SPLIT>(s, a, gu, gd, lg, lu, ldn, which);
    default: return launch_pair<BITS, 4, SPLIT>(s, a, gu, gd, lg, lu, ldn, which);
  }
}

}  // namespace

hipError_t launch_lora_a(hipStream_t s, int waves, int T, int n_in, int rank, int rmsnorm, const uint16_t* v,
                         size_t v_stride, const uint16_t* A, float* u, const uint16_t* A2, float* u2) {
  const LoraAJob j{T, n_in, rmsnorm, v, v_stride, A, u, rank, A2, u2, rank};
  if (waves != T * rank) return hipErrorInvalidValue;
  return launch(k_lora_a, dim3((j.waves() + 3) / 4), dim3(256), 0, s, j);
}

bool decode_shape_supported(int bits, int group, int d, int I) {
  return row_geo(bits, d).ok && row_geo(bits, I).ok && group >= 32;
}

hipError_t launch_expert_decode(hipStream_t s, const DecodeArgs& a) {
  const RowGeo gu = row_geo(a.bits, a.d), gd = row_geo(a.bits, a.I);
  LoraRef lg{}, lu{}, ldn{};
  const int rms = (a.flags & MOE_INPUT_RMSNORM) != 0;
  hipError_t err = hipSuccess;
  if (a.lora3) {
    const moe_lora* L3 = a.lora3;
    const int wg = a.T * L3[0].rank, wu = a.T * L3[1].rank;
    if (wg == wu) {  // gate's and up's A . x in one launch
      err = first_error(err, launch_lora_a(s, wg, a.T, a.d, L3[0].rank, rms, a.x, (size_t)a.d, L3[0].A, a.u_gate,
                                           L3[1].A, a.u_up));
    } else {
      err = first_error(err, launch_lora_a(s, wg, a.T, a.d, L3[0].rank, rms, a.x, (size_t)a.d, L3[0].A, a.u_gate));
      err = first_error(err, launch_lora_a(s, wu, a.T, a.d, L3[1].rank, rms, a.x, (size_t)a.d, L3[1].A, a.u_up));
    }
    lg = LoraRef{L3[0].B, a.u_gate, L3[0].rank, L3[0].alpha / (float)L3[0].rank};
    lu = LoraRef{L3[1].B, a.u_up, L3[1].rank, L3[1].alpha / (float)L3[1].rank};
    ldn = LoraRef{L3[2].B, a.u_down, L3[2].rank, L3[2].alpha / (float)L3[2].rank};
  }
  const bool split = a.bits == 2 && a.group < SegT<2>::COLS;
  for (int which = 0; which < 2 && err == hipSuccess; ++which) {
    if (which == 1 && a.lora3) {
      const int wd = a.T * a.lora3[2].rank;
      err = first_error(err, launch(k_lora_a_f32, dim3((wd + 3) / 4), dim3(256), 0, s, a.T, a.I, a.lora3[2].rank,
                                    (const float*)a.act, (size_t)a.K * a.I, a.lora3[2].A, a.u_down));
    }
    if (a.bits == 4)
      err = first_error(err, launch_p<4, false>(s, a, gu, gd, lg, lu, ldn, which));
    else if (split)
      err = first_error(err, launch_p<2, true>(s, a, gu, gd, lg, lu, ldn, which));
    else
      err = first_error(err, launch_p<2, false>(s, a, gu, gd, lg, lu, ldn, which));
  }
  return err;
}

hipError_t launch_gateup_decode(hipStream_t s, const DecodeArgs& a) {
  const RowGeo gu = row_geo(a.bits, a.d);
  const bool split = a.bits == 2 && a.group < SegT<2>::COLS;
  if (a.bits == 4) return launch_p<4, false>(s, a, gu, gu, LoraRef{}, LoraRef{}, LoraRef{}, 0);
  if (split) return launch_p<2, true>(s, a, gu, gu, LoraRef{}, LoraRef{}, LoraRef{}, 0);
  return launch_p<2, false>(s, a, gu, gu, LoraRef{}, LoraRef{}, LoraRef{}, 0);
}

hipError_t launch_combine(hipStream_t s, int T, int K, int d, const float* o, const float* w,
                          const uint16_t* r, const float* shared, uint16_t* y) {
  const size_t n = (size_t)T * d;
  if (d % 4 == 0 && n < ((size_t)1 << 31) && (((uintptr_t)o | (uintptr_t)shared) & 15) == 0 &&
      (((uintptr_t)r | (uintptr_t)y) & 7) == 0) {
    int blocks = (int)((n / 4 + 255) / 256);
    if (blocks > 4096) blocks = 4096;
    return launch(k_combine4, dim3(blocks), dim3(256), 0, s, T, K, d, (const float4*)o, w, (const uint2*)r,
                  (const float4*)shared, (uint2*)y);
  }
  int blocks = (int)((n + 255) / 256);
  if (blocks > 4096) blocks = 4096;
  return launch(k_combine, dim3(blocks), dim3(256), 0, s, T, K, d, o, w, r, shared, y);
}

}  // namespace moe
