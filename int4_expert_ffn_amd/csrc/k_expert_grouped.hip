// Batched (many-token) expert FFN on gfx950: tokens sorted by expert, then grouped GEMMs on the
// matrix cores.
//
// Steps: a stable counting sort of the T*K (token, slot) pairs by expert (ties keep ascending
// (t, k)); for each expert, the gate/up projections of its gathered token rows as MFMA tiles
// with SwiGLU in the epilogue; the down projection the same way, its rows scattered back to
// (token, slot) order; then the weighted combine + residual.  The unmerged LoRA delta of a
// single shared expert is added in the epilogues ("La otra mitad del muro de la memoria ...",
// section "Ejecucion del adaptador no fusionado"); the dequantised projections, SwiGLU and
// combine follow "Inferencia de LLM MoE en MacBook Pro ...", section "Arquitectura del Sistema".
//
// MFMA mapping (v_mfma_f32_16x16x16_f16): A = 16 token rows x 16 columns, B = 16 columns x 16
// weight rows, D = 16 tokens x 16 weight rows in float32.  A wave owns 16 weight rows; lane
// (n = lane % 16, q = lane / 16) loads one 16-byte segment of row n (32 int4 / 64 int2 columns,
// segment q of a 4-segment macro step) and dequantises it once to float16 pairs
// w = fma(code, scale, bias).  MFMA step s takes the lane's pairs 2s and 2s+1; the token rows
// are staged in LDS with columns permuted inside each 8 (int4) or 16 (int2) column block so the
// same four columns sit next to each other, so A is one 8-byte LDS read.  Which physical column
// feeds which k slot does not matter to the dot product as long as A and B agree.
#include "moe_device.h"
#include "moe_launch.h"

namespace moe {
namespace {

constexpr int GT_WAVES = 4;          // waves per block: 4 x 16 weight rows
constexpr int KCH = 512;             // columns of token rows staged per LDS pass
constexpr int XS_STRIDE = KCH + 8;   // halves per staged row (padding spreads LDS banks)

// ------------------------------------------------------------------------------------- sort
// One block.  counts[E+1], offsets[E+2] (bucket E collects indices outside [0, E)),
// perm[T*K]: pair indices grouped by expert, ascending inside each expert.
__global__ void __launch_bounds__(1024) k_sort(int TK, int E, const int32_t* __restrict__ idx,
                                               int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
                                               int32_t* __restrict__ perm) {
  extern __shared__ int sh[];
  int* run = sh;              // [E+1]
  int* offs = sh + E + 1;     // [E+2]
  int* ids = offs + E + 2;    // [blockDim]
  const int tid = threadIdx.x, bs = blockDim.x;
  for (int i = tid; i <= E; i += bs) run[i] = 0;
  __syncthreads();
  for (int p = tid; p < TK; p += bs) {
    int e = idx[p];
    if ((unsigned)e >= (unsigned)E) e = E;
    atomicAdd(&run[e], 1);
  }
  __syncthreads();
  if (tid == 0) {
    int acc = 0;
    for (int e = 0; e <= E; ++e) {
      offs[e] = acc;
      acc += run[e];
    }
    offs[E + 1] = acc;
  }
  __syncthreads();
  for (int i = tid; i <= E + 1; i += bs) {
    offsets[i] = offs[i];
    if (i <= E) counts[i] = run[i];
  }
  for (int i = tid; i <= E; i += bs) run[i] = 0;
  __syncthreads();
  for (int base = 0; base < TK; base += bs) {
    const int p = base + tid;
    int e = -1;
    if (p < TK) {
      e = idx[p];
      if ((unsigned)e >= (unsigned)E) e = E;
    }
    ids[tid] = e;
    __syncthreads();
    if (p < TK) {
      int rank = 0;
      for (int j = 0; j < tid; ++j) rank += ids[j] == e;
      perm[offs[e] + run[e] + rank] = p;
    }
    __syncthreads();
    if (p < TK) atomicAdd(&run[e], 1);
    __syncthreads();
  }
}

// rowscale[t] = 1 / sqrt(mean(x_t^2) + eps); one wave per token.
__global__ void __launch_bounds__(256) k_rowscale(int T, int d, const uint16_t* __restrict__ x,
                                                  float* __restrict__ rowscale) {
  const int t = (int)((blockIdx.x * blockDim.x + threadIdx.x) / WAVE), lane = threadIdx.x % WAVE;
  if (t >= T) return;
  float sq = 0.f;
  for (int c = lane * 8; c < d; c += WAVE * 8) {
    const uint4 v = *reinterpret_cast<const uint4*>(x + (size_t)t * d + c);
    const uint32_t a[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) sq = __builtin_amdgcn_fdot2(as_h2(a[i]), as_h2(a[i]), sq, false);
  }
  sq = group_sum(sq, WAVE);
  if (lane == 0) rowscale[t] = 1.f / sqrtf(sq / (float)d + RMS_EPS);
}

// ------------------------------------------------------------------------------------- MFMA core
template <int BITS>
struct GSeg {
  static constexpr int COLS = SegT<BITS>::COLS;     // columns per lane segment
  static constexpr int MACRO = 4 * COLS;            // columns per macro step (4 lane quads)
  static constexpr int STEPS = SegT<BITS>::PAIRS / 2;  // MFMA steps per macro step
  static constexpr int PB = BITS == 4 ? 8 : 16;     // columns per permutation block
};

// Stage 16 rows x KCH columns [c0, c0 + KCH) of the float16 matrix rows listed by `rows`
// (row < 0 = zero padding) into LDS, permuted per block so that each code pair's two
// activation columns are adjacent.
template <int BITS>
__device__ __forceinline__ void stage_rows(uint16_t* xs, const uint16_t* __restrict__ src, int ncols, int c0,
                                           const int* rows) {
  constexpr int PB = GSeg<BITS>::PB;
  constexpr int UNITS = 16 * KCH / PB;
  for (int u = threadIdx.x; u < UNITS; u += blockDim.x) {
    const int m = u / (KCH / PB), cb = u % (KCH / PB);
    const int col = c0 + cb * PB;
    const int r = rows[m];
    uint32_t outw[PB / 2];
    if (r >= 0 && col < ncols) {
      const uint4* p = reinterpret_cast<const uint4*>(src + (size_t)r * ncols + col);
      if constexpr (BITS == 4) {
        const uint4 v = p[0];
        outw[0] = (v.x & 0xFFFFu) | (v.z << 16);
        outw[1] = (v.x >> 16) | (v.z & 0xFFFF0000u);
        outw[2] = (v.y & 0xFFFFu) | (v.w << 16);
        outw[3] = (v.y >> 16) | (v.w & 0xFFFF0000u);
      } else {
        const uint4 a = p[0], b = p[1];
        const uint32_t av[4] = {a.x, a.y, a.z, a.w}, bv[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const uint32_t lo = (j & 1) ? (av[j >> 1] >> 16) : (av[j >> 1] & 0xFFFFu);
          const uint32_t hi = (j & 1) ? (bv[j >> 1] & 0xFFFF0000u) : (bv[j >> 1] << 16);
          outw[j] = lo | hi;
        }
      }
    } else {
#pragma unroll
      for (int j = 0; j < PB / 2; ++j) outw[j] = 0;
    }
    uint4* dst = reinterpret_cast<uint4*>(xs + m * XS_STRIDE + cb * PB);
    dst[0] = make_uint4(outw[0], outw[1], outw[2], outw[3]);
    if constexpr (PB == 16) dst[1] = make_uint4(outw[4], outw[5], outw[6], outw[7]);
  }
}

// Dequantise one 16-byte segment to float16 pairs w = fma(code, scale, bias) (pairs in the
// order the activation pairs use).  Segments at or past `ncols` give zeros.
template <int BITS, bool SPLIT>
__device__ __forceinline__ void dequant_segment(const moe_qmat& m, size_t row, int wpr, int ngr, int lg2g,
                                                int col, int ncols, uint32_t* w) {
  constexpr int PPW = SegT<BITS>::PAIRS_PER_WORD;
  constexpr uint32_t MASK = BITS == 4 ? 0x000F000Fu : 0x00030003u;
  if (col >= ncols) {
#pragma unroll
    for (int i = 0; i < 4 * PPW; ++i) w[i] = 0;
    return;
  }
  const uint4 q = *reinterpret_cast<const uint4*>(m.q + row * wpr + (size_t)col * BITS / 32);
  const size_t ga = row * ngr + (col >> lg2g);
  const size_t gb = SPLIT ? row * ngr + ((col + SegT<BITS>::COLS / 2) >> lg2g) : ga;
  const _Float16 sa = __builtin_bit_cast(_Float16, m.scales[ga]), ba = __builtin_bit_cast(_Float16, m.biases[ga]);
  const _Float16 sb = __builtin_bit_cast(_Float16, m.scales[gb]), bb = __builtin_bit_cast(_Float16, m.biases[gb]);
  const half2_t s0 = {sa, sa}, b0 = {ba, ba}, s1 = {sb, sb}, b1 = {bb, bb};
  const half2_t k1024 = {(_Float16)1024.0f, (_Float16)1024.0f};
  const uint32_t wd[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < PPW; ++j) {
      const half2_t c = as_h2(((wd[i] >> (BITS * j)) & MASK) | 0x64006400u) - k1024;
      const half2_t v = i < 2 ? __builtin_elementwise_fma(c, s0, b0) : __builtin_elementwise_fma(c, s1, b1);
      w[i * PPW + j] = __builtin_bit_cast(uint32_t, v);
    }
}

__device__ __forceinline__ half4_t pair2(uint32_t a, uint32_t b) {
  return __builtin_bit_cast(half4_t, make_uint2(a, b));
}

// acc += X[16 tokens][c0 .. c0 + KCH) * W[16 rows][same]^T for the wave's 16 rows.
template <int BITS, bool SPLIT, int NMAT>
__device__ __forceinline__ void mfma_chunk(const uint16_t* xs, const moe_qmat* mats, size_t row, int wpr, int ngr,
                                           int lg2g, int ncols, int c0, int ln, int lq, float4_t* acc) {
  using GS = GSeg<BITS>;
  for (int ms = 0; ms < KCH; ms += GS::MACRO) {
    const int col = c0 + ms + lq * GS::COLS;
    uint32_t w[NMAT][GS::STEPS * 2];
#pragma unroll
    for (int mi = 0; mi < NMAT; ++mi) dequant_segment<BITS, SPLIT>(mats[mi], row, wpr, ngr, lg2g, col, ncols, w[mi]);
    const uint16_t* xa = xs + ln * XS_STRIDE + ms + lq * GS::COLS;
#pragma unroll
    for (int s = 0; s < GS::STEPS; ++s) {
      const half4_t a = *reinterpret_cast<const half4_t*>(xa + 4 * s);
#pragma unroll
      for (int mi = 0; mi < NMAT; ++mi)
        acc[mi] = __builtin_amdgcn_mfma_f32_16x16x16f16(a, pair2(w[mi][2 * s], w[mi][2 * s + 1]), acc[mi], 0, 0, 0);
    }
  }
}

struct LoraRefG {
  const uint16_t* B;  // [rows][rank]
  const float* u;     // [T][rank]
  int rank;
  float scale;
};
__device__ __forceinline__ float lora_row_g(const LoraRefG& lr, int t, int row) {
  const uint16_t* b = lr.B + (size_t)row * lr.rank;
  const float* u = lr.u + (size_t)t * lr.rank;
  float acc = 0.f;
  for (int r = 0; r < lr.rank; ++r) acc = fmaf(h2f(b[r]), u[r], acc);
  return lr.scale * acc;
}

// gate/up + SwiGLU for expert blockIdx.x, weight rows blockIdx.y * 64 .. +64.
// act_sorted[pos][i] (float16) for the expert's sorted pair positions.
template <int BITS, bool SPLIT>
__global__ void __launch_bounds__(256) k_grouped_gateup(int K, int E, int d, int I, int lg2g,
                                                        const uint16_t* __restrict__ x,
                                                        const int32_t* __restrict__ offsets,
                                                        const int32_t* __restrict__ perm,
                                                        const float* __restrict__ rowscale, moe_qmat gate,
                                                        moe_qmat up, uint16_t* __restrict__ act_sorted,
                                                        LoraRefG lg, LoraRefG lu) {
  __shared__ __attribute__((aligned(16))) uint16_t xs[16 * XS_STRIDE];
  __shared__ int rows[16];
  const int e = blockIdx.x;
  if (e >= E) return;
  const int beg = offsets[e], n_e = offsets[e + 1] - beg;
  if (n_e == 0) return;
  const int wave = threadIdx.x / WAVE, lane = threadIdx.x % WAVE;
  const int ln = lane % 16, lq = lane / 16;
  const int n0 = blockIdx.y * (16 * GT_WAVES) + wave * 16;
  const bool active = n0 < I;
  const int wpr = d * BITS / 32, ngr = d >> lg2g;
  const size_t row = (size_t)e * I + (active ? n0 + ln : 0);
  const moe_qmat mats[2] = {gate, up};
  for (int mt = 0; mt < n_e; mt += 16) {
    float4_t acc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
    for (int c0 = 0; c0 < d; c0 += KCH) {
      __syncthreads();
      if (threadIdx.x < 16) {
        const int pos = mt + threadIdx.x;
        rows[threadIdx.x] = pos < n_e ? perm[beg + pos] / K : -1;
      }
      __syncthreads();
      stage_rows<BITS>(xs, x, d, c0, rows);
      __syncthreads();
      if (active) mfma_chunk<BITS, SPLIT, 2>(xs, mats, row, wpr, ngr, lg2g, d, c0, ln, lq, acc);
    }
    if (active) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int pos = mt + 4 * lq + i;
        if (pos >= n_e) continue;
        const int n = n0 + ln;
        const int t = perm[beg + pos] / K;
        const float sc = rowscale ? rowscale[t] : 1.f;
        float g = acc[0][i] * sc, u = acc[1][i] * sc;
        if (lg.B) g += lora_row_g(lg, t, n);
        if (lu.B) u += lora_row_g(lu, t, n);
        act_sorted[(size_t)(beg + pos) * I + n] = f2h(g / (1.f + expf(-g)) * u);
      }
    }
  }
}

// down projection for expert blockIdx.x, output rows blockIdx.y * 64 .. +64; rows scattered
// to out[pair][j] (float32, pair = t*K + k).  Bucket E (indices outside [0, E)) writes NaN.
template <int BITS, bool SPLIT>
__global__ void __launch_bounds__(256) k_grouped_down(int K, int E, int d, int I, int lg2g,
                                                      const uint16_t* __restrict__ act_sorted,
                                                      const int32_t* __restrict__ offsets,
                                                      const int32_t* __restrict__ perm, moe_qmat down,
                                                      float* __restrict__ out, LoraRefG ldn) {
  __shared__ __attribute__((aligned(16))) uint16_t xs[16 * XS_STRIDE];
  __shared__ int rows[16];
  const int e = blockIdx.x;
  const int beg = offsets[e], n_e = offsets[e + 1] - beg;
  if (n_e == 0) return;
  const int wave = threadIdx.x / WAVE, lane = threadIdx.x % WAVE;
  const int ln = lane % 16, lq = lane / 16;
  const int n0 = blockIdx.y * (16 * GT_WAVES) + wave * 16;
  if (e == E) {  // pairs whose expert index is out of range
    for (int pos = lq; pos < n_e; pos += 4)
      if (n0 + ln < d) out[(size_t)perm[beg + pos] * d + n0 + ln] = quiet_nan();
    return;
  }
  const bool active = n0 < d;
  const int wpr = I * BITS / 32, ngr = I >> lg2g;
  const size_t row = (size_t)e * d + (active ? n0 + ln : 0);
  for (int mt = 0; mt < n_e; mt += 16) {
    float4_t acc[1] = {{0.f, 0.f, 0.f, 0.f}};
    for (int c0 = 0; c0 < I; c0 += KCH) {
      __syncthreads();
      if (threadIdx.x < 16) {
        const int pos = mt + threadIdx.x;
        rows[threadIdx.x] = pos < n_e ? beg + pos : -1;
      }
      __syncthreads();
      stage_rows<BITS>(xs, act_sorted, I, c0, rows);
      __syncthreads();
      if (active) mfma_chunk<BITS, SPLIT, 1>(xs, &down, row, wpr, ngr, lg2g, I, c0, ln, lq, acc);
    }
    if (active) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int pos = mt + 4 * lq + i;
        if (pos >= n_e) continue;
        const int j = n0 + ln;
        const int pr = perm[beg + pos];
        float o = acc[0][i];
        if (ldn.B) o += lora_row_g(ldn, pr / K, j);
        out[(size_t)pr * d + j] = o;
      }
    }
  }
}

int ilog2g(int v) {
  int r = 0;
  while ((1 << r) < v) ++r;
  return r;
}

size_t al256(size_t v) { return (v + 255) / 256 * 256; }

template <int BITS, bool SPLIT>
hipError_t launch_gemms(hipStream_t s, const GroupedArgs& g, const float* rowscale, float* o_tk, LoraRefG lg,
                        LoraRefG lu, LoraRefG ldn, const DecodeArgs& a) {
  const int lg2g = ilog2g(a.group);
  const int rows_per_block = 16 * GT_WAVES;
  hipError_t err = launch(k_grouped_gateup<BITS, SPLIT>, dim3(a.E, (a.I + rows_per_block - 1) / rows_per_block),
                          dim3(WAVE * GT_WAVES), 0, s, a.K, a.E, a.d, a.I, lg2g, a.x, (const int32_t*)g.offsets,
                          (const int32_t*)g.perm, rowscale, a.ex.gate, a.ex.up, (uint16_t*)a.act, lg, lu);
  if (err != hipSuccess) return err;
  if (a.lora3) {
    const int wd = a.T * a.lora3[2].rank;
    err = launch_lora_a(s, wd, a.T, a.I, a.lora3[2].rank, 0, (const uint16_t*)a.act, (size_t)a.K * a.I,
                        a.lora3[2].A, a.u_down);
    if (err != hipSuccess) return err;
  }
  return launch(k_grouped_down<BITS, SPLIT>, dim3(a.E + 1, (a.d + rows_per_block - 1) / rows_per_block),
                dim3(WAVE * GT_WAVES), 0, s, a.K, a.E, a.d, a.I, lg2g, (const uint16_t*)a.act,
                (const int32_t*)g.offsets, (const int32_t*)g.perm, a.ex.down, o_tk, ldn);
}

}  // namespace

size_t grouped_workspace_extra(int T, int K, int E, int d) {
  return al256((size_t)(E + 1) * 4) + al256((size_t)(E + 2) * 4) + al256((size_t)T * K * 4) + al256((size_t)T * 4) +
         al256((size_t)T * K * d * 4);
}

hipError_t launch_sort(hipStream_t s, int TK, int E, const int32_t* idx, int32_t* counts, int32_t* offsets,
                       int32_t* perm) {
  const size_t lds = (size_t)(E + 1 + E + 2 + 1024) * sizeof(int);
  return launch(k_sort, dim3(1), dim3(1024), lds, s, TK, E, idx, counts, offsets, perm);
}

hipError_t launch_expert_grouped(hipStream_t s, const GroupedArgs& g) {
  const DecodeArgs& a = g.base;
  hipError_t err = launch_sort(s, a.T * a.K, a.E, a.idx, g.counts, g.offsets, g.perm);
  if (err != hipSuccess) return err;
  float* rowscale = nullptr;
  if (a.flags & MOE_INPUT_RMSNORM) {
    rowscale = g.rowscale;
    err = launch(k_rowscale, dim3((a.T + 3) / 4), dim3(256), 0, s, a.T, a.d, a.x, rowscale);
    if (err != hipSuccess) return err;
  }
  LoraRefG lg{}, lu{}, ldn{};
  if (a.lora3) {
    const moe_lora* L3 = a.lora3;
    const int rms = (a.flags & MOE_INPUT_RMSNORM) != 0;
    err = launch_lora_a(s, a.T * L3[0].rank, a.T, a.d, L3[0].rank, rms, a.x, (size_t)a.d, L3[0].A, a.u_gate);
    if (err == hipSuccess)
      err = launch_lora_a(s, a.T * L3[1].rank, a.T, a.d, L3[1].rank, rms, a.x, (size_t)a.d, L3[1].A, a.u_up);
    if (err != hipSuccess) return err;
    lg = LoraRefG{L3[0].B, a.u_gate, L3[0].rank, L3[0].alpha / (float)L3[0].rank};
    lu = LoraRefG{L3[1].B, a.u_up, L3[1].rank, L3[1].alpha / (float)L3[1].rank};
    ldn = LoraRefG{L3[2].B, a.u_down, L3[2].rank, L3[2].alpha / (float)L3[2].rank};
  }
  float* o_tk = a.out ? a.out : g.o_sorted;
  if (a.bits == 4)
    err = launch_gemms<4, false>(s, g, rowscale, o_tk, lg, lu, ldn, a);
  else if (a.group < SegT<2>::COLS)
    err = launch_gemms<2, true>(s, g, rowscale, o_tk, lg, lu, ldn, a);
  else
    err = launch_gemms<2, false>(s, g, rowscale, o_tk, lg, lu, ldn, a);
  if (err != hipSuccess) return err;
  if (a.y_fuse) err = launch_combine(s, a.T, a.K, a.d, o_tk, a.w_fuse, a.r_fuse, nullptr, a.y_fuse);
  return err;
}

}  // namespace moe
