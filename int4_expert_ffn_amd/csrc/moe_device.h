// Device helpers shared by the gfx950 kernels: float16 bit conversions, wave64 reductions and
// the 16-byte dequantise-and-dot step.
//
// A "segment" is 16 bytes of one packed row: 4 little-endian uint32 words holding 32 4-bit or
// 64 2-bit codes.  One lane loads one segment with a single 128-bit load.  The codes are turned
// into float16 pairs with the exponent trick: (word >> s) & 0x000F000F | 0x64006400 is the
// float16 pair (1024 + c_lo, 1024 + c_hi), exact; subtracting 1024 leaves the codes as exact
// float16, and v_dot2_f32_f16 multiplies them by an activation pair with float32 accumulation.
// The activation pairs are pre-permuted to match: for 4-bit, word w pairs columns (8w+j, 8w+j+4),
// j = 0..3; for 2-bit, (16w+j, 16w+j+8), j = 0..7.
//
// Per group the dot product is regrouped as  sum_j (c_j s + b) x_j = s sum_j c_j x_j + b sum_j x_j
// (the FMA rewrite of "nibble * scale + bias" in the Metal dequant listing of "Inferencia de LLM
// MoE en MacBook Pro: Streaming de Expertos desde SSD con Metal", section "Arquitectura del
// Sistema"), so scale and bias cost two FMAs per half segment instead of one per weight.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <tuple>
#include <utility>

namespace moe {

// Enqueue kernel `k` and return the status of this launch alone.  (hipGetLastError would also
// report errors other runtime users left behind, such as hipErrorNotReady from event queries.)
template <typename... KArgs, typename... Args>
inline hipError_t launch(void (*k)(KArgs...), dim3 grid, dim3 block, size_t shmem, hipStream_t s,
                         Args&&... args) {
  std::tuple<KArgs...> held(std::forward<Args>(args)...);
  void* argv[sizeof...(KArgs) > 0 ? sizeof...(KArgs) : 1];
  std::apply([&argv](auto&... a) {
    int i = 0;
    ((argv[i++] = (void*)&a), ...);
  }, held);
  return hipLaunchKernel((const void*)k, grid, block, argv, shmem, s);
}

inline hipError_t first_error(hipError_t a, hipError_t b) { return a != hipSuccess ? a : b; }

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));

constexpr int WAVE = 64;
constexpr float RMS_EPS = 1e-6f;

__device__ __forceinline__ float h2f(uint16_t b) { return (float)__builtin_bit_cast(_Float16, b); }
__device__ __forceinline__ uint16_t f2h(float v) { return __builtin_bit_cast(uint16_t, (_Float16)v); }
__device__ __forceinline__ half2_t as_h2(uint32_t v) { return __builtin_bit_cast(half2_t, v); }

// xor-butterfly sum over aligned groups of `width` lanes (power of two <= 64); every lane of a
// group ends with the group's sum, always added in the same order.
__device__ __forceinline__ float group_sum(float v, int width) {
  for (int m = width >> 1; m > 0; m >>= 1) v += __shfl_xor(v, m, WAVE);
  return v;
}

__device__ __forceinline__ float quiet_nan() { return __builtin_nanf(""); }

// Unsigned max over the 64 lanes of a wave with DPP moves (no LDS round trip): prefix max inside
// each row of 16 lanes (row_shr 1, 2, 4, 8), then row_bcast15 / row_bcast31 carry it across
// rows; lane 63 ends with the wave max, which readlane broadcasts.  Lanes whose DPP source is
// out of range keep their own value (the `old` operand), which is neutral for max.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint32_t dpp_max_step(uint32_t x) {
  const uint32_t o = (uint32_t)__builtin_amdgcn_update_dpp((int)x, (int)x, CTRL, ROW_MASK, 0xf, false);
  return o > x ? o : x;
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = dpp_max_step<0x111, 0xf>(v);  // row_shr:1
  v = dpp_max_step<0x112, 0xf>(v);  // row_shr:2
  v = dpp_max_step<0x114, 0xf>(v);  // row_shr:4
  v = dpp_max_step<0x118, 0xf>(v);  // row_shr:8
  v = dpp_max_step<0x142, 0xa>(v);  // row_bcast:15 into rows 1 and 3
  v = dpp_max_step<0x143, 0xc>(v);  // row_bcast:31 into rows 2 and 3
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

// ---------------------------------------------------------------------------------------------
// Segment geometry per code width.
// Workgroup barrier that orders LDS only: outstanding global loads stay in flight across it
// (a plain __syncthreads would wait for them).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

template <int BITS>
struct SegT;
template <>
struct SegT<4> {
  static constexpr int COLS = 32;    // columns per 16-byte segment
  static constexpr int PAIRS = 16;   // activation pairs per segment
  static constexpr int PAIRS_PER_WORD = 4;
};
template <>
struct SegT<2> {
  static constexpr int COLS = 64;
  static constexpr int PAIRS = 32;
  static constexpr int PAIRS_PER_WORD = 8;
};

// Build the permuted activation pairs of one segment from a float16 row (32 or 64 columns
// starting at `xs`, 16-byte aligned).  Also returns sum x over each half segment and sum x^2.
template <int BITS>
__device__ __forceinline__ void load_xpairs(const uint16_t* __restrict__ xs, uint32_t* xp, float* sx,
                                            float& sq) {
  const uint4* p = reinterpret_cast<const uint4*>(xs);
  if constexpr (BITS == 4) {
#pragma unroll
    for (int w = 0; w < 4; ++w) {  // word w: columns 8w..8w+7 = one uint4 of halves
      uint4 u = p[w];
      xp[w * 4 + 0] = (u.x & 0xFFFFu) | (u.z << 16);
      xp[w * 4 + 1] = (u.x >> 16) | (u.z & 0xFFFF0000u);
      xp[w * 4 + 2] = (u.y & 0xFFFFu) | (u.w << 16);
      xp[w * 4 + 3] = (u.y >> 16) | (u.w & 0xFFFF0000u);
    }
  } else {
#pragma unroll
    for (int w = 0; w < 4; ++w) {  // word w: columns 16w..16w+15 = two uint4 of halves
      uint4 a = p[2 * w], b = p[2 * w + 1];
      uint32_t av[4] = {a.x, a.y, a.z, a.w}, bv[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        uint32_t lo = (j & 1) ? (av[j >> 1] >> 16) : (av[j >> 1] & 0xFFFFu);
        uint32_t hi = (j & 1) ? (bv[j >> 1] & 0xFFFF0000u) : (bv[j >> 1] << 16);
        xp[w * 8 + j] = lo | hi;
      }
    }
  }
  const half2_t one = {(_Float16)1.0f, (_Float16)1.0f};
  float s0 = 0.f, s1 = 0.f, q = 0.f;
  constexpr int HP = SegT<BITS>::PAIRS / 2;
#pragma unroll
  for (int i = 0; i < SegT<BITS>::PAIRS; ++i) {
    half2_t v = as_h2(xp[i]);
    if (i < HP)
      s0 = __builtin_amdgcn_fdot2(v, one, s0, false);
    else
      s1 = __builtin_amdgcn_fdot2(v, one, s1, false);
    q = __builtin_amdgcn_fdot2(v, v, q, false);
  }
  sx[0] = s0;
  sx[1] = s1;
  sq += q;
}

// acc + sum_j w_j (g_j x_j) over eight float16 columns, in float32: the product g_j x_j of two
// float16 values is exact in float32, so a gained input loses nothing before the weight.
__device__ __forceinline__ float dot8_gained(uint4 w, uint4 x, uint4 g, float acc) {
  const uint32_t wv[4] = {w.x, w.y, w.z, w.w}, xv[4] = {x.x, x.y, x.z, x.w}, gv[4] = {g.x, g.y, g.z, g.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const half2_t a = as_h2(wv[i]), b = as_h2(xv[i]), c = as_h2(gv[i]);
    acc = fmaf((float)a[0], (float)b[0] * (float)c[0], acc);
    acc = fmaf((float)a[1], (float)b[1] * (float)c[1], acc);
  }
  return acc;
}

// sq + sum of x^2 over N float16 values (16-byte aligned, N a multiple of 8), in a fixed order.
template <int N>
__device__ __forceinline__ float sum_sq(const uint16_t* __restrict__ xs, float sq) {
#pragma unroll
  for (int i = 0; i < N / 8; ++i) {
    const uint4 v = reinterpret_cast<const uint4*>(xs)[i];
    sq = __builtin_amdgcn_fdot2(as_h2(v.x), as_h2(v.x), sq, false);
    sq = __builtin_amdgcn_fdot2(as_h2(v.y), as_h2(v.y), sq, false);
    sq = __builtin_amdgcn_fdot2(as_h2(v.z), as_h2(v.z), sq, false);
    sq = __builtin_amdgcn_fdot2(as_h2(v.w), as_h2(v.w), sq, false);
  }
  return sq;
}

// sum_j c_j x_j over the two half segments (words 0-1 and words 2-3) of one 16-byte segment.
template <int BITS>
__device__ __forceinline__ void dot_segment(uint4 q, const uint32_t* xp, float& d0, float& d1) {
  const uint32_t w[4] = {q.x, q.y, q.z, q.w};
  const half2_t k1024 = {(_Float16)1024.0f, (_Float16)1024.0f};
  constexpr int PPW = SegT<BITS>::PAIRS_PER_WORD;
  constexpr uint32_t MASK = BITS == 4 ? 0x000F000Fu : 0x00030003u;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int j = 0; j < PPW; ++j) {
      uint32_t t = ((w[i] >> (BITS * j)) & MASK) | 0x64006400u;
      half2_t c = as_h2(t) - k1024;
      if (i < 2)
        d0 = __builtin_amdgcn_fdot2(c, as_h2(xp[i * PPW + j]), d0, false);
      else
        d1 = __builtin_amdgcn_fdot2(c, as_h2(xp[i * PPW + j]), d1, false);
    }
  }
}

// Float32 activations as two float16 parts, hi = fp16(x) and lo = fp16(x - hi) (x ~ hi + lo to
// about 22 significant bits), in the same permuted pair order as load_xpairs.  sx gets the float32
// sum of each half segment.
template <int BITS>
__device__ __forceinline__ void load_xpairs_f32(const float* __restrict__ xs, uint32_t* hp, uint32_t* lp, float* sx) {
  constexpr int PPW = SegT<BITS>::PAIRS_PER_WORD;
  constexpr int CPW = 32 / BITS;  // columns per word
  float s[2] = {0.f, 0.f};
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    float v[CPW];
#pragma unroll
    for (int c = 0; c < CPW; c += 4) {
      const float4 f = *reinterpret_cast<const float4*>(xs + w * CPW + c);
      v[c] = f.x;
      v[c + 1] = f.y;
      v[c + 2] = f.z;
      v[c + 3] = f.w;
    }
#pragma unroll
    for (int j = 0; j < PPW; ++j) {
      const float a = v[j], b = v[j + PPW];
      const _Float16 ha = (_Float16)a, hb = (_Float16)b;
      const _Float16 la = (_Float16)(a - (float)ha), lb = (_Float16)(b - (float)hb);
      hp[w * PPW + j] = (uint32_t)__builtin_bit_cast(uint16_t, ha) | ((uint32_t)__builtin_bit_cast(uint16_t, hb) << 16);
      lp[w * PPW + j] = (uint32_t)__builtin_bit_cast(uint16_t, la) | ((uint32_t)__builtin_bit_cast(uint16_t, lb) << 16);
    }
#pragma unroll
    for (int c = 0; c < CPW; ++c) s[w >> 1] += v[c];
  }
  sx[0] = s[0];
  sx[1] = s[1];
}

// sum_j c_j (hi_j + lo_j) over the two half segments: the code pairs are decoded once and meet
// both activation parts.
template <int BITS>
__device__ __forceinline__ void dot_segment_split(uint4 q, const uint32_t* hp, const uint32_t* lp, float& d0,
                                                  float& d1) {
  const uint32_t w[4] = {q.x, q.y, q.z, q.w};
  const half2_t k1024 = {(_Float16)1024.0f, (_Float16)1024.0f};
  constexpr int PPW = SegT<BITS>::PAIRS_PER_WORD;
  constexpr uint32_t MASK = BITS == 4 ? 0x000F000Fu : 0x00030003u;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int j = 0; j < PPW; ++j) {
      const half2_t c = as_h2(((w[i] >> (BITS * j)) & MASK) | 0x64006400u) - k1024;
      float& d = i < 2 ? d0 : d1;
      d = __builtin_amdgcn_fdot2(c, as_h2(hp[i * PPW + j]), d, false);
      d = __builtin_amdgcn_fdot2(c, as_h2(lp[i * PPW + j]), d, false);
    }
  }
}

// The same dot products with the codes left biased: the exponent trick decodes a code pair to
// 1024 + q exactly, and dotting that directly gives sum (1024 + q) x = sum q x + 1024 sum x.  The
// caller folds the 1024 into the group bias, s * d' + (b - 1024 s) * sum x, which saves the float16
// subtract of every pair.
template <int BITS>
__device__ __forceinline__ void dot_segment_biased(uint4 q, const uint32_t* xp, float& d0, float& d1) {
  const uint32_t w[4] = {q.x, q.y, q.z, q.w};
  constexpr int PPW = SegT<BITS>::PAIRS_PER_WORD;
  constexpr uint32_t MASK = BITS == 4 ? 0x000F000Fu : 0x00030003u;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int j = 0; j < PPW; ++j) {
      const half2_t c = as_h2(((w[i] >> (BITS * j)) & MASK) | 0x64006400u);
      float& d = i < 2 ? d0 : d1;
      d = __builtin_amdgcn_fdot2(c, as_h2(xp[i * PPW + j]), d, false);
    }
  }
}
template <int BITS>
__device__ __forceinline__ void dot_segment_split_biased(uint4 q, const uint32_t* hp, const uint32_t* lp, float& d0,
                                                         float& d1) {
  const uint32_t w[4] = {q.x, q.y, q.z, q.w};
  constexpr int PPW = SegT<BITS>::PAIRS_PER_WORD;
  constexpr uint32_t MASK = BITS == 4 ? 0x000F000Fu : 0x00030003u;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int j = 0; j < PPW; ++j) {
      const half2_t c = as_h2(((w[i] >> (BITS * j)) & MASK) | 0x64006400u);
      float& d = i < 2 ? d0 : d1;
      d = __builtin_amdgcn_fdot2(c, as_h2(hp[i * PPW + j]), d, false);
      d = __builtin_amdgcn_fdot2(c, as_h2(lp[i * PPW + j]), d, false);
    }
  }
}

}  // namespace moe
