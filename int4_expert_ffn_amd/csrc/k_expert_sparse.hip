// ReLU activation-sparse down projection of the decode path on gfx950.
//
// "Arquitecturas nativas para device: MoE de grano fino y pre-attention router", section "Dos
// niveles de sparsity" (level 2, sparse FFN): with a ReLU-type nonlinearity every intermediate
// neuron whose gate is not positive outputs exactly zero, and its weights need be neither read
// nor multiplied.  The gate/up kernel of the dense path computes a = relu(gate) * up; here the
// down projection reads only the rows of neurons with a != 0.  The down matrix is stored
// neuron-major ([E][I][d], quantisation groups along d), so one neuron is one contiguous packed
// row and a skipped neuron is a skipped row of bytes.  Its scales and biases are stored
// group-major ([E][d/group][I]): a block's column slab lies in one or two groups, so the scales
// it reads sit in a short run of lines that no block of another XCD touches (row-major scales put
// every XCD's few bytes of a row in the same line, and each XCD fetched that line).
//
// Mapping.  Block (slab, k, t) owns SLAB output columns of o_tk.  It lists the active neurons of
// expert e = idx[t][k] (a != 0, ascending) in LDS from act[t][k][:] with wave ballots, then its
// four waves walk the list: a row's share of the slab is two 16-byte segments on two lanes, so a
// wave covers 32 rows per load and every lane keeps four rows' loads in flight.  A lane
// accumulates alpha * scale * code over its 32 (int4) or 64 (int2) columns in float32, and the
// alpha * bias term once per row and group.  The 128 partial rows of the slab are folded in
// pairs across the wave's halves, then summed through LDS, all in a fixed order, so results are
// reproducible run to run.  o_tk is stored; with the fused
// output, the last of the K blocks of a (token, slab), found with a device-scope counter, forms
// y = r + sum_k w_k o_tk over the slab in ascending k, the arithmetic of the combine kernel.
//
// Slabs that share 128-byte lines of a row go to blocks of one XCD (blocks are dealt to the XCDs
// round robin), so each line is fetched into one L2.
#include "moe_device.h"
#include "moe_launch.h"

namespace moe {
namespace {

constexpr int SP_WAVES = 4;
constexpr int SP_THREADS = SP_WAVES * WAVE;
constexpr int SP_LPR = 2;                           // lanes per row of a slab (16 bytes each)
constexpr int SP_SLOTS = SP_THREADS / SP_LPR;       // rows per block-wide load
constexpr int SP_HALF = SP_SLOTS / 2;               // partial rows left after the in-wave fold
constexpr int SP_NB = 4;                            // row loads in flight per lane
constexpr int SP_PAD = 4;                           // LDS row padding (floats) of the partial sums
constexpr int SP_MISC = 16;                         // LDS ints: wave counts, last-block flag

template <int BITS>
struct SpT {
  static constexpr int COLS = 128 / BITS;           // columns of one 16-byte segment
  static constexpr int SLAB = SP_LPR * COLS;        // columns per block
  static constexpr int RS = SLAB + SP_PAD;          // LDS stride of a partial row
  static constexpr int PARTS = SP_THREADS / SLAB;   // threads per column in the LDS sum
};

struct SpK {
  int K, E, d, I, lg2g, nslab;
  const float* act;      // [T][K][I]
  const int32_t* idx;    // [T][K]
  moe_qmat down;         // neuron-major: q [E][I][d*BITS/32]; scales / biases group-major, [E][d/group][I]
  float* o;              // [T][K][d]
  const float* wf;       // [T][K] or nullptr (no fused output)
  const uint16_t* rf;    // [T][d]
  uint16_t* yf;          // [T][d]
  int32_t* cnt;          // [T][nslab]
  int32_t* n_active;     // [T][K] or nullptr
};

template <int BITS>
size_t sp_lds_bytes(int I) {
  using G = SpT<BITS>;
  return (size_t)SP_HALF * G::RS * 4 + (size_t)SP_THREADS * 4 + SP_MISC * 4 + (size_t)I * 4 + (size_t)I * 2;
}

__device__ __forceinline__ void st_coherent(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_coherent(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int BITS, bool SPLIT>
__global__ void __launch_bounds__(SP_THREADS) k_down_sparse(SpK p) {
  using G = SpT<BITS>;
  extern __shared__ __align__(16) unsigned char smem[];
  float* red = reinterpret_cast<float*>(smem);                  // [SP_HALF][RS]
  float* red2 = red + SP_HALF * G::RS;                          // [PARTS][SLAB]
  int* misc = reinterpret_cast<int*>(red2 + SP_THREADS);        // [SP_MISC]
  float* list_a = reinterpret_cast<float*>(misc + SP_MISC);     // [I]
  uint16_t* list_i = reinterpret_cast<uint16_t*>(list_a + p.I); // [I]

  const int tid = threadIdx.x, lane = tid % WAVE, w = tid / WAVE;
  const int bx = blockIdx.x, k = blockIdx.y, t = blockIdx.z;
  const int slab = (p.nslab % 8 == 0) ? (bx % 8) * (p.nslab / 8) + bx / 8 : bx;
  int e = p.idx[(size_t)t * p.K + k];
  const bool bad = (unsigned)e >= (unsigned)p.E;
  if (bad) e = 0;

  // 1. the active neurons, ascending: each wave counts a contiguous range, then writes its
  //    entries after those of the waves before it
  const float* at = p.act + ((size_t)t * p.K + k) * p.I;
  const int per = (p.I + SP_THREADS - 1) / SP_THREADS * WAVE;
  const int i0 = w * per, i1 = min(p.I, i0 + per);
  int n_w = 0;
  for (int b = i0; b < i1; b += WAVE) {
    const int i = b + lane;
    const bool on = i < i1 && at[i] != 0.f;   // a NaN counts as active: it must reach the output
    n_w += __popcll(__ballot(on));
  }
  if (lane == 0) misc[w] = n_w;
  __syncthreads();
  int base = 0, n = 0;
#pragma unroll
  for (int v = 0; v < SP_WAVES; ++v) {
    const int c = misc[v];
    base += v < w ? c : 0;
    n += c;
  }
  for (int b = i0; b < i1; b += WAVE) {
    const int i = b + lane;
    const float a = i < i1 ? at[i] : 0.f;
    const bool on = a != 0.f;
    const uint64_t m = __ballot(on);
    if (on) {
      const int pos = base + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                                            __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
      list_a[pos] = a;
      list_i[pos] = (uint16_t)i;
    }
    base += __popcll(m);
  }
  __syncthreads();

  // 2. the listed rows' slab segments: alpha * (scale * code + bias), float32
  const int ls = lane % SP_LPR, gs = w * (WAVE / SP_LPR) + lane / SP_LPR;
  const int wpr = p.d * BITS / 32, ngr = p.d >> p.lg2g;
  const int c0 = slab * G::SLAB + ls * G::COLS;
  const uint32_t* qe = p.down.q + (size_t)e * p.I * wpr + (size_t)c0 * BITS / 32;
  const int ga = c0 >> p.lg2g, gb = (c0 + G::COLS / 2) >> p.lg2g;
  const size_t sga = ((size_t)e * ngr + ga) * p.I, sgb = ((size_t)e * ngr + gb) * p.I;
  float acc[G::COLS];
#pragma unroll
  for (int c = 0; c < G::COLS; ++c) acc[c] = 0.f;
  float bsa = 0.f, bsb = 0.f;
  for (int j0 = gs; j0 < n; j0 += SP_NB * SP_SLOTS) {
    uint4 q[SP_NB];
    uint16_t sa[SP_NB], ba[SP_NB], sb[SP_NB], bb[SP_NB];
    float al[SP_NB];
#pragma unroll
    for (int nb = 0; nb < SP_NB; ++nb) {   // past the list's end: reload its last row, weight 0
      const int j = j0 + nb * SP_SLOTS;
      const int jj = j < n ? j : n - 1;
      al[nb] = j < n ? list_a[jj] : 0.f;
      const size_t row = list_i[jj];
      q[nb] = *reinterpret_cast<const uint4*>(qe + row * wpr);
      sa[nb] = p.down.scales[sga + row];
      ba[nb] = p.down.biases[sga + row];
      if (SPLIT) {
        sb[nb] = p.down.scales[sgb + row];
        bb[nb] = p.down.biases[sgb + row];
      }
    }
#pragma unroll
    for (int nb = 0; nb < SP_NB; ++nb) {
      const float asa = al[nb] * h2f(sa[nb]);
      bsa = fmaf(al[nb], h2f(ba[nb]), bsa);
      float asb = asa;
      if (SPLIT) {
        asb = al[nb] * h2f(sb[nb]);
        bsb = fmaf(al[nb], h2f(bb[nb]), bsb);
      }
      const uint32_t wv[4] = {q[nb].x, q[nb].y, q[nb].z, q[nb].w};
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const float sc = (SPLIT && m >= 2) ? asb : asa;
        if (BITS == 4) {   // word m: columns 8m..8m+7; byte b holds 8m+2b (low nibble), 8m+2b+1
          const uint32_t lo = wv[m] & 0x0F0F0F0Fu, hi = (wv[m] >> 4) & 0x0F0F0F0Fu;
#pragma unroll
          for (int b = 0; b < 4; ++b) {
            acc[8 * m + 2 * b] = fmaf(sc, (float)((lo >> (8 * b)) & 0xFFu), acc[8 * m + 2 * b]);
            acc[8 * m + 2 * b + 1] = fmaf(sc, (float)((hi >> (8 * b)) & 0xFFu), acc[8 * m + 2 * b + 1]);
          }
        } else {           // word m: columns 16m..16m+15; byte b holds 16m+4b .. 16m+4b+3
#pragma unroll
          for (int sh = 0; sh < 4; ++sh) {
            const uint32_t v = (wv[m] >> (2 * sh)) & 0x03030303u;
#pragma unroll
            for (int b = 0; b < 4; ++b)
              acc[16 * m + 4 * b + sh] = fmaf(sc, (float)((v >> (8 * b)) & 0xFFu), acc[16 * m + 4 * b + sh]);
          }
        }
      }
    }
  }

  // 3. sum the partial rows of the slab in a fixed order.  First lanes l and l + 32 (same columns,
  //    different rows) fold their halves: the lower lane keeps the first half of the segment's
  //    columns, the upper lane the second.  Then the 64 half-rows go through LDS.
  const bool upper = lane >= WAVE / 2;
  float hv[G::COLS / 2];
#pragma unroll
  for (int c = 0; c < G::COLS / 2; ++c) {
    const float lo = acc[c] + bsa;
    const float hi = acc[c + G::COLS / 2] + (SPLIT ? bsb : bsa);
    const float got = __shfl_xor(upper ? lo : hi, WAVE / 2);
    hv[c] = (upper ? hi : lo) + got;
  }
  const int hs = w * (WAVE / SP_LPR / 2) + (lane / SP_LPR) % (WAVE / SP_LPR / 2);
  float* rr = red + hs * G::RS + ls * G::COLS + (upper ? G::COLS / 2 : 0);
#pragma unroll
  for (int c = 0; c < G::COLS / 2; c += 4)
    *reinterpret_cast<float4*>(rr + c) = make_float4(hv[c], hv[c + 1], hv[c + 2], hv[c + 3]);
  __syncthreads();
  {
    constexpr int PER = SP_HALF / G::PARTS;
    const int c = tid % G::SLAB, part = tid / G::SLAB;
    float s = 0.f;
    for (int j = 0; j < PER; ++j) s += red[(part * PER + j) * G::RS + c];
    red2[part * G::SLAB + c] = s;
  }
  __syncthreads();
  const int col = slab * G::SLAB + tid;
  if (tid < G::SLAB) {
    float o = 0.f;
#pragma unroll
    for (int part = 0; part < G::PARTS; ++part) o += red2[part * G::SLAB + tid];
    if (bad) o = quiet_nan();
    st_coherent(p.o + ((size_t)t * p.K + k) * p.d + col, o);
  }
  if (p.n_active && slab == 0 && tid == 0) p.n_active[(size_t)t * p.K + k] = bad ? -1 : n;

  // 4. fused combine by the last of the token's K blocks on this slab.  The o stores above and the
  //    loads below are agent-scope atomic accesses, coherent across the XCDs' L2s by themselves;
  //    waiting for the stores' completion before the counter's atomic add orders them.  (A full
  //    device fence would write back and invalidate the whole L2 instead, several microseconds.)
  if (p.wf) {
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): this thread's stores have completed
    __syncthreads();
    if (tid == 0) misc[SP_WAVES] = atomicAdd(&p.cnt[(size_t)t * p.nslab + slab], 1) == p.K - 1;
    __syncthreads();
    if (misc[SP_WAVES] && tid < G::SLAB) {
      float y = 0.f;
      for (int kk = 0; kk < p.K; ++kk)
        y = fmaf(p.wf[(size_t)t * p.K + kk], ld_coherent(p.o + ((size_t)t * p.K + kk) * p.d + col), y);
      p.yf[(size_t)t * p.d + col] = f2h(h2f(p.rf[(size_t)t * p.d + col]) + y);
    }
  }
}

template <int BITS, bool SPLIT>
hipError_t go(hipStream_t s, const SparseArgs& a, int nslab, int lg2g) {
  const DecodeArgs& b = a.base;
  SpK p{b.K, b.E, b.d, b.I, lg2g, nslab, (const float*)b.act, b.idx, b.ex.down, a.o,
        b.y_fuse ? b.w_fuse : nullptr, b.r_fuse, b.y_fuse, a.cnt, a.n_active};
  return launch(k_down_sparse<BITS, SPLIT>, dim3(nslab, b.K, b.T), dim3(SP_THREADS), sp_lds_bytes<BITS>(b.I), s, p);
}

int ilog2i(int v) {
  int r = 0;
  while ((1 << r) < v) ++r;
  return r;
}

}  // namespace

int sparse_slabs(int bits, int d) {
  const int slab = bits == 4 ? SpT<4>::SLAB : SpT<2>::SLAB;
  return (d % slab == 0) ? d / slab : 0;
}

size_t sparse_lds(int bits, int I) { return bits == 4 ? sp_lds_bytes<4>(I) : sp_lds_bytes<2>(I); }

hipError_t launch_down_sparse(hipStream_t s, const SparseArgs& a) {
  const DecodeArgs& b = a.base;
  const int nslab = sparse_slabs(b.bits, b.d);
  const int lg2g = ilog2i(b.group);
  if (b.bits == 4) return go<4, false>(s, a, nslab, lg2g);
  if (b.group < SpT<2>::COLS) return go<2, true>(s, a, nslab, lg2g);
  return go<2, false>(s, a, nslab, lg2g);
}

}  // namespace moe
