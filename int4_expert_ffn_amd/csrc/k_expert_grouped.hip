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
// MFMA mapping (gfx950's v_mfma_f32_16x16x32_f16): A = 16 token rows x 32 columns, B = 32 columns
// x 16 weight rows, D = 16 tokens x 16 weight rows in float32.  A wave owns 16 weight rows; lane
// (n = lane % 16, q = lane / 16) loads one 16-byte segment of row n (32 int4 / 64 int2 columns,
// segment q of a 4-segment macro step) and dequantises it once to float16 pairs
// w = fma(code, scale, bias).  MFMA step s takes the lane's pairs 4s .. 4s+3; the token rows
// are staged in LDS with columns permuted inside each 8 (int4) or 16 (int2) column block so the
// same four columns sit next to each other, so A is two 8-byte LDS reads.  Which physical column
// feeds which k slot does not matter to the dot product as long as A and B agree.
#include "moe_device.h"
#include "moe_launch.h"
#include "moe_lora.h"

namespace moe {
namespace {


// ------------------------------------------------------------------------------------- sort
constexpr int MT = 16;  // token rows per MFMA tile
// Work-list record of one tile: bucket, first sorted position inside the bucket, the bucket's
// start in perm and its pair count, then the tile's MT pair indices (-1 past the bucket's end).
// A GEMM block reads everything it needs before its first weight and activation loads from this
// one record, instead of a chain of dependent loads (bucket -> offsets -> perm -> activations).
constexpr int TREC = 4 + MT;

constexpr int SORT_THREADS = 1024, SORT_WAVES = SORT_THREADS / WAVE;

// Inclusive prefix sum over the 64 lanes with DPP moves: row_shr 1, 2, 4, 8 inside each row of 16
// lanes, then row_bcast15 / row_bcast31 carry the row totals into the rows after them.  A lane
// whose DPP source is out of range, or whose row is masked off, adds the `old` operand, 0.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ int dpp_add_step(int x) {
  return x + __builtin_amdgcn_update_dpp(0, x, CTRL, ROW_MASK, 0xf, false);
}
__device__ __forceinline__ int wave_incl_sum(int v) {
  v = dpp_add_step<0x111, 0xf>(v);  // row_shr:1
  v = dpp_add_step<0x112, 0xf>(v);  // row_shr:2
  v = dpp_add_step<0x114, 0xf>(v);  // row_shr:4
  v = dpp_add_step<0x118, 0xf>(v);  // row_shr:8
  v = dpp_add_step<0x142, 0xa>(v);  // row_bcast:15 into rows 1 and 3
  v = dpp_add_step<0x143, 0xc>(v);  // row_bcast:31 into rows 2 and 3
  return v;
}

// The lanes of `live` whose key equals this lane's (keys below 2^nbits), one ballot per key bit.
__device__ __forceinline__ uint64_t match_lanes(int key, int nbits, uint64_t live) {
  uint64_t m = live;
  for (int b = 0; b < nbits; ++b) {
    const bool s = (key >> b) & 1;
    const uint64_t bb = __ballot(s);
    m &= s ? bb : ~bb;
  }
  return m;
}

// rowscale[t] = 1 / sqrt(mean(x_t^2) + eps) of token row t (row length d), by one wave.
__device__ __forceinline__ void rowscale_wave(int t, int d, const uint16_t* __restrict__ x, float* __restrict__ rowscale,
                                              int lane) {
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

// Work that needs no sorted order, done beside the sort: the adapter's A . x, the RMS-norm factors
// of the token rows (rowscale null: none) and clearing nzero ints at zero (the GEMMs' tile counts).
struct SortSideJobs {
  LoraAJob lora;
  int T, d;
  const uint16_t* x;
  float* rowscale;
  int32_t* zero;
  int nzero;
  __host__ __device__ int waves() const {
    return lora.waves() + (rowscale ? T : 0) + (zero ? (nzero + WAVE - 1) / WAVE : 0);
  }
};


// Block 0 (SORT_THREADS threads) sorts.  counts[E+1], offsets[E+2] (bucket E collects indices
// outside [0, E)), perm[T*K]: pair indices grouped by expert, ascending inside each expert.  tiles
// (may be null): the grouped GEMMs' work list, tiles[0] = number of tiles, then one TREC-int record
// per MT-row tile, buckets in order.  Blocks 1, 2, ... run `side` on the compute units the sort
// leaves idle, SORT_WAVES waves each.
//
// A pair's position in its bucket is the number of earlier pairs with the same bucket: those of
// earlier chunks of SORT_THREADS pairs, of earlier waves of its chunk (per-wave counts prefixed over
// the waves) and of earlier lanes of its wave (the lanes with an equal bucket, found by ballots over
// the bucket's bits).  The lowest lane of each such set of lanes writes the wave's count, so no
// atomic ever serialises the lanes of one bucket.  The barriers order LDS only: no step reads what
// another thread stored to global memory, so no barrier waits for the stores of perm and tiles.
__global__ void __launch_bounds__(SORT_THREADS) k_sort(int TK, int E, const int32_t* __restrict__ idx,
                                                      int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
                                                      int32_t* __restrict__ perm, int32_t* __restrict__ tiles,
                                                      int max_tiles, int TS, SortSideJobs side) {
  if (blockIdx.x > 0) {
    const int wv = (blockIdx.x - 1) * SORT_WAVES + threadIdx.x / WAVE, nl = side.lora.waves();
    const int nr = side.rowscale ? side.T : 0, lane = threadIdx.x % WAVE;
    if (wv < nl)
      lora_a_wave(side.lora, wv, lane);
    else if (wv - nl < nr)
      rowscale_wave(wv - nl, side.d, side.x, side.rowscale, lane);
    else if (side.zero && (wv - nl - nr) * WAVE + lane < side.nzero)
      side.zero[(wv - nl - nr) * WAVE + lane] = 0;
    return;
  }
  // TS > 0: pairs TK .. TK + TS - 1 form one more bucket, E + 1 (a shared expert's, one per token)
  const int NB = E + 1 + (TS > 0 ? 1 : 0), LB = NB - 1;  // buckets, the last one
  extern __shared__ int sh[];
  int* cnt = sh;               // [NB] pairs of each bucket
  int* run = cnt + NB;         // [NB] pairs placed by earlier chunks
  int* offs = run + NB;        // [NB+1] first position of each bucket in perm
  int* toff = offs + NB + 1;   // [NB+1] first tile of each bucket
  int* ctot = toff + NB + 1;   // [NB] pairs of each bucket in the current chunk
  int* hist = ctot + NB;       // [SORT_WAVES][NB] per-wave counts of a chunk, then their prefixes
  const int tid = threadIdx.x, lane = tid % WAVE, w = tid / WAVE;
  const int nbits = 32 - __clz(LB);           // every bucket number fits in nbits bits
  const uint64_t below = (1ull << lane) - 1;  // the lanes before this one
  const auto bucket = [&](int p) {  // of routed pair p < TK
    const int e = idx[p];
    return (unsigned)e >= (unsigned)E ? E : e;
  };
  // the first chunk's buckets, loaded before the LDS set-up so that the load's latency overlaps it
  int e0 = tid < TK ? bucket(tid) : 0;
  uint64_t m0 = 0;  // the first chunk's match mask, kept for its placement
  for (int i = tid; i <= LB; i += SORT_THREADS) {
    cnt[i] = (TS > 0 && i == LB) ? TS : 0;  // the shared bucket: TS pairs
    run[i] = 0;
  }
  for (int i = tid; i < SORT_WAVES * NB; i += SORT_THREADS) hist[i] = 0;
  lds_barrier();
  for (int base = 0; base < TK; base += SORT_THREADS) {
    const int p = base + tid;
    const int e = base == 0 ? e0 : p < TK ? bucket(p) : 0;
    const uint64_t m = match_lanes(e, nbits, __ballot(p < TK));
    if (p < TK && (m & below) == 0) atomicAdd(&cnt[e], __popcll(m));
    if (base == 0) m0 = m;
  }
  lds_barrier();
  // exclusive scans of the pair and tile counts over the buckets, by wave 0: each lane sums a run
  // of consecutive buckets, one wave scan joins the runs
  if (w == 0) {
    const int per = (NB + WAVE - 1) / WAVE, b_lo = min(lane * per, NB), b_hi = min(b_lo + per, NB);
    int c = 0, t = 0;
    for (int b = b_lo; b < b_hi; ++b) {
      const int n = cnt[b];
      c += n;
      t += (n + MT - 1) / MT;
    }
    const int ci = wave_incl_sum(c), ti = wave_incl_sum(t);
    // the shared bucket's tiles go first in the work list (its weights are the same for every
    // tile, so they come from the caches, and the list's tail is left to HBM tiles)
    const int ts = TS > 0 ? (TS + MT - 1) / MT : 0;
    int ce = ci - c, te = ti - t;
    for (int b = b_lo; b < b_hi; ++b) {
      const int n = cnt[b];
      offs[b] = ce;
      toff[b] = TS > 0 && b == LB ? 0 : te + ts;
      ce += n;
      te += (n + MT - 1) / MT;
    }
    if (lane == WAVE - 1) {
      offs[NB] = ci;
      toff[NB] = ti;
    }
  }
  lds_barrier();
  for (int i = tid; i <= NB; i += SORT_THREADS) {
    offsets[i] = offs[i];
    if (i <= LB) counts[i] = cnt[i];
  }
  if (tiles != nullptr && tid == 0) tiles[0] = min(toff[NB], max_tiles);
  // pair p at position q of bucket e: its perm entry and its row of the tile's record; a tile's
  // first pair also writes the record's header, the bucket's last pair the padding rows after it
  const auto place = [&](int e, int q, int p) {
    perm[offs[e] + q] = p;
    const int k = toff[e] + q / MT;
    if (tiles == nullptr || k >= max_tiles) return;
    int32_t* rec = tiles + 1 + (size_t)TREC * k;
    rec[4 + q % MT] = p;
    if (q % MT == 0) {
      rec[0] = e;
      rec[1] = q;
      rec[2] = offs[e];
      rec[3] = cnt[e];
    }
    if (q == cnt[e] - 1)
      for (int i = q % MT + 1; i < MT; ++i) rec[4 + i] = -1;
  };
  // The shared bucket's pairs keep their order: pair TK + q is its q-th.
  for (int q = tid; q < TS; q += SORT_THREADS) place(LB, q, TK + q);
  for (int base = 0; base < TK; base += SORT_THREADS) {
    const int p = base + tid;
    int e = e0;
    uint64_t m = m0;
    if (base > 0) {
      e = p < TK ? bucket(p) : 0;
      m = match_lanes(e, nbits, __ballot(p < TK));
    }
    if (p < TK && (m & below) == 0) hist[w * NB + e] = __popcll(m);
    lds_barrier();
    for (int b = tid; b <= LB; b += SORT_THREADS) {  // exclusive prefix over the waves, per bucket
      int h[SORT_WAVES];
#pragma unroll
      for (int v = 0; v < SORT_WAVES; ++v) h[v] = hist[v * NB + b];
      int acc = 0;
#pragma unroll
      for (int v = 0; v < SORT_WAVES; ++v) {
        hist[v * NB + b] = acc;
        acc += h[v];
      }
      ctot[b] = acc;
    }
    lds_barrier();
    if (p < TK) place(e, run[e] + hist[w * NB + e] + __popcll(m & below), p);
    lds_barrier();
    for (int b = tid; b <= LB; b += SORT_THREADS) run[b] += ctot[b];
    for (int i = tid; i < SORT_WAVES * NB; i += SORT_THREADS) hist[i] = 0;
    lds_barrier();
  }
}

// ------------------------------------------------------------------------------------- MFMA core
constexpr int GW = 8;            // waves per block: GW x 16 weight rows
constexpr int XCH = 2048;        // columns of the token tile staged per LDS pass (d <= XCH: one pass)
// Staged rows are read 8 bytes per lane with the 16 lanes of a quad reading 16 different token
// rows: a row stride of 1 (mod 16) 8-byte bank slots, i.e. 4 (mod 64) halves, puts them in 16
// different slots, so a half-wave's read takes the minimum two passes (a stride of 10 slots put
// four lanes on each slot).
__host__ __device__ constexpr int lds_row_stride(int halves) { return halves + ((4 - halves) % 64 + 64) % 64; }
constexpr int XS = lds_row_stride(XCH);  // halves per staged row
constexpr int PF = 4;            // macro steps of weight segments in flight per wave
constexpr int PF64 = 4;          // the same for the lane-contiguous kernel (5 fits in 128 registers
                                 // but measured slower; deeper down prefetch gained nothing)

template <int BITS>
struct GSeg {
  static constexpr int COLS = SegT<BITS>::COLS;     // columns per lane segment
  static constexpr int MACRO = 4 * COLS;            // columns per macro step (4 lane quads)
  static constexpr int STEPS = SegT<BITS>::PAIRS / 2;  // MFMA steps per macro step
  static constexpr int PB = BITS == 4 ? 8 : 16;     // columns per permutation block
};

// Stage MT rows x `width` columns [c0, c0 + width) of the float16 matrix rows listed by `rows`
// (row < 0 = zero padding; columns at or past ncols are zero) into LDS, permuted per block so
// that each code pair's two activation columns are adjacent.
template <int BITS>
__device__ __forceinline__ void stage_rows(uint16_t* xs, const uint16_t* __restrict__ src, int ncols, int c0,
                                           int width, const int* rows) {
  constexpr int PB = GSeg<BITS>::PB;
  const int per_row = width / PB, units = MT * per_row;
  for (int u = threadIdx.x; u < units; u += blockDim.x) {
    const int m = u / per_row, cb = u % per_row;
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
    uint4* dst = reinterpret_cast<uint4*>(xs + m * XS + cb * PB);
    dst[0] = make_uint4(outw[0], outw[1], outw[2], outw[3]);
    if constexpr (PB == 16) dst[1] = make_uint4(outw[4], outw[5], outw[6], outw[7]);
  }
}

// One lane's weight segment of one macro step, for NMAT matrices: the 16 code bytes and the
// group scale/bias (two groups when a group is narrower than the segment).
template <int NMAT, bool SPLIT>
struct WStage {
  uint4 q[NMAT];
  uint16_t sa[NMAT], ba[NMAT], sb[NMAT], bb[NMAT];
};

// Load the segment starting at column `col` of weight row `row` (col is clamped into the row, so
// every issue is a valid load and the number of loads in flight never depends on the data).
template <int BITS, bool SPLIT, int NMAT>
__device__ __forceinline__ void issue_w(WStage<NMAT, SPLIT>& S, const moe_qmat* mats, size_t row, int wpr, int ngr,
                                        int lg2g, int ncols, int col) {
  constexpr int COLS = GSeg<BITS>::COLS;
  col = min(col, ncols - COLS);
  const size_t ga = row * ngr + (col >> lg2g);
#pragma unroll
  for (int mi = 0; mi < NMAT; ++mi) {
    S.q[mi] = *reinterpret_cast<const uint4*>(mats[mi].q + row * wpr + (size_t)col * BITS / 32);
    S.sa[mi] = mats[mi].scales[ga];
    S.ba[mi] = mats[mi].biases[ga];
    if constexpr (SPLIT) {
      const size_t gb = row * ngr + ((col + COLS / 2) >> lg2g);
      S.sb[mi] = mats[mi].scales[gb];
      S.bb[mi] = mats[mi].biases[gb];
    }
  }
}

// Dequantise a staged segment to float16 pairs w = fma(code, scale, bias), in the pair order
// the staged activations use (pair j of a word: codes j and j + PPW, one from each half); a
// segment past the row end (valid == false) gives zeros.  A code placed in the mantissa under
// the right exponent reads as (2^e + code) exactly: bits 0..1 / 0..3 under 1024, bits 2..3 under
// 256, bits 4..5 / 4..7 under 64, bits 6..7 under 16, so one mask-or and one subtract give the
// code as float16 with no shift for the lower byte of each half (and one shift per word for
// the upper byte).  mg[] holds the four magic words in registers, so the mask-or is one
// v_and_or_b32.
// One word of codes: its PPW pairs, with scale s and bias b (both halves of each).
template <int BITS>
__device__ __forceinline__ void dequant_word(uint32_t wd, half2_t s, half2_t b, const uint32_t* mg, uint32_t* w) {
  constexpr int PPW = SegT<BITS>::PAIRS_PER_WORD;
  const uint32_t lo = wd, hi = wd >> 8;
#pragma unroll
  for (int j = 0; j < PPW; ++j) {
    // pair j sits at bit BITS*j of each half: in the lower byte for j < PPW / 2
    const uint32_t src = j < PPW / 2 ? lo : hi;
    const int jb = j % (PPW / 2);  // position inside the byte, in codes
    const uint32_t mask = (BITS == 4 ? 0x000F000Fu : 0x00030003u) << (BITS * jb);
    const int m = BITS == 4 ? 2 * jb : jb;  // magic: 1024, 256, 64, 16 for shifts 0, 2, 4, 6 bits
    const half2_t c = as_h2((src & mask) | mg[m]);
    const _Float16 base = (_Float16)(1024 >> (2 * m));
    const half2_t k = {base, base};
    w[j] = __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(c - k, s, b));
  }
}

template <int BITS, bool SPLIT>
__device__ __forceinline__ void dequant_stage(uint4 q, uint16_t sa16, uint16_t ba16, uint16_t sb16, uint16_t bb16,
                                              bool valid, const uint32_t* mg, uint32_t* w) {
  constexpr int PPW = SegT<BITS>::PAIRS_PER_WORD;
  if (!SPLIT) {
    sb16 = sa16;
    bb16 = ba16;
  }
  const _Float16 sa = __builtin_bit_cast(_Float16, (uint16_t)(valid ? sa16 : 0)),
                 ba = __builtin_bit_cast(_Float16, (uint16_t)(valid ? ba16 : 0));
  const _Float16 sb = __builtin_bit_cast(_Float16, (uint16_t)(valid ? sb16 : 0)),
                 bb = __builtin_bit_cast(_Float16, (uint16_t)(valid ? bb16 : 0));
  const half2_t s0 = {sa, sa}, b0 = {ba, ba}, s1 = {sb, sb}, b1 = {bb, bb};
  const uint32_t wd[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) dequant_word<BITS>(wd[i], i < 2 ? s0 : s1, i < 2 ? b0 : b1, mg, w + i * PPW);
}

// The magic words of dequant_stage, kept in vector registers (an opaque copy stops the compiler
// from folding them back into literals, which v_and_or_b32 cannot take two of).
__device__ __forceinline__ void magic_words(uint32_t* mg) {
  mg[0] = 0x64006400u;  // 1024.0
  mg[1] = 0x5C005C00u;  // 256.0
  mg[2] = 0x54005400u;  // 64.0
  mg[3] = 0x4C004C00u;  // 16.0
  asm volatile("" : "+v"(mg[0]), "+v"(mg[1]), "+v"(mg[2]), "+v"(mg[3]));
}

// B operand of one v_mfma_f32_16x16x32_f16: four dequantised code pairs (eight columns).
__device__ __forceinline__ half8_t pair4(const uint32_t* w) {
  return __builtin_bit_cast(half8_t, make_uint4(w[0], w[1], w[2], w[3]));
}
// A operand: the eight staged activation columns the same four pairs cover, as two 8-byte LDS
// reads (a staged row is 8-byte aligned: its stride keeps the 16 rows a quad reads in distinct banks).
__device__ __forceinline__ half8_t lds_a8(const uint16_t* xa) {
  const half4_t lo = *reinterpret_cast<const half4_t*>(xa), hi = *reinterpret_cast<const half4_t*>(xa + 4);
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// acc[mi] += X[MT tokens][one macro step] * W_mi[16 rows][same]^T.
template <int BITS, bool SPLIT, int NMAT>
__device__ __forceinline__ void consume_w(const WStage<NMAT, SPLIT>& S, bool valid, const uint16_t* xa,
                                          const uint32_t* mg, float4_t* acc) {
  using GS = GSeg<BITS>;
  uint32_t w[NMAT][GS::STEPS * 2];
#pragma unroll
  for (int mi = 0; mi < NMAT; ++mi)
    dequant_stage<BITS, SPLIT>(S.q[mi], S.sa[mi], S.ba[mi], S.sb[mi], S.bb[mi], valid, mg, w[mi]);
#pragma unroll
  for (int s = 0; s < GS::STEPS / 2; ++s) {
    const half8_t a = lds_a8(xa + 8 * s);
#pragma unroll
    for (int mi = 0; mi < NMAT; ++mi)
      acc[mi] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, pair4(&w[mi][4 * s]), acc[mi], 0, 0, 0);
  }
}

struct LoraRefG {
  const uint16_t* B;  // [rows][rank]
  const float* u;     // [T][rank]; with nparts > 0, nparts partial sums [nparts][T][rank]
  int rank;
  float scale;
  int nparts;         // 0: u is the product itself
  int T;
};
// (alpha / rank) * B[row] . u: rank 16 (the common case) as two 16-byte reads of B and four of u
// issued together; other ranks element by element.  u: [rank] floats (global memory or LDS).
__device__ __forceinline__ float lora_dot_g(const LoraRefG& lr, const float* u, int row) {
  const uint16_t* b = lr.B + (size_t)row * lr.rank;
  float acc = 0.f;
  if (lr.rank == 16 && (((uintptr_t)lr.B | (uintptr_t)u) & 15) == 0) {
    const uint4 b0 = reinterpret_cast<const uint4*>(b)[0], b1 = reinterpret_cast<const uint4*>(b)[1];
    const float4 u0 = reinterpret_cast<const float4*>(u)[0], u1 = reinterpret_cast<const float4*>(u)[1];
    const float4 u2 = reinterpret_cast<const float4*>(u)[2], u3 = reinterpret_cast<const float4*>(u)[3];
    const uint32_t bw[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
    const float uv[16] = {u0.x, u0.y, u0.z, u0.w, u1.x, u1.y, u1.z, u1.w, u2.x, u2.y, u2.z, u2.w, u3.x, u3.y, u3.z, u3.w};
#pragma unroll
    for (int r = 0; r < 16; ++r) acc = fmaf(h2f((uint16_t)(bw[r / 2] >> (16 * (r % 2)))), uv[r], acc);
  } else {
    for (int r = 0; r < lr.rank; ++r) acc = fmaf(h2f(b[r]), u[r], acc);
  }
  return lr.scale * acc;
}
__device__ __forceinline__ float lora_row_g(const LoraRefG& lr, int t, int row) {
  return lora_dot_g(lr, lr.u + (size_t)t * lr.rank, row);
}

// The down adapter's A . act, taken in the gate/up kernel: each block of RB activation rows adds
// its rows' share, part[rb][t][r] = sum over the block's rows i of A[r][i] act[t][i]
// (act rounded to float16 as stored), and the down kernel sums the parts in order.
struct LoraPartG {
  const uint16_t* A;  // [rank][I] (null: no down adapter)
  float* part;        // [row blocks][T][rank]
  int rank, T;
};

// Gate/up epilogue of an adapter tile: the tile's activations av (lane (ln, lq): tile rows
// 4 lq .. + 3 of activation row rbase + wave * 16 + ln, 0 where there is none) go through LDS
// (`lds`, at least MT * RB floats, free once every wave is past the main loop), then thread
// (m, r) sums row m's share of u_down[t][r].  rows[m]: token of tile row m, -1 for none.  Every
// wave of the block calls this.
template <int RB>
__device__ __forceinline__ void lora_down_part(const LoraPartG& lp, const float (&av)[4], float* lds, const int* rows,
                                               int rb, int nrows) {
  const int rbase = rb * RB;
  const int wave = threadIdx.x / WAVE, lane = threadIdx.x % WAVE, ln = lane % 16, lq = lane / 16;
  lds_barrier();  // every wave is done with the staged tokens
#pragma unroll
  for (int i = 0; i < 4; ++i) lds[(4 * lq + i) * RB + wave * 16 + ln] = av[i];
  lds_barrier();
  const int nr = min(RB, nrows - rbase);
  for (int o = threadIdx.x; o < MT * lp.rank; o += blockDim.x) {
    const int m = o / lp.rank, r = o % lp.rank, t = rows[m];
    if (t < 0) continue;
    const uint16_t* a = lp.A + (size_t)r * nrows + rbase;
    const float* v = lds + m * RB;
    float acc = 0.f;
    if (nr == RB && ((uintptr_t)a & 15) == 0) {  // whole block row, 16-byte aligned: all loads at once
      uint4 a8[RB / 8];
#pragma unroll
      for (int k = 0; k < RB / 8; ++k) a8[k] = reinterpret_cast<const uint4*>(a)[k];
#pragma unroll
      for (int k = 0; k < RB / 8; ++k) {
        const uint32_t w4[4] = {a8[k].x, a8[k].y, a8[k].z, a8[k].w};
#pragma unroll
        for (int h = 0; h < 8; ++h) acc = fmaf(h2f((uint16_t)(w4[h / 2] >> (16 * (h % 2)))), v[8 * k + h], acc);
      }
    } else {
      for (int j = 0; j < nr; ++j) acc = fmaf(h2f(a[j]), v[j], acc);
    }
    lp.part[((size_t)rb * lp.T + t) * lp.rank + r] = acc;
  }
}

// Down kernel of an adapter tile: ul[m][r] = the parts of u_down[t][r] summed in order, t the
// token of the tile's pair rec4[m] (routed pair p < TK is token p / K, pair TK + t the shared
// expert's of token t; rec4[m] < 0: no pair, 0).  ul: LDS, [MT][rank] floats, free once every wave
// is past the main loop.  Every wave of the block calls this; ul is ready when it returns.
__device__ __forceinline__ void lora_down_gather(const LoraRefG& lr, float* ul, const int32_t* rec4, int TK, int K) {
  lds_barrier();  // every wave is done with the staged activations
  for (int o = threadIdx.x; o < MT * lr.rank; o += blockDim.x) {
    const int m = o / lr.rank, r = o % lr.rank, pr = rec4[m];
    const int t = pr < 0 ? -1 : (pr < TK ? pr / K : pr - TK);
    float acc = 0.f;
    if (t >= 0)
      for (int p = 0; p < lr.nparts; ++p) acc += lr.u[((size_t)p * lr.T + t) * lr.rank + r];
    ul[o] = acc;
  }
  lds_barrier();
}

// XCD-aware order of the GEMM blocks.  The blocks of a launch are dealt to the NXCD XCDs in turn
// (block b runs on XCD b mod NXCD), so XCD x takes the (b / NXCD)-th item of its own list: an equal
// share of the S shared-expert tiles (the first S of the work list), then an equal share of the
// routed tiles, each tile's NRB row blocks one after another.  A tile's row blocks (one token tile)
// and an expert's consecutive tiles (the same weight rows) then go through the same L2.  False:
// this block has no item.
constexpr int NXCD = 8;
__device__ __forceinline__ bool xcd_item(int nt, int S, int NRB, int& tile, int& rb) {
  const int b = blockIdx.x, x = b % NXCD, j = b / NXCD;
  const int s0 = S * x / NXCD, ns = S * (x + 1) / NXCD - s0;
  const int R = nt - S, r0 = S + R * x / NXCD, nr = S + R * (x + 1) / NXCD - r0;
  const int k = j / NRB;
  if (k >= ns + nr) return false;
  tile = k < ns ? s0 + k : r0 + (k - ns);
  rb = j % NRB;
  return true;
}

// One tile of the work list (MT sorted pairs of one expert) against weight rows rb * 16 GW .. + 16 GW
// of NMAT matrices (tile and row block rb from xcd_item), the input columns in chunks of NST macro
// steps (columns past ncols are zero).
//   NMAT == 2: gate/up of the tile's tokens (rows of x), SwiGLU, act_sorted[pos][row] float16;
//   NMAT == 1: down of the tile's activations (rows of act_sorted), out[pair][row] float32;
//              tiles of bucket E (indices outside [0, E)) write NaN.
// The token tile is staged in LDS once per XCH columns; each wave streams its 16 rows with PF
// macro steps of weight loads in flight, and the barriers order LDS only, so the loads issued
// before a barrier stay in flight across it.
template <int BITS, bool SPLIT, int NMAT, int NST>
__global__ void __launch_bounds__(GW * WAVE) k_grouped_mm(int K, int E, int ncols, int nrows, int lg2g,
                                                          const uint16_t* __restrict__ src,
                                                          const int32_t* __restrict__ offsets,
                                                          const int32_t* __restrict__ perm,
                                                          const int32_t* __restrict__ tiles,
                                                          const float* __restrict__ rowscale, moe_qmat m0, moe_qmat m1,
                                                          uint16_t* __restrict__ act_sorted, float* __restrict__ out,
                                                          LoraRefG l0, LoraRefG l1, moe_qmat s0, moe_qmat s1, int SB,
                                                          int TK, LoraPartG lp, int S, int NRB) {
  using GS = GSeg<BITS>;
  static_assert(NST % PF == 0 && NST * GS::MACRO <= XCH, "whole stages, one LDS pass per chunk");
  static_assert(XS * 2 >= (NMAT == 2 ? 16 * GW : LORA_MAX_RANK) * 4, "the adapter's tiles fit in the token tile's LDS");
  __shared__ __attribute__((aligned(16))) uint16_t xs[MT * XS];
  __shared__ int rows[MT];
  int tile, rb;
  if (!xcd_item(tiles[0], S, NRB, tile, rb)) return;
  const int32_t* rec = tiles + 1 + (size_t)TREC * tile;
  const int e = rec[0], mt = rec[1], beg = rec[2], n_e = rec[3];
  // bucket SB (when >= 0) holds the shared expert's pairs TK + t, one per token t: its tiles read
  // the shared weights (expert 0 of s0 / s1) and carry the LoRA terms; routed pair p is token p / K
  const bool shb = e == SB;
  const int ee = shb ? 0 : e;
  const bool lora_on = SB < 0 || shb;
  const auto tok = [&](int pr) { return pr < TK ? pr / K : pr - TK; };
  const int wave = threadIdx.x / WAVE, lane = threadIdx.x % WAVE;
  const int ln = lane % 16, lq = lane / 16;
  const int n0 = rb * (16 * GW) + wave * 16;
  if (e >= E && !shb) {
    if constexpr (NMAT == 1)  // pairs whose expert index is out of range
      for (int pos = mt + lq; pos < min(n_e, mt + MT); pos += 4)
        if (n0 + ln < nrows) out[(size_t)rec[4 + pos - mt] * nrows + n0 + ln] = quiet_nan();
    return;
  }
  if (threadIdx.x < MT) {
    const int pos = mt + threadIdx.x;
    rows[threadIdx.x] = pos < n_e ? (NMAT == 2 ? tok(rec[4 + threadIdx.x]) : beg + pos) : -1;
  }
  lds_barrier();
  const bool active = n0 < nrows;  // uniform over the wave
  const int wpr = ncols * BITS / 32, ngr = ncols >> lg2g;
  const size_t row = (size_t)ee * nrows + (active ? n0 + ln : 0);
  const moe_qmat mats[2] = {shb ? s0 : m0, shb ? s1 : m1};
  float4_t acc[NMAT];
#pragma unroll
  for (int mi = 0; mi < NMAT; ++mi) acc[mi] = float4_t{0.f, 0.f, 0.f, 0.f};
  uint32_t mg[4];
  magic_words(mg);
  WStage<NMAT, SPLIT> st[PF];
  for (int c0 = 0; c0 < ncols; c0 += NST * GS::MACRO) {
    if (c0 > 0) lds_barrier();  // every wave is done with the previous pass
    stage_rows<BITS>(xs, src, ncols, c0, NST * GS::MACRO, rows);
    const int lcol = c0 + lq * GS::COLS;  // this lane's column at macro step 0
    if (active) {
#pragma unroll
      for (int u = 0; u < PF; ++u) {
        issue_w<BITS, SPLIT, NMAT>(st[u], mats, row, wpr, ngr, lg2g, ncols, lcol + u * GS::MACRO);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    lds_barrier();
    if (!active) continue;
    const uint16_t* xa = xs + ln * XS + lq * GS::COLS;
    // The chunk is straight-line code (NST compile-time steps): consume stage step % PF, refill
    // it PF steps ahead.  In a loop the compiler merges the outstanding loads of the loop's entry
    // and back edge and its waits turn conservative; unrolled, every wait is exact.  The
    // scheduling barriers keep each stage's loads together and in program order.
#pragma unroll
    for (int step = 0; step < NST; ++step) {
      consume_w<BITS, SPLIT, NMAT>(st[step % PF], lcol + step * GS::MACRO < ncols, xa + step * GS::MACRO, mg, acc);
      __builtin_amdgcn_sched_barrier(0);
      if (step + PF < NST) {
        issue_w<BITS, SPLIT, NMAT>(st[step % PF], mats, row, wpr, ngr, lg2g, ncols, lcol + (step + PF) * GS::MACRO);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }
  // the down adapter's A . act: its parts summed here (down), or this block's part taken (gate/up)
  float* lds_f = reinterpret_cast<float*>(xs);
  const bool gather = NMAT == 1 && lora_on && l0.B != nullptr && l0.nparts > 0;  // uniform over the block
  if (gather) lora_down_gather(l0, lds_f, rec + 4, TK, K);
  float av[4] = {0.f, 0.f, 0.f, 0.f};
  if (active) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int pos = mt + 4 * lq + i;
      if (pos >= n_e || pos >= mt + MT) continue;
      const int n = n0 + ln;
      if constexpr (NMAT == 2) {
        const int t = tok(rec[4 + pos - mt]);
        const float sc = rowscale ? rowscale[t] : 1.f;
        float g = acc[0][i] * sc, u = acc[1][i] * sc;
        if (lora_on && l0.B) g += lora_row_g(l0, t, n);
        if (lora_on && l1.B) u += lora_row_g(l1, t, n);
        const uint16_t a16 = f2h(g / (1.f + expf(-g)) * u);
        act_sorted[(size_t)(beg + pos) * nrows + n] = a16;
        av[i] = n < nrows ? h2f(a16) : 0.f;
      } else {
        const int pr = rec[4 + pos - mt];
        float o = acc[0][i];
        if (lora_on && l0.B)
          o += gather ? lora_dot_g(l0, lds_f + (pos - mt) * l0.rank, n) : lora_row_g(l0, tok(pr), n);
        out[(size_t)pr * nrows + n] = o;
      }
    }
  }
  if (NMAT == 2 && lora_on && lp.A != nullptr)
    lora_down_part<16 * GW>(lp, av, lds_f, rows, rb, nrows);
}

// The same product for 64-column groups without per-step scale loads.  The columns are walked as
// in k_grouped_mm (at each macro step the four lanes of a row read 64 contiguous bytes, so every
// line is used whole within two steps), but the chunk's scales and biases of a row are loaded
// once: each of the row's four lanes reads a quarter of them (NG groups, one vector load per
// array) and packs scale | bias << 16 per group; at each step a lane takes the word of its
// group from the lane that holds it with ds_bpermute, which spends no vector-memory issue slot
// (per-step two-byte loads of them cost as much issue bandwidth as the weight bytes).  Needs the
// input width a multiple of the chunk and 16-byte aligned rows of scales and biases (the host
// checks); the token tile is staged with unconditional loads (zero rows selected afterwards) so
// that every wait stays exact.
// Halves of LDS the token tile of one mm64 item takes (MT rows of NST macro steps' columns).
template <int BITS, int NST>
constexpr int mm64_xs_halves() { return MT * lds_row_stride(NST * GSeg<BITS>::MACRO); }

// One (tile, row block) item of k_grouped_mm64, every thread of the block taking part; xs, rows and
// prs are the block's LDS (mm64_xs_halves halves, MT ints, MT ints).  ready() runs once, with every
// thread, after the first weight loads are issued and before the token tile is read: a wait for the
// tile's input rows there overlaps those loads.  It returns the same value in every thread; false
// (the input never became ready) makes the item store NaN in place of its outputs.
struct NoWait {
  __device__ bool operator()() const { return true; }
};
template <int BITS, int NMAT, int NST, int RG, typename Ready = NoWait>
__device__ __forceinline__ void mm64_item(
    int K, int E, int ncols, int nrows, const uint16_t* __restrict__ src, const int32_t* __restrict__ tiles,
    const float* __restrict__ rowscale, moe_qmat m0, moe_qmat m1, uint16_t* __restrict__ act_sorted,
    float* __restrict__ out, LoraRefG l0, LoraRefG l1, moe_qmat s0, moe_qmat s1, int SB, int TK, LoraPartG lp,
    int tile, int rb, uint16_t* __restrict__ xs, int* __restrict__ rows, int* __restrict__ prs,
    Ready ready = Ready{}) {
  using GS = GSeg<BITS>;
  constexpr int COLS = GS::COLS, MACRO = GS::MACRO, W = NST * MACRO, PB = GS::PB;
  constexpr int NG = W / 64 / 4;          // groups per lane (a quarter of the chunk's)
  constexpr int GPS = MACRO / 64;         // groups per macro step (2 for int4, 4 for int2)
  constexpr int LPG = 4 / GPS;            // lanes of a row per group at one step (2, 1)
  // 4-bit: PF64 stages (with each word dequantised just before its MFMA, gate/up holds four at 127
  // registers); 2-bit: two, which keeps it within its registers
  constexpr int PFD = BITS == 4 ? PF64 : 2;
  constexpr int PFN = RG * NST < PFD ? RG * NST : PFD;
  constexpr int XSW = lds_row_stride(W);
  constexpr int UNITS = MT * W / PB, PER_T = UNITS / (GW * WAVE);
  constexpr int NHALF = PER_T >= 2 ? 2 : 1;
  static_assert(NG >= 1 && NG <= 8 && (NG & (NG - 1)) == 0, "1..8 groups per lane");
  static_assert(UNITS % (NHALF * GW * WAVE) == 0 && MT * XSW * 2 <= 70 * 1024, "staging layout");
  static_assert(NMAT == 1 || RG == 1, "gate/up: one row group per wave");
  static_assert(XSW * 2 >= (NMAT == 2 ? 16 * GW : LORA_MAX_RANK) * 4, "the adapter's tiles fit in the token tile's LDS");
  const int32_t* rec = tiles + 1 + (size_t)TREC * tile;
  const int e = rec[0], mt = rec[1], beg = rec[2], n_e = rec[3];
  // bucket SB (when >= 0) holds the shared expert's pairs TK + t, one per token t: its tiles read
  // the shared weights (expert 0 of s0 / s1) and carry the LoRA terms; routed pair p is token p / K
  const bool shb = e == SB;
  const int ee = shb ? 0 : e;
  const bool lora_on = SB < 0 || shb;
  const auto tok = [&](int pr) { return pr < TK ? pr / K : pr - TK; };
  const int wave = threadIdx.x / WAVE, lane = threadIdx.x % WAVE;
  const int ln = lane % 16, lq = lane / 16;
  // row group rg of this wave: weight rows n0(rg) .. + 16
  auto n0 = [&](int rg) { return rb * (16 * GW * RG) + rg * 16 * GW + wave * 16; };
  // NaN in this item's output rows (down only): pairs whose expert index is out of range, or an
  // input that never became ready
  const auto poison = [&]() {
    if constexpr (NMAT == 1)
      for (int rg = 0; rg < RG; ++rg)
        for (int pos = mt + lq; pos < min(n_e, mt + MT); pos += 4)
          if (n0(rg) + ln < nrows) out[(size_t)rec[4 + pos - mt] * nrows + n0(rg) + ln] = quiet_nan();
  };
  if (e >= E && !shb) {
    poison();
    return;
  }
  if (threadIdx.x < MT) {
    const int pos = mt + threadIdx.x;
    rows[threadIdx.x] = pos < n_e ? (NMAT == 2 ? tok(rec[4 + threadIdx.x]) : beg + pos) : -1;
    prs[threadIdx.x] = rec[4 + min((int)threadIdx.x, n_e - mt - 1)];
  }
  lds_barrier();
  const bool active = n0(0) < nrows;  // uniform over the wave (later row groups checked at the stores)
  const int wpr = ncols * BITS / 32, ngr = ncols / 64;
  // weight row (inside the expert) of row group rg, clamped so that every load is valid; the
  // expert's base addresses are uniform over the block, the offsets from them 32-bit
  auto lrow = [&](int rg) { return (uint32_t)min(n0(rg) + ln, nrows - 1); };
  const moe_qmat mats[2] = {shb ? s0 : m0, shb ? s1 : m1};
  const uint32_t* qe[2];
  const uint16_t* se[2];
  const uint16_t* be[2];
#pragma unroll
  for (int mi = 0; mi < 2; ++mi) {
    qe[mi] = mats[mi].q + (size_t)ee * nrows * wpr;
    se[mi] = mats[mi].scales + (size_t)ee * nrows * ngr;
    be[mi] = mats[mi].biases + (size_t)ee * nrows * ngr;
  }
  const int row0 = rows[0];  // always a real row (the tile holds at least one pair)
  float4_t acc[RG][NMAT];
#pragma unroll
  for (int rg = 0; rg < RG; ++rg)
#pragma unroll
    for (int mi = 0; mi < NMAT; ++mi) acc[rg][mi] = float4_t{0.f, 0.f, 0.f, 0.f};
  uint32_t mg[4];
  magic_words(mg);
  for (int c0 = 0; c0 < ncols; c0 += W) {
    if (c0 > 0) lds_barrier();  // every wave is done with the previous chunk
    const int lcol = c0 + lq * COLS;  // this lane's column at macro step 0
    uint32_t sbw[RG][NMAT][NG];       // scale | bias << 16 of groups [c0 / 64 + lq NG, + NG) of each row
    uint4 q[PFN][NMAT];
    if (active) {
#pragma unroll
      for (int rg = 0; rg < RG; ++rg) {
      const uint32_t g0 = lrow(rg) * (uint32_t)ngr + (uint32_t)(c0 / 64 + lq * NG);
#pragma unroll
      for (int mi = 0; mi < NMAT; ++mi) {
        uint16_t sv[NG], bv[NG];
        if constexpr (NG == 8) {
          const uint4 s4 = *reinterpret_cast<const uint4*>(se[mi] + g0);
          const uint4 b4 = *reinterpret_cast<const uint4*>(be[mi] + g0);
          const uint32_t sa[4] = {s4.x, s4.y, s4.z, s4.w}, ba[4] = {b4.x, b4.y, b4.z, b4.w};
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            sv[j] = (uint16_t)(sa[j / 2] >> (16 * (j % 2)));
            bv[j] = (uint16_t)(ba[j / 2] >> (16 * (j % 2)));
          }
        } else if constexpr (NG == 4) {
          const uint2 s2 = *reinterpret_cast<const uint2*>(se[mi] + g0);
          const uint2 b2 = *reinterpret_cast<const uint2*>(be[mi] + g0);
          const uint32_t sa[2] = {s2.x, s2.y}, ba[2] = {b2.x, b2.y};
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            sv[j] = (uint16_t)(sa[j / 2] >> (16 * (j % 2)));
            bv[j] = (uint16_t)(ba[j / 2] >> (16 * (j % 2)));
          }
        } else if constexpr (NG == 2) {
          const uint32_t s1 = *reinterpret_cast<const uint32_t*>(se[mi] + g0);
          const uint32_t b1 = *reinterpret_cast<const uint32_t*>(be[mi] + g0);
          sv[0] = (uint16_t)s1; sv[1] = (uint16_t)(s1 >> 16);
          bv[0] = (uint16_t)b1; bv[1] = (uint16_t)(b1 >> 16);
        } else {
          sv[0] = se[mi][g0];
          bv[0] = be[mi][g0];
        }
#pragma unroll
        for (int j = 0; j < NG; ++j) sbw[rg][mi][j] = (uint32_t)sv[j] | ((uint32_t)bv[j] << 16);
      }
      }
#pragma unroll
      for (int u = 0; u < PFN; ++u)
#pragma unroll
        for (int mi = 0; mi < NMAT; ++mi)
          q[u][mi] = *reinterpret_cast<const uint4*>(qe[mi] + (lrow(u / NST) * (uint32_t)wpr +
                                                                (uint32_t)(lcol + (u % NST) * MACRO) * BITS / 32));
    }
    __builtin_amdgcn_sched_barrier(0);
    if (c0 == 0 && !ready()) {
      poison();
      return;
    }
    // stage the token tile: every load unconditional (padding rows read row0, then zeroed), in
    // two halves to bound the registers it holds
#pragma unroll
    for (int half = 0; half < NHALF; ++half) {
      constexpr int HT = PER_T / NHALF;
      uint4 xv[HT][PB / 8];
#pragma unroll
      for (int kk = 0; kk < HT; ++kk) {
        const int u = threadIdx.x + (half * HT + kk) * GW * WAVE, m = u / (W / PB), cb = u % (W / PB);
        const int r = rows[m];
        const uint4* p = reinterpret_cast<const uint4*>(src + (size_t)(r >= 0 ? r : row0) * ncols + c0 + cb * PB);
#pragma unroll
        for (int h = 0; h < PB / 8; ++h) xv[kk][h] = p[h];
      }
#pragma unroll
      for (int kk = 0; kk < HT; ++kk) {
        const int u = threadIdx.x + (half * HT + kk) * GW * WAVE, m = u / (W / PB), cb = u % (W / PB);
        const bool real = rows[m] >= 0;
        uint32_t outw[PB / 2];
        if constexpr (BITS == 4) {
          const uint4 v = xv[kk][0];
          outw[0] = (v.x & 0xFFFFu) | (v.z << 16);
          outw[1] = (v.x >> 16) | (v.z & 0xFFFF0000u);
          outw[2] = (v.y & 0xFFFFu) | (v.w << 16);
          outw[3] = (v.y >> 16) | (v.w & 0xFFFF0000u);
        } else {
          const uint4 a = xv[kk][0], b = xv[kk][1];
          const uint32_t av[4] = {a.x, a.y, a.z, a.w}, bv[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const uint32_t lo = (j & 1) ? (av[j >> 1] >> 16) : (av[j >> 1] & 0xFFFFu);
            const uint32_t hi = (j & 1) ? (bv[j >> 1] & 0xFFFF0000u) : (bv[j >> 1] << 16);
            outw[j] = lo | hi;
          }
        }
#pragma unroll
        for (int j = 0; j < PB / 2; ++j) outw[j] = real ? outw[j] : 0u;
        uint4* dst = reinterpret_cast<uint4*>(xs + m * XSW + cb * PB);
        dst[0] = make_uint4(outw[0], outw[1], outw[2], outw[3]);
        if constexpr (PB == 16) dst[1] = make_uint4(outw[4], outw[5], outw[6], outw[7]);
      }
    }
    lds_barrier();
    if (!active) continue;
    const uint16_t* xa = xs + ln * XSW + lq * COLS;
    const int sub = lq / LPG;  // which of the step's groups this lane's segment lies in
#pragma unroll
    for (int f = 0; f < RG * NST; ++f) {  // row group f / NST, macro step f % NST
      const int rg = f / NST, step = f % NST;
      uint32_t pick[NMAT];
#pragma unroll
      for (int mi = 0; mi < NMAT; ++mi) {
        // group step * GPS + g of the chunk lives in lane (ln, (step GPS + g) / NG), element (...) % NG
        pick[mi] = 0;
#pragma unroll
        for (int g = 0; g < GPS; ++g) {
          const int G = step * GPS + g;
          const uint32_t v = (uint32_t)__builtin_amdgcn_ds_bpermute((ln + 16 * (G / NG)) * 4, (int)sbw[rg][mi][G % NG]);
          pick[mi] = sub == g ? v : pick[mi];
        }
      }
      if constexpr (BITS == 4) {
        // word s of a lane's segment holds the eight columns MFMA s takes: each word is
        // dequantised just before its MFMA, so only one word's pairs are live per matrix
        const uint32_t* qw[NMAT];
#pragma unroll
        for (int mi = 0; mi < NMAT; ++mi) qw[mi] = reinterpret_cast<const uint32_t*>(&q[f % PFN][mi]);
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const half8_t a = lds_a8(xa + step * MACRO + 8 * s);
#pragma unroll
          for (int mi = 0; mi < NMAT; ++mi) {
            const half2_t sc = __builtin_bit_cast(half2_t, (pick[mi] & 0xFFFFu) * 0x10001u);
            const half2_t bi = __builtin_bit_cast(half2_t, (pick[mi] >> 16) * 0x10001u);
            uint32_t w4[4];
            dequant_word<4>(qw[mi][s], sc, bi, mg, w4);
            acc[rg][mi] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, pair4(w4), acc[rg][mi], 0, 0, 0);
          }
        }
      } else if constexpr (RG == 1) {
        uint32_t w[NMAT][GS::STEPS * 2];
#pragma unroll
        for (int mi = 0; mi < NMAT; ++mi)
          dequant_stage<BITS, false>(q[f % PFN][mi], (uint16_t)pick[mi], (uint16_t)(pick[mi] >> 16), 0, 0, true, mg,
                                     w[mi]);
#pragma unroll
        for (int s = 0; s < GS::STEPS / 2; ++s) {
          const half8_t a = lds_a8(xa + step * MACRO + 8 * s);
#pragma unroll
          for (int mi = 0; mi < NMAT; ++mi)
            acc[rg][mi] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, pair4(&w[mi][4 * s]), acc[rg][mi], 0, 0, 0);
        }
      } else {
        // 2-bit codes with four row groups: the 16-column form holds fewer activation registers
        // live and keeps this variant within its 128 registers without spilling
        uint32_t w[NMAT][GS::STEPS * 2];
#pragma unroll
        for (int mi = 0; mi < NMAT; ++mi)
          dequant_stage<BITS, false>(q[f % PFN][mi], (uint16_t)pick[mi], (uint16_t)(pick[mi] >> 16), 0, 0, true, mg,
                                     w[mi]);
#pragma unroll
        for (int s = 0; s < GS::STEPS; ++s) {
          const half4_t a = *reinterpret_cast<const half4_t*>(xa + step * MACRO + 4 * s);
#pragma unroll
          for (int mi = 0; mi < NMAT; ++mi)
            acc[rg][mi] = __builtin_amdgcn_mfma_f32_16x16x16f16(
                a, __builtin_bit_cast(half4_t, make_uint2(w[mi][2 * s], w[mi][2 * s + 1])), acc[rg][mi], 0, 0, 0);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      if (f + PFN < RG * NST) {
        const int fn = f + PFN;
#pragma unroll
        for (int mi = 0; mi < NMAT; ++mi)
          q[f % PFN][mi] = *reinterpret_cast<const uint4*>(qe[mi] + (lrow(fn / NST) * (uint32_t)wpr +
                                                                      (uint32_t)(lcol + (fn % NST) * MACRO) * BITS / 32));
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }
  // the down adapter's A . act: its parts summed here (down), or this block's part taken (gate/up)
  float* lds_f = reinterpret_cast<float*>(xs);
  const bool gather = NMAT == 1 && lora_on && l0.B != nullptr && l0.nparts > 0;  // uniform over the block
  if (gather) lora_down_gather(l0, lds_f, rec + 4, TK, K);
  float av[4] = {0.f, 0.f, 0.f, 0.f};
  if (active) {
#pragma unroll
    for (int rg = 0; rg < RG; ++rg)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int pos = mt + 4 * lq + i;
        const int n = n0(rg) + ln;
        if (pos >= n_e || pos >= mt + MT || n >= nrows) continue;
        if constexpr (NMAT == 2) {
          const int t = tok(prs[4 * lq + i]);
          const float sc = rowscale ? rowscale[t] : 1.f;
          float g = acc[rg][0][i] * sc, u = acc[rg][1][i] * sc;
          if (lora_on && l0.B) g += lora_row_g(l0, t, n);
          if (lora_on && l1.B) u += lora_row_g(l1, t, n);
          const uint16_t a16 = f2h(g / (1.f + expf(-g)) * u);
          act_sorted[(size_t)(beg + pos) * nrows + n] = a16;
          av[i] = h2f(a16);
        } else {
          const int pr = prs[4 * lq + i];
          float o = acc[rg][0][i];
          if (lora_on && l0.B)
            o += gather ? lora_dot_g(l0, lds_f + (pos - mt) * l0.rank, n) : lora_row_g(l0, tok(pr), n);
          out[(size_t)pr * nrows + n] = o;
        }
      }
  }
  if (NMAT == 2 && lora_on && lp.A != nullptr)
    lora_down_part<16 * GW>(lp, av, lds_f, rows, rb, nrows);
}

template <int BITS, int NMAT, int NST, int RG>
__global__ void __launch_bounds__(GW * WAVE) __attribute__((amdgpu_waves_per_eu(BITS == 4 || NMAT == 1 ? 4 : 3)))
k_grouped_mm64(
    int K, int E, int ncols, int nrows, const uint16_t* __restrict__ src, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ perm, const int32_t* __restrict__ tiles, const float* __restrict__ rowscale,
    moe_qmat m0, moe_qmat m1, uint16_t* __restrict__ act_sorted, float* __restrict__ out, LoraRefG l0, LoraRefG l1,
    moe_qmat s0, moe_qmat s1, int SB, int TK, LoraPartG lp, int S, int NRB) {
  __shared__ __attribute__((aligned(16))) uint16_t xs[mm64_xs_halves<BITS, NST>()];
  __shared__ int rows[MT];
  __shared__ int prs[MT];  // the tile's pair indices (padding rows: the last pair), for the epilogue
  int tile, rb;
  if (!xcd_item(tiles[0], S, NRB, tile, rb)) return;
  mm64_item<BITS, NMAT, NST, RG>(K, E, ncols, nrows, src, tiles, rowscale, m0, m1, act_sorted, out, l0, l1, s0, s1,
                                 SB, TK, lp, tile, rb, xs, rows, prs);
}

// The arguments of one projection of the fused launch below (those of k_grouped_mm64).
struct MM64Args {
  int K, E, ncols, nrows;
  const uint16_t* src;
  const int32_t* tiles;
  const float* rowscale;
  moe_qmat m0, m1;
  uint16_t* act_sorted;
  float* out;
  LoraRefG l0, l1;
  moe_qmat s0, s1;
  int SB, TK;
  LoraPartG lp;
};
constexpr int FUSED_SPIN_MAX = 1 << 20;  // polls of a tile count (each after a short sleep): ~0.1 s

// Gate/up and down in one launch.  XCD x (blocks b with b mod NXCD = x, in xcd_item's split of the
// tiles) first takes the gate/up items of its tiles, then their down items.  A gate/up block adds
// one to done[tile] once its activation rows (and adapter parts) are stored; a down block first
// waits for done[tile] == NRB_G.  The two launches' boundary made every down block wait for the
// last gate/up block of the grid, whose final round leaves a third of the slots idle; here the down
// items fill them.  Every gate/up block of an XCD is dealt before any of its down blocks, so the
// ones a down block waits for are running or done; the wait is bounded regardless, and a down
// block whose wait runs out stores NaN in its outputs, so the result shows it.  The down block
// issues its first weight loads before it waits.  Producer and consumer of a tile run on one XCD
// (gfx950 deals workgroup b to XCD b mod 8; a partition into 4, 2 or 1 XCDs keeps each class on
// one): the activations travel through that XCD's L2, and a down block reads them only after the
// count says they are complete.  done[]: zero at the launch (the sort's side blocks clear it).
template <int BITS, int NST_G, int NST_D, int RG_D>
__global__ void __launch_bounds__(GW * WAVE) __attribute__((amdgpu_waves_per_eu(4)))
k_grouped_fused64(MM64Args g, MM64Args dn, int S, int NRB_G, int NRB_D, int32_t* __restrict__ done) {
  constexpr int XG = mm64_xs_halves<BITS, NST_G>(), XD = mm64_xs_halves<BITS, NST_D>();
  __shared__ __attribute__((aligned(16))) uint16_t xs[XG > XD ? XG : XD];
  __shared__ int rows[MT];
  __shared__ int prs[MT];
  const int nt = g.tiles[0];
  const int x = blockIdx.x % NXCD, j = blockIdx.x / NXCD;
  const int s0 = S * x / NXCD, ns = S * (x + 1) / NXCD - s0;
  const int R = nt - S, r0 = S + R * x / NXCD, nr = S + R * (x + 1) / NXCD - r0;
  const int ntx = ns + nr;  // this XCD's tiles
  const auto tile_of = [&](int k) { return k < ns ? s0 + k : r0 + (k - ns); };
  if (j < ntx * NRB_G) {
    const int tile = tile_of(j / NRB_G), rb = j % NRB_G;
    mm64_item<BITS, 2, NST_G, 1>(g.K, g.E, g.ncols, g.nrows, g.src, g.tiles, g.rowscale, g.m0, g.m1, g.act_sorted,
                                 g.out, g.l0, g.l1, g.s0, g.s1, g.SB, g.TK, g.lp, tile, rb, xs, rows, prs);
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this lane's stores have completed
    __syncthreads();                     // ... and every other lane's
    if (threadIdx.x == 0) atomicAdd(done + tile, 1);
    return;
  }
  const int jd = j - ntx * NRB_G;
  if (jd >= ntx * NRB_D) return;
  const int tile = tile_of(jd / NRB_D), rb = jd % NRB_D;
  // the wait for the tile's activations, once the first down weight loads are in flight; the
  // activation loads stay behind the barrier (no reordering of memory accesses across it), and
  // after it they find the rows in this XCD's L2
  __shared__ int late;
  const auto ready = [&]() {
    if (threadIdx.x == 0) {
      bool ok = false;
      for (int spin = 0; spin < FUSED_SPIN_MAX && !ok; ++spin) {
        ok = __hip_atomic_load(done + tile, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= NRB_G;
        if (!ok) __builtin_amdgcn_s_sleep(2);
      }
      late = !ok;
    }
    asm volatile("" ::: "memory");
    lds_barrier();
    asm volatile("" ::: "memory");
    return late == 0;
  };
  mm64_item<BITS, 1, NST_D, RG_D>(dn.K, dn.E, dn.ncols, dn.nrows, dn.src, dn.tiles, dn.rowscale, dn.m0, dn.m1,
                                  dn.act_sorted, dn.out, dn.l0, dn.l1, dn.s0, dn.s1, dn.SB, dn.TK, dn.lp, tile, rb, xs,
                                  rows, prs, ready);
}

int ilog2g(int v) {
  int r = 0;
  while ((1 << r) < v) ++r;
  return r;
}

size_t al256(size_t v) { return (v + 255) / 256 * 256; }

// Upper bound of the work list's length: every nonempty bucket (at most NB of them, and at most
// N, the pairs) rounds up to whole tiles.
int max_tiles(int N, int NB) { return (N + MT - 1) / MT + min(NB, N); }
// Bytes of the work list (count + records) for N pairs in NB buckets; the per-tile completion counts
// of the fused GEMM launch follow it.
size_t tile_list_bytes(int N, int NB) { return al256((1 + TREC * (size_t)max_tiles(N, NB)) * 4); }
int32_t* tile_counts(int32_t* tiles, int N, int NB) {
  return reinterpret_cast<int32_t*>(reinterpret_cast<char*>(tiles) + tile_list_bytes(N, NB));
}

// Steps per chunk: a short chunk (PF macro steps) when the input row fits in it, else the
// longest one LDS holds.
template <int BITS, int NMAT>
auto grouped_kernel(bool split, int ncols) {
  constexpr int SHORT = PF, LONG = XCH / GSeg<BITS>::MACRO;
  const bool shrt = ncols <= SHORT * GSeg<BITS>::MACRO;
  if constexpr (BITS == 4)
    return shrt ? k_grouped_mm<4, false, NMAT, SHORT> : k_grouped_mm<4, false, NMAT, LONG>;
  else
    return split ? (shrt ? k_grouped_mm<2, true, NMAT, SHORT> : k_grouped_mm<2, true, NMAT, LONG>)
                 : (shrt ? k_grouped_mm<2, false, NMAT, SHORT> : k_grouped_mm<2, false, NMAT, LONG>);
}

// The lane-contiguous kernel for 64-column groups: the longest chunk (in segments per lane) that
// divides the input width, or nullptr when none does or the scale rows are not 16-byte aligned.
template <int BITS, int NMAT>
auto grouped_kernel64(int group, int ncols, const moe_qmat* mats, bool many_tiles) {
  using KT = decltype(&k_grouped_mm64<BITS, NMAT, 4, 1>);
  if (group != 64 || (ncols / 64) % 8 != 0) return (KT) nullptr;
  for (int mi = 0; mi < NMAT; ++mi)
    if (((uintptr_t)mats[mi].scales | (uintptr_t)mats[mi].biases) & 15) return (KT) nullptr;
  constexpr int MACRO = GSeg<BITS>::MACRO;
  constexpr int LONG = XCH / MACRO;  // 2048 columns per chunk
  // short chunks take several row groups per wave (one staged tile and prologue serve more rows)
  // Short chunks take four row groups per wave when the work list is long (one staged tile and
  // prologue then serve four times the rows); a short list keeps one so that it still spreads
  // over the chip.  (Two matrices' accumulators for four groups would spill.)
  constexpr int RGS = NMAT == 1 ? 4 : 1;
  if (ncols % (LONG * MACRO) == 0) return (KT)&k_grouped_mm64<BITS, NMAT, LONG, 1>;
  if (ncols % (4 * MACRO) == 0)
    return many_tiles ? (KT)&k_grouped_mm64<BITS, NMAT, 4, RGS> : (KT)&k_grouped_mm64<BITS, NMAT, 4, 1>;
  if (ncols % (2 * MACRO) == 0)
    return many_tiles ? (KT)&k_grouped_mm64<BITS, NMAT, 2, RGS> : (KT)&k_grouped_mm64<BITS, NMAT, 2, 1>;
  return (KT) nullptr;
}

// Row groups per wave of the kernel grouped_kernel64 picks for an input width.
template <int NMAT>
int rg64(int ncols, bool many_tiles) { return ncols % XCH == 0 || NMAT == 2 || !many_tiles ? 1 : 4; }
constexpr int MANY_TILES = 128;  // work lists at least this long take four row groups


// The two GEMMs over the work list.  With a shared expert (a.shared), its T pairs form bucket E + 1
// of the same list, so one launch per projection covers routed and shared tiles alike.
// Blocks of a GEMM launch over at most nt tiles (the first S the shared expert's) and NRB row
// blocks each, in xcd_item's order: every XCD's list padded to the longest one.
int xcd_grid(int nt, int S, int NRB) { return NXCD * ((S + NXCD - 1) / NXCD + (nt - S + NXCD - 1) / NXCD) * NRB; }

template <int BITS, bool SPLIT>
hipError_t launch_gemms(hipStream_t s, const GroupedArgs& g, const float* rowscale, float* o_tk, LoraRefG lg,
                        LoraRefG lu, LoraRefG ldn, const DecodeArgs& a) {
  const int lg2g = ilog2g(a.group);
  const int rows_per_block = 16 * GW;
  const int TK = a.T * a.K, TS = a.shared ? a.T : 0, SB = a.shared ? a.E + 1 : -1;
  const int nt = max_tiles(TK + TS, a.E + 1 + (TS > 0));
  const int S = (TS + MT - 1) / MT;  // the shared expert's tiles, first in the work list
  const moe_experts& sx = a.shared ? *a.shared : a.ex;  // the shared weights (unused without a shared expert)
  const moe_qmat gu[4] = {a.ex.gate, a.ex.up, sx.gate, sx.up};
  const moe_qmat dn[2] = {a.ex.down, sx.down};
  const bool many = nt >= MANY_TILES;
  // The down adapter's A . act is taken by the gate/up blocks of the adapter's tiles, one part per
  // row block (rows_per_block activation rows); the down kernel sums the parts.
  const int nparts = grouped_lora_parts(a.I);
  LoraPartG lp{};
  if (a.lora3) {
    lp = LoraPartG{a.lora3[2].A, a.u_down, a.lora3[2].rank, a.T};
    ldn.nparts = nparts;
    ldn.T = a.T;
  }
  const auto k64_gu = grouped_kernel64<BITS, 2>(a.group, a.d, gu, many);
  const auto k64_gu_s = grouped_kernel64<BITS, 2>(a.group, a.d, gu + 2, many);
  const auto k64_dn = grouped_kernel64<BITS, 1>(a.group, a.I, dn, many);
  const auto k64_dn_s = grouped_kernel64<BITS, 1>(a.group, a.I, dn + 1, many);
  if constexpr (BITS == 4) {
    // both projections in one launch where both take the lane-contiguous kernels of the fused one:
    // gate/up over whole 2,048-column chunks, down over 512-column chunks
    const bool gu_long = k64_gu && k64_gu == k64_gu_s && k64_gu == &k_grouped_mm64<4, 2, XCH / GSeg<4>::MACRO, 1>;
    const bool dn_rg4 = k64_dn && k64_dn == k64_dn_s && k64_dn == &k_grouped_mm64<4, 1, 4, 4>;
    const bool dn_rg1 = k64_dn && k64_dn == k64_dn_s && k64_dn == &k_grouped_mm64<4, 1, 4, 1>;
    if (gu_long && (dn_rg4 || dn_rg1)) {
      const int rg = dn_rg4 ? 4 : 1, nrb_d = (a.d + rows_per_block * rg - 1) / (rows_per_block * rg);
      const MM64Args ga{a.K, a.E, a.d, a.I, a.x, (const int32_t*)g.tiles, rowscale, a.ex.gate, a.ex.up,
                        (uint16_t*)a.act, (float*)nullptr, lg, lu, sx.gate, sx.up, SB, TK, lp};
      const MM64Args da{a.K, a.E, a.I, a.d, (const uint16_t*)a.act, (const int32_t*)g.tiles, (const float*)nullptr,
                        a.ex.down, a.ex.down, (uint16_t*)nullptr, o_tk, ldn, LoraRefG{}, sx.down, sx.down, SB, TK,
                        LoraPartG{}};
      const dim3 grid(xcd_grid(nt, S, nparts + nrb_d));
      int32_t* done = tile_counts(g.tiles, TK + TS, a.E + 1 + (TS > 0));
      return dn_rg4 ? launch(k_grouped_fused64<4, XCH / GSeg<4>::MACRO, 4, 4>, grid, dim3(WAVE * GW), 0, s, ga, da, S,
                             nparts, nrb_d, done)
                    : launch(k_grouped_fused64<4, XCH / GSeg<4>::MACRO, 4, 1>, grid, dim3(WAVE * GW), 0, s, ga, da, S,
                             nparts, nrb_d, done);
    }
  }
  const dim3 grid_gu(xcd_grid(nt, S, nparts));
  hipError_t err;
  if (k64_gu && k64_gu_s)
    err = launch(k64_gu, grid_gu, dim3(WAVE * GW), 0, s, a.K, a.E, a.d, a.I, a.x, (const int32_t*)g.offsets,
                 (const int32_t*)g.perm, (const int32_t*)g.tiles, rowscale, a.ex.gate, a.ex.up, (uint16_t*)a.act,
                 (float*)nullptr, lg, lu, sx.gate, sx.up, SB, TK, lp, S, nparts);
  else
    err = launch(grouped_kernel<BITS, 2>(SPLIT, a.d), grid_gu, dim3(WAVE * GW), 0, s, a.K, a.E, a.d, a.I, lg2g, a.x,
                 (const int32_t*)g.offsets, (const int32_t*)g.perm, (const int32_t*)g.tiles, rowscale, a.ex.gate,
                 a.ex.up, (uint16_t*)a.act, (float*)nullptr, lg, lu, sx.gate, sx.up, SB, TK, lp, S, nparts);
  if (err != hipSuccess) return err;
  if (k64_dn && k64_dn_s) {
    const int rb = rows_per_block * rg64<1>(a.I, many), nrb = (a.d + rb - 1) / rb;
    return launch(k64_dn, dim3(xcd_grid(nt, S, nrb)), dim3(WAVE * GW), 0, s, a.K, a.E, a.I, a.d,
                  (const uint16_t*)a.act, (const int32_t*)g.offsets, (const int32_t*)g.perm, (const int32_t*)g.tiles,
                  (const float*)nullptr, a.ex.down, a.ex.down, (uint16_t*)nullptr, o_tk, ldn, LoraRefG{}, sx.down,
                  sx.down, SB, TK, LoraPartG{}, S, nrb);
  }
  const int nrb = (a.d + rows_per_block - 1) / rows_per_block;
  return launch(grouped_kernel<BITS, 1>(SPLIT, a.I), dim3(xcd_grid(nt, S, nrb)), dim3(WAVE * GW), 0, s, a.K, a.E,
                a.I, a.d, lg2g, (const uint16_t*)a.act, (const int32_t*)g.offsets, (const int32_t*)g.perm,
                (const int32_t*)g.tiles, (const float*)nullptr, a.ex.down, a.ex.down, (uint16_t*)nullptr, o_tk, ldn,
                LoraRefG{}, sx.down, sx.down, SB, TK, LoraPartG{}, S, nrb);
}

}  // namespace

int grouped_lora_parts(int I) { return (I + 16 * GW - 1) / (16 * GW); }

GroupedLayout grouped_layout(int T, int K, int E, int d, int TS) {
  const int NB = E + 1 + (TS > 0), NP = T * K + TS;
  GroupedLayout l{};
  l.counts = 0;
  l.offsets = l.counts + al256((size_t)NB * 4);
  l.perm = l.offsets + al256((size_t)(NB + 1) * 4);
  l.rowscale = l.perm + al256((size_t)NP * 4);
  l.o_sorted = l.rowscale + al256((size_t)T * 4);
  l.tiles = l.o_sorted + al256((size_t)NP * d * 4);
  // the work list, then one completion count per tile (the fused GEMM launch's)
  l.total = l.tiles + tile_list_bytes(NP, NB) + al256((size_t)max_tiles(NP, NB) * 4);
  return l;
}

namespace {
// The sort, with `side` in the same launch.
hipError_t launch_sort_side(hipStream_t s, int TK, int E, const int32_t* idx, int32_t* counts, int32_t* offsets,
                            int32_t* perm, int32_t* tiles, int TS, const SortSideJobs& side) {
  const int NB = E + 1 + (TS > 0);
  const size_t lds = (size_t)(3 * NB + 2 * (NB + 1) + SORT_WAVES * NB) * sizeof(int);
  const int side_blocks = (side.waves() + SORT_WAVES - 1) / SORT_WAVES;
  return launch(k_sort, dim3(1 + side_blocks), dim3(SORT_THREADS), lds, s, TK, E, idx, counts, offsets, perm, tiles,
                max_tiles(TK + TS, NB), TS, side);
}
}  // namespace

hipError_t launch_sort(hipStream_t s, int TK, int E, const int32_t* idx, int32_t* counts, int32_t* offsets,
                       int32_t* perm, int32_t* tiles, int TS) {
  return launch_sort_side(s, TK, E, idx, counts, offsets, perm, tiles, TS, SortSideJobs{});
}

hipError_t launch_expert_grouped(hipStream_t s, const GroupedArgs& g) {
  const DecodeArgs& a = g.base;
  const int rms = (a.flags & MOE_INPUT_RMSNORM) != 0;
  float* rowscale = rms ? g.rowscale : nullptr;
  const int NP = a.T * a.K + (a.shared ? a.T : 0), NB = a.E + 1 + (a.shared ? 1 : 0);
  int32_t* done = tile_counts(g.tiles, NP, NB);
  SortSideJobs side{LoraAJob{}, a.T, a.d, a.x, rowscale, done, max_tiles(NP, NB)};
  const moe_lora* L3 = a.lora3;
  if (L3)  // gate's and up's A . x
    side.lora = LoraAJob{a.T, a.d, rms, a.x, (size_t)a.d, L3[0].A, a.u_gate, L3[0].rank, L3[1].A, a.u_up, L3[1].rank};
  hipError_t err = launch_sort_side(s, a.T * a.K, a.E, a.idx, g.counts, g.offsets, g.perm, g.tiles,
                                    a.shared ? a.T : 0, side);
  if (err != hipSuccess) return err;
  LoraRefG lg{}, lu{}, ldn{};
  if (L3) {
    lg = LoraRefG{L3[0].B, a.u_gate, L3[0].rank, L3[0].alpha / (float)L3[0].rank};
    lu = LoraRefG{L3[1].B, a.u_up, L3[1].rank, L3[1].alpha / (float)L3[1].rank};
    ldn = LoraRefG{L3[2].B, a.u_down, L3[2].rank, L3[2].alpha / (float)L3[2].rank, 0, a.T};
  }
  float* o_tk = a.out && !a.shared ? a.out : g.o_sorted;  // with a shared expert: [T*K + T][d]
  if (a.bits == 4)
    err = launch_gemms<4, false>(s, g, rowscale, o_tk, lg, lu, ldn, a);
  else if (a.group < SegT<2>::COLS)
    err = launch_gemms<2, true>(s, g, rowscale, o_tk, lg, lu, ldn, a);
  else
    err = launch_gemms<2, false>(s, g, rowscale, o_tk, lg, lu, ldn, a);
  if (err != hipSuccess) return err;
  if (a.y_fuse)
    err = launch_combine(s, a.T, a.K, a.d, o_tk, a.w_fuse, a.r_fuse,
                         a.shared ? o_tk + (size_t)a.T * a.K * a.d : nullptr, a.y_fuse);
  return err;
}

}  // namespace moe
