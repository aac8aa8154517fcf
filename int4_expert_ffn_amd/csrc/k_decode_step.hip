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
//   * The SwiGLU output travels as floats with a 16-bit significand (two per word) and meets the
//     down weights as a float16 hi + lo pair.
//   * Data moves between workgroups as tagged 8-byte words (32-bit payload and 32-bit tag naming
//     the token epoch and the phase; for the SwiGLU output 48 bits of payload and a 16-bit tag),
//     written by one lane with device-coherent stores and read with agent-scope relaxed atomic
//     loads; a reader polls until every tag matches, so no flag/data ordering is needed.
//   * Per workgroup, wave 0 only waits for and unpacks the vector the next phase needs (into
//     LDS); waves 1..8 compute (two per SIMD).  Their weight loads for a phase are issued one
//     phase early, and workgroup barriers fence LDS only, so those loads stay in flight while
//     the phase waits.
//   * Every reduction runs in a fixed order (the RMS norm of h_l too: each compute wave takes it
//     from its own reads of h_l), so equal inputs give bit-identical outputs from run to run.
//   * The heads are off the critical path (their output routes the next token).  The linear and
//     fc1 rows of head l run in phase A of layer l; the wave that computes linear row e keeps it
//     and adds it to fc2 row e, which runs in phase A of layer l+1, after the head's hidden vector
//     g_l has been fetched while the grid waited for h_{l+1}.  So the act exchange carries only
//     the SwiGLU outputs.  The top-Ks run after the last layer, spread over the workgroups.
//   * The whole token's routing state is staged in LDS at the start, so issuing a phase's weight
//     loads never waits on a global read of the expert indices.
//
// Phases per layer l: [R_l: own router + top-K, only for layer 0, layers with no prediction and
// the first token] -> A_l: gate/up + SwiGLU, fc2 rows of head l-1, linear and fc1 (+GELU) rows of
// head l -> B_l: down + combine + residual.  Every wait is bounded in time: one that runs out
// sets the error word and lets the kernel finish (its results are then invalid).
#include <algorithm>

#include "moe_device.h"
#include "moe_launch.h"

namespace moe {
namespace {

constexpr int MW = 8;                        // compute waves per workgroup (two per SIMD)
constexpr int NTHREADS = (MW + 1) * WAVE;
constexpr int NH_MAX = 2;                    // head fc1/linear rows per compute wave
constexpr int LDS_D = 4096, LDS_ACT = 4096, LDS_H = 2048, LDS_E = 1024, LDS_PART = 512, LDS_LK = 512;
constexpr int RWG = 2;                       // router rows per workgroup that LDS can stage
constexpr int LDS_RR = 8192;                 // halves of staged router rows (RWG rows of d <= 4096)
constexpr int POLL_MAX = 16;                 // words per lane per polling pass (1024 per wave), <= 64
static_assert(POLL_MAX >= 1 && POLL_MAX <= 64, "one done bit per polled word");
constexpr uint32_t TAG_SALT = 0x5A5A5A5Au;
constexpr uint64_t WAIT_TICKS = 20000000;       // 0.2 s of polling, in ticks of the 100 MHz real-time counter
constexpr uint64_t WAIT_STEP_MAX = 2000;        // at most 20 us charged per polling pass (see ll_wait)

struct StepParams {
  int L, E, K, d, I, H, lg2g;
  int G, GU, NH, NR, NO, DR, DI, PD, Ldn;
  const moe_decode_layer* layers;
  const uint16_t* h_in;
  uint16_t* h_out;
  uint16_t* h_layers;  // NULL or [L+1][d]: every layer's input and the final output
  int32_t* ridx;
  float* rw;
  int slot, bootstrap, given;  // given: every layer's routing supplied by the caller
  int gained;                  // every layer's input norm has a gain (else none has)
  int rstage;                  // the compute waves stage each self-routed layer's router rows in LDS
  int lshift;                  // router logit r fills words [r << lshift, (r + 1) << lshift), every one tagged
  uint32_t topk_flags;
  uint64_t *ll_logits, *ll_act, *ll_g, *ll_hlog, *ll_h;
  const uint64_t* spare;  // one 64-byte line per workgroup, never written
  // h and the SwiGLU outputs are written in xr_h / xr_a copies (strides in words); workgroup b
  // reads copy b % xr, so the 256 readers of one exchange spread over several sets of lines
  int xr_h, xr_a, h_stride, act_stride;
  uint32_t* epoch;
  int* err;
  const uint16_t* zero16;  // a float16 zero (stands in for an absent bias)
  const void* ws;          // the workspace (base of the tagged-word buffers)
  uint32_t ws_bytes;
  uint64_t* stamps;        // NULL or [G][L][NSTAMP] real-time-counter stamps (measurement aid)
};


// Tagged-word vectors are plain arrays of 8-byte words; each lives in its own 256-byte-aligned
// region of the workspace.  (Spreading their 64-byte lines over memory pages was measured slower.)
__host__ __device__ constexpr size_t ll_bytes(size_t words) { return (words * 8 + 255) / 256 * 256; }
__device__ __forceinline__ const uint64_t* ll_at(const uint64_t* base, size_t i) { return base + i; }

// Writers store a tagged word from ONE lane, without a branch: a buffer store whose other lanes
// carry an offset past the buffer's end, which the hardware range check drops.  (A branch around
// the store would blur the compiler's count of outstanding loads; 64 lanes storing the same word
// serialise in the memory system.)  The sc1 bit makes the 8-byte store visible device-wide, as a
// relaxed agent-scope atomic store is.
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
constexpr uint32_t OFF_NONE = 0x80000000u;  // past every buffer this kernel addresses
constexpr int CPOL_SC1 = 16;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_of(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, 0x00020000);
}
// Phase stamps (measurement aid, the kernel variant with STAMP set): slot `slot` of (workgroup,
// layer) receives the 100 MHz real-time counter, stored by lane 0 of the calling wave when `on`.
//   poll wave:      0 layer start, 1 h_l unpacked, 2 SwiGLU outputs of the layer unpacked
//   compute wave 1: 3 h_l seen (after the barrier), 4 this workgroup's SwiGLU outputs stored,
//                   5 down phase starts, 6 this workgroup's rows of h_{l+1} stored, 7 head rows done,
//                   8 gate/up dot products done, 9 its SwiGLU output ready (before the gathering
//                   barrier), 12 the combine starts, 13 down dot products done, 14 down partials
//                   stored; on a self-routed layer, 10 its router logit stored, 11 the routing known
//   poll wave (self-routed layer): 15 all router logits unpacked (the top-K starts)
// The plain variant compiles every stamp away.
constexpr int NSTAMP = 16;
template <bool STAMP>
__device__ __forceinline__ void stamp(const StepParams& p, int wg, int l, int slot, bool on = true) {
  if constexpr (STAMP) {
    const uint64_t t = __builtin_amdgcn_s_memrealtime();
    if (on && threadIdx.x % WAVE == 0) p.stamps[((size_t)wg * p.L + l) * NSTAMP + slot] = t;
  }
}
__device__ __forceinline__ void ll_put64(__amdgpu_buffer_rsrc_t ws, const StepParams& p, const uint64_t* vec, size_t i,
                                         bool on, uint64_t word) {
  u32x2 v;
  v.x = (uint32_t)word;
  v.y = (uint32_t)(word >> 32);
  const uint32_t off = (uint32_t)((const char*)ll_at(vec, i) - (const char*)p.ws);
  __builtin_amdgcn_raw_buffer_store_b64(v, ws, on ? off : OFF_NONE, 0, CPOL_SC1);
}
__device__ __forceinline__ void ll_put(__amdgpu_buffer_rsrc_t ws, const StepParams& p, const uint64_t* vec, size_t i,
                                       bool on, uint32_t payload, uint32_t tag) {
  u32x2 v;
  v.x = payload;
  v.y = tag;
  const uint32_t off = (uint32_t)((const char*)ll_at(vec, i) - (const char*)p.ws);
  __builtin_amdgcn_raw_buffer_store_b64(v, ws, on ? off : OFF_NONE, 0, CPOL_SC1);
}

// The SwiGLU outputs travel two to a word: each float32 rounded to its top 24 bits (sign,
// exponent, 15 mantissa bits; round to nearest even, NaN and Inf kept) beside a 16-bit tag.  A
// 16-bit significand keeps the chained decode well inside its tolerance (float16's 11 bits did
// not), and half the words make the exchange one polling pass.
__device__ __forceinline__ uint32_t f32_to_f24(float f) {
  const uint32_t u = __float_as_uint(f);
  if ((u & 0x7F800000u) == 0x7F800000u) return u >> 8;  // Inf / NaN: truncate (a NaN stays a NaN)
  return (u + 0x7Fu + ((u >> 8) & 1u)) >> 8;
}
__device__ __forceinline__ float f24_to_f32(uint32_t v) { return __uint_as_float(v << 8); }
__device__ __forceinline__ uint64_t ll_load(const uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Poll n tagged words until all carry `tag`; sink(i, payload) receives each word once.
// Whole wave, POLL_MAX words per lane per pass, chunk after chunk (wider passes were measured
// slower: more readers hammer the same lines at once).  Two passes are in flight: the next one
// is issued before the previous one is checked, so a word is seen about one memory round trip
// after it lands rather than one and a half.  Every pass loads all POLL_MAX slots (slots past
// the end read this workgroup's own spare line and are ignored), which keeps the count of
// outstanding loads exact for the compiler's waits.  (Pointing those slots at the vector's last
// word made every workgroup hit one line with twelve loads per lane and pass when polling the 256
// router logits: that exchange took 4.1 us against 2.4 us for the 1,024-word h.)  A wait is bounded in polling time: past WAIT_TICKS it raises
// the error word, sets `failed`, and every later wait of this wave returns at once, so a grid
// that cannot make progress still finishes quickly (with invalid results).  Each pass is charged
// the real time since the previous one, capped at WAIT_STEP_MAX: a pass takes a few us, so the
// cap only matters when the whole grid was paused (the queue preempted and later resumed), and
// such a pause, during which no producer could run either, does not count against the bound.
// TAGB: tag bits in the top of each word (32: a 32-bit payload; 16: a 48-bit payload).
template <int TAGB = 32, class Sink>
__device__ __forceinline__ void ll_wait(const uint64_t* src, size_t start, int n, uint32_t tag, int* err, bool& failed,
                                        const uint64_t* spare, Sink sink) {
  constexpr uint64_t PAY = (1ull << (64 - TAGB)) - 1;
  if (failed) return;
  const int lane = threadIdx.x % WAVE;
  constexpr uint64_t ALL = POLL_MAX == 64 ? ~0ull : (1ull << POLL_MAX) - 1;  // one bit per word slot of a lane
  uint64_t last = __builtin_amdgcn_s_memrealtime(), waited = 0;
  for (int base = 0; base < n; base += POLL_MAX * WAVE) {
    uint64_t done = 0;
#pragma unroll
    for (int j = 0; j < POLL_MAX; ++j)
      if (base + lane + j * WAVE >= n) done |= 1ull << j;
    uint64_t a[POLL_MAX], b[POLL_MAX];
    auto issue = [&](uint64_t (&v)[POLL_MAX]) {
#pragma unroll
      for (int j = 0; j < POLL_MAX; ++j) {
        const int i = base + lane + j * WAVE;
        v[j] = ll_load(i < n ? ll_at(src, start + i) : spare);
      }
    };
    auto check = [&](const uint64_t (&v)[POLL_MAX]) {
#pragma unroll
      for (int j = 0; j < POLL_MAX; ++j)
        if (!((done >> j) & 1u) && (uint32_t)(v[j] >> (64 - TAGB)) == tag) {
          sink(base + lane + j * WAVE, v[j] & PAY);
          done |= 1ull << j;
        }
    };
    issue(a);
    while (true) {
      issue(b);
      check(a);
      if (__all(done == ALL)) break;
      issue(a);
      check(b);
      if (__all(done == ALL)) break;
      const uint64_t now = __builtin_amdgcn_s_memrealtime();
      waited += min(now - last, WAIT_STEP_MAX);
      last = now;
      if (waited > WAIT_TICKS) {
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
// N independent wave sums, step by step in lockstep so that consecutive DPP operations never
// depend on each other; every lane receives every sum.
template <int N>
__device__ __forceinline__ void wave_sum_n(float (&v)[N]) {
#pragma unroll
  for (int i = 0; i < N; ++i) v[i] = dpp_add<0x111, 0xf>(v[i]);
#pragma unroll
  for (int i = 0; i < N; ++i) v[i] = dpp_add<0x112, 0xf>(v[i]);
#pragma unroll
  for (int i = 0; i < N; ++i) v[i] = dpp_add<0x114, 0xf>(v[i]);
#pragma unroll
  for (int i = 0; i < N; ++i) v[i] = dpp_add<0x118, 0xf>(v[i]);
#pragma unroll
  for (int i = 0; i < N; ++i) v[i] = dpp_add<0x142, 0xa>(v[i]);
#pragma unroll
  for (int i = 0; i < N; ++i) v[i] = dpp_add<0x143, 0xc>(v[i]);
#pragma unroll
  for (int i = 0; i < N; ++i) v[i] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v[i]), 63));
}

__device__ __forceinline__ uint32_t order_bits(float v) {
  uint32_t u = __float_as_uint(v);
  if (u == 0x80000000u) u = 0;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Sorts N keys of one lane into descending order (Batcher's odd-even merge network; N a power of 2).
template <int N>
__device__ __forceinline__ void sort_desc(uint64_t (&k)[N]) {
#pragma unroll
  for (int p = 1; p < N; p <<= 1)
#pragma unroll
    for (int q = p; q >= 1; q >>= 1)
#pragma unroll
      for (int j = q % p; j + q < N; j += 2 * q)
#pragma unroll
        for (int i = 0; i < q && i + j + q < N; ++i)
          if ((i + j) / (2 * p) == (i + j + q) / (2 * p)) {
            const uint64_t a = k[i + j], b = k[i + j + q];
            k[i + j] = a > b ? a : b;
            k[i + j + q] = a > b ? b : a;
          }
}

// Softmax top-K of E logits held in LDS (one wave, VPL >= E / 64 logits per lane); idx/w land in
// lanes 0..K-1 (larger logit first; equal logits by lower expert index).  Each lane first sorts its
// own VPL keys, so a round needs the wave maximum of one 32-bit word, the lanes' heads: the winner
// is the lane holding it (found by a ballot), which then drops its head.  Only when several heads
// share that word (equal logits) does a second maximum, over the index word, decide.  The weights
// follow the same arithmetic in the same order as a plain K-round selection would.
template <int VPL>
__device__ __forceinline__ void wave_topk_v(const float* lt, int E, int K, uint32_t flags, int& out_e, float& out_w) {
  const int lane = threadIdx.x % WAVE;
  uint64_t key[VPL];
  float val[VPL];
#pragma unroll
  for (int j = 0; j < VPL; ++j) {
    const int e = lane + j * WAVE;
    val[j] = e < E ? lt[e] : 0.f;
    key[j] = e < E ? ((uint64_t)order_bits(val[j]) << 32) | (uint32_t)(0xFFFFFFFFu - (uint32_t)e) : 0ull;
  }
  sort_desc<VPL>(key);
  float top = 0.f, mine_v = 0.f;
  int mine_e = 0;
  for (int k = 0; k < K; ++k) {
    const uint32_t hh = (uint32_t)(key[0] >> 32);
    const uint32_t hi = wave_max_u32(hh);
    uint64_t m = __ballot(hh == hi);
    uint32_t lo;
    if (__popcll(m) == 1) {
      lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)key[0], (int)__builtin_ctzll(m));
    } else {
      lo = wave_max_u32(hh == hi ? (uint32_t)key[0] : 0u);
      m = __ballot(key[0] == (((uint64_t)hi << 32) | lo));
    }
    if (lane == (int)__builtin_ctzll(m)) {
#pragma unroll
      for (int j = 0; j + 1 < VPL; ++j) key[j] = key[j + 1];
      key[VPL - 1] = 0;
    }
    const float v = __uint_as_float((hi & 0x80000000u) ? (hi & 0x7FFFFFFFu) : ~hi);
    if (k == 0) top = v;
    if (lane == k) {
      mine_e = (int)(0xFFFFFFFFu - lo);
      mine_v = v;
    }
  }
  const float x = expf(mine_v - top);
  float den = 0.f;
  if (flags & MOE_TOPK_RENORM) {
    for (int k = 0; k < K; ++k) den += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), k));
  } else {
    float part = 0.f;
#pragma unroll
    for (int j = 0; j < VPL; ++j)
      if (lane + j * WAVE < E) part += expf(val[j] - top);
    den = wave_sum(part);
  }
  out_e = mine_e;
  out_w = x / den;
}
// VPL from E: each lane holds only the E / 64 keys it needs (rather than the 16 of the largest E),
// which keeps its sort and its per-round shift short.  A single wave issues at a quarter of the
// SIMD's rate, so the selection is a chain of dependent instructions: K = 8 of 256 took 2.5 us as
// K rounds of two wave maxima over unsorted keys, 2.0 us with sorted heads.
__device__ __forceinline__ void wave_topk(const float* lt, int E, int K, uint32_t flags, int& out_e, float& out_w) {
  if (E <= 4 * WAVE)
    wave_topk_v<4>(lt, E, K, flags, out_e, out_w);
  else if (E <= 8 * WAVE)
    wave_topk_v<8>(lt, E, K, flags, out_e, out_w);
  else
    wave_topk_v<MOE_MAX_E / WAVE>(lt, E, K, flags, out_e, out_w);
}

__device__ __forceinline__ float gelu_erf(float a) { return 0.5f * a * (1.f + erff(a * 0.70710678118654752f)); }

// ------------------------------------------------------------------------------------------
// Per-layer weight loads held in registers between phases.
//
// The compute waves issue a phase's loads one phase early and consume them after the next
// barriers.  The hardware counter that orders those waits retires memory operations in issue
// order, so a vector load whose value is needed at once would also wait for every prefetch
// before it.  Hence: descriptor fields are read through the constant address space (scalar
// loads, counted apart), per-row biases travel with the prefetched weights, and the gate/up and
// down loads are unconditional (an item past the end re-reads the last item, and its result is
// not stored).  Head, fc2 and router rows go one per wave in the order (wave, workgroup), so the
// rows past the first G*MW land one per workgroup; a wave without such a row skips it (a
// branch uniform over the wave).
typedef const __attribute__((address_space(4))) moe_decode_layer* layer_cptr;

__device__ __forceinline__ layer_cptr layer_at(const StepParams& p, int l) { return (layer_cptr)(p.layers + l); }

// Whether layer l carries a head that predicts layer l+1.
__device__ __forceinline__ bool has_head(const StepParams& p, int l) {
  return !p.given && l + 1 < p.L && layer_at(p, l)->head.fc1_x != nullptr;
}

template <int BITS, int PG, int NSH, int NSF, int GU, int NH>
struct ABuf {  // gate/up row pairs, head linear/fc1 rows (+ K-hot terms, biases), previous head's fc2 row
  uint4 qg[GU][PG], qu[GU][PG];
  uint16_t sg[GU][PG], bg[GU][PG], su[GU][PG], bu[GU][PG];
  int item[GU];
  bool bad[GU];
  bool ok[GU];               // false: a repeat of the last item, not stored
  // head rows (none in a variant for stacks without heads, NH = 0: the head code folds away)
  uint4 hr[NH > 0 ? NH : 1][NSH];
  uint16_t kh[NH > 0 ? NH : 1], hb[NH > 0 ? NH : 1];  // raw float16: converted where used, so the loads stay in flight
  int khm;                  // K-hot term of this lane: 0 none, 1 the table value, 2 NaN (bad index)
  uint4 fr[NSF];            // fc2 row of the previous layer's head
  uint16_t fb;
};
template <int BITS, int NSF, int PD>
struct BBuf {  // down (expert, row group) items
  uint4 q[PD];
  uint16_t s[PD], b[PD];
  int k[PD], jr[PD];
  bool bad[PD];
  bool ok[PD];
};

// Head rows are numbered fc1 rows first (0..H-1), then linear rows (H..H+E-1); row r (r < NH) of
// a wave's head rows is head_row(r).  The wave that computes linear row e also computes fc2 row e
// (lin_row), so the linear output never leaves its registers; with H a multiple of the workgroup
// count those waves are the ones without an fc1 row.  e_row: the wave's router row.
__device__ __forceinline__ int head_row(const StepParams& p, int r, int wg, int cw) { return (r * MW + cw) * p.G + wg; }
__device__ __forceinline__ int e_row(const StepParams& p, int wg, int cw) { return cw * p.G + wg; }
template <int NH>
__device__ __forceinline__ int lin_row(const StepParams& p, int wg, int cw) {
#pragma unroll
  for (int r = 0; r < NH; ++r) {
    const int j = head_row(p, r, wg, cw);
    if (j >= p.H && j < p.H + p.E) return j - p.H;
  }
  return -1;
}

// Loads of phase A of layer l, in two parts: the gate/up rows (needed first), and the head rows of
// layer l plus the fc2 row of the head of layer l-1 when fc2_of_prev (the second half of that head
// runs in this phase; both are needed only after the SwiGLU outputs).  Descriptor fields are
// scalar loads.
template <int BITS, int PG, int NSH, int NSF, int GU, int NH>
__device__ __forceinline__ void issue_A_gu(const StepParams& p, int l, const int* re, int wg, int cw, int lane,
                                           ABuf<BITS, PG, NSH, NSF, GU, NH>& a) {
  const layer_cptr D = layer_at(p, l);
  const int gw = wg * MW + cw;
  const int wpr = p.d * BITS / 32, ngr = p.d >> p.lg2g;
  const int items = p.K * p.I;
#pragma unroll
  for (int u = 0; u < GU; ++u) {
    a.ok[u] = gw * GU + u < items;
    const int item = min(gw * GU + u, items - 1);
    const int k = item / p.I, i = item - k * p.I;
    int e = re[k];
    a.bad[u] = (unsigned)e >= (unsigned)p.E;
    e = a.bad[u] ? 0 : e;
    a.item[u] = item;
    const size_t row = (size_t)e * p.I + i;
#pragma unroll
    for (int q = 0; q < PG; ++q) {
      const int seg = lane + q * WAVE;
      const size_t wo = row * wpr + (size_t)seg * 4;
      a.qg[u][q] = *reinterpret_cast<const uint4*>(D->experts.gate.q + wo);
      a.qu[u][q] = *reinterpret_cast<const uint4*>(D->experts.up.q + wo);
      const size_t go = row * ngr + ((seg * SegT<BITS>::COLS) >> p.lg2g);
      a.sg[u][q] = D->experts.gate.scales[go];
      a.bg[u][q] = D->experts.gate.biases[go];
      a.su[u][q] = D->experts.up.scales[go];
      a.bu[u][q] = D->experts.up.biases[go];
    }
  }
}
template <int BITS, int PG, int NSH, int NSF, int GU, int NH>
__device__ __forceinline__ void issue_A_head(const StepParams& p, int l, const int* re, const int* prev,
                                             bool fc2_of_prev, int wg, int cw, int lane,
                                             ABuf<BITS, PG, NSH, NSF, GU, NH>& a) {
  const layer_cptr D = layer_at(p, l);
  if (NH > 0 && has_head(p, l)) {
    // K-hot gather: lane j < K reads row cur[j] of the routing table, lane K <= j < 2K row
    // E + prev[j - K] (none at the first token); other lanes re-read row cur[0] and add 0.
    const int j = lane < 2 * p.K ? lane : 0;
    const bool is_prev = j >= p.K;
    const bool use = lane < 2 * p.K && (!is_prev || prev != nullptr);
    int e = is_prev ? (prev ? prev[j - p.K] : 0) : re[j];
    const bool bad = (unsigned)e >= (unsigned)p.E;
    e = bad ? 0 : e;
    const int trow = is_prev && prev ? p.E + e : e;
    a.khm = use ? (bad ? 2 : 1) : 0;
#pragma unroll
    for (int r = 0; r < NH; ++r) {
      const int row = head_row(p, r, wg, cw);
      if (row >= p.H + p.E) break;  // uniform over the wave
      const bool fc1 = row < p.H;
      const int c = fc1 ? row : row - p.H;
      const uint16_t* W = (fc1 ? D->head.fc1_x : D->head.lin_x) + (size_t)c * p.d;
#pragma unroll
      for (int sg = 0; sg < NSH; ++sg) a.hr[r][sg] = *reinterpret_cast<const uint4*>(W + (size_t)(lane + sg * WAVE) * 8);
      const uint16_t* rtab = fc1 ? D->head.fc1_r : D->head.lin_r;
      a.kh[r] = rtab[(size_t)trow * (fc1 ? p.H : p.E) + c];
      const uint16_t* bias = fc1 ? D->head.fc1_b : D->head.lin_b;
      a.hb[r] = bias ? bias[c] : *p.zero16;
    }
  }
  const int row = lin_row<NH>(p, wg, cw);
  if (fc2_of_prev && row >= 0) {  // uniform over the wave
    const uint16_t* fc2 = layer_at(p, l - 1)->head.fc2;
    const uint16_t* fc2_b = layer_at(p, l - 1)->head.fc2_b;
#pragma unroll
    for (int sg = 0; sg < NSF; ++sg)
      a.fr[sg] = *reinterpret_cast<const uint4*>(fc2 + (size_t)row * p.H + (size_t)(lane + sg * WAVE) * 8);
    a.fb = fc2_b ? fc2_b[row] : *p.zero16;
  }
}
template <int BITS, int PG, int NSH, int NSF, int GU, int NH>
__device__ __forceinline__ void issue_A(const StepParams& p, int l, const int* re, const int* prev, bool fc2_of_prev,
                                        int wg, int cw, int lane, ABuf<BITS, PG, NSH, NSF, GU, NH>& a) {
  issue_A_gu(p, l, re, wg, cw, lane, a);
  issue_A_head(p, l, re, prev, fc2_of_prev, wg, cw, lane, a);
}

template <int BITS, int NSF, int PD>
__device__ __forceinline__ void issue_B(const StepParams& p, int l, const int* re, int wg, int cw, int lane,
                                        BBuf<BITS, NSF, PD>& b) {
  const layer_cptr D = layer_at(p, l);
  const int wpr = p.I * BITS / 32, ngr = p.I >> p.lg2g;
  const int RPI = WAVE / p.Ldn, slot = lane / p.Ldn;
  const int ls = min(lane % p.Ldn, p.I * BITS / 128 - 1);
  const int npairs = p.K * p.DI;
#pragma unroll
  for (int u = 0; u < PD; ++u) {
    const int pk = min(cw + u * MW, npairs - 1);
    const int k = pk / p.DI, q = pk - k * p.DI;
    int e = re[k];
    b.bad[u] = (unsigned)e >= (unsigned)p.E;
    e = b.bad[u] ? 0 : e;
    b.ok[u] = cw + u * MW < npairs;
    b.k[u] = k;
    b.jr[u] = q * RPI + slot;
    const int j = min(wg * p.DR + b.jr[u], p.d - 1);
    const size_t row = (size_t)e * p.d + j;
    b.q[u] = *reinterpret_cast<const uint4*>(D->experts.down.q + row * wpr + (size_t)ls * 4);
    const size_t go = row * ngr + ((ls * SegT<BITS>::COLS) >> p.lg2g);
    b.s[u] = D->experts.down.scales[go];
    b.b[u] = D->experts.down.biases[go];
  }
}

struct StepShared {
  uint16_t h[2][LDS_D];
  float act_f[LDS_ACT];  // the SwiGLU outputs of all K experts, as received
  // the same as float16 hi + lo parts (act ~ hi + lo), in the permuted pair order of the down
  // projection's code words (see act_pos); made by all compute waves together
  uint16_t act_hi[LDS_ACT], act_lo[LDS_ACT];
  float g[LDS_H];
  float logit[LDS_E];
  float part[LDS_PART];
  float aout[MW * 4];   // this workgroup's SwiGLU outputs of the phase, gathered for one store
  int route_e[LDS_LK];  // this token's routing of every layer: [l * K + k]
  float route_w[LDS_LK];
  int prev_e[LDS_LK];   // the previous token's routing (K-hot "previous" input of the heads)
  // Last, so that the arrays above keep LDS offsets below 64 KiB (the immediate offset of a ds
  // instruction is 16 bits; past it every access needs an address register):
  uint16_t gain[2][LDS_D];  // input-norm gains of layers l and l+1 (by layer parity), staged by the compute waves
  uint16_t xg[LDS_D];       // gain * h_l, formed by the compute waves once h_l is in (gained layers only)
  uint16_t rrow[LDS_RR];    // router rows of a self-routed layer, staged by the compute waves: slot cw holds row cw * G + wg
  uint64_t act_w[LDS_ACT / 2];  // the act words' payloads as received (two 24-bit floats each; RAW_ACT)
};

struct StepCtx {
  int wg, lane, cw, gw;
  const uint64_t* spare;  // this workgroup's own line in the workspace (the target of spare polling slots)
  uint32_t epoch;
  int32_t *cur_i, *nxt_i;
  float *cur_w, *nxt_w;
  const int32_t* prev_i;
  __device__ uint32_t tag(int ph) const { return ((epoch << 10) | (uint32_t)ph) ^ TAG_SALT; }
  // 16-bit tag of the packed act words: 9 bits of phase, 7 of the token counter.  Every act word
  // is rewritten in every layer of every token, so a word 128 tokens old cannot still be there.
  __device__ uint32_t tag16(int ph) const { return (((epoch & 0x7Fu) << 9) | (uint32_t)ph) ^ (TAG_SALT & 0xFFFFu); }
};

__device__ __forceinline__ bool self_routed(const StepParams& p, int l) {
  return !p.given && (p.bootstrap || l == 0 || !has_head(p, l - 1));
}

// Position of SwiGLU output n (n = k*I + column) in the LDS hi/lo arrays: the down projection's
// 16-byte segment of 32/BITS-column words pairs column j of a word with column j + PAIRS_PER_WORD
// (the two halves of one decoded code pair), so the activations are stored pair by pair.
template <int BITS>
__device__ __forceinline__ int act_pos(int n) {
  constexpr int PPW = SegT<BITS>::PAIRS_PER_WORD, CPW = 2 * PPW;
  return (n & ~(CPW - 1)) + 2 * (n & (PPW - 1)) + ((n / PPW) & 1);
}
template <int BITS>
__device__ __forceinline__ void put_act(StepShared& sm, int n, float f) {
  const _Float16 hi = (_Float16)f;
  const _Float16 lo = (_Float16)(f - (float)hi);
  const int q = act_pos<BITS>(n);
  sm.act_hi[q] = __builtin_bit_cast(uint16_t, hi);
  sm.act_lo[q] = __builtin_bit_cast(uint16_t, lo);
}

// Wave 0 of every workgroup: waits for the vectors each phase needs and unpacks them into LDS.
// GW0: 32-bit words of a d-row per lane (d = NSH 64 lanes x 8 halves).
// RAW_ACT: the act words go to LDS as received and the compute waves unpack them (the stacks
// without heads, whose layers all route themselves: there the poll wave's work per act word is on
// the critical path, measured 1-2 % per token; with heads unpacking here measured faster).
template <int BITS, int GW0, bool STAMP, bool RAW_ACT>
__device__ __forceinline__ void sync_role(const StepParams& p, const StepCtx& c, StepShared& sm) {
  const int lane = c.lane, dh = p.d / 2;
  bool failed = false;
  for (int l = 0; l < p.L; ++l) {
    const int hb = l & 1;
    uint32_t* hw = reinterpret_cast<uint32_t*>(sm.h[hb]);
    stamp<STAMP>(p, c.wg, l, 0);
    // (the RMS norm of h_l is taken by the compute waves from their own reads of it, in a fixed
    // order; summed here, as the words arrive, it would depend on their arrival order)
    if (l == 0) {
      for (int m = lane; m < dh; m += WAVE) hw[m] = reinterpret_cast<const uint32_t*>(p.h_in)[m];
      if (p.h_layers != nullptr && c.wg == 0)  // row 0 of the per-layer copies: the token's input
        for (int m = lane; m < dh; m += WAVE) reinterpret_cast<uint32_t*>(p.h_layers)[m] = hw[m];
    } else {
      ll_wait(p.ll_h + (size_t)(c.wg % p.xr_h) * p.h_stride, (size_t)l * dh, dh, c.tag(3 * (l - 1) + 2), p.err, failed, c.spare,
              [&](int i, uint32_t v) { hw[i] = v; });
    }
    stamp<STAMP>(p, c.wg, l, 1);
    lds_barrier();  // B1: h_l ready
    if (p.gained) lds_barrier();  // B1g: gain * h_l formed
    if (self_routed(p, l)) {
      ll_wait(p.ll_logits, 0, p.E << p.lshift, c.tag(3 * l), p.err, failed, c.spare, [&](int i, uint32_t v) { sm.logit[i >> p.lshift] = __uint_as_float(v); });
      int e;
      float w;
      stamp<STAMP>(p, c.wg, l, 15);
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
    lds_barrier();  // BA: this workgroup's SwiGLU outputs gathered (the compute waves store them)
    ll_wait<16>(p.ll_act + (size_t)(c.wg % p.xr_a) * p.act_stride, 0, p.K * p.I / 2, c.tag16(3 * l + 1), p.err, failed, c.spare,
                [&](int i, uint64_t v) {
      if constexpr (RAW_ACT) {
        sm.act_w[i] = v;
      } else {
        sm.act_f[2 * i] = f24_to_f32((uint32_t)v & 0xFFFFFFu);
        sm.act_f[2 * i + 1] = f24_to_f32((uint32_t)(v >> 24) & 0xFFFFFFu);
      }
    });
    stamp<STAMP>(p, c.wg, l, 2);
    lds_barrier();  // B3: act ready
    lds_barrier();  // B3b: act split into hi/lo pairs (by the compute waves)
    lds_barrier();  // B4: partial down sums ready (the combine runs in wave 1)
    // The head's hidden vector g_l feeds its fc2 rows in phase A of layer l+1; fetching it here
    // overlaps the wait for h_{l+1} instead of lengthening the act exchange.  This workgroup's
    // part of h_{l+1} has already left, so another workgroup may be writing g_{l+1} meanwhile:
    // g alternates between two buffers by layer parity (g_{l+2}, the next write into this
    // buffer, needs h_{l+2}, which needs this workgroup's combine of layer l+1, which comes after
    // this read).
    if (has_head(p, l))
      ll_wait(p.ll_g, (size_t)(l & 1) * p.H, p.H, tA, p.err, failed, c.spare,
              [&](int i, uint32_t v) { sm.g[i] = __uint_as_float(v); });
  }
  // Top-K of every head, off the token's critical path: head l predicts layer l+1's routing for
  // the next token; workgroup l % G handles head l.
  for (int l = c.wg; l + 1 < p.L; l += p.G) {
    if (!has_head(p, l)) continue;
    ll_wait(p.ll_hlog, (size_t)l * p.E, p.E, c.tag(3 * l + 2), p.err, failed, c.spare,
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
template <int BITS, int PG, int NSH, int NSF, int GU, int PD, int NH, bool STAMP>
__device__ __forceinline__ void compute_role(const StepParams& p, const StepCtx& c, StepShared& sm) {
  using GS = SegT<BITS>;
  const int cw = c.cw, wg = c.wg, dh = p.d / 2, K = p.K;
  int lane = c.lane;
  const __amdgpu_buffer_rsrc_t ws = buffer_of(p.ws, p.ws_bytes);
  const __amdgpu_buffer_rsrc_t hout = buffer_of(p.h_out, (uint32_t)p.d * 2);
  // per-layer copies of h: a zero-sized buffer when not asked for, so every store is dropped
  const __amdgpu_buffer_rsrc_t hall = buffer_of(p.h_layers, p.h_layers ? (uint32_t)(p.L + 1) * p.d * 2 : 0u);
  bool lead = lane == 0;
  ABuf<BITS, PG, NSH, NSF, GU, NH> A;
  BBuf<BITS, NSF, PD> B;
  float lin_keep = 0.f, lin_keep_next = 0.f;  // this wave's linear-row output of heads l-1 and l
  // Layer l's input-norm gain into LDS buffer l & 1, split over the compute waves (a few words per
  // lane, all loads first): layer 0's before the first barrier, layer l+1's while waiting for the
  // act exchange of layer l (buffer (l+1) & 1 was last read at layer l-1).
  const auto stage_gain = [&](int l) {
    if (!p.gained) return;
    const uint32_t* gs = reinterpret_cast<const uint32_t*>(layer_at(p, l)->norm_gain);
    constexpr int NWL = (NSH * 4 + MW - 1) / MW;  // words per lane: d/2 words over MW waves
    uint32_t gv[NWL];
#pragma unroll
    for (int j = 0; j < NWL; ++j) gv[j] = gs[min(cw * WAVE + lane + j * MW * WAVE, dh - 1)];
    uint32_t* gw = reinterpret_cast<uint32_t*>(sm.gain[l & 1]);
#pragma unroll
    for (int j = 0; j < NWL; ++j) {
      const int m = cw * WAVE + lane + j * MW * WAVE;
      if (m < dh) gw[m] = gv[j];
    }
  };
  // A self-routed layer's router row of this wave goes straight from memory into LDS slot cw
  // (16-byte global-to-LDS loads: no registers held), issued a layer early; the router phase then
  // waits for it with the wave's other loads long done.  Slot cw holds row cw * G + wg.
  const auto stage_router = [&](int l) {
    const int r = e_row(p, wg, cw);
    if (!p.rstage || r >= p.E) return;  // uniform over the wave
    // the row as a buffer: one lane offset serves every piece, the piece's offset goes in soffset
    const __amdgpu_buffer_rsrc_t rb = buffer_of(layer_at(p, l)->router + (size_t)r * p.d, (uint32_t)p.d * 2);
#pragma unroll
    for (int sg = 0; sg < NSH; ++sg)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (__attribute__((address_space(3))) void*)(sm.rrow + (size_t)cw * p.d + sg * WAVE * 8),
                                               16, (uint32_t)lane * 16, (uint32_t)sg * WAVE * 16, 0, 0);
  };
  stage_gain(0);
  if (self_routed(p, 0)) stage_router(0);
  for (int l = 0; l < p.L; ++l) {
    // At d = 4096 (NSH = 8) the address arithmetic derived from the lane, hoisted out of this loop
    // and held for the whole token, pushed the compute waves past their registers: the spilled
    // values came back with waits on every outstanding load, prefetches included.  There the lane
    // is made opaque in each layer, so that arithmetic is redone per layer instead (no spills;
    // large-int4 413 -> 378 and large-int2 396 -> 374 us per token).  At d = 2048 the hoisted form
    // fits and is faster.
    if constexpr (NSH > 4) {
      asm volatile("" : "+v"(lane));
      lead = lane == 0;
    }
    const bool self = self_routed(p, l);
    const bool head = has_head(p, l);
    const bool fc2_now = l > 0 && has_head(p, l - 1);  // fc2 of head l-1 runs in this layer
    const bool prefetch = l + 1 < p.L && !self_routed(p, l + 1);
    const int hb = l & 1;
    lds_barrier();  // B1
    stamp<STAMP>(p, wg, l, 3, cw == 0);
    float scale;  // 1 / rms(h_l), from this wave's own reads of h_l (a fixed summation order)
    const uint16_t* hl = sm.h[hb];
    // a layer with a norm gain: the gate/up dot products take g * h as float16 pairs, formed here
    // by all compute waves together (the router and head rows form the products in float32
    // themselves); the sum of squares stays that of h
    const bool gn = p.gained != 0;
    if (gn) {
      const uint32_t* hw = reinterpret_cast<const uint32_t*>(hl);
      const uint32_t* gw = reinterpret_cast<const uint32_t*>(sm.gain[l & 1]);
      uint32_t* xw = reinterpret_cast<uint32_t*>(sm.xg);
      for (int m = cw * WAVE + lane; m < dh; m += MW * WAVE)
        xw[m] = __builtin_bit_cast(uint32_t, as_h2(hw[m]) * as_h2(gw[m]));
      lds_barrier();  // B1g
    }
    const uint16_t* xl = gn ? sm.xg : hl;
    if (self) {
      // R_l: at most one router row per wave -> tagged logit
      const int r = e_row(p, wg, cw);
      if (r < p.E) {  // uniform over the wave
        uint4 wr[NSH];  // this wave's router row: slot cw of the staged rows, else from memory
        if (p.rstage) {
          __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the row's global-to-LDS loads have landed
          const uint4* W = reinterpret_cast<const uint4*>(sm.rrow + (size_t)cw * p.d);
#pragma unroll
          for (int sg = 0; sg < NSH; ++sg) wr[sg] = W[lane + sg * WAVE];
        } else {
          const uint4* W = reinterpret_cast<const uint4*>(layer_at(p, l)->router + (size_t)r * p.d);
#pragma unroll
          for (int sg = 0; sg < NSH; ++sg) wr[sg] = W[lane + sg * WAVE];
        }
        float red[2] = {0.f, 0.f};  // router dot, sum of squares of h_l
#pragma unroll
        for (int sg = 0; sg < NSH; ++sg) {
          const int g = lane + sg * WAVE;
          const uint4 wv = wr[sg];
          const uint4 xv = *reinterpret_cast<const uint4*>(hl + (size_t)g * 8);
          if (gn) {  // the routing decides indices: the gained product in float32, not rounded
            red[0] = dot8_gained(wv, xv, *reinterpret_cast<const uint4*>(sm.gain[l & 1] + (size_t)g * 8), red[0]);
          } else {
            red[0] = __builtin_amdgcn_fdot2(as_h2(wv.x), as_h2(xv.x), red[0], false);
            red[0] = __builtin_amdgcn_fdot2(as_h2(wv.y), as_h2(xv.y), red[0], false);
            red[0] = __builtin_amdgcn_fdot2(as_h2(wv.z), as_h2(xv.z), red[0], false);
            red[0] = __builtin_amdgcn_fdot2(as_h2(wv.w), as_h2(xv.w), red[0], false);
          }
          red[1] = __builtin_amdgcn_fdot2(as_h2(xv.x), as_h2(xv.x), red[1], false);
          red[1] = __builtin_amdgcn_fdot2(as_h2(xv.y), as_h2(xv.y), red[1], false);
          red[1] = __builtin_amdgcn_fdot2(as_h2(xv.z), as_h2(xv.z), red[1], false);
          red[1] = __builtin_amdgcn_fdot2(as_h2(xv.w), as_h2(xv.w), red[1], false);
        }
        wave_sum_n(red);
        const float acc = red[0] / sqrtf(red[1] / (float)p.d + RMS_EPS);
        // the logit in 1 << lshift consecutive words (one store from as many lanes): at E <= 256 four
        // writers share a 128-byte line instead of sixteen, and the exchange took 2.5 us against
        // 3.5 us; the pollers read the same count of lines as for the 1,024-word h
        ll_put(ws, p, p.ll_logits, ((size_t)r << p.lshift) + lane, lane < (1 << p.lshift), __float_as_uint(acc), c.tag(3 * l));
        stamp<STAMP>(p, wg, l, 10, cw == 0);
      }
      lds_barrier();  // B2
      stamp<STAMP>(p, wg, l, 11, cw == 0);
    }
    if (self || l == 0) {  // no earlier phase has loaded this layer's weights
      issue_A<BITS, PG, NSH, NSF, GU, NH>(p, l, sm.route_e + l * K, c.prev_i ? sm.prev_e + l * K : nullptr, fc2_now,
                                          wg, cw, lane, A);
      issue_B<BITS, NSF, PD>(p, l, sm.route_e + l * K, wg, cw, lane, B);
    }

    // ---- A_l: gate/up + SwiGLU, then linear and fc1 rows of head l, then fc2 rows of head l-1 ----
    // In order of urgency: the SwiGLU outputs gate the act exchange, g_l is needed a phase later,
    // and the head logits only at the end of the token, so they are computed while the exchange
    // is in flight.  Partials of one stage are reduced together (interleaved DPP chains).
    {
      const uint32_t tA = c.tag(3 * l + 1);
      {
        float red[2 * GU + 1];  // gate, up per pair | sum of squares of h_l
        uint32_t xp[PG][GS::PAIRS];
        float sx[PG][2], sq = 0.f;
#pragma unroll
        for (int q = 0; q < PG; ++q) load_xpairs<BITS>(xl + (size_t)(lane + q * WAVE) * GS::COLS, xp[q], sx[q], sq);
        if (gn) {  // the pairs above are of g * h: take the sum of squares from h itself
          sq = 0.f;
#pragma unroll
          for (int q = 0; q < PG; ++q) sq = sum_sq<GS::COLS>(hl + (size_t)(lane + q * WAVE) * GS::COLS, sq);
        }
#pragma unroll
        for (int u = 0; u < GU; ++u) {
          float pg = 0.f, pu = 0.f;
#pragma unroll
          for (int q = 0; q < PG; ++q) {
            float d0 = 0.f, d1 = 0.f;
            const float sxq = sx[q][0] + sx[q][1];
            dot_segment_biased<BITS>(A.qg[u][q], xp[q], d0, d1);
            const float s_g = h2f(A.sg[u][q]), s_u = h2f(A.su[u][q]);
            pg += s_g * (d0 + d1) + (h2f(A.bg[u][q]) - 1024.f * s_g) * sxq;
            d0 = d1 = 0.f;
            dot_segment_biased<BITS>(A.qu[u][q], xp[q], d0, d1);
            pu += s_u * (d0 + d1) + (h2f(A.bu[u][q]) - 1024.f * s_u) * sxq;
          }
          red[2 * u] = pg;
          red[2 * u + 1] = pu;
        }
        red[2 * GU] = sq;  // the segments of the 64 lanes cover all of h_l
        stamp<STAMP>(p, wg, l, 8, cw == 0);
        wave_sum_n(red);
        scale = 1.f / sqrtf(red[2 * GU] / (float)p.d + RMS_EPS);
#pragma unroll
        for (int u = 0; u < GU; ++u) {
          const float pg = red[2 * u] * scale, pu = red[2 * u + 1] * scale;
          const float a = pg / (1.f + expf(-pg)) * pu;
          if (lead) sm.aout[cw * GU + u] = A.bad[u] ? quiet_nan() : a;
        }
        stamp<STAMP>(p, wg, l, 9, cw == 0);
        // the workgroup's MW*GU consecutive outputs leave as one store of whole lines (partial
        // lines written by many waves were measured slower to reach the readers)
        lds_barrier();  // BA
        if (cw == 0) {  // lane j + n*copy sends outputs 2j, 2j+1 of the workgroup as one packed word of that copy
          constexpr int NW = MW * GU / 2;
          const int j = lane % NW, cpy = lane / NW;
          const int word = wg * NW + j;
          const uint64_t w = (uint64_t)f32_to_f24(sm.aout[2 * j]) | ((uint64_t)f32_to_f24(sm.aout[2 * j + 1]) << 24) |
                             ((uint64_t)c.tag16(3 * l + 1) << 48);
          ll_put64(ws, p, p.ll_act, (size_t)min(cpy, p.xr_a - 1) * p.act_stride + min(word, p.K * p.I / 2 - 1),
                   cpy < p.xr_a && 2 * word < p.K * p.I, w);
          stamp<STAMP>(p, wg, l, 4);
        }
      }
      // first half of this layer's head: fc1 rows (+GELU, sent) and the linear row (kept)
      if (NH > 0 && head && head_row(p, 0, wg, cw) < p.H + p.E) {  // uniform over the wave
        float red[2 * (NH > 0 ? NH : 1)];
#pragma unroll
        for (int r = 0; r < NH; ++r) {
          red[2 * r] = 0.f;
          red[2 * r + 1] = 0.f;
          if (head_row(p, r, wg, cw) < p.H + p.E) {  // uniform over the wave
            float acc = 0.f;
#pragma unroll
            for (int sg = 0; sg < NSH; ++sg) {
              const uint4 xv = *reinterpret_cast<const uint4*>(hl + (size_t)(lane + sg * WAVE) * 8);
              if (gn) {  // the head's logits decide the next token's experts: float32 gained products
                acc = dot8_gained(A.hr[r][sg], xv,
                                  *reinterpret_cast<const uint4*>(sm.gain[l & 1] + (size_t)(lane + sg * WAVE) * 8), acc);
              } else {
                acc = __builtin_amdgcn_fdot2(as_h2(A.hr[r][sg].x), as_h2(xv.x), acc, false);
                acc = __builtin_amdgcn_fdot2(as_h2(A.hr[r][sg].y), as_h2(xv.y), acc, false);
                acc = __builtin_amdgcn_fdot2(as_h2(A.hr[r][sg].z), as_h2(xv.z), acc, false);
                acc = __builtin_amdgcn_fdot2(as_h2(A.hr[r][sg].w), as_h2(xv.w), acc, false);
              }
            }
            red[2 * r] = acc;
            red[2 * r + 1] = A.khm == 1 ? h2f(A.kh[r]) : (A.khm == 2 ? quiet_nan() : 0.f);
          }
        }
        wave_sum_n(red);
#pragma unroll
        for (int r = 0; r < NH; ++r) {
          const int row = head_row(p, r, wg, cw);
          if (row < p.H + p.E) {  // uniform over the wave
            const float val = red[2 * r] * scale + red[2 * r + 1] + h2f(A.hb[r]);
            if (row >= p.H)
              lin_keep_next = val;  // linear row: this wave adds it to its fc2 row in the next layer
            else
              ll_put(ws, p, p.ll_g, (size_t)(l & 1) * p.H + row, lead, __float_as_uint(gelu_erf(val)), tA);
          }
        }
      }
      // second half of the previous layer's head: fc2 row `er` of this wave
      const int er = lin_row<NH>(p, wg, cw);
      if (fc2_now && er >= 0) {  // uniform over the wave
        float acc = 0.f;
#pragma unroll
        for (int sg = 0; sg < NSF; ++sg) {
          const float* gp = sm.g + (size_t)(lane + sg * WAVE) * 8;
          const half2_t w0 = as_h2(A.fr[sg].x), w1 = as_h2(A.fr[sg].y), w2 = as_h2(A.fr[sg].z),
                        w3 = as_h2(A.fr[sg].w);
          acc = fmaf((float)w0.x, gp[0], acc);
          acc = fmaf((float)w0.y, gp[1], acc);
          acc = fmaf((float)w1.x, gp[2], acc);
          acc = fmaf((float)w1.y, gp[3], acc);
          acc = fmaf((float)w2.x, gp[4], acc);
          acc = fmaf((float)w2.y, gp[5], acc);
          acc = fmaf((float)w3.x, gp[6], acc);
          acc = fmaf((float)w3.y, gp[7], acc);
        }
        ll_put(ws, p, p.ll_hlog, (size_t)(l - 1) * p.E + er, lead, __float_as_uint(wave_sum(acc) + lin_keep + h2f(A.fb)),
               c.tag(3 * (l - 1) + 2));
      }
      lin_keep = lin_keep_next;
      stamp<STAMP>(p, wg, l, 7, cw == 0);
    }
    if (l + 1 < p.L) stage_gain(l + 1);  // while the act exchange runs; its loads go before the prefetch's
    if (prefetch)  // gate/up weights of A_{l+1}, one phase early
      issue_A_gu<BITS, PG, NSH, NSF, GU, NH>(p, l + 1, sm.route_e + (l + 1) * K, wg, cw, lane, A);
    lds_barrier();  // B3
    // split act into float16 hi/lo pairs once per workgroup, every compute lane a few values
    for (int n = cw * WAVE + lane; n < K * p.I; n += MW * WAVE) {
      if constexpr (NH == 0)  // the poll wave stored the raw words (sync_role's RAW_ACT)
        put_act<BITS>(sm, n, f24_to_f32((uint32_t)(sm.act_w[n >> 1] >> (24 * (n & 1))) & 0xFFFFFFu));
      else
        put_act<BITS>(sm, n, sm.act_f[n]);
    }
    lds_barrier();  // B3b
    stamp<STAMP>(p, wg, l, 5, cw == 0);

    // ---- B_l: down partials of this workgroup's rows ----
    {
      const int S = p.I * BITS / 128;
      const int ls = lane % p.Ldn;
      const int lsc = min(ls, S - 1);
#pragma unroll
      for (int u = 0; u < PD; ++u) {
        const size_t so = (size_t)B.k[u] * p.I + (size_t)lsc * GS::COLS;  // segment start (halves)
        uint32_t hp[GS::PAIRS], lp[GS::PAIRS];
#pragma unroll
        for (int w = 0; w < GS::PAIRS / 4; ++w) {
          const uint4 a = reinterpret_cast<const uint4*>(sm.act_hi + so)[w];
          const uint4 b = reinterpret_cast<const uint4*>(sm.act_lo + so)[w];
          hp[4 * w] = a.x, hp[4 * w + 1] = a.y, hp[4 * w + 2] = a.z, hp[4 * w + 3] = a.w;
          lp[4 * w] = b.x, lp[4 * w + 1] = b.y, lp[4 * w + 2] = b.z, lp[4 * w + 3] = b.w;
        }
        float d0 = 0.f, d1 = 0.f, sx = 0.f;
        dot_segment_split_biased<BITS>(B.q[u], hp, lp, d0, d1);
        const half2_t one = {(_Float16)1.0f, (_Float16)1.0f};
#pragma unroll
        for (int j = 0; j < GS::PAIRS; ++j) {
          sx = __builtin_amdgcn_fdot2(as_h2(hp[j]), one, sx, false);
          sx = __builtin_amdgcn_fdot2(as_h2(lp[j]), one, sx, false);
        }
        const float s_d = h2f(B.s[u]);
        float po = ls < S ? s_d * (d0 + d1) + (h2f(B.b[u]) - 1024.f * s_d) * sx : 0.f;
        stamp<STAMP>(p, wg, l, 13, cw == 0);
        po = group_sum_last(po, p.Ldn);
        if (ls == p.Ldn - 1 && B.ok[u]) sm.part[B.k[u] * p.DR + B.jr[u]] = B.bad[u] ? quiet_nan() : po;
      }
    }
    stamp<STAMP>(p, wg, l, 14, cw == 0);
    if (prefetch)  // weights of B_{l+1}, one phase early
      issue_B<BITS, NSF, PD>(p, l + 1, sm.route_e + (l + 1) * K, wg, cw, lane, B);
    lds_barrier();  // B4
    stamp<STAMP>(p, wg, l, 12, cw == 0);
    // ---- combine + residual of this workgroup's rows -> h_{l+1} (wave 1; lane = row) ----
    if (cw == 0) {
      const int nrows = min(p.DR, p.d - wg * p.DR);  // >= 2 and even: the last workgroup may hold fewer
      const int jr = min(lane, nrows - 1);
      const int j = wg * p.DR + jr;
      const bool mine = lane < nrows;
      float acc = 0.f;
      for (int k = 0; k < K; ++k) acc = fmaf(sm.route_w[l * K + k], sm.part[k * p.DR + jr], acc);
      const uint32_t yb = f2h(h2f(hl[j]) + acc);
      __builtin_amdgcn_raw_buffer_store_b16((unsigned short)yb, hall, mine ? (uint32_t)((l + 1) * p.d + j) * 2 : OFF_NONE,
                                            0, 0);
      if (l + 1 == p.L) {
        __builtin_amdgcn_raw_buffer_store_b16((unsigned short)yb, hout, mine ? (uint32_t)j * 2 : OFF_NONE, 0, 0);
      } else {
        // lane m + n*copy sends word m (rows 2m, 2m+1) of that copy
        const int nw = nrows / 2, m = lane % nw, cpy = lane / nw;
        const uint32_t lo = __shfl(yb, 2 * m, WAVE), hi = __shfl(yb, 2 * m + 1, WAVE);
        ll_put(ws, p, p.ll_h, (size_t)min(cpy, p.xr_h - 1) * p.h_stride + (size_t)(l + 1) * dh + wg * (p.DR / 2) + m,
               cpy < p.xr_h, lo | (hi << 16), c.tag(3 * l + 2));
      }
      stamp<STAMP>(p, wg, l, 6);
    }
    // The head half of A_{l+1}'s weights (needed only after its SwiGLU outputs) goes out after the
    // combine: issued together with the gate/up half it slowed the act exchange that follows.
    if (prefetch)
      issue_A_head<BITS, PG, NSH, NSF, GU, NH>(p, l + 1, sm.route_e + (l + 1) * K,
                                               c.prev_i ? sm.prev_e + (l + 1) * K : nullptr, head, wg, cw, lane, A);
    if (l + 1 < p.L && self_routed(p, l + 1)) stage_router(l + 1);
  }
}

template <int BITS, int PG, int NSH, int NSF, int GU, int PD, int NH, bool STAMP>
__global__ void __launch_bounds__(NTHREADS) k_decode_step(StepParams p) {
  __shared__ __attribute__((aligned(16))) StepShared sm;
  StepCtx c;
  c.wg = blockIdx.x;
  c.lane = threadIdx.x % WAVE;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / WAVE);
  c.cw = wave - 1;
  c.gw = c.wg * MW + c.cw;
  c.spare = p.spare + (size_t)c.wg * 8;
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
  if (wave == 0) {
    sync_role<BITS, NSH * 4, STAMP, NH == 0>(p, c, sm);
  } else {
    // (all waves at the same issue priority: raising the compute waves' above the polling wave's,
    // which shares SIMD 0 with two of them, was measured 2 % slower per token)
    compute_role<BITS, PG, NSH, NSF, GU, PD, NH, STAMP>(p, c, sm);
  }
  if (c.wg == 0 && threadIdx.x == 0) *p.epoch = c.epoch + 1;
}

}  // namespace

// ------------------------------------------------------------------------------------------ host
struct StepPlan {
  bool ok;
  int G, GU, NH, NR, NO, DR, DI, PD, Ldn, PG, NSH, NSF;
};

static bool has_variant(int bits, int PG, int NSH, int NSF, int GU, int PD, int NH);

constexpr int SPARE_WGS = 1024;  // spare polling lines: one per workgroup

static StepPlan plan_step(const moe_decode_stack& st, int cus) {
  StepPlan pl{};
  const int d = st.d_model, I = st.d_ff, E = st.E, K = st.K, H = st.d_hidden, bits = st.bits;
  if (cus < 1 || d % 512 || d > LDS_D || (d * bits / 128) % WAVE) return pl;
  pl.PG = d * bits / 128 / WAVE;
  pl.NSH = d / 512;
  const int SI = I * bits / 128;
  if (SI < 1 || SI > WAVE || (I * bits) % 128) return pl;
  if (bits == 2 && st.group < 64) return pl;  // a 2-bit segment must sit inside one group
  if (K > 8 || K * I > LDS_ACT || E > LDS_E || st.L * K > LDS_LK) return pl;
  if (3 * st.L > 512) return pl;  // phases must fit the 9 phase bits of the packed act tags
  pl.Ldn = 1;
  while (pl.Ldn < SI) pl.Ldn <<= 1;
  const int RPI = WAVE / pl.Ldn;
  // down rows per workgroup: a multiple of the rows one wave covers at once, and even (h travels
  // as float16 pairs); then as many workgroups as it takes to cover d, each owning >= 2 rows
  pl.DR = (d + cus - 1) / cus;
  pl.DR = (pl.DR + RPI - 1) / RPI * RPI;
  pl.DR += pl.DR & 1;
  if (pl.DR > WAVE || K * pl.DR > LDS_PART) return pl;
  pl.G = (d + pl.DR - 1) / pl.DR;
  if (pl.G > SPARE_WGS) return pl;  // one spare polling line per workgroup
  const int GW = pl.G * MW;
  pl.DI = (pl.DR + RPI - 1) / RPI;
  pl.PD = (K * pl.DI + MW - 1) / MW;
  pl.GU = (K * I + GW - 1) / GW;
  pl.NR = (E + GW - 1) / GW;
  pl.NO = (E + GW - 1) / GW;
  if (pl.NR > 1 || pl.NO > 1) return pl;  // one router row and one fc2 row per compute wave
  if (H > 0) {
    if (H % 512 || H > LDS_H) return pl;
    pl.NSF = H / 512;
    pl.NH = (H + E + GW - 1) / GW;
    if (pl.NH > NH_MAX) return pl;
  } else {
    pl.NSF = 1;
    pl.NH = 0;
  }
  pl.ok = has_variant(bits, pl.PG, pl.NSH, pl.NSF, pl.GU, pl.PD, pl.NH);
  return pl;
}

struct StepWs {
  size_t epoch, err, zero, logits, act, g, hlog, h, spare, total;
};
constexpr int XR_MAX = 8;  // copies of h and of the SwiGLU outputs (one per XCD)
static StepWs step_ws(const moe_decode_stack& st) {
  StepWs w{};
  w.epoch = 0;
  w.err = 4;
  w.zero = 8;  // 8 bytes that stay zero
  w.logits = 256;
  w.act = w.logits + ll_bytes(4 * (size_t)st.E);  // E logits, each in up to 4 words
  w.g = w.act + XR_MAX * ll_bytes((size_t)st.K * st.d_ff);
  w.hlog = w.g + ll_bytes(st.d_hidden > 0 ? 2 * (size_t)st.d_hidden : 1);  // two buffers, by layer parity
  w.h = w.hlog + ll_bytes((size_t)st.L * st.E);
  w.spare = w.h + XR_MAX * ll_bytes((size_t)(st.L + 1) * (st.d_model / 2));
  w.total = w.spare + (size_t)SPARE_WGS * 64;
  return w;
}

static int device_cus() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  return cus;
}

template <int BITS, int PG, int NSH, int NSF, int GU, int PD, int NH>
static hipError_t go(hipStream_t s, const StepParams& p) {
  int occ = 0;
  auto k = p.stamps ? k_decode_step<BITS, PG, NSH, NSF, GU, PD, NH, true> : k_decode_step<BITS, PG, NSH, NSF, GU, PD, NH, false>;
  hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, k, NTHREADS, 0);
  if (e != hipSuccess) return e;
  if (occ < 1) return hipErrorInvalidConfiguration;  // every workgroup must be resident at once
  return launch(k, dim3(p.G), dim3(NTHREADS), 0, s, p);
}

// Instantiated shapes: (bits, gate/up segments per lane, fp16 segments per lane of a d-row and of
// an H-row, gate/up pairs per wave, down items per wave, head-row slots per wave).  The counts
// are exact, so every compute wave issues the same loads.
#define MOE_STEP_VARIANTS(X)                                                                       \
  X(4, 1, 4, 2, 1, 1, 1) /* d 2048, I 512, K 4, E 256, head hidden 1024 */                         \
  X(4, 1, 4, 1, 2, 2, 0) /* d 2048, I 512, K 8, E 256, no heads */                                 \
  X(4, 2, 8, 1, 2, 4, 0) /* d 4096, I 1024, K 4, E 512, int4, no heads */                          \
  X(2, 1, 8, 1, 2, 2, 0) /* d 4096, I 1024, K 4, E 512, int2, no heads */

static bool has_variant(int bits, int PG, int NSH, int NSF, int GU, int PD, int NH) {
#define MOE_STEP_HAS(B_, PG_, NSH_, NSF_, GU_, PD_, NH_) \
  if (bits == B_ && PG == PG_ && NSH == NSH_ && NSF == NSF_ && GU == GU_ && PD == PD_ && NH == NH_) return true;
  MOE_STEP_VARIANTS(MOE_STEP_HAS)
#undef MOE_STEP_HAS
  return false;
}

static hipError_t dispatch(hipStream_t s, const StepParams& p, int bits, int PG, int NSH, int NSF) {
#define MOE_STEP_GO(B_, PG_, NSH_, NSF_, GU_, PD_, NH_)                                          \
  if (bits == B_ && PG == PG_ && NSH == NSH_ && NSF == NSF_ && p.GU == GU_ && p.PD == PD_ && p.NH == NH_) \
    return go<B_, PG_, NSH_, NSF_, GU_, PD_, NH_>(s, p);
  MOE_STEP_VARIANTS(MOE_STEP_GO)
#undef MOE_STEP_GO
  return hipErrorInvalidValue;
}

bool decode_step_supported(const moe_decode_stack& st) { return plan_step(st, device_cus()).ok; }

size_t decode_step_workspace(const moe_decode_stack& st) { return step_ws(st).total; }

int decode_step_grid(const moe_decode_stack& st) { return decode_step_grid_for(st, device_cus()); }

int decode_step_grid_for(const moe_decode_stack& st, int cus) {
  const StepPlan pl = plan_step(st, cus);
  return pl.ok ? pl.G : 0;
}

hipError_t launch_decode_step(hipStream_t s, const moe_decode_stack& st, int token, uint32_t flags,
                              const uint16_t* h_in, uint16_t* h_out, uint16_t* h_layers, void* ws, uint64_t* stamps) {
  const int G = device_cus();
  const StepPlan pl = plan_step(st, G);
  if (!pl.ok) return hipErrorInvalidValue;
  const StepWs w = step_ws(st);
  if (w.total >= OFF_NONE || pl.G > SPARE_WGS) return hipErrorInvalidValue;
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
  p.h_layers = h_layers;
  p.ridx = st.route_idx;
  p.rw = st.route_w;
  p.slot = token % 3;
  p.given = (flags & MOE_DECODE_GIVEN_ROUTING) != 0;
  p.gained = st.norm_gains != 0;
  {
    const int rows = (st.E + pl.G - 1) / pl.G;  // router rows of the busiest workgroup (row r: wave r / G)
    p.rstage = rows <= RWG && rows * st.d_model <= LDS_RR;
  }
  p.lshift = st.E <= 256 ? 2 : st.E <= 512 ? 1 : 0;  // up to 1,024 polled words (one pass of 16 per lane)
  p.bootstrap = token == 0 && !p.given;
  p.topk_flags = flags & MOE_TOPK_RENORM;
  p.ll_logits = (uint64_t*)(b + w.logits);
  p.ll_act = (uint64_t*)(b + w.act);
  p.ll_g = (uint64_t*)(b + w.g);
  p.ll_hlog = (uint64_t*)(b + w.hlog);
  p.ll_h = (uint64_t*)(b + w.h);
  p.spare = (const uint64_t*)(b + w.spare);
  p.h_stride = (int)(ll_bytes((size_t)(st.L + 1) * (st.d_model / 2)) / 8);
  p.act_stride = (int)(ll_bytes((size_t)st.K * st.d_ff) / 8);
  p.xr_h = std::min(XR_MAX, WAVE / (pl.DR / 2));
  p.xr_a = std::min(XR_MAX, WAVE / (MW * pl.GU / 2));
  p.epoch = (uint32_t*)(b + w.epoch);
  p.err = (int*)(b + w.err);
  p.zero16 = (const uint16_t*)(b + w.zero);
  p.ws = ws;
  p.ws_bytes = (uint32_t)w.total;
  p.stamps = stamps;
  return dispatch(s, p, st.bits, pl.PG, pl.NSH, pl.NSF);
}

}  // namespace moe
