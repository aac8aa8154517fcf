/*
 * moe.h -- C ABI of the decode-time fine-grained MoE layer with low-bit experts,
 * for AMD Instinct MI355X (gfx950).
 *
 * The layer, per token (pages cited by title and section):
 *   1. router logits l = W_r x, or the prerouter head's logits
 *        ("La otra mitad del muro de la memoria: Servir MoEs de 35B desde SSD con prediccion
 *         de enrutamiento entrenada", section "Arquitectura del cabezal Prerouter");
 *   2. softmax top-K selection of experts
 *        ("Arquitecturas nativas para device: MoE de grano fino y pre-attention router",
 *         section "Dos niveles de sparsity");
 *   3. affine group-quantised 4-bit / 2-bit dequantise-and-matvec for each selected
 *      expert's gate, up and down projections, 4. fused SwiGLU, and 5. weighted expert
 *      combine plus residual
 *        ("Inferencia de LLM MoE en MacBook Pro: Streaming de Expertos desde SSD con Metal",
 *         section "Arquitectura del Sistema" and its Metal dequant listing);
 *   plus the unmerged low-rank adapter on the shared path, y = W_int4 x + (alpha/r) B A x
 *        (Edge0 reading guide, section "Ejecucion del adaptador no fusionado").
 *
 * Conventions for every call
 *   - Array pointers are DEVICE pointers owned by the caller; float16 values travel as their
 *     uint16_t bit patterns.  The library never allocates and keeps no state between calls.
 *   - `stream` is a hipStream_t (NULL = the null stream).  Each call checks its arguments on the
 *     host, then enqueues kernels on `stream` and returns without synchronising.  Calls are
 *     safe to record into a HIP graph (no memset or host round trip inside).
 *   - On an argument error nothing is enqueued and MOE_ERR_INVALID_ARG or MOE_ERR_UNSUPPORTED is
 *     returned.  A launch failure reported by the runtime returns MOE_ERR_HIP.  Faults inside a
 *     kernel surface at the caller's next synchronisation, as for any HIP call.
 *   - Device-side expert indices must lie in [0, E) and a row of them must hold distinct
 *     experts.  A kernel that meets an index outside [0, E) reads no weights for it and writes
 *     NaN where that expert's contribution would go.
 *   - No C++ exception crosses this boundary.
 *
 * Quantised matrix layout (one "stack" = the same projection of all E experts)
 *   q      : uint32 [E][rows][cols*bits/32], little-endian words; column j of a row is held in
 *            word j/(32/bits) at bit offset bits*(j%(32/bits)), lowest bits = lowest column.
 *   scales : float16 [E][rows][cols/group]; biases: float16 [E][rows][cols/group].
 *   weight[e][o][j] = code * scales[e][o][j/group] + biases[e][o][j/group].
 *   gate and up have rows = d_ff, cols = d_model; down has rows = d_model, cols = d_ff
 *   (moe_expert_ffn_sparse alone takes its down projection neuron-major: see there).
 *   q must be 16-byte aligned; rows must be a whole number of 16-byte segments
 *   (cols*bits % 128 == 0).
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = 1, /* null required pointer, bad size, K > E, misalignment ...     */
  MOE_ERR_UNSUPPORTED = 2, /* bits not in {2,4}, group not in {32,64,128}, shape off-grid   */
  MOE_ERR_HIP = 3,         /* the HIP runtime rejected a launch                              */
  MOE_ERR_TOO_LARGE = 4    /* moe_expert_ffn_q4_noalloc: the call needs more than its scratch */
} moe_status;

/* flags */
#define MOE_TOPK_RENORM 0x1u   /* top-K weights = softmax over the K selected logits; without
                                  it, the full softmax over all E logits read at the K experts */
#define MOE_INPUT_RMSNORM 0x2u /* consume x := x / sqrt(mean(x^2) + 1e-6) (weightless RMS norm,
                                  the glue between chained layers), computed in float32       */
#define MOE_DECODE_GIVEN_ROUTING 0x4u /* moe_decode_step only: every layer takes its experts and
                                  weights from route_idx / route_w slot token % 3 as the caller
                                  wrote them; no router or head runs, nothing else is written */

/* Limits checked by every call. */
#define MOE_MAX_E 1024
#define MOE_MAX_K 16
#define MOE_MAX_D 8192
#define MOE_POOL_MAX_SLOTS 4096
#define MOE_POOL_MAX_JOBS 8

typedef struct {
  const uint32_t* q;
  const uint16_t* scales;
  const uint16_t* biases;
} moe_qmat;

typedef struct {
  int32_t n_experts; /* E (1 for a shared expert)   */
  int32_t d_model;   /* d                            */
  int32_t d_ff;      /* expert intermediate size I   */
  int32_t bits;      /* 4 or 2                       */
  int32_t group;     /* 32, 64 or 128                */
  moe_qmat gate, up, down;
} moe_experts;

/* Unmerged low-rank adapter of one projection: delta = (alpha/rank) * B (A v).
   A: float16 [rank][in], B: float16 [out][rank]; rank in 1..64. */
typedef struct {
  const uint16_t* A;
  const uint16_t* B;
  int32_t rank;
  float alpha;
} moe_lora;

/* Prerouter head weights in split layout.  The head reads z = [x; khot(idx_cur); khot(idx_prev)]
   of length d + 2E; fc1 = [fc1_x | fc1_r^T] and l = [lin_x | lin_r^T] (row j of fc1_r / lin_r is
   column d + j of the dense matrix), so the K-hot columns are gathered as K rows.
   logits = fc2 * gelu_erf(fc1 z + fc1_b) + fc2_b + l z + lin_b.  Biases may be NULL. */
typedef struct {
  int32_t d_hidden;       /* H */
  const uint16_t* fc1_x;  /* [H][d]   */
  const uint16_t* fc1_r;  /* [2E][H]  */
  const uint16_t* fc1_b;  /* [H] or NULL */
  const uint16_t* fc2;    /* [E][H]   */
  const uint16_t* fc2_b;  /* [E] or NULL */
  const uint16_t* lin_x;  /* [E][d]   */
  const uint16_t* lin_r;  /* [2E][E]  */
  const uint16_t* lin_b;  /* [E] or NULL */
} moe_prerouter_w;

/* S1a + S2: router and softmax top-K.
   If w_router != NULL: logits[T][E] (float32, out) = W_r[E][d] x[T][d] (x optionally RMS-normed),
   then top-K.  If w_router == NULL: `logits` is the input and x is ignored.
   idx[T][K] (int32, out): experts by descending logit, equal logits -> lower index first.
   w[T][K] (float32, out): softmax weights (MOE_TOPK_RENORM: over the K selected).
   Limits: 1 <= T, 1 <= K <= min(E, 16), 1 <= E <= 1024, d % 8 == 0, d <= 8192. */
moe_status moe_route_topk(void* stream, int32_t T, int32_t d, int32_t E, int32_t K, uint32_t flags,
                          const uint16_t* x, const uint16_t* w_router, float* logits, int32_t* idx,
                          float* w);

/* Bytes of device workspace moe_prerouter needs for T tokens (float32 [T][H] + [T][E]). */
size_t moe_prerouter_workspace_size(int32_t T, int32_t E, int32_t d_hidden);

/* S1b: prerouter head of layer N; its logits route layer N+1 at the next token (feed them to
   moe_route_topk with w_router == NULL).  idx_cur[T][K]: this layer's routing at this token;
   idx_prev[T][K] or NULL: this layer's routing at the previous token (NULL = zero vector).
   logits[T][E] float32 out.  Limits as moe_route_topk, plus 1 <= H <= 8192, H % 8 == 0. */
moe_status moe_prerouter(void* stream, int32_t T, int32_t d, int32_t E, int32_t K, uint32_t flags,
                         const uint16_t* x, const int32_t* idx_cur, const int32_t* idx_prev,
                         const moe_prerouter_w* pw, float* logits, void* workspace,
                         size_t workspace_bytes);

/* Bytes of device workspace moe_expert_ffn_q4 needs for T tokens with K experts each. */
size_t moe_expert_ffn_workspace_size(int32_t T, int32_t K, const moe_experts* ex);

/* S3-S6: for each token t and slot k, expert e = idx[t][k]:
     a = silu(gate_e x_t) * (up_e x_t),  o_tk = down_e a   (float32 accumulation)
   With lora3 (only when ex->n_experts == 1): lora3[0], [1], [2] add their deltas to the gate,
   up and down projections.
   Outputs: out[T][K][d] float32 = unweighted o_tk (may be NULL), and/or the fused combine
     y[T][d] float16 = r[t] + sum_k w[t][k] o_tk  (w_fuse, r_fuse, y_fuse all set, or all NULL).
   Small T runs the batch-1 decode kernels; large T sorts the (token, slot) pairs by expert
   and runs an MFMA grouped GEMM.  workspace: moe_expert_ffn_workspace_size bytes, 256-byte
   aligned.  Limits: d, d_ff <= 8192; d, d_ff multiples of group; rows whole 16-byte segments. */
moe_status moe_expert_ffn_q4(void* stream, int32_t T, int32_t K, uint32_t flags, const uint16_t* x,
                             const int32_t* idx, const moe_experts* ex, const moe_lora* lora3,
                             float* out, const float* w_fuse, const uint16_t* r_fuse,
                             uint16_t* y_fuse, void* workspace, size_t workspace_bytes);

/* moe_expert_ffn_q4 without the workspace argument, for callers that cannot allocate device memory:
   code under HIP graph capture, tight serving loops, harnesses that forbid allocation.  Arguments,
   results and errors as moe_expert_ffn_q4.  The scratch it needs (moe_expert_ffn_workspace_size
   bytes) is a device array inside the library, MOE_NOALLOC_SCRATCH_BYTES per GPU, allocated once
   with the library's code on each GPU it runs on and held until the process ends; the call
   allocates nothing.  A call that needs more returns MOE_ERR_TOO_LARGE with nothing enqueued
   (e.g. T >= 32 large batches: use moe_expert_ffn_q4 with a workspace).  Every call on one GPU
   uses the same array: calls that may overlap on one GPU (other streams, other threads) race and
   must be ordered by the caller.  MOE_ERR_HIP if the array's device address cannot be found. */
#define MOE_NOALLOC_SCRATCH_BYTES (16u << 20)
moe_status moe_expert_ffn_q4_noalloc(void* stream, int32_t T, int32_t K, uint32_t flags, const uint16_t* x,
                                     const int32_t* idx, const moe_experts* ex, const moe_lora* lora3, float* out,
                                     const float* w_fuse, const uint16_t* r_fuse, uint16_t* y_fuse);

/* Bytes of device workspace moe_expert_ffn_q4_shared needs (0 when T < 32). */
size_t moe_expert_ffn_shared_workspace_size(int32_t T, int32_t K, const moe_experts* ex);

/* S3-S7 of a batched layer with a shared expert ("La otra mitad del muro de la memoria ...",
   section "Ejecución del adaptador no fusionado": an always-on shared path whose LoRA runs
   unmerged, W v + (alpha / r) B (A v)) in one call:
     y[t] = r[t] + sum_k w[t][k] FFN_{idx[t][k]}(x_t) + FFN_shared(x_t)        (float16 out)
   FFN as in moe_expert_ffn_q4; the LoRA (lora3, may be NULL) is the shared expert's.  The shared
   expert's T (token) rows join the routed (token, slot) pairs as one more expert of the sort, so
   the grouped GEMM launches cover both; the result equals moe_expert_ffn_q4 on the
   routed experts, moe_expert_ffn_q4 on the shared expert (K = 1, lora3) and moe_combine with its
   output as `shared`, to the bit.  shared: one expert (n_experts == 1) of the same d_model, d_ff,
   bits and group as ex.  w [T][K] float32, r [T][d] float16 and y all required.  T >= 32 (the
   batched path; MOE_ERR_UNSUPPORTED below it: use the two calls and moe_combine).  workspace:
   moe_expert_ffn_shared_workspace_size bytes, 256-byte aligned.  Other limits and errors as
   moe_expert_ffn_q4. */
moe_status moe_expert_ffn_q4_shared(void* stream, int32_t T, int32_t K, uint32_t flags, const uint16_t* x,
                                    const int32_t* idx, const moe_experts* ex, const moe_experts* shared,
                                    const moe_lora* lora3, const float* w, const uint16_t* r, uint16_t* y,
                                    void* workspace, size_t workspace_bytes);

/* Bytes of device workspace moe_expert_ffn_sparse needs for T tokens with K experts each. */
size_t moe_expert_ffn_sparse_workspace_size(int32_t T, int32_t K, const moe_experts* ex);

/* ReLU activation-sparse variant of S3-S6 ("Arquitecturas nativas para device: MoE de grano fino
   y pre-attention router", section "Dos niveles de sparsity", level 2: under a ReLU-type
   activation many intermediate neurons are exactly zero for a token, and the weights of a zero
   neuron are neither read nor multiplied).  For each token t and slot k, expert e = idx[t][k]:
     a = relu(gate_e x_t) * (up_e x_t)          (ReLU on the gate branch of the gated unit)
     o_tk = sum over the neurons i with a_i != 0 of a_i * down_e[i]
   ex->down is stored NEURON-MAJOR: row i holds the d_model weights neuron i feeds, groups of
   ex->group run along d_model, so a zero neuron's row is skipped whole: q [E][d_ff][d_model*bits/32]
   words; scales and biases float16 GROUP-MAJOR, [E][d_model/group][d_ff] (entry [e][g][i] belongs
   to neuron i, columns g*group .. g*group+group-1).  gate and up are as in moe_expert_ffn_q4.  Float32 accumulation; the fused combine is moe_combine's arithmetic.
   Outputs: out[T][K][d] float32 (may be NULL) and/or the fused y (w_fuse, r_fuse, y_fuse all set
   or all NULL), as moe_expert_ffn_q4; n_active[T][K] int32 (may be NULL) = the number of neurons
   with a != 0, i.e. the down rows read (-1 where idx lies outside [0, E)).  flags:
   MOE_INPUT_RMSNORM only.  No LoRA.  workspace: moe_expert_ffn_sparse_workspace_size bytes,
   256-byte aligned.  Limits: those of moe_expert_ffn_q4, and d_model a multiple of 64 (int4) or
   128 (int2), d_ff at most 4096 (MOE_ERR_UNSUPPORTED otherwise).  Every T runs the per-token
   kernels (the weights are read once per token). */
moe_status moe_expert_ffn_sparse(void* stream, int32_t T, int32_t K, uint32_t flags, const uint16_t* x,
                                 const int32_t* idx, const moe_experts* ex, float* out, const float* w_fuse,
                                 const uint16_t* r_fuse, uint16_t* y_fuse, int32_t* n_active, void* workspace,
                                 size_t workspace_bytes);

/* ---------------------------------------------------------------------------------------------
   Expert streaming from a slower memory tier into an HBM pool ("Arquitecturas nativas para device:
   MoE de grano fino y pre-attention router", section "Las matemáticas que importan": only the
   active experts and a cache of recent ones are resident, the rest is fetched when needed; "La otra
   mitad del muro de la memoria ...", section "Ideas clave": experts stream into a compact pool and
   the one-token-ahead prediction is the routing).

   A pool is n_slots experts in HBM, described by an moe_experts with n_experts = n_slots and the
   same d_model, d_ff, bits, group and layouts as the source.  Its state is device memory the caller
   owns: slot_expert[n_slots] (int32, the expert a slot holds, -1 = empty), slot_stamp[n_slots]
   (int32, the call that last used it, -1 = never) and clock[1] (int32, the number of calls so far,
   which is the stamp of the next call); fill slot_expert and slot_stamp with -1 and clock with 0
   before the first call.  One call per token makes a stamp a token number. */
typedef struct {
  int32_t n_slots;
  int32_t* slot_expert;
  int32_t* slot_stamp;
  int32_t* clock;
} moe_pool;

/* Bytes of device workspace moe_stream_in needs for K selected experts. */
size_t moe_stream_workspace_size(int32_t K);

/* Place a token's K selected experts idx[K] (int32, device) in the pool and copy the missing ones
   from src (E experts whose arrays may be pinned host memory the GPU can read, or device memory).
   Placement: an expert already in a slot is a hit and keeps its slot; then, in k order, each
   missing expert takes the least recently used slot among those this call has not claimed (empty
   slots first, then the oldest stamp, ties to the lowest slot); every slot used gets the call's
   stamp, *clock, and *clock then advances by one.  The stamp lives on the device, so a captured
   HIP graph replays correctly.  Writes idx_slot[K] (int32, device): the slot of each selected expert, for
   moe_expert_ffn_q4 / moe_expert_ffn_sparse on the pool (an index outside [0, E) gets -1, which
   those calls turn into NaN).  counters[2] (int32, device, may be NULL): the call's hits and copies
   (misses) are added; an index outside [0, E) is neither.
   Calls on one pool must not overlap.  With one call per token and n_slots >= 2K, a slot used by
   token t is not reused before token t+2, so the copy for token t+1 may run beside token t's
   expert FFN.
   Limits: 1 <= K <= 16, K <= n_slots <= MOE_POOL_MAX_SLOTS; src and pool of equal shape. */
moe_status moe_stream_in(void* stream, int32_t K, const int32_t* idx, const moe_experts* src,
                         const moe_experts* pool_experts, const moe_pool* pool, int32_t* idx_slot,
                         int32_t* counters, void* workspace, size_t workspace_bytes);

/* Several moe_stream_in calls in two launches: up to MOE_POOL_MAX_JOBS pools (one layer's each, say)
   of one shape (equal d_model, d_ff, bits, group), placed one wave per pool and copied by one grid.
   Each job is checked as moe_stream_in checks its arguments; the pools of one call must be distinct.
   workspace: n * moe_stream_workspace_size(K) bytes, 256-byte aligned.  Results equal n separate
   moe_stream_in calls. */
typedef struct {
  const int32_t* idx;               /* [K] selected experts (device) */
  const moe_experts* src;           /* E experts: pinned host or device memory */
  const moe_experts* pool_experts;  /* the pool's n_slots experts (HBM) */
  const moe_pool* pool;             /* the pool's state */
  int32_t* idx_slot;                /* [K] out: slot of each selected expert */
  int32_t* counters;                /* [2] hits, copies (added) or NULL */
} moe_stream_job;
moe_status moe_stream_in_many(void* stream, int32_t n, int32_t K, const moe_stream_job* jobs, void* workspace,
                              size_t workspace_bytes);

/* Measurement aid, not a step of the method: a plain streaming read of `bytes` bytes of device
   memory at buf (16-byte aligned, bytes a multiple of 16) with 16-byte loads, the measured read
   ceiling of HBM the layer kernels are compared with.  out[MOE_READ_PROBE_BLOCKS] (uint32, device)
   receives one fold of the data per block, so that no load can be dropped.  The caller owns both
   buffers.  MOE_ERR_INVALID_ARG (nothing enqueued) for a null pointer, bytes below 16 or not a
   multiple of 16, or buf not 16-byte aligned; MOE_ERR_HIP if the launch fails. */
#define MOE_READ_PROBE_BLOCKS 4096
moe_status moe_read_probe(void* stream, const void* buf, size_t bytes, uint32_t* out);

/* Measurement aid, not a step of the method: the latency of handing tagged 8-byte words between
   resident workgroups, the unit of every grid-wide exchange inside moe_decode_step.  n_wg
   workgroups of one wave each, one per compute unit, run `iters` phases of `pattern`:
     MOE_XCHG_ALL  : in every phase each member of a group stores words/group_size words of a
                     vector and then polls all `words` of it until each carries the phase's tag;
     MOE_XCHG_RING : one word is passed member to member, `iters` laps of the group.
   Groups: group_size consecutive workgroup numbers (xcd_local 0), or the workgroups b with equal
   b % (n_wg / group_size) (xcd_local 1; the dispatcher deals workgroups round robin over the 8
   XCDs, so each such group runs on one XCD when n_wg / group_size is a multiple of 8).
   load_scope / store_scope: MOE_XCHG_SCOPE_DEVICE (device-coherent: what crossing XCDs needs) or
   MOE_XCHG_SCOPE_XCD (loads bypass only the L1 and stores end in the XCD's L2: enough inside one
   XCD).  Every wait is bounded (0.1 s); one that runs out adds 1 to out[0] and the grid finishes.
   out (uint32, device, 1 + 3 n_wg words): out[0] += waits that ran out (zero it first); for
   workgroup b, out[1+3b] / out[2+3b] = low / high word of the real-time-counter ticks (100 MHz)
   from the common start to its end, out[3+3b] = the XCD it ran on.  workspace:
   moe_exchange_probe_workspace_size bytes, 256-byte aligned, zeroed once before the first call;
   `epoch` must differ between consecutive calls on one workspace (it tags the words).
   Limits: 1 <= n_wg <= compute units; group_size divides n_wg; ALL: words a multiple of
   group_size, words / group_size <= 64, words <= 16384; 1 <= iters <= 32767 (ALL) or
   iters * group_size <= 65535 (RING).  MOE_ERR_INVALID_ARG otherwise (nothing enqueued). */
#define MOE_XCHG_ALL 0
#define MOE_XCHG_RING 1
#define MOE_XCHG_SCOPE_DEVICE 0
#define MOE_XCHG_SCOPE_XCD 1
typedef struct {
  int32_t pattern, n_wg, group_size, xcd_local, words, iters, load_scope, store_scope;
  uint32_t epoch;
  int32_t replicas; /* ALL: each word is stored in `replicas` copies (1..8) and workgroup b reads copy
                       b % replicas (with 8, the copy of its XCD), which spreads the readers' traffic */
  int32_t wide_loads; /* ALL: 0 = 8-byte buffer loads, 1 = 16-byte buffer loads (two words per lane per
                         load), 2 = 8-byte agent-scope atomic loads through the global path (words <= 1024) */
} moe_xchg_cfg;
size_t moe_exchange_probe_workspace_size(const moe_xchg_cfg* cfg);
moe_status moe_exchange_probe(void* stream, const moe_xchg_cfg* cfg, void* workspace, size_t workspace_bytes,
                              uint32_t* out);

/* Grouping used by the batched path (tokens sorted by expert): a stable counting sort of the T*K
   (token, slot) pairs.  counts[E+1] and offsets[E+2] (int32, out): bucket E collects pairs whose
   index lies outside [0, E); perm[T*K] (int32, out) lists flat pair indices t*K + k grouped by
   expert, ascending inside each expert; offsets[e] is the first position of expert e.
   Limits: 1 <= T*K <= 2^24, 1 <= E <= 1024. */
moe_status moe_sort_by_expert(void* stream, int32_t T, int32_t K, int32_t E, const int32_t* idx,
                              int32_t* counts, int32_t* offsets, int32_t* perm);

/* RMS normalisation of a layer input with an optional gain ("Inferencia de LLM MoE en MacBook Pro
   ...", section "Arquitectura del Sistema", lists RMS normalisation among the GPU kernels; the
   prerouter head reads the normalised state, "La otra mitad del muro ...", section "Arquitectura
   del cabezal Prerouter"):  x[t][i] = float16(g[i] * h[t][i] / sqrt(mean_i(h[t][i]^2) + 1e-6)),
   the sum of squares and the product in float32, rounded to nearest even.  h, x: [T][d] float16
   (device, 16-byte aligned; x may be h); gain: [d] float16 (16-byte aligned) or NULL for g = 1.
   The result feeds the routing and expert calls without MOE_INPUT_RMSNORM (the residual is h).
   Limits: T >= 1, d a multiple of 8, d <= MOE_MAX_D. */
moe_status moe_rmsnorm(void* stream, int32_t T, int32_t d, const uint16_t* h, const uint16_t* gain, uint16_t* x);

/* S6: y[T][d] float16 = r + sum_k w[t][k] o[t][k] (+ shared[t], weight 1), accumulated in
   float32 in ascending k, rounded to nearest even. */
moe_status moe_combine(void* stream, int32_t T, int32_t K, int32_t d, const float* o, const float* w,
                       const uint16_t* r, const float* shared, uint16_t* y);

/* ---------------------------------------------------------------------------------------------
   Whole-token decode of a resident prerouted stack in one persistent kernel.

   One call runs token `token` through all L layers with the per-layer semantics of the calls
   above (MOE_INPUT_RMSNORM on every layer input, the residual is the un-normalised input):
     - layer 0, every layer whose predecessor has no head, and every layer at token 0 run their
       own router + top-K;
     - any other layer uses the experts and weights the head of the layer before it predicted
       at the previous token (the prediction is the routing: Edge0 reading guide, section
       "Ideas clave"); the head of layer l reads its layer input with the K-hot routing of layer
       l at this token and at the previous one (none at token 0) and writes layer l+1's routing
       for the next token ("Arquitectura del cabezal Prerouter").
   Routing state lives in route_idx / route_w [3][L][K], slot token % 3 (this token), slot
   (token + 2) % 3 (previous token), slot (token + 1) % 3 (written: next token).  Tokens must be
   issued in order 0, 1, 2, ...; a graph captured for token t replays correctly for any t' >= 1
   with t' % 3 == t % 3.

   One workgroup per compute unit stays resident for the whole token; workgroups hand vectors to
   each other through tagged words in the workspace.  Precondition: the launch has the device's
   compute units to itself (every workgroup must be resident at once).  A kernel running at the
   same time on another stream that holds compute units can keep workgroups from starting; the
   resident ones then wait, each wait is bounded (0.2 s of polling), and the call ends with the
   error word set and its outputs invalid (no hang).  The workspace must be zeroed once before
   the first call and then passed unchanged to every later call of the same stack; calls on one
   workspace must not overlap.  Its first 4 bytes hold a token counter, the next 4 an error
   word: nonzero means a wait inside the kernel exceeded its bound and that call's outputs are
   invalid (check it after synchronising when in doubt).
   Supported shapes: d_model 2048 or 4096 with d_model*bits/128 a multiple of 64 (at most 128),
   d_ff*bits/128 <= 64, K <= 8, K*d_ff <= 4096, L*K <= 512, E <= 4 * compute units, head width H a multiple
   of 512 up to 2048 (or no heads), 2-bit only with group >= 64; others return
   MOE_ERR_UNSUPPORTED (use the per-layer calls).  Device-side descriptors must match `st`. */
typedef struct {
  moe_experts experts;   /* this layer's routed experts (E, d_model, d_ff, bits, group as in the stack) */
  const uint16_t* router; /* [E][d]: needed by self-routed layers (layer 0, token 0, no predecessor head) */
  moe_prerouter_w head;  /* head predicting layer l+1 (d_hidden == stack d_hidden); fc1_x == NULL: none */
  const uint16_t* norm_gain; /* [d] float16 gain of this layer's input normalisation (x = g * h /
                                rms(h)), applied inside the kernel; read only when the stack's
                                norm_gains is 1 (then 16-byte aligned in every layer) */
} moe_decode_layer;

typedef struct {
  int32_t L, E, K, d_model, d_ff, bits, group, d_hidden; /* d_hidden 0 when no layer has a head */
  const moe_decode_layer* layers; /* DEVICE array of L descriptors */
  int32_t* route_idx;             /* DEVICE [3][L][K] */
  float* route_w;                 /* DEVICE [3][L][K] */
  int32_t norm_gains;             /* 1: every layer descriptor's norm_gain is set; 0: none is */
} moe_decode_stack;

size_t moe_decode_workspace_size(const moe_decode_stack* st);

/* h_in[d] float16 (device): the token's input hidden state; h_out[d] float16 (device): the output
   of layer L-1.  h_layers: NULL, or [L+1][d] float16 (device) receiving every layer's input (row l,
   row 0 = h_in) and the final output (row L), for inspection and layer-by-layer checking; 4-byte
   aligned.  flags: MOE_TOPK_RENORM (applies to every top-K) and/or MOE_DECODE_GIVEN_ROUTING (the
   expert FFN steps alone on routing the caller supplies for every layer; token 0 is then no
   bootstrap, the heads and routers of the descriptors are not read, and route_idx values must lie
   in [0, E), K distinct per layer). */
moe_status moe_decode_step(void* stream, const moe_decode_stack* st, int32_t token, uint32_t flags,
                           const uint16_t* h_in, uint16_t* h_out, uint16_t* h_layers, void* workspace,
                           size_t workspace_bytes);

/* Workgroups one moe_decode_step launch of this stack runs on the current device (one per compute
   unit that holds a slice of the rows), or 0 if the stack is not supported by it. */
int32_t moe_decode_step_grid(const moe_decode_stack* st);

/* The same for a device with `compute_units` compute units: the workgroups a launch there would
   use, or 0 if that device could not run the stack (moe_decode_step returns MOE_ERR_UNSUPPORTED
   there).  Host-only: reads only the shape fields of `st` (not its device arrays) and touches no
   device.  compute_units < 1 or a NULL or malformed stack gives 0. */
int32_t moe_decode_step_grid_for(const moe_decode_stack* st, int32_t compute_units);

/* Measurement aid, not a step of the method: moe_decode_step that also writes phase stamps of the
   device's 100 MHz real-time counter (one clock for every compute unit, so stamps of different
   workgroups compare).  stamps: uint64 [G][L][16] (device, 8-byte aligned, stamp_bytes >=
   G * L * 128, G = moe_decode_step_grid(st)); slot s of (workgroup g, layer l):
     0 the layer starts in g's polling wave, 1 g has unpacked the layer's input h_l,
     2 g has unpacked all SwiGLU outputs of the layer, 3 g's first compute wave sees h_l,
     4 g's SwiGLU outputs are stored, 5 g's down phase starts, 6 g's rows of the layer's output
     are stored, 7 g's first compute wave has finished its head rows of the layer; finer marks of
     the first compute wave: 8 gate/up dot products done, 9 its SwiGLU output ready, 12 the combine
     starts, 13 down dot products done, 14 down partials stored; on a layer that routes itself:
     10 the first compute wave's router logit stored, 11 that wave knows the routing, 15 the polling
     wave has all the router logits (slots 10, 11, 15 are left as they were on other layers).
   Results and every other argument as moe_decode_step.  This call runs a variant of the kernel with
   the stamp stores compiled in (a little slower); moe_decode_step runs the variant without them. */
moe_status moe_decode_step_stamped(void* stream, const moe_decode_stack* st, int32_t token, uint32_t flags,
                                   const uint16_t* h_in, uint16_t* h_out, uint16_t* h_layers, uint64_t* stamps,
                                   size_t stamp_bytes, void* workspace, size_t workspace_bytes);

const char* moe_status_string(moe_status s);

/* Library version (major*10000 + minor*100 + patch). */
int32_t moe_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */
