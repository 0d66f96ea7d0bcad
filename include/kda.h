/*
 * kda.h -- C ABI of the MI355X (gfx950) Kimi Delta Attention (KDA) library.
 *
 * The library evaluates the KDA gated delta rule, per head, on a 128 x 128
 * FP32 state S (row = key channel, column = value channel):
 *
 *   S_t = (I - beta_t k_t k_t^T) Diag(exp(g_t)) S_{t-1} + beta_t k_t v_t^T
 *   o_t = scale * S_t^T q_t
 *
 * through these calls:
 *
 *   kda_prefill  -- chunked prefill over packed variable-length sequences
 *                   ("FlashInfer PR #4262: CAKE KDA Prefill Highlights",
 *                   sections 1-3: 32-token chunks, fixed exponent anchor,
 *                   the fused per-chunk pipeline; and flashinfer PR #4571,
 *                   "optimize small-BH recurrent-KDA prefill": packed
 *                   layout with sequence offsets, caller-owned outputs,
 *                   caller's stream).
 *   kda_prefill_prepare, kda_prefill_chain
 *                -- the two passes of kda_prefill's SPLIT route as separate
 *                   calls (the note's section 5: chunk preparation is
 *                   parallel, state evolution is serial), so that a caller
 *                   can time them or overlap one batch's preparation with
 *                   another's chain.
 *   kda_prefill_pool
 *                -- kda_prefill with states in a slot-indexed FP32 pool and
 *                   optional intermediate-state checkpoints.
 *   kda_decode   -- the T=1 step over a slot-indexed state pool, updated in
 *                   place (flashinfer PR #5551, "Kimi K3 TP12 H=8 fused KDA
 *                   decode": positive unique slots, FP32 and BF16 state,
 *                   64-bit slot offsets).
 *   kda_decode_ex -- the same with the input front-end (raw gates, beta
 *                   logits, q/k L2 norm); kda_prefill_ex and
 *                   kda_prefill_pool_ex likewise for prefill.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - All tensor pointers are DEVICE pointers on the current HIP device, owned
 *   by the caller; the library allocates nothing per call and keeps no
 *   pointer after returning.
 * - bf16 means IEEE bfloat16 stored as uint16; fp32 is IEEE binary32.
 * - Work is enqueued on `stream` (NULL = the legacy default stream) and runs
 *   asynchronously.  No call synchronises the device or reads device memory
 *   on the host, so calls may be captured into a hipGraph.
 * - Return value: KDA_OK (0), or a negative kda_status.  Arguments are
 *   validated on the host before anything is enqueued; on error nothing is
 *   enqueued and kda_last_error() describes the problem.  Faults inside a
 *   kernel surface, as usual in HIP, at the caller's next synchronisation.
 * - Device-side preconditions that are NOT checked (they would need a
 *   device read): cu_seqlens non-decreasing with cu_seqlens[0] = 0 and
 *   cu_seqlens[N] = total_tokens; lower_bound <= g <= 0 for prefill (any
 *   g <= 0 with lower_bound = -INFINITY);
 *   beta in [0, 1]; decode slot indices unique among the non-negative ones.
 *   Kernels clamp every index they read so that a violated precondition
 *   gives wrong numbers, never an out-of-bounds access.
 */
#ifndef KDA_H_
#define KDA_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KDA_ABI_VERSION 9
#define KDA_HEAD_DIM 128

typedef enum {
  KDA_OK = 0,
  KDA_ERR_INVALID_ARGUMENT = -1, /* null pointer, bad size, misalignment   */
  KDA_ERR_UNSUPPORTED = -2,      /* valid but not implemented (e.g. dk!=128) */
  KDA_ERR_WORKSPACE = -3,        /* workspace missing or too small          */
  KDA_ERR_HIP = -4               /* a HIP runtime call failed               */
} kda_status;

typedef enum { KDA_STATE_F32 = 0, KDA_STATE_BF16 = 1 } kda_state_dtype;

/* Input front-end: how the gate and beta arrive, and whether q and k are
 * L2-normalised by the library.  "flashinfer PR #5551: Kimi K3 TP12 H=8 fused
 * KDA decode" gives the decode kernels a lower-bound switch, the bound and
 * norm_eps, and tests softplus and lower-bound gates; the PR #5565/#5573
 * notes feed beta as a sigmoid of logits and run the unbounded softplus gate
 * of Kimi-Linear.  The formulas (the pages print none) are read as:
 *   KDA_GATE_LOG          the g tensor is the natural-log decay itself;
 *   KDA_GATE_LOWER_BOUND  the g tensor holds a, decay = lower_bound * sigmoid(a);
 *   KDA_GATE_SOFTPLUS     the g tensor holds a, decay = -softplus(a)
 *                         = -log(1 + e^a) (no lower bound);
 *   beta_logits != 0      beta is used as sigmoid(beta);
 *   normalize_qk != 0     q and k of each (token, head) are scaled by
 *                         1 / sqrt(sum_c x_c^2 + norm_eps) (FP32, before use).
 * A NULL kda_frontend pointer means {KDA_GATE_LOG, 0, 0, 0, 0}. */
typedef enum { KDA_GATE_LOG = 0, KDA_GATE_LOWER_BOUND = 1, KDA_GATE_SOFTPLUS = 2 } kda_gate_mode;
typedef struct {
  int32_t gate_mode;    /* kda_gate_mode                                        */
  float lower_bound;    /* KDA_GATE_LOWER_BOUND: the bound (< 0, natural log)   */
  int32_t beta_logits;
  int32_t normalize_qk;
  float norm_eps;       /* >= 0, finite                                          */
} kda_frontend;

/* Prefill kernels ("routes").  AUTO lets kda_prefill_plan choose. */
typedef enum {
  KDA_ROUTE_AUTO = -1,
  KDA_ROUTE_SERIAL = 0, /* token-serial FP32 recurrence, no MFMA            */
  KDA_ROUTE_CHUNK = 1,  /* 32-token chunks on bf16/fp16 MFMA, each block
                           prepares and consumes its own chunks (many
                           (sequence, head) units)                         */
  KDA_ROUTE_SPLIT = 2,  /* same chunk math in two passes: all chunks are
                           prepared in parallel into the workspace, then a
                           short serial chain per (sequence, head) consumes
                           them (few units: AUTO picks it up to a quarter of
                           the device's compute units in (sequence, head)
                           units, 64 on MI355X, and only for batches of
                           more than 96 tokens)                            */
  KDA_ROUTE_STREAM = 3  /* token recurrence as a decode-style state stream:
                           one block per (sequence, head, value slice) keeps
                           the state in registers across the sequence's
                           tokens, one read and one write of it, a block
                           reduction per token (AUTO: many short sequences,
                           e.g. multi-token decode of a few new tokens per
                           row against a state pool, flashinfer PR #5551
                           "Kimi K3 TP12 H=8 fused KDA decode", its T > 1
                           path)                                           */
} kda_prefill_route;

/* Exponent handling of the chunk route's pairwise (Mqk, Akk) products,
 * "FlashInfer PR #4262: CAKE KDA Prefill Highlights", section 1. */
typedef enum {
  KDA_ANCHOR_FIXED = 0,  /* one anchor C = 16 * lower_bound * log2(e) per chunk:
                            operand exponents reach 16|lb|log2e, kept <= 116
                            (above it the operands' bf16 low halves lose
                            their precision before the bf16 range ends at
                            126), i.e. used for lower_bound >= -5.02       */
  KDA_ANCHOR_SPLIT16 = 1, /* per 16-token half anchors (the note's ordinary
                            16-token blocks) for bounds down to -10.05: the
                            factors reach about 2^{8 |lb| log2 e} <= 2^116 */
  KDA_ANCHOR_DATA = 2    /* no bound (lower_bound = -inf, or the softplus
                            gate), or a bound below -10.05: each 16-token
                            half of each chunk is anchored, per channel, at
                            the midpoint of its own gate-prefix range (a
                            data-dependent range strategy).  Where a half's
                            prefix falls by more than 2^232 (about 160.8
                            nats) in some channel, its products are formed
                            per 8-token quarter instead (each quarter at its
                            own midpoint, the cross-quarter block through
                            their boundary).  Exact to the usual rounding
                            while no quarter of a chunk falls by more than
                            2^232 (the gate summed over the quarter's last
                            seven tokens >= -160.8 in every channel);
                            kda_check_prefill_inputs flags inputs beyond
                            that (KDA_CHECK_GATE_STEEP)                    */
} kda_anchor_mode;

/* What kda_prefill will launch for a problem (a pure host function of the
 * sizes, the bound and the device's compute-unit count).  With the input
 * front-end (the _ex entry points) the CHUNK route always runs two 64-column
 * slices per (sequence, head), whatever dv_split says. */
typedef struct {
  int32_t route;       /* kda_prefill_route actually used                  */
  int32_t anchor_mode; /* kda_anchor_mode (chunk route only)               */
  int32_t dv_split;    /* value-column slices per (sequence, head)         */
  int32_t block_threads;
  int64_t grid_blocks;
  float anchor_log2;   /* C = 16 * lower_bound * log2(e), as used on device */
  int32_t windows;     /* SPLIT route: windows each sequence's chain is cut
                          into at most (1 = none); see below               */
  int32_t window_chunks; /* chunks per window of a sequence as long as the
                            batch (0 when windows == 1)                    */
} kda_prefill_plan_t;

/* ------------------------------------------------------------- prefill --
 * Packed varlen prefill.
 *
 *  q, k, g     bf16 [total_tokens, num_heads, 128], row-major, 16-byte aligned.
 *              g is the per-channel natural-log decay, lower_bound <= g <= 0.
 *              q and k are used as given (normalise them beforehand).
 *  v           bf16 [total_tokens, num_heads, 128], 16-byte aligned.
 *  beta        bf16 [total_tokens, num_heads], post-sigmoid write strength.
 *  cu_seqlens  int32 [num_seqs + 1] sequence offsets into the token axis.
 *  num_seqs    N >= 0 (0 = nothing to do).
 *  total_tokens  T_tot = cu_seqlens[N] (host copy, used for validation and
 *              to clamp device reads), 0 <= T_tot < 2^31.
 *  num_heads   H >= 1.
 *  head_dim_k, head_dim_v   must both be 128 (else KDA_ERR_UNSUPPORTED).
 *  scale       output scale (finite), e.g. 1/sqrt(128).
 *  lower_bound < 0: the bound g >= lower_bound that fixes the anchor, or
 *              -INFINITY for an unbounded gate (KDA_ANCHOR_DATA).
 *  initial_state  fp32 [N, H, 128, 128] (dv contiguous) or NULL for zeros.
 *  final_state    fp32 [N, H, 128, 128] or NULL (not stored).  May equal
 *              initial_state (each sequence-head reads its slice before it
 *              writes it); must not partially overlap it.
 *  out         bf16 [total_tokens, num_heads, 128]; must not alias inputs.
 *  workspace, workspace_bytes   device scratch of at least
 *              kda_prefill_workspace_size(...) bytes, owned by the caller,
 *              16-byte aligned; its contents on entry do not matter and it
 *              may be reused by the next call once this one has completed on
 *              `stream`.  NULL / 0 is fine when the size is 0.
 *  stream      HIP stream the kernels are enqueued on.
 * Sequences of length 0 copy initial_state to final_state. */
int kda_prefill(const void* q, const void* k, const void* v, const void* g,
                const void* beta, const int32_t* cu_seqlens, int32_t num_seqs,
                int64_t total_tokens, int32_t num_heads, int32_t head_dim_k,
                int32_t head_dim_v, float scale, float lower_bound,
                const float* initial_state, float* final_state, void* out,
                void* workspace, size_t workspace_bytes, hipStream_t stream);

/* kda_prefill with the input front-end `frontend` (kda_frontend; NULL =
 * kda_prefill).  The gate mode decides the bound the chunk routes rely on:
 * KDA_GATE_LOG uses `lower_bound` as kda_prefill does; KDA_GATE_LOWER_BOUND
 * uses frontend->lower_bound (g lies in (lower_bound, 0)) and ignores the
 * argument; KDA_GATE_SOFTPLUS is unbounded (KDA_ANCHOR_DATA) and ignores it.
 * The transforms run inside the prefill kernels on the bf16 inputs, in FP32
 * (the gate before its prefix sum; q, k scaled per token before any
 * product); nothing is written back.  A zero q or k vector with norm_eps = 0
 * stays zero. */
int kda_prefill_ex(const void* q, const void* k, const void* v, const void* g,
                   const void* beta, const int32_t* cu_seqlens, int32_t num_seqs,
                   int64_t total_tokens, int32_t num_heads, int32_t head_dim_k,
                   int32_t head_dim_v, float scale, float lower_bound,
                   const kda_frontend* frontend, const float* initial_state,
                   float* final_state, void* out, void* workspace, size_t workspace_bytes,
                   hipStream_t stream);

/* --------------------------------------------------- pooled prefill --
 * kda_prefill with the states of a serving engine: each sequence starts from
 * and ends in a slot of an FP32 state pool, addressed by a per-sequence slot
 * index and updated in place, and optionally the state after every
 * `checkpoint_tokens` tokens of each sequence is stored as a checkpoint row
 * (flashinfer PR #5551 "Kimi K3 TP12 H=8 fused KDA decode in the Cake
 * backend on SM100/SM103", embedded PR #5565: section "1. Kernel body" runs
 * FP32 checkpoint rows at a 64-token interval, and its "Baselines and their
 * source PRs" rows use a state pool with indices).  All other arguments, the
 * routes and the workspace are those of kda_prefill.
 *
 *  state_pool   fp32 [num_slots, H, 128, 128] (dv contiguous), 16-byte
 *               aligned, or NULL (zero initial states, final states not
 *               stored).
 *  num_slots    >= 1 when state_pool is set.
 *  slot_indices int32 [N] device array: the slot of each sequence.  A slot
 *               outside [0, num_slots) starts from zeros and is not stored.
 *               Slots in range must be unique.
 *  checkpoints  fp32 [kda_prefill_checkpoint_slots(N, T_tot, checkpoint_tokens),
 *               H, 128, 128], 16-byte aligned, or NULL (none).  The state of
 *               sequence n after j * checkpoint_tokens tokens (j = 1 ..
 *               floor(len_n / checkpoint_tokens)) is stored at slot
 *               n + floor(cu_seqlens[n] / checkpoint_tokens) + j - 1 (unique per
 *               (n, j)); other slots are not written.
 *  checkpoint_tokens  a positive multiple of 32 when checkpoints is set. */
int kda_prefill_pool(const void* q, const void* k, const void* v, const void* g,
                     const void* beta, const int32_t* cu_seqlens, int32_t num_seqs,
                     int64_t total_tokens, int32_t num_heads, int32_t head_dim_k,
                     int32_t head_dim_v, float scale, float lower_bound, float* state_pool,
                     int64_t num_slots, const int32_t* slot_indices, float* checkpoints,
                     int32_t checkpoint_tokens, void* out, void* workspace,
                     size_t workspace_bytes, hipStream_t stream);

/* kda_prefill_pool with the input front-end (as kda_prefill_ex), a pool of
 * either state type and a pool slot stride:
 *  state_dtype  KDA_STATE_F32 (as kda_prefill_pool) or KDA_STATE_BF16 (a
 *               bf16 pool; a sequence's state is widened to FP32 on entry,
 *               carried in FP32 and rounded to nearest-even when stored
 *               back; checkpoints stay FP32).  "FP32/BF16 pool with state
 *               indices" of the pages' serving rows (the composite-schedule
 *               rows include a BF16 pool).
 *  slot_stride  elements from the start of one slot to the next: 0 = the
 *               dense ("page") layout, num_heads * 128 * 128; otherwise the
 *               padded layout, >= that and a multiple of 16 bytes, e.g. one
 *               layer's view of a pool that keeps every layer's states of a
 *               slot together.  Within a slot the [H, 128, 128] state stays
 *               dense.
 * Unknown dtypes, bad strides: KDA_ERR_INVALID_ARGUMENT. */
int kda_prefill_pool_ex(const void* q, const void* k, const void* v, const void* g,
                        const void* beta, const int32_t* cu_seqlens, int32_t num_seqs,
                        int64_t total_tokens, int32_t num_heads, int32_t head_dim_k,
                        int32_t head_dim_v, float scale, float lower_bound,
                        const kda_frontend* frontend, void* state_pool, int32_t state_dtype,
                        int64_t num_slots, int64_t slot_stride, const int32_t* slot_indices,
                        float* checkpoints, int32_t checkpoint_tokens, void* out,
                        void* workspace, size_t workspace_bytes, hipStream_t stream);

/* N + T_tot / checkpoint_tokens + 1: the [H, 128, 128] slots a checkpoint
 * buffer of kda_prefill_pool must hold (0 for invalid arguments). */
size_t kda_prefill_checkpoint_slots(int32_t num_seqs, int64_t total_tokens,
                                    int32_t checkpoint_tokens);

/* Bytes of workspace kda_prefill needs for these sizes with the route it
 * would choose on the current device (or the forced route): 0 for SERIAL and
 * CHUNK; for SPLIT (N + T_tot / 32 + 1) * H * 49152 bytes of chunk records,
 * plus N * H * windows * 2 * 65536 bytes of window states when the plan cuts
 * the chain into windows. */
size_t kda_prefill_workspace_size(int32_t num_seqs, int64_t total_tokens,
                                  int32_t num_heads);

/* Fill *plan with what kda_prefill would launch.  `num_cus` is the device's
 * compute-unit count (<= 0: query the current device).  `route` forces a
 * route (KDA_ROUTE_AUTO to let the planner choose).  Pure host function:
 * it enqueues nothing and touches no device memory.
 *
 * Windows (SPLIT route): the chunk recurrence is affine in the state, S_end =
 * P S_in + B over any run of chunks (the affine composite of flashinfer PR
 * #5551's page, embedded PR #5573, section "1. Composite schedule").  When
 * the chains of a batch would occupy only a small part of the device, the
 * plan cuts every sequence into up to `windows` runs of chunks: the maps
 * (P, B) of the inner windows are computed concurrently with the first
 * window, the true initial state of each window follows by a short carry, and
 * all later windows then run concurrently.  Each sequence is cut by its own
 * length, into runs of max(8, ceil(chunks / windows)) chunks; `window_chunks`
 * reports that cut for a sequence as long as the whole batch (for one
 * sequence, its cut).  The result equals the unwindowed computation up to
 * rounding. */
int kda_prefill_plan(int32_t num_seqs, int64_t total_tokens, int32_t num_heads,
                     float lower_bound, int32_t num_cus, int32_t route,
                     kda_prefill_plan_t* plan);

/* Process-wide route override used by kda_prefill (KDA_ROUTE_AUTO restores
 * automatic selection).  Returns KDA_OK, or KDA_ERR_INVALID_ARGUMENT for an
 * unknown route (the override is then unchanged).  Intended for tests and
 * benchmarks that compare routes. */
int kda_set_prefill_route(int32_t route);

/* ------------------------------------------------- two-pass prefill --
 * kda_prefill_prepare followed by kda_prefill_chain computes exactly what
 * kda_prefill computes with the SPLIT route (bit for bit), whatever route
 * kda_prefill itself would choose.
 *
 * kda_prefill_prepare: every 32-token chunk of every (sequence, head) is
 *   prepared independently ("FlashInfer PR #4262: CAKE KDA Prefill
 *   Highlights", section 2, steps 1-3: gate prefix, anchored Mqk/Akk, the
 *   32x32 inverse T) and turned into a chunk record in `records`: the decayed
 *   queries and restored keys, Mqk, the chunk decay, and U0 = T Diag(b) V and
 *   M = T Diag(b) Kg, so that the chunk's U = U0 - M S for incoming state S.
 *   Inputs, lower_bound and the size arguments are as for kda_prefill.
 *
 * kda_prefill_chain: walks the records of each (sequence, head) in order
 *   (steps 4-7: U, the state update and the outputs) and writes out and
 *   final_state, as kda_prefill.  cu_seqlens, num_seqs, total_tokens and
 *   num_heads must be those the records were prepared with, and the prepare
 *   call must be ordered before it (same stream, or an event).
 *
 * records, records_bytes: caller-owned device memory of at least
 *   kda_prefill_records_size(num_seqs, total_tokens, num_heads) bytes,
 *   16-byte aligned (KDA_ERR_WORKSPACE if missing or too small).  The chain
 *   only reads it; it may be reused once the chain has completed. */
int kda_prefill_prepare(const void* q, const void* k, const void* v, const void* g,
                        const void* beta, const int32_t* cu_seqlens, int32_t num_seqs,
                        int64_t total_tokens, int32_t num_heads, int32_t head_dim_k,
                        int32_t head_dim_v, float lower_bound, void* records,
                        size_t records_bytes, hipStream_t stream);
int kda_prefill_chain(const int32_t* cu_seqlens, int32_t num_seqs, int64_t total_tokens,
                      int32_t num_heads, float scale, const float* initial_state,
                      float* final_state, void* out, const void* records,
                      size_t records_bytes, hipStream_t stream);
/* Bytes kda_prefill_prepare / kda_prefill_chain need on the current device:
 * the SPLIT route's workspace of kda_prefill_workspace_size (0 for invalid
 * sizes). */
size_t kda_prefill_records_size(int32_t num_seqs, int64_t total_tokens, int32_t num_heads);

/* -------------------------------------------------------------- decode --
 * One T=1 step for each row against a slot-indexed state pool.
 *
 *  q, k, g, v  bf16 [rows, num_heads, 128], 16-byte aligned; g = per-channel
 *              natural-log decay (any value <= 0; no bound is needed at T=1).
 *  beta        bf16 [rows, num_heads], post-sigmoid.
 *  state_pool  [num_slots, num_heads, 128, 128] (dv contiguous) of fp32
 *              (KDA_STATE_F32) or bf16 (KDA_STATE_BF16), 16-byte aligned,
 *              read and written in place.  BF16 states are widened to fp32,
 *              updated in fp32 and rounded back to nearest-even.
 *  num_slots   >= 1; offsets are computed in 64 bits (pools above 2^31
 *              elements are fine).
 *  slot_indices  int32 [rows]: pool slot of each row.  A negative entry
 *              skips the row (its out is zero-filled and no slot is touched);
 *              entries >= num_slots are treated the same way.  Non-negative
 *              entries must be unique.
 *  rows        >= 0 (0 = nothing to do).
 *  num_heads   >= 1;  head_dim_k = head_dim_v = 128.
 *  scale       output scale (finite).
 *  out         bf16 [rows, num_heads, 128].
 *  stream      HIP stream. */
int kda_decode(const void* q, const void* k, const void* v, const void* g,
               const void* beta, void* state_pool, int32_t state_dtype,
               int64_t num_slots, const int32_t* slot_indices, int32_t rows,
               int32_t num_heads, int32_t head_dim_k, int32_t head_dim_v,
               float scale, void* out, hipStream_t stream);

/* kda_decode with the input front-end `frontend` (see kda_frontend; NULL =
 * kda_decode) and a pool slot stride (`slot_stride`, as kda_prefill_pool_ex:
 * 0 = dense [num_slots, H, 128, 128], else the elements from one slot to the
 * next, >= num_heads * 128 * 128 and a multiple of 16 bytes).  With a raw
 * gate, the g tensor holds a and any finite value is allowed; with
 * beta_logits, beta holds logits.  The q/k normalisation is folded into the
 * step's reductions (no extra pass over the state).
 * Errors: KDA_ERR_INVALID_ARGUMENT for an unknown gate mode, a lower bound
 * that is not negative and finite (KDA_GATE_LOWER_BOUND), a negative or
 * non-finite norm_eps or a bad slot stride; everything else as kda_decode. */
int kda_decode_ex(const void* q, const void* k, const void* v, const void* g,
                  const void* beta, void* state_pool, int32_t state_dtype,
                  int64_t num_slots, int64_t slot_stride, const int32_t* slot_indices,
                  int32_t rows, int32_t num_heads, int32_t head_dim_k,
                  int32_t head_dim_v, float scale, const kda_frontend* frontend,
                  void* out, hipStream_t stream);

/* ------------------------------------------- allocation-free prefill --
 * kda_prefill for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.  It
 * takes no workspace; the SPLIT route's chunk records and window states live
 * in a static device array of KDA_NOALLOC_SCRATCH_BYTES bytes inside the
 * library (one copy per GPU, held from the first call on that GPU until the
 * process ends).  Nothing is allocated per call, by the library or through
 * any other library.
 *
 * Arguments, routes, results and errors are those of kda_prefill, plus:
 *  - KDA_ERR_WORKSPACE when kda_prefill_workspace_size(num_seqs,
 *    total_tokens, num_heads) exceeds KDA_NOALLOC_SCRATCH_BYTES (nothing is
 *    enqueued);
 *  - KDA_ERR_HIP when the scratch's device address cannot be resolved.
 * The first call on each device resolves that address (hipGetSymbolAddress,
 * no allocation); make it outside graph capture.
 * Every call on one GPU shares that GPU's scratch, whose contents are left
 * from the last call (nothing in it needs to start at zero): calls that can
 * overlap on one GPU (different streams without ordering between them) race
 * and must not be issued; calls ordered on one stream are fine. */
#define KDA_NOALLOC_SCRATCH_BYTES 134217728ULL /* 128 MiB */
int kda_prefill_noalloc(const void* q, const void* k, const void* v, const void* g,
                        const void* beta, const int32_t* cu_seqlens, int32_t num_seqs,
                        int64_t total_tokens, int32_t num_heads, int32_t head_dim_k,
                        int32_t head_dim_v, float scale, float lower_bound,
                        const float* initial_state, float* final_state, void* out,
                        hipStream_t stream);

/* -------------------------------------------------------- input checks --
 * The device-side preconditions that the entry points document but do not
 * check (a check would need a device read and a synchronisation, which a
 * call captured into a hipGraph cannot have), tested on the device -- for
 * tests and debugging, not for the hot path.  Each call enqueues on `stream`
 * two small kernels that set its flags in `flags` (caller-owned device int32
 * [KDA_CHECK_COUNT], 4-byte aligned) to 1 when the check fails anywhere and
 * to 0 otherwise, leaving the other flags alone; the caller synchronises and
 * reads them.  Host-side validation and return values as for the other entry
 * points. */
enum {
  KDA_CHECK_CU_SEQLENS = 0,    /* cu[0] = 0, cu[n] <= cu[n+1], cu[N] = total_tokens */
  KDA_CHECK_GATE_RANGE = 1,    /* lower_bound <= g <= 0, g not NaN (any g <= 0 with -inf) */
  KDA_CHECK_BETA_RANGE = 2,    /* 0 <= beta <= 1 */
  KDA_CHECK_QKV_FINITE = 3,    /* every q, k, v element finite */
  KDA_CHECK_SLOTS_UNIQUE = 4,  /* the slot indices in [0, num_slots) pairwise distinct */
  KDA_CHECK_GATE_STEEP = 5,    /* set when the gate falls by more than 2^232 (160.8 nats)
                                  within an 8-token quarter of a chunk (tokens 0-7, 8-15,
                                  ... of each sequence) in some (head, channel): the
                                  chunk routes are not exact there */
  KDA_CHECK_COUNT = 6
};

/* kda_prefill's inputs (as kda_prefill takes them, plain gates and beta);
 * writes flags KDA_CHECK_CU_SEQLENS .. KDA_CHECK_QKV_FINITE and
 * KDA_CHECK_GATE_STEEP.  Pointers may be NULL only when num_seqs = 0
 * (cu_seqlens) or total_tokens = 0 (the rest). */
int kda_check_prefill_inputs(const void* q, const void* k, const void* v, const void* g,
                             const void* beta, const int32_t* cu_seqlens, int32_t num_seqs,
                             int64_t total_tokens, int32_t num_heads, float lower_bound,
                             int32_t* flags, hipStream_t stream);

/* Slot indices as kda_decode and kda_prefill_pool take them: negative or
 * out-of-range entries are skipped rows (allowed), the others must be
 * distinct.  Writes flag KDA_CHECK_SLOTS_UNIQUE; O(rows^2) comparisons. */
int kda_check_slots(const int32_t* slot_indices, int32_t rows, int64_t num_slots,
                    int32_t* flags, hipStream_t stream);

/* ---------------------------------------------------------------- misc -- */
/* Text describing the last non-OK return on the calling thread ("" if none). */
const char* kda_last_error(void);
/* KDA_ABI_VERSION of the built library. */
int kda_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* KDA_H_ */
