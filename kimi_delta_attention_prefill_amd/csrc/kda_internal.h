// Internal launcher interface between the C ABI (kda_api.cpp) and the HIP
// kernels.  Not installed; the public interface is include/kda.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

constexpr int kHeadDim = 128;
constexpr float kLog2e = 1.4426950408889634f;
// Split-route chain blocks: 16-column value subtiles per block, blocks per
// (sequence, head), and chain blocks that fit one compute unit at once.
constexpr int kSplitSubtiles = 1;
constexpr int kSplitChainTiles = 8 / kSplitSubtiles;
constexpr int kSplitBlocksPerCU = 2;

// Input front-end: gate_mode 0 = g is the natural-log decay, 1 = g holds a
// and the decay is lower_bound * sigmoid(a), 2 = g holds a and the decay is
// -softplus(a); beta_logits: beta = sigmoid(beta); normalize_qk: q, k scaled
// by 1 / sqrt(sum x^2 + norm_eps) per (token, head).
struct FrontEnd {
  int32_t gate_mode = 0;
  float lower_bound = 0.f;
  int32_t beta_logits = 0;
  int32_t normalize_qk = 0;
  float norm_eps = 0.f;
};

// Whether any front-end transform is requested (kernels without it are
// compiled separately so the plain path carries none of its code).
inline __host__ __device__ bool frontend_active(const FrontEnd& fe) {
  return fe.gate_mode != 0 || fe.beta_logits != 0 || fe.normalize_qk != 0;
}

struct PrefillArgs {
  const uint16_t* q;      // bf16 [T, H, 128]
  const uint16_t* k;      // bf16 [T, H, 128]
  const uint16_t* v;      // bf16 [T, H, 128]
  const uint16_t* g;      // bf16 [T, H, 128], natural-log decay
  const uint16_t* beta;   // bf16 [T, H]
  const int32_t* cu_seqlens;  // int32 [N + 1]
  int32_t num_seqs;
  int32_t total_tokens;
  int32_t num_heads;
  float scale;
  float anchor_log2;      // C = 16 * lower_bound * log2(e)  (chunk route)
  float half_anchor_log2; // nearest integer to 8 * lower_bound * log2(e) (split-16 mode)
  const float* s0;        // fp32 [N, H, 128, 128] or null
  float* s1;              // fp32 [N, H, 128, 128] or null
  uint16_t* out;          // bf16 [T, H, 128]
  int32_t windows;        // split route: windows per sequence (1 = none)
  int32_t window_chunks;  // split route: chunks per window (0 = none)
  // State pool addressing (kda_prefill_pool): when `pool` is set, s0/s1 are
  // unused and sequence n starts from and ends in pool slot slots[n] (a slot
  // outside [0, num_slots) starts from zeros and is not stored).
  void* pool;             // fp32 or bf16 [num_slots, H, 128, 128] or null
  int32_t pool_bf16;      // the pool holds bf16 states (read widened, written RNE)
  const int32_t* slots;   // int32 [N]
  int64_t num_slots;
  int64_t slot_stride;    // elements from one slot to the next (>= H * 128 * 128)
  // Checkpoints: the state after every `ckpt_tokens` tokens (a multiple of
  // 32) of each sequence; the j-th (j >= 1) of sequence n goes to slot
  // n + floor(cu[n] / ckpt_tokens) + j - 1 of ckpt [., H, 128, 128].
  float* ckpt;            // fp32 or null
  int32_t ckpt_tokens;
  FrontEnd fe;            // how g and beta are given, q/k normalisation
  // Stream route only: a null cu_seqlens means one token per sequence (token
  // n of sequence n: the T = 1 decode), and with skip_null_slots a sequence
  // whose pool slot is out of range gets zero outputs (the decode's
  // skipped row) instead of a step from the zero state.
  int32_t skip_null_slots;
};

struct DecodeArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* g;
  const uint16_t* beta;
  void* pool;             // fp32 or bf16 [num_slots, H, 128, 128]
  const int32_t* slots;   // int32 [rows]
  int64_t num_slots;
  int64_t slot_stride;    // elements from one slot to the next (>= H * 128 * 128)
  int32_t rows;
  int32_t num_heads;
  float scale;
  uint16_t* out;          // bf16 [rows, H, 128]
  FrontEnd fe;            // how g and beta are given, q/k normalisation
};

// Token-serial FP32 prefill; `waves` value-column tiles of 16 per block.
hipError_t launch_prefill_serial(const PrefillArgs& a, int waves, hipStream_t s);
// Chunk-32 MFMA prefill.
hipError_t launch_prefill_chunk(const PrefillArgs& a, int anchor_mode, int dv_split,
                                hipStream_t s);
// Two-pass chunk-32 prefill (parallel chunk preparation, then the serial
// state chain); needs split_workspace_bytes() of device workspace.
// dv_split must be 8: one 16-column chain per block.
hipError_t launch_prefill_split(const PrefillArgs& a, int anchor_mode, int dv_split,
                                void* workspace, hipStream_t s);
// Its two passes on their own (the chain reads only cu_seqlens, the sizes,
// scale, s0, s1 and out of `a`).
hipError_t launch_prefill_split_prepare(const PrefillArgs& a, int anchor_mode, void* workspace,
                                        hipStream_t s);
hipError_t launch_prefill_split_chain(const PrefillArgs& a, const void* workspace,
                                      hipStream_t s);
size_t split_workspace_bytes(int32_t num_seqs, int64_t total_tokens, int32_t num_heads,
                             int32_t windows);
// Token stream over many short sequences (multi-token decode): the prefill
// with one block per (sequence, head, `cols` value columns, 128 or 64), the
// state in registers across the sequence's tokens.
hipError_t launch_prefill_stream(const PrefillArgs& a, int cols, hipStream_t s);
// Decode step; `cols` = value columns per block (32, 64 or 128 for FP32
// state, 64 or 128 for BF16), `threads` per block (256 or 512).
hipError_t launch_decode(const DecodeArgs& a, bool bf16_state, int cols, int threads,
                         hipStream_t s);

// Records `code` and the formatted text as the calling thread's last error
// (kda_last_error) and returns `code`.
int set_error(int code, const char* fmt, ...);

// Device-side precondition checks (debugging and tests).
struct CheckPrefillArgs {
  const uint16_t *q, *k, *v, *g, *beta;   // bf16 as kda_prefill takes them
  const int32_t* cu_seqlens;              // [num_seqs + 1]
  int32_t num_seqs;
  int64_t total_tokens;
  int32_t num_heads;
  float lower_bound;
  bool bounded;                           // lower_bound is finite
  int32_t* flags;                         // [KDA_CHECK_COUNT]
};
hipError_t launch_check_prefill(const CheckPrefillArgs& a, hipStream_t s);
hipError_t launch_check_slots(const int32_t* slots, int32_t rows, int64_t num_slots,
                              int32_t* flags, hipStream_t s);

}  // namespace kda
