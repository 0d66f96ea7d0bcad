// Small device helpers shared by the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kda_internal.h"

namespace kda {

// bf16 (stored as uint16) -> fp32: exact, a 16-bit left shift.
__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}
// Low / high bf16 of a packed 32-bit word -> fp32.
__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// fp32 -> bf16, round to nearest even (lowers to v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint16_t f32_to_bf16(float x) {
  __bf16 b = static_cast<__bf16>(x);
  return __builtin_bit_cast(uint16_t, b);
}

// 2^x on the hardware exponential unit (v_exp_f32).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Input front-end (FrontEnd): the natural-log decay g from the gate tensor's
// value x, and beta from the beta tensor's value.
__device__ __forceinline__ float frontend_gate(const FrontEnd& fe, float x) {
  if (fe.gate_mode == 1) return fe.lower_bound / (1.f + fast_exp2(-x * kLog2e));   // lb sigmoid(x)
  if (fe.gate_mode == 2) {   // -softplus(x) = -(max(x, 0) + ln(1 + e^-|x|))
    const float e = fast_exp2(-__builtin_fabsf(x) * kLog2e);
    return -(__builtin_fmaxf(x, 0.f) + __builtin_amdgcn_logf(1.f + e) * 0.6931471805599453f);
  }
  return x;
}
// 1 / sqrt(x) for a front-end L2 norm (x = sum of squares + eps); a zero
// vector (x == 0, e.g. a padding token) is left at zero instead of 0 * inf.
__device__ __forceinline__ float inv_norm(float x) { return x > 0.f ? 1.f / __builtin_sqrtf(x) : 0.f; }
__device__ __forceinline__ float frontend_beta(const FrontEnd& fe, float b) {
  return fe.beta_logits ? 1.f / (1.f + fast_exp2(-b * kLog2e)) : b;
}

// Raw buffer resource over [base, base + bytes): buffer loads outside return
// 0 and buffer stores outside are dropped by the hardware (gfx9 word 3).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_buffer(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}
// 16-bit store through a buffer resource at byte offset `off` (unconditional
// instruction; out-of-range offsets are discarded).
__device__ __forceinline__ void buffer_store_u16(uint16_t v, __amdgpu_buffer_rsrc_t r, uint32_t off) {
  __builtin_amdgcn_raw_buffer_store_b16(v, r, off, 0, 0);
}

// Block barrier that orders LDS accesses only: the LDS writes before it are
// complete and visible after it, while global loads and stores stay in
// flight across it.  __syncthreads() would also wait for every outstanding
// global access, exposing a prefetch's whole latency at the next barrier.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Clamp a device-read sequence offset into [0, total].
__device__ __forceinline__ int clamp_offset(int x, int total) {
  return x < 0 ? 0 : (x > total ? total : x);
}

// The [128][128] FP32 state a prefill of (sequence n, head h) starts from
// (null: zeros) and the one it ends in (null: not stored).
// One [128][128] state of a sequence-head: FP32, or BF16 in a bf16 state pool
// (widened on load, rounded to nearest-even on store), or none.
struct StateRef {
  void* p = nullptr;
  bool bf16 = false;
  __device__ __forceinline__ explicit operator bool() const { return p != nullptr; }
  __device__ __forceinline__ float load(int i) const {
    return bf16 ? bf16_to_f32(static_cast<const uint16_t*>(p)[i]) : static_cast<const float*>(p)[i];
  }
  __device__ __forceinline__ void store(int i, float v) const {
    if (bf16)
      static_cast<uint16_t*>(p)[i] = f32_to_bf16(v);
    else
      static_cast<float*>(p)[i] = v;
  }
};
__device__ __forceinline__ StateRef fp32_state(const float* p) {
  StateRef r;
  r.p = const_cast<float*>(p);
  return r;
}
__device__ __forceinline__ StateRef prefill_pool_state(const PrefillArgs& a, int n, int h) {
  const int64_t s = a.slots[n];
  StateRef r;
  if (s >= 0 && s < a.num_slots) {
    const int64_t off = s * a.slot_stride + h * (kHeadDim * kHeadDim);
    r.bf16 = a.pool_bf16 != 0;
    r.p = r.bf16 ? static_cast<void*>(static_cast<uint16_t*>(a.pool) + off)
                 : static_cast<void*>(static_cast<float*>(a.pool) + off);
  }
  return r;
}
__device__ __forceinline__ StateRef prefill_initial_state(const PrefillArgs& a, int n, int h) {
  if (a.pool) return prefill_pool_state(a, n, h);
  return fp32_state(a.s0 ? a.s0 + ((int64_t)n * a.num_heads + h) * (kHeadDim * kHeadDim) : nullptr);
}
__device__ __forceinline__ StateRef prefill_final_state(const PrefillArgs& a, int n, int h) {
  if (a.pool) return prefill_pool_state(a, n, h);
  return fp32_state(a.s1 ? a.s1 + ((int64_t)n * a.num_heads + h) * (kHeadDim * kHeadDim) : nullptr);
}
// Where the state after `done` tokens of sequence n (starting at token bos)
// is checkpointed, or null when checkpoints are off or `done` is not a
// positive multiple of the interval.
__device__ __forceinline__ float* prefill_checkpoint(const PrefillArgs& a, int n, int h, int bos,
                                                     int done) {
  if (!a.ckpt || done <= 0 || done % a.ckpt_tokens != 0) return nullptr;
  const int64_t slot = (int64_t)n + bos / a.ckpt_tokens + done / a.ckpt_tokens - 1;
  return a.ckpt + (slot * a.num_heads + h) * (int64_t)(kHeadDim * kHeadDim);
}

}  // namespace kda
