// Device-side checks of the preconditions the entry points document but do
// not check: packed sequence offsets, gate and beta ranges, finite q/k/v,
// distinct pool slots (for tests and debugging; see kda_check_prefill_inputs
// and kda_check_slots in kda.h).  A failing check sets its flag with a plain
// store of 1 (every writer stores the same value); the flags are cleared by
// a separate one-block kernel first, in stream order.
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {
namespace {

constexpr int kCheckThreads = 256;

__global__ void clear_flags(int32_t* flags, int first, int count) {
  if ((int)threadIdx.x < count) flags[first + threadIdx.x] = 0;
}

// The gate's fall over an 8-token quarter of a chunk (its prefix from the
// quarter's first to its last token, natural log) beyond which the chunk
// routes' quarter products, anchored at the quarter's midpoint, exceed the
// 2^116 factor budget within which the operands' bf16 low halves keep their
// precision: 2^232.
constexpr float kQuarterFallLimit = 232.f / 1.4426950408889634f;

// Sequence of token t (the largest n with cu[n] <= t), with the offsets
// clamped as the prefill kernels clamp them.
__device__ __forceinline__ int sequence_of(const CheckPrefillArgs& a, int64_t t) {
  int lo = 0, hi = a.num_seqs - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    const int64_t c = a.cu_seqlens[mid] < 0 ? 0 : a.cu_seqlens[mid];
    if (c <= t) lo = mid; else hi = mid - 1;
  }
  return lo;
}

__device__ __forceinline__ bool bf16_finite(uint16_t x) { return (x & 0x7F80u) != 0x7F80u; }

__global__ __launch_bounds__(kCheckThreads) void check_prefill_kernel(CheckPrefillArgs a) {
  const int64_t tid = (int64_t)blockIdx.x * kCheckThreads + threadIdx.x;
  const int64_t stride = (int64_t)gridDim.x * kCheckThreads;
  bool bad_cu = false, bad_gate = false, bad_beta = false, bad_qkv = false, steep = false;
  // sequence offsets
  for (int64_t i = tid; i <= a.num_seqs; i += stride) {
    const int32_t c = a.cu_seqlens[i];
    if (c < 0 || (int64_t)c > a.total_tokens) bad_cu = true;
    if (i == 0 && c != 0) bad_cu = true;
    if (i == a.num_seqs && (int64_t)c != a.total_tokens) bad_cu = true;
    if (i < a.num_seqs && c > a.cu_seqlens[i + 1]) bad_cu = true;
  }
  // per-element tensors [T, H, 128]
  const int64_t elems = a.total_tokens * a.num_heads * kHeadDim;
  for (int64_t i = tid; i < elems; i += stride) {
    if (!bf16_finite(a.q[i]) || !bf16_finite(a.k[i]) || !bf16_finite(a.v[i])) bad_qkv = true;
    const float gv = bf16_to_f32(a.g[i]);
    if (!(gv <= 0.f) || (a.bounded && !(gv >= a.lower_bound))) bad_gate = true;
    // element (t, h, c) that opens an 8-token quarter of a chunk of its sequence
    const int64_t t = i / ((int64_t)a.num_heads * kHeadDim);
    if (a.num_seqs > 0) {
      const int n = sequence_of(a, t);
      const int64_t bos = a.cu_seqlens[n] < 0 ? 0 : a.cu_seqlens[n];
      const int64_t eos = a.cu_seqlens[n + 1] > a.total_tokens ? a.total_tokens : a.cu_seqlens[n + 1];
      if (t >= bos && t < eos && (t - bos) % 8 == 0) {
        float fall = 0.f;
        for (int64_t u = t + 1; u < t + 8 && u < eos; ++u)
          fall -= bf16_to_f32(a.g[i + (u - t) * a.num_heads * kHeadDim]);
        if (fall > kQuarterFallLimit) steep = true;
      }
    }
  }
  const int64_t tokheads = a.total_tokens * a.num_heads;
  for (int64_t i = tid; i < tokheads; i += stride) {
    const float b = bf16_to_f32(a.beta[i]);
    if (!(b >= 0.f && b <= 1.f)) bad_beta = true;
  }
  if (bad_cu) a.flags[0] = 1;
  if (bad_gate) a.flags[1] = 1;
  if (bad_beta) a.flags[2] = 1;
  if (bad_qkv) a.flags[3] = 1;
  if (steep) a.flags[5] = 1;
}

__global__ __launch_bounds__(kCheckThreads) void check_slots_kernel(const int32_t* slots, int32_t rows,
                                                                    int64_t num_slots, int32_t* flag) {
  const int64_t tid = (int64_t)blockIdx.x * kCheckThreads + threadIdx.x;
  const int64_t stride = (int64_t)gridDim.x * kCheckThreads;
  bool dup = false;
  for (int64_t r = tid; r < rows; r += stride) {
    const int32_t s = slots[r];
    if (s < 0 || (int64_t)s >= num_slots) continue;   // a skipped row
    for (int64_t o = 0; o < r; ++o)
      if (slots[o] == s) dup = true;
  }
  if (dup) *flag = 1;
}

unsigned grid_for(int64_t work) {
  const int64_t blocks = (work + kCheckThreads - 1) / kCheckThreads;
  return (unsigned)(blocks < 1 ? 1 : (blocks > 4096 ? 4096 : blocks));
}

}  // namespace

hipError_t launch_check_prefill(const CheckPrefillArgs& a, hipStream_t s) {
  clear_flags<<<1, 64, 0, s>>>(a.flags, 0, 4);
  clear_flags<<<1, 64, 0, s>>>(a.flags, 5, 1);
  const int64_t work = a.total_tokens * a.num_heads * kHeadDim;
  check_prefill_kernel<<<grid_for(work > a.num_seqs + 1 ? work : a.num_seqs + 1), kCheckThreads, 0,
                         s>>>(a);
  return hipGetLastError();
}

hipError_t launch_check_slots(const int32_t* slots, int32_t rows, int64_t num_slots,
                              int32_t* flags, hipStream_t s) {
  clear_flags<<<1, 64, 0, s>>>(flags, 4, 1);
  if (rows > 0) check_slots_kernel<<<grid_for(rows), kCheckThreads, 0, s>>>(slots, rows, num_slots, flags + 4);
  return hipGetLastError();
}

}  // namespace kda
