// Token-serial FP32 KDA prefill for gfx950 (the reference-grade route).
//
// Evaluates, token by token in FP32, the gated delta rule
//   S_t = (I - b_t k_t k_t^T) Diag(exp(g_t)) S_{t-1} + b_t k_t v_t^T,
//   o_t = scale S_t^T q_t,
// the recurrence whose chunked form is described in "FlashInfer PR #4262:
// CAKE KDA Prefill Highlights", section 2.  Value columns evolve
// independently (the state update only mixes key rows), which is what the
// note's M64/M128 schedules exploit; here every wave owns 16 value columns of
// one (sequence, head) and needs no communication with other waves except the
// shared, LDS-staged token operands.
//
// Work decomposition: grid = (128 / (16 * W), H, N), block = 64 * W threads.
// Lane l of a wave owns value column (l & 15) and the 32 key rows
// c = 4 * i + (l >> 4), i = 0..31 (interleaved so the four row groups read
// different LDS banks).  The two dk-reductions of a step, w = S'^T k and
// p = S'^T q, are finished with two cross-lane xor shuffles; the output uses
// o = scale (p + (q . k) u), which equals scale S''^T q after the write.
// Tokens are staged 32 at a time through LDS, already widened to fp32, with
// exp(g) precomputed once per (token, channel).
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {
namespace {

constexpr int kStage = 32;  // tokens staged per round

template <int W>
__global__ __launch_bounds__(64 * W) void prefill_serial_kernel(PrefillArgs a) {
  __shared__ float sq[kStage][kHeadDim];
  __shared__ float sk[kStage][kHeadDim];
  __shared__ float sd[kStage][kHeadDim];  // exp(g)
  __shared__ float sv[kStage][16 * W];
  __shared__ float sb[kStage];

  const int H = a.num_heads;
  const int slice = blockIdx.x, h = blockIdx.y, n = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int jl = lane & 15;       // column within the wave's tile
  const int rg = lane >> 4;       // row group 0..3
  const int col = slice * 16 * W + wave * 16 + jl;

  const int bos = clamp_offset(a.cu_seqlens[n], a.total_tokens);
  const int eos = max(bos, clamp_offset(a.cu_seqlens[n + 1], a.total_tokens));
  const StateRef s0 = prefill_initial_state(a, n, h);

  float S[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) S[i] = s0 ? s0.load((4 * i + rg) * kHeadDim + col) : 0.f;

  for (int t0 = bos; t0 < eos; t0 += kStage) {
    const int L = min(kStage, eos - t0);
    __syncthreads();  // previous round finished reading the stage
    // q, k, g rows: 16 x 16-byte loads per token row.
    for (int e = tid; e < kStage * 16; e += 64 * W) {
      const int t = e >> 4, c8 = (e & 15) * 8;
      uint4 wq = {0, 0, 0, 0}, wk = {0, 0, 0, 0}, wg = {0, 0, 0, 0};
      if (t < L) {
        const int64_t off = ((int64_t)(t0 + t) * H + h) * kHeadDim + c8;
        wq = *reinterpret_cast<const uint4*>(a.q + off);
        wk = *reinterpret_cast<const uint4*>(a.k + off);
        wg = *reinterpret_cast<const uint4*>(a.g + off);
      }
      const uint32_t uq[4] = {wq.x, wq.y, wq.z, wq.w};
      const uint32_t uk[4] = {wk.x, wk.y, wk.z, wk.w};
      const uint32_t ug[4] = {wg.x, wg.y, wg.z, wg.w};
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        sq[t][c8 + 2 * m] = bf16lo(uq[m]);
        sq[t][c8 + 2 * m + 1] = bf16hi(uq[m]);
        sk[t][c8 + 2 * m] = bf16lo(uk[m]);
        sk[t][c8 + 2 * m + 1] = bf16hi(uk[m]);
        sd[t][c8 + 2 * m] = fast_exp2(frontend_gate(a.fe, bf16lo(ug[m])) * kLog2e);
        sd[t][c8 + 2 * m + 1] = fast_exp2(frontend_gate(a.fe, bf16hi(ug[m])) * kLog2e);
      }
    }
    for (int e = tid; e < kStage * 16 * W; e += 64 * W) {
      const int t = e / (16 * W), jj = e % (16 * W);
      sv[t][jj] = t < L ? bf16_to_f32(a.v[((int64_t)(t0 + t) * H + h) * kHeadDim +
                                          slice * 16 * W + jj])
                        : 0.f;
    }
    if (tid < kStage)
      sb[tid] = tid < L ? frontend_beta(a.fe, bf16_to_f32(a.beta[(int64_t)(t0 + tid) * H + h])) : 0.f;
    __syncthreads();

    for (int t = 0; t < L; ++t) {
      float w = 0.f, p = 0.f, qk = 0.f, qq = 0.f, kk = 0.f;
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        const int c = 4 * i + rg;
        S[i] *= sd[t][c];
        w = fmaf(sk[t][c], S[i], w);
        p = fmaf(sq[t][c], S[i], p);
        qk = fmaf(sq[t][c], sk[t][c], qk);
      }
      w += __shfl_xor(w, 16);
      w += __shfl_xor(w, 32);
      p += __shfl_xor(p, 16);
      p += __shfl_xor(p, 32);
      qk += __shfl_xor(qk, 16);
      qk += __shfl_xor(qk, 32);
      // q/k L2 norm: w, p, q.k are linear in k and q, so they are scaled
      // afterwards; the update adds k (u / |k|)^T.
      float rk = 1.f;
      if (a.fe.normalize_qk) {
#pragma unroll
        for (int i = 0; i < 32; ++i) {
          const int c = 4 * i + rg;
          qq = fmaf(sq[t][c], sq[t][c], qq);
          kk = fmaf(sk[t][c], sk[t][c], kk);
        }
        qq += __shfl_xor(qq, 16);
        qq += __shfl_xor(qq, 32);
        kk += __shfl_xor(kk, 16);
        kk += __shfl_xor(kk, 32);
        const float rq = inv_norm(qq + a.fe.norm_eps);
        rk = inv_norm(kk + a.fe.norm_eps);
        w *= rk;
        p *= rq;
        qk *= rq * rk;
      }
      const float u = sb[t] * (sv[t][wave * 16 + jl] - w);
      const float uk = u * rk;
#pragma unroll
      for (int i = 0; i < 32; ++i) S[i] = fmaf(sk[t][4 * i + rg], uk, S[i]);
      if (rg == 0)
        a.out[((int64_t)(t0 + t) * H + h) * kHeadDim + col] = f32_to_bf16(a.scale * fmaf(qk, u, p));
      if (float* cp = prefill_checkpoint(a, n, h, bos, t0 + t + 1 - bos)) {
#pragma unroll
        for (int i = 0; i < 32; ++i) cp[(4 * i + rg) * kHeadDim + col] = S[i];
      }
    }
  }
  if (const StateRef s1 = prefill_final_state(a, n, h)) {
#pragma unroll
    for (int i = 0; i < 32; ++i) s1.store((4 * i + rg) * kHeadDim + col, S[i]);
  }
}

}  // namespace

hipError_t launch_prefill_serial(const PrefillArgs& a, int waves, hipStream_t s) {
  if (a.num_seqs <= 0) return hipSuccess;
  switch (waves) {
    case 1:
      prefill_serial_kernel<1><<<dim3(8, a.num_heads, a.num_seqs), 64, 0, s>>>(a);
      break;
    case 2:
      prefill_serial_kernel<2><<<dim3(4, a.num_heads, a.num_seqs), 128, 0, s>>>(a);
      break;
    case 4:
      prefill_serial_kernel<4><<<dim3(2, a.num_heads, a.num_seqs), 256, 0, s>>>(a);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace kda
