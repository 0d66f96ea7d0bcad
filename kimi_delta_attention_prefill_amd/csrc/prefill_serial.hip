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
// Tokens are staged up to 16 at a time through LDS (only those the sequence
// has), already widened to fp32, with exp(g) precomputed once per (token,
// channel).
//
// The block's state tile (128 key rows x 16 W value columns) moves between
// HBM and the lanes' registers through an LDS transpose: global memory sees
// 16-byte vectors along the rows (whole 128-byte row pieces from W = 2 up),
// where the compute layout alone, one column per lane, would issue 4-byte
// accesses.  With many short sequences (multi-token decode, T = 2 ... 8 per
// row) the route is a stream over the states, so this is its hot path.
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {
namespace {

constexpr int kStage = 16;        // tokens staged per round
constexpr int kTileStride = 132;  // floats per tile column: 128 rows + 4, so
                                  // the 16 columns x 4 row groups a wave reads
                                  // fall on 64 distinct banks

typedef float f32x4v __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4v __attribute__((ext_vector_type(4)));

template <int W>
struct SerialSmem {
  union {
    struct {
      float q[kStage][kHeadDim];
      float k[kStage][kHeadDim];
      float d[kStage][kHeadDim];  // exp(g)
      float v[kStage][16 * W];
      float b[kStage];
    } st;
    float tile[16 * W][kTileStride];  // state tile, column-major
  };
};

// State tile (rows 0..127, columns c0 .. c0 + 16 W) from HBM into LDS.  The
// state is read once per call, so the loads are non-temporal.
template <int W>
__device__ __forceinline__ void tile_load(const StateRef& s, int c0, float (*tile)[kTileStride],
                                          int tid) {
  constexpr int NT = 64 * W, COLS = 16 * W;
  if (s.bf16) {
    constexpr int VPR = COLS / 8;  // 16-byte vectors per row
    const uint16_t* p = static_cast<const uint16_t*>(s.p) + c0;
    for (int e = tid; e < kHeadDim * VPR; e += NT) {
      const int r = e / VPR, c = (e % VPR) * 8;
      const u32x4v w =
          __builtin_nontemporal_load(reinterpret_cast<const u32x4v*>(p + r * kHeadDim + c));
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        tile[c + 2 * m][r] = bf16lo(w[m]);
        tile[c + 2 * m + 1][r] = bf16hi(w[m]);
      }
    }
  } else {
    constexpr int VPR = COLS / 4;
    const float* p = static_cast<const float*>(s.p) + c0;
    for (int e = tid; e < kHeadDim * VPR; e += NT) {
      const int r = e / VPR, c = (e % VPR) * 4;
      const f32x4v x =
          __builtin_nontemporal_load(reinterpret_cast<const f32x4v*>(p + r * kHeadDim + c));
#pragma unroll
      for (int m = 0; m < 4; ++m) tile[c + m][r] = x[m];
    }
  }
}

// The LDS state tile back to HBM (BF16: rounded to nearest even).
template <int W>
__device__ __forceinline__ void tile_store(const StateRef& s, int c0,
                                           const float (*tile)[kTileStride], int tid) {
  constexpr int NT = 64 * W, COLS = 16 * W;
  if (s.bf16) {
    constexpr int VPR = COLS / 8;
    uint16_t* p = static_cast<uint16_t*>(s.p) + c0;
    for (int e = tid; e < kHeadDim * VPR; e += NT) {
      const int r = e / VPR, c = (e % VPR) * 8;
      u32x4v w;
#pragma unroll
      for (int m = 0; m < 4; ++m)
        w[m] = (uint32_t)f32_to_bf16(tile[c + 2 * m][r]) |
               ((uint32_t)f32_to_bf16(tile[c + 2 * m + 1][r]) << 16);
      __builtin_nontemporal_store(w, reinterpret_cast<u32x4v*>(p + r * kHeadDim + c));
    }
  } else {
    constexpr int VPR = COLS / 4;
    float* p = static_cast<float*>(s.p) + c0;
    for (int e = tid; e < kHeadDim * VPR; e += NT) {
      const int r = e / VPR, c = (e % VPR) * 4;
      const f32x4v x = {tile[c][r], tile[c + 1][r], tile[c + 2][r], tile[c + 3][r]};
      __builtin_nontemporal_store(x, reinterpret_cast<f32x4v*>(p + r * kHeadDim + c));
    }
  }
}

template <int W>
__global__ __launch_bounds__(64 * W) void prefill_serial_kernel(PrefillArgs a) {
  __shared__ SerialSmem<W> sm;
  auto& st = sm.st;

  const int H = a.num_heads;
  const int slice = blockIdx.x, h = blockIdx.y, n = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int jl = lane & 15;       // column within the wave's tile
  const int rg = lane >> 4;       // row group 0..3
  const int c0 = slice * 16 * W;  // the block's first value column
  const int col = c0 + wave * 16 + jl;
  const int tc = wave * 16 + jl;  // the lane's column in the state tile

  const int bos = clamp_offset(a.cu_seqlens[n], a.total_tokens);
  const int eos = max(bos, clamp_offset(a.cu_seqlens[n + 1], a.total_tokens));

  float S[32];
  if (const StateRef s0 = prefill_initial_state(a, n, h)) {  // uniform over the block
    tile_load<W>(s0, c0, sm.tile, tid);
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 32; ++i) S[i] = sm.tile[tc][4 * i + rg];
  } else {
#pragma unroll
    for (int i = 0; i < 32; ++i) S[i] = 0.f;
  }

  for (int t0 = bos; t0 < eos; t0 += kStage) {
    const int L = min(kStage, eos - t0);
    __syncthreads();  // the previous round (or the state tile) finished reading LDS
    // q, k, g rows: 16 x 16-byte loads per token row.
    for (int e = tid; e < L * 16; e += 64 * W) {
      const int t = e >> 4, c8 = (e & 15) * 8;
      const int64_t off = ((int64_t)(t0 + t) * H + h) * kHeadDim + c8;
      const uint4 wq = *reinterpret_cast<const uint4*>(a.q + off);
      const uint4 wk = *reinterpret_cast<const uint4*>(a.k + off);
      const uint4 wg = *reinterpret_cast<const uint4*>(a.g + off);
      const uint32_t uq[4] = {wq.x, wq.y, wq.z, wq.w};
      const uint32_t uk[4] = {wk.x, wk.y, wk.z, wk.w};
      const uint32_t ug[4] = {wg.x, wg.y, wg.z, wg.w};
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        st.q[t][c8 + 2 * m] = bf16lo(uq[m]);
        st.q[t][c8 + 2 * m + 1] = bf16hi(uq[m]);
        st.k[t][c8 + 2 * m] = bf16lo(uk[m]);
        st.k[t][c8 + 2 * m + 1] = bf16hi(uk[m]);
        st.d[t][c8 + 2 * m] = fast_exp2(frontend_gate(a.fe, bf16lo(ug[m])) * kLog2e);
        st.d[t][c8 + 2 * m + 1] = fast_exp2(frontend_gate(a.fe, bf16hi(ug[m])) * kLog2e);
      }
    }
    for (int e = tid; e < L * 16 * W; e += 64 * W) {
      const int t = e / (16 * W), jj = e % (16 * W);
      st.v[t][jj] = bf16_to_f32(a.v[((int64_t)(t0 + t) * H + h) * kHeadDim + c0 + jj]);
    }
    if (tid < L)
      st.b[tid] = frontend_beta(a.fe, bf16_to_f32(a.beta[(int64_t)(t0 + tid) * H + h]));
    __syncthreads();

    for (int t = 0; t < L; ++t) {
      float w = 0.f, p = 0.f, qk = 0.f, qq = 0.f, kk = 0.f;
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        const int c = 4 * i + rg;
        S[i] *= st.d[t][c];
        w = fmaf(st.k[t][c], S[i], w);
        p = fmaf(st.q[t][c], S[i], p);
        qk = fmaf(st.q[t][c], st.k[t][c], qk);
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
          qq = fmaf(st.q[t][c], st.q[t][c], qq);
          kk = fmaf(st.k[t][c], st.k[t][c], kk);
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
      const float u = st.b[t] * (st.v[t][tc] - w);
      const float uk = u * rk;
#pragma unroll
      for (int i = 0; i < 32; ++i) S[i] = fmaf(st.k[t][4 * i + rg], uk, S[i]);
      if (rg == 0)
        a.out[((int64_t)(t0 + t) * H + h) * kHeadDim + col] = f32_to_bf16(a.scale * fmaf(qk, u, p));
      if (float* cp = prefill_checkpoint(a, n, h, bos, t0 + t + 1 - bos)) {
#pragma unroll
        for (int i = 0; i < 32; ++i) cp[(4 * i + rg) * kHeadDim + col] = S[i];
      }
    }
  }
  if (const StateRef s1 = prefill_final_state(a, n, h)) {  // uniform over the block
    __syncthreads();  // the last round finished reading the staged tokens
#pragma unroll
    for (int i = 0; i < 32; ++i) sm.tile[tc][4 * i + rg] = S[i];
    __syncthreads();
    tile_store<W>(s1, c0, sm.tile, tid);
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
