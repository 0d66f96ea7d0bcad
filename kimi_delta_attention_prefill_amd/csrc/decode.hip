// T=1 KDA decode over a slot-indexed state pool, for gfx950.
//
// One step of the gated delta rule per (row, head) item, in place on the
// pool slot the row names ("Kimi K3 TP12 H=8 fused KDA decode", flashinfer
// PR #5551: positive unique slots, FP32 and BF16 state, 64-bit slot
// offsets):
//   S'  = Diag(exp(g)) S,   w = S'^T k,   p = S'^T q,   u = b (v - w),
//   S'' = S' + k u^T  (stored),   o = scale (p + (q . k) u) = scale S''^T q.
//
// The step moves 128 KiB (FP32) or 64 KiB (BF16) of state per item and does
// ~7 flops per state element, so it is an HBM stream.  Each block owns one
// item's value-column slice of COLS columns: thread t holds four adjacent
// columns (one 16-byte FP32 or 8-byte BF16 vector per row) of the key rows
// c = rg + RG * i, so every wave reads and writes contiguous rows.  The item's
// base address is formed once in 64 bits; in-item offsets are 32-bit.
// The two dk-reductions (w, p) and q . k are finished with xor shuffles
// inside a wave and one LDS exchange across the four waves; the state is
// read once and written once.  Row counts too small to fill the chip use
// narrower slices (more blocks per item).
//
// Optional input front-end (the decode ABI of that PR carries a lower-bound
// switch, the bound and norm_eps; its tests use softplus and lower-bound
// gates): the decay from a raw gate input a, e^{lb sigmoid(a)} or
// e^{-softplus(a)} = sigmoid(-a); beta from logits; q and k L2-normalised.
// The normalisation costs no extra pass: w, p and q . k are linear in k and
// q, so they are reduced from the raw vectors and scaled by 1/|k|, 1/|q| (two
// more block sums), and 1/|k| is folded into u for the state update.
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {
namespace {

constexpr int kThreads = 256;

template <bool BF16>
struct StateIO;

// The state of a row is read once and written once per step, so its traffic
// is marked non-temporal (streamed past the caches).
typedef float f32x4v __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2v __attribute__((ext_vector_type(2)));

template <>
struct StateIO<false> {
  using elem = float;
  static __device__ __forceinline__ float4 load(const float* p) {
    const f32x4v x = __builtin_nontemporal_load(reinterpret_cast<const f32x4v*>(p));
    return make_float4(x[0], x[1], x[2], x[3]);
  }
  static __device__ __forceinline__ void store(float* p, float4 x) {
    const f32x4v v = {x.x, x.y, x.z, x.w};
    __builtin_nontemporal_store(v, reinterpret_cast<f32x4v*>(p));
  }
};

template <>
struct StateIO<true> {
  using elem = uint16_t;
  static __device__ __forceinline__ float4 load(const uint16_t* p) {
    const u32x2v w = __builtin_nontemporal_load(reinterpret_cast<const u32x2v*>(p));
    return make_float4(bf16lo(w[0]), bf16hi(w[0]), bf16lo(w[1]), bf16hi(w[1]));
  }
  static __device__ __forceinline__ void store(uint16_t* p, float4 x) {
    u32x2v w;
    w[0] = (uint32_t)f32_to_bf16(x.x) | ((uint32_t)f32_to_bf16(x.y) << 16);
    w[1] = (uint32_t)f32_to_bf16(x.z) | ((uint32_t)f32_to_bf16(x.w) << 16);
    __builtin_nontemporal_store(w, reinterpret_cast<u32x2v*>(p));
  }
};

template <int COLS, bool BF16>
__global__ __launch_bounds__(kThreads) void decode_kernel(DecodeArgs a) {
  using IO = StateIO<BF16>;
  using elem = typename IO::elem;
  constexpr int TPR = COLS / 4;        // threads per state row
  constexpr int RG = kThreads / TPR;   // row groups
  constexpr int RPT = kHeadDim / RG;   // rows per thread
  constexpr int SLICES = kHeadDim / COLS;
  constexpr int RG_PER_WAVE = 64 / TPR;

  __shared__ float sq[kHeadDim], sk[kHeadDim], sd[kHeadDim];
  __shared__ float red[4][TPR][9];
  __shared__ float nrm[2][2];   // [wave][q, k] partial sums of squares

  const int H = a.num_heads;
  const int64_t item = blockIdx.x / SLICES;
  const int slice = blockIdx.x % SLICES;
  const int r = (int)(item / H), h = (int)(item % H);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int jq = tid % TPR, rg = tid / TPR;
  const int col0 = slice * COLS + jq * 4;
  const int64_t rh = (int64_t)r * H + h;

  const int64_t slot = a.slots[r];
  if (slot < 0 || slot >= a.num_slots) {  // skipped row: zero output, pool untouched
    if (tid < COLS) a.out[rh * kHeadDim + slice * COLS + tid] = 0;
    return;
  }
  elem* S = reinterpret_cast<elem*>(a.pool) + slot * a.slot_stride + h * (kHeadDim * kHeadDim);

  // Issue the state loads first; they are independent of q/k/g.
  float4 s[RPT];
#pragma unroll
  for (int i = 0; i < RPT; ++i) s[i] = IO::load(S + (rg + RG * i) * kHeadDim + col0);

  if (tid < kHeadDim) {
    const float qv = bf16_to_f32(a.q[rh * kHeadDim + tid]);
    const float kv = bf16_to_f32(a.k[rh * kHeadDim + tid]);
    const float gv = bf16_to_f32(a.g[rh * kHeadDim + tid]);
    sq[tid] = qv;
    sk[tid] = kv;
    float d;
    if (a.fe.gate_mode == 1)
      d = fast_exp2(a.fe.lower_bound * kLog2e / (1.f + fast_exp2(-gv * kLog2e)));
    else if (a.fe.gate_mode == 2)
      d = 1.f / (1.f + fast_exp2(gv * kLog2e));     // e^{-softplus(a)} = sigmoid(-a)
    else
      d = fast_exp2(gv * kLog2e);
    sd[tid] = d;
    if (a.fe.normalize_qk) {   // waves 0 and 1 hold the 128 channels
      float sq2 = qv * qv, sk2 = kv * kv;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        sq2 += __shfl_xor(sq2, off);
        sk2 += __shfl_xor(sk2, off);
      }
      if (lane == 0) {
        nrm[wave][0] = sq2;
        nrm[wave][1] = sk2;
      }
    }
  }
  __syncthreads();
  float rq = 1.f, rk = 1.f;
  if (a.fe.normalize_qk) {
    rq = inv_norm(nrm[0][0] + nrm[1][0] + a.fe.norm_eps);
    rk = inv_norm(nrm[0][1] + nrm[1][1] + a.fe.norm_eps);
  }

  float w[4] = {0.f, 0.f, 0.f, 0.f}, p[4] = {0.f, 0.f, 0.f, 0.f}, qk = 0.f;
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    const int c = rg + RG * i;
    const float d = sd[c], kc = sk[c], qc = sq[c];
    s[i].x *= d;
    s[i].y *= d;
    s[i].z *= d;
    s[i].w *= d;
    w[0] = fmaf(kc, s[i].x, w[0]);
    w[1] = fmaf(kc, s[i].y, w[1]);
    w[2] = fmaf(kc, s[i].z, w[2]);
    w[3] = fmaf(kc, s[i].w, w[3]);
    p[0] = fmaf(qc, s[i].x, p[0]);
    p[1] = fmaf(qc, s[i].y, p[1]);
    p[2] = fmaf(qc, s[i].z, p[2]);
    p[3] = fmaf(qc, s[i].w, p[3]);
    qk = fmaf(qc, kc, qk);
  }
  // Reduce over the row groups of this wave (lanes differing in rg bits).
#pragma unroll
  for (int off = TPR; off < 64; off <<= 1) {
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      w[m] += __shfl_xor(w[m], off);
      p[m] += __shfl_xor(p[m], off);
    }
    qk += __shfl_xor(qk, off);
  }
  if (lane < TPR) {
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      red[wave][jq][m] = w[m];
      red[wave][jq][4 + m] = p[m];
    }
    red[wave][jq][8] = qk;
  }
  __syncthreads();
#pragma unroll
  for (int m = 0; m < 9; ++m) {
    float acc = red[0][jq][m] + red[1][jq][m] + red[2][jq][m] + red[3][jq][m];
    if (m < 4)
      w[m] = acc;
    else if (m < 8)
      p[m - 4] = acc;
    else
      qk = acc;
  }
  (void)RG_PER_WAVE;
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    w[m] *= rk;
    p[m] *= rq;
  }
  qk *= rq * rk;

  float b = bf16_to_f32(a.beta[rh]);
  if (a.fe.beta_logits) b = 1.f / (1.f + fast_exp2(-b * kLog2e));
  const uint2 vw = *reinterpret_cast<const uint2*>(a.v + rh * kHeadDim + col0);
  float u[4];
  u[0] = b * (bf16lo(vw.x) - w[0]);
  u[1] = b * (bf16hi(vw.x) - w[1]);
  u[2] = b * (bf16lo(vw.y) - w[2]);
  u[3] = b * (bf16hi(vw.y) - w[3]);

  // the update adds k_n u^T = k (u / |k|)^T; the output keeps u
  const float uk[4] = {u[0] * rk, u[1] * rk, u[2] * rk, u[3] * rk};
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    const float kc = sk[rg + RG * i];
    s[i].x = fmaf(kc, uk[0], s[i].x);
    s[i].y = fmaf(kc, uk[1], s[i].y);
    s[i].z = fmaf(kc, uk[2], s[i].z);
    s[i].w = fmaf(kc, uk[3], s[i].w);
    IO::store(S + (rg + RG * i) * kHeadDim + col0, s[i]);
  }
  if (rg == 0) {
    uint2 ow;
    ow.x = (uint32_t)f32_to_bf16(a.scale * fmaf(qk, u[0], p[0])) |
           ((uint32_t)f32_to_bf16(a.scale * fmaf(qk, u[1], p[1])) << 16);
    ow.y = (uint32_t)f32_to_bf16(a.scale * fmaf(qk, u[2], p[2])) |
           ((uint32_t)f32_to_bf16(a.scale * fmaf(qk, u[3], p[3])) << 16);
    *reinterpret_cast<uint2*>(a.out + rh * kHeadDim + col0) = ow;
  }
}

template <bool BF16>
hipError_t launch_cols(const DecodeArgs& a, int cols, hipStream_t s) {
  const int64_t items = (int64_t)a.rows * a.num_heads;
  switch (cols) {
    case 128:
      decode_kernel<128, BF16><<<dim3((unsigned)(items * 1)), kThreads, 0, s>>>(a);
      break;
    case 64:
      decode_kernel<64, BF16><<<dim3((unsigned)(items * 2)), kThreads, 0, s>>>(a);
      break;
    case 32:
      decode_kernel<32, BF16><<<dim3((unsigned)(items * 4)), kThreads, 0, s>>>(a);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& a, bool bf16_state, int cols, hipStream_t s) {
  if (a.rows <= 0) return hipSuccess;
  return bf16_state ? launch_cols<true>(a, cols, s) : launch_cols<false>(a, cols, s);
}

}  // namespace kda
