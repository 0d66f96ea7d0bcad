// Two-pass chunk-32 KDA prefill for few (sequence, head) units on gfx950.
//
// When the number of (sequence, head) recurrences is small (one long
// sequence with 8 heads, say) a kernel that prepares each chunk inside the
// block that consumes it leaves almost the whole chip idle and puts the
// preparation on the serial path.  This route separates the two dependency
// domains of "FlashInfer PR #4262: CAKE KDA Prefill Highlights" (section 5:
// chunk-local preparation is parallel, state evolution is serial) across
// kernels instead of across warps:
//
//   pass 1 (prefill_split_prep): one wave per (chunk, head), all chunks of
//     all sequences at once.  Steps 1-3 of section 2 (gate prefix, anchored
//     Mqk/Akk, the 32x32 inverse T) and then everything that depends only on
//     the chunk:
//        U0 = T Diag(b) V          (what U would be from a zero state)
//        M  = T Diag(b) Kg         (how U depends on the incoming state)
//     so that U = U0 - M S0.  Results go to a workspace record per
//     (chunk, head), laid out in MFMA-fragment order and written straight
//     from registers.
//   pass 2 (prefill_split_chain): one block per (sequence, head, 16 value
//     columns) walks the chunks in order:
//        U  = U0 + (-M) S0                    (fp16 MFMA, FP32 accumulate)
//        S1 = Diag(2^{G_L}) S0 + Kr^T U       (U as hi + lo fp16)
//        O  = scale (Qg S0 + Mqk U)
//     i.e. the note's fused [S | O] update, with the state resident in the
//     accumulators of one wave while other waves compute O and stream the
//     records through an LDS ring.
//
// Workspace record of (chunk slot s, head h) at ((s * H + h) * kRecBytes):
//   [0, 8192)        -M    fp16 A fragments [mt 2][kstep 4][lane 64][8]
//   [8192, 16384)    Qg    fp16 A fragments [mt 2][kstep 4][lane 64][8]
//   [16384, 24576)   Kr^T  fp16 A fragments [mt 8][lane 64][8]
//   [24576, 26624)   Mqk   fp16 A fragments [mt 2][lane 64][8]
//   [26624, 27136)   2^{G_L} fp32 [128]
//   [27136, 28672)   padding, never written or used (the staged part is
//                    7 x 4 KiB: one 16-byte load per thread per 4 KiB)
//   [28672, 45056)   U0    fp32 accumulator tiles [nt 8][mt 2][lane 64][4]
// Fragment K indices use the permuted slot order of chunk_common.h.  The chunk
// slot of chunk c of sequence n is n + floor(cu[n] / 32) + c, unique and
// below N + T / 32 + 1.
#include <cmath>
#include <type_traits>

#include "chunk_common.h"

namespace kda {

constexpr int kRecOffMneg = 0;
constexpr int kRecOffQg = 8192;
constexpr int kRecOffKrT = 16384;
constexpr int kRecOffMqk = 24576;
constexpr int kRecOffDec = 26624;
constexpr int kRecStageBytes = 28672;
constexpr int kRecOffU0 = 28672;
constexpr int kRecBytes = 45056;

size_t split_workspace_bytes(int32_t num_seqs, int64_t total_tokens, int32_t num_heads) {
  const int64_t slots = (int64_t)num_seqs + total_tokens / 32 + 1;
  return (size_t)slots * (size_t)num_heads * (size_t)kRecBytes;
}

namespace {

using namespace chunk;

typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// Inclusive prefix sum over the 16 lanes of each DPP row (lane i of a row
// ends with the sum of lanes 0..i of that row).
__device__ __forceinline__ float row_scan16(float x) {
  auto shr = [](float v, auto ctrl) __attribute__((always_inline)) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
        0, __builtin_bit_cast(int, v), decltype(ctrl)::value, 0xF, 0xF, true));
  };
  x += shr(x, std::integral_constant<int, 0x111>{});   // row_shr:1
  x += shr(x, std::integral_constant<int, 0x112>{});   // row_shr:2
  x += shr(x, std::integral_constant<int, 0x114>{});   // row_shr:4
  x += shr(x, std::integral_constant<int, 0x118>{});   // row_shr:8
  return x;
}

__device__ __forceinline__ float bf16_elem(const u32x4& w, int j) {
  return (j & 1) ? bf16hi(w[j >> 1]) : bf16lo(w[j >> 1]);
}

// Preparation pass: one wave per (chunk slot, head), no block barrier beyond
// the wave's own, LDS only for the 32x32 triangular inverse.
//
// Lane (g4 = lane/16, l16 = lane%16) owns tokens l16 and l16+16 of the chunk
// and, for each 32-channel K step p, the channels whose fragment K-slots are
// 8g4..8g4+7 (32p + 4g4 + {0..3} and 32p + 16 + 4g4 + {0..3}).  In that layout
//  - the gate prefix over tokens is a scan across the 16 lanes of a row;
//  - q 2^G is already the Qg A fragment of the record;
//  - the pairwise products are taken transposed (column side as the A
//    operand), so the accumulators of Mqk^T are the Mqk A fragments;
//  - Kr, b Kg and V, whose products contract over tokens, are transposed by
//    an MFMA against a one-hot matrix (exact: one nonzero product per output);
//    the transposed b Kg then gives M^T = (b Kg)^T T^T whose accumulators are
//    the -M A fragments.
template <int MODE>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(2))) void prefill_split_prep(PrefillArgs a, float exp2C,
                                                          uint8_t* __restrict__ ws) {
  __shared__ __align__(16) float Al[CH][36];   // Diag(b) stril(Akk); rows 0..15 cols 16..31 hold A21 T11
  __shared__ __align__(16) float Tl[CH][36];   // (I + A)^{-1}, lower triangle
  __shared__ __align__(16) float bl[CH];
  const int H = a.num_heads, N = a.num_seqs, T = a.total_tokens;
  const int slot = blockIdx.x, h = blockIdx.y;
  const int lane = threadIdx.x, l16 = lane & 15, g4 = lane >> 4;
  const float C = a.anchor_log2;

  // Which (sequence, chunk) owns this slot: the largest n with
  // n + floor(cu[n] / 32) <= slot.
  int lo = 0, hi = N - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (mid + clamp_offset(a.cu_seqlens[mid], T) / CH <= slot) lo = mid; else hi = mid - 1;
  }
  const int n = lo;
  const int bos = clamp_offset(a.cu_seqlens[n], T);
  const int eos = max(bos, clamp_offset(a.cu_seqlens[n + 1], T));
  const int c = slot - (n + bos / CH);
  if (c < 0 || CH * c >= eos - bos) return;  // slot not used by any chunk
  const int t0 = bos + CH * c;
  const int L = min(CH, eos - t0);
  uint8_t* rec = ws + ((int64_t)slot * H + h) * kRecBytes;

  // Rows t >= L of a final partial chunk lie outside these ranges and read as zero.
  const int64_t base = ((int64_t)t0 * H + h) * D;
  const uint32_t rows_bytes = (uint32_t)(((L - 1) * H + 1) * D * 2);
  const __amdgpu_buffer_rsrc_t rq = make_buffer(a.q + base, rows_bytes);
  const __amdgpu_buffer_rsrc_t rk = make_buffer(a.k + base, rows_bytes);
  const __amdgpu_buffer_rsrc_t rg = make_buffer(a.g + base, rows_bytes);
  const __amdgpu_buffer_rsrc_t rv = make_buffer(a.v + base, rows_bytes);
  const __amdgpu_buffer_rsrc_t rb =
      make_buffer(a.beta + (int64_t)t0 * H + h, (uint32_t)(((L - 1) * H + 1) * 2));
  const uint32_t tok_bytes = (uint32_t)H * D * 2;
  const float beta[2] = {
      bf16_to_f32(__builtin_amdgcn_raw_buffer_load_b16(rb, (uint32_t)(l16 * H * 2), 0, 0)),
      bf16_to_f32(__builtin_amdgcn_raw_buffer_load_b16(rb, (uint32_t)((l16 + 16) * H * 2), 0, 0))};
  auto load8 = [&](__amdgpu_buffer_rsrc_t r, int hf, int p) __attribute__((always_inline)) {
    const uint32_t off = (uint32_t)(l16 + 16 * hf) * tok_bytes + (uint32_t)(32 * p + 4 * g4) * 2;
    const u32x2 x0 = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0));
    const u32x2 x1 = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, off + 32, 0, 0));
    return u32x4{x0[0], x0[1], x1[0], x1[1]};
  };

  // One-hot transposers.  E[e] selects, for output column l16, the K-slot of
  // channel 16e + l16 of a 32-channel step in K-slot order; Ev[e] the same
  // for natural column order (value rows).
  f16x8 E[2];
  bf16x8 Ev[2];
#pragma unroll
  for (int e = 0; e < 2; ++e)
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      E[e][j] = (_Float16)((j == l16 - 4 * g4 + 4 * e && l16 - 4 * g4 >= 0 && l16 - 4 * g4 < 4) ? 1.f : 0.f);
      Ev[e][j] = (__bf16)(j == 16 * e + l16 - 8 * g4 ? 1.f : 0.f);
    }
  const f32x4 z = {0.f, 0.f, 0.f, 0.f};

  f32x4 acc[6] = {z, z, z, z, z, z};   // Mqk^T tiles (0,0) (0,1) (1,1), Akk^T tiles likewise
  // (b Kg)^T A fragments per 16-channel tile (hi, lo) wait for T in the
  // record's -M and U0 areas, which are written last: each lane reads back
  // only what it wrote.
  uint8_t* const xh_park = rec + kRecOffMneg;
  uint8_t* const xl_park = rec + kRecOffU0;

#pragma unroll
  for (int p = 0; p < 4; ++p) {
    u32x4 qw[2], kw[2], gw[2];
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      qw[hf] = load8(rq, hf, p);
      kw[hf] = load8(rk, hf, p);
      gw[hf] = load8(rg, hf, p);
    }
    // gate prefix (log2 domain) of both halves, and G at tokens 15 and 31
    float G[2][8], G15[8], GL[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float s0 = row_scan16(bf16_elem(gw[0], j));
      const float b0 = __shfl(s0, 15, 16);
      const float s1 = row_scan16(bf16_elem(gw[1], j)) + b0;
      G[0][j] = s0 * kLog2e;
      G[1][j] = s1 * kLog2e;
      G15[j] = b0 * kLog2e;
      GL[j] = __shfl(s1, 15, 16) * kLog2e;
    }
    if (l16 == 0) {
      f32x4 d0, d1;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        d0[i] = fast_exp2(GL[i]);
        d1[i] = fast_exp2(GL[4 + i]);
      }
      *reinterpret_cast<f32x4*>(rec + kRecOffDec + (32 * p + 4 * g4) * 4) = d0;
      *reinterpret_cast<f32x4*>(rec + kRecOffDec + (32 * p + 16 + 4 * g4) * 4) = d1;
    }
    float EL[8];
    if (MODE == 0) {
#pragma unroll
      for (int j = 0; j < 8; ++j) EL[j] = fast_exp2(GL[j] - C);
    }
    // anchored operands: row side (qa, ka), column side (kb); "o" = off-diagonal tile
    bf16x8 qah[2], qal[2], kah[2], kal[2], kbh[2], kbl[2];
    bf16x8 qoh, qol, koh, kol, boh, bol;
    f16x8 Qg[2], Kr[2], Bh[2], Bl[2];
#pragma unroll
    for (int hf = 0; hf < 2; ++hf)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float qf = bf16_elem(qw[hf], j), kf = bf16_elem(kw[hf], j);
        const float Gv = G[hf][j];
        float ep, em, P, R, fo = 0.f;
        if (MODE == 0) {
          ep = fast_exp2(Gv - C);                 // 2^{G-C}, |exponent| <= 16|b|
          em = fast_exp2(C - Gv);
          P = ep * exp2C;                         // 2^G
          R = EL[j] * em;                         // 2^{G_L - G}
        } else {
          const float Ch = (hf ? G15[j] : 0.f) + a.half_anchor_log2;
          ep = fast_exp2(Gv - Ch);
          em = fast_exp2(Ch - Gv);
          fo = hf ? fast_exp2(Gv - G15[j]) : fast_exp2(G15[j] - Gv);   // both <= 1
          P = fast_exp2(Gv);
          R = fast_exp2(GL[j] - Gv);
        }
        __bf16 h1, l1, h2, l2, h3, l3;
        split_bf16(qf * ep, h1, l1);
        split_bf16(kf * ep, h2, l2);
        split_bf16(kf * em, h3, l3);
        qah[hf][j] = h1; qal[hf][j] = l1;
        kah[hf][j] = h2; kal[hf][j] = l2;
        kbh[hf][j] = h3; kbl[hf][j] = l3;
        if (MODE == 1) {
          if (hf == 1) {
            split_bf16(qf * fo, h1, l1);
            split_bf16(kf * fo, h2, l2);
            qoh[j] = h1; qol[j] = l1; koh[j] = h2; kol[j] = l2;
          } else {
            split_bf16(kf * fo, h3, l3);
            boh[j] = h3; bol[j] = l3;
          }
        }
        Qg[hf][j] = static_cast<_Float16>(qf * P);
        Kr[hf][j] = static_cast<_Float16>(kf * R);
        _Float16 xh, xl;
        split_f16(beta[hf] * (kf * P), xh, xl);
        Bh[hf][j] = xh;
        Bl[hf][j] = xl;
      }
    if (MODE == 0) {
      // one anchor for the whole chunk: the off-diagonal tile reuses the diagonal operands
      qoh = qah[1]; qol = qal[1]; koh = kah[1]; kol = kal[1]; boh = kbh[0]; bol = kbl[0];
    }
    // transposed pairwise products, split K over the four steps
    acc[0] = mfma_bf16(kbh[0], qah[0], acc[0]);
    acc[0] = mfma_bf16(kbh[0], qal[0], acc[0]);
    acc[0] = mfma_bf16(kbl[0], qah[0], acc[0]);
    acc[1] = mfma_bf16(boh, qoh, acc[1]);
    acc[1] = mfma_bf16(boh, qol, acc[1]);
    acc[1] = mfma_bf16(bol, qoh, acc[1]);
    acc[2] = mfma_bf16(kbh[1], qah[1], acc[2]);
    acc[2] = mfma_bf16(kbh[1], qal[1], acc[2]);
    acc[2] = mfma_bf16(kbl[1], qah[1], acc[2]);
    acc[3] = mfma_bf16(kbh[0], kah[0], acc[3]);
    acc[3] = mfma_bf16(kbh[0], kal[0], acc[3]);
    acc[3] = mfma_bf16(kbl[0], kah[0], acc[3]);
    acc[4] = mfma_bf16(boh, koh, acc[4]);
    acc[4] = mfma_bf16(boh, kol, acc[4]);
    acc[4] = mfma_bf16(bol, koh, acc[4]);
    acc[5] = mfma_bf16(kbh[1], kah[1], acc[5]);
    acc[5] = mfma_bf16(kbh[1], kal[1], acc[5]);
    acc[5] = mfma_bf16(kbl[1], kah[1], acc[5]);
    // Qg fragments go out as they are
#pragma unroll
    for (int hf = 0; hf < 2; ++hf)
      *reinterpret_cast<f16x8*>(rec + kRecOffQg + ((hf * 4 + p) * 64 + lane) * 16) = Qg[hf];
    // transposes of Kr (stored) and b Kg (kept for M)
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const f32x4 r0 = mfma_f16(Kr[0], E[e], z), r1 = mfma_f16(Kr[1], E[e], z);
      const f32x4 h0 = mfma_f16(Bh[0], E[e], z), h1 = mfma_f16(Bh[1], E[e], z);
      const f32x4 w0 = mfma_f16(Bl[0], E[e], z), w1 = mfma_f16(Bl[1], E[e], z);
      f16x8 kt, xh, xl;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        kt[i] = (_Float16)r0[i];  kt[4 + i] = (_Float16)r1[i];
        xh[i] = (_Float16)h0[i];  xh[4 + i] = (_Float16)h1[i];
        xl[i] = (_Float16)w0[i];  xl[4 + i] = (_Float16)w1[i];
      }
      *reinterpret_cast<f16x8*>(rec + kRecOffKrT + ((2 * p + e) * 64 + lane) * 16) = kt;
      *reinterpret_cast<f16x8*>(xh_park + ((2 * p + e) * 64 + lane) * 16) = xh;
      *reinterpret_cast<f16x8*>(xl_park + ((2 * p + e) * 64 + lane) * 16) = xl;
    }
    __builtin_amdgcn_sched_barrier(0);
  }

  // Mqk fragments straight from the Mqk^T accumulators (rows s = 16a + 4g4 + i,
  // column r = 16b + l16), causal mask by select; A = Diag(b) stril(Akk) to LDS.
  {
    f16x8 m0, m1;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int s = 4 * g4 + i;
      m0[i] = (_Float16)(s <= l16 ? acc[0][i] : 0.f);
      m0[4 + i] = (_Float16)0.f;
      m1[i] = (_Float16)acc[1][i];
      m1[4 + i] = (_Float16)(s <= l16 ? acc[2][i] : 0.f);
      Al[l16][s] = s < l16 ? beta[0] * acc[3][i] : 0.f;
      Al[16 + l16][s] = beta[1] * acc[4][i];
      Al[16 + l16][16 + s] = s < l16 ? beta[1] * acc[5][i] : 0.f;
    }
    *reinterpret_cast<f16x8*>(rec + kRecOffMqk + lane * 16) = m0;
    *reinterpret_cast<f16x8*>(rec + kRecOffMqk + (64 + lane) * 16) = m1;
    if (g4 == 0) {
      bl[l16] = beta[0];
      bl[16 + l16] = beta[1];
    }
  }
  // value rows for U0, consumed after the inverse
  u32x4 vw[4][2];
#pragma unroll
  for (int p = 0; p < 4; ++p)
#pragma unroll
    for (int hf = 0; hf < 2; ++hf)
      vw[p][hf] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
          rv, (uint32_t)(l16 + 16 * hf) * tok_bytes + (uint32_t)(32 * p + 8 * g4) * 2, 0, 0));
  __syncthreads();

  // T = (I + A)^{-1}: diagonal 16x16 blocks by forward substitution (lane m
  // of each half-wave owns column m), then T21 = -T22 (A21 T11).
  if (lane < 32) {
    const int b0 = 16 * (lane >> 4), m = lane & 15;
    float x[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) x[i] = i == m ? 1.f : 0.f;
#pragma unroll
    for (int j = 0; j < 16; ++j)
#pragma unroll
      for (int i = j + 1; i < 16; ++i) x[i] = fmaf(-Al[b0 + i][b0 + j], x[j], x[i]);
#pragma unroll
    for (int i = 0; i < 16; ++i) Tl[b0 + i][b0 + m] = x[i];
  }
  __syncthreads();
  {
    const int m = l16;
    float acc4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const float t = Tl[j][m];
#pragma unroll
      for (int i = 0; i < 4; ++i) acc4[i] = fmaf(Al[16 + 4 * g4 + i][j], t, acc4[i]);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) Al[4 * g4 + i][16 + m] = acc4[i];
  }
  __syncthreads();
  {
    const int m = l16;
    float acc4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const float xv = Al[j][16 + m];
#pragma unroll
      for (int i = 0; i < 4; ++i) acc4[i] = fmaf(Tl[16 + 4 * g4 + i][16 + j], xv, acc4[i]);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) Tl[16 + 4 * g4 + i][m] = -acc4[i];
  }
  __syncthreads();

  // T and T Diag(b) as fp16 hi / lo A fragments (row t = 16mt + l16, K-slot
  // 8g4 + j <-> token 4g4 + j or 16 + 4g4 + j - 4); T12 = 0.
  f16x8 th[2], tl[2], tbh[2], tbl[2];
  {
    const f32x4 bb0 = *reinterpret_cast<const f32x4*>(&bl[4 * g4]);
    const f32x4 bb1 = *reinterpret_cast<const f32x4*>(&bl[16 + 4 * g4]);
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      const f32x4 ta = *reinterpret_cast<const f32x4*>(&Tl[16 * mt + l16][4 * g4]);
      const f32x4 tb = mt ? *reinterpret_cast<const f32x4*>(&Tl[16 + l16][16 + 4 * g4]) : z;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float tv = j < 4 ? ta[j] : tb[j - 4];
        const float bv = j < 4 ? bb0[j] : bb1[j - 4];
        _Float16 hh, ll;
        split_f16(tv, hh, ll);
        th[mt][j] = hh; tl[mt][j] = ll;
        split_f16(tv * bv, hh, ll);
        tbh[mt][j] = hh; tbl[mt][j] = ll;
      }
    }
  }

  // Read the parked (b Kg)^T fragments back before their areas are overwritten
  // (all earlier stores have completed first).
  __builtin_amdgcn_s_waitcnt(0x0f70);   // vmcnt(0)
  f16x8 Xh[8], Xl[8];
#pragma unroll
  for (int mc = 0; mc < 8; ++mc) {
    Xh[mc] = *reinterpret_cast<const f16x8*>(xh_park + (mc * 64 + lane) * 16);
    Xl[mc] = *reinterpret_cast<const f16x8*>(xl_park + (mc * 64 + lane) * 16);
  }
  __builtin_amdgcn_s_waitcnt(0x0f70);   // vmcnt(0): the reads complete before any store below
  __builtin_amdgcn_sched_barrier(0);

  // U0 = T Diag(b) V per 16-column tile: V transposed by the one-hot product.
#pragma unroll
  for (int p = 0; p < 4; ++p)
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const f32x4 v0 = mfma_bf16(__builtin_bit_cast(bf16x8, vw[p][0]), Ev[e], z);
      const f32x4 v1 = mfma_bf16(__builtin_bit_cast(bf16x8, vw[p][1]), Ev[e], z);
      f16x8 vt;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        vt[i] = (_Float16)v0[i];
        vt[4 + i] = (_Float16)v1[i];
      }
      const int nt = 2 * p + e;
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        f32x4 u = mfma_f16(tbh[mt], vt, z);
        u = mfma_f16(tbl[mt], vt, u);
        *reinterpret_cast<f32x4*>(rec + kRecOffU0 + ((nt * 2 + mt) * 64 + lane) * 16) = u;
      }
    }

  // M^T = (b Kg)^T T^T: accumulator rows are channels 16mc + 4g4 + i, column
  // token 16tt + l16, i.e. the -M A fragments of K step mc/2.
#pragma unroll
  for (int p = 0; p < 4; ++p)
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      f16x8 mf;
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int mc = 2 * p + e;
        f32x4 m = mfma_f16(Xh[mc], th[tt], z);
        m = mfma_f16(Xh[mc], tl[tt], m);
        m = mfma_f16(Xl[mc], th[tt], m);
#pragma unroll
        for (int i = 0; i < 4; ++i) mf[4 * e + i] = (_Float16)(-m[i]);
      }
      *reinterpret_cast<f16x8*>(rec + kRecOffMneg + ((tt * 4 + p) * 64 + lane) * 16) = mf;
    }
}


// Chain pass.  One block per (sequence, head, 16-column value tile), four
// waves with fixed roles, one barrier per chunk step:
//   wave 0 (state):  the serial recurrence only -- U = U0 + (-M) S0, the decay
//                    and S += Kr^T U -- with the state in registers for the
//                    whole sequence; during step c it already reads chunk
//                    c+1's operands from LDS.  It hands fp16 S0 and U (hi, lo)
//                    of chunk c to the output wave through LDS.
//   wave 1 (output): in step c computes O = scale (Qg S0 + Mqk U) for chunk
//                    c-1 and stores it.
//   waves 2-3 (loaders): in step c copy chunk c+2's record into the LDS ring
//                    (from registers loaded three steps earlier) and start
//                    loading chunk c+5.
// LDS ring of 4 chunk slots: in step c the state wave reads slot c+1, the
// output wave slot c-1 and the loaders write slot c+2 (mod 4), all distinct.
// Loads and stores are buffer operations issued unconditionally (a chunk past
// the end has an empty range: loads return zeros, stores are dropped), so
// every path issues the same memory operations and the compiler's wait
// counts stay exact.  Value columns evolve independently, so tiles never
// communicate.  Block b handles (sequence, head) unit b % units and tile
// b / units: with a unit count divisible by 8, all tiles of a unit run on
// one XCD and share its L2 copy of the records.
constexpr int kChainStage = kRecStageBytes + 2048;        // staged record + one U0 tile
constexpr int kChainSlots = 4;
constexpr int kExchBytes = 6 * 64 * 16;                   // Sb[4], Uh, Ul fragments
constexpr int kChainLds = kChainSlots * kChainStage + 2 * kExchBytes;
constexpr int kLoaderVecs = kChainStage / 16 / 128;      // 15 x 16 B per loader lane
constexpr int kLoadAhead = 3;                             // chunks in loader registers
static_assert(kChainStage % (16 * 128) == 0, "stage must split evenly over two loader waves");

// Operands of one chunk step of the state wave.
struct MUOps {
  f16x8 am[2][4];   // -M fragments, [mt][kstep]
  f32x4 u0[2];      // U0 accumulator tiles
};
struct KDOps {
  f16x8 ak[8];      // Kr^T fragments
  f32x4 dv[8];      // 2^{G_L} of the lane's state rows
};

__global__ __launch_bounds__(256) void prefill_split_chain(PrefillArgs a,
                                                            const uint8_t* __restrict__ ws) {
  extern __shared__ __align__(16) unsigned char lds[];
  const int H = a.num_heads;
  const int units = a.num_seqs * H;
  const int unit = blockIdx.x % units, tile = blockIdx.x / units;
  const int n = unit / H, h = unit % H;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g4 = lane >> 4;
  const int col = 16 * tile + (lane & 15);

  const int bos = clamp_offset(a.cu_seqlens[n], a.total_tokens);
  const int eos = max(bos, clamp_offset(a.cu_seqlens[n + 1], a.total_tokens));
  const int nch = (eos - bos + CH - 1) / CH;
  const int64_t slot0 = (int64_t)n + bos / CH;

  auto slot = [&](int c) __attribute__((always_inline)) {
    return lds + (c & (kChainSlots - 1)) * kChainStage;
  };
  auto exch = [&](int c) __attribute__((always_inline)) {
    return lds + kChainSlots * kChainStage + (c & 1) * kExchBytes;
  };

  if (wave >= 2) {
    // ------------------------------------------------------------ loaders
    const int lt = tid - 128;
    auto load = [&](u32x4* dst, int c) __attribute__((always_inline)) {
      const __amdgpu_buffer_rsrc_t r = make_buffer(
          ws + ((slot0 + c) * H + h) * kRecBytes, c < nch ? (uint32_t)kRecBytes : 0u);
#pragma unroll
      for (int m = 0; m < kLoaderVecs; ++m) {
        const int v = lt + 128 * m;
        const int off = v < kRecStageBytes / 16 ? v * 16
                                                : kRecOffU0 + tile * 2048 + (v - kRecStageBytes / 16) * 16;
        dst[m] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (uint32_t)off, 0, 0));
      }
    };
    auto store = [&](const u32x4* src, int c) __attribute__((always_inline)) {
#pragma unroll
      for (int m = 0; m < kLoaderVecs; ++m)
        reinterpret_cast<u32x4*>(slot(c))[lt + 128 * m] = src[m];
    };
    u32x4 buf[kLoadAhead][kLoaderVecs];
    load(buf[0], 0);
    store(buf[0], 0);
    load(buf[0], 1);
    store(buf[0], 1);
#pragma unroll
    for (int i = 0; i < kLoadAhead; ++i) load(buf[i], 2 + i);
    __syncthreads();
    auto step = [&](auto I_const, int c) __attribute__((always_inline)) {
      constexpr int I = decltype(I_const)::value;
      store(buf[I], c + 2);               // loaded three steps ago
      load(buf[I], c + 2 + kLoadAhead);
      __syncthreads();
    };
    for (int c = 0; c <= nch; c += kLoadAhead) {
      step(std::integral_constant<int, 0>{}, c);
      if (c + 1 > nch) break;
      step(std::integral_constant<int, 1>{}, c + 1);
      if (c + 2 > nch) break;
      step(std::integral_constant<int, 2>{}, c + 2);
    }
    return;
  }

  if (wave == 1) {
    // ------------------------------------------------------------- output
    __syncthreads();
    for (int c = 0; c <= nch; ++c) {
      if (c >= 1) {
        const int cp = c - 1;
        const uint8_t* st = slot(cp);
        const uint8_t* ex = exch(cp);
        f16x8 aq[2][4], amq[2], sb[4], uh, ul;
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
          for (int p = 0; p < 4; ++p)
            aq[mt][p] = *reinterpret_cast<const f16x8*>(st + kRecOffQg + ((mt * 4 + p) * 64 + lane) * 16);
          amq[mt] = *reinterpret_cast<const f16x8*>(st + kRecOffMqk + (mt * 64 + lane) * 16);
        }
#pragma unroll
        for (int p = 0; p < 4; ++p) sb[p] = *reinterpret_cast<const f16x8*>(ex + (p * 64 + lane) * 16);
        uh = *reinterpret_cast<const f16x8*>(ex + (4 * 64 + lane) * 16);
        ul = *reinterpret_cast<const f16x8*>(ex + (5 * 64 + lane) * 16);
        const f32x4 z = {0.f, 0.f, 0.f, 0.f};
        f32x4 O[2] = {z, z};
#pragma unroll
        for (int p = 0; p < 4; ++p)
#pragma unroll
          for (int mt = 0; mt < 2; ++mt) O[mt] = mfma_f16(aq[mt][p], sb[p], O[mt]);
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
          O[mt] = mfma_f16(amq[mt], uh, O[mt]);
          O[mt] = mfma_f16(amq[mt], ul, O[mt]);
        }
        // rows t >= L of a final partial chunk fall outside the range and are dropped
        const int t0 = bos + CH * cp;
        const int L = min(CH, eos - t0);
        const __amdgpu_buffer_rsrc_t orsrc = make_buffer(
            a.out + ((int64_t)t0 * H + h) * D, (uint32_t)(((L - 1) * H + 1) * D * 2));
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
          for (int i2 = 0; i2 < 4; ++i2) {
            const int t = 16 * mt + 4 * g4 + i2;
            buffer_store_u16(f32_to_bf16(a.scale * O[mt][i2]), orsrc,
                             (uint32_t)((t * H * D + col) * 2));
          }
      }
      __syncthreads();
    }
    return;
  }

  // --------------------------------------------------------------- state
  const int64_t sbase = ((int64_t)n * H + h) * D * D;
  f32x4 S[8];
  if (a.s0) {
#pragma unroll
    for (int mt = 0; mt < 8; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) S[mt][i] = a.s0[sbase + (int64_t)(16 * mt + 4 * g4 + i) * D + col];
  } else {
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) S[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  // All operands of a chunk step come from its ring slot, read early enough
  // that a step never waits on LDS: Kr^T and the decay of chunk c+1 at the
  // start of step c (double-buffered), -M and U0 of chunk c+1 as soon as the
  // U products of step c have consumed those of chunk c.
  auto read_mu = [&](MUOps& F, int c) __attribute__((always_inline)) {
    const uint8_t* st = slot(c);
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
      for (int p = 0; p < 4; ++p)
        F.am[mt][p] = *reinterpret_cast<const f16x8*>(st + kRecOffMneg + ((mt * 4 + p) * 64 + lane) * 16);
      F.u0[mt] = *reinterpret_cast<const f32x4*>(st + kRecStageBytes + (mt * 64 + lane) * 16);
    }
  };
  auto read_kd = [&](KDOps& K, int c) __attribute__((always_inline)) {
    const uint8_t* st = slot(c);
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) {
      K.ak[mt] = *reinterpret_cast<const f16x8*>(st + kRecOffKrT + (mt * 64 + lane) * 16);
      K.dv[mt] = *reinterpret_cast<const f32x4*>(st + kRecOffDec + (16 * mt + 4 * g4) * 4);
    }
  };
  MUOps F;
  KDOps K[2];
  __syncthreads();
  read_mu(F, 0);
  read_kd(K[0], 0);
  auto step = [&](auto I_const, int c) __attribute__((always_inline)) {
    constexpr int I = decltype(I_const)::value;
    if (c < nch) {
      read_kd(K[1 - I], c + 1);           // unused past the end
      const KDOps& k = K[I];
      f16x8 Sb[4];
#pragma unroll
      for (int p = 0; p < 4; ++p)
#pragma unroll
        for (int i2 = 0; i2 < 4; ++i2) {
          Sb[p][i2] = static_cast<_Float16>(S[2 * p][i2]);
          Sb[p][4 + i2] = static_cast<_Float16>(S[2 * p + 1][i2]);
        }
      f32x4 U[2] = {F.u0[0], F.u0[1]};
#pragma unroll
      for (int p = 0; p < 4; ++p)
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) U[mt] = mfma_f16(F.am[mt][p], Sb[p], U[mt]);
      read_mu(F, c + 1);                  // unused past the end
      // the decay does not depend on U: it fills the MFMA latency
#pragma unroll
      for (int mt = 0; mt < 8; ++mt)
#pragma unroll
        for (int i2 = 0; i2 < 4; ++i2) S[mt][i2] *= k.dv[mt][i2];
      uint8_t* ex = exch(c);
#pragma unroll
      for (int p = 0; p < 4; ++p) *reinterpret_cast<f16x8*>(ex + (p * 64 + lane) * 16) = Sb[p];
      f16x8 Uh, Ul;
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int i2 = 0; i2 < 4; ++i2) {
          _Float16 hh, ll;
          split_f16(U[mt][i2], hh, ll);
          Uh[4 * mt + i2] = hh;
          Ul[4 * mt + i2] = ll;
        }
#pragma unroll
      for (int mt = 0; mt < 8; ++mt) {
        S[mt] = mfma_f16(k.ak[mt], Uh, S[mt]);
        S[mt] = mfma_f16(k.ak[mt], Ul, S[mt]);
      }
      *reinterpret_cast<f16x8*>(ex + (4 * 64 + lane) * 16) = Uh;
      *reinterpret_cast<f16x8*>(ex + (5 * 64 + lane) * 16) = Ul;
    }
    __syncthreads();
  };
  for (int c = 0; c <= nch; c += 2) {
    step(std::integral_constant<int, 0>{}, c);
    if (c + 1 > nch) break;
    step(std::integral_constant<int, 1>{}, c + 1);
  }
  if (a.s1) {
#pragma unroll
    for (int mt = 0; mt < 8; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        a.s1[sbase + (int64_t)(16 * mt + 4 * g4 + i) * D + col] = S[mt][i];
  }
}

template <int MODE>
hipError_t launch_prep(const PrefillArgs& a, uint8_t* ws, hipStream_t s) {
  const float exp2C = MODE == 0 ? std::exp2(a.anchor_log2) : 0.f;
  const int64_t slots = (int64_t)a.num_seqs + a.total_tokens / CH + 1;
  prefill_split_prep<MODE><<<dim3((unsigned)slots, a.num_heads), 64, 0, s>>>(a, exp2C, ws);
  return hipGetLastError();
}

hipError_t launch_chain(const PrefillArgs& a, const uint8_t* ws, hipStream_t s) {
  static bool attr_set = false;   // idempotent; a race only repeats the call
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&prefill_split_chain),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, kChainLds);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  const int64_t blocks = (int64_t)a.num_seqs * a.num_heads * 8;
  prefill_split_chain<<<dim3((unsigned)blocks), 256, kChainLds, s>>>(a, ws);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill_split_prepare(const PrefillArgs& a, int anchor_mode, void* workspace,
                                        hipStream_t s) {
  if (a.num_seqs <= 0) return hipSuccess;
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  return anchor_mode == 0 ? launch_prep<0>(a, ws, s) : launch_prep<1>(a, ws, s);
}

hipError_t launch_prefill_split_chain(const PrefillArgs& a, const void* workspace,
                                      hipStream_t s) {
  if (a.num_seqs <= 0) return hipSuccess;
  return launch_chain(a, static_cast<const uint8_t*>(workspace), s);
}

hipError_t launch_prefill_split(const PrefillArgs& a, int anchor_mode, int dv_split,
                                void* workspace, hipStream_t s) {
  if (dv_split != 8) return hipErrorInvalidValue;   // one 16-column tile per chain block
  hipError_t e = launch_prefill_split_prepare(a, anchor_mode, workspace, s);
  if (e != hipSuccess) return e;
  return launch_prefill_split_chain(a, workspace, s);
}

}  // namespace kda
