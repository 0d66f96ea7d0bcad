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
//     all sequences at once (four consecutive chunks of a head per block).  Steps 1-3 of section 2 (gate prefix, anchored
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
//   [0, 8192)        -M'   fp16 A fragments [mt 2][kstep 4][lane 64][8]
//   [8192, 16384)    Qg    fp16 A fragments [mt 2][kstep 4][lane 64][8]
//   [16384, 24576)   Kr^T  fp16 A fragments [mt 8][lane 64][8]
//   [24576, 26624)   Mqk   fp16 A fragments [mt 2][lane 64][8]
//   [26624, 27136)   2^{G_L} fp32 [128]
//   [27136, 28672)   padding, never written or used
//   [28672, 30720)   -W    fp16 A fragments, hi part [mt 2][lane 64][8]
//   [30720, 32768)   -W    lo part (the staged part is 8 x 4 KiB)
//   [32768, 49152)   U0    fp32 accumulator tiles [nt 8][mt 2][lane 64][4]
// where, for chunk c of a sequence, M' = M Diag(2^{G_L}) and W = M Kr^T with
// the decay and restored keys of chunk c-1 (chunk 0: M' = M, W = 0).  They
// let the chain form U of chunk c from the state and U of chunk c-1:
//   S_c = Diag(2^{G_L,c-1}) S_{c-1} + Kr_{c-1}^T U_{c-1},  U_c = U0_c - M_c S_c
//   =>  U_c = U0_c - M'_c S_{c-1} - W_c U_{c-1},
// so the serial dependency from one chunk to the next is the 32-deep W U
// product instead of the 128-deep M S product behind a state update.
// Fragment K indices use the permuted slot order of chunk_common.h.  The chunk
// slot of chunk c of sequence n is n + floor(cu[n] / 32) + c, unique and
// below N + T / 32 + 1.
#include <climits>
#include <cmath>
#include <type_traits>

#include "chunk_common.h"

namespace kda {

constexpr int kRecOffMneg = 0;
constexpr int kRecOffQg = 8192;
constexpr int kRecOffKrT = 16384;
constexpr int kRecOffMqk = 24576;
constexpr int kRecOffDec = 26624;
constexpr int kRecOffWh = 28672;
constexpr int kRecOffWl = 30720;
constexpr int kRecStageBytes = 32768;
constexpr int kRecOffU0 = 32768;
constexpr int kRecBytes = 49152;
// Waves per preparation block: consecutive chunks of one head, so that all
// but the first take the previous chunk's restored keys and decays from its
// record instead of re-reading and re-deriving them.
constexpr int kPrepWaves = 4;

// Window states after the records: per (sequence, head, window) the end
// state E (zero-state end for windows >= 1, true end for window 0), the map
// P and the true initial state SI, 64 KiB each.
constexpr int64_t kStateBytes = 128 * 128 * 4;

size_t split_records_bytes(int32_t num_seqs, int64_t total_tokens, int32_t num_heads) {
  const int64_t slots = (int64_t)num_seqs + total_tokens / 32 + 1;
  return (size_t)slots * (size_t)num_heads * (size_t)kRecBytes;
}

size_t split_workspace_bytes(int32_t num_seqs, int64_t total_tokens, int32_t num_heads,
                             int32_t windows) {
  size_t b = split_records_bytes(num_seqs, total_tokens, num_heads);
  if (windows > 1) b += (size_t)num_seqs * num_heads * windows * 2 * kStateBytes;
  return b;
}

namespace {

using namespace chunk;

// Chunks per window of a sequence of `nch` chunks when the chains are cut
// into a.windows windows (0 when they are not): at least kMinWindowChunks,
// and at most a.windows windows per sequence, whatever the other sequences'
// lengths (each sequence is cut by its own length, which only the device
// knows).
constexpr int kMinWindowChunks = 8;
__device__ __forceinline__ int window_chunks_of(const PrefillArgs& a, int nch) {
  return a.windows <= 1 ? 0 : max(kMinWindowChunks, (nch + a.windows - 1) / a.windows);
}

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

// Preparation pass: one wave per (chunk slot, head), four consecutive slots
// of one head per block with one block barrier (the hand-over of each chunk's
// predecessor, below); LDS for the 32x32 triangular inverse and that hand-over.
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
template <int MODE, bool FE>
__global__ __launch_bounds__(64 * kPrepWaves) __attribute__((amdgpu_waves_per_eu(2))) void prefill_split_prep(PrefillArgs a, float exp2C,
                                                          uint8_t* __restrict__ ws) {
  // Per wave: (b Kg)^T hi fragments [0, 8) and lo fragments [8, 16), parked
  // until T is known; once they are back in registers the same bytes hold
  // the FP32 system and its inverse, so eight waves per compute unit still fit.
  __shared__ __align__(16) f16x8 park_all[kPrepWaves][16][64];
  __shared__ __align__(16) float bl_all[kPrepWaves][CH];
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform
  f16x8 (*const park)[64] = park_all[wv];
  float* const bl = bl_all[wv];
  float (*const Al)[36] = reinterpret_cast<float (*)[36]>(&park[0][0]);  // Diag(b) stril(Akk); rows 0..15 cols 16..31 hold A21 T11
  float (*const Tl)[36] = Al + CH;                                        // (I + A)^{-1}, lower triangle
  const int H = a.num_heads, N = a.num_seqs, T = a.total_tokens;
  // Work items are (head, chunk slot), head-major; a block's kPrepWaves waves
  // take consecutive slots of one head (the slots of a head padded to a
  // multiple of kPrepWaves), so the waves after the first find the previous
  // chunk's record in their own block.  XCD-aware order: consecutive block
  // indices go to the eight XCDs in turn, so block b takes group (b % 8) *
  // per + b / 8, and each XCD walks a contiguous run of chunks of one head
  // (the re-read of the previous block's last chunk can hit its L2).
  const int64_t slots = (int64_t)N + T / CH + 1;
  const int64_t slots_pad = (slots + kPrepWaves - 1) / kPrepWaves * kPrepWaves;
  const int64_t groups = slots_pad / kPrepWaves * H;
  const int64_t per = (groups + 7) / 8;
  const int64_t grp = (int64_t)(blockIdx.x & 7) * per + (blockIdx.x >> 3);
  const int64_t item = grp * kPrepWaves + wv;
  const int lane = threadIdx.x & 63, l16 = lane & 15, g4 = lane >> 4;
  // Every wave passes the block's one barrier exactly once, working or not.
  if (grp >= groups) {
    __syncthreads();
    return;
  }
  // The block's first chunk takes its predecessor's restored keys and decays
  // from the four waves together: wave w derives K step w (32 channels) of
  // them from that chunk's keys and gates into LDS before the barrier (not
  // with the front-end's key norm, which needs all channels: the first wave
  // then re-derives them alone).
  static_assert(kPrepWaves == 4, "one K step of the shared predecessor per wave");
  __shared__ __align__(16) f16x8 prev_kr[kPrepWaves][2][64];   // [K step][token half][lane]
  __shared__ __align__(16) float prev_dec[D];
  bool share = false;
  {
    const int64_t item0 = grp * kPrepWaves;
    const int slot0 = (int)(item0 % slots_pad), h0 = (int)(item0 / slots_pad);
    if (slot0 < slots) {
      int lo = 0, hi = N - 1;
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (mid + clamp_offset(a.cu_seqlens[mid], T) / CH <= slot0) lo = mid; else hi = mid - 1;
      }
      const int bos0 = clamp_offset(a.cu_seqlens[lo], T);
      const int len0 = max(bos0, clamp_offset(a.cu_seqlens[lo + 1], T)) - bos0;
      const int c0 = slot0 - (lo + bos0 / CH);
      const int wcn0 = window_chunks_of(a, (len0 + CH - 1) / CH);
      share = c0 > 0 && CH * c0 < len0 && (wcn0 <= 0 || c0 % wcn0 != 0) &&
              !(FE && a.fe.normalize_qk);
      if (share) {
        const __amdgpu_buffer_rsrc_t rk0 = make_buffer(
            a.k + ((int64_t)(bos0 + CH * (c0 - 1)) * H + h0) * D, (uint32_t)(((CH - 1) * H + 1) * D * 2));
        const __amdgpu_buffer_rsrc_t rg0 = make_buffer(
            a.g + ((int64_t)(bos0 + CH * (c0 - 1)) * H + h0) * D, (uint32_t)(((CH - 1) * H + 1) * D * 2));
        const uint32_t tb = (uint32_t)H * D * 2;
        u32x4 kq[2], gq[2];
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
          const uint32_t off = (uint32_t)(l16 + 16 * hf) * tb + (uint32_t)(32 * wv + 4 * g4) * 2;
          const u32x2 k0 = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rk0, off, 0, 0));
          const u32x2 k1 = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rk0, off + 32, 0, 0));
          const u32x2 q0 = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rg0, off, 0, 0));
          const u32x2 q1 = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rg0, off + 32, 0, 0));
          kq[hf] = u32x4{k0[0], k0[1], k1[0], k1[1]};
          gq[hf] = u32x4{q0[0], q0[1], q1[0], q1[1]};
        }
        f16x8 kr0, kr1;
        f32x4 d0, d1;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          float x0 = bf16_elem(gq[0], j), x1 = bf16_elem(gq[1], j);
          if (FE) {
            x0 = frontend_gate(a.fe, x0);
            x1 = frontend_gate(a.fe, x1);
          }
          const float s0 = row_scan16(x0);
          const float b0 = __shfl(s0, 15, 16);
          const float s1 = row_scan16(x1) + b0;
          const float gl = __shfl(s1, 15, 16) * kLog2e;
          const float dv = fast_exp2(gl);
          if (j < 4) d0[j] = dv; else d1[j - 4] = dv;
          kr0[j] = static_cast<_Float16>(bf16_elem(kq[0], j) * fast_exp2(gl - s0 * kLog2e));
          kr1[j] = static_cast<_Float16>(bf16_elem(kq[1], j) * fast_exp2(gl - s1 * kLog2e));
        }
        prev_kr[wv][0][lane] = kr0;
        prev_kr[wv][1][lane] = kr1;
        if (l16 == 0) {
          *reinterpret_cast<f32x4*>(&prev_dec[32 * wv + 4 * g4]) = d0;
          *reinterpret_cast<f32x4*>(&prev_dec[32 * wv + 16 + 4 * g4]) = d1;
        }
      }
    }
  }
  if (item % slots_pad >= slots) {
    __syncthreads();
    return;
  }
  const int h = (int)(item / slots_pad), slot = (int)(item % slots_pad);
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
  if (c < 0 || CH * c >= eos - bos) {   // slot not used by any chunk
    __syncthreads();
    return;
  }
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
  // The previous chunk of the same sequence (chunk 0, and the first chunk of
  // a window: an empty range, so its keys and gates read as zero, which
  // gives W = 0 and M' = M and lets a chain start there).
  // A wave after the block's first takes the previous chunk's restored keys
  // and decays from that chunk's record, written by the wave before it in
  // this block (`hand`); otherwise it re-reads that chunk's keys and gates.
  const int wcn = window_chunks_of(a, (eos - bos + CH - 1) / CH);
  const bool has_prev = c > 0 && (wcn <= 0 || c % wcn != 0);
  const bool hand = has_prev && wv > 0;
  const bool shared_prev = share && wv == 0;   // then has_prev too
  const int64_t base_prev = has_prev ? base - (int64_t)CH * H * D : base;
  const uint32_t prev_bytes =
      has_prev && !hand && !shared_prev ? (uint32_t)(((CH - 1) * H + 1) * D * 2) : 0u;
  const __amdgpu_buffer_rsrc_t rkp = make_buffer(a.k + base_prev, prev_bytes);
  const __amdgpu_buffer_rsrc_t rgp = make_buffer(a.g + base_prev, prev_bytes);
  const uint32_t tok_bytes = (uint32_t)H * D * 2;
  // Tokens past the sequence end (a final partial chunk) read as zero; their
  // transformed gate and beta are forced to zero as well.
  const bool live[2] = {l16 < L, l16 + 16 < L};
  float beta[2] = {
      bf16_to_f32(__builtin_amdgcn_raw_buffer_load_b16(rb, (uint32_t)(l16 * H * 2), 0, 0)),
      bf16_to_f32(__builtin_amdgcn_raw_buffer_load_b16(rb, (uint32_t)((l16 + 16) * H * 2), 0, 0))};
  if (FE) {
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) beta[hf] = live[hf] ? frontend_beta(a.fe, beta[hf]) : 0.f;
  }
  // the gate tensor's value x of a live token as the log-decay (no transform
  // without the front-end, where a padding token's zero is already exact)
  auto gate = [&](float x, bool ok) __attribute__((always_inline)) {
    return FE ? (ok ? frontend_gate(a.fe, x) : 0.f) : x;
  };
  auto load8 = [&](__amdgpu_buffer_rsrc_t r, int hf, int p) __attribute__((always_inline)) {
    const uint32_t off = (uint32_t)(l16 + 16 * hf) * tok_bytes + (uint32_t)(32 * p + 4 * g4) * 2;
    const u32x2 x0 = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0));
    const u32x2 x1 = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, off + 32, 0, 0));
    return u32x4{x0[0], x0[1], x1[0], x1[1]};
  };
  // Input front-end q/k L2 norm: 1 / sqrt(sum x^2 + eps) of this lane's two
  // tokens (a pass over the chunk's q and k before the main loop; the four
  // lanes g4 of a token hold its 128 channels).
  float nq[2] = {1.f, 1.f}, nk[2] = {1.f, 1.f};
  if (FE && a.fe.normalize_qk) {
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      float s2q = 0.f, s2k = 0.f;
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const u32x4 qw = load8(rq, hf, p), kw = load8(rk, hf, p);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float qv = bf16_elem(qw, j), kv = bf16_elem(kw, j);
          s2q = fmaf(qv, qv, s2q);
          s2k = fmaf(kv, kv, s2k);
        }
      }
      s2q += __shfl_xor(s2q, 16);
      s2q += __shfl_xor(s2q, 32);
      s2k += __shfl_xor(s2k, 16);
      s2k += __shfl_xor(s2k, 32);
      nq[hf] = inv_norm(s2q + a.fe.norm_eps);
      nk[hf] = inv_norm(s2k + a.fe.norm_eps);
    }
  }

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
  // (b Kg)^T A fragments per 16-channel tile wait for T in LDS (park).

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
    float G[2][8], G15[8], GL[8], Gf[2][8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float s0 = row_scan16(gate(bf16_elem(gw[0], j), live[0]));
      const float b0 = __shfl(s0, 15, 16);
      const float s1 = row_scan16(gate(bf16_elem(gw[1], j), live[1])) + b0;
      G[0][j] = s0 * kLog2e;
      G[1][j] = s1 * kLog2e;
      G15[j] = b0 * kLog2e;
      GL[j] = __shfl(s1, 15, 16) * kLog2e;
      if (MODE == 2) {   // G at the first token of each half
        Gf[0][j] = __shfl(s0, 0, 16) * kLog2e;
        Gf[1][j] = __shfl(s1, 0, 16) * kLog2e;
      }
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
        const float qf = nq[hf] * bf16_elem(qw[hf], j), kf = nk[hf] * bf16_elem(kw[hf], j);
        const float Gv = G[hf][j];
        float ep, em, P, R, fo = 0.f;
        if (MODE == 0) {
          ep = fast_exp2(Gv - C);                 // 2^{G-C}, |exponent| <= 16|b|
          em = fast_exp2(C - Gv);
          P = ep * exp2C;                         // 2^G
          R = EL[j] * em;                         // 2^{G_L - G}
        } else {
          if (MODE == 1) {
            const float Ch = (hf ? G15[j] : 0.f) + a.half_anchor_log2;
            ep = fast_exp2(Gv - Ch);
            em = fast_exp2(Ch - Gv);
          } else {
            // midpoint of this half's actual range; exponents clamped so that
            // a half that decays a channel past 2^-252 stays finite
            const float Ch = 0.5f * (Gf[hf][j] + (hf ? GL[j] : G15[j]));
            ep = fast_exp2(__builtin_fminf(Gv - Ch, 126.f));
            em = fast_exp2(__builtin_fminf(Ch - Gv, 126.f));
          }
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
        if (MODE >= 1) {
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
    auto mfma3 = [&](const bf16x8& ah, const bf16x8& al, const bf16x8& bh, const bf16x8& bl,
                     f32x4 c) __attribute__((always_inline)) {
      c = mfma_bf16(ah, bh, c);
      c = mfma_bf16(ah, bl, c);
      return mfma_bf16(al, bh, c);
    };
    acc[1] = mfma3(boh, bol, qoh, qol, acc[1]);
    acc[4] = mfma3(boh, bol, koh, kol, acc[4]);
    // Unbounded gates: a 16-token half whose prefix falls by more than
    // kSteepRange in some channel of this K step cannot take one anchor, so
    // its diagonal tile is formed from the 8-token quarters Q0 (tokens 0-7 of
    // the half) and Q1 (8-15): Q0 x Q0 and Q1 x Q1 anchored at their own
    // midpoints, Q1 x Q0 through the prefix at their boundary (factors <= 1);
    // exact to the usual rounding while no quarter falls by more than 2^232.
    // The lane of token l16 supplies row and column l16 of a tile, so its
    // quarter decides which products it takes part in.
    bool steep = false;
    if (MODE == 2) {
#pragma unroll
      for (int j = 0; j < 8; ++j)
        steep |= (Gf[0][j] - G15[j] > kSteepRange) || (Gf[1][j] - GL[j] > kSteepRange);
      steep = __builtin_amdgcn_ballot_w64(steep) != 0;
    }
    if (MODE == 2 && steep) {
      const bool q1 = l16 >= 8;
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        // the prefix at the quarter boundaries of this half (tokens 16hf + 7, + 8, + 15)
        float G7[8], G8[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          G7[j] = __shfl(G[hf][j], 7, 16);
          G8[j] = __shfl(G[hf][j], 8, 16);
        }
        const int im = hf ? 2 : 0, ia = hf ? 5 : 3;
#pragma unroll
        for (int qq = 0; qq < 2; ++qq) {
          const bool mine = q1 == (qq == 1);
          bf16x8 ah, al, bh, bl, ch, cl;   // row side q, row side k, column side k
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const float Ca = qq ? 0.5f * (G8[j] + (hf ? GL[j] : G15[j])) : 0.5f * (Gf[hf][j] + G7[j]);
            const float rowA = mine ? fast_exp2(G[hf][j] - Ca) : 0.f;
            const float colA = mine ? fast_exp2(Ca - G[hf][j]) : 0.f;
            const float qf = nq[hf] * bf16_elem(qw[hf], j), kf = nk[hf] * bf16_elem(kw[hf], j);
            __bf16 h1, l1;
            split_bf16(qf * rowA, h1, l1); ah[j] = h1; al[j] = l1;
            split_bf16(kf * rowA, h1, l1); bh[j] = h1; bl[j] = l1;
            split_bf16(kf * colA, h1, l1); ch[j] = h1; cl[j] = l1;
          }
          acc[im] = mfma3(ch, cl, ah, al, acc[im]);
          acc[ia] = mfma3(ch, cl, bh, bl, acc[ia]);
        }
        {
          bf16x8 ah, al, bh, bl, ch, cl;   // rows of Q1 (q, k), columns of Q0 (k)
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const float e3 = fast_exp2(q1 ? G[hf][j] - G7[j] : G7[j] - G[hf][j]);   // <= 1
            const float qf = nq[hf] * bf16_elem(qw[hf], j), kf = nk[hf] * bf16_elem(kw[hf], j);
            __bf16 h1, l1;
            split_bf16(q1 ? qf * e3 : 0.f, h1, l1); ah[j] = h1; al[j] = l1;
            split_bf16(q1 ? kf * e3 : 0.f, h1, l1); bh[j] = h1; bl[j] = l1;
            split_bf16(q1 ? 0.f : kf * e3, h1, l1); ch[j] = h1; cl[j] = l1;
          }
          acc[im] = mfma3(ch, cl, ah, al, acc[im]);
          acc[ia] = mfma3(ch, cl, bh, bl, acc[ia]);
        }
      }
    } else {
      acc[0] = mfma3(kbh[0], kbl[0], qah[0], qal[0], acc[0]);
      acc[2] = mfma3(kbh[1], kbl[1], qah[1], qal[1], acc[2]);
      acc[3] = mfma3(kbh[0], kbl[0], kah[0], kal[0], acc[3]);
      acc[5] = mfma3(kbh[1], kbl[1], kah[1], kal[1], acc[5]);
    }
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
      park[2 * p + e][lane] = xh;
      park[8 + 2 * p + e][lane] = xl;
    }
    __builtin_amdgcn_sched_barrier(0);
  }

  // Mqk fragments straight from the Mqk^T accumulators (rows s = 16a + 4g4 + i,
  // column r = 16b + l16), causal mask by select.
  {
    f16x8 m0, m1;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int s = 4 * g4 + i;
      m0[i] = (_Float16)(s <= l16 ? acc[0][i] : 0.f);
      m0[4 + i] = (_Float16)0.f;
      m1[i] = (_Float16)acc[1][i];
      m1[4 + i] = (_Float16)(s <= l16 ? acc[2][i] : 0.f);
    }
    *reinterpret_cast<f16x8*>(rec + kRecOffMqk + lane * 16) = m0;
    *reinterpret_cast<f16x8*>(rec + kRecOffMqk + (64 + lane) * 16) = m1;
    if (g4 == 0) {
      bl[l16] = beta[0];
      bl[16 + l16] = beta[1];
    }
  }
  // The parked (b Kg)^T fragments back into registers; the barrier orders
  // these reads before the system overwrites their bytes.  It is also the
  // block's one barrier: every wave's record so far (its restored keys and
  // decays) is written before it and read by the next wave after it.  A
  // work-group fence does not wait for global stores, so the wave first
  // waits for its own (s_waitcnt fields: vmcnt bits 3:0 and 15:14 = 0, expcnt
  // bits 6:4 = 7 and lgkmcnt bits 11:8 = 15, i.e. not waited on); the reads
  // after it are the first accesses of this kernel to those bytes.
  f16x8 Xh[8], Xl[8];
#pragma unroll
  for (int mc = 0; mc < 8; ++mc) {
    Xh[mc] = park[mc][lane];
    Xl[mc] = park[8 + mc][lane];
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);
  __syncthreads();
  // A = Diag(b) stril(Akk) to LDS.
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int s = 4 * g4 + i;
    Al[l16][s] = s < l16 ? beta[0] * acc[3][i] : 0.f;
    Al[16 + l16][s] = beta[1] * acc[4][i];
    Al[16 + l16][16 + s] = s < l16 ? beta[1] * acc[5][i] : 0.f;
  }
  // The value rows are requested now, so that the inverse hides their
  // latency.
  u32x4 vw[4][2];
#pragma unroll
  for (int p = 0; p < 4; ++p)
#pragma unroll
    for (int hf = 0; hf < 2; ++hf)
      vw[p][hf] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
          rv, (uint32_t)(l16 + 16 * hf) * tok_bytes + (uint32_t)(32 * p + 8 * g4) * 2, 0, 0));
  wave_lds_sync();

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
  wave_lds_sync();
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
  wave_lds_sync();
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
  wave_lds_sync();

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


  // The previous chunk's keys and gates -- or, handed over, that chunk's
  // Kr^T fragments and decays from its record -- for M' and W (requested
  // before U0's products, which cover part of their latency).
  u32x4 kpw[4][2], gpw[4][2];
  if (hand) {
    const uint8_t* prec = rec - (int64_t)H * kRecBytes;   // slot - 1, same head
#pragma unroll
    for (int p = 0; p < 4; ++p)
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        kpw[p][hf] = *reinterpret_cast<const u32x4*>(prec + kRecOffKrT + ((2 * p + hf) * 64 + lane) * 16);
        gpw[p][hf] = *reinterpret_cast<const u32x4*>(prec + kRecOffDec + (32 * p + 16 * hf + 4 * g4) * 4);
      }
  } else if (!shared_prev) {
#pragma unroll
    for (int p = 0; p < 4; ++p)
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        kpw[p][hf] = load8(rkp, hf, p);
        gpw[p][hf] = load8(rgp, hf, p);
      }
  }

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
  // token 16tt + l16, i.e. the M A fragments of K step mc/2.  Per K step the
  // previous chunk's restored keys Kr_p (this lane's tokens and channels, in
  // FP32 then fp16) and decay d_p give -M' = -M Diag(d_p) and accumulate
  // W^T = Kr_p M^T (M as fp16 hi + lo), whose accumulators (rows = previous
  // tokens s, column = token t) are the W A fragments.
  f32x4 wacc[2][2] = {{z, z}, {z, z}};   // [s half][t half]
  float nkp[2] = {1.f, 1.f};               // front-end norm of the previous chunk's keys
  if (FE && a.fe.normalize_qk && !hand && !shared_prev) {
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      float s2 = 0.f;
#pragma unroll
      for (int p = 0; p < 4; ++p)
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float kv = bf16_elem(kpw[p][hf], j);
          s2 = fmaf(kv, kv, s2);
        }
      s2 += __shfl_xor(s2, 16);
      s2 += __shfl_xor(s2, 32);
      nkp[hf] = inv_norm(s2 + a.fe.norm_eps);
    }
  }
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    float dp[8];
    f16x8 krp[2];
    if (hand) {
      // Kr^T fragments (channel rows 32p.., 32p+16..) back to rows of tokens
      // by the one-hot products (exact), decays as stored
#pragma unroll
      for (int sh = 0; sh < 2; ++sh) {
        const f32x4 r0 = mfma_f16(__builtin_bit_cast(f16x8, kpw[p][0]), E[sh], z);
        const f32x4 r1 = mfma_f16(__builtin_bit_cast(f16x8, kpw[p][1]), E[sh], z);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          krp[sh][i] = (_Float16)r0[i];
          krp[sh][4 + i] = (_Float16)r1[i];
        }
      }
      // (whole-vector casts: a cast of a single vector element has been
      // compiled to the wrong element)
      const f32x4 d0 = __builtin_bit_cast(f32x4, gpw[p][0]), d1 = __builtin_bit_cast(f32x4, gpw[p][1]);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        dp[i] = d0[i];
        dp[4 + i] = d1[i];
      }
    } else if (shared_prev) {
      krp[0] = prev_kr[p][0][lane];
      krp[1] = prev_kr[p][1][lane];
      const f32x4 d0 = *reinterpret_cast<const f32x4*>(&prev_dec[32 * p + 4 * g4]);
      const f32x4 d1 = *reinterpret_cast<const f32x4*>(&prev_dec[32 * p + 16 + 4 * g4]);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        dp[i] = d0[i];
        dp[4 + i] = d1[i];
      }
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        // no previous chunk (an empty range): zero gates, so d_p = 1 and M' = M
        const float s0 = row_scan16(gate(bf16_elem(gpw[p][0], j), has_prev));
        const float b0 = __shfl(s0, 15, 16);
        const float s1 = row_scan16(gate(bf16_elem(gpw[p][1], j), has_prev)) + b0;
        const float gl = __shfl(s1, 15, 16) * kLog2e;
        dp[j] = fast_exp2(gl);
        krp[0][j] = static_cast<_Float16>(nkp[0] * bf16_elem(kpw[p][0], j) * fast_exp2(gl - s0 * kLog2e));
        krp[1][j] = static_cast<_Float16>(nkp[1] * bf16_elem(kpw[p][1], j) * fast_exp2(gl - s1 * kLog2e));
      }
    }
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      float mv[8];
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int mc = 2 * p + e;
        f32x4 m = mfma_f16(Xh[mc], th[tt], z);
        m = mfma_f16(Xh[mc], tl[tt], m);
        m = mfma_f16(Xl[mc], th[tt], m);
#pragma unroll
        for (int i = 0; i < 4; ++i) mv[4 * e + i] = m[i];
      }
      f16x8 mf, mh, ml;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        mf[j] = static_cast<_Float16>(-(mv[j] * dp[j]));
        _Float16 hh, ll;
        split_f16(mv[j], hh, ll);
        mh[j] = hh;
        ml[j] = ll;
      }
      *reinterpret_cast<f16x8*>(rec + kRecOffMneg + ((tt * 4 + p) * 64 + lane) * 16) = mf;
#pragma unroll
      for (int sh = 0; sh < 2; ++sh) {
        wacc[sh][tt] = mfma_f16(krp[sh], mh, wacc[sh][tt]);
        wacc[sh][tt] = mfma_f16(krp[sh], ml, wacc[sh][tt]);
      }
    }
  }
  // -W fragments: row t = 16tt + l16, K-slot 8g4 + i + 4sh <-> previous token 16sh + 4g4 + i.
#pragma unroll
  for (int tt = 0; tt < 2; ++tt) {
    f16x8 wh, wl;
#pragma unroll
    for (int sh = 0; sh < 2; ++sh)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        _Float16 hh, ll;
        split_f16(-wacc[sh][tt][i], hh, ll);
        wh[4 * sh + i] = hh;
        wl[4 * sh + i] = ll;
      }
    *reinterpret_cast<f16x8*>(rec + kRecOffWh + (tt * 64 + lane) * 16) = wh;
    *reinterpret_cast<f16x8*>(rec + kRecOffWl + (tt * 64 + lane) * 16) = wl;
  }
}


// Chain pass.  One block per (sequence, head, 16-column value tile), four
// waves with fixed roles and one barrier per chunk step.  With the records'
// M' and W the recurrence splits into two coupled chains, each advanced from
// the other's previous value (S_{-1} = initial state, U_{-1} = 0):
//   P_c = U0_c - M'_c S_{c-1}                       (needs the previous state)
//   U_c = P_c - W_c U_{c-1}                          (the only 1-step dependency)
//   S_c = Diag(d_{c-1}) S_{c-1} + Kr_{c-1}^T U_{c-1} (c >= 1; S_0 = S_{-1})
//   O_c = scale (Qg_c S_c + Mqk_c U_c)
// so in step c every wave only consumes what others produced in step c-1:
//   waves 0-1 (state halves, key rows 0-63 / 64-127): S_c from U_{c-1}; fp16
//            S_c for the output; their K-half of P_{c+1} (each adding half of
//            U0's rows);
//            the state stays in VGPRs for the whole sequence;
//   wave 2 (U):   U_c = (P_c halves summed) - W_c U_{c-1}, split into fp16
//            hi + lo for the state waves and the output;
//   wave 3 (output): O_{c-1} from fp16 S_{c-1}, U_{c-1} and the record.
// Each wave loads the record fragments it needs itself, straight into
// registers, three chunks ahead of use (a ring of three register sets per
// operand stream).  LDS carries only the step-to-step exchange (fp16 S, the P
// halves, U hi/lo), double-buffered by step parity.  Loads and stores are
// buffer operations issued unconditionally (a chunk past the end has an empty
// range: loads return zeros, stores are dropped), so every path issues the
// same memory operations and the compiler's wait counts stay exact.  Value
// columns evolve independently, so tiles never communicate.  Block b handles
// (sequence, head) unit b % units and tile b / units: with a unit count
// divisible by 8, all tiles of a unit run on one XCD and share its L2 copy of
// the records.
constexpr int kNT = kSplitSubtiles;                      // 16-column subtiles per block
constexpr int kExSb = 0;                                   // fp16 S_c, [kstep 4][t][lane][8]
constexpr int kExUh = 4096 * kNT;                          // U_c hi, [t][lane][8]
constexpr int kExUl = kExUh + 1024 * kNT;                  // U_c lo
constexpr int kExP = kExUl + 1024 * kNT;                   // P halves, [half 2][t][mt 2][lane][4] f32
constexpr int kExchBytes = kExP + 4096 * kNT;
constexpr int kDecSlots = 4;                               // chunk decays, 512 B each
constexpr int kChainLds = 2 * kExchBytes + kDecSlots * 512;
constexpr int kChainThreads = 256;
constexpr int kAhead = 3;                                  // register sets per operand stream
constexpr int kChainTiles = 8 / kNT;                       // blocks per (sequence, head)

// Record fragments, as each wave consumes them.  Everything but U0 is the
// same for all value columns, so a block with kNT subtiles loads it once.
struct AOps {            // state half: -M' (its K half) and U0 (its row tile), of chunk c+1
  f16x8 am[2][2];
  f32x4 u0[kNT][2];        // only [t][hs] is used
};
struct BOps {            // state half: Kr^T rows of chunk c-1
  f16x8 ak[4];
};
typedef float f32x2 __attribute__((ext_vector_type(2)));
struct WOps {            // U wave: -W hi / lo of chunk c, and its decays (two per lane)
  f16x8 wh[2], wl[2];
  f32x2 dec;
};
struct QOps {            // output wave: Qg and Mqk of chunk c-1
  f16x8 aq[2][4], amq[2];
};

// One chain run: chunks [cb, ce) of sequence n, head h, value columns
// [16 kNT tile, 16 kNT (tile + 1)).
struct ChainJob {
  int n, h, tile;
  int cb, ce;
  StateRef s_init;       // [128][128] state entering chunk cb, or none
  const float* s_init_lds = nullptr;   // or this block's columns of it in LDS, [128][16 kNT]
  bool identity;         // start from the identity instead (a window's map)
  bool with_u0;          // false: drop U0 (the map of a window is linear)
  bool with_out;         // store the outputs of the chunks
  bool ckpt;             // store checkpoints (runs of the true state only)
  StateRef s_final;      // [128][128] state after chunk ce-1, or none
};

__device__ __forceinline__ void chain_body(const PrefillArgs& a, const uint8_t* __restrict__ ws,
                                           unsigned char* lds, const ChainJob job) {
  const int H = a.num_heads;
  const int n = job.n, h = job.h;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g4 = lane >> 4;
  const int sub0 = kNT * job.tile;                      // first 16-column subtile
  auto colof = [&](int t) __attribute__((always_inline)) { return 16 * (sub0 + t) + (lane & 15); };
  const f32x4 z = {0.f, 0.f, 0.f, 0.f};

  const int bos = clamp_offset(a.cu_seqlens[n], a.total_tokens);
  const int eos = max(bos, clamp_offset(a.cu_seqlens[n + 1], a.total_tokens));
  const int nch = max(0, job.ce - job.cb);             // chunks of this run
  const int64_t slot0 = (int64_t)n + bos / CH + job.cb;
  const int tok0 = bos + CH * job.cb;

  auto exch = [&](int c) __attribute__((always_inline)) { return lds + (c & 1) * kExchBytes; };
  // Chunk c's 128 decays 2^{G_L}, written by the U wave from its record loads
  // (one copy per block instead of one per lane that needs them).
  auto decs = [&](int c) __attribute__((always_inline)) {
    return reinterpret_cast<float*>(lds + 2 * kExchBytes + (c & (kDecSlots - 1)) * 512);
  };
  auto xfrag = [&](const uint8_t* base, int idx) __attribute__((always_inline)) {
    return *reinterpret_cast<const f16x8*>(base + (idx * 64 + lane) * 16);
  };
  auto xacc = [&](const uint8_t* base, int idx) __attribute__((always_inline)) {
    return *reinterpret_cast<const f32x4*>(base + (idx * 64 + lane) * 16);
  };
  // Each operand stream of a wave reads the records in chunk order, one
  // chunk per load, so it keeps a running address and advances it by the
  // chunk stride: recomputing ((slot0 + c) H + h) kRecBytes per load costs
  // about 20 scalar instructions (64-bit multiplies), and a chain step is
  // bound by instruction issue.  A chunk past the run is an empty range (its
  // loads return zeros without touching memory).
  struct RecStream {
    const uint8_t* p;
    int c;
  };
  const int64_t rec_stride = (int64_t)H * kRecBytes;
  auto rec_stream = [&]() __attribute__((always_inline)) {
    return RecStream{ws + (slot0 * H + h) * kRecBytes, 0};
  };
  auto next_rec = [&](RecStream& st) __attribute__((always_inline)) {
    const __amdgpu_buffer_rsrc_t r = make_buffer(st.p, st.c < nch ? (uint32_t)kRecBytes : 0u);
    st.p += rec_stride;
    ++st.c;
    return r;
  };
  auto ld16 = [&](__amdgpu_buffer_rsrc_t r, int off) __attribute__((always_inline)) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, (uint32_t)off, 0, 0);
  };
  auto gfrag = [&](__amdgpu_buffer_rsrc_t r, int base, int idx) __attribute__((always_inline)) {
    return __builtin_bit_cast(f16x8, ld16(r, base + (idx * 64 + lane) * 16));
  };
  auto gacc = [&](__amdgpu_buffer_rsrc_t r, int base, int idx) __attribute__((always_inline)) {
    return __builtin_bit_cast(f32x4, ld16(r, base + (idx * 64 + lane) * 16));
  };

  if (wave == 3) {
    // ------------------------------------------------------------- output
    if (!job.with_out) {
      for (int c = 0; c < nch + 2; ++c) __syncthreads();
      return;
    }
    QOps q[kAhead];
    RecStream qs = rec_stream();
    auto load_q = [&](QOps& o) __attribute__((always_inline)) {   // the stream's next chunk
      const __amdgpu_buffer_rsrc_t r = next_rec(qs);
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
        for (int p = 0; p < 4; ++p) o.aq[mt][p] = gfrag(r, kRecOffQg, mt * 4 + p);
        o.amq[mt] = gfrag(r, kRecOffMqk, mt);
      }
    };
#pragma unroll
    for (int i = 0; i < kAhead; ++i) load_q(q[i]);   // chunks 0 .. kAhead-1
    __syncthreads();   // P_0 published
    __syncthreads();   // step 0
    // output rows of chunk c-1 at step c, advanced by one chunk per step
    const uint16_t* optr = a.out + ((int64_t)tok0 * H + h) * D;
    int ot0 = tok0;
    // step c >= 1: O_{c-1}, whose fragments sit in set (c-1) % 3
    auto step = [&](auto I_const, int c) __attribute__((always_inline)) {
      constexpr int I = decltype(I_const)::value;
      const QOps& o = q[I];
      const uint8_t* ex = exch(c - 1);
      // O^T = S^T Qg^T + U^T Mqk^T: the same fragments with A and B swapped;
      // lane (g4, l16) gets value columns 4g4..4g4+3 of token 16mt + l16.
      f32x4 O[kNT][2];
#pragma unroll
      for (int t = 0; t < kNT; ++t) {
        f16x8 sb[4];
#pragma unroll
        for (int p = 0; p < 4; ++p) sb[p] = xfrag(ex + kExSb, p * kNT + t);
        const f16x8 uh = xfrag(ex + kExUh, t), ul = xfrag(ex + kExUl, t);
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) O[t][mt] = z;
#pragma unroll
        for (int p = 0; p < 4; ++p)
#pragma unroll
          for (int mt = 0; mt < 2; ++mt) O[t][mt] = mfma_f16(sb[p], o.aq[mt][p], O[t][mt]);
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
          O[t][mt] = mfma_f16(uh, o.amq[mt], O[t][mt]);
          O[t][mt] = mfma_f16(ul, o.amq[mt], O[t][mt]);
        }
      }
      load_q(q[I]);   // chunk c - 1 + kAhead
      // rows t >= L of a final partial chunk fall outside the range and are dropped
      const int L = min(CH, eos - ot0);
      const __amdgpu_buffer_rsrc_t orsrc = make_buffer(optr, (uint32_t)(((L - 1) * H + 1) * D * 2));
      optr += (int64_t)CH * H * D;
      ot0 += CH;
#pragma unroll
      for (int t = 0; t < kNT; ++t)
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
          const int tok = 16 * mt + (lane & 15);
          u32x2 pk;
          pk[0] = (uint32_t)f32_to_bf16(a.scale * O[t][mt][0]) |
                  ((uint32_t)f32_to_bf16(a.scale * O[t][mt][1]) << 16);
          pk[1] = (uint32_t)f32_to_bf16(a.scale * O[t][mt][2]) |
                  ((uint32_t)f32_to_bf16(a.scale * O[t][mt][3]) << 16);
          __builtin_amdgcn_raw_buffer_store_b64(
              pk, orsrc, (uint32_t)((tok * H * D + 16 * (sub0 + t) + 4 * g4) * 2), 0, 0);
        }
      __syncthreads();
    };
    // Whole triples, then the rest after the loop: a break inside the
    // unrolled triple would give the loop a second way back to its header,
    // and the wait counts for the first step's fragments would then assume
    // they were loaded one step earlier instead of three.
    int c = 1;
    for (; c + 2 <= nch; c += kAhead) {
      step(std::integral_constant<int, 0>{}, c);
      step(std::integral_constant<int, 1>{}, c + 1);
      step(std::integral_constant<int, 2>{}, c + 2);
    }
    if (c <= nch) step(std::integral_constant<int, 0>{}, c);
    if (c + 1 <= nch) step(std::integral_constant<int, 1>{}, c + 1);
    return;
  }

  if (wave == 2) {
    // ------------------------------------------------------------------ U
    WOps w[kAhead];
    RecStream wst = rec_stream();
    auto load_w = [&](WOps& o) __attribute__((always_inline)) {   // the stream's next chunk
      const __amdgpu_buffer_rsrc_t r = next_rec(wst);
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        o.wh[mt] = gfrag(r, kRecOffWh, mt);
        o.wl[mt] = gfrag(r, kRecOffWl, mt);
      }
      o.dec = __builtin_bit_cast(f32x2, __builtin_amdgcn_raw_buffer_load_b64(
          r, (uint32_t)(kRecOffDec + lane * 8), 0, 0));
    };
    auto put_dec = [&](const WOps& o, int c) __attribute__((always_inline)) {
      *reinterpret_cast<f32x2*>(decs(c) + 2 * lane) = o.dec;
    };
#pragma unroll
    for (int i = 0; i < kAhead; ++i) load_w(w[i]);   // chunks 0 .. kAhead-1
    put_dec(w[0], 0);                 // decays of chunk 0, used in step 1
    f16x8 Uh[kNT], Ul[kNT];
#pragma unroll
    for (int t = 0; t < kNT; ++t)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        Uh[t][j] = static_cast<_Float16>(0.f);
        Ul[t][j] = static_cast<_Float16>(0.f);
      }
    __syncthreads();   // P_0 published
    // step c: U_c from P_c and U_{c-1}; W_c sits in set c % 3
    auto step = [&](auto I_const, int c) __attribute__((always_inline)) {
      constexpr int I = decltype(I_const)::value;
      const WOps& o = w[I];
      const uint8_t* ex = exch(c - 1);
      f32x4 U[kNT][2];
#pragma unroll
      for (int t = 0; t < kNT; ++t)
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
          U[t][mt] = xacc(ex + kExP, t * 2 + mt) + xacc(ex + kExP, (kNT + t) * 2 + mt);
#pragma unroll
      for (int t = 0; t < kNT; ++t)
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
          U[t][mt] = mfma_f16(o.wh[mt], Uh[t], U[t][mt]);
          U[t][mt] = mfma_f16(o.wh[mt], Ul[t], U[t][mt]);
          U[t][mt] = mfma_f16(o.wl[mt], Uh[t], U[t][mt]);
        }
      load_w(w[I]);   // chunk c + kAhead
      put_dec(w[(I + 1) % kAhead], c + 1);   // applied at the end of step c+1
      uint8_t* exw = exch(c);
#pragma unroll
      for (int t = 0; t < kNT; ++t) {
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
          for (int i2 = 0; i2 < 4; ++i2) {
            _Float16 hh, ll;
            split_f16(U[t][mt][i2], hh, ll);
            Uh[t][4 * mt + i2] = hh;
            Ul[t][4 * mt + i2] = ll;
          }
        *reinterpret_cast<f16x8*>(exw + kExUh + (t * 64 + lane) * 16) = Uh[t];
        *reinterpret_cast<f16x8*>(exw + kExUl + (t * 64 + lane) * 16) = Ul[t];
      }
      __syncthreads();
    };
    // steps 0..nch (the last one's U is never read)
    // whole triples, then the rest (as in the output wave)
    int c = 0;
    for (; c + 2 <= nch; c += kAhead) {
      step(std::integral_constant<int, 0>{}, c);
      step(std::integral_constant<int, 1>{}, c + 1);
      step(std::integral_constant<int, 2>{}, c + 2);
    }
    if (c <= nch) step(std::integral_constant<int, 0>{}, c);
    if (c + 1 <= nch) step(std::integral_constant<int, 1>{}, c + 1);
    return;
  }

  // --------------------------------------------------------- state halves
  // Wave hs owns key rows 64hs..64hs+63: accumulator tiles mt = 4hs..4hs+3,
  // i.e. the fp16 B fragments (K steps) p = 2hs, 2hs+1.  The two halves are
  // separate code (hs a constant): half hs adds U0's row tile mt = hs (tokens
  // 16 hs..16 hs + 15) to its share of P, so each loads one U0 fragment.
  auto state_half = [&](auto hs_const) __attribute__((always_inline)) {
  constexpr int hs = decltype(hs_const)::value;
  f32x4 S[kNT][4];
#pragma unroll
  for (int t = 0; t < kNT; ++t)
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 16 * (4 * hs + m) + 4 * g4 + i, col = colof(t);
        S[t][m][i] = job.s_init_lds ? job.s_init_lds[row * (16 * kNT) + 16 * t + (lane & 15)]
                     : job.s_init   ? job.s_init.load(row * D + col)
                                    : (job.identity && row == col ? 1.f : 0.f);
      }
  AOps A[kAhead];
  BOps B[kAhead];
  RecStream ast = rec_stream(), bst = rec_stream();
  auto load_a = [&](AOps& o) __attribute__((always_inline)) {   // the A stream's next chunk
    const __amdgpu_buffer_rsrc_t r = next_rec(ast);
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
      for (int q = 0; q < 2; ++q) o.am[mt][q] = gfrag(r, kRecOffMneg, mt * 4 + 2 * hs + q);
      if (mt == hs) {
#pragma unroll
        for (int t = 0; t < kNT; ++t) o.u0[t][mt] = gacc(r, kRecOffU0 + (sub0 + t) * 2048, mt);
      }
    }
  };
  auto load_b = [&](BOps& o) __attribute__((always_inline)) {   // the B stream's next chunk
    const __amdgpu_buffer_rsrc_t r = next_rec(bst);
#pragma unroll
    for (int m = 0; m < 4; ++m) o.ak[m] = gfrag(r, kRecOffKrT, 4 * hs + m);
  };
  // fp16 S_c to exchange(c) and this half's share of P_{c+1} = U0_{c+1} -
  // M'_{c+1} S_c from the fragments of chunk c+1.
  auto publish = [&](const AOps& o, int c) __attribute__((always_inline)) {
    uint8_t* ex = exch(c);
#pragma unroll
    for (int t = 0; t < kNT; ++t) {
      f16x8 Sb[2];
#pragma unroll
      for (int q = 0; q < 2; ++q)
#pragma unroll
        for (int i2 = 0; i2 < 4; ++i2) {
          Sb[q][i2] = static_cast<_Float16>(S[t][2 * q][i2]);
          Sb[q][4 + i2] = static_cast<_Float16>(S[t][2 * q + 1][i2]);
        }
#pragma unroll
      for (int q = 0; q < 2; ++q)
        *reinterpret_cast<f16x8*>(ex + kExSb + (((2 * hs + q) * kNT + t) * 64 + lane) * 16) = Sb[q];
      f32x4 P[2];
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) P[mt] = z;
      if (job.with_u0) P[hs] = o.u0[t][hs];
#pragma unroll
      for (int q = 0; q < 2; ++q)
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) P[mt] = mfma_f16(o.am[mt][q], Sb[q], P[mt]);
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
        *reinterpret_cast<f32x4*>(ex + kExP + (((hs * kNT + t) * 2 + mt) * 64 + lane) * 16) = P[mt];
    }
  };
  // A set k % 3 holds chunk k's -M', U0 (consumed in step k-1); B set k % 3
  // holds chunk k's Kr^T and decays (consumed in step k+1).
#pragma unroll
  for (int i = 0; i < kAhead; ++i) {
    load_a(A[i]);   // chunks 0 .. kAhead-1 of both streams
    load_b(B[i]);
  }
  publish(A[0], -1);               // fp16 S_{-1} (unused) and P_0 from the initial state
  load_a(A[0]);                    // chunk kAhead
  __syncthreads();                 // P_0 published
  publish(A[1], 0);                // step 0: S_0 = S_{-1}; P_1
  load_a(A[1]);                    // chunk 1 + kAhead
  // The decay of chunk c is applied to S_c once S_c is published (fp16 copy
  // and P_{c+1} use the undecayed state), so that step c+1 starts with its
  // MFMAs.  Never after the last step: the final state is undecayed.
  auto read_decay = [&](f32x4 (&dv)[4], int c) __attribute__((always_inline)) {
    const float* dc = decs(c);
#pragma unroll
    for (int m = 0; m < 4; ++m) dv[m] = *reinterpret_cast<const f32x4*>(dc + 16 * (4 * hs + m) + 4 * g4);
  };
  auto decay = [&](const f32x4 (&dv)[4]) __attribute__((always_inline)) {
#pragma unroll
    for (int t = 0; t < kNT; ++t)
#pragma unroll
      for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int i2 = 0; i2 < 4; ++i2) S[t][m][i2] *= dv[m][i2];
  };
  if (nch > 0) {
    f32x4 dv[4];
    read_decay(dv, 0);
    decay(dv);
  }
  __syncthreads();
  // Checkpoints: after step c the state has consumed chunks 0..k-1 of the
  // sequence (k = cb + c); it is stored when k is a multiple of the interval
  // in chunks and those k chunks are full.  The next such k and its row are
  // kept as uniform counters (one loop for both cases, so the checkpoint
  // stores cost no registers beyond one offset).
  const int ck_per = (job.ckpt && a.ckpt) ? a.ckpt_tokens / CH : 0;
  const int ck_full = (eos - bos) / CH;
  int ck_next = ck_per ? ck_per * ((job.cb + ck_per) / ck_per) : INT_MAX;   // first multiple > cb
  int64_t ck_row = ck_per ? ((int64_t)n + bos / a.ckpt_tokens + ck_next / ck_per - 1) : 0;
  const uint32_t ck_off = (uint32_t)(((64 * hs + 4 * g4) * D + colof(0)) * 4);
  // step c >= 1: S_c = Diag(d_{c-1}) S_{c-1} + Kr_{c-1}^T U_{c-1} (S already
  // decayed), then P_{c+1}, then the decay of chunk c.
  auto step = [&](auto I_const, int c) __attribute__((always_inline)) {
    constexpr int I = decltype(I_const)::value;   // = c % 3 for the B set of chunk c-1: (I+2)%3
    constexpr int IB = (I + 2) % 3, IA = (I + 1) % 3;
    const BOps& kb = B[IB];
    const uint8_t* ex = exch(c - 1);
    f16x8 uh[kNT], ul[kNT];
#pragma unroll
    for (int t = 0; t < kNT; ++t) {
      uh[t] = xfrag(ex + kExUh, t);
      ul[t] = xfrag(ex + kExUl, t);
    }
    f32x4 dv[4];
    read_decay(dv, c);                                 // chunk c's decays, used at the end
#pragma unroll
    for (int t = 0; t < kNT; ++t)
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        S[t][m] = mfma_f16(kb.ak[m], uh[t], S[t][m]);
        S[t][m] = mfma_f16(kb.ak[m], ul[t], S[t][m]);
      }
    if (job.cb + c == ck_next) {
      if (ck_next <= ck_full) {
        const __amdgpu_buffer_rsrc_t cr =
            make_buffer(a.ckpt + (ck_row * H + h) * (int64_t)(D * D), (uint32_t)(D * D * 4));
#pragma unroll
        for (int t = 0; t < kNT; ++t)
#pragma unroll
          for (int m = 0; m < 4; ++m)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const float sv = S[t][m][i];   // a scalar first: a vector element is not a bit_cast source
              __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, sv), cr,
                                                    ck_off + (uint32_t)(i * D * 4 + 64 * t),
                                                    16 * m * D * 4, 0);
            }
      }
      ck_next += ck_per;
      ++ck_row;
    }
    load_b(B[IB]);                                    // chunk c - 1 + kAhead
    publish(A[IA], c);                                // unused past the end
    if (c < nch) decay(dv);
    load_a(A[IA]);                                    // chunk c + 1 + kAhead
    __syncthreads();
  };
  // whole triples, then the rest (as in the output wave)
  int c = 1;
  for (; c + 2 <= nch; c += kAhead) {
    step(std::integral_constant<int, 1>{}, c);
    step(std::integral_constant<int, 2>{}, c + 1);
    step(std::integral_constant<int, 0>{}, c + 2);
  }
  if (c <= nch) step(std::integral_constant<int, 1>{}, c);
  if (c + 1 <= nch) step(std::integral_constant<int, 2>{}, c + 1);
  if (job.s_final) {
#pragma unroll
    for (int t = 0; t < kNT; ++t)
#pragma unroll
      for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          job.s_final.store((16 * (4 * hs + m) + 4 * g4 + i) * D + colof(t), S[t][m][i]);
  }
  };
  if (wave == 0)
    state_half(std::integral_constant<int, 0>{});
  else
    state_half(std::integral_constant<int, 1>{});
}

__global__ __launch_bounds__(kChainThreads) void prefill_split_chain(PrefillArgs a,
                                                                     const uint8_t* __restrict__ ws) {
  extern __shared__ __align__(16) unsigned char lds[];
  const int H = a.num_heads;
  const int units = a.num_seqs * H;
  const int unit = blockIdx.x % units, tile = blockIdx.x / units;
  const int n = unit / H, h = unit % H;
  const int bos = clamp_offset(a.cu_seqlens[n], a.total_tokens);
  const int eos = max(bos, clamp_offset(a.cu_seqlens[n + 1], a.total_tokens));
  ChainJob job;
  job.n = n; job.h = h; job.tile = tile;
  job.cb = 0; job.ce = (eos - bos + CH - 1) / CH;
  job.s_init = prefill_initial_state(a, n, h);
  job.identity = false; job.with_u0 = true; job.with_out = true; job.ckpt = true;
  job.s_final = prefill_final_state(a, n, h);
  chain_body(a, ws, lds, job);
}

// ------------------------------------------------------------ windows
// A long sequence is cut into windows (window_chunks_of: up to a.windows per
// sequence, by its own length) whose first chunks carry M' = M and W = 0, so
// a chain can start at any window.  The
// state map of a window is affine, S_end = P_w S_in + B_w, which gives
//   phase A (all at once): window 0 from the initial state; for every window
//            w that is neither first nor last, B_w (its chain from zero) and
//            P_w (its chain from the identity, without U0);
//   phase C (all at once): windows 1.. from S_in(w), with outputs, where
//            S_in(1) = end of window 0 and S_in(w+1) = P_w S_in(w) + B_w is
//            composed by each block of window w before its chain.
// About 2 x window_chunks chain steps instead of the sequence's chunk count.
struct WinView {
  float* base;
  int H, W;
  __device__ float* at(int n, int h, int w, int kind) const {   // kind 0 E, 1 P
    return base + ((((int64_t)n * H + h) * W + w) * 2 + kind) * (128 * 128);
  }
};

__device__ __forceinline__ int seq_chunks(const PrefillArgs& a, int n) {
  const int bos = clamp_offset(a.cu_seqlens[n], a.total_tokens);
  const int eos = max(bos, clamp_offset(a.cu_seqlens[n + 1], a.total_tokens));
  return (eos - bos + CH - 1) / CH;
}

__global__ __launch_bounds__(kChainThreads) void prefill_split_window_a(PrefillArgs a,
                                                                        const uint8_t* __restrict__ ws,
                                                                        WinView wv) {
  extern __shared__ __align__(16) unsigned char lds[];
  const int H = a.num_heads, units = a.num_seqs * H, W = a.windows;
  const int jobs = 1 + 2 * (W - 2);
  const int tile = blockIdx.x / (units * jobs), r = blockIdx.x % (units * jobs);
  const int unit = r % units, j = r / units;
  const int n = unit / H, h = unit % H;
  const int nch = seq_chunks(a, n);
  const int WC = max(1, window_chunks_of(a, nch));
  const int nwin = max(1, (nch + WC - 1) / WC);
  ChainJob job;
  job.n = n; job.h = h; job.tile = tile;
  if (j == 0) {
    job.cb = 0; job.ce = min(WC, nch);
    job.s_init = prefill_initial_state(a, n, h);
    job.identity = false; job.with_u0 = true; job.with_out = true; job.ckpt = true;
    job.s_final = nwin <= 1 ? prefill_final_state(a, n, h) : fp32_state(wv.at(n, h, 0, 0));
  } else {
    const bool map = j > W - 2;
    const int w = map ? j - (W - 2) : j;
    if (w >= nwin - 1) return;            // the last window needs neither
    job.cb = w * WC; job.ce = min(nch, (w + 1) * WC);
    job.s_init = StateRef{};
    job.identity = map; job.with_u0 = !map; job.with_out = false; job.ckpt = false;
    job.s_final = fp32_state(wv.at(n, h, w, map ? 1 : 0));
  }
  chain_body(a, ws, lds, job);
}

// S_in(wt) = P_{wt-1}( ... (P_1 E_0 + B_1) ... ) + B_{wt-1} for this block's value
// columns, composed by the window_c block that runs window wt before its chain
// (a few short steps: a kernel of their own cost more to launch than they
// take).  Four waves, wave q owning rows 32q..32q+31 of a 16-column subtile;
// P as bf16 hi + lo A fragments (the next window's requested while a step
// computes), the current S as bf16 hi + lo B fragments in LDS (a step's
// accumulators are the next step's K step q), three products per pair, FP32
// accumulation on B.  bf16 rather than fp16: a state that has decayed far
// below fp16's range (no writes over thousands of tokens) keeps its relative
// precision, at ~16 significand bits per hi + lo pair.  The result lands in LDS as FP32 [128][16 kNT] at the
// first exchange buffer and the fragments use the second; both are free
// until the chain's first barrier.
__device__ __forceinline__ void carry_to_lds(const WinView& wv, int n, int h, int tile, int wt,
                                             unsigned char* lds) {
  bf16x8* const xh = reinterpret_cast<bf16x8*>(lds + kExchBytes);   // [kstep 4][lane 64]
  bf16x8* const xl = xh + 4 * 64;
  float* const sin = reinterpret_cast<float*>(lds);
  const int lane = threadIdx.x & 63, q = threadIdx.x >> 6;
  const int g4 = lane >> 4, l16 = lane & 15;
  // rows of this lane's accumulator entries: tile 2q+e, row 16(2q+e) + 4g4 + i
  auto row_of = [&](int e, int i) __attribute__((always_inline)) { return 32 * q + 16 * e + 4 * g4 + i; };
  auto put_frags = [&](const float* v) __attribute__((always_inline)) {
    bf16x8 hi, lo;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      __bf16 hh, ll;
      split_bf16(v[j], hh, ll);
      hi[j] = hh;
      lo[j] = ll;
    }
    xh[q * 64 + lane] = hi;
    xl[q * 64 + lane] = lo;
  };
  typedef float f32x4v __attribute__((ext_vector_type(4)));
  // P_w fragments of this wave's row tiles: [e][kstep p][half of the K-slots]
  auto load_p = [&](f32x4v (&pf)[2][4][2], int w) __attribute__((always_inline)) {
    const float* P = wv.at(n, h, w, 1);
#pragma unroll
    for (int e = 0; e < 2; ++e)
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const float* r = P + (32 * q + 16 * e + l16) * 128 + 32 * p + 4 * g4;
        pf[e][p][0] = *reinterpret_cast<const f32x4v*>(r);
        pf[e][p][1] = *reinterpret_cast<const f32x4v*>(r + 16);
      }
  };
  for (int t = 0; t < kNT; ++t) {
    const int col = 16 * (kNT * tile + t) + l16;
    f32x4v pf[2][4][2];
    load_p(pf, 1);
    {
      const float* e0 = wv.at(n, h, 0, 0);
      float v[8];
#pragma unroll
      for (int e = 0; e < 2; ++e)
#pragma unroll
        for (int i = 0; i < 4; ++i) v[4 * e + i] = e0[row_of(e, i) * 128 + col];
      put_frags(v);
    }
    for (int w = 1; w < wt; ++w) {
      __syncthreads();
      bf16x8 sh[4], sl[4];
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        sh[p] = xh[p * 64 + lane];
        sl[p] = xl[p * 64 + lane];
      }
      const float* B = wv.at(n, h, w, 0);
      f32x4 acc[2];
#pragma unroll
      for (int e = 0; e < 2; ++e)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[e][i] = B[row_of(e, i) * 128 + col];
#pragma unroll
      for (int e = 0; e < 2; ++e)
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          bf16x8 ph, pl;
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            __bf16 hh, ll;
            split_bf16(pf[e][p][j >> 2][j & 3], hh, ll);
            ph[j] = hh;
            pl[j] = ll;
          }
          acc[e] = mfma_bf16(ph, sh[p], acc[e]);
          acc[e] = mfma_bf16(ph, sl[p], acc[e]);
          acc[e] = mfma_bf16(pl, sh[p], acc[e]);
        }
      if (w + 1 < wt) load_p(pf, w + 1);
      __syncthreads();   // every wave has read this step's fragments
      float v[8];
#pragma unroll
      for (int e = 0; e < 2; ++e)
#pragma unroll
        for (int i = 0; i < 4; ++i) v[4 * e + i] = acc[e][i];
      if (w + 1 < wt) {
        put_frags(v);
      } else {
#pragma unroll
        for (int e = 0; e < 2; ++e)
#pragma unroll
          for (int i = 0; i < 4; ++i) sin[row_of(e, i) * (16 * kNT) + 16 * t + l16] = v[4 * e + i];
      }
    }
  }
  __syncthreads();   // the initial state is complete
}

__global__ __launch_bounds__(kChainThreads) void prefill_split_window_c(PrefillArgs a,
                                                                        const uint8_t* __restrict__ ws,
                                                                        WinView wv) {
  extern __shared__ __align__(16) unsigned char lds[];
  const int H = a.num_heads, units = a.num_seqs * H, W = a.windows;
  const int tile = blockIdx.x / (units * (W - 1)), r = blockIdx.x % (units * (W - 1));
  const int unit = r % units, w = 1 + r / units;
  const int n = unit / H, h = unit % H;
  const int nch = seq_chunks(a, n);
  const int WC = max(1, window_chunks_of(a, nch));
  const int nwin = max(1, (nch + WC - 1) / WC);
  if (w >= nwin) return;
  ChainJob job;
  job.n = n; job.h = h; job.tile = tile;
  job.cb = w * WC; job.ce = min(nch, (w + 1) * WC);
  job.s_init = fp32_state(w == 1 ? wv.at(n, h, 0, 0) : nullptr);   // window 1 starts from E_0
  job.s_init_lds = nullptr;
  if (w >= 2) {
    carry_to_lds(wv, n, h, tile, w, lds);
    job.s_init_lds = reinterpret_cast<const float*>(lds);
  }
  job.identity = false; job.with_u0 = true; job.with_out = true; job.ckpt = true;
  job.s_final = w == nwin - 1 ? prefill_final_state(a, n, h) : StateRef{};
  chain_body(a, ws, lds, job);
}

template <int MODE, bool FE>
hipError_t launch_prep(const PrefillArgs& a, uint8_t* ws, hipStream_t s) {
  const float exp2C = MODE == 0 ? std::exp2(a.anchor_log2) : 0.f;
  const int64_t slots = (int64_t)a.num_seqs + a.total_tokens / CH + 1;
  const int64_t groups = (slots + kPrepWaves - 1) / kPrepWaves * a.num_heads;
  const int64_t blocks = 8 * ((groups + 7) / 8);
  if (blocks > INT_MAX) return hipErrorInvalidValue;
  prefill_split_prep<MODE, FE><<<(unsigned)blocks, 64 * kPrepWaves, 0, s>>>(a, exp2C, ws);
  return hipGetLastError();
}

template <class K>
hipError_t set_lds(K* kernel, bool& done) {
  if (done) return hipSuccess;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kernel),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, kChainLds);
  if (e == hipSuccess) done = true;   // idempotent; a race only repeats the call
  return e;
}

hipError_t launch_chain(const PrefillArgs& a, const uint8_t* ws, hipStream_t s) {
  const int64_t units = (int64_t)a.num_seqs * a.num_heads;
  if (a.windows <= 1) {
    static bool done = false;
    hipError_t e = set_lds(&prefill_split_chain, done);
    if (e != hipSuccess) return e;
    prefill_split_chain<<<dim3((unsigned)(units * kChainTiles)), kChainThreads, kChainLds, s>>>(a, ws);
    return hipGetLastError();
  }
  static bool done_a = false, done_c = false;
  hipError_t e = set_lds(&prefill_split_window_a, done_a);
  if (e == hipSuccess) e = set_lds(&prefill_split_window_c, done_c);
  if (e != hipSuccess) return e;
  WinView wv;
  wv.base = reinterpret_cast<float*>(const_cast<uint8_t*>(ws) +
                                     split_records_bytes(a.num_seqs, a.total_tokens, a.num_heads));
  wv.H = a.num_heads;
  wv.W = a.windows;
  const int jobs = 1 + 2 * (a.windows - 2);
  prefill_split_window_a<<<dim3((unsigned)(units * jobs * kChainTiles)), kChainThreads, kChainLds, s>>>(a, ws, wv);
  prefill_split_window_c<<<dim3((unsigned)(units * (a.windows - 1) * kChainTiles)), kChainThreads, kChainLds, s>>>(
      a, ws, wv);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill_split_prepare(const PrefillArgs& a, int anchor_mode, void* workspace,
                                        hipStream_t s) {
  if (a.num_seqs <= 0) return hipSuccess;
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  if (frontend_active(a.fe)) {
    if (anchor_mode == 2) return launch_prep<2, true>(a, ws, s);
    return anchor_mode == 0 ? launch_prep<0, true>(a, ws, s) : launch_prep<1, true>(a, ws, s);
  }
  if (anchor_mode == 2) return launch_prep<2, false>(a, ws, s);
  return anchor_mode == 0 ? launch_prep<0, false>(a, ws, s) : launch_prep<1, false>(a, ws, s);
}

hipError_t launch_prefill_split_chain(const PrefillArgs& a, const void* workspace,
                                      hipStream_t s) {
  if (a.num_seqs <= 0) return hipSuccess;
  return launch_chain(a, static_cast<const uint8_t*>(workspace), s);
}

hipError_t launch_prefill_split(const PrefillArgs& a, int anchor_mode, int dv_split,
                                void* workspace, hipStream_t s) {
  if (dv_split != kChainTiles) return hipErrorInvalidValue;   // kNT 16-column subtiles per chain block
  hipError_t e = launch_prefill_split_prepare(a, anchor_mode, workspace, s);
  if (e != hipSuccess) return e;
  return launch_prefill_split_chain(a, workspace, s);
}

}  // namespace kda
