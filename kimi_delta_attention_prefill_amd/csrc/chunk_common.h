// Pieces shared by the chunk-32 prefill kernels (fused and split routes):
// MFMA operand types, the K-slot permutation, and the per-chunk preparation
// steps 1-3 of "FlashInfer PR #4262: CAKE KDA Prefill Highlights", section 2
// (gate prefix and anchored operands; causal Mqk and the triangular system;
// the 32x32 unit-lower-triangular inverse), with the fixed exponent anchor of
// section 1 or its 16-token split.  The preparation helpers run on the four
// producer waves of the fused kernel (256 threads, `tid` 0..255, `wave`
// 0..3 counted within the producers); they contain no barriers, the caller
// places them between its own.
#pragma once

#include "kda_device.h"
#include "kda_internal.h"

namespace kda {
namespace chunk {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int CH = 32;          // chunk length
constexpr int D = kHeadDim;     // 128
constexpr int RP = D + 8;       // padded row (elements) of [32 x 128] 16-bit arrays
constexpr int GP = D + 4;       // padded row of the FP32 gate prefix
constexpr int TP = CH + 8;      // padded row of [* x 32] fp16 arrays

// An accumulator tile of v_mfma_f32_16x16x32 gives lane l rows 4(l/16)+i of
// column l%16; two stacked tiles give rows {4(l/16)+i, 16+4(l/16)+i}.  Using
// that set as the lane's 8 K-slots lets an FP32 accumulator become the next
// product's B operand by a register conversion.  kslot(x) is the slot of
// K-index x (0..31): slot 8*grp + j holds index j<4 ? 4grp+j : 16+4grp+j-4.
__device__ __forceinline__ int kslot(int x) {
  const int hi = x >> 4, r = x & 15;
  return ((r >> 2) << 3) + (r & 3) + (hi << 2);
}

__device__ __forceinline__ f32x4 mfma_bf16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_f16(f16x8 a, f16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ void split_bf16(float x, __bf16& hi, __bf16& lo) {
  hi = static_cast<__bf16>(x);
  lo = static_cast<__bf16>(x - static_cast<float>(hi));
}
// Two values at once (one packed conversion for both his, one for both los;
// the same roundings as split_bf16), into elements j, j+1 of hi and lo.
__device__ __forceinline__ void split_bf16_pair(float a, float b, bf16x8& hi, bf16x8& lo, int j) {
  const f32x2 x = {a, b};
  const bf16x2 h = __builtin_convertvector(x, bf16x2);
  const bf16x2 l = __builtin_convertvector(x - __builtin_convertvector(h, f32x2), bf16x2);
  hi[j] = h[0];
  hi[j + 1] = h[1];
  lo[j] = l[0];
  lo[j + 1] = l[1];
}
__device__ __forceinline__ void split_f16(float x, _Float16& hi, _Float16& lo) {
  hi = static_cast<_Float16>(x);
  lo = static_cast<_Float16>(x - static_cast<float>(hi));
}

// One chunk's q, k, g rows in LDS, padded to RP.  Padding tokens (t >= L)
// are zero.
struct ChunkQKG {
  uint16_t q[CH][RP];
  uint16_t k[CH][RP];
  uint16_t g[CH][RP];
};

// A prepared chunk: everything the state chain of the fused route reads,
// one ring slot.  DVS = value columns of the block.
template <int DVS>
struct ChunkOps {
  _Float16 Kg[CH][RP];         // k 2^G      [token][dk, permuted]
  _Float16 Qg[CH][RP];         // q 2^G      [token][dk, permuted]
  _Float16 KrT[D][TP];         // (k 2^{G_L-G})^T [dk][token, permuted]
  _Float16 T[CH][TP];          // (I + A)^{-1}     [token][token, permuted]
  _Float16 Mqk[CH][TP];        // causal Mqk       [token][token, permuted]
  float dec[D];                // 2^{G_L}: chunk decay of each key row
  float beta[CH];              // zero for padding tokens
  uint16_t v[CH][DVS];         // the block's value columns, bf16
};

// The producers' working memory for one chunk: the gate prefix, and, over
// its bytes once the anchored operands are built, the triangular system and
// its inverse.  The split-K partials of the pairwise products live over the
// chunk's own q/k/g rows (part_entry).
struct PrepWork {
  float G[CH][GP];             // log2-domain inclusive gate prefix
  float EL[D];                 // fixed anchor: 2^{G_L - C}
  // 16-token anchors (h = 8 lb log2 e rounded to an integer, the half anchors
  // h and G_15 + h): per channel 2^{G_15 + h}, 2^{G_L - h}, 2^{G_L - G_15 - h},
  // 2^{G_15 - h}, so that each element needs only its two anchored factors
  // from the exponential unit and the rest are products with these
  float K16[4][D];
  float rq[CH], rk[CH];        // q/k L2-norm scales per token (1 without the front-end norm)
};
// Split-K partials of the six Mqk/Akk tiles, 16 bytes per (wave w, tile p,
// lane): entry e = 64 p + lane of wave w lies in the bytes [64 w, 64 w + 64)
// of the chunk's q, k and g rows -- the key channels 32w..32w+31, which only
// wave w reads (96 row segments of 64 bytes: array e / 128, row (e / 4) % 32)
// -- so each wave stores its partials as soon as its own products are done.
__device__ __forceinline__ float* part_entry(ChunkQKG& cr, int w, int p, int lane) {
  const int e = 64 * p + lane, seg = e >> 2;
  unsigned char* base = reinterpret_cast<unsigned char*>(&cr);
  return reinterpret_cast<float*>(base + (seg >> 5) * (int)sizeof(cr.q) + (seg & 31) * (RP * 2) +
                                  64 * w + 16 * (e & 3));
}
struct InvWork {
  float At[CH][CH + 4];        // (Diag(b) stril(Akk))^T, FP32; rows 16-byte aligned
  float Tf[CH][CH + 1];        // (I + A)^{-1}, FP32
  float X[16][17];             // W = T22 A21
};
static_assert(sizeof(InvWork) <= sizeof(float) * CH * GP, "inverse work must fit over G");

__device__ __forceinline__ InvWork& inv_of(PrepWork& pw) {
  return *reinterpret_cast<InvWork*>(&pw.G[0][0]);
}

typedef __attribute__((address_space(3))) void lds_void;

// Step 1: the chunk [t0, t0 + L) of head h -- its q, k, g rows and the value
// columns [col0, col0 + DVS) -- fetched into registers by 16-byte buffer
// loads (16 consecutive threads read one 256-byte row: coalesced), so that a
// block can load the next chunk while it works on the current one and write
// it to LDS (stage_chunk) at a point of its choosing.  The loads are range
// checked: rows t >= L read as zeros.  256 threads.
template <int DVS>
struct ChunkRegs {
  static constexpr int kV = DVS / 64;   // 16-byte pieces of the value rows per thread
  uint4 q[2], k[2], g[2], v[kV];
  uint16_t beta;
};

__device__ __forceinline__ uint4 load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

template <int DVS>
__device__ __forceinline__ void fetch_chunk(ChunkRegs<DVS>& x, const PrefillArgs& a, int t0, int L,
                                            int h, int col0, int tid) {
  const int H = a.num_heads;
  const int64_t base = ((int64_t)t0 * H + h) * D;
  const uint32_t rows_bytes = (uint32_t)(((L - 1) * H + 1) * D * 2);
  const uint32_t row_bytes = (uint32_t)H * D * 2;
  const __amdgpu_buffer_rsrc_t rq = make_buffer(a.q + base, rows_bytes);
  const __amdgpu_buffer_rsrc_t rk = make_buffer(a.k + base, rows_bytes);
  const __amdgpu_buffer_rsrc_t rg = make_buffer(a.g + base, rows_bytes);
  const __amdgpu_buffer_rsrc_t rv = make_buffer(a.v + base, rows_bytes);
#pragma unroll
  for (int i = 0; i < 2; ++i) {   // piece tid + 256 i: row / 16, 16-byte chunk % 16
    const int e = tid + 256 * i;
    const uint32_t off = (uint32_t)(e >> 4) * row_bytes + (uint32_t)(e & 15) * 16;
    x.q[i] = load16(rq, off);
    x.k[i] = load16(rk, off);
    x.g[i] = load16(rg, off);
  }
  constexpr int kCh = DVS / 8;    // 16-byte chunks per value row
#pragma unroll
  for (int i = 0; i < ChunkRegs<DVS>::kV; ++i) {
    const int e = tid + 256 * i;
    x.v[i] = load16(rv, (uint32_t)(e / kCh) * row_bytes + (uint32_t)col0 * 2 + (uint32_t)(e % kCh) * 16);
  }
  x.beta = a.beta[(int64_t)(t0 + min(tid & (CH - 1), L - 1)) * H + h];
}

// One part of fetch_chunk: PART 0 the q rows and beta, 1 the k rows, 2 the g
// rows, 3 the value rows, so that the loads can be spread over a step.
template <int PART, int DVS>
__device__ __forceinline__ void fetch_chunk_part(ChunkRegs<DVS>& x, const PrefillArgs& a, int t0, int L,
                                                 int h, int col0, int tid) {
  const int H = a.num_heads;
  const int64_t base = ((int64_t)t0 * H + h) * D;
  const uint32_t rows_bytes = (uint32_t)(((L - 1) * H + 1) * D * 2);
  const uint32_t row_bytes = (uint32_t)H * D * 2;
  if constexpr (PART < 3) {
    const uint16_t* src = PART == 0 ? a.q : PART == 1 ? a.k : a.g;
    const __amdgpu_buffer_rsrc_t r = make_buffer(src + base, rows_bytes);
    uint4* dst = PART == 0 ? x.q : PART == 1 ? x.k : x.g;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int e = tid + 256 * i;
      dst[i] = load16(r, (uint32_t)(e >> 4) * row_bytes + (uint32_t)(e & 15) * 16);
    }
    if (PART == 0) x.beta = a.beta[(int64_t)(t0 + min(tid & (CH - 1), L - 1)) * H + h];
  } else {
    constexpr int kCh = DVS / 8;
    const __amdgpu_buffer_rsrc_t rv = make_buffer(a.v + base, rows_bytes);
#pragma unroll
    for (int i = 0; i < ChunkRegs<DVS>::kV; ++i) {
      const int e = tid + 256 * i;
      x.v[i] = load16(rv, (uint32_t)(e / kCh) * row_bytes + (uint32_t)col0 * 2 + (uint32_t)(e % kCh) * 16);
    }
  }
}

// Writes the fetched rows into the padded q/k/g rows of `cr` and the value
// rows `v`.  256 threads.
template <int DVS>
__device__ __forceinline__ void stage_chunk(ChunkQKG& cr, uint16_t (&v)[CH][DVS],
                                            const ChunkRegs<DVS>& x, int tid) {
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int e = tid + 256 * i, t = e >> 4, c = (e & 15) * 8;
    *reinterpret_cast<uint4*>(&cr.q[t][c]) = x.q[i];
    *reinterpret_cast<uint4*>(&cr.k[t][c]) = x.k[i];
    *reinterpret_cast<uint4*>(&cr.g[t][c]) = x.g[i];
  }
  constexpr int kCh = DVS / 8;
#pragma unroll
  for (int i = 0; i < ChunkRegs<DVS>::kV; ++i) {
    const int e = tid + 256 * i;
    *reinterpret_cast<uint4*>(&v[e / kCh][(e % kCh) * 8]) = x.v[i];
  }
}

// The chunk's beta (zero for padding tokens), through the front-end's
// transform when it is compiled in.
template <bool FE>
__device__ __forceinline__ void stage_beta(float* beta, uint16_t beta_raw, const FrontEnd& fe,
                                           int L, int tid) {
  if (tid < CH) {
    const float b = tid < L ? bf16_to_f32(beta_raw) : 0.f;
    beta[tid] = FE && tid < L ? frontend_beta(fe, b) : b;
  }
}

// Step 1b (input front-end): 1 / sqrt(sum_c x_c^2 + norm_eps) of q and k per
// token of the staged chunk; eight threads per token, 16 channels each.
// Needs 256 threads (the producers); runs in the same phase as gate_prefix.
__device__ __forceinline__ void qk_norms(PrepWork& pw, const ChunkQKG& cr, const PrefillArgs& a,
                                         int tid) {
  const int t = tid >> 3, part = tid & 7;
  float sq2 = 0.f, sk2 = 0.f;
  if (a.fe.normalize_qk) {
#pragma unroll
    for (int c = 0; c < 16; ++c) {
      const float qv = bf16_to_f32(cr.q[t][16 * part + c]);
      const float kv = bf16_to_f32(cr.k[t][16 * part + c]);
      sq2 = fmaf(qv, qv, sq2);
      sk2 = fmaf(kv, kv, sk2);
    }
#pragma unroll
    for (int off = 1; off < 8; off <<= 1) {
      sq2 += __shfl_xor(sq2, off);
      sk2 += __shfl_xor(sk2, off);
    }
  }
  if (part == 0) {
    pw.rq[t] = a.fe.normalize_qk ? inv_norm(sq2 + a.fe.norm_eps) : 1.f;
    pw.rk[t] = a.fe.normalize_qk ? inv_norm(sk2 + a.fe.norm_eps) : 1.f;
  }
}

// Step 2: inclusive gate prefix per channel, chunk decay, and the anchor
// constants (fixed anchor: 2^{G_L - C}; 16-token anchors: the K16 factors).
// 512 threads, every wave of the fused block (the consumers' phase is
// otherwise idle): thread (wave w, lane l) sums 8 tokens, quarter q = l / 16,
// of key channel 16 w + l % 16, so each serial sum is 8 long; the quarters'
// totals come from the channel's three other lanes, and the last quarter's
// thread writes the decay and the constants.  Padding tokens (t >= L) add
// nothing: a transformed gate of their zero input would not be zero.
template <int MODE, bool FE>
__device__ __forceinline__ void gate_prefix(PrepWork& pw, float* dec, const ChunkQKG& cr,
                                            const FrontEnd& fe, float C, float Ch, int L, int tid) {
  const int lane = tid & 63, cl = lane & 15, q = lane >> 4;
  const int c = 16 * (tid >> 6) + cl;
  float pre[8];
  float acc = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int t = 8 * q + j;
    float x = bf16_to_f32(cr.g[t][c]);
    if (FE) x = t < L ? frontend_gate(fe, x) : 0.f;
    acc += x;
    pre[j] = acc;
  }
  float tq[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) tq[k] = __shfl(acc, cl + 16 * k);
  const float base = q == 0 ? 0.f : q == 1 ? tq[0] : q == 2 ? tq[0] + tq[1] : (tq[0] + tq[1]) + tq[2];
#pragma unroll
  for (int j = 0; j < 8; ++j) pw.G[8 * q + j][c] = (base + pre[j]) * kLog2e;
  if (q == 3) {
    const float GL = (base + acc) * kLog2e;
    dec[c] = fast_exp2(GL);
    if (MODE == 0) pw.EL[c] = fast_exp2(GL - C);
    if (MODE == 1) {
      const float G15 = (tq[0] + tq[1]) * kLog2e;
      pw.K16[0][c] = fast_exp2(G15 + Ch);
      pw.K16[1][c] = fast_exp2(GL - Ch);
      pw.K16[2][c] = fast_exp2(GL - G15 - Ch);
      // with the off-diagonal tile's column scale 2^z, z = floor(h / 2), folded in
      pw.K16[3][c] = fast_exp2(G15 - Ch) * __builtin_ldexpf(1.f, (int)Ch >> 1);
    }
  }
}

// Operands of one lane for the pairwise products: A rows (Qc, Kc') and B
// columns (Kc), hi and lo, for its two tokens (l%16 and l%16+16) and 8 key
// channels.  "o" variants feed the off-diagonal 16x16 tile.
struct PairOps {
  bf16x8 q0h, q0l, q1h, q1l, qoh, qol;
  bf16x8 k0h, k0l, k1h, k1l, koh, kol;
  bf16x8 b0h, b0l, b1h, b1l, boh, bol;
};

// Step 3: anchored operands and the split-K pairwise products.  Wave w (of 4)
// owns key channels 32w..32w+31; lane (g4, l16) owns channels 32w+8g4+j and
// tokens l16, l16+16.  For the 8 channels c0.. of each owned token t,
// emit(t, c0, kg, qg, kr) receives Kg = k 2^{G_t}, Qg = q 2^{G_t} and Kr =
// k 2^{G_L - G_t} in fp16 (from the anchored values times the anchor's
// remaining factor, or with data-dependent anchors from the raw k and q and
// their own exponentials), so the caller can store them.  Returns the six lower
// tiles of Mqk and Akk as partial sums over this wave's channels; the caller
// stores them (pair_store) once no producer reads the chunk's rows any more.
template <int MODE, bool FE, class Emit>
__device__ __forceinline__ void pair_products(f32x4 (&acc)[6], const PrepWork& pw,
                                              const ChunkQKG& cr, const PrefillArgs& a, float C,
                                              float exp2C, int wave, int lane, Emit&& emit) {
  const int l16 = lane & 15, g4 = lane >> 4;
  const int cb = 32 * wave, cl = 8 * g4;
  // 16-token anchors: the off-diagonal tile's rows reuse half 1's diagonal
  // operands (anchored at G_15 + h, h an integer), its half-0 columns carry
  // 2^{G_15 - G} 2^z (the 2^z in the channel constant), and the tile is
  // scaled back by 2^{h - z} afterwards (exact powers of two; z = floor(h / 2)
  // keeps the unscaled sums within 2^{|h|/2} of the products)
  const int hz = MODE == 1 ? (int)a.half_anchor_log2 : 0, zc = hz >> 1;
  const float accscale = __builtin_ldexpf(1.f, hz - zc);
  PairOps op;
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    const int t = l16 + 16 * half;
    const f32x4 G0 = *reinterpret_cast<const f32x4*>(&pw.G[t][cb + cl]);
    const f32x4 G1 = *reinterpret_cast<const f32x4*>(&pw.G[t][cb + cl + 4]);
    const uint4 qw = *reinterpret_cast<const uint4*>(&cr.q[t][cb + cl]);
    const uint4 kw = *reinterpret_cast<const uint4*>(&cr.k[t][cb + cl]);
    f32x4 Gs0, Gs1, GL0, GL1, EL0, EL1, Gf0, Gf1, Ka0, Ka1, Kb0, Kb1;
    const float rq = FE ? pw.rq[t] : 1.f, rk = FE ? pw.rk[t] : 1.f;
    if (MODE == 1) {
      Gs0 = *reinterpret_cast<const f32x4*>(&pw.G[15][cb + cl]);
      Gs1 = *reinterpret_cast<const f32x4*>(&pw.G[15][cb + cl + 4]);
      // half 0: the R and fo constants; half 1: the P and R constants
      Ka0 = *reinterpret_cast<const f32x4*>(&pw.K16[half ? 0 : 1][cb + cl]);
      Ka1 = *reinterpret_cast<const f32x4*>(&pw.K16[half ? 0 : 1][cb + cl + 4]);
      Kb0 = *reinterpret_cast<const f32x4*>(&pw.K16[half ? 2 : 3][cb + cl]);
      Kb1 = *reinterpret_cast<const f32x4*>(&pw.K16[half ? 2 : 3][cb + cl + 4]);
    } else if (MODE == 2) {
      Gs0 = *reinterpret_cast<const f32x4*>(&pw.G[15][cb + cl]);
      Gs1 = *reinterpret_cast<const f32x4*>(&pw.G[15][cb + cl + 4]);
      GL0 = *reinterpret_cast<const f32x4*>(&pw.G[CH - 1][cb + cl]);
      GL1 = *reinterpret_cast<const f32x4*>(&pw.G[CH - 1][cb + cl + 4]);
      // MODE 2: G at the half's first token (0 or 16) for the midpoint anchor
      Gf0 = *reinterpret_cast<const f32x4*>(&pw.G[16 * half][cb + cl]);
      Gf1 = *reinterpret_cast<const f32x4*>(&pw.G[16 * half][cb + cl + 4]);
    } else {
      EL0 = *reinterpret_cast<const f32x4*>(&pw.EL[cb + cl]);
      EL1 = *reinterpret_cast<const f32x4*>(&pw.EL[cb + cl + 4]);
    }
    const uint32_t qu[4] = {qw.x, qw.y, qw.z, qw.w};
    const uint32_t ku[4] = {kw.x, kw.y, kw.z, kw.w};
    f16x8 kg, qg, kr;   // Kg, Qg and Kr of the 8 channels
    // the anchored operand values, split into bf16 hi/lo pairs after the loop
    float xq[8], xk[8], xb[8], xqo[8], xko[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float Gv = j < 4 ? G0[j] : G1[j - 4];
      const float qf = rq * ((j & 1) ? bf16hi(qu[j >> 1]) : bf16lo(qu[j >> 1]));
      const float kf = rk * ((j & 1) ? bf16hi(ku[j >> 1]) : bf16lo(ku[j >> 1]));
      float ep, em, P, R, fo = 0.f;
      if (MODE == 0) {
        ep = fast_exp2(Gv - C);                       // 2^{G-C}, |exponent| <= 16|b|
        em = fast_exp2(C - Gv);                       // 2^{C-G}
        P = exp2C;                                    // Kg = (k 2^{G-C}) 2^C
        R = (j < 4 ? EL0[j] : EL1[j - 4]);            // Kr = (k 2^{C-G}) 2^{G_L-C}
      } else if (MODE == 1) {
        // anchor Ch = h (half 0) or G_15 + h (half 1), h = 8 lb log2 e rounded; the
        // factors below 2^-126 that a constant can lose belong to operands
        // far below fp16's range (they are zero either way)
        const float c1 = j < 4 ? Ka0[j] : Ka1[j - 4], c2 = j < 4 ? Kb0[j] : Kb1[j - 4];
        const float Ch = (half ? (j < 4 ? Gs0[j] : Gs1[j - 4]) : 0.f) + a.half_anchor_log2;
        ep = fast_exp2(Gv - Ch);
        em = fast_exp2(Ch - Gv);
        if (half) {
          P = c1;                                     // 2^{G_15 + h}
          R = c2;                                     // 2^{G_L - G_15 - h}
        } else {
          P = exp2C;                                  // 2^h
          R = c1;                                     // 2^{G_L - h}
          fo = c2;                                    // 2^{G_15 - h} 2^z
        }
      } else {
        const float g15 = j < 4 ? Gs0[j] : Gs1[j - 4];
        const float gl = j < 4 ? GL0[j] : GL1[j - 4];
        // midpoint of this half's actual range; exponents clamped so that a
        // half that decays a channel past 2^-252 stays finite
        const float gf = j < 4 ? Gf0[j] : Gf1[j - 4];
        const float Ch = 0.5f * (gf + (half ? gl : g15));
        ep = fast_exp2(__builtin_fminf(Gv - Ch, 126.f));
        em = fast_exp2(__builtin_fminf(Ch - Gv, 126.f));
        fo = half ? fast_exp2(Gv - g15) : fast_exp2(g15 - Gv);  // both <= 1
        P = fast_exp2(Gv);
        R = fast_exp2(gl - Gv);
      }
      xq[j] = qf * ep;
      xk[j] = kf * ep;
      xb[j] = kf * em;
      if (MODE == 2) {
        xqo[j] = qf * fo;
        xko[j] = kf * fo;
        kg[j] = static_cast<_Float16>(kf * P);
        qg[j] = static_cast<_Float16>(qf * P);
        kr[j] = static_cast<_Float16>(kf * R);
      } else {
        xqo[j] = 0.f;
        xko[j] = xb[j] * fo;
        kg[j] = static_cast<_Float16>(xk[j] * P);
        qg[j] = static_cast<_Float16>(xq[j] * P);
        kr[j] = static_cast<_Float16>(xb[j] * R);
      }
    }
#pragma unroll
    for (int j = 0; j < 8; j += 2) {
      if (half == 0) {
        split_bf16_pair(xq[j], xq[j + 1], op.q0h, op.q0l, j);
        split_bf16_pair(xk[j], xk[j + 1], op.k0h, op.k0l, j);
        split_bf16_pair(xb[j], xb[j + 1], op.b0h, op.b0l, j);
      } else {
        split_bf16_pair(xq[j], xq[j + 1], op.q1h, op.q1l, j);
        split_bf16_pair(xk[j], xk[j + 1], op.k1h, op.k1l, j);
        split_bf16_pair(xb[j], xb[j + 1], op.b1h, op.b1l, j);
      }
      if (MODE == 0) {
        // one anchor for the whole chunk: the off-diagonal tile reuses the diagonal operands
        if (half == 1) {
          op.qoh[j] = op.q1h[j]; op.qoh[j + 1] = op.q1h[j + 1];
          op.qol[j] = op.q1l[j]; op.qol[j + 1] = op.q1l[j + 1];
          op.koh[j] = op.k1h[j]; op.koh[j + 1] = op.k1h[j + 1];
          op.kol[j] = op.k1l[j]; op.kol[j + 1] = op.k1l[j + 1];
        } else {
          op.boh[j] = op.b0h[j]; op.boh[j + 1] = op.b0h[j + 1];
          op.bol[j] = op.b0l[j]; op.bol[j + 1] = op.b0l[j + 1];
        }
      } else if (half == 1) {
        if (MODE != 1) {   // MODE 1 uses half 1's diagonal operands
          split_bf16_pair(xqo[j], xqo[j + 1], op.qoh, op.qol, j);
          split_bf16_pair(xko[j], xko[j + 1], op.koh, op.kol, j);
        }
      } else {
        split_bf16_pair(xko[j], xko[j + 1], op.boh, op.bol, j);
      }
    }
    emit(t, cb + cl, kg, qg, kr);
  }
  const f32x4 z = {0.f, 0.f, 0.f, 0.f};
  acc[0] = mfma_bf16(op.q0h, op.b0h, z);
  acc[0] = mfma_bf16(op.q0h, op.b0l, acc[0]);
  acc[0] = mfma_bf16(op.q0l, op.b0h, acc[0]);
  const bf16x8& qoh = MODE == 1 ? op.q1h : op.qoh;
  const bf16x8& qol = MODE == 1 ? op.q1l : op.qol;
  const bf16x8& koh = MODE == 1 ? op.k1h : op.koh;
  const bf16x8& kol = MODE == 1 ? op.k1l : op.kol;
  acc[1] = mfma_bf16(qoh, op.boh, z);
  acc[1] = mfma_bf16(qoh, op.bol, acc[1]);
  acc[1] = mfma_bf16(qol, op.boh, acc[1]);
  acc[2] = mfma_bf16(op.q1h, op.b1h, z);
  acc[2] = mfma_bf16(op.q1h, op.b1l, acc[2]);
  acc[2] = mfma_bf16(op.q1l, op.b1h, acc[2]);
  acc[3] = mfma_bf16(op.k0h, op.b0h, z);
  acc[3] = mfma_bf16(op.k0h, op.b0l, acc[3]);
  acc[3] = mfma_bf16(op.k0l, op.b0h, acc[3]);
  acc[4] = mfma_bf16(koh, op.boh, z);
  acc[4] = mfma_bf16(koh, op.bol, acc[4]);
  acc[4] = mfma_bf16(kol, op.boh, acc[4]);
  acc[5] = mfma_bf16(op.k1h, op.b1h, z);
  acc[5] = mfma_bf16(op.k1h, op.b1l, acc[5]);
  acc[5] = mfma_bf16(op.k1l, op.b1h, acc[5]);
  if (MODE == 1) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc[1][i] *= accscale;
      acc[4][i] *= accscale;
    }
  }
}

// Data-dependent anchors (no gate bound): a 16-token half whose gate prefix
// falls by more than kSteepRange (log2 units, about 160.8 nats) in some
// channel cannot be anchored once (its factors, up to half the fall at the
// midpoint anchor, would exceed the 2^116 budget within which the operands'
// bf16 low halves keep their precision).  steep_wave tells, for the channels
// of this producer wave, whether any half of the chunk is that steep
// (wave-uniform).
constexpr float kSteepRange = 232.f;
__device__ __forceinline__ bool steep_wave(const PrepWork& pw, int wave, int lane) {
  bool steep = false;
  if ((lane & 15) < 2) {          // lane l16 = h checks half h of its row's 8 channels
    const int h = lane & 1, c0 = 32 * wave + 8 * (lane >> 4);
#pragma unroll
    for (int j = 0; j < 8; ++j) steep |= pw.G[16 * h][c0 + j] - pw.G[16 * h + 15][c0 + j] > kSteepRange;
  }
  return __builtin_amdgcn_ballot_w64(steep) != 0;
}

// The pairwise products for a wave whose channels have a steep half
// (steep_wave), exact to the usual rounding while no 8-token quarter falls by
// more than 2^232: each diagonal 16x16 tile is the sum of three products over
// the quarters Q0 (tokens 0-7 of the half) and Q1 (8-15),
//   Q0 x Q0 anchored at the middle of Q0's range,
//   Q1 x Q1 anchored at the middle of Q1's range,
//   Q1 x Q0 through the prefix at the quarters' boundary (factors <= 1),
// so no factor exceeds half of one quarter's range; the off-diagonal tile
// goes through the prefix at token 15 as in pair_products.  Lane (g4, l16)
// supplies row l16 and column l16 of a tile, so one mask per lane (its
// token's quarter) selects its part of each product.  Same interface as
// pair_products (MODE 2).
template <bool FE, class Emit>
__device__ __forceinline__ void pair_products_steep(f32x4 (&acc)[6], const PrepWork& pw,
                                                    const ChunkQKG& cr, int wave, int lane,
                                                    Emit&& emit) {
  const int l16 = lane & 15, g4 = lane >> 4;
  const int cb = 32 * wave, cl = 8 * g4;
  const bool q1 = l16 >= 8;       // this lane's token is in the second quarter of its half
  const f32x4 z = {0.f, 0.f, 0.f, 0.f};
  auto mfma3 = [&](const bf16x8& ah, const bf16x8& al, const bf16x8& bh, const bf16x8& bl,
                   f32x4 c) __attribute__((always_inline)) {
    c = mfma_bf16(ah, bh, c);
    c = mfma_bf16(ah, bl, c);
    return mfma_bf16(al, bh, c);
  };
  bf16x8 boh, bol;   // half 0 column operands of the off-diagonal tile
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    const int t = l16 + 16 * half, hb = 16 * half;
    const uint4 qw = *reinterpret_cast<const uint4*>(&cr.q[t][cb + cl]);
    const uint4 kw = *reinterpret_cast<const uint4*>(&cr.k[t][cb + cl]);
    const uint32_t qu[4] = {qw.x, qw.y, qw.z, qw.w};
    const uint32_t ku[4] = {kw.x, kw.y, kw.z, kw.w};
    const float rq = FE ? pw.rq[t] : 1.f, rk = FE ? pw.rk[t] : 1.f;
    auto qf_of = [&](int j) __attribute__((always_inline)) {
      return rq * ((j & 1) ? bf16hi(qu[j >> 1]) : bf16lo(qu[j >> 1]));
    };
    auto kf_of = [&](int j) __attribute__((always_inline)) {
      return rk * ((j & 1) ? bf16hi(ku[j >> 1]) : bf16lo(ku[j >> 1]));
    };
    const int im = half ? 2 : 0, ia = half ? 5 : 3;   // diagonal tiles of Mqk and Akk
#pragma unroll
    for (int qq = 0; qq < 2; ++qq) {
      // Qqq x Qqq anchored at the middle of quarter qq's range; lanes of the
      // other quarter supply zeros
      const bool mine = q1 == (qq == 1);
      bf16x8 qah, qal, kah, kal, bah, bal;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int c = cb + cl + j;
        const float Gv = pw.G[t][c];
        const float Ca = 0.5f * (pw.G[hb + 8 * qq][c] + pw.G[hb + 8 * qq + 7][c]);
        const float rowA = mine ? fast_exp2(Gv - Ca) : 0.f;
        const float colA = mine ? fast_exp2(Ca - Gv) : 0.f;
        __bf16 h, l;
        split_bf16(qf_of(j) * rowA, h, l); qah[j] = h; qal[j] = l;
        split_bf16(kf_of(j) * rowA, h, l); kah[j] = h; kal[j] = l;
        split_bf16(kf_of(j) * colA, h, l); bah[j] = h; bal[j] = l;
      }
      acc[im] = mfma3(qah, qal, bah, bal, qq ? acc[im] : z);
      acc[ia] = mfma3(kah, kal, bah, bal, qq ? acc[ia] : z);
      __builtin_amdgcn_sched_barrier(0);   // one pass's operands live at a time
    }
    {
      // Q1 x Q0 through the prefix at the quarters' boundary: rows of Q1, columns of Q0
      bf16x8 q3h, q3l, k3h, k3l, b3h, b3l;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int c = cb + cl + j;
        const float Gv = pw.G[t][c], G7 = pw.G[hb + 7][c];
        const float e3 = fast_exp2(q1 ? Gv - G7 : G7 - Gv);   // <= 1 either way
        const float qf = qf_of(j), kf = kf_of(j);
        __bf16 h, l;
        split_bf16(q1 ? qf * e3 : 0.f, h, l); q3h[j] = h; q3l[j] = l;
        split_bf16(q1 ? kf * e3 : 0.f, h, l); k3h[j] = h; k3l[j] = l;
        split_bf16(q1 ? 0.f : kf * e3, h, l); b3h[j] = h; b3l[j] = l;
      }
      acc[im] = mfma3(q3h, q3l, b3h, b3l, acc[im]);
      acc[ia] = mfma3(k3h, k3l, b3h, b3l, acc[ia]);
    }
    __builtin_amdgcn_sched_barrier(0);
    {
      // the off-diagonal tile's operands (through the prefix at token 15) and Kg, Qg, Kr
      bf16x8 qoh, qol, koh, kol;
      f16x8 kg, qg, kr;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int c = cb + cl + j;
        const float Gv = pw.G[t][c], g15 = pw.G[15][c], gl = pw.G[CH - 1][c];
        const float qf = qf_of(j), kf = kf_of(j);
        const float fo = half ? fast_exp2(Gv - g15) : fast_exp2(g15 - Gv);
        __bf16 h, l;
        if (half == 1) {
          split_bf16(qf * fo, h, l); qoh[j] = h; qol[j] = l;
          split_bf16(kf * fo, h, l); koh[j] = h; kol[j] = l;
        } else {
          split_bf16(kf * fo, h, l); boh[j] = h; bol[j] = l;
        }
        const float P = fast_exp2(Gv), R = fast_exp2(gl - Gv);
        kg[j] = static_cast<_Float16>(kf * P);
        qg[j] = static_cast<_Float16>(qf * P);
        kr[j] = static_cast<_Float16>(kf * R);
      }
      emit(t, cb + cl, kg, qg, kr);
      if (half == 1) {
        acc[1] = mfma3(qoh, qol, boh, bol, z);
        acc[4] = mfma3(koh, kol, boh, bol, z);
      }
    }
  }
}

// Stores this wave's partials over its own key-channel columns of the rows
// (part_entry); call after its last read of the rows.
__device__ __forceinline__ void pair_store(ChunkQKG& cr, const f32x4 (&acc)[6], int wave, int lane) {
#pragma unroll
  for (int p = 0; p < 6; ++p) *reinterpret_cast<f32x4*>(part_entry(cr, wave, p, lane)) = acc[p];
}

// A wave's own LDS accesses in program order: its writes before this point
// are seen by the reads of any of its lanes after it (one wave's LDS
// operations are performed in order; the fences keep the compiler from
// moving accesses across).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
}

// Sum of the four split-K partials of tile p, in a fixed order, for MFMA lane
// `lane` (rows 4 (lane / 16) + i of column lane % 16 of the tile).
__device__ __forceinline__ f32x4 sum_partials(ChunkQKG& cr, int p, int lane) {
  auto rd = [&](int w) __attribute__((always_inline)) {
    return *reinterpret_cast<const f32x4*>(part_entry(cr, w, p, lane));
  };
  return ((rd(0) + rd(1)) + rd(2)) + rd(3);
}

// Step 3b for Mqk on two waves: wave 0 sums the diagonal tiles (rows/columns
// 0-15 and 16-31) from their partials and emits the zero block (rows 0-15 x
// columns 16-31), wave 1 the tile of rows 16-31 x columns 0-15; the causal
// triangle is masked by select (masked anchored entries may be inf or NaN).
// emit_mqk(r, s, value) sees each entry.
template <class EmitMqk>
__device__ __forceinline__ void reduce_mqk(ChunkQKG& cr, int w, int lane, EmitMqk&& emit_mqk) {
#pragma unroll
  for (int p = 0; p < 3; ++p) {
    if ((p == 1) != (w == 1)) continue;
    const f32x4 mq = sum_partials(cr, p, lane);
    const int r0 = (p == 0 ? 0 : 16) + 4 * (lane >> 4), s = (p == 2 ? 16 : 0) + (lane & 15);
#pragma unroll
    for (int i = 0; i < 4; ++i) emit_mqk(r0 + i, s, s <= r0 + i ? mq[i] : 0.f);
    if (p == 0) {
#pragma unroll
      for (int i = 0; i < 4; ++i) emit_mqk(r0 + i, s + 16, 0.f);
    }
  }
}

// Steps 3b-4a for the triangular system, on two waves: wave `blk` sums its
// lower blocks of A = Diag(b) stril(Akk) from their partials (as Mqk's) into
// iw.At (A transposed, FP32) and solves with them.  With T11, T22 the
// inverses of the 16x16 diagonal blocks of I + A and A21 its lower-left
// block, T21 = -T22 A21 T11 = -W T11, W = T22 A21.  Wave 0 (block A11):
// lanes 0-15 invert I + A11, lane m forming column m of T11 from e_m.  Wave
// 1 (blocks A21, A22): lanes 0-15 invert I + A22 and lanes 16-31 solve
// (I + A22) W = A21 from column m of A21, so W needs no wait for T22.
// Forward substitution in FP32 with the block's strict lower triangle read
// into registers first, so the 16 dependent steps wait on no LDS read; the
// wave's other lanes repeat a solve and store nothing.  The blocks pass
// between the wave's lanes through LDS in the wave's own order.  emit_t(row,
// col, value) receives T11 and T22; T21 follows from iw.X and iw.Tf
// (invert_offdiag, after a block barrier); T12 = 0 is the caller's, once.
template <class EmitT>
__device__ __forceinline__ void reduce_invert(InvWork& iw, ChunkQKG& cr, const float* beta, int blk,
                                              int lane, EmitT&& emit_t) {
  // A's tiles 3 + q: (0,0) for wave 0, (1,0) and (1,1) for wave 1; At's
  // block (0,1) is never read
#pragma unroll
  for (int q = 0; q < 3; ++q) {
    if ((q == 0) != (blk == 0)) continue;
    const f32x4 ak = sum_partials(cr, 3 + q, lane);
    const int r0 = (q == 0 ? 0 : 16) + 4 * (lane >> 4), s = (q == 2 ? 16 : 0) + (lane & 15);
    f32x4 at;
#pragma unroll
    for (int i = 0; i < 4; ++i) at[i] = s < r0 + i ? beta[r0 + i] * ak[i] : 0.f;
    *reinterpret_cast<f32x4*>(&iw.At[s][r0]) = at;
  }
  wave_lds_sync();
  const int grp = lane >> 4, m = lane & 15;
  const bool w21 = blk == 1 && grp >= 1;
  const int base = blk == 0 ? 0 : 16;
  float x[16];
  if (w21) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const f32x4 a = *reinterpret_cast<const f32x4*>(&iw.At[m][16 + 4 * q]);
#pragma unroll
      for (int r = 0; r < 4; ++r) x[4 * q + r] = a[r];
    }
  } else {
#pragma unroll
    for (int i = 0; i < 16; ++i) x[i] = i == m ? 1.f : 0.f;
  }
  // column j of the block below the diagonal = row j of At; quads q >= j / 4
  // hold rows i > j.  Two rounds of eight columns (28 and 12 quads), so the
  // registers for the triangle stay within the wave's budget.
#pragma unroll
  for (int j0 = 0; j0 < 16; j0 += 8) {
    f32x4 c[8][4];
#pragma unroll
    for (int j = j0; j < j0 + 8; ++j)
#pragma unroll
      for (int q = j >> 2; q < 4; ++q)
        c[j - j0][q] = *reinterpret_cast<const f32x4*>(&iw.At[base + j][base + 4 * q]);
#pragma unroll
    for (int j = j0; j < j0 + 8; ++j)
#pragma unroll
      for (int i = j + 1; i < 16; ++i) x[i] = fmaf(-c[j - j0][i >> 2][i & 3], x[j], x[i]);
    __builtin_amdgcn_sched_barrier(0);
  }
  if (grp == 0) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      iw.Tf[base + i][base + m] = x[i];
      emit_t(base + i, base + m, x[i]);
    }
  } else if (blk == 1 && grp == 1) {
#pragma unroll
    for (int i = 0; i < 16; ++i) iw.X[i][m] = x[i];
  }
}

// Step 4b: T21 = -W T11 as four 16x16x4 FP32 matrix products (K = 16): in
// step kk lane l supplies W[l % 16][4 kk + l / 16] and T11[4 kk + l / 16][l %
// 16] and ends with T21[4 (l / 16) + i][l % 16], i < 4.  One wave.
template <class EmitT>
__device__ __forceinline__ void invert_offdiag(const InvWork& iw, int lane, EmitT&& emit_t) {
  const int r = lane & 15, kq = lane >> 4;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kk = 0; kk < 4; ++kk)
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(iw.X[r][4 * kk + kq], iw.Tf[4 * kk + kq][r], acc, 0, 0, 0);
#pragma unroll
  for (int i = 0; i < 4; ++i) emit_t(16 + 4 * kq + i, r, -acc[i]);
}

}  // namespace chunk
}  // namespace kda
