// Chunk-32 KDA prefill on gfx950 matrix cores.
//
// The per-chunk algorithm is the seven-step pipeline of "FlashInfer PR #4262:
// CAKE KDA Prefill Highlights", section 2, with the fixed exponent anchor of
// section 1.  For a chunk of 32 tokens starting from state S0 (dk x dv, FP32)
// and the log2-domain inclusive gate prefix G_r = log2(e) sum_{s<=r} g_s:
//   Mqk = tril(Qc Kc^T),  A = Diag(b) stril(Kc' Kc^T)          (anchored products)
//   T   = (I + A)^{-1}                                          (unit lower inverse)
//   W   = Kg S0,   O0 = Qg S0                                   (state projection)
//   U   = T Diag(b) (V - W)                                     (residual/beta)
//   S1  = Diag(2^{G_L}) S0 + Kr^T U,   O = scale (O0 + Mqk U)   (fused update)
// with Qc = q 2^{G-C}, Kc' = k 2^{G-C}, Kc = k 2^{C-G}, C = 16 lb log2(e),
// Kg = k 2^G, Qg = q 2^G, Kr[s] = k_s 2^{G_L - G_s}.  When 16|lb|log2(e) > 126
// the anchored operands would leave the bf16/fp32 exponent range, so the
// pairwise products are formed per 16-token half instead (diagonal blocks
// anchored at the prefix before the half plus 8 lb log2(e), the off-diagonal
// block factored through the prefix at the split point, whose factors are all
// <= 1): the note's "ordinary SafeGate" 16-token blocks.
//
// Number formats (chosen so the FP32-state result stays within 1e-2 RMS of
// the exact recurrence at the largest state entries; bf16 alone loses up to
// 2^-8 per rounding and the state is heavy-tailed):
//   * Mqk / Akk: bf16 operands split hi + lo, three products (hi.hi + hi.lo +
//     lo.hi) on v_mfma_f32_16x16x32_bf16 -- the anchored operands need bf16's
//     exponent range;
//   * every other product: fp16 operands (11-bit significand, same MFMA rate)
//     on v_mfma_f32_16x16x32_f16; V' and U enter as hi + lo fp16 pairs;
//   * gate prefix, inverse, decay and all accumulators in FP32.
// fp16 operands assume |v| < 2^15 and unit-norm keys/queries, as in KDA.
//
// Work decomposition.  One block of 4 waves per (sequence, head, value slice
// of DVS = 64 * NT columns).  Per chunk the four waves first prepare the
// chunk together (wave w owns key channels 32w..32w+31 of the pairwise
// products and of the operand preparation, a split-K whose partials are summed
// in a fixed order, so results are deterministic), then each wave runs the
// serial state chain on its own 16 * NT value columns: value columns evolve
// independently, so the chain needs no cross-wave exchange.  The state stays
// in the MFMA accumulators for the whole sequence.
//
// Accumulator-to-operand reuse.  An accumulator tile of v_mfma_f32_16x16x32
// gives lane l the rows 4(l/16)+i (i < 4) of column l%16, while the B operand
// wants 8 K-values per lane.  Two vertically adjacent tiles give lane l the
// rows {4(l/16)+i, 16+4(l/16)+i}; using that set as the lane's 8 K-slots (a
// fixed permutation of the 32-long K index applied to both operands) turns
// the FP32 state, V' and U into the next product's B operand with a register
// conversion only.  The A operands (Kg, Qg, Kr^T, T, Mqk) are therefore
// stored in LDS with their K index in that permuted order.
#include <cmath>

#include "chunk_common.h"

namespace kda {
namespace {

using namespace chunk;

template <int DVS>
struct FusedSmem {
  PrepSmem<DVS> p;
  _Float16 Kg[CH][RP];         // k 2^G      [token][dk, permuted]
  _Float16 Qg[CH][RP];         // q 2^G      [token][dk, permuted]
  _Float16 KrT[D][TP];         // (k 2^{G_L-G})^T [dk][token, permuted]
  _Float16 T[CH][TP];          // (I + A)^{-1}     [token][token, permuted]
  _Float16 Mqk[CH][TP];        // causal Mqk       [token][token, permuted]
};

// Blocks start in index order as compute units free up, and a block holds a
// compute unit for its whole sequence, so the sequence a block works on is
// taken in longest-first order (ties by index): in a varlen batch a long
// sequence otherwise may only start in the last round of blocks and end
// alone.  Returns the sequence of rank r by (length descending, index
// ascending); `tmp` is LDS scratch of at least N + 1 ints, free on entry and
// on return.  256 threads; contains barriers.
constexpr int kLongestFirstMaxSeqs = 256;

__device__ __forceinline__ int longest_first_sequence(const PrefillArgs& a, int r, int* tmp,
                                                      int tid) {
  const int N = a.num_seqs;
  for (int i = tid; i < N; i += 256) {
    const int b = clamp_offset(a.cu_seqlens[i], a.total_tokens);
    tmp[i] = max(b, clamp_offset(a.cu_seqlens[i + 1], a.total_tokens)) - b;
  }
  __syncthreads();
  for (int i = tid; i < N; i += 256) {
    const int li = tmp[i];
    int rank = 0;
    for (int m = 0; m < N; ++m) {
      const int lm = tmp[m];
      rank += (lm > li || (lm == li && m < i)) ? 1 : 0;
    }
    if (rank == r) tmp[N] = i;   // the ranks are a permutation: exactly one i
  }
  __syncthreads();
  const int n = tmp[N];
  __syncthreads();
  return n;
}

template <int MODE, int NT, bool FE>
__global__ __launch_bounds__(256) void prefill_chunk_kernel(PrefillArgs a, float exp2C) {
  constexpr int DVS = 64 * NT;
  extern __shared__ __align__(16) unsigned char smem_raw[];
  FusedSmem<DVS>& sm = *reinterpret_cast<FusedSmem<DVS>*>(smem_raw);
  PrepSmem<DVS>& ps = sm.p;

  const int H = a.num_heads;
  const int slice = blockIdx.x, h = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // the sequence of rank blockIdx.z, longest first (the split-K partials'
  // area is not in use yet)
  int* const rank_tmp = reinterpret_cast<int*>(&ps.part[0][0][0][0]);
  const int n = (a.num_seqs > 1 && a.num_seqs <= kLongestFirstMaxSeqs)
                    ? longest_first_sequence(a, blockIdx.z, rank_tmp, tid)
                    : (int)blockIdx.z;
  const int l16 = lane & 15, g4 = lane >> 4;
  const int col_base = slice * DVS;
  const int colw = wave * 16 * NT;          // first column of this wave, within the slice
  const float C = a.anchor_log2;

  const int bos = clamp_offset(a.cu_seqlens[n], a.total_tokens);
  const int eos = max(bos, clamp_offset(a.cu_seqlens[n + 1], a.total_tokens));
  const StateRef s0 = prefill_initial_state(a, n, h);

  // State accumulators: tile (mt, nt) holds rows 16 mt + 4 g4 + i and column
  // col_base + colw + 16 nt + l16.
  f32x4 S[8][NT];
  auto init_state = [&](auto load) __attribute__((always_inline)) {
#pragma unroll
    for (int mt = 0; mt < 8; ++mt)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          S[mt][nt][i] = load((16 * mt + 4 * g4 + i) * D + col_base + colw + 16 * nt + l16);
  };
  // one branch on the state's type, outside the element loops
  if (!s0)
    init_state([](int) { return 0.f; });
  else if (s0.bf16)
    init_state([&](int e) { return bf16_to_f32(static_cast<const uint16_t*>(s0.p)[e]); });
  else
    init_state([&](int e) { return static_cast<const float*>(s0.p)[e]; });
  auto store_state = [&](float* dst) __attribute__((always_inline)) {
#pragma unroll
    for (int mt = 0; mt < 8; ++mt)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          dst[(16 * mt + 4 * g4 + i) * D + col_base + colw + 16 * nt + l16] = S[mt][nt][i];
  };

  // The next chunk's inputs are fetched (straight into the other of the two
  // raw buffers) while the current one is prepared and consumed, so their
  // load latency is off the per-chunk path.
  uint16_t beta_raw = 0;
  if (bos < eos) fetch_chunk(ps.raw[0], beta_raw, a, bos, min(CH, eos - bos), h, col_base, tid);
  int buf = 0;
  for (int t0 = bos; t0 < eos; t0 += CH, buf ^= 1) {
    const int L = min(CH, eos - t0);
    const ChunkRaw<DVS>& cr = ps.raw[buf];
    fetch_wait();
    // The chunk has landed in raw[buf]; the previous chunk's steps are done
    // with raw[buf ^ 1] and with the LDS operands.
    __syncthreads();
    stage_beta<DVS, FE>(ps, beta_raw, a.fe, L, tid);
    if (t0 + CH < eos)
      fetch_chunk(ps.raw[buf ^ 1], beta_raw, a, t0 + CH, min(CH, eos - t0 - CH), h, col_base, tid);
    gate_prefix<MODE, 64 * NT, FE>(ps, cr, a.fe, C, L, tid);
    if (FE) qk_norms(ps, cr, a, tid);
    __syncthreads();
    pair_products<MODE, 64 * NT, FE>(ps, cr, a, C, exp2C, wave, lane,
                        [&](int t, int c0, const float* kv, const float* qv, const float* P,
                            const float* R) {
                          const int cb = c0 & ~31, cl = c0 & 31;
                          f16x4 kg_lo, kg_hi, qg_lo, qg_hi;
#pragma unroll
                          for (int j = 0; j < 4; ++j) {
                            kg_lo[j] = static_cast<_Float16>(kv[j] * P[j]);
                            kg_hi[j] = static_cast<_Float16>(kv[4 + j] * P[4 + j]);
                            qg_lo[j] = static_cast<_Float16>(qv[j] * P[j]);
                            qg_hi[j] = static_cast<_Float16>(qv[4 + j] * P[4 + j]);
                          }
#pragma unroll
                          for (int j = 0; j < 8; ++j)
                            sm.KrT[c0 + j][kslot(t)] = static_cast<_Float16>(kv[j] * R[j]);
                          // channels cl..cl+3 and cl+4..cl+7 land in two runs of 4 slots
                          *reinterpret_cast<f16x4*>(&sm.Kg[t][cb + kslot(cl)]) = kg_lo;
                          *reinterpret_cast<f16x4*>(&sm.Kg[t][cb + kslot(cl + 4)]) = kg_hi;
                          *reinterpret_cast<f16x4*>(&sm.Qg[t][cb + kslot(cl)]) = qg_lo;
                          *reinterpret_cast<f16x4*>(&sm.Qg[t][cb + kslot(cl + 4)]) = qg_hi;
                        });
    __syncthreads();
    // ---- the state chain, first part (this wave's 16 * NT value columns):
    // W = Kg S and O = Qg S need only the operands written so far, so their
    // MFMAs run here, beside the latency-bound reduction and inverse.
    f16x8 Sb[4][NT];
#pragma unroll
    for (int p = 0; p < 4; ++p)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          Sb[p][nt][i] = static_cast<_Float16>(S[2 * p][nt][i]);
          Sb[p][nt][4 + i] = static_cast<_Float16>(S[2 * p + 1][nt][i]);
        }
    const f32x4 z = {0.f, 0.f, 0.f, 0.f};
    f32x4 W[2][NT], O[2][NT];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) { W[mt][nt] = z; O[mt][nt] = z; }
#pragma unroll
    for (int p = 0; p < 4; ++p)
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        const f16x8 akg = *reinterpret_cast<const f16x8*>(&sm.Kg[16 * mt + l16][32 * p + 8 * g4]);
        const f16x8 aqg = *reinterpret_cast<const f16x8*>(&sm.Qg[16 * mt + l16][32 * p + 8 * g4]);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          W[mt][nt] = mfma_f16(akg, Sb[p][nt], W[mt][nt]);
          O[mt][nt] = mfma_f16(aqg, Sb[p][nt], O[mt][nt]);
        }
      }
    // V' = b (V - W) as hi + lo fp16 B operands (K = token, permuted)
    f16x8 Vh[NT], Vl[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int t = 16 * mt + 4 * g4 + i;
          const float vp =
              ps.beta[t] * (bf16_to_f32(cr.v[t][colw + 16 * nt + l16]) - W[mt][nt][i]);
          _Float16 hh, ll;
          split_f16(vp, hh, ll);
          Vh[nt][4 * mt + i] = hh;
          Vl[nt][4 * mt + i] = ll;
        }
    reduce_pairs(ps, tid, [&](int r, int s, float m) {
      sm.Mqk[r][kslot(s)] = static_cast<_Float16>(m);
    });
    __syncthreads();
    invert_unit_lower(ps, tid, [&](int r, int s, float t) {
      sm.T[r][kslot(s)] = static_cast<_Float16>(t);
    });
    __syncthreads();

    // ---- the rest of the state chain on this wave's 16 * NT value columns
    {
      f32x4 U[2][NT];
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        const f16x8 at = *reinterpret_cast<const f16x8*>(&sm.T[16 * mt + l16][8 * g4]);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          U[mt][nt] = mfma_f16(at, Vh[nt], z);
          U[mt][nt] = mfma_f16(at, Vl[nt], U[mt][nt]);
        }
      }
      f16x8 Uh[NT], Ul[NT];
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            _Float16 hh, ll;
            split_f16(U[mt][nt][i], hh, ll);
            Uh[nt][4 * mt + i] = hh;
            Ul[nt][4 * mt + i] = ll;
          }
      // S = Diag(2^{G_L}) S + Kr^T U
#pragma unroll
      for (int mt = 0; mt < 8; ++mt) {
        const f16x8 akr = *reinterpret_cast<const f16x8*>(&sm.KrT[16 * mt + l16][8 * g4]);
        const f32x4 d = *reinterpret_cast<const f32x4*>(&ps.dec[16 * mt + 4 * g4]);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
#pragma unroll
          for (int i = 0; i < 4; ++i) S[mt][nt][i] *= d[i];
          S[mt][nt] = mfma_f16(akr, Uh[nt], S[mt][nt]);
          S[mt][nt] = mfma_f16(akr, Ul[nt], S[mt][nt]);
        }
      }
      // O = scale (O0 + Mqk U)
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        const f16x8 am = *reinterpret_cast<const f16x8*>(&sm.Mqk[16 * mt + l16][8 * g4]);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          O[mt][nt] = mfma_f16(am, Uh[nt], O[mt][nt]);
          O[mt][nt] = mfma_f16(am, Ul[nt], O[mt][nt]);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int t = 16 * mt + 4 * g4 + i;
            if (t < L)
              a.out[((int64_t)(t0 + t) * H + h) * D + col_base + colw + 16 * nt + l16] =
                  f32_to_bf16(a.scale * O[mt][nt][i]);
          }
        }
      }
    }
    if (float* cp = prefill_checkpoint(a, n, h, bos, t0 + L - bos)) store_state(cp);
  }

  if (const StateRef s1 = prefill_final_state(a, n, h)) {
    if (!s1.bf16) {
      store_state(static_cast<float*>(s1.p));
    } else {
      uint16_t* dst = static_cast<uint16_t*>(s1.p);
#pragma unroll
      for (int mt = 0; mt < 8; ++mt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            dst[(16 * mt + 4 * g4 + i) * D + col_base + colw + 16 * nt + l16] = f32_to_bf16(S[mt][nt][i]);
    }
  }
}

template <int MODE, int NT, bool FE>
hipError_t launch_variant(const PrefillArgs& a, hipStream_t s) {
  constexpr size_t bytes = sizeof(FusedSmem<64 * NT>);
  static_assert(bytes <= 160 * 1024, "the fused kernel's LDS exceeds a compute unit's 160 KiB");
  static bool attr_set = false;   // idempotent; a race only repeats the call
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&prefill_chunk_kernel<MODE, NT, FE>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  const float exp2C = MODE == 0 ? std::exp2(a.anchor_log2) : 0.f;
  prefill_chunk_kernel<MODE, NT, FE>
      <<<dim3(2 / NT, a.num_heads, a.num_seqs), 256, bytes, s>>>(a, exp2C);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill_chunk(const PrefillArgs& a, int anchor_mode, int dv_split,
                                hipStream_t s) {
  if (a.num_seqs <= 0) return hipSuccess;
  if (dv_split != 1 && dv_split != 2) return hipErrorInvalidValue;
  const int nt = dv_split == 1 ? 2 : 1;
  // data-dependent anchors and the input front-end: 64-column blocks only
  // (their 128-column variants would exceed the register file)
  if ((anchor_mode == 2 || frontend_active(a.fe)) && dv_split != 2) return hipErrorInvalidValue;
  if (frontend_active(a.fe)) {
    if (anchor_mode == 0) return launch_variant<0, 1, true>(a, s);
    if (anchor_mode == 2) return launch_variant<2, 1, true>(a, s);
    return launch_variant<1, 1, true>(a, s);
  }
  if (anchor_mode == 0) return nt == 2 ? launch_variant<0, 2, false>(a, s) : launch_variant<0, 1, false>(a, s);
  if (anchor_mode == 2) return launch_variant<2, 1, false>(a, s);
  return nt == 2 ? launch_variant<1, 2, false>(a, s) : launch_variant<1, 1, false>(a, s);
}

}  // namespace kda
