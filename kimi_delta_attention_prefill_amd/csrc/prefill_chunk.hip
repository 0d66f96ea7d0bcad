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
// Kg = k 2^G, Qg = q 2^G, Kr[s] = k_s 2^{G_L - G_s}.  When 16|lb|log2(e) > 116
// the anchored operands' bf16 low halves would lose their precision, so the
// pairwise products are formed per 16-token half instead (diagonal blocks
// anchored at the prefix before the half plus 8 lb log2(e) rounded to an
// integer, the off-diagonal block factored through the prefix at the split
// point, whose factors are all <= 1): the note's "ordinary SafeGate" 16-token
// blocks.
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
// Work decomposition.  One block of 8 waves per (sequence, head, value slice
// of DVS = 64 * NT columns), organised as the producer/consumer pipeline of
// the note's sections 3-4 (a ring of prepared chunks between the waves that
// prepare chunks and the waves that consume them), sized for a CDNA4 compute
// unit's 160 KiB of LDS:
//   * waves 4-7 (producers) prepare chunk c+1 -- anchored operands, Mqk and
//     the triangular system and its inverse -- into ring slot (c+1) % 2 (wave
//     w owns key channels 32(w-4).. of the pairwise products, a split-K whose
//     partials are summed in a fixed order, so results are deterministic;
//     then two waves sum the system's blocks and form T11, T22 and W = T22
//     A21 while the others sum Mqk's), and fetch the rows of chunk c+2 into
//     registers, writing them to LDS at the step's end;
//   * waves 0-3 (consumers) meanwhile run the serial state chain of chunk c
//     from slot c % 2 on their own 16 * NT value columns (value columns
//     evolve independently, so the chain needs no cross-wave exchange); the
//     FP32 state stays in their MFMA accumulators for the whole sequence.
//     In the phases where the chain has nothing to do they take half of
//     chunk c+1's gate prefix and (one wave) the inverse's off-diagonal block
//     T21 = -W T11 (four FP32 matrix products).
// Both sides meet at the same four block barriers per chunk (barriers that
// order LDS only, so prefetches and output stores stay in flight across
// them), and the chain's products with the state (matrix-core work) sit in
// the phase of the producers' VALU-bound pair products, so a chunk costs
// about the longer of the two sides rather than their sum.  LDS per block
// (DVS = 128): two raw q/k/g buffers (2 x 25.5 KiB; the split-K partials of
// a chunk live over its own rows once its operands are built), the gate
// prefix (19.3 KiB with the anchor constants; the triangular system and its
// inverse live over it once the operands are built), and two ring slots of
// 40.6 KiB (Kg, Qg, Kr^T, T, Mqk, decays, beta and the value rows): 151.5
// KiB.
//
// Accumulator-to-operand reuse.  An accumulator tile of v_mfma_f32_16x16x32
// gives lane l the rows 4(l/16)+i (i < 4) of column l%16, while the B operand
// wants 8 K-values per lane.  Two vertically adjacent tiles give lane l the
// rows {4(l/16)+i, 16+4(l/16)+i}; using that set as the lane's 8 K-slots (a
// fixed permutation of the 32-long K index applied to both operands) turns
// the FP32 state, V' and U into the next product's B operand with a register
// conversion only.  The A operands (Kg, Qg, Kr^T, T, Mqk) are therefore
// stored in LDS with their K index in that permuted order.
#include <climits>
#include <cmath>

#include "chunk_common.h"

namespace kda {
namespace {

using namespace chunk;

typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

template <int DVS>
struct RingSmem {
  ChunkQKG raw[2];             // chunk c+1 in preparation, chunk c+2 landing
  PrepWork pw;                 // gate prefix (then the inverse's work)
  ChunkOps<DVS> slot[2];       // the ring: chunk c (consumed), chunk c+1 (prepared)
};

constexpr int kThreads = 512;
constexpr int kProducerBase = 256;   // first producer thread

// Blocks start in index order as compute units free up, and a block holds a
// compute unit for its whole sequence, so the sequence a block works on is
// taken in longest-first order (ties by index): in a varlen batch a long
// sequence otherwise may only start in the last round of blocks and end
// alone.  Returns the sequence of rank r by (length descending, index
// ascending); `tmp` is LDS scratch of at least N + 1 ints, free on entry and
// on return.  All threads; contains barriers.
constexpr int kLongestFirstMaxSeqs = 256;

__device__ __forceinline__ int longest_first_sequence(const PrefillArgs& a, int r, int* tmp,
                                                      int tid) {
  const int N = a.num_seqs;
  for (int i = tid; i < N; i += kThreads) {
    const int b = clamp_offset(a.cu_seqlens[i], a.total_tokens);
    tmp[i] = max(b, clamp_offset(a.cu_seqlens[i + 1], a.total_tokens)) - b;
  }
  __syncthreads();
  for (int i = tid; i < N; i += kThreads) {
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
__global__ __launch_bounds__(kThreads) void prefill_chunk_kernel(PrefillArgs a, float exp2C) {
  constexpr int DVS = 64 * NT;
  extern __shared__ __align__(16) unsigned char smem_raw[];
  RingSmem<DVS>& sm = *reinterpret_cast<RingSmem<DVS>*>(smem_raw);

  const int H = a.num_heads;
  const int slice = blockIdx.x, h = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const bool producer = tid >= kProducerBase;
  const int ptid = tid - kProducerBase, pwave = wave - 4;   // producer numbering
  // the sequence of rank blockIdx.z, longest first (the raw buffers are not in use yet)
  int* const rank_tmp = reinterpret_cast<int*>(&sm.raw[0]);
  const int n = (a.num_seqs > 1 && a.num_seqs <= kLongestFirstMaxSeqs)
                    ? longest_first_sequence(a, blockIdx.z, rank_tmp, tid)
                    : (int)blockIdx.z;
  const int l16 = lane & 15, g4 = lane >> 4;
  const int col_base = slice * DVS;
  const float C = a.anchor_log2;

  const int bos = clamp_offset(a.cu_seqlens[n], a.total_tokens);
  const int eos = max(bos, clamp_offset(a.cu_seqlens[n + 1], a.total_tokens));
  const int nch = (eos - bos + CH - 1) / CH;

  if (producer) {
    // ------------------------------------------------------------ producers
    // Nothing of this wave's is in flight here.  The compiler may lay the
    // producers' code after the consumers' and then count the consumers'
    // state loads as pending in the producers' waits (up to waiting for the
    // next chunk's prefetch in the middle of a step); an explicit vmcnt(0)
    // clears that count.  s_waitcnt fields: vmcnt bits 3:0 (and 15:14) = 0,
    // expcnt bits 6:4 = 7 and lgkmcnt bits 11:8 = 15, i.e. not waited on.
    __builtin_amdgcn_s_waitcnt(0x0F70);
    // Chunk c's rows are fetched into registers during step c-2 (the q and k
    // rows around the gate prefix, the g and value rows around the pair
    // products, so that the 16-byte loads find the compute unit's address
    // path free instead of queueing behind each other) and written
    // to LDS at that step's end: its q/k/g rows into raw[c % 2] (free since
    // chunk c-2 was prepared from it) and its value rows into ring slot c % 2
    // (the consumers finish reading chunk c-2's values before the last phase
    // of step c-2).  The first chunk is staged before the pipeline starts.
    ChunkRegs<DVS> x;
    if (nch > 0) {
      fetch_chunk(x, a, bos, min(CH, eos - bos), h, col_base, ptid);
      stage_chunk(sm.raw[0], sm.slot[0].v, x, ptid);
    }
    // Step s (s = -1 .. nch-1): chunk s+1 is prepared into ring slot (s+1) % 2
    // while the consumers run the chain of chunk s.  Every wave passes the
    // same four barriers per step.
    for (int s = -1; s < nch; ++s) {
      const bool prep = s + 1 < nch;
      ChunkQKG& cr = sm.raw[(s + 1) & 1];          // chunk s+1's rows
      ChunkOps<DVS>& sn = sm.slot[(s + 1) & 1];    // chunk s+1's ring slot
      const int tn0 = bos + CH * (s + 1), Ln = min(CH, eos - tn0);
      // B0: chunk s+1's rows and values and chunk s's slot are complete; the
      // consumers are done with slot s-1 (except its values, already chunk
      // s+1's), the producers with the inverse's work space.
      lds_barrier();
      if (prep) {
        stage_beta<FE>(sn.beta, x.beta, a.fe, Ln, ptid);
        if (s + 2 < nch) fetch_chunk_part<0>(x, a, tn0 + CH, min(CH, eos - tn0 - CH), h, col_base, ptid);
        gate_prefix<MODE, FE>(sm.pw, sn.dec, cr, a.fe, C, a.half_anchor_log2, Ln, tid);
        __builtin_amdgcn_sched_barrier(0);
        if (s + 2 < nch) fetch_chunk_part<1>(x, a, tn0 + CH, min(CH, eos - tn0 - CH), h, col_base, ptid);
        __builtin_amdgcn_sched_barrier(0);
        if (FE) qk_norms(sm.pw, cr, a, ptid);
      }
      lds_barrier();   // B1: gate prefix, anchor constants, beta and decays of chunk s+1 written
      if (prep) {
        if (s + 2 < nch) fetch_chunk_part<2>(x, a, tn0 + CH, min(CH, eos - tn0 - CH), h, col_base, ptid);
        __builtin_amdgcn_sched_barrier(0);
        f32x4 pacc[6];
        auto emit = [&](int t, int c0, const f16x8& kg, const f16x8& qg, const f16x8& kr) {
          const int cb = c0 & ~31, cl = c0 & 31;
          const f16x4 kg_lo = {kg[0], kg[1], kg[2], kg[3]}, kg_hi = {kg[4], kg[5], kg[6], kg[7]};
          const f16x4 qg_lo = {qg[0], qg[1], qg[2], qg[3]}, qg_hi = {qg[4], qg[5], qg[6], qg[7]};
#pragma unroll
          for (int j = 0; j < 8; ++j) sn.KrT[c0 + j][kslot(t)] = kr[j];
          // channels cl..cl+3 and cl+4..cl+7 land in two runs of 4 slots
          *reinterpret_cast<f16x4*>(&sn.Kg[t][cb + kslot(cl)]) = kg_lo;
          *reinterpret_cast<f16x4*>(&sn.Kg[t][cb + kslot(cl + 4)]) = kg_hi;
          *reinterpret_cast<f16x4*>(&sn.Qg[t][cb + kslot(cl)]) = qg_lo;
          *reinterpret_cast<f16x4*>(&sn.Qg[t][cb + kslot(cl + 4)]) = qg_hi;
        };
        if (MODE == 2 && steep_wave(sm.pw, pwave, lane))
          pair_products_steep<FE>(pacc, sm.pw, cr, pwave, lane, emit);
        else
          pair_products<MODE, FE>(pacc, sm.pw, cr, a, C, exp2C, pwave, lane, emit);
        pair_store(cr, pacc, pwave, lane);   // over this wave's own columns of the rows
        __builtin_amdgcn_sched_barrier(0);
        if (s + 2 < nch) fetch_chunk_part<3>(x, a, tn0 + CH, min(CH, eos - tn0 - CH), h, col_base, ptid);
      }
      lds_barrier();   // B2: split-K partials of chunk s+1 complete
      if (prep) {
        // the triangular system's diagonal blocks and W on two waves, Mqk's tiles on the others
        if (pwave < 2)
          reduce_invert(inv_of(sm.pw), cr, sn.beta, pwave, lane, [&](int r, int c, float t) {
            sn.T[r][kslot(c)] = static_cast<_Float16>(t);
          });
        else
          reduce_mqk(cr, pwave - 2, lane, [&](int r, int c, float m) {
            sn.Mqk[r][kslot(c)] = static_cast<_Float16>(m);
          });
      }
      lds_barrier();   // B3: chunk s+1's ring slot complete; the consumers are done with slot s
      if (s + 2 < nch) stage_chunk(sm.raw[s & 1], sm.slot[s & 1].v, x, ptid);   // chunk s+2
    }
    return;
  }

  // -------------------------------------------------------------- consumers
  // State tile (mt, nt) holds key rows 16 mt + 4 g4 + i and value column
  // col_base + colw + 16 nt + l16.
  const int colw = wave * 16 * NT;          // first column of this wave, within the slice
  f32x4 S[8][NT];
  auto state_elem = [&](int mt, int nt, int i) __attribute__((always_inline)) {
    return (16 * mt + 4 * g4 + i) * D + col_base + colw + 16 * nt + l16;
  };
  // A state store: one buffer resource over the [128][128] state, the lane's
  // part of each element offset in one register and the rest uniform, so
  // that no per-element 64-bit address stays live across the chunk loop.
  const uint32_t lane_elem = (uint32_t)(4 * g4 * D + colw + l16);
  auto store_state = [&](float* dst) __attribute__((always_inline)) {
    const __amdgpu_buffer_rsrc_t r = make_buffer(dst, (uint32_t)(D * D * 4));
#pragma unroll
    for (int mt = 0; mt < 8; ++mt)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float sv = S[mt][nt][i];
          __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, sv), r, lane_elem * 4,
                                                (int)(((16 * mt + i) * D + col_base + 16 * nt) * 4), 0);
        }
  };
  {
    const StateRef s0 = prefill_initial_state(a, n, h);
    auto init_state = [&](auto load) __attribute__((always_inline)) {
#pragma unroll
      for (int mt = 0; mt < 8; ++mt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
          for (int i = 0; i < 4; ++i) S[mt][nt][i] = load(state_elem(mt, nt, i));
    };
    // one branch on the state's type, outside the element loops
    if (!s0)
      init_state([](int) { return 0.f; });
    else if (s0.bf16)
      init_state([&](int e) { return bf16_to_f32(static_cast<const uint16_t*>(s0.p)[e]); });
    else
      init_state([&](int e) { return static_cast<const float*>(s0.p)[e]; });
  }
  {   // T12 = 0 in both ring slots, once: the inverse writes only T's other blocks
    const int i = tid >> 4, m = tid & 15;
#pragma unroll
    for (int sl = 0; sl < 2; ++sl) sm.slot[sl].T[i][kslot(16 + m)] = static_cast<_Float16>(0.f);
  }
  // Checkpoints (the state after every ckpt_tokens tokens): chunk count of
  // the next one and its row of the checkpoint buffer.
  const int ck_per = a.ckpt ? a.ckpt_tokens / CH : 0;
  int ck_next = a.ckpt ? ck_per : INT_MAX;
  int64_t ck_row = a.ckpt ? (int64_t)n + bos / a.ckpt_tokens : 0;
  for (int s = -1; s < nch; ++s) {
    const ChunkOps<DVS>& sc = sm.slot[s & 1];    // chunk s's ring slot
    lds_barrier();   // B0
    if (s + 1 < nch) {   // the consumers' share of chunk s+1's gate prefix (channels 0-63)
      const int tn0 = bos + CH * (s + 1);
      gate_prefix<MODE, FE>(sm.pw, sm.slot[(s + 1) & 1].dec, sm.raw[(s + 1) & 1], a.fe, C,
                            a.half_anchor_log2, min(CH, eos - tn0), tid);
    }
    lds_barrier();   // B1
    // ---- the state chain of chunk s on this wave's 16 * NT value columns.
    // Its products with the state (W, O: matrix-core work and little VALU)
    // run beside the producers' VALU-bound pair products; the rest beside
    // the producers' reduction and inverse
    f32x4 OT[NT][2];
    f16x8 Uh[NT], Ul[NT];
    f32x4 W[2][NT];
    float vv[NT][2][4];
    const int t0 = bos + CH * s, L = min(CH, eos - t0);
    const f32x4 z = {0.f, 0.f, 0.f, 0.f};
    if (s >= 0) {
      // this lane's value entries (tokens 16 mt + 4 g4 + i, column 16 nt +
      // l16), read before the products so that the reads are in flight together
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            vv[nt][mt][i] = sc.beta[16 * mt + 4 * g4 + i] * bf16_to_f32(sc.v[16 * mt + 4 * g4 + i][colw + 16 * nt + l16]);
      // the value and beta reads as one group ahead of the products
      __builtin_amdgcn_sched_group_barrier(0x0100, 16 * NT + 8, 0);
      // W = Kg S (rows = tokens) and O^T = S^T Qg^T (rows = value columns: the
      // same fragments with A and B swapped, so each lane ends with 4
      // adjacent columns of one token for the output store)
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) { W[mt][nt] = z; OT[nt][mt] = z; }
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        // fp16 S of K step p (key rows 32p..32p+31) as B (and, transposed, A) operand
        f16x8 Sb[NT];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            Sb[nt][i] = static_cast<_Float16>(S[2 * p][nt][i]);
            Sb[nt][4 + i] = static_cast<_Float16>(S[2 * p + 1][nt][i]);
          }
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
          const f16x8 akg = *reinterpret_cast<const f16x8*>(&sc.Kg[16 * mt + l16][32 * p + 8 * g4]);
          const f16x8 aqg = *reinterpret_cast<const f16x8*>(&sc.Qg[16 * mt + l16][32 * p + 8 * g4]);
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) {
            W[mt][nt] = mfma_f16(akg, Sb[nt], W[mt][nt]);
            OT[nt][mt] = mfma_f16(Sb[nt], aqg, OT[nt][mt]);
          }
        }
      }
    }
    lds_barrier();   // B2
    if (s >= 0) {
      // V' = b (V - W) as hi + lo fp16 B operands (K = token, permuted)
      f16x8 Vh[NT], Vl[NT];
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int t = 16 * mt + 4 * g4 + i;
            const float vp = vv[nt][mt][i] - sc.beta[t] * W[mt][nt][i];
            _Float16 hh, ll;
            split_f16(vp, hh, ll);
            Vh[nt][4 * mt + i] = hh;
            Vl[nt][4 * mt + i] = ll;
          }
      // U = T V'
      f32x4 U[2][NT];
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        const f16x8 at = *reinterpret_cast<const f16x8*>(&sc.T[16 * mt + l16][8 * g4]);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          U[mt][nt] = mfma_f16(at, Vh[nt], z);
          U[mt][nt] = mfma_f16(at, Vl[nt], U[mt][nt]);
        }
      }
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
    }
    if (s >= 0) {
      // S = Diag(2^{G_L}) S + Kr^T U
#pragma unroll
      for (int mt = 0; mt < 8; ++mt) {
        const f16x8 akr = *reinterpret_cast<const f16x8*>(&sc.KrT[16 * mt + l16][8 * g4]);
        const f32x4 d = *reinterpret_cast<const f32x4*>(&sc.dec[16 * mt + 4 * g4]);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
#pragma unroll
          for (int i = 0; i < 4; ++i) S[mt][nt][i] *= d[i];
          S[mt][nt] = mfma_f16(akr, Uh[nt], S[mt][nt]);
          S[mt][nt] = mfma_f16(akr, Ul[nt], S[mt][nt]);
        }
      }
      // O^T += U^T Mqk^T, then O = scale O0 stored as 4 adjacent bf16 columns
      // per lane (rows t >= L of a final partial chunk fall outside the
      // buffer range and are dropped)
      const __amdgpu_buffer_rsrc_t orsrc =
          make_buffer(a.out + ((int64_t)t0 * H + h) * D, (uint32_t)(((L - 1) * H + 1) * D * 2));
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        const f16x8 am = *reinterpret_cast<const f16x8*>(&sc.Mqk[16 * mt + l16][8 * g4]);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          OT[nt][mt] = mfma_f16(Uh[nt], am, OT[nt][mt]);
          OT[nt][mt] = mfma_f16(Ul[nt], am, OT[nt][mt]);
          const int t = 16 * mt + l16;
          u32x2 pk;
          pk[0] = (uint32_t)f32_to_bf16(a.scale * OT[nt][mt][0]) |
                  ((uint32_t)f32_to_bf16(a.scale * OT[nt][mt][1]) << 16);
          pk[1] = (uint32_t)f32_to_bf16(a.scale * OT[nt][mt][2]) |
                  ((uint32_t)f32_to_bf16(a.scale * OT[nt][mt][3]) << 16);
          __builtin_amdgcn_raw_buffer_store_b64(
              pk, orsrc, (uint32_t)((t * H * D + col_base + colw + 16 * nt + 4 * g4) * 2), 0, 0);
        }
      }
      // checkpoint after every ck_per full chunks (counters instead of a
      // division per chunk)
      if (s + 1 == ck_next) {
        if (L == CH) store_state(a.ckpt + (ck_row * H + h) * (int64_t)(D * D));
        ck_next += ck_per;
        ++ck_row;
      }
    }
    lds_barrier();   // B3
    if (s + 1 < nch && wave == 0)   // chunk s+1's T21 = -W T11, beside the producers' staging of chunk s+2
      invert_offdiag(inv_of(sm.pw), lane, [&](int r, int c, float t) {
        sm.slot[(s + 1) & 1].T[r][kslot(c)] = static_cast<_Float16>(t);
      });
  }

  if (const StateRef s1 = prefill_final_state(a, n, h)) {
    if (!s1.bf16) {
      store_state(static_cast<float*>(s1.p));
    } else {
      const __amdgpu_buffer_rsrc_t r = make_buffer(s1.p, (uint32_t)(D * D * 2));
#pragma unroll
      for (int mt = 0; mt < 8; ++mt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            buffer_store_u16(f32_to_bf16(S[mt][nt][i]), r,
                             lane_elem * 2 + (uint32_t)(((16 * mt + i) * D + col_base + 16 * nt) * 2));
    }
  }
}

template <int MODE, int NT, bool FE>
hipError_t launch_variant(const PrefillArgs& a, hipStream_t s) {
  constexpr size_t bytes = sizeof(RingSmem<64 * NT>);
  static_assert(bytes <= 160 * 1024, "the fused kernel's LDS exceeds a compute unit's 160 KiB");
  static bool attr_set = false;   // idempotent; a race only repeats the call
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&prefill_chunk_kernel<MODE, NT, FE>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  // the anchor's power of two: 2^C (one anchor per chunk) or 2^h, h = 8 lb
  // log2 e (16-token anchors)
  const float exp2C = MODE == 0 ? std::exp2(a.anchor_log2)
                                : MODE == 1 ? std::exp2(a.half_anchor_log2) : 0.f;
  prefill_chunk_kernel<MODE, NT, FE>
      <<<dim3(2 / NT, a.num_heads, a.num_seqs), kThreads, bytes, s>>>(a, exp2C);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill_chunk(const PrefillArgs& a, int anchor_mode, int dv_split,
                                hipStream_t s) {
  if (a.num_seqs <= 0) return hipSuccess;
  if (dv_split != 1 && dv_split != 2) return hipErrorInvalidValue;
  const int nt = dv_split == 1 ? 2 : 1;
  // data-dependent anchors and the input front-end: 64-column blocks only
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
