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
//   pass 1 (prefill_split_prep): one block per (chunk, head), all chunks of
//     all sequences at once.  Steps 1-3 of section 2 (gate prefix, anchored
//     Mqk/Akk, the 32x32 inverse T) and then everything that depends only on
//     the chunk:
//        U0 = T Diag(b) V          (what U would be from a zero state)
//        M  = T Diag(b) Kg         (how U depends on the incoming state)
//     so that U = U0 - M S0.  Results go to a workspace record per
//     (chunk, head), laid out in MFMA-fragment order.
//   pass 2 (prefill_split_chain): one block per (sequence, head, 64 value
//     columns); each wave owns 16 columns and walks the chunks in order:
//        U  = U0 + (-M) S0                    (fp16 MFMA, FP32 accumulate)
//        S1 = Diag(2^{G_L}) S0 + Kr^T U       (U as hi + lo fp16)
//        O  = scale (Qg S0 + Mqk U)
//     i.e. the note's fused [S | O] update, with the state resident in the
//     accumulators.  Chunk records are prefetched several chunks ahead into
//     registers and staged through a double-buffered LDS area shared by the
//     four waves.
//
// Workspace record of (chunk slot s, head h) at ((s * H + h) * kRecBytes):
//   [0, 8192)        -M    fp16 A fragments [mt 2][kstep 4][lane 64][8]
//   [8192, 16384)    Qg    fp16 A fragments [mt 2][kstep 4][lane 64][8]
//   [16384, 24576)   Kr^T  fp16 A fragments [mt 8][lane 64][8]
//   [24576, 26624)   Mqk   fp16 A fragments [mt 2][lane 64][8]
//   [26624, 27136)   2^{G_L} fp32 [128]
//   [27136, 28672)   zero padding (the staged part is 7 x 4 KiB: one 16-byte
//                    load per thread per 4 KiB, no tail)
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

struct PrepOut {
  PrepSmem<D> p;
  _Float16 frag[kRecStageBytes / 2];  // record bytes [0, kRecStageBytes), staged
  float bkgT[D][CH + 4];              // b_t k_t 2^{G_t}, transposed [channel][token]
};

// fp16 element index (within a record) of A-fragment entry (row, k) of a
// fragment set with 32-long K blocks: [row/16][k/32][lane][8].
__device__ __forceinline__ int frag_rowk(int row, int k, int ksteps) {
  const int s = kslot(k & 31);
  const int L = (row & 15) + ((s >> 3) << 4);
  return ((((row >> 4) * ksteps + (k >> 5)) * 64 + L) << 3) + (s & 7);
}

template <int MODE>
__global__ __launch_bounds__(256) void prefill_split_prep(PrefillArgs a, float exp2C,
                                                           uint8_t* __restrict__ ws) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  PrepOut& sm = *reinterpret_cast<PrepOut*>(smem_raw);
  PrepSmem<D>& ps = sm.p;
  const int H = a.num_heads, N = a.num_seqs, T = a.total_tokens;
  const int slot = blockIdx.x, h = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, g4 = lane >> 4;
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

  load_chunk(ps, a, t0, L, h, 0, tid, 256);
  __syncthreads();
  gate_prefix<MODE>(ps, C, tid);
  __syncthreads();
  pair_products<MODE>(ps, a, C, exp2C, wave, lane,
                      [&](int t, int c0, const float* kv, const float* qv, const float* P,
                          const float* R) {
                        const float bt = ps.beta[t];
#pragma unroll
                        for (int j = 0; j < 8; ++j) {
                          const int ch = c0 + j;
                          sm.frag[kRecOffQg / 2 + frag_rowk(t, ch, 4)] =
                              static_cast<_Float16>(qv[j] * P[j]);
                          sm.frag[kRecOffKrT / 2 + frag_rowk(ch, t, 1)] =
                              static_cast<_Float16>(kv[j] * R[j]);
                          sm.bkgT[ch][t] = bt * (kv[j] * P[j]);
                        }
                      });
  __syncthreads();
  reduce_pairs(ps, tid, [&](int r, int s, float m) {
    sm.frag[kRecOffMqk / 2 + frag_rowk(r, s, 1)] = static_cast<_Float16>(m);
  });
  __syncthreads();
  invert_unit_lower(ps, tid);
  __syncthreads();

  // U0 = T Diag(b) V and M = T Diag(b) Kg: wave w computes value / key
  // columns 32w..32w+31 for all 32 tokens, with hi + lo fp16 operands on both
  // sides (three products), so both are accurate to FP32 level.
  {
    const f32x4 z = {0.f, 0.f, 0.f, 0.f};
    f16x8 th[2], tl[2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        _Float16 hh, ll;
        split_f16(ps.Tf[16 * mt + l16][8 * g4 + j], hh, ll);
        th[mt][j] = hh;
        tl[mt][j] = ll;
      }
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int nt = 2 * wave + q;
      const int col = 16 * nt + l16;
      f16x8 vh, vl, kh, kl;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int t = 8 * g4 + j;
        _Float16 hh, ll;
        split_f16(ps.beta[t] * bf16_to_f32(ps.vraw[t][col]), hh, ll);
        vh[j] = hh;
        vl[j] = ll;
        split_f16(sm.bkgT[col][t], hh, ll);
        kh[j] = hh;
        kl[j] = ll;
      }
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        f32x4 u = mfma_f16(th[mt], vh, z);
        u = mfma_f16(th[mt], vl, u);
        u = mfma_f16(tl[mt], vh, u);
        f32x4 m = mfma_f16(th[mt], kh, z);
        m = mfma_f16(th[mt], kl, m);
        m = mfma_f16(tl[mt], kh, m);
        *reinterpret_cast<f32x4*>(rec + kRecOffU0 + ((nt * 2 + mt) * 64 + lane) * 16) = u;
#pragma unroll
        for (int i = 0; i < 4; ++i)
          sm.frag[kRecOffMneg / 2 + frag_rowk(16 * mt + 4 * g4 + i, col, 4)] =
              static_cast<_Float16>(-m[i]);
      }
    }
  }
  if (tid < D) reinterpret_cast<float*>(&sm.frag[kRecOffDec / 2])[tid] = ps.dec[tid];
  for (int e = (kRecOffDec + 4 * D) / 16 + tid; e < kRecStageBytes / 16; e += 256)
    reinterpret_cast<uint4*>(sm.frag)[e] = make_uint4(0, 0, 0, 0);
  __syncthreads();
  for (int e = tid; e < kRecStageBytes / 16; e += 256)
    reinterpret_cast<uint4*>(rec)[e] = reinterpret_cast<const uint4*>(sm.frag)[e];
}

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

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

// Operands of the first products of a chunk step, read one step ahead.
struct StateFrag {
  f16x8 am[2][4];   // -M fragments, [mt][kstep]
  f32x4 u0[2];      // U0 accumulator tiles
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
  auto read_frag = [&](StateFrag& F, int c) __attribute__((always_inline)) {
    const uint8_t* st = slot(c);
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
      for (int p = 0; p < 4; ++p)
        F.am[mt][p] = *reinterpret_cast<const f16x8*>(st + kRecOffMneg + ((mt * 4 + p) * 64 + lane) * 16);
      F.u0[mt] = *reinterpret_cast<const f32x4*>(st + kRecStageBytes + (mt * 64 + lane) * 16);
    }
  };
  StateFrag F[2];
  __syncthreads();
  read_frag(F[0], 0);
  auto step = [&](auto I_const, int c) __attribute__((always_inline)) {
    constexpr int I = decltype(I_const)::value;
    if (c < nch) {
      // Kr^T and the decay are first needed after the U products: read them
      // now, then the next step's -M and U0.
      const uint8_t* st = slot(c);
      f16x8 ak[8];
      f32x4 dv[8];
#pragma unroll
      for (int mt = 0; mt < 8; ++mt) {
        ak[mt] = *reinterpret_cast<const f16x8*>(st + kRecOffKrT + (mt * 64 + lane) * 16);
        dv[mt] = *reinterpret_cast<const f32x4*>(st + kRecOffDec + (16 * mt + 4 * g4) * 4);
      }
      read_frag(F[1 - I], c + 1);         // unused past the end
      __builtin_amdgcn_sched_barrier(0);
      const StateFrag& f = F[I];
      f16x8 Sb[4];
#pragma unroll
      for (int p = 0; p < 4; ++p)
#pragma unroll
        for (int i2 = 0; i2 < 4; ++i2) {
          Sb[p][i2] = static_cast<_Float16>(S[2 * p][i2]);
          Sb[p][4 + i2] = static_cast<_Float16>(S[2 * p + 1][i2]);
        }
      f32x4 U[2] = {f.u0[0], f.u0[1]};
#pragma unroll
      for (int p = 0; p < 4; ++p)
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) U[mt] = mfma_f16(f.am[mt][p], Sb[p], U[mt]);
      // the decay does not depend on U: it fills the MFMA latency
#pragma unroll
      for (int mt = 0; mt < 8; ++mt)
#pragma unroll
        for (int i2 = 0; i2 < 4; ++i2) S[mt][i2] *= dv[mt][i2];
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
        S[mt] = mfma_f16(ak[mt], Uh, S[mt]);
        S[mt] = mfma_f16(ak[mt], Ul, S[mt]);
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
  constexpr size_t bytes = sizeof(PrepOut);
  static bool attr_set = false;   // idempotent; a race only repeats the call
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&prefill_split_prep<MODE>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  const float exp2C = MODE == 0 ? std::exp2(a.anchor_log2) : 0.f;
  const int64_t slots = (int64_t)a.num_seqs + a.total_tokens / CH + 1;
  prefill_split_prep<MODE><<<dim3((unsigned)slots, a.num_heads), 256, bytes, s>>>(a, exp2C, ws);
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

hipError_t launch_prefill_split(const PrefillArgs& a, int anchor_mode, int dv_split,
                                void* workspace, hipStream_t s) {
  if (dv_split != 8) return hipErrorInvalidValue;   // one 16-column tile per chain block
  if (a.num_seqs <= 0) return hipSuccess;
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  hipError_t e = anchor_mode == 0 ? launch_prep<0>(a, ws, s) : launch_prep<1>(a, ws, s);
  if (e != hipSuccess) return e;
  return launch_chain(a, ws, s);
}

}  // namespace kda
