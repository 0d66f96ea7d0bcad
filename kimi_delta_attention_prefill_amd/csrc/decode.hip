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
// item's value-column slice of COLS columns: thread t holds one vector per
// state row (16 bytes: four FP32 or eight BF16 columns; 8 bytes, four BF16
// columns, in the BF16 64-column slices of calls with few items) of the key
// rows c = rg + RG * i, so every wave reads and writes whole 128-byte row
// pieces (narrower pieces cost partial-line writes).  The two dk-reductions (w, p)
// and q . k are finished in registers inside a wave (a DPP butterfly, then
// lane-swap reduce-scatter steps) and by one LDS fold across the waves; the
// state is read once and written once.  Row counts too small to fill the
// chip use narrower slices (more blocks per item).  Many rows go to the token
// stream below with one token per row: the same step in whole-item 512-thread
// blocks, two resident per compute unit, which measured faster at thousands
// of rows.
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

// The state of a row is read once and written once per step, so its traffic
// is marked non-temporal (streamed past the caches).  Every thread moves one
// vector per state row: 16 bytes, four FP32 or eight BF16 columns, or 8 bytes
// of BF16 where a slice is 64 columns wide (a 32-column BF16 slice would leave
// 64-byte row pieces, half a cache line, which cost a partial-line write on
// every store).
typedef float f32x4v __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4v __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2v __attribute__((ext_vector_type(2)));

// The item's state is read through one buffer resource (its base is uniform
// over the block), so each thread keeps a single 32-bit offset and the
// per-row steps are scalar offsets, instead of a 64-bit address per state
// row; kNT is the non-temporal cache policy of those loads.  The stores go
// through global instructions from a uniform row base plus the same 32-bit
// offset: a 16-byte buffer store whose offset sits in an SGPR is not given
// the wait state before its data registers are overwritten, and the next
// VALU write then reaches the store's data.
constexpr int kNT = 2;

template <bool BF16>
struct StateIO;

template <>
struct StateIO<false> {
  using elem = float;
  using raw = f32x4v;
  static constexpr int CPT = 4;   // columns per thread
  static __device__ __forceinline__ raw load(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    return __builtin_bit_cast(raw, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, kNT));
  }
  static __device__ __forceinline__ void unpack(const raw& w, float* x) {
#pragma unroll
    for (int m = 0; m < 4; ++m) x[m] = w[m];
  }
  static __device__ __forceinline__ void store(__attribute__((address_space(1))) float* p,
                                               const float* x) {
    const f32x4v w = {x[0], x[1], x[2], x[3]};
    __builtin_nontemporal_store(w, (__attribute__((address_space(1))) f32x4v*)p);
  }
};

// BF16 state stays packed in registers between the two passes over it (half
// the registers, so more blocks resident per CU and more bytes in flight).
template <>
struct StateIO<true> {
  using elem = uint16_t;
  using raw = u32x4v;
  static constexpr int CPT = 8;
  static __device__ __forceinline__ raw load(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    return __builtin_bit_cast(raw, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, kNT));
  }
  static __device__ __forceinline__ void unpack(const raw& w, float* x) {
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      x[2 * m] = bf16lo(w[m]);
      x[2 * m + 1] = bf16hi(w[m]);
    }
  }
  static __device__ __forceinline__ void store(__attribute__((address_space(1))) uint16_t* p,
                                               const float* x) {
    u32x4v w;
#pragma unroll
    for (int m = 0; m < 4; ++m)
      w[m] = (uint32_t)f32_to_bf16(x[2 * m]) | ((uint32_t)f32_to_bf16(x[2 * m + 1]) << 16);
    __builtin_nontemporal_store(w, (__attribute__((address_space(1))) u32x4v*)p);
  }
};

// BF16 state in 8-byte vectors (4 columns per thread).  In 64-column slices
// of 512 threads a row then spans 16 threads (whole 128-byte lines still), so
// each thread reduces 9 partial sums over 4 row groups of its wave instead of
// 17 over 8: the shape for calls with few items, where the reductions'
// latency rather than the bytes bounds the call.
struct StateIOBf16Narrow {
  using elem = uint16_t;
  using raw = u32x2v;
  static constexpr int CPT = 4;
  static __device__ __forceinline__ raw load(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    return __builtin_bit_cast(raw, __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, kNT));
  }
  static __device__ __forceinline__ void unpack(const raw& w, float* x) {
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      x[2 * m] = bf16lo(w[m]);
      x[2 * m + 1] = bf16hi(w[m]);
    }
  }
  static __device__ __forceinline__ void store(__attribute__((address_space(1))) uint16_t* p,
                                               const float* x) {
    u32x2v w;
#pragma unroll
    for (int m = 0; m < 2; ++m)
      w[m] = (uint32_t)f32_to_bf16(x[2 * m]) | ((uint32_t)f32_to_bf16(x[2 * m + 1]) << 16);
    __builtin_nontemporal_store(w, (__attribute__((address_space(1))) u32x2v*)p);
  }
};

template <int COLS, bool BF16, int NT>
struct DecodeIO { using type = StateIO<BF16>; };
template <>
struct DecodeIO<64, true, 512> { using type = StateIOBf16Narrow; };

// CPT consecutive bf16 values (8 or 16 bytes) as floats.
template <int CPT>
__device__ __forceinline__ void load_bf16_vec(const uint16_t* p, float* x) {
  if constexpr (CPT == 4) {
    const uint2 w = *reinterpret_cast<const uint2*>(p);
    x[0] = bf16lo(w.x);
    x[1] = bf16hi(w.x);
    x[2] = bf16lo(w.y);
    x[3] = bf16hi(w.y);
  } else {
    const uint4 w = *reinterpret_cast<const uint4*>(p);
    const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      x[2 * m] = bf16lo(ww[m]);
      x[2 * m + 1] = bf16hi(ww[m]);
    }
  }
}

template <int CPT>
__device__ __forceinline__ void store_bf16_vec(uint16_t* p, const float* x) {
  uint32_t w[CPT / 2];
#pragma unroll
  for (int m = 0; m < CPT / 2; ++m)
    w[m] = (uint32_t)f32_to_bf16(x[2 * m]) | ((uint32_t)f32_to_bf16(x[2 * m + 1]) << 16);
  if constexpr (CPT == 4)
    *reinterpret_cast<uint2*>(p) = make_uint2(w[0], w[1]);
  else
    *reinterpret_cast<uint4*>(p) = make_uint4(w[0], w[1], w[2], w[3]);
}

// x + (x from the lane 8 apart in the same 16-lane row), on every lane.
__device__ __forceinline__ float butterfly8(float x) {
  return x + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                 0, __builtin_bit_cast(int, x), 0x128 /* row_ror:8 */, 0xF, 0xF, true));
}

// Reduce-scatter steps for two values a, b summed across lane bit 4
// (16-lane rows 0+1 and 2+3) or bit 5 (the two 32-lane halves): one lane
// swap gives each lane the other half's copy of one of them, so the result
// holds the sum of a in the lower partner and of b in the upper one.  (The
// two swap results are copied to integers before the float casts: a bit cast
// applied to each element of the builtin's result in place compiles to the
// first element twice.)
__device__ __forceinline__ float swap_sum16(float a, float b) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false,
                                                  false);
  const uint32_t x0 = r[0], x1 = r[1];
  return __uint_as_float(x0) + __uint_as_float(x1);
}
__device__ __forceinline__ float swap_sum32(float a, float b) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false,
                                                  false);
  const uint32_t x0 = r[0], x1 = r[1];
  return __uint_as_float(x0) + __uint_as_float(x1);
}

// Values in[0..N) summed in pairs across one lane bit; an odd last value is
// paired with itself (so every lane ends with its full sum).
template <int N, bool BIT5>
__device__ __forceinline__ void scatter_level(const float* in, float* out) {
#pragma unroll
  for (int k = 0; k < N / 2; ++k)
    out[k] = BIT5 ? swap_sum32(in[2 * k], in[2 * k + 1]) : swap_sum16(in[2 * k], in[2 * k + 1]);
  if constexpr (N % 2) out[N / 2] = BIT5 ? swap_sum32(in[N - 1], in[N - 1]) : swap_sum16(in[N - 1], in[N - 1]);
}

// Sums N per-lane values over the lanes of a wave that share lane % TPR
// (TPR = 8, 16 or 32) and stores them to dst[0..N) of that column: lane bit
// 3 by a DPP butterfly, bits 4 and 5 by reduce-scatter swaps, after which
// lane group P j + gamma (gamma = the lane's row or half) holds value
// min(P j + gamma, N - 1) of register j.  Lanes holding the same value store
// the same word.  No LDS traffic and one VALU op per value and level.
template <int TPR, int N>
__device__ __forceinline__ void wave_reduce_store(float* v, float* dst, int lane) {
  static_assert(TPR == 8 || TPR == 16 || TPR == 32, "row-group reduction");
  if constexpr (TPR == 32) {
    float h[(N + 1) / 2];
    scatter_level<N, true>(v, h);
    const int gamma = lane >> 5;
#pragma unroll
    for (int j = 0; j < (N + 1) / 2; ++j) dst[min(2 * j + gamma, N - 1)] = h[j];
  } else {
    if constexpr (TPR == 8) {
#pragma unroll
      for (int m = 0; m < N; ++m) v[m] = butterfly8(v[m]);
    }
    constexpr int N1 = (N + 1) / 2, N2 = (N1 + 1) / 2;
    float h1[N1], h2[N2];
    scatter_level<N, false>(v, h1);
    scatter_level<N1, true>(h1, h2);
    const int gamma = lane >> 4;
#pragma unroll
    for (int j = 0; j < N2; ++j) dst[min(4 * j + gamma, N - 1)] = h2[j];
  }
}

// One block per work unit: value columns [slice COLS, (slice + 1) COLS) of
// item (row r, head h), NT threads.  Thread t holds CPT adjacent columns of
// the key rows rg + RG i (TPR threads per row, RG row groups, RPT rows each);
// a wave covers 64 / TPR whole rows, so each of its loads and stores is a
// contiguous run of rows.
template <int COLS, bool BF16, int NT>
struct DecodeBlock {
  using IO = typename DecodeIO<COLS, BF16, NT>::type;
  using elem = typename IO::elem;
  static constexpr int CPT = IO::CPT;
  static constexpr int TPR = COLS / CPT;
  static constexpr int RG = NT / TPR;
  static constexpr int RPT = kHeadDim / RG;
  static constexpr int SLICES = kHeadDim / COLS;
  static constexpr int WAVES = NT / 64;
  static constexpr int NRED = 2 * CPT + 1;   // w, p and q . k partial sums
  static_assert(TPR >= 8 && TPR <= 32 && RPT >= 1 && RG * RPT == kHeadDim, "decode tiling");

  struct Smem {
    float sq[kHeadDim], sk[kHeadDim], sd[kHeadDim];
    float red[WAVES][TPR][NRED + 1];
    float tot[TPR][NRED + 1];
    float nrm[2][2];   // [wave][q, k] partial sums of squares
  };

  __device__ __forceinline__ static void run(const DecodeArgs& a, Smem& sm) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int jq = tid % TPR, rg = tid / TPR;
    const int H = a.num_heads;
    const int64_t item = blockIdx.x / SLICES;
    const int slice = (int)(blockIdx.x % SLICES);
    const int r = (int)(item / H), h = (int)(item % H);
    const int col0 = slice * COLS + jq * CPT;
    const int64_t rh = (int64_t)r * H + h;
    // The slot lookup goes first; the row's inputs do not depend on it and
    // are requested while it is in flight (by every thread, so no divergent
    // branch makes the block wait for them), and the state loads are the
    // only memory round trip that waits on another.
    const int64_t slot = a.slots[r];
    const int ch = tid & (kHeadDim - 1);
    const uint16_t qb = a.q[rh * kHeadDim + ch];
    const uint16_t kb = a.k[rh * kHeadDim + ch];
    const uint16_t gb = a.g[rh * kHeadDim + ch];
    float vin[CPT];
    load_bf16_vec<CPT>(a.v + rh * kHeadDim + col0, vin);
    const uint16_t bb = a.beta[rh];
    if (slot < 0 || slot >= a.num_slots) {   // skipped row: zero output, pool untouched
      if (tid < COLS) a.out[rh * kHeadDim + slice * COLS + tid] = 0;
      return;
    }
    elem* S = reinterpret_cast<elem*>(a.pool) + slot * a.slot_stride + h * (kHeadDim * kHeadDim);
    const __amdgpu_buffer_rsrc_t rs = make_buffer(S, kHeadDim * kHeadDim * sizeof(elem));
    const uint32_t lane_elem = (uint32_t)(rg * kHeadDim + col0);
    const uint32_t voff = lane_elem * (uint32_t)sizeof(elem);
    constexpr uint32_t kStep = RG * kHeadDim * sizeof(elem);   // bytes between a thread's rows
    typename IO::raw sr[RPT];
#pragma unroll
    for (int i = 0; i < RPT; ++i) sr[i] = IO::load(rs, voff, i * kStep);

    if (tid < kHeadDim) {
      const float qv = bf16_to_f32(qb);
      const float kv = bf16_to_f32(kb);
      const float gv = bf16_to_f32(gb);
      sm.sq[tid] = qv;
      sm.sk[tid] = kv;
      float d;
      if (a.fe.gate_mode == 1)
        d = fast_exp2(a.fe.lower_bound * kLog2e / (1.f + fast_exp2(-gv * kLog2e)));
      else if (a.fe.gate_mode == 2)
        d = 1.f / (1.f + fast_exp2(gv * kLog2e));     // e^{-softplus(a)} = sigmoid(-a)
      else
        d = fast_exp2(gv * kLog2e);
      sm.sd[tid] = d;
      if (a.fe.normalize_qk) {   // waves 0 and 1 hold the 128 channels
        float sq2 = qv * qv, sk2 = kv * kv;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
          sq2 += __shfl_xor(sq2, off);
          sk2 += __shfl_xor(sk2, off);
        }
        if (lane == 0) {
          sm.nrm[wave][0] = sq2;
          sm.nrm[wave][1] = sk2;
        }
      }
    }
    __syncthreads();
    float rq = 1.f, rk = 1.f;
    if (a.fe.normalize_qk) {
      rq = inv_norm(sm.nrm[0][0] + sm.nrm[1][0] + a.fe.norm_eps);
      rk = inv_norm(sm.nrm[0][1] + sm.nrm[1][1] + a.fe.norm_eps);
    }

    // part[0, CPT) = w, part[CPT, 2 CPT) = p, part[2 CPT] = q . k
    float part[NRED];
#pragma unroll
    for (int m = 0; m < NRED; ++m) part[m] = 0.f;
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      const int c = rg + RG * i;
      const float d = sm.sd[c], kc = sm.sk[c], qc = sm.sq[c];
      float x[CPT];
      IO::unpack(sr[i], x);
#pragma unroll
      for (int m = 0; m < CPT; ++m) {
        x[m] *= d;
        part[m] = fmaf(kc, x[m], part[m]);
        part[CPT + m] = fmaf(qc, x[m], part[CPT + m]);
      }
      part[2 * CPT] = fmaf(qc, kc, part[2 * CPT]);
    }
    // The update unpacks the state again rather than keeping the unpacked
    // values live across the reductions (an empty asm hides that the packed
    // words are unchanged, so the two unpacks are not merged).
#pragma unroll
    for (int i = 0; i < RPT; ++i) asm volatile("" : "+v"(sr[i]));
    // Reduce over the row groups of this wave (lanes differing in rg bits)
    // and store each column's sums for the fold across waves.
    wave_reduce_store<TPR, NRED>(part, &sm.red[wave][jq][0], lane);
    __syncthreads();
    // fold the waves' partial sums, one (column, quantity) per thread
    for (int t = tid; t < TPR * NRED; t += NT) {
      const int j = t / NRED, m = t % NRED;
      float acc = sm.red[0][j][m];
#pragma unroll
      for (int w = 1; w < WAVES; ++w) acc += sm.red[w][j][m];
      sm.tot[j][m] = acc;
    }
    __syncthreads();
#pragma unroll
    for (int m = 0; m < NRED; ++m) part[m] = sm.tot[jq][m];
    const float qk = part[2 * CPT] * (rq * rk);

    float b = bf16_to_f32(bb);
    if (a.fe.beta_logits) b = 1.f / (1.f + fast_exp2(-b * kLog2e));
    float u[CPT], uk[CPT];
#pragma unroll
    for (int m = 0; m < CPT; ++m) {
      u[m] = b * (vin[m] - part[m] * rk);
      uk[m] = u[m] * rk;   // the update adds k_n u^T = k (u / |k|)^T; the output keeps u
    }
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      const int c = rg + RG * i;
      const float d = sm.sd[c], kc = sm.sk[c];
      float x[CPT];
      IO::unpack(sr[i], x);
#pragma unroll
      for (int m = 0; m < CPT; ++m) x[m] = fmaf(x[m], d, kc * uk[m]);
      // the row base stays uniform (scalar base + 32-bit lane offset form)
      auto* row = (__attribute__((address_space(1))) elem*)(S + i * (RG * kHeadDim));
      asm volatile("" : "+s"(row));
      IO::store(row + lane_elem, x);
    }
    if (rg == 0) {
      float o[CPT];
#pragma unroll
      for (int m = 0; m < CPT; ++m) o[m] = a.scale * fmaf(qk, u[m], part[CPT + m] * rq);
      store_bf16_vec<CPT>(a.out + rh * kHeadDim + col0, o);
    }
  }
};

template <int COLS, bool BF16, int NT>
__global__ __launch_bounds__(NT) void decode_kernel(DecodeArgs a) {
  using B = DecodeBlock<COLS, BF16, NT>;
  __shared__ typename B::Smem sm;
  B::run(a, sm);
}

template <int COLS, bool BF16, int NT>
hipError_t launch_shape(const DecodeArgs& a, hipStream_t s) {
  const int64_t units = (int64_t)a.rows * a.num_heads * (kHeadDim / COLS);
  decode_kernel<COLS, BF16, NT><<<dim3((unsigned)units), NT, 0, s>>>(a);
  return hipGetLastError();
}

template <bool BF16>
hipError_t launch_cols(const DecodeArgs& a, int cols, int threads, hipStream_t s) {
  if (threads != 256 && threads != 512) return hipErrorInvalidValue;
  const bool wide = threads == 512;
  if constexpr (BF16) {
    if (cols == 128)
      return wide ? launch_shape<128, true, 512>(a, s) : launch_shape<128, true, 256>(a, s);
    if (cols == 64)
      return wide ? launch_shape<64, true, 512>(a, s) : launch_shape<64, true, 256>(a, s);
  } else {
    if (cols == 128)
      return wide ? launch_shape<128, false, 512>(a, s) : launch_shape<128, false, 256>(a, s);
    if (cols == 64)
      return wide ? launch_shape<64, false, 512>(a, s) : launch_shape<64, false, 256>(a, s);
    if (cols == 32)
      return wide ? launch_shape<32, false, 512>(a, s) : launch_shape<32, false, 256>(a, s);
  }
  return hipErrorInvalidValue;
}

// ---------------------------------------------------------------------------
// Token stream: the prefill of many short sequences -- multi-token decode, a
// few new tokens per row appended to the row's pool state -- as a decode-style
// streamer.  One block per (sequence, head, value slice) keeps its slice of
// the FP32 state in registers across the sequence's tokens: one state read and
// one write (16-byte vectors, as the decode), and per token the decode step's
// two dk-reductions.  The next token's inputs are loaded while the current one
// is processed (the barriers order LDS only, so those loads stay in flight).
// The decay, beta and the q/k norm follow the decode step's front-end.
template <int COLS, bool BF16, int NT>
struct StreamBlock {
  using IO = StateIO<BF16>;
  using elem = typename IO::elem;
  using raw = typename IO::raw;
  static constexpr int CPT = IO::CPT;
  static constexpr int TPR = COLS / CPT;
  static constexpr int RG = NT / TPR;
  static constexpr int RPT = kHeadDim / RG;
  static constexpr int SLICES = kHeadDim / COLS;
  static constexpr int WAVES = NT / 64;
  static constexpr int NRED = 2 * CPT + 1;
  static_assert(TPR >= 8 && TPR <= 32 && RPT >= 1 && RG * RPT == kHeadDim, "stream tiling");

  struct Smem {
    float sq[2][kHeadDim], sk[2][kHeadDim], sd[2][kHeadDim];  // by token parity
    float red[WAVES][TPR][NRED + 1];
    float tot[TPR][NRED + 1];
    float nrm[2][2][2];   // [parity][wave][q, k] partial sums of squares
  };

  // One token's inputs as this thread needs them.
  struct Tok {
    uint16_t q, k, g, b;
    float v[CPT];
  };

  __device__ __forceinline__ static void fetch(Tok& x, const PrefillArgs& a, int t, int h, int ch,
                                               int col0) {
    const int64_t th = (int64_t)t * a.num_heads + h;
    x.q = a.q[th * kHeadDim + ch];
    x.k = a.k[th * kHeadDim + ch];
    x.g = a.g[th * kHeadDim + ch];
    x.b = a.beta[th];
    load_bf16_vec<CPT>(a.v + th * kHeadDim + col0, x.v);
  }

  __device__ __forceinline__ static void run(const PrefillArgs& a, Smem& sm) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int jq = tid % TPR, rg = tid / TPR;
    const int H = a.num_heads;
    const int slice = (int)(blockIdx.x % SLICES);
    const int64_t item = blockIdx.x / SLICES;
    const int h = (int)(item % H), n = (int)(item / H);
    const int col0 = slice * COLS + jq * CPT;
    const int ch = tid & (kHeadDim - 1);
    const int bos = a.cu_seqlens ? clamp_offset(a.cu_seqlens[n], a.total_tokens) : n;
    const int eos =
        a.cu_seqlens ? max(bos, clamp_offset(a.cu_seqlens[n + 1], a.total_tokens)) : n + 1;

    // where the state comes from and goes to (uniform over the block)
    const elem* src = nullptr;
    elem* dst = nullptr;
    if (a.pool) {
      const int64_t slot = a.slots[n];
      if (slot >= 0 && slot < a.num_slots) {
        dst = reinterpret_cast<elem*>(a.pool) + slot * a.slot_stride + h * (kHeadDim * kHeadDim);
        src = dst;
      } else if (a.skip_null_slots) {   // the decode's skipped row: zero output, pool untouched
        for (int t = bos; t < eos; ++t)
          if (tid < COLS) a.out[((int64_t)t * H + h) * kHeadDim + slice * COLS + tid] = 0;
        return;
      }
    } else {
      const int64_t off = ((int64_t)n * H + h) * (kHeadDim * kHeadDim);
      if (a.s0) src = reinterpret_cast<const elem*>(a.s0 + off);
      if (a.s1) dst = reinterpret_cast<elem*>(a.s1 + off);
    }
    Tok nxt;
    if (bos < eos) fetch(nxt, a, bos, h, ch, col0);

    const uint32_t lane_elem = (uint32_t)(rg * kHeadDim + col0);
    constexpr uint32_t kStep = RG * kHeadDim * sizeof(elem);
    float s[RPT][CPT];
    if (src) {
      const __amdgpu_buffer_rsrc_t rs = make_buffer(src, kHeadDim * kHeadDim * sizeof(elem));
      raw sr[RPT];
#pragma unroll
      for (int i = 0; i < RPT; ++i) sr[i] = IO::load(rs, lane_elem * (uint32_t)sizeof(elem), i * kStep);
#pragma unroll
      for (int i = 0; i < RPT; ++i) IO::unpack(sr[i], s[i]);
    } else {
#pragma unroll
      for (int i = 0; i < RPT; ++i)
#pragma unroll
        for (int m = 0; m < CPT; ++m) s[i][m] = 0.f;
    }

    for (int t = bos; t < eos; ++t) {
      const int pb = (t - bos) & 1;
      const Tok cur = nxt;
      if (t + 1 < eos) fetch(nxt, a, t + 1, h, ch, col0);
      if (tid < kHeadDim) {   // waves 0 and 1
        const float qv = bf16_to_f32(cur.q), kv = bf16_to_f32(cur.k), gv = bf16_to_f32(cur.g);
        sm.sq[pb][tid] = qv;
        sm.sk[pb][tid] = kv;
        float d;
        if (a.fe.gate_mode == 1)
          d = fast_exp2(a.fe.lower_bound * kLog2e / (1.f + fast_exp2(-gv * kLog2e)));
        else if (a.fe.gate_mode == 2)
          d = 1.f / (1.f + fast_exp2(gv * kLog2e));     // e^{-softplus(a)} = sigmoid(-a)
        else
          d = fast_exp2(gv * kLog2e);
        sm.sd[pb][tid] = d;
        if (a.fe.normalize_qk) {
          float sq2 = qv * qv, sk2 = kv * kv;
#pragma unroll
          for (int off = 1; off < 64; off <<= 1) {
            sq2 += __shfl_xor(sq2, off);
            sk2 += __shfl_xor(sk2, off);
          }
          if (lane == 0) {
            sm.nrm[pb][wave][0] = sq2;
            sm.nrm[pb][wave][1] = sk2;
          }
        }
      }
      lds_barrier();
      float rq = 1.f, rk = 1.f;
      if (a.fe.normalize_qk) {
        rq = inv_norm(sm.nrm[pb][0][0] + sm.nrm[pb][1][0] + a.fe.norm_eps);
        rk = inv_norm(sm.nrm[pb][0][1] + sm.nrm[pb][1][1] + a.fe.norm_eps);
      }
      float part[NRED];
#pragma unroll
      for (int m = 0; m < NRED; ++m) part[m] = 0.f;
#pragma unroll
      for (int i = 0; i < RPT; ++i) {
        const int c = rg + RG * i;
        const float d = sm.sd[pb][c], kc = sm.sk[pb][c], qc = sm.sq[pb][c];
#pragma unroll
        for (int m = 0; m < CPT; ++m) {
          s[i][m] *= d;
          part[m] = fmaf(kc, s[i][m], part[m]);
          part[CPT + m] = fmaf(qc, s[i][m], part[CPT + m]);
        }
        part[2 * CPT] = fmaf(qc, kc, part[2 * CPT]);
      }
      wave_reduce_store<TPR, NRED>(part, &sm.red[wave][jq][0], lane);
      lds_barrier();
      for (int e = tid; e < TPR * NRED; e += NT) {
        const int j = e / NRED, m = e % NRED;
        float acc = sm.red[0][j][m];
#pragma unroll
        for (int w = 1; w < WAVES; ++w) acc += sm.red[w][j][m];
        sm.tot[j][m] = acc;
      }
      lds_barrier();
#pragma unroll
      for (int m = 0; m < NRED; ++m) part[m] = sm.tot[jq][m];
      const float qk = part[2 * CPT] * (rq * rk);
      float b = bf16_to_f32(cur.b);
      if (a.fe.beta_logits) b = 1.f / (1.f + fast_exp2(-b * kLog2e));
      float u[CPT], uk[CPT];
#pragma unroll
      for (int m = 0; m < CPT; ++m) {
        u[m] = b * (cur.v[m] - part[m] * rk);
        uk[m] = u[m] * rk;   // the update adds k_n u^T = k (u / |k|)^T; the output keeps u
      }
#pragma unroll
      for (int i = 0; i < RPT; ++i) {
        const float kc = sm.sk[pb][rg + RG * i];
#pragma unroll
        for (int m = 0; m < CPT; ++m) s[i][m] = fmaf(kc, uk[m], s[i][m]);
      }
      if (rg == 0) {
        float o[CPT];
#pragma unroll
        for (int m = 0; m < CPT; ++m) o[m] = a.scale * fmaf(qk, u[m], part[CPT + m] * rq);
        store_bf16_vec<CPT>(a.out + ((int64_t)t * H + h) * kHeadDim + col0, o);
      }
      if (float* cp = prefill_checkpoint(a, n, h, bos, t + 1 - bos)) {   // FP32 rows
#pragma unroll
        for (int i = 0; i < RPT; ++i)
#pragma unroll
          for (int m = 0; m < CPT; m += 4)
            StateIO<false>::store(
                (__attribute__((address_space(1))) float*)(cp + lane_elem + i * (RG * kHeadDim) + m),
                s[i] + m);
      }
    }
    if (dst) {
#pragma unroll
      for (int i = 0; i < RPT; ++i) {
        auto* row = (__attribute__((address_space(1))) elem*)(dst + i * (RG * kHeadDim));
        asm volatile("" : "+s"(row));
        IO::store(row + lane_elem, s[i]);
      }
    }
  }
};

template <int COLS, bool BF16, int NT>
__global__ __launch_bounds__(NT) void stream_kernel(PrefillArgs a) {
  using B = StreamBlock<COLS, BF16, NT>;
  __shared__ typename B::Smem sm;
  B::run(a, sm);
}

template <int COLS, bool BF16, int NT>
hipError_t launch_stream_shape(const PrefillArgs& a, hipStream_t s) {
  const int64_t units = (int64_t)a.num_seqs * a.num_heads * (kHeadDim / COLS);
  stream_kernel<COLS, BF16, NT><<<dim3((unsigned)units), NT, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill_stream(const PrefillArgs& a, int cols, hipStream_t s) {
  if (a.num_seqs <= 0) return hipSuccess;
  const bool bf16 = a.pool && a.pool_bf16;
  if (cols == 128)
    return bf16 ? launch_stream_shape<128, true, 512>(a, s) : launch_stream_shape<128, false, 512>(a, s);
  if (cols == 64)
    return bf16 ? launch_stream_shape<64, true, 512>(a, s) : launch_stream_shape<64, false, 512>(a, s);
  return hipErrorInvalidValue;
}

hipError_t launch_decode(const DecodeArgs& a, bool bf16_state, int cols, int threads,
                         hipStream_t s) {
  if (a.rows <= 0) return hipSuccess;
  return bf16_state ? launch_cols<true>(a, cols, threads, s)
                    : launch_cols<false>(a, cols, threads, s);
}

}  // namespace kda
