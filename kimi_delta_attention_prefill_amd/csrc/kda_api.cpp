// C ABI of the KDA library: host-side validation, route planning and launch.
// See include/kda.h for the contract of every entry point.
#include "kda.h"

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "kda_internal.h"

namespace {

thread_local char g_last_error[512] = "";
std::atomic<int> g_forced_route{KDA_ROUTE_AUTO};

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return code;
}

int ok() {
  g_last_error[0] = '\0';
  return KDA_OK;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Validates a kda_frontend (NULL = defaults) into *out; KDA_OK or the error.
int frontend_args(const kda_frontend* f, const char* fn, kda::FrontEnd* out) {
  *out = kda::FrontEnd{};
  if (!f) return KDA_OK;
  if (f->gate_mode != KDA_GATE_LOG && f->gate_mode != KDA_GATE_LOWER_BOUND &&
      f->gate_mode != KDA_GATE_SOFTPLUS)
    return fail(KDA_ERR_INVALID_ARGUMENT, "%s: unknown gate mode %d", fn, f->gate_mode);
  if (f->gate_mode == KDA_GATE_LOWER_BOUND && !(std::isfinite(f->lower_bound) && f->lower_bound < 0.f))
    return fail(KDA_ERR_INVALID_ARGUMENT, "%s: the lower-bound gate needs a finite bound < 0 (got %g)",
                fn, (double)f->lower_bound);
  if (!(std::isfinite(f->norm_eps) && f->norm_eps >= 0.f))
    return fail(KDA_ERR_INVALID_ARGUMENT, "%s: norm_eps must be finite and >= 0 (got %g)", fn,
                (double)f->norm_eps);
  out->gate_mode = f->gate_mode;
  out->lower_bound = f->lower_bound;
  out->beta_logits = f->beta_logits != 0;
  out->normalize_qk = f->normalize_qk != 0;
  out->norm_eps = f->norm_eps;
  return KDA_OK;
}

// Compute-unit count of the current device, cached per device id.
int current_device_cus() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
  if (dev < 64) {
    int c = cache[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return 0;
  if (dev < 64) cache[dev].store(cus, std::memory_order_relaxed);
  return cus;
}

// Largest |exponent| E of an anchored chunk-32 operand factor 2^{G-C} or
// 2^{C-G} when lower_bound <= g <= 0: 16 |lb| log2(e) (CAKE prefill note,
// section 1).  The pairwise products split each operand x into bf16 hi + lo,
// and lo is about 2^-9 |x|: for an entry of a unit-norm 128-channel row
// (|x| ~ 2^-3.5) scaled by 2^-E, lo keeps some 4 significant bits at E = 116
// and falls below bf16's subnormals at E = 126, where such products drop to
// bf16 precision (every gate at lower_bound = -10.875, E = 126: output errors
// of 8-12% of RMS).  The budget is therefore E <= 116, not the normal
// range's 126.
constexpr double kAnchorExpBudget = 116.0;
bool fixed_anchor_fits(float lower_bound) {
  return 16.0 * std::fabs((double)lower_bound) * 1.4426950408889634 <= kAnchorExpBudget;
}

// The same for the 16-token anchors at h' = the integer nearest h = 8 lb
// log2(e): a half's factors reach 2^{|h'|} and 2^{|2h - h'|}, so they fit
// while lower_bound >= -10.05; wider bounds take the data-dependent anchors.
bool half_anchor_fits(float lower_bound) {
  const double h = 8.0 * (double)lower_bound * 1.4426950408889634, hr = std::nearbyint(h);
  return std::fabs(hr) <= kAnchorExpBudget && std::fabs(2.0 * h - hr) <= kAnchorExpBudget;
}

// Argument checks shared by the prefill entry points; each returns KDA_OK or
// records the error and returns its code.
int check_sizes(const char* fn, int32_t num_seqs, int64_t total_tokens, int32_t num_heads,
                int32_t head_dim_k, int32_t head_dim_v) {
  if (head_dim_k != KDA_HEAD_DIM || head_dim_v != KDA_HEAD_DIM)
    return fail(KDA_ERR_UNSUPPORTED, "%s: head dims must be 128 (got dk=%d, dv=%d)", fn,
                head_dim_k, head_dim_v);
  if (num_seqs < 0 || num_heads < 1)
    return fail(KDA_ERR_INVALID_ARGUMENT, "%s: num_seqs=%d num_heads=%d", fn, num_seqs, num_heads);
  if (total_tokens < 0 || total_tokens > INT32_MAX)
    return fail(KDA_ERR_INVALID_ARGUMENT, "%s: total_tokens=%lld out of [0, 2^31)", fn,
                (long long)total_tokens);
  return KDA_OK;
}

// Pool slot stride in elements: 0 selects the dense layout (H * 128 * 128);
// otherwise slots must not overlap and every slot must start 16-byte
// aligned, as the pool does.  Rewrites 0 to the dense stride.
int check_slot_stride(const char* fn, int32_t num_heads, int32_t state_dtype,
                      int64_t* slot_stride) {
  const int64_t dense = (int64_t)num_heads * KDA_HEAD_DIM * KDA_HEAD_DIM;
  if (*slot_stride == 0) {
    *slot_stride = dense;
    return KDA_OK;
  }
  const int64_t elem = state_dtype == KDA_STATE_BF16 ? 2 : 4;
  if (*slot_stride < dense || (*slot_stride * elem) % 16 != 0)
    return fail(KDA_ERR_INVALID_ARGUMENT,
                "%s: slot_stride=%lld must be 0 or >= num_heads * 128 * 128 = %lld and a "
                "multiple of 16 bytes",
                fn, (long long)*slot_stride, (long long)dense);
  return KDA_OK;
}

// lower_bound: finite and < 0, or -infinity for an unbounded gate.
bool bound_ok(float lower_bound) {
  return lower_bound < 0.f && (std::isfinite(lower_bound) || std::isinf(lower_bound));
}

int check_bound(const char* fn, float lower_bound) {
  if (!bound_ok(lower_bound))
    return fail(KDA_ERR_INVALID_ARGUMENT, "%s: lower_bound must be < 0, finite or -inf (got %g)",
                fn, (double)lower_bound);
  return KDA_OK;
}

// The bound the chunk routes may rely on for the front-end's gate mode: the
// caller's bound for a log-decay gate, the sigmoid's scale for the
// lower-bound gate, none (-inf) for the softplus gate.
float effective_bound(const kda::FrontEnd& fe, float lower_bound) {
  if (fe.gate_mode == KDA_GATE_LOWER_BOUND) return fe.lower_bound;
  if (fe.gate_mode == KDA_GATE_SOFTPLUS) return -INFINITY;
  return lower_bound;
}

int check_inputs(const char* fn, const void* q, const void* k, const void* v, const void* g,
                 const void* beta, const int32_t* cu_seqlens, int64_t total_tokens) {
  if (!cu_seqlens) return fail(KDA_ERR_INVALID_ARGUMENT, "%s: cu_seqlens is NULL", fn);
  if (total_tokens == 0) return KDA_OK;
  const void* need[] = {q, k, v, g, beta};
  const char* names[] = {"q", "k", "v", "g", "beta"};
  for (int i = 0; i < 5; ++i) {
    if (!need[i]) return fail(KDA_ERR_INVALID_ARGUMENT, "%s: %s is NULL", fn, names[i]);
    if (i < 4 && !aligned(need[i], 16))
      return fail(KDA_ERR_INVALID_ARGUMENT, "%s: %s is not 16-byte aligned", fn, names[i]);
  }
  if (!aligned(beta, 2))
    return fail(KDA_ERR_INVALID_ARGUMENT, "%s: beta is not 2-byte aligned", fn);
  return KDA_OK;
}

int check_outputs(const char* fn, const float* initial_state, const float* final_state,
                  const void* out, int32_t num_seqs, int32_t num_heads, int64_t total_tokens) {
  if (total_tokens > 0) {
    if (!out) return fail(KDA_ERR_INVALID_ARGUMENT, "%s: out is NULL", fn);
    if (!aligned(out, 16))
      return fail(KDA_ERR_INVALID_ARGUMENT, "%s: out is not 16-byte aligned", fn);
  }
  if ((initial_state && !aligned(initial_state, 16)) || (final_state && !aligned(final_state, 16)))
    return fail(KDA_ERR_INVALID_ARGUMENT, "%s: states must be 16-byte aligned", fn);
  if (initial_state && final_state && initial_state != final_state) {
    const size_t bytes = (size_t)num_seqs * num_heads * KDA_HEAD_DIM * KDA_HEAD_DIM * 4;
    const char* a0 = reinterpret_cast<const char*>(initial_state);
    const char* b0 = reinterpret_cast<const char*>(final_state);
    if (a0 < b0 + bytes && b0 < a0 + bytes)
      return fail(KDA_ERR_INVALID_ARGUMENT, "%s: final_state partially overlaps initial_state", fn);
  }
  return KDA_OK;
}

int check_records(const char* fn, const void* ws, size_t bytes, size_t need) {
  if (!ws || bytes < need)
    return fail(KDA_ERR_WORKSPACE, "%s: workspace of %zu bytes needed (got %zu)", fn, need, bytes);
  if (!aligned(ws, 16))
    return fail(KDA_ERR_INVALID_ARGUMENT, "%s: workspace is not 16-byte aligned", fn);
  return KDA_OK;
}

kda::PrefillArgs make_args(const void* q, const void* k, const void* v, const void* g,
                           const void* beta, const int32_t* cu_seqlens, int32_t num_seqs,
                           int64_t total_tokens, int32_t num_heads, float scale,
                           float lower_bound, const float* initial_state, float* final_state,
                           void* out) {
  kda::PrefillArgs a;
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.g = static_cast<const uint16_t*>(g);
  a.beta = static_cast<const uint16_t*>(beta);
  a.cu_seqlens = cu_seqlens;
  a.num_seqs = num_seqs;
  a.total_tokens = (int32_t)total_tokens;
  a.num_heads = num_heads;
  a.scale = scale;
  // an unbounded gate (-inf) uses data-dependent anchors; the constants are unused
  const double lb = std::isfinite(lower_bound) ? (double)lower_bound : 0.0;
  a.anchor_log2 = (float)(16.0 * lb * 1.4426950408889634);
  // an integer, so that the off-diagonal tile can be rescaled by powers of two
  a.half_anchor_log2 = (float)std::nearbyint(8.0 * lb * 1.4426950408889634);
  a.s0 = initial_state;
  a.s1 = final_state;
  a.out = static_cast<uint16_t*>(out);
  a.windows = 1;
  a.window_chunks = 0;
  a.pool = nullptr;
  a.pool_bf16 = 0;
  a.slots = nullptr;
  a.num_slots = 0;
  a.slot_stride = 0;
  a.ckpt = nullptr;
  a.skip_null_slots = 0;
  a.ckpt_tokens = 0;
  return a;
}

}  // namespace

namespace kda {
int set_error(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return code;
}
}  // namespace kda

extern "C" {

size_t kda_prefill_workspace_size(int32_t num_seqs, int64_t total_tokens, int32_t num_heads) {
  if (num_seqs <= 0 || total_tokens < 0 || num_heads < 1) return 0;
  kda_prefill_plan_t plan;
  // The workspace does not depend on the bound; any valid one gives the route.
  if (kda_prefill_plan(num_seqs, total_tokens, num_heads, -1.0f, 0, g_forced_route.load(),
                       &plan) != KDA_OK)
    return 0;
  return plan.route == KDA_ROUTE_SPLIT
             ? kda::split_workspace_bytes(num_seqs, total_tokens, num_heads, plan.windows)
             : 0;
}

const char* kda_last_error(void) { return g_last_error; }

int kda_abi_version(void) { return KDA_ABI_VERSION; }

int kda_check_prefill_inputs(const void* q, const void* k, const void* v, const void* g,
                             const void* beta, const int32_t* cu_seqlens, int32_t num_seqs,
                             int64_t total_tokens, int32_t num_heads, float lower_bound,
                             int32_t* flags, hipStream_t stream) {
  if (num_seqs < 0 || total_tokens < 0 || num_heads < 1)
    return fail(KDA_ERR_INVALID_ARGUMENT,
                "kda_check_prefill_inputs: num_seqs=%d total_tokens=%lld num_heads=%d", num_seqs,
                (long long)total_tokens, num_heads);
  if (std::isnan(lower_bound) || !(lower_bound < 0.f))
    return fail(KDA_ERR_INVALID_ARGUMENT, "kda_check_prefill_inputs: lower_bound must be < 0");
  if (!flags || !aligned(flags, 4))
    return fail(KDA_ERR_INVALID_ARGUMENT, "kda_check_prefill_inputs: flags NULL or misaligned");
  if (!cu_seqlens || !aligned(cu_seqlens, 4))
    return fail(KDA_ERR_INVALID_ARGUMENT, "kda_check_prefill_inputs: cu_seqlens NULL or misaligned");
  if (total_tokens > 0) {
    const void* need[] = {q, k, v, g, beta};
    const char* names[] = {"q", "k", "v", "g", "beta"};
    for (int i = 0; i < 5; ++i)
      if (!need[i] || !aligned(need[i], 2))
        return fail(KDA_ERR_INVALID_ARGUMENT, "kda_check_prefill_inputs: %s NULL or misaligned",
                    names[i]);
  }
  kda::CheckPrefillArgs a;
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.g = static_cast<const uint16_t*>(g);
  a.beta = static_cast<const uint16_t*>(beta);
  a.cu_seqlens = cu_seqlens;
  a.num_seqs = num_seqs;
  a.total_tokens = total_tokens;
  a.num_heads = num_heads;
  a.lower_bound = lower_bound;
  a.bounded = std::isfinite(lower_bound);
  a.flags = flags;
  const hipError_t e = kda::launch_check_prefill(a, stream);
  if (e != hipSuccess)
    return fail(KDA_ERR_HIP, "kda_check_prefill_inputs: launch failed: %s", hipGetErrorString(e));
  return ok();
}

int kda_check_slots(const int32_t* slot_indices, int32_t rows, int64_t num_slots,
                    int32_t* flags, hipStream_t stream) {
  if (rows < 0 || num_slots < 1)
    return fail(KDA_ERR_INVALID_ARGUMENT, "kda_check_slots: rows=%d num_slots=%lld", rows,
                (long long)num_slots);
  if (!flags || !aligned(flags, 4))
    return fail(KDA_ERR_INVALID_ARGUMENT, "kda_check_slots: flags NULL or misaligned");
  if (rows > 0 && (!slot_indices || !aligned(slot_indices, 4)))
    return fail(KDA_ERR_INVALID_ARGUMENT, "kda_check_slots: slot_indices NULL or misaligned");
  const hipError_t e = kda::launch_check_slots(slot_indices, rows, num_slots, flags, stream);
  if (e != hipSuccess)
    return fail(KDA_ERR_HIP, "kda_check_slots: launch failed: %s", hipGetErrorString(e));
  return ok();
}

int kda_set_prefill_route(int32_t route) {
  if (route != KDA_ROUTE_AUTO && route != KDA_ROUTE_SERIAL && route != KDA_ROUTE_CHUNK &&
      route != KDA_ROUTE_SPLIT && route != KDA_ROUTE_STREAM)
    return fail(KDA_ERR_INVALID_ARGUMENT, "kda_set_prefill_route: unknown route %d", route);
  g_forced_route.store(route);
  return ok();
}


int kda_prefill_plan(int32_t num_seqs, int64_t total_tokens, int32_t num_heads,
                     float lower_bound, int32_t num_cus, int32_t route,
                     kda_prefill_plan_t* plan) {
  if (!plan) return fail(KDA_ERR_INVALID_ARGUMENT, "kda_prefill_plan: plan is NULL");
  if (num_seqs < 0 || total_tokens < 0 || num_heads < 1)
    return fail(KDA_ERR_INVALID_ARGUMENT, "kda_prefill_plan: bad sizes (N=%d, T=%lld, H=%d)",
                num_seqs, (long long)total_tokens, num_heads);
  if (!bound_ok(lower_bound))
    return fail(KDA_ERR_INVALID_ARGUMENT,
                "kda_prefill_plan: lower_bound must be < 0, finite or -inf (got %g)",
                (double)lower_bound);
  if (num_cus <= 0) num_cus = current_device_cus();
  if (num_cus <= 0) num_cus = 256;
  const int64_t units = (int64_t)num_seqs * num_heads;
  if (route == KDA_ROUTE_AUTO) {
    // Few recurrences: one block per (sequence, head) would idle most of the
    // chip and serialise chunk preparation, so prepare all chunks in
    // parallel first.  Many recurrences: keep everything in one pass.  The
    // split chain runs 8 blocks per recurrence, two per CU; measured on 256
    // CUs at T=8192 per sequence against the fused pipeline (1.10-1.15 ms
    // for up to 128 units): 64 units 0.73 ms, 80 units 1.14 vs 1.12 ms, 96
    // units 1.28 vs 1.14 ms, so the split route takes up to a quarter of
    // the CU count in units.
    // At most three chunks in the whole batch (so in every sequence): the
    // fused kernel's short serial loop beats the two-pass route's second
    // launch (measured at H=2: 8.8 vs 19.8 us at 32 tokens, 19.6 vs 20.8 us
    // at 96, 24.8 vs 21.2 us at 128).
    // Many short sequences (multi-token decode): the stream kernel reads and
    // writes each state once and runs the few token steps on it in
    // registers, where a fused block sets up its whole chunk pipeline for one
    // short chunk.  Measured from a 4096-slot FP32 pool at H = 8: 4096 rows
    // 0.74 / 0.92 / 1.59 / 2.71 ms at T = 2 / 4 / 8 / 16 against the fused
    // route's 2.30 / 2.33 / 2.41 / 2.56 ms; one row 8.8 vs 10.8 us at T = 4
    // but 15.0 vs 11.2 us at T = 8 (eight blocks, per-token latency exposed).
    const int64_t per_seq8 = 8 * (int64_t)num_seqs;
    if (total_tokens <= 4 * (int64_t)num_seqs ||
        (total_tokens <= per_seq8 && units >= (int64_t)num_cus))
      route = KDA_ROUTE_STREAM;
    else
      route = (4 * units <= (int64_t)num_cus && total_tokens > 3 * 32) ? KDA_ROUTE_SPLIT
                                                                       : KDA_ROUTE_CHUNK;
  }
  if (route != KDA_ROUTE_SERIAL && route != KDA_ROUTE_CHUNK && route != KDA_ROUTE_SPLIT &&
      route != KDA_ROUTE_STREAM)
    return fail(KDA_ERR_INVALID_ARGUMENT, "kda_prefill_plan: unknown route %d", route);
  std::memset(plan, 0, sizeof(*plan));
  plan->route = route;
  plan->windows = 1;
  plan->anchor_mode = !std::isfinite(lower_bound)       ? KDA_ANCHOR_DATA
                      : fixed_anchor_fits(lower_bound) ? KDA_ANCHOR_FIXED
                      : half_anchor_fits(lower_bound)  ? KDA_ANCHOR_SPLIT16
                                                       : KDA_ANCHOR_DATA;
  plan->anchor_log2 = std::isfinite(lower_bound)
                          ? (float)(16.0 * (double)lower_bound * 1.4426950408889634) : 0.f;
  if (route == KDA_ROUTE_STREAM) {
    // Whole 128-column items (512 threads) once there are enough of them to
    // fill the device, else two 64-column slices per (sequence, head).
    plan->dv_split = units >= 2 * (int64_t)num_cus ? 1 : 2;
    plan->block_threads = 512;
    plan->grid_blocks = units * plan->dv_split;
  } else if (route == KDA_ROUTE_SERIAL) {
    // 16 value columns per wave; fewer waves per block (more blocks) when
    // there are few (sequence, head) units to spread over the compute units.
    int waves = 4;
    if (2 * units < (int64_t)num_cus) waves = 4 * units < (int64_t)num_cus ? 1 : 2;
    plan->dv_split = 8 / waves;
    plan->block_threads = 64 * waves;
    plan->grid_blocks = units * plan->dv_split;
  } else if (route == KDA_ROUTE_SPLIT) {
    // Chain pass: one block (two state waves, a U wave and an output wave)
    // per 16 kSplitSubtiles value columns of each (sequence, head); two blocks
    // fit a CU.
    plan->dv_split = kda::kSplitChainTiles;
    plan->block_threads = 256;
    plan->grid_blocks = units * kda::kSplitChainTiles;
    plan->windows = 1;
    // Chains that fill a small part of the device: cut each sequence into up
    // to W windows so that phase A (first window + inner windows' maps, 1 +
    // 2 (W - 2) chains per (sequence, head)) and phase C (W - 1 chains) each
    // fit the CUs at kSplitBlocksPerCU blocks each.  The device cuts every
    // sequence by its own length (max(8, ceil(chunks / W)) chunks per
    // window), so W is sized here from the average sequence (windows of at
    // least 8 chunks); window_chunks reports the cut of a sequence as long as
    // the whole batch.
    const int64_t chunks = (total_tokens + 31) / 32;
    if (num_seqs >= 1) {
      const int64_t tiles = units * kda::kSplitChainTiles;
      const int64_t slots = kda::kSplitBlocksPerCU * (int64_t)num_cus;
      int64_t w = 1;
      while (w < 8 && tiles * (1 + 2 * (w + 1 - 2)) <= slots && tiles * w <= slots) ++w;
      w = std::min<int64_t>(w, chunks / num_seqs / 8);   // windows of at least 8 chunks
      // Three windows shorten a chain to about 2/3 of its steps plus the
      // carry: measured on 4 x 4096 tokens at H = 4 (128 chunks per sequence)
      // that no longer pays (116.9 vs 114.5 us), on 2 x 8192 at H = 8 (256
      // chunks) it does (242 vs 263 us).
      if (w == 3 && chunks / num_seqs < 192) w = 1;
      if (w >= 3) {
        const int64_t wc = std::max<int64_t>(8, (chunks + w - 1) / w);
        plan->window_chunks = (int32_t)wc;
        // one sequence: the windows its cut actually yields
        plan->windows = num_seqs == 1 ? (int32_t)((chunks + wc - 1) / wc) : (int32_t)w;
      }
    }
  } else {
    // One block per (sequence, head, value slice).  Two 64-column slices
    // halve the per-block chain work at the cost of duplicated chunk
    // preparation; worth it only while every block still gets its own CU.
    plan->dv_split = 2 * units <= (int64_t)num_cus ? 2 : 1;
    if (plan->anchor_mode == KDA_ANCHOR_DATA) plan->dv_split = 2;   // 64-column blocks only
    plan->block_threads = 256;
    plan->grid_blocks = units * plan->dv_split;
  }
  return ok();
}

}  // extern "C"

namespace {

// Plan, check the workspace and launch a prefill whose arguments have been
// validated.
int run_prefill(const char* fn, kda::PrefillArgs a, float lower_bound, void* workspace,
                size_t workspace_bytes, hipStream_t stream) {
  kda_prefill_plan_t plan;
  int rc = kda_prefill_plan(a.num_seqs, a.total_tokens, a.num_heads, lower_bound, 0,
                            g_forced_route.load(), &plan);
  if (rc != KDA_OK) return rc;
  if (plan.route == KDA_ROUTE_SPLIT &&
      (rc = check_records(fn, workspace, workspace_bytes,
                          kda::split_workspace_bytes(a.num_seqs, a.total_tokens, a.num_heads,
                                                     plan.windows))) != KDA_OK)
    return rc;
  a.windows = plan.windows;
  a.window_chunks = plan.window_chunks;
  hipError_t e;
  if (plan.route == KDA_ROUTE_SERIAL)
    e = kda::launch_prefill_serial(a, plan.block_threads / 64, stream);
  else if (plan.route == KDA_ROUTE_STREAM)
    e = kda::launch_prefill_stream(a, 128 / plan.dv_split, stream);
  else if (plan.route == KDA_ROUTE_SPLIT)
    e = kda::launch_prefill_split(a, plan.anchor_mode, plan.dv_split, workspace, stream);
  else   // with the input front-end the fused route runs 64-column blocks only
    e = kda::launch_prefill_chunk(a, plan.anchor_mode,
                                  kda::frontend_active(a.fe) ? 2 : plan.dv_split, stream);
  if (e == hipErrorNotSupported)
    return fail(KDA_ERR_UNSUPPORTED, "%s: route %d is not available", fn, plan.route);
  if (e != hipSuccess) return fail(KDA_ERR_HIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
  return ok();
}

}  // namespace

extern "C" {

int kda_prefill_ex(const void* q, const void* k, const void* v, const void* g, const void* beta,
                   const int32_t* cu_seqlens, int32_t num_seqs, int64_t total_tokens,
                   int32_t num_heads, int32_t head_dim_k, int32_t head_dim_v, float scale,
                   float lower_bound, const kda_frontend* frontend,
                   const float* initial_state, float* final_state, void* out,
                   void* workspace, size_t workspace_bytes, hipStream_t stream) {
  const char* fn = "kda_prefill";
  kda::FrontEnd fe;
  int rc = frontend_args(frontend, fn, &fe);
  if (rc != KDA_OK) return rc;
  if ((rc = check_sizes(fn, num_seqs, total_tokens, num_heads, head_dim_k, head_dim_v)) != KDA_OK)
    return rc;
  if (!std::isfinite(scale)) return fail(KDA_ERR_INVALID_ARGUMENT, "%s: scale is not finite", fn);
  if (fe.gate_mode == KDA_GATE_LOG && (rc = check_bound(fn, lower_bound)) != KDA_OK) return rc;
  lower_bound = effective_bound(fe, lower_bound);
  if (num_seqs == 0) return ok();
  if ((rc = check_inputs(fn, q, k, v, g, beta, cu_seqlens, total_tokens)) != KDA_OK) return rc;
  if ((rc = check_outputs(fn, initial_state, final_state, out, num_seqs, num_heads,
                          total_tokens)) != KDA_OK)
    return rc;
  kda::PrefillArgs a = make_args(q, k, v, g, beta, cu_seqlens, num_seqs, total_tokens, num_heads,
                                 scale, lower_bound, initial_state, final_state, out);
  a.fe = fe;
  return run_prefill(fn, a, lower_bound, workspace, workspace_bytes, stream);
}

int kda_prefill(const void* q, const void* k, const void* v, const void* g, const void* beta,
                const int32_t* cu_seqlens, int32_t num_seqs, int64_t total_tokens,
                int32_t num_heads, int32_t head_dim_k, int32_t head_dim_v, float scale,
                float lower_bound, const float* initial_state, float* final_state, void* out,
                void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return kda_prefill_ex(q, k, v, g, beta, cu_seqlens, num_seqs, total_tokens, num_heads,
                        head_dim_k, head_dim_v, scale, lower_bound, nullptr, initial_state,
                        final_state, out, workspace, workspace_bytes, stream);
}

int kda_prefill_pool_ex(const void* q, const void* k, const void* v, const void* g,
                        const void* beta, const int32_t* cu_seqlens, int32_t num_seqs,
                        int64_t total_tokens, int32_t num_heads, int32_t head_dim_k,
                        int32_t head_dim_v, float scale, float lower_bound,
                        const kda_frontend* frontend, void* state_pool, int32_t state_dtype,
                        int64_t num_slots, int64_t slot_stride, const int32_t* slot_indices,
                        float* checkpoints, int32_t checkpoint_tokens, void* out,
                        void* workspace, size_t workspace_bytes, hipStream_t stream) {
  const char* fn = "kda_prefill_pool";
  kda::FrontEnd fe;
  int rc = frontend_args(frontend, fn, &fe);
  if (rc != KDA_OK) return rc;
  if ((rc = check_sizes(fn, num_seqs, total_tokens, num_heads, head_dim_k, head_dim_v)) != KDA_OK)
    return rc;
  if (!std::isfinite(scale)) return fail(KDA_ERR_INVALID_ARGUMENT, "%s: scale is not finite", fn);
  if (fe.gate_mode == KDA_GATE_LOG && (rc = check_bound(fn, lower_bound)) != KDA_OK) return rc;
  lower_bound = effective_bound(fe, lower_bound);
  if (state_dtype != KDA_STATE_F32 && state_dtype != KDA_STATE_BF16)
    return fail(KDA_ERR_INVALID_ARGUMENT, "%s: unknown state dtype %d", fn, state_dtype);
  if (state_pool) {
    if (num_slots < 1)
      return fail(KDA_ERR_INVALID_ARGUMENT, "%s: num_slots=%lld", fn, (long long)num_slots);
    if (!aligned(state_pool, 16))
      return fail(KDA_ERR_INVALID_ARGUMENT, "%s: state_pool is not 16-byte aligned", fn);
    if ((rc = check_slot_stride(fn, num_heads, state_dtype, &slot_stride)) != KDA_OK) return rc;
  }
  if (checkpoints) {
    if (checkpoint_tokens <= 0 || checkpoint_tokens % 32 != 0)
      return fail(KDA_ERR_INVALID_ARGUMENT,
                  "%s: checkpoint_tokens must be a positive multiple of 32 (got %d)", fn,
                  checkpoint_tokens);
    if (!aligned(checkpoints, 16))
      return fail(KDA_ERR_INVALID_ARGUMENT, "%s: checkpoints are not 16-byte aligned", fn);
  }
  if (num_seqs == 0) return ok();
  if (state_pool && (!slot_indices || !aligned(slot_indices, 4)))
    return fail(KDA_ERR_INVALID_ARGUMENT, "%s: slot_indices is NULL or misaligned", fn);
  if ((rc = check_inputs(fn, q, k, v, g, beta, cu_seqlens, total_tokens)) != KDA_OK) return rc;
  if ((rc = check_outputs(fn, nullptr, nullptr, out, num_seqs, num_heads, total_tokens)) != KDA_OK)
    return rc;
  kda::PrefillArgs a = make_args(q, k, v, g, beta, cu_seqlens, num_seqs, total_tokens, num_heads,
                                 scale, lower_bound, nullptr, nullptr, out);
  a.pool = state_pool;
  a.pool_bf16 = state_dtype == KDA_STATE_BF16;
  a.slots = slot_indices;
  a.num_slots = num_slots;
  a.slot_stride = slot_stride;
  a.ckpt = checkpoints;
  a.ckpt_tokens = checkpoints ? checkpoint_tokens : 0;
  a.fe = fe;
  return run_prefill(fn, a, lower_bound, workspace, workspace_bytes, stream);
}

int kda_prefill_pool(const void* q, const void* k, const void* v, const void* g,
                     const void* beta, const int32_t* cu_seqlens, int32_t num_seqs,
                     int64_t total_tokens, int32_t num_heads, int32_t head_dim_k,
                     int32_t head_dim_v, float scale, float lower_bound, float* state_pool,
                     int64_t num_slots, const int32_t* slot_indices, float* checkpoints,
                     int32_t checkpoint_tokens, void* out, void* workspace,
                     size_t workspace_bytes, hipStream_t stream) {
  return kda_prefill_pool_ex(q, k, v, g, beta, cu_seqlens, num_seqs, total_tokens, num_heads,
                             head_dim_k, head_dim_v, scale, lower_bound, nullptr, state_pool,
                             KDA_STATE_F32, num_slots, 0, slot_indices, checkpoints,
                             checkpoint_tokens, out, workspace, workspace_bytes, stream);
}

size_t kda_prefill_checkpoint_slots(int32_t num_seqs, int64_t total_tokens,
                                    int32_t checkpoint_tokens) {
  if (num_seqs < 0 || total_tokens < 0 || checkpoint_tokens <= 0) return 0;
  return (size_t)num_seqs + (size_t)(total_tokens / checkpoint_tokens) + 1;
}

// The SPLIT route's plan for these sizes on the current device.
int split_plan(const char* fn, int32_t num_seqs, int64_t total_tokens, int32_t num_heads,
               float lower_bound, kda_prefill_plan_t* plan) {
  const int rc = kda_prefill_plan(num_seqs, total_tokens, num_heads, lower_bound, 0,
                                  KDA_ROUTE_SPLIT, plan);
  if (rc != KDA_OK) return fail(rc, "%s: %s", fn, kda_last_error());
  return KDA_OK;
}

size_t kda_prefill_records_size(int32_t num_seqs, int64_t total_tokens, int32_t num_heads) {
  if (num_seqs <= 0 || total_tokens < 0 || total_tokens > INT32_MAX || num_heads < 1) return 0;
  kda_prefill_plan_t plan;
  if (kda_prefill_plan(num_seqs, total_tokens, num_heads, -1.0f, 0, KDA_ROUTE_SPLIT, &plan) !=
      KDA_OK)
    return 0;
  return kda::split_workspace_bytes(num_seqs, total_tokens, num_heads, plan.windows);
}

int kda_prefill_prepare(const void* q, const void* k, const void* v, const void* g,
                        const void* beta, const int32_t* cu_seqlens, int32_t num_seqs,
                        int64_t total_tokens, int32_t num_heads, int32_t head_dim_k,
                        int32_t head_dim_v, float lower_bound, void* records,
                        size_t records_bytes, hipStream_t stream) {
  const char* fn = "kda_prefill_prepare";
  int rc = check_sizes(fn, num_seqs, total_tokens, num_heads, head_dim_k, head_dim_v);
  if (rc != KDA_OK) return rc;
  if ((rc = check_bound(fn, lower_bound)) != KDA_OK) return rc;
  if (num_seqs == 0) return ok();
  if ((rc = check_inputs(fn, q, k, v, g, beta, cu_seqlens, total_tokens)) != KDA_OK) return rc;
  kda_prefill_plan_t plan;
  if ((rc = split_plan(fn, num_seqs, total_tokens, num_heads, lower_bound, &plan)) != KDA_OK)
    return rc;
  if ((rc = check_records(fn, records, records_bytes,
                          kda::split_workspace_bytes(num_seqs, total_tokens, num_heads,
                                                     plan.windows))) != KDA_OK)
    return rc;
  kda::PrefillArgs a = make_args(q, k, v, g, beta, cu_seqlens, num_seqs, total_tokens, num_heads,
                                 1.f, lower_bound, nullptr, nullptr, nullptr);
  a.windows = plan.windows;
  a.window_chunks = plan.window_chunks;
  const hipError_t e = kda::launch_prefill_split_prepare(a, plan.anchor_mode, records, stream);
  if (e != hipSuccess) return fail(KDA_ERR_HIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
  return ok();
}

int kda_prefill_chain(const int32_t* cu_seqlens, int32_t num_seqs, int64_t total_tokens,
                      int32_t num_heads, float scale, const float* initial_state,
                      float* final_state, void* out, const void* records, size_t records_bytes,
                      hipStream_t stream) {
  const char* fn = "kda_prefill_chain";
  int rc = check_sizes(fn, num_seqs, total_tokens, num_heads, KDA_HEAD_DIM, KDA_HEAD_DIM);
  if (rc != KDA_OK) return rc;
  if (!std::isfinite(scale)) return fail(KDA_ERR_INVALID_ARGUMENT, "%s: scale is not finite", fn);
  if (num_seqs == 0) return ok();
  if (!cu_seqlens) return fail(KDA_ERR_INVALID_ARGUMENT, "%s: cu_seqlens is NULL", fn);
  if ((rc = check_outputs(fn, initial_state, final_state, out, num_seqs, num_heads,
                          total_tokens)) != KDA_OK)
    return rc;
  kda_prefill_plan_t plan;
  if ((rc = split_plan(fn, num_seqs, total_tokens, num_heads, -1.f, &plan)) != KDA_OK) return rc;
  if ((rc = check_records(fn, records, records_bytes,
                          kda::split_workspace_bytes(num_seqs, total_tokens, num_heads,
                                                     plan.windows))) != KDA_OK)
    return rc;
  kda::PrefillArgs a = make_args(nullptr, nullptr, nullptr, nullptr, nullptr, cu_seqlens,
                                 num_seqs, total_tokens, num_heads, scale, -1.f, initial_state,
                                 final_state, out);
  a.windows = plan.windows;
  a.window_chunks = plan.window_chunks;
  const hipError_t e = kda::launch_prefill_split_chain(a, records, stream);
  if (e != hipSuccess) return fail(KDA_ERR_HIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
  return ok();
}

int kda_decode_ex(const void* q, const void* k, const void* v, const void* g, const void* beta,
                  void* state_pool, int32_t state_dtype, int64_t num_slots,
                  int64_t slot_stride, const int32_t* slot_indices, int32_t rows,
                  int32_t num_heads, int32_t head_dim_k, int32_t head_dim_v, float scale,
                  const kda_frontend* frontend, void* out, hipStream_t stream) {
  kda::FrontEnd fe;
  if (const int st = frontend_args(frontend, "kda_decode", &fe)) return st;
  if (head_dim_k != KDA_HEAD_DIM || head_dim_v != KDA_HEAD_DIM)
    return fail(KDA_ERR_UNSUPPORTED, "kda_decode: head dims must be 128 (got dk=%d, dv=%d)",
                head_dim_k, head_dim_v);
  if (state_dtype != KDA_STATE_F32 && state_dtype != KDA_STATE_BF16)
    return fail(KDA_ERR_INVALID_ARGUMENT, "kda_decode: unknown state dtype %d", state_dtype);
  if (rows < 0 || num_heads < 1 || num_slots < 1)
    return fail(KDA_ERR_INVALID_ARGUMENT, "kda_decode: rows=%d num_heads=%d num_slots=%lld",
                rows, num_heads, (long long)num_slots);
  if (!std::isfinite(scale)) return fail(KDA_ERR_INVALID_ARGUMENT, "kda_decode: scale not finite");
  if (const int st = check_slot_stride("kda_decode", num_heads, state_dtype, &slot_stride))
    return st;
  if ((int64_t)rows * num_heads * 4 > (int64_t)UINT32_MAX)
    return fail(KDA_ERR_INVALID_ARGUMENT, "kda_decode: rows * num_heads too large");
  if (rows == 0) return ok();
  const void* need[] = {q, k, v, g, beta, state_pool, slot_indices, out};
  const char* names[] = {"q", "k", "v", "g", "beta", "state_pool", "slot_indices", "out"};
  for (int i = 0; i < 8; ++i)
    if (!need[i]) return fail(KDA_ERR_INVALID_ARGUMENT, "kda_decode: %s is NULL", names[i]);
  const void* al16[] = {q, k, v, g, out, state_pool};
  const char* n16[] = {"q", "k", "v", "g", "out", "state_pool"};
  for (int i = 0; i < 6; ++i)
    if (!aligned(al16[i], 16))
      return fail(KDA_ERR_INVALID_ARGUMENT, "kda_decode: %s is not 16-byte aligned", n16[i]);
  if (!aligned(beta, 2) || !aligned(slot_indices, 4))
    return fail(KDA_ERR_INVALID_ARGUMENT, "kda_decode: beta/slot_indices misaligned");

  kda::DecodeArgs a;
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.g = static_cast<const uint16_t*>(g);
  a.beta = static_cast<const uint16_t*>(beta);
  a.pool = state_pool;
  a.slots = slot_indices;
  a.num_slots = num_slots;
  a.slot_stride = slot_stride;
  a.rows = rows;
  a.num_heads = num_heads;
  a.scale = scale;
  a.out = static_cast<uint16_t*>(out);
  a.fe = fe;

  // Many items: the token-stream kernel with one token per row (whole-item
  // 512-thread blocks, two resident per CU; 4096 rows x H=8 FP32 0.74 ms
  // against 0.77-0.81 ms for the decode blocks below; BF16 gains only from
  // about 2048 rows, 204 vs 207 us).  Fewer: decode blocks, narrow
  // value-column slices when the items cannot fill the chip.
  int cus = current_device_cus();
  if (cus <= 0) cus = 256;
  const int64_t items = (int64_t)rows * num_heads;
  const bool bf16 = state_dtype == KDA_STATE_BF16;
  hipError_t e;
  if (items >= (bf16 ? 16LL : 8LL) * cus) {
    kda::PrefillArgs p = make_args(q, k, v, g, beta, nullptr, rows, rows, num_heads, scale, -1.f,
                                   nullptr, nullptr, out);
    p.pool = state_pool;
    p.pool_bf16 = bf16;
    p.slots = slot_indices;
    p.num_slots = num_slots;
    p.slot_stride = slot_stride;
    p.fe = fe;
    p.skip_null_slots = 1;
    e = kda::launch_prefill_stream(p, 128, stream);
  } else {
    int cols = 128, threads = 512;
    if (items < 2LL * cus) {
      if (bf16) {
        cols = 64;
      } else {
        cols = items >= cus ? 64 : 32;
        threads = 256;
      }
    }
    e = kda::launch_decode(a, bf16, cols, threads, stream);
  }
  if (e != hipSuccess)
    return fail(KDA_ERR_HIP, "kda_decode: launch failed: %s", hipGetErrorString(e));
  return ok();
}

int kda_decode(const void* q, const void* k, const void* v, const void* g, const void* beta,
               void* state_pool, int32_t state_dtype, int64_t num_slots,
               const int32_t* slot_indices, int32_t rows, int32_t num_heads, int32_t head_dim_k,
               int32_t head_dim_v, float scale, void* out, hipStream_t stream) {
  return kda_decode_ex(q, k, v, g, beta, state_pool, state_dtype, num_slots, 0, slot_indices,
                       rows, num_heads, head_dim_k, head_dim_v, scale, nullptr, out, stream);
}

}  // extern "C"
