// api.hip -- the C ABI of libgdn (include/gdn.h): argument validation, then
// kernel launches on the caller's stream.  Every argument check runs on the
// host before any HIP call, so invalid calls return without touching the
// device (and can be exercised without a GPU).
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <mutex>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <vector>

#include "../../include/gdn.h"
#include "launch.h"

namespace {

thread_local std::string g_last_error;

gdn_status fail(gdn_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
gdn_status fail(gdn_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

gdn_status hip_status(hipError_t e, const char* where) {
  if (e == hipSuccess) return GDN_OK;
  return fail(GDN_ERR_HIP, "%s: %s", where, hipGetErrorString(e));
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Byte range [lo, hi) of a tensor with `rows` rows of `width` elements at a
// row stride of `stride` elements.
struct Range {
  uintptr_t lo = 0, hi = 0;
};
Range range_of(const void* p, int64_t rows, int64_t stride, int64_t width, size_t elem) {
  Range r;
  if (!p || rows <= 0 || width <= 0) return r;
  r.lo = reinterpret_cast<uintptr_t>(p);
  r.hi = r.lo + static_cast<uintptr_t>(((rows - 1) * stride + width) * static_cast<int64_t>(elem));
  return r;
}
bool overlap(const Range& a, const Range& b) {
  return a.lo < a.hi && b.lo < b.hi && a.lo < b.hi && b.lo < a.hi;
}

bool env_validate_seqlens() {
  const char* v = std::getenv("GDN_VALIDATE_CU_SEQLENS");
  return v && v[0] == '1';
}

// Sequence-count / length consistency when cu_seqlens is absent.
gdn_status check_equal_split(int32_t n_seqs, int32_t T_total) {
  if (n_seqs < 0 || T_total < 0) return fail(GDN_ERR_SHAPE, "negative n_seqs or T_total");
  if (n_seqs == 0 && T_total != 0) return fail(GDN_ERR_SHAPE, "T_total > 0 with no sequences");
  if (n_seqs > 0 && T_total % n_seqs != 0)
    return fail(GDN_ERR_SHAPE, "T_total %d not divisible by n_seqs %d without cu_seqlens",
                T_total, n_seqs);
  return GDN_OK;
}

}  // namespace

extern "C" {

const char* gdn_status_string(gdn_status s) {
  switch (s) {
    case GDN_OK: return "GDN_OK";
    case GDN_ERR_NULL: return "GDN_ERR_NULL";
    case GDN_ERR_SHAPE: return "GDN_ERR_SHAPE";
    case GDN_ERR_UNSUPPORTED: return "GDN_ERR_UNSUPPORTED";
    case GDN_ERR_WORKSPACE: return "GDN_ERR_WORKSPACE";
    case GDN_ERR_ALIAS: return "GDN_ERR_ALIAS";
    case GDN_ERR_HIP: return "GDN_ERR_HIP";
    case GDN_ERR_SEQLENS: return "GDN_ERR_SEQLENS";
    default: return "GDN_ERR_UNKNOWN";
  }
}

const char* gdn_last_error(void) { return g_last_error.c_str(); }

int32_t gdn_abi_version(void) { return GDN_ABI_VERSION; }

gdn_status gdn_validate_cu_seqlens(const int32_t* cu_seqlens, int32_t n_seqs, int32_t T_total,
                                   void* stream) {
  if (!cu_seqlens) return fail(GDN_ERR_NULL, "cu_seqlens is NULL");
  if (n_seqs < 0 || T_total < 0) return fail(GDN_ERR_SHAPE, "negative n_seqs or T_total");
  std::vector<int32_t> h(static_cast<size_t>(n_seqs) + 1);
  hipStream_t st = static_cast<hipStream_t>(stream);
  gdn_status s = hip_status(hipMemcpyAsync(h.data(), cu_seqlens, h.size() * sizeof(int32_t),
                                           hipMemcpyDeviceToHost, st),
                            "gdn_validate_cu_seqlens copy");
  if (s) return s;
  s = hip_status(hipStreamSynchronize(st), "gdn_validate_cu_seqlens sync");
  if (s) return s;
  if (h[0] != 0) return fail(GDN_ERR_SEQLENS, "cu_seqlens[0] = %d, expected 0", h[0]);
  for (int32_t i = 0; i < n_seqs; ++i)
    if (h[i + 1] < h[i])
      return fail(GDN_ERR_SEQLENS, "cu_seqlens decreases at %d (%d -> %d)", i, h[i], h[i + 1]);
  if (h[n_seqs] != T_total)
    return fail(GDN_ERR_SEQLENS, "cu_seqlens[%d] = %d, expected T_total %d", n_seqs, h[n_seqs],
                T_total);
  return GDN_OK;
}

gdn_status gdn_conv1d_fwd(const uint16_t* x, int64_t x_row_stride, const uint16_t* w,
                          const float* bias, uint16_t* y, int64_t y_row_stride,
                          uint16_t* conv_state, const int32_t* cu_seqlens, int32_t n_seqs,
                          int32_t T_total, int32_t C, int32_t n_l2_heads, int32_t head_dim,
                          float l2_eps, void* stream) {
  if (T_total > 0 && (!x || !w || !y))
    return fail(GDN_ERR_NULL, "gdn_conv1d_fwd: x, w and y are required");
  if (n_seqs < 0 || T_total < 0 || C <= 0 || n_l2_heads < 0)
    return fail(GDN_ERR_SHAPE, "gdn_conv1d_fwd: bad sizes");
  if (head_dim != 128) return fail(GDN_ERR_UNSUPPORTED, "gdn_conv1d_fwd: head_dim must be 128");
  if (C % 8) return fail(GDN_ERR_UNSUPPORTED, "gdn_conv1d_fwd: C must be a multiple of 8");
  if (static_cast<int64_t>(n_l2_heads) * head_dim > C)
    return fail(GDN_ERR_SHAPE, "gdn_conv1d_fwd: n_l2_heads * head_dim > C");
  if (x_row_stride < C || y_row_stride < C || x_row_stride % 8 || y_row_stride % 8)
    return fail(GDN_ERR_SHAPE, "gdn_conv1d_fwd: row strides must be >= C and multiples of 8");
  if (!aligned(x, 16) || !aligned(y, 16) || !aligned(w, 16) || !aligned(conv_state, 16) ||
      !aligned(bias, 4) || !aligned(cu_seqlens, 4))
    return fail(GDN_ERR_SHAPE, "gdn_conv1d_fwd: x, y, w, conv_state must be 16-byte aligned");
  if (!(l2_eps >= 0.f) || !std::isfinite(l2_eps))
    return fail(GDN_ERR_SHAPE, "gdn_conv1d_fwd: l2_eps must be finite and >= 0");
  if (!cu_seqlens) {
    const gdn_status s = check_equal_split(n_seqs, T_total);
    if (s) return s;
  } else if (n_seqs == 0 && T_total != 0) {
    return fail(GDN_ERR_SHAPE, "gdn_conv1d_fwd: T_total > 0 with no sequences");
  }
  const Range rx = range_of(x, T_total, x_row_stride, C, 2);
  const Range ry = range_of(y, T_total, y_row_stride, C, 2);
  const Range rs = range_of(conv_state, n_seqs, 3LL * C, 3LL * C, 2);
  const Range rw = range_of(w, C, 4, 4, 2);
  if (overlap(rx, ry) || overlap(ry, rs) || overlap(rx, rs) || overlap(rw, ry) || overlap(rw, rs))
    return fail(GDN_ERR_ALIAS, "gdn_conv1d_fwd: x, y, w and conv_state must not overlap");
  if (cu_seqlens && env_validate_seqlens()) {
    const gdn_status s = gdn_validate_cu_seqlens(cu_seqlens, n_seqs, T_total, stream);
    if (s) return s;
  }
  return hip_status(gdn::launch_conv1d(x, x_row_stride, w, bias, y, y_row_stride, conv_state,
                                       cu_seqlens, n_seqs, T_total, C, n_l2_heads * head_dim,
                                       l2_eps, static_cast<hipStream_t>(stream)),
                    "gdn_conv1d_fwd launch");
}

size_t gdn_chunk_fwd_workspace_bytes(int32_t n_seqs, int32_t T_total, int32_t Hk, int32_t Hv,
                                     int32_t d) {
  (void)d;
  if (n_seqs < 0 || T_total < 0 || Hk <= 0 || Hv <= 0) return 0;
  return gdn::chunk_workspace_layout(n_seqs, T_total, Hk, Hv).total;
}

gdn_status gdn_chunk_map(const int32_t* cu_seqlens, int32_t n_seqs, int32_t T_total,
                         int32_t* order, int32_t* chunk_off, int32_t* chunk_tab, void* stream) {
  if (!cu_seqlens || !order || !chunk_off || !chunk_tab)
    return fail(GDN_ERR_NULL, "gdn_chunk_map: all pointers are required");
  if (n_seqs < 0 || T_total < 0) return fail(GDN_ERR_SHAPE, "gdn_chunk_map: bad sizes");
  if (!aligned(cu_seqlens, 4) || !aligned(order, 4) || !aligned(chunk_off, 4) ||
      !aligned(chunk_tab, 4))
    return fail(GDN_ERR_SHAPE, "gdn_chunk_map: arrays must be 4-byte aligned");
  if (env_validate_seqlens()) {
    const gdn_status s = gdn_validate_cu_seqlens(cu_seqlens, n_seqs, T_total, stream);
    if (s) return s;
  }
  return hip_status(gdn::launch_chunk_map(cu_seqlens, n_seqs, T_total, order, chunk_off,
                                          chunk_tab, static_cast<hipStream_t>(stream)),
                    "gdn_chunk_map launch");
}

// ---- static workspace of gdn_chunk_fwd_noalloc ------------------------------
// A file-scope device array stands in for the caller's workspace in the one
// prefill entry point that allocates nothing.  Each GPU the library runs on
// holds its own copy from module load until the process ends.  In host code
// `scratch` names a host-side stand-in, never the device memory: the device
// address of the current GPU's copy comes from hipGetSymbolAddress, looked up
// once per device with that device current, and only that address is passed on.
constexpr size_t kScratchBytes = static_cast<size_t>(64) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::once_flag g_scratch_once[kMaxDevices];
void* g_scratch_ptr[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];

// The device address of the current GPU's copy of `scratch`.
gdn_status scratch_address(void** out) {
  int dev = -1;
  const hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, "gdn_chunk_fwd_noalloc: hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices)
    return fail(GDN_ERR_UNSUPPORTED, "gdn_chunk_fwd_noalloc: device %d beyond the %d supported", dev,
                kMaxDevices);
  std::call_once(g_scratch_once[dev], [dev] {
    void* ptr = nullptr;
    g_scratch_err[dev] = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    g_scratch_ptr[dev] = ptr;
  });
  if (g_scratch_err[dev] != hipSuccess)
    return hip_status(g_scratch_err[dev], "gdn_chunk_fwd_noalloc: hipGetSymbolAddress(scratch)");
  *out = g_scratch_ptr[dev];
  return GDN_OK;
}
}  // namespace

// Shared by gdn_chunk_fwd (fp32 o) and gdn_chunk_fwd_bf16o (bf16 o).
// The common host side of the prefill entry points.  `gates` holds either g,
// beta or the projections a, b with A_log, dt_bias; with `state_slot` the
// initial and final states are one pool (h0 == hT) indexed per sequence.
static gdn_status chunk_fwd(const char* fn, const uint16_t* q, int64_t q_tok_stride,
                            const uint16_t* k, int64_t k_tok_stride, const uint16_t* v,
                            int64_t v_tok_stride, const gdn::GateInputs& gates, void* o, bool o_bf16,
                            const float* initial_state, float* final_state,
                            const int32_t* state_slot, int32_t n_slots,
                            const int32_t* cu_seqlens, int32_t n_seqs, int32_t T_total, int32_t Hk,
                            int32_t Hv, int32_t dk, int32_t dv, float scale, void* workspace,
                            size_t workspace_bytes, void* stream, bool use_scratch = false) {
  const bool projected = gates.a != nullptr || gates.b != nullptr || gates.A_log != nullptr ||
                         gates.dt_bias != nullptr;
  const bool gates_given = projected ? (gates.a && gates.b && gates.A_log && gates.dt_bias)
                                     : (gates.g && gates.beta);
  if (T_total > 0 && (!q || !k || !v || !gates_given || !o))
    return fail(GDN_ERR_NULL, "%s: q, k, v, the gates and o are required", fn);
  if (state_slot && n_seqs > 0 && !initial_state)
    return fail(GDN_ERR_NULL, "%s: the state pool is required", fn);
  if (n_seqs < 0 || T_total < 0 || Hk <= 0 || Hv <= 0 || Hv % Hk)
    return fail(GDN_ERR_SHAPE, "%s: bad sizes or Hv %% Hk != 0", fn);
  if (dk != 128 || dv != 128) return fail(GDN_ERR_UNSUPPORTED, "%s: dk = dv = 128 only", fn);
  if (q_tok_stride < static_cast<int64_t>(Hk) * dk || k_tok_stride < static_cast<int64_t>(Hk) * dk ||
      v_tok_stride < static_cast<int64_t>(Hv) * dv || q_tok_stride % 8 || k_tok_stride % 8 ||
      v_tok_stride % 8)
    return fail(GDN_ERR_SHAPE, "%s: token strides too small or not multiples of 8", fn);
  if (projected && (gates.a_stride < Hv || gates.b_stride < Hv))
    return fail(GDN_ERR_SHAPE, "%s: a and b token strides must be at least Hv", fn);
  if (state_slot && n_slots < 0) return fail(GDN_ERR_SHAPE, "%s: n_slots < 0", fn);
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) ||
      !aligned(initial_state, 16) || !aligned(final_state, 16) || !aligned(gates.g, 4) ||
      !aligned(gates.beta, 4) || !aligned(gates.a, 2) || !aligned(gates.b, 2) ||
      !aligned(gates.A_log, 4) || !aligned(gates.dt_bias, 4) || !aligned(cu_seqlens, 4) ||
      !aligned(state_slot, 4))
    return fail(GDN_ERR_SHAPE,
                "%s: misaligned pointer (q, k, v, o, states: 16 bytes; a, b: 2; the rest: 4)", fn);
  if (!std::isfinite(scale)) return fail(GDN_ERR_SHAPE, "%s: scale must be finite", fn);
  if (!cu_seqlens) {
    const gdn_status s = check_equal_split(n_seqs, T_total);
    if (s) return s;
  } else if (n_seqs == 0 && T_total != 0) {
    return fail(GDN_ERR_SHAPE, "%s: T_total > 0 with no sequences", fn);
  }
  // grid size: ceil(n_seqs * Hk / 8) * 8 * (Hv / Hk) * 4 blocks
  if (static_cast<int64_t>(n_seqs) * Hv * 4 + 32LL * Hv > 0x7fffffffLL)
    return fail(GDN_ERR_SHAPE, "%s: too many (sequence, head) pairs", fn);
  const size_t ws_total = gdn::chunk_workspace_layout(n_seqs, T_total, Hk, Hv).total;
  const Range rq = range_of(q, T_total, q_tok_stride, static_cast<int64_t>(Hk) * dk, 2);
  const Range rk = range_of(k, T_total, k_tok_stride, static_cast<int64_t>(Hk) * dk, 2);
  const Range rv = range_of(v, T_total, v_tok_stride, static_cast<int64_t>(Hv) * dv, 2);
  const Range rg = range_of(gates.g, T_total, Hv, Hv, 4);
  const Range rb = range_of(gates.beta, T_total, Hv, Hv, 4);
  const Range ra = range_of(gates.a, T_total, gates.a_stride, Hv, 2);
  const Range rb2 = range_of(gates.b, T_total, gates.b_stride, Hv, 2);
  const Range rA = range_of(gates.A_log, 1, 0, Hv, 4);
  const Range rdt = range_of(gates.dt_bias, 1, 0, Hv, 4);
  const Range rsl = range_of(state_slot, n_seqs, 1, 1, 4);
  const Range ro = range_of(o, T_total, static_cast<int64_t>(Hv) * dv, static_cast<int64_t>(Hv) * dv, o_bf16 ? 2 : 4);
  const int64_t ssz = static_cast<int64_t>(Hv) * dv * dk;
  const int32_t n_states = state_slot ? n_slots : n_seqs;
  const Range r0 = range_of(initial_state, n_states, ssz, ssz, 4);
  const Range rT = range_of(final_state, n_states, ssz, ssz, 4);
  const Range rw = range_of(use_scratch ? nullptr : workspace, 1, 0, static_cast<int64_t>(ws_total), 1);
  for (const Range* in : {&rq, &rk, &rv, &rg, &rb, &ra, &rb2, &rA, &rdt, &rsl, &r0})
    if (overlap(*in, ro)) return fail(GDN_ERR_ALIAS, "%s: o overlaps an input", fn);
  for (const Range* in : {&rq, &rk, &rv, &rg, &rb, &ra, &rb2, &rA, &rdt, &rsl, &ro})
    if (overlap(*in, rT)) return fail(GDN_ERR_ALIAS, "%s: final_state overlaps o or an input", fn);
  if (overlap(r0, rT) && initial_state != final_state)
    return fail(GDN_ERR_ALIAS, "%s: final_state partially overlaps initial_state", fn);
  for (const Range* in : {&rq, &rk, &rv, &rg, &rb, &ra, &rb2, &rA, &rdt, &rsl, &ro, &r0, &rT})
    if (overlap(*in, rw)) return fail(GDN_ERR_ALIAS, "%s: workspace overlaps a tensor", fn);
  if (n_seqs > 0 && use_scratch) {
    if (ws_total > kScratchBytes)
      return fail(GDN_ERR_WORKSPACE,
                  "%s: needs %zu bytes of workspace, the static buffer holds %zu (use gdn_chunk_fwd "
                  "with a caller workspace)", fn, ws_total, kScratchBytes);
  } else if (n_seqs > 0) {
    if (!workspace || workspace_bytes < ws_total)
      return fail(GDN_ERR_WORKSPACE, "%s: workspace of %zu bytes needed", fn, ws_total);
    if (!aligned(workspace, 256))
      return fail(GDN_ERR_WORKSPACE, "%s: workspace must be 256-byte aligned", fn);
  }
  if (cu_seqlens && env_validate_seqlens()) {
    const gdn_status s = gdn_validate_cu_seqlens(cu_seqlens, n_seqs, T_total, stream);
    if (s) return s;
  }
  if (use_scratch && n_seqs > 0) {   // every argument is valid: only now touch the device
    const gdn_status s = scratch_address(&workspace);
    if (s) return s;
  }
  hipStream_t st = static_cast<hipStream_t>(stream);
  return hip_status(gdn::launch_chunk_fwd(q, q_tok_stride, k, k_tok_stride, v, v_tok_stride, gates,
                                          o, o_bf16, initial_state, final_state, state_slot,
                                          n_states, cu_seqlens, n_seqs, T_total, Hk, Hv, scale,
                                          workspace, st),
                    "prefill launch");
}

static gdn::GateInputs given_gates(const float* g, const float* beta) {
  gdn::GateInputs gi;
  gi.g = g;
  gi.beta = beta;
  return gi;
}

gdn_status gdn_chunk_fwd(const uint16_t* q, int64_t q_tok_stride, const uint16_t* k,
                         int64_t k_tok_stride, const uint16_t* v, int64_t v_tok_stride,
                         const float* g, const float* beta, float* o,
                         const float* initial_state, float* final_state,
                         const int32_t* cu_seqlens, int32_t n_seqs, int32_t T_total, int32_t Hk,
                         int32_t Hv, int32_t dk, int32_t dv, float scale, void* workspace,
                         size_t workspace_bytes, void* stream) {
  return chunk_fwd("gdn_chunk_fwd", q, q_tok_stride, k, k_tok_stride, v, v_tok_stride,
                   given_gates(g, beta), o, false, initial_state, final_state, nullptr, 0,
                   cu_seqlens, n_seqs, T_total, Hk, Hv, dk, dv, scale, workspace, workspace_bytes,
                   stream);
}

gdn_status gdn_chunk_fwd_noalloc(const uint16_t* q, int64_t q_tok_stride, const uint16_t* k,
                                 int64_t k_tok_stride, const uint16_t* v, int64_t v_tok_stride,
                                 const float* g, const float* beta, float* o,
                                 const float* initial_state, float* final_state,
                                 const int32_t* cu_seqlens, int32_t n_seqs, int32_t T_total,
                                 int32_t Hk, int32_t Hv, int32_t dk, int32_t dv, float scale,
                                 void* stream) {
  return chunk_fwd("gdn_chunk_fwd_noalloc", q, q_tok_stride, k, k_tok_stride, v, v_tok_stride,
                   given_gates(g, beta), o, false, initial_state, final_state, nullptr, 0,
                   cu_seqlens, n_seqs, T_total, Hk, Hv, dk, dv, scale, nullptr, 0, stream, true);
}

gdn_status gdn_chunk_fwd_bf16o(const uint16_t* q, int64_t q_tok_stride, const uint16_t* k,
                               int64_t k_tok_stride, const uint16_t* v, int64_t v_tok_stride,
                               const float* g, const float* beta, uint16_t* o,
                               const float* initial_state, float* final_state,
                               const int32_t* cu_seqlens, int32_t n_seqs, int32_t T_total,
                               int32_t Hk, int32_t Hv, int32_t dk, int32_t dv, float scale,
                               void* workspace, size_t workspace_bytes, void* stream) {
  return chunk_fwd("gdn_chunk_fwd_bf16o", q, q_tok_stride, k, k_tok_stride, v, v_tok_stride,
                   given_gates(g, beta), o, true, initial_state, final_state, nullptr, 0,
                   cu_seqlens, n_seqs, T_total, Hk, Hv, dk, dv, scale, workspace, workspace_bytes,
                   stream);
}

gdn_status gdn_chunk_fwd_pooled(const uint16_t* q, int64_t q_tok_stride, const uint16_t* k,
                                int64_t k_tok_stride, const uint16_t* v, int64_t v_tok_stride,
                                const float* g, const float* beta, void* o, int32_t o_is_bf16,
                                float* state, const int32_t* state_slot, int32_t n_slots,
                                const int32_t* cu_seqlens, int32_t n_seqs, int32_t T_total,
                                int32_t Hk, int32_t Hv, int32_t dk, int32_t dv, float scale,
                                void* workspace, size_t workspace_bytes, void* stream) {
  if (n_seqs > 0 && !state_slot)
    return fail(GDN_ERR_NULL, "gdn_chunk_fwd_pooled: state_slot is required");
  return chunk_fwd("gdn_chunk_fwd_pooled", q, q_tok_stride, k, k_tok_stride, v, v_tok_stride,
                   given_gates(g, beta), o, o_is_bf16 != 0, state, state,
                   n_seqs > 0 ? state_slot : nullptr, n_slots, cu_seqlens, n_seqs, T_total, Hk, Hv,
                   dk, dv, scale, workspace, workspace_bytes, stream);
}

gdn_status gdn_chunk_fwd_gated(const uint16_t* q, int64_t q_tok_stride, const uint16_t* k,
                               int64_t k_tok_stride, const uint16_t* v, int64_t v_tok_stride,
                               const uint16_t* a, int64_t a_tok_stride, const uint16_t* b,
                               int64_t b_tok_stride, const float* A_log, const float* dt_bias,
                               float* o, const float* initial_state, float* final_state,
                               const int32_t* cu_seqlens, int32_t n_seqs, int32_t T_total,
                               int32_t Hk, int32_t Hv, int32_t dk, int32_t dv, float scale,
                               void* workspace, size_t workspace_bytes, void* stream) {
  if (T_total > 0 && (!a || !b || !A_log || !dt_bias))
    return fail(GDN_ERR_NULL, "gdn_chunk_fwd_gated: a, b, A_log and dt_bias are required");
  gdn::GateInputs gi;
  gi.a = a; gi.a_stride = a_tok_stride; gi.b = b; gi.b_stride = b_tok_stride;
  gi.A_log = A_log; gi.dt_bias = dt_bias;
  return chunk_fwd("gdn_chunk_fwd_gated", q, q_tok_stride, k, k_tok_stride, v, v_tok_stride, gi,
                   o, false, initial_state, final_state, nullptr, 0, cu_seqlens, n_seqs, T_total,
                   Hk, Hv, dk, dv, scale, workspace, workspace_bytes, stream);
}

gdn_status gdn_decode_step(const uint16_t* q, int64_t q_stride, const uint16_t* k,
                           int64_t k_stride, const uint16_t* v, int64_t v_stride, const float* g,
                           const float* beta, float* state, const int32_t* state_slot,
                           int32_t n_slots, float* o, int32_t n_seqs, int32_t Hk, int32_t Hv,
                           int32_t dk, int32_t dv, float scale, void* stream) {
  if (n_seqs > 0 && (!q || !k || !v || !g || !beta || !state || !o))
    return fail(GDN_ERR_NULL, "gdn_decode_step: q, k, v, g, beta, state and o are required");
  if (n_seqs < 0 || n_slots < 0 || Hk <= 0 || Hv <= 0 || Hv % Hk)
    return fail(GDN_ERR_SHAPE, "gdn_decode_step: bad sizes or Hv %% Hk != 0");
  if (dk != 128 || dv != 128) return fail(GDN_ERR_UNSUPPORTED, "gdn_decode_step: dk = dv = 128 only");
  if (!state_slot && n_slots < n_seqs)
    return fail(GDN_ERR_SHAPE, "gdn_decode_step: n_slots < n_seqs without a slot map");
  if (q_stride < static_cast<int64_t>(Hk) * dk || k_stride < static_cast<int64_t>(Hk) * dk ||
      v_stride < static_cast<int64_t>(Hv) * dv || q_stride % 8 || k_stride % 8 || v_stride % 8)
    return fail(GDN_ERR_SHAPE, "gdn_decode_step: strides too small or not multiples of 8");
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(state, 16) ||
      !aligned(o, 4) || !aligned(g, 4) || !aligned(beta, 4) || !aligned(state_slot, 4))
    return fail(GDN_ERR_SHAPE, "gdn_decode_step: q, k, v and state must be 16-byte aligned");
  if (!std::isfinite(scale)) return fail(GDN_ERR_SHAPE, "gdn_decode_step: scale must be finite");
  if (static_cast<int64_t>(n_seqs) * Hv > 0x7fffffffLL)
    return fail(GDN_ERR_SHAPE, "gdn_decode_step: too many (sequence, head) pairs");
  const int64_t ssz = static_cast<int64_t>(Hv) * dv * dk;
  const Range rs = range_of(state, n_slots, ssz, ssz, 4);
  const Range ro = range_of(o, n_seqs, static_cast<int64_t>(Hv) * dv, static_cast<int64_t>(Hv) * dv, 4);
  const Range rq = range_of(q, n_seqs, q_stride, static_cast<int64_t>(Hk) * dk, 2);
  const Range rk = range_of(k, n_seqs, k_stride, static_cast<int64_t>(Hk) * dk, 2);
  const Range rv = range_of(v, n_seqs, v_stride, static_cast<int64_t>(Hv) * dv, 2);
  const Range rg = range_of(g, n_seqs, Hv, Hv, 4);
  const Range rb = range_of(beta, n_seqs, Hv, Hv, 4);
  const Range rsl = range_of(state_slot, n_seqs, 1, 1, 4);
  for (const Range* in : {&rq, &rk, &rv, &rg, &rb, &rsl, &rs})
    if (overlap(*in, ro)) return fail(GDN_ERR_ALIAS, "gdn_decode_step: o overlaps an input or the state");
  for (const Range* in : {&rq, &rk, &rv, &rg, &rb, &rsl})
    if (overlap(*in, rs)) return fail(GDN_ERR_ALIAS, "gdn_decode_step: state overlaps an input");
  return hip_status(gdn::launch_decode_step(q, q_stride, k, k_stride, v, v_stride, g, beta, state,
                                            state_slot, n_slots, o, n_seqs, Hk, Hv, scale,
                                            static_cast<hipStream_t>(stream)),
                    "gdn_decode_step launch");
}

gdn_status gdn_decode_tokens(const uint16_t* q, int64_t q_stride, const uint16_t* k,
                             int64_t k_stride, const uint16_t* v, int64_t v_stride,
                             const float* g, const float* beta, float* state,
                             const int32_t* state_slot, int32_t n_slots, float* o,
                             int32_t n_seqs, int32_t n_tokens, int32_t Hk, int32_t Hv,
                             int32_t dk, int32_t dv, float scale, void* stream) {
  if (n_seqs > 0 && (!q || !k || !v || !g || !beta || !state || !o))
    return fail(GDN_ERR_NULL, "gdn_decode_tokens: q, k, v, g, beta, state and o are required");
  if (n_seqs < 0 || n_slots < 0 || Hk <= 0 || Hv <= 0 || Hv % Hk)
    return fail(GDN_ERR_SHAPE, "gdn_decode_tokens: bad sizes or Hv %% Hk != 0");
  if (n_tokens < 1 || n_tokens > 8)
    return fail(GDN_ERR_UNSUPPORTED, "gdn_decode_tokens: n_tokens must be 1..8");
  if (dk != 128 || dv != 128) return fail(GDN_ERR_UNSUPPORTED, "gdn_decode_tokens: dk = dv = 128 only");
  if (!state_slot && n_slots < n_seqs)
    return fail(GDN_ERR_SHAPE, "gdn_decode_tokens: n_slots < n_seqs without a slot map");
  if (q_stride < static_cast<int64_t>(Hk) * dk || k_stride < static_cast<int64_t>(Hk) * dk ||
      v_stride < static_cast<int64_t>(Hv) * dv || q_stride % 8 || k_stride % 8 || v_stride % 8)
    return fail(GDN_ERR_SHAPE, "gdn_decode_tokens: strides too small or not multiples of 8");
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(state, 16) ||
      !aligned(o, 4) || !aligned(g, 4) || !aligned(beta, 4) || !aligned(state_slot, 4))
    return fail(GDN_ERR_SHAPE, "gdn_decode_tokens: q, k, v and state must be 16-byte aligned");
  if (!std::isfinite(scale)) return fail(GDN_ERR_SHAPE, "gdn_decode_tokens: scale must be finite");
  if (static_cast<int64_t>(n_seqs) * Hv > 0x7fffffffLL)
    return fail(GDN_ERR_SHAPE, "gdn_decode_tokens: too many (sequence, head) pairs");
  const int64_t rows = static_cast<int64_t>(n_seqs) * n_tokens;
  const int64_t ssz = static_cast<int64_t>(Hv) * dv * dk;
  const Range rs = range_of(state, n_slots, ssz, ssz, 4);
  const Range ro = range_of(o, rows, static_cast<int64_t>(Hv) * dv, static_cast<int64_t>(Hv) * dv, 4);
  const Range rq = range_of(q, rows, q_stride, static_cast<int64_t>(Hk) * dk, 2);
  const Range rk = range_of(k, rows, k_stride, static_cast<int64_t>(Hk) * dk, 2);
  const Range rv = range_of(v, rows, v_stride, static_cast<int64_t>(Hv) * dv, 2);
  const Range rg = range_of(g, rows, Hv, Hv, 4);
  const Range rb = range_of(beta, rows, Hv, Hv, 4);
  const Range rsl = range_of(state_slot, n_seqs, 1, 1, 4);
  for (const Range* in : {&rq, &rk, &rv, &rg, &rb, &rsl, &rs})
    if (overlap(*in, ro)) return fail(GDN_ERR_ALIAS, "gdn_decode_tokens: o overlaps an input or the state");
  for (const Range* in : {&rq, &rk, &rv, &rg, &rb, &rsl})
    if (overlap(*in, rs)) return fail(GDN_ERR_ALIAS, "gdn_decode_tokens: state overlaps an input");
  return hip_status(gdn::launch_decode_tokens(q, q_stride, k, k_stride, v, v_stride, g, beta, state,
                                              state_slot, n_slots, o, n_seqs, n_tokens, Hk, Hv, scale,
                                              static_cast<hipStream_t>(stream)),
                    "gdn_decode_tokens launch");
}

// The gate source of a whole-mixer call: g and beta, or the projections a, b
// with A_log and dt_bias (exactly one of the two sets).  Fills `gi` and the
// byte ranges the aliasing checks use.
static gdn_status mixer_gates(const char* fn, const float* g, const float* beta, const uint16_t* a,
                              int64_t a_stride, const uint16_t* b, int64_t b_stride,
                              const float* A_log, const float* dt_bias, int64_t rows, int32_t Hv,
                              gdn::GateInputs& gi, Range (&r)[6]) {
  const bool given = g || beta;
  const bool projected = a || b || A_log || dt_bias;
  if (rows > 0 && (given == projected || (given && !(g && beta)) ||
                   (projected && !(a && b && A_log && dt_bias))))
    return fail(GDN_ERR_NULL, "%s: pass either g and beta or a, b, A_log and dt_bias", fn);
  if (projected && (a_stride < Hv || b_stride < Hv))
    return fail(GDN_ERR_SHAPE, "%s: a and b token strides must be at least Hv", fn);
  if (!aligned(g, 4) || !aligned(beta, 4) || !aligned(a, 2) || !aligned(b, 2) || !aligned(A_log, 4) ||
      !aligned(dt_bias, 4))
    return fail(GDN_ERR_SHAPE, "%s: misaligned gate pointer", fn);
  gi.g = g; gi.beta = beta; gi.a = a; gi.a_stride = a_stride; gi.b = b; gi.b_stride = b_stride;
  gi.A_log = A_log; gi.dt_bias = dt_bias;
  r[0] = range_of(g, rows, Hv, Hv, 4);
  r[1] = range_of(beta, rows, Hv, Hv, 4);
  r[2] = range_of(a, rows, a_stride, Hv, 2);
  r[3] = range_of(b, rows, b_stride, Hv, 2);
  r[4] = range_of(A_log, 1, 0, Hv, 4);
  r[5] = range_of(dt_bias, 1, 0, Hv, 4);
  return GDN_OK;
}

gdn_status gdn_decode_mixer_step(const uint16_t* x, int64_t x_stride, const uint16_t* conv_w,
                                 const float* conv_bias, uint16_t* conv_state, const float* g,
                                 const float* beta, const uint16_t* a, int64_t a_stride,
                                 const uint16_t* b, int64_t b_stride, const float* A_log,
                                 const float* dt_bias, const uint16_t* z, int64_t z_stride,
                                 const float* norm_w, float* state, const int32_t* state_slot,
                                 int32_t n_slots, void* out, int32_t out_is_bf16, int32_t n_seqs,
                                 int32_t Hk, int32_t Hv, int32_t d, float scale, float l2_eps,
                                 float norm_eps, void* stream) {
  const char* fn = "gdn_decode_mixer_step";
  if (n_seqs > 0 && (!x || !conv_w || !conv_state || !z || !norm_w || !state || !out))
    return fail(GDN_ERR_NULL, "%s: x, conv_w, conv_state, z, norm_w, state and out are required", fn);
  if (n_seqs < 0 || n_slots < 0 || Hk <= 0 || Hv <= 0 || Hv % Hk)
    return fail(GDN_ERR_SHAPE, "%s: bad sizes or Hv %% Hk != 0", fn);
  gdn::GateInputs gi;
  Range rgates[6];
  {
    const gdn_status st = mixer_gates(fn, g, beta, a, a_stride, b, b_stride, A_log, dt_bias, n_seqs, Hv,
                                      gi, rgates);
    if (st) return st;
  }
  if (d != 128) return fail(GDN_ERR_UNSUPPORTED, "%s: d = 128 only", fn);
  if (Hv / Hk > 4) return fail(GDN_ERR_UNSUPPORTED, "%s: Hv / Hk must be at most 4", fn);
  if (!state_slot && n_slots < n_seqs)
    return fail(GDN_ERR_SHAPE, "%s: n_slots < n_seqs without a slot map", fn);
  const int64_t C = static_cast<int64_t>(2 * Hk + Hv) * d;
  if (x_stride < C || z_stride < static_cast<int64_t>(Hv) * d)
    return fail(GDN_ERR_SHAPE, "%s: row strides too small", fn);
  if (!aligned(state, 16) || !aligned(x, 2) || !aligned(conv_w, 2) || !aligned(conv_state, 2) ||
      !aligned(z, 2) || !aligned(norm_w, 4) || !aligned(conv_bias, 4) || !aligned(state_slot, 4) ||
      !aligned(out, out_is_bf16 ? 2 : 4))
    return fail(GDN_ERR_SHAPE, "%s: misaligned pointer (state needs 16 bytes)", fn);
  if (!std::isfinite(scale) || !(l2_eps >= 0.f) || !std::isfinite(l2_eps) || !(norm_eps >= 0.f) ||
      !std::isfinite(norm_eps))
    return fail(GDN_ERR_SHAPE, "%s: scale and eps must be finite, eps >= 0", fn);
  if (static_cast<int64_t>(n_seqs) * Hk > 0x7fffffffLL)
    return fail(GDN_ERR_SHAPE, "%s: too many (sequence, head) pairs", fn);
  const int64_t ssz = static_cast<int64_t>(Hv) * d * d;
  const Range rs = range_of(state, n_slots, ssz, ssz, 4);
  const Range rc = range_of(conv_state, n_slots, C * 3, C * 3, 2);
  const Range rx = range_of(x, n_seqs, x_stride, C, 2);
  const Range rw = range_of(conv_w, 1, 0, C * 4, 2);
  const Range rbias = range_of(conv_bias, 1, 0, C, 4);
  const Range rz = range_of(z, n_seqs, z_stride, static_cast<int64_t>(Hv) * d, 2);
  const Range rn = range_of(norm_w, 1, 0, d, 4);
  const Range rsl = range_of(state_slot, n_seqs, 1, 1, 4);
  const Range ro = range_of(out, n_seqs, static_cast<int64_t>(Hv) * d, static_cast<int64_t>(Hv) * d,
                            out_is_bf16 ? 2 : 4);
  const Range* inputs[] = {&rx, &rw, &rbias, &rz, &rn, &rsl, &rgates[0], &rgates[1], &rgates[2],
                           &rgates[3], &rgates[4], &rgates[5]};
  for (const Range* in : inputs)
    if (overlap(*in, ro) || overlap(*in, rs) || overlap(*in, rc))
      return fail(GDN_ERR_ALIAS, "%s: out, state or conv_state overlaps an input", fn);
  if (overlap(ro, rs) || overlap(ro, rc) || overlap(rs, rc))
    return fail(GDN_ERR_ALIAS, "%s: out, state and conv_state overlap", fn);
  return hip_status(gdn::launch_decode_mixer(x, x_stride, conv_w, conv_bias, conv_state, gi, z,
                                             z_stride, norm_w, state, state_slot, n_slots, out,
                                             out_is_bf16 != 0,
                                             n_seqs, Hk, Hv, scale, l2_eps, norm_eps,
                                             static_cast<hipStream_t>(stream)),
                    "gdn_decode_mixer_step launch");
}

static size_t mixer_o_bytes(int32_t T_total, int32_t Hv, int32_t out_is_bf16) {
  return out_is_bf16 ? ((static_cast<size_t>(T_total) * Hv * 128 * 4 + 255) & ~static_cast<size_t>(255)) : 0;
}

size_t gdn_mixer_fwd_workspace_bytes(int32_t n_seqs, int32_t T_total, int32_t Hk, int32_t Hv,
                                     int32_t d, int32_t out_is_bf16) {
  (void)d;
  if (n_seqs < 0 || T_total < 0 || Hk <= 0 || Hv <= 0) return 0;
  return gdn::chunk_workspace_layout(n_seqs, T_total, Hk, Hv).total +
         mixer_o_bytes(T_total, Hv, out_is_bf16);
}

gdn_status gdn_mixer_fwd(const uint16_t* x, int64_t x_stride, const uint16_t* conv_w,
                         const float* conv_bias, uint16_t* conv_state, const float* g,
                         const float* beta, const uint16_t* a, int64_t a_stride, const uint16_t* b,
                         int64_t b_stride, const float* A_log, const float* dt_bias,
                         const uint16_t* z, int64_t z_stride,
                         const float* norm_w, void* out, int32_t out_is_bf16,
                         const float* initial_state, float* final_state,
                         const int32_t* state_slot, int32_t n_slots,
                         const int32_t* cu_seqlens, int32_t n_seqs, int32_t T_total, int32_t Hk,
                         int32_t Hv, int32_t d, float scale, float l2_eps, float norm_eps,
                         void* workspace, size_t workspace_bytes, void* stream) {
  const char* fn = "gdn_mixer_fwd";
  if (state_slot && n_seqs > 0 && (!initial_state || initial_state != final_state))
    return fail(GDN_ERR_SHAPE, "%s: with a slot map, initial_state and final_state must be the same pool", fn);
  if (state_slot && n_slots < 0) return fail(GDN_ERR_SHAPE, "%s: n_slots < 0", fn);
  const int32_t n_rows = state_slot ? n_slots : n_seqs;   // rows of the state and conv-state buffers
  if (T_total > 0 && (!x || !conv_w || !z || !norm_w || !out))
    return fail(GDN_ERR_NULL, "%s: x, conv_w, z, norm_w and out are required", fn);
  if (n_seqs < 0 || T_total < 0 || Hk <= 0 || Hv <= 0 || Hv % Hk)
    return fail(GDN_ERR_SHAPE, "%s: bad sizes or Hv %% Hk != 0", fn);
  gdn::GateInputs gi;
  Range rgates[6];
  {
    const gdn_status st = mixer_gates(fn, g, beta, a, a_stride, b, b_stride, A_log, dt_bias, T_total,
                                      Hv, gi, rgates);
    if (st) return st;
  }
  if (d != 128) return fail(GDN_ERR_UNSUPPORTED, "%s: d = 128 only", fn);
  const int64_t C = static_cast<int64_t>(2 * Hk + Hv) * d;
  const int64_t width = static_cast<int64_t>(Hv) * d;
  if (x_stride < C || x_stride % 8 || z_stride < width || z_stride % 8)
    return fail(GDN_ERR_SHAPE, "%s: x and z row strides too small or not multiples of 8", fn);
  if (!aligned(x, 16) || !aligned(conv_w, 16) || !aligned(conv_bias, 16) ||
      !aligned(conv_state, 16) || !aligned(z, 16) || !aligned(norm_w, 16) || !aligned(out, 16) ||
      !aligned(initial_state, 16) || !aligned(final_state, 16) || !aligned(cu_seqlens, 4) ||
      !aligned(state_slot, 4))
    return fail(GDN_ERR_SHAPE, "%s: misaligned pointer (16 bytes; cu_seqlens: 4)", fn);
  if (!std::isfinite(scale) || !(l2_eps >= 0.f) || !std::isfinite(l2_eps) || !(norm_eps >= 0.f) ||
      !std::isfinite(norm_eps))
    return fail(GDN_ERR_SHAPE, "%s: scale and eps must be finite, eps >= 0", fn);
  if (!cu_seqlens) {
    const gdn_status st = check_equal_split(n_seqs, T_total);
    if (st) return st;
  } else if (n_seqs == 0 && T_total != 0) {
    return fail(GDN_ERR_SHAPE, "%s: T_total > 0 with no sequences", fn);
  }
  if (static_cast<int64_t>(n_seqs) * Hv * 2 + 16LL * Hv > 0x7fffffffLL)
    return fail(GDN_ERR_SHAPE, "%s: too many (sequence, head) pairs", fn);
  const gdn::ChunkWorkspace ws = gdn::chunk_workspace_layout(n_seqs, T_total, Hk, Hv);
  const size_t need = ws.total + mixer_o_bytes(T_total, Hv, out_is_bf16);
  const int64_t ssz = width * d;
  const Range rx = range_of(x, T_total, x_stride, C, 2);
  const Range rw = range_of(conv_w, 1, 0, C * 4, 2);
  const Range rbias = range_of(conv_bias, 1, 0, C, 4);
  const Range rcs = range_of(conv_state, n_rows, 3 * C, 3 * C, 2);
  const Range rsl = range_of(state_slot, n_seqs, 1, 1, 4);
  const Range& rg = rgates[0];
  const Range& rb = rgates[1];
  const Range rz = range_of(z, T_total, z_stride, width, 2);
  const Range rn = range_of(norm_w, 1, 0, d, 4);
  const Range rcu = range_of(cu_seqlens, 1, 0, static_cast<int64_t>(n_seqs) + 1, 4);
  const Range ro = range_of(out, T_total, width, width, out_is_bf16 ? 2 : 4);
  const Range r0 = range_of(initial_state, n_rows, ssz, ssz, 4);
  const Range rT = range_of(final_state, n_rows, ssz, ssz, 4);
  const Range rws = range_of(workspace, 1, 0, static_cast<int64_t>(need), 1);
  for (const Range* in : {&rsl})
    if (overlap(*in, rcs) || overlap(*in, rT) || overlap(*in, rws))
      return fail(GDN_ERR_ALIAS, "%s: state_slot overlaps a state or the workspace", fn);
  for (const Range* in : {&rx, &rw, &rbias, &rcs, &rg, &rb, &rz, &rn, &rcu, &r0, &rT, &rws})
    if (overlap(*in, ro)) return fail(GDN_ERR_ALIAS, "%s: out overlaps another buffer", fn);
  for (int i = 2; i < 6; ++i)
    if (overlap(rgates[i], ro) || overlap(rgates[i], rcs) || overlap(rgates[i], rT) ||
        overlap(rgates[i], rws))
      return fail(GDN_ERR_ALIAS, "%s: a gate input overlaps an output or the workspace", fn);
  for (const Range* in : {&rx, &rw, &rbias, &rg, &rb, &rz, &rn, &rcu, &r0, &rT, &rws})
    if (overlap(*in, rcs)) return fail(GDN_ERR_ALIAS, "%s: conv_state overlaps another buffer", fn);
  for (const Range* in : {&rx, &rw, &rbias, &rg, &rb, &rz, &rn, &rcu, &rws})
    if (overlap(*in, rT)) return fail(GDN_ERR_ALIAS, "%s: final_state overlaps an input or the workspace", fn);
  if (overlap(r0, rT) && initial_state != final_state)
    return fail(GDN_ERR_ALIAS, "%s: final_state partially overlaps initial_state", fn);
  for (const Range* in : {&rx, &rw, &rbias, &rg, &rb, &rz, &rn, &rcu, &r0})
    if (overlap(*in, rws)) return fail(GDN_ERR_ALIAS, "%s: workspace overlaps a tensor", fn);
  if (n_seqs > 0) {
    if (!workspace || workspace_bytes < need)
      return fail(GDN_ERR_WORKSPACE, "%s: workspace of %zu bytes needed", fn, need);
    if (!aligned(workspace, 256))
      return fail(GDN_ERR_WORKSPACE, "%s: workspace must be 256-byte aligned", fn);
  }
  if (cu_seqlens && env_validate_seqlens()) {
    const gdn_status st = gdn_validate_cu_seqlens(cu_seqlens, n_seqs, T_total, stream);
    if (st) return st;
  }
  if (n_seqs == 0) return GDN_OK;
  hipStream_t st = static_cast<hipStream_t>(stream);
  // o: fp32 in out itself (normalised in place), or in the workspace for bf16 out
  float* o = out_is_bf16 ? reinterpret_cast<float*>(static_cast<unsigned char*>(workspace) + ws.total)
                         : static_cast<float*>(out);
  gdn::ConvFront cf;
  cf.x = x; cf.xs = x_stride; cf.w = conv_w; cf.bias = conv_bias; cf.state = conv_state;
  cf.slots = state_slot;
  cf.n_slots = n_rows;
  cf.l2_eps = l2_eps;
  gdn_status s = hip_status(gdn::launch_chunk_fwd(nullptr, 0, nullptr, 0, nullptr, 0,
                                                  gi, o, false, initial_state,
                                                  final_state, state_slot, n_rows, cu_seqlens,
                                                  n_seqs, T_total, Hk, Hv, scale, workspace, st,
                                                  &cf),
                            "gdn_mixer_fwd prefill launch");
  if (s) return s;
  s = hip_status(gdn::launch_conv_state(x, x_stride, conv_state, cu_seqlens, n_seqs, T_total,
                                        static_cast<int>(C), st, state_slot, n_rows),
                 "gdn_mixer_fwd conv state launch");
  if (s) return s;
  return hip_status(gdn::launch_gated_rmsnorm(o, z, z_stride, norm_w, out, out_is_bf16 != 0, T_total,
                                              Hv, norm_eps, st),
                    "gdn_mixer_fwd norm launch");
}

gdn_status gdn_gated_rmsnorm(const float* o, const uint16_t* z, int64_t z_row_stride,
                             const float* w, void* out, int32_t out_is_bf16, int64_t rows,
                             int32_t Hv, int32_t dv, float eps, void* stream) {
  if (rows > 0 && (!o || !z || !w || !out))
    return fail(GDN_ERR_NULL, "gdn_gated_rmsnorm: all pointers are required");
  if (rows < 0 || Hv <= 0) return fail(GDN_ERR_SHAPE, "gdn_gated_rmsnorm: bad sizes");
  if (dv != 128) return fail(GDN_ERR_UNSUPPORTED, "gdn_gated_rmsnorm: dv must be 128");
  if (z_row_stride < static_cast<int64_t>(Hv) * dv || z_row_stride % 8)
    return fail(GDN_ERR_SHAPE, "gdn_gated_rmsnorm: z row stride too small or not a multiple of 8");
  if (!aligned(o, 16) || !aligned(z, 16) || !aligned(w, 16) || !aligned(out, 16))
    return fail(GDN_ERR_SHAPE, "gdn_gated_rmsnorm: pointers must be 16-byte aligned");
  if (!(eps >= 0.f) || !std::isfinite(eps))
    return fail(GDN_ERR_SHAPE, "gdn_gated_rmsnorm: eps must be finite and >= 0");
  const int64_t width = static_cast<int64_t>(Hv) * dv;
  const Range ro = range_of(o, rows, width, width, 4);
  const Range rz = range_of(z, rows, z_row_stride, width, 2);
  const Range rw = range_of(w, 1, dv, dv, 4);
  const Range rout = range_of(out, rows, width, width, out_is_bf16 ? 2 : 4);
  if (overlap(rout, rz) || overlap(rout, rw))
    return fail(GDN_ERR_ALIAS, "gdn_gated_rmsnorm: out overlaps z or w");
  if (overlap(rout, ro) && !(static_cast<const void*>(o) == out && !out_is_bf16))
    return fail(GDN_ERR_ALIAS, "gdn_gated_rmsnorm: out may alias o only exactly and in fp32");
  return hip_status(gdn::launch_gated_rmsnorm(o, z, z_row_stride, w, out, out_is_bf16 != 0, rows,
                                              Hv, eps, static_cast<hipStream_t>(stream)),
                    "gdn_gated_rmsnorm launch");
}

double gdn_calib_mfma_loop_flops(int32_t n_iter, int32_t n_blocks) {
  if (n_iter <= 0 || n_blocks <= 0) return 0.0;
  return gdn::mfma_loop_flops(n_iter, n_blocks);
}

gdn_status gdn_calib_mfma_loop(int32_t n_iter, int32_t n_blocks, float* out, void* stream) {
  if (!out) return fail(GDN_ERR_NULL, "gdn_calib_mfma_loop: out is NULL");
  if (n_iter <= 0 || n_blocks <= 0 || n_blocks > (1 << 20))
    return fail(GDN_ERR_SHAPE, "gdn_calib_mfma_loop: n_iter %d and n_blocks %d must be in 1 .. "
                "and n_blocks <= 2^20", n_iter, n_blocks);
  if (!aligned(out, 4)) return fail(GDN_ERR_SHAPE, "gdn_calib_mfma_loop: out misaligned");
  return hip_status(gdn::launch_mfma_loop(n_iter, n_blocks, out, static_cast<hipStream_t>(stream)),
                    "gdn_calib_mfma_loop launch");
}

gdn_status gdn_calib_stream_inplace(void* buf, int64_t bytes, int32_t n_blocks, void* stream) {
  if (!buf) return fail(GDN_ERR_NULL, "gdn_calib_stream_inplace: buf is NULL");
  if (bytes <= 0 || bytes % 16 || n_blocks <= 0 || n_blocks > (1 << 20))
    return fail(GDN_ERR_SHAPE, "gdn_calib_stream_inplace: bytes %lld (a positive multiple of 16) "
                "and n_blocks %d (1 .. 2^20)", static_cast<long long>(bytes), n_blocks);
  if (!aligned(buf, 16)) return fail(GDN_ERR_SHAPE, "gdn_calib_stream_inplace: buf misaligned");
  return hip_status(gdn::launch_stream_inplace(buf, bytes, n_blocks, static_cast<hipStream_t>(stream)),
                    "gdn_calib_stream_inplace launch");
}

size_t gdn_backward_workspace_bytes(int32_t n_seqs, int32_t T_total, int32_t Hv) {
  if (n_seqs <= 0 || T_total <= 0 || Hv <= 0) return 0;
  return gdn::chunked_backward_workspace_bytes(n_seqs, T_total, Hv);
}

gdn_status gdn_backward(const uint16_t* q, int64_t q_tok_stride, const uint16_t* k,
                        int64_t k_tok_stride, const uint16_t* v, int64_t v_tok_stride,
                        const float* g, const float* beta, const float* initial_state,
                        const float* grad_o, const float* grad_final_state,
                        const int32_t* cu_seqlens, int32_t n_seqs, int32_t T_total, int32_t Hk,
                        int32_t Hv, int32_t dk, int32_t dv, float scale, float* grad_q,
                        float* grad_k, float* grad_v, float* grad_g, float* grad_beta,
                        float* grad_initial_state, void* workspace, size_t workspace_bytes,
                        void* stream) {
  const char* fn = "gdn_backward";
  if (T_total > 0 && (!q || !k || !v || !g || !beta || !grad_o || !grad_q || !grad_k || !grad_v ||
                      !grad_g || !grad_beta))
    return fail(GDN_ERR_NULL, "%s: q, k, v, g, beta, grad_o and the token gradients are required", fn);
  if (n_seqs < 0 || T_total < 0 || Hk <= 0 || Hv <= 0 || Hv % Hk)
    return fail(GDN_ERR_SHAPE, "%s: bad sizes or Hv %% Hk != 0", fn);
  if (dk != 128 || dv != 128) return fail(GDN_ERR_UNSUPPORTED, "%s: dk = dv = 128 only", fn);
  if (q_tok_stride < static_cast<int64_t>(Hk) * dk || k_tok_stride < static_cast<int64_t>(Hk) * dk ||
      v_tok_stride < static_cast<int64_t>(Hv) * dv || q_tok_stride % 8 || k_tok_stride % 8 ||
      v_tok_stride % 8)
    return fail(GDN_ERR_SHAPE, "%s: token strides too small or not multiples of 8", fn);
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(initial_state, 16) ||
      !aligned(grad_final_state, 16) || !aligned(grad_initial_state, 16) || !aligned(grad_o, 4) ||
      !aligned(grad_q, 4) || !aligned(grad_k, 4) || !aligned(grad_v, 4) || !aligned(g, 4) ||
      !aligned(beta, 4) || !aligned(grad_g, 4) || !aligned(grad_beta, 4) || !aligned(cu_seqlens, 4))
    return fail(GDN_ERR_SHAPE, "%s: misaligned pointer (q, k, v, states: 16 bytes; the rest: 4)", fn);
  if (!std::isfinite(scale)) return fail(GDN_ERR_SHAPE, "%s: scale must be finite", fn);
  if (!cu_seqlens) {
    const gdn_status s = check_equal_split(n_seqs, T_total);
    if (s) return s;
  } else if (n_seqs == 0 && T_total != 0) {
    return fail(GDN_ERR_SHAPE, "%s: T_total > 0 with no sequences", fn);
  }
  if (static_cast<int64_t>(n_seqs) * Hv > 0x7fffffffLL)
    return fail(GDN_ERR_SHAPE, "%s: too many (sequence, head) pairs", fn);
  const size_t need = gdn_backward_workspace_bytes(n_seqs, T_total, Hv);
  const int64_t wk = static_cast<int64_t>(Hk) * dk, wv = static_cast<int64_t>(Hv) * dv;
  const int64_t ssz = static_cast<int64_t>(Hv) * dv * dk;
  const Range in_ranges[] = {
      range_of(q, T_total, q_tok_stride, wk, 2), range_of(k, T_total, k_tok_stride, wk, 2),
      range_of(v, T_total, v_tok_stride, wv, 2), range_of(g, T_total, Hv, Hv, 4),
      range_of(beta, T_total, Hv, Hv, 4),        range_of(initial_state, n_seqs, ssz, ssz, 4),
      range_of(grad_o, T_total, wv, wv, 4),      range_of(grad_final_state, n_seqs, ssz, ssz, 4),
      range_of(cu_seqlens, 1, 0, static_cast<int64_t>(n_seqs) + 1, 4)};
  const Range out_ranges[] = {
      range_of(grad_q, T_total, wk, wk, 4),   range_of(grad_k, T_total, wk, wk, 4),
      range_of(grad_v, T_total, wv, wv, 4),   range_of(grad_g, T_total, Hv, Hv, 4),
      range_of(grad_beta, T_total, Hv, Hv, 4), range_of(grad_initial_state, n_seqs, ssz, ssz, 4),
      range_of(workspace, 1, 0, static_cast<int64_t>(need), 1)};
  const int n_out = sizeof(out_ranges) / sizeof(out_ranges[0]);
  for (int i = 0; i < n_out; ++i) {
    for (const Range& r : in_ranges)
      if (overlap(out_ranges[i], r)) return fail(GDN_ERR_ALIAS, "%s: an output or the workspace overlaps an input", fn);
    for (int j = i + 1; j < n_out; ++j)
      if (overlap(out_ranges[i], out_ranges[j]))
        return fail(GDN_ERR_ALIAS, "%s: outputs (or the workspace) overlap each other", fn);
  }
  if (T_total > 0 || (n_seqs > 0 && grad_initial_state)) {
    if (need > 0 && (!workspace || workspace_bytes < need))
      return fail(GDN_ERR_WORKSPACE, "%s: workspace of %zu bytes needed", fn, need);
    if (!aligned(workspace, 256))
      return fail(GDN_ERR_WORKSPACE, "%s: workspace must be 256-byte aligned", fn);
  }
  if (cu_seqlens && env_validate_seqlens()) {
    const gdn_status s = gdn_validate_cu_seqlens(cu_seqlens, n_seqs, T_total, stream);
    if (s) return s;
  }
  return hip_status(gdn::launch_backward_chunked(q, q_tok_stride, k, k_tok_stride, v, v_tok_stride, g, beta,
                                         initial_state, grad_o, grad_final_state, cu_seqlens,
                                         n_seqs, T_total, Hk, Hv, scale, grad_q, grad_k, grad_v,
                                         grad_g, grad_beta, grad_initial_state, workspace,
                                         static_cast<hipStream_t>(stream)),
                    "gdn_backward launch");
}

}  // extern "C"
