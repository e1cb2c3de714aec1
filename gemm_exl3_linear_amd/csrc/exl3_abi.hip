// C ABI of the EXL3 library (declared in include/exl3.h): host-side
// validation, fail-closed on anything unsupported, then dispatch to the
// kernels.  Nothing is enqueued when validation fails, and nothing is
// allocated: the caller provides every buffer, including the workspace.
#include <stdio.h>
#include <stdlib.h>

#include <atomic>
#include <mutex>

#include "exl3.h"
#include "exl3_gemv.hpp"
#include "exl3_internal.hpp"

namespace {

constexpr int kGemvMaxRows = 16;  // rows up to this use the decode GEMV
constexpr int64_t kMaxRows = (int64_t)1 << 24;  // activation rows of one call
// Workgroups of one launch: a grid of 256-thread workgroups must stay below
// 2^32 threads.
constexpr int64_t kMaxWorkgroups = ((int64_t)1 << 24) - 1;
// Bytes of one tensor's trellis: the kernels address it with 32-bit offsets.
constexpr int64_t kMaxTrellisBytes = (int64_t)1 << 32;

int64_t trellis_bytes(int64_t k, int64_t n, int64_t bits) { return k * n / 8 * bits; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

bool trace_on() {
  static const int on = [] {
    const char* v = getenv("EXL3_TRACE");
    return (v && v[0] && v[0] != '0') ? 1 : 0;
  }();
  return on != 0;
}

void trace(const char* what, long long a, long long b, long long c, long long d) {
  if (trace_on()) fprintf(stderr, "[exl3] %s %lld %lld %lld %lld\n", what, a, b, c, d);
}

exl3_status from_hip(hipError_t e) { return e == hipSuccess ? EXL3_OK : EXL3_E_HIP; }

// EXL3_CHECK_IDS set and not "0": the grouped calls check their routing ids
// on the device first (read at every call, so it can be switched at run time).
bool check_ids_on() {
  const char* v = getenv("EXL3_CHECK_IDS");
  return v && v[0] && v[0] != '0';
}

// EXL3_FORCE_DEVICE_SCOPE set and not "0" (debug): every workgroup of the
// grouped token-parallel path takes the device-scope hand-off that a
// workgroup dispatched to another XCD than planned takes (read at every call).
bool force_device_scope_on() {
  const char* v = getenv("EXL3_FORCE_DEVICE_SCOPE");
  return v && v[0] && v[0] != '0';
}

// Common checks of a tensor record; `mult` is the required multiple of k, n.
exl3_status check_weight(const exl3_weight* w, int mult, bool need_signs) {
  if (!w) return EXL3_E_INVALID;
  if (w->bits < 1 || w->bits > 8) return EXL3_E_INVALID;
  if (w->codebook != EXL3_CODEBOOK_MUL1) return EXL3_E_UNSUPPORTED;
  if (w->k <= 0 || w->n <= 0 || w->k % mult || w->n % mult) return EXL3_E_INVALID;
  // tile counts index the kernels' 32-bit work plans
  if ((int64_t)(w->k / 16) * (w->n / 16) >= ((int64_t)1 << 31)) return EXL3_E_INVALID;
  if (!w->trellis || !aligned16(w->trellis)) return EXL3_E_INVALID;
  if (need_signs) {
    if (!w->suh || !w->svh || !aligned16(w->suh) || !aligned16(w->svh)) return EXL3_E_INVALID;
    if (w->bias && !aligned16(w->bias)) return EXL3_E_INVALID;
  }
  return EXL3_OK;
}

exl3_status check_arena(const exl3_expert_weights* a, int slots) {
  if (!a) return EXL3_E_INVALID;
  if (a->bits < 1 || a->bits > 8) return EXL3_E_INVALID;
  if (a->codebook != EXL3_CODEBOOK_MUL1) return EXL3_E_UNSUPPORTED;
  if (a->slots != slots || a->experts <= 0) return EXL3_E_INVALID;
  if (a->k <= 0 || a->n <= 0 || a->k % 128 || a->n % 128) return EXL3_E_INVALID;
  // one (expert, slot) tensor: tile counts index 32-bit work plans, and the
  // grouped GEMM addresses its trellis through a 32-bit buffer descriptor
  if ((int64_t)(a->k / 16) * (a->n / 16) >= ((int64_t)1 << 31)) return EXL3_E_INVALID;
  if (trellis_bytes(a->k, a->n, a->bits) >= kMaxTrellisBytes) return EXL3_E_INVALID;
  if (!a->trellis || !a->suh || !a->svh) return EXL3_E_INVALID;
  if (!aligned16(a->trellis) || !aligned16(a->suh) || !aligned16(a->svh)) return EXL3_E_INVALID;
  return EXL3_OK;
}

size_t linear_ws(const exl3_weight* w, int64_t m) {
  if (m <= kGemvMaxRows) return exl3::plan_gemv(w->k, w->n, (int)m).ws;
  return exl3::gemm_workspace(w->k, w->n, (int)m);
}

// Common checks of a multi-tensor call: 1..EXL3_MAX_MULTI valid records that
// share k.
exl3_status check_multi(const exl3_weight* const* w, int32_t count) {
  if (!w || count < 1 || count > EXL3_MAX_MULTI) return EXL3_E_INVALID;
  for (int i = 0; i < count; ++i) {
    const exl3_status st = check_weight(w[i], 128, true);
    if (st != EXL3_OK) return st;
    if (w[i]->k != w[0]->k) return EXL3_E_INVALID;
    if (trellis_bytes(w[i]->k, w[i]->n, w[i]->bits) >= kMaxTrellisBytes) return EXL3_E_INVALID;
  }
  return EXL3_OK;
}

size_t multi_ws(const exl3_weight* const* w, int32_t count, int64_t m) {
  if (m == 1) {
    exl3::MultiTensor t[EXL3_MAX_MULTI];
    for (int i = 0; i < count; ++i) t[i] = {w[i]->trellis, w[i]->suh, w[i]->svh, w[i]->bias, w[i]->n, w[i]->bits};
    return exl3::plan_gemv_multi(t, count, w[0]->k).ws;
  }
  size_t need = 0;
  for (int i = 0; i < count; ++i) {
    const size_t s = linear_ws(w[i], m);
    if (s > need) need = s;
  }
  return need;
}

// An arena whose experts each have their own width: the record's bits is 0
// and the widths record supplies them, checked on the host from bits_host;
// the rest is checked as for a uniform arena.
exl3_status check_mixed_arena(const exl3_expert_weights* a, const exl3_expert_widths* w, int slots) {
  if (!a || !w) return EXL3_E_INVALID;
  if (a->bits != 0) return EXL3_E_INVALID;
  exl3_expert_weights u = *a;
  u.bits = 8;  // the size limits for the widest width an expert may have
  const exl3_status st = check_arena(&u, slots);
  if (st != EXL3_OK) return st;
  if (!w->bits_host || !w->bits || !w->offsets) return EXL3_E_INVALID;
  if (!aligned4(w->bits) || (reinterpret_cast<uintptr_t>(w->offsets) & 7u)) return EXL3_E_INVALID;
  for (int e = 0; e < a->experts; ++e) {
    const int32_t b = w->bits_host[e];
    if (b < 1 || b > 8) return EXL3_E_INVALID;
  }
  return EXL3_OK;
}

exl3::ArenaDesc desc(const exl3_expert_weights* a) {
  return exl3::ArenaDesc{a->trellis, a->suh, a->svh, a->experts, a->slots, a->k, a->n, a->bits};
}

exl3::ArenaDesc desc_mixed(const exl3_expert_weights* a, const exl3_expert_widths* w) {
  exl3::ArenaDesc d{a->trellis, a->suh, a->svh, a->experts, a->slots, a->k, a->n, 0};
  d.ebits = w->bits;
  d.eoff = w->offsets;
  return d;
}

// Checks shared by both grouped entry points, after the arenas' own: the
// arenas fit together and the routing sizes are in range.
exl3_status check_grouped_pair(const exl3_expert_weights* gu, const exl3_expert_weights* dn,
                               int64_t t, int32_t topk) {
  if (dn->experts != gu->experts || dn->k != gu->n || dn->n != gu->k) return EXL3_E_INVALID;
  if (t < 0 || topk < 1 || topk > EXL3_MAX_TOPK) return EXL3_E_INVALID;
  // bounds the pair indices, the tile list and the grouped GEMM's grid
  // (tiles x slots x column blocks) well inside 32-bit ranges
  if (t * topk > (int64_t)1 << 21) return EXL3_E_INVALID;
  return EXL3_OK;
}

exl3_status check_grouped(const exl3_expert_weights* gu, const exl3_expert_weights* dn, int64_t t,
                          int32_t topk) {
  exl3_status st = check_arena(gu, 2);
  if (st != EXL3_OK) return st;
  if ((st = check_arena(dn, 1)) != EXL3_OK) return st;
  return check_grouped_pair(gu, dn, t, topk);
}

exl3_status check_grouped_mixed(const exl3_expert_weights* gu, const exl3_expert_widths* guw,
                                const exl3_expert_weights* dn, const exl3_expert_widths* dnw,
                                int64_t t, int32_t topk) {
  exl3_status st = check_mixed_arena(gu, guw, 2);
  if (st != EXL3_OK) return st;
  if ((st = check_mixed_arena(dn, dnw, 1)) != EXL3_OK) return st;
  return check_grouped_pair(gu, dn, t, topk);
}

// The common part of both grouped entry points, once the arenas are checked.
exl3_status run_grouped(const exl3::ArenaDesc& gu, const exl3::ArenaDesc& dn, const void* x,
                        const int32_t* topk_ids, const float* topk_weights, int64_t t,
                        int32_t topk, float* y, void* ws, size_t ws_bytes, exl3_stream_t stream) {
  if (t == 0) return EXL3_OK;
  if (!x || !topk_ids || !topk_weights || !y) return EXL3_E_INVALID;
  if (!aligned16(x) || !aligned16(y) || !aligned4(topk_ids) || !aligned4(topk_weights))
    return EXL3_E_INVALID;
  const size_t need = exl3::grouped_workspace(gu, dn, t, topk);
  if (!ws || ws_bytes < need || !aligned16(ws)) return EXL3_E_WORKSPACE;
  trace("grouped t topk experts bits", t, topk, gu.experts, gu.bits);
  if (check_ids_on()) {
    // The check waits on the host for a device count, which a stream being
    // captured into a graph cannot do: refuse before anything is enqueued,
    // so the caller's capture stays valid.
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(reinterpret_cast<hipStream_t>(stream), &cs) != hipSuccess) {
      (void)hipGetLastError();
      return EXL3_E_HIP;
    }
    if (cs != hipStreamCaptureStatusNone) return EXL3_E_INVALID;
    unsigned int bad = 0;
    const hipError_t e = exl3::count_bad_ids(gu, dn, topk_ids, t, topk, ws,
                                             reinterpret_cast<hipStream_t>(stream), bad);
    if (e != hipSuccess) return EXL3_E_HIP;
    trace("grouped routing ids out of range", (long long)bad, t, topk, gu.experts);
    if (bad) return EXL3_E_INVALID;
  }
  return from_hip(exl3::launch_grouped(gu, dn, static_cast<const uint16_t*>(x), topk_ids,
                                       topk_weights, t, topk, y, ws, ws_bytes, force_device_scope_on(),
                                       reinterpret_cast<hipStream_t>(stream)));
}

// Arguments of exl3_linear other than the workspace (EXL3_OK for m == 0 too).
exl3_status check_linear_args(const exl3_weight* w, const void* x, int64_t m, int64_t ldx, const void* y,
                              int64_t ldy, int32_t y_dtype) {
  exl3_status st = check_weight(w, 128, true);
  if (st != EXL3_OK) return st;
  if (m < 0 || m > kMaxRows) return EXL3_E_INVALID;
  if (y_dtype != EXL3_F16 && y_dtype != EXL3_F32) return EXL3_E_INVALID;
  if (ldx < w->k || ldy < w->n || ldx % 8 || ldy % 8) return EXL3_E_INVALID;
  // the kernels address a tensor's trellis with 32-bit byte offsets
  if (trellis_bytes(w->k, w->n, w->bits) >= kMaxTrellisBytes) return EXL3_E_INVALID;
  if (m > kGemvMaxRows && exl3::gemm_max_workgroups(w->k, w->n, m) > kMaxWorkgroups) return EXL3_E_INVALID;
  if (m == 0) return EXL3_OK;
  if (!x || !y || !aligned16(x) || !aligned16(y)) return EXL3_E_INVALID;
  return EXL3_OK;
}

// Eight threads per tile, in 256-thread workgroups.
bool reconstruct_fits(const exl3_weight* w) {
  return ((int64_t)(w->k / 16) * (w->n / 16) * 8 + 255) / 256 <= kMaxWorkgroups;
}

}  // namespace

// ---------------------------------------------------------------------------
// Scratch for exl3_linear_no_workspace: the workspace of one call, in a
// file-scope device array (every GPU the library runs on holds its own copy
// until the process ends).  Host code never uses the array's name as an
// address: the device address comes from hipGetSymbolAddress, taken once per
// device with that device current, and is kept per device.
// ---------------------------------------------------------------------------
static __device__ __align__(256) unsigned char scratch[EXL3_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
std::atomic<void*> g_scratch_ptr[kMaxDevices];

// Device address of `scratch` on the current device (looked up on the first
// call on that device).
exl3_status scratch_on_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) {
    (void)hipGetLastError();
    return EXL3_E_HIP;
  }
  if (dev < 0 || dev >= kMaxDevices) return EXL3_E_HIP;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (!p) {
      void* q = nullptr;
      if (hipGetSymbolAddress(&q, HIP_SYMBOL(scratch)) != hipSuccess || !q) {
        (void)hipGetLastError();
        return EXL3_E_HIP;
      }
      g_scratch_ptr[dev].store(q, std::memory_order_release);
      p = q;
    }
  }
  *out = p;
  return EXL3_OK;
}

}  // namespace

extern "C" {

int32_t exl3_abi_version(void) { return EXL3_ABI_VERSION; }

const char* exl3_status_str(exl3_status status) {
  switch (status) {
    case EXL3_OK: return "ok";
    case EXL3_E_INVALID: return "invalid argument (size, width, pointer or alignment)";
    case EXL3_E_UNSUPPORTED: return "unsupported codebook (only mul1 is decoded)";
    case EXL3_E_WORKSPACE: return "workspace missing or too small";
    case EXL3_E_HIP: return "HIP launch error";
    default: return "unknown status";
  }
}

exl3_status exl3_reconstruct(const exl3_weight* w, uint16_t* w_out, exl3_stream_t stream) {
  exl3_status st = check_weight(w, 16, false);
  if (st != EXL3_OK) return st;
  if (!reconstruct_fits(w)) return EXL3_E_INVALID;
  if (!w_out || !aligned16(w_out)) return EXL3_E_INVALID;
  trace("reconstruct k n bits", w->k, w->n, w->bits, 0);
  return from_hip(exl3::launch_reconstruct(w->trellis, w_out, w->k, w->n, w->bits,
                                           reinterpret_cast<hipStream_t>(stream)));
}

exl3_status exl3_hadamard(const void* in, void* out, int32_t dtype, int64_t rows, int64_t dim,
                          int64_t ld_in, int64_t ld_out, const uint16_t* sign_before,
                          const uint16_t* sign_after, exl3_stream_t stream) {
  if (dtype != EXL3_F16 && dtype != EXL3_F32) return EXL3_E_INVALID;
  if (rows < 0 || dim <= 0 || dim % 128) return EXL3_E_INVALID;
  // four 128-element blocks per 256-thread workgroup
  if (rows > kMaxWorkgroups * 4 || (rows * (dim / 128) + 3) / 4 > kMaxWorkgroups) return EXL3_E_INVALID;
  if (ld_in < dim || ld_out < dim || ld_in % 8 || ld_out % 8) return EXL3_E_INVALID;
  if (rows == 0) return EXL3_OK;
  if (!in || !out || !aligned16(in) || !aligned16(out)) return EXL3_E_INVALID;
  if (sign_before && !aligned16(sign_before)) return EXL3_E_INVALID;
  if (sign_after && !aligned16(sign_after)) return EXL3_E_INVALID;
  if (in == out && ld_in != ld_out) return EXL3_E_INVALID;
  const bool f32 = dtype == EXL3_F32;
  trace("hadamard rows dim dtype", rows, dim, dtype, 0);
  return from_hip(exl3::launch_hadamard(in, f32, out, f32, rows, dim, ld_in, ld_out, sign_before,
                                        sign_after, reinterpret_cast<hipStream_t>(stream)));
}

size_t exl3_linear_workspace_size(const exl3_weight* w, int64_t m) {
  if (check_weight(w, 128, false) != EXL3_OK || m < 0 || m > kMaxRows) return 0;
  if (m == 0) return 0;
  return linear_ws(w, m);
}

exl3_status exl3_linear_no_workspace(const exl3_weight* w, const void* x, int64_t m, int64_t ldx,
                                     void* y, int64_t ldy, int32_t y_dtype, exl3_stream_t stream) {
  exl3_status st = check_linear_args(w, x, m, ldx, y, ldy, y_dtype);
  if (st != EXL3_OK || m == 0) return st;
  const size_t need = linear_ws(w, m);
  if (need > EXL3_SCRATCH_BYTES) return EXL3_E_WORKSPACE;
  void* ws = nullptr;
  if (need > 0 && (st = scratch_on_current_device(&ws)) != EXL3_OK) return st;
  trace("linear_no_workspace k n m bytes", w->k, w->n, m, (long long)need);
  return exl3_linear(w, x, m, ldx, y, ldy, y_dtype, ws, need, stream);
}

exl3_status exl3_linear(const exl3_weight* w, const void* x, int64_t m, int64_t ldx, void* y,
                        int64_t ldy, int32_t y_dtype, void* ws, size_t ws_bytes,
                        exl3_stream_t stream) {
  exl3_status st = check_linear_args(w, x, m, ldx, y, ldy, y_dtype);
  if (st != EXL3_OK || m == 0) return st;
  const size_t need = linear_ws(w, m);
  if (need > 0 && (!ws || ws_bytes < need || !aligned16(ws))) return EXL3_E_WORKSPACE;
  const hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const bool f32 = y_dtype == EXL3_F32;
  if (m <= kGemvMaxRows) {
    const exl3::GemvPlan plan = exl3::plan_gemv(w->k, w->n, (int)m);
    trace("linear/gemv k n m splits", w->k, w->n, m, plan.splits);
    return from_hip(exl3::launch_gemv(w->trellis, w->suh, w->svh, w->bias, w->k, w->n, w->bits,
                                      static_cast<const uint16_t*>(x), (int)m, ldx, y, ldy, f32,
                                      ws, plan, s));
  }
  trace("linear/gemm k n m bits", w->k, w->n, m, w->bits);
  return from_hip(exl3::launch_gemm(w->trellis, w->suh, w->svh, w->bias, w->k, w->n, w->bits,
                                    static_cast<const uint16_t*>(x), (int)m, ldx, y, ldy, f32, ws,
                                    s));
}

size_t exl3_linear_int8_workspace_size(const exl3_weight* w, int64_t m) {
  if (check_weight(w, 128, false) != EXL3_OK || m <= 0 || m > kMaxRows) return 0;
  return exl3::linear_int8_workspace(w->k, m);
}

exl3_status exl3_linear_int8(const exl3_weight* w, const void* x, int64_t m, int64_t ldx, void* y,
                             int64_t ldy, int32_t y_dtype, void* ws, size_t ws_bytes,
                             exl3_stream_t stream) {
  exl3_status st = check_weight(w, 128, true);
  if (st != EXL3_OK) return st;
  if (m < 0 || m > kMaxRows) return EXL3_E_INVALID;
  if (y_dtype != EXL3_F16 && y_dtype != EXL3_F32) return EXL3_E_INVALID;
  if (ldx < w->k || ldy < w->n || ldx % 8 || ldy % 8) return EXL3_E_INVALID;
  if (trellis_bytes(w->k, w->n, w->bits) >= kMaxTrellisBytes) return EXL3_E_INVALID;
  // the GEMM addresses a 256-row tile of int8 activations with 32-bit offsets
  if ((int64_t)w->k * 256 >= ((int64_t)1 << 31)) return EXL3_E_INVALID;
  if (exl3::linear_int8_max_workgroups(w->k, w->n, m) > kMaxWorkgroups) return EXL3_E_INVALID;
  if (m == 0) return EXL3_OK;
  if (!x || !y || !aligned16(x) || !aligned16(y)) return EXL3_E_INVALID;
  const size_t need = exl3::linear_int8_workspace(w->k, m);
  if (!ws || ws_bytes < need || !aligned16(ws)) return EXL3_E_WORKSPACE;
  trace("linear_int8 k n m bits", w->k, w->n, m, w->bits);
  return from_hip(exl3::launch_linear_int8(w->trellis, w->suh, w->svh, w->bias, w->k, w->n, w->bits,
                                           static_cast<const uint16_t*>(x), m, ldx, y, ldy,
                                           y_dtype == EXL3_F32, ws,
                                           reinterpret_cast<hipStream_t>(stream)));
}

exl3_status exl3_reconstruct_int8(const exl3_weight* w, int8_t* w_out, exl3_stream_t stream) {
  exl3_status st = check_weight(w, 16, false);
  if (st != EXL3_OK) return st;
  if (!reconstruct_fits(w)) return EXL3_E_INVALID;
  if (!w_out || !aligned16(w_out)) return EXL3_E_INVALID;
  trace("reconstruct_int8 k n bits", w->k, w->n, w->bits, 0);
  return from_hip(exl3::launch_reconstruct_int8(w->trellis, w_out, w->k, w->n, w->bits,
                                                reinterpret_cast<hipStream_t>(stream)));
}

size_t exl3_linear_multi_workspace_size(const exl3_weight* const* w, int32_t count, int64_t m) {
  if (check_multi(w, count) != EXL3_OK || m <= 0 || m > kMaxRows) return 0;
  return multi_ws(w, count, m);
}

exl3_status exl3_linear_multi(const exl3_weight* const* w, int32_t count, const void* x, int64_t m,
                              int64_t ldx, void* const* y, const int64_t* ldy, int32_t y_dtype,
                              void* ws, size_t ws_bytes, exl3_stream_t stream) {
  exl3_status st = check_multi(w, count);
  if (st != EXL3_OK) return st;
  if (m < 0 || m > kMaxRows) return EXL3_E_INVALID;
  if (y_dtype != EXL3_F16 && y_dtype != EXL3_F32) return EXL3_E_INVALID;
  if (!y || !ldy || ldx < w[0]->k || ldx % 8) return EXL3_E_INVALID;
  if (m > kGemvMaxRows)
    for (int i = 0; i < count; ++i)
      if (exl3::gemm_max_workgroups(w[i]->k, w[i]->n, m) > kMaxWorkgroups) return EXL3_E_INVALID;
  for (int i = 0; i < count; ++i)
    if (ldy[i] < w[i]->n || ldy[i] % 8) return EXL3_E_INVALID;
  if (m == 0) return EXL3_OK;
  if (!x || !aligned16(x)) return EXL3_E_INVALID;
  for (int i = 0; i < count; ++i)
    if (!y[i] || !aligned16(y[i])) return EXL3_E_INVALID;
  const size_t need = multi_ws(w, count, m);
  if (need > 0 && (!ws || ws_bytes < need || !aligned16(ws))) return EXL3_E_WORKSPACE;
  const hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (m == 1) {
    exl3::MultiTensor t[EXL3_MAX_MULTI];
    for (int i = 0; i < count; ++i) t[i] = {w[i]->trellis, w[i]->suh, w[i]->svh, w[i]->bias, w[i]->n, w[i]->bits};
    const exl3::MultiPlan mp = exl3::plan_gemv_multi(t, count, w[0]->k);
    trace("linear_multi/gemv count k waves tasks", count, w[0]->k, mp.wbase[count], mp.fbase[count]);
    // x has one row; its stride does not matter
    return from_hip(exl3::launch_gemv_multi(t, count, w[0]->k, static_cast<const uint16_t*>(x), y,
                                            ldy, y_dtype == EXL3_F32, ws, mp, s));
  }
  // several rows: each tensor in turn on the single-tensor path (the same
  // kernels and results as separate exl3_linear calls), sharing the workspace
  for (int i = 0; i < count; ++i) {
    st = exl3_linear(w[i], x, m, ldx, y[i], ldy[i], y_dtype, ws, ws_bytes, stream);
    if (st != EXL3_OK) return st;
  }
  return EXL3_OK;
}

size_t exl3_grouped_experts_workspace_size(const exl3_expert_weights* gate_up,
                                           const exl3_expert_weights* down, int64_t t,
                                           int32_t topk) {
  if (check_grouped(gate_up, down, t, topk) != EXL3_OK || t == 0) return 0;
  return exl3::grouped_workspace(desc(gate_up), desc(down), t, topk);
}

exl3_status exl3_grouped_experts(const exl3_expert_weights* gate_up,
                                 const exl3_expert_weights* down, const void* x,
                                 const int32_t* topk_ids, const float* topk_weights, int64_t t,
                                 int32_t topk, float* y, void* ws, size_t ws_bytes,
                                 exl3_stream_t stream) {
  const exl3_status st = check_grouped(gate_up, down, t, topk);
  if (st != EXL3_OK) return st;
  return run_grouped(desc(gate_up), desc(down), x, topk_ids, topk_weights, t, topk, y, ws,
                     ws_bytes, stream);
}

size_t exl3_grouped_experts_mixed_workspace_size(const exl3_expert_weights* gate_up,
                                                 const exl3_expert_widths* gate_up_widths,
                                                 const exl3_expert_weights* down,
                                                 const exl3_expert_widths* down_widths, int64_t t,
                                                 int32_t topk) {
  if (check_grouped_mixed(gate_up, gate_up_widths, down, down_widths, t, topk) != EXL3_OK || t == 0)
    return 0;
  return exl3::grouped_workspace(desc_mixed(gate_up, gate_up_widths), desc_mixed(down, down_widths),
                                 t, topk);
}

exl3_status exl3_grouped_experts_mixed(const exl3_expert_weights* gate_up,
                                       const exl3_expert_widths* gate_up_widths,
                                       const exl3_expert_weights* down,
                                       const exl3_expert_widths* down_widths, const void* x,
                                       const int32_t* topk_ids, const float* topk_weights,
                                       int64_t t, int32_t topk, float* y, void* ws,
                                       size_t ws_bytes, exl3_stream_t stream) {
  const exl3_status st = check_grouped_mixed(gate_up, gate_up_widths, down, down_widths, t, topk);
  if (st != EXL3_OK) return st;
  return run_grouped(desc_mixed(gate_up, gate_up_widths), desc_mixed(down, down_widths), x,
                     topk_ids, topk_weights, t, topk, y, ws, ws_bytes, stream);
}

}  // extern "C"
