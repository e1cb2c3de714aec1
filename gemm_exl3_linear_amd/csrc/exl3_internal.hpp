// Host-side declarations shared by the kernel files and the C-ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "exl3_sk_split.hpp"

namespace exl3 {

// Dispatch a runtime width K (1..8) to a template instantiation.
template <template <int> class F, typename... Args>
hipError_t dispatch_bits(int bits, Args&&... args) {
  switch (bits) {
    case 1: return F<1>::run(args...);
    case 2: return F<2>::run(args...);
    case 3: return F<3>::run(args...);
    case 4: return F<4>::run(args...);
    case 5: return F<5>::run(args...);
    case 6: return F<6>::run(args...);
    case 7: return F<7>::run(args...);
    case 8: return F<8>::run(args...);
    default: return hipErrorInvalidValue;
  }
}

// --- reconstruct -----------------------------------------------------------
hipError_t launch_reconstruct(const uint16_t* trellis, uint16_t* out, int k, int n, int bits,
                              hipStream_t s);

// --- Hadamard --------------------------------------------------------------
// out = ((in .* sign_before) H) .* sign_after, blocks of 128, fp32 arithmetic.
// in_f32 / out_f32 select the element types.  Rows are independent.
// x' = (x .* suh) H for the dense prefill GEMM, fp16, fragment-major, rows
// padded with zeros to a multiple of 16
hipError_t launch_input_frag(const uint16_t* x, int64_t ldx, int64_t m, int64_t k,
                             const uint16_t* suh, uint16_t* out, hipStream_t s);
hipError_t launch_hadamard(const void* in, bool in_f32, void* out, bool out_f32, int64_t rows,
                           int64_t dim, int64_t ld_in, int64_t ld_out,
                           const uint16_t* sign_before, const uint16_t* sign_after,
                           hipStream_t s);

// --- dense linear ----------------------------------------------------------
struct GemvPlan {
  SkSplit split;     // runs of the workgroups
  int splits;        // workgroups of the grid
  int kc;            // longest run of units
  int slots;         // partial-sum slots per 256-column pair
  size_t xprep_off;  // offset of the transformed rows x' (m > 4)
  size_t ws;         // workspace bytes (partials + x')
};
GemvPlan plan_gemv(int k, int n, int m);
hipError_t launch_gemv(const uint16_t* trellis, const uint16_t* suh, const uint16_t* svh,
                       const uint16_t* bias, int k, int n, int bits, const uint16_t* x,
                       int m, int64_t ldx, void* y, int64_t ldy, bool y_f32, void* ws,
                       const GemvPlan& plan, hipStream_t s);

// several tensors sharing one activation row (m == 1), one launch pair
constexpr int kMultiMax = 8;
struct MultiTensor {
  const uint16_t* trellis;
  const uint16_t* suh;
  const uint16_t* svh;
  const uint16_t* bias;
  int n, bits;
};
struct MultiPlan {
  int count;
  SkSplit split[kMultiMax];
  int waves[kMultiMax];
  int slots[kMultiMax];
  size_t part_off[kMultiMax];
  int wbase[kMultiMax + 1];
  int fbase[kMultiMax + 1];
  size_t ws;
};
MultiPlan plan_gemv_multi(const MultiTensor* t, int count, int k);
hipError_t launch_gemv_multi(const MultiTensor* t, int count, int k, const uint16_t* x, void* const* y,
                             const int64_t* ldy, bool y_f32, void* ws, const MultiPlan& mp,
                             hipStream_t s);

size_t gemm_workspace(int k, int n, int m);
// Largest workgroup count of the launches of a prefill call (input transform
// and GEMM), for the host's check that every grid fits a launch.
int64_t gemm_max_workgroups(int k, int n, int64_t m);
hipError_t launch_gemm(const uint16_t* trellis, const uint16_t* suh, const uint16_t* svh,
                       const uint16_t* bias, int k, int n, int bits, const uint16_t* x,
                       int m, int64_t ldx, void* y, int64_t ldy, bool y_f32, void* ws,
                       hipStream_t s);

// --- int8 prefill ------------------------------------------------------------
// workspace: x_q (int8, fragment-major, rows padded to 16) and the row scales
size_t linear_int8_workspace(int k, int64_t m);
int64_t linear_int8_max_workgroups(int k, int n, int64_t m);
hipError_t launch_linear_int8(const uint16_t* trellis, const uint16_t* suh, const uint16_t* svh,
                              const uint16_t* bias, int k, int n, int bits, const uint16_t* x,
                              int64_t m, int64_t ldx, void* y, int64_t ldy, bool y_f32, void* ws,
                              hipStream_t s);
hipError_t launch_reconstruct_int8(const uint16_t* trellis, int8_t* out, int k, int n, int bits,
                                   hipStream_t s);

// --- grouped experts -------------------------------------------------------
struct ArenaDesc {
  const uint16_t* trellis;
  const uint16_t* suh;
  const uint16_t* svh;
  int experts, slots, k, n, bits;  // bits == 0: a width per expert (below)
  const int32_t* ebits = nullptr;  // device int32 [experts]: width of expert e
  const int64_t* eoff = nullptr;   // device int64 [experts]: first word of expert e
};
size_t grouped_workspace(const ArenaDesc& gu, const ArenaDesc& dn, int64_t t, int topk);
// Counts the routing ids outside [0, experts) on the device and waits for
// the count (a host synchronisation on s).
hipError_t count_bad_ids(const ArenaDesc& gu, const ArenaDesc& dn, const int32_t* ids, int64_t t,
                         int topk, void* ws, hipStream_t s, unsigned int& bad);
// off_xcd_all: every workgroup of the token-parallel path takes the
// device-scope hand-off (as one dispatched off its planned XCD does).
hipError_t launch_grouped(const ArenaDesc& gu, const ArenaDesc& dn, const uint16_t* x,
                          const int32_t* ids, const float* w, int64_t t, int topk, float* y,
                          void* ws, size_t ws_bytes, bool off_xcd_all, hipStream_t s);

}  // namespace exl3
