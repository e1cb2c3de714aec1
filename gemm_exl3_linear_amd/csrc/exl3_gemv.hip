// Decode GEMV for 1..16 activation rows (the memory-bound regime: each
// trellis word is read from HBM exactly once per call).
//
// y = ((x .* suh) Hk  W~  Hn) .* svh (+ bias)   (exl3xpu README, "Prefill:
// int8 linears ...": the product runs in the Hadamard domain; "Layout": the
// Hadamard-in and Hadamard-out kernels around the vector GEMV).
//
// Kernel 1 (gemv_kernel), one workgroup per (128-column block, k range[, unit]):
//   prologue  x' = (x .* suh) H for the workgroup's k range, fp16, into LDS
//   main loop each wave walks k tiles; lane (t, p) streams the row pair p of
//             n-tile t with one coalesced load, decodes 32 weights in
//             registers into k-pairs, and hands them to the matrix cores
//             through a small per-wave LDS transpose (MFMA 16x16x16 f16, the
//             activation rows padded to 16, fp32 accumulation)
//   end       the four waves' partial sums are added in a fixed order and
//             written to the fp32 workspace, one slice per k range
// Kernel 2 (gemv_epilogue): adds the k-range slices in a fixed order, applies
//   the output transform, svh and bias, and casts.  No atomics: the result is
//   bit-reproducible and every row is computed the same way whatever m is.
#include "exl3_device.hpp"
#include "exl3_gemv.hpp"
#include "exl3_internal.hpp"

namespace exl3 {

// ---------------------------------------------------------------------------
// epilogue: y = (sum_s partial_s) H .* svh (+ bias), one wave per (row, block)
// ---------------------------------------------------------------------------
template <bool Y_F32>
__global__ __launch_bounds__(256) void gemv_epilogue(const float* __restrict__ partial, int splits,
                                                     int m, int n, const uint16_t* __restrict__ svh,
                                                     const uint16_t* __restrict__ bias, void* y,
                                                     int64_t ldy) {
  const int nblocks = n >> 7;
  const int task = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (task >= m * nblocks) return;
  const int i = task / nblocks, nb = task - i * nblocks;
  const int col = nb * 128 + 2 * (int)lane_id();
  float a = 0.f, b = 0.f;
  for (int s = 0; s < splits; ++s) {
    const float2 v = *reinterpret_cast<const float2*>(partial + ((int64_t)s * m + i) * n + col);
    a += v.x;
    b += v.y;
  }
  fwht128_pair(a, b);
  a *= kInvSqrt128;
  b *= kInvSqrt128;
  const uint32_t sv = *reinterpret_cast<const uint32_t*>(svh + col);
  a *= h2f((uint16_t)(sv & 0xFFFF));
  b *= h2f((uint16_t)(sv >> 16));
  if (bias) {
    const uint32_t bv = *reinterpret_cast<const uint32_t*>(bias + col);
    a += h2f((uint16_t)(bv & 0xFFFF));
    b += h2f((uint16_t)(bv >> 16));
  }
  if constexpr (Y_F32) {
    *reinterpret_cast<float2*>(static_cast<float*>(y) + (int64_t)i * ldy + col) = make_float2(a, b);
  } else {
    *reinterpret_cast<uint32_t*>(static_cast<uint16_t*>(y) + (int64_t)i * ldy + col) =
        (uint32_t)f2h(a) | ((uint32_t)f2h(b) << 16);
  }
}

// ---------------------------------------------------------------------------
// planning and launch (dense tensors)
// ---------------------------------------------------------------------------
size_t gemv_lds_bytes(int kc, int m) {
  const size_t xs = ((size_t)kc * m * 2 + 15) & ~(size_t)15;
  const size_t tr = 4 * 64 * 20 * 4;
  const size_t red = (size_t)4 * m * 128 * 4;
  return xs + (tr > red ? tr : red);
}

int gemv_choose_splits(int k, int groups, int m, int target_wgs) {
  const int kb = k / 128;
  int best = kb;
  for (int s = 1; s <= kb; ++s) {
    if (kb % s) continue;
    const int kc = k / s;
    if (gemv_lds_bytes(kc, m) > kGemvMaxLds) continue;
    if ((int64_t)groups * s >= target_wgs) { best = s; break; }
  }
  return best;
}

GemvPlan plan_gemv(int k, int n, int m) {
  GemvPlan p;
  // The split is chosen for the largest row count (16) so that it does not
  // depend on m: every row then sees the same summation order at any m <= 16.
  p.splits = gemv_choose_splits(k, n / 128, 16, kGemvTargetWorkgroups);
  p.kc = k / p.splits;
  p.lds = gemv_lds_bytes(p.kc, m);
  p.ws = (size_t)p.splits * m * n * sizeof(float);
  return p;
}

struct DenseGemvRes {
  const uint16_t* trellis;
  const uint16_t* suh;
  const uint16_t* x;
  int64_t ldx;
  int m;
  int n;
  float* ws;
  __device__ GemvTask task(int /*unit*/, int split) const {
    GemvTask T;
    T.valid = true;
    T.trellis = trellis;
    T.suh = suh;
    T.x = x;
    T.ldx = ldx;
    T.m = m;
    T.partial = ws + (int64_t)split * m * n;
    return T;
  }
};

template <int K>
struct DenseGemvRun {
  static hipError_t run(const DenseGemvRes& r, int k, int n, const GemvPlan& plan,
                        hipStream_t s) {
    hipLaunchKernelGGL((gemv_kernel<K, DenseGemvRes>), dim3(n / 128, plan.splits, 1), dim3(256),
                       plan.lds, s, r, k, n, plan.kc);
    return hipGetLastError();
  }
};

hipError_t launch_gemv_epilogue(const float* partial, int splits, int m, int n,
                                const uint16_t* svh, const uint16_t* bias, void* y, int64_t ldy,
                                bool y_f32, hipStream_t s) {
  const int tasks = m * (n / 128);
  const unsigned blocks = (unsigned)((tasks + 3) / 4);
  if (y_f32)
    hipLaunchKernelGGL(gemv_epilogue<true>, dim3(blocks), dim3(256), 0, s, partial, splits, m, n,
                       svh, bias, y, ldy);
  else
    hipLaunchKernelGGL(gemv_epilogue<false>, dim3(blocks), dim3(256), 0, s, partial, splits, m, n,
                       svh, bias, y, ldy);
  return hipGetLastError();
}

hipError_t launch_gemv(const uint16_t* trellis, const uint16_t* suh, const uint16_t* svh,
                       const uint16_t* bias, int k, int n, int bits, const uint16_t* x, int m,
                       int64_t ldx, void* y, int64_t ldy, bool y_f32, void* ws,
                       const GemvPlan& plan, hipStream_t s) {
  DenseGemvRes r{trellis, suh, x, ldx, m, n, static_cast<float*>(ws)};
  hipError_t e = dispatch_bits<DenseGemvRun>(bits, r, k, n, plan, s);
  if (e != hipSuccess) return e;
  return launch_gemv_epilogue(static_cast<const float*>(ws), plan.splits, m, n, svh, bias, y, ldy,
                              y_f32, s);
}

}  // namespace exl3
