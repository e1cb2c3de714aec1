// Standalone randomized Hadamard transform: out = ((in .* sb) H) .* sa, with
// H the orthonormal 128-point Sylvester Walsh-Hadamard matrix applied to each
// block of 128 consecutive elements of every row (exl3xpu README, "Layout":
// Hadamard in/out kernels; all linear dims are multiples of 128 per "Adding a
// model").  One wave transforms one block: lane l holds elements 2l, 2l+1.
#include "exl3_device.hpp"
#include "exl3_internal.hpp"

namespace exl3 {

template <bool IN_F32, bool OUT_F32>
__global__ __launch_bounds__(256) void hadamard_kernel(const void* __restrict__ in,
                                                       void* __restrict__ out, int64_t rows,
                                                       int64_t blocks_per_row, int64_t ld_in,
                                                       int64_t ld_out,
                                                       const uint16_t* __restrict__ sb,
                                                       const uint16_t* __restrict__ sa) {
  const int64_t task = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (task >= rows * blocks_per_row) return;  // whole waves leave together
  const int64_t row = task / blocks_per_row;
  const int64_t col = (task % blocks_per_row) * 128 + 2 * (int64_t)lane_id();
  float a, b;
  if constexpr (IN_F32) {
    const float2 v = *reinterpret_cast<const float2*>(static_cast<const float*>(in) + row * ld_in + col);
    a = v.x; b = v.y;
  } else {
    const uint32_t v = *reinterpret_cast<const uint32_t*>(static_cast<const uint16_t*>(in) + row * ld_in + col);
    a = h2f((uint16_t)(v & 0xFFFF)); b = h2f((uint16_t)(v >> 16));
  }
  if (sb) {
    const uint32_t s = *reinterpret_cast<const uint32_t*>(sb + col);
    a *= h2f((uint16_t)(s & 0xFFFF)); b *= h2f((uint16_t)(s >> 16));
  }
  fwht128_pair(a, b);
  a *= kInvSqrt128; b *= kInvSqrt128;
  if (sa) {
    const uint32_t s = *reinterpret_cast<const uint32_t*>(sa + col);
    a *= h2f((uint16_t)(s & 0xFFFF)); b *= h2f((uint16_t)(s >> 16));
  }
  if constexpr (OUT_F32) {
    *reinterpret_cast<float2*>(static_cast<float*>(out) + row * ld_out + col) = make_float2(a, b);
  } else {
    const uint32_t v = (uint32_t)f2h(a) | ((uint32_t)f2h(b) << 16);
    *reinterpret_cast<uint32_t*>(static_cast<uint16_t*>(out) + row * ld_out + col) = v;
  }
}

hipError_t launch_hadamard(const void* in, bool in_f32, void* out, bool out_f32, int64_t rows,
                           int64_t dim, int64_t ld_in, int64_t ld_out,
                           const uint16_t* sign_before, const uint16_t* sign_after,
                           hipStream_t s) {
  const int64_t bpr = dim / 128;
  const int64_t tasks = rows * bpr;
  const unsigned blocks = (unsigned)((tasks + 3) / 4);
  if (blocks == 0) return hipSuccess;
#define EXL3_HAD(I, O)                                                                       \
  hipLaunchKernelGGL((hadamard_kernel<I, O>), dim3(blocks), dim3(256), 0, s, in, out, rows, bpr, \
                     ld_in, ld_out, sign_before, sign_after)
  if (in_f32 && out_f32) EXL3_HAD(true, true);
  else if (in_f32) EXL3_HAD(true, false);
  else if (out_f32) EXL3_HAD(false, true);
  else EXL3_HAD(false, false);
#undef EXL3_HAD
  return hipGetLastError();
}

}  // namespace exl3
