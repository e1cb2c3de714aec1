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

// The dense prefill GEMM's input: x' = (x .* suh) H (fp16 in and out), written
// fragment-major (kGemmFragBytes): element (r, c) at
// ((r / 16 * (k / 32) + c / 32) * 64 + 16 ((c % 32) / 8) + r % 16) * 8 + c % 8.
// Rows m .. m_pad - 1 (up to a multiple of 16) are written as zeros.
// One workgroup per (16-row group, kFragBlocks consecutive 128-element
// blocks): wave w transforms rows 4 w .. 4 w + 3 of the group (fwht128_x8
// layout, one row per 16 lanes, lane j = l % 16 holding elements 8 j .. 8 j +
// 7), with the loads of all its blocks issued first, and the group's output
// for a block, four whole fragments (4 KB, contiguous), comes from one
// workgroup: every 128-byte line is written by one CU into one L2.  (A line
// holds eight rows of the group; with one row per workgroup, lines were
// assembled from workgroups on different XCDs and went to memory as partial
// writes.)  Large grids take kFragBlocks blocks per workgroup, the loads of
// all of them issued first (4096 x 17408: 49 us against 65 with one block per
// workgroup); small ones keep one block per workgroup, to spread over the CUs.
constexpr int kFragBlocks = 4;
constexpr int64_t kFragWideGrid = 8192;  // one-block grids at least this large take kFragBlocks

__global__ __launch_bounds__(256) void input_frag_kernel(const uint16_t* __restrict__ x, int64_t ldx,
                                                         int64_t m, int64_t bpr,
                                                         const uint16_t* __restrict__ suh, int per,
                                                         uint16_t* __restrict__ out) {
  const int64_t nbw = (bpr + per - 1) / per;  // workgroups per group
  const int64_t G = (int64_t)blockIdx.x / nbw;
  const int64_t b0 = ((int64_t)blockIdx.x - G * nbw) * per;
  const int wave = (int)(threadIdx.x >> 6), lane = (int)(threadIdx.x & 63);
  const int r = 4 * wave + (lane >> 4);  // row inside the group
  const int j = lane & 15;
  const int64_t row = 16 * G + r;
  uint4 xv[kFragBlocks], sv[kFragBlocks];
#pragma unroll
  for (int u = 0; u < kFragBlocks; ++u) {
    if (u < per) {  // uniform
      const int64_t b = b0 + u < bpr ? b0 + u : b0;  // past the row's end: its first block again (not stored)
      const int64_t col = b * 128 + 8 * j;
      xv[u] = row < m ? *reinterpret_cast<const uint4*>(x + row * ldx + col) : make_uint4(0u, 0u, 0u, 0u);
      sv[u] = *reinterpret_cast<const uint4*>(suh + col);
    }
  }
  const int64_t kb = bpr * 4;  // 32-element k blocks per row
#pragma unroll
  for (int u = 0; u < kFragBlocks; ++u) {
    const int64_t b = b0 + u;
    if (u >= per || b >= bpr) break;  // uniform
    float v[8];
    const uint32_t xw[4] = {xv[u].x, xv[u].y, xv[u].z, xv[u].w};
    const uint32_t sw[4] = {sv[u].x, sv[u].y, sv[u].z, sv[u].w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[2 * e] = h2f((uint16_t)(xw[e] & 0xFFFF)) * h2f((uint16_t)(sw[e] & 0xFFFF));
      v[2 * e + 1] = h2f((uint16_t)(xw[e] >> 16)) * h2f((uint16_t)(sw[e] >> 16));
    }
    if (row >= m) {
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = 0.f;
    }
    fwht128_x8(v);  // every lane of the wave takes part (zero rows included)
    uint32_t o[4];
#pragma unroll
    for (int e = 0; e < 4; ++e)
      o[e] = (uint32_t)f2h(v[2 * e] * kInvSqrt128) | ((uint32_t)f2h(v[2 * e + 1] * kInvSqrt128) << 16);
    // 16-byte piece (k block j / 4 of the four, lane group j % 4, row r)
    uint16_t* dst = out + ((G * kb + 4 * b) * 64 + (j >> 2) * 64 + (j & 3) * 16 + r) * 8;
    *reinterpret_cast<uint4*>(dst) = make_uint4(o[0], o[1], o[2], o[3]);
  }
}

hipError_t launch_input_frag(const uint16_t* x, int64_t ldx, int64_t m, int64_t k,
                             const uint16_t* suh, uint16_t* out, hipStream_t s) {
  const int64_t bpr = k / 128;
  const int64_t groups = (m + 15) / 16;
  const int per = groups * bpr >= kFragWideGrid ? kFragBlocks : 1;
  const unsigned blocks = (unsigned)(groups * ((bpr + per - 1) / per));
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL(input_frag_kernel, dim3(blocks), dim3(256), 0, s, x, ldx, m, bpr, suh, per, out);
  return hipGetLastError();
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
