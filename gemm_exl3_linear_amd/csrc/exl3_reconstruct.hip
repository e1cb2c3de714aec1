// Whole-tensor decode to the Hadamard-domain weight W~ (fp16, [k][n]).
// The exl3xpu README ("Correctness") gates every kernel path on bit-identical
// dequantized weights; this kernel runs the same decode routine as the GEMV,
// GEMM and grouped kernels and writes its result out for that check.
#include "exl3_device.hpp"
#include "exl3_internal.hpp"

namespace exl3 {

template <int K>
__global__ __launch_bounds__(256) void reconstruct_kernel(const uint16_t* __restrict__ trellis,
                                                          uint16_t* __restrict__ out, int nt,
                                                          int64_t tiles, int n) {
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t tile = gid >> 3;
  const int p = (int)(gid & 7);
  if (tile >= tiles) return;  // whole 8-lane groups leave together
  const int64_t a = tile / nt, b = tile % nt;
  const uint32_t* src =
      reinterpret_cast<const uint32_t*>(trellis + tile * (16 * K)) + (int64_t)K * p;
  uint32_t D[K];
  load_rowpair<K>(src, D);
  const uint32_t spill = spill_from_next(D[0]);
  uint32_t wp[16];
  decode_rowpair<K>(D, spill, wp);
  // row 2p gets the low halves, row 2p+1 the high halves
  uint32_t r0[8], r1[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    r0[c] = __builtin_amdgcn_perm(wp[2 * c + 1], wp[2 * c], 0x05040100u);
    r1[c] = __builtin_amdgcn_perm(wp[2 * c + 1], wp[2 * c], 0x07060302u);
  }
  uint16_t* o0 = out + (16 * a + 2 * p) * (int64_t)n + 16 * b;
  uint16_t* o1 = o0 + n;
  uint4* q0 = reinterpret_cast<uint4*>(o0);
  uint4* q1 = reinterpret_cast<uint4*>(o1);
  q0[0] = make_uint4(r0[0], r0[1], r0[2], r0[3]);
  q0[1] = make_uint4(r0[4], r0[5], r0[6], r0[7]);
  q1[0] = make_uint4(r1[0], r1[1], r1[2], r1[3]);
  q1[1] = make_uint4(r1[4], r1[5], r1[6], r1[7]);
}

template <int K>
struct ReconstructRun {
  static hipError_t run(const uint16_t* trellis, uint16_t* out, int k, int n, hipStream_t s) {
    const int64_t tiles = (int64_t)(k / 16) * (n / 16);
    const int64_t threads = tiles * 8;
    const unsigned blocks = (unsigned)((threads + 255) / 256);
    hipLaunchKernelGGL(reconstruct_kernel<K>, dim3(blocks), dim3(256), 0, s, trellis, out, n / 16,
                       tiles, n);
    return hipGetLastError();
  }
};

hipError_t launch_reconstruct(const uint16_t* trellis, uint16_t* out, int k, int n, int bits,
                              hipStream_t s) {
  return dispatch_bits<ReconstructRun>(bits, trellis, out, k, n, s);
}

}  // namespace exl3
