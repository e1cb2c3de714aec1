// Measurement kernels for the benchmark (not part of the EXL3 library's
// interface): a plain streaming read, the practical HBM read ceiling that the
// decode GEMV's rate is compared with.  Built into libexl3_bench.so.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

// Every thread reads 16-byte words at a grid stride, UNROLL of them in
// flight, and folds them into one word; one word per workgroup is stored so
// that no load can be dropped.
template <int UNROLL>
__global__ __launch_bounds__(256) void stream_read_kernel(const uint4* __restrict__ p, int64_t words,
                                                          uint32_t* __restrict__ sink) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  uint32_t acc = 0;
  for (; i + (UNROLL - 1) * stride < words; i += UNROLL * stride) {
    uint4 v[UNROLL];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) v[u] = p[i + u * stride];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < words; i += stride) {
    const uint4 v = p[i];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  __shared__ uint32_t red[256];
  red[threadIdx.x] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t a = 0;
    for (int t = 0; t < 256; ++t) a ^= red[t];
    sink[blockIdx.x] = a;
  }
}

typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef float float4_t __attribute__((ext_vector_type(4)));

// A chain of kMfmaChain v_mfma_f32_16x16x16_f16 per wave, each on its own A
// and B fragments (lane l holds A[l % 16][4 (l / 16) .. + 3] and
// B[4 (l / 16) .. + 3][l % 16]), accumulating into the previous result as a
// decode GEMV accumulates over k: once with every A and once with every A
// negated (sign bits flipped), nothing else around them.  out holds the
// result for problem w at [w][0][lane][4], the negated one at [w][1][lane][4].
constexpr int kMfmaChain = 4;
__global__ __launch_bounds__(64) void mfma_negation_kernel(const uint16_t* __restrict__ a,
                                                           const uint16_t* __restrict__ b,
                                                           float* __restrict__ out) {
  const int w = blockIdx.x, l = threadIdx.x;
  float4_t dp = {0.f, 0.f, 0.f, 0.f}, dn = {0.f, 0.f, 0.f, 0.f};
  for (int c = 0; c < kMfmaChain; ++c) {
    half4_t av, an, bv;
    for (int i = 0; i < 4; ++i) {
      const int64_t e = (((int64_t)w * kMfmaChain + c) * 64 + l) * 4 + i;
      const uint16_t x = a[e];
      av[i] = __builtin_bit_cast(_Float16, x);
      an[i] = __builtin_bit_cast(_Float16, (uint16_t)(x ^ 0x8000u));
      bv[i] = __builtin_bit_cast(_Float16, b[e]);
    }
    dp = __builtin_amdgcn_mfma_f32_16x16x16f16(av, bv, dp, 0, 0, 0);
    dn = __builtin_amdgcn_mfma_f32_16x16x16f16(an, bv, dn, 0, 0, 0);
  }
  for (int i = 0; i < 4; ++i) {
    out[((w * 2 + 0) * 64 + l) * 4 + i] = dp[i];
    out[((w * 2 + 1) * 64 + l) * 4 + i] = dn[i];
  }
}

}  // namespace

extern "C" {

// `problems` independent chains of four 16x16x16 fp16 products on the
// matrix cores, each with A and with -A: a, b fp16 [problems][4][64][4]
// (lane fragments), out fp32 [problems][2][64][4].  Returns 0, -1 for invalid arguments, or the HIP
// error code of the launch.
int exl3_bench_mfma_negation(const uint16_t* a, const uint16_t* b, float* out, int problems,
                             hipStream_t stream) {
  if (!a || !b || !out || problems < 1 || problems > (1 << 20)) return -1;
  hipLaunchKernelGGL(mfma_negation_kernel, dim3(problems), dim3(64), 0, stream, a, b, out);
  return (int)hipGetLastError();
}

// Reads `bytes` bytes (a multiple of 16) at the 16-byte aligned device
// pointer p on `stream` with `workgroups` workgroups of 256 threads and
// `unroll` (4 or 8) loads in flight per thread; sink is a device buffer of
// at least `workgroups` uint32.  Returns 0, or -1 for invalid arguments, or
// the HIP error code of the launch.
int exl3_bench_stream_read(const void* p, size_t bytes, uint32_t* sink, int workgroups, int unroll,
                           hipStream_t stream) {
  if (!p || !sink || bytes % 16 || ((uintptr_t)p & 15) || workgroups < 1 || workgroups > (1 << 20))
    return -1;
  const int64_t words = (int64_t)(bytes / 16);
  if (unroll == 8)
    hipLaunchKernelGGL(stream_read_kernel<8>, dim3(workgroups), dim3(256), 0, stream,
                       static_cast<const uint4*>(p), words, sink);
  else if (unroll == 4)
    hipLaunchKernelGGL(stream_read_kernel<4>, dim3(workgroups), dim3(256), 0, stream,
                       static_cast<const uint4*>(p), words, sink);
  else
    return -1;
  return (int)hipGetLastError();
}

}  // extern "C"
