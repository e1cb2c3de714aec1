// int8 prefill linear (exl3xpu README, "Prefill: int8 linears and oneDNN
// fused attention": activations take one int8 scale per row inside the input
// Hadamard, weights one static scale inside the decode, the product runs in
// int8 with both scales applied and writes fp16).
//
//   quant_groups_held_kernel / quant_pairs_kernel / quant_rows_kernel
//                      x' = (x .* suh) H_k in fp32 per row, a = max |x'|,
//                      x_q = RNE(127 x' / a) (int8, fragment-major) and a / 127.
//   gemm_i8_kernel     decode to int8 + v_mfma_i32_16x16x64_i8, epilogue with
//                      both scales, the output transform, svh, bias, cast.
//   reconstruct_i8_kernel  the int8 weights W_q [k][n], for the bit-exact
//                      decode check.
#include "exl3_gemm_i8.hpp"
#include "exl3_internal.hpp"

namespace exl3 {

// ---------------------------------------------------------------------------
// input transform with per-row int8 quantization
// ---------------------------------------------------------------------------
// Launch shapes of one computation (the same per-element arithmetic and the
// same maximum, so their outputs are identical):
//   quant_groups_held_kernel (m >= kQuantGroupMinRows, rows of at most
//     4 kQuantHeldPasses blocks): one workgroup of 16 waves per 16-row group,
//     wave w on row w of the group, so every 128-byte line of x_q (eight rows
//     of one 16-k piece) is written by one CU into one L2; the transformed
//     row stays in registers between its maximum and its codes;
//   quant_pairs_kernel (m >= kQuantGroupMinRows, longer rows): two waves per
//     row, eight rows per workgroup, each wave holding part of its half;
//   quant_rows_kernel (smaller m): one workgroup of four waves per row, four
//     times the waves for batches too small to fill the GPU with groups.
// A wave transforms four 128-element blocks at a time (lane l holds elements
// 8 (l % 16) .. + 7 of block l / 16, the layout of fwht128_x8).  Where a row
// is not held it is transformed twice, once for its maximum and once to
// quantize: k has no upper bound and the second pass reads the row from
// cache.
// Measured on MI355X (k = 5120, n = 17408, K = 4, whole int8 linear): m = 4096
// 0.498 ms by groups against 0.512 by rows; m = 1000 0.191 against 0.181.
constexpr int kQuantGroupMinRows = 2048;
constexpr int kQuantGroupThreads = 1024;
constexpr int kQuantRowThreads = 256;

__device__ __forceinline__ void quant_load4(const uint16_t* __restrict__ xr,
                                           const uint16_t* __restrict__ suh, int nb, int b, int j,
                                           uint4& xv, uint4& sv) {
  const int bb = b < nb ? b : nb - 1;  // past the end: re-read the last block (unused)
  xv = *reinterpret_cast<const uint4*>(xr + bb * 128 + 8 * j);
  sv = *reinterpret_cast<const uint4*>(suh + bb * 128 + 8 * j);
}

__device__ __forceinline__ void quant_transform4(const uint4& xv, const uint4& sv, float (&v)[8]) {
  const uint32_t xw[4] = {xv.x, xv.y, xv.z, xv.w};
  const uint32_t sw[4] = {sv.x, sv.y, sv.z, sv.w};
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    v[2 * e] = h2f((uint16_t)(xw[e] & 0xFFFF)) * h2f((uint16_t)(sw[e] & 0xFFFF));
    v[2 * e + 1] = h2f((uint16_t)(xw[e] >> 16)) * h2f((uint16_t)(sw[e] >> 16));
  }
  fwht128_x8(v);
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] *= kInvSqrt128;
}

// Fragment-major destination of lane `lane`'s 8 bytes of row `row` (elements
// 128 b + 8 jj .. + 7, jj = lane % 16): 64-k block 2 b + jj / 8, lane group
// (jj % 8) / 2 of the fragment, byte 8 (jj % 2) of its 16.
struct QuantDst {
  int8_t* base;
  int jj;
  __device__ QuantDst(int8_t* xq, int64_t row, int k, int lane) {
    jj = lane & 15;
    base = xq + ((row >> 4) * (k / kGemmI8BK) * 64 + 16 * ((jj & 7) >> 1) + (row & 15)) * 16 + 8 * (jj & 1);
  }
  __device__ int8_t* at(int b) const { return base + (int64_t)(2 * b + (jj >> 3)) * kI8FragBytes; }
};

// Blocks b0 + lane / 16 for b0 = first, first + stride, ...: the maximum of
// |x'| (quantize = false) or the codes written with 127 / a (quantize = true).
template <bool QUANT>
__device__ __forceinline__ float quant_pass(const uint16_t* __restrict__ xr,
                                            const uint16_t* __restrict__ suh, int nb, int first,
                                            int stride, float inv, const QuantDst& dst) {
  const int lane = (int)lane_id();
  const int jj = lane & 15;
  float amax = 0.f;
  uint4 xv, sv;
  quant_load4(xr, suh, nb, first + (lane >> 4), jj, xv, sv);
  for (int b0 = first; b0 < nb; b0 += stride) {
    uint4 xn, sn;
    quant_load4(xr, suh, nb, b0 + stride + (lane >> 4), jj, xn, sn);
    const int b = b0 + (lane >> 4);
    float v[8];
    quant_transform4(xv, sv, v);
    if constexpr (QUANT) {
      uint32_t w[2] = {0u, 0u};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float qf = fminf(fmaxf(rintf(v[e] * inv), -127.f), 127.f);
        w[e >> 2] |= ((uint32_t)(int32_t)qf & 0xFFu) << (8 * (e & 3));
      }
      if (b < nb) *reinterpret_cast<uint2*>(dst.at(b)) = make_uint2(w[0], w[1]);
    } else if (b < nb) {
#pragma unroll
      for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(v[e]));
    }
    xv = xn;
    sv = sn;
  }
  return amax;
}

__device__ __forceinline__ void quant_zero_row(int nb, int first, int stride, const QuantDst& dst) {
  for (int b0 = first; b0 < nb; b0 += stride) {
    const int b = b0 + (int)(lane_id() >> 4);
    if (b < nb) *reinterpret_cast<uint2*>(dst.at(b)) = make_uint2(0u, 0u);
  }
}

// In every shape, rows m .. m_pad - 1 (up to the next multiple of 16) are
// written as zeros with scale 0, so every 16-row group of x_q is complete.

// Rows of at most 4 NP blocks, one wave per row of a 16-row group: the
// transformed row stays in registers between the maximum and the codes.
template <int NP>
__global__ __launch_bounds__(kQuantGroupThreads) void quant_groups_held_kernel(
    const uint16_t* __restrict__ x, int64_t ldx, const uint16_t* __restrict__ suh, int k, int64_t m,
    int8_t* __restrict__ xq, float* __restrict__ scale) {
  const int wave = (int)(threadIdx.x >> 6), lane = (int)(threadIdx.x & 63);
  const int64_t row = (int64_t)blockIdx.x * 16 + wave;
  const int nb = k / 128;
  const QuantDst dst(xq, row, k, lane);
  if (row >= m) {  // padding row of the last 16-row group (uniform per wave)
    quant_zero_row(nb, 0, 4, dst);
    if (lane == 0) scale[row] = 0.f;
    return;
  }
  const uint16_t* xr = x + row * ldx;
  const int jj = lane & 15;
  float v[NP][8];
  float amax = 0.f;
  uint4 xv, sv;
  quant_load4(xr, suh, nb, lane >> 4, jj, xv, sv);
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    if (4 * p < nb) {  // uniform
      uint4 xn, sn;
      quant_load4(xr, suh, nb, 4 * p + 4 + (lane >> 4), jj, xn, sn);
      quant_transform4(xv, sv, v[p]);
      if (4 * p + (lane >> 4) < nb) {
#pragma unroll
        for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(v[p][e]));
      }
      xv = xn;
      sv = sn;
    }
  }
#pragma unroll
  for (int msk = 32; msk >= 1; msk >>= 1) amax = fmaxf(amax, shfl_xor_f(amax, msk));
  const float a = amax;
  const float inv = a > 0.f ? 127.0f / a : 0.f;
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    const int b = 4 * p + (lane >> 4);
    if (4 * p < nb && b < nb) {
      uint32_t w[2] = {0u, 0u};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float qf = fminf(fmaxf(rintf(v[p][e] * inv), -127.f), 127.f);
        w[e >> 2] |= ((uint32_t)(int32_t)qf & 0xFFu) << (8 * (e & 3));
      }
      *reinterpret_cast<uint2*>(dst.at(b)) = make_uint2(w[0], w[1]);
    }
  }
  if (lane == 0) scale[row] = a / 127.0f;
}
constexpr int kQuantHeldPasses = 10;  // rows of up to 40 blocks (k <= 5120) held in registers

// Longer rows: two waves per row (wave h of a row takes the passes h, h + 2,
// ...), eight rows per workgroup (a 128-byte line of x_q still comes from one
// workgroup), each wave holding its first HP passes in registers and
// transforming only the rest twice; the pair's maxima meet in LDS.
template <int HP>
__global__ __launch_bounds__(kQuantGroupThreads) void quant_pairs_kernel(
    const uint16_t* __restrict__ x, int64_t ldx, const uint16_t* __restrict__ suh, int k, int64_t m,
    int8_t* __restrict__ xq, float* __restrict__ scale) {
  __shared__ float wmax[kQuantGroupThreads / 64];
  const int wave = (int)(threadIdx.x >> 6), lane = (int)(threadIdx.x & 63);
  const int64_t row = (int64_t)blockIdx.x * 8 + (wave >> 1);
  const int h = wave & 1;
  const int nb = k / 128;
  const int np = (nb + 3) >> 2;  // four-block passes of the row
  const int jj = lane & 15;
  const QuantDst dst(xq, row, k, lane);
  const bool pad = row >= m;  // padding row of the last 16-row group (uniform per wave)
  const uint16_t* xr = x + (pad ? 0 : row) * ldx;
  float v[HP][8];
  float amax = 0.f;
  if (!pad) {
#pragma unroll
    for (int i = 0; i < HP; ++i) {
      const int p = h + 2 * i;
      if (p < np) {  // uniform
        uint4 xv, sv;
        quant_load4(xr, suh, nb, 4 * p + (lane >> 4), jj, xv, sv);
        quant_transform4(xv, sv, v[i]);
        if (4 * p + (lane >> 4) < nb) {
#pragma unroll
          for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(v[i][e]));
        }
      }
    }
    for (int p = h + 2 * HP; p < np; p += 2) {
      uint4 xv, sv;
      quant_load4(xr, suh, nb, 4 * p + (lane >> 4), jj, xv, sv);
      float t[8];
      quant_transform4(xv, sv, t);
      if (4 * p + (lane >> 4) < nb) {
#pragma unroll
        for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(t[e]));
      }
    }
  }
#pragma unroll
  for (int msk = 32; msk >= 1; msk >>= 1) amax = fmaxf(amax, shfl_xor_f(amax, msk));
  if (lane == 0) wmax[wave] = amax;
  __syncthreads();
  const float a = fmaxf(wmax[wave & ~1], wmax[wave | 1]);
  if (pad) {
    quant_zero_row(nb, 4 * h, 8, dst);
    if (lane == 0 && h == 0) scale[row] = 0.f;
    return;
  }
  const float inv = a > 0.f ? 127.0f / a : 0.f;
  auto store = [&](const float (&t)[8], int b) {
    uint32_t w[2] = {0u, 0u};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float qf = fminf(fmaxf(rintf(t[e] * inv), -127.f), 127.f);
      w[e >> 2] |= ((uint32_t)(int32_t)qf & 0xFFu) << (8 * (e & 3));
    }
    if (b < nb) *reinterpret_cast<uint2*>(dst.at(b)) = make_uint2(w[0], w[1]);
  };
#pragma unroll
  for (int i = 0; i < HP; ++i) {
    const int p = h + 2 * i;
    if (p < np) store(v[i], 4 * p + (lane >> 4));
  }
  for (int p = h + 2 * HP; p < np; p += 2) {
    uint4 xv, sv;
    quant_load4(xr, suh, nb, 4 * p + (lane >> 4), jj, xv, sv);
    float t[8];
    quant_transform4(xv, sv, t);
    store(t, 4 * p + (lane >> 4));
  }
  if (lane == 0 && h == 0) scale[row] = a / 127.0f;
}
constexpr int kQuantPairHeld = 10;  // passes each wave of a pair holds

__global__ __launch_bounds__(kQuantRowThreads) void quant_rows_kernel(
    const uint16_t* __restrict__ x, int64_t ldx, const uint16_t* __restrict__ suh, int k, int64_t m,
    int8_t* __restrict__ xq, float* __restrict__ scale) {
  __shared__ float wmax[kQuantRowThreads / 64];
  const int64_t row = blockIdx.x;
  const int wave = (int)(threadIdx.x >> 6), lane = (int)(threadIdx.x & 63);
  const int nb = k / 128;
  const QuantDst dst(xq, row, k, lane);
  if (row >= m) {  // padding row (uniform per workgroup)
    quant_zero_row(nb, 4 * wave, 16, dst);
    if (threadIdx.x == 0) scale[row] = 0.f;
    return;
  }
  const uint16_t* xr = x + row * ldx;
  float amax = quant_pass<false>(xr, suh, nb, 4 * wave, 16, 0.f, dst);
#pragma unroll
  for (int msk = 32; msk >= 1; msk >>= 1) amax = fmaxf(amax, shfl_xor_f(amax, msk));
  if (lane == 0) wmax[wave] = amax;
  __syncthreads();
  const float a = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
  quant_pass<true>(xr, suh, nb, 4 * wave, 16, a > 0.f ? 127.0f / a : 0.f, dst);
  if (threadIdx.x == 0) scale[row] = a / 127.0f;
}

// ---------------------------------------------------------------------------
// int8 GEMM dispatch (dense tensor)
// ---------------------------------------------------------------------------
struct DenseGemmI8Res {
  const int8_t* a;      // fragment-major x_q
  const float* ascale;
  int64_t lda;          // bytes per 16-row group
  int m;
  int bm;
  int mt;   // row tiles
  int nbt;  // 128-column tiles
  const uint16_t* trellis;
  const uint16_t* svh;
  const uint16_t* bias;
  void* y;
  int64_t ldy;
  bool y_f32;
  // Workgroup -> (row tile, column tile), the XCD-aware order of the fp16
  // prefill GEMM: with a tile count that is a multiple of eight, the
  // workgroups of one XCD take one contiguous range of the tile order, which
  // walks two row tiles across all column tiles, so their int8 row panels
  // (2.6 MB for 256-row tiles at k = 5120) stay in that XCD's 4 MB L2.
  __device__ GemmI8Task task() const {
    const int total = mt * nbt;
    const int bid = (int)blockIdx.x;
    const int u = (total % 8 == 0) ? (bid % 8) * (total / 8) + bid / 8 : bid;
    constexpr int G = 2;
    const int grp = u / (G * nbt), within = u - grp * (G * nbt);
    const int g0 = grp * G;
    const int gs = (mt - g0) < G ? (mt - g0) : G;
    const int mtile = g0 + within % gs;
    GemmI8Task T;
    T.nb = within / gs;
    const int r0 = mtile * bm;
    T.valid = r0 < m;
    T.a = a + (int64_t)(r0 >> 4) * lda;  // r0 is a multiple of 16
    T.ascale = ascale + r0;
    T.lda = lda;
    T.rows = (m - r0) < bm ? (m - r0) : bm;
    T.trellis = trellis;
    T.svh = svh;
    T.bias = bias;
    T.y = y_f32 ? (void*)(static_cast<float*>(y) + (int64_t)r0 * ldy)
                : (void*)(static_cast<uint16_t*>(y) + (int64_t)r0 * ldy);
    T.ldy = ldy;
    return T;
  }
};

// Rows per tile.  At K = 7 and 8 the 256-row tile needs a few more than 256
// VGPRs and the compiler spills 16-28 bytes; measured at 4096 rows it is
// still faster than the 128-row tile.  (An eight-wave 512-row tile, which
// halves the decode per MFMA, measured 1-18 % slower than this once the
// activations were fragment-major.)
// Tile height by the rule of the fp16 GEMM (256 rows unless the grid would
// have fewer than kGemmI8MinGrid workgroups).  Measured on MI355X (K=4):
// 5120x5120 at m = 200 / 500 took 49 / 57 us against 68 / 73 with the
// m-only choice, 17408x5120 at m = 200 148 against 203 us, 5120x17408 at
// m = 300 84 against 106 us.
constexpr int64_t kGemmI8MinGrid = 128;
static int choose_bm_i8(int64_t m, int64_t nbt) {
  if (m <= 64) return 64;
  const int64_t t256 = (m + 255) / 256, t128 = (m + 127) / 128;
  if (t256 * nbt >= kGemmI8MinGrid) return (t256 <= 2 && t128 * 128 < t256 * 256) ? 128 : 256;
  return t128 * nbt >= kGemmI8MinGrid ? 128 : 64;
}

template <int K>
struct DenseGemmI8Run {
  static hipError_t run(const DenseGemmI8Res& r, int k, int n, hipStream_t s) {
    const dim3 grid(r.mt * r.nbt);
#define EXL3_GEMM_I8_LAUNCH(BM)                                                                    \
  do {                                                                                             \
    if (r.y_f32)                                                                                   \
      hipLaunchKernelGGL((gemm_i8_kernel<K, BM, true, DenseGemmI8Res>), grid, dim3(kGemmThreads), 0, s, r, k, n); \
    else                                                                                           \
      hipLaunchKernelGGL((gemm_i8_kernel<K, BM, false, DenseGemmI8Res>), grid, dim3(kGemmThreads), 0, s, r, k, n); \
  } while (0)
    if (r.bm == 256) EXL3_GEMM_I8_LAUNCH(256);
    else if (r.bm == 128) EXL3_GEMM_I8_LAUNCH(128);
    else EXL3_GEMM_I8_LAUNCH(64);
#undef EXL3_GEMM_I8_LAUNCH
    return hipGetLastError();
  }
};

// Workspace: x_q (int8, fragment-major, m rounded up to 16 rows) then the row
// scales (fp32, same rows), each on a 256-byte boundary.
static int64_t i8_rows(int64_t m) { return (m + 15) & ~(int64_t)15; }
static size_t i8_scale_offset(int k, int64_t m) { return ((size_t)i8_rows(m) * k + 255) & ~(size_t)255; }

size_t linear_int8_workspace(int k, int64_t m) {
  return i8_scale_offset(k, m) + (((size_t)i8_rows(m) * sizeof(float) + 255) & ~(size_t)255);
}

int64_t linear_int8_max_workgroups(int k, int n, int64_t m) {
  const int64_t quant = m < kQuantGroupMinRows ? i8_rows(m)
                        : (k <= 4 * 128 * kQuantHeldPasses ? i8_rows(m) / 16 : i8_rows(m) / 8);
  const int64_t bm = choose_bm_i8(m, n / kGemmBN);
  const int64_t gemm = (m + bm - 1) / bm * (n / kGemmBN);
  return quant > gemm ? quant : gemm;
}

hipError_t launch_linear_int8(const uint16_t* trellis, const uint16_t* suh, const uint16_t* svh,
                              const uint16_t* bias, int k, int n, int bits, const uint16_t* x,
                              int64_t m, int64_t ldx, void* y, int64_t ldy, bool y_f32, void* ws,
                              hipStream_t s) {
  unsigned char* base = static_cast<unsigned char*>(ws);
  int8_t* xq = reinterpret_cast<int8_t*>(base);
  float* sc = reinterpret_cast<float*>(base + i8_scale_offset(k, m));
  if (m >= kQuantGroupMinRows && k <= 4 * 128 * kQuantHeldPasses)
    hipLaunchKernelGGL(quant_groups_held_kernel<kQuantHeldPasses>, dim3((unsigned)(i8_rows(m) / 16)),
                       dim3(kQuantGroupThreads), 0, s, x, ldx, suh, k, m, xq, sc);
  else if (m >= kQuantGroupMinRows)
    hipLaunchKernelGGL(quant_pairs_kernel<kQuantPairHeld>, dim3((unsigned)(i8_rows(m) / 8)),
                       dim3(kQuantGroupThreads), 0, s, x, ldx, suh, k, m, xq, sc);
  else
    hipLaunchKernelGGL(quant_rows_kernel, dim3((unsigned)i8_rows(m)), dim3(kQuantRowThreads), 0, s, x, ldx,
                       suh, k, m, xq, sc);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int bm = choose_bm_i8(m, n / kGemmBN);
  DenseGemmI8Res r{xq, sc, (int64_t)16 * k, (int)m, bm, (int)((m + bm - 1) / bm), n / kGemmBN, trellis,
                   svh, bias, y, ldy, y_f32};
  return dispatch_bits<DenseGemmI8Run>(bits, r, k, n, s);
}

// ---------------------------------------------------------------------------
// int8 weights of a whole tensor
// ---------------------------------------------------------------------------
template <int K>
__global__ __launch_bounds__(256) void reconstruct_i8_kernel(const uint16_t* __restrict__ trellis,
                                                             int8_t* __restrict__ out, int nt,
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
  uint32_t B[K + 1];
#pragma unroll
  for (int i = 0; i < K; ++i) B[i] = stream_dword(D[i]);
  B[K] = spill_from_next(D[0]);
  uint32_t r0[4], r1[4];  // rows 2p and 2p + 1, four columns per dword
  static_for<0, 4>([&](auto cc) {
    constexpr int c = 4 * decltype(cc)::value;
    r0[decltype(cc)::value] = pack_i8x4(state_i8<K, K * c>(B), state_i8<K, K * (c + 1)>(B),
                                        state_i8<K, K * (c + 2)>(B), state_i8<K, K * (c + 3)>(B));
    r1[decltype(cc)::value] =
        pack_i8x4(state_i8<K, K * (16 + c)>(B), state_i8<K, K * (17 + c)>(B),
                  state_i8<K, K * (18 + c)>(B), state_i8<K, K * (19 + c)>(B));
  });
  int8_t* o0 = out + (16 * a + 2 * p) * (int64_t)n + 16 * b;
  *reinterpret_cast<uint4*>(o0) = make_uint4(r0[0], r0[1], r0[2], r0[3]);
  *reinterpret_cast<uint4*>(o0 + n) = make_uint4(r1[0], r1[1], r1[2], r1[3]);
}

template <int K>
struct ReconstructI8Run {
  static hipError_t run(const uint16_t* trellis, int8_t* out, int k, int n, hipStream_t s) {
    const int64_t tiles = (int64_t)(k / 16) * (n / 16);
    const unsigned blocks = (unsigned)((tiles * 8 + 255) / 256);
    hipLaunchKernelGGL(reconstruct_i8_kernel<K>, dim3(blocks), dim3(256), 0, s, trellis, out, n / 16,
                       tiles, n);
    return hipGetLastError();
  }
};

hipError_t launch_reconstruct_int8(const uint16_t* trellis, int8_t* out, int k, int n, int bits,
                                   hipStream_t s) {
  return dispatch_bits<ReconstructI8Run>(bits, trellis, out, k, n, s);
}

}  // namespace exl3
