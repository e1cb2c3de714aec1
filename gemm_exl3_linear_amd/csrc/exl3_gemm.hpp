// Fused decode + MFMA GEMM kernel template (the prefill regime, m > 16),
// shared by the dense linear and the grouped experts.
//
// One workgroup computes a BM x 128 output tile over the full k range:
//   per k step of 64 rows  - the A panel (activations already in the
//                            Hadamard domain, fp16) is staged into LDS;
//                          - the 4 x 8 trellis tiles of the step are decoded
//                            in registers (one row pair per thread, the same
//                            routine as every other kernel) and written to LDS
//                            as k-contiguous fp16 columns;
//                          - four waves run MFMA 16x16x16 f16 with fp32
//                            accumulation on their BM/4 x 128 slice.
//   epilogue               - the 128 output columns are exactly one Hadamard
//                            block: the output transform runs on the
//                            accumulators (3 stages in registers, 4 across
//                            lanes), then svh, bias and the cast.
// The next step's global loads are issued before the current step's MFMAs.
#pragma once

#include "exl3_device.hpp"

namespace exl3 {

struct GemmTask {
  bool valid;
  const uint16_t* a;        // fp16 rows of x' for this tile, row 0
  int64_t lda;
  int rows;                 // valid rows in this tile (<= BM)
  const uint16_t* trellis;  // tensor base [k/16][n/16][16K]
  const uint16_t* svh;      // fp16 [n]
  const uint16_t* bias;     // fp16 [n] or nullptr
  void* y;                  // output row 0 of this tile
  int64_t ldy;
};

constexpr int kGemmBK = 64;                    // k rows per step (4 tiles)
constexpr int kGemmRowDw = 36;                 // LDS row stride in dwords (64 halves + pad)
constexpr int kGemmBTileDw = 16 * kGemmRowDw + 8;  // per n-tile block of B (bank spread)

template <int K, int BM, bool Y_F32, class R>
__global__ __launch_bounds__(256) void gemm_kernel(R r, int k, int n) {
  constexpr int MI = BM / 64;          // 16-row subtiles per wave
  constexpr int AQ = BM / 32;          // uint4 A chunks per thread per step
  __shared__ __align__(16) uint32_t As[BM * kGemmRowDw];
  __shared__ __align__(16) uint32_t Bs[8 * kGemmBTileDw];

  const GemmTask T = r.task(blockIdx.y, blockIdx.z);
  if (!T.valid) return;
  const int nb = blockIdx.x;
  const int nt = n >> 4;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int g = lane >> 4, j = lane & 15;

  // decode role of this thread: k tile ktl of the step, n tile t, row pair p
  const int ktl = tid >> 6, t = (tid >> 3) & 7, p = tid & 7;
  const uint32_t* tb = reinterpret_cast<const uint32_t*>(T.trellis) +
                       ((int64_t)ktl * nt + nb * 8 + t) * (8 * K) + K * p;
  const int64_t step_dw = (int64_t)4 * nt * (8 * K);

  float4_t acc[MI][8];
#pragma unroll
  for (int mi = 0; mi < MI; ++mi)
#pragma unroll
    for (int q = 0; q < 8; ++q) acc[mi][q] = float4_t{0.f, 0.f, 0.f, 0.f};

  uint4 ra[AQ];
  uint32_t rt[K];
  auto load_step = [&](int ks) {
#pragma unroll
    for (int q = 0; q < AQ; ++q) {
      const int idx = tid + 256 * q;
      const int row = idx >> 3, ch = idx & 7;
      if (row < T.rows)
        ra[q] = *reinterpret_cast<const uint4*>(T.a + (int64_t)row * T.lda + ks * kGemmBK + ch * 8);
      else
        ra[q] = make_uint4(0, 0, 0, 0);
    }
    load_rowpair<K>(tb + ks * step_dw, rt);
  };

  const int nsteps = k / kGemmBK;
  load_step(0);
  for (int ks = 0; ks < nsteps; ++ks) {
#pragma unroll
    for (int q = 0; q < AQ; ++q) {
      const int idx = tid + 256 * q;
      const int row = idx >> 3, ch = idx & 7;
      *reinterpret_cast<uint4*>(As + row * kGemmRowDw + ch * 4) = ra[q];
    }
    {
      const uint32_t spill = spill_from_next(rt[0]);
      uint32_t wp[16];
      decode_rowpair<K>(rt, spill, wp);
      uint32_t* bdst = Bs + t * kGemmBTileDw + 8 * ktl + p;
#pragma unroll
      for (int c = 0; c < 16; ++c) bdst[c * kGemmRowDw] = wp[c];
    }
    __syncthreads();
    if (ks + 1 < nsteps) load_step(ks + 1);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      half4_t av[MI];
#pragma unroll
      for (int mi = 0; mi < MI; ++mi) {
        const int row = wave * (BM / 4) + 16 * mi + j;
        av[mi] = *reinterpret_cast<const half4_t*>(As + row * kGemmRowDw + 8 * kk + 2 * g);
      }
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const half4_t bv =
            *reinterpret_cast<const half4_t*>(Bs + q * kGemmBTileDw + j * kGemmRowDw + 8 * kk + 2 * g);
#pragma unroll
        for (int mi = 0; mi < MI; ++mi)
          acc[mi][q] = __builtin_amdgcn_mfma_f32_16x16x16f16(av[mi], bv, acc[mi][q], 0, 0, 0);
      }
    }
    __syncthreads();
  }

  // epilogue: output Hadamard over the 128 columns, svh, bias, cast
  const int col0 = nb * 128;
#pragma unroll
  for (int mi = 0; mi < MI; ++mi) {
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      float v[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) v[q] = acc[mi][q][rr];
#pragma unroll
      for (int h = 1; h < 8; h <<= 1)
#pragma unroll
        for (int q = 0; q < 8; ++q)
          if ((q & h) == 0) {
            const float u0 = v[q], u1 = v[q + h];
            v[q] = u0 + u1;
            v[q + h] = u0 - u1;
          }
#pragma unroll
      for (int msk = 1; msk < 16; msk <<= 1) {
        const bool upper = (j & msk) != 0;
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const float pv = shfl_xor_f(v[q], msk);
          v[q] = upper ? (pv - v[q]) : (v[q] + pv);
        }
      }
      const int row = wave * (BM / 4) + 16 * mi + 4 * g + rr;
      if (row < T.rows) {
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const int col = col0 + 16 * q + j;
          float o = v[q] * kInvSqrt128 * h2f(T.svh[col]);
          if (T.bias) o += h2f(T.bias[col]);
          if constexpr (Y_F32)
            static_cast<float*>(T.y)[(int64_t)row * T.ldy + col] = o;
          else
            static_cast<uint16_t*>(T.y)[(int64_t)row * T.ldy + col] = f2h(o);
        }
      }
    }
  }
}

}  // namespace exl3
