// Fused decode + int8 MFMA GEMM (the int8 prefill: exl3xpu README, "Prefill:
// int8 linears and oneDNN fused attention").  Activations arrive as int8 rows
// with one fp32 scale per row (the input transform quantizes them); weights
// are decoded straight to int8 with the static scale 127 / 3.453125
// (state_i8); the product accumulates exactly in int32 and the epilogue
// applies both scales, the output transform, svh, bias and the cast.
//
// Same workgroup structure as gemm_kernel (exl3_gemm.hpp): four waves, a
// BM x 128 output tile over the full k range, wave w owning BM/4 rows and all
// 128 columns; two workgroups per CU.  Differences:
//   - a k step is 64 rows (four trellis tiles), the depth of one
//     v_mfma_i32_16x16x64_i8, gfx950's full-rate int8 contraction (twice the
//     fp16 rate);
//   - every thread decodes two consecutive row pairs of one tile (rows
//     4 p2 .. 4 p2 + 3) for eight columns, so each column's four k values
//     pack into one dword and go to LDS in one 4-byte store; the decoded
//     stage is 128 columns x 64 k bytes, read as one 16-byte B fragment per
//     MFMA, in the same swizzled chunk layout as the fp16 stage;
//   - the A fragment is 16 int8 activations straight from global memory,
//     from the fragment-major layout the input transform writes.
#pragma once

#include "exl3_device.hpp"
#include "exl3_gemm.hpp"

namespace exl3 {

constexpr int kGemmI8BK = 64;  // k rows per step: the depth of one int8 MFMA

// Fragment-major int8 activations: for every group of 16 rows and every 64
// k, the MFMA A operand in lane order, lane (g, j) = 16 g + j holding the 16
// bytes of row j at k 16 g .. 16 g + 15:
//   x_q[16 G + j][64 B + 16 g + e] at byte ((G * (k / 64) + B) * 64 + 16 g + j) * 16 + e.
// One fragment is one contiguous kilobyte, so the GEMM reads it with fully
// used 128-byte lines (a row-major layout gives each load 16 rows x 64
// bytes, half-used lines, and measured about twice the time for the loads).
constexpr int kI8FragBytes = 1024;

typedef int32_t i32x4_t __attribute__((ext_vector_type(4)));

// 3.453125 / 127: the weight step of the int8 decode
constexpr float kI8WeightStep = 3.453125f / 127.0f;

struct GemmI8Task {
  bool valid;
  int nb;                   // 128-column tile
  const int8_t* a;          // x_q of this tile, fragment-major (first 16-row group)
  const float* ascale;      // fp32 row scales (max |x'| / 127), row 0
  int64_t lda;              // bytes per 16-row group of a (16 k)
  int rows;                 // valid rows in this tile (<= BM)
  const uint16_t* trellis;  // tensor base [k/16][n/16][16K]
  const uint16_t* svh;      // fp16 [n]
  const uint16_t* bias;     // fp16 [n] or nullptr
  void* y;                  // output row 0 of this tile
  int64_t ldy;
};

// First dword (stream order) of the next lane in a group of four, cyclic
// (DPP quad permutation 1, 2, 3, 0).  All four lanes must be active.
__device__ __forceinline__ uint32_t spill_from_next4(uint32_t my_first_le) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)stream_dword(my_first_le), 0x39, 0xF, 0xF, false);
}

// Epilogue of a wave's rows r0 .. r0 + 16 MI - 1 and the tile's 128 columns:
// int32 -> fp32, output Hadamard over the 128 columns, then both scales with
// svh, bias and the cast.
template <int MI, bool Y_F32>
__device__ __forceinline__ void gemm_i8_epilogue(const GemmI8Task& T,
                                                 const i32x4_t (&acc)[MI][8], int r0,
                                                 int col0, int j, int g) {
  float sv[8], bv[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    sv[q] = kInvSqrt128 * kI8WeightStep * h2f(T.svh[col0 + 16 * q + j]);
    bv[q] = T.bias ? h2f(T.bias[col0 + 16 * q + j]) : 0.f;
  }
#pragma unroll
  for (int mi = 0; mi < MI; ++mi) {
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const int row = r0 + 16 * mi + 4 * g + rr;
      float v[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) v[q] = (float)acc[mi][q][rr];
      gemm_col_fwht(v);
      if (row < T.rows) {
        const float rs = T.ascale[row];
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const int col = col0 + 16 * q + j;
          float o = v[q] * rs * sv[q];
          if (T.bias) o += bv[q];
          if constexpr (Y_F32)
            static_cast<float*>(T.y)[(int64_t)row * T.ldy + col] = o;
          else
            static_cast<uint16_t*>(T.y)[(int64_t)row * T.ldy + col] = f2h(o);
        }
      }
    }
  }
}

template <int K, int BM, bool Y_F32, class R>
__global__ __launch_bounds__(kGemmThreads, 2) void gemm_i8_kernel(R r, int k, int n) {
  constexpr int WM = BM / 4;  // rows per wave tile
  constexpr int MI = WM / 16; // 16-row MFMA tiles per wave
  static_assert(MI >= 1, "BM must be a multiple of 64");
  __shared__ uint4 bst0[kGemmBN * 4], bst1[kGemmBN * 4];

  const GemmI8Task T = r.task();
  if (!T.valid) return;
  const int nt16 = n >> 4;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int g = lane >> 4, j = lane & 15;
  const int col0 = T.nb * kGemmBN;

  // decode role: rows 4 p2 .. 4 p2 + 3 (row pairs 2 p2 and 2 p2 + 1) of k
  // tile kt of the step, n tile t, column half h (uniform per wave)
  const int p2 = tid & 3, kt = (tid >> 2) & 3, t = (tid >> 4) & 7, h = tid >> 7;
  constexpr int K2 = 2 * K;  // dwords of two row pairs
  constexpr uint32_t kTileBytes = 32 * K;
  const __amdgpu_buffer_rsrc_t t_rs =
      make_rsrc(T.trellis, (uint32_t)((uint64_t)(k >> 4) * nt16 * kTileBytes));
  const uint32_t t_voff = (uint32_t)(kt * nt16 + T.nb * 8 + t) * kTileBytes + 8 * K * p2;
  const uint32_t t_step = 4u * (uint32_t)nt16 * kTileBytes;
  // LDS dword of each decoded column: dword p2 (k 4 p2 .. 4 p2 + 3) of chunk
  // kt (k 16 kt .. 16 kt + 15) of columns 16 t + 8 h + c
  int bw_dw[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) bw_dw[c] = gemm_b_chunk(16 * t + 8 * h + c, kt) * 4 + p2;
  // A fragment of rows 16 mi .. 16 mi + 15 at the step's 64 k: one
  // contiguous kilobyte of the fragment-major x_q, 16 bytes per lane; row
  // groups past the tile's rows read as zero (outside the descriptor)
  const __amdgpu_buffer_rsrc_t a_rs = make_rsrc(T.a, (uint32_t)((uint64_t)((T.rows + 15) >> 4) * T.lda));
  uint32_t a_voff[MI];
#pragma unroll
  for (int mi = 0; mi < MI; ++mi)
    a_voff[mi] = (uint32_t)((int64_t)(wave * MI + mi) * T.lda + 16 * lane);
  // B fragment: chunk g (k 16 g .. 16 g + 15) of column 16 q + j
  int br_ch[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) br_ch[q] = gemm_b_chunk(16 * q + j, g);

  typedef i32x4_t i32x4;
  i32x4 acc[MI][8];
#pragma unroll
  for (int mi = 0; mi < MI; ++mi)
#pragma unroll
    for (int q = 0; q < 8; ++q) acc[mi][q] = i32x4{0, 0, 0, 0};

  const int nsteps = k / kGemmI8BK;  // k is a multiple of 128: nsteps is even
  i32x4 ra[2][MI];
  uint32_t rt[2][K2];
  auto load_a = [&](int set, int ks) {
    ks = ks < nsteps ? ks : nsteps - 1;  // past the end: re-read the last step (unused)
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
      ra[set][mi] = __builtin_bit_cast(
          i32x4, __builtin_amdgcn_raw_buffer_load_b128(a_rs, (int)a_voff[mi], ks * kI8FragBytes, 0));
  };
  auto load_t = [&](int set, int ks) {
    ks = ks < nsteps ? ks : nsteps - 1;
    load_rowpair_buf<K2>(t_rs, t_voff, (uint32_t)ks * t_step, rt[set]);
  };
  // eight columns 8 H .. 8 H + 7 of this thread's four rows, each column's
  // four int8 weights packed (row 4 p2 in byte 0)
  auto decode8 = [&](const uint32_t (&B)[K2 + 1], uint32_t (&wv)[8], auto hc) {
    constexpr int H = decltype(hc)::value;
    const uint32_t(&B0)[K + 1] = *reinterpret_cast<const uint32_t(*)[K + 1]>(&B[0]);
    const uint32_t(&B1)[K + 1] = *reinterpret_cast<const uint32_t(*)[K + 1]>(&B[K]);
    static_for<0, 8>([&](auto cc) {
      constexpr int c = 8 * H + decltype(cc)::value;
      const uint32_t w0 = state_i8<K, K * c>(B0);
      const uint32_t w1 = state_i8<K, K * (16 + c)>(B0);
      const uint32_t w2 = state_i8<K, K * c>(B1);
      const uint32_t w3 = state_i8<K, K * (16 + c)>(B1);
      wv[decltype(cc)::value] = pack_i8x4(w0, w1, w2, w3);
    });
  };
  auto stream_of = [&](int tset, uint32_t (&B)[K2 + 1]) {
#pragma unroll
    for (int i = 0; i < K2; ++i) B[i] = stream_dword(rt[tset][i]);
    B[K2] = spill_from_next4(rt[tset][0]);
  };
  // One step: the MFMAs on stage `cur` with A set `aset`, the decode of the
  // next step's trellis (set `tset`) into stage `nxt`; the schedule is fixed
  // as in gemm_kernel (fragment reads, then each MFMA followed by decode
  // instructions, then the decoded stores and the next loads).
  auto step = [&](const uint4* cur, uint4* nxt, int aset, int tset, auto hc) {
    uint32_t B[K2 + 1];
    stream_of(tset, B);
    i32x4 bv[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) bv[q] = __builtin_bit_cast(i32x4, cur[br_ch[q]]);
    uint32_t wv[8];
    decode8(B, wv, hc);
#pragma unroll
    for (int q = 0; q < 8; ++q)
#pragma unroll
      for (int mi = 0; mi < MI; ++mi)
        acc[mi][q] = __builtin_amdgcn_mfma_i32_16x16x64_i8(ra[aset][mi], bv[q], acc[mi][q], 0, 0, 0);
    uint32_t* nd = reinterpret_cast<uint32_t*>(nxt);
#pragma unroll
    for (int c = 0; c < 8; ++c) nd[bw_dw[c]] = wv[c];
    __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 8, 0);
    static_for<0, 8 * MI>([&](auto) {
      __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
      __builtin_amdgcn_sched_group_barrier(kSchedValu, 144 / (8 * MI) + 1, 0);
    });
    __builtin_amdgcn_sched_group_barrier(kSchedDsWrite, 8, 0);
    __builtin_amdgcn_sched_group_barrier(kSchedVmemRead, MI + (K2 + 3) / 4, 0);
  };

  auto run = [&](auto hc) {
    // prologue: step 0 decoded into stage 0; A of steps 0, 1 and trellis of
    // steps 1, 2 in flight, issued in the order that leaves the loop's entry
    // with as many later loads behind each register set as its back edge (the
    // loop's wait counts are the minimum over both edges; see gemm_tile)
    load_t(0, 0);
    load_t(1, 1);
    __builtin_amdgcn_sched_barrier(0);
    {
      uint32_t B[K2 + 1], wv[8];
      stream_of(0, B);
      decode8(B, wv, hc);
      uint32_t* nd = reinterpret_cast<uint32_t*>(bst0);
#pragma unroll
      for (int c = 0; c < 8; ++c) nd[bw_dw[c]] = wv[c];
    }
    __builtin_amdgcn_sched_barrier(0);
    load_a(0, 0);
    __builtin_amdgcn_sched_barrier(0);
    load_a(1, 1);
    __builtin_amdgcn_sched_barrier(0);
    load_t(0, 2);
    __syncthreads();
    __builtin_amdgcn_sched_barrier(0);
    for (int ks = 0; ks < nsteps; ks += 2) {
      step(bst0, bst1, 0, 1, hc);
      load_a(0, ks + 2);
      load_t(1, ks + 3);
      __syncthreads();
      __builtin_amdgcn_sched_barrier(0);
      step(bst1, bst0, 1, 0, hc);
      load_a(1, ks + 3);
      load_t(0, ks + 4);
      __syncthreads();
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  if (h == 0)
    run(IntC<0>{});
  else
    run(IntC<1>{});

  gemm_i8_epilogue<MI, Y_F32>(T, acc, wave * WM, col0, j, g);
}


}  // namespace exl3
