// Fused decode + MFMA GEMM kernel template (the prefill regime, m > 16),
// shared by the dense linear and the grouped experts.
//
// One workgroup (four waves) computes a BM x 128 output tile over the full k
// range: wave w owns the 16-row groups w, w + 4, w + 8, ... (BM/64 of them)
// and all 128 columns, one whole Hadamard block.  Interleaved groups keep the
// waves' shares of a short tile even: a wave runs MFMAs only for its groups
// that hold valid rows (for every group count when R::kFineSkip, else all or
// none), while all four decode.  Two workgroups share each CU (two waves per SIMD: a
// single wave cannot issue v_mfma_f32_16x16x32_f16 back to back), and being
// independent they fill each other's barrier and memory stalls.
//   per k step of 32 rows  - each wave loads its A fragments (activations
//                            already in the Hadamard domain, fp16) straight
//                            from global memory into registers, in the MFMA
//                            operand layout (no LDS for A);
//                          - the 2 x 8 trellis tiles of the next step are
//                            decoded in registers, half a row pair per thread
//                            (the routine every other kernel uses), and
//                            written to the other LDS stage column-major (k
//                            contiguous), so each B fragment is one 16-byte
//                            LDS read;
//                          - v_mfma_f32_16x16x32_f16 (gfx950's full-rate fp16
//                            contraction) with fp32 accumulation, the decode
//                            interleaved with the MFMAs.
//   epilogue               - the output transform runs on the accumulators
//                            (3 stages in registers, 4 across lanes), then
//                            svh, bias and the cast.
// One barrier per step; the loads of the next steps are in flight meanwhile.
// R::kGateUp (routed experts' gate and up): the k loop runs twice over the
// same rows, for gate and then for up; the transformed gate block waits in
// LDS as fp16, and the epilogue forms silu(g) u and the next projection's
// input transform of the block instead of storing the product.
#pragma once

#include "exl3_device.hpp"

namespace exl3 {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));

struct GemmTask {
  bool valid;
  int nb;                   // 128-column tile
  const uint16_t* a;        // fp16 rows of x' for this tile, row 0
  int64_t lda;
  int rows;                 // valid rows in this tile (<= BM)
  const uint16_t* trellis;  // tensor base [k/16][n/16][16K]
  const uint16_t* svh;      // fp16 [n]
  const uint16_t* bias;     // fp16 [n] or nullptr
  void* y;                  // output row 0 of this tile
  int64_t ldy;
  // R::kGateUp only: the second (up) projection of the same rows and shape,
  // and the sign vector of the next layer's input transform
  const uint16_t* a2;
  const uint16_t* trellis2;
  const uint16_t* svh2;
  const uint16_t* snext;    // fp16 [n]
  int bits;                 // width of the tensors, read when the kernel's K is 0
};

__device__ __forceinline__ float silu_f(float z) { return z / (1.0f + __expf(-z)); }

constexpr int kGemmBN = 128;        // columns per workgroup tile (one Hadamard block)
constexpr int kGemmBK = 32;         // k rows per step (two trellis tiles)
constexpr int kGemmThreads = 256;   // four waves, each BM/4 rows x 128 columns

// Fragment-major fp16 activations (the dense prefill's x'): for every group of
// 16 rows and every 32 k, the MFMA A operand in lane order, lane (g, j) =
// 16 g + j holding the 8 elements of row j at k 8 g .. 8 g + 7:
//   x'[16 G + j][32 B + 8 g + e] at element ((G * (k / 32) + B) * 64 + 16 g + j) * 8 + e.
// One fragment is one contiguous kilobyte, read with fully used 128-byte
// lines (row-major, each load covers 16 rows x 64 bytes, half of each line).
constexpr int kGemmFragBytes = 1024;

// Decoded-weight stage: 128 columns x 32 k (fp16) as 512 chunks of 16 bytes
// (four k-pairs of one column each).  Chunk gc of the 16 columns q = col / 16
// fill the 16 consecutive chunks 16 (4 q + gc) .. + 15 (256 bytes, one pass
// over 64 LDS banks), column col % 16 at position (col % 16) ^ (gc + 4 (q % 4)).
// The MFMA fragment reads (sixteen consecutive columns of one gc) then cover
// all 16 positions, and each half of them (eight columns) the eight positions
// of one 128-byte line of 32 banks, so a 16-byte read is conflict free in
// passes of 16 lanes over 64 banks and of 8 lanes over 32; the decoder's
// 4-byte writes (64 lanes: the four gc of four column groups q, one column)
// touch 16 distinct positions, and each 32 lanes (two column groups) eight
// distinct positions modulo 8.
__device__ __forceinline__ int gemm_b_chunk(int col, int gc) {
  const int q = col >> 4;
  return 16 * (4 * q + gc) + ((col & 15) ^ (gc | ((q & 3) << 2)));
}

// The 128-point transform across a wave's 128 columns: v[q] holds column
// 16 q + j (j = lane % 16) of one row; three stages over q in registers, four
// across the lanes of each 16-lane group (unnormalised).
__device__ __forceinline__ void gemm_col_fwht(float (&v)[8]) {
  const uint32_t j = lane_id() & 15u;
#pragma unroll
  for (int sd = 1; sd < 8; sd <<= 1)
#pragma unroll
    for (int q = 0; q < 8; ++q)
      if ((q & sd) == 0) {
        const float u0 = v[q], u1 = v[q + sd];
        v[q] = u0 + u1;
        v[q + sd] = u0 - u1;
      }
  static_for_pow2<1, 16>([&](auto mc) {
    constexpr int msk = decltype(mc)::value;
    const bool upper = (j & (uint32_t)msk) != 0;
#pragma unroll
    for (int q = 0; q < 8; ++q) v[q] = bfly(v[q], xor_partner<msk>(v[q]), upper);
  });
}

// __builtin_amdgcn_sched_group_barrier instruction classes
constexpr int kSchedValu = 0x002, kSchedMfma = 0x008, kSchedVmemRead = 0x020,
              kSchedDsRead = 0x100, kSchedDsWrite = 0x200;

template <int V>
struct IntC {
  static constexpr int value = V;
};

template <int I, int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(IntC<I>{});
    static_for<I + 1, N>(f);
  }
}

// The workgroup's tile at width K; LDS comes from the kernel (two decoded
// stages, and the gate results between the passes of R::kGateUp).
template <int K, int BM, bool Y_F32, class R>
__device__ __forceinline__ void gemm_tile(const R& r, const GemmTask& T, int k, int n, uint4* bst0,
                                          uint4* bst1, uint2* gst) {
  constexpr int WM = BM / 4;           // rows per wave tile
  constexpr int MI = WM / 16;          // 16-row MFMA tiles per wave
  static_assert(MI >= 1, "BM must be a multiple of 64");
  const int nt16 = n >> 4;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int g = lane >> 4, j = lane & 15;
  const int wm = wave, wn = 0;
  const int col0 = T.nb * kGemmBN;

  // decode role: row pair p, k tile kt of the step, n tile t of the workgroup
  // tile, column half h (uniform per wave: waves 0-1 decode columns 0-7 of
  // each n tile, waves 2-3 columns 8-15)
  const int p = tid & 7, kt = (tid >> 3) & 1, t = (tid >> 4) & 7, h = tid >> 7;
  constexpr uint32_t kTileBytes = 32 * K;
  const uint32_t t_bytes = (uint32_t)((uint64_t)(k >> 4) * nt16 * kTileBytes);
  __amdgpu_buffer_rsrc_t t_rs = make_rsrc(T.trellis, t_bytes);
  const uint32_t t_voff = (uint32_t)(kt * nt16 + T.nb * 8 + t) * kTileBytes + 4 * K * p;
  const uint32_t t_step = 2u * (uint32_t)nt16 * kTileBytes;
  // LDS dword of each decoded k-pair this thread writes (k-pair 8 kt + p of
  // columns 16 t + 8 h + c)
  const int kp = 8 * kt + p;
  int bw_dw[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) bw_dw[c] = gemm_b_chunk(16 * t + 8 * h + c, kp >> 2) * 4 + (kp & 3);
  // A fragment rows; rows at or past T.rows read as zero (outside the range)
  // R::kAFrag: x' is fragment-major (see kGemmFragBytes), T.lda elements per
  // 16-row group, and a fragment is one contiguous kilobyte; otherwise x' is
  // row-major, T.lda elements per row
  // (group 4 mi + wm of the tile is this wave's mi-th)
  uint32_t a_bytes, a_voff[MI];
  if constexpr (R::kAFrag) {
    a_bytes = (uint32_t)((uint64_t)((T.rows + 15) >> 4) * T.lda * 2);
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
      a_voff[mi] = (uint32_t)((int64_t)(4 * mi + wm) * T.lda * 2 + 16 * lane);
  } else {
    a_bytes = (uint32_t)((uint64_t)T.rows * T.lda * 2);
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
      a_voff[mi] = (uint32_t)(((int64_t)(16 * (4 * mi + wm) + j) * T.lda + 8 * g) * 2);
  }
  __amdgpu_buffer_rsrc_t a_rs = make_rsrc(T.a, a_bytes);
  constexpr int kAStep = R::kAFrag ? kGemmFragBytes : kGemmBK * 2;  // bytes per k step
  // B fragment chunks this lane reads (column 128 wn + 16 q + j, chunk g)
  int br_ch[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) br_ch[q] = gemm_b_chunk(128 * wn + 16 * q + j, g);

  float4_t acc[MI][8];
#pragma unroll
  for (int mi = 0; mi < MI; ++mi)
#pragma unroll
    for (int q = 0; q < 8; ++q) acc[mi][q] = float4_t{0.f, 0.f, 0.f, 0.f};

  const int nsteps = k / kGemmBK;  // k is a multiple of 128: nsteps is a multiple of 4
  // two register sets: A fragments of step s and trellis words of step s live in set s % 2
  half8_t ra[2][MI];
  uint32_t rt[2][K];
  auto load_t = [&](int set, int ks) {
    ks = ks < nsteps ? ks : nsteps - 1;
    load_rowpair_buf<K>(t_rs, t_voff, (uint32_t)ks * t_step, rt[set]);
  };
  // decode the eight columns 8 H .. 8 H + 7 of this thread's row pair from
  // the stream dwords B (the register set of the next step)
  auto decode8 = [&](const uint32_t (&B)[K + 1], uint32_t (&wv)[8], auto hc) {
    constexpr int H = decltype(hc)::value;
    uint32_t wp[16];
    static_for<0, 8>([&](auto cc) {
      constexpr int c = decltype(cc)::value;
      decode_column<K, 8 * H + c, false>(B, kMul1Multiplier, wp);
      wv[c] = wp[8 * H + c];
    });
  };
  auto stream_of = [&](int tset, uint32_t (&B)[K + 1]) {
#pragma unroll
    for (int i = 0; i < K; ++i) B[i] = stream_dword(rt[tset][i]);
    B[K] = spill_from_next(rt[tset][0]);
  };
  // One step: the MFMAs on stage `cur` with the A fragments of register set
  // `aset`, and the decode of the next step's trellis (register set `tset`)
  // into stage `nxt`.  The schedule is fixed explicitly: the B fragment reads
  // first, then each MFMA followed by two decode instructions (the matrix
  // core runs while the wave decodes), then the decoded stores.
  //
  // NA (0..MI) is the number of this wave's row groups that run: A loads, B
  // reads and MFMAs cover groups 0..NA-1 only.  A wave with NA = 0 (all its
  // rows at or past T.rows) only decodes its share of B and joins the
  // barriers.
  auto step = [&](const uint4* cur, uint4* nxt, int aset, int tset, auto hc, auto ac) {
    constexpr int NA = decltype(ac)::value;
    uint32_t B[K + 1];
    stream_of(tset, B);
    half8_t bv[8];
    if constexpr (NA > 0) {
#pragma unroll
      for (int q = 0; q < 8; ++q) bv[q] = __builtin_bit_cast(half8_t, cur[br_ch[q]]);
    }
    uint32_t wv[8];
    decode8(B, wv, hc);
#pragma unroll
    for (int q = 0; q < 8; ++q)
#pragma unroll
      for (int mi = 0; mi < NA; ++mi)
        acc[mi][q] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ra[aset][mi], bv[q], acc[mi][q], 0, 0, 0);
    uint32_t* nd = reinterpret_cast<uint32_t*>(nxt);
#pragma unroll
    for (int c = 0; c < 8; ++c) nd[bw_dw[c]] = wv[c];
    if constexpr (NA > 0) {
      __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 9, 0);
      static_for<0, 8 * NA>([&](auto) {
        __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
        __builtin_amdgcn_sched_group_barrier(kSchedValu, 64 / (8 * NA) + 1, 0);
      });
      __builtin_amdgcn_sched_group_barrier(kSchedDsWrite, 8, 0);
      __builtin_amdgcn_sched_group_barrier(kSchedVmemRead, NA + (K + 3) / 4, 0);
    }
  };

  auto run = [&](auto hc, auto ac) {
    constexpr int NA = decltype(ac)::value;
    auto load_a_act = [&](int set, int ks) {
      ks = ks < nsteps ? ks : nsteps - 1;  // past the end: re-read the last step (unused)
#pragma unroll
      for (int mi = 0; mi < NA; ++mi)
        ra[set][mi] = __builtin_bit_cast(
            half8_t, __builtin_amdgcn_raw_buffer_load_b128(a_rs, (int)a_voff[mi], ks * kAStep, 0));
    };
    // prologue: step 0 decoded into stage 0; A of steps 0, 1 and trellis of
    // steps 1, 2 in flight.  The loads go out in a fixed order (scheduling
    // barriers) that leaves, at the loop's entry, at least as many loads
    // issued after each register set as the loop body leaves at its back
    // edge: the wait counts the compiler derives for the loop are the minimum
    // over both edges, so a prologue that ended on the trellis set the first
    // step needs would make every step wait for nearly all loads in flight.
    load_t(0, 0);
    load_t(1, 1);
    __builtin_amdgcn_sched_barrier(0);
    {
      uint32_t B[K + 1], wv[8];
      stream_of(0, B);
      decode8(B, wv, hc);
      uint32_t* nd = reinterpret_cast<uint32_t*>(bst0);
#pragma unroll
      for (int c = 0; c < 8; ++c) nd[bw_dw[c]] = wv[c];
    }
    __builtin_amdgcn_sched_barrier(0);
    load_a_act(0, 0);
    __builtin_amdgcn_sched_barrier(0);
    load_a_act(1, 1);
    __builtin_amdgcn_sched_barrier(0);
    load_t(0, 2);
    __syncthreads();
    __builtin_amdgcn_sched_barrier(0);
    // Step s: MFMAs on stage s % 2 with A set s % 2; decode of step s + 1
    // (trellis set (s + 1) % 2) into the other stage; then A set s % 2 is
    // refilled with step s + 2 and trellis set (s + 1) % 2 with step s + 3.
    // Past the last step the decode and loads repeat valid data that is unused.
    // (sched_barrier: the compiler would otherwise hoist the next step's
    // register-only decode above the barrier, which forces a wait on the
    // loads issued one step earlier)
    for (int ks = 0; ks < nsteps; ks += 2) {
      step(bst0, bst1, 0, 1, hc, ac);
      load_a_act(0, ks + 2);
      load_t(1, ks + 3);
      __syncthreads();
      __builtin_amdgcn_sched_barrier(0);
      step(bst1, bst0, 1, 0, hc, ac);
      load_a_act(1, ks + 3);
      load_t(0, ks + 4);
      __syncthreads();
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // row groups of this wave holding valid rows (uniform per wave)
  const int g16 = (T.rows + 15) >> 4;
  int na = (g16 - wm + 3) >> 2;
  na = na < 0 ? 0 : (na > MI ? MI : na);
  auto go = [&](auto hc) {
    if constexpr (R::kFineSkip) {
      static_for<0, MI + 1>([&](auto nc) {
        if (na == decltype(nc)::value) run(hc, nc);
      });
    } else {
      if (na > 0) run(hc, IntC<MI>{});
      else run(hc, IntC<0>{});
    }
  };
  const int cb = col0 + 128 * wn;
  // R::kGateUp: two passes over the same rows and columns, gate then up; the
  // gate result goes to LDS as fp16, four rows of one column per entry (each
  // lane reads back only what it wrote).  One call site of the k loop, so it
  // stays inlined.
  constexpr int kPasses = R::kGateUp ? 2 : 1;
  for (int pass = 0; pass < kPasses; ++pass) {
    if (pass == 1) {
#pragma unroll
      for (int mi = 0; mi < MI; ++mi)
#pragma unroll
        for (int q = 0; q < 8; ++q) acc[mi][q] = float4_t{0.f, 0.f, 0.f, 0.f};
      t_rs = make_rsrc(T.trellis2, t_bytes);
      a_rs = make_rsrc(T.a2, a_bytes);
    }
    if (h == 0)
      go(IntC<0>{});
    else
      go(IntC<1>{});
    if constexpr (R::kGateUp) {
      if (pass == 0 && na > 0) {
        float sg[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) sg[q] = kInvSqrt128 * h2f(T.svh[cb + 16 * q + j]);
#pragma unroll
        for (int mi = 0; mi < MI; ++mi) {
          if (mi >= na) break;
          float v[4][8];
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) {
#pragma unroll
            for (int q = 0; q < 8; ++q) v[rr][q] = acc[mi][q][rr];
            gemm_col_fwht(v[rr]);
          }
#pragma unroll
          for (int q = 0; q < 8; ++q)
            gst[((wm * MI + mi) * 8 + q) * 64 + lane] =
                make_uint2((uint32_t)f2h(v[0][q] * sg[q]) | ((uint32_t)f2h(v[1][q] * sg[q]) << 16),
                           (uint32_t)f2h(v[2][q] * sg[q]) | ((uint32_t)f2h(v[3][q] * sg[q]) << 16));
        }
      }
    }
  }
  if (na == 0) return;  // no barrier follows

  if constexpr (R::kGateUp) {
    // a = silu(g) u, then the next projection's input transform on this
    // 128-column block: (a .* snext) H / sqrt(128), fp16
    float su[8], sn[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      su[q] = kInvSqrt128 * h2f(T.svh2[cb + 16 * q + j]);
      sn[q] = kInvSqrt128 * h2f(T.snext[cb + 16 * q + j]);
    }
#pragma unroll
    for (int mi = 0; mi < MI; ++mi) {
      if (mi >= na) break;
      uint2 gw[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) gw[q] = gst[((wm * MI + mi) * 8 + q) * 64 + lane];
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        float v[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) v[q] = acc[mi][q][rr];
        gemm_col_fwht(v);
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const uint32_t w2 = (rr < 2) ? gw[q].x : gw[q].y;
          const float gv = h2f((uint16_t)((rr & 1) ? (w2 >> 16) : (w2 & 0xFFFF)));
          v[q] = silu_f(gv) * (v[q] * su[q]) * sn[q];
        }
        gemm_col_fwht(v);
        const int row = 16 * (4 * mi + wm) + 4 * g + rr;
        if (row < T.rows) {
#pragma unroll
          for (int q = 0; q < 8; ++q)
            static_cast<uint16_t*>(T.y)[(int64_t)row * T.ldy + cb + 16 * q + j] = f2h(v[q]);
        }
      }
    }
    return;
  }

  // epilogue: output Hadamard over each wave's 128 columns, svh, bias, cast
  float sv[8], bv[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    sv[q] = kInvSqrt128 * h2f(T.svh[cb + 16 * q + j]);
    bv[q] = T.bias ? h2f(T.bias[cb + 16 * q + j]) : 0.f;
  }
#pragma unroll
  for (int mi = 0; mi < MI; ++mi) {
    if (mi >= na) break;
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      float v[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) v[q] = acc[mi][q][rr];
      gemm_col_fwht(v);
      const int row = 16 * (4 * mi + wm) + 4 * g + rr;
      if (row < T.rows) {
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const int col = cb + 16 * q + j;
          float o = v[q] * sv[q];
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

// K = 1..8: every tile has that width.  K = 0: each tile has its own width
// (T.bits, a width per expert), taken in the workgroup from one launch; the
// eight bodies share the kernel's LDS.
template <int K, int BM, bool Y_F32, class R>
__global__ __launch_bounds__(kGemmThreads, 2) void gemm_kernel(R r, int k, int n) {
  constexpr int MI = BM / 64;
  __shared__ uint4 bst0[kGemmBN * 4], bst1[kGemmBN * 4];
  // R::kGateUp: the gate result of every lane's rows and columns (fp16,
  // four rows per 8-byte entry) between the two passes
  __shared__ uint2 gst[R::kGateUp ? 4 * MI * 8 * 64 : 1];

  const GemmTask T = r.task();
  if (!T.valid) return;
  if constexpr (K == 0) {
    switch (T.bits) {
      case 1: gemm_tile<1, BM, Y_F32>(r, T, k, n, bst0, bst1, gst); break;
      case 2: gemm_tile<2, BM, Y_F32>(r, T, k, n, bst0, bst1, gst); break;
      case 3: gemm_tile<3, BM, Y_F32>(r, T, k, n, bst0, bst1, gst); break;
      case 4: gemm_tile<4, BM, Y_F32>(r, T, k, n, bst0, bst1, gst); break;
      case 5: gemm_tile<5, BM, Y_F32>(r, T, k, n, bst0, bst1, gst); break;
      case 6: gemm_tile<6, BM, Y_F32>(r, T, k, n, bst0, bst1, gst); break;
      case 7: gemm_tile<7, BM, Y_F32>(r, T, k, n, bst0, bst1, gst); break;
      case 8: gemm_tile<8, BM, Y_F32>(r, T, k, n, bst0, bst1, gst); break;
      default: break;
    }
  } else {
    gemm_tile<K, BM, Y_F32>(r, T, k, n, bst0, bst1, gst);
  }
}

}  // namespace exl3
