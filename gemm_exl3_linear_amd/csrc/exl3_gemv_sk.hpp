// Persistent decode GEMV for 1..16 activation rows (dense EXL3 linear).
//
// Work decomposition ("stream-k" at wave granularity).  A row step is one k
// tile (16 rows of k) of one 128-column block (8 n tiles of 16 columns): the
// R = (n/128) * (k/16) row steps are ordered block-major and every wave of the
// persistent grid takes one contiguous run of them, so runs differ by at most
// one row step.  Waves never wait for each other: each keeps PF row-pair loads
// in flight from the start to the end of its run, across block boundaries.
//
// gemv_sk_kernel, per wave:
//   1. m == 1: x' = (x .* suh) H for the (at most a few) k blocks its run
//      touches, computed in the wave after the first trellis loads went out;
//      m > 1: x' comes from one input-transform launch and each row step's
//      A fragment travels with the trellis loads.
//   2. Row step: lane (t, p) loads row pair p of n tile t (one coalesced
//      4K-byte load per lane), decodes 32 weights into k-pairs of biased
//      codes b = 1024 + sigma (decode_rowpair<K, true>) and contracts:
//        m == 1 : v_dot2_f32_f16 with the x' pair of its two rows, 16 column
//                 accumulators per lane, no LDS traffic;
//        m >= 2 : k-pairs through a per-wave LDS transpose into MFMA
//                 16x16x16 f16 (rows padded to 16).
//      alongside, the sum of the segment's x' (a dot with ones at m == 1, a
//      ninth MFMA against an all-ones B at m >= 2).
//   3. Segment end (block changes or run ends): sum b x' - 1534 sum x' for
//      each column goes to the segment's partial slot in the fp32 workspace
//      (the codebook scale 1775 / 2^18 is applied once, in the finish).
// gemv_sk_finish, one wave per (activation row, 128-column block): adds the
// block's slots in slot order, applies the output transform, svh and bias,
// casts and stores y.  The hand-off between the two is the kernel boundary:
// no wave waits on another and no cache maintenance runs inside a kernel
// (the L2 of one XCD does not see another XCD's writes before a device-scope
// release, which at kernel granularity costs nothing extra).
// The sums never depend on timing, so results are bit-reproducible; the plan
// depends on (k, n) only, so a row's arithmetic does not depend on m within
// the MFMA range (2..16).
#pragma once

#include "exl3_device.hpp"

namespace exl3 {

constexpr int kGemvSkWaves = 2048;  // 8 waves per CU of the 256-CU MI355X
constexpr int kSkSlotBatch = 32;    // partial slots loaded per batch in the finish
constexpr int kSkMaxXBlocks = 8;    // k blocks a run may touch (m == 1)

struct SkArgs {
  const uint16_t* trellis;  // [k/16][n/16][16K]
  const uint16_t* suh;      // fp16 [k]
  const uint16_t* x;        // fp16 [m][ldx]
  int64_t ldx;
  const uint16_t* xprep;    // fp16 [m][k] already transformed (m > 1), else nullptr
  int m;
  int k, n;
  int KT;                   // k / 16
  int64_t R;                // row steps = (n / 128) * KT
  int W;                    // waves of the grid
  int slots;                // partial slots per block
  float* part;              // fp32 [n/128][slots][m][128]
  const uint16_t* svh;
  const uint16_t* bias;
  void* y;
  int64_t ldy;
  int y_f32;
};

// wave whose run contains row step r (runs are [w R / W, (w+1) R / W))
__device__ __forceinline__ int sk_owner(int64_t r, int64_t R, int W) {
  return (int)(((r + 1) * W - 1) / R);
}

// dot2 accumulators: sum over the 8 row-pair lanes of a tile; lane p ends with
// the sums of columns 2p and 2p+1 of its n tile
__device__ __forceinline__ void reduce_rowpairs(float (&acc)[16], float& c0, float& c1) {
  const uint32_t l = lane_id();
  float v8[8];
  const bool up4 = (l & 4u) != 0;
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    const float send = up4 ? acc[c] : acc[c + 8];
    const float keep = up4 ? acc[c + 8] : acc[c];
    v8[c] = keep + shfl_xor_f(send, 4);
  }
  float v4[4];
  const bool up2 = (l & 2u) != 0;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const float send = up2 ? v8[c] : v8[c + 4];
    const float keep = up2 ? v8[c + 4] : v8[c];
    v4[c] = keep + shfl_xor_f(send, 2);
  }
  const bool up1 = (l & 1u) != 0;
  {
    const float send = up1 ? v4[0] : v4[2];
    const float keep = up1 ? v4[2] : v4[0];
    c0 = keep + shfl_xor_f(send, 1);
  }
  {
    const float send = up1 ? v4[1] : v4[3];
    const float keep = up1 ? v4[3] : v4[1];
    c1 = keep + shfl_xor_f(send, 1);
  }
}

// LDS per wave: m == 1: x' blocks [kSkMaxXBlocks][128] fp16 (2 KB);
// m >= 2: transpose region [8 n tiles][8 row pairs][20] dwords (5 KB)
constexpr int kSkWaveLdsDot = kSkMaxXBlocks * 128 * 2;
constexpr int kSkWaveLdsMfma = 64 * 20 * 4;

template <int K, bool DOT, int PF>
__global__ __launch_bounds__(256) void gemv_sk_kernel(SkArgs a) {
  constexpr int WAVE_LDS = DOT ? kSkWaveLdsDot : kSkWaveLdsMfma;
  __shared__ __align__(16) unsigned char smem[4 * WAVE_LDS];

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wid = blockIdx.x * 4 + wave;
  const int64_t r0 = (int64_t)wid * a.R / a.W;
  const int64_t r1 = (int64_t)(wid + 1) * a.R / a.W;
  const int len = (int)(r1 - r0);
  if (len <= 0) return;
  const int m = a.m;
  const int nt = a.n >> 4;
  const int KT = a.KT;
  const int lane = threadIdx.x & 63;
  const int t = lane >> 3, p = lane & 7;   // decode role
  const int g = lane >> 4, j = lane & 15;  // MFMA role
  unsigned char* wl = smem + wave * WAVE_LDS;

  // Row-step cursors are uniform: (nb, kt) advance by one k tile per step and
  // wrap to the next block at k/16, so no division happens inside the loop.
  const int64_t nb0 = r0 / KT;
  const int kt0 = (int)(r0 - nb0 * KT);
  const int64_t tile_dw = 8 * K;                 // dwords per 16x16 tile
  const int64_t kt_dw = (int64_t)nt * tile_dw;   // dwords per k tile row
  const uint32_t* tr_lane = reinterpret_cast<const uint32_t*>(a.trellis) + K * p + t * tile_dw;
  // prefetch cursor
  int64_t pf_nb = nb0;
  int pf_kt = kt0;
  int pf_left = len;  // row steps the prefetch cursor may still visit
  auto pf_ptr = [&]() -> const uint32_t* {
    return tr_lane + (int64_t)pf_kt * kt_dw + pf_nb * 8 * tile_dw;
  };
  auto pf_afrag = [&]() -> const uint2* {
    const int row = j < m ? j : 0;
    return reinterpret_cast<const uint2*>(a.xprep + (int64_t)row * a.k + pf_kt * 16 + 4 * g);
  };
  auto pf_advance = [&]() {  // stays on the last row step once the run is exhausted
    const int adv = pf_left > 1 ? 1 : 0;  // selects, not branches: the loads
    pf_left -= adv;                       // around stay unconditional
    pf_kt += adv;
    const int wrap = pf_kt == KT ? 1 : 0;
    pf_kt = wrap ? 0 : pf_kt;
    pf_nb += wrap;
  };

  // ---- m == 1: x' for the k blocks of the run; block b of the run is k block
  // (kt0 / 8 + b) mod k/128.  These loads go out first (a fixed number of them,
  // so the wait below counts only the trellis loads issued after them).
  const int kb0 = kt0 >> 3;
  const int KBn = KT >> 3;
  uint32_t xv[DOT ? kSkMaxXBlocks : 1], sv[DOT ? kSkMaxXBlocks : 1];
  const int nblk = ((kt0 & 7) + len + 7) >> 3;
  if constexpr (DOT) {
#pragma unroll
    for (int b = 0; b < kSkMaxXBlocks; ++b) {
      const int bb = b < nblk ? b : nblk - 1;
      const int kb = (kb0 + bb) % KBn;
      const int kk = kb * 128 + 2 * lane;
      xv[b] = *reinterpret_cast<const uint32_t*>(a.x + kk);
      sv[b] = *reinterpret_cast<const uint32_t*>(a.suh + kk);
    }
  }

  uint32_t ring[PF][K];
  uint2 aring[DOT ? 1 : PF];
#pragma unroll
  for (int s = 0; s < PF; ++s) {
    load_rowpair<K>(pf_ptr(), ring[s]);
    if constexpr (!DOT) aring[s] = *pf_afrag();
    pf_advance();
  }

  if constexpr (DOT) {
    uint16_t* xs = reinterpret_cast<uint16_t*>(wl);
#pragma unroll
    for (int b = 0; b < kSkMaxXBlocks; ++b) {
      if (b < nblk) {
        float x0 = h2f((uint16_t)(xv[b] & 0xFFFF)) * h2f((uint16_t)(sv[b] & 0xFFFF));
        float x1 = h2f((uint16_t)(xv[b] >> 16)) * h2f((uint16_t)(sv[b] >> 16));
        fwht128_pair(x0, x1);
        *reinterpret_cast<uint32_t*>(xs + b * 128 + 2 * lane) =
            (uint32_t)f2h(x0 * kInvSqrt128) | ((uint32_t)f2h(x1 * kInvSqrt128) << 16);
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
  }

  // ---- main loop
  float dacc[16];
  float dxs;        // m == 1: sum of the lane's x' pairs over the segment
  float4_t macc[8];
  float4_t mxs;     // m >= 2: sum of x' over the segment, per row (any column)
  auto clear_acc = [&]() {
    if constexpr (DOT) {
#pragma unroll
      for (int c = 0; c < 16; ++c) dacc[c] = 0.f;
      dxs = 0.f;
    } else {
#pragma unroll
      for (int q = 0; q < 8; ++q) macc[q] = float4_t{0.f, 0.f, 0.f, 0.f};
      mxs = float4_t{0.f, 0.f, 0.f, 0.f};
    }
  };
  clear_acc();
  uint32_t* tr = reinterpret_cast<uint32_t*>(wl);
  uint32_t* my = tr + (t * 8 + p) * 20;

  // segment end: the wave's column sums to the segment's slot (no wait)
  auto flush = [&](int64_t nb) {
    const int slot = wid - sk_owner(nb * KT, a.R, a.W);
    float* dst = a.part + ((int64_t)nb * a.slots + slot) * m * 128;
    if constexpr (DOT) {
#pragma unroll
      for (int c = 0; c < 16; ++c) dacc[c] = __builtin_fmaf(-kSigmaBiasPlus1024, dxs, dacc[c]);
      float c0, c1;
      reduce_rowpairs(dacc, c0, c1);
      *reinterpret_cast<float2*>(dst + 16 * t + 2 * p) = make_float2(c0, c1);
    } else {
#pragma unroll
      for (int q = 0; q < 8; ++q)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const int i = 4 * g + rr;
          if (i < m) dst[i * 128 + 16 * q + j] = __builtin_fmaf(-kSigmaBiasPlus1024, mxs[rr], macc[q][rr]);
        }
    }
    clear_acc();
  };

  // consumption cursor
  int64_t c_nb = nb0;
  int c_kt = kt0;
  int c_b = 0;  // x' block of the run (m == 1)
  for (int base = 0; base < len; base += PF) {
#pragma unroll
    for (int s = 0; s < PF; ++s) {
      const int it = base + s;
      if (it < len) {
        const uint32_t spill = spill_from_next(ring[s][0]);
        uint32_t wp[16];
        decode_rowpair<K, true>(ring[s], spill, wp);
        if constexpr (DOT) {
          const uint16_t* xs = reinterpret_cast<const uint16_t*>(wl);
          const half2_t xp =
              *reinterpret_cast<const half2_t*>(xs + c_b * 128 + (c_kt & 7) * 16 + 2 * p);
          const half2_t ones = {(_Float16)1.0f, (_Float16)1.0f};
          dxs = __builtin_amdgcn_fdot2(xp, ones, dxs, false);
#pragma unroll
          for (int c = 0; c < 16; ++c)
            dacc[c] = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, wp[c]), xp, dacc[c], false);
        } else {
          uint4* my4 = reinterpret_cast<uint4*>(my);
          my4[0] = make_uint4(wp[0], wp[1], wp[2], wp[3]);
          my4[1] = make_uint4(wp[4], wp[5], wp[6], wp[7]);
          my4[2] = make_uint4(wp[8], wp[9], wp[10], wp[11]);
          my4[3] = make_uint4(wp[12], wp[13], wp[14], wp[15]);
          __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
          __builtin_amdgcn_wave_barrier();
          __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
          half4_t av = {0, 0, 0, 0};
          if (j < m) av = __builtin_bit_cast(half4_t, aring[DOT ? 0 : s]);
#pragma unroll
          for (int q = 0; q < 8; ++q) {
            const uint32_t b0 = tr[(q * 8 + 2 * g) * 20 + j];
            const uint32_t b1 = tr[(q * 8 + 2 * g + 1) * 20 + j];
            const half4_t bv = __builtin_bit_cast(half4_t, make_uint2(b0, b1));
            macc[q] = __builtin_amdgcn_mfma_f32_16x16x16f16(av, bv, macc[q], 0, 0, 0);
          }
          const half4_t ones4 = {(_Float16)1.0f, (_Float16)1.0f, (_Float16)1.0f, (_Float16)1.0f};
          mxs = __builtin_amdgcn_mfma_f32_16x16x16f16(av, ones4, mxs, 0, 0, 0);
          __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
          __builtin_amdgcn_wave_barrier();
          __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
        }
        // advance the consumption cursor; segment end at a block end or run end
        const bool block_end = (c_kt + 1 == KT);
        if (block_end || it + 1 == len) flush(c_nb);
        c_kt = block_end ? 0 : c_kt + 1;
        c_nb += block_end ? 1 : 0;
        c_b += (c_kt & 7) == 0 ? 1 : 0;
      }
      // refill the slot (unconditionally: every step issues the same loads, so
      // the wait counts stay static); past the end, re-read the last step
      load_rowpair<K>(pf_ptr(), ring[s]);
      if constexpr (!DOT) aring[s] = *pf_afrag();
      pf_advance();
    }
  }
}

// Slots of block nb: the waves whose runs intersect it, in run order.
__device__ __forceinline__ int sk_arrivals(int64_t nb, int64_t KT, int64_t R, int W) {
  return sk_owner((nb + 1) * KT - 1, R, W) - sk_owner(nb * KT, R, W) + 1;
}

// One wave per (activation row i, 128-column block nb); lane l owns columns
// 2l, 2l+1 of the block.
__global__ __launch_bounds__(256) void gemv_sk_finish(SkArgs a) {
  const int NB = a.n >> 7;
  const int task = blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (task >= NB * a.m) return;
  const int m = a.m;
  const int i = task / NB, nb = task - i * NB;
  const int lane = threadIdx.x & 63;
  const int col = nb * 128 + 2 * lane;
  const int arrivals = sk_arrivals(nb, a.KT, a.R, a.W);
  const float* src = a.part + ((int64_t)nb * a.slots * m + i) * 128 + 2 * lane;
  const uint32_t svv = *reinterpret_cast<const uint32_t*>(a.svh + col);
  uint32_t bv = 0;
  if (a.bias) bv = *reinterpret_cast<const uint32_t*>(a.bias + col);
  // slots in order, up to kSkSlotBatch loads in flight
  float x0 = 0.f, x1 = 0.f;
  for (int s0 = 0; s0 < arrivals; s0 += kSkSlotBatch) {
    float2 v[kSkSlotBatch];
#pragma unroll
    for (int q = 0; q < kSkSlotBatch; ++q)
      if (s0 + q < arrivals)
        v[q] = *reinterpret_cast<const float2*>(src + (int64_t)(s0 + q) * m * 128);
#pragma unroll
    for (int q = 0; q < kSkSlotBatch; ++q)
      if (s0 + q < arrivals) {
        x0 += v[q].x;
        x1 += v[q].y;
      }
  }
  fwht128_pair(x0, x1);
  // codebook scale and the transform's normalisation as one constant
  constexpr float kOut = kMul1Scale * kInvSqrt128;
  x0 *= kOut * h2f((uint16_t)(svv & 0xFFFF));
  x1 *= kOut * h2f((uint16_t)(svv >> 16));
  if (a.bias) {
    x0 += h2f((uint16_t)(bv & 0xFFFF));
    x1 += h2f((uint16_t)(bv >> 16));
  }
  if (a.y_f32)
    *reinterpret_cast<float2*>(static_cast<float*>(a.y) + (int64_t)i * a.ldy + col) =
        make_float2(x0, x1);
  else
    *reinterpret_cast<uint32_t*>(static_cast<uint16_t*>(a.y) + (int64_t)i * a.ldy + col) =
        (uint32_t)f2h(x0) | ((uint32_t)f2h(x1) << 16);
}

}  // namespace exl3
