// Decode GEMV of several tensors that share one activation row (m == 1) in
// one launch pair: the projections that read the same input (q, k and v;
// gate and up) through exl3_linear_multi.
//
// Work decomposition ("stream-k" at wave granularity).  A row step is one k
// tile (16 rows of k) of one 128-column block (8 n tiles of 16 columns): a
// tensor's R = (n/128) * (k/16) row steps are ordered block-major and every
// wave of its share of the persistent grid takes one contiguous run of them.
// Waves never wait for each other: each keeps PF row-pair loads in flight from
// the start to the end of its run, across block boundaries.  The row
// contracts on the vector units (v_dot2).  Run lengths come in two tiers
// (SkSplit).  With two waves per SIMD, the wave dispatched in the first round
// (one per SIMD, the lower wave ids) is the older one and wins the
// instruction arbiter whenever both are ready; measured on MI355X at
// 5120 x 17408, it completes about 1.9 times the row steps of its younger
// partner in the same time, so equal runs leave the younger waves finishing
// alone.  The first-round waves therefore take runs kSkTierWeight1 /
// kSkTierWeight2 times longer than the rest.  The split is part of the plan
// (a function of k, n and the grid only), never of timing.
//
// sk_run, per wave:
//   1. x' = (x .* suh) H for the (at most eight) k blocks its run touches,
//      four blocks at a time, after the first trellis loads went out.
//   2. Row step: lane (t, p) loads row pair p of n tile t (one coalesced
//      4K-byte load per lane) and the first dword of the next row pair (its
//      spill word), decodes 32 weights into k-pairs of biased codes
//      b = 1024 + sigma (decode_rowpair<K, true>) and contracts them with
//      v_dot2_f32_f16 against the row's x' pair of its two k rows, 16 column
//      accumulators per lane; alongside, the sum of the segment's x' (a dot
//      with ones).
//   3. Segment end (block changes or run ends): sum b x' - 1534 sum x' for
//      each column goes to the segment's partial slot in the fp32 workspace
//      (the codebook scale 1775 / 2^18 is applied once, in the finish).
// gemv_sk_multi_finish, one wave per 128-column block: adds the block's slots
// in slot order, applies the output transform, svh and bias, casts and stores
// y.  The hand-off between the two is the kernel boundary.  The sums never
// depend on timing, so results are bit-reproducible.
#pragma once

#include "exl3_device.hpp"
#include "exl3_sk_split.hpp"

namespace exl3 {

constexpr int kGemvSkWaves = 2048;    // 8 waves per CU of the 256-CU MI355X
constexpr int kGemvRoundWaves = 1024; // one wave per SIMD: 256 CUs x 4 SIMDs
constexpr int kSkTierWeight1 = 13;    // relative run length, first-round waves
constexpr int kSkTierWeight2 = 7;     // relative run length, the others
constexpr int kSkMaxRun = 48;         // longest run (the x' region of a wave)
constexpr int kSkSlotBatch = 8;     // partial slots per lane loaded per batch in the finish
constexpr int kSkMaxXBlocks = 8;    // k blocks a run may touch

struct SkArgs {
  const uint16_t* trellis;  // [k/16][n/16][16K]
  const uint16_t* suh;      // fp16 [k]
  const uint16_t* x;        // fp16 [m][ldx]
  int64_t ldx;
  int m;
  int k, n;
  int KT;                   // k / 16
  int R;                    // row steps = (n / 128) * KT
  int W;                    // waves of the grid
  SkSplit sp;               // run of every wave
  int slots;                // partial slots per block
  float* part;              // fp32 [n/128][slots][m][128]
  const uint16_t* svh;
  const uint16_t* bias;
  void* y;
  int64_t ldy;
  int y_f32;
};

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

// LDS per wave: x' blocks [kSkMaxXBlocks][128] fp16 (2 KB) per row
constexpr int kSkWaveLdsDot = kSkMaxXBlocks * 128 * 2;
// a run of kSkMaxRun steps starting anywhere in a k block fits the x' region
static_assert(32 * (kSkMaxRun + 8) + 32 <= kSkWaveLdsDot, "x' region too small");
static_assert((7 + kSkMaxRun + 7) / 8 <= kSkMaxXBlocks, "run touches too many k blocks");

// The work of wave `wid` of a tensor's grid; wl is the wave's LDS region:
// the v_dot2 contraction for up to NR activation rows (x' of row i in the
// wave's i-th kSkWaveLdsDot region).
template <int K, int NR, int PF>
__device__ __forceinline__ void sk_run(const SkArgs& a, int wid, unsigned char* wl) {
  const int len = sk_run_len(a.sp, wid);
  if (len <= 0) return;
  const int r0 = sk_run_start(a.sp, wid);
  const int m = a.m;
  const int KT = a.KT;
  const int lane = threadIdx.x & 63;
  const int t = lane >> 3, p = lane & 7;   // decode role
  const int g = lane >> 4, j = lane & 15;  // input-transform role

  // The run starts at k tile kt0 of block nb0; the wave is partial slot
  // slot0 of that block and slot 0 of every later one.
  const int nb0 = r0 / KT;
  const int kt0 = r0 - nb0 * KT;
  const int slot0 = wid - sk_run_owner(a.sp, nb0 * KT);

  // Trellis addressing.  One buffer descriptor per 128-column block covers
  // its k range; a row step is a uniform offset (kt * bytes of a k-tile row),
  // a lane adds its row pair and the first dword of the next row pair of the
  // same tile (the spill word, cyclic inside the tile).
  constexpr int kTileBytes = 32 * K;
  constexpr int kBlkBytes = 8 * kTileBytes;
  const uint32_t kt_bytes = (uint32_t)(a.n >> 4) * kTileBytes;  // whole tensor < 2^32 B
  const uint32_t col_bytes = (uint32_t)(KT - 1) * kt_bytes + kBlkBytes;
  const uint32_t lane_off = (uint32_t)(t * kTileBytes + 4 * K * p);
  const uint32_t spill_off = (uint32_t)(t * kTileBytes + 4 * K * ((p + 1) & 7));
  const unsigned char* tr0 = reinterpret_cast<const unsigned char*>(a.trellis);
  int pf_nb = nb0, pf_kt = kt0, pf_left = len;
  uint32_t pf_soff = (uint32_t)kt0 * kt_bytes;
  __amdgpu_buffer_rsrc_t pf_rs = make_rsrc(tr0 + (int64_t)pf_nb * kBlkBytes, col_bytes);
  auto pf_load = [&](uint32_t (&D)[K + 1]) {
    load_rowpair_buf<K>(pf_rs, lane_off, pf_soff, D);
    D[K] = __builtin_amdgcn_raw_buffer_load_b32(pf_rs, (int)spill_off, (int)pf_soff, 0);
  };
  auto pf_advance = [&]() {  // stays on the last row step once the run is exhausted
    if (pf_left > 1) {
      --pf_left;
      ++pf_kt;
      pf_soff += kt_bytes;
      if (pf_kt == KT) {
        pf_kt = 0;
        pf_soff = 0;
        ++pf_nb;
        pf_rs = make_rsrc(tr0 + (int64_t)pf_nb * kBlkBytes, col_bytes);
      }
    }
  };

  // ---- x and suh of the k blocks the run touches go out first: k block b of
  // the run is (kt0 / 8 + b) mod k/128; lane l loads 8 elements of run block
  // l / 16 (first round) and 4 + l / 16 (second round), of every row.
  const int nblk = ((kt0 & 7) + len + 7) >> 3;
  uint4 xv[NR][2], sv[2];
  {
    const int kb0 = kt0 >> 3, KBn = KT >> 3;
#pragma unroll
    for (int rd = 0; rd < 2; ++rd) {
      const int b = 4 * rd + g;
      const int bb = b < nblk ? b : nblk - 1;
      const int kk = ((kb0 + bb) % KBn) * 128 + 8 * j;
      sv[rd] = *reinterpret_cast<const uint4*>(a.suh + kk);
#pragma unroll
      for (int i = 0; i < NR; ++i)  // rows past m read row 0 (their sums are not stored)
        xv[i][rd] = *reinterpret_cast<const uint4*>(a.x + (i < m ? i : 0) * a.ldx + kk);
    }
  }

  uint32_t ring[PF][K + 1];
#pragma unroll
  for (int s = 0; s < PF; ++s) {
    pf_load(ring[s]);
    pf_advance();
  }

  {
#pragma unroll
    for (int i = 0; i < NR; ++i) {
      uint16_t* xs = reinterpret_cast<uint16_t*>(wl + i * kSkWaveLdsDot);
#pragma unroll
      for (int rd = 0; rd < 2; ++rd) {
        if (4 * rd < nblk) {
          const uint32_t xw[4] = {xv[i][rd].x, xv[i][rd].y, xv[i][rd].z, xv[i][rd].w};
          const uint32_t sw[4] = {sv[rd].x, sv[rd].y, sv[rd].z, sv[rd].w};
          float v[8];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            v[2 * e] = h2f((uint16_t)(xw[e] & 0xFFFF)) * h2f((uint16_t)(sw[e] & 0xFFFF));
            v[2 * e + 1] = h2f((uint16_t)(xw[e] >> 16)) * h2f((uint16_t)(sw[e] >> 16));
          }
          fwht128_x8(v);
          uint32_t o[4];
#pragma unroll
          for (int e = 0; e < 4; ++e)
            o[e] = (uint32_t)f2h(v[2 * e] * kInvSqrt128) | ((uint32_t)f2h(v[2 * e + 1] * kInvSqrt128) << 16);
          if (4 * rd + g < nblk)
            *reinterpret_cast<uint4*>(xs + (4 * rd + g) * 128 + 8 * j) = make_uint4(o[0], o[1], o[2], o[3]);
        }
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
  }

  // ---- main loop
  float dacc[NR][16];
  float dxs[NR];    // sum of the lane's x' pairs over the segment, per row
  auto clear_acc = [&]() {
#pragma unroll
    for (int i = 0; i < NR; ++i) {
#pragma unroll
      for (int c = 0; c < 16; ++c) dacc[i][c] = 0.f;
      dxs[i] = 0.f;
    }
  };
  clear_acc();

  // segment end: the wave's column sums to the segment's slot (no wait)
  auto flush = [&](int nb, int slot) {
    float* dst = a.part + ((int64_t)nb * a.slots + slot) * m * 128;
#pragma unroll
    for (int i = 0; i < NR; ++i) {
      if (i < m) {  // uniform
#pragma unroll
        for (int c = 0; c < 16; ++c) dacc[i][c] = __builtin_fmaf(-kSigmaBiasPlus1024, dxs[i], dacc[i][c]);
        float c0, c1;
        reduce_rowpairs(dacc[i], c0, c1);
        *reinterpret_cast<float2*>(dst + i * 128 + 16 * t + 2 * p) = make_float2(c0, c1);
      }
    }
    clear_acc();
  };

  // The x' pair of step `it` is at byte 32 (it + kt0 % 8) + 4 p of the wave's
  // region: one k tile is 32 bytes of x', and k blocks of the run follow each
  // other (a block column ends at a k-block boundary).  It is read one step
  // ahead; the read after the last step stays inside the region
  // (runs are at most kSkMaxRun steps).
  const unsigned char* xlane = wl + 32 * (kt0 & 7) + 4 * p;
  half2_t xp[NR];
#pragma unroll
  for (int i = 0; i < NR; ++i) {
    xp[i] = *reinterpret_cast<const half2_t*>(xlane + i * kSkWaveLdsDot);
  }
  int c_nb = nb0, c_slot = slot0;
  int to_end = KT - kt0;  // row steps left in the current block
  for (int base = 0; base < len; base += PF) {
    const unsigned char* xg = xlane + 32 * base;
#pragma unroll
    for (int s = 0; s < PF; ++s) {
      const int it = base + s;
      if (it < len) {
        uint32_t wp[16];
        decode_rowpair<K, true>(*reinterpret_cast<const uint32_t(*)[K]>(ring[s]),
                                stream_dword(ring[s][K]), wp);
        const half2_t ones = {(_Float16)1.0f, (_Float16)1.0f};
#pragma unroll
        for (int i = 0; i < NR; ++i) {
          const half2_t xc = xp[i];
          xp[i] = *reinterpret_cast<const half2_t*>(xg + i * kSkWaveLdsDot + 32 * (s + 1));
          dxs[i] = __builtin_amdgcn_fdot2(xc, ones, dxs[i], false);
#pragma unroll
          for (int c = 0; c < 16; ++c)
            dacc[i][c] = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, wp[c]), xc, dacc[i][c], false);
        }
        // segment end at a block end or the run's end
        --to_end;
        if (to_end == 0 || it + 1 == len) {
          flush(c_nb, c_slot);
          c_slot = 0;
          if (to_end == 0) {
            ++c_nb;
            to_end = KT;
          }
        }
      }
      // refill the slot (unconditionally: every step issues the same loads, so
      // the wait counts stay static); past the end, re-read the last step
      pf_load(ring[s]);
      pf_advance();
    }
  }
}

// Finish of (activation row i, 128-column block nb), by one wave.  Lane l
// owns columns 8 (l % 16) .. 8 (l % 16) + 7 of the block and sums the block's
// slots l / 16, l / 16 + 4, l / 16 + 8, ... in that order; the four slot
// groups are then combined as (g0 + g1) + (g2 + g3) (fp32 addition commutes,
// so every lane ends with the same total whichever of a pair it holds).  The
// output transform is three in-lane butterfly stages and four lane swizzles
// inside each group of 16 lanes; lanes 0..15 store.
__device__ __forceinline__ void sk_finish(const SkArgs& a, int i, int nb) {
  const int m = a.m;
  const int lane = (int)(threadIdx.x & 63);
  const int c8 = 8 * (lane & 15);
  const int sg = lane >> 4;
  const int col = nb * 128 + c8;
  const int arrivals = sk_arrivals(a.sp, nb, a.KT);
  const float* src = a.part + ((int64_t)nb * a.slots * m + i) * 128 + c8;
  const uint4 svv = *reinterpret_cast<const uint4*>(a.svh + col);
  uint4 bv = make_uint4(0, 0, 0, 0);
  if (a.bias) bv = *reinterpret_cast<const uint4*>(a.bias + col);
  float v[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int s0 = sg; s0 < arrivals; s0 += 4 * kSkSlotBatch) {
    float4 lo[kSkSlotBatch], hi[kSkSlotBatch];
#pragma unroll
    for (int q = 0; q < kSkSlotBatch; ++q)
      if (s0 + 4 * q < arrivals) {
        const float4* p4 = reinterpret_cast<const float4*>(src + (int64_t)(s0 + 4 * q) * m * 128);
        lo[q] = p4[0];
        hi[q] = p4[1];
      }
#pragma unroll
    for (int q = 0; q < kSkSlotBatch; ++q)
      if (s0 + 4 * q < arrivals) {
        v[0] += lo[q].x; v[1] += lo[q].y; v[2] += lo[q].z; v[3] += lo[q].w;
        v[4] += hi[q].x; v[5] += hi[q].y; v[6] += hi[q].z; v[7] += hi[q].w;
      }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] += swizzle_xor_f<16>(v[e]);
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] += shfl_xor_f(v[e], 32);
  fwht128_x8(v);
  // codebook scale and the transform's normalisation as one constant
  constexpr float kOut = kMul1Scale * kInvSqrt128;
  const uint32_t sw[4] = {svv.x, svv.y, svv.z, svv.w};
  const uint32_t bw[4] = {bv.x, bv.y, bv.z, bv.w};
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    v[2 * e] *= kOut * h2f((uint16_t)(sw[e] & 0xFFFF));
    v[2 * e + 1] *= kOut * h2f((uint16_t)(sw[e] >> 16));
    if (a.bias) {
      v[2 * e] += h2f((uint16_t)(bw[e] & 0xFFFF));
      v[2 * e + 1] += h2f((uint16_t)(bw[e] >> 16));
    }
  }
  if (sg != 0) return;
  if (a.y_f32) {
    float4* yp = reinterpret_cast<float4*>(static_cast<float*>(a.y) + (int64_t)i * a.ldy + col);
    yp[0] = make_float4(v[0], v[1], v[2], v[3]);
    yp[1] = make_float4(v[4], v[5], v[6], v[7]);
  } else {
    uint32_t o[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] = (uint32_t)f2h(v[2 * e]) | ((uint32_t)f2h(v[2 * e + 1]) << 16);
    *reinterpret_cast<uint4*>(static_cast<uint16_t*>(a.y) + (int64_t)i * a.ldy + col) =
        make_uint4(o[0], o[1], o[2], o[3]);
  }
}


// ---------------------------------------------------------------------------
// Several tensors that share one activation row (m == 1) in one launch pair:
// the projections that read the same input (q, k, v; gate and up), each with
// its own width K, shape and signs (TensorFold issue #832, "Description":
// widths are mixed per tensor).  Every tensor keeps its own stream-k plan over
// W_i waves (W_i in proportion to its trellis bytes); the waves of the grid
// are the tensors' waves one after the other, and a wave dispatches on its
// tensor's K.  One finishing launch covers all tensors' blocks.
// ---------------------------------------------------------------------------
constexpr int kSkMaxMulti = 8;

struct SkMulti {
  int count;
  int wbase[kSkMaxMulti + 1];  // first wave of tensor i; wbase[count] = all waves
  int fbase[kSkMaxMulti + 1];  // first finishing task of tensor i
  int bits[kSkMaxMulti];
  SkArgs t[kSkMaxMulti];
};

template <int PF, int K = 1>
__device__ __forceinline__ void sk_run_bits(int bits, const SkArgs& a, int wid, unsigned char* wl) {
  if constexpr (K <= 8) {
    if (bits == K)
      sk_run<K, 1, PF>(a, wid, wl);
    else
      sk_run_bits<PF, K + 1>(bits, a, wid, wl);
  }
}

template <int PF>
__global__ __launch_bounds__(256) void gemv_sk_multi_kernel(SkMulti ma) {
  __shared__ __align__(16) unsigned char smem[4 * kSkWaveLdsDot];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int gw = (int)blockIdx.x * 4 + wave;
  int i = 0;
  while (i + 1 < ma.count && gw >= ma.wbase[i + 1]) ++i;
  if (gw >= ma.wbase[i + 1]) return;
  sk_run_bits<PF>(ma.bits[i], ma.t[i], gw - ma.wbase[i], smem + wave * kSkWaveLdsDot);
}

__global__ __launch_bounds__(64) void gemv_sk_multi_finish(SkMulti ma) {
  const int task = (int)blockIdx.x;
  int i = 0;
  while (i + 1 < ma.count && task >= ma.fbase[i + 1]) ++i;
  if (task >= ma.fbase[i + 1]) return;
  sk_finish(ma.t[i], 0, task - ma.fbase[i]);
}

}  // namespace exl3
