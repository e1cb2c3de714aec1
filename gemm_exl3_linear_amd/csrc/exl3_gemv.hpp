// Decode-GEMV kernel template shared by the dense linear and the grouped
// experts (see exl3_gemv.hip for the design).  A resolver R maps
// (blockIdx.z, blockIdx.y) to the tensor, activations and workspace slice of
// one workgroup.
#pragma once

#include "exl3_device.hpp"

namespace exl3 {

struct GemvTask {
  bool valid;
  const uint16_t* trellis;  // tensor base, [k/16][n/16][16K]
  const uint16_t* suh;      // fp16 [k]; nullptr: x is already in the Hadamard domain
  const uint16_t* x;        // fp16 row 0, rows at stride ldx
  int64_t ldx;
  int m;                    // activation rows, 1..16
  float* partial;           // fp32 [m][n] slice of this k range
};

constexpr size_t kGemvMaxLds = 64 * 1024;
constexpr int kGemvTargetWorkgroups = 1024;

size_t gemv_lds_bytes(int kc, int m);
int gemv_choose_splits(int k, int groups, int m, int target_wgs);
hipError_t launch_gemv_epilogue(const float* partial, int splits, int m, int n,
                                const uint16_t* svh, const uint16_t* bias, void* y, int64_t ldy,
                                bool y_f32, hipStream_t s);

// ---------------------------------------------------------------------------
// prologue: x' = (x .* suh) H over the workgroup's k range into LDS, layout
// xs[kt][i][16] (k tile, activation row, 16 k values) as fp16.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void gemv_prologue(const GemvTask& T, int k0, int kc, uint16_t* xs) {
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int kblocks = kc >> 7;
  const int m = T.m;
  for (int task = wave; task < kblocks * m; task += 4) {
    const int i = task / kblocks;
    const int blk = task - i * kblocks;
    const int kk = k0 + blk * 128 + 2 * lane;
    const uint32_t xv = *reinterpret_cast<const uint32_t*>(T.x + (int64_t)i * T.ldx + kk);
    float a = h2f((uint16_t)(xv & 0xFFFF)), b = h2f((uint16_t)(xv >> 16));
    if (T.suh) {
      const uint32_t s = *reinterpret_cast<const uint32_t*>(T.suh + kk);
      a *= h2f((uint16_t)(s & 0xFFFF));
      b *= h2f((uint16_t)(s >> 16));
      fwht128_pair(a, b);
      a *= kInvSqrt128;
      b *= kInvSqrt128;
    }
    const int ktl = blk * 8 + (lane >> 3);
    const uint32_t v = (uint32_t)f2h(a) | ((uint32_t)f2h(b) << 16);
    *reinterpret_cast<uint32_t*>(xs + ((ktl * m + i) << 4) + ((2 * lane) & 15)) = v;
  }
}

template <int K, class R>
__global__ __launch_bounds__(256) void gemv_kernel(R r, int k, int n, int kc) {
  extern __shared__ __align__(16) unsigned char smem[];
  const GemvTask T = r.task(blockIdx.z, blockIdx.y);
  if (!T.valid) return;  // uniform over the workgroup
  const int m = T.m;
  const int nb = blockIdx.x;
  const int k0 = blockIdx.y * kc;
  const int ktiles = kc >> 4;
  const int nt = n >> 4;
  uint16_t* xs = reinterpret_cast<uint16_t*>(smem);
  const size_t xs_bytes = ((size_t)kc * m * 2 + 15) & ~(size_t)15;
  uint32_t* tr_all = reinterpret_cast<uint32_t*>(smem + xs_bytes);
  float* red = reinterpret_cast<float*>(smem + xs_bytes);

  gemv_prologue(T, k0, kc, xs);
  __syncthreads();

  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int t = lane >> 3, p = lane & 7;    // decode role: n-tile, row pair
  const int g = lane >> 4, j = lane & 15;   // MFMA role: k group, row/column
  uint32_t* tr = tr_all + wave * (64 * 20);
  uint32_t* my = tr + (t * 8 + p) * 20;

  // lane's row pair in k tile kt: dword offset ((k0/16 + kt) * nt + nb*8 + t) * 8K + K p
  const uint32_t* tbase = reinterpret_cast<const uint32_t*>(T.trellis) +
                          ((int64_t)(k0 >> 4) * nt + nb * 8 + t) * (8 * K) + K * p;
  const int64_t kt_stride = (int64_t)nt * (8 * K);

  float4_t acc[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) acc[q] = float4_t{0.f, 0.f, 0.f, 0.f};

  const int cnt = (ktiles - wave + 3) >> 2;  // k tiles wave, wave+4, ...
  constexpr int PF = (K <= 4) ? 8 : 4;
  uint32_t ring[PF][K];
#pragma unroll
  for (int s = 0; s < PF; ++s)
    if (s < cnt) load_rowpair<K>(tbase + (int64_t)(wave + 4 * s) * kt_stride, ring[s]);

  for (int base = 0; base < cnt; base += PF) {
#pragma unroll
    for (int s = 0; s < PF; ++s) {
      const int it = base + s;
      if (it < cnt) {
        uint32_t D[K];
#pragma unroll
        for (int q = 0; q < K; ++q) D[q] = ring[s][q];
        if (it + PF < cnt)
          load_rowpair<K>(tbase + (int64_t)(wave + 4 * (it + PF)) * kt_stride, ring[s]);
        const int kt = wave + 4 * it;
        const uint32_t spill = spill_from_next(D[0]);
        uint32_t wp[16];
        decode_rowpair<K>(D, spill, wp);
        uint4* my4 = reinterpret_cast<uint4*>(my);
        my4[0] = make_uint4(wp[0], wp[1], wp[2], wp[3]);
        my4[1] = make_uint4(wp[4], wp[5], wp[6], wp[7]);
        my4[2] = make_uint4(wp[8], wp[9], wp[10], wp[11]);
        my4[3] = make_uint4(wp[12], wp[13], wp[14], wp[15]);
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        half4_t av = {0, 0, 0, 0};
        if (j < m) av = *reinterpret_cast<const half4_t*>(xs + ((kt * m + j) << 4) + 4 * g);
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const uint32_t b0 = tr[(q * 8 + 2 * g) * 20 + j];
          const uint32_t b1 = tr[(q * 8 + 2 * g + 1) * 20 + j];
          const uint2 bb = make_uint2(b0, b1);
          const half4_t bv = __builtin_bit_cast(half4_t, bb);
          acc[q] = __builtin_amdgcn_mfma_f32_16x16x16f16(av, bv, acc[q], 0, 0, 0);
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      }
    }
  }

  // fixed-order reduction of the four waves' partials
  __syncthreads();
#pragma unroll
  for (int q = 0; q < 8; ++q) {
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const int i = 4 * g + rr;
      if (i < m) red[(wave * m + i) * 128 + q * 16 + j] = acc[q][rr];
    }
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < m * 128; idx += 256) {
    const int i = idx >> 7, c = idx & 127;
    float s = red[i * 128 + c];
    s += red[(m + i) * 128 + c];
    s += red[(2 * m + i) * 128 + c];
    s += red[(3 * m + i) * 128 + c];
    T.partial[(int64_t)i * n + nb * 128 + c] = s;
  }
}

}  // namespace exl3
