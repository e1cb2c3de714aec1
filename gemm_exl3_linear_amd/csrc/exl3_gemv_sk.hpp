// Persistent decode GEMV for 1..16 activation rows (dense EXL3 linear).
//
// Work decomposition ("stream-k"): the product is cut into units of one
// 128-column block (nb) by one 128-row block of k (kb); units are ordered
// nb-major and every workgroup takes one contiguous run of them, so the
// number of trellis bytes per workgroup differs by at most one unit.  The
// grid holds two workgroups per CU, all resident at once: each wave keeps PF
// row-pair loads in flight across the whole run, including across n-block
// boundaries, and the only drain is at the end of the run.
//
// Per workgroup:
//   1. x' = (x .* suh) H for the k blocks of its units (fp16, LDS); these
//      loads go out first, the trellis loads right after.
//   2. Main loop.  Iteration `it` of wave w covers k tile 8 kb + w + 4 (it&1)
//      of unit it/2 over the 8 n tiles of the block: lane (t, p) loads row
//      pair p of n tile t (one coalesced 4K-byte load per lane), decodes 32
//      weights into k-pairs, and contracts them:
//        m == 1 : v_dot2_f32_f16 with the x' pair of its two rows, 16 column
//                 accumulators per lane (no LDS traffic);
//        m >= 2 : the k-pairs go through a per-wave LDS transpose into MFMA
//                 16x16x16 f16 (rows padded to 16).
//   3. At the end of each n-block segment of the run, the waves' sums are
//      reduced in a fixed order and stored to the segment's partial slot with
//      agent-coherent stores (they write through to the device coherence
//      point; no cache write-back of the whole L2 is needed).
//   4. After the run: one wait for those stores, one relaxed agent-scope
//      atomic increment per segment; the workgroup that completes an n block
//      sums its slots in slot order (agent-coherent loads), applies the
//      output transform, svh and bias, casts, stores y and resets the counter.
// The sums never depend on timing, so results are bit-reproducible; a row's
// arithmetic does not depend on m within the MFMA range.
#pragma once

#include "exl3_device.hpp"

namespace exl3 {

constexpr int kGemvSkWorkgroups = 512;
constexpr int kSkMaxSlots = 16;  // partial slots per n block (the planner keeps below this)

struct SkArgs {
  const uint16_t* trellis;  // [k/16][n/16][16K]
  const uint16_t* suh;      // fp16 [k]
  const uint16_t* x;        // fp16 [m][ldx]
  int64_t ldx;
  const uint16_t* xprep;    // fp16 [m][k] already transformed, or nullptr (m == 1)
  int m;
  int k, n;
  int KB, NB;               // k/128, n/128
  int64_t U;                // units = NB * KB
  int G;                    // workgroups (grid)
  int slots;                // partial slots per n block
  float* part;              // fp32 [NB][slots][m][128]
  unsigned int* ctr;        // [NB] arrival counters (zero between calls)
  const uint16_t* svh;
  const uint16_t* bias;
  void* y;
  int64_t ldy;
  int y_f32;
};

// workgroup whose run contains unit u (runs are [w U / G, (w+1) U / G))
__device__ __forceinline__ int sk_owner(int64_t u, int64_t U, int G) {
  return (int)(((u + 1) * G - 1) / U);
}

__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

__device__ __forceinline__ void store_coherent(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_coherent(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// dot2 reduction over the 8 row-pair lanes of a tile: lane p ends with the
// sums of columns 2p and 2p+1 of its n tile
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
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const float send = up1 ? v4[c] : v4[c + 2];
    const float keep = up1 ? v4[c + 2] : v4[c];
    (c == 0 ? c0 : c1) = keep + shfl_xor_f(send, 1);
  }
}

template <int K, bool DOT, int PF>
__global__ __launch_bounds__(256) void gemv_sk_kernel(SkArgs a) {
  extern __shared__ __align__(16) unsigned char smem[];
  __shared__ int last_flags[64];

  const int w = blockIdx.x;
  const int64_t u0 = (int64_t)w * a.U / a.G;
  const int64_t u1 = (int64_t)(w + 1) * a.U / a.G;
  const int nu = (int)(u1 - u0);
  if (nu <= 0) return;
  const int m = a.m;
  const int nt = a.n >> 4;
  const int KB = a.KB;

  uint16_t* xs = reinterpret_cast<uint16_t*>(smem);  // [nu][m][128]
  const size_t xs_bytes = ((size_t)nu * m * 256 + 15) & ~(size_t)15;
  float* red = reinterpret_cast<float*>(smem + xs_bytes);                 // [4][m][128]
  uint32_t* tr_all = reinterpret_cast<uint32_t*>(smem + xs_bytes + (size_t)4 * m * 512);

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int t = lane >> 3, p = lane & 7;   // decode role
  const int g = lane >> 4, j = lane & 15;  // MFMA role

  // ---- 1. input transform, first batch of loads before the trellis loads
  const int tasks = nu * m;
  constexpr int XB = 4;  // tasks per wave per batch
  uint32_t xv[XB], sv[XB];
  auto load_tasks = [&](int first) {
#pragma unroll
    for (int q = 0; q < XB; ++q) {
      const int task = first + 4 * q;
      if (task < tasks) {
        const int ui = task / m, i = task - ui * m;
        const int kb = (int)((u0 + ui) % KB);
        const int kk = kb * 128 + 2 * lane;
        xv[q] = *reinterpret_cast<const uint32_t*>(a.x + (int64_t)i * a.ldx + kk);
        sv[q] = *reinterpret_cast<const uint32_t*>(a.suh + kk);
      }
    }
  };
  auto transform_tasks = [&](int first) {
#pragma unroll
    for (int q = 0; q < XB; ++q) {
      const int task = first + 4 * q;
      if (task < tasks) {
        float x0 = h2f((uint16_t)(xv[q] & 0xFFFF)) * h2f((uint16_t)(sv[q] & 0xFFFF));
        float x1 = h2f((uint16_t)(xv[q] >> 16)) * h2f((uint16_t)(sv[q] >> 16));
        fwht128_pair(x0, x1);
        x0 *= kInvSqrt128;
        x1 *= kInvSqrt128;
        *reinterpret_cast<uint32_t*>(xs + (size_t)task * 128 + 2 * lane) =
            (uint32_t)f2h(x0) | ((uint32_t)f2h(x1) << 16);
      }
    }
  };
  if (!a.xprep) load_tasks(wave);

  // ---- trellis ring: iteration it -> unit it/2, k tile w + 4 (it & 1)
  const int iters = 2 * nu;
  const uint32_t* tr_base = reinterpret_cast<const uint32_t*>(a.trellis) + K * p;
  auto tile_ptr = [&](int it) -> const uint32_t* {
    const int64_t u = u0 + (it >> 1);
    const int64_t nb = u / KB;
    const int64_t kt = (u - nb * KB) * 8 + wave + 4 * (it & 1);
    return tr_base + ((kt * nt + nb * 8 + t) * (8 * K));
  };
  uint32_t ring[PF][K];
#pragma unroll
  for (int s = 0; s < PF; ++s) load_rowpair<K>(tile_ptr(s < iters ? s : iters - 1), ring[s]);

  if (!a.xprep) {
    transform_tasks(wave);
    for (int first = wave + 4 * XB; first < tasks; first += 4 * XB) {
      load_tasks(first);
      transform_tasks(first);
    }
  } else {
    // x' was prepared by the input-transform kernel: copy the run's blocks
    const int chunks = tasks * 16;  // 16-byte chunks
#pragma unroll 4
    for (int idx = threadIdx.x; idx < chunks; idx += 256) {
      const int task = idx >> 4, ofs = (idx & 15) * 8;
      const int ui = task / m, i = task - ui * m;
      const int kb = (int)((u0 + ui) % KB);
      *reinterpret_cast<uint4*>(xs + (size_t)task * 128 + ofs) =
          *reinterpret_cast<const uint4*>(a.xprep + (int64_t)i * a.k + kb * 128 + ofs);
    }
  }
  lds_barrier();

  // ---- 2. main loop
  float dacc[16];
  float4_t macc[8];
  auto clear_acc = [&]() {
    if constexpr (DOT) {
#pragma unroll
      for (int c = 0; c < 16; ++c) dacc[c] = 0.f;
    } else {
#pragma unroll
      for (int q = 0; q < 8; ++q) macc[q] = float4_t{0.f, 0.f, 0.f, 0.f};
    }
  };
  clear_acc();
  uint32_t* tr = tr_all + wave * (64 * 20);
  uint32_t* my = tr + (t * 8 + p) * 20;
  const int64_t nb_first = u0 / KB;

  // end of an n-block segment: fixed-order sum over the waves, coherent store
  auto flush = [&](int64_t nb) {
    if constexpr (DOT) {
      float c0, c1;
      reduce_rowpairs(dacc, c0, c1);
      *reinterpret_cast<float2*>(red + wave * 128 + 16 * t + 2 * p) = make_float2(c0, c1);
    } else {
#pragma unroll
      for (int q = 0; q < 8; ++q)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const int i = 4 * g + rr;
          if (i < m) red[(wave * m + i) * 128 + q * 16 + j] = macc[q][rr];
        }
    }
    lds_barrier();
    const int slot = w - sk_owner(nb * KB, a.U, a.G);
    float* dst = a.part + ((int64_t)nb * a.slots + slot) * m * 128;
    for (int idx = threadIdx.x; idx < m * 128; idx += 256) {
      float s = red[idx];
      s += red[m * 128 + idx];
      s += red[2 * m * 128 + idx];
      s += red[3 * m * 128 + idx];
      store_coherent(dst + idx, s);
    }
    lds_barrier();
    clear_acc();
  };

  for (int base = 0; base < iters; base += PF) {
#pragma unroll
    for (int s = 0; s < PF; ++s) {
      const int it = base + s;
      if (it < iters) {
        const int ui = it >> 1;
        const int ktl = wave + 4 * (it & 1);
        const uint32_t spill = spill_from_next(ring[s][0]);
        uint32_t wp[16];
        decode_rowpair<K>(ring[s], spill, wp);
        if constexpr (DOT) {
          const half2_t xp = *reinterpret_cast<const half2_t*>(xs + (size_t)ui * 128 + ktl * 16 + 2 * p);
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
          if (j < m)
            av = *reinterpret_cast<const half4_t*>(xs + ((size_t)ui * m + j) * 128 + ktl * 16 + 4 * g);
#pragma unroll
          for (int q = 0; q < 8; ++q) {
            const uint32_t b0 = tr[(q * 8 + 2 * g) * 20 + j];
            const uint32_t b1 = tr[(q * 8 + 2 * g + 1) * 20 + j];
            const half4_t bv = __builtin_bit_cast(half4_t, make_uint2(b0, b1));
            macc[q] = __builtin_amdgcn_mfma_f32_16x16x16f16(av, bv, macc[q], 0, 0, 0);
          }
          __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
          __builtin_amdgcn_wave_barrier();
          __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
        }
        // segment end: last k tile pair of the last unit of an n block in the run
        if (it & 1) {
          const int64_t u = u0 + ui;
          if (u + 1 == u1 || (u + 1) % KB == 0) flush(u / KB);
        }
      }
      // refill the slot (unconditionally, so every step issues exactly one
      // load and the wait counts stay static); past the end, re-read the last
      // tile, a cache hit
      const int nxt = (it + PF < iters) ? it + PF : iters - 1;
      load_rowpair<K>(tile_ptr(nxt), ring[s]);
    }
  }

  // ---- 4. arrivals, then the finishing step of completed n blocks
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the coherent stores are done
  __syncthreads();
  const int64_t nb_last = (u1 - 1) / KB;
  const int nseg = (int)(nb_last - nb_first + 1);
  if (threadIdx.x < nseg) {
    const int64_t nb = nb_first + threadIdx.x;
    const int arrivals = sk_owner((nb + 1) * KB - 1, a.U, a.G) - sk_owner(nb * KB, a.U, a.G) + 1;
    const unsigned int old =
        __hip_atomic_fetch_add(a.ctr + nb, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    last_flags[threadIdx.x] = (old + 1u == (unsigned int)arrivals) ? arrivals : 0;
  }
  __syncthreads();
  for (int sg = 0; sg < nseg; ++sg) {
    const int arrivals = last_flags[sg];
    if (!arrivals) continue;
    const int64_t nb = nb_first + sg;
    const int col = (int)nb * 128 + 2 * lane;
    const float* src = a.part + (int64_t)nb * a.slots * m * 128;
    for (int i = wave; i < m; i += 4) {
      // all slot loads first (they go to the coherence point), then the sum
      // in slot order
      float v0[kSkMaxSlots], v1[kSkMaxSlots];
#pragma unroll
      for (int s = 0; s < kSkMaxSlots; ++s) {
        if (s < arrivals) {
          v0[s] = load_coherent(src + ((int64_t)s * m + i) * 128 + 2 * lane);
          v1[s] = load_coherent(src + ((int64_t)s * m + i) * 128 + 2 * lane + 1);
        }
      }
      float x0 = 0.f, x1 = 0.f;
#pragma unroll
      for (int s = 0; s < kSkMaxSlots; ++s) {
        if (s < arrivals) {
          x0 += v0[s];
          x1 += v1[s];
        }
      }
      fwht128_pair(x0, x1);
      const uint32_t svv = *reinterpret_cast<const uint32_t*>(a.svh + col);
      x0 *= kInvSqrt128 * h2f((uint16_t)(svv & 0xFFFF));
      x1 *= kInvSqrt128 * h2f((uint16_t)(svv >> 16));
      if (a.bias) {
        const uint32_t bv = *reinterpret_cast<const uint32_t*>(a.bias + col);
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
    if (threadIdx.x == 0) a.ctr[nb] = 0u;  // every arrival is in: ready for the next call
  }
}

}  // namespace exl3
