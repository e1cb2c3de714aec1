// Decode-GEMV kernel template of the grouped experts' small-batch path (one
// workgroup per (unit, 128 columns, k range); planning helpers in
// exl3_gemv.hip).  A resolver R supplies, per
// workgroup, the tensor, the activations and the partial-sum slice, and
// implements the finishing step that the last-arriving workgroup of an
// output group runs (split-k sum in a fixed order, output transform, ...):
// R::FinishPre holds what the finish reads that does not depend on the
// partial sums, loaded by every workgroup during its k range
// (finish_prefetch), and R::finish runs on all the finisher's waves.
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
  int bits;                 // width of the tensor, read when the kernel's K is 0
};

constexpr size_t kGemvMaxLds = 64 * 1024;
// Waves of a workgroup (NW below): wave w takes the k tiles w, w + NW, ... of
// its range.  A grid of at most kGemvWideGrid workgroups (two per CU) runs
// eight waves, which halves each wave's serial chain of tiles (what a small
// call waits for); larger grids run four, where eight cost occupancy.
// Measured on MI355X, routed experts 256 x (2048 -> 2 x 512 -> 2048), K=3,
// top-8 (both launches per call): T=1 20.9 us against 22.2 with four waves
// everywhere, T=2 22.3 against 25.0, T=4 31.6 against 33.2; with eight waves
// for every grid T=8 took 52.0 against 48.7 and T=48 220 against 194.
constexpr int kGemvMaxWaves = 8;
constexpr int kGemvWideGrid = 512;
inline int gemv_waves(int grid) { return grid <= kGemvWideGrid ? 8 : 4; }
constexpr int kGemvTargetWorkgroups = 256;
constexpr int kGemvMaxKc = 1024;  // longest k range of one workgroup in small grids

size_t gemv_lds_bytes(int kc, int m, int nw = kGemvMaxWaves);
int gemv_choose_splits(int k, int groups, int m, int target_wgs);
int gemv_prefetch(int kc, int nw = 4);

// ---------------------------------------------------------------------------
// prologue: x' = (x .* suh) H over the workgroup's k range into LDS, layout
// xs[kt][i][16] (k tile, activation row, 16 k values) as fp16.
// ---------------------------------------------------------------------------
template <int NW>
__device__ __forceinline__ void gemv_prologue(const GemvTask& T, int k0, int kc, uint16_t* xs) {
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int kblocks = kc >> 7;
  const int m = T.m;
  for (int task = wave; task < kblocks * m; task += NW) {
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

// Workgroups are dispatched to the eight XCDs of MI355X round robin: within
// one launch, the workgroups b with the same b % 8 all run on one XCD
// (verified by reading the XCC_ID hardware register of every workgroup).
// Which XCD that is can change for the life of a process: once a second
// stream has run work, launches on the first one have been seen rotated by
// one XCD, every workgroup b on XCD (b + 7) % 8.  An output group's
// workgroups (all k ranges of all units that one finish reads) are given
// indices congruent mod 8, so they share one XCD and its L2 whatever the
// rotation, and the group's partial sums can be handed over without an L2
// write-back or invalidate.  Index b: residue x = b % 8, position i = b / 8;
// group 8 (i / members) + x, member i % members.
//
// The XCD a group is expected on is learned: its finisher records its own XCD
// in the group's arrival counter for the next call (see GemvCtr), and a group
// with no record yet expects XCD b % 8.  Every workgroup compares its XCC_ID
// with that expectation (gemv_off_xcd).  The partial sums are stored with
// device-scope stores and read with device-scope loads whatever the
// placement; a workgroup found on another XCD (or every workgroup, when the
// caller forces it) also takes the device-scope release before it arrives and
// marks its arrival, and the finisher of a marked group, or one that is
// itself off the expected XCD, takes the device-scope acquire.  A placement
// that differs from the expectation then costs time, not correctness, for
// one call.
constexpr int kGemvXcds = 8;

// Arrival counter word of an output group: bits 0..13 count the arrivals,
// bits 14..27 count the arrivals that took the device-scope release, bits
// 28..31 hold 1 + the XCD the group was finished on in the previous call (0:
// none).  The finisher stores the record, count fields zero, for the next
// call.  Groups have at most kMaxArrivals members (checked on the host).
struct GemvCtr {
  static constexpr unsigned int kCountMask = (1u << 14) - 1u;
  static constexpr unsigned int kOffOne = 1u << 14;
  static constexpr unsigned int kOffMask = ((1u << 14) - 1u) << 14;
  static constexpr int kXcdShift = 28;
  static constexpr int kMaxArrivals = (1 << 14) - 1;
};

// XCC_ID hardware register (bits 3:0: the XCD this wave runs on)
__device__ __forceinline__ int xcc_id() {
  return __builtin_amdgcn_s_getreg((3 << 11) | 20) & 15;  // hwreg(HW_REG_XCC_ID, 0, 4)
}
// rec: the record field of the group's counter word (0: none)
__device__ __forceinline__ bool gemv_off_xcd(int b, unsigned int rec, int force) {
  const int expect = rec ? (int)rec - 1 : b % kGemvXcds;
  return force != 0 || xcc_id() != expect;
}
__device__ __forceinline__ bool gemv_place(int b, int groups, int members, int& group, int& member) {
  const int x = b % kGemvXcds, i = b / kGemvXcds;
  group = (i / members) * kGemvXcds + x;
  member = i - (i / members) * members;
  return group < groups;
}
inline int gemv_grid(int groups, int members) {
  return (groups + kGemvXcds - 1) / kGemvXcds * kGemvXcds * members;
}

// One k tile of one wave: decode the lane's row pair, hand the k-pairs to the
// matrix cores through the wave's LDS transpose region, accumulate.
template <int K>
__device__ __forceinline__ void gemv_tile(const uint32_t (&D)[K], int kt, int m, const uint16_t* xs,
                                          uint32_t* tr, uint32_t* my, int g, int j,
                                          float4_t (&acc)[8]) {
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

// One unit's k range, its partial store and its arrival; last_flag (shared,
// valid after the final barrier) is 0, or 1 / 2 for the group's last arrival
// (2: the finish takes the device-scope acquire).  PF = loads kept in flight
// per lane; the per-wave trip count kc/64 must be a multiple of PF (the
// planner guarantees it), so the loop has no tail and no branch around its
// loads.
template <int K, int PF, int NW, class R>
__device__ __forceinline__ void gemv_unit(const R& r, const GemvTask& T, int unit, int split, int nb,
                                          int n, int kc, unsigned char* smem, int& last_flag,
                                          typename R::FinishPre& pre) {
  const int m = T.m;
  const int k0 = split * kc;
  const int nt = n >> 4;
  uint16_t* xs = reinterpret_cast<uint16_t*>(smem);
  const size_t xs_bytes = ((size_t)kc * m * 2 + 15) & ~(size_t)15;
  uint32_t* tr_all = reinterpret_cast<uint32_t*>(smem + xs_bytes);
  float* red = reinterpret_cast<float*>(smem + xs_bytes);

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int t = lane >> 3, p = lane & 7;    // decode role: n-tile, row pair
  const int g = lane >> 4, j = lane & 15;   // MFMA role: k group, row/column
  uint32_t* tr = tr_all + wave * (64 * 20);
  uint32_t* my = tr + (t * 8 + p) * 20;

  // wave w handles k tiles w, w + NW, ... of the range; iteration it -> tile
  // w + NW it
  const uint32_t* tbase = reinterpret_cast<const uint32_t*>(T.trellis) +
                          ((int64_t)((k0 >> 4) + wave) * nt + nb * 8 + t) * (8 * K) + K * p;
  const int64_t it_stride = (int64_t)NW * nt * (8 * K);
  const int cnt = kc / (16 * NW);

  // the group's XCD record (constant during the call: arrivals change only
  // the count fields, and the finisher rewrites it after every arrival),
  // read first so that its latency hides behind the whole unit
  unsigned int* const ctr = r.counter(unit, nb);
  const unsigned int rec =
      __hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >> GemvCtr::kXcdShift;

  // the first PF trellis loads go out before the prologue so that their
  // latency overlaps the input transform
  uint32_t ring[PF][K];
#pragma unroll
  for (int s = 0; s < PF; ++s) load_rowpair<K>(tbase + s * it_stride, ring[s]);

  gemv_prologue<NW>(T, k0, kc, xs);
  __syncthreads();
  // what the finish needs besides the partial sums, in case this workgroup
  // arrives last: issued after the input transform (which waits for its own
  // loads) so that its latency hides behind the k range instead
  pre = r.finish_prefetch(unit, nb);

  float4_t acc[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) acc[q] = float4_t{0.f, 0.f, 0.f, 0.f};

  for (int base = 0; base < cnt; base += PF) {
#pragma unroll
    for (int s = 0; s < PF; ++s) {
      const int it = base + s;
      gemv_tile<K>(ring[s], wave + NW * it, m, xs, tr, my, g, j, acc);
      // refill the slot just consumed (same registers, so no copy and no wait
      // at the loop edge); the last block re-reads the final tile, a cache
      // hit, instead of branching
      const int nxt = (it + PF < cnt) ? (it + PF) : (cnt - 1);
      load_rowpair<K>(tbase + nxt * it_stride, ring[s]);
    }
  }

  // fixed-order reduction of the waves' partials (wave order)
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
  for (int idx = threadIdx.x; idx < m * 128; idx += 64 * NW) {
    const int i = idx >> 7, c = idx & 127;
    float s = red[i * 128 + c];
#pragma unroll
    for (int w = 1; w < NW; ++w) s += red[(w * m + i) * 128 + c];
    __hip_atomic_store(T.partial + (int64_t)i * n + nb * 128 + c, s, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
  }

  // arrival: the last workgroup of the output group finishes it.  Every
  // thread's partial stores are complete (vmcnt(0)) before the workgroup
  // barrier, and the counter moves after it.  Off the expected XCD, the
  // device-scope release comes first and the arrival is marked.
  const bool off = gemv_off_xcd((int)blockIdx.x, rec, r.off_xcd_all);
  if (off)
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
  else
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  __syncthreads();
  if (threadIdx.x == 0) {
    const unsigned int inc = off ? 1u + GemvCtr::kOffOne : 1u;
    const unsigned int now = __hip_atomic_fetch_add(ctr, inc, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + inc;
    const bool last = (now & GemvCtr::kCountMask) == r.arrivals(unit);
    last_flag = !last ? 0 : (((now & GemvCtr::kOffMask) != 0 || off) ? 2 : 1);
  }
  __syncthreads();
}

// The finish of an output group, run by its last-arriving workgroup (one copy
// for every width of a width-0 kernel).
template <class R>
__device__ __forceinline__ void gemv_group_finish(const R& r, int unit, int nb, int n, int last_flag,
                                                  const typename R::FinishPre& pre, unsigned char* smem) {
  if (last_flag == 2)
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  else
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
  r.finish(unit, nb, n, pre, smem);
  if (threadIdx.x == 0)  // counts zero and this XCD recorded, for the next call
    __hip_atomic_store(r.counter(unit, nb), (unsigned int)(xcc_id() + 1) << GemvCtr::kXcdShift,
                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// K = 1..8: every unit has that width.  K = 0: each unit has its own width
// (T.bits, a width per expert), all of them in one launch.
template <int K, int PF, int NW, class R>
__global__ __launch_bounds__(64 * NW) void gemv_kernel(R r, int /*k*/, int n, int kc) {
  extern __shared__ __align__(16) unsigned char smem[];
  __shared__ int last_flag;
  typename R::FinishPre pre;
  int unit, split, nb;
  if (!r.place((int)blockIdx.x, unit, split, nb)) return;  // uniform over the workgroup
  const GemvTask T = r.task(unit, split);
  if (!T.valid) return;
  if constexpr (K == 0) {
    switch (T.bits) {
      case 1: gemv_unit<1, PF, NW>(r, T, unit, split, nb, n, kc, smem, last_flag, pre); break;
      case 2: gemv_unit<2, PF, NW>(r, T, unit, split, nb, n, kc, smem, last_flag, pre); break;
      case 3: gemv_unit<3, PF, NW>(r, T, unit, split, nb, n, kc, smem, last_flag, pre); break;
      case 4: gemv_unit<4, PF, NW>(r, T, unit, split, nb, n, kc, smem, last_flag, pre); break;
      case 5: gemv_unit<5, PF, NW>(r, T, unit, split, nb, n, kc, smem, last_flag, pre); break;
      case 6: gemv_unit<6, PF, NW>(r, T, unit, split, nb, n, kc, smem, last_flag, pre); break;
      case 7: gemv_unit<7, PF, NW>(r, T, unit, split, nb, n, kc, smem, last_flag, pre); break;
      case 8: gemv_unit<8, PF, NW>(r, T, unit, split, nb, n, kc, smem, last_flag, pre); break;
      default: return;  // a width outside 1..8: the unit is left out
    }
  } else {
    gemv_unit<K, PF, NW>(r, T, unit, split, nb, n, kc, smem, last_flag, pre);
  }
  if (last_flag) gemv_group_finish(r, unit, nb, n, last_flag, pre, smem);
}

// Launch with the waves the grid size calls for and the prefetch depth the k
// range allows.
template <int K, int NW, class R>
void launch_gemv_nw(const R& r, dim3 grid, int m, hipStream_t s, int k, int n, int kc) {
  const dim3 block(64 * NW);
  const size_t lds = gemv_lds_bytes(kc, m, NW);
  switch (gemv_prefetch(kc, NW)) {
    case 8: hipLaunchKernelGGL((gemv_kernel<K, 8, NW, R>), grid, block, lds, s, r, k, n, kc); break;
    case 4: hipLaunchKernelGGL((gemv_kernel<K, 4, NW, R>), grid, block, lds, s, r, k, n, kc); break;
    case 2: hipLaunchKernelGGL((gemv_kernel<K, 2, NW, R>), grid, block, lds, s, r, k, n, kc); break;
    default: hipLaunchKernelGGL((gemv_kernel<K, 1, NW, R>), grid, block, lds, s, r, k, n, kc); break;
  }
}
template <int K, class R>
hipError_t launch_gemv_kernel(const R& r, dim3 grid, int m, hipStream_t s, int k, int n, int kc) {
  if (gemv_waves((int)grid.x) == 8)
    launch_gemv_nw<K, 8>(r, grid, m, s, k, n, kc);
  else
    launch_gemv_nw<K, 4>(r, grid, m, s, k, n, kc);
  return hipGetLastError();
}

}  // namespace exl3
