// Persistent decode GEMV for 1..16 activation rows on the matrix cores (dense
// EXL3 linear).
//
// One contraction for every row count.  The decoded weights go straight into
// the B operand of v_mfma_f32_16x16x16_f16, in registers: lane l = 16 g + T
// decodes rows 4g .. 4g+3 of n tile T (four consecutive trellis rows, a
// contiguous 64K-bit stretch of the tile's stream, plus the first dword of the
// next row quad for the windows that run past it), which is exactly the
// operand's lane layout (lane l holds k = 4 (l / 16) .. + 3 of column l % 16).
// The unit's 16 tiles are loaded with whole cache lines (load_halves) and
// each lane's quad assembled with one DPP move per dword (quad_assemble).
// Sixteen n tiles make one unit of work: a k tile (16 rows of k) of a
// 256-column pair of Hadamard blocks, sixteen MFMAs, one per column q of the
// tiles.  Activation row i of the A operand is x'[i][16 kt + 4 g .. + 3]; rows
// past m are zero.  Each output element is the sum of its own row's products
// only, in an order fixed by the plan, so a row's result does not depend on m.
//
// Decomposition: the R = (n/256 rounded up) * (k/16) units are ordered
// pair-major and split into contiguous runs, one per workgroup of a grid that
// is resident at once (stream-k at workgroup granularity, SkSplit, in two
// tiers: the workgroups dispatched first, the older of the two on each CU,
// take longer runs).  Wave w of a workgroup takes units w, w + 4, ... of the
// run and ends a segment at each pair boundary of the run and at its end:
// its column sums for the pair, s_w = (b x' summed) - 1534 (x' summed) (the
// second sum from a seventeenth MFMA against ones), zero for a wave without
// units in the pair.  The workgroup's term for the pair is
// t = ((s_0 + s_1) + s_2) + s_3 and the pair's column sums are the terms of
// its workgroups added in a fixed order by the finishing launch, which then
// applies the output transform, the codebook scale, svh and bias.
//
// Where t is formed depends on m, its value does not: for m <= kMfLdsRows
// each wave stores s_w to a slot of its own and the finish forms t (the
// waves never wait for each other); above, the four waves meet in LDS at each
// segment end and the workgroup stores t (a quarter of the partial traffic).
//
// x': for m <= kMfLdsRows the four waves transform the k blocks the
// workgroup's run touches into one LDS region of the workgroup, a round of
// four blocks each, then meet at one workgroup barrier (a region per wave,
// each wave transforming every block, made m = 2 and 4 calls 0.8 and 1.3 us
// longer on 5120 x 17408); above, one input-transform launch
// (gemv_xprep_kernel) writes x' for all rows first and the A fragments are
// loaded with the trellis.  Both compute x' with the same function (xform8),
// so a row's x' is the same bits either way.
#pragma once

#include "exl3_device.hpp"
#include "exl3_sk_split.hpp"

namespace exl3 {

constexpr int kMfWorkgroups = 512;  // two workgroups of four waves per CU of the 256-CU MI355X
constexpr int kMfRoundWorkgroups = 256;  // the first dispatch round: one per CU
// Tensors of at most kMfRoundWorkgroups x kMfSmallRun units take one
// workgroup per CU (kMfRoundWorkgroups, one tier) instead of kMfWorkgroups.
constexpr int kMfSmallRun = 50;
// Relative run lengths of the first-round workgroups (the older of the two on
// a CU, which wins the instruction arbiter) and the others.
constexpr int kMfTierWeight1 = 13;
constexpr int kMfTierWeight2 = 7;
constexpr int kMfMaxRunWG = 80;    // longest run of units of a workgroup (bounds the LDS x' region)
constexpr int kMfLdsRows = 4;      // rows whose x' the workgroup stages in LDS itself
constexpr int kMfXBlocks = 12;     // k blocks a workgroup's run may touch
constexpr int kMfXRowBytes = kMfXBlocks * 128 * 2;  // LDS x' bytes per row
constexpr int kMfGroupBatch = 8;   // workgroup slots per lane loaded per batch in the finish

// the x' positions read (one unit ahead of the last) stay inside the region
static_assert(7 + kMfMaxRunWG - 1 + 4 < kMfXBlocks * 8, "run touches too many k blocks");
static_assert(kMfXBlocks % 4 == 0, "transform rounds of four blocks");

struct MfArgs {
  const uint16_t* trellis;  // [k/16][n/16][16K]
  const uint16_t* suh;      // fp16 [k]
  const uint16_t* x;        // fp16 [m][ldx]
  int64_t ldx;
  const uint16_t* xprep;    // fp16 [m][k] already transformed (m > kMfLdsRows), else nullptr
  int m;
  int k, n;
  int KT;                   // k / 16
  int NP;                   // 256-column pairs (the last one half when n / 128 is odd)
  int R;                    // units = NP * KT
  int W;                    // workgroups of the grid
  SkSplit sp;               // runs of the workgroups
  int slots;                // workgroup slots per pair
  float* part;              // fp32 [NP][slots][4 (m <= kMfLdsRows) or 1][m][256]
  const uint16_t* svh;
  const uint16_t* bias;
  void* y;
  int64_t ldy;
  int y_f32;
};

// x' = ((x .* s) H) / sqrt(128) for the eight consecutive elements a lane
// holds in the fwht128_x8 layout (16 lanes per 128-element block), packed to
// fp16.  The waves' own transform and the input-transform launch both call
// this one function, so they round alike: the compiler turns the scale and
// the fp16 conversion into one multiply with a single rounding
// (v_fma_mixlo_f16), which differs now and then from an fp32 multiply
// followed by a separate conversion (the standalone Hadamard kernel's way).
__device__ __forceinline__ uint4 xform8(const uint4& xv, const uint4& sv) {
  const uint32_t xw[4] = {xv.x, xv.y, xv.z, xv.w};
  const uint32_t sw[4] = {sv.x, sv.y, sv.z, sv.w};
  float v[8];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    v[2 * e] = h2f((uint16_t)(xw[e] & 0xFFFF)) * h2f((uint16_t)(sw[e] & 0xFFFF));
    v[2 * e + 1] = h2f((uint16_t)(xw[e] >> 16)) * h2f((uint16_t)(sw[e] >> 16));
  }
  fwht128_x8(v);
  uint32_t o[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float a = v[2 * e] * kInvSqrt128;
    const float b = v[2 * e + 1] * kInvSqrt128;
    o[e] = (uint32_t)f2h(a) | ((uint32_t)f2h(b) << 16);
  }
  return make_uint4(o[0], o[1], o[2], o[3]);
}

// The funnel-shift amounts 32 - o (o = 1..15) as values the compiler cannot
// see through.  A window that starts o bits into stream dword i is
// alignbit(B[i], B[i+1], 32 - o): its high half is the state at offset o and
// its low half the state 16 bits later, and both hashes select their half
// with the multiply's SDWA operand.  With a constant shift the compiler
// rewrites the high half's extraction as a bit-field extract of one dword,
// which no longer shares the funnel shift and costs an extra instruction per
// state pair.
struct WindowShifts {
  uint32_t s[16];
  __device__ __forceinline__ WindowShifts() {
#pragma unroll
    for (int o = 0; o < 16; ++o) {
      uint32_t v = 32u - (uint32_t)o;
      asm volatile("" : "+s"(v));
      s[o] = v;
    }
  }
};

// Hash of the state that starts at bit P of the stream held in the
// stream-ordered dwords B[0 .. N-1].
template <int N, int P>
__device__ __forceinline__ uint32_t quad_hash(const uint32_t (&B)[N], const WindowShifts& ws, uint32_t mult) {
  constexpr int i = P / 32;
  constexpr int o = P % 32;
  constexpr int o16 = o & 15;
  static_assert(i + (o16 ? 1 : 0) < N, "state past the loaded stream");
  uint32_t w;
  if constexpr (o16 == 0)
    w = B[i];
  else
    w = __builtin_amdgcn_alignbit(B[i], B[i + 1], ws.s[o16]);
  // the half's extraction folds into the multiply's SDWA operand selector
  if constexpr (o < 16)
    return __umul24(w >> 16, mult);
  else
    return __umul24(w & 0xFFFFu, mult);
}

// Biased codes b = 1024 + sigma of column C of the lane's row quad, as the
// MFMA B fragment {rows 4g, 4g+1} (lo) and {4g+2, 4g+3} (hi).
template <int K, int C>
__device__ __forceinline__ void quad_column(const uint32_t (&B)[2 * K + 1], const WindowShifts& ws,
                                            uint32_t mult, uint32_t& lo, uint32_t& hi) {
  const uint32_t h0 = quad_hash<2 * K + 1, K * C>(B, ws, mult);
  const uint32_t h1 = quad_hash<2 * K + 1, K * (16 + C)>(B, ws, mult);
  const uint32_t h2 = quad_hash<2 * K + 1, K * (32 + C)>(B, ws, mult);
  const uint32_t h3 = quad_hash<2 * K + 1, K * (48 + C)>(B, ws, mult);
  lo = __builtin_amdgcn_sad_hi_u8(h1, 0u, __builtin_amdgcn_sad_u8(h0, 0u, kHalf1024Pair));
  hi = __builtin_amdgcn_sad_hi_u8(h3, 0u, __builtin_amdgcn_sad_u8(h2, 0u, kHalf1024Pair));
}

// One unit: decode the sixteen columns and run their MFMAs (plus the one
// against ones that sums x').
template <int K, int C = 0>
__device__ __forceinline__ void quad_mfmas(const uint32_t (&B)[2 * K + 1], const WindowShifts& ws,
                                           const half4_t& av, float4_t (&acc)[16]) {
  if constexpr (C < 16) {
    uint32_t lo, hi;
    quad_column<K, C>(B, ws, kMul1Multiplier, lo, hi);
    const half4_t bv = __builtin_bit_cast(half4_t, make_uint2(lo, hi));
    acc[C] = __builtin_amdgcn_mfma_f32_16x16x16f16(av, bv, acc[C], 0, 0, 0);
    quad_mfmas<K, C + 1>(B, ws, av, acc);
  }
}

// Loading a unit (16 tiles of 32K bytes, contiguous) with whole cache lines:
// the first load covers tiles 0..7 and the second tiles 8..15, each tile by
// the 8 lanes (g, t) and (g, t + 8), g = 0..3, which take the first and the
// second half (4K bytes) of row quad g.  Lane (g, T) therefore receives
// half T / 8 of quad g of tile T % 8 (first load) and of tile 8 + T % 8
// (second load); its own quad's missing half sits in lane T ^ 8 and one DPP
// rotation by 8 inside the row of 16 lanes moves it over (quad_assemble).
template <int K>
__device__ __forceinline__ void load_halves(__amdgpu_buffer_rsrc_t rs, uint32_t off1, uint32_t off2,
                                            uint32_t soff, uint32_t (&D)[2 * K]) {
  uint32_t (&R1)[K] = *reinterpret_cast<uint32_t(*)[K]>(&D[0]);
  uint32_t (&R2)[K] = *reinterpret_cast<uint32_t(*)[K]>(&D[K]);
  load_rowpair_buf<K>(rs, off1, soff, R1);
  load_rowpair_buf<K>(rs, off2, soff, R2);
}

// D = {R1, R2} as loaded -> the lane's quad as stream-ordered dwords B[0 .. 2K-1]
// (first half, second half) and B[2K], the first dword of the next row quad
// of the same tile (lane 16 ((g + 1) % 4) + T after the assembly).
constexpr int kDppRor8 = 0x128;  // row_ror:8: lane l takes lane l ^ 8 in each row of 16
template <int K>
__device__ __forceinline__ void quad_assemble(const uint32_t (&D)[2 * K], int spill_src, uint32_t (&B)[2 * K + 1]) {
#pragma unroll
  for (int i = 0; i < K; ++i) {
    // lanes T >= 8 (banks 2, 3) take their first half from lane T - 8's second load
    const uint32_t first =
        (uint32_t)__builtin_amdgcn_update_dpp((int)D[i], (int)D[K + i], kDppRor8, 0xF, 0xC, false);
    // lanes T < 8 (banks 0, 1) take their second half from lane T + 8's first load
    const uint32_t second =
        (uint32_t)__builtin_amdgcn_update_dpp((int)D[K + i], (int)D[i], kDppRor8, 0xF, 0x3, false);
    B[i] = first;
    B[K + i] = second;
  }
  const uint32_t spill = (uint32_t)__builtin_amdgcn_ds_bpermute(spill_src, (int)B[0]);
#pragma unroll
  for (int i = 0; i < 2 * K; ++i) B[i] = stream_dword(B[i]);
  B[2 * K] = stream_dword(spill);
}

// Finish of (activation row i, 128-column block nb), by one wave: block nb is
// half nb % 2 of pair nb / 2.  Lane l owns columns 8 (l % 16) .. + 7 of the
// block and adds the pair's workgroup terms t_g for g = l / 16, l / 16 + 4,
// ... in that order (WS: t_g = ((s_0 + s_1) + s_2) + s_3 from the four wave
// slots of workgroup g; else the workgroup stored t_g); the four lane groups'
// sums are combined as (u0 + u1) + (u2 + u3).  Then the output transform
// (three in-lane butterfly stages, four lane swizzles in each group of 16
// lanes), the codebook scale with the transform's normalisation, svh and
// bias; lanes 0..15 store.
template <bool WS>
__device__ __forceinline__ void mf_finish(const MfArgs& a, int i, int nb) {
  constexpr int NW = WS ? 4 : 1;        // slots per workgroup term
  constexpr int GB = WS ? 4 : kMfGroupBatch;  // terms per lane per batch
  const int m = a.m;
  const int lane = (int)(threadIdx.x & 63);
  const int c8 = 8 * (lane & 15);
  const int sg = lane >> 4;
  const int col = nb * 128 + c8;
  const int p = nb >> 1;
  const int groups = sk_arrivals(a.sp, p, a.KT);
  const float* src = a.part + ((int64_t)p * a.slots * NW * m + i) * 256 + 128 * (nb & 1) + c8;
  const int64_t gstride = (int64_t)NW * m * 256;  // floats between workgroup terms
  const uint4 svv = *reinterpret_cast<const uint4*>(a.svh + col);
  uint4 bv = make_uint4(0, 0, 0, 0);
  if (a.bias) bv = *reinterpret_cast<const uint4*>(a.bias + col);
  float4_t ulo = {0.f, 0.f, 0.f, 0.f}, uhi = {0.f, 0.f, 0.f, 0.f};
  for (int g0 = sg; g0 < groups; g0 += 4 * GB) {
    float4_t lo[GB][NW], hi[GB][NW];
#pragma unroll
    for (int q = 0; q < GB; ++q)
      if (g0 + 4 * q < groups) {
#pragma unroll
        for (int w = 0; w < NW; ++w) {
          const float4_t* p4 = reinterpret_cast<const float4_t*>(src + (g0 + 4 * q) * gstride + (int64_t)w * m * 256);
          lo[q][w] = p4[0];
          hi[q][w] = p4[1];
        }
      }
#pragma unroll
    for (int q = 0; q < GB; ++q)
      if (g0 + 4 * q < groups) {
        float4_t tlo = lo[q][0], thi = hi[q][0];
#pragma unroll
        for (int w = 1; w < NW; ++w) {
          tlo += lo[q][w];
          thi += hi[q][w];
        }
        ulo += tlo;
        uhi += thi;
      }
  }
  float v[8] = {ulo[0], ulo[1], ulo[2], ulo[3], uhi[0], uhi[1], uhi[2], uhi[3]};
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] += swizzle_xor_f<16>(v[e]);
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] += shfl_xor_f(v[e], 32);
  fwht128_x8(v);
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

// LDS of one workgroup: XR > 0, a region of XR rows of x' shared by the
// waves; XR = 0, the combine buffer (a row block of 256 floats per wave and
// row).
template <int XR>
struct MfLds {
  static constexpr int kXBytes = XR * kMfXRowBytes;
  static constexpr int kCombineBytes = XR > 0 ? 0 : 4 * 16 * 256 * 4;
  static constexpr int kBytes = XR > 0 ? kXBytes : kCombineBytes;
};

// The work of workgroup `wg`: the units [r0, r0 + len) of its run, wave w
// taking units r0 + w, r0 + w + 4, ...  XR = rows whose x' the workgroup
// stages in LDS itself (1 or kMfLdsRows; the waves store their own slots), or
// 0: x' comes from the input-transform launch and the workgroup combines its
// waves' sums in LDS.
template <int K, int XR>
__device__ __forceinline__ void mf_wg(const MfArgs& a, int wg, unsigned char* smem) {
  constexpr bool LDSX = XR > 0;
  const int len = sk_run_len(a.sp, wg);
  if (len <= 0) return;  // uniform over the workgroup
  const int r0 = sk_run_start(a.sp, wg);
  const int m = a.m;
  const int KT = a.KT;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int lane = threadIdx.x & 63;
  const int g = lane >> 4, T = lane & 15;  // decode: row quad, n tile of the pair
  const int j = lane & 15;                 // A operand: activation row
  unsigned char* xl = smem;  // the workgroup's x' region
  float* cbuf = reinterpret_cast<float*>(smem);          // combine buffer (XR == 0)

  const int p_first = r0 / KT;
  const int kt0 = r0 - p_first * KT;
  const int p_last = (r0 + len - 1) / KT;
  const int slot0 = wg - sk_run_owner(a.sp, p_first * KT);
  const int nw = len > wave ? (len - wave + 3) >> 2 : 0;  // this wave's units

  // Trellis addressing: one buffer descriptor per pair covers its k range; a
  // unit is a uniform offset (kt * bytes of a k-tile row) plus the lane's
  // offsets of its two loads (load_halves).  In a half pair (the last one
  // when n / 128 is odd) the second load re-reads tiles 0..7: the lanes
  // T >= 8 compute columns that are never stored.
  constexpr int kTileBytes = 32 * K;
  constexpr int kPairBytes = 16 * kTileBytes;
  const int NT = a.n >> 4;
  const uint32_t kt_bytes = (uint32_t)NT * kTileBytes;  // whole tensor < 2^32 B
  const uint32_t col_bytes = (uint32_t)(KT - 1) * kt_bytes + kPairBytes;
  const uint32_t half_off = (uint32_t)((T & 7) * kTileBytes + 8 * K * g + 4 * K * (T >> 3));
  const uint32_t off2_full = half_off + 8 * kTileBytes;
  const int spill_src = (16 * ((g + 1) & 3) + T) << 2;  // bpermute byte address of the next quad's lane
  const unsigned char* tr0 = reinterpret_cast<const unsigned char*>(a.trellis);
  auto off2_of = [&](int p) { return (16 * p + 8 < NT) ? off2_full : half_off; };
  // prefetch state: the wave's unit r0 + wave + 4 i, as (pair, k tile)
  int pf_p = (r0 + wave) / KT;
  int pf_kt = r0 + wave - pf_p * KT;
  int pf_left = nw;  // units of the wave not yet requested
  uint32_t pf_soff = (uint32_t)pf_kt * kt_bytes;
  __amdgpu_buffer_rsrc_t pf_rs = make_rsrc(tr0 + (int64_t)pf_p * kPairBytes, col_bytes);
  uint32_t pf_off2 = off2_of(pf_p);
  // Loads past the wave's last unit go through a descriptor of no bytes:
  // every access is out of range, returns zero and reaches no cache, and the
  // loop still issues the same loads every step (static wait counts).
  const __amdgpu_buffer_rsrc_t null_rs = make_rsrc(tr0, 0u);
  // XR == 0: the A fragment of a unit, x'[j][16 kt + 4 g .. + 3]
  __amdgpu_buffer_rsrc_t x_rs = make_rsrc(a.xprep, LDSX ? 0u : (uint32_t)m * a.k * 2);
  const uint32_t x_voff = (uint32_t)(((j < m ? j : 0) * a.k + 4 * g) * 2);
  auto pf_load = [&](uint32_t (&D)[2 * K], uint2& A) {
    const bool live = pf_left > 0;  // uniform
    load_halves<K>(live ? pf_rs : null_rs, half_off, pf_off2, pf_soff, D);
    if constexpr (!LDSX) {
      typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
      const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(live ? x_rs : null_rs, (int)x_voff, pf_kt * 32, 0);
      A = make_uint2(v.x, v.y);
    }
  };
  auto pf_advance = [&]() {
    if (pf_left > 1) {
      pf_kt += 4;
      if (pf_kt >= KT) {  // k >= 128: at most one pair change per step
        pf_kt -= KT;
        ++pf_p;
        pf_rs = make_rsrc(tr0 + (int64_t)pf_p * kPairBytes, col_bytes);
        pf_off2 = off2_of(pf_p);
      }
      pf_soff = (uint32_t)pf_kt * kt_bytes;
    }
    if (pf_left > 0) --pf_left;
  };

  // ---- x' of rows < m staged by the workgroup: block b of the run is
  // (kt0 / 8 + b) mod k/128; wave rd takes round rd (rd = 0, 1, 2; wave 3
  // none), whose lane (g, j) loads 8 elements of run block 4 rd + g (rounds
  // past the run's blocks skipped).
  constexpr int XRD = kMfXBlocks / 4;
  const int nblk = ((kt0 & 7) + len + 7) >> 3;
  uint4 xv[LDSX ? XR : 1][LDSX ? XRD : 1], sv[LDSX ? XRD : 1];
  if constexpr (LDSX) {
    const int kb0 = kt0 >> 3, KBn = KT >> 3;
#pragma unroll
    for (int rd = 0; rd < XRD; ++rd) {
      if (rd == wave && 4 * rd < nblk) {  // uniform
        const int b = 4 * rd + g;
        const int bb = b < nblk ? b : nblk - 1;
        const int kk = ((kb0 + bb) % KBn) * 128 + 8 * j;
        sv[rd] = *reinterpret_cast<const uint4*>(a.suh + kk);
#pragma unroll
        for (int i = 0; i < XR; ++i)  // rows past m read row 0 (never used)
          xv[i][rd] = *reinterpret_cast<const uint4*>(a.x + (i < m ? i : 0) * a.ldx + kk);
      }
    }
  }

  constexpr int PF = 4;
  uint32_t ring[PF][2 * K];
  uint2 aring[PF];
#pragma unroll
  for (int s = 0; s < PF; ++s) {
    pf_load(ring[s], aring[s]);
    pf_advance();
  }

  if constexpr (LDSX) {
#pragma unroll
    for (int i = 0; i < XR; ++i) {
      if (i < m) {  // uniform
        uint16_t* xs = reinterpret_cast<uint16_t*>(xl + i * kMfXRowBytes);
#pragma unroll
        for (int rd = 0; rd < XRD; ++rd) {
          if (rd == wave && 4 * rd < nblk) {  // uniform
            const int b = 4 * rd + g;
            const uint4 o = xform8(xv[i][rd], sv[rd]);
            if (b < nblk) *reinterpret_cast<uint4*>(xs + b * 128 + 8 * j) = o;
          }
        }
      }
    }
    __syncthreads();  // every round written before any wave reads
  }

  // ---- main loop
  float4_t acc[16];
  float4_t xsum;  // sum of x' over the wave's units of the segment, per row (any column)
  auto clear_acc = [&]() {
#pragma unroll
    for (int q = 0; q < 16; ++q) acc[q] = float4_t{0.f, 0.f, 0.f, 0.f};
    xsum = float4_t{0.f, 0.f, 0.f, 0.f};
  };
  clear_acc();

  // Segment end (every wave, once per pair of the run, in pair order): lane
  // (g, T) holds rows 4g .. 4g+3 of pair columns 16 T .. 16 T + 15 of s_w.
  // XR > 0: the wave stores s_w to its own slot.  XR == 0: the four waves'
  // sums meet in LDS, are added in wave order and the workgroup stores t.
  auto combine = [&](int p, int slot) {
    if constexpr (LDSX) {
      float* dst = a.part + (((int64_t)p * a.slots + slot) * 4 + wave) * m * 256 + 16 * T;
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int i = 4 * g + rr;
        if (i < m) {
          float v[16];
#pragma unroll
          for (int q = 0; q < 16; ++q) v[q] = __builtin_fmaf(-kSigmaBiasPlus1024, xsum[rr], acc[q][rr]);
          float4* d4 = reinterpret_cast<float4*>(dst + i * 256);
#pragma unroll
          for (int q = 0; q < 4; ++q) d4[q] = make_float4(v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]);
        }
      }
    } else {
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int i = 4 * g + rr;
        if (i < m) {
          float v[16];
#pragma unroll
          for (int q = 0; q < 16; ++q) v[q] = __builtin_fmaf(-kSigmaBiasPlus1024, xsum[rr], acc[q][rr]);
          float4* d4 = reinterpret_cast<float4*>(cbuf + (wave * 16 + i) * 256 + 16 * T);
#pragma unroll
          for (int q = 0; q < 4; ++q) d4[q] = make_float4(v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]);
        }
      }
      __syncthreads();
      float* dst = a.part + ((int64_t)p * a.slots + slot) * m * 256;
      const int c = threadIdx.x;  // one pair column per thread
      for (int i = 0; i < m; ++i) {
        const float s01 = cbuf[(0 * 16 + i) * 256 + c] + cbuf[(1 * 16 + i) * 256 + c];
        const float s012 = s01 + cbuf[(2 * 16 + i) * 256 + c];
        dst[i * 256 + c] = s012 + cbuf[(3 * 16 + i) * 256 + c];
      }
      __syncthreads();
    }
    clear_acc();
  };

  // A fragment of the wave's unit i from LDS: x'[j][...] at byte
  // 32 (kt0 % 8 + wave + 4 i) + 8 g of row j's region (one k tile is 32
  // bytes of x'; the run's k blocks follow each other); rows past m are zero.
  // Read one unit ahead; the read after the last unit stays inside the
  // region (runs are at most kMfMaxRunWG units).
  const unsigned char* xlane = xl + (j < XR ? j : 0) * kMfXRowBytes + 32 * ((kt0 & 7) + wave) + 8 * g;
  const bool arow = j < m;
  const half4_t ones4 = {(_Float16)1.0f, (_Float16)1.0f, (_Float16)1.0f, (_Float16)1.0f};
  uint2 xnext = make_uint2(0, 0);
  if constexpr (LDSX) xnext = *reinterpret_cast<const uint2*>(xlane);
  const WindowShifts ws;
  int c_p = p_first, c_slot = slot0;
  int u_p = (r0 + wave) / KT;  // the wave's current unit, as (pair, k tile)
  int u_kt = r0 + wave - u_p * KT;
  for (int base = 0; base < nw; base += PF) {
#pragma unroll
    for (int s = 0; s < PF; ++s) {
      const int it = base + s;
      if (it < nw) {
        // segments the wave has moved past (possibly without units in them)
        while (c_p < u_p) {
          combine(c_p, c_slot);
          c_slot = 0;
          ++c_p;
        }
        uint32_t B[2 * K + 1];
        quad_assemble<K>(ring[s], spill_src, B);
        half4_t av = {0, 0, 0, 0};
        if constexpr (LDSX) {
          const uint2 xa = xnext;
          xnext = *reinterpret_cast<const uint2*>(xlane + 128 * (it + 1));
          if (arow) av = __builtin_bit_cast(half4_t, xa);
        } else {
          if (arow) av = __builtin_bit_cast(half4_t, aring[s]);
        }
        quad_mfmas<K>(B, ws, av, acc);
        xsum = __builtin_amdgcn_mfma_f32_16x16x16f16(av, ones4, xsum, 0, 0, 0);
        u_kt += 4;
        if (u_kt >= KT) {
          u_kt -= KT;
          ++u_p;
        }
      }
      // refill the slot (unconditionally: every step issues the same loads, so
      // the wait counts stay static); past the end, the empty descriptor
      pf_load(ring[s], aring[s]);
      pf_advance();
    }
  }
  while (c_p <= p_last) {
    combine(c_p, c_slot);
    c_slot = 0;
    ++c_p;
  }
}

template <int K, int XR>
__global__ __launch_bounds__(256) void gemv_mf_kernel(MfArgs a) {
  __shared__ __align__(16) unsigned char smem[MfLds<XR>::kBytes];
  mf_wg<K, XR>(a, (int)blockIdx.x, smem);
}

// x' of every row for m > kMfLdsRows, [m][k] fp16: wave task t covers row
// t / ceil(KB / 4) and four consecutive k blocks of it (lanes 16 g .. 16 g +
// 15 block g), with the arithmetic of the waves' own transform (xform8).
__global__ __launch_bounds__(256) void gemv_xprep_kernel(const uint16_t* __restrict__ x, int64_t ldx,
                                                         const uint16_t* __restrict__ suh, int m, int k,
                                                         uint16_t* __restrict__ out) {
  const int KB = k >> 7;
  const int per_row = (KB + 3) >> 2;
  const int task = (int)blockIdx.x * 4 + (int)(threadIdx.x >> 6);
  if (task >= m * per_row) return;  // whole waves leave together
  const int i = task / per_row;
  const int lane = (int)(threadIdx.x & 63);
  const int b = 4 * (task - i * per_row) + (lane >> 4);
  const int bb = b < KB ? b : KB - 1;  // lanes past the last block repeat it (not stored)
  const int kk = bb * 128 + 8 * (lane & 15);
  const uint4 xv = *reinterpret_cast<const uint4*>(x + (int64_t)i * ldx + kk);
  const uint4 sv = *reinterpret_cast<const uint4*>(suh + kk);
  const uint4 o = xform8(xv, sv);
  if (b < KB) *reinterpret_cast<uint4*>(out + (int64_t)i * k + kk) = o;
}

// One wave (a 64-thread workgroup, so the tasks spread over the CUs) per
// (activation row i, 128-column block nb).  WS: the waves stored their own
// slots (m <= kMfLdsRows).
template <bool WS>
__global__ __launch_bounds__(64) void gemv_mf_finish(MfArgs a) {
  const int NB = a.n >> 7;
  const int task = (int)blockIdx.x;
  const int i = task / NB;
  mf_finish<WS>(a, i, task - i * NB);
}

}  // namespace exl3
