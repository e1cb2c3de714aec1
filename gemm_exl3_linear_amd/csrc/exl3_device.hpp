// Device-side building blocks shared by every EXL3 kernel of this library
// (gfx950 / CDNA4, wave64).
//
// Format (exl3xpu README "MoE (routed experts)"; Arc 140V MoE post, section
// 2A; TensorFold issue #832 "Description"): a tensor's 16x16 tiles are stored
// as 16*K uint16 words, trellis[k/16][n/16][16*K].  The words of a tile, read
// in index order and most-significant bit first, form a cyclic stream of
// 256*K bits; state j is the 16-bit window starting at bit K*j; the mul1
// codebook maps state S to fp16_RN((sigma - 510) * 1775 / 2^18), sigma being
// the byte sum of (S * 0x9E3779) mod 2^32 (bounded by +-3.453125, exl3xpu
// README "Prefill: int8 linears ..."); state j is tile row j/16, column j%16.
//
// Work unit of the decode: one lane owns a *row pair* of a tile (rows 2p and
// 2p+1, p = 0..7): the 2K consecutive words 2K*p .. 2K*p+2K-1 plus the first
// word of the next row pair (the "spill" word, taken cyclically inside the
// tile).  Eight consecutive lanes own one tile, so a wave's loads of a run of
// tiles are contiguous.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace exl3 {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef float float2_t __attribute__((ext_vector_type(2)));

// Codebook constants of the mul1 reading (one definition each).
constexpr uint32_t kMul1Multiplier = 0x9E3779u;  // < 2^24: one v_mul_u32_u24
constexpr uint32_t kHalf1024Pair = 0x64006400u;  // fp16 bit pattern of 1024.0, both halves
constexpr float kSigmaBiasPlus1024 = 1534.0f;    // 1024 + 510
constexpr float kMul1Scale = 1775.0f / 262144.0f;  // 1775 * 2^-18, exact in fp16
constexpr float kInvSqrt128 = 0.08838834764831845f;

__device__ __forceinline__ uint32_t lane_id() { return __lane_id(); }

// Stream-ordered dword: a little-endian dword holds w[2i] in its low half;
// rotating by 16 puts w[2i] (the earlier word) in the high half.
__device__ __forceinline__ uint32_t stream_dword(uint32_t le) {
  return __builtin_amdgcn_alignbit(le, le, 16);
}

// h = S * multiplier for the state held in the high (HI = true) or low half
// of `w`.  The half is selected by the SDWA operand selector, so no separate
// extract instruction is needed.
template <bool HI>
__device__ __forceinline__ uint32_t hash_half(uint32_t w, uint32_t mult) {
  uint32_t h;
  if constexpr (HI)
    asm("v_mul_u32_u24_sdwa %0, %1, %2 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:WORD_1 "
        "src1_sel:DWORD"
        : "=v"(h)
        : "v"(w), "v"(mult));
  else
    asm("v_mul_u32_u24_sdwa %0, %1, %2 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:WORD_0 "
        "src1_sel:DWORD"
        : "=v"(h)
        : "v"(w), "v"(mult));
  return h;
}

// Hash of the state that starts at bit P of the row-pair stream held in the
// stream-ordered dwords B[0..K] (B[K] carries the spill word in its high half).
template <int K, int P>
__device__ __forceinline__ uint32_t state_hash(const uint32_t (&B)[K + 1], uint32_t mult) {
  constexpr int i = P / 32;
  constexpr int o = P % 32;
  constexpr int o16 = o & 15;
  uint32_t w;
  if constexpr (o16 == 0)
    w = B[i];
  else
    w = __builtin_amdgcn_alignbit(B[i], B[i + 1], 32 - o16);  // bits [o16, o16+32) of the stream
  return hash_half<(o < 16)>(w, mult);
}

// Decode one row pair.  D[0..K-1] are the lane's 2K words as little-endian
// dwords, spill_b is the stream-ordered first dword of the next row pair.
// Output: out[c] = half2 {W[2p][c], W[2p+1][c]} for the 16 columns c of the
// tile, i.e. two consecutive k values of one output column.
//
// BIASED = true stops before the codebook's affine step and returns the
// biased codes b = 1024 + sigma (exact fp16 integers 1024..2044) instead:
// W = (b - 1534) * 1775 / 2^18 holds exactly before W's own fp16 rounding, so
// a contraction sum_r b_r x_r - 1534 sum_r x_r, scaled once by 1775 / 2^18,
// is the product with the unrounded codebook values (relative difference to
// the fp16-rounded weights at most 2^-12 per weight).  That saves the packed
// subtract and multiply per weight pair, a quarter of the decode's VALU work.
template <int K, int C, bool BIASED>
__device__ __forceinline__ void decode_column(const uint32_t (&B)[K + 1], uint32_t mult,
                                              uint32_t (&out)[16]) {
  const uint32_t h0 = state_hash<K, K * C>(B, mult);
  const uint32_t h1 = state_hash<K, K * (16 + C)>(B, mult);
  // sigma + 1024 as fp16 bit patterns, packed: low half <- row 2p, high <- 2p+1
  const uint32_t s0 = __builtin_amdgcn_sad_u8(h0, 0u, kHalf1024Pair);
  const uint32_t packed = __builtin_amdgcn_sad_hi_u8(h1, 0u, s0);
  if constexpr (BIASED) {
    out[C] = packed;
  } else {
    const half2_t bias = {(_Float16)kSigmaBiasPlus1024, (_Float16)kSigmaBiasPlus1024};
    const half2_t scale = {(_Float16)kMul1Scale, (_Float16)kMul1Scale};
    half2_t v = __builtin_bit_cast(half2_t, packed);
    v = (v - bias) * scale;  // exact subtraction, then the single fp16 rounding
    out[C] = __builtin_bit_cast(uint32_t, v);
  }
}

// int8 weight of the state that starts at bit P (exl3xpu README, "Prefill:
// int8 linears ...": weights take one static scale, 127 / 3.453125, inside
// the decode).  W_q = RNE((sigma - 510) * 1775 / 2^18 * 127 / 3.453125),
// with |W_q| <= 127, is the top byte (two's complement) of
// sigma * kI8Mul + kI8Add mod 2^32 for every sigma in [0, 1020]:
// floor(((sigma - 510) * kI8Mul + 8388607) / 2^24), where
// kI8Mul / 2^24 = 0.2490313... approximates the slope
// 1775 * 127 * 64 / (2^18 * 221) closely enough that no sigma changes side
// of a rounding boundary (the nearest is 0.0015 away), and the sum stays in
// (-2^31, 2^31).  sigma * kI8Mul < 2^32 and kI8Mul < 2^24, so the product
// is one v_mad_u32_u24.  Returned with W_q in byte 3 and the rest junk.
constexpr uint32_t kI8Mul = 4178012u;
constexpr uint32_t kI8Add = 0x817EC8B7u;  // 8388607 - 510 * kI8Mul mod 2^32

template <int K, int P>
__device__ __forceinline__ uint32_t state_i8(const uint32_t (&B)[K + 1]) {
  const uint32_t h = state_hash<K, P>(B, kMul1Multiplier);
  const uint32_t sigma = __builtin_amdgcn_sad_u8(h, 0u, 0u);
  return __umul24(sigma, kI8Mul) + kI8Add;
}

// Four int8 weights (byte 3 of each) packed little-endian: a in byte 0.
__device__ __forceinline__ uint32_t pack_i8x4(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  const uint32_t lo = __builtin_amdgcn_perm(b, a, 0x0C0C0703u);  // a.b3, b.b3, 0, 0
  const uint32_t hi = __builtin_amdgcn_perm(d, c, 0x07030C0Cu);  // 0, 0, c.b3, d.b3
  return lo | hi;
}

template <int K, bool BIASED, int C = 0>
__device__ __forceinline__ void decode_columns(const uint32_t (&B)[K + 1], uint32_t mult,
                                               uint32_t (&out)[16]) {
  if constexpr (C < 16) {
    decode_column<K, C, BIASED>(B, mult, out);
    decode_columns<K, BIASED, C + 1>(B, mult, out);
  }
}

template <int K, bool BIASED = false>
__device__ __forceinline__ void decode_rowpair(const uint32_t (&D)[K], uint32_t spill_b,
                                               uint32_t (&out)[16]) {
  uint32_t B[K + 1];
#pragma unroll
  for (int i = 0; i < K; ++i) B[i] = stream_dword(D[i]);
  B[K] = spill_b;
  const uint32_t mult = kMul1Multiplier;
  decode_columns<K, BIASED>(B, mult, out);
}

// Stream-ordered first dword of the next row pair in the same tile: lane
// group of 8 (one tile), lane p reads lane (p+1) mod 8.  All 8 lanes of a tile
// must be active together.
__device__ __forceinline__ uint32_t spill_from_next(uint32_t my_first_le) {
  const uint32_t l = lane_id();
  const uint32_t src = (l & ~7u) | ((l + 1u) & 7u);
  return (uint32_t)__builtin_amdgcn_ds_bpermute((int)(src << 2), (int)stream_dword(my_first_le));
}

// Load the lane's 2K words (4K bytes at a 4-byte aligned address).
template <int K>
__device__ __forceinline__ void load_rowpair(const uint32_t* __restrict__ p, uint32_t (&D)[K]) {
  if constexpr (K % 4 == 0) {
#pragma unroll
    for (int i = 0; i < K; i += 4) {
      const uint4 v = *reinterpret_cast<const uint4*>(p + i);
      D[i] = v.x; D[i + 1] = v.y; D[i + 2] = v.z; D[i + 3] = v.w;
    }
  } else if constexpr (K == 2 || K == 6) {
#pragma unroll
    for (int i = 0; i < K; i += 2) {
      const uint2 v = *reinterpret_cast<const uint2*>(p + i);
      D[i] = v.x; D[i + 1] = v.y;
    }
  } else {
#pragma unroll
    for (int i = 0; i < K; ++i) D[i] = p[i];
  }
}

// Buffer-descriptor word 3 of a raw (unformatted, stride 0) buffer on gfx9
// parts: 32-bit data format, no swizzle.
constexpr int kBufferRsrcWord3 = 0x00020000;

// Raw buffer descriptor over [base, base + bytes): out-of-range loads return 0.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           kBufferRsrcWord3);
}

// The lane's 2K words through a buffer descriptor: byte offset voff + soff
// (soff uniform), K dwords in the widest loads K allows.
template <int K, int N>
__device__ __forceinline__ void load_rowpair_buf(__amdgpu_buffer_rsrc_t rs, uint32_t voff,
                                                 uint32_t soff, uint32_t (&D)[N]) {
  static_assert(N >= K, "destination too small");
  typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
  typedef uint32_t u32x3 __attribute__((ext_vector_type(3)));
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
#pragma unroll
  for (int i = 0; i + 4 <= K; i += 4) {
    const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rs, (int)voff + 4 * i, (int)soff, 0);
    D[i] = v.x; D[i + 1] = v.y; D[i + 2] = v.z; D[i + 3] = v.w;
  }
  if constexpr (K % 4 == 3) {
    const u32x3 v = __builtin_amdgcn_raw_buffer_load_b96(rs, (int)voff + 4 * (K - 3), (int)soff, 0);
    D[K - 3] = v.x; D[K - 2] = v.y; D[K - 1] = v.z;
  } else if constexpr (K % 4 == 2) {
    const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(rs, (int)voff + 4 * (K - 2), (int)soff, 0);
    D[K - 2] = v.x; D[K - 1] = v.y;
  } else if constexpr (K % 4 == 1) {
    D[K - 1] = __builtin_amdgcn_raw_buffer_load_b32(rs, (int)voff + 4 * (K - 1), (int)soff, 0);
  }
}

// ---------------------------------------------------------------------------
// 128-point Walsh-Hadamard transform held by one wave: lane l owns elements
// 2l (a) and 2l+1 (b).  Butterfly (u, v) -> (u + v, u - v) with u the lower
// index, strides 1..64, Sylvester (natural) order; no normalisation here.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float shfl_xor_f(float v, int mask) {
  const int src = (int)(lane_id() ^ (uint32_t)mask);
  return __int_as_float(__builtin_amdgcn_ds_bpermute(src << 2, __float_as_int(v)));
}

template <int V>
struct PowC {
  static constexpr int value = V;
};
// f(PowC<I>), f(PowC<2 I>), ... while below N
template <int I, int N, class F>
__device__ __forceinline__ void static_for_pow2(F&& f) {
  if constexpr (I < N) {
    f(PowC<I>{});
    static_for_pow2<2 * I, N>(f);
  }
}

// DPP moves that pair lane l with l ^ 1, l ^ 2 (quad permutations) and l ^ 8
// (rotation by 8 inside each row of 16 lanes): full-rate VALU moves, no LDS.
constexpr int kDppXor1 = 0xB1;    // quad_perm [1, 0, 3, 2]
constexpr int kDppXor2 = 0x4E;    // quad_perm [2, 3, 0, 1]
constexpr int kDppXor8 = 0x128;   // row_ror:8
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, true));
}

// One butterfly across lanes: the lower lane of a pair keeps v + partner, the
// upper one partner - v, written as one fma with a +-1 factor (exact: the
// product is v itself or its negation).
__device__ __forceinline__ float bfly(float v, float partner, bool upper) {
  return __builtin_fmaf(v, upper ? -1.f : 1.f, partner);
}

template <int MASK>
__device__ __forceinline__ float swizzle_xor_f(float v) {
  // bitmask mode: source lane = (lane & 0x1F) ^ MASK inside each 32 lanes
  return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), (MASK << 10) | 0x1F));
}

// Value of lane l ^ MASK: DPP for 1, 2 and 8, ds_swizzle (no LDS memory, no
// address operand) for 4 and 16, ds_bpermute for 32.
template <int MASK>
__device__ __forceinline__ float xor_partner(float v) {
  if constexpr (MASK == 1) return dpp_f<kDppXor1>(v);
  else if constexpr (MASK == 2) return dpp_f<kDppXor2>(v);
  else if constexpr (MASK == 8) return dpp_f<kDppXor8>(v);
  else if constexpr (MASK < 32) return swizzle_xor_f<MASK>(v);
  else return shfl_xor_f(v, MASK);
}

__device__ __forceinline__ void fwht128_pair(float& a, float& b) {
  const float s = a + b, d = a - b;
  a = s;
  b = d;
  const uint32_t l = lane_id();
  static_for_pow2<1, 64>([&](auto mc) {
    constexpr int m = decltype(mc)::value;
    const bool upper = (l & (uint32_t)m) != 0;
    const float pa = xor_partner<m>(a);
    const float pb = xor_partner<m>(b);
    a = bfly(a, pa, upper);
    b = bfly(b, pb, upper);
  });
}

// Transform of up to four 128-element blocks at once by one wave: lane
// l holds elements 8 (l % 16) .. 8 (l % 16) + 7 of block l / 16, so the three
// lowest butterfly strides stay inside the lane and the other four pair
// lanes l ^ 1, 2, 4, 8 of the same 16-lane group (xor_partner: no LDS
// memory).  v[e] = x * suh on entry, the unnormalised transform on exit.
template <int MASK>
__device__ __forceinline__ void fwht_lane_stage(float (&v)[8]) {
  float pv[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) pv[e] = xor_partner<MASK>(v[e]);
  const bool upper = (lane_id() & (uint32_t)MASK) != 0;
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] = bfly(v[e], pv[e], upper);
}

__device__ __forceinline__ void fwht128_x8(float (&v)[8]) {
#pragma unroll
  for (int h = 1; h < 8; h <<= 1)
#pragma unroll
    for (int e = 0; e < 8; ++e)
      if ((e & h) == 0) {
        const float u = v[e], w = v[e + h];
        v[e] = u + w;
        v[e + h] = u - w;
      }
  fwht_lane_stage<1>(v);
  fwht_lane_stage<2>(v);
  fwht_lane_stage<4>(v);
  fwht_lane_stage<8>(v);
}

__device__ __forceinline__ float h2f(uint16_t h) {
  return (float)__builtin_bit_cast(_Float16, h);
}
__device__ __forceinline__ uint16_t f2h(float f) {
  return __builtin_bit_cast(uint16_t, (_Float16)f);
}

}  // namespace exl3
