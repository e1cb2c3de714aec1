// Routed-expert SwiGLU MLP over packed EXL3 arenas, routed contribution only.
//
// exl3xpu README, "MoE (routed experts)": the contribution is computed in
// fp32 with the routing weight applied to the down-projection output; one
// launch per projection, routing kept on device.  Arc 140V MoE post, section 2:
// gate+up as one launch over (expert, slot) units sharing the input row, SiLU
// between the launches, device-side binning of tokens into contiguous
// per-expert slices (2D), fp32 weighted gather (2D).  An arena has one width,
// or one per expert (TensorFold issue #832, "Activity"); then each launch's
// workgroups take their expert's width from the device (width-0 kernels).
//
// Two regimes, chosen on the host from the number of (token, slot) pairs
// P = t * topk (no device data is read back):
//
// Small P (P <= 224: decode, token-parallel verify, short prompts): every pair is an independent M=1
// unit (the README's "per-unit x stride" idea).
//   1. gemv_kernel over units (pair, gate|up); the last workgroup to arrive on
//      a (pair, 128 columns) group sums the k slices of gate and up, applies
//      the output transform and svh, forms a = silu(g) * u and writes the
//      down projection's input (a .* suh_down) H as fp16
//   2. gemv_kernel over units (pair); the last workgroup to arrive on a
//      (token, 128 columns) group adds, for slots in order, the transformed
//      down output times the routing weight in fp32 and writes y
//
// Large P (prefill): device binning, then one grouped MFMA GEMM launch per
// projection over a device-built tile list (expert, first row, rows), so each
// expert's weights are decoded once per tile (128 or 256 rows) instead of once
// per row.
//   1-3. count the pairs per expert and chunk, scan the counts into offsets
//      and the tile list (one workgroup), scatter the pairs into expert order
//   4. x'_g, x'_u = (x_token .* suh_e,slot) H for each sorted row   -> fp16
//   5. gemm_kernel over (tile, 128 cols): g, then u (transformed, svh), then
//      a = silu(g) * u and x'_d = (a .* suh_down_e) H on the block    -> fp16
//   6. gemm_kernel over (tile, 128 cols)        -> d fp32 (transformed, svh)
//   7. y[token] = sum over slots in order of w * d                  -> fp32
#include "exl3_device.hpp"
#include "exl3_gemm.hpp"
#include "exl3_gemv.hpp"
#include "exl3_internal.hpp"

namespace exl3 {

// P at or below this uses the unit path: measured on MI355X for 256 experts x
// (2048 -> 2 x 512 -> 2048), K=3, top-8, random routing, the unit path is
// faster up to T = 24 (P = 192: 119-122 us against 132 us for the binned
// path), about even at T = 28 and slower from T = 29 (144-149 against
// 138 us) on (T = 32: 153-157 against 143 us; T = 48: 230 against 179 us).
constexpr int kGroupedUnitMaxPairs = 224;
// Rows per tile of the grouped GEMM: 256 when the experts average at least
// 96 rows (one tile per expert instead of two, so each expert's weights are
// decoded once per column block), else 128.  A wave runs MFMAs only for its
// row groups that hold rows, so a half-filled 256-row tile costs about the
// MFMA work of its rows.  Measured on MI355X at 256 experts x (2048 -> 2 x
// 512 -> 2048), K=3, top-8: T=4096 (128 rows per expert on average) takes
// 0.69 ms with 256-row tiles against 0.77 ms with 128; T=512 (16 rows)
// 0.27 ms either way.
constexpr int kGroupedMinRowsBig = 96;
static inline int grouped_bm(int64_t P, int E) { return P >= (int64_t)kGroupedMinRowsBig * E ? 256 : 128; }
// routing binning: pairs per chunk (one workgroup of the count and scatter
// launches each)
constexpr int kBinThreads = 256;
constexpr int kBinPerThread = 8;
constexpr int kBinIds = kBinThreads * kBinPerThread;

static inline int64_t bin_chunks(int64_t P) { return (P + kBinIds - 1) / kBinIds; }


static inline size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

// Where an expert's tensors start and how wide they are.  A uniform arena
// (bits == nullptr) packs expert e at e * slots tensors of the launch's one
// width; an arena with a width per expert gives each expert's first word and
// width, and one launch (kernel width 0) serves every width, each workgroup
// taking its own.
struct ExpertWidths {
  const int32_t* bits = nullptr;  // device int32 [experts]
  const int64_t* off = nullptr;   // device int64 [experts]
  int64_t words_per_bit = 0;      // words of one (expert, slot) tensor per bit of width
};
struct ExpertTensors {
  const uint16_t* base;  // slot 0
  int64_t stride;        // words from one slot to the next
  int bits;              // 0 in a uniform arena (the kernel's own width)
};
__device__ __forceinline__ ExpertTensors expert_tensors(const uint16_t* trellis,
                                                        const ExpertWidths& w, int e, int slots,
                                                        int64_t tensor_words) {
  if (!w.bits) return ExpertTensors{trellis + (int64_t)e * slots * tensor_words, tensor_words, 0};
  const int b = w.bits[e];
  return ExpertTensors{trellis + w.off[e], w.words_per_bit * b, b};
}

// ---------------------------------------------------------------------------
// small-P path
// ---------------------------------------------------------------------------
// Per-row sums over k ranges of the fp32 partials of two adjacent columns:
// row r (r < rows <= R) has its slices j = 0..splits-1 at p + r * row_stride +
// j * stride.  Each row is summed in slice order from 0.f (the order of a
// plain loop over the slices); the loads of B slices of every row are issued
// before any of them is added, so the finish waits one round trip per B
// slices, not one per slice and row.  The slices were written by other
// workgroups of the same launch with device-scope stores, so the loads are
// device scope too.
template <int R, int B>
__device__ __forceinline__ void sum_slices(const float* p, int64_t row_stride, int splits,
                                           int64_t stride, float (&sum)[R][2], int rows = R) {
#pragma unroll
  for (int r = 0; r < R; ++r) sum[r][0] = sum[r][1] = 0.f;
  for (int j0 = 0; j0 < splits; j0 += B) {
    float v[R][B][2];
#pragma unroll
    for (int r = 0; r < R; ++r) {
#pragma unroll
      for (int q = 0; q < B; ++q) {
        if (r < rows && j0 + q < splits) {
          const float* a = p + r * row_stride + (int64_t)(j0 + q) * stride;
          v[r][q][0] = __hip_atomic_load(a, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          v[r][q][1] = __hip_atomic_load(a + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
      }
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
#pragma unroll
      for (int q = 0; q < B; ++q) {
        if (r < rows && j0 + q < splits) {
          sum[r][0] += v[r][q][0];
          sum[r][1] += v[r][q][1];
        }
      }
    }
  }
}

// Slots of one token per wave in a down finish (four or eight waves, top-k <= 16).
constexpr int kDnSlotsPerWave = 4;

struct GuUnitRes {
  const uint16_t* trellis;
  const uint16_t* suh;
  const uint16_t* svh;
  int64_t tensor_words;  // words of one (expert, slot) tensor
  int k;                 // hidden
  int n;                 // intermediate
  const uint16_t* x;
  int topk;
  const int32_t* ids;
  float* part;           // fp32 [P][2][splits][n]
  int splits;
  unsigned int* ctr;     // [P][n/128]
  const uint16_t* suh_dn;
  uint16_t* xd;          // fp16 [P][n]: input of the down projection, Hadamard domain
  int pairs;             // P
  ExpertWidths ew;
  int off_xcd_all = 0;   // 1: every workgroup takes the device-scope hand-off
  // output group (pair, 128 columns); members (gate|up, k range)
  __device__ bool place(int b, int& u, int& split, int& nb) const {
    int grp, mem;
    if (!gemv_place(b, pairs * (n >> 7), 2 * splits, grp, mem)) return false;
    const int pair = grp / (n >> 7);
    nb = grp - pair * (n >> 7);
    u = 2 * pair + mem / splits;
    split = mem - (mem / splits) * splits;
    return true;
  }
  __device__ GemvTask task(int u, int split) const {
    GemvTask T;
    const int pair = u >> 1, slot = u & 1;
    const int e = ids[pair];
    const int tok = pair / topk;
    const ExpertTensors et = expert_tensors(trellis, ew, e, 2, tensor_words);
    T.valid = true;
    T.trellis = et.base + slot * et.stride;
    T.bits = et.bits;
    T.suh = suh + (int64_t)(e * 2 + slot) * k;
    T.x = x + (int64_t)tok * k;
    T.ldx = k;
    T.m = 1;
    T.partial = part + ((int64_t)u * splits + split) * n;
    return T;
  }
  __device__ unsigned int* counter(int u, int nb) const { return ctr + (u >> 1) * (n >> 7) + nb; }
  __device__ unsigned int arrivals(int) const { return 2u * (unsigned int)splits; }
  // gate and up of one pair: sum, output transform, svh; a = silu(g) * u;
  // then the down projection's input transform (a .* suh_down) H.  Wave 0
  // takes the gate, wave 1 the up projection; wave 0 finishes.
  struct FinishPre {
    uint32_t sv;  // svh of this wave's slot (waves 0, 1)
    uint32_t su;  // suh of the down projection (wave 0)
  };
  __device__ FinishPre finish_prefetch(int u, int nb) const {
    FinishPre f{0u, 0u};
    const int wave = threadIdx.x >> 6;
    if (wave < 2) {
      const int e = ids[u >> 1];
      const int col = nb * 128 + 2 * (int)lane_id();
      f.sv = *reinterpret_cast<const uint32_t*>(svh + (int64_t)(e * 2 + wave) * n + col);
      if (wave == 0) f.su = *reinterpret_cast<const uint32_t*>(suh_dn + (int64_t)e * n + col);
    }
    return f;
  }
  __device__ void finish(int u, int nb, int, const FinishPre& f, unsigned char* smem) const {
    const int wave = threadIdx.x >> 6;
    const int pair = u >> 1;
    const int col = nb * 128 + 2 * (int)lane_id();
    float* up = reinterpret_cast<float*>(smem);  // [128]: the transformed up projection
    float a = 0.f, b = 0.f;
    if (wave < 2) {
      // slices (pair, slot = wave, 0..splits-1)
      float sum[1][2];
      sum_slices<1, 4>(part + (int64_t)(pair * 2 + wave) * splits * n + col, 0, splits, n, sum);
      a = sum[0][0];
      b = sum[0][1];
      fwht128_pair(a, b);
      a *= kInvSqrt128 * h2f((uint16_t)(f.sv & 0xFFFF));
      b *= kInvSqrt128 * h2f((uint16_t)(f.sv >> 16));
      if (wave == 1) *reinterpret_cast<float2*>(up + 2 * lane_id()) = make_float2(a, b);
    }
    __syncthreads();
    if (wave != 0) return;
    const float2 uv = *reinterpret_cast<const float2*>(up + 2 * lane_id());
    a = silu_f(a) * uv.x;
    b = silu_f(b) * uv.y;
    a *= h2f((uint16_t)(f.su & 0xFFFF));
    b *= h2f((uint16_t)(f.su >> 16));
    fwht128_pair(a, b);
    a *= kInvSqrt128;
    b *= kInvSqrt128;
    *reinterpret_cast<uint32_t*>(xd + (int64_t)pair * n + col) =
        (uint32_t)f2h(a) | ((uint32_t)f2h(b) << 16);
  }
};

struct DnUnitRes {
  const uint16_t* trellis;
  const uint16_t* svh;
  int64_t tensor_words;
  int k;               // intermediate
  int n;               // hidden
  const uint16_t* xd;  // fp16 [P][k], already in the Hadamard domain
  const int32_t* ids;
  const float* w;
  int topk;
  float* part;         // fp32 [P][splits][n]
  int splits;
  unsigned int* ctr;   // [t][n/128]
  float* y;            // fp32 [t][n]
  int tokens;          // t
  ExpertWidths ew;
  int off_xcd_all = 0; // 1: every workgroup takes the device-scope hand-off
  // output group (token, 128 columns); members (slot, k range)
  __device__ bool place(int b, int& u, int& split, int& nb) const {
    int grp, mem;
    if (!gemv_place(b, tokens * (n >> 7), topk * splits, grp, mem)) return false;
    const int tok = grp / (n >> 7);
    nb = grp - tok * (n >> 7);
    u = tok * topk + mem / splits;
    split = mem - (mem / splits) * splits;
    return true;
  }
  __device__ GemvTask task(int u, int split) const {
    GemvTask T;
    const int e = ids[u];
    const ExpertTensors et = expert_tensors(trellis, ew, e, 1, tensor_words);
    T.valid = true;
    T.trellis = et.base;
    T.bits = et.bits;
    T.suh = nullptr;
    T.x = xd + (int64_t)u * k;
    T.ldx = k;
    T.m = 1;
    T.partial = part + ((int64_t)u * splits + split) * n;
    return T;
  }
  __device__ unsigned int* counter(int u, int nb) const { return ctr + (u / topk) * (n >> 7) + nb; }
  __device__ unsigned int arrivals(int) const { return (unsigned int)(topk * splits); }
  // y[token, block] = sum over slots in order of w * ((sum_s partial) H .* svh).
  // Wave w takes slots w, w + nw, ... (nw waves); each slot's weighted term goes through
  // LDS and wave 0 adds them in slot order.
  struct FinishPre {
    uint32_t sv[kDnSlotsPerWave];  // svh of this wave's slots
    float wt[kDnSlotsPerWave];     // their routing weights
  };
  __device__ FinishPre finish_prefetch(int u, int nb) const {
    FinishPre f;
    const int wave = threadIdx.x >> 6;
    const int nw = (int)(blockDim.x >> 6);
    const int p0 = (u / topk) * topk;
    const int col = nb * 128 + 2 * (int)lane_id();
#pragma unroll
    for (int q = 0; q < kDnSlotsPerWave; ++q) {
      const int s = wave + nw * q;
      f.sv[q] = 0u;
      f.wt[q] = 0.f;
      if (s < topk) {
        const int e = ids[p0 + s];
        f.sv[q] = *reinterpret_cast<const uint32_t*>(svh + (int64_t)e * n + col);
        f.wt[q] = w[p0 + s];
      }
    }
    return f;
  }
  __device__ void finish(int u, int nb, int, const FinishPre& f, unsigned char* smem) const {
    const int wave = threadIdx.x >> 6;
    const int nw = (int)(blockDim.x >> 6);
    const int tok = u / topk;
    const int p0 = tok * topk;
    const int col = nb * 128 + 2 * (int)lane_id();
    float* terms = reinterpret_cast<float*>(smem);  // [topk][128]
    const int mine = wave < topk ? (topk - wave + nw - 1) / nw : 0;  // slots of this wave
    // slices (pair p0 + wave + 4 q, 0..splits-1)
    float sum[kDnSlotsPerWave][2];
    sum_slices<kDnSlotsPerWave, 2>(part + (int64_t)(p0 + wave) * splits * n + col, (int64_t)nw * splits * n,
                                   splits, n, sum, mine);
#pragma unroll
    for (int q = 0; q < kDnSlotsPerWave; ++q) {
      if (q < mine) {
        float a = sum[q][0], b = sum[q][1];
        fwht128_pair(a, b);
        const float ta = f.wt[q] * (a * kInvSqrt128 * h2f((uint16_t)(f.sv[q] & 0xFFFF)));
        const float tb = f.wt[q] * (b * kInvSqrt128 * h2f((uint16_t)(f.sv[q] >> 16)));
        *reinterpret_cast<float2*>(terms + (wave + nw * q) * 128 + 2 * lane_id()) = make_float2(ta, tb);
      }
    }
    __syncthreads();
    if (wave != 0) return;
    float ya = 0.f, yb = 0.f;
    for (int s = 0; s < topk; ++s) {
      const float2 t = *reinterpret_cast<const float2*>(terms + s * 128 + 2 * lane_id());
      ya += t.x;
      yb += t.y;
    }
    *reinterpret_cast<float2*>(y + (int64_t)tok * n + col) = make_float2(ya, yb);
  }
};

template <int K>
struct GuUnitRun {
  static hipError_t run(const GuUnitRes& r, int k, int n, int /*units*/, int kc, hipStream_t s) {
    const int grid = gemv_grid(r.pairs * (n / 128), 2 * r.splits);
    return launch_gemv_kernel<K>(r, dim3(grid), 1, s, k, n, kc);
  }
};

template <int K>
struct DnUnitRun {
  static hipError_t run(const DnUnitRes& r, int k, int n, int /*units*/, int kc, hipStream_t s) {
    const int grid = gemv_grid(r.tokens * (n / 128), r.topk * r.splits);
    return launch_gemv_kernel<K>(r, dim3(grid), 1, s, k, n, kc);
  }
};

// Arrival counters of the unit path live at the start of the workspace, in a
// region whose size depends only on the arena shapes (enough for the largest
// unit-path call).  A unit-path call leaves every counter it used with zero
// counts (and the XCD record of GemvCtr), the binned path does not touch the
// region, so one workspace can serve calls of any size.
static size_t counter_region(const ArenaDesc& gu, const ArenaDesc& dn) {
  const size_t c = (size_t)kGroupedUnitMaxPairs * (gu.n / 128) +
                   (size_t)kGroupedUnitMaxPairs * (dn.n / 128);
  return align256(c * 4);
}

struct UnitLayout {
  int s_gu, s_dn;
  size_t ctr_gu, ctr_dn, part_gu, xd, part_dn, total;
};

static UnitLayout unit_layout(const ArenaDesc& gu, const ArenaDesc& dn, int64_t P) {
  UnitLayout L;
  L.s_gu = gemv_choose_splits(gu.k, (gu.n / 128) * (int)P * 2, 1, kGemvTargetWorkgroups);
  L.s_dn = gemv_choose_splits(dn.k, (dn.n / 128) * (int)P, 1, kGemvTargetWorkgroups);
  L.ctr_gu = 0;
  L.ctr_dn = (size_t)kGroupedUnitMaxPairs * (gu.n / 128) * 4;
  size_t off = counter_region(gu, dn);
  L.part_gu = off; off += align256((size_t)P * 2 * L.s_gu * gu.n * sizeof(float));
  L.xd = off;      off += align256((size_t)P * gu.n * sizeof(uint16_t));
  L.part_dn = off; off += align256((size_t)P * L.s_dn * dn.n * sizeof(float));
  L.total = off;
  return L;
}

// ---------------------------------------------------------------------------
// large-P path
// ---------------------------------------------------------------------------
struct TileEntry {
  int e, row0, rows, pad;
};

struct GemmLayout {
  int bm;  // rows per tile
  int max_tiles;
  size_t hist, offsets, ntiles, tiles, pos, sorted, xg, xd, d, total;
};

static GemmLayout gemm_layout(const ArenaDesc& gu, const ArenaDesc& dn, int64_t P) {
  GemmLayout L;
  const int E = gu.experts;
  L.bm = grouped_bm(P, E);
  L.max_tiles = (int)((P + L.bm - 1) / L.bm) + (int)(P < E ? P : E);
  size_t off = counter_region(gu, dn);
  L.hist = off;    off += align256((size_t)bin_chunks(P) * E * 4);
  L.offsets = off; off += align256((size_t)E * 4);
  L.ntiles = off;  off += 256;
  L.tiles = off;   off += align256((size_t)L.max_tiles * sizeof(TileEntry));
  L.pos = off;     off += align256((size_t)P * 4);
  L.sorted = off;  off += align256((size_t)P * 4);
  L.xg = off;      off += align256((size_t)2 * P * gu.k * sizeof(uint16_t));
  L.xd = off;      off += align256((size_t)P * dn.k * sizeof(uint16_t));
  L.d = off;       off += align256((size_t)P * dn.n * sizeof(float));
  L.total = off;
  return L;
}

// Routing binning, three launches.  The pairs are cut into chunks of
// kBinIds; chunk c is handled by workgroup c of bin_count and of bin_scatter.
//   bin_count    per-chunk, per-expert counts hist[c][e] (LDS integer
//                atomics: exact)
//   bin_plan     one workgroup: the expert totals, their exclusive scan
//                (offsets), the scan of the tile counts ceil(count / bm) (the
//                tile list), and hist[c][e] replaced by the first row of
//                chunk c's pairs of expert e
//   bin_scatter  every chunk places its pairs from those first rows on,
//                through per-expert cursors in LDS
// Experts go through LDS kBinChunk at a time (one pass for up to kBinChunk
// experts).  The order of the pairs inside a chunk's share of an expert is
// not fixed (LDS atomics), but every row is computed independently of its
// position, so the output does not depend on it.
constexpr int kBinChunk = 8192;  // experts per pass (32 KB of LDS)
constexpr int kPlanThreads = 256;
constexpr int kCombineBatch = 8;  // slots whose loads the combine issues together

__device__ __forceinline__ void bin_load_ids(const int32_t* __restrict__ ids, int64_t P,
                                             int (&ev)[kBinPerThread]) {
  const int64_t i0 = (int64_t)blockIdx.x * kBinIds + threadIdx.x;
#pragma unroll
  for (int q = 0; q < kBinPerThread; ++q) {
    const int64_t i = i0 + (int64_t)q * kBinThreads;
    ev[q] = i < P ? ids[i] : -1;
  }
}

__global__ __launch_bounds__(kBinThreads) void bin_count(const int32_t* __restrict__ ids, int64_t P,
                                                         int E, int32_t* __restrict__ hist) {
  __shared__ int cnt[kBinChunk];
  int ev[kBinPerThread];
  bin_load_ids(ids, P, ev);
  int32_t* h = hist + (int64_t)blockIdx.x * E;
  for (int c0 = 0; c0 < E; c0 += kBinChunk) {
    const int ce = (E - c0) < kBinChunk ? (E - c0) : kBinChunk;
    for (int e = threadIdx.x; e < ce; e += kBinThreads) cnt[e] = 0;
    __syncthreads();
#pragma unroll
    for (int q = 0; q < kBinPerThread; ++q)
      if ((unsigned)(ev[q] - c0) < (unsigned)ce) atomicAdd(&cnt[ev[q] - c0], 1);
    __syncthreads();
    for (int e = threadIdx.x; e < ce; e += kBinThreads) h[c0 + e] = cnt[e];
    __syncthreads();
  }
}

// Exclusive scans of two values over the workgroup (in thread order) and
// their totals: an inclusive scan inside each wave (lane shuffles), then the
// wave totals through LDS.  Integer sums, so the result is exact.
__device__ __forceinline__ void block_exclusive_scan2(int a, int b, int* sh, int& ea, int& eb, int& ta,
                                                      int& tb) {
  constexpr int NW = kPlanThreads / 64;
  const int lane = (int)(threadIdx.x & 63), wave = (int)(threadIdx.x >> 6);
  int ia = a, ib = b;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int xa = __shfl_up(ia, d), xb = __shfl_up(ib, d);
    if (lane >= d) {
      ia += xa;
      ib += xb;
    }
  }
  if (lane == 63) {
    sh[wave] = ia;
    sh[NW + wave] = ib;
  }
  __syncthreads();
  int pa = 0, pb = 0, sa = 0, sb = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const int va = sh[w], vb = sh[NW + w];
    if (w < wave) {
      pa += va;
      pb += vb;
    }
    sa += va;
    sb += vb;
  }
  __syncthreads();  // sh is written again by the next call
  ea = pa + ia - a;
  eb = pb + ib - b;
  ta = sa;
  tb = sb;
}

__global__ __launch_bounds__(kPlanThreads) void bin_plan(int32_t* __restrict__ hist, int chunks, int E,
                                                         int bm, int32_t* __restrict__ offsets,
                                                         int32_t* __restrict__ ntiles,
                                                         TileEntry* __restrict__ tiles) {
  __shared__ int sh[2 * (kPlanThreads / 64)];
  int row_base = 0, tile_base = 0;
  for (int e0 = 0; e0 < E; e0 += kPlanThreads) {
    const int e = e0 + (int)threadIdx.x;
    int c = 0;
    if (e < E) {
#pragma unroll 8
      for (int ch = 0; ch < chunks; ++ch) c += hist[(int64_t)ch * E + e];
    }
    const int nt = (c + bm - 1) / bm;
    int rows_total, tiles_total, off, toff;
    block_exclusive_scan2(c, nt, sh, off, toff, rows_total, tiles_total);
    off += row_base;
    toff += tile_base;
    if (e < E) {
      offsets[e] = off;
      int run = off;
#pragma unroll 8
      for (int ch = 0; ch < chunks; ++ch) {
        const int64_t hi = (int64_t)ch * E + e;
        const int v = hist[hi];
        hist[hi] = run;
        run += v;
      }
      for (int t = 0; t < nt; ++t) {
        TileEntry te;
        te.e = e;
        te.row0 = off + t * bm;
        te.rows = (c - t * bm) < bm ? (c - t * bm) : bm;
        te.pad = 0;
        tiles[toff + t] = te;
      }
    }
    row_base += rows_total;
    tile_base += tiles_total;
  }
  if (threadIdx.x == 0) *ntiles = tile_base;
}

__global__ __launch_bounds__(kBinThreads) void bin_scatter(const int32_t* __restrict__ ids, int64_t P,
                                                           int E, const int32_t* __restrict__ first,
                                                           int32_t* __restrict__ pos,
                                                           int32_t* __restrict__ sorted) {
  __shared__ int cur[kBinChunk];
  int ev[kBinPerThread];
  bin_load_ids(ids, P, ev);
  const int32_t* f = first + (int64_t)blockIdx.x * E;
  const int64_t i0 = (int64_t)blockIdx.x * kBinIds + threadIdx.x;
  for (int c0 = 0; c0 < E; c0 += kBinChunk) {
    const int ce = (E - c0) < kBinChunk ? (E - c0) : kBinChunk;
    for (int e = threadIdx.x; e < ce; e += kBinThreads) cur[e] = f[c0 + e];
    __syncthreads();
#pragma unroll
    for (int q = 0; q < kBinPerThread; ++q)
      if ((unsigned)(ev[q] - c0) < (unsigned)ce) {
        const int64_t i = i0 + (int64_t)q * kBinThreads;
        const int r = atomicAdd(&cur[ev[q] - c0], 1);
        sorted[r] = (int32_t)i;
        pos[i] = r;
      }
    __syncthreads();
  }
}

// x'_slot[r] = (x[token(r)] .* suh[e(r)][slot]) H for both slots, one wave
// per sorted row, 16 blocks of 128 elements per pass.  Lane l holds the 32
// elements 32 i + 8 (l % 4) + e (i < 4, e < 8) of block l / 4: the strides 1,
// 2, 4 (e) and 32, 64 (i) stay inside the lane and 8, 16 pair the lanes of a
// quad (DPP moves).  The stages run in the order 1, 2, ..., 64 and each
// butterfly is the same sum or difference as in fwht128_x8, so the result
// has the same bits as that layout's.
constexpr int kGuBlocks = 16;  // blocks per pass (four lanes each)

__device__ __forceinline__ void fwht128_x32(float (&v)[32]) {
#pragma unroll
  for (int h = 1; h < 8; h <<= 1)
#pragma unroll
    for (int e = 0; e < 32; ++e)
      if ((e & h) == 0) {
        const float u = v[e], w = v[e + h];
        v[e] = u + w;
        v[e + h] = u - w;
      }
#pragma unroll
  for (int mi = 0; mi < 2; ++mi) {
    const int m = 1 << mi;
    float pv[32];
#pragma unroll
    for (int e = 0; e < 32; ++e) pv[e] = mi == 0 ? xor_partner<1>(v[e]) : xor_partner<2>(v[e]);
    const bool upper = (lane_id() & (uint32_t)m) != 0;
#pragma unroll
    for (int e = 0; e < 32; ++e) v[e] = bfly(v[e], pv[e], upper);
  }
#pragma unroll
  for (int h = 8; h < 32; h <<= 1)
#pragma unroll
    for (int e = 0; e < 32; ++e)
      if ((e & h) == 0) {
        const float u = v[e], w = v[e + h];
        v[e] = u + w;
        v[e + h] = u - w;
      }
}

__global__ __launch_bounds__(256) void gu_input_transform(
    const uint16_t* __restrict__ x, int topk, int64_t P, int hidden,
    const int32_t* __restrict__ sorted, const int32_t* __restrict__ ids,
    const uint16_t* __restrict__ suh_gu, uint16_t* __restrict__ xg) {
  const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= P) return;
  const int pair = sorted[r];
  const int e = ids[pair];
  const int64_t tok = pair / topk;
  const int lane = (int)lane_id();
  const int bq = lane >> 2, q = lane & 3;
  const int nblk = hidden >> 7;
  const uint16_t* xr = x + tok * hidden;
  const uint16_t* s0 = suh_gu + (int64_t)e * 2 * hidden;
  const uint16_t* s1 = s0 + hidden;
  uint16_t* d0 = xg + r * hidden;
  uint16_t* d1 = xg + (P + r) * hidden;
  for (int b0 = 0; b0 < nblk; b0 += kGuBlocks) {
    const int b = b0 + bq;
    const int base = (b < nblk ? b : nblk - 1) * 128 + 8 * q;  // lanes past the last block repeat it (not stored)
    uint4 xv[4], sv0[4], sv1[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      xv[i] = *reinterpret_cast<const uint4*>(xr + base + 32 * i);
      sv0[i] = *reinterpret_cast<const uint4*>(s0 + base + 32 * i);
      sv1[i] = *reinterpret_cast<const uint4*>(s1 + base + 32 * i);
    }
    float v0[32], v1[32];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t xw[4] = {xv[i].x, xv[i].y, xv[i].z, xv[i].w};
      const uint32_t w0[4] = {sv0[i].x, sv0[i].y, sv0[i].z, sv0[i].w};
      const uint32_t w1[4] = {sv1[i].x, sv1[i].y, sv1[i].z, sv1[i].w};
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const float xa = h2f((uint16_t)(xw[c] & 0xFFFF)), xb = h2f((uint16_t)(xw[c] >> 16));
        v0[8 * i + 2 * c] = xa * h2f((uint16_t)(w0[c] & 0xFFFF));
        v0[8 * i + 2 * c + 1] = xb * h2f((uint16_t)(w0[c] >> 16));
        v1[8 * i + 2 * c] = xa * h2f((uint16_t)(w1[c] & 0xFFFF));
        v1[8 * i + 2 * c + 1] = xb * h2f((uint16_t)(w1[c] >> 16));
      }
    }
    fwht128_x32(v0);
    fwht128_x32(v1);
    if (b < nblk) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        uint32_t o0[4], o1[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          o0[c] = (uint32_t)f2h(v0[8 * i + 2 * c] * kInvSqrt128) |
                  ((uint32_t)f2h(v0[8 * i + 2 * c + 1] * kInvSqrt128) << 16);
          o1[c] = (uint32_t)f2h(v1[8 * i + 2 * c] * kInvSqrt128) |
                  ((uint32_t)f2h(v1[8 * i + 2 * c + 1] * kInvSqrt128) << 16);
        }
        *reinterpret_cast<uint4*>(d0 + base + 32 * i) = make_uint4(o0[0], o0[1], o0[2], o0[3]);
        *reinterpret_cast<uint4*>(d1 + base + 32 * i) = make_uint4(o1[0], o1[1], o1[2], o1[3]);
      }
    }
  }
}

// y[token] = sum over slots in order of w[token, slot] * d[pos(token, slot)]
__global__ __launch_bounds__(256) void combine_rows(const float* __restrict__ d,
                                                   const int32_t* __restrict__ pos,
                                                   const float* __restrict__ w, int64_t t_count,
                                                   int topk, int hidden, float* __restrict__ y) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;  // float4 index
  const int q = hidden >> 2;
  if (idx >= t_count * q) return;
  const int64_t tok = idx / q;
  const int c4 = (int)(idx - tok * q);
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int s0 = 0; s0 < topk; s0 += kCombineBatch) {
    // every load of the batch first, then the sums in slot order
    float wt[kCombineBatch];
    float4 v[kCombineBatch];
#pragma unroll
    for (int u = 0; u < kCombineBatch; ++u) {
      if (s0 + u < topk) {
        const int64_t pr = tok * topk + s0 + u;
        wt[u] = w[pr];
        v[u] = reinterpret_cast<const float4*>(d + (int64_t)pos[pr] * hidden)[c4];
      }
    }
#pragma unroll
    for (int u = 0; u < kCombineBatch; ++u) {
      if (s0 + u < topk) {
        acc.x += wt[u] * v[u].x;
        acc.y += wt[u] * v[u].y;
        acc.z += wt[u] * v[u].z;
        acc.w += wt[u] * v[u].w;
      }
    }
  }
  reinterpret_cast<float4*>(y + tok * hidden)[c4] = acc;
}

// Workgroup -> (tile, slot, 128-column block).  Dispatch hands workgroup b to
// XCD b % 8, so the grid is laid out for that: group G = (tile, slot), with
// the slot fastest, belongs to XCD G % 8, and that XCD's workgroups take its
// groups in order, each across all column blocks.  The column blocks of one
// group read the same gathered rows, which then come from that XCD's L2
// instead of once per block; the groups past the tile count (the tile list's
// length is known on the device only) spread evenly over the XCDs.
struct GroupedGemmRes {
  static constexpr bool kAFrag = false;  // gathered rows stay row-major
  static constexpr bool kFineSkip = true;  // tiles end wherever an expert's rows do
  static constexpr bool kGateUp = false;
  const TileEntry* tiles;
  const int32_t* ntiles;
  const uint16_t* a;       // fp16 [slots][P][k]
  int64_t P;
  int k, n;
  const uint16_t* trellis;
  const uint16_t* svh;
  int slots;
  int64_t tensor_words;
  float* y;                // fp32 [slots][P][n]
  ExpertWidths ew;
  __device__ GemmTask task() const {
    const int nbt = n / kGemmBN;
    const int b = (int)blockIdx.x;
    const int l = b >> 3;
    const int gq = l / nbt;
    const int G = 8 * gq + (b & 7);
    const int tile = G / slots, slot = G - tile * slots;
    GemmTask T;
    T.nb = l - gq * nbt;
    T.valid = tile < *ntiles;
    if (!T.valid) return T;
    const TileEntry te = tiles[tile];
    const ExpertTensors et = expert_tensors(trellis, ew, te.e, slots, tensor_words);
    T.a = a + ((int64_t)slot * P + te.row0) * k;
    T.lda = k;
    T.rows = te.rows;
    T.trellis = et.base + slot * et.stride;
    T.bits = et.bits;
    T.svh = svh + (int64_t)(te.e * slots + slot) * n;
    T.bias = nullptr;
    T.y = y + ((int64_t)slot * P + te.row0) * n;
    T.ldy = n;
    return T;
  }
};

template <int K>
struct GroupedGemmRun {
  static hipError_t run(const GroupedGemmRes& r, int bm, int max_tiles, hipStream_t s) {
    const int64_t groups = ((int64_t)max_tiles * r.slots + 7) / 8 * 8;
    const dim3 grid((unsigned)(groups * (r.n / kGemmBN)));
    if (bm == 256)
      hipLaunchKernelGGL((gemm_kernel<K, 256, true, GroupedGemmRes>), grid, dim3(kGemmThreads), 0, s, r, r.k, r.n);
    else
      hipLaunchKernelGGL((gemm_kernel<K, 128, true, GroupedGemmRes>), grid, dim3(kGemmThreads), 0, s, r, r.k, r.n);
    return hipGetLastError();
  }
};

// Gate and up of one (tile, 128-column block) in one workgroup, one after the
// other over the same gathered rows, then a = silu(g) u and the down
// projection's input transform on that block (the down input's 128-element
// Hadamard blocks are the gate/up column blocks), written as fp16 x'_d rows.
// Same XCD-aware order as GroupedGemmRes with one group per tile.
struct GroupedGateUpRes {
  static constexpr bool kAFrag = false;
  static constexpr bool kFineSkip = true;
  static constexpr bool kGateUp = true;
  const TileEntry* tiles;
  const int32_t* ntiles;
  const uint16_t* a;       // fp16 [2][P][k]: x'_gate, x'_up
  int64_t P;
  int k, n;
  const uint16_t* trellis; // arena [E][2][k/16][n/16][16K]
  const uint16_t* svh;     // fp16 [E][2][n]
  const uint16_t* suh_dn;  // fp16 [E][n], the down projection's input signs
  int64_t tensor_words;
  uint16_t* y;             // fp16 [P][n]: x'_d
  ExpertWidths ew;
  __device__ GemmTask task() const {
    const int nbt = n / kGemmBN;
    const int b = (int)blockIdx.x;
    const int l = b >> 3;
    const int gq = l / nbt;
    const int tile = 8 * gq + (b & 7);
    GemmTask T;
    T.nb = l - gq * nbt;
    T.valid = tile < *ntiles;
    if (!T.valid) return T;
    const TileEntry te = tiles[tile];
    const ExpertTensors et = expert_tensors(trellis, ew, te.e, 2, tensor_words);
    T.a = a + te.row0 * (int64_t)k;
    T.a2 = a + (P + te.row0) * (int64_t)k;
    T.lda = k;
    T.rows = te.rows;
    T.trellis = et.base;
    T.trellis2 = et.base + et.stride;
    T.bits = et.bits;
    T.svh = svh + (int64_t)te.e * 2 * n;
    T.svh2 = T.svh + n;
    T.snext = suh_dn + (int64_t)te.e * n;
    T.bias = nullptr;
    T.y = y + te.row0 * (int64_t)n;
    T.ldy = n;
    return T;
  }
};

template <int K>
struct GroupedGateUpRun {
  static hipError_t run(const GroupedGateUpRes& r, int bm, int max_tiles, hipStream_t s) {
    const int64_t groups = ((int64_t)max_tiles + 7) / 8 * 8;
    const dim3 grid((unsigned)(groups * (r.n / kGemmBN)));
    if (bm == 256)
      hipLaunchKernelGGL((gemm_kernel<K, 256, false, GroupedGateUpRes>), grid, dim3(kGemmThreads), 0, s, r, r.k, r.n);
    else
      hipLaunchKernelGGL((gemm_kernel<K, 128, false, GroupedGateUpRes>), grid, dim3(kGemmThreads), 0, s, r, r.k, r.n);
    return hipGetLastError();
  }
};

// ---------------------------------------------------------------------------
// Words of one (expert, slot) tensor per bit of width.
static int64_t words_per_bit(const ArenaDesc& a) { return (int64_t)(a.k / 16) * (a.n / 16) * 16; }
static ExpertWidths arena_widths(const ArenaDesc& a) {
  ExpertWidths w;
  if (a.bits == 0) {
    w.bits = a.ebits;
    w.off = a.eoff;
    w.words_per_bit = words_per_bit(a);
  }
  return w;
}
// One launch of F at the arena's width, or at width 0 (each workgroup takes
// its expert's width) when the arena has a width per expert.
template <template <int> class F, class... Args>
static hipError_t run_widths(const ArenaDesc& a, Args&&... args) {
  if (a.bits == 0) return F<0>::run(args...);
  return dispatch_bits<F>(a.bits, args...);
}

// The layout's own bytes; the routing check's count follows them.
// The small-P path, unless a group would have more members than its arrival
// counter can count (k ranges of at most kGemvMaxKc rows keep that far off
// for any realistic width).
static bool unit_path(const ArenaDesc& gu, const ArenaDesc& dn, int64_t P, int topk) {
  if (P > kGroupedUnitMaxPairs) return false;
  const UnitLayout L = unit_layout(gu, dn, P);
  return 2 * L.s_gu <= GemvCtr::kMaxArrivals && topk * L.s_dn <= GemvCtr::kMaxArrivals;
}

static size_t layout_bytes(const ArenaDesc& gu, const ArenaDesc& dn, int64_t P, int topk) {
  return unit_path(gu, dn, P, topk) ? unit_layout(gu, dn, P).total : gemm_layout(gu, dn, P).total;
}

size_t grouped_workspace(const ArenaDesc& gu, const ArenaDesc& dn, int64_t t, int topk) {
  return layout_bytes(gu, dn, t * topk, topk) + 256;
}

// Routing check (debug option): one workgroup counts the ids outside
// [0, E) and stores the count (no atomics on global memory, no clearing
// launch).  Reads ids[0 .. P) only.
constexpr int kCheckThreads = 1024;
__global__ __launch_bounds__(kCheckThreads) void check_ids_kernel(const int32_t* __restrict__ ids,
                                                                  int64_t P, int E,
                                                                  unsigned int* __restrict__ bad) {
  __shared__ unsigned int cnt;
  if (threadIdx.x == 0) cnt = 0;
  __syncthreads();
  unsigned int mine = 0;
  for (int64_t i = threadIdx.x; i < P; i += kCheckThreads) {
    const int e = ids[i];
    mine += (e < 0 || e >= E) ? 1u : 0u;
  }
  if (mine) atomicAdd(&cnt, mine);
  __syncthreads();
  if (threadIdx.x == 0) *bad = cnt;
}

hipError_t count_bad_ids(const ArenaDesc& gu, const ArenaDesc& dn, const int32_t* ids, int64_t t,
                         int topk, void* ws, hipStream_t s, unsigned int& bad) {
  const int64_t P = t * topk;
  unsigned int* dev = reinterpret_cast<unsigned int*>(static_cast<unsigned char*>(ws) +
                                                      layout_bytes(gu, dn, P, topk));
  hipLaunchKernelGGL(check_ids_kernel, dim3(1), dim3(kCheckThreads), 0, s, ids, P, gu.experts, dev);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if ((e = hipMemcpyAsync(&bad, dev, sizeof(bad), hipMemcpyDeviceToHost, s)) != hipSuccess) return e;
  return hipStreamSynchronize(s);
}

hipError_t launch_grouped(const ArenaDesc& gu, const ArenaDesc& dn, const uint16_t* x,
                          const int32_t* ids, const float* w, int64_t t, int topk, float* y,
                          void* ws, size_t /*ws_bytes*/, bool off_xcd_all, hipStream_t s) {
  const int64_t P = t * topk;
  const int hidden = gu.k, inter = gu.n;
  unsigned char* base = static_cast<unsigned char*>(ws);
  hipError_t e;
  if (unit_path(gu, dn, P, topk)) {
    const UnitLayout L = unit_layout(gu, dn, P);
    unsigned int* ctr_gu = reinterpret_cast<unsigned int*>(base + L.ctr_gu);
    unsigned int* ctr_dn = reinterpret_cast<unsigned int*>(base + L.ctr_dn);
    float* part_gu = reinterpret_cast<float*>(base + L.part_gu);
    uint16_t* xd = reinterpret_cast<uint16_t*>(base + L.xd);
    float* part_dn = reinterpret_cast<float*>(base + L.part_dn);
    GuUnitRes rg{gu.trellis, gu.suh, gu.svh, words_per_bit(gu) * gu.bits, hidden, inter, x, topk,
                 ids, part_gu, L.s_gu, ctr_gu, dn.suh, xd, (int)P};
    rg.ew = arena_widths(gu);
    rg.off_xcd_all = off_xcd_all ? 1 : 0;
    const int kc_g = hidden / L.s_gu;
    e = run_widths<GuUnitRun>(gu, rg, hidden, inter, (int)(P * 2), kc_g, s);
    if (e != hipSuccess) return e;
    DnUnitRes rd{dn.trellis, dn.svh, words_per_bit(dn) * dn.bits, inter, hidden, xd, ids, w, topk,
                 part_dn, L.s_dn, ctr_dn, y, (int)t};
    rd.ew = arena_widths(dn);
    rd.off_xcd_all = off_xcd_all ? 1 : 0;
    const int kc_d = inter / L.s_dn;
    return run_widths<DnUnitRun>(dn, rd, inter, hidden, (int)P, kc_d, s);
  }

  const GemmLayout L = gemm_layout(gu, dn, P);
  const int E = gu.experts;
  int32_t* hist = reinterpret_cast<int32_t*>(base + L.hist);
  int32_t* offsets = reinterpret_cast<int32_t*>(base + L.offsets);
  int32_t* ntiles = reinterpret_cast<int32_t*>(base + L.ntiles);
  TileEntry* tiles = reinterpret_cast<TileEntry*>(base + L.tiles);
  int32_t* pos = reinterpret_cast<int32_t*>(base + L.pos);
  int32_t* sorted = reinterpret_cast<int32_t*>(base + L.sorted);
  uint16_t* xg = reinterpret_cast<uint16_t*>(base + L.xg);
  uint16_t* xd = reinterpret_cast<uint16_t*>(base + L.xd);
  float* dbuf = reinterpret_cast<float*>(base + L.d);

  const int64_t chunks = bin_chunks(P);
  hipLaunchKernelGGL(bin_count, dim3((unsigned)chunks), dim3(kBinThreads), 0, s, ids, P, E, hist);
  hipLaunchKernelGGL(bin_plan, dim3(1), dim3(kPlanThreads), 0, s, hist, (int)chunks, E, L.bm,
                     offsets, ntiles, tiles);
  hipLaunchKernelGGL(bin_scatter, dim3((unsigned)chunks), dim3(kBinThreads), 0, s, ids, P, E, hist,
                     pos, sorted);
  {
    const int64_t tasks = P;  // one wave each
    hipLaunchKernelGGL(gu_input_transform, dim3((unsigned)((tasks + 3) / 4)), dim3(256), 0, s, x,
                       topk, P, hidden, sorted, ids, gu.suh, xg);
  }
  if ((e = hipGetLastError()) != hipSuccess) return e;
  GroupedGateUpRes rg{tiles, ntiles, xg, P, hidden, inter, gu.trellis, gu.svh, dn.suh,
                      words_per_bit(gu) * gu.bits, xd};
  rg.ew = arena_widths(gu);
  e = run_widths<GroupedGateUpRun>(gu, rg, L.bm, L.max_tiles, s);
  if (e != hipSuccess) return e;
  GroupedGemmRes rd{tiles, ntiles, xd, P, inter, hidden, dn.trellis, dn.svh, 1,
                    words_per_bit(dn) * dn.bits, dbuf};
  rd.ew = arena_widths(dn);
  e = run_widths<GroupedGemmRun>(dn, rd, L.bm, L.max_tiles, s);
  if (e != hipSuccess) return e;
  {
    const int64_t n4 = t * (hidden / 4);
    hipLaunchKernelGGL(combine_rows, dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, s, dbuf, pos,
                       w, t, topk, hidden, y);
  }
  return hipGetLastError();
}

}  // namespace exl3
