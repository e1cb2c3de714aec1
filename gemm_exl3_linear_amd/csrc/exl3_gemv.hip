// Decode GEMV for 1..16 activation rows (the memory-bound regime: each
// trellis word is read from HBM exactly once per call).
//
// y = ((x .* suh) Hk  W~  Hn) .* svh (+ bias)   (exl3xpu README, "Prefill:
// int8 linears ...": the product runs in the Hadamard domain; "Layout": the
// Hadamard-in and Hadamard-out kernels around the vector GEMV).
//
// gemv_kernel, one workgroup per (128-column block, k range[, unit]):
//   prologue  x' = (x .* suh) H for the workgroup's k range, fp16, into LDS
//   main loop each wave walks k tiles; lane (t, p) streams the row pair p of
//             n-tile t with one coalesced load, decodes 32 weights in
//             registers into k-pairs, and hands them to the matrix cores
//             through a small per-wave LDS transpose (MFMA 16x16x16 f16, the
//             activation rows padded to 16, fp32 accumulation)
//   end       the four waves' partial sums are added in a fixed order and
//             written to the fp32 workspace, one slice per k range; the
//             workgroup then counts itself in on its 128-column block, and
//             the last one to arrive adds the slices in k order, applies the
//             output transform, svh and bias, casts, and resets the counter.
// One launch per call.  The sums never depend on arrival order, so results
// are bit-reproducible, and every row is computed the same way whatever m is.
#include "exl3_device.hpp"
#include "exl3_gemv.hpp"
#include "exl3_gemv_sk.hpp"
#include "exl3_internal.hpp"

namespace exl3 {

// ---------------------------------------------------------------------------
// planning and launch (dense tensors)
// ---------------------------------------------------------------------------
size_t gemv_lds_bytes(int kc, int m) {
  const size_t xs = ((size_t)kc * m * 2 + 15) & ~(size_t)15;
  const size_t tr = 4 * 64 * 20 * 4;
  const size_t red = (size_t)4 * m * 128 * 4;
  return xs + (tr > red ? tr : red);
}

int gemv_prefetch(int kc) {
  const int cnt = kc / 64;  // k tiles per wave
  return (cnt % 8 == 0) ? 8 : (cnt % 4 == 0) ? 4 : 2;
}

// Split of k into ranges of kc rows (kc a multiple of 128).  Preference: at
// least target_wgs workgroups in all, then the deepest prefetch (8 loads in
// flight per lane), then the fewest splits.
int gemv_choose_splits(int k, int groups, int m, int target_wgs) {
  const int kb = k / 128;
  int best = -1, best_score = -1;
  for (int s = 1; s <= kb; ++s) {
    if (kb % s) continue;
    const int kc = k / s;
    if (gemv_lds_bytes(kc, m) > kGemvMaxLds) continue;
    const bool enough = (int64_t)groups * s >= target_wgs;
    const int score = (enough ? 100 : 0) + gemv_prefetch(kc);
    if (score > best_score) { best = s; best_score = score; }
  }
  return best > 0 ? best : kb;
}

// Stream-k plan of the dense decode GEMV: G workgroups (kGemvSkWorkgroups =
// two per CU of the 256-CU MI355X, fewer for small tensors, enough that a run
// spans at most 48 units), the number of partial slots an n block can
// receive, LDS and workspace sizes.  The plan depends on (k, n) only, so every
// m <= 16 sees the same summation order, and it needs no device query.
GemvPlan plan_gemv(int k, int n, int m) {
  GemvPlan p;
  const int64_t KB = k / 128, NB = n / 128, U = KB * NB;
  int64_t G = kGemvSkWorkgroups;
  if (G > U) G = U;
  if (G < (U + 47) / 48) G = (U + 47) / 48;
  // at most kSkMaxSlots runs may meet one n block: runs of >= KB / (slots - 2) units
  {
    const int64_t min_run = (KB + kSkMaxSlots - 3) / (kSkMaxSlots - 2);
    if (U / G < min_run) G = U / min_run > 0 ? U / min_run : 1;
  }
  const int64_t run_min = U / G, run_max = (U + G - 1) / G;
  p.splits = (int)G;
  p.kc = (int)run_max;  // units per workgroup at most
  p.slots = (int)((KB - 1 + run_min - 1) / run_min + 1);
  p.lds = (((size_t)run_max * m * 256 + 15) & ~(size_t)15) + (size_t)4 * m * 512 +
          (m > 1 ? (size_t)4 * 64 * 20 * 4 : 0);
  p.ctr_bytes = ((size_t)NB * 4 + 255) & ~(size_t)255;
  p.xprep_off = p.ctr_bytes + (((size_t)NB * p.slots * m * 128 * sizeof(float) + 255) & ~(size_t)255);
  p.ws = p.xprep_off + (m > 1 ? (size_t)m * k * sizeof(uint16_t) : 0);
  return p;
}

template <int K>
struct SkRun {
  static hipError_t run(const SkArgs& a, const GemvPlan& plan, hipStream_t s) {
    const dim3 grid((unsigned)a.G);
    if (a.m == 1)
      hipLaunchKernelGGL((gemv_sk_kernel<K, true, 8>), grid, dim3(256), plan.lds, s, a);
    else
      hipLaunchKernelGGL((gemv_sk_kernel<K, false, 8>), grid, dim3(256), plan.lds, s, a);
    return hipGetLastError();
  }
};

hipError_t launch_gemv(const uint16_t* trellis, const uint16_t* suh, const uint16_t* svh,
                       const uint16_t* bias, int k, int n, int bits, const uint16_t* x, int m,
                       int64_t ldx, void* y, int64_t ldy, bool y_f32, void* ws,
                       const GemvPlan& plan, hipStream_t s) {
  unsigned char* base = static_cast<unsigned char*>(ws);
  uint16_t* xprep = nullptr;
  if (m > 1) {
    // several rows: one input-transform launch for all of them, instead of
    // every workgroup transforming the blocks it needs
    xprep = reinterpret_cast<uint16_t*>(base + plan.xprep_off);
    const hipError_t e = launch_hadamard(x, false, xprep, false, m, k, ldx, k, suh, nullptr, s);
    if (e != hipSuccess) return e;
  }
  SkArgs a;
  a.trellis = trellis;
  a.suh = suh;
  a.x = x;
  a.ldx = ldx;
  a.xprep = xprep;
  a.m = m;
  a.k = k;
  a.n = n;
  a.KB = k / 128;
  a.NB = n / 128;
  a.U = (int64_t)a.KB * a.NB;
  a.G = plan.splits;
  a.slots = plan.slots;
  a.part = reinterpret_cast<float*>(base + plan.ctr_bytes);
  a.ctr = reinterpret_cast<unsigned int*>(base);
  a.svh = svh;
  a.bias = bias;
  a.y = y;
  a.ldy = ldy;
  a.y_f32 = y_f32 ? 1 : 0;
  return dispatch_bits<SkRun>(bits, a, plan, s);
}

}  // namespace exl3
