// Decode GEMV for 1..16 activation rows (the memory-bound regime: each
// trellis word is read from HBM exactly once per call).
//
// y = ((x .* suh) Hk  W~  Hn) .* svh (+ bias)   (exl3xpu README, "Prefill:
// int8 linears ...": the product runs in the Hadamard domain; "Layout": the
// Hadamard-in and Hadamard-out kernels around the vector GEMV).
//
// Dense tensors run the persistent stream-k kernel of exl3_gemv_sk.hpp
// followed by its finishing launch.  The workgroup-per-(block, k range)
// gemv_kernel of exl3_gemv.hpp serves the grouped experts' small-batch path;
// its planning helpers live here.
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

// Plan of the dense decode GEMV: W waves (kGemvSkWaves = eight per CU of the
// 256-CU MI355X; more when runs would exceed 48 row steps, fewer for small
// tensors), the number of partial slots a block can receive, and the
// workspace (fp32 partials, then the transformed activations when m > 1).
// The plan depends on (k, n) only, so every m <= 16 sees the same summation
// order, and it needs no device query.
GemvPlan plan_gemv(int k, int n, int m) {
  GemvPlan p;
  const int64_t KT = k / 16, NB = n / 128, R = KT * NB;
  int64_t W = kGemvSkWaves;
  if (W < (R + 47) / 48) W = (R + 47) / 48;
  W = (W + 3) / 4 * 4;
  if (W > R) W = (R + 3) / 4 * 4;  // runs of at least one row step (extra waves idle)
  const int64_t run_min = R / W > 0 ? R / W : 1;
  p.splits = (int)W;
  p.kc = (int)((R + W - 1) / W);
  p.slots = (int)((KT - 1 + run_min - 1) / run_min + 1);
  p.lds = 0;
  p.ctr_bytes = 0;
  p.xprep_off = (((size_t)NB * p.slots * m * 128 * sizeof(float) + 255) & ~(size_t)255);
  p.ws = p.xprep_off + (m > 1 ? (size_t)m * k * sizeof(uint16_t) : 0);
  return p;
}

template <int K>
struct SkRun {
  static hipError_t run(const SkArgs& a, const GemvPlan& plan, hipStream_t s) {
    const dim3 grid((unsigned)(a.W / 4));
    if (a.m == 1)
      hipLaunchKernelGGL((gemv_sk_kernel<K, true, 4>), grid, dim3(256), 0, s, a);
    else
      hipLaunchKernelGGL((gemv_sk_kernel<K, false, 8>), grid, dim3(256), 0, s, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int tasks = (a.n / 128) * a.m;  // one 64-thread workgroup each
    hipLaunchKernelGGL(gemv_sk_finish, dim3((unsigned)tasks), dim3(64), 0, s, a);
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
  a.KT = k / 16;
  a.R = a.KT * (n / 128);
  a.W = plan.splits;
  a.q = a.R / a.W;
  a.rem = a.R - a.q * a.W;
  a.slots = plan.slots;
  a.part = reinterpret_cast<float*>(base + plan.ctr_bytes);
  a.svh = svh;
  a.bias = bias;
  a.y = y;
  a.ldy = ldy;
  a.y_f32 = y_f32 ? 1 : 0;
  return dispatch_bits<SkRun>(bits, a, plan, s);
}

// ---------------------------------------------------------------------------
// several tensors sharing one activation row (m == 1), one launch pair
// ---------------------------------------------------------------------------
// Waves per tensor: kGemvSkWaves in proportion to the tensors' trellis bytes,
// each at least ceil(R_i / 48) (runs of at most 48 row steps) and at most R_i,
// rounded up to a multiple of 4.  Partials of tensor i follow those of i - 1.
static_assert(kMultiMax == kSkMaxMulti, "multi-tensor limits differ");

MultiPlan plan_gemv_multi(const MultiTensor* t, int count, int k) {
  MultiPlan mp;
  mp.count = count;
  double total = 0;
  for (int i = 0; i < count; ++i) total += (double)t[i].n * t[i].bits;
  const int64_t KT = k / 16;
  size_t off = 0;
  int64_t wsum = 0, tasks = 0;
  for (int i = 0; i < count; ++i) {
    const int64_t NB = t[i].n / 128, R = KT * NB;
    int64_t W = (int64_t)((double)kGemvSkWaves * t[i].n * t[i].bits / total + 0.5);
    if (W < (R + 47) / 48) W = (R + 47) / 48;
    W = (W + 3) / 4 * 4;
    if (W > R) W = (R + 3) / 4 * 4;
    if (W < 4) W = 4;
    const int64_t run_min = R / W > 0 ? R / W : 1;
    mp.waves[i] = (int)W;
    mp.slots[i] = (int)((KT - 1 + run_min - 1) / run_min + 1);
    mp.part_off[i] = off;
    off += ((size_t)NB * mp.slots[i] * 128 * sizeof(float) + 255) & ~(size_t)255;
    mp.wbase[i] = (int)wsum;
    mp.fbase[i] = (int)tasks;
    wsum += W;
    tasks += NB;
  }
  mp.wbase[count] = (int)wsum;
  mp.fbase[count] = (int)tasks;
  mp.ws = off;
  return mp;
}

hipError_t launch_gemv_multi(const MultiTensor* t, int count, int k, const uint16_t* x, void* const* y,
                             const int64_t* ldy, bool y_f32, void* ws, const MultiPlan& mp,
                             hipStream_t s) {
  SkMulti ma;
  ma.count = count;
  unsigned char* base = static_cast<unsigned char*>(ws);
  for (int i = 0; i <= count; ++i) {
    ma.wbase[i] = mp.wbase[i];
    ma.fbase[i] = mp.fbase[i];
  }
  for (int i = 0; i < count; ++i) {
    SkArgs& a = ma.t[i];
    a.trellis = t[i].trellis;
    a.suh = t[i].suh;
    a.x = x;
    a.ldx = k;
    a.xprep = nullptr;
    a.m = 1;
    a.k = k;
    a.n = t[i].n;
    a.KT = k / 16;
    a.R = a.KT * (a.n / 128);
    a.W = mp.waves[i];
    a.q = a.R / a.W;
    a.rem = a.R - a.q * a.W;
    a.slots = mp.slots[i];
    a.part = reinterpret_cast<float*>(base + mp.part_off[i]);
    a.svh = t[i].svh;
    a.bias = t[i].bias;
    a.y = y[i];
    a.ldy = ldy[i];
    a.y_f32 = y_f32 ? 1 : 0;
    ma.bits[i] = t[i].bits;
  }
  hipLaunchKernelGGL((gemv_sk_multi_kernel<4>), dim3((unsigned)(mp.wbase[count] / 4)), dim3(256), 0, s,
                     ma);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(gemv_sk_multi_finish, dim3((unsigned)mp.fbase[count]), dim3(64), 0, s, ma);
  return hipGetLastError();
}

}  // namespace exl3
