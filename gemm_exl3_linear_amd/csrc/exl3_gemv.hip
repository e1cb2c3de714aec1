// Decode GEMV for 1..16 activation rows (the memory-bound regime: each
// trellis word is read from HBM exactly once per call).
//
// y = ((x .* suh) Hk  W~  Hn) .* svh (+ bias)   (exl3xpu README, "Prefill:
// int8 linears ...": the product runs in the Hadamard domain; "Layout": the
// Hadamard-in and Hadamard-out kernels around the vector GEMV).
//
// Dense tensors run the matrix-core kernel of exl3_gemv_mf.hpp followed by
// its finishing launch; the several-tensor call (m == 1) runs the persistent
// stream-k kernel of exl3_gemv_sk.hpp followed by its finishing launch.  The workgroup-per-(block, k range)
// gemv_kernel of exl3_gemv.hpp serves the grouped experts' small-batch path;
// its planning helpers live here.
#include "exl3_device.hpp"
#include "exl3_gemv.hpp"
#include "exl3_gemv_mf.hpp"
#include "exl3_gemv_sk.hpp"
#include "exl3_internal.hpp"

namespace exl3 {

// ---------------------------------------------------------------------------
// planning and launch (dense tensors)
// ---------------------------------------------------------------------------
size_t gemv_lds_bytes(int kc, int m, int nw) {
  const size_t xs = ((size_t)kc * m * 2 + 15) & ~(size_t)15;
  const size_t tr = (size_t)nw * 64 * 20 * 4;
  const size_t red = (size_t)nw * m * 128 * 4;
  return xs + (tr > red ? tr : red);
}

int gemv_prefetch(int kc, int nw) {
  const int cnt = kc / (16 * nw);  // k tiles per wave
  return (cnt % 8 == 0) ? 8 : (cnt % 4 == 0) ? 4 : (cnt % 2 == 0) ? 2 : 1;
}

// Split of k into ranges of kc rows (kc a multiple of 128).  Preference: at
// least target_wgs workgroups in all, then the deepest prefetch (8 loads in
// flight per lane), then the fewest splits.  While the grid has fewer than
// 4 target_wgs output groups, a range is at most kGemvMaxKc rows: there each
// workgroup's serial chain (input transform, loads, decode, partial store,
// arrival) is what the call waits for.  Measured on MI355X for the routed
// experts (256 x (2048 -> 2 x 512 -> 2048), K=3, top-8): T=1 21.8 us and
// T=2 24.8 us against 28.7 and 33.8 with 1024 target workgroups and no cap;
// T=4 34.0 against 36.2; T=16..64 unchanged.
int gemv_choose_splits(int k, int groups, int m, int target_wgs) {
  const int kb = k / 128;
  int best = -1, best_score = -1;
  for (int s = 1; s <= kb; ++s) {
    if (kb % s) continue;
    const int kc = k / s;
    if (gemv_lds_bytes(kc, m) > kGemvMaxLds) continue;
    if (kc > kGemvMaxKc && (int64_t)groups < 4 * target_wgs) continue;
    const bool enough = (int64_t)groups * s >= target_wgs;
    const int score = (enough ? 100 : 0) + gemv_prefetch(kc);
    if (score > best_score) { best = s; best_score = score; }
  }
  return best > 0 ? best : kb;
}

// Runs of R row steps over W waves (or workgroups), the first H of which (the
// first-round ones) take runs w1 / w2 times longer than the others.  Falls back to equal runs (H = W) when the weighted split would
// leave a wave without a step or exceed max_run.
SkSplit make_sk_split(int64_t R, int64_t W, int64_t H, int64_t max_run, int64_t w1, int64_t w2) {
  SkSplit s;
  int64_t B1 = R;
  if (H > 0 && H < W) {
    const int64_t den = H * w1 + (W - H) * w2;
    B1 = (R * H * w1 + den / 2) / den;
    if (B1 < H || R - B1 < W - H || (B1 + H - 1) / H > max_run) {
      H = W;
      B1 = R;
    }
  } else if (H <= 0 && W > 0) {
    H = 0;
    B1 = 0;
  } else {
    H = W;
  }
  s.H = (int)H;
  s.B1 = (int)B1;
  s.q = H > 0 ? (int)(B1 / H) : 0;
  s.rem = H > 0 ? (int)(B1 - (int64_t)s.q * H) : 0;
  s.q2 = W > H ? (int)((R - B1) / (W - H)) : 0;
  s.rem2 = W > H ? (int)((R - B1) - (int64_t)s.q2 * (W - H)) : 0;
  return s;
}

// first-tier waves of a grid whose waves [first, first + W) are part of a
// launch: those dispatched in the first round, when the launch has a second
// round at all
int sk_first_round(int64_t first, int64_t W, int64_t total) {
  if (total <= kGemvRoundWaves || total > 2 * kGemvRoundWaves) return (int)W;
  const int64_t h = kGemvRoundWaves - first;
  return (int)(h < 0 ? 0 : h > W ? W : h);
}

// most partial slots any block receives, and the longest run
static void sk_split_extent(const SkSplit& s, int64_t KT, int64_t NB, int64_t W, int& slots, int& longest) {
  slots = 1;
  for (int64_t nb = 0; nb < NB; ++nb) {
    const int a = sk_arrivals(s, (int)nb, (int)KT);
    if (a > slots) slots = a;
  }
  longest = 0;
  if (s.H > 0) longest = s.q + (s.rem > 0 ? 1 : 0);
  if (W > s.H && s.q2 + (s.rem2 > 0 ? 1 : 0) > longest) longest = s.q2 + (s.rem2 > 0 ? 1 : 0);
}

// Plan of the dense decode GEMV (exl3_gemv_mf.hpp): W workgroups
// (kMfWorkgroups = two per CU of the 256-CU MI355X, all resident at once;
// one per CU for tensors of at most kMfRoundWorkgroups x kMfSmallRun units,
// which then have half the partial slots and no CU shared by two workgroups;
// more when runs would exceed kMfMaxRunWG units, fewer for tiny tensors),
// their runs over the units (k tile x 256-column pair) in two tiers (the
// kMfRoundWorkgroups dispatched first take runs kMfTierWeight1 /
// kMfTierWeight2 longer), the number of partial slots a pair can receive,
// and the workspace (fp32 partials: four wave slots per workgroup slot for
// m <= kMfLdsRows, one otherwise; then the transformed activations when
// m > kMfLdsRows).  The plan depends on (k, n) only, so every m from 1 to 16
// sums in the same order.  No device query.
static GemvPlan plan_gemv_new(int k, int n, int m) {
  GemvPlan p;
  const int64_t KT = k / 16, NB = n / 128, NP = (NB + 1) / 2, R = KT * NP;
  int64_t W = R <= (int64_t)kMfRoundWorkgroups * kMfSmallRun ? kMfRoundWorkgroups : kMfWorkgroups;
  if (W < (R + kMfMaxRunWG - 1) / kMfMaxRunWG) W = (R + kMfMaxRunWG - 1) / kMfMaxRunWG;
  if (W > R) W = R;  // runs of at least one unit
  p.split = make_sk_split(R, W, W > kMfRoundWorkgroups ? kMfRoundWorkgroups : W, kMfMaxRunWG, kMfTierWeight1,
                          kMfTierWeight2);
  p.splits = (int)W;
  sk_split_extent(p.split, KT, NP, W, p.slots, p.kc);
  const size_t per_slot = (m <= kMfLdsRows ? 4 : 1) * (size_t)m * 256 * sizeof(float);  // wave or workgroup slots
  p.xprep_off = ((size_t)NP * p.slots * per_slot + 255) & ~(size_t)255;
  p.ws = p.xprep_off + (m > kMfLdsRows ? (size_t)m * k * sizeof(uint16_t) : 0);
  return p;
}

// A plan depends on (k, n, m) only; each host thread keeps the last few it
// made, so a call (which plans twice: the workspace check, then the launch)
// costs a lookup instead of the split arithmetic.
constexpr int kPlanMemo = 16;
GemvPlan plan_gemv(int k, int n, int m) {
  struct Entry {
    int k, n, m;
    GemvPlan p;
  };
  static thread_local Entry memo[kPlanMemo];
  static thread_local int used = 0, next = 0;
  for (int i = 0; i < used; ++i)
    if (memo[i].k == k && memo[i].n == n && memo[i].m == m) return memo[i].p;
  const GemvPlan p = plan_gemv_new(k, n, m);
  memo[next] = Entry{k, n, m, p};
  next = (next + 1) % kPlanMemo;
  if (used < kPlanMemo) ++used;
  return p;
}

template <int K>
struct MfRun {
  static hipError_t run(const MfArgs& a, const GemvPlan& plan, hipStream_t s) {
    (void)plan;
    const dim3 grid((unsigned)a.W);
    if (a.m == 1)
      hipLaunchKernelGGL((gemv_mf_kernel<K, 1>), grid, dim3(256), 0, s, a);
    else if (a.m <= kMfLdsRows)
      hipLaunchKernelGGL((gemv_mf_kernel<K, kMfLdsRows>), grid, dim3(256), 0, s, a);
    else
      hipLaunchKernelGGL((gemv_mf_kernel<K, 0>), grid, dim3(256), 0, s, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int tasks = (a.n / 128) * a.m;  // one 64-thread workgroup each
    if (a.m <= kMfLdsRows)
      hipLaunchKernelGGL(gemv_mf_finish<true>, dim3((unsigned)tasks), dim3(64), 0, s, a);
    else
      hipLaunchKernelGGL(gemv_mf_finish<false>, dim3((unsigned)tasks), dim3(64), 0, s, a);
    return hipGetLastError();
  }
};

hipError_t launch_gemv(const uint16_t* trellis, const uint16_t* suh, const uint16_t* svh,
                       const uint16_t* bias, int k, int n, int bits, const uint16_t* x, int m,
                       int64_t ldx, void* y, int64_t ldy, bool y_f32, void* ws,
                       const GemvPlan& plan, hipStream_t s) {
  unsigned char* base = static_cast<unsigned char*>(ws);
  uint16_t* xprep = nullptr;
  if (m > kMfLdsRows) {
    // one input-transform launch for all rows (the arithmetic of the waves'
    // own transform at fewer rows, so a row's x' does not depend on m)
    xprep = reinterpret_cast<uint16_t*>(base + plan.xprep_off);
    const int tasks = m * ((k / 128 + 3) / 4);
    hipLaunchKernelGGL(gemv_xprep_kernel, dim3((unsigned)((tasks + 3) / 4)), dim3(256), 0, s, x, ldx, suh, m, k,
                       xprep);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  MfArgs a;
  a.trellis = trellis;
  a.suh = suh;
  a.x = x;
  a.ldx = ldx;
  a.xprep = xprep;
  a.m = m;
  a.k = k;
  a.n = n;
  a.KT = k / 16;
  a.NP = (n / 128 + 1) / 2;
  a.R = a.KT * a.NP;
  a.W = plan.splits;
  a.sp = plan.split;
  a.slots = plan.slots;
  a.part = reinterpret_cast<float*>(base);  // the partials start the workspace
  a.svh = svh;
  a.bias = bias;
  a.y = y;
  a.ldy = ldy;
  a.y_f32 = y_f32 ? 1 : 0;
  return dispatch_bits<MfRun>(bits, a, plan, s);
}

// ---------------------------------------------------------------------------
// several tensors sharing one activation row (m == 1), one launch pair
// ---------------------------------------------------------------------------
// Waves per tensor: kGemvSkWaves (kGemvRoundWaves, one per SIMD, for calls
// of at most 16384 units) in proportion to the tensors' trellis bytes,
// each at least ceil(R_i / kSkMaxRun) and at most R_i, rounded up to a
// multiple of 4; each tensor's waves split their runs in two tiers by the
// launch's first round.  Partials of tensor i follow those of i - 1.
static_assert(kMultiMax == kSkMaxMulti, "multi-tensor limits differ");

static MultiPlan plan_gemv_multi_new(const MultiTensor* t, int count, int k) {
  MultiPlan mp;
  mp.count = count;
  double total = 0;
  for (int i = 0; i < count; ++i) total += (double)t[i].n * t[i].bits;
  const int64_t KT = k / 16;
  int64_t units = 0;
  for (int i = 0; i < count; ++i) units += KT * (t[i].n / 128);
  const int waves_total = units <= 16384 ? kGemvRoundWaves : kGemvSkWaves;
  int64_t wsum = 0, tasks = 0;
  for (int i = 0; i < count; ++i) {
    const int64_t NB = t[i].n / 128, R = KT * NB;
    int64_t W = (int64_t)((double)waves_total * t[i].n * t[i].bits / total + 0.5);
    if (W < (R + kSkMaxRun - 1) / kSkMaxRun) W = (R + kSkMaxRun - 1) / kSkMaxRun;
    W = (W + 3) / 4 * 4;
    if (W > R) W = (R + 3) / 4 * 4;
    if (W < 4) W = 4;
    mp.waves[i] = (int)W;
    mp.wbase[i] = (int)wsum;
    mp.fbase[i] = (int)tasks;
    wsum += W;
    tasks += NB;
  }
  mp.wbase[count] = (int)wsum;
  mp.fbase[count] = (int)tasks;
  // runs once the whole grid is known (the first round spans tensors)
  size_t off = 0;
  for (int i = 0; i < count; ++i) {
    const int64_t NB = t[i].n / 128, R = KT * NB, W = mp.waves[i];
    mp.split[i] = make_sk_split(R, W, sk_first_round(mp.wbase[i], W, wsum), kSkMaxRun, kSkTierWeight1,
                                kSkTierWeight2);
    int longest;
    sk_split_extent(mp.split[i], KT, NB, W, mp.slots[i], longest);
    mp.part_off[i] = off;
    off += ((size_t)NB * mp.slots[i] * 128 * sizeof(float) + 255) & ~(size_t)255;
  }
  mp.ws = off;
  return mp;
}

// Memo of the last few multi-tensor plans of this host thread, keyed by k
// and the tensors' (n, bits) in order, as for plan_gemv.
MultiPlan plan_gemv_multi(const MultiTensor* t, int count, int k) {
  struct Entry {
    int count, k;
    int n[kMultiMax], bits[kMultiMax];
    MultiPlan p;
  };
  static thread_local Entry memo[kPlanMemo];
  static thread_local int used = 0, next = 0;
  for (int i = 0; i < used; ++i) {
    const Entry& e = memo[i];
    if (e.count != count || e.k != k) continue;
    bool same = true;
    for (int j = 0; j < count && same; ++j) same = e.n[j] == t[j].n && e.bits[j] == t[j].bits;
    if (same) return e.p;
  }
  Entry e;
  e.count = count;
  e.k = k;
  for (int j = 0; j < count; ++j) {
    e.n[j] = t[j].n;
    e.bits[j] = t[j].bits;
  }
  e.p = plan_gemv_multi_new(t, count, k);
  memo[next] = e;
  next = (next + 1) % kPlanMemo;
  if (used < kPlanMemo) ++used;
  return e.p;
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
    a.m = 1;
    a.k = k;
    a.n = t[i].n;
    a.KT = k / 16;
    a.R = a.KT * (a.n / 128);
    a.W = mp.waves[i];
    a.sp = mp.split[i];
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
