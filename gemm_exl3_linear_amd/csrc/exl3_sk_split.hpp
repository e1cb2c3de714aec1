// Stream-k runs of the dense decode GEMV: which contiguous range of row steps
// each wave of the persistent grid takes.  Shared by the planner (host) and
// the kernels (device), so both derive the same runs and partial slots.
#pragma once

#include <hip/hip_runtime.h>

namespace exl3 {

// Runs of R row steps over W waves.  Waves 0 .. H-1 share the first B1 steps
// (runs of q + 1 steps for the first rem of them, q for the rest); waves
// H .. W-1 share the remaining R - B1 steps the same way with (q2, rem2).
struct SkSplit {
  int H, q, rem;
  int B1, q2, rem2;
};

__host__ __device__ inline int sk_tier_start(int w, int q, int rem) {
  return w * q + (w < rem ? w : rem);
}
__host__ __device__ inline int sk_tier_owner(int r, int q, int rem) {
  const int big = rem * (q + 1);  // steps covered by the longer runs
  return r < big ? r / (q + 1) : rem + (r - big) / q;
}
// length and first row step of wave w's run
__host__ __device__ inline int sk_run_len(const SkSplit& s, int w) {
  return w < s.H ? s.q + (w < s.rem ? 1 : 0) : s.q2 + (w - s.H < s.rem2 ? 1 : 0);
}
__host__ __device__ inline int sk_run_start(const SkSplit& s, int w) {
  return w < s.H ? sk_tier_start(w, s.q, s.rem) : s.B1 + sk_tier_start(w - s.H, s.q2, s.rem2);
}
// wave whose run contains row step r
__host__ __device__ inline int sk_run_owner(const SkSplit& s, int r) {
  return r < s.B1 ? sk_tier_owner(r, s.q, s.rem) : s.H + sk_tier_owner(r - s.B1, s.q2, s.rem2);
}
// Slots of block nb: the waves whose runs intersect it, in run order.
__host__ __device__ inline int sk_arrivals(const SkSplit& s, int nb, int KT) {
  return sk_run_owner(s, (nb + 1) * KT - 1) - sk_run_owner(s, nb * KT) + 1;
}

}  // namespace exl3
