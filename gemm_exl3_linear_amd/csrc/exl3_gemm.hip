// Dense prefill linear (m > 16): x' = (x .* suh) H is written once to the
// workspace, fragment-major, by the input kernel, then one fused decode + MFMA GEMM launch
// computes y = (x' W~) H .* svh (+ bias).  See exl3_gemm.hpp for the kernel.
#include "exl3_gemm.hpp"
#include "exl3_internal.hpp"

namespace exl3 {

struct DenseGemmRes {
  static constexpr bool kAFrag = true;  // x' is fragment-major
  static constexpr bool kFineSkip = false;  // only the last row tile is short
  static constexpr bool kGateUp = false;
  const uint16_t* a;
  int64_t lda;  // elements per 16-row group (16 k)
  int m;
  int bm;
  int mt;   // row tiles
  int nbt;  // 128-column tiles
  const uint16_t* trellis;
  const uint16_t* svh;
  const uint16_t* bias;
  void* y;
  int64_t ldy;
  bool y_f32;
  // Workgroup -> (row tile, column tile).  Workgroups are dispatched to the
  // eight XCDs round robin, so when the tile count is a multiple of eight the
  // workgroups of one XCD are given one contiguous range of the tile order.
  // The order walks groups of two row tiles across all column tiles, so the
  // workgroups resident on one XCD at a time share two row panels of x' (in
  // that XCD's L2) and each trellis column panel between two of them.
  __device__ GemmTask task() const {
    const int total = mt * nbt;
    const int bid = (int)blockIdx.x;
    const int u = (total % 8 == 0) ? (bid % 8) * (total / 8) + bid / 8 : bid;
    constexpr int G = 2;
    const int grp = u / (G * nbt), within = u - grp * (G * nbt);
    const int g0 = grp * G;
    const int gs = (mt - g0) < G ? (mt - g0) : G;
    const int mtile = g0 + within % gs;
    GemmTask T;
    T.nb = within / gs;
    const int r0 = mtile * bm;
    T.valid = r0 < m;
    T.a = a + (int64_t)(r0 >> 4) * lda;  // r0 is a multiple of 16
    T.lda = lda;
    T.rows = (m - r0) < bm ? (m - r0) : bm;
    T.trellis = trellis;
    T.svh = svh;
    T.bias = bias;
    T.y = y_f32 ? (void*)(static_cast<float*>(y) + (int64_t)r0 * ldy)
                : (void*)(static_cast<uint16_t*>(y) + (int64_t)r0 * ldy);
    T.ldy = ldy;
    return T;
  }
};

// Tile height: 256 rows, unless the grid would be small.  A launch of fewer
// than kGemmMinGrid workgroups leaves most CUs idle, so a narrow tensor at a
// few hundred rows takes 128- or 64-row tiles (more workgroups, each
// decoding its column block for fewer rows); with one or two row tiles the
// 128-row tile is taken when it pads fewer rows.  Measured on MI355X (fp16,
// K=4): 5120x5120 at m = 200 / 300 / 500 took 61 / 63 / 74 us against 94 /
// 95 / 97 with 256-row tiles, 17408x5120 at m = 200 188 against 292 us,
// 5120x17408 at m = 300 105 against 134 us; from m = 1000 256-row tiles were
// the fastest on every shape measured.
constexpr int64_t kGemmMinGrid = 128;
static int choose_bm(int64_t m, int64_t nbt) {
  if (m <= 64) return 64;
  const int64_t t256 = (m + 255) / 256, t128 = (m + 127) / 128;
  if (t256 * nbt >= kGemmMinGrid) return (t256 <= 2 && t128 * 128 < t256 * 256) ? 128 : 256;
  return t128 * nbt >= kGemmMinGrid ? 128 : 64;
}

template <int K>
struct DenseGemmRun {
  static hipError_t run(const DenseGemmRes& r, int k, int n, hipStream_t s) {
    const dim3 grid(r.mt * r.nbt);
#define EXL3_GEMM_LAUNCH(BM)                                                                    \
  do {                                                                                          \
    if (r.y_f32)                                                                                \
      hipLaunchKernelGGL((gemm_kernel<K, BM, true, DenseGemmRes>), grid, dim3(kGemmThreads), 0, s, r, k, n); \
    else                                                                                        \
      hipLaunchKernelGGL((gemm_kernel<K, BM, false, DenseGemmRes>), grid, dim3(kGemmThreads), 0, s, r, k, n); \
  } while (0)
    if (r.bm == 256) EXL3_GEMM_LAUNCH(256);
    else if (r.bm == 128) EXL3_GEMM_LAUNCH(128);
    else EXL3_GEMM_LAUNCH(64);
#undef EXL3_GEMM_LAUNCH
    return hipGetLastError();
  }
};

// The workspace holds x' (fp16, fragment-major, m rounded up to 16 rows).
static int64_t frag_rows(int64_t m) { return (m + 15) & ~(int64_t)15; }

size_t gemm_workspace(int k, int /*n*/, int m) { return (size_t)frag_rows(m) * k * sizeof(uint16_t); }

int64_t gemm_max_workgroups(int k, int n, int64_t m) {
  const int64_t frag = (m + 15) / 16 * (k / 128);  // launch_input_frag's grid at one block per workgroup (its largest)
  const int64_t nbt = (n + kGemmBN - 1) / kGemmBN;
  const int64_t bm = choose_bm(m, nbt);
  const int64_t gemm = (m + bm - 1) / bm * nbt;
  return frag > gemm ? frag : gemm;
}

hipError_t launch_gemm(const uint16_t* trellis, const uint16_t* suh, const uint16_t* svh,
                       const uint16_t* bias, int k, int n, int bits, const uint16_t* x, int m,
                       int64_t ldx, void* y, int64_t ldy, bool y_f32, void* ws, hipStream_t s) {
  uint16_t* xp = static_cast<uint16_t*>(ws);
  hipError_t e = launch_input_frag(x, ldx, m, k, suh, xp, s);
  if (e != hipSuccess) return e;
  const int bm = choose_bm(m, (n + kGemmBN - 1) / kGemmBN);
  DenseGemmRes r{xp, (int64_t)16 * k, m, bm, (m + bm - 1) / bm, (n + kGemmBN - 1) / kGemmBN, trellis,
                 svh, bias, y, ldy, y_f32};
  return dispatch_bits<DenseGemmRun>(bits, r, k, n, s);
}

}  // namespace exl3
