/*
 * exl3.h - C ABI of the MI355X (gfx950) EXL3 quantized-linear library.
 *
 * The operation (sources: the exl3xpu README, sections "MoE (routed experts)",
 * "Prefill: int8 linears ..." and "Adding a model"; the Arc 140V MoE post,
 * sections 1 and 2A-2D; TensorFold issue #832, "Description"):
 *
 *   An EXL3 tensor of shape k x n (k = in_features, n = out_features, both
 *   multiples of 128) stores 16x16 weight tiles as K-bit trellis codes
 *   (K = 1..8): a uint16 array trellis[k/16][n/16][16*K], plus fp16 sign
 *   vectors suh[k] and svh[n] and an optional fp16 bias[n].  Decoding a tile
 *   gives the Hadamard-domain weight W~ (fp16, k x n), and the layer is
 *
 *       y = ((x .* suh) Hk  W~  Hn) .* svh (+ bias)
 *
 *   where Hd applies the orthonormal 128-point Walsh-Hadamard transform
 *   (Sylvester order, scaled by 1/sqrt(128)) to each block of 128 consecutive
 *   elements.
 *
 *   Decode of tile (a, b): its 16*K words, read in index order and each word
 *   most-significant bit first, form a cyclic bitstream of 256*K bits.  State
 *   j (0..255) is the 16-bit window starting at bit K*j (wrapping around).
 *   The mul1 codebook (marker EXL3_CODEBOOK_MUL1, the pages' "cb=2") maps a
 *   state S to fp16_RN((sigma - 510) * 1775 / 2^18), sigma being the sum of
 *   the four bytes of (S * 0x9E3779) mod 2^32; every value lies within
 *   +-3.453125.  State j is weight W~[16a + j/16][16b + j%16].
 *
 * Conventions for every entry point:
 *   - Pointers named as device pointers must point to GPU memory of the
 *     current HIP device; the caller allocates and owns every buffer.  The
 *     library keeps no pointer after a call returns and allocates nothing.
 *   - Every call only enqueues work on `stream` (NULL = the default stream):
 *     no host synchronisation, no read-back of device data.
 *   - Arguments are validated on the host before anything is enqueued; on any
 *     error nothing is enqueued and a status other than EXL3_OK is returned.
 *     There is no fallback to another code path.
 *   - Device pointers must be 16-byte aligned unless stated otherwise.
 *   - A tensor holds fewer than 2^31 tiles: (k/16) * (n/16) < 2^31, and its
 *     trellis is smaller than 4 GiB (k * n * bits / 8 < 2^32 bytes); for an
 *     arena this holds for each (expert, slot) tensor, at width 8 when the
 *     width is per expert.
 *   - Sizes whose launches would not fit the hardware's grid limit (2^24 - 1
 *     workgroups of 256 threads) return EXL3_E_INVALID: calls with m > 2^24
 *     rows; prefill calls with ceil(m/16) * (k/128) or ceil(m/64) * (n/128)
 *     at or above that limit; exl3_reconstruct* with (k/16) * (n/16) >= 2^29;
 *     exl3_hadamard with rows * (dim/128) >= 2^26.  Workspace-size queries
 *     return 0 for m > 2^24.
 *   - Calls on different streams may run concurrently; a call must not
 *     overlap another call that writes the same output or workspace.
 */
#ifndef EXL3_H
#define EXL3_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define EXL3_ABI_VERSION 1

/* The only codebook this library decodes (the pages' "mul1", marker cb=2). */
#define EXL3_CODEBOOK_MUL1 2

/* Largest supported routing fan-out for exl3_grouped_experts. */
#define EXL3_MAX_TOPK 16

/* Largest number of tensors in one exl3_linear_multi call. */
#define EXL3_MAX_MULTI 8

typedef struct ihipStream_t* exl3_stream_t; /* same type as hipStream_t */

typedef enum exl3_status {
    EXL3_OK = 0,
    EXL3_E_INVALID = 1,     /* bad size, width, pointer or alignment */
    EXL3_E_UNSUPPORTED = 2, /* codebook other than mul1 (fail-closed) */
    EXL3_E_WORKSPACE = 3,   /* workspace missing or too small */
    EXL3_E_HIP = 4          /* a HIP launch reported an error */
} exl3_status;

typedef enum exl3_dtype {
    EXL3_F16 = 0,
    EXL3_F32 = 1
} exl3_dtype;

/* One EXL3 tensor (all pointers are device pointers).
 *   trellis  uint16 [k/16][n/16][16*bits], row-major, 16-byte aligned
 *   suh      fp16 [k] (sign applied before the input transform)
 *   svh      fp16 [n] (sign applied after the output transform)
 *   bias     fp16 [n] or NULL (added last)
 *   k, n     multiples of 128 (16 suffices for exl3_reconstruct)
 *   bits     trellis width K, 1..8
 *   codebook must be EXL3_CODEBOOK_MUL1                                   */
typedef struct exl3_weight {
    const uint16_t* trellis;
    const uint16_t* suh;
    const uint16_t* svh;
    const uint16_t* bias;
    int32_t k;
    int32_t n;
    int32_t bits;
    int32_t codebook;
} exl3_weight;

/* A packed arena of per-expert EXL3 tensors, one allocation per tensor kind
 * (Arc 140V MoE post, section 2A: w13 [E, 2, ...] and w2 [E, 1, ...]).
 *   trellis  uint16 [experts][slots][k/16][n/16][16*bits]
 *   suh      fp16 [experts][slots][k]
 *   svh      fp16 [experts][slots][n]
 * Width and codebook are uniform over the arena (exl3_grouped_experts), or
 * the width is per expert (exl3_expert_widths, exl3_grouped_experts_mixed). */
typedef struct exl3_expert_weights {
    const uint16_t* trellis;
    const uint16_t* suh;
    const uint16_t* svh;
    int32_t experts;
    int32_t slots;
    int32_t k;
    int32_t n;
    int32_t bits;
    int32_t codebook;
} exl3_expert_weights;

/* Returns EXL3_ABI_VERSION of the built library. */
int32_t exl3_abi_version(void);

/* Static, NUL-terminated description of a status code (never NULL). */
const char* exl3_status_str(exl3_status status);

/* exl3_reconstruct - decode a whole tensor to W~ (Hadamard domain, no signs).
 * The exl3xpu README ("Correctness") gates every kernel path on bit-identical
 * dequantized weights; this entry point exposes the decode for that check.
 *   w_out  fp16 [k][n] row-major, device pointer, 16-byte aligned.
 * Requires k, n multiples of 16.  Output is bit-exact by definition.       */
exl3_status exl3_reconstruct(const exl3_weight* w, uint16_t* w_out, exl3_stream_t stream);

/* exl3_hadamard - out = ((in .* sign_before) Hdim) .* sign_after, row by row
 * (the standalone randomized Hadamard transform of the exl3xpu README,
 * "Layout": Hadamard in/out kernels; and the MoE post, section 2C).
 *   in, out      [rows][ld_*] of `dtype` (EXL3_F16 or EXL3_F32); in-place
 *                (in == out with equal strides) is allowed
 *   dim          multiple of 128; transformed in blocks of 128
 *   ld_in/ld_out row strides in elements, >= dim, multiples of 8
 *   sign_before, sign_after  fp16 [dim] device pointers or NULL
 * Arithmetic is fp32; an fp16 output is rounded to nearest.               */
exl3_status exl3_hadamard(const void* in, void* out, int32_t dtype, int64_t rows, int64_t dim,
                          int64_t ld_in, int64_t ld_out, const uint16_t* sign_before,
                          const uint16_t* sign_after, exl3_stream_t stream);

/* Bytes of device workspace exl3_linear needs for m rows of this tensor
 * (0 if the arguments are invalid). */
size_t exl3_linear_workspace_size(const exl3_weight* w, int64_t m);

/* exl3_linear - y = ((x .* suh) Hk W~ Hn) .* svh (+ bias).
 * (exl3xpu README "Layout": the linear op dispatches on the row count; the
 * GEMM runs in the Hadamard domain per "Prefill: int8 linears ...";
 * TensorFold issue #832: rows are computed independently of the batch.)
 *   x      fp16 [m][ldx] device pointer, ldx >= k, ldx multiple of 8
 *   y      [m][ldy] of y_dtype (EXL3_F16 or EXL3_F32; fp32 outputs are the
 *          issue's "decodeF32/promptF32" contract), ldy >= n, multiple of 8
 *   ws     device workspace of at least exl3_linear_workspace_size(w, m)
 *          bytes (may be NULL when that size is 0): scratch of the call
 *          (partial sums, the transformed activations).  Nothing is kept in
 *          it between calls, so it needs no clearing and serves later calls
 *          of any size on the same stream; calls that overlap on it race.
 * m == 0 returns EXL3_OK without enqueueing anything.  The kernel (decode
 * GEMV for m <= 16, MFMA GEMM above) is chosen internally from m.  Within
 * each of the ranges 1 <= m <= 16 and m > 16 a row's result does not depend
 * on m or on the other rows (bit for bit); across them the summation order
 * differs, so results agree to rounding.
 * The trellis of the tensor must be smaller than 4 GiB (k * n * bits / 8 <
 * 2^32 bytes), else EXL3_E_INVALID.                                        */
exl3_status exl3_linear(const exl3_weight* w, const void* x, int64_t m, int64_t ldx, void* y,
                        int64_t ldy, int32_t y_dtype, void* ws, size_t ws_bytes,
                        exl3_stream_t stream);

/* Bytes of the device array behind exl3_linear_no_workspace (32 MiB). */
#define EXL3_SCRATCH_BYTES ((size_t)32 << 20)

/* exl3_linear_no_workspace - exl3_linear without a workspace argument, for
 * callers that cannot allocate device memory at all: code recorded into a
 * graph, tight serving loops, harnesses that forbid allocation.  The same
 * operation, arguments (minus ws and ws_bytes), validation, kernels and
 * results, bit for bit, as exl3_linear with a workspace.  The workspace is a
 * device array of EXL3_SCRATCH_BYTES that the library holds on every GPU it
 * runs on until the process ends; the call itself allocates nothing.
 *   - A call that needs more than EXL3_SCRATCH_BYTES of workspace
 *     (exl3_linear_workspace_size(w, m) > EXL3_SCRATCH_BYTES) returns
 *     EXL3_E_WORKSPACE with nothing enqueued.  Every decode call (m <= 16)
 *     of tensors up to 5120 x 17408 fits, and prefill calls while
 *     m * k * 2 bytes (plus a small head) fit.
 *   - All calls on one GPU share that GPU's array: two calls whose work
 *     overlaps in time on one GPU (other streams, other host threads) race
 *     and give undefined results.  Calls in order on one stream are safe.
 *     Nothing in the array needs to start at zero (these kernels keep no
 *     state in it between calls).
 *   - The first call on each GPU looks up the array's device address (a
 *     host-side query, nothing enqueued); make it outside graph capture.   */
exl3_status exl3_linear_no_workspace(const exl3_weight* w, const void* x, int64_t m, int64_t ldx,
                                     void* y, int64_t ldy, int32_t y_dtype, exl3_stream_t stream);

/* Bytes of device workspace exl3_linear_multi needs for m rows of these
 * tensors (0 if the arguments are invalid). */
size_t exl3_linear_multi_workspace_size(const exl3_weight* const* w, int32_t count, int64_t m);

/* exl3_linear_multi - y[i] = exl3_linear(w[i], x) for i < count, for the
 * projections that read one input (q, k and v; gate and up), each tensor with
 * its own width, shape, signs and bias (TensorFold issue #832,
 * "Description": widths are mixed per tensor; the fused multi-tensor launch
 * is the issue's "fused-shard" idea).
 *   w      host array of count tensor records, 1 <= count <= EXL3_MAX_MULTI,
 *          all with the same k (the records' buffers are device pointers)
 *   x      fp16 [m][ldx] device pointer, as for exl3_linear
 *   y      host array of count device pointers, y[i] is [m][ldy[i]] of
 *          y_dtype with ldy[i] >= w[i]->n, multiple of 8
 *   ws     device workspace of at least exl3_linear_multi_workspace_size
 *          bytes, scratch of the call as for exl3_linear
 * m == 1 runs all tensors in one decode-GEMV launch and one finishing
 * launch (each tensor keeps its own split over a share of the waves, in
 * proportion to its trellis bytes, so its results agree with exl3_linear to
 * rounding); m >= 2 runs the tensors one after another through exl3_linear
 * (bit-identical to separate calls).  m == 0 returns EXL3_OK.  Validation of
 * every tensor happens before anything is enqueued.                       */
exl3_status exl3_linear_multi(const exl3_weight* const* w, int32_t count, const void* x, int64_t m,
                              int64_t ldx, void* const* y, const int64_t* ldy, int32_t y_dtype,
                              void* ws, size_t ws_bytes, exl3_stream_t stream);

/* exl3_reconstruct_int8 - the int8 weights W_q of the int8 prefill (exl3xpu
 * README, "Prefill: int8 linears ...": one static weight scale fused into
 * reconstruct).  W_q = RNE((sigma - 510) * 1775 / 2^18 * 127 / 3.453125) for
 * each state's byte sum sigma, taken from the codebook value before its fp16
 * rounding; |W_q| <= 127.
 *   w_out  int8 [k][n] row-major, device pointer, 16-byte aligned.
 * Requires k, n multiples of 16.  Output is bit-exact by definition.       */
exl3_status exl3_reconstruct_int8(const exl3_weight* w, int8_t* w_out, exl3_stream_t stream);

/* Bytes of device workspace exl3_linear_int8 needs for m rows of this tensor
 * (0 if the arguments are invalid or m == 0). */
size_t exl3_linear_int8_workspace_size(const exl3_weight* w, int64_t m);

/* exl3_linear_int8 - the int8 prefill linear (exl3xpu README, "Prefill: int8
 * linears ..."): activations get one int8 scale per row inside the input
 * transform, weights the static scale of exl3_reconstruct_int8, and the
 * product runs on int8 matrix cores with both scales applied:
 *   x' = (x .* suh) Hk;  a_r = max |x'_r|;  x_q = RNE(127 x' / a_r)
 *   y  = ((x_q W_q) * (a_r / 127) * (3.453125 / 127)) Hn .* svh (+ bias)
 * The integer product is exact; x' and the scales are fp32.
 *   x, y, ldx, ldy, y_dtype  as for exl3_linear
 *   ws     device workspace of at least exl3_linear_int8_workspace_size(w, m)
 *          bytes (x_q and the row scales; no state is kept between calls)
 * Any m >= 1 is accepted (the pages use it for prefill, more than 128 rows);
 * rows are independent, so a row's result does not depend on m or on the
 * other rows, bit for bit.  An all-zero row gives y = bias.  m == 0 returns
 * EXL3_OK.  Compared with exl3_linear the outputs differ by the int8
 * rounding of activations and weights (about 1e-2 relative).              */
exl3_status exl3_linear_int8(const exl3_weight* w, const void* x, int64_t m, int64_t ldx, void* y,
                             int64_t ldy, int32_t y_dtype, void* ws, size_t ws_bytes,
                             exl3_stream_t stream);

/* Bytes of device workspace exl3_grouped_experts needs (0 if invalid). */
size_t exl3_grouped_experts_workspace_size(const exl3_expert_weights* gate_up,
                                           const exl3_expert_weights* down, int64_t t,
                                           int32_t topk);

/* exl3_grouped_experts - routed-expert SwiGLU MLP, routed contribution only.
 * (exl3xpu README "MoE (routed experts)": computed in fp32 with the routing
 * weight applied to the down-projection output, never to its input; one
 * launch per projection with routing kept on device; MoE post section 2:
 * SiLU between the two launches, device-side token binning, fp32 gather.)
 *   gate_up  arena with slots == 2 (slot 0 = gate, slot 1 = up), k = hidden,
 *            n = intermediate
 *   down     arena with slots == 1, k = intermediate, n = hidden, same
 *            number of experts
 *   x             fp16 [t][hidden] device pointer (row stride = hidden)
 *   topk_ids      int32 [t][topk] device pointer, each in [0, experts)
 *   topk_weights  fp32 [t][topk] device pointer
 *   y             fp32 [t][hidden] device pointer, overwritten with
 *                 Y[i] = sum over s in slot order of w[i][s] * down_e(a),
 *                 a = silu(gate_e(x_i)) * up_e(x_i), e = topk_ids[i][s]
 *   ws            device workspace of at least the queried size, zero-filled
 *                 before its first use; calls leave its arrival counts at
 *                 zero, so it serves later calls without clearing
 * 1 <= topk <= EXL3_MAX_TOPK.  t == 0 returns EXL3_OK without work.
 * Out-of-range ids are a contract violation and are not checked by default.
 * With the environment variable EXL3_CHECK_IDS set (not "0"; read at every
 * call), the call first counts the ids outside [0, experts) on the device,
 * waits for that count on the host (so such calls block and cannot be
 * graph-captured), and returns EXL3_E_INVALID, with nothing else enqueued,
 * if there is any.  With EXL3_CHECK_IDS set, a call on a stream that is
 * being captured returns EXL3_E_INVALID without enqueueing anything (the
 * capture stays valid).  The same holds for exl3_grouped_experts_mixed.
 * Small calls (t * topk <= 224) hand partial sums between workgroups planned
 * on one XCD (the XCD each group was finished on in the previous call, kept
 * in the workspace's counters); a workgroup that finds itself on another XCD
 * takes a device-scope release/acquire hand-off instead, so results never
 * depend on the dispatch order.  The environment variable
 * EXL3_FORCE_DEVICE_SCOPE (not "0"; read at every call) makes every
 * workgroup take that hand-off: the results are the same bits, only slower
 * (a debug check of the guard).                                            */
exl3_status exl3_grouped_experts(const exl3_expert_weights* gate_up,
                                 const exl3_expert_weights* down, const void* x,
                                 const int32_t* topk_ids, const float* topk_weights, int64_t t,
                                 int32_t topk, float* y, void* ws, size_t ws_bytes,
                                 exl3_stream_t stream);

/* The widths of an arena whose experts each have their own width
 * (TensorFold issue #832, "Activity": the consolidated module keeps a width
 * per expert in the representation).  The arena record then has bits == 0,
 * and expert e's tensors are bits_host[e] bits wide:
 *   bits_host  int32 [experts] host pointer, each in 1..8; checked on the
 *              host during the call (nothing is enqueued if one is not)
 *   bits       int32 [experts] device pointer, 4-byte aligned, the same
 *              values (read by the kernels)
 *   offsets    int64 [experts] device pointer, 8-byte aligned: the word
 *              index in the arena's trellis where expert e's slot 0 starts,
 *              a multiple of 8; slot s follows at
 *              offsets[e] + s * (k/16) * (n/16) * 16 * bits[e].
 *              Experts may be packed in any order.
 * suh and svh keep the uniform layout [experts][slots][k or n].  Device
 * values that differ from bits_host, or offsets past the trellis allocation,
 * are a contract violation and are not checked on device (a device width
 * outside 1..8 leaves that expert's pairs uncomputed, the output undefined
 * and the workspace to be zero-filled again before its next use).        */
typedef struct exl3_expert_widths {
    const int32_t* bits_host;
    const int32_t* bits;
    const int64_t* offsets;
} exl3_expert_widths;

/* Bytes of device workspace exl3_grouped_experts_mixed needs (0 if
 * invalid); the same figure as for uniform arenas of the same shapes.     */
size_t exl3_grouped_experts_mixed_workspace_size(const exl3_expert_weights* gate_up,
                                                 const exl3_expert_widths* gate_up_widths,
                                                 const exl3_expert_weights* down,
                                                 const exl3_expert_widths* down_widths,
                                                 int64_t t, int32_t topk);

/* exl3_grouped_experts_mixed - exl3_grouped_experts over arenas with a width
 * per expert (gate_up_widths for the gate/up arena, down_widths for the down
 * arena; an expert's gate and up share its width).  Arguments, workspace
 * rules, errors and the result are those of exl3_grouped_experts; each
 * (token, slot) pair is computed by the same kernels and in the same order
 * as a uniform arena of its expert's width would compute it, so when every
 * expert has one width the result is bit-identical to exl3_grouped_experts.
 * Each projection is still one launch: every workgroup reads its expert's
 * width and runs the decode of that width.                                 */
exl3_status exl3_grouped_experts_mixed(const exl3_expert_weights* gate_up,
                                       const exl3_expert_widths* gate_up_widths,
                                       const exl3_expert_weights* down,
                                       const exl3_expert_widths* down_widths, const void* x,
                                       const int32_t* topk_ids, const float* topk_weights,
                                       int64_t t, int32_t topk, float* y, void* ws,
                                       size_t ws_bytes, exl3_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* EXL3_H */
