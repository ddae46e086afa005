/*
 * vla.h - C ABI of the MI355X (gfx950) FP8/BF16-weight GEMM library for
 * small-batch vision-language-action inference.
 *
 * Conventions (all entry points):
 *  - Arguments come in the order device pointers, sizes, scalars, stream,
 *    the order of the kernel calls shown on "FlashRT: an inference engine for
 *    real-time robot control" (itsolotime.com), section 3.3 (pipeline table:
 *    pointers, then dims, then eps, then stream).
 *  - Every pointer named "device" is device memory owned by the caller; the
 *    library never allocates, frees or retains device memory, except that a
 *    chain handle records the pointers it was created with.
 *  - bf16 tensors are passed as uint16_t bit patterns.  FP8 tensors are
 *    uint8_t E4M3 codes.  Matrices are row-major unless a layout says
 *    otherwise.  Weights are N x K: one row per output channel.
 *  - `stream` is a hipStream_t (NULL = the null stream).  Calls enqueue work
 *    on it and return without synchronising; they are safe to record under
 *    stream capture (no allocation, no host reads of device values, no
 *    memset nodes) - the property the page "Deploying DeepSeek-V4-Flash on
 *    AMD MI300X" (lehuy.net), section "HIP Graphs", requires of captured
 *    launches.
 *  - Return value: VLA_OK (0) or a positive VLA_E* code; nothing is thrown.
 *    vla_status_string() names a code and vla_last_error() gives a message
 *    for the calling thread's last failure.  Launch failures are read with
 *    hipGetLastError right after the launch and reported as VLA_EHIP.
 *  - Alignment: every device pointer must be 16-byte aligned (VLA_EALIGN).
 *
 * Shapes: N must be a multiple of 16 and K a multiple of 32 (one 16x16x32
 * MFMA tile); M >= 1 is free (ragged rows are masked).
 */
#ifndef VLA_H
#define VLA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---------------------------------------------------------------- status */
#define VLA_OK 0
#define VLA_EINVAL 1      /* NULL pointer, non-positive size, unknown enum */
#define VLA_ESHAPE 2      /* N % 16, K % 32, or mismatched shapes */
#define VLA_EALIGN 3      /* a device pointer is not 16-byte aligned */
#define VLA_EWORKSPACE 4  /* workspace or scratch smaller than required */
#define VLA_EHIP 5        /* a HIP runtime call or kernel launch failed */
#define VLA_ESTATE 6      /* chain handle not created, or already destroyed */

/* Weight formats. */
#define VLA_WFMT_BF16 0
#define VLA_WFMT_E4M3_OCP 1   /* OCP E4M3: bias 7, max 448, NaN S.1111.111, no inf */
#define VLA_WFMT_E4M3_FNUZ 2  /* E4M3 FNUZ: bias 8, max 240, NaN 0x80 only, no -0, no inf */
#define VLA_WFMT_MXFP4 3      /* OCP MX FP4: E2M1 codes + one E8M0 scale per 32 values of K */

/* Weight layouts. */
#define VLA_LAYOUT_ROWMAJOR 0
/* MFMA lane layout for gfx950's 16x16x32 BF16/FP8 MFMA (8 values per lane;
 * "Real-time VLA inference on AMD hardware" (cyberneticphysics.com),
 * introduction and section "Packing around the instruction", which gives
 * the 4-values-per-lane CDNA3 form).  Element (n, k), n = 16 n0 + n1,
 * k = 32 k0 + 8 k1 + k2, sits at element offset
 *     ((n0 * (K / 32) + k0) * 64 + 16 k1 + n1) * 8 + k2,
 * so each lane's 8 values (8 bytes FP8, 16 bytes BF16) are contiguous and a
 * wavefront's 64 slices of one 16x32 fragment form one contiguous block. */
#define VLA_LAYOUT_MFMA 1

const char *vla_status_string(int status);
/* Message of the calling thread's last failed call ("" if none). */
const char *vla_last_error(void);

/* Bounded in-kernel waits.  Kernels that wait for other workgroups (the wide
 * GEMM's split-K hand-over, the fused chain's phase barriers) poll at most
 * `polls` times (about 0.5 us per poll), then give up, write NaN over the
 * output they were waiting to produce, record the cause in the workspace's
 * status word and exit normally, so no wait can hang the device.  0 restores
 * the default (2^22 polls, never reached by a grid that is resident).  The
 * bound is read when a call is enqueued (or captured).  Process-wide. */
void vla_set_wait_limit(uint32_t polls);

/* Read and clear the status word of a GEMM workspace or chain scratch
 * buffer (byte 61440 of it): VLA_OK when no in-kernel wait of a call that
 * used `ws` has given up since the last query, else VLA_EHIP naming the
 * cause (its output is incomplete).  Copies 4 bytes to the host and
 * synchronises `stream` (which must have run those calls): not for use under
 * stream capture.  Errors: EINVAL/EALIGN for ws, EHIP if a copy fails. */
int vla_workspace_status(void *ws, void *stream);

/* --------------------------------------------------------- weight codecs */

/* Bytes of an N x K weight in format `wfmt` (either layout; MXFP4: codes
 * and block scales, N*K/2 + N*P with P = K/32 rounded up to 8). */
size_t vla_packed_bytes(int64_t N, int64_t K, int wfmt);

/* Quantize (FP8) or round (BF16) an fp32 weight and lay it out.
 * "Real-time VLA inference on AMD hardware", section "Packing around the
 * instruction": weights are quantized and packed once at load time and stay
 * at fixed addresses.
 *   W      device fp32, N x K row-major (one row per output channel).
 *   Wq     device output, vla_packed_bytes(N, K, wfmt) bytes, in `layout`.
 *   scales device fp32[N] output for FP8 formats, must be NULL for BF16.
 * FP8: scales[n] = fp32(max_k |W[n,k]| / 448) (OCP) or / 240 (FNUZ), 1 for an
 * all-zero row; code = encode(fp32(W[n,k] / scales[n])), IEEE division,
 * round to nearest even, saturating at +-max.  BF16: round to nearest even.
 * MXFP4 (OCP Microscaling Formats v1.0; 4-bit weights as in "FlashRT: an
 * inference engine for real-time robot control", section 7.2, here in the
 * MX form gfx950 converts in hardware): per block of 32 values of K in one
 * row, shared exponent e = floor(log2 max|w|) - 2 clamped to [-127, 127]
 * (0 for an all-zero block), code = nearest E2M1 of w * 2^-e (ties to the
 * even code, saturating at +-6); only VLA_LAYOUT_MFMA, scales must be NULL:
 * Wq holds the codes in the FP8 fragment order, two per byte (even position
 * in the low nibble), N*K/2 bytes, then the E8M0 bytes (127 + e) row-major,
 * each row padded to P = K/32 rounded up to 8 bytes (pad bytes 127): byte
 * N*K/2 + n * P + k/32.
 * W must be finite.  Errors: EINVAL, ESHAPE, EALIGN, EHIP. */
int vla_quantize_pack(const float *W, void *Wq, float *scales, int64_t N, int64_t K, int wfmt,
                      int layout, void *stream);

/* Reorder an N x K row-major FP8 code matrix into VLA_LAYOUT_MFMA (a pure
 * byte permutation).  q_rowmajor and q_packed must not overlap. */
int vla_pack_fp8(const uint8_t *q_rowmajor, uint8_t *q_packed, int64_t N, int64_t K,
                 void *stream);

/* Re-encode E4M3 FNUZ codes + per-row scales to OCP E4M3 codes + scales so
 * that every value dec(q) * s is preserved.  The pages ("Real-time VLA
 * inference on AMD hardware", introduction and "Different FP8
 * representation"; "Deploying DeepSeek-V4-Flash on AMD MI300X", FP8 dialect
 * section) state that a byte reads as half the value under FNUZ.  Per row n:
 * j = 1 when the row holds no +-240 code (0x7F / 0xFF): every byte is kept
 * and s' = s / 2 (value-exact); otherwise j = 0: q' = encode_ocp(dec_fnuz(q))
 * (exact except the 16 odd-mantissa codes below 2^-6, which are ties and go
 * to the even code, error <= 2^-10 * s) and s' = s.  FNUZ NaN (0x80) -> 0x7F.
 *   q_fnuz, s_fnuz  device inputs, N x K codes in `layout`, fp32[N].
 *   q_ocp,  s_ocp   device outputs, same shapes; may alias the inputs
 *                   exactly (in-place) but not partially. */
int vla_reencode_fnuz_to_ocp(const uint8_t *q_fnuz, const float *s_fnuz, uint8_t *q_ocp,
                             float *s_ocp, int64_t N, int64_t K, int layout, void *stream);

/* Per-tensor OCP quantization of bf16 activations for the FP8 x FP8 GEMM:
 * s_a = fp32(max |A| / 448) (1 if A is all zero), qa = encode_ocp(fp32(A / s_a)).
 *   A   device bf16 M x K;  qa device uint8 M x K;  s_a device float[1].
 *   ws  device workspace of vla_quantize_act_workspace_bytes(M, K) bytes
 *       (no initial contents required).
 * s_a stays on the device (no host read), so the call can be captured. */
size_t vla_quantize_act_workspace_bytes(int64_t M, int64_t K);
int vla_quantize_act(const uint16_t *A, uint8_t *qa, float *s_a, void *ws, size_t ws_bytes,
                     int64_t M, int64_t K, void *stream);

/* The same encoding under a calibrated, frozen scale: qa = encode_ocp(fp32(A / s_a))
 * with s_a given ("FlashRT: an inference engine for real-time robot control",
 * section 3.2: the first real input sets the FP8 activation scales; section
 * 7.1: the calibrated scales are captured into the graph).  One pass, no
 * absmax, no workspace; vla_quantize_act's s_a output is one way to calibrate.
 *   A   device bf16 M x K;  s_a device float[1], read by the kernel (any fp32
 *       value: values of |A / s_a| >= 448 saturate to +-448, NaN gives 0x7F
 *       or 0xFF, exactly as the encoder rules state);  qa device uint8 M x K.
 * Shape rules as vla_quantize_act (K a multiple of 32); pointers 16-byte
 * aligned, else VLA_EALIGN. */
int vla_quantize_act_static(const uint16_t *A, const float *s_a, uint8_t *qa, int64_t M, int64_t K,
                            void *stream);

/* ------------------------------------------------------- decoder boundary */

/* Fused decoder boundary ("Real-time VLA inference on AMD hardware",
 * section "Fusing the BF16 decoder boundary"): the gated residual update
 * followed by the adaptive RMS norm of its result, per row m and channel d:
 *   residual_out = bf16(residual + out * gate)              (one rounding)
 *   normalized   = bf16(r / sqrt(mean_d(r^2) + eps) * (1 + scale) + shift)
 *   next_gate    = the style row's gate block (a copy)
 * with r = residual_out and style rows holding three consecutive D-wide bf16
 * blocks [scale | shift | next gate].  The page names the operation and its
 * two steps; the modulation reading (scale, shift, gate per channel, no
 * separate norm weight) is this library's.  residual_out is the correctly
 * rounded sum bit for bit; normalized is computed in fp64 and rounded once.
 *   residual, out, gate   device bf16 M x D (row-major);
 *   style                 device bf16, M x 3D when style_per_row != 0, else
 *                         one 3D row shared by every row;
 *   eps                   finite, >= 0 (else VLA_EINVAL);
 *   residual_out          device bf16 M x D; may be `residual` itself;
 *   normalized            device bf16 M x D;
 *   next_gate             device bf16 M x D, or NULL to skip the copy.
 * No output may overlap an input or another output (residual_out ==
 * residual excepted): VLA_EINVAL.  D a multiple of 4, at most 8192
 * (VLA_ESHAPE); M in 1 .. 2^24; pointers 16-byte aligned (VLA_EALIGN). */
int vla_gate_residual_ada_norm(const uint16_t *residual, const uint16_t *out, const uint16_t *gate,
                               const uint16_t *style, int style_per_row, float eps, uint16_t *residual_out,
                               uint16_t *normalized, uint16_t *next_gate, int64_t M, int64_t D, void *stream);

/* ----------------------------------------------------------- measurement */

/* Streaming-read probe: one launch of `blocks` workgroups of 256 threads
 * reads `bytes` from src (16-byte loads, four in flight per thread) and
 * keeps nothing.  It is the floor under a weight-streaming GEMM call that
 * reads the same bytes ("Real-time VLA inference on AMD hardware", section
 * "FP8 helps the encoder and hurts the decoder": the decoder GEMMs are bound
 * by streaming their weights).
 *   src   device, 16-byte aligned, `bytes` readable (a positive multiple of 16,
 *         else VLA_ESHAPE);
 *   sink  device uint32[1], 16-byte aligned; written only in the rare case
 *         that the XOR of a thread's data equals a fixed constant;
 *   blocks 1..65536, else VLA_EINVAL. */
int vla_probe_stream_read(const void *src, size_t bytes, uint32_t *sink, int blocks, void *stream);

/* Matrix-core rate probe: one launch of `blocks` workgroups of 256 threads;
 * every wave runs `iters` rounds of four independent MFMA chains of the
 * given form on operands it holds in registers, so the launch measures the
 * issue rate of that instruction on that data.  The skinny and wide GEMMs
 * are built on these instructions ("Real-time VLA inference on AMD
 * hardware", section "How FlashRT works": the GEMMs are shaped around the
 * matrix instruction), and the rate they can reach depends on the operand
 * values, so a GEMM's roofline fraction is read against this rate on
 * operands like its own as well as against the published peak.
 *   form      VLA_MFMA_* below, else VLA_EINVAL;
 *   operands  device uint32[256 * 64], 16-byte aligned: lane t of every
 *             workgroup takes words 64t .. 64t+63 as four operand sets
 *             (A in words 16j .. 16j+7, B in 16j+8 .. 16j+15 of set j; the
 *             bf16 forms use the first four words of each: 8 bf16 values;
 *             the FP8 forms all eight: 32 OCP E4M3 codes);
 *   iters     1 .. 2^24 (VLA_EINVAL otherwise);
 *   out       device float[blocks * 256], 16-byte aligned: lane t of
 *             workgroup b writes the sum of its four accumulators at
 *             b*256 + t (accumulators start at zero);
 *   clocks    NULL, or device uint64[2 * blocks], 8-byte aligned
 *             (VLA_EALIGN): workgroup b's first wave writes the shader-clock
 *             cycles (s_memtime) and the 100 MHz real-time ticks
 *             (s_memrealtime) its instruction loop took at 2b and 2b + 1;
 *             cycles / (ticks * 10 ns) is the clock the loop ran at, which
 *             falls under the chip's power limit on busy, non-zero operands;
 *   blocks    1 .. 65536, else VLA_EINVAL.
 * One launch does blocks * 4 * iters * 4 instructions, each of
 * 2*m*n*k floating-point operations for its m x n x k form. */
#define VLA_MFMA_BF16_32X32X16 0  /* v_mfma_f32_32x32x16_bf16 (wide GEMM, bf16 activations) */
#define VLA_MFMA_BF16_16X16X32 1  /* v_mfma_f32_16x16x32_bf16 (skinny GEMM, gated-MLP chain) */
#define VLA_MFMA_FP8_32X32X64 2   /* v_mfma_scale_f32_32x32x64_f8f6f4, E4M3 x E4M3 (wide GEMM, FP8 x FP8) */
#define VLA_MFMA_FP8_16X16X128 3  /* v_mfma_scale_f32_16x16x128_f8f6f4, E4M3 x E4M3 */
int vla_probe_mfma_rate(int form, const uint32_t *operands, int iters, float *out, uint64_t *clocks, int blocks,
                        void *stream);

/* ------------------------------------------------------------------ GEMM */

/* Workspace for vla_gemm_fp8w / vla_gemm_bf16 / vla_gemm_fp8w_gelu_mul at
 * this shape (N = weight rows; for gelu_mul N = 2 I).  Its first 60 KiB
 * hold the split-K arrival counters (the same place for every shape), the
 * next 4 KiB the status word (vla_workspace_status) and unused bytes; the
 * rest holds split-K partial sums.  The workspace must be
 * ZERO-FILLED before its first use; every completed call leaves the
 * counters at zero again, so one zeroed buffer (sized for the largest
 * shape) serves any number of later calls and graph replays, of any
 * shapes, that run one after another.  Calls that run concurrently must
 * not share a workspace. */
size_t vla_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K, int wfmt);

/* Host-only query, no device work: VLA_OK when a GEMM of this shape has a
 * compiled kernel configuration (wfmt VLA_WFMT_BF16 or VLA_WFMT_E4M3_OCP;
 * fp8_act: FP8 x FP8 with OCP activations; gelu_mul: the merged gate/up
 * GEMM with N = 2I), else the status the GEMM call itself would return
 * (EINVAL, ESHAPE). */
int vla_gemm_supported(int64_t M, int64_t N, int64_t K, int wfmt, int fp8_act, int gelu_mul);

/* Host-only query, no device work: the launch plan a GEMM of this shape
 * takes (arguments as vla_gemm_supported).  Writes min(n_info, 10) values:
 *   [0] kernel (0 = skinny, M <= 64; 1 = wide)
 *   [1] skinny: 16-column weight tiles per workgroup; wide: tile width
 *   [2] [3] [4] grid x, y, z (skinny: column groups, K splits, row blocks;
 *               wide: column groups, 192-row blocks, K splits)
 *   [5] K splits across workgroups
 *   [6] workspace bytes (vla_gemm_workspace_bytes for this operand class)
 *   [7] split-K partial bytes (addressed with 32-bit offsets: < 2^32)
 *   [8] threads per workgroup
 *   [9] split-K counters used (at most 15360)
 * Returns what vla_gemm_supported returns; the values are written in
 * either case when the shape passes the argument checks. */
int vla_gemm_plan(int64_t M, int64_t N, int64_t K, int wfmt, int fp8_act, int gelu_mul, int64_t *info,
                  int n_info);

/* Y = bf16( s[n] * sum_k A[m,k] * dec(Wq[n,k]) + bias[n] ), optionally
 * followed by Y = bf16(residual + Y).
 * "Real-time VLA inference on AMD hardware", sections "FP8 helps the encoder
 * and hurts the decoder" and "Merging gate and up" (bias in the epilogue).
 *   A        device: bf16 M x K when s_a == NULL (BF16 x FP8 weights);
 *            OCP E4M3 codes M x K when s_a != NULL (FP8 x FP8, the value of
 *            A is dec(A) * s_a[0]; s_a is a device float[1]).
 *   Wq, s_w  OCP E4M3 weight in VLA_LAYOUT_MFMA and its fp32[N] scales.
 *   bias     device bf16[N] or NULL.
 *   residual device bf16 M x N or NULL; may alias Y exactly (in-place add).
 *   Y        device bf16 M x N output.
 * Arithmetic: fp32 accumulation of exact bf16 (or fp8) products; epilogue
 * y = acc * s_w[n] (FP8 x FP8: acc * (s_a * s_w[n])) + bias, rounded to
 * bf16 nearest-even; residual added in fp32 and rounded again.  The
 * summation order is fixed per shape, so repeated calls are bitwise equal.
 * Errors: EINVAL, ESHAPE (also when M > 64 and A or Wq reaches 2 GiB: the
 * wide kernel addresses them with 32-bit offsets), EALIGN, EWORKSPACE, EHIP. */
int vla_gemm_fp8w(const void *A, const float *s_a, const uint8_t *Wq, const float *s_w,
                  const uint16_t *bias, const uint16_t *residual, uint16_t *Y, void *ws,
                  size_t ws_bytes, int64_t M, int64_t N, int64_t K, void *stream);

/* vla_gemm_fp8w without a workspace argument, for callers that cannot
 * allocate device memory (code recorded under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc).  Same arguments,
 * arithmetic, kernels and results as vla_gemm_fp8w.  The split-K counters
 * and partials live in an array the library holds in each GPU's memory
 * (65536 + 32 MiB bytes per GPU, until the process ends), set up on the
 * first call on a device (its counters cleared by a kernel on `stream`);
 * nothing is allocated and no hipMalloc, hipFree or allocating library call
 * is made.  Shapes whose workspace (vla_gemm_workspace_bytes) exceeds that
 * array fail with VLA_EWORKSPACE before any device work; every shape at or
 * below 768 rows of the encoder sizes fits.  All calls on one GPU share the
 * array: calls that overlap in time on one GPU (concurrent streams, or
 * graphs replayed concurrently) race and give wrong results; calls that run
 * one after another are safe.  A bounded split-K wait that gives up writes
 * NaN over the output it could not finish (the status word is not
 * reported for this variant). */
int vla_gemm_fp8w_noalloc(const void *A, const float *s_a, const uint8_t *Wq, const float *s_w,
                          const uint16_t *bias, const uint16_t *residual, uint16_t *Y, int64_t M,
                          int64_t N, int64_t K, void *stream);

/* As vla_gemm_fp8w with BF16 weights (VLA_LAYOUT_MFMA) and no weight scale:
 * Y = bf16( sum_k A[m,k] * Wq[n,k] + bias[n] ) (+ residual). */
int vla_gemm_bf16(const uint16_t *A, const uint16_t *Wq, const uint16_t *bias,
                  const uint16_t *residual, uint16_t *Y, void *ws, size_t ws_bytes, int64_t M,
                  int64_t N, int64_t K, void *stream);

/* Merged gate/up GEMM with the GELU-tanh * up epilogue of a gated MLP.
 * "Real-time VLA inference on AMD hardware", section "Merging gate and up":
 * the gate and up weights are concatenated, W = [W_gate; W_up] (2I x K,
 * rows 0..I-1 gate, I..2I-1 up), and one GEMM computes both.
 *   g = bf16(s[n] * A @ W_gate^T + b[n]), u = bf16(s[I+n] * A @ W_up^T + b[I+n]),
 *   act = bf16( 0.5 g (1 + tanh(sqrt(2/pi) (g + 0.044715 g^3))) * u ).
 * The bias is added in the same epilogue, as that section describes.
 *   A     device bf16 M x K.
 *   Wgu   OCP E4M3 2I x K in VLA_LAYOUT_MFMA, s_gu its fp32[2I] scales.
 *   bias  device bf16[2I] = [b_gate, b_up], or NULL for none.
 *   act   device bf16 M x I output.
 *   gu    device bf16 M x 2I output of [g, u], or NULL.
 * I must be a multiple of 16.  Workspace: vla_gemm_workspace_bytes(M, 2I, K, OCP). */
int vla_gemm_fp8w_gelu_mul(const uint16_t *A, const uint8_t *Wgu, const float *s_gu, const uint16_t *bias,
                           uint16_t *act, uint16_t *gu, void *ws, size_t ws_bytes, int64_t M,
                           int64_t I, int64_t K, void *stream);

/* As vla_gemm_fp8w with MXFP4 weights (bf16 activations, no per-channel
 * scale: each 32-value block of a weight row carries its E8M0 scale):
 *   Y = bf16(A @ (dec(q) * 2^(e - 127))^T + bias) (+ residual, as above)
 * 4-bit weights ("FlashRT: an inference engine for real-time robot
 * control", section 7.2) in the OCP MX form; the kernel converts each code
 * to bf16 with its block scale in one gfx950 instruction per pair, exactly,
 * and streams half the bytes of FP8.  Any M: M <= 64 runs the skinny kernel,
 * larger M the wide one (the section's 4-bit encoder FFN shapes), which
 * stages each K tile's E8M0 bytes beside its codes.  Wq from
 * vla_quantize_pack(..., VLA_WFMT_MXFP4, VLA_LAYOUT_MFMA); workspace
 * vla_gemm_workspace_bytes(M, N, K, VLA_WFMT_MXFP4). */
int vla_gemm_mxfp4w(const uint16_t *A, const uint8_t *Wq, const uint16_t *bias, const uint16_t *residual,
                    uint16_t *Y, void *ws, size_t ws_bytes, int64_t M, int64_t N, int64_t K, void *stream);

/* ------------------------------------------------------- gated-MLP chain */

/* L gated-MLP layers applied to x (M x H bf16):
 *   act = gelu_mul(x @ [Wgate_l; Wup_l]^T)        (vla_gemm_fp8w_gelu_mul)
 *   x   = bf16(x + bf16(act @ Wdown_l^T))         (vla_gemm_fp8w, residual)
 * "Real-time VLA inference on AMD hardware", section "How FlashRT works":
 * the whole sequence is recorded once as a HIP graph and replayed, with
 * weights at fixed addresses.
 *   wgu, sgu  host arrays of L device pointers: OCP 2I x H weights
 *             (VLA_LAYOUT_MFMA) and fp32[2I] scales.
 *   wd, sd    host arrays of L device pointers: OCP H x I weights and
 *             fp32[H] scales.
 *   x_in      device bf16 M x H input (read only).
 *   x_out     device bf16 M x H output (must not overlap x_in or scratch).
 *   scratch   device, vla_mlp_chain_scratch_bytes(M, H, I) bytes,
 *             ZERO-FILLED before first use (it embeds a GEMM workspace; its
 *             per-layer buffers cover up to 32 layers).
 * Every device pointer must stay valid, at the same address, for the life
 * of a handle. */
size_t vla_mlp_chain_scratch_bytes(int64_t M, int64_t H, int64_t I);

/* 1 when the chain of this shape runs as one persistent launch on the
 * current device, else 0 (then each layer runs as two GEMM launches).  The
 * single launch covers M <= 64 rows with (H, I) = (1024, 4096) or
 * (256, 512) and L <= 32, on a device whose 256 compute units can each hold
 * one of its workgroups; the enqueue/create calls also need the scratch
 * buffer (and any stage outputs) 256-byte aligned to take it.  It meets at a
 * grid barrier between the gate/up and the down phase of each layer (every
 * wait bounded, see vla_set_wait_limit; a give-up leaves NaN in x_out and
 * sets the scratch buffer's status word) and streams each phase's weights
 * while the previous phase finishes.  Both forms compute the same stages;
 * their fp32 summation orders differ, so results may differ in the last
 * bit.  Host query: reads device attributes, enqueues nothing. */
int vla_mlp_chain_fused_supported(int64_t M, int64_t H, int64_t I, int L);

/* Enqueue the chain's 2L kernels directly (no graph). */
int vla_mlp_chain_enqueue(const uint8_t *const *wgu, const float *const *sgu,
                          const uint8_t *const *wd, const float *const *sd,
                          const uint16_t *x_in, uint16_t *x_out, void *scratch,
                          size_t scratch_bytes, int L, int64_t M, int64_t H, int64_t I,
                          void *stream);

/* vla_mlp_chain_enqueue that also writes every layer's intermediate
 * results, so each rounding point of the chain ("Real-time VLA inference
 * on AMD hardware", "Merging gate and up" and "Fusing the BF16 decoder
 * boundary") can be checked on its own inputs.  Each output is nullable:
 *   gu_out    device bf16 L x M x 2I: [g | u] of layer l (before GELU * mul)
 *   act_out   device bf16 L x M x I:  act of layer l
 *   down_out  device bf16 L x M x H:  bf16(act @ Wdown_l^T), before the
 *             residual add (x_l+1 = bf16(x_l + down_l))
 *   x_layers  device bf16 L x M x H:  x after layer l (x_layers[L-1] equals
 *             x_out)
 * Outputs must not overlap each other, x_in, x_out or scratch (EINVAL).
 * x_out equals vla_mlp_chain_enqueue's result bit for bit. */
int vla_mlp_chain_enqueue_staged(const uint8_t *const *wgu, const float *const *sgu,
                                 const uint8_t *const *wd, const float *const *sd,
                                 const uint16_t *x_in, uint16_t *x_out, uint16_t *gu_out,
                                 uint16_t *act_out, uint16_t *down_out, uint16_t *x_layers,
                                 void *scratch, size_t scratch_bytes, int L, int64_t M, int64_t H,
                                 int64_t I, void *stream);

typedef struct vla_mlp_chain vla_mlp_chain;

/* Record the chain once on `capture_stream` (relaxed capture mode, which
 * records only that stream's work; it must not be the null stream) and
 * instantiate it.  *out receives a host handle owned by the caller. */
int vla_mlp_chain_create(const uint8_t *const *wgu, const float *const *sgu,
                         const uint8_t *const *wd, const float *const *sd,
                         const uint16_t *x_in, uint16_t *x_out, void *scratch,
                         size_t scratch_bytes, int L, int64_t M, int64_t H, int64_t I,
                         void *capture_stream, vla_mlp_chain **out);

/* Launch the recorded graph on `stream`.  ESTATE for a NULL or destroyed
 * handle (the page "FlashRT: an inference engine for real-time robot
 * control", section 4.1, raises "No graph captured" on replay before
 * capture). */
int vla_mlp_chain_replay(vla_mlp_chain *chain, void *stream);

/* Free the graph and the handle.  The handle must not be used afterwards;
 * destroying NULL is a no-op returning VLA_OK. */
int vla_mlp_chain_destroy(vla_mlp_chain *chain);

/* ---------------------------------------------------- decoder-block chain */

/* L action-decoder MLP blocks closed by the fused decoder boundary
 * ("Real-time VLA inference on AMD hardware", sections "Merging gate and
 * up" and "Fusing the BF16 decoder boundary"): per layer l, from the
 * residual x, the normalized input h and the gate g (each M x H bf16),
 *   act       = gelu_mul(h @ [Wgate_l; Wup_l]^T)    (vla_gemm_fp8w_gelu_mul)
 *   d         = bf16(act @ Wdown_l^T)               (vla_gemm_fp8w)
 *   (x, h, g) = vla_gate_residual_ada_norm(x, d, g, style_l, eps)
 * The final x, h and g are the outputs.  Where
 * vla_decoder_chain_fused_supported says so and the scratch and stage
 * buffers are 256-byte aligned, the chain is one persistent launch: the gated
 * residual is formed in the down-projection's epilogue together with each
 * 16-column tile's partial sum of squares of the new residual, and the next
 * layer normalizes its staged input rows from those partials (fp32 after the
 * fp64 sum; 1/rms in fp64), so the layers meet only at the chain's own
 * phase barriers (bounded waits: a give-up leaves NaN in x_out, h_out and
 * gate_out and sets the scratch buffer's status word).  Otherwise three kernels per layer are recorded once as a
 * HIP graph like the gated-MLP chain's.  The residual is bit-exact on both
 * paths; h agrees with the fp64 boundary within one bf16 ulp.
 *   wgu, sgu, wd, sd  as for the gated-MLP chain.
 *   style        host array of L device pointers: bf16 (style_per_row ? M : 1)
 *                x 3H, [scale | shift | next gate] (see the boundary).
 *   eps          finite, >= 0.
 *   x_in, h_in, gate_in     device bf16 M x H inputs (read only).
 *   x_out, h_out, gate_out  device bf16 M x H outputs; none may overlap
 *                another output, an input, a style array or scratch.
 *   scratch      device, vla_decoder_chain_scratch_bytes(M, H, I) bytes,
 *                ZERO-FILLED before first use (it embeds a GEMM workspace);
 *                the inputs must not overlap it.
 * H and I multiples of 32, H at most 8192.  The handle from
 * vla_decoder_chain_create is replayed and destroyed with
 * vla_mlp_chain_replay / vla_mlp_chain_destroy. */
size_t vla_decoder_chain_scratch_bytes(int64_t M, int64_t H, int64_t I);

/* 1 if the decoder-block chain of this shape runs as one persistent launch
 * on the current device (given 256-byte aligned scratch and stage
 * buffers), 0 if it takes the graph of launches: the gated-MLP chain's
 * conditions (vla_mlp_chain_fused_supported), H <= 1024, and with a style
 * row per activation row (style_per_row != 0) M <= 16, beyond which the
 * graph of launches measured faster.  Never fails. */
int vla_decoder_chain_fused_supported(int64_t M, int64_t H, int64_t I, int L, int style_per_row);

int vla_decoder_chain_enqueue(const uint8_t *const *wgu, const float *const *sgu,
                              const uint8_t *const *wd, const float *const *sd,
                              const uint16_t *const *style, int style_per_row, float eps,
                              const uint16_t *x_in, const uint16_t *h_in, const uint16_t *gate_in,
                              uint16_t *x_out, uint16_t *h_out, uint16_t *gate_out, void *scratch,
                              size_t scratch_bytes, int L, int64_t M, int64_t H, int64_t I, void *stream);

/* vla_decoder_chain_enqueue, keeping every stage of every layer (for parity
 * checks): each of these may be NULL; non-NULL ones are device bf16, 16-byte
 * aligned, and must not overlap each other, an input, an output, a style
 * array or the scratch (VLA_EINVAL):
 *   gu_out    L x M x 2I  [g | u] of the merged gate/up GEMM, layer after layer;
 *   act_out   L x M x I   GELU(g) * u;
 *   down_out  L x M x H   the down-projection d (before the boundary);
 *   x_layers  L x M x H   the residual x after each layer;
 *   h_layers  L x M x H   the normalized h after each layer.
 * x_out, h_out and gate_out are written as by vla_decoder_chain_enqueue. */
int vla_decoder_chain_enqueue_staged(const uint8_t *const *wgu, const float *const *sgu,
                                     const uint8_t *const *wd, const float *const *sd,
                                     const uint16_t *const *style, int style_per_row, float eps,
                                     const uint16_t *x_in, const uint16_t *h_in, const uint16_t *gate_in,
                                     uint16_t *x_out, uint16_t *h_out, uint16_t *gate_out, uint16_t *gu_out,
                                     uint16_t *act_out, uint16_t *down_out, uint16_t *x_layers, uint16_t *h_layers,
                                     void *scratch, size_t scratch_bytes, int L, int64_t M, int64_t H, int64_t I,
                                     void *stream);

int vla_decoder_chain_create(const uint8_t *const *wgu, const float *const *sgu,
                             const uint8_t *const *wd, const float *const *sd,
                             const uint16_t *const *style, int style_per_row, float eps,
                             const uint16_t *x_in, const uint16_t *h_in, const uint16_t *gate_in,
                             uint16_t *x_out, uint16_t *h_out, uint16_t *gate_out, void *scratch,
                             size_t scratch_bytes, int L, int64_t M, int64_t H, int64_t I,
                             void *capture_stream, vla_mlp_chain **out);

#ifdef __cplusplus
}
#endif

#endif /* VLA_H */
