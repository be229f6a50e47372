/*
 * ocq.h -- C ABI of the quantized speculative-verify MLP block for AMD
 * MI355X (gfx950).
 *
 * What one call computes (the post "OCRia 推理栈：单卡 B200 提速近 10 倍"):
 *   x [M, hidden] bf16                            (M = requests x (1 + drafts),
 *                                                   section "Generate more tokens
 *                                                   per target pass")
 *   xq, sx = per-token E4M3 quantization of x     (sx = amax/448)
 *   G = (xq Wg^T) sx sw_g ;  U = (xq Wu^T) sx sw_u (weights FP8 or NVFP4, section
 *                                                   "Reducing the data moved:
 *                                                   workload-aware quantization")
 *   h = SiLU(G) * U, quantized per token to E4M3  (German page "Wie es
 *                                                   funktioniert": SiLU fused with
 *                                                   the quantization, kept in
 *                                                   registers)
 *   y = bf16( h Wd^T )                            (down projection in the
 *                                                   precision chosen for the
 *                                                   layer: FP8, BF16 or NVFP4)
 * Formats: E4M3 = OCP FP8 E4M3FN (max 448); E2M1 = OCP MX FP4; NVFP4 = E2M1
 * elements with one E4M3 scale per 16 inputs and one fp32 per-tensor scale.
 * Rounding: nearest, ties to even, saturating.  Scales: fl32(amax / 448) for
 * E4M3 rows, fl32(amax / 2688) per NVFP4 tensor, fl32(block amax / (6 S)) per
 * NVFP4 block before its own E4M3 rounding.  A zero row gets scale 0 and codes 0.
 *
 * Conventions for every entry point
 *   - Pointers named *_dev are device pointers (hipMalloc / torch CUDA
 *     tensors); *_host are host pointers.  The caller owns all memory and
 *     the stream; the library allocates nothing and frees nothing.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *   - A negative ocq_status is returned on failure, before anything is
 *     launched; ocq_last_error() then gives a message (thread-local, valid
 *     until the next call on the same thread).  Argument checks are
 *     synchronous; faults inside a kernel surface at the caller's next
 *     synchronization, as with any stream API.
 *   - Shapes: hidden and inter must be multiples of 128, 128 <= each <= 65536;
 *     1 <= M <= 8192.  Device pointers must be 16-byte aligned.
 */
#ifndef OCQ_H
#define OCQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  OCQ_OK = 0,
  OCQ_ERR_INVALID_ARG = -1,      /* null / misaligned pointer, bad M, bad enum   */
  OCQ_ERR_UNSUPPORTED = -2,      /* shape outside the supported set              */
  OCQ_ERR_DEVICE = -3,           /* HIP runtime error (no device, launch failure) */
  OCQ_ERR_BUFFER_TOO_SMALL = -4, /* packed blob or workspace smaller than needed  */
  OCQ_ERR_BAD_BLOB = -5          /* blob header does not match the call          */
} ocq_status;

typedef enum {
  OCQ_PREC_FP8 = 0,           /* gate/up FP8 E4M3, down FP8 E4M3                */
  OCQ_PREC_FP8_DOWN_BF16 = 1, /* gate/up FP8 E4M3, down BF16 (sensitive layer)  */
  OCQ_PREC_FP4 = 2            /* gate/up/down NVFP4                              */
} ocq_prec_mode;

/* Library version (major * 10000 + minor * 100 + patch). */
int ocq_version(void);

/* Bytes of the packed weight blob for one block; 0 if the shape or mode is
 * invalid.  The blob holds a 256-byte header followed by the quantized
 * gate/up and down weights in the kernels' fragment order and their scales. */
size_t ocq_packed_bytes(int hidden, int inter, int prec_mode);

/* Quantize and pack one block's weights into a HOST buffer (no GPU used).
 * w_gate_host, w_up_host: fp32 [inter, hidden] row-major ([out, in]).
 * w_down_host: fp32 [hidden, inter] row-major.  Weights must be finite.
 * FP8: one fp32 scale per output row, codes E4M3(fl32(w / scale)).
 * BF16 (down in OCQ_PREC_FP8_DOWN_BF16): round to nearest even.
 * NVFP4: per-tensor S, per-16-input E4M3 block scale, E2M1 codes.
 * packed_host must hold ocq_packed_bytes() bytes.  Thread-safe. */
ocq_status ocq_pack_weights_host(const float* w_gate_host, const float* w_up_host,
                                 const float* w_down_host, int hidden, int inter,
                                 int prec_mode, void* packed_host, size_t packed_bytes);

/* Same, then copy the blob to device memory with hipMemcpyAsync on `stream`
 * and wait for that copy (the staging buffer is freed before returning). */
ocq_status ocq_pack_weights(const float* w_gate_host, const float* w_up_host,
                            const float* w_down_host, int hidden, int inter, int prec_mode,
                            void* packed_dev, size_t packed_bytes, void* stream);

/* Activation-aware smoothing (optional).  The per-token E4M3 scale of x is
 * set by its largest channel, so a few outlier input channels cost every
 * other channel precision.  Per-input-channel factors s[k] move that range
 * into the gate/up weights: the blob holds the codes of fl32(W[n][k] s[k]),
 * and the block multiplies x by fl32(1 / s[k]) before quantizing it, which
 * leaves x W^T unchanged in exact arithmetic.  (The pages' precision is
 * chosen and calibrated per workload: "OCRia 推理栈：单卡 B200 提速近 10 倍",
 * section "Reducing the data moved: workload-aware quantization"; the rule
 * for s below is the published SmoothQuant one.)
 *
 * ocq_calibrate_smoothing_host: s[k] = amax_x[k]^alpha / amax_w[k]^(1-alpha)
 * in double, rounded once to float, where amax_x[k] is max |x[t][k]| over the
 * `rows` calibration rows (bf16 bits [rows, hidden], host) and amax_w[k] is
 * max |W[n][k]| over the rows of both W_gate and W_up (host fp32 [inter,
 * hidden]); s[k] = 1 where either is 0; clamped to [2^-20, 2^20].
 * alpha in [0, 1].  s_out: host float [hidden].
 *
 * ocq_pack_weights_smoothed_host / ocq_pack_weights_smoothed: as the plain
 * packers, with smooth_host = s (host float [hidden], every s[k] finite and
 * > 0; NULL = no smoothing, the same blob as the plain packers).  The down
 * projection is not smoothed.  Blobs are used by ocq_mlp_forward unchanged. */
ocq_status ocq_calibrate_smoothing_host(const void* x_calib_bf16_host, int rows, int hidden,
                                        const float* w_gate_host, const float* w_up_host, int inter,
                                        float alpha, float* s_out);
ocq_status ocq_pack_weights_smoothed_host(const float* w_gate_host, const float* w_up_host,
                                          const float* w_down_host, const float* smooth_host,
                                          int hidden, int inter, int prec_mode, void* packed_host,
                                          size_t packed_bytes);
ocq_status ocq_pack_weights_smoothed(const float* w_gate_host, const float* w_up_host,
                                     const float* w_down_host, const float* smooth_host, int hidden,
                                     int inter, int prec_mode, void* packed_dev, size_t packed_bytes,
                                     void* stream);

/* Inverse of the packing layout, for inspection and tests: from a HOST copy
 * of a blob, write one projection in plain row-major form.
 *   which = 0 gate, 1 up, 2 down, 3 the x multiplier (float [hidden] into
 *   scales_out; codes_out unused).
 *   codes_out: uint8 [rows, cols] (E4M3 or E2M1 code per byte) or uint16
 *              bf16 bits [rows, cols] for a BF16 projection.
 *   scales_out: FP8 -> float [rows]; NVFP4 -> uint8 E4M3 [rows, cols/16];
 *               BF16 -> unused (may be NULL).
 *   tensor_scale_out: NVFP4 -> S; others -> 0 (may be NULL). */
ocq_status ocq_unpack_weights_host(const void* packed_host, size_t packed_bytes, int which,
                                   void* codes_out, void* scales_out, float* tensor_scale_out);

/* Device workspace bytes needed by ocq_mlp_forward for this call shape. */
size_t ocq_workspace_bytes(int M, int hidden, int inter, int prec_mode);

/* Optional plain-layout copies of the intermediates, for parity checks,
 * written by the call's own kernels as they produce them.  Each pointer is a
 * 16-byte-aligned device pointer or NULL.
 *   x_codes [M, hidden] uint8, x_scales [M] float,
 *   h_out:  FP8/NVFP4 modes -> E4M3 codes [M, inter] uint8;
 *           BF16-down mode  -> bf16 bits [M, inter] uint16,
 *   h_scales [M] float (FP8/NVFP4 modes; untouched in BF16-down mode). */
typedef struct {
  void* x_codes;
  void* x_scales;
  void* h_out;
  void* h_scales;
} ocq_taps;

/* One MLP block over M rows, enqueued on `stream` (asynchronous).
 * packed_dev: blob from ocq_pack_weights for (hidden, inter, prec_mode),
 *             packed_bytes >= ocq_packed_bytes(...).
 * x_bf16_dev: bf16 [M, hidden] row-major, finite values.
 * y_bf16_dev: bf16 [M, hidden] row-major, written by the call.
 * workspace_dev: >= ocq_workspace_bytes(M, hidden, inter, prec_mode) bytes;
 *             contents need not be initialized; calls that share a
 *             workspace must be ordered on one stream.
 * taps: NULL or optional intermediate copies (see ocq_taps).
 * The blob header is not read back to the host (that would synchronize);
 * a blob packed for other dimensions or another mode gives wrong results
 * but all reads stay inside packed_bytes.  Use ocq_check_blob to verify. */
ocq_status ocq_mlp_forward(const void* packed_dev, size_t packed_bytes, const void* x_bf16_dev,
                           int M, int hidden, int inter, int prec_mode, void* y_bf16_dev,
                           void* workspace_dev, size_t workspace_bytes, const ocq_taps* taps,
                           void* stream);

/* The same forward call for callers that cannot allocate device memory
 * (code under HIP graph capture that may not call hipMalloc, tight serving
 * loops, hosts that forbid allocation): no workspace argument.  The
 * workspace is a fixed array of ocq_noalloc_scratch_bytes() bytes (32 MiB)
 * in device memory that the library holds on each device it runs on until
 * the process ends; the entry point itself allocates nothing.
 * Arguments, results and errors are those of ocq_mlp_forward, plus
 * OCQ_ERR_BUFFER_TOO_SMALL (before any launch) when
 * ocq_workspace_bytes(M, hidden, inter, prec_mode) exceeds the array.
 * Every call on one device shares that device's array: calls that overlap
 * on one device (different streams, or different threads without ordering)
 * race and give wrong results; calls ordered on one stream are safe.  The
 * array keeps the last call's contents; no call depends on them. */
size_t ocq_noalloc_scratch_bytes(void);
ocq_status ocq_mlp_forward_noalloc(const void* packed_dev, size_t packed_bytes, const void* x_bf16_dev, int M,
                                   int hidden, int inter, int prec_mode, void* y_bf16_dev, const ocq_taps* taps,
                                   void* stream);

/* A stack of L MLP blocks with a precision mode per layer (the pages'
 * mixed-precision scheme at model scale: each layer's weights in the
 * precision chosen for it, BF16 kept for sensitive layers; "OCRia 推理栈：单卡
 * B200 提速近 10 倍", section "Reducing the data moved: workload-aware
 * quantization").  Block l takes the previous block's bf16 output as its x
 * (block 0 takes x_bf16_dev) and the last block writes y_bf16_dev; each block
 * computes exactly what ocq_mlp_forward computes for its mode.
 *
 * ocq_stack_workspace_bytes: device workspace for the call shape (0 if any
 * argument is invalid): the largest block workspace of the schedule plus one
 * bf16 [M, hidden] buffer for the alternating intermediate outputs.
 *
 * ocq_mlp_stack_forward (asynchronous, on `stream`):
 * packed_devs[l]: blob of layer l packed for (hidden, inter, prec_modes[l]),
 *             packed_bytes[l] >= ocq_packed_bytes(hidden, inter, prec_modes[l]);
 * prec_modes: L modes (0, 1 or 2); 1 <= L <= 1024; host arrays, read during
 *             the call only.
 * x_bf16_dev, y_bf16_dev: bf16 [M, hidden]; x is only read, and y must not
 *             overlap x or the workspace.
 * workspace_dev: >= ocq_stack_workspace_bytes(...) bytes.
 * Errors: as ocq_mlp_forward, checked for every layer before any launch.
 * Stage events (ocq_set_stage_events) are not recorded by stack calls. */
size_t ocq_stack_workspace_bytes(int M, int hidden, int inter, const int* prec_modes, int L);
ocq_status ocq_mlp_stack_forward(const void* const* packed_devs, const size_t* packed_bytes,
                                 const int* prec_modes, int L, const void* x_bf16_dev, int M,
                                 int hidden, int inter, void* y_bf16_dev, void* workspace_dev,
                                 size_t workspace_bytes, void* stream);

/* Synchronously read a device blob's header and check it against
 * (hidden, inter, prec_mode): OCQ_OK or OCQ_ERR_BAD_BLOB. */
ocq_status ocq_check_blob(const void* packed_dev, size_t packed_bytes, int hidden, int inter,
                          int prec_mode, void* stream);

/* Per-stage timing hook (profiling).  When set, every later ocq_mlp_forward
 * on this thread records events[i] (hipEvent_t passed as void*, owned by the
 * caller; NULL entries are skipped) on the call's stream at stage boundary i:
 *   0 before the x quantization, 1 start of the gate/up + SiLU kernel,
 *   2 end of the gate/up kernel, 3 before the down projection, 4 after it.
 * Events 1 and 2 are taken by the gate/up launch itself (the kernel's own
 * start and end), so their difference is that kernel's execution time; the
 * others are recorded on the stream between launches.  Not for use while the
 * stream is being captured into a graph.  count must be 5 to enable, 0 (or
 * events == NULL) to disable.  The pointer array is copied; the events must
 * stay valid while the hook is set. */
ocq_status ocq_set_stage_events(void* const* events, int count);

/* Measurement helpers (not part of the block; used by the benchmark and the
 * tests to state what the block's timings and arithmetic are measured
 * against).  All are asynchronous on `stream` and return OCQ_OK,
 * OCQ_ERR_INVALID_ARG (bad size or pointer, checked before any launch) or
 * OCQ_ERR_DEVICE (launch failure).
 *
 * ocq_diag_stream_read: read `bytes` bytes (a multiple of 16, > 0) of the
 *   16-byte-aligned device buffer src_dev with 16-byte loads, `blocks`
 *   workgroups of 256 lanes (1 <= blocks <= 65536), each writing one uint32
 *   to out_dev[block] so the loads are kept: the practical HBM read ceiling
 *   for one launch of that many bytes (the block streams its weights the
 *   same way: "Why decoding dominates latency" in the post, weights read on
 *   every step).
 * ocq_diag_window_read: `blocks` workgroups of 256 lanes each read the same
 *   window of `window_bytes` bytes (a multiple of 32768, at most 2^30) at
 *   src_dev `passes` times with 16-byte loads, each writing one uint32 to
 *   out_dev[block]: with a window that fits L2, the rate at which L2 feeds
 *   the CUs (bytes read = blocks * passes * window_bytes), the ceiling for
 *   operands that many workgroups re-read.
 * ocq_diag_mfma_rate: `blocks` workgroups of 8 waves each issue iters x 16
 *   independent f16 MFMA 16x16x32 on register operands (1 <= iters <= 2^20);
 *   out_dev receives blocks * 512 floats (kept so the work is not dead);
 *   *flops (if non-null) the floating-point operations of the launch: the
 *   matrix-core rate the chip sustains, beside the published dense peak.
 * ocq_diag_empty: one empty kernel (the fixed cost of a launch).
 * ocq_diag_mfma_dot: c[m][n] = sum_k dec(a[m][k]) dec(b[n][k]) over E4M3
 *   codes (a: uint8 [M][K], b: uint8 [N][K], c: float [M][N], row-major,
 *   device, 16-byte aligned; M, N multiples of 16, K a multiple of 128,
 *   M, N, K <= 65536) through one matrix-core instruction form, with the
 *   block's fragment order and per-chunk instruction sequence:
 *     form 0: operands converted exactly to fp16, MFMA 16x16x32 f16 (fp32 sums)
 *     form 1: MFMA 16x16x128 f8f6f4 on the E4M3 codes (unit scales)
 *     form 2: MFMA 16x16x32 fp8 x fp8 on the E4M3 codes
 *   so that each form's sums can be compared against exact ones. */
ocq_status ocq_diag_stream_read(const void* src_dev, size_t bytes, void* out_dev, int blocks, void* stream);
ocq_status ocq_diag_window_read(const void* src_dev, size_t window_bytes, int passes, void* out_dev, int blocks,
                                void* stream);
ocq_status ocq_diag_mfma_rate(int iters, void* out_dev, int blocks, void* stream, double* flops);
ocq_status ocq_diag_empty(void* stream);
ocq_status ocq_diag_mfma_dot(int form, const void* a_dev, const void* b_dev, int M, int N, int K, float* c_dev,
                             void* stream);

/* Per-wave phase stamps of the GEMM main loops, for finding where a kernel's
 * time goes (the roofline method of "Why decoding dominates latency" in the
 * post, applied inside one kernel).  Only a library built with
 * `python -m quantized_memory_bound_amd.build --phase-stamps`
 * (libocq_phases.so) records them; the plain library returns
 * OCQ_ERR_UNSUPPORTED.  Copies, synchronously, the table of the last launch
 * of the chosen kernel family into host_out (caller-owned host memory of at
 * least the stated bytes, else OCQ_ERR_BUFFER_TOO_SMALL), as uint64 values
 * for workgroups 0..511:
 *   kernel 0, LDS-tiled GEMMs (524,288 B): [gate/up, down][workgroup][wave
 *     0..7][load wait, barrier, MFMA batches, LDS-read wait after the batches,
 *     whole loop, stage count], totals in shader-clock ticks;
 *   kernel 1, producer/consumer gate/up (393,216 B): [workgroup][wave 0..11:
 *     8 consumers, then 4 producers][entry, consumer loop start, loop end,
 *     partial tiles stored, wave end, 0, 0, 0], 100 MHz time stamps (the
 *     consumer-only fields are 0 for producers);
 *   kernel 2, x quantization and requantization (32,768 B): [x-quant,
 *     requant][workgroup 0..1023][start, end once its stores have landed],
 *     100 MHz time stamps (0 for workgroups that end early: padding rows,
 *     unused slots of the last group of m-tiles).
 * OCQ_ERR_INVALID_ARG for another kernel value or a null pointer,
 * OCQ_ERR_DEVICE if the copy fails. */
ocq_status ocq_diag_phase_stamps(int kernel, void* host_out, size_t bytes);

/* Where the per-token requantization of h runs (process-wide; mode 0 or 1,
 * default 1; another value: OCQ_ERR_INVALID_ARG).
 * 1: inside the gate/up kernel whenever its whole grid can be resident at
 * once (an occupancy check on the host before each launch): h stays in
 * registers, the row maxima meet through device-scope atomics and the
 * workgroups wait once for each other, bounded by 0.1 s (German page "Wie es
 * funktioniert" of the post: SiLU fused with the quantization, the
 * intermediate kept on chip).  Such a call must not share the GPU with
 * kernels that keep its workgroups from becoming resident for that long; if
 * the wait times out the call's y is NaN.  Where the grid does not fit (the
 * NVFP4 gate/up at 208 rows, the LDS-tiled kernels from 384 rows) or in the
 * BF16-down mode the call takes the two-pass form.  0: always the two-pass
 * form (fp32 h to the workspace, then a requantization kernel).  On MI355X
 * mode 1 is faster by 0.3-1.2 us per block.  Both give bit-identical
 * results. */
ocq_status ocq_set_fused_requant(int mode);

/* Where the last forward call on this thread (ocq_mlp_forward and its
 * no-allocation form, or the last block of ocq_mlp_stack_forward) requantized
 * h: 1 inside the gate/up kernel, 0 in a separate kernel (also the BF16-down
 * mode, which has no requantization), -1 before the first call. */
int ocq_last_requant_in_gateup(void);

/* Message for the last failure on this thread ("" if none). */
const char* ocq_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* OCQ_H */
