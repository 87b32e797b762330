/*
 * qgemm.h - C ABI of libqgemm.so: weight-only low-bit matrix multiply
 *           y = x . dequant(W)^T on AMD Instinct MI355X (gfx950).
 *
 * The operation is the "dequantizing matmul" of the skyzh/tiny-llm feature
 * list (items "Dequantizing Runtimes", "Quantized Matrix Multiplication",
 * "Dequantization Matrix Multiplications"): low-bit weights are turned back
 * into full precision inside the compute pass, so the fp16 weight matrix is
 * never written to memory.  The weight formats are
 *   - QG_INT4_ASYM: 4-bit codes with per-group fp16 scale and zero point (the
 *     INT4 "GPTQ zero points" weights of the TinyLoop README, section "Status");
 *   - QG_INT2_ASYM: 2-bit codes with per-group fp16 scale and zero point (the
 *     INT2 body weights of the TinyLoop README, "Current Runtime Snapshot");
 *   - QG_Q4_0: symmetric blocks of 32 with one fp16 scale and no zero point
 *     (q4_0 of the torchnative guide "Inference with real transformers",
 *     section "Quantise while loading"), codes stored offset-binary u = q + 8;
 *   - QG_Q8_0: the 8-bit sibling of q4_0 named in the same section: blocks of
 *     32, one fp16 scale, signed 8-bit codes stored offset-binary u = q + 128;
 *   - QG_Q4K: the 4-bit k-quant named in the same section (widths divisible
 *     by 256), read as super-blocks of 256 weights with fp16 factors (d, dmin)
 *     and sub-blocks of 32 with 6-bit integers (sc, m):
 *     w = d * sc * q - dmin * m, q in 0..15.
 * For the group formats  w[n,k] = s[n, k/group] * (q[n,k] - z[n, k/group])
 * with z == 8 for q4_0 and z == 128 for q8_0; y[m,n] = sum_k x[m,k] * w[n,k].
 *
 * Conventions shared by every entry point
 *   - Pointers named "device" are device memory (hipMalloc or torch tensors on
 *     the GPU) owned by the caller; the library never keeps or frees them.
 *     Outputs are caller-allocated and written in place.
 *   - fp16 buffers are passed as uint16_t (IEEE binary16 bit patterns).
 *   - Matrices are row-major.  W is [N, K]: groups run along K in one row n.
 *   - Canonical words: uint32 [N, K/cpw], cpw = 8 (INT4, q4_0, q4k), 16 (INT2)
 *     or 4 (q8_0);
 *     code k of row n sits at bits [b*(k%cpw), b*(k%cpw)+b) of word k/cpw.
 *   - Scales (and zero points) are fp16 [N, K/group], canonical.  Zero points
 *     hold integers in [0, 2^b - 1]; other values give unspecified results.
 *     QG_Q4K (group = 256) instead takes scales = fp16 [N, K/256, 2], the
 *     pair (d, dmin) of each super-block, and zeros = uint16 [N, K/32], sc in
 *     the low byte and m in the high byte of each sub-block (both < 64).
 *   - Ownership follows the Mobilint qbruntime.model.Model reference
 *     ("infer_pinned_memory", "infer_npu_data"): the caller allocates the
 *     outputs and the library fills them in place; it allocates nothing the
 *     caller must free.
 *   - "stream" is a hipStream_t (NULL = the default stream).  Every device
 *     call is stream-ordered and asynchronous: QG_OK means "validated and
 *     launched"; a kernel fault is reported by the caller's next sync.
 *   - Arguments are validated on the host before any HIP call.  On error the
 *     function returns a named status (the convention of the named errors of
 *     the same Mobilint reference, e.g. "Model_InvalidVariantIdx") and
 *     launches nothing; nothing aborts or prints.
 *   - QGEMM_CHECK=1 in the environment also asks HIP about every pointer
 *     before any launch and rejects host memory with QG_E_NOT_DEVICE (the
 *     residency rule of "infer_npu_data" in the same reference: a mixed set of
 *     host and device buffers is an error).  Off by default: it costs one
 *     hipPointerGetAttributes per pointer.
 *   - Shapes: group in {32, 64, 128} for INT4/INT2, group == 32 for q4_0 and
 *     q8_0, group == 256 for q4k;
 *     K % group == 0; M, N, K >= 0.  Any N and any M are accepted.
 *   - Device pointers to x, packed, scales, zeros, y and residual must be
 *     16-byte aligned; leading dimensions must be multiples of 8 elements.
 *   - Thread safety: calls are re-entrant, unlike the serialised model of the
 *     TinyLoop "Async API" page ("Concurrency model").  Calls that use the
 *     library-owned split-K workspace (qgemm, or qgemm_ex with workspace ==
 *     NULL) must not overlap on different streams of one device; give each
 *     concurrent stream its own workspace through qgemm_ex.
 */
#ifndef QGEMM_H
#define QGEMM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  QG_INT4_ASYM = 0,
  QG_INT2_ASYM = 1,
  QG_Q4_0 = 2,
  QG_Q8_0 = 3,
  QG_Q4K = 4
} qg_format_t;

typedef enum {
  QG_OK = 0,
  QG_E_ARG = 1,          /* a size, format, group or required pointer is invalid */
  QG_E_UNSUPPORTED = 2,  /* valid request outside what the kernels implement    */
  QG_E_ALIGN = 3,        /* pointer or leading dimension misaligned              */
  QG_E_DEVICE = 4,       /* no usable HIP device, or a HIP call failed            */
  QG_E_NOMEM = 5,        /* the library could not allocate its workspace          */
  QG_E_WORKSPACE = 6,    /* caller workspace too small                            */
  QG_E_NOT_DEVICE = 7    /* QGEMM_CHECK=1: a pointer is not device memory of the current device */
} qg_status_t;

/* Library version as 10000*major + 100*minor + patch. */
int qg_version(void);

/* Human-readable name of a status code (static string, never NULL); the
 * named-error convention of the Mobilint qbruntime.model.Model reference. */
const char* qg_status_str(int status);

/* Text of the last HIP error the library met on this thread (after a
 * QG_E_DEVICE status); "no error" when there was none.  Static string. */
const char* qg_last_error(void);

/* The QGEMM_CHECK=1 pointer rule as a pure function (no HIP call), for tests
 * and callers that query pointer attributes themselves: given the return code
 * of hipPointerGetAttributes, the reported hipMemoryType, the pointer's
 * device and the current device, QG_OK for device memory of the current
 * device or managed / unified memory, QG_E_NOT_DEVICE otherwise (an error
 * code, host memory, arrays).  The residency rule of the Mobilint
 * qbruntime.model.Model reference, "infer_npu_data". */
int qg_classify_pointer(int hip_rc, int memory_type, int ptr_device, int current_device);

/* Bytes of the packed (qpack) code buffer for an [N, K] weight in format fmt
 * (the repacked form of the TinyLoop README, section "Status"):
 * N and K/cpw are rounded up to multiples of 16 (the tile of 16 rows by 16
 * words); padding holds zero codes.  Returns 0 for an invalid request. */
size_t qg_packed_bytes(int64_t N, int64_t K, int fmt);

/*
 * qpack: one-time repack of canonical words into the tile order the kernels
 * stream (the analogue of the repack step the TinyLoop README, section
 * "Status", describes for its tensor-core INT4 path).  A bijection on codes:
 * qunpack(qpack(c)) == c bit for bit.
 *   canon  [device, in]  uint32 [N, K/cpw] canonical words.
 *   packed [device, out] qg_packed_bytes(N, K, fmt) bytes.
 * Packed order: uint32 [ceil(N/16)][ceil(K/cpw/16)][64 lanes][4 words]; lane
 * l = 16*g + r holds words 4g..4g+3 of the 16-word slice of row 16*rb + r,
 * each word with its codes reordered so that even codes fill the low half and
 * odd codes the high half (code j -> slot (j&1)*cpw/2 + j/2).
 * Errors: QG_E_ARG (bad format, N or K < 0, K % cpw != 0, NULL with N*K > 0),
 *         QG_E_ALIGN, QG_E_DEVICE.
 */
int qpack(const uint32_t* canon, uint32_t* packed, int N, int K, int fmt, void* stream);

/* Inverse of qpack (TinyLoop README, "Status": the repack is one-time and
 * lossless): packed -> canonical words [N, K/cpw] (device).  Same errors. */
int qunpack(const uint32_t* packed, uint32_t* canon, int N, int K, int fmt, void* stream);

/* Host versions of qpack / qunpack on host memory (no HIP call): the same
 * permutation, for offline packing (the one-time repack of the TinyLoop
 * README, "Status").  Same errors except QG_E_DEVICE and QG_E_NOT_DEVICE. */
int qpack_host(const uint32_t* canon, uint32_t* packed, int N, int K, int fmt);
int qunpack_host(const uint32_t* packed, uint32_t* canon, int N, int K, int fmt);

/*
 * qgemm: y[M,N] = x[M,K] . dequant(W)^T with fp32 accumulation and one
 * round-to-nearest-even to fp16 at the end -- the dequantizing matmul of the
 * skyzh/tiny-llm feature list ("Dequantizing Runtimes", "Quantized Matrix
 * Multiplication": low-bit weights turned back to full precision inside the
 * compute pass).
 *   x      [device, in]  fp16 [M, K], row-major, leading dimension K.
 *   packed [device, in]  qpack output for W [N, K].
 *   scales [device, in]  fp16 [N, K/group].
 *   zeros  [device, in]  fp16 [N, K/group]; must be NULL for QG_Q4_0 and
 *                        QG_Q8_0 and non-NULL for the asymmetric formats
 *                        (QG_Q4K: the (sc, m) bytes, see above).
 *   y      [device, out] fp16 [M, N], row-major, leading dimension N.
 * M == 1 runs the decode GEMV (packed-fp16 dequant, fp32 dot products);
 * 2 <= M <= 16 the decode GEMV on 16 x 16 matrix-core blocks; M > 16 the
 * MFMA GEMM.  All dequantize to fp16 in registers and accumulate in fp32;
 * split-K partials are reduced in a fixed order, so the result is
 * deterministic.  M == 0 or N == 0 is a no-op; K == 0 writes zeros.
 * Uses a library-owned per-device workspace, allocated (hipMalloc) on first
 * need and grown as needed; call once before capturing into a HIP graph (an
 * allocation cannot happen during capture).  Growing never frees a buffer:
 * an outgrown one is kept until the process ends, so a graph captured before
 * a later, larger call still replays into valid memory.
 * Errors: QG_E_ARG, QG_E_ALIGN, QG_E_UNSUPPORTED, QG_E_DEVICE, QG_E_NOMEM,
 * QG_E_NOT_DEVICE.
 */
int qgemm(const uint16_t* x, const uint32_t* packed, const uint16_t* scales,
          const uint16_t* zeros, int M, int N, int K, int group, int fmt,
          uint16_t* y, void* stream);

/*
 * qgemm_ex: qgemm with leading dimensions, an optional fused residual and an
 * optional caller workspace:  y = x . dequant(W)^T + residual.  The residual
 * is the add around each pair of linears of the looped block (TinyLoop
 * README, "Why TinyLoop Exists"); the leading dimension lets the O
 * projection read the V third of the QKV output in place.
 *   ldx, ldy, ldr  leading dimensions in elements (>= K, >= N, >= N; multiples of 8).
 *   residual       [device, in] fp16 [M, N] with leading dimension ldr, or NULL.
 *                  It may alias y only when ldr == ldy (in-place update).
 *   workspace      [device] caller scratch of ws_bytes >= qgemm_workspace_bytes()
 *                  (fp32 split-K partials; no initial contents needed), or NULL
 *                  for the library's own.
 * Errors: as qgemm, plus QG_E_WORKSPACE.
 */
int qgemm_ex(const uint16_t* x, int ldx, const uint32_t* packed, const uint16_t* scales,
             const uint16_t* zeros, const uint16_t* residual, int ldr,
             int M, int N, int K, int group, int fmt, uint16_t* y, int ldy,
             void* workspace, size_t ws_bytes, void* stream);

/*
 * qgemm_noalloc: qgemm_ex for callers that cannot allocate device memory --
 * code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  Same arguments, kernels and results as qgemm_ex with
 * workspace == NULL, but it never allocates (no hipMalloc, no library
 * routine that allocates): the split-K partials go to a fixed array of
 * QGEMM_NOALLOC_SCRATCH_BYTES in device memory, one per GPU, held from the
 * library's load until the process ends.  Problems whose plan needs more
 * partials than that return QG_E_WORKSPACE (qgemm_workspace_bytes() gives
 * the need).  Every call on one GPU shares that GPU's array and leaves its
 * partials there: calls that overlap on one GPU (different streams, or
 * several host threads) race and must be serialised by the caller.
 * Errors: as qgemm_ex.
 */
#define QGEMM_NOALLOC_SCRATCH_BYTES ((size_t)8 << 20)
int qgemm_noalloc(const uint16_t* x, int ldx, const uint32_t* packed, const uint16_t* scales,
                  const uint16_t* zeros, const uint16_t* residual, int ldr, int M, int N, int K,
                  int group, int fmt, uint16_t* y, int ldy, void* stream);

/* Workspace bytes qgemm_ex needs for this problem (0 when none): the fp32
 * split-K partials of the caller-owned workspace convention above (Mobilint
 * qbruntime.model.Model, "infer_pinned_memory": pre-allocated buffers). */
size_t qgemm_workspace_bytes(int M, int N, int K, int group, int fmt);

/*
 * qloop_block: the weight-shared looped block of the TinyLoop README (section
 * "Why TinyLoop Exists": one block applied L times with the same weights).
 * For l = 1..L, with D = K of the QKV linear:
 *     qkv = x . Wqkv^T                  [M, 3D]
 *     h   = x + qkv[:, 2D:3D] . Wo^T    [M, D]    (residual fused)
 *     u   = h . Wup^T                   [M, F]
 *     x   = h + u . Wdown^T             [M, D]    (residual fused)
 * All four linears share one format and group.
 *   x        [device, in/out] fp16 [M, D]: x_0 on entry, x_L on return.
 *   packed4  host array of 4 device pointers (QKV, O, up, down), qpack output.
 *   scales4, zeros4  host arrays of 4 device pointers (zeros4 entries NULL for q4_0 and q8_0).
 *   F        the MLP width (N of up, K of down).
 *   scratch  [device] fp16 buffer of at least M*(3D + D + F) elements.
 *   events   NULL, or a host array of L+1 hipEvent_t recorded on the stream
 *            before loop 1 and after each loop (per-loop timing).
 * All four calls are validated before any event is recorded or kernel
 * launched, and the split-K workspace is obtained up front, so on error
 * nothing is launched and x is untouched.
 * Errors: as qgemm_ex.
 */
int qloop_block(uint16_t* x, const uint32_t* const* packed4, const uint16_t* const* scales4,
                const uint16_t* const* zeros4, int M, int D, int F, int group, int fmt,
                int L, uint16_t* scratch, void* const* events, void* stream);

/*
 * qloop_block_persistent: qloop_block at M = 1 with one launch per loop (the
 * shared block of the TinyLoop README, "Why TinyLoop Exists", run L times;
 * "Status": the shared weights stay cache-resident across the iterations).
 * Each launch is a grid of one workgroup per compute unit (never more than
 * the occupancy calculator says are resident together); they run the loop's
 * four GEMVs as phases over blocks of 8 rows of W, separated by grid
 * barriers on counters in device memory the library keeps for the process.
 * Same arguments, layouts and results as qloop_block, plus
 *   mode   0: one launch per loop (three barriers in each); 1: one launch for
 *          all L loops (a fourth barrier between loops; x and the residuals
 *          are then read with agent scope, and the workgroup that runs a block
 *          of rows in one loop runs it in every loop, so its XCD's L2 can keep
 *          those rows' weights across loops).  With mode 1 every per-loop
 *          event is recorded after the one launch.
 *   status [device, out] int32, 16-byte aligned: 0 after the call's loops
 *          complete, 1 if a barrier stopped waiting (its wait is bounded:
 *          QGEMM_LOOP_SPIN_CAP polls, 2^18 by default; then x holds no
 *          meaningful result).
 *          Written in stream order; read it after the stream is synchronized.
 * Supported: M == 1; formats QG_INT4_ASYM, QG_INT2_ASYM, QG_Q4_0, QG_Q4K;
 * K of every linear at most 64 word tiles (8192 for 4-bit codes).  Calls that
 * overlap on one device (the counter is shared) race.
 * Errors: as qloop_block, QG_E_ARG (status NULL, mode not 0 or 1),
 * QG_E_UNSUPPORTED (M != 1, format or K outside the above).
 */
int qloop_block_persistent(uint16_t* x, const uint32_t* const* packed4, const uint16_t* const* scales4,
                           const uint16_t* const* zeros4, int M, int D, int F, int group, int fmt, int L,
                           uint16_t* scratch, int mode, int* status, void* const* events, void* stream);

/* Debug: packed -> integer codes uint8 [N, K] (device), for the bit-exact
 * check of the kernels' unpack (the nibble / crumb unpack of the TinyLoop
 * README, "Status").  Errors as qunpack. */
int qg_unpack_codes(const uint32_t* packed, uint8_t* codes, int N, int K, int fmt,
                    void* stream);

/* Debug and the dequantize-at-load comparison (TinyLoop README, "Current
 * Runtime Snapshot": an FP16 body whose weights are dequantized once):
 * packed + scales + zeros -> fp16 w [N, K] (device) through the same device
 * dequant the GEMM uses: fp16_rne(s * (q - z)); for QG_Q4K
 * fp16_rne(fp16_rne(d*sc) * q - fp16_rne(dmin*m)) (one fused multiply-add).
 * scales and zeros must be 16-byte aligned like the other buffers.
 * Errors as qgemm. */
int qg_dequant(const uint32_t* packed, const uint16_t* scales, const uint16_t* zeros,
               uint16_t* w, int N, int K, int group, int fmt, void* stream);

/* Launch plan the library would use (for tracing and tests; no HIP call; the
 * phase timings of the TinyLoop README, "Quick CLI Tour", need the kernel
 * behind each call):
 * out[0] = path (1 GEMV, 2 GEMM), out[1] = K splits, out[2] = workgroups,
 * out[3] = tile rows (M), out[4] = tile columns (N) -- for the GEMV, the rows of
 * x per launch (1, 2, 4, 8 or 16) and the rows of W per workgroup (16, or 8 when
 * M <= 2 and 8-row workgroups need fewer launches or spread more evenly over
 * the compute units; M = 3, 4 only when QGEMM_GEMV_ROWS=8 forces it).
 * Errors as qgemm. */
int qg_plan(int M, int N, int K, int group, int fmt, int out[5]);

/*
 * Measurement helpers: the ceilings a qGEMM kernel is read against, taken on
 * the device it runs on (the hot-op microbenchmarks of the TinyLoop README,
 * "Validation", and the phase timings of its "Quick CLI Tour", "Benchmark").
 * They are not on the qGEMM path.  Launches are asynchronous on `stream`
 * (NULL: the default stream); the return code reports the launch only.
 */

/* Plain streaming read of `bytes` bytes at src (device, 16-byte aligned) by
 * `workgroups` workgroups of 256 lanes, 16-byte non-temporal loads at a grid
 * stride: the bandwidth one launch reaches over that many bytes.
 *   sink [device, out] uint32 [workgroups]; written only in the (practically
 *        impossible) case that the folded data equals a fixed constant.
 * Errors: QG_E_ARG (NULL pointer, workgroups <= 0), QG_E_ALIGN, QG_E_DEVICE. */
int qg_stream_read(const void* src, size_t bytes, uint32_t* sink, int workgroups, void* stream);

/* An empty kernel of `workgroups` x `threads` (1..1024): the launch floor of
 * that grid.  Errors: QG_E_ARG, QG_E_DEVICE. */
int qg_empty_launch(int workgroups, int threads, void* stream);

/* `iters` rounds of 16 independent v_mfma_f32_16x16x32_f16 (16*16*32*2 flops
 * each) in every wave of `workgroups` workgroups of 4 waves: the sustained
 * dense fp16 matrix rate.  out [device, out] float [workgroups * 256].
 * Errors: QG_E_ARG, QG_E_DEVICE. */
int qg_mfma_probe(float* out, int workgroups, int iters, void* stream);

/* Compute units, shader clock (kHz), memory clock (kHz) and memory bus width
 * (bits) of `device`, as the HIP runtime reports them.
 * Errors: QG_E_ARG (NULL pointer), QG_E_DEVICE. */
int qg_device_info(int device, int* compute_units, int* clock_khz, int* memory_clock_khz,
                   int* memory_bus_bits);

/* One wave stores the device's constant-rate clock (the counter that
 * qg_clock_rate reports) into out[0], in stream order: it runs after every
 * earlier launch on `stream` has completed and before any later one starts,
 * so two stamps bracket exactly the launches between them on the device.
 * Inside a captured graph this keeps the graph's own launch latency out of
 * the bracket, which events recorded around the graph would include (events
 * cannot be recorded inside a graph on this runtime).  Follows the phase
 * timings of the TinyLoop README, "Quick CLI Tour", "Benchmark".
 * out [device, out] uint64 [1], 8-byte aligned; written asynchronously.
 * Errors: QG_E_ARG (NULL), QG_E_ALIGN, QG_E_DEVICE. */
int qg_clock_stamp(uint64_t* out, void* stream);

/* Rate (kHz) of the clock qg_clock_stamp reads, as the HIP runtime reports it.
 * Errors: QG_E_ARG (NULL pointer), QG_E_DEVICE. */
int qg_clock_rate(int device, int* khz);

#ifdef __cplusplus
}
#endif

#endif /* QGEMM_H */
