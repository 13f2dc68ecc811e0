/*
 * trace_fp4.h — C ABI of the rollout-guided FP4 fake-quantization library
 * (MI355X / gfx950).
 *
 * The operations follow "TRACE: Rollout-Guided Quantization-Aware Training
 * for FP4 Reinforcement Learning of MoE Language Models" (arXiv 2610.07767),
 * cited below by section of its reader-view page.
 *
 * Conventions shared by every call
 * --------------------------------
 * Tensors. A tensor is a contiguous row-major [rows, cols] array of bf16 bit
 * patterns (uint16_t). Blocks run along the last dimension: B = 16 elements
 * for NVFP4, 32 for MXFP4, and cols must be a multiple of B. N = rows * cols.
 * Block j covers elements [j*B, (j+1)*B) of the flattened tensor.
 *
 * Global-scale groups (NVFP4). group_rows > 0 splits the rows into
 * G = rows / group_rows consecutive groups (group_rows must divide rows), each
 * quantized as its own tensor with its own FP32 global scale; group_rows == 0
 * means one group holding every row (G = 1). This lets one call cover, e.g.,
 * all 8192-token chunks of a streamed layer. For MXFP4 (no global scale) the
 * grouping has no effect on the results.
 *
 * Pointers. Every pointer argument is a DEVICE pointer owned by the caller;
 * nothing is retained after the call returns. Input arrays are only read.
 * bf16 arrays must be 16-byte aligned; code planes 4-byte aligned; 2-bit
 * planes 2-byte aligned; global scales 4-byte aligned; workspaces, float64
 * accumulators and int64 counts 8-byte aligned. Other planes have no
 * alignment requirement. When N == 0 the data pointers
 * may be NULL.
 *
 * Planes written or read by the calls:
 *   codes   uint8[N/2]  E2M1 codes, code = sign << 3 | k, k the 3-bit magnitude
 *                       index (magnitudes 0, .5, 1, 1.5, 2, 3, 4, 6); element
 *                       2i in the low nibble of byte i, 2i+1 in the high one.
 *   mbits   uint8[N/8]  one bit per element, the mantissa bit k & 1; element
 *                       8i+j in bit j of byte i (LSB first).
 *   lowb    uint8[N*b/8] b = 1, 2 or 3 low bits of each magnitude index k
 *                       (b = 1 is mbits), as one LSB-first bit string: element
 *                       i occupies bits b*i .. b*i+b-1 (b = 2: element 4j+i at
 *                       bits 2i of byte j; b = 3: element 8j+i at bits 3i of
 *                       the little-endian 24-bit group in bytes 3j..3j+2).
 *   scales  uint8[N/B]  NVFP4: E4M3 (bias 7, OCP "fn") block scale; MXFP4:
 *                       E8M0 block scale (byte = E + 127). One byte per block,
 *                       block order. Bytes read by a call must be valid
 *                       non-negative finite values (E4M3 <= 0x7E, E8M0 <= 254);
 *                       otherwise results are unspecified (memory-safe).
 *   gscale  float32[2G] NVFP4 only: for group g, [2g] = the FP32 global scale
 *                       S, [2g+1] = the group amax A it came from.
 *
 * Scaling (NVFP4). A = max|x| over the group; S = 2688 / A (1 if A == 0, at
 * most FLT_MAX). Per block with max a: u = (a / 6) * S, e = E4M3 of
 * min(u, 448) rounded to nearest even; decode factor d = e / S, encode factor
 * r = min(S / e, FLT_MAX), both 0 when e == 0. The normalized value of an
 * element is t = |x| * r. Binary32 arithmetic, each operation rounded, no
 * fused multiply-add. (Paper §3.1 "Key Design", Fig. 4(a): the same global
 * and block scales; Algorithm 1 prose: s combines block and global scales.)
 *
 * Scaling (MXFP4). E = clamp(floor(log2 a) - 2, -127, 127), -127 for an
 * all-zero block; t = |x| * 2^-E, d = 2^E. (Paper §4.3, MXFP4 variants.)
 *
 * Rounding. RTN rounds t to the nearest E2M1 magnitude, ties to the even
 * index, saturating at 6. Every code and output keeps its input's sign bit
 * (a negative value that rounds to zero gives code 0x8 and bf16 -0.0). The
 * dequantized output is y = sign * bf16(v(k) * d), bf16 rounded to nearest
 * even. (Paper §3.1 "Motivation": FP4 fake quantization in the forward pass.)
 *
 * Global scale source (quantize_rtn, encode_guidance). For NVFP4 exactly one
 * of gscale_in / gscale_out is non-NULL: gscale_in holds a caller-chosen S
 * per group (read at [2g]); gscale_out receives {S, A} per group computed from
 * the tensor, and then `work` must hold trace_quant_workspace_bytes(...)
 * bytes. For MXFP4 both must be NULL (and work may be NULL).
 *
 * Sizes. A call takes at most 2^35 elements (N = rows * cols) and, with
 * row offsets, at most 2^22 groups; beyond that it returns TRACE_ESHAPE. These
 * keep every launch within the 32-bit work-item count of a dispatch.
 *
 * Streams and errors. Every call validates its arguments on the host before
 * any HIP call, then enqueues its kernels on `stream` (a hipStream_t; NULL is
 * the null stream) and returns without synchronizing. Calls allocate no
 * memory. Results are bit-deterministic. A call that returns an error has
 * enqueued nothing, except TRACE_ELAUNCH, which reports a HIP error seen at
 * launch. Calls are reentrant and may run concurrently on different streams
 * when their buffers (workspaces included) are disjoint. Workspace contents
 * on entry do not matter and are left undefined.
 */
#ifndef TRACE_FP4_H
#define TRACE_FP4_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define TRACE_ABI_VERSION 9

/* Entries of the mismatch diagnostics of guided_fake_quant_stats. */
#define TRACE_MISMATCH_COUNTS 32

/* Bytes of the library's own per-device workspace of encode_guidance_noalloc. */
#define TRACE_NOALLOC_SCRATCH_BYTES (4 << 20)

enum trace_fmt { TRACE_FMT_NVFP4 = 0, TRACE_FMT_MXFP4 = 1 };

enum trace_status {
  TRACE_OK = 0,
  TRACE_EINVAL = -1,  /* NULL required pointer, bad fmt/bits/flag, bad gscale combination */
  TRACE_ESHAPE = -2,  /* negative size, cols % B != 0, group_rows not dividing rows, N above 2^35,
                         workspace too small */
  TRACE_EALIGN = -3,  /* a pointer misses its alignment */
  TRACE_EALIAS = -4,  /* an output overlaps an input or another output */
  TRACE_EDEVICE = -5, /* no current gfx950 device */
  TRACE_ELAUNCH = -6, /* HIP reported an error when the kernels were enqueued */
  TRACE_EBUSY = -7    /* trace_ring_push: the next slot has not been released */
};

/* TRACE_ABI_VERSION of the built library. */
int trace_abi_version(void);

/* Static name of a status code ("TRACE_OK", ...); "unknown status" otherwise. */
const char* trace_status_str(int status);

/* How NVFP4 calls that derive S from the amax schedule their work.
 * groups_per_batch = 0 (the default): a call of two or more groups of at
 * most (2 x CUs - 1) x 33792 elements (17.3M on a 256-CU MI355X, e.g. 8192 x
 * 2048 chunks) is encoded in ONE pass over the input by a launch of at most
 * as many workgroups as the device holds at once, which keep their tiles on
 * chip while each group's amax is combined (it needs 2 resident workgroups
 * of 768 threads per CU; otherwise, for larger groups, and for a call of a
 * single group, which is faster in two launches, the two-pass schedule
 * below is used). Row-offset groups (encode_guidance_grouped, at most 4096
 * groups) take one pass too, over a table of 32768-element tiles built on
 * the device from the offsets; when a group has more tiles than the launch
 * has tile workgroups, that launch reads every tile's maxima first and then
 * quantizes (still one launch, two reads of the input).
 * n > 0 forces two passes (amax, then quantize) with n groups per batch: each
 * launch quantizes one batch while it reads the next batch for its amax
 * (n >= G: one amax pass over every group, then one quantize pass); with 0,
 * two-pass batches are about 96 MiB of input. Results are bit-identical for
 * every setting; the knob exists to exercise and compare schedules.
 * Single-pass launches of a process run one after another on each device,
 * whatever their streams (each needs the whole device at once), without any
 * host synchronization: the first one on a second stream waits (on the
 * device) for an event recorded at that moment on the stream of the previous
 * single-pass launch, so that stream must not have been destroyed yet; later
 * ones wait on the previous one's event. A graph capture adds no ordering (a
 * graph runs in order). Two graphs or processes that encode at the same time
 * on one device are not ordered: a workgroup whose wait on another then runs
 * too long stops waiting and reads what it waited for from the input itself,
 * so the results stay exact and only the time grows (see
 * trace_set_wait_limit and trace_encode_wait_failures).
 * Process-wide. Returns the previous setting, or TRACE_EINVAL for a negative
 * value. */
int64_t trace_set_encode_batch(int64_t groups_per_batch);

/* Bound of every wait of the single-pass encode on other workgroups, in
 * polls (0 = the default, 4,194,304 polls, about 0.25 s). A wait that reaches
 * it gives up and takes what it waited for from the input instead: the
 * combining wave reads the tiles whose maxima were not published, a
 * workgroup whose group scale did not arrive reduces the group's amax
 * itself. Both give the exact maximum, so every output is the same as
 * without the give-up; the call only runs longer. Each give-up adds 1 to the
 * device's count (trace_encode_wait_failures). For callers and tests that
 * exercise that path (a limit of 1 makes nearly every wait give up at once).
 * Process-wide. Returns the previous setting, or TRACE_EINVAL for a value
 * below 0 or above 2^31 - 1. */
int64_t trace_set_wait_limit(int64_t polls);

/* *count = number of bounded waits of the single-pass encode that gave up on
 * the current device since the library was loaded (0 when every launch had
 * the whole device to itself). Reads device memory with a synchronous copy
 * on the null stream: synchronize the streams of the encode calls first.
 * EINVAL: count is NULL; EDEVICE: no gfx950 device is current; ELAUNCH: the
 * copy failed. */
int trace_encode_wait_failures(uint64_t* count);

/* Workspace bytes quantize_rtn / encode_guidance need to derive the global
 * scales from the amax (NVFP4 with gscale_out): 8192 * G (per group 1024
 * partial maxima and 1024 words for the published S), except 0 when a
 * group's element count is a power of two from 16 to 8192 and G > 1 (such
 * groups, e.g. one token's row for a per-token global scale, are reduced
 * and quantized in one pass); 0 for MXFP4. -1 for an invalid shape. */
int64_t trace_quant_workspace_bytes(int fmt, int64_t rows, int64_t cols, int64_t group_rows);

/* Workspace bytes guided_fake_quant_stats needs. -1 for an invalid shape. */
int64_t trace_guided_stats_workspace_bytes(int fmt, int64_t rows, int64_t cols,
                                           int64_t group_rows);

/* Workspace bytes discrepancy_stats needs for n elements (>= 16). */
int64_t trace_stats_workspace_bytes(int64_t n);

/*
 * quantize_rtn — vanilla FP4 fake quantization of one tensor (or of each
 * group) with its own scales (paper §3.1 "Motivation": QAT fake
 * quantization; Fig. 4(a): RTN).
 *
 *   x       in   bf16[N]
 *   codes   out  uint8[N/2]      E2M1 codes of RTN(t)
 *   scales  out  uint8[N/B]      block scales
 *   gscale_in / gscale_out       see "Global scale source"
 *   y_opt   out  bf16[N] or NULL dequantized output y
 *   work, work_bytes             see "Global scale source"
 */
int quantize_rtn(int fmt, int64_t rows, int64_t cols, int64_t group_rows, const uint16_t* x,
                 const float* gscale_in, uint8_t* codes, uint8_t* scales, float* gscale_out,
                 uint16_t* y_opt, void* work, int64_t work_bytes, void* stream);

/*
 * encode_guidance — rollout side: quantize with RTN and emit the guidance
 * record (paper §3.2 "Key Design", Fig. 6; §4.2 "Rollout Efficiency": one
 * mantissa bit plus the amortized block scale, 1.5 bits per element for
 * NVFP4; Algorithm 1 prose: packed low-bit rollout codes plus the rollout
 * scales).
 *
 *   bits    1: guide = mbits uint8[N/8] (mantissa bit of each rollout code)
 *           2, 3: guide = lowb uint8[N*bits/8] (the low 2 or 3 magnitude
 *              bits: Algorithm 1's parameter b; 2.5 and 3.5 bits per
 *              element with the NVFP4 scale)
 *           4: guide = codes uint8[N/2] (the full signed rollout codes, the
 *              full-information record of §3.1)
 *   x_rollout      in   bf16[N]
 *   guide          out  see bits
 *   scales         out  uint8[N/B]
 *   gscale_in / gscale_out, work   see "Global scale source"
 *   y_rollout_opt  out  bf16[N] or NULL, the rollout's own dequantized output
 */
int encode_guidance(int fmt, int bits, int64_t rows, int64_t cols, int64_t group_rows,
                    const uint16_t* x_rollout, const float* gscale_in, uint8_t* guide,
                    uint8_t* scales, float* gscale_out, uint16_t* y_rollout_opt, void* work,
                    int64_t work_bytes, void* stream);

/*
 * encode_guidance_noalloc — encode_guidance for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation. Same arguments (without work and work_bytes) and
 * bit-identical results. Where encode_guidance needs a workspace (NVFP4 with
 * gscale_out: S from each group's amax), this call uses the library's own
 * device array of TRACE_NOALLOC_SCRATCH_BYTES (4 MiB) instead; each device
 * holds its copy from the library's load until the process ends, and the call
 * itself allocates nothing.
 * Limit: trace_quant_workspace_bytes(fmt, rows, cols, group_rows) at most
 * TRACE_NOALLOC_SCRATCH_BYTES, i.e. at most 512 global-scale groups that need
 * the amax workspace (packed small groups, S supplied and MXFP4 need none);
 * beyond it the call returns TRACE_ESHAPE and enqueues nothing.
 * Every call on a device shares that device's array, and the array keeps what
 * the last call left: each call clears what must start at zero itself (on its
 * stream, with a kernel), so results never depend on earlier calls. Calls
 * whose executions overlap on one device (on other streams or threads, or
 * graphs replayed at the same time) race on the array and give undefined
 * results: order them.
 */
int encode_guidance_noalloc(int fmt, int bits, int64_t rows, int64_t cols, int64_t group_rows,
                            const uint16_t* x_rollout, const float* gscale_in, uint8_t* guide,
                            uint8_t* scales, float* gscale_out, uint16_t* y_rollout_opt, void* stream);

/*
 * decode_guidance — training side, compact record: Reconstruct (Algorithm 1
 * prose). For each element, t = |x_train| * r under the ROLLOUT block scale;
 * the reference index is the E2M1 magnitude nearest t whose low `bits`
 * magnitude bits equal the rollout's, ties toward the larger magnitude; its
 * sign is the training sign. A rollout block whose scale is zero gives t = 0.
 *
 *   bits      1, 2 or 3
 *   x_train   in   bf16[N]
 *   guide     in   uint8[N*bits/8]   from encode_guidance(bits)
 *   scales    in   uint8[N/B]   rollout block scales
 *   gscale    in   float[2G]    NVFP4: rollout S of group g at [2g]; MXFP4: NULL
 *   ref_codes out  uint8[N/2]
 */
int decode_guidance(int fmt, int bits, int64_t rows, int64_t cols, int64_t group_rows,
                    const uint16_t* x_train, const uint8_t* guide, const uint8_t* scales,
                    const float* gscale, uint8_t* ref_codes, void* stream);

/*
 * guided_fake_quant — training side, rollout-guided rounding (paper §3.1
 * "Key Design", Eq. 2 prose; Algorithm 1 prose: BracketFP4 then the candidate
 * nearest the reference, STE forward value). Under the ROLLOUT scales,
 * t = |x_train| * r is bracketed by its two neighbouring E2M1 magnitudes
 * {q-, q+} (a single one when t is a codeword or t >= 6) and one is chosen:
 *
 *   bits 0  RTN (the q_RTN of the local guarantee, §3.1); guide must be NULL
 *   bits 1, 2, 3  the candidate nearest the Reconstruct reference from the
 *           low `bits` magnitude bits (decode fused); guide = lowb
 *           uint8[N*bits/8]
 *   bits 4  the candidate nearest the exact rollout codeword, both signed
 *           (candidates carry the training sign); guide = codes uint8[N/2]
 *
 *   x_train    in   bf16[N]
 *   guide      in   see bits
 *   scales     in   uint8[N/B]   rollout block scales
 *   gscale     in   float[2G]    NVFP4: rollout S of group g at [2g]; MXFP4: NULL
 *   y          out  bf16[N]      sign(x_train) * bf16(v(k) * d_rollout)
 *   codes_opt  out  uint8[N/2] or NULL, the chosen codes
 */
int guided_fake_quant(int fmt, int bits, int64_t rows, int64_t cols, int64_t group_rows,
                      const uint16_t* x_train, const uint8_t* guide, const uint8_t* scales,
                      const float* gscale, uint16_t* y, uint8_t* codes_opt, void* stream);

/*
 * guided_fake_quant_stats — guided_fake_quant plus, in the same pass over
 * the data, the discrepancy sums of discrepancy_stats(x_train, x_rollout, y,
 * y_rollout), where y_rollout is the rollout's RTN output under the same
 * rollout scales (what encode_guidance writes to y_rollout_opt); it is
 * recomputed from x_rollout instead of being read. Paper §3.1 Eq. 1 and
 * Fig. 4(b) (D_BF16, D_FP4 and the relative excess).
 *
 *   x_rollout  in   bf16[N], the rollout input the record was encoded from
 *   acc3, accumulate           as in discrepancy_stats
 *   counts_opt out  int64[TRACE_MISMATCH_COUNTS] or NULL: mismatch
 *              diagnostics (paper §3.2 "Key Design", Fig. 6: how far the
 *              training codes land from the rollout codes, and in which
 *              direction guidance moves them). With p(c) = the signed grid
 *              position of code c (magnitude index k with the code's sign,
 *              -7..7, +-0 both 0), guided codes c_t, rollout RTN codes c_r
 *              and training RTN codes c_b (both under the rollout scales):
 *                [0..14]  number of elements with |p(c_t) - p(c_r)| = 0..14
 *                [15..29] number of elements with |p(c_b) - p(c_r)| = 0..14
 *                [30]     elements whose guided magnitude index exceeds c_b's
 *                [31]     elements whose guided magnitude index is below c_b's
 *              Overwritten or, with accumulate = 1, added to (as acc3).
 *              Exact integer counts. Computing them costs extra time.
 *   work, work_bytes           trace_guided_stats_workspace_bytes(...) bytes
 *   other arguments            as in guided_fake_quant
 *
 * The sums equal discrepancy_stats' within 5 * 2^-24 relative (binary32
 * squares of single pairs, exact binary64 fallback outside a safe range); the
 * summation order is fixed by the shape, so results are bit-deterministic.
 */
int guided_fake_quant_stats(int fmt, int bits, int64_t rows, int64_t cols, int64_t group_rows,
                            const uint16_t* x_train, const uint16_t* x_rollout,
                            const uint8_t* guide, const uint8_t* scales, const float* gscale,
                            uint16_t* y, uint8_t* codes_opt, double* acc3, int64_t* counts_opt,
                            int accumulate, void* work, int64_t work_bytes, void* stream);

/*
 * discrepancy_stats — the sums behind the train–rollout discrepancy
 * measures (paper §3.1 "Motivation", Eq. 1; "Key Design", Fig. 4(b):
 * D_FP4, D_BF16 and the relative excess (D_FP4 - D_BF16) / D_BF16).
 *
 *   n          number of elements in each of the four arrays
 *   x_t, x_r   in  bf16[n]  training / rollout inputs
 *   y_t, y_r   in  bf16[n]  training / rollout FP4 outputs
 *   acc3       out float64[3] = {SB, SF, count}: SB = sum (x_t - x_r)^2,
 *              SF = sum (y_t - y_r)^2, count = n. accumulate = 0 overwrites,
 *              1 adds to the previous contents (a per-layer sum over chunks).
 *   work       trace_stats_workspace_bytes(n) bytes of device memory
 *   work_bytes size of `work`
 *
 * Each sum is within 5 * 2^-24 relative of the exact value (see
 * guided_fake_quant_stats) and taken in a fixed order determined by n alone,
 * so the result is bit-identical from run to run.
 */
int discrepancy_stats(int64_t n, const uint16_t* x_t, const uint16_t* x_r,
                      const uint16_t* y_t, const uint16_t* y_r, double* acc3,
                      int accumulate, void* work, int64_t work_bytes, void* stream);

/*
 * Groups of unequal size: row-offset groups (paper Algorithm 1 prose: s
 * combines block and token/global scales; here one FP32 global scale per
 * expert of a grouped MoE input, whose routed rows are contiguous per
 * expert). row_offsets is a DEVICE int64[groups + 1] array of row offsets,
 * read on the device (it may come straight from routing); group g is rows
 * [off[g], off[g + 1]). Offsets are clamped into [0, rows] and made
 * nondecreasing (a running max), so a bad array cannot cause out-of-range
 * accesses; rows outside [off[0], off[groups]) are not written. An empty
 * group gets {S, A} = {1, 0}. Results equal separate calls on each group's
 * rows. NVFP4 only matters here: for MXFP4 (no global scale) the offsets are
 * not read and the call equals the ungrouped one (gscale pointers NULL).
 * groups in [1, 2^22]; otherwise ESHAPE.
 */

/* Workspace bytes of the two calls below; 0 for MXFP4, -1 for an invalid
 * shape or group count. */
int64_t trace_grouped_workspace_bytes(int fmt, int64_t rows, int64_t cols, int64_t groups);

/* encode_guidance with one global scale per row-offset group: gscale_out
 * receives {S, A} of group g at [2g], [2g + 1] (required for NVFP4). Other
 * arguments as in encode_guidance (bits 1..4; bits = 4 with y_rollout_opt
 * is exactly quantize_rtn per group). Scheduled as trace_set_encode_batch
 * describes (one pass for at most 4096 groups, else two); the results are
 * bit-identical either way. */
int encode_guidance_grouped(int fmt, int bits, int64_t rows, int64_t cols, int64_t groups,
                            const int64_t* row_offsets, const uint16_t* x_rollout, uint8_t* guide,
                            uint8_t* scales, float* gscale_out, uint16_t* y_rollout_opt, void* work,
                            int64_t work_bytes, void* stream);

/* guided_fake_quant under per-group rollout scales: gscale holds S of group g
 * at [2g]. Other arguments as in guided_fake_quant (bits 0..4). */
int guided_fake_quant_grouped(int fmt, int bits, int64_t rows, int64_t cols, int64_t groups,
                              const int64_t* row_offsets, const uint16_t* x_train, const uint8_t* guide,
                              const uint8_t* scales, const float* gscale, uint16_t* y, uint8_t* codes_opt,
                              void* work, int64_t work_bytes, void* stream);

/*
 * Record path (paper §3.2 "Motivation": records are cached during generation
 * and transferred to the training side; "Key Design": records are indexed by
 * trajectory, token and site, and the KV guidance already sits in the FP4 KV
 * cache). These calls move finished records off the GPU; the guidance calls
 * above produce them.
 *
 * trace_ring — a ring of `slots` pinned host buffers of `slot_bytes` each,
 * with its own copy stream (default priority) and one event per slot. Slots
 * are used in ring order and cycle FREE -> IN FLIGHT (push) -> DONE (wait or
 * query) -> FREE (release). A ring belongs to the device current at creation
 * and is used from that device. Calls on one ring are thread-safe.
 */
typedef struct trace_ring trace_ring;

/* Allocates the pinned slots (hipHostMalloc), the copy stream and the events.
 * *ring receives the handle (NULL on error). ESHAPE: slot_bytes <= 0, slots
 * outside [1, 4096] or more than 2^40 bytes in total; EDEVICE: the current
 * device is not a gfx950; ELAUNCH: an allocation failed. */
int trace_ring_create(int64_t slot_bytes, int32_t slots, trace_ring** ring);

/* Waits for the ring's copies, then frees everything. */
int trace_ring_destroy(trace_ring* ring);

/* Copies n device buffers srcs[i] of bytes[i] bytes, back to back, into the
 * next slot, after all work enqueued so far on after_stream (a hipStream_t,
 * NULL = null stream); the producer stream is not blocked. *slot receives the
 * slot index. The copies run later, on the ring's stream: every source
 * buffer must stay allocated and unmodified until the slot's copies are done
 * (trace_ring_wait returned, or trace_ring_query returned 1); freeing or
 * reusing one earlier (e.g. through a caching allocator that hands it to the
 * producer stream's next allocation) leaves undefined bytes in the slot.
 * ESHAPE: a negative size or more than slot_bytes in total; EBUSY: the next
 * slot is still in flight or not released (nothing is enqueued); EDEVICE:
 * called from another device. */
int trace_ring_push(trace_ring* ring, const void* const* srcs, const int64_t* bytes, int32_t n,
                    void* after_stream, int32_t* slot);

/* Blocks until the slot's copies are done (slot becomes DONE). EINVAL for a
 * FREE slot. */
int trace_ring_wait(trace_ring* ring, int32_t slot);

/* 1 when the slot's copies are done (slot becomes DONE), 0 when still in
 * flight; EINVAL for a FREE slot. Never blocks. */
int trace_ring_query(trace_ring* ring, int32_t slot);

/* Host address of a DONE slot's bytes (valid until it is released) and, in
 * *bytes (optional), how many were pushed; NULL when the slot is not DONE. */
const void* trace_ring_slot(trace_ring* ring, int32_t slot, int64_t* bytes);

/* Returns a DONE slot to the ring. EINVAL otherwise. */
int trace_ring_release(trace_ring* ring, int32_t slot);

/*
 * trace_gather_pages — collects a finished request's pages of a paged record
 * (for example the code or scale plane of the FP4 KV cache) into one
 * contiguous buffer before its transfer: page i of out = page page_ids[i] of
 * pool. An id outside [0, pool_pages) gives a page of zero bytes and adds 1 to
 * *bad_ids (if given); the kernel never reads outside the pool.
 *
 *   pool       in   uint8[pool_pages * page_bytes]   device
 *   page_ids   in   int32[n]                          device, 4-byte aligned
 *   out        out  uint8[n * page_bytes]             device
 *   bad_ids    in/out uint32 or NULL                  device, 4-byte aligned;
 *                   incremented, never cleared
 *
 * Moves 16-byte words when page_bytes is a multiple of 16 and pool and out
 * are 16-byte aligned, single bytes otherwise. ESHAPE: negative sizes,
 * page_bytes <= 0, more than 2^46 bytes; EALIAS: out overlaps an input.
 */
int trace_gather_pages(const uint8_t* pool, int64_t pool_pages, int64_t page_bytes,
                       const int32_t* page_ids, int64_t n, uint8_t* out, uint32_t* bad_ids,
                       void* stream);

/*
 * Measurement references, not steps of the method: plain streams of 16-byte
 * words with the same access policy as the path's kernels (nontemporal loads
 * and stores, 256 threads of 4 words per workgroup), so a benchmark can time,
 * on the same device and in the same run, the HBM rates its kernels are
 * compared with.
 *
 * trace_stream_copy: dst[i] = src[i]; one stream read, one written.
 * trace_stream_mix:  out[i] = a[i] XOR b[i]; two streams read, one written
 *                    (the mix of the fused guided pass).
 *
 *   src, a, b   in   bytes of device memory, 16-byte aligned
 *   dst, out    out  bytes of device memory, 16-byte aligned, disjoint from the inputs
 *   bytes       a multiple of 16, at most 2^37 (else ESHAPE; one launch of up to 2^23
 *               workgroups)
 */
int trace_stream_copy(const void* src, void* dst, int64_t bytes, void* stream);
int trace_stream_mix(const void* a, const void* b, void* out, int64_t bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* TRACE_FP4_H */
