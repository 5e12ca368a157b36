/*
 * lutq -- weight-only LUT-quantized matrix product on AMD MI355X (gfx950).
 *
 *   y[m, n] = sum_k x[m, k] * T[c[n, k]] * s[n, k / group]
 *
 * c are b-bit codes (b = 2, 3 or 4) that index a 2^b-entry fp16 lookup table
 * T; s is one fp16 scale per `group` consecutive weights along K, or a single
 * scale for the whole tensor (group == 0). The product is fused with the
 * dequantization, so only the packed codes (plus scales) stream from HBM.
 *
 * Sources: "FLUTE: flexible lookup table engine" abstract (weight-only
 * quantization with the dequantization fused into the matmul; offline
 * restructuring of the quantized matrix to cut unpacking work; a vectorized,
 * duplicated lookup table in on-chip memory; 3-bit and non-uniform tables;
 * group size 128, batch below 32); "LogbQuant" abstract (logarithmic tables
 * with an adjustable base; tensor-wise granularity); "BitMoD" abstract
 * (rescaling per-group partial sums).
 *
 * Conventions for every entry point:
 *  - Device pointers are HIP device memory owned by the caller; the library
 *    never frees them. Host pointers are marked "host".
 *  - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *    Work is enqueued on it asynchronously; a return of LUTQ_OK means
 *    "validated and enqueued". Device faults surface at the caller's next
 *    synchronization, as with any HIP launch.
 *  - On any error nothing is enqueued and outputs are untouched.
 *  - fp16 values are passed as raw IEEE binary16 bit patterns (uint16_t).
 *  - No C++ exception crosses this boundary.
 *
 * Scratch memory. A product split along K across workgroups (see
 * lutq_options_t.ksplit; the automatic plan splits narrow matrices with a
 * long K) and the tensor-wise quantizer keep fp32 partial results and
 * arrival counters in a scratch buffer that the library allocates, one per
 * (device, stream), on the first call that needs it. A later call needing
 * more gets a larger buffer; the outgrown one is not freed until
 * lutq_shutdown, so work still queued and HIP graphs captured earlier keep
 * using it safely. No memory is allocated while the stream is being
 * captured: such a call returns LUTQ_ECAPTURE and enqueues nothing, so run
 * each call once eagerly on a stream before capturing it there. A graph
 * holding split launches uses the buffer of the stream it was captured on:
 * do not replay it concurrently with other lutq work on that stream (or
 * with another replay of itself). lutq_matmul_noalloc (below) uses a fixed
 * array instead and never allocates.
 */
#ifndef LUTQ_H
#define LUTQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ------------------------------------------------------ */
enum {
  LUTQ_OK = 0,
  LUTQ_EINVAL = -1,      /* null pointer, negative size, bad option value   */
  LUTQ_EBITS = -2,       /* bits not in {2, 3, 4}                           */
  LUTQ_EGROUP = -3,      /* group not 0 and not a multiple of 128, or K is
                            not a multiple of group (and of 128)            */
  LUTQ_EALIGN = -4,      /* x or packed data not 16-byte aligned, lut not
                            4-byte aligned, or another pointer not 2-byte
                            aligned                                         */
  LUTQ_EMISMATCH = -5,   /* N/K differ from the descriptor; bad magic or
                            layout version                                  */
  LUTQ_ESIZE = -6,       /* destination buffer too small                    */
  LUTQ_EHIP = -7,        /* a HIP runtime call failed (see lutq_last_hip_error) */
  LUTQ_EUNSUPPORTED = -8, /* a size beyond the limits below                 */
  LUTQ_ECAPTURE = -9      /* the call needs new scratch memory while its
                             stream is being captured into a HIP graph
                             (see "Scratch memory" below)                   */
};

/* Limits: 0 <= M; 0 <= N <= 2^24; 0 <= K <= 2^20; N*K <= 2^36 (32 GiB of
 * 4-bit codes). Batches above the per-launch capacity of a path (8 rows for
 * GEMV, 32 for MFMA) are processed in slices; the weights are streamed once
 * per slice. */
#define LUTQ_MAX_N (1 << 24)
#define LUTQ_MAX_K (1 << 20)
#define LUTQ_MAX_NK (1LL << 36)

/* ---- packed weights ------------------------------------------------------
 * Filled by lutq_repack. The layout ("wave-block", version 1) is the offline
 * restructuring of the FLUTE abstract, redesigned for 64-lane wavefronts:
 *
 *   rows are cut into tiles of 16, K into chunks of 128 codes; chunk c of
 *   tile t is one block of 64 lane slots x (4*bits) bytes, stored at byte
 *   offset (t * (K/128) + c) * 256 * bits. Lane slot L = 16*q + r (q = 0..3,
 *   r = 0..15) holds the 32 codes of row 16*t + r at
 *   k = 128*c + 32*j + 8*q + e   (j = 0..3, e = 0..7).
 *   Within a slot, code (j, e) pairs with (j, e^1) into a pair index:
 *     bits=4: 4 dwords; dword j, byte e/2 = code(j,e even) | code(j,e odd)<<4
 *     bits=2: 2 dwords; dword j/2, byte e/2, nibble j%2 =
 *             code(j,e even) | code(j,e odd)<<2
 *     bits=3: 3 dwords (lo0, lo1, hi); the low 2 bits of each code are laid
 *             out as bits=2 in lo0/lo1; the high bits of pair (j, e/2) sit in
 *             byte e/2 of hi at bit offset {4, 6, 0, 2}[j] as
 *             hi(code e even) | hi(code e odd)<<1.
 *   Rows past N in the last tile hold code 0.
 * One 16-row block is one coalesced 64-lane load (1 KiB at bits=4).
 */
#define LUTQ_MAGIC 0x5154554Cu /* "LUTQ" */
#define LUTQ_LAYOUT_VERSION 1u

typedef struct lutq_packed {
  uint32_t magic;   /* LUTQ_MAGIC                                          */
  uint32_t version; /* LUTQ_LAYOUT_VERSION                                 */
  int32_t N, K;     /* weight matrix is N x K (out x in)                   */
  int32_t bits;     /* 2, 3 or 4                                           */
  int32_t group;    /* 0 = one scale per tensor; else a multiple of 128
                       that divides K                                      */
  uint64_t nbytes;  /* bytes used at data (lutq_packed_bytes)              */
  void* data;       /* device, caller-owned, 16-byte aligned               */
} lutq_packed_t;

/* Bytes lutq_repack writes for an N x K matrix: ceil(N/16)*16 * K * bits / 8.
 * Returns 0 for invalid arguments (bits, group, K alignment) and for N == 0
 * or K == 0. */
size_t lutq_packed_bytes(int N, int K, int bits, int group);

/* Offline restructuring (FLUTE abstract: restructure the quantized weight
 * matrix offline so that unpacking needs few bit operations).
 *   codes : device, uint8 [N, K] row-major, one code per byte, 8-byte
 *           aligned (read 8 codes at a time); bits above `bits` are ignored
 *           (masked).
 *   dst   : device, >= lutq_packed_bytes(N, K, bits, group) bytes, 16-byte
 *           aligned; must not overlap `codes`.
 *   out   : host; filled with the descriptor (data = dst) on success.
 * Errors: LUTQ_EINVAL, LUTQ_EBITS, LUTQ_EGROUP, LUTQ_EALIGN, LUTQ_ESIZE,
 * LUTQ_EUNSUPPORTED, LUTQ_EHIP. N == 0 or K == 0 fills the descriptor
 * (nbytes = 0) and enqueues nothing. */
int lutq_repack(const uint8_t* codes, int N, int K, int bits, int group,
                void* dst, size_t dst_bytes, lutq_packed_t* out, void* stream);

/* Inverse of lutq_repack, for tests: writes uint8 codes [N, K] (device,
 * row-major) from the packed layout. Errors as lutq_repack. */
int lutq_unpack(const lutq_packed_t* packed, uint8_t* codes_out, void* stream);

/* The fused LUT-dequantize + matmul (FLUTE abstract; per-group partial sums
 * rescaled once per group as in the BitMoD abstract):
 *   x      : device, fp16 [M, K] row-major, 16-byte aligned.
 *   packed : host descriptor from lutq_repack (its data stays on device).
 *   lut    : device, fp16 [2^bits], 4-byte aligned.
 *   scales : device, fp16 [N, K/group] row-major, or [1] when group == 0.
 *   y      : device, fp16 [M, N] row-major (output; written, never read).
 * Accumulation is fp32; y is rounded to nearest-even fp16. The table values
 * are used unscaled inside a group and each group's fp32 partial sum is
 * multiplied by its scale. Results are deterministic (no float atomics).
 * M == 0 or N == 0: nothing to do (LUTQ_OK). K == 0: y is set to zero.
 * Errors: LUTQ_EINVAL, LUTQ_EMISMATCH, LUTQ_EALIGN, LUTQ_EUNSUPPORTED,
 * LUTQ_ECAPTURE, LUTQ_EHIP. Calls may run concurrently on different streams. */
int lutq_matmul(const uint16_t* x, const lutq_packed_t* packed, const uint16_t* lut,
                const uint16_t* scales, uint16_t* y, int M, int N, int K, void* stream);

/* Path selection for lutq_matmul_ex. */
enum {
  LUTQ_PATH_AUTO = 0, /* by M: GEMV for small batches, MFMA above            */
  LUTQ_PATH_GEMV = 1, /* VALU dot2 path (any M; slices of 8 rows)            */
  LUTQ_PATH_MFMA = 2  /* fp16 MFMA path (any M; slices of 32 rows)           */
};

typedef struct lutq_options {
  int32_t path;   /* LUTQ_PATH_*                                              */
  int32_t ksplit; /* workgroups per row block along K; 0 = automatic.
                     Clamped to the number of 128-code chunks.               */
  int32_t tiles;  /* 16-row output tiles per wave (the workgroup covers
                     16 * tiles rows); 0 = automatic. Needs an explicit
                     path: GEMV takes 1 or 2, MFMA 1, 2, 4, 7 or 8; anything
                     else gives LUTQ_EINVAL.                                 */
  int32_t dtype;  /* activations x and output y: LUTQ_DTYPE_F16 (0) or
                     LUTQ_DTYPE_BF16 (1); bf16 works with plain tables
                     (lutq_matmul_ex, lutq_matmul_multi without zero
                     points) and gives LUTQ_EUNSUPPORTED with zero points,
                     data types or binary coding.                            */
  int32_t reserved[4]; /* must be zero                                        */
} lutq_options_t;

/* Activation dtypes (lutq_options_t.dtype). bf16 activations are converted
 * on chip per (batch row, 128-weight chunk): scaled by a power of two that
 * puts the chunk's largest magnitude in [2^14, 2^15), every bf16 value
 * within 2^31 of it is exactly an fp16 value, so the fp16 arithmetic runs
 * unchanged and the chunk's partial sums are scaled back exactly. Values
 * smaller than 2^-31 of their chunk's largest lose bits. y is bf16, rounded
 * to nearest even from the fp32 result. */
enum { LUTQ_DTYPE_F16 = 0, LUTQ_DTYPE_BF16 = 1 };

/* lutq_matmul with explicit options (host pointer; NULL = automatic). */
int lutq_matmul_ex(const uint16_t* x, const lutq_packed_t* packed, const uint16_t* lut,
                   const uint16_t* scales, uint16_t* y, int M, int N, int K,
                   const lutq_options_t* opts, void* stream);

/* lutq_matmul_ex for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * The split-K partial sums and arrival counters live in a fixed array in the
 * library's device image (LUTQ_NOALLOC_SCRATCH_BYTES per GPU, each GPU the
 * library runs on holding its own copy until the process ends) instead of
 * the per-stream buffer lutq_matmul_ex allocates; the call allocates no
 * device memory at all. Arguments, options and numerics are those of
 * lutq_matmul_ex, and the result is bit-identical to lutq_matmul_ex with the
 * same options. A call whose K split needs more partial sums than the array
 * holds (only an explicit large ksplit does: the automatic plan needs at
 * most 2 MiB) returns LUTQ_EUNSUPPORTED and enqueues nothing.
 * Every call on one GPU shares that GPU's array: calls that overlap in time
 * on one GPU (on different streams, or a graph replayed alongside other
 * lutq_matmul_noalloc work) race and give wrong results, so serialize them.
 * The array is zero when the library is loaded; each launch leaves its
 * counters at zero, and the first call on a device clears them once more
 * on its stream. */
#define LUTQ_NOALLOC_SCRATCH_BYTES (8u << 20)
int lutq_matmul_noalloc(const uint16_t* x, const lutq_packed_t* packed, const uint16_t* lut,
                        const uint16_t* scales, uint16_t* y, int M, int N, int K,
                        const lutq_options_t* opts, void* stream);

/* The options lutq_matmul_ex resolves for this call (host-side heuristic
 * only, no device work): `req` (host, may be NULL = all automatic) is
 * validated as in lutq_matmul_ex and its automatic fields are filled in;
 * the result goes to `out` (host). With several batch slices the shape is
 * the one of the first slice, and all slices use it. */
int lutq_plan(int M, int N, int K, int bits, const lutq_options_t* req, lutq_options_t* out);

/* ---- fused launch of several matrices ---------------------------------------
 * The products of one decoder layer that read the same activations (the q,
 * k and v projections, or gate and up) in one launch per batch slice:
 *     y_i = x . W_i^T,   i < count <= LUTQ_MAX_FUSED.
 * Narrow matrices (k, v at batch 1) cannot fill the device alone; sharing a
 * launch also saves the launches themselves. Every matrix has the same K,
 * bits and group; each has its own packed codes, table, scales and output,
 * with the layouts, alignment and numerics of lutq_matmul. Workgroups never
 * span two matrices, so each y_i is bit-identical to what lutq_matmul_ex
 * gives for that matrix alone with the same path, shape and K split. The
 * plan (lutq_plan with N = the sum of the widths rounded up to 16) is made
 * for the whole launch; `opts` as lutq_matmul_ex (NULL = automatic).
 *   items : host array of `count` entries (read during the call only).
 * A matrix with N == 0 is skipped. Errors as lutq_matmul_ex, plus
 * LUTQ_EINVAL for count outside [1, LUTQ_MAX_FUSED] or a NULL items, and
 * LUTQ_EMISMATCH for a matrix whose K, bits or group differ. */
#define LUTQ_MAX_FUSED 4
typedef struct lutq_matmul_item {
  const lutq_packed_t* packed; /* host descriptor                           */
  const uint16_t* lut;         /* device, fp16 [2^bits]                      */
  const uint16_t* scales;      /* device, fp16 [N, K/group] or [1]           */
  const uint16_t* zeros;       /* device, fp16 [N, K/group] zero points as
                                  lutq_matmul_zp, or NULL (none)             */
  uint16_t* y;                 /* device, fp16 [M, N] (output)               */
} lutq_matmul_item_t;
int lutq_matmul_multi(const uint16_t* x, const lutq_matmul_item_t* items, int count, int M, int K,
                      const lutq_options_t* opts, void* stream);

/* ---- per-group zero points ---------------------------------------------------
 * Asymmetric quantization with a zero point per group (LogbQuant abstract:
 * asymmetric linear quantization; BitMoD abstract: quantization parameters
 * and partial-sum rescaling per group):
 *     W_hat[n, k] = s[n, g] * (T[c[n, k]] - z[n, g]),   g = k / group,
 *     y = x . W_hat^T.
 *   zeros : device, fp16 [N, K/group] row-major (the layout of the scales),
 *           2-byte aligned; group must be > 0 (LUTQ_EGROUP otherwise).
 * Computed as s * (sum_k x T[c] - z * sum_k x) per group: the activation sums
 * come once per group for all output rows, so the zero points cost their
 * own loads (0.125 bit per weight at group 128) and one multiply-add per
 * group and output. Other arguments, numerics and errors as lutq_matmul_ex;
 * NULL zeros with N * K > 0 is LUTQ_EINVAL. */
int lutq_matmul_zp(const uint16_t* x, const lutq_packed_t* packed, const uint16_t* lut,
                   const uint16_t* scales, const uint16_t* zeros, uint16_t* y, int M, int N, int K,
                   const lutq_options_t* opts, void* stream);

/* ---- per-group data types ----------------------------------------------------
 * A few tables, one chosen per group (BitMoD abstract: the data type is
 * chosen per group of weights):
 *     W_hat[n, k] = s[n, g] * (T_{types[n, g]}[c[n, k]] - z[n, g]),  g = k / group,
 * with z = 0 when `zeros` is NULL (zero points as lutq_matmul_zp).
 *   luts  : device, fp16 [ntypes][2^bits] (tables one after another),
 *           4-byte aligned; 1 <= ntypes <= LUTQ_MAX_TYPES.
 *   types : device, uint8 [N, K/group] row-major type ids. An id is taken
 *           modulo LUTQ_MAX_TYPES; one (mod 4) at or above ntypes reads table 0.
 * group must be > 0 (LUTQ_EGROUP otherwise). The tables share the on-chip
 * duplicated table (16 copies each instead of 64), and the ids are fetched
 * with the scales (0.0625 bit per weight at group 128). Other arguments,
 * numerics and errors as lutq_matmul_ex; LUTQ_EINVAL for ntypes outside
 * [1, LUTQ_MAX_TYPES] or NULL types with N * K > 0. */
#define LUTQ_MAX_TYPES 4
int lutq_matmul_typed(const uint16_t* x, const lutq_packed_t* packed, const uint16_t* luts,
                      int ntypes, const uint8_t* types, const uint16_t* scales,
                      const uint16_t* zeros, uint16_t* y, int M, int N, int K,
                      const lutq_options_t* opts, void* stream);

/* ---- binary-coded weights ----------------------------------------------------
 * Binary-coding quantization (AlphaTuning abstract: the weights factorize
 * into binary parameters and separate scaling factors): q = bits binary
 * planes, bit p of the q-bit code c[n, k] being plane p, and one fp16
 * factor per plane, row and group:
 *     W_hat[n, k] = sum_p alphas[p][n][g] * (2 bit_p(c[n, k]) - 1),  g = k / group,
 * i.e. a 2^q-entry table per row and group. Computed as
 * sum_p alpha_p (2 S_p - X) per group, with S_p = sum_k x bit_p(c) and
 * X = sum_k x (as lutq_matmul_zp).
 *   packed : lutq_repack of the codes with bits = q (2, 3 or 4), group > 0
 *            (LUTQ_EGROUP otherwise).
 *   alphas : device, fp16 [q][N][K/group] (plane-major), 2-byte aligned.
 * The GEMV path reads each pair's plane bits from an on-chip table; the
 * MFMA path decodes them in registers. Other arguments, options, numerics
 * and errors as lutq_matmul_ex. */
int lutq_matmul_bcq(const uint16_t* x, const lutq_packed_t* packed, const uint16_t* alphas,
                    uint16_t* y, int M, int N, int K, const lutq_options_t* opts, void* stream);

/* ---- quantizer ------------------------------------------------------------
 * Round-to-nearest onto a lookup table: the step that produces the codes and
 * scales lutq_repack and lutq_matmul consume ("PTQ-damage" abstract:
 * round-to-nearest at group-128 granularity; FLUTE abstract: arbitrary,
 * non-uniform tables; LogbQuant abstract: tensor-wise scales and log tables
 * with an adjustable base).
 *
 *   scale (fp64, then rounded once to fp16, nearest even; a zero scale
 *   becomes 1, one above 65504 is clamped to 65504):
 *     LUTQ_RULE_ABSMAX: max|w| / max|T|
 *     LUTQ_RULE_RANGE : max(max(w) / max(T), min(w) / min(T)), for tables
 *                       with min(T) < 0 < max(T); on the uniform table
 *                       T[i] = i - z this is asymmetric INT round-to-nearest
 *   code: the entry nearest to w / s (fp64 quotient of the fp32 weight and
 *         the fp16 scale, exact comparison), an exact tie to the lower index.
 * Table entries must be distinct (results are unspecified otherwise).
 */
enum { LUTQ_RULE_ABSMAX = 0, LUTQ_RULE_RANGE = 1 };

/*   w      : device, fp32 [N, K] row-major, finite, 16-byte aligned.
 *   lut    : device, fp16 [2^bits], 2-byte aligned.
 *   codes  : device, uint8 [N, K] out (one code per byte, the lutq_repack
 *            input), 4-byte aligned.
 *   scales : device, fp16 out: [N, K/group] row-major, or [1] (group == 0).
 * group: 0 or a multiple of 128 that divides K (as lutq_repack).
 * Errors: LUTQ_EINVAL, LUTQ_EBITS, LUTQ_EGROUP, LUTQ_EALIGN, LUTQ_EUNSUPPORTED,
 * LUTQ_EHIP. N == 0 or K == 0: nothing to do. Work is enqueued on `stream`;
 * tensor-wise scales use the library's per-stream scratch buffer. */
int lutq_quantize(const float* w, const uint16_t* lut, int bits, int N, int K, int group,
                  int rule, uint8_t* codes, uint16_t* scales, void* stream);

/* The weight error of that quantization, sum over all weights of
 * (w - s * T[c])^2 in fp64, without writing codes or scales; summed in a
 * fixed order, so repeated calls agree bit for bit. *err is host memory;
 * the call waits for the stream. Errors as lutq_quantize. */
int lutq_quant_error(const float* w, const uint16_t* lut, int bits, int N, int K, int group,
                     int rule, double* err, void* stream);

/* LogbQuant base search: for each candidate base (host array, each > 1),
 * the table T[s, k] = (-1)^s * base^-k (code = sign bit on top of the
 * bits - 1 exponent bits, values rounded to fp16), absmax scales, and its
 * weight error as lutq_quant_error. Writes the index of the smallest error to
 * *best (host; the first one on equal errors) and every error to errors
 * (host, nbases entries, may be NULL). Waits for the stream.
 * Errors as lutq_quantize, plus LUTQ_EINVAL for nbases < 1 or a base <= 1
 * or one whose table repeats an fp16 value. */
int lutq_log_base_search(const float* w, int bits, int N, int K, int group, const double* bases,
                         int nbases, int* best, double* errors, void* stream);

/* The quantizer entry points for 16-bit weights as models ship them: `w` is
 * fp32 (LUTQ_WEIGHT_F32, 16-byte aligned), fp16 (LUTQ_WEIGHT_F16) or bf16
 * (LUTQ_WEIGHT_BF16), both 8-byte aligned. 16-bit weights are widened to
 * fp32 exactly, so the results are those of lutq_quantize on the same
 * values. Otherwise as lutq_quantize, lutq_quant_error and
 * lutq_log_base_search; LUTQ_EINVAL for another wdtype. */
enum { LUTQ_WEIGHT_F32 = 0, LUTQ_WEIGHT_F16 = 1, LUTQ_WEIGHT_BF16 = 2 };
int lutq_quantize_ex(const void* w, int wdtype, const uint16_t* lut, int bits, int N, int K,
                     int group, int rule, uint8_t* codes, uint16_t* scales, void* stream);
int lutq_quant_error_ex(const void* w, int wdtype, const uint16_t* lut, int bits, int N, int K,
                        int group, int rule, double* err, void* stream);
int lutq_log_base_search_ex(const void* w, int wdtype, int bits, int N, int K, int group,
                            const double* bases, int nbases, int* best, double* errors,
                            void* stream);

/* Table tuning on the weight error (FLUTE abstract: NormalFloat tables;
 * TurboQuant/EDEN note: the Lloyd-Max algorithm), no data needed: the scales
 * come from the initial table under `rule` and stay fixed; each iteration
 * codes the weights by round-to-nearest and replaces every used entry by the
 * fp16 (nearest even) value of sum(w s) / sum(s^2) over the weights holding
 * that code (fp64 sums in a fixed order); an unused entry keeps its value.
 * An update that would repeat an fp16 value stops the iterations.
 *   w, wdtype, bits, N, K, group, rule : as lutq_quantize_ex.
 *   lut     : device, fp16 [2^bits]: the initial table in, the tuned one out.
 *   iters   : at most this many updates (>= 0).
 *   scales  : device, fp16, the fixed scales out (layout of lutq_quantize),
 *             2-byte aligned, or NULL.
 *   errors  : host, iters + 1 entries, or NULL: errors[k] is the weight
 *             error of the k-th table, for k = 0 .. *updates.
 *   updates : host, the number of updates made.
 * Waits for the stream. Errors as lutq_quantize_ex, plus LUTQ_EINVAL for a
 * NULL updates or iters < 0. */
int lutq_tune_table(const void* w, int wdtype, uint16_t* lut, int bits, int N, int K, int group,
                    int rule, int iters, uint16_t* scales, double* errors, int* updates,
                    void* stream);

/* Static string for a status code. */
const char* lutq_strerror(int status);

/* The last HIP error code seen by this thread (hipError_t as int). */
int lutq_last_hip_error(void);

/* Frees the library's scratch buffers (per device and stream, including
 * outgrown ones kept for earlier graphs). Call only when no lutq work is in
 * flight and no graph that used them will be replayed again. */
void lutq_shutdown(void);

#ifdef __cplusplus
}
#endif

#endif /* LUTQ_H */
