/*
 * ck_int8.h -- C ABI of the MI355X (gfx950) INT8 linear layer.
 *
 * The layer is the one the comfy-kitchen pages keep returning to:
 *   1. per-row (or tensor-wide) activation quantisation, bf16 -> int8 codes
 *      plus an fp32 scale (issue #278 "int8_linear silently falls back ...",
 *      section "Two separate problems", item 2, names quantize_int8_rowwise;
 *      issue #280 "INT8 linears on sm_121 ...", Summary, names tensor-wide
 *      scales);
 *   2. an int8 x int8 product with an exact int32 accumulator over K
 *      (issue #280, sections "Kernel used" and "Exactness");
 *   3. an fp32 epilogue out = acc * x_scale[m] * w_scale[n] (+ bias[n]),
 *      evaluated left to right, rounded once to the output type: bf16, or
 *      the fp16 and fp32 outputs that the exactness audit also covers (issue
 *      #280, sections "Kernel used" and "Exactness");
 * with 64-bit row/column offsets throughout, so that outputs and inputs past
 * 2^31 elements are addressed correctly (issue #136 "INT8 GEMM kernels index
 * the output in int32 ...", sections "Summary" and "Suggested fix").
 *
 * Conventions shared by every entry point:
 *   - All tensor pointers are DEVICE pointers on the current HIP device,
 *     owned by the caller; the library never frees or retains them.
 *   - bf16 values travel as their uint16_t bit patterns.
 *   - Matrices are row-major with an explicit leading dimension (elements
 *     between the starts of consecutive rows).
 *   - Calls are asynchronous: they validate, enqueue kernels on `stream`
 *     (0 = the null stream) and return without synchronising.  Results are
 *     ready when the stream has reached that point.
 *   - No call allocates device memory (no hipMalloc is reachable from any
 *     entry point).  State kept between calls:
 *       * device counters.  The persistent GEMMs (tile 13, the heuristic's
 *         choice for large shapes, and the dequant path above 256 tiles)
 *         and the tensor-wide quantisation use a 64-byte slot of counters
 *         per (device, stream) pair.  The slots live in a 64 KiB
 *         file-scope device array of this library (1024 slots), which the
 *         HIP runtime places on each device with the library's code and
 *         which lasts until the process ends.  A slot is zeroed by a small
 *         kernel on its stream before its first use.  The GEMMs leave their
 *         tile counters at zero when they finish (the last block to finish
 *         clears them); the quantisation keeps its amax in one of two
 *         cells and clears the other for its next call.  Calls on one
 *         stream use a slot in stream order, calls on different streams
 *         never share one.  Under graph capture, or past 1024 streams on a
 *         device, no slot is used: the one-block-per-tile kernels run, and
 *         the quantisation uses scale[0] as its amax cell (four launches
 *         instead of two).
 *       * host bookkeeping: which slot belongs to which (device, stream),
 *         and which amax cell a stream's next tensor-wide call uses.
 *       * optional host settings: the measured tile table, the forced tile
 *         and the path-log switch (see the end of this header).
 *   - Arguments are validated on the host before any HIP call; a failed
 *     check launches nothing.  The detail of the last failure on the
 *     calling thread is available from ck_last_error().
 *   - There is no fallback path: a case the kernels do not handle returns
 *     CK_ERR_UNSUPPORTED, a non-gfx950 device returns CK_ERR_WRONG_ARCH.
 *
 * Status codes:
 *   CK_OK               success (also for empty problems: nothing launched)
 *   CK_ERR_INVALID_ARG  a NULL required pointer, a negative size, a leading
 *                       dimension smaller than the row length, a bad mode
 *   CK_ERR_UNSUPPORTED  valid but outside what the kernels handle: GEMM
 *                       operand rows (q, w) not 16-byte aligned, a
 *                       misaligned scale, bias or output, K > CK_MAX_K
 *   CK_ERR_HIP          a HIP runtime call or launch failed (ck_last_error
 *                       holds HIP's message)
 *   CK_ERR_WRONG_ARCH   the current device is not gfx950
 */
#ifndef CK_INT8_H
#define CK_INT8_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    CK_OK = 0,
    CK_ERR_INVALID_ARG = 1,
    CK_ERR_UNSUPPORTED = 2,
    CK_ERR_HIP = 3,
    CK_ERR_WRONG_ARCH = 4
} ck_status;

/* How a scale vector is indexed: one value for the whole tensor, or one per
 * row of x (x_scale[m]) / per output column (w_scale[n]). */
typedef enum {
    CK_SCALE_TENSOR = 0,
    CK_SCALE_ROW = 1
} ck_scale_mode;

/* Largest K for which |acc| <= K * 127 * 128 still fits in int32. */
#define CK_MAX_K 132104

/* Element type of the linear layer's output.  The bias, when given, has the
 * same type (fp32 for CK_OUT_FP32); bf16 and fp16 travel as uint16_t bits. */
typedef enum {
    CK_OUT_BF16 = 0,
    CK_OUT_FP16 = 1,
    CK_OUT_FP32 = 2
} ck_out_dtype;

/* Number of GEMM tile configurations compiled into the library. */
#define CK_NUM_TILES 14

/*
 * Step 1: quantise bf16 activations to int8 codes.
 *
 * Follows issue #278, section "Two separate problems", item 2
 * (quantize_int8_rowwise) for CK_SCALE_ROW, and the tensor-wide scales of
 * issue #280 (Summary; "Exactness") for CK_SCALE_TENSOR.
 *
 *   amax  = max |x| over the row (ROW) or over all m*k elements (TENSOR)
 *   s     = amax / 127                     (fp32, correctly rounded)
 *   q     = clamp(rint(x / s), -127, 127)  (fp32 division, ties to even;
 *                                           s == 0 gives q == 0)
 *
 * x      [in]  bf16 bits, [m, ldx], row-major; ldx >= k, 2-byte aligned.
 * q      [out] int8 codes, [m, ldq]; ldq >= k.  Bytes of a q row past k are
 *              left untouched.  (16-byte aligned x rows with ldx % 8 == 0
 *              and 8-byte aligned q rows with ldq % 8 == 0 take the vector
 *              kernels; other layouts a slower element-wise kernel.)
 * scale  [out] fp32, m values (ROW) or 1 value (TENSOR).  In TENSOR mode
 *              scale[0] is also used as the reduction cell while the call
 *              runs, so it must not alias x or q.
 * m, k   sizes; m == 0 (or k == 0) is allowed: codes are empty, scales 0.
 * Inputs must be finite.
 */
ck_status ck_quantize_int8_rowwise(const uint16_t* x, int64_t m, int64_t k,
                                   int64_t ldx, int8_t* q, int64_t ldq,
                                   float* scale, ck_scale_mode mode,
                                   hipStream_t stream);

/*
 * Step 0 + step 1 for ConvRot checkpoints: quantise the rotated activation
 * x H (issue #278, "Suggested fix": the weight is stored as W H^T and the
 * activation is rotated online, so the product runs in the rotated basis).
 *
 * H is block diagonal: k / block copies of the Sylvester-Hadamard matrix of
 * order `block` scaled by r = fl(1/sqrt(block)).  Per block the rotation is
 * computed in fp32 from the exact values of x: butterfly stages h = 1, 2,
 * 4, ..., block/2 (elements i and i+h with bit h of i clear become u + v and
 * u - v), then every value times r, each operation one fp32 rounding.  The
 * scale and codes then follow the formula of ck_quantize_int8_rowwise on
 * those fp32 values (amax of |x_rot| per row, or over the whole tensor).
 *
 * block  power of two in [1, 512]; k % block == 0 (else CK_ERR_INVALID_ARG).
 * x, q   as for ck_quantize_int8_rowwise, but this entry needs k % 8 == 0,
 *        ldx % 8 == 0 with a 16-byte aligned x, and ldq % 8 == 0 with an
 *        8-byte aligned q (else CK_ERR_UNSUPPORTED).
 * scale  as for ck_quantize_int8_rowwise.
 */
ck_status ck_quantize_int8_rotated(const uint16_t* x, int64_t m, int64_t k, int64_t ldx,
                                   int64_t block, int8_t* q, int64_t ldq, float* scale,
                                   ck_scale_mode mode, hipStream_t stream);

/*
 * Steps 2 and 3: out = bf16( ((fp32(acc) * xs) * ws) + fp32(bias[n]) ),
 * acc[i, j] = sum_t q[i, t] * w[j, t] exact in int32, the epilogue in fp32
 * with one rounding per operation (no fused multiply-add), bf16 round to
 * nearest even.  Follows issue #280, sections "Kernel used" and
 * "Exactness"; 64-bit offsets per issue #136, "Suggested fix".  The int32
 * accumulator never leaves registers.
 *
 * q        [in]  int8 codes [m, ldq]; ldq >= k, ldq % 16 == 0, 16-B aligned.
 * x_scale  [in]  fp32, m values (x_mode ROW) or 1 value (x_mode TENSOR).
 * w        [in]  int8 weight [n, ldw] (row j is output feature j, K
 *                contiguous); ldw >= k, ldw % 16 == 0, 16-B aligned.
 *                K needs no alignment: rows whose k is not a multiple of 16
 *                are stored padded (ld a multiple of 16), and the bytes of a
 *                row from k up to the next multiple of 16 are read but
 *                treated as zero, which leaves the integer sums exact.
 * w_scale  [in]  fp32, n values (w_mode ROW) or 1 value (w_mode TENSOR).
 * bias     [in]  bf16 bits [n], or NULL for no bias.
 * out      [out] bf16 bits [m, ldo]; ldo >= n.
 * m, n, k  sizes; m == 0 or n == 0 is a no-op; k == 0 gives out = bias
 *          (or +0); k <= CK_MAX_K.
 */
ck_status ck_int8_linear(const int8_t* q, int64_t ldq, const float* x_scale,
                         ck_scale_mode x_mode, const int8_t* w, int64_t ldw,
                         const float* w_scale, ck_scale_mode w_mode,
                         const uint16_t* bias, uint16_t* out, int64_t ldo,
                         int64_t m, int64_t n, int64_t k, hipStream_t stream);

/*
 * ck_int8_linear with an explicit tile configuration, for sweeps.
 * tile in [0, CK_NUM_TILES) picks the compiled configuration (-1 = the
 * built-in heuristic): ids 0..3 are block shapes 256x256, 256x128,
 * 128x128 and 64x64 (4 waves) fed by direct global->LDS loads in 64-byte K
 * stages (a K tail shorter than a stage is loaded through registers); ids
 * 4..7 are the same shapes on a register-staged main loop; ids 8..12 are
 * 256x256 blocks of 8 waves (8, 9: 128x64 / 64x128 per wave; 10, 11: refill
 * loads spread over the products, 4 or 8 waves; 12: as 11 with 128-byte K
 * stages).  Id 13 is tile 12 run persistently (one block per compute unit
 * walks several tiles, overlapping a tile's output stores with the next
 * tile's first loads) for bf16 / fp16 outputs (and the int32 accumulators
 * of ck_int8_gemm_i32) when k is a multiple of 128 and there are more tiles
 * than compute units; otherwise it runs as tile 12.  group_m >= 1 is the
 * number of row tiles that a launch-order group spans (0 = the heuristic's
 * choice; a group larger than the shape's row tiles is cut to them).  An
 * unknown tile id returns CK_ERR_INVALID_ARG; a valid one is never replaced
 * by another.
 */
ck_status ck_int8_linear_tiled(const int8_t* q, int64_t ldq, const float* x_scale,
                               ck_scale_mode x_mode, const int8_t* w, int64_t ldw,
                               const float* w_scale, ck_scale_mode w_mode,
                               const uint16_t* bias, uint16_t* out, int64_t ldo,
                               int64_t m, int64_t n, int64_t k, int tile,
                               int group_m, hipStream_t stream);

/*
 * ck_int8_linear_tiled with the output type as a parameter: out (and bias)
 * are bf16 or fp16 bits (uint16_t) or fp32, per out_dtype; ldo counts
 * elements.  The epilogue is the same fp32 chain; the final rounding is to
 * bf16 or fp16 (nearest, ties to even; fp16 overflows to infinity from
 * 65520 on), or none for fp32.  Issue #280, "Exactness" (the audit's fp16 /
 * fp32 outputs).  A bad out_dtype returns CK_ERR_INVALID_ARG; out and bias
 * must be aligned to their element size.
 */
ck_status ck_int8_linear_ex(const int8_t* q, int64_t ldq, const float* x_scale,
                            ck_scale_mode x_mode, const int8_t* w, int64_t ldw,
                            const float* w_scale, ck_scale_mode w_mode, const void* bias,
                            void* out, int64_t ldo, ck_out_dtype out_dtype, int64_t m,
                            int64_t n, int64_t k, int tile, int group_m, hipStream_t stream);

/*
 * The whole layer from bf16 activations: ck_quantize_int8_rowwise(x -> q,
 * x_scale, x_mode) followed by ck_int8_linear_ex on those codes, with the
 * same results in every buffer (q, x_scale and out).  Issue #280,
 * "Kernel used" (activations quantised per row, or per tensor, then the
 * int8 GEMM with the dequant epilogue); the pages' int8_linear(x, w, ws).
 * With few rows the two steps run as one kernel: every 64 x 64 output
 * block quantises its own (at most 64) rows of x into LDS with the
 * quantisation kernel's arithmetic and multiplies them there while the
 * weight streams in; the blocks of the first 64 columns also write q and
 * x_scale.  This saves the quantisation's launch, which for a row or two
 * costs more than its work.
 *
 * x        [in]  bf16 bits [m, ldx], ldx >= k.
 * q        [out] int8 codes [m, ldq] (a workspace the caller owns; as for
 *                ck_int8_linear: ldq >= k, ldq % 16 == 0, 16-B aligned).
 * x_scale  [out] fp32, m values (ROW) or 1 value (TENSOR; also the
 *                reduction cell of the two-kernel path, so it must not
 *                alias x or q).
 * w, w_scale, w_mode, bias, out, ldo, out_dtype, m, n, k: as
 *                ck_int8_linear_ex.
 * fused    -1: the library picks (one kernel when m <= 2 and the layout
 *              allows it, else two: with more rows every block quantising
 *              them again costs more than the launch it saves);
 *           0: always the two kernels;
 *           1: one kernel, or CK_ERR_UNSUPPORTED when it does not apply:
 *              it needs m, n >= 1, k a positive multiple of 64, x rows
 *              16-byte aligned (x 16-B aligned, ldx % 8 == 0), per-row x
 *              scales or m <= 64, and the block's LDS to fit 160 KiB:
 *              17,408 + 128 r (rounded up to 256) + r k <= 163,840 bytes,
 *              r = min(m, 64) (the codes of a block's rows stay in LDS
 *              beside 16 KiB of weight stages).
 * Every argument of both steps is checked before anything is launched.
 */
ck_status ck_int8_layer(const uint16_t* x, int64_t ldx, int8_t* q, int64_t ldq, float* x_scale,
                        ck_scale_mode x_mode, const int8_t* w, int64_t ldw, const float* w_scale,
                        ck_scale_mode w_mode, const void* bias, void* out, int64_t ldo,
                        ck_out_dtype out_dtype, int64_t m, int64_t n, int64_t k, int fused,
                        hipStream_t stream);

/*
 * ck_int8_linear_ex for callers that cannot allocate device memory or keep
 * per-stream state: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  Same arguments, kernels and results as
 * ck_int8_linear_ex.  Where the persistent kernel runs (tile 13, k a
 * positive multiple of 128, more tiles than compute units) its ten 32-bit
 * tile-claim counters come from one 256-byte array per device that every
 * call of this entry point shares (a file-scope device array of the
 * library, placed on each device with the library's code; nothing is
 * allocated), instead of the stream's counter slot: each call first
 * zeroes them with a one-block kernel on `stream`, then launches the GEMM,
 * so the call may also be captured into a graph (the persistent kernel then
 * runs in the graph too, unlike ck_int8_linear_ex under capture).  The
 * array keeps the last call's contents.  Calls whose kernels overlap on one
 * device (on several streams, or graph replays running at the same time)
 * race on the counters and give wrong results: order them.  The first call
 * on a device looks up that device's copy of the array
 * (hipGetSymbolAddress).  Shapes with more than 2^31 - 1 tiles, which the
 * counters cannot count, return CK_ERR_UNSUPPORTED, as for every GEMM entry.
 */
ck_status ck_int8_linear_noalloc(const int8_t* q, int64_t ldq, const float* x_scale,
                                 ck_scale_mode x_mode, const int8_t* w, int64_t ldw,
                                 const float* w_scale, ck_scale_mode w_mode, const void* bias,
                                 void* out, int64_t ldo, ck_out_dtype out_dtype, int64_t m,
                                 int64_t n, int64_t k, int tile, int group_m, hipStream_t stream);

/*
 * Dequant-on-the-fly path (W8A16): out = round_out(S + bias[j]) with
 *   S = sum_t x[i, t] * wdq[j, t],  wdq[j, t] = bf16(fp32(w[j, t]) * w_scale[j])
 * on the bf16 matrix cores, x not quantised, W read as int8 (issue #278,
 * "Suggested fix": dequantise the int8 weight to the 16-bit compute type on
 * the fly).  Products are exact in fp32; the sum is accumulated in fp32 by
 * the hardware in an order of its own, so results are not bit-reproducible
 * against a sequential sum: |error of S| <= k * 2^-24 * sum_t |x * wdq|.
 *
 * x        [in]  bf16 bits [m, ldx]; ldx >= k, ldx % 8 == 0, 16-B aligned.
 * w        [in]  int8 [n, ldw]; ldw >= k, ldw % 16 == 0, 16-B aligned (bytes
 *                from k up to the next multiple of 16 are read and ignored;
 *                any k is allowed).
 * w_scale  [in]  fp32, n values (w_mode ROW) or 1 value (TENSOR).
 * bias, out, ldo, out_dtype  as for ck_int8_linear_ex.
 * Up to 64 rows run a kernel of their own for streaming W (32 columns per
 * block, K split over its waves, the partial sums added in a fixed order);
 * more rows run 64 x 64 or 256 x 256 blocks.
 * Errors as for ck_int8_linear_ex; rows longer than 32-bit offsets allow
 * give CK_ERR_UNSUPPORTED (up to 64 rows: 128 * ldx or 32 * ldw >= 2^31;
 * more: 256 * 2 * ldx or 256 * ldw >= 2^31).
 */
ck_status ck_int8_linear_dequant(const uint16_t* x, int64_t ldx, const int8_t* w, int64_t ldw,
                                 const float* w_scale, ck_scale_mode w_mode, const void* bias,
                                 void* out, int64_t ldo, ck_out_dtype out_dtype, int64_t m,
                                 int64_t n, int64_t k, hipStream_t stream);

/*
 * Step 2 alone: acc[i, j] = sum_t q[i, t] * w[j, t] written as int32
 * [m, ldacc] (ldacc >= n, ldacc % 4 == 0, 16-B aligned).  The tile is
 * chosen as for ck_int8_linear (tile -1: forced tile, table, heuristic) and
 * the same kernel runs with an int32 epilogue that stores the raw
 * accumulators: for tile 13 with k a positive multiple of 128 and more
 * tiles than compute units, the persistent kernel with its tile claiming
 * and main loop (the kernel that ck_int8_linear runs there for bf16 and
 * fp16 outputs); otherwise the one-block-per-tile kernel of the tile.
 * Exists to check accumulators bit-exactly (issue #280, "Exactness": the
 * int32 accumulation is exact); the int32 matrix is written to HBM only
 * here.
 */
ck_status ck_int8_gemm_i32(const int8_t* q, int64_t ldq, const int8_t* w,
                           int64_t ldw, int32_t* acc, int64_t ldacc, int64_t m,
                           int64_t n, int64_t k, int tile, hipStream_t stream);

/*
 * The tile configuration and launch-order group the heuristic picks for a
 * shape (host only, no HIP call).  Writes the tile id, its block tile
 * (bm x bn) and the group size.  Any output pointer may be NULL.
 */
ck_status ck_int8_select_tile(int64_t m, int64_t n, int64_t k, int* tile,
                              int* bm, int* bn, int* group_m);

/* Static description of compiled tile `tile`: block rows, block columns,
 * threads per block.  CK_ERR_INVALID_ARG for an unknown id. */
ck_status ck_int8_tile_info(int tile, int* bm, int* bn, int* threads);

/*
 * Measured tile table, forced tile and path log (PR #142 "sm86 INT8 GEMM
 * tuning: measured tile heuristic, per-shape cfg cache, and path logging",
 * section "What this does", items 1-3).  Host-side, process-wide,
 * thread-safe; no HIP call.
 *
 * How a GEMM call picks its tile (ck_int8_linear*, ck_int8_gemm_i32,
 * ck_int8_select_tile): an explicit tile argument; else the forced tile;
 * else the table entry for exactly (m, n, k); else the built-in heuristic.
 * A positive group_m argument wins over the table's and the heuristic's.
 * The chosen tile is never replaced by another.
 *
 * ck_int8_table_set     registers (tile, group_m) for (m, n, k); tile in
 *                       [0, CK_NUM_TILES) with group_m >= 1, or tile == -1
 *                       to remove the entry.  CK_ERR_INVALID_ARG otherwise.
 *                       Tables hold measurements of this library on gfx950;
 *                       the Python binding loads only tables written for
 *                       the device's architecture.
 * ck_int8_table_clear   removes every entry.
 * ck_int8_table_size    number of entries.
 * ck_int8_set_forced_tile  tile in [-1, CK_NUM_TILES): every call without an
 *                       explicit tile uses it (-1: none).  Initial value:
 *                       the environment variable CK_INT8_FORCE_TILE.
 * ck_int8_forced_tile   the current forced tile (-1 if none).
 * ck_int8_set_path_log  non-zero: after each launch, one line per unique
 *                       (shape, output type, tile, group) on stderr naming
 *                       the kernel that ran (main loop kind, K stage, K
 *                       tail, blocks) and where its tile came from.  Initial
 *                       value: CK_INT8_LOG_PATH (non-zero integer = on).
 */
ck_status ck_int8_table_set(int64_t m, int64_t n, int64_t k, int tile, int group_m);
ck_status ck_int8_table_clear(void);
int64_t ck_int8_table_size(void);
ck_status ck_int8_set_forced_tile(int tile);
int ck_int8_forced_tile(void);
ck_status ck_int8_set_path_log(int on);

/*
 * Measurement aid (not a step of the layer): the HBM rate a kernel with the
 * quantisation's memory traffic reaches without its arithmetic.  Reads
 * `chunks` 16-byte chunks of src and writes one 8-byte word per chunk to
 * dst (2 bytes read and 1 written per bf16 element, the 2 : 1 mix of step
 * 1), both streamed past the caches, from `blocks` blocks of 256 threads
 * that keep `unroll` (1, 2, 4 or 8) loads in flight per lane.  src 16-byte
 * and dst 8-byte aligned, device pointers; chunks == 0 is a no-op.
 * Benchmarks run it over the activations of a workload and report the
 * quantisation's rate against the best configuration's.
 */
ck_status ck_hbm_stream(const void* src, int64_t chunks, void* dst, int blocks, int unroll,
                        hipStream_t stream);

/*
 * Measurement aid (not a step of the layer): the int8 matrix cores with
 * nothing else to do, the most the part delivers from them under its power
 * limit.  256 blocks of 512 threads (one per compute unit, two waves per
 * SIMD as in the GEMM).  Every block first fills a table of 12288 32-bit
 * words in LDS, word i = lowbias32(i + 12288 * seed) (C. Wellons' integer
 * hash: x ^= x >> 16; x *= 0x7feb352d; x ^= x >> 15; x *= 0x846ca68b;
 * x ^= x >> 16; all mod 2^32), seen as 8 slices of 6 fragments of 64 lanes
 * x 16 bytes: lane l's fragment f of slice s is the 4 words at 16-byte
 * index (6 s + f) 64 + l.  Every wave holds 8 accumulator tiles (as the
 * GEMM's waves do); a half-step with slice s runs the 8 products of
 * v_mfma_i32_32x32x32_i8 that add to tile 2i + j the product with fragment
 * 4 + j of s as the first operand and fragment i of s as the second
 * (i < 4, j < 2).  Each of the `iters` iterations is two half-steps:
 *   mode 0: slices 0 and 1, both kept in registers (products only);
 *   mode 1: half-step q (counting from 0 over the launch) uses slice q % 8,
 *           its fragments read from LDS every half-step.
 * out[512 b + t] receives the xor of lane t's 128 accumulator values
 * (int32, wrapping).  One launch is 2 * 256 * 8 * 16 * iters * 32768
 * integer operations (blocks, waves, products per iteration,
 * multiply-adds).  out: 256 * 512 int32, device memory.  Errors:
 * CK_ERR_INVALID_ARG for iters < 0, a mode other than 0 or 1 or a NULL out.
 */
ck_status ck_mfma_ceiling(int64_t iters, int mode, int32_t* out, uint32_t seed, hipStream_t stream);

/* Name of a status code (static string). */
const char* ck_status_string(ck_status s);

/* Detail message of the last failed call on this thread ("" if none). */
const char* ck_last_error(void);

/* ABI version of this header: bumped when a signature changes. */
int ck_abi_version(void);

#define CK_ABI_VERSION 11

#ifdef __cplusplus
}
#endif

#endif /* CK_INT8_H */
