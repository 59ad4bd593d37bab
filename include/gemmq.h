/*
 * gemmq.h -- C ABI of libgemmq, the packed-weight linear layer for AMD Instinct
 * MI355X (gfx950).
 *
 * The operation is gemm_quant from the PocketLLM pages: a Qwen3 linear layer
 * y = W x evaluated directly on ggml K-quant packed weights (the K-quant rung
 * of the pages' width ladder, q2_K through q6_K), with the weights
 * decoded inside the kernel and never widened in device memory (PocketLLM
 * README, "What it runs" and "Roadmap": the K-quant rung is decoded in-kernel,
 * packed, never widened), after the activations have been quantized to int8
 * blocks (molayo article "PocketLLM: 단일 가속기에서 대규모 언어 모델 실행",
 * status row "src/ -- C++ engine": the CPU gemm_quant quantizes activations to
 * int8 the way llama.cpp does).  One process owns one device and the ABI has no
 * rank or collective (README, "The rule").
 *
 * Conventions for every entry point:
 *  - Pointers named X, Xq, W, Wf, Y are DEVICE pointers on the current HIP device.
 *    The caller allocates and frees every buffer; the library allocates nothing
 *    and keeps no per-call state, so calls are reentrant.
 *  - `stream` is a hipStream_t passed as void*; NULL means the default stream.
 *    A return of GEMMQ_OK means the work is enqueued on that stream; results are
 *    valid once the stream has synchronised.  The library never synchronises.
 *  - Arguments are validated before anything is launched; a negative status
 *    names the failing condition (gemmq_status_str) and nothing was launched.
 *    No C++ exception crosses this ABI.  The calling thread's pending HIP error
 *    (hipGetLastError) is cleared just before a launch, so GEMMQ_E_LAUNCH always
 *    refers to the library's own launch.
 *  - M == 0 or N == 0 is a valid empty call: GEMMQ_OK, nothing is touched.
 *  - Layouts: X is f32 [M, K] row-major; Y is f32 [M, N] row-major and is
 *    overwritten (no accumulation into it); W is N rows, each K/256 consecutive
 *    super-blocks (row n's block b at byte offset (n*K/256 + b) * block_bytes);
 *    Xq is M rows of K/256 consecutive q8_K blocks, same order.
 *
 * Block formats (little-endian; the pages name the ggml formats but print no
 * layout, so these are the public ggml layouts):
 *  q2_K   84 B / 256 weights: 16 B of 4-bit scale (low nibble) and min (high
 *        nibble) per sub-block | 64 B of 2-bit quants | f16 d | f16 dmin;
 *        sub-block j (16 weights): w = d*sc_j*q - dmin*m_j, q in 0..3.
 *  q3_K  110 B / 256 weights: 32 B high-bit mask | 64 B of 2-bit low parts |
 *        12 B of 6-bit scales | f16 d; sub-block j (16 weights):
 *        w = d*(sc_j - 32)*q, q = low part, minus 4 where the mask bit is clear.
 *  q4_K  144 B / 256 weights: f16 d | f16 dmin | 12 B of 6-bit scales and mins |
 *        128 B of 4-bit quants; sub-block j (32 weights): w = d*sc_j*q - dmin*m_j.
 *  q5_K  176 B / 256 weights: q4_K's 16-byte header | 32 B of high bits | 128 B
 *        of 4-bit low parts laid out as q4_K's quants; w as q4_K, q in 0..31.
 *  q6_K  210 B / 256 weights: 128 B low nibbles | 64 B 2-bit highs | 16 int8
 *        scales | f16 d; sub-block j (16 weights): w = d*sc_j*(q - 32).
 *  q8_K  292 B / 256 activations: f32 d | 256 int8 q | 16 int16 group sums.
 */
#ifndef GEMMQ_H
#define GEMMQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GEMMQ_ABI_VERSION 10

/* Weight formats, numbered as the GGUF tensor type ids. */
#define GEMMQ_Q2_K 10
#define GEMMQ_Q3_K 11
#define GEMMQ_Q4_K 12
#define GEMMQ_Q5_K 13
#define GEMMQ_Q6_K 14

/* The load-time repacked layouts of q3_K and q6_K (gemmq_repack): the type id
 * plus 256.  Accepted wherever a weight format is, except gemmq_decode. */
#define GEMMQ_Q3_K_R (256 + GEMMQ_Q3_K)
#define GEMMQ_Q6_K_R (256 + GEMMQ_Q6_K)

#define GEMMQ_Q2_K_BYTES 84
#define GEMMQ_Q3_K_BYTES 110
#define GEMMQ_Q4_K_BYTES 144
#define GEMMQ_Q5_K_BYTES 176
#define GEMMQ_Q6_K_BYTES 210
#define GEMMQ_Q8_K_BYTES 292
#define GEMMQ_QK 256
#define GEMMQ_MAX_GROUP 4 /* matrices per gemmq_gemm_group call */

#define GEMMQ_OK 0
/* Status codes.  Formats the library does not implement are refused by name
 * rather than guessed at, as the pages' engine refuses unimplemented formats
 * at load (PocketLLM README, "Roadmap" and "Current status"). */
#define GEMMQ_E_INVALID_ARG (-1)        /* null pointer, negative size, bad path id or count */
#define GEMMQ_E_UNSUPPORTED_FORMAT (-2) /* fmt is not one of GEMMQ_Q2_K .. GEMMQ_Q6_K, _R
                                           (or not accepted by the entry point or path) */
#define GEMMQ_E_SHAPE (-3)              /* K not a positive multiple of 256 up to 2^24, rows
                                           above 2^31, or M above the path's limit */
#define GEMMQ_E_ALIGNMENT (-4)          /* a pointer breaks the alignment stated below */
#define GEMMQ_E_DEVICE (-5)             /* current device is not gfx950, or no device */
#define GEMMQ_E_LAUNCH (-6)             /* the HIP runtime rejected a launch or a kernel
                                           attribute the launch needs */

/* Paths for gemmq_gemm_ex, each with its limit on M (GEMMQ_E_SHAPE beyond). */
#define GEMMQ_PATH_AUTO 0 /* decode GEMV (M <= 8; q4_K M <= 2), small-M MFMA (q4_K 3..64; q6_K 3..16), GEMM; see gemmq_gemm */
#define GEMMQ_PATH_GEMV 1 /* decode GEMV, M in 1..8 only */
#define GEMMQ_PATH_GEMM 2 /* MFMA GEMM, M up to GEMMQ_GEMM_MAX_M */
#define GEMMQ_PATH_SKINNY 3 /* small-M MFMA kernels: q4_K M in 1..64; q6_K and q6_K_R M in 1..16 */
#define GEMMQ_GEMM_MAX_M 4194240 /* 65535 tiles of 64 activation rows */

/* ABI version (GEMMQ_ABI_VERSION of the library that was loaded): the C core
 * is a separately versioned library loaded through ctypes, as the pages' engine
 * core is (PocketLLM README, "Current status").  Never fails. */
int gemmq_abi_version(void);

/* Static string naming a status code and the condition behind it (the pages
 * refuse by name: PocketLLM README, "Roadmap"); never NULL, "GEMMQ_E_UNKNOWN..."
 * for a value that is not a status. */
const char *gemmq_status_str(int status);

/* Bytes of one super-block of `fmt` (84, 110, 144, 176, 210: the K-quant block
 * sizes of the formats the pages' width ladder names, PocketLLM README "What it
 * runs"), or 0 for an unknown format. */
size_t gemmq_block_bytes(int fmt);

/* Bytes of an N x K packed weight matrix: N * K/256 * block_bytes; 0 when fmt is
 * unknown, N or K is negative, K % 256 != 0, K > 2^24 or N > 2^31. */
size_t gemmq_weight_bytes(int fmt, int64_t N, int64_t K);

/* Bytes of M x K activations in q8_K (the int8 activation blocks of the pages'
 * CPU gemm_quant, molayo article, status row "src/"): M * K/256 * 292; 0 on bad
 * sizes (as gemmq_weight_bytes). */
size_t gemmq_q8K_bytes(int64_t M, int64_t K);

/*
 * Quantize f32 activations to q8_K blocks (step a1).  For every 256 consecutive
 * values of a row: amax = max|x|, d = amax/127 (f32, correctly rounded division),
 * q = round-half-even(x/d) clamped to [-127, 127], group sums over 16 values;
 * a block whose d is 0 is stored as all zeros.  Inputs must be finite.
 * This is the int8 activation quantization that precedes the packed dot in the
 * molayo article's description of the CPU gemm_quant (status row "src/").
 *   X   device, f32 [M, K], 16-byte aligned.
 *   Xq  device, gemmq_q8K_bytes(M, K) bytes, 4-byte aligned; fully overwritten.
 * Errors: GEMMQ_E_INVALID_ARG (null pointer when M > 0, M < 0),
 *         GEMMQ_E_SHAPE (K <= 0 or K % 256 != 0), GEMMQ_E_ALIGNMENT,
 *         GEMMQ_E_DEVICE, GEMMQ_E_LAUNCH.
 */
int gemmq_quantize_q8K(const float *X, void *Xq, int64_t M, int64_t K, void *stream);

/*
 * Y[m, n] = sum_k w[n, k] * d_x[m, k/256] * q_x[m, k]  -- the packed linear layer,
 * the pages' gemm_quant operator (PocketLLM README, "Current status": the kernel
 * layer declares gemm_quant; molayo article, status row "src/": the packed dot
 * walks each weight row once per tile of activation rows, and the reordered f32
 * sums are held to a 1e-5 scaled relative bound)
 * (steps a2..a5: in-kernel unpack; the path chosen by GEMMQ_PATH_AUTO: the decode
 * GEMV for M <= 8 -- for q4_K M <= 2, and M = 3, 4 on launches large enough
 * that it stages the activation in LDS (rows of at most 16 blocks, M*K/256 <=
 * 64, output columns x M x K/256 >= 2^18) --, the small-M MFMA kernel for q4_K
 * at 3 <= M <= 64 when M <= 16 or when the launch's output columns times
 * ceil(M/16) are at most 20480, and for q6_K and q6_K_R at 9 <= M <= 16 and at 3 <= M <= 8
 * when the launch has at least 16384 output columns (at M <= 4 only where
 * M*K/256 > 32: below that the GEMV holds the activation in LDS and is faster),
 * and for plain q6_K at 5 <= M <= 8 on rows of more than 8 super-blocks also
 * when output columns x K/256 >= 2^16, at M = 3, 4 on rows of more than 64
 * when it is >= 2^18, the MFMA GEMM otherwise; the choice is made once per launch, from M, K and
 * the sum of the N of the matrices it serves).
 *   fmt  GEMMQ_Q2_K, GEMMQ_Q3_K, GEMMQ_Q4_K, GEMMQ_Q5_K, GEMMQ_Q6_K, or a
 *        repacked GEMMQ_Q3_K_R / GEMMQ_Q6_K_R (weights from gemmq_repack).
 *   W    device, gemmq_weight_bytes(fmt, N, K) bytes; 16-byte aligned for q4_K,
 *        q5_K and the repacked layouts, 4-byte aligned for q2_K, q3_K and q6_K.
 *   Xq   device, gemmq_q8K_bytes(M, K) bytes from gemmq_quantize_q8K (or any
 *        valid q8_K blocks: |q| <= 127 and sums equal to the sums of q),
 *        4-byte aligned.
 *   Y    device, f32 [M, N], 4-byte aligned; overwritten.
 * The f32 result differs from the exact value by at most 1e-5 * sum_k|w_k*xhat_k|
 * + 1e-6 (xhat = d_x*q_x); within one path, an output depends only on its own
 * activation row and weight row, so any subset of rows gives identical bits.
 * Errors: GEMMQ_E_INVALID_ARG, GEMMQ_E_UNSUPPORTED_FORMAT, GEMMQ_E_SHAPE,
 *         GEMMQ_E_ALIGNMENT, GEMMQ_E_DEVICE, GEMMQ_E_LAUNCH.
 */
int gemmq_gemm(int fmt, const void *W, const void *Xq, float *Y, int64_t M, int64_t N,
               int64_t K, void *stream);

/* gemmq_gemm with an explicit path (GEMMQ_PATH_*).  GEMMQ_PATH_GEMV with M > 8,
 * GEMMQ_PATH_SKINNY with M > 64 (q6_K and q6_K_R: M > 16) and GEMMQ_PATH_GEMM (also
 * when chosen by GEMMQ_PATH_AUTO) with M > GEMMQ_GEMM_MAX_M return GEMMQ_E_SHAPE;
 * GEMMQ_PATH_SKINNY with a format other than GEMMQ_Q4_K, GEMMQ_Q6_K and GEMMQ_Q6_K_R
 * returns GEMMQ_E_UNSUPPORTED_FORMAT.  Same arguments, layout and errors
 * otherwise.  GEMMQ_PATH_SKINNY is the batched decode kernel (the pages keep
 * q6_K on a row path of its own: molayo article, status row "src/"): q4_K
 * holds the activation rows in one to four 16 x 16 x 64 int8 MFMA tiles, q6_K
 * in one 32 x 32 x 16 tile per 16-weight sub-block; either splits the
 * super-blocks of a row over the waves of a workgroup by K alone. */
int gemmq_gemm_ex(int fmt, const void *W, const void *Xq, float *Y, int64_t M, int64_t N,
                  int64_t K, int path, void *stream);

/*
 * Several weight matrices of one format that read the same activations, in one
 * launch: for g < count, Y[g] = W[g] applied to Xq exactly as
 * gemmq_gemm_ex(fmt, W[g], Xq, Y[g], M, N[g], K, p, stream) computes it (the
 * same bits), where p is `path`, or for GEMMQ_PATH_AUTO the path chosen for the
 * whole launch (from M and N[0] + ... + N[count-1], as gemmq_gemm describes).  Sharing one input is what a transformer layer's q/k/v
 * projections and its gate/up projections do; one launch instead of several
 * removes the per-launch cost that dominates at small M.
 *   count  1..4.
 *   W, Y, N  HOST arrays of `count` entries, read during the call only; each
 *        W[g] / Y[g] / N[g] as in gemmq_gemm.  N[g] == 0 entries are skipped.
 *   Xq, M, K, path, stream  as in gemmq_gemm_ex.
 * Errors: those of gemmq_gemm_ex for any entry, and GEMMQ_E_INVALID_ARG for a
 * count outside 1..4 or a null array; nothing is launched on an error.
 */
int gemmq_gemm_group(int fmt, int count, const void *const *W, float *const *Y, const int64_t *N,
                     const void *Xq, int64_t M, int64_t K, int path, void *stream);

/*
 * The whole linear layer from f32 activations: quantize X to q8_K into Xq, then
 * apply every W[g] to it -- the same bits as gemmq_quantize_q8K(X, Xq, M, K)
 * followed by gemmq_gemm_group(fmt, count, W, Y, N, Xq, M, K, path), for Xq and
 * for every Y[g].  At decode shapes (GEMV path, M <= 4 and M*K/256 small) it is
 * one launch: every workgroup quantizes X into its own LDS while its weight
 * loads are in flight, and workgroup 0 also writes Xq -- unless the call is
 * large (rows x M x K/256 from 2^19, or from 2^18 where each wave would
 * quantize four blocks, e.g. M = 3, 4 at K = 2048), where quantizing once in a
 * launch of its own costs less.  Otherwise it enqueues the two launches.  Quantizing in the consuming launch is how the CPU
 * gemm_quant on the pages treats the int8 activation step, as part of the
 * matmul (molayo article, status row "src/").
 *   X      device, f32 [M, K], 16-byte aligned (as gemmq_quantize_q8K).
 *   Xq     device, gemmq_q8K_bytes(M, K) bytes, 4-byte aligned; fully
 *          overwritten with the q8_K blocks of X when M > 0.
 *   fmt, count, W, Y, N, M, K, path, stream  as in gemmq_gemm_group; all N[g]
 *          == 0 still quantizes X.
 * Errors: those of gemmq_quantize_q8K and gemmq_gemm_group; nothing is launched
 * on an error (the matmul's limits are checked before the quantizer is
 * enqueued, so Xq is untouched when the call fails).
 */
int gemmq_linear_group(int fmt, int count, const void *const *W, float *const *Y,
                       const int64_t *N, const float *X, void *Xq, int64_t M, int64_t K,
                       int path, void *stream);

/*
 * The MLP's gated up-projection in one call: quantize X to q8_K into Xq, then
 *   Y[m, n] = silu(G[m, n]) * U[m, n],   G = Wg x, U = Wu x,
 * where G and U are exactly the values gemmq_linear_group(fmt, 2, {Wg, Wu}, ...)
 * computes (same bits), and the product is taken in f32 as e = expf(-g),
 * s = g / (1 + e) (correctly rounded division), y = s * u.  This is the silu_mul
 * step the pages run right after the gate/up matmuls (molayo article, status row
 * "src/"), moved into the matmul's output: one output matrix instead of two.  At
 * decode shapes it is one launch (quantizer fused, as in gemmq_linear_group).
 *   Wg, Wu  device, gemmq_weight_bytes(fmt, N, K) bytes each, alignment as in
 *           gemmq_gemm; the gate and the up matrix, N rows each.
 *   X, Xq   as in gemmq_linear_group (Xq receives the q8_K blocks of X).
 *   Y       device, f32 [M, N], 4-byte aligned; overwritten.
 *   fmt, M, K, path, stream  as in gemmq_gemm_ex; N == 0 still quantizes X.
 * Accuracy: with g, u within the matmul bound of gemmq_gemm, |y - silu(g*) u*|
 * is at most 1.1 |u| dg + |silu(g)| du plus a few f32 roundings of y (g*, u*
 * exact; dg, du the matmul bounds), and, from the f32 range, |g u| 2^-126 +
 * 2^-149 (exp(-g) overflows for g < -88.72, where y is +-0).
 * Errors: those of gemmq_linear_group for the two matrices; nothing is launched
 * on an error.
 */
int gemmq_linear_silu_mul(int fmt, const void *Wg, const void *Wu, const float *X, void *Xq,
                          float *Y, int64_t M, int64_t N, int64_t K, int path, void *stream);

/* gemmq_linear_group for one matrix with GEMMQ_PATH_AUTO. */
int gemmq_linear(int fmt, const void *W, const float *X, void *Xq, float *Y, int64_t M, int64_t N,
                 int64_t K, void *stream);

/*
 * Load-time repack of a q3_K or q6_K matrix into its GEMMQ_Q3_K_R /
 * GEMMQ_Q6_K_R layout: the same bytes (gemmq_weight_bytes(fmt, N, K)), with the
 * NB = N*K/256 blocks' fields each stored for all blocks in block order --
 *   q6_K: ql[NB][128] | qh[NB][64] | sc[NB][16] | d[NB][2]
 *   q3_K: hmask[NB][32] | qs[NB][64] | scales[NB][12] | d[NB][2]
 * -- so that every field of 16 or more bytes per block is 16-byte aligned and
 * the kernels load it without realigning (the 110- and 210-byte blocks
 * otherwise start on any even address).  The matmul on repacked weights gives
 * the same bits as on the original ones.  This is the GPU counterpart of the
 * pages' load-time q4_K 8-column panels (molayo article, status row "src/"),
 * for the two formats whose block size breaks alignment.  The layout belongs
 * to a whole matrix: a repacked matrix cannot be sliced by rows.
 *   fmt  GEMMQ_Q3_K or GEMMQ_Q6_K (the layout of W).
 *   W    device, 4-byte aligned.   Wr  device, 16-byte aligned, not overlapping W.
 * Errors: GEMMQ_E_UNSUPPORTED_FORMAT (another fmt), GEMMQ_E_INVALID_ARG (null,
 *         N < 0, overlap), GEMMQ_E_SHAPE, GEMMQ_E_ALIGNMENT, GEMMQ_E_DEVICE,
 *         GEMMQ_E_LAUNCH.
 */
int gemmq_repack(int fmt, const void *W, void *Wr, int64_t N, int64_t K, void *stream);

/*
 * Diagnostic export: decode packed weights to f32 with the same device unpacker
 * (step a2) the matmul kernels use: the weights the pages decode inside the
 * kernel and never widen (PocketLLM README, "What it runs"), widened here only
 * for inspection.  Never used on the compute path.
 *   W   device, gemmq_weight_bytes(fmt, N, K) bytes, alignment as in gemmq_gemm.
 *   Wf  device, f32 [N, K], 16-byte aligned; overwritten.
 * q2_K, q4_K and q5_K weights are the single f32 rounding of d*sc*q - dmin*m;
 * q3_K and q6_K weights are exact.  Errors as gemmq_gemm.
 */
int gemmq_decode(int fmt, const void *W, float *Wf, int64_t N, int64_t K, void *stream);

/*
 * Measurement export: the int8 matrix-core ceiling the matmul kernels are read
 * against (the pages state no GPU figure for this operator; this measures the
 * device's own).  Never used on the compute path.  Launches `blocks` workgroups of
 * four waves; each wave runs `iters` rounds of GEMMQ_PROBE_CHAINS independent
 * v_mfma_i32_32x32x32_i8 (32 x 32 x 32 int8 multiply-adds each) on register
 * operands, with no memory traffic, so the time of the launch gives the
 * sustained dense int8 MFMA rate:
 *   int8 ops = 2 * 32768 * GEMMQ_PROBE_CHAINS * 4 * blocks * iters.
 *   iters   1..GEMMQ_PROBE_MAX_ITERS.  blocks in 1..65535.
 *   out     device, int32 [blocks * 256], 4-byte aligned; each lane's sum of its
 *           accumulators (keeps the work live; identical in every workgroup).
 *   clocks  device, uint64 [2], 8-byte aligned: shader-clock cycles
 *           (s_memtime) and 100 MHz counter ticks (s_memrealtime) across the
 *           loop of the first wave, so cycles / ticks * 100 MHz is the shader
 *           clock the loop ran at.
 * Errors: GEMMQ_E_INVALID_ARG (null pointer, iters or blocks out of range),
 * GEMMQ_E_ALIGNMENT, GEMMQ_E_DEVICE, GEMMQ_E_LAUNCH.
 */
#define GEMMQ_PROBE_CHAINS 4
#define GEMMQ_PROBE_MAX_ITERS 1000000
int gemmq_probe_mfma_i8(int64_t iters, int64_t blocks, int32_t *out, uint64_t *clocks,
                        void *stream);

/*
 * Measurement export: the loop of gemmq_probe_mfma_i8 with `valu` independent
 * f32 FMAs (no operand taken from a matrix result) issued after every MFMA,
 * valu in {0, 4, 8, 12, 16}.  Never used on the compute path.  The launch time
 * against valu gives the time of one MFMA with that much vector work beside it:
 * how much vector work a matrix instruction hides and what each vector
 * instruction costs past that, the terms of the GEMMs' per-super-block budget.
 * Launched with two waves per SIMD (blocks = 2 x compute units), as the GEMMs
 * run.  Arguments, outputs, operation count and errors as gemmq_probe_mfma_i8;
 * any other valu is GEMMQ_E_INVALID_ARG.
 */
int gemmq_probe_mfma_valu(int64_t iters, int64_t blocks, int32_t valu, int32_t *out,
                          uint64_t *clocks, void *stream);

/*
 * Measurement export: the read-only device-memory ceiling the decode GEMV is
 * read against (the GEMV streams each packed weight once and writes next to
 * nothing).  Never used on the compute path.  Reads `bytes` from `src` with
 * GEMMQ_PROBE_READ_WORDS waves, every lane keeping eight 16-byte loads in
 * flight, and stores one XOR fold per wave, so the launch time gives the
 * sustained read rate: bytes / time.
 *   src    device, `bytes` bytes, 16-byte aligned; bytes a positive multiple of
 *          16, at most 2^40.  Contents are arbitrary.
 *   out    device, uint32 [GEMMQ_PROBE_READ_WORDS], 4-byte aligned; overwritten.
 * Errors: GEMMQ_E_INVALID_ARG, GEMMQ_E_ALIGNMENT, GEMMQ_E_DEVICE, GEMMQ_E_LAUNCH.
 */
#define GEMMQ_PROBE_READ_WORDS 2048
int gemmq_probe_read(const void *src, int64_t bytes, uint32_t *out, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* GEMMQ_H */
