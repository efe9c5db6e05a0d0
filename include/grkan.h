/*
 * grkan.h -- C ABI of the MI355X (gfx950) GR-KAN safe Pade activation library
 * (libgrkan.so).
 *
 * Pages cited
 *   [FlashKAT notes]  "FlashKAT: Understanding and Addressing Performance
 *                     Bottlenecks in the Kolmogorov-Arnold Transformer",
 *                     Paper-Notes page (AAAI 2026), arXiv 2505.13813.
 *
 * The operation.  GR-KAN shares one rational function among the channels of
 * each of n_groups contiguous channel groups and uses the "safe" Pade unit
 * ([FlashKAT notes], section "KAT 的突破与残留问题"), with 6 numerator and 4
 * denominator coefficients per group (section "损失函数 / 训练策略"):
 *
 *     F_g(x) = P_g(x) / (1 + |Q_g(x)|),
 *     P_g(x) = a_g0 + a_g1 x + ... + a_g5 x^5,
 *     Q_g(x) = b_g1 x + b_g2 x^2 + b_g3 x^3 + b_g4 x^4   (no constant term).
 *
 * Channel c of a row of d channels belongs to group c / (d / n_groups).
 * The backward pass (section "2. 原始 KAT 的 atomic add 问题分析") produces
 * dX elementwise and the coefficient gradients dA, dB, each summed over every
 * element (all rows, all channels) of its group; with s = sign(Q),
 * sign(0) = 0 and D = 1 + |Q|:
 *
 *     dX      = dY (P'/D - s P Q'/D^2)
 *     dA[g,i] = sum dY x^i / D                (i = 0..5)
 *     dB[g,j] = sum -dY s P x^(j+1) / D^2     (j = 0..3, i.e. b_g1..b_g4)
 *
 * Conventions shared by every entry point
 *   - Tensors are row-major [rows][d], rows = batch * sequence; x, y, dy and
 *     dx have the I/O dtype `io`; A is fp32 [n_groups][6] (a_0..a_5), B is
 *     fp32 [n_groups][4] (b_1..b_4), dA and dB are fp32 with the same shapes.
 *     Arithmetic is fp32; group sums are carried in fp64 inside the library.
 *     Q is evaluated in fp64; where a bound does not prove its sign, the
 *     sign of Q = x q(x) is decided again: exactly, in integers over the
 *     fp32 mantissas, for denominator degrees n >= 5 (unless the terms span
 *     more than ~250 bits), and by compensated Horner in fp64 for n <= 4.
 *   - All pointers are device pointers on the current HIP device, owned by
 *     the caller.  The library allocates no device memory and keeps no state
 *     beyond a per-device cache of launch limits.
 *   - Work is enqueued on `stream` and the call returns without waiting.
 *     Faults inside a kernel surface at the caller's next synchronisation.
 *   - Arguments are validated before any HIP call; an invalid call changes
 *     nothing on the device.  No C++ exception crosses this interface.
 *
 * The PAU family.  The pages note that the same kernel restructuring applies
 * to PAU and its variants ([FlashKAT notes], section "局限性与未来工作"): the
 * safe rational unit with other numerator / denominator degrees (m, n),
 *
 *     F_g(x) = (a_g0 + ... + a_gm x^m) / (1 + |b_g1 x + ... + b_gn x^n|),
 *
 * with A [n_groups][m+1], B [n_groups][n] and m + 1 + n gradient sums per
 * group; n = 0 is a plain polynomial (B, dB unused and may be NULL), and
 * n_groups = 1 is a single PAU shared by all channels.  The grkan_pau_*
 * entry points take (m, n) explicitly; the grkan_* ones are GR-KAN's
 * (m, n) = (5, 4).  grkan_pau_supported() says which pairs are compiled in.
 */
#ifndef GRKAN_H
#define GRKAN_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifndef GRKAN_API
#define GRKAN_API __attribute__((visibility("default")))
#endif

#ifdef __cplusplus
extern "C" {
#endif

/* The enumerations are ints (as every C enum is); under C++ they are given
 * that underlying type explicitly, so that any int a C caller passes -- an
 * unknown status or dtype included -- is a valid value to test and reject. */
#ifdef __cplusplus
#define GRKAN_ENUM_INT : int
#else
#define GRKAN_ENUM_INT
#endif

typedef enum GRKAN_ENUM_INT {
    GRKAN_OK = 0,
    GRKAN_ERR_INVALID_ARG = 1, /* null pointer, bad shape, overlap, small workspace, bad flags */
    GRKAN_ERR_UNSUPPORTED = 2, /* misaligned pointer, a degree pair not compiled in, more than
                                  65535 groups whose row segments are whole 16-byte vectors,
                                  a shape past the launch limits                               */
    GRKAN_ERR_HIP = 3          /* the HIP runtime reported an error on query or launch          */
} grkan_status_t;

typedef enum GRKAN_ENUM_INT {
    GRKAN_F32 = 0,  /* fp32 x, y, dy, dx                                   */
    GRKAN_BF16 = 1  /* bf16 x, y, dy, dx; outputs rounded to nearest even  */
} grkan_dtype_t;

enum {
    /* Backward reduction schemes (the `flags` argument).
       GRKAN_DETERMINISTIC (or flags = 0, the same request): one partial sum
       per (row tile, group, coefficient) goes to `workspace` and a second
       kernel adds them in fp64 in a fixed order -- bitwise reproducible for a
       given shape and library build, on any device, and accurate to the fp32
       rounding of the individual terms; the two-stage reduction of [PolyKAN]
       ("PolyKAN: Efficient Fused GPU Operators for Polynomial
       Kolmogorov-Arnold Network Variants", abstract page, arXiv 2511.14852).
       The two atomic flags select the schemes the pages compare ([FlashKAT
       notes], sections "2. 原始 KAT 的 atomic add 问题分析" and "3. FlashKAT
       核函数重构（Algorithm 2）"); they are kept for measurement, are not
       reproducible run to run, and their fp32 accumulation error grows with
       the number of workgroups or elements, as the pages' rounding-error
       table shows for their GPUs.  At most one of the three bits may be
       set; any other bit is GRKAN_ERR_INVALID_ARG. */
    GRKAN_DETERMINISTIC = 1u << 0, /* fixed-order two-stage reduction (also flags = 0) */
    GRKAN_BLOCK_ATOMIC = 1u << 1,  /* one fp32 atomic add per coefficient per workgroup */
    GRKAN_NAIVE_ATOMIC = 1u << 2   /* ten fp32 atomic adds per element (KAT's original) */
};

/*
 * Forward: y = F(x) elementwise.
 *   x, y      [rows][d], dtype io, 16-byte aligned; y == x (in place) is
 *             allowed, any other overlap is GRKAN_ERR_INVALID_ARG.  May be
 *             NULL when rows == 0.
 *   A, B      fp32 coefficients [n_groups][6] and [n_groups][4], 4-byte aligned.
 *   rows >= 0 (0 is a no-op), d >= 1, n_groups >= 1, d % n_groups == 0.
 *   Any such n_groups is served: groups whose row segment (d / n_groups
 *   elements) is a whole number of 16-byte vectors take kernels with one
 *   16-byte vector per lane, narrower ones -- down to one function per
 *   channel, n_groups = d -- kernels with one channel column per lane.
 */
GRKAN_API grkan_status_t grkan_forward(const void *x, void *y, const float *A, const float *B,
                             int64_t rows, int64_t d, int32_t n_groups,
                             grkan_dtype_t io, hipStream_t stream);

/*
 * Backward: dx = dy * dF/dx elementwise, and dA, dB = the group sums above.
 *   x, dy     inputs [rows][d], dtype io, 16-byte aligned.
 *   dx        output [rows][d], dtype io, 16-byte aligned; dx may equal x or
 *             dy exactly (in place), any other overlap is INVALID_ARG.
 *   dA, dB    fp32 outputs [n_groups][6], [n_groups][4]; overwritten, not
 *             accumulated; must not overlap any other argument.  rows == 0
 *             writes zeros.
 *   flags     0 or GRKAN_DETERMINISTIC (two-stage fixed-order reduction),
 *             GRKAN_BLOCK_ATOMIC or GRKAN_NAIVE_ATOMIC (both zero dA, dB
 *             first).  Two of these bits together, or any other bit, are
 *             INVALID_ARG.
 *   workspace device memory of at least grkan_backward_workspace_size()
 *             bytes, 16-byte aligned, for the deterministic scheme; ignored
 *             (may be NULL) with an atomic flag.  Its contents on entry do not
 *             matter.  Two calls in flight at once must not share one
 *             workspace.
 */
GRKAN_API grkan_status_t grkan_backward(const void *x, const void *dy, const float *A, const float *B,
                              void *dx, float *dA, float *dB,
                              int64_t rows, int64_t d, int32_t n_groups,
                              grkan_dtype_t io, uint32_t flags,
                              void *workspace, size_t workspace_bytes, hipStream_t stream);

/* Bytes of workspace grkan_backward needs for these arguments (0 when it
 * needs none, or for arguments grkan_backward would reject).  It takes the
 * I/O dtype because the row tiles depend on it: a workgroup covers a fixed
 * number of 16-byte vectors, i.e. twice as many bf16 channels as fp32 ones,
 * so the number of tiles -- one partial sum each -- differs between the two.
 * Host-only: it makes no HIP call and works without a GPU. */
GRKAN_API size_t grkan_backward_workspace_size(int64_t rows, int64_t d, int32_t n_groups,
                                     grkan_dtype_t io, uint32_t flags);

/*
 * Streaming ceiling probe (a measurement tool, like grkan_inflated_*): c = a
 * XOR b, word by word, over `bytes` bytes -- the backward's memory traffic
 * (two tensors read, one written, 16-byte non-temporal accesses, one-shot
 * grid) with no arithmetic to speak of.  Its rate is the ceiling the
 * benchmark rates the backward against, next to the published HBM peak.
 *   a, b, c   device buffers of `bytes` bytes, 16-byte aligned; c may equal a
 *             or b exactly, any other overlap is GRKAN_ERR_INVALID_ARG.
 *   bytes     >= 0 (0 is a no-op), a multiple of 16 (else UNSUPPORTED).
 */
GRKAN_API grkan_status_t grkan_stream_probe(const void *a, const void *b, void *c, int64_t bytes,
                                  hipStream_t stream);

/*
 * grkan_backward without a workspace, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation).  The deterministic two-stage scheme of grkan_backward
 * (same kernels, same bits), with its partial sums in a fixed device array of
 * GRKAN_NOALLOC_SCRATCH_BYTES inside the library: one copy per device, held
 * until the process ends, its address looked up on the first call on each
 * device.  The call allocates nothing and frees nothing.
 *   Arguments and errors as grkan_backward (no flags, no workspace); a shape
 *   whose partial sums need more than GRKAN_NOALLOC_SCRATCH_BYTES (what
 *   grkan_backward_workspace_size() reports for it) is GRKAN_ERR_UNSUPPORTED,
 *   before any HIP call.  16 MiB covers the partial sums of every GR-KAN
 *   shape up to four times the KAT-B hidden activations in bf16 (4.0 MB
 *   there, as at KAT-S hidden in fp32).
 *   Calls on one device share the array and must not overlap in time (e.g.
 *   run on different streams without ordering): they would race on it.
 *   Nothing in it needs to start at zero -- every partial sum is written
 *   before it is read -- so no clearing is done between calls.
 */
#define GRKAN_NOALLOC_SCRATCH_BYTES (16u << 20)
GRKAN_API grkan_status_t grkan_backward_noalloc(const void *x, const void *dy, const float *A,
                                      const float *B, void *dx, float *dA, float *dB,
                                      int64_t rows, int64_t d, int32_t n_groups,
                                      grkan_dtype_t io, hipStream_t stream);

/* Static English text for a status code (never NULL). */
GRKAN_API const char *grkan_status_string(grkan_status_t status);

/* Launch geometry of a pass (0 = forward, 1 = backward, 2 = backward with
 * GRKAN_BLOCK_ATOMIC).  The geometry is a function of the shape, dtype and
 * degrees; cus and blocks_per_cu describe the current device (queried on
 * first use). */
typedef struct {
    int32_t block;          /* threads per workgroup (part_vecs * rows_per_iter)      */
    int32_t rows_per_iter;  /* rows a workgroup's lanes cover in one pass             */
    int32_t unroll;         /* passes per workgroup (loads issued together)           */
    int64_t tiles;          /* row tiles (unroll * rows_per_iter rows each)           */
    int64_t grid;           /* workgroups: one per (tile, group, part), padded to 8
                               tiles                                                  */
    int32_t cus;            /* compute units on the device                            */
    int32_t blocks_per_cu;  /* resident workgroups per CU for this kernel             */
    int32_t parts;          /* column parts per group row segment                     */
    int32_t part_vecs;      /* 16-byte vectors per part                               */
} grkan_launch_t;

GRKAN_API grkan_status_t grkan_query_launch(int64_t rows, int64_t d, int32_t n_groups,
                                  grkan_dtype_t io, int32_t pass, grkan_launch_t *out);

/* 1 if the degree pair (m, n) is compiled into this library, else 0.
 * Host-only. */
GRKAN_API int grkan_pau_supported(int32_t m, int32_t n);

/* grkan_forward for degrees (m, n): A [n_groups][m+1], B [n_groups][n]
 * (B may be NULL when n == 0).  Pairs not compiled in return
 * GRKAN_ERR_UNSUPPORTED, negative degrees GRKAN_ERR_INVALID_ARG. */
GRKAN_API grkan_status_t grkan_pau_forward(const void *x, void *y, const float *A, const float *B,
                                 int64_t rows, int64_t d, int32_t n_groups, int32_t m,
                                 int32_t n, grkan_dtype_t io, hipStream_t stream);

/* grkan_backward for degrees (m, n): dA [n_groups][m+1], dB [n_groups][n]
 * (B and dB may be NULL when n == 0).  GRKAN_NAIVE_ATOMIC exists for
 * (5, 4) only (GRKAN_ERR_UNSUPPORTED otherwise). */
GRKAN_API grkan_status_t grkan_pau_backward(const void *x, const void *dy, const float *A,
                                  const float *B, void *dx, float *dA, float *dB,
                                  int64_t rows, int64_t d, int32_t n_groups, int32_t m,
                                  int32_t n, grkan_dtype_t io, uint32_t flags,
                                  void *workspace, size_t workspace_bytes, hipStream_t stream);

/* Workspace bytes for grkan_pau_backward (0 when none is needed or the
 * arguments would be rejected).  Host-only. */
GRKAN_API size_t grkan_pau_backward_workspace_size(int64_t rows, int64_t d, int32_t n_groups,
                                         int32_t m, int32_t n, grkan_dtype_t io,
                                         uint32_t flags);

/* grkan_query_launch for degrees (m, n). */
GRKAN_API grkan_status_t grkan_pau_query_launch(int64_t rows, int64_t d, int32_t n_groups,
                                      int32_t m, int32_t n, grkan_dtype_t io, int32_t pass,
                                      grkan_launch_t *out);

/*
 * FLOP-inflation probe ([FlashKAT notes], section "1. 性能瓶颈诊断",
 * Insight 2: the rational's arithmetic multiplied by 8 through nested loops
 * left the pages' run time unchanged).  grkan_forward / grkan_backward with
 * every element evaluated `repeat` times instead of once -- the rational in
 * the forward; P, P', Q, Q', 1 + |Q|, the sign guard and dx in the backward --
 * and the results of the last evaluation used.  The outputs are bit for bit
 * those of grkan_forward / grkan_backward with the same arguments; the
 * memory traffic and launch geometry are the same too, so the run time
 * against `repeat` shows how far the activation is from being bound by its
 * arithmetic.  A measurement tool, not a faster path.
 *   repeat    1, 2, 4 or 8 (1 runs the plain kernels); anything else is
 *             GRKAN_ERR_INVALID_ARG.
 *   Other arguments as in grkan_forward / grkan_backward, with two limits:
 *   shapes whose group row segment (d / n_groups * bytes(io)) is not a
 *   multiple of 16 bytes, and GRKAN_NAIVE_ATOMIC, are GRKAN_ERR_UNSUPPORTED
 *   for repeat > 1.  The workspace is grkan_backward_workspace_size()'s.
 */
GRKAN_API grkan_status_t grkan_inflated_forward(const void *x, void *y, const float *A,
                                      const float *B, int64_t rows, int64_t d,
                                      int32_t n_groups, grkan_dtype_t io, int32_t repeat,
                                      hipStream_t stream);

GRKAN_API grkan_status_t grkan_inflated_backward(const void *x, const void *dy, const float *A,
                                       const float *B, void *dx, float *dA, float *dB,
                                       int64_t rows, int64_t d, int32_t n_groups,
                                       grkan_dtype_t io, uint32_t flags, int32_t repeat,
                                       void *workspace, size_t workspace_bytes,
                                       hipStream_t stream);

/*
 * The GR-KAN layer ([FlashKAT notes], section "1. 性能瓶颈诊断", Insight 2:
 * the activation's (2m+2n+3) d_in FLOPs feed a linear map of 2 d_in d_out):
 * z = F(x) W^T, GR-KAN degrees (5, 4), no bias (the pages print none).
 * bf16 throughout: F is evaluated in fp32 as grkan_forward does, rounded to
 * nearest-even bf16 and multiplied on the matrix cores with fp32
 * accumulation; z is rounded to nearest-even bf16.  F is applied while x is
 * staged for the matrix product, so F(x) never goes to memory.
 *   x         bf16 [rows][d_in], 16-byte aligned (may be NULL when rows == 0).
 *   A, B      fp32 [n_groups][6], [n_groups][4], 4-byte aligned.
 *   W         bf16 [d_out][d_in] (row o holds output o's weights), 16-byte aligned.
 *   z         bf16 [rows][d_out], 2-byte aligned; must not overlap x, W, A, B.
 *   rows >= 0 (0 is a no-op); d_in, d_out >= 1; d_in % n_groups == 0.
 *   GRKAN_ERR_UNSUPPORTED: d_in not a multiple of 64, d_in / n_groups not a
 *   multiple of 8, more than 64 groups, rows / d_in / d_out >= 2^31, or a
 *   misaligned pointer.
 */
GRKAN_API grkan_status_t grkan_layer_forward(const void *x, const float *A, const float *B,
                                   const void *W, void *z, int64_t rows, int64_t d_in,
                                   int64_t d_out, int32_t n_groups, hipStream_t stream);

/*
 * grkan_layer_forward with a workspace, which lets the library take the
 * faster form for the shape: the fused form evaluates F again for every
 * 256-column tile of z, so for d_out > 256 F is evaluated once into the
 * workspace (bf16 [rows][d_in], as the fused form rounds it) and the plain
 * matrix product follows -- the same bits either way.  Arguments and limits
 * as grkan_layer_forward, plus
 *   workspace  grkan_layer_forward_workspace_size() bytes (0 when the fused
 *              form is taken; then it may be NULL), 16-byte aligned, not
 *              overlapping any other argument; contents on entry do not matter.
 */
GRKAN_API grkan_status_t grkan_layer_forward_ws(const void *x, const float *A, const float *B,
                                      const void *W, void *z, int64_t rows, int64_t d_in,
                                      int64_t d_out, int32_t n_groups, void *workspace,
                                      size_t workspace_bytes, hipStream_t stream);

/* Bytes of workspace grkan_layer_forward_ws needs (0 when it takes the fused
 * form, for rows == 0, or for arguments it would reject).  Host-only. */
GRKAN_API size_t grkan_layer_forward_workspace_size(int64_t rows, int64_t d_in, int64_t d_out,
                                          int32_t n_groups);

/*
 * The same linear map without the activation: z = y W^T, bf16 y [rows][d_in]
 * (16-byte aligned), W and z as above, the same matrix-core kernel and
 * limits.  With y = grkan_forward(x) (bf16) it is the unfused form of
 * grkan_layer_forward and gives the same bits.
 */
GRKAN_API grkan_status_t grkan_linear_forward(const void *y, const void *W, void *z, int64_t rows,
                                    int64_t d_in, int64_t d_out, hipStream_t stream);

/*
 * Backward of grkan_layer_forward: given dz = dL/dz (bf16 [rows][d_out]),
 *   dW = dz^T bf16(F(x))       fp32 [d_out][d_in]
 *   dy = bf16(dz W)            (bf16, internal)
 *   dx, dA, dB                 the activation's backward on (x, dy), as
 *                              grkan_backward computes them (bf16 dx,
 *                              deterministic two-stage sums for dA, dB)
 * all on the matrix cores except the activation's own kernels.  bf16(F(x))
 * for dW comes out of the activation's backward kernel, which evaluates F in
 * fp32 from the powers of x it forms anyway (grkan_layer_forward uses Horner's
 * rule): both are correctly rounded fp32 evaluations, so where F lies within
 * fp32 rounding of a bf16 midpoint the two bf16 values may differ by one step.
 * dW sums over all rows: fixed-size row splits are summed in fp32 on the
 * matrix cores and the splits in a fixed order in fp64, so the result is
 * bitwise reproducible.
 *   dx may be x itself; every other output must overlap nothing.
 *   workspace: grkan_layer_backward_workspace_size() bytes, 256-byte aligned.
 *   Limits as grkan_layer_forward, and d_out a multiple of 64.
 *   rows == 0 writes zeros to dA, dB, dW.
 */
GRKAN_API grkan_status_t grkan_layer_backward(const void *x, const void *dz, const float *A,
                                    const float *B, const void *W, void *dx, float *dA,
                                    float *dB, float *dW, int64_t rows, int64_t d_in,
                                    int64_t d_out, int32_t n_groups, void *workspace,
                                    size_t workspace_bytes, hipStream_t stream);

/* Bytes of workspace grkan_layer_backward needs (0 for rows <= 0 or
 * arguments it would reject).  Host-only. */
GRKAN_API size_t grkan_layer_backward_workspace_size(int64_t rows, int64_t d_in, int64_t d_out,
                                           int32_t n_groups);

/*
 * Chebyshev-KAN layer ([PolyKAN]: "PolyKAN: Efficient Fused GPU Operators for
 * Polynomial Kolmogorov-Arnold Network Variants", abstract page, arXiv
 * 2511.14852, whose case study it is):
 *   y[r][o] = sum_i sum_{k=0..D} C[o][i][k] T_k(tanh(x[r][i]))
 * with T_k the Chebyshev polynomials of the first kind.  bf16 x, C, y; the
 * basis is computed in fp32 and rounded to nearest-even bf16 as the matrix
 * operand, products accumulate in fp32 on the matrix cores; the basis is
 * built while x is staged for the product, so it never goes to memory.
 *   x     bf16 [rows][d_in] (2-byte aligned; 16-byte aligned for the backward).
 *   C     bf16 [d_out][d_in][D + 1] (degree fastest), 16-byte aligned.
 *   y     bf16 [rows][d_out]; must not overlap x or C.
 *   degree D = 7 only (8 basis functions; others GRKAN_ERR_UNSUPPORTED);
 *   d_in a multiple of 8; rows >= 0 (0 is a no-op).
 */
GRKAN_API grkan_status_t grkan_chebykan_forward(const void *x, const void *C, void *y, int64_t rows,
                                      int64_t d_in, int64_t d_out, int32_t degree,
                                      hipStream_t stream);

/*
 * Its backward, given dy = dL/dy (bf16 [rows][d_out], 16-byte aligned):
 *   dC[o][i][k] = sum_r dy[r][o] T_k(tanh x[r][i])     fp32 [d_out][d_in][D+1]
 *   dx[r][i]    = (1 - t^2) sum_k T_k'(t) G[r][i][k]   bf16, t = tanh x[r][i]
 * with G = dy C formed on the matrix cores and held in bf16 (as a bf16
 * layer's gradient of its basis), turned into dx by the same kernel (G
 * never goes to memory); dC sums row splits in fp32 and the
 * splits in a fixed order in fp64 (bitwise reproducible).  dx may be x
 * itself; workspace: grkan_chebykan_backward_workspace_size() bytes,
 * 256-byte aligned.  Also needs d_out a multiple of 64.  rows == 0 writes
 * zeros to dC.
 */
GRKAN_API grkan_status_t grkan_chebykan_backward(const void *x, const void *dy, const void *C,
                                       void *dx, float *dC, int64_t rows, int64_t d_in,
                                       int64_t d_out, int32_t degree, void *workspace,
                                       size_t workspace_bytes, hipStream_t stream);

GRKAN_API size_t grkan_chebykan_backward_workspace_size(int64_t rows, int64_t d_in, int64_t d_out,
                                              int32_t degree);

#ifdef __cplusplus
}
#endif

#endif /* GRKAN_H */
