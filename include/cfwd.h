/*
 * cfwd.h -- forward 2-D convolution for CNN inference on one AMD Instinct
 * MI355X (gfx950).  Plain C ABI: no C++ types, no exceptions, no torch types.
 *
 * What is computed (every entry point that writes y):
 *   The forward convolution of CNN inference as the naive loop nest of the
 *   blog post "卷积总结" (convolution summary), section "最原始的卷积实现",
 *   defines it -- a cross-correlation, output[k, oh, ow] = sum over c, r, s of
 *   w[k, c, r, s] * x[c, oh*stride + r*dil - pad, ow*stride + s*dil - pad],
 *   with a batch loop, symmetric zero padding, stride, dilation and groups
 *   (output channel k reads input channels of group k / (K/G) only), and
 *   OH = floor((H + 2*pad_h - dil_h*(R-1) - 1) / stride_h) + 1 (OW likewise).
 *
 * Algorithms (MegEngine inference article, sections "Im2col+MatMul",
 * "Winograd" and "Fast-Run"; Momenta talk "Paper Reading | 讓深度學習更高效運行
 * 的兩個視角", section "優化2：Depthwise卷積" for the depthwise / 1x1 layers):
 *   IMPLICIT_GEMM   im2col x matmul without materialising im2col: input patches
 *                   are staged in LDS and multiplied on the matrix cores.  Its
 *                   last config(s) are the NHWC kernel, the only ones that take
 *                   NHWC problems (and they take nothing else): both operands
 *                   are staged by plain 16-byte copies, the channels of a
 *                   pixel being contiguous.
 *   WINOGRAD_F2X2_3X3 / WINOGRAD_F6X6_3X3
 *                   F(m x m, 3 x 3) minimal filtering for 3x3, stride 1,
 *                   dilation 1, groups 1; float dtypes, and int8 for
 *                   F(2x2) config 0 (below).  bf16 runs its
 *                   transformed operands in fp16 (11 significant bits); to
 *                   keep them in fp16's range, input and filter are scaled by
 *                   powers of two that bring each one's largest magnitude
 *                   (found on the device: the input's on every call, the
 *                   filter's when it is prepared) into [2^7, 2^8), and the
 *                   output is scaled back -- exactly, so any finite
 *                   magnitudes work.  Values below 2^-22 of their tensor's
 *                   largest magnitude become fp16 subnormals and lose
 *                   precision; the Fast-Run accuracy gate sees that on the
 *                   caller's data.
 *                   int8 F(2x2) (MegEngine Beta release article, section
 *                   "业界领先的原生 ARM 推理性能": int8 Winograd with float as
 *                   the intermediate format, no narrowing of the weights):
 *                   B^T d B (multiples of 1/4, |.| <= 512) and G g G^T
 *                   (integers, |.| <= 1152) are fp16 operands, exactly; the
 *                   channel sums and the output transform are fp32, then
 *                   rounded to the nearest integer and requantised as below.
 *                   Exact while every fp32 partial sum stays below 2^22 in
 *                   magnitude; beyond that an output can be 1 away from the
 *                   exact one.  Runs when named explicitly; a Fast-Run
 *                   candidate only after cfwd_fastrun_allow_inexact_int8(1).
 *   DIRECT          direct summation; the depthwise (G = C = K) path.
 *   POINTWISE       1x1 convolution as a low-K matrix product.
 *   AUTO            resolved per problem: a Fast-Run map entry if one exists,
 *                   else (or a search with CFWD_FASTRUN_MODE=search) a fixed
 *                   preference: depthwise -> DIRECT, 1x1 -> POINTWISE, else
 *                   IMPLICIT_GEMM.  Winograd is never chosen without timing.
 *
 * Tensors (all device memory, owned by the caller, 16-byte aligned, dense):
 *   x  activations  NCHW  [N][C][H][W]
 *                   NCHWX [N][ceil(C/x)][H][W][x], x = 4 or 8 (MegEngine
 *                   inference article, section "NCHWX"); channels past C are
 *                   ignored on input.
 *                   NHWC  [N][H][W][C] (channels contiguous; fp32 / bf16, groups
 *                   1, C a multiple of 4 (fp32) or 8 (bf16); runs on the NHWC
 *                   implicit GEMM configs, see IMPLICIT_GEMM).
 *   w  weights      KCRS  [K][C/G][R][S] in every layout, activation dtype.
 *   y  output       same layout and dtype as x, with K channels; in NCHWX the
 *                   channels past K are written as 0.
 *   requant_scale   int8 only: fp32 [K] on the device; the int32 accumulator
 *                   becomes int8 as clamp(rne(fp32(acc) * scale[k]), -127, 127)
 *                   (round to nearest even, symmetric clamp, zero point 0).
 * Dtypes: fp32 (fp32 accumulate), bf16 (fp32 accumulate, output rounded to
 * nearest even), int8 (int32 accumulate, requantised output).
 *
 * Streams: `stream` is a hipStream_t passed as void* (NULL = the default
 * stream).  Calls that only enqueue work return without waiting.
 *
 * Environment (read once per process):
 *   CFWD_FASTRUN_MODE  readonly (default): AUTO takes the Fast-Run map entry,
 *                      else the fixed preference; off: AUTO ignores the map;
 *                      search: a map miss of cfwd_conv2d_fwd with a workspace
 *                      of cfwd_fastrun_workspace_size bytes runs the selection.
 *   CFWD_FASTRUN_CACHE a map file merged into the map before the first AUTO
 *                      resolution; in search mode rewritten after each
 *                      selection.
 *   CFWD_LOG           0 silent (default); 1 every failure's reason on stderr;
 *                      2 also each AUTO resolution and how it was made; 3 also
 *                      the algorithm of every convolution call.
 *
 * Errors: every call returns a cfwd_status; on failure nothing has been
 * enqueued and cfwd_last_error() (per thread) describes why.  Validation
 * failures never touch y.  No call allocates device memory.
 */
#ifndef CFWD_H
#define CFWD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    CFWD_OK = 0,
    CFWD_ERR_INVALID_ARG = 1,  /* bad descriptor, NULL or misaligned pointer */
    CFWD_ERR_UNSUPPORTED = 2,  /* valid problem this algorithm cannot run   */
    CFWD_ERR_WORKSPACE = 3,    /* workspace / prepared buffer too small      */
    CFWD_ERR_NO_CANDIDATE = 4, /* Fast-Run found no candidate passing its gate */
    CFWD_ERR_HIP = 5,          /* a HIP runtime call failed (message kept)   */
    CFWD_ERR_CACHE_IO = 6      /* Fast-Run map file could not be written    */
} cfwd_status;

typedef enum { CFWD_LAYOUT_NCHW = 0, CFWD_LAYOUT_NCHWX = 1, CFWD_LAYOUT_NHWC = 2 } cfwd_layout;

typedef enum { CFWD_F32 = 0, CFWD_BF16 = 1, CFWD_I8 = 2 } cfwd_dtype;

typedef enum {
    CFWD_ALGO_AUTO = 0,
    CFWD_ALGO_IMPLICIT_GEMM = 1,
    CFWD_ALGO_WINOGRAD_F2X2_3X3 = 2,
    CFWD_ALGO_WINOGRAD_F6X6_3X3 = 3,
    CFWD_ALGO_DIRECT = 4,
    CFWD_ALGO_POINTWISE = 5
} cfwd_algo_kind;

/* One convolution problem.  pad_* >= 0; every other integer >= 1;
 * C and K divisible by groups; x is 4 or 8 when layout is NCHWX (ignored for
 * NCHW).  Each of x and y must hold fewer than 2^31 elements per image. */
typedef struct {
    int n, c, h, w, k, r, s;
    int stride_h, stride_w, pad_h, pad_w, dil_h, dil_w, groups;
    cfwd_layout layout;
    int x;
    cfwd_dtype dtype;
} cfwd_conv_desc;

/* An algorithm choice: family, tile configuration within the family
 * (-1 = the family's default for the problem), and the median time Fast-Run
 * measured for it in milliseconds (0 when not measured). */
typedef struct {
    cfwd_algo_kind kind;
    int config_id;
    float median_ms;
} cfwd_algo;

/* Activation of the fused epilogue. */
typedef enum { CFWD_ACT_NONE = 0, CFWD_ACT_RELU = 1 } cfwd_activation;

/* Fused epilogue of cfwd_conv2d_fwd_ex: what a ResNet block applies after
 * its convolution, folded into the convolution's own output pass (Momenta
 * talk "Paper Reading | 讓深度學習更高效運行的兩個視角", section "Graph層面":
 * conv, bias and ReLU computed as one operation, the output written once).
 *   bias      device [K]: fp32 for fp32 / bf16 problems, int32 for int8;
 *             NULL = none.  4-byte aligned.
 *   residual  device tensor of y's shape, layout and dtype (the skip
 *             connection); NULL = none.  16-byte aligned, must not overlap y.
 *   act       CFWD_ACT_NONE or CFWD_ACT_RELU.
 * fp32 / bf16: y = act(conv + bias[k] + residual), in fp32, then one
 *   conversion to the output dtype (bf16: round to nearest even).
 * int8: y = clamp(rne(fp32(acc + bias[k]) * scale[k] + fp32(residual)), lo, 127)
 *   with the bias added to the int32 accumulator (acc + bias must stay in
 *   int32), one fp32 multiply, one fp32 add, ties to even, lo = 0 under ReLU
 *   and -127 otherwise (the residual is taken to be in y's quantised scale). */
typedef struct {
    const void *bias;
    const void *residual;
    cfwd_activation act;
} cfwd_epilogue;

/* Library version string, e.g. "cfwd 0.1.0 gfx950". */
const char *cfwd_version(void);

/* OH, OW of the problem (the floor formula above).  INVALID_ARG if the
 * descriptor is invalid or the window does not fit. */
cfwd_status cfwd_output_dims(const cfwd_conv_desc *desc, int *oh, int *ow);

/* Resolve `algo` (AUTO, or a family with config_id -1) to the concrete
 * (kind, config_id) conv2d_fwd would run.  UNSUPPORTED if the family cannot
 * run this problem. */
cfwd_status cfwd_resolve_algo(const cfwd_conv_desc *desc, cfwd_algo algo, cfwd_algo *resolved);

/* Every (kind, config_id) that can run the problem, in Fast-Run's fixed
 * candidate order (IMPLICIT_GEMM < POINTWISE < DIRECT < WINOGRAD_F2 <
 * WINOGRAD_F6, then config id).  Writes at most `cap` entries to out (out may
 * be NULL when cap is 0) and the total count to *count. */
cfwd_status cfwd_list_candidates(const cfwd_conv_desc *desc, cfwd_algo *out, int cap, int *count);

/* Bytes of the prepared (re-laid-out or transformed) filter the algorithm
 * reads; 0 means it reads the KCRS weights directly. */
cfwd_status cfwd_filter_size(const cfwd_conv_desc *desc, cfwd_algo algo, size_t *bytes);

/* Build the prepared filter of `algo` from KCRS weights into w_prepared
 * (`bytes` >= cfwd_filter_size).  Enqueued on `stream`.  Winograd: the
 * G g G^T filter transform (MegEngine inference article, section "Winograd",
 * step one); implicit GEMM: the weight tile order its matrix-core loop reads
 * (the pack step the article's "融合 PACK" section folds away on the
 * activation side). */
cfwd_status cfwd_prepare_filter(const cfwd_conv_desc *desc, cfwd_algo algo, const void *w_kcrs,
                                void *w_prepared, size_t bytes, void *stream);

/* Workspace bytes conv2d_fwd needs for `algo` when it is given no prepared
 * filter: the prepared filter (built into the workspace first), rounded up to
 * 256 bytes, plus the algorithm's scratch.  0 when none. */
cfwd_status cfwd_workspace_size(const cfwd_conv_desc *desc, cfwd_algo algo, size_t *bytes);

/* Workspace bytes conv2d_fwd needs for `algo` when it is given a prepared
 * filter: the algorithm's scratch only (Winograd: the transformed input
 * tiles B^T d B, alpha^2 x ceil(C / chunk) x tiles x 64 bytes, and for bf16
 * 8 KiB for the input's largest magnitude; implicit GEMM split
 * reductions: their int32 partial tiles).  0 when none. */
cfwd_status cfwd_scratch_size(const cfwd_conv_desc *desc, cfwd_algo algo, size_t *bytes);

/* y = conv(x, w).  w_kcrs is required.  w_prepared may be NULL; when it is
 * not, it must hold cfwd_prepare_filter's output for the same descriptor and
 * resolved algorithm, and the filter is not re-prepared.  requant_scale is
 * required for int8 and must be NULL otherwise.  Enqueued on `stream`. */
cfwd_status cfwd_conv2d_fwd(const cfwd_conv_desc *desc, cfwd_algo algo, const void *x,
                            const void *w_kcrs, const void *w_prepared,
                            const float *requant_scale, void *y, void *workspace,
                            size_t ws_bytes, void *stream);

/* cfwd_conv2d_fwd with a fused epilogue (see cfwd_epilogue; NULL = none,
 * which is exactly cfwd_conv2d_fwd).  Every algorithm and config applies it
 * in its own output pass, so AUTO dispatch from the Fast-Run map works
 * unchanged (the map is chosen on the convolution alone; a
 * CFWD_FASTRUN_MODE=search miss with an epilogue falls back to the fixed
 * preference instead of searching).  INVALID_ARG for an unknown activation,
 * a misaligned bias or residual, or a residual overlapping y. */
cfwd_status cfwd_conv2d_fwd_ex(const cfwd_conv_desc *desc, cfwd_algo algo, const void *x,
                               const void *w_kcrs, const void *w_prepared,
                               const float *requant_scale, const cfwd_epilogue *epilogue, void *y,
                               void *workspace, size_t ws_bytes, void *stream);

/* Scratch capacity of cfwd_conv2d_fwd_noalloc, per device (64 MiB). */
#define CFWD_NOALLOC_SCRATCH_BYTES (64u << 20)

/* Allocation-free variant of cfwd_conv2d_fwd, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Same arguments and result as
 * cfwd_conv2d_fwd without the workspace: what that call takes from the
 * workspace (the prepared filter when w_prepared is NULL, plus the
 * algorithm's scratch -- split-reduction partial tiles, Winograd transformed
 * input) lives instead in a library-owned device array of
 * CFWD_NOALLOC_SCRATCH_BYTES, one per device, held until the process ends.
 * Returns CFWD_ERR_WORKSPACE, enqueuing nothing, when the resolved algorithm
 * needs more than that (cfwd_scratch_size / cfwd_workspace_size tell in
 * advance).  AUTO resolves from the Fast-Run map or the fixed preference,
 * never by a search.  Every call on one device shares that device's array:
 * calls that overlap on one GPU (other streams, other host threads) race on
 * it; calls in one stream are ordered.  No kernel needs the array zeroed --
 * each overwrites what it reads -- so the previous call's contents are
 * harmless.  Allocates nothing, frees nothing. */
cfwd_status cfwd_conv2d_fwd_noalloc(const cfwd_conv_desc *desc, cfwd_algo algo, const void *x,
                                    const void *w_kcrs, const void *w_prepared,
                                    const float *requant_scale, void *y, void *stream);

/* Fast-Run selection phase (MegEngine inference article, section "Fast-Run"):
 * time every candidate of cfwd_list_candidates on this device with these
 * buffers (median of 7 runs after 2 warm-ups; before each run the Infinity
 * Cache and L2 are flushed by overwriting a 512 MiB region of the workspace
 * unless x and y together already exceed that, so candidates are timed from
 * HBM), reject any whose output fails the accuracy gate against the generic
 * DIRECT kernel's result on the same data (for NHWC, run on x converted to
 * NCHW and converted back; bit-identical for int8, except
 * int8 Winograd F(2x2): no output more than 1 away;
 * normalised error <= 1e-5 fp32 except Winograd F(6x6), 1e-3 fp32 F(6x6),
 * 1e-2 bf16; NaN or infinity fails), keep the fastest (times within 1% count
 * as equal and the earlier candidate wins), record it in the map and return
 * it in *best.  Synchronises `stream`; overwrites y.  workspace must hold
 * cfwd_fastrun_workspace_size bytes. */
cfwd_status cfwd_fastrun_select(const cfwd_conv_desc *desc, const void *x, const void *w_kcrs,
                                const float *requant_scale, void *y, void *workspace,
                                size_t ws_bytes, void *stream, cfwd_algo *best);

/* Workspace for cfwd_fastrun_select: the largest candidate workspace, the
 * reference output and error normaliser, and the cache-flush region. */
cfwd_status cfwd_fastrun_workspace_size(const cfwd_conv_desc *desc, size_t *bytes);

/* Fast-Run execution-phase map (host memory, process-wide, thread-safe).
 * lookup: CFWD_OK and *algo when the problem has an entry on this device,
 * UNSUPPORTED otherwise.  load: merge a map file (one record per line); a
 * missing, corrupt or other-device file is ignored with CFWD_OK.
 * save: write the whole map (CACHE_IO on failure).  clear: empty it. */
cfwd_status cfwd_fastrun_lookup(const cfwd_conv_desc *desc, cfwd_algo *algo);
cfwd_status cfwd_fastrun_load(const char *path);
cfwd_status cfwd_fastrun_save(const char *path);
cfwd_status cfwd_fastrun_clear(void);

/* Copy an activation tensor of n x c x h x w elements of `dtype` from one
 * layout to another (NCHW, NHWC, NCHWX with x = src_x / dst_x = 4 or 8; the
 * x arguments are ignored for the others).  NCHWX destinations get their
 * channels past c written as 0; NCHWX sources' are not read.  For networks
 * whose layers prefer different layouts (MegEngine CPU-inference article,
 * section "结论": a network-wide mixed choice of layouts).  src and dst
 * (device, element-aligned) must not overlap.  Enqueued on `stream`. */
cfwd_status cfwd_convert_layout(int n, int c, int h, int w, cfwd_dtype dtype, cfwd_layout src_layout,
                                int src_x, const void *src, cfwd_layout dst_layout, int dst_x, void *dst,
                                void *stream);

/* 4-bit weights (MegEngine CPU-inference article, section "结论": lower-bit
 * quantisation after int8).  gfx950's matrix cores have no int4 operands, so
 * 4-bit weights are stored packed and widened once, when loaded, to the int8
 * KCRS tensor every int8 call takes; results are then the int8 path's, bit
 * for bit.  out_int8[i] = signed value i of `packed`: byte i / 2, low nibble
 * for even i, high nibble for odd i, two's complement (-8 .. 7).  packed
 * holds (count + 1) / 2 bytes and must be 16-byte aligned, out_int8 count
 * bytes, 16-byte aligned, not overlapping packed.  Enqueued on `stream`. */
cfwd_status cfwd_unpack_int4(const void *packed, void *out_int8, long long count, void *stream);

/* Whether int8 candidates whose results are not always bit-identical to the
 * integer ones (int8 Winograd F(2x2), see WINOGRAD_F2X2_3X3 above) take part
 * in cfwd_list_candidates and cfwd_fastrun_select: 0 (the default) = no,
 * nonzero = yes.  Process-wide; an algorithm named explicitly runs either
 * way, and a Fast-Run map entry chosen while they were allowed stays in use. */
cfwd_status cfwd_fastrun_allow_inexact_int8(int allow);

/* The host-side part of Fast-Run's choice, for callers that time candidates
 * themselves (and for testing the rule without a GPU): cands[n] in Fast-Run
 * order, times[n * reps] row-major in ms, gate_ok[n] nonzero when the
 * candidate passed the accuracy gate.  *chosen = index of the candidate with
 * the smallest median time, where a later candidate wins only if its median is
 * more than 1% below the current best's; -1 if none passed. */
cfwd_status cfwd_fastrun_choose(const cfwd_algo *cands, const float *times, int n, int reps,
                                const int *gate_ok, int *chosen);

/* ---- Fused bottleneck block.
 * The ResNet bottleneck (Momenta talk "Paper Reading | 讓深度學習更高效運行的兩個
 * 視角", section "優化1：Bottleneck") as one operation, with the spatial tiling
 * of its section "Operator的粒度": each workgroup computes a band of output
 * rows and keeps the two 64-channel intermediates on chip, so x is read and y
 * written once, with no intermediate tensor in memory.
 *   t1 = act1(conv1x1(x, w1) + b1)            C -> mid
 *   t2 = act2(conv3x3(t1, w2, pad 1) + b2)    mid -> mid
 *   y  = act3(conv1x1(t2, w3) + b3 + residual) mid -> K
 * all stride 1, cross-correlation as above, act = ReLU where asked.
 * t1 and t2 are rounded to bf16 (what three separate bf16 layers store);
 * each stage accumulates in fp32 and applies its epilogue in fp32 before its
 * single rounding.  Supported: bf16, NCHW, mid = 64, C and K multiples of
 * 32, W a multiple of 8 and at most 64, any N and H. */
typedef struct {
    int n, c, h, w; /* x: [N][C][H][W] */
    int mid;        /* channels of the two inner convolutions */
    int k;          /* channels of y: [N][K][H][W] */
    cfwd_dtype dtype;
} cfwd_bottleneck_desc;

/* Per-stage epilogue: fp32 biases b1 [mid], b2 [mid], b3 [K] (NULL = none,
 * 4-byte aligned); residual: bf16 of y's shape added before act3 (NULL =
 * none, 16-byte aligned, must not overlap y); relu1..3 nonzero = ReLU. */
typedef struct {
    const void *b1, *b2, *b3;
    const void *residual;
    int relu1, relu2, relu3;
} cfwd_bottleneck_epilogue;

/* CFWD_OK when the fused kernel runs this block, UNSUPPORTED (reason in
 * cfwd_last_error) when not, INVALID_ARG for a NULL descriptor. */
cfwd_status cfwd_bottleneck_check(const cfwd_bottleneck_desc *desc);

/* Bytes of the prepared 3x3 weights (9 x mid x mid bf16, tap-major). */
cfwd_status cfwd_bottleneck_filter_size(const cfwd_bottleneck_desc *desc, size_t *bytes);

/* Prepare w2 (KCRS [mid][mid][3][3], bf16, device) into w2_prepared
 * (>= cfwd_bottleneck_filter_size bytes, 16-byte aligned).  Enqueued on
 * `stream`. */
cfwd_status cfwd_bottleneck_prepare(const cfwd_bottleneck_desc *desc, const void *w2, void *w2_prepared,
                                    size_t bytes, void *stream);

/* y = the block of x.  w1 KCRS [mid][C][1][1], w3 KCRS [K][mid][1][1] (bf16,
 * device, as given), w2_prepared from cfwd_bottleneck_prepare; epilogue may
 * be NULL (no bias, no residual, no ReLU).  x, w1, w2_prepared, w3, y
 * 16-byte aligned; y must not overlap x or the residual.  Allocates
 * nothing; enqueued on `stream`. */
cfwd_status cfwd_bottleneck_fwd(const cfwd_bottleneck_desc *desc, const void *x, const void *w1,
                                const void *w2_prepared, const void *w3,
                                const cfwd_bottleneck_epilogue *epilogue, void *y, void *stream);

/* Static description of a status code. */
const char *cfwd_status_string(cfwd_status status);

/* Detail of this thread's most recent failure ("" if none). */
const char *cfwd_last_error(void);

/* Name of an algorithm, e.g. "implicit_gemm/3". */
const char *cfwd_algo_name(cfwd_algo algo);

#ifdef __cplusplus
}
#endif

#endif /* CFWD_H */
