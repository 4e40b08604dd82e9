/*
 * CPU oracle for forward 2-D convolution -- TEST INFRASTRUCTURE ONLY.
 *
 * Only the test suite, the package smoke check and the CPU-baseline leg of the
 * benchmark may load this library.  It shares no source, header, table or
 * helper with the GPU library, and the GPU library never calls it.
 *
 * What it computes is the plain definition of a CNN forward convolution, as
 * spelled out by the naive loop nest in the blog post "卷积总结" (convolution
 * summary), section "最原始的卷积实现" (the most primitive convolution):
 *
 *     output[f, oh, ow] += kernel[f, c, kh, kw] * input[c, oh + kh, ow + kw]
 *
 * i.e. a cross-correlation (the input index is the output position plus the
 * kernel offset; the kernel is not flipped), with shapes
 * input [C, H, W], kernel [K, C, R, S], output [K, OH, OW].  The printed
 * listing writes the output index as [filter, channel, out_h, out_h]; the shape
 * comment above it fixes the output as [filter, out_h, out_w], summed over the
 * channel, and that is the reading used here.  The same post, section
 * "卷积的优势" (advantages of convolution), works a 4x4 input with a 2x2 kernel at
 * stride 2 (s1 = a*k1 + b*k2 + e*k3 + f*k4, s2 = c*k1 + d*k2 + g*k3 + h*k4),
 * which fixes how stride enters: input row = oh*stride + kh.
 *
 * Generalised here, as the loop nest's own remark invites (it says a seventh
 * loop covers batches and that stride, dilation and the rest were left out):
 *   - batch n;
 *   - stride (sh, sw), symmetric zero padding (ph, pw) and dilation (dh, dw):
 *       ih = oh*sh - ph + r*dh,   iw = ow*sw - pw + s*dw,
 *     with the input read as 0 outside [0,H) x [0,W);
 *   - groups G: output channel k belongs to group g = k / (K/G) and reads input
 *     channels g*(C/G) .. g*(C/G) + C/G - 1; the kernel is [K, C/G, R, S].
 *   - output size OH = floor((H + 2ph - dh*(R-1) - 1)/sh) + 1 (same for OW).
 *
 * Arithmetic:
 *   - floating point: inputs are given as double (fp32 and bf16 values widen
 *     exactly); every product and sum is an IEEE double operation, summed per
 *     output in the fixed order c' -> r -> s; the library is compiled with
 *     -O2 -fno-fast-math -ffp-contract=off so no FMA contraction or
 *     reassociation changes that.  Alongside y the oracle returns
 *     den = sum |x|*|w| over the same terms, the normaliser of the error metric.
 *   - int8: products are exact integers, accumulated in int64.
 *   - int8 output conversion (the pages name int8 quantised inference but give
 *     no rule; the reading used is:)
 *       y = clamp(rne(fp32(acc) * scale[k]), -127, 127)
 *     with fp32(acc) the IEEE round-to-nearest-even int->float conversion, one
 *     IEEE fp32 multiply (no contraction), rne = rintf under the default
 *     rounding mode (ties to even), a symmetric clamp, zero point 0, no bias.
 *
 * Parallelism: OpenMP over (n, k) output planes only; each plane is summed by
 * one thread in the order above, so results do not depend on the thread count.
 *
 * Parameter block p[14] (all functions): N, C, H, W, K, R, S, sh, sw, ph, pw,
 * dh, dw, G.  Tensors are dense row-major: x [N][C][H][W], w [K][C/G][R][S],
 * y/den/acc [N][K][OH][OW].
 */
#include <math.h>
#include <stdint.h>
#include <stddef.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { PN, PC, PH, PW, PK, PR, PS, PSH, PSW, PPH, PPW, PDH, PDW, PG };

/* Output extent of one spatial dimension; <= 0 means the window does not fit. */
int oracle_output_size(int in, int k, int stride, int pad, int dil)
{
    if (in <= 0 || k <= 0 || stride <= 0 || pad < 0 || dil <= 0)
        return 0;
    long span = (long)in + 2L * pad - (long)dil * (k - 1) - 1;
    if (span < 0)
        return 0;
    return (int)(span / stride) + 1;
}

/* 0 when the parameter block describes a valid problem, -1 otherwise. */
int oracle_check(const int *p)
{
    for (int i = 0; i < 14; ++i)
        if (i != PPH && i != PPW && p[i] <= 0)
            return -1;
    if (p[PPH] < 0 || p[PPW] < 0)
        return -1;
    if (p[PC] % p[PG] != 0 || p[PK] % p[PG] != 0)
        return -1;
    if (oracle_output_size(p[PH], p[PR], p[PSH], p[PPH], p[PDH]) <= 0 ||
        oracle_output_size(p[PW], p[PS], p[PSW], p[PPW], p[PDW]) <= 0)
        return -1;
    return 0;
}

int oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Floating-point convolution in fp64: y and den are [N][K][OH][OW]. */
int oracle_conv2d_f64(const double *x, const double *w, const int *p,
                      double *y, double *den)
{
    if (oracle_check(p))
        return -1;
    const int N = p[PN], C = p[PC], H = p[PH], W = p[PW], K = p[PK];
    const int R = p[PR], S = p[PS], G = p[PG];
    const int sh = p[PSH], sw = p[PSW], ph = p[PPH], pw = p[PPW];
    const int dh = p[PDH], dw = p[PDW];
    const int OH = oracle_output_size(H, R, sh, ph, dh);
    const int OW = oracle_output_size(W, S, sw, pw, dw);
    const int Cg = C / G, Kg = K / G;

#pragma omp parallel for collapse(2) schedule(dynamic)
    for (int n = 0; n < N; ++n) {
        for (int k = 0; k < K; ++k) {
            const int g = k / Kg;
            double *yp = y + ((size_t)n * K + k) * OH * OW;
            double *dp = den + ((size_t)n * K + k) * OH * OW;
            for (int i = 0; i < OH * OW; ++i) {
                yp[i] = 0.0;
                dp[i] = 0.0;
            }
            for (int cc = 0; cc < Cg; ++cc) {
                const int c = g * Cg + cc;
                const double *xp = x + ((size_t)n * C + c) * H * W;
                for (int r = 0; r < R; ++r) {
                    for (int s = 0; s < S; ++s) {
                        const double wv = w[(((size_t)k * Cg + cc) * R + r) * S + s];
                        for (int oh = 0; oh < OH; ++oh) {
                            const int ih = oh * sh - ph + r * dh;
                            if (ih < 0 || ih >= H)
                                continue; /* zero padding contributes 0 */
                            for (int ow = 0; ow < OW; ++ow) {
                                const int iw = ow * sw - pw + s * dw;
                                if (iw < 0 || iw >= W)
                                    continue;
                                const double prod = xp[(size_t)ih * W + iw] * wv;
                                yp[(size_t)oh * OW + ow] += prod;
                                dp[(size_t)oh * OW + ow] += fabs(prod);
                            }
                        }
                    }
                }
            }
        }
    }
    return 0;
}

/* int8 convolution: exact int64 accumulators acc [N][K][OH][OW]. */
int oracle_conv2d_i8(const int8_t *x, const int8_t *w, const int *p, int64_t *acc)
{
    if (oracle_check(p))
        return -1;
    const int N = p[PN], C = p[PC], H = p[PH], W = p[PW], K = p[PK];
    const int R = p[PR], S = p[PS], G = p[PG];
    const int sh = p[PSH], sw = p[PSW], ph = p[PPH], pw = p[PPW];
    const int dh = p[PDH], dw = p[PDW];
    const int OH = oracle_output_size(H, R, sh, ph, dh);
    const int OW = oracle_output_size(W, S, sw, pw, dw);
    const int Cg = C / G, Kg = K / G;

#pragma omp parallel for collapse(2) schedule(dynamic)
    for (int n = 0; n < N; ++n) {
        for (int k = 0; k < K; ++k) {
            const int g = k / Kg;
            int64_t *ap = acc + ((size_t)n * K + k) * OH * OW;
            for (int i = 0; i < OH * OW; ++i)
                ap[i] = 0;
            for (int cc = 0; cc < Cg; ++cc) {
                const int c = g * Cg + cc;
                const int8_t *xp = x + ((size_t)n * C + c) * H * W;
                for (int r = 0; r < R; ++r) {
                    for (int s = 0; s < S; ++s) {
                        const int64_t wv = w[(((size_t)k * Cg + cc) * R + r) * S + s];
                        for (int oh = 0; oh < OH; ++oh) {
                            const int ih = oh * sh - ph + r * dh;
                            if (ih < 0 || ih >= H)
                                continue;
                            for (int ow = 0; ow < OW; ++ow) {
                                const int iw = ow * sw - pw + s * dw;
                                if (iw < 0 || iw >= W)
                                    continue;
                                ap[(size_t)oh * OW + ow] += (int64_t)xp[(size_t)ih * W + iw] * wv;
                            }
                        }
                    }
                }
            }
        }
    }
    return 0;
}

/* One int8 output from its accumulator: clamp(rne(fp32(acc) * scale), -127, 127).
 * acc must fit in int32 (the caller checks); the conversion is the IEEE
 * round-to-nearest-even int32 -> fp32 conversion. */
int8_t oracle_requant_one(int64_t acc, float scale)
{
    const float a = (float)(int32_t)acc;
    const float prod = a * scale; /* one IEEE fp32 multiply; contraction is off */
    const float q = rintf(prod);  /* default rounding mode: ties to even */
    if (q > 127.0f)
        return 127;
    if (q < -127.0f)
        return -127;
    return (int8_t)q;
}

/* Requantise a whole [N][K][HW] accumulator tensor with per-channel scale[K].
 * Returns -1 (and writes nothing) if any accumulator is outside int32. */
int oracle_requant_i8(const int64_t *acc, const float *scale, int N, int K, long HW,
                      int8_t *y)
{
    const size_t total = (size_t)N * K * HW;
    for (size_t i = 0; i < total; ++i)
        if (acc[i] > INT32_MAX || acc[i] < INT32_MIN)
            return -1;
    for (int n = 0; n < N; ++n)
        for (int k = 0; k < K; ++k)
            for (long i = 0; i < HW; ++i) {
                const size_t o = ((size_t)n * K + k) * HW + i;
                y[o] = oracle_requant_one(acc[o], scale[k]);
            }
    return 0;
}

/* Single outputs of the fp64 convolution, for sampled checks at full size.
 * idx holds npts quadruples (n, k, oh, ow). */
int oracle_conv2d_f64_points(const double *x, const double *w, const int *p,
                             long npts, const int64_t *idx, double *y, double *den)
{
    if (oracle_check(p))
        return -1;
    const int C = p[PC], H = p[PH], W = p[PW], K = p[PK];
    const int R = p[PR], S = p[PS], G = p[PG];
    const int sh = p[PSH], sw = p[PSW], ph = p[PPH], pw = p[PPW];
    const int dh = p[PDH], dw = p[PDW];
    const int OH = oracle_output_size(H, R, sh, ph, dh);
    const int OW = oracle_output_size(W, S, sw, pw, dw);
    const int Cg = C / G, Kg = K / G;
    for (long i = 0; i < npts; ++i) {
        const int64_t n = idx[4 * i], k = idx[4 * i + 1];
        const int64_t oh = idx[4 * i + 2], ow = idx[4 * i + 3];
        if (n < 0 || n >= p[PN] || k < 0 || k >= K || oh < 0 || oh >= OH || ow < 0 || ow >= OW)
            return -1;
    }
#pragma omp parallel for schedule(dynamic)
    for (long i = 0; i < npts; ++i) {
        const int64_t n = idx[4 * i], k = idx[4 * i + 1];
        const int64_t oh = idx[4 * i + 2], ow = idx[4 * i + 3];
        const int g = (int)(k / Kg);
        double acc = 0.0, dacc = 0.0;
        for (int cc = 0; cc < Cg; ++cc) {
            const int c = g * Cg + cc;
            for (int r = 0; r < R; ++r) {
                const int64_t ih = oh * sh - ph + (int64_t)r * dh;
                for (int s = 0; s < S; ++s) {
                    const int64_t iw = ow * sw - pw + (int64_t)s * dw;
                    if (ih < 0 || ih >= H || iw < 0 || iw >= W)
                        continue;
                    const double prod = x[(((size_t)n * C + c) * H + ih) * W + iw] *
                                        w[(((size_t)k * Cg + cc) * R + r) * S + s];
                    acc += prod;
                    dacc += fabs(prod);
                }
            }
        }
        y[i] = acc;
        den[i] = dacc;
    }
    return 0;
}

/* Single outputs of the int8 convolution (exact int64 accumulators). */
int oracle_conv2d_i8_points(const int8_t *x, const int8_t *w, const int *p,
                            long npts, const int64_t *idx, int64_t *acc)
{
    if (oracle_check(p))
        return -1;
    const int C = p[PC], H = p[PH], W = p[PW], K = p[PK];
    const int R = p[PR], S = p[PS], G = p[PG];
    const int sh = p[PSH], sw = p[PSW], ph = p[PPH], pw = p[PPW];
    const int dh = p[PDH], dw = p[PDW];
    const int OH = oracle_output_size(H, R, sh, ph, dh);
    const int OW = oracle_output_size(W, S, sw, pw, dw);
    const int Cg = C / G, Kg = K / G;
    for (long i = 0; i < npts; ++i) {
        const int64_t n = idx[4 * i], k = idx[4 * i + 1];
        const int64_t oh = idx[4 * i + 2], ow = idx[4 * i + 3];
        if (n < 0 || n >= p[PN] || k < 0 || k >= K || oh < 0 || oh >= OH || ow < 0 || ow >= OW)
            return -1;
    }
#pragma omp parallel for schedule(dynamic)
    for (long i = 0; i < npts; ++i) {
        const int64_t n = idx[4 * i], k = idx[4 * i + 1];
        const int64_t oh = idx[4 * i + 2], ow = idx[4 * i + 3];
        const int g = (int)(k / Kg);
        int64_t a = 0;
        for (int cc = 0; cc < Cg; ++cc) {
            const int c = g * Cg + cc;
            for (int r = 0; r < R; ++r) {
                const int64_t ih = oh * sh - ph + (int64_t)r * dh;
                for (int s = 0; s < S; ++s) {
                    const int64_t iw = ow * sw - pw + (int64_t)s * dw;
                    if (ih < 0 || ih >= H || iw < 0 || iw >= W)
                        continue;
                    a += (int64_t)x[(((size_t)n * C + c) * H + ih) * W + iw] *
                         (int64_t)w[(((size_t)k * Cg + cc) * R + r) * S + s];
                }
            }
        }
        acc[i] = a;
    }
    return 0;
}

/*
 * Fused epilogue.  The Momenta talk (section "Graph層面") folds the bias add
 * and the ReLU that follow a convolution into the convolution itself, so the
 * output is written once.  What is computed is the tail of a ResNet block in
 * inference: a per-output-channel bias (the folded batch norm), then the
 * skip connection (a residual tensor of the output's shape), then the
 * activation.  Reading taken (the pages give no formula):
 *
 *   float: y = act(conv + bias[k] + residual), every step in fp64, and the
 *          error normaliser grows by the absolute values of the added
 *          terms: den' = den + |bias[k]| + |residual|.
 *   int8:  y = clamp(rne(fp32(acc + bias[k]) * scale[k] + fp32(residual)), lo, 127)
 *          with acc + bias an exact integer sum (it must fit in int32), the
 *          IEEE int32 -> fp32 conversion, one fp32 multiply, one fp32 add
 *          (no contraction), ties to even, lo = 0 with ReLU and -127 without.
 *
 * bias / residual may be NULL (absent); act is 0 (none) or 1 (ReLU).
 */

/* In place on y and den, both [N][K][HW]; bias [K], residual [N][K][HW]. */
int oracle_epilogue_f64(double *y, double *den, const double *bias, const double *res, int relu,
                        int N, int K, long HW)
{
    for (int n = 0; n < N; ++n)
        for (int k = 0; k < K; ++k)
            for (long i = 0; i < HW; ++i) {
                const size_t o = ((size_t)n * K + k) * HW + i;
                double v = y[o];
                double d = den[o];
                if (bias) {
                    v += bias[k];
                    d += fabs(bias[k]);
                }
                if (res) {
                    v += res[o];
                    d += fabs(res[o]);
                }
                if (relu && v < 0.0)
                    v = 0.0;
                y[o] = v;
                den[o] = d;
            }
    return 0;
}

/* One int8 output of the fused epilogue (see above).  acc + bias must fit in
 * int32 (the caller checks). */
int8_t oracle_requant_epi_one(int64_t acc, float scale, int64_t bias, int has_res, int8_t res, int relu)
{
    const float a = (float)(int32_t)(acc + bias);
    float q = a * scale; /* one IEEE fp32 multiply */
    if (has_res)
        q = q + (float)res; /* one IEEE fp32 add */
    q = rintf(q);
    const float lo = relu ? 0.0f : -127.0f;
    if (q > 127.0f)
        return 127;
    if (q < lo)
        return (int8_t)lo;
    return (int8_t)q;
}

/* Whole tensors: acc and res [N][K][HW], scale [K], bias [K] (int32, or
 * NULL), res (or NULL).  Returns -1, writing nothing, if any acc + bias is
 * outside int32. */
int oracle_requant_epi_i8(const int64_t *acc, const float *scale, const int32_t *bias, const int8_t *res,
                          int relu, int N, int K, long HW, int8_t *y)
{
    for (int n = 0; n < N; ++n)
        for (int k = 0; k < K; ++k)
            for (long i = 0; i < HW; ++i) {
                const size_t o = ((size_t)n * K + k) * HW + i;
                const int64_t s = acc[o] + (bias ? bias[k] : 0);
                if (s > INT32_MAX || s < INT32_MIN)
                    return -1;
            }
    for (int n = 0; n < N; ++n)
        for (int k = 0; k < K; ++k)
            for (long i = 0; i < HW; ++i) {
                const size_t o = ((size_t)n * K + k) * HW + i;
                y[o] = oracle_requant_epi_one(acc[o], scale[k], bias ? bias[k] : 0, res != NULL,
                                              res ? res[o] : 0, relu);
            }
    return 0;
}
