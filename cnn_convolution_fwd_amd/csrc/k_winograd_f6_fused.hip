// Fused Winograd F(6x6, 3x3) for NCHW activations, bf16 or fp32 (gfx950).
//
// MegEngine inference article, section "Winograd": F(6x6,3x3) computes a 6x6
// output tile from an 8x8 input tile with 64 multiplies instead of 324, in
// three steps (transform input and weights, multiply the transformed tiles
// as a batched matrix product over the 64 positions, transform back); its
// engineering subsection blocks the tiles so that one block's transformed
// data is consumed while it is still close to the core.
//
// Here the transformed input never reaches HBM.  A workgroup (four waves,
// one per SIMD) owns up to 32 output tiles -- TR tile rows of TCB tiles,
// the tile rows taken consecutively across the batch -- and 32 output
// channels, for all 64 positions, and walks the input channels in steps of
// 16 (bf16) or 8 (fp32):
//   * staging: the 8 input rows of each of its tile rows (6 TCB + 2 columns,
//     widened to whole 16-byte loads) are loaded one step ahead with 16-byte
//     buffer loads -- pixels outside the image are given an offset past the
//     buffer's end and read as zero -- and written to LDS as planes of one
//     channel pair (bf16: converted to fp16 pairs after a power-of-two scale
//     into fp16's range) or one channel (fp32: copied);
//   * input transform: thread (tile slot, plane) reads its 8x8 window and
//     forms U = B^T d B in registers (packed fp16 for bf16, fp32 otherwise);
//     the rows of B^T are rescaled so that every entry is a small dyadic
//     number and rows 2p-1, 2p share their even-column part and negate their
//     odd-column part, which makes an 8-point transform 26 operations; after
//     a barrier U goes to LDS in the matrix cores' A-operand order;
//   * batched product: wave w owns Winograd rows 2w and 2w+1 (16 positions)
//     and multiplies U[xi] (32 tiles x the step's channels) by the prepared
//     filter V[xi] (read from L2 and reloaded for the next step right after
//     use) on v_mfma_f32_32x32x16_f16 (bf16) or four v_mfma_f32_32x32x2f32
//     (fp32): 16 positions x 32 tiles x 32 channels = 256 fp32 accumulators
//     per lane.  A step's products run in the same stretch of code as the
//     next step's transform;
//   * output transform: the accumulators go through LDS in two slices of 16
//     output channels, and each thread forms Y = A^T M A for (tile, channel)
//     pairs and writes the cropped 6x6 tile to the output.
// Scaling: with the rescaled B^T each row's absolute sum is at most 15, so
// |U| <= 225 max|d|; bf16 inputs are scaled so that max|x| < 256, which keeps
// U below 57600 (fp16 holds up to 65504).  G's rows carry the inverse row
// factors, so (G g G^T) * (B^T d B) is unchanged elementwise.
#include "igemm_impl.h"
#include "winograd_mats.h"
#include "winograd_f6_fused.h"

namespace cfwd {
namespace wf6 {

using ig::f32x16;
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int TB = 32;                  // tile slots per workgroup (rows of the products)
constexpr int KB = 32;                  // output channels per workgroup
constexpr int NTHR = 256;               // four waves
constexpr int XPW = 16;                 // positions per wave
constexpr int KS = 16;                  // output channels per slice of the output transform
constexpr int MP = 36;                  // LDS pitch (floats) of one (position, channel) row of 32 tiles
constexpr int M_LDS = 64 * KS * MP * 4;
constexpr int LDS_MAX = 160 * 1024;

// ---------------------------------------------------------------- matrices

struct F6 {
    float bs[8][8];  // B^T with row i multiplied by s_i = 1 / B^T[i][6] (1 where that entry is 0)
    float gs[8][3];  // G with row i divided by s_i
    float at[6][8];  // A^T
};

constexpr double round64(double v) {  // nearest multiple of 1/64
    const double t = v * 64.0;
    const long long r = t < 0 ? -static_cast<long long>(-t + 0.5) : static_cast<long long>(t + 0.5);
    return static_cast<double>(r) / 64.0;
}

constexpr double row_scale(const wg::Mats<6>& m, int i) { return m.bt[i][6] != 0.0 ? 1.0 / m.bt[i][6] : 1.0; }

constexpr F6 build_f6() {
    constexpr wg::Mats<6> m = wg::build_mats<6>();
    F6 f{};
    for (int i = 0; i < 8; ++i) {
        const double s = row_scale(m, i);
        for (int k = 0; k < 8; ++k) f.bs[i][k] = static_cast<float>(round64(m.bt[i][k] * s));
        for (int r = 0; r < 3; ++r) f.gs[i][r] = static_cast<float>(m.g[i][r] / s);
    }
    for (int p = 0; p < 6; ++p)
        for (int q = 0; q < 8; ++q) f.at[p][q] = static_cast<float>(m.at[p][q]);
    return f;
}

constexpr F6 kF6 = build_f6();

constexpr bool check_f6() {
    constexpr wg::Mats<6> m = wg::build_mats<6>();
    double maxrow = 0.0;
    for (int i = 0; i < 8; ++i) {
        double rs = 0.0;
        for (int k = 0; k < 8; ++k) {
            // the rescaled entries are dyadic (exact in fp16)
            const double d = m.bt[i][k] * row_scale(m, i) - kF6.bs[i][k];
            if (d > 1e-9 || d < -1e-9) return false;
            rs += kF6.bs[i][k] < 0 ? -kF6.bs[i][k] : kF6.bs[i][k];
        }
        if (rs > maxrow) maxrow = rs;
    }
    // fp16 range: |U| <= maxrow^2 * 256
    if (maxrow * maxrow * 256.0 >= 65504.0) return false;
    // rows 2p-1 and 2p of B^T (p = 1..3): equal on even columns, opposite on odd ones
    for (int p = 1; p < 7; p += 2)
        for (int k = 0; k < 8; ++k) {
            const float a = kF6.bs[p][k], b = kF6.bs[p + 1][k];
            if ((k & 1) ? (a != -b) : (a != b)) return false;
        }
    // columns 2k-1 and 2k of A^T (k = 1..3): equal on even rows, opposite on
    // odd rows; column 1 is all ones; column 0 only in row 0, column 7 only in row 5
    for (int k = 1; k < 7; k += 2)
        for (int p = 0; p < 6; ++p) {
            const float a = kF6.at[p][k], b = kF6.at[p][k + 1];
            if ((p & 1) ? (a != -b) : (a != b)) return false;
        }
    for (int p = 0; p < 6; ++p) {
        if (kF6.at[p][1] != 1.0f) return false;
        if ((p == 0) ? kF6.at[p][0] != 1.0f : kF6.at[p][0] != 0.0f) return false;
        if ((p == 5) ? kF6.at[p][7] != 1.0f : kF6.at[p][7] != 0.0f) return false;
    }
    return true;
}
static_assert(check_f6(), "F(6,3) transforms do not have the structure the kernel relies on");

// ---------------------------------------------------------------- transforms

template <typename T> struct Op;
template <> struct Op<bf16_t> {
    using V = h2;  // a channel pair
    static __device__ __forceinline__ V splat(float c) {
        const _Float16 v = static_cast<_Float16>(c);
        return V{v, v};
    }
    static __device__ __forceinline__ V splat_bits(uint32_t b) { return __builtin_bit_cast(V, b); }
};
template <> struct Op<float> {
    using V = float;
    static __device__ __forceinline__ V splat(float c) { return c; }
    static __device__ __forceinline__ V splat_bits(uint32_t b) { return __uint_as_float(b); }
};

// The rescaled B^T has the form the transforms below are written for:
//   row 0:           d6 - d0 + c (d2 - d4)          row 7: d7 - d1 + c (d3 - d5)
//   rows P, P+1 (P = 1, 3, 5): E +- s O with E = d6 + a d2 + b d4 and
//   O = d1 + g d3 + e d5
struct PairCoef {
    float a, b, g, e, s;
};
constexpr PairCoef pair_coef(int P) {
    const float s = kF6.bs[P][1];
    return PairCoef{kF6.bs[P][2], kF6.bs[P][4], kF6.bs[P][3] / s, kF6.bs[P][5] / s, s};
}
constexpr bool check_form() {
    const float c = kF6.bs[0][2];
    const float r0[8] = {-1, 0, c, 0, -c, 0, 1, 0};
    const float r7[8] = {0, -1, 0, c, 0, -c, 0, 1};
    for (int k = 0; k < 8; ++k)
        if (kF6.bs[0][k] != r0[k] || kF6.bs[7][k] != r7[k]) return false;
    for (int P = 1; P < 7; P += 2) {
        const PairCoef q = pair_coef(P);
        for (int sg = 0; sg < 2; ++sg) {
            const float ss = sg ? -q.s : q.s;
            const float r[8] = {0, ss, q.a, ss * q.g, q.b, ss * q.e, 1, 0};
            for (int k = 0; k < 8; ++k)
                if (kF6.bs[P + sg][k] != r[k]) return false;
        }
    }
    return true;
}
static_assert(check_form(), "rescaled B^T does not have the factored form");

// d <- (rescaled B^T) d for one 8-point line: 24 operations
template <typename T>
__device__ __forceinline__ void bt8(typename Op<T>::V (&d)[8]) {
    using O = Op<T>;
    typename O::V o[8];
    const auto c = O::splat(kF6.bs[0][2]);
    o[0] = c * (d[2] - d[4]) + (d[6] - d[0]);
    o[7] = c * (d[3] - d[5]) + (d[7] - d[1]);
#pragma unroll
    for (int P = 1; P < 7; P += 2) {
        const PairCoef q = pair_coef(P);
        const auto e = O::splat(q.b) * d[4] + (O::splat(q.a) * d[2] + d[6]);
        const auto od = O::splat(q.e) * d[5] + (O::splat(q.g) * d[3] + d[1]);
        o[P] = O::splat(q.s) * od + e;
        o[P + 1] = O::splat(-q.s) * od + e;
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) d[k] = o[k];
}

// o = A^T m for one 8-point line (fp32): sums and differences of the column
// pairs, then two multiply-adds per output
__device__ __forceinline__ void at8(const float (&m)[8], float (&o)[6]) {
    const float s1 = m[1] + m[2], d1 = m[1] - m[2];
    const float s2 = m[3] + m[4], d2 = m[3] - m[4];
    const float s3 = m[5] + m[6], d3 = m[5] - m[6];
#pragma unroll
    for (int p = 0; p < 6; ++p) {
        float acc = (p & 1) ? d1 : s1;
        acc = fmaf(kF6.at[p][3], (p & 1) ? d2 : s2, acc);
        acc = fmaf(kF6.at[p][5], (p & 1) ? d3 : s3, acc);
        if (p == 0) acc += m[0];
        if (p == 5) acc += m[7];
        o[p] = acc;
    }
}

// ---------------------------------------------------------------- kernel

struct Args {
    const uint8_t* x;  // NCHW input
    const uint8_t* v;  // prepared filter
    uint8_t* y;        // NCHW output
    int C, H, W, K, OH, OW, ph, pw;
    long long x_img, y_img;  // elements per image
    int x_bytes;             // bytes of the whole input (< 2 GiB): the buffer bound
    int v_bytes;             // bytes of the prepared filter (< 2 GiB)
    int th, tw, NR;          // tile rows and columns per image; tile rows in the batch
    int tcb, tr;             // tile block: tr tile rows of tcb tiles
    int nrb, ncb, ntk, nchunks, nsteps;
    int kgrp;                // filter slices per group of the work order (divides ntk)
    int nbk, nunits;         // 16-byte load blocks per patch row; staging units
    int nbkp, rp, sk;        // patch layout (16-byte slots): block pitch, row pitch, skew per tile row
    int patch_bytes;         // one patch buffer
    Epi e;
    // bf16: largest input / filter magnitudes (bit patterns), for the fp16 scaling
    const unsigned* xmax;
    const unsigned* wmax;
};

__device__ __forceinline__ uint32_t word_of(const uint4& v, int i) {
    return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

// fp16 pair (lo: channel of wlo, hi: channel of whi) of the bf16 half p of
// the two words, times the power-of-two scale sc.  bf16 values in fp16's
// normal range convert exactly, so rounding toward zero is exact there.
__device__ __forceinline__ uint32_t bf16_pair_to_f16(uint32_t wlo, uint32_t whi, int p, float sc) {
    const float flo = __uint_as_float(p ? (wlo & 0xffff0000u) : (wlo << 16)) * sc;
    const float fhi = __uint_as_float(p ? (whi & 0xffff0000u) : (whi << 16)) * sc;
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(flo, fhi));
}

template <typename T>
__device__ __forceinline__ void mma(f32x16& c, const uint4& a, const uint4& b, int i) {
    if constexpr (sizeof(T) == 2) {
        c = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0, 0,
                                                   0);
    } else {
        c = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(word_of(a, i)), __uint_as_float(word_of(b, i)), c, 0,
                                                 0, 0);
    }
}

template <bool B> struct BoolC {
    static constexpr bool value = B;
};

// MAXU: staging units per thread at most; EPI: fused epilogue compiled in.
template <typename T, int MAXU, bool EPI>
__global__ __launch_bounds__(NTHR) void wf6_kernel(Args a) {
    constexpr bool BF = sizeof(T) == 2;
    constexpr int ES = static_cast<int>(sizeof(T));
    constexpr int E = 16 / ES;  // pixels per 16-byte load; channels per staging slot
    using O = Op<T>;
    using V = typename O::V;
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lrow = lane & 31;
    const int h = lane >> 5;
    const float xsc = BF ? wg_norm(a.xmax) : 1.0f;  // bf16: input scale into the fp16 range

    // work order: groups of kgrp filter slices are the slowest index and the
    // slice within a group the fastest, so each XCD's contiguous range of
    // blocks shares kgrp slices in its L2 and reads each input patch once
    // from beyond it for the kgrp slices
    int lin = xcd_linear(static_cast<int>(blockIdx.x), static_cast<int>(gridDim.x));
    const int nblk = a.nrb * a.ncb;
    const int kg = lin / (nblk * a.kgrp);
    lin -= kg * nblk * a.kgrp;
    const int kt = kg * a.kgrp + lin % a.kgrp;
    lin /= a.kgrp;
    const int cb = lin % a.ncb;
    const int rb = lin / a.ncb;
    const int R0 = rb * a.tr;        // first tile row of the block (over the batch)
    const int tc0 = cb * a.tcb;      // first tile column
    const int cw0 = 6 * tc0 - a.pw;  // first window column
    const int cs = cw0 >= 0 ? (cw0 / E) * E : -((-cw0 + E - 1) / E) * E;  // staged from here (16-byte aligned)
    const int off = cw0 - cs;
    const int HW = a.H * a.W;
    const int PH = 8 * a.tr;  // patch rows

    // ---- patch: two buffers of 16-byte slots, one per (half h, patch row r,
    // pixel p), holding the step's channels 8h .. 8h+7 as fp16 (bf16) or its
    // four fp32 channels of half h, at slot
    //   (h PH + r) rp + (h TR + r / 8) sk + (p % E) nbkp + p / E
    // -- pixel p % E of every 16-byte load block together, so the E stores
    // of the staging units run through consecutive slots across the lanes,
    // and an odd row pitch and a skew per tile row spread the window reads
    // over the banks -- then a 128-byte area that staging threads without a
    // unit write into
    const int dummy = 2 * a.patch_bytes;
    // staging units (half j, patch row pr, 16-byte column block cbk), cbk fastest
    int u_voff[MAXU];  // byte offset of the unit's first channel (none / outside the image: past the bound)
    int u_lds[MAXU];   // byte offset in a patch buffer (no unit: -1)
#pragma unroll
    for (int i = 0; i < MAXU; ++i) {
        const int u = tid + i * NTHR;
        const bool has = u < a.nunits;
        const int cbk = u % a.nbk;
        const int t = u / a.nbk;
        const int pr = t % PH;
        const int j = t / PH;
        const int R = R0 + (pr >> 3);
        const int n = R / a.th;
        const int ih = 6 * (R - n * a.th) - a.ph + (pr & 7);
        const int iw = cs + cbk * E;
        const bool in = has && R < a.NR && static_cast<unsigned>(ih) < static_cast<unsigned>(a.H) &&
                        static_cast<unsigned>(iw) < static_cast<unsigned>(a.W);
        u_voff[i] = in ? static_cast<int>((n * a.x_img + static_cast<long long>(8 * j) * HW +
                                           static_cast<long long>(ih) * a.W + iw) * ES)
                       : static_cast<int>(0x80000000u);
        u_lds[i] = has ? ((j * PH + pr) * a.rp + (j * a.tr + (pr >> 3)) * a.sk + cbk) * 16 : -1;
    }
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(a.x), 0, a.x_bytes, 0x00020000);
    // one step's staged data: bf16 loads 8 channels x 8 pixels per unit and
    // converts them in place to 8 pixels x 8 fp16 channels; fp32 loads 4
    // channels x 4 pixels, stored transposed (4 pixels x 4 channels)
    uint4 stg[MAXU][8];
    // units [i0, i1) of the thread
    auto stage_load = [&](int st, int i0, int i1) __attribute__((always_inline)) {
        // channels of step st: bf16 16 st + 8 j + e; fp32 16 (st/2) + 8 j + 4 (st%2) + e
        const int cbase = BF ? st * 16 : (st >> 1) * 16 + (st & 1) * 4;
        const int soff = cbase * HW * ES;
#pragma unroll
        for (int i = i0; i < i1; ++i)
#pragma unroll
            for (int e = 0; e < E; ++e) {
                // lane part in the vector offset, the step's channel part in the scalar
                // one (a unit outside the image stays past the bound either way)
                const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rs, u_voff[i], soff + e * HW * ES, 0);
                stg[i][e] = make_uint4(v.x, v.y, v.z, v.w);
            }
    };
    auto stage_convert = [&](int i0, int i1) __attribute__((always_inline)) {
#pragma unroll
        for (int i = i0; i < i1; ++i) {
            uint4 o[8];
            if constexpr (BF) {
#pragma unroll
                for (int x = 0; x < 8; ++x) {
                    uint32_t w[4];
#pragma unroll
                    for (int p = 0; p < 4; ++p)
                        w[p] = bf16_pair_to_f16(word_of(stg[i][2 * p], x >> 1),
                                                    word_of(stg[i][2 * p + 1], x >> 1), x & 1, xsc);
                    o[x] = make_uint4(w[0], w[1], w[2], w[3]);
                }
            } else {
#pragma unroll
                for (int x = 0; x < 4; ++x)
                    o[x] = make_uint4(word_of(stg[i][0], x), word_of(stg[i][1], x), word_of(stg[i][2], x),
                                      word_of(stg[i][3], x));
            }
#pragma unroll
            for (int x = 0; x < E; ++x) stg[i][x] = o[x];
        }
    };
    auto stage_store = [&](int buf, int i0, int i1) __attribute__((always_inline)) {
#pragma unroll
        for (int i = i0; i < i1; ++i) {
            uint8_t* base = lds + (u_lds[i] >= 0 ? buf + u_lds[i] : dummy);
            const int xs = u_lds[i] >= 0 ? a.nbkp * 16 : 16;
#pragma unroll
            for (int x = 0; x < E; ++x) *reinterpret_cast<uint4*>(base + xs * x) = stg[i][x];
        }
    };

    // ---- transform: lane (tile slot lrow, half h) forms this wave's two
    // Winograd rows -- (1,2), (3,4), (5,6) for waves 0-2, (0,7) for wave 3 --
    // for the four units (bf16 channel pairs, fp32 channels) of half h
    const int tr_ = lrow / a.tcb;
    const bool slot_ok = lrow < a.tr * a.tcb;
    const int trw = slot_ok ? tr_ : 0, tcw = slot_ok ? lrow - tr_ * a.tcb : 0;
    // byte offset of the window's column j (row 0 of the window)
    const int px0 = off + 6 * tcw;
    const int wrow = ((h * PH + 8 * trw) * a.rp + (h * a.tr + trw) * a.sk) * 16;
    const int nbkp16 = a.nbkp * 16;
    auto wcol = [&](int j) __attribute__((always_inline)) { return wrow + ((px0 + j) & (E - 1)) * nbkp16 + ((px0 + j) / E) * 16; };
    const int rpb = a.rp * 16;  // bytes per patch row
    const int P = 2 * wave + 1;  // first row of the pair (waves 0-2)
    const PairCoef c1 = pair_coef(1), c3 = pair_coef(3), c5 = pair_coef(5);
    const V ca = O::splat(wave == 0 ? c1.a : wave == 1 ? c3.a : c5.a);
    const V cbb = O::splat(wave == 0 ? c1.b : wave == 1 ? c3.b : c5.b);
    const V cg = O::splat(wave == 0 ? c1.g : wave == 1 ? c3.g : c5.g);
    const V ce = O::splat(wave == 0 ? c1.e : wave == 1 ? c3.e : c5.e);
    const V csp = O::splat(wave == 0 ? c1.s : wave == 1 ? c3.s : c5.s);
    const V csn = O::splat(wave == 0 ? -c1.s : wave == 1 ? -c3.s : -c5.s);
    const V c07 = O::splat(kF6.bs[0][2]);
    V t[2][8][4];  // [row of the pair][window column][unit], then U in place
    // column pass: t[r][j] = (row r of the rescaled B^T) . d[.][j]
    // Two passes over the window's columns, even rows then odd rows (one
    // column ahead in registers): the pair waves form E (rows 2, 4, 6) and
    // O (rows 1, 3, 5) and then E +- s O; wave 3 forms row 0 from the even
    // rows and row 7 from the odd ones.  W3: wave 3's code or the pair waves'.
    auto column_loop = [&](auto w3c, int buf) __attribute__((always_inline)) {
        constexpr bool W3 = decltype(w3c)::value;
        const uint8_t* src = lds + buf;
#pragma unroll
        for (int par = 0; par < 2; ++par) {
            // rows of this pass: wave 3 par, par+2, par+4, par+6; pairs 2-par, 4-par, 6-par
            constexpr int NRW = W3 ? 4 : 3;
            const int r0 = W3 ? par : 2 - par;
            uint4 dc[4], dn[4];
#pragma unroll
            for (int k = 0; k < NRW; ++k) dc[k] = *reinterpret_cast<const uint4*>(src + (r0 + 2 * k) * rpb + wcol(0));
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                if (j < 7) {
#pragma unroll
                    for (int k = 0; k < NRW; ++k)
                        dn[k] = *reinterpret_cast<const uint4*>(src + (r0 + 2 * k) * rpb + wcol(j + 1));
                }
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    V dv[4];
#pragma unroll
                    for (int k = 0; k < NRW; ++k) dv[k] = O::splat_bits(word_of(dc[k], u));
                    if constexpr (W3) {
                        // rows (0 2 4 6) or (1 3 5 7): c (d[1] - d[2]) + (d[3] - d[0])
                        t[par][j][u] = c07 * (dv[1] - dv[2]) + (dv[3] - dv[0]);
                    } else if (par == 0) {
                        // rows 2 4 6: E = b d4 + (a d2 + d6)
                        t[0][j][u] = cbb * dv[1] + (ca * dv[0] + dv[2]);
                    } else {
                        // rows 1 3 5: O = e d5 + (g d3 + d1)
                        t[1][j][u] = ce * dv[2] + (cg * dv[1] + dv[0]);
                    }
                }
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int k = 0; k < NRW; ++k) dc[k] = dn[k];
            }
        }
        if constexpr (!W3) {
#pragma unroll
            for (int j = 0; j < 8; ++j)
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const V ev = t[0][j][u], od = t[1][j][u];
                    t[0][j][u] = csp * od + ev;
                    t[1][j][u] = csn * od + ev;
                }
        }
    };
    auto column_pass = [&](int buf) __attribute__((always_inline)) {
        if (wave == 3)
            column_loop(BoolC<true>{}, buf);
        else
            column_loop(BoolC<false>{}, buf);
    };
    // row pass of row r: U[r][c] = sum_j t[r][j] B^T[c][j]
    auto row_pass = [&](int r) __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            V line[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) line[j] = t[r][j][u];
            bt8<T>(line);
#pragma unroll
            for (int j = 0; j < 8; ++j) t[r][j][u] = line[j];
        }
    };
    auto a_op = [&](int r, int c) __attribute__((always_inline)) {
        return make_uint4(__builtin_bit_cast(uint32_t, t[r][c][0]), __builtin_bit_cast(uint32_t, t[r][c][1]),
                          __builtin_bit_cast(uint32_t, t[r][c][2]), __builtin_bit_cast(uint32_t, t[r][c][3]));
    };

    // ---- product: position x of this wave = (row x / 8 of its pair, column
    // x % 8); prepared filter V[xi][kt][chunk][piece][32 rows][half][16 B],
    // step st = 2 chunk + piece
    const int ra = wave == 3 ? 0 : P, rbw = wave == 3 ? 7 : P + 1;
    // (a buffer resource over the prepared filter: the lane's part of an
    // offset in a vector register, the position and step part in a scalar one)
    const int vxs = a.ntk * a.nchunks * 2048;
    const __amdgpu_buffer_rsrc_t rv =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(a.v), 0, a.v_bytes, 0x00020000);
    const int vlane = lrow * 32 + h * 16;
    const int vrow0 = 8 * ra * vxs + kt * a.nchunks * 2048, vrow1 = 8 * rbw * vxs + kt * a.nchunks * 2048;
    // filter operands: a ring of 8 -- slot c holds row ra's column c, then
    // (after its products) row rbw's column c, then the next step's row ra
    uint4 vr[8];
    f32x16 acc[XPW];
#pragma unroll
    for (int x = 0; x < XPW; ++x) acc[x] = f32x16{};
    auto load_v = [&](int r, int c, int st) __attribute__((always_inline)) {
        const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rv, vlane, (r ? vrow1 : vrow0) + c * vxs + st * 1024, 0);
        vr[c] = make_uint4(v.x, v.y, v.z, v.w);
    };
    // the products of row r of the pair for step st; the ring reloads with
    // (row 1, step st) after row 0 and (row 0, step st_next) after row 1
    auto mfma_row = [&](int r, int st, int st_next) __attribute__((always_inline)) {
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            const uint4 av = a_op(r, c);
#pragma unroll
            for (int i = 0; i < (BF ? 1 : 4); ++i) mma<T>(acc[8 * r + c], av, vr[c], i);
            if (r == 0)
                load_v(1, c, st);
            else
                load_v(0, c, st_next);
        }
    };

    // ---- pipeline: step st transforms from buffer st % 2 while step st+1's
    // patch is loaded and stored into the other buffer; one barrier per step.
    // The last step loads its own patch again (into a buffer no longer read),
    // so every step runs the same code.
    // Staging two steps ahead: the end of step st loads the patch of step
    // st+2, which step st+1 converts and stores in two halves (the second
    // half while the first half's registers hold the next loads' targets).
    constexpr int UH = (MAXU + 1) / 2;
    const int ns = a.nsteps;
    const int pb = a.patch_bytes;
    stage_load(0, 0, MAXU);
    stage_convert(0, MAXU);
    stage_store(0, 0, MAXU);
    stage_load(min(1, ns - 1), 0, MAXU);
#pragma unroll
    for (int c = 0; c < 8; ++c) load_v(0, c, 0);
    __syncthreads();
    // the products of one row interleaved with the vector work that follows
    constexpr int MFR = BF ? 8 : 32;  // MFMAs per row of the pair
    for (int st = 0; st < ns; ++st) {
        const int cur = (st & 1) * pb;
        const int nxt = pb - cur;
        const int st2 = min(st + 2, ns - 1);
        column_pass(cur);
        __builtin_amdgcn_sched_barrier(0);
        stage_convert(0, UH);
        stage_store(nxt, 0, UH);
        row_pass(0);
        __builtin_amdgcn_sched_barrier(0);
        mfma_row(0, st, min(st + 1, ns - 1));
        row_pass(1);
#pragma unroll
        for (int i = 0; i < MFR; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);            // one MFMA
            __builtin_amdgcn_sched_group_barrier(0x002, BF ? 12 : 3, 0);  // vector ALU
        }
        __builtin_amdgcn_sched_barrier(0);
        mfma_row(1, st, min(st + 1, ns - 1));
        stage_convert(UH, MAXU);
        stage_store(nxt, UH, MAXU);
#pragma unroll
        for (int i = 0; i < MFR; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x002, BF ? 20 : 1, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
        // both halves of step st+2 are loaded after every filter load this
        // step waits for: loads complete in order, so a filter wait issued
        // behind a staging load would wait for the staging load as well
        stage_load(st2, 0, MAXU);
        __syncthreads();
    }
    __syncthreads();

    // ---- output transform, 16 output channels at a time: M[xi][channel][tile]
    // (fp32, pitch MP) in LDS, then Y = A^T M A per (tile, channel)
    const int osx = BF ? wg_shift(a.xmax) : 0, osw = BF ? wg_shift(a.wmax) : 0;
    float* Ms = reinterpret_cast<float*>(lds);
#pragma unroll 1
    for (int sl = 0; sl < 2; ++sl) {
        // accumulator v of position x: tile slot 8 (v/4) + 4 h + v%4, output channel lrow
        if ((lrow >> 4) == sl) {
            const int col = lrow & 15;
#pragma unroll
            for (int x = 0; x < XPW; ++x) {
                const int xi = 8 * (x < 8 ? ra : rbw) + (x & 7);
#pragma unroll
                for (int v4 = 0; v4 < 4; ++v4)
                    *reinterpret_cast<float4*>(Ms + (xi * KS + col) * MP + 8 * v4 + 4 * h) =
                        make_float4(acc[x][4 * v4], acc[x][4 * v4 + 1], acc[x][4 * v4 + 2], acc[x][4 * v4 + 3]);
            }
        }
        __syncthreads();
        for (int pq = tid; pq < TB * KS; pq += NTHR) {
            const int row = pq & 31, kl = pq >> 5;
            const int k = kt * KB + sl * KS + kl;
            const int trr = row / a.tcb, tcc = row - trr * a.tcb;
            const int R = R0 + trr, tx = tc0 + tcc;
            if (row >= a.tr * a.tcb || R >= a.NR || tx >= a.tw || k >= a.K) continue;
            const int n = R / a.th, ty = R - n * a.th;
            // t = A^T M, one column of M at a time
            float tt[6][8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                float mc[8], o6[6];
#pragma unroll
                for (int i = 0; i < 8; ++i) mc[i] = Ms[((i * 8 + j) * KS + kl) * MP + row];
                at8(mc, o6);
#pragma unroll
                for (int p = 0; p < 6; ++p) tt[p][j] = o6[p];
            }
#pragma unroll
            for (int p = 0; p < 6; ++p) {
                const int oh = 6 * ty + p;
                if (oh >= a.OH) continue;
                float yr[6];
                at8(tt[p], yr);
                const long long rowoff = n * a.y_img + (static_cast<long long>(k) * a.OH + oh) * a.OW;
#pragma unroll
                for (int qq = 0; qq < 6; ++qq) {
                    const int ow = 6 * tx + qq;
                    if (ow >= a.OW) continue;
                    const long long o = rowoff + ow;
                    float sv = BF ? wg_denorm(yr[qq], osx, osw) : yr[qq];
                    if constexpr (EPI) sv = epi_float<T>(sv, a.e, k, o);
                    if constexpr (BF)
                        reinterpret_cast<uint16_t*>(a.y)[o] = float_to_bf16(sv);
                    else
                        reinterpret_cast<float*>(a.y)[o] = sv;
                }
            }
        }
        __syncthreads();
    }
}

// ---------------------------------------------------------------- filter prepare
// V[xi][kt][chunk][piece][32 rows][half][16 B] = (G' g G'^T)[xi] (G' = G with
// the B^T row factors divided out), in the operand type: for bf16 (fp16,
// times the filter's power-of-two scale) half h of piece i holds channels
// 32 chunk + 16 i + 8 h + e; for fp32 channels 16 chunk + 4 (2 h + i) + e.
// Rows past K and channels past C are zero.
template <typename T>
__global__ __launch_bounds__(256) void wf6_prepare_kernel(const T* __restrict__ w, uint8_t* __restrict__ out, int K, int C,
                                                          int ntk, int nchunks, const unsigned* __restrict__ wmax) {
    constexpr bool BF = sizeof(T) == 2;
    constexpr int CK = BF ? 32 : 16;  // channels per 64-byte chunk
    constexpr int EP = BF ? 8 : 4;    // elements per 16 bytes
    const float wsc = BF ? wg_norm(wmax) : 1.0f;
    const long long total = static_cast<long long>(ntk) * KB * nchunks * CK;
    for (long long idx = blockIdx.x * 256LL + threadIdx.x; idx < total; idx += static_cast<long long>(gridDim.x) * 256) {
        const int c = static_cast<int>(idx % (nchunks * CK));
        const int k = static_cast<int>(idx / (nchunks * CK));
        float gg[3][3] = {};
        if (k < K && c < C)
            for (int r = 0; r < 3; ++r)
                for (int s = 0; s < 3; ++s) gg[r][s] = Elem<T>::to_f(w[(static_cast<long long>(k) * C + c) * 9 + r * 3 + s]);
        float tmp[8][3];
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int s = 0; s < 3; ++s) {
                float acc = 0.0f;
#pragma unroll
                for (int r = 0; r < 3; ++r) acc = fmaf(kF6.gs[i][r], gg[r][s], acc);
                tmp[i][s] = acc;
            }
        const int kt = k / KB, row = k % KB;
        const int chunk = c / CK, cl = c % CK;
        int piece, half, e;
        if (BF) {
            piece = cl / 16;
            half = (cl % 16) / 8;
            e = cl % 8;
        } else {
            const int slot = cl / 4;  // = 2 half + piece
            half = slot / 2;
            piece = slot % 2;
            e = cl % 4;
        }
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                float acc = 0.0f;
#pragma unroll
                for (int s = 0; s < 3; ++s) acc = fmaf(tmp[i][s], kF6.gs[j][s], acc);
                const long long x16 =
                    ((((static_cast<long long>(i * 8 + j) * ntk + kt) * nchunks + chunk) * 2 + piece) * 32 + row) * 2 + half;
                if constexpr (BF)
                    reinterpret_cast<_Float16*>(out)[x16 * EP + e] = static_cast<_Float16>(acc * wsc);
                else
                    reinterpret_cast<float*>(out)[x16 * EP + e] = acc;
            }
    }
}

// ---------------------------------------------------------------- host plan

struct Plan {
    int E, th, tw, NR, tcb, tr, nrb, ncb, ntk, nchunks, nsteps, kgrp;
    int pws, nbk, nbkp, rp, sk, patch_bytes, nunits, maxu;
    size_t lds, v_bytes;
};

constexpr int kMaxuBf16 = 2, kMaxuF32 = 4;  // staging units per thread the kernels are built for

inline bool plan(const Prob& p, Plan* pl, std::string* why) {
    auto no = [&](const char* s) __attribute__((always_inline)) {
        if (why) *why = s;
        return false;
    };
    if (p.r != 3 || p.s != 3 || p.sh != 1 || p.sw != 1 || p.dh != 1 || p.dw != 1 || p.g != 1)
        return no("winograd F(6x6) fused: needs 3x3, stride 1, dilation 1, groups 1");
    if (p.dtype != CFWD_BF16 && p.dtype != CFWD_F32) return no("winograd F(6x6) fused: bf16 or fp32 only");
    if (p.xb != 1) return no("winograd F(6x6) fused: NCHW only");
    if (p.c % 16 != 0) return no("winograd F(6x6) fused: C must be a multiple of 16");
    // bf16: the fp16 transform's rounding, relative to the sum of |x*w| an
    // output is normalised by, shrinks like one over the square root of the
    // channel count; from 64 channels on it stays well inside the bf16 bound
    if (p.dtype == CFWD_BF16 && p.c < 64)
        return no("winograd F(6x6) fused: bf16 needs at least 64 input channels to meet its error bound");
    if (p.ph > 2 || p.pw > 2) return no("winograd F(6x6) fused: padding at most 2");
    // bf16 with padding 2: a corner output sees one input pixel per channel,
    // so its normalising sum of |x*w| is small next to the fp16 rounding of
    // the tile's 64 transformed values
    if (p.dtype == CFWD_BF16 && (p.ph > 1 || p.pw > 1))
        return no("winograd F(6x6) fused: bf16 needs padding 0 or 1 to meet its error bound");
    if (p.oh < 1 || p.ow < 1) return no("winograd F(6x6) fused: empty output");
    const int E = 16 / p.esize;
    if (p.w % E != 0) return no("winograd F(6x6) fused: W must be a multiple of 16 bytes of pixels");
    const long long xbytes = static_cast<long long>(p.n) * p.x_img * p.esize;
    if (xbytes >= (1LL << 31)) return no("winograd F(6x6) fused: input of 2 GiB or more");
    pl->E = E;
    pl->th = (p.oh + 5) / 6;
    pl->tw = (p.ow + 5) / 6;
    const long long NR = static_cast<long long>(p.n) * pl->th;
    if (NR >= (1LL << 30)) return no("winograd F(6x6) fused: too many tile rows");
    pl->NR = static_cast<int>(NR);
    pl->ntk = (p.k + KB - 1) / KB;
    const int ck = 64 / p.esize;
    pl->nchunks = (p.c + ck - 1) / ck;
    pl->nsteps = p.c / (p.dtype == CFWD_BF16 ? 16 : 8);
    const int maxu = p.dtype == CFWD_BF16 ? kMaxuBf16 : kMaxuF32;
    // tile block: the shape with the least modelled work -- a transform per
    // tile slot and step, plus staging per patch pixel (bf16 converts, fp32
    // copies) -- over whole rounds of 256 workgroups
    const double cst = p.dtype == CFWD_BF16 ? 2.5 : 0.5;
    double best = -1.0;
    for (int tcb = 1; tcb <= std::min(pl->tw, TB); ++tcb) {
        for (int tr = std::min<long long>(TB / tcb, NR); tr >= 1; --tr) {
            const int pws = (E - 1 + 6 * tcb + 2 + E - 1) / E * E;
            const int nunits = 8 * tr * (pws / E) * 2;
            const int nbkp = (pws / E) | 1;
            const long long patch = 2LL * (2 * 8 * tr * (E * nbkp + 1) + 2 * 6 * tr) * 16;  // two buffers
            if (nunits > maxu * NTHR || patch + 128 > LDS_MAX) continue;
            const long long nrb = (NR + tr - 1) / tr, ncb = (pl->tw + tcb - 1) / tcb;
            const long long blocks = nrb * ncb * pl->ntk;
            const double rounds = static_cast<double>((blocks + 255) / 256);
            const double cost = rounds * (TB * 384.0 + 8.0 * tr * pws * cst);
            if (best < 0 || cost < best) {
                best = cost;
                pl->tcb = tcb;
                pl->tr = tr;
                pl->pws = pws;
                pl->nbk = pws / E;
                pl->nunits = nunits;
                pl->nrb = static_cast<int>(nrb);
                pl->ncb = static_cast<int>(ncb);
            }
            break;  // the tallest block that fits for this width
        }
    }
    if (best < 0) return no("winograd F(6x6) fused: no tile block fits");
    const long long blocks = static_cast<long long>(pl->nrb) * pl->ncb * pl->ntk;
    if (blocks >= (1LL << 31)) return no("winograd F(6x6) fused: too many workgroups");
    // patch layout: odd block pitch, odd row pitch and a skew per tile row,
    // chosen with a model of the bank conflicts of the window reads and the
    // staging stores over the blocks' shapes
    pl->nbkp = pl->nbk | 1;
    pl->rp = E * pl->nbkp + 1;
    pl->sk = 6;
    pl->patch_bytes = (2 * 8 * pl->tr * pl->rp + 2 * pl->tr * pl->sk) * 16;
    pl->maxu = maxu;
    // two filter slices per group when together they take at most half an
    // XCD's L2 (a slice is 64 positions x C x 32 channels: 1 MiB in bf16's
    // fp16 form and 2 MiB in fp32 at C = 256)
    const size_t slice = static_cast<size_t>(64) * p.c * KB * (p.dtype == CFWD_BF16 ? 2 : 4);
    pl->kgrp = (pl->ntk % 2 == 0 && 2 * slice <= (size_t(2) << 20)) ? 2 : 1;
    pl->lds = std::max<size_t>(2 * static_cast<size_t>(pl->patch_bytes) + 128, M_LDS);
    pl->v_bytes = static_cast<size_t>(64) * pl->ntk * pl->nchunks * 2048;
    if (pl->v_bytes >= (size_t(1) << 31)) return no("winograd F(6x6) fused: prepared filter of 2 GiB or more");
    return true;
}

template <typename T, bool EPI>
cfwd_status launch_t(const Prob& p, const Plan& pl, const void* x, const void* vp, void* y, const Epi& e,
                     const unsigned* xmax, const unsigned* wmax, hipStream_t st) {
    constexpr int MAXU = sizeof(T) == 2 ? kMaxuBf16 : kMaxuF32;
    if (pl.nunits > MAXU * NTHR || pl.lds > static_cast<size_t>(LDS_MAX))
        return set_error(CFWD_ERR_UNSUPPORTED, "winograd F(6x6) fused: block larger than planned");
    static bool attr = false;
    auto kern = wf6_kernel<T, MAXU, EPI>;
    cfwd_status s = ig::allow_big_lds(kern, pl.lds, &attr);
    if (s != CFWD_OK) return s;
    Args a;
    a.x = static_cast<const uint8_t*>(x);
    a.v = static_cast<const uint8_t*>(vp);
    a.y = static_cast<uint8_t*>(y);
    a.C = p.c; a.H = p.h; a.W = p.w; a.K = p.k; a.OH = p.oh; a.OW = p.ow; a.ph = p.ph; a.pw = p.pw;
    a.x_img = p.x_img; a.y_img = p.y_img;
    a.x_bytes = static_cast<int>(static_cast<long long>(p.n) * p.x_img * p.esize);
    a.v_bytes = static_cast<int>(pl.v_bytes);
    a.th = pl.th; a.tw = pl.tw; a.NR = pl.NR; a.tcb = pl.tcb; a.tr = pl.tr;
    a.nrb = pl.nrb; a.ncb = pl.ncb; a.ntk = pl.ntk; a.nchunks = pl.nchunks; a.nsteps = pl.nsteps;
    a.kgrp = pl.kgrp;
    a.nbk = pl.nbk; a.nunits = pl.nunits; a.nbkp = pl.nbkp; a.rp = pl.rp; a.sk = pl.sk;
    a.patch_bytes = pl.patch_bytes;
    a.e = e;
    a.xmax = xmax;
    a.wmax = wmax;
    const unsigned blocks = static_cast<unsigned>(static_cast<long long>(pl.nrb) * pl.ncb * pl.ntk);
    kern<<<blocks, NTHR, pl.lds, st>>>(a);
    return check_hip(hipGetLastError(), "winograd F(6x6) fused launch");
}

}  // namespace wf6

bool winograd_f6_fused_supported(const Prob& p, std::string* why) {
    wf6::Plan pl;
    return wf6::plan(p, &pl, why);
}

size_t winograd_f6_fused_filter_bytes(const Prob& p) {
    wf6::Plan pl;
    if (!wf6::plan(p, &pl, nullptr)) return 0;
    // bf16: 8 KiB after the transformed filter hold its largest magnitude
    return pl.v_bytes + (p.dtype == CFWD_BF16 ? 8192 : 0);
}

size_t winograd_f6_fused_scratch_bytes(const Prob& p) {
    // bf16 only: the input's largest magnitude (no transformed data)
    return (p.dtype == CFWD_BF16 && winograd_f6_fused_supported(p, nullptr)) ? 8192 : 0;
}

cfwd_status winograd_f6_fused_prepare(const Prob& p, const void* w, void* wp, hipStream_t st) {
    wf6::Plan pl;
    std::string why;
    if (!wf6::plan(p, &pl, &why)) return set_error(CFWD_ERR_UNSUPPORTED, why);
    const int ck = 64 / p.esize;
    const long long total = static_cast<long long>(pl.ntk) * wf6::KB * pl.nchunks * ck;
    const unsigned nb = static_cast<unsigned>(std::min<long long>((total + 255) / 256, 65536));
    uint8_t* out = static_cast<uint8_t*>(wp);
    if (p.dtype == CFWD_F32) {
        wf6::wf6_prepare_kernel<float><<<nb, 256, 0, st>>>(static_cast<const float*>(w), out, p.k, p.c, pl.ntk,
                                                           pl.nchunks, nullptr);
    } else {
        unsigned* wmax = reinterpret_cast<unsigned*>(out + pl.v_bytes);
        cfwd_status s = bf16_absmax(w, static_cast<long long>(p.k) * p.c * 9, wmax, st);
        if (s != CFWD_OK) return s;
        wf6::wf6_prepare_kernel<bf16_t><<<nb, 256, 0, st>>>(static_cast<const bf16_t*>(w), out, p.k, p.c, pl.ntk,
                                                            pl.nchunks, wmax);
    }
    return check_hip(hipGetLastError(), "winograd F(6x6) fused filter transform launch");
}

cfwd_status winograd_f6_fused_launch(const Prob& p, const void* x, const void* wp, void* scratch, void* y,
                                     const Epi& e, hipStream_t st) {
    wf6::Plan pl;
    std::string why;
    if (!wf6::plan(p, &pl, &why)) return set_error(CFWD_ERR_UNSUPPORTED, why);
    if (wp == nullptr) return set_error(CFWD_ERR_WORKSPACE, "winograd F(6x6) fused: prepared filter required");
    const bool epi = e.bias || e.res || e.relu;
    if (p.dtype == CFWD_F32)
        return epi ? wf6::launch_t<float, true>(p, pl, x, wp, y, e, nullptr, nullptr, st)
                   : wf6::launch_t<float, false>(p, pl, x, wp, y, e, nullptr, nullptr, st);
    if (scratch == nullptr) return set_error(CFWD_ERR_WORKSPACE, "winograd F(6x6) fused: bf16 needs 8 KiB of scratch");
    unsigned* xmax = static_cast<unsigned*>(scratch);
    cfwd_status s = bf16_absmax(x, static_cast<long long>(p.n) * p.x_img, xmax, st);
    if (s != CFWD_OK) return s;
    const unsigned* wmax = reinterpret_cast<const unsigned*>(static_cast<const uint8_t*>(wp) + pl.v_bytes);
    return epi ? wf6::launch_t<bf16_t, true>(p, pl, x, wp, y, e, xmax, wmax, st)
               : wf6::launch_t<bf16_t, false>(p, pl, x, wp, y, e, xmax, wmax, st);
}

}  // namespace cfwd
