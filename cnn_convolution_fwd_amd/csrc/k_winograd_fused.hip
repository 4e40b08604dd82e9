// Fused Winograd F(2x2, 3x3) for bf16 NCHW activations (gfx950).
//
// MegEngine inference article, section "Winograd": F(2x2,3x3) computes a 2x2
// output tile from a 4x4 input tile with 16 multiplies instead of 36, in three
// steps (transform input and weights, multiply the transformed tiles as a
// batched matrix product, transform back); its engineering subsection blocks
// the tiles so that one block's transformed data stays close to the core.
//
// Here the transformed input never leaves the compute unit.  One workgroup
// owns 64 output tiles (TR tile rows x TCB tile columns of one image) and 64
// output channels, and loops over the input channels in chunks of 32:
//   * the input patch of its tiles ((2TR+2) x (2TCB+2) pixels x 32 channels)
//     is staged in LDS with 16-byte global loads along W, transposed in
//     registers to channel-innermost order and converted to fp16 (bf16 values
//     in fp16's normal range convert exactly);
//   * wave w owns Winograd row w: the four positions (w, j).  For each tile a
//     lane reads the two patch rows that row w of B^T combines, forms
//     t = B^T d for the four patch columns, then U[w][j] = t B for j = 0..3
//     (packed fp16 adds; every entry of the scaled B^T is 0 or +-1, so these
//     adds are the only rounding), and feeds U as the A operand of
//     v_mfma_f32_32x32x16_f16 against the prepared filter V[w][j] (B operand,
//     read from L2 one chunk ahead);
//   * 4 positions x 64 tiles x 64 channels per wave = 256 fp32 accumulators
//     per lane;
//   * after the last chunk each wave folds its four positions over j with
//     A^T (Z[w][q] = sum_j A^T[q][j] M[w][j]), writes Z through LDS, and
//     every thread finishes Y[p][q] = sum_w A^T[p][w] Z[w][q] for runs of 8
//     output columns, stored as 16-byte bf16 vectors.
// Scaling: B^T has entries +-1/2 in rows 1 and 2 as constructed; those rows
// are scaled to +-1 and G's rows scaled by the same factors instead, which
// leaves (G g G^T) * (B^T d B) unchanged elementwise.
#include "igemm_impl.h"
#include "winograd_mats.h"

namespace cfwd {
namespace wf {

using ig::f32x16;

constexpr int TBL = 64;   // tiles per workgroup
constexpr int KB = 64;    // output channels per workgroup
constexpr int CK = 32;    // input channels per chunk (64 bytes of fp16)
constexpr int PIX = 80;   // LDS bytes per patch pixel: 64 of channels + 16 pad
constexpr int ZP = 132;   // epilogue LDS pitch, floats per output-channel row
constexpr int NTHR = 256;

typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------- matrices

struct F2 {
    int bt[4][4];      // scaled B^T: entries 0, +-1
    float gp[4][3];    // G with rows scaled to match
    int at[2][4];      // A^T
    int ra[4], rb[4];  // row w of bt: t = sa * d[ra] + d[rb]
    int sa[4];
};

constexpr F2 build_f2() {
    constexpr wg::Mats<2> m = wg::build_mats<2>();
    F2 f{};
    for (int i = 0; i < 4; ++i) {
        double mx = 0;
        for (int k = 0; k < 4; ++k) {
            const double v = m.bt[i][k] < 0 ? -m.bt[i][k] : m.bt[i][k];
            if (v > mx) mx = v;
        }
        for (int k = 0; k < 4; ++k) {
            const double v = m.bt[i][k] / mx;
            f.bt[i][k] = v > 0.5 ? 1 : (v < -0.5 ? -1 : 0);
        }
        for (int r = 0; r < 3; ++r) f.gp[i][r] = static_cast<float>(m.g[i][r] * mx);
        int pos = -1, other = -1;
        for (int k = 0; k < 4; ++k) {
            if (f.bt[i][k] == 1 && pos < 0)
                pos = k;
            else if (f.bt[i][k] != 0)
                other = k;
        }
        f.rb[i] = pos;
        f.ra[i] = other;
        f.sa[i] = other >= 0 ? f.bt[i][other] : 0;
    }
    for (int q = 0; q < 2; ++q)
        for (int j = 0; j < 4; ++j) {
            const double v = m.at[q][j];
            f.at[q][j] = v > 0.5 ? 1 : (v < -0.5 ? -1 : 0);
        }
    return f;
}

constexpr F2 kF2 = build_f2();

constexpr bool check_f2() {
    // the kernel relies on: every row of the scaled B^T has exactly two
    // nonzeros, one of them +1, and all entries of B^T and A^T are 0 / +-1
    for (int i = 0; i < 4; ++i) {
        int nz = 0;
        for (int k = 0; k < 4; ++k) nz += kF2.bt[i][k] != 0;
        if (nz != 2 || kF2.rb[i] < 0 || kF2.ra[i] < 0) return false;
    }
    return true;
}
static_assert(check_f2(), "F(2,3) input transform does not have the expected sparsity");

// ---------------------------------------------------------------- kernel

struct Args {
    const uint16_t* x;  // bf16 bits, NCHW
    const uint8_t* v;   // prepared filter
    uint16_t* y;        // bf16 bits, NCHW
    int N, C, H, W, K, OH, OW, ph, pw;
    long long x_img, y_img;
    int tbh, tbw, ntk, nchunks;
    int nblk;  // 8-column load blocks per patch row
    Epi e;     // fused epilogue
    // largest input / filter magnitudes (bf16 bit patterns): the operands are
    // scaled into the fp16 range by wg_norm and the outputs back by wg_denorm
    const unsigned* xmax;
    const unsigned* wmax;
};

// Fused epilogue (bias, residual, ReLU) on 8 consecutive outputs of channel
// k starting at element offset `off`, of which the first nv are real.
__device__ __forceinline__ void epi8(float* yv, const Epi& e, int k, long long off, int nv) {
#pragma unroll
    for (int i = 0; i < 8; ++i)
        if (i < nv) yv[i] = epi_float<bf16_t>(yv[i], e, k, off + i);
}

// Two bf16 (the halves of dword w), times the power-of-two scale sc -> fp16
// pair; p selects the half of each source word (0: low, 1: high).
__device__ __forceinline__ uint32_t cvt_pair(uint32_t wlo, uint32_t whi, int p, float sc) {
    const float flo = __uint_as_float(p ? (wlo & 0xffff0000u) : (wlo << 16)) * sc;
    const float fhi = __uint_as_float(p ? (whi & 0xffff0000u) : (whi << 16)) * sc;
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(flo, fhi));
}

__device__ __forceinline__ uint32_t word_of(const uint4& v, int i) {
    return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

template <int TCB> struct Geo {
    static constexpr int TR = TBL / TCB;
    static constexpr int PH = 2 * TR + 2;
    // patch columns are held from 8 before the window to 8 after it (so every
    // 8-pixel staging unit lands inside), split by column parity into two
    // planes of PUE pixels
    static constexpr int PUE = TCB + 9;
    static constexpr int PATCH = PH * 2 * PUE * PIX;  // bytes per patch buffer
    static constexpr int NBMAX = (2 * TCB + 16) / 8;  // load blocks per row, at most (pad <= 1)
    static constexpr int MAXU = (PH * NBMAX * 4 + NTHR - 1) / NTHR;
    // two patch buffers, then a dummy area that staging threads without a
    // unit write into (reached from either buffer's offset)
    static constexpr int LDS_MAIN = 3 * PATCH + 4096;
    static constexpr int LDS_EPI = 4 * KB * ZP * 4;
    static constexpr int LDS = LDS_MAIN > LDS_EPI ? LDS_MAIN : LDS_EPI;
};

// Scheduling masks for __builtin_amdgcn_sched_group_barrier.
constexpr int kSchedVALU = 0x002, kSchedMFMA = 0x008;

// The eight MFMAs of one step interleaved with NV VALU instructions each of
// the next step's work.
template <int NV>
__device__ __forceinline__ void interleave3() {
#pragma unroll
    for (int i = 0; i < 24; ++i) {
        __builtin_amdgcn_sched_group_barrier(kSchedMFMA, 1, 0);
        __builtin_amdgcn_sched_group_barrier(kSchedVALU, NV, 0);
    }
}

template <int NV>
__device__ __forceinline__ void interleave() {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        __builtin_amdgcn_sched_group_barrier(kSchedMFMA, 1, 0);
        __builtin_amdgcn_sched_group_barrier(kSchedVALU, NV, 0);
    }
}

// EPI: the fused epilogue compiled in (a separate instantiation, so the
// plain kernel carries none of its registers).
template <int TCB, int PWO, bool EPI>
__global__ __launch_bounds__(NTHR) void wf2_kernel(Args a) {
    using G = Geo<TCB>;
    constexpr int TR = G::TR, PUE = G::PUE, MAXU = G::MAXU;
    constexpr F2 f2 = build_f2();
    const float xsc = wg_norm(a.xmax);  // input scale into the fp16 range
    const int osx = wg_shift(a.xmax), osw = wg_shift(a.wmax);  // and the shifts undoing both
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int m = lane & 31;
    const int h = lane >> 5;

    // work order: the output-channel blocks of one tile block are adjacent
    // (same XCD, so the re-staged input comes from its L2)
    int lin = xcd_linear(static_cast<int>(blockIdx.x), static_cast<int>(gridDim.x));
    const int kt = lin % a.ntk;
    lin /= a.ntk;
    const int tbc = lin % a.tbw;
    lin /= a.tbw;
    const int tbr = lin % a.tbh;
    const int n = lin / a.tbh;
    const int tr0 = tbr * TR, tc0 = tbc * TCB;
    const int ih0 = 2 * tr0 - a.ph, iw0 = 2 * tc0 - PWO;
    const int HW = a.H * a.W;
    const int HW2 = 2 * HW;
    const uint8_t* __restrict__ xn = reinterpret_cast<const uint8_t*>(a.x + n * a.x_img);

    // ---- staging units: (patch row, 8-column load block, 16-byte channel slot)
    // Loads go through a buffer resource whose size ends at the last channel
    // of the tensor: pixels outside the image get an offset past any size and
    // read as zero, as do channels past C, without a select.
    const int cbf = (iw0 >= 0) ? iw0 / 8 : -((-iw0 + 7) / 8);
    int u_voff[MAXU];  // byte offset of the unit's first channel and pixel
    int u_lds[MAXU];   // LDS byte offset of the unit's first pixel (no unit: the dummy area)
#pragma unroll
    for (int i = 0; i < MAXU; ++i) {
        const int u = tid + i * NTHR;
        const int t = u >> 2;
        const int cb = t % a.nblk;
        const int row = t / a.nblk;
        const int j = u & 3;
        const int ih = ih0 + row;
        const int iwb = (cbf + cb) * 8;
        const bool unit = row < G::PH;
        const bool in = unit && static_cast<unsigned>(ih) < static_cast<unsigned>(a.H) &&
                        static_cast<unsigned>(iwb) < static_cast<unsigned>(a.W);
        u_voff[i] = in ? (j * 8 * HW + ih * a.W + iwb) * 2 : static_cast<int>(0x80000000u);
        const int colx0 = iwb - iw0 + 8;  // >= 1; parity PWO
        u_lds[i] = unit ? ((row * 2) * PUE + (colx0 >> 1)) * PIX + j * 16 : 2 * G::PATCH;
    }
    uint4 stg[MAXU][8];
    auto stage_load = [&](int chunk) {
        const int cleft = a.C - chunk * CK;
        const int nrec = cleft > 0 ? cleft * HW2 : 0;
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint8_t*>(xn) + static_cast<long long>(chunk) * CK * HW2, 0, nrec, 0x00020000);
#pragma unroll
        for (int i = 0; i < MAXU; ++i)
#pragma unroll
            for (int l = 0; l < 8; ++l) {
                const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rs, u_voff[i] + l * HW2, 0, 0);
                stg[i][l] = make_uint4(v.x, v.y, v.z, v.w);
            }
    };
    auto stage_store = [&](int bufoff) {
#pragma unroll
        for (int i = 0; i < MAXU; ++i) {
            uint8_t* base = lds + bufoff + u_lds[i];
#pragma unroll
            for (int p = 0; p < 8; ++p) {
                const int off = (((PWO + p) & 1) * PUE + ((PWO + p) >> 1)) * PIX;
                uint4 o;
                o.x = cvt_pair(word_of(stg[i][0], p >> 1), word_of(stg[i][1], p >> 1), p & 1, xsc);
                o.y = cvt_pair(word_of(stg[i][2], p >> 1), word_of(stg[i][3], p >> 1), p & 1, xsc);
                o.z = cvt_pair(word_of(stg[i][4], p >> 1), word_of(stg[i][5], p >> 1), p & 1, xsc);
                o.w = cvt_pair(word_of(stg[i][6], p >> 1), word_of(stg[i][7], p >> 1), p & 1, xsc);
                *reinterpret_cast<uint4*>(base + off) = o;
            }
        }
    };

    // ---- this wave's Winograd row and the lane's tiles
    const int ra = wave == 0 ? f2.ra[0] : wave == 1 ? f2.ra[1] : wave == 2 ? f2.ra[2] : f2.ra[3];
    const int rb = wave == 0 ? f2.rb[0] : wave == 1 ? f2.rb[1] : wave == 2 ? f2.rb[2] : f2.rb[3];
    const int sa = wave == 0 ? f2.sa[0] : wave == 1 ? f2.sa[1] : wave == 2 ? f2.sa[2] : f2.sa[3];
    const h2 sa2 = {static_cast<_Float16>(sa), static_cast<_Float16>(sa)};
    // tile slot s = m + 32 f (f = tile fragment) -> (tr, tc) = (s / TCB, s % TCB);
    // its window column c is patch column 2 tc + c, held in parity plane c & 1
    // at plane pixel tc + 4 + c / 2
    int tbase[2];
#pragma unroll
    for (int f = 0; f < 2; ++f) {
        const int s = m + 32 * f;
        const int tr = s / TCB, tc = s % TCB;
        tbase[f] = ((2 * tr) * 2 * PUE + tc + 4) * PIX + h * 16;
    }
    const int offA = ra * 2 * PUE * PIX, offB = rb * 2 * PUE * PIX;

    // ---- prepared filter: [kt][chunk][xi][b][ks][32 rows][half][16 B]
    const uint8_t* __restrict__ vbase =
        a.v + static_cast<long long>(kt) * a.nchunks * 65536 + wave * 16384 + m * 32 + h * 16;
    uint4 vb[2][4][2];
    auto load_v = [&](int chunk, int ks) {
        const uint8_t* p = vbase + static_cast<long long>(chunk) * 65536 + ks * 1024;
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int b = 0; b < 2; ++b) vb[ks][j][b] = *reinterpret_cast<const uint4*>(p + (j * 2 + b) * 2048);
    };

    // ---- one step = (k-step ks, tile fragment f) of a chunk
    uint4 da[4], db[4];  // patch reads of the next step to transform
    auto read_d = [&](int bufoff, int ks, int f) {
        const uint8_t* q = lds + bufoff + tbase[f] + ks * 32;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const int co = ((c & 1) * PUE + (c >> 1)) * PIX;
            da[c] = *reinterpret_cast<const uint4*>(q + offA + co);
            db[c] = *reinterpret_cast<const uint4*>(q + offB + co);
        }
    };
    auto transform = [&](uint4 (&U)[4]) {
        h2 t[4][4];
#pragma unroll
        for (int c = 0; c < 4; ++c)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                t[c][e] = __builtin_bit_cast(h2, word_of(da[c], e)) * sa2 + __builtin_bit_cast(h2, word_of(db[c], e));
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            uint32_t w[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                h2 s = {0, 0};
                bool first = true;
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    const int co = f2.bt[j][c];
                    if (co == 0) continue;
                    if (first) {
                        s = co > 0 ? t[c][e] : -t[c][e];
                        first = false;
                    } else {
                        s = co > 0 ? s + t[c][e] : s - t[c][e];
                    }
                }
                w[e] = __builtin_bit_cast(uint32_t, s);
            }
            U[j] = make_uint4(w[0], w[1], w[2], w[3]);
        }
    };

    f32x16 acc[4][2][2];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int f = 0; f < 2; ++f)
#pragma unroll
            for (int b = 0; b < 2; ++b) acc[j][f][b] = f32x16{};
    auto mma = [&](const uint4 (&U)[4], int ks, int f) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int b = 0; b < 2; ++b)
                acc[j][f][b] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
                    __builtin_bit_cast(f16x8, U[j]), __builtin_bit_cast(f16x8, vb[ks][j][b]), acc[j][f][b], 0, 0, 0);
    };

    // ---- prologue: chunk 0 in buffer 0, its first step transformed, the
    // second step's patch reads in flight
    stage_load(0);
    load_v(0, 0);
    load_v(0, 1);
    stage_store(0);
    __syncthreads();
    uint4 ucur[4], unext[4];
    read_d(0, 0, 0);
    transform(ucur);
    read_d(0, 0, 1);
    // drain every counter here, so the loop's waits are derived from its own
    // steady state (otherwise the prologue's load order makes the first
    // steps of every chunk wait for filter loads issued just before)
    __builtin_amdgcn_s_waitcnt(0);

    // Steps of chunk c: (ks 0, f 0), (0, 1), (1, 0), then the chunk barrier,
    // then (1, 1), whose MFMAs need no LDS and so overlap the next chunk's
    // first transform.  Past the last chunk the staging loads read nothing
    // (the buffer resource is empty) and the extra reads and transforms
    // touch only LDS and registers.
    for (int chunk = 0; chunk < a.nchunks; ++chunk) {
        const int cur = (chunk & 1) * G::PATCH;
        const int nb = G::PATCH - cur;
        const int nxt = chunk + 1 < a.nchunks ? chunk + 1 : chunk;
        stage_load(chunk + 1);
        __builtin_amdgcn_sched_barrier(0);
        // step (0, 0)
        mma(ucur, 0, 0);
        transform(unext);
        interleave<5>();
        __builtin_amdgcn_sched_barrier(0);
        read_d(cur, 1, 0);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int j = 0; j < 4; ++j) ucur[j] = unext[j];
        // step (0, 1)
        mma(ucur, 0, 1);
        transform(unext);
        interleave<5>();
        __builtin_amdgcn_sched_barrier(0);
        read_d(cur, 1, 1);
        load_v(nxt, 0);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int j = 0; j < 4; ++j) ucur[j] = unext[j];
        // step (1, 0), with the next chunk's staging stores
        mma(ucur, 1, 0);
        transform(unext);
        stage_store(nb);  // past the last chunk: zeros into a buffer no longer read
        interleave<16>();
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int j = 0; j < 4; ++j) ucur[j] = unext[j];
        __syncthreads();
        read_d(nb, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
        // step (1, 1) of this chunk; first transform of the next
        mma(ucur, 1, 1);
        transform(unext);
        interleave<5>();
        __builtin_amdgcn_sched_barrier(0);
        read_d(nb, 0, 1);
        load_v(nxt, 1);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int j = 0; j < 4; ++j) ucur[j] = unext[j];
    }
    __syncthreads();

    // ---- output transform
    // accumulator v of fragment (f, b): tile slot 32f + 8(v/4) + 4h + v%4,
    // output channel 32b + m
    float* Zs = reinterpret_cast<float*>(lds);
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int f = 0; f < 2; ++f)
#pragma unroll
            for (int v4 = 0; v4 < 4; ++v4) {
                float z[8];
#pragma unroll
                for (int vv = 0; vv < 4; ++vv) {
                    const int v = 4 * v4 + vv;
#pragma unroll
                    for (int q = 0; q < 2; ++q) {
                        float s = 0.0f;
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            const int co = f2.at[q][j];
                            if (co > 0) s += acc[j][f][b][v];
                            if (co < 0) s -= acc[j][f][b][v];
                        }
                        z[2 * vv + q] = s;
                    }
                }
                const int s0 = 32 * f + 8 * v4 + 4 * h;
                float* dst = Zs + (wave * KB + 32 * b + m) * ZP + 2 * s0;
                *reinterpret_cast<float4*>(dst) = make_float4(z[0], z[1], z[2], z[3]);
                *reinterpret_cast<float4*>(dst + 4) = make_float4(z[4], z[5], z[6], z[7]);
            }
    __syncthreads();

    constexpr int GPR = TCB / 4;  // runs of 8 output columns per tile row
    const bool vec_ok = (a.OW % 8) == 0;
    for (int job = tid; job < KB * TR * GPR; job += NTHR) {
        const int g = job % GPR;
        const int rest = job / GPR;
        const int tr = rest % TR;
        const int kl = rest / TR;
        const int k = kt * KB + kl;
        if (k >= a.K) continue;
        const int pos0 = tr * 2 * TCB + 8 * g;
        float z[4][8];
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const float* src = Zs + (w * KB + kl) * ZP + pos0;
            const float4 lo = *reinterpret_cast<const float4*>(src);
            const float4 hi = *reinterpret_cast<const float4*>(src + 4);
            z[w][0] = lo.x; z[w][1] = lo.y; z[w][2] = lo.z; z[w][3] = lo.w;
            z[w][4] = hi.x; z[w][5] = hi.y; z[w][6] = hi.z; z[w][7] = hi.w;
        }
        const int ow0 = 2 * tc0 + 8 * g;
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            const int oh = 2 * (tr0 + tr) + p;
            if (oh >= a.OH) continue;
            float yv[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                float s = 0.0f;
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    const int co = f2.at[p][w];
                    if (co > 0) s += z[w][e];
                    if (co < 0) s -= z[w][e];
                }
                yv[e] = wg_denorm(s, osx, osw);
            }
            const long long yo = n * a.y_img + (static_cast<long long>(k) * a.OH + oh) * a.OW + ow0;
            if constexpr (EPI) epi8(yv, a.e, k, yo, a.OW - ow0);
            uint16_t* dst = a.y + yo;
            if (vec_ok && ow0 + 8 <= a.OW) {
                const u32x4 o = {pack_bf16x2(yv[0], yv[1]), pack_bf16x2(yv[2], yv[3]), pack_bf16x2(yv[4], yv[5]),
                                 pack_bf16x2(yv[6], yv[7])};
                __builtin_nontemporal_store(o, reinterpret_cast<u32x4*>(dst));
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    if (ow0 + e < a.OW) dst[e] = float_to_bf16(yv[e]);
            }
        }
    }
}

// ---------------------------------------------------------------- folded form (config 2)
// The same staging and input transform, with A^T's fold over j moved into
// the reduction: Z[w][q] = sum_j A^T[q][j] (U[w][j] V[w][j]) is accumulated
// directly (A^T has three nonzeros per row, entries +-1, so 6 MFMAs per tile
// fragment and k-step instead of 4, with U[j] negated where A^T[q][j] = -1).
// That halves the accumulators per output channel, so a workgroup covers
// KB2 = 128 output channels (2 q x 2 tile fragments x 4 channel fragments =
// 256 accumulators per lane), and each staged patch, LDS read, transform
// and filter byte feeds three times the MFMA work of config 1.  The filter
// of one k-step (64 VGPRs) is reloaded fragment by fragment right after its
// last MFMA, so it needs no second register set.
constexpr int KB2 = 128;

template <int TCB, int PWO, bool EPI>
__global__ __launch_bounds__(NTHR) void wf2f_kernel(Args a) {
    using G = Geo<TCB>;
    constexpr int TR = G::TR, PUE = G::PUE, MAXU = G::MAXU;
    constexpr F2 f2 = build_f2();
    const float xsc = wg_norm(a.xmax);  // input scale into the fp16 range
    const int osx = wg_shift(a.xmax), osw = wg_shift(a.wmax);  // and the shifts undoing both
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int m = lane & 31;
    const int h = lane >> 5;

    int lin = xcd_linear(static_cast<int>(blockIdx.x), static_cast<int>(gridDim.x));
    const int kt = lin % a.ntk;
    lin /= a.ntk;
    const int tbc = lin % a.tbw;
    lin /= a.tbw;
    const int tbr = lin % a.tbh;
    const int n = lin / a.tbh;
    const int tr0 = tbr * TR, tc0 = tbc * TCB;
    const int ih0 = 2 * tr0 - a.ph, iw0 = 2 * tc0 - PWO;
    const int HW = a.H * a.W;
    const int HW2 = 2 * HW;
    const uint8_t* __restrict__ xn = reinterpret_cast<const uint8_t*>(a.x + n * a.x_img);

    const int cbf = (iw0 >= 0) ? iw0 / 8 : -((-iw0 + 7) / 8);
    int u_voff[MAXU];
    int u_lds[MAXU];
#pragma unroll
    for (int i = 0; i < MAXU; ++i) {
        const int u = tid + i * NTHR;
        const int t = u >> 2;
        const int cb = t % a.nblk;
        const int row = t / a.nblk;
        const int j = u & 3;
        const int ih = ih0 + row;
        const int iwb = (cbf + cb) * 8;
        const bool unit = row < G::PH;
        const bool in = unit && static_cast<unsigned>(ih) < static_cast<unsigned>(a.H) &&
                        static_cast<unsigned>(iwb) < static_cast<unsigned>(a.W);
        u_voff[i] = in ? (j * 8 * HW + ih * a.W + iwb) * 2 : static_cast<int>(0x80000000u);
        const int colx0 = iwb - iw0 + 8;
        u_lds[i] = unit ? ((row * 2) * PUE + (colx0 >> 1)) * PIX + j * 16 : 2 * G::PATCH;
    }
    uint4 stg[MAXU][8];
    auto stage_load = [&](int chunk) {
        const int cleft = a.C - chunk * CK;
        const int nrec = cleft > 0 ? cleft * HW2 : 0;
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint8_t*>(xn) + static_cast<long long>(chunk) * CK * HW2, 0, nrec, 0x00020000);
#pragma unroll
        for (int i = 0; i < MAXU; ++i)
#pragma unroll
            for (int l = 0; l < 8; ++l) {
                const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rs, u_voff[i] + l * HW2, 0, 0);
                stg[i][l] = make_uint4(v.x, v.y, v.z, v.w);
            }
    };
    auto stage_store = [&](int bufoff) {
#pragma unroll
        for (int i = 0; i < MAXU; ++i) {
            uint8_t* base = lds + bufoff + u_lds[i];
#pragma unroll
            for (int p = 0; p < 8; ++p) {
                const int off = (((PWO + p) & 1) * PUE + ((PWO + p) >> 1)) * PIX;
                uint4 o;
                o.x = cvt_pair(word_of(stg[i][0], p >> 1), word_of(stg[i][1], p >> 1), p & 1, xsc);
                o.y = cvt_pair(word_of(stg[i][2], p >> 1), word_of(stg[i][3], p >> 1), p & 1, xsc);
                o.z = cvt_pair(word_of(stg[i][4], p >> 1), word_of(stg[i][5], p >> 1), p & 1, xsc);
                o.w = cvt_pair(word_of(stg[i][6], p >> 1), word_of(stg[i][7], p >> 1), p & 1, xsc);
                *reinterpret_cast<uint4*>(base + off) = o;
            }
        }
    };

    const int ra = wave == 0 ? f2.ra[0] : wave == 1 ? f2.ra[1] : wave == 2 ? f2.ra[2] : f2.ra[3];
    const int rb = wave == 0 ? f2.rb[0] : wave == 1 ? f2.rb[1] : wave == 2 ? f2.rb[2] : f2.rb[3];
    const int sa = wave == 0 ? f2.sa[0] : wave == 1 ? f2.sa[1] : wave == 2 ? f2.sa[2] : f2.sa[3];
    const h2 sa2 = {static_cast<_Float16>(sa), static_cast<_Float16>(sa)};
    int tbase[2];
#pragma unroll
    for (int f = 0; f < 2; ++f) {
        const int s = m + 32 * f;
        const int tr = s / TCB, tc = s % TCB;
        tbase[f] = ((2 * tr) * 2 * PUE + tc + 4) * PIX + h * 16;
    }
    const int offA = ra * 2 * PUE * PIX, offB = rb * 2 * PUE * PIX;

    // prepared filter: [kt][chunk][xi][b (4)][ks][32 rows][half][16 B], 128 KiB
    // per (kt, chunk); this wave's four positions are 32 KiB
    constexpr int VCH = 16 * (KB2 / 32) * 2048;
    const uint8_t* __restrict__ vbase =
        a.v + static_cast<long long>(kt) * a.nchunks * VCH + wave * 4 * (KB2 / 32) * 2048 + m * 32 + h * 16;
    uint4 vb[4][4];  // [j][b] of the current k-step
    auto load_vb = [&](int chunk, int ks, int b) {
        const uint8_t* p = vbase + static_cast<long long>(chunk) * VCH + ks * 1024 + b * 2048;
#pragma unroll
        for (int j = 0; j < 4; ++j) vb[j][b] = *reinterpret_cast<const uint4*>(p + j * (KB2 / 32) * 2048);
    };

    uint4 da[4], db[4];
    auto read_d = [&](int bufoff, int ks, int f) {
        const uint8_t* q = lds + bufoff + tbase[f] + ks * 32;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const int co = ((c & 1) * PUE + (c >> 1)) * PIX;
            da[c] = *reinterpret_cast<const uint4*>(q + offA + co);
            db[c] = *reinterpret_cast<const uint4*>(q + offB + co);
        }
    };
    // U[j] for j = 0..3, and -U[j] in slot 4 + j where A^T needs it
    auto transform = [&](uint4 (&U)[8]) {
        h2 t[4][4];
#pragma unroll
        for (int c = 0; c < 4; ++c)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                t[c][e] = __builtin_bit_cast(h2, word_of(da[c], e)) * sa2 + __builtin_bit_cast(h2, word_of(db[c], e));
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            bool neg = false;
#pragma unroll
            for (int q = 0; q < 2; ++q) neg = neg || f2.at[q][j] < 0;
            uint32_t wp[4], wn[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                h2 s = {0, 0};
                bool first = true;
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    const int co = f2.bt[j][c];
                    if (co == 0) continue;
                    if (first) {
                        s = co > 0 ? t[c][e] : -t[c][e];
                        first = false;
                    } else {
                        s = co > 0 ? s + t[c][e] : s - t[c][e];
                    }
                }
                wp[e] = __builtin_bit_cast(uint32_t, s);
                wn[e] = wp[e] ^ 0x80008000u;
            }
            U[j] = make_uint4(wp[0], wp[1], wp[2], wp[3]);
            if (neg) U[4 + j] = make_uint4(wn[0], wn[1], wn[2], wn[3]);
        }
    };

    f32x16 acc[2][2][4];  // [q][f][b]
#pragma unroll
    for (int q = 0; q < 2; ++q)
#pragma unroll
        for (int f = 0; f < 2; ++f)
#pragma unroll
            for (int b = 0; b < 4; ++b) acc[q][f][b] = f32x16{};
    // MFMAs of channel fragment b of one step
    auto mma_b = [&](const uint4 (&U)[8], int f, int b) {
#pragma unroll
        for (int q = 0; q < 2; ++q)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int co = f2.at[q][j];
                if (co == 0) continue;
                acc[q][f][b] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
                    __builtin_bit_cast(f16x8, co > 0 ? U[j] : U[4 + j]), __builtin_bit_cast(f16x8, vb[j][b]),
                    acc[q][f][b], 0, 0, 0);
            }
    };
    // one step: its 24 MFMAs with the next step's VALU work between them;
    // with `reload`, each channel fragment's filter is reloaded for
    // (rchunk, rks) right after its last MFMA of this k-step
    auto step = [&](const uint4 (&U)[8], int f, bool reload, int rchunk, int rks) {
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            mma_b(U, f, b);
            if (reload) load_vb(rchunk, rks, b);
        }
    };

    // ---- prologue
    stage_load(0);
#pragma unroll
    for (int b = 0; b < 4; ++b) load_vb(0, 0, b);
    stage_store(0);
    __syncthreads();
    uint4 ucur[8], unext[8];
    read_d(0, 0, 0);
    transform(ucur);
    read_d(0, 0, 1);
    __builtin_amdgcn_s_waitcnt(0);

    for (int chunk = 0; chunk < a.nchunks; ++chunk) {
        const int cur = (chunk & 1) * G::PATCH;
        const int nb = G::PATCH - cur;
        const int nxt = chunk + 1 < a.nchunks ? chunk + 1 : chunk;
        stage_load(chunk + 1);
        __builtin_amdgcn_sched_barrier(0);
        // step (ks 0, f 0)
        step(ucur, 0, false, 0, 0);
        transform(unext);
        interleave3<4>();
        __builtin_amdgcn_sched_barrier(0);
        read_d(cur, 1, 0);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int j = 0; j < 8; ++j) ucur[j] = unext[j];
        // step (0, 1): the last use of k-step 0's filter; reload k-step 1's
        step(ucur, 1, true, chunk, 1);
        transform(unext);
        interleave3<4>();
        __builtin_amdgcn_sched_barrier(0);
        read_d(cur, 1, 1);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int j = 0; j < 8; ++j) ucur[j] = unext[j];
        // step (1, 0), with the next chunk's staging stores
        step(ucur, 0, false, 0, 0);
        transform(unext);
        stage_store(nb);
        interleave3<8>();
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int j = 0; j < 8; ++j) ucur[j] = unext[j];
        __syncthreads();
        read_d(nb, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
        // step (1, 1): last use of k-step 1's filter; reload the next chunk's
        // k-step 0
        step(ucur, 1, true, nxt, 0);
        transform(unext);
        interleave3<4>();
        __builtin_amdgcn_sched_barrier(0);
        read_d(nb, 0, 1);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int j = 0; j < 8; ++j) ucur[j] = unext[j];
    }
    __syncthreads();

    // ---- output transform, one half of the channel fragments at a time:
    // accumulator v of fragment (q, f, b) is Z[w][q] of tile slot
    // 32f + 8(v/4) + 4h + v%4 and output channel 32b + m
    float* Zs = reinterpret_cast<float*>(lds);
    constexpr int GPR = TCB / 4;
    const bool vec_ok = (a.OW % 8) == 0;
    // whole-row runs: one column block spans the output width, the 2TR rows
    // lie inside the output, and rows are whole 16-byte pieces
    const bool runs = vec_ok && a.tbw == 1 && 2 * (tr0 + TR) <= a.OH;
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
#pragma unroll
        for (int bb = 0; bb < 2; ++bb)
#pragma unroll
            for (int f = 0; f < 2; ++f)
#pragma unroll
                for (int v4 = 0; v4 < 4; ++v4) {
                    const int b = 2 * hb + bb;
                    float z[8];
#pragma unroll
                    for (int vv = 0; vv < 4; ++vv) {
                        z[2 * vv] = acc[0][f][b][4 * v4 + vv];
                        z[2 * vv + 1] = acc[1][f][b][4 * v4 + vv];
                    }
                    const int s0 = 32 * f + 8 * v4 + 4 * h;
                    float* dst = Zs + (wave * 64 + 32 * bb + m) * ZP + 2 * s0;
                    *reinterpret_cast<float4*>(dst) = make_float4(z[0], z[1], z[2], z[3]);
                    *reinterpret_cast<float4*>(dst + 4) = make_float4(z[4], z[5], z[6], z[7]);
                }
        __syncthreads();
        if (runs) {
            // the block covers whole output rows: each channel's 2TR rows are
            // one contiguous run of 2TR * OW outputs, written as consecutive
            // 16-byte pieces (8 columns of one row) by consecutive lanes
            const int ppr = a.OW / 8;        // pieces per row
            const int ppc = 2 * TR * ppr;    // pieces per channel
            const int nk = min(64, a.K - (kt * KB2 + hb * 64));
            uint16_t* ybase = a.y + n * a.y_img + static_cast<long long>(kt * KB2 + hb * 64) * a.OH * a.OW +
                              static_cast<long long>(2 * tr0) * a.OW;
            for (int job = tid; job < nk * ppc; job += NTHR) {
                const int kl = job / ppc;
                const int pc = job - kl * ppc;
                const int row = pc / ppr;
                const int g = pc - row * ppr;
                const int tr = row >> 1, p = row & 1;
                const int pos0 = tr * 2 * TCB + 8 * g;
                float yv[8] = {};
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    const int co = f2.at[p][w];
                    const float* src = Zs + (w * 64 + kl) * ZP + pos0;
                    const float4 lo = *reinterpret_cast<const float4*>(src);
                    const float4 hi = *reinterpret_cast<const float4*>(src + 4);
                    const float zz[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        if (co > 0) yv[e] += zz[e];
                        if (co < 0) yv[e] -= zz[e];
                    }
                }
#pragma unroll
                for (int e = 0; e < 8; ++e) yv[e] = wg_denorm(yv[e], osx, osw);
                if constexpr (EPI)
                    epi8(yv, a.e, kt * KB2 + hb * 64 + kl,
                         (ybase - a.y) + static_cast<long long>(kl) * a.OH * a.OW + pc * 8, 8);
                const u32x4 o = {pack_bf16x2(yv[0], yv[1]), pack_bf16x2(yv[2], yv[3]), pack_bf16x2(yv[4], yv[5]),
                                 pack_bf16x2(yv[6], yv[7])};
                __builtin_nontemporal_store(
                    o, reinterpret_cast<u32x4*>(ybase + static_cast<long long>(kl) * a.OH * a.OW + pc * 8));
            }
            __syncthreads();
            continue;
        }
        for (int job = tid; job < 64 * TR * GPR; job += NTHR) {
            const int g = job % GPR;
            const int rest = job / GPR;
            const int tr = rest % TR;
            const int kl = rest / TR;
            const int k = kt * KB2 + hb * 64 + kl;
            if (k >= a.K) continue;
            const int pos0 = tr * 2 * TCB + 8 * g;
            float z[4][8];
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                const float* src = Zs + (w * 64 + kl) * ZP + pos0;
                const float4 lo = *reinterpret_cast<const float4*>(src);
                const float4 hi = *reinterpret_cast<const float4*>(src + 4);
                z[w][0] = lo.x; z[w][1] = lo.y; z[w][2] = lo.z; z[w][3] = lo.w;
                z[w][4] = hi.x; z[w][5] = hi.y; z[w][6] = hi.z; z[w][7] = hi.w;
            }
            const int ow0 = 2 * tc0 + 8 * g;
#pragma unroll
            for (int p = 0; p < 2; ++p) {
                const int oh = 2 * (tr0 + tr) + p;
                if (oh >= a.OH) continue;
                float yv[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    float s = 0.0f;
#pragma unroll
                    for (int w = 0; w < 4; ++w) {
                        const int co = f2.at[p][w];
                        if (co > 0) s += z[w][e];
                        if (co < 0) s -= z[w][e];
                    }
                    yv[e] = wg_denorm(s, osx, osw);
                }
                const long long yo = n * a.y_img + (static_cast<long long>(k) * a.OH + oh) * a.OW + ow0;
                if constexpr (EPI) epi8(yv, a.e, k, yo, a.OW - ow0);
                uint16_t* dst = a.y + yo;
                if (vec_ok && ow0 + 8 <= a.OW) {
                    const u32x4 o = {pack_bf16x2(yv[0], yv[1]), pack_bf16x2(yv[2], yv[3]), pack_bf16x2(yv[4], yv[5]),
                                     pack_bf16x2(yv[6], yv[7])};
                    __builtin_nontemporal_store(o, reinterpret_cast<u32x4*>(dst));
                } else {
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        if (ow0 + e < a.OW) dst[e] = float_to_bf16(yv[e]);
                }
            }
        }
        __syncthreads();
    }
}

// ---------------------------------------------------------------- filter prepare
// V[kt][chunk][xi = 4i + j][b][ks][m][h][8 fp16] = (G' g G'^T)[i][j] for output
// channel kt*KBT + 32b + m (KBT = 64 for config 1, 128 for config 2) and input channel chunk*32 + 16ks + 8h + e; zero past
// K and C.
template <int KBT>
__global__ __launch_bounds__(256) void wf2_prepare_kernel(const uint16_t* __restrict__ w, _Float16* __restrict__ out,
                                                          int K, int C, int ntk, int nchunks,
                                                          const unsigned* __restrict__ wmax) {
    constexpr F2 f2 = build_f2();
    const float wsc = wg_norm(wmax);  // filter scale into the fp16 range
    const long long total = static_cast<long long>(ntk) * KBT * nchunks * CK;
    for (long long idx = blockIdx.x * 256LL + threadIdx.x; idx < total; idx += static_cast<long long>(gridDim.x) * 256) {
        const int c = static_cast<int>(idx % (nchunks * CK));
        const int k = static_cast<int>(idx / (nchunks * CK));
        float gg[3][3] = {};
        if (k < K && c < C)
            for (int r = 0; r < 3; ++r)
                for (int s = 0; s < 3; ++s) gg[r][s] = bf16_to_float(w[(static_cast<long long>(k) * C + c) * 9 + r * 3 + s]);
        float tmp[4][3];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int s = 0; s < 3; ++s) {
                float acc = 0.0f;
#pragma unroll
                for (int r = 0; r < 3; ++r) acc = fmaf(f2.gp[i][r], gg[r][s], acc);
                tmp[i][s] = acc;
            }
        const int kt = k / KBT, kl = k % KBT, b = kl / 32, mm = kl % 32;
        const int chunk = c / CK, cl = c % CK, ks = cl / 16, hh = (cl % 16) / 8, e = cl % 8;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                float acc = 0.0f;
#pragma unroll
                for (int s = 0; s < 3; ++s) acc = fmaf(tmp[i][s], f2.gp[j][s], acc);
                const long long base =
                    ((((((static_cast<long long>(kt) * nchunks + chunk) * 16 + (4 * i + j)) * (KBT / 32) + b) * 2 + ks) * 32 +
                      mm) * 2 + hh) * 8 + e;
                out[base] = static_cast<_Float16>(acc * wsc);
            }
    }
}

struct Plan {
    int tcb, tr, th, tw, tbh, tbw, ntk, nchunks, nblk;
    size_t v_bytes;
};

inline bool plan(const Prob& p, int kb, Plan* pl, std::string* why) {
    auto no = [&](const char* s) {
        if (why) *why = s;
        return false;
    };
    if (p.r != 3 || p.s != 3 || p.sh != 1 || p.sw != 1 || p.dh != 1 || p.dw != 1 || p.g != 1)
        return no("winograd fused: needs 3x3, stride 1, dilation 1, groups 1");
    if (p.dtype != CFWD_BF16) return no("winograd fused: bf16 only");
    if (p.xb != 1) return no("winograd fused: NCHW only");
    if (p.ph > 1 || p.pw > 1) return no("winograd fused: padding 0 or 1 only");
    if (p.w % 8 != 0) return no("winograd fused: W must be a multiple of 8 (16-byte row loads)");
    if (p.oh < 1 || p.ow < 1) return no("winograd fused: empty output");
    // staging offsets are 32-bit: one chunk of 32 channel planes must stay under 2 GiB
    if (static_cast<long long>(p.h) * p.w * 64 >= (1LL << 31)) return no("winograd fused: channel planes too large");
    pl->th = (p.oh + 1) / 2;
    pl->tw = (p.ow + 1) / 2;
    pl->tcb = pl->tw > 16 ? 32 : (pl->tw > 8 ? 16 : 8);
    pl->tr = TBL / pl->tcb;
    pl->tbh = (pl->th + pl->tr - 1) / pl->tr;
    pl->tbw = (pl->tw + pl->tcb - 1) / pl->tcb;
    pl->ntk = (p.k + kb - 1) / kb;
    pl->nchunks = (p.c + CK - 1) / CK;
    const int pw_cols = 2 * pl->tcb + 2;
    const int first = (p.pw > 0) ? -1 : 0;  // floor(-pw / 8)
    const int last = (-p.pw + pw_cols - 1) / 8;
    pl->nblk = last - first + 1;
    const long long blocks = static_cast<long long>(p.n) * pl->tbh * pl->tbw * pl->ntk;
    if (blocks > (1LL << 31) - 1) return no("winograd fused: too many workgroups");
    pl->v_bytes = static_cast<size_t>(pl->ntk) * pl->nchunks * 16 * kb * CK * 2;
    return true;
}

template <int TCB, int PWO, bool FOLD>
cfwd_status launch_tcb(const Prob& p, const Plan& pl, const void* x, const void* vp, void* y, const Epi& e,
                       const unsigned* xmax, const unsigned* wmax, hipStream_t st) {
    using G = Geo<TCB>;
    static_assert(G::LDS <= 160 * 1024, "LDS budget");
    if (pl.nblk > G::NBMAX) return set_error(CFWD_ERR_UNSUPPORTED, "winograd fused: patch wider than planned");
    const bool epi = e.bias || e.res || e.relu;
    static bool attr[2] = {false, false};
    auto kern = FOLD ? (epi ? wf2f_kernel<TCB, PWO, true> : wf2f_kernel<TCB, PWO, false>)
                     : (epi ? wf2_kernel<TCB, PWO, true> : wf2_kernel<TCB, PWO, false>);
    cfwd_status s = ig::allow_big_lds(kern, G::LDS, &attr[epi]);
    if (s != CFWD_OK) return s;
    Args a;
    a.x = static_cast<const uint16_t*>(x);
    a.v = static_cast<const uint8_t*>(vp);
    a.y = static_cast<uint16_t*>(y);
    a.N = p.n; a.C = p.c; a.H = p.h; a.W = p.w; a.K = p.k; a.OH = p.oh; a.OW = p.ow; a.ph = p.ph; a.pw = p.pw;
    a.x_img = p.x_img; a.y_img = p.y_img;
    a.tbh = pl.tbh; a.tbw = pl.tbw; a.ntk = pl.ntk; a.nchunks = pl.nchunks; a.nblk = pl.nblk;
    a.e = e;
    a.xmax = xmax;
    a.wmax = wmax;
    const unsigned blocks = static_cast<unsigned>(static_cast<long long>(p.n) * pl.tbh * pl.tbw * pl.ntk);
    kern<<<blocks, NTHR, G::LDS, st>>>(a);
    return check_hip(hipGetLastError(), "winograd fused launch");
}

template <bool FOLD>
cfwd_status launch_fold(const Prob& p, const Plan& pl, const void* x, const void* wp, void* y, const Epi& e,
                        const unsigned* xmax, const unsigned* wmax, hipStream_t st) {
    const bool p1 = p.pw == 1;
    switch (pl.tcb) {
        case 32:
            return p1 ? launch_tcb<32, 1, FOLD>(p, pl, x, wp, y, e, xmax, wmax, st) : launch_tcb<32, 0, FOLD>(p, pl, x, wp, y, e, xmax, wmax, st);
        case 16:
            return p1 ? launch_tcb<16, 1, FOLD>(p, pl, x, wp, y, e, xmax, wmax, st) : launch_tcb<16, 0, FOLD>(p, pl, x, wp, y, e, xmax, wmax, st);
        default:
            return p1 ? launch_tcb<8, 1, FOLD>(p, pl, x, wp, y, e, xmax, wmax, st) : launch_tcb<8, 0, FOLD>(p, pl, x, wp, y, e, xmax, wmax, st);
    }
}

inline int kb_of(int cfg) { return cfg == 2 ? KB2 : KB; }

}  // namespace wf

// cfg 1: the fused kernel (64 output channels per workgroup); cfg 2: the
// folded form (128 output channels per workgroup).
bool winograd_fused_supported(const Prob& p, int cfg, std::string* why) {
    wf::Plan pl;
    return wf::plan(p, wf::kb_of(cfg), &pl, why);
}

size_t winograd_fused_filter_bytes(const Prob& p, int cfg) {
    wf::Plan pl;
    // the transformed filter, then 8 KiB holding its largest magnitude
    return wf::plan(p, wf::kb_of(cfg), &pl, nullptr) ? pl.v_bytes + 8192 : 0;
}

cfwd_status winograd_fused_prepare(const Prob& p, int cfg, const void* w, void* wp, hipStream_t st) {
    wf::Plan pl;
    std::string why;
    const int kb = wf::kb_of(cfg);
    if (!wf::plan(p, kb, &pl, &why)) return set_error(CFWD_ERR_UNSUPPORTED, why);
    const long long total = static_cast<long long>(pl.ntk) * kb * pl.nchunks * wf::CK;
    const unsigned nb = static_cast<unsigned>(std::min<long long>((total + 255) / 256, 65536));
    unsigned* wmax = reinterpret_cast<unsigned*>(static_cast<uint8_t*>(wp) + pl.v_bytes);
    cfwd_status s = bf16_absmax(w, static_cast<long long>(p.k) * p.c * 9, wmax, st);
    if (s != CFWD_OK) return s;
    if (kb == wf::KB2)
        wf::wf2_prepare_kernel<wf::KB2><<<nb, 256, 0, st>>>(static_cast<const uint16_t*>(w), static_cast<_Float16*>(wp),
                                                             p.k, p.c, pl.ntk, pl.nchunks, wmax);
    else
        wf::wf2_prepare_kernel<wf::KB><<<nb, 256, 0, st>>>(static_cast<const uint16_t*>(w), static_cast<_Float16*>(wp),
                                                            p.k, p.c, pl.ntk, pl.nchunks, wmax);
    return check_hip(hipGetLastError(), "winograd fused filter transform launch");
}

cfwd_status winograd_fused_launch(const Prob& p, int cfg, const void* x, const void* wp, void* scratch, void* y,
                                  const Epi& e, hipStream_t st) {
    wf::Plan pl;
    std::string why;
    if (!wf::plan(p, wf::kb_of(cfg), &pl, &why)) return set_error(CFWD_ERR_UNSUPPORTED, why);
    if (wp == nullptr || scratch == nullptr)
        return set_error(CFWD_ERR_WORKSPACE, "winograd fused: prepared filter and scratch are required");
    // this call's largest input magnitude, in the scratch
    unsigned* xmax = static_cast<unsigned*>(scratch);
    cfwd_status s = bf16_absmax(x, static_cast<long long>(p.n) * p.x_img, xmax, st);
    if (s != CFWD_OK) return s;
    const unsigned* wmax = reinterpret_cast<const unsigned*>(static_cast<const uint8_t*>(wp) + pl.v_bytes);
    return cfg == 2 ? wf::launch_fold<true>(p, pl, x, wp, y, e, xmax, wmax, st)
                    : wf::launch_fold<false>(p, pl, x, wp, y, e, xmax, wmax, st);
}

}  // namespace cfwd
