// Winograd minimal filtering F(m x m, 3 x 3), m = 2 or 6 (gfx950).
//
// MegEngine inference article, section "Winograd": F(2x2,3x3) and F(6x6,3x3)
// trade multiplies for additions (2.25x and 5.06x fewer), in three steps --
// transform the input tiles and the weights, multiply the transformed tiles as
// a batched matrix product, transform the products back -- and its
// engineering subsection blocks the tiles so one block's working set stays in
// cache.  Momenta talk, section "優化3：FFT / Winograd的卷積演算法": accuracy
// drops as the tile grows.
//
// Construction (written from the mathematics, here at compile time): with
// alpha = m + 2 interpolation points (one may be "infinity", which evaluates a
// polynomial to its leading coefficient), V_n evaluates an n-coefficient
// polynomial at the points; linear convolution is V^-1 [(V_3 g) * (V_m u)] and
// correlation is its transpose, so A^T = V_m^T, G = V_3, B^T = V^-T and
//   Y = A^T [ (G g G^T) * (B^T d B) ] A   over alpha x alpha input tiles d.
// Points: {0, 1, -1, inf} for m = 2; {0, +-1, +-2, +-1/2, inf} for m = 6.
//
// GPU structure (stride 1, dilation 1, groups 1, R = S = 3):
//   prepare  V[xi][c][k] = (G g G^T)[xi] per (k, c), laid out like the
//            implicit-GEMM B operand (32-column fragments, 64-byte K chunks);
//   input    U[xi][chunk][tile][CK] = (B^T d B)[xi]: one thread per (tile,
//            channel group), written channel-contiguous;
//   gemm     per workgroup a block of TB tiles x KB output channels for all
//            alpha^2 positions (split over the waves: four for F(2x2), eight
//            for F(6x6)), reduced over the
//            input channels on the matrix cores; the alpha^2 products of each
//            (tile, channel) are then exchanged through LDS in channel slices
//            and transformed back, Y = A^T M A, straight into the output.
// bf16 inputs use fp16 transformed operands (fp16 keeps 11 bits; the
// transform entries reach 32, so bf16's 8 bits lose too much for F(6x6)); fp32
// inputs keep fp32 operands on the fp32 matrix cores.  Accumulation is fp32.
#include <type_traits>

#include "igemm_impl.h"
#include "winograd_i8.h"
#include "winograd_mats.h"
#include "winograd_f6_fused.h"

namespace cfwd {
namespace wg {

using ig::f32x16;

// ------------------------------------------------------------ operand types

template <typename T> struct OpT;       // transformed operand storage
template <> struct OpT<float> {
    using type = float;
    static __device__ __forceinline__ float from(float v) { return v; }
};
template <> struct OpT<bf16_t> {
    using type = _Float16;
    static __device__ __forceinline__ _Float16 from(float v) { return static_cast<_Float16>(v); }
};
// int8 F(2x2): B^T d B holds multiples of 1/4 of magnitude <= 512 and G g G^T
// integers of magnitude <= 1152 (G has entries 0, +-1), both exact in fp16
template <> struct OpT<int8_t> {
    using type = _Float16;
    static __device__ __forceinline__ _Float16 from(float v) { return static_cast<_Float16>(v); }
};

// 32x32 fragments with fp16 operands (bf16 inputs) or fp32 operands.
template <typename T> struct WMma;
template <> struct WMma<bf16_t> {
    static __device__ __forceinline__ void piece(f32x16& c, const uint4& a, const uint4& b) {
        c = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0,
                                                   0, 0);
    }
    static constexpr int pslot(int i, int h) { return 2 * i + h; }
};
template <> struct WMma<int8_t> : WMma<bf16_t> {};
template <> struct WMma<float> {
    static __device__ __forceinline__ void piece(f32x16& c, const uint4& a, const uint4& b) {
        c = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.x), __uint_as_float(b.x), c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.y), __uint_as_float(b.y), c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.z), __uint_as_float(b.z), c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.w), __uint_as_float(b.w), c, 0, 0, 0);
    }
    static constexpr int pslot(int i, int h) { return 2 * h + i; }
};

// ------------------------------------------------------------ geometry

struct Geo {
    int m, alpha, xi;       // tile size, alpha = m + 2, alpha^2
    int th, tw, T, Tpad;    // tiles per image row/col, total tiles, padded to TB
    int CK, nchunks;        // channels per 64-byte chunk, chunks
    int TB, KB, ntk, ntb;   // tile block, output-channel block, block counts
    size_t u_bytes;         // transformed-input workspace
    size_t v_bytes;         // prepared filter
    size_t hdr;             // bf16: 8 KiB after each for the operand maxima (wg_norm)
};

inline bool geometry(const Prob& p, int m, Geo* g, std::string* why) {
    if (p.r != 3 || p.s != 3 || p.sh != 1 || p.sw != 1 || p.dh != 1 || p.dw != 1 || p.g != 1) {
        if (why) *why = "winograd: needs 3x3, stride 1, dilation 1, groups 1";
        return false;
    }
    if (p.dtype == CFWD_I8 && m != 2) {
        if (why) *why = "winograd: int8 only with F(2x2) (the F(6x6) transforms are not exact in fp16)";
        return false;
    }
    g->m = m;
    g->alpha = m + 2;
    g->xi = g->alpha * g->alpha;
    g->th = (p.oh + m - 1) / m;
    g->tw = (p.ow + m - 1) / m;
    const long long T = static_cast<long long>(p.n) * g->th * g->tw;
    if (T > (1LL << 30)) {
        if (why) *why = "winograd: too many tiles";
        return false;
    }
    g->T = static_cast<int>(T);
    g->TB = (m == 6) ? 32 : 64;
    g->KB = (m == 6) ? 32 : 64;
    g->Tpad = (g->T + g->TB - 1) / g->TB * g->TB;
    g->CK = (p.dtype == CFWD_F32) ? 16 : 32;
    g->nchunks = (p.c + g->CK - 1) / g->CK;
    g->ntk = (p.k + g->KB - 1) / g->KB;
    g->ntb = g->Tpad / g->TB;
    g->u_bytes = static_cast<size_t>(g->xi) * g->nchunks * g->Tpad * 64;
    g->v_bytes = static_cast<size_t>(g->xi) * g->ntk * g->nchunks * g->KB * 64;
    g->hdr = (p.dtype == CFWD_BF16) ? 8192 : 0;
    return true;
}

// ------------------------------------------------------------ filter prepare
// V[xi][kt][chunk][KB/32 frags][piece][32 rows][half][16 B] = G g G^T, in the
// operand type; rows past K and channels past C are zero.

template <typename T, int M>
__global__ __launch_bounds__(256) void prepare_kernel(const T* __restrict__ w, uint8_t* __restrict__ out, int K, int C,
                                                      int KB, int ntk, int nchunks, const unsigned* __restrict__ wmax) {
    using O = typename OpT<T>::type;
    const float wsc = wg_norm(wmax);  // bf16: filter scale for the fp16 range
    constexpr int A = M + 2;
    constexpr int E16 = 16 / static_cast<int>(sizeof(O));
    constexpr int CK = 4 * E16;
    constexpr Mats<M> mt = build_mats<M>();
    // one thread per (k, c): transform, then scatter the alpha^2 values
    const long long total = static_cast<long long>(ntk) * KB * nchunks * CK;
    for (long long idx = blockIdx.x * 256LL + threadIdx.x; idx < total; idx += static_cast<long long>(gridDim.x) * 256) {
        const int c = static_cast<int>(idx % (nchunks * CK));
        const int k = static_cast<int>(idx / (nchunks * CK));
        float gg[3][3] = {};
        if (k < K && c < C)
            for (int r = 0; r < 3; ++r)
                for (int s = 0; s < 3; ++s) gg[r][s] = Elem<T>::to_f(w[(static_cast<long long>(k) * C + c) * 9 + r * 3 + s]);
        float tmp[A][3];
#pragma unroll
        for (int i = 0; i < A; ++i)
#pragma unroll
            for (int s = 0; s < 3; ++s) {
                float acc = 0.0f;
#pragma unroll
                for (int r = 0; r < 3; ++r) acc = fmaf(static_cast<float>(mt.g[i][r]), gg[r][s], acc);
                tmp[i][s] = acc;
            }
        const int kt = k / KB, kl = k % KB;
        const int chunk = c / CK, cc = c % CK;
        const int slot = cc / E16, e = cc % E16;
        // which (piece, half) holds this slot
        int piece = 0, half = 0;
        for (int i = 0; i < 2; ++i)
            for (int h = 0; h < 2; ++h)
                if (WMma<T>::pslot(i, h) == slot) {
                    piece = i;
                    half = h;
                }
        const int nfr = kl / 32, row = kl % 32;
#pragma unroll
        for (int i = 0; i < A; ++i)
#pragma unroll
            for (int j = 0; j < A; ++j) {
                float acc = 0.0f;
#pragma unroll
                for (int s = 0; s < 3; ++s) acc = fmaf(tmp[i][s], static_cast<float>(mt.g[j][s]), acc);
                const int x = i * A + j;
                const long long base =
                    ((((static_cast<long long>(x) * ntk + kt) * nchunks + chunk) * (KB / 32) + nfr) * 2 + piece) * 32 + row;
                O* dst = reinterpret_cast<O*>(out + (base * 2 + half) * 16) + e;
                *dst = OpT<T>::from(acc * wsc);
            }
    }
}

// ------------------------------------------------------------ input transform
// U[xi][chunk][tile][CK], tile = (n * th + ty) * tw + tx; padded tiles are 0.
// A workgroup covers TXB consecutive tiles of one tile row and one channel
// chunk: the alpha input rows they read are staged in LDS with loads
// coalesced along W ([row][col][channel], fp32), then thread (tile, channel)
// transforms its alpha x alpha tile and the lanes of one tile write the
// chunk's CK channels as one contiguous 64-byte run per position.

template <int M, int CK> struct InGeo {
    static constexpr int A = M + 2;
    static constexpr int TXB = 256 / CK;               // tiles per workgroup
    static constexpr int COLS = TXB * M + 2;           // input columns staged
    static constexpr int LDS_FLOATS = A * COLS * CK;
};

template <typename T, int XB, int M>
__global__ __launch_bounds__(256) void input_kernel(const T* __restrict__ x, uint8_t* __restrict__ U, int N, int C, int H,
                                                    int W, int ph, int pw, long long x_img, int th, int tw, int T_,
                                                    int Tpad, int nchunks, int tblocks_w,
                                                    const unsigned* __restrict__ xmax) {
    using O = typename OpT<T>::type;
    const float xsc = wg_norm(xmax);  // bf16: input scale for the fp16 range
    constexpr int A = M + 2;
    constexpr int CK = 64 / static_cast<int>(sizeof(O));
    using IG = InGeo<M, CK>;
    constexpr int TXB = IG::TXB;
    constexpr int COLS = IG::COLS;
    constexpr Mats<M> mt = build_mats<M>();
    __shared__ float patch[IG::LDS_FLOATS];

    // block -> (image n, tile row ty, tile column block bx, chunk)
    int b = blockIdx.x;
    const int bx = b % tblocks_w;
    b /= tblocks_w;
    const int ty = b % th;
    const int n = b / th;
    const int chunk = blockIdx.y;
    const int tx0 = bx * TXB;
    const int ih0 = ty * M - ph, iw0 = tx0 * M - pw;
    const T* xn = x + n * x_img;

    // stage: A rows x COLS cols x CK channels, column fastest across threads
    for (int e = threadIdx.x; e < A * COLS * CK; e += 256) {
        const int col = e % COLS;
        const int t = e / COLS;
        const int row = t % A;
        const int cc = t / A;
        const int c = chunk * CK + cc;
        const int ih = ih0 + row, iw = iw0 + col;
        float v = 0.0f;
        if (c < C && ih >= 0 && ih < H && iw >= 0 && iw < W) v = Elem<T>::to_f(xn[act_off<XB>(c, ih, iw, H, W)]);
        patch[(row * COLS + col) * CK + cc] = v;
    }
    __syncthreads();

    const int cc = threadIdx.x % CK;
    const int tl = threadIdx.x / CK;
    const int tx = tx0 + tl;
    int tile = (n * th + ty) * tw + tx;
    const bool real = tx < tw;
    float d[A][A];
#pragma unroll
    for (int i = 0; i < A; ++i)
#pragma unroll
        for (int j = 0; j < A; ++j) d[i][j] = patch[(i * COLS + tl * M + j) * CK + cc];
    float t[A][A];
#pragma unroll
    for (int i = 0; i < A; ++i)
#pragma unroll
        for (int j = 0; j < A; ++j) {
            float acc = 0.0f;
#pragma unroll
            for (int k = 0; k < A; ++k) {
                const float bk = static_cast<float>(mt.bt[i][k]);
                if (bk != 0.0f) acc = fmaf(bk, d[k][j], acc);
            }
            t[i][j] = acc;
        }
    if (!real) return;
    O* dst = reinterpret_cast<O*>(U + (static_cast<long long>(chunk) * Tpad + tile) * 64) + cc;
    const long long xstride = static_cast<long long>(nchunks) * Tpad * 64 / static_cast<long long>(sizeof(O));
#pragma unroll
    for (int i = 0; i < A; ++i)
#pragma unroll
        for (int j = 0; j < A; ++j) {
            float acc = 0.0f;
#pragma unroll
            for (int k = 0; k < A; ++k) {
                const float bk = static_cast<float>(mt.bt[j][k]);
                if (bk != 0.0f) acc = fmaf(t[i][k], bk, acc);
            }
            dst[(i * A + j) * xstride] = OpT<T>::from(acc * xsc);
        }
}

// Largest magnitude of n bf16 values, as a bit pattern with the sign
// cleared (for non-negative values the bit patterns order like the values):
// each of kAbsmaxBlocks workgroups writes the maximum of its share to a slot,
// then one workgroup reduces the slots (no atomics, nothing to clear first).
constexpr int kAbsmaxBlocks = 1024;

__device__ __forceinline__ unsigned block_max(unsigned m) {
    __shared__ unsigned part[4];
    for (int off = 32; off > 0; off >>= 1) m = max(m, static_cast<unsigned>(__shfl_down(static_cast<int>(m), off)));
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = m;
    __syncthreads();
    return max(max(part[0], part[1]), max(part[2], part[3]));
}

__global__ __launch_bounds__(256) void bf16_absmax_partial(const uint16_t* __restrict__ x, long long n,
                                                           unsigned* __restrict__ slots) {
    unsigned m = 0;
    const long long n8 = n / 8;
    const uint4* x8 = reinterpret_cast<const uint4*>(x);
    const long long stride = static_cast<long long>(gridDim.x) * 256;
    // four independent 16-byte loads in flight per thread
    long long i = blockIdx.x * 256LL + threadIdx.x;
    for (; i + 3 * stride < n8; i += 4 * stride) {
        uint4 v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) v[u] = x8[i + u * stride];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const uint32_t w4[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
            for (int q = 0; q < 4; ++q) m = max(m, max(w4[q] & 0x7fffu, (w4[q] >> 16) & 0x7fffu));
        }
    }
    for (; i < n8; i += stride) {
        const uint4 v = x8[i];
        const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int q = 0; q < 4; ++q) m = max(m, max(w4[q] & 0x7fffu, (w4[q] >> 16) & 0x7fffu));
    }
    for (long long t = n8 * 8 + blockIdx.x * 256LL + threadIdx.x; t < n; t += stride)
        m = max(m, static_cast<unsigned>(x[t]) & 0x7fffu);
    m = block_max(m);
    if (threadIdx.x == 0) slots[blockIdx.x] = m;
}

__global__ __launch_bounds__(256) void absmax_final(const unsigned* __restrict__ slots, unsigned* __restrict__ out) {
    unsigned m = 0;
    for (int i = threadIdx.x; i < kAbsmaxBlocks; i += 256) m = max(m, slots[i]);
    m = block_max(m);
    if (threadIdx.x == 0) *out = m;
}

// Zero rows of U for the padding tiles T .. Tpad-1 (they feed the last tile
// block's MFMAs; their outputs are discarded, but must not be NaN garbage).
__global__ __launch_bounds__(256) void zero_pad_tiles(uint8_t* __restrict__ U, int xi_chunks, int T_, int Tpad) {
    const int per = (Tpad - T_) * 4;  // uint4 per (xi, chunk)
    const long long total = static_cast<long long>(xi_chunks) * per;
    for (long long i = blockIdx.x * 256LL + threadIdx.x; i < total; i += static_cast<long long>(gridDim.x) * 256) {
        const long long xc = i / per;
        const int r = static_cast<int>(i % per);
        *reinterpret_cast<uint4*>(U + (xc * Tpad + T_) * 64 + r * 16) = make_uint4(0, 0, 0, 0);
    }
}

// ------------------------------------------------------------ batched GEMM + output transform
// Workgroup: TB tiles x KB output channels, all alpha^2 positions; wave w owns
// positions [w * XPW, (w+1) * XPW).  Operands come straight from L2:
// U (A operand, rows = tiles) and V (B operand, columns = output channels),
// each lane feeding two 16-byte K pieces per 64-byte chunk.

template <int M> struct GemmGeo {
    static constexpr int NW = (M == 6) ? 8 : 4;  // waves: positions split over them
    static constexpr int NTHR = NW * 64;
};

template <typename T, int XB, int M, bool EPI>  // EPI: fused epilogue compiled in
__global__ __launch_bounds__(GemmGeo<M>::NTHR) void gemm_kernel(const uint8_t* __restrict__ U, const uint8_t* __restrict__ V,
                                                   T* __restrict__ y, int K, int OH, int OW, long long y_img, int th,
                                                   int tw, int T_, int Tpad, int nchunks, int ntk, Epi ep,
                                                   const unsigned* __restrict__ xmax, const unsigned* __restrict__ wmax,
                                                   const float* __restrict__ scale) {
    constexpr int A = M + 2;
    constexpr int XI = A * A;
    constexpr int NW = GemmGeo<M>::NW;
    constexpr int NTHR = GemmGeo<M>::NTHR;
    constexpr int XPW = XI / NW;              // positions per wave
    constexpr int TB = (M == 6) ? 32 : 64;
    constexpr int KB = (M == 6) ? 32 : 64;
    constexpr int TF = TB / 32, KF = KB / 32;  // fragments per wave per position
    constexpr Mats<M> mt = build_mats<M>();
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int lrow = lane & 31, h = lane >> 5;
    const int osx = wg_shift(xmax), osw = wg_shift(wmax);  // bf16: shifts undoing the operand scales
    // tile block fastest: consecutive workgroups share the same filter slice
    const int tb = blockIdx.x % (Tpad / TB);
    const int kt = blockIdx.x / (Tpad / TB);

    f32x16 acc[XPW][TF][KF];
#pragma unroll
    for (int x = 0; x < XPW; ++x)
#pragma unroll
        for (int a = 0; a < TF; ++a)
#pragma unroll
            for (int b = 0; b < KF; ++b) acc[x][a][b] = f32x16{};

    const int ps0 = WMma<T>::pslot(0, h), ps1 = WMma<T>::pslot(1, h);
    // operands of one (chunk, position) step; two slots alternate so that the
    // next step's loads are in flight during this step's MFMAs (XPW is even,
    // so the slot of a position is the same in every chunk)
    uint4 ua[2][TF][2], vb[2][KF][2];
    // per-lane byte offsets (the same for every position and chunk); the
    // position / chunk part of each address is uniform across the wave
    int uoff[TF][2], voff[KF];
#pragma unroll
    for (int a = 0; a < TF; ++a) {
        uoff[a][0] = (tb * TB + a * 32 + lrow) * 64 + ps0 * 16;
        uoff[a][1] = (tb * TB + a * 32 + lrow) * 64 + ps1 * 16;
    }
#pragma unroll
    for (int b = 0; b < KF; ++b) voff[b] = b * 2048 + lrow * 32 + h * 16;
    auto load = [&](int slot, int chunk, int x) {
        const int xi = wave * XPW + x;
        const uint8_t* ub = U + (static_cast<long long>(xi) * nchunks + chunk) * Tpad * 64;
        const uint8_t* vbase = V + ((static_cast<long long>(xi) * ntk + kt) * nchunks + chunk) * KF * 2048;
#pragma unroll
        for (int a = 0; a < TF; ++a) {
            ua[slot][a][0] = *reinterpret_cast<const uint4*>(ub + uoff[a][0]);
            ua[slot][a][1] = *reinterpret_cast<const uint4*>(ub + uoff[a][1]);
        }
#pragma unroll
        for (int b = 0; b < KF; ++b) {
            vb[slot][b][0] = *reinterpret_cast<const uint4*>(vbase + voff[b]);
            vb[slot][b][1] = *reinterpret_cast<const uint4*>(vbase + voff[b] + 1024);
        }
    };
    static_assert(XPW % 2 == 0, "positions per wave must be even");
    load(0, 0, 0);
    for (int chunk = 0; chunk < nchunks; ++chunk) {
#pragma unroll
        for (int x = 0; x < XPW; ++x) {
            const int cur = x & 1;
            if (x + 1 < XPW)
                load(cur ^ 1, chunk, x + 1);
            else
                load(cur ^ 1, min(chunk + 1, nchunks - 1), 0);
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int a = 0; a < TF; ++a)
#pragma unroll
                    for (int b = 0; b < KF; ++b) WMma<T>::piece(acc[x][a][b], ua[cur][a][i], vb[cur][b][i]);
        }
    }

    // Output transform, one slice of KS output channels at a time:
    // M[xi][tile][KS] (fp32) in LDS, then Y = A^T M A per (tile, channel).
    constexpr int KS = (M == 6) ? 8 : 16;
    float* Ms = reinterpret_cast<float*>(lds);
#pragma unroll 1
    for (int ks = 0; ks < KB; ks += KS) {
        // fragment D[row = tile][col = channel]: lane holds column lrow (+32*b),
        // accumulator v is row 8*(v/4) + 4*h + v%4 (+32*a)
#pragma unroll
        for (int b = 0; b < KF; ++b) {
            const int col = b * 32 + lrow;
            if (col >= ks && col < ks + KS) {
#pragma unroll
                for (int x = 0; x < XPW; ++x)
#pragma unroll
                    for (int a = 0; a < TF; ++a)
#pragma unroll
                        for (int v = 0; v < 16; ++v) {
                            const int row = a * 32 + 8 * (v / 4) + 4 * h + (v % 4);
                            Ms[((wave * XPW + x) * TB + row) * KS + (col - ks)] = acc[x][a][b][v];
                        }
            }
        }
        __syncthreads();
        for (int pr = tid; pr < TB * KS; pr += NTHR) {
            const int row = pr % TB, kl = pr / TB;  // tile fastest across lanes
            const int tile = tb * TB + row;
            const int k = kt * KB + ks + kl;
            if (tile < T_ && k < K) {
                // t = A^T M, one column of M at a time (keeps registers low)
                float t[M][A];
#pragma unroll
                for (int j = 0; j < A; ++j) {
                    float col[A];
#pragma unroll
                    for (int q = 0; q < A; ++q) col[q] = Ms[((q * A + j) * TB + row) * KS + kl];
#pragma unroll
                    for (int i = 0; i < M; ++i) {
                        float s = 0.0f;
#pragma unroll
                        for (int q = 0; q < A; ++q) {
                            const float c = static_cast<float>(mt.at[i][q]);
                            if (c != 0.0f) s = fmaf(c, col[q], s);
                        }
                        t[i][j] = s;
                    }
                }
                const int tx = tile % tw;
                const int t2 = tile / tw;
                const int ty = t2 % th;
                const int n = t2 / th;
#pragma unroll
                for (int i = 0; i < M; ++i) {
                    const int oh = ty * M + i;
                    if (oh >= OH) continue;
#pragma unroll
                    for (int j = 0; j < M; ++j) {
                        const int ow = tx * M + j;
                        if (ow >= OW) continue;
                        float s = 0.0f;
#pragma unroll
                        for (int q = 0; q < A; ++q) {
                            const float c = static_cast<float>(mt.at[j][q]);
                            if (c != 0.0f) s = fmaf(t[i][q], c, s);
                        }
                        const long long o = n * y_img + act_off<XB>(k, oh, ow, OH, OW);
                        T* dst = y + o;
                        if constexpr (std::is_same_v<T, int8_t>) {
                            // the exact result is an integer: round the float
                            // one to it, then requantise as the integer paths do
                            const int acc = __float2int_rn(s);
                            const uint32_t q = EPI ? requant_i8_epi_bits(acc, scale[k], ep, k, o)
                                                   : requant_i8_bits(acc, scale[k]);
                            *dst = static_cast<int8_t>(q & 0xffu);
                        } else {
                            s = wg_denorm(s, osx, osw);  // bf16: undo the operand scales
                            if constexpr (EPI) s = epi_float<T>(s, ep, k, o);  // fused epilogue
                            if constexpr (sizeof(T) == 4)
                                *dst = s;
                            else
                                dst->bits = float_to_bf16(s);
                        }
                    }
                }
            }
        }
        __syncthreads();
    }
}

template <typename T, int XB, int M>
cfwd_status launch_t(const Prob& p, const Geo& g, const void* x, const void* vprep, void* ubuf, void* y, const Epi& e,
                     const float* scale, hipStream_t st) {
    // bf16: the operands' maxima sit after the transformed input (this
    // call's) and after the prepared filter (written by the prepare step)
    unsigned* xmax = g.hdr ? reinterpret_cast<unsigned*>(static_cast<uint8_t*>(ubuf) + g.u_bytes) : nullptr;
    const unsigned* wmax = g.hdr ? reinterpret_cast<const unsigned*>(static_cast<const uint8_t*>(vprep) + g.v_bytes)
                                 : nullptr;
    {
        using O = typename OpT<T>::type;
        constexpr int TXB = InGeo<M, 64 / static_cast<int>(sizeof(O))>::TXB;
        const int tblocks_w = (g.tw + TXB - 1) / TXB;
        const dim3 grid(static_cast<unsigned>(static_cast<long long>(p.n) * g.th * tblocks_w),
                        static_cast<unsigned>(g.nchunks));
        if (xmax) {
            cfwd_status s = bf16_absmax(x, static_cast<long long>(p.n) * p.x_img, xmax, st);
            if (s != CFWD_OK) return s;
        }
        input_kernel<T, XB, M><<<grid, 256, 0, st>>>(static_cast<const T*>(x), static_cast<uint8_t*>(ubuf), p.n, p.c,
                                                     p.h, p.w, p.ph, p.pw, p.x_img, g.th, g.tw, g.T, g.Tpad,
                                                     g.nchunks, tblocks_w, xmax);
        cfwd_status s = check_hip(hipGetLastError(), "winograd input transform launch");
        if (s != CFWD_OK) return s;
        if (g.Tpad > g.T) {
            const long long n16 = static_cast<long long>(g.xi) * g.nchunks * (g.Tpad - g.T) * 4;
            const unsigned zb = static_cast<unsigned>(std::min<long long>((n16 + 255) / 256, 4096));
            zero_pad_tiles<<<zb, 256, 0, st>>>(static_cast<uint8_t*>(ubuf), g.xi * g.nchunks, g.T, g.Tpad);
            s = check_hip(hipGetLastError(), "winograd pad-tile clear launch");
            if (s != CFWD_OK) return s;
        }
    }
    constexpr int A = M + 2;
    constexpr int TB = (M == 6) ? 32 : 64;
    constexpr int KS = (M == 6) ? 8 : 16;
    const size_t lds = static_cast<size_t>(A * A) * TB * KS * 4;
    const bool epi = e.bias || e.res || e.relu;
    auto kern = epi ? gemm_kernel<T, XB, M, true> : gemm_kernel<T, XB, M, false>;
    static bool attr[2] = {false, false};
    if (lds > 65536 && !attr[epi]) {
        hipError_t he = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                            hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
        if (he != hipSuccess) return check_hip(he, "hipFuncSetAttribute(winograd gemm)");
        attr[epi] = true;
    }
    const unsigned blocks = static_cast<unsigned>(g.ntb * g.ntk);
    kern<<<blocks, GemmGeo<M>::NTHR, lds, st>>>(static_cast<const uint8_t*>(ubuf), static_cast<const uint8_t*>(vprep),
                                   static_cast<T*>(y), p.k, p.oh, p.ow, p.y_img, g.th, g.tw, g.T, g.Tpad, g.nchunks,
                                   g.ntk, e, xmax, wmax, scale);
    return check_hip(hipGetLastError(), "winograd gemm launch");
}

template <typename T, int M>
cfwd_status launch_m(const Prob& p, const Geo& g, const void* x, const void* vprep, void* ubuf, void* y, const Epi& e,
                     hipStream_t st, const float* scale = nullptr) {
    switch (p.xb) {
        case 1: return launch_t<T, 1, M>(p, g, x, vprep, ubuf, y, e, scale, st);
        case 4: return launch_t<T, 4, M>(p, g, x, vprep, ubuf, y, e, scale, st);
        case 8: return launch_t<T, 8, M>(p, g, x, vprep, ubuf, y, e, scale, st);
        default: return set_error(CFWD_ERR_UNSUPPORTED, "winograd: bad channel block");
    }
}

}  // namespace wg

cfwd_status bf16_absmax(const void* x, long long n, unsigned* out, hipStream_t st) {
    unsigned* slots = out + 64;  // words 64 .. 64 + kAbsmaxBlocks of the 8 KiB area
    wg::bf16_absmax_partial<<<wg::kAbsmaxBlocks, 256, 0, st>>>(static_cast<const uint16_t*>(x), n, slots);
    cfwd_status s = check_hip(hipGetLastError(), "bf16_absmax_partial launch");
    if (s != CFWD_OK) return s;
    wg::absmax_final<<<1, 256, 0, st>>>(slots, out);
    return check_hip(hipGetLastError(), "absmax_final launch");
}

// F(2x2): config 0 = the three-launch form above (any float dtype and
// layout), configs 1 and 2 = the fused single-launch kernels (bf16 NCHW).
// F(6x6): config 0 = the three-launch form, config 1 = the fused kernel
// (bf16 or fp32 NCHW).
int winograd_num_configs(int m) { return m == 2 ? 3 : 2; }

bool winograd_supported(const Prob& p, int m, int cfg, std::string* why) {
    if (m == 2 && (cfg == 1 || cfg == 2)) return winograd_fused_supported(p, cfg, why);
    if (m == 6 && cfg == 1) return winograd_f6_fused_supported(p, why);
    if (cfg != 0 || (m != 2 && m != 6)) {
        if (why) *why = "winograd: no such config";
        return false;
    }
    // F(6x6) rounds its transformed operands to fp16 for bf16 inputs; the
    // error that adds, relative to the sum of |x*w| an output is normalised
    // by, falls off like one over the square root of the channel count (about
    // 0.02 at 4 channels, 0.01 at 16, 0.005 at 32 for unit-scale data), so
    // below 32 channels per group it would not stay within the bf16 bound
    if (m == 6 && p.dtype == CFWD_BF16 && p.cg < 32) {
        if (why) *why = "winograd F(6x6): bf16 needs at least 32 input channels per group to meet its error bound";
        return false;
    }
    // with padding 2 a corner output sees a single input pixel per channel,
    // so the sum of |x*w| it is normalised by is small, while the rounding of
    // the tile's 64 transformed values reaches it in full
    if (m == 6 && p.dtype == CFWD_BF16 && (p.ph > 1 || p.pw > 1)) {
        if (why) *why = "winograd F(6x6): bf16 needs padding 0 or 1 to meet its error bound";
        return false;
    }
    wg::Geo g;
    return wg::geometry(p, m, &g, why);
}

size_t winograd_filter_bytes(const Prob& p, int m, int cfg) {
    if (m == 2 && (cfg == 1 || cfg == 2)) return winograd_fused_filter_bytes(p, cfg);
    if (m == 6 && cfg == 1) return winograd_f6_fused_filter_bytes(p);
    wg::Geo g;
    if (!wg::geometry(p, m, &g, nullptr)) return 0;
    return g.v_bytes + g.hdr;
}

size_t winograd_scratch_bytes(const Prob& p, int m, int cfg) {
    if (m == 2 && (cfg == 1 || cfg == 2))  // the fused form: only the input's largest magnitude
        return winograd_fused_supported(p, cfg, nullptr) ? 8192 : 0;
    if (m == 6 && cfg == 1) return winograd_f6_fused_scratch_bytes(p);
    wg::Geo g;
    if (!wg::geometry(p, m, &g, nullptr)) return 0;
    return g.u_bytes + g.hdr;
}

cfwd_status winograd_prepare(const Prob& p, int m, int cfg, const void* w, void* wp, hipStream_t st) {
    if (m == 2 && (cfg == 1 || cfg == 2)) return winograd_fused_prepare(p, cfg, w, wp, st);
    if (m == 6 && cfg == 1) return winograd_f6_fused_prepare(p, w, wp, st);
    wg::Geo g;
    std::string why;
    if (!wg::geometry(p, m, &g, &why)) return set_error(CFWD_ERR_UNSUPPORTED, why);
    const long long total = static_cast<long long>(g.ntk) * g.KB * g.nchunks * g.CK;
    long long blocks = (total + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    const unsigned nb = static_cast<unsigned>(blocks);
    uint8_t* out = static_cast<uint8_t*>(wp);
    if (p.dtype == CFWD_I8) {  // F(2x2) only (geometry): integer G, no scaling
        wg::prepare_kernel<int8_t, 2><<<nb, 256, 0, st>>>(static_cast<const int8_t*>(w), out, p.k, p.c, g.KB, g.ntk,
                                                          g.nchunks, nullptr);
    } else if (p.dtype == CFWD_F32) {
        if (m == 2)
            wg::prepare_kernel<float, 2><<<nb, 256, 0, st>>>(static_cast<const float*>(w), out, p.k, p.c, g.KB, g.ntk,
                                                             g.nchunks, nullptr);
        else
            wg::prepare_kernel<float, 6><<<nb, 256, 0, st>>>(static_cast<const float*>(w), out, p.k, p.c, g.KB, g.ntk,
                                                             g.nchunks, nullptr);
    } else {
        // the filter's largest magnitude goes after the transformed filter
        unsigned* wmax = reinterpret_cast<unsigned*>(out + g.v_bytes);
        cfwd_status s = bf16_absmax(w, static_cast<long long>(p.k) * p.cg * 9, wmax, st);
        if (s != CFWD_OK) return s;
        if (m == 2)
            wg::prepare_kernel<bf16_t, 2><<<nb, 256, 0, st>>>(static_cast<const bf16_t*>(w), out, p.k, p.c, g.KB,
                                                              g.ntk, g.nchunks, wmax);
        else
            wg::prepare_kernel<bf16_t, 6><<<nb, 256, 0, st>>>(static_cast<const bf16_t*>(w), out, p.k, p.c, g.KB,
                                                              g.ntk, g.nchunks, wmax);
    }
    return check_hip(hipGetLastError(), "winograd filter transform launch");
}

cfwd_status winograd_launch(const Prob& p, int m, int cfg, const void* x, const void* wp, void* scratch, void* y,
                            const Epi& e, hipStream_t st) {
    if (m == 2 && (cfg == 1 || cfg == 2)) return winograd_fused_launch(p, cfg, x, wp, scratch, y, e, st);
    if (m == 6 && cfg == 1) return winograd_f6_fused_launch(p, x, wp, scratch, y, e, st);
    wg::Geo g;
    std::string why;
    if (!wg::geometry(p, m, &g, &why)) return set_error(CFWD_ERR_UNSUPPORTED, why);
    if (scratch == nullptr || wp == nullptr)
        return set_error(CFWD_ERR_WORKSPACE, "winograd: prepared filter and scratch are required");
    if (p.dtype == CFWD_I8) return set_error(CFWD_ERR_INVALID_ARG, "winograd: int8 goes through winograd_i8_launch");
    if (p.dtype == CFWD_F32)
        return (m == 2) ? wg::launch_m<float, 2>(p, g, x, wp, scratch, y, e, st)
                        : wg::launch_m<float, 6>(p, g, x, wp, scratch, y, e, st);
    return (m == 2) ? wg::launch_m<bf16_t, 2>(p, g, x, wp, scratch, y, e, st)
                    : wg::launch_m<bf16_t, 6>(p, g, x, wp, scratch, y, e, st);
}

cfwd_status winograd_i8_launch(const Prob& p, const void* x, const void* wp, const float* scale, void* scratch,
                               void* y, const Epi& e, hipStream_t st) {
    wg::Geo g;
    std::string why;
    if (p.dtype != CFWD_I8) return set_error(CFWD_ERR_INVALID_ARG, "winograd_i8_launch: int8 problems only");
    if (!wg::geometry(p, 2, &g, &why)) return set_error(CFWD_ERR_UNSUPPORTED, why);
    if (scratch == nullptr || wp == nullptr)
        return set_error(CFWD_ERR_WORKSPACE, "winograd: prepared filter and scratch are required");
    if (scale == nullptr) return set_error(CFWD_ERR_INVALID_ARG, "winograd int8: requant scales are required");
    return wg::launch_m<int8_t, 2>(p, g, x, wp, scratch, y, e, st, scale);
}

}  // namespace cfwd
