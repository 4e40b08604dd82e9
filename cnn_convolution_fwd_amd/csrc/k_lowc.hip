// Implicit GEMM for layers with few input channels (the stem of a CNN: 3
// image channels, 3x3 or 7x7 filters, stride 2), gfx950.
//
// MegEngine inference article, section "Im2col+MatMul": the convolution is a
// matrix product of the weights with the im2col matrix.  When C*R*S is small
// the tiled implicit GEMM of igemm_impl.h wastes most of each 64-byte channel
// chunk (3 real channels of 32 or 64), so this variant gathers the reduction
// dimension directly instead of staging channel chunks:
//   * MFMA rows = output channels (A = prepared weights, 16 bytes per lane
//     per step, from L1/L2), MFMA columns = output pixels (B = gathered
//     input, one column per lane);
//   * the reduction index u runs over (c, r, s) for fp32/bf16 (one element
//     per unit), or over taps (r, s) for int8 NCHW4 with C <= 4, where one
//     unit is the aligned dword holding a pixel's four channels;
//   * a per-workgroup LDS table maps u to (row delta, column delta, channel
//     offset); each lane adds its own pixel's origin, tests the bounds (zero
//     padding) and loads with a clamped, always-valid address -- no branches;
//   * staged variants first copy the input rows their pixels read into LDS,
//     zero-padded around the image, and keep only each unit's byte offset
//     from a pixel's base there: every gather is then one unconditional LDS
//     load;
//   * gathers of the next step are in flight while the current one is on the
//     matrix cores (two-deep pipeline, last pair peeled);
//   * the epilogue writes D[k][pixel] in the caller's layout; for int8 NCHW4
//     a lane's four consecutive channels of one pixel leave as one dword.
//     For fp32/bf16 NCHW, where a workgroup's output is a run of consecutive
//     pixels of each of its channels, the tile is first transposed through
//     LDS ([channel][pixel]) and leaves as 16-byte streaming stores, each
//     channel's run written by consecutive lanes.
// Step (units per MFMA step): fp32 8 (four v_mfma_f32_32x32x2f32), bf16 16
// (one v_mfma_f32_32x32x16_bf16), int8 8 dwords = 32 bytes (one
// v_mfma_i32_32x32x32_i8).
#include "internal.h"

namespace cfwd {

namespace {

using f32x16_t = float __attribute__((ext_vector_type(16)));
using i32x16_t = int __attribute__((ext_vector_type(16)));
typedef int i32x4_t __attribute__((ext_vector_type(4)));

constexpr int kMaxUnits = 1024;  // unit table entries at most (12 KB of LDS)

struct LcArgs {
    int N, C, H, W, K, OH, OW, R, S, sh, sw, ph, pw, dh, dw;
    long long x_img, y_img;  // elements (bytes for int8)
    int units, nss, nkb, KW, ngk;
    long long npix;
    int vec_ok;  // output pieces of 16 bytes are aligned (checked on the host)
    // staged variants: each workgroup copies the input rows its pixels read
    // into LDS, [channel][ROWS][RW] gather elements, the image columns at
    // padL .. padL + W - 1 and zeros around them
    int ROWS, RW, padL, st_bytes;
    // staged fp32/bf16: element offset of a zero-filled region of ROWS * RW
    // elements after the staged rows, read by the reduction's padding units
    int zoff;
    Epi e;  // fused epilogue
};

struct Tap {
    int dr, ds, off;
};

template <typename T> struct Lc;
template <> struct Lc<float> {
    static constexpr int SSU = 8;   // units per step
    static constexpr int NG = 4;    // gathers per lane per step
    using G = float;
    using Acc = f32x16_t;
    static __device__ __forceinline__ int unit(int g, int h) { return 2 * g + h; }
    static __device__ __forceinline__ void mma(Acc& acc, const uint4& a, const G* v, int i) {
        const uint32_t av[4] = {a.x, a.y, a.z, a.w};
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(av[i]), v[i], acc, 0, 0, 0);
    }
    static constexpr int SUB = 4;  // MFMAs per step
};
template <> struct Lc<bf16_t> {
    static constexpr int SSU = 16;
    static constexpr int NG = 8;
    using G = uint16_t;
    using Acc = f32x16_t;
    static __device__ __forceinline__ int unit(int g, int h) { return 8 * h + g; }
    static __device__ __forceinline__ void mma(Acc& acc, const uint4& a, const G* v, int) {
        const uint4 b = make_uint4(v[0] | (static_cast<uint32_t>(v[1]) << 16), v[2] | (static_cast<uint32_t>(v[3]) << 16),
                                   v[4] | (static_cast<uint32_t>(v[5]) << 16), v[6] | (static_cast<uint32_t>(v[7]) << 16));
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), acc,
                                                      0, 0, 0);
    }
    static constexpr int SUB = 1;
};
template <> struct Lc<int8_t> {
    static constexpr int SSU = 8;  // dwords (32 bytes)
    static constexpr int NG = 4;
    using G = uint32_t;
    using Acc = i32x16_t;
    static __device__ __forceinline__ int unit(int g, int h) { return 4 * h + g; }
    static __device__ __forceinline__ void mma(Acc& acc, const uint4& a, const G* v, int) {
        const i32x4_t av = {static_cast<int>(a.x), static_cast<int>(a.y), static_cast<int>(a.z), static_cast<int>(a.w)};
        const i32x4_t bv = {static_cast<int>(v[0]), static_cast<int>(v[1]), static_cast<int>(v[2]), static_cast<int>(v[3])};
        acc = __builtin_amdgcn_mfma_i32_32x32x32_i8(av, bv, acc, 0, 0, 0);
    }
    static constexpr int SUB = 1;
};

// Prepared weights: [k block of 32][step][lane 64][16 bytes].
template <typename T>
__global__ __launch_bounds__(256) void lc_prepare_kernel(const T* __restrict__ w, uint8_t* __restrict__ out, int K,
                                                         int C, int RS, int units, int nkb, int nss) {
    const long long total = static_cast<long long>(nkb) * nss * 64 * 16;  // bytes
    for (long long i = blockIdx.x * 256LL + threadIdx.x; i < total; i += static_cast<long long>(gridDim.x) * 256) {
        const int byte = static_cast<int>(i % 16);
        long long t = i / 16;
        const int lane = static_cast<int>(t % 64);
        t /= 64;
        const int ss = static_cast<int>(t % nss);
        const int kb = static_cast<int>(t / nss);
        const int k = kb * 32 + (lane & 31), h = lane >> 5;
        if constexpr (sizeof(T) == 1) {
            const int u = ss * Lc<int8_t>::SSU + Lc<int8_t>::unit(byte / 4, h);  // tap
            const int c = byte % 4;
            int8_t v = 0;
            if (k < K && u < RS && c < C) v = w[(static_cast<long long>(k) * C + c) * RS + u];
            out[i] = static_cast<uint8_t>(v);
        } else {
            constexpr int E = 16 / static_cast<int>(sizeof(T));
            if (byte % sizeof(T) != 0) continue;
            const int e = byte / static_cast<int>(sizeof(T));
            // fp32: element e of the 16 bytes feeds sub-step e; bf16: element e
            const int u = ss * Lc<T>::SSU + Lc<T>::unit(e, h);
            T v{};
            if (k < K && u < units) v = w[static_cast<long long>(k) * units + u];
            *reinterpret_cast<T*>(out + i) = v;
            (void)E;
        }
    }
}

// Bytes of the LDS-transposed output tile of one workgroup (0: not used):
// (4 / KW) * NCB * 32 pixels x KW * KBW * 32 channels, whatever KW is.
template <typename T, int XB, int NCB, int KBW>
constexpr int lc_tile_bytes() {
    constexpr int b = 4 * NCB * KBW * 32 * 32 * static_cast<int>(sizeof(T));
    return (sizeof(T) != 1 && XB == 1 && b <= 32768) ? b : 0;
}

// Workgroup: 4 waves = (4 / KW) pixel groups x KW k groups; a wave owns NCB
// columns blocks of 32 pixels x KBW blocks of 32 output channels.
// EPI: the fused epilogue compiled in (a separate instantiation, so the
// plain kernels carry none of its registers).
template <typename T, int XB, int NCB, int KBW, bool STG, bool EPI>
__global__ __launch_bounds__(256) void lc_kernel(const T* __restrict__ x, const uint8_t* __restrict__ wp,
                                                 const float* __restrict__ scale, T* __restrict__ y, LcArgs a) {
    using L = Lc<T>;
    using G = typename L::G;
    constexpr int TILE = lc_tile_bytes<T, XB, NCB, KBW>();
    // dynamic LDS (sized by lc_lds_bytes): [staged input rows and zero
    // region (STG)][unit table] while gathering, then, after a barrier, the
    // transposed output tile in the same bytes
    extern __shared__ __attribute__((aligned(16))) uint8_t lds_dyn[];
    Tap* tab = reinterpret_cast<Tap*>(lds_dyn + (STG ? a.st_bytes : 0));
    int* toff = reinterpret_cast<int*>(lds_dyn + a.st_bytes);  // STG's table
    uint8_t* otile = lds_dyn;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int j = lane & 31, h = lane >> 5;
    const int ohw = a.OH * a.OW;
    const int wk = wave % a.KW, wpx = wave / a.KW;
    const int kg = static_cast<int>(blockIdx.x) % a.ngk;
    const long long pg = static_cast<long long>(blockIdx.x) / a.ngk;
    const int wpix = (4 / a.KW) * NCB * 32;  // pixels of this workgroup (all in one image when STG)

    const int RS = a.R * a.S;
    const int ntab = a.nss * L::SSU;
    if constexpr (STG) {
        // staged: byte offset of each unit's element from a pixel's base in
        // LDS, ordered [step][lane half][gather] so that a lane reads a
        // step's offsets with 16-byte loads.  Padding units read zeros from
        // the zero region (fp32/bf16: an Inf times a zero weight would be
        // NaN), or, for int8, the pixel's own first tap: their weights are
        // zero and int8 products are finite.
        for (int i = tid; i < ntab; i += 256) {
            const int ss = i / L::SSU, rem = i % L::SSU;
            const int u = ss * L::SSU + L::unit(rem % L::NG, rem / L::NG);
            int off = (sizeof(T) == 1) ? 0 : a.zoff;
            const int nu = (sizeof(T) == 1) ? RS : a.units;
            if (u < nu) {
                const int c = (sizeof(T) == 1) ? 0 : u / RS;
                const int tap = (sizeof(T) == 1) ? u : u % RS;
                const int r = tap / a.S, s = tap % a.S;
                off = (c * a.ROWS + r * a.dh) * a.RW + s * a.dw;
            }
            toff[i] = off * static_cast<int>(sizeof(G));
        }
    }
    // gathers from global memory: reduction unit -> (row delta, column
    // delta, channel offset)
    for (int u = tid; u < (STG ? 0 : ntab); u += 256) {
        Tap t;
        t.dr = -(1 << 28);  // padding unit: always out of range -> 0
        t.ds = 0;
        t.off = 0;
        const int nu = (sizeof(T) == 1) ? RS : a.units;
        if (u < nu) {
            const int c = (sizeof(T) == 1) ? 0 : u / RS;
            const int tap = (sizeof(T) == 1) ? u : u % RS;
            const int r = tap / a.S, s = tap % a.S;
            t.dr = r * a.dh;
            t.ds = s * a.dw;
            if (sizeof(T) != 1) t.off = (XB == 1) ? c * a.H * a.W : (c / XB) * a.H * a.W * XB + c % XB;
        }
        tab[u] = t;
    }
    // staged: first input row of this workgroup and its image
    int st_n = 0, st_row0 = 0, st_pix0 = 0;
    if constexpr (STG) {
        const long long W0 = pg * wpix;
        st_n = static_cast<int>(static_cast<unsigned>(W0) / static_cast<unsigned>(ohw));
        st_pix0 = static_cast<int>(static_cast<unsigned>(W0) - static_cast<unsigned>(st_n) * ohw);
        st_row0 = st_pix0 / a.OW * a.sh - a.ph;
        // 16-byte chunks of every staged row; chunks are wholly inside or
        // wholly outside the image (W and padL are multiples of a chunk)
        constexpr int CE = 16 / static_cast<int>(sizeof(G));  // gather elements per chunk
        const int cpr = a.RW / CE;
        const int nch = (sizeof(T) == 1) ? 1 : a.C;
        const G* xg = reinterpret_cast<const G*>(x) + static_cast<long long>(st_n) * (sizeof(T) == 1 ? a.x_img / 4 : a.x_img);
        // chunk q = (c * ROWS + rr) * cpr + col, stepped by 256 without
        // divisions inside the loop, four chunks per thread at a time: the
        // four loads (from a clamped, always valid address; zeros outside the
        // image) are all in flight before the first LDS write
        int col = tid % cpr, rr = tid / cpr, c = 0;
        while (rr >= a.ROWS) rr -= a.ROWS, ++c;
        const int dcol = 256 % cpr, drow = 256 / cpr;
        constexpr int NB = 4;
        while (c < nch) {
            uint4 v[NB];
            int dst[NB];
#pragma unroll
            for (int i = 0; i < NB; ++i) {
                const bool live = c < nch;
                const int ih = st_row0 + rr, iw = col * CE - a.padL;
                const bool in = live && static_cast<unsigned>(ih) < static_cast<unsigned>(a.H) && iw >= 0 && iw < a.W;
                const uint4 t = *reinterpret_cast<const uint4*>(xg + (in ? (static_cast<long long>(c) * a.H + ih) * a.W + iw : 0));
                v[i] = in ? t : make_uint4(0, 0, 0, 0);
                dst[i] = live ? ((c * a.ROWS + rr) * a.RW + col * CE) * static_cast<int>(sizeof(G)) : -1;
                col += dcol;
                rr += drow;
                if (col >= cpr) col -= cpr, ++rr;
                while (rr >= a.ROWS) rr -= a.ROWS, ++c;
            }
#pragma unroll
            for (int i = 0; i < NB; ++i)
                if (dst[i] >= 0) *reinterpret_cast<uint4*>(lds_dyn + dst[i]) = v[i];
        }
        if constexpr (sizeof(T) != 1)
            for (int q = tid; q < a.ROWS * cpr; q += 256)
                *reinterpret_cast<uint4*>(lds_dyn + (a.zoff + q * CE) * sizeof(G)) = make_uint4(0, 0, 0, 0);
    }
    __syncthreads();

    const int kb0 = (kg * a.KW + wk) * KBW;
    // a wave past the last k block has no work; with the transposed epilogue
    // it still takes part in the workgroup's barrier
    const bool active = kb0 < a.nkb;
    if (TILE == 0 && !active) return;  // after the only barrier
    const long long P0 = (pg * (4 / a.KW) + wpx) * (NCB * 32);

    // this lane's pixel in each column block
    long long xbase[NCB];
    int ih0[NCB], iw0[NCB], lbase[NCB], pn[NCB], ppix[NCB];
    bool pok[NCB];
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
        // pixel indices fit in 31 bits (checked on the host): 32-bit
        // divisions, which are several times cheaper than 64-bit ones
        const unsigned G0 = static_cast<unsigned>(P0) + cb * 32 + j;
        pok[cb] = G0 < static_cast<unsigned>(a.npix);
        const unsigned Gc = pok[cb] ? G0 : 0u;
        const int n = static_cast<int>(Gc / static_cast<unsigned>(ohw));
        const int pix = static_cast<int>(Gc - static_cast<unsigned>(n) * ohw);
        pn[cb] = n;
        ppix[cb] = pix;
        const int oh = pix / a.OW, ow = pix - (pix / a.OW) * a.OW;
        ih0[cb] = oh * a.sh - a.ph;
        iw0[cb] = ow * a.sw - a.pw;
        xbase[cb] = (sizeof(T) == 1) ? n * (a.x_img / 4) : n * a.x_img;
        // staged: byte offset of tap (0, 0), channel 0 of this pixel in LDS
        lbase[cb] = pok[cb] ? ((ih0[cb] - st_row0) * a.RW + iw0[cb] + a.padL) * static_cast<int>(sizeof(G)) : 0;
    }

    // staged: this lane's pixel in LDS, one address per column block
    const uint8_t* lpix[NCB];
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) lpix[cb] = lds_dyn + lbase[cb];

    typename L::Acc acc[KBW][NCB];
#pragma unroll
    for (int b = 0; b < KBW; ++b)
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) acc[b][cb] = typename L::Acc{};

    const G* xg = reinterpret_cast<const G*>(x);
    auto gather = [&](int ss, G (*v)[L::NG], uint4* wv) {
        if constexpr (STG) {
            int4 o[L::NG / 4];
#pragma unroll
            for (int i = 0; i < L::NG / 4; ++i)
                o[i] = *reinterpret_cast<const int4*>(toff + (ss * 2 + h) * L::NG + 4 * i);
#pragma unroll
            for (int g = 0; g < L::NG; ++g) {
                const int og = (g % 4 == 0) ? o[g / 4].x : (g % 4 == 1) ? o[g / 4].y : (g % 4 == 2) ? o[g / 4].z : o[g / 4].w;
#pragma unroll
                for (int cb = 0; cb < NCB; ++cb) v[cb][g] = *reinterpret_cast<const G*>(lpix[cb] + og);
            }
        }
#pragma unroll
        for (int g = 0; g < (STG ? 0 : L::NG); ++g) {
            const Tap t = tab[ss * L::SSU + L::unit(g, h)];
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb) {
                const int ih = ih0[cb] + t.dr, iw = iw0[cb] + t.ds;
                const bool ok = static_cast<unsigned>(ih) < static_cast<unsigned>(a.H) &&
                                static_cast<unsigned>(iw) < static_cast<unsigned>(a.W);
                const long long pix = static_cast<long long>(ih) * a.W + iw;
                const long long o = xbase[cb] + t.off + ((sizeof(T) == 1) ? pix : pix * XB);
                const G val = xg[ok ? o : 0];
                v[cb][g] = ok ? val : G{};
            }
        }
#pragma unroll
        for (int b = 0; b < KBW; ++b)
            wv[b] = *reinterpret_cast<const uint4*>(wp + ((static_cast<long long>(kb0 + b) * a.nss + ss) * 64 + lane) * 16);
    };
    auto compute = [&](G (*v)[L::NG], const uint4* wv) {
#pragma unroll
        for (int i = 0; i < L::SUB; ++i)
#pragma unroll
            for (int b = 0; b < KBW; ++b)
#pragma unroll
                for (int cb = 0; cb < NCB; ++cb) L::mma(acc[b][cb], wv[b], v[cb], i);
    };

    if (active) {
        G va[NCB][L::NG], vb[NCB][L::NG];
        uint4 wa[KBW], wb[KBW];
        gather(0, va, wa);
        int ss = 0;
        for (; ss + 2 < a.nss; ss += 2) {
            gather(ss + 1, vb, wb);
            compute(va, wa);
            gather(ss + 2, va, wa);
            compute(vb, wb);
        }
        gather(ss + 1, vb, wb);
        compute(va, wa);
        compute(vb, wb);
    }

    if constexpr (TILE > 0) {
        // [channel of the workgroup][pixel of the workgroup], row pitch padded
        // by 16 bytes; then each thread stores 16-byte pieces of channel rows
        constexpr int E = static_cast<int>(sizeof(T));
        const int wch = a.KW * KBW * 32;         // channels of this workgroup
        const int pitch = wpix * E + 16;
        __syncthreads();  // every wave is done with the unit table
        if (active) {
#pragma unroll
            for (int b = 0; b < KBW; ++b)
#pragma unroll
                for (int cb = 0; cb < NCB; ++cb) {
                    const int pl = (wpx * NCB + cb) * 32 + j;
                    // fused epilogue: the 16 channels' bias and residual values
                    // of this lane's pixel, all requested before any is used
                    float ebias[16], eres[16];
                    if constexpr (EPI) {
#pragma unroll
                        for (int v = 0; v < 16; ++v) {
                            const int k = kg * a.KW * KBW * 32 + (wk * KBW + b) * 32 + 8 * (v / 4) + 4 * h + (v % 4);
                            const bool kin = k < a.K;
                            ebias[v] = (a.e.bias && kin) ? static_cast<const float*>(a.e.bias)[k] : 0.0f;
                            eres[v] = (a.e.res && kin && pok[cb])
                                          ? Elem<T>::to_f(static_cast<const T*>(a.e.res)[pn[cb] * a.y_img +
                                                                                        static_cast<long long>(k) * ohw +
                                                                                        ppix[cb]])
                                          : 0.0f;
                        }
                    }
#pragma unroll
                    for (int v = 0; v < 16; ++v) {
                        const int cl = (wk * KBW + b) * 32 + 8 * (v / 4) + 4 * h + (v % 4);
                        uint8_t* d = otile + cl * pitch + pl * E;
                        float val = acc[b][cb][v];
                        if constexpr (EPI) {  // fused epilogue, before the conversion
                            const float t = val + ebias[v] + eres[v];
                            val = a.e.relu ? fmaxf(t, 0.0f) : t;
                        }
                        if constexpr (sizeof(T) == 4)
                            *reinterpret_cast<float*>(d) = val;
                        else
                            *reinterpret_cast<uint16_t*>(d) = float_to_bf16(val);
                    }
                }
        }
        __syncthreads();
        constexpr int PE = 16 / E;  // pixels per 16-byte piece
        const int pieces = wpix / PE;
        const long long W0 = pg * wpix;  // first pixel of this workgroup
        const int kbase = kg * a.KW * KBW * 32;
        // piece (cl, pc) = channel row cl, pixels pc * PE ..; stepped by 256
        // pieces without divisions; staged workgroups lie in one image
        int cl = tid / pieces, pc = tid - (tid / pieces) * pieces;
        const int dcl = 256 / pieces, dpc = 256 - (256 / pieces) * pieces;
        for (; cl < wch; pc += dpc, cl += dcl, cl += (pc >= pieces), pc -= (pc >= pieces) ? pieces : 0) {
            const int k = kbase + cl;
            if (k >= a.K) continue;
            const long long G0 = W0 + pc * PE;
            if (G0 >= a.npix) continue;
            int n, pix;
            if constexpr (STG) {
                n = st_n;
                pix = st_pix0 + pc * PE;
            } else {
                n = static_cast<int>(static_cast<unsigned>(G0) / static_cast<unsigned>(ohw));
                pix = static_cast<int>(static_cast<unsigned>(G0) - static_cast<unsigned>(n) * ohw);
            }
            const uint8_t* src = otile + cl * pitch + pc * 16;
            T* dst = y + n * a.y_img + static_cast<long long>(k) * ohw + pix;
            if (a.vec_ok && G0 + PE <= a.npix && pix + PE <= ohw) {
                const uint4 v = *reinterpret_cast<const uint4*>(src);
                typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
                const u32x4_t w = {v.x, v.y, v.z, v.w};
                __builtin_nontemporal_store(w, reinterpret_cast<u32x4_t*>(dst));
            } else {
                // a piece that crosses an image boundary or the end
                for (int e = 0; e < PE; ++e) {
                    long long Ge = G0 + e;
                    if (Ge >= a.npix) break;
                    const int ne = static_cast<int>(static_cast<unsigned>(Ge) / static_cast<unsigned>(ohw));
                    const int pe = static_cast<int>(static_cast<unsigned>(Ge) - static_cast<unsigned>(ne) * ohw);
                    T* de = y + ne * a.y_img + static_cast<long long>(k) * ohw + pe;
                    if constexpr (sizeof(T) == 4)
                        *de = *reinterpret_cast<const float*>(src + e * E);
                    else
                        de->bits = *reinterpret_cast<const uint16_t*>(src + e * E);
                }
            }
        }
        return;
    }

    // D[row = channel][col = pixel]: lane (j, hh), element v -> channel
    // 8 (v / 4) + 4 hh + v % 4 of the block
    // int8: requantisation scales of this lane's 16 channels of each k block
    // (channel 8 (v / 4) + 4 h + v % 4, as the accumulator holds them), all
    // requested at once, at constant offsets from one address where the
    // block lies inside K; channels past K get scale 0, which requantises to
    // the zero bytes that NCHW4 keeps in its padding channels
    float sc[KBW][16];
    if constexpr (sizeof(T) == 1) {
#pragma unroll
        for (int b = 0; b < KBW; ++b) {
            const int kb = (kb0 + b) * 32 + 4 * h;
            if ((kb0 + b) * 32 + 32 <= a.K) {
                const float* sp = scale + kb;
#pragma unroll
                for (int v = 0; v < 16; ++v) sc[b][v] = sp[8 * (v / 4) + (v % 4)];
            } else {
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int k = kb + 8 * (v / 4) + (v % 4);
                    const float t = scale[min(k, a.K - 1)];
                    sc[b][v] = k < a.K ? t : 0.0f;
                }
            }
        }
    }
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
        if (!pok[cb]) continue;
        const int n = pn[cb], pix = ppix[cb];
        const int oh = pix / a.OW, ow = pix - (pix / a.OW) * a.OW;
#pragma unroll
        for (int b = 0; b < KBW; ++b) {
            if constexpr (sizeof(T) == 1) {
                // four consecutive channels of one pixel -> one NCHW4 dword, at
                // a wave-uniform offset from this lane's first one
                const long long ohw4 = static_cast<long long>(ohw) * 4;
                uint8_t* yb = reinterpret_cast<uint8_t*>(y) + n * a.y_img + static_cast<long long>(pix) * 4 +
                              static_cast<long long>(kb0 * 8 + h) * ohw4;
                // fused epilogue: the residual dwords (4 channels of this
                // lane's pixel) of the block's four channel groups, requested
                // before any is used; channels past K (scale 0, zeroed
                // afterwards) take the last real channel's bias
                uint32_t eres[4] = {0u, 0u, 0u, 0u};
                if constexpr (EPI) {
                    if (a.e.res) {
#pragma unroll
                        for (int q = 0; q < 4; ++q) {
                            const int k0 = (kb0 + b) * 32 + 8 * q + 4 * h;
                            if (k0 < a.K)
                                eres[q] = *reinterpret_cast<const uint32_t*>(
                                    static_cast<const int8_t*>(a.e.res) + n * a.y_img +
                                    (static_cast<long long>(k0 / 4) * ohw + pix) * 4);
                        }
                    }
                }
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int k0 = (kb0 + b) * 32 + 8 * q + 4 * h;
                    if (k0 >= a.K) continue;
                    const typename L::Acc& ac = acc[b][cb];
                    uint32_t word;
                    if constexpr (EPI) {
                        uint32_t qb[4];
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const int kb = min(k0 + i, a.K - 1);
                            const int bi = a.e.bias ? static_cast<const int32_t*>(a.e.bias)[kb] : 0;
                            const float r = static_cast<float>(static_cast<int8_t>((eres[q] >> (8 * i)) & 0xffu));
                            qb[i] = requant_i8_fused(ac[4 * q + i], bi, sc[b][4 * q + i], r, a.e.relu ? 0.0f : -127.0f);
                        }
                        word = pack_low_bytes(qb[0], qb[1], qb[2], qb[3]);
                    } else {
                        word = pack_low_bytes(
                            requant_i8_bits(ac[4 * q], sc[b][4 * q]), requant_i8_bits(ac[4 * q + 1], sc[b][4 * q + 1]),
                            requant_i8_bits(ac[4 * q + 2], sc[b][4 * q + 2]),
                            requant_i8_bits(ac[4 * q + 3], sc[b][4 * q + 3]));
                    }
                    *reinterpret_cast<uint32_t*>(yb + (b * 8 + 2 * q) * ohw4) = word;
                }
            } else {
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int k = (kb0 + b) * 32 + 8 * (v / 4) + 4 * h + (v % 4);
                    if (k >= a.K) continue;
                    const long long o = n * a.y_img + act_off<XB>(k, oh, ow, a.OH, a.OW);
                    T* dst = y + o;
                    const float val = EPI ? epi_float<T>(acc[b][cb][v], a.e, k, o) : acc[b][cb][v];
                    if constexpr (sizeof(T) == 4)
                        *dst = val;
                    else
                        dst->bits = float_to_bf16(val);
                }
            }
        }
    }
}

struct LcCfg {
    int ncb, kbw;
};
// configs 0-5 gather from global memory; 6-11 are the same tiles gathering
// from input rows staged in LDS
constexpr LcCfg kLc[6] = {{4, 1}, {2, 2}, {4, 2}, {1, 1}, {1, 2}, {2, 1}};
constexpr int kLcBase = 6;
constexpr int kLcN = 2 * kLcBase;
constexpr size_t kLcStageMax = 48 * 1024;  // LDS for staged rows + unit table

bool lc_geometry(const Prob& p, int cfg, LcArgs* a, std::string* why) {
    auto fail = [&](const char* m) {
        if (why) *why = m;
        return false;
    };
    if (cfg < 0 || cfg >= kLcN) return fail("implicit GEMM (gather): no such config");
    const bool staged = cfg >= kLcBase;
    const LcCfg lc = kLc[cfg % kLcBase];
    if (p.g != 1) return fail("implicit GEMM (gather): groups must be 1");
    int units, ssu;
    if (p.dtype == CFWD_I8) {
        if (p.layout != CFWD_LAYOUT_NCHWX || p.xb != 4 || p.c > 4)
            return fail("implicit GEMM (gather): int8 needs NCHW4 with C <= 4");
        units = p.r * p.s;
        ssu = Lc<int8_t>::SSU;
    } else {
        units = p.c * p.r * p.s;
        ssu = (p.dtype == CFWD_F32) ? Lc<float>::SSU : Lc<bf16_t>::SSU;
    }
    int nss = (units + ssu - 1) / ssu;
    nss += nss & 1;
    if (nss * ssu > kMaxUnits) return fail("implicit GEMM (gather): C*R*S too large");
    if (static_cast<long long>(p.h) * p.w * p.c >= (1LL << 31) || static_cast<long long>(p.oh) * p.ow >= (1LL << 31))
        return fail("implicit GEMM (gather): image too large");
    a->N = p.n; a->C = p.c; a->H = p.h; a->W = p.w; a->K = p.k; a->OH = p.oh; a->OW = p.ow;
    a->R = p.r; a->S = p.s; a->sh = p.sh; a->sw = p.sw; a->ph = p.ph; a->pw = p.pw; a->dh = p.dh; a->dw = p.dw;
    a->x_img = p.x_img; a->y_img = p.y_img;
    a->units = units;
    a->nss = nss;
    const int kbw = lc.kbw;
    const int kwaves = ((p.k + 31) / 32 + kbw - 1) / kbw;
    a->nkb = kwaves * kbw;
    a->KW = kwaves >= 4 ? 4 : (kwaves >= 2 ? 2 : 1);
    a->ngk = (kwaves + a->KW - 1) / a->KW;
    a->npix = static_cast<long long>(p.n) * p.oh * p.ow;
    if (a->npix + 1024 >= (1LL << 31)) return fail("implicit GEMM (gather): more than 2^31 output pixels");
    const long long per_wg = static_cast<long long>(4 / a->KW) * lc.ncb * 32;
    const long long pgroups = (a->npix + per_wg - 1) / per_wg;
    if (pgroups * a->ngk >= (1LL << 31)) return fail("implicit GEMM (gather): grid too large");
    a->ROWS = a->RW = a->padL = a->st_bytes = a->zoff = 0;
    if (staged) {
        // gather element: the dtype's element, or an NCHW4 int8 pixel's dword
        const int gsz = (p.dtype == CFWD_I8) ? 4 : p.esize;
        const int ce = 16 / gsz;  // elements per 16-byte chunk
        const long long ohw = static_cast<long long>(p.oh) * p.ow;
        if (p.dtype != CFWD_I8 && p.xb != 1) return fail("implicit GEMM (gather, staged): NCHW only");
        if (ohw % per_wg != 0) return fail("implicit GEMM (gather, staged): workgroups would straddle images");
        if (p.w % ce != 0 || p.pw > ce) return fail("implicit GEMM (gather, staged): row width or padding");
        const long long spanned = (p.ow - 1 + per_wg - 1) / p.ow + 1;  // output rows a workgroup can touch
        const long long rows = (spanned - 1) * p.sh + static_cast<long long>(p.r - 1) * p.dh + 1;
        const long long need = ce + static_cast<long long>(p.ow - 1) * p.sw - p.pw + static_cast<long long>(p.s - 1) * p.dw + 1;
        long long rw = std::max<long long>(ce + p.w, need);
        rw = (rw + ce - 1) / ce * ce;
        const long long nch = (p.dtype == CFWD_I8) ? 1 : p.c;
        // fp32/bf16: a zero region of one channel's rows after the staged rows
        const long long zrows = (p.dtype == CFWD_I8) ? 0 : rows;
        const long long sb = ((nch * rows + zrows) * rw * gsz + 15) / 16 * 16;
        if (sb + static_cast<long long>(nss) * ssu * static_cast<long long>(sizeof(Tap)) > static_cast<long long>(kLcStageMax))
            return fail("implicit GEMM (gather, staged): input rows of a workgroup exceed the LDS budget");
        a->ROWS = static_cast<int>(rows);
        a->RW = static_cast<int>(rw);
        a->padL = ce;
        a->st_bytes = static_cast<int>(sb);
        a->zoff = static_cast<int>(nch * rows * rw);
    }
    return true;
}

// Dynamic LDS of one workgroup: the larger of the unit table and the
// transposed output tile (with its 16-byte row padding).
template <typename T, int XB, int NCB, int KBW>
size_t lc_lds_bytes(const LcArgs& a) {
    const size_t tabb = static_cast<size_t>(a.st_bytes) + static_cast<size_t>(a.nss) * Lc<T>::SSU * sizeof(Tap);
    size_t tile = 0;
    if (lc_tile_bytes<T, XB, NCB, KBW>() > 0)
        tile = static_cast<size_t>(a.KW) * KBW * 32 * ((4 / a.KW) * NCB * 32 * sizeof(T) + 16);
    return std::max(tabb, tile);
}

template <typename T, int XB, int NCB, int KBW>
void lc_launch_cfg(bool staged, unsigned blocks, const LcArgs& b, const T* xt, const uint8_t* w8, const float* scale,
                   T* yt, hipStream_t st) {
    const size_t lds = lc_lds_bytes<T, XB, NCB, KBW>(b);
    const bool epi = b.e.bias || b.e.res || b.e.relu;
    if constexpr (sizeof(T) == 1 || XB == 1) {
        if (staged) {
            auto kern = epi ? lc_kernel<T, XB, NCB, KBW, true, true> : lc_kernel<T, XB, NCB, KBW, true, false>;
            kern<<<blocks, 256, lds, st>>>(xt, w8, scale, yt, b);
            return;
        }
    }
    auto kern = epi ? lc_kernel<T, XB, NCB, KBW, false, true> : lc_kernel<T, XB, NCB, KBW, false, false>;
    kern<<<blocks, 256, lds, st>>>(xt, w8, scale, yt, b);
}

template <typename T, int XB>
cfwd_status lc_launch_t(int cfg, const LcArgs& a, const void* x, const void* wp, const float* scale, void* y,
                        const Epi& e, hipStream_t st) {
    const bool staged = cfg >= kLcBase;
    cfg %= kLcBase;
    const long long per_wg = static_cast<long long>(4 / a.KW) * kLc[cfg].ncb * 32;
    const unsigned blocks = static_cast<unsigned>((a.npix + per_wg - 1) / per_wg * a.ngk);
    const T* xt = static_cast<const T*>(x);
    const uint8_t* w8 = static_cast<const uint8_t*>(wp);
    T* yt = static_cast<T*>(y);
    // 16-byte output pieces start at pixel multiples of 16 / sizeof(T) of a
    // channel plane: aligned when the planes and the tensor are
    LcArgs b = a;
    b.e = e;
    const long long pe = 16 / static_cast<long long>(sizeof(T));
    b.vec_ok = (reinterpret_cast<uintptr_t>(y) % 16 == 0) && (static_cast<long long>(a.OH) * a.OW) % pe == 0 &&
               a.y_img % pe == 0;
    switch (cfg) {
        case 0: lc_launch_cfg<T, XB, 4, 1>(staged, blocks, b, xt, w8, scale, yt, st); break;
        case 1: lc_launch_cfg<T, XB, 2, 2>(staged, blocks, b, xt, w8, scale, yt, st); break;
        case 2: lc_launch_cfg<T, XB, 4, 2>(staged, blocks, b, xt, w8, scale, yt, st); break;
        case 3: lc_launch_cfg<T, XB, 1, 1>(staged, blocks, b, xt, w8, scale, yt, st); break;
        case 4: lc_launch_cfg<T, XB, 1, 2>(staged, blocks, b, xt, w8, scale, yt, st); break;
        default: lc_launch_cfg<T, XB, 2, 1>(staged, blocks, b, xt, w8, scale, yt, st); break;
    }
    return check_hip(hipGetLastError(), "implicit GEMM (gather) launch");
}

template <typename T>
cfwd_status lc_launch_layout(const Prob& p, int cfg, const LcArgs& a, const void* x, const void* wp,
                             const float* scale, void* y, const Epi& e, hipStream_t st) {
    switch (p.xb) {
        case 1: return lc_launch_t<T, 1>(cfg, a, x, wp, scale, y, e, st);
        case 4: return lc_launch_t<T, 4>(cfg, a, x, wp, scale, y, e, st);
        case 8: return lc_launch_t<T, 8>(cfg, a, x, wp, scale, y, e, st);
        default: return set_error(CFWD_ERR_UNSUPPORTED, "implicit GEMM (gather): bad channel block");
    }
}

}  // namespace

int lowc_num_configs() { return kLcN; }

bool lowc_supported(const Prob& p, int cfg, std::string* why) {
    LcArgs a;
    return lc_geometry(p, cfg, &a, why);
}

size_t lowc_filter_bytes(const Prob& p, int cfg) {
    LcArgs a;
    if (!lc_geometry(p, cfg, &a, nullptr)) return 0;
    return static_cast<size_t>(a.nkb) * a.nss * 64 * 16;
}

cfwd_status lowc_prepare(const Prob& p, int cfg, const void* w, void* wp, hipStream_t st) {
    LcArgs a;
    std::string why;
    if (!lc_geometry(p, cfg, &a, &why)) return set_error(CFWD_ERR_UNSUPPORTED, why);
    const long long total = static_cast<long long>(a.nkb) * a.nss * 64 * 16;
    const unsigned blocks = static_cast<unsigned>(std::min<long long>((total + 255) / 256, 65536));
    uint8_t* out = static_cast<uint8_t*>(wp);
    const int RS = p.r * p.s;
    if (p.dtype == CFWD_F32)
        lc_prepare_kernel<float><<<blocks, 256, 0, st>>>(static_cast<const float*>(w), out, p.k, p.c, RS, a.units,
                                                         a.nkb, a.nss);
    else if (p.dtype == CFWD_BF16)
        lc_prepare_kernel<bf16_t><<<blocks, 256, 0, st>>>(static_cast<const bf16_t*>(w), out, p.k, p.c, RS, a.units,
                                                          a.nkb, a.nss);
    else
        lc_prepare_kernel<int8_t><<<blocks, 256, 0, st>>>(static_cast<const int8_t*>(w), out, p.k, p.c, RS, a.units,
                                                          a.nkb, a.nss);
    return check_hip(hipGetLastError(), "implicit GEMM (gather) filter prepare launch");
}

cfwd_status lowc_launch(const Prob& p, int cfg, const void* x, const void* wp, const float* scale, void* y,
                        const Epi& e, hipStream_t st) {
    LcArgs a;
    std::string why;
    if (!lc_geometry(p, cfg, &a, &why)) return set_error(CFWD_ERR_UNSUPPORTED, why);
    if (wp == nullptr) return set_error(CFWD_ERR_WORKSPACE, "implicit GEMM (gather): prepared filter required");
    if (p.dtype == CFWD_F32) return lc_launch_layout<float>(p, cfg, a, x, wp, scale, y, e, st);
    if (p.dtype == CFWD_BF16) return lc_launch_layout<bf16_t>(p, cfg, a, x, wp, scale, y, e, st);
    return lc_launch_t<int8_t, 4>(cfg, a, x, wp, scale, y, e, st);
}

}  // namespace cfwd
