// Fused bottleneck block: 1x1 (C -> 64), 3x3 pad 1 (64 -> 64), 1x1 (64 -> K),
// stride 1, bf16 NCHW, in one launch (gfx950).
//
// Momenta talk "Paper Reading | 讓深度學習更高效運行的兩個視角": section
// "優化1：Bottleneck" has the block cut the FLOPs about tenfold while moving
// as many bytes, so its arithmetic intensity falls and it becomes bound by
// memory; section "Operator的粒度" splits the second convolution's output
// into spatial tiles so that the first and second convolutions hand their
// tiles over in cache instead of through memory, at the price of recomputing
// the tiles' overlap.  Here the hand-over is in LDS and covers all three
// convolutions: only x is read from HBM and only y is written.
//
// Workgroup = TH = 4 output rows (all W columns) of one image, 8 waves (two
// workgroups per CU: four waves per SIMD to cover each stage's latencies):
//   A  t1 = act1(w1 . x + b1) on the TH + 2 rows the 3x3 needs (its halo is
//      recomputed by the neighbouring workgroups: 1.5x the first 1x1's
//      work).  x arrives in chunks of 32 channels, copied from NCHW rows as
//      they are ([channel][pixel] in LDS); the matrix-core B operand (pixels
//      x channels) comes out of gfx950's transposing LDS read.  w1 is
//      copied once into the area t1 takes afterwards, in operand order, so
//      the four waves share one copy instead of each fetching it.  t1 goes to
//      LDS as bf16 records of 64 channels per pixel, with a zero column on
//      each side and zero rows outside the image (the 3x3's padding).
//   B  t2 = act2(w2 . t1 + b2): nine taps, each a shifted window of the t1
//      records; w2 passes through the idle x staging area three taps at a
//      time (the next three fetched while these run); t2 is then written
//      over that area, same record format.
//   C  y = act3(w3 . t2 + b3 + residual), 32 output channels per pass; each
//      wave owns 64 consecutive output pixels and turns its fragments around
//      through its own LDS slice (no workgroup barrier), so that 8 lanes
//      store one channel's 128 contiguous bytes (16-byte streaming stores);
//      the pass's bias and residual are requested before its products.
// Matrix-core fragments are 16 x 16 (v_mfma_f32_16x16x32_bf16, fp32
// accumulate).  Both intermediates are rounded to bf16, as the three
// separate layers store them.
#include "internal.h"
#include "bottleneck.h"

namespace cfwd {
namespace bn {

constexpr int TH = 4;      // output rows per workgroup
constexpr int MID = 64;    // inner channels
constexpr int NW = 8;      // waves per workgroup (four per SIMD with two workgroups per CU)
constexpr int NTHR = 64 * NW;
constexpr int KC = 32;     // input channels per staged chunk
constexpr int MAXW = 64;
constexpr int TA = 24 / NW;   // stage-A pixel tiles per wave: ceil(3W/8 / NW) for W <= 64
constexpr int TBW = 16 / NW;  // stage-B pixel tiles per wave: ceil(W/4 / NW)
constexpr int TCW = 4;        // stage-C pixel tiles per wave (64 pixels: one 128-byte run per channel)
constexpr int KP = 32;     // output channels per stage-C pass
constexpr int XP = 1536 / NTHR;  // staged 16-byte pieces per thread per chunk: 32 * 6W/8 / NTHR
constexpr int SPITCH = 68; // floats per channel row of a wave's output slice (64 pixels + 4: rows 16 bytes apart in the banks)
constexpr int TG = 3;      // 3x3 taps per staged w2 group
constexpr int W2G = TG * 2 * 4 * 1024;  // bytes of one staged w2 group: [tap][half][mt][lane][16 B]
constexpr int W2P = W2G / (16 * NTHR);  // 16-byte pieces per thread per group

typedef short s4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) s4 lds_s4;

struct Args {
    const uint16_t* x;
    const uint16_t* w1;   // [64][C] (KCRS, 1x1)
    const uint16_t* w2p;  // [9 taps][64][64] (prepared)
    const uint16_t* w3;   // [K][64] (KCRS, 1x1)
    const float* b1;
    const float* b2;
    const float* b3;
    const uint16_t* res;  // [N][K][H][W] or null
    uint16_t* y;
    int C, H, W, K;
    int relu1, relu2, relu3;
    int tiles_h, ntiles, xcd_remap;
    int px_a, px_b;       // (TH + 2) * W, TH * W
    int pitch_x;          // x staging row pitch (elements)
    int r1;               // byte offset of the second LDS region
};

// 16-byte slot of a 128-byte pixel record, spread over the banks: record p
// keeps slot s at s ^ ((p >> 1) & 7), so 16 consecutive records read at one
// slot touch 16 different bank groups.
__device__ __forceinline__ int rec_off(int p, int slot) { return p * 128 + ((slot ^ ((p >> 1) & 7)) << 4); }

__device__ __forceinline__ uint4 mfma_in(uint2 lo, uint2 hi) { return make_uint4(lo.x, lo.y, hi.x, hi.y); }

// 16-byte load / store as one vector access (a plain uint4 struct copy can
// become a memcpy through private memory)
__device__ __forceinline__ uint4 ld16(const void* p) { return __builtin_bit_cast(uint4, *reinterpret_cast<const i32x4*>(p)); }
__device__ __forceinline__ void st16(void* p, const uint4& v) { *reinterpret_cast<i32x4*>(p) = __builtin_bit_cast(i32x4, v); }

__device__ __forceinline__ f32x4 mma(const uint4& a, const uint4& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0, 0,
                                                   0);
}

__device__ __forceinline__ float act(float v, int relu) { return relu ? fmaxf(v, 0.0f) : v; }

__global__ __launch_bounds__(NTHR, 2) void bottleneck_kernel(Args a) {
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    uint8_t* R0 = lds;          // x staging, then t2
    uint8_t* R1 = lds + a.r1;   // t1, then the output staging
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 4, i = lane & 15;
    const int C = a.C, H = a.H, W = a.W, K = a.K;

    int b = blockIdx.x;
    if (a.xcd_remap) b = (b & 7) * (a.ntiles >> 3) + (b >> 3);  // neighbouring row tiles on one XCD
    const int n = b / a.tiles_h;
    const int oh0 = (b % a.tiles_h) * TH;

    // ------------------------------------------------------------ stage A
    const int wp = W >> 3;             // 16-byte pieces per row
    const int ppc = (TH + 2) * wp;     // per channel of a chunk
    const int npieces = KC * ppc;
    int xg[XP], xl[XP];                // global element offset (chunk 0), LDS byte offset; xg < 0: zero
#pragma unroll
    for (int u = 0; u < XP; ++u) {
        const int q = tid + NTHR * u;
        xl[u] = -1;
        xg[u] = -1;
        if (q < npieces) {
            const int ch = q / ppc, pc = q % ppc;
            const int row = pc / wp, c8 = pc % wp;
            const int ih = oh0 - 1 + row;
            xl[u] = (ch * a.pitch_x + pc * 8) * 2;
            if (ih >= 0 && ih < H) xg[u] = (ch * H + ih) * W + c8 * 8;
        }
    }
    const uint16_t* xn = a.x + static_cast<long long>(n) * C * H * W;
    const long long chunk_elems = static_cast<long long>(KC) * H * W;
    // two register sets, so that two chunks are in flight while one is used
    uint4 xa[XP], xb[XP];
    auto load_x = [&](uint4 (&xr)[XP], int chunk) __attribute__((always_inline)) {
        const uint16_t* xc = xn + chunk * chunk_elems;
#pragma unroll
        for (int u = 0; u < XP; ++u) xr[u] = (xg[u] >= 0) ? ld16(xc + xg[u]) : make_uint4(0, 0, 0, 0);
    };
    auto store_x = [&](const uint4 (&xr)[XP]) __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < XP; ++u)
            if (xl[u] >= 0) st16(R0 + xl[u], xr[u]);
    };
    // transposing-read byte offsets of this lane's pixel tiles: lane j of a
    // 16-lane group reads 4 pixels (4 * (j & 3) ..) of channel row 4g + j / 4
    // (+16 for the second read); the group's lanes then hold channels
    // 4g .. 4g + 3 (and 16 + 4g ..) of pixel i of the tile
    const int ntA = a.px_a >> 4;
    int troff[TA];
#pragma unroll
    for (int u = 0; u < TA; ++u) {
        const int jt = min(wave + NW * u, ntA - 1);
        troff[u] = ((4 * g + (i >> 2)) * a.pitch_x + 16 * jt + 4 * (i & 3)) * 2;
    }
    const int tr2 = 16 * a.pitch_x * 2;
    // w1 in R1 as A operands, [chunk][mt][lane][16 B]: lane (g, i) of tile mt
    // holds row 16 mt + i, channels 4g .. 4g + 3 and 16 + 4g .. of the chunk
    // (the channel order of the B operand)
    for (int q = tid; q < (C / KC) * 4 * 64; q += NTHR) {
        const int ln = q & 63, mt = (q >> 6) & 3, chunk = q >> 8;
        const uint16_t* r = a.w1 + (16 * mt + (ln & 15)) * C + chunk * KC + 4 * (ln >> 4);
        *reinterpret_cast<uint4*>(R1 + q * 16) =
            mfma_in(*reinterpret_cast<const uint2*>(r), *reinterpret_cast<const uint2*>(r + 16));
    }

    f32x4 accA[TA][4];
#pragma unroll
    for (int u = 0; u < TA; ++u)
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) accA[u][mt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    const int nch = C / KC;
    auto chunk_mma = [&](int c) __attribute__((always_inline)) {
        uint4 w1c[4];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) w1c[mt] = ld16(R1 + ((c * 4 + mt) * 64 + lane) * 16);
#pragma unroll
        for (int u = 0; u < TA; ++u) {
            const s4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4*)(R0 + troff[u]));
            const s4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4*)(R0 + troff[u] + tr2));
            const uint4 bx = mfma_in(__builtin_bit_cast(uint2, lo), __builtin_bit_cast(uint2, hi));
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) accA[u][mt] = mma(w1c[mt], bx, accA[u][mt]);
        }
    };
    // chunk c + 1 waits in one register set while chunk c + 2 loads into the
    // other; the loop takes two chunks per iteration so each set is fixed
    load_x(xa, 0);
    store_x(xa);
    if (nch > 1) load_x(xa, 1);
    if (nch > 2) load_x(xb, 2);
    __syncthreads();
    for (int c = 0; c < nch; c += 2) {
        chunk_mma(c);
        __syncthreads();  // every wave is done with chunk c
        if (c + 1 < nch) {
            store_x(xa);
            if (c + 3 < nch) load_x(xa, c + 3);
        }
        __syncthreads();  // chunk c + 1 is in LDS
        if (c + 1 < nch) {
            chunk_mma(c + 1);
            __syncthreads();
            if (c + 2 < nch) {
                store_x(xb);
                if (c + 4 < nch) load_x(xb, c + 4);
            }
            __syncthreads();
        }
    }

    // w2 passes through R0 (free until t2 is written) one filter row (TG = 3
    // taps) at a time: [tap][half][mt][lane][16 B], lane (g, i) of tile mt
    // holding row 16 mt + i, inner channels 32 half + 8g .. + 7 of the tap.
    // Each thread moves the same W2P pieces of every row: src_w2 is their
    // offset in the prepared w2 of filter row 0.
    int src_w2[W2P];
#pragma unroll
    for (int u = 0; u < W2P; ++u) {
        const int q = tid + NTHR * u;
        const int ln = q & 63, mt = (q >> 6) & 3, hh = (q >> 8) & 1, lt = q >> 9;
        src_w2[u] = (lt * MID + 16 * mt + (ln & 15)) * MID + 32 * hh + 8 * (ln >> 4);
    }
    uint4 w2s[W2P];
#pragma unroll
    for (int u = 0; u < W2P; ++u) w2s[u] = ld16(a.w2p + src_w2[u]);

    // t1 records: [TH + 2 rows][W + 2 columns], zero columns at both ends
    const int W2 = W + 2;
    if (tid < 12 * 8) {
        const int rec = tid >> 3, part = tid & 7;
        const int p = (rec >> 1) * W2 + ((rec & 1) ? W + 1 : 0);
        *reinterpret_cast<uint4*>(R1 + p * 128 + part * 16) = make_uint4(0, 0, 0, 0);
    }
    {
        float bias[4][4];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int v = 0; v < 4; ++v) bias[mt][v] = a.b1 ? a.b1[16 * mt + 4 * g + v] : 0.0f;
#pragma unroll
        for (int u = 0; u < TA; ++u) {
            const int jt = wave + NW * u;
            if (jt >= ntA) continue;
            const int p = 16 * jt + i;
            const int row = p / W, col = p - row * W;
            const int ih = oh0 - 1 + row;
            const bool in = ih >= 0 && ih < H;
            const int rp = row * W2 + col + 1;
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) {
                float v0 = act(accA[u][mt][0] + bias[mt][0], a.relu1), v1 = act(accA[u][mt][1] + bias[mt][1], a.relu1);
                float v2 = act(accA[u][mt][2] + bias[mt][2], a.relu1), v3 = act(accA[u][mt][3] + bias[mt][3], a.relu1);
                uint2 d = in ? make_uint2(pack_bf16x2(v0, v1), pack_bf16x2(v2, v3)) : make_uint2(0, 0);
                *reinterpret_cast<uint2*>(R1 + rec_off(rp, 2 * mt + (g >> 1)) + (g & 1) * 8) = d;
            }
        }
    }
    __syncthreads();

    // ------------------------------------------------------------ stage B
    const int ntB = a.px_b >> 4;
    int rp0[TBW];
#pragma unroll
    for (int u = 0; u < TBW; ++u) {
        const int jt = min(wave + NW * u, ntB - 1);
        const int p = 16 * jt + i;
        const int orow = p / W, ocol = p - orow * W;
        rp0[u] = (orow + 1) * W2 + ocol + 1;
    }
    f32x4 accB[TBW][4];
#pragma unroll
    for (int u = 0; u < TBW; ++u)
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) accB[u][mt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int u = 0; u < W2P; ++u) st16(R0 + (tid + NTHR * u) * 16, w2s[u]);
    __syncthreads();
#pragma unroll 1
    for (int fr = 0; fr < 3; ++fr) {  // filter row
        const bool more = fr + 1 < 3;
        if (more) {
#pragma unroll
            for (int u = 0; u < W2P; ++u)
                w2s[u] = ld16(a.w2p + (fr + 1) * TG * MID * MID + src_w2[u]);
        }
#pragma unroll
        for (int ls = 0; ls < 2 * TG; ++ls) {  // (filter column, inner-channel half)
            const int shift = (fr - 1) * W2 + ((ls >> 1) - 1);
            uint4 wa[4], bt[TBW];
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
                wa[mt] = *reinterpret_cast<const uint4*>(R0 + ((ls * 4 + mt) * 64 + lane) * 16);
#pragma unroll
            for (int u = 0; u < TBW; ++u)
                bt[u] = *reinterpret_cast<const uint4*>(R1 + rec_off(rp0[u] + shift, 4 * (ls & 1) + g));
#pragma unroll
            for (int u = 0; u < TBW; ++u)
#pragma unroll
                for (int mt = 0; mt < 4; ++mt) accB[u][mt] = mma(wa[mt], bt[u], accB[u][mt]);
        }
        __syncthreads();  // every wave is done with this filter row
        if (more) {
#pragma unroll
            for (int u = 0; u < W2P; ++u) st16(R0 + (tid + NTHR * u) * 16, w2s[u]);
            __syncthreads();
        }
    }
    // t2 records [TH * W] over the x staging (stage A is done with it)
    {
        float bias[4][4];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int v = 0; v < 4; ++v) bias[mt][v] = a.b2 ? a.b2[16 * mt + 4 * g + v] : 0.0f;
#pragma unroll
        for (int u = 0; u < TBW; ++u) {
            const int jt = wave + NW * u;
            if (jt >= ntB) continue;
            const int p = 16 * jt + i;
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) {
                float v0 = act(accB[u][mt][0] + bias[mt][0], a.relu2), v1 = act(accB[u][mt][1] + bias[mt][1], a.relu2);
                float v2 = act(accB[u][mt][2] + bias[mt][2], a.relu2), v3 = act(accB[u][mt][3] + bias[mt][3], a.relu2);
                *reinterpret_cast<uint2*>(R0 + rec_off(p, 2 * mt + (g >> 1)) + (g & 1) * 8) =
                    make_uint2(pack_bf16x2(v0, v1), pack_bf16x2(v2, v3));
            }
        }
    }
    __syncthreads();

    // ------------------------------------------------------------ stage C
    // (R1 is free: every wave passed the barrier above after its last read
    // of t1.)  Wave w owns the band's output pixels [64 pg, 64 pg + 64),
    // pg = w % 4 (pixel tiles 4 pg .. 4 pg + 3; tiles past the band repeat
    // the last one, unstored), and channels 16 kh .. 16 kh + 15 of each pass
    // of 32, kh = w / 4.  Per pass its fragments go through a private LDS
    // slice [16 channels][68-float pitch] and come back as 8 consecutive
    // pixels of one channel per lane: 16-byte streaming stores, 8 lanes per
    // channel (128 contiguous bytes).
    const int pg = wave & 3, kh = wave >> 2;
    uint4 ta[TCW][2];
#pragma unroll
    for (int u = 0; u < TCW; ++u) {
        const int jt = min(4 * pg + u, ntB - 1);
        const int p = 16 * jt + i;
#pragma unroll
        for (int s = 0; s < 2; ++s) ta[u][s] = ld16(R0 + rec_off(p, 4 * s + g));
    }
    uint4 wc[2], wn[2];
    auto load_w3 = [&](uint4 (&w)[2], int k0) __attribute__((always_inline)) {
#pragma unroll
        for (int s = 0; s < 2; ++s) w[s] = ld16(a.w3 + (k0 + 16 * kh + i) * MID + 32 * s + 8 * g);
    };
    float* ST = reinterpret_cast<float*>(R1) + wave * (16 * SPITCH);
    const uint16_t* resn = a.res ? a.res + static_cast<long long>(n) * K * H * W : nullptr;
    uint16_t* yn = a.y + static_cast<long long>(n) * K * H * W;
    const long long plane = static_cast<long long>(H) * W;
    // store pieces q = lane + 64 r: channel 16 kh + q / 8 of the pass, pixels 8 (q % 8) ..
    int pofs[2];  // offset in a channel plane; < 0: nothing to store
#pragma unroll
    for (int r = 0; r < 2; ++r) {
        const int q = lane + 64 * r;
        const int px = 64 * pg + 8 * (q & 7);
        const int orow = px / W, col = px - orow * W;
        const int oh = oh0 + orow;
        pofs[r] = (px < a.px_b && oh < H) ? oh * W + col : -1;
    }
    const int npass = K / KP;
    load_w3(wc, 0);
    for (int kp = 0; kp < npass; ++kp) {
        if (kp + 1 < npass) load_w3(wn, (kp + 1) * KP);
        const int k0 = kp * KP + 16 * kh;
        // the epilogue operands of this pass, requested before its products
        float bk[2];
        uint4 rv[2];
#pragma unroll
        for (int r = 0; r < 2; ++r) {
            const int k = k0 + ((lane + 64 * r) >> 3);
            bk[r] = a.b3 ? a.b3[k] : 0.0f;
            rv[r] = (resn && pofs[r] >= 0) ? ld16(resn + k * plane + pofs[r]) : make_uint4(0, 0, 0, 0);
        }
        // D[pixel][channel]: lane holds channel i (of this wave's 16), pixels 16 u + 4g .. + 3
#pragma unroll
        for (int u = 0; u < TCW; ++u) {
            f32x4 c4 = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int s = 0; s < 2; ++s) c4 = mma(ta[u][s], wc[s], c4);
            *reinterpret_cast<f32x4*>(ST + i * SPITCH + 16 * u + 4 * g) = c4;
        }
#pragma unroll
        for (int r = 0; r < 2; ++r) {
            const int q = lane + 64 * r;
            const float* src = ST + (q >> 3) * SPITCH + 8 * (q & 7);
            const f32x4 lo = *reinterpret_cast<const f32x4*>(src);
            const f32x4 hi = *reinterpret_cast<const f32x4*>(src + 4);
            const float v[8] = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            // a missing residual reads as +0, which changes nothing but a -0
            const uint32_t rw[4] = {rv[r].x, rv[r].y, rv[r].z, rv[r].w};
            uint32_t o[4];
#pragma unroll
            for (int e = 0; e < 4; ++e)
                o[e] = pack_bf16x2(act(v[2 * e] + bk[r] + bf16_to_float(static_cast<uint16_t>(rw[e] & 0xffffu)), a.relu3),
                                   act(v[2 * e + 1] + bk[r] + bf16_to_float(static_cast<uint16_t>(rw[e] >> 16)), a.relu3));
            // streaming store: y is not read again by this kernel
            if (pofs[r] >= 0)
                __builtin_nontemporal_store(i32x4{static_cast<int>(o[0]), static_cast<int>(o[1]), static_cast<int>(o[2]),
                                                  static_cast<int>(o[3])},
                                            reinterpret_cast<i32x4*>(yn + (k0 + (q >> 3)) * plane + pofs[r]));
        }
#pragma unroll
        for (int s = 0; s < 2; ++s) wc[s] = wn[s];
    }
}

// w2p[tap][m2][m] = w2[m2][m][tap / 3][tap % 3]
__global__ __launch_bounds__(256) void prepare_w2_kernel(const uint16_t* __restrict__ w2, uint16_t* __restrict__ w2p) {
    const int idx = blockIdx.x * 256 + threadIdx.x;
    if (idx >= 9 * MID * MID) return;
    const int m = idx % MID, m2 = (idx / MID) % MID, tap = idx / (MID * MID);
    w2p[idx] = w2[(m2 * MID + m) * 9 + tap];
}

struct Plan {
    int tiles_h, ntiles, px_a, px_b, pitch_x, r1, lds;
};

inline int round_to_residue(int v, int mod, int res) {  // smallest v' >= v with v' % mod == res
    const int r = ((res - v % mod) % mod + mod) % mod;
    return v + r;
}

bool plan(const cfwd_bottleneck_desc* d, Plan* pl, std::string* why) {
    auto no = [&](const char* m) {
        if (why) *why = m;
        return false;
    };
    if (d->dtype != CFWD_BF16) return no("bottleneck block: bf16 only");
    if (d->n < 1 || d->c < 1 || d->h < 1 || d->w < 1 || d->k < 1 || d->mid < 1) return no("bottleneck block: sizes must be positive");
    if (d->mid != MID) return no("bottleneck block: the inner convolutions must have 64 channels");
    if (d->c % KC != 0) return no("bottleneck block: input channels must be a multiple of 32");
    if (d->k % KP != 0) return no("bottleneck block: output channels must be a multiple of 32");
    if (d->w % 8 != 0 || d->w > MAXW) return no("bottleneck block: width must be a multiple of 8, at most 64");
    if (static_cast<long long>(d->c) * d->h * d->w >= (1LL << 31) || static_cast<long long>(d->k) * d->h * d->w >= (1LL << 31))
        return no("bottleneck block: an image of x or y must hold fewer than 2^31 elements");
    pl->tiles_h = (d->h + TH - 1) / TH;
    const long long nt = static_cast<long long>(d->n) * pl->tiles_h;
    if (nt > (1LL << 30)) return no("bottleneck block: too many tiles");
    pl->ntiles = static_cast<int>(nt);
    pl->px_a = (TH + 2) * d->w;
    pl->px_b = TH * d->w;
    // x staging rows 32 banks apart modulo 64 (conflict-free transposing
    // reads)
    pl->pitch_x = round_to_residue(pl->px_a, 32, 16);
    const int r0 = std::max(std::max(KC * pl->pitch_x * 2, pl->px_b * 128), W2G);
    pl->r1 = (r0 + 255) / 256 * 256;
    // t1; w1 in operand order during the first 1x1; the waves' output slices
    const int r1b = std::max(std::max((TH + 2) * (d->w + 2) * 128, d->c * 128), NW * 16 * SPITCH * 4);
    pl->lds = pl->r1 + r1b;
    if (pl->lds > 160 * 1024) return no("bottleneck block: too many input channels for LDS (w1 is staged whole)");
    return true;
}

}  // namespace bn

cfwd_status bottleneck_check(const cfwd_bottleneck_desc* d, std::string* why) {
    if (!d) {
        if (why) *why = "desc must not be NULL";
        return CFWD_ERR_INVALID_ARG;
    }
    bn::Plan pl;
    return bn::plan(d, &pl, why) ? CFWD_OK : CFWD_ERR_UNSUPPORTED;
}

size_t bottleneck_filter_bytes() { return static_cast<size_t>(9) * bn::MID * bn::MID * 2; }

cfwd_status bottleneck_prepare(const void* w2, void* w2p, hipStream_t st) {
    bn::prepare_w2_kernel<<<(9 * bn::MID * bn::MID + 255) / 256, 256, 0, st>>>(static_cast<const uint16_t*>(w2),
                                                                               static_cast<uint16_t*>(w2p));
    return check_hip(hipGetLastError(), "bottleneck w2 prepare launch");
}

cfwd_status bottleneck_launch(const cfwd_bottleneck_desc* d, const void* x, const void* w1, const void* w2p,
                              const void* w3, const cfwd_bottleneck_epilogue* e, void* y, hipStream_t st) {
    bn::Plan pl;
    std::string why;
    if (!bn::plan(d, &pl, &why)) return set_error(CFWD_ERR_UNSUPPORTED, why);
    bn::Args a;
    a.x = static_cast<const uint16_t*>(x);
    a.w1 = static_cast<const uint16_t*>(w1);
    a.w2p = static_cast<const uint16_t*>(w2p);
    a.w3 = static_cast<const uint16_t*>(w3);
    a.b1 = e ? static_cast<const float*>(e->b1) : nullptr;
    a.b2 = e ? static_cast<const float*>(e->b2) : nullptr;
    a.b3 = e ? static_cast<const float*>(e->b3) : nullptr;
    a.res = e ? static_cast<const uint16_t*>(e->residual) : nullptr;
    a.y = static_cast<uint16_t*>(y);
    a.C = d->c;
    a.H = d->h;
    a.W = d->w;
    a.K = d->k;
    a.relu1 = e ? (e->relu1 != 0) : 0;
    a.relu2 = e ? (e->relu2 != 0) : 0;
    a.relu3 = e ? (e->relu3 != 0) : 0;
    a.tiles_h = pl.tiles_h;
    a.ntiles = pl.ntiles;
    a.xcd_remap = (pl.ntiles % 8 == 0) ? 1 : 0;
    a.px_a = pl.px_a;
    a.px_b = pl.px_b;
    a.pitch_x = pl.pitch_x;
    a.r1 = pl.r1;
    static bool attr = false;
    if (!attr) {
        hipError_t he = hipFuncSetAttribute(reinterpret_cast<const void*>(bn::bottleneck_kernel),
                                            hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
        if (he != hipSuccess) return check_hip(he, "hipFuncSetAttribute(bottleneck)");
        attr = true;
    }
    bn::bottleneck_kernel<<<pl.ntiles, bn::NTHR, pl.lds, st>>>(a);
    return check_hip(hipGetLastError(), "bottleneck launch");
}

}  // namespace cfwd
