// Persistent implicit GEMM for int8 NCHW4 layers whose reduction is one
// channel chunk (C <= 64: ResNet-18's 56x56 stage, its first stride-2 3x3
// and 1x1 layers).
//
// The MegEngine inference article (section "Im2col+MatMul") blocks the
// im2col matrix along oh*ow so a block's data stays close to the core; the
// tiled kernel of igemm_impl.h does that per workgroup.  With a single
// channel chunk, though, a tile is one load, nine taps and one store: each
// workgroup's life is mostly waiting, first for its input rows and then for
// its stores, and all workgroups wait at the same time.  Here a fixed set of
// workgroups (as many as fit on the CUs at once) walks the tiles, and while
// tile i is on the matrix cores the input rows of tile i + 1 are already in
// flight to a second LDS buffer:
//
//   load rows(i+1) -> registers | taps of tile i from LDS buffer i%2
//   requantise tile i into the output-staging region, barrier, store it
//   write rows(i+1) to buffer (i+1)%2, barrier
//
// Tiles are whole output rows of one image (TH rows x OW columns) and one
// output-channel block of NT = WN*FN*32 channels; 32x32x32 int8 MFMA, two
// per 64-byte channel chunk (pieces 0 and 1, channel slots 2i + h as in the
// tiled kernel, whose prepared filter this kernel reads).  The input rows are
// staged with 16-byte loads along W (4 pixels x 4 channels of NCHW4),
// transposed in registers to channel-innermost 80-byte pixel slots.
// Requantisation (and the fused epilogue) is the library's rule.
#include "igemm_impl.h"

namespace cfwd {
namespace st {

using ig::f32x16;
using ig::i32x16;
using ig::u32x4_t;

struct Args {
    const int8_t* x;
    const uint8_t* wp;
    const float* scale;
    int8_t* y;
    int N, K, H, W, OH, OW, S, sh, sw, ph, pw, dh, dw;
    int cb_in;  // channel blocks of x (C / 4)
    long long x_img, y_img;
    int TH, PH, PW, npix, ncb, cb0;  // tile rows, input rows / columns staged, first 4-column block
    int tiles_h, ntk, ntiles;
    Epi e;
};

constexpr int PIXB = 80;   // LDS bytes per staged pixel (64 of channels + 16 pad)
constexpr int SMAXU = 4;   // staging units per thread (a unit: 4 pixels x 16 channels)

struct Cfg {
    int wm, wn, fm, fn;
    int threads() const { return wm * wn * 64; }
    int pixels() const { return wm * fm * 32; }
    int nt() const { return wn * fn * 32; }
};
constexpr Cfg kCfgs[] = {
    {2, 2, 4, 1},  // 0: 256 px x  64 ch
    {4, 1, 2, 2},  // 1: 256 px x  64 ch
    {2, 2, 2, 2},  // 2: 128 px x 128 ch
    {2, 2, 4, 2},  // 3: 256 px x 128 ch
};
constexpr int kNumCfgs = sizeof(kCfgs) / sizeof(kCfgs[0]);
// the tiled kernel's config whose prepared filter (same N tile, 32x32
// fragments) each of these reads
constexpr int kFilterOf[kNumCfgs] = {13, 13, 11, 10};

template <int WM, int WN, int FM, int FN, int RS, bool EPI>
__global__ __launch_bounds__(WM* WN * 64) void stream_kernel(Args a) {
    constexpr int NTHR = WM * WN * 64;
    constexpr int NT = WN * FN * 32;
    constexpr int D = (RS == 9) ? 3 : 2;  // weight ring (taps ahead + 1)
    // 3x3 layers: every load and store of a tile is issued unconditionally
    // (buffer accesses whose padding ones fall past the range), so that the
    // compiler's waits count them exactly and leave the next tile's input
    // rows and the previous tile's stores in flight.  1x1 layers (one tap,
    // nothing to overlap the rows with) keep the plain form, measured
    // faster there.
    constexpr bool PIPE = RS > 1;
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave % WM, wn = wave / WM;
    const int lrow = lane & 31, h = lane >> 5;
    const int patch_bytes = a.npix * PIXB;
    uint8_t* const ebuf = lds + 2 * patch_bytes;  // output staging
    const int tile_pix = a.TH * a.OW;
    const int pitch = tile_pix * 4 + 16;  // bytes per output channel block in ebuf

    // XCD-aware tile order: the workgroups of one XCD (blockIdx % 8) walk a
    // contiguous range of tiles, so neighbouring row bands (which share
    // halo rows) and the channel blocks of one band meet in one L2
    const int G = gridDim.x;
    const int xcd = blockIdx.x & 7, local = blockIdx.x >> 3;
    const int gx = (G >> 3) + (xcd < (G & 7) ? 1 : 0);  // workgroups on this XCD
    const int tper = a.ntiles >> 3, trem = a.ntiles & 7;
    const int tfirst = xcd * tper + min(xcd, trem);
    const int tcount = tper + (xcd < trem ? 1 : 0);

    // ---- staging: unit u = (patch row, 4-column block, 16-channel slot j)
    const int nunits = a.PH * a.ncb * 4;
    const unsigned HW4 = static_cast<unsigned>(a.H * a.W) * 4u;  // bytes per channel-block plane
    uint4 stg[SMAXU][4];
    auto tile_of = [&](int k, int& n, int& th, int& kt) {
        const int lin = tfirst + k;
        kt = lin % a.ntk;
        const int r = lin / a.ntk;
        th = r % a.tiles_h;
        n = r / a.tiles_h;
    };
    auto stage_load = [&](int n, int th) {
        const int ih0 = th * a.TH * a.sh - a.ph;
        // the image, also as a buffer: loads past its range return zeros
        const int8_t* xn = a.x + static_cast<long long>(n) * a.x_img;
        const __amdgpu_buffer_rsrc_t xr =
            __builtin_amdgcn_make_buffer_rsrc(const_cast<int8_t*>(xn), 0, static_cast<int>(a.x_img), 0x00020000);
#pragma unroll
        for (int m = 0; m < SMAXU; ++m) {
            const int u = tid + m * NTHR;
            const int j = u & 3, t = u >> 2;
            const int cbk = t % a.ncb, prow = t / a.ncb;
            const int ih = ih0 + prow, iwb = (a.cb0 + cbk) * 4;
            const bool rowok = u < nunits && static_cast<unsigned>(ih) < static_cast<unsigned>(a.H) && iwb >= 0 &&
                               iwb < a.W;
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                const int cbi = 4 * j + b;  // input channel block
                const bool ok = rowok && cbi < a.cb_in;
                if constexpr (PIPE) {
                    // every load is issued, the padding ones past the
                    // buffer's range (zeros from the hardware): with a select
                    // or branch here the compiler makes the loads conditional
                    const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(
                        xr,
                        ok ? static_cast<unsigned>(cbi) * HW4 + static_cast<unsigned>((ih * a.W + iwb) * 4) : 0x80000000u,
                        0, 0);
                    stg[m][b] = make_uint4(v[0], v[1], v[2], v[3]);
                } else {
                    const int8_t* src = xn + (ok ? static_cast<long long>(cbi) * HW4 + (ih * a.W + iwb) * 4 : 0);
                    const uint4 v = *reinterpret_cast<const uint4*>(src);
                    stg[m][b] = ok ? v : make_uint4(0, 0, 0, 0);
                }
            }
        }
    };
    auto stage_store = [&](uint8_t* buf) {
#pragma unroll
        for (int m = 0; m < SMAXU; ++m) {
            const int u = tid + m * NTHR;
            if (u >= nunits) continue;
            const int j = u & 3, t = u >> 2;
            const int cbk = t % a.ncb, prow = t / a.ncb;
            const int pcol0 = (a.cb0 + cbk) * 4 + a.pw;  // patch column of the block's first pixel
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                const int pcol = pcol0 + p;
                if (pcol >= 0 && pcol < a.PW)
                    *reinterpret_cast<uint4*>(buf + (prow * a.PW + pcol) * PIXB + j * 16) = ig::wide_pick<4>(stg[m], p);
            }
        }
    };

    // ---- A: per fragment the patch pixel of tap (0, 0) (tile rows past the
    // tile read pixel 0; their outputs are never stored)
    int qb[FM];
#pragma unroll
    for (int f = 0; f < FM; ++f) {
        const int p = (wm * FM + f) * 32 + lrow;
        int q = 0;
        if (p < tile_pix) {
            const int ohl = p / a.OW, owl = p - (p / a.OW) * a.OW;
            q = ohl * a.sh * a.PW + owl * a.sw;
        }
        qb[f] = q * PIXB + h * 16;  // piece 0: slot h; piece 1: slot 2 + h (+32 bytes)
    }
    int toff[RS];
#pragma unroll
    for (int t = 0; t < RS; ++t) toff[t] = ((t / a.S) * a.dh * a.PW + (t % a.S) * a.dw) * PIXB;

    // ---- B: prepared filter [ntk][1 chunk][RS][NT/32][piece][32 rows][half][16 B]
    const int boff = (wn * FN * 2 * 32 + lrow) * 32 + h * 16;
    auto load_b = [&](uint4 (&b)[FN][2], int kt, int t) {
        const uint8_t* p = a.wp + (static_cast<long long>(kt) * RS + t) * NT * 64 + boff;
#pragma unroll
        for (int nf = 0; nf < FN; ++nf)
#pragma unroll
            for (int i = 0; i < 2; ++i) b[nf][i] = *reinterpret_cast<const uint4*>(p + (nf * 2 + i) * 1024);
    };

    if (local >= tcount) return;  // more workgroups than tiles on this XCD
    int n, th, kt;
    tile_of(local, n, th, kt);
    stage_load(n, th);
    stage_store(lds);
    uint4 wr[D][FN][2];
    load_b(wr[0], kt, 0);
    if constexpr (RS == 9) load_b(wr[1], kt, 1);
    if constexpr (PIPE) {
        // On the loop's back edge the carried weights are followed by the
        // tile's FM * FN stores; on entry the same number of stores follow
        // them, all past a zero-sized buffer (dropped by the hardware), so
        // that the waits at the first taps, which must hold on both paths,
        // leave the real stores in flight.
        const __amdgpu_buffer_rsrc_t none = __builtin_amdgcn_make_buffer_rsrc(a.y, 0, 0, 0x00020000);
        const u32x4_t z = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int it = 0; it < FM * FN; ++it) __builtin_amdgcn_raw_buffer_store_b128(z, none, 0x80000000u, 0, 2);
    }
    __syncthreads();

    int buf = 0;
    for (int k = local; k < tcount; k += gx) {
        const int kn = k + gx;
        const bool more = kn < tcount;
        int nn = n, thn = th, ktn = kt;
        if (more) tile_of(kn, nn, thn, ktn);
        if constexpr (!PIPE) {
            if (more) stage_load(nn, thn);
        }
        const uint8_t* pb = lds + buf * patch_bytes;

        i32x16 acc[FM][FN];
#pragma unroll
        for (int f = 0; f < FM; ++f)
#pragma unroll
            for (int nf = 0; nf < FN; ++nf) acc[f][nf] = i32x16{};
        uint4 ra[2][FM][2];
#pragma unroll
        for (int f = 0; f < FM; ++f) {
            ra[0][f][0] = *reinterpret_cast<const uint4*>(pb + qb[f] + toff[0]);
            ra[0][f][1] = *reinterpret_cast<const uint4*>(pb + qb[f] + toff[0] + 32);
        }
#pragma unroll
        for (int t = 0; t < RS; ++t) {
            // weights: tap t + D - 1 of this tile, or the first taps of the
            // next (of this tile's block again after the last tile: a valid
            // load that is never used).  No branch around the loads, so
            // the waits for them count exactly the operations issued after
            // them and leave the previous tile's stores in flight.
            {
                const int tt = t + D - 1;
                if (tt < RS)
                    load_b(wr[tt % D], kt, tt);
                else if (PIPE || more)
                    load_b(wr[tt % D], ktn, tt - RS);
            }
            if (t + 1 < RS) {
#pragma unroll
                for (int f = 0; f < FM; ++f) {
                    ra[(t + 1) & 1][f][0] = *reinterpret_cast<const uint4*>(pb + qb[f] + toff[t + 1]);
                    ra[(t + 1) & 1][f][1] = *reinterpret_cast<const uint4*>(pb + qb[f] + toff[t + 1] + 32);
                }
            }
            // piece-major: the two MFMAs into one accumulator are FM * FN
            // instructions apart (back to back, the second would wait for
            // the first's result)
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int f = 0; f < FM; ++f)
#pragma unroll
                    for (int nf = 0; nf < FN; ++nf)
                        ig::Mma32<int8_t>::piece(acc[f][nf], wr[t % D][nf][i], ra[t & 1][f][i], i);
            if constexpr (PIPE) {
                // The next tile's input rows (on the last tile its own rows
                // again, never written to LDS), issued once the first two
                // taps have waited for the weights carried over from the
                // previous tile: issued before those waits, these loads
                // (which the compiler places in branches) would be drained
                // by them, together with the previous tile's stores.  The
                // scheduler barriers keep them here: left alone, the
                // compiler moves them to the end of the taps.
                if (t == 1) {
                    __builtin_amdgcn_sched_barrier(0);
                    stage_load(nn, thn);
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
        }

        // ---- epilogue: requantise into ebuf as [channel block][tile pixel][4 channels].
        // The weights are the products' A operand, so D is [channel][pixel]:
        // a lane holds pixel (wm FM + f) 32 + lrow and, for each j, the 4
        // consecutive channels (wn FN + nf) 32 + 8 j + 4 h + v of one NCHW4
        // block -- one requantised dword, no transpose across lanes.
        const int oh0 = th * a.TH;
        const int kt0 = kt * NT;
#pragma unroll
        for (int nf = 0; nf < FN; ++nf) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int kb = (wn * FN + nf) * 32 + 8 * j + 4 * h;  // the block's first channel in the tile
                const int kc0 = kt0 + kb;
                const bool kval = kc0 < a.K;  // K % 4 == 0: the whole block is real or padding
                float sc[4];
                int eb[4];
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const float s0 = a.scale[kval ? kc0 + v : 0];
                    sc[v] = kval ? s0 : 0.0f;
                    eb[v] = (EPI && a.e.bias && kval) ? static_cast<const int32_t*>(a.e.bias)[kc0 + v] : 0;
                }
                const float elo = (EPI && a.e.relu) ? 0.0f : -127.0f;
                uint8_t* cbrow = ebuf + (kb >> 2) * pitch;  // this block's row of ebuf
#pragma unroll
                for (int f = 0; f < FM; ++f) {
                    const int p = (wm * FM + f) * 32 + lrow;
                    float eres[4] = {0.0f, 0.0f, 0.0f, 0.0f};
                    if constexpr (EPI) {
                        if (a.e.res && kval && p < tile_pix && oh0 * a.OW + p < a.OH * a.OW) {
                            const uint32_t rw = *reinterpret_cast<const uint32_t*>(
                                static_cast<const int8_t*>(a.e.res) + static_cast<long long>(n) * a.y_img +
                                (static_cast<long long>(kc0 >> 2) * a.OH * a.OW + static_cast<long long>(oh0) * a.OW + p) * 4);
#pragma unroll
                            for (int v = 0; v < 4; ++v)
                                eres[v] = static_cast<float>(static_cast<int8_t>((rw >> (8 * v)) & 0xffu));
                        }
                    }
                    uint32_t q[4];
#pragma unroll
                    for (int v = 0; v < 4; ++v) {
                        if constexpr (EPI)
                            q[v] = requant_i8_fused(acc[f][nf][j * 4 + v], eb[v], sc[v], eres[v], elo);
                        else
                            q[v] = requant_i8_bits(acc[f][nf][j * 4 + v], sc[v]);
                    }
                    if (p < tile_pix) *reinterpret_cast<uint32_t*>(cbrow + p * 4) = pack_low_bytes(q[0], q[1], q[2], q[3]);
                }
            }
        }
        __syncthreads();
        {
            // the tile's rows that exist (the last band may be short), its
            // channel blocks (K % 4 == 0): one channel block's tile pixels are
            // contiguous in the output
            const int rows = min(a.TH, a.OH - oh0);
            const int npx = rows * a.OW;
            const int nkb = min(NT, a.K - kt0) / 4;
            const long long plane = static_cast<long long>(a.OH) * a.OW * 4;
            const int pieces = npx / 4;  // 16-byte pieces (4 pixels) per channel block; OW % 4 == 0
            // At most FM * FN pieces per thread (NT / 4 channel blocks x the
            // tile's pixels / 4 pieces over NTHR threads), all issued, the
            // absent ones past the buffer's range (dropped by the hardware),
            // so that later waits count them exactly.  Streaming stores.
            if constexpr (PIPE) {
                const __amdgpu_buffer_rsrc_t yr = __builtin_amdgcn_make_buffer_rsrc(
                    a.y + static_cast<long long>(n) * a.y_img, 0, static_cast<int>(a.y_img), 0x00020000);
                const unsigned ybase = static_cast<unsigned>(oh0 * a.OW * 4);
#pragma unroll
                for (int it = 0; it < FM * FN; ++it) {
                    const int q0 = tid + it * NTHR;
                    const bool okq = q0 < nkb * pieces;
                    const int q = okq ? q0 : 0;
                    const int kb = q / pieces, jj = q - (q / pieces) * pieces;
                    const uint4 v = *reinterpret_cast<const uint4*>(ebuf + kb * pitch + jj * 16);
                    const u32x4_t w = {v.x, v.y, v.z, v.w};
                    __builtin_amdgcn_raw_buffer_store_b128(
                        w, yr, okq ? ybase + static_cast<unsigned>((kt0 / 4 + kb) * plane + jj * 16) : 0x80000000u, 0, 2);
                }
            } else {
                int8_t* yb = a.y + static_cast<long long>(n) * a.y_img + static_cast<long long>(oh0) * a.OW * 4;
                for (int q = tid; q < nkb * pieces; q += NTHR) {
                    const int kb = q / pieces, jj = q - (q / pieces) * pieces;
                    const uint4 v = *reinterpret_cast<const uint4*>(ebuf + kb * pitch + jj * 16);
                    const u32x4_t w = {v.x, v.y, v.z, v.w};
                    __builtin_nontemporal_store(w, reinterpret_cast<u32x4_t*>(yb + (kt0 / 4 + kb) * plane + jj * 16));
                }
            }
        }
        if (more) stage_store(lds + (buf ^ 1) * patch_bytes);
        __syncthreads();
        // the weight ring continues into the next tile, whose tap 0 sits in
        // slot RS % D (RS = 9, D = 3: slot 0 already; RS = 1, D = 2: slot 1,
        // moved here, long after its load was issued)
        if constexpr (RS % D != 0) {
#pragma unroll
            for (int nf = 0; nf < FN; ++nf)
#pragma unroll
                for (int i = 0; i < 2; ++i) wr[0][nf][i] = wr[RS % D][nf][i];
        }
        buf ^= 1;
        n = nn;
        th = thn;
        kt = ktn;
    }
}

}  // namespace st

// ---- host side

int stream_num_configs() { return st::kNumCfgs; }

namespace {

bool stream_geometry(const Prob& p, int sc, st::Args* a, size_t* lds, std::string* why) {
    if (sc < 0 || sc >= st::kNumCfgs) {
        if (why) *why = "implicit GEMM streaming: no such config";
        return false;
    }
    const st::Cfg c = st::kCfgs[sc];
    if (p.dtype != CFWD_I8 || p.layout != CFWD_LAYOUT_NCHWX || p.xb != 4 || p.g != 1) {
        if (why) *why = "implicit GEMM streaming: int8 NCHW4 with groups 1 only";
        return false;
    }
    if (p.cg > 64) {
        if (why) *why = "implicit GEMM streaming: one channel chunk (C <= 64) only";
        return false;
    }
    if (!((p.r == 3 && p.s == 3) || (p.r == 1 && p.s == 1))) {
        if (why) *why = "implicit GEMM streaming: 3x3 or 1x1 filters only";
        return false;
    }
    if (p.w % 4 != 0 || p.ow % 4 != 0 || p.k % 4 != 0) {
        if (why) *why = "implicit GEMM streaming: W, OW and K must be multiples of 4";
        return false;
    }
    if (p.ow > c.pixels()) {
        if (why) *why = "implicit GEMM streaming: an output row is wider than the tile";
        return false;
    }
    if (static_cast<long long>(p.n) * p.x_img >= (1LL << 31) || static_cast<long long>(p.n) * p.y_img >= (1LL << 31)) {
        if (why) *why = "implicit GEMM streaming: tensors must be below 2 GiB";
        return false;
    }
    int TH = std::min(p.oh, c.pixels() / p.ow);
    int PH = 0, PW = 0, ncb = 0, cb0 = 0;
    size_t bytes = 0;
    for (;;) {
        PH = (TH - 1) * p.sh + (p.r - 1) * p.dh + 1;
        PW = (p.ow - 1) * p.sw + (p.s - 1) * p.dw + 1;
        const int iw0 = -p.pw;
        cb0 = (iw0 >= 0) ? iw0 / 4 : -((-iw0 + 3) / 4);
        const int last = iw0 + PW - 1;
        const int cb1 = (last >= 0) ? last / 4 : -((-last + 3) / 4);
        ncb = cb1 - cb0 + 1;
        const long long units = 4LL * PH * ncb;
        bytes = 2 * static_cast<size_t>(PH) * PW * st::PIXB +
                static_cast<size_t>(c.nt() / 4) * (static_cast<size_t>(TH) * p.ow * 4 + 16);
        if (units <= static_cast<long long>(st::SMAXU) * c.threads() && bytes <= ig::kLdsBytes) break;
        if (TH == 1) {
            if (why) *why = "implicit GEMM streaming: one output row's input does not fit this config";
            return false;
        }
        --TH;
    }
    st::Args& g = *a;
    g.N = p.n; g.K = p.k; g.H = p.h; g.W = p.w; g.OH = p.oh; g.OW = p.ow; g.S = p.s;
    g.sh = p.sh; g.sw = p.sw; g.ph = p.ph; g.pw = p.pw; g.dh = p.dh; g.dw = p.dw;
    g.cb_in = p.c / 4 + (p.c % 4 ? 1 : 0);
    g.x_img = p.x_img; g.y_img = p.y_img;
    g.TH = TH; g.PH = PH; g.PW = PW; g.npix = PH * PW; g.ncb = ncb; g.cb0 = cb0;
    g.tiles_h = (p.oh + TH - 1) / TH;
    g.ntk = (p.k + c.nt() - 1) / c.nt();
    const long long nt = static_cast<long long>(p.n) * g.tiles_h * g.ntk;
    if (nt > 0x7fffffffLL) {
        if (why) *why = "implicit GEMM streaming: too many tiles";
        return false;
    }
    g.ntiles = static_cast<int>(nt);
    *lds = bytes;
    return true;
}

template <int WM, int WN, int FM, int FN, int RS, bool EPI>
cfwd_status launch_s(const st::Args& a, size_t lds, hipStream_t stream) {
    auto kern = st::stream_kernel<WM, WN, FM, FN, RS, EPI>;
    static bool attr_done = false;
    if (lds > 65536 && !attr_done) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
        if (e != hipSuccess) return check_hip(e, "hipFuncSetAttribute(stream)");
        attr_done = true;
    }
    // as many workgroups as are resident at once (at least one per XCD)
    int dev = 0, cus = 0, per_cu = 0;
    cfwd_status s = check_hip(hipGetDevice(&dev), "hipGetDevice");
    if (s != CFWD_OK) return s;
    s = check_hip(hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev), "CU count");
    if (s != CFWD_OK) return s;
    s = check_hip(hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void*>(kern),
                                                               WM * WN * 64, lds),
                  "occupancy");
    if (s != CFWD_OK) return s;
    const long long want = static_cast<long long>(std::max(per_cu, 1)) * std::max(cus, 8);
    const unsigned grid = static_cast<unsigned>(std::max<long long>(8, std::min<long long>(want, a.ntiles)));
    kern<<<grid, WM * WN * 64, lds, stream>>>(a);
    return check_hip(hipGetLastError(), "stream_kernel launch");
}

template <bool EPI>
cfwd_status launch_cfg_s(int sc, const st::Args& a, int rs, size_t lds, hipStream_t stream) {
    switch (sc) {
#define CFWD_ST(ID)                                                                                 \
    case ID: {                                                                                      \
        constexpr st::Cfg c = st::kCfgs[ID];                                                        \
        return rs == 9 ? launch_s<c.wm, c.wn, c.fm, c.fn, 9, EPI>(a, lds, stream)                   \
                       : launch_s<c.wm, c.wn, c.fm, c.fn, 1, EPI>(a, lds, stream);                  \
    }
        CFWD_ST(0)
        CFWD_ST(1)
        CFWD_ST(2)
        CFWD_ST(3)
#undef CFWD_ST
        default:
            return set_error(CFWD_ERR_UNSUPPORTED, "implicit GEMM streaming: no such config");
    }
}

}  // namespace

bool stream_supported(const Prob& p, int sc, std::string* why) {
    st::Args a;
    size_t lds;
    return stream_geometry(p, sc, &a, &lds, why);
}

int stream_filter_config(int sc) { return st::kFilterOf[sc]; }

cfwd_status stream_launch(const Prob& p, int sc, const void* x, const void* wp, const float* scale, void* y,
                          const Epi& e, hipStream_t stream) {
    st::Args a;
    size_t lds;
    std::string why;
    if (!stream_geometry(p, sc, &a, &lds, &why)) return set_error(CFWD_ERR_UNSUPPORTED, why);
    a.x = static_cast<const int8_t*>(x);
    a.wp = static_cast<const uint8_t*>(wp);
    a.scale = scale;
    a.y = static_cast<int8_t*>(y);
    a.e = e;
    if (e.bias || e.res || e.relu) return launch_cfg_s<true>(sc, a, p.r * p.s, lds, stream);
    return launch_cfg_s<false>(sc, a, p.r * p.s, lds, stream);
}

}  // namespace cfwd
