// int8 image stems in NCHW4 (C <= 4, e.g. ResNet's 7x7 stride-2 first layer):
// implicit GEMM with operands loaded straight from global memory (gfx950).
//
// MegEngine inference article, section "Im2col+MatMul": the convolution as a
// matrix product over the im2col matrix.  For a stem the K dimension is
// (r, s, c) with only 4 channels; in NCHW4 the 4 channels of a pixel are one
// 4-byte word, so the S taps of one filter row for one output pixel are S
// consecutive words of one input row.  K is laid out as 8 filter rows x 8
// taps x 4 channels (256 bytes, zero past R, S, C): each 16-byte matrix-core
// operand piece is then 4 consecutive input words, loaded with one 16-byte
// load -- no gather, no LDS staging; only fragments at the image's edges
// shift or zero the words (MegEngine inference article, section "NCHWX": the
// blocked layout that makes the channel vector one aligned word).
//
// Matrix product per 16-pixel fragment (16 consecutive output columns of one
// output row) and 64 output channels: v_mfma_i32_16x16x64_i8 with the
// weights as A (rows = channels) and the pixels as B, so each lane ends with
// 4 consecutive channels of one pixel: one requantised NCHW4 word per store,
// 16 lanes = 64 contiguous bytes.  Persistent waves take FPW fragments at a
// time; the weights of a 64-channel group (4 K steps x 4 tiles x 16 bytes)
// stay in registers, and the next fragments' pixels load during the
// current ones' products and stores.
#include "internal.h"
#include "stem_i8.h"

namespace cfwd {
namespace st8 {

constexpr int NTHR = 256;
constexpr int FPW = 2;  // 16-pixel fragments per wave and unit
constexpr int KG = 64;  // output channels per group

struct Args {
    const uint32_t* x;   // NCHW4 words: [N][H][W] (one channel block)
    const uint4* wp;     // prepared: [group][K step][tile][lane][16 B]
    const float* scale;
    int8_t* y;
    int H, W, K, OH, OW, sh, sw, ph, pw, R;
    int W2, lastrow;     // 2 W; (H - 1) W: word offsets of a row step and of the last row
    unsigned plane4;     // bytes per output channel block (OH OW 4)
    int nsteps;          // ceil(R / 2)
    int ngroups;         // ceil(K / 64)
    int fw;              // fragments per output row: ceil(OW / 16)
    long long nfrag;     // N * OH * fw
    long long y_img;     // bytes per image of y
    Epi e;
};

template <bool EPI>
__global__ __launch_bounds__(NTHR) void stem_kernel(Args a) {
    const int tid = threadIdx.x, lane = tid & 63;
    const int g = lane >> 4, i = lane & 15;
    // Persistent waves, each bound to one 64-channel group whose weights,
    // scales and biases it loads once.  Workgroups are dealt round robin to
    // the 8 XCDs (workgroup b runs on XCD b % 8; the grid is a multiple of
    // 8), so each XCD takes one contiguous eighth of the fragment groups
    // (FPW fragments each), which its waves walk with a stride of the
    // XCD's waves that share the channel group: the input rows then meet
    // in one L2 instead of all eight.
    // The loop body has no branch: the next group's pixels are loaded right
    // after the current products (from a clamped group on the last pass),
    // and dead lanes store out of the buffer's range, which the hardware
    // drops, so the wait before the products covers only those loads.
    // Indices fit 32 bits: the host rejects larger problems.
    const unsigned xcd = blockIdx.x % 8;
    const unsigned lw = (blockIdx.x / 8) * (NTHR / 64) + static_cast<unsigned>(__builtin_amdgcn_readfirstlane(tid >> 6));
    const unsigned ng = static_cast<unsigned>(a.ngroups);
    const unsigned wpg = gridDim.x / 8 * (NTHR / 64) / ng;  // waves per channel group and XCD
    if (lw >= wpg * ng) return;
    const int kg = static_cast<int>(lw % ng);
    const unsigned nfrag = static_cast<unsigned>(a.nfrag);
    const unsigned ngf = (nfrag + FPW - 1) / FPW;
    const unsigned fg_lo = xcd * ngf / 8, fg_hi = (xcd + 1) * ngf / 8;
    if (fg_lo >= fg_hi) return;
    // fragment group fg: fragments FPW fg .. + FPW - 1 (image n, output row
    // oh uniform across the wave; lane i takes output column 16 owf + i)
    auto decode = [&](unsigned fg, int (&n)[FPW], int (&oh)[FPW], int (&ow)[FPW], bool (&live)[FPW])
        __attribute__((always_inline)) {
#pragma unroll
        for (int f = 0; f < FPW; ++f) {
            unsigned fr = fg * FPW + f;
            live[f] = fr < nfrag;
            if (!live[f]) fr = nfrag - 1;
            const unsigned t = fr / static_cast<unsigned>(a.fw);
            const int owf = static_cast<int>(fr - t * static_cast<unsigned>(a.fw));
            const unsigned q = t / static_cast<unsigned>(a.OH);
            oh[f] = static_cast<int>(t - q * static_cast<unsigned>(a.OH));
            n[f] = static_cast<int>(q);
            ow[f] = owf * 16 + i;
            live[f] = live[f] && ow[f] < a.OW;
        }
    };
    // K step t, lane group g: filter row 2t + g / 2, taps 4 (g % 2) .. + 3.
    // Every load is issued from an address clamped into the image (W >= 4):
    // the 4 words at b = clamp(iw0, 0, W - 4).  The fix-up waits until the
    // words are consumed, so the loads stay in flight: lanes whose window
    // leaves the row shift the words by iw0 - b (the same for every filter
    // row) and zero what lies outside; rows outside the image
    // are zeroed (rlo: the fragment's first input row).  Filter rows and
    // taps past R, S and channels past C have zero weights, so what is
    // loaded there does not matter.
    auto load_x = [&](uint4 (&b)[4][FPW], int (&shf)[FPW], int (&rlo)[FPW], const int (&n)[FPW], const int (&oh)[FPW],
                      const int (&ow)[FPW]) __attribute__((always_inline)) {
#pragma unroll
        for (int f = 0; f < FPW; ++f) {
            const int iw0 = ow[f] * a.sw - a.pw + 4 * (g & 1);
            const int bw = min(max(iw0, 0), a.W - 4);
            shf[f] = iw0 - bw;
            rlo[f] = oh[f] * a.sh - a.ph;  // the fragment's first input row (uniform)
            // the fragment's image (n is uniform): 32-bit byte offsets from it
            const char* img = reinterpret_cast<const char*>(a.x + static_cast<long long>(n[f]) * a.H * a.W);
            // word offset of this lane's first row; K step t is 2 t rows
            // further, clamped into the image on the product (W > 0), so one
            // multiply per fragment instead of one per load
            const int row0 = (rlo[f] + (g >> 1)) * a.W;
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const int rw = min(max(row0 + t * a.W2, 0), a.lastrow);
                uint32_t v[4];
                __builtin_memcpy(v, img + static_cast<unsigned>((rw + bw) * 4), 16);
                b[t][f] = make_uint4(v[0], v[1], v[2], v[3]);
            }
        }
    };
    // word e of the result is word e + sh of v, zero outside 0 .. 3; a
    // two-stage barrel shift of selects for |sh| <= 3, all zero when the
    // row is outside the image or |sh| >= 4 (the whole window lies past one
    // end of the row: wide padding, or a late tap of a stride-1 filter at
    // the last output columns)
    auto fix = [](uint4 v, int sh, bool in) __attribute__((always_inline)) -> i32x4 {
        uint32_t x0 = v.x, x1 = v.y, x2 = v.z, x3 = v.w;
        const bool up = sh > 0;
        const int m = up ? sh : -sh;
        if (m & 2) {
            const uint32_t y0 = up ? x2 : 0u, y1 = up ? x3 : 0u, y2 = up ? 0u : x0, y3 = up ? 0u : x1;
            x0 = y0; x1 = y1; x2 = y2; x3 = y3;
        }
        if (m & 1) {
            const uint32_t y0 = up ? x1 : 0u, y1 = up ? x2 : x0, y2 = up ? x3 : x1, y3 = up ? 0u : x2;
            x0 = y0; x1 = y1; x2 = y2; x3 = y3;
        }
        const uint32_t k = (in && m < 4) ? 0xffffffffu : 0u;
        return i32x4{static_cast<int>(x0 & k), static_cast<int>(x1 & k), static_cast<int>(x2 & k),
                     static_cast<int>(x3 & k)};
    };
    // weights [K step][channel tile] and the lane's 16 channels of the group
    // (64 kg + 16 mt + 4 g + v): scale and bias
    uint4 w[4][4];
    float sc[4][4];
    int bi[4][4];
    // byte offset of the lane's channel block 16 kg + 4 mt + g in an image of y
    unsigned cofs[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) cofs[mt] = static_cast<unsigned>(kg * (KG / 4) + 4 * mt + g) * a.plane4;
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
            w[t][mt] = (t < a.nsteps) ? a.wp[((static_cast<long long>(kg) * 4 + t) * 4 + mt) * 64 + lane]
                                      : make_uint4(0, 0, 0, 0);
    int n[FPW], oh[FPW], ow[FPW];
    bool live[FPW];
    uint4 bx[4][FPW];
    int shf[FPW], rlo[FPW];
    unsigned fg = fg_lo + lw / ng;
    decode(min(fg, fg_hi - 1), n, oh, ow, live);
    load_x(bx, shf, rlo, n, oh, ow);
    // Loaded after the first pixels, unconditionally (clamped channel) and
    // kept after them: on entry to the loop, as on its back edge (the
    // stores), other memory operations follow the pixel loads, so the waits
    // before the products never have to drain the stores.
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            // channels past K take channel K - 1's; the padding bytes they
            // give are zeroed after the launch, as for every algorithm
            const int kc = min(kg * KG + 16 * mt + 4 * g + v, a.K - 1);
            sc[mt][v] = a.scale[kc];
            if constexpr (EPI) bi[mt][v] = a.e.bias ? static_cast<const int32_t*>(a.e.bias)[kc] : 0;
        }
    for (; fg < fg_hi; fg += wpg) {
        i32x4 acc[FPW][4];
#pragma unroll
        for (int f = 0; f < FPW; ++f)
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) acc[f][mt] = i32x4{0, 0, 0, 0};
        // interior fragments (the filter's R rows inside the image, no
        // lane's window leaving its row: decided for the whole wave) skip
        // the fix-up
        bool edge[FPW];
#pragma unroll
        for (int f = 0; f < FPW; ++f)
            edge[f] = rlo[f] < 0 || rlo[f] + a.R > a.H || __builtin_amdgcn_ballot_w64(shf[f] != 0) != 0;
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int f = 0; f < FPW; ++f) {
                const i32x4 xv = edge[f] ? fix(bx[t][f], shf[f],
                                               static_cast<unsigned>(rlo[f] + 2 * t + (g >> 1)) < static_cast<unsigned>(a.H))
                                         : __builtin_bit_cast(i32x4, bx[t][f]);
#pragma unroll
                for (int mt = 0; mt < 4; ++mt)
                    acc[f][mt] = __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(i32x4, w[t][mt]), xv,
                                                                      acc[f][mt], 0, 0, 0);
            }
        // this group's pixels, then the next group's loads before the stores
        int sn[FPW], soh[FPW], sow[FPW];
        bool slive[FPW];
#pragma unroll
        for (int f = 0; f < FPW; ++f) {
            sn[f] = n[f];
            soh[f] = oh[f];
            sow[f] = ow[f];
            slive[f] = live[f];
        }
        decode(min(fg + wpg, fg_hi - 1), n, oh, ow, live);
        load_x(bx, shf, rlo, n, oh, ow);
        // D[channel][pixel]: lane holds pixel i of the fragment and channels
        // 64 kg + 16 mt + 4g .. + 3: one NCHW4 word
#pragma unroll
        for (int f = 0; f < FPW; ++f) {
            const unsigned pofs = static_cast<unsigned>(soh[f] * a.OW + sow[f]) * 4u;  // the lane's pixel in a plane
            // the fragment's image of y as a buffer (n is uniform across the
            // wave): offsets at or past y_img are dropped
            const __amdgpu_buffer_rsrc_t ybuf = __builtin_amdgcn_make_buffer_rsrc(
                a.y + static_cast<long long>(sn[f]) * a.y_img, 0, static_cast<int>(a.y_img), 0x00020000);
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) {
                const int k0 = kg * KG + 16 * mt + 4 * g;
                const bool ok = slive[f] && k0 < a.K;
                const unsigned off = cofs[mt] + pofs;
                uint32_t word = 0;
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    uint32_t q;
                    if constexpr (EPI) {
                        const float r = (a.e.res && ok)
                            ? static_cast<float>(static_cast<const int8_t*>(a.e.res)[sn[f] * a.y_img + off + v])
                            : 0.0f;
                        q = requant_i8_fused(acc[f][mt][v], bi[mt][v], sc[mt][v], r, a.e.relu ? 0.0f : -127.0f);
                    } else {
                        q = requant_i8_bits(acc[f][mt][v], sc[mt][v]);
                    }
                    word |= (q & 0xffu) << (8 * v);
                }
                __builtin_amdgcn_raw_buffer_store_b32(word, ybuf, ok ? off : 0x80000000u, 0, 0);
            }
        }
    }
}

// wp[group][t][mt][lane][16 B]: lane (g, i) of tile mt at K step t holds
// channel 64 group + 16 mt + i, filter row 2t + g / 2, taps 4 (g % 2) + e
// (e = 0 .. 3), input channels 0 .. 3 (byte 4 e + c); zero past K, R, S, C
__global__ __launch_bounds__(256) void stem_prepare_kernel(const int8_t* __restrict__ w, int8_t* __restrict__ wp, int K,
                                                           int C, int R, int S, int ngroups) {
    const long long total = static_cast<long long>(ngroups) * 4 * 4 * 64 * 16;
    for (long long idx = blockIdx.x * 256LL + threadIdx.x; idx < total; idx += static_cast<long long>(gridDim.x) * 256) {
        const int byte = static_cast<int>(idx & 15);
        const int lane = static_cast<int>((idx >> 4) & 63);
        const int mt = static_cast<int>((idx >> 10) & 3);
        const int t = static_cast<int>((idx >> 12) & 3);
        const int grp = static_cast<int>(idx >> 14);
        const int g = lane >> 4, i = lane & 15;
        const int k = grp * KG + 16 * mt + i;
        const int r = 2 * t + (g >> 1);
        const int s = 4 * (g & 1) + (byte >> 2);
        const int c = byte & 3;
        int8_t v = 0;
        if (k < K && c < C && r < R && s < S) v = w[((static_cast<long long>(k) * C + c) * R + r) * S + s];
        wp[idx] = v;
    }
}

}  // namespace st8

int stem_i8_num_configs() { return 1; }

bool stem_i8_supported(const Prob& p, int cfg, std::string* why) {
    auto no = [&](const char* m) {
        if (why) *why = m;
        return false;
    };
    if (cfg != 0) return no("implicit GEMM (int8 stem): no such config");
    if (p.dtype != CFWD_I8 || p.layout != CFWD_LAYOUT_NCHWX || p.xb != 4)
        return no("implicit GEMM (int8 stem): int8 NCHW4 only");
    if (p.c > 4 || p.g != 1) return no("implicit GEMM (int8 stem): at most 4 input channels, groups 1");
    if (p.dh != 1 || p.dw != 1) return no("implicit GEMM (int8 stem): dilation 1 only");
    if (p.r > 8 || p.s > 8) return no("implicit GEMM (int8 stem): filters up to 8 x 8");
    if (p.w < 4) return no("implicit GEMM (int8 stem): input rows of at least 4 pixels");
    const long long nfrag = static_cast<long long>(p.n) * p.oh * ((p.ow + 15) / 16);
    // 32-bit indices in the kernel: fragments and (channel group, fragment
    // group) units below 2^28, an image's pixels below 2^30, its output
    // bytes below 2^31
    if (nfrag >= (1LL << 28) || (nfrag + st8::FPW - 1) / st8::FPW * ((p.k + st8::KG - 1) / st8::KG) >= (1LL << 28) ||
        static_cast<long long>(p.h) * p.w > 0x3fffffffLL || p.y_img > 0x7fffffffLL)
        return no("implicit GEMM (int8 stem): too many output fragments");
    return true;
}

size_t stem_i8_filter_bytes(const Prob& p, int cfg) {
    if (!stem_i8_supported(p, cfg, nullptr)) return 0;
    return static_cast<size_t>((p.k + st8::KG - 1) / st8::KG) * 4 * 4 * 64 * 16;
}

cfwd_status stem_i8_prepare(const Prob& p, int cfg, const void* w, void* wp, hipStream_t st) {
    std::string why;
    if (!stem_i8_supported(p, cfg, &why)) return set_error(CFWD_ERR_UNSUPPORTED, why);
    const int ngroups = (p.k + st8::KG - 1) / st8::KG;
    const long long total = static_cast<long long>(ngroups) * 16384;
    st8::stem_prepare_kernel<<<static_cast<unsigned>(std::min<long long>((total + 255) / 256, 4096)), 256, 0, st>>>(
        static_cast<const int8_t*>(w), static_cast<int8_t*>(wp), p.k, p.c, p.r, p.s, ngroups);
    return check_hip(hipGetLastError(), "int8 stem filter prepare launch");
}

cfwd_status stem_i8_launch(const Prob& p, int cfg, const void* x, const void* wp, const float* scale, void* y,
                           const Epi& e, hipStream_t st) {
    std::string why;
    if (!stem_i8_supported(p, cfg, &why)) return set_error(CFWD_ERR_UNSUPPORTED, why);
    if (wp == nullptr) return set_error(CFWD_ERR_WORKSPACE, "implicit GEMM (int8 stem): the prepared filter is required");
    st8::Args a;
    a.x = static_cast<const uint32_t*>(x);
    a.wp = static_cast<const uint4*>(wp);
    a.scale = scale;
    a.y = static_cast<int8_t*>(y);
    a.H = p.h; a.W = p.w; a.K = p.k; a.OH = p.oh; a.OW = p.ow;
    a.W2 = 2 * p.w; a.lastrow = (p.h - 1) * p.w;
    a.plane4 = static_cast<unsigned>(p.oh) * static_cast<unsigned>(p.ow) * 4u;
    a.sh = p.sh; a.sw = p.sw; a.ph = p.ph; a.pw = p.pw; a.R = p.r;
    a.nsteps = (p.r + 1) / 2;
    a.ngroups = (p.k + st8::KG - 1) / st8::KG;
    a.fw = (p.ow + 15) / 16;
    a.nfrag = static_cast<long long>(p.n) * p.oh * a.fw;
    a.y_img = p.y_img;
    a.e = e;
    // persistent grid: as many workgroups as stay resident on every CU (the
    // kernels' register use allows two or three waves per SIMD), never many
    // more than units of work need, a multiple of 8 (one share per XCD),
    // and at least one wave per channel group on each XCD
    const bool epi = e.bias || e.res || e.relu;
    const void* fn = epi ? reinterpret_cast<const void*>(&st8::stem_kernel<true>)
                         : reinterpret_cast<const void*>(&st8::stem_kernel<false>);
    int dev = 0, cus = 256, per_cu = 2;
    if (hipGetDevice(&dev) == hipSuccess) (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, st8::NTHR, 0) != hipSuccess || per_cu < 1) per_cu = 1;
    (void)hipGetLastError();
    constexpr int WPB = st8::NTHR / 64;
    const long long units = (a.nfrag + st8::FPW - 1) / st8::FPW * a.ngroups;
    const long long want = (units + WPB - 1) / WPB;
    const long long least = 8 * ((a.ngroups + WPB - 1) / WPB);
    const long long most = std::max<long long>(8, static_cast<long long>(per_cu) * cus / 8 * 8);
    const unsigned blocks = static_cast<unsigned>(
        std::max<long long>(least, (std::min<long long>(want, most) + 7) / 8 * 8));
    if (epi) st8::stem_kernel<true><<<blocks, st8::NTHR, 0, st>>>(a);
    else st8::stem_kernel<false><<<blocks, st8::NTHR, 0, st>>>(a);
    return check_hip(hipGetLastError(), "int8 stem launch");
}

}  // namespace cfwd
