// Implicit GEMM with a split reduction, int8 NCHW4 (configs after the
// gather form; see kSplitCfgs in igemm_impl.h).
//
// Deep int8 layers with small images (ResNet-18's 14x14 and 7x7 stages) have
// a long reduction (up to 512 channels x 9 taps) and few output pixels: their
// tiles are too few to fill the GPU, and each walks the whole reduction
// alone, waiting on its own loads.  Here the channel chunks of every tile are
// divided among several workgroups.  Each writes its int32 partial tile in
// the output's NCHW4 order; the reduce kernel below adds the partial tiles of
// each output and requantises.  int32 addition is exact, so the result is
// the same bit for bit as a single pass (the accumulator bound 127^2 * C * R
// * S < 2^31 holds for every partial sum as for the whole).  The requant rule
// is the library's: clamp(rne(fp32(acc) * scale[k]), -127, 127).
#include "igemm_impl.h"

namespace cfwd {

namespace {

// One thread per (image, channel block, pixel): the S partial 16-byte pieces
// of its four channels are summed and requantised into one NCHW4 dword.
// Index i runs over [n][channel block][pixel], the layout of both the partial
// tiles and the output, so loads and stores are coalesced.  Channels past K
// take scale 0, which writes the zero bytes NCHW4 keeps in its padding.
__global__ __launch_bounds__(256) void split_reduce_i8(const int4* __restrict__ part, const float* __restrict__ scale,
                                                       uint32_t* __restrict__ y, int n4, int S, int OHW, int KB,
                                                       int K, Epi ep) {
    const int i = static_cast<int>(blockIdx.x) * 256 + static_cast<int>(threadIdx.x);
    if (i >= n4) return;
    int4 acc = part[i];
    for (int s = 1; s < S; ++s) {
        const int4 v = part[static_cast<long long>(s) * n4 + i];
        acc.x += v.x;
        acc.y += v.y;
        acc.z += v.z;
        acc.w += v.w;
    }
    const int kb = (i / OHW) % KB;
    const int k0 = kb * 4;
    float sc[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        const bool ok = k0 + c < K;
        const float v = scale[ok ? k0 + c : 0];  // no branch around the load
        sc[c] = ok ? v : 0.0f;
    }
    if (ep.bias || ep.res || ep.relu) {
        // fused epilogue; channels past K take the last real channel's bias
        // (their scale is 0 and they are zeroed afterwards)
        const long long o = 4LL * i;
        y[i] = pack_low_bytes(requant_i8_epi_bits(acc.x, sc[0], ep, min(k0, K - 1), o),
                              requant_i8_epi_bits(acc.y, sc[1], ep, min(k0 + 1, K - 1), o + 1),
                              requant_i8_epi_bits(acc.z, sc[2], ep, min(k0 + 2, K - 1), o + 2),
                              requant_i8_epi_bits(acc.w, sc[3], ep, min(k0 + 3, K - 1), o + 3));
        return;
    }
    y[i] = pack_low_bytes(requant_i8_bits(acc.x, sc[0]), requant_i8_bits(acc.y, sc[1]),
                          requant_i8_bits(acc.z, sc[2]), requant_i8_bits(acc.w, sc[3]));
}

}  // namespace

cfwd_status igemm_launch_i8_split(int sc, const Prob& p, const ig::Geo& g, int cps, const void* x, const void* wp,
                                  const float* scale, void* y, void* part, const Epi& e, hipStream_t st) {
    using namespace ig;
    const int base = kSplitCfgs[sc].base;
    const int nsplit = kSplitCfgs[sc].splits;
    int32_t* pt = static_cast<int32_t*>(part);
    cfwd_status s = CFWD_OK;
    switch (base) {
#define CFWD_IG_SPLIT(ID)                                                                                        \
    case ID: {                                                                                                   \
        constexpr Cfg c = kCfgs[ID];                                                                             \
        if (g.stg == 1) {                                                                                        \
            if (p.r * p.s == 9)                                                                                  \
                s = launch_one<int8_t, 4, c.wm, c.wn, c.fm, c.fn, 1, c.fr, 9, true>(p, g, x, wp, scale, y, Epi{}, st, cps, \
                                                                                    nsplit, pt);                 \
            else                                                                                                 \
                s = launch_one<int8_t, 4, c.wm, c.wn, c.fm, c.fn, 1, c.fr, 0, true>(p, g, x, wp, scale, y, Epi{}, st, cps, \
                                                                                    nsplit, pt);                 \
        } else if (c.fr == 16 && p.r * p.s == 9) {                                                               \
            s = launch_one<int8_t, 4, c.wm, c.wn, c.fm, c.fn, 0, c.fr, (c.fr == 16 ? 9 : 0), true>(              \
                p, g, x, wp, scale, y, Epi{}, st, cps, nsplit, pt);                                                     \
        } else {                                                                                                 \
            s = launch_one<int8_t, 4, c.wm, c.wn, c.fm, c.fn, 0, c.fr, 0, true>(p, g, x, wp, scale, y, Epi{}, st, cps,  \
                                                                                nsplit, pt);                     \
        }                                                                                                        \
        break;                                                                                                   \
    }
        CFWD_IG_SPLIT(2)
        CFWD_IG_SPLIT(9)
        CFWD_IG_SPLIT(10)
        CFWD_IG_SPLIT(11)
        CFWD_IG_SPLIT(13)
        CFWD_IG_SPLIT(16)
#undef CFWD_IG_SPLIT
        default:
            return set_error(CFWD_ERR_UNSUPPORTED, "implicit GEMM split reduction: no such base config");
    }
    if (s != CFWD_OK) return s;
    const int OHW = p.oh * p.ow;
    const int KB = static_cast<int>(p.y_img / (4LL * OHW));
    const int n4 = static_cast<int>(static_cast<long long>(p.n) * p.y_img / 4);
    split_reduce_i8<<<(n4 + 255) / 256, 256, 0, st>>>(reinterpret_cast<const int4*>(pt), scale,
                                                     static_cast<uint32_t*>(y), n4, nsplit, OHW, KB, p.k, e);
    return check_hip(hipGetLastError(), "split_reduce_i8 launch");
}

}  // namespace cfwd
