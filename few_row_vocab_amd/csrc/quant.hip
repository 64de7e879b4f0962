// Load-time quantization of a bf16 head to FP8 on gfx950.
//
//  per row  ("dsv41 Zig: the TFE draft head (TF_DS_DRAFTER=eagle), off by default", commit
//           notes and 'Update' on FP8 linears): s = float(amax / 448), code = E4M3 RNE of
//           float(w / s).
//  32x32    ("dsv41 metal: the DSpark drafter on an FP8 head, ...", 'FP8 draft head': E4M3
//           codes with an E8M0 scale per 32x32 block, quantized from the bf16 head at load):
//           e = least integer with amax <= 448 * 2^e, byte e + 127 clamped to [0, 254],
//           code = E4M3 RNE of w * 2^-e.
// E4M3 is the OCP format (bias 7, no infinity, 448 the largest magnitude); rounding
// saturates at +-448.  The codes go out row-major, or (format | DH_TILED) straight into the
// GEMV's tiled layout (dh.h), zero past V and H.
#include "dh_internal.h"
#include "launch.h"

namespace dh {
namespace {

// float -> E4M3 code, round to nearest even on the float's bits, saturating.
__device__ inline uint32_t e4m3_rne(float f)
{
    const uint32_t u = __float_as_uint(f);
    const uint32_t sign = (u >> 24) & 0x80u;
    const uint32_t a = u & 0x7fffffffu;
    if (a > 0x7f800000u)
        return sign | 0x7fu;                              // NaN
    if (a >= 0x43e00000u)
        return sign | 0x7eu;                              // |f| >= 448 (and inf)
    if (a < 0x3c800000u) {                                // |f| < 2^-6: quantum 2^-9
        const float q = __uint_as_float(a) * 512.0f;      // exact
        return sign | (uint32_t)__builtin_rintf(q);       // 0..8; 8 is the least normal
    }
    const uint32_t e = (a >> 23) - 120u;                  // E4M3 biased exponent, 1..15
    const uint32_t man = a & 0x7fffffu;
    uint32_t m = man >> 20;
    const uint32_t rest = man & 0xfffffu;
    if (rest > 0x80000u || (rest == 0x80000u && (m & 1u)))
        m++;                                              // m == 8 carries into e
    return sign | ((e << 3) + m);
}

__device__ inline float bf16_value(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// Where code (v, h) goes: row-major, or in the tiled layout (16-row tiles of 64-column
// 1 KiB blocks; lane 16 (h % 64 / 16) + v % 16 holds bytes h % 16 of its 16).
__device__ inline int64_t code_at(int64_t v, int h, int H, int nkb, bool tiled)
{
    if (!tiled)
        return v * H + h;
    return (((v >> 4) * nkb + (h >> 6)) << 10) + (int64_t)(((((h & 63) >> 4) << 4) +
                                                           (int)(v & 15)) << 4) + (h & 15);
}

// e = least integer with amax <= 448 * 2^e = 1.75 * 2^(e+8), clamped to [-127, 127].
__device__ inline int block_exponent(float amax)
{
    if (amax == 0.0f)
        return 0;
    const uint32_t u = __float_as_uint(amax);
    const int ef = (int)((u >> 23) & 0xffu);
    if (ef == 0xff)
        return 127;                                       // infinite maximum
    if (ef == 0)
        return -127;                                      // below 2^-126: 448 * 2^-127 covers it
    const int a = ef - 127;                               // amax = f * 2^a, 1 <= f < 2
    int e = (u & 0x7fffffu) <= 0x600000u ? a - 8 : a - 7; // f <= 1.75 ?
    return e < -127 ? -127 : (e > 127 ? 127 : e);
}

// One workgroup per (256-column panel, 32-row band); lanes 32q..32q+31 of a wave share
// one 32x32 block.  Tiled: the band's rows up to the next multiple of 16 and the columns up
// to the next multiple of 64 past V and H get zero codes.
__global__ __launch_bounds__(256) void quant_block32_kernel(const uint16_t *w, int64_t V,
                                                            int H, uint8_t *codes,
                                                            uint8_t *scales, int tiled)
{
    const int h = blockIdx.x * 256 + threadIdx.x;
    const int64_t v0 = (int64_t)blockIdx.y * 32;
    const int nrows = V - v0 < 32 ? (int)(V - v0) : 32;
    const int nkb = (H + 63) / 64;
    float amax = 0.0f;
    if (h < H)
        for (int i = 0; i < nrows; i++) {
            const float a = __builtin_fabsf(bf16_value(w[(v0 + i) * H + h]));
            amax = a > amax ? a : amax;
        }
    for (int off = 16; off > 0; off >>= 1) {
        const float o = __shfl_xor(amax, off);
        amax = o > amax ? o : amax;
    }
    const int e = block_exponent(amax);
    if (h < H) {
        if ((threadIdx.x & 31) == 0)
            scales[(int64_t)blockIdx.y * (H / 32) + h / 32] = (uint8_t)(e + 127);
        for (int i = 0; i < nrows; i++) {
            const float q = __builtin_ldexpf(bf16_value(w[(v0 + i) * H + h]), -e);
            codes[code_at(v0 + i, h, H, nkb, tiled)] = (uint8_t)e4m3_rne(q);
        }
    }
    if (tiled && h < 64 * nkb) {
        // padding: rows past V up to the tile's end, and (all rows) columns past H
        const int padded = (int)(((V + 15) & ~(int64_t)15) - v0);
        const int prows = padded < 32 ? padded : 32;
        for (int i = h < H ? nrows : 0; i < prows; i++)
            codes[code_at(v0 + i, h, H, nkb, true)] = 0;
    }
}

// One workgroup per row.  Tiled: rows past V up to the next multiple of 16 get zero codes
// (no scale), and every row zero codes past H up to the next multiple of 64.
__global__ __launch_bounds__(256) void quant_row_kernel(const uint16_t *w, int64_t V, int H,
                                                        uint8_t *codes, float *scale,
                                                        int tiled)
{
    __shared__ float part[4];
    const int64_t v = blockIdx.x;
    const int nkb = (H + 63) / 64;
    if (v >= V) {
        for (int h = threadIdx.x; h < 64 * nkb; h += 256)
            codes[code_at(v, h, H, nkb, true)] = 0;
        return;
    }
    const uint16_t *row = w + v * H;
    float amax = 0.0f;
    for (int h = threadIdx.x; h < H; h += 256) {
        const float a = __builtin_fabsf(bf16_value(row[h]));
        amax = a > amax ? a : amax;
    }
    for (int off = 32; off > 0; off >>= 1) {
        const float o = __shfl_xor(amax, off);
        amax = o > amax ? o : amax;
    }
    if ((threadIdx.x & 63) == 0)
        part[threadIdx.x >> 6] = amax;
    __syncthreads();
    amax = part[0];
    for (int i = 1; i < 4; i++)
        amax = part[i] > amax ? part[i] : amax;
    const float s = amax / 448.0f;
    if (threadIdx.x == 0)
        scale[v] = s;
    for (int h = threadIdx.x; h < H; h += 256)
        codes[code_at(v, h, H, nkb, tiled)] =
            s == 0.0f ? 0 : (uint8_t)e4m3_rne(bf16_value(row[h]) / s);
    if (tiled)
        for (int h = H + threadIdx.x; h < 64 * nkb; h += 256)
            codes[code_at(v, h, H, nkb, true)] = 0;
}

}  // namespace

hipError_t launch_quantize(int format, const uint16_t *w, int64_t vocab, int64_t hidden,
                           uint8_t *codes, void *scale, hipStream_t stream)
{
    const int tiled = (format & DH_TILED) ? 1 : 0;
    if ((format & ~DH_TILED) == DH_FP8_BLOCK32) {
        // tiled: the panels reach the last 64-column block (padding columns included)
        const int64_t cols = tiled ? (hidden + 63) / 64 * 64 : hidden;
        const dim3 grid((unsigned)((cols + 255) / 256), (unsigned)((vocab + 31) / 32));
        return launch(quant_block32_kernel, grid, dim3(256), 0, stream, w, vocab, (int)hidden,
                      codes, static_cast<uint8_t *>(scale), tiled);
    }
    const int64_t rows = tiled ? (vocab + 15) / 16 * 16 : vocab;
    return launch(quant_row_kernel, dim3((unsigned)rows), dim3(256), 0, stream, w, vocab,
                  (int)hidden, codes, static_cast<float *>(scale), tiled);
}

}  // namespace dh
