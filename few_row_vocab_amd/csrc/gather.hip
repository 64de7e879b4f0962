// Load-time relayouts of a head on gfx950: the row gather of the draft-vocabulary subset
// head, and the tiled copy the GEMV streams fastest.  The row gather's source: "nemotron:
// Super's MTP drafts on the draft vocabulary's FP8 rows while a stream's text is covered,
// same replies", 'What this changes' (the FP8 rows of the draft vocabulary's ids are packed
// into a weight of their own, with the head's scales, and their vocabulary ids go along).
//
// Design: a copy, bound by HBM (2 * n * H bytes for FP8, 4 * n * H for bf16).  One wave per
// output row; each lane moves 16-byte vectors of the row, four in flight.  An id outside
// [0, V) reads nothing and writes a zero row (and a zero row scale).
#include "dh_internal.h"
#include "launch.h"

namespace dh {
namespace {

constexpr int kGatherWaves = 4;
constexpr int kGatherUnroll = 4;

__global__ __launch_bounds__(kGatherWaves * kWave) void gather_rows(
    const uint4 *W, const float *S, int64_t V, int row_vecs, const int32_t *ids, int64_t n,
    uint4 *out, float *out_s)
{
    const int64_t j = (int64_t)blockIdx.x * kGatherWaves + (threadIdx.x >> 6);
    if (j >= n)
        return;
    const int lane = threadIdx.x & 63;
    const int64_t id = ids[j];
    const bool ok = id >= 0 && id < V;
    const uint4 *src = W + (ok ? id : 0) * row_vecs;
    uint4 *dst = out + j * row_vecs;
    const uint4 zero = {0u, 0u, 0u, 0u};
    for (int c0 = 0; c0 < row_vecs; c0 += kGatherUnroll * kWave) {
        uint4 v[kGatherUnroll];
#pragma unroll
        for (int u = 0; u < kGatherUnroll; u++) {
            const int c = c0 + u * kWave + lane;
            v[u] = zero;
            if (ok && c < row_vecs)
                v[u] = src[c];
        }
#pragma unroll
        for (int u = 0; u < kGatherUnroll; u++) {
            const int c = c0 + u * kWave + lane;
            if (c < row_vecs)
                dst[c] = v[u];
        }
    }
    if (out_s && lane == 0)
        out_s[j] = ok ? S[id] : 0.f;
}

// The tiled copy of a row-major head (dh.h, DH_TILED): output unit n (16 bytes) is lane
// l = n % 64 of part q of block b of tile t, i.e. row 16 t + l % 16 from element
// 64 b + 16 (l / 16) + 8 q (bf16; E4M3 has one part of 16 elements).  Writes are contiguous;
// a unit past the head's rows or columns is zero.
__global__ __launch_bounds__(256) void tile_head(const uint4 *W, int64_t V, int H, int nkb,
                                                 int parts, int64_t units, uint4 *out)
{
    const int64_t n = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (n >= units)
        return;
    const int l = (int)(n & 63);
    int64_t rest = n >> 6;
    const int q = (int)(rest % parts);
    rest /= parts;
    const int b = (int)(rest % nkb);
    const int64_t t = rest / nkb;
    const int64_t v = 16 * t + (l & 15);
    const int esz = parts;                                     // bytes of an element
    const int c = 64 * b + 16 * (l >> 4) + 8 * q;              // first element of the unit
    uint4 val = {0u, 0u, 0u, 0u};
    if (v < V && c < H)
        val = W[((int64_t)v * H + c) * esz / 16];
    out[n] = val;
}

}  // namespace

size_t tiled_bytes(int format, int64_t vocab, int64_t hidden)
{
    const int esz = (format & ~DH_TILED) == DH_BF16 ? 2 : 1;
    return (size_t)((vocab + 15) / 16) * (size_t)((hidden + 63) / 64) * 1024u * (size_t)esz;
}

hipError_t launch_tile_head(const dh_head &head, void *tiled, hipStream_t stream)
{
    const int parts = head.format == DH_BF16 ? 2 : 1;
    const int nkb = (int)((head.hidden + 63) / 64);
    const int64_t units = (int64_t)(tiled_bytes(head.format, head.vocab, head.hidden) / 16);
    return launch(tile_head, dim3((unsigned)((units + 255) / 256)), dim3(256), 0, stream,
                  static_cast<const uint4 *>(head.weight), (int64_t)head.vocab,
                  (int)head.hidden, nkb, parts, units, static_cast<uint4 *>(tiled));
}

hipError_t launch_gather_rows(const dh_head &head, const int32_t *ids, int64_t n, void *weight,
                              float *scale, hipStream_t stream)
{
    const int row_bytes = (int)head.hidden * (head.format == DH_BF16 ? 2 : 1);
    const int64_t blocks = (n + kGatherWaves - 1) / kGatherWaves;
    return launch(gather_rows, dim3((unsigned)blocks), dim3(kGatherWaves * kWave), 0, stream,
                  static_cast<const uint4 *>(head.weight),
                  head.format == DH_FP8_ROW ? static_cast<const float *>(head.scale) : nullptr,
                  (int64_t)head.vocab, row_bytes / 16, ids, n, static_cast<uint4 *>(weight),
                  head.format == DH_FP8_ROW ? scale : nullptr);
}

}  // namespace dh
