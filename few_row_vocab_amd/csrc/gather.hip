// Row gather of a head on gfx950: the draft-vocabulary subset head.  Source: "nemotron:
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
            v[u] = ok && c < row_vecs ? src[c] : zero;
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

}  // namespace

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
