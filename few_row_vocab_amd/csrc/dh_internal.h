// Internal declarations shared by the library's translation units (kernels and the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dh.h"

namespace dh {

// Vector types the gfx950 builtins take.
typedef __bf16 bf16x8 __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef __bf16 bf16x2 __attribute__((__vector_size__(2 * sizeof(__bf16))));
typedef float f32x4 __attribute__((__vector_size__(4 * sizeof(float))));

constexpr int kWave = 64;

// Launchers: argument checking has been done by the caller (api.hip).  Each returns the
// hipError_t of its launches.
// zero, nzero, zstride: nzero pairs of words, zstride words apart, that the kernel sets to
// zero (the sync lines of the kernels that follow it on the stream), or NULL.
// cut: NULL, or the draft's fused top-k cut (up to 16 rows): each workgroup also leaves, per
// row, the keys of its tiles' logits in the value bins at and above the bin of its m-th
// largest (those strictly above when they would not fit `slots`), and a floor key above
// every key it left out (0 when it left none out), for the merge of topk.h.  The cut is made
// when the launch's grid is at most kCutMaxChunks and grid * slots <= max_keys;
// grid_used (host) receives the grid.
struct GemvCut {
    uint64_t *keys;     // [rows][grid][slots], 0 past a workgroup's cut
    uint64_t *floors;   // [rows][grid]
    int m, slots, max_keys;
};
constexpr int kCutMaxChunks = 1024;
hipError_t launch_gemv(const dh_head &head, const uint16_t *x, int rows, float *logits,
                       hipStream_t stream, uint32_t *zero = nullptr, int nzero = 0,
                       int zstride = 1, const GemvCut *cut = nullptr, int *grid_used = nullptr);
// The same GEMV with an output mode (dh_out_mode): fp32, bf16, or bf16 of residual + sum.
// scratch: optional device memory; with a few tiles and linear_split_bytes of it, the work
// is split over more workgroups with bit-identical results.
hipError_t launch_linear(const dh_head &head, const uint16_t *x, int rows, int mode,
                         const uint16_t *residual, void *out, hipStream_t stream,
                         void *scratch = nullptr, size_t scratch_bytes = 0,
                         uint32_t *zero = nullptr, int nzero = 0, int zstride = 1,
                         const GemvCut *cut = nullptr, int *grid_used = nullptr);
size_t linear_split_bytes(int64_t vocab, int64_t hidden, int rows);
// The scratch dh_linear_ws takes: the few-tile split's partials, or the wide split's.
size_t linear_ws_bytes(int64_t vocab, int64_t hidden, int rows);

// sync: NULL (a second kernel picks the drafts), or zeroed sync lines (ticket lines, then
// best-key lines, `rows` of each, kTicketStride words apart: a top-k workspace's, or
// dh_rescore_sync's buffer): the candidates' last workgroup of a row picks its draft and
// sets the row's two lines back to zero.
hipError_t launch_rescore(const dh_head &dense, const uint16_t *x, int rows,
                          const int32_t *cand_ids, const float *cand_vals, int cand_k,
                          float *exact, int32_t *draft, hipStream_t stream,
                          uint32_t *sync = nullptr);
hipError_t launch_gather_rows(const dh_head &head, const int32_t *ids, int64_t n, void *weight,
                              float *scale, hipStream_t stream);
hipError_t launch_sample(const int32_t *ids, const float *vals, int rows, int k, double T,
                         double top_p, double min_p, uint64_t seed, const int64_t *pos,
                         int32_t *token, int32_t *kept, hipStream_t stream);
// The tiled copy of a row-major head's weight (dh.h, DH_TILED), and its size in bytes.
hipError_t launch_tile_head(const dh_head &head, void *tiled, hipStream_t stream);
size_t tiled_bytes(int format, int64_t vocab, int64_t hidden);
hipError_t launch_quantize(int format, const uint16_t *w, int64_t vocab, int64_t hidden,
                           uint8_t *codes, void *scale, hipStream_t stream);

// The streaming-read probe (dh_stream_read).
hipError_t launch_stream_read(const void *buf, size_t bytes, uint32_t *sink, hipStream_t stream);

// Number of compute units of the current device (cached per device).
int device_cus();

}  // namespace dh
