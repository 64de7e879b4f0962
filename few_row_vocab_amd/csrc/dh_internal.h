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

// Top-k layout: a row is cut into chunks; pass 1 keeps each chunk's best min(k, chunk)
// entries, pass 2 merges a row's lists (chunks * k keys, at most kMergeSlots).  The chunk is
// the smallest of 2048, 4096, 8192 logits whose lists fit: small chunks spread pass 1 over
// more compute units.
constexpr int kMaxChunk = 8192;
constexpr int kP1PerThread = 8;      // logits a pass-1 thread holds
constexpr int kMergeThreads = 1024;
constexpr int kMergeSlots = 16384;   // (262144 / kMaxChunk) * 512

inline int topk_chunk(int64_t vocab, int k)
{
    for (int c = 2048; c < kMaxChunk; c *= 2)
        if ((vocab + c - 1) / c * k <= kMergeSlots)
            return c;
    return kMaxChunk;
}
inline int64_t topk_chunks(int64_t vocab, int k)
{
    const int c = topk_chunk(vocab, k);
    return (vocab + c - 1) / c;
}

// Workspace layout of the top-k (offsets in bytes, each 256-byte aligned): the chunk lists
// of 64-bit keys, [rows][chunks][k], then the chunks' softmax statistics [rows][chunks]
// (float2: the largest eligible logit and the sum of exp(l - it)).
struct TopkWs {
    size_t val_off, id_off, cnt_off, stats_off, bytes;
};
TopkWs topk_ws_layout(int rows, int64_t vocab, int k);

// Launchers: argument checking has been done by the caller (api.cpp).  Each returns the
// hipError_t of its launches.
hipError_t launch_gemv(const dh_head &head, const uint16_t *x, int rows, float *logits,
                       hipStream_t stream);
// The same GEMV with an output mode (dh_out_mode): fp32, bf16, or bf16 of residual + sum.
hipError_t launch_linear(const dh_head &head, const uint16_t *x, int rows, int mode,
                         const uint16_t *residual, void *out, hipStream_t stream);
// idmap: NULL, or the vocabulary id of each logit column (ids and argmax are mapped).
// probs, lse: NULL, or the softmax probability of each kept entry [rows][k] and each row's
// log-sum-exp [rows] (both or neither).
hipError_t launch_topk(const float *logits, int rows, int64_t vocab, int k,
                       const int32_t *idmap, int32_t *ids, float *vals, int32_t *argmax,
                       void *ws, hipStream_t stream, float *probs = nullptr,
                       float *lse = nullptr);

hipError_t launch_rescore(const dh_head &dense, const uint16_t *x, int rows,
                          const int32_t *cand_ids, const float *cand_vals, int cand_k,
                          float *exact, int32_t *draft, hipStream_t stream);
hipError_t launch_gather_rows(const dh_head &head, const int32_t *ids, int64_t n, void *weight,
                              float *scale, hipStream_t stream);
hipError_t launch_quantize(int format, const uint16_t *w, int64_t vocab, int64_t hidden,
                           uint8_t *codes, void *scale, hipStream_t stream);

// Number of compute units of the current device (cached per device).
int device_cus();

}  // namespace dh
