// Top-k layout and launcher, shared by the top-k kernels and the C ABI.
#pragma once

#include "dh_internal.h"

namespace dh {

// Top-k layout: a row is cut into chunks; pass 1 keeps each chunk's best min(k, chunk)
// entries, pass 2 merges a row's lists (chunks * k keys, at most kMergeSlots).  The chunk is
// the smallest of 2048, 4096, 8192 logits whose lists fit: small chunks spread pass 1 over
// more compute units.  Above 256 kept entries the chunk is 8192: halving the merge's keys
// saved more (measured 3 us at k = 512) than the larger chunks cost pass 1.
constexpr int kMaxChunk = 8192;
constexpr int kP1PerThread = 8;      // logits a pass-1 thread holds
constexpr int kMergeThreads = 1024;
constexpr int kMergeSlots = 16384;   // (262144 / kMaxChunk) * 512

inline int topk_chunk(int64_t vocab, int k)
{
    if (k > 256)
        return kMaxChunk;
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
    size_t keys_off, stats_off, bytes;
};
TopkWs topk_ws_layout(int rows, int64_t vocab, int k);

// idmap: NULL, or the vocabulary id of each logit column (ids and argmax are mapped).
// probs, lse: NULL, or the softmax probability of each kept entry [rows][k] and each row's
// log-sum-exp [rows] (both or neither).
hipError_t launch_topk(const float *logits, int rows, int64_t vocab, int k,
                       const int32_t *idmap, int32_t *ids, float *vals, int32_t *argmax,
                       void *ws, hipStream_t stream, float *probs = nullptr,
                       float *lse = nullptr);

}  // namespace dh
