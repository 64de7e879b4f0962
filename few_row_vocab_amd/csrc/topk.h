// Top-k layout and launcher, shared by the top-k kernel and the C ABI.
#pragma once

#include "dh_internal.h"

namespace dh {

// Top-k layout: a row is cut into chunks; a workgroup of nt threads per (row, chunk) keeps
// the chunk's best min(k, chunk) entries (a thread holds `per` of its chunk = nt * per
// logits), and the last workgroup of a row to finish merges the row's lists (nchunks * k
// keys, at most kMergePer a thread).  Measured on MI355X at V = 129,280 (one launch each):
//  * when the call's logits are few (rows * V <= 2^20), 4 logits a thread spread the chunk
//    pass over more compute units (one row, k = 64: 10.4 us against 12.9 with 8);
//  * otherwise 8 (16 rows, k = 64: 12.4 us against 18.2 with 4);
//  * the merge is slow with 16 keys a thread (12.9 us against 10.4 with 8 at one row), so the
//    workgroup is the smallest of 256 (512 with 4 logits a thread), 512 and 1024 threads whose
//    merge holds at most 8 keys a thread; above kCountMax kept entries the merge ranks with a
//    wave per 64 survivors, so the workgroup must also have at least k threads.
// Past those, 1024 threads of 8 logits (chunk 8192: at most 32 chunks of 512, 16 keys a
// thread) always fit.
constexpr int kMaxChunk = 8192;
constexpr int kMergePer = 16;        // keys a thread holds in the merge, at most
constexpr int kCountMax = 128;       // up to this many survivors the merge ranks by counting

struct TopkShape {
    int nt, per, chunk;
    int64_t nchunks;
};

inline TopkShape topk_shape(int rows, int64_t vocab, int k)
{
    const int per = (int64_t)rows * vocab <= ((int64_t)1 << 20) ? 4 : 8;
    for (int nt = per == 4 ? 512 : 256; nt <= 1024; nt *= 2) {
        const int chunk = nt * per;
        const int64_t nc = (vocab + chunk - 1) / chunk;
        if (nc * k <= (int64_t)8 * nt && (k <= kCountMax || nt >= k))
            return TopkShape{nt, per, chunk, nc};
    }
    return TopkShape{1024, 8, kMaxChunk, (vocab + kMaxChunk - 1) / kMaxChunk};
}

// Workspace layout of the top-k (offsets in bytes, each 256-byte aligned): the chunk lists
// of 64-bit keys, [rows][chunks][k]; the chunks' softmax statistics [rows][chunks] (float2:
// the largest eligible logit and the sum of exp(l - it)); then the sync lines, kSyncKinds
// 256-byte lines a row ([kind][row]), each zero when its kernel starts:
//   kind 0: the top-k's ticket (the row's chunks that are done);
//   kind 1: the draft's rescore ticket (the row's candidate workgroups that are done);
//   kind 2: the rescore's best 64-bit key of the row so far.
// Each in a line of its own: rows sharing a line serialize their workgroups' atomics
// (measured up to 8 us at 16 rows).
constexpr int kTicketStride = 64;    // words from one sync line to the next
constexpr int kSyncKinds = 3;
struct TopkWs {
    size_t keys_off, stats_off, tickets_off, bytes;
};
TopkWs topk_ws_layout(int rows, int64_t vocab, int k);

// idmap: NULL, or the vocabulary id of each logit column (ids and argmax are mapped).
// probs, lse: NULL, or the softmax probability of each kept entry [rows][k] and each row's
// log-sum-exp [rows] (both or neither).  tickets_zeroed: the previous kernel on `stream` has
// zeroed the workspace's tickets (the GEMV does, see launch_gemv); otherwise a small kernel
// zeroes them first.
hipError_t launch_topk(const float *logits, int rows, int64_t vocab, int k,
                       const int32_t *idmap, int32_t *ids, float *vals, int32_t *argmax,
                       void *ws, hipStream_t stream, float *probs = nullptr,
                       float *lse = nullptr, bool tickets_zeroed = false);

// The sync lines of a workspace (kSyncKinds * rows of them, kTicketStride words apart), for
// the GEMV to zero (two words of each).
uint32_t *topk_tickets(void *ws, int rows, int64_t vocab, int k);

}  // namespace dh
