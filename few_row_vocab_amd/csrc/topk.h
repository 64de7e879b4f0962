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
// Then the draft's fused top-k cut (GemvCut): the cut keys, [rows][grid][slots], and the
// floors, [rows][grid], sized for a grid of up to min(ntiles, kCutMaxChunks) workgroups.
struct TopkWs {
    size_t keys_off, stats_off, tickets_off, cut_keys_off, cut_floors_off, bytes;
};
TopkWs topk_ws_layout(int rows, int64_t vocab, int k);

// dh_draft's top-k for up to 16 rows, fused into the GEMV: each GEMV workgroup's tiles are a
// chunk of the row, and the GEMV leaves each chunk's cut (launch_gemv's GemvCut: the keys of
// the value bins at and above the bin of its m-th largest, at most `slots` of them, and a
// floor above every key it left out).  One workgroup per row then merges: the k best of all
// cuts, and the k-th of them, t; a chunk whose floor beats t may hold more keys above t, and
// only then are such chunks' logits read back whole (at most k / m chunks: each holds m keys
// of the k, unless its boundary bin was crowded).  Every key left out of the merge is below
// its chunk's floor, which is at most t, so below k keys of the row: the result is exact.
// m is set so a chunk rarely holds more than m of the row's k best (k / grid of them on
// average, about k / 256 here): m = ceil(L + 4 sqrt(L) + 3) for L = k / 256, at most k.
struct CutShape {
    int m, slots;
};
// With `chunks` chunks a row (the GEMV's about 256 workgroups by default): L = k / chunks.
constexpr int kCutShapeChunks = 256;
CutShape cut_shape(int k, int chunks = kCutShapeChunks);
constexpr int kCutThreads = 1024;    // threads of a merging workgroup
constexpr int kCutMaxFast = 8192 / kCutThreads;   // cut keys a merging thread holds (8192 in all)
// the merge ranks more than kCountMax survivors with a wave per 64 of them
static_assert(kCutThreads >= DH_MAX_K, "a merging workgroup has a wave per 64 of k survivors");
// The cut's part of a workspace (launch_gemv's argument).
GemvCut topk_cut(void *ws, int rows, int64_t vocab, int k);
// The merge of the cuts a GEMV of `grid` workgroups (chunk 0: chunk c is the tiles c + j *
// grid) or the standalone top-k's cut pass (chunk c: the `chunk` entries from c * chunk on)
// left in ws, `slots` keys a chunk (0: cut_shape(k)'s); grid <= kCutMaxChunks, grid * slots
// <= kCutThreads * kCutMaxFast.  logits: the cut logits.  Outputs as launch_topk's.
hipError_t launch_cut_merge(const float *logits, int rows, int64_t vocab, int k,
                            const int32_t *idmap, int32_t *ids, float *vals, int32_t *argmax,
                            void *ws, int grid, hipStream_t stream, int slots = 0,
                            int64_t chunk = 0);

// Without probs: the cut pass over the logits' chunks, then cut_merge (two launches, no
// tickets).  With probs: topk_kernel (one launch, after a small kernel that zeroes the
// tickets unless tickets_zeroed: the previous kernel on `stream` has zeroed them, as the
// GEMV does, see launch_gemv).
// idmap: NULL, or the vocabulary id of each logit column (ids and argmax are mapped).
// probs, lse: NULL, or the softmax probability of each kept entry [rows][k] and each row's
// log-sum-exp [rows] (both or neither).
hipError_t launch_topk(const float *logits, int rows, int64_t vocab, int k,
                       const int32_t *idmap, int32_t *ids, float *vals, int32_t *argmax,
                       void *ws, hipStream_t stream, float *probs = nullptr,
                       float *lse = nullptr, bool tickets_zeroed = false);

// The sync lines of a workspace (kSyncKinds * rows of them, kTicketStride words apart), for
// the GEMV to zero (two words of each).
uint32_t *topk_tickets(void *ws, int rows, int64_t vocab, int k);

}  // namespace dh
