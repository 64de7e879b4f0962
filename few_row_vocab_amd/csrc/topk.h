// Top-k layout and launcher, shared by the top-k kernel and the C ABI.
#pragma once

#include "dh_internal.h"

namespace dh {

// The merge ranks its kept keys by counting up to kCountMax of them, and above that with a
// wave per 64 survivors (so a merging workgroup has at least k threads).
constexpr int kCountMax = 128;

// Workspace layout of the top-k (offsets in bytes, each 256-byte aligned): the chunks'
// softmax statistics [rows][up to 256 chunks] (float2: the largest eligible logit and the
// sum of exp(l - it), dh_topk_softmax only); then the sync lines, kSyncKinds 256-byte lines a
// row ([kind][row]), each zero when its kernel starts:
//   kind 0: the draft's rescore ticket (the row's candidate workgroups that are done);
//   kind 1: the rescore's best 64-bit key of the row so far.
// Each in a line of its own: rows sharing a line serialize their workgroups' atomics
// (measured up to 8 us at 16 rows).
constexpr int kTicketStride = 64;    // words from one sync line to the next
constexpr int kSyncKinds = 2;
// Then the top-k's cut (GemvCut): the cut keys, [rows][grid][slots], and the floors,
// [rows][grid], sized for a grid of up to min(ntiles, kCutMaxChunks) workgroups.
struct TopkWs {
    size_t stats_off, tickets_off, cut_keys_off, cut_floors_off, bytes;
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
// probs, lse: as launch_topk's, with the chunks' statistics in ws (grid <= 256).
hipError_t launch_cut_merge(const float *logits, int rows, int64_t vocab, int k,
                            const int32_t *idmap, int32_t *ids, float *vals, int32_t *argmax,
                            void *ws, int grid, hipStream_t stream, int slots = 0,
                            int64_t chunk = 0, float *probs = nullptr, float *lse = nullptr);

// The cut pass over the logits' chunks (cut_pass: a workgroup per chunk of a row), then
// cut_merge (a workgroup per row): two launches, no tickets, exact for any input.
// idmap: NULL, or the vocabulary id of each logit column (ids and argmax are mapped).
// probs, lse: NULL, or the softmax probability of each kept entry [rows][k] and each row's
// log-sum-exp [rows] (both or neither): the cut pass also takes each chunk's statistics and
// the merge combines them.
hipError_t launch_topk(const float *logits, int rows, int64_t vocab, int k,
                       const int32_t *idmap, int32_t *ids, float *vals, int32_t *argmax,
                       void *ws, hipStream_t stream, float *probs = nullptr,
                       float *lse = nullptr);

// The sync lines of a workspace (kSyncKinds * rows of them, kTicketStride words apart), for
// the GEMV to zero (two words of each).
uint32_t *topk_tickets(void *ws, int rows, int64_t vocab, int k);
// The chunks' softmax statistics of a workspace, [rows][chunks].
float2 *topk_stats(void *ws, int rows, int64_t vocab, int k);

}  // namespace dh
