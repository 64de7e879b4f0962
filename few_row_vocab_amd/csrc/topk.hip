// Per-row top-k and argmax of fp32 logits on gfx950, exact (comparisons only).
//
// Ordering: entry u beats entry v iff u is eligible and (v is not, or l_u > l_v, or
// l_u == l_v and u < v); NaN and -inf are not eligible, -0 == +0; a row with fewer than k
// eligible logits is padded with (id 0, -inf).  Sources: "dsv41 Zig: the TFE draft head
// (TF_DS_DRAFTER=eagle), off by default" (two_stage commit note and 'Update': top cand_k,
// k in 1..512, a tie at the k-th value to the lower token id; commit notes: the top-1 of a
// vocabulary row split into parts and a join) and "nemotron: Super's MTP drafts on the draft
// vocabulary's FP8 rows ..." (commit note on the few-row top-k: rank by the number of
// entries that beat one, higher score then lower index; picks past the finite scores are
// index 0).
//
// Design: every entry gets a 64-bit key, (order-preserving 32-bit image of the logit) << 32
// | (0xffffffff - id), and 0 when the entry is not eligible.  Eligible keys are distinct and
// their numeric order is exactly the ordering above, so the top-k is "the k largest keys".
//  * Pass 1, a workgroup per (row, 4096-logit chunk): a radix select over the keys held in
//    registers (8-bit digits from the top, LDS histograms, stopping as soon as the digit's
//    bin is taken whole) finds the chunk's k-th largest key; the chunk's best min(k, n)
//    keys go to the workspace.  Any entry of the row's top-k is in its chunk's top-k.
//  * Pass 2, a workgroup per row: the same radix select over the row's chunk lists (held
//    in registers), then each of the k survivors takes the slot equal to the number of
//    survivors that beat it (the pages' rank-by-count, applied only after pruning), and
//    reads its value back from the logits so the original bits (e.g. -0) come out.
#include "dh_internal.h"
#include "launch.h"

namespace dh {
namespace {

__device__ inline uint32_t order_key(float f)
{
    uint32_t u = __float_as_uint(f);
    if (f != f || u == 0xff800000u)
        return 0u;                       // NaN or -inf: not eligible
    if ((u << 1) == 0u)
        u = 0u;                          // -0 and +0 are equal
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ inline uint64_t entry_key(float f, uint32_t id)
{
    const uint32_t k = order_key(f);
    return k ? ((uint64_t)k << 32) | (uint64_t)(0xffffffffu - id) : 0ull;
}

__device__ inline uint32_t key_id(uint64_t key) { return 0xffffffffu - (uint32_t)key; }

__device__ inline uint32_t lanes_below(uint64_t mask)
{
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                     __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

template <int NT>
__device__ inline int block_sum(int v, int *sh)
{
    for (int off = 32; off > 0; off >>= 1)
        v += __shfl_xor(v, off);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (lane == 0)
        sh[wave] = v;
    __syncthreads();
    int t = 0;
    for (int w = 0; w < NT / 64; w++)
        t += sh[w];
    __syncthreads();
    return t;
}

struct SelectShared {
    uint32_t hist[256];
    uint32_t digit, above, count;
};

// The smallest key T such that exactly k of the non-zero keys are >= T.  Requires at least
// k non-zero keys in the block.  All threads of the block must call it.
template <int N, int NT>
__device__ uint64_t radix_select(const uint64_t (&key)[N], int k, SelectShared &sh)
{
    uint64_t prefix = 0, mask = 0;
    uint32_t remaining = (uint32_t)k;
    const int lane = threadIdx.x & 63;
    for (int shift = 56; shift >= 0; shift -= 8) {
        for (int i = threadIdx.x; i < 256; i += NT)
            sh.hist[i] = 0;
        __syncthreads();
#pragma unroll
        for (int i = 0; i < N; i++)
            if (key[i] != 0 && (key[i] & mask) == prefix)
                atomicAdd(&sh.hist[(uint32_t)(key[i] >> shift) & 255u], 1u);
        __syncthreads();
        if (threadIdx.x < 64) {
            // lane l owns bins 4l..4l+3; find the bin d with above(d) < remaining <=
            // above(d) + hist[d], above(d) counting the keys in bins > d
            uint32_t h[4], s = 0;
#pragma unroll
            for (int b = 0; b < 4; b++) {
                h[b] = sh.hist[4 * lane + b];
                s += h[b];
            }
            uint32_t suf = s;   // sum over lanes >= this one
            for (int off = 1; off < 64; off <<= 1) {
                const uint32_t t = __shfl_down(suf, off);
                if (lane + off < 64)
                    suf += t;
            }
            uint32_t cum = suf - s;
#pragma unroll
            for (int b = 3; b >= 0; b--) {
                if (cum < remaining && remaining <= cum + h[b]) {
                    sh.digit = 4 * lane + b;
                    sh.above = cum;
                    sh.count = h[b];
                }
                cum += h[b];
            }
        }
        __syncthreads();
        const uint32_t d = sh.digit, above = sh.above, cnt = sh.count;
        __syncthreads();
        prefix |= (uint64_t)d << shift;
        mask |= (uint64_t)0xff << shift;
        remaining -= above;
        if (cnt == remaining)
            break;                      // the whole bin is taken: keys >= prefix are the set
    }
    return prefix;
}

// Pass 1: one workgroup per (chunk, row).
__global__ __launch_bounds__(kP1Threads) void topk_pass1(const float *logits, int64_t V, int k,
                                                         int nchunks, uint64_t *cand,
                                                         int *cand_cnt)
{
    __shared__ SelectShared sh;
    __shared__ int red[kP1Threads / 64];
    __shared__ uint32_t fill;
    const int r = blockIdx.y, c = blockIdx.x;
    const int64_t base = (int64_t)c * kChunk;
    const float *row = logits + (int64_t)r * V;

    uint64_t key[kP1PerThread];
    int n = 0;
#pragma unroll
    for (int i = 0; i < kP1PerThread; i++) {
        const int64_t e = base + i * kP1Threads + threadIdx.x;
        key[i] = e < V ? entry_key(row[e], (uint32_t)e) : 0ull;
        n += key[i] != 0;
    }
    n = block_sum<kP1Threads>(n, red);
    const uint64_t T = n > k ? radix_select<kP1PerThread, kP1Threads>(key, k, sh) : 1ull;

    if (threadIdx.x == 0)
        fill = 0;
    __syncthreads();
    uint64_t *out = cand + ((int64_t)r * nchunks + c) * k;
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int i = 0; i < kP1PerThread; i++) {
        const bool f = key[i] != 0 && key[i] >= T;
        const uint64_t m = __ballot(f);
        if (m) {
            uint32_t at = 0;
            if (lane == 0)
                at = atomicAdd(&fill, (uint32_t)__popcll(m));
            at = __shfl(at, 0);
            if (f)
                out[at + lanes_below(m)] = key[i];
        }
    }
    if (threadIdx.x == 0)
        cand_cnt[r * nchunks + c] = n < k ? n : k;
}

// Pass 2: one workgroup per row.
__global__ __launch_bounds__(kMergeThreads) void topk_merge(const float *logits, int64_t V,
                                                            int k, int nchunks,
                                                            const uint64_t *cand,
                                                            const int *cand_cnt, int32_t *ids,
                                                            float *vals, int32_t *argmax)
{
    __shared__ SelectShared sh;
    __shared__ int red[kMergeThreads / 64];
    __shared__ uint64_t sel[DH_MAX_K];
    __shared__ uint32_t fill;
    const int r = blockIdx.x;
    const int slots = nchunks * k;
    const int *cnt = cand_cnt + r * nchunks;
    const uint64_t *list = cand + (int64_t)r * slots;

    uint64_t key[kMergePerThread];
    int n = 0;
#pragma unroll
    for (int e = 0; e < kMergePerThread; e++) {
        const int s = e * kMergeThreads + threadIdx.x;
        uint64_t kv = 0;
        if (s < slots) {
            const int c = s / k;
            if (s - c * k < cnt[c])
                kv = list[s];
        }
        key[e] = kv;
        n += kv != 0;
    }
    n = block_sum<kMergeThreads>(n, red);
    const int kk = n < k ? n : k;
    const uint64_t T = n > k ? radix_select<kMergePerThread, kMergeThreads>(key, k, sh) : 1ull;

    if (threadIdx.x == 0)
        fill = 0;
    __syncthreads();
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int e = 0; e < kMergePerThread; e++) {
        const bool f = key[e] != 0 && key[e] >= T;
        const uint64_t m = __ballot(f);
        if (m) {
            uint32_t at = 0;
            if (lane == 0)
                at = atomicAdd(&fill, (uint32_t)__popcll(m));
            at = __shfl(at, 0);
            if (f)
                sel[at + lanes_below(m)] = key[e];
        }
    }
    __syncthreads();

    int32_t *rid = ids + (int64_t)r * k;
    float *rval = vals + (int64_t)r * k;
    for (int i = threadIdx.x; i < kk; i += kMergeThreads) {
        const uint64_t mine = sel[i];
        int pos = 0;
        for (int j = 0; j < kk; j++)
            pos += sel[j] > mine;
        const uint32_t id = key_id(mine);
        rid[pos] = (int32_t)id;
        rval[pos] = logits[(int64_t)r * V + id];
        if (pos == 0 && argmax)
            argmax[r] = (int32_t)id;
    }
    for (int p = kk + threadIdx.x; p < k; p += kMergeThreads) {
        rid[p] = 0;
        rval[p] = -__builtin_inff();
    }
    if (kk == 0 && argmax && threadIdx.x == 0)
        argmax[r] = 0;
}

}  // namespace

TopkWs topk_ws_layout(int rows, int64_t vocab, int k)
{
    auto up = [](size_t b) { return (b + 255) & ~(size_t)255; };
    const size_t nc = (size_t)topk_chunks(vocab);
    TopkWs w;
    w.val_off = 0;   // the chunk lists hold keys that carry both the value and the id
    w.id_off = 0;
    w.cnt_off = up((size_t)rows * nc * (size_t)k * sizeof(uint64_t));
    w.bytes = w.cnt_off + up((size_t)rows * nc * sizeof(int));
    return w;
}

hipError_t launch_topk(const float *logits, int rows, int64_t vocab, int k, int32_t *ids,
                       float *vals, int32_t *argmax, void *ws, hipStream_t stream)
{
    const TopkWs w = topk_ws_layout(rows, vocab, k);
    const int nc = (int)topk_chunks(vocab);
    uint64_t *cand = reinterpret_cast<uint64_t *>(static_cast<char *>(ws) + w.val_off);
    int *cnt = reinterpret_cast<int *>(static_cast<char *>(ws) + w.cnt_off);
    hipError_t e = launch(topk_pass1, dim3(nc, rows), dim3(kP1Threads), 0, stream, logits,
                          vocab, k, nc, cand, cnt);
    if (e != hipSuccess)
        return e;
    return launch(topk_merge, dim3(rows), dim3(kMergeThreads), 0, stream, logits, vocab, k,
                  nc, (const uint64_t *)cand, (const int *)cnt, ids, vals, argmax);
}

}  // namespace dh
