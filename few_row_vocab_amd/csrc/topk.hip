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
// Keys: a logit's order-preserving 32-bit image (0 when not eligible); with the id,
// (image << 32) | (0xffffffff - id) is a 64-bit key that is distinct per entry and whose
// numeric order is exactly the ordering above.
//  * Pass 1, a workgroup per (row, 8192-logit chunk): the chunk's images pass through LDS
//    (coalesced loads, then each thread takes a contiguous run of ids) and a radix select
//    over them (12-bit then 8-bit digits from the top, histograms in
//    LDS, wave scans in DPP, stopping as soon as the boundary digit's bin is taken whole)
//    finds the chunk's k-th value; ties on it go to the lower ids.  The chunk's best
//    min(k, n) entries go to the workspace as 64-bit keys, the rest of its k slots as zeros.
//    Any entry of the row's top-k is in its chunk's top-k.
//  * Pass 2, a workgroup per row: the same radix select over the row's chunk lists (64-bit
//    keys, all distinct, in registers) keeps k; a bitonic sort of the k survivors (in-wave
//    shuffles for strides below 64) puts each in the slot equal to the number that beat it
//    (the pages' rank-by-count order); values come back from the images (zeros, whose
//    sign the image drops, are read from the logits, so -0 stays -0).
// These kernels are short chains of dependent steps, so the design counts round trips:
// every thread issues all of its global loads before using any, keys stay in registers,
// and LDS reads that do not depend on each other are issued together.
#include "dh_internal.h"
#include "launch.h"

namespace dh {
namespace {

constexpr int kRsrcWord3 = 0x00020000;   // gfx9-family raw buffer: 32-bit data format
typedef unsigned int v2u32 __attribute__((ext_vector_type(2)));

constexpr int kBins = 4096;              // 12-bit digits
__host__ __device__ constexpr int digit_bits(int round) { return round < 2 ? 12 : 8; }

__device__ inline uint32_t order_key(float f)
{
    uint32_t u = __float_as_uint(f);
    if (f != f || u == 0xff800000u)
        return 0u;                       // NaN or -inf: not eligible
    if ((u << 1) == 0u)
        u = 0u;                          // -0 and +0 are equal
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ inline uint64_t entry_key(uint32_t image, uint32_t id)
{
    return ((uint64_t)image << 32) | (uint64_t)(0xffffffffu - id);
}

__device__ inline uint32_t key_id(uint64_t key) { return 0xffffffffu - (uint32_t)key; }

// The logit of a key, from its image; a zero's sign is not in the image, so zeros are read
// back from the logits (`src`).
__device__ inline float image_value(uint64_t key, const float *src)
{
    const uint32_t im = (uint32_t)(key >> 32);
    if (im == 0x80000000u)
        return *src;
    return __uint_as_float((im & 0x80000000u) ? (im & 0x7fffffffu) : ~im);
}

// Inclusive prefix sum over the 64 lanes of a wave: shifts within rows of 16 lanes, then
// the row totals broadcast to the later rows (gfx9 DPP row_shr / row_bcast).
__device__ inline uint32_t wave_scan(uint32_t v)
{
    v += __builtin_amdgcn_update_dpp(0u, v, 0x111, 0xf, 0xf, false);   // row_shr:1
    v += __builtin_amdgcn_update_dpp(0u, v, 0x112, 0xf, 0xf, false);   // row_shr:2
    v += __builtin_amdgcn_update_dpp(0u, v, 0x114, 0xf, 0xf, false);   // row_shr:4
    v += __builtin_amdgcn_update_dpp(0u, v, 0x118, 0xf, 0xf, false);   // row_shr:8
    v += __builtin_amdgcn_update_dpp(0u, v, 0x142, 0xa, 0xf, false);   // row_bcast:15
    v += __builtin_amdgcn_update_dpp(0u, v, 0x143, 0xc, 0xf, false);   // row_bcast:31
    return v;
}

template <int NT>
struct Scratch {
    uint32_t hist[2][kBins];                       // double-buffered across rounds
    uint32_t wtot[NT / 64];
    uint32_t digit, above, count;
};

// Exclusive prefix sum of v over the block (in thread order); `total` gets the sum.  The
// wave totals are read with independent loads (one LDS round trip, not one per wave).
template <int NT>
__device__ inline uint32_t block_exclusive(uint32_t v, Scratch<NT> &sh, uint32_t &total)
{
    const uint32_t incl = wave_scan(v);
    if ((threadIdx.x & 63) == 63)
        sh.wtot[threadIdx.x >> 6] = incl;
    __syncthreads();
    uint32_t w[NT / 64];
#pragma unroll
    for (int i = 0; i < NT / 64; i++)
        w[i] = sh.wtot[i];
    const int me = threadIdx.x >> 6;
    uint32_t before = 0, t = 0;
#pragma unroll
    for (int i = 0; i < NT / 64; i++) {
        before += i < me ? w[i] : 0u;
        t += w[i];
    }
    __syncthreads();
    total = t;
    return before + incl - v;
}

template <int NT>
__device__ inline void clear_bins(uint32_t *h)
{
    constexpr int PER = kBins / NT;
#pragma unroll
    for (int j = 0; j < PER; j++)
        h[threadIdx.x * PER + j] = 0;
}

// Radix select over the non-zero keys held in registers (more than k of them in the
// block): returns the prefix P of the boundary bin.  Every key whose determined digits
// exceed P's is taken, and of the `count` keys in the boundary bin (keys x with
// (x & mask) == P) the first `need` in id order are; need == count unless the select ran to
// the last digit (then the bin holds exactly equal keys).  sh.hist[0] must be zero on entry;
// a round clears the other buffer for the next one.
template <typename K, int N, int NT>
__device__ K radix_select(const K (&key)[N], int k, Scratch<NT> &sh, K &mask_out,
                          uint32_t &count, uint32_t &need)
{
    constexpr int BITS = 8 * sizeof(K);
    constexpr int PER = kBins / NT;                 // bins a thread scans
    K prefix = 0, mask = 0;
    uint32_t remaining = (uint32_t)k;
    int shift = BITS, b = 0;
#pragma unroll 1
    for (int round = 0;; round++) {
        const int nb = digit_bits(round);
        shift -= nb;
        const uint32_t dmask = (1u << nb) - 1u;
        uint32_t *h = sh.hist[b];
#pragma unroll
        for (int i = 0; i < N; i++)
            if (key[i] != 0 && (key[i] & mask) == prefix)
                atomicAdd(&h[(uint32_t)(key[i] >> shift) & dmask], 1u);
        clear_bins<NT>(sh.hist[b ^ 1]);
        __syncthreads();
        // thread t owns the PER bins just below kBins - t*PER: a prefix sum over threads is
        // a suffix sum over bins (bins past the digit's range are zero)
        const int top = kBins - 1 - (int)threadIdx.x * PER;
        uint32_t c[PER], mine = 0;
#pragma unroll
        for (int j = 0; j < PER; j++) {
            c[j] = h[top - j];
            mine += c[j];
        }
        uint32_t total;
        uint32_t above = block_exclusive<NT>(mine, sh, total);
#pragma unroll
        for (int j = 0; j < PER; j++) {
            if (above < remaining && remaining <= above + c[j]) {
                sh.digit = top - j;
                sh.above = above;
                sh.count = c[j];
            }
            above += c[j];
        }
        __syncthreads();
        const uint32_t d = sh.digit, ab = sh.above, cnt = sh.count;
        prefix |= (K)d << shift;
        mask |= (K)dmask << shift;
        remaining -= ab;
        b ^= 1;
        if (cnt == remaining || shift == 0) {
            count = cnt;
            need = remaining;
            mask_out = mask;
            __syncthreads();                       // sh.digit and hist reusable
            return prefix;
        }
    }
}

// Pass 1: one workgroup per (chunk, row).
__global__ __launch_bounds__(kP1Threads) void topk_pass1(const float *logits, int64_t V, int k,
                                                         int nchunks, uint64_t *cand)
{
    __shared__ __align__(16) uint32_t img[kChunk];   // the chunk's images, index = id - base
    __shared__ Scratch<kP1Threads> sh;
    constexpr int PER = kChunk / kP1Threads;       // entries a thread owns
    const int r = blockIdx.y, c = blockIdx.x;
    const int64_t base = (int64_t)c * kChunk;
    const int n = V - base < kChunk ? (int)(V - base) : kChunk;

    // coalesced buffer loads bounded by the row, all issued before any is used; entries
    // past V read as 0 and are masked by their index
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(logits + (int64_t)r * V), (short)0, (int)(V * 4), kRsrcWord3);
    uint32_t u[PER];
#pragma unroll
    for (int j = 0; j < PER; j++)
        u[j] = __builtin_amdgcn_raw_buffer_load_b32(
            rs, (uint32_t)(base + j * kP1Threads + threadIdx.x) * 4u, 0, 0);
    uint32_t elig = 0;
#pragma unroll
    for (int j = 0; j < PER; j++) {
        const int i = j * kP1Threads + threadIdx.x;
        const uint32_t x = i < n ? order_key(__uint_as_float(u[j])) : 0u;
        img[i] = x;
        elig += x != 0;
    }
    clear_bins<kP1Threads>(sh.hist[0]);
    uint32_t ne;
    block_exclusive<kP1Threads>(elig, sh, ne);       // its barriers also publish img

    // thread t now takes the contiguous ids [t*PER, t*PER + PER): block scans of per-thread
    // counts then give ranks and output positions in id order
    const int i0 = threadIdx.x * PER;
    uint32_t key[PER];
#pragma unroll
    for (int j = 0; j < PER; j += 4) {
        const uint4 q = *reinterpret_cast<const uint4 *>(&img[i0 + j]);
        key[j] = q.x;
        key[j + 1] = q.y;
        key[j + 2] = q.z;
        key[j + 3] = q.w;
    }

    // kept: image > P, or image == P when the whole boundary bin is taken or when it is
    // among the `need` lowest ids equal to P
    uint32_t P = 1, mask = 0xffffffffu, count = 0, need = 0;
    if (ne > (uint32_t)k)
        P = radix_select<uint32_t, PER, kP1Threads>(key, k, sh, mask, count, need);
    const bool ties = ne > (uint32_t)k && count != need;
    uint32_t eq_before = 0;
    if (ties) {
        uint32_t eq = 0;
#pragma unroll
        for (int j = 0; j < PER; j++)
            eq += key[j] == P;
        uint32_t tot;
        eq_before = block_exclusive<kP1Threads>(eq, sh, tot);
    }
    uint32_t keepmask = 0, eqs = eq_before;
#pragma unroll
    for (int j = 0; j < PER; j++) {
        const uint32_t x = key[j];
        const bool kp = x != 0 && (x > P || (x == P && (!ties || eqs < need)));
        keepmask |= (uint32_t)kp << j;
        eqs += x == P;
    }
    uint32_t nk;
    uint32_t at = block_exclusive<kP1Threads>((uint32_t)__builtin_popcount(keepmask), sh, nk);
    uint64_t *out = cand + ((int64_t)r * nchunks + c) * k;
#pragma unroll
    for (int j = 0; j < PER; j++)
        if (((keepmask >> j) & 1u) && at < (uint32_t)k)   // exactly min(k, ne) are kept
            out[at++] = entry_key(key[j], (uint32_t)(base + i0 + j));
#pragma unroll 1
    for (int s = nk + threadIdx.x; s < k; s += kP1Threads)
        out[s] = 0ull;                               // empty slots
}

// One step of a descending bitonic network on the element x held by slot i: the partner
// is slot i ^ stride, and in a block of `size` whose size bit is clear the lower slot keeps
// the larger key.
__device__ inline uint64_t bitonic_step(uint64_t x, uint64_t y, int i, int size, int stride)
{
    const bool lower = (i & stride) == 0, desc = (i & size) == 0;
    const uint64_t hi = x > y ? x : y, lo = x > y ? y : x;
    return lower == desc ? hi : lo;
}

// Pass 2: one workgroup per row.
__global__ __launch_bounds__(kMergeThreads) void topk_merge(const float *logits, int64_t V,
                                                            int k, int nchunks,
                                                            const uint64_t *cand, int32_t *ids,
                                                            float *vals, int32_t *argmax)
{
    __shared__ Scratch<kMergeThreads> sh;
    __shared__ uint64_t sel[DH_MAX_K];
    constexpr int PER = kMergeSlots / kMergeThreads;
    const int r = blockIdx.x;
    const int slots = nchunks * k;
    const uint64_t *src = cand + (int64_t)r * slots;

    // all loads issued together (bounded buffer loads: slots past the end read as 0)
    const __amdgpu_buffer_rsrc_t ls = __builtin_amdgcn_make_buffer_rsrc(
        (void *)src, (short)0, slots * 8, kRsrcWord3);
    uint64_t key[PER];
#pragma unroll
    for (int j = 0; j < PER; j++) {
        const v2u32 q = __builtin_amdgcn_raw_buffer_load_b64(
            ls, (uint32_t)(j * kMergeThreads + threadIdx.x) * 8u, 0, 0);
        key[j] = ((uint64_t)q.y << 32) | q.x;
    }
    uint32_t nz = 0;
#pragma unroll
    for (int j = 0; j < PER; j++)
        nz += key[j] != 0;
    clear_bins<kMergeThreads>(sh.hist[0]);
    uint32_t n;
    block_exclusive<kMergeThreads>(nz, sh, n);
    const int kk = n < (uint32_t)k ? (int)n : k;
    uint64_t P = 1, mask = ~0ull;                   // n <= k: every non-zero key
    uint32_t count, need;                           // distinct keys: count == need
    if (n > (uint32_t)k)
        P = radix_select<uint64_t, PER, kMergeThreads>(key, k, sh, mask, count, need);

    // the survivors, in any order, to sel[0..kk)
    uint32_t keepmask = 0;
#pragma unroll
    for (int j = 0; j < PER; j++)
        keepmask |= (uint32_t)(key[j] != 0 && key[j] >= P) << j;
    uint32_t tot;
    uint32_t at = block_exclusive<kMergeThreads>((uint32_t)__builtin_popcount(keepmask), sh, tot);
#pragma unroll
    for (int j = 0; j < PER; j++)
        if (((keepmask >> j) & 1u) && at < (uint32_t)kk)   // exactly kk survive
            sel[at++] = key[j];
    __syncthreads();

    // bitonic sort, descending, of np2 >= kk slots (zero keys pad and sort last); keys
    // are distinct, so slot i ends up holding the survivor that exactly i others beat.
    // Strides below 64 stay inside a wave (shuffles); larger ones go through LDS.
    int np2 = 1;
    while (np2 < kk)
        np2 <<= 1;
    const int i = threadIdx.x;
    uint64_t x = i < kk ? sel[i] : 0ull;
#pragma unroll 1
    for (int size = 2; size <= np2; size <<= 1) {
#pragma unroll 1
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            uint64_t y;
            if (stride >= 64) {
                __syncthreads();
                if (i < np2)
                    sel[i] = x;
                __syncthreads();
                y = i < np2 ? sel[i ^ stride] : 0ull;
            } else {
                y = __shfl_xor(x, stride);
            }
            if (i < np2)
                x = bitonic_step(x, y, i, size, stride);
        }
    }

    int32_t *rid = ids + (int64_t)r * k;
    float *rval = vals + (int64_t)r * k;
    if (i < kk) {
        const uint32_t id = key_id(x);
        rid[i] = (int32_t)id;
        rval[i] = image_value(x, logits + (int64_t)r * V + id);
        if (i == 0 && argmax)
            argmax[r] = (int32_t)id;
    }
#pragma unroll 1
    for (int p = kk + i; p < k; p += kMergeThreads) {
        rid[p] = 0;
        rval[p] = -__builtin_inff();
    }
    if (kk == 0 && argmax && i == 0)
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
    w.cnt_off = 0;
    w.bytes = up((size_t)rows * nc * (size_t)k * sizeof(uint64_t));
    return w;
}

hipError_t launch_topk(const float *logits, int rows, int64_t vocab, int k, int32_t *ids,
                       float *vals, int32_t *argmax, void *ws, hipStream_t stream)
{
    const TopkWs w = topk_ws_layout(rows, vocab, k);
    const int nc = (int)topk_chunks(vocab);
    uint64_t *cand = reinterpret_cast<uint64_t *>(static_cast<char *>(ws) + w.val_off);
    hipError_t e = launch(topk_pass1, dim3(nc, rows), dim3(kP1Threads), 0, stream, logits,
                          vocab, k, nc, cand);
    if (e != hipSuccess)
        return e;
    return launch(topk_merge, dim3(rows), dim3(kMergeThreads), 0, stream, logits, vocab, k,
                  nc, (const uint64_t *)cand, ids, vals, argmax);
}

}  // namespace dh
