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
// numeric order is exactly the ordering above, so ties need no special case.  Ineligible
// entries get the key 0.
//  * Pass 1, a workgroup per (row, chunk of 2048 to 8192 logits): a radix select over the chunk's keys
//    (most significant byte first, histograms in LDS, stopping as soon as the boundary
//    byte's bin is taken whole) finds the chunk's best min(k, n); they go to the workspace
//    in any order, the rest of the chunk's k slots as zeros.  Any entry of the row's top-k
//    is in its chunk's top-k.
//  * Pass 2, a workgroup per row: the same select over the row's chunk lists keeps k; each
//    survivor's slot is the number of survivors that beat it (the pages' rank-by-count
//    order).  Values come back from the images (zeros, whose sign the image drops, are
//    read from the logits, so -0 stays -0).
// Softmax statistics (STATS, for dh_topk_softmax): pass 1 also writes each chunk's largest
// eligible logit m_c and s_c = sum over its eligible logits of exp(l - m_c) (1 for l == m_c,
// so +inf entries count 1 each); the merge combines them in chunk order into the row's m and
// z = sum_c s_c exp(m_c - m), and gives each kept entry exp(l - m) / z and the row
// log(z) + m.  Sums are in fp32 in a fixed order (deterministic).
// These kernels are short chains of dependent steps, so the design counts barriers and LDS
// round trips: every thread issues all of its global loads before using any, keys stay in
// registers, a select round costs one barrier (every wave scans the round's histogram
// itself), and survivors are placed through an LDS counter (one atomic per wave) rather
// than a block scan.
#include "dh_internal.h"
#include "topk.h"
#include "keys.h"
#include "launch.h"

namespace dh {
namespace {

constexpr int kRsrcWord3 = 0x00020000;   // gfx9-family raw buffer: 32-bit data format
typedef unsigned int v2u32 __attribute__((ext_vector_type(2)));

// Radix select over 64-bit keys by ranges: a round sorts the keys of the current range into
// 256 bins of width 2^shift from its base, the boundary bin becomes the next range (its width
// 2^shift, the next bins 2^(shift - 8) wide), and the select stops as soon as that bin is
// taken whole.  The
// first range is [min, max] of the block's non-zero keys, so the first round spreads the keys
// over the bins even when they share their leading bits (top logits share their exponent).
// Each round has a histogram of its own (all cleared once at the start): after a round's one
// barrier every wave scans the histogram itself (four bins a lane) and reaches the same
// decision.  Eight rounds at most (the first shift is at most 56).
constexpr int kRounds = 8;
constexpr int kHistWords = kRounds * 256;

template <int NT>
struct SelectLds {
    uint32_t hist[kHistWords];
    uint64_t wmin[NT / 64], wmax[NT / 64];         // per-wave extremes of the non-zero keys
    float smax[NT / 64], ssum[NT / 64];            // per-wave softmax statistics (STATS)
    uint32_t fill;                                 // survivors placed so far
};

// exp(l - m) of an eligible l below or at the maximum m; 1 when l == m (also for +inf).
__device__ inline float rel_exp(float l, float m) { return l == m ? 1.0f : expf(l - m); }

__device__ inline float wave_max(float v)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        const float w = __shfl_xor(v, o);
        v = w > v ? w : v;
    }
    return v;
}

// A butterfly over the wave's lanes: a fixed association order, so the sum is reproducible.
__device__ inline float wave_sum(float v)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1)
        v += __shfl_xor(v, o);
    return v;
}

template <int NT>
__device__ inline void clear_select(SelectLds<NT> &sh)
{
    for (int i = threadIdx.x; i < kHistWords; i += NT)
        sh.hist[i] = 0;
    if (threadIdx.x == 0)
        sh.fill = 0;
}

// This wave's extremes to LDS (call before the barrier that follows clear_select).
template <int N, int NT>
__device__ inline void publish_min_max(const uint64_t (&key)[N], SelectLds<NT> &sh)
{
    uint64_t mn = ~0ull, mx = 0;
#pragma unroll
    for (int i = 0; i < N; i++) {
        mn = key[i] != 0 && key[i] < mn ? key[i] : mn;
        mx = key[i] > mx ? key[i] : mx;
    }
    wave_min_max(mn, mx);
    if ((threadIdx.x & 63) == 0) {
        sh.wmin[threadIdx.x >> 6] = mn;
        sh.wmax[threadIdx.x >> 6] = mx;
    }
}

// Selects among the non-zero keys held in registers (all distinct).  Returns P such that
// the keys >= P are exactly the min(k, n) largest, where n (returned in `total`) is the
// number of non-zero keys.  RANGED: the first range is [min, max] of the non-zero keys (call
// publish_min_max before the barrier); otherwise it is the whole key space, i.e. the digits
// are the keys' bytes from the top, which costs no reduction and suits keys whose top byte
// already varies.  Before the call: clear_select (and publish_min_max), a barrier.
template <bool RANGED, int N, int NT>
__device__ uint64_t select_top(const uint64_t (&key)[N], uint32_t k, SelectLds<NT> &sh,
                               uint32_t &total)
{
    uint64_t lo = 0, hi = ~0ull;
    if constexpr (RANGED) {
        lo = ~0ull;
        hi = 0;
#pragma unroll
        for (int w = 0; w < NT / 64; w++) {
            lo = sh.wmin[w] < lo ? sh.wmin[w] : lo;
            hi = sh.wmax[w] > hi ? sh.wmax[w] : hi;
        }
        total = 0;
        if (hi == 0)
            return 1;                              // no non-zero key
    }
    const uint64_t span = hi - lo;
    int shift = span >> 8 ? 64 - __builtin_clzll(span >> 8) : 0;   // span >> shift < 256
    uint64_t base = lo;
    uint32_t rem = k;
    int wshift = 64;                               // the range's width is 2^wshift (64: all)
#pragma unroll 1
    for (int round = 0; round < kRounds; round++) {
        uint32_t *h = sh.hist + 256 * round;
        if constexpr (RANGED) {
#pragma unroll
            for (int i = 0; i < N; i++) {
                const uint64_t off = key[i] - base;
                if (key[i] != 0 && key[i] >= base && (wshift == 64 || (off >> wshift) == 0))
                    atomicAdd(&h[(uint32_t)(off >> shift)], 1u);
            }
        } else {
            // whole key space: the range is the keys sharing base's bits above wshift
            const uint64_t mask = wshift == 64 ? 0ull : ~0ull << wshift;
#pragma unroll
            for (int i = 0; i < N; i++)
                if (key[i] != 0 && (key[i] & mask) == base)
                    atomicAdd(&h[(uint32_t)(key[i] >> shift) & 255u], 1u);
        }
        __syncthreads();
        uint32_t d, above, count;
        const uint32_t t = locate<256>(h, rem, d, above, count);
        if (round == 0) {
            total = t;
            if (t <= k)
                return 1;                          // every non-zero key
        }
        rem -= above;
        base += (uint64_t)d << shift;
        if (count == rem || shift == 0)            // the boundary bin is taken whole
            return base;
        wshift = shift;                            // the boundary bin is the next range
        shift = shift > 8 ? shift - 8 : 0;
    }
    return base;                                   // not reached: shift 0 ends by then
}

// Pass 1: one workgroup of NT threads per (chunk of NT * kP1PerThread logits, row); thread
// t holds entries base + j*NT + t.  STATS: the chunk's (m_c, s_c) to stats[row][chunk].
template <int NT, bool STATS>
__global__ __launch_bounds__(NT) void topk_pass1(const float *logits, int64_t V, int k,
                                                 int nchunks, uint64_t *cand, float2 *stats)
{
    __shared__ __align__(16) SelectLds<NT> sh;
    constexpr int PER = kP1PerThread;
    const int r = blockIdx.y, c = blockIdx.x;
    const int64_t base = (int64_t)c * (NT * PER);

    // coalesced buffer loads bounded by the row, all issued before any is used; entries
    // past V read as 0 and are masked by their index
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(logits + (int64_t)r * V), (short)0, (int)(V * 4), kRsrcWord3);
    uint32_t u[PER];
#pragma unroll
    for (int j = 0; j < PER; j++)
        u[j] = __builtin_amdgcn_raw_buffer_load_b32(
            rs, (uint32_t)(base + j * NT + threadIdx.x) * 4u, 0, 0);
    clear_select<NT>(sh);
    uint64_t key[PER];
#pragma unroll
    for (int j = 0; j < PER; j++) {
        const int64_t id = base + j * NT + threadIdx.x;
        const uint32_t im = id < V ? order_key(__uint_as_float(u[j])) : 0u;
        key[j] = im ? entry_key(im, (uint32_t)id) : 0ull;
    }
    float lmax = -__builtin_inff();
    if constexpr (STATS) {
#pragma unroll
        for (int j = 0; j < PER; j++) {
            const float f = __uint_as_float(u[j]);
            if (key[j] != 0 && f > lmax)
                lmax = f;
        }
        lmax = wave_max(lmax);
        if ((threadIdx.x & 63) == 0)
            sh.smax[threadIdx.x >> 6] = lmax;
    }
    __syncthreads();
    if constexpr (STATS) {
        // the chunk's maximum, then this wave's sum; select_top's first barrier publishes it
        lmax = sh.smax[0];
#pragma unroll
        for (int w = 1; w < NT / 64; w++)
            lmax = sh.smax[w] > lmax ? sh.smax[w] : lmax;
        float s = 0.f;
#pragma unroll
        for (int j = 0; j < PER; j++)
            if (key[j] != 0)
                s += rel_exp(__uint_as_float(u[j]), lmax);
        s = wave_sum(s);
        if ((threadIdx.x & 63) == 0)
            sh.ssum[threadIdx.x >> 6] = s;
    }
    uint32_t n;
    const uint64_t P = select_top<false, PER, NT>(key, (uint32_t)k, sh, n);
    if constexpr (STATS) {
        if (threadIdx.x == 0) {
            float s = 0.f;
            for (int w = 0; w < NT / 64; w++)
                s += sh.ssum[w];
            stats[(int64_t)r * nchunks + c] = float2{lmax, s};
        }
    }
    const uint32_t kept = n < (uint32_t)k ? n : (uint32_t)k;

    // survivors in any order (the merge takes the lists as sets)
    uint32_t mine = 0;
#pragma unroll
    for (int j = 0; j < PER; j++)
        mine += key[j] != 0 && key[j] >= P;
    uint64_t *out = cand + ((int64_t)r * nchunks + c) * k;
    uint32_t at = wave_reserve(mine, &sh.fill);
    if (mine) {
#pragma unroll
        for (int j = 0; j < PER; j++)
            if (key[j] != 0 && key[j] >= P && at < (uint32_t)k)   // exactly `kept` survive
                out[at++] = key[j];
    }
    for (int s = kept + threadIdx.x; s < k; s += NT)
        out[s] = 0ull;                             // empty slots
}

// One step of a descending bitonic network on the key x held by slot i (a lane): the
// partner is slot i ^ stride, and in a block of `size` whose size bit is clear the lower
// slot keeps the larger key.
__device__ inline uint64_t bitonic_step(uint64_t x, uint64_t y, int i, int size, int stride)
{
    const bool lower = (i & stride) == 0, desc = (i & size) == 0;
    const uint64_t hi = x > y ? x : y, lo = x > y ? y : x;
    return lower == desc ? hi : lo;
}

// The key of lane l ^ S, through the cheapest cross-lane path for the stride: DPP quad
// permutes for 1 and 2 (no LDS), ds_swizzle's xor mode within 32 lanes for 4..16, a
// bpermute for 32.
template <int S>
__device__ inline uint32_t lane_xor(uint32_t v)
{
    if constexpr (S == 1)
        return __builtin_amdgcn_update_dpp(0u, v, 0xB1, 0xf, 0xf, false);   // quad_perm 1,0,3,2
    else if constexpr (S == 2)
        return __builtin_amdgcn_update_dpp(0u, v, 0x4E, 0xf, 0xf, false);   // quad_perm 2,3,0,1
    else if constexpr (S <= 16)
        return __builtin_amdgcn_ds_swizzle(v, 0x1F | (S << 10));           // and 31, xor S
    else
        return __shfl_xor(v, S);
}

template <int SIZE, int S>
__device__ inline uint64_t bitonic(uint64_t x, int l)
{
    const uint64_t y = ((uint64_t)lane_xor<S>((uint32_t)(x >> 32)) << 32) |
                       lane_xor<S>((uint32_t)x);
    return bitonic_step(x, y, l, SIZE, S);
}

// Sorts the 64 keys of a wave in descending order (lane 0 the largest).
__device__ inline uint64_t wave_sort_desc(uint64_t x, int l)
{
    x = bitonic<2, 1>(x, l);
    x = bitonic<4, 2>(x, l);
    x = bitonic<4, 1>(x, l);
    x = bitonic<8, 4>(x, l);
    x = bitonic<8, 2>(x, l);
    x = bitonic<8, 1>(x, l);
    x = bitonic<16, 8>(x, l);
    x = bitonic<16, 4>(x, l);
    x = bitonic<16, 2>(x, l);
    x = bitonic<16, 1>(x, l);
    x = bitonic<32, 16>(x, l);
    x = bitonic<32, 8>(x, l);
    x = bitonic<32, 4>(x, l);
    x = bitonic<32, 2>(x, l);
    x = bitonic<32, 1>(x, l);
    x = bitonic<64, 32>(x, l);
    x = bitonic<64, 16>(x, l);
    x = bitonic<64, 8>(x, l);
    x = bitonic<64, 4>(x, l);
    x = bitonic<64, 2>(x, l);
    return bitonic<64, 1>(x, l);
}

// Up to this many survivors the merge ranks by counting; above, by sorted runs of 64.
constexpr int kCountMax = 128;
// Above this k the merge's select ranges over [min, max] of the keys (measured: for k = 1
// the reduction costs more than the rounds it saves).
constexpr int kRangedMinK = 8;

// Pass 2: one workgroup per row; a thread holds PER of the row's nchunks * k list slots
// (PER * kMergeThreads >= nchunks * k).  The lists hold the chunks' top values, which share
// their leading bits, so for more than a few winners the select ranges over [min, max].
// STATS: the row's softmax statistics from the chunks' (m_c, s_c): probs[r][slot] and lse[r].
template <int PER, bool RANGED, bool STATS>
__global__ __launch_bounds__(kMergeThreads) void topk_merge(const float *logits, int64_t V,
                                                            int k, int nchunks,
                                                            const uint64_t *cand,
                                                            const int32_t *idmap, int32_t *ids,
                                                            float *vals, int32_t *argmax,
                                                            const float2 *stats, float *probs,
                                                            float *lse)
{
    __shared__ __align__(16) SelectLds<kMergeThreads> sh;
    __shared__ __align__(16) uint64_t sel[DH_MAX_K];
    __shared__ float row_m, row_z;
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
    clear_select<kMergeThreads>(sh);
    if constexpr (RANGED)
        publish_min_max<PER, kMergeThreads>(key, sh);
    if constexpr (STATS) {
        // wave 0: m = max_c m_c, then z = sum_c s_c exp(m_c - m), chunks c = lane, lane + 64,
        // ... summed in that order per lane, then across lanes by a butterfly
        if (threadIdx.x < 64) {
            const float2 *st = stats + (int64_t)r * nchunks;
            float m = -__builtin_inff();
            for (int c = threadIdx.x; c < nchunks; c += 64)
                m = st[c].x > m ? st[c].x : m;
            m = wave_max(m);
            float z = 0.f;
            for (int c = threadIdx.x; c < nchunks; c += 64)
                if (st[c].y > 0.f)
                    z += st[c].y * rel_exp(st[c].x, m);
            z = wave_sum(z);
            if (threadIdx.x == 0) {
                row_m = m;
                row_z = z;
                lse[r] = z > 0.f ? m + logf(z) : -__builtin_inff();
            }
        }
    }
    __syncthreads();
    uint32_t n;
    const uint64_t P = select_top<RANGED, PER, kMergeThreads>(key, (uint32_t)k, sh, n);
    const int kk = n < (uint32_t)k ? (int)n : k;

    // the survivors, in any order, to sel[0..kk)
    uint32_t mine = 0;
#pragma unroll
    for (int j = 0; j < PER; j++)
        mine += key[j] != 0 && key[j] >= P;
    uint32_t at = wave_reserve(mine, &sh.fill);
    if (mine) {
#pragma unroll
        for (int j = 0; j < PER; j++)
            if (key[j] != 0 && key[j] >= P && at < (uint32_t)kk)   // exactly kk survive
                sel[at++] = key[j];
    }
    __syncthreads();

    // slot of a survivor = the number of survivors that beat it (keys are distinct)
    int32_t *rid = ids + (int64_t)r * k;
    float *rval = vals + (int64_t)r * k;
    const int i = threadIdx.x;
    uint32_t rank = 0;
    uint64_t x = 0;
    if (kk <= kCountMax) {
        // few survivors: count directly
        if (i < kk) {
            x = sel[i];
            int j = 0;
            for (; j + 2 <= kk; j += 2) {
                const uint4 q = *reinterpret_cast<const uint4 *>(&sel[j]);
                rank += (((uint64_t)q.y << 32) | q.x) > x;
                rank += (((uint64_t)q.w << 32) | q.z) > x;
            }
            if (j < kk)
                rank += sel[j] > x;
        }
    } else {
        // many: each wave sorts a run of 64 (descending, zero keys pad and sort last), then
        // a survivor's rank is its place in its run plus, for each other run, the number of
        // that run's keys above it (a binary search)
        const int nruns = (kk + 63) >> 6;
        const int w = i >> 6, l = i & 63;
        if (w < nruns) {
            x = wave_sort_desc(i < kk ? sel[i] : 0ull, l);
        }
        __syncthreads();
        if (w < nruns)
            sel[i] = x;
        __syncthreads();
        if (w < nruns && x != 0) {
            // the searches of all runs advance together (independent LDS reads per step);
            // run q keeps run[0..lo) > x >= run[hi..64), and 7 halvings settle 64 keys
            constexpr int kMaxRuns = DH_MAX_K / 64;
            int lo[kMaxRuns], hi[kMaxRuns];
#pragma unroll
            for (int q = 0; q < kMaxRuns; q++) {
                lo[q] = 0;
                hi[q] = q < nruns && q != w ? 64 : 0;
            }
            // every run's probe is read each step, without a branch, so the step's eight LDS
            // reads are in flight together (a settled or absent run reads a slot it ignores)
#pragma unroll
            for (int step = 0; step < 7; step++) {
                int mid[kMaxRuns];
                uint64_t y[kMaxRuns];
#pragma unroll
                for (int q = 0; q < kMaxRuns; q++) {
                    mid[q] = (lo[q] + hi[q]) >> 1;
                    y[q] = sel[64 * q + (mid[q] & 63)];
                }
#pragma unroll
                for (int q = 0; q < kMaxRuns; q++) {
                    const bool open = lo[q] < hi[q], above = y[q] > x;
                    lo[q] = open && above ? mid[q] + 1 : lo[q];
                    hi[q] = open && !above ? mid[q] : hi[q];
                }
            }
            rank = (uint32_t)l;
#pragma unroll
            for (int q = 0; q < kMaxRuns; q++)
                rank += (uint32_t)lo[q];
        }
    }
    if (x != 0 && rank < (uint32_t)kk) {
        const uint32_t id = key_id(x);
        // a subset head's entry id is vocabulary id idmap[id]
        const int32_t out = idmap ? idmap[id] : (int32_t)id;
        rid[rank] = out;
        const float v = image_value(x, logits + (int64_t)r * V + id);
        rval[rank] = v;
        if constexpr (STATS)
            probs[(int64_t)r * k + rank] = rel_exp(v, row_m) / row_z;
        if (rank == 0 && argmax)
            argmax[r] = out;
    }
    for (int p = kk + i; p < k; p += kMergeThreads) {
        rid[p] = 0;
        rval[p] = -__builtin_inff();
        if constexpr (STATS)
            probs[(int64_t)r * k + p] = 0.f;
    }
    if (kk == 0 && argmax && i == 0)
        argmax[r] = 0;
}

}  // namespace

TopkWs topk_ws_layout(int rows, int64_t vocab, int k)
{
    auto up = [](size_t b) { return (b + 255) & ~(size_t)255; };
    const size_t nc = (size_t)topk_chunks(vocab, k);
    TopkWs w;
    w.keys_off = 0;   // the chunk lists hold keys that carry both the value and the id
    w.stats_off = up((size_t)rows * nc * (size_t)k * sizeof(uint64_t));
    w.bytes = w.stats_off + up((size_t)rows * nc * 2 * sizeof(float));
    return w;
}

template <int PER, bool STATS>
hipError_t launch_merge2(const float *logits, int rows, int64_t vocab, int k, int nc,
                         const uint64_t *cand, const int32_t *idmap, int32_t *ids, float *vals,
                         int32_t *argmax, const float2 *stats, float *probs, float *lse,
                         hipStream_t stream)
{
    if (k > kRangedMinK)
        return launch(topk_merge<PER, true, STATS>, dim3(rows), dim3(kMergeThreads), 0, stream,
                      logits, vocab, k, nc, cand, idmap, ids, vals, argmax, stats, probs, lse);
    return launch(topk_merge<PER, false, STATS>, dim3(rows), dim3(kMergeThreads), 0, stream,
                  logits, vocab, k, nc, cand, idmap, ids, vals, argmax, stats, probs, lse);
}

template <int PER>
hipError_t launch_merge(const float *logits, int rows, int64_t vocab, int k, int nc,
                        const uint64_t *cand, const int32_t *idmap, int32_t *ids, float *vals,
                        int32_t *argmax, const float2 *stats, float *probs, float *lse,
                        hipStream_t stream)
{
    if (probs)
        return launch_merge2<PER, true>(logits, rows, vocab, k, nc, cand, idmap, ids, vals,
                                        argmax, stats, probs, lse, stream);
    return launch_merge2<PER, false>(logits, rows, vocab, k, nc, cand, idmap, ids, vals, argmax,
                                     nullptr, nullptr, nullptr, stream);
}

template <int NT>
hipError_t launch_pass1(const float *logits, int rows, int64_t vocab, int k, int nc,
                        uint64_t *cand, float2 *stats, hipStream_t stream)
{
    const dim3 g1(nc, rows);
    if (stats)
        return launch(topk_pass1<NT, true>, g1, dim3(NT), 0, stream, logits, vocab, k, nc, cand,
                      stats);
    return launch(topk_pass1<NT, false>, g1, dim3(NT), 0, stream, logits, vocab, k, nc, cand,
                  stats);
}

hipError_t launch_topk(const float *logits, int rows, int64_t vocab, int k,
                       const int32_t *idmap, int32_t *ids, float *vals, int32_t *argmax,
                       void *ws, hipStream_t stream, float *probs, float *lse)
{
    const TopkWs w = topk_ws_layout(rows, vocab, k);
    const int chunk = topk_chunk(vocab, k);
    const int nc = (int)topk_chunks(vocab, k);
    uint64_t *cand = reinterpret_cast<uint64_t *>(static_cast<char *>(ws) + w.keys_off);
    float2 *stats = probs ? reinterpret_cast<float2 *>(static_cast<char *>(ws) + w.stats_off)
                          : nullptr;
    hipError_t e;
    switch (chunk) {
    case 2048:
        e = launch_pass1<2048 / kP1PerThread>(logits, rows, vocab, k, nc, cand, stats, stream);
        break;
    case 4096:
        e = launch_pass1<4096 / kP1PerThread>(logits, rows, vocab, k, nc, cand, stats, stream);
        break;
    default:
        e = launch_pass1<8192 / kP1PerThread>(logits, rows, vocab, k, nc, cand, stats, stream);
        break;
    }
    if (e != hipSuccess)
        return e;
    const uint64_t *cc = cand;
    const int64_t slots = (int64_t)nc * k;         // <= kMergeSlots by the chunk choice
    if (slots <= kMergeThreads)
        return launch_merge<1>(logits, rows, vocab, k, nc, cc, idmap, ids, vals, argmax,
                               stats, probs, lse, stream);
    if (slots <= 2 * kMergeThreads)
        return launch_merge<2>(logits, rows, vocab, k, nc, cc, idmap, ids, vals, argmax,
                               stats, probs, lse, stream);
    if (slots <= 4 * kMergeThreads)
        return launch_merge<4>(logits, rows, vocab, k, nc, cc, idmap, ids, vals, argmax,
                               stats, probs, lse, stream);
    if (slots <= 8 * kMergeThreads)
        return launch_merge<8>(logits, rows, vocab, k, nc, cc, idmap, ids, vals, argmax,
                               stats, probs, lse, stream);
    return launch_merge<16>(logits, rows, vocab, k, nc, cc, idmap, ids, vals, argmax,
                            stats, probs, lse, stream);
}

}  // namespace dh
