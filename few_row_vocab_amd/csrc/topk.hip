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
//  * dh_topk, dh_topk_mapped and dh_topk_softmax: the pages' top-1 "in parts and a join",
//    for k keys.  The parts: a cut pass over each row's chunks (cut_pass, a workgroup per
//    chunk of a row; the same cut as the draft's below) keeps each chunk's keys of the value
//    bins at and above the bin of its m-th largest, with a floor above every key it left out.
//    The join: cut_merge, a workgroup per row, selects the k best of the cuts, and re-reads
//    the logits of any chunk whose floor beats the k-th of them, so the result is exact for
//    any input.  Each kept key's slot is the number of kept keys that beat it (the pages'
//    rank-by-count order).  Values come back from the images (zeros, whose sign the image
//    drops, are read from the logits, so -0 stays -0).
//  * dh_draft up to 16 rows fuses the cut pass into the GEMV (topk.h): each GEMV workgroup
//    leaves the cut of its tiles' logits, and cut_merge joins them the same way.
// Softmax statistics (STATS, for dh_topk_softmax): the cut pass also writes each chunk's
// largest eligible logit m_c and s_c = sum over its eligible logits of exp(l - m_c) (1 for
// l == m_c, so +inf entries count 1 each); the merge combines them in chunk order into the
// row's m and z = sum_c s_c exp(m_c - m), and gives each kept entry exp(l - m) / z and the
// row log(z) + m.  Sums are in fp32 in a fixed order (deterministic).
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


// The merge's select over the 64-bit keys a workgroup holds in registers (all distinct, 0
// for an ineligible entry) finds the keys of the min(k, n) largest, n being the number of
// non-zero keys, in two ways:
//  * usually one histogram round over the keys' values, in 256 bins of equal width between
//    the smallest and the largest value (a monotone map, so a higher bin only holds larger
//    values).  Logits spread over such bins; their order-preserving bits do not (the best
//    logits of a row share their exponent, so a first round on the top byte of the bits puts
//    most of them in one bin and serializes its LDS atomics).  The bin holding the k-th key
//    is then resolved exactly: its keys are gathered in LDS and each counts the keys of the
//    bin above it;
//  * select_top, the fallback for a crowded boundary bin (many equal or nearly equal
//    values): a radix select over the keys' bytes from the top, a round per byte, stopping as
//    soon as the boundary byte's bin is taken whole.  Each round has a histogram of its own,
//    and after a round's one barrier every wave scans the histogram itself (four bins a lane)
//    and reaches the same decision.  Eight rounds at most.
constexpr int kRounds = 8;
constexpr int kHistWords = kRounds * 256;
constexpr int kBoundMax = 512;   // keys of a boundary bin resolved by counting (in hist[256..])

template <int NT>
struct SelectLds {
    uint32_t hist[kHistWords];                     // round histograms; [256..) the bin's keys
    uint32_t imin[NT / 64], imax[NT / 64];         // per-wave extremes of the non-zero images
    uint64_t bkey;                                 // the boundary bin's cut
    uint32_t fill, bfill;                          // survivors / boundary keys placed so far
};

// exp(l - m) of an eligible l below or at the maximum m; 1 when l == m (also for +inf).
__device__ __forceinline__ float rel_exp(float l, float m) { return l == m ? 1.0f : expf(l - m); }

__device__ __forceinline__ float wave_max(float v)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        const float w = __shfl_xor(v, o);
        v = w > v ? w : v;
    }
    return v;
}

// A butterfly over the wave's lanes: a fixed association order, so the sum is reproducible.
__device__ __forceinline__ float wave_sum(float v)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1)
        v += __shfl_xor(v, o);
    return v;
}

// Clears what the value-bin round needs (its histogram and the counters); the fallback
// clears the other rounds' histograms itself.
template <int NT>
__device__ __forceinline__ void clear_select(SelectLds<NT> &sh)
{
    for (int i = threadIdx.x; i < 256; i += NT)
        sh.hist[i] = 0;
    if (threadIdx.x == 0) {
        sh.fill = 0;
        sh.bfill = 0;
    }
}

// This wave's extremes of the non-zero images to LDS (call before the barrier that follows
// clear_select).
template <int N, int NT>
__device__ __forceinline__ void publish_range(const uint64_t (&key)[N], SelectLds<NT> &sh)
{
    uint32_t mn = ~0u, mx = 0;
#pragma unroll
    for (int i = 0; i < N; i++) {
        const uint32_t im = (uint32_t)(key[i] >> 32);
        mn = im != 0 && im < mn ? im : mn;
        mx = im > mx ? im : mx;
    }
    wave_min_max32(mn, mx);
    if ((threadIdx.x & 63) == 0) {
        sh.imin[threadIdx.x >> 6] = mn;
        sh.imax[threadIdx.x >> 6] = mx;
    }
}

// The number of keys of list[0..n) above x, with several LDS reads in flight.
__device__ __forceinline__ uint32_t count_above(const uint64_t *list, int n, uint64_t x)
{
    uint32_t c = 0;
    int j = 0;
    for (; j + 8 <= n; j += 8) {
        uint4 q[4];
#pragma unroll
        for (int t = 0; t < 4; t++)
            q[t] = *reinterpret_cast<const uint4 *>(&list[j + 2 * t]);
#pragma unroll
        for (int t = 0; t < 4; t++) {
            c += (((uint64_t)q[t].y << 32) | q[t].x) > x;
            c += (((uint64_t)q[t].w << 32) | q[t].z) > x;
        }
    }
    for (; j < n; j++)
        c += list[j] > x;
    return c;
}

// Radix select (the fallback; see above) among the non-zero keys i with inc(i).  Returns P
// such that those keys >= P are exactly the min(k, n) largest of them; n in `total`.
// Before the call: the whole histogram cleared, a barrier.
template <int N, int NT, typename Inc>
__device__ __forceinline__ uint64_t select_top(const uint64_t (&key)[N], uint32_t k, SelectLds<NT> &sh,
                               uint32_t &total, Inc inc)
{
    int shift = 56;
    uint64_t base = 0;
    uint32_t rem = k;
    int wshift = 64;                               // the range: keys sharing base above wshift
#pragma unroll 1
    for (int round = 0; round < kRounds; round++) {
        uint32_t *h = sh.hist + 256 * round;
        const uint64_t mask = wshift == 64 ? 0ull : ~0ull << wshift;
#pragma unroll
        for (int i = 0; i < N; i++)
            if (key[i] != 0 && inc(i) && (key[i] & mask) == base)
                atomicAdd(&h[(uint32_t)(key[i] >> shift) & 255u], 1u);
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
        shift -= 8;
    }
    return base;                                   // not reached: shift 0 ends by then
}

// The outcome of the value-bin round: the survivors are the non-zero keys whose bin is above
// d, or is d with a key >= P (rem of them); when not binned, every non-zero key.  Unless
// crowded (the fallback ran), hist[0..256) still holds every bin's count of non-zero keys.
struct Cut {
    bool binned, crowded;
    uint32_t d, rem;
    uint64_t P;
};

__device__ __forceinline__ bool survives(const Cut &c, uint64_t key, uint32_t bin)
{
    return key != 0 && (!c.binned || bin > c.d || (bin == c.d && key >= c.P));
}


// One step of a descending bitonic network on the key x held by slot i (a lane): the
// partner is slot i ^ stride, and in a block of `size` whose size bit is clear the lower
// slot keeps the larger key.
__device__ __forceinline__ uint64_t bitonic_step(uint64_t x, uint64_t y, int i, int size, int stride)
{
    const bool lower = (i & stride) == 0, desc = (i & size) == 0;
    const uint64_t hi = x > y ? x : y, lo = x > y ? y : x;
    return lower == desc ? hi : lo;
}

// The key of lane l ^ S, through the cheapest cross-lane path for the stride: DPP quad
// permutes for 1 and 2 (no LDS), ds_swizzle's xor mode within 32 lanes for 4..16, a
// bpermute for 32.
template <int S>
__device__ __forceinline__ uint32_t lane_xor(uint32_t v)
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
__device__ __forceinline__ uint64_t bitonic(uint64_t x, int l)
{
    const uint64_t y = ((uint64_t)lane_xor<S>((uint32_t)(x >> 32)) << 32) |
                       lane_xor<S>((uint32_t)x);
    return bitonic_step(x, y, l, SIZE, S);
}

// Sorts the 64 keys of a wave in descending order (lane 0 the largest).
__device__ __forceinline__ uint64_t wave_sort_desc(uint64_t x, int l)
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

// The merge's select, select_sorted: the value-bin round that also puts the survivors in
// order.  The histogram's atomics return each key's index among its bin's keys; bin b's
// survivors then take the slots [start[b], start[b] + s(b)) of the output, s(b) being the
// bin's count above the boundary bin d and rem in it (start: a suffix sum over the bins).  A
// survivor of a bin above d goes to start[b] + its index, and the final pass counts the keys
// of its bin above it; the survivors of bin d are picked by ranking its keys against each
// other (the exact resolution of the boundary bin above), and that rank is already their
// place.  Bins are narrow, so the final counts are short.  start and the bin of each slot
// live in the histogram words past the boundary keys.
constexpr int kStartOff = 256 + 2 * kBoundMax;
constexpr int kBinOfOff = kStartOff + 256;
constexpr uint32_t kPlaced = 0xffffffffu;   // a slot's bin when its key is already in order
static_assert(kBinOfOff + DH_MAX_K <= kHistWords, "the merge's slots fit the histogram words");

// One wave: start[] of every bin (a suffix sum over the bins, as locate's lanes hold them).
__device__ __forceinline__ void bin_starts(const uint32_t *h, const Cut &c, uint32_t *start)
{
    const int lo = 256 - 4 * ((threadIdx.x & 63) + 1);   // this lane's four bins
    uint32_t s[4], sum = 0;
#pragma unroll
    for (int j = 0; j < 4; j++) {
        const uint32_t b = (uint32_t)(lo + j);
        s[j] = !c.binned || b > c.d ? h[b] : b == c.d ? c.rem : 0u;
        sum += s[j];
    }
    uint32_t run = wave_scan(sum) - sum;           // survivors in the bins above this lane's
#pragma unroll
    for (int j = 3; j >= 0; j--) {
        start[lo + j] = run;
        run += s[j];
    }
}

// The number of keys of list[lo..lo + n) above x (8-byte reads: a segment may start at any
// slot), several in flight.
__device__ __forceinline__ uint32_t count_above_at(const uint64_t *list, uint32_t lo,
                                                   uint32_t n, uint64_t x)
{
    uint32_t c = 0, j = 0;
    for (; j + 4 <= n; j += 4) {
        uint64_t y[4];
#pragma unroll
        for (int t = 0; t < 4; t++)
            y[t] = list[lo + j + t];
#pragma unroll
        for (int t = 0; t < 4; t++)
            c += y[t] > x;
    }
    for (; j < n; j++)
        c += list[lo + j] > x;
    return c;
}

// Before the call: clear_select, publish_range, a barrier.  Returns the number of survivors
// kk, written to sel[0..kk) with each slot's bin (or kPlaced) in hist[kBinOfOff + slot]; or
// -1 when the boundary bin is crowded, with c and bin[] set for the caller's fallback (and
// nothing placed).
template <int N, int NT>
__device__ __forceinline__ int select_sorted(const uint64_t (&key)[N], uint32_t k,
                                             SelectLds<NT> &sh, uint64_t *sel, Cut &c,
                                             uint32_t (&bin)[N])
{
    uint32_t mn = ~0u, mx = 0;
#pragma unroll
    for (int w = 0; w < NT / 64; w++) {
        mn = sh.imin[w] < mn ? sh.imin[w] : mn;
        mx = sh.imax[w] > mx ? sh.imax[w] : mx;
    }
    c = Cut{false, false, 0u, 0u, 1ull};
#pragma unroll
    for (int i = 0; i < N; i++)
        bin[i] = 0;
    if (mx == 0)
        return 0;                                  // no eligible entry
    const float lo = image_float(mn);              // the value bins
    const float scale = 256.0f / (image_float(mx) - lo);
    uint32_t *h = sh.hist;
    uint32_t idx[N];
#pragma unroll
    for (int i = 0; i < N; i++) {
        bin[i] = (uint32_t)fminf((image_float((uint32_t)(key[i] >> 32)) - lo) * scale, 255.0f);
        idx[i] = key[i] != 0 ? atomicAdd(&h[bin[i]], 1u) : 0u;
    }
    __syncthreads();
    uint32_t d, above, count;
    const uint32_t total = locate<256>(h, k, d, above, count);
    bool pick = false;                             // bin d's survivors picked through the list
    if (total > k) {
        c.binned = true;
        c.d = d;
        c.rem = k - above;
        if (count > c.rem) {
            if (count > (uint32_t)kBoundMax || count > (uint32_t)NT) {
                c.crowded = true;
                return -1;
            }
            pick = true;
        }
    }
    uint32_t *start = sh.hist + kStartOff, *binof = sh.hist + kBinOfOff;
    uint64_t *list = reinterpret_cast<uint64_t *>(sh.hist + 256);
    if (threadIdx.x < 64)
        bin_starts(h, c, start);
    if (pick) {
        uint32_t mine = 0;
#pragma unroll
        for (int i = 0; i < N; i++)
            mine += key[i] != 0 && bin[i] == d;
        uint32_t at = wave_reserve(mine, &sh.bfill);
        if (mine) {
#pragma unroll
            for (int i = 0; i < N; i++)
                if (key[i] != 0 && bin[i] == d)
                    list[at++] = key[i];
        }
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < N; i++)
        if (key[i] != 0 && (!c.binned || bin[i] > d || (bin[i] == d && !pick))) {
            const uint32_t s = start[bin[i]] + idx[i];
            sel[s] = key[i];
            binof[s] = bin[i];
        }
    if (pick && threadIdx.x < count) {
        const uint64_t x = list[threadIdx.x];
        const uint32_t rk = count_above(list, (int)count, x);
        if (rk < c.rem) {
            sel[start[d] + rk] = x;
            binof[start[d] + rk] = kPlaced;
        }
    }
    __syncthreads();
    return total < k ? (int)total : (int)k;
}

// LDS of the merge beyond the select's: the survivors, and the row's softmax statistics.
struct MergeLds {
    uint64_t sel[DH_MAX_K];
    float row_m, row_z;
};

// The select of a merge: keeps the min(k, n) largest of the non-zero keys the workgroup holds
// in registers (MPER a thread, distinct) and ranks them.  Returns kk = min(k, n); this
// thread's survivor x (0 when it has none) and its rank (the number of survivors that beat
// it, so the slot of x in the descending order).  Before the call the select's LDS may be
// reused freely (the call clears what it needs; ml.sel is its output space); after it, a
// barrier before the LDS is reused.
template <int MPER, int NT>
__device__ __forceinline__ int select_rank(const uint64_t (&key)[MPER], int k, SelectLds<NT> &sh,
                                           MergeLds &ml, uint64_t &x, uint32_t &rank)
{
    uint64_t *sel = ml.sel;
    const int i = threadIdx.x;
    clear_select<NT>(sh);
    publish_range<MPER, NT>(key, sh);
    __syncthreads();
    uint32_t bin[MPER];
    Cut cut;
    int kk = select_sorted<MPER, NT>(key, (uint32_t)k, sh, sel, cut, bin);
    x = 0;
    rank = 0;
    if (kk >= 0) {
        // the survivors sit in their bins' slots: a key of the boundary bin is in its place,
        // one of a bin above it adds the keys of its bin that beat it (keys are distinct)
        if (i < kk) {
            x = sel[i];
            const uint32_t b = sh.hist[kBinOfOff + i];
            rank = (uint32_t)i;
            if (b != kPlaced) {
                const uint32_t s0 = sh.hist[kStartOff + b];
                rank = s0 + count_above_at(sel, s0, sh.hist[b], x);
            }
        }
        return kk;
    }
    // a crowded boundary bin (many equal or nearly equal values): the radix select among its
    // keys, then the survivors ranked among themselves
    kk = k;
    __syncthreads();
    for (int j = threadIdx.x; j < kHistWords; j += NT)
        sh.hist[j] = 0;
    __syncthreads();
    uint32_t n2;
    cut.P = select_top<MPER, NT>(key, cut.rem, sh, n2, [&](int j) { return bin[j] == cut.d; });
    // the survivors, in any order, to sel[0..kk)
    uint32_t mine = 0;
#pragma unroll
    for (int j = 0; j < MPER; j++)
        mine += survives(cut, key[j], bin[j]);
    uint32_t at = wave_reserve(mine, &sh.fill);
    if (mine) {
#pragma unroll
        for (int j = 0; j < MPER; j++)
            if (survives(cut, key[j], bin[j]) && at < (uint32_t)kk)   // exactly kk survive
                sel[at++] = key[j];
    }
    __syncthreads();

    // slot of a survivor = the number of survivors that beat it (keys are distinct)
    if (kk <= kCountMax) {
        // few survivors: count directly
        if (i < kk) {
            x = sel[i];
            rank = count_above(sel, kk, x);
        }
    } else {
        // many: each wave sorts a run of 64 (descending, zero keys pad and sort last), then a
        // survivor's rank is its place in its run plus, for each other run, the number of
        // that run's keys above it (a binary search); the workgroup has a wave per run
        const int nruns = (kk + 63) >> 6;
        const int w = i >> 6, l = i & 63;
        uint64_t y0 = 0;
        if (w < nruns)
            y0 = wave_sort_desc(i < kk ? sel[i] : 0ull, l);
        __syncthreads();
        if (w < nruns)
            sel[i] = y0;
        __syncthreads();
        if (w < nruns && y0 != 0) {
            // the searches of all runs advance together (independent LDS reads per step);
            // run q keeps run[0..lo) > y0 >= run[hi..64), and 7 halvings settle 64 keys
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
                    const bool open = lo[q] < hi[q], above = y[q] > y0;
                    lo[q] = open && above ? mid[q] + 1 : lo[q];
                    hi[q] = open && !above ? mid[q] : hi[q];
                }
            }
            uint32_t rk = (uint32_t)l;
#pragma unroll
            for (int q = 0; q < kMaxRuns; q++)
                rk += (uint32_t)lo[q];
            if (rk < (uint32_t)kk) {
                x = y0;
                rank = rk;
            }
        }
    }
    return kk;
}

// The outputs of row r for a ranked survivor: its id (through idmap) and value at slot rank,
// and the argmax from rank 0.  STATS: its softmax probability from ml.row_m and ml.row_z.
template <bool STATS>
__device__ __forceinline__ void emit_survivor(uint64_t x, uint32_t rank, const float *lrow,
                                              const int32_t *idmap, int32_t *rid, float *rval,
                                              float *rprob, int32_t *argmax, int r,
                                              const MergeLds &ml)
{
    const uint32_t id = key_id(x);
    // a subset head's entry id is vocabulary id idmap[id]
    const int32_t out = idmap ? idmap[id] : (int32_t)id;
    rid[rank] = out;
    const float v = image_value(x, lrow + id);
    rval[rank] = v;
    if constexpr (STATS)
        rprob[rank] = rel_exp(v, ml.row_m) / ml.row_z;
    if (rank == 0 && argmax)
        argmax[r] = out;
}

// The slots of row r past its kk survivors: id 0, value -inf (probability 0); argmax 0 when
// the row has no eligible entry.
template <bool STATS>
__device__ __forceinline__ void emit_padding(int kk, int k, int32_t *rid, float *rval,
                                             float *rprob, int32_t *argmax, int r)
{
    for (int p = kk + (int)threadIdx.x; p < k; p += blockDim.x) {
        rid[p] = 0;
        rval[p] = -__builtin_inff();
        if constexpr (STATS)
            rprob[p] = 0.f;
    }
    if (kk == 0 && argmax && threadIdx.x == 0)
        argmax[r] = 0;
}

// The merge of the GEMV's cuts (topk.h, dh_draft's fused top-k).
struct CutArgs {
    const float *logits;    // [rows][V], as the GEMV wrote them
    int64_t V, ntiles;      // ntiles: 16-row tiles of the head
    int k, grid, slots;     // grid: the GEMV's workgroups (the chunks)
    int64_t chunk;          // 0: chunk c is tiles c + j * grid; else entries [c chunk, +chunk)
    const uint64_t *keys;   // [rows][grid][slots]
    const uint64_t *floors; // [rows][grid]
    const int32_t *idmap;
    int32_t *ids;
    float *vals;
    int32_t *argmax;
    const float2 *stats;    // STATS: the chunks' (m_c, s_c), [rows][grid]
    float *probs, *lse;     // STATS: [rows][k], [rows]
};
constexpr int kCutPass = 16;   // keys a thread holds in a pass over the re-read chunks
constexpr int kStatsMaxChunks = 256;   // STATS: chunks a row, at most (cut_pass's grid)

struct CutLds {
    uint64_t run[DH_MAX_K];          // the best k of the passes so far, by rank
    uint64_t t;                      // the k-th best key of the cuts (0: fewer than k)
    uint32_t nfail;
    uint8_t failed[kCutMaxChunks];   // chunk c's floor beats t
    uint16_t faillist[kCutMaxChunks];
};

// The row's softmax statistics from its chunks' (m_c, s_c), by wave 0: m = max_c m_c, then
// z = sum_c s_c exp(m_c - m) over the chunks c = lane + 64 j of each lane in j order, then
// across the lanes by a fixed butterfly, so the sums are reproducible.  m and z go to ml (for
// the probabilities; the select's first barrier publishes them), log-sum-exp m + log z to lse.
template <int J>
__device__ __forceinline__ void row_stats(const float2 *st, int nchunks, float *lse, MergeLds &ml)
{
    float cm[J], cs[J];
#pragma unroll
    for (int j = 0; j < J; j++) {
        const int c = (int)threadIdx.x + 64 * j;
        const float2 v = c < nchunks ? st[c] : float2{-__builtin_inff(), 0.f};
        cm[j] = v.x;
        cs[j] = v.y;
    }
    float m = -__builtin_inff();
#pragma unroll
    for (int j = 0; j < J; j++)
        m = cm[j] > m ? cm[j] : m;
    m = wave_max(m);
    float z = 0.f;
#pragma unroll
    for (int j = 0; j < J; j++)
        if (cs[j] > 0.f)
            z += cs[j] * rel_exp(cm[j], m);
    z = wave_sum(z);
    if (threadIdx.x == 0) {
        ml.row_m = m;
        ml.row_z = z;
        *lse = z > 0.f ? m + logf(z) : -__builtin_inff();
    }
}

// One workgroup per row: the k best of the row's cuts (MF keys a thread), the floors checked
// against the k-th of them, and when a chunk's floor beats it, passes over the other chunks'
// cuts and those chunks' logits (read back whole), each pass keeping the k best so far.
// STATS: the row's softmax statistics as well (the chunks' (m_c, s_c) from cut_pass), each
// kept entry's probability and the row's log-sum-exp.
template <int MF, bool STATS>
__global__ __launch_bounds__(kCutThreads) void cut_merge(CutArgs a)
{
    constexpr int NT = kCutThreads;
    __shared__ __align__(16) SelectLds<NT> sh;
    __shared__ __align__(16) MergeLds ml;
    __shared__ CutLds cl;
    const int r = blockIdx.x, tid = threadIdx.x;
    const int nfast = a.grid * a.slots;
    const uint64_t *src = a.keys + (int64_t)r * nfast;
    // the GEMV before this kernel has ended, so plain loads see its cuts; bounded buffer
    // loads, all issued together (slots past the cuts read as 0)
    const __amdgpu_buffer_rsrc_t ls = __builtin_amdgcn_make_buffer_rsrc(
        (void *)src, (short)0, nfast * 8, kRsrcWord3);
    uint64_t key[MF];
#pragma unroll
    for (int j = 0; j < MF; j++) {
        const v2u32 q = __builtin_amdgcn_raw_buffer_load_b64(
            ls, (uint32_t)(j * NT + tid) * 8u, 0, 0);
        key[j] = ((uint64_t)q.y << 32) | q.x;
    }
    const uint64_t fl = tid < a.grid ? a.floors[(int64_t)r * a.grid + tid] : 0ull;
    if (tid == 0) {
        cl.nfail = 0;
        cl.t = 0;
    }
    if constexpr (STATS)
        if (tid < kWave)
            row_stats<kStatsMaxChunks / kWave>(a.stats + (int64_t)r * a.grid, a.grid, a.lse + r,
                                               ml);
    uint64_t x;
    uint32_t rank;
    int kk = select_rank<MF, NT>(key, a.k, sh, ml, x, rank);
    if (kk == a.k && x != 0 && rank == (uint32_t)a.k - 1u)
        cl.t = x;
    __syncthreads();
    const bool fail = tid < a.grid && fl > cl.t;
    if (tid < a.grid)
        cl.failed[tid] = fail;
    if (fail)
        cl.faillist[atomicAdd(&cl.nfail, 1u)] = (uint16_t)tid;
    __syncthreads();
    const uint32_t nf = cl.nfail;
    const float *lrow = a.logits + (int64_t)r * a.V;
    int32_t *rid = a.ids + (int64_t)r * a.k;
    float *rval = a.vals + (int64_t)r * a.k;
    if (nf != 0) {
        // the stream of the passes: the cuts of the chunks that stand, then every entry of
        // the chunks that fell (chunk c: tiles c + j * grid, j < per, or the `chunk` entries
        // from c * chunk); at most 8192 + 1024 * 1024 items, so 32-bit indices
        const uint32_t per = (uint32_t)((a.ntiles + a.grid - 1) / a.grid);
        const uint32_t C = a.chunk ? (uint32_t)a.chunk : per * 16u;
        const uint32_t total = (uint32_t)nfast + nf * C;
        auto item = [&](uint32_t q) -> uint64_t {
            if (q < (uint32_t)nfast)
                return cl.failed[q / (uint32_t)a.slots] ? 0ull : src[q];
            const uint32_t e2 = q - (uint32_t)nfast;
            const uint32_t f = e2 / C, e = e2 - f * C;
            const int64_t tile = (int64_t)cl.faillist[f] + (int64_t)(e >> 4) * a.grid;
            const int64_t v =
                a.chunk ? (int64_t)cl.faillist[f] * a.chunk + e : tile * 16 + (e & 15);
            if ((!a.chunk && tile >= a.ntiles) || v >= a.V)
                return 0ull;
            const uint32_t im = order_key(lrow[v]);
            return im ? entry_key(im, (uint32_t)v) : 0ull;
        };
        int nrun = 0;
        uint32_t q0 = 0;
        for (;;) {
            uint64_t key2[kCutPass];
#pragma unroll
            for (int j = 0; j < kCutPass; j++) {
                const int u = j * NT + tid;
                const uint32_t q = q0 + (uint32_t)(u - nrun);
                key2[j] = u < nrun ? cl.run[u] : q < total ? item(q) : 0ull;
            }
            q0 += (uint32_t)(kCutPass * NT - nrun);
            kk = select_rank<kCutPass, NT>(key2, a.k, sh, ml, x, rank);
            if (q0 >= total)
                break;
            if (x != 0)
                cl.run[rank] = x;
            nrun = kk;
            __syncthreads();
        }
    }
    float *rprob = STATS ? a.probs + (int64_t)r * a.k : nullptr;
    if (x != 0)
        emit_survivor<STATS>(x, rank, lrow, a.idmap, rid, rval, rprob, a.argmax, r, ml);
    emit_padding<STATS>(kk, a.k, rid, rval, rprob, a.argmax, r);
}

// The standalone top-k's cut (dh_topk and dh_topk_mapped without softmax statistics): the
// work of the GEMV's fused cut, on logits already in memory.  Workgroup (c, r) takes row r's
// chunk c -- the `chunk` entries from c * chunk on -- and cuts it as the GEMV does (256 value
// bins over the chunk's range of eligible images, d the bin of the m-th largest key; the keys
// of bins >= d, or of bins > d when those would not fit the slots; the floor the smallest key
// cut, 0 when none was left out).  cut_merge then merges the cuts and re-reads any chunk
// whose floor beats the row's k-th key, so the result is exact for any input.  A thread
// holds PER entries (thread t takes entries t + 256 u of the chunk), all loaded before any
// is used.  (Chunks of the GEMV's layout -- every grid-th 16-entry tile -- read 64-byte
// pieces: 8.2 us for the pass at 16 rows, against 6.6 us with contiguous chunks.)
struct CutPassArgs {
    const float *logits;    // [rows][V]
    int64_t V, chunk;       // chunk: entries a chunk
    int m, slots;
    uint64_t *keys;         // [rows][grid][slots]
    uint64_t *floors;       // [rows][grid]
    float2 *stats;          // STATS: [rows][grid]
};
constexpr int kCutPassThreads = 256;   // one histogram bin a thread (512 measured slower)
static_assert(kCutPassThreads == 256, "a thread clears one of the 256 bins");
constexpr int kCutPassMaxPer = 16;    // entries a thread holds, at most
constexpr int kCutPassMaxGrid = 256;  // chunks a row: 1024 / rows within these bounds (fewer
constexpr int kCutPassMinGrid = 64;   // when the row has fewer tiles)
static_assert(kCutPassMaxGrid <= kStatsMaxChunks, "the merge reads every chunk's statistics");

// STATS: the chunk's largest eligible logit m_c and s_c = the sum of exp(l - m_c) over its
// eligible logits (a thread's entries in order, then the wave's butterfly, then the waves in
// order) to stats[r][c]; (-inf, 0) for a chunk with no eligible logit.
template <int PER, bool STATS>
__global__ __launch_bounds__(kCutPassThreads) void cut_pass(CutPassArgs a)
{
    constexpr int NW = kCutPassThreads / kWave;
    __shared__ __align__(16) uint32_t hist[256];
    __shared__ uint32_t wmn[NW], wmx[NW];
    __shared__ float wlm[NW], wls[NW];   // STATS: per-wave largest logit, then sum
    __shared__ uint32_t cnt;
    __shared__ unsigned long long gfloor;
    const int c = blockIdx.x, r = blockIdx.y, tid = threadIdx.x;
    const int G = gridDim.x;
    const float *lrow = a.logits + (int64_t)r * a.V;
    const int64_t c0 = (int64_t)c * a.chunk;
    const int64_t c1 = c0 + a.chunk < a.V ? c0 + a.chunk : a.V;   // the chunk's end
    auto entry = [&](int u) -> int64_t { return c0 + u * kCutPassThreads + tid; };
    float l[PER];
#pragma unroll
    for (int u = 0; u < PER; u++) {
        const int64_t v = entry(u);
        l[u] = v < c1 ? lrow[v] : __builtin_nanf("");
    }
    hist[tid] = 0;   // 256 threads, 256 bins
    if (tid == 0) {
        cnt = 0;
        gfloor = ~0ull;
    }
    // 1: the chunk's range of eligible images
    uint32_t im[PER];
    uint32_t mn = ~0u, mx = 0;
#pragma unroll
    for (int u = 0; u < PER; u++) {
        im[u] = order_key(l[u]);
        mn = im[u] != 0 && im[u] < mn ? im[u] : mn;
        mx = im[u] > mx ? im[u] : mx;
    }
    wave_min_max32(mn, mx);
    float lmax = -__builtin_inff();
    if constexpr (STATS) {
#pragma unroll
        for (int u = 0; u < PER; u++)
            lmax = im[u] != 0 && l[u] > lmax ? l[u] : lmax;
        lmax = wave_max(lmax);
    }
    if ((tid & 63) == 0) {
        wmn[tid >> 6] = mn;
        wmx[tid >> 6] = mx;
        if constexpr (STATS)
            wlm[tid >> 6] = lmax;
    }
    __syncthreads();
#pragma unroll
    for (int w = 0; w < NW; w++) {
        mn = wmn[w] < mn ? wmn[w] : mn;
        mx = wmx[w] > mx ? wmx[w] : mx;
        if constexpr (STATS)
            lmax = wlm[w] > lmax ? wlm[w] : lmax;
    }
    uint64_t *out = a.keys + ((int64_t)r * G + c) * a.slots;
    uint64_t *floor = a.floors + (int64_t)r * G + c;
    if (mx == 0) {   // no eligible entry (the same for the whole workgroup)
        for (int q = tid; q < a.slots; q += kCutPassThreads)
            out[q] = 0;
        if (tid == 0) {
            *floor = 0;
            if constexpr (STATS)
                a.stats[(int64_t)r * G + c] = float2{-__builtin_inff(), 0.f};
        }
        return;
    }
    if constexpr (STATS) {
        float sum = 0.f;
#pragma unroll
        for (int u = 0; u < PER; u++)
            if (im[u] != 0)
                sum += rel_exp(l[u], lmax);
        sum = wave_sum(sum);
        if ((tid & 63) == 0)
            wls[tid >> 6] = sum;   // read after the histogram's barrier
    }
    // 2: the histogram (the select's bin map; a NaN product, from a zero or infinite width,
    // goes to 255)
    const float lo = image_float(mn);
    const float scale = 256.0f / (image_float(mx) - lo);
    auto bin_of = [&](uint32_t x) -> uint32_t {
        return (uint32_t)fminf((image_float(x) - lo) * scale, 255.0f);
    };
#pragma unroll
    for (int u = 0; u < PER; u++)
        if (im[u] != 0)
            atomicAdd(&hist[bin_of(im[u])], 1u);
    __syncthreads();
    if constexpr (STATS)
        if (tid == 0) {
            float sum = 0.f;
#pragma unroll
            for (int w = 0; w < NW; w++)
                sum += wls[w];
            a.stats[(int64_t)r * G + c] = float2{lmax, sum};
        }
    // 3: the cut (every key when at most m, bins >= d, or bins > d) to the slots
    uint32_t d, above, count;
    const uint32_t total = locate<256>(hist, (uint32_t)a.m, d, above, count);
    bool all = total <= (uint32_t)a.m;
    uint32_t dmin = 0;
    if (!all) {
        dmin = above + count <= (uint32_t)a.slots ? d : d + 1;
        all = dmin == d && above + count == total;
    }
#pragma unroll
    for (int u = 0; u < PER; u++) {
        if (im[u] != 0 && (all || bin_of(im[u]) >= dmin)) {
            const uint64_t key = entry_key(im[u], (uint32_t)entry(u));
            out[atomicAdd(&cnt, 1u)] = key;
            atomicMin(&gfloor, (unsigned long long)key);
        }
    }
    __syncthreads();
    // 4: zeros after the cut; the floor
    for (int q = (int)cnt + tid; q < a.slots; q += kCutPassThreads)
        out[q] = 0;
    if (tid == 0)
        *floor = all ? 0ull : gfloor;
}

}  // namespace

CutShape cut_shape(int k, int chunks)
{
    const double L = (double)k / chunks;
    int m = (int)ceil(L + 4.0 * sqrt(L) + 3.0);
    m = m > k ? k : m < 1 ? 1 : m;
    return CutShape{m, m + (m / 2 > 4 ? m / 2 : 4)};
}

TopkWs topk_ws_layout(int rows, int64_t vocab, int k)
{
    auto up = [](size_t b) { return (b + 255) & ~(size_t)255; };
    TopkWs w;
    w.stats_off = 0;
    w.tickets_off = up((size_t)rows * kStatsMaxChunks * sizeof(float2));
    const int64_t ntiles = (vocab + 15) / 16;
    const size_t gcap = (size_t)(ntiles < kCutMaxChunks ? ntiles : kCutMaxChunks);
    w.cut_keys_off =
        w.tickets_off + up((size_t)kSyncKinds * rows * kTicketStride * sizeof(uint32_t));
    // a row's cuts: those of up to gcap GEMV workgroups, or of the standalone top-k's chunks
    // (at most the merge's kCutThreads * kCutMaxFast keys)
    size_t per_row = gcap * (size_t)cut_shape(k).slots;
    per_row = per_row > (size_t)kCutThreads * kCutMaxFast ? per_row
                                                          : (size_t)kCutThreads * kCutMaxFast;
    w.cut_floors_off = w.cut_keys_off + up((size_t)rows * per_row * sizeof(uint64_t));
    w.bytes = w.cut_floors_off + up((size_t)rows * gcap * sizeof(uint64_t));
    return w;
}

GemvCut topk_cut(void *ws, int rows, int64_t vocab, int k)
{
    const TopkWs w = topk_ws_layout(rows, vocab, k);
    const CutShape cs = cut_shape(k);
    char *b = static_cast<char *>(ws);
    return GemvCut{reinterpret_cast<uint64_t *>(b + w.cut_keys_off),
                   reinterpret_cast<uint64_t *>(b + w.cut_floors_off), cs.m, cs.slots,
                   kCutThreads * kCutMaxFast};
}

template <bool STATS>
hipError_t launch_merge(const CutArgs &a, int rows, int nfast, hipStream_t stream)
{
    const dim3 g(rows), b(kCutThreads);
    // the smallest instance holding the cuts
    const int mf = (nfast + kCutThreads - 1) / kCutThreads;
    if (mf <= 1) return launch(cut_merge<1, STATS>, g, b, 0, stream, a);
    if (mf <= 2) return launch(cut_merge<2, STATS>, g, b, 0, stream, a);
    if (mf <= 3) return launch(cut_merge<3, STATS>, g, b, 0, stream, a);
    if (mf <= 4) return launch(cut_merge<4, STATS>, g, b, 0, stream, a);
    if (mf <= 6) return launch(cut_merge<6, STATS>, g, b, 0, stream, a);
    static_assert(kCutMaxFast == 8, "the instances above and below cover the fast keys");
    return launch(cut_merge<8, STATS>, g, b, 0, stream, a);
}

hipError_t launch_cut_merge(const float *logits, int rows, int64_t vocab, int k,
                            const int32_t *idmap, int32_t *ids, float *vals, int32_t *argmax,
                            void *ws, int grid, hipStream_t stream, int slots, int64_t chunk,
                            float *probs, float *lse)
{
    GemvCut cut = topk_cut(ws, rows, vocab, k);
    if (slots > 0)
        cut.slots = slots;
    const int nfast = grid * cut.slots;
    if (grid < 1 || grid > kCutMaxChunks || nfast > kCutThreads * kCutMaxFast ||
        (probs && grid > kStatsMaxChunks))
        return hipErrorInvalidValue;
    CutArgs a;
    a.logits = logits;
    a.V = vocab;
    a.ntiles = (vocab + 15) / 16;
    a.k = k;
    a.grid = grid;
    a.slots = cut.slots;
    a.chunk = chunk;
    a.keys = cut.keys;
    a.floors = cut.floors;
    a.idmap = idmap;
    a.ids = ids;
    a.vals = vals;
    a.argmax = argmax;
    a.stats = probs ? topk_stats(ws, rows, vocab, k) : nullptr;
    a.probs = probs;
    a.lse = lse;
    return probs ? launch_merge<true>(a, rows, nfast, stream)
                 : launch_merge<false>(a, rows, nfast, stream);
}

float2 *topk_stats(void *ws, int rows, int64_t vocab, int k)
{
    return reinterpret_cast<float2 *>(static_cast<char *>(ws) +
                                      topk_ws_layout(rows, vocab, k).stats_off);
}

uint32_t *topk_tickets(void *ws, int rows, int64_t vocab, int k)
{
    return reinterpret_cast<uint32_t *>(static_cast<char *>(ws) +
                                        topk_ws_layout(rows, vocab, k).tickets_off);
}

template <bool STATS>
hipError_t launch_pass(int pt, dim3 g, dim3 b, const CutPassArgs &c, hipStream_t stream)
{
    return pt <= 1   ? launch(cut_pass<1, STATS>, g, b, 0, stream, c)
           : pt <= 2 ? launch(cut_pass<2, STATS>, g, b, 0, stream, c)
           : pt <= 4 ? launch(cut_pass<4, STATS>, g, b, 0, stream, c)
           : pt <= 8 ? launch(cut_pass<8, STATS>, g, b, 0, stream, c)
                     : launch(cut_pass<16, STATS>, g, b, 0, stream, c);
}

hipError_t launch_topk(const float *logits, int rows, int64_t vocab, int k,
                       const int32_t *idmap, int32_t *ids, float *vals, int32_t *argmax,
                       void *ws, hipStream_t stream, float *probs, float *lse)
{
    // the cut of every chunk, then their merge (two launches, no tickets).  Chunks a row: 256
    // for up to 4 rows, then fewer and larger ones, so that the call has about 1024
    // workgroups (at 16 rows, 4096 workgroups of 512 entries took 8.6 us against 3.4 us for
    // the 256 of one row); each chunk's cut is sized for its share of the k.
    const int64_t ntiles = (vocab + 15) / 16;
    int G = 1024 / rows;
    G = G < kCutPassMinGrid ? kCutPassMinGrid : G > kCutPassMaxGrid ? kCutPassMaxGrid : G;
    G = (int)(ntiles < G ? ntiles : G);
    const CutShape cs = cut_shape(k, G);
    const int64_t chunk = (ntiles + G - 1) / G * 16;   // whole tiles, so G chunks cover V
    const int pt = (int)((chunk + kCutPassThreads - 1) / kCutPassThreads);
    // within the library's limits (V <= 2^18: at most 4096 entries a chunk; k <= 512: at
    // most 64 x 34 or 256 x 16 cut keys a row) both always hold
    if (pt > kCutPassMaxPer || (int64_t)G * cs.slots > kCutThreads * kCutMaxFast)
        return hipErrorInvalidValue;
    const GemvCut cut = topk_cut(ws, rows, vocab, k);
    CutPassArgs c;
    c.logits = logits;
    c.V = vocab;
    c.chunk = chunk;
    c.m = cs.m;
    c.slots = cs.slots;
    c.keys = cut.keys;
    c.floors = cut.floors;
    c.stats = probs ? topk_stats(ws, rows, vocab, k) : nullptr;
    const dim3 g((unsigned)G, (unsigned)rows), b(kCutPassThreads);
    hipError_t e = probs ? launch_pass<true>(pt, g, b, c, stream)
                         : launch_pass<false>(pt, g, b, c, stream);
    if (e != hipSuccess)
        return e;
    return launch_cut_merge(logits, rows, vocab, k, idmap, ids, vals, argmax, ws, G, stream,
                            cs.slots, chunk, probs, lse);
}

}  // namespace dh
