// Keyed sampling over a row's top-k candidates on gfx950.  Source: "DeepSeek-V4.1:
// performance hooks and host checks", commit notes on the serving module's sampler (a
// window's choices come from the candidates, their nucleus statistics and a pick keyed by
// seed, position and token id, so a drafted token equals the serial one).  The pages give no
// formula; the reading implemented here:
//   q_j = exp((v_j - v_0) / T) over the eligible candidates in list order (1 when v_j == v_0);
//   the nucleus keeps j while the mass before it is below top_p * sum(q) (j = 0 always), and
//   min-p drops q_j < min_p;
//   the pick maximises (v_j - v_0) / T - ln(-ln u_j) over the kept (Gumbel-max), u_j the
//   uniform of (seed, position, id_j) from Philox4x64-10, the lower id on a tie.
// Everything is in double: the pick is an argmax decided by floating point.
//
// Design: a small latency-bound step (k <= 512 candidates a row): one workgroup per row, two
// adjacent candidates a thread, a block-wide scan for the mass before each candidate and a
// block-wide argmax.
#include "dh_internal.h"
#include "launch.h"

namespace dh {
namespace {

constexpr int kSampleThreads = 256;   // 2 candidates a thread: k <= 512

// Philox4x64-10 (Salmon, Moraes, Dror and Shaw, SC 2011): ten rounds of two 64 x 64 -> 128
// products on counter words 0 and 2, the key bumped by two Weyl constants between rounds.
__device__ inline uint64_t philox_first_word(uint64_t c0, uint64_t c1, uint64_t c2, uint64_t c3,
                                             uint64_t k0, uint64_t k1)
{
    constexpr uint64_t M0 = 0xD2E7470EE14C6C93ull, M1 = 0xCA5A826395121157ull;
#pragma unroll
    for (int round = 0; round < 10; round++) {
        if (round) {
            k0 += 0x9E3779B97F4A7C15ull;
            k1 += 0xBB67AE8584CAA73Bull;
        }
        const uint64_t h0 = __umul64hi(M0, c0), l0 = M0 * c0;
        const uint64_t h1 = __umul64hi(M1, c2), l1 = M1 * c2;
        c0 = h1 ^ c1 ^ k0;
        c1 = l1;
        c2 = h0 ^ c3 ^ k1;
        c3 = l0;
    }
    return c0;
}

// The uniform in (0, 1) of (seed, position, id): counter (position, id, 0, 0), key (seed, 0).
__device__ inline double keyed_uniform(uint64_t seed, int64_t position, int32_t id)
{
    const uint64_t w = philox_first_word((uint64_t)position, (uint64_t)(uint32_t)id, 0, 0, seed, 0);
    return ((double)(w >> 11) + 0.5) * 0x1p-53;
}

__device__ inline double wave_scan_f64(double v)
{
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const double u = __shfl_up(v, o);
        if (lane >= o)
            v += u;
    }
    return v;
}

// a beats b: higher score, then the lower id
__device__ inline bool wins(double sa, int32_t ia, double sb, int32_t ib)
{
    return sa > sb || (sa == sb && ia < ib);
}

__global__ __launch_bounds__(kSampleThreads) void sample_kernel(
    const int32_t *ids, const float *vals, int k, double T, double top_p, double min_p,
    uint64_t seed, const int64_t *pos, int32_t *token, int32_t *kept)
{
    __shared__ double wsum[kSampleThreads / 64];
    __shared__ double bscore[kSampleThreads / 64];
    __shared__ int32_t bid[kSampleThreads / 64];
    __shared__ int32_t bkept[kSampleThreads / 64];
    const int r = blockIdx.x;
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int32_t *ri = ids + (int64_t)r * k;
    const float *rv = vals + (int64_t)r * k;
    const float v0 = rv[0];
    if (!(v0 > -__builtin_inff()) || T == 0.0) {       // no eligible candidate, or greedy
        if (t == 0) {
            const bool any = v0 > -__builtin_inff();
            token[r] = any ? ri[0] : 0;
            if (kept)
                kept[r] = any ? 1 : 0;
        }
        return;
    }
    // this thread's candidates j = 2t, 2t + 1
    double q[2], d[2];
    int32_t id[2];
    bool el[2];
#pragma unroll
    for (int h = 0; h < 2; h++) {
        const int j = 2 * t + h;
        const float v = j < k ? rv[j] : -__builtin_inff();
        id[h] = j < k ? ri[j] : 0;
        el[h] = v > -__builtin_inff();
        d[h] = v == v0 ? 0.0 : ((double)v - (double)v0) / T;
        q[h] = !el[h] ? 0.0 : (v == v0 ? 1.0 : exp(d[h]));
    }
    // mass before each candidate: an inclusive scan of the pair sums, block-wide
    const double pair = q[0] + q[1];
    double incl = wave_scan_f64(pair);
    if (lane == 63)
        wsum[wave] = incl;
    __syncthreads();
    double base = 0.0, z = 0.0;
#pragma unroll
    for (int w = 0; w < kSampleThreads / 64; w++) {
        base += w < wave ? wsum[w] : 0.0;
        z += wsum[w];
    }
    const double before0 = base + incl - pair;
    const double before[2] = {before0, before0 + q[0]};
    double best = -__builtin_inf();
    int32_t bi = 0x7fffffff;
    int nk = 0;
#pragma unroll
    for (int h = 0; h < 2; h++) {
        const int j = 2 * t + h;
        const bool keep = el[h] && (j == 0 || (before[h] < top_p * z && q[h] >= min_p));
        if (keep) {
            nk++;
            const double s = d[h] - log(-log(keyed_uniform(seed, pos[r], id[h])));
            if (wins(s, id[h], best, bi)) {
                best = s;
                bi = id[h];
            }
        }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        const double os = __shfl_xor(best, o);
        const int32_t oi = __shfl_xor(bi, o);
        nk += __shfl_xor(nk, o);
        if (wins(os, oi, best, bi)) {
            best = os;
            bi = oi;
        }
    }
    if (lane == 0) {
        bscore[wave] = best;
        bid[wave] = bi;
        bkept[wave] = nk;
    }
    __syncthreads();
    if (t == 0) {
        int total = 0;
        for (int w = 0; w < kSampleThreads / 64; w++) {
            total += bkept[w];
            if (wins(bscore[w], bid[w], best, bi)) {
                best = bscore[w];
                bi = bid[w];
            }
        }
        token[r] = bi;
        if (kept)
            kept[r] = total;
    }
}

}  // namespace

hipError_t launch_sample(const int32_t *ids, const float *vals, int rows, int k, double T,
                         double top_p, double min_p, uint64_t seed, const int64_t *pos,
                         int32_t *token, int32_t *kept, hipStream_t stream)
{
    return launch(sample_kernel, dim3(rows), dim3(kSampleThreads), 0, stream, ids, vals, k, T,
                  top_p, min_p, seed, pos, token, kept);
}

}  // namespace dh
