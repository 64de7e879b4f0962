// Two-stage rescore on gfx950: exact logits of each row's candidate tokens from a dense bf16
// head, and the winning candidate.  Source: "dsv41 Zig: the TFE draft head
// (TF_DS_DRAFTER=eagle), off by default" (two_stage commit note and 'Update': the draft is the
// argmax of the candidates' exact logits from a dense bf16 copy of the target's head, through
// the candidates' id map).
//
// Design: the work is a gather of rows*cand_k head rows (10 KB each at H = 5120) -- memory
// bound, with one activation row per gathered head row, so plain FP32 FMAs on the vector
// ALUs.  One wave per (row, slot): each lane reads 16 bytes of the head row and of the
// activation row per step (a wave covers 1 KB of the head row per load), with five steps
// in flight before any is summed, sums its products in order, and the wave sums lanes with
// a fixed butterfly.  A second small kernel picks
// each row's winner under the same ordering as the top-k.
#include "dh_internal.h"
#include "launch.h"

namespace dh {
namespace {

constexpr int kRescoreWaves = 4;
// 512-column steps a lane has in flight: a 10 KB row (H = 5120) is two rounds.  Over four
// rotated sets of 16 x 512 random candidates (a cold gather) five measured 18.4 us, two
// 18.4-18.7, four 19.0 and eight 20.1: with 32 waves a compute unit, more in flight only
// queues.
constexpr int kSteps = 5;
constexpr int kRsrcWord3 = 0x00020000;   // gfx9-family raw buffer: 32-bit data format

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ inline float lo_bf16(uint32_t w) { return __uint_as_float(w << 16); }
__device__ inline float hi_bf16(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__global__ __launch_bounds__(kRescoreWaves * kWave) void rescore_dot(
    const uint16_t *W, int64_t V, int H, const uint16_t *x, const int32_t *cand,
    const float *cand_vals, int ck, float *exact)
{
    const int lane = threadIdx.x & 63;
    const int slot = blockIdx.x * kRescoreWaves + (threadIdx.x >> 6);
    const int r = blockIdx.y;
    if (slot >= ck)
        return;
    const int64_t t = (int64_t)r * ck + slot;
    const int64_t id = cand[t];
    float out;
    if (cand_vals && !(cand_vals[t] > -__builtin_inff())) {
        out = -__builtin_inff();          // a pad of the stage-1 list: not a candidate
    } else if (id < 0 || id >= V) {
        out = __builtin_nanf("");         // not a token of this head: never read
    } else {
        // bounded buffer loads (bytes past the row read as 0, adding nothing), kSteps steps of
        // 512 columns issued before any is used
        const __amdgpu_buffer_rsrc_t wrs = __builtin_amdgcn_make_buffer_rsrc(
            (void *)(W + id * H), (short)0, H * 2, kRsrcWord3);
        const __amdgpu_buffer_rsrc_t xrs = __builtin_amdgcn_make_buffer_rsrc(
            (void *)(x + (int64_t)r * H), (short)0, H * 2, kRsrcWord3);
        float acc = 0.f;
        for (int h0 = 0; h0 < H; h0 += kSteps * 8 * kWave) {
            u32x4 wq[kSteps], xq[kSteps];
#pragma unroll
            for (int j = 0; j < kSteps; j++) {
                const uint32_t off = (uint32_t)(h0 + j * 8 * kWave + lane * 8) * 2u;
                wq[j] = __builtin_amdgcn_raw_buffer_load_b128(wrs, off, 0, 0);
                xq[j] = __builtin_amdgcn_raw_buffer_load_b128(xrs, off, 0, 0);
            }
#pragma unroll
            for (int j = 0; j < kSteps; j++) {
                acc = __builtin_fmaf(lo_bf16(xq[j].x), lo_bf16(wq[j].x), acc);
                acc = __builtin_fmaf(hi_bf16(xq[j].x), hi_bf16(wq[j].x), acc);
                acc = __builtin_fmaf(lo_bf16(xq[j].y), lo_bf16(wq[j].y), acc);
                acc = __builtin_fmaf(hi_bf16(xq[j].y), hi_bf16(wq[j].y), acc);
                acc = __builtin_fmaf(lo_bf16(xq[j].z), lo_bf16(wq[j].z), acc);
                acc = __builtin_fmaf(hi_bf16(xq[j].z), hi_bf16(wq[j].z), acc);
                acc = __builtin_fmaf(lo_bf16(xq[j].w), lo_bf16(wq[j].w), acc);
                acc = __builtin_fmaf(hi_bf16(xq[j].w), hi_bf16(wq[j].w), acc);
            }
        }
        for (int off = 32; off > 0; off >>= 1)
            acc += __shfl_xor(acc, off);
        out = acc;
    }
    if (lane == 0)
        exact[t] = out;
}

__device__ inline bool eligible(float l) { return l == l && l > -__builtin_inff(); }

// (la, ia) beats (lb, ib) under the top-k ordering.
__device__ inline bool beats(float la, int32_t ia, float lb, int32_t ib)
{
    if (!eligible(la))
        return false;
    if (!eligible(lb))
        return true;
    if (la != lb)
        return la > lb;
    return ia < ib;
}

constexpr int kPickThreads = 256;

__global__ __launch_bounds__(kPickThreads) void rescore_pick(const float *exact,
                                                             const int32_t *cand, int ck,
                                                             int32_t *draft)
{
    __shared__ float bl[kPickThreads / 64];
    __shared__ int32_t bi[kPickThreads / 64];
    const int r = blockIdx.x;
    float best = __builtin_nanf("");
    int32_t bid = 0;
    for (int j = threadIdx.x; j < ck; j += kPickThreads) {
        const float l = exact[(int64_t)r * ck + j];
        const int32_t id = cand[(int64_t)r * ck + j];
        if (beats(l, id, best, bid)) {
            best = l;
            bid = id;
        }
    }
    for (int off = 32; off > 0; off >>= 1) {
        const float ol = __shfl_xor(best, off);
        const int32_t oi = __shfl_xor(bid, off);
        if (beats(ol, oi, best, bid)) {
            best = ol;
            bid = oi;
        }
    }
    if ((threadIdx.x & 63) == 0) {
        bl[threadIdx.x >> 6] = best;
        bi[threadIdx.x >> 6] = bid;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        for (int w = 1; w < kPickThreads / 64; w++)
            if (beats(bl[w], bi[w], best, bid)) {
                best = bl[w];
                bid = bi[w];
            }
        draft[r] = eligible(best) ? bid : 0;
    }
}

}  // namespace

hipError_t launch_rescore(const dh_head &dense, const uint16_t *x, int rows,
                          const int32_t *cand_ids, const float *cand_vals, int cand_k,
                          float *exact, int32_t *draft, hipStream_t stream)
{
    const dim3 grid((cand_k + kRescoreWaves - 1) / kRescoreWaves, rows);
    hipError_t e = launch(rescore_dot, grid, dim3(kRescoreWaves * kWave), 0, stream,
                          static_cast<const uint16_t *>(dense.weight), (int64_t)dense.vocab,
                          (int)dense.hidden, x, cand_ids, cand_vals, cand_k, exact);
    if (e != hipSuccess)
        return e;
    return launch(rescore_pick, dim3(rows), dim3(kPickThreads), 0, stream, (const float *)exact,
                  cand_ids, cand_k, draft);
}

}  // namespace dh
