// Two-stage rescore on gfx950: exact logits of each row's candidate tokens from a dense bf16
// head, and the winning candidate.  Source: "dsv41 Zig: the TFE draft head
// (TF_DS_DRAFTER=eagle), off by default" (two_stage commit note and 'Update': the draft is the
// argmax of the candidates' exact logits from a dense bf16 copy of the target's head, through
// the candidates' id map).
//
// Design: the work is a gather of rows*cand_k head rows (10 KB each at H = 5120) -- memory
// bound, with one activation row per gathered head row, so no matrix instructions: each lane
// takes 32-bit pairs of bf16 products with the two-way bf16 dot instruction (v_dot2c_f32_bf16,
// fp32 accumulation).  One wave per (row, slot), four waves a workgroup, all of one
// activation row: the workgroup stages that row in LDS once (every wave reading it from L2
// doubled the cache traffic of the gather).  The activation loads are issued first, then the
// wave's first round of head-row loads, so the LDS stores wait only for the activations.
// Each lane reads 16 bytes of the head row per step (a wave covers 1 KB of the row per load),
// with five steps in flight, sums its products in order, and the wave sums lanes with a fixed
// butterfly.  The winning candidate is picked either by a second small kernel, or -- when the
// call brings zeroed sync lines (dh_draft's workspace, dh_rescore_sync's buffer) -- by the
// candidates' workgroups themselves: each takes the 64-bit maximum of its candidates' (exact
// logit, token id) keys into the row's best word, then a ticket, and the row's last workgroup
// writes the draft and sets both words back to zero.  (A ticket per wave instead of per
// workgroup was slower, 22.3 us against 15.8 for 16 x 512 candidates: four times the atomics
// on each row's two lines.  Eight waves a workgroup measured the same as four.)
#include <algorithm>

#include "dh_internal.h"
#include "keys.h"
#include "launch.h"
#include "topk.h"

namespace dh {
namespace {

constexpr int kRescoreWaves = 4;
// 512-column steps a lane has in flight.  Over four rotated sets of 16 x 512 random
// candidates (a cold gather), one round of five steps at a time measured best; eight or ten
// steps were slower, with more waves than registers allow at once (20.7, 20.6 us against
// 18.3), and so was a second round kept in flight (18.7).
constexpr int kSteps = 5;
// activation vectors a thread loads before the head rows: 8192 columns a workgroup
constexpr int kXPre = 8192 / (8 * kRescoreWaves * kWave);
constexpr size_t kXLds = (size_t)kXPre * kRescoreWaves * kWave * 16;   // 16 KiB
constexpr int kRsrcWord3 = 0x00020000;   // gfx9-family raw buffer: 32-bit data format

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// acc + the two products of a 32-bit pair of bf16 values each
__device__ inline float dot2(uint32_t a, uint32_t b, float acc)
{
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a),
                                           __builtin_bit_cast(bf16x2, b), acc, false);
}

struct RescoreArgs {
    const uint16_t *W;      // dense bf16 head [V][H]
    int64_t V;
    int H;
    const uint16_t *x;      // bf16 [rows][H]
    const int32_t *cand;    // [rows][ck]
    const float *cand_vals; // stage-1 values [rows][ck], or NULL
    int ck;
    float *exact;           // [rows][ck]
    // PICK: the zeroed ticket lines and best-key lines of the rows (kTicketStride words
    // apart), and the drafts [rows]
    uint32_t *tickets;
    uint64_t *best;
    int32_t *draft;
};

// exact[r][slot] for one slot a wave; PICK: and the row's draft (see above).
template <bool PICK>
__global__ __launch_bounds__(kRescoreWaves * kWave) void rescore_dot(RescoreArgs a)
{
    extern __shared__ __align__(16) uint16_t xs[];   // the activation row (H, at least 8192)
    __shared__ uint64_t wbest[kRescoreWaves];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // uniform: scalar
    const int slot = blockIdx.x * kRescoreWaves + wave;
    const int r = blockIdx.y;
    const int H = a.H;
    const int64_t t = (int64_t)r * a.ck + slot;
    // the activation row's first kXPre * 256 16-byte vectors (bounded: past the row, 0),
    // loaded before anything else, so that neither the candidate's id nor its head row waits
    // on them
    const __amdgpu_buffer_rsrc_t xrs = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(a.x + (int64_t)r * H), (short)0, H * 2, kRsrcWord3);
    u32x4 xv[kXPre];
#pragma unroll
    for (int u = 0; u < kXPre; u++)
        xv[u] = __builtin_amdgcn_raw_buffer_load_b128(
            xrs, (uint32_t)(u * kRescoreWaves * kWave + threadIdx.x) * 16u, 0, 0);
    const bool live = slot < a.ck;
    // the wave's candidate (uniform over the wave: taken from lane 0, so the head row's
    // buffer descriptor is scalar)
    const int64_t id = __builtin_amdgcn_readfirstlane(live ? a.cand[t] : -1);
    // a pad of the stage-1 list is not a candidate; an id outside the head is not read
    const bool pad = __builtin_amdgcn_readfirstlane(
        live && a.cand_vals && !(a.cand_vals[t] > -__builtin_inff()));
    const bool read = live && !pad && id >= 0 && id < a.V;

    // the head row in rounds of kSteps steps of 512 columns (bounded buffer loads: bytes past
    // the row read as 0, adding nothing)
    const __amdgpu_buffer_rsrc_t wrs = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(a.W + (read ? id : 0) * H), (short)0, read ? H * 2 : 0, kRsrcWord3);
    u32x4 wq[kSteps];
    auto issue = [&](int h0) {
#pragma unroll
        for (int j = 0; j < kSteps; j++)
            wq[j] = __builtin_amdgcn_raw_buffer_load_b128(
                wrs, (uint32_t)(h0 + j * 8 * kWave + lane * 8) * 2u, 0, 0);
    };
    issue(0);
    // (unconditional: the LDS holds at least kXPre * 256 vectors)
#pragma unroll
    for (int u = 0; u < kXPre; u++)
        reinterpret_cast<u32x4 *>(xs)[u * kRescoreWaves * kWave + threadIdx.x] = xv[u];
    const int nx = H / 8;
    const u32x4 *xg = reinterpret_cast<const u32x4 *>(a.x + (int64_t)r * H);
    for (int i = kXPre * kRescoreWaves * kWave + threadIdx.x; i < nx; i += kRescoreWaves * kWave)
        reinterpret_cast<u32x4 *>(xs)[i] = xg[i];   // H > 8192
    __syncthreads();

    float acc = 0.f;
    constexpr int kRound = kSteps * 8 * kWave;
    for (int h0 = 0; h0 < H; h0 += kRound) {
        if (h0)
            issue(h0);
#pragma unroll
        for (int j = 0; j < kSteps; j++) {
            const int c = h0 + j * 8 * kWave + lane * 8;
            const u32x4 xq = c < H ? *reinterpret_cast<const u32x4 *>(&xs[c])
                                   : u32x4{0u, 0u, 0u, 0u};
            acc = dot2(xq.x, wq[j].x, acc);
            acc = dot2(xq.y, wq[j].y, acc);
            acc = dot2(xq.z, wq[j].z, acc);
            acc = dot2(xq.w, wq[j].w, acc);
        }
    }
    for (int off = 32; off > 0; off >>= 1)
        acc += __shfl_xor(acc, off);
    const float out = pad ? -__builtin_inff() : read ? acc : __builtin_nanf("");
    if (live && lane == 0)
        a.exact[t] = out;
    if constexpr (PICK) {
        // the workgroup's best (exact, token id) key; 0 when none of its candidates is
        // eligible (NaN, -inf, or no slot)
        if (lane == 0) {
            const uint32_t im = live ? order_key(out) : 0u;
            wbest[wave] = im ? entry_key(im, (uint32_t)id) : 0ull;
        }
        __syncthreads();
        if (threadIdx.x == 0) {
            uint64_t m = 0;
#pragma unroll
            for (int w = 0; w < kRescoreWaves; w++)
                m = wbest[w] > m ? wbest[w] : m;
            uint64_t *bw = a.best + (int64_t)r * (kTicketStride / 2);
            if (m != 0)
                atomicMax((unsigned long long *)bw, (unsigned long long)m);
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // the maximum is in place
            const uint32_t nb = (uint32_t)gridDim.x;   // the row's workgroups
            uint32_t *tw = &a.tickets[(int64_t)r * kTicketStride];
            if (atomicAdd(tw, 1u) == nb - 1u) {
                // every other workgroup of the row is done with both words
                const uint64_t b = __hip_atomic_load(bw, __ATOMIC_RELAXED,
                                                     __HIP_MEMORY_SCOPE_AGENT);
                a.draft[r] = b ? (int32_t)key_id(b) : 0;
                __hip_atomic_store(bw, (uint64_t)0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                __hip_atomic_store(tw, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
        }
    }
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
                          float *exact, int32_t *draft, hipStream_t stream, uint32_t *sync)
{
    RescoreArgs a;
    a.W = static_cast<const uint16_t *>(dense.weight);
    a.V = dense.vocab;
    a.H = (int)dense.hidden;
    a.x = x;
    a.cand = cand_ids;
    a.cand_vals = cand_vals;
    a.ck = cand_k;
    a.exact = exact;
    a.tickets = sync;
    a.best = sync ? reinterpret_cast<uint64_t *>(sync + (size_t)rows * kTicketStride) : nullptr;
    a.draft = draft;
    const dim3 grid((cand_k + kRescoreWaves - 1) / kRescoreWaves, rows);
    // the activation row, at least the kXPre vectors a thread stores (up to 64 KiB)
    const size_t lds = std::max((size_t)a.H * sizeof(uint16_t), kXLds);
    static int lds_set[64];                              // per device: the limit raised
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return e;
    if (dev < 0 || dev >= 64)
        return hipErrorInvalidDevice;
    if (!__atomic_load_n(&lds_set[dev], __ATOMIC_RELAXED)) {
        for (const void *k : {(const void *)rescore_dot<true>, (const void *)rescore_dot<false>}) {
            e = hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize,
                                    DH_MAX_HIDDEN * (int)sizeof(uint16_t));
            if (e != hipSuccess)
                return e;
        }
        __atomic_store_n(&lds_set[dev], 1, __ATOMIC_RELAXED);
    }
    if (sync)
        return launch(rescore_dot<true>, grid, dim3(kRescoreWaves * kWave), lds, stream, a);
    e = launch(rescore_dot<false>, grid, dim3(kRescoreWaves * kWave), lds, stream, a);
    if (e != hipSuccess)
        return e;
    return launch(rescore_pick, dim3(rows), dim3(kPickThreads), 0, stream, (const float *)exact,
                  cand_ids, cand_k, draft);
}

}  // namespace dh
