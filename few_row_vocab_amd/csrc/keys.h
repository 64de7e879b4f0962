// Device helpers of the top-k kernels: the 64-bit ordering keys of logits and the one-wave
// scan and bin search of a radix-select round.
//
// Ordering (from "nemotron: Super's MTP drafts on the draft vocabulary's FP8 rows ...",
// commit note on the few-row top-k, and "dsv41 Zig: the TFE draft head
// (TF_DS_DRAFTER=eagle), off by default", 'Update'): entry u beats entry v iff u is eligible
// and (v is not, or l_u > l_v, or l_u == l_v and u < v); NaN and -inf are not eligible and
// -0 == +0.  A logit's order-preserving 32-bit image is 0 when not eligible; with the id,
// (image << 32) | (0xffffffff - id) is distinct per entry and its numeric order is exactly
// this ordering.  Ineligible entries get the key 0.
#pragma once

#include "dh_internal.h"

namespace dh {

__device__ __forceinline__ uint32_t order_key(float f)
{
    uint32_t u = __float_as_uint(f);
    if (f != f || u == 0xff800000u)
        return 0u;                       // NaN or -inf: not eligible
    if ((u << 1) == 0u)
        u = 0u;                          // -0 and +0 are equal
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ uint64_t entry_key(uint32_t image, uint32_t id)
{
    return ((uint64_t)image << 32) | (uint64_t)(0xffffffffu - id);
}

__device__ __forceinline__ uint32_t key_id(uint64_t key) { return 0xffffffffu - (uint32_t)key; }

// The logit of a key, from its image; a zero's sign is not in the image, so zeros are read
// back from the logits (`src`).
__device__ __forceinline__ float image_value(uint64_t key, const float *src)
{
    const uint32_t im = (uint32_t)(key >> 32);
    if (im == 0x80000000u)
        return *src;
    return __uint_as_float((im & 0x80000000u) ? (im & 0x7fffffffu) : ~im);
}

// Inclusive prefix sum over the 64 lanes of a wave: shifts within rows of 16 lanes, then
// the row totals broadcast to the later rows (gfx9 DPP row_shr / row_bcast).
__device__ __forceinline__ uint32_t wave_scan(uint32_t v)
{
    v += __builtin_amdgcn_update_dpp(0u, v, 0x111, 0xf, 0xf, false);   // row_shr:1
    v += __builtin_amdgcn_update_dpp(0u, v, 0x112, 0xf, 0xf, false);   // row_shr:2
    v += __builtin_amdgcn_update_dpp(0u, v, 0x114, 0xf, 0xf, false);   // row_shr:4
    v += __builtin_amdgcn_update_dpp(0u, v, 0x118, 0xf, 0xf, false);   // row_shr:8
    v += __builtin_amdgcn_update_dpp(0u, v, 0x142, 0xa, 0xf, false);   // row_bcast:15
    v += __builtin_amdgcn_update_dpp(0u, v, 0x143, 0xc, 0xf, false);   // row_bcast:31
    return v;
}

// Reserves `mine` consecutive slots per lane from an LDS counter with one atomic per wave
// (a lane's slots follow those of the lanes below it); returns the lane's first slot.  All
// 64 lanes must take part.
__device__ __forceinline__ uint32_t wave_reserve(uint32_t mine, uint32_t *fill)
{
    const uint32_t incl = wave_scan(mine);
    const uint32_t total = __builtin_amdgcn_readlane(incl, 63);
    uint32_t base = 0;
    if (total != 0) {
        if ((threadIdx.x & 63) == 63)
            base = atomicAdd(fill, total);
        base = __builtin_amdgcn_readlane(base, 63);
    }
    return base + incl - mine;
}

// The smallest and largest of the non-zero 64-bit keys over the 64 lanes of a wave (the same
// DPP pattern as wave_scan; masked lanes keep the identity).  An all-zero wave gives
// (~0, 0).
__device__ __forceinline__ void wave_min_max(uint64_t &mn, uint64_t &mx)
{
#define DH_MINMAX_STEP(ctrl, rmask)                                                            \
    {                                                                                          \
        const uint32_t al = __builtin_amdgcn_update_dpp(0xffffffffu, (uint32_t)mn, ctrl, rmask, \
                                                        0xf, false);                           \
        const uint32_t ah = __builtin_amdgcn_update_dpp(0xffffffffu, (uint32_t)(mn >> 32),     \
                                                        ctrl, rmask, 0xf, false);              \
        const uint32_t bl = __builtin_amdgcn_update_dpp(0u, (uint32_t)mx, ctrl, rmask, 0xf,    \
                                                        false);                                \
        const uint32_t bh = __builtin_amdgcn_update_dpp(0u, (uint32_t)(mx >> 32), ctrl, rmask, \
                                                        0xf, false);                           \
        const uint64_t a = ((uint64_t)ah << 32) | al, b = ((uint64_t)bh << 32) | bl;           \
        mn = a < mn ? a : mn;                                                                  \
        mx = b > mx ? b : mx;                                                                  \
    }
    DH_MINMAX_STEP(0x111, 0xf)   // row_shr:1
    DH_MINMAX_STEP(0x112, 0xf)   // row_shr:2
    DH_MINMAX_STEP(0x114, 0xf)   // row_shr:4
    DH_MINMAX_STEP(0x118, 0xf)   // row_shr:8
    DH_MINMAX_STEP(0x142, 0xa)   // row_bcast:15
    DH_MINMAX_STEP(0x143, 0xc)   // row_bcast:31
#undef DH_MINMAX_STEP
    // lane 63 now holds the wave's extremes
    mn = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(mn >> 32), 63) << 32) |
         (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)mn, 63);
    mx = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(mx >> 32), 63) << 32) |
         (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)mx, 63);
}

// The smallest non-zero and the largest of 32-bit images over the 64 lanes of a wave (DPP,
// as wave_scan; masked lanes keep the identity), returned in every lane.  An all-zero wave
// gives (~0, 0).
__device__ __forceinline__ void wave_min_max32(uint32_t &mn, uint32_t &mx)
{
#define DH_MINMAX32_STEP(ctrl, rmask)                                                          \
    {                                                                                          \
        const uint32_t a = __builtin_amdgcn_update_dpp(0xffffffffu, mn, ctrl, rmask, 0xf, false); \
        const uint32_t b = __builtin_amdgcn_update_dpp(0u, mx, ctrl, rmask, 0xf, false);       \
        mn = a < mn ? a : mn;                                                                  \
        mx = b > mx ? b : mx;                                                                  \
    }
    DH_MINMAX32_STEP(0x111, 0xf)   // row_shr:1
    DH_MINMAX32_STEP(0x112, 0xf)   // row_shr:2
    DH_MINMAX32_STEP(0x114, 0xf)   // row_shr:4
    DH_MINMAX32_STEP(0x118, 0xf)   // row_shr:8
    DH_MINMAX32_STEP(0x142, 0xa)   // row_bcast:15
    DH_MINMAX32_STEP(0x143, 0xc)   // row_bcast:31
#undef DH_MINMAX32_STEP
    mn = (uint32_t)__builtin_amdgcn_readlane((int)mn, 63);
    mx = (uint32_t)__builtin_amdgcn_readlane((int)mx, 63);
}

// The float of an eligible image (+0 for a zero of either sign).
__device__ __forceinline__ float image_float(uint32_t im)
{
    return __uint_as_float((im & 0x80000000u) ? (im & 0x7fffffffu) : ~im);
}

// One wave's view of a round's histogram: lane l holds the bins just below NB - l * (NB/64),
// in descending order, so a prefix sum over lanes is a suffix sum over bins.  Finds the bin d
// with above < rem <= above + count, where `above` counts the keys in higher bins.  Returns
// the total of the histogram.
template <int NB>
__device__ __forceinline__ uint32_t locate(const uint32_t *h, uint32_t rem, uint32_t &d, uint32_t &above,
                                  uint32_t &count)
{
    constexpr int PER = NB / 64;
    const int lane = threadIdx.x & 63;
    const int lo = NB - PER * (lane + 1);          // lowest bin of this lane
    uint32_t c[PER];
#pragma unroll
    for (int j = 0; j < PER; j += 4) {
        const uint4 q = *reinterpret_cast<const uint4 *>(&h[lo + j]);
        c[j] = q.x;
        c[j + 1] = q.y;
        c[j + 2] = q.z;
        c[j + 3] = q.w;
    }
    uint32_t sum = 0;
#pragma unroll
    for (int j = 0; j < PER; j++)
        sum += c[j];
    const uint32_t incl = wave_scan(sum);
    uint32_t a = incl - sum;                       // keys in bins above this lane's
    uint32_t hd = 0, ha = 0, hc = 0;
    bool hit = false;
#pragma unroll
    for (int j = PER - 1; j >= 0; j--) {           // this lane's bins, highest first
        const bool h1 = a < rem && rem <= a + c[j];
        hd = h1 ? (uint32_t)(lo + j) : hd;
        ha = h1 ? a : ha;
        hc = h1 ? c[j] : hc;
        hit |= h1;
        a += c[j];
    }
    const uint64_t b = __builtin_amdgcn_ballot_w64(hit);
    const int L = b ? (int)__builtin_ctzll(b) : 0;
    d = (uint32_t)__builtin_amdgcn_readlane((int)hd, L);
    above = (uint32_t)__builtin_amdgcn_readlane((int)ha, L);
    count = (uint32_t)__builtin_amdgcn_readlane((int)hc, L);
    return (uint32_t)__builtin_amdgcn_readlane((int)incl, 63);
}

}  // namespace dh
