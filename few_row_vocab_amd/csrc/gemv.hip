// Few-row vocabulary GEMV on gfx950 matrix cores.
//
// logits[r][v] = sum_h x[r][h] * w[v][h] for up to 16 activation rows r against a [V][H]
// head stored as bf16, as E4M3 codes with E8M0 scales per 32x32 block, or as E4M3 codes with
// an fp32 scale per row.  Sources: "dsv41 Zig: the TFE draft head (TF_DS_DRAFTER=eagle), off
// by default" (commit notes: the own GEMV for up to 16 rows, fp32 output; 'What this
// changes': fp32 sums; 'Update': FP8 linears with a row scale) and "dsv41 metal: the DSpark
// drafter on an FP8 head, a concurrent propose and resident buffers" ('FP8 draft head':
// E4M3 codes with E8M0 scales per 32x32 block).
//
// Design (MI355X):
//  * The head is streamed from HBM exactly once; it is the whole cost (>98% of the bytes).
//  * One v_mfma_f32_16x16x32_bf16 multiplies a 16-row x 32-column weight tile by the
//    32 x 16 activation block; its N = 16 columns are the (up to) 16 activation rows, so
//    the same instruction sequence serves 1..16 rows and a row's sums never depend on how
//    many rows share the call.
//  * FP8 codes are widened to bf16 in registers with v_cvt_scalef32_pk_bf16_fp8, the block
//    scale applied in the same instruction.  E4M3 times a power of two is exact in bf16, so
//    the products are the exact products; only fp32 accumulation rounds.
//  * A workgroup splits H over its waves (up to 16).  Each wave keeps its H-slice of the
//    activations in VGPRs for the whole kernel, so activations are read once per workgroup,
//    and streams 16-row tiles of the head: lane l reads 16 contiguous bytes (bf16: 32) of
//    row l%16 at column 16*(l/16) of each 64-column block.  The waves' partial 16x16 tiles
//    are summed through LDS in a fixed wave order (deterministic) and written as fp32.
//  * Persistent grid: one workgroup per CU slot, tiles taken round-robin; each 64-column
//    block's registers are refilled as soon as they are widened (row-major heads: with the
//    same block of the next tile, so a tile of loads is always in flight; tiled heads: with
//    the block a fixed window ahead, wrapping into the next tile), also across the
//    reduction's barrier.  The loop has no branches around loads and no stores (logits wait
//    in LDS until the end).
//  * Tiled heads (DH_TILED, made at load): each 1 KiB of the weight is one wave's operand
//    in lane order, so every load reads whole lines and carries the non-temporal hint; the
//    lanes receive the same bytes as from the row-major head, so the results are the same
//    bits.
#include "dh_internal.h"
#include "keys.h"
#include "launch.h"

namespace dh {
namespace {

constexpr int kMaxWaves = 16;
// 17..32 activation rows: two 16-row MFMA column blocks.  Their activations double the VGPRs a
// wave holds, so such launches run half the waves (256 VGPRs each), each wave doing the work
// of two waves of the 16-row launch with separate sums (so a row's sums are the same bits
// as in a 16-row call), for H <= 5120 (4096 for a row-major bf16 head, whose tile spills
// at 5120); wider heads take two 16-row launches.
constexpr int kMaxWaves2 = kMaxWaves / 2;
constexpr int kRsrcWord3 = 0x00020000;   // gfx9-family raw buffer: 32-bit data format
// Row-major heads: plain loads.  A wave's load covers 16 rows x 64 bytes there, and with the
// non-temporal hint such part-line reads measured ~15% slower.  Tiled heads: every load reads
// 1 KiB of whole lines, and there the non-temporal hint streams ~11% faster than plain loads.
constexpr int kCachePolicy = 0;
constexpr int kCacheNT = 2;              // gfx950 cache policy bit 1: non-temporal
// Tiled heads: weight bytes a workgroup keeps in flight (KiB), so a wave refills only a
// window of blocks ahead rather than a whole tile.  A streaming-read probe with the
// non-temporal hint peaked with about 32 KiB in flight per compute unit (7.0 TB/s) and fell
// with more (6.65 TB/s at 64 KiB).  In the GEMV at H = 5120, 32 KiB (FP8) and 48 KiB (bf16)
// measured best, by about 1% over a whole tile in flight; 16 and 24 KiB (one FP8 block a
// wave) were slower.  16-row launches whose waves take 7 or 8 FP8 blocks (H from 6,145 to
// 8,192) do better with one block a wave in flight (16 KiB): H = 7168, 169.6-169.9 against 172.8-173.2 us at one row (176.7
// against 179.2-179.6 at 16 rows); H = 8192, 160.2-160.6 against 162.1-163.0 at one row;
// at 6 blocks (H = 6144) one block was slower (119.8-120.3 against 116.1-116.6).
template <int FMT>
constexpr int tiled_ahead_kib() { return FMT == DH_BF16 ? 48 : 32; }
template <int FMT, int KW>
constexpr bool tiled_one_block() { return FMT != DH_BF16 && (KW == 7 || KW == 8); }
constexpr int kMaxStageBytes = 64 * 1024;   // logits a block keeps in LDS until its end
// A tile's sums in the stage.  Up to 16 rows (the draft's cut runs there) a tile is padded by
// 16 floats: the cut reads one row's entries of four tiles in one instruction, and unpadded
// tiles (a multiple of 64 floats apart) would put all four on the same LDS banks.  32-row
// tiles are not padded: at 129,280 rows a workgroup keeps 32 of them, which padding would
// push past the stage's 64 KiB (and the launch past one workgroup per compute unit).
constexpr int stage_stride(int outs) { return outs == 256 ? outs + 16 : outs; }
// Heads wider than 16 waves of 8 blocks (H > 8192) are streamed in column chunks of 16 * 8
// 64-column blocks (CH below): a wave holds one chunk's activations at a time.  Both layouts
// take the same chunks and the same 16 virtual waves (so they keep giving the same bits); a
// row-major chunked launch runs 8 waves of two virtual waves (256 VGPRs) and keeps 4 blocks
// of loads in flight, as 16 waves with a tile in flight spill registers.
constexpr int kChunkKbw = 8;
constexpr int kMaxDevices = 64;

struct GemvArgs {
    const uint8_t *w;       // weight bytes
    const uint8_t *bscale;  // E8M0 [ceil(V/32)][H/32] (block format)
    const float *rscale;    // fp32 [V] (row format)
    const uint16_t *x;      // bf16 [R][H]
    float *logits;          // fp32 [R][V] (mode DH_OUT_F32)
    uint16_t *out16;        // bf16 [R][V] (modes DH_OUT_BF16, DH_OUT_ADD_BF16)
    const uint16_t *residual;   // bf16 [R][V] (mode DH_OUT_ADD_BF16; may equal out16)
    int mode;               // dh_out_mode
    int64_t V;
    int H;
    int R;
    int ntiles;
    int nkb;                // number of 64-column blocks, ceil(H / 64)
    int tile_bytes;         // tiled layout: bytes of one 16-row tile, nkb * 1024 * (bytes/weight)
    uint32_t *zero;         // nzero pairs of words, zstride apart, the first workgroup zeroes
    int nzero, zstride;
    // the draft's fused top-k cut (GemvCut; cut_m == 0: none)
    uint64_t *cut_keys, *cut_floors;
    int cut_m, cut_slots, cut_max;
    float *part;            // SPL: the chunks' partial sums, fp32 [chunks][R][V]
};

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

union Pack8 {
    bf16x8 v;
    uint32_t u[4];
    u32x4 q;
};

template <bool HI>
__device__ inline uint32_t cvt2(uint32_t src, float scale)
{
    bf16x2 r = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)src, scale, HI);
    return __builtin_bit_cast(uint32_t, r);
}

// 16 E4M3 codes -> two groups of 8 bf16 (bytes 0..7 and 8..15), each times `scale`.
__device__ inline void widen16(u32x4 q, float scale, bf16x8 &a0, bf16x8 &a1)
{
    Pack8 p0, p1;
    p0.u[0] = cvt2<false>(q.x, scale);
    p0.u[1] = cvt2<true>(q.x, scale);
    p0.u[2] = cvt2<false>(q.y, scale);
    p0.u[3] = cvt2<true>(q.y, scale);
    p1.u[0] = cvt2<false>(q.z, scale);
    p1.u[1] = cvt2<true>(q.z, scale);
    p1.u[2] = cvt2<false>(q.w, scale);
    p1.u[3] = cvt2<true>(q.w, scale);
    a0 = p0.v;
    a1 = p1.v;
}

// float -> bf16 bits, round to nearest even (NaN stays NaN).
__device__ inline uint16_t bf16_bits(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }

// An E8M0 byte as the fp32 scale operand: the bit pattern b << 23, which is the power of
// two 2^(b-127) for bytes 1..254.
__device__ inline float e8m0_scale(uint32_t b) { return __uint_as_float(b << 23); }

// A sum s of head row v with the row scale applied (FP8 row format).
__device__ inline float row_scaled(const GemvArgs &a, int64_t v, float s)
{
    return a.rscale ? s * a.rscale[v] : s;
}

// The output of one (activation row c, head row v) scaled sum s, in the mode.
__device__ inline void store_out(const GemvArgs &a, int c, int64_t v, float s)
{
    const int64_t at = (int64_t)c * a.V + v;
    if (a.mode == DH_OUT_F32) {
        a.logits[at] = s;
    } else {
        // the sum, plus the residual for the add mode, rounded to bf16 once
        if (a.mode == DH_OUT_ADD_BF16)
            s += __uint_as_float((uint32_t)a.residual[at] << 16);
        a.out16[at] = bf16_bits(s);
    }
}

// The output of one (activation row c, head row v) sum s: the row scale, then the mode.
__device__ inline void write_out(const GemvArgs &a, int c, int64_t v, float s)
{
    store_out(a, c, v, row_scaled(a, v, s));
}

// The draft's fused top-k cut of every row over this workgroup's entries, by the whole
// workgroup (every thread calls it; nw waves).  The workgroup did tiles blockIdx.x + t *
// gridDim.x for t < ntl; entry 16 t + i is head row 16 (blockIdx.x + t * gridDim.x) + i.
// The writer of the logits leaves in stage[t * SST + 16 r + i] the image of the entry's
// logit (topk.hip's order-preserving image; 0 when not eligible or past the head's rows) and
// each row's range of images in rng (rng[r] the smallest non-zero one, rng[16 + r] the
// largest).  An entry's key is topk.hip's (image, id).  Per row, the keys are binned over the
// range (256 bins of equal width, as the top-k's select: a higher bin holds only larger
// values); with d the bin of the m-th largest key, the cut is the keys of bins >= d, or of
// bins > d (fewer than m) when those would not fit `slots`.  They go to the workgroup's slots
// in any order, zeros after them; the floor is the smallest key of the cut, every key left
// out being smaller, or 0 when none was left out.
// A row is cut by a group of g waves, g a power of two up to 4 with g R <= nw (one wave a
// row from nw / 2 rows up, a batch of rows after another when there are more than nw); lane
// l of the group's wave q takes entries 64 (g j + q) + l.  The workgroup's 16 waves share 4
// SIMDs, so a pass's fixed work costs once per wave there: more than 4 waves a row only
// repeat it.  The code runs once per workgroup, from a cold instruction cache, so it is kept
// short: each of the two passes (histogram, cut) re-reads the images from LDS rather than
// holding them in registers (unrolled into registers, the code grew several-fold and
// measured several microseconds slower).
// ws: 16 KiB + 256 B of free LDS (the reduction buffer), set up by cut_init.
constexpr int kCutLgWavesPerRow = 2;
constexpr int kRscPre = 1024;   // row scales a block prefetches, at most (one a thread)   // log2 of the waves that cut one row, at most
// The smallest non-zero and the largest of (mn, mx) over each row of 16 lanes, in the row's
// last lane (DPP row shifts; lanes with no source keep the identity).
__device__ __forceinline__ void row_min_max32(uint32_t &mn, uint32_t &mx)
{
#define DH_ROW_STEP(ctrl)                                                                      \
    {                                                                                          \
        const uint32_t p = __builtin_amdgcn_update_dpp(0xffffffffu, mn, ctrl, 0xf, 0xf, false); \
        const uint32_t q = __builtin_amdgcn_update_dpp(0u, mx, ctrl, 0xf, 0xf, false);          \
        mn = p < mn ? p : mn;                                                                  \
        mx = q > mx ? q : mx;                                                                  \
    }
    DH_ROW_STEP(0x111)   // row_shr:1
    DH_ROW_STEP(0x112)   // row_shr:2
    DH_ROW_STEP(0x114)   // row_shr:4
    DH_ROW_STEP(0x118)   // row_shr:8
#undef DH_ROW_STEP
}
// A workgroup barrier for the cut's LDS only: this wave's LDS operations complete, then
// s_barrier.  __syncthreads() would also wait for every global store still in flight (the
// logits, the cut keys), which nothing in the workgroup reads: that wait measured about
// 0.4 us a barrier.
__device__ __forceinline__ void lds_barrier()
{
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}
struct CutLdsView {
    uint32_t *hist;                 // [16][256]
    uint32_t *gcnt;                 // [16] per group: cut keys placed
    unsigned long long *gfloor;     // [16] per group: the smallest cut key
};
__device__ __forceinline__ CutLdsView cut_view(uint32_t *ws)
{
    CutLdsView v;
    v.hist = ws;
    v.gcnt = ws + 16 * 256;
    v.gfloor = reinterpret_cast<unsigned long long *>(v.gcnt + 16);
    return v;
}
// Every group's counters and histogram to their start (call before a barrier).
__device__ __forceinline__ void cut_init(uint32_t *ws)
{
    const CutLdsView v = cut_view(ws);
    for (int q = threadIdx.x; q < 16 * 256; q += blockDim.x)
        v.hist[q] = 0;
    if (threadIdx.x < 16) {
        v.gcnt[threadIdx.x] = 0;
        v.gfloor[threadIdx.x] = ~0ull;
    }
}

template <int SST>
__device__ __forceinline__ void cut_rows(const GemvArgs &a, const uint32_t *stage, int ntl,
                                         uint32_t *ws, const uint32_t *rng)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int nw = blockDim.x >> 6;
    // waves a row: a power of two, at most kCutWavesPerRow (more only repeat the fixed work
    // of a pass on every SIMD), with lg = log2 of it
    int lg = 0;
    while (lg < kCutLgWavesPerRow && (a.R << (lg + 1)) <= nw)
        lg++;
    const int rows_per_batch = nw >> lg;
    const int grp = wave >> lg, wig = wave & ((1 << lg) - 1);
    // lane l of wave wig takes entries 64 (g j + wig) + l: tiles t = 4 (g j + wig) + l / 16,
    // head rows 16 (blockIdx.x + t * gridDim.x) + l % 16
    const int t0 = 4 * wig + (lane >> 4), tstep = 4 << lg;
    const int i = lane & 15;
    const uint32_t id0 = ((uint32_t)blockIdx.x + (uint32_t)t0 * gridDim.x) * 16u + (uint32_t)i;
    const uint32_t idstep = (uint32_t)tstep * gridDim.x * 16u;
    const CutLdsView v = cut_view(ws);
    uint32_t *hist = v.hist + grp * 256;
    const int slots = a.cut_slots;
    for (int b0 = 0; b0 < a.R; b0 += rows_per_batch) {
        const int r = b0 + grp;
        const bool act = grp < rows_per_batch && r < a.R;
        // the image of the entry of tile t (0 when not eligible, or past the head's rows)
        const uint32_t *srow = stage + 16 * r + i;
        auto image = [&](int t) -> uint32_t { return srow[t * SST]; };
        // 1: the histogram over the range of the row's eligible images (rng, from the writer)
        const uint32_t mn = act ? rng[r] : ~0u, mx = act ? rng[16 + r] : 0u;
        const float lo = image_float(mn);
        const float scale = 256.0f / (image_float(mx) - lo);
        // the select's bin map (a NaN product, from a zero or infinite width, goes to 255)
        auto bin_of = [&](uint32_t x) -> uint32_t {
            return (uint32_t)fminf((image_float(x) - lo) * scale, 255.0f);
        };
        if (act && mx != 0) {
#pragma unroll 2
            for (int t = t0; t < ntl; t += tstep) {
                const uint32_t im = image(t);
                if (im != 0)
                    atomicAdd(&hist[bin_of(im)], 1u);
            }
        }
        lds_barrier();
        // 2: the cut (every key when at most m, bins >= d, or bins > d) to the slots
        uint64_t *out = a.cut_keys + ((int64_t)r * gridDim.x + blockIdx.x) * slots;
        bool all = true;
        if (act && mx != 0) {
            uint32_t d, above, count;
            const uint32_t total = locate<256>(hist, (uint32_t)a.cut_m, d, above, count);
            all = total <= (uint32_t)a.cut_m;
            uint32_t dmin = 0;
            if (!all) {
                dmin = above + count <= (uint32_t)slots ? d : d + 1;
                all = dmin == d && above + count == total;
            }
            uint32_t id = id0;
#pragma unroll 2
            for (int t = t0; t < ntl; t += tstep, id += idstep) {
                const uint32_t im = image(t);
                if (im != 0 && (all || bin_of(im) >= dmin)) {
                    const uint64_t key = entry_key(im, id);
                    out[atomicAdd(&v.gcnt[grp], 1u)] = key;
                    atomicMin(&v.gfloor[grp], (unsigned long long)key);
                }
            }
        }
        lds_barrier();
        // 3: zeros after the cut; the floor; the group's counters back to their start
        if (act && wig == 0) {
            const uint32_t placed = v.gcnt[grp];
            for (int q = (int)placed + lane; q < slots; q += kWave)
                out[q] = 0;
            if (lane == 0)
                a.cut_floors[(int64_t)r * gridDim.x + blockIdx.x] = all ? 0ull : v.gfloor[grp];
        }
        if (b0 + rows_per_batch < a.R) {           // another batch: reset, then a barrier
            lds_barrier();
            cut_init(ws);
            lds_barrier();
        }
    }
}

// The writer and the draft's cut when every wave owns whole rows (R > nw / 2): wave w writes
// the logits of rows w, w + nw, ... and cuts each (as cut_rows: the same bins, cut and floor),
// with no workgroup barrier (rsc: the block's row scales in LDS, or NULL to load them).
// Lane l takes entries l + 64 j (tiles l / 16 + 4 j, head rows
// 16 (blockIdx.x + t gridDim.x) + l % 16); the range stays in registers, the wave's own 256
// histogram words and cut counter sit in ws (the free reduction buffer), and the floor is a
// wave reduction.  The wave's LDS operations complete in order between its passes.
template <int SST>
__device__ __forceinline__ void write_cut_own_rows(const GemvArgs &a, float *stage, int ntl,
                                                   uint32_t *ws, const float *rsc)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int nw = blockDim.x >> 6;
    uint32_t *hist = ws + wave * 256;
    uint32_t *cnt = ws + 16 * 256 + wave;
    const int t0 = lane >> 4, i = lane & 15;
    const uint32_t id0 = ((uint32_t)blockIdx.x + (uint32_t)t0 * gridDim.x) * 16u + (uint32_t)i;
    const uint32_t idstep = 4u * gridDim.x * 16u;
    const int slots = a.cut_slots;
    for (int r = wave; r < a.R; r += nw) {
        float *srow = stage + 16 * r + i;
        const uint32_t *irow = reinterpret_cast<const uint32_t *>(srow);
        // 1: the row's logits written, their images left in the stage; the range.  Four
        // entries at a time, their sums and row scales loaded before any of their stores
        // (which the compiler may not move a row-scale load past)
        uint32_t mn = ~0u, mx = 0;
        {
            uint32_t id = id0;
            for (int t = t0; t < ntl; t += 16, id += 4 * idstep) {
                float sv[4], rs[4];
#pragma unroll
                for (int u = 0; u < 4; u++) {
                    const int tu = t + 4 * u;
                    const uint32_t idu = id + (uint32_t)u * idstep;
                    sv[u] = tu < ntl ? srow[tu * SST] : 0.f;
                    rs[u] = rsc && tu < ntl ? rsc[tu * 16 + i]
                            : a.rscale && tu < ntl && (int64_t)idu < a.V ? a.rscale[idu] : 1.0f;
                }
#pragma unroll
                for (int u = 0; u < 4; u++) {
                    const int tu = t + 4 * u;
                    const uint32_t idu = id + (uint32_t)u * idstep;
                    if (tu < ntl) {
                        uint32_t im = 0;
                        if ((int64_t)idu < a.V) {
                            const float s = a.rscale ? sv[u] * rs[u] : sv[u];   // row_scaled
                            store_out(a, r, idu, s);
                            im = order_key(s);
                        }
                        *reinterpret_cast<uint32_t *>(srow + tu * SST) = im;
                        mn = im != 0 && im < mn ? im : mn;
                        mx = im > mx ? im : mx;
                    }
                }
            }
        }
        wave_min_max32(mn, mx);
        uint64_t *out = a.cut_keys + ((int64_t)r * gridDim.x + blockIdx.x) * slots;
        uint64_t *floor = a.cut_floors + (int64_t)r * gridDim.x + blockIdx.x;
        if (mx == 0) {                             // no eligible entry
            for (int q = lane; q < slots; q += kWave)
                out[q] = 0;
            if (lane == 0)
                *floor = 0;
            continue;
        }
        const float lo = image_float(mn);
        const float scale = 256.0f / (image_float(mx) - lo);
        auto bin_of = [&](uint32_t x) -> uint32_t {
            return (uint32_t)fminf((image_float(x) - lo) * scale, 255.0f);
        };
        reinterpret_cast<uint4 *>(hist)[lane] = uint4{0u, 0u, 0u, 0u};
        if (lane == 0)
            *cnt = 0;
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        // 2: the histogram
#pragma unroll 2
        for (int t = t0; t < ntl; t += 4) {
            const uint32_t im = irow[t * SST];
            if (im != 0)
                atomicAdd(&hist[bin_of(im)], 1u);
        }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        // 3: the cut (every key when at most m, bins >= d, or bins > d) to the slots
        uint32_t d, above, count;
        const uint32_t total = locate<256>(hist, (uint32_t)a.cut_m, d, above, count);
        bool all = total <= (uint32_t)a.cut_m;
        uint32_t dmin = 0;
        if (!all) {
            dmin = above + count <= (uint32_t)slots ? d : d + 1;
            all = dmin == d && above + count == total;
        }
        uint64_t kmin = ~0ull, kmax = 0;
        {
            uint32_t id = id0;
#pragma unroll 2
            for (int t = t0; t < ntl; t += 4, id += idstep) {
                const uint32_t im = irow[t * SST];
                if (im != 0 && (all || bin_of(im) >= dmin)) {
                    const uint64_t key = entry_key(im, id);
                    out[atomicAdd(cnt, 1u)] = key;
                    kmin = key < kmin ? key : kmin;
                }
            }
        }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        const uint32_t placed = *cnt;
        for (int q = (int)placed + lane; q < slots; q += kWave)
            out[q] = 0;
        wave_min_max(kmin, kmax);                  // kmin: the cut's smallest key (~0: none)
        if (lane == 0)
            *floor = all ? 0ull : kmin;
    }
}

// FULL: every wave's 64-column blocks lie inside the row (H a multiple of 64 and the
// blocks split evenly over the waves), so no load needs a guard.
// TR: 16-row MFMA groups per tile (a tile is 16 * TR head rows, inside one 32-row block
// of scales); two groups double the bytes in flight and halve the barriers per byte.
// NB: 16-row blocks of activation rows (1: up to 16 rows; 2: up to 32).  Each weight tile
// is widened once and multiplied by every block.
// VW: "virtual waves" per wave.  The H split is always that of a 16-wave launch (virtual
// waves of KBW blocks each); a wave covers VW of them with a sum apiece, and the reduction
// adds the virtual waves' sums in order, so VW changes neither a result nor its bits -- only
// how many waves share the work (VW = 2: 8 waves of up to 256 VGPRs).
// CH: the head is streamed in column chunks of 16 * KBW blocks (for H > 8192, whose
// activations do not fit the waves' registers at once): for each chunk the waves load that
// chunk's activations, every tile of the block streams that chunk of its rows, and the
// tile's reduced sums are added to its running sums in LDS, chunk after chunk (so a row's
// sums still do not depend on how many rows share the call).
// SPL (with CH): one launch over (tile, chunk) pairs instead -- workgroup (x, y) streams
// chunk y of its tiles and stores that chunk's sums to part[y]; gemv_chunk_reduce then adds
// the chunks in order, as the stage does, so the bits are those of the one-chunk-at-a-time
// launch.  For heads with few tiles (a linear's N), where chunks in turn leave most compute
// units idle.
// TL: the head is tiled (DH_TILED): a tile's 64-column block is RQ KiB in which lane l's
// 16 bytes sit at 16 l, so a wave's load reads 1 KiB of whole lines, with the non-temporal
// hint; rows past V and columns past H are zeros in the tiled copy.  The lanes receive the
// same bytes as from the row-major head, so the sums and their bits are the same.
template <int FMT, int KBW, bool FULL, int TR, int NB, int VW, bool TL, bool CH = false,
          bool SPL = false>
__global__ __launch_bounds__(VW == 1 ? 1024 : 64 * kMaxWaves2) void gemv_kernel(GemvArgs a)
{
    constexpr int RQ = FMT == DH_BF16 ? 2 : 1;   // 16-byte loads per lane per 64 columns
    constexpr int ES = FMT == DH_BF16 ? 2 : 1;   // bytes per weight element
    constexpr int TILE = 16 * TR;                // head rows per tile
    constexpr int OUTS = TILE * 16 * NB;         // (head row, activation row) sums per tile
    constexpr int SST = stage_stride(OUTS);      // floats a tile takes in the stage
    constexpr int KW = VW * KBW;                 // 64-column blocks of one wave
    // blocks a wave keeps in flight: a whole tile (row-major heads), or a window sized so a
    // full workgroup (16 / VW waves) holds about tiled_ahead_kib (tiled heads)
    constexpr int AHW = tiled_ahead_kib<FMT>() * VW / (kMaxWaves * RQ);
    constexpr bool ONE = !CH && NB == 1 && VW == 1 && tiled_one_block<FMT, KW>();
    constexpr int AH = !TL ? (CH ? 4 : KW) : ONE || AHW < 1 ? 1 : AHW > KW ? KW : AHW;
    __shared__ float red[2][kMaxWaves][NB][4 * TR][kWave];   // [virtual wave][act block]
    extern __shared__ float stage[];             // [tile of this block][c][i] (TR == 1)
    __shared__ uint32_t cut_rng[2][16];          // the cut: each row's image range (min, max)
    // FP8 row scale: the row scales of this block's tiles (entry 16 t + i: head row 16 (tile
    // t) + i), loaded at the start -- one a thread, held in a register through the loop --
    // and put in LDS for the writer, when the block's tiles have at most kRscPre rows; else
    // the writer loads them itself (a dependent global load per tile, which cost about
    // 1.5 us at the end of the kernel)
    __shared__ float rsc[FMT == DH_FP8_ROW && (TL || VW * KBW < 8) && !SPL ? kRscPre : 1];

    static_assert(!CH || !FULL, "a chunked launch guards its loads");
    static_assert(!SPL || (CH && NB == 1), "a split launch is a chunked one, up to 16 rows");
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int nw = blockDim.x >> 6;
    if (blockIdx.x == 0)                       // for the kernels that follow on the stream
        for (int i = threadIdx.x; i < a.nzero; i += blockDim.x) {
            a.zero[i * a.zstride] = 0u;
            a.zero[i * a.zstride + 1] = 0u;
        }
    if (threadIdx.x < 32)                      // seen by the writer after the loop's barriers
        cut_rng[threadIdx.x >> 4][threadIdx.x & 15] = threadIdx.x < 16 ? ~0u : 0u;
    const int rr = lane & 15;
    const int g = lane >> 4;
    const int H = a.H;
    const int64_t V = a.V;
    // (not for the row-major 8-block instance, whose registers are full: it spilled)
    constexpr bool RPRE = FMT == DH_FP8_ROW && (TL || KW < 8) && !SPL;
    int ntl = 0;
    bool rpre = false;
    float rsv = 1.0f;
    if constexpr (RPRE) {
        ntl = (a.ntiles - (int)blockIdx.x + (int)gridDim.x - 1) / (int)gridDim.x;
        rpre = ntl * 16 <= (int)blockDim.x && ntl * 16 <= kRscPre;
        const int64_t vr = (int64_t)(blockIdx.x + (threadIdx.x >> 4) * gridDim.x) * TILE +
                           (threadIdx.x & 15);
        if (rpre && (int)(threadIdx.x >> 4) < ntl && vr < V)
            rsv = a.rscale[vr];
    }
    constexpr int CB = kMaxWaves * KBW;          // CH: blocks a chunk
    const int nch = CH ? (a.nkb + CB - 1) / CB : 1;
    int it = 0, buf = 0;
    for (int ch = SPL ? (int)blockIdx.y : 0; ch < (SPL ? (int)blockIdx.y + 1 : nch); ch++) {
    const int cb = CH ? ch * CB : 0;            // the chunk's first 64-column block
    const int nkbc = CH ? (a.nkb - cb < CB ? a.nkb - cb : CB) : a.nkb;
    const int nvw = (nkbc + KBW - 1) / KBW;   // virtual waves: the waves of a 16-row launch

    // This wave's H-slice of the activations: the B operands of every tile.
    bf16x8 xb[NB][KW][2];
#pragma unroll
    for (int nb = 0; nb < NB; nb++)
#pragma unroll
        for (int kb = 0; kb < KW; kb++) {
            const int blk = wave * KW + kb;
            const int k0 = blk * 64 + 16 * g;
            const int row = 16 * nb + rr;
            Pack8 p0, p1;
            p0.q = u32x4{0u, 0u, 0u, 0u};
            p1.q = u32x4{0u, 0u, 0u, 0u};
            if (row < a.R && (FULL || (blk < nkbc && cb * 64 + k0 < H))) {
                const u32x4 *px =
                    reinterpret_cast<const u32x4 *>(a.x + (int64_t)row * H + cb * 64 + k0);
                p0.q = px[0];
                p1.q = px[1];
            }
            xb[nb][kb][0] = p0.v;
            xb[nb][kb][1] = p1.v;
        }

    // One register slot per (group, 64-column block).  A slot is refilled with the next
    // tile's block as soon as its current contents have been widened, so a whole tile of
    // loads stays in flight (through the reduction below) with a single set of registers.
    u32x4 raw[TR][KW][RQ];

    // Buffer loads: descriptors (SGPRs) are rebased on each tile, one per 16-row group, and
    // bounded by the group's existing rows, so rows past V read as zeros (a descriptor of
    // length 0 makes the loads after the last tile empty); a lane's offset within a group
    // is the same for every tile, and a block adds a constant offset.  No load sits under
    // a branch, so the wait before each block is a fixed count of younger loads.
    static_assert(!TL || TR == 1, "a tiled tile is one 16-row group");
    const uint32_t wrow = (uint32_t)H * ES;
    const uint32_t woff =
        TL ? (uint32_t)(16 * lane + (cb + wave * KW) * RQ * 1024)
           : (uint32_t)rr * wrow + (uint32_t)((cb + wave * KW) * 64 + 16 * g) * ES;
    const uint32_t sbase = (uint32_t)(2 * (cb + wave * KW));
    auto load_block = [&](const __amdgpu_buffer_rsrc_t (&wr)[TR], int kb) {
        const int blk = wave * KW + kb;
        // tiled: blocks past the tile read as zeros through the descriptor's bound (a chunk
        // guards the blocks past its own end, which belong to the next chunk)
        if (FULL || (TL && !CH) ||
            (blk < nkbc && (TL || (cb + blk) * 64 + 16 * g < H))) {
#pragma unroll
            for (int r = 0; r < TR; r++)
#pragma unroll
                for (int q = 0; q < RQ; q++)
                    raw[r][kb][q] = __builtin_amdgcn_raw_buffer_load_b128(
                        wr[r], woff, TL ? (kb * RQ + q) * 1024 : kb * 64 * ES + 16 * q,
                        TL ? kCacheNT : kCachePolicy);
        } else {
#pragma unroll
            for (int r = 0; r < TR; r++)
#pragma unroll
                for (int q = 0; q < RQ; q++)
                    raw[r][kb][q] = u32x4{0u, 0u, 0u, 0u};
        }
    };
    // E8M0 scales of a tile: lane i loads byte i of this wave's 2 * KW scale bytes (one
    // load per tile instead of one per block); a block's scale is then read from lane
    // 2 * kb (lanes with g < 2) or 2 * kb + 1 (the second 32 columns).  Bytes past the row
    // read as 0, which only meet zero codes.
    auto load_scales = [&](__amdgpu_buffer_rsrc_t sr) -> uint32_t {
        return FMT == DH_FP8_BLOCK32
                   ? (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(sr, sbase + lane, 0, 0)
                   : 0u;
    };
    auto rsrcs = [&](int tile, bool live, __amdgpu_buffer_rsrc_t (&wr)[TR],
                     __amdgpu_buffer_rsrc_t &sr) {
#pragma unroll
        for (int r = 0; r < TR; r++) {
            if constexpr (TL) {
                wr[r] = __builtin_amdgcn_make_buffer_rsrc(
                    (void *)(a.w + (int64_t)tile * a.tile_bytes), (short)0,
                    live ? a.tile_bytes : 0, kRsrcWord3);
            } else {
                const int64_t v0 = (int64_t)tile * TILE + 16 * r;
                int64_t rows = V - v0 < 16 ? V - v0 : 16;
                rows = rows < 0 || !live ? 0 : rows;
                wr[r] = __builtin_amdgcn_make_buffer_rsrc(
                    (void *)(a.w + (rows ? v0 : 0) * wrow), (short)0, (int)(rows * wrow),
                    kRsrcWord3);
            }
        }
        const uint8_t *p = FMT == DH_FP8_BLOCK32
                               ? a.bscale + (((int64_t)tile * TILE) >> 5) * (H >> 5)
                               : a.w;
        sr = __builtin_amdgcn_make_buffer_rsrc((void *)p, (short)0, live ? (H >> 5) : 0,
                                               kRsrcWord3);
    };

    int tile = blockIdx.x;   // the launch keeps gridDim.x <= ntiles (the same tiles each chunk)
    uint32_t sbytes;
    __amdgpu_buffer_rsrc_t wcur[TR];             // this tile's descriptors
    {
        __amdgpu_buffer_rsrc_t sr;
        rsrcs(tile, true, wcur, sr);
        sbytes = load_scales(sr);
#pragma unroll
        for (int kb = 0; kb < AH; kb++)
            load_block(wcur, kb);
    }
    for (it = 0;; it++) {
        const int next = tile + gridDim.x;
        const bool more = next < a.ntiles;
        __amdgpu_buffer_rsrc_t wr[TR], sr;       // the next tile's descriptors
        rsrcs(more ? next : tile, more, wr, sr);
        const uint32_t sbytes_next = load_scales(sr);

        f32x4 acc[NB][VW][TR];                   // [act block][virtual wave][group]
#pragma unroll
        for (int nb = 0; nb < NB; nb++)
#pragma unroll
            for (int u = 0; u < VW; u++)
#pragma unroll
                for (int r = 0; r < TR; r++)
                    acc[nb][u][r] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < KW; kb++) {
            bf16x8 a0[TR], a1[TR];
#pragma unroll
            for (int r = 0; r < TR; r++) {
                if constexpr (FMT == DH_BF16) {
                    Pack8 p0, p1;
                    p0.q = raw[r][kb][0];
                    p1.q = raw[r][kb][RQ - 1];
                    a0[r] = p0.v;
                    a1[r] = p1.v;
                } else {
                    float scale = 1.0f;
                    if constexpr (FMT == DH_FP8_BLOCK32) {
                        const uint32_t lo = __builtin_amdgcn_readlane(sbytes, 2 * kb);
                        const uint32_t hi = __builtin_amdgcn_readlane(sbytes, 2 * kb + 1);
                        scale = e8m0_scale(g < 2 ? lo : hi);
                    }
                    widen16(raw[r][kb][0], scale, a0[r], a1[r]);
                }
            }
            // the refill: AH blocks ahead, wrapping into the next tile (AH == KW: this slot's
            // block of the next tile)
            if (kb + AH < KW)
                load_block(wcur, kb + AH);
            else
                load_block(wr, kb + AH - KW);
            // keep the refill here: the scheduler would otherwise sink every load below the
            // last MFMA, and the pipeline would drain once per tile
            __builtin_amdgcn_sched_barrier(0);
            const int u = kb / KBW;              // the virtual wave of this block
#pragma unroll
            for (int nb = 0; nb < NB; nb++)
#pragma unroll
                for (int r = 0; r < TR; r++) {
                    acc[nb][u][r] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        a0[r], xb[nb][kb][0], acc[nb][u][r], 0, 0, 0);
                    acc[nb][u][r] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        a1[r], xb[nb][kb][1], acc[nb][u][r], 0, 0, 0);
                }
        }

        // acc[nb][u][r][j] of lane l is the partial sum of head row 16r + 4*(l/16) + j of
        // the tile for activation row 16nb + l%16 over virtual wave VW*wave + u's H-slice.
        // The partials are summed in virtual-wave order and kept in LDS until the end, so
        // the loop issues no stores.
#pragma unroll
        for (int nb = 0; nb < NB; nb++)
#pragma unroll
            for (int u = 0; u < VW; u++)
#pragma unroll
                for (int r = 0; r < TR; r++)
#pragma unroll
                    for (int j = 0; j < 4; j++)
                        red[buf][VW * wave + u][nb][4 * r + j][lane] = acc[nb][u][r][j];
        __syncthreads();
        for (int o = threadIdx.x; o < OUTS; o += blockDim.x) {
            const int r = o / (256 * NB);          // row group
            const int c = (o >> 4) % (16 * NB);    // activation row
            const int i = o & 15;                  // head row within the group
            const int src = (c & 15) + 16 * (i >> 2);
            const int j = 4 * r + (i & 3);
            float s = 0.f;
            for (int w = 0; w < nvw; w++)
                s += red[buf][w][c >> 4][j][src];
            if (CH && !SPL && ch > 0)
                s = stage[it * SST + o] + s;      // the earlier chunks' sums, then this one's
            stage[it * SST + o] = s;
        }
        buf ^= 1;
        if (!more)
            break;
        tile = next;
        sbytes = sbytes_next;
#pragma unroll
        for (int r = 0; r < TR; r++)
            wcur[r] = wr[r];
    }
    }   // chunks
    if constexpr (RPRE)
        if (rpre && (int)threadIdx.x < ntl * 16)
            rsc[threadIdx.x] = rsv;
    __syncthreads();
    if constexpr (SPL) {
        // this chunk's sums of every tile of the block, unscaled, to part[chunk][c][v]
        float *pc = a.part + (int64_t)blockIdx.y * a.R * V;
        for (int t = wave; t <= it; t += nw) {
            const int64_t v0 = (int64_t)(blockIdx.x + t * gridDim.x) * TILE;
            for (int o = lane; o < a.R * 16; o += kWave) {
                const int c = o >> 4, i = o & 15;
                if (v0 + i < V)
                    pc[(int64_t)c * V + v0 + i] = stage[t * SST + c * 16 + i];
            }
        }
        return;
    }
    // it + 1 tiles were done by this block: tile blockIdx.x + t * gridDim.x for t <= it.  Wave
    // w writes tiles w, w + nw, ...; a lane takes (activation row c, head row i) pairs.
    static_assert(TR == 1, "the writer below assumes one 16-row group per tile");
    const bool cut = a.cut_m > 0 && NB == 1 && (int)gridDim.x <= kCutMaxChunks &&
                     (int)gridDim.x * a.cut_slots <= a.cut_max;
    // from nw / 2 rows up every wave owns whole rows: it writes and cuts them alone
    if (cut && (a.R << 1) > nw) {
        static_assert(sizeof(red) >= 16 * 256 * sizeof(uint32_t) + 256, "the cut's LDS fits");
        write_cut_own_rows<SST>(a, stage, it + 1, reinterpret_cast<uint32_t *>(&red[0][0][0][0][0]),
                                rpre ? rsc : nullptr);
        return;
    }
    const int per_tile = a.R * 16;
    // the cut: the images' range of activation rows 4 q + lane / 16, q < 4, as they are written
    uint32_t rmn[4] = {~0u, ~0u, ~0u, ~0u}, rmx[4] = {0u, 0u, 0u, 0u};
    for (int t = wave; t <= it; t += nw) {
        const int64_t v0 = (int64_t)(blockIdx.x + t * gridDim.x) * TILE;
        // a lane's head row is v0 + lane % 16 for every activation row it writes, so its row
        // scale is loaded once, before the stores (which the compiler may not move it past)
        const int64_t vl = v0 + (lane & 15);
        const float rs = rpre ? rsc[t * 16 + (lane & 15)]
                              : a.rscale && vl < V ? a.rscale[vl] : 1.0f;
#pragma unroll
        for (int q = 0; q < 32 * 16 / kWave; q++) {
            const int o = lane + kWave * q;
            const int c = o >> 4, i = o & 15;
            const int64_t v = v0 + i;
            if (o < per_tile) {
                float *sp = &stage[t * SST + c * 16 + i];
                uint32_t im = 0;
                if (v < V) {
                    const float s = a.rscale ? *sp * rs : *sp;   // row_scaled
                    store_out(a, c, v, s);
                    im = order_key(s);               // the cut ranks the logits as written
                }
                if (cut && q < 4) {
                    // the slot keeps the image (0 past the head's rows) for the cut
                    *reinterpret_cast<uint32_t *>(sp) = im;
                    rmn[q & 3] = im != 0 && im < rmn[q & 3] ? im : rmn[q & 3];
                    rmx[q & 3] = im > rmx[q & 3] ? im : rmx[q & 3];
                }
            }
        }
    }
    if (cut) {
        // each row's range over its 16 lanes (lane 15 of a row of lanes ends with it), then
        // over the waves
#pragma unroll
        for (int q = 0; q < 4; q++) {
            row_min_max32(rmn[q], rmx[q]);
            const int c = 4 * q + (lane >> 4);
            if ((lane & 15) == 15 && c < a.R) {
                atomicMin(&cut_rng[0][c], rmn[q]);
                atomicMax(&cut_rng[1][c], rmx[q]);
            }
        }
        // the cut's LDS in the reduction buffer, which is free now
        static_assert(sizeof(red) >= 16 * 256 * sizeof(uint32_t) + 256, "the cut's LDS fits");
        uint32_t *cws = reinterpret_cast<uint32_t *>(&red[0][0][0][0][0]);
        cut_init(cws);
        lds_barrier();                               // the scaled sums, ranges, the cut's LDS
        cut_rows<SST>(a, reinterpret_cast<const uint32_t *>(stage), it + 1, cws, &cut_rng[0][0]);
    }
}

// Few tiles (a linear with few output rows): the streaming kernel would leave most compute
// units idle, so the work is split by virtual wave instead.  One wave per (tile, virtual
// wave v) computes the same MFMA chain over the same kbw blocks as virtual wave v of the
// streaming kernel and stores its 16 x 16 (or 16 x 32) partial to part[v][c][head row];
// gemv_reduce then adds the partials in virtual-wave order, starting from 0, exactly as the
// streaming kernel's reduction does -- the same sums, the same bits.
constexpr int kSplitMaxKbw = 8;

template <int FMT, int NB, bool TL>
__global__ __launch_bounds__(kWave) void gemv_split(GemvArgs a, int kbw, float *part)
{
    constexpr int RQ = FMT == DH_BF16 ? 2 : 1;
    constexpr int ES = FMT == DH_BF16 ? 2 : 1;
    const int lane = threadIdx.x, rr = lane & 15, g = lane >> 4;
    const int tile = blockIdx.x, vw = blockIdx.y;
    const int H = a.H;
    const int64_t V = a.V;
    const int64_t v0 = (int64_t)tile * 16;
    const int64_t rows = V - v0 < 16 ? V - v0 : 16;
    const uint32_t wrow = (uint32_t)H * ES;
    const __amdgpu_buffer_rsrc_t wr =
        TL ? __builtin_amdgcn_make_buffer_rsrc((void *)(a.w + (int64_t)tile * a.tile_bytes),
                                               (short)0, a.tile_bytes, kRsrcWord3)
           : __builtin_amdgcn_make_buffer_rsrc((void *)(a.w + v0 * wrow), (short)0,
                                               (int)(rows * wrow), kRsrcWord3);
    // every load first (a block past the row or an activation row past R is zero)
    u32x4 raw[kSplitMaxKbw][RQ];
    Pack8 xq[NB][kSplitMaxKbw][2];
    uint32_t sb[kSplitMaxKbw];
#pragma unroll
    for (int kb = 0; kb < kSplitMaxKbw; kb++) {
        const int blk = vw * kbw + kb;
        const int k0 = blk * 64 + 16 * g;
        const bool in = kb < kbw && blk < a.nkb && k0 < H;
#pragma unroll
        for (int q = 0; q < RQ; q++)
            raw[kb][q] = in ? __builtin_amdgcn_raw_buffer_load_b128(
                                  wr,
                                  TL ? (uint32_t)((blk * RQ + q) * 1024 + 16 * lane)
                                     : (uint32_t)rr * wrow + (uint32_t)k0 * ES + 16 * q,
                                  0, TL ? kCacheNT : kCachePolicy)
                            : u32x4{0u, 0u, 0u, 0u};
        sb[kb] = FMT == DH_FP8_BLOCK32 && in
                     ? a.bscale[(v0 >> 5) * (H >> 5) + 2 * blk + (g >= 2 ? 1 : 0)]
                     : 0u;
#pragma unroll
        for (int nb = 0; nb < NB; nb++) {
            const int row = 16 * nb + rr;
            xq[nb][kb][0].q = u32x4{0u, 0u, 0u, 0u};
            xq[nb][kb][1].q = u32x4{0u, 0u, 0u, 0u};
            if (in && row < a.R) {
                const u32x4 *px = reinterpret_cast<const u32x4 *>(a.x + (int64_t)row * H + k0);
                xq[nb][kb][0].q = px[0];
                xq[nb][kb][1].q = px[1];
            }
        }
    }
    f32x4 acc[NB];
#pragma unroll
    for (int nb = 0; nb < NB; nb++)
        acc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < kSplitMaxKbw; kb++) {
        if (kb >= kbw)
            break;
        bf16x8 a0, a1;
        if constexpr (FMT == DH_BF16) {
            Pack8 p0, p1;
            p0.q = raw[kb][0];
            p1.q = raw[kb][RQ - 1];
            a0 = p0.v;
            a1 = p1.v;
        } else {
            widen16(raw[kb][0], FMT == DH_FP8_BLOCK32 ? e8m0_scale(sb[kb]) : 1.0f, a0, a1);
        }
#pragma unroll
        for (int nb = 0; nb < NB; nb++) {
            acc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, xq[nb][kb][0].v, acc[nb], 0, 0, 0);
            acc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, xq[nb][kb][1].v, acc[nb], 0, 0, 0);
        }
    }
    // acc[nb][j]: head row 4 * (lane / 16) + j, activation row 16 nb + lane % 16
#pragma unroll
    for (int nb = 0; nb < NB; nb++) {
        const int c = 16 * nb + rr;
        if (c >= a.R)
            continue;
#pragma unroll
        for (int j = 0; j < 4; j++) {
            const int64_t v = v0 + 4 * g + j;
            if (v < V)
                part[((int64_t)vw * a.R + c) * V + v] = acc[nb][j];
        }
    }
}

__global__ __launch_bounds__(256) void gemv_reduce(GemvArgs a, int nvw, const float *part)
{
    const int64_t n = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (n >= (int64_t)a.R * a.V)
        return;
    const int c = (int)(n / a.V);
    const int64_t v = n - (int64_t)c * a.V;
    // nvw <= kMaxWaves: every partial's load is in flight before the first add
    float p[kMaxWaves];
#pragma unroll
    for (int w = 0; w < kMaxWaves; w++)
        p[w] = w < nvw ? part[((int64_t)w * a.R + c) * a.V + v] : 0.f;
    float s = 0.f;
#pragma unroll
    for (int w = 0; w < kMaxWaves; w++)
        if (w < nvw)
            s += p[w];
    write_out(a, c, v, s);
}

// The split chunked launch's sums: for each (row c, head row v), part[0] + part[1] + ... in
// chunk order (the stage's order in the one-launch form), then the row scale and the output
// mode, as the writer applies them.
__global__ __launch_bounds__(256) void gemv_chunk_reduce(GemvArgs a, int nch, const float *part)
{
    const int64_t n = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t rv = (int64_t)a.R * a.V;
    if (n >= rv)
        return;
    const int c = (int)(n / a.V);
    const int64_t v = n - (int64_t)c * a.V;
    float s = part[n];
    for (int ch = 1; ch < nch; ch++)
        s = s + part[(int64_t)ch * rv + n];
    write_out(a, c, v, s);
}

template <int FMT, int KBW, bool FULL, int TR, int NB, int VW, bool TL, bool CH = false>
hipError_t run(GemvArgs a, hipStream_t stream, int *grid_used)
{
    static int occ_cache[kMaxWaves + 1];
    static int lds_set[kMaxDevices];               // per device: the LDS limit has been raised
    const int nkb = CH && a.nkb > kMaxWaves * KBW ? kMaxWaves * KBW : a.nkb;   // blocks a pass
    const int nw = (nkb + VW * KBW - 1) / (VW * KBW);
    const int block = nw * kWave;
    auto kern = gemv_kernel<FMT, KBW, FULL, TR, NB, VW, TL, CH>;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return e;
    if (dev < 0 || dev >= kMaxDevices)
        return hipErrorInvalidDevice;
    if (!__atomic_load_n(&lds_set[dev], __ATOMIC_RELAXED)) {
        e = hipFuncSetAttribute((const void *)kern, hipFuncAttributeMaxDynamicSharedMemorySize,
                                kMaxStageBytes);
        if (e != hipSuccess)
            return e;
        __atomic_store_n(&lds_set[dev], 1, __ATOMIC_RELAXED);
    }
    a.ntiles = (int)((a.V + 16 * TR - 1) / (16 * TR));
    const int occ = occupancy(kern, block, occ_cache[nw]);
    int64_t grid = (int64_t)device_cus() * occ;
    // each block keeps its tiles' logits in LDS: at most kMaxStageBytes of them
    const int64_t max_per = kMaxStageBytes / (stage_stride(TR * 256 * NB) * (int)sizeof(float));
    const int64_t min_grid = (a.ntiles + max_per - 1) / max_per;
    if (grid < min_grid)
        grid = min_grid;
    if (grid > a.ntiles)
        grid = a.ntiles;
    // the draft's cut: at most as many workgroups as the merge takes cuts of (a small-H GEMV
    // runs several workgroups a compute unit; rank 512, 16 rows: 1024 of them left the top-k
    // to a launch of its own, and capping them at 512 took 58.7 us a draft against 62.5)
    if (a.cut_m > 0 && NB == 1) {
        int64_t cap = a.cut_max / a.cut_slots;
        cap = cap < kCutMaxChunks ? cap : kCutMaxChunks;
        if (grid > cap && cap >= min_grid)
            grid = cap;
    }
    const int64_t per = (a.ntiles + grid - 1) / grid;
    if (grid_used)
        *grid_used = (int)grid;
    return launch(kern, dim3((unsigned)grid), dim3(block),
                  (size_t)per * stage_stride(TR * 256 * NB) * sizeof(float), stream, a);
}

template <int FMT, int KBW, int NB, int VW, bool TL>
hipError_t run_kbw(const GemvArgs &a, hipStream_t stream, int *grid_used)
{
    constexpr int TR = 1;   // two groups measured slower: the loop is not latency-bound
    if (a.H % 64 == 0 && a.nkb % (VW * KBW) == 0)
        return run<FMT, KBW, true, TR, NB, VW, TL>(a, stream, grid_used);
    return run<FMT, KBW, false, TR, NB, VW, TL>(a, stream, grid_used);
}

// grid_used: the grid of the (last) launch.
template <int FMT, bool TL>
hipError_t run_fmt(const GemvArgs &a, hipStream_t stream, int *grid_used)
{
    const int kbw = (a.nkb + kMaxWaves - 1) / kMaxWaves;   // the 16-row split, for any R
    if (a.R > 16) {
        switch (kbw) {
        case 1: return run_kbw<FMT, 1, 2, 2, TL>(a, stream, grid_used);
        case 2: return run_kbw<FMT, 2, 2, 2, TL>(a, stream, grid_used);
        case 3: return run_kbw<FMT, 3, 2, 2, TL>(a, stream, grid_used);
        case 4: return run_kbw<FMT, 4, 2, 2, TL>(a, stream, grid_used);
        // H <= 5120: 32 rows of activations fill 160 of a wave's 256 VGPRs, which still leaves
        // room (218-246 VGPRs in all) except for the row-major bf16 tile, which spills
        case 5:
            if constexpr (FMT != DH_BF16 || TL)
                return run_kbw<FMT, 5, 2, 2, TL>(a, stream, grid_used);
            [[fallthrough]];
        default: {
            // wider heads: 32 rows of activations do not fit the registers, so rows 0..15 and
            // 16.. take a launch each (the weights are read twice; every row keeps its bits)
            GemvArgs lo = a, hi = a;
            lo.R = 16;
            hi.R = a.R - 16;
            hi.x = a.x + (int64_t)16 * a.H;
            const int64_t skip = (int64_t)16 * a.V;
            hi.logits = a.logits ? a.logits + skip : nullptr;
            hi.out16 = a.out16 ? a.out16 + skip : nullptr;
            hi.residual = a.residual ? a.residual + skip : nullptr;
            const hipError_t e = run_fmt<FMT, TL>(lo, stream, grid_used);
            return e != hipSuccess ? e : run_fmt<FMT, TL>(hi, stream, grid_used);
        }
        }
    }
    switch (kbw) {
    case 1: return run_kbw<FMT, 1, 1, 1, TL>(a, stream, grid_used);
    case 2: return run_kbw<FMT, 2, 1, 1, TL>(a, stream, grid_used);
    case 3: return run_kbw<FMT, 3, 1, 1, TL>(a, stream, grid_used);
    case 4: return run_kbw<FMT, 4, 1, 1, TL>(a, stream, grid_used);
    // a bf16 tile of 5 blocks a wave does not fit 16 waves' 128 VGPRs next to the
    // activations (8 spilled); 8 waves of two virtual waves each (the same bits) fit and
    // measured 3.6% faster at H = 5120.  Wider bf16 tiles spill either way, FP8 tiles fit.
    case 5:
        if (FMT == DH_BF16)
            return run_kbw<FMT, 5, 1, 2, TL>(a, stream, grid_used);
        return run_kbw<FMT, 5, 1, 1, TL>(a, stream, grid_used);
    case 6: return run_kbw<FMT, 6, 1, 1, TL>(a, stream, grid_used);
    case 7: return run_kbw<FMT, 7, 1, 1, TL>(a, stream, grid_used);
    case 8: return run_kbw<FMT, 8, 1, 1, TL>(a, stream, grid_used);
    default:   // H > 8192: column chunks
        if constexpr (TL)
            return run<FMT, kChunkKbw, false, 1, 1, 1, true, true>(a, stream, grid_used);
        else
            return run<FMT, kChunkKbw, false, 1, 1, 2, false, true>(a, stream, grid_used);
    }
}

}  // namespace

hipError_t launch_gemv(const dh_head &head, const uint16_t *x, int rows, float *logits,
                       hipStream_t stream, uint32_t *zero, int nzero, int zstride,
                       const GemvCut *cut, int *grid_used)
{
    return launch_linear(head, x, rows, DH_OUT_F32, nullptr, logits, stream, nullptr, 0, zero,
                         nzero, zstride, cut, grid_used);
}

size_t linear_split_bytes(int64_t vocab, int64_t hidden, int rows)
{
    const int nkb = (int)((hidden + 63) / 64);
    const int kbw = (nkb + kMaxWaves - 1) / kMaxWaves;
    const int nvw = (nkb + kbw - 1) / kbw;
    return (size_t)nvw * (size_t)rows * (size_t)vocab * sizeof(float);
}

// The split chunked launch's partials: one fp32 [R][V] a column chunk.
static size_t chunk_split_bytes(int64_t vocab, int64_t hidden, int rows)
{
    constexpr int CB = kMaxWaves * kChunkKbw;
    const int64_t nch = ((hidden + 63) / 64 + CB - 1) / CB;
    return (size_t)nch * (size_t)rows * (size_t)vocab * sizeof(float);
}

size_t linear_ws_bytes(int64_t vocab, int64_t hidden, int rows)
{
    const size_t a = linear_split_bytes(vocab, hidden, rows);
    const size_t b = chunk_split_bytes(vocab, hidden, rows);
    return a > b ? a : b;
}

template <int FMT, bool TL>
hipError_t run_split(const GemvArgs &a, float *part, hipStream_t stream)
{
    const int kbw = (a.nkb + kMaxWaves - 1) / kMaxWaves;
    const int nvw = (a.nkb + kbw - 1) / kbw;
    const int ntiles = (int)((a.V + 15) / 16);
    hipError_t e =
        a.R > 16
            ? launch(gemv_split<FMT, 2, TL>, dim3(ntiles, nvw), dim3(kWave), 0, stream, a, kbw, part)
            : launch(gemv_split<FMT, 1, TL>, dim3(ntiles, nvw), dim3(kWave), 0, stream, a, kbw, part);
    if (e != hipSuccess)
        return e;
    const int64_t n = (int64_t)a.R * a.V;
    return launch(gemv_reduce, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, a, nvw,
                  (const float *)part);
}

template <int FMT, bool TL>
hipError_t run_chunk_split(GemvArgs a, float *part, hipStream_t stream)
{
    constexpr int VW = TL ? 1 : 2;                 // as the one-chunk-at-a-time launch
    constexpr int CB = kMaxWaves * kChunkKbw;
    a.ntiles = (int)((a.V + 15) / 16);
    a.part = part;
    const int nch = (a.nkb + CB - 1) / CB;
    // about one workgroup per compute unit in all: each keeps its chunk's activations and
    // streams several tiles, one ahead of the other (a workgroup per (tile, chunk) pays the
    // start of a stream for each 128 KiB tile)
    int gx = device_cus() / nch;
    gx = gx < 1 ? 1 : gx > a.ntiles ? a.ntiles : gx;
    const int per = (a.ntiles + gx - 1) / gx;
    hipError_t e = launch(gemv_kernel<FMT, kChunkKbw, false, 1, 1, VW, TL, true, true>,
                          dim3((unsigned)gx, (unsigned)nch), dim3(kMaxWaves / VW * kWave),
                          (size_t)per * stage_stride(256) * sizeof(float), stream, a);
    if (e != hipSuccess)
        return e;
    const int64_t n = (int64_t)a.R * a.V;
    return launch(gemv_chunk_reduce, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, a,
                  nch, (const float *)part);
}

hipError_t launch_linear(const dh_head &head, const uint16_t *x, int rows, int mode,
                         const uint16_t *residual, void *out, hipStream_t stream,
                         void *scratch, size_t scratch_bytes, uint32_t *zero, int nzero,
                         int zstride, const GemvCut *cut, int *grid_used)
{
    const int fmt = head.format & ~DH_TILED;
    GemvArgs a;
    a.w = static_cast<const uint8_t *>(head.weight);
    a.bscale = fmt == DH_FP8_BLOCK32 ? static_cast<const uint8_t *>(head.scale) : nullptr;
    a.rscale = fmt == DH_FP8_ROW ? static_cast<const float *>(head.scale) : nullptr;
    a.x = x;
    a.logits = mode == DH_OUT_F32 ? static_cast<float *>(out) : nullptr;
    a.out16 = mode == DH_OUT_F32 ? nullptr : static_cast<uint16_t *>(out);
    a.residual = mode == DH_OUT_ADD_BF16 ? residual : nullptr;
    a.mode = mode;
    a.V = head.vocab;
    a.H = (int)head.hidden;
    a.R = rows;
    a.ntiles = 0;   // set per tile height by run()
    a.nkb = (int)((head.hidden + 63) / 64);
    a.tile_bytes = a.nkb * 1024 * (fmt == DH_BF16 ? 2 : 1);
    a.zero = zero;
    a.nzero = zero ? nzero : 0;
    a.zstride = zstride;
    const bool with_cut = cut && mode == DH_OUT_F32 && rows <= 16;
    a.cut_keys = with_cut ? cut->keys : nullptr;
    a.cut_floors = with_cut ? cut->floors : nullptr;
    a.cut_m = with_cut ? cut->m : 0;
    a.cut_slots = with_cut ? cut->slots : 0;
    a.cut_max = with_cut ? cut->max_keys : 0;
    a.part = nullptr;
    if (grid_used)
        *grid_used = 0;
    // few tiles and room for the partials: split by virtual wave (the same bits)
    const int64_t ntiles = (a.V + 15) / 16;
    if (scratch && ntiles <= device_cus() / 2 && (a.nkb + kMaxWaves - 1) / kMaxWaves <= kSplitMaxKbw &&
        scratch_bytes >= linear_split_bytes(a.V, head.hidden, rows)) {
        float *part = static_cast<float *>(scratch);
        switch (head.format) {
        case DH_BF16: return run_split<DH_BF16, false>(a, part, stream);
        case DH_FP8_BLOCK32: return run_split<DH_FP8_BLOCK32, false>(a, part, stream);
        case DH_FP8_ROW: return run_split<DH_FP8_ROW, false>(a, part, stream);
        case DH_BF16 | DH_TILED: return run_split<DH_BF16, true>(a, part, stream);
        case DH_FP8_BLOCK32 | DH_TILED: return run_split<DH_FP8_BLOCK32, true>(a, part, stream);
        case DH_FP8_ROW | DH_TILED: return run_split<DH_FP8_ROW, true>(a, part, stream);
        default: return hipErrorInvalidValue;
        }
    }
    // wider than a chunk, few tiles and room for the chunks' partials: every (tile, chunk)
    // at once, then their sum in chunk order (the same bits); N = 5120, K = 18,432: 320 tiles
    // of 3 chunks in turn left most compute units idle
    constexpr int kCB = kMaxWaves * kChunkKbw;
    const int64_t nch = (a.nkb + kCB - 1) / kCB;
    if (scratch && !with_cut && rows <= 16 && nch > 1 && ntiles * nch <= 4 * device_cus() &&
        scratch_bytes >= chunk_split_bytes(a.V, head.hidden, rows)) {
        float *part = static_cast<float *>(scratch);
        switch (head.format) {
        case DH_BF16: return run_chunk_split<DH_BF16, false>(a, part, stream);
        case DH_FP8_BLOCK32: return run_chunk_split<DH_FP8_BLOCK32, false>(a, part, stream);
        case DH_FP8_ROW: return run_chunk_split<DH_FP8_ROW, false>(a, part, stream);
        case DH_BF16 | DH_TILED: return run_chunk_split<DH_BF16, true>(a, part, stream);
        case DH_FP8_BLOCK32 | DH_TILED: return run_chunk_split<DH_FP8_BLOCK32, true>(a, part, stream);
        case DH_FP8_ROW | DH_TILED: return run_chunk_split<DH_FP8_ROW, true>(a, part, stream);
        default: return hipErrorInvalidValue;
        }
    }
    switch (head.format) {
    case DH_BF16: return run_fmt<DH_BF16, false>(a, stream, grid_used);
    case DH_FP8_BLOCK32: return run_fmt<DH_FP8_BLOCK32, false>(a, stream, grid_used);
    case DH_FP8_ROW: return run_fmt<DH_FP8_ROW, false>(a, stream, grid_used);
    case DH_BF16 | DH_TILED: return run_fmt<DH_BF16, true>(a, stream, grid_used);
    case DH_FP8_BLOCK32 | DH_TILED: return run_fmt<DH_FP8_BLOCK32, true>(a, stream, grid_used);
    case DH_FP8_ROW | DH_TILED: return run_fmt<DH_FP8_ROW, true>(a, stream, grid_used);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace dh
