// The C ABI (include/dh.h): host-side checks, then the launches.  Every refusal happens
// before anything is enqueued, so a refused call leaves the outputs untouched -- the pages'
// stance of refusing a larger span rather than clipping it ("dsv41 Zig: the TFE draft head
// (TF_DS_DRAFTER=eagle), off by default", commit notes on absorb and the review thread).
#include <atomic>
#include <initializer_list>
#include <mutex>
#include <stdint.h>

#include "dh_internal.h"
#include "topk.h"

namespace dh {

int device_cus()
{
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0)
        dev = 0;
    const int slot = dev < 64 ? dev : 63;
    int n = cache[slot].load(std::memory_order_relaxed);
    if (n > 0 && dev < 64)
        return n;
    n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n < 1)
        n = 256;
    if (dev < 64)
        cache[slot].store(n, std::memory_order_relaxed);
    return n;
}

}  // namespace dh

namespace {

using dh::TopkWs;

bool aligned(const void *p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

struct Span {
    uintptr_t lo, hi;
};

Span span(const void *p, size_t bytes) { return Span{(uintptr_t)p, (uintptr_t)p + bytes}; }

bool overlap(Span a, Span b) { return a.lo < b.hi && b.lo < a.hi && a.lo != a.hi && b.lo != b.hi; }

size_t elem_bytes(int format) { return (format & ~DH_TILED) == DH_BF16 ? 2 : 1; }

// The storage format without the layout modifier.
int base_format(int format) { return format & ~DH_TILED; }

bool known_format(int format)
{
    const int f = base_format(format);
    return (format & ~(DH_TILED | 3)) == 0 &&
           (f == DH_BF16 || f == DH_FP8_BLOCK32 || f == DH_FP8_ROW);
}

size_t scale_bytes(const dh_head &h)
{
    if (base_format(h.format) == DH_FP8_BLOCK32)
        return (size_t)((h.vocab + 31) / 32) * (size_t)(h.hidden / 32);
    if (base_format(h.format) == DH_FP8_ROW)
        return (size_t)h.vocab * sizeof(float);
    return 0;
}

dh_status check_head(const dh_head *h)
{
    if (!h || !h->weight)
        return DH_ERR_INVALID;
    if (!known_format(h->format))
        return DH_ERR_INVALID;
    if (h->vocab < 1 || h->hidden < 32 || h->hidden % 32 != 0)
        return DH_ERR_INVALID;
    if (h->hidden > DH_MAX_HIDDEN || h->vocab > ((int64_t)1 << 25))
        return DH_ERR_UNSUPPORTED;
    if (!aligned(h->weight, 16))
        return DH_ERR_INVALID;
    if (base_format(h->format) == DH_BF16) {
        if (h->scale)
            return DH_ERR_INVALID;
    } else {
        if (!h->scale)
            return DH_ERR_INVALID;
        if (base_format(h->format) == DH_FP8_ROW && !aligned(h->scale, 4))
            return DH_ERR_INVALID;
    }
    return DH_OK;
}

// A head whose weight must be row-major (a rescore's dense head, a gather's source).
dh_status check_row_major(const dh_head *h)
{
    const dh_status st = check_head(h);
    if (st != DH_OK)
        return st;
    return (h->format & DH_TILED) ? DH_ERR_INVALID : DH_OK;
}

Span head_weight(const dh_head &h)
{
    if (h.format & DH_TILED)
        return span(h.weight, dh::tiled_bytes(h.format, h.vocab, h.hidden));
    return span(h.weight, (size_t)h.vocab * (size_t)h.hidden * elem_bytes(h.format));
}

Span head_scale(const dh_head &h) { return span(h.scale, scale_bytes(h)); }

dh_status check_rows(int32_t rows)
{
    if (rows < 1)
        return DH_ERR_INVALID;
    if (rows > DH_MAX_ROWS)
        return DH_ERR_UNSUPPORTED;
    return DH_OK;
}

dh_status check_gemv_rows(int32_t rows, int64_t hidden)
{
    (void)hidden;   // above 16 rows a wide head takes two launches
    return check_rows(rows);
}

dh_status check_k(int32_t k, int64_t vocab)
{
    if (k < 1 || k > vocab)
        return DH_ERR_INVALID;
    if (k > DH_MAX_K)
        return DH_ERR_UNSUPPORTED;
    return DH_OK;
}

dh_status device_status(hipError_t e) { return e == hipSuccess ? DH_OK : DH_ERR_DEVICE; }

#define DH_TRY(expr)                        \
    do {                                    \
        const dh_status s_ = (expr);        \
        if (s_ != DH_OK)                    \
            return s_;                      \
    } while (0)

}  // namespace

namespace {

// The fixed scratch of dh_draft_noalloc: one array per GPU, made when the library's code is
// loaded on that GPU and held until the process ends.  In host code `scratch` names a
// host-side stand-in, not device memory: host code only ever uses the device address that
// hipGetSymbolAddress gives for the current device (scratch_address).
__device__ __align__(256) unsigned char scratch[DH_NOALLOC_SCRATCH_BYTES];

constexpr int kScratchDevices = 64;
std::mutex scratch_mu;
void *scratch_at[kScratchDevices];   // device address of `scratch` per device, once looked up

// The current device's copy of `scratch` (looked up on the first call on that device, with
// that device current), or NULL if the runtime cannot give it.
void *scratch_address()
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kScratchDevices)
        return nullptr;
    std::lock_guard<std::mutex> g(scratch_mu);
    if (!scratch_at[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p)
            return nullptr;
        scratch_at[dev] = p;
    }
    return scratch_at[dev];
}

}  // namespace

extern "C" {

dh_status dh_gemv(const dh_head *head, const uint16_t *x, int32_t rows, float *logits,
                  void *stream)
{
    DH_TRY(check_head(head));
    DH_TRY(check_gemv_rows(rows, head->hidden));
    if (!x || !logits || !aligned(x, 16) || !aligned(logits, 4))
        return DH_ERR_INVALID;
    const Span out = span(logits, (size_t)rows * (size_t)head->vocab * sizeof(float));
    if (overlap(out, head_weight(*head)) || overlap(out, head_scale(*head)) ||
        overlap(out, span(x, (size_t)rows * (size_t)head->hidden * 2)))
        return DH_ERR_INVALID;
    return device_status(dh::launch_gemv(*head, x, rows, logits, (hipStream_t)stream));
}

static dh_status check_linear(const dh_head *w, const uint16_t *x, int32_t rows, int32_t mode,
                              const uint16_t *residual, void *out)
{
    DH_TRY(check_head(w));
    DH_TRY(check_gemv_rows(rows, w->hidden));
    if (mode != DH_OUT_F32 && mode != DH_OUT_BF16 && mode != DH_OUT_ADD_BF16)
        return DH_ERR_INVALID;
    const size_t ob = mode == DH_OUT_F32 ? 4 : 2;
    if (!x || !out || !aligned(x, 16) || !aligned(out, ob))
        return DH_ERR_INVALID;
    if ((mode == DH_OUT_ADD_BF16) != (residual != nullptr) || (residual && !aligned(residual, 2)))
        return DH_ERR_INVALID;
    const Span so = span(out, (size_t)rows * (size_t)w->vocab * ob);
    if (overlap(so, head_weight(*w)) || overlap(so, head_scale(*w)) ||
        overlap(so, span(x, (size_t)rows * (size_t)w->hidden * 2)))
        return DH_ERR_INVALID;
    if (residual && (const void *)residual != out && overlap(so, span(residual, so.hi - so.lo)))
        return DH_ERR_INVALID;
    return DH_OK;
}

dh_status dh_linear(const dh_head *w, const uint16_t *x, int32_t rows, int32_t mode,
                    const uint16_t *residual, void *out, void *stream)
{
    DH_TRY(check_linear(w, x, rows, mode, residual, out));
    return device_status(
        dh::launch_linear(*w, x, rows, mode, residual, out, (hipStream_t)stream));
}

size_t dh_linear_workspace_bytes(int32_t rows, int64_t n, int64_t k)
{
    if (check_rows(rows) != DH_OK || n < 1 || n > DH_MAX_GEMV_VOCAB || k < 32 || k % 32 != 0 ||
        k > DH_MAX_HIDDEN)
        return 0;
    const size_t b = dh::linear_ws_bytes(n, k, rows);
    return (b + 255) & ~(size_t)255;
}

dh_status dh_linear_ws(const dh_head *w, const uint16_t *x, int32_t rows, int32_t mode,
                       const uint16_t *residual, void *out, void *workspace,
                       size_t workspace_bytes, void *stream)
{
    DH_TRY(check_linear(w, x, rows, mode, residual, out));
    const size_t need = dh_linear_workspace_bytes(rows, w->vocab, w->hidden);
    if (!workspace || !aligned(workspace, 256) || workspace_bytes < need)
        return DH_ERR_WORKSPACE;
    const size_t ob = mode == DH_OUT_F32 ? 4 : 2;
    const Span sw = span(workspace, need);
    const Span others[] = {span(out, (size_t)rows * (size_t)w->vocab * ob), head_weight(*w),
                           head_scale(*w), span(x, (size_t)rows * (size_t)w->hidden * 2),
                           span(residual, residual ? (size_t)rows * (size_t)w->vocab * 2 : 0)};
    for (const Span &o : others)
        if (overlap(sw, o))
            return DH_ERR_INVALID;
    return device_status(dh::launch_linear(*w, x, rows, mode, residual, out, (hipStream_t)stream,
                                           workspace, workspace_bytes));
}

size_t dh_workspace_bytes(int32_t rows, int64_t vocab, int32_t k)
{
    if (check_rows(rows) != DH_OK || vocab < 1 || vocab > DH_MAX_VOCAB ||
        check_k(k, vocab) != DH_OK)
        return 0;
    const TopkWs w = dh::topk_ws_layout(rows, vocab, k);
    const size_t logits = (size_t)rows * (size_t)vocab * sizeof(float);
    return w.bytes + ((logits + 255) & ~(size_t)255);
}

// own_scratch: the workspace is the library's fixed scratch (dh_draft_noalloc), which no
// caller buffer can overlap; `workspace` is then NULL, and so is `logits` when the logits
// are to live in that scratch.
static dh_status check_topk(const float *logits, int32_t rows, int64_t vocab, int32_t k,
                            int32_t *ids, float *vals, int32_t *argmax, void *workspace,
                            size_t workspace_bytes, bool own_scratch = false)
{
    DH_TRY(check_rows(rows));
    if (vocab < 1)
        return DH_ERR_INVALID;
    if (vocab > DH_MAX_VOCAB)
        return DH_ERR_UNSUPPORTED;
    DH_TRY(check_k(k, vocab));
    if ((!logits && !own_scratch) || !ids || !vals || !aligned(logits, 4) ||
        !aligned(ids, 4) || !aligned(vals, 4) || (argmax && !aligned(argmax, 4)))
        return DH_ERR_INVALID;
    if (!own_scratch && (!workspace || !aligned(workspace, 256) ||
                         workspace_bytes < dh::topk_ws_layout(rows, vocab, k).bytes))
        return DH_ERR_WORKSPACE;
    const Span in = span(logits, logits ? (size_t)rows * (size_t)vocab * sizeof(float) : 0);
    const Span si = span(ids, (size_t)rows * k * 4), sv = span(vals, (size_t)rows * k * 4);
    const Span sa = span(argmax, argmax ? (size_t)rows * 4 : 0);
    const Span sw = span(workspace, own_scratch ? 0 : dh::topk_ws_layout(rows, vocab, k).bytes);
    if (overlap(in, si) || overlap(in, sv) || overlap(in, sa) || overlap(si, sv) ||
        overlap(si, sa) || overlap(sv, sa) || overlap(sw, in) || overlap(sw, si) ||
        overlap(sw, sv) || overlap(sw, sa))
        return DH_ERR_INVALID;
    return DH_OK;
}

dh_status dh_topk(const float *logits, int32_t rows, int64_t vocab, int32_t k, int32_t *ids,
                  float *vals, int32_t *argmax, void *workspace, size_t workspace_bytes,
                  void *stream)
{
    DH_TRY(check_topk(logits, rows, vocab, k, ids, vals, argmax, workspace, workspace_bytes));
    return device_status(dh::launch_topk(logits, rows, vocab, k, nullptr, ids, vals, argmax,
                                         workspace, (hipStream_t)stream));
}

dh_status dh_topk_softmax(const float *logits, int32_t rows, int64_t vocab, int32_t k,
                          int32_t *ids, float *vals, int32_t *argmax, float *probs, float *lse,
                          void *workspace, size_t workspace_bytes, void *stream)
{
    DH_TRY(check_topk(logits, rows, vocab, k, ids, vals, argmax, workspace, workspace_bytes));
    if (!probs || !lse || !aligned(probs, 4) || !aligned(lse, 4))
        return DH_ERR_INVALID;
    const Span sp = span(probs, (size_t)rows * k * 4), sl = span(lse, (size_t)rows * 4);
    const Span others[] = {span(logits, (size_t)rows * (size_t)vocab * sizeof(float)),
                           span(ids, (size_t)rows * k * 4), span(vals, (size_t)rows * k * 4),
                           span(argmax, argmax ? (size_t)rows * 4 : 0),
                           span(workspace, dh::topk_ws_layout(rows, vocab, k).bytes)};
    if (overlap(sp, sl))
        return DH_ERR_INVALID;
    for (const Span &o : others)
        if (overlap(sp, o) || overlap(sl, o))
            return DH_ERR_INVALID;
    return device_status(dh::launch_topk(logits, rows, vocab, k, nullptr, ids, vals, argmax,
                                         workspace, (hipStream_t)stream, probs, lse));
}

// The id map of a subset head is an input: no output may overlap it.
static dh_status check_idmap(const int32_t *idmap, int64_t vocab, std::initializer_list<Span> outs)
{
    if (!idmap || !aligned(idmap, 4))
        return DH_ERR_INVALID;
    const Span sm = span(idmap, (size_t)vocab * 4);
    for (const Span &o : outs)
        if (overlap(sm, o))
            return DH_ERR_INVALID;
    return DH_OK;
}

dh_status dh_topk_mapped(const float *logits, int32_t rows, int64_t vocab, int32_t k,
                         const int32_t *idmap, int32_t *ids, float *vals, int32_t *argmax,
                         void *workspace, size_t workspace_bytes, void *stream)
{
    DH_TRY(check_topk(logits, rows, vocab, k, ids, vals, argmax, workspace, workspace_bytes));
    DH_TRY(check_idmap(idmap, vocab,
                       {span(ids, (size_t)rows * k * 4), span(vals, (size_t)rows * k * 4),
                        span(argmax, argmax ? (size_t)rows * 4 : 0),
                        span(workspace, dh::topk_ws_layout(rows, vocab, k).bytes)}));
    return device_status(dh::launch_topk(logits, rows, vocab, k, idmap, ids, vals, argmax,
                                         workspace, (hipStream_t)stream));
}

dh_status dh_gather_rows(const dh_head *head, const int32_t *ids, int64_t n, void *weight,
                         void *scale, void *stream)
{
    DH_TRY(check_row_major(head));
    if (head->format == DH_FP8_BLOCK32)
        return DH_ERR_UNSUPPORTED;
    if (n < 1)
        return DH_ERR_INVALID;
    if (n > ((int64_t)1 << 25))
        return DH_ERR_UNSUPPORTED;
    if (!ids || !weight || !aligned(ids, 4) || !aligned(weight, 16))
        return DH_ERR_INVALID;
    const bool row_scale = head->format == DH_FP8_ROW;
    if (row_scale ? (!scale || !aligned(scale, 4)) : scale != nullptr)
        return DH_ERR_INVALID;
    const Span sw = span(weight, (size_t)n * (size_t)head->hidden * elem_bytes(head->format));
    const Span ss = span(scale, row_scale ? (size_t)n * 4 : 0);
    const Span in[] = {head_weight(*head), head_scale(*head), span(ids, (size_t)n * 4)};
    for (const Span &s : in)
        if (overlap(sw, s) || overlap(ss, s))
            return DH_ERR_INVALID;
    if (overlap(sw, ss))
        return DH_ERR_INVALID;
    return device_status(dh::launch_gather_rows(*head, ids, n, weight,
                                                static_cast<float *>(scale),
                                                (hipStream_t)stream));
}

static dh_status check_rescore(const dh_head *dense, const uint16_t *x, int32_t rows,
                               const int32_t *cand_ids, int32_t cand_k, float *exact,
                               int32_t *draft)
{
    DH_TRY(check_row_major(dense));
    if (dense->format != DH_BF16)
        return DH_ERR_INVALID;
    DH_TRY(check_rows(rows));
    if (cand_k < 1)
        return DH_ERR_INVALID;
    if (cand_k > DH_MAX_K)
        return DH_ERR_UNSUPPORTED;
    if (!x || !cand_ids || !exact || !draft || !aligned(x, 16) || !aligned(cand_ids, 4) ||
        !aligned(exact, 4) || !aligned(draft, 4))
        return DH_ERR_INVALID;
    const Span se = span(exact, (size_t)rows * cand_k * 4), sd = span(draft, (size_t)rows * 4);
    const Span sc = span(cand_ids, (size_t)rows * cand_k * 4);
    const Span sx = span(x, (size_t)rows * (size_t)dense->hidden * 2);
    const Span sw = head_weight(*dense);
    if (overlap(se, sd) || overlap(se, sc) || overlap(sd, sc) || overlap(se, sx) ||
        overlap(sd, sx) || overlap(se, sw) || overlap(sd, sw))
        return DH_ERR_INVALID;
    return DH_OK;
}

dh_status dh_rescore(const dh_head *dense, const uint16_t *x, int32_t rows,
                     const int32_t *cand_ids, int32_t cand_k, float *exact, int32_t *draft,
                     void *stream)
{
    DH_TRY(check_rescore(dense, x, rows, cand_ids, cand_k, exact, draft));
    return device_status(dh::launch_rescore(*dense, x, rows, cand_ids, nullptr, cand_k, exact,
                                            draft, (hipStream_t)stream));
}

dh_status dh_rescore_sync(const dh_head *dense, const uint16_t *x, int32_t rows,
                          const int32_t *cand_ids, int32_t cand_k, float *exact,
                          int32_t *draft, uint32_t *sync, void *stream)
{
    DH_TRY(check_rescore(dense, x, rows, cand_ids, cand_k, exact, draft));
    if (!sync || !aligned(sync, 256))
        return DH_ERR_INVALID;
    const Span ss = span(sync, DH_RESCORE_SYNC_BYTES);
    const Span others[] = {span(exact, (size_t)rows * cand_k * 4), span(draft, (size_t)rows * 4),
                           span(cand_ids, (size_t)rows * cand_k * 4),
                           span(x, (size_t)rows * (size_t)dense->hidden * 2),
                           head_weight(*dense)};
    for (const Span &o : others)
        if (overlap(ss, o))
            return DH_ERR_INVALID;
    // the rows' ticket lines, then their best-key lines (2 * rows lines of 256 bytes)
    static_assert(2 * DH_MAX_ROWS * dh::kTicketStride * 4 <= DH_RESCORE_SYNC_BYTES,
                  "the sync buffer holds two lines a row");
    return device_status(dh::launch_rescore(*dense, x, rows, cand_ids, nullptr, cand_k, exact,
                                            draft, (hipStream_t)stream, sync));
}

// dh_draft, dh_draft_mapped, dh_draft_lowrank and dh_draft_noalloc: with an id map the head
// is a subset head whose entry j is vocabulary id idmap[j], and the dense head spans the
// whole vocabulary; with `down` the stage-1 head is low rank: t = bf16(x down^T), and
// `head` projects t.  own_scratch (workspace NULL): the workspace is the library's fixed
// scratch, whose device address is looked up only once every argument has passed.
static dh_status run_draft(const dh_head *head, const dh_head *down, uint16_t *t,
                           const int32_t *idmap, const dh_head *dense, const uint16_t *x,
                           int32_t rows, int32_t k, int32_t *ids, float *vals, int32_t *draft,
                           float *exact, float *logits, void *workspace,
                           size_t workspace_bytes, void *stream, bool own_scratch = false)
{
    DH_TRY(check_head(head));
    DH_TRY(check_gemv_rows(rows, head->hidden));
    if (head->vocab > DH_MAX_VOCAB)
        return DH_ERR_UNSUPPORTED;
    DH_TRY(check_k(k, head->vocab));
    if (!x || !aligned(x, 16) || !draft || !aligned(draft, 4) || (logits && !aligned(logits, 4)))
        return DH_ERR_INVALID;
    if (down) {
        DH_TRY(check_head(down));
        DH_TRY(check_gemv_rows(rows, down->hidden));
        if (down->vocab != head->hidden || !t || !aligned(t, 16))
            return DH_ERR_INVALID;
    }
    const int64_t xw = down ? down->hidden : head->hidden;   // the width of x
    if (dense) {
        DH_TRY(check_head(dense));
        if (dense->format != DH_BF16 || (!idmap && dense->vocab != head->vocab) ||
            dense->hidden != xw || !exact)
            return DH_ERR_INVALID;
    } else if (exact) {
        return DH_ERR_INVALID;
    }
    const TopkWs tw = dh::topk_ws_layout(rows, head->vocab, k);
    const size_t lbytes = (size_t)rows * (size_t)head->vocab * sizeof(float);
    const size_t need = tw.bytes + (logits ? 0 : ((lbytes + 255) & ~(size_t)255));
    if (own_scratch) {
        if (need > DH_NOALLOC_SCRATCH_BYTES)
            return DH_ERR_SCRATCH;
    } else if (!workspace || !aligned(workspace, 256) || workspace_bytes < need) {
        return DH_ERR_WORKSPACE;
    }
    float *L = logits || own_scratch
                   ? logits
                   : reinterpret_cast<float *>(static_cast<char *>(workspace) + tw.bytes);
    DH_TRY(check_topk(L, rows, head->vocab, k, ids, vals, dense ? nullptr : draft, workspace,
                      tw.bytes, own_scratch));
    if (dense)
        DH_TRY(check_rescore(dense, x, rows, ids, k, exact, draft));
    // Every buffer the call writes -- the logits, the workspace's top-k part, ids, vals,
    // draft, exact and t -- must be clear of every buffer it reads and of every other one it
    // writes (the rescore reads the stage-1 ids and values while it writes exact and draft).
    const size_t rk = (size_t)rows * (size_t)k * 4;
    const Span in[] = {head_weight(*head), head_scale(*head), span(x, (size_t)rows * xw * 2),
                       dense ? head_weight(*dense) : Span{0, 0},
                       down ? head_weight(*down) : Span{0, 0},
                       down ? head_scale(*down) : Span{0, 0},
                       span(idmap, idmap ? (size_t)head->vocab * 4 : 0)};
    const Span outs[] = {span(L, L ? lbytes : 0), span(workspace, own_scratch ? 0 : tw.bytes),
                         span(ids, rk),
                         span(vals, rk), span(draft, (size_t)rows * 4),
                         span(exact, exact ? rk : 0),
                         span(t, down ? (size_t)rows * (size_t)head->hidden * 2 : 0)};
    constexpr int nouts = sizeof(outs) / sizeof(outs[0]);
    for (int i = 0; i < nouts; i++) {
        for (const Span &s : in)
            if (overlap(outs[i], s))
                return DH_ERR_INVALID;
        for (int j = i + 1; j < nouts; j++)
            if (overlap(outs[i], outs[j]))
                return DH_ERR_INVALID;
    }
    if (idmap && !aligned(idmap, 4))
        return DH_ERR_INVALID;
    if (own_scratch) {
        workspace = scratch_address();
        if (!workspace)
            return DH_ERR_DEVICE;
        if (!logits)
            L = reinterpret_cast<float *>(static_cast<char *>(workspace) + tw.bytes);
    }
    const hipStream_t st = (hipStream_t)stream;
    hipError_t e = hipSuccess;
    if (down)   // nothing else is live in the checked workspace yet: it may hold partials
        e = dh::launch_linear(*down, x, rows, DH_OUT_BF16, nullptr, t, st, workspace, need);
    // Up to 16 rows, the GEMV also cuts each of its workgroups' logits for the top-k, which
    // one workgroup per row then merges; else (or when the GEMV's grid is too large for the
    // merge) the top-k is one launch of its own.  The GEMV zeroes the sync lines of the
    // kernels after it.
    const dh::GemvCut cut = dh::topk_cut(workspace, rows, head->vocab, k);
    int grid = 0;
    if (e == hipSuccess)
        e = dh::launch_gemv(*head, down ? t : x, rows, L, st,
                            dh::topk_tickets(workspace, rows, head->vocab, k),
                            dh::kSyncKinds * rows, dh::kTicketStride, rows <= 16 ? &cut : nullptr,
                            &grid);
    const bool cut_made = rows <= 16 && grid >= 1 && grid <= dh::kCutMaxChunks &&
                          grid * cut.slots <= cut.max_keys;
    if (e == hipSuccess)
        e = cut_made ? dh::launch_cut_merge(L, rows, head->vocab, k, idmap, ids, vals,
                                            dense ? nullptr : draft, workspace, grid, st)
                     : dh::launch_topk(L, rows, head->vocab, k, idmap, ids, vals,
                                       dense ? nullptr : draft, workspace, st);
    if (e == hipSuccess && dense)   // its sync lines were zeroed by the GEMV
        e = dh::launch_rescore(*dense, x, rows, ids, vals, k, exact, draft, st,
                               dh::topk_tickets(workspace, rows, head->vocab, k));
    return device_status(e);
}

dh_status dh_draft(const dh_head *head, const dh_head *dense, const uint16_t *x, int32_t rows,
                   int32_t k, int32_t *ids, float *vals, int32_t *draft, float *exact,
                   float *logits, void *workspace, size_t workspace_bytes, void *stream)
{
    return run_draft(head, nullptr, nullptr, nullptr, dense, x, rows, k, ids, vals, draft,
                     exact, logits, workspace, workspace_bytes, stream);
}

dh_status dh_draft_noalloc(const dh_head *head, const dh_head *dense, const uint16_t *x,
                           int32_t rows, int32_t k, int32_t *ids, float *vals, int32_t *draft,
                           float *exact, float *logits, void *stream)
{
    return run_draft(head, nullptr, nullptr, nullptr, dense, x, rows, k, ids, vals, draft,
                     exact, logits, nullptr, DH_NOALLOC_SCRATCH_BYTES, stream, true);
}

dh_status dh_draft_mapped(const dh_head *head, const int32_t *idmap, const dh_head *dense,
                          const uint16_t *x, int32_t rows, int32_t k, int32_t *ids,
                          float *vals, int32_t *draft, float *exact, float *logits,
                          void *workspace, size_t workspace_bytes, void *stream)
{
    if (!idmap)
        return DH_ERR_INVALID;
    return run_draft(head, nullptr, nullptr, idmap, dense, x, rows, k, ids, vals, draft,
                     exact, logits, workspace, workspace_bytes, stream);
}

dh_status dh_draft_lowrank(const dh_head *down, const dh_head *up, const dh_head *dense,
                           const uint16_t *x, int32_t rows, int32_t k, uint16_t *t,
                           int32_t *ids, float *vals, int32_t *draft, float *exact,
                           float *logits, void *workspace, size_t workspace_bytes,
                           void *stream)
{
    if (!down)
        return DH_ERR_INVALID;
    return run_draft(up, down, t, nullptr, dense, x, rows, k, ids, vals, draft, exact, logits,
                     workspace, workspace_bytes, stream);
}

dh_status dh_sample(const int32_t *ids, const float *vals, int32_t rows, int32_t k,
                    double temperature, double top_p, double min_p, uint64_t seed,
                    const int64_t *positions, int32_t *token, int32_t *kept, void *stream)
{
    DH_TRY(check_rows(rows));
    if (k < 1)
        return DH_ERR_INVALID;
    if (k > DH_MAX_K)
        return DH_ERR_UNSUPPORTED;
    if (!(temperature >= 0.0) || !(temperature < __builtin_inf()) || !(top_p > 0.0) ||
        !(top_p <= 1.0) || !(min_p >= 0.0) || !(min_p <= 1.0))
        return DH_ERR_INVALID;
    if (!ids || !vals || !positions || !token || !aligned(ids, 4) || !aligned(vals, 4) ||
        !aligned(positions, 8) || !aligned(token, 4) || (kept && !aligned(kept, 4)))
        return DH_ERR_INVALID;
    const Span st = span(token, (size_t)rows * 4), sk = span(kept, kept ? (size_t)rows * 4 : 0);
    const Span in[] = {span(ids, (size_t)rows * k * 4), span(vals, (size_t)rows * k * 4),
                       span(positions, (size_t)rows * 8)};
    for (const Span &i : in)
        if (overlap(st, i) || overlap(sk, i))
            return DH_ERR_INVALID;
    if (overlap(st, sk))
        return DH_ERR_INVALID;
    return device_status(dh::launch_sample(ids, vals, rows, k, temperature, top_p, min_p, seed,
                                           positions, token, kept, (hipStream_t)stream));
}

dh_status dh_tile_head(const dh_head *head, void *tiled, void *stream)
{
    DH_TRY(check_row_major(head));
    if (!tiled || !aligned(tiled, 16))
        return DH_ERR_INVALID;
    const Span st = span(tiled, dh::tiled_bytes(head->format, head->vocab, head->hidden));
    if (overlap(st, head_weight(*head)) || overlap(st, head_scale(*head)))
        return DH_ERR_INVALID;
    return device_status(dh::launch_tile_head(*head, tiled, (hipStream_t)stream));
}

size_t dh_tiled_bytes(int32_t format, int64_t vocab, int64_t hidden)
{
    if (!known_format(format) || vocab < 1 || hidden < 32 || hidden % 32 != 0 ||
        hidden > DH_MAX_HIDDEN || vocab > ((int64_t)1 << 25))
        return 0;
    return dh::tiled_bytes(format, vocab, hidden);
}

dh_status dh_stream_read(const void *buf, size_t bytes, uint32_t *sink, void *stream)
{
    if (!buf || !sink || !aligned(buf, 16) || !aligned(sink, 4) || bytes == 0 || bytes % 4096)
        return DH_ERR_INVALID;
    if (overlap(span(buf, bytes), span(sink, DH_STREAM_SINK_WORDS * sizeof(uint32_t))))
        return DH_ERR_INVALID;
    return device_status(dh::launch_stream_read(buf, bytes, sink, (hipStream_t)stream));
}

dh_status dh_quantize(int32_t format, const uint16_t *w, int64_t vocab, int64_t hidden,
                      uint8_t *codes, void *scale, void *stream)
{
    const int base = format & ~DH_TILED;   // codes row-major or (DH_TILED) tiled
    if (!known_format(format) || (base != DH_FP8_BLOCK32 && base != DH_FP8_ROW))
        return DH_ERR_INVALID;
    if (vocab < 1 || hidden < 32 || hidden % 32 != 0)
        return DH_ERR_INVALID;
    if (hidden > DH_MAX_HIDDEN || vocab > (int64_t)INT32_MAX / 2)
        return DH_ERR_UNSUPPORTED;
    if (!w || !codes || !scale || !aligned(w, 2) || (base == DH_FP8_ROW && !aligned(scale, 4)) ||
        ((format & DH_TILED) && !aligned(codes, 16)))
        return DH_ERR_INVALID;
    dh_head h{format, vocab, hidden, codes, scale};
    const Span sw = span(w, (size_t)vocab * (size_t)hidden * 2), sc = head_weight(h),
               ss = head_scale(h);
    if (overlap(sw, sc) || overlap(sw, ss) || overlap(sc, ss))
        return DH_ERR_INVALID;
    return device_status(
        dh::launch_quantize(format, w, vocab, hidden, codes, scale, (hipStream_t)stream));
}

const char *dh_status_string(int32_t status)
{
    switch (status) {
    case DH_OK: return "ok";
    case DH_ERR_INVALID: return "invalid argument (null or misaligned pointer, bad format, "
                                "bad size, or overlapping buffers)";
    case DH_ERR_UNSUPPORTED: return "size outside the implemented limits (rows <= 32, "
                                    "k <= 512, hidden <= 32768, vocab <= 262144)";
    case DH_ERR_WORKSPACE: return "workspace missing, misaligned or too small "
                                  "(see dh_workspace_bytes)";
    case DH_ERR_DEVICE: return "the HIP runtime reported an error at launch";
    case DH_ERR_SCRATCH: return "the call needs more than the fixed scratch of "
                                "dh_draft_noalloc (DH_NOALLOC_SCRATCH_BYTES)";
    default: return "unknown status";
    }
}

}  // extern "C"
