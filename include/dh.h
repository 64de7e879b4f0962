/*
 * dh.h -- C ABI of the few-row draft-head vocabulary projection for MI355X (gfx950).
 *
 * A speculative-decoding draft head ends in a projection of its last hidden rows onto the
 * vocabulary: a GEMV of 1..32 bf16 activation rows against a [V][H] head, fp32 logits, a
 * per-row top-k and argmax, and optionally a rescore of the top-k candidates against a dense
 * bf16 head.  Sources (web pages on one inference engine, cited by title and section):
 *   [TFE]   "dsv41 Zig: the TFE draft head (TF_DS_DRAFTER=eagle), off by default"
 *   [SUPER] "nemotron: Super's MTP drafts on the draft vocabulary's FP8 rows while a
 *            stream's text is covered, same replies"
 *   [METAL] "dsv41 metal: the DSpark drafter on an FP8 head, a concurrent propose and
 *            resident buffers"
 *   [DSV]   "DeepSeek-V4.1: performance hooks and host checks"
 *
 * Conventions for every entry point:
 *  - Pointers named as device pointers must point to device memory of the current HIP
 *    device; the caller allocates and frees every buffer and keeps it alive until the work
 *    on `stream` has completed.  The library allocates nothing, frees nothing and keeps no
 *    pointer past the call.
 *  - `stream` is a hipStream_t (NULL: the null stream).  Calls only enqueue work and return;
 *    outputs are valid once the stream has reached that point.
 *  - Every argument is checked on the host before anything is enqueued.  On a refusal the
 *    call returns a non-zero dh_status, enqueues nothing and leaves every output untouched.
 *    Sizes out of range are refused, never clipped.
 *  - A failure reported by the HIP runtime at launch returns DH_ERR_DEVICE.
 *  - Outputs must not overlap inputs or each other.
 *  - The library keeps no mutable global state: calls on different streams may overlap.
 *  - Matrices are row-major and dense (row stride == row length).
 */
#ifndef DH_H
#define DH_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    DH_OK = 0,
    DH_ERR_INVALID = 1,     /* null/misaligned pointer, bad format code, negative size,
                               outputs overlapping inputs */
    DH_ERR_UNSUPPORTED = 2, /* a size outside what the kernels implement (see limits) */
    DH_ERR_WORKSPACE = 3,   /* workspace missing or smaller than required */
    DH_ERR_DEVICE = 4,      /* the HIP runtime reported an error at launch */
    DH_ERR_SCRATCH = 5      /* dh_draft_noalloc: the sizes need more than its fixed scratch */
} dh_status;

/* Storage formats of a vocabulary head [V][H].
 *  DH_BF16        weight: bf16 bits, uint16 [V][H]; scale: NULL.  [TFE] two_stage commit
 *                 note and 'Update': the dense bf16 copy of the target's head.
 *  DH_FP8_BLOCK32 weight: OCP E4M3 codes, uint8 [V][H]; scale: E8M0 bytes, uint8
 *                 [ceil(V/32)][H/32], the value of weight (v,h) being
 *                 e4m3(code[v][h]) * 2^(scale[v/32][h/32] - 127).  [METAL] 'FP8 draft head'.
 *  DH_FP8_ROW     weight: OCP E4M3 codes, uint8 [V][H]; scale: float32 [V], the value of
 *                 weight (v,h) being e4m3(code[v][h]) * scale[v].  [TFE] commit notes and
 *                 'Update' on FP8 linears (one fp32 scale a row).
 * The GPU widens each scaled weight to bf16 before its products; that is exact while
 * e4m3(code) * 2^(byte-127) is a normal bf16 number, which holds for every code when the
 * scale byte is in 10..246 (a head the quantizer below makes from weights whose 32x32 block
 * maxima lie in [2^-100, 2^100] always is). */
typedef enum { DH_BF16 = 0, DH_FP8_BLOCK32 = 1, DH_FP8_ROW = 2 } dh_format;

/* Layout modifier: `format | DH_TILED` names the same head with its weight stored tiled for
 * the GEMV (made once, at load, by dh_tile_head; the scale keeps its layout above).  A tile
 * is 16 rows, a block 64 columns, and E the bytes of an element (bf16 2, E4M3 1).  Block b of
 * tile t is E KiB at byte (t * ceil(H/64) + b) * 1024 * E.  In it, the 16 bytes at
 * (q * 64 + l) * 16 (q < E, lane l < 64) are row 16 t + l % 16's elements
 *   E4M3: 64 b + 16 (l / 16) .. + 15;
 *   bf16: 64 b + 16 (l / 16) + 8 q .. + 7.
 * Rows past V and elements past H are zero.  Size: dh_tiled_bytes.  A wave's 1 KiB read is
 * then exactly the operand of one 16-row x 64-column multiply, in whole cache lines, which
 * the hardware streams faster than the row-major layout's 64-byte pieces of 16 rows.  The
 * GEMV forms (dh_gemv, dh_linear, the stage-1 head of the dh_draft family) take tiled heads
 * and give bitwise the same results as from the row-major head; dh_rescore's dense head and
 * dh_gather_rows's source must be row-major (a tiled one is refused with DH_ERR_INVALID). */
#define DH_TILED 16

/* A head: a host struct naming device buffers.  `weight` must be 16-byte aligned; a float32
 * row scale must be 4-byte aligned. */
typedef struct dh_head {
    int32_t format;     /* dh_format */
    int64_t vocab;      /* V >= 1 rows (token ids 0..V-1) */
    int64_t hidden;     /* H >= 32 columns, a multiple of 32 */
    const void *weight; /* device */
    const void *scale;  /* device, or NULL for DH_BF16 */
} dh_head;

/* Limits of this implementation (refused with DH_ERR_UNSUPPORTED beyond them).
 * Rows: [TFE] commit notes -- the head's own GEMV takes up to 16 rows; [SUPER] commit notes
 * on 32-row windows -- calls of 17 to 32 rows take the few-row forms too, each giving the same
 * bits as the 16-row form.  Up to H = DH_MAX_HIDDEN_WIDE (4096 for a row-major bf16 head)
 * such a call reads the head once (32 rows of activations held in registers); a wider head is
 * read once per 16 rows.
 * k: [TFE] 'Update' -- the candidate count runs from 1 to 512.
 * H: [TFE] commit notes -- the head's own linears (wo, w2) go through the same few-row GEMV,
 * and w2's input is the FFN width; up to DH_MAX_HIDDEN columns (heads and linears alike). */
#define DH_MAX_ROWS 32
#define DH_MAX_HIDDEN_WIDE 5120    /* one pass over the head for more than 16 rows */
#define DH_MAX_K 512
#define DH_MAX_HIDDEN 32768         /* wider than 8192: streamed in 8192-column chunks */
#define DH_MAX_VOCAB 262144        /* dh_topk / dh_draft */
#define DH_MAX_GEMV_VOCAB 33554432 /* dh_gemv, dh_rescore: 2^25 rows */

/* dh_gemv -- logits[r][v] = sum_h x[r][h] * w[v][h] for r < rows, v < V, in fp32.
 * [TFE] commit notes: the own GEMV for up to 16 rows with fp32 output; 'What this changes':
 * fp32 sums.  x: device bf16 bits [rows][H], 16-byte aligned.  logits: device float32
 * [rows][V].  Summation order is fixed by the kernel and independent of `rows`, so a row's
 * logits are bitwise the same in a 1-row, a 16-row and a 32-row call.  NaN and infinities propagate
 * as in IEEE arithmetic. */
dh_status dh_gemv(const dh_head *head, const uint16_t *x, int32_t rows, float *logits,
                  void *stream);

/* Output modes of dh_linear.  [TFE] commit notes on the head's own GEMV: its few-row
 * kernels write fp32, bf16, or the bf16 sum added to a bf16 row (the residual stream), and
 * that add is rounded once. */
typedef enum { DH_OUT_F32 = 0, DH_OUT_BF16 = 1, DH_OUT_ADD_BF16 = 2 } dh_out_mode;

/* dh_linear -- one of the draft head's own linears through the same few-row GEMV: with
 * s[r][n] = sum_k x[r][k] * w[n][k] (the weight as a dh_head: `vocab` = N output features,
 * `hidden` = K input features, any format; [TFE] commit notes: the wo and w2 linears go
 * through the own GEMV, FP8 with a row scale among the forms it loads), out[r][n] is
 *   DH_OUT_F32:      s, float32 [rows][N];
 *   DH_OUT_BF16:     bf16(s), bf16 bits [rows][N];
 *   DH_OUT_ADD_BF16: bf16(residual[r][n] + s), bf16 bits [rows][N], one rounding to bf16
 *                    of the fp32 sum.
 * residual: device bf16 bits [rows][N] for DH_OUT_ADD_BF16 (else NULL); it may be `out`
 * itself (in place) but must not overlap it otherwise.  Sums as dh_gemv (fp32, a fixed
 * order independent of `rows`); bf16 rounding is to nearest even.  out: 4-byte aligned
 * (float32) or 2-byte aligned (bf16).  Rows 1..DH_MAX_ROWS. */
dh_status dh_linear(const dh_head *w, const uint16_t *x, int32_t rows, int32_t mode,
                    const uint16_t *residual, void *out, void *stream);

/* dh_linear_ws -- dh_linear with a workspace, for linears with few output rows: with up to
 * 16 rows and K above 8192 columns the column chunks of every output tile run at once (a
 * partial sum per chunk in the workspace, then their sum in chunk order); with K up to 8192
 * and few tiles, each tile's sum is split by its 64-column parts the same way.  The results
 * are bitwise dh_linear's.  Same passages as dh_linear.
 * workspace: device, 256-byte aligned, at least dh_linear_workspace_bytes(rows, N, K) bytes,
 * scratch (no state between calls); it must not overlap any other argument's buffer.
 * Other arguments and errors as dh_linear; a missing or short workspace is
 * DH_ERR_WORKSPACE. */
dh_status dh_linear_ws(const dh_head *w, const uint16_t *x, int32_t rows, int32_t mode,
                       const uint16_t *residual, void *out, void *workspace,
                       size_t workspace_bytes, void *stream);

/* The workspace dh_linear_ws needs for `rows` rows, N = n outputs and K = k inputs (0 for
 * sizes outside the limits). */
size_t dh_linear_workspace_bytes(int32_t rows, int64_t n, int64_t k);

/* dh_topk -- per row, the k best logits in order: entry u beats entry v iff u is eligible
 * and (v is not, or l_u > l_v, or l_u == l_v and u < v); NaN and -inf are not eligible, so
 * they are never returned; -0 == +0.  Slot j holds the entry that exactly j others beat.
 * When a row has fewer than k eligible logits the remaining slots hold (id 0, -inf).
 * [TFE] two_stage commit note and 'Update': top cand_k fp32 logits, a tie at the k-th value
 * going to the lower token id, cand_k from 1 to 512.  [SUPER] commit note on the few-row
 * top-k: ranking by how many others beat an entry (higher score, then lower index), and
 * every pick after the finite scores run out being index 0.
 * logits: device float32 [rows][vocab].  ids: device int32 [rows][k].  vals: device float32
 * [rows][k] (the logits' own bits, so -0 stays -0).  argmax: device int32 [rows], or NULL;
 * argmax[r] == ids[r][0].  workspace: device, 256-byte aligned, at least
 * dh_workspace_bytes(rows, vocab, k) bytes; its contents are scratch. */
dh_status dh_topk(const float *logits, int32_t rows, int64_t vocab, int32_t k, int32_t *ids,
                  float *vals, int32_t *argmax, void *workspace, size_t workspace_bytes,
                  void *stream);

/* dh_topk_softmax -- dh_topk plus the softmax statistics of each row, in the same two
 * passes over the logits.  [TFE] commit notes: the head's row kernels include a top-1 with a
 * confidence; the pages do not define it, and the reading here is the softmax probability.
 * Over a row's eligible logits (NaN and -inf excluded), with m the largest:
 *   z = sum_v exp(l_v - m), an entry equal to m counting 1 (so every +inf counts 1 and the
 *   finite entries 0 when m = +inf);  lse[r] = m + ln z (-inf when the row has no eligible
 *   logit, +inf when m = +inf);  probs[r][j] = exp(vals[r][j] - m) / z (0 for pads).
 * probs[r][0] is the top-1's confidence.  fp32 arithmetic, sums in a fixed order
 * (reproducible).  probs: device float32 [rows][k]; lse: device float32 [rows].  Other
 * arguments, workspace and refusals as dh_topk. */
dh_status dh_topk_softmax(const float *logits, int32_t rows, int64_t vocab, int32_t k,
                          int32_t *ids, float *vals, int32_t *argmax, float *probs, float *lse,
                          void *workspace, size_t workspace_bytes, void *stream);

/* dh_rescore -- the exact logits of candidate tokens from a dense bf16 head and the
 * candidate that wins among them.  [TFE] two_stage commit note and 'Update': the draft is
 * the argmax of the candidates' exact logits from a dense bf16 copy of the target's head,
 * taken through the candidates' id map.
 * dense: a DH_BF16 head.  x: device bf16 bits [rows][H].  cand_ids: device int32
 * [rows][cand_k].  exact: device float32 [rows][cand_k]: exact[r][j] = sum_h x[r][h] *
 * dense[cand_ids[r][j]][h] (fp32); an id outside [0, V) is not read and gets NaN.
 * draft: device int32 [rows]: the candidate token that beats every other candidate of the
 * row under the dh_topk rule applied to (exact, token id); 0 if none is eligible. */
dh_status dh_rescore(const dh_head *dense, const uint16_t *x, int32_t rows,
                     const int32_t *cand_ids, int32_t cand_k, float *exact, int32_t *draft,
                     void *stream);

/* dh_rescore_sync -- dh_rescore in one launch, with the same results bit for bit: the
 * candidates' workgroups pick the draft themselves (dh_rescore runs a second, small kernel
 * for the pick), counting finished workgroups in `sync`.  Same passages as dh_rescore.
 * sync: device, 256-byte aligned, DH_RESCORE_SYNC_BYTES bytes, owned by the caller; it must
 * be all zero when the call's kernel starts -- zero-fill it once when it is allocated: every
 * call leaves it all zero again when its kernel ends.  Calls that share a sync buffer must
 * not run at the same time (order them on one stream).  It must not overlap any other
 * argument's buffer.  Other arguments and errors as dh_rescore. */
#define DH_RESCORE_SYNC_BYTES (DH_MAX_ROWS * 2 * 256)
dh_status dh_rescore_sync(const dh_head *dense, const uint16_t *x, int32_t rows,
                          const int32_t *cand_ids, int32_t cand_k, float *exact,
                          int32_t *draft, uint32_t *sync, void *stream);

/* dh_draft -- the whole projection in one call: dh_gemv, then dh_topk (k), then -- when
 * `dense` is not NULL -- the two-stage rescore of the top k candidates.  [TFE] two_stage
 * commit note: a draft pass's vocabulary head gives each row its draft, either the argmax
 * of its logits (the top-1 kernel) or, for a two_stage head, the argmax of the exact
 * logits of its top cand_k candidates from the dense bf16 copy of the target's head,
 * taken through the candidates' id map; 'What this changes': the head runs on one rank
 * and its drafts need no collective; 'Update (8d8691c..ce9a427)': the two_stage head with
 * cand_k up to 512 and a tie at the k-th value to the lower token id.  In the two-stage
 * form the pad slots of a row with fewer than k eligible logits are not candidates: their
 * exact logit is -inf and they are never drafted.
 * head: the stage-1 head (any format).  dense: NULL (one stage) or a DH_BF16 head of the
 * same V and H.  ids/vals: device [rows][k].  draft: device int32 [rows]: the argmax (one
 * stage) or the rescored winner (two stage).  exact: device float32 [rows][k] when dense is
 * given, else NULL.  logits: device float32 [rows][V] to receive the logits, or NULL (they
 * then live in the workspace).  workspace: as for dh_topk, sized by dh_workspace_bytes. */
dh_status dh_draft(const dh_head *head, const dh_head *dense, const uint16_t *x, int32_t rows,
                   int32_t k, int32_t *ids, float *vals, int32_t *draft, float *exact,
                   float *logits, void *workspace, size_t workspace_bytes, void *stream);

/* dh_draft_noalloc -- dh_draft without a workspace argument, for callers that cannot
 * allocate device memory around the call: code under HIP graph capture, tight serving loops
 * and harnesses that forbid hipMalloc.  The call allocates nothing; its scratch (the top-k's
 * chunk lists, and the logits when `logits` is NULL) is a fixed array of
 * DH_NOALLOC_SCRATCH_BYTES in the library's device code, one per GPU, held from the first
 * use of the library on that GPU until the process ends.  Sizes that need more than that
 * (dh_workspace_bytes(rows, V, k), less rows * V * 4 rounded up to 256 when `logits` is
 * given) are refused with DH_ERR_SCRATCH; 16 MiB covers every size with `logits` given, and
 * without it e.g. 16 rows of 129,280 logits at any k.  All calls on one GPU share that GPU's
 * array and leave their contents in it, so calls that may overlap on one GPU (other
 * streams, other host threads) race and give undefined results: serialize them.  Every other
 * argument, result and refusal is dh_draft's. */
#define DH_NOALLOC_SCRATCH_BYTES (16u << 20)
dh_status dh_draft_noalloc(const dh_head *head, const dh_head *dense, const uint16_t *x,
                           int32_t rows, int32_t k, int32_t *ids, float *vals, int32_t *draft,
                           float *exact, float *logits, void *stream);

/* dh_quantize -- make an FP8 head from a bf16 head (load-time preparation).
 *  DH_FP8_ROW ([TFE] 'Update' on FP8 linears): s[v] = float(max_h |w[v][h]| / 448) and
 *    code = E4M3 round-to-nearest-even of float(w / s[v]); an all-zero row gets s = 0 and
 *    codes 0.  scale: device float32 [V].
 *  DH_FP8_BLOCK32 ([METAL] 'FP8 draft head': E4M3 codes with E8M0 scales per 32x32 block,
 *    made from the bf16 head at load): e is the least integer with block amax <= 448 * 2^e,
 *    stored as e + 127 clamped to [0, 254] (127 for an all-zero block), and code = E4M3
 *    round-to-nearest-even of w * 2^-e.  scale: device uint8 [ceil(V/32)][H/32].
 * E4M3 rounding saturates at +-448.  w: device bf16 bits [V][H] (finite values).  codes:
 * device uint8 [V][H]; or, with format | DH_TILED, the codes go straight into the tiled
 * layout (zeros past V and H): device buffer of dh_tiled_bytes(format, V, H) bytes, 16-byte
 * aligned, the same bytes dh_tile_head makes from the row-major codes.  The scale is the same
 * either way. */
dh_status dh_quantize(int32_t format, const uint16_t *w, int64_t vocab, int64_t hidden,
                      uint8_t *codes, void *scale, void *stream);

/* dh_draft_lowrank -- dh_draft with a low-rank stage 1.  [TFE] two_stage commit note and
 * 'Update': the two_stage head takes its top cand_k candidates from low-rank logits and
 * drafts the argmax of their exact logits from a dense bf16 copy of the target's head.
 *   t[r][j]      = bf16(sum_h x[r][h] * down[j][h])   (dh_linear, DH_OUT_BF16)
 *   logits[r][v] = sum_j t[r][j] * up[v][j]           (dh_gemv, fp32)
 * then dh_draft's top-k and argmax, and with `dense` its rescore from x.  down: a dh_head
 * with `vocab` = the rank and `hidden` = H; up: `vocab` = V, `hidden` = the rank; any
 * format each.  dense: bf16 [V][H] or NULL (one stage).  t: device bf16 bits [rows][rank],
 * 16-byte aligned, written (the rank-r activations; the pages do not give their precision,
 * and like every GEMM input on those pages they are bf16).  Other arguments, refusals and
 * the workspace (dh_workspace_bytes(rows, V, k)) as dh_draft. */
dh_status dh_draft_lowrank(const dh_head *down, const dh_head *up, const dh_head *dense,
                           const uint16_t *x, int32_t rows, int32_t k, uint16_t *t,
                           int32_t *ids, float *vals, int32_t *draft, float *exact,
                           float *logits, void *workspace, size_t workspace_bytes,
                           void *stream);

/* dh_sample -- a keyed pick from each row's top-k candidates.  [DSV] commit notes on the
 * serving module's sampler: a window's choices come from the candidates, their nucleus
 * statistics and a pick keyed by seed, position and token id, so a drafted token equals the
 * serial one.  The pages define no formula; the reading implemented:
 *   over the eligible candidates j in list order (vals[r][j] > -inf; v_0 the first),
 *   q_j = exp((v_j - v_0) / temperature) (1 when v_j == v_0);
 *   nucleus: j is kept while the sum of q before it is below top_p * sum(q) (j = 0 always),
 *   min-p: and q_j >= min_p;
 *   the pick is the kept j maximising (v_j - v_0) / temperature - ln(-ln u_j), the lower id
 *   on a tie, with u_j in (0, 1) the first word w of Philox4x64-10 (Salmon et al., SC 2011)
 *   with key (seed, 0) and counter (positions[r], ids[r][j], 0, 0), as (w >> 11 + 1/2) * 2^-53
 *   (Gumbel-max: the pick has probability q_j / sum of the kept q).
 * temperature == 0 picks ids[r][0].  A row without an eligible candidate gives token 0.
 * Arithmetic in double.  ids, vals: device [rows][k], a dh_topk list (descending, pads
 * last).  positions: device int64 [rows].  token: device int32 [rows]; kept: device int32
 * [rows] (the number of candidates the filters kept) or NULL.  temperature >= 0 and finite,
 * 0 < top_p <= 1, 0 <= min_p <= 1, else DH_ERR_INVALID. */
dh_status dh_sample(const int32_t *ids, const float *vals, int32_t rows, int32_t k,
                    double temperature, double top_p, double min_p, uint64_t seed,
                    const int64_t *positions, int32_t *token, int32_t *kept, void *stream);

/* Draft-vocabulary subset heads.  [SUPER] 'What this changes': a draft head packs the FP8
 * rows of its draft vocabulary's ids into a weight of their own (keeping the head's scales)
 * and uploads their vocabulary ids; a level projects over that subset only, and the ids it
 * proposes are vocabulary ids.
 *
 * dh_gather_rows -- the subset head: row j of the output is row ids[j] of `head`, codes and
 * (DH_FP8_ROW) its row scale.  head: DH_BF16 or DH_FP8_ROW; DH_FP8_BLOCK32 is refused with
 * DH_ERR_UNSUPPORTED (a 32x32 scale block cannot be split by rows).  ids: device int32 [n];
 * an id outside [0, V) gives a row of zero codes (and scale 0), never a read outside the
 * head.  weight: device buffer of n * H elements of the head's format, 16-byte aligned;
 * scale: device float32 [n] for DH_FP8_ROW, else NULL.  The subset head is then
 * {head->format, n, H, weight, scale}. */
dh_status dh_gather_rows(const dh_head *head, const int32_t *ids, int64_t n, void *weight,
                         void *scale, void *stream);

/* dh_topk_mapped -- dh_topk over logits [rows][vocab] of a subset head, whose entry j is
 * vocabulary id idmap[j]: ids (and argmax) are vocabulary ids, values and pads as dh_topk
 * (a pad is vocabulary id 0).  idmap: device int32 [vocab], strictly increasing, so that the
 * lower entry of a tie is the lower vocabulary id (a precondition: not checked).  Workspace
 * as dh_topk. */
dh_status dh_topk_mapped(const float *logits, int32_t rows, int64_t vocab, int32_t k,
                         const int32_t *idmap, int32_t *ids, float *vals, int32_t *argmax,
                         void *workspace, size_t workspace_bytes, void *stream);

/* dh_draft_mapped -- dh_draft on a subset head (see dh_gather_rows) whose row j is
 * vocabulary id idmap[j] (device int32 [head->vocab], strictly increasing): ids and drafts
 * are vocabulary ids.  In the two-stage form `dense` is the full-vocabulary bf16 head (same
 * H; any V) and the candidates' exact logits come from its rows at their vocabulary ids.
 * Workspace: dh_workspace_bytes(rows, head->vocab, k). */
dh_status dh_draft_mapped(const dh_head *head, const int32_t *idmap, const dh_head *dense,
                          const uint16_t *x, int32_t rows, int32_t k, int32_t *ids,
                          float *vals, int32_t *draft, float *exact, float *logits,
                          void *workspace, size_t workspace_bytes, void *stream);

/* dh_tile_head -- the tiled copy of a row-major head's weight (layout: DH_TILED above),
 * made once at load.  head: DH_BF16, DH_FP8_BLOCK32 or DH_FP8_ROW, row-major.  tiled: device
 * buffer of dh_tiled_bytes(head->format, V, H) bytes, 16-byte aligned, not overlapping the
 * head.  The tiled head is then {head->format | DH_TILED, V, H, tiled, head->scale}.  A copy
 * bound by HBM bandwidth. */
dh_status dh_tile_head(const dh_head *head, void *tiled, void *stream);

/* Bytes of a tiled weight: ceil(V/16) * ceil(H/64) * 1024 * (2 for bf16, else 1).  Pure
 * host function; the format may carry DH_TILED; returns 0 for a format or size the library
 * refuses. */
size_t dh_tiled_bytes(int32_t format, int64_t vocab, int64_t hidden);

/* dh_stream_read -- a diagnostic, not a step of the projection: reads `bytes` of device
 * memory once, the way the GEMV streams a tiled head (1 KiB contiguous loads with the
 * non-temporal hint, about 32 KiB in flight per compute unit), so that its duration gives
 * the device's practical streaming-read bandwidth to report beside the GEMV's.  buf: device,
 * 16-byte aligned; bytes: a positive multiple of 4096.  sink: device uint32
 * [DH_STREAM_SINK_WORDS]; afterwards its words sum (mod 2^32) to the sum of buf's 32-bit
 * words, which shows that every byte was read exactly once.  sink must not overlap buf. */
#define DH_STREAM_SINK_WORDS 8192
dh_status dh_stream_read(const void *buf, size_t bytes, uint32_t *sink, void *stream);

/* Bytes of workspace dh_topk and dh_draft need for these sizes (dh_draft with logits ==
 * NULL included).  Pure host function; returns 0 for sizes the library refuses. */
size_t dh_workspace_bytes(int32_t rows, int64_t vocab, int32_t k);

/* A static, NUL-terminated description of a status code. */
const char *dh_status_string(int32_t status);

#ifdef __cplusplus
}
#endif

#endif /* DH_H */
