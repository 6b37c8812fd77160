/*
 * zz.h -- C ABI of libzz: zigzag varlen ring attention on one AMD MI355X (gfx950).
 *
 * The library computes causal attention over packed variable-length sequences
 * as context-parallel ring steps with zigzag load balancing, with every
 * simulated CP rank running on the one GPU.  All entry points take plain
 * pointers and sizes; none takes or returns a framework type.
 *
 * Sources of the operations (page title, then the passage):
 *  - ring-attention-pytorch issue #20, "Zigzag attention support?": the
 *    extract_local snippet -- cut a sequence into 2*CP chunks; rank r keeps
 *    chunk r then chunk 2*CP-1-r.
 *  - MaxText PR #1133, "Add Context Parallelism support to cudnn Flash
 *    Attention": softmax scale 1/sqrt(head_dim) passed as scale_factor; the
 *    load-balanced (causal) CP attention needs the tokens reordered first.
 *  - EasyDeL issue #129, "Attention Mask for Packed Sequences (via Attention
 *    Bias)": packed examples must not attend to one another (-inf bias); the
 *    packed lengths are passed as a list (cu_seqlens here).
 *  - MiniMax-01 issue #6, "Question about varlen ring attention": varlen
 *    ring attention over packed data; causal load imbalance across CP ranks.
 *  - FlagScale PR #910, "[Train] Support custom attention with context
 *    parallel": a ring driver with replaceable per-step forward and backward,
 *    pruning of redundant (masked) work, load balancing across CP ranks.
 *
 * Conventions
 *  - Layouts.  Token-major packed tensors [T, H, d], row-major, tokens on dim
 *    0.  "Zigzag layout" is the same shape with rows reordered rank-major:
 *    rows [r*T/CP, (r+1)*T/CP) belong to rank r; inside a rank, each
 *    sequence contributes chunk r then chunk 2CP-1-r, sequences in order.
 *    LSE and delta are fp32 [Hq, T] (natural log), indexed by zigzag row.
 *    Query head h uses key/value head h / (Hq/Hkv).
 *  - Ownership.  The caller owns every device buffer, including the plan
 *    workspace (except with zz_plan_upload_static, whose workspace is a
 *    static array of the library).  libzz allocates no device memory.  libzz
 *    owns the plan's host memory; zz_plan_destroy frees it.
 *  - Errors.  Every call returns zz_status; nothing throws across the ABI.
 *    Arguments are checked on the host before any launch; device pointers
 *    must be 16-byte aligned (ZZ_ERR_ALIGN).  A buffer a call writes must
 *    not overlap any other buffer of that call, measured over the whole
 *    buffer the plan's shape gives it (ZZ_ERR_ARG, naming the two buffers);
 *    buffers that are only read may share memory.  A failed launch returns
 *    ZZ_ERR_HIP; zz_last_error() gives a message for the calling thread.
 *  - Execution.  Device calls are asynchronous on the given stream (a
 *    hipStream_t passed as void*; NULL = the default stream).  A plan is
 *    immutable after zz_plan_upload and may be shared across streams.
 */
#ifndef ZZ_H
#define ZZ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct zz_plan zz_plan;

typedef enum {
    ZZ_OK = 0,
    ZZ_ERR_ARG = 1,       /* null pointer, value out of range            */
    ZZ_ERR_SHAPE = 2,     /* lengths / CP / heads / head_dim inconsistent */
    ZZ_ERR_DTYPE = 3,     /* dtype not supported for this call           */
    ZZ_ERR_ALIGN = 4,     /* device pointer or row size not 16-byte aligned */
    ZZ_ERR_WORKSPACE = 5, /* workspace too small                         */
    ZZ_ERR_HIP = 6,       /* HIP runtime / launch failure                */
    ZZ_ERR_STATE = 7      /* plan not uploaded                           */
} zz_status;

typedef enum { ZZ_F32 = 0, ZZ_BF16 = 1 } zz_dtype;

/* The three tile walks of the library.  FWD: query-major forward step.
 * BWD_DQ: query-major backward (dQ).  BWD_DKV: key-major backward (dK, dV). */
typedef enum { ZZ_PASS_FWD = 0, ZZ_PASS_BWD_DQ = 1, ZZ_PASS_BWD_DKV = 2 } zz_pass;

enum { ZZ_ALL_RANKS = -1, ZZ_ALL_STEPS = -1 };

/* Tile kinds in tile lists: every pair visible, or only some (masked). */
enum { ZZ_TILE_FULL = 1, ZZ_TILE_PARTIAL = 2 };

const char *zz_status_str(zz_status s);
/* Message of the last failing call on this thread ("" if none). */
const char *zz_last_error(void);

/* ------------------------------------------------------------------ plan */

/*
 * Build a plan for one packed batch.  The zigzag split of each sequence into
 * 2*cp equal chunks, rank r holding chunk r then chunk 2*cp-1-r, is the one of
 * ring-attention-pytorch issue #20 ("Zigzag attention support?", the
 * extract_local snippet); the lengths arrive as a list as in EasyDeL issue
 * #129 ("Attention Mask for Packed Sequences (via Attention Bias)", the
 * packed-batch request); the divisibility check mirrors the assertion that
 * FlagScale PR #910 ("[Train] Support custom attention with context
 * parallel", flex-attention notes) places on sequence lengths under CP.
 *  cu_seqlens  host int32[nseq+1], cu[0] = 0, strictly increasing; every
 *              length L_i = cu[i+1]-cu[i] must be a multiple of 2*cp (the
 *              zigzag split needs 2*cp equal chunks per sequence).
 *  cp          simulated context-parallel ranks, 1..64.
 *  hq, hkv     query / key-value heads, hq % hkv == 0.
 *  head_dim    32, 64 or 128.
 *  dtype       element type of Q, K, V, dO and O.
 *  bm, bn      forward tile: query rows x key rows, 1 <= bm <= 128,
 *              1 <= bn <= 64.  Tiles start at every zigzag chunk boundary.
 * On success *out owns a new plan.  Errors: ZZ_ERR_ARG, ZZ_ERR_SHAPE.
 */
zz_status zz_plan_create(const int32_t *cu_seqlens, int32_t nseq, int32_t cp, int32_t hq,
                         int32_t hkv, int32_t head_dim, zz_dtype dtype, int32_t bm, int32_t bn,
                         zz_plan **out);
void zz_plan_destroy(zz_plan *plan);

/* Bytes of device workspace that zz_plan_upload fills (tile lists, work lists,
 * the zigzag row map). */
size_t zz_plan_workspace_bytes(const zz_plan *plan);

/*
 * Copy the plan's device tables into d_ws (caller-allocated device memory of
 * at least zz_plan_workspace_bytes, 16-byte aligned) on `stream`, and bind the
 * plan to it.  d_ws must stay alive and unmodified while the plan is used.
 * Errors: ZZ_ERR_ARG, ZZ_ERR_ALIGN, ZZ_ERR_WORKSPACE, ZZ_ERR_HIP.
 */
zz_status zz_plan_upload(zz_plan *plan, void *d_ws, size_t ws_bytes, void *stream);

/* Size of the library's own per-GPU plan workspace (96 MiB). */
#define ZZ_STATIC_WORKSPACE_BYTES (96u << 20)

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture set up ahead, tight serving loops, harnesses that forbid
 * hipMalloc): zz_plan_upload into the library's own workspace on the current
 * device instead of a caller buffer.  It allocates nothing: the workspace is
 * a static device array of ZZ_STATIC_WORKSPACE_BYTES that every GPU the
 * library runs on holds until the process ends.  The caller still passes
 * every input and output buffer of the later calls.
 *  - One workspace per GPU, shared by every plan uploaded this way on it: the
 *    upload overwrites the tables of the plan bound there before, which from
 *    then on is refused (ZZ_ERR_STATE) until it is uploaded again.  An upload
 *    while kernels of the previously bound plan are still running on that
 *    GPU (another stream) races with them; so do two uploads at once.
 *  - The plan must then be used with the same device current (ZZ_ERR_STATE
 *    otherwise); a later zz_plan_upload rebinds it to a caller buffer.
 * Errors: ZZ_ERR_ARG (null plan), ZZ_ERR_WORKSPACE (zz_plan_workspace_bytes
 * above ZZ_STATIC_WORKSPACE_BYTES: use zz_plan_upload), ZZ_ERR_HIP.
 */
zz_status zz_plan_upload_static(zz_plan *plan, void *stream);

/* Shape queries.  Any output pointer may be NULL. */
zz_status zz_plan_shape(const zz_plan *plan, int64_t *total_tokens, int32_t *nseq, int32_t *cp,
                        int32_t *hq, int32_t *hkv, int32_t *head_dim, int32_t *dtype);

/* Rank-local cu_seqlens (host int32[nseq+1]): cu[i]/cp, the same on every rank. */
zz_status zz_plan_local_cu_seqlens(const zz_plan *plan, int32_t *out);

/* Host copy of the zigzag map: out[p] = zigzag row of packed token p (int64[T]). */
zz_status zz_plan_zigzag_dst(const zz_plan *plan, int64_t *out);

/* Tile shape (query rows, key rows) of a pass. */
zz_status zz_plan_tile_shape(const zz_plan *plan, zz_pass pass, int32_t *bm, int32_t *bn);

/*
 * Tiles that hold at least one visible (query, key) pair in ring step
 * (rank, step) -- the pruning of fully masked work that FlagScale PR #910
 * ("[Train] Support custom attention with context parallel", description)
 * lists -- in canonical order sorted by (q0, k0): out[5*t .. 5*t+4] =
 * q0, q1, k0, k1, kind with rank-local query rows [q0,q1) and shard-local key
 * rows [k0,k1); kind is ZZ_TILE_FULL or ZZ_TILE_PARTIAL.  Tiles with no
 * visible pair are never listed and never visited by the kernels.
 * *n receives the count; if it exceeds cap, nothing past cap is written and
 * ZZ_ERR_WORKSPACE is returned.
 */
zz_status zz_plan_tiles(const zz_plan *plan, zz_pass pass, int32_t rank, int32_t step,
                        int32_t *out, int64_t cap, int64_t *n);

/*
 * Tiles the all-gather form walks (zz_varlen_gathered_fwd / _bwd; the
 * gather of keys and values across ranks is the reading of zigzag attention
 * in ring-attention-pytorch issue #20, "Zigzag attention support?") for one
 * stationary owner: the query rows of rank `owner` (ZZ_PASS_FWD,
 * ZZ_PASS_BWD_DQ) or the key rows of shard `owner` (ZZ_PASS_BWD_DKV),
 * against the rows of every shard or rank.  Same layout, order, kinds and
 * capacity rule as zz_plan_tiles, but every row index is a GLOBAL zigzag row
 * (rank or shard j's rows start at j*T/cp).  Each list is the union over the
 * ring steps of the corresponding zz_plan_tiles lists, shifted to global rows.
 * Errors: ZZ_ERR_ARG for a null plan, bad pass, owner outside [0, cp) or a
 * null output; ZZ_ERR_WORKSPACE as above.
 */
zz_status zz_plan_gathered_tiles(const zz_plan *plan, zz_pass pass, int32_t owner,
                                 int32_t *out, int64_t cap, int64_t *n);

/*
 * Pair counts for rank/step (either may be ZZ_ALL_RANKS / ZZ_ALL_STEPS):
 * useful = visible (query, key) pairs per head; issued = pairs covered by the
 * pass's visited tiles (what the MFMA units process).  The per-rank balance
 * these counts measure is the point of the zigzag split: causal work piles up
 * on the late ranks of a contiguous split (MiniMax-01 issue #6, "Question
 * about varlen ring attention"; ring-attention-pytorch issue #20).
 * Errors: ZZ_ERR_ARG (null plan, bad pass, rank or step out of range).
 */
zz_status zz_plan_pair_counts(const zz_plan *plan, zz_pass pass, int32_t rank, int32_t step,
                              int64_t *useful, int64_t *issued);

/*
 * Useful (visible) pairs per head of every rank over the whole ring:
 * out int64[cp] (host), out[r] = sum over steps of rank r's visible pairs,
 * equal to sum_i L_i (L_i + 1) / (2 cp) on every rank under the zigzag split
 * (same passages as zz_plan_pair_counts).  Errors: ZZ_ERR_ARG.
 */
zz_status zz_plan_rank_useful_pairs(const zz_plan *plan, int64_t *out);

/* ------------------------------------------------------------ device ops */

/*
 * Zigzag reorder of dim 0 (MaxText PR #1133: tokens must be reordered before
 * load-balanced CP attention).  x_packed and x_zz are [T, row_bytes] byte
 * matrices (any element type; row_bytes % 16 == 0), distinct buffers.
 * permute: x_zz[dst(p)] = x_packed[p];  unpermute: x_packed[p] = x_zz[dst(p)].
 */
zz_status zz_zigzag_permute(const zz_plan *plan, const void *x_packed, void *x_zz,
                            int64_t row_bytes, void *stream);
zz_status zz_zigzag_unpermute(const zz_plan *plan, const void *x_zz, void *x_packed,
                              int64_t row_bytes, void *stream);

/*
 * One forward ring step (FlagScale PR #910: per-step forward of a ring
 * driver).  Rank r's queries attend to shard j = (r - step) mod cp, with the
 * causal and document masks; fully masked tiles are skipped.
 *  rank        0..cp-1, or ZZ_ALL_RANKS: every rank of this step in one launch.
 *  q_zz        [T, hq, d]  dtype, zigzag layout (whole buffer).
 *  k_zz, v_zz  [T, hkv, d] dtype, zigzag layout (whole buffers; the shard is
 *              located from the plan).
 *  o_acc       fp32 [T, hq, d], lse_acc fp32 [hq, T] (whole buffers; only
 *              the rows of the launched ranks are touched).
 *  merge = 0   write this step's partial: normalized O and LSE of every row of
 *              the rank (rows with no visible key get O = 0, LSE = -inf).
 *  merge = 1   merge the partial into (o_acc, lse_acc) by log-sum-exp:
 *              L = log(e^a + e^b), O = e^(a-L) O_a + e^(b-L) O_b; rows with
 *              no visible key are left untouched.
 * Errors: ZZ_ERR_ARG, ZZ_ERR_ALIGN, ZZ_ERR_STATE, ZZ_ERR_HIP.
 */
zz_status zz_varlen_ring_step_fwd(const zz_plan *plan, int32_t rank, int32_t step,
                                  const void *q_zz, const void *k_zz, const void *v_zz,
                                  float *o_acc, float *lse_acc, int32_t merge, void *stream);

/*
 * Forward of rank r's queries against every shard at once (ring-attention-
 * pytorch issue #20, "Zigzag attention support?": the maintainer reads the
 * zigzag scheme as an all-gather of keys and values across ranks, which GQA
 * makes affordable, and plans to offer that gather as an option).  With all
 * K/V resident, each query row's visible keys are walked in one launch with
 * one online softmax: no step partials and no merges.
 *  rank        0..cp-1, or ZZ_ALL_RANKS.
 *  q_zz, k_zz, v_zz  as zz_varlen_ring_step_fwd (whole zigzag buffers).
 *  o           fp32 [T, hq, d]: normalized output of the launched ranks' rows.
 *  lse         fp32 [hq, T]: natural-log LSE of the same rows.
 * The result equals the merged ring forward up to rounding order (the same
 * tiles are visited, grouped per row instead of per step).
 * Errors: ZZ_ERR_ARG, ZZ_ERR_ALIGN, ZZ_ERR_STATE, ZZ_ERR_HIP.
 */
zz_status zz_varlen_gathered_fwd(const zz_plan *plan, int32_t rank, const void *q_zz, const void *k_zz,
                                 const void *v_zz, float *o, float *lse, void *stream);

/*
 * Backward of the gathered form (same passage as zz_varlen_gathered_fwd):
 * rank r's dQ rows against every shard, and the dK, dV rows of shard r
 * against every rank's queries, one launch per kernel, no per-step
 * accumulation.
 *  rank        0..cp-1 (its query rows and its own K/V shard), or ZZ_ALL_RANKS.
 *  q_zz, k_zz, v_zz, do_zz, lse, delta  as zz_varlen_ring_step_bwd (lse from
 *              the forward, delta from zz_bwd_preprocess).
 *  dq fp32 [T, hq, d]; dk, dv fp32 [T, hkv, d]: the launched rows are
 *              written (not accumulated).
 * The result equals the sum over the ring steps up to rounding order.
 * Errors: ZZ_ERR_ARG, ZZ_ERR_ALIGN, ZZ_ERR_STATE, ZZ_ERR_HIP.
 */
zz_status zz_varlen_gathered_bwd(const zz_plan *plan, int32_t rank, const void *q_zz, const void *k_zz,
                                 const void *v_zz, const void *do_zz, const float *lse, const float *delta,
                                 float *dq, float *dk, float *dv, void *stream);

/*
 * Standalone log-sum-exp merge: (o_acc, lse_acc) <- merge with (o_part,
 * lse_part).  o: fp32 [rows, heads, head_dim]; lse: fp32 [heads, rows].
 * (0, -inf) is the identity; two -inf rows give (0, -inf).
 * The pages state that ring steps emit partial outputs that are combined
 * (FlagScale PR #910, per-step forward of the ring driver) but give no
 * formula: this natural-log log-sum-exp merge, L = log(e^a + e^b),
 * O = e^(a-L) O_a + e^(b-L) O_b in fp32, is this library's reading of that
 * silence (the plainest combination of two softmaxes over disjoint key sets).
 * o_acc / lse_acc must not overlap o_part / lse_part (ZZ_ERR_ARG).
 * Errors: ZZ_ERR_ARG, ZZ_ERR_ALIGN, ZZ_ERR_HIP.
 */
zz_status zz_lse_merge(float *o_acc, float *lse_acc, const float *o_part, const float *lse_part,
                       int64_t rows, int32_t heads, int32_t head_dim, void *stream);

/*
 * o_out = o_acc converted to the plan dtype (round to nearest even for bf16).
 * o_acc fp32 [T, hq, d] zigzag layout.  unpermute = 1 writes o_out in packed
 * token order, 0 keeps the zigzag order (MaxText PR #1133, "Add Context
 * Parallelism support to cudnn Flash Attention", review: the reordered
 * tokens are the framework's to restore).  o_out must not overlap o_acc.
 * Errors: ZZ_ERR_ARG, ZZ_ERR_ALIGN, ZZ_ERR_STATE, ZZ_ERR_HIP.
 */
zz_status zz_finalize_fwd(const zz_plan *plan, const float *o_acc, void *o_out, int32_t unpermute,
                          void *stream);

/*
 * Backward pre-pass: delta[h, z] = sum_e dO[z,h,e] * O[z,h,e] in fp32, from
 * the forward output O and upstream gradient dO (plan dtype, zigzag layout
 * [T, hq, d]).  delta fp32 [hq, T].  FlagScale PR #910 ("[Train] Support
 * custom attention with context parallel", description) names a per-step
 * backward of the ring driver without its arithmetic; delta is the row term
 * of the softmax gradient, dS = P (dP - delta), computed once per backward
 * from the final O so that every step can use it.
 * Errors: ZZ_ERR_ARG, ZZ_ERR_ALIGN, ZZ_ERR_STATE, ZZ_ERR_HIP.
 */
zz_status zz_bwd_preprocess(const zz_plan *plan, const void *o_zz, const void *do_zz, float *delta,
                            void *stream);

/*
 * One backward ring step (FlagScale PR #910: per-step backward).  With the
 * global LSE of the merged forward and delta from zz_bwd_preprocess, this
 * step's contributions are: dq rows of rank r, and dk / dv rows of shard
 * j = (r - step) mod cp (summed over the query heads of each group).
 *  q_zz [T,hq,d], k_zz / v_zz [T,hkv,d], do_zz [T,hq,d]: plan dtype, zigzag.
 *  lse, delta: fp32 [hq, T].
 *  dq_acc fp32 [T, hq, d]; dk_acc, dv_acc fp32 [T, hkv, d]; zigzag layout.
 *  accumulate = 1 adds the contributions (plain read-add-write: launches on
 *  one buffer must not overlap in time); 0 overwrites the rows this step
 *  touches (step 0 of the ring touches every row, so a driver needs no
 *  zero-fill).
 * zz_varlen_ring_step_bwd launches both kernels of the step; the _dkv / _dq
 * variants launch one each (they write disjoint buffers and may run on
 * different streams).
 * Errors: as zz_varlen_ring_step_fwd.
 */
zz_status zz_varlen_ring_step_bwd(const zz_plan *plan, int32_t rank, int32_t step,
                                  const void *q_zz, const void *k_zz, const void *v_zz,
                                  const void *do_zz, const float *lse, const float *delta,
                                  float *dq_acc, float *dk_acc, float *dv_acc, int32_t accumulate,
                                  void *stream);
zz_status zz_varlen_ring_step_bwd_dkv(const zz_plan *plan, int32_t rank, int32_t step,
                                      const void *q_zz, const void *k_zz, const void *v_zz,
                                      const void *do_zz, const float *lse, const float *delta,
                                      float *dk_acc, float *dv_acc, int32_t accumulate, void *stream);
zz_status zz_varlen_ring_step_bwd_dq(const zz_plan *plan, int32_t rank, int32_t step,
                                     const void *q_zz, const void *k_zz, const void *v_zz,
                                     const void *do_zz, const float *lse, const float *delta,
                                     float *dq_acc, int32_t accumulate, void *stream);

/*
 * Gradients to the plan dtype: dq_out [T,hq,d], dk_out/dv_out [T,hkv,d];
 * unpermute = 1 writes packed token order.  No output may overlap another
 * output or an input.
 */
zz_status zz_finalize_bwd(const zz_plan *plan, const float *dq_acc, const float *dk_acc,
                          const float *dv_acc, void *dq_out, void *dk_out, void *dv_out,
                          int32_t unpermute, void *stream);

/*
 * Debug: the visibility a pass's kernels apply in ring step (rank, step) --
 * the causal mask (MaxText PR #1133, description: CP attention is causal) and
 * the document mask (EasyDeL issue #129: no attention across packed
 * examples) -- walking the same device tile lists and the same in-tile mask:
 * d_mask uint8 [(T/cp) x (T/cp)], row = rank-local query row, column =
 * shard-local key row; 1 = visible.  Every byte is written.
 */
zz_status zz_debug_mask(const zz_plan *plan, zz_pass pass, int32_t rank, int32_t step,
                        uint8_t *d_mask, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* ZZ_H */
