/*
 * vggt_attn.h -- C ABI of an MI355X (gfx950) library for the forward pass of VGGT's global
 * cross-frame self-attention, out = softmax(Q K^T / sqrt(d)) V, over N frames of
 * L = n_special + gh*gw tokens, in four forms:
 *
 *   dense        every token is a key ("AVGGT: Rethinking Global Attention for Accelerating
 *                VGGT", papernotes.org CVPR 2026 notes, 关键设计 2, the attention equation);
 *   SGA          all queries kept; K/V restricted to the set S = the first patch of every
 *                s_h x s_w window, every camera/register token, and (VGGT) all of frame 0;
 *                sigma = s_h*s_w with 2->(1,2), 4->(2,2), 6->(2,3), 9->(3,3) (same notes,
 *                关键设计 2; gist.science summary of the paper, "Technische Zusammenfassung" 2.B);
 *   enhanced SGA S plus a diagonal self term and one mean K/V per compressed frame, all under a
 *                single softmax (AVGGT notes, 关键设计 3); the weight of the mean term is a flag:
 *                unit, or ln|D_f| added to its logit, the size bias of "RegimeVGGT: Layer-Wise
 *                Spatially Preserving Redundancy Removal ..." (papernotes.org NeurIPS 2026
 *                notes, 关键设计 2);
 *   G2F          Global-to-Frame: each frame attends only to its own L tokens (AVGGT notes,
 *                关键设计 1);
 *   G2M          Global-to-Mean: K/V of every query is one token, the mean of K and of V over
 *                all T tokens (AVGGT notes, ablation table, row VGGT(G2M)), so every output row
 *                is that mean value.
 * Two options refine SGA: a phase-shifted sampling grid (RegimeVGGT notes, 关键设计 3: the grid
 * of frame f is offset per frame so that consecutive frames together cover every patch) and a
 * global scope for the mean term (one mean over every dropped patch of every frame).  Size-aware
 * keys (RegimeVGGT notes, 关键设计 2): with LOG_SIZE each token carries a caller-supplied
 * log g (the number of source tokens it stands for) added to its logit wherever it is a key.
 *
 * Conventions shared by every entry point
 *   - Tensors q, k, v, out are dense row-major [H][T][d], T = N*L, batch 1.  Within a frame
 *     the n_special camera/register tokens come first, then the patches row-major (token
 *     f*L + n_special + r*gw + c is patch (r, c) of frame f).
 *   - Device pointers are HIP device addresses owned by the caller; the library never
 *     allocates, frees or retains device memory.  `workspace` is caller-owned scratch of at
 *     least vggt_attn_workspace_bytes() bytes; its contents between calls are not meaningful
 *     except as documented for vggt_attn_pack / vggt_attn_copy_index_set.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).  Device work is
 *     only enqueued; execution errors surface at the caller's next synchronisation.
 *   - Every int-returning call returns a vggt_attn_status (0 = success) and on failure
 *     vggt_attn_last_error() holds a description (thread-local).  Every argument and plan check
 *     comes before the first launch, so a failure other than EHIP enqueues nothing.  EHIP means
 *     a launch was refused by the runtime; a call that launches several kernels (the pack stage:
 *     means, then pack; the attention stage: main kernel, split pieces, merge) may then have
 *     enqueued the kernels before the refused one, and the output and workspace contents are
 *     undefined until a later call succeeds.
 *   - Plans are immutable host objects: concurrent calls with one plan are safe as long as
 *     each call has its own workspace and output.
 *   - The pack, attend and forward entry points enqueue kernel launches only (no memset, copy,
 *     allocation or host synchronisation), so a caller may capture them into a HIP graph and
 *     replay it; vggt_attn_copy_index_set copies to host memory and synchronises, so it may not.
 */
#ifndef VGGT_ATTN_H
#define VGGT_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  VGGT_ATTN_OK = 0,
  VGGT_ATTN_EINVAL = -1,       /* invalid argument or descriptor                          */
  VGGT_ATTN_EUNSUPPORTED = -2, /* valid request the library does not implement (head_dim) */
  VGGT_ATTN_ENOSPC = -3,       /* workspace smaller than vggt_attn_workspace_bytes()      */
  VGGT_ATTN_EALIGN = -4,       /* a device pointer is not 16-byte aligned                 */
  VGGT_ATTN_EALIAS = -5,       /* out overlaps q, k, v or the workspace                   */
  VGGT_ATTN_EHIP = -6          /* a HIP runtime call or kernel launch failed              */
} vggt_attn_status;

/* Element types. */
enum { VGGT_ATTN_BF16 = 0, VGGT_ATTN_FP32 = 1 };

/* Form flags (bitwise OR). */
enum {
  VGGT_ATTN_G2F = 1u << 0,        /* per-frame attention; needs sigma == 1, no DIAG/MEAN       */
  VGGT_ATTN_REF_DENSE = 1u << 1,  /* frame 0 kept dense as K/V (VGGT); clear = every frame
                                     compressed alike (pi^3) -- AVGGT notes, 关键设计 2         */
  VGGT_ATTN_DIAG = 1u << 2,       /* diagonal self term for queries whose token is not in S    */
  VGGT_ATTN_MEAN = 1u << 3,       /* one mean K/V per compressed frame, over its dropped patches */
  VGGT_ATTN_MEAN_COUNT = 1u << 4, /* mean logit += ln|D_f|, else the mean is one plain token    */
  VGGT_ATTN_PRESCALE_Q = 1u << 5, /* bf16 path: fold the softmax scale into Q and form Q K^T on
                                     the f16 matrix cores.  The pack stage converts the packed keys
                                     of head h to f16 after scaling them by 2^-e_h, where e_h puts
                                     the head's largest packed |k| in [128, 256) (exact for every
                                     |k| above 2^-21 of that maximum); the attention stage rounds
                                     Q * tau * log2(e) * 2^e_h to f16 once.  Saves one multiply
                                     per score (5-6% faster at 800 frames); each logit term then carries a
                                     relative error of up to 2^-11.  Without the flag Q and K are
                                     used exactly as given and the scale is applied in float32.
                                     G2F plans with the flag pack K and V like the global forms.
                                     Ignored for fp32 inputs and with LOG_SIZE.                    */
  VGGT_ATTN_PHASE_SHIFT = 1u << 6, /* SGA grid of frame f offset by row (f div s_w) mod s_h and
                                     column f mod s_w (RegimeVGGT notes, 关键设计 3, whose t x t
                                     formula this is for square windows): frame f keeps patch
                                     (r, c) iff r % s_h and c % s_w equal those offsets.  Frame 0
                                     (with REF_DENSE) and the specials stay dense.  |D_f| then
                                     depends on f; no effect when sigma == 1.                     */
  VGGT_ATTN_MEAN_GLOBAL = 1u << 7, /* with MEAN: one mean K/V over the union of all frames'
                                     dropped patches instead of one per frame; MEAN_COUNT then adds
                                     ln(sum_f |D_f|).  Requires MEAN.                              */
  VGGT_ATTN_G2M = 1u << 8,         /* Global-to-Mean (see above); needs sigma == 1 and none of
                                     G2F, DIAG, MEAN, MEAN_GLOBAL, PHASE_SHIFT.                     */
  VGGT_ATTN_LOG_SIZE = 1u << 9     /* size-aware keys: the logit of token key t (in S, the diagonal
                                     self term, a G2F frame) gets + log_g[t], log_g passed to the
                                     *_sized entry points.  Not with MEAN or G2M (EINVAL); the
                                     bf16 path then ignores PRESCALE_Q.                            */
};

typedef struct vggt_attn_plan_s vggt_attn_plan_t;

/* Where each part of a workspace lives, in bytes from its start (all 256-byte aligned), and
 * the packed key geometry.  Packed keys of one head form `segments` segments of
 * `segment_rows` rows (one segment per head in the global forms, one per frame under G2F);
 * rows [0, keys_per_segment) are valid, the rest are zero padding up to a multiple of 64. */
typedef struct {
  int64_t segments;          /* per head                                                     */
  int64_t segment_rows;      /* padded rows per segment (multiple of 64)                     */
  int64_t keys_per_segment;  /* |S| + M (global forms) or L (G2F)                            */
  int64_t off_index;         /* int32[|S|]: S as ascending global token ids                  */
  int64_t off_dcount;        /* int32[N]: |D_f| per frame (0 for dense frames)               */
  int64_t off_means;         /* [H][M][2][d] input dtype: mean key, mean value               */
  int64_t off_partial;       /* float [H][F][2][d]: per-frame sums of a global mean (F frames
                                contribute; MEAN_GLOBAL and G2M only, else empty)             */
  int64_t off_kbias;         /* float [segments*segment_rows]: logit bias of each packed key
                                in raw-score units, log_g[t] * sqrt(d) (LOG_SIZE only)        */
  int64_t off_logsize;       /* float [T]: copy of log_g (LOG_SIZE only)                      */
  int64_t off_part;          /* float: partial softmax states (running max, sum, unnormalised
                                output) of the key-range pieces of a split last round of
                                work-groups, merged before the call returns (bf16 inputs)     */
  int64_t split_pieces;      /* key-range pieces per work item of that round (0 = no split)   */
  int64_t off_kmax;          /* uint32 [H]: bf16 bits of the largest |k| among the packed keys
                                of each head, which sets the f16 key scale (PRESCALE_Q only) */
  int64_t off_kpack;         /* [H][segments*segment_rows][d] input dtype (PRESCALE_Q: f16,
                                each head's rows scaled by 2^-e_h, see the flag)              */
  int64_t off_vpack;         /* bf16: [H][rows/64][d][64] key-minor tiles (see below);
                                fp32: [H][rows][d].  Both parts are empty (off_kpack ==
                                off_vpack == total_bytes) for bf16 G2F plans without
                                PRESCALE_Q, whose attention stage reads k and v directly (a
                                frame's keys are its tokens)                                  */
  int64_t total_bytes;
} vggt_attn_layout_t;

/* Build a plan (host only; no device call is made, so it works without a GPU).
 * Operation: AVGGT notes 关键设计 1-3 and RegimeVGGT notes 关键设计 3 as summarised at the top
 * of this header.
 *   frames >= 1, grid_h >= 1, grid_w >= 1, 0 <= n_special, heads >= 1;
 *   head_dim must be 64 (else EUNSUPPORTED);
 *   sigma in {1, 2, 4, 6, 9} (else EINVAL); sigma = 1 is dense attention (DIAG/MEAN/PHASE_SHIFT
 *     then have no effect: no token is dropped);
 *   G2F requires sigma == 1 and none of DIAG, MEAN, MEAN_GLOBAL, PHASE_SHIFT, G2M (EINVAL);
 *   G2M requires sigma == 1 and none of G2F, DIAG, MEAN, MEAN_GLOBAL, PHASE_SHIFT (EINVAL);
 *   MEAN_GLOBAL requires MEAN (EINVAL); LOG_SIZE excludes MEAN and G2M (EINVAL);
 *   a mean key exists for each frame whose dropped set is nonempty (one in all under
 *     MEAN_GLOBAL and G2M); with PHASE_SHIFT a one-patch-wide grid can leave some frames'
 *     dropped sets empty;
 *   (in_dtype, out_dtype) in {(BF16, FP32), (BF16, BF16), (FP32, FP32)} (EINVAL);
 *   T = frames*L must not exceed 8,000,000 and heads 4096 (EINVAL).
 * On success *out owns a plan to be released with vggt_attn_plan_destroy(). */
int vggt_attn_plan(vggt_attn_plan_t** out, int frames, int grid_h, int grid_w, int n_special,
                   int heads, int head_dim, int sigma, unsigned flags, int in_dtype,
                   int out_dtype);

/* Release a plan (NULL is ignored). */
void vggt_attn_plan_destroy(vggt_attn_plan_t* plan);

/* Workspace size in bytes for vggt_attn_forward / vggt_attn_pack (0 if plan is NULL). */
size_t vggt_attn_workspace_bytes(const vggt_attn_plan_t* plan);

/* Sizes of the call: n_kv = |S| (L under G2F, 0 under G2M), n_mean = M (number of mean keys),
 * n_diag = number of queries with a diagonal term, flops = algorithmic FLOPs of one forward:
 * 4*d*H*(T*(|S|+M) + n_diag) for the global forms (G2M: |S| = 0, M = 1), 4*d*H*N*L^2 for G2F
 * (QK^T and PV multiply-adds of attended keys only).  Any output pointer may be NULL. */
int vggt_attn_counts(const vggt_attn_plan_t* plan, int64_t* n_kv, int64_t* n_mean,
                     int64_t* n_diag, double* flops);

/* Workspace layout of the plan (see vggt_attn_layout_t). */
int vggt_attn_layout(const vggt_attn_plan_t* plan, vggt_attn_layout_t* out);

/* Full forward: vggt_attn_pack followed by vggt_attn_attend on `stream` (not for LOG_SIZE plans:
 * see vggt_attn_forward_sized).  Computes, for every query token t and head h, out[h][t] =
 * sum_j w_j v_j with w = softmax over the plan's keys of tau * <q_t, k_j> (tau = 1/sqrt(d)), one
 * normalisation over the kept set S, the diagonal self term and the mean keys together (AVGGT
 * notes, 关键设计 2, the attention equation restricted to S; 关键设计 3, the three terms under a
 * single softmax; 关键设计 1, G2F keys = the query's own frame).
 * q, k, v: [H][T][d] of the input dtype; out: [H][T][d] of the output dtype; every pointer
 * 16-byte aligned; out must not overlap q, k, v or the workspace (EALIAS). */
int vggt_attn_forward(const vggt_attn_plan_t* plan, const void* q, const void* k, const void* v,
                      void* out, void* workspace, size_t workspace_bytes, void* stream);

/* Gather/pack stage (AVGGT notes 关键设计 2 and 3): writes S (ascending token ids) and |D_f|
 * into the workspace, the mean keys/values (float32 sums divided by the number of tokens they
 * stand for, rounded to the input dtype: per frame over its dropped patches, or once over all
 * dropped patches with MEAN_GLOBAL, or once over all T tokens with G2M) and their logit
 * biases, and the packed keys and values: rows [0,|S|) are exact copies of K/V rows of S, rows
 * [|S|, |S|+M) the means, padding rows zero.  Under sigma = 1 it packs every token; under G2F
 * float32 plans pack every token frame by frame, while bf16 plans write |D_f| only, since their
 * attention stage reads k and v in place (with PRESCALE_Q they pack frame by frame too).  With
 * PRESCALE_Q the packed keys are then converted to f16 as the flag describes, and off_kmax holds
 * each head's largest packed |k|.  |D_f| is L for every frame under G2M.  Reads k and v only. */
int vggt_attn_pack(const vggt_attn_plan_t* plan, const void* k, const void* v, void* workspace,
                   size_t workspace_bytes, void* stream);

/* Attention stage (AVGGT notes, 关键设计 2 and 3: softmax(tau Q K^T) V over the packed keys,
 * the diagonal self term and the mean keys in one normalisation; 关键设计 1 for G2F) on a
 * workspace already filled by vggt_attn_pack for the same plan and the
 * same k, v (k and v are read again for the diagonal term, and for every key by bf16 G2F
 * plans without PRESCALE_Q, which keep no packed copy).  Writes every element of out.  It
 * uses the workspace's off_part area as scratch (the partial softmax states of a split last
 * round of work-groups, see vggt_attn_layout_t) and leaves the packed parts unchanged, so it
 * may be called again on the same workspace. */
int vggt_attn_attend(const vggt_attn_plan_t* plan, const void* q, const void* k, const void* v,
                     void* out, void* workspace, size_t workspace_bytes, void* stream);

/* The same calls for a LOG_SIZE plan (vggt_attn_forward and vggt_attn_pack return EINVAL for
 * one, and these return EINVAL for a plan without LOG_SIZE).  log_g: device float [T], 4-byte
 * aligned, the natural log of the number of source tokens token t stands for (0 for a plain
 * token), shared by all heads; values must be finite.  The pack stage copies what the attention
 * stage needs into the workspace, so vggt_attn_attend takes no log_g.  out must not overlap
 * log_g, and the workspace must not overlap log_g (EALIAS). */
int vggt_attn_forward_sized(const vggt_attn_plan_t* plan, const void* q, const void* k,
                            const void* v, const float* log_g, void* out, void* workspace,
                            size_t workspace_bytes, void* stream);
int vggt_attn_pack_sized(const vggt_attn_plan_t* plan, const void* k, const void* v,
                         const float* log_g, void* workspace, size_t workspace_bytes,
                         void* stream);

/* vggt_attn_forward for callers that cannot allocate device memory or pass a workspace --
 * code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.  The
 * workspace is a static device array inside the library, 256 MiB (268,435,456 bytes) on each GPU
 * the library runs on, held from the library's load until the process ends; its device address
 * is looked up once per device on the first call (a host-side lookup, no allocation).  The call
 * itself allocates and frees nothing and only enqueues kernels on `stream`.
 *   - Plans whose vggt_attn_workspace_bytes() exceeds 268,435,456 are refused with ENOSPC
 *     (800 frames of 1374 tokens at 16 heads need about 800 MiB: use vggt_attn_forward).
 *   - LOG_SIZE plans are refused (EINVAL).  Tensor checks as for vggt_attn_forward.
 *   - Every call on one GPU uses that GPU's single array, which keeps the last call's
 *     contents (no part of it needs to start cleared: the pack stage writes everything the
 *     attention stage reads).  Calls that can run at the same time on one GPU -- on different
 *     streams, or from several host threads without ordering -- race on it and give undefined
 *     results; calls on one stream are ordered and safe. */
int vggt_attn_forward_noalloc(const vggt_attn_plan_t* plan, const void* q, const void* k,
                              const void* v, void* out, void* stream);

/* Models whose global-layer schedule vggt_attn_layer_schedule knows. */
enum { VGGT_ATTN_MODEL_VGGT = 0, VGGT_ATTN_MODEL_PI3 = 1 };

/* The form of global layer `layer` (0..23) under AVGGT (AVGGT notes, 整体框架: the 24 global
 * layers, numbered 0-23, fall into an early part converted to Global-to-Frame -- indices below
 * t_early, 9 for VGGT and 10 for pi^3 --, a middle part that keeps global attention with K/V
 * subsampled by sigma and the diagonal and mean terms, and a late part kept unchanged; the
 * ablation table's row AVGGT(2)- names the late part as layers 20-23).  Host only.
 * Writes the sigma and flags to pass to vggt_attn_plan: G2F (sigma 1) for an early layer;
 * sigma with DIAG | MEAN, plus REF_DENSE for VGGT (frame 0 kept dense; pi^3 compresses every
 * frame, 关键设计 2), for a middle layer; sigma 1 and no flag (dense) for a late layer.
 * model: VGGT_ATTN_MODEL_VGGT or VGGT_ATTN_MODEL_PI3; sigma in {1, 2, 4, 6, 9} (1 keeps the
 * middle layers dense); layer in [0, 24).  Anything else: EINVAL.  Either output may be NULL. */
int vggt_attn_layer_schedule(int model, int layer, int sigma, int* out_sigma, unsigned* out_flags);

/* Copy S (|S| int32, ascending token ids) and |D_f| (N int32) from a packed workspace to host
 * memory; waits for `stream`.  S is the kept set of AVGGT notes 关键设计 2 (the first patch of
 * each s_h x s_w window of every compressed frame, every special token, every token of a dense
 * frame; RegimeVGGT notes 关键设计 3 for the phase-shifted grid); |D_f| counts the patches of
 * frame f outside S, the tokens its mean key stands for (关键设计 3).  Either host pointer may be
 * NULL.  Under G2F there is no S and host_idx is left untouched. */
int vggt_attn_copy_index_set(const vggt_attn_plan_t* plan, const void* workspace,
                             int32_t* host_idx, int32_t* host_dcount, void* stream);

/* Thread-local description of the last failure on this thread ("" if none). */
const char* vggt_attn_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* VGGT_ATTN_H */
