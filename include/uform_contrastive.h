/*
 * uform_contrastive.h -- C ABI of the fused Matryoshka contrastive loss on
 * AMD Instinct MI355X (gfx950): forward and backward in one asynchronous call.
 *
 * What it computes (pages cited by title and section):
 *  - "Scaling-Up Contrastive Learning over NVLink Multicast", section "One Set
 *    or Two": CLIP's row softmax over the batch and SigLIP's pairwise sigmoid
 *    loss L = -(1/N) sum_i sum_j log sigmoid(z_ij (t cos(x_i, y_j) + b)), with
 *    z = +1 for the positive pair and -1 for every negative; Matryoshka
 *    prefixes make every nested prefix of the embedding its own grid.
 *  - Same page, section "On the Chip: Tensor Memory & the Matryoshka Sweep":
 *    one sweep over the embedding serves every prefix; each cell's cosine is
 *    normalised with stored inverse norms; the N x N grid never reaches memory.
 *  - UForm README ("Multimodal Perception from 64 to 1024 Dimensions"),
 *    Matryoshka paragraph: nested prefixes {64, 128, 256, 512, 1024}; its
 *    training-stack paragraphs: BF16 storage, FP32 accumulation, FP32
 *    log-sum-exps and FP32 partial-gradient slabs.
 *  - "UForm for Swift", sections "Errors" and "Design": one C verb per
 *    operation named uform_<noun>_<verb>, statuses uform_status_*_k whose
 *    names read like "invalid-argument".
 *
 * Definitions (q: R query rows, k: N key rows, both D wide; prefix widths
 * P_1 < ... < P_n; weights w_p, W = sum w_p; s = scale, b = bias; the positive
 * of local row i is key row_offset + i):
 *   cos^p_ij = <q_i[:P_p], k_j[:P_p]> / (|q_i[:P_p]| |k_j[:P_p]|),
 *   l^p_ij   = s * cos^p_ij + b,
 *   INFONCE       (R == N, row_offset == 0): L^p = (1/2N) [ sum_i (LSE_j l_ij - l_ii)
 *                                                        + sum_j (LSE_i l_ij - l_jj) ]
 *   INFONCE_ROWS  L^p = (1/N) sum_{i<R} (LSE_{j<N} l_ij - l_{i,off+i}); also the
 *                 column partial log-sum-exp PLSE^p_j = LSE_{i<R} l_ij
 *   SIGLIP        L^p = (1/N) sum_{i<R} sum_{j<N} log(1 + exp(-z_ij l_ij))
 *   loss = sum_p w_p L^p / W.  Gradients dq = dloss/dq, dk = dloss/dk (FP32);
 *   entries beyond the widest prefix are 0.
 *
 * Ownership: the caller owns every buffer and the stream; the library never
 * frees caller memory.  Without a caller workspace the library keeps one
 * grow-only device workspace per (device, stream), allocated on first use
 * (synchronising that stream once when it grows) and freed by
 * uform_contrastive_release().
 *
 * Errors: every argument check runs on the host before any launch or write;
 * a failed check returns invalid-argument or unsupported and touches nothing.
 * A failed launch returns device-error.  Faults inside kernels surface at the
 * caller's next synchronisation.  No call synchronises the host with the
 * device except a workspace growth.  Calls that share a library workspace
 * must be ordered on one stream.
 */
#ifndef UFORM_CONTRASTIVE_H
#define UFORM_CONTRASTIVE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t *hipStream_t; /* NULL = the device's default stream */

typedef enum {
    uform_contrastive_infonce_k = 0,      /* symmetric CLIP 1/2 (row CE + column CE) */
    uform_contrastive_siglip_k = 1,       /* pairwise sigmoid, z = +1 at (i, off + i) */
    uform_contrastive_infonce_rows_k = 2, /* row CE of the R local rows + column PLSE */
    uform_contrastive_oneset_siglip_k = 3, /* one set scored against itself, sigmoid form (below) */
    uform_contrastive_oneset_siglip_edges_k = 4, /* the same with every positive listed as a relation (below) */
} uform_contrastive_kind_t;

/* The one-set sigmoid form ("Scaling-Up Contrastive Learning over NVLink
 * Multicast", section "One Set or Two": one set scored against itself, an
 * image and its caption two rows of the set marked as a positive pair,
 * mirrored cells with the same labels, the owner of a row differentiating
 * both).  k is the whole set [N][D] (N even; rows 2m and 2m + 1 are a pair),
 * q = k + row_offset * D its rows row_offset .. row_offset + R - 1 (checked).
 * loss_out is this share's part, (1/N) sum over its rows g and every j != g
 * of softplus(-z_gj l_gj), z = +1 at j = g xor 1; a cell of a row with
 * itself is not scored.  dq is the gradient of the whole set's loss with
 * respect to the share's rows (both mirrored cells); dk must be NULL.  One
 * backward pass, over the share's rows.
 *
 * The one-set form with listed relations (uform_contrastive_oneset_siglip_edges_k;
 * "UForm for Swift", section "Training": a training step takes relations
 * Relations(attract: Edges(offsets, ids)), CSR edge lists naming the items each
 * item attracts): the same loss, share and gradient, but no cell is an
 * implicit positive.  The options' pos_row_ptr / pos_col list the share's
 * rows' relations (set indices, any rows of the set other than the row
 * itself; a row may list none or several), and exactly the listed cells take
 * z = +1.  N may be odd.  Mirrored cells carry one label, so the whole set's
 * lists must be symmetric: a pair of two rows of the share listed one way only
 * is invalid-argument (a partner outside the share cannot be checked).  No
 * lists: every cell is a negative.  pos_logit_out must be NULL (a row has no
 * single positive). */

typedef enum {
    uform_status_success_k = 0,
    uform_status_invalid_argument_k = 1, /* a null or misaligned pointer, a bad size or prefix list */
    uform_status_unsupported_k = 2,      /* valid request outside the library's limits */
    uform_status_out_of_memory_k = 3,    /* workspace allocation failed */
    uform_status_device_error_k = 4,     /* a HIP call or a kernel launch failed */
} uform_status_t;

/* Limits of the library. */
#define UFORM_CONTRASTIVE_MAX_PREFIXES 8
#define UFORM_CONTRASTIVE_MAX_DIM 2048
/* Softmax kinds use one fixed log-sum-exp shift per call, exact while
 * 2 * |scale| * log2(e) stays inside FP32's normal exponent range. */
#define UFORM_CONTRASTIVE_MAX_SOFTMAX_SCALE 40.0f

/*
 * uform_contrastive_fwd_bwd -- loss and gradients in one call.
 *
 *  q, k        device, BF16 bit patterns, row-major [R][D] and [N][D] with
 *              leading dimension D, 16-byte aligned.
 *  R, N, D     1 <= R <= N; D % 64 == 0 and D <= 2048 (else unsupported):
 *              the widths of the UForm README's tier table, whose Large and
 *              XL tiers train the prefixes {64, ..., 1024, 2048}.
 *  prefixes    HOST array of n_prefixes widths, read during the call only:
 *              strictly increasing multiples of 32, last <= D;
 *              1 <= n_prefixes <= 8.
 *  scale, bias finite; softmax kinds need |scale| <= 40 (else unsupported).
 *  kind        a uform_contrastive_kind_t; INFONCE needs R == N; the one-set
 *              forms need q inside k and dk = NULL (see above).
 *  loss_out    device, 1 float: the weighted loss (written asynchronously).
 *  dq, dk      device FP32 [R][D] and [N][D], 16-byte aligned, overwritten;
 *              NULL skips that gradient.
 *  stream      every launch is enqueued on it in order; nothing waits.
 * Prefix weights default to 1 and the positive of row i is key i.
 */
uform_status_t uform_contrastive_fwd_bwd(const void *q, const void *k, int64_t R, int64_t N, int64_t D,
                                         const int32_t *prefixes, int32_t n_prefixes, float scale,
                                         float bias, int32_t kind, float *loss_out, float *dq, float *dk,
                                         hipStream_t stream);

typedef struct {
    const float *prefix_weights; /* host [n_prefixes], finite and > 0; NULL = all 1            */
    /* Key index of local row 0's positive; 0 <= off, off + R <= N.  A GPU that owns rows
     * off .. off + R - 1 of a batch scores them against every key with their global offset
     * ("Scaling-Up Contrastive Learning over NVLink Multicast", section "Across the Box:
     * Pointers, Not Gathers": each score call carries the local and the peer row offsets). */
    int64_t row_offset;
    float *prefix_losses_out;    /* device [n_prefixes]: unweighted L^p; nullable               */
    float *col_lse_out;          /* device [n_prefixes][N]: LSE over the R rows of column j
                                    (INFONCE: full column LSE; INFONCE_ROWS: the PLSE);
                                    softmax kinds only; nullable                                */
    float *row_lse_out;          /* device [n_prefixes][R]: LSE over the N keys of row i;
                                    softmax kinds only; nullable                                */
    float *pos_logit_out;        /* device [n_prefixes][R]: l^p_{i, off+i}; nullable            */
    /* Caller-lent device memory for every intermediate of the call ("UForm for Swift", section
     * "Arenas": results land in memory the caller passes, rewound by each call, so a steady
     * loop allocates nothing once it reaches its high-water mark).  256-byte aligned, at least
     * uform_contrastive_workspace_bytes(...) bytes (_ex with a positive list); its contents are
     * scratch, overwritten by the call; it serves one call at a time (calls that share it must
     * be ordered on one stream).  NULL = the library's cached workspace of (device, stream). */
    void *workspace;
    size_t workspace_bytes;
    uint32_t flags;              /* UFORM_CONTRASTIVE_* bits below (accumulate, diagnostics)    */
    /* Gradients of the loss with respect to the logit scale s and bias b (the
     * learned temperature and bias of "Scaling-Up Contrastive Learning over
     * NVLink Multicast", section "One Set or Two"): dL/ds = sum_p (w_p/W)
     * sum_ij g^p_ij cos^p_ij and dL/db = sum_p (w_p/W) sum_ij g^p_ij, g^p =
     * dL^p/dl^p.  dL/db is 0 for the softmax kinds (a common shift of a
     * softmax's logits cancels).  Device, 1 float each, overwritten (also with
     * UFORM_CONTRASTIVE_ACCUMULATE); they come from a gradient pass, so a call
     * that sets either must give dq or dk (else invalid-argument).  Nullable. */
    float *dscale_out;
    float *dbias_out;
    /* Several positives per entry, sigmoid kinds only (UForm README,
     * "Multimodal Perception from 64 to 1024 Dimensions", the training-stack
     * paragraph on loader-side properties: an entry may carry several
     * positives and explicit hard negatives, gathered as extra columns).  HOST CSR lists, read during the
     * call only: local row i's extra positives are the key (set) indices
     * pos_col[pos_row_ptr[i] .. pos_row_ptr[i + 1] - 1], and every listed cell
     * gets the label z = +1 like the row's own positive (loss, dq, dk,
     * dL/dscale, dL/dbias and L^p all follow).  pos_row_ptr has R + 1 entries
     * with pos_row_ptr[0] = 0 and never decreasing; a row's columns are
     * strictly increasing, in [0, N), and none of them is the row's own
     * positive (row_offset + i; in the one-set form its pair partner
     * (row_offset + i) xor 1 and the row itself).  A list that breaks this,
     * or a list with a softmax kind, is invalid-argument; more than 2^31 - 2
     * listed cells in one call is unsupported.  In the
     * one-set form list both (i, j) and (j, i) so that mirrored cells keep
     * equal labels.  Explicit hard negatives need no list: append them to k
     * as extra key rows (N > R), which every row scores as negatives.  The
     * lists reach the device through a pinned staging buffer per stream and a
     * copy enqueued on the stream; the call waits (on the host) only for the
     * previous call's list copy on that stream.  Such a call cannot be captured
     * into a graph.  A caller-given workspace must hold
     * uform_contrastive_workspace_bytes_ex(..., pos_row_ptr[R]) bytes.
     * pos_row_ptr = NULL: no extra positives. */
    const int64_t *pos_row_ptr;
    const int32_t *pos_col;
} uform_contrastive_options_t;

#define UFORM_CONTRASTIVE_ACCUMULATE 1u
/* Diagnostics: bracket each kernel launch of the call with a pair of events
 * on the stream (read them with uform_contrastive_profile). */
#define UFORM_CONTRASTIVE_PROFILE 2u
/* Diagnostics: run each backward pass as one inner split (no split partials; the
 * backward kernel applies the finalize terms itself, as it does whenever the
 * problem is large enough for one split to fill the GPU). */
#define UFORM_CONTRASTIVE_ONE_SPLIT 4u

/* As uform_contrastive_fwd_bwd, with the options above (options may be NULL). */
uform_status_t uform_contrastive_fwd_bwd_ex(const void *q, const void *k, int64_t R, int64_t N, int64_t D,
                                            const int32_t *prefixes, int32_t n_prefixes, float scale,
                                            float bias, int32_t kind, float *loss_out, float *dq, float *dk,
                                            hipStream_t stream, const uform_contrastive_options_t *options);

/* For callers that cannot allocate: code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc.  The same call as
 * uform_contrastive_fwd_bwd_ex (same arguments, checks, results and stream
 * order), but its workspace is a fixed device array of
 * UFORM_CONTRASTIVE_NOALLOC_SCRATCH_BYTES bytes per GPU, held from the first use
 * of the library on that GPU until the process ends; the call allocates
 * nothing (no hipMalloc, no pinned or event allocation).  A call whose
 * workspace would exceed the array (e.g. 16384 x 16384 InfoNCE) returns unsupported; so does a call with positive
 * lists or UFORM_CONTRASTIVE_PROFILE; options->workspace must be NULL
 * (invalid-argument otherwise).  Every call on one GPU shares that GPU's
 * array: calls that overlap on one GPU (on different streams, or from
 * different threads without ordering) race and give wrong results; order them
 * on one stream.  The array keeps the last call's contents; each call writes
 * every part of it that it reads. */
#define UFORM_CONTRASTIVE_NOALLOC_SCRATCH_BYTES (128u << 20)
uform_status_t uform_contrastive_fwd_bwd_noalloc(const void *q, const void *k, int64_t R, int64_t N, int64_t D,
                                                 const int32_t *prefixes, int32_t n_prefixes, float scale,
                                                 float bias, int32_t kind, float *loss_out, float *dq, float *dk,
                                                 hipStream_t stream, const uform_contrastive_options_t *options);

/* Device workspace a call of this shape needs, in bytes (gradients included,
 * enough for any prefix ladder of this count up to D); 0 for arguments the call
 * would reject.  The size of the caller-lent memory
 * of the options' workspace ("UForm for Swift", section "Arenas": the caller
 * sizes the memory a call lands in, and a loop that reuses it allocates once). */
size_t uform_contrastive_workspace_bytes(int64_t R, int64_t N, int64_t D, int32_t n_prefixes, int32_t kind);

/* As above, for a call that lists n_positives extra positives (pos_row_ptr[R];
 * sigmoid kinds only, else 0); n_positives < 0 means no list ("UForm for Swift",
 * section "Arenas", as above; the lists of the UForm README's loader-side
 * paragraph take n_positives int32 entries of it). */
size_t uform_contrastive_workspace_bytes_ex(int64_t R, int64_t N, int64_t D, int32_t n_prefixes, int32_t kind,
                                            int64_t n_positives);

/* Whether a call with this width, prefix ladder and kind can run, without
 * touching any device: success, invalid-argument or unsupported (the reason
 * is in uform_contrastive_last_error()).  The ladders are the nested prefixes
 * of the UForm README's Matryoshka paragraph ({64, 128, 256, 512, 1024} and
 * the shorter ladders of the narrower tiers); the statuses those of "UForm
 * for Swift", section "Errors".  The backward has kernels compiled for the
 * ladders {64,128,256,512,1024}, {64,128,256,512}, {64,128,256}, {64,128}
 * and the single widths {128}, {256}, {512}, {1024} (the fast path); every
 * other ladder, and every width above 1024, takes a generic backward, compiled
 * for the Large and XL tiers' {64, ..., 1024, 2048} and reading any other
 * ladder at run time.  Its LDS bounds the ladders it takes: above 1024 at most 6
 * prefixes, at most 3 of them ending strictly inside a quarter of the widest
 * (as 64, 128 and 256 do in {64, ..., 2048}); a ladder past that is
 * unsupported.  A softmax call without gradients accepts any valid ladder. */
uform_status_t uform_contrastive_supported(int64_t D, const int32_t *prefixes, int32_t n_prefixes, int32_t kind,
                                          int32_t with_gradients);

/* "success", "invalid-argument", "unsupported", "out-of-memory", "device-error";
 * "unknown" otherwise.  Static strings ("UForm for Swift", section "Errors":
 * statuses uform_status_*_k whose names read like "invalid-argument"). */
const char *uform_status_name(uform_status_t status);

/* Human-readable reason of this thread's last non-success status ("" if none)
 * ("UForm for Swift", section "Errors": a failed verb reports its status and
 * the reason beside it). */
const char *uform_contrastive_last_error(void);

/* Diagnostics for calls made with UFORM_CONTRASTIVE_PROFILE: waits for their
 * events and writes up to cap (kernel name, summed milliseconds) pairs, one
 * per kernel, covering every profiled call since the previous read (which it
 * clears).  Returns the number of distinct kernels.  Names are static.  (The
 * per-stage times behind a loss-step time such as "Scaling-Up Contrastive
 * Learning over NVLink Multicast", section "Bird's Eye View & the Results",
 * reports; section "On the Chip" attributes the step to its kernels.) */
int32_t uform_contrastive_profile(const char **names, float *ms, int32_t cap);

/* Frees the library's cached workspaces and pinned list staging (waits for
 * their streams first).  The cached workspace is the library's own arena of
 * "UForm for Swift", section "Arenas" (allocated once at its high-water mark
 * per device and stream); this returns it. */
void uform_contrastive_release(void);

#ifdef __cplusplus
}
#endif

#endif /* UFORM_CONTRASTIVE_H */
