"""FP64 oracle: the Matryoshka contrastive loss written out from its definition.

TEST INFRASTRUCTURE ONLY (see the package docstring).  Slow on purpose: every
prefix is normalised on its own, every logit is formed explicitly, and the
gradients are the textbook chain rule through the L2 normalisation.  Rows are
processed in blocks only to bound memory; each block is the same formula
applied to a slice of rows (or columns), and partial column statistics are
merged in fixed block order.

Sources (cited by page title and section):

* "Scaling-Up Contrastive Learning over NVLink Multicast", section "One Set or
  Two": CLIP turns each row of cosines into a softmax over the batch; the
  SigLIP equation L = -(1/N) sum_i sum_j log sigmoid(z_ij (t cos(x_i, y_j) + b))
  with z = +1 for the positive pair and -1 for every negative; Matryoshka
  prefixes 64/128/256/512 plus the full width give five grids.
* Same page, section "On the Chip: Tensor Memory & the Matryoshka Sweep":
  every cell of every prefix needs a normalised cosine.
* UForm README ("Multimodal Perception from 64 to 1024 Dimensions"), the
  Matryoshka paragraph (nested prefixes {64, 128, 256, 512, 1024}) and the
  training-stack paragraphs (BF16 storage, FP32 accumulation, FP32
  log-sum-exps and partial-gradient slabs).

Readings where the pages leave a step open:

* two-set loss: queries q (R rows) against keys k (N rows); the positive of
  local row i is column ``row_offset + i``;
* symmetric InfoNCE is the CLIP convention 1/2 (row CE + column CE);
* every kind is normalised by the global N so that row shards sum to the
  whole loss; SigLIP's 1/N is the printed one;
* prefixes are combined as the weighted mean sum_p w_p L^p / sum_p w_p;
* ``scale`` multiplies the cosine as given (no exp() reparametrisation).
"""

from __future__ import annotations

import contextlib
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

INFONCE = 0
SIGLIP = 1
INFONCE_ROWS = 2
ONESET_SIGLIP = 3
ONESET_EDGES = 4
KIND_NAMES = {INFONCE: "infonce", SIGLIP: "siglip", INFONCE_ROWS: "infonce_rows", ONESET_SIGLIP: "oneset_siglip",
              ONESET_EDGES: "oneset_siglip_edges"}


# --------------------------------------------------------------------------
# small numerical helpers, each a plain definition
# --------------------------------------------------------------------------

def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Widen BF16 bit patterns (uint16) to float64 exactly."""
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def prefix_normalise(x: np.ndarray, width: int):
    """Return (x[:, :width] / ||x[:, :width]||, ||x[:, :width]||) row by row."""
    xp = x[:, :width]
    norm = np.sqrt(np.sum(xp * xp, axis=1))
    return xp / norm[:, None], norm


def logsumexp(a: np.ndarray, axis: int) -> np.ndarray:
    """log(sum(exp(a))) along ``axis`` with the usual max shift."""
    m = np.max(a, axis=axis, keepdims=True)
    return np.squeeze(m + np.log(np.sum(np.exp(a - m), axis=axis, keepdims=True)), axis=axis)


def softplus(x: np.ndarray) -> np.ndarray:
    """log(1 + e^x) = -log sigmoid(-x), written without overflow."""
    return np.maximum(x, 0.0) + np.log1p(np.exp(-np.abs(x)))


def sigmoid(x: np.ndarray) -> np.ndarray:
    """1 / (1 + e^-x), written without overflow."""
    e = np.exp(-np.abs(x))
    return np.where(x >= 0, 1.0 / (1.0 + e), e / (1.0 + e))


# --------------------------------------------------------------------------
# the loss
# --------------------------------------------------------------------------

def _positive_mask(rows: np.ndarray, cols: np.ndarray, row_offset: int, kind: int) -> np.ndarray:
    """E[a, b] = 1 where column cols[b] is the implicit positive of row rows[a]: key row_offset + row
    for the two-set kinds; for the one-set form, the other row of the row's pair,
    (row_offset + row) xor 1; none for the one-set form whose positives are all listed."""
    g = rows[:, None] + row_offset
    if kind == ONESET_EDGES:
        return np.zeros((len(rows), len(cols)))
    return (cols[None, :] == (g ^ 1 if kind == ONESET_SIGLIP else g)).astype(np.float64)


def _listed_mask(rows: np.ndarray, cols: np.ndarray, positives) -> np.ndarray:
    """1 where (rows[a], cols[b]) is one of the listed extra positive pairs (CSR: row_ptr, col);
    rows and cols are contiguous index ranges."""
    E = np.zeros((len(rows), len(cols)))
    if positives is None:
        return E
    row_ptr, pcol = positives
    r0, r1, c0 = int(rows[0]), int(rows[-1]) + 1, int(cols[0])
    owner = np.repeat(np.arange(r0, r1), np.diff(row_ptr[r0:r1 + 1]))  # the row of each listed entry
    col = pcol[row_ptr[r0]:row_ptr[r1]]
    inside = (col >= c0) & (col < c0 + len(cols))
    E[owner[inside] - r0, col[inside] - c0] = 1.0
    return E


def check_positives(positives, R: int, N: int, row_offset: int, kind: int):
    """Validate a positive list and return it as (row_ptr int64 [R + 1], col int64 [nnz]).

    Row i's listed positives are col[row_ptr[i]:row_ptr[i + 1]]: strictly increasing key (set)
    indices in [0, N), none of them the row's implicit positive (row_offset + i, or its pair partner
    (row_offset + i) xor 1 in the one-set form) and, in both one-set forms, not the row itself.  In
    the one-set forms mirrored cells carry one label, so a listed pair of two rows of the share
    must be listed both ways."""
    row_ptr = np.asarray(positives[0], dtype=np.int64)
    col = np.asarray(positives[1], dtype=np.int64)
    if row_ptr.shape != (R + 1,) or row_ptr[0] != 0 or np.any(np.diff(row_ptr) < 0) or row_ptr[-1] != len(col):
        raise ValueError("row_ptr must have R + 1 non-decreasing entries from 0 to len(col)")
    oneset = kind in (ONESET_SIGLIP, ONESET_EDGES)
    for i in range(R):
        c = col[row_ptr[i]:row_ptr[i + 1]]
        g = row_offset + i
        own = {SIGLIP: g, ONESET_SIGLIP: g ^ 1}.get(kind, -1)
        if np.any(c < 0) or np.any(c >= N) or np.any(np.diff(c) <= 0) or np.any(c == own) or (oneset and np.any(c == g)):
            raise ValueError(f"row {i}: listed positives must be increasing, in [0, N), and not the row's own pair")
    if oneset:
        listed = set(zip(np.repeat(np.arange(R) + row_offset, np.diff(row_ptr)).tolist(), col.tolist()))
        for g, j in listed:
            if row_offset <= j < row_offset + R and (j, g) not in listed:
                raise ValueError(f"rows {g} and {j} of the share: a one-set pair must be listed both ways")
    return row_ptr, col


def _self_mask(rows: np.ndarray, cols: np.ndarray, row_offset: int) -> np.ndarray:
    """1 where column cols[b] is row rows[a] itself (one-set form: the cell is not scored)."""
    return (cols[None, :] == (rows[:, None] + row_offset)).astype(np.float64)


def _default_block(n: int) -> int:
    return int(max(16, min(512, (1 << 23) // max(n, 1))))


def contrastive_fwd_bwd(q, k, prefixes, scale, bias, kind, weights=None, row_offset=0,
                        grads=True, threads=None, block=None, positives=None):
    """Loss, per-prefix losses, statistics and gradients of the Matryoshka loss.

    q: [R, D] queries, k: [N, D] keys (any real values; the tests pass
    BF16-rounded values widened to float64).  ``prefixes`` are the nested
    widths P_1 < ... < P_P <= D, ``weights`` their weights (default all 1).
    ``kind`` is INFONCE (symmetric CLIP, needs R == N and row_offset == 0),
    INFONCE_ROWS (row cross-entropy of the R local rows against all N keys,
    plus the column partial log-sum-exp over the local rows), SIGLIP, or
    ONESET_SIGLIP: one set scored against itself ("Scaling-Up Contrastive
    Learning over NVLink Multicast", section "One Set or Two": an image and its
    caption are two rows of the set marked as a positive pair; mirrored cells
    carry the same labels, and the owner of a row differentiates both).  Then
    ``k`` is the whole set [N, D] (N even; rows 2m and 2m + 1 are a pair), ``q``
    its rows row_offset .. row_offset + R - 1, the loss is this share's part
    (1/N) sum over local rows i and every j other than i itself of
    softplus(-z_ij l_ij), and ``dq`` is the gradient of the whole set's loss
    with respect to those rows (both mirrored cells), with no ``dk``.
    ONESET_EDGES is the same one-set form with no implicit pairs: every
    positive of the set is listed in ``positives`` (the relation edges of
    "UForm for Swift", section "Training": an item attracts the items its
    edge list names), a row may list none, several, or any other row of the
    set, N may be odd, and there is no ``pos_logit``.  Mirrored cells carry one
    label, so the whole set's lists are symmetric (checked within the share).

    ``positives`` (sigmoid kinds only) = (row_ptr, col) lists extra positive
    pairs in CSR form: each entry of the batch may carry several positives
    (UForm README, "Multimodal Perception from 64 to 1024 Dimensions", the
    training-stack paragraph on loader-side properties), and a listed cell gets the label
    z = +1 like the row's own positive.  In the one-set form the caller lists
    both (i, j) and (j, i) so that mirrored cells keep equal labels.

    Returns a dict with ``loss`` (float), ``prefix_losses`` [P], ``row_lse``
    [P, R] (log-sum-exp of each row's logits; InfoNCE kinds), ``pos_logit``
    [P, R], ``col_lse`` [P, N] (log-sum-exp over the R rows of each column's
    logits; InfoNCE kinds) and, when ``grads``, ``dq`` [R, D], ``dk`` [N, D],
    ``dscale`` = dL/ds = sum_p (w_p/W) sum_ij g^p_ij cos^p_ij and ``dbias`` =
    dL/db = sum_p (w_p/W) sum_ij g^p_ij, with g^p = dL^p/dl^p the residual
    (the learned temperature and bias of the sigmoid form: "Scaling-Up
    Contrastive Learning over NVLink Multicast", section "One Set or Two").
    """
    q = np.ascontiguousarray(q, dtype=np.float64)
    k = np.ascontiguousarray(k, dtype=np.float64)
    if q.ndim != 2 or k.ndim != 2 or q.shape[1] != k.shape[1]:
        raise ValueError("q and k must be [R, D] and [N, D]")
    R, D = q.shape
    N = k.shape[0]
    prefixes = [int(p) for p in prefixes]
    P = len(prefixes)
    if P < 1 or any(b <= a for a, b in zip(prefixes, prefixes[1:])) or prefixes[0] < 1 or prefixes[-1] > D:
        raise ValueError("prefixes must be strictly increasing widths in [1, D]")
    if kind not in KIND_NAMES:
        raise ValueError("unknown kind")
    if R < 1 or R > N or row_offset < 0 or row_offset + R > N:
        raise ValueError("need 1 <= R <= N and row_offset + R <= N")
    if kind == INFONCE and (R != N or row_offset != 0):
        raise ValueError("symmetric InfoNCE needs R == N and row_offset == 0")
    oneset = kind in (ONESET_SIGLIP, ONESET_EDGES)
    if oneset and not np.array_equal(q, k[row_offset:row_offset + R]):
        raise ValueError("the one-set forms need q = k[row_offset:row_offset + R]")
    if kind == ONESET_SIGLIP and N % 2 != 0:
        raise ValueError("the one-set form with pairs needs an even set (rows 2m and 2m + 1 pair up)")
    if positives is not None:
        if kind not in (SIGLIP, ONESET_SIGLIP, ONESET_EDGES):
            raise ValueError("listed positives are defined for the sigmoid kinds")
        positives = check_positives(positives, R, N, row_offset, kind)
    w = np.ones(P) if weights is None else np.asarray(weights, dtype=np.float64)
    W = float(np.sum(w))
    s = float(scale)
    b = float(bias)
    threads = threads or len(os.sched_getaffinity(0))
    block = block or _default_block(N)

    row_blocks = [(r0, min(R, r0 + block)) for r0 in range(0, R, block)]
    col_blocks = [(c0, min(N, c0 + block)) for c0 in range(0, N, block)]
    all_rows = np.arange(R)
    all_cols = np.arange(N)
    pos_col = row_offset + all_rows

    prefix_losses = np.zeros(P)
    row_lse = np.zeros((P, R))
    col_lse = np.zeros((P, N))
    pos_logit = np.zeros((P, R))
    dq = np.zeros((R, D)) if grads else None
    dk = np.zeros((N, D)) if grads and not oneset else None
    dscale = 0.0
    dbias = 0.0

    with _blas_single_thread(), ThreadPoolExecutor(max_workers=threads) as pool:
        for p, width in enumerate(prefixes):
            qh, qnorm = prefix_normalise(q, width)
            kh, knorm = prefix_normalise(k, width)

            # ---- forward: every logit l_ij = s * cos_ij + b, one row block at a time
            def forward_rows(rb):
                r0, r1 = rb
                logits = s * (qh[r0:r1] @ kh.T) + b
                rows = all_rows[r0:r1]
                pos = logits[rows - r0, pos_col[r0:r1]]
                out = {"pos": pos}
                if oneset:
                    if kind == ONESET_SIGLIP:
                        out["pos"] = logits[rows - r0, pos_col[r0:r1] ^ 1]
                    z = 2.0 * (_positive_mask(rows, all_cols, row_offset, kind)
                               + _listed_mask(rows, all_cols, positives)) - 1.0
                    keep = 1.0 - _self_mask(rows, all_cols, row_offset)
                    out["siglip_rows"] = np.sum(keep * softplus(-z * logits), axis=1)
                elif kind == SIGLIP:
                    z = 2.0 * (_positive_mask(rows, all_cols, row_offset, kind)
                               + _listed_mask(rows, all_cols, positives)) - 1.0
                    out["siglip_rows"] = np.sum(softplus(-z * logits), axis=1)
                else:
                    out["row_lse"] = logsumexp(logits, axis=1)
                    cmax = np.max(logits, axis=0)
                    out["col_max"] = cmax
                    out["col_sum"] = np.sum(np.exp(logits - cmax[None, :]), axis=0)
                return out

            parts = list(pool.map(forward_rows, row_blocks))
            for (r0, r1), part in zip(row_blocks, parts):
                pos_logit[p, r0:r1] = part["pos"]
            if kind in (SIGLIP, ONESET_SIGLIP, ONESET_EDGES):
                siglip_rows = np.concatenate([part["siglip_rows"] for part in parts])
                prefix_losses[p] = np.sum(siglip_rows) / N
            else:
                # merge the per-block column statistics in block order
                m_run = np.full(N, -np.inf)
                s_run = np.zeros(N)
                for part in parts:
                    m_new = np.maximum(m_run, part["col_max"])
                    s_run = s_run * np.exp(m_run - m_new) + part["col_sum"] * np.exp(part["col_max"] - m_new)
                    m_run = m_new
                col_lse[p] = m_run + np.log(s_run)
                row_lse[p] = np.concatenate([part["row_lse"] for part in parts])
                row_ce = row_lse[p] - pos_logit[p]
                if kind == INFONCE:
                    # column j's positive is row j (R == N, no offset): l_jj = pos_logit[j]
                    col_ce = col_lse[p] - pos_logit[p]
                    prefix_losses[p] = (np.sum(row_ce) + np.sum(col_ce)) / (2.0 * N)
                else:
                    prefix_losses[p] = np.sum(row_ce) / N

            if not grads:
                continue

            # ---- residuals g_ij = dL^p / dl_ij on a slice of the grid
            def residual(logits, rows, cols):
                if oneset:
                    E = _positive_mask(rows, cols, row_offset, kind) + _listed_mask(rows, cols, positives)
                    return (sigmoid(logits) - E) * (1.0 - _self_mask(rows, cols, row_offset)) / N
                E = _positive_mask(rows, cols, row_offset, kind)
                if kind == SIGLIP:
                    E = E + _listed_mask(rows, cols, positives)
                    return (sigmoid(logits) - E) / N
                p_row = np.exp(logits - row_lse[p][rows][:, None])
                if kind == INFONCE_ROWS:
                    return (p_row - E) / N
                p_col = np.exp(logits - col_lse[p][cols][None, :])
                return (p_row - E + p_col - E) / (2.0 * N)

            # ---- dq: u_i = sum_j g_ij * s * kh_j, then through the normalisation of q_i;
            # with it the block's sums of g * cos (dL^p/ds) and of g (dL^p/db)
            def grad_rows(rb):
                r0, r1 = rb
                cos = qh[r0:r1] @ kh.T
                logits = s * cos + b
                g = residual(logits, all_rows[r0:r1], all_cols)
                u = s * (g @ kh)
                radial = np.sum(u * qh[r0:r1], axis=1)
                return (u - radial[:, None] * qh[r0:r1]) / qnorm[r0:r1, None], np.sum(g * cos), np.sum(g)

            # one set: cell (j, i) has the residual and the derivative of cell (i, j)
            mirror = 2.0 if oneset else 1.0
            for (r0, r1), (part, gc, gs) in zip(row_blocks, pool.map(grad_rows, row_blocks)):
                dq[r0:r1, :width] += mirror * (w[p] / W) * part
                dscale += (w[p] / W) * gc
                dbias += (w[p] / W) * gs
            if oneset:
                continue

            # ---- dk: v_j = sum_i g_ij * s * qh_i, then through the normalisation of k_j
            def grad_cols(cb):
                c0, c1 = cb
                logits = s * (qh @ kh[c0:c1].T) + b
                g = residual(logits, all_rows, all_cols[c0:c1])
                v = s * (g.T @ qh)
                radial = np.sum(v * kh[c0:c1], axis=1)
                return (v - radial[:, None] * kh[c0:c1]) / knorm[c0:c1, None]

            for (c0, c1), part in zip(col_blocks, pool.map(grad_cols, col_blocks)):
                dk[c0:c1, :width] += (w[p] / W) * part

    result = {
        "loss": float(np.sum(w * prefix_losses) / W),
        "prefix_losses": prefix_losses,
    }
    if kind != ONESET_EDGES:  # every other kind has one implicit positive per row
        result["pos_logit"] = pos_logit
    if kind in (INFONCE, INFONCE_ROWS):
        result["row_lse"] = row_lse
        result["col_lse"] = col_lse
    if grads:
        result["dq"] = dq
        result["dk"] = dk
        result["dscale"] = float(dscale)
        result["dbias"] = float(dbias)
    return result


def _blas_single_thread():
    """Run BLAS single-threaded while the block pool supplies the parallelism."""
    try:
        from threadpoolctl import threadpool_limits
    except ImportError:  # BLAS keeps its own threads
        return contextlib.nullcontext()
    return threadpool_limits(limits=1, user_api="blas")
