"""Seeded synthetic embeddings for the contrastive loss, as BF16 bit patterns.

This module holds no loss arithmetic: it only draws random numbers and rounds
them to BF16.  Both the HIP path's tests/benchmarks and the FP64 oracle take
their inputs from here; nothing else is shared between them.

Every draw uses NumPy's PCG64 ``default_rng(seed)`` in FP64, in the order
stated per workload, then FP64 -> FP32 -> BF16 with round-to-nearest-even.
The pages name no dataset for the loss; these recipes stand in for batches of
1024-wide embeddings (UForm README, Matryoshka paragraph; "Scaling-Up
Contrastive Learning over NVLink Multicast", section "Bird's Eye View & the
Results": R rows of 1024-dimensional BF16 embeddings per GPU).
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

INFONCE = 0
SIGLIP = 1
INFONCE_ROWS = 2
ONESET_SIGLIP = 3
ONESET_SIGLIP_EDGES = 4

DEFAULT_PREFIXES = (64, 128, 256, 512, 1024)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to BF16 (round to nearest, ties to even); uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


@dataclass(frozen=True)
class Workload:
    name: str
    kind: int
    R: int
    N: int
    D: int = 1024
    prefixes: tuple = DEFAULT_PREFIXES
    weights: tuple | None = None
    scale: float = float(np.float32(1.0 / 0.07))
    bias: float = 0.0
    row_offset: int = 0
    recipe: str = "gauss"          # gauss | clustered | student_t | pairs
    noise: float = 0.3
    seed: int = 0
    extra: dict = field(default_factory=dict)


# The five workloads the loss is specified on (sizes, noise, scale, bias, weights).
WORKLOADS = {
    "tiny_infonce_256": Workload("tiny_infonce_256", INFONCE, 256, 256, noise=0.3, seed=0),
    "infonce_4096": Workload("infonce_4096", INFONCE, 4096, 4096, noise=0.5, seed=1),
    "siglip_16384": Workload("siglip_16384", SIGLIP, 16384, 16384, scale=10.0, bias=-10.0,
                             noise=0.5, seed=2),
    "rows_4096x65536": Workload("rows_4096x65536", INFONCE_ROWS, 4096, 65536, recipe="clustered",
                                noise=0.2, seed=3, extra={"centroids": 256}),
    "infonce_32768": Workload("infonce_32768", INFONCE, 32768, 32768, weights=(1, 1, 1, 1, 2),
                              scale=float(np.float32(1.0 / 0.05)), recipe="student_t",
                              noise=0.4, seed=4),
    # the one-set sigmoid form at one GPU's share of an eight-GPU set: 16384 rows of 131072
    "oneset_16384x131072": Workload("oneset_16384x131072", ONESET_SIGLIP, 16384, 131072, scale=10.0,
                                    bias=-10.0, recipe="pairs", noise=0.5, seed=5),
}


def draw_f64(R: int, N: int, D: int, recipe: str = "gauss", noise: float = 0.3, seed: int = 0,
             centroids: int = 256, row_offset: int = 0):
    """FP64 draws (before rounding) of q [R, D] and k [N, D].

    gauss:      q ~ N(0,1); k_j = q_{j-off} + noise * N(0,1) for the R paired
                keys, fresh N(0,1) rows for any extra keys (drawn after).
    student_t:  q ~ Student-t(3) i.i.d.; keys as for gauss.
    clustered:  centroids C ~ N(0,1) [centroids, D]; assignment a(j) ~ U{0..C-1}
                for every key j; k_j = C_{a(j)} + noise * N(0,1); then
                q_i = C_{a(off+i)} + noise * N(0,1) with independent noise.
    pairs:      one set (the one-set form): x_{2m} ~ N(0,1) for the N/2 pairs, then
                x_{2m+1} = x_{2m} + noise * N(0,1); k = x, q = x[off:off+R].
    """
    rng = np.random.default_rng(seed)
    if recipe in ("gauss", "student_t"):
        q = rng.standard_normal((R, D)) if recipe == "gauss" else rng.standard_t(3, size=(R, D))
        k_pairs = q + noise * rng.standard_normal((R, D))
        if N == R and row_offset == 0:
            k = k_pairs
        else:
            k = rng.standard_normal((N, D)) if recipe == "gauss" else rng.standard_t(3, size=(N, D))
            k[row_offset:row_offset + R] = k_pairs
        return q, k
    if recipe == "clustered":
        C = rng.standard_normal((centroids, D))
        assign = rng.integers(0, centroids, size=N)
        k = C[assign] + noise * rng.standard_normal((N, D))
        q = C[assign[row_offset:row_offset + R]] + noise * rng.standard_normal((R, D))
        return q, k
    if recipe == "pairs":
        if N % 2:
            raise ValueError("the pairs recipe needs an even N")
        x = np.empty((N, D))
        x[0::2] = rng.standard_normal((N // 2, D))
        x[1::2] = x[0::2] + noise * rng.standard_normal((N // 2, D))
        return x[row_offset:row_offset + R].copy(), x
    raise ValueError(f"unknown recipe {recipe!r}")


def make_inputs(R: int, N: int, D: int, recipe: str = "gauss", noise: float = 0.3, seed: int = 0,
                centroids: int = 256, row_offset: int = 0):
    """BF16 bit patterns (uint16) of q [R, D] and k [N, D]: FP64 -> FP32 -> BF16 (RNE)."""
    q, k = draw_f64(R, N, D, recipe, noise, seed, centroids, row_offset)
    return f32_to_bf16_bits(q.astype(np.float32)), f32_to_bf16_bits(k.astype(np.float32))


def workload_inputs(w: Workload):
    if w.recipe == "band":
        return make_band_inputs(w.R, w.D, w.extra["extra_pos"], w.extra["hard_neg"], w.noise,
                                w.extra["hard_noise"], w.seed)[:2]
    return make_inputs(w.R, w.N, w.D, w.recipe, w.noise, w.seed,
                       w.extra.get("centroids", 256), w.row_offset)


def band_lists(R: int, extra_pos: int, hard_neg: int):
    """Key layout of the band recipe: entry i carries m_i = i mod (2 extra_pos + 1) extra positives
    and hard_neg hard negatives, appended in entry order after the R own keys.  Returns the CSR
    lists (row_ptr int64 [R + 1], col int32) of the extra positive columns and the key count N."""
    m = np.arange(R, dtype=np.int64) % (2 * extra_pos + 1)
    first = R + np.concatenate([[0], np.cumsum(m + hard_neg)[:-1]])  # first appended key of each entry
    row_ptr = np.concatenate([[0], np.cumsum(m)]).astype(np.int64)
    col = (np.repeat(first - row_ptr[:-1], m) + np.arange(int(row_ptr[-1]))).astype(np.int32)
    return row_ptr, col, int(R + m.sum() + R * hard_neg)


def make_band_inputs(R: int, D: int, extra_pos: int = 2, hard_neg: int = 2, noise: float = 0.3,
                     hard_noise: float = 1.0, seed: int = 0):
    """Entries with several positives and explicit hard negatives, gathered as extra key rows.

    Each entry may carry several positives and explicit hard negatives that the
    loss gathers as extra columns (UForm README, "Multimodal Perception from 64
    to 1024 Dimensions", the training-stack paragraph on loader-side
    properties).  Layout
    as in ``band_lists``.  Draws, in order: q ~ N(0,1) [R, D]; own keys
    k_i = q_i + noise * N(0,1); then one N(0,1) matrix for all appended keys in
    key order, each appended key being its entry's q_i plus noise (extra
    positives) or hard_noise (hard negatives) times its row of that matrix.
    Returns the BF16 bits of q [R, D] and k [N, D] and the CSR lists.
    """
    row_ptr, col, N = band_lists(R, extra_pos, hard_neg)
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((R, D))
    own = q + noise * rng.standard_normal((R, D))
    m = np.diff(row_ptr)
    entry = np.repeat(np.arange(R), m + hard_neg)  # the entry of each appended key
    # within an entry: its m_i positives first, then its hard negatives
    rank = np.arange(N - R) - np.repeat(np.concatenate([[0], np.cumsum(m + hard_neg)[:-1]]), m + hard_neg)
    amp = np.where(rank < m[entry], noise, hard_noise)
    k = np.concatenate([own, q[entry] + amp[:, None] * rng.standard_normal((N - R, D))])
    to_bits = lambda x: f32_to_bf16_bits(x.astype(np.float32))  # noqa: E731
    return to_bits(q), to_bits(k), row_ptr, col


def random_positive_lists(R: int, N: int, row_offset: int, mean: float, seed: int, oneset: bool = False,
                          dense_row: int | None = None):
    """Seeded random extra-positive lists (CSR) over R local rows of N keys.

    Each cell (i, j) other than the row's own positive (row_offset + i; in the
    one-set form its partner (row_offset + i) xor 1 and the row itself) is
    listed with probability mean / N; row ``dense_row`` (if given) lists every
    allowed column.  The one-set form draws over the whole set and keeps
    (i, j) and (j, i) together (a dense row is listed by every other row as
    well), then returns the rows of the share.
    """
    rng = np.random.default_rng(seed)
    Rs, off = (N, 0) if oneset else (R, row_offset)
    pick = rng.random((Rs, N)) < mean / N
    if oneset:
        pick = np.triu(pick, 1)
        pick = pick | pick.T
    if dense_row is not None:
        d = row_offset + dense_row if oneset else dense_row
        pick[d] = True
        if oneset:
            pick[:, d] = True
    g = np.arange(Rs) + off
    own = g ^ 1 if oneset else g
    pick[np.arange(Rs), own] = False
    if oneset:
        pick[np.arange(Rs), g] = False
        pick = pick[row_offset:row_offset + R]
    counts = pick.sum(axis=1)
    row_ptr = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    return row_ptr, np.nonzero(pick)[1].astype(np.int32)


# Two-set sigmoid batches whose entries carry several positives (0..4, two on average) and two
# explicit hard negatives each, appended as extra key rows (16384 entries: N = 16384 * 5).
WORKLOADS["siglip_band_16384"] = Workload(
    "siglip_band_16384", SIGLIP, 16384, band_lists(16384, 2, 2)[2], scale=10.0, bias=-10.0, recipe="band",
    noise=0.5, seed=6, extra={"extra_pos": 2, "hard_neg": 2, "hard_noise": 1.0})


# The Large and XL tiers' width: 8192 x 8192 rows of 2048 with prefixes {64, ..., 1024, 2048}
# (UForm README, tier table and Matryoshka paragraph), the last prefix weighted 2.
WORKLOADS["infonce_8192_d2048"] = Workload(
    "infonce_8192_d2048", INFONCE, 8192, 8192, D=2048, prefixes=(64, 128, 256, 512, 1024, 2048),
    weights=(1, 1, 1, 1, 1, 2), noise=0.5, seed=7)


def workload_positives(w: Workload):
    """The extra-positive lists of a workload (band recipe), else None."""
    if w.recipe != "band":
        return None
    row_ptr, col, _ = band_lists(w.R, w.extra["extra_pos"], w.extra["hard_neg"])
    return row_ptr, col


def random_edge_lists(N: int, mean: float, seed: int, far: int = 0, lonely: int = 0):
    """Seeded symmetric relation lists (CSR over all N rows of one set) for the one-set form with
    listed relations ("UForm for Swift", section "Training": Edges(offsets, ids)).

    Each unordered pair {i, j}, i != j, is an edge with probability mean / N; ``far`` extra edges
    join rows far apart (i, i + N // 2); the first ``lonely`` rows have no edge at all.  Returns
    (row_ptr int64 [N + 1], col int32): row g's partners, ascending.
    """
    rng = np.random.default_rng(seed)
    pick = np.triu(rng.random((N, N)) < mean / N, 1)
    for i in range(far):
        pick[i, i + N // 2] = True
    pick = pick | pick.T
    pick[:lonely, :] = False
    pick[:, :lonely] = False
    counts = pick.sum(axis=1)
    return np.concatenate([[0], np.cumsum(counts)]).astype(np.int64), np.nonzero(pick)[1].astype(np.int32)


def share_lists(lists, off: int, R: int):
    """The CSR lists of rows off .. off + R - 1 of a whole set's lists."""
    rp, col = lists
    return (rp[off:off + R + 1] - rp[off]).astype(np.int64), col[rp[off]:rp[off + R]]
