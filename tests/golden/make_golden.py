"""Write sampled expected values of the large workloads from the FP64 oracle.

Run from the repository root:  python tests/golden/make_golden.py [workload ...]

For each workload the oracle runs once on the full seeded BF16 inputs (the
same arrays the GPU receives) and this script stores, in
``tests/golden/<workload>.npz``:

* ``loss`` and ``prefix_losses`` (float64);
* ``dq_rows`` / ``dk_rows``: 16 seeded row indices (first and last row
  included) with those rows of dq / dk (float32), and ``dq_absmax`` /
  ``dk_absmax``: max |dq|, max |dk| over the whole tensors (the scale of the
  gradient tolerance); the one-set form has no dk;
* ``dscale`` and ``dbias``: dL/dscale and dL/dbias (float64);
* ``tab_idx``: 256 seeded row/column indices with ``pos_logit`` (and for the
  softmax kinds ``row_lse`` / ``col_lse``) at those indices, all prefixes.

Only ``oracle/`` and the seeded input generator are used; no value comes from
the GPU path.
"""

from __future__ import annotations

import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

from contrastive_embedding_loss_amd.inputs import (  # noqa: E402
    ONESET_SIGLIP, SIGLIP, WORKLOADS, workload_inputs, workload_positives)
from oracle import bf16_bits_to_f64, contrastive_fwd_bwd  # noqa: E402

LARGE = ("siglip_16384", "rows_4096x65536", "infonce_32768", "oneset_16384x131072", "siglip_band_16384")


def sample_indices(n: int, count: int, seed: int) -> np.ndarray:
    rng = np.random.default_rng(seed)
    idx = set([0, n - 1])
    while len(idx) < min(count, n):
        idx.add(int(rng.integers(0, n)))
    return np.array(sorted(idx), dtype=np.int64)


def make(name: str) -> str:
    w = WORKLOADS[name]
    qb, kb = workload_inputs(w)
    t0 = time.time()
    ref = contrastive_fwd_bwd(bf16_bits_to_f64(qb), bf16_bits_to_f64(kb), w.prefixes, w.scale, w.bias, w.kind,
                              weights=w.weights, row_offset=w.row_offset, positives=workload_positives(w))
    out = {
        "loss": np.float64(ref["loss"]),
        "prefix_losses": np.asarray(ref["prefix_losses"], dtype=np.float64),
        "dq_absmax": np.float64(np.abs(ref["dq"]).max()),
        "dscale": np.float64(ref["dscale"]),
        "dbias": np.float64(ref["dbias"]),
    }
    out["dq_rows"] = sample_indices(w.R, 16, 1000 + w.seed)
    out["dq"] = ref["dq"][out["dq_rows"]].astype(np.float32)
    if w.kind != ONESET_SIGLIP:
        out["dk_absmax"] = np.float64(np.abs(ref["dk"]).max())
        out["dk_rows"] = sample_indices(w.N, 16, 2000 + w.seed)
        out["dk"] = ref["dk"][out["dk_rows"]].astype(np.float32)
    out["tab_idx"] = sample_indices(w.R, 256, 3000 + w.seed)
    out["pos_logit"] = ref["pos_logit"][:, out["tab_idx"]].astype(np.float64)
    if w.kind not in (SIGLIP, ONESET_SIGLIP):
        out["row_lse"] = ref["row_lse"][:, out["tab_idx"]].astype(np.float64)
        out["col_idx"] = sample_indices(w.N, 256, 4000 + w.seed)
        out["col_lse"] = ref["col_lse"][:, out["col_idx"]].astype(np.float64)
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), f"{name}.npz")
    np.savez_compressed(path, **out)
    print(f"{name}: loss {ref['loss']:.10f} in {time.time() - t0:.1f} s -> {path}", flush=True)
    return path


if __name__ == "__main__":
    for n in (sys.argv[1:] or LARGE):
        make(n)
