"""Pins for the FP64 oracle, each independent of the oracle's own formulas.

* closed forms (identical rows, orthonormal one-hot pairs) derived by hand;
* library routines: torch's cross_entropy / logsigmoid / normalize and its
  autograd, in float64 on the CPU, for single and nested prefixes;
* central finite differences of the oracle's own loss;
* invariants: pair permutation, power-of-two row scaling, Q<->K swap, bias
  invariance of the softmax form, the Euler identity q . dq = 0, and the
  row-shard identity that rebuilds the symmetric loss from shards.

Sources: "Scaling-Up Contrastive Learning over NVLink Multicast", section
"One Set or Two" (CLIP row softmax; SigLIP equation; Matryoshka prefixes).
"""

import math

import numpy as np
import pytest

from oracle import INFONCE, INFONCE_ROWS, ONESET_SIGLIP, SIGLIP, contrastive_fwd_bwd

torch = pytest.importorskip("torch")
F = torch.nn.functional


def _softplus(x):
    return max(x, 0.0) + math.log1p(math.exp(-abs(x)))


def _sigmoid(x):
    return 1.0 / (1.0 + math.exp(-x))


# ----------------------------------------------------------------------------- closed forms

@pytest.mark.parametrize("N", [1, 5, 16])
def test_identical_rows_infonce_is_ln_n(rng, N):
    v = rng.standard_normal(128)
    q = np.tile(v, (N, 1))
    out = contrastive_fwd_bwd(q, q.copy(), [32, 64, 128], 1 / 0.07, 0.0, INFONCE, weights=[1, 2, 3])
    assert out["loss"] == pytest.approx(math.log(N), abs=1e-12)
    np.testing.assert_allclose(out["prefix_losses"], math.log(N), atol=1e-12)
    np.testing.assert_allclose(out["dq"], 0.0, atol=1e-12)
    np.testing.assert_allclose(out["dk"], 0.0, atol=1e-12)


def test_identical_rows_rows_kind(rng):
    R, N, s, b = 6, 20, 14.0, 0.5
    v = rng.standard_normal(64)
    out = contrastive_fwd_bwd(np.tile(v, (R, 1)), np.tile(v, (N, 1)), [32, 64], s, b, INFONCE_ROWS,
                              row_offset=9)
    assert out["loss"] == pytest.approx(R / N * math.log(N), abs=1e-12)
    np.testing.assert_allclose(out["col_lse"], s + b + math.log(R), atol=1e-12)
    np.testing.assert_allclose(out["dq"], 0.0, atol=1e-12)
    np.testing.assert_allclose(out["dk"], 0.0, atol=1e-12)


def test_identical_rows_siglip(rng):
    N, s, b = 9, 10.0, -10.0
    v = rng.standard_normal(64)
    out = contrastive_fwd_bwd(np.tile(v, (N, 1)), np.tile(v, (N, 1)), [32, 64], s, b, SIGLIP)
    expect = _softplus(-(s + b)) + (N - 1) * _softplus(s + b)
    assert out["loss"] == pytest.approx(expect, rel=1e-13)
    np.testing.assert_allclose(out["dq"], 0.0, atol=1e-12)


@pytest.mark.parametrize("s", [1.0, 14.285714149475098, 30.0])
def test_orthonormal_pairs_infonce(s):
    N, D = 16, 64
    q = np.eye(N, D)
    out = contrastive_fwd_bwd(q, q.copy(), [16, 32, 64], s, 0.25, INFONCE, weights=[2, 1, 1])
    # LSE - l_ii cancels ~s in FP64, so the bound is absolute at the logits' rounding level
    assert out["loss"] == pytest.approx(math.log1p((N - 1) * math.exp(-s)), rel=1e-12, abs=1e-13)
    g = s / (N * (math.exp(s) + N - 1))
    expect = np.zeros((N, D))
    expect[:, :N] = g
    expect[np.arange(N), np.arange(N)] = 0.0
    np.testing.assert_allclose(out["dq"], expect, rtol=1e-11, atol=1e-300)
    np.testing.assert_allclose(out["dk"], expect, rtol=1e-11, atol=1e-300)


def test_orthonormal_pairs_siglip():
    N, D, s, b = 12, 32, 10.0, -10.0
    q = np.eye(N, D)
    out = contrastive_fwd_bwd(q, q.copy(), [16, 32], s, b, SIGLIP)
    assert out["loss"] == pytest.approx(_softplus(-(s + b)) + (N - 1) * _softplus(b), rel=1e-13)
    expect = np.zeros((N, D))
    expect[:, :N] = s * _sigmoid(b) / N
    expect[np.arange(N), np.arange(N)] = 0.0
    np.testing.assert_allclose(out["dq"], expect, rtol=1e-11)
    np.testing.assert_allclose(out["dk"], expect, rtol=1e-11)


# ----------------------------------------------------------------------------- library routines

def _torch_loss(q, k, prefixes, s, b, kind, weights, off):
    """Weighted mean over prefixes of the textbook loss, built from torch library calls."""
    R, N = q.shape[0], k.shape[0]
    w = torch.ones(len(prefixes), dtype=torch.float64) if weights is None else torch.tensor(
        weights, dtype=torch.float64)
    target = torch.arange(R) + off
    total = 0.0
    for p, width in enumerate(prefixes):
        qh = F.normalize(q[:, :width], dim=1)
        kh = F.normalize(k[:, :width], dim=1)
        logits = s * qh @ kh.T + b
        if kind == INFONCE:
            lp = 0.5 * (F.cross_entropy(logits, target, reduction="sum")
                        + F.cross_entropy(logits.T, target, reduction="sum")) / N
        elif kind == INFONCE_ROWS:
            lp = F.cross_entropy(logits, target, reduction="sum") / N
        else:
            z = -torch.ones(R, N, dtype=torch.float64)
            z[torch.arange(R), target] = 1.0
            lp = -F.logsigmoid(z * logits).sum() / N
        total = total + w[p] * lp
    return total / w.sum()


CASES = [
    (INFONCE, 10, 10, 0, [48], None),
    (INFONCE, 10, 10, 0, [16, 32, 48], [1, 1, 2]),
    (INFONCE_ROWS, 5, 13, 4, [16, 48], [3, 1]),
    (SIGLIP, 7, 7, 0, [16, 32, 48], None),
    (SIGLIP, 4, 9, 5, [32, 48], [1, 2]),
]


@pytest.mark.parametrize("kind,R,N,off,prefixes,weights", CASES)
def test_matches_torch_library_loss_and_autograd(rng, kind, R, N, off, prefixes, weights):
    D = 48
    q = rng.standard_normal((R, D))
    k = rng.standard_normal((N, D))
    k[off:off + R] += 2.0 * q
    s, b = 7.5, -1.25
    out = contrastive_fwd_bwd(q, k, prefixes, s, b, kind, weights=weights, row_offset=off)
    qt = torch.tensor(q, requires_grad=True)
    kt = torch.tensor(k, requires_grad=True)
    st = torch.tensor(s, dtype=torch.float64, requires_grad=True)
    bt = torch.tensor(b, dtype=torch.float64, requires_grad=True)
    lt = _torch_loss(qt, kt, prefixes, st, bt, kind, weights, off)
    lt.backward()
    assert out["loss"] == pytest.approx(lt.item(), rel=1e-12)
    np.testing.assert_allclose(out["dq"], qt.grad.numpy(), rtol=1e-9, atol=1e-13)
    np.testing.assert_allclose(out["dk"], kt.grad.numpy(), rtol=1e-9, atol=1e-13)
    assert out["dscale"] == pytest.approx(st.grad.item(), rel=1e-9, abs=1e-14)
    assert out["dbias"] == pytest.approx(bt.grad.item(), rel=1e-9, abs=1e-14)
    for p, width in enumerate(prefixes):
        logits = s * F.normalize(qt[:, :width], dim=1) @ F.normalize(kt[:, :width], dim=1).T + b
        # the positive cell's logit of every kind, read off torch's grid at (i, off + i)
        np.testing.assert_allclose(out["pos_logit"][p], logits[torch.arange(R), torch.arange(R) + off].detach().numpy(),
                                   rtol=1e-12, atol=1e-14)
        if kind == INFONCE_ROWS:
            np.testing.assert_allclose(out["col_lse"][p], torch.logsumexp(logits, 0).detach().numpy(),
                                       rtol=1e-12)
            np.testing.assert_allclose(out["row_lse"][p], torch.logsumexp(logits, 1).detach().numpy(),
                                       rtol=1e-12)


# ----------------------------------------------------------------------------- finite differences

@pytest.mark.parametrize("kind,R,N,off", [(INFONCE, 6, 6, 0), (INFONCE_ROWS, 4, 7, 2), (SIGLIP, 5, 8, 3)])
def test_gradients_match_central_differences(rng, kind, R, N, off):
    D, prefixes, weights = 96, [32, 64, 96], [1, 2, 3]
    q = rng.standard_normal((R, D))
    k = rng.standard_normal((N, D))
    k[off:off + R] += q
    s, b = 6.0, -2.0
    out = contrastive_fwd_bwd(q, k, prefixes, s, b, kind, weights=weights, row_offset=off)

    def loss(qq, kk):
        return contrastive_fwd_bwd(qq, kk, prefixes, s, b, kind, weights=weights, row_offset=off,
                                   grads=False)["loss"]

    picks = [(0, i, d) for i in range(R) for d in rng.choice(D, 12, replace=False)]
    picks += [(1, j, d) for j in range(N) for d in rng.choice(D, 12, replace=False)]
    for which, i, d in picks:
        x = q if which == 0 else k
        h = 1e-6 * max(1.0, abs(x[i, d]))
        xp, xm = x.copy(), x.copy()
        xp[i, d] += h
        xm[i, d] -= h
        fd = (loss(xp, k) - loss(xm, k)) / (2 * h) if which == 0 else (loss(q, xp) - loss(q, xm)) / (2 * h)
        an = out["dq"][i, d] if which == 0 else out["dk"][i, d]
        assert an == pytest.approx(fd, rel=1e-6, abs=1e-9), (which, i, d)

    # the temperature and the bias
    def loss_sb(ss, bb):
        return contrastive_fwd_bwd(q, k, prefixes, ss, bb, kind, weights=weights, row_offset=off,
                                   grads=False)["loss"]

    h = 1e-5
    fd_s = (loss_sb(s + h, b) - loss_sb(s - h, b)) / (2 * h)
    fd_b = (loss_sb(s, b + h) - loss_sb(s, b - h)) / (2 * h)
    assert out["dscale"] == pytest.approx(fd_s, rel=1e-6, abs=1e-9)
    assert out["dbias"] == pytest.approx(fd_b, rel=1e-6, abs=1e-9)


# ----------------------------------------------------------------------------- invariants

def _rand_pairs(rng, R, N, D, off=0):
    q = rng.standard_normal((R, D))
    k = rng.standard_normal((N, D))
    k[off:off + R] = q + 0.5 * rng.standard_normal((R, D))
    return q, k


@pytest.mark.parametrize("kind", [INFONCE, SIGLIP])
def test_pair_permutation_equivariance(rng, kind):
    q, k = _rand_pairs(rng, 11, 11, 64)
    perm = rng.permutation(11)
    a = contrastive_fwd_bwd(q, k, [16, 64], 9.0, -3.0, kind)
    c = contrastive_fwd_bwd(q[perm], k[perm], [16, 64], 9.0, -3.0, kind)
    assert c["loss"] == pytest.approx(a["loss"], rel=1e-13)
    np.testing.assert_allclose(c["dq"], a["dq"][perm], rtol=1e-10, atol=1e-15)
    np.testing.assert_allclose(c["dk"], a["dk"][perm], rtol=1e-10, atol=1e-15)


def test_band_coordinate_permutation_equivariance(rng):
    q, k = _rand_pairs(rng, 9, 9, 64)
    perm = np.concatenate([rng.permutation(16), 16 + rng.permutation(48)])  # within bands [0,16), [16,64)
    a = contrastive_fwd_bwd(q, k, [16, 64], 9.0, 0.0, INFONCE)
    c = contrastive_fwd_bwd(q[:, perm], k[:, perm], [16, 64], 9.0, 0.0, INFONCE)
    assert c["loss"] == pytest.approx(a["loss"], rel=1e-13)
    np.testing.assert_allclose(c["dq"], a["dq"][:, perm], rtol=1e-10, atol=1e-15)


@pytest.mark.parametrize("kind", [INFONCE, INFONCE_ROWS, SIGLIP])
def test_power_of_two_row_scaling(rng, kind):
    R, N = (7, 7) if kind != INFONCE_ROWS else (4, 10)
    q, k = _rand_pairs(rng, R, N, 64)
    a = contrastive_fwd_bwd(q, k, [32, 64], 12.0, -1.0, kind)
    q2 = q.copy()
    q2[3] *= 4.0
    k2 = k.copy()
    k2[1] *= 0.5
    c = contrastive_fwd_bwd(q2, k2, [32, 64], 12.0, -1.0, kind)
    assert c["loss"] == pytest.approx(a["loss"], rel=1e-13)
    expect_dq = a["dq"].copy()
    expect_dq[3] /= 4.0
    expect_dk = a["dk"].copy()
    expect_dk[1] /= 0.5
    np.testing.assert_allclose(c["dq"], expect_dq, rtol=1e-10, atol=1e-15)
    np.testing.assert_allclose(c["dk"], expect_dk, rtol=1e-10, atol=1e-15)


def test_qk_swap_symmetry_infonce(rng):
    q, k = _rand_pairs(rng, 10, 10, 64)
    a = contrastive_fwd_bwd(q, k, [32, 64], 14.0, 0.0, INFONCE)
    c = contrastive_fwd_bwd(k, q, [32, 64], 14.0, 0.0, INFONCE)
    assert c["loss"] == pytest.approx(a["loss"], rel=1e-13)
    np.testing.assert_allclose(c["dq"], a["dk"], rtol=1e-10, atol=1e-15)
    np.testing.assert_allclose(c["dk"], a["dq"], rtol=1e-10, atol=1e-15)


def test_bias_invariance_infonce(rng):
    q, k = _rand_pairs(rng, 8, 8, 64)
    a = contrastive_fwd_bwd(q, k, [32, 64], 14.0, 0.0, INFONCE)
    c = contrastive_fwd_bwd(q, k, [32, 64], 14.0, 3.5, INFONCE)
    assert c["loss"] == pytest.approx(a["loss"], rel=1e-12)
    np.testing.assert_allclose(c["dq"], a["dq"], rtol=1e-9, atol=1e-15)
    # a softmax does not see a shift common to its logits: dL/db vanishes for both softmax kinds
    assert abs(c["dbias"]) <= 1e-15
    r = contrastive_fwd_bwd(q[:5], k, [32, 64], 14.0, 3.5, INFONCE_ROWS, row_offset=2)
    assert abs(r["dbias"]) <= 1e-15


@pytest.mark.parametrize("kind", [INFONCE, INFONCE_ROWS, SIGLIP])
def test_euler_identity(rng, kind):
    R, N = (8, 8) if kind != INFONCE_ROWS else (5, 12)
    q, k = _rand_pairs(rng, R, N, 64)
    out = contrastive_fwd_bwd(q, k, [16, 32, 64], 11.0, -2.0, kind, weights=[1, 3, 2])
    np.testing.assert_allclose(np.sum(q * out["dq"], axis=1), 0.0, atol=1e-13)
    np.testing.assert_allclose(np.sum(k * out["dk"], axis=1), 0.0, atol=1e-13)


def test_row_shards_rebuild_symmetric_loss(rng):
    """Row shards of INFONCE_ROWS (each with its row_offset) rebuild the symmetric loss."""
    N, D, shard = 12, 64, 4
    q, k = _rand_pairs(rng, N, N, D)
    prefixes, s = [16, 64], 14.0
    full = contrastive_fwd_bwd(q, k, prefixes, s, 0.0, INFONCE, grads=False)
    parts = [contrastive_fwd_bwd(q[o:o + shard], k, prefixes, s, 0.0, INFONCE_ROWS, row_offset=o, grads=False)
             for o in range(0, N, shard)]
    for p in range(len(prefixes)):
        col_lse = np.logaddexp.reduce(np.stack([part["col_lse"][p] for part in parts]), axis=0)
        np.testing.assert_allclose(col_lse, full["col_lse"][p], rtol=1e-13)
        pos = np.concatenate([part["pos_logit"][p] for part in parts])
        rows = sum(part["prefix_losses"][p] for part in parts)
        rebuilt = 0.5 * rows + np.sum(col_lse - pos) / (2 * N)
        assert rebuilt == pytest.approx(full["prefix_losses"][p], rel=1e-13)


def test_blocking_does_not_change_results(rng):
    q, k = _rand_pairs(rng, 13, 13, 64)
    a = contrastive_fwd_bwd(q, k, [32, 64], 14.0, 0.0, INFONCE, block=3, threads=3)
    c = contrastive_fwd_bwd(q, k, [32, 64], 14.0, 0.0, INFONCE, block=64, threads=1)
    assert c["loss"] == pytest.approx(a["loss"], rel=1e-14)
    np.testing.assert_allclose(c["dq"], a["dq"], rtol=1e-12, atol=1e-16)
    np.testing.assert_allclose(c["dk"], a["dk"], rtol=1e-12, atol=1e-16)


# ----------------------------------------------------------------------------- one-set sigmoid form

def _oneset(x, prefixes, s, b, R=None, off=0, weights=None, grads=True):
    R = x.shape[0] if R is None else R
    return contrastive_fwd_bwd(x[off:off + R], x, prefixes, s, b, ONESET_SIGLIP, weights=weights, row_offset=off,
                               grads=grads)


def test_oneset_identical_rows_closed_form():
    # every cosine is 1, so every scored cell has l = s + b: one positive and N - 2 negatives per row
    N, D, s, b = 10, 64, 6.0, -2.0
    x = np.tile(np.linspace(-1.0, 1.0, D), (N, 1))
    out = _oneset(x, [32, 64], s, b, grads=False)
    want = (N * _softplus(-(s + b)) + N * (N - 2) * _softplus(s + b)) / N
    assert out["loss"] == pytest.approx(want, rel=1e-12)


def test_oneset_matches_torch_autograd_of_the_whole_set():
    rng = np.random.default_rng(5)
    N, D, prefixes, weights, s, b = 10, 48, [16, 48], [1, 2], 7.0, -3.0
    x = rng.standard_normal((N, D))
    x[1::2] = x[0::2] + 0.6 * rng.standard_normal((N // 2, D))
    out = _oneset(x, prefixes, s, b, weights=weights)
    xt = torch.tensor(x, requires_grad=True)
    st = torch.tensor(s, dtype=torch.float64, requires_grad=True)
    bt = torch.tensor(b, dtype=torch.float64, requires_grad=True)
    z = -torch.ones(N, N, dtype=torch.float64)
    z[torch.arange(N), torch.arange(N) ^ 1] = 1.0
    keep = 1.0 - torch.eye(N, dtype=torch.float64)
    total = 0.0
    for p, width in enumerate(prefixes):
        xh = F.normalize(xt[:, :width], dim=1)
        logits = st * xh @ xh.T + bt
        total = total + weights[p] * (-(keep * F.logsigmoid(z * logits)).sum() / N)
    total = total / sum(weights)
    total.backward()
    assert out["loss"] == pytest.approx(total.item(), rel=1e-12)
    np.testing.assert_allclose(out["dq"], xt.grad.numpy(), rtol=1e-9, atol=1e-13)
    assert out["dscale"] == pytest.approx(st.grad.item(), rel=1e-9)
    assert out["dbias"] == pytest.approx(bt.grad.item(), rel=1e-9)
    assert out["dk"] is None
    # each row's positive logit is its cell with the pair partner g xor 1
    for p, width in enumerate(prefixes):
        xh = F.normalize(xt[:, :width], dim=1)
        logits = (s * xh @ xh.T + b).detach()
        np.testing.assert_allclose(out["pos_logit"][p], logits[torch.arange(N), torch.arange(N) ^ 1].numpy(),
                                   rtol=1e-12, atol=1e-14)


def test_oneset_central_differences_of_the_set():
    rng = np.random.default_rng(6)
    N, D, prefixes, s, b = 8, 64, [32, 64], 5.0, -1.5
    x = rng.standard_normal((N, D))
    out = _oneset(x, prefixes, s, b)
    for i in range(N):
        for d in rng.choice(D, 6, replace=False):
            h = 1e-6
            xp, xm = x.copy(), x.copy()
            xp[i, d] += h
            xm[i, d] -= h
            fd = (_oneset(xp, prefixes, s, b, grads=False)["loss"] - _oneset(xm, prefixes, s, b, grads=False)["loss"]) / (2 * h)
            assert out["dq"][i, d] == pytest.approx(fd, rel=1e-6, abs=1e-9)


def test_oneset_shards_rebuild_the_set():
    rng = np.random.default_rng(7)
    N, D, prefixes, s, b = 12, 64, [32, 64], 9.0, -4.0
    x = rng.standard_normal((N, D))
    full = _oneset(x, prefixes, s, b)
    parts = [_oneset(x, prefixes, s, b, R=4, off=o) for o in (0, 4, 8)]
    assert sum(p["loss"] for p in parts) == pytest.approx(full["loss"], rel=1e-12)
    np.testing.assert_allclose(np.concatenate([p["dq"] for p in parts]), full["dq"], rtol=1e-10, atol=1e-14)
    assert sum(p["dscale"] for p in parts) == pytest.approx(full["dscale"], rel=1e-10)


# ----------------------------------------------------------------------------- several positives per entry

def _csr(pairs, R):
    """CSR lists (row_ptr, col) of a set of (row, column) pairs."""
    rows = [sorted(c for r, c in pairs if r == i) for i in range(R)]
    row_ptr = np.cumsum([0] + [len(c) for c in rows])
    return row_ptr, np.array([c for cs in rows for c in cs], dtype=np.int64)


def test_extra_positives_identical_rows_closed_form():
    # every cosine is 1: row i has 1 + m_i cells at l = s + b labelled +1 and N - 1 - m_i labelled -1
    R, N, off, s, b = 4, 9, 2, 5.0, -3.0
    x = np.tile(np.linspace(-1.0, 2.0, 64), (N, 1))
    pairs = {(0, 0), (0, 5), (0, 8), (2, 1), (3, 0)}
    out = contrastive_fwd_bwd(x[:R], x, [32, 64], s, b, SIGLIP, row_offset=off, positives=_csr(pairs, R))
    m = [sum(1 for r, _ in pairs if r == i) for i in range(R)]
    want = sum((1 + mi) * _softplus(-(s + b)) + (N - 1 - mi) * _softplus(s + b) for mi in m) / N
    assert out["loss"] == pytest.approx(want, rel=1e-12)
    want_db = sum((1 + mi) * (_sigmoid(s + b) - 1.0) + (N - 1 - mi) * _sigmoid(s + b) for mi in m) / N
    assert out["dbias"] == pytest.approx(want_db, rel=1e-12)


@pytest.mark.parametrize("R,N,off", [(5, 5, 0), (4, 9, 3)])
def test_extra_positives_match_torch_autograd(rng, R, N, off):
    D, prefixes, weights, s, b = 96, [32, 96], [2, 1], 6.0, -2.5
    q = rng.standard_normal((R, D))
    k = rng.standard_normal((N, D))
    pairs = {(i, j) for i in range(R) for j in range(N) if j != off + i and rng.random() < 0.3}
    out = contrastive_fwd_bwd(q, k, prefixes, s, b, SIGLIP, weights=weights, row_offset=off,
                              positives=_csr(pairs, R))
    qt = torch.tensor(q, requires_grad=True)
    kt = torch.tensor(k, requires_grad=True)
    st = torch.tensor(s, dtype=torch.float64, requires_grad=True)
    bt = torch.tensor(b, dtype=torch.float64, requires_grad=True)
    z = -torch.ones(R, N, dtype=torch.float64)
    for i in range(R):
        z[i, off + i] = 1.0
    for i, j in pairs:
        z[i, j] = 1.0
    total = 0.0
    for p, width in enumerate(prefixes):
        logits = st * F.normalize(qt[:, :width], dim=1) @ F.normalize(kt[:, :width], dim=1).T + bt
        total = total + weights[p] * (-F.logsigmoid(z * logits).sum() / N)
    total = total / sum(weights)
    total.backward()
    assert out["loss"] == pytest.approx(total.item(), rel=1e-12)
    np.testing.assert_allclose(out["dq"], qt.grad.numpy(), rtol=1e-9, atol=1e-13)
    np.testing.assert_allclose(out["dk"], kt.grad.numpy(), rtol=1e-9, atol=1e-13)
    assert out["dscale"] == pytest.approx(st.grad.item(), rel=1e-9)
    assert out["dbias"] == pytest.approx(bt.grad.item(), rel=1e-9)


def test_oneset_extra_positives_match_torch_autograd_of_the_whole_set():
    rng = np.random.default_rng(11)
    N, D, prefixes, s, b = 10, 64, [32, 64], 7.0, -3.0
    x = rng.standard_normal((N, D))
    pairs = set()
    for i in range(N):
        for j in range(i + 1, N):
            if j != i ^ 1 and rng.random() < 0.3:
                pairs |= {(i, j), (j, i)}
    out = contrastive_fwd_bwd(x, x, prefixes, s, b, ONESET_SIGLIP, positives=_csr(pairs, N))
    xt = torch.tensor(x, requires_grad=True)
    z = -torch.ones(N, N, dtype=torch.float64)
    z[torch.arange(N), torch.arange(N) ^ 1] = 1.0
    for i, j in pairs:
        z[i, j] = 1.0
    keep = 1.0 - torch.eye(N, dtype=torch.float64)
    total = 0.0
    for width in prefixes:
        xh = F.normalize(xt[:, :width], dim=1)
        total = total + (-(keep * F.logsigmoid(z * (s * xh @ xh.T + b))).sum() / N)
    total = total / len(prefixes)
    total.backward()
    assert out["loss"] == pytest.approx(total.item(), rel=1e-12)
    np.testing.assert_allclose(out["dq"], xt.grad.numpy(), rtol=1e-9, atol=1e-13)
    # a share of the set carries the rows' own lists; the shares rebuild the set
    rp, col = _csr(pairs, N)
    parts = []
    for o in (0, 4, 8):
        R = min(4, N - o)
        prp = rp[o:o + R + 1] - rp[o]
        parts.append(contrastive_fwd_bwd(x[o:o + R], x, prefixes, s, b, ONESET_SIGLIP, row_offset=o,
                                         positives=(prp, col[rp[o]:rp[o + R]])))
    assert sum(p["loss"] for p in parts) == pytest.approx(out["loss"], rel=1e-12)
    np.testing.assert_allclose(np.concatenate([p["dq"] for p in parts]), out["dq"], rtol=1e-10, atol=1e-14)


@pytest.mark.parametrize("kind,row_ptr,col,off", [
    (SIGLIP, [0, 1, 1], [1], 1),          # row 0's own positive (column 1)
    (SIGLIP, [0, 2, 2], [3, 3], 0),       # repeated column
    (SIGLIP, [0, 2, 2], [4, 2], 0),       # not increasing
    (SIGLIP, [0, 1, 1], [6], 0),          # past N
    (SIGLIP, [0, 1, 1], [-1], 0),         # negative
    (SIGLIP, [0, 1], [2], 0),             # row_ptr too short
    (SIGLIP, [0, 2, 1], [2, 3], 0),       # row_ptr decreasing
    (ONESET_SIGLIP, [0, 1, 1], [1], 0),   # row 0's pair partner
    (ONESET_SIGLIP, [0, 1, 1], [0], 0),   # the row itself
    (INFONCE_ROWS, [0, 1, 1], [3], 0),    # softmax kinds take no list
])
def test_extra_positive_lists_are_checked(rng, kind, row_ptr, col, off):
    x = rng.standard_normal((6, 32))
    q = x[off:off + 2]
    with pytest.raises(ValueError):
        contrastive_fwd_bwd(q, x, [32], 4.0, -1.0, kind, row_offset=off, grads=False,
                            positives=(np.array(row_ptr), np.array(col)))


# ----------------------------------------------------------------------------- one set, listed relations only

def _edges_csr(N, edges, rows):
    """CSR lists of the given rows from undirected edges (both directions listed)."""
    nb = {g: set() for g in range(N)}
    for a, b in edges:
        nb[a].add(b)
        nb[b].add(a)
    cols = [sorted(nb[g]) for g in rows]
    rp = np.concatenate([[0], np.cumsum([len(c) for c in cols])]).astype(np.int64)
    return rp, np.array([j for c in cols for j in c], dtype=np.int64)


EDGES_9 = [(0, 5), (1, 2), (1, 7), (3, 4), (6, 8), (2, 7)]  # odd N; row 0's partner far away; several per row


def test_oneset_edges_match_torch_autograd_of_the_whole_set():
    from oracle import ONESET_EDGES
    rng = np.random.default_rng(7)
    N, D, prefixes, weights, s, b = 9, 48, [16, 48], [2, 1], 6.0, -2.5
    x = rng.standard_normal((N, D))
    for a, c in EDGES_9:
        x[c] = x[a] + 0.5 * rng.standard_normal(D)
    pos = _edges_csr(N, EDGES_9, range(N))
    out = contrastive_fwd_bwd(x, x, prefixes, s, b, ONESET_EDGES, weights=weights, positives=pos)
    xt = torch.tensor(x, requires_grad=True)
    st = torch.tensor(s, dtype=torch.float64, requires_grad=True)
    bt = torch.tensor(b, dtype=torch.float64, requires_grad=True)
    z = -torch.ones(N, N, dtype=torch.float64)
    for a, c in EDGES_9:
        z[a, c] = z[c, a] = 1.0
    keep = 1.0 - torch.eye(N, dtype=torch.float64)
    total = 0.0
    for p, width in enumerate(prefixes):
        xh = F.normalize(xt[:, :width], dim=1)
        total = total + weights[p] * (-(keep * F.logsigmoid(z * (st * xh @ xh.T + bt))).sum() / N)
    total = total / sum(weights)
    total.backward()
    assert out["loss"] == pytest.approx(total.item(), rel=1e-12)
    np.testing.assert_allclose(out["dq"], xt.grad.numpy(), rtol=1e-9, atol=1e-13)
    assert out["dscale"] == pytest.approx(st.grad.item(), rel=1e-9)
    assert out["dbias"] == pytest.approx(bt.grad.item(), rel=1e-9)
    assert out["dk"] is None and "pos_logit" not in out


def test_oneset_edges_of_the_pairs_equal_the_pairs_form():
    # listing exactly the pairs (2m, 2m + 1) as relations gives the pairs form, rows and shares alike
    from oracle import ONESET_EDGES
    rng = np.random.default_rng(8)
    N, D, R, off = 12, 64, 5, 3
    x = rng.standard_normal((N, D))
    x[1::2] = x[0::2] + 0.4 * rng.standard_normal((N // 2, D))
    pos = _edges_csr(N, [(2 * m, 2 * m + 1) for m in range(N // 2)], range(off, off + R))
    a = contrastive_fwd_bwd(x[off:off + R], x, [32, 64], 7.0, -3.0, ONESET_SIGLIP, row_offset=off)
    e = contrastive_fwd_bwd(x[off:off + R], x, [32, 64], 7.0, -3.0, ONESET_EDGES, row_offset=off, positives=pos)
    assert e["loss"] == pytest.approx(a["loss"], rel=1e-13)
    np.testing.assert_allclose(e["dq"], a["dq"], rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(e["prefix_losses"], a["prefix_losses"], rtol=1e-13)
    assert e["dscale"] == pytest.approx(a["dscale"], rel=1e-12)
    assert e["dbias"] == pytest.approx(a["dbias"], rel=1e-12)


def test_oneset_edges_identical_rows_closed_form():
    # every cosine is 1: row g has m_g positives and N - 1 - m_g negatives, each with l = s + b
    from oracle import ONESET_EDGES
    N, D, s, b = 9, 64, 5.0, -1.0
    x = np.tile(np.linspace(-1.0, 2.0, D), (N, 1))
    pos = _edges_csr(N, EDGES_9, range(N))
    m = np.diff(pos[0])
    out = contrastive_fwd_bwd(x, x, [32, 64], s, b, ONESET_EDGES, positives=pos)
    want = float(np.sum(m * _softplus(-(s + b)) + (N - 1 - m) * _softplus(s + b))) / N
    assert out["loss"] == pytest.approx(want, rel=1e-12)
    np.testing.assert_allclose(out["dq"], 0.0, atol=1e-12)
    # no relations at all: every cell is a negative
    none = (np.zeros(N + 1, dtype=np.int64), np.zeros(0, dtype=np.int64))
    out0 = contrastive_fwd_bwd(x, x, [32, 64], s, b, ONESET_EDGES, positives=none)
    assert out0["loss"] == pytest.approx((N - 1) * _softplus(s + b), rel=1e-12)


def test_oneset_edges_shares_rebuild_the_set():
    from oracle import ONESET_EDGES
    rng = np.random.default_rng(9)
    N, D = 9, 64
    x = rng.standard_normal((N, D))
    whole = contrastive_fwd_bwd(x, x, [32, 64], 6.0, -2.0, ONESET_EDGES, positives=_edges_csr(N, EDGES_9, range(N)))
    loss, dq = 0.0, np.zeros((N, D))
    for off, R in ((0, 4), (4, 1), (5, 4)):
        part = contrastive_fwd_bwd(x[off:off + R], x, [32, 64], 6.0, -2.0, ONESET_EDGES, row_offset=off,
                                   positives=_edges_csr(N, EDGES_9, range(off, off + R)))
        loss += part["loss"]
        dq[off:off + R] = part["dq"]
    assert loss == pytest.approx(whole["loss"], rel=1e-13)
    np.testing.assert_allclose(dq, whole["dq"], rtol=1e-12, atol=1e-15)


def test_oneset_relations_must_be_symmetric_within_the_share():
    from oracle import ONESET_EDGES
    x = np.random.default_rng(10).standard_normal((6, 32))
    one_way = (np.array([0, 1, 1, 1, 1, 1, 1]), np.array([3]))  # row 0 lists 3, row 3 does not list 0
    with pytest.raises(ValueError):
        contrastive_fwd_bwd(x, x, [32], 5.0, -1.0, ONESET_EDGES, positives=one_way)
    self_edge = (np.array([0, 0, 1, 1, 1, 1, 1]), np.array([1]))  # row 1 lists itself
    with pytest.raises(ValueError):
        contrastive_fwd_bwd(x, x, [32], 5.0, -1.0, ONESET_EDGES, positives=self_edge)
    # a partner outside the share cannot be checked from the share's lists, and is accepted
    part = (np.array([0, 1]), np.array([5]))
    contrastive_fwd_bwd(x[2:3], x, [32], 5.0, -1.0, ONESET_EDGES, row_offset=2, positives=part)
