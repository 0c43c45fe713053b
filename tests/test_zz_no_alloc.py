"""The allocation-free entry point against the workspace entry point it mirrors.

``uform_contrastive_fwd_bwd_noalloc`` runs the same kernels on the library's
fixed per-GPU scratch.  Two calls in a row (the second smaller, so the scratch
holds the first call's contents when it starts) must each match
``uform_contrastive_fwd_bwd_ex`` on the same inputs: the loss within 1e-3
relative, dq and dk within 2e-3 x max|grad|, and, since the kernels and the
launch configuration are the same, bitwise.  A call whose workspace would not
fit the scratch is refused on the host.
"""

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from contrastive_embedding_loss_amd import binding  # noqa: E402
from contrastive_embedding_loss_amd.inputs import (  # noqa: E402
    INFONCE, INFONCE_ROWS, ONESET_SIGLIP, SIGLIP, bf16_bits_to_f32, make_inputs)

pytestmark = pytest.mark.gpu
LADDER = (64, 128, 256, 512, 1024)


def _dev(bits):
    return torch.from_numpy(bf16_bits_to_f32(bits)).to("cuda").to(torch.bfloat16)


@pytest.mark.parametrize("kind,s,b", [(INFONCE, 14.0, 0.0), (SIGLIP, 10.0, -10.0)])
def test_noalloc_matches_workspace_entry_point_on_two_calls(kind, s, b):
    for R in (1024, 300):  # the second call is smaller
        print(f"[case] noalloc kind={kind} R=N={R}", flush=True)
        qb, kb = make_inputs(R, R, 1024, noise=0.5, seed=241 + R)
        q, k = _dev(qb), _dev(kb)
        ref = binding.fwd_bwd(q, k, LADDER, s, b, kind, weights=(1, 1, 1, 1, 2), extras=True)
        got = binding.fwd_bwd(q, k, LADDER, s, b, kind, weights=(1, 1, 1, 1, 2), extras=True, noalloc=True)
        torch.cuda.synchronize()
        assert abs(got[0].item() - ref[0].item()) <= 1e-3 * abs(ref[0].item())
        for a, c in ((got[1], ref[1]), (got[2], ref[2])):
            assert (a - c).abs().max().item() <= 2e-3 * c.abs().max().item()
            assert torch.equal(a, c)
        for name in ref[3]:
            assert torch.equal(got[3][name], ref[3][name]), name


@pytest.mark.parametrize("kind", [INFONCE_ROWS, ONESET_SIGLIP])
def test_noalloc_shares_on_two_calls(kind):
    # a share of rows at an offset: inner splits, their partials and k_finalize in the scratch
    # (the row kind), and the one-set form's single pass over its share
    for R, N, off in ((256, 1024, 64), (100, 300, 33)):
        print(f"[case] noalloc share kind={kind} R={R} N={N} off={off}", flush=True)
        oneset = kind == ONESET_SIGLIP
        qb, kb = make_inputs(R, N, 1024, recipe="pairs" if oneset else "gauss", noise=0.5, seed=261 + R,
                             row_offset=off)
        k = _dev(kb)
        q = k[off:off + R] if oneset else _dev(qb)
        s, b = (10.0, -6.0) if oneset else (14.0, 0.0)
        ref = binding.fwd_bwd(q, k, LADDER, s, b, kind, row_offset=off, extras=True)
        got = binding.fwd_bwd(q, k, LADDER, s, b, kind, row_offset=off, extras=True, noalloc=True)
        torch.cuda.synchronize()
        assert abs(got[0].item() - ref[0].item()) <= 1e-3 * abs(ref[0].item())
        for a, c in ((got[1], ref[1]), (got[2], ref[2])):
            if c is None:
                assert a is None
                continue
            assert (a - c).abs().max().item() <= 2e-3 * c.abs().max().item()
            assert torch.equal(a, c)
        for name in ref[3]:
            assert torch.equal(got[3][name], ref[3][name]), name


@pytest.mark.parametrize("kind,s,b", [(INFONCE, 14.0, 0.0), (SIGLIP, 10.0, -10.0)])
def test_noalloc_wide_rows_on_two_calls(kind, s, b):
    # D = 2048 with the wide tiers' ladder: the generic backward's split partials and k_finalize in
    # the scratch
    xl, w = (64, 128, 256, 512, 1024, 2048), (1, 1, 1, 1, 1, 2)
    for R in (384, 200):
        print(f"[case] noalloc wide kind={kind} R=N={R}", flush=True)
        qb, kb = make_inputs(R, R, 2048, noise=0.5, seed=281 + R)
        q, k = _dev(qb), _dev(kb)
        ref = binding.fwd_bwd(q, k, xl, s, b, kind, weights=w, extras=True)
        got = binding.fwd_bwd(q, k, xl, s, b, kind, weights=w, extras=True, noalloc=True)
        torch.cuda.synchronize()
        assert abs(got[0].item() - ref[0].item()) <= 1e-3 * abs(ref[0].item())
        for a, c in ((got[1], ref[1]), (got[2], ref[2])):
            assert (a - c).abs().max().item() <= 2e-3 * c.abs().max().item()
            assert torch.equal(a, c)
        for name in ref[3]:
            assert torch.equal(got[3][name], ref[3][name]), name


def test_noalloc_refuses_what_it_cannot_hold():
    qb, kb = make_inputs(64, 64, 1024, seed=251)
    q, k = _dev(qb), _dev(kb)
    # no caller workspace, no lists, no profiling
    with pytest.raises(binding.UformError):
        binding.fwd_bwd(q, k, LADDER, 14.0, 0.0, INFONCE, noalloc=True,
                        workspace=torch.empty(1 << 20, dtype=torch.uint8, device="cuda"))
    with pytest.raises(binding.UformError):
        binding.fwd_bwd(q, k, LADDER, 10.0, -10.0, SIGLIP, noalloc=True,
                        positives=(np.zeros(65, dtype=np.int64), np.zeros(0, dtype=np.int32)))
    # 16384 x 16384 InfoNCE needs more than the 128 MiB of scratch: refused before any launch
    big = torch.zeros(16384, 1024, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(binding.UformError) as e:
        binding.fwd_bwd(big, big, LADDER, 14.0, 0.0, INFONCE, noalloc=True)
    assert e.value.status == 2 and "scratch" in e.value.message
    torch.cuda.synchronize()
