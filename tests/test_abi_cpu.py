"""The C ABI without a GPU: the library loads, exports every declared symbol,
and rejects every invalid argument on the host before touching the device."""

import ctypes
import os
import re

import numpy as np
import pytest

from contrastive_embedding_loss_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "uform_contrastive.h")
PREFIXES = [64, 128, 256, 512, 1024]

pytestmark = pytest.mark.skipif(not os.path.exists(binding.LIB_PATH), reason="library not built")


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*(uform_[a-z_0-9]+)\s*\(", text, re.M)))


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert len(names) == 10, names
    lib = binding.library()
    for n in names:
        assert hasattr(lib, n), n


PAGE_TITLES = ("Scaling-Up Contrastive Learning over NVLink Multicast", "UForm for Swift", "UForm README")


def _comment_before(text, pos):
    """The block comment that ends closest before ``pos`` (the declaration's own comment)."""
    end = text.rfind("*/", 0, pos)
    start = text.rfind("/*", 0, end)
    return _flat(text[start:end])


def _flat(c):
    """Comment text on one line: the leading '*' of continuation lines dropped."""
    return re.sub(r"\s+", " ", re.sub(r"\n\s*\*(?!/)", " ", c))


def test_every_declaration_cites_the_pages():
    # each exported function and the options that carry a separate idea (offset, caller
    # memory, extra positives) name the page and section that define them
    text = open(HEADER).read()
    missing = []
    for name in declared_functions():
        pos = re.search(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*" + name + r"\s*\(", text, re.M).start()
        comment = _comment_before(text, pos)
        if name == "uform_contrastive_fwd_bwd":  # described by the file's opening comment
            comment = _flat(text[:text.index("#ifndef")])
        if name == "uform_contrastive_fwd_bwd_ex":  # its options carry their own citations
            continue
        if name == "uform_contrastive_fwd_bwd_noalloc":  # names the callers it is for instead
            if "cannot allocate" not in comment:
                missing.append(name)
            continue
        if not any(t in comment for t in PAGE_TITLES):
            missing.append(name)
    for field in ("row_offset;", "void *workspace;", "const int64_t *pos_row_ptr;", "float *dscale_out;"):
        if not any(t in _comment_before(text, text.index(field)) for t in PAGE_TITLES):
            missing.append(field)
    assert not missing, missing


def test_status_names():
    assert [binding.status_name(s) for s in range(5)] == [
        "success", "invalid-argument", "unsupported", "out-of-memory", "device-error"]
    assert binding.status_name(17) == "unknown"


def _call(q=0x10000, k=0x20000, R=256, N=256, D=1024, prefixes=PREFIXES, scale=14.0, bias=0.0, kind=0,
          loss=0x30000, dq=0x40000, dk=0x50000, opt=None, n_prefixes=None):
    """Call the ABI with fake device addresses: argument checks must fail before any device call."""
    lib = binding.library()
    P = (len(prefixes) if prefixes is not None else 5) if n_prefixes is None else n_prefixes
    pw = (ctypes.c_int32 * max(1, len(prefixes)))(*prefixes) if prefixes is not None else None
    args = [ctypes.c_void_p(q), ctypes.c_void_p(k), R, N, D, pw, P, scale, bias, kind, ctypes.c_void_p(loss),
            ctypes.c_void_p(dq), ctypes.c_void_p(dk), None]
    if opt is None:
        return lib.uform_contrastive_fwd_bwd(*args)
    return lib.uform_contrastive_fwd_bwd_ex(*args, ctypes.byref(opt))


INVALID = [
    dict(q=0), dict(k=0), dict(loss=0), dict(q=0x10008), dict(dq=0x40004), dict(loss=0x30002),
    dict(R=0), dict(N=0), dict(D=0), dict(R=300, N=256, kind=2), dict(kind=3), dict(kind=-1), dict(kind=5),
    dict(R=128, N=256, kind=0), dict(prefixes=None), dict(prefixes=[64, 64, 1024]),
    dict(prefixes=[64, 48, 1024]), dict(prefixes=[100, 1024]), dict(prefixes=[64, 2048]),
    dict(prefixes=PREFIXES, n_prefixes=0), dict(prefixes=[32 * (i + 1) for i in range(9)]),
    dict(scale=float("inf")), dict(scale=float("nan")), dict(bias=float("nan")), dict(scale=0.0),
    # one-set form: q must be k's rows, the set even, and no dk
    dict(kind=3, dk=0), dict(kind=3, q=0x20000, dk=0, N=255, R=255, D=1024),
    dict(kind=3, q=0x20000 + 2048 * 3, dk=0, R=64, N=256),
]


@pytest.mark.parametrize("kw", INVALID)
def test_invalid_arguments_are_rejected_on_the_host(kw):
    assert _call(**kw) == 1, binding.last_error()
    assert binding.last_error() != ""


UNSUPPORTED = [
    dict(D=1000, prefixes=[64, 992]), dict(D=4096, prefixes=[64, 4096]), dict(D=2112, prefixes=[64, 2112]),
    dict(scale=50.0),
    # the generic backward's LDS at widths above 1024: at most 6 prefixes, 3 of them inside a quarter
    dict(D=2048, prefixes=[64, 128, 256, 384, 1024, 2048]),
    dict(D=2048, prefixes=[64, 128, 256, 512, 1024, 1536, 2048]),
]


@pytest.mark.parametrize("kw", UNSUPPORTED)
def test_unsupported_requests_are_reported(kw):
    assert _call(**kw) == 2, binding.last_error()


def test_softmax_scale_limit_names_the_scale():
    assert _call(scale=100.0, kind=0) == 2
    assert "scale" in binding.last_error()


def test_option_checks():
    opt = binding.Options()
    opt.row_offset = 10
    assert _call(R=250, N=256, kind=2, opt=opt) == 1  # off + R > N
    opt.row_offset = -1
    assert _call(R=100, N=256, kind=2, opt=opt) == 1
    opt.row_offset = 0
    w = (ctypes.c_float * 5)(1, 1, 0, 1, 1)
    opt.prefix_weights = ctypes.cast(w, ctypes.POINTER(ctypes.c_float))
    assert _call(opt=opt) == 1
    opt.prefix_weights = None
    opt.workspace = 0x1000010
    assert _call(opt=opt) == 1
    opt.workspace = None
    # dL/dscale and dL/dbias come from a gradient pass and need an aligned float
    opt.dscale_out = 0x60000
    assert _call(dq=0, dk=0, opt=opt) == 1
    assert "dq or dk" in binding.last_error()
    opt.dscale_out = 0x60002
    assert _call(opt=opt) == 1
    opt.dscale_out = None
    opt.dbias_out = 0x60000
    assert _call(dq=0, dk=0, kind=1, opt=opt) == 1


def test_workspace_bytes():
    small = binding.workspace_bytes(256, 256, 1024, 5, 0)
    big = binding.workspace_bytes(32768, 32768, 1024, 5, 0)
    assert 0 < small < big
    assert binding.workspace_bytes(300, 256, 1024, 5, 0) == 0
    assert binding.workspace_bytes(256, 256, 1000, 5, 0) == 0
    assert binding.workspace_bytes(256, 256, 1024, 9, 0) == 0


COMPILED = [(1024, (64, 128, 256, 512, 1024)), (512, (64, 128, 256, 512)), (256, (64, 128, 256)),
            (128, (64, 128)), (1024, (1024,)), (512, (512,)), (256, (256,)), (128, (128,)),
            (1024, (64, 128, 256, 512)), (768, (64, 128))]


@pytest.mark.parametrize("D,prefixes", COMPILED)
@pytest.mark.parametrize("kind", [0, 1, 2])
def test_compiled_ladders_are_supported(D, prefixes, kind):
    assert binding.supported(D, prefixes, kind) == 0, binding.last_error()


@pytest.mark.parametrize("D,prefixes", [
    (1024, (96, 1024)), (1024, (64, 256, 1024)), (1024, (32, 64)), (1024, (64, 128, 256, 512, 768)),
    (256, tuple(range(32, 257, 32))), (2048, (64, 128, 256, 512, 1024, 2048)), (2048, (2048,)),
    (1536, (64, 128, 256, 512, 1024, 1536)), (2048, (512, 1024, 1536, 2048))])
@pytest.mark.parametrize("kind", [0, 1, 2, 3, 4])
def test_every_other_ladder_takes_the_generic_backward(D, prefixes, kind):
    # ladders without a compiled backward, and the wide tiers' ladders, have gradients too
    assert binding.supported(D, prefixes, kind) == 0, binding.last_error()
    assert binding.supported(D, prefixes, kind, with_gradients=False) == 0


@pytest.mark.parametrize("kind,R,N,off,row_ptr,col", [
    (1, 2, 8, 0, [1, 1, 1], []),            # row_ptr[0] != 0
    (1, 2, 8, 0, [0, 2, 1], [3, 4]),        # decreasing row_ptr
    (1, 2, 8, 0, [0, 1, 1], [0]),           # row 0's own positive
    (1, 2, 8, 3, [0, 0, 1], [4]),           # row 1's own positive (offset 3)
    (1, 2, 8, 0, [0, 2, 2], [5, 5]),        # repeated column
    (1, 2, 8, 0, [0, 2, 2], [6, 2]),        # decreasing columns
    (1, 2, 8, 0, [0, 1, 1], [8]),           # past N
    (1, 2, 8, 0, [0, 1, 1], [-2]),          # negative
    (0, 8, 8, 0, [0] * 8 + [1], [3]),       # softmax kinds take no list
    (2, 2, 8, 0, [0, 1, 1], [3]),
    (3, 2, 8, 0, [0, 1, 1], [1]),           # one-set: row 0's pair partner
    (3, 2, 8, 0, [0, 0, 1], [1]),           # one-set: row 1 itself
    (4, 3, 7, 0, [0, 1, 1, 1], [1]),        # one-set relations: row 0 lists row 1, row 1 not row 0
    (4, 2, 7, 2, [0, 0, 1], [3]),           # one-set relations: row 3 (share row 1) lists itself
    (4, 2, 7, 0, [0, 1, 1], [7]),           # one-set relations: past N
])
def test_positive_list_checks(kind, R, N, off, row_ptr, col):
    rp = np.asarray(row_ptr, dtype=np.int64)
    pc = np.asarray(col if col else [0], dtype=np.int32)
    opt = binding.Options()
    opt.row_offset = off
    opt.pos_row_ptr = rp.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))
    opt.pos_col = pc.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    k = 0x20000
    q = k + 2 * off * 1024 if kind in (3, 4) else 0x10000
    dk = 0 if kind in (3, 4) else 0x50000
    assert _call(q=q, k=k, R=R, N=N, kind=kind, dk=dk, opt=opt) == 1, binding.last_error()
    msg = binding.last_error()
    assert ("sigmoid" in msg) if kind in (0, 2) else ("pos_row_ptr" in msg or "row" in msg), msg


def test_positive_list_needs_col_array():
    rp = np.asarray([0, 1, 1], dtype=np.int64)
    opt = binding.Options()
    opt.pos_row_ptr = rp.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))
    assert _call(R=2, N=8, kind=1, opt=opt) == 1
    assert "pos_col" in binding.last_error()


def test_workspace_bytes_with_positives():
    base = binding.workspace_bytes(256, 1024, 1024, 5, 1)
    with_list = binding.workspace_bytes(256, 1024, 1024, 5, 1, 5000)
    assert with_list >= base + 4 * (257 + 1025 + 2 * 5000)
    assert binding.workspace_bytes(256, 1024, 1024, 5, 1, -1) == base
    assert binding.workspace_bytes(256, 256, 1024, 5, 0, 10) == 0  # softmax kinds take no list
    assert binding.workspace_bytes(256, 1024, 1024, 5, 3, 5000) > binding.workspace_bytes(256, 1024, 1024, 5, 3)


def test_binding_refuses_gradient_buffers_the_kernels_would_overrun():
    import torch
    dev = torch.device("cpu")
    ok = torch.empty(4, 8, dtype=torch.float32)
    binding._check_grad_buffer("dq", ok, (4, 8), dev)
    binding._check_grad_buffer("dq", None, (4, 8), dev)
    with pytest.raises(TypeError):
        binding._check_grad_buffer("dq", ok.to(torch.bfloat16), (4, 8), dev)
    with pytest.raises(ValueError):
        binding._check_grad_buffer("dq", ok, (4, 16), dev)
    with pytest.raises(ValueError):
        binding._check_grad_buffer("dk", torch.empty(8, 4, dtype=torch.float32).t(), (4, 8), dev)
    with pytest.raises(ValueError):
        binding._check_grad_buffer("dk", ok, (4, 8), torch.device("cuda", 0))


def test_package_exports():
    import contrastive_embedding_loss_amd as pkg
    assert (pkg.INFONCE, pkg.SIGLIP, pkg.INFONCE_ROWS, pkg.ONESET_SIGLIP) == (0, 1, 2, 3)
    assert pkg.ONESET_SIGLIP == binding.ONESET_SIGLIP
    for name in pkg._BINDING_NAMES:
        assert getattr(pkg, name) is getattr(binding, name), name
    with pytest.raises(AttributeError):
        pkg.fwd_bwd_ex


def test_oneset_relations_call_checks():
    # the one-set form with listed relations: q inside k, no dk, no positive logit; an odd set and
    # no lists at all are valid (checked with supported(), which touches no device)
    k = 0x20000
    assert _call(q=k, k=k, R=7, N=7, kind=4, dk=0x50000) == 1 and "dk" in binding.last_error()
    assert _call(q=0x10000, k=k, R=7, N=7, kind=4, dk=0) == 1
    opt = binding.Options()
    opt.pos_logit_out = 0x70000
    assert _call(q=k, k=k, R=7, N=7, kind=4, dk=0, opt=opt) == 1 and "positive logit" in binding.last_error()
    assert binding.supported(1024, PREFIXES, 4) == 0
    assert binding.workspace_bytes(7, 7, 1024, 5, 4) == binding.workspace_bytes(7, 7, 1024, 5, 3)
    assert binding.workspace_bytes(7, 7, 1024, 5, 4, 10) > binding.workspace_bytes(7, 7, 1024, 5, 4)
