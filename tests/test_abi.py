"""The C-ABI library: exports, signatures, workspace queries and argument
validation.  No compute call is made; nothing here needs a GPU."""
import ctypes
import os
import re

import pytest
import torch

from newton_schulz_08_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dmuon.h")


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dmuon_[a-z_0-9]+)\s*\(", text)))


def header_defines():
    return dict(re.findall(r"#define\s+(DMUON_[A-Z_0-9]+)\s+(\d+)", open(HEADER).read()))


@pytest.fixture(scope="module")
def lib():
    return _lib.load()


def test_library_exports_every_declared_symbol(lib):
    funcs = header_functions()
    assert len(funcs) >= 9
    for f in funcs:
        assert hasattr(lib, f), f"{f} declared in dmuon.h but not exported"


def test_binding_signatures_cover_header():
    assert sorted(_lib.SIGNATURES) == header_functions()


def test_constants_match_header():
    for name, val in header_defines().items():
        if hasattr(_lib, name):
            assert getattr(_lib, name) == int(val), name
    for name in ("DMUON_F32", "DMUON_BF16", "DMUON_OK", "DMUON_ERR_INVALID_ARG", "DMUON_ERR_WORKSPACE",
                 "DMUON_ERR_NO_DEVICE", "DMUON_MIN_NS_NUMEL"):
        assert name in header_defines()


def test_status_strings(lib):
    for s in range(7):
        assert lib.dmuon_status_string(s).decode() not in ("", "unknown status")
    assert lib.dmuon_status_string(99).decode() == "unknown status"
    assert b"gfx950" in lib.dmuon_backend_info()


def _ws(lib, shapes, dt=0, fn="dmuon_muon_step_workspace_bytes", cfg=None):
    n = len(shapes)
    rows = (ctypes.c_int64 * max(n, 1))(*[s[0] for s in shapes])
    cols = (ctypes.c_int64 * max(n, 1))(*[s[1] for s in shapes])
    out = ctypes.c_size_t(0)
    st = getattr(lib, fn)(n, rows, cols, dt, ctypes.byref(cfg) if cfg is not None else None, ctypes.byref(out))
    return st, out.value


def _cfg(backend=0, terms=0, per_step=0, coeffs=()):
    c = _lib.NsConfig()
    c.backend, c.num_terms, c.per_step = backend, terms, per_step
    arr = (ctypes.c_float * max(len(coeffs), 1))(*coeffs)
    c.coeffs = ctypes.cast(arr, ctypes.POINTER(ctypes.c_float)) if coeffs else None
    c._keep = arr
    return c


def test_workspace_layout_exact(lib):
    # one 512x2048 fp32 matrix: descriptor 128 B, prefix 8 B, the sum-of-squares
    # partials of its 16 x 64 blocks (1024 blocks, 4 KB), scales 16 B -- each
    # region 256-aligned -- then the fp32 iterate in two buffers that
    # alternate between steps, and A; an fp32 matrix with m' = 512 runs on
    # 128 x 128 tiles, and its Gram's K = 2048 is cut into 2 slices whose fp32
    # 128x128 partial products (sized for all 4 x 4 tiles) follow
    st, nbytes = _ws(lib, [(512, 2048)], dt=0)
    assert st == 0
    mb = 512 * 2048 * 4
    small_part = 4 * 4 * 2 * 128 * 128 * 4
    assert nbytes == 256 + 256 + 4096 + 256 + 2 * mb + 512 * 512 * 4 + small_part
    # bf16: the iterate's low half + two operand copies (its high half, one per
    # step parity) + bf16 Gram; 256 x 256 tiles, two tile rows, so K = 2048 is
    # cut into 4 slices of partial products sized for all 2 x 2 tiles
    part = 2 * 2 * 4 * 256 * 256 * 4
    st, nb16 = _ws(lib, [(512, 2048)], dt=1)
    assert nb16 == 256 + 256 + 4096 + 256 + 512 * 2048 * (2 + 2 + 2) + 512 * 512 * 2 + part
    # a three-term polynomial adds the m' x m' buffer B = c1 A + c2 A^2 (its
    # square product, K = 512 in 2 slices, shares the partial products)
    st, nb3 = _ws(lib, [(512, 2048)], dt=1, cfg=_cfg(terms=3, coeffs=(3.4445, -4.775, 2.0315)))
    assert st == 0 and nb3 == nb16 + 512 * 512 * 2
    # three tile rows or more: no slices, no partial products
    st, big = _ws(lib, [(768, 2048)], dt=0)
    assert big == 256 + 256 + (768 // 16) * (2048 // 64) * 4 + 256 + 2 * 768 * 2048 * 4 + 768 * 768 * 4
    # two terms or another backend need nothing extra
    assert _ws(lib, [(512, 2048)], dt=1, cfg=_cfg(terms=2, coeffs=(1.5, -0.5)))[1] == nb16
    assert _ws(lib, [(512, 2048)], dt=1, cfg=_cfg(backend=1))[1] == nb16


def test_ns_config_validation(lib):
    E = _lib
    for bad in (_cfg(backend=2), _cfg(terms=1, coeffs=(1.0,)), _cfg(terms=4, coeffs=(1, 2, 3, 4)),
                _cfg(per_step=2), _cfg(terms=2)):
        assert _ws(lib, [(64, 64)], cfg=bad)[0] == E.DMUON_ERR_INVALID_ARG
    nan = _cfg(terms=2, coeffs=(1.5, float("nan")))
    assert _step(lib, cfg=nan) == E.DMUON_ERR_INVALID_ARG
    assert "finite" in _lib.last_error()


def test_workspace_route_and_padding(lib):
    # 2048x32 (65,536 elements) takes the elementwise route: no NS buffers
    st, small = _ws(lib, [(2048, 32)])
    assert st == 0 and small < 64 * 1024
    # ns_batched orthogonalises every matrix, so the same shape needs buffers
    st, ns = _ws(lib, [(2048, 32)], fn="dmuon_ns_workspace_bytes")
    assert st == 0 and ns > 2048 * 256 * 4
    # ragged shapes pad to 256 in both wide dimensions
    st, a = _ws(lib, [(300, 700)])
    st, b = _ws(lib, [(512, 768)])
    assert a == b
    st, t = _ws(lib, [(700, 300)])
    assert t == a


def test_workspace_query_errors(lib):
    assert _ws(lib, [(0, 5)])[0] == _lib.DMUON_ERR_INVALID_ARG
    assert _ws(lib, [(5, 70000)])[0] == _lib.DMUON_ERR_INVALID_ARG
    assert _ws(lib, [(5, 5)], dt=7)[0] == _lib.DMUON_ERR_UNSUPPORTED_DTYPE
    assert _ws(lib, [])[0] == 0 and _ws(lib, [])[1] == 0
    rows = (ctypes.c_int64 * 1)(4)
    assert lib.dmuon_muon_step_workspace_bytes(1, rows, rows, 0, None, None) == _lib.DMUON_ERR_INVALID_ARG


def _step(lib, count=1, shapes=((64, 64),), ptrs=None, dt=0, steps=5, mu=0.95, lr=0.02, ws=None, wsb=0,
          upd=None, cfg=None, wd=0.0, mode=0):
    n = len(shapes)
    rows = (ctypes.c_int64 * max(n, 1))(*[s[0] for s in shapes])
    cols = (ctypes.c_int64 * max(n, 1))(*[s[1] for s in shapes])
    base = 0x10000000
    if ptrs is None:
        ptrs = ([base + 0x100000 * i for i in range(n)], [base + 0x100000 * (i + n) for i in range(n)],
                [base + 0x100000 * (i + 2 * n) for i in range(n)])
    P = lambda v: (ctypes.c_void_p * max(n, 1))(*v)  # noqa: E731
    return lib.dmuon_muon_step(count, P(ptrs[0]), P(ptrs[1]), P(ptrs[2]), rows, cols, dt, steps,
                               ctypes.byref(cfg) if cfg is not None else None, ctypes.c_float(mu), 1,
                               ctypes.c_float(lr), ctypes.c_float(wd), mode, None, upd, None,
                               ctypes.c_void_p(ws), wsb, None)


def test_validation_before_any_device_work(lib):
    E = _lib
    assert _step(lib, count=-1) == E.DMUON_ERR_INVALID_ARG
    assert _step(lib, count=0) == E.DMUON_OK
    assert _step(lib, shapes=((0, 4),)) == E.DMUON_ERR_INVALID_ARG
    assert _step(lib, dt=3) == E.DMUON_ERR_UNSUPPORTED_DTYPE
    assert _step(lib, steps=-1) == E.DMUON_ERR_INVALID_ARG
    assert _step(lib, steps=65) == E.DMUON_ERR_INVALID_ARG
    assert _step(lib, mu=float("nan")) == E.DMUON_ERR_INVALID_ARG
    assert _step(lib, lr=float("inf")) == E.DMUON_ERR_INVALID_ARG
    assert _step(lib, wd=float("nan")) == E.DMUON_ERR_INVALID_ARG
    assert _step(lib, mode=2) == E.DMUON_ERR_INVALID_ARG
    per_step_short = _cfg(terms=2, per_step=1, coeffs=(1.5, -0.5))   # 1 set read for steps=1 only
    assert _step(lib, steps=1, cfg=per_step_short, ws=None) == E.DMUON_ERR_WORKSPACE
    assert _step(lib, ptrs=([0], [0x2000], [0x3000])) == E.DMUON_ERR_INVALID_ARG
    assert "params[0] is NULL" in _lib.last_error()
    assert _step(lib, ptrs=([0x1000], [0x1000], [0x3000])) == E.DMUON_ERR_INVALID_ARG
    assert "alias" in _lib.last_error()
    two = ((64, 64), (64, 64))
    assert _step(lib, count=2, shapes=two, ptrs=([0x1000, 0x1000], [0x2000, 0x2100], [0x3000, 0x3100])) == \
        E.DMUON_ERR_INVALID_ARG
    # workspace missing / short / misaligned
    assert _step(lib, ws=None) == E.DMUON_ERR_WORKSPACE
    assert _step(lib, ws=0x100000, wsb=16) == E.DMUON_ERR_WORKSPACE
    st, need = _ws(lib, [(64, 64)])
    assert _step(lib, ws=0x100010, wsb=need) == E.DMUON_ERR_WORKSPACE
    assert "aligned" in _lib.last_error()


def test_ns_batched_validation(lib):
    rows = (ctypes.c_int64 * 2)(8, 8)
    P = (ctypes.c_void_p * 2)
    E = _lib
    assert lib.dmuon_ns_batched(2, P(0x1000, 0x2000), P(0x3000, 0x3000), rows, rows, 0, 5, None, None, 0,
                                None) == E.DMUON_ERR_INVALID_ARG
    assert lib.dmuon_ns_batched(2, P(0x1000, 0x2000), P(0x3000, 0x4000), rows, rows, 0, -2, None, None, 0,
                                None) == E.DMUON_ERR_INVALID_ARG
    assert lib.dmuon_ns_batched(2, P(0x1000, 0x2000), P(0x3000, 0x4000), rows, rows, 0, 5, None, None, 0,
                                None) == E.DMUON_ERR_WORKSPACE
    assert lib.dmuon_ns_batched(0, None, None, None, None, 0, 5, None, None, 0, None) == E.DMUON_OK
    bad = _cfg(backend=5)
    assert lib.dmuon_ns_batched(2, P(0x1000, 0x2000), P(0x3000, 0x4000), rows, rows, 0, 5, ctypes.byref(bad),
                                None, 0, None) == E.DMUON_ERR_INVALID_ARG


@pytest.mark.skipif(torch.cuda.device_count() > 0, reason="checks the no-device path; a GPU is visible")
def test_no_device_reported(lib):
    st, need = _ws(lib, [(64, 64)])
    assert _step(lib, ws=0x10000000, wsb=need) == _lib.DMUON_ERR_NO_DEVICE


def test_profile_read_empty(lib):
    stats = (_lib.KernelStat * 4)()
    n = ctypes.c_int(-1)
    assert lib.dmuon_profile_read(stats, 4, ctypes.byref(n)) == 0
    assert n.value == 0


def test_clip_workspace_and_validation(lib):
    E = _lib
    n = (ctypes.c_int64 * 3)(4096, 10, 0)
    out = ctypes.c_size_t(0)
    assert lib.dmuon_clip_grad_norm_workspace_bytes(3, n, 2, ctypes.byref(out)) == 0
    # descriptors, prefix, segment starts, max_norm, coefficients, 2 tile partials: 256-aligned regions
    assert out.value == 6 * 256
    assert lib.dmuon_clip_grad_norm_workspace_bytes(3, n, 0, ctypes.byref(out)) == E.DMUON_ERR_INVALID_ARG
    bad = (ctypes.c_int64 * 1)(-1)
    assert lib.dmuon_clip_grad_norm_workspace_bytes(1, bad, 1, ctypes.byref(out)) == E.DMUON_ERR_INVALID_ARG
    P = (ctypes.c_void_p * 2)
    nn = (ctypes.c_int64 * 2)(8, 8)
    seg = (ctypes.c_int * 2)(0, 1)
    mn = (ctypes.c_float * 2)(1.0, 1.0)
    call = lambda ptrs=P(0x1000, 0x2000), segs=seg, m=mn, p=2.0, dt=0, nseg=2, ws=None: lib.dmuon_clip_grad_norm(  # noqa: E731
        2, ptrs, nn, dt, segs, nseg, m, ctypes.c_float(p), None, ws, 1 << 20, None)
    assert call(p=0.0) == E.DMUON_ERR_INVALID_ARG
    assert call(p=float("nan")) == E.DMUON_ERR_INVALID_ARG
    assert call(dt=5) == E.DMUON_ERR_UNSUPPORTED_DTYPE
    assert call(segs=(ctypes.c_int * 2)(0, 2)) == E.DMUON_ERR_INVALID_ARG
    assert call(m=(ctypes.c_float * 2)(1.0, -1.0)) == E.DMUON_ERR_INVALID_ARG
    assert call(ptrs=P(0x1000, 0x1000)) == E.DMUON_ERR_INVALID_ARG
    assert "alias" in _lib.last_error()
    assert call() == E.DMUON_ERR_WORKSPACE
    assert call(ws=0x100010) == E.DMUON_ERR_WORKSPACE


def test_adamw_workspace_and_validation(lib):
    E = _lib
    n = (ctypes.c_int64 * 3)(4096, 10, 0)
    out = ctypes.c_size_t(0)
    assert lib.dmuon_adamw_step_workspace_bytes(3, n, ctypes.byref(out)) == 0
    assert out.value == 2 * 256       # descriptors (3 x 48 B) and the tile prefix, 256-aligned regions
    assert lib.dmuon_adamw_step_workspace_bytes(0, None, ctypes.byref(out)) == 0 and out.value == 0
    bad = (ctypes.c_int64 * 1)(-1)
    assert lib.dmuon_adamw_step_workspace_bytes(1, bad, ctypes.byref(out)) == E.DMUON_ERR_INVALID_ARG
    P = (ctypes.c_void_p * 2)
    nn = (ctypes.c_int64 * 2)(8, 8)

    def call(p=P(0x1000, 0x2000), g=P(0x3000, 0x4000), m=P(0x5000, 0x6000), v=P(0x7000, 0x8000), dt=0, step=1,
             lr=1e-3, b1=0.9, b2=0.999, eps=1e-8, wd=0.01, ws=None, wsb=1 << 20, numel=nn):
        return lib.dmuon_adamw_step(2, p, g, m, v, numel, dt, step, ctypes.c_float(lr), ctypes.c_float(b1),
                                    ctypes.c_float(b2), ctypes.c_float(eps), ctypes.c_float(wd), ws, wsb, None)

    assert call(dt=5) == E.DMUON_ERR_UNSUPPORTED_DTYPE
    assert call(step=0) == E.DMUON_ERR_INVALID_ARG
    assert call(lr=float("nan")) == E.DMUON_ERR_INVALID_ARG
    assert call(wd=float("inf")) == E.DMUON_ERR_INVALID_ARG
    assert call(eps=-1.0) == E.DMUON_ERR_INVALID_ARG
    assert call(b1=1.0) == E.DMUON_ERR_INVALID_ARG
    assert call(b2=-0.5) == E.DMUON_ERR_INVALID_ARG
    assert call(b2=float("nan")) == E.DMUON_ERR_INVALID_ARG
    assert call(p=P(0, 0x2000)) == E.DMUON_ERR_INVALID_ARG
    assert "NULL" in _lib.last_error()
    assert call(m=P(0x5000, 0x3000)) == E.DMUON_ERR_INVALID_ARG
    assert "alias" in _lib.last_error()
    assert call(p=P(0x1001, 0x2000)) == E.DMUON_ERR_INVALID_ARG
    assert "aligned" in _lib.last_error()
    assert call(p=P(0x1002, 0x2000), g=P(0x3002, 0x4000), dt=_lib.DMUON_BF16) == E.DMUON_ERR_WORKSPACE
    # an empty tensor's pointers are not looked at
    assert call(p=P(0, 0x2000), g=P(0, 0x4000), numel=(ctypes.c_int64 * 2)(0, 8)) == E.DMUON_ERR_WORKSPACE
    assert call() == E.DMUON_ERR_WORKSPACE
    assert call(ws=0x100010) == E.DMUON_ERR_WORKSPACE
    assert lib.dmuon_adamw_step(0, None, None, None, None, None, 0, 1, ctypes.c_float(1e-3), ctypes.c_float(0.9),
                                ctypes.c_float(0.999), ctypes.c_float(1e-8), ctypes.c_float(0.0), None, 0,
                                None) == E.DMUON_OK
    if torch.cuda.device_count() == 0:
        assert call(ws=0x10000000) == E.DMUON_ERR_NO_DEVICE


def test_noalloc_rejects_oversized_sets_before_device_work(lib):
    E = _lib
    shapes = ((4096, 4096), (4096, 4096))
    need = _ws(lib, shapes, dt=1)[1]
    assert need > E.DMUON_NOALLOC_SCRATCH_BYTES
    rows = (ctypes.c_int64 * 2)(4096, 4096)
    P = (ctypes.c_void_p * 2)
    st = lib.dmuon_muon_step_noalloc(2, P(0x1000, 0x2000), P(0x3000, 0x4000), P(0x5000, 0x6000), rows, rows, 1, 5,
                                     None, ctypes.c_float(0.95), 1, ctypes.c_float(0.02), ctypes.c_float(0.0), 0,
                                     None, None, None, None)
    assert st == E.DMUON_ERR_WORKSPACE
    assert "DMUON_NOALLOC_SCRATCH_BYTES" in _lib.last_error()
    # the same argument checks as dmuon_muon_step run first
    st = lib.dmuon_muon_step_noalloc(2, P(0x1000, 0x1000), P(0x3000, 0x4000), P(0x5000, 0x6000), rows, rows, 1, 5,
                                     None, ctypes.c_float(0.95), 1, ctypes.c_float(0.02), ctypes.c_float(0.0), 0,
                                     None, None, None, None)
    assert st == E.DMUON_ERR_INVALID_ARG and "alias" in _lib.last_error()


def _summary(lib, shapes, dt=1, steps=5, muon=1, cfg=None):
    n = len(shapes)
    rows = (ctypes.c_int64 * n)(*[s[0] for s in shapes])
    cols = (ctypes.c_int64 * n)(*[s[1] for s in shapes])
    need = ctypes.c_size_t(0)
    c = ctypes.byref(cfg) if cfg is not None else None
    assert lib.dmuon_plan_summary(n, rows, cols, dt, c, steps, muon, None, 0, ctypes.byref(need)) == 0
    buf = ctypes.create_string_buffer(need.value)
    assert lib.dmuon_plan_summary(n, rows, cols, dt, c, steps, muon, buf, need.value, None) == 0
    return buf.value.decode(), need.value, (n, rows, cols, c)


def test_plan_summary(lib):
    """The plan text names the routes, shape groups, orientation counts, K
    slices and launches, with the algorithmic flops of one Newton-Schulz step
    (the same count the benchmark uses)."""
    import bench
    shapes = [(4096, 4096), (14336, 4096), (4096, 14336), (14336, 4096), (1024, 4096), (2048, 32), (512, 2048)]
    text, need, args = _summary(lib, shapes)
    lines = text.splitlines()
    assert "7 matrices (bf16)" in lines[0] and "6 Newton-Schulz in 4 shape groups" in lines[0]
    assert "(2 iterated on the transpose), 1 elementwise" in lines[0]
    assert "group 0: 3 x padded 4096 x 14336 (2 transposed)" in lines[1]
    assert "K 2048 in 4 slices" in text                      # the 512 x 2048 matrix
    assert "1 Gram launch(es) + 1 slice-sum launch(es), 1 update launch(es)" in text
    syrk, gemm = bench.ns_flops([s for s in shapes if s[0] * s[1] >= 100000], 1)
    assert f"{syrk + gemm:.4g} flop algorithmic" in text
    # ns_batched plans orthogonalise every matrix; truncation keeps the NUL
    assert "7 Newton-Schulz" in _summary(lib, shapes, muon=0)[0]
    small = ctypes.create_string_buffer(16)
    n, rows, cols, c = args
    assert lib.dmuon_plan_summary(n, rows, cols, 1, c, 5, 1, small, 16, None) == 0
    assert small.value.decode() == text[:15]
    assert lib.dmuon_plan_summary(n, rows, cols, 1, c, -1, 1, None, 0, None) == _lib.DMUON_ERR_INVALID_ARG
    direct = _cfg(backend=1)
    assert "Gram 136 lower-triangle 256x256 tiles each" in _summary(lib, [(4096, 4096)])[0]
    # fp32 with m' <= 512: 128 x 128 tiles in launches of their own
    t32 = _summary(lib, [(4096, 4096), (2048, 512)], dt=0)[0]
    assert "Gram 10 lower-triangle 128x128 tiles each, K 2048 in 2 slices; update 64 tiles each" in t32
    assert "2 Gram launch(es) + 1 slice-sum launch(es), 2 update launch(es)" in t32
    assert "Gram 256 full 256x256 tiles each" in _summary(lib, [(4096, 4096)], cfg=direct)[0]
