"""The C ABI without a GPU: the library loads, exports every function the
header declares, and rejects bad arguments on the host (no launch happens on
any of these paths, so they run on a machine without a GPU)."""
import ctypes
import os
import re

import pytest

from bit_trainable_attention_block_amd import binding as bd

INCLUDE = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include")
HEADER = os.path.join(INCLUDE, "sage.h")


def _declared_functions():
    """Every function any header under include/ declares."""
    names = set()
    for f in sorted(os.listdir(INCLUDE)):
        if f.endswith(".h"):
            text = re.sub(r"/\*.*?\*/", "", open(os.path.join(INCLUDE, f)).read(), flags=re.S)
            names |= set(re.findall(r"\b(sage_[a-z_0-9]+)\s*\(", text))
    return sorted(names)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(bd.LIB_PATH):
        pytest.skip("libsage.so not built")
    return bd.load()


def test_every_declared_symbol_is_exported(lib):
    names = _declared_functions()
    assert {"sage_quantize", "sage_fwd", "sage_bwd_pre", "sage_bwd"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(bd.SIGNATURES), "binding signatures out of sync with the header"


def test_struct_layouts_match_header():
    assert ctypes.sizeof(bd.c_shape) == 15 * 4
    assert ctypes.sizeof(bd.c_qtensors) == 12 * 8
    assert ctypes.sizeof(bd.c_dotensors) == 4 * 8


def _shape(**kw):
    base = dict(B=1, H=2, N=256, D=128, bq=128, bkv=64, dtype=1, causal=0, k_smooth=1, q_smooth=0, sm_scale=0.0,
                dp_int8=0, p_static=0, qk_norm=0, fp8=0)
    base.update(kw)
    return bd.c_shape(**base)


FAKE = 0x10000  # aligned, never dereferenced: every case below fails validation first


def _qt(**kw):
    vals = {f: FAKE for f in bd.QT_FIELDS}
    vals.update(kw)
    return bd.c_qtensors(**vals)


def _dot(**kw):
    vals = {f: FAKE for f in bd.DO_FIELDS}
    vals.update(kw)
    return bd.c_dotensors(**vals)


BAD_SHAPES = [
    (dict(D=96), bd.SAGE_EUNSUPPORTED),
    (dict(D=256), bd.SAGE_EUNSUPPORTED),
    (dict(bq=32), bd.SAGE_EUNSUPPORTED),
    (dict(bkv=128), bd.SAGE_EUNSUPPORTED),
    (dict(dtype=2), bd.SAGE_EUNSUPPORTED),
    (dict(N=200), bd.SAGE_EUNSUPPORTED),          # ragged: not a multiple of the blocks
    (dict(N=192, bq=128), bd.SAGE_EUNSUPPORTED),
    (dict(N=-64), bd.SAGE_EINVAL),
    (dict(B=-1), bd.SAGE_EINVAL),
    (dict(causal=2), bd.SAGE_EINVAL),
    (dict(dp_int8=2), bd.SAGE_EINVAL),
    (dict(p_static=-1), bd.SAGE_EINVAL),
    (dict(qk_norm=3), bd.SAGE_EINVAL),
    (dict(fp8=2), bd.SAGE_EINVAL),
    (dict(fp8=1, dp_int8=1), bd.SAGE_EUNSUPPORTED),   # INT8-only ablations have no E4M3 form
    (dict(fp8=1, p_static=1), bd.SAGE_EUNSUPPORTED),
    (dict(sm_scale=-1.0), bd.SAGE_EINVAL),
    (dict(sm_scale=float("nan")), bd.SAGE_EINVAL),
    (dict(B=70000, H=1), bd.SAGE_EUNSUPPORTED),
    (dict(N=1 << 24), bd.SAGE_EUNSUPPORTED),
]


@pytest.mark.parametrize("kw,code", BAD_SHAPES)
def test_bad_shapes_rejected_by_every_call(lib, kw, code):
    s = _shape(**kw)
    qt, dot = _qt(), _dot()
    assert lib.sage_quantize(ctypes.byref(s), FAKE, FAKE, FAKE, ctypes.byref(qt), FAKE, None) == code
    assert lib.sage_fwd(ctypes.byref(s), ctypes.byref(qt), FAKE, FAKE, None) == code
    assert lib.sage_bwd_pre(ctypes.byref(s), FAKE, FAKE, ctypes.byref(dot), None) == code
    assert lib.sage_bwd(ctypes.byref(s), ctypes.byref(qt), ctypes.byref(dot), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                        FAKE, None) == code
    assert lib.sage_cast_grads(ctypes.byref(s), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == code
    assert lib.sage_quantize_workspace_bytes(ctypes.byref(s)) == 0
    assert lib.sage_bwd_workspace_bytes(ctypes.byref(s)) == 0


def test_null_shape(lib):
    assert lib.sage_fwd(None, ctypes.byref(_qt()), FAKE, FAKE, None) == bd.SAGE_EINVAL


@pytest.mark.parametrize("field", bd.QT_FIELDS)
def test_missing_or_misaligned_qtensor(lib, field):
    s = _shape(q_smooth=1, qk_norm=1, dp_int8=1)   # every field required
    for bad in (None, FAKE + 4):
        qt = _qt(**{field: bad})
        assert lib.sage_fwd(ctypes.byref(s), ctypes.byref(qt), FAKE, FAKE, None) == bd.SAGE_EINVAL
        assert lib.sage_quantize(ctypes.byref(s), FAKE, FAKE, FAKE, ctypes.byref(qt), FAKE, None) == bd.SAGE_EINVAL


def test_qsmooth_buffers_only_needed_with_qsmooth(lib):
    # mu_q / qk_bias may be NULL without Q-smoothing; then the call gets past
    # validation, so only check the ones that must fail here.
    s = _shape(q_smooth=1)
    qt = _qt(mu_q=None)
    assert lib.sage_fwd(ctypes.byref(s), ctypes.byref(qt), FAKE, FAKE, None) == bd.SAGE_EINVAL


@pytest.mark.parametrize("field", bd.DO_FIELDS)
def test_missing_dotensor(lib, field):
    s = _shape(dp_int8=1)   # every field required (dor only with the INT8-dP ablation)
    dot = _dot(**{field: None})
    assert lib.sage_bwd_pre(ctypes.byref(s), FAKE, FAKE, ctypes.byref(dot), None) == bd.SAGE_EINVAL
    assert lib.sage_bwd(ctypes.byref(s), ctypes.byref(_qt()), ctypes.byref(dot), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                        FAKE, None) == bd.SAGE_EINVAL


def test_ablation_buffers_required_only_with_dp_int8(lib):
    """vr and dor hold the INT8-dP ablation's row-tile codes: with dp_int8 a
    missing one is refused on the host (the method's path never reads them)."""
    s = _shape(dp_int8=1)
    assert lib.sage_fwd(ctypes.byref(s), ctypes.byref(_qt(vr=None)), FAKE, FAKE, None) == bd.SAGE_EINVAL
    assert lib.sage_bwd_pre(ctypes.byref(s), FAKE, FAKE, ctypes.byref(_dot(dor=None)), None) == bd.SAGE_EINVAL


def test_io_pointers_checked(lib):
    s = _shape()
    qt = ctypes.byref(_qt())
    assert lib.sage_quantize(ctypes.byref(s), None, FAKE, FAKE, qt, FAKE, None) == bd.SAGE_EINVAL
    assert lib.sage_quantize(ctypes.byref(s), FAKE, FAKE, FAKE, qt, None, None) == bd.SAGE_EINVAL  # workspace
    assert lib.sage_quantize(ctypes.byref(s), FAKE, FAKE, FAKE, qt, FAKE + 4, None) == bd.SAGE_EINVAL
    assert lib.sage_fwd(ctypes.byref(s), qt, FAKE + 2, FAKE, None) == bd.SAGE_EINVAL
    assert lib.sage_fwd(ctypes.byref(s), qt, FAKE, None, None) == bd.SAGE_EINVAL
    dot = ctypes.byref(_dot())
    # sage_bwd(shape, qk, dos, V, dO, L, workspace, dQ, dK, dV, stream): each pointer checked
    for k in range(7):
        args = [FAKE] * 7
        args[k] = None
        assert lib.sage_bwd(ctypes.byref(s), qt, dot, *args, None) == bd.SAGE_EINVAL, k
        args[k] = FAKE + 2
        assert lib.sage_bwd(ctypes.byref(s), qt, dot, *args, None) == bd.SAGE_EINVAL, k


def test_empty_problem_is_a_no_op(lib):
    for kw in (dict(B=0), dict(H=0), dict(N=0)):
        s = _shape(**kw)
        # NULL everywhere: nothing may be dereferenced or launched
        assert lib.sage_quantize(ctypes.byref(s), None, None, None, None, None, None) == bd.SAGE_OK
        assert lib.sage_fwd(ctypes.byref(s), None, None, None, None) == bd.SAGE_OK
        assert lib.sage_bwd_pre(ctypes.byref(s), None, None, None, None) == bd.SAGE_OK
        assert lib.sage_bwd(ctypes.byref(s), None, None, None, None, None, None, None, None, None, None) == bd.SAGE_OK


def test_cast_grads_checks(lib):
    s = ctypes.byref(_shape())
    f = lib.sage_cast_grads
    assert f(None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == bd.SAGE_EINVAL
    # a pair with one side missing, or a misaligned side
    assert f(s, FAKE, None, None, None, None, None, None) == bd.SAGE_EINVAL
    assert f(s, None, None, None, FAKE, None, None, None) == bd.SAGE_EINVAL
    assert f(s, FAKE, FAKE, None, FAKE, FAKE, FAKE, None) == bd.SAGE_EINVAL
    assert f(s, FAKE + 4, None, None, FAKE, None, None, None) == bd.SAGE_EINVAL
    assert f(s, None, FAKE, None, None, FAKE + 2, None, None) == bd.SAGE_EINVAL
    # nothing to convert, or an empty problem: no launch
    assert f(s, None, None, None, None, None, None, None) == bd.SAGE_OK
    for kw in (dict(B=0), dict(H=0), dict(N=0)):
        assert f(ctypes.byref(_shape(**kw)), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == bd.SAGE_OK


def test_workspace_size_and_strings(lib):
    s = _shape(B=2, H=3, D=64)
    # the float64 column sums of K of every 64-row block: B*H*(N/64)*D*8
    assert lib.sage_quantize_workspace_bytes(ctypes.byref(s)) == 2 * 3 * (256 // 64) * 64 * 8
    # N = 256, bq = 128, bkv = 64: 2 x 4 tiles of 128 x 64 codes + a float each, per head
    tiles = 2 * 3 * 2 * 4
    codes = -(-tiles * 128 * 64 // 256) * 256
    assert lib.sage_bwd_workspace_bytes(ctypes.byref(s)) == codes + tiles * 4
    c = _shape(B=1, H=1, N=512, causal=1)      # causal: only the visible tiles (2 + 4 + 6 + 8)
    assert lib.sage_bwd_workspace_bytes(ctypes.byref(c)) == 20 * 128 * 64 + 20 * 4
    for code in (0, -1, -2, -3, 7):
        assert lib.sage_status_str(code)
    assert b"gfx950" in lib.sage_version()
    assert lib.sage_last_hip_error() == 0


def test_layout_offsets_are_permutations():
    import numpy as np
    for kind in ("R32", "C64P"):
        for N, D in ((64, 64), (128, 128), (192, 64)):
            off = bd.layout_offsets(kind, N, D)
            assert np.array_equal(np.sort(off.ravel()), np.arange(N * D)), (kind, N, D)


def test_probe_rejects_bad_arguments(lib):
    buf = (ctypes.c_uint64 * 4)()
    base = ctypes.addressof(buf)
    for blocks, iters, ptr in ((0, 1, base), (1, 0, base), (1, 1, None), (1, 1, base + 4)):
        assert lib.sage_probe_mfma_i8(blocks, iters, ptr, None) == bd.SAGE_EINVAL
        assert lib.sage_probe_mfma_bf16(blocks, iters, ptr, None) == bd.SAGE_EINVAL


def test_fp8_probe_rejects_bad_arguments(lib):
    buf = (ctypes.c_uint8 * 8192)()
    base = ctypes.addressof(buf) + (-ctypes.addressof(buf)) % 16
    for a, b, c, d in ((None, base, base, base), (base, base + 4, base, base), (base, base, base, None)):
        assert lib.sage_probe_fp8_products(a, b, c, d, None) == bd.SAGE_EINVAL


def test_autograd_wrapper_rejects_cpu_tensors():
    """The training wrapper is argument marshalling only: on CPU tensors it
    raises before touching the library (there is no CPU fallback)."""
    import torch

    from bit_trainable_attention_block_amd.autograd import sage_attention
    x = torch.zeros((1, 1, 64, 64), dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        sage_attention(x, x, x)


def test_qk_norm_buffers_and_backward_checks(lib):
    """With qk_norm the quantise call needs rq and rk; sage_qk_norm_bwd needs
    the flag and every pointer (rejected on the host, nothing launched)."""
    sh = _shape(qk_norm=1)
    qt = _qt(rq=None)
    assert lib.sage_quantize(ctypes.byref(sh), FAKE, FAKE, FAKE, ctypes.byref(qt), FAKE, None) == bd.SAGE_EINVAL
    full = _qt()
    plain = _shape()
    assert lib.sage_qk_norm_bwd(ctypes.byref(plain), FAKE, FAKE, ctypes.byref(full), FAKE, FAKE, None) == bd.SAGE_EINVAL
    assert lib.sage_qk_norm_bwd(ctypes.byref(sh), FAKE, FAKE, ctypes.byref(_qt(rk=None)), FAKE, FAKE,
                                None) == bd.SAGE_EINVAL
    assert lib.sage_qk_norm_bwd(ctypes.byref(sh), FAKE, FAKE, ctypes.byref(full), None, FAKE, None) == bd.SAGE_EINVAL
    assert lib.sage_qk_norm_bwd(ctypes.byref(sh), FAKE, FAKE, None, FAKE, FAKE, None) == bd.SAGE_EINVAL
