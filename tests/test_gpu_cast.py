"""sage_cast_grads through the C ABI: float32 gradients to the 16-bit I/O
dtype, round to nearest with ties to even, checked bit for bit against
torch's CPU bfloat16 conversion and numpy's float16 conversion (each an
implementation of IEEE round-to-nearest-even of its own), on values that
include exact ties, the largest finite values, fp16 overflow, subnormals,
signed zeros, infinities and NaN."""
import numpy as np
import pytest

from bit_trainable_attention_block_amd import binding as bd
from bit_trainable_attention_block_amd import workloads as wl

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    bd.load()


def _values(n, seed):
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal(n) * np.exp2(rng.integers(-30, 30, n))).astype(np.float32)
    bits = x.view(np.uint32)
    # every 8th value an exact bf16 tie (low 16 bits 0x8000), both parities
    bits[::8] = (bits[::8] & 0xFFFF0000) | 0x8000
    # fp16 ties: 13 low mantissa bits at half an fp16 ulp for normal fp16 range values
    y = (rng.uniform(1, 2, n // 8) * np.exp2(rng.integers(-14, 15, n // 8))).astype(np.float32)
    yb = y.view(np.uint32)
    yb[:] = (yb & ~np.uint32(0x1FFF)) | 0x1000
    x[1::8] = y
    specials = np.array([0.0, -0.0, np.inf, -np.inf, np.nan, 65504.0, 65520.0, 70000.0, -1e9, 3.4e38,
                         np.float32(np.finfo(np.float32).tiny), 1e-40, -1e-45, 6e-8, 3e-8, 1.0 + 2**-8,
                         1.0 + 3 * 2**-8, 2**-24, 2**-25],
                        dtype=np.float32)
    x[2:2 + len(specials)] = specials
    return x


@pytest.mark.parametrize("dtype", [wl.BF16, wl.FP16], ids=["bf16", "fp16"])
def test_cast_is_round_to_nearest_even(dtype):
    import torch
    cfg = wl.Config("cast", 0, 1, 2, 128, 64, dtype, 128, 64, causal=False)
    sh = bd.Shape.of(cfg)
    n = cfg.B * cfg.H * cfg.N * cfg.D
    src = [_values(n, s).reshape(cfg.B, cfg.H, cfg.N, cfg.D) for s in (1, 2, 3)]
    dev = [torch.from_numpy(a).cuda() for a in src]
    out = bd.cast_grads(sh, *dev)
    torch.cuda.synchronize()
    for a, o in zip(src, out):
        got = o.view(torch.int16).cpu().numpy().view(np.uint16)
        if dtype == wl.BF16:
            want = torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
            nan_got = (got & 0x7F80) == 0x7F80
            nan_got &= (got & 0x007F) != 0
        else:
            with np.errstate(over="ignore"):   # fp16 overflow to infinity is one of the cases
                want = a.astype(np.float16).view(np.uint16)
            nan_got = ((got & 0x7C00) == 0x7C00) & ((got & 0x03FF) != 0)
        nan = np.isnan(a)
        assert np.all(nan_got == nan)
        np.testing.assert_array_equal(got[~nan], want[~nan])


def test_cast_subset_and_repeat():
    """Only dV given: dQ16, dK16 stay None; two calls give the same bits."""
    import torch
    cfg = wl.Config("cast", 0, 2, 1, 64, 128, wl.BF16, 64, 64, causal=False)
    sh = bd.Shape.of(cfg)
    a = _values(cfg.B * cfg.H * cfg.N * cfg.D, 7).reshape(cfg.B, cfg.H, cfg.N, cfg.D)
    dv = torch.from_numpy(a).cuda()
    q, k, v1 = bd.cast_grads(sh, None, None, dv)
    _, _, v2 = bd.cast_grads(sh, None, None, dv)
    torch.cuda.synchronize()
    assert q is None and k is None
    assert torch.equal(v1.view(torch.int16), v2.view(torch.int16))
