"""The E4M3 matrix products of the variant (sage_shape.fp8), one wave through
the library's probe entry point: their operand layout, and how far their float
sums are from exact products (the reason the variant's parity bar differs
from the INT8 one).  The exact reference decodes the E4M3 bytes with torch and
multiplies in float64."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from bit_trainable_attention_block_amd import binding
    binding.load()


def _exact(a_bytes, b_bytes, kper):
    """C[m, n] = sum_k A[m, k] B[k, n] with lane l holding row/column l % 16 and
    contraction indices kper * (l // 16) + e; returned in the result-register
    order (lane l, register j = row 4 (l // 16) + j, column l % 16)."""
    dec = lambda x: torch.from_numpy(x.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    A, B = dec(a_bytes[:, :kper]), dec(b_bytes[:, :kper])
    Am = np.zeros((16, 4 * kper))
    Bm = np.zeros((4 * kper, 16))
    for l in range(64):
        Am[l % 16, kper * (l // 16):kper * (l // 16 + 1)] = A[l]
        Bm[kper * (l // 16):kper * (l // 16 + 1), l % 16] = B[l]
    C = Am @ Bm
    return np.array([[C[4 * (l // 16) + j, l % 16] for j in range(4)] for l in range(64)])


@pytest.mark.parametrize("scale", ["full_range", "unit"])
def test_fp8_products_layout_and_summation(scale):
    from bit_trainable_attention_block_amd import binding as bd
    from tests import gpu_parity_lib as gp
    rng = np.random.default_rng(91)
    if scale == "full_range":
        a = rng.integers(0, 256, (64, 32)).astype(np.uint8)
        b = rng.integers(0, 256, (64, 32)).astype(np.uint8)
        a[(a & 0x7F) == 0x7F] ^= 1      # no NaN encodings
        b[(b & 0x7F) == 0x7F] ^= 1
    else:
        vals = rng.standard_normal((2, 64, 32)) * 100   # codes of a typical block
        enc = torch.from_numpy(vals.astype(np.float32)).clamp(-448, 448).to(torch.float8_e4m3fn)
        a, b = enc.view(torch.uint8).numpy()
    da, db = (torch.from_numpy(x.view(np.int8)).cuda() for x in (a, b))
    c32 = torch.empty((64, 4), dtype=torch.float32, device="cuda")
    c128 = torch.empty_like(c32)
    gp.say(f"[gpu] fp8 products probe {scale}")
    bd.probe_fp8_products(da, db, c32, c128)
    torch.cuda.synchronize()
    for got, kper in ((c32.cpu().numpy(), 8), (c128.cpu().numpy(), 32)):
        ref = _exact(a, b, kper)
        # the largest product bounds the summation error the instruction makes
        dec = lambda x: torch.from_numpy(x.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
        pmax = np.max(np.abs(dec(a[:, :kper]))) * np.max(np.abs(dec(b[:, :kper])))
        err = np.max(np.abs(got - ref)) / pmax
        gp.CURRENT_CASE[0] = f"fp8_products_{scale}"
        gp.record(f"k{4 * kper}", {"max_err_over_max_product": float(err)})
        # layout right (a wrong pairing errs by O(1) of the result), summation
        # within 2^-12 of the largest product
        assert err < 2.0 ** -12, (kper, err)
