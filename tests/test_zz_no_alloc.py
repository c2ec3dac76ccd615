"""sage_quantize_noalloc: sage_quantize with the library's own fixed device
scratch in place of the caller's workspace (for callers that cannot
allocate).  Its outputs must equal sage_quantize's bit for bit, also on a
second call right after the first with a smaller problem (the scratch keeps
the previous call's contents), and problems beyond the scratch are refused on
the host."""
import ctypes

import numpy as np
import pytest

from bit_trainable_attention_block_amd import binding as bd
from bit_trainable_attention_block_amd import workloads as wl

FAKE = 0x10000  # aligned, never dereferenced: the call fails validation first


def test_problem_beyond_the_scratch_is_refused_on_the_host():
    import os
    if not os.path.exists(bd.LIB_PATH):
        pytest.skip("libsage.so not built")
    lib = bd.load()
    # 64 heads of N = 32768, d = 128: 64 * 512 * 128 * 8 B = 32 MiB of K-mean partial sums
    big = bd.c_shape(B=1, H=64, N=32768, D=128, bq=128, bkv=64, dtype=1, causal=1, k_smooth=1, q_smooth=0,
                     sm_scale=0.0, dp_int8=0, p_static=0, qk_norm=0, fp8=0)
    assert lib.sage_quantize_workspace_bytes(ctypes.byref(big)) > bd.NOALLOC_SCRATCH_BYTES
    qt = bd.c_qtensors(**{f: FAKE for f in bd.QT_FIELDS})
    assert lib.sage_quantize_noalloc(ctypes.byref(big), FAKE, FAKE, FAKE, ctypes.byref(qt), None) == bd.SAGE_ESCRATCH
    # without K-smoothing nothing goes through the scratch, so there is no limit
    big.k_smooth = 0
    assert lib.sage_quantize_noalloc(ctypes.byref(big), FAKE, FAKE, FAKE, None, None) == bd.SAGE_EINVAL
    assert lib.sage_status_str(bd.SAGE_ESCRATCH).decode().startswith("problem too large")


CASES = [
    # the first call fills more of the scratch than the second
    wl.Config("noalloc_a", 21, 2, 4, 2048, 128, wl.BF16, 128, 64, causal=True, k_offset_sigma=2.0,
              qk_norm_fused=True),
    wl.Config("noalloc_b", 22, 1, 2, 512, 64, wl.FP16, 64, 64, causal=False, q_smooth=True, k_offset_sigma=1.0),
]


@pytest.mark.gpu
def test_noalloc_matches_the_workspace_call_twice_in_a_row():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    bd.load()
    for cfg in CASES:
        print(f"[gpu] noalloc {cfg.name} B={cfg.B} H={cfg.H} N={cfg.N} D={cfg.D}", flush=True)
        sh = bd.Shape.of(cfg)
        x = wl.generate(cfg)
        Q, K, V = (torch.from_numpy(x[n]["bits"].view(np.int16)).to("cuda").view(sh.torch_dtype)
                   for n in ("q", "k", "v"))
        ref = bd.quantize(sh, Q, K, V)
        got = bd.alloc_qtensors(sh)
        for t in got.values():
            if t is not None:
                t.fill_(-7 if t.dtype != torch.float32 else float("nan"))   # no stale match by accident
        bd.quantize_noalloc(sh, Q, K, V, out=got)
        torch.cuda.synchronize()
        for name, t in ref.items():
            if t is None or name == "ws":
                continue
            a = t.cpu().numpy()
            b = got[name].cpu().numpy()
            assert a.dtype == b.dtype and np.array_equal(a.view(np.uint8), b.view(np.uint8)), (cfg.name, name)
