"""GPU path against the CPU oracle, through the C ABI.

Small problems compare the whole chain element by element; the five
workload configurations run at full size, in the launch configuration the
benchmark times, and are checked on sampled heads and blocks the oracle
computes one by one (codes and scales of those heads bit for bit).
"""
import numpy as np
import pytest

from bit_trainable_attention_block_amd import workloads as wl
from tests import gpu_parity_lib as gp

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from bit_trainable_attention_block_amd import binding
    binding.load()


def small(name, N, D, bq, causal, dtype=wl.BF16, k_smooth=True, q_smooth=False, B=1, H=2, sigma=1.0, index=9,
          k_offset=1.5):
    return wl.Config(name, index, B, H, N, D, dtype, bq, 64, causal=causal, k_smooth=k_smooth,
                     q_smooth=q_smooth, sigma=sigma, qk_norm=False, k_offset_sigma=k_offset)


SMALL = [
    wl.C1,
    wl.C1.replace(name="tiny_causal", causal=True),
    small("n192_d64_bq64_causal", 192, 64, 64, True),            # ragged against the backward's 128-key workgroup
    # a single 64-token block: one forward tile, one key block of two
    small("n64_d64_bq64_causal", 64, 64, 64, True),
    small("n64_d128_bq64", 64, 128, 64, False, q_smooth=True),
    small("n320_d128_bq64_causal_qsmooth", 320, 128, 64, True, q_smooth=True),
    # K-smoothing off is only well conditioned without a common K offset: with
    # one, dQ cancels K's mean and a single dS code rounded the other way at a
    # .5 boundary moves dQ by ~1e-3 (the method keeps K-smoothing on for this).
    small("n384_d128_nosmooth", 384, 128, 128, False, k_smooth=False, k_offset=0.0),
    small("n256_d64_fp16_causal", 256, 64, 128, True, dtype=wl.FP16),
    small("n320_d128_fp16_bq64_causal", 320, 128, 64, True, dtype=wl.FP16),
    small("n256_d128_fp16_qsmooth_b2h3", 256, 128, 128, False, dtype=wl.FP16, q_smooth=True, B=2, H=3),
    small("n256_d128_qsmooth", 256, 128, 128, False, q_smooth=True, sigma=3.0),
    small("n512_d128_causal_b2", 512, 128, 128, True, B=2, H=1),
    # the INT8-dP ablation: ragged, bq=64 with d=64, Q-smoothing, fp16
    small("n192_d64_bq64_causal_dpint8", 192, 64, 64, True).replace(dp_int8=True),
    small("n384_d128_dpint8", 384, 128, 128, False).replace(dp_int8=True),
    small("n320_d128_bq64_causal_qsmooth_dpint8", 320, 128, 64, True, q_smooth=True).replace(dp_int8=True),
    small("n256_d64_fp16_dpint8", 256, 64, 128, False, dtype=wl.FP16).replace(dp_int8=True),
    # the static-P ablation
    small("n320_d128_bq64_causal_pstatic", 320, 128, 64, True).replace(p_static=True),
    small("n256_d64_qsmooth_pstatic", 256, 64, 128, False, q_smooth=True, sigma=2.0).replace(p_static=True),
    # QK-norm fused into sage_quantize, and the gradient through it
    small("n256_d128_causal_qknorm", 256, 128, 128, True, sigma=3.0).replace(qk_norm_fused=True),
    small("n192_d64_bq64_qsmooth_qknorm", 192, 64, 64, False, q_smooth=True, sigma=2.0).replace(qk_norm_fused=True),
    small("n256_d64_fp16_causal_qknorm", 256, 64, 128, True, dtype=wl.FP16).replace(qk_norm_fused=True),
    # the E4M3 variant: d=128 (16x16x128 products) and d=64, bq 64 and 128,
    # ragged, Q-smoothing, fp16, QK-norm
    wl.C1.replace(name="tiny_fp8", fp8=True),
    small("n256_d128_causal_fp8", 256, 128, 128, True).replace(fp8=True),
    small("n192_d64_bq64_fp8", 192, 64, 64, False).replace(fp8=True),
    small("n256_d128_fp16_causal_fp8", 256, 128, 128, True, dtype=wl.FP16).replace(fp8=True),
    small("n320_d128_bq64_causal_qsmooth_fp8", 320, 128, 64, True, q_smooth=True).replace(fp8=True),
    small("n256_d64_fp16_causal_qknorm_fp8", 256, 64, 128, True, dtype=wl.FP16).replace(fp8=True,
                                                                                        qk_norm_fused=True),
]


@pytest.mark.parametrize("cfg", SMALL, ids=lambda c: c.name)
def test_small_full_chain(cfg):
    gp.say(f"[gpu] small full chain {cfg.name} N={cfg.N} D={cfg.D} bq={cfg.bq} causal={cfg.causal}")
    gp.CURRENT_CASE[0] = cfg.name
    x = wl.generate(cfg)
    g = gp.run_gpu(cfg, x)
    try:
        gp.check_full_chain(cfg, x, g)
        for b in range(cfg.B):
            for h in range(cfg.H):
                gp.check_bwd_pre(cfg, x, g, b, h)
    except AssertionError:
        gp.dump(cfg.name, g)
        raise


def test_degenerate_zero_blocks():
    """Q = 0 (uniform attention), a V block and a dO block of zeros: scale 0 and
    zero codes on those blocks; dS = 0 where dO is 0."""
    cfg = small("zeros", 256, 64, 64, False, H=1)
    x = wl.generate(cfg)
    for name in ("q",):
        x[name]["bits"][:] = 0
        x[name]["f32"][:] = 0
    x["v"]["bits"][0, 0, 64:128] = 0
    x["v"]["f32"][0, 0, 64:128] = 0
    x["do"]["bits"][0, 0, 0:64] = 0
    x["do"]["f32"][0, 0, 0:64] = 0
    gp.say("[gpu] degenerate zero blocks")
    g = gp.run_gpu(cfg, x)
    assert g["qt"]["sv"][0, 0, 1] == 0 and g["dot"]["sdo"][0, 0, 0] == 0
    assert np.all(g["qt"]["sq"] == 0)
    gp.check_full_chain(cfg, x, g)


def test_largest_head_count():
    """B*H = 65535, the most heads the library takes (the quantisation grids
    put the heads on their second dimension): small causal heads (N = 64,
    d = 64), so every launch runs at its largest grid.  The first, a middle and
    the last head against the oracle, and every output finite."""
    cfg = small("heads65535_n64_d64_bq64_causal", 64, 64, 64, True, B=5, H=13107)
    assert cfg.B * cfg.H == 65535
    gp.say(f"[gpu] largest head count B={cfg.B} H={cfg.H} N={cfg.N} D={cfg.D} (input generation takes ~30 s)")
    gp.CURRENT_CASE[0] = cfg.name
    x = wl.generate(cfg)
    g = gp.run_gpu(cfg, x)
    for b, h in ((0, 0), (2, 6553), (4, 13106)):
        qz = gp.check_quantize(cfg, x, g, b, h)
        gp.check_fwd(cfg, x, g, b, h, qz, [0])
        gp.check_bwd(cfg, x, g, b, h, qz, [0], [0])
    for k in ("O", "L", "dQ", "dK", "dV"):
        assert np.all(np.isfinite(g[k])), k


FULL = [
    (wl.C2, [(0, 0), (3, 15)]),
    (wl.C2_CAUSAL, [(1, 7)]),
    (wl.C3, [(0, 0), (1, 15)]),
    (wl.C4[0], [(0, 3)]),
    (wl.C4[1], [(0, 12)]),
    (wl.C4[2], [(0, 17)]),
    (wl.C4[3], [(0, 24)]),
    (wl.C4[4], [(0, 31)]),
    (wl.C5, [(0, 0), (0, 7)]),
    (wl.C5_QSMOOTH, [(0, 5)]),
    (wl.C3_DPINT8, [(1, 3)]),
    (wl.C3_PSTATIC, [(0, 9)]),
    (wl.C3_QKNORM_FUSED, [(1, 11)]),
    (wl.C3_FP8, [(0, 2)]),
]


@pytest.mark.parametrize("cfg,heads", FULL, ids=lambda v: v.name if hasattr(v, "name") else "")
def test_full_size_sampled(cfg, heads):
    gp.say(f"[gpu] full size {cfg.name} B={cfg.B} H={cfg.H} N={cfg.N} D={cfg.D} causal={cfg.causal} "
           f"q_smooth={cfg.q_smooth}")
    gp.CURRENT_CASE[0] = cfg.name
    x = wl.generate(cfg)
    g = gp.run_gpu(cfg, x)
    Tm, Tn = cfg.N // cfg.bq, cfg.N // cfg.bkv
    q_blocks = sorted({0, Tm // 2, Tm - 1})
    kv_blocks = sorted({0, Tn // 3, Tn - 1})
    for k, (b, h) in enumerate(heads):
        qz = gp.check_quantize(cfg, x, g, b, h)
        O = gp.check_fwd(cfg, x, g, b, h, qz, q_blocks)
        dQ, dK, dV = gp.check_bwd(cfg, x, g, b, h, qz, kv_blocks, q_blocks)
        if k == 0:
            gp.report_vs_fpa(cfg, x, g, b, h, q_blocks, kv_blocks, {"O": O, "dQ": dQ, "dK": dK, "dV": dV})
    # every head: all block scales, the means and the codes of the first Q, K
    # and V blocks bit-exact (cheap), and finite outputs
    for b in range(cfg.B):
        for h in range(cfg.H):
            gp.check_head_codes(cfg, x, g, b, h)
    for k in ("O", "L", "dQ", "dK", "dV"):
        assert np.all(np.isfinite(g[k])), k


@pytest.mark.parametrize("ks,qs", [(False, False), (True, False), (True, True)], ids=["none", "k", "qk"])
def test_smoothing_variants_on_offset_heads(ks, qs):
    """The three smoothing settings on one head whose Q and K carry channel
    offsets shared by all tokens: parity with the oracle on every block, and
    both sides' accuracy against full-precision attention recorded (the
    report prints them side by side)."""
    name = {(False, False): "smoothing_none", (True, False): "smoothing_k", (True, True): "smoothing_qk"}[(ks, qs)]
    cfg = wl.Config(name, 11, 1, 1, 1024, 128, wl.BF16, 128, 64, causal=False, k_smooth=ks, q_smooth=qs,
                    k_offset_sigma=4.0, q_offset_sigma=3.0)
    gp.say(f"[gpu] smoothing variant {name}")
    gp.CURRENT_CASE[0] = name
    x = wl.generate(cfg)
    g = gp.run_gpu(cfg, x)
    allq, allk = list(range(cfg.N // cfg.bq)), list(range(cfg.N // cfg.bkv))
    qz = gp.check_quantize(cfg, x, g, 0, 0)
    O = gp.check_fwd(cfg, x, g, 0, 0, qz, allq)
    dQ, dK, dV = gp.check_bwd(cfg, x, g, 0, 0, qz, allk, allq)
    gp.report_vs_fpa(cfg, x, g, 0, 0, allq, allk, {"O": O, "dQ": dQ, "dK": dK, "dV": dV})


@pytest.mark.parametrize("causal,qk_norm,fp8", [(False, False, False), (True, False, False), (True, True, False),
                                                (True, False, True)])
def test_autograd_wrapper_matches_the_oracle(causal, qk_norm, fp8):
    """sage_attention (a torch.autograd.Function over the four calls): O and
    the gradients it returns through autograd against the oracle's chain, and
    identical to calling the four entry points directly."""
    import torch

    from bit_trainable_attention_block_amd.autograd import sage_attention
    from oracle import sage as osage
    cfg = small("autograd", 256, 128, 128, causal, H=2, sigma=2.0).replace(qk_norm_fused=qk_norm, fp8=fp8)
    gp.say(f"[gpu] autograd wrapper causal={causal} qk_norm={qk_norm} fp8={fp8}")
    gp.CURRENT_CASE[0] = f"autograd_causal{int(causal)}_qknorm{int(qk_norm)}_fp8{int(fp8)}"
    x = wl.generate(cfg)
    dev = gp.to_device(x)
    Q, K, V, dO = (dev[n].view(torch.bfloat16).clone() for n in ("q", "k", "v", "do"))
    for t in (Q, K, V):
        t.requires_grad_(True)
    O = sage_attention(Q, K, V, causal=causal, qk_norm=qk_norm, fp8=fp8)
    O.backward(dO)
    torch.cuda.synchronize()
    direct = gp.run_gpu(cfg, x)
    np.testing.assert_array_equal(O.detach().view(torch.int16).cpu().numpy().view(np.uint16), direct["O_bits"])
    grads = (("dQ_in", Q), ("dK_in", K), ("dV", V)) if qk_norm else (("dQ", Q), ("dK", K), ("dV", V))
    for name, t in grads:
        ref16 = torch.from_numpy(direct[name]).to(torch.bfloat16)
        np.testing.assert_array_equal(t.grad.cpu().view(torch.int16).numpy(), ref16.view(torch.int16).numpy())
    shp = osage.Shape.of(cfg)
    chain = gp.CHAIN_REL_L2_MAX * (2 if fp8 else 1)   # the E4M3 variant's looser bar (gpu_parity_lib)
    for h in range(cfg.H):
        r = osage.run_head(*gp.head_inputs(x, 0, h), shp)
        gp.close(f"O[0,{h}]", O.detach()[0, h].float().cpu().numpy(), r["O"], rel_max=chain)
        for name, t in grads:
            # bf16 gradients: the 16-bit rounding (2^-9 relative) bounds the
            # difference on top of the float32 chain bar
            gp.close(f"{name}[0,{h}]", t.grad[0, h].float().cpu().numpy(), r[name], rel_max=chain, cos_min=0.9999)
            # the RNE-cast gradients against the oracle's own RNE cast: the two
            # differ by one 16-bit ulp only where a float32 difference of ~1e-5
            # straddles a rounding boundary
            ref_rne = torch.from_numpy(np.ascontiguousarray(r[name], dtype=np.float32)).to(torch.bfloat16).float()
            gp.close(f"{name}_rne[0,{h}]", t.grad[0, h].float().cpu().numpy(), ref_rne.numpy().astype(np.float64),
                     rel_max=chain, cos_min=0.9999)


@pytest.mark.parametrize("fp8,qk_norm", [(False, False), (True, False), (False, True)])
def test_repeat_is_deterministic(fp8, qk_norm):
    """Two runs on the same inputs give identical codes, scales, means, O, L,
    dQ, dK and dV (no atomics anywhere: mu_K adds block sums in a fixed order,
    dQ is a separate pass with a fixed order).  With QK-norm fused, the K-mean
    summands are float32 rows spanning many binades, where a float64 sum in a
    varying order would round differently."""
    if qk_norm:
        cfg = wl.C3_QKNORM_FUSED.replace(B=1, H=4, N=4096)
    else:
        cfg = wl.C2_CAUSAL.replace(B=1, H=4, fp8=fp8)
    x = wl.generate(cfg)
    gp.say(f"[gpu] determinism fp8={fp8} qk_norm={qk_norm}")
    g1 = gp.run_gpu(cfg, x)
    g2 = gp.run_gpu(cfg, x)
    for k in ("q", "k", "vt", "sq", "sk", "sv", "mu_k") + (("rq", "rk") if qk_norm else ()):
        np.testing.assert_array_equal(g1["qt"][k], g2["qt"][k])
    for k in ("O_bits", "L", "dQ", "dK", "dV"):
        np.testing.assert_array_equal(g1[k], g2[k])
