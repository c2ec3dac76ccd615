"""Helpers of the GPU parity tests: run the HIP path through the C ABI and the
oracle on the same seeded inputs, and compare.  Imported only by tests."""
from __future__ import annotations

import json
import os
import tempfile

import numpy as np
import torch

from bit_trainable_attention_block_amd import binding as bd
from bit_trainable_attention_block_amd import workloads as wl
from oracle import fpa, metrics, sage

# Floating-point bar for O, dQ, dK, dV against the oracle.
REL_L2_MAX = 1e-3
COS_MIN = 0.99999
# The E4M3 variant's relative-L2 bar.  Its matrix instruction does not sum
# exactly: on random E4M3 operands it is off by up to ~1.3e-4 of the largest
# product (tests/test_gpu_fp8_products.py), where the INT8 one is exact.  The logits then differ
# from the oracle's exact sums by ~1e-4 relative, and an E4M3 code whose exact
# quotient lies that close to a rounding midpoint moves by one step, 1/8 of
# its value (an INT8 step is 1/127 of the block maximum).  Each such move
# shifts its output row by up to ~1%; they are rare, so they show in the
# relative L2 (measured up to 2.2e-3) and barely in the cosine, which keeps
# the method's bar.
FP8_REL_L2_MAX = 5e-3


def bar(cfg):
    """(relative-L2 maximum, cosine minimum) of one call's outputs."""
    return (FP8_REL_L2_MAX if getattr(cfg, "fp8", False) else REL_L2_MAX), COS_MIN


# Local bars beside the tensor-wide ones, so that one bad row or lane cannot
# hide under a norm taken over the whole tensor.  Rows are query rows (O, dQ)
# or key rows (dK, dV).  A row's error is ||x_r - ref_r|| over the larger of
# ||ref_r|| and the RMS row norm of the reference (a key that hardly any query
# attends has a tiny dV row, where a single legitimate code difference is a
# large relative change); an element's error is |x - ref| over the larger of
# its row's RMS and the tensor's RMS.  An element of at least half its row's
# RMS that is off by 10% breaks the element bar; a row off by 1% of its norm
# breaks the row bar.  The E4M3 variant's codes move in steps of 1/8 of their value, hence
# its looser local bars.
ROW_REL_MAX = 1e-2
ELEM_REL_MAX = 5e-2
FP8_ROW_REL_MAX = 4e-2
FP8_ELEM_REL_MAX = 2e-1


def local_bar(cfg):
    """(row maximum, element maximum) of one call's outputs."""
    if getattr(cfg, "fp8", False):
        return FP8_ROW_REL_MAX, FP8_ELEM_REL_MAX
    return ROW_REL_MAX, ELEM_REL_MAX


def local_errors(ours, ref):
    """(worst row error, worst element error) as defined above, for 2-D
    [rows, D] arrays."""
    a = np.asarray(ours, dtype=np.float64).reshape(-1, np.shape(ref)[-1])
    b = np.asarray(ref, dtype=np.float64).reshape(a.shape)
    diff = a - b
    row_norm = np.linalg.norm(b, axis=1)
    rms_row_norm = np.sqrt(np.mean(row_norm ** 2))
    if rms_row_norm == 0:
        return float(np.max(np.abs(diff), initial=0.0)), float(np.max(np.abs(diff), initial=0.0))
    row_err = np.linalg.norm(diff, axis=1) / np.maximum(row_norm, rms_row_norm)
    row_rms = row_norm / np.sqrt(b.shape[1])
    elem_scale = np.maximum(row_rms, rms_row_norm / np.sqrt(b.shape[1]))[:, None]
    elem_err = np.abs(diff) / elem_scale
    return float(row_err.max()), float(elem_err.max())


# where the metrics log and failing-case dumps go (set SAGE_PARITY_OUT to keep
# them with a run's other output)
OUT_DIR = os.environ.get("SAGE_PARITY_OUT", os.path.join(tempfile.gettempdir(), "sage_parity"))


def say(msg):
    print(msg, flush=True)


def record(name, m):
    """Append one comparison's metrics to a JSON-lines log (margins, not just pass/fail)."""
    try:
        os.makedirs(OUT_DIR, exist_ok=True)
        with open(os.path.join(OUT_DIR, "parity_metrics.jsonl"), "a") as f:
            f.write(json.dumps({"case": CURRENT_CASE[0], "tensor": name, **m}) + "\n")
    except OSError:
        pass


def dump(tag, g):
    """Save the GPU outputs of a failing case for offline analysis."""
    try:
        os.makedirs(OUT_DIR, exist_ok=True)
        flat = {k: v for k, v in g.items() if isinstance(v, np.ndarray)}
        for grp in ("qt", "dot"):
            for k, v in g.get(grp, {}).items():
                if v is not None:
                    flat[f"{grp}_{k}"] = v
        np.savez_compressed(os.path.join(OUT_DIR, f"fail_{tag}.npz"), **flat)
    except OSError:
        pass


CURRENT_CASE = [""]


def to_device(inputs):
    """uint16 bit patterns -> 16-bit torch tensors on cuda:0."""
    out = {}
    for k, v in inputs.items():
        t = torch.from_numpy(np.ascontiguousarray(v["bits"]).view(np.int16)).to("cuda")
        out[k] = t
    return out


def run_gpu(cfg, inputs):
    sh = bd.Shape.of(cfg)
    dev = to_device(inputs)
    dt = sh.torch_dtype
    Q, K, V, dO = (dev[n].view(dt) for n in ("q", "k", "v", "do"))
    res = bd.run(sh, Q, K, V, dO)
    torch.cuda.synchronize()
    host = {}
    for k in ("O", "L", "dQ", "dK", "dV", "dQ_in", "dK_in"):
        if k not in res:
            continue
        t = res[k]
        host[k] = (t.float() if t.dtype in (torch.bfloat16, torch.float16) else t).cpu().numpy()
    host["O_bits"] = res["O"].view(torch.int16).cpu().numpy().view(np.uint16)
    host["qt"] = {k: (v.cpu().numpy() if v is not None else None) for k, v in res["qt"].items()}
    host["dot"] = {k: (v.cpu().numpy() if v is not None else None) for k, v in res["dot"].items()}
    return host


def head_inputs(inputs, b, h):
    return [inputs[n]["f32"][b, h].astype(np.float64) for n in ("q", "k", "v", "do")]


def code_bytes(codes, fp8):
    """The bytes the GPU stores for the oracle's code values: INT8, or the
    E4M3 encodings (as int8, the dtype the layouts unpack to)."""
    return sage.e4m3_bits(codes).view(np.int8) if fp8 else codes.astype(np.int8)


def check_quantize(cfg, inputs, g, b, h):
    """Bit-exact codes, scales and means of one head."""
    shp = sage.Shape.of(cfg)
    Q, K, V, dO = head_inputs(inputs, b, h)
    qz = sage.quantize(Q, K, V, shp)
    N, D = cfg.N, cfg.D
    qt = g["qt"]
    un = lambda name, kind: bd.unpack_codes(qt[name][b, h], kind, N, D)
    f8 = shp.fp8
    np.testing.assert_array_equal(un("q", "R32"), code_bytes(qz.Qc, f8))
    np.testing.assert_array_equal(un("k", "R32"), code_bytes(qz.Kc, f8))
    np.testing.assert_array_equal(un("vt", "C64P"), code_bytes(qz.Vc, f8))
    np.testing.assert_array_equal(qt["sq"][b, h], qz.sQ.astype(np.float32))
    np.testing.assert_array_equal(qt["sk"][b, h], qz.sK.astype(np.float32))
    np.testing.assert_array_equal(qt["sv"][b, h], qz.sV.astype(np.float32))
    if cfg.dp_int8:
        # the ablation's second copy of V's codes, R32
        np.testing.assert_array_equal(un("vr", "R32"), qz.Vc.astype(np.int8))
    if getattr(cfg, "qk_norm_fused", False):
        np.testing.assert_array_equal(qt["rq"][b, h], qz.rq.astype(np.float32))
        np.testing.assert_array_equal(qt["rk"][b, h], qz.rk.astype(np.float32))
    if cfg.k_smooth:
        np.testing.assert_array_equal(qt["mu_k"][b, h], qz.mu_k.astype(np.float32))
    if cfg.q_smooth:
        np.testing.assert_array_equal(qt["mu_q"][b, h], qz.mu_q.astype(np.float32))
        bias = np.stack([sage.qsmooth_bias(qz, i, j, shp) for i in range(shp.Tm) for j in range(shp.Tn)])
        bias = bias.reshape(shp.Tm, shp.Tn, cfg.bkv).reshape(shp.Tm, cfg.N)
        got = qt["qk_bias"][b, h]
        if cfg.causal:
            # written for query blocks from the first one that sees the key's
            # 128-key pair on (include/sage.h)
            first = (np.arange(cfg.N) // 128 * 128) // cfg.bq
            keep = np.arange(shp.Tm)[:, None] >= first[None, :]
            got, bias = got[keep], bias[keep]
        np.testing.assert_allclose(got, bias, rtol=2e-6, atol=1e-6)
    return qz


def check_head_codes(cfg, inputs, g, b, h):
    """Cheap bit-exact check of every head at full size: all block scales of
    Q, K and V, mu_K (and mu_Q), and the codes of the first Q, K and V blocks,
    against the oracle's quantiser on the whole head."""
    shp = sage.Shape.of(cfg)
    Q, K, V, _ = head_inputs(inputs, b, h)
    qz = sage.quantize(Q, K, V, shp)
    qt = g["qt"]
    for name, ref in (("sq", qz.sQ), ("sk", qz.sK), ("sv", qz.sV)):
        np.testing.assert_array_equal(qt[name][b, h], ref.astype(np.float32), err_msg=f"{name}[{b},{h}]")
    if cfg.k_smooth:
        np.testing.assert_array_equal(qt["mu_k"][b, h], qz.mu_k.astype(np.float32))
    if cfg.q_smooth:
        np.testing.assert_array_equal(qt["mu_q"][b, h], qz.mu_q.astype(np.float32))
    N, D = cfg.N, cfg.D
    nq, nk = cfg.bq * D, cfg.bkv * D          # bytes of the first block in every layout
    first = lambda name, kind, n: bd.unpack_codes(qt[name][b, h][:n], kind, n // D, D)
    np.testing.assert_array_equal(first("q", "R32", nq), code_bytes(qz.Qc[:cfg.bq], shp.fp8))
    np.testing.assert_array_equal(first("k", "R32", nk), code_bytes(qz.Kc[:cfg.bkv], shp.fp8))
    np.testing.assert_array_equal(first("vt", "C64P", nk), code_bytes(qz.Vc[:cfg.bkv], shp.fp8))


def check_bwd_pre(cfg, inputs, g, b, h):
    """delta and dO codes of one head, from the GPU's own O."""
    shp = sage.Shape.of(cfg)
    _, _, _, dO = head_inputs(inputs, b, h)
    O = g["O"][b, h].astype(np.float64)
    delta, dOc, sdO = sage.backward_pre(O, dO, shp)
    dot = g["dot"]
    np.testing.assert_array_equal(bd.unpack_codes(dot["dot"][b, h], "C64P", cfg.N, cfg.D), code_bytes(dOc, shp.fp8))
    np.testing.assert_array_equal(dot["sdo"][b, h], sdO.astype(np.float32))
    np.testing.assert_allclose(dot["delta"][b, h], delta, rtol=1e-6, atol=1e-6)
    if cfg.dp_int8:
        # the ablation's second copy of dO's codes, R32
        np.testing.assert_array_equal(bd.unpack_codes(dot["dor"][b, h], "R32", cfg.N, cfg.D), dOc.astype(np.int8))
    return delta, dOc, sdO


def close(name, ours, ref, rel_max=REL_L2_MAX, cos_min=COS_MIN, log=None, local=None):
    """Tensor-wide bar (relative L2, cosine); with local = (row maximum,
    element maximum), the row and element bars too.  The worst row and
    element errors are always recorded."""
    m = metrics.all_metrics(ours, ref)
    m["row_max"], m["elem_max"] = local_errors(ours, ref)
    record(name, m)
    if log is not None:
        log.append((name, m))
    assert np.all(np.isfinite(ours)), name
    assert m["rel_l2"] <= rel_max and m["cos"] >= cos_min, f"{name}: {m}"
    if local is not None:
        assert m["row_max"] <= local[0] and m["elem_max"] <= local[1], f"{name} (row / element bar): {m}"
    return m


def check_fwd(cfg, inputs, g, b, h, qz, q_blocks, log=None):
    shp = sage.Shape.of(cfg)
    O, L = sage.forward(qz, shp, q_blocks=q_blocks)
    rows = np.concatenate([np.arange(i * cfg.bq, (i + 1) * cfg.bq) for i in q_blocks])
    rel, cmin = bar(cfg)
    close(f"O[{b},{h}]", g["O"][b, h][rows], O[rows], rel_max=rel, cos_min=cmin, log=log, local=local_bar(cfg))
    np.testing.assert_allclose(g["L"][b, h][rows], L[rows], rtol=2e-5, atol=2e-5)
    return O


def check_bwd(cfg, inputs, g, b, h, qz, kv_blocks, q_blocks, log=None):
    """dK, dV of kv_blocks and dQ of q_blocks, given the GPU's O, L."""
    shp = sage.Shape.of(cfg)
    _, _, V, dO = head_inputs(inputs, b, h)
    delta, dOc, sdO = check_bwd_pre(cfg, inputs, g, b, h)
    L = g["L"][b, h].astype(np.float64)
    delta_gpu = g["dot"]["delta"][b, h].astype(np.float64)
    dQ, dK, dV = sage.backward(qz, V, dO, dOc, sdO, L, delta_gpu, shp, kv_blocks=kv_blocks, q_blocks=q_blocks)
    kr = np.concatenate([np.arange(j * cfg.bkv, (j + 1) * cfg.bkv) for j in kv_blocks])
    qr = np.concatenate([np.arange(i * cfg.bq, (i + 1) * cfg.bq) for i in q_blocks])
    rel, cmin = bar(cfg)
    loc = local_bar(cfg)
    close(f"dK[{b},{h}]", g["dK"][b, h][kr], dK[kr], rel_max=rel, cos_min=cmin, log=log, local=loc)
    close(f"dV[{b},{h}]", g["dV"][b, h][kr], dV[kr], rel_max=rel, cos_min=cmin, log=log, local=loc)
    close(f"dQ[{b},{h}]", g["dQ"][b, h][qr], dQ[qr], rel_max=rel, cos_min=cmin, log=log, local=loc)
    return dQ, dK, dV


# Heads up to this length get dK, dV against full-precision attention too (the
# float64 N x N intermediates of a longer head are too large for the check).
FPA_FULL_MAX_N = 8192


def fpa_rows(Q, K, V, dO, scale, causal, rows):
    """Full-precision O and dQ of the given query rows only (float64; the
    textbook definitions of oracle/fpa.py restricted to those rows)."""
    S = (Q[rows] @ K.T) * scale
    if causal:
        S = np.where(np.arange(K.shape[0])[None, :] <= rows[:, None], S, -np.inf)
    m = S.max(axis=1, keepdims=True)
    E = np.exp(S - m)
    P = E / E.sum(axis=1, keepdims=True)
    O = P @ V
    dP = dO[rows] @ V.T
    delta = np.sum(dO[rows] * O, axis=1)
    dQ = scale * ((P * (dP - delta[:, None])) @ K)
    return O, dQ


def report_vs_fpa(cfg, inputs, g, b, h, q_blocks, kv_blocks, ours):
    """Accuracy against full-precision float64 attention on the sampled rows:
    the GPU's and the oracle's outputs, each compared with the same reference
    (recorded, not asserted: SageBwd approximates attention).  `ours` holds
    the oracle's O, dQ, dK, dV on those rows."""
    shp = sage.Shape.of(cfg)
    Q, K, V, dO = (a.astype(np.float64) for a in head_inputs(inputs, b, h))
    if shp.qk_norm:
        # the attention inputs are the normalised Q and K; dQ and dK are
        # gradients with respect to them
        Q, K = sage.rms_norm(Q, quant=False)[0], sage.rms_norm(K, quant=False)[0]
    qr = np.concatenate([np.arange(i * cfg.bq, (i + 1) * cfg.bq) for i in q_blocks])
    kr = np.concatenate([np.arange(j * cfg.bkv, (j + 1) * cfg.bkv) for j in kv_blocks])
    O_f, dQ_f = fpa_rows(Q, K, V, dO, shp.scale, cfg.causal, qr)
    pairs = [("O", g["O"][b, h][qr], ours["O"][qr], O_f), ("dQ", g["dQ"][b, h][qr], ours["dQ"][qr], dQ_f)]
    if cfg.N <= FPA_FULL_MAX_N:
        r = fpa.backward(Q, K, V, dO, shp.scale, cfg.causal)
        pairs += [("dK", g["dK"][b, h][kr], ours["dK"][kr], r["dK"][kr]),
                  ("dV", g["dV"][b, h][kr], ours["dV"][kr], r["dV"][kr])]
    for name, gpu, orc, ref in pairs:
        record(f"fpa_gpu_{name}[{b},{h}]", metrics.all_metrics(gpu, ref))
        record(f"fpa_oracle_{name}[{b},{h}]", metrics.all_metrics(orc, ref))


# End-to-end chain bar.  sage_bwd is judged on the O and L it is given (the
# GPU's own, above); the whole chain is checked against the oracle's own chain
# with a looser relative-L2 bar: O is stored rounded to 16 bits, and where
# the two sides' O land on different sides of a rounding boundary, delta =
# rowsum(dO o O) moves by up to one 16-bit ulp of O times dO, which shifts a
# whole row of dS and can move a tile's dS scale and codes (the SageBwd pages
# note that forward output error reaches the backward pass through delta).
# tests/test_oracle_chain_sensitivity.py measures it on the oracle alone: four
# such flips of O (rel-L2 5e-5) move its own chain's dQ and dK by 1.1e-3.
# The E4M3 variant takes twice it, for the reason given at FP8_REL_L2_MAX.
CHAIN_REL_L2_MAX = 5e-3


def check_full_chain(cfg, inputs, g, log=None):
    """Small problems: every call against the oracle on identical inputs
    (codes bit-exact; O, L; delta and dO codes from the GPU's O; dQ, dK, dV
    given the GPU's O and L), plus the whole chain against the oracle's chain."""
    shp = sage.Shape.of(cfg)
    allq = list(range(shp.Tm))
    allk = list(range(shp.Tn))
    for b in range(cfg.B):
        for h in range(cfg.H):
            Q, K, V, dO = head_inputs(inputs, b, h)
            qz = check_quantize(cfg, inputs, g, b, h)
            check_fwd(cfg, inputs, g, b, h, qz, allq, log=log)
            check_bwd(cfg, inputs, g, b, h, qz, allk, allq, log=log)
            r = sage.run_head(Q, K, V, dO, shp)
            names = ("O", "dQ", "dK", "dV") + (("dQ_in", "dK_in") if shp.qk_norm else ())
            for name in names:
                close(f"chain_{name}[{b},{h}]", g[name][b, h], r[name],
                      rel_max=CHAIN_REL_L2_MAX * (2 if getattr(cfg, "fp8", False) else 1), log=log)
