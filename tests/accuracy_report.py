"""Accuracy summary from the GPU parity run's metrics log (not a test module).

    python -m tests.accuracy_report $SAGE_PARITY_OUT/parity_metrics.jsonl > profiles/accuracy_d128_workloads.md

For every full-size workload: the GPU against the oracle (the parity gate),
and the GPU and the oracle each against full-precision float64 attention on
the same sampled rows (CosSim, Rel-L2, Rel-L1, RMSE).  The sigma sweep is
printed beside the SageBwd paper's Table 1 (its shapes are not stated, so
the absolute values are context, not a target).
"""
import json
import os
import sys
from collections import OrderedDict

HERE = os.path.dirname(os.path.abspath(__file__))
TENSORS = ("O", "dQ", "dK", "dV")


def load(path):
    rows = [json.loads(l) for l in open(path) if l.strip()]
    by_case = OrderedDict()
    for r in rows:
        by_case.setdefault(r["case"], []).append(r)
    return by_case


def table1():
    out = {}
    for line in open(os.path.join(HERE, "golden", "table1_sigma_sweep.txt")):
        if line.startswith("#") or not line.strip():
            continue
        v = line.split()
        out[int(v[0])] = {t: (float(v[1 + 2 * k]), float(v[2 + 2 * k])) for k, t in enumerate(TENSORS)}
    return out


def main(path):
    cases = load(path)
    print("| workload | tensor | GPU vs oracle rel-L2 (max) | GPU vs FPA cos | GPU vs FPA rel-L2 | GPU vs FPA rel-L1 "
          "| oracle vs FPA cos | oracle vs FPA rel-L2 |")
    print("|---|---|---|---|---|---|---|---|")
    sig = {}
    for case, rows in cases.items():
        if not any(r["tensor"].startswith("fpa_") for r in rows):
            continue
        for t in TENSORS:
            gate = [r["rel_l2"] for r in rows if r["tensor"].startswith(t + "[")]
            g = [r for r in rows if r["tensor"].startswith(f"fpa_gpu_{t}[")]
            o = [r for r in rows if r["tensor"].startswith(f"fpa_oracle_{t}[")]
            if not g:
                continue
            g, o = g[0], o[0]
            print(f"| {case} | {t} | {max(gate):.2e} | {g['cos']:.6f} | {g['rel_l2']:.4f} | {g['rel_l1']:.4f} "
                  f"| {o['cos']:.6f} | {o['rel_l2']:.4f} |")
            if case.startswith("sigma"):
                sig.setdefault(case, {})[t] = g
    if sig:
        t1 = table1()
        print()
        print("| sigma | tensor | GPU vs FPA cos | GPU vs FPA rel-L2 | Table 1 cos | Table 1 rel-L2 |")
        print("|---|---|---|---|---|---|")
        for case, d in sig.items():
            s = int(case[len("sigma"):].split("_")[0])
            for t in TENSORS:
                if t in d:
                    c, r = t1.get(s, {}).get(t, (float("nan"), float("nan")))
                    print(f"| {s} | {t} | {d[t]['cos']:.4f} | {d[t]['rel_l2']:.4f} | {c:.4f} | {r:.4f} |")
    fp8_products(cases)


def fp8_products(cases):
    """The E4M3 product probe: summation error over the largest product."""
    rows = [(c, r) for c, rs in cases.items() if c.startswith("fp8_products_") for r in rs]
    if not rows:
        return
    print()
    print("| E4M3 product probe operands | instruction | max error / largest product |")
    print("|---|---|---|")
    for c, r in rows:
        inst = {"k32": "v_mfma_f32_16x16x32_fp8_fp8", "k128": "v_mfma_f32_16x16x128_f8f6f4"}.get(r["tensor"],
                                                                                             r["tensor"])
        print(f"| {c[len('fp8_products_'):]} | {inst} | {r['max_err_over_max_product']:.2e} |")


if __name__ == "__main__":
    main(sys.argv[1])
