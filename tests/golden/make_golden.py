"""Write tests/golden/adamw_small.json: small fixed inputs and the oracle's outputs.

Run from the repository root:  python tests/golden/make_golden.py
It calls only oracle/ (plus numpy for the inputs).  The fixture is a
regression guard: if the oracle's arithmetic ever changes, the tests that
replay this file fail and the change has to be justified from the pages.

Content: three tensors of 5, 8 and 13 elements (ragged), one AdamW step at
t = 3 with the workloads' hyperparameters and the delta on, then a second
case with an fp32 accumulated gradient built from 3 bf16 micro-batches.
Special values are planted: +-0 weights, a zero gradient, a bf16 subnormal
gradient, a weight whose update lands on a bf16 rounding tie region.
"""
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)
import oracle  # noqa: E402

HP = dict(lr=1e-4, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01)
OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "adamw_small.json")


def hexes(a):
    a = np.ascontiguousarray(a)
    if a.dtype == np.float32:
        return [f"{x:08x}" for x in a.view(np.uint32).tolist()]
    return [f"{x:04x}" for x in a.astype(np.uint16).tolist()]


def main():
    rng = np.random.default_rng(20261202)
    sizes = [5, 8, 13]
    n = sum(sizes)
    master = (rng.standard_normal(n) * 0.02).astype(np.float32)
    m = (rng.standard_normal(n) * 1e-4).astype(np.float32)
    v = np.square((rng.standard_normal(n) * 1e-3).astype(np.float32))
    grad = oracle.rne16((rng.standard_normal(n) * 1e-3).astype(np.float32))
    master[0], master[1] = 0.0, -0.0
    grad[2] = 0x0000            # zero gradient
    grad[3] = 0x0001            # bf16 subnormal gradient
    m[4], v[4] = 0.0, 0.0       # fresh-state element
    orig = oracle.rne16(master)
    micro = [oracle.rne16((rng.standard_normal(n) * 1e-3).astype(np.float32)) for _ in range(3)]

    cases = []
    t = 3
    c = oracle.adamw_constants(HP["lr"], HP["beta1"], HP["beta2"], HP["eps"], HP["weight_decay"], t)
    w2, m2, v2 = master.copy(), m.copy(), v.copy()
    wb, delta = oracle.adamw_step(w2, m2, v2, grad, c, orig=orig)
    cases.append(dict(name="bf16_grad_delta", step=t, grad_dtype="bf16",
                      inputs=dict(master=hexes(master), m=hexes(m), v=hexes(v),
                                  grad=hexes(grad), orig=hexes(orig)),
                      expect=dict(master=hexes(w2), m=hexes(m2), v=hexes(v2),
                                  weight=hexes(wb), delta=hexes(delta))))

    acc = np.empty(n, np.float32)
    oracle.grad_accum(acc, micro[0], overwrite=True)
    for g in micro[1:]:
        oracle.grad_accum(acc, g, overwrite=False)
    t = 7
    c = oracle.adamw_constants(HP["lr"], HP["beta1"], HP["beta2"], HP["eps"], HP["weight_decay"], t)
    w3, m3, v3 = master.copy(), m.copy(), v.copy()
    wb3, _ = oracle.adamw_step(w3, m3, v3, acc, c)
    cases.append(dict(name="fp32_accumulated_grad", step=t, grad_dtype="fp32",
                      inputs=dict(master=hexes(master), m=hexes(m), v=hexes(v),
                                  micro_batches=[hexes(g) for g in micro]),
                      expect=dict(acc=hexes(acc), master=hexes(w3), m=hexes(m3),
                                  v=hexes(v3), weight=hexes(wb3))))

    doc = dict(written_by="tests/golden/make_golden.py (calls only oracle/)",
               hyperparameters=HP, segment_sizes=sizes, cases=cases)
    with open(OUT, "w") as f:
        json.dump(doc, f, indent=1)
    print("wrote", OUT)


if __name__ == "__main__":
    main()
