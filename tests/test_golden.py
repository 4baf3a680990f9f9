"""Replay of tests/golden/adamw_small.json against the oracle (regression guard)."""
import json
import os

import numpy as np

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "adamw_small.json")


def arr(hexes):
    if hexes and len(hexes[0]) == 8:
        return np.array([int(h, 16) for h in hexes], np.uint32).view(np.float32)
    return np.array([int(h, 16) for h in hexes], np.uint16)


def load():
    return json.load(open(GOLDEN))


def test_oracle_reproduces_golden():
    doc = load()
    hp = doc["hyperparameters"]
    for case in doc["cases"]:
        c = oracle.adamw_constants(hp["lr"], hp["beta1"], hp["beta2"], hp["eps"],
                                   hp["weight_decay"], case["step"])
        ins, exp = case["inputs"], case["expect"]
        master, m, v = arr(ins["master"]).copy(), arr(ins["m"]).copy(), arr(ins["v"]).copy()
        if case["grad_dtype"] == "bf16":
            grad = arr(ins["grad"])
            orig = arr(ins["orig"])
        else:
            micro = [arr(x) for x in ins["micro_batches"]]
            grad = np.empty(len(master), np.float32)
            oracle.grad_accum(grad, micro[0], overwrite=True)
            for g in micro[1:]:
                oracle.grad_accum(grad, g, overwrite=False)
            assert np.array_equal(grad.view(np.uint32), arr(exp["acc"]).view(np.uint32))
            orig = None
        wb, delta = oracle.adamw_step(master, m, v, grad, c, orig=orig)
        for name, got in (("master", master), ("m", m), ("v", v)):
            assert np.array_equal(got.view(np.uint32), arr(exp[name]).view(np.uint32)), name
        assert np.array_equal(wb, arr(exp["weight"]))
        if delta is not None:
            assert np.array_equal(delta.view(np.uint32), arr(exp["delta"]).view(np.uint32))
