"""The oracle on hand-derived worked examples (tests/golden/worked_examples.json).

Every expected value there is a closed form derived by hand from the passage
of the diffusion_gemma_sampler page that the entry cites.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle

HERE = os.path.dirname(__file__)
with open(os.path.join(HERE, "golden", "worked_examples.json")) as f:
    GOLDEN = json.load(f)

ENV = {"log": math.log, "exp": math.exp, "inf": math.inf}


def _row(vals):
    return np.array([[float(v) for v in vals]], np.float32)


def _bf16_value(bits):
    return float(np.array([int(bits) << 16], np.uint32).view(np.float32)[0])


@pytest.mark.parametrize("case", GOLDEN["rowstats"], ids=lambda c: c["name"])
def test_rowstats_worked_example(case):
    x = _row(case["logits"])
    out = oracle.rowstats(x, [0], [case["temp"]], 1, seed=42, probs_dtype=oracle.PROBS_BF16)
    assert out["argmax"][0] == case["argmax"]
    if "sample" in case:
        assert out["sample"][0] == case["sample"]
    assert out["entropy"][0] == pytest.approx(eval(case["entropy"], ENV), abs=1e-12)
    if "probs_value" in case:
        want = eval(case["probs_value"], ENV)
        assert all(_bf16_value(b) == want for b in out["probs"][0])
    for col, expr in case.get("probs_value_at", {}).items():
        assert _bf16_value(out["probs"][0, int(col)]) == eval(expr, ENV)


@pytest.mark.parametrize("case", GOLDEN["topk"], ids=lambda c: c["name"])
def test_topk_worked_example(case):
    x = _row(case["logits"])
    vals, idx = oracle.topk_logprobs(x, [0], [case["temp"]], 1, [1], case["K"])
    assert idx[0].tolist() == case["idx"]
    want = [eval(e, ENV) for e in case["logprobs"]]
    assert np.allclose(vals[0], want, rtol=1e-6, atol=1e-6)
