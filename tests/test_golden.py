"""The hand-worked routing / capacity / layout example in tests/golden/ (derived by hand
from the capacity rule and the prefix-sum layout; weights in closed form)."""
import json
import os

import numpy as np

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "capacity_handworked.json")


def test_handworked_example():
    g = json.load(open(GOLDEN))
    l = np.array(g["logits"], np.float32)
    ids, w = oracle.route(l, g["k"])
    assert ids.tolist() == g["topk_ids"]
    ref = np.array(g["topk_w"])
    assert (np.abs(w - ref) / ref).max() <= (g["k"] + 4) * 2.0 ** -24
    for case in g["cases"]:
        keep = oracle.capacity(ids, w, g["E"], case["C"])
        assert keep.tolist() == case["keep"], case["C"]
        lay = oracle.layout(ids, keep, g["E"])
        assert lay["counts"].tolist() == case["counts"]
        assert lay["offsets"].tolist() == case["offsets"]
        assert lay["row_token"][:lay["N"]].tolist() == case["row_token"]
        assert lay["slot_to_row"].tolist() == case["slot_to_row"]
