"""The synthetic workloads carry the shapes the pages state (tests/golden/page_shapes.json)
and the routing statistics their descriptions call for."""

import json
import os

import numpy as np

from synth import WORKLOADS, make_routing, routing_stats

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_shapes.json")))


def test_shapes_from_pages():
    assert WORKLOADS["decode7"].E == GOLD["routed_experts"]["value"]
    assert WORKLOADS["prefill32k"].E == GOLD["routed_experts"]["value"]
    assert WORKLOADS["decode7"].T == GOLD["verify_tokens"]["value"]
    assert WORKLOADS["prefill32k"].T == GOLD["prefill_chunk_tokens"]["value"]
    tp = WORKLOADS["tp8rank32k"]
    assert tp.full_I == tp.I * GOLD["moe_tp_degree"]["value"]


def test_routing_is_topk_distinct_and_normalised():
    for name in ["tiny", "decode7", "decode256"]:
        w = WORKLOADS[name]
        ids, wts = make_routing(w)
        assert ids.shape == (w.T, w.K) and ids.dtype == np.int32
        assert all(len(set(r)) == w.K for r in ids.tolist())
        assert np.all((ids >= 0) & (ids < w.E))
        np.testing.assert_allclose(wts.sum(1), 1.0, rtol=1e-6)


def test_routing_is_seeded_and_skewed():
    a, _ = make_routing(WORKLOADS["decode256"])
    b, _ = make_routing(WORKLOADS["decode256"])
    assert np.array_equal(a, b)
    st = routing_stats(a, 384)
    # per-request affinity concentrates picks: far fewer than 384 experts' worth of spread
    assert 250 < st["distinct"] < 384 and st["max"] > 50
