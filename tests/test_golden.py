"""Golden fixtures: the oracle still reproduces its stored tiny case, and the
page-shaped workloads agree with the figures the pages print (as context:
the pages state no hardware and no throughput)."""
import json
import os

import numpy as np

from oracle import tis_oracle as O
import workloads

HERE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _load(name):
    with open(os.path.join(HERE, name)) as f:
        return json.load(f)


def test_oracle_reproduces_tiny_decode():
    g = _load("tiny_decode.json")
    geo = g["geometry"]
    K, V, Q = (np.array(g[k], dtype=np.float32) for k in ("K", "V", "Q"))
    res = O.decode(Q, K, V, "f32", geo["branching"], geo["leaf_block"], geo["levels"], geo["beam"])
    for got, want in zip(res["tree"]["stored"], g["summaries"]):
        np.testing.assert_array_equal(got, np.array(want, dtype=np.float32))
    np.testing.assert_array_equal(res["route"]["indices"], np.array(g["indices"]))
    np.testing.assert_array_equal(res["route"]["trace"], np.array(g["trace"]))
    np.testing.assert_allclose(res["out"], np.array(g["out"]), rtol=1e-14, atol=1e-15)


def test_page_figures_and_workload_shapes():
    f = {x["name"]: x["value"] for x in _load("page_figures.json")["figures"]}
    w = workloads.get("alhr_1k")
    # the 1,024-token binary-tree workload matches the ALHR test's size and arity
    assert w.n_keys == f["alhr_tokens"] and w.branching == f["alhr_tree_arity"]
    keys_read = w.beam * w.leaf_block
    # reads 32 keys per query, within 10% of the ~30 the post reports
    assert keys_read == 32 and abs(keys_read - f["alhr_keys_per_query"]) / f["alhr_keys_per_query"] < 0.1
    # the post's 512 dense keys read as the causal average over 1,024 positions
    assert int(sum(range(1, f["alhr_tokens"] + 1)) / f["alhr_tokens"]) == f["dense_keys_per_query"]
    # 35.3x compression corresponds to 1024 / 35.3 = 29.0 keys per query
    assert round(f["alhr_tokens"] / f["alhr_kv_compression"], 1) == 29.0
    # the deep workload uses the deepest tree the ZHA abstract reports
    assert workloads.get("deep_planted").levels == f["zha_max_levels"]
    assert workloads.get("long_1m").n_keys > f["zha_context_tokens"]
