"""Quality of the packed cache against its ablations, on the CPU (oracle/quality.py).

On every synthetic workload the method (rotation, then T = 4 normalisation passes, then round to
nearest) rebuilds the keys with clearly less error than without the rotation, without the
normalisation, or without both (KVarN blog post, "KVarN Nasıl Çalışır?": the rotation spreads the
outlier channels and the normalisation evens out rows and columns before rounding).  The values (2
bits: four levels per token group) carry a grid error near 0.5 whatever the variant, so only the keys
separate the variants.  The full table is in the design notes; it comes from `python -m oracle.quality`.
"""
import numpy as np
import pytest

from kv_cache_quantization_kvarn_amd import synth
from oracle import kvarn_oracle as o
from oracle import quality as Q


def test_method_variant_is_the_oracle():
    w = synth.WORKLOADS["tiny_1x1024"]
    k, v = synth.layer_kv(w, 0, 128, "cpu")
    for x, is_v in ((k.numpy()[:, 3], False), (v.numpy()[:, 5], True)):
        a = Q.quantize_dequantize(x, is_v)
        b = o.dequantize_tile(o.quantize_tile(x, is_v), is_v)
        assert np.array_equal(a, b)


@pytest.mark.parametrize("name", ["llama3_8b_layer_16x8192", "long_context_1x131072", "paged_mixed_128xU1k_32k"])
def test_method_rebuilds_outlier_keys_best(name):
    r = Q.workload_quality(synth.WORKLOADS[name], n_blocks=4)["variants"]
    method = r["rotation + T=4 (the method)"]["k_rel"]
    others = [e["k_rel"] for n, e in r.items() if not n.endswith("(the method)")]
    assert method < 0.95 * min(others), (method, others)
    assert method < 0.09
    # the values' 2-bit grid: about half the signal for every variant
    for e in r.values():
        assert 0.4 < e["v_rel"] < 0.6
