"""The layer geometry the oracle and the library use agrees with the figures the pages print
(tests/golden/dsa_geometry.txt, each figure with its page and section)."""
import os

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "dsa_geometry.txt")


def _golden():
    vals = {}
    for line in open(GOLDEN, encoding="utf-8"):
        line = line.split("#")[0].strip()
        if line:
            k, v = line.split("=")
            vals[k.strip()] = int(v)
    return vals


def test_oracle_geometry_matches_pages():
    import oracle
    g = _golden()
    assert oracle.REGION == g["region_size"] and oracle.PROXY == g["proxy_dim"]
    assert oracle.TOPK == g["topk"] and oracle.IDX_HEADS == g["indexer_heads"]
    assert oracle.Q_HEADS == g["q_heads"] and oracle.GROUPS == g["kv_groups"]
    assert oracle.HEAD_DIM == g["head_dim"] and oracle.WINDOW == g["sliding_window"]


def test_derived_figures():
    g = _golden()
    # 1M tokens split into regions of 8
    assert g["context_1m_tokens"] // g["region_size"] == g["regions_at_1m"]
    # K and V, 4 groups, 192 dims, 2-byte bf16 per token per full-attention layer
    assert 2 * g["kv_groups"] * g["head_dim"] * 2 == g["kv_bytes_per_token_per_layer"]
    # the sparse budget: top-512 regions of 8 tokens
    assert g["topk"] * g["region_size"] == g["tokens_attended_per_query_approx"]
