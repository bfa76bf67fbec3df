"""Pins against numbers the pages print (L4 server log listing)."""
import os

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))


def _read(name):
    vals = {}
    with open(os.path.join(HERE, "golden", name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                k, v = (s.strip() for s in line.split("=", 1))
                vals[k] = v
    return vals


def test_l4_pool_size_is_token_major_without_padding():
    g = _read("l4_server_log.txt")
    tokens = int(g["pool_tokens"])
    heads = int(g["layers"]) * int(g["kv_heads"])
    per_pool = oracle.pool_bytes(tokens, heads, int(g["head_dim"]), 2)
    # the log's "GB" is GiB: 24,094 x 73,728 B = 1.654 GiB, printed as 1.65
    assert f"{per_pool / 2**30:.2f}" == g["k_size_printed"] == g["v_size_printed"]
    # a decimal-GB reading would print 1.78 instead
    assert f"{per_pool / 1e9:.2f}" != g["k_size_printed"]


def test_l4_token_usage_is_used_over_pool():
    g = _read("l4_server_log.txt")
    assert f"{int(g['cached_tokens']) / int(g['pool_tokens']):.2f}" == g["token_usage_printed"]
