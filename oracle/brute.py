"""Pure-Python brute force for tiny shapes -- TEST INFRASTRUCTURE ONLY.

An implementation independent of oracle.c: storage is decoded with
``struct`` and the e4m3fn definition written out again, sums use
``math.fsum``, and softmax is exp(s - max) / sum.  It exists to cross-check
the C oracle on shapes small enough for Python loops.
"""
from __future__ import annotations

import math
import struct
from typing import List, Sequence


def bf16_to_float(bits: int) -> float:
    return struct.unpack("<f", struct.pack("<I", (int(bits) & 0xFFFF) << 16))[0]


def f32_to_float(x) -> float:
    return float(x)


def e4m3fn_to_float(code: int) -> float:
    code = int(code) & 0xFF
    s = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return math.nan
    if e == 0:
        return s * (m / 8.0) * 2.0 ** (-6)
    return s * (1.0 + m / 8.0) * 2.0 ** (e - 7)


def decode_storage(raw, dtype: str, scale: float = 1.0) -> List[float]:
    flat = raw.reshape(-1).tolist()
    if dtype == "f32":
        return [float(x) for x in flat]
    if dtype == "bf16":
        return [bf16_to_float(x) for x in flat]
    return [e4m3fn_to_float(x) * scale for x in flat]


def attention(seq_lens: Sequence[int], extend_lens, page_table, page_size: int, q, q_dtype: str,
              k_pool, v_pool, kv_dtype: str, scale: float, k_scale: float = 1.0,
              v_scale: float = 1.0):
    """Returns (out, lse) as nested lists out[token][head][d], lse[token][head]."""
    N, Hq, D = q.shape            # key width D; values may be wider or narrower
    Hkv = k_pool.shape[1]
    Dv = v_pool.shape[2]
    G = Hq // Hkv
    qv = decode_storage(q, q_dtype)
    kv = decode_storage(k_pool, kv_dtype, k_scale)
    vv = decode_storage(v_pool, kv_dtype, v_scale)
    B = len(seq_lens)
    n_new = [1] * B if extend_lens is None else [int(x) for x in extend_lens]
    out, lse = [], []
    tok = 0
    for b in range(B):
        L = int(seq_lens[b])
        for i in range(n_new[b]):
            pos = L - n_new[b] + i
            row_o, row_l = [], []
            for h in range(Hq):
                g = h // G
                qrow = qv[(tok * Hq + h) * D:(tok * Hq + h + 1) * D]
                scores, vrows = [], []
                for t in range(pos + 1):
                    slot = int(page_table[b][t // page_size]) * page_size + t % page_size
                    krow = kv[(slot * Hkv + g) * D:(slot * Hkv + g + 1) * D]
                    scores.append(scale * math.fsum(a * c for a, c in zip(qrow, krow)))
                    vrows.append(vv[(slot * Hkv + g) * Dv:(slot * Hkv + g + 1) * Dv])
                m = max(scores)
                w = [math.exp(s - m) for s in scores]
                z = math.fsum(w)
                row_o.append([math.fsum(w[t] * vrows[t][d] for t in range(len(w))) / z
                              for d in range(Dv)])
                row_l.append(m + math.log(z))
            out.append(row_o)
            lse.append(row_l)
            tok += 1
    return out, lse
