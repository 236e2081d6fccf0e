"""Pure-Python brute force of single-token GQA decode (test infrastructure only).

Written independently of ``gqa_oracle.c`` to cross-check it on tiny inputs: its own decoders, exact
summation with ``math.fsum`` and the textbook softmax, one query head at a time.

Definition followed: per query head h, the KV head is h // G with G = Hq // Hkv (contiguous groups;
"Grouped-Query Attention: How Sharing KV Heads Shrinks Inference Memory", section "How grouped-query
attention works"), score_t = scale * (q . k_t) and output = sum_t softmax(score)_t * v_t
("Grouped Query Attention (GQA): Efficient Multi-Head Attention", Worked example 2).  seq_len 0 gives a
zero row.
"""
import math
import struct


def bf16_bits_to_float(bits):
    return struct.unpack("<f", struct.pack("<I", (int(bits) & 0xFFFF) << 16))[0]


def fp8_e4m3_code_to_float(code):
    code = int(code) & 0xFF
    neg = code >= 128
    e, m = (code >> 3) & 0xF, code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    # integer significand times a power of two: normal (8 + m) * 2^(e - 10), subnormal m * 2^-9
    val = math.ldexp(8 + m, e - 10) if e else math.ldexp(m, -9)
    return -val if neg else val


def _decode(x, dtype):
    if dtype == "f32":
        return float(x)
    if dtype == "bf16":
        return bf16_bits_to_float(x)
    if dtype == "fp8_e4m3":
        return fp8_e4m3_code_to_float(x)
    raise ValueError(dtype)


def decode(q, k, v, seq_lens, scale, q_dtype="f32", kv_dtype="f32", k_descale=1.0, v_descale=1.0):
    """q: nested [B][Hq][d]; k, v: nested [B][Hkv][L][d] (raw storage values); returns nested floats."""
    B = len(q)
    Hq = len(q[0]) if B else 0
    Hkv = len(k[0]) if B else 1
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    G = Hq // Hkv
    out = []
    for b in range(B):
        n = int(seq_lens[b])
        rows = []
        for h in range(Hq):
            j = h // G
            qv = [_decode(x, q_dtype) for x in q[b][h]]
            d = len(qv)
            if n == 0:
                rows.append([0.0] * d)
                continue
            scores = []
            for t in range(n):
                kv = [_decode(x, kv_dtype) * k_descale for x in k[b][j][t]]
                scores.append(scale * math.fsum(a * c for a, c in zip(qv, kv)))
            top = max(scores)
            e = [math.exp(s - top) for s in scores]
            z = math.fsum(e)
            p = [x / z for x in e]
            vals = [[_decode(x, kv_dtype) * v_descale for x in v[b][j][t]] for t in range(n)]
            rows.append([math.fsum(p[t] * vals[t][c] for t in range(n)) for c in range(d)])
        out.append(rows)
    return out
