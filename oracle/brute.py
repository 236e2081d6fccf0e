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


def decode_paged(q, k_pages, v_pages, block_table, seq_lens, scale, q_dtype="f32", kv_dtype="f32",
                 k_descale=1.0, v_descale=1.0):
    """Paged cache: k_pages, v_pages nested [num_blocks][Hkv][block_size][d]; block_table nested
    [B][max_blocks].  Position t of sequence b is row t % block_size of page block_table[b][t //
    block_size].  Gathers each sequence's rows into a dense nested cache and applies ``decode``."""
    B = len(q)
    Hkv = len(k_pages[0]) if k_pages else 1
    bs = len(k_pages[0][0]) if k_pages else 1
    d = len(q[0][0]) if B else 0
    L = max([int(n) for n in seq_lens] + [1])
    kd, vd = [], []
    for b in range(B):
        n = int(seq_lens[b])
        kb, vb = [], []
        for j in range(Hkv):
            rows_k, rows_v = [], []
            for t in range(L):
                if t < n:
                    page = int(block_table[b][t // bs])
                    rows_k.append(list(k_pages[page][j][t % bs]))
                    rows_v.append(list(v_pages[page][j][t % bs]))
                else:
                    rows_k.append([0] * d)
                    rows_v.append([0] * d)
            kb.append(rows_k)
            vb.append(rows_v)
        kd.append(kb)
        vd.append(vb)
    return decode(q, kd, vd, seq_lens, scale, q_dtype, kv_dtype, k_descale, v_descale)


def _to_f32(v):
    """Round a Python float to binary32 (nearest even), overflowing to infinity."""
    if math.isnan(v) or math.isinf(v):
        return v
    try:
        return struct.unpack("<f", struct.pack("<f", v))[0]
    except OverflowError:  # beyond the binary32 range after rounding
        return math.copysign(math.inf, v)


def encode_fp8_e4m3(x, descale=1.0):
    """e4m3fn code of x / descale, both taken as binary32 and divided in binary32: exponent by
    math.frexp, three mantissa bits rounded half to even by round(); saturates at +-448; NaN -> 0x7F
    with the sign bit.  (An independent route to the oracle's nearest-code search.)"""
    x32, s32 = _to_f32(x), _to_f32(descale)
    if math.isnan(x32):
        return 0x7F | (0x80 if math.copysign(1.0, x32) < 0 else 0)
    # the double quotient rounded to binary32 is the correctly rounded binary32 quotient (53 >= 2*24+2)
    y = _to_f32(x32 / s32) if s32 != 0 else _to_f32(math.copysign(math.inf, x32) if x32 else math.nan)
    neg = math.copysign(1.0, y) < 0
    sign = 0x80 if neg else 0
    if math.isnan(y):
        return 0x7F | sign
    a = abs(y)
    if a >= 448.0:
        return 0x7E | sign
    if a < 2.0 ** -6:
        return sign | round(a * 512.0)            # subnormal multiples of 2^-9 (8 -> smallest normal)
    m, e = math.frexp(a)                          # a = m * 2^e, m in [0.5, 1)
    e -= 1                                        # a = (2m) * 2^e, 2m in [1, 2)
    frac = round((2.0 * m - 1.0) * 8.0)
    if frac == 8:
        frac, e = 0, e + 1
    return sign | ((e + 7) << 3) | frac


def encode_bf16(x):
    """bf16 bits of binary32 x, rounded to nearest even by integer arithmetic on its bits."""
    u = struct.unpack("<I", struct.pack("<f", float(x)))[0]
    if (u & 0x7FFFFFFF) > 0x7F800000:
        return 0x7FC0 | ((u >> 16) & 0x8000)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) & 0xFFFF


def prefill(q, k, v, scale, dtype="f32", causal=True):
    """q nested [B][Hq][S][d], k, v nested [B][Hkv][S][d] (raw storage); position i of head h attends
    to positions t <= i (all t when not causal) of KV head h // G.  Builds each row's decode problem
    over the first i + 1 positions and hands it to ``decode``."""
    B = len(q)
    Hq, S = len(q[0]), len(q[0][0])
    Hkv = len(k[0])
    out = []
    for b in range(B):
        heads = []
        for h in range(Hq):
            rows = []
            for i in range(S):
                n = i + 1 if causal else S
                # a one-sequence decode with Hkv query slots (group size 1): slot j reads KV head j
                res = decode([[q[b][h][i]] * Hkv], [k[b]], [v[b]], [n], scale, dtype, dtype)
                rows.append(res[0][h // (Hq // Hkv)])
            heads.append(rows)
        out.append(heads)
    return out
