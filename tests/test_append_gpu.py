"""GPU cache append (gqa_append_kv, gqa_append_kv_paged) against the oracle, through the C ABI.

Storage codes are integers decided by floating point, so the bar is bit-exact: the whole cache after the
GPU append must equal, byte for byte, the oracle's cache after its append of the same rows.  The fp8
encoder is checked on every bf16 input, and on random binary32 bit patterns (NaN, infinities, huge and
subnormal values included).  The end-to-end test appends the new token, then decodes over it.
"""
import numpy as np
import pytest
import torch

import grouped_query_attention_04_amd as gqa
import workloads
from oracle import ref
from tests.test_parity_gpu import DEV, compare, say

pytestmark = pytest.mark.gpu

RAW_TORCH = {"f32": torch.int32, "bf16": torch.int16, "fp8_e4m3": torch.uint8}


def _raw(t, dt):
    return t.detach().cpu().contiguous().view(RAW_TORCH[dt]).numpy()


def _new_rows(B, Hkv, d, new, seed, scale=3.0):
    g = torch.Generator().manual_seed(seed)
    kn = torch.randn(B, Hkv, d, generator=g) * scale
    vn = torch.randn(B, Hkv, d, generator=g) * scale
    if new == "bf16":
        kn, vn = kn.to(torch.bfloat16), vn.to(torch.bfloat16)
    return kn, vn


@pytest.mark.parametrize("kv", ["f32", "bf16", "fp8_e4m3"])
@pytest.mark.parametrize("new", ["f32", "bf16"])
@pytest.mark.parametrize("d", [64, 128])
def test_append_dense_bit_exact(kv, new, d):
    say(f"append dense kv={kv} new={new} d={d}")
    B, Hkv, L = 5, 4, 40
    qd = "f32" if kv == "f32" else "bf16"
    c = workloads.make_case(B, 2 * Hkv, Hkv, d, L, qd, kv, seq_lens=[L] * B, seed=70 + d)
    kn, vn = _new_rows(B, Hkv, d, new, 71 + d)
    pos = torch.tensor([0, 39, -1, 40, 17], dtype=torch.int32)     # 40 is past the cache: skipped
    kd, vd = (0.5, 1.75) if kv == "fp8_e4m3" else (1.0, 1.0)
    kc, vc = c["k"].to(DEV), c["v"].to(DEV)
    skipped = torch.zeros(1, dtype=torch.int32, device=DEV)
    gqa.append_kv(kn.to(DEV), vn.to(DEV), kc, vc, pos.to(DEV), k_descale=kd, v_descale=vd, skipped=skipped)
    torch.cuda.synchronize()
    wk, wv, wskip = ref.append(kn, vn, new, c["k"], c["v"], kv, pos.numpy(), kd, vd)
    assert int(skipped.item()) == wskip == 1
    assert np.array_equal(_raw(kc, kv), wk.view(_raw(kc, kv).dtype))
    assert np.array_equal(_raw(vc, kv), wv.view(_raw(vc, kv).dtype))


@pytest.mark.parametrize("kv", ["bf16", "fp8_e4m3"])
@pytest.mark.parametrize("bs", [16, 64])
def test_append_paged_bit_exact(kv, bs):
    say(f"append paged kv={kv} bs={bs}")
    B, Hkv, d, L = 4, 2, 128, 200
    c = workloads.make_case(B, 8, Hkv, d, L, "bf16", kv, seq_lens=[200, 130, 64, 100], seed=72)
    pg = workloads.paginate(c, bs, seed=11, spare_pages=3)
    table = pg["block_table"].clone()
    table[3, 99 // bs] = pg["num_blocks"] + 7         # the target page of sequence 3 is outside the pool
    kn, vn = _new_rows(B, Hkv, d, "bf16", 73)
    pos = torch.tensor([199, 64, 63, 99], dtype=torch.int32)
    kp, vp = pg["k_pages"].to(DEV), pg["v_pages"].to(DEV)
    skipped = torch.zeros(1, dtype=torch.int32, device=DEV)
    gqa.append_kv_paged(kn.to(DEV), vn.to(DEV), kp, vp, table.to(DEV), pos.to(DEV), k_descale=0.75,
                        v_descale=0.75, skipped=skipped)
    torch.cuda.synchronize()
    wk, wv, wskip = ref.append(kn, vn, "bf16", pg["k_pages"], pg["v_pages"], kv, pos.numpy(), 0.75, 0.75,
                               block_table=table.numpy())
    assert int(skipped.item()) == wskip == 1
    assert np.array_equal(_raw(kp, kv), wk.view(_raw(kp, kv).dtype))
    assert np.array_equal(_raw(vp, kv), wv.view(_raw(vp, kv).dtype))


@pytest.mark.parametrize("descale", [1.0, 0.375, 3.0, 2.0 ** -6])
def test_fp8_encoder_on_every_bf16_input(descale):
    say(f"fp8 encoder, all bf16 inputs, descale {descale}")
    B, Hkv, d = 64, 8, 128                            # 65536 elements = every bf16 pattern
    bits = torch.arange(65536, dtype=torch.int32).to(torch.int16).view(torch.bfloat16).reshape(B, Hkv, d)
    kc = torch.zeros(B, Hkv, 1, d, dtype=torch.float8_e4m3fn)
    kd, vd = kc.clone(), kc.clone()
    kcd, vcd = kd.to(DEV), vd.to(DEV)
    pos = torch.zeros(B, dtype=torch.int32)
    gqa.append_kv(bits.to(DEV), bits.flip(-1).contiguous().to(DEV), kcd, vcd, pos.to(DEV), k_descale=descale,
                  v_descale=descale)
    torch.cuda.synchronize()
    wk, wv, _ = ref.append(bits, bits.flip(-1).contiguous(), "bf16", kc, kc.clone(), "fp8_e4m3", pos.numpy(),
                           descale, descale)
    assert np.array_equal(_raw(kcd, "fp8_e4m3"), wk)
    assert np.array_equal(_raw(vcd, "fp8_e4m3"), wv)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_fp8_and_bf16_encoders_on_random_f32_bit_patterns(seed):
    say(f"encoders on random binary32 bit patterns, seed {seed}")
    B, Hkv, d = 64, 8, 128
    g = torch.Generator().manual_seed(80 + seed)
    bits = torch.randint(-2 ** 31, 2 ** 31 - 1, (B, Hkv, d), generator=g, dtype=torch.int64).to(torch.int32)
    x = bits.view(torch.float32)
    # and values of fp8 range, where rounding decisions are dense
    y = (torch.randn(B, Hkv, d, generator=g) * 100).float()
    pos = torch.zeros(B, dtype=torch.int32)
    for kv, dt in (("fp8_e4m3", torch.float8_e4m3fn), ("bf16", torch.bfloat16)):
        kc = torch.zeros(B, Hkv, 1, d, dtype=dt)
        kcd, vcd = kc.to(DEV), kc.to(DEV)
        gqa.append_kv(x.to(DEV), y.to(DEV), kcd, vcd, pos.to(DEV), k_descale=1.5, v_descale=1.5)
        torch.cuda.synchronize()
        wk, wv, _ = ref.append(x, y, "f32", kc, kc.clone(), kv, pos.numpy(), 1.5, 1.5)
        assert np.array_equal(_raw(kcd, kv), wk.view(_raw(kcd, kv).dtype)), kv
        assert np.array_equal(_raw(vcd, kv), wv.view(_raw(vcd, kv).dtype)), kv


@pytest.mark.parametrize("paged", [False, True])
def test_append_then_decode_end_to_end(paged):
    """One decode step of the long-context fp8 layer shape at reduced length: append the new token's
    K/V (bf16 rows quantised into the fp8 cache) at seq_lens[b], then decode over seq_lens[b] + 1."""
    say(f"append + decode, fp8 cache, paged={paged}")
    B, Hq, Hkv, d, L = 2, 64, 8, 128, 2048
    c = workloads.make_case(B, Hq, Hkv, d, L, "bf16", "fp8_e4m3", seq_lens=(2047, 1500), seed=74)
    kd, vd = 0.5, 0.5
    c["k_descale"], c["v_descale"] = kd, vd
    kn, vn = _new_rows(B, Hkv, d, "bf16", 75, scale=1.0)
    pos = c["seq_lens"].clone()
    after = c["seq_lens"] + 1
    if paged:
        pg = workloads.paginate(dict(c, seq_lens=after), 64, seed=12, spare_pages=2)
        kp, vp, table = pg["k_pages"].to(DEV), pg["v_pages"].to(DEV), pg["block_table"].to(DEV)
        gqa.append_kv_paged(kn.to(DEV), vn.to(DEV), kp, vp, table, pos.to(DEV), k_descale=kd, v_descale=vd)
        got = gqa.decode_paged(c["q"].to(DEV), kp, vp, table, after.to(DEV), c["scale"], k_descale=kd,
                               v_descale=vd)
        wk, wv, _ = ref.append(kn, vn, "bf16", pg["k_pages"], pg["v_pages"], "fp8_e4m3", pos.numpy(), kd, vd,
                               block_table=pg["block_table"].numpy())
        want = ref.decode_paged(c["q"], wk, wv, pg["block_table"].numpy(), after.numpy(), c["scale"], None,
                                "bf16", "fp8_e4m3", kd, vd)
    else:
        kc, vc = c["k"].to(DEV), c["v"].to(DEV)
        gqa.append_kv(kn.to(DEV), vn.to(DEV), kc, vc, pos.to(DEV), k_descale=kd, v_descale=vd)
        got = gqa.decode(c["q"].to(DEV), kc, vc, after.to(DEV), c["scale"], k_descale=kd, v_descale=vd)
        wk, wv, _ = ref.append(kn, vn, "bf16", c["k"], c["v"], "fp8_e4m3", pos.numpy(), kd, vd)
        want = ref.decode(c["q"], wk, wv, after.numpy(), c["scale"], "bf16", "fp8_e4m3", kd, vd)
    torch.cuda.synchronize()
    compare(got, want, "fp8_e4m3", "append + decode")
