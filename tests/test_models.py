"""Host-side models pinned to the chapter's printed outputs.

* the closed-form traffic table of "Shared memory and tensor cores" 13.1
* the bank-conflict passes of 13.6
"""
import os

import pytest

from dense_gemm_06_amd import lds_model, traffic

HERE = os.path.dirname(os.path.abspath(__file__))


def _lines(name):
    with open(os.path.join(HERE, "golden", name)) as f:
        return [l.rstrip("\n") for l in f if l.strip() and not l.startswith("#")]


def test_traffic_table_matches_page():
    assert traffic.format_table_13_1(4096) == _lines("traffic_table_13_1.txt")


def test_traffic_closed_forms():
    N = 4096
    for T in (16, 32, 64, 128, 256):
        e = traffic.tiled_elements(N, N, N, T, T)
        assert e == (N // T) * (N // T) * (T + T) * N
        # intensity = T/4 FLOP/byte for fp32 square tiles
        assert traffic.flops(N, N, N) / (4 * e) == pytest.approx(T / 4)
        assert traffic.intensity(T, T, 4) == pytest.approx(T / 4)
    # rectangular tiles: BM*BN/(2(BM+BN)) for 4-byte elements
    assert traffic.intensity(256, 128, 4) == pytest.approx(256 * 128 / (2 * 384))
    # ragged: exact masked count
    assert traffic.tiled_elements(3001, 5003, 1037, 256, 256) == 3001 * 1037 * 20 + 1037 * 5003 * 12
    assert traffic.compulsory_read_bytes(N, N, N, 4) == 134217728


def test_bank_model_reproduces_13_6():
    gold = {}
    for l in _lines("bank_passes_13_6.txt"):
        k, v = [p.strip() for p in l.split("|")]
        gold[k] = int(v)
    T, k = 16, 3
    tid = lambda t: (t // T, t % T)
    got = {
        "smem_gemm T=16 store sA[ty*T+tx]": lds_model.passes(lambda t: tid(t)[0] * T + tid(t)[1]),
        "smem_gemm T=16 load sA[ty*T+k] (k=3)": lds_model.passes(lambda t: tid(t)[0] * T + k),
        "smem_gemm T=16 load sB[k*T+tx] (k=3)": lds_model.passes(lambda t: k * T + tid(t)[1]),
    }
    T = 32
    tid = lambda t: (t // T, t % T)
    got["column walk T=32 load s[tx*32+k]"] = lds_model.passes(lambda t: tid(t)[1] * 32 + k)
    got["column walk T=32 load s[tx*33+k] (padded row)"] = lds_model.passes(lambda t: tid(t)[1] * 33 + k)
    assert got == gold
