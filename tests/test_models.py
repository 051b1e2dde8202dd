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


# ---- the kernels' LDS layouts under the measured gfx950 bank rules ----------------
def _kmaj(r):            # chunk swizzle of k-major tiles (A, column-major B)
    return r & 7


def _nmaj(k, chunks=32):  # chunk swizzle of a 16-bit row-major B tile
    return (((k & 3) | (((k >> 3) & 1) << 2)) << 1) & (chunks - 1)


def test_gfx950_model_reproduces_probe_signatures():
    """The measured signatures: contiguous 16-byte reads are conflict-free, 8-lane
    groups at a 256-byte stride conflict 2-way, 32-lane 8-byte groups are served together."""
    P = lds_model.gfx950_passes
    assert P(lambda l: l * 16, 16) == 1
    assert P(lambda l: (l % 16) * 16 + (l // 16) * 512, 16) == 1
    assert P(lambda l: (l % 8) * 16 + (l // 8) * 256, 16) == 2
    assert P(lambda l: (l % 4) * 16 + (l // 4) * 128, 16) == 2
    assert P(lambda l: l * 8, 8) == 1
    assert P(lambda l: (l % 16) * 8 + (l // 16) * 256, 8) == 2
    assert P(lambda l: (l % 32) * 8 + (l // 32) * 512, 8) == 1
    # the first A-fragment swizzle, (r ^ (r >> 3)) & 7, measured 2-way
    old = lambda l: (l & 15) * 128 + (((l >> 4) ^ (((l & 15) ^ ((l & 15) >> 3)) & 7)) << 4)
    assert P(old, 16) == 2


@pytest.mark.parametrize("ks", [0, 1])
def test_a_fragment_reads_conflict_free(ks):
    """16 rows x 2 chunk columns per 16-byte read, rows of 128 bytes (BK = 64 halfs or 32 floats)."""
    for r0 in (0, 16, 112):
        addr = lambda l: (r0 + (l & 15)) * 128 + ((((ks * 4 + (l >> 4)) ^ _kmaj(r0 + (l & 15)))) << 4)
        assert lds_model.gfx950_passes(addr, 16) == 1


@pytest.mark.parametrize("bn", [128, 256])
def test_transpose_reads_conflict_free(bn):
    chunks = bn // 8
    for j in range(bn // 16 if bn < 256 else 4):
        for hh in (0, 1):
            for ks in (0, 1):
                def addr(l):
                    l16, lg = l & 15, l >> 4
                    col = j * 16 + ((l16 & 3) << 2)
                    k = ks * 32 + lg * 8 + hh * 4 + (l16 >> 2)
                    return k * bn * 2 + (((col >> 3) ^ _nmaj(k, chunks)) << 4) + (col & 7) * 2
                assert lds_model.gfx950_passes(addr, 8) == 1


def test_fp32_row_major_b_reads_conflict_free():
    """fp32 MFMA kernel: lane reads a float4 along n of row kk + 4*(l//16) + s."""
    for s_ in range(4):
        addr = lambda l: (4 * (l >> 4) + s_) * 256 * 4 + 4 * (l & 15) * 4
        assert lds_model.gfx950_passes(addr, 16) == 1


def _tr32_addr(j, hh, ks, wn, swz):
    """Byte address of lane l's ds_read_b64_tr_b16 in the 32x32x16 kernels: k-row
    (l // 32) * 8 + (l % 16) // 4 (+ 16 ks + 4 hh), columns wn*64 + 32 j + 16 ((l // 16) % 2)
    + 4 (l % 4), 512-byte rows."""
    def addr(l):
        l16, lg = l & 15, l >> 4
        col = wn * 64 + j * 32 + (lg & 1) * 16 + ((l16 & 3) << 2)
        k = (lg >> 1) * 8 + (l16 >> 2) + ks * 16 + hh * 4
        return k * 512 + (((col >> 3) ^ swz(k)) << 4) + (col & 7) * 2
    return addr


@pytest.mark.parametrize("wn", [0, 1, 2, 3])
def test_transpose32_reads_conflict_free(wn):
    """The 32x32x16 kernels' transpose reads are conflict-free; each 32-lane phase
    falls into two 256-byte windows, which measured no slower than four (a swizzle
    that also flips chunk bit 4 for k-rows 2 and 3: 116.0 against 116.3 us at 4096^3)."""
    for j in (0, 1):
        for hh in (0, 1):
            for ks in (0, 1):
                addr = _tr32_addr(j, hh, ks, wn, lambda k: (k & 3) << 2)
                assert lds_model.gfx950_passes(addr, 8) == 1
                assert lds_model.gfx950_window_load(addr, 8) == 2


@pytest.mark.parametrize("ks", [0, 1])
def test_a32_fragment_reads_window_balanced(ks):
    """32x32x16 A (and column-major B) fragments: 64-byte k-major rows, 32 rows per
    read, chunk (2 ks + l // 32) ^ ((r >> 2) & 3)."""
    for r0 in (0, 32, 96):
        addr = lambda l: (r0 + (l & 31)) * 64 + (((ks * 2 + (l >> 5)) ^ (((l & 31) >> 2) & 3)) << 4)
        assert lds_model.gfx950_passes(addr, 16) == 1
        assert lds_model.gfx950_window_load(addr, 16) == 1
