"""LDS layout of the backward's streamed tiles (host check of the kernel source).

The two sparse backward loops keep 64-row bf16 tiles in LDS with the 8-byte
units of each row XOR-swizzled by `sw_unit<D>(r)` (csrc/k_bwd.hip).  This test
takes the two XOR expressions from that source and checks, for D = 128:
  * each row's XOR is a permutation of its 32 units (no two elements collide);
  * the MFMA row reads, the transposing reads and the 16-byte tile stores each
    touch 32 distinct 8-byte slots modulo 256 bytes in every half-wave (the
    gfx950 LDS: 64 four-byte banks, 8-byte accesses served 32 lanes a pass),
    and every 16-byte store stays 16-byte aligned;
and for D = 64 (16 units, a row of 128 bytes) that the XOR is a permutation and
separates 16 consecutive rows of an MFMA row read.
"""
import os
import re

import pytest

SRC = os.path.join(os.path.dirname(__file__), "..", "sparse_bit_attention_amd", "csrc", "k_bwd.hip")


def _sw_unit_exprs():
    text = open(SRC).read()
    body = re.search(r"int sw_unit\(int r\) \{(.*?)\n\}", text, re.S).group(1)
    e128 = re.search(r"if constexpr \(D == 128\) return (.*?);", body).group(1)
    e64 = re.search(r"\n\s*return (.*?);", body).group(1)
    # the expressions use only r, integer literals and & << >> | ( ): the same in Python
    for e in (e128, e64):
        assert re.fullmatch(r"[r0-9&|<>() ]+", e), e
    return (lambda r: eval(e128, {}, {"r": r})), (lambda r: eval(e64, {}, {"r": r}))


F128, F64 = _sw_unit_exprs()


def _slot(f, units, r, u):
    return r * units + (u ^ f(r))


def _worst(addrs, period, group):
    worst = 1
    for g0 in range(0, len(addrs), group):
        seen = {}
        for a in addrs[g0:g0 + group]:
            seen[a % period] = seen.get(a % period, 0) + 1
        worst = max(worst, max(seen.values()))
    return worst


@pytest.mark.parametrize("f,units", [(F128, 32), (F64, 16)], ids=["d128", "d64"])
def test_row_xor_is_a_permutation(f, units):
    for r in range(64):
        assert sorted(u ^ f(r) for u in range(units)) == list(range(units))


def test_d128_reads_and_stores_are_conflict_free():
    f = F128
    # MFMA row reads (sw_rows): lane l reads row 16t + l%16 at unit 8kc + l/16 (+4)
    for t in range(4):
        for kc in range(4):
            for h in range(2):
                a = [_slot(f, 32, 16 * t + (l & 15), 8 * kc + (l >> 4) + 4 * h) for l in range(64)]
                assert _worst(a, 32, 32) == 1
    # transposing reads (sw_frag): lane l = 16g + j reads row 32kc2 + 4g + j/4 (+16)
    # at unit 4x + j%4
    for kc2 in range(2):
        for x in range(8):
            for h in range(2):
                a = [_slot(f, 32, 32 * kc2 + 4 * (l >> 4) + ((l & 15) >> 2) + 16 * h, 4 * x + (l & 3))
                     for l in range(64)]
                assert _worst(a, 32, 32) == 1
    # tile stores (tile_store_sw): thread x writes units 2(x%16), 2(x%16)+1 of row
    # x/16 as one 16-byte store, 16 lanes (256 bytes) a pass
    for e in range(16):
        a = [_slot(f, 32, 4 * e + (l >> 4), 2 * (l & 15)) for l in range(64)]
        assert all(s % 2 == 0 for s in a)  # 16-byte aligned, pair adjacent
        assert all(_slot(f, 32, 4 * e + (l >> 4), 2 * (l & 15) + 1) == a[l] + 1 for l in range(64))
        assert _worst([s // 2 for s in a], 16, 16) == 1


def test_d64_row_reads_are_conflict_free():
    f = F64
    for t in range(4):
        for kc in range(2):
            for h in range(2):
                a = [_slot(f, 16, 16 * t + (l & 15), 8 * kc + (l >> 4) + 4 * h) for l in range(64)]
                assert _worst(a, 16, 16) == 1


def test_d128_load_to_lds_copy_matches_the_swizzled_store():
    # tile_dma_sw128: wave w, instruction e, lane l writes the 16 bytes at
    # byte 16 l of the 1 KiB piece at rows 16w + 4e .. +3 (LDS row r = 16w +
    # 4e + l/16, 16-byte chunk p = l % 16) and fetches source chunk
    # k = p ^ (sw_unit(r) >> 1) of row r.  tile_store_sw puts source unit u
    # (8 bytes) of row r at unit u ^ sw_unit(r).  Every destination unit must
    # receive exactly the source unit the swizzled store would put there.
    f = F128
    written = {}
    for w in range(4):
        for e in range(4):
            for lane in range(64):
                r, p = 16 * w + 4 * e + lane // 16, lane % 16
                assert f(r) % 2 == 0  # a 16-byte piece stays whole under the XOR
                k = p ^ (f(r) >> 1)
                for h in range(2):  # the two 8-byte units of the piece
                    dst = (r, 2 * p + h)
                    assert dst not in written
                    written[dst] = (r, 2 * k + h)
    assert len(written) == 64 * 32
    for r in range(64):
        for u in range(32):
            assert written[(r, u ^ f(r))] == (r, u)
