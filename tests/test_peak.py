"""The peak-measurement library the benchmark quotes roofline fractions
against: host checks (exports, op counts, argument rejection before any
launch) and, on the GPU, that each measured rate is plausible next to the
published dense peak (a counting mistake shows up as a rate above it)."""
import ctypes
import os

import pytest

from sparse_bit_attention_amd import peak


@pytest.fixture(scope="module", autouse=True)
def built():
    if not os.path.exists(peak.LIB_PATH):
        from sparse_bit_attention_amd import build
        build.build()


def test_exports():
    L = ctypes.CDLL(peak.LIB_PATH)
    for n in ("slapeak_mfma", "slapeak_mfma_ops", "slapeak_issue", "slapeak_stream"):
        assert hasattr(L, n)


@pytest.mark.parametrize("kind,mnk,chains", [(0, (16, 16, 64), 8), (1, (32, 32, 32), 4),
                                             (2, (16, 16, 32), 8), (3, (32, 32, 16), 4)])
def test_ops_count(kind, mnk, chains):
    m, n, k = mnk
    # 2 M N K per MFMA, `chains` MFMAs per iteration per wave, 4 waves per workgroup
    assert peak.ops_per_launch(kind, 7, 3) == 2 * m * n * k * chains * 7 * 4 * 3


def test_bad_arguments_rejected_before_launch():
    L = peak.lib()
    assert L.slapeak_mfma(4, 1, 1, ctypes.c_void_p(16), None) == 1
    assert L.slapeak_mfma(-1, 1, 1, ctypes.c_void_p(16), None) == 1
    assert L.slapeak_mfma(0, 0, 1, ctypes.c_void_p(16), None) == 1
    assert L.slapeak_mfma(0, 1, 0, ctypes.c_void_p(16), None) == 1
    assert L.slapeak_mfma(0, 1, 1, None, None) == 1
    assert L.slapeak_mfma_ops(5, 1, 1) == -1
    with pytest.raises(ValueError):
        peak.ops_per_launch(-1, 1, 1)
    p = ctypes.c_void_p(16)
    assert L.slapeak_issue(4, 1, 1, 1, p, p, None) == 1
    assert L.slapeak_issue(0, 0, 1, 1, p, p, None) == 1
    assert L.slapeak_issue(0, 3, 1, 1, p, p, None) == 1
    assert L.slapeak_issue(0, 1, 0, 1, p, p, None) == 1
    assert L.slapeak_issue(0, 1, 1, 0, p, p, None) == 1
    assert L.slapeak_issue(0, 1, 1, 1, None, p, None) == 1
    assert L.slapeak_issue(0, 1, 1, 1, p, None, None) == 1
    assert L.slapeak_stream(2, 4, 1, 1, p, p, p, None) == 1
    assert L.slapeak_stream(0, 0, 1, 1, p, p, p, None) == 1
    assert L.slapeak_stream(0, 9, 1, 1, p, p, p, None) == 1
    assert L.slapeak_stream(0, 4, 0, 1, p, p, p, None) == 1
    assert L.slapeak_stream(0, 4, 1, 0, p, p, p, None) == 1
    assert L.slapeak_stream(0, 4, 1, 1, None, p, p, None) == 1
    assert L.slapeak_stream(1, 4, 1, 1, None, None, p, None) == 1
    assert L.slapeak_stream(1, 4, 1, 1, None, p, None, None) == 1


@pytest.mark.gpu
def test_measured_rates_are_plausible():
    for kind, (instr, typ) in peak.KINDS.items():
        r = peak.mfma_rate(kind, target_ms=5.0, reps=2)
        pub = peak.PUBLISHED[typ]
        print(f"[peak] {instr}: {r / 1e12:.0f} T/s ({100 * r / pub:.1f}% of published)", flush=True)
        assert 0.3 * pub < r < 1.02 * pub, instr
    c = peak.copy_rate(1 << 28, reps=3)
    print(f"[peak] device copy {c / 1e9:.0f} GB/s", flush=True)
    assert 1e12 < c < 8.2e12


@pytest.mark.gpu
def test_issue_probe_cycles_are_plausible():
    # a 16x16x32 bf16 MFMA occupies the matrix core 16 cycles at the
    # published rate, so no slot holding one can take fewer; a lone vector
    # instruction takes at least one cycle
    t = peak.issue_table()
    for name, per_wps in t.items():
        for wps, r in per_wps.items():
            c = r["cycles_per_slot_per_simd"]
            print(f"[issue] {name} {wps}: {c:.1f} cycles per slot per SIMD at "
                  f"{r['clock_GHz']:.2f} GHz", flush=True)
            lo = 15.0 if "mfma" in name else 1.0
            assert lo <= c < 200.0, (name, wps, c)
            assert 0.5 < r["clock_GHz"] < 3.0, (name, wps, r)


@pytest.mark.gpu
def test_operand_rates_are_plausible():
    # 16-byte reads: at least a few bytes per cycle, and no more than 64
    # lanes x 16 bytes per cycle from either source
    t = peak.stream_table()
    for name, per_w in t.items():
        for w, r in per_w.items():
            print(f"[stream] {name} {w}: {r:.1f} bytes per cycle per CU", flush=True)
            assert 4.0 < r < 1024.0, (name, w, r)
