"""Host-side checks of the C ABI (no GPU): the library loads, exports every
symbol declared in include/sagesla.h, and validates plans on the host."""
import ctypes
import math
import os
import re

import numpy as np
import pytest

import oracle
from sparse_bit_attention_amd import sla

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sagesla.h")


@pytest.fixture(scope="module", autouse=True)
def built():
    if not os.path.exists(sla.LIB_PATH):
        from sparse_bit_attention_amd import build
        build.build()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sla_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ("sla_plan", "sla_quantize", "sla_attention_fwd"):
        assert n in names
    assert set(names) == set(sla.EXPORTS)


def test_library_exports_every_declared_symbol():
    L = ctypes.CDLL(sla.LIB_PATH)
    for n in declared_functions():
        assert hasattr(L, n), n


def test_status_strings():
    for s in range(6):
        assert sla.status_string(s)
    assert sla.status_string(0) == "ok"


def plan_status(**kw):
    cfg = dict(B=1, H=2, N=1024, d=64, block=64, topk=0.25, use_linear=1, sm_scale=0.0, qk_int8=1,
               qk_fine=0, backward=0)
    cfg.update(kw)
    c = sla.sla_config(*(cfg[f] for f, _ in sla.sla_config._fields_))
    h = ctypes.c_void_p()
    st = sla.lib().sla_plan(ctypes.byref(c), ctypes.byref(h))
    if st == 0:
        sla.lib().sla_plan_destroy(h)
    return st


@pytest.mark.parametrize("kw,status", [
    ({}, sla.SLA_OK),
    ({"d": 128}, sla.SLA_OK),
    ({"d": 96}, sla.SLA_EUNSUPPORTED),
    ({"block": 128}, sla.SLA_EUNSUPPORTED),
    ({"N": 0}, sla.SLA_EINVAL),
    ({"B": 0}, sla.SLA_EINVAL),
    ({"H": -1}, sla.SLA_EINVAL),
    ({"topk": -0.01}, sla.SLA_EINVAL),
    ({"topk": 1.5}, sla.SLA_EINVAL),
    ({"topk": float("nan")}, sla.SLA_EINVAL),
    ({"use_linear": 2}, sla.SLA_EINVAL),
    ({"sm_scale": -1.0}, sla.SLA_EINVAL),
    ({"sm_scale": float("inf")}, sla.SLA_EINVAL),
    ({"topk": 0.0}, sla.SLA_OK),
    ({"topk": 1.0}, sla.SLA_OK),
    ({"N": 1}, sla.SLA_OK),
    ({"N": 2_000_000}, sla.SLA_OK),
    ({"N": 2_000_000_000}, sla.SLA_EUNSUPPORTED),
    ({"qk_int8": 0}, sla.SLA_OK),
    ({"qk_int8": 0, "d": 128}, sla.SLA_OK),
    ({"qk_int8": 2}, sla.SLA_EINVAL),
    ({"qk_fine": 1}, sla.SLA_OK),
    ({"qk_fine": 1, "qk_int8": 0}, sla.SLA_EINVAL),
    ({"qk_fine": 2}, sla.SLA_EINVAL),
    ({"backward": 1, "qk_int8": 0}, sla.SLA_OK),
    ({"backward": 1, "qk_int8": 0, "use_linear": 0}, sla.SLA_OK),
    ({"backward": 1}, sla.SLA_EUNSUPPORTED),  # the backward is plain SLA's
    ({"backward": 2, "qk_int8": 0}, sla.SLA_EINVAL),
])
def test_plan_validation(kw, status):
    assert plan_status(**kw) == status


def test_plan_null_arguments():
    L = sla.lib()
    h = ctypes.c_void_p()
    assert L.sla_plan(None, ctypes.byref(h)) == sla.SLA_EINVAL
    assert L.sla_plan_info(None, None, None, None) == sla.SLA_EINVAL
    assert L.sla_plan_destroy(None) == sla.SLA_OK


@pytest.mark.parametrize("N,topk", [(1024, 0.25), (32760, 0.1), (75600, 0.1), (32760, 1.0),
                                    (1000, 0.29), (64, 0.05), (65, 0.5), (75600, 0.15),
                                    (75600, 0.05), (4096, 0.0)])
def test_plan_kb_matches_oracle(N, topk):
    p = sla.Plan(1, 1, N, 128, topk)
    T = oracle.nblocks(N)
    assert p.info.T == T
    # the plan receives topk as float32
    assert p.info.kb == oracle.kb_for(T, float(np.float32(topk)))


def test_workspace_size_and_regions():
    B, H, N, d = 1, 40, 75600, 128
    p = sla.Plan(B, H, N, d, 0.1)
    T, kb = p.info.T, p.info.kb
    BH = B * H
    assert (T, kb) == (1182, 118)
    sizes = {}
    for r in sla.WS_REGIONS:
        off, n = p.ws_region(0, r)
        assert off % 256 == 0
        assert off + n <= p.info.workspace_bytes
        sizes[r] = n
    assert sizes["Q8"] == sizes["K8"] == BH * T * 64 * d
    assert sizes["MASK"] == BH * T * math.ceil(T / 64) * 8
    assert sizes["KEPT"] == BH * T * kb * 4
    assert sizes["QBAR"] == BH * T * d * 4
    # linear states dominate: two bf16 [BH][T][d*d + d] arrays
    assert p.info.workspace_bytes > 2 * BH * T * (d * d + d) * 2
    q = sla.Plan(B, H, N, d, 0.1, use_linear=False)
    assert q.info.workspace_bytes < p.info.workspace_bytes / 2


def test_calls_reject_bad_arguments_before_launch():
    """Null pointers, misalignment and short workspaces are refused on the host
    (no HIP call is made, so this runs without a GPU)."""
    p = sla.Plan(1, 2, 1024, 64, 0.25)
    L = sla.lib()
    big = p.info.workspace_bytes
    fake = ctypes.c_void_p(1 << 40)  # never dereferenced: validation fails first
    assert L.sla_quantize(p.handle, None, fake, fake, big, None) == sla.SLA_EINVAL
    assert L.sla_quantize(p.handle, fake, fake, None, big, None) == sla.SLA_EINVAL
    assert L.sla_quantize(p.handle, fake, fake, fake, big - 1, None) == sla.SLA_EWORKSPACE
    assert L.sla_quantize(p.handle, ctypes.c_void_p((1 << 40) + 2), fake, fake, big, None) == sla.SLA_EINVAL
    assert L.sla_quantize(p.handle, fake, fake, ctypes.c_void_p((1 << 40) + 16), big, None) == sla.SLA_EINVAL
    # linear branch on: the projection is required
    assert L.sla_attention_fwd(p.handle, fake, fake, fake, None, fake, fake, big, None) == sla.SLA_EINVAL
    assert L.sla_attention_fwd(p.handle, fake, fake, fake, fake, fake, fake, big - 256, None) == sla.SLA_EWORKSPACE
    assert L.sla_debug_qk_int32(p.handle, fake, None, 1, None, None) == sla.SLA_EINVAL
    assert L.sla_ws_view(p.handle, fake, 99, ctypes.byref(ctypes.c_void_p()),
                         ctypes.byref(ctypes.c_size_t())) == sla.SLA_EINVAL


def test_i8_unswizzle_is_a_permutation():
    x = np.arange(64 * 128).astype(np.int64)
    y = sla.i8_unswizzle(x, 128)
    assert sorted(y.ravel().tolist()) == list(range(64 * 128))
    x = np.arange(64 * 64).astype(np.int64)
    assert sorted(sla.i8_unswizzle(x, 64).ravel().tolist()) == list(range(64 * 64))


def test_workspace_bf16_qk_mode():
    """Plain SLA (bf16 QK^T) has no INT8 regions and a bf16 copy of K instead."""
    B, H, N, d = 1, 40, 75600, 128
    p8 = sla.Plan(B, H, N, d, 0.1)
    pb = sla.Plan(B, H, N, d, 0.1, qk_int8=False)
    assert pb.info.T == p8.info.T and pb.info.kb == p8.info.kb
    assert pb.ws_region(0, "Q8")[1] == 0 and pb.ws_region(0, "K8")[1] == 0
    T = pb.info.T
    # two INT8 [BH][T][64 d] regions out, one bf16 [BH][T][64 d] region in
    grow = pb.info.workspace_bytes - p8.info.workspace_bytes
    assert abs(grow) <= 4 * 256


def test_w8a8_argument_checks_without_gpu():
    """Host-side validation returns before any launch, so fake aligned
    addresses are safe here."""
    L = sla.lib()
    a = 1 << 20  # 16-byte aligned, never dereferenced
    assert L.sla_w8a8_gemm(None, a, a, a, 4, 4, 128, a, None) == sla.SLA_EINVAL
    assert L.sla_w8a8_gemm(a, a, a, a, 0, 4, 128, a, None) == sla.SLA_EINVAL
    assert L.sla_w8a8_gemm(a, a, a, a, 4, 4, 100, a, None) == sla.SLA_EUNSUPPORTED
    assert L.sla_w8a8_gemm(a + 8, a, a, a, 4, 4, 128, a, None) == sla.SLA_EINVAL
    assert L.sla_quant_b128(a, 4, 20, a, a, None) == sla.SLA_EUNSUPPORTED
    assert L.sla_quant_b128(a, 0, 16, a, a, None) == sla.SLA_EINVAL
    assert L.sla_quant_b128(None, 4, 16, a, a, None) == sla.SLA_EINVAL


def test_backward_workspace_and_argument_checks():
    """Backward plans add the transposed mask, rowsum(dO O), O_l, the two
    state-gradient arrays and the dW partials; forward-only plans refuse the
    backward call; bad arguments are refused on the host."""
    B, H, N, d = 1, 40, 75600, 128
    pf = sla.Plan(B, H, N, d, 0.1, qk_int8=False)
    pb = sla.Plan(B, H, N, d, 0.1, qk_int8=False, backward=True)
    T = pb.info.T
    BH = B * H
    F = (d * d + d + 127) // 128 * 128
    grow = pb.info.workspace_bytes - pf.info.workspace_bytes
    expect = (2 * BH * T * math.ceil(T / 64) * 8 + BH * T * 64 * 4 + 2 * BH * T * 64 * d * 2
              + 2 * BH * T * F * 2 + math.ceil(BH * T / 64) * d * d * 4 + 3 * BH * T * 64 * d * 4)
    assert 0 <= grow - expect <= 11 * 256
    assert pb.ws_region(0, "LSE")[1] == BH * T * 64 * 4
    L = sla.lib()
    fake = ctypes.c_void_p(1 << 40)  # never dereferenced: validation fails first
    big = pb.info.workspace_bytes
    args = [fake] * 9
    assert L.sla_attention_bwd(pf.handle, *args, fake, pf.info.workspace_bytes, None) == sla.SLA_EUNSUPPORTED
    assert L.sla_attention_bwd(pb.handle, *args, fake, big - 1, None) == sla.SLA_EWORKSPACE
    for k in range(9):
        a = list(args)
        if k in (3, 8):  # w_proj, dw: required while the linear branch is on
            a[k] = None
            assert L.sla_attention_bwd(pb.handle, *a, fake, big, None) == sla.SLA_EINVAL, k
            continue
        a[k] = None
        assert L.sla_attention_bwd(pb.handle, *a, fake, big, None) == sla.SLA_EINVAL, k
        a[k] = ctypes.c_void_p((1 << 40) + 8)
        assert L.sla_attention_bwd(pb.handle, *a, fake, big, None) == sla.SLA_EINVAL, k
    pn = sla.Plan(1, 2, 1000, 64, 0.3, use_linear=False, qk_int8=False, backward=True)
    assert pn.ws_region(0, "LSE")[1] == 2 * 16 * 64 * 4
