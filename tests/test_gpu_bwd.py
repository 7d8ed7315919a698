"""GPU parity of the plain-SLA backward (sla_attention_bwd) against the float64
oracle in oracle/backward.py, through the C ABI.

Tolerance (derived from the arithmetic: bf16 operands and outputs, P and dS
rounded to bf16 for their products, linear states and their gradients stored
as bf16, float32 sums): for each of dQ, dK, dV and dW, relative L2 error
<= 1e-2 and max-abs error <= 2e-2 times the largest reference magnitude.
The measured errors are printed and are several times smaller.  The forward's
row normalisers (LSE region) are checked against the oracle's to 2e-2 in
log2 units.
"""
import math

import numpy as np
import pytest

import oracle
from oracle import backward as obwd
from sparse_bit_attention_amd import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("no GPU", allow_module_level=True)

from sparse_bit_attention_amd import sla  # noqa: E402  (raises if the library is missing)

REL_L2, MAX_REL = 1e-2, 2e-2


def say(*a):
    print(*a, flush=True)


def dev(a):
    t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16))
    return t.view(torch.bfloat16).cuda()


def host_f64(t):
    if t.dtype == torch.bfloat16:
        b = t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
        return synth.bf16_bits_to_f32(b).astype(np.float64)
    return t.cpu().numpy().astype(np.float64)


def f64(b):
    return synth.bf16_bits_to_f32(b).astype(np.float64)


def unpack_mask(words, T):
    bits = np.unpackbits(np.ascontiguousarray(words).view(np.uint8).reshape(*words.shape, 8),
                         axis=-1, bitorder="little")
    return bits.reshape(words.shape[0], -1)[:, :T]


def close(got, ref, label):
    err = np.abs(got - ref)
    mx = float(err.max()) if err.size else 0.0
    scale = float(np.abs(ref).max()) if ref.size else 0.0
    nrm = float(np.linalg.norm(ref))
    rel = float(np.linalg.norm(got - ref) / nrm) if nrm > 0 else 0.0
    say(f"[parity] {label}: rel-L2 {rel:.3e} max-abs {mx:.3e} (max |ref| {scale:.3e})")
    if nrm > 0 and got.ndim == 2 and rel > REL_L2:  # where the error sits
        rows = np.argsort(-np.linalg.norm(got - ref, axis=1))[:6]
        for r in rows:
            say(f"    row {r}: |err| {np.linalg.norm(got[r] - ref[r]):.3e} |ref| "
                f"{np.linalg.norm(ref[r]):.3e} |got| {np.linalg.norm(got[r]):.3e}")
    assert np.all(np.isfinite(got))
    if nrm > 0:
        assert rel <= REL_L2
        assert mx <= MAX_REL * scale
    else:
        assert mx == 0.0


def run_bwd(wl, sm_scale=0.0):
    q, k, v, w = synth.all_inputs(wl)
    do = synth.grad_output(wl)
    Q, K, V, W, dO = dev(q), dev(k), dev(v), dev(w), dev(do)
    m = sla.SageSLA(wl.B, wl.H, wl.N, wl.d, wl.topk, use_linear=bool(wl.use_linear),
                    sm_scale=sm_scale, qk_int8=False, backward=True)
    say(f"[gpu] backward {wl.name} B={wl.B} H={wl.H} N={wl.N} d={wl.d} topk={wl.topk} "
        f"lin={wl.use_linear} kb={m.plan.info.kb}")
    o = m(Q, K, V, W if wl.use_linear else None)
    dq, dk, dv, dw = m.backward(Q, K, V, W if wl.use_linear else None, dO)
    torch.cuda.synchronize()
    return m, (q, k, v, w, do), o, (dq, dk, dv, dw)


def full_compare(wl, sm_scale=0.0):
    m, (q, k, v, w, do), o, (dq, dk, dv, dw) = run_bwd(wl, sm_scale)
    T = m.plan.info.T
    sc = sm_scale if sm_scale > 0 else oracle.default_sm_scale(wl.d)
    gq, gk, gv = host_f64(dq), host_f64(dk), host_f64(dv)
    lse = m.region("LSE").cpu().numpy().astype(np.float64)
    masks = unpack_mask(m.region("MASK").cpu().numpy().reshape(wl.B * wl.H * T, -1), T)
    R = {"dQ": [], "dK": [], "dV": []}
    G = {"dQ": [], "dK": [], "dV": []}
    dW = np.zeros((wl.d, wl.d))
    lse_err = 0.0
    for b, h in wl.heads():
        bh = b * wl.H + h
        prep = oracle.head_prep(q[b, h], k[b, h], float(np.float32(wl.topk)))
        mask = masks[bh * T:(bh + 1) * T]
        assert np.array_equal(mask, prep.mask)
        Qf, Kf, Vf, Wf, dOf = f64(q[b, h]), f64(k[b, h]), f64(v[b, h]), f64(w), f64(do[b, h])
        fwd = obwd.forward(Qf, Kf, Vf, Wf, mask.astype(bool), sc, bool(wl.use_linear))
        g = obwd.backward(Qf, Kf, Vf, Wf, dOf, mask.astype(bool), sc, bool(wl.use_linear), fwd=fwd)
        for name, ref, got in (("dQ", g.dQ, gq[b, h]), ("dK", g.dK, gk[b, h]), ("dV", g.dV, gv[b, h])):
            R[name].append(ref)
            G[name].append(got)
        dW += g.dW
        if m.plan.info.kb > 0:
            ref_l2 = fwd.lse * math.log2(math.e)
            got_l2 = lse[bh].reshape(-1)[:wl.N]
            lse_err = max(lse_err, float(np.abs(got_l2 - ref_l2).max()))
    for name in ("dQ", "dK", "dV"):
        close(np.concatenate(G[name]), np.concatenate(R[name]), f"{wl.name} {name}")
    if wl.use_linear:
        close(host_f64(dw), dW, f"{wl.name} dW")
    else:
        assert dw is None
    say(f"[parity] {wl.name} LSE: max-abs {lse_err:.3e} (log2 units)")
    assert lse_err <= 2e-2


SMALL = [
    synth.Workload("bwd-tiny", 1, 2, 1024, 64, 0.25, seed=41),
    synth.Workload("bwd-d128-ragged", 1, 2, 1000, 128, 0.25, seed=42),
    synth.Workload("bwd-two-blocks", 1, 1, 65, 64, 0.5, seed=43),
    synth.Workload("bwd-one-token", 1, 1, 1, 128, 0.1, seed=44),
    synth.Workload("bwd-pure-linear", 1, 2, 700, 128, 0.0, seed=45),
    synth.Workload("bwd-all-kept", 1, 1, 640, 128, 1.0, seed=46),
    synth.Workload("bwd-sparse-only-b2", 2, 1, 2000, 128, 0.3, use_linear=0, seed=47),
    synth.Workload("bwd-sparse-only-d64", 1, 2, 1500, 64, 0.2, use_linear=0, seed=48),
    synth.Workload("bwd-b2h2", 2, 2, 1300, 128, 0.2, seed=49),
    # logits ~6x sharper: the forward's logit bound fails, so its rows go
    # through the exact-row-max launch (which then writes their LSE)
    synth.Workload("bwd-sharp", 1, 1, 2000, 128, 0.2, seed=50, q_std=6.0),
]


@pytest.mark.parametrize("wl", SMALL, ids=[w.name for w in SMALL])
def test_backward_small_full_parity(wl):
    full_compare(wl)


def test_backward_explicit_sm_scale():
    full_compare(synth.Workload("bwd-scale", 1, 1, 777, 128, 0.2, seed=51), sm_scale=0.05)


def test_backward_deterministic_and_repeatable():
    """Two backward calls on the same forward give identical bits (no atomics)."""
    wl = synth.Workload("bwd-det", 1, 2, 1500, 128, 0.2, seed=52)
    m, (q, k, v, w, do), o, g1 = run_bwd(wl)
    Q, K, V, W, dO = dev(q), dev(k), dev(v), dev(w), dev(do)
    g2 = m.backward(Q, K, V, W, dO)
    torch.cuda.synchronize()
    for a, b in zip(g1, g2):
        assert torch.equal(a.view(torch.int32) if a.dtype == torch.float32 else a.view(torch.int16),
                           b.view(torch.int32) if b.dtype == torch.float32 else b.view(torch.int16))


def test_backward_is_linear_in_dout():
    """The gradients are linear in dO with P fixed: scaling dO by 2 scales dQ, dK, dV, dW
    by 2 exactly (powers of two commute with every rounding)."""
    wl = synth.Workload("bwd-lin", 1, 1, 1200, 64, 0.25, seed=53)
    m, (q, k, v, w, do), o, g1 = run_bwd(wl)
    Q, K, V, W = dev(q), dev(k), dev(v), dev(w)
    dO2 = (dev(do).float() * 2.0).to(torch.bfloat16)
    g2 = m.backward(Q, K, V, W, dO2)
    torch.cuda.synchronize()
    for a, b in zip(g1, g2):
        assert torch.equal((a.float() * 2.0).to(a.dtype), b)


def test_backward_needs_backward_plan():
    wl = synth.Workload("bwd-noplan", 1, 1, 300, 64, 0.5, seed=54)
    q, k, v, w = synth.all_inputs(wl)
    Q, K, V, W = dev(q), dev(k), dev(v), dev(w)
    m = sla.SageSLA(wl.B, wl.H, wl.N, wl.d, wl.topk, qk_int8=False)
    o = m(Q, K, V, W)
    with pytest.raises(sla.SlaError):
        m.backward(Q, K, V, W, o)


# ---------------------------------------------------------------- full size ---

def sampled_compare(wl, heads, check_dw):
    say(f"[gpu] generating {wl.name}")
    m, (q, k, v, w, do), o, (dq, dk, dv, dw) = run_bwd(wl)
    T = m.plan.info.T
    sc = oracle.default_sm_scale(wl.d)
    for t in (dq, dk, dv):
        assert bool(torch.isfinite(t.float()).all())
    qbl = sorted({0, 1, T // 2, T - 1})
    kbl = sorted({0, T // 2, T - 1})
    masks = unpack_mask(m.region("MASK").cpu().numpy().reshape(wl.B * wl.H * T, -1), T)
    G = {"dQ": [], "dK": [], "dV": []}
    R = {"dQ": [], "dK": [], "dV": []}
    dW = np.zeros((wl.d, wl.d))
    for b, h in heads:
        bh = b * wl.H + h
        # the reference takes the oracle's own selection; the GPU plan's mask
        # must equal it bit for bit before it is used
        prep = oracle.head_prep(q[b, h], k[b, h], float(np.float32(wl.topk)))
        assert np.array_equal(masks[bh * T:(bh + 1) * T], prep.mask), f"mask of head {(b, h)}"
        mask = prep.mask.astype(bool)
        rq, rk, rv, rw = obwd.backward_sampled(f64(q[b, h]), f64(k[b, h]), f64(v[b, h]), f64(w),
                                               f64(do[b, h]), mask, sc, qbl, kbl,
                                               bool(wl.use_linear))
        dW += rw
        hq = dq[b, h]
        for i in qbl:
            n = rq[i].shape[0]
            G["dQ"].append(host_f64(hq[64 * i:64 * i + n]))
            R["dQ"].append(rq[i])
        for j in kbl:
            n = rk[j].shape[0]
            G["dK"].append(host_f64(dk[b, h, 64 * j:64 * j + n]))
            R["dK"].append(rk[j])
            G["dV"].append(host_f64(dv[b, h, 64 * j:64 * j + n]))
            R["dV"].append(rv[j])
    for name in ("dQ", "dK", "dV"):
        close(np.concatenate(G[name]), np.concatenate(R[name]), f"{wl.name} {name} (sampled)")
    if check_dw:
        close(host_f64(dw), dW, f"{wl.name} dW")


def test_backward_wan14b_720p_sampled():
    """The Wan2.1-14B 720P layer (40 heads, N = 75600, topk 0.1) in the launch
    configuration the backward benchmark times; dQ rows of four query blocks
    and dK, dV rows of three key blocks (first, middle, ragged last) on two heads."""
    wl = synth.WORKLOADS["wan14b-720p"]
    sampled_compare(wl, [(0, 0), (0, wl.H - 1)], check_dw=False)


def test_backward_full_length_two_heads_dw():
    """Full 720P sequence length with two heads, so the oracle can also form
    the whole projection gradient (a sum over every row of every head)."""
    wl = synth.Workload("wan14b-720p-h2", 1, 2, 21 * 45 * 80, 128, 0.1)
    sampled_compare(wl, wl.heads(), check_dw=True)


def test_backward_plan_forward_is_unchanged():
    """A backward plan's forward also stores the row normalisers and O_sparse;
    its output is bit-identical to a forward-only plan's."""
    wl = synth.Workload("bwd-fwd-same", 1, 2, 1500, 128, 0.2, seed=55)
    q, k, v, w = synth.all_inputs(wl)
    Q, K, V, W = dev(q), dev(k), dev(v), dev(w)
    outs = []
    for backward in (False, True):
        m = sla.SageSLA(wl.B, wl.H, wl.N, wl.d, wl.topk, qk_int8=False, backward=backward)
        outs.append(m(Q, K, V, W))
    torch.cuda.synchronize()
    assert torch.equal(outs[0].view(torch.int16), outs[1].view(torch.int16))
