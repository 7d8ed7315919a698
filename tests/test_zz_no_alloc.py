"""sla_attention_fwd_noalloc (the forward on the library's static per-GPU
workspace, for callers that cannot allocate device memory) against
sla_quantize + sla_attention_fwd on a caller-allocated workspace, through the
C ABI: the same kernels on the same inputs, so the outputs are compared bit
for bit.  Several calls in a row share the static workspace; each later call
is smaller than the first, so it runs on what the earlier calls left there.
"""
import numpy as np
import pytest

from sparse_bit_attention_amd import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("no GPU", allow_module_level=True)

from sparse_bit_attention_amd import sla  # noqa: E402  (raises if the library is missing)


def say(*a):
    print(*a, flush=True)


def dev(a):
    t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16))
    return t.view(torch.bfloat16).cuda()


# (workload, qk mode): a call that fills most of the static workspace, then
# smaller ones (ragged N, the other head dim, fine scales, no linear branch,
# plain SLA with bf16 QK^T)
CALLS = [
    (synth.Workload("noalloc-big", 1, 2, 16384, 128, 0.1, seed=31), "int8"),
    (synth.Workload("noalloc-small", 1, 1, 1000, 128, 0.5, seed=32), "int8"),
    (synth.Workload("noalloc-d64", 2, 2, 2500, 64, 0.3, use_linear=0, seed=33), "int8-fine"),
    (synth.Workload("noalloc-bf16", 1, 2, 3000, 128, 0.2, seed=35), "bf16"),
]


def test_noalloc_matches_workspace_entry_point():
    for n, (wl, mode) in enumerate(CALLS):
        q, k, v, w = synth.all_inputs(wl)
        Q, K, V, W = dev(q), dev(k), dev(v), dev(w)
        Wp = W if wl.use_linear else None
        m = sla.SageSLA(wl.B, wl.H, wl.N, wl.d, wl.topk, use_linear=bool(wl.use_linear),
                        qk_int8=mode != "bf16", qk_fine=mode == "int8-fine")
        need = m.plan.info.workspace_bytes
        assert need <= sla.NOALLOC_WS_BYTES
        if n > 0:
            assert need < first_need
        else:
            first_need = need
        say(f"[gpu] noalloc call {n}: {wl.name} B={wl.B} H={wl.H} N={wl.N} d={wl.d} "
            f"topk={wl.topk} lin={wl.use_linear} qk={mode} workspace={need} bytes")
        ref = m.forward(Q, K, V, Wp)
        got = torch.full_like(Q, float("nan"))
        sla.attention_fwd_noalloc(m.plan, Q, K, V, Wp, got)
        torch.cuda.synchronize()
        assert torch.equal(got.view(torch.int16), ref.view(torch.int16)), wl.name
        del m


def test_noalloc_rejects_what_does_not_fit():
    wl = synth.Workload("noalloc-too-big", 1, 3, 16000, 128, 0.2, seed=34)
    plan = sla.Plan(wl.B, wl.H, wl.N, wl.d, wl.topk)
    assert plan.info.workspace_bytes > sla.NOALLOC_WS_BYTES
    x = torch.zeros((wl.B, wl.H, wl.N, wl.d), dtype=torch.bfloat16, device="cuda")
    w = torch.zeros((wl.d, wl.d), dtype=torch.bfloat16, device="cuda")
    out = torch.full_like(x, 7.0)
    with pytest.raises(sla.SlaError) as e:
        sla.attention_fwd_noalloc(plan, x, x, x, w, out)
    assert e.value.status == sla.SLA_ETOOLARGE
    # a linear-branch plan without its projection: rejected before any launch
    small = sla.Plan(1, 1, 256, 64, 0.5)
    xs = torch.zeros((1, 1, 256, 64), dtype=torch.bfloat16, device="cuda")
    outs = torch.full_like(xs, 7.0)
    L = sla.lib()
    import ctypes
    p = lambda t: ctypes.c_void_p(t.data_ptr())
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    assert L.sla_attention_fwd_noalloc(small.handle, p(xs), p(xs), p(xs), None, p(outs), st) \
        == sla.SLA_EINVAL
    torch.cuda.synchronize()
    assert bool((out == 7.0).all()) and bool((outs == 7.0).all())
