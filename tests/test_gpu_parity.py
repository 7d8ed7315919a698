"""GPU parity of the HIP path against the CPU oracle, through the C ABI.

Bit-exact: block means and sums, K mean, mask bits, kept lists, INT8 codes and
scales, int32 QK^T tiles.  Outputs: max-abs <= 2e-2 and relative L2 <= 1e-2
against the float64 oracle (the bar the operator is specified with); the
measured values are printed and are far below it.

Small cases compare every head and every query block.  The Wan-shaped
workloads run at full size in the launch configuration the benchmark times
and compare sampled heads (all masks and codes of those heads) and sampled
query blocks (outputs), plus properties checked on every head.
"""
import math

import numpy as np
import pytest

import oracle
from sparse_bit_attention_amd import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("no GPU", allow_module_level=True)

from sparse_bit_attention_amd import sla  # noqa: E402  (raises if the library is missing)

MAX_ABS, REL_L2 = 2e-2, 1e-2


def say(*a):
    print(*a, flush=True)


def dev(a):
    t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16))
    return t.view(torch.bfloat16).cuda()


def host_u16(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def f32(b):
    return synth.bf16_bits_to_f32(b).astype(np.float64)


def qk_label(qk_int8, fine):
    return ("int8-fine" if fine else "int8") if qk_int8 else "bf16"


def run(wl: synth.Workload, inputs=None, sm_scale=0.0, out=None, qk_int8=True, fine=False):
    if inputs is None:
        inputs = synth.all_inputs(wl)
    q, k, v, w = inputs
    Q, K, V, W = dev(q), dev(k), dev(v), dev(w)
    m = sla.SageSLA(wl.B, wl.H, wl.N, wl.d, wl.topk, use_linear=bool(wl.use_linear),
                    sm_scale=sm_scale, qk_int8=qk_int8, qk_fine=fine)
    say(f"[gpu] forward {wl.name} B={wl.B} H={wl.H} N={wl.N} d={wl.d} topk={wl.topk} "
        f"lin={wl.use_linear} kb={m.plan.info.kb} qk={qk_label(qk_int8, fine)}")
    o = m(Q, K, V, W if wl.use_linear else None, out=out)
    torch.cuda.synchronize()
    return m, o, (Q, K, V, W), inputs


def unpack_mask(words, T):
    bits = np.unpackbits(np.ascontiguousarray(words).view(np.uint8).reshape(*words.shape, 8),
                         axis=-1, bitorder="little")
    return bits.reshape(words.shape[0], -1)[:, :T]


def check_head_prep(m, wl, b, h, Qh, Kh, qk_int8=True, fine=False):
    bh = b * wl.H + h
    prep = oracle.head_prep(Qh, Kh, float(np.float32(wl.topk)), fine=fine)
    T, kb, d = m.plan.info.T, m.plan.info.kb, wl.d
    g = {r: m.region(r)[bh].cpu().numpy() for r in ("QBAR", "KSUM", "KBAR", "MU", "DQ", "DK")}
    assert np.array_equal(g["QBAR"].view(np.uint32), prep.qbar.view(np.uint32))
    assert np.array_equal(g["KSUM"].view(np.uint32), prep.ksum.view(np.uint32))
    assert np.array_equal(g["KBAR"].view(np.uint32), prep.kbar.view(np.uint32))
    assert np.array_equal(g["MU"].view(np.uint32), prep.mu.view(np.uint32))
    mask = unpack_mask(m.region("MASK")[bh].cpu().numpy(), T)
    assert np.array_equal(mask, prep.mask), f"mask differs in {int((mask != prep.mask).sum())} places"
    if kb:
        assert np.array_equal(m.region("KEPT")[bh].cpu().numpy(), prep.kept)
    if not qk_int8:  # plain SLA: no INT8 step, unit key-block scales
        assert np.all(g["DK"] == 1.0)
        return prep
    q8 = sla.i8_unswizzle(m.region("Q8")[bh].cpu().numpy(), d).reshape(T * 64, d)
    k8 = sla.i8_unswizzle(m.region("K8")[bh].cpu().numpy(), d).reshape(T * 64, d)
    assert np.array_equal(q8, prep.q8)
    assert np.array_equal(k8, prep.k8)
    assert np.array_equal(g["DQ"].view(np.uint32), prep.dq.view(np.uint32))
    assert np.array_equal(g["DK"].view(np.uint32), prep.dk.view(np.uint32))
    return prep


def compare_blocks(o_head, wl, Qh, Kh, Vh, W, prep, blocks, sm_scale=None, qk_int8=True):
    res = oracle.head_forward(Qh, Kh, Vh, W, float(np.float32(wl.topk)),
                              use_linear=bool(wl.use_linear), blocks=blocks, prep=prep,
                              sm_scale=sm_scale, qk_int8=qk_int8)
    got, ref = [], []
    for i in blocks:
        n = res[i].shape[0]
        got.append(f32(o_head[64 * i:64 * i + n]))
        ref.append(res[i])
    got, ref = np.concatenate(got), np.concatenate(ref)
    return got, ref


def assert_close(got, ref, label):
    err = np.abs(got - ref)
    mx = float(err.max()) if err.size else 0.0
    rms = float(np.sqrt((ref ** 2).mean())) if ref.size else 0.0
    rel = float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300))
    say(f"[parity] {label}: max-abs {mx:.3e} rel-L2 {rel:.3e} max-abs/rms {mx / max(rms, 1e-300):.3e}")
    assert np.all(np.isfinite(got))
    assert mx <= MAX_ABS
    if np.linalg.norm(ref) > 0:
        assert rel <= REL_L2
    else:
        assert mx == 0.0


def full_compare(wl, sm_scale=0.0, inputs=None, qk_int8=True, fine=False):
    m, o, dv, inputs = run(wl, inputs=inputs, sm_scale=sm_scale, qk_int8=qk_int8, fine=fine)
    q, k, v, w = inputs
    out = host_u16(o)
    scale = sm_scale if sm_scale > 0 else None
    G, R = [], []
    for b, h in wl.heads():
        prep = check_head_prep(m, wl, b, h, q[b, h], k[b, h], qk_int8=qk_int8, fine=fine)
        got, ref = compare_blocks(out[b, h], wl, q[b, h], k[b, h], v[b, h], w, prep,
                                  list(range(m.plan.info.T)), sm_scale=scale, qk_int8=qk_int8)
        G.append(got)
        R.append(ref)
    assert_close(np.concatenate(G), np.concatenate(R), f"{wl.name} ({qk_label(qk_int8, fine)})")
    return m, o, dv, inputs


SMALL = [
    synth.Workload("tiny", 1, 2, 1024, 64, 0.25),
    synth.Workload("tiny-d128-ragged", 1, 2, 1000, 128, 0.25),
    synth.Workload("two-blocks", 1, 1, 65, 64, 0.5),
    synth.Workload("one-token", 1, 1, 1, 128, 0.1),
    synth.Workload("pure-linear", 1, 2, 700, 128, 0.0),
    synth.Workload("all-kept-linear-on", 1, 1, 640, 128, 1.0),
    synth.Workload("sparse-only-b2", 2, 1, 2000, 128, 0.3, use_linear=0),
    synth.Workload("dense-outlier-small", 1, 2, 2048, 128, 1.0, use_linear=0, koff_std=4.0,
                   outlier_frac=0.01, outlier_scale=20.0),
    synth.Workload("preview-topk", 1, 1, 4000, 128, 0.05, seed=5),
    synth.Workload("quality-topk", 1, 1, 4000, 64, 0.15, seed=6),
    # logits ~6x sharper: the per-row logit bound exceeds its limit, so these
    # query blocks go through the online-max attention launch
    synth.Workload("sharp-online-max", 1, 2, 3000, 128, 0.2, seed=11, q_std=6.0),
    synth.Workload("sharp-online-max-d64", 1, 1, 2000, 64, 0.3, seed=12, q_std=8.0),
]


@pytest.mark.parametrize("wl", SMALL, ids=[w.name for w in SMALL])
def test_small_full_parity(wl):
    full_compare(wl)


def tied_inputs(wl, period):
    """Synthetic inputs whose K block j repeats K block j % period: key blocks
    with equal means give equal scores, so every row has ties at its
    threshold (broken towards the lower block index)."""
    q, k, v, w = synth.all_inputs(wl)
    k = k.copy()
    for j in range(period, wl.T):
        n = min(64, wl.N - 64 * j)
        s = j % period
        k[:, :, 64 * j:64 * j + n] = k[:, :, 64 * s:64 * s + n]
    return q, k, v, w


@pytest.mark.parametrize("period", [3, 40])
def test_tied_block_scores(period):
    # period 3: a third of all scores share each value (many candidates at
    # the threshold); period 40: pairs of equal scores near the threshold
    wl = synth.Workload(f"ties-{period}", 1, 2, 64 * 64, 128, 0.3, seed=13)
    full_compare(wl, inputs=tied_inputs(wl, period))


def anti_aligned_inputs(wl, beta, seed):
    """Every query block keeps key blocks 0 .. T/2-1 (block means: channel 0
    of Q is 1, of those keys +1, of the others -1).  Channel 1 alternates
    +beta / -beta over the query rows, is -beta on the kept keys and +beta on
    the others (so the K mean stays ~0): the even rows' logits over their
    kept keys all sit near minus their Cauchy-Schwarz bound (about
    0.1275 beta^2 in log2 units), the odd rows' near plus it."""
    rng = np.random.default_rng(seed)
    N, d = wl.N, wl.d
    q = rng.standard_normal((N, d)) * 0.05
    k = rng.standard_normal((N, d)) * 0.05
    q[:, 0] = 1.0
    q[:, 1] = np.where(np.arange(N) % 2 == 0, beta, -beta)
    kept = np.arange(N) < 64 * (wl.T // 2)
    k[:, 0] = np.where(kept, 1.0, -1.0)
    k[:, 1] = np.where(kept, -beta, beta)
    _, _, v, w = synth.all_inputs(wl)
    return (synth.f64_to_bf16_bits(q).reshape(1, 1, N, d),
            synth.f64_to_bf16_bits(k).reshape(1, 1, N, d), v, w)


@pytest.mark.parametrize("qk", ["int8", "int8-fine", "bf16"])
@pytest.mark.parametrize("beta", [17.75, 22.25])
def test_rows_with_every_kept_logit_near_minus_the_bound(beta, qk):
    """Rows whose kept logits all lie near -m, m their logit bound: with
    beta = 17.75 (m ~ 40) they stay in the bound launch and their
    probabilities are ~2^-80; with beta = 22.25 (m ~ 63, where 2^(-2m) would
    leave the float32 normal range) they must go to the second launch.  Both
    match the oracle."""
    wl = synth.Workload(f"anti-aligned-{beta}", 1, 1, 512, 128, 0.5, use_linear=0, seed=21)
    inputs = anti_aligned_inputs(wl, beta, seed=22)
    prep = oracle.head_prep(inputs[0][0, 0], inputs[1][0, 0], 0.5)
    assert np.array_equal(prep.kept, np.tile(np.arange(4), (wl.T, 1)))
    full_compare(wl, inputs=inputs, qk_int8=qk != "bf16", fine=qk == "int8-fine")


def test_kmean_block_order_hand_case():
    """The hand case of tests/golden/hand_cases.json (kmean_order), scaled by
    2^-20 (exact: no value becomes subnormal) so the logits stay moderate: the
    K mean must be the block-order float32 sum of the block sums; a reversed
    block order, a token-order or a float64 sum give different bits."""
    import json
    import os
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "hand_cases.json")))["kmean_order"]
    wl = synth.Workload("kmean-order", 1, 1, g["N"], 128, 0.5, seed=23)
    q, _, v, w = synth.all_inputs(wl)
    kf = np.zeros((wl.N, wl.d))
    for r, val in g["rows_and_values"]:
        kf[r, :] = val * 2.0 ** -20
    k = synth.f64_to_bf16_bits(kf).reshape(1, 1, wl.N, wl.d)
    m, o, dv, inputs = full_compare(wl, inputs=(q, k, v, w))
    mu = m.region("MU")[0].cpu().numpy()
    assert np.all(mu == np.float32(g["mu"] * 2.0 ** -20))


def test_explicit_sm_scale():
    full_compare(synth.Workload("scale", 1, 1, 777, 128, 0.2, seed=9), sm_scale=0.05)


@pytest.mark.parametrize("d", [128, 64])
def test_int32_qk_tiles_bit_exact(d):
    """The score accumulators of the attention kernel's own bound-path loop,
    read back, equal the exact int32 products of the oracle's codes (the last
    block, 15, is ragged: 40 keys)."""
    wl = synth.Workload("qk", 1, 2, 1000, d, 0.5, seed=2)
    m, o, dv, (q, k, v, w) = run(wl)
    T = m.plan.info.T
    triples = [(0, 0, 0), (0, 3, 15), (1, 15, 15), (1, 7, 2), (0, 15, 0)]
    tiles = m.debug_qk_int32(triples).cpu().numpy()
    for n, (bh, i, j) in enumerate(triples):
        prep = oracle.head_prep(q[0, bh], k[0, bh], float(np.float32(wl.topk)))
        ref = oracle.qk_int32(prep.q8, prep.k8, i, j)
        assert np.array_equal(tiles[n], ref), (bh, i, j)
    bad = m.debug_qk_int32([(5, 0, 0), (0, T, 0)]).cpu().numpy()
    assert np.all(bad == 0)


def test_deterministic_reruns():
    wl = synth.Workload("det", 1, 2, 3000, 128, 0.1, seed=4)
    m, o1, dv, inputs = run(wl)
    o2 = m(*dv)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))


def test_value_scaling_by_power_of_two_is_exact():
    wl = synth.Workload("scale2", 1, 2, 1500, 128, 0.2, seed=8)
    m, o1, (Q, K, V, W), _ = run(wl)
    o2 = m(Q, K, (V.float() * 4.0).to(torch.bfloat16), W)
    torch.cuda.synchronize()
    assert torch.equal((o1.float() * 4.0).to(torch.bfloat16).view(torch.int16), o2.view(torch.int16))


def test_head_permutation_equivariance():
    wl = synth.Workload("perm", 1, 3, 1300, 64, 0.25, seed=7)
    m, o, (Q, K, V, W), _ = run(wl)
    perm = [2, 0, 1]
    o2 = m(Q[:, perm].contiguous(), K[:, perm].contiguous(), V[:, perm].contiguous(), W)
    torch.cuda.synchronize()
    assert torch.equal(o[:, perm].contiguous().view(torch.int16), o2.view(torch.int16))


# ------------------------------------------------ plain SLA (bf16 QK^T) ---

# The same small workloads with QK^T in bf16: the oracle's exact-logit mode.
# dense-outlier-small and the sharp workloads have per-row logit bounds past
# the limit, so their query blocks go through the exact-row-max launch.
SMALL_BF16 = [w for w in SMALL if w.name in (
    "tiny", "tiny-d128-ragged", "two-blocks", "one-token", "pure-linear", "all-kept-linear-on",
    "sparse-only-b2", "dense-outlier-small", "quality-topk", "sharp-online-max",
    "sharp-online-max-d64")]


@pytest.mark.parametrize("wl", SMALL_BF16, ids=[w.name for w in SMALL_BF16])
def test_sla_bf16_small_full_parity(wl):
    full_compare(wl, qk_int8=False)


def test_sla_bf16_debug_qk_unsupported():
    wl = synth.Workload("qk-bf16", 1, 1, 300, 64, 0.5, seed=3)
    m, o, dv, _ = run(wl, qk_int8=False)
    with pytest.raises(sla.SlaError):
        m.debug_qk_int32([(0, 0, 0)])


# ---------------------------------------------------------------- full size ---

BIG = ["wan1.3b-480p", "wan14b-480p", "wan14b-720p", "dense-outlier"]


def mask_properties(m):
    """Every row of every head keeps exactly kb blocks, listed ascending."""
    T, kb = m.plan.info.T, m.plan.info.kb
    words = m.region("MASK")
    cnt = torch.zeros(words.shape[:2], dtype=torch.int64, device=words.device)
    for b in range(64):
        cnt += ((words >> b) & 1).sum(-1)
    assert bool((cnt == kb).all())
    kept = m.region("KEPT")
    if kb > 1:
        assert bool((kept[:, :, 1:] > kept[:, :, :-1]).all())
    if kb:
        assert bool((kept[:, :, 0] >= 0).all()) and bool((kept[:, :, -1] < T).all())


@pytest.mark.parametrize("name", BIG)
def test_full_size_sampled_parity(name):
    wl = synth.WORKLOADS[name]
    say(f"[gpu] generating {name}")
    inputs = synth.all_inputs(wl)
    m, o, dv, _ = run(wl, inputs=inputs)
    mask_properties(m)
    assert bool(torch.isfinite(o.float()).all())
    q, k, v, w = inputs
    out = host_u16(o)
    T = m.plan.info.T
    blocks = sorted({0, 1, T // 2, T - 1})
    heads = [(0, 0), (wl.B - 1, wl.H - 1)]
    G, R = [], []
    for b, h in heads:
        prep = check_head_prep(m, wl, b, h, q[b, h], k[b, h])
        got, ref = compare_blocks(out[b, h], wl, q[b, h], k[b, h], v[b, h], w, prep, blocks)
        G.append(got)
        R.append(ref)
        bh = b * wl.H + h
        pairs = [(bh, i, int(prep.kept[i][0])) for i in blocks if prep.kept.shape[1]]
        tiles = m.debug_qk_int32(pairs).cpu().numpy()
        for n, (_, i, j) in enumerate(pairs):
            assert np.array_equal(tiles[n], oracle.qk_int32(prep.q8, prep.k8, i, j))
    assert_close(np.concatenate(G), np.concatenate(R), name)
    if name == "wan14b-720p":
        # head sharding: one GPU's share (heads 0..4) alone gives exactly
        # those heads of the full layer, bit for bit
        sw = synth.WORKLOADS["wan14b-720p-shard8"]
        del m, o, dv
        torch.cuda.empty_cache()
        _, os_, _, _ = run(sw, inputs=(q[:, :sw.H], k[:, :sw.H], v[:, :sw.H], w))
        assert np.array_equal(host_u16(os_), out[:, :sw.H])


def test_long_sequence_selection():
    """T = 2188 key blocks, more than the 2048 whose keys a selection wave
    holds in registers (the selection then re-reads them each pass): masks,
    kept lists, means and codes bit-exact on the head, outputs at the bar on
    sampled blocks (ragged last block: 32 rows)."""
    wl = synth.Workload("long", 1, 1, 140000, 64, 0.02, seed=41)
    inputs = synth.all_inputs(wl)
    m, o, dv, _ = run(wl, inputs=inputs)
    assert m.plan.info.T == 2188
    mask_properties(m)
    q, k, v, w = inputs
    T = m.plan.info.T
    prep = check_head_prep(m, wl, 0, 0, q[0, 0], k[0, 0])
    got, ref = compare_blocks(host_u16(o)[0, 0], wl, q[0, 0], k[0, 0], v[0, 0], w, prep,
                              sorted({0, 1, T // 2, T - 1}))
    assert_close(got, ref, wl.name)


@pytest.mark.parametrize("N", [44000, 64000, 96000, 108800, 128000])
def test_selection_register_buckets(N):
    """Selection holds ceil(T/64) keys per lane in 12, 16, 24, 28 or 32
    registers (T = 688, 1000, 1500, 1700, 2000): masks, kept lists, means and
    codes of the head bit-exact."""
    wl = synth.Workload(f"sel{N}", 1, 1, N, 64, 0.07, use_linear=0, seed=N % 997)
    inputs = synth.all_inputs(wl)
    m, o, dv, _ = run(wl, inputs=inputs)
    mask_properties(m)
    q, k, v, w = inputs
    check_head_prep(m, wl, 0, 0, q[0, 0], k[0, 0])


def test_dense_outlier_against_float64_dense_attention():
    """The dense INT8 stress workload (topk 1, no linear branch, K offsets
    ~N(0,16) with one channel x20) at full size against float64 dense softmax
    attention of the same bf16 inputs (the oracle's exact-logit mode), on
    sampled query blocks of two heads, with block scales and with fine scales.
    This is an accuracy characterisation of INT8 QK^T, not the GPU-versus-
    oracle bar: quantisation alone puts the output ~1.3e-2 (block scales) and
    ~1.15e-2 (16-row / 4-key scales) from float64 in relative L2, the oracle's
    analytic model and its own pin agree, and the assertion is that model's
    bound (2e-2) plus max-abs 2e-2."""
    wl = synth.WORKLOADS["dense-outlier"]
    say(f"[gpu] generating {wl.name}")
    inputs = synth.all_inputs(wl)
    q, k, v, w = inputs
    T = wl.T
    blocks = [0, 1, T // 2, T - 1]
    heads = [(0, 0), (wl.B - 1, wl.H - 1)]
    ref = []
    for b, h in heads:
        exact = oracle.head_forward(q[b, h], k[b, h], v[b, h], w, 1.0, use_linear=False,
                                    blocks=blocks, qk_int8=False)
        ref.append(np.concatenate([exact[i] for i in blocks]))
    ref = np.concatenate(ref)
    errs = {}
    for fine in (False, True):
        m, o, _, _ = run(wl, inputs=inputs, fine=fine)
        out = host_u16(o)
        got = np.concatenate([f32(out[b, h, 64 * i:64 * i + min(64, wl.N - 64 * i)])
                              for b, h in heads for i in blocks])
        mx = float(np.abs(got - ref).max())
        errs[fine] = float(np.linalg.norm(got - ref) / np.linalg.norm(ref))
        say(f"[accuracy] dense-outlier vs float64 dense, {'fine' if fine else 'block'} scales: "
            f"rel-L2 {errs[fine]:.3e} max-abs {mx:.3e}")
        assert mx <= MAX_ABS and errs[fine] <= 2e-2
        del m, o
    assert errs[True] < errs[False]


@pytest.mark.parametrize("name", ["wan14b-720p"])
def test_sla_bf16_full_size_sampled_parity(name):
    wl = synth.WORKLOADS[name]
    say(f"[gpu] generating {name}")
    inputs = synth.all_inputs(wl)
    m, o, dv, _ = run(wl, inputs=inputs, qk_int8=False)
    mask_properties(m)
    assert bool(torch.isfinite(o.float()).all())
    q, k, v, w = inputs
    out = host_u16(o)
    T = m.plan.info.T
    blocks = sorted({0, 1, T // 2, T - 1})
    G, R = [], []
    for b, h in [(0, 0), (wl.B - 1, wl.H - 1)]:
        prep = check_head_prep(m, wl, b, h, q[b, h], k[b, h], qk_int8=False)
        got, ref = compare_blocks(out[b, h], wl, q[b, h], k[b, h], v[b, h], w, prep, blocks,
                                  qk_int8=False)
        G.append(got)
        R.append(ref)
    assert_close(np.concatenate(G), np.concatenate(R), name + " (bf16 QK)")


# ------------------------------- fine INT8 scales (16 query rows, 4 keys) ---

# The INT8 path with one Q scale per 16 rows and one K' scale per 4 keys;
# codes, both scale arrays and the outputs against the oracle's group-scale
# quantisers and exact branch.
SMALL_FINE = [w for w in SMALL if w.name in (
    "tiny", "tiny-d128-ragged", "two-blocks", "one-token", "sparse-only-b2",
    "dense-outlier-small", "quality-topk", "sharp-online-max", "sharp-online-max-d64")]


@pytest.mark.parametrize("wl", SMALL_FINE, ids=[w.name for w in SMALL_FINE])
def test_fine_scales_small_full_parity(wl):
    full_compare(wl, fine=True)


def test_fine_scales_outlier_tokens_reduce_error():
    """Per-group scales bound each code's step by its own group's maximum: with
    one Q row and one K row in 64 scaled x8, the fine path lands closer to
    float64 dense attention than the block-scale path, both run on the GPU."""
    wl = synth.Workload("outlier-tokens", 1, 1, 2048, 128, 1.0, use_linear=0, seed=4)
    q, k, v, w = synth.all_inputs(wl)
    rng = np.random.default_rng(24)
    sq, sk = np.ones((wl.N, 1)), np.ones((wl.N, 1))
    sq[rng.choice(wl.N, wl.N // 64, replace=False)] = 8.0
    sk[rng.choice(wl.N, wl.N // 64, replace=False)] = 8.0
    q = q.copy()
    k = k.copy()
    q[0, 0] = synth.f64_to_bf16_bits(f32(q[0, 0]) * sq)
    k[0, 0] = synth.f64_to_bf16_bits(f32(k[0, 0]) * sk)
    exact = oracle.head_forward(q[0, 0], k[0, 0], v[0, 0], w, 1.0, use_linear=False,
                                qk_int8=False)
    ref = np.concatenate([exact[i] for i in range(wl.T)])
    errs = {}
    for fine in (False, True):
        m, o, _, _ = run(wl, inputs=(q, k, v, w), fine=fine)
        got = f32(host_u16(o)[0, 0])
        errs[fine] = float(np.linalg.norm(got - ref) / np.linalg.norm(ref))
    say(f"[parity] outlier tokens: rel-L2 to exact, block scales {errs[False]:.3e}, "
        f"fine scales {errs[True]:.3e}")
    assert errs[True] < 0.75 * errs[False]


def test_fine_int32_qk_tiles_bit_exact():
    wl = synth.Workload("qk-fine", 1, 2, 1000, 128, 0.5, seed=2)
    m, o, dv, (q, k, v, w) = run(wl, fine=True)
    triples = [(0, 0, 0), (1, 15, 15), (1, 7, 2)]
    tiles = m.debug_qk_int32(triples).cpu().numpy()
    for n, (bh, i, j) in enumerate(triples):
        prep = oracle.head_prep(q[0, bh], k[0, bh], float(np.float32(wl.topk)), fine=True)
        assert np.array_equal(tiles[n], oracle.qk_int32(prep.q8, prep.k8, i, j)), (bh, i, j)


@pytest.mark.parametrize("name", ["wan14b-720p"])
def test_fine_full_size_sampled_parity(name):
    wl = synth.WORKLOADS[name]
    say(f"[gpu] generating {name}")
    inputs = synth.all_inputs(wl)
    m, o, dv, _ = run(wl, inputs=inputs, fine=True)
    mask_properties(m)
    assert bool(torch.isfinite(o.float()).all())
    q, k, v, w = inputs
    out = host_u16(o)
    T = m.plan.info.T
    blocks = sorted({0, 1, T // 2, T - 1})
    G, R = [], []
    for b, h in [(0, 0), (wl.B - 1, wl.H - 1)]:
        prep = check_head_prep(m, wl, b, h, q[b, h], k[b, h], fine=True)
        got, ref = compare_blocks(out[b, h], wl, q[b, h], k[b, h], v[b, h], w, prep, blocks)
        G.append(got)
        R.append(ref)
    assert_close(np.concatenate(G), np.concatenate(R), name + " (int8-fine)")
