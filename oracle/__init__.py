"""CPU oracle for the SageSLA forward.  TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package; the HIP product path never does.  The
arithmetic lives in ``sla_oracle.c`` (plain, single threaded C, float64 for the
softmax and linear branches, float32/integer exactly as written for the steps
that decide integers); this file only builds it, marshals numpy arrays and
composes the steps per head in the order the method applies them.

Pins: every function is checked in ``tests/test_oracle_pins.py`` against
brute force, closed forms and invariants that do not reuse this code.
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "sla_oracle.c")
_LIB = os.path.join(_HERE, "libsla_oracle.so")
BLOCK = 64

CFLAGS = ["-O2", "-std=c99", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared"]


def build(force: bool = True) -> str:
    """Compile the oracle with gcc into oracle/libsla_oracle.so."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", *CFLAGS, _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        L = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        i32 = ctypes.c_int
        L.sla_ref_kb.argtypes = [i32, ctypes.c_double]
        L.sla_ref_kb.restype = i32
        L.sla_ref_pool.argtypes = [P, i32, i32, P, P]
        L.sla_ref_kmean.argtypes = [P, i32, i32, P]
        L.sla_ref_scores.argtypes = [P, P, P, i32, i32, P]
        L.sla_ref_topk.argtypes = [P, i32, i32, P, P]
        L.sla_ref_quant_q.argtypes = [P, i32, i32, P, P]
        L.sla_ref_quant_k.argtypes = [P, P, i32, i32, P, P]
        L.sla_ref_qk_int32.argtypes = [P, P, i32, i32, i32, P]
        L.sla_ref_sparse_block.argtypes = [i32, P, P, P, P, P, P, P, i32, i32, ctypes.c_float,
                                           P, i32, i32, P]
        L.sla_ref_linear_states.argtypes = [P, P, i32, i32, P, P]
        L.sla_ref_linear_block.argtypes = [P, P, P, P, i32, i32, i32, P]
        L.sla_ref_combine.argtypes = [P, P, P, i32, i32, i32, P]
        L.sla_ref_quant_b128.argtypes = [P, i32, i32, P, P]
        L.sla_ref_quant_q_g.argtypes = [P, i32, i32, i32, P, P]
        L.sla_ref_quant_k_g.argtypes = [P, P, i32, i32, i32, P, P]
        L.sla_ref_sparse_block_g.argtypes = [i32, P, P, P, P, i32, i32, P, P, P, i32, i32,
                                             ctypes.c_float, P, i32, i32, P]
        L.sla_ref_w8a8_gemm.argtypes = [P, P, P, P, i32, i32, i32, P, P]
        _lib = L
    return _lib


def _p(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.c_void_p)


def _u16(x):
    return np.ascontiguousarray(x, dtype=np.uint16)


def nblocks(N: int) -> int:
    return (N + BLOCK - 1) // BLOCK


def kb_for(T: int, topk: float) -> int:
    return lib().sla_ref_kb(T, float(topk))


def default_sm_scale(d: int) -> float:
    return float(np.float32(1.0 / math.sqrt(d)))


# ---- single steps (one head) -------------------------------------------------

def pool(X):
    X = _u16(X)
    N, d = X.shape
    T = nblocks(N)
    sums = np.empty((T, d), np.float32)
    means = np.empty((T, d), np.float32)
    lib().sla_ref_pool(_p(X), N, d, _p(sums), _p(means))
    return sums, means


def kmean(ksums, N):
    ksums = np.ascontiguousarray(ksums, np.float32)
    d = ksums.shape[1]
    mu = np.empty(d, np.float32)
    lib().sla_ref_kmean(_p(ksums), N, d, _p(mu))
    return mu


def scores(qbar, kbar, mu):
    qbar = np.ascontiguousarray(qbar, np.float32)
    kbar = np.ascontiguousarray(kbar, np.float32)
    mu = np.ascontiguousarray(mu, np.float32)
    T, d = qbar.shape
    s = np.empty((T, T), np.float32)
    lib().sla_ref_scores(_p(qbar), _p(kbar), _p(mu), T, d, _p(s))
    return s


def topk(s, kb):
    s = np.ascontiguousarray(s, np.float32)
    T = s.shape[0]
    mask = np.empty((T, T), np.uint8)
    kept = np.empty((T, max(kb, 1)), np.int32)
    lib().sla_ref_topk(_p(s), T, kb, _p(mask), _p(kept))
    return mask, kept[:, :kb]


# Scale granularity: rows per scale group of Q and of K' (64 = one per block;
# the finer SageAttention2++-style mode uses 16 query rows and 4 keys).
QGROUP_FINE, KGROUP_FINE = 16, 4


def quant_q(Q, g=BLOCK):
    """INT8 codes [T*64, d] and scales: [T] for g = 64, else [T, 64/g]."""
    Q = _u16(Q)
    N, d = Q.shape
    T = nblocks(N)
    q8 = np.empty((T * BLOCK, d), np.int8)
    dq = np.empty((T, BLOCK // g), np.float32)
    lib().sla_ref_quant_q_g(_p(Q), N, d, g, _p(q8), _p(dq))
    return q8, (dq[:, 0].copy() if g == BLOCK else dq)


def quant_k(K, mu, g=BLOCK):
    """INT8 codes of K - mu [T*64, d] and scales: [T] for g = 64, else [T, 64/g]."""
    K = _u16(K)
    N, d = K.shape
    T = nblocks(N)
    mu = np.ascontiguousarray(mu, np.float32)
    k8 = np.empty((T * BLOCK, d), np.int8)
    dk = np.empty((T, BLOCK // g), np.float32)
    lib().sla_ref_quant_k_g(_p(K), _p(mu), N, d, g, _p(k8), _p(dk))
    return k8, (dk[:, 0].copy() if g == BLOCK else dk)


def qk_int32(q8, k8, i, j):
    q8 = np.ascontiguousarray(q8, np.int8)
    k8 = np.ascontiguousarray(k8, np.int8)
    A = np.empty((BLOCK, BLOCK), np.int32)
    lib().sla_ref_qk_int32(_p(q8), _p(k8), q8.shape[1], i, j, _p(A))
    return A


def sparse_block(i, kept_i, Q, K, V, sm_scale, q8=None, dq=None, k8=None, dk=None):
    """Exact branch for query block i; quantised when q8/k8 are given (the
    scale granularity follows from the shape of dq / dk: [T] per block,
    [T, 64/g] per group of g rows)."""
    Q, K, V = _u16(Q), _u16(K), _u16(V)
    N, d = Q.shape
    kept_i = np.ascontiguousarray(kept_i, np.int32)
    kb = int(kept_i.shape[0])
    quantized = q8 is not None
    if not quantized:
        q8 = np.zeros((1, 1), np.int8)
        k8 = np.zeros((1, 1), np.int8)
        dq = np.zeros(1, np.float32)
        dk = np.zeros(1, np.float32)
    ni = min(BLOCK, N - i * BLOCK)
    out = np.empty((ni, d), np.float64)
    kp = kept_i if kb else np.zeros(1, np.int32)
    dq = np.ascontiguousarray(dq, np.float32)
    dk = np.ascontiguousarray(dk, np.float32)
    gq = BLOCK // dq.shape[1] if dq.ndim == 2 else BLOCK
    gk = BLOCK // dk.shape[1] if dk.ndim == 2 else BLOCK
    lib().sla_ref_sparse_block_g(int(quantized), _p(np.ascontiguousarray(q8)), _p(dq),
                                 _p(np.ascontiguousarray(k8)), _p(dk), gq, gk, _p(Q), _p(K), _p(V),
                                 N, d, ctypes.c_float(sm_scale), _p(kp), kb, i, _p(out))
    return out


def linear_states(K, V):
    K, V = _u16(K), _u16(V)
    N, d = K.shape
    T = nblocks(N)
    Hb = np.empty((T, d, d), np.float64)
    zb = np.empty((T, d), np.float64)
    lib().sla_ref_linear_states(_p(K), _p(V), N, d, _p(Hb), _p(zb))
    return Hb, zb


def linear_block(i, mask_i, Q, Hb, zb):
    Q = _u16(Q)
    N, d = Q.shape
    ni = min(BLOCK, N - i * BLOCK)
    out = np.empty((ni, d), np.float64)
    lib().sla_ref_linear_block(_p(Q), _p(np.ascontiguousarray(Hb, np.float64)),
                               _p(np.ascontiguousarray(zb, np.float64)),
                               _p(np.ascontiguousarray(mask_i, np.uint8)), N, d, i, _p(out))
    return out


def combine(Os, Ol, W, use_linear):
    Os = np.ascontiguousarray(Os, np.float64)
    Ol = np.ascontiguousarray(Ol, np.float64)
    n, d = Os.shape
    out = np.empty((n, d), np.float64)
    lib().sla_ref_combine(_p(Os), _p(Ol), _p(_u16(W)), int(use_linear), n, d, _p(out))
    return out


# ---- one head, composed ------------------------------------------------------

@dataclass
class HeadPrep:
    """Everything the selection and quantisation steps produce for one head."""
    qsum: np.ndarray
    qbar: np.ndarray
    ksum: np.ndarray
    kbar: np.ndarray
    mu: np.ndarray
    scores: np.ndarray
    mask: np.ndarray
    kept: np.ndarray
    q8: np.ndarray
    dq: np.ndarray
    k8: np.ndarray
    dk: np.ndarray


def head_prep(Q, K, topk_frac, smooth=True, fine=False) -> HeadPrep:
    """Steps 1-6 for one head (pool, K mean, scores, top-k, Q and K INT8);
    ``fine``: SageAttention2++-style scale groups (16 query rows, 4 keys)."""
    N, d = np.shape(Q)
    T = nblocks(N)
    kb = kb_for(T, topk_frac)
    if kb < 0:
        raise ValueError("topk outside [0, 1]")
    qsum, qbar = pool(Q)
    ksum, kbar = pool(K)
    mu = kmean(ksum, N)
    s = scores(qbar, kbar, mu)
    mask, kept = topk(s, kb)
    q8, dq = quant_q(Q, QGROUP_FINE if fine else BLOCK)
    k8, dk = quant_k(K, mu if smooth else np.zeros_like(mu), KGROUP_FINE if fine else BLOCK)
    return HeadPrep(qsum, qbar, ksum, kbar, mu, s, mask, kept, q8, dq, k8, dk)


def head_forward(Q, K, V, W, topk_frac, use_linear=True, sm_scale=None, blocks=None,
                 prep: HeadPrep | None = None, states=None, smooth=True, parts=False,
                 qk_int8=True, fine=False):
    """SageSLA forward of one head in float64 for the query blocks ``blocks``
    (all by default).  Returns {i: out[n_i, d]} (and the two branches when
    ``parts``).  ``qk_int8=False`` is plain SLA: the same selection and linear
    branch, the exact branch's logits from the bf16 inputs themselves."""
    Q, K, V = _u16(Q), _u16(K), _u16(V)
    N, d = Q.shape
    T = nblocks(N)
    if sm_scale is None:
        sm_scale = default_sm_scale(d)
    if prep is None:
        prep = head_prep(Q, K, topk_frac, smooth=smooth, fine=fine)
    if use_linear and states is None:
        states = linear_states(K, V)
    res = {}
    for i in (range(T) if blocks is None else blocks):
        if qk_int8:
            Os = sparse_block(i, prep.kept[i], Q, K, V, sm_scale, prep.q8, prep.dq, prep.k8, prep.dk)
        else:
            Os = sparse_block(i, prep.kept[i], Q, K, V, sm_scale)
        if use_linear:
            Ol = linear_block(i, prep.mask[i], Q, states[0], states[1])
        else:
            Ol = np.zeros_like(Os)
        O = combine(Os, Ol, W, use_linear)
        res[i] = (O, Os, Ol) if parts else O
    return res


# ---- W8A8 linear layers --------------------------------------------------------

WBLOCK = 128


def quant_b128(X):
    """bf16 bits [R][C] -> (int8 codes [R][C], float32 scales [ceil(R/128)][ceil(C/128)])."""
    X = _u16(X)
    R, C = X.shape
    codes = np.empty((R, C), np.int8)
    scales = np.empty(((R + WBLOCK - 1) // WBLOCK, (C + WBLOCK - 1) // WBLOCK), np.float32)
    lib().sla_ref_quant_b128(_p(X), R, C, _p(codes), _p(scales))
    return codes, scales


def w8a8_gemm(xq, sx, wq, sw):
    """Block-scaled INT8 GEMM, Y = X W^T: (float32 [M][N], bf16 bits [M][N])."""
    xq = np.ascontiguousarray(xq, np.int8)
    wq = np.ascontiguousarray(wq, np.int8)
    M, K = xq.shape
    N = wq.shape[0]
    assert wq.shape[1] == K and K % WBLOCK == 0
    y32 = np.empty((M, N), np.float32)
    y = np.empty((M, N), np.uint16)
    lib().sla_ref_w8a8_gemm(_p(xq), _p(np.ascontiguousarray(sx, np.float32)), _p(wq),
                            _p(np.ascontiguousarray(sw, np.float32)), M, N, K, _p(y32), _p(y))
    return y32, y
