"""CPU oracle for the backward pass of plain SLA.  TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this module; the HIP product path never does.

What it computes: the gradients of trainable SLA (pages: "揭秘TurboDiffusion…"
section "支柱二：稀疏线性注意力 – SLA", the sparse pattern and the linear
component are learned; aiho.net news report (量子位, 2025-12-26)
section "2. SLA稀疏线性注意力")
for one head, with the block mask held fixed (top-k selection is a discrete
choice and passes no gradient).  The forward is the bf16-QK^T operator (plain
SLA): per query block i, softmax attention over the rows of its kept key
blocks, plus phi(Q_i) H_i / (phi(Q_i) . z_i) over the marginal blocks,
projected by W and added.  Everything is float64 numpy, written as the
definitions read: no blocking or fusion beyond the block structure the
method itself has.

The gradient formulas are the chain rule through those definitions (softmax:
dS = P (dP - rowsum(dO O_s)); channel softmax phi: dx = phi (dphi - phi . dphi);
the quotient num / den; the block sums H_i = sum of Hb_j over marginal j).
Pins (tests/test_oracle_pins.py): ``forward`` equals the C oracle's exact-logit
forward; central finite differences of ``forward`` match ``backward`` in every
input; Euler identities <dV, V> = <dO, O> and <dW, W> = <dO, O_l W^T>.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

BLOCK = 64


def _rows(t, N):
    return slice(BLOCK * t, min(BLOCK * (t + 1), N))


def phi(X):
    """Softmax over the channels of each row (the linear branch's feature map)."""
    e = np.exp(X - X.max(axis=1, keepdims=True))
    return e / e.sum(axis=1, keepdims=True)


def phi_grad(A, dA):
    """Gradient through phi at output A = phi(X): A (dA - rowsum(A dA))."""
    return A * (dA - (A * dA).sum(axis=1, keepdims=True))


@dataclass
class Forward:
    O: np.ndarray      # [N, d] combined output
    Os: np.ndarray     # [N, d] sparse branch
    Ol: np.ndarray     # [N, d] linear branch before the projection
    lse: np.ndarray    # [N] natural-log normaliser of each row's softmax (-inf: no kept key)


def _key_rows(kept_i, N):
    return np.concatenate([np.arange(BLOCK * j, min(BLOCK * (j + 1), N)) for j in kept_i]) \
        if len(kept_i) else np.zeros(0, np.int64)


def forward(Q, K, V, W, mask, sm_scale, use_linear=True) -> Forward:
    """Plain-SLA forward of one head in float64 for float64 inputs Q, K, V
    [N, d], W [d_out, d_in] and the boolean block mask [T, T] (True = kept)."""
    N, d = Q.shape
    T = mask.shape[0]
    Os = np.zeros((N, d))
    Ol = np.zeros((N, d))
    lse = np.full(N, -np.inf)
    if use_linear:
        Hb = np.zeros((T, d, d))
        zb = np.zeros((T, d))
        for j in range(T):
            B = phi(K[_rows(j, N)])
            Hb[j] = B.T @ V[_rows(j, N)]
            zb[j] = B.sum(axis=0)
    for i in range(T):
        r = _rows(i, N)
        kept = np.flatnonzero(mask[i])
        s = _key_rows(kept, N)
        if s.size:
            L = Q[r] @ K[s].T * sm_scale
            m = L.max(axis=1, keepdims=True)
            E = np.exp(L - m)
            l = E.sum(axis=1, keepdims=True)
            Os[r] = (E / l) @ V[s]
            lse[r] = (m + np.log(l))[:, 0]
        if use_linear:
            marg = np.flatnonzero(~mask[i])
            if marg.size:
                H = Hb[marg].sum(axis=0)
                z = zb[marg].sum(axis=0)
                A = phi(Q[r])
                Ol[r] = (A @ H) / (A @ z)[:, None]
    O = Os + Ol @ W.T if use_linear else Os.copy()
    return Forward(O, Os, Ol, lse)


@dataclass
class Grads:
    dQ: np.ndarray
    dK: np.ndarray
    dV: np.ndarray
    dW: np.ndarray


def backward(Q, K, V, W, dO, mask, sm_scale, use_linear=True, fwd: Forward | None = None) -> Grads:
    """Gradients of sum(dO * O) with respect to Q, K, V and W (float64)."""
    N, d = Q.shape
    T = mask.shape[0]
    if fwd is None:
        fwd = forward(Q, K, V, W, mask, sm_scale, use_linear)
    dQ = np.zeros((N, d))
    dK = np.zeros((N, d))
    dV = np.zeros((N, d))
    dW = np.zeros_like(W, dtype=np.float64)

    # sparse branch: each query block's softmax over its kept keys
    for i in range(T):
        r = _rows(i, N)
        s = _key_rows(np.flatnonzero(mask[i]), N)
        if not s.size:
            continue
        P = np.exp(Q[r] @ K[s].T * sm_scale - fwd.lse[r][:, None])
        dP = dO[r] @ V[s].T
        D = (dO[r] * fwd.Os[r]).sum(axis=1, keepdims=True)
        dS = P * (dP - D)
        dQ[r] += sm_scale * dS @ K[s]
        np.add.at(dK, s, sm_scale * dS.T @ Q[r])
        np.add.at(dV, s, P.T @ dO[r])

    if use_linear:
        dW += dO.T @ fwd.Ol
        G = dO @ W  # gradient at O_l
        Hb = np.zeros((T, d, d))
        zb = np.zeros((T, d))
        for j in range(T):
            B = phi(K[_rows(j, N)])
            Hb[j] = B.T @ V[_rows(j, N)]
            zb[j] = B.sum(axis=0)
        dH = np.zeros((T, d, d))
        dz = np.zeros((T, d))
        for i in range(T):
            r = _rows(i, N)
            marg = np.flatnonzero(~mask[i])
            if not marg.size:
                continue
            H = Hb[marg].sum(axis=0)
            z = zb[marg].sum(axis=0)
            A = phi(Q[r])
            den = (A @ z)[:, None]
            Ol = (A @ H) / den
            dnum = G[r] / den
            dden = -(G[r] * Ol).sum(axis=1, keepdims=True) / den
            dA = dnum @ H.T + dden * z[None, :]
            dQ[r] += phi_grad(A, dA)
            dH[i] = A.T @ dnum
            dz[i] = (A * dden).sum(axis=0)
        # H_i sums Hb_j over the marginal j, so Hb_j collects dH_i over the
        # query blocks i for which j is marginal
        for j in range(T):
            users = np.flatnonzero(~mask[:, j])
            if not users.size:
                continue
            dHb = dH[users].sum(axis=0)
            dzb = dz[users].sum(axis=0)
            rj = _rows(j, N)
            B = phi(K[rj])
            dV[rj] += B @ dHb
            dB = V[rj] @ dHb.T + dzb[None, :]
            dK[rj] += phi_grad(B, dB)
    return Grads(dQ, dK, dV, dW)


def head_backward(Q, K, V, W, dO, mask, sm_scale, use_linear=True):
    """bf16 bit patterns in (uint16 [N, d], W [d, d], dO [N, d]), float64
    gradients out, mask as the oracle's selection step returns it."""
    f = _bf16_to_f64
    return backward(f(Q), f(K), f(V), f(W), f(dO), np.asarray(mask, bool), sm_scale, use_linear)


def _bf16_to_f64(b):
    b = np.ascontiguousarray(b, np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _block_states(K, V, T):
    """Hb [T, d, d] and zb [T, d]: phi(K_j)^T V_j and phi(K_j)^T 1 per key block."""
    N, d = K.shape
    Hb = np.zeros((T, d, d))
    zb = np.zeros((T, d))
    for j in range(T):
        B = phi(K[_rows(j, N)])
        Hb[j] = B.T @ V[_rows(j, N)]
        zb[j] = B.sum(axis=0)
    return Hb, zb


def backward_sampled(Q, K, V, W, dO, mask, sm_scale, qblocks, kblocks, use_linear=True):
    """The same gradients as ``backward`` restricted to the rows of the query
    blocks ``qblocks`` (dQ) and the key blocks ``kblocks`` (dK, dV), plus the
    whole dW, for heads too large for ``backward``.  The marginal sums
    H_i = sum over marginal j of Hb_j (and their transposes for dHb_j) are
    written as one matrix product with the complement mask.
    Returns ({i: dQ rows}, {j: dK rows}, {j: dV rows}, dW)."""
    N, d = Q.shape
    T = mask.shape[0]
    comp = (~mask).astype(np.float64)
    dQ = {i: np.zeros((min(BLOCK, N - BLOCK * i), d)) for i in qblocks}
    dK = {j: np.zeros((min(BLOCK, N - BLOCK * j), d)) for j in kblocks}
    dV = {j: np.zeros((min(BLOCK, N - BLOCK * j), d)) for j in kblocks}
    dW = np.zeros((d, d))

    def sparse_rows(i):
        """P, dS and the key rows of query block i's softmax."""
        r = _rows(i, N)
        s = _key_rows(np.flatnonzero(mask[i]), N)
        L = Q[r] @ K[s].T * sm_scale
        m = L.max(axis=1, keepdims=True)
        E = np.exp(L - m)
        P = E / E.sum(axis=1, keepdims=True)
        Os = P @ V[s]
        dP = dO[r] @ V[s].T
        D = (dO[r] * Os).sum(axis=1, keepdims=True)
        return s, P, P * (dP - D)

    for i in qblocks:
        if mask[i].any():
            s, P, dS = sparse_rows(i)
            dQ[i] += sm_scale * dS @ K[s]
    users = sorted({int(i) for j in kblocks for i in np.flatnonzero(mask[:, j])})
    for i in users:
        s, P, dS = sparse_rows(i)
        r = _rows(i, N)
        for j in kblocks:
            if not mask[i, j]:
                continue
            # positions of key block j's rows inside s
            pos = np.flatnonzero((s >= BLOCK * j) & (s < BLOCK * j + dK[j].shape[0]))
            dK[j] += sm_scale * dS[:, pos].T @ Q[r]
            dV[j] += P[:, pos].T @ dO[r]

    if use_linear:
        Hb, zb = _block_states(K, V, T)
        H = (comp @ Hb.reshape(T, d * d)).reshape(T, d, d)
        z = comp @ zb
        G = dO @ W
        dH = np.zeros((T, d, d))
        dz = np.zeros((T, d))
        for i in range(T):
            if not comp[i].any():
                continue
            r = _rows(i, N)
            A = phi(Q[r])
            den = (A @ z[i])[:, None]
            Ol = (A @ H[i]) / den
            dW += dO[r].T @ Ol
            dnum = G[r] / den
            dden = -(G[r] * Ol).sum(axis=1, keepdims=True) / den
            dH[i] = A.T @ dnum
            dz[i] = (A * dden).sum(axis=0)
            if i in dQ:
                dA = dnum @ H[i].T + dden * z[i][None, :]
                dQ[i] += phi_grad(A, dA)
        dHb = (comp.T @ dH.reshape(T, d * d)).reshape(T, d, d)
        dzb = comp.T @ dz
        for j in kblocks:
            rj = _rows(j, N)
            B = phi(K[rj])
            dV[j] += B @ dHb[j]
            dK[j] += phi_grad(B, V[rj] @ dHb[j].T + dzb[j][None, :])
    return dQ, dK, dV, dW
