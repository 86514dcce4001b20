"""Dense float64 RACE Attention oracle (NumPy) — TEST INFRASTRUCTURE ONLY.

One (batch, head) sequence at a time: Q, K, V are [N, d] float64, the
hyperplanes W are [L, P, d] float64 (the exact values of whatever dtype the
caller used).  Steps follow the pages' order (arXiv 2510.04008 summaries):

  1. unit-normalise queries and keys (the similarity is a function of the
     normalised dot product: Japanese gist.science page, section 2.1, and
     Italian page, Sommario tecnico section 2, Concetti Chiave 1);
  2. project on P random hyperplanes per table, L tables (Korean page,
     기술 요약 section 2, algorithm flow; Italian page, section 2, Concetti
     Chiave 2);
  3. soften with tanh and take a softmax over the 2^P hypercube corners with
     temperature beta (Italian page, section 2, Concetti Chiave 2; Japanese
     page, section 2.2, differentiability);
  4. keys write per-bucket mass and value sums (Italian page, section 2,
     Algoritmo; Japanese page, section 2.1, bucket aggregation);
  5. each query reads its own soft buckets, and the output is the normalised
     weighted average over the L tables (Italian page, section 2, Algoritmo;
     Japanese page, section 2.1, reconstruction);
  6. causal mode restricts the sums to keys j <= i through prefix sums
     (Japanese page, section 2.2, causal support).

Readings taken where the pages are silent (each also listed in the design
notes):
  * x_hat = x / max(||x||, 1e-12); V is not normalised.
  * corner r has sign c[r, p] = +1 when bit p of r is set, else -1; the
    corner logit is beta * sum_p c[r, p] * tanh(h_p).
  * tables combine as a ratio of sums: O_i = sum_l num_l / sum_l den_l.
  * causal sums include the diagonal (j <= i).
  * one W of shape [L, P, d] is shared by queries and keys and by all heads.
  * hard-hash id of a table = sum_p [h_p > 0] 2^p.

Beyond the training path: ``hard_forward`` (one-hot buckets, the beta -> inf
limit, output 0 when a query collides with no key) and the causal decode step
against a running sketch (``sketch`` of a prompt, then ``decode_step`` per new
token), the sketch standing in for the key-value cache at inference.

The backward is the exact gradient of this forward (the pages state the
method is differentiable end to end: Japanese page, section 2.2), written out
by the chain rule.
"""
from __future__ import annotations

import numpy as np

EPS = 1e-12
NEAR_ZERO = 1e-5


def corner_signs(P: int) -> np.ndarray:
    """[R, P] matrix of hypercube corners: +1 where bit p of r is set, else -1."""
    r = np.arange(1 << P)[:, None]
    p = np.arange(P)[None, :]
    return np.where((r >> p) & 1, 1.0, -1.0)


def unit_rows(X: np.ndarray):
    nrm = np.sqrt(np.sum(X * X, axis=-1, keepdims=True))
    return X / np.maximum(nrm, EPS), nrm


def soft_buckets(X: np.ndarray, W: np.ndarray, beta: float):
    """Soft bucket assignment a[n, l, r] of rows X (steps 1-3).

    Returns (a, cache) where cache keeps what the backward needs.
    """
    L, P, d = W.shape
    Xh, nrm = unit_rows(X)
    h = np.einsum("nd,lpd->nlp", Xh, W)
    u = np.tanh(h)
    C = corner_signs(P)
    logits = beta * np.einsum("nlp,rp->nlr", u, C)
    logits = logits - logits.max(axis=-1, keepdims=True)
    e = np.exp(logits)
    a = e / e.sum(axis=-1, keepdims=True)
    return a, (Xh, nrm, u, C)


def aggregate_readout(aQ, aK, V, causal: bool):
    """Steps 4-6: bucket sums and the per-query readout.

    Returns O [N, d], D [N] (the denominators) and, for the backward, the
    per-query state (S_i, z_i) as a generator-free list when causal, else the
    single global state.
    """
    N, L, R = aQ.shape
    d = V.shape[1]
    if not causal:
        S = np.einsum("jlr,jd->lrd", aK, V)
        z = aK.sum(axis=0)
        num = np.einsum("ilr,lrd->id", aQ, S)
        den = np.einsum("ilr,lr->i", aQ, z)
        return num / den[:, None], den, (S, z)
    S = np.zeros((L, R, d))
    z = np.zeros((L, R))
    O = np.empty((N, d))
    D = np.empty(N)
    states = []
    for i in range(N):
        S += aK[i][:, :, None] * V[i][None, None, :]
        z += aK[i]
        num = np.einsum("lr,lrd->d", aQ[i], S)
        den = np.sum(aQ[i] * z)
        O[i] = num / den
        D[i] = den
        states.append((S.copy(), z.copy()))
    return O, D, states


def forward(Q, K, V, W, beta: float = 1.0, causal: bool = False):
    """RACE Attention output O [N, d] for one (batch, head)."""
    aQ, _ = soft_buckets(Q, W, beta)
    aK, _ = soft_buckets(K, W, beta)
    O, _, _ = aggregate_readout(aQ, aK, V, causal)
    return O


def soft_buckets_backward(dA, a, cache, W, beta: float):
    """Chain rule back through steps 3, 2 and 1 for one set of rows."""
    Xh, nrm, u, C = cache
    dlogit = a * (dA - np.sum(a * dA, axis=-1, keepdims=True))
    du = beta * np.einsum("nlr,rp->nlp", dlogit, C)
    dh = du * (1.0 - u * u)
    dXh = np.einsum("nlp,lpd->nd", dh, W)
    radial = np.sum(Xh * dXh, axis=-1, keepdims=True)
    big = nrm > EPS
    return np.where(big, (dXh - Xh * radial) / np.where(big, nrm, 1.0), dXh / EPS)


def backward(Q, K, V, W, dO, beta: float = 1.0, causal: bool = False):
    """Gradients (dQ, dK, dV) of <dO, O> for one (batch, head)."""
    aQ, cQ = soft_buckets(Q, W, beta)
    aK, cK = soft_buckets(K, W, beta)
    O, D, st = aggregate_readout(aQ, aK, V, causal)
    N, L, R = aQ.shape
    d = V.shape[1]
    g = dO / D[:, None]
    e = -np.sum(dO * O, axis=1) / D
    G = np.concatenate([g, e[:, None]], axis=1)            # [N, d+1]
    Vaug = np.concatenate([V, np.ones((N, 1))], axis=1)    # [N, d+1]
    # query side: dA_Q[i] = S_i . g_i + z_i e_i
    if causal:
        dAQ = np.empty((N, L, R))
        for i in range(N):
            S, z = st[i]
            dAQ[i] = np.einsum("lrd,d->lr", S, g[i]) + z * e[i]
    else:
        S, z = st
        dAQ = np.einsum("lrd,id->ilr", S, g) + z[None] * e[:, None, None]
    # key side: T_j = sum over queries i >= j (all i when non-causal) of a_Q[i] G_i
    dV = np.empty((N, d))
    dAK = np.empty((N, L, R))
    if causal:
        T = np.zeros((L, R, d + 1))
        for j in range(N - 1, -1, -1):
            T += aQ[j][:, :, None] * G[j][None, None, :]
            dV[j] = np.einsum("lr,lrd->d", aK[j], T[:, :, :d])
            dAK[j] = T @ Vaug[j]
    else:
        T = np.einsum("ilr,ic->lrc", aQ, G)
        dV = np.einsum("jlr,lrd->jd", aK, T[:, :, :d])
        dAK = np.einsum("lrc,jc->jlr", T, Vaug)
    dQ = soft_buckets_backward(dAQ, aQ, cQ, W, beta)
    dK = soft_buckets_backward(dAK, aK, cK, W, beta)
    return dQ, dK, dV


def hard_hash(X, W):
    """Hard bucket ids [N, L] (int32) and the count of |h| < 1e-5 projections."""
    L, P, d = W.shape
    Xh, _ = unit_rows(X)
    h = np.einsum("nd,lpd->nlp", Xh, W)
    bits = (h > 0).astype(np.int64)
    ids = np.sum(bits << np.arange(P)[None, None, :], axis=-1).astype(np.int32)
    return ids, int(np.sum(np.abs(h) < NEAR_ZERO))


def hard_buckets(X, W):
    """One-hot assignment a[n, l, r] = [r == id_l(x_n)]: the limit beta -> inf
    of the soft assignment, i.e. the discrete hash of the original RACE sketch
    that the temperature beta softens (Japanese gist.science page, section
    2.2, differentiability; Italian page, section 2, on hard binary LSH)."""
    ids, _ = hard_hash(X, W)
    R = 1 << W.shape[1]
    return (ids[..., None] == np.arange(R)[None, None, :]).astype(np.float64)


def assign(X, W, beta):
    """Soft assignment for finite beta, the one-hot hard assignment for beta = inf."""
    if np.isinf(beta):
        return hard_buckets(X, W)
    return soft_buckets(X, W, beta)[0]


def hard_forward(Q, K, V, W, causal: bool = False):
    """Hard-hash RACE output for one (batch, head): keys add [v | 1] to the one
    bucket their sign pattern picks in each table, a query reads the bucket it
    falls in, and O_i = sum of the read value sums / sum of the read counts;
    O_i = 0 when no key shares a bucket with the query in any table (the
    pages' bucket aggregation and reconstruction with one-hot assignments)."""
    aQ, aK = hard_buckets(Q, W), hard_buckets(K, W)
    N, L, R = aQ.shape
    d = V.shape[1]
    S = np.zeros((L, R, d))
    z = np.zeros((L, R))
    if not causal:
        S = np.einsum("jlr,jd->lrd", aK, V)
        z = aK.sum(axis=0)
    O = np.zeros((N, d))
    for i in range(N):
        if causal:
            S += aK[i][:, :, None] * V[i][None, None, :]
            z += aK[i]
        den = np.sum(aQ[i] * z)
        if den != 0:
            O[i] = np.einsum("lr,lrd->d", aQ[i], S) / den
    return O


def sketch(K, V, W, beta: float = 1.0):
    """Key sketch of a whole sequence: S [L, R, d] = sum_j a(k_j) v_j^T and
    z [L, R] = sum_j a(k_j) (bucket aggregation: Italian page, section 2,
    Algoritmo; Japanese page, section 2.1). beta = inf uses the hard buckets.
    This is the state a causal decode continues from after a prompt."""
    aK = assign(K, W, beta)
    return np.einsum("jlr,jd->lrd", aK, V), aK.sum(axis=0)


def decode_step(S, z, q, k, v, W, beta: float = 1.0):
    """One causal decode step against a running sketch (S, z): the new key k
    with value v joins the sketch first (causal sums include the diagonal),
    then the query q reads it out. Returns (S', z', o); o = 0 when the
    denominator is 0 (possible only for hard buckets). The sketch replaces the
    key-value cache: its size L * R * (d + 1) does not grow with the sequence
    (efficient key-value caching at inference: Japanese gist.science page,
    section 6; Korean page, section 5)."""
    aq = assign(q[None], W, beta)[0]
    ak = assign(k[None], W, beta)[0]
    S = S + ak[:, :, None] * v[None, None, :]
    z = z + ak
    den = np.sum(aq * z)
    o = np.einsum("lr,lrd->d", aq, S) / den if den != 0 else np.zeros(v.shape[0])
    return S, z, o


def forward_batched(Q, K, V, W, beta=1.0, causal=False):
    """Apply ``forward`` to every (batch, head) of [B, H, N, d] arrays."""
    B, H = Q.shape[:2]
    out = np.empty(Q.shape[:3] + (V.shape[-1],))
    for b in range(B):
        for hh in range(H):
            out[b, hh] = forward(Q[b, hh], K[b, hh], V[b, hh], W, beta, causal)
    return out


def backward_batched(Q, K, V, W, dO, beta=1.0, causal=False):
    B, H = Q.shape[:2]
    dQ = np.empty(Q.shape)
    dK = np.empty(K.shape)
    dV = np.empty(V.shape)
    for b in range(B):
        for hh in range(H):
            dQ[b, hh], dK[b, hh], dV[b, hh] = backward(Q[b, hh], K[b, hh], V[b, hh], W,
                                                       dO[b, hh], beta, causal)
    return dQ, dK, dV
