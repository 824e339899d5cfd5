"""Independent closed forms of the same recurrence -- oracle, TEST INFRASTRUCTURE ONLY.

Each function here evaluates h_t = Abar_t h_{t-1} + Bbar_t x_t, y_t = C_t h_t by
a different route than the sequential loop, so the loop can be pinned against
them on small inputs.  All work on one channel; arrays indexed [t] or [t, n];
float64 throughout; h before the first step is zero.

* ``discretize``        -- eq. (2) of "Understanding Mamba" section 2.2
                           (Abar = exp(Delta A)) with either input term.
* ``combine`` and scans -- the affine-pair operator of "Understanding Mamba"
                           section 7.1 eq. (8) and its reorderings (section 7.2).
* ``unrolled_states``   -- the unrolled sum of "Mathematical Prerequisites for
                           Mamba" section 6 (sum over inputs of the product of
                           the later decays times the input term).
* ``semiseparable``     -- the lower-triangular matrix of cumulative decays of
                           section 7 of the same page; h = L diag(Bbar) x.
* ``convolution_*``     -- the LTI kernel Kbar_i = C Abar^i Bbar of
                           "Understanding Mamba" section 3.1 eq. (5).
"""
from __future__ import annotations

import itertools
import math

import numpy as np


def discretize(delta, A, B, mode: str = "euler"):
    """Return (Abar, Bbar) for one step: Abar = exp(delta*A); Bbar = delta*B
    (first-order) or (Abar - 1)/A * B (zero-order hold, diagonal A != 0)."""
    A = np.asarray(A, dtype=np.float64)
    B = np.asarray(B, dtype=np.float64)
    Abar = np.exp(delta * A)
    if mode == "euler":
        Bbar = delta * B
    elif mode == "zoh":
        Bbar = (Abar - 1.0) / A * B
    else:
        raise ValueError(mode)
    return Abar, Bbar


def combine(P, Q):
    """(a_i, b_i) . (a_j, b_j) = (a_i a_j, a_j b_i + b_j): step i then step j."""
    a_p, b_p = P
    a_q, b_q = Q
    return (a_p * a_q, a_q * b_p + b_q)


def fold_left(pairs):
    """Prefix compositions by strict left-to-right folding: the reference order."""
    out = []
    acc = None
    for p in pairs:
        acc = p if acc is None else combine(acc, p)
        out.append(acc)
    return out


def bracketings(lo: int, hi: int):
    """Every full binary bracketing of the index range [lo, hi) as nested tuples."""
    if hi - lo == 1:
        yield lo
        return
    for mid in range(lo + 1, hi):
        for left in bracketings(lo, mid):
            for right in bracketings(mid, hi):
                yield (left, right)


def reduce_tree(pairs, tree):
    """Compose ``pairs`` following the bracketing ``tree`` (from ``bracketings``)."""
    if isinstance(tree, int):
        return pairs[tree]
    left, right = tree
    return combine(reduce_tree(pairs, left), reduce_tree(pairs, right))


def doubling_scan(pairs):
    """Inclusive scan in ceil(log2 L) rounds (recursive doubling): in round k
    every position i >= 2^k absorbs the composite ending at i - 2^k."""
    cur = list(pairs)
    step = 1
    while step < len(cur):
        nxt = list(cur)
        for i in range(step, len(cur)):
            nxt[i] = combine(cur[i - step], cur[i])
        cur = nxt
        step *= 2
    return cur


def chunked_scan(pairs, chunk_lengths):
    """Scan each chunk from an empty prefix, then carry the running composite
    from chunk to chunk -- the chunk-carry reordering a GPU scan uses."""
    if sum(chunk_lengths) != len(pairs):
        raise ValueError("chunk lengths must cover the sequence")
    out = []
    carry = None
    start = 0
    for ln in chunk_lengths:
        local = fold_left(pairs[start:start + ln])
        if carry is not None:
            local = [combine(carry, p) for p in local]
        out.extend(local)
        carry = local[-1]
        start += ln
    return out


def unrolled_states(Abar, Bbar, x):
    """h_t = sum_{j<=t} (prod_{j<k<=t} Abar_k) Bbar_j x_j, evaluated term by term
    (O(L^2)).  Abar, Bbar: [L, N]; x: [L].  Returns h: [L, N]."""
    Abar = np.asarray(Abar, dtype=np.float64)
    Bbar = np.asarray(Bbar, dtype=np.float64)
    x = np.asarray(x, dtype=np.float64)
    L, N = Abar.shape
    h = np.zeros((L, N))
    for t in range(L):
        for j in range(t + 1):
            decay = np.ones(N)
            for k in range(j + 1, t + 1):
                decay = decay * Abar[k]
            h[t] += decay * Bbar[j] * x[j]
    return h


def semiseparable(Abar_n):
    """Lower-triangular L with L[t, j] = prod_{j<k<=t} Abar_n[k] (1 on the
    diagonal, 0 above), for one state channel; Abar_n: [L]."""
    a = np.asarray(Abar_n, dtype=np.float64)
    T = len(a)
    M = np.zeros((T, T))
    for t in range(T):
        for j in range(t + 1):
            M[t, j] = math.prod(a[j + 1:t + 1])
    return M


def semiseparable_states(Abar, Bbar, x):
    """h[:, n] = L_n diag(Bbar[:, n]) x for each state channel n."""
    Abar = np.asarray(Abar, dtype=np.float64)
    Bbar = np.asarray(Bbar, dtype=np.float64)
    x = np.asarray(x, dtype=np.float64)
    L, N = Abar.shape
    h = np.zeros((L, N))
    for n in range(N):
        h[:, n] = semiseparable(Abar[:, n]) @ (Bbar[:, n] * x)
    return h


def convolution_kernel(Abar, Bbar, C, length: int):
    """Kbar_i = C . (Abar^i * Bbar) for i < length, with constant Abar, Bbar, C [N]."""
    Abar = np.asarray(Abar, dtype=np.float64)
    Bbar = np.asarray(Bbar, dtype=np.float64)
    C = np.asarray(C, dtype=np.float64)
    return np.array([float(C @ (Abar ** i * Bbar)) for i in range(length)])


def convolution_output(x, K):
    """Causal convolution y_t = sum_{i<=t} K_i x_{t-i}, by direct summation."""
    x = np.asarray(x, dtype=np.float64)
    return np.array([sum(K[i] * x[t - i] for i in range(t + 1)) for t in range(len(x))])


def all_chunkings(L: int):
    """Every composition of L into positive chunk lengths (2^(L-1) of them)."""
    for cuts in itertools.product([0, 1], repeat=max(L - 1, 0)):
        lengths = []
        run = 1
        for c in cuts:
            if c:
                lengths.append(run)
                run = 1
            else:
                run += 1
        lengths.append(run)
        yield lengths
