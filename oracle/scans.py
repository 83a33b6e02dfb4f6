"""Affine-pair prefix scans in fp64 (oracle side, TEST INFRASTRUCTURE ONLY).

A first-order linear recurrence h_t = a_t * h_{t-1} + b_t is the prefix
composition of the affine maps e_t = (a_t, b_t).  The combine rule, as given
in "Selective State-Space Models (Mamba) and Hardware-Aware Scans" section 3
and in the Transformer-math "Selective state space" article ("The associative
scan restores parallel depth"), composes "first e1, then e2":

    (a1, b1) (+) (a2, b2) = (a2 * a1, a2 * b1 + b2)

Four orders of evaluation are implemented here.  They must agree (the
operator is associative); the tests pin them against each other, against
closed forms, and count the combines of the Blelloch sweep (O(L)) against the
doubling scan (O(L log L)), as the exercises of the temporalbook section ask.
The state axis is the leading one; any trailing axes are independent lanes.
"""
from __future__ import annotations

import numpy as np


def combine(e1, e2):
    """(a1,b1) then (a2,b2)."""
    a1, b1 = e1
    a2, b2 = e2
    return a2 * a1, a2 * b1 + b2


def scan_sequential(a, b, h0=None):
    """Left-to-right loop: returns h[t] for t = 0..L-1 (h before t=0 is h0)."""
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    h = np.zeros(a.shape[1:]) if h0 is None else np.asarray(h0, dtype=np.float64)
    out = np.empty_like(b)
    for t in range(a.shape[0]):
        h = a[t] * h + b[t]
        out[t] = h
    return out


def scan_hillis_steele(a, b):
    """Doubling (Hillis-Steele) inclusive scan with h0 = 0.

    Round k combines every element with the one 2^k positions earlier;
    log2(L) rounds, each touching all L elements.  Returns (h, combines).
    """
    A = np.array(a, dtype=np.float64, copy=True)
    Bv = np.array(b, dtype=np.float64, copy=True)
    L = A.shape[0]
    combines = 0
    step = 1
    while step < L:
        newA, newB = combine((A[:L - step], Bv[:L - step]), (A[step:], Bv[step:]))
        A = np.concatenate([A[:step], newA], axis=0)
        Bv = np.concatenate([Bv[:step], newB], axis=0)
        combines += L - step
        step *= 2
    return Bv, combines


def scan_blelloch(a, b):
    """Work-efficient (Blelloch) scan: up-sweep reduction tree, then a
    down-sweep that hands each node the composition of everything to its left.
    Pads to a power of two with the identity map (1, 0).  Returns the
    inclusive states h (h0 = 0) and the number of combines performed.
    """
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    L = a.shape[0]
    n = 1
    while n < L:
        n *= 2
    A = np.ones((n,) + a.shape[1:])
    Bv = np.zeros((n,) + b.shape[1:])
    A[:L] = a
    Bv[:L] = b
    combines = 0
    # up-sweep: node at index i (right end of its span) holds the span total
    d = 1
    while d < n:
        for i in range(2 * d - 1, n, 2 * d):
            A[i], Bv[i] = combine((A[i - d], Bv[i - d]), (A[i], Bv[i]))
            combines += 1
        d *= 2
    # down-sweep to an exclusive scan: root gets the identity
    A[n - 1] = 1.0
    Bv[n - 1] = 0.0
    d = n // 2
    while d >= 1:
        for i in range(2 * d - 1, n, 2 * d):
            left = (A[i - d].copy(), Bv[i - d].copy())
            here = (A[i].copy(), Bv[i].copy())
            # left child takes the prefix arriving at this node
            A[i - d], Bv[i - d] = here
            # right child: prefix, then the left child's span
            A[i], Bv[i] = combine(here, left)
            combines += 1
        d //= 2
    # exclusive prefix P_t applied to h0 = 0 is Bv[t]; inclusive adds step t
    h = a * Bv[:L] + b
    return h, combines


def scan_chunked(a, b, chunk, h0=None):
    """Split the sequence into chunks: reduce each chunk to one affine pair
    (product of a, end state from zero), scan those pairs to obtain each
    chunk's incoming state, then rerun each chunk from its incoming state.
    This is the chunked prefill of the Transformer-math article ("What it
    costs at inference, and on a CPU"): each block is scanned on its own and
    its end state is handed on to the next.
    """
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    L = a.shape[0]
    starts = list(range(0, L, chunk))
    aggs = []
    for s in starts:
        blk_a = a[s:s + chunk]
        blk_b = b[s:s + chunk]
        prod = np.prod(blk_a, axis=0)
        end = scan_sequential(blk_a, blk_b)[-1]
        aggs.append((prod, end))
    h = np.zeros(a.shape[1:]) if h0 is None else np.asarray(h0, dtype=np.float64)
    out = np.empty_like(b)
    for (s, (prod, end)) in zip(starts, aggs):
        out[s:s + chunk] = scan_sequential(a[s:s + chunk], b[s:s + chunk], h0=h)
        h = prod * h + end
    return out
