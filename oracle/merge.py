"""The printed forms of the partial-result merge, in float64 (test infrastructure only).

All four must agree with each other and with one full softmax; the tests pin
them that way.  Empty partials (m = -inf or LSE = -inf) carry zero weight.
"""
from __future__ import annotations

import numpy as np


def _w(a, ref):
    """exp(a - ref) with exp(-inf - finite) = 0."""
    a = np.asarray(a, dtype=np.float64)
    with np.errstate(invalid="ignore"):
        out = np.exp(a - ref)
    return np.where(np.isneginf(a), 0.0, out)


def por_pair(O1, m1, s1, O2, m2, s2):
    """CoDec's binary POR merge (section 块内内核原语, POR kernel paragraph).

    m = max(m1, m2); s = s1 e^{m1-m} + s2 e^{m2-m};
    O = (O1 s1 e^{m1-m} + O2 s2 e^{m2-m}) / s.
    ``O*`` are normalised partial outputs [..., d]; ``m*``, ``s*`` the row
    maximum and the sum of exponentials relative to it.
    """
    m = np.maximum(m1, m2)
    a1 = np.asarray(s1) * _w(m1, m)
    a2 = np.asarray(s2) * _w(m2, m)
    s = a1 + a2
    # A side with zero weight (an empty partial) contributes nothing, even if its O is undefined.
    t1 = np.where(a1[..., None] > 0, np.asarray(O1) * a1[..., None], 0.0)
    t2 = np.where(a2[..., None] > 0, np.asarray(O2) * a2[..., None], 0.0)
    with np.errstate(invalid="ignore", divide="ignore"):
        O = np.where(s[..., None] > 0, (t1 + t2) / s[..., None], 0.0)
    return O, m, s


def por_chain(parts):
    """Fold a list of (O, m, s) with :func:`por_pair`, left to right.

    CoDec (section 块间启动与树归约) turns the tree reduction into one
    independent chain per query; the merge is associative and commutative, so
    any order gives the same value.
    """
    O, m, s = parts[0]
    for O2, m2, s2 in parts[1:]:
        O, m, s = por_pair(O, m, s, O2, m2, s2)
    return O, m, s


def flashdecoding_merge(outs, ms, ls):
    """FlashDecoding's second-level reduction of G partials.

    KV cache engineering blog (KV cache 优化工程实战 2026), section 4
    (FlashDecoding): out = sum_g exp(m_g - m*) l_g out_g / sum_g exp(m_g - m*) l_g
    with m* = max_g m_g.  ``outs`` [G, ..., d], ``ms``/``ls`` [G, ...].
    """
    outs = np.asarray(outs, dtype=np.float64)
    ms = np.asarray(ms, dtype=np.float64)
    ls = np.asarray(ls, dtype=np.float64)
    mstar = ms.max(axis=0)
    a = _w(ms, mstar) * ls
    return (a[..., None] * outs).sum(axis=0) / a.sum(axis=0)[..., None]


def lse_merge(outs, lses):
    """Merge normalised partials by their natural-log LSE (DEFT, section 速读 and A.4).

    L* = max_i LSE_i; w_i = exp(LSE_i - L*); O = sum w_i O_i / sum w_i;
    LSE = L* + ln sum w_i.  ``outs`` [G, ..., d], ``lses`` [G, ...].
    """
    outs = np.asarray(outs, dtype=np.float64)
    lses = np.asarray(lses, dtype=np.float64)
    lstar = lses.max(axis=0)
    w = _w(lses, lstar)
    z = w.sum(axis=0)
    return (w[..., None] * outs).sum(axis=0) / z[..., None], lstar + np.log(z)


def streaming_merge(parts):
    """CoDec's streaming accumulators over nodes (section KV缓存管理, last paragraph).

    Each part is the unnormalised node contribution (m, d, u): m the node's
    row maximum, d = sum_j e^{s_j - m}, u = sum_j e^{s_j - m} V_j.  The global
    accumulators (M, D, U) are updated at the common reference
    M^ = max(M, m): D <- D e^{M - M^} + d e^{m - M^}, U likewise, M <- M^.
    Returns O = U / D and LSE = M + ln D.
    """
    M, D, U = None, None, None
    for m, d, u in parts:
        m = np.asarray(m, dtype=np.float64)
        d = np.asarray(d, dtype=np.float64)
        u = np.asarray(u, dtype=np.float64)
        if M is None:
            M, D, U = m, d, u
            continue
        Mh = np.maximum(M, m)
        a, b = _w(M, Mh), _w(m, Mh)
        D = D * a + d * b
        U = U * a[..., None] + u * b[..., None]
        M = Mh
    return U / D[..., None], M + np.log(D)
