"""Oracle: exact softmax attention over one GPU's share, with its gradients.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Forward (Ring Attention glossary page, "Como funciona la atencion en anillo": the
full result is softmax(q k^T / sqrt(dim)) v, which the blockwise method reproduces
exactly).  For query head h (key/value head h // (Hq/Hkv)) and query row i:

    s_ij  = scale * <q_i, k_j>                    if key j is visible to row i
          = -inf                                  otherwise
    m_i   = max_j s_ij,  p_ij = exp(s_ij - m_i),  l_i = sum_j p_ij
    O_i   = sum_j p_ij v_j / l_i,   LSE_i = m_i + ln l_i   (natural log)

A row that sees no key gets O_i = 0 and LSE_i = -inf.

Visibility (aitoolresearcher Ulysses SP review, section 3: the causal mask is carried
by O(n) position_ids instead of an n x n mask).  Reading adopted: query row i is the
global token gq = q_start + q_stride i, key j is gk = k_start + k_stride j (strides 1
for contiguous blocks; P for the striped layout of the Ring Attention glossary page,
where rank r holds tokens r, r + P, ...); position_ids restart at 0 at each packed
document, so gq - pos[gq] is the first token of gq's document and

    visible(i, j)  <=>  gq - pos[gq] <= gk <= gq      (causal)
    visible(i, j)  <=>  True                          (non-causal)

Backward (the pages are silent; this is the analytic adjoint of the forward):

    dV_j = sum_i p_ij dO_i / l_i           (P = normalised probabilities)
    dP_ij = <dO_i, v_j>,   D_i = <dO_i, O_i>,   dS_ij = P_ij (dP_ij - D_i)
    dQ_i = scale * sum_j dS_ij k_j,   dK_j = scale * sum_i dS_ij q_i

with dK, dV of a key/value head summed over the query heads that share it.

Evaluation is row-chunked only to bound memory, and the rows of a chunk are
evaluated against the key index interval that can hold visible keys for them:
keys outside [min_i(gq - pos[gq]), max_i gq] have probability exactly zero under
the visibility rule, so leaving them out changes no value.  All arithmetic is
float64.
"""

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

try:
    from threadpoolctl import threadpool_limits
except ImportError:  # pragma: no cover - threadpoolctl is installed in this image
    threadpool_limits = None

_NEG_INF = -np.inf


def _threads(threads):
    if threads is not None:
        return max(1, int(threads))
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def visible_mask(gq, gk, pos, causal):
    """Boolean [len(gq)][len(gk)]: key gk visible to query gq (global indices)."""
    gq = np.asarray(gq, dtype=np.int64)
    gk = np.asarray(gk, dtype=np.int64)
    if not causal:
        return np.ones((gq.size, gk.size), dtype=bool)
    start = gq - np.asarray(pos, dtype=np.int64)[gq]
    return (gk[None, :] >= start[:, None]) & (gk[None, :] <= gq[:, None])


def _key_range(rows_g, pos, causal, k_start, Sk, k_stride=1):
    """Local key interval [lo, hi) that can be visible to any of the global rows:
    local keys j with min(start) <= k_start + k_stride j <= max(gq)."""
    if not causal:
        return 0, Sk
    start = rows_g - np.asarray(pos, dtype=np.int64)[rows_g]
    lo = max(-((k_start - int(start.min())) // k_stride), 0)       # ceil division
    hi = min((int(rows_g.max()) - k_start) // k_stride + 1, Sk)    # floor division
    return lo, max(lo, hi)


def _row_probs(qh, kh, rows_g, keys_g, pos, causal, scale):
    """Scores restricted to visibility, then normalised probabilities.

    Returns (P [n][m], m_i [n], l_i [n]) with P = 0 on rows that see no key.
    """
    s = scale * (qh @ kh.T)
    vis = visible_mask(rows_g, keys_g, pos, causal)
    s = np.where(vis, s, _NEG_INF)
    m = s.max(axis=1) if s.shape[1] else np.full(s.shape[0], _NEG_INF)
    has = np.isfinite(m)
    m_safe = np.where(has, m, 0.0)
    p = np.exp(s - m_safe[:, None])          # exp(-inf) = 0 on hidden keys
    l = p.sum(axis=1)
    P = np.where(has[:, None], p / np.where(has, l, 1.0)[:, None], 0.0)
    return P, m, l


def _chunks(rows, n_keys_hint):
    per = max(1, (1 << 21) // max(1, n_keys_hint))
    return [rows[i:i + per] for i in range(0, rows.size, per)]


def _run(jobs, threads):
    nt = _threads(threads)
    if nt == 1 or len(jobs) == 1:
        return [j() for j in jobs]
    # one BLAS thread per worker: the pool provides the parallelism
    limiter = threadpool_limits(limits=1) if threadpool_limits else None
    try:
        with ThreadPoolExecutor(max_workers=nt) as ex:
            return list(ex.map(lambda j: j(), jobs))
    finally:
        if limiter is not None:
            limiter.restore_original_limits()


def _check(q, k, v, pos, causal):
    if q.ndim != 3 or k.ndim != 3 or v.ndim != 3 or v.shape[:2] != k.shape[:2] \
            or q.shape[2] != k.shape[2]:
        raise ValueError("q [Sq][Hq][D], k [Sk][Hkv][D] and v [Sk][Hkv][Dv] expected")
    if q.shape[1] % k.shape[1]:
        raise ValueError("query heads must be a multiple of key/value heads")
    if causal and pos is None:
        raise ValueError("causal attention needs position_ids")


def attention_fwd(q, k, v, pos=None, q_start=0, k_start=0, causal=False,
                  scale=None, rows=None, threads=None, q_stride=1, k_stride=1):
    """Exact attention.  q [Sq][Hq][D], k, v [Sk][Hkv][D] (any float dtype).

    ``rows``: optional local query rows to evaluate (default all).
    Returns O [n][Hq][D] float64 and LSE [Hq][n] float64 (natural log).
    """
    _check(q, k, v, pos, causal)
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    Sq, Hq, D = q.shape
    Sk, Hkv, _ = k.shape
    grp = Hq // Hkv
    scale = 1.0 / np.sqrt(D) if scale is None else float(scale)
    rows = np.arange(Sq) if rows is None else np.asarray(rows, dtype=np.int64)
    O = np.zeros((rows.size, Hq, v.shape[2]))
    LSE = np.full((Hq, rows.size), _NEG_INF)
    idx = np.arange(rows.size)
    jobs = []
    for h in range(Hq):
        hk = h // grp
        for sel in _chunks(idx, Sk):
            def job(h=h, hk=hk, sel=sel):
                rg = q_start + q_stride * rows[sel]
                lo, hi = _key_range(rg, pos, causal, k_start, Sk, k_stride)
                P, m, l = _row_probs(q[rows[sel], h], k[lo:hi, hk], rg,
                                     k_start + k_stride * np.arange(lo, hi), pos, causal, scale)
                O[sel, h] = P @ v[lo:hi, hk]
                LSE[h, sel] = np.where(np.isfinite(m), m + np.log(np.where(l > 0, l, 1.0)),
                                       _NEG_INF)
            jobs.append(job)
    _run(jobs, threads)
    return O, LSE


def attention_probs(q, k, pos=None, q_start=0, k_start=0, causal=False, scale=None,
                    q_stride=1, k_stride=1):
    """Normalised probabilities P [Hq][Sq][Sk] (small inputs only)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    Sq, Hq, D = q.shape
    Sk, Hkv, _ = k.shape
    scale = 1.0 / np.sqrt(D) if scale is None else float(scale)
    out = np.zeros((Hq, Sq, Sk))
    for h in range(Hq):
        P, _, _ = _row_probs(q[:, h], k[:, h // (Hq // Hkv)], q_start + q_stride * np.arange(Sq),
                             k_start + k_stride * np.arange(Sk), pos, causal, scale)
        out[h] = P
    return out


def attention_bwd(q, k, v, do, pos=None, q_start=0, k_start=0, causal=False,
                  scale=None, rows=None, threads=None, q_stride=1, k_stride=1):
    """Analytic gradients of the forward above for upstream gradient dO [Sq][Hq][D].

    ``rows``: optional local query rows whose contributions are taken (default
    all).  dQ is returned for those rows only ([n][Hq][D]); dK and dV have the
    full key shape and hold the contributions of those rows, which is the whole
    gradient for every key that no other row can see.
    """
    _check(q, k, v, pos, causal)
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    Sq, Hq, D = q.shape
    Sk, Hkv, _ = k.shape
    grp = Hq // Hkv
    scale = 1.0 / np.sqrt(D) if scale is None else float(scale)
    rows = np.arange(Sq) if rows is None else np.asarray(rows, dtype=np.int64)
    dq = np.zeros((rows.size, Hq, D))
    idx = np.arange(rows.size)
    jobs = []
    for h in range(Hq):
        hk = h // grp
        for sel in _chunks(idx, Sk):
            def job(h=h, hk=hk, sel=sel):
                r = rows[sel]
                rg = q_start + q_stride * r
                lo, hi = _key_range(rg, pos, causal, k_start, Sk, k_stride)
                kh, vh = k[lo:hi, hk], v[lo:hi, hk]
                P, _, _ = _row_probs(q[r, h], kh, rg, k_start + k_stride * np.arange(lo, hi),
                                     pos, causal, scale)
                dO = do[r, h]
                O = P @ vh
                dP = dO @ vh.T
                Di = np.sum(dO * O, axis=1)
                dS = P * (dP - Di[:, None])
                dq[sel, h] = scale * (dS @ kh)
                return hk, lo, hi, scale * (dS.T @ q[r, h]), P.T @ dO
            jobs.append(job)
    dk = np.zeros((Sk, Hkv, D))
    dv = np.zeros((Sk, Hkv, v.shape[2]))
    for hk, lo, hi, dk_part, dv_part in _run(jobs, threads):
        dk[lo:hi, hk] += dk_part
        dv[lo:hi, hk] += dv_part
    return dq, dk, dv


def causal_visible_pairs(doc_lengths):
    """Visible (query, key) pairs per head for packed causal documents: sum L(L+1)/2."""
    L = np.asarray(doc_lengths, dtype=np.int64)
    return int(np.sum(L * (L + 1) // 2))
