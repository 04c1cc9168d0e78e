"""Oracle: the four-device ring example of the Ring Attention glossary page.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Ultralytics glossary, "Ring Attention", section "Como funciona la atencion en anillo":
the sequence is cut into N equal blocks and device i keeps query block i while the
key/value blocks travel round the ring, so that every device sees every key/value
block once.  Per query row a device keeps two running sums over the blocks it has
seen, the exponentiated scores weighted by the values (numerator) and the
exponentiated scores alone (denominator), and divides one by the other at the end.
The page adds that production kernels subtract a running maximum before
exponentiating, for numerical safety.

``ring_sim_raw`` is the first form written as one sum over key blocks (the order in
which a ring delivers the blocks changes only rounding); ``ring_sim_online`` is the
running-maximum form, stepping all devices through the ring at once.  Both equal full
(non-causal) softmax attention in exact arithmetic.  float64 throughout.
"""

import numpy as np


def full_attention_noncausal(q, k, v):
    """softmax(q k^T / sqrt(dim)) v for one head, q, k, v [S][dim]."""
    q, k, v = (np.asarray(a, dtype=np.float64) for a in (q, k, v))
    s = q @ k.T / np.sqrt(q.shape[-1])
    e = np.exp(s - s.max(axis=1, keepdims=True))
    return (e / e.sum(axis=1, keepdims=True)) @ v


def _blocks(a, n):
    a = np.asarray(a, dtype=np.float64)
    if a.shape[0] % n:
        raise ValueError("the sequence must split into equal blocks")
    return a.reshape(n, a.shape[0] // n, a.shape[1])


def ring_sim_raw(q, k, v, n_devices):
    """Raw exponentials, no maximum: for every query, the per-key-block numerators
    (exp(scores) @ values) and denominators (sum of exp(scores)) summed over all
    key blocks, then divided.  q, k, v [S][dim]; returns O [S][dim]."""
    kb, vb = _blocks(k, n_devices), _blocks(v, n_devices)
    q = np.asarray(q, dtype=np.float64)
    dim = q.shape[-1]
    e = np.exp(np.einsum("sd,jbd->sjb", q, kb) / np.sqrt(dim))   # [query][key block][key]
    numer = np.einsum("sjb,jbd->sjd", e, vb).sum(axis=1)
    denom = e.sum(axis=(1, 2))
    return numer / denom[:, None]


def ring_sim_online(q, k, v, n_devices):
    """Running-maximum form.  At ring step t device i holds key/value block
    (i - t) mod N (the block its predecessor held one step earlier) and updates, per
    query row, the running max m, the running denominator l and the running
    numerator; returns (O [S][dim], LSE [S], natural log)."""
    qb, kb, vb = _blocks(q, n_devices), _blocks(k, n_devices), _blocks(v, n_devices)
    n, rows, dim = qb.shape
    m = np.full((n, rows), -np.inf)
    l = np.zeros((n, rows))
    numer = np.zeros((n, rows, dim))
    for t in range(n):
        kt, vt = np.roll(kb, t, axis=0), np.roll(vb, t, axis=0)   # device i: block (i - t) mod n
        s = np.einsum("ird,icd->irc", qb, kt) / np.sqrt(dim)
        m_new = np.maximum(m, s.max(axis=2))
        alpha = np.exp(m - m_new)
        p = np.exp(s - m_new[:, :, None])
        l = alpha * l + p.sum(axis=2)
        numer = alpha[:, :, None] * numer + np.einsum("irc,icd->ird", p, vt)
        m = m_new
    return (numer / l[:, :, None]).reshape(n * rows, dim), (m + np.log(l)).reshape(n * rows)
