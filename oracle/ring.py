"""Oracle: the four-device ring simulation of the Ring Attention glossary page.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Ultralytics glossary, "Ring Attention", section "Como funciona la atencion en anillo":
the sequence is split into N blocks; device i keeps query block i and, at step
``step``, holds key/value block j = (i - step) mod N.  It accumulates a numerator
(sum of exp(score) times values) and a denominator (sum of exp(score)) and
divides them at the end.  The page notes that production kernels also subtract a
running maximum before exponentiating; ``ring_sim_online`` is that form, carrying
per row the running max m, the running denominator l and the running numerator.
Both equal full (non-causal) attention in exact arithmetic.  float64 throughout.
"""

import numpy as np


def full_attention_noncausal(q, k, v):
    """softmax(q k^T / sqrt(dim)) v for one head, q, k, v [S][dim]."""
    q, k, v = (np.asarray(a, dtype=np.float64) for a in (q, k, v))
    s = q @ k.T / np.sqrt(q.shape[-1])
    e = np.exp(s - s.max(axis=1, keepdims=True))
    return (e / e.sum(axis=1, keepdims=True)) @ v


def ring_sim_raw(q, k, v, n_devices):
    """The page's loop: raw exp, numerator/denominator, divide at the end."""
    q, k, v = (np.asarray(a, dtype=np.float64) for a in (q, k, v))
    dim = q.shape[-1]
    qb, kb, vb = (np.split(a, n_devices) for a in (q, k, v))
    outs = []
    for i in range(n_devices):
        num = np.zeros((qb[i].shape[0], dim))
        den = np.zeros((qb[i].shape[0], 1))
        for step in range(n_devices):
            j = (i - step) % n_devices
            p = np.exp(qb[i] @ kb[j].T / np.sqrt(dim))
            num += p @ vb[j]
            den += p.sum(axis=-1, keepdims=True)
        outs.append(num / den)
    return np.concatenate(outs)


def ring_sim_online(q, k, v, n_devices):
    """Running-max form: per row (m, l, acc); returns (O, LSE) with LSE natural-log."""
    q, k, v = (np.asarray(a, dtype=np.float64) for a in (q, k, v))
    dim = q.shape[-1]
    qb, kb, vb = (np.split(a, n_devices) for a in (q, k, v))
    outs, lses = [], []
    for i in range(n_devices):
        rows = qb[i].shape[0]
        m = np.full(rows, -np.inf)
        l = np.zeros(rows)
        acc = np.zeros((rows, dim))
        for step in range(n_devices):
            j = (i - step) % n_devices
            s = qb[i] @ kb[j].T / np.sqrt(dim)
            m_new = np.maximum(m, s.max(axis=1))
            alpha = np.exp(m - m_new)
            p = np.exp(s - m_new[:, None])
            l = alpha * l + p.sum(axis=1)
            acc = alpha[:, None] * acc + p @ vb[j]
            m = m_new
        outs.append(acc / l[:, None])
        lses.append(m + np.log(l))
    return np.concatenate(outs), np.concatenate(lses)
