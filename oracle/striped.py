"""Oracle: the striped token layout and ring attention over stripes.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Ultralytics glossary "Ring Attention", section "Como funciona la atencion en anillo",
its Striped Attention remark: instead of contiguous blocks, every device gets tokens
spread evenly over the sequence, so that under a causal mask no device sits idle.
Reading adopted (the page gives no formula): with P ranks, rank r holds tokens
r, r + P, r + 2P, ... in order (S / P of them).

A ring step pairs the queries of stripe i with the keys / values of stripe j.  Its
attention is the plain attention of ``attention_fwd`` with strided global indices
(query row a is token i + P a, key b is token j + P b; the position_ids mask is
unchanged), and the P partial results of a query stripe combine by the cumulative
softmax (``merge.lse_merge``), as the page's ring does for contiguous blocks.
"""

import numpy as np

from .attention import attention_fwd
from .merge import lse_merge


def seq_to_stripe(x, P):
    """[S][...] -> [P][S/P][...] with y[r][j] = x[r + P j]."""
    x = np.asarray(x)
    S = x.shape[0]
    if S % P:
        raise ValueError("sequence length must be a multiple of the rank count")
    return np.stack([x[r::P] for r in range(P)])


def stripe_to_seq(y):
    """[P][n][...] -> [P n][...], the inverse of seq_to_stripe."""
    y = np.asarray(y)
    P, n = y.shape[:2]
    x = np.empty((P * n,) + y.shape[2:], dtype=y.dtype)
    for r in range(P):
        x[r::P] = y[r]
    return x


def striped_pair_fwd(q_s, k_s, v_s, P, i, j, pos=None, causal=True, scale=None):
    """Attention of stripe i's queries against stripe j's keys / values.

    q_s [n][Hq][D], k_s, v_s [n][Hkv][D] are the stripes themselves.  Returns the
    pair's O [n][Hq][D] and LSE [Hq][n] (float64)."""
    return attention_fwd(q_s, k_s, v_s, pos=pos, q_start=i, k_start=j, causal=causal,
                         scale=scale, q_stride=P, k_stride=P)


def striped_ring_fwd(q, k, v, P, pos=None, causal=True, scale=None):
    """Ring attention over P stripes of the sequence q [S][Hq][D], k, v [S][Hkv][D]:
    every query stripe meets every key stripe, partial results are merged in ring
    order, and the stripes are put back in sequence order.  Returns O [S][Hq][D] and
    LSE [Hq][S]."""
    qs, ks, vs = seq_to_stripe(q, P), seq_to_stripe(k, P), seq_to_stripe(v, P)
    n = qs.shape[1]
    Hq = qs.shape[2]
    outs, lses = [], []
    for i in range(P):
        o_acc = np.zeros(qs[i].shape)
        lse_acc = np.full((Hq, n), -np.inf)
        for step in range(P):
            j = (i - step) % P            # the key stripe that reaches rank i at this step
            o_part, lse_part = striped_pair_fwd(qs[i], ks[j], vs[j], P, i, j, pos, causal, scale)
            o_acc, lse_acc = lse_merge(o_acc, lse_acc, o_part, lse_part)
        outs.append(o_acc)
        lses.append(lse_acc)
    O = stripe_to_seq(np.stack(outs))
    LSE = stripe_to_seq(np.stack([l.T for l in lses])).T
    return O, LSE
