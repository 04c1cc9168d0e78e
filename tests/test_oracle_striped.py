"""Pins of the striped-layout oracle (Ultralytics glossary "Ring Attention", section
"Como funciona la atencion en anillo", the Striped Attention remark: every rank gets
tokens spread evenly over the sequence; read as rank r holding tokens r, r + P, ...).

Each check ties the oracle to something other than itself: a hand-written layout
example, brute-force probabilities from the visibility definition written out per
(row, key) pair, the identity that the ring over stripes reproduces full attention
of the original sequence, and the degenerate one-rank case."""

import numpy as np
import pytest

import oracle


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _pos(lengths):
    return np.concatenate([np.arange(L, dtype=np.int32) for L in lengths])


def test_stripe_layout_example_and_inverse():
    x = np.arange(12)
    y = oracle.seq_to_stripe(x, 3)
    assert y.tolist() == [[0, 3, 6, 9], [1, 4, 7, 10], [2, 5, 8, 11]]
    assert np.array_equal(oracle.stripe_to_seq(y), x)
    z = _rand((20, 2, 3), 1)
    assert np.array_equal(oracle.stripe_to_seq(oracle.seq_to_stripe(z, 5)), z)
    with pytest.raises(ValueError):
        oracle.seq_to_stripe(np.arange(10), 3)


@pytest.mark.parametrize("P,i,j", [(4, 1, 2), (4, 2, 1), (3, 0, 0), (5, 4, 0)])
def test_stripe_pair_probabilities_brute_force(P, i, j):
    """Probabilities of a stripe pair against a per-pair loop over the definition:
    global query g = i + P a, key t = j + P b, visible iff g - pos[g] <= t <= g."""
    n, D = 9, 4
    lengths = [7, 1, 10, P * n - 18]
    pos = _pos(lengths)
    q = _rand((n, 1, D), 2)
    k = _rand((n, 1, D), 3)
    scale = 0.7
    got = oracle.attention_probs(q, k, pos=pos, q_start=i, k_start=j, causal=True, scale=scale,
                                 q_stride=P, k_stride=P)[0]
    want = np.zeros((n, n))
    for a in range(n):
        g = i + P * a
        s = []
        for b in range(n):
            t = j + P * b
            if g - pos[g] <= t <= g:
                s.append((b, scale * float(q[a, 0] @ k[b, 0])))
        if s:
            m = max(v for _, v in s)
            den = sum(np.exp(v - m) for _, v in s)
            for b, v in s:
                want[a, b] = np.exp(v - m) / den
    assert np.allclose(got, want, atol=1e-14, rtol=0)
    # the forward's key-range restriction gives the same rows
    v = _rand((n, 1, D), 4)
    o, lse = oracle.attention_fwd(q, k, v, pos=pos, q_start=i, k_start=j, causal=True, scale=scale,
                                  q_stride=P, k_stride=P)
    assert np.allclose(o[:, 0], want @ v[:, 0], atol=1e-12)


@pytest.mark.parametrize("P,lengths", [(4, [50, 1, 29, 48]), (8, [128]), (2, [3, 61])])
def test_striped_ring_equals_full_attention(P, lengths):
    S = sum(lengths)
    pos = _pos(lengths)
    q, k, v = _rand((S, 4, 8), 5), _rand((S, 2, 8), 6), _rand((S, 2, 8), 7)
    o_ref, lse_ref = oracle.attention_fwd(q, k, v, pos=pos, causal=True)
    o, lse = oracle.striped_ring_fwd(q, k, v, P, pos=pos, causal=True)
    assert np.allclose(o, o_ref, atol=1e-12)
    assert np.allclose(lse, lse_ref, atol=1e-12)


def test_one_rank_is_the_contiguous_case():
    S = 40
    pos = _pos([17, 23])
    q, k, v = _rand((S, 2, 8), 8), _rand((S, 1, 8), 9), _rand((S, 1, 8), 10)
    a = oracle.striped_pair_fwd(q, k, v, 1, 0, 0, pos=pos)
    b = oracle.attention_fwd(q, k, v, pos=pos, causal=True)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_striped_pairs_are_balanced_under_the_causal_mask():
    """The page's point: with stripes every rank does about the same causal work at
    every ring step, while contiguous blocks leave early ranks idle."""
    P, n = 8, 64
    S = P * n
    pos = np.arange(S, dtype=np.int32)
    q = np.zeros((n, 1, 2))
    work_striped = np.zeros((P, P))
    work_contig = np.zeros((P, P))
    for i in range(P):
        for j in range(P):
            ps = oracle.attention_probs(q, q, pos=pos, q_start=i, k_start=j, causal=True,
                                        q_stride=P, k_stride=P)[0]
            work_striped[i, j] = np.count_nonzero(ps)
            pc = oracle.attention_probs(q, q, pos=pos, q_start=i * n, k_start=j * n, causal=True)[0]
            work_contig[i, j] = np.count_nonzero(pc)
    assert work_striped.sum() == work_contig.sum() == S * (S + 1) // 2
    # every stripe pair holds about half a block of pairs; contiguous pairs are 0, half or full
    assert work_striped.min() >= n * (n - 1) // 2 and work_striped.max() <= n * (n + 1) // 2
    assert work_contig.min() == 0 and work_contig.max() == n * n
