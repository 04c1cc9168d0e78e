"""GPU parity over seeded random calls: forward and backward of blockattn through the
C ABI against the fp64 oracle, on shapes nobody picked by hand.

Each case draws a sequence length, query / key-value head counts (GQA ratios 1, 2,
4, 8), a packed-document mix (multinomial lengths, one-token documents allowed),
causal or not, and for causal calls a ring-style query block and key block at
global offsets (rows with no visible key included).  Bars as in
test_gpu_parity.py: O within 2e-2 abs + 1e-2 rel, LSE within 1e-3, gradients within
5e-2 of the reference's max-norm.
"""

import numpy as np
import pytest
import torch

import oracle
from sequence_parallelism_amd import inputs

pytestmark = pytest.mark.gpu

O_ATOL, O_RTOL, LSE_ATOL, GRAD_REL = 2e-2, 1e-2, 1e-3, 5e-2
DEV = "cuda:0"
N_CASES = 48          # small calls (S <= 1600): the 4-wave kernels
N_SPLIT = 16          # S in [2048, 4096], 1-4 query heads: the split key / query ranges


def f64(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def draw_case(i, split=False):
    """Case i of the sweep (independent of the others' draws)."""
    rng = np.random.default_rng(2026 + 7919 * i + (104729 if split else 0))
    S = int(rng.integers(2048, 4097)) if split else int(rng.integers(1, 1601))
    hq = int(rng.choice([1, 2, 4] if split else [1, 2, 4, 8]))
    hkv = int(rng.choice([d for d in (1, 2, 4, 8) if d <= hq and hq % d == 0]))
    causal = bool(rng.random() < 0.8)
    lengths = None
    if causal and S > 1:
        n_docs = int(rng.integers(1, min(6, S) + 1))
        share = rng.dirichlet(np.full(n_docs, 0.4))                          # skewed mix
        lengths = rng.multinomial(S - n_docs, share) + 1                      # every doc >= 1
        lengths = [int(x) for x in lengths]
    qa, qb, ka, kb = 0, S, 0, S
    if causal and rng.random() < 0.5:   # ring-style block pair at global offsets
        qa, qb = sorted(int(x) for x in rng.integers(0, S + 1, size=2))
        ka, kb = sorted(int(x) for x in rng.integers(0, S + 1, size=2))
        if qb == qa:   # at least one query row (the key block may be empty)
            if qa < S:
                qb = qa + 1
            else:
                qa = qb - 1
    return dict(S=S, hq=hq, hkv=hkv, causal=causal, lengths=lengths, qa=qa, qb=qb, ka=ka, kb=kb,
                seed=int(rng.integers(1 << 30)))


@pytest.mark.parametrize("i,split", [(i, False) for i in range(N_CASES)] +
                         [(i, True) for i in range(N_SPLIT)])
def test_random_call_fwd_bwd(usp, i, split):
    c = draw_case(i, split)
    print("random case", i, "split" if split else "small", c, flush=True)
    S, hq, hkv, causal = c["S"], c["hq"], c["hkv"], c["causal"]
    qa, qb, ka, kb = c["qa"], c["qb"], c["ka"], c["kb"]
    if qb <= qa:
        pytest.skip("empty query block")
    q, k, v, do, pos = inputs.attention_case(S, hq, hkv, 128, seed=c["seed"], lengths=c["lengths"])
    qs, ks, vs, dos = q[qa:qb], k[ka:kb], v[ka:kb], do[qa:qb]
    qd, kd, vd, dod = (t.to(DEV).contiguous() for t in (qs, ks, vs, dos))
    posd = torch.from_numpy(pos).to(DEV) if causal else None
    o, lse = usp.blockattn_fwd(qd, kd, vd, posd, q_start=qa, k_start=ka, causal=causal)
    dq, dk, dv = usp.blockattn_bwd(qd, kd, vd, o, lse, dod, posd, q_start=qa, k_start=ka, causal=causal)
    torch.cuda.synchronize()

    kw = dict(pos=pos, q_start=qa, k_start=ka, causal=True) if causal else dict(causal=False)
    args = (f64(qs), f64(ks), f64(vs))
    ref_o, ref_l = oracle.attention_fwd(*args, **kw)
    og = f64(o)
    err = np.abs(og - ref_o)
    assert np.all(err <= O_ATOL + O_RTOL * np.abs(ref_o)), ("o", float(err.max()))
    lg = lse.detach().cpu().numpy().astype(np.float64)
    fin = np.isfinite(ref_l)
    assert np.array_equal(np.isfinite(lg), fin), "lse finiteness"
    assert np.all(lg[~fin] == ref_l[~fin])
    if fin.any():
        assert np.abs(lg[fin] - ref_l[fin]).max() <= LSE_ATOL, ("lse", float(np.abs(lg[fin] - ref_l[fin]).max()))
    assert np.all(og[np.repeat(~fin.T[:, :, None], og.shape[2], axis=2)] == 0), "rows with no key: O = 0"

    grads = oracle.attention_bwd(*args, f64(dos), **kw)
    for name, g, r in zip(("dq", "dk", "dv"), (dq, dk, dv), grads):
        den = max(np.abs(r).max(), 1e-3)
        rel = np.abs(f64(g) - r).max() / den
        assert rel <= GRAD_REL, (name, float(rel))
