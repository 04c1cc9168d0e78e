"""GPU parity at sizes whose launch orders exceed what the schedule kernels sort in
LDS (12288 units): more than 12288 key blocks of 128 keys for the dK/dV kernel, more
than 12288 query tiles of 256 rows for the forward and dQ kernels, which then run
their units in natural order.  Checked against the oracle on sampled rows, and at
every key / row through properties that hold at any size: with all keys visible,
sum_j dK_j = 0 (the rows of dS sum to zero) and sum_j dV_j = sum_i dO_i summed over
the query heads of a group (the rows of P sum to one); gradients are written over
NaN so that a unit that never ran shows.  Also a causal launch past the 8192 query
tiles whose first visible keys the dK/dV schedule keeps in LDS."""

import numpy as np
import pytest
import torch

import oracle
from sequence_parallelism_amd import inputs
from test_gpu_parity import DEV, check_grad, check_lse, check_o, f64, say
from test_gpu_workloads import sample_rows

pytestmark = pytest.mark.gpu


def _case(Sq, Sk, Hq, Hkv, seed):
    gen = inputs.generator(seed)
    return (inputs.normal((Sq, Hq, 128), gen), inputs.normal((Sk, Hkv, 128), gen),
            inputs.normal((Sk, Hkv, 128), gen), inputs.normal((Sq, Hq, 128), gen))


def _run(usp, q, k, v, do):
    qd, kd, vd, dod = (t.to(DEV) for t in (q, k, v, do))
    o, lse = usp.blockattn_fwd(qd, kd, vd, None, causal=False)
    nan = lambda t: torch.full_like(t, float("nan"))
    dq, dk, dv = usp.blockattn_bwd(qd, kd, vd, o, lse, dod, None, causal=False,
                                   dq=nan(qd), dk=nan(kd), dv=nan(vd))
    torch.cuda.synchronize()
    return dod, o, lse, dq, dk, dv


def _rss(t):
    """root-sum-square over dim 0: the size of a sum of these terms without cancellation"""
    return t.double().pow(2).sum(0).sqrt()


def _check_sums(dod, dk, dv, Hq, Hkv):
    """The identities to 5% of the terms' root-sum-square: the bf16 rounding of the
    outputs and of P inside the kernels is ~0.2% of it, while a key block or a row
    that went missing or twice shifts a sum by a sizeable fraction of its terms."""
    for name, t in (("dk", dk), ("dv", dv)):
        assert bool(torch.isfinite(t).all()), name
    grp = Hq // Hkv
    sk = dk.double().sum(0)
    assert (sk.abs() <= 0.05 * _rss(dk)).all(), "sum_j dK_j = 0"
    dog = dod.double().reshape(dod.shape[0], Hkv, grp, 128)
    want = dog.sum((0, 2))
    got = dv.double().sum(0)
    tol = 0.05 * (_rss(dv) + dog.pow(2).sum((0, 2)).sqrt())
    assert ((got - want).abs() <= tol).all(), "sum_j dV_j = sum_i dO_i"


@pytest.mark.parametrize("Sq,Sk,Hq,Hkv", [
    (64, 12300 * 128, 2, 1),      # 12300 key blocks
    (12300 * 256, 256, 1, 1),     # 12300 query tiles
])
def test_large_grids_sampled_and_sums(usp, Sq, Sk, Hq, Hkv):
    say("large grids", Sq, Sk, Hq, Hkv)
    q, k, v, do = _case(Sq, Sk, Hq, Hkv, seed=51)
    dod, o, lse, dq, dk, dv = _run(usp, q, k, v, do)
    assert bool(torch.isfinite(dq).all()), "dq"
    _check_sums(dod, dk, dv, Hq, Hkv)
    rows = sample_rows(Sq, 8, 52, tile=min(128, Sq // 2))
    rd = torch.from_numpy(rows).to(DEV)
    k64, v64 = f64(k), f64(v)
    ref_o, ref_l = oracle.attention_fwd(f64(q[rows]), k64, v64, causal=False)
    check_o(o[rd].cpu(), ref_o, "o")
    check_lse(lse[:, rd].cpu(), ref_l, "lse")
    rq, _, _ = oracle.attention_bwd(f64(q[rows]), k64, v64, f64(do[rows]), causal=False)
    check_grad(dq[rd].cpu(), rq, "dq")


def test_causal_beyond_schedule_tile_table(usp):
    """Causal packed documents over 8193 query tiles of 64 rows, one more than the dK/dV
    schedule keeps in LDS for its binary searches (which then read position_ids): one
    whole document in the middle checked against the oracle run on that document alone
    (packed documents do not see each other), and every output finite (written over NaN)."""
    S = 8193 * 64
    say("causal beyond the schedule's tile table", S)
    lengths = inputs.doc_lengths(S, 64, 53)
    q, k, v, do, pos = inputs.attention_case(S, 1, 1, 128, seed=54, lengths=lengths)
    qd, kd, vd, dod = (t.to(DEV) for t in (q, k, v, do))
    posd = torch.from_numpy(pos).to(DEV)
    o, lse = usp.blockattn_fwd(qd, kd, vd, posd, causal=True)
    nan = lambda t: torch.full_like(t, float("nan"))
    dq, dk, dv = usp.blockattn_bwd(qd, kd, vd, o, lse, dod, posd, causal=True,
                                   dq=nan(qd), dk=nan(kd), dv=nan(vd))
    torch.cuda.synchronize()
    for name, t in (("dq", dq), ("dk", dk), ("dv", dv)):
        assert bool(torch.isfinite(t).all()), name
    starts = np.concatenate([[0], np.cumsum(lengths)])
    d = len(lengths) // 2
    a, b = int(starts[d]), int(starts[d + 1])
    qs, ks, vs, ds = f64(q[a:b]), f64(k[a:b]), f64(v[a:b]), f64(do[a:b])
    dpos = pos[a:b]   # the document alone: its positions 0 .. L-1
    ref_o, ref_l = oracle.attention_fwd(qs, ks, vs, pos=dpos, causal=True)
    check_o(o[a:b].cpu(), ref_o, "o")
    check_lse(lse[:, a:b].cpu(), ref_l, "lse")
    rq, rk, rv = oracle.attention_bwd(qs, ks, vs, ds, pos=dpos, causal=True)
    check_grad(dq[a:b].cpu(), rq, "dq")
    check_grad(dk[a:b].cpu(), rk, "dk")
    check_grad(dv[a:b].cpu(), rv, "dv")


def test_causal_query_block_past_sorted_key_blocks(usp):
    """A ring-style causal call whose key block is more than 12288 key blocks long (a
    ragged last block included): the dK/dV schedule then keeps natural order and works
    out every block's query tiles from position_ids alone.  The 200 query rows are the
    last tokens of the sequence, inside its last document of 1000 tokens; every key
    before that document gets dK = dV = 0 exactly (no row sees it, and every unit writes
    its block over the NaN fill), and the document's keys, the output and dQ match the
    oracle run on that document alone."""
    T, L, Sq = 12300 * 128 + 77, 1000, 200
    say("causal query block past the sorted key blocks", T, L, Sq)
    lengths = [T - L - 333, 333, L]
    pos = inputs.position_ids(lengths)
    gen = inputs.generator(55)
    q, do = inputs.normal((Sq, 2, 128), gen), inputs.normal((Sq, 2, 128), gen)
    k, v = inputs.normal((T, 1, 128), gen), inputs.normal((T, 1, 128), gen)
    qd, kd, vd, dod = (t.to(DEV) for t in (q, k, v, do))
    posd = torch.from_numpy(pos).to(DEV)
    qa = T - Sq
    o, lse = usp.blockattn_fwd(qd, kd, vd, posd, q_start=qa, k_start=0, causal=True)
    nan = lambda t: torch.full_like(t, float("nan"))
    dq, dk, dv = usp.blockattn_bwd(qd, kd, vd, o, lse, dod, posd, q_start=qa, k_start=0, causal=True,
                                   dq=nan(qd), dk=nan(kd), dv=nan(vd))
    torch.cuda.synchronize()
    for name, t in (("dq", dq), ("dk", dk), ("dv", dv)):
        assert bool(torch.isfinite(t).all()), name
    assert not bool(dk[:T - L].any()) and not bool(dv[:T - L].any()), "keys no row sees"
    dpos = np.arange(L, dtype=np.int32)
    args = (f64(q), f64(k[T - L:]), f64(v[T - L:]))
    kw = dict(pos=dpos, q_start=L - Sq, k_start=0, causal=True)
    ref_o, ref_l = oracle.attention_fwd(*args, **kw)
    check_o(o.cpu(), ref_o, "o")
    check_lse(lse.cpu(), ref_l, "lse")
    rq, rk, rv = oracle.attention_bwd(*args, f64(do), **kw)
    check_grad(dq.cpu(), rq, "dq")
    check_grad(dk[T - L:].cpu(), rk, "dk")
    check_grad(dv[T - L:].cpu(), rv, "dv")
