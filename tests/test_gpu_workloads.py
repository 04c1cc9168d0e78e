"""GPU parity at the full workload sizes: every output of the Ulysses share (one
32768-token document), every document of the packed 128K input whole (packed
attention is exactly per-document attention), and sampled rows of the 256K ring
(a row's output needs only its own row of scores)."""

import numpy as np
import pytest
import torch

import oracle
from sequence_parallelism_amd import inputs
from test_gpu_parity import (DEV, check_grad, check_lse, check_o, f64, say, to_dev)

pytestmark = pytest.mark.gpu


def sample_rows(S, n, seed, tile=128):
    rng = np.random.default_rng(seed)
    fixed = [0, 1, tile - 1, tile, S // 2, S - tile, S - 2, S - 1]
    return np.unique(np.concatenate([fixed, rng.integers(0, S, n)]))


def test_ulysses_sp8_share_fwd_bwd(usp):
    """[8 ranks][4096][32 heads][128] -> rank 0's share [32768][4][128]; causal
    attention on its 4 heads; inverse re-layout of O and of the gradients."""
    say("ulysses sp8 share")
    P, S_l, H, D = 8, 4096, 32, 128
    xq, xk, xv, xdo, pos = inputs.ulysses_sp8()
    S = P * S_l
    share = lambda x: f64(torch.from_numpy(oracle.seq_to_head(x.view(torch.int16).numpy(), group=0)
                                           .copy()).view(torch.bfloat16))
    q64, k64, v64, do64 = share(xq), share(xk), share(xv), share(xdo)
    dq_, dk_, dv_, do_ = to_dev(xq, xk, xv, xdo)
    posd = torch.from_numpy(pos).to(DEV)
    q = usp.seq_to_head(dq_, P, group=0)
    k = usp.seq_to_head(dk_, P, group=0)
    v = usp.seq_to_head(dv_, P, group=0)
    o, lse = usp.blockattn_fwd(q, k, v, posd)
    o_seq = torch.zeros_like(dq_)
    usp.head_to_seq(o, P, H, out=o_seq, group=0)
    dO = usp.seq_to_head(do_, P, group=0)
    dq, dk, dv = usp.blockattn_bwd(q, k, v, o, lse, dO, posd)
    g_seq = [torch.zeros_like(dq_) for _ in range(3)]
    for gs, gt in zip(g_seq, (dq, dk, dv)):
        usp.head_to_seq(gt, P, H, out=gs, group=0)
    torch.cuda.synchronize()
    del dk_, dv_
    assert torch.all(o_seq[:, :, 4:] == 0)            # other ranks' heads untouched

    # every output of rank 0's share (one 32768-token document, 4 heads)
    ref_o, ref_l = oracle.attention_fwd(q64, k64, v64, pos=pos, causal=True)
    check_o(o_seq[:, :, :4].reshape(S, 4, D).cpu(), ref_o, "o via head_to_seq")
    check_lse(lse.cpu(), ref_l, "lse")
    rq, rk, rv = oracle.attention_bwd(q64, k64, v64, do64, pos=pos, causal=True)
    check_grad(g_seq[0][:, :, :4].reshape(S, 4, D).cpu(), rq, "dq")
    check_grad(g_seq[1][:, :, :4].reshape(S, 4, D).cpu(), rk, "dk")
    check_grad(g_seq[2][:, :, :4].reshape(S, 4, D).cpu(), rv, "dv")


def test_packed_128k_fwd_bwd(usp):
    """S = 131072, 4 query heads sharing 1 key/value head, 16 packed documents."""
    say("packed 128k")
    q, k, v, do, pos, lengths = inputs.packed_128k()
    qd, kd, vd, dod = to_dev(q, k, v, do)
    posd = torch.from_numpy(pos).to(DEV)
    o, lse = usp.blockattn_fwd(qd, kd, vd, posd)
    dq, dk, dv = usp.blockattn_bwd(qd, kd, vd, o, lse, dod, posd)
    torch.cuda.synchronize()
    starts = np.concatenate([[0], np.cumsum(lengths)[:-1]])
    for doc in range(len(lengths)):                    # every document, whole
        a, L = int(starts[doc]), int(lengths[doc])
        say("  doc", doc, a, L)
        sl = slice(a, a + L)
        dpos = np.arange(L, dtype=np.int32)
        args = (f64(q[sl]), f64(k[sl]), f64(v[sl]))
        ref_o, ref_l = oracle.attention_fwd(*args, pos=dpos, causal=True)
        check_o(o[sl].cpu(), ref_o, ("o doc", doc))
        check_lse(lse[:, sl].cpu(), ref_l, ("lse doc", doc))
        rq, rk, rv = oracle.attention_bwd(*args, f64(do[sl]), pos=dpos, causal=True)
        check_grad(dq[sl].cpu(), rq, ("dq doc", doc))
        check_grad(dk[sl].cpu(), rk, ("dk doc", doc))
        check_grad(dv[sl].cpu(), rv, ("dv doc", doc))
    rows = sample_rows(131072, 64, 2)
    ref_o, ref_l = oracle.attention_fwd(f64(q), f64(k), f64(v), pos=pos, causal=True, rows=rows)
    check_o(o[rows].cpu(), ref_o, "o sampled rows")
    check_lse(lse[:, rows].cpu(), ref_l, "lse sampled rows")


def test_single_doc_causal_128k_fwd_bwd(usp):
    """The packed 128K tensors as ONE causal document (position_ids 0..131071): O and
    LSE at sampled rows, dQ at sampled rows, and dK, dV of the last 128 keys, which
    only the last 128 rows see (so those rows' contributions are their whole
    gradient)."""
    say("single-document causal 128k")
    q, k, v, do, _, _ = inputs.packed_128k()
    S = q.shape[0]
    pos = np.arange(S, dtype=np.int32)
    qd, kd, vd, dod = to_dev(q, k, v, do)
    posd = torch.from_numpy(pos).to(DEV)
    o, lse = usp.blockattn_fwd(qd, kd, vd, posd)
    dq, dk, dv = usp.blockattn_bwd(qd, kd, vd, o, lse, dod, posd)
    torch.cuda.synchronize()
    args = (f64(q), f64(k), f64(v))
    rows = sample_rows(S, 24, 3)
    ref_o, ref_l = oracle.attention_fwd(*args, pos=pos, causal=True, rows=rows)
    check_o(o[rows].cpu(), ref_o, "o sampled rows")
    check_lse(lse[:, rows].cpu(), ref_l, "lse sampled rows")
    rq, _, _ = oracle.attention_bwd(*args, f64(do), pos=pos, causal=True, rows=rows)
    check_grad(dq[rows].cpu(), rq, "dq sampled rows")
    tail = np.arange(S - 128, S)
    _, rk, rv = oracle.attention_bwd(*args, f64(do), pos=pos, causal=True, rows=tail)
    check_grad(dk[S - 128:].cpu(), rk[S - 128:], "dk last 128 keys")
    check_grad(dv[S - 128:].cpu(), rv[S - 128:], "dv last 128 keys")


def test_ring_256k_blockwise_merge(usp):
    """S = 262144, 2 heads, causal: query block i (16384 rows) attends key blocks
    0..i one call at a time (fp32 partials), merged into an accumulator
    initialised to (0, -inf)."""
    say("ring 256k")
    q, k, v, pos = inputs.ring_256k()
    S, H, D, nb = 262144, 2, 128, 16
    blk = S // nb
    qd, kd, vd = to_dev(q, k, v)
    posd = torch.from_numpy(pos).to(DEV)
    acc = torch.zeros((S, H, D), dtype=torch.float32, device=DEV)
    acc_l = torch.full((H, S), -float("inf"), dtype=torch.float32, device=DEV)
    po = torch.empty((blk, H, D), dtype=torch.float32, device=DEV)
    pl = torch.empty((H, blk), dtype=torch.float32, device=DEV)
    for i in range(nb):
        qs = slice(i * blk, (i + 1) * blk)
        for j in range(i + 1):
            ks = slice(j * blk, (j + 1) * blk)
            usp.blockattn_fwd(qd[qs], kd[ks], vd[ks], posd, q_start=i * blk, k_start=j * blk,
                              o=po, lse=pl)
            usp.lse_merge(acc[qs], acc_l[:, qs], po, pl)
    torch.cuda.synchronize()
    rows = sample_rows(S, 40, 3, tile=blk)
    ref_o, ref_l = oracle.attention_fwd(f64(q), f64(k), f64(v), pos=pos, causal=True, rows=rows)
    check_o(acc[rows].cpu(), ref_o, "merged o")
    check_lse(acc_l[:, rows].cpu(), ref_l, "merged lse")
