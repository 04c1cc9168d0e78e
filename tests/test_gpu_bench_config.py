"""GPU parity of the benchmark's exact call: usp_ulysses_attn_fwd / usp_ulysses_attn_bwd
on the sequence-sharded layer (8 ranks, 16384 tokens each, 32 query heads, 8 key/value
heads, head dim 128, 16 packed documents), rank 0's share, with the inputs and the
launch configuration bench.py times.  Packed causal attention is exactly per-document
attention, so every one of the 16 documents is compared whole with the oracle: O,
LSE, dQ, dK, dV of rank 0's heads.  The other heads of the outputs stay untouched."""

import numpy as np
import pytest
import torch

import oracle
from sequence_parallelism_amd import inputs
from test_gpu_parity import DEV, check_grad, check_lse, check_o, f64, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("group", [0, 5])
def test_bench_layer_every_document(usp, group):
    say("bench layer, rank", group)
    xq, xk, xv, xdo, posd, lengths = inputs.bench_layer(DEV)
    c = inputs.BENCH_LAYER
    P = c["P"]
    hq, hkv = c["Hq"] // P, c["Hkv"] // P
    S = c["S"]
    ws_f = torch.empty(usp.fwd_workspace_bytes(S, S, hq, hkv, 128), dtype=torch.uint8, device=DEV)
    ws_b = torch.empty(usp.bwd_workspace_bytes(S, S, hq, hkv, 128), dtype=torch.uint8, device=DEV)
    o_seq, lse = usp.ulysses_attn_fwd(xq, xk, xv, group, posd, workspace=ws_f)
    dxq, dxk, dxv = usp.ulysses_attn_bwd(xq, xk, xv, o_seq, lse, xdo, group, posd, workspace=ws_b)
    torch.cuda.synchronize()
    # other ranks' heads untouched (the outputs were allocated zero-filled)
    for t, h in ((o_seq, hq), (dxq, hq), (dxk, hkv), (dxv, hkv)):
        rest = torch.cat([t[:, :, :group * h], t[:, :, (group + 1) * h:]], dim=2)
        assert torch.all(rest == 0)
    share = lambda t: inputs.share_of(t, P, group).cpu()
    q, k, v, do = share(xq), share(xk), share(xv), share(xdo)
    o, dq, dk, dv = share(o_seq), share(dxq), share(dxk), share(dxv)
    lse = lse.cpu()
    del xq, xk, xv, xdo, o_seq, dxq, dxk, dxv
    starts = np.concatenate([[0], np.cumsum(lengths)[:-1]])
    for doc, (a, L) in enumerate(zip(starts, lengths)):
        a, L = int(a), int(L)
        say("  doc", doc, a, L)
        sl = slice(a, a + L)
        dpos = np.arange(L, dtype=np.int32)
        args = (f64(q[sl]), f64(k[sl]), f64(v[sl]))
        ref_o, ref_l = oracle.attention_fwd(*args, pos=dpos, causal=True)
        check_o(o[sl], ref_o, ("o doc", doc))
        check_lse(lse[:, sl], ref_l, ("lse doc", doc))
        rq, rk, rv = oracle.attention_bwd(*args, f64(do[sl]), pos=dpos, causal=True)
        check_grad(dq[sl], rq, ("dq doc", doc))
        check_grad(dk[sl], rk, ("dk doc", doc))
        check_grad(dv[sl], rv, ("dv doc", doc))
