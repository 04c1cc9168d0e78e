"""blockattn_fwd_noalloc, the entry point for callers that cannot allocate, against
blockattn_fwd on the same inputs, through the C ABI: several calls in a row on one
device, each smaller than the one before, sharing the library's scratch array.  Where
both entry points launch the same kernels (no key-range split, or a split whose
partials fit the scratch array) the results are bit-identical; where blockattn_fwd
would split and the partials do not fit, the no-allocation call runs unsplit and
agrees to the acceptance tolerances (O within 2e-2 + 1e-2 |ref|, LSE within 1e-3 of
the oracle and of blockattn_fwd)."""

import numpy as np
import pytest
import torch

import oracle
from sequence_parallelism_amd import inputs
from test_gpu_parity import DEV, check_lse, check_o, f64, say

pytestmark = pytest.mark.gpu

# (Sq, Sk, Hq, Hkv, q_start, document lengths, same kernels as blockattn_fwd)
CASES = [
    (16384, 16384, 4, 1, 0, [6000, 10384], True),    # 256 workgroups: no split
    (1792, 4096, 1, 1, 2304, [4096], True),         # split whose partials fit (112 chunks)
    (3000, 3000, 4, 2, 0, [1200, 1800], False),      # split too large: run unsplit
    (1000, 1000, 2, 1, 0, [1000], True),             # short keys: no split
]


def test_noalloc_matches_blockattn_fwd(usp):
    for Sq, Sk, Hq, Hkv, q_start, lengths, same in CASES:
        say("noalloc", Sq, Sk, Hq, Hkv, q_start)
        n = max(q_start + Sq, Sk)
        q, k, v, _, pos = inputs.attention_case(n, Hq, Hkv, 128, seed=Sq + Hq, lengths=lengths)
        q = q[q_start:q_start + Sq].contiguous()
        k, v = k[:Sk].contiguous(), v[:Sk].contiguous()
        qd, kd, vd = (t.to(DEV) for t in (q, k, v))
        posd = torch.from_numpy(pos).to(DEV)
        o_ref, lse_ref = usp.blockattn_fwd(qd, kd, vd, posd, q_start=q_start)
        o = torch.full_like(o_ref, float("nan"))
        lse = torch.full_like(lse_ref, float("nan"))
        usp.blockattn_fwd_noalloc(qd, kd, vd, o, lse, posd, q_start=q_start)
        torch.cuda.synchronize()
        if same:
            assert torch.equal(o, o_ref) and torch.equal(lse, lse_ref), (Sq, Sk, Hq)
        else:
            check_o(o.cpu(), f64(o_ref), ("o vs blockattn_fwd", Sq))
            check_lse(lse, lse_ref.cpu().numpy().astype(np.float64), ("lse vs blockattn_fwd", Sq))
        ref_o, ref_l = oracle.attention_fwd(f64(q), f64(k), f64(v), pos=pos, q_start=q_start,
                                            causal=True)
        check_o(o.cpu(), ref_o, ("o vs oracle", Sq))
        check_lse(lse, ref_l, ("lse vs oracle", Sq))
