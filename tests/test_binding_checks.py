"""Host-side argument checks of the Python binding (no GPU needed): position_ids
coverage and well-formedness, dtypes and shapes of inputs and caller-supplied
outputs.  Every check runs before the device check and before any launch, so the
calls below raise on CPU tensors with the specific error they are about."""

import numpy as np
import pytest
import torch

import sequence_parallelism_amd as usp
from sequence_parallelism_amd import inputs


def bf(*shape):
    return torch.zeros(shape, dtype=torch.bfloat16)


def pos_for(n):
    return torch.from_numpy(inputs.position_ids([n]))


def test_position_ids_problem_accepts_packed_documents():
    p = inputs.position_ids([5, 1, 3, 7])
    assert usp.position_ids_problem(p, len(p)) is None
    assert usp.position_ids_problem(p, 3) is None
    assert usp.position_ids_problem(np.zeros(0, np.int32), 0) is None
    assert usp.position_ids_problem(np.zeros(4, np.int32), 4) is None   # four one-token documents


@pytest.mark.parametrize("bad, where", [
    ([1, 2, 3], 0),              # starts inside a document
    ([0, 1, 3], 2),              # skips a position
    ([0, 1, 1], 2),              # repeats a position
    ([0, 1, 2, 5, 6], 3),        # restarts at neither 0 nor +1
])
def test_position_ids_problem_names_the_first_bad_token(bad, where):
    msg = usp.position_ids_problem(np.array(bad, np.int32), len(bad))
    assert msg is not None and f"position_ids[{where}]" in msg
    # a prefix before the problem is fine
    assert usp.position_ids_problem(np.array(bad, np.int32), where) is None


def test_debug_flag_and_environment(monkeypatch):
    monkeypatch.delenv("USP_DEBUG", raising=False)
    assert not usp.debug_enabled()
    assert usp.debug_enabled(True)
    monkeypatch.setenv("USP_DEBUG", "1")
    assert usp.debug_enabled()
    assert not usp.debug_enabled(False)


def test_fwd_rejects_short_position_ids():
    q, k, v = bf(256, 4, 128), bf(256, 1, 128), bf(256, 1, 128)
    with pytest.raises(ValueError, match="position_ids has 255 entries"):
        usp.blockattn_fwd(q, k, v, pos_for(255))
    # global offsets count: keys at k_start + 256 need that many entries
    with pytest.raises(ValueError, match="touches global tokens up to 511"):
        usp.blockattn_fwd(q, k, v, pos_for(300), k_start=256)
    with pytest.raises(ValueError, match="required for causal"):
        usp.blockattn_fwd(q, k, v, None)


def test_fwd_rejects_wrong_position_ids_dtype():
    q, k, v = bf(64, 2, 128), bf(64, 2, 128), bf(64, 2, 128)
    with pytest.raises(TypeError, match="position_ids must be torch.int32"):
        usp.blockattn_fwd(q, k, v, pos_for(64).long())


def test_debug_check_rejects_malformed_position_ids():
    q, k, v = bf(64, 2, 128), bf(64, 2, 128), bf(64, 2, 128)
    p = pos_for(64)
    p[10] = 7
    with pytest.raises(ValueError, match=r"position_ids\[10\] = 7"):
        usp.blockattn_fwd(q, k, v, p, debug=True)
    # without the debug flag the host does not read the values: the call gets as far
    # as the device check
    with pytest.raises(ValueError, match="must be a device tensor"):
        usp.blockattn_fwd(q, k, v, p, debug=False)


def test_fwd_rejects_bad_inputs_and_outputs():
    q, k, v, p = bf(64, 4, 128), bf(64, 2, 128), bf(64, 2, 128), pos_for(64)
    with pytest.raises(ValueError, match="must both have shape"):
        usp.blockattn_fwd(q, k, bf(63, 2, 128), p)
    with pytest.raises(TypeError, match="share one dtype"):
        usp.blockattn_fwd(q, k.float(), v, p)
    with pytest.raises(ValueError, match="multiple of key/value heads"):
        usp.blockattn_fwd(q, bf(64, 3, 128), bf(64, 3, 128), p)
    with pytest.raises(ValueError, match="o must have shape"):
        usp.blockattn_fwd(q, k, v, p, o=bf(64, 4, 64))
    with pytest.raises(TypeError, match="o must be torch.float32"):
        usp.blockattn_fwd(q, k, v, p, o=bf(64, 4, 128), o_dtype=torch.float32)
    with pytest.raises(TypeError, match="lse must be float32"):
        usp.blockattn_fwd(q, k, v, p, lse=torch.zeros(4, 64, dtype=torch.float64))
    with pytest.raises(ValueError, match=r"lse must have shape \(4, >= 64\)"):
        usp.blockattn_fwd(q, k, v, p, lse=torch.zeros(4, 32))
    with pytest.raises(ValueError, match="unit-stride"):
        usp.blockattn_fwd(q, k, v, p, lse=torch.zeros(64, 4).t())
    with pytest.raises(ValueError, match="contiguous"):
        usp.blockattn_fwd(q.transpose(0, 1).contiguous().transpose(0, 1), k, v, p)


def test_bwd_rejects_bad_arguments():
    q, k, v, p = bf(128, 4, 128), bf(128, 1, 128), bf(128, 1, 128), pos_for(128)
    o, do, lse = bf(128, 4, 128), bf(128, 4, 128), torch.zeros(4, 128)
    with pytest.raises(ValueError, match="position_ids has 100 entries"):
        usp.blockattn_bwd(q, k, v, o, lse, do, pos_for(100))
    with pytest.raises(TypeError, match="position_ids must be torch.int32"):
        usp.blockattn_bwd(q, k, v, o, lse, do, p.long())
    with pytest.raises(TypeError, match="bfloat16 inputs only"):
        usp.blockattn_bwd(q.float(), k.float(), v.float(), o.float(), lse, do.float(), p)
    with pytest.raises(ValueError, match="dout must have shape"):
        usp.blockattn_bwd(q, k, v, o, lse, bf(127, 4, 128), p)
    with pytest.raises(TypeError, match="o must be torch.bfloat16"):
        usp.blockattn_bwd(q, k, v, o.float(), lse, do, p)
    with pytest.raises(ValueError, match="dk must have shape"):
        usp.blockattn_bwd(q, k, v, o, lse, do, p, dk=bf(128, 4, 128))
    with pytest.raises(TypeError, match="dv must be torch.bfloat16"):
        usp.blockattn_bwd(q, k, v, o, lse, do, p, dv=torch.zeros(128, 1, 128))


def test_ulysses_rejects_bad_arguments():
    xq, xk, xv = bf(4, 256, 8, 128), bf(4, 256, 4, 128), bf(4, 256, 4, 128)
    p = pos_for(1024)
    with pytest.raises(ValueError, match="position_ids has 1000 entries"):
        usp.ulysses_attn_fwd(xq, xk, xv, 1, pos_for(1000))
    with pytest.raises(ValueError, match="group must be in"):
        usp.ulysses_attn_fwd(xq, xk, xv, 4, p)
    with pytest.raises(ValueError, match="split evenly"):
        usp.ulysses_attn_fwd(bf(4, 256, 6, 128), xk, xv, 0, p)
    with pytest.raises(ValueError, match="o_seq must have shape"):
        usp.ulysses_attn_fwd(xq, xk, xv, 0, p, o_seq=bf(4, 256, 4, 128))
    lse = torch.zeros(2, 1024)
    with pytest.raises(ValueError, match="dxk must have shape"):
        usp.ulysses_attn_bwd(xq, xk, xv, bf(4, 256, 8, 128), lse, bf(4, 256, 8, 128), 0, p,
                             dxk=bf(4, 256, 8, 128))
    with pytest.raises(ValueError, match=r"lse must have shape \(2, >= 1024\)"):
        usp.ulysses_attn_bwd(xq, xk, xv, bf(4, 256, 8, 128), torch.zeros(2, 512),
                             bf(4, 256, 8, 128), 0, p)


def test_striped_needs_the_whole_sequence_of_position_ids():
    q, k, v = bf(64, 2, 128), bf(64, 2, 128), bf(64, 2, 128)
    with pytest.raises(ValueError, match="position_ids has 64 entries"):
        usp.striped_attn_fwd(q, k, v, 4, 1, 0, pos_for(64))
    with pytest.raises(ValueError, match="ranks must be in"):
        usp.striped_attn_fwd(q, k, v, 4, 4, 0, pos_for(256))


def test_permute_and_merge_reject_bad_outputs():
    x = bf(4, 16, 8, 128)
    with pytest.raises(ValueError, match="out must have shape"):
        usp.seq_to_head(x, 4, out=bf(4, 64, 2, 64))
    with pytest.raises(TypeError, match="out must be torch.bfloat16"):
        usp.seq_to_head(x, 4, group=1, out=torch.zeros(64, 2, 128))
    with pytest.raises(ValueError, match="out must have shape"):
        usp.head_to_seq(bf(64, 2, 128), 4, 8, out=bf(4, 16, 4, 128), group=0)
    with pytest.raises(ValueError, match="not a head share"):
        usp.head_to_seq(bf(64, 3, 128), 4, 8, out=bf(4, 16, 8, 128), group=0)
    acc, part = torch.zeros(32, 2, 16), torch.zeros(32, 2, 16)
    with pytest.raises(ValueError, match="o_part must have shape"):
        usp.lse_merge(acc, torch.zeros(2, 32), torch.zeros(16, 2, 16), torch.zeros(2, 32))
    with pytest.raises(ValueError, match=r"lse_part must have shape \(2, >= 32\)"):
        usp.lse_merge(acc, torch.zeros(2, 32), part, torch.zeros(2, 16))
