"""The device-side input validator (pav2_check_inputs) on valid and on
deliberately inconsistent block tables / sequence lengths.  The validator
only reads the tables; nothing here runs the decode kernels on bad data."""
import pytest
import torch

import decode_attention_paged_v2_amd as pav2
from decode_attention_paged_v2_amd import workloads as W

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _tables():
    wl = W.generate(W.SMALL_SPECS["ragged_alibi"])
    return wl.block_tables.clone(), wl.seq_lens.clone(), wl.block_size, wl.num_blocks


def test_valid_inputs_pass():
    bt, sl, bs, nb = _tables()
    r = pav2.check_inputs(bt.to(DEV), sl.to(DEV), bs, nb)
    assert r == {"bad_sequences": 0, "first_sequence": -1, "first_column": -1, "value": 0}


def test_first_violation_is_reported():
    bt, sl, bs, nb = _tables()
    S, mbps = bt.shape
    used = [(s, (int(L) + bs - 1) // bs) for s, L in enumerate(sl.tolist())]
    with_blocks = [s for s, n in used if n >= 3]
    a, b = with_blocks[1], with_blocks[-1]
    bt[b, 0] = -5                      # a later sequence with a negative block id
    bt[a, 2] = nb                      # the first offending sequence: a block past the pool
    c = with_blocks[2]
    sl[c] = mbps * bs + 1              # a length past the table row
    r = pav2.check_inputs(bt.to(DEV), sl.to(DEV), bs, nb)
    assert r == {"bad_sequences": 3, "first_sequence": a, "first_column": 2, "value": nb}


def test_bad_length_and_unused_padding():
    bt, sl, bs, nb = _tables()
    S, mbps = bt.shape
    # entries past a sequence's used blocks are not checked (padding)
    s0 = next(s for s, L in enumerate(sl.tolist()) if 0 < L and (L + bs - 1) // bs < mbps)
    bt[s0, (int(sl[s0]) + bs - 1) // bs:] = -7
    r = pav2.check_inputs(bt.to(DEV), sl.to(DEV), bs, nb)
    assert r["bad_sequences"] == 0
    sl[0] = -1
    r = pav2.check_inputs(bt.to(DEV), sl.to(DEV), bs, nb)
    assert r == {"bad_sequences": 1, "first_sequence": 0, "first_column": -1, "value": -1}


def test_empty_batch():
    r = pav2.check_inputs(torch.zeros((0, 4), dtype=torch.int32, device=DEV),
                          torch.zeros((0,), dtype=torch.int32, device=DEV), 16, 10)
    assert r["bad_sequences"] == 0 and r["first_sequence"] == -1
