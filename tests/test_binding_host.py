"""CPU tests of the Python binding's argument checks: the C ABI trusts raw
pointers (block-table rows are read max_pages_per_seq entries long, logits
written batch x vocab floats), so Decoder.step checks shapes, dtypes and
placement first and raises MkError before any call."""
import ctypes

import numpy as np
import pytest
import torch

from persistent_megakernel_03_amd import configs, mk

CFG = configs.TINY
V = CFG["vocab"]


def _args(B=2, pages=6):
    dims = mk.make_dims(CFG, 4, pages, 32)
    return (dims, [5, 9][:B] + [0] * max(0, B - 2), np.zeros((B, pages), np.int32),
            torch.zeros(B, dtype=torch.int32), torch.zeros(B, V, dtype=torch.float32))


def test_valid_arguments_pass_and_come_back_as_int32():
    dims, pos, bt, tok, lg = _args()
    p, b = mk.check_step_args(dims, V, pos, bt, tok, lg, "cpu")
    assert p.dtype == np.int32 and b.dtype == np.int32 and b.flags.c_contiguous and b.shape == (2, 6)


@pytest.mark.parametrize("what", ["short_rows", "few_rows", "small_logits", "narrow_logits", "tok_dtype",
                                  "logit_dtype", "device", "noncontig", "few_tokens", "empty", "seq_ids"])
def test_bad_arguments_raise_before_the_call(what):
    dims, pos, bt, tok, lg = _args()
    seq = None
    if what == "short_rows":
        bt = np.zeros((2, 5), np.int32)           # rows shorter than max_pages_per_seq: a heap over-read
    elif what == "few_rows":
        bt = np.zeros((1, 6), np.int32)
    elif what == "small_logits":
        lg = torch.zeros(1, V, dtype=torch.float32)   # device writes past the end
    elif what == "narrow_logits":
        lg = torch.zeros(2, V // 2, dtype=torch.float32)
    elif what == "tok_dtype":
        tok = torch.zeros(2, dtype=torch.int64)
    elif what == "logit_dtype":
        lg = torch.zeros(2, V, dtype=torch.float16)
    elif what == "device":
        tok = torch.zeros(2, dtype=torch.int32, device="meta")
    elif what == "noncontig":
        lg = torch.zeros(V, 2, dtype=torch.float32).t()
    elif what == "few_tokens":
        tok = torch.zeros(1, dtype=torch.int32)
    elif what == "empty":
        pos = []
    elif what == "seq_ids":
        seq = [1]
    with pytest.raises(mk.MkError) as e:
        mk.check_step_args(dims, V, pos, bt, tok, lg, "cpu", seq)
    assert e.value.status == mk.MK_ERR_INVALID


def test_plan_validation_option_is_in_the_options_struct():
    o = mk.make_options(validate_plans=True)
    assert o.validate_plans == 1 and o.mfma_min_batch == 0 and o.poison_exchange == 0
    assert mk.make_options(poison_exchange=True).poison_exchange == 1
    assert o.mm_row_blocks == 0 and mk.make_options(mm_row_blocks=2).mm_row_blocks == 2
    # the C struct: 8-byte watchdog after two words, ten more words (the last one padding)
    assert ctypes.sizeof(mk.mk_options) == 56
    assert mk.mk_options.mm_row_blocks.offset == 48
