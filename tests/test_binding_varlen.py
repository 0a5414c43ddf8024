"""The Python binding's host-side check of packed-sequence offsets (no GPU needed): the
contract of fa_fwd_varlen ("FlashAttention-2 and -3", section "Variable-length batches without
padding": offsets of length num_seqs + 1 starting at 0)."""
import numpy as np
import pytest

from io_aware_softmax_03_amd import check_cu_seqlens


def test_good_offsets():
    assert check_cu_seqlens([0, 5, 5, 12], 12) == 7
    assert check_cu_seqlens(np.array([0, 3], dtype=np.int32), 3, max_seqlen=3) == 3
    assert check_cu_seqlens([0], 0) == 0


@pytest.mark.parametrize("cu,T,max_seqlen,msg", [
    ([1, 5, 12], 12, None, "start with 0"),          # the page's stub without the leading 0
    ([0, 7, 5, 12], 12, None, "nondecreasing"),
    ([0, 5, 11], 12, None, "end at total_tokens"),
    ([0, 5, 13], 12, None, "end at total_tokens"),
    ([0, 5, 12], 12, 6, "exceeds max_seqlen"),
    ([], 0, None, "start with 0"),
])
def test_bad_offsets_raise(cu, T, max_seqlen, msg):
    with pytest.raises(ValueError, match=msg):
        check_cu_seqlens(cu, T, max_seqlen)
