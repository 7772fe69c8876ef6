"""Host-side checks of the decode driver (no GPU): the offload stack refuses
a step whose window block moves back or jumps ahead by more than one block,
before it enqueues anything (one position per decode step means a window
stays or moves on by one block, and the block it leaves is the only one to
pool and insert)."""
import types

import numpy as np
import pytest

from kv_cache_offload_amd import runner as R


def _stack(B, block):
    st = object.__new__(R.OffloadStack)
    st.layers = [types.SimpleNamespace(B=B)]
    st.block = block
    return st


@pytest.mark.parametrize("prev,new", [(10, 12), (10, 9), (np.array([5, 6, 7]), np.array([6, 8, 7])),
                                      (np.array([5, 6, 7]), np.array([5, 5, 7])), (4, np.array([5, 6, 4]))])
def test_offload_stack_rejects_window_jumps(prev, new):
    st = _stack(3, prev)
    with pytest.raises(ValueError, match="move on by one"):
        st.step(0, [None], None, new)
