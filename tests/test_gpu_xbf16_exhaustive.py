"""fp32 -> bf16 round to nearest even on the GPU against the oracle over every
one of the 2^32 binary32 bit patterns, in 64 chunks of 2^26.

Non-NaN inputs must give identical bits; NaN inputs must give a NaN (the
payload bits of a NaN are not specified). The bit patterns are generated on
the host; the expected values come from the oracle alone.
"""
import numpy as np
import pytest
import torch

import oracle as O
from gpu_util import need_gpu, say

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
CHUNK = 1 << 26


def test_bf16_round_every_bit_pattern():
    need_gpu()
    import adamw_optimizer_step_amd as M
    for c in range((1 << 32) // CHUNK):
        bits = (np.arange(CHUNK, dtype=np.uint64) + np.uint64(c * CHUNK)).astype(np.uint32)
        x = bits.view(np.float32)
        got = M.bf16_round(torch.from_numpy(x).to(DEV)).cpu().numpy().view(np.uint16)
        ref = O.f32_to_bf16_bits(x)
        nan = np.isnan(x)
        bad = np.nonzero((got != ref) & ~nan)[0]
        assert bad.size == 0, f"chunk {c}: {bad.size} mismatches; first input bits {bits[bad[0]]:#010x}: " \
                              f"got {got[bad[0]]:#06x} expected {ref[bad[0]]:#06x}"
        assert np.all(np.isnan(O.bf16_bits_to_f32(got[nan])))
        if c % 8 == 7:
            say("bf16 exhaustive: chunks done", c + 1)
