"""The plain read kernel used for the read-bandwidth ceiling reads every byte:
the XOR of its per-workgroup results equals the XOR of the buffer's words."""

import numpy as np
import pytest
import torch

from attention_int8_quantized_amd import ops
from gpu_util import note

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("n_words", [0, 4, 4004, 1 << 22, (1 << 22) + 36])
def test_stream_read_covers_every_word(n_words):
    note(f"stream read {n_words} words")
    rng = np.random.default_rng(n_words + 3)
    x = rng.integers(0, 2**32, size=n_words, dtype=np.uint32)
    t = torch.from_numpy(x.view(np.int32)).cuda()
    sink = ops.stream_read(t)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    assert got == (np.bitwise_xor.reduce(x) if n_words else 0)
