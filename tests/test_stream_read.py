"""The read-ceiling helper (verify_attn_stream_read) reads every 16-byte word
exactly once: the XOR it folds into the sink equals the XOR of all the
buffer's 32-bit words, which a skipped or doubled word would change."""
import numpy as np
import pytest
import torch

import speculative_tree_verify_mla_amd as va
from test_parity import DEV, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes,words", [(16, 1), (4096, 1), ((1 << 20) + 48, 4096),
                                          (37 * (1 << 20) + 16 * 7, 4096), (37 * (1 << 20) + 16 * 7, 3)])
def test_every_word_read_once(nbytes, words):
    rng = np.random.default_rng(nbytes)
    host = rng.integers(0, 2**32, size=nbytes // 4, dtype=np.uint32)
    buf = torch.from_numpy(host.view(np.int32)).to(DEV)
    sink = torch.zeros(words, dtype=torch.int32, device=DEV)
    va.verify_attn_stream_read(buf, sink)
    torch.cuda.synchronize()
    want = int(np.bitwise_xor.reduce(host))
    got = int(np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32)))
    say(f"  stream read {nbytes} B: xor {got:#010x} (expected {want:#010x})")
    assert got == want
