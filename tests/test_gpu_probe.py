"""GPU check of the read-only HBM probe (qbl_hbm_probe): the XOR of the
workgroups' sink words equals the XOR of the whole buffer, so every 16-byte
word was read exactly once (a word read twice would cancel, one skipped would
be missing), for buffers that end mid-sweep and for small grids."""
import numpy as np
import pytest

from tests.gpu_harness import log

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes,sink_words", [(16, 1), (64 << 20, 4096), ((64 << 20) + 16 * 12345, 2048),
                                               (16 * 1000003, 7)])
def test_probe_reads_every_word_once(nbytes, sink_words):
    import torch
    import quantized_base_linear_amd as q
    log(f"hbm probe: {nbytes} bytes, {sink_words} sink words")
    rng = np.random.default_rng(nbytes ^ sink_words)
    host = rng.integers(0, 2**32, size=nbytes // 4, dtype=np.uint32)
    buf = torch.from_numpy(host.view(np.int32)).cuda()
    sink = torch.zeros(sink_words, dtype=torch.int32, device="cuda")
    wg = q.qbl_hbm_probe(buf, sink)
    torch.cuda.synchronize()
    assert 1 <= wg <= sink_words
    got = np.bitwise_xor.reduce(sink[:wg].cpu().numpy().view(np.uint32))
    assert got == np.bitwise_xor.reduce(host)
