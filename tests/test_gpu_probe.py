"""The streaming-read probe (a measurement aid beside the decode step): it
reads every word of the buffer exactly once (the XOR of its per-block
results equals the XOR of the buffer's words, ragged ends included) and
rejects bad arguments before launching."""
import numpy as np
import pytest
import torch

import moe_decode_layer_seam_amd as mdl

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes", [16, 4096 * 16 + 48, (64 << 20) + 16 * 777])
def test_read_probe_reads_every_word_once(nbytes):
    rng = np.random.default_rng(nbytes)
    host = rng.integers(0, 2**32, size=nbytes // 4, dtype=np.uint32)
    buf = torch.from_numpy(host.view(np.uint8)).cuda()
    sink = mdl.read_probe(buf)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    assert got == np.bitwise_xor.reduce(host)
    # a word counted twice or skipped changes the XOR: flip one word's bits
    host2 = host.copy()
    host2[len(host2) // 2] ^= np.uint32(0x5A5A5A5A)
    sink2 = mdl.read_probe(torch.from_numpy(host2.view(np.uint8)).cuda())
    torch.cuda.synchronize()
    assert np.bitwise_xor.reduce(sink2.cpu().numpy().view(np.uint32)) == got ^ np.uint32(0x5A5A5A5A)


def test_read_probe_rejects_bad_arguments():
    L = mdl.lib()
    buf = torch.zeros(4096, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(mdl.PROBE_BLOCKS, dtype=torch.int32, device="cuda")
    s = torch.cuda.current_stream().cuda_stream
    assert L.moe_decode_read_probe(buf.data_ptr(), 4000 + 8, sink.data_ptr(), s) == mdl.EINVAL
    assert L.moe_decode_read_probe(buf.data_ptr() + 8, 1024, sink.data_ptr(), s) == mdl.EINVAL
    assert L.moe_decode_read_probe(buf.data_ptr(), 0, sink.data_ptr(), s) == mdl.EINVAL
    assert L.moe_decode_read_probe(buf.data_ptr(), 1024, None, s) == mdl.EINVAL
    assert L.moe_decode_read_probe(buf.data_ptr(), 1024, sink.data_ptr() + 2, s) == mdl.EINVAL
    torch.cuda.synchronize()
