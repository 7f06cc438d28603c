"""GPU check of the HBM streaming-read probe through the C ABI: every 16-byte
chunk is read exactly once, so the XOR of the buffer's 32-bit words it
returns equals numpy's, for any grid size and a buffer that is not a
multiple of the grid's stride."""
import numpy as np
import pytest
import torch

import paged_kv_cache_decode_amd as pda

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes", [16, 4096 + 48, (1 << 20) + 16 * 37])
@pytest.mark.parametrize("workgroups", [1, 3, 2048])
def test_probe_reads_every_chunk_once(nbytes, workgroups):
    rng = np.random.default_rng(nbytes + workgroups)
    words = rng.integers(-2**31, 2**31, size=nbytes // 4, dtype=np.int64).astype(np.int32)
    src = torch.from_numpy(words).cuda()
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    pda.pda_read_probe(src, sink, workgroups)
    torch.cuda.synchronize()
    want = np.bitwise_xor.reduce(words.view(np.uint32))
    assert int(sink.cpu().numpy().view(np.uint32)[0]) == int(want)


def test_probe_rejects_bad_sizes():
    src = torch.zeros(5, dtype=torch.int32, device="cuda")  # 20 bytes
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    with pytest.raises(pda.PdaError):
        pda.pda_read_probe(src, sink, 4)
    with pytest.raises(pda.PdaError):
        pda.pda_read_probe(src[:4], sink, 0)
