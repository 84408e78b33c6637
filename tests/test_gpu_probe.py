"""The read probes (measurement helpers) read what their sweep assigns: 256 workgroups of 1,024
threads, thread t of the grid reading 16-byte chunks t, t + 262,144, ...; each workgroup's
first wave XORs its lanes' words into the workgroup's sink word (the other waves' loads are
timed, not checked).  Plain and non-temporal forms, at sizes that do and do not fill whole
sweeps."""
import numpy as np
import pytest
import torch

from kivi_testlib import gpu_or_skip

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes", [16, 4096 + 48, (1 << 20) * 5 + 16 * 37, 256 * 1024 * 16 * 4 + 16])
@pytest.mark.parametrize("streaming", [False, True])
def test_probe_sink_words(nbytes, streaming):
    dev = gpu_or_skip()
    from kv_cache_bit_quantize_amd import kivi
    rng = np.random.default_rng(nbytes)
    words = rng.integers(0, 2 ** 32, nbytes // 4, dtype=np.uint64).astype(np.uint32)
    buf = torch.from_numpy(words.view(np.int32)).to(dev)
    sink = kivi.kivi_read_probe(buf, streaming=streaming)
    torch.cuda.synchronize()
    chunks = np.bitwise_xor.reduce(words.reshape(-1, 4), axis=1)      # one word per 16-byte chunk
    idx = np.arange(chunks.size)
    thread = idx % (256 * 1024)
    want = np.zeros(256, np.uint32)
    first_wave = thread % 1024 < 64
    np.bitwise_xor.at(want, thread[first_wave] // 1024, chunks[first_wave])
    assert np.array_equal(sink.cpu().numpy().view(np.uint32), want)
