"""The streaming-read probe (a measurement aid beside the decode path): it
reads the whole buffer and leaves the sink untouched unless a thread's fold
of its words hits the sentinel, which a constant buffer of ones never does."""

import pytest
import torch

pytestmark = pytest.mark.gpu

kvd = pytest.importorskip("kv_cache_decode_02_amd")


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@pytest.mark.parametrize("nbytes", [16, 4096 + 16, 3 << 20, (64 << 20) + 48])
def test_stream_read_runs_and_writes_nothing(nbytes):
    src = torch.ones(nbytes, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(kvd.stream_read_sink_bytes(), dtype=torch.uint8, device="cuda")
    kvd.stream_read(src, sink)
    torch.cuda.synchronize()
    assert torch.count_nonzero(sink).item() == 0


def test_stream_read_rejects_bad_sizes():
    src = torch.ones(24, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(kvd.stream_read_sink_bytes(), dtype=torch.uint8, device="cuda")
    with pytest.raises(kvd.KvdError):
        kvd.stream_read(src, sink)                  # not a multiple of 16
    with pytest.raises(kvd.KvdError):
        kvd.stream_read(src[:16], sink[:16])        # sink too small
