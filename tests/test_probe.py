"""The streaming-read probe (a measurement helper, not a product): it reads the buffer and leaves the sink
untouched unless a workgroup's checksum hits its fixed constant; bad arguments are refused on the host."""
import pytest
import torch

import bit_quantized_matvec_q1_amd.lowbit as L

pytestmark = pytest.mark.gpu


def test_read_probe_runs_and_validates():
    print("case read probe 64 MiB", flush=True)
    a = torch.zeros(64 << 20, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(65536, dtype=torch.int32, device="cuda")
    L.lowbit_read_probe(a, a.numel(), sink)
    torch.cuda.synchronize()
    assert int(sink.abs().sum()) == 0  # the checksum of zero bytes is 0, never the constant
    assert L.lib.lowbit_read_probe(a.data_ptr(), 24, sink.data_ptr(), None) == L.LB_ESHAPE
    assert L.lib.lowbit_read_probe(a.data_ptr() + 8, 64, sink.data_ptr(), None) == L.LB_EALIGN
    with pytest.raises(ValueError, match="buf: needs at least"):
        L.lowbit_read_probe(a[:16], 32, sink)
