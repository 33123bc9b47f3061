"""The streaming-read probe (spec_verify_read_probe) that bench.py uses for
the practical read ceiling: it must read every 8 KB span it is given (a
planted word in the last span reaches the sink) and write nothing otherwise."""
import numpy as np
import pytest

from tests.gpu_helpers import log

pytestmark = pytest.mark.gpu

MAGIC = 0x9E3779B9


@pytest.mark.parametrize("nontemporal", [True, False])
@pytest.mark.parametrize("spans", [1, 3, 1000])
def test_probe_reads_every_span(nontemporal, spans):
    import torch
    from rejection_sampling_verify_08_amd.binding import read_probe
    log(f"[probe] spans={spans} nontemporal={nontemporal}")
    dev = torch.device("cuda", 0)
    words = np.zeros(spans * 2048, dtype=np.uint32)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    buf = torch.from_numpy(words.view(np.int32)).to(dev)
    read_probe(buf, sink, nontemporal=nontemporal)
    torch.cuda.synchronize()
    assert int(sink.item()) == 0
    # one word in the last 8 KB span: only that wave's fold equals MAGIC
    words[-2048 + 777] = MAGIC
    buf = torch.from_numpy(words.view(np.int32)).to(dev)
    read_probe(buf, sink, nontemporal=nontemporal)
    torch.cuda.synchronize()
    assert int(sink.item()) & 0xFFFFFFFF == MAGIC


def test_probe_timing_events():
    import torch
    from rejection_sampling_verify_08_amd.binding import read_probe
    dev = torch.device("cuda", 0)
    buf = torch.full((64 << 20,), 7, dtype=torch.uint8, device=dev)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    for e in ev:
        e.record()
    read_probe(buf, sink, events=ev)
    torch.cuda.synchronize()
    ms = ev[0].elapsed_time(ev[1])
    log(f"[probe] 64 MiB in {ms * 1e3:.1f} us")
    assert 0.0 < ms < 50.0
    assert int(sink.item()) == 0
