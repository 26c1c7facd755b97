"""The HBM read probe (the measured read-stream reference of bench.py) reads
every 32-bit word of its buffer: with all words zero but one equal to the fixed
word 0x9e3779b9, the XOR of the buffer is that word and the sink is written;
with that word moved to a place the probe would skip, it would not be."""
import numpy as np
import pytest
import torch

import embedding_table_gather_amd as etg
from tests.gpu_util import note

pytestmark = pytest.mark.gpu

MAGIC = np.uint32(0x9E3779B9).view(np.int32)


@pytest.mark.parametrize("nbytes", [16, 1008, 1024, 65536 + 48, 64 << 20])
@pytest.mark.parametrize("where", ["first", "middle", "last"])
def test_probe_reads_every_word(nbytes, where):
    n = nbytes // 4
    pos = {"first": 0, "middle": n // 2, "last": n - 1}[where]
    x = torch.zeros(n, dtype=torch.int32, device="cuda")
    x[pos] = int(MAGIC)
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    note(f"read probe {nbytes} B, magic word at {where}")
    etg.hbm_read_probe(x, sink)
    torch.cuda.synchronize()
    assert int(sink.item()) == int(MAGIC)


def test_probe_writes_nothing_for_other_data():
    x = torch.arange(1 << 20, dtype=torch.int32, device="cuda")
    sink = torch.full((1,), 7, dtype=torch.int32, device="cuda")
    note("read probe, no magic word")
    etg.hbm_read_probe(x, sink)
    torch.cuda.synchronize()
    assert int(sink.item()) == 7


@pytest.mark.parametrize("nbytes", [16, 1008, 1024, 65536 + 48, 64 << 20])
def test_write_probe_writes_every_word_and_nothing_else(nbytes):
    # the buffer sits between two guard regions that must stay untouched
    n = nbytes // 4
    buf = torch.full((n + 2048,), -1, dtype=torch.int32, device="cuda")
    x = buf[1024:1024 + n]
    note(f"write probe {nbytes} B")
    etg.hbm_write_probe(x, 0x12345678)
    torch.cuda.synchronize()
    assert torch.all(x == 0x12345678)
    assert torch.all(buf[:1024] == -1) and torch.all(buf[1024 + n:] == -1)
