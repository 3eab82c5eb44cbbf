"""The measurement probes through the C ABI: they run, read what they are
given and write nothing (their sink is stored only for a value no sum of
these loads takes), and the paged-read probe takes the attention call's
grid over a real pool and block table.  Their timings are the bench's
ceilings, not results to compare."""
import pytest
import torch

import paged_kv_transformer_amd as pkv
import synth
from gpu_util import dev

pytestmark = pytest.mark.gpu


def test_probe_read_reads_and_writes_nothing():
    buf = torch.arange(1 << 18, dtype=torch.int32, device="cuda")   # 1 MiB
    sink = torch.full((1,), 7.0, dtype=torch.float32, device="cuda")
    for wg in (1, 64, 1024):
        pkv.probe_read(buf, sink, workgroups=wg)
    pkv.probe_read(buf, sink, workgroups=16, nbytes=4096)
    torch.cuda.synchronize()
    assert float(sink.item()) == 7.0


def test_probe_paged_read_over_an_attention_workload():
    wl = synth.attention_workload(1002, batch=4, pool_bytes=16 << 20)
    pool_t = dev(wl["pool"])
    pool = pkv.kv_pool_create(pool_t, wl["shape"].kv_heads)
    sink = torch.full((1,), 3.0, dtype=torch.float32, device="cuda")
    pkv.probe_paged_read(pool, wl["shape"].heads, dev(wl["block_table"]), dev(wl["lens"]), sink)
    torch.cuda.synchronize()
    assert float(sink.item()) == 3.0


def test_probe_empty_launches():
    pkv.probe_empty(0)
    pkv.probe_empty(4, workgroups=256)
    torch.cuda.synchronize()
