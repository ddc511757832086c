"""The streaming probes read every byte once: the XOR of what the read probe
leaves in its sink equals the XOR of every 32-bit word of the buffer, in
order and with the 4 KiB blocks in a scrambled order (XOR does not depend on
the order, and a block read twice or skipped would change it on random
data); the copy probe copies bit for bit."""
from __future__ import annotations

import numpy as np
import pytest
import torch

from paged_kv_cache_207_amd import pkv
from tests.gpu_helpers import require_gpu, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes,scrambled", [(4096, False), (4096 * 16 + 48, False),
                                              (4096 * 37 + 4000, False), (4096 * 64, True),
                                              (4096, True), (1 << 24, True), (1 << 24, False)])
def test_read_probe_covers_every_byte_once(nbytes, scrambled):
    require_gpu()
    say(f"read probe: {nbytes} bytes, scrambled {scrambled}")
    g = torch.Generator().manual_seed(nbytes)
    host = torch.randint(0, 256, (nbytes,), dtype=torch.uint8, generator=g)
    src = host.cuda()
    sink = torch.zeros(pkv.lib().pkv_probe_blocks(nbytes), dtype=torch.float32, device="cuda")
    pkv.probe_stream(src, sink=sink, scrambled=scrambled)
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    want = np.bitwise_xor.reduce(host.numpy().view(np.uint32))
    assert got == want


def test_copy_probe_copies():
    require_gpu()
    src = torch.randint(0, 256, (1 << 20,), dtype=torch.uint8, device="cuda")
    dst = torch.zeros_like(src)
    pkv.probe_stream(src, dst)
    assert torch.equal(src, dst)
