"""The measuring aids (not steps of the layer) run and fold their reads
deterministically: the streaming-read probe and the L2 load probe in each of
their modes give the same per-workgroup / per-wave fold on repeated runs."""
import pytest
import torch

import token_adaptive_expert_amd as ace

pytestmark = pytest.mark.gpu


def test_hbm_read_probe_repeatable(dev):
    g = torch.Generator(device="cpu").manual_seed(3)
    buf = torch.randint(-2 ** 31, 2 ** 31 - 1, (1 << 20,), dtype=torch.int32, generator=g).to(dev)
    sink = torch.zeros(64, dtype=torch.int32, device=dev)
    ace.moe_hbm_read_probe(buf, sink, 64)
    first = sink.clone()
    ace.moe_hbm_read_probe(buf, sink, 64)
    torch.cuda.synchronize()
    assert torch.equal(first, sink)
    # the folds of all workgroups together are the XOR of every word read
    import numpy as np
    host = buf.cpu().numpy().view(np.uint32)
    folds = first.cpu().numpy().view(np.uint32)
    assert int(np.bitwise_xor.reduce(folds)) == int(np.bitwise_xor.reduce(host))


@pytest.mark.parametrize("loads,mfma,stride", [(6, 0, 0), (6, 4, 0), (6, 4, 1), (8, 8, 0), (8, 0, 1)])
def test_l2_load_probe_repeatable(dev, loads, mfma, stride):
    g = torch.Generator(device="cpu").manual_seed(5)
    buf = torch.randint(0, 255, (2 << 20,), dtype=torch.uint8, generator=g).to(dev)
    wg = 16
    sink = torch.zeros(wg * 4, dtype=torch.int32, device=dev)
    ace.moe_l2_load_probe(buf, sink, wg, 7, loads, mfma, stride)
    first = sink.clone()
    sink.zero_()
    ace.moe_l2_load_probe(buf, sink, wg, 7, loads, mfma, stride)
    torch.cuda.synchronize()
    assert torch.equal(first, sink)
    assert int((first != 0).sum()) > 0
