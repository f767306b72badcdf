"""The plain streaming read that the KV-read rates are compared with.

It computes nothing of the method; these tests check only that it runs on
every size the sweep gives it, leaves its sink alone for data whose XOR is
not the trigger constant, and rejects sizes it cannot stream.
"""
import pytest
import torch

import speculative_decode_verify_amd as va


@pytest.mark.gpu
@pytest.mark.parametrize("nbytes", [16, 4096, 1 << 20, (1 << 24) + 48])
def test_read_probe_runs(nbytes):
    src = torch.ones(nbytes, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    va.va_read_probe(src, nbytes, sink)
    torch.cuda.synchronize()
    assert int(sink.item()) == 0


@pytest.mark.gpu
def test_read_probe_rejects_bad_sizes():
    src = torch.ones(1024, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    with pytest.raises(RuntimeError):
        va.va_read_probe(src, 1000, sink)  # not a multiple of 16
    with pytest.raises(RuntimeError):
        va.va_read_probe(src[1:], 512, sink)  # misaligned
    with pytest.raises(ValueError):
        va.va_read_probe(src, 2048, sink)  # beyond the tensor
    va.va_read_probe(src, 0, sink)
    torch.cuda.synchronize()
    assert int(sink.item()) == 0
