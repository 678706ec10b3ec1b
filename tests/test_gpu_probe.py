"""The bandwidth probes on the GPU: the copy probe moves every byte (the read and copy
ceilings the measurement reports come from these two launches), and the read probe leaves
its sink alone unless the data fold to its marker word."""

import pytest
import torch

from gpu_harness import log
from rejection_sampling_verify_specdec_amd import binding

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes", [16, 4096, 32768 + 48, (64 << 20) + 16 * 7])
def test_copy_probe_moves_every_byte(nbytes):
    d = torch.device("cuda:0")
    log(f"[probe] copy of {nbytes} bytes")
    g = torch.Generator(device="cpu").manual_seed(nbytes)
    src = torch.randint(0, 256, (nbytes,), dtype=torch.uint8, generator=g).to(d)
    dst = torch.zeros(nbytes + 64, dtype=torch.uint8, device=d)
    binding.specdec_probe_copy(dst, src)
    torch.cuda.synchronize()
    assert torch.equal(dst[:nbytes], src)
    assert int(dst[nbytes:].sum()) == 0                 # nothing past the end


def test_read_probe_runs_and_keeps_its_sink():
    d = torch.device("cuda:0")
    src = torch.zeros(1 << 24, dtype=torch.uint8, device=d)     # folds to 0, not the marker
    sink = torch.full((1,), 7, dtype=torch.int32, device=d)
    binding.specdec_probe_read(src, sink)
    torch.cuda.synchronize()
    assert int(sink.item()) == 7
