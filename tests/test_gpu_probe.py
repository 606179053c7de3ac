"""GPU checks of the measurement probes (include/moe_probe.h): the stream
kernels move exactly the bytes asked for, and the MFMA loop runs and leaves
its sink alone on ordinary data."""
import pytest
import torch

from mixture_experts_layer_topkrouter_amd import moe


@pytest.mark.gpu
@pytest.mark.parametrize("nbytes", [16, 16 * 1023, (1 << 20) + 48])
@pytest.mark.parametrize("nt", [False, True])
def test_stream_probe_copy_and_write_exact(nbytes, nt):
    g = torch.Generator(device="cuda").manual_seed(nbytes)
    src = torch.randint(0, 256, (nbytes + 64,), dtype=torch.uint8, device="cuda", generator=g)
    dst = torch.zeros(nbytes + 64, dtype=torch.uint8, device="cuda")
    moe.stream_probe("copy", src, dst, nbytes, nontemporal=nt)
    torch.cuda.synchronize()
    assert torch.equal(dst[:nbytes], src[:nbytes])
    assert torch.all(dst[nbytes:] == 0)  # nothing past the size
    out = torch.zeros(nbytes + 64, dtype=torch.uint8, device="cuda")
    moe.stream_probe("write", src, out, nbytes, nontemporal=nt)
    torch.cuda.synchronize()
    assert torch.all(out[nbytes:] == 0)
    words = out[:nbytes].view(torch.int32).view(-1, 4)
    assert torch.all(words[:, :3] == 0x3f803f80)  # the pattern; its last word is the writing
    j = torch.arange(words.shape[0], dtype=torch.int32, device="cuda")  # thread's first 16-B index:
    assert torch.equal(words[:, 3], (j // 1024) * 1024 + (j % 1024) % 256)  # 256 threads x 4 per block
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    moe.stream_probe("read", src, dst, nbytes, nontemporal=nt, sink=sink)
    torch.cuda.synchronize()
    assert torch.all(sink == 0)


@pytest.mark.gpu
def test_mfma_probe_runs_and_leaves_sink():
    blocks, iters = 8, 64
    g = torch.Generator(device="cuda").manual_seed(3)
    ops = torch.randn(blocks * 16384, device="cuda", generator=g).to(torch.bfloat16)
    sink = torch.zeros(blocks * 4, dtype=torch.float32, device="cuda")
    moe.mfma_probe(blocks, iters, ops, sink=sink)
    torch.cuda.synchronize()
    assert torch.all(sink == 0)
    with pytest.raises(ValueError):
        moe.mfma_probe(blocks + 1, iters, ops)
