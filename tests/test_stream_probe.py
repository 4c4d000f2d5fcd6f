"""The bandwidth probe that bench.py reports the streaming ceiling with: it
must really read both sources and, in its writing mode, write every byte of
the destination (otherwise the ceiling it measures would be too high)."""
import pytest
import torch

import gated_linear_attention_forward_amd as gla


@pytest.mark.gpu
@pytest.mark.parametrize("nbytes", [16, 64 * 1024, 5 * 64 * 1024 + 48, 3 << 20])
def test_probe_write_mode_writes_the_xor(nbytes):
    dev = torch.device("cuda:0")
    gen = torch.Generator(device="cpu").manual_seed(nbytes)
    a = torch.randint(0, 256, (nbytes,), generator=gen, dtype=torch.uint8)
    b = torch.randint(0, 256, (nbytes,), generator=gen, dtype=torch.uint8)
    ad, bd = a.to(dev), b.to(dev)
    dd = torch.zeros(nbytes + 256, dtype=torch.uint8, device=dev)
    print(f"stream probe mode 1, {nbytes} bytes", flush=True)
    gla.gla_stream_probe(ad, bd, dd[:nbytes], 1)
    torch.cuda.synchronize()
    d = dd.cpu()
    assert torch.equal(d[:nbytes], a ^ b)
    assert not d[nbytes:].any()  # nothing past the end


@pytest.mark.gpu
def test_probe_read_mode_leaves_the_destination():
    dev = torch.device("cuda:0")
    nbytes = 1 << 20
    a = torch.zeros(nbytes, dtype=torch.uint8, device=dev)
    b = torch.ones(nbytes, dtype=torch.uint8, device=dev)
    d = torch.full((nbytes,), 7, dtype=torch.uint8, device=dev)
    print("stream probe mode 0", flush=True)
    gla.gla_stream_probe(a, b, d, 0)
    torch.cuda.synchronize()
    assert (d == 7).all()


@pytest.mark.gpu
@pytest.mark.parametrize("nsrc,ndst", [(1, 1), (2, 2), (3, 2), (3, 1)])
@pytest.mark.parametrize("nbytes", [16, 5 * 16 * 1024 + 48])
def test_probe_mix_writes_the_xor_to_every_destination(nsrc, ndst, nbytes):
    dev = torch.device("cuda:0")
    gen = torch.Generator(device="cpu").manual_seed(nbytes + 10 * nsrc + ndst)
    srcs = [torch.randint(0, 256, (nbytes,), generator=gen, dtype=torch.uint8)
            for _ in range(nsrc)]
    want = srcs[0].clone()
    for t in srcs[1:]:
        want ^= t
    dbufs = [torch.zeros(nbytes + 256, dtype=torch.uint8, device=dev) for _ in range(ndst)]
    print(f"stream probe mix {nsrc} reads {ndst} writes, {nbytes} bytes", flush=True)
    gla.gla_stream_probe_mix([t.to(dev) for t in srcs], [d[:nbytes] for d in dbufs])
    torch.cuda.synchronize()
    for d in dbufs:
        d = d.cpu()
        assert torch.equal(d[:nbytes], want)
        assert not d[nbytes:].any()  # nothing past the end
