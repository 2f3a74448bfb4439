"""GPU: pa_decode_read_probe, the read-rate measurement tool behind
bench.py's read ceilings.  It must read exactly the chunks it is given: the
XOR of its sink words (one per probe wave) is the XOR of every 32-bit word
of them, checked against numpy for contiguous and gathered chunks, every
chunk size, chunk counts below, at and far above the wave count, and
uneven splits over the waves."""
import numpy as np
import pytest
import torch

from paged_kv_decode_amd import binding as B

pytestmark = pytest.mark.gpu


def _xor_words(t: torch.Tensor) -> int:
    return int(np.bitwise_xor.reduce(t.cpu().numpy().view(np.uint32).ravel(), initial=0))


def _sink(fill=0):
    """A sink array, pre-filled so that a word the probe fails to write shows."""
    return torch.full((B.PA_DECODE_PROBE_WAVES,), fill, dtype=torch.int32, device="cuda")


@pytest.mark.parametrize("chunk", [2048, 3072, 4096, 8192])
@pytest.mark.parametrize("n", [1, 3, 4, 5, 1023, 1024, 1027, 5000])
def test_contiguous_reads_every_word(chunk, n):
    gen = torch.Generator().manual_seed(chunk + n)
    data = torch.randint(-2**31, 2**31 - 1, (n * chunk // 4,), generator=gen, dtype=torch.int32)
    d = data.cuda()
    sink = _sink(0x5A5A5A5A)
    B.pa_decode_read_probe(d.data_ptr(), 0, n, chunk, sink.data_ptr())
    torch.cuda.synchronize()
    assert _xor_words(sink) == _xor_words(data)
    # Waves without chunks store 0 (n < waves: waves w with no chunk in
    # [w n / W, (w + 1) n / W)).
    W = B.PA_DECODE_PROBE_WAVES
    empty = [w for w in range(W) if (w * n) // W == ((w + 1) * n) // W]
    if empty:
        assert (sink.cpu()[empty] == 0).all()


@pytest.mark.parametrize("chunk", [2048, 8192])
def test_gathered_chunks_in_any_order_with_repeats(chunk):
    gen = torch.Generator().manual_seed(7 + chunk)
    pool_chunks = 300
    pool = torch.randint(-2**31, 2**31 - 1, (pool_chunks * chunk // 4,), generator=gen,
                         dtype=torch.int32)
    d = pool.cuda()
    idx = torch.randint(0, pool_chunks, (1001,), generator=gen)   # repeats included
    addrs = (d.data_ptr() + idx * chunk).to(torch.int64).cuda()
    sink = _sink(0x5A5A5A5A)
    B.pa_decode_read_probe(0, addrs.data_ptr(), idx.numel(), chunk, sink.data_ptr())
    torch.cuda.synchronize()
    words = pool.view(pool_chunks, chunk // 4)[idx]
    assert _xor_words(sink) == _xor_words(words)


def test_probe_is_capturable_and_replays():
    chunk, n = 4096, 64
    gen = torch.Generator().manual_seed(11)
    data = torch.randint(-2**31, 2**31 - 1, (n * chunk // 4,), generator=gen, dtype=torch.int32)
    d = data.cuda()
    sink = _sink()
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        B.pa_decode_read_probe(d.data_ptr(), 0, n, chunk, sink.data_ptr(), s.cuda_stream)
        s.synchronize()
        with torch.cuda.graph(g, stream=s):
            B.pa_decode_read_probe(d.data_ptr(), 0, n, chunk, sink.data_ptr(), s.cuda_stream)
    torch.cuda.synchronize()
    x = _xor_words(data)
    # one eager run and the capture (not executed)
    assert _xor_words(sink) == x
    for rep in range(3):
        sink.fill_(0x5A5A5A5A)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert _xor_words(sink) == x, rep
