"""The library's read-stream probe (a measurement aid for the achievable HBM
read rate) reads every 16-byte word of its buffer exactly once: each sink word
must equal the XOR of the words its thread's grid-stride walk covers."""
import numpy as np
import pytest

from ragged_paged_attention_splitfuse_amd import binding

pytestmark = pytest.mark.gpu


def _expected_sink(words_u32, cus, threads=256):
    per16 = (words_u32[0::4] ^ words_u32[1::4] ^ words_u32[2::4] ^ words_u32[3::4])
    stride = cus * threads
    pad = (-per16.size) % stride
    grid = np.concatenate([per16, np.zeros(pad, np.uint32)]).reshape(-1, stride)
    return np.bitwise_xor.reduce(grid, axis=0)


@pytest.mark.parametrize("n_words16", [1, 4099, 256 * 256 * 8 * 3 + 77])
def test_read_stream_probe_reads_each_word_once(n_words16):
    import torch
    dev = torch.device("cuda:0")
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    rng = np.random.default_rng(n_words16)
    host = rng.integers(0, 2 ** 32, size=4 * n_words16, dtype=np.uint64).astype(np.uint32)
    buf = torch.from_numpy(host.view(np.uint8).copy()).to(dev)
    sink = torch.zeros(1 << 20, dtype=torch.uint8, device=dev)
    print(f"read-stream probe: {n_words16} words of 16 B, {cus} CUs", flush=True)
    binding.fg_probe_read_stream(buf, sink)
    torch.cuda.synchronize()
    got = sink[: cus * 256 * 4].cpu().numpy().view(np.uint32)
    np.testing.assert_array_equal(got, _expected_sink(host, cus))


def test_read_stream_probe_rejects_a_short_sink():
    import torch
    dev = torch.device("cuda:0")
    buf = torch.zeros(4096, dtype=torch.uint8, device=dev)
    sink = torch.zeros(1024, dtype=torch.uint8, device=dev)
    with pytest.raises(binding.FgError) as e:
        binding.fg_probe_read_stream(buf, sink)
    assert e.value.status == binding.FG_E_WORKSPACE


def test_mfma_loop_probe_computes_exactly_and_reports_a_clock():
    import torch
    dev = torch.device("cuda:0")
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    iters = 64
    sink = torch.full((cus * 2 * 256,), -1.0, dtype=torch.float32, device=dev)
    clocks = torch.zeros(cus * 2 * 2, dtype=torch.int64, device=dev)
    binding.fg_probe_mfma_loop(iters, sink, clocks)
    torch.cuda.synchronize()
    # all-ones operands: every accumulator element is 16 * 8 * iters
    assert bool(torch.all(sink == 8192.0 * iters))
    c = clocks.view(-1, 2).cpu().numpy().astype(np.float64)
    assert (c > 0).all()
    ghz = c[:, 0] / (c[:, 1] / 100e6) / 1e9
    assert 0.5 < float(np.median(ghz)) < 3.0


def test_mfma_loop_probe_rejects_short_buffers():
    import torch
    dev = torch.device("cuda:0")
    sink = torch.zeros(16, dtype=torch.float32, device=dev)
    clocks = torch.zeros(16, dtype=torch.int64, device=dev)
    with pytest.raises(binding.FgError) as e:
        binding.fg_probe_mfma_loop(4, sink, clocks)
    assert e.value.status == binding.FG_E_WORKSPACE
