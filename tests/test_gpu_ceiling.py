"""The measurement kernels of include/kitty_bench.h on the GPU: the
read-and-write stream kernel's output against a host computation of what
the header specifies (bit-exact), and the read-only kernels' return codes
and untouched sink."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")


def _expected(src_u32, units, rb, wb):
    """Word j of unit u: XOR of the unit's 16-byte words j mod 128 + 128 i,
    each 32-bit lane XORed with j."""
    words = src_u32.reshape(units, rb // 2048, 128, 4)
    acc = np.bitwise_xor.reduce(words, axis=1)  # [units, 128, 4]
    nw = wb // 16
    j = np.arange(nw, dtype=np.uint32)
    return acc[:, j % 128, :] ^ j[None, :, None]


@pytest.mark.parametrize("units,rb,wb", [(300, 16384, 3360), (77, 2048, 2048), (5, 65536, 65536)])
def test_stream_ceiling_writes_what_the_header_specifies(units, rb, wb):
    import torch
    from mixed_precision_bit_kitty_amd import binding as B
    lib = B.load_bench()
    rng = np.random.default_rng([units, rb, wb])
    host_src = rng.integers(0, 2 ** 32, units * rb // 4, dtype=np.uint32)
    src = torch.from_numpy(host_src.view(np.int32)).cuda()
    dst = torch.full((units * wb // 4,), -1, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()
    print(f"stream ceiling: units {units}, read {rb} B, write {wb} B", flush=True)
    rc = lib.kitty_stream_ceiling(src.data_ptr(), dst.data_ptr(), units, rb, wb, stream.cuda_stream)
    assert rc == 0
    torch.cuda.synchronize()
    got = dst.cpu().numpy().view(np.uint32).reshape(units, wb // 16, 4)
    assert np.array_equal(got, _expected(host_src, units, rb, wb))


def test_read_ceiling_runs_and_leaves_the_sink():
    import torch
    from mixed_precision_bit_kitty_amd import binding as B
    lib = B.load_bench()
    nbytes = 64 * 3360 * 16
    src = torch.ones(nbytes, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(1 << 16, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()
    for mode, waves, depth in [(0, 8, 4), (0, 32, 8), (1, 12, 3), (1, 8, 4), (2, 12, 2), (2, 4, 1)]:
        print(f"read ceiling: mode {mode}, {waves} waves/CU, depth {depth}", flush=True)
        rc = lib.kitty_read_ceiling(src.data_ptr(), nbytes, mode, waves, depth, sink.data_ptr(), sink.numel(),
                                    stream.cuda_stream)
        assert rc == 0
    torch.cuda.synchronize()
    assert int(sink.abs().sum()) == 0
