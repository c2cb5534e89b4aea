"""The measurement probes through the C ABI: the device bandwidth probe
reads (XOR of every 32-bit word, exact) and copies whole buffers, ragged
sizes and every grid shape included; the shared-memory probe returns the
XOR of exactly the words its lanes were to read, for conflict-free and
conflicting strides."""
import numpy as np
import pytest

from gpu_helpers import log
from roofline_driven_optimisation_amd import binding

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch():
    t = pytest.importorskip("torch")
    if not t.cuda.is_available():
        pytest.skip("no GPU")
    binding.library()
    return t


def xor_all(words: np.ndarray) -> int:
    return int(np.bitwise_xor.reduce(words.astype(np.uint32))) if words.size else 0


# bytes: empty, one chunk, less than a grid step, ragged tails, the decode
# GEMMs' weight size (4096 x 11008 bf16)
SIZES = [0, 16, 4096, (1 << 20) + 48, 3 * 4096 * 256 * 16 + 16 * 999, 4096 * 11008 * 2]


@pytest.mark.parametrize("nbytes", SIZES)
@pytest.mark.parametrize("blocks", [1, 7, 2048])
def test_stream_read_xor(torch, nbytes, blocks):
    log("  stream read %d bytes, %d workgroups" % (nbytes, blocks))
    rng = np.random.default_rng(nbytes + blocks)
    host = rng.integers(0, 2 ** 32, nbytes // 4, dtype=np.uint64).astype(np.uint32)
    src = torch.from_numpy(host.view(np.int32)).cuda()
    out = torch.full((blocks + 3,), -1, dtype=torch.int32, device="cuda")
    binding.probe_stream(src, out=out, blocks=blocks)
    assert binding.last_kernel() == "stream_probe_read"
    got = out.cpu().numpy().view(np.uint32)
    assert xor_all(got[:blocks]) == xor_all(host)
    assert (got[blocks:] == 0xFFFFFFFF).all()  # nothing past `blocks` words is written


@pytest.mark.parametrize("nbytes", SIZES[1:])
@pytest.mark.parametrize("blocks", [1, 5, 1024])
def test_stream_copy(torch, nbytes, blocks):
    log("  stream copy %d bytes, %d workgroups" % (nbytes, blocks))
    rng = np.random.default_rng(nbytes * 3 + blocks)
    host = rng.integers(-2 ** 31, 2 ** 31, nbytes // 4, dtype=np.int64).astype(np.int32)
    src = torch.from_numpy(host).cuda()
    dst = torch.full((nbytes // 4 + 8,), 7, dtype=torch.int32, device="cuda")
    binding.probe_stream(src, dst=dst, blocks=blocks)
    assert binding.last_kernel() == "stream_probe_copy"
    d = dst.cpu().numpy()
    assert np.array_equal(d[:nbytes // 4], host)
    assert (d[nbytes // 4:] == 7).all()  # the guard words past the copy are untouched


def lds_expected(stride: int, steps: int) -> int:
    """XOR of table word i = i * 2654435761 (mod 2^32) over the words
    l * stride + 17 w + j of every lane l < 64, wave w < 4, step j < steps."""
    lane = np.arange(64, dtype=np.uint64)[:, None, None]
    wave = np.arange(4, dtype=np.uint64)[None, :, None]
    j = np.arange(steps, dtype=np.uint64)[None, None, :]
    idx = lane * stride + 17 * wave + j
    vals = (idx * 2654435761) % (2 ** 32)
    return xor_all(vals.ravel())


@pytest.mark.parametrize("stride,steps", [(1, 0), (1, 5), (1, 1000), (2, 40), (33, 64),
                                          (64, 4096), (255, 123)])
def test_lds_probe_reads_the_right_words(torch, stride, steps):
    log("  lds probe stride %d, %d steps" % (stride, steps))
    blocks = 3
    out = torch.full((blocks + 1,), -1, dtype=torch.int32, device="cuda")
    binding.probe_lds(stride, steps, out, blocks=blocks)
    assert binding.last_kernel() == "lds_probe"
    got = out.cpu().numpy().view(np.uint32)
    want = lds_expected(stride, steps)
    assert all(int(g) == want for g in got[:blocks]), (got, want)
    assert got[blocks] == 0xFFFFFFFF


def test_probe_argument_errors(torch):
    src = torch.zeros(64, dtype=torch.int32, device="cuda")
    out = torch.zeros(4, dtype=torch.int32, device="cuda")
    with pytest.raises(binding.GemmError):
        binding.probe_stream(src[1:61], out=out, blocks=4)  # misaligned start
    with pytest.raises(ValueError):
        binding.probe_stream(src, out=out, blocks=8)  # out shorter than the grid
    with pytest.raises(binding.GemmError):
        binding.probe_lds(300, 8, out, blocks=4)  # lanes past the table
