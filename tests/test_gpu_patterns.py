"""The access-pattern streams (measurement-only ceilings) move the bytes they claim to move.

Each stream's output is a plain function of its inputs (a copy, an XOR of two
halves or of two buffers, a token-major to head-major transpose), so the
checks are exact; ragged row counts and widths exercise the tails of each
launch shape.
"""
import pytest
import torch

import video_diffusion_transformer_dit_amd as dit

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")
    dit.load_library()
    torch.cuda.synchronize()
    yield
    torch.cuda.synchronize()


def words(rows, row_bytes, seed):
    g = torch.Generator(device=DEV).manual_seed(seed)
    return torch.randint(-2 ** 31, 2 ** 31 - 1, (rows, row_bytes // 4), generator=g, dtype=torch.int32, device=DEV)


SHAPES = [(1, 16), (7, 48), (33, 8192), (5, 16384), (3, 4112)]


@pytest.mark.parametrize("rows,row_bytes", SHAPES)
def test_split_rows_and_two_in(rows, row_bytes):
    a = words(rows, 2 * row_bytes, 1)
    out = torch.empty((rows, row_bytes // 4), dtype=torch.int32, device=DEV)
    dit.dit_stream_pattern(dit.DIT_STREAM_SPLIT_ROWS, rows, row_bytes, in0=a, out0=out)
    half = row_bytes // 4
    torch.cuda.synchronize()
    assert torch.equal(out, a[:, :half] ^ a[:, half:])
    x, y = words(rows, row_bytes, 2), words(rows, row_bytes, 3)
    dit.dit_stream_pattern(dit.DIT_STREAM_TWO_IN, rows, row_bytes, in0=x, in1=y, out0=out)
    torch.cuda.synchronize()
    assert torch.equal(out, x ^ y)


@pytest.mark.parametrize("rows,row_bytes", SHAPES)
def test_row_wave_copies(rows, row_bytes):
    x, y = words(rows, row_bytes, 4), words(rows, row_bytes, 5)
    ox, oy = torch.zeros_like(x), torch.zeros_like(y)
    dit.dit_stream_pattern(dit.DIT_STREAM_ROW_WAVE, rows, row_bytes, in0=x, out0=ox)
    torch.cuda.synchronize()
    assert torch.equal(ox, x)
    ox.zero_()
    dit.dit_stream_pattern(dit.DIT_STREAM_ROW_WAVE_2X2, rows, row_bytes, in0=x, in1=y, out0=ox, out1=oy)
    torch.cuda.synchronize()
    assert torch.equal(ox, x) and torch.equal(oy, y)


@pytest.mark.parametrize("rows,heads,head_bytes", [(5, 32, 256), (17, 4, 128), (3, 3, 16), (2, 48, 256)])
def test_head_major_copy(rows, heads, head_bytes):
    row_bytes = heads * head_bytes
    x = words(rows, row_bytes, 6)
    out = torch.empty((heads, rows, head_bytes // 4), dtype=torch.int32, device=DEV)
    dit.dit_stream_pattern(dit.DIT_STREAM_HEAD_MAJOR, rows, row_bytes, in0=x, out0=out, heads=heads)
    torch.cuda.synchronize()
    assert torch.equal(out, x.view(rows, heads, -1).transpose(0, 1))


def test_read_and_write():
    rows, row_bytes = 9, 4096
    out = torch.full((rows, row_bytes // 4), 7, dtype=torch.int32, device=DEV)
    dit.dit_stream_pattern(dit.DIT_STREAM_WRITE, rows, row_bytes, out0=out)
    torch.cuda.synchronize()
    # vector c holds four copies of its index c
    idx = torch.arange(rows * row_bytes // 16, device=DEV, dtype=torch.int32).repeat_interleave(4)
    assert torch.equal(out.view(-1), idx)
    # the read stream leaves its sink untouched unless the XOR of everything read is its key;
    # an all-zero input XORs to 0, which is not the key
    sink = torch.full((4,), 5, dtype=torch.int32, device=DEV)
    zeros = torch.zeros((rows, row_bytes // 4), dtype=torch.int32, device=DEV)
    dit.dit_stream_pattern(dit.DIT_STREAM_READ, rows, row_bytes, in0=zeros, out0=sink)
    torch.cuda.synchronize()
    assert torch.equal(sink, torch.full((4,), 5, dtype=torch.int32, device=DEV))
