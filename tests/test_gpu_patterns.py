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
def test_row_group_copies(rows, row_bytes):
    x, y = words(rows, row_bytes, 4), words(rows, row_bytes, 5)
    ox, oy = torch.zeros_like(x), torch.zeros_like(y)
    dit.dit_stream_pattern(dit.DIT_STREAM_ROW_GROUP, rows, row_bytes, in0=x, out0=ox)
    torch.cuda.synchronize()
    assert torch.equal(ox, x)
    ox.zero_()
    dit.dit_stream_pattern(dit.DIT_STREAM_ROW_GROUP_2X2, rows, row_bytes, in0=x, in1=y, out0=ox, out1=oy)
    torch.cuda.synchronize()
    assert torch.equal(ox, x) and torch.equal(oy, y)


@pytest.mark.parametrize("rows,heads,head_bytes", [(5, 32, 256), (17, 4, 128), (3, 3, 16), (2, 48, 256), (7, 3, 512),
                                                   (130, 32, 256), (1, 1, 16)])
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


@pytest.mark.parametrize("planes,n,ld", [(1, 1, 4), (2, 5, 8), (3, 127, 128), (2, 128, 132), (2, 129, 132),
                                         (1, 300, 304), (2, 1953, 1984), (32, 1953, 1984)])
def test_score_tiles(planes, n, ld):
    """Every word of each plane's n x n block (columns up to n rounded up to 4) is written with its tag when the
    means are zero; the rest of each row keeps its fill; non-zero means change the words (the loads are live)."""
    rows, row_bytes = planes * n, 4 * ld
    print(f"[score_tiles] planes={planes} n={n} ld={ld}", flush=True)
    qm = torch.zeros((rows, 128), dtype=torch.float32, device=DEV)
    km = torch.zeros_like(qm)
    out = torch.full((rows, ld), -7, dtype=torch.int32, device=DEV)
    dit.dit_stream_pattern(dit.DIT_STREAM_SCORE_TILES, rows, row_bytes, in0=qm, in1=km, out0=out, heads=n)
    torch.cuda.synchronize()
    cols = -(-n // 4) * 4
    r = torch.arange(rows, device=DEV, dtype=torch.int64).unsqueeze(1)
    c = torch.arange(cols, device=DEV, dtype=torch.int64).unsqueeze(0)
    tags = (r * 65536 + c) & 0xFFFFFFFF
    assert torch.equal(out[:, :cols].to(torch.int64) & 0xFFFFFFFF, tags)
    assert bool((out[:, cols:] == -7).all())
    del tags
    g = torch.Generator(device=DEV).manual_seed(8)
    qm.copy_(torch.randn(qm.shape, generator=g, device=DEV))
    km.copy_(torch.randn(km.shape, generator=g, device=DEV))
    before = out.clone()
    dit.dit_stream_pattern(dit.DIT_STREAM_SCORE_TILES, rows, row_bytes, in0=qm, in1=km, out0=out, heads=n)
    torch.cuda.synchronize()
    assert not torch.equal(out[:, :cols], before[:, :cols])
    assert bool((out[:, cols:] == -7).all())


@pytest.mark.parametrize("planes,n,ld", [(1, 1, 4), (2, 5, 8), (3, 200, 200), (2, 256, 260), (2, 257, 260),
                                         (1, 1000, 1000), (2, 1953, 1984), (32, 1953, 1984), (1, 4096, 4096)])
def test_topk_rows(planes, n, ld):
    """Each row's ceil(n / 4) kept words carry their tags when the scores are zero (and nothing past them is
    written); non-zero scores in the first n words change them, words past n in the row do not."""
    rows, keep = planes * n, -(-n // 4)
    print(f"[topk_rows] planes={planes} n={n} ld={ld}", flush=True)
    scores = torch.zeros((rows, ld), dtype=torch.float32, device=DEV)
    out = torch.full((rows * keep + 64,), -7, dtype=torch.int32, device=DEV)
    dit.dit_stream_pattern(dit.DIT_STREAM_TOPK_ROWS, rows, 4 * ld, in0=scores, out0=out, heads=n)
    torch.cuda.synchronize()
    r = torch.arange(rows, device=DEV, dtype=torch.int64).unsqueeze(1)
    j = torch.arange(keep, device=DEV, dtype=torch.int64).unsqueeze(0)
    tags = ((r * 65536 + j) & 0xFFFFFFFF).reshape(-1)
    got = out[:rows * keep].to(torch.int64) & 0xFFFFFFFF
    assert torch.equal(got, tags)
    assert bool((out[rows * keep:] == -7).all())
    if ld > n:  # words past n are outside the loads' range: a change there changes nothing
        scores[:, n:] = 3.0
        dit.dit_stream_pattern(dit.DIT_STREAM_TOPK_ROWS, rows, 4 * ld, in0=scores, out0=out, heads=n)
        torch.cuda.synchronize()
        assert torch.equal(out[:rows * keep].to(torch.int64) & 0xFFFFFFFF, tags)
    g = torch.Generator(device=DEV).manual_seed(9)
    scores[:, :n] = torch.randn((rows, n), generator=g, device=DEV)
    dit.dit_stream_pattern(dit.DIT_STREAM_TOPK_ROWS, rows, 4 * ld, in0=scores, out0=out, heads=n)
    torch.cuda.synchronize()
    assert not torch.equal(out[:rows * keep].to(torch.int64) & 0xFFFFFFFF, tags)
