"""GPU tests of the streaming diagnostics, through the C ABI.

tq_stream_rw moves the write side's bytes with no arithmetic: per row, the XOR
of the 16-byte input chunks g, g + 4, ... (g < 4) goes to output chunks g,
g + 4, ..., and plane p (p < nplanes) gets bits 0..29 of the first dword of
fold p as a float.  Checked exactly against numpy on ragged row counts (a
partial last 16-row tile) and two row shapes; rows past `rows` are untouched."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def tq():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from compressed_decode_attention_kv_amd import tq as lib
    return lib


def _expect(src, out_chunks, nplanes):
    rows, in_chunks = src.shape[0], src.shape[1]
    folds = np.zeros((rows, 4, 4), dtype=np.uint32)
    for g in range(4):
        for c in range(g, in_chunks, 4):
            folds[:, g] ^= src[:, c]
    out = np.zeros((rows, out_chunks, 4), dtype=np.uint32)
    for c in range(out_chunks):
        out[:, c] = folds[:, c % 4]
    planes = (folds[:, :nplanes, 0] & np.uint32(0x3FFFFFFF)).view(np.float32).T.copy()
    return out, planes


@pytest.mark.parametrize("rows,in_row,out_row,nplanes", [(1000, 256, 64, 2), (37, 1024, 128, 1), (16, 64, 64, 0)])
def test_stream_rw_moves_the_expected_bytes(tq, rows, in_row, out_row, nplanes):
    rng = np.random.default_rng(rows)
    src = rng.integers(0, 2**32, size=(rows, in_row // 16, 4), dtype=np.uint32)
    dsrc = torch.from_numpy(src.view(np.int32)).cuda()
    spare = 3  # rows past the end keep their sentinel
    dst = torch.full(((rows + spare) * out_row // 4,), -7, dtype=torch.int32, device="cuda")
    pl = torch.empty((max(nplanes, 1), rows), dtype=torch.float32, device="cuda")
    tq.stream_rw(dsrc, rows, in_row, dst, out_row, pl if nplanes else None, nplanes)
    torch.cuda.synchronize()
    want_out, want_pl = _expect(src, out_row // 16, nplanes)
    got = dst.cpu().numpy().view(np.uint32)
    assert np.array_equal(got[:rows * out_row // 4].reshape(rows, out_row // 16, 4), want_out)
    assert np.all(got[rows * out_row // 4:] == np.uint32(2**32 - 7))
    if nplanes:
        assert np.array_equal(pl.cpu().numpy()[:nplanes].view(np.uint32), want_pl.view(np.uint32))
