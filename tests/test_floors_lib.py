"""The floor probes' library (libattn_floors.so, timed by `bench.py --floors`) without a GPU:
it loads, exports its four probes, links no torch, and refuses sizes that its kernels could
not cover exactly, on the host before any HIP call."""
import ctypes
import os

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PATH = os.path.join(ROOT, "transformer_attention_03_amd", "libattn_floors.so")
P = 0x10000          # a fake 16-byte-aligned device address; never dereferenced


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(PATH):
        pytest.skip("libattn_floors.so not built")
    import bench
    return bench.floors_lib()


def test_exports_and_links_no_torch(L):
    for n in ("floor_empty", "floor_stream", "floor_stream_merge", "floor_gather", "floor_lds_read",
              "floor_lds_read64"):
        assert hasattr(L, n), n
    out = os.popen("ldd %s" % PATH).read()
    # library names only: the hexadecimal load addresses can hold any digit string
    names = [ln.split()[0] for ln in out.splitlines() if ln.strip()]
    assert names and not any("torch" in n or "c10" in n for n in names), names


@pytest.mark.parametrize("args", [
    (0, None), (65536, None),
])
def test_empty_refuses_bad_grids(L, args):
    assert L.floor_empty(*args) == -1


@pytest.mark.parametrize("src,nbytes,grid", [
    (None, 1 << 20, 128),          # null source
    (P + 4, 1 << 20, 128),         # misaligned source
    (P, 1000, 128),                # not a multiple of 16 * grid
    (P, 1 << 20, 0),
    (P, 0, 128),
])
def test_stream_refuses_bad_sizes(L, src, nbytes, grid):
    assert L.floor_stream(src, nbytes, grid, P, None) == -1


def test_stream_merge_refuses_uneven_split(L):
    assert L.floor_stream_merge(P, 16 * 127, 16, 8, P, P, P, None) == -1
    assert L.floor_stream_merge(P, 1 << 20, 0, 8, P, P, P, None) == -1
    assert L.floor_stream_merge(P, 1 << 20, 16, 8, None, P, P, None) == -1


def test_gather_refuses_bad_pools(L):
    assert L.floor_gather(P, P, P, 10, 4, 0, P, None) == -1          # empty pool
    assert L.floor_gather(P, P, P, 0, 4, 100, P, None) == -1         # no blocks
    assert L.floor_gather(P + 8, P, P, 10, 4, 100, P, None) == -1    # misaligned k
    assert L.floor_gather(P, P, P, 10 ** 8, 1, 100, P, None) == -1   # grid beyond 65535


def test_lds_read_refuses_bad_shapes(L):
    assert L.floor_lds_read(256, 384, 10, P, None) == -1      # threads not built
    assert L.floor_lds_read(0, 512, 10, P, None) == -1
    assert L.floor_lds_read(256, 512, 0, P, None) == -1
    assert L.floor_lds_read(256, 512, 10, None, None) == -1


def test_lds_read64_refuses_bad_modes(L):
    assert L.floor_lds_read64(256, 2, 10, P, None) == -1      # neither plain nor transposing
    assert L.floor_lds_read64(0, 0, 10, P, None) == -1
    assert L.floor_lds_read64(256, 1, 0, P, None) == -1
    assert L.floor_lds_read64(256, 0, 10, None, None) == -1
