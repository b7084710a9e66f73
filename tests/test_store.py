"""The storage tier's reader (e0_store, host code only): per-layer stacked
bundle files read by byte range on a pool of I/O threads. Bundles land byte
for byte in their destinations, in buffered and (where the file system
allows it) O_DIRECT mode, also into unaligned destinations; bad ids, O_DIRECT
bundle sizes that are not 4096-byte multiples and missing files are rejected
with their error codes; tickets report blocked and read times.
"""

import mmap

import numpy as np
import pytest


@pytest.fixture(scope="module")
def api():
    from sparse_moe_decode_amd import api as _api
    return _api


def _files(tmp_path, L, E, bundle, seed=5):
    rng = np.random.default_rng(seed)
    data = rng.integers(0, 256, size=(L, E, bundle), dtype=np.uint8)
    paths = []
    for l in range(L):
        p = tmp_path / f"layer{l}.bin"
        data[l].tofile(p)
        paths.append(str(p))
    return data, paths


def _aligned(nbytes):
    """Page-aligned host buffer (anonymous mapping) as a numpy view."""
    m = mmap.mmap(-1, nbytes)
    return m, np.frombuffer(m, dtype=np.uint8)


def test_store_reads_into_unaligned_destinations(api, tmp_path):
    """Direct reads go through the threads' own aligned buffers, so any
    destination works (pinned pools of the driver cannot take direct reads)."""
    L, E, bundle = 1, 4, 4096
    data, paths = _files(tmp_path, L, E, bundle)
    try:
        st = api.Store(paths, E, bundle, io_threads=2, direct=True)
    except api.E0Error as e:
        if e.code == api.E0_ERR_IO:
            pytest.skip("O_DIRECT not supported by this file system")
        raise
    m, buf = _aligned(E * bundle + 64)
    base = buf.ctypes.data + 8
    st.wait(st.read(0, list(range(E)), [base + e * bundle for e in range(E)]))
    got = buf[8:8 + E * bundle].reshape(E, bundle)
    assert np.array_equal(got, data[0])
    st.close()
    del got, buf
    m.close()


@pytest.mark.parametrize("direct", [False, True])
def test_store_reads_bundles(api, tmp_path, direct):
    L, E, bundle = 3, 8, 3 * 4096
    data, paths = _files(tmp_path, L, E, bundle)
    try:
        st = api.Store(paths, E, bundle, io_threads=4, direct=direct)
    except api.E0Error as e:
        if direct and e.code == api.E0_ERR_IO:
            pytest.skip("O_DIRECT not supported by this file system")
        raise
    m, buf = _aligned(L * E * bundle)
    base = buf.ctypes.data
    rng = np.random.default_rng(6)
    want = []
    tickets = []
    for l in range(L):
        ids = rng.choice(E, size=5, replace=False)
        dst = [base + (l * E + int(e)) * bundle for e in ids]
        tickets.append(st.read(l, ids, dst))
        want += [(l, int(e)) for e in ids]
    for tk in tickets:
        blocked, read = st.wait(tk)
        assert blocked >= 0.0 and read >= 0.0
    view = buf.reshape(L, E, bundle)
    for l, e in want:
        assert np.array_equal(view[l, e], data[l, e]), f"layer {l} bundle {e}"
    assert st.bytes_read() == len(want) * bundle
    st.close()
    del view, buf
    m.close()


def test_store_errors(api, tmp_path):
    L, E, bundle = 2, 4, 4096
    data, paths = _files(tmp_path, L, E, bundle)
    with pytest.raises(api.E0Error) as ei:
        api.Store(paths + [str(tmp_path / "missing.bin")], E, bundle, direct=False)
    assert ei.value.code == api.E0_ERR_IO
    with pytest.raises(api.E0Error) as ei:
        api.Store(paths, E, 1000, direct=True)  # O_DIRECT needs 4096-byte multiples
    assert ei.value.code == api.E0_ERR_ALIGN
    st = api.Store(paths, E, bundle, io_threads=2, direct=False)
    m, buf = _aligned(bundle * 2)
    with pytest.raises(api.E0Error) as ei:
        st.read(0, [E], [buf.ctypes.data])
    assert ei.value.code == api.E0_ERR_RANGE
    with pytest.raises(api.E0Error) as ei:
        st.wait(12345)
    assert ei.value.code == api.E0_ERR_STATE
    st.close()
    del buf
    m.close()
