"""The C ABI without a GPU: the library loads, exports every entry point the
header declares, reports sizes, and rejects bad arguments before launching
anything (validation never touches the device)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "backlite.h")


@pytest.fixture(scope="module")
def L():
    from block_sparse_attention_fa_amd import _lib
    if not os.path.exists(_lib.LIB_PATH):
        pytest.fail("libbacklite.so is not built (run __graft_entry__.build())")
    return _lib.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(backlite_\w+)\s*\(", text)))


def test_exports_every_declared_symbol(L):
    names = declared_functions()
    assert len(names) >= 8
    for nm in names:
        assert hasattr(L, nm), f"{nm} not exported"


def test_sizes(L):
    assert L.backlite_tile_lse_elems(1, 2, 1024, 0) == 2 * 64 * 128
    assert L.backlite_tile_lse_elems(1, 1, 300, 1) == 6 * 128          # T = 3 -> 6 pairs
    assert L.backlite_tile_lse_elems(1, 40, 75600, 0) == 40 * 591 * 591 * 128
    assert L.backlite_mask_elems(2, 3, 129, 128) == 2 * 3 * 4
    assert L.backlite_mask_elems(2, 3, 129, 64) == 2 * 3 * 3 * 2      # Tq = 3 query tiles x T = 2
    assert L.backlite_mask_elems(2, 3, 129, 96) == 0
    assert L.backlite_count_elems(2, 3, 129, 128) == 2 * 3 * 2
    assert L.backlite_count_elems(2, 3, 129, 64) == 2 * 3 * 3
    # D and LSE*log2(e): 1*2*100 floats = 800 B -> 1024 each; kbar: 1*2*1*64 floats = 512 B;
    # G_K/G_V chunk plan: NK = 2 key tiles, 4 + 11*2 int32 = 104 B -> 256; partial sums:
    # 2 x 2 x 128 x 64 floats = 131072 B
    base = 2 * 1024 + 512 + 256 + 131072
    assert L.backlite_bwd_workspace_bytes(1, 2, 2, 100, 64) == base
    assert L.backlite_tile_lse_elems(0, 1, 1, 0) == 0
    # stored-G_S workspace: base, 256 B of state words, qbase (2 x 1 uint32 -> 256 B),
    # kslot (2 x 1 x 1 uint32 -> 256 B), then 34816 B (32 KB G_S + 2 KB row sums) per slot
    assert L.backlite_bwd_workspace_bytes_stored(1, 2, 2, 100, 64, 128, 0) == base
    assert L.backlite_bwd_workspace_bytes_stored(1, 2, 2, 100, 64, 128, 3) == base + 3 * 256 + 3 * 34816
    # 64-row query tiles: Tq = 2; qbase 2 x 2 uint32, kslot 2 x 1 x 2 uint32 (each -> 256 B);
    # 16 KB G_S + 1 KB sums per slot
    assert L.backlite_bwd_workspace_bytes_stored(1, 2, 2, 100, 64, 64, 3) == base + 3 * 256 + 3 * 17408
    assert L.backlite_bwd_state_offset(1, 2, 2, 100, 64) == base
    # the 32k-token video shape: T = 256, 40 heads
    big = L.backlite_bwd_workspace_bytes(1, 40, 40, 32760, 128)
    assert L.backlite_bwd_workspace_bytes_stored(1, 40, 40, 32760, 128, 128, 1000) == \
        big + 256 + 40 * 256 * 4 + 40 * 256 * 256 * 4 + 1000 * 34816


FAKE = ctypes.c_void_p(1 << 20)          # 16-byte aligned, never dereferenced
MIS = ctypes.c_void_p((1 << 20) + 2)     # misaligned


def _fwd(L, B=1, n=128, H=2, Hk=2, d=64, scale=0.125, q=FAKE, tl=FAKE, causal=0, window=0, tw=None):
    return L.backlite_fwd(q, FAKE, FAKE, B, n, H, Hk, d, scale, causal, window, FAKE, None, FAKE, tl, tw, None)


@pytest.mark.parametrize("kw,code", [
    (dict(H=3, Hk=2), -1), (dict(n=0), -1), (dict(B=0), -1), (dict(d=96), -2), (dict(d=256), -2),
    (dict(n=131073), -2), (dict(scale=0.0), -1), (dict(scale=float("nan")), -1),
    (dict(scale=float("inf")), -1), (dict(q=None), -1), (dict(q=MIS), -1), (dict(tl=MIS), -1),
    (dict(window=64), -1), (dict(causal=1, window=-1), -1),
    (dict(tl=None, tw=FAKE), -1), (dict(tw=MIS), -1),
])
def test_fwd_validation(L, kw, code):
    assert _fwd(L, **kw) == code
    assert L.backlite_last_error()


def _mask(L, negl=0.05, tl=FAKE, keep=FAKE, n=256, causal=0, window=0, q_tile=128):
    return L.backlite_mask(tl, FAKE, 1, 2, n, causal, window, q_tile, negl, keep, FAKE, FAKE, FAKE, FAKE, None, None)


@pytest.mark.parametrize("kw,code", [
    (dict(negl=-0.1), -1), (dict(negl=1.0), -1), (dict(negl=float("nan")), -1),
    (dict(tl=None), -1), (dict(keep=None), -1), (dict(keep=MIS), -1), (dict(n=0), -1),
    (dict(window=64), -1), (dict(causal=1, window=-5), -1), (dict(q_tile=32), -2), (dict(q_tile=0), -2),
])
def test_mask_validation(L, kw, code):
    assert _mask(L, **kw) == code


@pytest.mark.parametrize("kw,code", [
    (dict(tw=None), -1), (dict(negl=1.0), -1), (dict(tw=MIS), -1), (dict(causal=0, window=8), -1),
    (dict(n=131073), -2), (dict(q_tile=256), -2),
])
def test_mask_compact_validation(L, kw, code):
    a = dict(tw=FAKE, n=256, causal=1, window=0, negl=0.05, q_tile=128)
    a.update(kw)
    assert L.backlite_mask_compact(a["tw"], 1, 2, a["n"], a["causal"], a["window"], a["q_tile"], a["negl"], FAKE,
                                   FAKE, FAKE, FAKE, FAKE, None, None) == code


def test_bwd_validation(L):
    args = [FAKE] * 11 + [1, 256, 4, 2, 128, 0.1, 0, 0, 128, FAKE, FAKE, FAKE]
    # workspace too small / missing
    assert L.backlite_bwd(*args, FAKE, 16, None) == -3
    assert L.backlite_bwd(*args, None, 1 << 20, None) == -3
    bad = list(args)
    bad[14] = 3                                   # H_k does not divide H
    assert L.backlite_bwd(*bad, FAKE, 1 << 20, None) == -1
    bad = list(args)
    bad[15] = 80                                  # head_dim
    assert L.backlite_bwd(*bad, FAKE, 1 << 20, None) == -2
    bad = list(args)
    bad[18] = 64                                  # a window without causal
    assert L.backlite_bwd(*bad, FAKE, 1 << 20, None) == -1
    bad = list(args)
    bad[19] = 32                                  # q_tile
    assert L.backlite_bwd(*bad, FAKE, 1 << 20, None) == -2


def test_status_strings(L):
    for c in (0, -1, -2, -3, -4):
        assert L.backlite_status_string(c)


def test_bwd_noalloc_rejects_shapes_beyond_the_scratch(L):
    """The allocation-free backward's fixed scratch is 256 MiB: the 32k-token
    shape with 1024 heads needs more for its D and key-mean arrays alone, so the
    call returns the workspace status before touching the device."""
    assert L.backlite_bwd_noalloc_scratch_bytes() == 256 << 20
    args = [FAKE] * 11 + [1, 32760, 1024, 1024, 128, 0.088, 0, 0, 128, FAKE, FAKE, FAKE, None]
    assert L.backlite_bwd_noalloc(*args) == -3
    assert b"scratch" in L.backlite_last_error()
    bad = list(args)
    bad[15] = 96                                  # head_dim: validated first
    assert L.backlite_bwd_noalloc(*bad) == -2
