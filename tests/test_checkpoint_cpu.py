"""Checkpoint host logic without a GPU: the layout fingerprint against its
documented definition (64-bit FNV-1a over little-endian int64 fields), what
it tells apart, and every check zs_checkpoint_load makes on a file before
it touches device memory (files built here from the documented format)."""

import ctypes
import struct

import pytest

import zero_sharded_optimizer_shard_amd as zs
from oracle.layout import build_layout
from zero_sharded_optimizer_shard_amd._zs import ZS_EALIGN, ZS_EINVAL

NUMELS = [1000, 70000, 7, 129, 20000]
FAKE_DEV = 0x10000          # aligned, never dereferenced: the calls fail first


def fnv1a64(data: bytes) -> int:
    h = 0xcbf29ce484222325
    for b in data:
        h = ((h ^ b) * 0x100000001b3) % (1 << 64)
    return h


def test_fnv1a64_published_vectors():
    # the FNV-1a 64-bit test vectors of its authors' reference list
    assert fnv1a64(b"") == 0xcbf29ce484222325
    assert fnv1a64(b"a") == 0xaf63dc4c8601ec8c
    assert fnv1a64(b"foobar") == 0x85944171f73967e8


def documented_fingerprint(mode, world, rank, align_elems, bucket_elems,
                           numels):
    fields = [mode, world, rank, align_elems, bucket_elems, len(numels),
              *numels]
    return fnv1a64(b"".join(struct.pack("<q", v) for v in fields))


@pytest.mark.parametrize("W,rank,cap,align", [(3, 1, 25 << 20, 256),
                                              (8, 7, 3 * 256 * 40, 512),
                                              (1, 0, 0, 16)])
def test_fingerprint_is_the_documented_hash(W, rank, cap, align):
    lay = zs.zs_layout_build(NUMELS, W, rank, cap, align)
    # the full bucket size by the layout rule (oracle's tensor offsets)
    unit = W * (align // 2)
    if cap > 0:
        full = (cap // 2 // unit) * unit
    else:
        o = build_layout(NUMELS, W, rank, cap, align)
        end = o.tensor_flat_off[-1] + NUMELS[-1]
        full = max(-(-end // unit) * unit, unit)
    assert zs.zs_layout_fingerprint(lay) == documented_fingerprint(
        0, W, rank, align // 2, full, NUMELS)
    lt = zs.zs_layout_build_tensors(NUMELS, W, rank, align)
    assert zs.zs_layout_fingerprint(lt) == documented_fingerprint(
        1, W, rank, align // 2, 0, NUMELS)


def test_fingerprint_tells_layouts_apart():
    def fp(numels=NUMELS, W=3, rank=1, cap=3 * 256 * 40, align=256):
        return zs.zs_layout_fingerprint(
            zs.zs_layout_build(numels, W, rank, cap, align))

    base = fp()
    assert fp() == base                                   # deterministic
    others = [fp(W=4), fp(rank=2), fp(cap=3 * 256 * 41), fp(align=512),
              fp(numels=NUMELS[:-1] + [20001]),
              fp(numels=NUMELS[::-1]), fp(numels=NUMELS + [0]),
              zs.zs_layout_fingerprint(zs.zs_layout_build_tensors(
                  NUMELS, 3, 1, 256))]
    assert base not in others and len(set(others)) == len(others)
    # caps that round to the same bucket size give the same layout
    assert fp(cap=3 * 256 * 40 + 300) == base


def header(lay, rows=3, step=5, magic=b"ZSCKPT01", version=1, fp=None,
           payload=None, world=None, rank=None, n_tiles=None):
    f, n, nt, W, _ = lay.sizes()
    r = zs.zs_layout_rank(lay)[1]
    return struct.pack(
        "<8sIIQqqqiiQ", magic, version, rows,
        zs.zs_layout_fingerprint(lay) if fp is None else fp, step,
        nt if n_tiles is None else n_tiles, n, W if world is None else world,
        r if rank is None else rank,
        nt * rows * zs.ZS_TILE * 4 if payload is None else payload)


def load(lay, path, rows=3, state=FAKE_DEV):
    step = ctypes.c_int64(-1)
    rc = zs.lib().zs_checkpoint_load(
        lay.handle, None if path is None else str(path).encode(),
        ctypes.c_void_p(state), rows, ctypes.byref(step), None)
    return rc, step.value


def test_header_is_64_bytes():
    assert len(header(zs.zs_layout_build(NUMELS, 3, 1))) == 64


def test_load_refuses_before_touching_the_state(tmp_path):
    lay = zs.zs_layout_build(NUMELS, 3, 1)
    other_rank = zs.zs_layout_build(NUMELS, 3, 2)
    other_list = zs.zs_layout_build(NUMELS[:-1] + [20001], 3, 1)
    p = tmp_path / "ck"
    cases = [
        ("missing file", None, zs.ZS_EIO),
        ("empty file", b"", zs.ZS_EIO),
        ("short header", header(lay)[:40], zs.ZS_EIO),
        ("wrong magic", header(lay, magic=b"ZSCKPT02"), zs.ZS_EIO),
        ("wrong version", header(lay, version=2), zs.ZS_EIO),
        ("another rank", header(other_rank), zs.ZS_EMISMATCH),
        ("another tensor list", header(other_list), zs.ZS_EMISMATCH),
        ("fingerprint of this layout, another world",
         header(lay, world=4), zs.ZS_EMISMATCH),
        ("tile count differs", header(lay, n_tiles=1), zs.ZS_EMISMATCH),
        ("pure-bf16 rows", header(lay, rows=2), zs.ZS_EMISMATCH),
        ("payload size inconsistent", header(lay, payload=8),
         zs.ZS_EIO),
        ("negative step", header(lay, step=-1), zs.ZS_EIO),
    ]
    for name, data, code in cases:
        if data is None:
            path = tmp_path / "does-not-exist"
        else:
            p.write_bytes(data)
            path = p
        rc, step = load(lay, path)
        assert rc == code, (name, rc, zs.zs_last_error())
        assert step == -1, name
        assert zs.zs_last_error(), name


def test_argument_errors(tmp_path):
    lay = zs.zs_layout_build(NUMELS, 3, 1)
    p = str(tmp_path / "ck").encode()
    L = zs.lib()
    assert load(lay, None)[0] == ZS_EINVAL
    assert load(lay, tmp_path / "ck", rows=4)[0] == ZS_EINVAL
    assert load(lay, tmp_path / "ck", state=0)[0] == ZS_EINVAL
    assert load(lay, tmp_path / "ck", state=FAKE_DEV + 4)[0] == ZS_EALIGN
    assert L.zs_checkpoint_load(lay.handle, p, ctypes.c_void_p(FAKE_DEV), 3,
                                None, None) == ZS_EINVAL
    assert L.zs_checkpoint_load(None, p, ctypes.c_void_p(FAKE_DEV), 3,
                                None, None) == ZS_EINVAL
    save = L.zs_checkpoint_save
    dev = ctypes.c_void_p(FAKE_DEV)
    assert save(lay.handle, None, dev, 3, 1, None) == ZS_EINVAL
    assert save(None, p, dev, 3, 1, None) == ZS_EINVAL
    assert save(lay.handle, p, None, 3, 1, None) == ZS_EINVAL
    assert save(lay.handle, p, dev, 1, 1, None) == ZS_EINVAL
    assert save(lay.handle, p, dev, 3, -1, None) == ZS_EINVAL
    assert save(lay.handle, p, ctypes.c_void_p(FAKE_DEV + 8), 3, 1,
                None) == ZS_EALIGN
    assert not (tmp_path / "ck").exists()
    assert not (tmp_path / "ck.tmp").exists()
    out = ctypes.c_uint64()
    assert L.zs_layout_fingerprint(None, ctypes.byref(out)) == ZS_EINVAL
    assert L.zs_layout_fingerprint(lay.handle, None) == ZS_EINVAL
    assert zs.zs_strerror(zs.ZS_EIO).startswith("checkpoint file")
    assert zs.zs_strerror(zs.ZS_EMISMATCH).startswith("checkpoint written")
