"""Helpers shared by the GPU tests: host-side packing of masks (written from
the layout documented in include/scape.h, independent of the library) and
comparisons against the oracle."""

import numpy as np

TILE = 4096


def words_per_partition(n_p):
    return (n_p + 63) // 64


def tiles_per_partition(n_p):
    return (n_p + TILE - 1) // TILE


def pack_mask(local_idx_per_partition, n_p):
    """(bits u64 [P*W], idx u32 [P*k], tile_off u32 [P*T]) on the host."""
    P = len(local_idx_per_partition)
    W, T = words_per_partition(n_p), tiles_per_partition(n_p)
    bits = np.zeros((P, W * 64), dtype=np.uint8)
    idx, toff = [], []
    for p, loc in enumerate(local_idx_per_partition):
        loc = np.asarray(loc, dtype=np.int64)
        bits[p, loc] = 1
        idx.append(loc + p * n_p)
        toff.append(np.searchsorted(loc, np.arange(T, dtype=np.int64) * TILE, side="left"))
    words = np.packbits(bits, axis=1, bitorder="little").view("<u8").reshape(-1)
    return (words.astype(np.uint64), np.concatenate(idx).astype(np.uint32),
            np.concatenate(toff).astype(np.uint32))


def unpack_bits(words, P, n_p):
    """bool [P][W*64] from the packed words (int64/uint64 array)."""
    W = words_per_partition(n_p)
    w = np.ascontiguousarray(np.asarray(words).view(np.uint64).reshape(P, W))
    return np.unpackbits(w.view(np.uint8), axis=1, bitorder="little").astype(bool)


def check_mask(bits_t, idx_t, toff_t, want_local, n_p):
    """The three views of a device mask equal the oracle's selection."""
    P = len(want_local)
    wb, wi, wt = pack_mask(want_local, n_p)
    got_bits = bits_t.cpu().numpy().view(np.uint64)
    got_idx = idx_t.cpu().numpy().view(np.uint32)
    got_toff = toff_t.cpu().numpy().view(np.uint32)
    if not np.array_equal(got_bits, wb):
        ub = unpack_bits(got_bits, P, n_p)
        for p in range(P):
            have = np.flatnonzero(ub[p])
            if not np.array_equal(have, want_local[p]):
                extra = np.setdiff1d(have, want_local[p])[:8]
                miss = np.setdiff1d(want_local[p], have)[:8]
                raise AssertionError(f"partition {p}: {have.size} bits set (want {len(want_local[p])}); "
                                     f"extra {extra.tolist()} missing {miss.tolist()}")
        raise AssertionError("mask words differ in padding bits")
    assert np.array_equal(got_idx, wi), "index list differs"
    assert np.array_equal(got_toff, wt), "tile offsets differ"


def assert_close(got, want, rtol, name=""):
    """Element-wise |got - want| <= rtol * |want| (zero <-> zero exactly);
    reports the number of bitwise-equal entries."""
    got = np.asarray(got, dtype=np.float32)
    want = np.asarray(want, dtype=np.float32)
    assert got.shape == want.shape, name
    gd, wd = got.astype(np.float64), want.astype(np.float64)
    bad = np.abs(gd - wd) > rtol * np.abs(wd)
    bad |= (wd == 0) & (gd != 0)
    bad |= np.isnan(gd) != np.isnan(wd)
    if bad.any():
        i = np.flatnonzero(bad)[:5]
        raise AssertionError(f"{name}: {int(bad.sum())} entries beyond rtol={rtol}; first {i.tolist()} "
                             f"got {gd[i].tolist()} want {wd[i].tolist()}")
    return int(np.sum(got.view(np.uint32) == want.view(np.uint32)))
