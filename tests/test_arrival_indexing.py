"""CPU emulation of the arrival copy kernel's addressing (arrival.hip).

Replays, for every workgroup (piece) and thread, the index arithmetic the copy
kernel runs -- the host's chunking of the gathered matrix into row chunks x
slabs of K, the thread's stepping through its piece without division, the
repeat of the first element by lanes past the end -- and checks that every
load stays inside its shard, every store inside gather_out, and that the
stores of a piece cover exactly that piece.  No GPU is involved.
"""
import numpy as np
import pytest

THREADS, BATCH = 256, 16


def chunking(r, m_local, k, rows_chunk, max_flags=65535, max_slabs=16):
    """The host's split (api.cpp, arrival mode): slabs of whole 64-element steps."""
    m = r * m_local
    slabs = min((k + 63) // 64, max_slabs)
    slab_cols = ((k + slabs - 1) // slabs + 63) // 64 * 64
    slabs = (k + slab_cols - 1) // slab_cols
    while ((m + rows_chunk - 1) // rows_chunk) * slabs > max_flags:
        rows_chunk *= 2
    chunks = (m + rows_chunk - 1) // rows_chunk
    return m, slabs, slab_cols, rows_chunk, chunks


def emulate_piece(w, r, m_local, k, rows_chunk, slab_cols, slabs, chunks, first_chunk):
    """(shard index, element offset in the shard, element offset in gather_out) of every
    16-byte load / store of workgroup w, vector path (k and slab_cols multiples of 8)."""
    m = r * m_local
    sl, g = w // chunks, (first_chunk + w % chunks) % chunks
    row0 = g * rows_chunk
    rows = rows_chunk if row0 + rows_chunk <= m else m - row0
    c0 = sl * slab_cols
    cols = slab_cols if c0 + slab_cols <= k else k - c0
    b0 = row0 // m_local
    one_shard = (row0 + rows - 1) // m_local == b0
    per_row = cols // 8
    n = rows * per_row
    dq, dc = THREADS // per_row, THREADS % per_row
    t = np.arange(THREADS, dtype=np.int64)
    rr, cc = t // per_row, t % per_row
    shard, soff, doff = [], [], []
    i0 = t.copy()
    while True:
        live = i0 < n                      # threads still in the loop
        if not live.any():
            break
        R0 = col0 = None
        for j in range(BATCH):
            R = row0 + rr
            col = c0 + cc * 8
            if j == 0:
                R0, col0 = R.copy(), col.copy()
            else:
                past = i0 + j * THREADS >= n
                R = np.where(past, R0, R)
                col = np.where(past, col0, col)
            bb = np.full_like(R, b0) if one_shard else R // m_local
            shard.append(bb[live])
            soff.append(((R - bb * m_local) * k + col)[live])
            doff.append((R * k + col)[live])
            rr = rr + dq
            cc = cc + dc
            wrap = cc >= per_row
            cc = np.where(wrap, cc - per_row, cc)
            rr = np.where(wrap, rr + 1, rr)
        i0 = i0 + BATCH * THREADS
    return (np.concatenate(shard), np.concatenate(soff), np.concatenate(doff),
            (row0, rows, c0, cols))


# every shape the arrival tests and the benchmark use, with the tile heights the GEMM can pick
SHAPES = [(2, 1, 256), (4, 16, 512), (8, 5, 1000), (4, 100, 264), (8, 33, 768), (2, 129, 256),
          (8, 128, 512), (4, 64, 512), (4, 64, 1024), (8, 512, 4096)]


@pytest.mark.parametrize("r,m_local,k", SHAPES)
@pytest.mark.parametrize("tile_rows", [128, 224, 256])
def test_arrival_copy_addresses(r, m_local, k, tile_rows):
    if k % 8:
        pytest.skip("element path (k not a multiple of 8): one element per thread, no batching")
    m, slabs, slab_cols, rows_chunk, chunks = chunking(r, m_local, k, tile_rows)
    covered = np.zeros(m * k // 8, dtype=np.int64)
    for first_chunk in sorted({0, chunks - 1}):
        covered[:] = 0
        for w in range(chunks * slabs):
            shard, soff, doff, (row0, rows, c0, cols) = emulate_piece(
                w, r, m_local, k, rows_chunk, slab_cols, slabs, chunks, first_chunk)
            assert np.all((shard >= 0) & (shard < r))
            assert np.all((soff >= 0) & (soff + 8 <= m_local * k)), "load outside its shard"
            assert np.all((doff >= 0) & (doff + 8 <= m * k)), "store outside gather_out"
            assert np.all(doff % 8 == 0)
            # the source element is the gathered element the store writes
            assert np.array_equal(shard * m_local * k + soff, doff)
            # the stores cover exactly this piece (repeats allowed)
            rows_idx, cols_idx = doff // k, doff % k
            assert np.all((rows_idx >= row0) & (rows_idx < row0 + rows))
            assert np.all((cols_idx >= c0) & (cols_idx < c0 + cols))
            uniq = np.unique(doff)
            assert uniq.size == rows * cols // 8, "piece not fully covered"
            covered[uniq // 8] += 1
        assert np.all(covered == 1), "pieces overlap or leave gaps"
