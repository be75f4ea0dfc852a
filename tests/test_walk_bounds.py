"""Host-side bounds check of the attention kernels' address arithmetic (no GPU).

The bf16 kernels expand the Vertical-Slash index on the device into tiles of
key rows (query-major forward / dQ) or query rows (key-major dK / dV) and load
them with direct global -> LDS loads.  This test repeats that arithmetic on
the host, with the same integer formulas as the device code (local / global
block relabelling of a striped call, the prepared vertical lists, the
covered-column test, the tile-list capacities, the direct-load byte offsets
and LDS destinations), over every work item of a launch, and asserts that
every address stays inside its tensor or LDS array.  It runs on the shapes of
a 32-rank striped worker at N = 524288 (each rank's chunk, and all chunks in
one call) and of packed documents, with seeded random indices that include
the extreme entries (block-diagonals 0 and nb - 1, the first and last key of
a segment).
"""
import numpy as np
import pytest

BLOCK = 64


class Call:
    """The relabelling of one call (mirrors the device helpers)."""

    def __init__(self, n_global, cu, W=1, q_rank=0, k_rank=0, k_all=False):
        self.n_global, self.cu, self.W = n_global, list(cu), W
        self.q_rank, self.k_rank, self.k_all = q_rank, k_rank, k_all
        self.n_q = n_global if W == 1 else n_global // W
        self.n_k = n_global if (W == 1 or k_all) else n_global // W
        self.nqb, self.nkb = self.n_q // BLOCK, self.n_k // BLOCK

    def local_key_block(self, kb):
        kb = np.asarray(kb, np.int64)
        if self.W == 1:
            return np.where((kb >= 0) & (kb < self.nkb), kb, -1)
        if self.k_all:
            nc = self.nkb // self.W
            j = kb // self.W
            return np.where((kb >= 0) & (j < nc), (kb % self.W) * nc + j, -1)
        d = kb - self.k_rank
        j = d // self.W
        return np.where((kb >= 0) & (d >= 0) & (d % self.W == 0) & (j < self.nkb), j, -1)

    def global_key_block(self, j):
        j = np.asarray(j, np.int64)
        if self.W == 1:
            return j
        if self.k_all:
            nc = self.nkb // self.W
            return j // nc + self.W * (j % nc)
        return self.k_rank + self.W * j

    def local_query_block(self, qb):
        qb = np.asarray(qb, np.int64)
        if self.W == 1:
            return np.where((qb >= 0) & (qb < self.nqb), qb, -1)
        d = qb - self.q_rank
        i = d // self.W
        return np.where((d >= 0) & (d % self.W == 0) & (i < self.nqb), i, -1)

    def local_key_pos(self, m):
        m = np.asarray(m, np.int64)
        if self.W == 1:
            return m
        return self.local_key_block(m // BLOCK) * BLOCK + m % BLOCK

    def row_block(self, i):
        """(global query block, segment, segment start block, beta, blocks in segment)."""
        if self.W == 1:
            starts = np.asarray(self.cu) // BLOCK
            s = int(np.searchsorted(starts, i, side="right") - 1)
            return i, s, starts[s], i - starts[s], starts[s + 1] - starts[s]
        qb = self.q_rank + self.W * i
        return qb, 0, 0, qb, self.n_global // BLOCK


def random_index(rng, cu, k_v, k_g):
    """Sorted lists per segment with the extreme entries included."""
    out = []
    for a, e in zip(cu[:-1], cu[1:]):
        L, nb = e - a, (e - a) // BLOCK
        v = set(rng.choice(L, size=min(k_v, L), replace=False).tolist()) | {0, L - 1}
        g = set(rng.choice(nb, size=min(k_g, nb), replace=False).tolist()) | {0, nb - 1}
        out.append((np.array(sorted(v), np.int64) + a, np.array(sorted(g), np.int64)))
    return out


def prep_vertical(call, v_idx, seg):
    """vs_prep_vertical_kernel: the list's columns this call holds, ascending."""
    a, e = (call.cu[seg], call.cu[seg + 1]) if call.W == 1 else (0, call.n_global)
    m = np.asarray(v_idx)
    keep = (m >= a) & (m < e) & (call.local_key_block(m // BLOCK) >= 0)
    return m[keep]


def rows_tile_geometry(D):
    """RowsTiles<D> constants: (rows per direct load, loads per 32-row tile,
    padded group bytes, tile bytes)."""
    cpr = D // 8
    rpi = 64 // cpr
    nvl = 32 // rpi
    group = 1024 + 16
    return rpi, nvl, group, nvl * group


def check_dma_part(D, NP, row_bytes, n_rows, key_rows):
    """dma_part: every lane's byte offset row * rb + chunk byte stays inside the
    K / V rows of one (batch, head) and is representable in 32 bits, and the
    LDS destinations of all loads of a half-tile stay inside its tile."""
    rpi, nvl, group, tb = rows_tile_geometry(D)
    cpr = D // 8
    lanes = np.arange(64)
    rr, cb = lanes // cpr, ((lanes % cpr) ^ np.array([4 * (b & 3) if D == 128 else
                                                       4 * ((b >> 1) & 1) + 2 * ((b >> 2) & 1)
                                                       for b in lanes // cpr])) * 16
    assert cb.max() + 16 <= D * 2
    rows = np.asarray(key_rows, np.int64)
    assert rows.min() >= 0 and rows.max() < n_rows
    off = rows.max() * row_bytes + cb.max() + 16
    assert off < 2 ** 32 and off <= (n_rows - 1) * row_bytes + D * 2
    nu = nvl // NP
    for part in range(NP):
        for u0 in range(nu):
            dst = (part * nu + u0) * group
            assert dst + 64 * 16 <= tb
    assert rr.max() < rpi


def query_major_walk(call, lists, h_q, n_seg, D, row_bytes):
    """Tiles of the forward / dQ walk (qmajor_drive with one key stream of
    two waves: 128 threads, column batches of 256), for every (Q head, local
    query block): slash key blocks and gathered vertical columns."""
    nt, ncols = 128, 256
    R = ncols // nt - 1
    key_rows = []
    words_max = (max((e - a) // BLOCK for a, e in zip(call.cu[:-1], call.cu[1:]))
                 if call.W == 1 else call.n_global // BLOCK) + 31 >> 5
    for h in range(h_q):
        for i in range(call.nqb):
            qb, seg, a_blk, beta, nb_seg = call.row_block(i)
            iv, is_ = lists[h * n_seg + seg]
            assert (nb_seg + 31) >> 5 <= words_max
            g = is_[(is_ >= 0) & (is_ <= beta)]
            assert g.size == 0 or g.max() < nb_seg
            j = call.local_key_block(a_blk + beta - g)
            j = j[j >= 0]
            assert j.size == 0 or (j.min() >= 0 and j.max() < call.nkb)
            key_rows.append(j * BLOCK)
            key_rows.append(j * BLOCK + BLOCK - 1)
            vsel = prep_vertical(call, iv, seg)
            lim = (qb + 1) * BLOCK
            m = vsel[vsel < lim]
            bm = m // BLOCK - a_blk
            off = beta - bm
            assert off.size == 0 or (off.min() >= 0 and off.max() < nb_seg)
            covered = np.isin(off, is_)
            cols = call.local_key_pos(m[~covered])
            assert cols.size == 0 or (cols.min() >= 0 and cols.max() < call.n_k)
            key_rows.append(cols)
            # the column buffer never holds more than one batch plus a partial tile
            assert R * nt + 63 <= ncols
    key_rows = np.concatenate([np.atleast_1d(x) for x in key_rows if np.size(x)])
    check_dma_part(D, 2, row_bytes, call.n_k, key_rows)


def key_major_slash(call, lists, h_q, h_kv, n_seg):
    """Tiles of the slash dK/dV kernel for every (KV head, local key block):
    query blocks kb + g of the group's heads, the tile encoding and the list
    capacity (512 entries, appended 128 at a time, emptied above 384)."""
    G = h_q // h_kv
    starts = np.asarray(call.cu) // BLOCK
    j = np.arange(call.nkb)
    kb = call.global_key_block(j)
    assert np.array_equal(call.local_key_block(kb), j)
    if call.W == 1:
        seg = np.searchsorted(starts, j, side="right") - 1
        a_blk, nb_seg = starts[seg], starts[seg + 1] - starts[seg]
    else:
        seg = np.zeros_like(j)
        a_blk, nb_seg = np.zeros_like(j), np.full_like(j, call.n_global // BLOCK)
    beta_k = kb - a_blk
    assert beta_k.min() >= 0 and np.all(beta_k < nb_seg)
    i0 = call.local_query_block(kb)  # the diagonal tile (g = 0)
    assert np.all((i0 == -1) | ((i0 >= 0) & (i0 < call.nqb)))
    for kvh in range(h_kv):
        count = np.zeros(call.nkb, np.int64)
        for hh in range(G):
            assert hh < 32  # the head index sits in the tile word's top bits
            for s in range(n_seg):
                mine = seg == s
                _, is_ = lists[(kvh * G + hh) * n_seg + s]
                for base in range(0, is_.size, 128):
                    g = is_[base:base + 128]
                    ok = (g[None, :] > 0) & (beta_k[mine, None] + g[None, :] < nb_seg[mine, None])
                    i = call.local_query_block(kb[mine, None] + g[None, :])
                    i = np.where(ok, i, -1)
                    assert i.max(initial=-1) < min(call.nqb, 2 ** 25)
                    count[mine] += (i >= 0).sum(axis=1)
                    assert count.max(initial=0) <= 512
                    count[count > 512 - 128] = 0


def slash_parts(units, G, cus=256):
    """Workgroups per key block of the slash dK/dV kernel (mirrors the
    launcher): doubled while the grid is under two rounds of four resident
    workgroups per CU, up to 4, as long as the part count divides the group."""
    parts = 1
    while parts < 4 and units * parts < 2 * 4 * cus and G % (2 * parts) == 0:
        parts *= 2
    return parts


def slash_grid(batch, h_kv, nkb, G, n_k, D):
    """Decode of every workgroup of the slash dK/dV grid, as the kernel does:
    (batch, KV head) fastest, then the part, then the key block.  Every
    (batch, KV head, key block, head) is walked by exactly one workgroup, the
    head ranges stay inside the group, and the atomic epilogue's rows and
    channels (part count above one), the zero fill and the LDS staging stay
    inside dK / dV and the tile buffers."""
    parts = slash_parts(batch * h_kv * nkb, G)
    BH = batch * h_kv
    wg = np.arange(BH * nkb * parts)
    bh = wg % BH
    part = (wg // BH) % parts
    j = wg // BH // parts
    assert j.max() < nkb
    hpp = G // parts
    assert hpp * parts == G
    seen = np.zeros((BH, nkb, G), np.int64)
    for hh in range(hpp):
        np.add.at(seen, (bh, j, part * hpp + hh), 1)
    assert np.all(seen == 1)
    if parts > 1:
        # epilogue: rows j*64 + 32*kh + r (kh < 2, r < 32), channels 32*ct + l32
        b, kvh = bh // h_kv, bh % h_kv
        last_row = ((b * n_k + j * BLOCK + 32 + 31) * h_kv + kvh) * D + (D - 32) + 31
        assert last_row.max() < batch * n_k * h_kv * D
        assert (batch * n_k * h_kv * D) % 4 == 0  # the zero fill's 16-byte stores
        q_bytes = 32 * D * 2
        assert 2 * (2 * q_bytes + 3 * 32 * 4) >= 2 * 32 * 33 * 4
    return parts


@pytest.mark.parametrize("shape", [(1, 2, 512, 8), (1, 2, 256, 8), (1, 2, 2048, 8), (1, 1, 128, 8),
                                   (16, 1, 128, 8), (2, 2, 64, 8), (1, 1, 48, 3), (1, 1, 16, 32),
                                   (1, 4, 32, 1), (1, 2, 8192, 8)])
def test_slash_parts_grid(shape):
    """The split of a key block's heads over workgroups, at the benchmark
    shapes (N = 32768 and 131072, a striped chunk call of 16384 keys, the
    one-call worker) and the small test shapes."""
    batch, h_kv, nkb, G = shape
    for D in (64, 128):
        parts = slash_grid(batch, h_kv, nkb, G, nkb * BLOCK, D)
    want = {(1, 2, 512, 8): 2, (1, 2, 256, 8): 4, (1, 2, 2048, 8): 1, (16, 1, 128, 8): 1,
            (1, 2, 8192, 8): 1, (1, 1, 48, 3): 1}
    if shape in want:
        assert parts == want[shape]


def column_units(call, lists, h_q, n_seg, v_cap, cols_per_unit=128):
    """Column dK/dV units (128 columns each in the bf16 kernel, 64 in the
    fp32 one): columns of the prepared list, their local key positions and
    the query-block range."""
    col_tiles = (64 * ((v_cap + 63) // 64) + cols_per_unit - 1) // cols_per_unit
    qrange_len = 16 if (call.W > 1 and not call.k_all) else 48
    qranges = (call.nqb + qrange_len - 1) // qrange_len
    while qranges > 1 and qranges % 2 == 0:
        qrange_len += 1
        qranges = (call.nqb + qrange_len - 1) // qrange_len
    for h in range(h_q):
        for seg in range(n_seg):
            vsel = prep_vertical(call, lists[h * n_seg + seg][0], seg)
            assert vsel.size <= max(v_cap, 1)
            for ct in range(col_tiles):
                if cols_per_unit * ct >= vsel.size:
                    continue
                cols = vsel[cols_per_unit * ct: cols_per_unit * (ct + 1)]
                kpos = call.local_key_pos(cols)
                assert kpos.min() >= 0 and kpos.max() < call.n_k
                first_blk = int(cols[0] // BLOCK)
                if call.W == 1:
                    i_first = first_blk
                    i_lo, i_hi = call.cu[seg] // BLOCK, call.cu[seg + 1] // BLOCK
                else:
                    i_first = 0 if first_blk <= call.q_rank else (first_blk - call.q_rank + call.W - 1) // call.W
                    i_lo, i_hi = 0, call.nqb
                for qr in range(qranges):
                    r_lo = max(i_lo, qr * qrange_len, i_first)
                    r_hi = min(i_hi, (qr + 1) * qrange_len)
                    if r_lo < r_hi:
                        assert 0 <= r_lo and r_hi <= call.nqb


@pytest.mark.parametrize("mode", ["rank-chunks", "all-chunks"])
def test_striped_worker_shape_in_bounds(mode):
    """32 ranks, 64-token stripes, N = 524288, 16 Q / 2 KV heads, d = 128;
    worker 0 and a middle worker, against several chunks or all of them."""
    rng = np.random.default_rng(40)
    n, W, h_q, h_kv = 524288, 32, 16, 2
    cu = [0, n]
    lists = [random_index(rng, cu, 4096, 320)[0] for _ in range(h_q)]
    v_cap = max(l[0].size for l in lists)
    for w in (0, 17):
        calls = ([Call(n, cu, W, w, u) for u in (w, (w - 1) % W, (w + 16) % W)] if mode == "rank-chunks"
                 else [Call(n, cu, W, w, 0, k_all=True)])
        for call in calls:
            query_major_walk(call, lists, h_q, 1, 128, h_kv * 128 * 2)
            key_major_slash(call, lists, h_q, h_kv, 1)
            column_units(call, lists, h_q, 1, v_cap)
            column_units(call, lists, h_q, 1, v_cap, cols_per_unit=64)


def test_all_chunks_relabelling_is_a_bijection():
    """Local key block u * (nkb / W) + j <-> global block u + W * j."""
    call = Call(8192 * 64, [0, 8192 * 64], 32, 5, 0, k_all=True)
    j = np.arange(call.nkb)
    g = call.global_key_block(j)
    assert np.array_equal(np.sort(g), np.arange(call.nkb))
    assert np.array_equal(call.local_key_block(g), j)
    # chunk u holds the blocks of rank u, in order
    nc = call.nkb // call.W
    assert np.array_equal(g[3 * nc: 4 * nc] % call.W, np.full(nc, 3))


def test_packed_documents_in_bounds():
    rng = np.random.default_rng(41)
    n, h_q, h_kv = 262144, 16, 2
    cuts = np.sort(rng.choice(np.arange(1, n // BLOCK), size=7, replace=False)) * BLOCK
    cu = [0] + cuts.tolist() + [n]
    per = [random_index(rng, cu, 512 + 400 * h, 40 + 20 * h) for h in range(h_q)]
    lists = [per[h][s] for h in range(h_q) for s in range(len(cu) - 1)]
    v_cap = max(l[0].size for l in lists)
    call = Call(n, cu)
    query_major_walk(call, lists, h_q, len(cu) - 1, 128, h_kv * 128 * 2)
    key_major_slash(call, lists, h_q, h_kv, len(cu) - 1)
    column_units(call, lists, h_q, len(cu) - 1, v_cap)


def block_selection_walks(n, batch, h_q, h_kv, sel_p, rng):
    """Block-selection index (one segment, 128-token blocks, 64-token tiles):
    the bitmap words the query-major block phase and the slash dK/dV walk
    read, the tiles they form, and the dK/dV list capacity."""
    nb = n // BLOCK
    nI = -(-n // 128)
    words = (nI + 31) >> 5
    n_words = batch * h_q * nI * words
    sel = rng.random((batch * h_q, nI, nI)) < sel_p
    sel &= np.tril(np.ones((nI, nI), bool))[None]

    def bit(bh, I, J):
        w = (bh * nI + I) * words + (J >> 5)
        assert np.all((w >= 0) & (w < n_words))
        return sel[bh, I, J]

    beta = np.arange(nb)
    for bh in range(batch * h_q):
        # query-major: key blocks kb <= beta, NT = 128 per compaction round
        for b in range(nb):
            kb = np.arange(b + 1)
            on = bit(bh, b >> 1, kb >> 1)
            for base in range(0, b + 1, 128):
                assert on[base:base + 128].sum() <= 128  # the tiles[NT] array
            assert np.all(kb[on] < nb)
    G = h_q // h_kv
    for b in range(batch):
        for kvh in range(h_kv):
            count = np.zeros(nb, np.int64)
            for hh in range(G):
                bh = b * h_q + kvh * G + hh
                bit(bh, beta >> 1, beta >> 1)  # the diagonal walk
                nq = nb - 1 - beta
                for base in range(0, int(nq.max(initial=0)), 128):
                    e = base + np.arange(128)
                    ib = beta[:, None] + 1 + e[None, :]
                    live = e[None, :] < nq[:, None]
                    ibc = np.where(live, ib, 0)
                    on = live & bit(bh, ibc >> 1, (beta[:, None] >> 1) + 0 * ibc)
                    assert np.all(ib[on] < nb)
                    count += on.sum(axis=1)
                    assert count.max(initial=0) <= 512
                    count[count > 512 - 128] = 0


def query_major_pairs(n, batch, h_q, selected, word_index):
    """The paired query-major walk of block selections (four waves over query
    blocks 2I and 2I + 1): the grid of pairs, the rows each wave reads (an
    absent second block's waves read the first block's), the selection words
    read, the tiles of each compaction round (at most 256) and their word
    bits."""
    nqb = n // BLOCK
    npair = (nqb + 1) // 2
    for bh in range(batch * h_q):
        for ip in range(npair):
            i0 = 2 * ip
            last = min(i0 + 1, nqb - 1)
            for w in range(4):
                qh = w >> 1
                live = i0 + qh < nqb
                r = 32 * w + np.arange(32)
                rl = r if live else r - 64
                rows = i0 * BLOCK + rl
                assert rows.min() >= 0 and rows.max() < n
            for base in range(0, last + 1, 256):
                kb = base + np.arange(min(256, last + 1 - base))
                for x in kb:
                    word_index(bh, i0, int(x))
                on = np.array([bool(selected(bh, i0, int(x))) for x in kb])
                assert on.sum() <= 256
                tv = 4 * kb[on] + 3
                assert tv.max(initial=0) < 2 ** 31 and np.all(kb[on] * BLOCK + 63 < n)


def key_major_pairs(n, batch, h_q, h_kv, selected, word_index, rm_shift=None):
    """The paired dK/dV walk of block and per-row selections (workgroups of
    four waves owning key blocks 2 jp and 2 jp + 1): its grid, the key rows
    each wave loads, the selection words it reads (word_index(bh, ib, jp) ->
    flat index, checked by the caller's closure), the tiles of its diagonal
    and main walks (tile word bits, query rows staged) and the tile list
    capacity (512 entries, appended 256 at a time, emptied above 256)."""
    nb = n // BLOCK
    G = h_q // h_kv
    assert G <= 32 and (31 << 26) < 2 ** 31
    npair = (nb + 1) // 2
    for b in range(batch):
        for kvh in range(h_kv):
            for jp in range(npair):
                kb0 = 2 * jp
                for kp in (0, 1):
                    kbw = kb0 + kp
                    live = kbw < nb
                    kpos = (kbw if live else kb0) * BLOCK + np.arange(64)
                    assert kpos.max() < n
                    if rm_shift is not None and live:
                        assert (kbw >> rm_shift) < 32
                if rm_shift is not None:
                    assert ((kb0 + 1) >> rm_shift) < 32   # the picks mask, also for an absent block
                diag = 0
                for hh in range(G):
                    bh = b * h_q + kvh * G + hh
                    for ib in (kb0, kb0 + 1):
                        if ib < nb:
                            word_index(bh, ib, jp)
                            diag += bool(selected(bh, ib, jp))
                assert diag <= 2 * G <= 512
                count = 0
                ns = nb - kb0 - 2
                for hh in range(G):
                    bh = b * h_q + kvh * G + hh
                    for base in range(0, max(ns, 0), 256):
                        ib = kb0 + 2 + base + np.arange(min(256, ns - base))
                        for x in ib:
                            word_index(bh, int(x), jp)
                        on = np.array([bool(selected(bh, int(x), jp)) for x in ib])
                        assert np.all(ib[on] < nb) and np.all(ib[on] < 2 ** 25)
                        assert np.all(ib[on] * BLOCK + 63 < n)   # both 32-row halves staged
                        count += int(on.sum())
                        assert count <= 512
                        if count > 512 - 256:
                            count = 0


def xattn_estimator_addresses(n, batch, h_q, h_kv, d):
    """Cell and selection kernels: the (row tile, column tile) decode of the
    triangle index, every Q / K row and channel a direct load fetches, every
    LDS destination and operand read, every log-sum-exp written and read,
    every output word (stride 16, block 128, 128 x 128 cell tiles, stages of
    one sample offset and 64 channels)."""
    nC, nI = n // 16, -(-n // 128)
    words = (nI + 31) >> 5
    nt = -(-nC // 128)
    per_head = nt * (nt + 1) // 2
    stage_bytes = 128 * 128          # one operand of a stage: 128 rows x 64 channels bf16
    seen = set()
    for t in range(per_head):
        ta = int((np.sqrt(np.float32(8.0) * np.float32(t) + np.float32(1.0)) - np.float32(1.0)) * np.float32(0.5))
        while ta * (ta + 1) // 2 > t:
            ta -= 1
        while (ta + 1) * (ta + 2) // 2 <= t:
            ta += 1
        tc = t - ta * (ta + 1) // 2
        assert 0 <= tc <= ta < nt
        seen.add((ta, tc))
    assert len(seen) == per_head
    lane = np.arange(64)
    for A0 in {0, 128 * (nt - 1)}:
        for st in range(16 * d // 64):
            u, ch0 = st // (d // 64), 64 * (st % (d // 64))
            for w in range(4):
                for t0 in range(8):
                    tt = w * 8 + t0
                    row = 8 * (tt & 15) + lane // 8
                    chunk = (lane & 7) ^ ((row >> 1) & 7)
                    cell = np.minimum(A0 + row, nC - 1)
                    tok = 16 * cell + u if tt < 16 else 16 * cell + 15 - u
                    assert tok.min() >= 0 and tok.max() < n
                    assert ch0 + 8 * chunk.max() + 8 <= d
                    dst = 1024 * (tt & 15) + 16 * lane
                    assert dst.max() + 16 <= stage_bytes
                    # the LDS slot a lane fills holds the chunk the readers expect
                    r = dst // 128
                    slot = (dst % 128) // 16
                    assert np.array_equal(r, row) and np.array_equal(slot ^ ((r >> 1) & 7), chunk)
    # operand reads: rows < 128, chunk (2 ks + hl) ^ ((r / 2) % 8) inside a row
    r = np.arange(128)[:, None]
    c = np.arange(8)[None, :]
    off = r * 128 + 16 * (c ^ ((r >> 1) & 7))
    assert off.max() + 16 <= stage_bytes and len(np.unique(off)) == off.size
    # conflict-free: each 16-lane pass (16 consecutive rows, one chunk) hits 16 bank groups
    for r0 in range(0, 128, 16):
        for cc in range(8):
            rows = np.arange(r0, r0 + 16)
            groups = ((rows * 128 + 16 * (cc ^ ((rows >> 1) & 7))) // 16) % 16
            assert len(set(groups.tolist())) == 16
    # epilogue writes ((bh nI + J) nC + A) for A < nC, J < nI; the selection
    # reads (bh nI + J) nC + 8 I + a for J <= I, 8 I + a < nC
    cell = batch * h_q * nI * nC
    assert ((batch * h_q - 1) * nI + nI - 1) * nC + nC - 1 < cell
    for I in range(nI):
        assert I + 1 <= 1024 and words <= 1024 // 32
        na = min(8, nC - 8 * I)
        assert na >= 1 and 8 * I + na <= nC
    assert d % 64 == 0
    # (mass << 10 | 1023 - J) keys: mass <= 8.001 * 2^50 fits above 10 index bits
    assert (int(8.001 * 2 ** 50) << 10) < 2 ** 64


@pytest.mark.parametrize("n,batch,h_q,h_kv", [(1024, 1, 2, 1), (4160, 2, 4, 1), (8192, 1, 16, 2),
                                              (131072, 1, 2, 1)])
def test_block_selection_in_bounds(n, batch, h_q, h_kv):
    rng = np.random.default_rng(42 + n)
    if n <= 8192:
        block_selection_walks(n, batch, h_q, h_kv, 0.6, rng)
        nI = -(-n // 128)
        words = (nI + 31) >> 5
        sel = rng.random((batch * h_q, nI, nI)) < 0.6

        def word_index(bh, ib, jp):
            w = (bh * nI + (ib >> 1)) * words + (jp >> 5)
            assert 0 <= w < batch * h_q * nI * words
            return w

        key_major_pairs(n, batch, h_q, h_kv, lambda bh, ib, jp: sel[bh, ib >> 1, jp], word_index)
        query_major_pairs(n, batch, h_q, lambda bh, i0, kb: sel[bh, i0 >> 1, kb >> 1],
                          lambda bh, i0, kb: word_index(bh, i0, kb >> 1))
    for d in (64, 128):
        xattn_estimator_addresses(n, batch, h_q, h_kv, d)



@pytest.mark.parametrize("n,batch,h_q,h_kv,blk", [(4096, 2, 4, 1, 256), (4160, 1, 2, 1, 512),
                                                 (131072, 1, 16, 2, 4096), (2048, 1, 4, 1, 64),
                                                 (4032, 1, 4, 2, 128)])
def test_per_row_selection_in_bounds(n, batch, h_q, h_kv, blk):
    """MoBA gate and per-row selection walks: the gate's workgroups (256 rows
    inside one key block), the mean and score indices, the query-major walk's
    row words and tiles, the key-major walk's union words, staged row words
    and picked-block bit."""
    assert blk >= 64 and blk & (blk - 1) == 0 and n <= 32 * blk
    nB = -(-n // blk)
    nqb = n // BLOCK
    shift = int(np.log2(blk // BLOCK))
    if n <= 8192:
        rng = np.random.default_rng(7 + n)
        uni = rng.integers(0, 2 ** 32, size=(batch * h_q, nqb), dtype=np.uint64)

        def union_index(bh, ib, jp):
            u = bh * nqb + ib
            assert 0 <= u < batch * h_q * nqb
            return u

        def picked(bh, ib, jp):
            picks = (1 << ((2 * jp) >> shift)) | (1 << ((2 * jp + 1) >> shift))
            return int(uni[bh, ib]) & picks

        key_major_pairs(n, batch, h_q, h_kv, picked, union_index, rm_shift=shift)
    if blk < 256:
        return  # the gate needs blocks of 256 or more; the per-row index does not
    rows_words = batch * h_q * n
    # gate: workgroup of rows r0 .. r0 + 255 shares its own block
    for r0 in range(0, n, 256):
        rows = np.arange(r0, min(r0 + 256, n))
        assert np.all(rows // blk == r0 // blk)
        own = r0 // blk
        assert own < nB <= 32 and own * 128 <= 32 * 128      # the LDS block means
    for J in range(nB):
        r0, r1 = J * blk, min((J + 1) * blk, n)
        assert 0 <= r0 < r1 <= n
    assert (batch * h_q * n - 1) * nB + nB - 1 < batch * h_q * n * nB   # gate scores
    # query-major: 64 row words of query block i, tiles kb <= beta
    nqb = n // BLOCK
    shift = int(np.log2(blk // BLOCK))
    for bh in (0, batch * h_q - 1):
        for i in (0, nqb // 2, nqb - 1):
            idx = bh * n + i * BLOCK + np.arange(BLOCK)
            assert idx.max() < rows_words
            kb = np.arange(i + 1)
            assert np.all((kb >> shift) < 32) and np.all(4 * kb + 3 < 2 ** 31)
    # key-major: union word of (bh, query block), staged words of 32-row halves
    for bh in (0, batch * h_q - 1):
        for j in (0, nqb // 2, nqb - 1):
            ib = np.arange(j + 1, nqb)
            assert np.all(bh * nqb + ib < batch * h_q * nqb)
            pick = j >> shift
            assert pick < 32
            for i in ib[:3]:
                for half in (0, 1):
                    li = bh * n + i * BLOCK + 32 * half + np.arange(32)
                    assert li.max() < rows_words


def topk_two_stage(L, k, chunk=16384, cand=16384):
    """The top-k's choice for a list of L scores and k picks (mirrors the
    device): (chunks, chunk length) of the two-stage select, or None."""
    if k <= 0 or k >= L:
        return None
    n = -(-L // chunk)
    if n * k > cand:
        n = cand // k
    if n < 2:
        return None
    return n, -(-L // n)


@pytest.mark.parametrize("n,cu_frac", [(131072, None), (262144, "docs"), (524288, None), (40960, None)])
def test_topk_chunks_in_bounds(n, cu_frac):
    """The two-stage top-k: every list's chunks cover it exactly, fit the
    workspace's slots (the longest list's 16384-entry chunk count per list,
    16384 candidate pairs per slot) and their candidates fit the merge's LDS
    (16384); the workspace bytes match the host's sizing."""
    rng = np.random.default_rng(5 + n)
    if cu_frac == "docs":
        cuts = np.sort(rng.choice(np.arange(1, n // BLOCK), 7, replace=False)) * BLOCK
        cu = [0] + cuts.tolist() + [n]
    else:
        cu = [0, n]
    lens = np.diff(cu)
    nslots = -(-int(lens.max()) // 16384)
    h_q, batch = 16, 1
    n_lists = batch * h_q * len(lens)
    ws_pairs = n_lists * nslots * 16384 if nslots >= 2 else 0
    for L in lens:
        for k in (1, 2, 63, 64, 100, 1024, 2048, 2078, 4096, 8191, 8192, 8193, L - 1, L, L + 5):
            r = topk_two_stage(int(L), int(k))
            if r is None:
                continue
            nch, ch = r
            assert 2 <= nch <= nslots and nch * k <= 16384
            assert k < 16384                                  # a chunk's candidates fit its slot
            lens_c = [max(min(ch, L - c * ch), 0) for c in range(nch)]
            assert sum(lens_c) == L and min(lens_c) >= 0
            assert sum(min(k, x) for x in lens_c) <= 16384    # the merge's LDS
            for list_ in (0, n_lists - 1):
                for c in range(nch):
                    slot = (list_ * nslots + c) * 16384
                    assert slot + min(k, lens_c[c]) <= ws_pairs
