"""Host emulation of the launch geometry and per-thread memory ranges of the pack, unpack,
forward and backward kernels (semi_structured_sparsity_amd/csrc/nm_pack.hip, nm_forward.hip,
nm_backward.hpp), at the full LLaMA- and Nemotron-shaped sizes and at ragged shapes.

Each model below restates, in numpy, the index arithmetic of one kernel: which kernel the
launcher picks for a shape, the grid it launches, and for every thread the byte ranges it reads
and writes.  The checks prove, for the dispatch the library makes:
  * every byte of every output buffer is written by exactly one thread (no gaps, no overlap);
  * every read lies inside its input buffer.
No GPU is needed; a change to a kernel's indexing must be mirrored here.
"""
import itertools
import math

import numpy as np
import pytest

THREADS = 256
SUPPORTED = [(n, 4) for n in (1, 2, 3)] + [(n, 8) for n in range(1, 8)]


def K_of(n, m):
    return math.comb(m, n)


def bits_of(m):
    return (m - 1).bit_length()


def grid_for(threads):
    return (threads + THREADS - 1) // THREADS


class Buf:
    """Byte ranges [start, start + len) recorded against a buffer of `size` bytes."""

    def __init__(self, size):
        self.size = int(size)
        self.starts, self.lens = [], []

    def add(self, starts, lens):
        starts = np.asarray(starts, np.int64).reshape(-1)
        lens = np.broadcast_to(np.asarray(lens, np.int64), starts.shape).reshape(-1)
        keep = lens > 0
        self.starts.append(starts[keep])
        self.lens.append(lens[keep])

    def _cat(self):
        if not self.starts:
            return np.zeros(0, np.int64), np.zeros(0, np.int64)
        return np.concatenate(self.starts), np.concatenate(self.lens)

    def assert_in_bounds(self, what):
        s, l = self._cat()
        assert (s >= 0).all() and (s + l <= self.size).all(), f"{what}: read outside [0, {self.size})"

    def assert_written_once(self, what):
        s, l = self._cat()
        if self.size == 0:
            assert s.size == 0
            return
        order = np.argsort(s, kind="stable")
        s, l = s[order], l[order]
        assert s[0] == 0, f"{what}: bytes [0, {s[0]}) never written"
        gap = s[1:] != s[:-1] + l[:-1]
        assert not gap.any(), f"{what}: gap or overlap at byte {s[1:][gap][0]}"
        assert s[-1] + l[-1] == self.size, f"{what}: ends at {s[-1] + l[-1]}, size {self.size}"


# ---------------------------------------------------------------------------------------------
# dispatch (the launchers in nm_pack.hip)

def byte_path(n, m, gpr):
    return m == 4 and n in (1, 2) and (gpr * n * 2) % 32 == 0


def flat8(n, m, gpr):
    return m == 8 and (gpr * n * 3) % 32 == 0


def pack_kernel(n, m, gpr):
    if byte_path(n, m, gpr):
        return "k_pack_bytes"
    if flat8(n, m, gpr):
        return "k_pack_flat8"
    return "k_pack"


def unpack_kernel(n, m, gpr):
    if m == 4 and n == 1 and byte_path(n, m, gpr):
        return "k_unpack_1of4"
    if m == 4 and n == 2 and byte_path(n, m, gpr):
        return "k_unpack_bytes"
    if flat8(n, m, gpr):
        return "k_unpack_flat8"
    return "k_unpack"


def wpr_of(n, m, cols):
    return (cols // m * n * bits_of(m) + 31) // 32


def buffers(rows, cols, n, m, wb):
    gpr, K = cols // m, K_of(n, m)
    return dict(w=Buf(rows * cols * wb), logits=Buf(rows * gpr * K * 4), values=Buf(rows * gpr * n * wb),
                indices=Buf(rows * wpr_of(n, m, cols) * 4), hard=Buf(rows * gpr), dense=Buf(rows * cols * wb))


# ---------------------------------------------------------------------------------------------
# flat kernels: one tile per thread

def model_pack_bytes(b, rows, cols, n, wb):
    m, K = 4, K_of(n, 4)
    gpr = cols // m
    groups = rows * gpr
    U = 8 // (2 * n)
    t = np.arange(grid_for(groups // U) * THREADS, dtype=np.int64)
    g0 = t * U
    t, g0 = t[g0 < groups], g0[g0 < groups]
    blk, tid = t // THREADS, t % THREADS
    staged = (blk + 1) * THREADS * U <= groups
    per = U * K // 4
    for i in range(per):  # a staged block's logits: consecutive lanes on consecutive float4
        b["logits"].add((blk[staged] * THREADS * U * K) * 4 + (tid[staged] + i * THREADS) * 16, 16)
    b["logits"].add(g0[~staged] * K * 4, U * K * 4)
    b["w"].add(g0 * m * wb, U * m * wb)
    b["values"].add(g0 * n * wb, U * n * wb)
    b["indices"].add(t, 1)
    b["hard"].add(g0, U)


def model_unpack_bytes(b, rows, cols, wb):
    n, m, U = 2, 4, 2
    groups = rows * (cols // m)
    t = np.arange(grid_for(groups // U) * THREADS, dtype=np.int64)
    g0 = t * U
    t, g0 = t[g0 < groups], g0[g0 < groups]
    b["indices"].add(t, 1)
    b["values"].add(g0 * n * wb, U * n * wb)
    b["dense"].add(g0 * m * wb, U * m * wb)


def model_unpack_1of4(b, rows, cols, wb):
    m = 4
    groups = rows * (cols // m)
    G = 16 // (4 * wb)
    t = np.arange(grid_for(groups // G) * THREADS, dtype=np.int64)
    g0 = t * G
    t, g0 = t[g0 < groups], g0[g0 < groups]
    b["indices"].add(g0 >> 2, 1)
    b["values"].add(t * 4, 4)  # one uint32: the G kept values
    b["dense"].add(g0 * m * wb, 16)


def sample_tiling(n, m):
    """(K, P, PK, LALIGN, STAGE) of the sampling kernels (struct Sample in nm_layer.hpp)."""
    K = K_of(n, m)
    P = 1 if (K % 4 == 0 or K == 70) else (2 if K % 2 == 0 else 4)
    PK = P * K
    lalign = 16 if (PK * 4) % 16 == 0 else 8
    return K, P, PK, lalign, PK * 4 > lalign


def add_logit_span(buf, n, m, groups, blk, tid, g0, nvalid):
    """Logit (or logit-gradient) accesses of the sampling kernels: a staged block moves its span
    as consecutive vectors, other threads access their own nvalid groups directly."""
    K, P, PK, lalign, stage = sample_tiling(n, m)
    staged = ((blk + 1) * THREADS * P <= groups) if stage else np.zeros(blk.shape, bool)
    for i in range(PK * 4 // lalign):
        buf.add(blk[staged] * THREADS * PK * 4 + (tid[staged] + i * THREADS) * lalign, lalign)
    buf.add(g0[~staged] * K * 4, nvalid[~staged] * K * 4)


def model_pack_flat8(b, rows, cols, n, wb):
    m = 8
    gpr, K = cols // m, K_of(n, m)
    groups = rows * gpr
    t = np.arange(grid_for(groups) * THREADS, dtype=np.int64)
    blk, tid, lane = t // THREADS, t % THREADS, t % 64
    full = t < groups
    add_logit_span(b["logits"], n, m, groups, blk, tid, t, full.astype(np.int64))
    g = t[full]
    b["w"].add(g * m * wb, m * wb)
    b["values"].add(g * n * wb, n * wb)
    b["hard"].add(g, 1)
    gw0 = (t - lane)[lane == 0]  # each wave stores its groups' whole index words
    gw0 = gw0[gw0 < groups]
    ngw = np.minimum(groups - gw0, 64)
    nwords = (ngw * n * 3 + 31) // 32
    for i in range(int(nwords.max(initial=0))):
        sel = i < nwords
        b["indices"].add((gw0[sel] * n * 3 // 32 + i) * 4, 4)


def model_unpack_flat8(b, rows, cols, n, wb):
    m = 8
    groups = rows * (cols // m)
    g0 = np.arange(grid_for(groups) * THREADS, dtype=np.int64)
    g0 = g0[g0 < groups]
    b["values"].add(g0 * n * wb, n * wb)
    lb = g0 * n * 3
    b["indices"].add(lb // 32 * 4, 4)
    two = (lb % 32) + n * 3 > 32
    b["indices"].add((lb[two] // 32 + 1) * 4, 4)
    b["dense"].add(g0 * m * wb, m * wb)


# ---------------------------------------------------------------------------------------------
# general tile kernels: grid (tiles per row, min(rows, 65535)), rows looped over grid y

def tile_shape(n, m, wb):
    GT = 1 if m * wb >= 16 else 16 // (m * wb)
    return GT, THREADS * GT


def _tile_threads(rows, gpr, GT, TILE):
    """(r, q_begin, tid, lq, mine, wave's ngw) for every row, tile and thread of the grid."""
    tiles = (gpr + TILE - 1) // TILE
    r, x, tid = np.meshgrid(np.arange(rows, dtype=np.int64), np.arange(tiles, dtype=np.int64),
                            np.arange(THREADS, dtype=np.int64), indexing="ij")
    r, x, tid = r.reshape(-1), x.reshape(-1), tid.reshape(-1)
    q_begin = x * TILE
    ng = np.minimum(gpr - q_begin, TILE)
    lq = tid * GT
    mine = np.clip(ng - lq, 0, GT)
    wq = (tid // 64) * 64 * GT
    ngw = np.clip(ng - wq, 0, 64 * GT)
    return r, q_begin, tid, lq, mine, wq, ngw


def model_pack_general(b, rows, cols, n, m, wb):
    gpr, K, BITS = cols // m, K_of(n, m), bits_of(m)
    GT, TILE = tile_shape(n, m, wb)
    wpr = wpr_of(n, m, cols)
    r, q_begin, tid, lq, mine, wq, ngw = _tile_threads(rows, gpr, GT, TILE)
    live = ngw > 0  # a wave with no groups returns before the row loop
    r, q_begin, tid, lq, mine, wq, ngw = (a[live] for a in (r, q_begin, tid, lq, mine, wq, ngw))
    g0 = r * gpr + q_begin + lq
    b["logits"].add(g0 * K * 4, mine * K * 4)
    b["w"].add(g0 * m * wb, mine * m * wb)
    b["values"].add(g0 * n * wb, mine * n * wb)
    b["hard"].add(g0, mine)
    lane = tid % 64
    nwords = (ngw * n * BITS + 31) // 32
    base = r * wpr + (q_begin + wq) * n * BITS // 32
    for i in range(int(nwords.max(initial=0)) // 64 + 1):
        word = lane + 64 * i
        sel = word < nwords
        b["indices"].add((base[sel] + word[sel]) * 4, 4)


def model_unpack_general(b, rows, cols, n, m, wb):
    gpr, BITS = cols // m, bits_of(m)
    GT, TILE = tile_shape(n, m, wb)
    wpr = wpr_of(n, m, cols)
    r, q_begin, tid, lq, mine, wq, ngw = _tile_threads(rows, gpr, GT, TILE)
    live = mine > 0
    r, q_begin, lq, mine = r[live], q_begin[live], lq[live], mine[live]
    g0 = r * gpr + q_begin + lq
    b["values"].add(g0 * n * wb, mine * n * wb)
    lb = (q_begin + lq) * n * BITS
    first = r * wpr + lb // 32
    b["indices"].add(first * 4, 4)
    two = (lb % 32) + mine * n * BITS > 32
    assert ((lb[two] // 32 + 1) < wpr).all(), "second index word past the row"
    b["indices"].add((first[two] + 1) * 4, 4)
    b["dense"].add(g0 * m * wb, mine * m * wb)


# ---------------------------------------------------------------------------------------------
# forward / backward: P groups per thread on a flat grid

def thread_slot(tid, n, m):
    """The thread's place in its block (thread_group in nm_layer.hpp): for K = 70 the waves of a
    block take groups of one parity, waves 0-1 the even ones and waves 2-3 the odd ones."""
    K, P, PK, lalign, stage = sample_tiling(n, m)
    if (P * K) % 4 == 0:
        return tid
    return 2 * ((tid & 63) + 64 * ((tid >> 6) & 1)) + (tid >> 7)


def model_forward_backward(rows, cols, n, m, wb):
    gpr = cols // m
    groups = rows * gpr
    K, P, PK, lalign, stage = sample_tiling(n, m)
    t = np.arange(grid_for((groups + P - 1) // P) * THREADS, dtype=np.int64)
    blk, tid = t // THREADS, t % THREADS
    q = thread_slot(tid, n, m)
    g0 = (blk * THREADS + q) * P
    live = g0 < groups
    blk, tid, g0 = blk[live], q[live], g0[live]
    if (P * K) % 4 != 0:  # every wave's groups share a parity, so the noise phase is wave-uniform
        wave = (blk * THREADS + t[live] % THREADS) // 64
        par = g0 % 2
        assert all(len(set(par[wave == wv])) == 1 for wv in np.unique(wave)[:512])
    nvalid = np.minimum(groups - g0, P)
    fwd = dict(w=Buf(rows * cols * wb), logits=Buf(groups * K * 4), out=Buf(rows * cols * wb))
    bwd = dict(w=Buf(rows * cols * wb), grad=Buf(rows * cols * wb), logits=Buf(groups * K * 4),
               dlogits=Buf(groups * K * 4))
    for d in (fwd, bwd):
        add_logit_span(d["logits"], n, m, groups, blk, tid, g0, nvalid)
        d["w"].add(g0 * m * wb, nvalid * m * wb)
    fwd["out"].add(g0 * m * wb, nvalid * m * wb)
    bwd["grad"].add(g0 * m * wb, nvalid * m * wb)
    add_logit_span(bwd["dlogits"], n, m, groups, blk, tid, g0, nvalid)
    return fwd, bwd


# ---------------------------------------------------------------------------------------------

def run_pack_unpack(rows, cols, n, m, wb):
    gpr = cols // m
    b = buffers(rows, cols, n, m, wb)
    pk, uk = pack_kernel(n, m, gpr), unpack_kernel(n, m, gpr)
    if pk == "k_pack_bytes":
        model_pack_bytes(b, rows, cols, n, wb)
    elif pk == "k_pack_flat8":
        model_pack_flat8(b, rows, cols, n, wb)
    else:
        model_pack_general(b, rows, cols, n, m, wb)
    for k in ("values", "indices", "hard"):
        b[k].assert_written_once(f"{pk} {k}")
    for k in ("w", "logits"):
        b[k].assert_in_bounds(f"{pk} {k}")
    u = buffers(rows, cols, n, m, wb)
    if uk == "k_unpack_bytes":
        model_unpack_bytes(u, rows, cols, wb)
    elif uk == "k_unpack_1of4":
        model_unpack_1of4(u, rows, cols, wb)
    elif uk == "k_unpack_flat8":
        model_unpack_flat8(u, rows, cols, n, wb)
    else:
        model_unpack_general(u, rows, cols, n, m, wb)
    u["dense"].assert_written_once(f"{uk} dense")
    for k in ("values", "indices"):
        u[k].assert_in_bounds(f"{uk} {k}")
    return pk, uk


FULL = [(6144, 6144, 2, 4, 2), (4096, 4096, 2, 4, 2), (11008, 4096, 2, 4, 2), (4096, 11008, 2, 4, 2),
        (24576, 6144, 2, 4, 2), (256, 256, 2, 4, 4), (4096, 11008, 1, 4, 2), (4096, 11008, 2, 8, 2),
        (4096, 11008, 4, 8, 2)]


@pytest.mark.parametrize("rows,cols,n,m,wb", FULL)
def test_full_size_pack_unpack_index_maps(rows, cols, n, m, wb):
    pk, uk = run_pack_unpack(rows, cols, n, m, wb)
    if (rows, cols, n, m) in ((6144, 6144, 2, 4), (4096, 4096, 2, 4)):
        assert (pk, uk) == ("k_pack_bytes", "k_unpack_bytes")


RAGGED_COLS = {4: [4, 12, 20, 28, 36, 44, 64, 132, 1028], 8: [8, 24, 40, 88, 136, 264, 1032]}


@pytest.mark.parametrize("n,m", SUPPORTED)
@pytest.mark.parametrize("wb", [2, 4])
def test_ragged_pack_unpack_index_maps(n, m, wb):
    kinds = set()
    for rows, cols in itertools.product([1, 3, 7], RAGGED_COLS[m]):
        kinds.add(run_pack_unpack(rows, cols, n, m, wb))
    assert kinds  # every shape dispatched and checked


@pytest.mark.parametrize("rows,cols,n,m,wb", FULL[:2] + [(3, 20, 2, 4, 2), (5, 24, 3, 8, 4), (7, 88, 4, 8, 2),
                                                          (1, 12, 1, 4, 4), (3, 36, 3, 4, 2), (4096, 11008, 4, 8, 2),
                                                          (37, 184, 4, 8, 2)])
def test_forward_backward_index_maps(rows, cols, n, m, wb):
    fwd, bwd = model_forward_backward(rows, cols, n, m, wb)
    fwd["out"].assert_written_once("k_forward out")
    bwd["dlogits"].assert_written_once("k_backward dlogits")
    for d, name in ((fwd, "k_forward"), (bwd, "k_backward")):
        for k, buf in d.items():
            if k not in ("out", "dlogits"):
                buf.assert_in_bounds(f"{name} {k}")


def test_model_catches_a_read_past_the_end():
    """The general pack's element path once read GT*M weights for a thread owning fewer groups:
    at an odd number of groups of four bf16 weights per row that passes the end of w on the last
    row.  The emulation flags such a read."""
    rows, cols, n, m, wb = 3, 20, 2, 4, 2
    gpr = cols // m
    GT, TILE = tile_shape(n, m, wb)
    r, q_begin, tid, lq, mine, wq, ngw = _tile_threads(rows, gpr, GT, TILE)
    live = mine > 0
    g0 = r[live] * gpr + q_begin[live] + lq[live]
    w = Buf(rows * cols * wb)
    w.add(g0 * m * wb, GT * m * wb)  # the old read: GT*M elements whatever `mine` is
    with pytest.raises(AssertionError):
        w.assert_in_bounds("old k_pack w")


def model_prior(rows, cols, n, m, wb):
    """k_prior (nm_forward.hip): a thread reads its P groups' weights and writes their prior
    indices; each block writes its kThreads*P groups' logits as consecutive 16-byte vectors,
    thread t taking vectors t, t + kThreads, ..., then the floats past the last whole vector one
    by one.  Each vector's two groups come from the thread's running (group, remainder) pair,
    which is checked against the division it replaces."""
    K, P = sample_tiling(n, m)[:2]
    groups = rows * (cols // m)
    b = dict(w=Buf(rows * cols * wb), logits=Buf(groups * K * 4), idx=Buf(groups))
    nblocks = grid_for(-(-groups // P))
    t = np.arange(nblocks * THREADS, dtype=np.int64)
    g0 = t * P
    live = g0 < groups
    nvalid = np.minimum(groups - g0[live], P)
    b["w"].add(g0[live] * m * wb, nvalid * m * wb)
    for p in range(P):
        sel = p < nvalid
        b["idx"].add(g0[live][sel] + p, 1)
    bg0 = np.arange(nblocks, dtype=np.int64) * THREADS * P
    ng = np.minimum(groups - bg0, THREADS * P)
    nf = ng * K
    nv = nf // 4
    step, sq, sr = 4 * THREADS, (4 * THREADS) // K, (4 * THREADS) % K
    for tid in range(THREADS):
        f = 4 * tid
        qa, ra = f // K, f - (f // K) * K
        for v in range(tid, int(nv.max(initial=0)), THREADS):
            assert qa == f // K and ra == f % K
            sel = v < nv
            qb = qa + (1 if ra + 3 >= K else 0)
            assert (ng[sel] > qb).all()  # the ks entries read exist
            b["logits"].add(bg0[sel] * K * 4 + 16 * v, 16)
            f, qa, ra = f + step, qa + sq, ra + sr
            if ra >= K:
                ra, qa = ra - K, qa + 1
        for x in range(tid, 4, THREADS):  # at most three tail floats per block
            sel = 4 * nv + x < nf
            b["logits"].add((bg0[sel] * K + 4 * nv[sel] + x) * 4, 4)
    return b


@pytest.mark.parametrize("n,m", SUPPORTED)
@pytest.mark.parametrize("rows,cols_groups", [(1, 1), (3, 5), (37, 23), (2, 129), (512, 384)])
def test_prior_index_maps(n, m, rows, cols_groups):
    b = model_prior(rows, cols_groups * m, n, m, 2)
    b["logits"].assert_written_once("k_prior logits")
    b["idx"].assert_written_once("k_prior idx")
    b["w"].assert_in_bounds("k_prior w")


# ---------------------------------------------------------------------------------------------
# The monitored forward's in-launch sums (k_forward_monitor and monitor_sums in nm_forward.hip;
# workspace layout monitor_layout): blocks finish in any order; each adds (1 << 57) + its sum to
# its parent's word of a 64-ary tree (node i of a level of c nodes under parent i % ceil(c/64))
# with one fetch-and-add, and the add that completes a node
# carries the node's sum one level up and sets the word back to zero.  The model replays the
# protocol with arbitrary finishing orders (each fetch-and-add is one step, as the hardware
# orders the updates of one word), and checks that each sum reaches the root exactly once, that
# no word overflows into its arrival count, that every index stays inside the tree, and that
# every word is left at zero.

ONE = 1 << 57


def monitor_layout(n, m, groups):
    """(blocks of the launch, nodes per tree level, words, bytes, F)."""
    P = sample_tiling(n, m)[1]
    blocks = grid_for(-(-groups // P))
    levels, below = [], blocks
    while below > 1:
        below = -(-below // 64)
        levels.append(below)
    words = 2 * sum(levels)
    frac = 56 - int(groups).bit_length()
    return blocks, levels, words, 8 * max(words, 2), frac


def run_monitor_protocol(blocks, levels, tree, order, contrib):
    """contrib[b] = (p, l) integer sums of block b; returns the (p, l) totals written."""
    written = [[], []]
    for b in order:
        vals, carry = list(contrib[b]), [True, True]
        node, below, base = b, blocks, 0
        for nodes in levels:
            parent = node % nodes
            expect = -(-(below - parent) // nodes)
            assert 1 <= expect <= 64
            for q in range(2):
                if not carry[q]:
                    continue
                i = base + 2 * parent + q
                assert 0 <= i < len(tree)
                old = tree[i]
                tree[i] = old + (ONE | vals[q])
                assert tree[i] < 1 << 64 and (tree[i] & (ONE - 1)) < ONE
                carry[q] = (old >> 57) + 1 == expect
                if carry[q]:
                    vals[q] += old & (ONE - 1)
                    tree[i] = 0
            base += 2 * nodes
            node, below = parent, nodes
        for q in range(2):
            if carry[q]:
                written[q].append(vals[q])
    return written


@pytest.mark.parametrize("n,m,rows,cols", [(2, 4, 16, 16), (2, 4, 1000, 4096), (1, 4, 4100, 16384),
                                           (4, 8, 11008, 4096), (2, 4, 24576, 6144), (3, 8, 37, 23 * 8)])
def test_monitor_sums_protocol(n, m, rows, cols):
    groups = rows * cols // m
    blocks, levels, words, size, frac = monitor_layout(n, m, groups)
    assert groups * 2 ** frac < 2 ** 56 and frac >= 16
    rng = np.random.default_rng(blocks)
    per_block = THREADS * sample_tiling(n, m)[1]
    # the largest sums a block can hold: every p_max 1 (rounded up by 1/2), every l1 2n
    contrib = [(g * 2 ** frac + 1, g * 2 * n) for g in
               (min(per_block, groups - b * per_block) for b in range(blocks))]
    assert sum(c[0] for c in contrib) < 2 ** 57
    want = (sum(c[0] for c in contrib), sum(c[1] for c in contrib))
    tree = [0] * words
    for trial in range(3):  # three calls in a row on one workspace: each leaves it zero
        order = rng.permutation(blocks) if trial != 2 else np.arange(blocks)[::-1]
        written = run_monitor_protocol(blocks, levels, tree, order, contrib)
        assert written == [[want[0]], [want[1]]]
        assert not any(tree)
