"""Host replica of the 256x256-tile GEMM's address generation (CPU only).

The index formulas of transformer_block_norm0_amd/csrc/rm_gemm256.hip are
restated here in NumPy: the persistent, XCD-aware tile schedule (which tiles
each workgroup takes), tile_of, the per-lane slab offsets of both operand
layouts (K-major rows with the (row/2)%8 chunk swizzle, M/N-major k-rows with
the 4*(k%4) swizzle), the per-slab offset, the bias copy, the residual loads
and the epilogue stores.  For every 16-bit GEMM of the block that the kernel
takes, over a grid of shapes inside the envelope of page 1 ("Public checks and
instructor coverage"), the test checks that

  * every tile of every token is visited exactly once by the schedule;
  * every 16-byte copy reads 8 valid elements of the token's operand (clamped
    rows or columns are valid ones), and lies inside the buffer resource the
    kernel builds for that operand, so the range check never zeroes data;
  * each slab's copies fill each LDS stage exactly once, and the fragment
    reads find there the element the swizzle says;
  * the bias copy, the residual loads and the epilogue stores stay inside
    their tensors, and the stores write every element of C exactly once.

The forward and backward GEMM arguments are those the library passes
(page 1, "Exact computation": one GEMM per token t, activations [B,T,.]
row-major with the token stride between rows)."""
from __future__ import annotations

import itertools

import numpy as np
import pytest

BM = BN = 256
BK = 64
CUS = 256   # MI355X compute units


def gemms_of_block(B, T, D, k):
    """The six GEMMs of one forward+backward with the library's operand layouts.

    Returns name -> dict(M, N, K, batch, a_kmajor, b_kmajor, A, a_bs, a_ld, B, b_bs, b_ld,
    C, c_bs, c_ld, bias, bias_bs, res, res_bs, res_ld) with tensors named by what they
    hold; tensor sizes in elements are in the second return value."""
    H = k * D
    N = B * T
    sizes = {"h1": N * D, "Z": N * 2 * H, "hid": N * H, "r2": N * D, "do2": N * D, "dhid": N * H,
             "dZ": N * 2 * H, "dh1": N * D, "w1": T * D * 2 * H, "b1": T * 2 * H, "wout": T * H * D,
             "bout": T * D, "dw1": T * D * 2 * H, "dwout": T * H * D}
    g = {}
    g["up"] = dict(M=B, N=2 * H, K=D, a_kmajor=True, b_kmajor=False, A="h1", a_bs=D, a_ld=T * D,
                   B="w1", b_bs=D * 2 * H, b_ld=2 * H, C="Z", c_bs=2 * H, c_ld=T * 2 * H,
                   bias="b1", bias_bs=2 * H, res=None)
    g["down"] = dict(M=B, N=D, K=H, a_kmajor=True, b_kmajor=False, A="hid", a_bs=H, a_ld=T * H,
                     B="wout", b_bs=H * D, b_ld=D, C="r2", c_bs=D, c_ld=T * D,
                     bias="bout", bias_bs=D, res="h1", res_bs=D, res_ld=T * D)
    g["dhid"] = dict(M=B, N=H, K=D, a_kmajor=True, b_kmajor=True, A="do2", a_bs=D, a_ld=T * D,
                     B="wout", b_bs=H * D, b_ld=D, C="dhid", c_bs=H, c_ld=T * H, bias=None, res=None)
    g["dwout"] = dict(M=H, N=D, K=B, a_kmajor=False, b_kmajor=False, A="hid", a_bs=H, a_ld=T * H,
                      B="do2", b_bs=D, b_ld=T * D, C="dwout", c_bs=H * D, c_ld=D, bias=None, res=None)
    g["dw1"] = dict(M=D, N=2 * H, K=B, a_kmajor=False, b_kmajor=False, A="h1", a_bs=D, a_ld=T * D,
                    B="dZ", b_bs=2 * H, b_ld=T * 2 * H, C="dw1", c_bs=D * 2 * H, c_ld=2 * H,
                    bias=None, res=None)
    g["dh1"] = dict(M=B, N=D, K=2 * H, a_kmajor=True, b_kmajor=True, A="dZ", a_bs=2 * H, a_ld=T * 2 * H,
                    B="w1", b_bs=D * 2 * H, b_ld=2 * H, C="dh1", c_bs=D, c_ld=T * D,
                    bias=None, res="do2", res_bs=D, res_ld=T * D)
    for v in g.values():
        v["batch"] = T
    return g, sizes


def supported(g):
    """The kernel's eligibility test for 16-bit operands and output (all base pointers 256-byte
    aligned, as the workspace regions and tensor allocations are)."""
    M, N, K = g["M"], g["N"], g["K"]
    if K % (2 * BK) or K < 4 * BK:
        return False
    a_cont = K if g["a_kmajor"] else M
    b_cont = K if g["b_kmajor"] else N
    if a_cont % 8 or b_cont % 8 or g["a_ld"] % 8 or g["b_ld"] % 8 or g["a_bs"] % 8 or g["b_bs"] % 8:
        return False
    if (not g["a_kmajor"] and M < 8) or (not g["b_kmajor"] and N < 8):
        return False
    a_rows = M if g["a_kmajor"] else K
    b_rows = N if g["b_kmajor"] else K
    if a_rows * g["a_ld"] * 2 > 0xFFFFFFFF or b_rows * g["b_ld"] * 2 > 0xFFFFFFFF:
        return False
    if N % 8 or g["c_ld"] % 4 or g["c_bs"] % 4:
        return False
    if g["bias"] and g["bias_bs"] % 8:
        return False
    if g["res"] and (g["res_ld"] % 4 or g["res_bs"] % 4):
        return False
    if M * g["c_ld"] * 2 > 0x7FFFFFFF:
        return False
    if g["res"] and M * g["res_ld"] * 2 > 0x7FFFFFFF:
        return False
    return True


def schedule(M, N, batch):
    """Logical tiles each workgroup takes, in order: list of arrays."""
    tiles_m, tiles_n = -(-M // BM), -(-N // BN)
    total = tiles_m * tiles_n * batch
    grid = max(8, CUS & ~7)
    grid = min(grid, (total + 7) & ~7)
    nslots = grid >> 3
    q, rem = total >> 3, total & 7
    out = []
    for blk in range(grid):
        xcd, slot = blk & 7, blk >> 3
        lo = xcd * q + min(xcd, rem)
        hi = lo + q + (1 if xcd < rem else 0)
        out.append(np.arange(lo + slot, hi, nslots))
    return out, tiles_m, tiles_n


def tile_of(logical, tiles_m, per_t):
    t = logical // per_t
    in_t = logical - t * per_t
    tn = in_t // tiles_m
    return t, (in_t - tn * tiles_m) * BM, tn * BN


def operand_extent(kmajor, ld, K, MN):
    return ((MN - 1) * ld + K) * 2 if kmajor else ((K - 1) * ld + MN) * 2


def slab_offsets(kmajor, ld, mn0, MN):
    """Per (wave, i, lane): byte offset, element row/col of the piece, and its LDS byte address
    within the stage, for the slab at k0 = 0.  Arrays of shape [4, 8, 64]."""
    wave, i, lane = np.meshgrid(np.arange(4), np.arange(8), np.arange(64), indexing="ij")
    if kmajor:
        row = 64 * wave + 8 * i + (lane >> 3)
        chunk = (lane & 7) ^ ((row >> 1) & 7)
        mn = np.minimum(mn0 + row, MN - 1)
        off = (mn * ld + chunk * 8) * 2
        lds = (64 * wave + 8 * i) * 128 + 16 * lane
        return off, mn, chunk * 8, lds, row      # row: tile row of the piece (k within slab = chunk*8..)
    krow = 16 * wave + 2 * i + (lane >> 5)
    chunk = (lane & 31) ^ ((krow & 3) << 2)
    mn = np.minimum(mn0 + chunk * 8, MN - 8)
    off = (krow * ld + mn) * 2
    lds = (16 * wave + 2 * i) * 512 + 16 * lane
    return off, mn, krow, lds, chunk


def kswz(row, chunk):
    return row * 128 + ((chunk ^ ((row >> 1) & 7)) << 4)


def mswz(krow, chunk):
    return krow * 512 + ((chunk ^ ((krow & 3) << 2)) << 4)


def check_operand(kmajor, ld, bs, K, MN, mn0, batch, total_elems):
    ext = operand_extent(kmajor, ld, K, MN)
    # the resource of the last token stays inside the tensor
    assert (batch - 1) * bs * 2 + ext <= total_elems * 2
    off, mn, sub, lds, slot = slab_offsets(kmajor, ld, mn0, MN)
    nk = K // BK
    # every LDS byte of the 32 KB stage is written exactly once per slab (A: 2 stages, B: 3 stages,
    # 160 KB in all)
    assert np.array_equal(np.sort(lds.ravel()), np.arange(0, 256 * BK * 2, 16))
    if kmajor:
        # LDS slot holds row `slot` (tile-local), logical chunk sub/8; the fragment read of
        # that (row, chunk) addresses the same slot
        assert np.array_equal(kswz(slot, sub // 8), lds)
        assert np.all(mn < MN) and np.all(mn >= 0)
    else:
        assert np.array_equal(mswz(sub, slot), lds)
        assert np.all(mn >= 0) and np.all(mn + 7 < MN)
    for ks in (0, nk - 1):
        k0 = ks * BK
        koff = k0 * 2 if kmajor else k0 * ld * 2
        byte = off + koff
        assert np.all(byte >= 0) and np.all(byte + 16 <= ext), "copy outside the operand resource"
        assert np.all(byte + 16 <= 0xFFFFFFFF)
        if kmajor:
            assert np.all(k0 + sub + 7 < K)
        else:
            assert np.all(k0 + sub < K)


def check_epilogue(g, m0, n0, written, sizes):
    M, N = g["M"], g["N"]
    lane = np.arange(64)
    r, h = lane & 31, lane >> 5
    c_ext = min(M * g["c_ld"] * 2, 0x7FFFFFFF)
    for wave in range(4):
        wm, wn = wave >> 1, wave & 1
        mb = m0 + wm * 128 + r
        # staged through LDS (check_output_staging): store s of block i holds, in lane l,
        # row 32i + 4s + l/16 and columns 8(l%16) .. + 7 of the wave's 128
        stores = [(m0 + wm * 128 + 32 * i + 4 * s8 + (lane >> 4), n0 + wn * 128 + 8 * (lane & 15))
                  for i in range(4) for s8 in range(8)]
        assert len(stores) == 32      # EPI_STORES, every one issued
        for m, ns in stores:
            ok = (m < M) & (ns < N)
            co = m * g["c_ld"] * 2 + ns * 2
            assert np.all(co[ok] + 16 <= c_ext)
            np.add.at(written, (m[ok][:, None], ns[ok][:, None] + np.arange(8)), 1)
        if g["res"]:
            check_residual_copy(g, m0, n0, wm, wn)
    if g["bias"]:
        # the bias fragment: lane l < 32 reads the one value at column n0 + wn*128 + 32j + l
        for wn in range(2):
            for j in range(4):
                n = n0 + wn * 128 + 32 * j + lane
                ok = (lane < 32) & (n < N)
                assert np.all(n[ok] * 2 + 2 <= N * 2)


OUT_OF_RANGE = 0x80000000


def check_output_staging(read_swizzle=15):
    """The LDS pass of the epilogue without a residual, for one wave's 32 x 128 block: lane l
    writes the 4 columns 32j + 8q + 4h .. + 3 of row l%32 (h = l/32) at byte
    r*256 + 16((4j + q) ^ (r % 16)) + 8h, then reads 16 bytes of row 4s + l/16 at logical chunk
    l%16; every read must return the 8 columns 8(l%16) .. + 7 of that row, in order."""
    lane = np.arange(64)
    r, h = lane & 31, lane >> 5
    region = {}
    for j, q in itertools.product(range(4), range(4)):
        addr = r * 256 + (((4 * j + q) ^ (r & 15)) << 4) + 8 * h
        assert np.all(addr + 8 <= 8192)
        for l_ in range(64):
            for e in range(4):
                pos = int(addr[l_]) + 2 * e
                assert pos not in region, "two lanes write one element"
                region[pos] = (int(r[l_]), 32 * j + 8 * q + 4 * int(h[l_]) + e)
    assert len(region) == 32 * 128
    rr0, ch = lane >> 4, lane & 15
    for s8 in range(8):
        rr = 4 * s8 + rr0
        addr = rr * 256 + ((ch ^ (rr & read_swizzle)) << 4)
        for l_ in range(64):
            got = [region[int(addr[l_]) + 2 * e] for e in range(8)]
            assert got == [(int(rr[l_]), 8 * int(ch[l_]) + e) for e in range(8)], (s8, l_, got)


def check_residual_copy(g, m0, n0, wm, wn, read_swizzle=15):
    """The residual's way through LDS for one wave: the copies' source offsets (res_offsets,
    res_piece) stay inside the token's residual or read zero (rows past M lie beyond the
    extent, columns past N get OUT_OF_RANGE), and the epilogue's reads (lane l: row l%32 of
    block i, 8 bytes h = l/32 of logical chunk 4j + q) find exactly the elements of the rows
    and columns the accumulators hold."""
    M, N, rld = g["M"], g["N"], g["res_ld"] * 2
    r_ext = min(M * rld, 0x7FFFFFFF)
    lane = np.arange(64)
    # the kernel keeps the offsets of pieces 0..3 (res_offsets); piece p + 4 is 16 rows on
    row4 = np.array([4 * p + (lane >> 4) for p in range(4)])          # [piece, lane]
    lc4 = (lane & 15) ^ (row4 & 15)
    off4 = np.where(n0 + wn * 128 + 8 * lc4 < N, (m0 + wm * 128 + row4) * rld + (n0 + wn * 128 + 8 * lc4) * 2,
                    OUT_OF_RANGE)
    row = np.concatenate([row4, row4 + 16])
    lc = np.concatenate([lc4, lc4])
    m = m0 + wm * 128 + row
    n = n0 + wn * 128 + 8 * lc
    for blk in range(4):
        o = np.array([np.where(off4[p & 3] == OUT_OF_RANGE, OUT_OF_RANGE,
                               off4[p & 3] + blk * 32 * rld + (16 * rld if p >= 4 else 0)) for p in range(8)])
        # the same element the row formula names
        assert np.all((o == OUT_OF_RANGE) | (o == (m + 32 * blk) * rld + n * 2))
        mb = m + 32 * blk
        valid = (o != OUT_OF_RANGE) & (mb < M)
        assert np.all(o[valid] + 16 <= r_ext)                          # whole 16 bytes inside
        assert np.all((o[(o != OUT_OF_RANGE) & (mb >= M)]) >= r_ext)   # rows past M read zero
        assert np.all(o < 2 ** 32)
        # LDS image of the region: byte p*1024 + 16*lane holds the 8 columns from n, row mb
        region = {}
        for p_, l_ in itertools.product(range(8), range(64)):
            pos = p_ * 1024 + 16 * l_
            assert 0 <= pos and pos + 16 <= 8192
            region[pos] = (int(mb[p_, l_]), int(n[p_, l_])) if valid[p_, l_] else None
        r, h = lane & 31, lane >> 5
        for x in range(16):                  # logical chunk 4j + q
            addr = r * 256 + ((x ^ (r & read_swizzle)) << 4) + 8 * h
            assert np.all(addr + 8 <= 8192)
            for l_ in range(64):
                want_m = m0 + wm * 128 + 32 * blk + int(r[l_])
                want_n = n0 + wn * 128 + 8 * x + 4 * int(h[l_])
                got = region[int(addr[l_]) - 8 * int(h[l_])]
                if want_m < M and want_n < N:
                    assert got == (want_m, want_n - 4 * int(h[l_])), (blk, x, l_, got)
                else:
                    assert got is None or got[0] >= M or got[1] >= N


def check_gemm(name, g, sizes):
    M, N, K, batch = g["M"], g["N"], g["K"], g["batch"]
    sched, tiles_m, tiles_n = schedule(M, N, batch)
    per_t = tiles_m * tiles_n
    visited = np.concatenate(sched)
    assert np.array_equal(np.sort(visited), np.arange(per_t * batch)), f"{name}: schedule"
    # the kernel's own copies of the next tile use the next logical tile of the same slot
    assert (batch - 1) * g["c_bs"] * 2 + M * g["c_ld"] * 2 >= 0
    # last token's C region inside the tensor
    assert (batch - 1) * g["c_bs"] + (M - 1) * g["c_ld"] + N <= sizes[g["C"]]
    if g["res"]:
        assert (batch - 1) * g["res_bs"] + (M - 1) * g["res_ld"] + N <= sizes[g["res"]]
    if g["bias"]:
        assert (batch - 1) * g["bias_bs"] + N <= sizes[g["bias"]]
    written = np.zeros((M, N), dtype=np.int32)
    for logical in range(per_t):      # one token's tiles; other tokens differ by the base only
        t, m0, n0 = tile_of(logical, tiles_m, per_t)
        assert t == 0
        check_operand(g["a_kmajor"], g["a_ld"], g["a_bs"], K, M, m0, batch, sizes[g["A"]])
        check_operand(g["b_kmajor"], g["b_ld"], g["b_bs"], K, N, n0, batch, sizes[g["B"]])
        check_epilogue(g, m0, n0, written, sizes)
    assert np.all(written == 1), f"{name}: epilogue coverage"


SHAPES = [  # (B, T, D, k): the production shape, the envelope's corners, tile tails of every size
    (1024, 64, 1280, 2), (1024, 64, 1280, 3), (1024, 32, 512, 2), (256, 16, 256, 3), (1024, 40, 1000, 3),
    (512, 16, 640, 3), (384, 8, 384, 3), (300, 8, 384, 3), (256, 8, 64, 2), (128, 8, 72, 3),
    (640, 8, 136, 2), (896, 64, 1216, 3), (1000, 40, 1120, 2), (768, 16, 1280, 2), (257, 32, 1024, 3),
    (128, 64, 128, 2), (1024, 8, 1272, 3), (512, 32, 992, 2)]


@pytest.mark.parametrize("shape", SHAPES)
def test_gemm256_addresses_stay_in_bounds(shape):
    B, T, D, k = shape
    gemms, sizes = gemms_of_block(B, T, D, k)
    taken = 0
    for name, g in gemms.items():
        if supported(g):
            check_gemm(name, g, sizes)
            taken += 1
    if shape in ((1024, 64, 1280, 2), (1024, 32, 512, 2)):
        assert taken == 6


def test_output_staging_planted_swizzle_slip_caught():
    check_output_staging()
    with pytest.raises(AssertionError):
        check_output_staging(read_swizzle=7)


def test_residual_copy_checked_and_a_planted_swizzle_slip_caught():
    gemms, _ = gemms_of_block(1024, 64, 1280, 2)
    for name in ("down", "dh1"):
        g = gemms[name]
        assert supported(g) and g["res"]
        check_residual_copy(g, 768, 1024, 1, 1)
        with pytest.raises(AssertionError):
            check_residual_copy(g, 768, 1024, 1, 1, read_swizzle=7)


def test_replica_catches_a_planted_slip():
    """The checks are not vacuous: a copy offset one row too far fails them."""
    B, T, D, k = 384, 8, 384, 3
    gemms, sizes = gemms_of_block(B, T, D, k)
    g = gemms["dwout"]
    ext = operand_extent(False, g["a_ld"], g["K"], g["M"])
    off, *_ = slab_offsets(False, g["a_ld"], 2 * BM, g["M"])
    koff = (g["K"] // BK - 1) * BK * g["a_ld"] * 2
    assert np.all(off + koff + 16 <= ext)
    assert not np.all(off + koff + g["a_ld"] * 2 * BK + 16 <= ext)


# ---------------------------------------------------------------------------
# the copy pipeline: stages, issue order and wait counts of one wave

DMA_PER_OPERAND = 8
EPI_STORES = 32
# B pieces of a slab issued in the last k step of the step that frees its stage; the
# rest follow, spread over the first three k steps of the next step
B_LATE = 0


# A pieces of the last k step after MFMAs A_STRIDE * x; late B pieces in the other slots
A_STRIDE = 2


def b_early_begin(ks):
    return B_LATE + ((DMA_PER_OPERAND - B_LATE) * ks) // 3


def last_kstep_slots():
    """Operand of the copy issued after each of the last k step's 16 MFMAs (or None)."""
    slots = []
    for x in range(16):
        if x % A_STRIDE == 0 and x // A_STRIDE < DMA_PER_OPERAND:
            slots.append("A")
        elif (A_STRIDE == 1 and DMA_PER_OPERAND <= x < DMA_PER_OPERAND + B_LATE) or \
                (A_STRIDE == 2 and x % 2 == 1 and x // 2 < B_LATE):
            slots.append("B")
        else:
            slots.append(None)
    return slots


WAIT_STEADY = DMA_PER_OPERAND
WAIT_AFTER_EPILOGUE = DMA_PER_OPERAND + EPI_STORES
RES_INTERLEAVED = False
RES_WAIT = [DMA_PER_OPERAND, EPI_STORES // 4 + DMA_PER_OPERAND, EPI_STORES // 4 + DMA_PER_OPERAND, EPI_STORES // 4]


def simulate_pipeline(nk, ntiles, epilogue_extra=0, res=False):
    """Replays the kernel's per-wave event sequence for `ntiles` tiles of `nk` slabs: copy issues
    piece by piece (A ring of 2 stages, B ring of 3; A slab k+2 and the first B_LATE pieces of
    B slab k+3 in step k's last k step, the other B pieces of slab k+2 in the first k steps of
    step k; the last tile's next-tile copies are issued too, through a resource of extent 0),
    the epilogue's vector-memory operations, waits (vmcnt N + barrier) and the fragment reads of
    each slab.  Vector-memory operations complete in issue order, so after a wait with count N
    every operation but the newest N is complete.  Checks that every slab's copies are all
    issued and complete before its first read, that no copy targets a stage whose previous slab
    may still be read, and that no copy is in flight at the end.

    res: the kernels with a residual.  The tile's last step copies residual blocks 0 and 1
    (this wave's rows) into the two stages its last slab leaves, instead of the next tile's A
    slab 1; the epilogue waits for block i with the count RES_WAIT[i], reads it, stores its 8
    rows and copies block i+2 into the same region (i < 2); the next tile's A slab 1 follows
    the epilogue, and the next tile's first step waits with the steady count."""
    ops = []               # ("A"|"B"|"E", slab)
    done = 0               # ops[:done] complete
    stage_of = {}          # (operand, global slab) -> stage
    pieces = {}            # (operand, global slab) -> pieces issued
    reading = {}           # (operand, stage) -> global slab whose reads are not yet fenced

    def issue(op, slab, n):
        ring = 2 if op == "A" else 3
        st = slab % ring
        assert (op, st) not in reading or reading[(op, st)] is None, f"{op} stage {st} overwritten while read"
        stage_of[(op, slab)] = st
        pieces[(op, slab)] = pieces.get((op, slab), 0) + n
        assert pieces[(op, slab)] <= DMA_PER_OPERAND
        ops.extend([(op, slab)] * n)   # one 16-byte copy per lane and instruction

    def wait(n):
        nonlocal done
        done = max(done, len(ops) - n)
        for key in reading:        # the barrier: every wave's reads before it are finished
            reading[key] = None

    def read(slab):
        for op in ("A", "B"):
            assert pieces.get((op, slab), 0) == DMA_PER_OPERAND, f"slab {slab} {op} not fully copied"
            last = len(ops) - 1 - ops[::-1].index((op, slab))
            assert last < done, f"slab {slab} {op} read before its copy completed"
            reading[(op, stage_of[(op, slab)])] = slab

    res_region = {}        # (tile, block) -> (operand, stage) holding it
    res_read_done = set()

    def res_issue(t, i, region):
        # a wave overwrites only its own region, after its reads of the block there
        for (tt, ii), reg in res_region.items():
            if reg == region and (tt, ii) not in res_read_done:
                raise AssertionError(f"residual block {ii} overwritten before it was read")
        res_region[(t, i)] = region
        ops.extend([("R", (t, i))] * DMA_PER_OPERAND)

    def res_read(t, i):
        last = len(ops) - 1 - ops[::-1].index(("R", (t, i)))
        assert last < done, f"residual block {i} of tile {t} read before its copy completed"
        res_read_done.add((t, i))

    def wait_vm(n):        # a wave's own wait, no barrier
        nonlocal done
        done = max(done, len(ops) - n)

    S = lambda t, k: t * nk + k          # global slab index
    # prologue
    issue("A", S(0, 0), DMA_PER_OPERAND)
    issue("B", S(0, 0), DMA_PER_OPERAND)
    issue("A", S(0, 1), DMA_PER_OPERAND)
    issue("B", S(0, 1), DMA_PER_OPERAND)
    issue("B", S(0, 2), B_LATE)
    wait(2 * DMA_PER_OPERAND + B_LATE)
    read(S(0, 0))                          # first k step's fragments
    for t in range(ntiles):
        has_next = t + 1 < ntiles
        for k in range(nk):
            # k steps 0..2: the rest of B slab k+2, then k steps 1..3's fragments of slab k
            for ks in range(3):
                issue("B", S(t, k + 2), b_early_begin(ks + 1) - b_early_begin(ks))
            read(S(t, k))
            wait(WAIT_AFTER_EPILOGUE if (k == 0 and t > 0 and not res) else WAIT_STEADY)
            # copies of the next tile are issued even without one (slab indices past the last
            # tile: empty copies into freed stages)
            if res and k == nk - 1:
                assert B_LATE == 0
                xb, ya = ("B", S(t, k) % 3), ("A", S(t, k) % 2)   # stages of the last slab
                for region in (xb, ya):
                    assert reading.get(region) is None, "residual copied over a slab still read"
                if RES_INTERLEAVED:        # a planted mistake: blocks 0 and 1 slot by slot
                    res_region[(t, 0)], res_region[(t, 1)] = xb, ya
                    for _ in range(DMA_PER_OPERAND):
                        ops.extend([("R", (t, 0)), ("R", (t, 1))])
                else:
                    res_issue(t, 0, xb)
                    res_issue(t, 1, ya)
            else:
                for op in last_kstep_slots():
                    if op is not None:
                        issue(op, S(t, k + 2) if op == "A" else S(t, k + 3), 1)
            if k + 1 < nk:
                read(S(t, k + 1))          # next slab's first fragments
            elif has_next:
                read(S(t + 1, 0))
        if res:
            for i in range(4):
                wait_vm(RES_WAIT[i])
                res_read(t, i)
                for e in range(EPI_STORES // 4):
                    ops.append(("E", (t, i, e)))
                if i < 2:
                    res_issue(t, i + 2, res_region[(t, i)])
            for e in range(epilogue_extra):
                ops.append(("E", (t, "x", e)))
            issue("A", S(t, nk + 1), DMA_PER_OPERAND)   # the next tile's A slab 1
        else:
            for e in range(EPI_STORES + epilogue_extra):
                ops.append(("E", (t, e)))
    wait(0)                                # the kernel's final wait
    assert done == len(ops)


@pytest.mark.parametrize("nk", [4, 6, 16, 20, 40, 80, 120])
@pytest.mark.parametrize("ntiles", [1, 2, 3, 7])
def test_gemm256_pipeline_waits(nk, ntiles):
    simulate_pipeline(nk, ntiles)
    simulate_pipeline(nk, ntiles, res=True)


def test_pipeline_replica_catches_interleaved_residual_blocks():
    """Blocks 0 and 1 copied slot by slot leave one copy after block 0's last piece, not
    DMA_PER_OPERAND: the first epilogue wait would not cover block 0."""
    global RES_INTERLEAVED
    RES_INTERLEAVED = True
    try:
        with pytest.raises(AssertionError):
            simulate_pipeline(20, 2, res=True)
    finally:
        RES_INTERLEAVED = False


def test_pipeline_replica_catches_a_short_residual_wait():
    """The epilogue's second wait one block too loose (block 1 could still be in flight)."""
    saved = RES_WAIT[1]
    RES_WAIT[1] = saved + DMA_PER_OPERAND
    try:
        with pytest.raises(AssertionError):
            simulate_pipeline(20, 2, res=True)
    finally:
        RES_WAIT[1] = saved


def test_pipeline_replica_catches_late_b_between_a_pieces():
    """Late B pieces interleaved with A's leave fewer than DMA_PER_OPERAND copies after A's
    last piece, so the steady wait would let A pieces stay in flight: the replica must say so."""
    global A_STRIDE, B_LATE
    saved = A_STRIDE, B_LATE
    A_STRIDE, B_LATE = 2, 2
    try:
        with pytest.raises(AssertionError):
            simulate_pipeline(20, 2)
    finally:
        A_STRIDE, B_LATE = saved


def test_pipeline_replica_catches_a_short_wait():
    """A steady-state wait one slab too loose (two B slabs left in flight) is caught."""
    global WAIT_STEADY
    saved = WAIT_STEADY
    WAIT_STEADY = 2 * DMA_PER_OPERAND
    try:
        with pytest.raises(AssertionError):
            simulate_pipeline(20, 2)
    finally:
        WAIT_STEADY = saved
