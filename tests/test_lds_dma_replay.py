"""Host-side replay of the address arithmetic of every direct HBM -> LDS copy
(buffer_load ... lds) in the gfx950 kernels, at the tested shapes.

A direct copy writes lane l's 16 (or 4) bytes to the LDS address held in M0
plus 16*l (4*l), for every active lane, and reads its global bytes at the
buffer resource's base plus the lane's offset; an offset at or past the
resource's size reads zeros without touching memory.  For each copy site this
restates the kernel's index arithmetic and checks:
  * every LDS byte written lies inside the slot it is meant for, and so inside
    the kernel's static LDS;
  * the copies of one tile write every (row, 16-byte chunk) of it exactly once
    and no pad chunk;
  * a lane's LDS row and chunk are those of the global row and chunk it reads;
  * every in-range global byte lies inside the tensor the resource covers.
For the prefill ring it also replays the kernel's tile schedule (band limits,
runs of query tiles, the copies issued two tiles ahead) and checks that a slot
is only refilled once every wave has passed the barrier after its last read,
and that a tile's copies were waited for before any read of it.

The constants below restate those of the kernels' sources (the row pads, the
rows per copy instruction, the waves per workgroup).
"""
import itertools

import pytest

LDS_BYTES = 160 * 1024


# ---------------------------------------------------------------------------
# generic: one wave-wide 16-byte copy instruction covering whole rows
# ---------------------------------------------------------------------------

def rows_copy(chunks_per_lds_row, rows_per_copy, data_chunks, row0, valid_rows, lds_slot_base, row_bytes_lds,
              global_row_bytes):
    """Lanes of one instruction that copies rows row0 .. row0+rows_per_copy-1:
    lane l -> (row l // chunks_per_lds_row, chunk l % chunks_per_lds_row); pad
    chunks and rows past `valid_rows` are inactive.  Returns a list of
    (row, chunk, lds_byte, global_offset)."""
    out = []
    m0 = lds_slot_base + row0 * row_bytes_lds
    for lane in range(64):
        lr, ch = lane // chunks_per_lds_row, lane % chunks_per_lds_row
        if lr >= rows_per_copy or ch >= data_chunks or row0 + lr >= valid_rows:
            continue
        out.append((row0 + lr, ch, m0 + 16 * lane, (row0 + lr) * global_row_bytes + 16 * ch))
    return out


def check_tile(writes, n_rows, data_chunks, slot_base, slot_bytes, row_bytes_lds):
    seen = set()
    for row, ch, lds, _ in writes:
        assert slot_base <= lds and lds + 16 <= slot_base + slot_bytes, (row, ch, lds)
        assert lds == slot_base + row * row_bytes_lds + 16 * ch          # the chunk lands where it belongs
        assert (row, ch) not in seen
        seen.add((row, ch))
    assert seen == {(r, c) for r in range(n_rows) for c in range(data_chunks)}


# ---------------------------------------------------------------------------
# prefill: K and V ring, 3 slots of 64 rows, 8 waves
# ---------------------------------------------------------------------------

PF_BN = 64
PF_WAVES = 8
K_CH, V_CH = 192 // 8 + 2, 128 // 8 + 2        # 16-byte chunks per padded LDS row
K_ROW_LDS, V_ROW_LDS = 16 * K_CH, 16 * V_CH
K_SLOT, V_SLOT = PF_BN * K_ROW_LDS, PF_BN * V_ROW_LDS
PF_XCH = 4 * 64 * 16 * 4                          # H_N handed between the waves of a SIMD
PF_LDS = 3 * K_SLOT + 3 * V_SLOT + PF_XCH + 8


def prefill_tile_copies(wave, n_kv):
    """The copies wave `wave` issues for one tile (kernel: issue_tile)."""
    k_rb, v_rb = n_kv * 384, n_kv * 256
    ks, vs = [], []
    for c in range(PF_BN // 2 // PF_WAVES):                    # 4 K copies of 2 rows
        row0 = 2 * (wave + PF_WAVES * c)
        ks += rows_copy(K_CH, 2, 24, row0, PF_BN, 0, K_ROW_LDS, k_rb)
    n_v = (PF_BN + 2) // 3
    for c in range((n_v + PF_WAVES - 1) // PF_WAVES):           # 3 or 2 V copies of 3 rows
        row0 = 3 * (wave + PF_WAVES * c)
        if row0 < PF_BN:
            vs += rows_copy(V_CH, 3, 16, row0, PF_BN, 0, V_ROW_LDS, v_rb)
    return ks, vs


def test_prefill_lds_fits():
    assert PF_LDS <= LDS_BYTES


@pytest.mark.parametrize("n_kv", [1, 2, 16, 42])
def test_prefill_ring_copies_cover_each_tile_once(n_kv):
    ks, vs = [], []
    counts = []
    for w in range(PF_WAVES):
        k, v = prefill_tile_copies(w, n_kv)
        ks += k
        vs += v
        counts.append(len({r // 2 for r, _, _, _ in k}) + len({r // 3 for r, _, _, _ in v}))
    check_tile(ks, PF_BN, 24, 0, K_SLOT, K_ROW_LDS)
    check_tile(vs, PF_BN, 16, 0, V_SLOT, V_ROW_LDS)
    # copy instructions per wave and tile: the counts the tile-end waits leave in flight
    assert counts == [7] * 6 + [6] * 2


@pytest.mark.parametrize("T,n_kv", [(1, 1), (63, 2), (64, 1), (65, 3), (4096, 16), (131072, 16), (300, 2)])
def test_prefill_global_offsets_inside_sequence(T, n_kv):
    """Rows past the sequence end read zeros (offset >= T * row_bytes, the
    resource's size); every other byte lies inside sequence b's rows of the
    K/V tensor: resource base = first row of the sequence plus the head's column."""
    k_rb, v_rb = n_kv * 384, n_kv * 256
    n_tiles = (T + PF_BN - 1) // PF_BN
    for kt in {0, n_tiles - 1}:
        for w in range(PF_WAVES):
            k, v = prefill_tile_copies(w, n_kv)
            for writes, rb, width in ((k, k_rb, 384), (v, v_rb, 256)):
                for row, ch, _, off in writes:
                    g = kt * PF_BN * rb + off
                    if g >= T * rb:
                        continue                                  # reads zeros
                    key = kt * PF_BN + row
                    assert key < T
                    assert g == key * rb + 16 * ch and 16 * ch + 16 <= width     # head j's own bytes of row key
    # the resource size itself stays below 2^32 for every shape the API admits
    assert ((T + 64) * n_kv * 384) < 2 ** 31


def prefill_schedule(T, window, P=0, run_len=None):
    """Replay of the kernel's tile schedule for one work item's runs: for each
    query tile, the reference pass (which reads the diagonal tile's K rows from
    the ring while that tile is still there), the tiles it reads, at each tile
    end the copies issued and the wait, and the epilogue's wait for every copy
    issued before it and its barrier.  Yields events (kind, tile) in program
    order for one wave."""
    BM = 64
    q0 = P // BM * BM
    Tk = T
    n_qt = ((P % BM) + (T - P) + BM - 1) // BM
    tile_lo = lambda qt: max(0, q0 + qt * BM - window + 1) // PF_BN if window > 0 else 0
    tile_hi = lambda qt: (min(q0 + qt * BM + BM, Tk) - 1) // PF_BN
    if run_len is None:
        run_len = 1 if not (0 < window <= 2 * PF_BN + 1) else n_qt
    runs = [(s, min(s + run_len, n_qt)) for s in range(0, n_qt, run_len)]
    for first, end in runs:
        events = []
        run_last = tile_hi(end - 1)
        nxt = tile_lo(first)
        events.append(("copy", nxt)); nxt += 1
        if nxt <= tile_hi(first):
            events.append(("copy", nxt)); nxt += 1
        events.append(("wait_all", None))
        events.append(("barrier", None))
        for qt in range(first, end):
            lo, hi = tile_lo(qt), tile_hi(qt)
            next_lo = tile_lo(qt + 1) if qt + 1 < end else 1 << 30
            if nxt - 3 <= hi < nxt:
                events.append(("read", hi))                 # reference pass from LDS
            for kt in range(lo, hi + 1):
                events.append(("read", kt))
                last = kt == hi
                nt = kt + 1 if not last else next_lo
                limit = min(min(kt, nt) + 2, run_last)
                while nxt <= limit:
                    events.append(("copy", nxt)); nxt += 1
                events.append(("wait_but_newest", nxt - 1) if nxt - 1 > nt else ("wait_all", None))
                events.append(("barrier", None))
            events.append(("wait_all", None))               # epilogue: copies older than its loads
            events.append(("barrier", None))
        yield events


def test_prefill_reference_pass_reads_ring_in_window_runs():
    """In a run of query tiles of a 128-token window every reference pass
    after the first finds the diagonal tile in the ring."""
    for events in prefill_schedule(4096, 128, 0):
        reads = [t for kind, t in events if kind == "read"]
        n_qt = 4096 // 64
        # three key tiles per query tile (two for the first two) plus one
        # reference read per query tile
        assert len(reads) == sum(min(qt, 2) + 1 for qt in range(n_qt)) + n_qt


def check_schedule(events):
    """Slot discipline of the 3-slot ring: a copy into slot s only after the
    barrier that follows the last read of the tile s held, and every read of a
    tile after a wait that covers its copies and a barrier."""
    slot_tile = {}          # slot -> tile it holds (or is receiving)
    read_since_barrier = set()
    landed = set()          # tiles whose copies this wave waited for
    in_flight = []
    visible = set()         # tiles landed in every wave (after a barrier)
    for kind, t in events:
        if kind == "copy":
            s = t % 3
            assert s not in read_since_barrier, ("slot refilled before the barrier after its read", t)
            slot_tile[s] = t
            in_flight.append(t)
        elif kind == "wait_all":
            landed |= set(in_flight)
            in_flight = []
        elif kind == "wait_but_newest":
            # everything but the copies of the newest tile
            landed |= {x for x in in_flight if x != t}
            in_flight = [x for x in in_flight if x == t]
        elif kind == "barrier":
            visible |= landed
            read_since_barrier = set()
        elif kind == "read":
            assert slot_tile.get(t % 3) == t, ("tile not in its slot", t)
            assert t in visible, ("tile read before its copies were waited for", t)
            read_since_barrier.add(t % 3)


@pytest.mark.parametrize("T,window,P", [
    (1, 0, 0), (64, 0, 0), (65, 0, 0), (333, 0, 0), (4096, 0, 0), (300, 1, 0), (300, 64, 0), (300, 65, 0),
    (333, 128, 0), (16384, 128, 0), (16384, 129, 0), (300, 1000, 0), (228, 0, 100), (256, 128, 127),
    (4224, 128, 128), (32768, 0, 28672)])
def test_prefill_ring_schedule(T, window, P):
    for events in prefill_schedule(T, window, P):
        check_schedule(events)
    # runs of several lengths for the window cases
    if 0 < window <= 129:
        for rl in (1, 2, 3, 8):
            for events in prefill_schedule(T, window, P, run_len=rl):
                check_schedule(events)


# ---------------------------------------------------------------------------
# window decode: V rows of the window, 4 waves x 32 rows
# ---------------------------------------------------------------------------

DW_VCH = 128 // 8 + 2
DW_VROW = 16 * DW_VCH
DW_LDS = 128 * DW_VROW + 2 * 4 * 16 * 4


@pytest.mark.parametrize("n_vis,n_kv", [(128, 16), (1, 1), (37, 3), (0, 2)])
def test_window_decode_copies(n_vis, n_kv):
    assert DW_LDS <= LDS_BYTES
    v_rb = n_kv * 256
    writes = []
    for wave in range(4):
        for c in range((32 + 2) // 3):
            if 3 * c >= 32:
                continue
            row0 = 32 * wave + 3 * c
            # rows past the wave's 32 are inactive (the kernel's row-in-wave test)
            ws = rows_copy(DW_VCH, 3, 16, row0, 32 * wave + 32, 0, DW_VROW, v_rb)
            writes += ws
    check_tile(writes, 128, 16, 0, 128 * DW_VROW, DW_VROW)
    for row, ch, _, off in writes:
        if off < n_vis * v_rb:
            assert row < n_vis


# ---------------------------------------------------------------------------
# backward: 64-row tiles, rows of 192 or 128 values (+32-byte pad), and one
# float per lane for the rows' statistics; the dK/dV kernel runs 4 waves (32
# keys each), the dQ kernel 8 (16 queries each)
# ---------------------------------------------------------------------------

DKDV_WAVES, DQ_WAVES = 4, 8


def backward_tile_writes(cols, rs, n_waves):
    """The copies of one 64-row tile by n_waves waves: (writes, copies per wave)."""
    ch_per_row = rs // 8
    rows = 64 // ch_per_row
    n = (64 + rows - 1) // rows
    writes = []
    per_wave = []
    for wave in range(n_waves):
        k = 0
        for c in range((n + n_waves - 1) // n_waves):
            row0 = rows * (wave + n_waves * c)
            if row0 < 64:
                writes += rows_copy(ch_per_row, rows, cols // 8, row0, 64, 0, rs * 2, 1234)
                k += 1
        per_wave.append(k)
    return writes, per_wave


@pytest.mark.parametrize("n_waves", [DKDV_WAVES, DQ_WAVES])
@pytest.mark.parametrize("cols,rs", [(192, 208), (128, 144)])
def test_backward_tile_copies(cols, rs, n_waves):
    writes, _ = backward_tile_writes(cols, rs, n_waves)
    check_tile(writes, 64, cols // 8, 0, 64 * rs * 2, rs * 2)


def test_backward_step_wait_leaves_only_the_newest_step():
    """At a step's end a wave waits with vmcnt(13) (dK/dV, 4 waves) or
    vmcnt(6) (dQ, 8 waves): it must have issued at least that many copies for
    the step just requested, so every older copy has landed."""
    for n_waves, wait in ((DKDV_WAVES, 13), (DQ_WAVES, 6)):
        q = backward_tile_writes(192, 208, n_waves)[1]
        v = backward_tile_writes(128, 144, n_waves)[1]
        for w in range(n_waves):
            assert q[w] + v[w] >= wait, (n_waves, w, q[w], v[w])


def test_backward_lds_fits_and_stat_copies():
    q_slot, v_slot = 64 * 208 * 2, 64 * 144 * 2
    dkdv = 3 * q_slot + 3 * v_slot + 2 * 3 * 64 * 4
    dq = 3 * q_slot + 3 * v_slot
    assert dkdv <= LDS_BYTES and dq <= LDS_BYTES
    # one float per lane: lane l -> LDS + 4l, global row l of the tile
    for n_valid in (1, 37, 64):
        for lane in range(64):
            lds = 4 * lane
            assert lds + 4 <= 64 * 4
            # rows past n_valid read zeros (offset past the resource's size)
            n_h = 80
            assert (lane * n_h * 4 < n_valid * n_h * 4) == (lane < n_valid)


# ---------------------------------------------------------------------------
# latent decode: 32-row tiles of 576 values, c part (512, +16 pad) and rotary
# part (64) in two rings of 4 slots; 4 waves
# ---------------------------------------------------------------------------

LT_BN, LT_ROW_B, LT_CS_B, LT_R_B = 32, 1152, 1056, 128


def test_latent_copies():
    c_ring, r_ring = 4 * LT_BN * LT_CS_B, 4 * LT_BN * LT_R_B
    pbuf = 2 * 4 * 64 * 16
    assert c_ring + r_ring + pbuf + 16 <= LDS_BYTES
    for slot in range(4):
        c_writes, r_writes = set(), set()
        for wave in range(4):
            for k in range(LT_BN // 4):
                row = wave + 4 * k
                base = (slot * LT_BN + row) * LT_CS_B
                for lane in range(64):
                    lds, off = base + 16 * lane, row * LT_ROW_B + 16 * lane
                    assert slot * LT_BN * LT_CS_B <= lds and lds + 16 <= (slot + 1) * LT_BN * LT_CS_B
                    assert lds + 16 <= base + LT_CS_B               # inside the padded row
                    assert off + 16 <= row * LT_ROW_B + 1024        # the c part of the row
                    c_writes.add((row, lane))
            base = (slot * LT_BN + 8 * wave) * LT_R_B
            for lane in range(64):
                lds = base + 16 * lane
                off = (8 * wave + lane // 8) * LT_ROW_B + 1024 + 16 * (lane % 8)
                assert slot * LT_BN * LT_R_B <= lds and lds + 16 <= (slot + 1) * LT_BN * LT_R_B
                # the chunk lands in its row's rotary slot
                row = 8 * wave + lane // 8
                assert lds == (slot * LT_BN + row) * LT_R_B + 16 * (lane % 8)
                assert row * LT_ROW_B + 1024 <= off and off + 16 <= (row + 1) * LT_ROW_B
                r_writes.add((row, lane % 8))
        assert c_writes == set(itertools.product(range(LT_BN), range(64)))
        assert r_writes == set(itertools.product(range(LT_BN), range(8)))
