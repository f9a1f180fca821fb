"""CPU model of how an MLA key tile is laid out in LDS and loaded.

A tile holds 32 cache rows of 576 bf16 values (1,152 bytes) at a row pitch of
1,184 bytes, filled by direct loads of 64 lanes x 16 bytes: load i writes LDS
slots [64 i, 64 i + 64), and slot s holds 16-byte chunk s mod 74 of row
s div 74.  Chunks 72 and 73 of a row are padding and re-fetch chunk 0 of the
same row; slots past the 32 rows re-fetch chunk 0 of the last row.  The
head-split kernel's key-half-1 waves (four of them) issue the loads,
wave w taking loads w, w + 4, ...

The model checks what the kernel relies on: every chunk of every row is
fetched into its own slot, no load reads outside the tile's 32 rows or writes
past the tile's bytes, each load is issued by exactly one wave, and the
pitch keeps both LDS read forms free of bank conflicts (64 banks of 4 bytes)
in the groups of lanes the LDS serves together: eight lanes of a 16-byte K
read (eight rows at one column), and the half-wave of a transposing V read
(eight rows x 32 bytes).  That grouping is the one under which the
head-split kernel's measured SQ_LDS_BANK_CONFLICT count is zero at this pitch
(at 1,168 bytes the V reads conflicted)."""

ROW_BYTES = 576 * 2
PITCH = ROW_BYTES + 32
SLOTS = PITCH // 16
CHUNKS = ROW_BYTES // 16
ROWS = 32
LOADS = (ROWS * SLOTS + 63) // 64
TILE_BYTES = LOADS * 1024
LOADERS = 4


def slot_source(slot):
    """(row, byte offset in the row) a slot's lane fetches."""
    row, ch = divmod(slot, SLOTS)
    if row >= ROWS:
        return ROWS - 1, 0
    return row, (ch * 16 if ch < CHUNKS else 0)


def test_every_chunk_lands_in_its_slot():
    seen = set()
    for i in range(LOADS):
        for lane in range(64):
            slot = 64 * i + lane
            assert 16 * slot + 16 <= TILE_BYTES
            row, off = slot_source(slot)
            assert 0 <= row < ROWS and 0 <= off and off + 16 <= ROW_BYTES
            r, ch = divmod(slot, SLOTS)
            if r < ROWS and ch < CHUNKS:
                assert (row, off) == (r, 16 * ch)
                seen.add((r, ch))
    assert seen == {(r, c) for r in range(ROWS) for c in range(CHUNKS)}
    assert TILE_BYTES >= ROWS * PITCH


def test_each_load_has_one_loader():
    per_wave = (LOADS + LOADERS - 1) // LOADERS
    issued = [w + LOADERS * j for w in range(LOADERS) for j in range(per_wave) if w + LOADERS * j < LOADS]
    assert sorted(issued) == list(range(LOADS))
    # the wait counts assume every loader has at least LOADS // LOADERS loads per tile
    for w in range(LOADERS):
        assert sum(1 for j in range(per_wave) if w + LOADERS * j < LOADS) >= LOADS // LOADERS


def banks(addr, nbytes):
    return {((addr + b) // 4) % 64 for b in range(0, nbytes, 4)}


def test_pitch_is_free_of_bank_conflicts():
    assert not conflict_free(PITCH - 16), "the former pitch should conflict on the V reads"
    assert conflict_free(PITCH)


def conflict_free(pitch):
    for col in range(0, ROW_BYTES, 16):
        for r0 in (0, 8, 16, 24):
            used = [b for r in range(r0, r0 + 8) for b in banks(r * pitch + col, 16)]
            if len(used) != len(set(used)):
                return False
    for col in range(0, 1024, 32):
        for r0 in (0, 8, 16, 24):
            used = [b for r in range(r0, r0 + 8) for b in banks(r * pitch + col, 32)]
            if len(used) != len(set(used)):
                return False
    return True

