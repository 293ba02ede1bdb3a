"""Host check of the LDS row placement of the pipelined backward kernels.

The streamed tiles (query tiles in dK/dV, key tiles in dQ) sit in rows of
D + 8 bf16 elements, row r of each 16-row group in slot 4 (r mod 4) + r / 4
(tile_slot in fa_bwd.hip).  The claim is that both read patterns of those
tiles then touch every one of LDS's 64 four-byte banks at most once per
group of lanes served together:
  * row reads (ds_read_b128): 16 lanes, 16 consecutive rows, 16 bytes each;
  * transposed reads (ds_read_b64_tr_b16): 32 lanes, 4 consecutive rows
    starting at a multiple of 4, 64 contiguous bytes of each row.
The banks are modelled as (byte address / 4) mod 64.
"""
import pytest


def tile_slot(r: int) -> int:
    return (r & ~15) | ((r & 3) << 2) | ((r >> 2) & 3)


def banks(byte_addr: int, nbytes: int):
    return [((byte_addr + b) // 4) % 64 for b in range(0, nbytes, 4)]


@pytest.mark.parametrize("d", [64, 128])
def test_slot_map_is_an_involution(d):
    for r in range(256):
        assert tile_slot(tile_slot(r)) == r


@pytest.mark.parametrize("d", [64, 128])
def test_row_reads_conflict_free(d):
    row_bytes = 2 * (d + 8)
    for first in range(0, 64, 16):          # 16-lane groups of a wavefront
        for chunk in range(d // 8):         # the 16-byte column read
            used = []
            for r in range(first, first + 16):
                used += banks(tile_slot(r) * row_bytes + 16 * chunk, 16)
            assert len(used) == len(set(used)) == 64, (d, first, chunk)


@pytest.mark.parametrize("d", [64, 128])
def test_transposed_reads_conflict_free(d):
    row_bytes = 2 * (d + 8)
    for base in range(0, 64, 4):            # 4 consecutive rows
        for col in range(0, 2 * d, 64):     # 64 contiguous bytes per row
            used = []
            for r in range(base, base + 4):
                used += banks(tile_slot(r) * row_bytes + col, 64)
            assert len(used) == len(set(used)) == 64, (d, base, col)


def test_plain_padding_serves_only_one_pattern():
    # Without the placement, 304-byte rows (the small-grid kernels') keep the
    # row reads conflict-free but not the transposed reads.
    row_bytes = 304
    used = []
    for r in range(4):
        used += banks(r * row_bytes, 64)
    assert len(set(used)) < len(used)
