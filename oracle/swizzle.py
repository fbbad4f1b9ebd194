"""128-byte XOR swizzle of a stage-relative LDS byte offset (oracle).

Source: "copy_async -> tma", section "Demonstration program" (the shared
layout built with swizzle mode 3, described as a 128-byte swizzle) and section
"How inputs change the algorithm" (the swizzle mode sets the descriptor's
swizzle field and splits the inner axis into 128-byte atoms).

The pages name the mode but never print its formula.  Reading adopted: the
stage is viewed as 128-byte rows of eight 16-byte chunks; the chunk index
(offset bits 4..6) is XORed with the row index modulo 8 (offset bits 7..9).
The map only permutes whole 16-byte chunks inside one 128-byte row, is its
own inverse, and is a bijection on every 1 KiB block (one swizzle atom of
8 rows x 128 bytes).  Stage bases are 1 KiB aligned, so stage-relative and
absolute offsets give the same pattern.
"""

ATOM_ROW_BYTES = 128
CHUNK_BYTES = 16
ROWS_PER_ATOM = 8


def swizzle128(offset: int) -> int:
    """Physical LDS byte offset holding logical byte ``offset`` (and vice versa)."""
    row = offset // ATOM_ROW_BYTES
    chunk = (offset % ATOM_ROW_BYTES) // CHUNK_BYTES
    within = offset % CHUNK_BYTES
    phys_chunk = chunk ^ (row % ROWS_PER_ATOM)
    return row * ATOM_ROW_BYTES + phys_chunk * CHUNK_BYTES + within


def apply(offset: int, swizzled: bool) -> int:
    return swizzle128(offset) if swizzled else offset
