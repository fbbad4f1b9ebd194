"""XOR swizzle of a stage-relative LDS byte offset (oracle).

Source: "copy_async -> tma", section "Demonstration program" (the shared
layout built with swizzle mode 3, described as a 128-byte swizzle) and section
"How inputs change the algorithm" (the swizzle mode sets the descriptor's
swizzle field and the innermost-box constraint, and splits a wider inner axis
into swizzle atoms).

The pages name mode 3 (128 bytes) but never print its formula, and name no
other mode.  Readings adopted:

* Mode 3 (128 bytes): the stage is viewed as 128-byte rows of eight 16-byte
  chunks; the chunk index (offset bits 4..6) is XORed with the row index
  modulo 8 (offset bits 7..9).
* Modes 1 and 2 follow the mode numbering (mode m spans 16 * 2**m bytes:
  32 and 64 bytes) with the same construction on m bits: the 16-byte chunk
  index within its 16 * 2**m-byte span (bits 4 .. 4+m-1) is XORed with the
  128-byte row index modulo 2**m (bits 7 .. 7+m-1).  Mode 0 is no swizzle.

Every mode only permutes whole 16-byte chunks inside one 16 * 2**m-byte span,
is its own inverse, and is a bijection on every 128 * 2**m-byte block.  Stage
bases are 1 KiB aligned, so stage-relative and absolute offsets give the same
pattern.
"""

ATOM_ROW_BYTES = 128
CHUNK_BYTES = 16
ROWS_PER_ATOM = 8

MODES = (0, 1, 2, 3)


def span_bytes(mode: int) -> int:
    """Bytes over which mode ``mode`` permutes chunks (its atom width)."""
    return CHUNK_BYTES << mode if mode else 0


def swizzle(offset: int, mode: int) -> int:
    """Physical LDS byte offset holding logical byte ``offset`` (and vice
    versa) under swizzle mode ``mode``."""
    if mode == 0:
        return offset
    if mode not in MODES:
        raise ValueError("swizzle mode must be 0..3")
    chunks = 1 << mode                          # chunks in one span
    span = CHUNK_BYTES * chunks
    row = offset // ATOM_ROW_BYTES              # 128-byte row index
    span_base = (offset // span) * span
    chunk = (offset % span) // CHUNK_BYTES      # chunk within its span
    within = offset % CHUNK_BYTES
    phys_chunk = chunk ^ (row % chunks)
    return span_base + phys_chunk * CHUNK_BYTES + within


def swizzle128(offset: int) -> int:
    """Mode 3 (128 bytes)."""
    return swizzle(offset, 3)


def apply(offset: int, mode) -> int:
    """``mode`` may be a swizzle mode or a bool (True = 128 bytes)."""
    if mode is True:
        mode = 3
    elif mode is False or mode is None:
        mode = 0
    return swizzle(offset, int(mode))
