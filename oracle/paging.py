"""Entry counts, windows, eligibility and paged slot mapping (oracle, test infrastructure).

Sources:
* Window rule: [P3] "KV 缓存压缩" states that c4a entry i covers raw positions
  4i .. 4i+7 with its RoPE anchor at 4i; [P1] "DeepSeek V4 Attention
  Architecture" gives the c4a (8 tokens, stride 4) and c128a (128 tokens,
  stride 128) shapes.
* Block unit: [P1] "KV Cache Memory Management" and [P2] "3.1 顯存" fix one
  logical block of 256 raw positions for every compressed layer, i.e. 64 c4a
  entries or 2 c128a entries per block.
* Eligibility: [P3] "注意力计算剪枝" -- a compressed entry may not contain
  future tokens, so an entry is usable at query position p only once its whole
  window lies at or before p.

Readings: the c128a anchor is 128 i (R2); no partial or padded entries (R3);
an entry lives in the block of its anchor (R18); raw positions use the same
256-position paging (R19).
"""
from __future__ import annotations

import numpy as np

BLOCK = 256  # raw positions per logical block
SHAPES = {4: 8, 128: 128}  # ratio m -> window w (c4a: coff 2, c128a: coff 1)


def check_shape(ratio: int, window: int) -> None:
    if SHAPES.get(ratio) != window:
        raise ValueError(f"unsupported (ratio, window) = ({ratio}, {window})")


def entries_per_block(ratio: int) -> int:
    return BLOCK // ratio


def num_entries(n_raw: int, ratio: int, window: int) -> int:
    """Entries whose full window lies inside raw positions 0 .. n_raw-1."""
    check_shape(ratio, window)
    return (n_raw - window) // ratio + 1 if n_raw >= window else 0


def num_eligible(q_pos: int, ratio: int, window: int) -> int:
    """Entries usable by a query at position q_pos (window end <= q_pos)."""
    return num_entries(q_pos + 1, ratio, window)


def entry_window(i: int, ratio: int, window: int):
    """(first raw position, last raw position, RoPE anchor) of entry i."""
    check_shape(ratio, window)
    return ratio * i, ratio * i + window - 1, ratio * i


def entry_slot(bt_row: np.ndarray, i: int, ratio: int) -> int:
    """Physical row of compressed entry i for a sequence with block-table row bt_row."""
    e = entries_per_block(ratio)
    return int(bt_row[i // e]) * e + i % e


def raw_slot(bt_row: np.ndarray, j: int) -> int:
    """Physical row of raw position j (state or sliding-window pages)."""
    return int(bt_row[j // BLOCK]) * BLOCK + j % BLOCK


def new_entries(start: int, n_new: int, ratio: int, window: int) -> range:
    """Entries completed by raw positions start .. start+n_new-1."""
    return range(num_entries(start, ratio, window), num_entries(start + n_new, ratio, window))
