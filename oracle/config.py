"""Format parameters of the packed cache (oracle side).

Reading adopted (the pages name no sizes): head_dim D in {64, 128, 256}, b in {2, ..., 8}
bits, token block B in {64, 128}, pack run R = 32 tokens with R dividing B.
The run is the unit that gets its own width and offset; the block is the unit
of quantisation (K), permutation and append.  A run's header entry holds its
width w (0..b) and minimum m (0..2^b - 1): one byte (w << 4 | m) up to b = 4,
two bytes (little-endian w << 8 | m) for b = 5..8, where m no longer fits a
nibble.  The pages give no header encoding; this one is the plainest that
holds both fields.

Payload order (a format variant; the explainer page's "Block matrix before
and after repacking" asks that the packed layout suit the GPU that consumes
it): 0 stores a record's (run, channel) entries run-major, then by channel;
1 stores each run row of a K record by decreasing width, ties by increasing
channel, so that neighbouring entries share a width.  V records and headers
keep order 0 in both.
"""

from __future__ import annotations

import dataclasses


@dataclasses.dataclass(frozen=True)
class Config:
    head_dim: int = 128
    bits: int = 4
    block: int = 64
    run: int = 32
    permute: int = 1          # 0 identity, 1 greedy grouping, 2 sort key (oracle.perm)
    payload_order: int = 0    # 0 run-major then channel; 1 K rows by decreasing width

    def __post_init__(self):
        assert 2 <= self.bits <= 8, "b must be 2 .. 8"
        assert self.block in (64, 128), "B must be 64 or 128"
        assert self.run == 32, "R must be 32"
        assert self.block % self.run == 0
        assert self.head_dim in (64, 128, 256), "D must be 64, 128 or 256"
        assert int(self.permute) in (0, 1, 2), "permute must be 0, 1 or 2"
        assert self.payload_order in (0, 1), "payload_order must be 0 or 1"

    @property
    def levels(self) -> int:
        """L = 2^b - 1, the largest quantised value."""
        return (1 << self.bits) - 1

    @property
    def header_bytes(self) -> int:
        """Bytes of one (run, channel) header entry: 1 up to b = 4, else 2."""
        return 1 if self.bits <= 4 else 2

    def runs(self, n: int) -> int:
        """Number of runs in a block holding n tokens: ceil(n / R)."""
        return -(-n // self.run)
