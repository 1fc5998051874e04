"""The synthetic workloads: five measured configurations, then two volumes of
2^20 and 2^22 tokens for the million-token reach.

Grid is (Z, Y, X) with x fastest in raster order; block is (bz, by, bx).
"""
from dataclasses import dataclass, field
from typing import Tuple


@dataclass(frozen=True)
class Workload:
    wid: int
    name: str
    grid: Tuple[int, int, int]
    B: int
    H: int
    D: int
    block: Tuple[int, int, int]
    dtype: str               # "f32" or "bf16"
    values: str              # "iid" or "smooth"
    packing: str             # packing of the primary run
    repack: str              # packing of the equivariance check
    rope_base: float = 10000.0
    Hkv: int = 0             # key/value heads (grouped-query attention); 0 means H

    @property
    def kv_heads(self) -> int:
        return self.Hkv if self.Hkv > 0 else self.H

    @property
    def N(self) -> int:
        z, y, x = self.grid
        return z * y * x

    @property
    def M(self) -> int:
        return _ceil(self.grid[0], self.block[0]) * _ceil(self.grid[1], self.block[1]) * \
            _ceil(self.grid[2], self.block[2])

    @property
    def tokens(self) -> int:
        return self.B * self.N

    def seed(self, what: str) -> int:
        return 1000 * self.wid + {"q": 0, "k": 1, "v": 2, "g": 3, "perm": 4, "perm2": 5,
                                  "dout": 6}[what]


def _ceil(a: int, b: int) -> int:
    return -(-a // b)


WORKLOADS = {
    1: Workload(1, "grid8_fp32", (8, 8, 8), 1, 1, 24, (2, 2, 2), "f32", "iid", "raster", "morton"),
    2: Workload(2, "grid16_bf16", (16, 16, 16), 2, 4, 48, (2, 2, 2), "bf16", "iid", "morton", "block"),
    3: Workload(3, "grid32x32x64_bf16", (32, 32, 64), 1, 8, 48, (2, 2, 2), "bf16", "iid", "block", "group"),
    4: Workload(4, "grid64_bf16_random", (64, 64, 64), 1, 8, 48, (4, 4, 4), "bf16", "iid", "random", "random2"),
    5: Workload(5, "grid16x64x64_bf16_smooth", (16, 64, 64), 4, 4, 96, (2, 2, 4), "bf16", "smooth", "block", "raster"),
    # million-token reach: 2^20 tokens with 4,096 summaries per head (256
    # tokens per 4x8x8 block), and 2^22 tokens at the same block volume
    6: Workload(6, "grid64x128x128_bf16_1m", (64, 128, 128), 1, 8, 48, (4, 8, 8), "bf16", "iid", "block", "random"),
    7: Workload(7, "grid128x128x256_bf16_4m", (128, 128, 256), 1, 8, 48, (4, 8, 8), "bf16", "iid", "block", "random"),
    # 2^23 tokens, 32,768 summaries per head: a token tensor holds 3.2e9
    # elements, past 32-bit element offsets
    8: Workload(8, "grid128x256x256_bf16_8m", (128, 256, 256), 1, 8, 48, (4, 8, 8), "bf16", "iid", "block", "random"),
}


def workload(wid: int) -> Workload:
    return WORKLOADS[wid]
