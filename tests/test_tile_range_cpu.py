"""The byte range of a tile's buffer resource (tile_range_bytes in
prefill_tiles.hpp), built for the host and checked against its definition:
the rows of the tile that exist, rows = Nk - n0 clamped to [0, tile rows],
times d * 2 bytes.  The values near 2^23 and 2^24 rows are where the
unclamped rows * d * 2 (d = 128) leaves 32 bits; 2^28 is the largest length
the library accepts."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "exact_io_aware_fwd_amd", "csrc")
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"

PROGRAM = r"""
#include "prefill_tiles.hpp"
#include <cstdio>
int main() {
    const long long rows[] = {%s};
    for (long long r : rows)
        printf("%%lld %%u %%u %%u\n", r, xattn::tile_range_bytes<128>((int)r, 64),
               xattn::tile_range_bytes<64>((int)r, 64), xattn::tile_range_bytes<128>((int)r, 32));
    return 0;
}
"""

ROWS = [-(1 << 20), -5, -1, 0, 1, 31, 32, 33, 37, 63, 64, 65, 4096,
        (1 << 23) - 1, 1 << 23, (1 << 23) + 1, (1 << 24) - 1, 1 << 24, (1 << 24) + 1, (1 << 28) - 1, 1 << 28]


def expected(rows: int, d: int, tile_rows: int) -> int:
    return min(max(rows, 0), tile_rows) * d * 2


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not installed")
def test_tile_range_bytes_near_32_bit_limits(tmp_path):
    src = tmp_path / "range.cpp"
    exe = tmp_path / "range"
    src.write_text(PROGRAM % ", ".join(f"{r}LL" for r in ROWS))
    subprocess.run([HIPCC, "-std=c++17", "--cuda-host-only", "-x", "hip", "-I", CSRC,
                    "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)],
                   check=True, capture_output=True, timeout=300)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True, timeout=60).stdout.split("\n")
    lines = [ln.split() for ln in out if ln.strip()]
    assert len(lines) == len(ROWS)
    for r, line in zip(ROWS, lines):
        got = [int(x) for x in line]
        assert got[0] == r
        assert got[1] == expected(r, 128, 64), (r, got)
        assert got[2] == expected(r, 64, 64), (r, got)
        assert got[3] == expected(r, 128, 32), (r, got)
