"""The query rows a key tile's dK/dV workgroup streams (query_rows_seeing in
common.hpp), built for the host and checked on random masks: the closed forms
(no mask, causal, sliding window with and without sink tokens) and the
document search give the same range as binary searches over row_interval,
and every row that sees a key of the tile (brute force over rows and keys
with row_interval's interval plus the sink keys) lies inside the range."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "exact_io_aware_fwd_amd", "csrc")
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"

PROGRAM = r"""
#include "common.hpp"
#include <cstdio>
#include <cstdlib>
#include <vector>
using namespace xattn;

static unsigned long long rng = 88172645463325252ull;
static int rnd(int n) { rng ^= rng << 13; rng ^= rng >> 7; rng ^= rng << 17; return (int)(rng % (unsigned long long)n); }

int main() {
    int cases = 0, bad = 0;
    for (int t = 0; t < 40000; ++t) {
        PrefillParams p{};
        p.mask_kind = rnd(4);
        p.Nq = 1 + rnd(t % 4 == 0 ? 2000 : 300);
        p.Nk = 1 + rnd(t % 4 == 0 ? 2000 : 300);
        p.window = 0;
        p.sink_end = 0;
        std::vector<int32_t> off;
        if (p.mask_kind == kMaskWindow) {
            int w = 1 + rnd(p.Nk + 20);
            p.window = w < p.Nk ? w : p.Nk;   // clamped as the library does
            if (rnd(2)) p.sink_end = 1 + rnd(p.Nk);
        }
        if (p.mask_kind == kMaskDocument) {
            off.push_back(0);
            while (off.back() < p.Nk) off.push_back(off.back() + 1 + rnd(60));
            off.back() = p.Nk;
            p.doc_offsets = off.data();
            p.num_docs = (int)off.size() - 1;
        }
        const int bk = rnd(2) ? 128 : 32;
        for (int k0 = 0; k0 < p.Nk; k0 += bk) {
            const int k_last = (k0 + bk < p.Nk ? k0 + bk : p.Nk) - 1;
            int first, last;
            query_rows_seeing(p, k0, k_last, first, last);
            // binary searches over row_interval
            int a = 0, z = p.Nq;
            while (a < z) { int mid = (a + z) >> 1, l, h; row_interval(p, mid, l, h); if (h >= k0) z = mid; else a = mid + 1; }
            int f2 = a, l2;
            if (k0 < p.sink_end) l2 = p.Nq - 1;
            else {
                a = -1; z = p.Nq - 1;
                while (a < z) { int mid = (a + z + 1) >> 1, l, h; row_interval(p, mid, l, h); if (l <= k_last) a = mid; else z = mid - 1; }
                l2 = a;
            }
            // brute force: rows that see a key of the tile lie inside [first, last]
            int outside = 0, seen = 0;
            for (int i = 0; i < p.Nq; ++i) {
                int l, h;
                row_interval(p, i, l, h);
                bool sees = false;
                for (int k = k0; k <= k_last && !sees; ++k)
                    sees = k <= h && (k >= l || k < p.sink_end);
                if (sees) { ++seen; if (i < first || i > last) ++outside; }
            }
            ++cases;
            if (first != f2 || last != l2 || outside) {
                if (bad < 10) printf("BAD kind %d Nq %d Nk %d W %d sink %d k0 %d: %d %d vs %d %d, outside %d\n",
                                     p.mask_kind, p.Nq, p.Nk, p.window, p.sink_end, k0, first, last, f2, l2, outside);
                ++bad;
            }
        }
    }
    printf("cases %d bad %d\n", cases, bad);
    return bad != 0;
}
"""


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not installed")
def test_query_rows_seeing_matches_searches_and_brute_force(tmp_path):
    src = tmp_path / "rows.cpp"
    exe = tmp_path / "rows"
    src.write_text(PROGRAM)
    subprocess.run([HIPCC, "-std=c++17", "-O2", "--cuda-host-only", "-x", "hip", "-I", CSRC,
                    "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)],
                   check=True, capture_output=True, timeout=300)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=600)
    print(r.stdout[-2000:])
    assert r.returncode == 0, r.stdout[-2000:]
    assert "bad 0" in r.stdout
