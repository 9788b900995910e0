"""Host-side argument logic (csrc/host_logic.h) compiled alone with g++ and
checked against brute force: strided-view overlap, access width, launch plan.
Built with AddressSanitizer and UndefinedBehaviorSanitizer (host code only)."""

from __future__ import annotations

import os
import shutil
import subprocess

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "swiglu_activation_amd", "csrc")

DRIVER = r'''
#include <cstdio>
#include <cstdint>
#include "host_logic.h"
using namespace swiglu_host;
int main() {
    char op;
    while (std::scanf(" %c", &op) == 1) {
        if (op == 'o') {
            unsigned long long pa, pb; long long sa, sb, wa, wb, rows, esz;
            std::scanf("%llu %lld %lld %llu %lld %lld %lld %lld", &pa, &sa, &wa, &pb, &sb, &wb, &rows, &esz);
            Operand a{(const void*)(uintptr_t)pa, sa}, b{(const void*)(uintptr_t)pb, sb};
            std::printf("%d\n", views_overlap(a, wa, b, wb, rows, esz) ? 1 : 0);
        } else if (op == 'v' || op == 'c') {
            // 'v': the access width; 'c': the columns the plan's vectors cover
            int esz, nops; long long n; std::scanf("%d %lld %d", &esz, &n, &nops);
            Operand ops[8];
            for (int i = 0; i < nops; ++i) {
                unsigned long long p; long long s; std::scanf("%llu %lld", &p, &s);
                ops[i] = Operand{(const void*)(uintptr_t)p, s};
            }
            const int vb = vec_bytes(esz, n, ops, nops);
            if (op == 'v') {
                std::printf("%d\n", vb);
            } else {
                const int vec = vb / esz;
                Plan P = make_plan(n, vec, 256, 65535);
                std::printf("%d %lld %lld\n", vec, (long long)P.nv * vec, (long long)P.rows_per_launch);
            }
        } else if (op == 'p') {
            long long n; int vec; unsigned block, maxgy;
            std::scanf("%lld %d %u %u", &n, &vec, &block, &maxgy);
            Plan P = make_plan(n, vec, block, maxgy);
            std::printf("%d %u %u %lld\n", P.wide ? 1 : 0, P.nv, P.tiles,
                        (long long)P.rows_per_launch);
        } else if (op == 'f') {
            long long rows; unsigned nv, block;
            std::scanf("%lld %u %u", &rows, &nv, &block);
            std::printf("%u\n", flat_blocks(rows, nv, block));
        } else if (op == 'F') {
            long long n, tf, tt, maxt, threads;
            std::scanf("%lld %lld %lld %lld %lld", &n, &tf, &tt, &maxt, &threads);
            std::printf("%lld\n", (long long)fc1_rows_per_launch(n, tf, tt, maxt, threads));
        } else if (op == 'P') {
            unsigned tiles; long long cus, threads;
            std::scanf("%u %lld %lld", &tiles, &cus, &threads);
            Fc1Pool q = fc1_pool(tiles, cus, threads);
            std::printf("%u %u\n", q.n_fixed, q.grid);
        }
    }
    return 0;
}
'''


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not available")
    d = tmp_path_factory.mktemp("hostlogic")
    src = d / "driver.cpp"
    src.write_text(DRIVER)
    exe = d / "driver"
    # The sanitizer runtime must be first in the process; where something is
    # preloaded, the driver is built without it.
    san = [] if os.environ.get("LD_PRELOAD") else ["-fsanitize=address,undefined",
                                                   "-fno-sanitize-recover=all"]
    subprocess.run([gxx, "-std=c++17", "-O1", "-g", *san, "-I", CSRC, str(src), "-o", str(exe)],
                   check=True)

    def run(lines):
        env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0")
        out = subprocess.run([str(exe)], input="\n".join(lines) + "\n", capture_output=True,
                             text=True, check=True, env=env)
        return out.stdout.split("\n")[:-1]
    return run


def _bytes_of(p, stride, width, rows, esz):
    s = set()
    for r in range(rows):
        base = p + r * stride * esz
        s.update(range(base, base + width * esz))
    return s


def test_view_overlap_bruteforce(driver):
    rng = np.random.default_rng(0)
    cases, want = [], []
    for _ in range(3000):
        esz = int(rng.choice([2, 4]))
        rows = int(rng.integers(1, 7))
        wa, wb = int(rng.integers(1, 9)), int(rng.integers(1, 9))
        same = rng.random() < 0.7
        sa = int(rng.integers(max(wa, 1), 20))
        sb = sa if same else int(rng.integers(max(wb, 1), 20))
        pa = 4096 + int(rng.integers(0, 64)) * esz
        pb = 4096 + int(rng.integers(0, 200)) * esz
        cases.append(f"o {pa} {sa} {wa} {pb} {sb} {wb} {rows} {esz}")
        truth = bool(_bytes_of(pa, sa, wa, rows, esz) & _bytes_of(pb, sb, wb, rows, esz))
        want.append((truth, sa == sb, cases[-1]))
    got = driver(cases)
    for g, (truth, exact, case) in zip(got, want):
        if exact:
            assert int(g) == int(truth), case       # exact for equal strides
        else:
            assert int(g) >= int(truth), case       # never misses a real overlap


def test_packed_halves_do_not_overlap(driver):
    # the two halves of a packed [rows, 2n] tensor, and a tensor next to it
    rows, n, esz, base = 8192, 32768, 2, 1 << 20
    got = driver([
        f"o {base} {2 * n} {n} {base + n * esz} {2 * n} {n} {rows} {esz}",
        f"o {base} {2 * n} {n + 1} {base + n * esz} {2 * n} {n} {rows} {esz}",
        f"o {base} {2 * n} {2 * n} {base + rows * 2 * n * esz} {n} {n} {rows} {esz}",
        f"o {base} {2 * n} {2 * n} {base + rows * 2 * n * esz - esz} {n} {n} {rows} {esz}",
    ])
    assert got == ["0", "1", "0", "1"]


def test_vec_bytes(driver):
    got = driver([
        "v 2 8 3 4096 8 8192 16 12288 8",    # all 16-byte aligned
        "v 2 8 2 4098 8 8192 16",            # pointer 2-byte aligned
        "v 2 8 2 4096 12 8192 16",           # stride 24 bytes -> 8
        "v 4 4 2 4096 3 8192 4",             # fp32 stride 12 bytes -> 4
        "v 2 8 1 4100 8",                    # pointer 4-byte aligned
        # padded two-tensor views: pointers and strides 16-byte aligned, but
        # the row width n is not a multiple of 16 bytes
        "v 4 5 3 4096 8 8192 8 12288 8",     # fp32 n=5 in rows of 8 -> 4 bytes
        "v 4 3 3 4096 4 8192 4 12288 4",     # fp32 n=3 in rows of 4 -> 4 bytes
        "v 2 12 3 4096 16 8192 16 12288 16",  # bf16 n=12 in rows of 16 -> 8 bytes
        "v 4 6 2 4096 8 8192 8",             # fp32 n=6 -> 8 bytes
        "v 2 1 2 4096 8 8192 8",             # bf16 n=1 -> one element
    ])
    assert got == ["16", "2", "8", "4", "4", "4", "4", "8", "8", "2"]


def test_plan_covers_every_column(driver):
    """For every n in [1, 300], both element sizes, and pointers and strides
    aligned to 16, 8, 4 or 2 bytes (two or five operands, as the two-tensor
    forward and backward pass them), the chosen vectors cover exactly n
    columns and the width divides every operand's alignment (brute force over
    the definition of the access width)."""
    rng = np.random.default_rng(11)
    cases, want = [], []
    for esz in (2, 4):
        for n in range(1, 301):
            for _ in range(4):
                nops = int(rng.choice([2, 3, 5]))
                ops = []
                for _ in range(nops):
                    pal = int(rng.choice([16, 8, 4, 2]))
                    pal = max(pal, esz)
                    p = 1 << 20
                    p += pal if rng.random() < 0.5 else 0           # aligned to pal exactly
                    p -= p % esz
                    extra = int(rng.integers(0, 9))
                    s = n + extra
                    ops.append((p, s))
                line = f"c {esz} {n} {nops} " + " ".join(f"{p} {s}" for p, s in ops)
                cases.append(line)
                # brute force: the largest b in {16, 8, 4, 2} (b >= esz) with
                # every pointer, every stride*esz and n*esz divisible by b
                b = esz
                for cand in (16, 8, 4):
                    if cand < esz:
                        continue
                    if (n * esz) % cand == 0 and all(p % cand == 0 and (s * esz) % cand == 0
                                                     for p, s in ops):
                        b = cand
                        break
                want.append(b // esz)
    got = driver(cases)
    for line, g, vec in zip(cases, got, want):
        gv, covered, rpl = (int(t) for t in g.split())
        assert gv == vec, line
        assert covered == int(line.split()[2]), line     # nv * VEC == n
        assert rpl > 0, line


def test_launch_plan(driver):
    got = driver(["p 32768 8 256 65535", "p 1792 8 256 65535", "p 11008 4 256 65535",
                  "p 1 1 256 65535", "p 2048 8 256 65535"])
    assert got[0] == "1 4096 16 65535"            # wide: 16 tiles per row
    assert got[1] == f"0 224 0 {2 ** 31 // 224}"   # narrow: flat, at most 2^31 lanes per launch
    assert got[2] == "1 2752 11 65535"            # ragged last tile
    assert got[3] == f"0 1 0 {2 ** 31}"
    assert got[4] == "1 256 1 65535"
    # flat grid: ceil(rows * nv / 256) blocks, and the largest launch stays below 2^23 blocks
    got = driver(["f 8192 224 256", "f 1 1 256", "f 3 100 256", f"f {2 ** 31 // 224} 224 256"])
    assert got == ["7168", "1", "2", str(-(-(2 ** 31 // 224) * 224 // 256))]


def test_flat_lane_to_row_division_is_exact():
    """The narrow-row kernels split a flat lane index L into (row, vector) as
    floor((L + 1/2) * fp64(1/nv)) and L - row * nv. Checked here in IEEE
    double (the same arithmetic as the GPU's fp64 ops) for every nv below 256,
    on lanes around every multiple of nv near 0 and near the top of the
    largest launch (2^31 / nv rows, plus one block of overshoot)."""
    import numpy as np
    for nv in range(1, 256):
        inv = 1.0 / nv
        top = (2 ** 31 // nv) * nv + 255
        ks = np.concatenate([np.arange(0, 64), np.arange(top // nv - 64, top // nv + 2)])
        L = (ks[:, None] * nv + np.arange(-2, 3)[None, :]).ravel()
        L = L[(L >= 0) & (L <= top)].astype(np.uint64)
        q = np.floor((L.astype(np.float64) + 0.5) * inv).astype(np.uint64)
        assert np.array_equal(q, L // nv), nv


@pytest.mark.parametrize("threads", [256, 512])
def test_fc1_launch_chunks(driver, threads):
    """fc1's token rows per launch: the largest whole number of 256-token
    tiles (at most 65535) whose grid of f_tiles x t_tiles workgroups stays
    below 2^32 work-items, for n across its whole range; 0 only where not
    one tile fits."""
    ns = sorted({64, 128, 192, 4096, 32768, 1 << 20, (1 << 23) + 64, (1 << 24) - 64,
                 (1 << 29) + 128, (1 << 30) - 128, 1 << 30}
                | {int(v) * 64 for v in np.random.default_rng(5).integers(1, 1 << 24, 40)})
    got = driver([f"F {n} 128 256 65535 {threads}" for n in ns])
    for n, line in zip(ns, got):
        rpl = int(line)
        f_tiles = -(-n // 128)
        fits = lambda t: f_tiles * t * threads < (1 << 32) and t <= 65535
        assert rpl % 256 == 0
        t = rpl // 256
        if t == 0:
            assert not fits(1), n
        else:
            assert fits(t) and not fits(t + 1), (n, t)
    # at the default 256 threads every n up to 2^30 gets at least one tile
    if threads == 256:
        assert all(int(line) > 0 for line in got)


def test_fc1_pool(driver):
    """fc1's tile pool: none without a workspace or below 16 tiles per CU;
    otherwise the fixed tiles are a multiple of 8, about three quarters of
    the launch, the pool workgroups are at least as many as the pool tiles
    (every tile is taken), and the grid stays below 2^32 work-items."""
    rng = np.random.default_rng(11)
    tiles = sorted({1, 7, 8, 4095, 4096, 4097, 8192, 8193, 65535, 1 << 20, (1 << 24) - 1}
                   | {int(t) for t in rng.integers(1, 1 << 24, 60)})
    # (a launch never holds more tiles than fit below 2^32 work-items)
    cases = [(t, c, th) for t in tiles for c in (0, 32, 256) for th in (256, 512)
             if t * th < (1 << 32)]
    got = driver([f"P {t} {c} {th}" for t, c, th in cases])
    for (t, c, th), line in zip(cases, got):
        n_fixed, grid = map(int, line.split())
        if c == 0 or t < 16 * c:
            assert (n_fixed, grid) == (t, t), (t, c)
            continue
        assert grid * th < (1 << 32), (t, c, th)
        if grid == t:                       # no room for a surplus: no pool
            assert n_fixed == t
            continue
        assert n_fixed % 8 == 0 and n_fixed < t, (t, c)
        pool = t - n_fixed
        assert abs(pool - t / 4) <= 16, (t, pool)
        assert grid - n_fixed > pool, (t, c, th)
        if t * th * 5 // 4 + 4096 * th < (1 << 32):
            assert grid - n_fixed >= pool + pool // 4, (t, c)
