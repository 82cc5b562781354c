"""Host-only check of the expert-GEMM launch plan (csrc/plan.h): whenever a
shape is sent to the many-row kernel, no workgroup of its persistent grid
(G workgroups per wave, big_grid_mult waves) gets more work items than the
four descriptor registers it keeps (256), in either mode, for the
worst-case spread of rows over experts.

The plan header is plain C++; a tiny driver built with g++ prints its
decisions.  The item count of the kernel is recomputed here from the
kernel's own tiling rules (m-tiles of 256 rows per expert, 128 H columns per
gate/up tile, 256 output columns per down tile, a half-empty last round cut
into row slices), independently of the header's bound."""

import itertools
import os
import subprocess
import tempfile

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "sparse_moe_layer_03_amd", "csrc")

DRIVER = r"""
#include <stdio.h>
#include "plan.h"
int main() {
  long T, k, N, Z, d, dff, bf16, gather, G;
  while (scanf("%ld %ld %ld %ld %ld %ld %ld %ld %ld", &T, &k, &N, &Z, &d, &dff, &bf16,
               &gather, &G) == 9) {
    printf("%d %ld %d %ld\n", (int)moe::plan::ffn_use_big(T, k, N, Z, d, dff, bf16 != 0, gather != 0, G),
           moe::plan::big_mtiles_max(T * k, N), (int)moe::plan::ffn_use_r320(T, k, N, d, dff, G),
           moe::plan::big_grid_mult(T, k, N, d, dff, G));
  }
  return 0;
}
"""


@pytest.fixture(scope="module")
def plan_driver():
    d = tempfile.mkdtemp(prefix="moe_plan_")
    src, exe = os.path.join(d, "drv.cpp"), os.path.join(d, "drv")
    with open(src, "w") as f:
        f.write(DRIVER)
    subprocess.run(["g++", "-std=c++17", "-O1", f"-I{CSRC}", src, "-o", exe], check=True)

    def run(rows):
        inp = "\n".join(" ".join(str(v) for v in r) for r in rows) + "\n"
        out = subprocess.run([exe], input=inp, capture_output=True, text=True, check=True).stdout
        return [tuple(int(v) for v in ln.split()) for ln in out.splitlines()]
    return run


def cdiv(a, b):
    return -(-a // b)


def kernel_items_per_wg(counts, ntiles, G, rows=256):
    """Largest number of work items any workgroup runs, by the kernel's rules
    (m-tiles of `rows` rows per group)."""
    mt = sum(cdiv(int(c), rows) for c in counts)
    tiles = mt * ntiles
    full = tiles - tiles % G
    rem = tiles - full
    f = min(8, G // rem) if (rem > 0 and 2 * rem <= G) else 1
    total = full + rem * f
    return cdiv(total, G)


def worst_counts(rows, n_groups):
    """Rows spread over the groups so that the m-tile count is largest."""
    if rows <= n_groups:
        return [1] * rows + [0] * (n_groups - rows)
    c = [1] * n_groups
    extra = rows - n_groups
    c[0] += (extra // 256) * 256
    return c


def test_mtile_bound_is_the_brute_force_maximum():
    # every composition of a few rows over a few groups, tile height 256
    # scaled down: compare the closed form on rows up to 3 tiles
    for n_groups in (1, 2, 3):
        for rows in (0, 1, 2, 255, 256, 257, 511, 512, 513, 770):
            best = 0
            step = 1 if rows <= 3 else max(1, rows // 40)
            vals = sorted(set(list(range(0, rows + 1, step)) + [1, 255, 256, 257, rows]))
            for comb in itertools.product([v for v in vals if v <= rows], repeat=n_groups - 1):
                last = rows - sum(comb)
                if last < 0:
                    continue
                best = max(best, sum(cdiv(c, 256) for c in list(comb) + [last]))
            # the host plan's bound for this case (T = rows, k = 1)
            mx = rows if rows <= n_groups else n_groups + (rows - n_groups) // 256
            assert best <= mx, (n_groups, rows, best, mx)
            assert sum(cdiv(c, 256) for c in worst_counts(rows, n_groups)) == mx


SHAPES = [
    # T, k, N, Z, d_model, d_ff
    (16384, 12, 512, 256, 6144, 2048),    # prefill
    (32768, 12, 512, 256, 6144, 2048),    # twice the prefill batch
    (65536, 12, 512, 256, 6144, 2048),    # four times: two waves of workgroups
    (8192, 8, 256, 128, 4096, 1536),      # skewed
    (4096, 8, 64, 32, 2048, 1024),        # small
    (2048, 4, 16, 8, 512, 384),
    (6_000_000 // 8, 8, 64, 0, 640, 256),  # d_model % 256 == 128: down has ceil(d/256) n-tiles
    (400_000, 8, 64, 0, 640, 256),
    (694_000, 8, 64, 0, 640, 256),        # just inside the 256-item limit
    (1_000_000, 4, 1024, 0, 384, 128),
    (60_000, 16, 1000, 24, 128, 1024),
    (200_000, 16, 1024, 0, 128, 4096),
]


@pytest.mark.parametrize("G", [256, 248, 64, 8])
def test_many_row_kernel_items_fit_the_descriptor_registers(plan_driver, G):
    rows = [(T, k, N, Z, d, dff, 1, 1, G) for (T, k, N, Z, d, dff) in SHAPES]
    res = plan_driver(rows)
    rng = np.random.default_rng(G)
    n_big, most = 0, 0
    for (T, k, N, Z, d, dff), (big, mt_max, _, mult) in zip(SHAPES, res):
        if not big:
            continue
        n_big += 1
        assert 1 <= mult <= 64
        if mult > 1:   # the smallest multiple: one wave fewer would not fit
            assert cdiv(mt_max * max(cdiv(dff, 128), cdiv(d, 256)), G * (mult - 1)) > 256
        Tk = T * k
        dists = [worst_counts(Tk, N), rng.multinomial(Tk, np.full(N, 1.0 / N)),
                 rng.multinomial(Tk, rng.dirichlet(np.full(N, 0.3)))]
        for counts in dists:
            assert sum(cdiv(int(c), 256) for c in counts) <= mt_max
            for ntiles in (cdiv(dff, 128), cdiv(d, 256)):     # gate/up, down
                items = kernel_items_per_wg(counts, ntiles, G * mult)
                most = max(most, items)
                assert items <= 256, (T, k, N, d, dff, G)
    if G == 256:
        # the bound is exercised, not vacuous: several shapes take the kernel
        # and one of them comes within a few items of the limit
        assert n_big >= 5 and most >= 240, (n_big, most)


def test_plan_refuses_shapes_past_the_limits(plan_driver):
    res = plan_driver([
        (16384, 12, 512, 256, 6144, 2048, 0, 1, 256),   # fp32: never the bf16 kernel
        (16384, 12, 512, 256, 6144, 2048, 1, 1, 256),   # the prefill batch: yes
        (400_000, 12, 512, 256, 6144, 2048, 1, 1, 256),  # x of 4.9 GB, gathered: no
        (400_000, 12, 512, 256, 6144, 2048, 1, 0, 256),  # same rows contiguous: tile count decides
        (6_000_000 // 8, 8, 64, 0, 640, 256, 1, 1, 256),
        (32768, 12, 512, 256, 6144, 2048, 1, 1, 256),   # twice the prefill batch: yes
        (65536, 12, 512, 256, 6144, 2048, 1, 1, 256),   # four times: yes, two waves
        (1_000_000, 16, 1024, 0, 128, 4096, 1, 1, 8),   # 8 CUs: more than 64 waves needed
    ])
    assert res[0][0] == 0 and res[1][0] == 1 and res[2][0] == 0
    assert res[1][3] == 1 and res[5][3] == 1
    # 6M assignments at d_model 640: the down GEMM's 3 n-tiles per m-tile
    # would give a workgroup of a one-wave grid more than 256 items; two
    # waves of workgroups hold them
    mt = res[4][1]
    assert cdiv(mt * 3, 256) > 256 and res[4][0] == 1 and res[4][3] == 2
    assert res[5][0] == 1
    assert res[6][0] == 1 and res[6][3] == 2
    assert res[7][0] == 0 and res[7][3] == 0


def counts_320(Tk, N, rng):
    """Row spreads with as many groups of 257..320 rows as the rows allow."""
    n = min(N, Tk // 257)
    c = np.zeros(N, dtype=np.int64)
    c[:n] = 257
    c[0] += Tk - 257 * n          # the rest on one group (a 256-row tile group)
    return [c, rng.multinomial(Tk, np.full(N, 1.0 / N))]


@pytest.mark.parametrize("G", [256, 64, 8])
def test_320_row_kernel_items_fit_the_descriptor_registers(plan_driver, G):
    """When a shape also uses the 320 x 192 tiles (experts of 257..320 rows),
    that launch's work items per workgroup stay within the 256 descriptor
    slots in both modes, and the 256-row launch's (which skips those
    experts) too, on the grid both launches share."""
    rows = [(T, k, N, Z, d, dff, 1, 1, G) for (T, k, N, Z, d, dff) in SHAPES]
    res = plan_driver(rows)
    rng = np.random.default_rng(7 + G)
    used = 0
    for (T, k, N, Z, d, dff), (big, _, r320, mult) in zip(SHAPES, res):
        if not (big and r320):
            continue
        used += 1
        for counts in counts_320(T * k, N, rng):
            tall = [int(c) for c in counts if 257 <= c <= 320]
            rest = [int(c) for c in counts if not 257 <= c <= 320]
            for nt320, nt256 in ((cdiv(dff, 96), cdiv(dff, 128)), (cdiv(d, 192), cdiv(d, 256))):
                # both launches run on the same grid of G * mult workgroups
                assert kernel_items_per_wg(tall, nt320, G * mult, rows=320) <= 256
                assert kernel_items_per_wg(rest, nt256, G * mult) <= 256
    if G == 256:
        assert used >= 3, used


def test_grid_multiple_over_random_shapes(plan_driver):
    """Seeded random shapes and CU counts: whenever the plan takes the
    many-row kernel, the worst-case and sampled row spreads keep every
    workgroup of the G * mult grid within 256 items in both modes, and one
    wave fewer would not."""
    rng = np.random.default_rng(2024)
    rows, shapes = [], []
    for _ in range(300):
        N = int(rng.choice([8, 64, 256, 512, 1000, 1024]))
        Z = int(rng.integers(0, 1025 - N))
        k = int(rng.integers(1, min(16, N + Z) + 1))
        d = 128 * int(rng.integers(1, 65))
        dff = 128 * int(rng.integers(1, 65))
        T = int(rng.integers(1, min(2 ** 31 // k - 1, 3_000_000)))
        G = int(rng.choice([8, 32, 64, 248, 256]))
        rows.append((T, k, N, Z, d, dff, 1, 0, G))
        shapes.append((T, k, N, Z, d, dff, G))
    res = plan_driver(rows)
    n_big = n_mult = 0
    for (T, k, N, Z, d, dff, G), (big, mt_max, _, mult) in zip(shapes, res):
        if not big:
            continue
        n_big += 1
        n_mult += mult > 1
        assert 1 <= mult <= 64
        nt = max(cdiv(dff, 128), cdiv(d, 256))
        assert cdiv(mt_max * nt, G * mult) <= 256
        if mult > 1:
            assert cdiv(mt_max * nt, G * (mult - 1)) > 256
        Tk = T * k
        for counts in (worst_counts(Tk, N), rng.multinomial(Tk, np.full(N, 1.0 / N))):
            for ntiles in (cdiv(dff, 128), cdiv(d, 256)):
                assert kernel_items_per_wg(counts, ntiles, G * mult) <= 256, (T, k, N, d, dff, G)
    assert n_big >= 50 and n_mult >= 10, (n_big, n_mult)
