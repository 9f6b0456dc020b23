"""Host logic of the 16-bit backward's dK/dV work plan (bwd_chunks.h,
compiled here with g++ alone): the items cover every step of every key tile
exactly once, the chunks of cut key tiles keep their partial sums inside
dq's memory without overlap, tiles of one chunk write directly, the
reduction's view of the plan matches the items', and the chosen chunk
length is the one its definition asks for (a brute-force search here)."""
import os
import subprocess

import pytest

from exact_attention_15_amd import build

CHECKER = r"""
#include <cstdio>
#include <cstdlib>
#include <vector>
#include "bwd_chunks.h"
using namespace attn::bwdplan;

// Prints "chunk items" for the plan, then "ok" or the first broken invariant.
int main(int argc, char** argv) {
    const long long N = atoll(argv[1]);
    const int G = atoi(argv[2]), BH_kv = atoi(argv[3]), causal = atoi(argv[4]), D = atoi(argv[5]);
    const int target = atoi(argv[6]);
    const int chunk = choose_chunk(N, G, BH_kv, causal != 0, target);
    const int n_qs = n_query_stages(N), n_kt = n_key_tiles(N);
    if (chunk == 0) { printf("0 %lld\nok\n", (long long)n_kt * BH_kv); return 0; }
    const long long items = plan_items(N, G, BH_kv, causal != 0, chunk);
    printf("%d %lld\n", chunk, items);
    // dq's memory: B*H*N*D 16-bit values = BH_kv*G*N*D/2 floats.
    const long long cap = (long long)BH_kv * G * N * D / 2;
    std::vector<unsigned char> used(cap, 0);
    std::vector<std::vector<int>> seen(n_kt * (size_t)BH_kv);
    for (int kt = 0; kt < n_kt; ++kt)
        for (int s = 0; s < BH_kv; ++s) seen[kt * (size_t)BH_kv + s].assign(kv_steps(G, n_qs, kt, causal != 0), 0);
    for (long long w = 0; w < items; ++w) {
        const Item it = locate((int)w, N, G, BH_kv, causal != 0, chunk);
        if (!it.valid) { printf("item %lld not located\n", w); return 1; }
        if (it.s1 <= it.s0 || it.s1 - it.s0 > chunk) { printf("item %lld length\n", w); return 1; }
        std::vector<int>& sv = seen[it.kt * (size_t)BH_kv + it.slice];
        for (int s = it.s0; s < it.s1; ++s) sv[s] += 1;
        const int nc = n_chunks(kv_steps(G, n_qs, it.kt, causal != 0), chunk);
        if (it.partial != (nc > 1)) { printf("item %lld: direct/partial mismatch\n", w); return 1; }
        if (!it.partial) {
            if (it.s0 != 0 || it.s1 != (int)sv.size()) { printf("item %lld: direct item not a whole tile\n", w); return 1; }
            continue;
        }
        const int rows = tile_rows(N, it.kt);
        const long long blk = (it.part_row * BH_kv + (long long)it.slice * rows) * 2 * D;
        if (blk < 0 || blk + 2LL * rows * D > cap) { printf("item %lld partials out of dq\n", w); return 1; }
        for (long long e = blk; e < blk + 2LL * rows * D; ++e) {
            if (used[e]) { printf("item %lld partials overlap\n", w); return 1; }
            used[e] = 1;
        }
        // The reduction reads chunk (s0 / chunk) of the key tile at the same block.
        const int first = first_chunk(it.kt, N, G, causal != 0, chunk);
        const long long blk_r = (((long long)first * kKeyBlock + (long long)(it.s0 / chunk) * rows) * BH_kv +
                                 (long long)it.slice * rows) * 2 * D;
        if (blk_r != blk || it.s0 % chunk != 0) { printf("item %lld: reduction sees another block\n", w); return 1; }
    }
    if (locate((int)items, N, G, BH_kv, causal != 0, chunk).valid) { printf("item past the plan located\n"); return 1; }
    for (size_t i = 0; i < seen.size(); ++i)
        for (size_t s = 0; s < seen[i].size(); ++s)
            if (seen[i][s] != 1) { printf("tile %zu step %zu covered %d times\n", i, s, seen[i][s]); return 1; }
    printf("ok\n");
    return 0;
}
"""


@pytest.fixture(scope="module")
def checker(tmp_path_factory):
    d = tmp_path_factory.mktemp("plan")
    src = d / "plan.cpp"
    src.write_text(CHECKER)
    exe = d / "plan"
    subprocess.run(["g++", "-std=c++17", "-O1", "-I", build.CSRC, str(src), "-o", str(exe)],
                   check=True)
    return str(exe)


def _run(checker, N, G, BH_kv, causal, D=128, target=512):
    r = subprocess.run([checker, str(N), str(G), str(BH_kv), str(int(causal)), str(D), str(target)],
                       capture_output=True, text=True, timeout=60)
    lines = r.stdout.split()
    assert r.returncode == 0 and r.stdout.strip().endswith("ok"), r.stdout
    return int(lines[0]), int(lines[1])


def _expected_chunk(N, G, BH_kv, causal, target=512):
    """The plan's definition, searched by brute force: the shortest chunk
    length L whose items (over all K/V slices) number at most `target` and
    whose partial rows (key tiles cut into two or more chunks only) fit
    G*N/4 rows, kept only if L cuts the longest key tile to <= 3/4 of its
    steps."""
    kb, qs = 128, 64
    n_qs = -(-N // qs)
    n_kt = -(-N // kb)
    steps = [G * (n_qs - 2 * kt if causal else n_qs) for kt in range(n_kt)]
    rows = [min(kb, N - kt * kb) for kt in range(n_kt)]
    for L in range(1, 3 * steps[0] // 4 + 1):
        items = BH_kv * sum(-(-w // L) for w in steps)
        if items <= target and sum(-(-w // L) * r for w, r in zip(steps, rows) if w > L) <= G * N // 4:
            return L
    return 0


SHAPES = [
    # N, G, BH_kv, causal
    (1, 8, 1, True), (65, 16, 1, True), (130, 8, 1, True), (257, 8, 2, True), (1111, 8, 1, True),
    (1111, 8, 1, False), (2048, 16, 1, True), (2048, 16, 1, False), (4096, 8, 16, True),
    (4096, 4, 16, True), (4096, 1, 64, True), (3000, 32, 3, True), (8192, 32, 1, True),
    (8192, 32, 1, False), (16384, 64, 1, True), (777, 2, 5, False),
]


@pytest.mark.parametrize("N,G,BH_kv,causal", SHAPES)
def test_plan_covers_steps_and_fits_dq(checker, N, G, BH_kv, causal):
    chunk, items = _run(checker, N, G, BH_kv, causal)
    assert chunk == _expected_chunk(N, G, BH_kv, causal)
    if chunk:
        # D = 64 partials take half the floats of D = 128: the same plan fits.
        assert _run(checker, N, G, BH_kv, causal, D=64) == (chunk, items)


def test_plan_for_multi_query_d128():
    """32 query heads on one K/V head, N = 8192, causal: one round of at
    most 512 items of ~270 steps instead of whole key tiles (up to 4096
    steps), the partial sums within dq's memory."""
    n_kt, n_qs, G = 64, 128, 32
    L = _expected_chunk(8192, G, 1, True)
    steps = [G * (n_qs - 2 * kt) for kt in range(n_kt)]
    n_items = sum(-(-w // L) for w in steps)
    cut_rows = sum(-(-w // L) * 128 for w in steps if w > L)
    assert 256 < L < 300 and 480 < n_items <= 512
    assert cut_rows <= G * 8192 // 4


def test_no_plan_when_items_fill_the_device(checker):
    """Four query heads per K/V head, B*H_kv = 16, N = 4096, causal: the 512
    whole key tiles already fill one round, and cutting any of them would
    start a second round, so whole key tiles are kept."""
    assert _run(checker, 4096, 4, 16, True) == (0, 512)


def test_no_plan_without_grouped_heads(checker):
    """One query head per K/V head: dq's memory holds partial sums for a
    quarter of the key tiles, too few to cut the long ones in two, so whole
    key tiles are kept."""
    for N in (64, 1000, 4096, 65536):
        assert _run(checker, N, 1, 4, True)[0] == 0


def test_plan_for_the_two_group_kernel(checker):
    """At d = 64 grouped-query items run in the three-group kernel, one per
    compute unit (256 at once): its plan keeps to 256 items, so one round.
    B*H_kv = 4, G = 16, N = 4096, causal."""
    chunk, items = _run(checker, 4096, 16, 4, True, D=64, target=256)
    assert chunk == _expected_chunk(4096, 16, 4, True, target=256) and items <= 256
    assert chunk > _expected_chunk(4096, 16, 4, True, target=512) > 0


GROUPS_CHECKER = r"""
#include <cstdio>
#include <cstdlib>
#include "bwd_chunks.h"
using namespace attn::bwdplan;
int main(int argc, char** argv) {
    const int D = atoi(argv[1]), causal = atoi(argv[2]), G = atoi(argv[3]);
    const long long N = atoll(argv[4]);
    const int BH_kv = atoi(argv[5]);
    const int groups = dkdv_groups(D, causal != 0, G, N, BH_kv, 256);
    printf("%d %d\n", groups, dkdv_resident(D, groups, 256));
    return 0;
}
"""


@pytest.fixture(scope="module")
def groups_checker(tmp_path_factory):
    d = tmp_path_factory.mktemp("groups")
    src = d / "groups.cpp"
    src.write_text(GROUPS_CHECKER)
    exe = d / "groups"
    subprocess.run(["g++", "-std=c++17", "-O1", "-I", build.CSRC, str(src), "-o", str(exe)],
                   check=True)
    return str(exe)


@pytest.mark.parametrize("D,causal,G,N,BH_kv,want", [
    # non-causal multi-head d = 64: one group while its rounds of 768 fill
    (64, 0, 1, 1280, 64, (1, 768)),      # B1 H64 N1280: 640 items
    (64, 0, 1, 8192, 64, (1, 768)),      # B4 H16 N8192: 4096 items
    (64, 0, 1, 2048, 48, (1, 768)),      # 768 items, one full round
    (64, 0, 1, 16384, 8, (3, 256)),      # 1024 items: second round of 768 mostly empty
    (64, 0, 1, 300, 12, (3, 256)),       # 36 items
    (64, 0, 1, 4096, 8, (3, 256)),       # 256 items
    # causal and grouped-query items, and d = 128
    (64, 1, 1, 4096, 64, (1, 768)),
    (64, 1, 4, 4096, 16, (3, 256)),
    (64, 0, 2, 1280, 32, (3, 256)),
    (128, 0, 1, 16384, 8, (1, 512)),
    (128, 1, 32, 8192, 1, (1, 512)),
])
def test_dkdv_group_choice(groups_checker, D, causal, G, N, BH_kv, want):
    """Which dK/dV kernel a call runs (the one-group or the three-group one)
    and the resident-workgroup count its plan targets."""
    r = subprocess.run([groups_checker, str(D), str(causal), str(G), str(N), str(BH_kv)],
                       check=True, capture_output=True, text=True)
    assert tuple(int(x) for x in r.stdout.split()) == want
