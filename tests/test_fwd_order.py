"""Host logic of the forward kernels' work order (fwd_order.h, compiled here
with g++ alone): both orders visit every (query tile, slice) item exactly
once, pair each query slice with the K/V slice its head reads, and the
XCD-major order keeps an XCD's workgroups on its own K/V slices, each
slice's tiles longest first."""
import subprocess

import pytest

from exact_attention_15_amd import build

CHECKER = r"""
#include <cstdio>
#include <cstdlib>
#include <vector>
#include "fwd_order.h"
using namespace attn::fwdorder;
int main(int argc, char** argv) {
    const int B = atoi(argv[1]), H = atoi(argv[2]), H_kv = atoi(argv[3]), n_qtiles = atoi(argv[4]);
    const int xcd = atoi(argv[5]);
    const int G = H / H_kv, BH = B * H, BH_kv = B * H_kv;
    const long long total = (long long)BH * n_qtiles;
    std::vector<int> seen(total, 0);
    std::vector<int> last_tile(BH_kv * G, 1 << 30);
    for (long long w = 0; w < total; ++w) {
        const Item it = item(xcd != 0, (int)w, n_qtiles, BH, BH_kv, H_kv, G);
        if (it.tile < 0 || it.tile >= n_qtiles || it.bh < 0 || it.bh >= BH) { printf("item %lld out of range\n", w); return 1; }
        const int b = it.bh / H, h = it.bh % H;
        if (it.kv_bh != b * H_kv + h / G) { printf("item %lld: wrong K/V slice\n", w); return 1; }
        if (seen[(long long)it.bh * n_qtiles + it.tile]++) { printf("item %lld visited twice\n", w); return 1; }
        if (xcd) {
            if (it.kv_bh % kXcds != (int)(w % kXcds)) { printf("item %lld on another XCD\n", w); return 1; }
            if (it.tile > last_tile[it.bh]) { printf("item %lld: tiles not longest first\n", w); return 1; }
            last_tile[it.bh] = it.tile;
        }
    }
    printf("ok\n");
    return 0;
}
"""


@pytest.fixture(scope="module")
def checker(tmp_path_factory):
    d = tmp_path_factory.mktemp("order")
    src = d / "order.cpp"
    src.write_text(CHECKER)
    exe = d / "order"
    subprocess.run(["g++", "-std=c++17", "-O1", "-I", build.CSRC, str(src), "-o", str(exe)],
                   check=True)
    return str(exe)


@pytest.mark.parametrize("B,H,H_kv,n_qtiles", [
    (4, 16, 16, 16), (1, 32, 32, 32), (1, 8, 8, 32), (4, 16, 4, 16), (1, 32, 1, 32),
    (2, 12, 4, 7), (3, 5, 5, 3), (1, 1, 1, 1), (2, 64, 64, 2), (8, 8, 8, 5),
])
@pytest.mark.parametrize("xcd", [0, 1])
def test_order_visits_every_item_once(checker, B, H, H_kv, n_qtiles, xcd):
    if xcd and (B * H_kv) % 8 != 0:
        pytest.skip("the XCD-major order needs a multiple of 8 K/V slices")
    r = subprocess.run([checker, str(B), str(H), str(H_kv), str(n_qtiles), str(xcd)],
                       capture_output=True, text=True)
    assert r.returncode == 0 and r.stdout.strip() == "ok", r.stdout
