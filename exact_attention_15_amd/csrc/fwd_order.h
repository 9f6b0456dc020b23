// fwd_order.h — the order in which the forward kernels take their work items
// (one query tile of one (b, h) slice each), as plain constexpr functions:
// the kernels call them on the device and a host test compiles this header
// with g++ alone to check that every order visits every item exactly once.
//
// Workgroup w runs on XCD w % 8 (the dispatcher deals workgroups out to the
// 8 XCDs in turn) and each XCD starts its workgroups in the order of their
// ids, so the order decides both the balance (longest query tiles first
// under a causal mask) and which K/V slices share an XCD's 4 MB L2 at once.
#ifndef ATTN_FWD_ORDER_H
#define ATTN_FWD_ORDER_H

#include <stdint.h>

namespace attn {
namespace fwdorder {

constexpr int kXcds = 8;

struct Item {
    int tile;    // query tile
    int bh;      // query slice b*H + h
    int kv_bh;   // key/value slice b*H_kv + h / G
};

// Query slice and K/V slice of slice index r in [0, BH): the G query heads
// of one K/V head take r = kv, kv + BH_kv, kv + 2 BH_kv, ... (the same
// position modulo 8 whenever BH_kv is a multiple of 8).
constexpr Item slice_item(int tile, int r, int BH_kv, int H_kv, int G) {
    const int kv_bh = r % BH_kv;
    const int g = r / BH_kv;
    const int b = kv_bh / H_kv;
    const int h = (kv_bh - b * H_kv) * G + g;
    return {tile, b * H_kv * G + h, kv_bh};
}

// Tile-major order: the longest query tiles of every slice first, then the
// next, consecutive ids on different slices. Every slice is spread over all
// XCDs' rounds: an XCD runs BH / 8 slices at once.
constexpr Item tile_major(int w, int n_qtiles, int BH, int BH_kv, int H_kv, int G) {
    const int t = w / BH;
    return slice_item(n_qtiles - 1 - t, w - t * BH, BH_kv, H_kv, G);
}

// XCD-major order (needs BH_kv % 8 == 0): XCD x takes the K/V slices
// x, x + 8, x + 16, ... one after another, and for each of them the query
// tiles of all G query heads reading it, longest first. An XCD then holds
// as few K/V slices at once as its slots allow, and each slice's K/V
// stream through its L2 once per tile round instead of once per slice
// round; under a causal mask the tiles of consecutive slices pair up
// (longest with shortest) as the workgroups finish, as in tile-major order.
constexpr Item xcd_major(int w, int n_qtiles, int BH_kv, int H_kv, int G) {
    const int x = w % kXcds;
    const int j = w / kXcds;
    const int per_kv = G * n_qtiles;
    const int kv_local = j / per_kv;
    const int rem = j - kv_local * per_kv;
    const int tile = n_qtiles - 1 - rem / G;
    const int g = rem - (rem / G) * G;
    const int kv_bh = x + kXcds * kv_local;
    const int b = kv_bh / H_kv;
    const int h = (kv_bh - b * H_kv) * G + g;
    return {tile, b * H_kv * G + h, kv_bh};
}

constexpr bool xcd_major_applies(int BH_kv) { return BH_kv % kXcds == 0; }

constexpr Item item(bool xcd, int w, int n_qtiles, int BH, int BH_kv, int H_kv, int G) {
    return xcd ? xcd_major(w, n_qtiles, BH_kv, H_kv, G) : tile_major(w, n_qtiles, BH, BH_kv, H_kv, G);
}

}  // namespace fwdorder
}  // namespace attn

#endif  // ATTN_FWD_ORDER_H
