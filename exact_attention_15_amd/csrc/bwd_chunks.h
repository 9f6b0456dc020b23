// bwd_chunks.h — how the dK/dV work of the 16-bit backward pass is dealt out
// as workgroup items.
//
// The dK/dV work of one key tile (kKeyBlock keys of one K/V slice) is a
// sequence of steps, one per (query head of the K/V head's group, query tile
// of kQStage rows that can see the keys), head-major. Without grouped-query
// heads an item is a whole key tile. With G query heads per K/V head the
// items become G times fewer and longer, and under a causal mask key tile kt
// has (n_qs - 2 kt) G steps, so one round of items is as long as its first
// key tile. Then every key tile's steps are cut into chunks of one length
// L (the last chunk of a tile shorter), each chunk an item of its own. A
// tile of more than one chunk has its chunks write fp32 partial sums of
// dK^T and dV^T, which a reduction adds in chunk order (deterministic) into
// dK and dV; a tile of one chunk is written directly, as without a plan.
//
// Partial sums live in dq's memory (2 G N D bytes per K/V slice for
// f16/bf16, written by the last kernel only). Chunk c of a cut key tile kt
// holds rows(kt) partial rows (of 2 D floats: dK^T and dV^T) per K/V slice,
// so the plan must satisfy  sum over cut tiles of n_chunks(kt) rows(kt) * 8 D
// <= 2 G N D, i.e. that sum of rows <= G N / 4.
//
// Layout of the partials (floats from the start of dq's memory), chunk c of
// cut key tile kt, K/V slice s, key row r < rows(kt), column j < D:
//   block = (first(kt) kKeyBlock + c rows(kt)) BH_kv 2D + s rows(kt) 2D
//   dK^T partial at block + r D + j, dV^T partial at block + (rows(kt) + r) D + j
// with first(kt) the chunks of the earlier cut key tiles; as every key tile
// but the last has kKeyBlock rows, the blocks tile the rows without overlap.
//
// Plain constexpr functions: the kernels call them on device, the launcher on
// the host, and a host test compiles this header with g++ alone.
#ifndef ATTN_BWD_CHUNKS_H
#define ATTN_BWD_CHUNKS_H

#include <stdint.h>

namespace attn {
namespace bwdplan {

constexpr int kKeyBlock = 128;   // keys per dK/dV item (4 waves x 32)
constexpr int kQStage = 64;      // query rows per step

constexpr int n_query_stages(int64_t N) { return (int)((N + kQStage - 1) / kQStage); }
constexpr int n_key_tiles(int64_t N) { return (int)((N + kKeyBlock - 1) / kKeyBlock); }

// Steps of key tile kt of one K/V slice.
constexpr int kv_steps(int G, int n_qs, int kt, bool causal) {
    return G * (causal ? n_qs - kt * (kKeyBlock / kQStage) : n_qs);
}

// Keys of key tile kt (kKeyBlock except for a ragged last tile).
constexpr int tile_rows(int64_t N, int kt) {
    const int64_t left = N - (int64_t)kt * kKeyBlock;
    return left < kKeyBlock ? (int)left : kKeyBlock;
}

constexpr int n_chunks(int steps, int chunk) { return (steps + chunk - 1) / chunk; }

// Partial slots of a tile of nc chunks: none when it is written directly.
constexpr int partial_slots(int nc) { return nc > 1 ? nc : 0; }

// Item number w (over all K/V slices, key tile major, then chunk, then slice)
// of a chunked plan.
struct Item {
    int kt;      // key tile
    int slice;   // K/V slice b * H_kv + h_kv
    int s0;      // first step
    int s1;      // one past the last step
    int64_t part_row;   // first(kt) kKeyBlock + c rows(kt): the block's row offset
    bool partial;       // the tile is cut: write partial sums at part_row
    bool valid;  // w lies inside the plan
};

constexpr Item locate(int w, int64_t N, int G, int BH_kv, bool causal, int chunk) {
    Item it{0, 0, 0, 0, 0, false, false};
    const int n_qs = n_query_stages(N);
    const int n_kt = n_key_tiles(N);
    int rem = w / BH_kv;
    it.slice = w - rem * BH_kv;
    int first = 0;
    for (int kt = 0; kt < n_kt; ++kt) {
        const int steps = kv_steps(G, n_qs, kt, causal);
        const int nc = n_chunks(steps, chunk);
        if (rem < nc) {
            it.kt = kt;
            it.s0 = rem * chunk;
            it.s1 = it.s0 + chunk < steps ? it.s0 + chunk : steps;
            it.part_row = (int64_t)first * kKeyBlock + (int64_t)rem * tile_rows(N, kt);
            it.partial = nc > 1;
            it.valid = true;
            return it;
        }
        rem -= nc;
        first += partial_slots(nc);
    }
    return it;
}

// Partial slots of the key tiles before kt (the reduction's view of the plan).
constexpr int first_chunk(int kt, int64_t N, int G, bool causal, int chunk) {
    const int n_qs = n_query_stages(N);
    int first = 0;
    for (int k = 0; k < kt; ++k) first += partial_slots(n_chunks(kv_steps(G, n_qs, k, causal), chunk));
    return first;
}

// Items of a plan with chunk length `chunk` (all K/V slices).
constexpr int64_t plan_items(int64_t N, int G, int BH_kv, bool causal, int chunk) {
    const int n_qs = n_query_stages(N);
    int64_t n = 0;
    for (int kt = 0; kt < n_key_tiles(N); ++kt) n += n_chunks(kv_steps(G, n_qs, kt, causal), chunk);
    return n * BH_kv;
}

// Partial rows per K/V slice: the sum over cut tiles of n_chunks(kt) rows(kt).
constexpr int64_t plan_partial_rows(int64_t N, int G, bool causal, int chunk) {
    const int n_qs = n_query_stages(N);
    int64_t rows = 0;
    for (int kt = 0; kt < n_key_tiles(N); ++kt)
        rows += (int64_t)partial_slots(n_chunks(kv_steps(G, n_qs, kt, causal), chunk)) * tile_rows(N, kt);
    return rows;
}

// The chunk length for a call, or 0 for one item per key tile (partials not
// used): the shortest chunk whose items number at most `target` (the
// workgroups the device holds at once: items past them would start a
// second round, as long again) and whose partial sums fit dq's memory;
// whole key tiles are kept unless chunks cut the longest item to at most
// 3/4 of its steps.
constexpr int choose_chunk(int64_t N, int G, int BH_kv, bool causal, int target) {
    const int n_qs = n_query_stages(N);
    const int longest = kv_steps(G, n_qs, 0, causal);
    const int hi = (3 * (int64_t)longest) / 4;
    if (hi < 1) return 0;
    const int64_t cap_rows = (int64_t)G * N / 4;
    if (plan_items(N, G, BH_kv, causal, hi) > target || plan_partial_rows(N, G, causal, hi) > cap_rows)
        return 0;
    // Both conditions hold from some length on (longer chunks: fewer items,
    // fewer cut tiles), so the shortest length meeting both is found by
    // bisection over [1, hi].
    int lo = 1, top = hi;
    while (lo < top) {
        const int mid = lo + (top - lo) / 2;
        if (plan_items(N, G, BH_kv, causal, mid) <= target &&
            plan_partial_rows(N, G, causal, mid) <= cap_rows)
            top = mid;
        else
            lo = mid + 1;
    }
    return top;
}

// Wave groups of a dK/dV item and how many such workgroups a compute unit
// holds. The one-group kernel is 4 waves (one per SIMD); its d = 64 build
// takes 156-166 VGPRs, so three waves fit a SIMD's 512 registers and three
// workgroups a compute unit, its d = 128 build takes 256 (two). The
// three-group kernel (12 waves, d = 64 only) fits once per compute unit.
// tests/test_build_flags.py checks these counts against the compiler's.
constexpr int kGroupedWaveGroups = 3;
constexpr int one_group_per_cu(int D) { return D == 64 ? 3 : 2; }
constexpr int dkdv_resident(int D, int groups, int compute_units) {
    return compute_units * (groups > 1 ? 1 : one_group_per_cu(D));
}

// Wave groups per dK/dV item. Grouped-query items at d = 64 take three. So
// do multi-head non-causal ones at d = 64 when the last round of equal
// items would leave the one-group kernel's slots mostly idle: the
// three-group kernel gives ~0.70 of the one-group throughput per compute
// unit (fp16 B1 H8 N16384: 1024 items, 2.04 ms with one group in two
// rounds of 768, 1.94 ms with three in four rounds of 256) but its rounds
// come out fuller. Causal items differ in length and, longest first, fill
// their rounds (bf16 causal B4 H16 N4096: one group 0.48 ms, three 0.54 ms).
constexpr int dkdv_groups(int D, bool causal, int G, int64_t N, int BH_kv, int compute_units) {
    if (D != 64) return 1;
    if (G > 1) return kGroupedWaveGroups;
    if (causal) return 1;
    const int64_t items = (int64_t)n_key_tiles(N) * BH_kv;
    const int64_t slots1 = dkdv_resident(D, 1, compute_units);
    const int64_t slots3 = dkdv_resident(D, kGroupedWaveGroups, compute_units);
    const double fill1 = (double)items / (double)(((items + slots1 - 1) / slots1) * slots1);
    const double fill3 = (double)items / (double)(((items + slots3 - 1) / slots3) * slots3);
    return 0.70 * fill3 > 1.02 * fill1 ? kGroupedWaveGroups : 1;
}

}  // namespace bwdplan
}  // namespace attn

#endif  // ATTN_BWD_CHUNKS_H
