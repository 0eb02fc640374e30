// Work mapping of the forward kernels: workgroup id -> (batch*head, query tile).
//
// Plain C++ (no HIP types) so the host test suite can compile it with g++ and check that
// the mapping is a bijection.  Under hipcc the functions are also device functions.
#pragma once

#if defined(__HIPCC__)
#define FA_HD __host__ __device__
#else
#define FA_HD
#endif

namespace fa {

// MI355X has 8 accelerator complex dies (XCDs), each with its own L2.  The dispatcher hands
// consecutive workgroup ids to the XCDs round-robin, so id w runs on XCD (w % 8).  Remapping
// makes the logical work items one XCD receives contiguous: all query tiles of one head then
// run on the same XCD and reuse that head's K/V tiles from its L2.
constexpr int kNumXcd = 8;

FA_HD inline int xcd_remap(int wg, int total) {
    const int per = (total + kNumXcd - 1) / kNumXcd;  // items on the fuller XCDs
    int full = total % kNumXcd;                        // XCDs that hold `per` items
    if (full == 0) full = kNumXcd;
    const int xcd = wg % kNumXcd;
    const int local = wg / kNumXcd;
    return xcd < full ? xcd * per + local : full * per + (xcd - full) * (per - 1) + local;
}

struct TileCoord {
    int bh;  // b * H + h
    int qt;  // query tile index
};

// Logical item -> (head, query tile).  Items of one head are contiguous.  With a causal mask
// the tiles of a head are visited from the last (most keys, most work) to the first, so the
// long tiles start early and the short ones fill the tail of the launch.
FA_HD inline TileCoord tile_of(int logical, int n_qtiles, bool causal) {
    TileCoord t;
    t.bh = logical / n_qtiles;
    const int r = logical - t.bh * n_qtiles;
    t.qt = causal ? (n_qtiles - 1 - r) : r;
    return t;
}

// Pairs of query tiles per work item (causal mask): under the causal mask query tile t of a
// head carries t+1 tile-rows of work, so tile t is paired with tile n-1-t and every work item
// carries the same amount (n+1 tile-rows); an odd middle tile forms an item alone.  Without
// the causal mask every tile is its own item.  Items of one head are contiguous.
struct TilePair {
    int bh;
    int qt0;  // first query tile (the heavier one under the causal mask)
    int qt1;  // second query tile, or -1
};

FA_HD inline int items_per_head(int n_qtiles, bool causal) { return causal ? (n_qtiles + 1) / 2 : n_qtiles; }

FA_HD inline TilePair pair_of(int logical, int n_qtiles, bool causal) {
    TilePair t;
    const int per = items_per_head(n_qtiles, causal);
    t.bh = logical / per;
    const int it = logical - t.bh * per;
    if (!causal) {
        t.qt0 = it;
        t.qt1 = -1;
    } else {
        t.qt0 = n_qtiles - 1 - it;
        t.qt1 = (it == t.qt0) ? -1 : it;
    }
    return t;
}

// Packed sequences: workgroup id w -> (head, work item) with head bh on XCD bh % kNumXcd and
// the `per` items of a head contiguous among that XCD's ids.  The grid holds
// ceil(n_heads / kNumXcd) * kNumXcd * per ids; ids whose head is >= n_heads get bh = -1.
struct HeadItem {
    int bh;
    int it;
};

FA_HD inline HeadItem head_item_xcd(int w, int n_heads, int per) {
    HeadItem r;
    const int local = w / kNumXcd;
    const int m = local / per;
    r.it = local - m * per;
    r.bh = w % kNumXcd + kNumXcd * m;
    if (r.bh >= n_heads) r.bh = -1;
    return r;
}

}  // namespace fa
