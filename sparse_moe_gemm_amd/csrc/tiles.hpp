// tiles.hpp - the tile walker of the persistent grouped GEMMs: which
// (expert, m-tile, n-tile, K split) a tile index stands for, derived on the
// device from the dispatch's expert offsets, so the host never learns the
// per-expert row counts. Experts without rows have no m-tiles (their weights
// are never read).
//
// Two classes of experts: those with more than SM rows (class 0) and small
// ones with 1..SM rows (class 1, one m-tile each; SM = 0: no small class).
// A small expert's tile does little matrix work but still streams a whole
// weight panel from HBM, so the small experts' tiles are spread evenly over
// the big experts' ones instead of running last, all together: the tile
// sequence is cut into units of 8 consecutive indices (one per XCD, as the
// workgroups go to the XCDs round robin) and the small units are placed among
// the big ones in proportion (Bresenham), so within a unit the tile order of
// each class, and the XCD each tile of a group lands on, stay as they were.
// Each class keeps the order expert -> K split -> group of GN n-tiles ->
// m-tile -> n-tile (GN > 0: within a group every m-tile of one n-tile lands
// on one XCD, which reads that weight panel into its L2 once), or, with
// GN = -G, K split -> group of G consecutive m-tiles (across experts) ->
// n-tile -> m-tile (every n-tile of one m-tile lands on one XCD, which reads
// that m-tile's token rows once; for experts of one or two m-tiles, whose
// weight panels are used once or twice anyway).
#pragma once

#include "common.hpp"

namespace cmoe {

constexpr int kUnit = 8;  // tiles per interleave unit (XCDs)

// M-tiles of an expert with c rows: c / BM full tiles and a ragged last one.
template <int BM>
__device__ __forceinline__ int mtiles_of(int c)
{
    return (c + BM - 1) / BM;
}

// Class of an expert with c > 0 rows.
template <int SM>
__device__ __forceinline__ int class_of(int c)
{
    return c <= SM ? 1 : 0;
}

// Per-lane view of the m-tiles: lane l holds experts 4l .. 4l+3 (E <= 256).
struct TileTable {
    int off[4];   // segment start offsets[e]
    int cnt[4];   // rows of the expert
    int mpre[2];  // per class: m-tiles of that class's experts below 4l
    int msum[2];  // per class: m-tiles of this lane's experts of that class
    int tiles[2]; // per class: tiles (m-tiles x tiles per m-tile), uniform
};

// Builds the table; returns the number of tiles (uniform). per_m: tiles per
// m-tile (n-tiles x K splits).
template <int BM, int SM = 0>
__device__ __forceinline__ int make_table(const int32_t* offsets, int E, int lane, int per_m, TileTable& t)
{
    int ms[2] = {0, 0};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int e = lane * 4 + q;
        const int o0 = e < E ? offsets[e] : 0;
        const int o1 = e < E ? offsets[e + 1] : 0;
        t.off[q] = o0;
        t.cnt[q] = o1 - o0;
        const int m = mtiles_of<BM>(o1 - o0);
        if (SM == 0 || class_of<SM>(o1 - o0) == 0)
            ms[0] += m;
        else
            ms[1] += m;
    }
    t.mpre[1] = t.msum[1] = t.tiles[1] = 0;
#pragma unroll
    for (int c = 0; c < (SM > 0 ? 2 : 1); ++c) {
        int incl = ms[c];
#pragma unroll
        for (int d = 1; d < kWave; d <<= 1) {
            const int o = __shfl_up(incl, d, kWave);
            if (lane >= d)
                incl += o;
        }
        t.mpre[c] = incl - ms[c];
        t.msum[c] = ms[c];
        t.tiles[c] = __builtin_amdgcn_readfirstlane(__shfl(incl, kWave - 1, kWave)) * per_m;
    }
    return t.tiles[0] + t.tiles[1];
}

// Most rows any expert holds, from a table make_table filled (every lane of
// the wave gets the same value).
__device__ __forceinline__ int table_max_rows(const TileTable& t)
{
    int m = max(max(t.cnt[0], t.cnt[1]), max(t.cnt[2], t.cnt[3]));
#pragma unroll
    for (int d = kWave / 2; d >= 1; d >>= 1)
        m = max(m, __shfl_xor(m, d, kWave));
    return __builtin_amdgcn_readfirstlane(m);
}

// Tile behind launch index L, or -1 for none. Workgroups go to the 8 XCDs
// round robin and a persistent workgroup takes indices L, L + grid, ..., so
// index L runs on XCD L % 8. Plain placement (xm false): tile L, so tiles
// next to each other in the order run on different XCDs. XCD-contiguous
// placement (xm true, grid a multiple of 8): XCD x runs the x-th eighth of
// the tile order, in order, so the tiles that share an m-tile's token rows
// or an expert's weight panel run on one XCD, close together in time, and
// read that data into its L2 once. Each workgroup's indices stay on its XCD
// and map to increasing tiles, so it stops at its first -1.
__device__ __forceinline__ int tile_index(int L, int total, bool xm)
{
    if (!xm)
        return L < total ? L : -1;
    const int q = total >> 3, r = total & 7, x = L & 7, i = L >> 3;
    if (i >= q + (x < r ? 1 : 0))
        return -1;
    return x * q + min(x, r) + i;
}

struct Tile {
    int e, m, n, s;
    int row0, rows;  // first sorted row and valid rows of the m-tile
    int kt0, nkt;    // K stages of the split
};

// Tile behind index L (< total). First the class and the index inside it
// (the unit interleave above), then, within the class, tiles of one m-tile are
// consecutive, NT * S of them, so idx / (NT * S) is the class's m-tile index
// j; the lane whose experts cover j holds the expert.
template <int BM, int SM = 0>
__device__ __forceinline__ Tile decode(const TileTable& t, int L, int NT, int S, int GN, int KT)
{
    int cls = 0, idx = L;
    if constexpr (SM > 0) {
        const int TA = t.tiles[0], TB = t.tiles[1];
        const int nb = TA / kUnit, ns = TB / kUnit, nu = nb + ns;
        if (L < kUnit * nu) {
            const int u = L / kUnit, r = L - u * kUnit;
            const int s0 = (int)((int64_t)u * ns / nu), s1 = (int)((int64_t)(u + 1) * ns / nu);
            if (s1 > s0) {
                cls = 1;
                idx = kUnit * s0 + r;
            } else {
                idx = kUnit * (u - s0) + r;
            }
        } else {
            const int rem = L - kUnit * nu, ra = TA - kUnit * nb;
            if (rem < ra) {
                idx = kUnit * nb + rem;
            } else {
                cls = 1;
                idx = kUnit * ns + rem - ra;
            }
        }
        cls = __builtin_amdgcn_readfirstlane(cls);
        idx = __builtin_amdgcn_readfirstlane(idx);
    }
    const int per_m = NT * S;
    int j, ms = 0, mn = 0, mm = 0;  // class m-tile index; m-group order: split, n-tile, m-tile in group
    if (GN < 0) {
        const int GM = -GN;
        const int mtot = (SM > 0 && cls ? t.tiles[1] : t.tiles[0]) / per_m;
        const int per_split = mtot * NT;
        ms = idx / per_split;
        const int rem = idx - ms * per_split;
        const int grp = rem / (GM * NT);
        const int gm = min(GM, mtot - grp * GM);
        const int r2 = rem - grp * GM * NT;
        mn = r2 / gm;
        mm = r2 - mn * gm;
        j = grp * GM + mm;
    } else {
        j = idx / per_m;
    }
    j = __builtin_amdgcn_readfirstlane(j);
    const int mp = SM > 0 && cls ? t.mpre[1] : t.mpre[0];
    const int msm = SM > 0 && cls ? t.msum[1] : t.msum[0];
    const uint64_t hit = __ballot(j >= mp && j < mp + msm);
    const int ln = __builtin_ctzll(hit);
    int base = __builtin_amdgcn_readlane(mp, ln);
    int e = 0, Me = 0, cnt = 0, seg0 = 0;
    bool found = false;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int c = __builtin_amdgcn_readlane(t.cnt[q], ln);
        const int o = __builtin_amdgcn_readlane(t.off[q], ln);
        const int me = SM == 0 || class_of<SM>(c) == cls ? mtiles_of<BM>(c) : 0;
        if (!found) {
            if (j < base + me) {
                found = true;
                e = ln * 4 + q;
                Me = me;
                cnt = c;
                seg0 = o;
            } else {
                base += me;
            }
        }
    }
    Tile r;
    r.e = e;
    if (GN < 0) {
        r.s = ms;
        r.m = j - base;
        r.n = mn;
    } else {
        const int local = idx - base * per_m;
        r.s = local / (Me * NT);
        const int rem = local - r.s * Me * NT;
        const int grp = rem / (Me * GN);
        const int gn = min(GN, NT - grp * GN);
        const int id2 = rem - grp * Me * GN;
        r.m = id2 / gn;
        r.n = grp * GN + (id2 - r.m * gn);
    }
    r.row0 = seg0 + r.m * BM;
    r.rows = min(BM, cnt - r.m * BM);
    const int per_s = KT / S;
    r.kt0 = r.s * per_s;
    r.nkt = (r.s == S - 1) ? KT - r.kt0 : per_s;
    // The divisions above run on the vector ALU; pin the (uniform) results to
    // scalar registers so everything derived from them stays scalar.
    r.e = __builtin_amdgcn_readfirstlane(r.e);
    r.m = __builtin_amdgcn_readfirstlane(r.m);
    r.n = __builtin_amdgcn_readfirstlane(r.n);
    r.s = __builtin_amdgcn_readfirstlane(r.s);
    r.row0 = __builtin_amdgcn_readfirstlane(r.row0);
    r.rows = __builtin_amdgcn_readfirstlane(r.rows);
    r.kt0 = __builtin_amdgcn_readfirstlane(r.kt0);
    r.nkt = __builtin_amdgcn_readfirstlane(r.nkt);
    return r;
}

}  // namespace cmoe
