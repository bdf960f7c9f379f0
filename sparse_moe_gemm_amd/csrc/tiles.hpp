// tiles.hpp - the tile walker of the persistent grouped GEMMs: which
// (expert, m-tile, n-tile, K split) a tile index stands for, derived on the
// device from the dispatch's expert offsets, so the host never learns the
// per-expert row counts. Experts without rows have no m-tiles (their weights
// are never read).
#pragma once

#include "common.hpp"

namespace cmoe {

// Per-lane view of the m-tiles: lane l holds experts 4l .. 4l+3 (E <= 256).
struct TileTable {
    int off[4];  // segment start offsets[e]
    int cnt[4];  // rows of the expert
    int mpre;    // m-tiles of all experts below 4l
    int msum;    // m-tiles of this lane's experts
};

template <int BM>
__device__ __forceinline__ int make_table(const int32_t* offsets, int E, int lane, TileTable& t)
{
    int ms = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int e = lane * 4 + q;
        const int o0 = e < E ? offsets[e] : 0;
        const int o1 = e < E ? offsets[e + 1] : 0;
        t.off[q] = o0;
        t.cnt[q] = o1 - o0;
        ms += (o1 - o0 + BM - 1) / BM;
    }
    int incl = ms;
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
        const int o = __shfl_up(incl, d, kWave);
        if (lane >= d)
            incl += o;
    }
    t.mpre = incl - ms;
    t.msum = ms;
    return __builtin_amdgcn_readfirstlane(__shfl(incl, kWave - 1, kWave));  // total m-tiles (uniform)
}

struct Tile {
    int e, m, n, s;
    int row0, rows;  // first sorted row and valid rows of the m-tile
    int kt0, nkt;    // K stages of the split
};

// Tile behind index L (< total). Tiles of one m-tile are consecutive in the
// global m-tile order, NT * S of them, so L / (NT * S) is the global m-tile
// index j; the lane whose experts cover j holds the expert.
template <int BM>
__device__ __forceinline__ Tile decode(const TileTable& t, int L, int NT, int S, int GN, int KT)
{
    const int per_m = NT * S;
    const int j = L / per_m;
    const uint64_t hit = __ballot(j >= t.mpre && j < t.mpre + t.msum);
    const int ln = __builtin_ctzll(hit);
    int base = __builtin_amdgcn_readlane(t.mpre, ln);
    int e = 0, Me = 0, cnt = 0, seg0 = 0;
    bool found = false;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int c = __builtin_amdgcn_readlane(t.cnt[q], ln);
        const int o = __builtin_amdgcn_readlane(t.off[q], ln);
        const int me = (c + BM - 1) / BM;
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
    const int local = L - base * per_m;
    r.s = local / (Me * NT);
    const int rem = local - r.s * Me * NT;
    const int grp = rem / (Me * GN);
    const int gn = min(GN, NT - grp * GN);
    const int idx = rem - grp * Me * GN;
    r.e = e;
    r.m = idx / gn;
    r.n = grp * GN + (idx - r.m * gn);
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
