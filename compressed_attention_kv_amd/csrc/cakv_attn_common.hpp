// cakv_attn_common.hpp -- the key-slot geometry shared by the attention
// forward (attention.hip) and backward (backward.hip) kernels.
//
// [V4-Pro card, Hybrid attention] a query at position t attends to the
// compressed entries the indexer selected (CSA) or every visible one (HCA),
// then the raw window of positions max(0, t - n_win + 1) .. t; a compressed
// entry j is visible iff its whole block precedes t (j < floor(t/m)).
#pragma once

#include "cakv_device.hpp"
#include "cakv_internal.hpp"

namespace cakv {

constexpr int TK = 32;  // key slots per tile

// Per-query key-slot geometry: slots [0, n_c) are compressed entries
// (selected idx slots, or entries 0..n_vis-1), slots [n_c, n_c + n_w) are the
// window positions p_lo .. t.
struct QueryGeom {
    int64_t b;
    int32_t t;
    int32_t n_vis;
    int32_t n_c;
    int32_t n_w;
    int32_t p_lo;
    int32_t raw0;
};

template <bool SPARSE>
__device__ __forceinline__ QueryGeom query_geom(const AttnArgs& a, int64_t bq) {
    QueryGeom g;
    g.b = bq / a.Q;
    int32_t t = a.q_pos[bq];
    t = t < 0 ? 0 : t;
    g.t = t;
    int64_t nv = t / a.m;
    g.n_vis = (int32_t)(nv < a.N ? nv : a.N);
    g.n_c = SPARSE ? a.K : g.n_vis;
    int32_t lo = t - a.n_win + 1;
    g.p_lo = lo < 0 ? 0 : lo;
    g.n_w = a.n_win > 0 ? t - g.p_lo + 1 : 0;
    // ring mode: position p sits at row p mod R; raw0 is the position of row
    // 0 in the ring's current lap, so rows of earlier positions wrap around
    g.raw0 = a.raw_ring ? (int32_t)(t - t % a.R) : a.raw_pos0[g.b];
    return g;
}

// Compressed entry index held by key slot `slot` (sparse: the selection,
// dense: the slot itself); only meaningful for slot < n_c.
template <bool SPARSE>
__device__ __forceinline__ int32_t slot_entry(const AttnArgs& a, const QueryGeom& g, int64_t bq, int slot) {
    if (!SPARSE) return slot;
    return slot < g.n_c ? a.idx[bq * a.K + slot] : 0;
}

// Source row of key slot `slot` whose entry index is j (from slot_entry);
// nullptr for an empty or invalid slot.
template <typename TIn>
__device__ __forceinline__ const TIn* slot_row(const AttnArgs& a, const QueryGeom& g, int slot, int32_t j, int D) {
    if (slot < g.n_c) {
        if (j < 0 || j >= g.n_vis) return nullptr;
        return reinterpret_cast<const TIn*>(a.kv_c) + (g.b * a.N + j) * (int64_t)D;
    }
    int s = slot - g.n_c;
    if (s >= g.n_w) return nullptr;
    int32_t p = g.p_lo + s;
    int64_t row = (int64_t)p - g.raw0;
    if (a.raw_ring && row < 0) row += a.R;
    if (row < 0 || row >= a.R) return nullptr;
    return reinterpret_cast<const TIn*>(a.kv_raw) + (g.b * a.R + row) * (int64_t)D;
}

// Workgroups are dispatched round-robin over the 8 XCDs (linear id mod 8).
// xcd_order maps linear ids to an order in which contiguous ranges sit on
// one XCD, so that consecutive work items (the splits of a query, the head
// pairs of a query in the combine) share that XCD's L2.  A bijection on
// [0, total).
__device__ __forceinline__ int64_t xcd_order(int64_t lin, int64_t total) {
    const int64_t q = total >> 3, rem = total & 7;
    const int64_t x = lin & 7, r = lin >> 3;
    const int64_t o = x < rem ? x * (q + 1) + r : rem * (q + 1) + (x - rem) * q + r;
    CAKV_DCHECK(o >= 0 && o < total);
    return o;
}

}  // namespace cakv
