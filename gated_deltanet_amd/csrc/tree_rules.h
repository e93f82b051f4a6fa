// tree_rules.h -- validity rules of a round's tree and the per-segment
// derivations (first position, depth, ancestor chain), written once and used
// by both the device builder and the host validator, so the two cannot drift.
//
// Rules (Flide section 3.2: tokens of a segment are contiguous in the flat
// stream and positions continue from the fork; section 3.4: a cached history
// is continued from its end; ForkServe item 1: a child sees a prefix of its
// parent; section 3.3.2: a round fills a graph captured for a larger
// capacity, with padding only at the tail):
//   phase 0  every token names a segment in [0, S), or is padding   FK_E_SEG_RANGE
//            (FK_PAD_TOKEN) followed only by padding
//   phase 1  a live segment has >= 1 token in one contiguous run;   FK_E_EMPTY /
//            a cached segment, and an unused slot                   FK_E_NONCONTIG
//            (FK_UNUSED_SEGMENT), has no stream tokens
//   phase 2  parent in [-1, S), not itself, not an unused slot;     FK_E_PARENT,
//            root fork 0; child
//            fork in [0, len(parent)]; cached only under cached;    FK_E_FORK,
//            a live child of a cached segment forks at its end;     FK_E_CACHED,
//            chain reaches a root within max_depth levels;          FK_E_CYCLE,
//            state slots in range, a cached parent brings a state;  FK_E_STATE_SLOT,
//            page lists are long enough for the segment             FK_E_PAGES
//   phase 3  capacities: live segments per level, fork points;      FK_E_CAPACITY,
//            every page id a segment uses lies in [0, n_pages)      FK_E_PAGES
// A phase runs only when the previous ones found nothing; the reported code
// is the most negative one of the first failing phase.
#pragma once

#include <stdint.h>

#include "../../include/forkgdn.h"

namespace fk {

#if defined(__HIPCC__)
#define FK_HD __host__ __device__ __forceinline__
#else
#define FK_HD inline
#endif

FK_HD int imin(int a, int b) { return a < b ? a : b; }

FK_HD bool is_unused(int cached_len) { return cached_len == FK_UNUSED_SEGMENT; }

// phase 1: segment length from its token runs (nrun) or cached length; an
// unused slot has length 0 and no tokens
FK_HD int rule_length(int cached_len, int nrun, int run_len, int *len_out)
{
    int code = FK_OK;
    if (is_unused(cached_len)) {
        *len_out = 0;
        return nrun > 0 ? FK_E_EMPTY : FK_OK;
    }
    if (cached_len < 0) code = imin(code, FK_E_EMPTY);
    if (cached_len > 0 && nrun > 0) code = imin(code, FK_E_EMPTY);
    if (cached_len == 0 && nrun == 0) code = imin(code, FK_E_EMPTY);
    if (nrun > 1) code = imin(code, FK_E_NONCONTIG);
    *len_out = cached_len > 0 ? cached_len : run_len;
    return code;
}

struct SegDerived {
    int depth;
    int pos0;
    int anc[FK_MAX_DEPTH];   // root first, the segment itself at [depth]
};

// phase 2: links, chain, slots and pages of segment s.  `len` holds phase-1
// lengths of every segment.  Optional arrays may be null (no pages / slots).
FK_HD int rule_links(int s, int S, int max_depth, const int32_t *parent, const int32_t *fork,
                     const int32_t *cached_len, const int32_t *len, const int32_t *state_in_slot,
                     int n_state_in, const int32_t *state_out_slot, int n_state_out,
                     const int32_t *page_off, const int32_t *pages, int page_size, int n_pages,
                     SegDerived *out)
{
    int code = FK_OK;
    const int p = parent[s];
    const bool cached = cached_len[s] > 0;
    if (is_unused(cached_len[s])) {   // an unused slot: nothing to derive
        out->depth = 0;
        out->pos0 = 0;
        out->anc[0] = s;
        return FK_OK;
    }
    if (p < -1 || p >= S || p == s || (p >= 0 && is_unused(cached_len[p]))) {
        code = imin(code, FK_E_PARENT);
    } else if (p == -1) {
        if (fork[s] != 0) code = imin(code, FK_E_FORK);
    } else {
        if (fork[s] < 0 || fork[s] > len[p]) code = imin(code, FK_E_FORK);
        if (cached && cached_len[p] == 0) code = imin(code, FK_E_CACHED);
        if (cached_len[p] > 0 && !cached) {
            if (fork[s] != len[p]) code = imin(code, FK_E_CACHED);
            if (state_in_slot) {
                const int slot = state_in_slot[p];
                if (slot < 0 || slot >= n_state_in) code = imin(code, FK_E_STATE_SLOT);
            } else {
                code = imin(code, FK_E_STATE_SLOT);
            }
        }
    }
    // chain: walk parents, bounded by max_depth (also catches cycles)
    int chain[FK_MAX_DEPTH];
    int n = 0, pos0 = 0, i = s;
    bool ok = true;
    while (true) {
        if (n >= max_depth) { code = imin(code, FK_E_CYCLE); ok = false; break; }
        chain[n++] = i;
        const int pi = parent[i];
        if (pi < 0) break;
        if (pi >= S || pi == i) { ok = false; break; }   // reported by i's own check
        pos0 += fork[i];
        i = pi;
    }
    if (ok) {
        out->depth = n - 1;
        out->pos0 = pos0;
        for (int j = 0; j < n; ++j) out->anc[j] = chain[n - 1 - j];
    } else {
        out->depth = 0;
        out->pos0 = 0;
        out->anc[0] = s;
    }
    if (state_out_slot) {
        const int so = state_out_slot[s];
        if (so < -1 || so >= n_state_out || (so >= 0 && cached)) code = imin(code, FK_E_STATE_SLOT);
    }
    if (page_off) {
        const int a = page_off[s], b = page_off[s + 1];
        const int need = (len[s] + page_size - 1) / page_size;
        if (a < 0 || b < a || b - a < need) code = imin(code, FK_E_PAGES);
    }
    return code;
}

// phase 3: page ids of segment s (its first ceil(len/page_size) entries)
FK_HD bool rule_page_id(int page, int n_pages) { return page >= 0 && page < n_pages; }

}  // namespace fk
