// tree_build.hip -- the tree-metadata builder (Flide section 3.3.1: every
// variable set by the round composition -- segment lengths, positions, key
// ranges, state indices -- lives in device buffers, and the attention tile
// table is built on the GPU; section 3.3.2: launch sizes come from host-known
// capacities, so the host never reads the tree).
//
// Kernels (four launches):
//   k_clear    grid          clears the status and the per-segment counters
//   k_tokens   grid          token runs of every segment (start, end, run
//                            count), padding and segment-id checks
//   k_build    one block     validation, lengths, first positions, ancestor
//                            chains, tile / chunk / level offsets, fork points
//   k_post     grid          tile order (heaviest first, by root within a
//                            band of work) and each level's
//                            segments by decreasing chunk count (1 + levels
//                            blocks), tile and chunk lists, page-id checks (a
//                            block per segment), per-token positions
// No dense T x T mask is ever formed: a tile's key ranges follow from its
// segment's ancestor chain and the forks along it.
#include <hip/hip_runtime.h>

#include <vector>

#include "fk_common.h"
#include "tree_rules.h"

namespace fk {

constexpr int BUILD_THREADS = 1024;

// Exclusive prefix sum over the block (BUILD_THREADS threads, wave64).
__device__ int block_scan(int x, int *lds, int *total)
{
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6, nw = blockDim.x >> 6;
    int v = x;
    for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(v, o, 64);
        if (lane >= o) v += y;
    }
    if (lane == 63) lds[wid] = v;
    __syncthreads();
    if (wid == 0) {
        int w = lane < nw ? lds[lane] : 0;
        for (int o = 1; o < 64; o <<= 1) {
            const int y = __shfl_up(w, o, 64);
            if (lane >= o) w += y;
        }
        if (lane < nw) lds[lane] = w;
    }
    __syncthreads();
    const int before = wid ? lds[wid - 1] : 0;
    *total = lds[nw - 1];
    __syncthreads();
    return before + v - x;
}

// Maximum over the block (BUILD_THREADS threads, wave64).
__device__ int block_max(int x, int *lds)
{
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6, nw = blockDim.x >> 6;
    int v = x;
    for (int o = 32; o > 0; o >>= 1) v = max(v, __shfl_xor(v, o, 64));
    if (lane == 0) lds[wid] = v;
    __syncthreads();
    int r = lds[0];
    for (int i = 1; i < nw; ++i) r = max(r, lds[i]);
    __syncthreads();
    return r;
}

struct BuildArgs {
    fk_tree_meta m;
    int32_t *header, *seg_start, *seg_end, *seg_nrun, *seg_len, *seg_pos0, *seg_depth, *seg_anc;
    int32_t *seg_src, *seg_owner, *kid_cnt, *kid_off, *kid_fill, *kids, *emit_off, *emit_pos;
    int32_t *tile_seg, *tile_row0, *lvl_seg, *chunk_seg, *chunk_row0, *seg_chunk0;
    int32_t *seg_tile0, *seg_coff;
};

// k_build is the only writer of the status while it runs, so it mirrors its
// own errors in an LDS flag: a phase boundary is then a barrier, not a round
// trip to global memory.
__device__ __forceinline__ void build_error(int32_t *header, int *flag, int code)
{
    set_error(header, code);
    *flag = code;   // any nonzero value marks the failure
}

__device__ bool block_failed(int *flag)
{
    __threadfence_block();
    __syncthreads();
    return *flag != FK_OK;
}

// Phase 0, over the whole grid: k_clear zeroes the status and the
// per-segment counters; then k_tokens checks every token's segment id, and the
// first token of every run records the run start, the last its end, and
// counts the run (an integer atomic: order-independent).
__global__ void __launch_bounds__(BUILD_THREADS) k_clear(BuildArgs A)
{
    const int i = blockIdx.x * BUILD_THREADS + threadIdx.x;
    if (i < H_WORDS) A.header[i] = 0;
    if (i < A.m.S) {
        A.seg_nrun[i] = 0;
        A.kid_cnt[i] = 0;
        A.kid_fill[i] = 0;
    }
}

constexpr int TOKENS_PER_THREAD = 8;   // their loads in flight together
__global__ void __launch_bounds__(BUILD_THREADS) k_tokens(BuildArgs A)
{
    const fk_tree_meta &m = A.m;
    const int S = m.S, T = m.T;
    constexpr int TB = TOKENS_PER_THREAD;
    const int base = blockIdx.x * TB * BUILD_THREADS;
    int sv[TB], pv[TB], nv[TB];
#pragma unroll
    for (int u = 0; u < TB; ++u) {
        const int t = base + u * BUILD_THREADS + threadIdx.x;
        sv[u] = t < T ? m.tok_seg[t] : 0;
        pv[u] = t < T && t > 0 ? m.tok_seg[t - 1] : -1;
        nv[u] = t + 1 < T ? m.tok_seg[t + 1] : -1;
    }
#pragma unroll
    for (int u = 0; u < TB; ++u) {
        const int t = base + u * BUILD_THREADS + threadIdx.x, s = sv[u];
        if (t >= T) continue;
        if (s == FK_PAD_TOKEN) {   // padding: only more padding may follow
            if (t + 1 < T && nv[u] != FK_PAD_TOKEN) set_error(A.header, FK_E_SEG_RANGE);
            continue;
        }
        if (s < 0 || s >= S) {
            set_error(A.header, FK_E_SEG_RANGE);
            continue;
        }
        if (t == 0 || pv[u] != s) {
            atomicAdd(A.seg_nrun + s, 1);
            A.seg_start[s] = t;   // meaningful only when the run count is 1
        }
        if (t == T - 1 || nv[u] != s) A.seg_end[s] = t + 1;
    }
}

__global__ void __launch_bounds__(BUILD_THREADS) k_build(BuildArgs A)
{
    __shared__ int lds[32];
    __shared__ int lvl_lds[FK_MAX_DEPTH];
    __shared__ int flag;
    const fk_tree_meta &m = A.m;
    const int S = m.S;
    // phase 0 ran in k_clear and k_tokens; their errors are in the status
    if (threadIdx.x == 0) flag = A.header[H_STATUS];
    if (block_failed(&flag)) return;

    // phase 1: lengths
    for (int s = threadIdx.x; s < S; s += blockDim.x) {
        const int nrun = A.seg_nrun[s];
        int len = 0;
        const int code = rule_length(m.seg_cached_len[s], nrun,
                                     nrun == 1 ? A.seg_end[s] - A.seg_start[s] : 0, &len);
        if (code) build_error(A.header, &flag, code);
        A.seg_len[s] = len;
        if (m.seg_cached_len[s] != 0) A.seg_start[s] = -1;   // cached or unused: no stream tokens
    }
    if (block_failed(&flag)) return;

    // phase 2: links, chains, slots, pages; GDN sources of children of cached
    // or fresh roots; child counts of live parents
    for (int s = threadIdx.x; s < S; s += blockDim.x) {
        SegDerived d;
        const int code = rule_links(s, S, m.max_depth, m.seg_parent, m.seg_fork, m.seg_cached_len,
                                    A.seg_len, m.seg_state_in, m.n_state_in, m.seg_state_out,
                                    m.n_state_out, m.seg_page_off, m.seg_pages, m.page_size,
                                    m.n_pages, &d);
        if (code) build_error(A.header, &flag, code);
        A.seg_depth[s] = d.depth;
        A.seg_pos0[s] = d.pos0;
        for (int j = 0; j < FK_MAX_DEPTH; ++j) A.seg_anc[s * FK_MAX_DEPTH + j] = j <= d.depth ? d.anc[j] : -1;
        const int p = m.seg_parent[s];
        const bool live = m.seg_cached_len[s] == 0;
        int src = -1;
        if (live && p >= 0 && p < S) {
            if (m.seg_cached_len[p] > 0) src = -2 - (m.seg_state_in ? m.seg_state_in[p] : 0);
            else atomicAdd(A.kid_cnt + p, 1);
        }
        A.seg_src[s] = src;
    }
    if (block_failed(&flag)) return;

    // phase 3a: scans -- attention tiles, children CSR, level lists
    if (threadIdx.x < FK_MAX_DEPTH) lvl_lds[threadIdx.x] = 0;
    __syncthreads();
    int tile_base = 0, kid_base = 0, chunk_base = 0, max_keys = 1;
    for (int base = 0; base < S; base += blockDim.x) {
        const int s = base + threadIdx.x;
        const bool in = s < S;
        const bool live = in && m.seg_cached_len[s] == 0;
        const int len = in ? A.seg_len[s] : 0;
        const int ntile = live ? (len + FK_TILE_TOKENS - 1) / FK_TILE_TOKENS : 0;
        int tot;
        const int toff = tile_base + block_scan(ntile, lds, &tot);
        tile_base += tot;
        // the most keys a row of this segment sees (its last tile's rows)
        max_keys = max(max_keys, block_max(live ? A.seg_pos0[s] + len : 0, lds));
        const int nchunk = live ? (len + FK_GDN_CHUNK - 1) / FK_GDN_CHUNK : 0;
        const int coff = chunk_base + block_scan(nchunk, lds, &tot);
        chunk_base += tot;
        if (in) {
            // the tile and chunk lists themselves are written by k_post
            A.seg_tile0[s] = toff;
            A.seg_coff[s] = coff;
            A.seg_chunk0[s] = live ? coff : -1;
        }
        const int kc = in ? A.kid_cnt[s] : 0;
        const int koff = kid_base + block_scan(kc, lds, &tot);
        kid_base += tot;
        if (in) A.kid_off[s] = koff;
        // level lists: a rank per live segment from its level's LDS counter
        // (order within a level is whatever the atomics give: k_post sorts
        // each level, and every segment computes the same way in any order)
        const int depth = in ? A.seg_depth[s] : -1;
        if (live && depth >= 0 && depth < m.max_depth) {
            const int rank = atomicAdd(&lvl_lds[depth], 1);
            if (rank < m.level_cap) A.lvl_seg[depth * m.level_cap + rank] = s;
            else build_error(A.header, &flag, FK_E_CAPACITY);
        }
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        A.kid_off[S] = kid_base;
        A.header[H_NTILES] = tile_base;
        A.header[H_NCHUNKS] = chunk_base;
        A.header[H_MAXKEYS] = max_keys;
        for (int dd = 0; dd < FK_MAX_DEPTH; ++dd) A.header[H_LEVEL0 + dd] = dd < m.max_depth ? lvl_lds[dd] : 0;
    }
    __syncthreads();
    // children lists (filled in arbitrary order; every later rule compares
    // (fork, index) so the order does not matter)
    for (int s = threadIdx.x; s < S; s += blockDim.x) {
        const int p = m.seg_parent[s];
        if (m.seg_cached_len[s] == 0 && p >= 0 && m.seg_cached_len[p] == 0) {
            const int at = atomicAdd(A.kid_fill + p, 1);
            A.kids[A.kid_off[p] + at] = s;
        }
    }
    if (block_failed(&flag)) return;

    // phase 3b: fork points -- one slot per distinct (parent, fork offset);
    // the lowest-index child at an offset owns it
    for (int c = threadIdx.x; c < S; c += blockDim.x) {
        const int p = m.seg_parent[c];
        int owner = 0;
        if (m.seg_cached_len[c] == 0 && p >= 0 && m.seg_cached_len[p] == 0) {
            owner = 1;
            for (int j = A.kid_off[p]; j < A.kid_off[p + 1]; ++j) {
                const int o = A.kids[j];
                if (o < c && m.seg_fork[o] == m.seg_fork[c]) owner = 0;
            }
        }
        A.seg_owner[c] = owner;
    }
    __syncthreads();
    __threadfence_block();
    int emit_base = 0;
    for (int base = 0; base < S; base += blockDim.x) {
        const int s = base + threadIdx.x;
        int n = 0;
        if (s < S)
            for (int j = A.kid_off[s]; j < A.kid_off[s + 1]; ++j) n += A.seg_owner[A.kids[j]];
        int tot;
        const int off = emit_base + block_scan(n, lds, &tot);
        emit_base += tot;
        if (s < S) A.emit_off[s] = off;
    }
    if (threadIdx.x == 0) {
        A.emit_off[S] = emit_base;
        A.header[H_NFORKS] = emit_base;
        if (emit_base > m.fork_cap) build_error(A.header, &flag, FK_E_CAPACITY);
    }
    if (block_failed(&flag)) return;
    for (int c = threadIdx.x; c < S; c += blockDim.x) {
        const int p = m.seg_parent[c];
        if (m.seg_cached_len[c] == 0 && p >= 0 && m.seg_cached_len[p] == 0) {
            int rank = 0;
            for (int j = A.kid_off[p]; j < A.kid_off[p + 1]; ++j) {
                const int o = A.kids[j];
                if (A.seg_owner[o] && m.seg_fork[o] < m.seg_fork[c]) ++rank;
            }
            const int slot = A.emit_off[p] + rank;
            A.seg_src[c] = slot;
            if (A.seg_owner[c]) A.emit_pos[slot] = m.seg_fork[c];
        }
    }
}

// the segment of list entry i: the last s with first[s] <= i (segments with
// no entries share the next one's offset, so the last such s owns entry i)
__device__ __forceinline__ int owner_of(const int32_t *__restrict__ first, int S, int i)
{
    int lo = 0, hi = S - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (first[mid] <= i) lo = mid;
        else hi = mid - 1;
    }
    return lo;
}

// Attention tiles and GDN chunks of every live segment, one thread per entry.
__device__ void lists_thread(int i, int S, const int32_t *__restrict__ header, const int32_t *__restrict__ seg_tile0,
                             const int32_t *__restrict__ seg_coff, int32_t *__restrict__ tile_seg,
                             int32_t *__restrict__ tile_row0, int32_t *__restrict__ chunk_seg,
                             int32_t *__restrict__ chunk_row0)
{
    if (i < header[H_NTILES]) {
        const int s = owner_of(seg_tile0, S, i);
        tile_seg[i] = s;
        tile_row0[i] = (i - seg_tile0[s]) * FK_TILE_TOKENS;
    }
    if (i < header[H_NCHUNKS]) {
        const int s = owner_of(seg_coff, S, i);
        chunk_seg[i] = s;
        chunk_row0[i] = (i - seg_coff[s]) * FK_GDN_CHUNK;
    }
}

// Tiles by decreasing work, grouped by root: a bucket sort over (band of the
// tile's visible keys, root of its segment).  The bands split [0, most keys
// of any tile] into ORDER_BANDS equal parts, so the launch runs heaviest
// first at that granularity and does not end on a long tile started late;
// within a band a root's tiles are consecutive ranks, so the work-groups
// resident on an XCD at one time (consecutive ranks of one kv head) mostly
// walk one request's history and share it in L2 -- on the expanding-history
// resume round, heaviest first alone interleaves all 64 requests.  Order
// within a bucket is whatever the atomics give; only the schedule depends on
// the order (every tile computes the same way in any order).  It runs beside
// the blocks that write the tile list, so it finds each tile's segment
// itself, with the same search over seg_tile0 (staged in LDS when S fits
// there).
constexpr int ORDER_BUCKETS = 2 * BUILD_THREADS;
constexpr int ORDER_BANDS = 64, ORDER_ROOTS = ORDER_BUCKETS / ORDER_BANDS;
constexpr int ORDER_STAGE = 4096;
__device__ void tile_order_block(const int32_t *__restrict__ header, int S, const int32_t *__restrict__ seg_tile0,
                                 const int32_t *__restrict__ seg_pos0, const int32_t *__restrict__ seg_len,
                                 const int32_t *__restrict__ seg_anc, int32_t *__restrict__ tile_order, int *cnt,
                                 int *lds, int *stage)
{
    const int n = header[H_NTILES];
    const int64_t max_keys = header[H_MAXKEYS];
    const bool staged = S <= ORDER_STAGE;
    if (staged)
        for (int i = threadIdx.x; i < S; i += blockDim.x) stage[i] = seg_tile0[i];
    for (int b = threadIdx.x; b < ORDER_BUCKETS; b += blockDim.x) cnt[b] = 0;
    __syncthreads();
    const int32_t *first = staged ? stage : seg_tile0;
    auto bucket = [&](int t) {
        const int s = owner_of(first, S, t), r0 = (t - first[s]) * FK_TILE_TOKENS;
        const int keys = seg_pos0[s] + min(r0 + FK_TILE_TOKENS, seg_len[s]);
        const int band = min(ORDER_BANDS - 1, (int)((int64_t)keys * ORDER_BANDS / (max_keys + 1)));
        const int root = seg_anc[s * FK_MAX_DEPTH];
        return band * ORDER_ROOTS + (ORDER_ROOTS - 1 - root % ORDER_ROOTS);
    };
    for (int t = threadIdx.x; t < n; t += blockDim.x) atomicAdd(&cnt[bucket(t)], 1);
    __syncthreads();
    // offsets with the largest bucket first: thread j owns buckets B-1-2j, B-2-2j
    const int b0 = ORDER_BUCKETS - 1 - 2 * threadIdx.x, b1 = b0 - 1;
    int tot;
    const int before = block_scan(cnt[b0] + cnt[b1], lds, &tot);
    const int c0 = cnt[b0];
    __syncthreads();
    cnt[b0] = before;
    cnt[b1] = before + c0;
    __syncthreads();
    for (int t = threadIdx.x; t < n; t += blockDim.x) tile_order[atomicAdd(&cnt[bucket(t)], 1)] = t;
}

// Each level's live segments in the order the GDN chunk walk deals them out
// (one block per level; a bucket sort, order within a bucket is whatever the
// atomics give).  Level 0 (roots): by decreasing number of chunks, so the
// longest items start first.  Deeper levels: grouped by entering state
// (fork point, or the cached history's state slot), so siblings that start
// from the same state are adjacent and a work-group stages it once.  Only
// the schedule of a level's launch depends on it; every item computes the
// same way in any order.
__device__ void level_order_block(int lvl, const int32_t *__restrict__ header, const int32_t *__restrict__ lvl_seg,
                                  const int32_t *__restrict__ seg_len, const int32_t *__restrict__ seg_src,
                                  int level_cap, int32_t *__restrict__ lvl_sorted, int *cnt, int *lds)
{
    const int n = header[H_LEVEL0 + lvl];
    if (n == 0) return;
    const int32_t *src = lvl_seg + (size_t)lvl * level_cap;
    int32_t *dst = lvl_sorted + (size_t)lvl * level_cap;
    for (int b = threadIdx.x; b < ORDER_BUCKETS; b += blockDim.x) cnt[b] = 0;
    __syncthreads();
    auto bucket = [&](int i) {
        if (lvl == 0) return min((seg_len[src[i]] + FK_GDN_CHUNK - 1) / FK_GDN_CHUNK, ORDER_BUCKETS - 1);
        const int e = seg_src[src[i]];   // >= 0 fork slot, <= -2 state_in slot
        return (e >= 0 ? e : -2 - e) % ORDER_BUCKETS;
    };
    for (int i = threadIdx.x; i < n; i += blockDim.x) atomicAdd(&cnt[bucket(i)], 1);
    __syncthreads();
    const int b0 = ORDER_BUCKETS - 1 - 2 * threadIdx.x, b1 = b0 - 1;
    int tot;
    const int before = block_scan(cnt[b0] + cnt[b1], lds, &tot);
    const int c0 = cnt[b0];
    __syncthreads();
    cnt[b0] = before;
    cnt[b1] = before + c0;
    __syncthreads();
    for (int i = threadIdx.x; i < n; i += blockDim.x) dst[atomicAdd(&cnt[bucket(i)], 1)] = src[i];
}

// Phase 3 (pages): one block per segment checks the page ids the segment
// uses, in parallel.  Runs only when the tree passed every other check.
__device__ void check_pages_block(int s, const int32_t *__restrict__ seg_len, const int32_t *__restrict__ page_off,
                                  const int32_t *__restrict__ pages, int page_size, int n_pages, int32_t *header)
{
    const int need = (seg_len[s] + page_size - 1) / page_size, a = page_off[s];
    for (int j = threadIdx.x; j < need; j += blockDim.x)
        if (!rule_page_id(pages[a + j], n_pages)) set_error(header, FK_E_PAGES);
}

__device__ void positions_thread(int t, const int32_t *__restrict__ tok_seg, int T, const int32_t *seg_start,
                                 const int32_t *seg_pos0, int32_t *tok_pos)
{
    if (t >= T) return;
    const int s = tok_seg[t];
    tok_pos[t] = s >= 0 ? seg_pos0[s] + (t - seg_start[s]) : -1;   // padding: no position
}

// After k_build, in one launch of BUILD_THREADS-thread blocks: the orders
// (block 0 the tiles, block 1 + l level l; [0, no)), the tile and chunk
// lists ([no, no + nl)), the page checks (one block per segment,
// [no + nl, no + nl + np)), the token positions (the rest).  No block reads
// what another writes.
__global__ void __launch_bounds__(BUILD_THREADS)
k_post(int no, int nl, int np, int S, int T, int32_t *header, const int32_t *__restrict__ seg_tile0,
       const int32_t *__restrict__ seg_coff, int32_t *__restrict__ tile_seg, int32_t *__restrict__ tile_row0,
       int32_t *__restrict__ chunk_seg, int32_t *__restrict__ chunk_row0, const int32_t *__restrict__ seg_len,
       const int32_t *__restrict__ page_off, const int32_t *__restrict__ pages, int page_size, int n_pages,
       const int32_t *__restrict__ tok_seg, const int32_t *__restrict__ seg_start,
       const int32_t *__restrict__ seg_pos0, int32_t *__restrict__ tok_pos, int32_t *__restrict__ tile_order,
       const int32_t *__restrict__ lvl_seg, const int32_t *__restrict__ seg_src, int level_cap,
       int32_t *__restrict__ lvl_sorted, const int32_t *__restrict__ seg_anc)
{
    __shared__ int cnt[ORDER_BUCKETS];
    __shared__ int stage[ORDER_STAGE];
    __shared__ int lds[32];
    if (header[H_STATUS] != FK_OK) return;
    const int b = blockIdx.x;
    if (b == 0)
        tile_order_block(header, S, seg_tile0, seg_pos0, seg_len, seg_anc, tile_order, cnt, lds, stage);
    else if (b < no)
        level_order_block(b - 1, header, lvl_seg, seg_len, seg_src, level_cap, lvl_sorted, cnt, lds);
    else if (b < no + nl)
        lists_thread((b - no) * BUILD_THREADS + threadIdx.x, S, header, seg_tile0, seg_coff, tile_seg, tile_row0,
                     chunk_seg, chunk_row0);
    else if (b < no + nl + np)
        check_pages_block(b - no - nl, seg_len, page_off, pages, page_size, n_pages, header);
    else
        positions_thread((b - no - nl - np) * BUILD_THREADS + threadIdx.x, tok_seg, T, seg_start, seg_pos0,
                         tok_pos);
}

int check_meta_scalars(const fk_tree_meta *m)
{
    if (!m) return FK_E_INVALID_ARG;
    if (m->T < 0 || m->S < 1 || m->max_depth < 1 || m->max_depth > FK_MAX_DEPTH ||
        m->level_cap < 1 || m->fork_cap < 0 || m->n_state_in < 0 || m->n_state_out < 0 ||
        m->n_pages < 0)
        return FK_E_INVALID_ARG;
    if (m->seg_page_off && m->page_size != FK_TILE_TOKENS) return FK_E_UNSUPPORTED;
    if ((m->T > 0 && !m->tok_seg) || !m->seg_parent || !m->seg_fork || !m->seg_cached_len)
        return FK_E_INVALID_ARG;
    if (m->seg_page_off && !m->seg_pages) return FK_E_INVALID_ARG;
    return FK_OK;
}

}  // namespace fk

using namespace fk;

extern "C" size_t fk_workspace_bytes(const fk_tree_meta *meta, int32_t gdn_Hv, int32_t gdn_dk, int32_t gdn_dv)
{
    if (!meta || gdn_Hv < 0 || gdn_dk < 0 || gdn_dv < 0) return 0;
    return ws_layout(*meta, gdn_Hv, gdn_dk, gdn_dv).total;
}

extern "C" int fk_tree_build(const fk_tree_meta *meta, void *ws, size_t ws_bytes, fk_stream_t stream)
{
    int rc = check_meta_scalars(meta);
    if (rc) return rc;
    if (!ws) return FK_E_INVALID_ARG;
    const WsLayout L = ws_layout(*meta, 0, 0, 0);
    if (ws_bytes < L.total) return FK_E_WORKSPACE;
    hipStream_t st = (hipStream_t)stream;
    BuildArgs A;
    A.m = *meta;
    A.header = ws_at<int32_t>(ws, L.header);
    A.seg_start = ws_at<int32_t>(ws, L.seg_start);
    A.seg_end = ws_at<int32_t>(ws, L.seg_end);
    A.seg_nrun = ws_at<int32_t>(ws, L.seg_nrun);
    A.seg_len = ws_at<int32_t>(ws, L.seg_len);
    A.seg_pos0 = ws_at<int32_t>(ws, L.seg_pos0);
    A.seg_depth = ws_at<int32_t>(ws, L.seg_depth);
    A.seg_anc = ws_at<int32_t>(ws, L.seg_anc);
    A.seg_src = ws_at<int32_t>(ws, L.seg_src);
    A.seg_owner = ws_at<int32_t>(ws, L.seg_owner);
    A.kid_cnt = ws_at<int32_t>(ws, L.kid_cnt);
    A.kid_off = ws_at<int32_t>(ws, L.kid_off);
    A.kid_fill = ws_at<int32_t>(ws, L.kid_fill);
    A.kids = ws_at<int32_t>(ws, L.kids);
    A.emit_off = ws_at<int32_t>(ws, L.emit_off);
    A.emit_pos = ws_at<int32_t>(ws, L.emit_pos);
    A.tile_seg = ws_at<int32_t>(ws, L.tile_seg);
    A.tile_row0 = ws_at<int32_t>(ws, L.tile_row0);
    A.lvl_seg = ws_at<int32_t>(ws, L.lvl_seg);
    A.chunk_seg = ws_at<int32_t>(ws, L.chunk_seg);
    A.chunk_row0 = ws_at<int32_t>(ws, L.chunk_row0);
    A.seg_chunk0 = ws_at<int32_t>(ws, L.seg_chunk0);
    A.seg_tile0 = ws_at<int32_t>(ws, L.seg_tile0);
    A.seg_coff = ws_at<int32_t>(ws, L.seg_coff);
    const int S = meta->S, T = meta->T;
    {
        const int nc = ((S > H_WORDS ? S : H_WORDS) + BUILD_THREADS - 1) / BUILD_THREADS;
        const int per = TOKENS_PER_THREAD * BUILD_THREADS, nt = T > 0 ? (T + per - 1) / per : 1;
        k_clear<<<(unsigned)nc, BUILD_THREADS, 0, st>>>(A);
        k_tokens<<<(unsigned)nt, BUILD_THREADS, 0, st>>>(A);
    }
    k_build<<<1, BUILD_THREADS, 0, st>>>(A);
    if ((rc = launch_status())) return rc;
    {
        const int64_t n = L.tile_cap > L.chunk_cap ? L.tile_cap : L.chunk_cap;
        const int no = 1 + meta->max_depth, nl = (int)((n + BUILD_THREADS - 1) / BUILD_THREADS);
        const int np = meta->seg_page_off ? S : 0, nt = (T + BUILD_THREADS - 1) / BUILD_THREADS;
        k_post<<<(unsigned)(no + nl + np + nt), BUILD_THREADS, 0, st>>>(
            no, nl, np, S, T, A.header, A.seg_tile0, A.seg_coff, A.tile_seg, A.tile_row0, A.chunk_seg,
            A.chunk_row0, A.seg_len, meta->seg_page_off, meta->seg_pages, meta->page_size, meta->n_pages,
            meta->tok_seg, A.seg_start, A.seg_pos0, ws_at<int32_t>(ws, L.tok_pos), ws_at<int32_t>(ws, L.tile_order),
            A.lvl_seg, ws_at<int32_t>(ws, L.seg_src), meta->level_cap, ws_at<int32_t>(ws, L.lvl_sorted), A.seg_anc);
        if ((rc = launch_status())) return rc;
    }
    return FK_OK;
}

extern "C" int fk_tree_validate_host(const fk_tree_meta *m)
{
    int rc = check_meta_scalars(m);
    if (rc) return rc;
    const int S = m->S, T = m->T;
    std::vector<int32_t> nrun(S, 0), start(S, 0), end(S, 0), len(S, 0);
    int code = FK_OK;
    for (int t = 0; t < T; ++t) {
        const int s = m->tok_seg[t];
        if (s == FK_PAD_TOKEN) {   // padding: only more padding may follow
            if (t + 1 < T && m->tok_seg[t + 1] != FK_PAD_TOKEN) code = imin(code, FK_E_SEG_RANGE);
            continue;
        }
        if (s < 0 || s >= S) { code = imin(code, FK_E_SEG_RANGE); continue; }
        if (t == 0 || m->tok_seg[t - 1] != s) { nrun[s]++; start[s] = t; }
        if (t == T - 1 || m->tok_seg[t + 1] != s) end[s] = t + 1;
    }
    if (code) return code;
    for (int s = 0; s < S; ++s)
        code = imin(code, rule_length(m->seg_cached_len[s], nrun[s], nrun[s] == 1 ? end[s] - start[s] : 0,
                                      &len[s]));
    if (code) return code;
    for (int s = 0; s < S; ++s) {
        SegDerived d;
        code = imin(code, rule_links(s, S, m->max_depth, m->seg_parent, m->seg_fork, m->seg_cached_len,
                                     len.data(), m->seg_state_in, m->n_state_in, m->seg_state_out,
                                     m->n_state_out, m->seg_page_off, m->seg_pages, m->page_size,
                                     m->n_pages, &d));
    }
    if (code) return code;
    // phase 3: capacities
    std::vector<int> per_level(FK_MAX_DEPTH, 0);
    for (int s = 0; s < S; ++s) {
        if (m->seg_cached_len[s] != 0) continue;   // cached or unused
        int depth = 0;
        for (int i = s; m->seg_parent[i] >= 0; i = m->seg_parent[i]) ++depth;
        per_level[depth]++;
    }
    for (int dd = 0; dd < FK_MAX_DEPTH; ++dd)
        if (per_level[dd] > m->level_cap) code = imin(code, FK_E_CAPACITY);
    long long forks = 0;
    for (int c = 0; c < S; ++c) {
        const int p = m->seg_parent[c];
        if (m->seg_cached_len[c] != 0 || p < 0 || m->seg_cached_len[p] != 0) continue;
        bool owner = true;
        for (int o = 0; o < c; ++o)
            if (m->seg_parent[o] == p && m->seg_cached_len[o] == 0 && m->seg_fork[o] == m->seg_fork[c])
                owner = false;
        forks += owner;
    }
    if (forks > m->fork_cap) code = imin(code, FK_E_CAPACITY);
    if (code || !m->seg_page_off || !m->seg_pages) return code;
    for (int s = 0; s < S; ++s) {
        const int need = (len[s] + m->page_size - 1) / m->page_size;
        for (int j = 0; j < need; ++j)
            if (!rule_page_id(m->seg_pages[m->seg_page_off[s] + j], m->n_pages)) return FK_E_PAGES;
    }
    return code;
}

extern "C" int fk_token_positions(const fk_tree_meta *meta, const void *ws, int32_t *pos, fk_stream_t stream)
{
    int rc = check_meta_scalars(meta);
    if (rc) return rc;
    if (!ws || (meta->T > 0 && !pos)) return FK_E_INVALID_ARG;
    if (meta->T == 0) return FK_OK;
    const WsLayout L = ws_layout(*meta, 0, 0, 0);
    FK_HIP(hipMemcpyAsync(pos, ws_at<int32_t>(ws, L.tok_pos), (size_t)meta->T * 4, hipMemcpyDeviceToDevice,
                          (hipStream_t)stream));
    return FK_OK;
}

extern "C" int fk_read_status(const void *ws, fk_stream_t stream, int32_t *status_out)
{
    if (!ws || !status_out) return FK_E_INVALID_ARG;
    int32_t v = 0;
    FK_HIP(hipMemcpyAsync(&v, ws, sizeof(int32_t), hipMemcpyDeviceToHost, (hipStream_t)stream));
    FK_HIP(hipStreamSynchronize((hipStream_t)stream));
    *status_out = v;
    return FK_OK;
}

extern "C" const char *fk_strerror(int code)
{
    switch (code) {
    case FK_OK: return "ok";
    case FK_E_INVALID_ARG: return "invalid argument";
    case FK_E_UNSUPPORTED: return "unsupported shape or dtype";
    case FK_E_WORKSPACE: return "workspace too small";
    case FK_E_HIP: return "HIP runtime error";
    case FK_E_SEG_RANGE: return "token names a segment outside [0, S)";
    case FK_E_NONCONTIG: return "segment tokens are not contiguous in the stream";
    case FK_E_PARENT: return "parent index out of range";
    case FK_E_CYCLE: return "parent chain loops or exceeds max_depth";
    case FK_E_FORK: return "fork offset outside the parent";
    case FK_E_EMPTY: return "live segment without tokens, or cached segment with tokens";
    case FK_E_CACHED: return "cached segment misplaced, or child forks inside a cached history";
    case FK_E_PAGES: return "page list too short or page id out of range";
    case FK_E_CAPACITY: return "level or fork-point capacity exceeded";
    case FK_E_STATE_SLOT: return "state slot missing or out of range";
    default: return "unknown status";
    }
}

extern "C" int fk_abi_version(void) { return 1; }
