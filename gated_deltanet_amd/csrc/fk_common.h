// fk_common.h -- internal definitions shared by the library's translation
// units: workspace layout, launch helpers, and bf16 conversion.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/forkgdn.h"

namespace fk {

// ---------------------------------------------------------------------------
// Workspace layout (derived metadata of one round + GDN fork-point states).
// Every region is 256-byte aligned.  The header holds the status word and the
// device-computed counts that size the work of later kernels.
// ---------------------------------------------------------------------------
enum HeaderSlot {
    H_STATUS = 0,       // FK_OK or the first (most negative) tree error
    H_NTILES = 1,       // attention tiles in tile_seg / tile_row0
    H_NFORKS = 2,       // distinct fork points (GDN fork-state slots used)
    H_NCHUNKS = 3,      // GDN chunks in chunk_seg / chunk_row0
    H_LEVEL0 = 4,       // live segments per level: H_LEVEL0 + d, d < FK_MAX_DEPTH
    H_MAXKEYS = H_LEVEL0 + FK_MAX_DEPTH,   // most keys any tile's rows see (>= 1)
    H_WORDS = 64
};
static_assert(H_MAXKEYS < H_WORDS, "header slots");

struct WsLayout {
    size_t header;        // int32[H_WORDS]
    size_t seg_start;     // int32[S]  first stream token (-1 for cached)
    size_t seg_end;       // int32[S]  one past the last stream token (scratch)
    size_t seg_nrun;      // int32[S]  contiguous token runs (scratch, must be 1)
    size_t seg_len;       // int32[S]  tokens (stream count, or cached length)
    size_t seg_pos0;      // int32[S]  first position
    size_t seg_depth;     // int32[S]
    size_t seg_anc;       // int32[S*FK_MAX_DEPTH] ancestors root-first, self last
    size_t seg_src;       // int32[S]  GDN start state: -1 zero, >=0 fork slot,
                          //           <= -2: state_in slot (-2 - value)
    size_t seg_owner;     // int32[S]  scratch: first child at its fork offset
    size_t kid_cnt;       // int32[S]
    size_t kid_off;       // int32[S+1]
    size_t kid_fill;      // int32[S]
    size_t kids;          // int32[S]
    size_t emit_off;      // int32[S+1] fork points of each segment (CSR)
    size_t emit_pos;      // int32[fork_cap] offset of each fork point
    size_t tok_pos;       // int32[T]
    size_t tile_seg;      // int32[tile_cap]
    size_t tile_row0;     // int32[tile_cap]
    size_t tile_order;    // int32[tile_cap]   tiles by decreasing work, grouped by root
    size_t seg_tile0;     // int32[S]  first tile of each segment (non-decreasing)
    size_t seg_coff;      // int32[S]  first chunk of each segment (non-decreasing)
    size_t lvl_seg;       // int32[FK_MAX_DEPTH*level_cap]
    size_t lvl_sorted;    // int32[FK_MAX_DEPTH*level_cap] each level by decreasing chunk count
    size_t chunk_seg;     // int32[chunk_cap] segment of each GDN chunk
    size_t chunk_row0;    // int32[chunk_cap] first local token of each chunk
    size_t seg_chunk0;    // int32[S] index of a live segment's first chunk
    size_t fork_states;   // float[fork_cap * Hv * dv * dk]
    size_t tmat;          // bf16[chunk_cap * Hv * FK_GDN_CHUNK^2] per-chunk (I + A)^-1
    size_t pmat;          // bf16[chunk_cap * Hv * FK_GDN_CHUNK^2] per-chunk Gamma o Q K^T
    size_t lvec;          // float[chunk_cap * Hv * FK_GDN_CHUNK] per-chunk log-decay prefix l_i
    size_t total;
    int64_t tile_cap;
    int64_t chunk_cap;
};

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

inline int64_t tile_capacity(int64_t T, int64_t S)
{
    return (T + FK_TILE_TOKENS - 1) / FK_TILE_TOKENS + S;
}

inline int64_t chunk_capacity(int64_t T, int64_t S)
{
    return (T + FK_GDN_CHUNK - 1) / FK_GDN_CHUNK + S;
}

// Hv, dk, dv: the largest Gated DeltaNet layer that will use the workspace
// (0 if none).
inline WsLayout ws_layout(const fk_tree_meta &m, int64_t Hv, int64_t dk, int64_t dv)
{
    const int64_t state_elems = Hv * dk * dv;
    WsLayout L{};
    size_t off = 0;
    auto take = [&](size_t bytes) {
        size_t at = off;
        off = align256(off + bytes);
        return at;
    };
    const size_t S = (size_t)(m.S > 0 ? m.S : 0), T = (size_t)(m.T > 0 ? m.T : 0);
    const size_t fc = (size_t)(m.fork_cap > 0 ? m.fork_cap : 0);
    L.tile_cap = tile_capacity((int64_t)T, (int64_t)S);
    L.chunk_cap = chunk_capacity((int64_t)T, (int64_t)S);
    L.header = take(H_WORDS * 4);
    L.seg_start = take(S * 4);
    L.seg_end = take(S * 4);
    L.seg_nrun = take(S * 4);
    L.seg_len = take(S * 4);
    L.seg_pos0 = take(S * 4);
    L.seg_depth = take(S * 4);
    L.seg_anc = take(S * FK_MAX_DEPTH * 4);
    L.seg_src = take(S * 4);
    L.seg_owner = take(S * 4);
    L.kid_cnt = take(S * 4);
    L.kid_off = take((S + 1) * 4);
    L.kid_fill = take(S * 4);
    L.kids = take(S * 4);
    L.emit_off = take((S + 1) * 4);
    L.emit_pos = take((fc > 0 ? fc : 1) * 4);
    L.tok_pos = take((T > 0 ? T : 1) * 4);
    L.tile_seg = take((size_t)L.tile_cap * 4);
    L.tile_row0 = take((size_t)L.tile_cap * 4);
    L.tile_order = take((size_t)L.tile_cap * 4);
    L.seg_tile0 = take(S * 4);
    L.seg_coff = take(S * 4);
    L.lvl_seg = take((size_t)FK_MAX_DEPTH * (size_t)(m.level_cap > 0 ? m.level_cap : 1) * 4);
    L.lvl_sorted = take((size_t)FK_MAX_DEPTH * (size_t)(m.level_cap > 0 ? m.level_cap : 1) * 4);
    L.chunk_seg = take((size_t)L.chunk_cap * 4);
    L.chunk_row0 = take((size_t)L.chunk_cap * 4);
    L.seg_chunk0 = take(S * 4);
    L.fork_states = take(fc * (size_t)(state_elems > 0 ? state_elems : 0) * 4);
    L.tmat = take((size_t)L.chunk_cap * (size_t)(Hv > 0 ? Hv : 0) * FK_GDN_CHUNK * FK_GDN_CHUNK * 2);
    L.pmat = take((size_t)L.chunk_cap * (size_t)(Hv > 0 ? Hv : 0) * FK_GDN_CHUNK * FK_GDN_CHUNK * 2);
    L.lvec = take((size_t)L.chunk_cap * (size_t)(Hv > 0 ? Hv : 0) * FK_GDN_CHUNK * 4);
    L.total = off;
    return L;
}

template <typename T>
inline T *ws_at(void *ws, size_t off) { return reinterpret_cast<T *>(static_cast<char *>(ws) + off); }
template <typename T>
inline const T *ws_at(const void *ws, size_t off)
{
    return reinterpret_cast<const T *>(static_cast<const char *>(ws) + off);
}

// Scalar checks of the round description that need no device data.
int check_meta_scalars(const fk_tree_meta *m);

#define FK_HIP(call)                                   \
    do {                                               \
        if ((call) != hipSuccess) return FK_E_HIP;     \
    } while (0)

inline int launch_status() { return hipGetLastError() == hipSuccess ? FK_OK : FK_E_HIP; }

// ---------------------------------------------------------------------------
// Device helpers
// ---------------------------------------------------------------------------
__device__ __forceinline__ void set_error(int32_t *header, int code)
{
    atomicMin(header + H_STATUS, code);   // deterministic: the most negative code wins
}

__device__ __forceinline__ float bf16_to_f32(uint16_t x)
{
    return __uint_as_float(((uint32_t)x) << 16);
}

// fp32 -> bf16, round to nearest even (finite inputs; NaN stays NaN).
__device__ __forceinline__ uint16_t f32_to_bf16(float f)
{
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

}  // namespace fk
