// conv.hip -- the short causal convolution in front of the Gated DeltaNet
// rule, forked through the tree (Flide, section 3.2.2: the convolution mixes
// each token with its few predecessors and reads them through the same kind
// of index as the recurrent state, so the first tokens of a question see the
// last tokens of the state it forks from; section 3.4: a checkpoint keeps the
// convolution window of every Gated DeltaNet layer).
//
// Depthwise and linear, width W:  y_t[c] = sum_{i<W} w[c][i] x_{p_i(t)}[c],
// where p_0(t) = t and p_i(t) is the i-th predecessor of t along its isolated
// root-to-leaf sequence (zero before that sequence's first row).  The sum runs
// in fp32, i = 0 .. W-1 in that order, so a row's bits depend only on its own
// path (batch invariant).
//
// Work item = (16-token attention tile of one segment, 2048 / 1024 channels).
// A thread owns one 16-byte channel vector of the tile: it loads the W-1 rows
// before the tile (the halo) and the tile's rows into registers once, and
// writes each output row once -- an HBM-bound stream, read once and written
// once, halo rows aside (neighbouring tiles of one XCD share them in L2).
// The tile's own rows are read and the outputs written with non-temporal
// accesses (streamed, not kept in the caches).
// Halo rows before a segment's first token come from the ancestor chain the
// builder derived: a live ancestor's token, or, below a cached history, the
// history's saved window (window_in of its state slot).  The tile holding a
// segment's last token also writes the segment's window (its path's last W-1
// inputs) to window_out when the segment has a state_out slot.
#include <hip/hip_runtime.h>

#include "fk_common.h"

namespace fk {
namespace convk {

constexpr int TILE = FK_TILE_TOKENS;   // 16 rows per work item
constexpr int THREADS = 256;
constexpr int XCDS = 8;                // work-groups are dealt to the 8 XCDs round-robin

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

struct ConvArgs {
    const void *x;          // [T, C]
    const float *w;         // [C, W]
    const void *window_in;  // [n_state_in, W-1, C] or null
    void *window_out;       // [n_state_out, W-1, C] or null
    void *y;                // [T, C]
    int32_t *header;
    const int32_t *tile_seg, *tile_row0;
    const int32_t *seg_start, *seg_len, *seg_pos0, *seg_depth, *seg_anc;
    const int32_t *seg_cached_len, *seg_state_in, *seg_state_out;
    int C;
    int n_cb;               // channel blocks per tile
};

template <typename E>
struct VecOf;
template <>
struct VecOf<uint16_t> {
    static constexpr int N = 8;
    __device__ static void to_f32(const uint4 &u, float *f)
    {
        const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            f[2 * j] = __uint_as_float(w[j] << 16);
            f[2 * j + 1] = __uint_as_float(w[j] & 0xffff0000u);
        }
    }
    __device__ static uint4 from_f32(const float *f)
    {
        uint32_t w[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) w[j] = (uint32_t)f32_to_bf16(f[2 * j]) | ((uint32_t)f32_to_bf16(f[2 * j + 1]) << 16);
        return make_uint4(w[0], w[1], w[2], w[3]);
    }
};
template <>
struct VecOf<float> {
    static constexpr int N = 4;
    __device__ static void to_f32(const uint4 &u, float *f)
    {
        f[0] = __uint_as_float(u.x);
        f[1] = __uint_as_float(u.y);
        f[2] = __uint_as_float(u.z);
        f[3] = __uint_as_float(u.w);
    }
    __device__ static uint4 from_f32(const float *f)
    {
        return make_uint4(__float_as_uint(f[0]), __float_as_uint(f[1]), __float_as_uint(f[2]), __float_as_uint(f[3]));
    }
};

// Where path row `rho` of segment s's isolated sequence lives, for a row
// before s's own tokens: *tok = stream token, or *wrow = row of window_in
// (slot * (W-1) + index), or neither (zero: before the sequence's start).
// Walks s's ancestors deepest first: a live ancestor a shows the rows
// [pos0[a], pos0[next on the chain]); the first cached ancestor met holds the
// last W-1 rows of everything above, in its saved window.
__device__ __forceinline__ void locate(const ConvArgs &A, int s, int rho, int W, int64_t *tok, int64_t *wrow)
{
    *tok = -1;
    *wrow = -1;
    if (rho < 0) return;
    const int depth = A.seg_depth[s];
    const int32_t *anc = A.seg_anc + (size_t)s * FK_MAX_DEPTH;
    for (int l = depth - 1; l >= 0; --l) {
        const int a = anc[l], next = anc[l + 1];
        if (A.seg_cached_len[a] > 0) {
            const int slot = A.seg_state_in ? A.seg_state_in[a] : -1;
            if (slot < 0 || !A.window_in) {
                set_error(A.header, FK_E_STATE_SLOT);
                return;
            }
            *wrow = (int64_t)slot * (W - 1) + (rho - (A.seg_pos0[next] - (W - 1)));
            return;
        }
        if (rho >= A.seg_pos0[a]) {
            *tok = (int64_t)A.seg_start[a] + (rho - A.seg_pos0[a]);
            return;
        }
    }
}

template <typename E, int W>
__global__ void __launch_bounds__(THREADS) k_conv(ConvArgs A)
{
    using V = VecOf<E>;
    constexpr int NV = V::N;
    constexpr int H = W - 1;   // halo rows
    if (A.header[H_STATUS] != FK_OK) return;
    // XCD-aware order: XCD x takes a contiguous run of tiles, channel blocks
    // of one tile back to back, so halo rows are shared inside one L2.
    const int n_tiles = A.header[H_NTILES];
    const int per_xcd = (n_tiles + XCDS - 1) / XCDS;
    const int xcd = blockIdx.x % XCDS, k = blockIdx.x / XCDS;
    const int t_in = k / A.n_cb, cb = k % A.n_cb;
    if (t_in >= per_xcd) return;
    const int tile = xcd * per_xcd + t_in;
    if (tile >= n_tiles) return;
    const int c0 = (cb * THREADS + threadIdx.x) * NV;
    if (c0 >= A.C) return;

    const int s = A.tile_seg[tile], row0 = A.tile_row0[tile];
    const int len = A.seg_len[s];
    const int count = min(TILE, len - row0);
    const int64_t t0 = (int64_t)A.seg_start[s] + row0;
    const size_t C = (size_t)A.C;
    const E *x = static_cast<const E *>(A.x);
    const E *win = static_cast<const E *>(A.window_in);

    // rows[h]: path row (pos0 + row0 - H + h); h < H is the halo
    uint4 rows[H + TILE];
#pragma unroll
    for (int h = 0; h < H; ++h) {
        const int local = row0 - H + h;   // local index in s (may be negative)
        rows[h] = make_uint4(0, 0, 0, 0);
        if (local >= 0) {
            rows[h] = *reinterpret_cast<const uint4 *>(x + (size_t)(A.seg_start[s] + local) * C + c0);
        } else {
            int64_t tok, wrow;
            locate(A, s, A.seg_pos0[s] + local, W, &tok, &wrow);
            if (tok >= 0) rows[h] = *reinterpret_cast<const uint4 *>(x + (size_t)tok * C + c0);
            else if (wrow >= 0) rows[h] = *reinterpret_cast<const uint4 *>(win + (size_t)wrow * C + c0);
        }
    }
#pragma unroll
    for (int r = 0; r < TILE; ++r) {
        rows[H + r] = make_uint4(0, 0, 0, 0);
        if (r < count) {
            const u32x4 vv = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(x + (size_t)(t0 + r) * C + c0));
            rows[H + r] = make_uint4(vv.x, vv.y, vv.z, vv.w);
        }
    }

    float wt[W][NV];
#pragma unroll
    for (int j = 0; j < NV; ++j)
#pragma unroll
        for (int i = 0; i < W; ++i) wt[i][j] = A.w[(size_t)(c0 + j) * W + i];

    E *y = static_cast<E *>(A.y);
#pragma unroll
    for (int r = 0; r < TILE; ++r) {
        if (r < count) {
            float acc[NV], xv[NV];
            V::to_f32(rows[H + r], xv);
#pragma unroll
            for (int j = 0; j < NV; ++j) acc[j] = wt[0][j] * xv[j];
#pragma unroll
            for (int i = 1; i < W; ++i) {
                V::to_f32(rows[H + r - i], xv);
#pragma unroll
                for (int j = 0; j < NV; ++j) acc[j] = fmaf(wt[i][j], xv[j], acc[j]);
            }
            const uint4 vv = V::from_f32(acc);
            __builtin_nontemporal_store(u32x4{vv.x, vv.y, vv.z, vv.w}, reinterpret_cast<u32x4 *>(y + (size_t)(t0 + r) * C + c0));
        }
    }

    // the segment's window: inputs of its path's last W-1 rows, oldest first
    if (H > 0 && A.window_out && row0 + count == len) {
        const int slot = A.seg_state_out ? A.seg_state_out[s] : -1;
        if (slot >= 0) {
            E *wo = static_cast<E *>(A.window_out) + (size_t)slot * H * C + c0;
#pragma unroll
            for (int kk = 0; kk < (H > 0 ? H : 1); ++kk) {
                // path row pos0 + len - H + kk  ->  rows[H + (len - H + kk - row0)] = rows[count + kk]
#pragma unroll
                for (int h = 0; h < H + TILE; ++h)
                    if (h == count + kk) *reinterpret_cast<uint4 *>(wo + (size_t)kk * C) = rows[h];
            }
        }
    }
}

template <typename E, int W>
void launch_w(const ConvArgs &A, unsigned blocks, hipStream_t st)
{
    k_conv<E, W><<<blocks, THREADS, 0, st>>>(A);
}

template <typename E>
int launch(const ConvArgs &A, int W, unsigned blocks, hipStream_t st)
{
    switch (W) {
    case 1: launch_w<E, 1>(A, blocks, st); break;
    case 2: launch_w<E, 2>(A, blocks, st); break;
    case 3: launch_w<E, 3>(A, blocks, st); break;
    case 4: launch_w<E, 4>(A, blocks, st); break;
    case 5: launch_w<E, 5>(A, blocks, st); break;
    case 6: launch_w<E, 6>(A, blocks, st); break;
    case 7: launch_w<E, 7>(A, blocks, st); break;
    case 8: launch_w<E, 8>(A, blocks, st); break;
    default: return FK_E_UNSUPPORTED;
    }
    return launch_status();
}

}  // namespace convk
}  // namespace fk

using namespace fk;

extern "C" int gdn_conv_forward(const fk_tree_meta *meta, const void *x, int dtype, int C, int W, const float *w,
                                const void *window_in, void *window_out, void *y, void *ws, size_t ws_bytes,
                                fk_stream_t stream)
{
    int rc = check_meta_scalars(meta);
    if (rc) return rc;
    if (!ws || (meta->T > 0 && (!x || !w || !y))) return FK_E_INVALID_ARG;
    if (dtype != FK_F32 && dtype != FK_BF16) return FK_E_UNSUPPORTED;
    const int nv = dtype == FK_BF16 ? 8 : 4;
    if (C < 1 || C % nv || W < 1 || W > FK_CONV_MAX_W) return FK_E_UNSUPPORTED;
    if (((uintptr_t)x | (uintptr_t)y | (uintptr_t)window_in | (uintptr_t)window_out) & 15) return FK_E_INVALID_ARG;
    if (W > 1 && meta->n_state_out > 0 && meta->seg_state_out && !window_out) return FK_E_INVALID_ARG;
    const WsLayout L = ws_layout(*meta, 0, 0, 0);
    if (ws_bytes < L.total) return FK_E_WORKSPACE;
    if (meta->T == 0) return FK_OK;
    convk::ConvArgs A;
    A.x = x;
    A.w = w;
    A.window_in = W > 1 ? window_in : nullptr;
    A.window_out = W > 1 ? window_out : nullptr;
    A.y = y;
    A.header = ws_at<int32_t>(ws, L.header);
    A.tile_seg = ws_at<int32_t>(ws, L.tile_seg);
    A.tile_row0 = ws_at<int32_t>(ws, L.tile_row0);
    A.seg_start = ws_at<int32_t>(ws, L.seg_start);
    A.seg_len = ws_at<int32_t>(ws, L.seg_len);
    A.seg_pos0 = ws_at<int32_t>(ws, L.seg_pos0);
    A.seg_depth = ws_at<int32_t>(ws, L.seg_depth);
    A.seg_anc = ws_at<int32_t>(ws, L.seg_anc);
    A.seg_cached_len = meta->seg_cached_len;
    A.seg_state_in = meta->seg_state_in;
    A.seg_state_out = meta->seg_state_out;
    A.C = C;
    A.n_cb = (C / nv + convk::THREADS - 1) / convk::THREADS;
    const int64_t per_xcd = (L.tile_cap + convk::XCDS - 1) / convk::XCDS;
    const int64_t blocks = per_xcd * convk::XCDS * A.n_cb;
    if (blocks > 0x7fffffff) return FK_E_UNSUPPORTED;
    hipStream_t st = (hipStream_t)stream;
    return dtype == FK_BF16 ? convk::launch<uint16_t>(A, W, (unsigned)blocks, st)
                            : convk::launch<float>(A, W, (unsigned)blocks, st);
}
