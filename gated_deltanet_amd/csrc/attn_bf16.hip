// attn_bf16.hip -- ForkAttention prefill on bf16 MFMA for gfx950
// (Flide section 3.2.1, Eq. 3; section 3.3.1: fully visible key blocks are
// read without a mask and only the partially visible ones are masked).
//
// Work item: one 16-token tile of one segment x one kv head.  The tile's
// 16 tokens x 8 q heads of the GQA group form 128 query rows; each of the 4
// waves owns 32 rows (4 tokens x 8 heads), so a key/value block staged once in
// LDS feeds the whole group.  Keys are visited range by range along the
// tile's ancestor chain (each ancestor's first `fork` tokens, then the own
// segment causally), in 32-key blocks anchored at every range start; a row's
// reduction order therefore depends only on its own chain (Flide 3.5).
// A block pair of LDS buffers takes 38 KB, and the kernel 161 VGPRs, so three
// work-groups (12 waves) share a compute unit.
//
// Per block and wave, with v_mfma_f32_32x32x16_bf16 (fp32 accumulate):
//   S^T[32 keys x 32 rows] = K_blk[32 x 128] . Q^T[128 x 32]       8 MFMAs
//   online softmax on S^T in registers (row = lane % 32; the two halves of
//   the wave hold disjoint keys of the same row; max via one permlane32 swap)
//   O^T[128 x 32] += V^T[128 x 32] . P^T[32 x 32]                  8 MFMAs
// The four 32-dim output chains are interleaved, and LDS operand reads are
// issued LOOKAHEAD instructions ahead of their MFMAs.
// A row's reference maximum moves only when a block exceeds it by more than
// 2^RESCALE_LOG2 (the exponentials stay bounded by that factor), so most
// blocks skip the rescale of the output accumulators; the decision is per
// row, and a row that does not move multiplies by exactly 1.
// The accumulator layout of S^T is reused directly as the P^T operand: the
// K rows are loaded under a fixed permutation (bits 2 and 3 of the row index
// swapped) so that each lane's accumulator registers hold 8 consecutive keys
// of the V^T operand.  Values sit transposed in their pages ([d][slot]), so
// V^T rows are contiguous in LDS.
#include <hip/hip_runtime.h>

#include "fk_common.h"

namespace fk {
namespace attn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int D = 128;           // head dim
constexpr int G = 8;             // q heads per kv head
constexpr int BN = 32;           // keys per block
constexpr int MT = BN / 32;      // 32-key MFMA tiles per block
constexpr int WAVES = 4;
constexpr int THREADS = WAVES * 64;
constexpr int K_STRIDE = D + 8;  // LDS row stride (bf16) of the key tile, padded
constexpr int V_STRIDE = BN + 8; // LDS row stride (bf16) of the transposed value tile
constexpr int K_LDS = BN * K_STRIDE;
constexpr int V_LDS = D * V_STRIDE;

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 u) { return __builtin_bit_cast(bf16x8, u); }

// max / sum of a lane's value and that of lane (lane ^ 32): one permlane32
// swap gives every lane both values (the two halves of a wave hold disjoint
// keys of the same rows); the sum is commutative, so both halves agree
__device__ __forceinline__ float pair_max(float x)
{
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __builtin_fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x)
{
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

constexpr float RESCALE_LOG2 = 8.f;
constexpr int LOOKAHEAD = 2;   // LDS operand reads issued ahead of the MFMAs

__device__ __forceinline__ uint4 pack8(const float *x)
{
    bf16x8 v;
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = (__bf16)x[e];
    return __builtin_bit_cast(uint4, v);
}

// One block of a range = BN / 16 pages of 16 keys.  Keys [BN][D] and
// transposed values [D][BN] of a block are loaded into registers (two 16-byte
// pieces per page and thread) and later written into one of two LDS buffers.
// Pages past the range's valid keys are zero, so no page-list entry beyond
// the range is ever read.
struct BlockRegs {
    uint4 k[BN / FK_TILE_TOKENS], v[BN / FK_TILE_TOKENS];
};

__device__ __forceinline__ void load_block(BlockRegs &R, const uint16_t *__restrict__ kp,
                                           const uint16_t *__restrict__ vp, const int32_t *__restrict__ plist,
                                           int key0, int count, int g, int Hkv)
{
    const int tid = threadIdx.x;
#pragma unroll
    for (int p = 0; p < BN / FK_TILE_TOKENS; ++p) {
        const int kbase = key0 + p * FK_TILE_TOKENS;
        R.k[p] = R.v[p] = make_uint4(0, 0, 0, 0);
        if (kbase < count) {
            const size_t pb = ((size_t)plist[kbase / FK_TILE_TOKENS] * Hkv + g) * (FK_TILE_TOKENS * D);
            R.k[p] = *reinterpret_cast<const uint4 *>(kp + pb + tid * 8);   // slot tid/16, dims (tid%16)*8
            R.v[p] = *reinterpret_cast<const uint4 *>(vp + pb + tid * 8);   // dim tid/2, slots (tid%2)*8
        }
    }
}

__device__ __forceinline__ void store_block(uint16_t *__restrict__ ks, uint16_t *__restrict__ vs, const BlockRegs &R)
{
    const int tid = threadIdx.x;
#pragma unroll
    for (int p = 0; p < BN / FK_TILE_TOKENS; ++p) {
        *reinterpret_cast<uint4 *>(ks + (p * FK_TILE_TOKENS + tid / 16) * K_STRIDE + (tid % 16) * 8) = R.k[p];
        *reinterpret_cast<uint4 *>(vs + (tid / 2) * V_STRIDE + p * FK_TILE_TOKENS + (tid % 2) * 8) = R.v[p];
    }
}

// Visibility rules (Flide section 3.2.1): causal (t_y <= t_x); a sliding
// window of width W that also requires t_x - t_y < W; and two-way, where a row
// sees every token of its own segment (models that read each block both
// ways, Flide appendix H) -- ancestors always show their first `fork` tokens.
enum Rule { CAUSAL = FK_RULE_CAUSAL, WINDOW = FK_RULE_WINDOW, TWO_WAY = FK_RULE_TWO_WAY };

// What a tile's key walk needs to know about its chain.
struct TileCtx {
    int depth, row0, len, pos0, window;
    const int *anc;
    const int32_t *seg_fork, *seg_pos0, *page_off, *pages;
};

// Walks a tile's key blocks in order: each ancestor's visible prefix, then the
// own segment; blocks are anchored at the start of every range.  Under the
// window rule a range starts at the first block that holds a key inside the
// window of the tile's first row (earlier blocks are invisible to every row
// of the tile and are skipped whole).
struct BlockCursor {
    int lvl, key0, count, pdiff;   // pdiff = pos0(tile segment) - pos0(range segment)
    bool own;
    const int32_t *plist;
};

template <int RULE>
__device__ __forceinline__ void cursor_level(BlockCursor &c, int lvl, const TileCtx &t)
{
    c.lvl = lvl;
    c.own = lvl == t.depth;
    c.count = c.own ? (RULE == TWO_WAY ? t.len : min(t.row0 + FK_TILE_TOKENS, t.len)) : t.seg_fork[t.anc[lvl + 1]];
    c.plist = t.pages + t.page_off[t.anc[lvl]];
    c.pdiff = t.pos0 - t.seg_pos0[t.anc[lvl]];
    c.key0 = 0;
    if (RULE == WINDOW) {
        const int lo = c.pdiff + t.row0 - t.window + 1;   // first key the tile's first row sees
        if (lo > 0) c.key0 = (lo / BN) * BN;
    }
}

// first block at or after level `lvl` (a range whose blocks all lie outside
// the window, or an empty range, is passed over); the own range is never empty
template <int RULE>
__device__ __forceinline__ void cursor_settle(BlockCursor &c, const TileCtx &t)
{
    while (c.key0 >= c.count && c.lvl < t.depth) cursor_level<RULE>(c, c.lvl + 1, t);
}

// move to the next block; returns false past the last one
template <int RULE>
__device__ __forceinline__ bool cursor_next(BlockCursor &c, const TileCtx &t)
{
    c.key0 += BN;
    if (c.key0 < c.count) return true;
    if (c.lvl >= t.depth) return false;
    cursor_level<RULE>(c, c.lvl + 1, t);
    cursor_settle<RULE>(c, t);
    return true;
}

// READOUT (selective readout, Flide section 3.3.3): work item = (selected
// row, kv head) instead of (tile, kv head).
// The work-group runs the tile that holds the selected token exactly as the
// full launch does, but only the wave that owns the token computes, its
// other rows read zero queries, and only the token's 8 rows are stored --
// so a readout row has the same bits as the same row of the full launch.
template <int RULE, bool READOUT>
__global__ void __launch_bounds__(THREADS, 3)
k_attn_bf16(const uint16_t *__restrict__ q, int Hq, int Hkv, float scale_log2e, int window,
            const int32_t *__restrict__ sel_rows, const int32_t *__restrict__ tok_seg, int T,
            const int32_t *__restrict__ seg_pos0, const uint16_t *__restrict__ kp,
            const uint16_t *__restrict__ vp, uint16_t *__restrict__ out, const int32_t *__restrict__ header,
            const int32_t *__restrict__ tile_seg, const int32_t *__restrict__ tile_row0,
            const int32_t *__restrict__ tile_order, const int32_t *__restrict__ seg_start,
            const int32_t *__restrict__ seg_len, const int32_t *__restrict__ seg_depth,
            const int32_t *__restrict__ seg_anc, const int32_t *__restrict__ seg_fork,
            const int32_t *__restrict__ page_off, const int32_t *__restrict__ pages)
{
    __shared__ __attribute__((aligned(16))) uint16_t k_lds[2][K_LDS];
    __shared__ __attribute__((aligned(16))) uint16_t v_lds[2][V_LDS];
    if (header[H_STATUS] != FK_OK) return;
    // heaviest tiles first (both kv heads of a tile side by side), so the
    // launch does not end on a long tile started late
    const int rank = blockIdx.x / Hkv, g = blockIdx.x % Hkv;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int half = lane >> 5, n = lane & 31;
    int s, row0, sel_local = 0;
    if (READOUT) {
        const int t = sel_rows[rank];
        if (t < 0 || t >= T) return;   // an unused entry of the row buffer
        s = tok_seg[t];
        sel_local = t - seg_start[s];
        row0 = sel_local & ~(FK_TILE_TOKENS - 1);
    } else {
        if (rank >= header[H_NTILES]) return;
        const int tile = tile_order[rank];
        s = tile_seg[tile];
        row0 = tile_row0[tile];
    }
    const int len = seg_len[s];
    const int tok = row0 + w * 4 + n / 8;          // local token of this lane's row
    const int h = g * G + (n % 8);
    const bool row_valid = READOUT ? tok == sel_local : tok < len;
    // the wave that owns the selected token (all waves in a full launch)
    const bool active = !READOUT || w == ((sel_local - row0) >> 2);
    const size_t t_glob = (size_t)seg_start[s] + tok;
    // query / output row: the stream token, or the row buffer's entry
    const size_t qrow = READOUT ? (size_t)rank * Hq + h : t_glob * Hq + h;

    // Q^T as the B operand: lane holds its row's dims 16*ks + 8*half + [0, 8)
    bf16x8 qf[D / 16];
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
        uint4 u = make_uint4(0, 0, 0, 0);
        if (row_valid) u = *reinterpret_cast<const uint4 *>(q + qrow * D + ks * 16 + half * 8);
        qf[ks] = as_bf16x8(u);
    }
    f32x16 o[D / 32];
#pragma unroll
    for (int i = 0; i < D / 32; ++i) o[i] = f32x16{};
    // a finite floor for the reference max: under the window rule a row may
    // meet a block with no visible key before its first visible one
    float m = -1e30f, l = 0.f;

    const int depth = seg_depth[s];
    const int *anc = seg_anc + s * FK_MAX_DEPTH;
    // MFMA row m of a 32-key tile holds key perm(m): bits 2 and 3 swapped
    const int prow = (n & ~12) | ((n & 4) << 1) | ((n & 8) >> 1);

    TileCtx tc;
    tc.depth = depth;
    tc.row0 = row0;
    tc.len = len;
    tc.pos0 = seg_pos0[s];
    tc.window = window;
    tc.anc = anc;
    tc.seg_fork = seg_fork;
    tc.seg_pos0 = seg_pos0;
    tc.page_off = page_off;
    tc.pages = pages;
    BlockCursor cur;
    cursor_level<RULE>(cur, 0, tc);
    cursor_settle<RULE>(cur, tc);
    {
        BlockRegs R;
        load_block(R, kp, vp, cur.plist, cur.key0, cur.count, g, Hkv);
        store_block(k_lds[0], v_lds[0], R);
    }
    __syncthreads();
    for (int buf = 0;; buf ^= 1) {
        // prefetch the next block into registers while this one is computed
        BlockCursor nxt = cur;
        const bool more = cursor_next<RULE>(nxt, tc);
        BlockRegs R;
        if (more) load_block(R, kp, vp, nxt.plist, nxt.key0, nxt.count, g, Hkv);
        if (active) {   // wave-uniform
            const int key0 = cur.key0, count = cur.count, pdiff = cur.pdiff;
            const bool own = cur.own;
            const uint16_t *kl = k_lds[buf], *vl = v_lds[buf];
            // S^T = K . Q^T
            f32x16 sacc[MT];
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) sacc[mt] = f32x16{};
            {
                const uint16_t *krow = kl + prow * K_STRIDE + half * 8;
    #pragma unroll
                for (int ks = 0; ks < D / 16; ++ks)
    #pragma unroll
                    for (int mt = 0; mt < MT; ++mt) {
                        const bf16x8 kf = as_bf16x8(*reinterpret_cast<const uint4 *>(krow + mt * 32 * K_STRIDE + ks * 16));
                        sacc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[ks], sacc[mt], 0, 0, 0);
                    }
                // keep LOOKAHEAD operand reads in flight ahead of the MFMAs
                __builtin_amdgcn_sched_group_barrier(0x100, LOOKAHEAD, 0);
    #pragma unroll
                for (int j = 0; j < 8 * MT - LOOKAHEAD; ++j) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                }
                __builtin_amdgcn_sched_group_barrier(0x008, LOOKAHEAD, 0);
            }
            // mask: register r of tile mt holds key 32*mt + 16*(r/8) + 8*half + r%8
            // of the block.  Only blocks that cross the diagonal, the end of a
            // visible range or the window's edge are masked, in place.  hi / lo:
            // last / first visible key offset within the block, minus 8 * half.
            const bool causal_own = own && RULE != TWO_WAY;
            const int hi = (causal_own ? tok - key0 : count - 1 - key0) - half * 8;
            const int lo = (RULE == WINDOW ? pdiff + tok - window + 1 - key0 : 0) - half * 8;
            const bool full = (causal_own ? (key0 + BN - 1 <= row0) : (key0 + BN <= count)) &&
                              (RULE != WINDOW || key0 >= pdiff + row0 + FK_TILE_TOKENS - window);
            if (!full) {
    #pragma unroll
                for (int mt = 0; mt < MT; ++mt)
    #pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int koff = mt * 32 + (r / 8) * 16 + (r % 8);
                        bool vis = koff <= hi;
                        if (RULE == WINDOW) vis = vis && koff >= lo;
                        sacc[mt][r] = vis ? sacc[mt][r] : -INFINITY;
                    }
            }
            // row max on raw scores (scale > 0); the two wave halves hold disjoint
            // keys of the same row and swap maxima with one permlane
            float mloc = sacc[0][0];
    #pragma unroll
            for (int mt = 0; mt < MT; ++mt)
    #pragma unroll
                for (int r = (mt == 0 ? 1 : 0); r < 16; ++r) mloc = __builtin_fmaxf(mloc, sacc[mt][r]);
            const float mrow = pair_max(mloc) * scale_log2e;
            // lazy rescale: a row moves its reference max only when the block's
            // max exceeds it by more than RESCALE_LOG2 (the exponents then stay
            // <= 2^RESCALE_LOG2); rows that do not move multiply by exactly 1
            const bool need = mrow > m + RESCALE_LOG2;
            if (__any(need)) {   // wave-uniform branch
                const float mnew = need ? mrow : m;
                const float corr = __builtin_amdgcn_exp2f(m - mnew);
                l *= corr;
    #pragma unroll
                for (int i = 0; i < D / 32; ++i) o[i] *= corr;
                m = mnew;
            }
            float ps[4] = {0.f, 0.f, 0.f, 0.f};
            bf16x8 pf[2 * MT];
    #pragma unroll
            for (int mt = 0; mt < MT; ++mt)
    #pragma unroll
                for (int hh = 0; hh < 2; ++hh) {
                    float pv[8];
    #pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        pv[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[mt][hh * 8 + e], scale_log2e, -m));
                        ps[e & 3] += pv[e];
                    }
                    pf[mt * 2 + hh] = as_bf16x8(pack8(pv));
                }
            l += (ps[0] + ps[1]) + (ps[2] + ps[3]);
            // O^T += V^T . P^T ; k-step kk covers keys 16*kk + [0, 16)
            {
                const uint16_t *vrow = vl + n * V_STRIDE + half * 8;
    #pragma unroll
                for (int kk = 0; kk < 2 * MT; ++kk)
    #pragma unroll
                    for (int i = 0; i < D / 32; ++i) {
                        const bf16x8 vf = as_bf16x8(*reinterpret_cast<const uint4 *>(vrow + i * 32 * V_STRIDE + kk * 16));
                        o[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[kk], o[i], 0, 0, 0);
                    }
            }
        }
        if (!more) break;
        store_block(k_lds[buf ^ 1], v_lds[buf ^ 1], R);
        cur = nxt;
        __syncthreads();   // next block staged; this buffer free for reuse
    }
    // epilogue: the row's sum is split over the two halves of the wave
    const float lsum = pair_sum(l);
    if (!row_valid) return;
    const float inv = 1.f / lsum;
    uint16_t *orow = out + qrow * D;
#pragma unroll
    for (int i = 0; i < D / 32; ++i)
#pragma unroll
        for (int rq = 0; rq < 4; ++rq) {
            // registers 4*rq .. 4*rq+3 hold dims 32*i + 8*rq + 4*half + [0, 4)
            uint2 packed;
            __bf16 b4[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) b4[e] = (__bf16)(o[i][rq * 4 + e] * inv);
            packed.x = (uint32_t)__builtin_bit_cast(uint16_t, b4[0]) | ((uint32_t)__builtin_bit_cast(uint16_t, b4[1]) << 16);
            packed.y = (uint32_t)__builtin_bit_cast(uint16_t, b4[2]) | ((uint32_t)__builtin_bit_cast(uint16_t, b4[3]) << 16);
            *reinterpret_cast<uint2 *>(orow + i * 32 + rq * 8 + half * 4) = packed;
        }
}

}  // namespace attn
}  // namespace fk

using namespace fk;

template <int RULE, bool READOUT>
static void launch_rule(const fk_tree_meta *meta, const WsLayout &L, const void *q, int Hq, int Hkv, float scale,
                        int window, const int32_t *rows, int n_rows, const void *k_pool, const void *v_pool,
                        void *out, const void *ws, hipStream_t st)
{
    dim3 grid((unsigned)((READOUT ? (int64_t)n_rows : L.tile_cap) * Hkv));
    attn::k_attn_bf16<RULE, READOUT><<<grid, attn::THREADS, 0, st>>>(
        (const uint16_t *)q, Hq, Hkv, scale * 1.4426950408889634f, window, rows, meta->tok_seg, meta->T,
        ws_at<int32_t>(ws, L.seg_pos0),
        (const uint16_t *)k_pool,
        (const uint16_t *)v_pool, (uint16_t *)out, ws_at<int32_t>(ws, L.header), ws_at<int32_t>(ws, L.tile_seg),
        ws_at<int32_t>(ws, L.tile_row0), ws_at<int32_t>(ws, L.tile_order), ws_at<int32_t>(ws, L.seg_start),
        ws_at<int32_t>(ws, L.seg_len),
        ws_at<int32_t>(ws, L.seg_depth), ws_at<int32_t>(ws, L.seg_anc), meta->seg_fork, meta->seg_page_off,
        meta->seg_pages);
}

// rows == NULL: the full launch over the round's tiles; otherwise readout of
// the n_rows entries of `rows` (q and out then hold one row per entry)
int fk_launch_attn_bf16(const fk_tree_meta *meta, const void *q, int Hq, int Hkv, float scale, int rule, int window,
                        const int32_t *rows, int n_rows, const void *k_pool, const void *v_pool, void *out,
                        const void *ws, hipStream_t st)
{
    const WsLayout L = ws_layout(*meta, 0, 0, 0);
#define FK_ATTN_LAUNCH(R)                                                                                   \
    do {                                                                                                   \
        if (rows)                                                                                          \
            launch_rule<R, true>(meta, L, q, Hq, Hkv, scale, window, rows, n_rows, k_pool, v_pool, out, ws, st); \
        else                                                                                               \
            launch_rule<R, false>(meta, L, q, Hq, Hkv, scale, window, rows, n_rows, k_pool, v_pool, out, ws, st); \
    } while (0)
    if (rule == FK_RULE_WINDOW)
        FK_ATTN_LAUNCH(attn::WINDOW);
    else if (rule == FK_RULE_TWO_WAY)
        FK_ATTN_LAUNCH(attn::TWO_WAY);
    else
        FK_ATTN_LAUNCH(attn::CAUSAL);
#undef FK_ATTN_LAUNCH
    return launch_status();
}
