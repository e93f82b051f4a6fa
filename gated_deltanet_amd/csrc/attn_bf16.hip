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
// Blocks are staged in a ring of three 16 KB LDS stages by direct global->LDS
// loads two blocks ahead (48 KB), and the kernels take at most 158 VGPRs, so
// three work-groups (12 waves) share a compute unit.
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

#include <atomic>
#include <type_traits>

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

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 u) { return __builtin_bit_cast(bf16x8, u); }

// Read-only metadata read through the constant address space: with a uniform
// index it stays a scalar load even where the compiler cannot prove that no
// store in the loop aliases it (the block loads below are opaque to it), so
// it never waits on the vector-memory counter the block loads use.
__device__ __forceinline__ int ldc(const int32_t *p, int i)
{
    return ((const __attribute__((address_space(4))) int32_t *)p)[i];
}

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
    const int a = ldc(t.anc, lvl);
    c.count = c.own ? (RULE == TWO_WAY ? t.len : min(t.row0 + FK_TILE_TOKENS, t.len)) : ldc(t.seg_fork, ldc(t.anc, lvl + 1));
    c.plist = t.pages + ldc(t.page_off, a);
    c.pdiff = t.pos0 - ldc(t.seg_pos0, a);
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

// Epilogue through LDS: the row's sum is split over the two halves of the
// wave; every row's O / l is written as bf16 into this wave's 8 KB quarter of
// the ring (idle once every wave has passed the barrier below), row-major with
// the 16-byte units XORed by the row (registers 4*rq .. 4*rq+3 of tile i hold
// dims 32*i + 8*rq + 4*half + [0, 4)), then read back and stored by whole
// rows: instruction j stores rows 4j .. 4j+3 of the wave (heads 4(j%2) .. +3
// of its token j/2: 1 KB, eight full lines), for a token whose rows are valid.
// Row r of the wave (token r/8, head r%8) goes to orow0 + (r/8) tstride +
// (r%8) D.
__device__ __forceinline__ void store_rows(const f32x16 (&o)[D / 32], float l, bool row_valid, uint16_t *stage,
                                           uint16_t *orow0, size_t tstride, int n, int half, int lane)
{
    const float inv = 1.f / pair_sum(l);
    // tokens 0-3 of the wave: lanes 0, 8, 16, 24 (a token's rows are all valid or not)
    const uint64_t tok_valid = __ballot(row_valid);
    __syncthreads();   // every wave is done with the ring
#pragma unroll
    for (int i = 0; i < D / 32; ++i)
#pragma unroll
        for (int rq = 0; rq < 4; ++rq) {
            uint2 packed;
            __bf16 b4[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) b4[e] = (__bf16)(o[i][rq * 4 + e] * inv);
            packed.x = (uint32_t)__builtin_bit_cast(uint16_t, b4[0]) | ((uint32_t)__builtin_bit_cast(uint16_t, b4[1]) << 16);
            packed.y = (uint32_t)__builtin_bit_cast(uint16_t, b4[2]) | ((uint32_t)__builtin_bit_cast(uint16_t, b4[3]) << 16);
            *reinterpret_cast<uint2 *>(stage + n * D + (((4 * i + rq) ^ (n & 15)) * 8) + half * 4) = packed;
        }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int r = 4 * j + (lane >> 4), up = lane & 15;
        const uint4 v = *reinterpret_cast<const uint4 *>(stage + r * D + up * 8);
        if ((tok_valid >> ((j >> 1) * 8)) & 1)
            *reinterpret_cast<uint4 *>(orow0 + (size_t)(j >> 1) * tstride + (r & 7) * D + ((up ^ (r & 15)) * 8)) = v;
    }
}

// One key block for one wave's 32 rows: S^T = K . Q^T on MFMA, masking (only
// when the block is not `full` for every row of the wave: hi / lo = last /
// first visible key offset of the lane's row within the block, minus
// 8 * half), online softmax with the per-row lazy rescale, O^T += V^T . P^T.
// Where a lane's operands sit in a staged block (bf16 elements): K fragment
// (key tile mt, k-step ks) at krow + mt * KMT + (ks ^ kd) * KS, value
// fragment (dim tile i, key step kk) at vrow + i * VI + kk * VKK (the ring
// layout below; kd is the lane's swizzle of the k-step).

// `mid` runs once the score products are issued (the full launch issues a
// later block's loads there, while the matrix cores work on this one).
struct NoMid {
    __device__ void operator()() const {}
};

template <int RULE, class LAY, class MID = NoMid>
__device__ __forceinline__ void block_compute(const uint16_t *krow, const uint16_t *vrow, const bf16x8 (&qf)[D / 16],
                                              f32x16 (&o)[D / 32], float &m, float &l, bool full, int hi, int lo,
                                              int kd, float scale_log2e, const MID &mid = MID())
{
    // S^T = K . Q^T
    f32x16 sacc[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) sacc[mt] = f32x16{};
    {
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                const bf16x8 kf = as_bf16x8(*reinterpret_cast<const uint4 *>(krow + mt * LAY::KMT + (ks ^ kd) * LAY::KS));
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
    mid();
    // mask: register r of tile mt holds key 32*mt + 16*(r/8) + 8*half + r%8
    // of the block; masked in place unless the block is `full`
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
    // exponentials against the row's current reference max m
    float ps[4];
    bf16x8 pf[2 * MT];
    auto exponentials = [&]() {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                float pv[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    pv[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[mt][hh * 8 + e], scale_log2e, -m));
                    // the first four start the partial sums (exactly 0 + p)
                    ps[e & 3] = (mt == 0 && hh == 0 && e < 4) ? pv[e] : ps[e & 3] + pv[e];
                }
                pf[mt * 2 + hh] = as_bf16x8(pack8(pv));
            }
    };
    exponentials();
    float lblk = (ps[0] + ps[1]) + (ps[2] + ps[3]);
    // lazy rescale: a row moves its reference max only when the block's max
    // exceeds it by more than 2^RESCALE_LOG2 (the exponentials then stay
    // <= 2^RESCALE_LOG2); rows that do not move multiply by exactly 1.  Such
    // a row has an exponential above 2^(RESCALE_LOG2 - 1) in one half of the
    // wave, so that lane's partial sum exceeds it too: only then is the
    // block's row max taken, and the decision is the same as if it were
    // always taken (a block that passes this test moves no row).
    if (__any(!(lblk <= __builtin_exp2f(RESCALE_LOG2 - 1.f)))) {   // wave-uniform branch
        // row max on raw scores (scale > 0); the two wave halves hold
        // disjoint keys of the same row and swap maxima with one permlane
        float mloc = sacc[0][0];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int r = (mt == 0 ? 1 : 0); r < 16; ++r) mloc = __builtin_fmaxf(mloc, sacc[mt][r]);
        const float mrow = pair_max(mloc) * scale_log2e;
        const bool need = mrow > m + RESCALE_LOG2;
        if (__any(need)) {   // wave-uniform branch
            const float mnew = need ? mrow : m;
            const float corr = __builtin_amdgcn_exp2f(m - mnew);
            l *= corr;
#pragma unroll
            for (int i = 0; i < D / 32; ++i) o[i] *= corr;
            m = mnew;
            exponentials();
            lblk = (ps[0] + ps[1]) + (ps[2] + ps[3]);
        }
    }
    l += lblk;
    // O^T += V^T . P^T ; k-step kk covers keys 16*kk + [0, 16)
    {
#pragma unroll
        for (int kk = 0; kk < 2 * MT; ++kk)
#pragma unroll
            for (int i = 0; i < D / 32; ++i) {
                const bf16x8 vf = as_bf16x8(*reinterpret_cast<const uint4 *>(vrow + i * LAY::VI + kk * LAY::VKK));
                o[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[kk], o[i], 0, 0, 0);
            }
    }
}

// The full launch stages blocks in a ring of three LDS stages filled by
// direct global->LDS loads (global_load_lds_dwordx4: each lane's 16 bytes land
// at M0 + 16 * lane), two blocks ahead of the one computed, so no register
// holds a block in flight.  Stage layout (bf16 elements): K of the block's two
// pages row by row, [page][slot 16][unit 16][8], the 16-byte unit u of a key
// row at position u ^ slot; V^T at 4096 + [page][dim tile 4][half 2][dim 32]
// [8].  A 16-lane read group then meets 16 distinct 16-byte bank groups
// (keys: 16 slots, so 16 distinct positions of one unit; values: 16 dims).
// A value read is its lane's base plus an immediate offset; a key read adds
// (ks ^ kd) * 32 bytes, kd = slot / 2, since unit 2 ks + half of slot s sits at
// 2 (ks ^ (s / 2)) + (half ^ (s % 2)).  Each wave loads four whole key rows and
// 32 whole value rows of a page (1 KB, eight 128-byte lines an instruction);
// the lane that fills 16-byte unit c of a page region loads the unit of the
// page that belongs there (ring_k_off, ring_v_off).
struct RingTiles {
    static constexpr int KS = 16, KMT = 0, VI = 512, VKK = 2048;
};
constexpr int RING = 3;                 // stages
constexpr int STAGE = 2 * BN * D;       // bf16 elements per stage: K and V^T of one block
static_assert(MT == 1 && BN == 2 * FK_TILE_TOKENS, "the ring layout holds two 16-key pages per block");

// byte offsets inside a 4 KB K / V page of the 16 bytes lane `lane` of wave
// `w` loads (see the stage layout above)
__device__ __forceinline__ uint32_t ring_k_off(int w, int lane)
{
    const int row = 4 * w + (lane >> 4);
    return row * 256 + (((lane & 15) ^ (row & 15)) * 16);
}
__device__ __forceinline__ uint32_t ring_v_off(int w, int lane) { return (32 * w + (lane & 31)) * 32 + (lane >> 5) * 16; }

__device__ __forceinline__ const uint16_t *uniform_ptr(const uint16_t *p)
{
    const uint64_t u = (uint64_t)p;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)u), hi = __builtin_amdgcn_readfirstlane((uint32_t)(u >> 32));
    return (const uint16_t *)(((uint64_t)hi << 32) | lo);
}

// one 16-byte direct global->LDS load per lane: global address gbase + voff,
// LDS address m0 + 16 * lane
__device__ __forceinline__ void lds_dma16(const uint16_t *gbase, uint32_t voff, uint32_t m0)
{
    asm volatile("global_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(gbase), "{m0}"(m0) : "memory");
}

// The two page ids of a block.  Pages past the range's last key repeat its
// last page: those keys are masked, so their scores are -inf and their
// weights exactly 0, and the repeated values are finite.
struct BlockPages {
    int p0, p1;
};
__device__ __forceinline__ BlockPages ring_pages(const int32_t *__restrict__ plist, int key0, int count)
{
    // count >= 1 and key0 >= 0: shifts, not signed divisions
    const int last = (int)((uint32_t)(count - 1) >> 4), pi = (int)((uint32_t)key0 >> 4);
    static_assert(FK_TILE_TOKENS == 16, "page index by shift");
    return BlockPages{ldc(plist, min(pi, last)), ldc(plist, min(pi + 1, last))};
}

// Issue the four loads (K and V of the two pages) of one block into a stage;
// every wave issues exactly four loads per block.  kg / vg: the pools at this
// kv head's first page (page p at + p * pstride elements); m0: the stage's
// LDS byte address plus this wave's 1 KB quarter (all wave-uniform).
__device__ __forceinline__ void ring_issue(uint32_t m0, const uint16_t *kg, const uint16_t *vg, BlockPages pg,
                                           uint32_t pstride, uint32_t koff, uint32_t voff)
{
#pragma unroll
    for (int p = 0; p < BN / FK_TILE_TOKENS; ++p) {
        const size_t pb = (size_t)(uint32_t)(p ? pg.p1 : pg.p0) * pstride;
        lds_dma16(kg + pb, koff, m0 + p * 4096);
        lds_dma16(vg + pb, voff, m0 + 8192 + p * 4096);
    }
}

// wait until at most N of this wave's loads are in flight, then meet the
// work-group at a barrier (the loads are in-order, so the older block's
// loads have landed in LDS)
template <int N>
__device__ __forceinline__ void ring_wait_barrier()
{
    asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(N) : "memory");
}

template <int RULE>
__global__ void __launch_bounds__(THREADS, 3)
k_attn_bf16(const uint16_t *__restrict__ q, int Hq, int Hkv, float scale_log2e, int window,
            const int32_t *__restrict__ seg_pos0, const uint16_t *__restrict__ kp,
            const uint16_t *__restrict__ vp, uint16_t *__restrict__ out, const int32_t *__restrict__ header,
            const int32_t *__restrict__ tile_seg, const int32_t *__restrict__ tile_row0,
            const int32_t *__restrict__ tile_order, const int32_t *__restrict__ seg_start,
            const int32_t *__restrict__ seg_len, const int32_t *__restrict__ seg_depth,
            const int32_t *__restrict__ seg_anc, const int32_t *__restrict__ seg_fork,
            const int32_t *__restrict__ page_off, const int32_t *__restrict__ pages)
{
    __shared__ __attribute__((aligned(1024))) uint16_t ring[RING * STAGE];
    if (header[H_STATUS] != FK_OK) return;
    // tiles in the builder's order -- heaviest first by band of work, a
    // request's tiles together within a band -- the kv heads of a tile side
    // by side (so with work-groups dealt to the XCDs in turn, an XCD sees one
    // kv head's tiles of a few requests at a time)
    const int rank = blockIdx.x / Hkv, g = blockIdx.x % Hkv;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int half = lane >> 5, n = lane & 31;
    if (rank >= header[H_NTILES]) return;
    const int tile = tile_order[rank];
    const int s = tile_seg[tile], row0 = tile_row0[tile];
    const int len = seg_len[s];
    const int tok = row0 + w * 4 + n / 8;          // local token of this lane's row
    const int h = g * G + (n % 8);
    const bool row_valid = tok < len;
    const bool wave_live = __builtin_amdgcn_readfirstlane(row0 + w * 4 < len);   // wave-uniform
    const size_t t_glob = (size_t)seg_start[s] + tok;
    const size_t qrow = t_glob * Hq + h;

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
    const uint32_t koff = ring_k_off(w, lane), voff = ring_v_off(w, lane);
    // this wave's quarter of stage 0 (LDS bytes), and the pools at head g
    const uint32_t ring_bytes =
        __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint16_t *)ring + w * 1024);
    const uint16_t *kg = uniform_ptr(kp + (size_t)g * (FK_TILE_TOKENS * D));
    const uint16_t *vg = uniform_ptr(vp + (size_t)g * (FK_TILE_TOKENS * D));
    const uint32_t pstride = (uint32_t)Hkv * (FK_TILE_TOKENS * D);
    const uint16_t *krow0 = ring + (n >> 4) * 2048 + (prow & 15) * 128 + (half ^ (prow & 1)) * 8;
    const int kd = (prow & 15) >> 1;
    const uint16_t *vrow0 = ring + 4096 + half * 256 + n * 8;

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
    // blocks j and j+1 in flight before the walk starts, block j+2's page ids
    // known: each iteration issues block j+2's loads right after its barrier
    // and, after computing block j, finds block j+3 and reads its page ids --
    // scalar loads that land while the wave waits at the next barrier, not
    // while LDS operand reads (which share their wait counter) are in flight
    ring_issue(ring_bytes, kg, vg, ring_pages(cur.plist, cur.key0, cur.count), pstride, koff, voff);
    BlockCursor nxt = cur;
    bool more = cursor_next<RULE>(nxt, tc);
    if (more) ring_issue(ring_bytes + STAGE * 2, kg, vg, ring_pages(nxt.plist, nxt.key0, nxt.count), pstride, koff, voff);
    BlockCursor nxt2 = nxt;
    bool more2 = more && cursor_next<RULE>(nxt2, tc);
    BlockPages pg2 = more2 ? ring_pages(nxt2.plist, nxt2.key0, nxt2.count) : BlockPages{0, 0};
    // the query loads (and the first two blocks) complete here, so the
    // compiler's own wait for them is not repeated inside the walk, where a
    // full wait would also drain the block loads in flight
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
    // one block in stage ST; returns false after the last block.  The walk is
    // unrolled over the three stages so that every LDS offset is an immediate.
    auto step = [&](auto STC) {
        constexpr int ST = decltype(STC)::value, ST2 = (ST + 2) % RING;
        // block j landed in every wave, and every wave is done with block j-1,
        // whose stage block j+2 now takes
        if (more)
            ring_wait_barrier<4>();
        else
            ring_wait_barrier<0>();
        // block j+2's loads are issued once this block's score products are
        // (their issue can stall on the memory pipeline while those run)
        auto issue_next = [&]() {
            if (more2) ring_issue(ring_bytes + ST2 * (STAGE * 2), kg, vg, pg2, pstride, koff, voff);
        };
        {
            const int key0 = cur.key0, count = cur.count, pdiff = cur.pdiff;
            const bool own = cur.own;
            // Only blocks that cross the diagonal, the end of a visible range or
            // the window's edge are masked.
            const bool causal_own = own && RULE != TWO_WAY;
            const int hi = (causal_own ? tok - key0 : count - 1 - key0) - half * 8;
            const int lo = (RULE == WINDOW ? pdiff + tok - window + 1 - key0 : 0) - half * 8;
            const bool full = (causal_own ? (key0 + BN - 1 <= row0) : (key0 + BN <= count)) &&
                              (RULE != WINDOW || key0 >= pdiff + row0 + FK_TILE_TOKENS - window);
            // a wave whose four tokens all lie past the segment's end (in the
            // segment's last tile) only helps stage the blocks
            if (wave_live)
                block_compute<RULE, RingTiles>(krow0 + ST * STAGE, vrow0 + ST * STAGE, qf, o, m, l, full, hi, lo,
                                               kd, scale_log2e, issue_next);
            else
                issue_next();
        }
        if (!more) return false;
        BlockCursor nxt3 = nxt2;
        const bool more3 = more2 && cursor_next<RULE>(nxt3, tc);
        if (more3) pg2 = ring_pages(nxt3.plist, nxt3.key0, nxt3.count);
        cur = nxt;
        nxt = nxt2;
        nxt2 = nxt3;
        more = more2;
        more2 = more3;
        return true;
    };
    static_assert(RING == 3, "the walk is unrolled over three stages");
    while (step(std::integral_constant<int, 0>()) && step(std::integral_constant<int, 1>()) &&
           step(std::integral_constant<int, 2>())) {
    }
    store_rows(o, l, row_valid, ring + w * (32 * D), out + ((size_t)seg_start[s] + row0 + 4 * w) * Hq * D + (size_t)g * G * D,
               (size_t)Hq * D, n, half, lane);
}

// Selective readout (Flide section 3.3.3): work item = (group of up to 16
// entries of the row buffer, part, kv head), a part being the group's leading
// entries of one request or the rest (below).  The group's entries take the 16 token
// slots of a tile (wave w: slots 4w .. 4w+3, 8 q heads each), and the key walk
// covers the union of their chains: depth by depth, every distinct segment
// met at that depth, up to the largest count any entry sees of it.  A row
// masks what its own chain does not show -- blocks off its chain or past its
// limit contribute exactly nothing (no key, no max change, zero weights), so
// each row meets its own chain's blocks in chain order, anchored as in the
// full launch, and its output has the same bits as that token's row of the
// full launch, whatever its group.  Grouping only fills the tile's rows: one
// pass over a shared trunk serves up to 16 questions.  Blocks are staged in
// the full launch's ring, so operands and arithmetic are the same.
constexpr int RO_CAND = FK_TILE_TOKENS * FK_MAX_DEPTH;   // (slot, depth) candidates

template <int RULE>
__global__ void __launch_bounds__(THREADS, 3)
k_attn_readout_bf16(const uint16_t *__restrict__ q_rows, const int32_t *__restrict__ sel_rows, int n_rows,
                    int group, int Hq, int Hkv, float scale_log2e, int window, const int32_t *__restrict__ tok_seg,
                    int T, const int32_t *__restrict__ seg_pos0, const uint16_t *__restrict__ kp,
                    const uint16_t *__restrict__ vp, uint16_t *__restrict__ out_rows,
                    const int32_t *__restrict__ header, const int32_t *__restrict__ seg_start,
                    const int32_t *__restrict__ seg_len, const int32_t *__restrict__ seg_depth,
                    const int32_t *__restrict__ seg_anc, const int32_t *__restrict__ seg_fork,
                    const int32_t *__restrict__ page_off, const int32_t *__restrict__ pages)
{
    __shared__ __attribute__((aligned(1024))) uint16_t ring[RING * STAGE];
    __shared__ int c_seg[RO_CAND], c_lim[RO_CAND], c_lo[RO_CAND];   // per (slot, depth)
    // planning only: these three live in the ring, which no block occupies
    // before the walk (the barrier after the range table is built precedes
    // the first block load), so three work-groups still fit a CU's LDS
    int *const c_rep = reinterpret_cast<int *>(ring), *const c_cnt = c_rep + RO_CAND, *const c_key0 = c_cnt + RO_CAND;
    int *const c_root = c_key0 + RO_CAND;   // per slot
    __shared__ int r_seg[RO_CAND], r_depth[RO_CAND], r_count[RO_CAND], r_key0[RO_CAND];
    __shared__ int n_ranges;
    if (header[H_STATUS] != FK_OK) return;
    const int grp = blockIdx.x / Hkv / 2, part = blockIdx.x / Hkv % 2, g = blockIdx.x % Hkv;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int half = lane >> 5, n = lane & 31;

    // The group's entries split in two parts, each walked by its own work-group:
    // part 0 is the slots before the first used entry whose root segment differs
    // from that of the group's first used entry, part 1 the rest (usually none,
    // and that work-group ends here).  So a group that straddles two requests
    // does not walk both histories in one work-group.
    if (threadIdx.x < FK_TILE_TOKENS) {
        const int ce = grp * group + (int)threadIdx.x;
        const int ct = ((int)threadIdx.x < group && ce < n_rows) ? sel_rows[ce] : -1;
        const int cs = (ct >= 0 && ct < T) ? tok_seg[ct] : -1;
        c_root[threadIdx.x] = cs >= 0 ? seg_anc[(size_t)cs * FK_MAX_DEPTH] : -1;
    }
    __syncthreads();
    int split = group, root0 = -1;
    for (int i = 0; i < group; ++i) {
        const int r = c_root[i];
        if (r < 0) continue;
        if (root0 < 0) root0 = r;
        else if (r != root0) {
            split = i;
            break;
        }
    }
    if (part == 1 && split == group) return;   // the whole work-group
    auto in_part = [&](int sl) { return part == 0 ? sl < split : sl >= split; };

    // this lane's row: entry of slot w*4 + n/8, q head g*G + n%8
    const int slot = w * 4 + n / 8, e = grp * group + slot;
    const int t = (slot < group && e < n_rows && in_part(slot)) ? sel_rows[e] : -1;
    const bool row_valid = t >= 0 && t < T && tok_seg[t] >= 0;   // not unused, not padding
    const int h = g * G + (n % 8);
    const size_t qrow = (size_t)e * Hq + h;

    // candidate (slot ci / FK_MAX_DEPTH, depth ci % FK_MAX_DEPTH): the segment
    // that slot's entry meets at that depth, how many of its keys the entry
    // sees, and (window) the first one inside the entry's window
    if (threadIdx.x < RO_CAND) {
        const int ci = threadIdx.x, cslot = ci / FK_MAX_DEPTH, cd = ci % FK_MAX_DEPTH;
        const int ce = grp * group + cslot;
        int cseg = -1, clim = 0, clo = 0;
        const int ct = (cslot < group && ce < n_rows && in_part(cslot)) ? sel_rows[ce] : -1;
        const int cs = (ct >= 0 && ct < T) ? tok_seg[ct] : -1;
        if (cs >= 0) {
            const int cdep = seg_depth[cs];
            const int cloc = ct - seg_start[cs];
            if (cd <= cdep) {
                const int32_t *ca = seg_anc + (size_t)cs * FK_MAX_DEPTH;
                cseg = ca[cd];
                clim = cd == cdep ? (RULE == TWO_WAY ? seg_len[cs] : cloc + 1) : seg_fork[ca[cd + 1]];
                if (RULE == WINDOW) clo = max(0, seg_pos0[cs] + cloc - seg_pos0[cseg] - window + 1);
            }
        }
        c_seg[ci] = cseg;
        c_lim[ci] = clim;
        c_lo[ci] = clo;
    }
    __syncthreads();
    // a candidate is a range when no earlier slot meets its segment at that
    // depth; its count / start cover every slot that does
    int rep = 0, cnt = 0, key0c = 0;
    if (threadIdx.x < RO_CAND) {
        const int ci = threadIdx.x, cslot = ci / FK_MAX_DEPTH, cd = ci % FK_MAX_DEPTH;
        const int a = c_seg[ci];
        int lo = 0x7fffffff;
        rep = a >= 0;
        if (a >= 0)
            for (int o2 = 0; o2 < FK_TILE_TOKENS; ++o2) {
                const int oi = o2 * FK_MAX_DEPTH + cd;
                if (c_seg[oi] != a) continue;
                if (o2 < cslot) rep = 0;
                cnt = max(cnt, c_lim[oi]);
                lo = min(lo, c_lo[oi]);
            }
        key0c = RULE == WINDOW ? (lo / BN) * BN : 0;
        if (rep && key0c >= cnt) rep = 0;
    }
    if (threadIdx.x < RO_CAND) {
        c_rep[threadIdx.x] = rep;
        c_cnt[threadIdx.x] = cnt;
        c_key0[threadIdx.x] = key0c;
    }
    __syncthreads();
    // ranges in (depth, first slot) order
    if (threadIdx.x == 0) {
        int nr = 0;
        for (int cd = 0; cd < FK_MAX_DEPTH; ++cd)
            for (int cslot = 0; cslot < FK_TILE_TOKENS; ++cslot) {
                const int ci = cslot * FK_MAX_DEPTH + cd;
                if (!c_rep[ci]) continue;
                r_seg[nr] = c_seg[ci];
                r_depth[nr] = cd;
                r_count[nr] = c_cnt[ci];
                r_key0[nr] = c_key0[ci];
                ++nr;
            }
        n_ranges = nr;
    }
    __syncthreads();
    // walk values are the same in every lane: keep them scalar, so page ids
    // are read with scalar loads as in the full launch
    auto uni = [](int x) { return __builtin_amdgcn_readfirstlane(x); };
    const int nr = uni(n_ranges);
    if (nr == 0) return;   // no used entry in this group

    // wave-uniform (readfirstlane), so the walk branches on it with scalar branches
    const bool wave_has_rows = __builtin_amdgcn_readfirstlane(__any(row_valid));
    bf16x8 qf[D / 16];
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
        uint4 u = make_uint4(0, 0, 0, 0);
        if (row_valid) u = *reinterpret_cast<const uint4 *>(q_rows + qrow * D + ks * 16 + half * 8);
        qf[ks] = as_bf16x8(u);
    }

    f32x16 o[D / 32];
#pragma unroll
    for (int i = 0; i < D / 32; ++i) o[i] = f32x16{};
    float m = -1e30f, l = 0.f;
    const int prow = (n & ~12) | ((n & 4) << 1) | ((n & 8) >> 1);

    // the lane's visible keys [lo_r, lim_r) of range ri (none off its chain),
    // from the planning tables in LDS (no global load in the walk)
    int lim_r = 0, lo_r = 0, lane_ri = 0;
    auto lane_range = [&](int ri) {
        const int a = uni(r_seg[ri]), dd = uni(r_depth[ri]);
        const int ci = slot * FK_MAX_DEPTH + dd;
        const bool on = row_valid && c_seg[ci] == a;
        lim_r = on ? c_lim[ci] : 0;
        lo_r = (RULE == WINDOW && on) ? c_lo[ci] : 0;
        lane_ri = ri;
    };
    // Blocks are staged as in the full launch (three-stage ring, direct
    // loads two blocks ahead, every wave four loads per block), so each row's
    // operands and arithmetic are the full launch's.  Walk position: range
    // ri, block key0 (ranges are never empty).
    struct RCursor {
        int ri, key0, count;
        const int32_t *plist;
    };
    auto r_range = [&](RCursor &c, int ri) {
        c.ri = ri;
        c.key0 = uni(r_key0[ri]);
        c.count = uni(r_count[ri]);
        c.plist = pages + ldc(page_off, uni(r_seg[ri]));
    };
    auto r_next = [&](RCursor &c) {
        c.key0 += BN;
        if (c.key0 < c.count) return true;
        if (c.ri + 1 >= nr) return false;
        r_range(c, c.ri + 1);
        return true;
    };
    const uint32_t koff = ring_k_off(w, lane), voff = ring_v_off(w, lane);
    const uint32_t ring_bytes =
        __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint16_t *)ring + w * 1024);
    const uint16_t *kg = uniform_ptr(kp + (size_t)g * (FK_TILE_TOKENS * D));
    const uint16_t *vg = uniform_ptr(vp + (size_t)g * (FK_TILE_TOKENS * D));
    const uint32_t pstride = (uint32_t)Hkv * (FK_TILE_TOKENS * D);
    const uint16_t *krow0 = ring + (n >> 4) * 2048 + (prow & 15) * 128 + (half ^ (prow & 1)) * 8;
    const int kd = (prow & 15) >> 1;
    const uint16_t *vrow0 = ring + 4096 + half * 256 + n * 8;

    RCursor cur;
    r_range(cur, 0);
    lane_range(0);
    ring_issue(ring_bytes, kg, vg, ring_pages(cur.plist, cur.key0, cur.count), pstride, koff, voff);
    RCursor nxt = cur;
    bool more = r_next(nxt);
    if (more) ring_issue(ring_bytes + STAGE * 2, kg, vg, ring_pages(nxt.plist, nxt.key0, nxt.count), pstride, koff, voff);
    RCursor nxt2 = nxt;
    bool more2 = more && r_next(nxt2);
    BlockPages pg2 = more2 ? ring_pages(nxt2.plist, nxt2.key0, nxt2.count) : BlockPages{0, 0};
    // the query loads (and the first two blocks) complete here, so the
    // compiler's own wait for them is not repeated inside the walk
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
    // one block in stage ST; returns false after the last block (the walk is
    // unrolled over the three stages, as in the full launch)
    auto step = [&](auto STC) {
        constexpr int ST = decltype(STC)::value, ST2 = (ST + 2) % RING;
        // block j landed in every wave, and every wave is done with block j-1,
        // whose stage block j+2 now takes
        if (more)
            ring_wait_barrier<4>();
        else
            ring_wait_barrier<0>();
        const uint32_t st2_bytes = ring_bytes + ST2 * (STAGE * 2);
        if (cur.ri != lane_ri) lane_range(cur.ri);
        if (wave_has_rows) {   // wave-uniform
            const int key0 = cur.key0;
            const bool lane_full = !row_valid || (key0 + BN <= lim_r && (RULE != WINDOW || key0 >= lo_r));
            const bool full = __all(lane_full);
            const int hi = lim_r - 1 - key0 - half * 8;
            const int lo = (RULE == WINDOW ? lo_r - key0 : 0) - half * 8;
            // block j+2's loads go out once this block's score products are
            block_compute<RULE, RingTiles>(krow0 + ST * STAGE, vrow0 + ST * STAGE, qf, o, m, l, full, hi, lo,
                                           kd, scale_log2e, [&]() {
                                               if (more2) ring_issue(st2_bytes, kg, vg, pg2, pstride, koff, voff);
                                           });
        } else if (more2) {
            ring_issue(st2_bytes, kg, vg, pg2, pstride, koff, voff);
        }
        if (!more) return false;
        RCursor nxt3 = nxt2;
        const bool more3 = more2 && r_next(nxt3);
        if (more3) pg2 = ring_pages(nxt3.plist, nxt3.key0, nxt3.count);
        cur = nxt;
        nxt = nxt2;
        nxt2 = nxt3;
        more = more2;
        more2 = more3;
        return true;
    };
    while (step(std::integral_constant<int, 0>()) && step(std::integral_constant<int, 1>()) &&
           step(std::integral_constant<int, 2>())) {
    }
    store_rows(o, l, row_valid, ring + w * (32 * D), out_rows + ((size_t)grp * group + 4 * w) * Hq * D + (size_t)g * G * D,
               (size_t)Hq * D, n, half, lane);
}

}  // namespace attn
}  // namespace fk

using namespace fk;

template <int RULE>
static void launch_rule(const fk_tree_meta *meta, const WsLayout &L, const void *q, int Hq, int Hkv, float scale,
                        int window, const int32_t *rows, int n_rows, int group, const void *k_pool,
                        const void *v_pool, void *out, const void *ws, hipStream_t st)
{
    const float sl = scale * 1.4426950408889634f;
    if (rows) {
        const int64_t groups = (n_rows + group - 1) / group;
        attn::k_attn_readout_bf16<RULE><<<dim3((unsigned)(groups * 2 * Hkv)), attn::THREADS, 0, st>>>(
            (const uint16_t *)q, rows, n_rows, group, Hq, Hkv, sl, window, meta->tok_seg, meta->T,
            ws_at<int32_t>(ws, L.seg_pos0), (const uint16_t *)k_pool, (const uint16_t *)v_pool, (uint16_t *)out,
            ws_at<int32_t>(ws, L.header), ws_at<int32_t>(ws, L.seg_start), ws_at<int32_t>(ws, L.seg_len),
            ws_at<int32_t>(ws, L.seg_depth), ws_at<int32_t>(ws, L.seg_anc), meta->seg_fork, meta->seg_page_off,
            meta->seg_pages);
        return;
    }
    attn::k_attn_bf16<RULE><<<dim3((unsigned)(L.tile_cap * Hkv)), attn::THREADS, 0, st>>>(
        (const uint16_t *)q, Hq, Hkv, sl, window, ws_at<int32_t>(ws, L.seg_pos0), (const uint16_t *)k_pool,
        (const uint16_t *)v_pool, (uint16_t *)out, ws_at<int32_t>(ws, L.header), ws_at<int32_t>(ws, L.tile_seg),
        ws_at<int32_t>(ws, L.tile_row0), ws_at<int32_t>(ws, L.tile_order), ws_at<int32_t>(ws, L.seg_start),
        ws_at<int32_t>(ws, L.seg_len), ws_at<int32_t>(ws, L.seg_depth), ws_at<int32_t>(ws, L.seg_anc),
        meta->seg_fork, meta->seg_page_off, meta->seg_pages);
}

// rows == NULL: the full launch over the round's tiles; otherwise readout of
// the n_rows entries of `rows` (q and out then hold one row per entry),
// grouped so that the launch fills about three work-groups per compute unit
// (two work-groups per group: one for each part of a group split at a request
// boundary; the second usually ends at once)
int fk_launch_attn_bf16(const fk_tree_meta *meta, const void *q, int Hq, int Hkv, float scale, int rule, int window,
                        const int32_t *rows, int n_rows, const void *k_pool, const void *v_pool, void *out,
                        const void *ws, hipStream_t st)
{
    const WsLayout L = ws_layout(*meta, 0, 0, 0);
    int group = 1;
    if (rows) {
        int dev = 0;
        FK_HIP(hipGetDevice(&dev));
        static std::atomic<int> n_cu_dev[64];   // per device, queried once
        if (dev < 0 || dev >= 64) return FK_E_HIP;
        int n_cu = n_cu_dev[dev].load(std::memory_order_relaxed);
        if (!n_cu) {
            FK_HIP(hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev));
            n_cu_dev[dev].store(n_cu, std::memory_order_relaxed);
        }
        const int64_t g = (int64_t)n_rows * Hkv / (3 * (int64_t)n_cu);
        group = (int)(g < 1 ? 1 : g > FK_TILE_TOKENS ? FK_TILE_TOKENS : g);
    }
    if (rule == FK_RULE_WINDOW)
        launch_rule<attn::WINDOW>(meta, L, q, Hq, Hkv, scale, window, rows, n_rows, group, k_pool, v_pool, out, ws, st);
    else if (rule == FK_RULE_TWO_WAY)
        launch_rule<attn::TWO_WAY>(meta, L, q, Hq, Hkv, scale, window, rows, n_rows, group, k_pool, v_pool, out, ws,
                                   st);
    else
        launch_rule<attn::CAUSAL>(meta, L, q, Hq, Hkv, scale, window, rows, n_rows, group, k_pool, v_pool, out, ws, st);
    return launch_status();
}
