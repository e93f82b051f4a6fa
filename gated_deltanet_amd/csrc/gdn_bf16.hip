// gdn_bf16.hip -- forked Gated DeltaNet, chunked form on bf16 MFMA (gfx950).
//
// Eq. 4 of Flide section 3.2.2, S_t = a_t S_{t-1} (I - b_t k_t k_t^T) +
// b_t v_t k_t^T and o_t = S_t q_t (S is dv x dk), rewritten exactly over a
// chunk of c <= 64 tokens.  With l_i = sum_{j<=i} ln a_j (log space), S0 the
// state entering the chunk and rows = tokens:
//   A_ij = b_i e^{l_i - l_j} (k_i . k_j) for j < i,   T = (I + A)^-1
//   U    = T diag(b) (V - diag(e^l) K S0^T)          (the corrected writes)
//   O    = diag(e^l) Q S0^T + (Gamma o Q K^T) U,  Gamma_ij = e^{l_i - l_j}, j <= i
//   S^T after r tokens = e^{l_{r-1}} S0^T + K_{<r}^T diag(e^{l_{r-1} - l_j}) U_{<r}
// (unrolling Eq. 4 inside the chunk: S_i = g_i S0 + sum_{j<=i} (g_i/g_j) u_j k_j^T
// with u_i = b_i (v_i - a_i S_{i-1} k_i); every ratio g_i/g_j <= 1 is taken as
// e^{l_i - l_j}).  Chunks are anchored at the start of every segment, so a
// trunk's arithmetic never depends on its branches (Flide section 3.5).
//
// k_gdn_prep  (all chunks of the round at once, before the level launches):
//             T of every (chunk, v-head) in fp32 by forward substitution,
//             stored as bf16, with P and the chunk's log-decay prefix l.  It
//             depends only on q, k, a, b -- never on a state.
// k_gdn_chunk (one launch per tree level, persistent work-groups): each
//             item (segment, v-head, 64-wide dv slice) walks its chunks in
//             order.  Each consumer wave keeps its 128 x 16 slice of S^T in fp32 MFMA
//             accumulator registers for the whole segment and feeds it
//             straight back as an MFMA operand (a fixed permutation of the
//             reduction index makes the accumulator layout the operand
//             layout), so the state never leaves registers between chunks.
//             It starts from the zero state, state_in, or the parent's
//             fork-point state (by index), and writes the states at the
//             segment's fork points once each.
#include <hip/hip_runtime.h>

#include <atomic>

#include "fk_common.h"

namespace fk {
namespace gdnk {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int C = FK_GDN_CHUNK;   // 64 tokens
constexpr int DK = 128, DV = 128;
constexpr int DVS = 64;           // dv columns of one work-group (4 waves x 16)
constexpr int KS = DK;            // LDS stride (bf16) of key/query rows (swizzled, unpadded)
constexpr int RS = C;             // LDS stride (bf16) of 64-wide rows (T, P, values / output), swizzled

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 u) { return __builtin_bit_cast(bf16x8, u); }

__device__ __forceinline__ f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 pack(f32x4 lo, f32x4 hi)
{
    bf16x8 v;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        v[e] = (__bf16)lo[e];
        v[e + 4] = (__bf16)hi[e];
    }
    return v;
}

// Operands with a permuted reduction index: for a k-step over 32 positions,
// lane group G = lane/16 supplies positions 4G..4G+3 and 16+4G..16+4G+3 --
// exactly the rows a 16x16 accumulator pair holds in that lane group.  Rows
// that serve as such operands are stored with each 32-position block
// reordered so that those eight positions are contiguous: the group of four
// positions q (0..7) of a block sits at element perm4(q) of the block.
// One 16-byte LDS read then gives a lane its operand.
__device__ __forceinline__ int perm4(int q) { return 8 * (q & 3) + 4 * (q >> 2); }

// element offset, within a row, of the group of four positions starting at p (p % 4 == 0)
__device__ __forceinline__ int perm_off(int p) { return (p & ~31) + perm4((p >> 2) & 7); }

// 64-wide rows in LDS (T, P, and the value / output slice): 128 B per row, no
// padding, the eight 16-byte units of row r XOR-swizzled by r mod 8.  Every
// access to them -- 16-byte operand reads of 16 rows, 16-byte row writes,
// transpose reads of 4 rows x 4 columns, 4-byte output writes -- is then free
// of LDS bank conflicts on gfx950 (measured, not only by bank arithmetic).
__device__ __forceinline__ int r64_off(int row, int e) { return row * RS + ((((e >> 3) ^ (row & 7)) << 3) | (e & 7)); }

__device__ __forceinline__ bf16x8 load_perm(const uint16_t *buf, int row, int ks, int G)
{
    return as_bf16x8(*reinterpret_cast<const uint4 *>(buf + r64_off(row, ks * 32 + 8 * G)));
}

// Key and query rows in LDS: 256 B per row, no padding; the sixteen 16-byte
// units of row r are XOR-swizzled by r's low nibble with its bits reordered
// (unit bits 0..3 take row bits 0, 3, 1, 2).  Of the orders that keep the
// operand read (16 rows, one unit each), the transpose read (4 rows x 4 units
// of one block) and the producers' 8-byte row writes free of bank conflicts,
// this is one that gfx950 also serves at full rate (measured).
__device__ __forceinline__ int kq_swz(int row)
{
    return (row & 1) | (((row >> 3) & 1) << 1) | (((row >> 1) & 1) << 2) | (((row >> 2) & 1) << 3);
}

// element offset of element `e` (a multiple of 4) of row `row`
__device__ __forceinline__ int kq_off(int row, int e) { return row * KS + ((((e >> 3) ^ kq_swz(row)) << 3) | (e & 7)); }

__device__ __forceinline__ bf16x8 load_kq(const uint16_t *buf, int row, int ks, int G)
{
    return as_bf16x8(*reinterpret_cast<const uint4 *>(buf + kq_off(row, ks * 32 + 8 * G)));
}

// raw buffer resource (gfx9 data format dword) over `bytes` bytes at `p`
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *p, size_t bytes)
{
    const int n = bytes > 0x7fffffffull ? 0x7fffffff : (int)bytes;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, n, 0x00020000);
}

__device__ __forceinline__ uint4 buf_load(__amdgpu_buffer_rsrc_t r, int byte_off)
{
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 0));
}

__device__ __forceinline__ bf16x8 load_row8(const uint16_t *row, int ks, int G)
{
    return as_bf16x8(*reinterpret_cast<const uint4 *>(row + ks * 32 + 8 * G));
}

// ---------------------------------------------------------------------------
// Per (chunk, v-head), everything that does not depend on a state:
//   T = (I + A)^-1 (fp32, by 16 x 16 blocks) and
//   P = Gamma o Q K^T (lower triangle incl. the diagonal), both stored bf16.
// Key and query rows are loaded straight into MFMA operand registers (the
// A and B operand layouts of a 16x16x32 product coincide); LDS holds the
// diagonal blocks and the finished T.  Four items per work-group, one wave
// each.  Query tiles are loaded one at a time, as P uses them, so a wave
// fits in 128 VGPRs and four work-groups share a CU.
// ---------------------------------------------------------------------------
constexpr int PREP_WAVES = 4;
constexpr int TBS = C + 8;        // LDS stride (bf16) of the finished T rows
constexpr int PREP_SCR = C * TBS * 2 > 4 * (16 * 16 + 16) * 4 ? C * TBS * 2 : 4 * (16 * 16 + 16) * 4;

__global__ void __launch_bounds__(64 * PREP_WAVES, 4)
k_gdn_prep(const uint16_t *__restrict__ q, const uint16_t *__restrict__ k, const float *__restrict__ a,
           const float *__restrict__ b, int Hk, int Hv, const int32_t *__restrict__ header,
           const int32_t *__restrict__ chunk_seg, const int32_t *__restrict__ chunk_row0,
           const int32_t *__restrict__ seg_start, const int32_t *__restrict__ seg_len,
           uint16_t *__restrict__ tmat, uint16_t *__restrict__ pmat, float *__restrict__ lvec)
{
    // per wave: the fp32 diagonal blocks of A (then of T), later the finished
    // T as bf16 rows -- the two uses never overlap in time
    __shared__ __attribute__((aligned(16))) char scr_all[PREP_WAVES][PREP_SCR];
    __shared__ float lsh_all[PREP_WAVES][C], esh_all[PREP_WAVES][C];
    if (header[H_STATUS] != FK_OK) return;
    const int nitems = header[H_NCHUNKS] * Hv;
    if ((int)blockIdx.x * PREP_WAVES >= nitems) return;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, G = lane >> 4, c16 = lane & 15;
    const int item = blockIdx.x * PREP_WAVES + w;
    const bool valid = item < nitems;   // every wave reaches every barrier
    const int c = valid ? item / Hv : 0, h = valid ? item % Hv : 0;
    float *am = reinterpret_cast<float *>(scr_all[w]), *lsh = lsh_all[w], *esh = esh_all[w];
    uint16_t *tb = reinterpret_cast<uint16_t *>(scr_all[w]);
    const int s = chunk_seg[c], r0 = chunk_row0[c];
    const int n = __builtin_amdgcn_readfirstlane(valid ? min(C, seg_len[s] - r0) : 1);
    // a chunk of at most 32 tokens needs only the top-left 32 x 32 blocks of
    // T and P (the rest belongs to rows past its last token, never stored;
    // the blocks it needs do not depend on them, so their bits are the same)
    const bool shortc = n <= C / 2;
    const size_t t0 = (size_t)seg_start[s] + r0;
    const int g = h / (Hv / Hk);
    // operand fragments: rows 16*t + c16, dims 32*kk + 8*G .. +8 (zero past n);
    // all key tiles are held, query tiles only while P uses them
    auto frag = [&](const uint16_t *src, int t, bf16x8 *f) {
        const int row = t * 16 + c16, rr = row < n ? row : n - 1;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            uint4 v = *reinterpret_cast<const uint4 *>(src + ((t0 + rr) * Hk + g) * DK + kk * 32 + G * 8);
            if (row >= n) v = make_uint4(0, 0, 0, 0);
            f[kk] = as_bf16x8(v);
        }
    };
    bf16x8 kf[4][4], qc[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        if (t < 2 || !shortc) {
            frag(k, t, kf[t]);
        } else {
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) kf[t][kk] = as_bf16x8(make_uint4(0, 0, 0, 0));
        }
    }
    const int lr = lane < n ? lane : n - 1;
    float la = lane < n ? logf(a[(t0 + lr) * Hv + h]) : 0.f;
    const float eta = lane < n ? b[(t0 + lr) * Hv + h] : 0.f;
    for (int o = 1; o < 64; o <<= 1) {
        const float y = __shfl_up(la, o, 64);
        if (lane >= o) la += y;
    }
    lsh[lane] = la;
    esh[lane] = eta;
    if (valid) lvec[((size_t)c * Hv + h) * C + lane] = la;   // read back by the chunk walk
    __syncthreads();
    // P^T tiles K_j Q_i^T: lane holds (row j = 16*jt + 4G + r, col i = 16*it + c16),
    // i.e. four consecutive j of one row i of P -> one 8-byte store per tile
    uint16_t *pdst = pmat + ((size_t)c * Hv + h) * C * C;
#pragma unroll
    for (int it = 0; it < 4; ++it) {
        if (it >= 2 && shortc) continue;   // rows 32..63: none
        frag(q, it, qc);
        const int i = it * 16 + c16;
        const float li = lsh[i];
#pragma unroll
        for (int jt = 0; jt < 4; ++jt) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            if (jt <= it) {
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) acc = mfma(kf[jt][kk], qc[kk], acc);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int j = jt * 16 + G * 4 + r;
                    acc[r] = j <= i ? __expf(li - lsh[j]) * acc[r] : 0.f;
                }
            }
            __bf16 p4[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) p4[r] = (__bf16)acc[r];
            // rows past the chunk's last token are never read, nor is the
            // zero block of rows 0-31 x columns 32-63
            if (valid && i < n && !(it < 2 && jt >= 2))
                *reinterpret_cast<uint2 *>(pdst + i * C + perm_off(jt * 16 + G * 4)) = __builtin_bit_cast(uint2, p4);
        }
    }
    // T = (I + A)^-1 by 16 x 16 blocks, A = the strictly lower part of
    // diag(b) (Gamma o K K^T):  diagonal blocks T_bb = (I + A_bb)^-1 by
    // forward substitution (lane = block x column), then
    //   T_ij = -T_ii sum_{k=j}^{i-1} A_ik T_kj   (i > j)
    // on fp32 MFMA, in an order where every T_kj on the right is known.  The
    // 16x16x4 fp32 products take reduction position 4G + s in instruction s
    // from lane group G, so a product's accumulator (rows 4G..4G+3 of a
    // column) is directly the B operand of the next one.
    // (1) off-diagonal blocks of A as A operands: lane (G, c16) holds
    //     A_{bi,bk}[c16][4G + s] in register s, from the tile K_bk K_bi^T
    constexpr int BI[6] = {1, 2, 2, 3, 3, 3}, BK[6] = {0, 0, 1, 0, 1, 2};
    f32x4 aop[6];
#pragma unroll
    for (int p = 0; p < 6; ++p) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        if (BI[p] >= 2 && shortc) {
            aop[p] = acc;
            continue;
        }
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) acc = mfma(kf[BK[p]][kk], kf[BI[p]][kk], acc);
        const int i = BI[p] * 16 + c16;
        const float ei = esh[i], li = lsh[i];
#pragma unroll
        for (int r = 0; r < 4; ++r) aop[p][r] = ei * __expf(li - lsh[BK[p] * 16 + G * 4 + r]) * acc[r];
    }
    // (2) diagonal blocks of A, row-major in LDS: ad[b][row][col]
    constexpr int DB = 16 * 16 + 16;   // block stride (floats): blocks on different banks
    float *ad = am;
#pragma unroll
    for (int bk = 0; bk < 4; ++bk) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        if (bk < 2 || !shortc)
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) acc = mfma(kf[bk][kk], kf[bk][kk], acc);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int ri = G * 4 + r, i = bk * 16 + ri, j = bk * 16 + c16;
            ad[bk * DB + ri * 16 + c16] = c16 < ri ? esh[i] * __expf(lsh[i] - lsh[j]) * acc[r] : 0.f;
        }
    }
    __syncthreads();
    // (3) T_bb column cc in lane (bb, cc)
    const int bb = lane >> 4, cc = lane & 15;
    float x[16];
#pragma unroll
    for (int kr = 0; kr < 16; ++kr) {
        float acc0 = kr == cc ? 1.f : 0.f, acc1 = 0.f;
        const float *arow = ad + bb * DB + kr * 16;
#pragma unroll
        for (int j = 0; j < kr; j += 2) {
            acc0 -= arow[j] * x[j];
            if (j + 1 < kr) acc1 -= arow[j + 1] * x[j + 1];
        }
        x[kr] = acc0 + acc1;
    }
    __syncthreads();
    float *td = am;   // T_bb, row-major, same place
#pragma unroll
    for (int kr = 0; kr < 16; ++kr) td[bb * DB + kr * 16 + cc] = x[kr];
    __syncthreads();
    auto tB = [&](int b_) {   // T_bb as a B operand: rows 4G..4G+3, column c16
        f32x4 v;
#pragma unroll
        for (int r = 0; r < 4; ++r) v[r] = td[b_ * DB + (G * 4 + r) * 16 + c16];
        return v;
    };
    auto tA = [&](int b_) {   // T_bb as an A operand: row c16, columns 4G..4G+3
        return *reinterpret_cast<const f32x4 *>(td + b_ * DB + c16 * 16 + G * 4);
    };
    auto mm = [](f32x4 A_, f32x4 B_, f32x4 acc) {
#pragma unroll
        for (int s_ = 0; s_ < 4; ++s_) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(A_[s_], B_[s_], acc, 0, 0, 0);
        return acc;
    };
    const f32x4 z = {0.f, 0.f, 0.f, 0.f};
    const f32x4 t00 = tB(0), t11 = tB(1), t22 = tB(2);
    const f32x4 a1 = tA(1), a2 = tA(2), a3 = tA(3);
    const f32x4 t10 = -mm(a1, mm(aop[0], t00, z), z);
    f32x4 t21 = z, t32 = z, t20 = z, t31 = z, t30 = z;
    if (!shortc) {
        t21 = -mm(a2, mm(aop[2], t11, z), z);
        t32 = -mm(a3, mm(aop[5], t22, z), z);
        t20 = -mm(a2, mm(aop[2], t10, mm(aop[1], t00, z)), z);
        t31 = -mm(a3, mm(aop[5], t21, mm(aop[4], t11, z)), z);
        t30 = -mm(a3, mm(aop[5], t20, mm(aop[4], t10, mm(aop[3], t00, z))), z);
    }
    __syncthreads();
    // (4) T as bf16 rows (the blocks above the diagonal are never read)
    auto tbw = [&](int row, int col, float v_) { tb[row * TBS + col] = __builtin_bit_cast(uint16_t, (__bf16)v_); };
#pragma unroll
    for (int kr = 0; kr < 16; ++kr) tbw(bb * 16 + kr, bb * 16 + cc, x[kr]);
    auto put = [&](int bi, int bj, f32x4 t) {
#pragma unroll
        for (int r = 0; r < 4; ++r) tbw(bi * 16 + G * 4 + r, bj * 16 + c16, t[r]);
    };
    put(1, 0, t10);
    put(2, 1, t21);
    put(3, 2, t32);
    put(2, 0, t20);
    put(3, 1, t31);
    put(3, 0, t30);
    __syncthreads();
    if (!valid || lane >= n) return;   // rows past the chunk's last token are never read
    // row `lane` of T, stored permuted (both T and P serve as A operands);
    // the zero block of rows 0-31 x columns 32-63 (stored units 4-7) is
    // never read
    uint16_t *dst = tmat + (((size_t)c * Hv + h) * C + lane) * C;
#pragma unroll
    for (int j8 = 0; j8 < C / 8; ++j8) {
        if (j8 >= 4 && lane < 32) continue;
        // stored elements [8 j8, 8 j8 + 8): positions 4G'..4G'+3 and
        // 16+4G'..16+4G'+3 of block j8/4, G' = j8 % 4 (each group of four
        // lies in one 16-column block, above the diagonal block or not)
        const int base = (j8 >> 2) * 32 + 4 * (j8 & 3);
        uint2 lo = *reinterpret_cast<const uint2 *>(tb + lane * TBS + base);
        uint2 hi = *reinterpret_cast<const uint2 *>(tb + lane * TBS + base + 16);
        if ((base >> 4) > (lane >> 4)) lo = make_uint2(0, 0);
        if (((base + 16) >> 4) > (lane >> 4)) hi = make_uint2(0, 0);
        *reinterpret_cast<uint4 *>(dst + j8 * 8) = make_uint4(lo.x, lo.y, hi.x, hi.y);
    }
}

// ---------------------------------------------------------------------------
// Chunk walk of one tree level, persistent: item = (segment, v-head, 64-wide
// dv slice), dealt to the work-groups as `Walk` describes; a work-group runs
// its items, and within an item its chunks, in order -- one flat sequence of
// steps.  Waves 0-3 (consumers) own the state slice and run the
// state-dependent products of step j; waves 4-11 (producers, 8 token rows
// each) meanwhile write step j+1 (already in their registers) into the other
// LDS buffer, issue the global loads of step j+2, and store the output of
// step j-1 that the consumers left in the value buffer.  When a step starts an item, the
// producers have staged that item's entering state (zero, state_in, or the
// parent's fork-point state) in LDS, so no wave waits on HBM at an item
// boundary.  The assignment of items to work-groups never changes an item's
// arithmetic.
// ---------------------------------------------------------------------------
struct ChunkArgs {
    const uint16_t *q, *k, *v;
    const float *b;
    uint16_t *out;
    int T, Hk, Hv, level, level_cap;
    const int32_t *header, *lvl_sorted, *seg_start, *seg_len, *seg_src, *seg_chunk0, *emit_off, *emit_pos,
        *seg_state_out;
    const uint16_t *tmat, *pmat;
    const float *lvec;
    const float *state_in;
    float *state_out, *fork_states;
};

constexpr int CONSUMERS = DVS / 16;           // 4 waves, 16 dv columns each
constexpr int PRODUCERS = 8;
constexpr int CHUNK_THREADS = (CONSUMERS + PRODUCERS) * 64;
constexpr int PROWS = C / PRODUCERS;          // token rows (and state rows) a producer stages
constexpr int KQ_LD = PROWS / 4;              // key / query loads: 4 rows x 16 lanes each
constexpr int ROW_LD = PROWS / 8;             // 64-wide row loads: 8 rows x 8 lanes each
constexpr int S0_LD = DVS / PRODUCERS / 2;    // entering-state loads: 2 rows x 32 lanes each
constexpr int S0S = DK + 4;                   // LDS stride (fp32) of the staged entering state
constexpr int NSL = DV / DVS;                 // dv slices per v-head

struct ChunkBuf {
    uint16_t kr[C * KS];     // key rows
    uint16_t qr[C * KS];     // query rows
    uint16_t tm[C * RS];     // T = (I + A)^-1
    uint16_t pm[C * RS];     // P = Gamma o Q K^T
    uint16_t vs[C * RS];     // values of this dv slice, then the chunk's output
    float lsh[C];            // log-decay prefix l_i
    float esh[C];            // write strength b_i
    float gsh[C];            // e^{l_i}
    float dsh[C];            // e^{l_last - l_i}
};

constexpr size_t CHUNK_LDS = 2 * sizeof(ChunkBuf) + sizeof(float) * DVS * S0S;

// Round metadata is never written while the level runs, so it is read
// through the constant address space: uniform indices then become scalar
// loads, which wait on nothing but themselves (a vector load's wait would
// also drain the producers' prefetches).
__device__ __forceinline__ int ldc(const int32_t *p, int i)
{
    return ((const __attribute__((address_space(4))) int32_t *)p)[i];
}

struct Item {
    int s, h, dv0, len, chunk0, t0, src;
};

__device__ __forceinline__ int item_nch(const Item &I) { return (I.len + C - 1) / C; }

// How a level's items are dealt to the G work-groups.  The items of one
// segment that read the same key and query rows -- every v-head of a k-head
// and every dv slice, M of them -- form a group, and M work-groups on one
// XCD (work-group b runs on XCD b mod 8) take the M members of the same
// groups in the same order, so the M reads of a chunk's keys and queries
// (and the two reads of its T and P per v-head) meet in that XCD's L2 at
// about the same time: the members of a group walk the same number of chunks.
// Groups are numbered k-head major, segment rank minor, so a member's
// consecutive groups are sibling segments on the same v-head and slice --
// they enter from the same fork-point state.  A level with at least 4 Q
// groups per member set (Q = G / M sets) is dealt in contiguous runs (set q
// takes groups [q per, q per + per)), so a run of siblings stages their
// common entering state once; a smaller level is dealt forward and backward
// in turn (groups q, 2Q-1-q, 2Q+q, ...), pairing its long segments with its
// short ones.  When G is not a multiple of 8 M, every item is its own group
// (M = 1).  Item id = group * M + member; once an id reaches n_items every
// later id of the same work-group does too.
struct Walk {
    int n_items, nseg, n_grp, Q, per, M, set, mem;
    bool runs;
};

__device__ __forceinline__ Walk make_walk(int nseg, int Hv, int Hk, int G, int b)
{
    Walk W;
    W.nseg = nseg;
    W.n_items = nseg * Hv * NSL;
    const int M = (Hv / Hk) * NSL;
    W.M = G % (8 * M) == 0 ? M : 1;
    // work-group b: XCD x = b mod 8, y = b / 8; member y mod M of set x + 8 (y / M)
    const int x = b & 7, y = b >> 3;
    W.mem = W.M == 1 ? 0 : y % W.M;
    W.set = W.M == 1 ? b : x + 8 * (y / W.M);
    W.Q = G / W.M;
    W.n_grp = W.n_items / W.M;
    W.runs = W.n_grp >= 4 * W.Q;
    W.per = (W.n_grp + W.Q - 1) / W.Q;
    return W;
}

__device__ __forceinline__ int item_id(const Walk &W, int k)
{
    int g;
    if (W.runs)
        g = k < W.per ? W.set * W.per + k : W.n_grp;
    else
        g = k * W.Q + ((k & 1) ? W.Q - 1 - W.set : W.set);
    return g >= W.n_grp ? 0x7fffffff : g * W.M + W.mem;
}

__device__ __forceinline__ Item item_at(const ChunkArgs &A, const Walk &W, int it)
{
    Item I;
    // group g = (k-head block, segment rank); member m -> (v-head, slice)
    const int g = it / W.M, m = it % W.M;
    const int rank = g % W.nseg, hs = (g / W.nseg) * W.M + m;
    I.s = ldc(A.lvl_sorted, A.level * A.level_cap + rank);
    I.h = hs / NSL;
    I.dv0 = (hs % NSL) * DVS;
    I.len = ldc(A.seg_len, I.s);
    I.chunk0 = ldc(A.seg_chunk0, I.s);
    I.t0 = ldc(A.seg_start, I.s);
    I.src = ldc(A.seg_src, I.s);
    return I;
}

// the entering state of an item: null = zero state
__device__ __forceinline__ const float *item_s0(const ChunkArgs &A, const Item &I)
{
    const size_t SZ = (size_t)DV * DK;
    if (I.src == -1) return nullptr;
    return I.src >= 0 ? A.fork_states + ((size_t)I.src * A.Hv + I.h) * SZ
                      : A.state_in + ((size_t)(-2 - I.src) * A.Hv + I.h) * SZ;
}

// fork points of an item's segment (range e .. e_end of emit_pos), the
// offset of the next one (INT_MAX when none is left) and its state_out slot
struct Emits {
    int e, e_end, next, so;
};

__device__ __forceinline__ Emits item_emits(const ChunkArgs &A, const Item &I)
{
    Emits E;
    E.e = ldc(A.emit_off, I.s);
    E.e_end = ldc(A.emit_off, I.s + 1);
    E.next = E.e < E.e_end ? ldc(A.emit_pos, E.e) : 0x7fffffff;
    E.so = ldc(A.seg_state_out, I.s);
    return E;
}

__device__ __forceinline__ void emit_advance(const ChunkArgs &A, Emits &E)
{
    ++E.e;
    E.next = E.e < E.e_end ? ldc(A.emit_pos, E.e) : 0x7fffffff;
}

// 16 dk x 4-row fp32 state fragment <-> global [dv][dk] row (4 consecutive dk)
__device__ __forceinline__ void store_state(float *base, int dvc, int G, const f32x4 *st)
{
#pragma unroll
    for (int i = 0; i < DK / 16; ++i)
        *reinterpret_cast<f32x4 *>(base + (size_t)dvc * DK + i * 16 + G * 4) = st[i];
}

// producer `part`: store token rows [PROWS part, +PROWS) of the output slice of
// chunk `c` of item I (left in B.vs by the consumers), 8 lanes x 16 B per row
__device__ __forceinline__ void flush_out(const ChunkBuf &B, const ChunkArgs &A, const Item &I, int c, int lane,
                                          int part)
{
    const int n = min(C, I.len - c * C);
    const size_t t0 = (size_t)I.t0 + (size_t)c * C;
#pragma unroll
    for (int j = 0; j < ROW_LD; ++j) {
        const int idx = j * 64 + lane, row = part * PROWS + (idx >> 3), c8 = idx & 7;
        if (row < n)
            *reinterpret_cast<uint4 *>(A.out + ((t0 + row) * A.Hv + I.h) * DV + I.dv0 + c8 * 8) =
                *reinterpret_cast<const uint4 *>(B.vs + r64_off(row, c8 * 8));
    }
}

// Operand of K^T for the state update, read from the key rows with the LDS
// transpose read: within each 16-lane group, source lane s points at token
// row t0 + s/4, key dims d0 + 4(s%4) .. +3 (a group of four, wherever the
// permuted row stores it), and lane i receives key dim d0 + i of tokens
// t0 .. t0+3.  Two reads give the permuted reduction index
// (tokens 32 ks + 4G .. +3 and 32 ks + 16 + 4G .. +3) of lane group G.
typedef short v4s __attribute__((ext_vector_type(4)));
__device__ __forceinline__ bf16x8 load_kT(const uint16_t *kr, int d0, int ks, int lane)
{
    const int G = lane >> 4, sl = lane & 15;
    const int row = ks * 32 + 4 * G + (sl >> 2), e = perm_off(d0 + 4 * (sl & 3));
    typedef __attribute__((address_space(3))) v4s lds_v4s;
    const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s *)(kr + kq_off(row, e)));
    const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s *)(kr + kq_off(row + 16, e)));
    const uint2 l2 = __builtin_bit_cast(uint2, lo), h2 = __builtin_bit_cast(uint2, hi);
    return as_bf16x8(make_uint4(l2.x, l2.y, h2.x, h2.y));
}

// transpose read (see load_kT) of four consecutive rows of 16 columns
__device__ __forceinline__ v4s load_tr(const uint16_t *p)
{
    typedef __attribute__((address_space(3))) v4s lds_v4s;
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s *)p);
}

// two fp32 -> two bf16 (RNE) in one word, the first in the low half
__device__ __forceinline__ uint32_t pack2(float a, float b)
{
    return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)a) | ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)b) << 16);
}

// One step's worth of a producer's loads, held in registers between the
// interval that issues them and the interval that writes them to LDS.
struct StepRegs {
    uint4 kv[KQ_LD], qv[KQ_LD], tv[ROW_LD], pv[ROW_LD], vv[ROW_LD];
    f32x4 s0[S0_LD];
    float l_raw, b_raw;
    bool s0_write;   // this step starts an item whose entering state is not staged yet
};

// issue the loads of chunk c of item I (and, when `stage_s0`, of its entering
// state); rows [PROWS part, +PROWS) of the chunk, dv rows of the state
// likewise.  Coalesced: consecutive lanes read consecutive 16 B of a row.
// Rows past the chunk's last token are not read (zero): nothing uses them --
// T and P are lower triangular, and zero key rows keep them out of the state.
__device__ __forceinline__ void load_step(StepRegs &R, const ChunkArgs &A, const Item &I, int c, int lane, int part,
                                          bool stage_s0)
{
    const int n = min(C, I.len - c * C);
    const size_t t0 = (size_t)I.t0 + (size_t)c * C;
    const size_t mat = ((size_t)(I.chunk0 + c) * A.Hv + I.h) * C * C;
    const int rb = part * PROWS;
    // buffer resources based at this chunk's first row: 32-bit offsets, and
    // the hardware range check returns zeros past the end of each tensor
    const size_t kq_base = (t0 * A.Hk + I.h / (A.Hv / A.Hk)) * DK, kq_end = (size_t)A.T * A.Hk * DK;
    const size_t v_base = (t0 * A.Hv + I.h) * DV + I.dv0, v_end = (size_t)A.T * A.Hv * DV;
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(A.k + kq_base, (kq_end - kq_base) * 2);
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(A.q + kq_base, (kq_end - kq_base) * 2);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(A.v + v_base, (v_end - v_base) * 2);
    const __amdgpu_buffer_rsrc_t rt = make_rsrc(A.tmat + mat, (size_t)C * C * 2);
    const __amdgpu_buffer_rsrc_t rp = make_rsrc(A.pmat + mat, (size_t)C * C * 2);
    const int kq_row = A.Hk * DK * 2, v_row = A.Hv * DV * 2;   // bytes between tokens
#pragma unroll
    for (int j = 0; j < KQ_LD; ++j) {           // 4 rows x 16 lanes per instruction
        const int idx = j * 64 + lane, row = rb + (idx >> 4), c8 = idx & 15;
        R.kv[j] = R.qv[j] = make_uint4(0, 0, 0, 0);
        if (row < n) {
            R.kv[j] = buf_load(rk, row * kq_row + c8 * 16);
            R.qv[j] = buf_load(rq, row * kq_row + c8 * 16);
        }
    }
#pragma unroll
    for (int j = 0; j < ROW_LD; ++j) {          // 8 rows x 8 lanes per instruction
        const int idx = j * 64 + lane, row = rb + (idx >> 3), c8 = idx & 7;
        R.tv[j] = R.pv[j] = R.vv[j] = make_uint4(0, 0, 0, 0);
        if (row < n) {
            // T and P: the block of rows 0-31 x columns 32-63 (units 4-7)
            // is zero and never read, and is not stored
            if (row >= 32 || c8 < 4) {
                R.tv[j] = buf_load(rt, row * C * 2 + c8 * 16);
                R.pv[j] = buf_load(rp, row * C * 2 + c8 * 16);
            }
            R.vv[j] = buf_load(rv, row * v_row + c8 * 16);
        }
    }
    R.l_raw = 0.f;
    R.b_raw = 0.f;
    if (part == 0) {
        const int rr = lane < n ? lane : n - 1;
        R.l_raw = A.lvec[((size_t)(I.chunk0 + c) * A.Hv + I.h) * C + lane];
        R.b_raw = A.b[(t0 + rr) * A.Hv + I.h];
    }
    R.s0_write = c == 0 && stage_s0;
    if (R.s0_write) {
        // dv rows [DVS / PRODUCERS part, +DVS / PRODUCERS) of the slice, 32 lanes x 16 B per row
        const float *S0 = item_s0(A, I);
#pragma unroll
        for (int j = 0; j < S0_LD; ++j) {
            const int idx = j * 64 + lane, row = part * (DVS / PRODUCERS) + (idx >> 5), c4 = idx & 31;
            R.s0[j] = S0 ? *reinterpret_cast<const f32x4 *>(S0 + (size_t)(I.dv0 + row) * DK + c4 * 4)
                         : f32x4{0.f, 0.f, 0.f, 0.f};
        }
    }
}

// write a step's registers into LDS buffer B (and the entering state into s0)
__device__ __forceinline__ void write_step(ChunkBuf &B, float *s0, StepRegs &R, const Item &I, int c, int lane,
                                           int part)
{
    const int n = min(C, I.len - c * C);
    const int rb = part * PROWS;
#pragma unroll
    for (int j = 0; j < KQ_LD; ++j) {
        const int idx = j * 64 + lane, row = rb + (idx >> 4), c8 = idx & 15;
        if (row >= n) R.kv[j] = R.qv[j] = make_uint4(0, 0, 0, 0);
        // key dims 8 c8 .. 8 c8 + 7 = position groups 2 c8 and 2 c8 + 1; lanes
        // of the upper 64 dims write their second group first, so each
        // instruction's 16 lanes cover 128 distinct bytes of the bank space
        const bool sw = c8 >= 8;
        const int o0 = kq_off(row, perm_off(c8 * 8 + (sw ? 4 : 0))), o1 = kq_off(row, perm_off(c8 * 8 + (sw ? 0 : 4)));
        *reinterpret_cast<uint2 *>(B.kr + o0) = sw ? make_uint2(R.kv[j].z, R.kv[j].w) : make_uint2(R.kv[j].x, R.kv[j].y);
        *reinterpret_cast<uint2 *>(B.kr + o1) = sw ? make_uint2(R.kv[j].x, R.kv[j].y) : make_uint2(R.kv[j].z, R.kv[j].w);
        *reinterpret_cast<uint2 *>(B.qr + o0) = sw ? make_uint2(R.qv[j].z, R.qv[j].w) : make_uint2(R.qv[j].x, R.qv[j].y);
        *reinterpret_cast<uint2 *>(B.qr + o1) = sw ? make_uint2(R.qv[j].x, R.qv[j].y) : make_uint2(R.qv[j].z, R.qv[j].w);
    }
#pragma unroll
    for (int j = 0; j < ROW_LD; ++j) {
        const int idx = j * 64 + lane, row = rb + (idx >> 3), c8 = idx & 7;
        if (row >= n) R.vv[j] = make_uint4(0, 0, 0, 0);
        *reinterpret_cast<uint4 *>(B.tm + r64_off(row, c8 * 8)) = R.tv[j];
        *reinterpret_cast<uint4 *>(B.pm + r64_off(row, c8 * 8)) = R.pv[j];
        *reinterpret_cast<uint4 *>(B.vs + r64_off(row, c8 * 8)) = R.vv[j];
    }
    if (part == 0) {
        // l as the prep kernel computed it (lanes past the chunk hold l_{n-1})
        const bool live = lane < n;
        const float la = R.l_raw;
        const float eta = live ? R.b_raw : 0.f;
        const float last = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(la), C - 1));
        B.lsh[lane] = la;
        B.esh[lane] = eta;
        B.gsh[lane] = __expf(la);
        B.dsh[lane] = __expf(last - la);
    }
    if (c == 0 && R.s0_write) {
#pragma unroll
        for (int j = 0; j < S0_LD; ++j) {
            const int idx = j * 64 + lane, row = part * (DVS / PRODUCERS) + (idx >> 5), c4 = idx & 31;
            *reinterpret_cast<f32x4 *>(s0 + row * S0S + c4 * 4) = R.s0[j];
        }
    }
}

__global__ void __launch_bounds__(CHUNK_THREADS) k_gdn_chunk(ChunkArgs A)
{
    extern __shared__ __attribute__((aligned(16))) char smem[];
    ChunkBuf *buf = reinterpret_cast<ChunkBuf *>(smem);
    float *s0buf = reinterpret_cast<float *>(smem + 2 * sizeof(ChunkBuf));
    if (ldc(A.header, H_STATUS) != FK_OK) return;
    // item ids: (segment rank, v-head, dv slice), slice fastest
    const Walk W = make_walk(ldc(A.header, H_LEVEL0 + A.level), A.Hv, A.Hk, gridDim.x, blockIdx.x);
    const int n_items = W.n_items;
    const int b0 = item_id(W, 0);
    if (b0 >= n_items) return;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int G = lane >> 4, c16 = lane & 15;

    // Both roles walk the same step sequence and meet at the same barriers:
    // one before step 0, one extra at the start of every item (the entering
    // state has been read), one at the end of every step.  Roles are
    // wave-uniform and run separate loops, so their registers are allocated
    // independently.
    if (w >= CONSUMERS) {
        const int part = w - CONSUMERS;
        StepRegs R;
        int c = 0;
        Item cur = item_at(A, W, b0);
        // the item after the last one handed to a step, looked up one item
        // ahead so its (dependent) scalar loads are long done when it is used
        int la_k = 1;
        int la_it = item_id(W, la_k);
        Item la = la_it < n_items ? item_at(A, W, la_it) : cur;
        auto take = [&](Item &I) {
            I = la;
            la_it = item_id(W, ++la_k);
            if (la_it < n_items) la = item_at(A, W, la_it);
        };
        // the entering state staged last (in item order): a sibling entering
        // from the same state on the same head and slice finds it in LDS
        int ls_src = 0, ls_h = -1, ls_dv0 = -1;
        auto stage = [&](const Item &I, int cc) {
            if (cc != 0) return false;
            const bool same = I.src == ls_src && I.h == ls_h && I.dv0 == ls_dv0;
            ls_src = I.src;
            ls_h = I.h;
            ls_dv0 = I.dv0;
            return !same;
        };
        load_step(R, A, cur, 0, lane, part, stage(cur, 0));
        write_step(buf[0], s0buf, R, cur, 0, lane, part);
        // step 1 into registers
        int c1 = 1;
        bool has1 = true;
        Item nx1 = cur;
        if (c1 == item_nch(cur)) {
            c1 = 0;
            has1 = la_it < n_items;
            if (has1) take(nx1);
        }
        if (has1) load_step(R, A, nx1, c1, lane, part, stage(nx1, c1));
        __syncthreads();
        Item prev = cur;
        int pc = -1;
        for (int j = 0;; ++j) {
            // step j = (cur, c) is being consumed; step j+1 = (nx1, c1) sits in R
            if (c == 0) __syncthreads();   // consumers have read the entering state
            // step j+2
            int c2 = c1 + 1;
            bool has2 = has1;
            Item nx2 = nx1;
            if (has1 && c2 == item_nch(nx1)) {
                c2 = 0;
                has2 = la_it < n_items;
                if (has2) take(nx2);
            }
            if (has1) {
                ChunkBuf &Bn = buf[(j + 1) & 1];
                if (pc >= 0) flush_out(Bn, A, prev, pc, lane, part);
                write_step(Bn, s0buf, R, nx1, c1, lane, part);
            }
            if (has2) load_step(R, A, nx2, c2, lane, part, stage(nx2, c2));
            __syncthreads();   // step j consumed, step j+1 staged
            if (!has1) {
                // outputs of steps j-1 and j are still in LDS
                if (pc >= 0) flush_out(buf[(j + 1) & 1], A, prev, pc, lane, part);
                flush_out(buf[j & 1], A, cur, c, lane, part);
                return;
            }
            prev = cur;
            pc = c;
            cur = nx1;
            c = c1;
            c1 = c2;
            has1 = has2;
            nx1 = nx2;
        }
    }

    const int wv = w;   // consumer wave: dv columns [16 w, 16 w + 16) of the slice
    f32x4 st[DK / 16];
    int ik = 0, c = 0;
    Item cur = item_at(A, W, b0);
    Emits E = item_emits(A, cur);
    const size_t SZ = (size_t)DV * DK;
    __syncthreads();
    for (int j = 0;; ++j) {
        ChunkBuf &B = buf[j & 1];
        const int dvc = cur.dv0 + wv * 16 + c16;   // this lane's state column (dv index)
        const bool last = c + 1 == item_nch(cur);
        // the next item's metadata, fetched while this step computes
        const int next_it = item_id(W, ik + 1);
        const bool more = !last || next_it < n_items;
        Item nxt = cur;
        Emits nE = E;
        if (last && more) {
            nxt = item_at(A, W, next_it);
            nE = item_emits(A, nxt);
        }
        if (c == 0) {
#pragma unroll
            for (int i = 0; i < DK / 16; ++i)
                st[i] = *reinterpret_cast<const f32x4 *>(s0buf + (wv * 16 + c16) * S0S + i * 16 + G * 4);
            __syncthreads();   // the producers may now stage the next entering state
            while (E.next == 0) {
                store_state(A.fork_states + ((size_t)E.e * A.Hv + cur.h) * SZ, dvc, G, st);
                emit_advance(A, E);
            }
        }
        const int n = min(C, cur.len - c * C);
        // X = K S0^T, Y = Q S0^T for this wave's 16 dv columns
        f32x4 xa[C / 16], ya[C / 16];
#pragma unroll
        for (int mt = 0; mt < C / 16; ++mt) xa[mt] = ya[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks2 = 0; ks2 < DK / 32; ++ks2) {
            const bf16x8 sb = pack(st[2 * ks2], st[2 * ks2 + 1]);
#pragma unroll
            for (int mt = 0; mt < C / 16; ++mt) {
                xa[mt] = mfma(load_kq(B.kr, mt * 16 + c16, ks2, G), sb, xa[mt]);
                ya[mt] = mfma(load_kq(B.qr, mt * 16 + c16, ks2, G), sb, ya[mt]);
            }
        }
        __builtin_amdgcn_sched_barrier(0);   // bound the operand loads kept in flight
        // R = diag(b) (V - diag(e^l) X);  U = T R.  A lane's four rows are
        // 4 consecutive tokens of one dv column: one transpose read of V.
#pragma unroll
        for (int mt = 0; mt < C / 16; ++mt) {
            const int i0 = mt * 16 + G * 4;
            const v4s vq = load_tr(B.vs + r64_off(i0 + (c16 >> 2), wv * 16 + 4 * (c16 & 3)));
            const f32x4 eb = *reinterpret_cast<const f32x4 *>(B.esh + i0);
            const f32x4 gb = *reinterpret_cast<const f32x4 *>(B.gsh + i0);
#pragma unroll
            for (int r = 0; r < 4; ++r)
                xa[mt][r] = eb[r] * (bf16_to_f32((uint16_t)vq[r]) - gb[r] * xa[mt][r]);
        }
        const bf16x8 rb0 = pack(xa[0], xa[1]), rb1 = pack(xa[2], xa[3]);
        f32x4 ua[C / 16];
#pragma unroll
        for (int mt = 0; mt < C / 16; ++mt) {
            ua[mt] = mfma(load_perm(B.tm, mt * 16 + c16, 0, G), rb0, f32x4{0.f, 0.f, 0.f, 0.f});
            // T is lower triangular: rows 0..31 have no entries in columns 32..63
            if (mt >= 2) ua[mt] = mfma(load_perm(B.tm, mt * 16 + c16, 1, G), rb1, ua[mt]);
        }
        __builtin_amdgcn_sched_barrier(0);
        // O = diag(e^l) Y + P U  -> left in the value buffer for the producers
        const bf16x8 ub0 = pack(ua[0], ua[1]), ub1 = pack(ua[2], ua[3]);
        const bool odd = c16 & 1;
#pragma unroll
        for (int mt = 0; mt < C / 16; ++mt) {
            const int i0 = mt * 16 + G * 4;
            const f32x4 gb = *reinterpret_cast<const f32x4 *>(B.gsh + i0);
            f32x4 oa;
#pragma unroll
            for (int r = 0; r < 4; ++r) oa[r] = gb[r] * ya[mt][r];
            oa = mfma(load_perm(B.pm, mt * 16 + c16, 0, G), ub0, oa);
            if (mt >= 2) oa = mfma(load_perm(B.pm, mt * 16 + c16, 1, G), ub1, oa);
            // lanes c16 and c16^1 hold neighbouring dv columns of the same 4
            // rows: swap halves so each lane writes two rows x two columns
            const uint32_t lo = pack2(oa[0], oa[1]), hi = pack2(oa[2], oa[3]);   // (row0,row1), (row2,row3)
            const uint32_t mine = odd ? lo : hi;                                   // what the partner needs
            const uint32_t got = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)mine, 0xB1, 0xF, 0xF, false);
            const uint32_t keep = odd ? hi : lo;                                   // rows this lane writes
            // even lane: rows 0,1 of columns (c16, c16+1); odd lane: rows 2,3 of (c16-1, c16)
            const int col = wv * 16 + (c16 & ~1), rr = i0 + (odd ? 2 : 0);
            const uint32_t w0 = odd ? ((got & 0xffffu) | (keep << 16)) : ((keep & 0xffffu) | (got << 16));
            const uint32_t w1 = odd ? ((got >> 16) | (keep & 0xffff0000u)) : ((keep >> 16) | (got & 0xffff0000u));
            *reinterpret_cast<uint32_t *>(B.vs + r64_off(rr, col)) = w0;
            *reinterpret_cast<uint32_t *>(B.vs + r64_off(rr + 1, col)) = w1;
        }
        // fork points strictly inside this chunk: state after `off` tokens
        while (E.next < c * C + n) {
            const int off = E.next - c * C;   // 1 .. n-1
            const float lr = B.lsh[off - 1];
            f32x4 u0[C / 16];
#pragma unroll
            for (int mt = 0; mt < C / 16; ++mt)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int jj = mt * 16 + G * 4 + r;
                    u0[mt][r] = jj < off ? __expf(lr - B.lsh[jj]) * ua[mt][r] : 0.f;
                }
            const bf16x8 eb0 = pack(u0[0], u0[1]), eb1 = pack(u0[2], u0[3]);
            const float gr = __expf(lr);
            f32x4 tmp[DK / 16];
#pragma unroll
            for (int i = 0; i < DK / 16; ++i) {
                tmp[i] = mfma(load_kT(B.kr, i * 16, 0, lane), eb0, st[i] * gr);
                tmp[i] = mfma(load_kT(B.kr, i * 16, 1, lane), eb1, tmp[i]);
            }
            store_state(A.fork_states + ((size_t)E.e * A.Hv + cur.h) * SZ, dvc, G, tmp);
            emit_advance(A, E);
        }
        __builtin_amdgcn_sched_barrier(0);
        // S^T <- e^{l_last} S^T + K^T diag(e^{l_last - l}) U, unless nothing
        // reads the state after the item's last chunk
        if (!last || E.e < E.e_end || E.so >= 0) {
#pragma unroll
            for (int mt = 0; mt < C / 16; ++mt) {
                const f32x4 db = *reinterpret_cast<const f32x4 *>(B.dsh + mt * 16 + G * 4);
#pragma unroll
                for (int r = 0; r < 4; ++r) ua[mt][r] *= db[r];
            }
            const bf16x8 wb0 = pack(ua[0], ua[1]), wb1 = pack(ua[2], ua[3]);
            const float gl = B.gsh[C - 1];
#pragma unroll
            for (int i = 0; i < DK / 16; ++i) {
                st[i] = mfma(load_kT(B.kr, i * 16, 0, lane), wb0, st[i] * gl);
                st[i] = mfma(load_kT(B.kr, i * 16, 1, lane), wb1, st[i]);
            }
            // a fork point at the end of this chunk
            while (E.next == c * C + n) {
                store_state(A.fork_states + ((size_t)E.e * A.Hv + cur.h) * SZ, dvc, G, st);
                emit_advance(A, E);
            }
            if (last && E.so >= 0) store_state(A.state_out + ((size_t)E.so * A.Hv + cur.h) * SZ, dvc, G, st);
        }
        __syncthreads();   // step j consumed, step j+1 staged
        if (!more) return;
        if (!last) {
            ++c;
        } else {
            ++ik;
            cur = nxt;
            E = nE;
            c = 0;
        }
    }
}

}  // namespace gdnk
}  // namespace fk

using namespace fk;

int fk_launch_gdn_bf16_prep(const fk_tree_meta *meta, const void *q, const void *k, const float *a, const float *b,
                            int Hk, int Hv, const void *ws, hipStream_t st)
{
    const WsLayout L = ws_layout(*meta, Hv, gdnk::DK, gdnk::DV);
    const int64_t items = L.chunk_cap * Hv;
    dim3 grid((unsigned)((items + gdnk::PREP_WAVES - 1) / gdnk::PREP_WAVES));
    gdnk::k_gdn_prep<<<grid, 64 * gdnk::PREP_WAVES, 0, st>>>((const uint16_t *)q, (const uint16_t *)k, a, b, Hk, Hv,
                                                           ws_at<int32_t>(ws, L.header),
                                          ws_at<int32_t>(ws, L.chunk_seg), ws_at<int32_t>(ws, L.chunk_row0),
                                          ws_at<int32_t>(ws, L.seg_start), ws_at<int32_t>(ws, L.seg_len),
                                          const_cast<uint16_t *>(ws_at<uint16_t>(ws, L.tmat)),
                                          const_cast<uint16_t *>(ws_at<uint16_t>(ws, L.pmat)),
                                          const_cast<float *>(ws_at<float>(ws, L.lvec)));
    return launch_status();
}

int fk_launch_gdn_bf16(const fk_tree_meta *meta, int level, const void *q, const void *k, const void *v,
                       const float *a, const float *b, int Hk, int Hv, const float *state_in, float *state_out,
                       void *out, const void *ws, float *fork_states, hipStream_t st)
{
    const WsLayout L = ws_layout(*meta, Hv, gdnk::DK, gdnk::DV);
    gdnk::ChunkArgs A;
    A.q = (const uint16_t *)q;
    A.k = (const uint16_t *)k;
    A.v = (const uint16_t *)v;
    A.b = b;
    A.out = (uint16_t *)out;
    A.T = meta->T;
    A.Hk = Hk;
    A.Hv = Hv;
    A.level = level;
    A.level_cap = meta->level_cap;
    A.header = ws_at<int32_t>(ws, L.header);
    A.lvl_sorted = ws_at<int32_t>(ws, L.lvl_sorted);
    A.seg_start = ws_at<int32_t>(ws, L.seg_start);
    A.seg_len = ws_at<int32_t>(ws, L.seg_len);
    A.seg_src = ws_at<int32_t>(ws, L.seg_src);
    A.seg_chunk0 = ws_at<int32_t>(ws, L.seg_chunk0);
    A.emit_off = ws_at<int32_t>(ws, L.emit_off);
    A.emit_pos = ws_at<int32_t>(ws, L.emit_pos);
    A.seg_state_out = meta->seg_state_out;
    A.tmat = ws_at<uint16_t>(ws, L.tmat);
    A.pmat = ws_at<uint16_t>(ws, L.pmat);
    A.lvec = ws_at<float>(ws, L.lvec);
    A.state_in = state_in;
    A.state_out = state_out;
    A.fork_states = fork_states;
    // persistent: at most one work-group per compute unit (the LDS holds one)
    // per device, once: the compute-unit count, published only after the
    // kernel's LDS limit is raised (a caller on another thread that sees the
    // count may launch at once; one that sees 0 repeats the idempotent setup)
    int dev = 0;
    FK_HIP(hipGetDevice(&dev));
    static std::atomic<int> n_cu_dev[64];
    if (dev < 0 || dev >= 64) return FK_E_HIP;
    int n_cu = n_cu_dev[dev].load(std::memory_order_acquire);
    if (!n_cu) {
        FK_HIP(hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev));
        FK_HIP(hipFuncSetAttribute((const void *)gdnk::k_gdn_chunk, hipFuncAttributeMaxDynamicSharedMemorySize,
                                   (int)gdnk::CHUNK_LDS));
        n_cu_dev[dev].store(n_cu, std::memory_order_release);
    }
    const int64_t cap = (int64_t)meta->level_cap * Hv * gdnk::NSL;
    dim3 grid((unsigned)(cap < n_cu ? cap : n_cu));
    const size_t lds = gdnk::CHUNK_LDS;
    gdnk::k_gdn_chunk<<<grid, gdnk::CHUNK_THREADS, lds, st>>>(A);
    return launch_status();
}
