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
//             stored as bf16.  It depends only on k, a, b -- never on a state.
// k_gdn_chunk (one launch per tree level): one work-group per (segment,
//             v-head, 64-wide dv slice) walks the segment's chunks in order.
//             Each wave keeps its 128 x 16 slice of S^T in fp32 MFMA
//             accumulator registers for the whole segment and feeds it
//             straight back as an MFMA operand (a fixed permutation of the
//             reduction index makes the accumulator layout the operand
//             layout), so the state never leaves registers between chunks.
//             It starts from the zero state, state_in, or the parent's
//             fork-point state (by index), and writes the states at the
//             segment's fork points once each.
#include <hip/hip_runtime.h>

#include "fk_common.h"

namespace fk {
namespace gdnk {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int C = FK_GDN_CHUNK;   // 64 tokens
constexpr int DK = 128, DV = 128;
constexpr int DVS = 64;           // dv columns of one work-group (4 waves x 16)
constexpr int KS = DK + 8;        // LDS stride (bf16) of key/query rows
constexpr int TS = C + 8;         // LDS stride (bf16) of 64-wide rows written 16 B at a time (T, P)
constexpr int KTS = C + 4;        // LDS stride (bf16) of the transposed keys (written 2 B at a time)
constexpr int AS = C + 4;         // LDS stride (fp32) of the prep matrix

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

// Operand with a permuted reduction index: for a k-step over 32 positions,
// lane group G = lane/16 supplies positions 4G..4G+3 and 16+4G..16+4G+3 --
// exactly the rows a 16x16 accumulator pair holds in that lane group.
__device__ __forceinline__ bf16x8 load_perm(const uint16_t *row, int ks, int G)
{
    const uint2 lo = *reinterpret_cast<const uint2 *>(row + ks * 32 + 4 * G);
    const uint2 hi = *reinterpret_cast<const uint2 *>(row + ks * 32 + 16 + 4 * G);
    return as_bf16x8(make_uint4(lo.x, lo.y, hi.x, hi.y));
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
//   T = (I + A)^-1 (fp32 forward substitution, lane = column) and
//   P = Gamma o Q K^T (lower triangle incl. the diagonal), both stored bf16.
// Key and query rows are loaded straight into MFMA operand registers (the
// A and B operand layouts of a 16x16x32 product coincide), so LDS holds
// only the fp32 A matrix.  Four items per work-group, one wave each.
// ---------------------------------------------------------------------------
constexpr int PREP_WAVES = 4;

__global__ void __launch_bounds__(64 * PREP_WAVES)
k_gdn_prep(const uint16_t *__restrict__ q, const uint16_t *__restrict__ k, const float *__restrict__ a,
           const float *__restrict__ b, int Hk, int Hv, const int32_t *__restrict__ header,
           const int32_t *__restrict__ chunk_seg, const int32_t *__restrict__ chunk_row0,
           const int32_t *__restrict__ seg_start, const int32_t *__restrict__ seg_len,
           uint16_t *__restrict__ tmat, uint16_t *__restrict__ pmat)
{
    __shared__ __attribute__((aligned(16))) float am_all[PREP_WAVES][C * AS];
    __shared__ float lsh_all[PREP_WAVES][C], esh_all[PREP_WAVES][C];
    if (header[H_STATUS] != FK_OK) return;
    const int nitems = header[H_NCHUNKS] * Hv;
    if ((int)blockIdx.x * PREP_WAVES >= nitems) return;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, G = lane >> 4, c16 = lane & 15;
    const int item = blockIdx.x * PREP_WAVES + w;
    const bool valid = item < nitems;   // every wave reaches every barrier
    const int c = valid ? item / Hv : 0, h = valid ? item % Hv : 0;
    float *am = am_all[w], *lsh = lsh_all[w], *esh = esh_all[w];
    const int s = chunk_seg[c], r0 = chunk_row0[c];
    const int n = valid ? min(C, seg_len[s] - r0) : 1;
    const size_t t0 = (size_t)seg_start[s] + r0;
    const int g = h / (Hv / Hk);
    // operand fragments: rows 16*t + c16, dims 32*kk + 8*G .. +8 (zero past n)
    bf16x8 kf[4][4], qf[4][4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        const int row = t * 16 + c16, rr = row < n ? row : n - 1;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            uint4 kv = *reinterpret_cast<const uint4 *>(k + ((t0 + rr) * Hk + g) * DK + kk * 32 + G * 8);
            uint4 qv = *reinterpret_cast<const uint4 *>(q + ((t0 + rr) * Hk + g) * DK + kk * 32 + G * 8);
            if (row >= n) kv = qv = make_uint4(0, 0, 0, 0);
            kf[t][kk] = as_bf16x8(kv);
            qf[t][kk] = as_bf16x8(qv);
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
    __syncthreads();
    // P^T tiles K_j Q_i^T: lane holds (row j = 16*jt + 4G + r, col i = 16*it + c16),
    // i.e. four consecutive j of one row i of P -> one 8-byte store per tile
    uint16_t *pdst = pmat + ((size_t)c * Hv + h) * C * C;
#pragma unroll
    for (int it = 0; it < 4; ++it) {
        const int i = it * 16 + c16;
        const float li = lsh[i];
#pragma unroll
        for (int jt = 0; jt < 4; ++jt) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            if (jt <= it) {
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) acc = mfma(kf[jt][kk], qf[it][kk], acc);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int j = jt * 16 + G * 4 + r;
                    acc[r] = j <= i ? __expf(li - lsh[j]) * acc[r] : 0.f;
                }
            }
            __bf16 p4[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) p4[r] = (__bf16)acc[r];
            if (valid) *reinterpret_cast<uint2 *>(pdst + i * C + jt * 16 + G * 4) = __builtin_bit_cast(uint2, p4);
        }
    }
    // A = strictly lower part of diag(b) (Gamma o K K^T)
#pragma unroll
    for (int ti = 0; ti < 4; ++ti)
#pragma unroll
        for (int tj = 0; tj <= ti; ++tj) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) acc = mfma(kf[ti][kk], kf[tj][kk], acc);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int i = ti * 16 + G * 4 + r, j = tj * 16 + c16;
                am[i * AS + j] = j < i ? esh[i] * __expf(lsh[i] - lsh[j]) * acc[r] : 0.f;
            }
        }
    __syncthreads();
    // forward substitution: T[i][col] = delta(i, col) - sum_{j<i} A[i][j] T[j][col]
    float x[C];
#pragma unroll
    for (int i = 0; i < C; ++i) {
        float acc0 = i == lane ? 1.f : 0.f, acc1 = 0.f;
#pragma unroll
        for (int j = 0; j < i; j += 2) {
            acc0 -= am[i * AS + j] * x[j];
            if (j + 1 < i) acc1 -= am[i * AS + j + 1] * x[j + 1];
        }
        x[i] = acc0 + acc1;
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < C; ++i) am[i * AS + lane] = x[i];
    __syncthreads();
    if (!valid) return;
    uint16_t *dst = tmat + (((size_t)c * Hv + h) * C + lane) * C;
#pragma unroll
    for (int j8 = 0; j8 < C / 8; ++j8) {
        bf16x8 v;
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = (__bf16)am[lane * AS + j8 * 8 + e];
        *reinterpret_cast<uint4 *>(dst + j8 * 8) = __builtin_bit_cast(uint4, v);
    }
}

// ---------------------------------------------------------------------------
// Sequential chunk walk of one (segment, v-head, dv slice).
// Waves 0-3 (consumers) own the state and run the state-dependent products
// of chunk c; waves 4-7 (producers) meanwhile stage chunk c+1 into the other
// LDS buffer -- key rows and their transpose, query rows, T, P, the dv slice
// of the values, decay vectors -- each producer 16 token rows, with every
// global load of its rows in flight at once.  Consumers leave
// O in the value buffer; producers store it to HBM with 16-byte writes.
// ---------------------------------------------------------------------------
struct ChunkArgs {
    const uint16_t *q, *k, *v;
    const float *a, *b;
    uint16_t *out;
    int T, Hk, Hv, level, level_cap;
    const int32_t *header, *lvl_seg, *seg_start, *seg_len, *seg_src, *seg_chunk0, *emit_off, *emit_pos,
        *seg_state_out;
    const uint16_t *tmat, *pmat;
    const float *state_in;
    float *state_out, *fork_states;
};

constexpr int CONSUMERS = DVS / 16;           // 4 waves, 16 dv columns each
constexpr int PRODUCERS = 4;
constexpr int CHUNK_THREADS = (CONSUMERS + PRODUCERS) * 64;
constexpr int VS = DVS + 8;                   // LDS stride (bf16) of the value / output slice

struct ChunkBuf {
    uint16_t kr[C * KS];     // key rows
    uint16_t qr[C * KS];     // query rows
    uint16_t kt[DK * KTS];   // keys transposed
    uint16_t tm[C * TS];     // T = (I + A)^-1
    uint16_t pm[C * TS];     // P = Gamma o Q K^T
    uint16_t vs[C * VS];     // values of this dv slice, then the chunk's output
    float lsh[C];            // log-decay prefix l_i
    float esh[C];            // write strength b_i
    float gsh[C];            // e^{l_i}
    float dsh[C];            // e^{l_last - l_i}
};

// 16 dk x 4-row fp32 state fragment <-> global [dv][dk] row (4 consecutive dk)
__device__ __forceinline__ void store_state(float *base, int dvc, int G, const f32x4 *st)
{
#pragma unroll
    for (int i = 0; i < DK / 16; ++i)
        *reinterpret_cast<f32x4 *>(base + (size_t)dvc * DK + i * 16 + G * 4) = st[i];
}

// producer `part`: store token rows [16 part, +16) of the output slice of
// chunk `c` (left in B.vs by the consumers), 8 lanes x 16 B per row
__device__ __forceinline__ void flush_out(const ChunkBuf &B, const ChunkArgs &A, int s, int c, int h, int lane,
                                          int part, int dv0)
{
    const int n = min(C, A.seg_len[s] - c * C);
    const size_t t0 = (size_t)A.seg_start[s] + (size_t)c * C;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int idx = j * 64 + lane, row = part * (C / PRODUCERS) + (idx >> 3), c8 = idx & 7;
        if (row < n)
            *reinterpret_cast<uint4 *>(A.out + ((t0 + row) * A.Hv + h) * DV + dv0 + c8 * 8) =
                *reinterpret_cast<const uint4 *>(B.vs + row * VS + c8 * 8);
    }
}

// The transposed keys are stored with the token index XOR-swizzled per key
// dim (a multiple of 4, so groups of 4 tokens stay contiguous for the MFMA
// operand reads): row d holds token t at column t ^ kt_swz(d).  This spreads
// the producers' 2-byte transposed writes over the LDS banks.
__device__ __forceinline__ int kt_swz(int d) { return ((d >> 3) & 15) << 2; }

__device__ __forceinline__ bf16x8 load_kt(const uint16_t *kt, int d, int ks, int G)
{
    const uint16_t *row = kt + d * KTS;
    const int m = kt_swz(d);
    const uint2 lo = *reinterpret_cast<const uint2 *>(row + ((ks * 32 + 4 * G) ^ m));
    const uint2 hi = *reinterpret_cast<const uint2 *>(row + ((ks * 32 + 16 + 4 * G) ^ m));
    return as_bf16x8(make_uint4(lo.x, lo.y, hi.x, hi.y));
}

// producer `part` stages token rows [16 part, 16 part + 16) of chunk `c`
// into `B`.  Loads are coalesced (consecutive lanes read consecutive 16 B of
// a row), and all of them are issued before the first LDS write.
__device__ __forceinline__ void stage_chunk(ChunkBuf &B, const ChunkArgs &A, int s, int c, int h, int g, int lane,
                                            int part, int dv0, int chunk0)
{
    const int len = A.seg_len[s];
    const int n = min(C, len - c * C);
    const size_t t0 = (size_t)A.seg_start[s] + (size_t)c * C;
    const size_t mat = ((size_t)(chunk0 + c) * A.Hv + h) * C * C;
    const int rb = part * (C / PRODUCERS);
    // buffer resources based at this chunk's first row: 32-bit offsets, and
    // the hardware range check returns zeros past the end of each tensor
    const size_t kq_base = (t0 * A.Hk + g) * DK, kq_end = (size_t)A.T * A.Hk * DK;
    const size_t v_base = (t0 * A.Hv + h) * DV + dv0, v_end = (size_t)A.T * A.Hv * DV;
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(A.k + kq_base, (kq_end - kq_base) * 2);
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(A.q + kq_base, (kq_end - kq_base) * 2);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(A.v + v_base, (v_end - v_base) * 2);
    const __amdgpu_buffer_rsrc_t rt = make_rsrc(A.tmat + mat, (size_t)C * C * 2);
    const __amdgpu_buffer_rsrc_t rp = make_rsrc(A.pmat + mat, (size_t)C * C * 2);
    const int kq_row = A.Hk * DK * 2, v_row = A.Hv * DV * 2;   // bytes between tokens
    uint4 kv[4], qv[4], tv[2], pv[2], vv[2];
#pragma unroll
    for (int j = 0; j < 4; ++j) {               // 4 rows x 16 lanes per instruction
        const int idx = j * 64 + lane, row = rb + (idx >> 4), c8 = idx & 15;
        kv[j] = buf_load(rk, row * kq_row + c8 * 16);
        qv[j] = buf_load(rq, row * kq_row + c8 * 16);
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {               // 8 rows x 8 lanes per instruction
        const int idx = j * 64 + lane, row = rb + (idx >> 3), c8 = idx & 7;
        tv[j] = buf_load(rt, row * C * 2 + c8 * 16);
        pv[j] = buf_load(rp, row * C * 2 + c8 * 16);
        vv[j] = buf_load(rv, row * v_row + c8 * 16);
    }
    float a_raw = 1.f, b_raw = 0.f;
    if (part == 0) {
        const int rr = lane < n ? lane : n - 1;
        a_raw = A.a[(t0 + rr) * A.Hv + h];
        b_raw = A.b[(t0 + rr) * A.Hv + h];
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int idx = j * 64 + lane, row = rb + (idx >> 4), c8 = idx & 15;
        if (row >= n) kv[j] = qv[j] = make_uint4(0, 0, 0, 0);
        *reinterpret_cast<uint4 *>(B.kr + row * KS + c8 * 8) = kv[j];
        *reinterpret_cast<uint4 *>(B.qr + row * KS + c8 * 8) = qv[j];
        const uint16_t *k8 = reinterpret_cast<const uint16_t *>(&kv[j]);
        const int col = row ^ kt_swz(c8 * 8);
#pragma unroll
        for (int x = 0; x < 8; ++x) B.kt[(c8 * 8 + x) * KTS + col] = k8[x];
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int idx = j * 64 + lane, row = rb + (idx >> 3), c8 = idx & 7;
        if (row >= n) vv[j] = make_uint4(0, 0, 0, 0);
        *reinterpret_cast<uint4 *>(B.tm + row * TS + c8 * 8) = tv[j];
        *reinterpret_cast<uint4 *>(B.pm + row * TS + c8 * 8) = pv[j];
        *reinterpret_cast<uint4 *>(B.vs + row * VS + c8 * 8) = vv[j];
    }
    if (part == 0) {
        const bool live = lane < n;
        float la = live ? logf(a_raw) : 0.f;
        const float eta = live ? b_raw : 0.f;
        for (int o = 1; o < 64; o <<= 1) {
            const float y = __shfl_up(la, o, 64);
            if (lane >= o) la += y;
        }
        const float last = __shfl(la, C - 1, 64);
        B.lsh[lane] = la;
        B.esh[lane] = eta;
        B.gsh[lane] = __expf(la);
        B.dsh[lane] = __expf(last - la);
    }
}

__global__ void __launch_bounds__(CHUNK_THREADS) k_gdn_chunk(ChunkArgs A)
{
    extern __shared__ __attribute__((aligned(16))) char smem[];
    ChunkBuf *buf = reinterpret_cast<ChunkBuf *>(smem);
    if (A.header[H_STATUS] != FK_OK) return;
    // 1-D grid, work item = (segment rank, v-head, dv slice) with the slice
    // fastest: the live items are the lowest ids, so they spread over all XCDs
    constexpr int NSL = DV / DVS;
    const int rank = blockIdx.x / (A.Hv * NSL);
    if (rank >= A.header[H_LEVEL0 + A.level]) return;
    const int s = A.lvl_seg[A.level * A.level_cap + rank];
    const int h = (blockIdx.x / NSL) % A.Hv, g = h / (A.Hv / A.Hk);
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const bool producer = w >= CONSUMERS;
    const int part = w - CONSUMERS;
    const int G = lane >> 4, c16 = lane & 15;
    const int dv0 = (blockIdx.x % NSL) * DVS;
    const int dvc = dv0 + w * 16 + c16;   // a consumer lane's state column (dv index)
    const size_t SZ = (size_t)DV * DK;
    const int len = A.seg_len[s], chunk0 = A.seg_chunk0[s];
    const int nch = (len + C - 1) / C;

    // The two roles run separate loops with the same number of barriers, so
    // their registers are allocated independently (roles are wave-uniform).
    if (producer) {
        stage_chunk(buf[0], A, s, 0, h, g, lane, part, dv0, chunk0);
        __syncthreads();
        for (int c = 0; c < nch; ++c) {
            if (c + 1 < nch) {
                ChunkBuf &Bn = buf[(c + 1) & 1];
                if (c >= 1) flush_out(Bn, A, s, c - 1, h, lane, part, dv0);
                stage_chunk(Bn, A, s, c + 1, h, g, lane, part, dv0, chunk0);
            }
            __syncthreads();   // chunk c consumed, chunk c+1 staged
        }
        // the last two chunks' outputs have not been flushed yet
        if (nch >= 2) flush_out(buf[(nch - 2) & 1], A, s, nch - 2, h, lane, part, dv0);
        flush_out(buf[(nch - 1) & 1], A, s, nch - 1, h, lane, part, dv0);
        return;
    }

    f32x4 st[DK / 16];
    int e = A.emit_off[s];
    const int e_end = A.emit_off[s + 1];
    {
        const int src = A.seg_src[s];
        const float *S0 = src == -1 ? nullptr
                                    : (src >= 0 ? A.fork_states + ((size_t)src * A.Hv + h) * SZ
                                                : A.state_in + ((size_t)(-2 - src) * A.Hv + h) * SZ);
#pragma unroll
        for (int i = 0; i < DK / 16; ++i)
            st[i] = S0 ? *reinterpret_cast<const f32x4 *>(S0 + (size_t)dvc * DK + i * 16 + G * 4)
                       : f32x4{0.f, 0.f, 0.f, 0.f};
        while (e < e_end && A.emit_pos[e] == 0) {
            store_state(A.fork_states + ((size_t)e * A.Hv + h) * SZ, dvc, G, st);
            ++e;
        }
    }
    __syncthreads();
    for (int c = 0; c < nch; ++c) {
        ChunkBuf &B = buf[c & 1];
        const int n = min(C, len - c * C);
        // X = K S0^T, Y = Q S0^T for this wave's 16 dv columns
        f32x4 xa[C / 16], ya[C / 16];
#pragma unroll
        for (int mt = 0; mt < C / 16; ++mt) xa[mt] = ya[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks2 = 0; ks2 < DK / 32; ++ks2) {
            const bf16x8 sb = pack(st[2 * ks2], st[2 * ks2 + 1]);
#pragma unroll
            for (int mt = 0; mt < C / 16; ++mt) {
                xa[mt] = mfma(load_perm(B.kr + (mt * 16 + c16) * KS, ks2, G), sb, xa[mt]);
                ya[mt] = mfma(load_perm(B.qr + (mt * 16 + c16) * KS, ks2, G), sb, ya[mt]);
            }
        }
        __builtin_amdgcn_sched_barrier(0);   // bound the operand loads kept in flight
        // R = diag(b) (V - diag(e^l) X);  U = T R
#pragma unroll
        for (int mt = 0; mt < C / 16; ++mt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int i = mt * 16 + G * 4 + r;
                const float vv = bf16_to_f32(B.vs[i * VS + w * 16 + c16]);
                xa[mt][r] = B.esh[i] * (vv - B.gsh[i] * xa[mt][r]);
            }
        const bf16x8 rb0 = pack(xa[0], xa[1]), rb1 = pack(xa[2], xa[3]);
        f32x4 ua[C / 16];
#pragma unroll
        for (int mt = 0; mt < C / 16; ++mt) {
            ua[mt] = mfma(load_perm(B.tm + (mt * 16 + c16) * TS, 0, G), rb0, f32x4{0.f, 0.f, 0.f, 0.f});
            ua[mt] = mfma(load_perm(B.tm + (mt * 16 + c16) * TS, 1, G), rb1, ua[mt]);
        }
        __builtin_amdgcn_sched_barrier(0);
        // O = diag(e^l) Y + P U  -> left in the value buffer for the producers
        const bf16x8 ub0 = pack(ua[0], ua[1]), ub1 = pack(ua[2], ua[3]);
#pragma unroll
        for (int mt = 0; mt < C / 16; ++mt) {
            f32x4 oa;
#pragma unroll
            for (int r = 0; r < 4; ++r) oa[r] = B.gsh[mt * 16 + G * 4 + r] * ya[mt][r];
            oa = mfma(load_perm(B.pm + (mt * 16 + c16) * TS, 0, G), ub0, oa);
            if (mt >= 2) oa = mfma(load_perm(B.pm + (mt * 16 + c16) * TS, 1, G), ub1, oa);
#pragma unroll
            for (int r = 0; r < 4; ++r)
                B.vs[(mt * 16 + G * 4 + r) * VS + w * 16 + c16] = __builtin_bit_cast(uint16_t, (__bf16)oa[r]);
        }
        // fork points strictly inside this chunk: state after `off` tokens
        while (e < e_end && A.emit_pos[e] < c * C + n) {
            const int off = A.emit_pos[e] - c * C;   // 1 .. n-1
            const float lr = B.lsh[off - 1];
            f32x4 u0[C / 16];
#pragma unroll
            for (int mt = 0; mt < C / 16; ++mt)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int j = mt * 16 + G * 4 + r;
                    u0[mt][r] = j < off ? __expf(lr - B.lsh[j]) * ua[mt][r] : 0.f;
                }
            const bf16x8 eb0 = pack(u0[0], u0[1]), eb1 = pack(u0[2], u0[3]);
            const float gr = __expf(lr);
            f32x4 tmp[DK / 16];
#pragma unroll
            for (int i = 0; i < DK / 16; ++i) {
                tmp[i] = mfma(load_kt(B.kt, i * 16 + c16, 0, G), eb0, st[i] * gr);
                tmp[i] = mfma(load_kt(B.kt, i * 16 + c16, 1, G), eb1, tmp[i]);
            }
            store_state(A.fork_states + ((size_t)e * A.Hv + h) * SZ, dvc, G, tmp);
            ++e;
        }
        __builtin_amdgcn_sched_barrier(0);
        // S^T <- e^{l_last} S^T + K^T diag(e^{l_last - l}) U
#pragma unroll
        for (int mt = 0; mt < C / 16; ++mt)
#pragma unroll
            for (int r = 0; r < 4; ++r) ua[mt][r] *= B.dsh[mt * 16 + G * 4 + r];
        const bf16x8 wb0 = pack(ua[0], ua[1]), wb1 = pack(ua[2], ua[3]);
        const float gl = B.gsh[C - 1];
#pragma unroll
        for (int i = 0; i < DK / 16; ++i) {
            st[i] = mfma(load_kt(B.kt, i * 16 + c16, 0, G), wb0, st[i] * gl);
            st[i] = mfma(load_kt(B.kt, i * 16 + c16, 1, G), wb1, st[i]);
        }
        // a fork point at the end of this chunk
        while (e < e_end && A.emit_pos[e] == c * C + n) {
            store_state(A.fork_states + ((size_t)e * A.Hv + h) * SZ, dvc, G, st);
            ++e;
        }
        __syncthreads();   // chunk c consumed, chunk c+1 staged
    }
    const int so = A.seg_state_out[s];
    if (so >= 0) store_state(A.state_out + ((size_t)so * A.Hv + h) * SZ, dvc, G, st);
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
                                          const_cast<uint16_t *>(ws_at<uint16_t>(ws, L.pmat)));
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
    A.a = a;
    A.b = b;
    A.out = (uint16_t *)out;
    A.T = meta->T;
    A.Hk = Hk;
    A.Hv = Hv;
    A.level = level;
    A.level_cap = meta->level_cap;
    A.header = ws_at<int32_t>(ws, L.header);
    A.lvl_seg = ws_at<int32_t>(ws, L.lvl_seg);
    A.seg_start = ws_at<int32_t>(ws, L.seg_start);
    A.seg_len = ws_at<int32_t>(ws, L.seg_len);
    A.seg_src = ws_at<int32_t>(ws, L.seg_src);
    A.seg_chunk0 = ws_at<int32_t>(ws, L.seg_chunk0);
    A.emit_off = ws_at<int32_t>(ws, L.emit_off);
    A.emit_pos = ws_at<int32_t>(ws, L.emit_pos);
    A.seg_state_out = meta->seg_state_out;
    A.tmat = ws_at<uint16_t>(ws, L.tmat);
    A.pmat = ws_at<uint16_t>(ws, L.pmat);
    A.state_in = state_in;
    A.state_out = state_out;
    A.fork_states = fork_states;
    dim3 grid((unsigned)((int64_t)meta->level_cap * Hv * (gdnk::DV / gdnk::DVS)));
    static bool configured = false;
    const size_t lds = 2 * sizeof(gdnk::ChunkBuf);
    if (!configured) {
        FK_HIP(hipFuncSetAttribute((const void *)gdnk::k_gdn_chunk, hipFuncAttributeMaxDynamicSharedMemorySize,
                                   (int)lds));
        configured = true;
    }
    gdnk::k_gdn_chunk<<<grid, gdnk::CHUNK_THREADS, lds, st>>>(A);
    return launch_status();
}
