// proj.hip -- the projection either side of the token mixers, on bf16 MFMA
// (gfx950), with a fixed reduction order.
//
// Flide section 3.5: a batch-invariant engine makes every matrix product sum
// each output element in one order whatever the number of rows, so a row's
// bits never depend on the batch it runs in.  Section 3.3.3: in the last
// layer the products run only at the rows of the readout index buffer.
//
//   y[m, n] = sum_k x[r(m), k] w[n, k],   r(m) = rows[m] (or m)
//
// Every output element is accumulated in fp32 over k in 16-wide MFMA steps,
// k ascending, always by one work-group (no split of k, no choice that depends
// on M), so its bits depend only on its own row of x and column of w.
//
// Tiles: a work-group of 4 waves computes a 128 (n) x 128 (m) block of y^T
// = w x^T with v_mfma_f32_32x32x16_bf16 (A = rows of w, B = rows of x; each
// wave a 64 x 64 quarter, 2 x 2 products), k in steps of 64 through a
// double-buffered LDS tile (32 KB per stage), the next step's global loads in
// registers under the current step's products.  A lane's accumulator then
// holds 4 consecutive output features of one row: 8-byte stores.  LDS rows
// are 128 bytes, their 16-byte units XOR-swizzled by bits 1-3 of the row, so
// the operand reads (16 lanes: 16 rows, one unit) and the row writes (8 lanes:
// one row) are free of bank conflicts.  Tiles are dealt to the eight XCDs in
// contiguous ranges of row blocks, and within an XCD in groups of GM row
// blocks (row block fastest), so blocks that run together share their x and
// w tiles in that XCD's L2.
#include <hip/hip_runtime.h>

#include "fk_common.h"

namespace fk {
namespace proj {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int BM = 128, BN = 128, BK = 64;
constexpr int THREADS = 256;
constexpr int TILE = BM * BK;   // bf16 elements of one operand tile in LDS
constexpr int GM = 8;           // row blocks per group within an XCD
constexpr int XCDS = 8;

__device__ __forceinline__ int swz(int row, int unit) { return row * BK + ((unit ^ ((row >> 1) & 7)) << 3); }

struct Args {
    const uint16_t *x, *w;
    const int32_t *rows;
    uint16_t *y;
    int M, Mx, K, N;
    int mt, nt;   // row blocks, feature blocks
};

// the tile of block-id `b` (dealt round-robin to the XCDs): XCD b % 8 owns row
// blocks [x m_per, (x+1) m_per); its j-th tile is (row block, feature block)
// in groups of GM row blocks, row block fastest.  Returns false when the XCD's
// range holds fewer tiles than j.
__device__ __forceinline__ bool tile_of(const Args &A, int b, int &mb, int &nb)
{
    const int x = b % XCDS, j = b / XCDS;
    const int m_per = (A.mt + XCDS - 1) / XCDS;
    const int m0 = x * m_per, m1 = min(A.mt, m0 + m_per);
    if (m0 >= m1) return false;
    const int span = m1 - m0;
    if (j >= span * A.nt) return false;
    const int grp = j / (GM * A.nt), in = j % (GM * A.nt);
    const int g0 = grp * GM, gsz = min(GM, span - g0);
    mb = m0 + g0 + in % gsz;
    nb = in / gsz;
    return true;
}

__global__ void __launch_bounds__(THREADS, 2) k_proj_bf16(Args A)
{
    __shared__ __attribute__((aligned(16))) uint16_t lw[2][TILE];
    __shared__ __attribute__((aligned(16))) uint16_t lx[2][TILE];
    int mb, nb;
    if (!tile_of(A, blockIdx.x, mb, nb)) return;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int wn = w & 1, wm = w >> 1, half = lane >> 5, c32 = lane & 31;
    const int m0 = mb * BM, n0 = nb * BN;

    // loader: thread t moves unit t % 8 of rows t / 8 + 32 i (i < 4) of both tiles
    const int lunit = tid & 7, lrow = tid >> 3;
    const uint16_t *wsrc[4];
    const uint16_t *xsrc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = lrow + 32 * i;
        wsrc[i] = A.w + (size_t)(n0 + r) * A.K + lunit * 8;
        const int m = m0 + r;
        int src = -1;
        if (m < A.M) src = A.rows ? A.rows[m] : m;
        xsrc[i] = (src >= 0 && src < A.Mx) ? A.x + (size_t)src * A.K + lunit * 8 : nullptr;
    }
    uint4 rw[4], rx[4];
    auto load = [&](int k0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            rw[i] = *reinterpret_cast<const uint4 *>(wsrc[i] + k0);
            rx[i] = xsrc[i] ? *reinterpret_cast<const uint4 *>(xsrc[i] + k0) : make_uint4(0, 0, 0, 0);
        }
    };
    auto store = [&](int buf) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int off = swz(lrow + 32 * i, lunit);
            *reinterpret_cast<uint4 *>(&lw[buf][off]) = rw[i];
            *reinterpret_cast<uint4 *>(&lx[buf][off]) = rx[i];
        }
    };

    f32x16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};

    const int nk = A.K / BK;
    load(0);
    store(0);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        const int buf = kt & 1;
        const bool more = kt + 1 < nk;
        if (more) load((kt + 1) * BK);
#pragma unroll
        for (int ks = 0; ks < BK / 16; ++ks) {
            const int unit = ks * 2 + half;
            bf16x8 a[2], b[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                a[i] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4 *>(
                                                      &lw[buf][swz(wn * 64 + i * 32 + c32, unit)]));
                b[i] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4 *>(
                                                      &lx[buf][swz(wm * 64 + i * 32 + c32, unit)]));
            }
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
        }
        if (more) store(buf ^ 1);
        __syncthreads();
    }
    // y^T tile: lane holds row m = .. + c32 and features 8 (r / 4) + 4 half + r % 4
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int m = m0 + wm * 64 + j * 32 + c32;
        if (m >= A.M) continue;
        if (A.rows) {
            const int src = A.rows[m];
            if (src < 0 || src >= A.Mx) continue;
        }
        uint16_t *yrow = A.y + (size_t)m * A.N + n0 + wn * 64;
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                uint2 p;
                p.x = (uint32_t)f32_to_bf16(acc[i][j][4 * g]) | ((uint32_t)f32_to_bf16(acc[i][j][4 * g + 1]) << 16);
                p.y = (uint32_t)f32_to_bf16(acc[i][j][4 * g + 2]) | ((uint32_t)f32_to_bf16(acc[i][j][4 * g + 3]) << 16);
                *reinterpret_cast<uint2 *>(yrow + i * 32 + 8 * g + 4 * half) = p;
            }
    }
}

}  // namespace proj
}  // namespace fk

using namespace fk;

extern "C" int fk_proj_gemm(const void *x, int32_t Mx, const int32_t *rows, int32_t M, int32_t K, const void *w,
                            int32_t N, int dtype, void *y, fk_stream_t stream)
{
    if (dtype != FK_BF16) return FK_E_UNSUPPORTED;
    if (M < 0 || Mx < 0 || K <= 0 || N <= 0) return FK_E_INVALID_ARG;
    if (K % proj::BK || N % proj::BN) return FK_E_UNSUPPORTED;
    if (!rows && M > Mx) return FK_E_INVALID_ARG;
    if (M == 0) return FK_OK;
    if (!x || !w || !y) return FK_E_INVALID_ARG;
    proj::Args A;
    A.x = (const uint16_t *)x;
    A.w = (const uint16_t *)w;
    A.rows = rows;
    A.y = (uint16_t *)y;
    A.M = M;
    A.Mx = Mx;
    A.K = K;
    A.N = N;
    A.mt = (M + proj::BM - 1) / proj::BM;
    A.nt = N / proj::BN;
    const int m_per = (A.mt + proj::XCDS - 1) / proj::XCDS;
    const int64_t blocks = (int64_t)proj::XCDS * m_per * A.nt;
    if (blocks > INT32_MAX) return FK_E_UNSUPPORTED;
    proj::k_proj_bf16<<<dim3((unsigned)blocks), proj::THREADS, 0, (hipStream_t)stream>>>(A);
    return launch_status();
}
