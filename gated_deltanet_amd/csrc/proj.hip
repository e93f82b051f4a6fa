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
// Tiles: waves compute 32-row x 32-feature products of y^T = w x^T with
// v_mfma_f32_32x32x16_bf16 (A = rows of w, B = rows of x), k in steps
// through a ring of LDS stages (the w and x tiles of one step) filled by
// direct global->LDS loads (global_load_lds_dwordx4: each lane's 16 bytes
// land at M0 + 16 * lane) ahead of use, so no register holds a tile in
// flight.  When N is a multiple of 256 a work-group of eight waves computes a
// 256-feature x 256-row block (a wave 128 x 64: four w and two x fragments
// per 16-wide k-slice for eight products), k in steps of 64 through two
// 64 KB stages (one step ahead; one work-group a CU), its two groups of four
// waves taking turns: one multiplies while the other reads its next operands
// (k_proj_pp); otherwise four waves compute 128 x 128 (a wave 64 x 64), k in
// steps of 32 through three 16 KB stages (two steps ahead; three work-groups
// a CU).  LDS rows hold one
// step's k (64 or 128 bytes), their 16-byte units XOR-swizzled by bits 2-3
// (or 1-3) of the row, so the operand reads (16 lanes: 16 rows, one unit)
// are free of bank conflicts; the lane that fills unit u of row r loads the
// unit that belongs there.  A lane's accumulator holds 4 consecutive output features of one
// row: 8-byte stores.
// Tiles are dealt to the eight XCDs in contiguous ranges of row blocks, and
// within an XCD in groups of GM row blocks (row block fastest), so blocks
// that run together share their x and w tiles in that XCD's L2.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "fk_common.h"

namespace fk {
namespace proj {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int BM = 128, BN = 128;
constexpr int K_MULT = 64;      // K must be a multiple of this (the documented contract)
constexpr int WIDE_WM = 4;      // waves along the rows of the 256-feature blocks
constexpr int GM = 8;           // row blocks per group within an XCD
constexpr int XCDS = 8;
// NF: 32-feature fragments per wave (2: 128 x 128 blocks on four waves, three
// work-groups a CU; 4 with WM = 4: 256 x 256 blocks on eight waves, one
// work-group a CU and half the LDS operand bytes per product, used when N is
// a multiple of 256)
template <int NF, int WM, int BK_ = 32>   // WM: waves along the rows (64 rows each)
struct Shape {
    static constexpr int BK = BK_;                 // k per step
    static constexpr int RN = BK == 32 ? 3 : 2;    // ring stages (loads RN - 1 steps ahead)
    static constexpr int UNITS = BK / 8;           // 16-byte units per LDS row
    static constexpr int RPL = 64 / UNITS;         // rows per 1 KB load
    static constexpr int BNW = 64 * NF;            // features per work-group
    static constexpr int BMW = 64 * WM;            // rows per work-group
    static constexpr int NT = 128 * WM;            // threads (2 x WM waves)
    static constexpr int WT = BNW * BK, XT = BMW * BK;   // bf16 elements of the w / x tiles
    static constexpr int STAGE = WT + XT;
    static constexpr int OCC = NF == 2 ? 3 : (WM == 2 ? 2 : 1);   // work-groups a CU
    // rows of UNITS 16-byte units, XOR-swizzled so that a 16-lane read of
    // one unit in 16 consecutive rows meets 16 distinct bank groups
    static __device__ __forceinline__ int swz_unit(int row, int unit)
    {
        return BK == 32 ? unit ^ ((row >> 2) & 3) : unit ^ ((row >> 1) & 7);
    }
    static __device__ __forceinline__ int swz(int row, int unit) { return row * BK + (swz_unit(row, unit) << 3); }
};

// one 16-byte direct global->LDS load per lane: global address g (per lane),
// LDS address m0 + 16 * lane
__device__ __forceinline__ void lds_dma16(const uint16_t *g, uint32_t m0)
{
    asm volatile("global_load_lds_dwordx4 %0, off" ::"v"(g), "{m0}"(m0) : "memory");
}

template <int N>
__device__ __forceinline__ void wait_barrier()
{
    asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(N) : "memory");
}

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

template <int NF, int WM, int BK_>
__global__ void __launch_bounds__((Shape<NF, WM, BK_>::NT), (Shape<NF, WM, BK_>::OCC)) k_proj_bf16(Args A)
{
    using SH = Shape<NF, WM, BK_>;
    constexpr int BK = SH::BK, RNG = SH::RN, RPL = SH::RPL, UNITS = SH::UNITS;
    __shared__ __attribute__((aligned(1024))) uint16_t ring[RNG * SH::STAGE];
    int mb, nb;
    if (!tile_of(A, blockIdx.x, mb, nb)) return;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int wn = w & 1, wm = w >> 1, half = lane >> 5, c32 = lane & 31;
    const int m0 = mb * SH::BMW, n0 = nb * SH::BNW;
    constexpr int WF = SH::BNW / RPL / (2 * WM);   // w loads a wave (RPL rows each)
    constexpr int XL = 32 / RPL;                   // x loads a wave (32 rows)

    // loads, 16 rows (1 KB) an instruction, lane l: row r0 + l / 4, LDS unit
    // l % 4.  Wave w fills w rows 16 WF w .. +16 WF and x rows 32 w .. +32.
    const uint16_t *wsrc[WF], *xsrc[XL];
#pragma unroll
    for (int i = 0; i < WF; ++i) {
        const int r = RPL * WF * w + RPL * i + lane / UNITS, u = SH::swz_unit(r, lane % UNITS);
        wsrc[i] = A.w + (size_t)(n0 + r) * A.K + u * 8;
    }
#pragma unroll
    for (int i = 0; i < XL; ++i) {
        const int r = 32 * w + RPL * i + lane / UNITS, u = SH::swz_unit(r, lane % UNITS);
        // a row past M, or an unused index entry, reads row 0 of x: that
        // output row is never stored, and no other row uses it
        const int m = m0 + r;
        int src = -1;
        if (m < A.M) src = A.rows ? A.rows[m] : m;
        if (src < 0 || src >= A.Mx) src = 0;
        xsrc[i] = A.x + (size_t)src * A.K + u * 8;
    }
    const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint16_t *)ring;
    const uint32_t wq = __builtin_amdgcn_readfirstlane(lds0 + w * RPL * WF * BK * 2);
    const uint32_t xq = __builtin_amdgcn_readfirstlane(lds0 + SH::WT * 2 + w * 32 * BK * 2);
    // stage s of k-step kt: w tile, then x tile (WF + 2 loads a wave)
    auto issue = [&](int kt, int s) {
        const int k0 = kt * BK;
        const uint32_t so = s * (SH::STAGE * 2);
#pragma unroll
        for (int i = 0; i < WF; ++i) lds_dma16(wsrc[i] + k0, wq + so + i * 1024);
#pragma unroll
        for (int i = 0; i < XL; ++i) lds_dma16(xsrc[i] + k0, xq + so + i * 1024);
    };

    f32x16 acc[NF][2];
#pragma unroll
    for (int i = 0; i < NF; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};

    const int nk = A.K / BK;   // >= 1
#pragma unroll
    for (int p = 0; p < RNG - 1; ++p)
        if (p < nk) issue(p, p);
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): the index reads and the first stages
    // k-step kt in stage S (= kt mod RN); the loop is unrolled over the
    // stages so that every LDS offset is an immediate
    auto kstep = [&](auto SC, int kt) {
        constexpr int S = decltype(SC)::value, SN = (S + RNG - 1) % RNG;
        // step kt landed in every wave; every wave is done with step kt-1,
        // whose stage step kt+RN-1 now takes (the loads complete in order)
        if (RNG == 3 && kt + 1 < nk)
            wait_barrier<WF + XL>();
        else
            wait_barrier<0>();
        const uint16_t *lw = ring + S * SH::STAGE, *lx = lw + SH::WT;
#pragma unroll
        for (int ks = 0; ks < BK / 16; ++ks) {
            const int unit = ks * 2 + half;
            bf16x8 a[NF], b[2];
#pragma unroll
            for (int i = 0; i < NF; ++i)
                a[i] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4 *>(
                                                      &lw[SH::swz(wn * 32 * NF + i * 32 + c32, unit)]));
#pragma unroll
            for (int j = 0; j < 2; ++j)
                b[j] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4 *>(
                                                      &lx[SH::swz(wm * 64 + j * 32 + c32, unit)]));
#pragma unroll
            for (int i = 0; i < NF; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
            // step kt+RN-1's loads go out once the first products are issued
            if (ks == 0 && kt + RNG - 1 < nk) issue(kt + RNG - 1, SN);
        }
    };
    int kt = 0;
    if constexpr (RNG == 3) {
        for (; kt + 3 <= nk; kt += 3) {
            kstep(std::integral_constant<int, 0>(), kt);
            kstep(std::integral_constant<int, 1>(), kt + 1);
            kstep(std::integral_constant<int, 2>(), kt + 2);
        }
        if (kt < nk) kstep(std::integral_constant<int, 0>(), kt);
        if (kt + 1 < nk) kstep(std::integral_constant<int, 1>(), kt + 1);
    } else {
        for (; kt + 2 <= nk; kt += 2) {
            kstep(std::integral_constant<int, 0>(), kt);
            kstep(std::integral_constant<int, 1>(), kt + 1);
        }
        if (kt < nk) kstep(std::integral_constant<int, 0>(), kt);
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
        uint16_t *yrow = A.y + (size_t)m * A.N + n0 + wn * 32 * NF;
#pragma unroll
        for (int i = 0; i < NF; ++i)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                uint2 p;
                p.x = (uint32_t)f32_to_bf16(acc[i][j][4 * g]) | ((uint32_t)f32_to_bf16(acc[i][j][4 * g + 1]) << 16);
                p.y = (uint32_t)f32_to_bf16(acc[i][j][4 * g + 2]) | ((uint32_t)f32_to_bf16(acc[i][j][4 * g + 3]) << 16);
                *reinterpret_cast<uint2 *>(yrow + i * 32 + 8 * g + 4 * half) = p;
            }
    }
}

// Wide blocks in two wave groups that take turns (group 0: waves 0-3, group
// 1: waves 4-7, one wave of each on every SIMD).  A phase covers half a
// k-step (two 16-wide k-slices): group 0 reads half j's operands from LDS
// into registers in phase 2j and runs its 16 products in phase 2j+1; group 1
// does the same one phase later; a barrier ends every phase.  Each element
// still sums its 16-wide k-slices in ascending order in one wave.  Stage
// (s mod 2) holds step s (halves 2s and 2s+1), read last in phase 4s+3.  In
// phase 4t both groups issue step t+1's loads into the stage step t-1 left
// (group 0 while reading half 2t, group 1 while multiplying half 2t-1), and
// each wave waits for its loads before the barrier that ends phase 4t+3
// (group 0 after multiplying half 2t+1, group 1 after reading it), so step
// t+1 is in LDS when group 0 reads it in phase 4t+4.  Every wave meets the
// same number of barriers: group 1's extra one at the start is matched by
// group 0's after its stores.
__global__ void __launch_bounds__((Shape<4, WIDE_WM, 64>::NT), 1) k_proj_pp(Args A)
{
    using SH = Shape<4, WIDE_WM, 64>;
    static_assert(SH::NT == 512, "two groups of four waves");
    constexpr int BK = SH::BK, RPL = SH::RPL, UNITS = SH::UNITS;
    __shared__ __attribute__((aligned(1024))) uint16_t ring[2 * SH::STAGE];
    int mb, nb;
    if (!tile_of(A, blockIdx.x, mb, nb)) return;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int wn = w & 1, wm = w >> 1, half = lane >> 5, c32 = lane & 31;
    const int grp = __builtin_amdgcn_readfirstlane(tid >> 8);
    const int m0 = mb * SH::BMW, n0 = nb * SH::BNW;
    constexpr int WF = SH::BNW / RPL / 8;   // w loads a wave (RPL rows each)
    constexpr int XL = 32 / RPL;            // x loads a wave (32 rows)
    const uint16_t *wsrc[WF], *xsrc[XL];
#pragma unroll
    for (int i = 0; i < WF; ++i) {
        const int r = RPL * WF * w + RPL * i + lane / UNITS, u = SH::swz_unit(r, lane % UNITS);
        wsrc[i] = A.w + (size_t)(n0 + r) * A.K + u * 8;
    }
#pragma unroll
    for (int i = 0; i < XL; ++i) {
        const int r = 32 * w + RPL * i + lane / UNITS, u = SH::swz_unit(r, lane % UNITS);
        const int m = m0 + r;
        int src = -1;
        if (m < A.M) src = A.rows ? A.rows[m] : m;
        if (src < 0 || src >= A.Mx) src = 0;
        xsrc[i] = A.x + (size_t)src * A.K + u * 8;
    }
    const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint16_t *)ring;
    const uint32_t wq = __builtin_amdgcn_readfirstlane(lds0 + w * RPL * WF * BK * 2);
    const uint32_t xq = __builtin_amdgcn_readfirstlane(lds0 + SH::WT * 2 + w * 32 * BK * 2);
    auto issue = [&](int kt, int s) {
        const int k0 = kt * BK;
        const uint32_t so = s * (SH::STAGE * 2);
#pragma unroll
        for (int i = 0; i < WF; ++i) lds_dma16(wsrc[i] + k0, wq + so + i * 1024);
#pragma unroll
        for (int i = 0; i < XL; ++i) lds_dma16(xsrc[i] + k0, xq + so + i * 1024);
    };
    f32x16 acc[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};
    const int nk = A.K / BK;   // >= 1
    issue(0, 0);
    if (nk > 1) {
        issue(1, 1);
        wait_barrier<WF + XL>();
    } else {
        wait_barrier<0>();
    }
    if (grp) {
        __builtin_amdgcn_sched_barrier(0);
        asm volatile("s_barrier" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
    }
    // a phase covers half a step (two 16-wide k-slices): 48 operand registers
    bf16x8 a[2][4], b[2][2];
    auto read_ops = [&](auto SC, auto HC) {
        constexpr int S = decltype(SC)::value, H = decltype(HC)::value;
        const uint16_t *lw = ring + S * SH::STAGE, *lx = lw + SH::WT;
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            const int unit = (2 * H + kk) * 2 + half;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                a[kk][i] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4 *>(
                                                          &lw[SH::swz(wn * 128 + i * 32 + c32, unit)]));
#pragma unroll
            for (int j = 0; j < 2; ++j)
                b[kk][j] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4 *>(
                                                          &lx[SH::swz(wm * 64 + j * 32 + c32, unit)]));
        }
    };
    // the products of one phase; `mid` runs after the first k-slice's
    auto products = [&](auto mid) {
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[kk][i], b[kk][j], acc[i][j], 0, 0, 0);
            if (kk == 0) mid();
        }
    };
    auto nothing = []() {};
#define FK_PP_BAR(text)                           \
    do {                                          \
        __builtin_amdgcn_sched_barrier(0);        \
        asm volatile(text ::: "memory");          \
        __builtin_amdgcn_sched_barrier(0);        \
    } while (0)
    // group 0, half H of step s (stage S): read it (the first half also
    // issues step s+1's loads), then multiply; step s+1 is waited for at the
    // end of the second half
    auto half0 = [&](auto SC, auto HC, int s) {
        constexpr int S = decltype(SC)::value, H = decltype(HC)::value;
        read_ops(SC, HC);
        if (H == 0 && s >= 1 && s + 1 < nk) issue(s + 1, 1 - S);
        FK_PP_BAR("s_waitcnt lgkmcnt(0)\n\ts_barrier");
        products(nothing);
        if (H == 1)
            FK_PP_BAR("s_waitcnt vmcnt(0)\n\ts_barrier");
        else
            FK_PP_BAR("s_barrier");
    };
    // group 1, half H of step s (stage S): read it (step s+1's loads, issued
    // in the previous phase, are waited for at the end of the second half),
    // then multiply; the second half issues step s+2's loads into stage S
    auto half1 = [&](auto SC, auto HC, int s) {
        constexpr int S = decltype(SC)::value, H = decltype(HC)::value;
        read_ops(SC, HC);
        if (H == 1)
            FK_PP_BAR("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier");
        else
            FK_PP_BAR("s_waitcnt lgkmcnt(0)\n\ts_barrier");
        products([&]() {
            if (H == 1 && s + 2 < nk) issue(s + 2, S);
        });
        FK_PP_BAR("s_barrier");
    };
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    int kt = 0;
    if (grp == 0) {
        for (; kt + 2 <= nk; kt += 2) {
            half0(I0(), I0(), kt);
            half0(I0(), I1(), kt);
            half0(I1(), I0(), kt + 1);
            half0(I1(), I1(), kt + 1);
        }
        if (kt < nk) {
            half0(I0(), I0(), kt);
            half0(I0(), I1(), kt);
        }
    } else {
        for (; kt + 2 <= nk; kt += 2) {
            half1(I0(), I0(), kt);
            half1(I0(), I1(), kt);
            half1(I1(), I0(), kt + 1);
            half1(I1(), I1(), kt + 1);
        }
        if (kt < nk) {
            half1(I0(), I0(), kt);
            half1(I0(), I1(), kt);
        }
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int m = m0 + wm * 64 + j * 32 + c32;
        if (m >= A.M) continue;
        if (A.rows) {
            const int src = A.rows[m];
            if (src < 0 || src >= A.Mx) continue;
        }
        uint16_t *yrow = A.y + (size_t)m * A.N + n0 + wn * 128;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                uint2 p;
                p.x = (uint32_t)f32_to_bf16(acc[i][j][4 * g]) | ((uint32_t)f32_to_bf16(acc[i][j][4 * g + 1]) << 16);
                p.y = (uint32_t)f32_to_bf16(acc[i][j][4 * g + 2]) | ((uint32_t)f32_to_bf16(acc[i][j][4 * g + 3]) << 16);
                *reinterpret_cast<uint2 *>(yrow + i * 32 + 8 * g + 4 * half) = p;
            }
    }
    if (grp == 0) FK_PP_BAR("s_barrier");
#undef FK_PP_BAR
}

}  // namespace proj
}  // namespace fk

using namespace fk;

extern "C" int fk_proj_gemm(const void *x, int32_t Mx, const int32_t *rows, int32_t M, int32_t K, const void *w,
                            int32_t N, int dtype, void *y, fk_stream_t stream)
{
    if (dtype != FK_BF16) return FK_E_UNSUPPORTED;
    if (M < 0 || Mx < 0 || K <= 0 || N <= 0) return FK_E_INVALID_ARG;
    if (K % proj::K_MULT || N % proj::BN) return FK_E_UNSUPPORTED;
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
    const bool wide = N % 256 == 0;
    using S2 = proj::Shape<2, 2, 32>;
    using S4 = proj::Shape<4, proj::WIDE_WM, 64>;
    A.mt = (M + (wide ? S4::BMW : S2::BMW) - 1) / (wide ? S4::BMW : S2::BMW);
    A.nt = N / (wide ? S4::BNW : S2::BNW);
    const int m_per = (A.mt + proj::XCDS - 1) / proj::XCDS;
    const int64_t blocks = (int64_t)proj::XCDS * m_per * A.nt;
    if (blocks > INT32_MAX) return FK_E_UNSUPPORTED;
    if (wide)
        proj::k_proj_pp<<<dim3((unsigned)blocks), S4::NT, 0, (hipStream_t)stream>>>(A);
    else
        proj::k_proj_bf16<2, 2, 32><<<dim3((unsigned)blocks), S2::NT, 0, (hipStream_t)stream>>>(A);
    return launch_status();
}
