// kv_append.hip -- write the stream's keys and values into the paged pool.
// ForkServe item 1: a write allocates the writer's own pages only, and a
// child reads its ancestors' pages through their page lists (an alias), never
// through a copy.  Flide section 3.4: cached keys/values precede the new ones
// in each state's history buffer -- here, the cached segment's pages.
//
// One block per (16-token tile = one page, kv head).  Keys keep their row
// layout [slot][d]; values are stored transposed inside the page, [d][slot],
// so the attention kernel's value operand reads keys contiguously.  Slots
// after a segment's last token are zero-filled.  bf16 at d = 128 (the
// attention kernel's shape) has a 16-byte-access kernel of its own.
#include <hip/hip_runtime.h>

#include "fk_common.h"

namespace fk {

template <typename E>
__global__ void __launch_bounds__(256) k_kv_append(const E *__restrict__ k, const E *__restrict__ v, int Hkv,
                                                   int d, const int32_t *__restrict__ header,
                                                   const int32_t *__restrict__ tile_seg,
                                                   const int32_t *__restrict__ tile_row0,
                                                   const int32_t *__restrict__ seg_start,
                                                   const int32_t *__restrict__ seg_len,
                                                   const int32_t *__restrict__ page_off,
                                                   const int32_t *__restrict__ pages, E *__restrict__ kp,
                                                   E *__restrict__ vp)
{
    if (header[H_STATUS] != FK_OK) return;
    const int tile = blockIdx.x, h = blockIdx.y;
    if (tile >= header[H_NTILES]) return;
    const int s = tile_seg[tile], row0 = tile_row0[tile];
    const int count = min(FK_TILE_TOKENS, seg_len[s] - row0);
    const int page = pages[page_off[s] + row0 / FK_TILE_TOKENS];
    const int t0 = seg_start[s] + row0;
    const size_t page_base = ((size_t)page * Hkv + h) * (size_t)FK_TILE_TOKENS * d;
    const int n = FK_TILE_TOKENS * d;
    for (int e = threadIdx.x; e < n; e += blockDim.x) {
        // keys: e -> (slot, dim), coalesced on both sides
        const int r = e / d, x = e % d;
        E kv = E(0);
        if (r < count) kv = k[((size_t)(t0 + r) * Hkv + h) * d + x];
        kp[page_base + e] = kv;
        // values: e -> (dim, slot), coalesced on the page side
        const int xv = e / FK_TILE_TOKENS, rv = e % FK_TILE_TOKENS;
        E vv = E(0);
        if (rv < count) vv = v[((size_t)(t0 + rv) * Hkv + h) * d + xv];
        vp[page_base + e] = vv;
    }
}

// bf16, d = 128: 16-byte accesses on both sides, HPB kv heads of one page
// per block (a page's metadata is read once for all of them, and every
// thread has 2 HPB loads in flight).  Thread (r, c8) moves key dims
// [8 c8, 8 c8 + 8) of slot r; values go through LDS ([slot][d], padded rows)
// and leave as 8 consecutive slots of one dim row of the page.  The stream's
// keys and values are read once, so their loads are non-temporal.
constexpr int KV_D = 128;
constexpr int KV_VS = KV_D + 8;   // LDS row stride (bf16): slot rows on different banks

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint4 load_nt(const uint16_t *p)
{
    const u32x4 x = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
    return make_uint4(x[0], x[1], x[2], x[3]);
}

template <int HPB>
__global__ void __launch_bounds__(256) k_kv_append_bf16(const uint16_t *__restrict__ k,
                                                        const uint16_t *__restrict__ v, int Hkv,
                                                        const int32_t *__restrict__ header,
                                                        const int32_t *__restrict__ tile_seg,
                                                        const int32_t *__restrict__ tile_row0,
                                                        const int32_t *__restrict__ seg_start,
                                                        const int32_t *__restrict__ seg_len,
                                                        const int32_t *__restrict__ page_off,
                                                        const int32_t *__restrict__ pages, uint16_t *__restrict__ kp,
                                                        uint16_t *__restrict__ vp)
{
    __shared__ __attribute__((aligned(16))) uint16_t vt[HPB][FK_TILE_TOKENS * KV_VS];
    if (header[H_STATUS] != FK_OK) return;
    const int tile = blockIdx.x, h0 = blockIdx.y * HPB;
    if (tile >= header[H_NTILES]) return;
    const int s = tile_seg[tile], row0 = tile_row0[tile];
    const int count = min(FK_TILE_TOKENS, seg_len[s] - row0);
    const int page = pages[page_off[s] + row0 / FK_TILE_TOKENS];
    const int t0 = seg_start[s] + row0;
    const size_t page_base = ((size_t)page * Hkv + h0) * (size_t)FK_TILE_TOKENS * KV_D;
    const int r = threadIdx.x >> 4, c8 = threadIdx.x & 15;
    uint4 kv[HPB], vv[HPB];
#pragma unroll
    for (int hh = 0; hh < HPB; ++hh) {
        kv[hh] = vv[hh] = make_uint4(0, 0, 0, 0);
        if (r < count) {
            const size_t src = ((size_t)(t0 + r) * Hkv + h0 + hh) * KV_D + c8 * 8;
            kv[hh] = load_nt(k + src);
            vv[hh] = load_nt(v + src);
        }
    }
#pragma unroll
    for (int hh = 0; hh < HPB; ++hh) {
        *reinterpret_cast<uint4 *>(kp + page_base + ((size_t)hh * FK_TILE_TOKENS + r) * KV_D + c8 * 8) = kv[hh];
        *reinterpret_cast<uint4 *>(vt[hh] + r * KV_VS + c8 * 8) = vv[hh];
    }
    __syncthreads();
    // dim x = tid / 2, slots [8 (tid % 2), +8).  The two lanes of a pair read
    // slot rows 8 apart (8 x 68 dwords: the same bank); the odd lane walks its
    // rows rotated by four (rows 68 x 4 dwords further on: 16 banks away), so
    // every read of a wave is free of bank conflicts, and swaps the halves of
    // its result back into slot order.
    const int x = threadIdx.x >> 1, odd = threadIdx.x & 1, r8 = odd * 8;
#pragma unroll
    for (int hh = 0; hh < HPB; ++hh) {
        uint16_t e[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) e[j] = vt[hh][(r8 + ((j + 4 * odd) & 7)) * KV_VS + x];
        const uint32_t p0 = e[0] | ((uint32_t)e[1] << 16), p1 = e[2] | ((uint32_t)e[3] << 16);
        const uint32_t p2 = e[4] | ((uint32_t)e[5] << 16), p3 = e[6] | ((uint32_t)e[7] << 16);
        const uint4 out = odd ? make_uint4(p2, p3, p0, p1) : make_uint4(p0, p1, p2, p3);
        *reinterpret_cast<uint4 *>(vp + page_base + (size_t)hh * FK_TILE_TOKENS * KV_D + x * FK_TILE_TOKENS + r8) =
            out;
    }
}

}  // namespace fk

using namespace fk;

// shared with fork_attn_forward
int fk_launch_kv_append(const fk_tree_meta *meta, const void *k, const void *v, int dtype, int Hkv, int d,
                        void *k_pool, void *v_pool, const void *ws, hipStream_t st)
{
    const WsLayout L = ws_layout(*meta, 0, 0, 0);
    dim3 grid((unsigned)L.tile_cap, (unsigned)Hkv);
    const int32_t *hdr = ws_at<int32_t>(ws, L.header);
    const int32_t *ts = ws_at<int32_t>(ws, L.tile_seg), *tr = ws_at<int32_t>(ws, L.tile_row0);
    const int32_t *ss = ws_at<int32_t>(ws, L.seg_start), *sl = ws_at<int32_t>(ws, L.seg_len);
    if (dtype == FK_BF16 && d == KV_D) {
        // heads per block: 4, 2 or 1, whichever divides Hkv
        const int hpb = Hkv % 4 == 0 ? 4 : Hkv % 2 == 0 ? 2 : 1;
        dim3 g2((unsigned)L.tile_cap, (unsigned)(Hkv / hpb));
        auto kern = hpb == 4 ? k_kv_append_bf16<4> : hpb == 2 ? k_kv_append_bf16<2> : k_kv_append_bf16<1>;
        kern<<<g2, 256, 0, st>>>((const uint16_t *)k, (const uint16_t *)v, Hkv, hdr, ts, tr, ss, sl,
                                 meta->seg_page_off, meta->seg_pages, (uint16_t *)k_pool, (uint16_t *)v_pool);
    } else if (dtype == FK_BF16)
        k_kv_append<uint16_t><<<grid, 256, 0, st>>>((const uint16_t *)k, (const uint16_t *)v, Hkv, d, hdr, ts, tr,
                                                   ss, sl, meta->seg_page_off, meta->seg_pages,
                                                   (uint16_t *)k_pool, (uint16_t *)v_pool);
    else
        k_kv_append<float><<<grid, 256, 0, st>>>((const float *)k, (const float *)v, Hkv, d, hdr, ts, tr, ss, sl,
                                                meta->seg_page_off, meta->seg_pages, (float *)k_pool,
                                                (float *)v_pool);
    return launch_status();
}

int fk_check_kv_args(const fk_tree_meta *meta, const void *k, const void *v, int dtype, int Hkv, int d,
                     void *k_pool, void *v_pool, const void *ws)
{
    int rc = check_meta_scalars(meta);
    if (rc) return rc;
    if (!ws || !k_pool || !v_pool || (meta->T > 0 && (!k || !v))) return FK_E_INVALID_ARG;
    if (!meta->seg_page_off || meta->n_pages < 1) return FK_E_INVALID_ARG;
    if (dtype != FK_F32 && dtype != FK_BF16) return FK_E_UNSUPPORTED;
    if (Hkv < 1 || d < 1 || d > 128) return FK_E_UNSUPPORTED;
    return FK_OK;
}

extern "C" int kv_append(const fk_tree_meta *meta, const void *k, const void *v, int dtype, int Hkv, int d,
                         void *k_pool, void *v_pool, const void *ws, fk_stream_t stream)
{
    int rc = fk_check_kv_args(meta, k, v, dtype, Hkv, d, k_pool, v_pool, ws);
    if (rc) return rc;
    if (meta->T == 0) return FK_OK;
    return fk_launch_kv_append(meta, k, v, dtype, Hkv, d, k_pool, v_pool, ws, (hipStream_t)stream);
}
