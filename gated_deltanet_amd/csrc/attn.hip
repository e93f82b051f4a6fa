// attn.hip -- ForkAttention prefill, float32 path, and the fork_attn_forward
// entry point (Flide section 3.2.1, Eq. 3; section 3.3.1).
//
// A query token x of segment s sees, in this fixed order:
//   the first fork(a_{i+1}) tokens of every strict ancestor a_i on its chain
//   (a cached history is simply a cached ancestor), then its own segment up
//   to and including x.  Under the sliding-window rule it also needs
//   t_x - t_y < W; under the two-way rule it sees its whole own segment
//   (Flide section 3.2.1 and appendix H).
// Keys are visited in blocks anchored at the start of every range, so the
// order of a row's reductions depends only on its own chain -- never on the
// other segments of the round (Flide section 3.5).
//
// The float32 kernel is the simple form: one wave per (16-row tile, q head),
// an online softmax over 64-key chunks with wave reductions, keys and values
// read from the page pool.  The bf16 MFMA kernel lives in attn_bf16.hip.
#include <hip/hip_runtime.h>
#include <math.h>

#include "fk_common.h"

int fk_launch_kv_append(const fk_tree_meta *meta, const void *k, const void *v, int dtype, int Hkv, int d,
                        void *k_pool, void *v_pool, const void *ws, hipStream_t st);
int fk_check_kv_args(const fk_tree_meta *meta, const void *k, const void *v, int dtype, int Hkv, int d,
                     void *k_pool, void *v_pool, const void *ws);
int fk_launch_attn_bf16(const fk_tree_meta *meta, const void *q, int Hq, int Hkv, float scale, int rule, int window,
                        const int32_t *rows, int n_rows, const void *k_pool, const void *v_pool, void *out,
                        const void *ws, hipStream_t st);

namespace fk {

__device__ __forceinline__ float wave_max(float x)
{
    for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
    return x;
}

__device__ __forceinline__ float wave_sum(float x)
{
    for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, 64);
    return x;
}

// grid: (tile capacity, Hq); block: one wave.  d <= 128: lane owns dims
// lane and lane + 64.  Readout (sel_rows != NULL): grid (rows, Hq), the one
// selected token, its query and output at the row buffer's entry.
__global__ void __launch_bounds__(64) k_attn_f32(const float *__restrict__ q, int Hq, int Hkv, int d, float scale,
                                                 int rule, int window, const int32_t *__restrict__ sel_rows,
                                                 const int32_t *__restrict__ tok_seg, int T,
                                                 const int32_t *__restrict__ seg_pos0,
                                                 const float *__restrict__ kp, const float *__restrict__ vp,
                                                 float *__restrict__ out, const int32_t *__restrict__ header,
                                                 const int32_t *__restrict__ tile_seg,
                                                 const int32_t *__restrict__ tile_row0,
                                                 const int32_t *__restrict__ seg_start,
                                                 const int32_t *__restrict__ seg_len,
                                                 const int32_t *__restrict__ seg_depth,
                                                 const int32_t *__restrict__ seg_anc,
                                                 const int32_t *__restrict__ seg_fork,
                                                 const int32_t *__restrict__ page_off,
                                                 const int32_t *__restrict__ pages)
{
    if (header[H_STATUS] != FK_OK) return;
    const int tile = blockIdx.x, h = blockIdx.y, lane = threadIdx.x;
    int s, row0, nrows;
    if (sel_rows) {
        const int t = sel_rows[tile];
        if (t < 0 || t >= T) return;   // an unused entry of the row buffer
        s = tok_seg[t];
        if (s < 0) return;             // a padding token: no output
        row0 = t - seg_start[s];
        nrows = 1;
    } else {
        if (tile >= header[H_NTILES]) return;
        s = tile_seg[tile];
        row0 = tile_row0[tile];
        nrows = min(FK_TILE_TOKENS, seg_len[s] - row0);
    }
    const int g = h / (Hq / Hkv);
    const int depth = seg_depth[s];
    const int *anc = seg_anc + s * FK_MAX_DEPTH;
    const size_t page_elems = (size_t)FK_TILE_TOKENS * d;
    for (int r = 0; r < nrows; ++r) {
        const int t = seg_start[s] + row0 + r;
        const size_t qrow = sel_rows ? (size_t)tile * Hq + h : (size_t)t * Hq + h;
        const float *qr = q + qrow * d;
        float m = -INFINITY, l = 0.f, o0 = 0.f, o1 = 0.f;
        for (int lvl = 0; lvl <= depth; ++lvl) {
            const int a = anc[lvl];
            const int count = lvl < depth ? seg_fork[anc[lvl + 1]]
                                          : (rule == FK_RULE_TWO_WAY ? seg_len[s] : row0 + r + 1);
            // window: keys before klo are outside it; chunks stay anchored at 0
            const int klo = rule == FK_RULE_WINDOW ? max(0, seg_pos0[s] + row0 + r - seg_pos0[a] - window + 1) : 0;
            if (klo >= count) continue;
            const int *pl = pages + page_off[a];
            for (int c0 = (klo / 64) * 64; c0 < count; c0 += 64) {
                const int key = c0 + lane;
                float sc = -INFINITY;
                if (key < count && key >= klo) {
                    const float *kr = kp + ((size_t)pl[key / FK_TILE_TOKENS] * Hkv + g) * page_elems +
                                      (size_t)(key % FK_TILE_TOKENS) * d;
                    float acc = 0.f;
                    for (int x = 0; x < d; ++x) acc += qr[x] * kr[x];
                    sc = acc * scale;
                }
                const float mc = wave_max(sc);
                const float mn = fmaxf(m, mc);
                const float corr = expf(m - mn);          // 0 on the first chunk (m = -inf)
                const float p = (key < count && key >= klo) ? expf(sc - mn) : 0.f;
                l = l * corr + wave_sum(p);
                o0 *= corr;
                o1 *= corr;
                const int nk = min(64, count - c0);
                for (int j = 0; j < nk; ++j) {
                    const float pj = __shfl(p, j, 64);
                    const int kj = c0 + j;
                    const float *vb = vp + ((size_t)pl[kj / FK_TILE_TOKENS] * Hkv + g) * page_elems;
                    const int slot = kj % FK_TILE_TOKENS;
                    if (lane < d) o0 += pj * vb[(size_t)lane * FK_TILE_TOKENS + slot];
                    if (lane + 64 < d) o1 += pj * vb[(size_t)(lane + 64) * FK_TILE_TOKENS + slot];
                }
                m = mn;
            }
        }
        float *orow = out + qrow * d;
        if (lane < d) orow[lane] = o0 / l;
        if (lane + 64 < d) orow[lane + 64] = o1 / l;
    }
}

}  // namespace fk

using namespace fk;

// The full launch (rows == NULL) or the readout of `rows`.
static int attn_entry(const fk_tree_meta *meta, const void *q, const void *k, const void *v, int dtype, int Hq,
                      int Hkv, int d, float scale, int rule, int window, const int32_t *rows, int n_rows,
                      void *k_pool, void *v_pool, void *out, void *ws, size_t ws_bytes, hipStream_t st)
{
    if (rule != FK_RULE_CAUSAL && rule != FK_RULE_WINDOW && rule != FK_RULE_TWO_WAY) return FK_E_INVALID_ARG;
    if (rule == FK_RULE_WINDOW && window < 1) return FK_E_INVALID_ARG;
    // k == v == NULL: this round's keys/values are already in the pool
    const bool append = k || v;
    int rc = fk_check_kv_args(meta, append ? k : q, append ? v : q, dtype, Hkv, d, k_pool, v_pool, ws);
    if (rc) return rc;
    if (Hq < 1 || Hq % Hkv) return FK_E_UNSUPPORTED;
    const bool any = rows ? n_rows > 0 : meta->T > 0;
    if (any && (!q || !out)) return FK_E_INVALID_ARG;
    if (!(scale > 0.f) || !isfinite(scale)) return FK_E_INVALID_ARG;
    const WsLayout L = ws_layout(*meta, 0, 0, 0);
    if (ws_bytes < L.total) return FK_E_WORKSPACE;
    if (dtype == FK_BF16 && (d != 128 || Hq / Hkv != 8)) return FK_E_UNSUPPORTED;
    if (meta->T == 0) return FK_OK;
    if (append) {
        rc = fk_launch_kv_append(meta, k, v, dtype, Hkv, d, k_pool, v_pool, ws, st);
        if (rc) return rc;
    }
    if (!any) return FK_OK;
    if (dtype == FK_BF16)
        return fk_launch_attn_bf16(meta, q, Hq, Hkv, scale, rule, window, rows, n_rows, k_pool, v_pool, out, ws, st);
    dim3 grid((unsigned)(rows ? (int64_t)n_rows : L.tile_cap), (unsigned)Hq);
    k_attn_f32<<<grid, 64, 0, st>>>((const float *)q, Hq, Hkv, d, scale, rule, window, rows, meta->tok_seg, meta->T,
                                    ws_at<int32_t>(ws, L.seg_pos0), (const float *)k_pool,
                                    (const float *)v_pool, (float *)out, ws_at<int32_t>(ws, L.header),
                                    ws_at<int32_t>(ws, L.tile_seg), ws_at<int32_t>(ws, L.tile_row0),
                                    ws_at<int32_t>(ws, L.seg_start), ws_at<int32_t>(ws, L.seg_len),
                                    ws_at<int32_t>(ws, L.seg_depth), ws_at<int32_t>(ws, L.seg_anc), meta->seg_fork,
                                    meta->seg_page_off, meta->seg_pages);
    return launch_status();
}

extern "C" int fork_attn_forward_rule(const fk_tree_meta *meta, const void *q, const void *k, const void *v,
                                      int dtype, int Hq, int Hkv, int d, float scale, int rule, int window,
                                      void *k_pool, void *v_pool, void *out, void *ws, size_t ws_bytes,
                                      fk_stream_t stream)
{
    return attn_entry(meta, q, k, v, dtype, Hq, Hkv, d, scale, rule, window, nullptr, 0, k_pool, v_pool, out, ws,
                      ws_bytes, (hipStream_t)stream);
}

extern "C" int fork_attn_forward(const fk_tree_meta *meta, const void *q, const void *k, const void *v, int dtype,
                                 int Hq, int Hkv, int d, float scale, void *k_pool, void *v_pool, void *out,
                                 void *ws, size_t ws_bytes, fk_stream_t stream)
{
    return attn_entry(meta, q, k, v, dtype, Hq, Hkv, d, scale, FK_RULE_CAUSAL, 0, nullptr, 0, k_pool, v_pool, out,
                      ws, ws_bytes, (hipStream_t)stream);
}

extern "C" int fork_attn_readout(const fk_tree_meta *meta, const void *q_rows, const int32_t *rows, int32_t n_rows,
                                 int dtype, int Hq, int Hkv, int d, float scale, int rule, int window,
                                 const void *k_pool, const void *v_pool, void *out_rows, void *ws, size_t ws_bytes,
                                 fk_stream_t stream)
{
    if (n_rows < 0 || (n_rows > 0 && !rows)) return FK_E_INVALID_ARG;
    if (n_rows == 0) return FK_OK;
    return attn_entry(meta, q_rows, nullptr, nullptr, dtype, Hq, Hkv, d, scale, rule, window, rows, n_rows,
                      const_cast<void *>(k_pool), const_cast<void *>(v_pool), out_rows, ws, ws_bytes,
                      (hipStream_t)stream);
}
