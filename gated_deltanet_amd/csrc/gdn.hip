// gdn.hip -- forked Gated DeltaNet: the float32 per-token kernel and the
// gdn_fork_forward entry point (Flide section 3.2.2, Eq. 4 and its two-call
// scheme, generalised to one launch per tree level).
//
// Level d processes every live segment at depth d.  A segment starts from
//   the zero state (fresh root), state_in[slot] (child of a cached history,
//   Flide section 3.4), or the fork-point state its parent's launch wrote
//   (read by index: one write per distinct fork point, no copy per child).
// While it runs, a segment writes its state at every offset where children
// fork (in offset order), and its final state to state_out if requested.
// Chunking, where used, is anchored at the segment start, so a trunk's
// arithmetic never depends on its branches (Flide section 3.5).
#include <hip/hip_runtime.h>

#include "fk_common.h"

int fk_launch_gdn_bf16_prep(const fk_tree_meta *meta, const void *q, const void *k, const float *a, const float *b,
                            int Hk, int Hv, const void *ws, hipStream_t st);
int fk_launch_gdn_bf16(const fk_tree_meta *meta, int level, const void *q, const void *k, const void *v,
                       const float *a, const float *b, int Hk, int Hv, const float *state_in, float *state_out,
                       void *out, const void *ws, float *fork_states, hipStream_t st);

namespace fk {

struct GdnCommon {
    const int32_t *header, *lvl_seg, *seg_start, *seg_len, *seg_src, *emit_off, *emit_pos, *seg_state_out;
    const float *state_in;
    float *state_out, *fork_states;
    int level, level_cap;
};

// grid: (level_cap, Hv); block 256.  Thread layout: TPR = 256 / dv threads
// per state row, each holding dk / TPR consecutive-stride columns.
template <int DK, int DV>
__global__ void __launch_bounds__(256) k_gdn_f32(const float *__restrict__ q, const float *__restrict__ k,
                                                 const float *__restrict__ v, const float *__restrict__ a,
                                                 const float *__restrict__ b, float *__restrict__ out, int Hk,
                                                 int Hv, GdnCommon C)
{
    constexpr int TPR = 256 / DV;
    constexpr int NC = DK / TPR;
    static_assert(TPR >= 1 && TPR <= 64 && NC >= 1, "shape");
    if (C.header[H_STATUS] != FK_OK) return;
    if ((int)blockIdx.x >= C.header[H_LEVEL0 + C.level]) return;
    const int s = C.lvl_seg[C.level * C.level_cap + blockIdx.x];
    const int h = blockIdx.y, g = h / (Hv / Hk);
    const int row = threadIdx.x / TPR, sub = threadIdx.x % TPR;
    const size_t SZ = (size_t)DV * DK;
    float S[NC];
    const int src = C.seg_src[s];
    const float *S0 = src == -1 ? nullptr
                                : (src >= 0 ? C.fork_states + ((size_t)src * Hv + h) * SZ
                                            : C.state_in + ((size_t)(-2 - src) * Hv + h) * SZ);
#pragma unroll
    for (int c = 0; c < NC; ++c) S[c] = S0 ? S0[(size_t)row * DK + sub + c * TPR] : 0.f;
    int e = C.emit_off[s];
    const int e_end = C.emit_off[s + 1];
    const int len = C.seg_len[s], t0 = C.seg_start[s];
    auto emit_upto = [&](int done) {
        while (e < e_end && C.emit_pos[e] == done) {
            float *dst = C.fork_states + ((size_t)e * Hv + h) * SZ + (size_t)row * DK;
#pragma unroll
            for (int c = 0; c < NC; ++c) dst[sub + c * TPR] = S[c];
            ++e;
        }
    };
    emit_upto(0);
    for (int i = 0; i < len; ++i) {
        const int t = t0 + i;
        const float *kt = k + ((size_t)t * Hk + g) * DK;
        const float *qt = q + ((size_t)t * Hk + g) * DK;
        const float at = a[(size_t)t * Hv + h], bt = b[(size_t)t * Hv + h];
        const float vt = v[((size_t)t * Hv + h) * DV + row];
        float kc[NC], qc[NC];
        float u = 0.f;
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            kc[c] = kt[sub + c * TPR];
            qc[c] = qt[sub + c * TPR];
            u += S[c] * kc[c];
        }
        for (int o = TPR / 2; o > 0; o >>= 1) u += __shfl_xor(u, o, 64);
        float y = 0.f;
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            S[c] = at * (S[c] - bt * u * kc[c]) + bt * vt * kc[c];
            y += S[c] * qc[c];
        }
        for (int o = TPR / 2; o > 0; o >>= 1) y += __shfl_xor(y, o, 64);
        if (sub == 0) out[((size_t)t * Hv + h) * DV + row] = y;
        emit_upto(i + 1);
    }
    const int so = C.seg_state_out[s];
    if (so >= 0) {
        float *dst = C.state_out + ((size_t)so * Hv + h) * SZ + (size_t)row * DK;
#pragma unroll
        for (int c = 0; c < NC; ++c) dst[sub + c * TPR] = S[c];
    }
}

template <int DK, int DV>
void launch_f32(dim3 grid, hipStream_t st, const void *q, const void *k, const void *v, const float *a,
                const float *b, void *out, int Hk, int Hv, const GdnCommon &C)
{
    k_gdn_f32<DK, DV><<<grid, 256, 0, st>>>((const float *)q, (const float *)k, (const float *)v, a, b,
                                            (float *)out, Hk, Hv, C);
}

using LaunchFn = void (*)(dim3, hipStream_t, const void *, const void *, const void *, const float *,
                          const float *, void *, int, int, const GdnCommon &);

LaunchFn pick_f32(int dk, int dv)
{
#define FK_CASE(DK, DV) \
    if (dk == DK && dv == DV) return launch_f32<DK, DV>;
    FK_CASE(16, 16) FK_CASE(16, 32) FK_CASE(16, 64) FK_CASE(16, 128)
    FK_CASE(32, 16) FK_CASE(32, 32) FK_CASE(32, 64) FK_CASE(32, 128)
    FK_CASE(64, 16) FK_CASE(64, 32) FK_CASE(64, 64) FK_CASE(64, 128)
    FK_CASE(128, 16) FK_CASE(128, 32) FK_CASE(128, 64) FK_CASE(128, 128)
#undef FK_CASE
    return nullptr;
}

}  // namespace fk

using namespace fk;

extern "C" int gdn_fork_forward(const fk_tree_meta *meta, const void *q, const void *k, const void *v,
                                const float *a, const float *b, int dtype, int Hk, int Hv, int dk, int dv,
                                const float *state_in, float *state_out, void *out, void *ws, size_t ws_bytes,
                                fk_stream_t stream)
{
    int rc = check_meta_scalars(meta);
    if (rc) return rc;
    if (!ws || (meta->T > 0 && (!q || !k || !v || !a || !b || !out))) return FK_E_INVALID_ARG;
    if (meta->n_state_in > 0 && !state_in) return FK_E_INVALID_ARG;
    if (meta->n_state_out > 0 && !state_out) return FK_E_INVALID_ARG;
    if (Hk < 1 || Hv < 1 || Hv % Hk) return FK_E_UNSUPPORTED;
    if (dtype == FK_F32) {
        if (!pick_f32(dk, dv)) return FK_E_UNSUPPORTED;
    } else if (dtype == FK_BF16) {
        if (dk != 128 || dv != 128) return FK_E_UNSUPPORTED;
    } else {
        return FK_E_UNSUPPORTED;
    }
    const WsLayout L = ws_layout(*meta, Hv, dk, dv);
    if (ws_bytes < L.total) return FK_E_WORKSPACE;
    hipStream_t st = (hipStream_t)stream;
    float *fork_states = ws_at<float>(ws, L.fork_states);
    GdnCommon C;
    C.header = ws_at<int32_t>(ws, L.header);
    C.lvl_seg = ws_at<int32_t>(ws, L.lvl_seg);
    C.seg_start = ws_at<int32_t>(ws, L.seg_start);
    C.seg_len = ws_at<int32_t>(ws, L.seg_len);
    C.seg_src = ws_at<int32_t>(ws, L.seg_src);
    C.emit_off = ws_at<int32_t>(ws, L.emit_off);
    C.emit_pos = ws_at<int32_t>(ws, L.emit_pos);
    C.seg_state_out = meta->seg_state_out;
    C.state_in = state_in;
    C.state_out = state_out;
    C.fork_states = fork_states;
    C.level_cap = meta->level_cap;
    if (!meta->seg_state_out) return FK_E_INVALID_ARG;
    if (meta->T == 0) return FK_OK;
    if (dtype == FK_BF16) {
        // per-chunk T = (I + A)^-1 and P of every chunk of the round, before any level
        rc = fk_launch_gdn_bf16_prep(meta, q, k, a, b, Hk, Hv, ws, st);
        if (rc) return rc;
    }
    for (int level = 0; level < meta->max_depth; ++level) {
        C.level = level;
        if (dtype == FK_F32) {
            dim3 grid((unsigned)meta->level_cap, (unsigned)Hv);
            pick_f32(dk, dv)(grid, st, q, k, v, a, b, out, Hk, Hv, C);
            if ((rc = launch_status())) return rc;
        } else {
            rc = fk_launch_gdn_bf16(meta, level, q, k, v, a, b, Hk, Hv, state_in, state_out, out, ws, fork_states,
                                    st);
            if (rc) return rc;
        }
    }
    return FK_OK;
}
