/*
 * forkgdn.h -- C ABI of the MI355X (gfx950) library for exact state forking.
 *
 * A round of decision requests is one flat token stream (Flide, section 3.2,
 * Eq. 2).  Every request is a tree of segments: a trunk (the shared state),
 * question branches forked from it, possibly deeper forks, and optionally a
 * cached history saved by an earlier pass (Flide, section 3.4).  Each branch
 * token must see exactly its own root-to-leaf ancestry, so that every branch
 * equals an isolated forward pass of its path (Flide, Proposition 3.1):
 *   - causal GQA softmax attention under the visibility rule of Flide
 *     section 3.2.1, Eq. 3, generalised to deeper trees as a sequence of
 *     aliases (ForkServe, item 1);
 *   - the gated delta rule of Flide section 3.2.2, Eq. 4,
 *       S_t = a_t S_{t-1} (I - b_t k_t k_t^T) + b_t v_t k_t^T,  o_t = S_t q_t,
 *     where a child continues from its parent's state at the fork point by
 *     index, without copying it.
 *
 * Conventions for every entry point:
 *   - Pointers are DEVICE pointers unless marked (host).  The caller owns and
 *     allocates every buffer (activations, K/V page pool, states, checkpoints,
 *     workspace); the library never allocates device memory.
 *   - Calls enqueue work on `stream` (a hipStream_t; NULL = the default
 *     stream) and return without synchronising, except fk_read_status.
 *   - Return value: FK_OK (0), or a negative FK_E_* code detected on the host
 *     (nothing is enqueued then).  Errors in the tree that only the device can
 *     see (the tree arrays are device-resident and never read by the host) are
 *     recorded in a status word inside the workspace; every later kernel of
 *     the round then exits early and outputs are unspecified.  Read it with
 *     fk_read_status.
 *   - Tensors are dense, row-major, in stream order.  dtype FK_F32 (float) or
 *     FK_BF16 (bfloat16, round-to-nearest-even on output).  a, b and all
 *     recurrent states are always float32 (Flide section 3.4 stores the
 *     recurrent state in float32).
 *   - Results are batch invariant: a branch's output bits depend only on its
 *     own path and segment boundaries, never on the other requests of the
 *     round (Flide, section 3.5).  No reduction uses atomics.
 */
#ifndef FORKGDN_H
#define FORKGDN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef void *fk_stream_t; /* hipStream_t */

enum fk_dtype { FK_F32 = 0, FK_BF16 = 1 };

enum fk_status {
    FK_OK = 0,
    FK_E_INVALID_ARG = -1,   /* null pointer, bad size, slot out of range        */
    FK_E_UNSUPPORTED = -2,   /* shape/dtype combination without a kernel        */
    FK_E_WORKSPACE = -3,     /* workspace smaller than fk_workspace_bytes        */
    FK_E_HIP = -4,           /* a HIP runtime call failed                        */
    /* tree errors: host validator and device status word */
    FK_E_SEG_RANGE = -10,    /* a token names a segment outside [0, S)           */
    FK_E_NONCONTIG = -11,    /* a segment's tokens are not contiguous            */
    FK_E_PARENT = -12,       /* parent index out of range, or a segment's own    */
    FK_E_CYCLE = -13,        /* parent chain loops or is deeper than max_depth   */
    FK_E_FORK = -14,         /* fork outside [0, parent length]; root fork != 0  */
    FK_E_EMPTY = -15,        /* live segment without tokens, cached with tokens  */
    FK_E_CACHED = -16,       /* cached segment below a live one; live child of a
                                cached segment not forked at its end             */
    FK_E_PAGES = -17,        /* page list too short or a page id out of range    */
    FK_E_CAPACITY = -18,     /* more segments on one level than level_cap, or
                                more distinct fork points than fork_cap          */
    FK_E_STATE_SLOT = -19    /* state slot missing or out of range               */
};

/* Deepest supported tree (levels 0 .. FK_MAX_DEPTH-1). */
#define FK_MAX_DEPTH 8
/* Query rows of one attention tile (tokens per tile, anchored at the start of
   every segment, so tiles never straddle segments). */
#define FK_TILE_TOKENS 16
/* Tokens per Gated DeltaNet chunk of the bf16 path (anchored at the start of
   every segment, so a trunk's chunking never depends on its branches). */
#define FK_GDN_CHUNK 64
/* tok_seg value of a padding token (the stream's tail past the round's live
   tokens, when T is a capacity), and seg_cached_len value of an unused
   segment slot (when S is a capacity). */
#define FK_PAD_TOKEN (-1)
#define FK_UNUSED_SEGMENT (-1)

/*
 * Round description (Flide section 3.3.1: all variables set by the round
 * composition live in device buffers; section 3.3.2: launches are sized by
 * host-known capacities, so the host never reads the tree).
 *
 * A segment is LIVE (its tokens are in the stream, contiguous and in position
 * order) or CACHED (seg_cached_len > 0: no stream tokens; its K/V are already
 * in the page pool and its final recurrent state is state_in[seg_state_in]).
 * seg_fork[c] is how many of the parent's tokens child c sees (0..len(parent);
 * a root has 0).  A segment's first position is its parent's first position
 * plus its fork, so question positions continue from the state (Flide 3.2).
 * Cached segments must be roots or children of cached segments, and a live
 * child of a cached segment must fork at the cached segment's end.
 *
 * Capacities (Flide section 3.3.2: graphs are captured once per stream
 * capacity and a round pads only at the tail): T and S may exceed the round.
 * Tokens past the round's last live token are padding (tok_seg ==
 * FK_PAD_TOKEN; padding may be followed only by padding) and segment slots
 * the round does not use have seg_cached_len == FK_UNUSED_SEGMENT (no tokens;
 * no segment may name one as its parent; their other fields are ignored).
 * Padding and unused slots get no tile, chunk, page write, position (-1) or
 * output row, so a round padded into a larger capacity gives the bits of the
 * same round described exactly.
 *
 * K/V pages: segment s owns pages seg_pages[seg_page_off[s] ..
 * seg_page_off[s+1]); its token i lives in page seg_pages[off + i/page_size],
 * slot i % page_size.  Every segment starts on a fresh page; a child aliases
 * its ancestors' pages by reading them, never by copying (ForkServe item 1:
 * fork copies the parent page table and an alias length).
 */
typedef struct fk_tree_meta {
    int32_t T;           /* stream tokens, live + padding (>= 0)                 */
    int32_t S;           /* segment slots, live + cached + unused (>= 1)         */
    int32_t max_depth;   /* capacity: tree levels, 1..FK_MAX_DEPTH               */
    int32_t level_cap;   /* capacity: live segments on any one level (>= 1)      */
    int32_t fork_cap;    /* capacity: distinct (parent, fork offset) fork points */
    int32_t page_size;   /* tokens per K/V page; must be 16                      */
    int32_t n_pages;     /* pages in the K/V pool                                */
    int32_t n_state_in;  /* slots in state_in (may be 0)                         */
    int32_t n_state_out; /* slots in state_out (may be 0)                        */
    const int32_t *tok_seg;        /* [T]   segment of every stream token, or
                                            FK_PAD_TOKEN                          */
    const int32_t *seg_parent;     /* [S]   parent segment, -1 for a root         */
    const int32_t *seg_fork;       /* [S]   parent tokens this segment sees       */
    const int32_t *seg_cached_len; /* [S]   history length if cached, 0 if live,
                                            FK_UNUSED_SEGMENT if unused           */
    const int32_t *seg_page_off;   /* [S+1] CSR offsets into seg_pages            */
    const int32_t *seg_pages;      /* [seg_page_off[S]] page ids                  */
    const int32_t *seg_state_in;   /* [S]   state_in slot of a cached segment, -1 */
    const int32_t *seg_state_out;  /* [S]   state_out slot to receive the final
                                            state of a live segment, or -1        */
} fk_tree_meta;

/*
 * Workspace bytes for a round: derived metadata (segment starts, positions,
 * ancestor chains, attention tiles, GDN chunks, level lists, fork-point
 * routing, status) plus the scratch of one Gated DeltaNet layer: fork_cap
 * fork-point states (Hv * dv * dk floats each) and two bf16 64 x 64 matrices
 * per chunk and v-head.  gdn_Hv, gdn_dk, gdn_dv describe the largest GDN
 * layer that will use the workspace (all 0 if none).  `meta` is (host); only
 * its scalar fields are read.
 */
size_t fk_workspace_bytes(const fk_tree_meta *meta, int32_t gdn_Hv, int32_t gdn_dk, int32_t gdn_dv);

/*
 * fk_tree_build -- the tree-metadata builder (Flide section 3.3.1: the
 * attention tile table and the GDN chunk work are built on the GPU).  Turns
 * (tok_seg, seg_parent, seg_fork, ...) into per-segment starts, lengths,
 * first positions, depths and ancestor chains; per-token positions; the
 * attention tile list (FK_TILE_TOKENS rows per tile, each with its ancestor
 * KV ranges implied by the chain -- no dense mask); the GDN chunk list
 * (FK_GDN_CHUNK tokens per chunk); per-level GDN segment lists; and the
 * fork-point routing (one state slot per distinct fork point,
 * shared by all children forked there).  Validates the tree on the device
 * and records the first error class in the status word.  Must run before
 * kv_append / fork_attn_forward / gdn_fork_forward of the same round; the
 * workspace then holds the round's metadata for every layer.
 * meta: (host) struct of device arrays.  ws: >= fk_workspace_bytes.
 */
int fk_tree_build(const fk_tree_meta *meta, void *ws, size_t ws_bytes, fk_stream_t stream);

/*
 * fk_tree_validate_host -- the same checks as fk_tree_build, on HOST arrays
 * (meta's pointers are host pointers here).  Returns FK_OK or the error
 * class.  For callers holding host copies of the tree, and for tests.
 */
int fk_tree_validate_host(const fk_tree_meta *meta_host);

/*
 * fk_token_positions -- copy the builder's per-token positions (int32 [T],
 * device) to `pos` (device): position = segment first position + local index
 * (Flide section 3.2: positions of a question continue from the state).
 */
int fk_token_positions(const fk_tree_meta *meta, const void *ws, int32_t *pos, fk_stream_t stream);

/*
 * kv_append -- write the stream's keys and values into the paged pool
 * (ForkServe item 1: a write allocates the writer's own pages only; children
 * alias the parent's).  k, v: [T, Hkv, d] in `dtype`.  k_pool: [n_pages, Hkv,
 * page_size, d]; v_pool: [n_pages, Hkv, d, page_size] (values are stored
 * transposed inside a page so that the attention kernel reads them with keys
 * contiguous).  Cached segments' pages are left untouched.  Slots past a
 * segment's last token in its last page are zero-filled: readers give them a
 * zero weight, which keeps an output finite only if the slot is finite.
 * Pages of cached segments that the caller wrote itself must therefore hold
 * finite values (zero) past the history's last token; pages written by
 * kv_append always do.
 */
int kv_append(const fk_tree_meta *meta, const void *k, const void *v, int dtype, int Hkv, int d,
              void *k_pool, void *v_pool, const void *ws, fk_stream_t stream);

/*
 * fork_attn_forward -- ForkAttention prefill over the whole round (Flide
 * section 3.2.1, Eq. 3; section 3.3.1: fully visible key blocks load without
 * a mask, only partially visible ones are masked; other requests' keys are
 * never read).  Appends k, v of the live tokens into the page pool (as
 * kv_append), then for every stream token x and q head h computes
 *   out[x,h] = sum_{y in vis(x)} softmax_y(scale * q[x,h] . k_y) v_y
 * where vis(x) is the cached history of x's root, each ancestor's first
 * `fork` tokens, and x's own segment up to and including x; q head h reads
 * kv head h / (Hq / Hkv).
 * q, out: [T, Hq, d]; k, v: [T, Hkv, d]; pools as in kv_append.  With k and
 * v both NULL the append is skipped (the round's keys/values are already in
 * the pool, e.g. written by kv_append).
 * Supported: FK_F32 with d <= 128; FK_BF16 with d == 128 and Hq/Hkv == 8.
 */
int fork_attn_forward(const fk_tree_meta *meta, const void *q, const void *k, const void *v,
                      int dtype, int Hq, int Hkv, int d, float scale, void *k_pool, void *v_pool,
                      void *out, void *ws, size_t ws_bytes, fk_stream_t stream);

/* Visibility rules of fork_attn_forward_rule (Flide section 3.2.1). */
enum fk_attn_rule {
    FK_RULE_CAUSAL = 0,  /* t_y <= t_x (fork_attn_forward)                          */
    FK_RULE_WINDOW = 1,  /* t_y <= t_x and t_x - t_y < window (a sliding-window layer) */
    FK_RULE_TWO_WAY = 2  /* every token of the own segment (models that read each
                            block both ways, Flide appendix H)                       */
};

/*
 * fork_attn_forward_rule -- fork_attn_forward under another visibility rule
 * of the same section, on the same tile table.  FK_RULE_WINDOW: a
 * sliding-window layer of width `window` (>= 1) also requires t_x - t_y <
 * window, with positions continuing from the fork, so a branch selects the
 * same keys as its standalone sequence; key blocks wholly outside every
 * row's window are skipped.  FK_RULE_TWO_WAY: t_y <= t_x is dropped, so a
 * row sees every token of its own segment and each ancestor's first `fork`
 * tokens -- the state still never reads a question, so questions still fork
 * it (Flide appendix H).  `window` is ignored unless rule == FK_RULE_WINDOW.
 * Other arguments, layouts, support and errors as fork_attn_forward;
 * FK_E_INVALID_ARG for an unknown rule or window < 1.
 */
int fork_attn_forward_rule(const fk_tree_meta *meta, const void *q, const void *k, const void *v, int dtype,
                           int Hq, int Hkv, int d, float scale, int rule, int window, void *k_pool, void *v_pool,
                           void *out, void *ws, size_t ws_bytes, fk_stream_t stream);

/*
 * fork_attn_readout -- attention at selected rows only (Flide section 3.3.3:
 * the output head reads only the last token of every question, so in the
 * final layer every token still contributes its keys and values while the
 * rest of the layer runs only at these rows, listed in an index buffer of
 * fixed size).  rows: int32 [n_rows] (device), stream token index of each
 * entry, or -1 for an unused entry (its output row is left untouched; so is
 * that of an entry naming a padding token).
 * q_rows, out_rows: [n_rows, Hq, d] -- the queries and outputs of the entries.
 * The round's keys/values must already be in the pool (kv_append or a full
 * fork_attn_forward of the round).  Each entry's output has the same bits as
 * that token's row of fork_attn_forward_rule with the same rule: the work of
 * an entry is the tile that holds its token, run the same way.  Other
 * arguments, support and errors as fork_attn_forward_rule.
 */
int fork_attn_readout(const fk_tree_meta *meta, const void *q_rows, const int32_t *rows, int32_t n_rows, int dtype,
                      int Hq, int Hkv, int d, float scale, int rule, int window, const void *k_pool,
                      const void *v_pool, void *out_rows, void *ws, size_t ws_bytes, fk_stream_t stream);

/*
 * gdn_fork_forward -- forked Gated DeltaNet (Flide section 3.2.2, Eq. 4, and
 * its two-call scheme generalised to one launch per tree level).  A fresh
 * root starts from the zero state; a child of a cached segment from
 * state_in[seg_state_in[parent]]; any other child from its parent's state
 * after `fork` tokens, which the parent's launch writes once per distinct
 * fork point into the workspace and every child reads by index (no copy per
 * child).  Each live segment with seg_state_out >= 0 writes its final state
 * to state_out[slot] (a checkpoint, Flide section 3.4).
 * q, k: [T, Hk, dk]; v, out: [T, Hv, dv] in `dtype`; a, b: [T, Hv] float
 * (decay and write strength, after the sigmoid); v-head h reads q/k head
 * h / (Hv / Hk).  state_in: [n_state_in, Hv, dv, dk] float, state_out:
 * [n_state_out, Hv, dv, dk] float (S is dv x dk, row-major).
 * Supported: FK_F32 with dk, dv in {16, 32, 64, 128}; FK_BF16 with
 * dk == dv == 128 (chunked form on MFMA, fp32 state).
 */
int gdn_fork_forward(const fk_tree_meta *meta, const void *q, const void *k, const void *v,
                     const float *a, const float *b, int dtype, int Hk, int Hv, int dk, int dv,
                     const float *state_in, float *state_out, void *out, void *ws, size_t ws_bytes,
                     fk_stream_t stream);

/* Size of the library's fixed per-GPU metadata array used by
   fork_attn_forward_noalloc. */
#define FK_NOALLOC_SCRATCH_BYTES (16u << 20)

/*
 * fork_attn_forward_noalloc -- for callers that cannot allocate device
 * memory or pass a workspace (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation): fk_tree_build followed by
 * fork_attn_forward in one call, with the round's derived metadata kept in
 * the library's own fixed array of FK_NOALLOC_SCRATCH_BYTES per GPU instead
 * of a caller workspace.  Same kernels, so the same output bits.  Arguments
 * as fork_attn_forward (k and v NULL: the keys/values are already paged);
 * status: int32 (device) or NULL -- receives the round's status word (FK_OK
 * or a tree error), copied on `stream` after the attention.  Returns
 * FK_E_WORKSPACE when fk_workspace_bytes(meta, 0, 0, 0) exceeds
 * FK_NOALLOC_SCRATCH_BYTES.  Calls no allocator.  All calls on one GPU share
 * its array (the first call on a device looks up the array's address there);
 * calls that overlap on one GPU race.
 */
int fork_attn_forward_noalloc(const fk_tree_meta *meta, const void *q, const void *k, const void *v, int dtype,
                              int Hq, int Hkv, int d, float scale, void *k_pool, void *v_pool, void *out,
                              int32_t *status, fk_stream_t stream);

/* Widest short convolution of gdn_conv_forward. */
#define FK_CONV_MAX_W 8

/*
 * gdn_conv_forward -- the short causal convolution in front of the Gated
 * DeltaNet rule, forked through the tree (Flide section 3.2.2: it mixes each
 * token with its few predecessors, read through the same kind of index as
 * the recurrent state, so the first tokens of a question see the last tokens
 * of the state it forks from; section 3.4: a checkpoint keeps the
 * convolution window).  Depthwise and linear, width W:
 *   y[t, c] = sum_{i < W} w[c, i] * x[p_i(t), c]
 * where p_0(t) = t and p_i(t) is the i-th predecessor of t along t's
 * isolated root-to-leaf sequence (a zero row before the sequence's first
 * row).  Accumulates in float32, i = 0 .. W-1 in order; bf16 output rounds to
 * nearest even.  (Any activation after the convolution is pointwise and is
 * the caller's.)
 * x, y: [T, C] in `dtype`, 16-byte aligned; w: [C, W] float.
 * window_in: [n_state_in, W-1, C] in `dtype`: the saved window of every
 * cached segment, in the segment's state_in slot (seg_state_in) -- the
 * inputs of the last W-1 rows of the cached sequence, oldest first, zero rows
 * where it is shorter.  May be NULL if no live segment has a cached parent
 * (otherwise the status word records FK_E_STATE_SLOT).
 * window_out: [n_state_out, W-1, C] in `dtype`: every live segment with
 * seg_state_out >= 0 writes its own window there (same definition), which a
 * later round reads back as window_in.  Required when n_state_out > 0 and
 * W > 1; both windows are ignored when W == 1.
 * Needs fk_tree_build of the same round in `ws` (any GDN sizes).
 * Supported: FK_BF16 with C % 8 == 0, FK_F32 with C % 4 == 0; 1 <= W <=
 * FK_CONV_MAX_W.
 */
int gdn_conv_forward(const fk_tree_meta *meta, const void *x, int dtype, int C, int W, const float *w,
                     const void *window_in, void *window_out, void *y, void *ws, size_t ws_bytes,
                     fk_stream_t stream);

/*
 * gdn_checkpoint_save -- copy the float32 recurrent states of `count`
 * consecutive slots state_out[slot .. slot+count) ([count, Hv, dv, dk])
 * into caller storage `ckpt` (Flide section 3.4: a checkpoint keeps the
 * float32 state; the keys/values before the checkpoint stay in their pages,
 * which the caller retains by id).  n_slots: slots in state_out.
 */
int gdn_checkpoint_save(const float *state_out, int32_t slot, int32_t count, int32_t n_slots, int32_t Hv,
                        int32_t dk, int32_t dv, float *ckpt, fk_stream_t stream);

/*
 * gdn_checkpoint_resume -- copy `count` saved states `ckpt` ([count, Hv, dv,
 * dk] float) into state_in[slot .. slot+count), so that cached segments of a
 * later round continue exactly where the saved pass stopped (Flide section
 * 3.4).  n_slots: slots in state_in.
 */
int gdn_checkpoint_resume(const float *ckpt, float *state_in, int32_t slot, int32_t count, int32_t n_slots,
                          int32_t Hv, int32_t dk, int32_t dv, fk_stream_t stream);

/*
 * fk_proj_gemm -- a projection either side of the token mixers (the linear
 * layers of a full model), with a fixed reduction order.  Flide section 3.5:
 * a batch-invariant engine makes every matrix product sum each output
 * element in one order whatever the number of rows; section 3.3.3: in the
 * last layer the products run only at the rows of the readout index buffer.
 *   y[m, n] = sum_k x[r(m), k] * w[n, k],   r(m) = rows[m], or m if rows is NULL
 * accumulated in float32 over k in ascending steps of 16, by one work-group
 * per output element whatever M is, so a row's bits depend only on that row
 * of x and on w (never on M or on the other rows); output rounded to nearest
 * even.
 * x: [Mx, K] bf16 (device); rows: int32 [M] (device) or NULL (then M <= Mx);
 * an entry outside [0, Mx) selects no row and leaves row m of y untouched;
 * w: [N, K] bf16 (device; row n holds output feature n, as a linear layer
 * stores its weight); y: [M, N] bf16 (device).
 * Supported: FK_BF16 with K % 64 == 0 and N % 128 == 0 (FK_E_UNSUPPORTED
 * otherwise); FK_E_INVALID_ARG for a negative size, a null pointer, or
 * M > Mx without an index buffer.  M == 0 enqueues nothing.
 */
int fk_proj_gemm(const void *x, int32_t Mx, const int32_t *rows, int32_t M, int32_t K, const void *w, int32_t N,
                 int dtype, void *y, fk_stream_t stream);

/*
 * fk_read_status -- synchronise `stream` and read the device status word
 * written by fk_tree_build into *status_out (host): FK_OK or a tree error.
 */
int fk_read_status(const void *ws, fk_stream_t stream, int32_t *status_out);

/* Static description of a status code (host). */
const char *fk_strerror(int code);

/* ABI version of this header (host). */
int fk_abi_version(void);

/*
 * Measurement utility (not part of the method; used to report the dense bf16
 * MFMA rate the device sustains next to its published peak).
 * fk_peak_mfma_bf16 -- launch n_wg work-groups of four waves, each running
 * `iters` rounds of eight independent 32x32x16 bf16 matrix-core products on
 * register operands; *flops (host) receives the launch's product flops
 * (n_wg * 4 * iters * 8 * 32768).  The caller times the launch on `stream`.
 * sink: n_wg floats of device memory (one result per work-group, written so
 * the products are not removed).  FK_E_INVALID_ARG for a null pointer or a
 * count below 1.
 */
int fk_peak_mfma_bf16(float *sink, int32_t n_wg, int32_t iters, double *flops, fk_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* FORKGDN_H */
