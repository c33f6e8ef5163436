/*
 * wavefilter.h -- C ABI of the WaveFilter per-step sparse-attention path on
 * AMD Instinct MI355X (gfx950).
 *
 * Method: WaveFilter, "Enhancing the Long-Context Capability of Diffusion
 * LLMs via Wavelet-Guided KV Cache Filtering" (arXiv 2606.00724).  Per layer
 * and denoising step, the cached prompt keys are decomposed along the token
 * axis by a discrete wavelet transform (section 2.2, equation 5; section 3.1),
 * the step's query block is scored against the low-frequency keys and a
 * Top-K keeps candidate regions (Figure 2 (c)), the regions are refined
 * recursively across scales down to single tokens (Figure 2 (d)), and the
 * queries attend over the kept prompt tokens plus the generated-position
 * cache (section 2.1, equation 3, restricted to that set).
 *
 * Two calls carry the work:
 *   wf_build_pyramid  -- once per cache refresh: orthonormal Haar
 *                        approximation of the prompt keys;
 *   wf_select_attend  -- once per denoising step: scoring, Top-K,
 *                        refinement and the sparse attention.
 *
 * Conventions for every entry point:
 *   - Device pointers are HIP device memory owned by the caller; the library
 *     never allocates, frees or synchronises.  Its only global state is the
 *     static scratch array of wf_select_attend_noalloc (one per device) and
 *     that array's looked-up address.  Work is enqueued on `stream` (a
 *     hipStream_t; NULL = the null stream) and completes asynchronously.
 *   - Arguments are checked on the host before anything is enqueued; on an
 *     error the call returns a negative status and enqueues nothing, and the
 *     outputs are untouched.  A failed kernel launch returns WF_ERR_HIP.
 *     Device-side faults surface at the caller's next synchronisation.
 *   - Tensors are row-major and dense unless a stride argument says
 *     otherwise.  Base pointers must be 16-byte aligned.
 *   - Concurrent calls need distinct workspaces; calls on one workspace must
 *     be ordered (same stream, or synchronised).
 */
#ifndef WAVEFILTER_H
#define WAVEFILTER_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
enum {
    WF_OK = 0,
    WF_ERR_NULL = -1,      /* a required pointer is NULL */
    WF_ERR_SHAPE = -2,     /* a size is out of range or inconsistent */
    WF_ERR_DTYPE = -3,     /* unknown element type, or q/k/v types differ from the pyramid's */
    WF_ERR_LEVELS = -4,    /* level count out of range or N_p not a multiple of 2^L */
    WF_ERR_BUDGET = -5,    /* per-level keep counts infeasible or beyond the supported size */
    WF_ERR_WORKSPACE = -6, /* workspace or pyramid buffer too small */
    WF_ERR_ALIGN = -7,     /* a pointer or stride is not 16-byte aligned */
    WF_ERR_HIP = -8,       /* a HIP launch or runtime call failed */
    WF_ERR_PYRAMID = -9,   /* pyramid descriptor not built by wf_build_pyramid */
    WF_ERR_OPTION = -10    /* an option argument has no defined meaning */
};

/*
 * Debug checks (option bit): OR WF_OPT_CHECK into the `aggregation` argument
 * of wf_select_attend / wf_select_attend_noalloc / wf_select_attend_layers,
 * or pass it as `options` to wf_attend_selected.  The call then scans its
 * inputs first and records, in a status word at the start of its workspace,
 * every precondition they break (bits below; 0 = none).  The selection and
 * attention kernels still clamp each index they read into its buffer, so an
 * out-of-range entry never leads to an access outside the buffers; with the
 * checks on, every such clamp is reported.  Read the word with
 * wf_check_status after the call.  The scan reads all of q, k, v (rows
 * [0, n_tot) of every head) and A_L once: a debugging aid, not for the timed
 * path.
 */
#define WF_OPT_CHECK 0x100
#define WF_CHECK_GEN_INDEX 1u          /* a gen_idx entry outside [0, n_tot) */
#define WF_CHECK_SEL_INDEX 2u          /* a sel entry outside [0, n_tot) (wf_attend_selected) */
#define WF_CHECK_NONFINITE_Q 4u        /* a NaN or infinity in q */
#define WF_CHECK_NONFINITE_K 8u        /* ... in k */
#define WF_CHECK_NONFINITE_V 16u       /* ... in v */
#define WF_CHECK_NONFINITE_PYRAMID 32u /* ... in the pyramid's A_L */

/*
 * The status word the last call with WF_OPT_CHECK left in `workspace` (the
 * workspace that call was given; NULL: the scratch array of
 * wf_select_attend_noalloc on the stream's device).  Copies the word to
 * *status after the work queued on `stream` so far has finished: this call
 * synchronises the stream and may not be captured into a graph.  Returns
 * WF_ERR_NULL for a NULL status pointer, WF_ERR_HIP if the copy fails.
 */
int wf_check_status(const void* workspace, void* stream, uint32_t* status);

/* How the n_q query rows combine into one region score (Figure 2 (c) scores
 * regions by the queries' correlation with the low-frequency keys and leaves
 * the combination of the rows open): the maximum over the rows of the
 * scaled logits l_i[c] = q_i . A_j[c] / sqrt(d), or their mean (which equals
 * the score of the averaged query row); or, with each row's logits turned
 * into attention probabilities by a softmax over the level's candidate set
 * (all n_L regions at level L, the children of the kept regions below;
 * section 1 names the attention mechanism as the measure of relevance),
 * p_i[c] = exp(l_i[c]) / sum_c' exp(l_i[c']), the maximum or the mean over
 * the rows of p_i[c].  The softmax variants need a covered set of at most
 * 8 192 positions (k_L 2^L), one layer per call and a Haar pyramid without
 * stored bands (else WF_ERR_BUDGET / WF_ERR_OPTION), and a workspace with
 * every row's logits. */
enum { WF_AGG_MAX = 0, WF_AGG_MEAN = 1, WF_AGG_SOFTMAX_MAX = 2, WF_AGG_SOFTMAX_MEAN = 3 };

/* Element types of q, k and v. */
enum { WF_F32 = 0, WF_BF16 = 1 };

/* wf_build_pyramid flags. */
#define WF_PYR_ALL_LEVELS 1u /* also store A_1..A_{L-1} and D_1..D_L (test/inspection) */
#define WF_PYR_DB2 2u        /* Daubechies' four-tap basis instead of Haar (section 3.1 leaves
                                the basis psi open): A_j[n] = sum_m g[m] A_{j-1}[(2n + m) mod N_j-1],
                                g = (1+r3, 3+r3, 3-r3, 1-r3) / (4 r2), D_j likewise with
                                h[m] = (-1)^m g[3-m] (the signal is extended periodically); every
                                band is stored as with WF_PYR_ALL_LEVELS, and wf_select_attend
                                scores the finer levels from the stored A_j (a coefficient is no
                                longer the scaled sum of its own 2^j tokens) */

/* Supported sizes. */
#define WF_MAX_LEVELS 7      /* region of 2^L tokens, L <= 7 */
#define WF_MAX_QUERIES 64    /* query-block rows n_q */
#define WF_MAX_HEADS 65535   /* batch * heads */
#define WF_MAX_KEEP_TOP 16384 /* k_L, the kept coarse regions */

/*
 * Pyramid descriptor, filled by wf_build_pyramid.  `base` points to the
 * caller's device buffer; the library reads it in wf_select_attend.
 * Layout of the buffer (float32, row-major):
 *   A_L  [batch, heads, N_p / 2^L, head_dim]                   at offset 0
 * and with WF_PYR_ALL_LEVELS or WF_PYR_DB2 additionally, in this order,
 *   D_1 .. D_L   then   A_1 .. A_{L-1},   each [batch, heads, N_p / 2^j, head_dim]
 * (use wf_pyramid_offset for the byte offset of each band).
 */
typedef struct wf_pyramid {
    int32_t batch;
    int32_t heads;
    int32_t n_prompt;
    int32_t head_dim;
    int32_t levels;
    int32_t dtype;     /* element type of the keys it was built from */
    uint32_t flags;
    uint32_t magic;    /* set by wf_build_pyramid */
    void* base;
    uint64_t bytes;
} wf_pyramid;

/* Library version string (static storage). */
const char* wf_version(void);

/* Human-readable text of a status code (static storage). */
const char* wf_status_string(int status);

/*
 * Bytes of device memory wf_build_pyramid needs for the given shape and
 * flags, or 0 if the shape is invalid.
 */
uint64_t wf_pyramid_bytes(int32_t batch, int32_t heads, int32_t n_prompt, int32_t head_dim,
                          int32_t levels, uint32_t flags);

/*
 * Byte offset inside the pyramid buffer of band `band` (0 = approximation A,
 * 1 = detail D) at level `level`, or UINT64_MAX when that band is not stored.
 */
uint64_t wf_pyramid_offset(const wf_pyramid* pyr, int32_t band, int32_t level);

/*
 * Haar pyramid of the cached prompt keys along the token axis (WaveFilter
 * section 2.2, equation 5, iterated on the approximation band; section 3.1:
 * applied to the prompt positions only).  Orthonormal Haar filters; output
 * coefficient n of level j is built from tokens [n 2^j, (n+1) 2^j):
 *     A_j[n] = (A_{j-1}[2n] + A_{j-1}[2n+1]) / sqrt(2),  A_0 = K_prompt,
 *     D_j[n] = (A_{j-1}[2n] - A_{j-1}[2n+1]) / sqrt(2).
 * Float32 accumulation; the coefficients are stored as float32.
 *
 *   k_prompt     device, element type `dtype`; head (b, h) starts at
 *                k_prompt + (b*heads + h) * head_stride elements and holds
 *                n_prompt rows of head_dim contiguous elements
 *   head_stride  elements between consecutive heads (>= n_prompt*head_dim,
 *                a multiple of 16 bytes); e.g. N_tot*head_dim when the prompt
 *                is the first n_prompt rows of a [B, H, N_tot, d] cache
 *   head_dim     64 or 128
 *   levels       0 <= L <= WF_MAX_LEVELS, n_prompt a multiple of 2^L
 *   flags        0, WF_PYR_ALL_LEVELS, WF_PYR_DB2 or both
 *   pyr_mem      device buffer of pyr_bytes >= wf_pyramid_bytes(...)
 *   out          host descriptor, filled on success
 * The streaming pass runs one workgroup per run of max(2^L, 2 to 8) rows of
 * a head; more than 2^31 - 1 such runs over all heads is WF_ERR_SHAPE.
 */
int wf_build_pyramid(const void* k_prompt, int64_t head_stride, int32_t batch, int32_t heads,
                     int32_t n_prompt, int32_t head_dim, int32_t dtype, int32_t levels,
                     uint32_t flags, void* pyr_mem, uint64_t pyr_bytes, wf_pyramid* out,
                     void* stream);

/*
 * Incremental pyramid refresh, batched over layers (or any pyramids that share
 * dtype and head_dim).  The cached prompt keys change on the cache's own
 * schedule (section 2.1, eq. 4 updates cache rows between steps); the
 * low-frequency keys of section 3.1 must follow.  For every item and every
 * (sequence, head) of its pyramid, each listed level-L block n is recomputed
 * from the item's current prompt keys, rows [n 2^L, (n+1) 2^L):
 * A_L[n] = 2^{-L/2} * sum of those rows (equation 5 iterated L times, as in
 * wf_build_pyramid, and bit for bit what a full rebuild writes).  Rows not
 * listed are left as they are.  One kernel launch for the whole batch.
 *
 *   items[i].k_prompt    device keys of the layer, laid out as for
 *                        wf_build_pyramid (its head_stride)
 *   items[i].pyr         host descriptor from wf_build_pyramid, without
 *                        WF_PYR_ALL_LEVELS or WF_PYR_DB2 (else
 *                        WF_ERR_OPTION: stored finer bands are not refreshed)
 *   items[i].blocks      device int32 [n_blocks]: level-L block indices shared
 *                        by all heads of the layer; entries outside
 *                        [0, N_p / 2^L) are skipped; repeats are harmless
 *   items[i].n_blocks    >= 0 (0: nothing to do for this item)
 *   n_items              1 .. WF_MAX_REFRESH_ITEMS
 * The sum over items of n_blocks * batch * heads is at most 2^31 - 1 (one
 * workgroup each), else WF_ERR_SHAPE.
 * Errors: WF_ERR_NULL, WF_ERR_SHAPE, WF_ERR_PYRAMID, WF_ERR_OPTION,
 * WF_ERR_DTYPE (items differ in dtype or head_dim), WF_ERR_ALIGN, WF_ERR_HIP.
 */
#define WF_MAX_REFRESH_ITEMS 32
typedef struct {
    const void* k_prompt;
    int64_t head_stride;
    const wf_pyramid* pyr;
    const int32_t* blocks;
    int32_t n_blocks;
} wf_refresh_item;

int wf_refresh_pyramids(const wf_refresh_item* items, int32_t n_items, void* stream);

/*
 * Bytes of workspace wf_select_attend needs, or 0 if the arguments are
 * invalid.  `budgets` is the host array k_L, ..., k_0 (levels + 1 entries).
 */
uint64_t wf_select_attend_workspace_bytes(const wf_pyramid* pyr, int32_t n_q, int32_t n_gen,
                                          const int32_t* budgets, int32_t aggregation);

/*
 * One denoising step of WaveFilter for every (sequence, head):
 *   1. s_L[n] = max_i (q_i . A_L[n]) / sqrt(d) for every level-L region n
 *      (mean_i with WF_AGG_MEAN), and keep the k_L best (Figure 2 (c)).
 *   2. For j = L-1 .. 0: the candidates are the two children of each region
 *      kept at level j+1, scored as s_j[c] = max_i (q_i . A_j[c]) / sqrt(d)
 *      (mean_i with WF_AGG_MEAN), and the k_j best are kept (Figure 2 (d)).  A_j is never stored: its
 *      dot products are the 2^{-j/2}-scaled sums of the token dot products
 *      q_i . k_t over the region (linearity of the transform).
 *   3. O_i = softmax over T of (q_i . k_t / sqrt(d)) applied to v_t, with T
 *      the kept prompt tokens followed by the generated positions gen_idx
 *      (equation 3 restricted to T; no mask).
 * "Best" means higher score, and on equal scores the lower index.  Scores
 * and accumulation are float32.
 *
 *   q            device [batch, heads, n_q, head_dim], element type of the pyramid
 *   pyr          built by wf_build_pyramid from k's prompt rows
 *   k, v         device [batch, heads, n_tot, head_dim]; rows [0, N_p) are
 *                the prompt, the rows named by gen_idx the generated positions
 *   gen_idx      device int32 [n_gen], row indices in [0, n_tot) shared by all
 *                heads (normally N_p .. n_tot-1); NULL allowed when n_gen == 0;
 *                out-of-range entries are clamped into range, and reported
 *                in the status word when WF_OPT_CHECK is set
 *   budgets      HOST int32 [levels + 1] = k_L, ..., k_0 with
 *                1 <= k_L <= min(N_p/2^L, WF_MAX_KEEP_TOP) and
 *                1 <= k_j <= min(2 k_{j+1}, N_p/2^j); WF_ERR_BUDGET also when
 *                the refinement state would not fit one workgroup's LDS
 *   n_q          1 .. WF_MAX_QUERIES
 *   aggregation  WF_AGG_MAX, WF_AGG_MEAN, WF_AGG_SOFTMAX_MAX or
 *                WF_AGG_SOFTMAX_MEAN, optionally ORed with WF_OPT_CHECK
 *                (anything else: WF_ERR_OPTION): how the query rows combine
 *                into the scores s_j at every level
 *   out          device float32 [batch, heads, n_q, head_dim]
 *   sel_out      NULL, or device int32 [batch, heads, k_0]: kept prompt
 *                tokens, ascending
 *   sel_levels   NULL, or device int32 [batch, heads, k_L + ... + k_0]: the
 *                kept region indices of level L, then L-1, ..., then 0, each
 *                ascending (level-j region n covers tokens [n 2^j, (n+1) 2^j))
 *   score_levels NULL, or device float32 of the same shape: each kept
 *                region's score s_j
 *   workspace    device buffer of ws_bytes >= wf_select_attend_workspace_bytes;
 *                scratch only: its contents on entry do not matter
 */
int wf_select_attend(const void* q, const wf_pyramid* pyr, const void* k, const void* v,
                     int32_t n_tot, const int32_t* gen_idx, int32_t n_gen, const int32_t* budgets,
                     int32_t n_q, int32_t aggregation, float* out, int32_t* sel_out,
                     int32_t* sel_levels, float* score_levels, void* workspace, uint64_t ws_bytes,
                     void* stream);

/*
 * Several layers in one call: wf_select_attend for every (layer, sequence,
 * head) of up to WF_MAX_LAYER_ITEMS layers that share one shape, so that the
 * heads of all layers fill the chip in one chain of launches instead of one
 * chain per layer (the pyramid of each layer built beforehand, as for
 * wf_select_attend).  Per layer and head the computation is that of
 * wf_select_attend; the kept tokens are identical, and O agrees up to the
 * rounding of the float32 accumulation (the attention is split over more or
 * fewer workgroups when more heads share the chip).
 *
 *   items        host array of n_items descriptors, one per layer:
 *                  q, k, v, out, sel_out as for wf_select_attend (sel_out may
 *                  be NULL); pyr built by wf_build_pyramid without
 *                  WF_PYR_ALL_LEVELS or WF_PYR_DB2, all with the same batch,
 *                  heads, N_p, head dim, levels and element type
 *   n_items      1 .. WF_MAX_LAYER_ITEMS
 *   n_tot, gen_idx, n_gen, budgets, n_q, aggregation
 *                shared by every layer, as for wf_select_attend
 *   workspace    device buffer of ws_bytes >=
 *                wf_select_attend_layers_workspace_bytes; scratch only
 * Returns WF_ERR_SHAPE when the layers differ in shape or n_items * batch *
 * heads exceeds WF_MAX_HEADS, WF_ERR_OPTION for a pyramid with stored finer
 * bands, else the statuses of wf_select_attend, before anything is enqueued.
 * No per-level outputs (sel_levels / score_levels) in this form.
 */
#define WF_MAX_LAYER_ITEMS 32
typedef struct {
    const void* q;
    const wf_pyramid* pyr;
    const void* k;
    const void* v;
    float* out;
    int32_t* sel_out;
} wf_layer_item;

/* Bytes of workspace wf_select_attend_layers needs for n_items layers of the
 * pyramid's shape, or 0 if the arguments are invalid. */
uint64_t wf_select_attend_layers_workspace_bytes(const wf_pyramid* pyr, int32_t n_items, int32_t n_q,
                                                 int32_t n_gen, const int32_t* budgets);
int wf_select_attend_layers(const wf_layer_item* items, int32_t n_items, int32_t n_tot, const int32_t* gen_idx,
                            int32_t n_gen, const int32_t* budgets, int32_t n_q, int32_t aggregation,
                            void* workspace, uint64_t ws_bytes, void* stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc):
 * wf_select_attend with the workspace taken from a static device array of
 * WF_NOALLOC_SCRATCH_BYTES that the library holds on every device it runs
 * on until the process ends.  Arguments, outputs, results and errors are
 * those of wf_select_attend, and the same kernels run.  The call allocates
 * and frees nothing; its first call on a device looks up that device's copy
 * of the array (with the stream's device made current for the lookup, then
 * restored), so a caller that captures should make one call beforehand.
 *
 *   stream       the device of the stream (the current device for the null
 *                stream) decides whose scratch array is used
 * Returns WF_ERR_WORKSPACE, before anything is enqueued, when the call's
 * workspace (wf_select_attend_workspace_bytes) exceeds
 * WF_NOALLOC_SCRATCH_BYTES; WF_ERR_HIP when the array cannot be located.
 * Every call on one device shares that device's array and leaves its
 * contents behind: calls that overlap on one device (on different streams,
 * or from several host threads onto streams that are not ordered) race and
 * must be serialised by the caller, e.g. by issuing them on one stream.
 */
#define WF_NOALLOC_SCRATCH_BYTES (16u << 20)
int wf_select_attend_noalloc(const void* q, const wf_pyramid* pyr, const void* k, const void* v,
                             int32_t n_tot, const int32_t* gen_idx, int32_t n_gen, const int32_t* budgets,
                             int32_t n_q, int32_t aggregation, float* out, int32_t* sel_out,
                             int32_t* sel_levels, float* score_levels, void* stream);

/*
 * Bytes of workspace wf_attend_selected needs, or 0 if the arguments are
 * invalid.
 */
uint64_t wf_attend_selected_workspace_bytes(int32_t batch, int32_t heads, int32_t head_dim, int32_t dtype,
                                            int32_t n_q, int32_t k0, int32_t n_gen);

/*
 * Attention only, over a selection made earlier: step 3 of wf_select_attend
 * with the kept prompt tokens handed in (equation 3 restricted to T = sel
 * followed by gen_idx; no mask; float32 accumulation).  This serves the
 * reading of WaveFilter section 1 and section 3.1 in which the key tokens
 * located at one denoising step are kept for the following steps: select
 * with wf_select_attend (its sel_out), then call this on the next steps with
 * their queries.
 *
 *   q            device [batch, heads, n_q, head_dim], element type `dtype`
 *   k, v         device [batch, heads, n_tot, head_dim]
 *   sel          device int32 [batch, heads, k0]: prompt rows per head (any
 *                order; ascending as wf_select_attend returns them); NULL
 *                allowed when k0 == 0; out-of-range entries are clamped
 *                (reported with WF_OPT_CHECK)
 *   gen_idx      device int32 [n_gen], shared by all heads; NULL allowed when
 *                n_gen == 0; out-of-range entries are clamped (reported with
 *                WF_OPT_CHECK)
 *   k0 + n_gen   >= 1
 *   options      0 or WF_OPT_CHECK (else WF_ERR_OPTION)
 *   out          device float32 [batch, heads, n_q, head_dim]
 *   workspace    device buffer of ws_bytes >= wf_attend_selected_workspace_bytes;
 *                scratch only
 * Returns WF_ERR_SHAPE / WF_ERR_DTYPE / WF_ERR_NULL / WF_ERR_ALIGN /
 * WF_ERR_WORKSPACE / WF_ERR_BUDGET (T too long for one workgroup's list) /
 * WF_ERR_OPTION on invalid arguments, before anything is enqueued.
 */
int wf_attend_selected(const void* q, const void* k, const void* v, int32_t batch, int32_t heads, int32_t n_tot,
                       int32_t head_dim, int32_t dtype, const int32_t* sel, int32_t k0, const int32_t* gen_idx,
                       int32_t n_gen, int32_t n_q, int32_t options, float* out, void* workspace, uint64_t ws_bytes,
                       void* stream);

#ifdef __cplusplus
}
#endif

#endif /* WAVEFILTER_H */
