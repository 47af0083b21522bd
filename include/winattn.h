/*
 * winattn.h — C-ABI of the MI355X (gfx950) windowed grouped-query attention library.
 *
 * Two operations, both defined on the pages of crate cortiq-engine:
 *
 *  attn_window_chunk — exact softmax attention of a chunk of rows over a per-KV-group ring
 *    buffer window with optional sink keys and causal visibility inside the chunk. Defined by
 *    the o1c page ("A sealed layer's attention for a chunk of rows, on Metal"): the layout
 *    header comment, `wgf`, `o1c_score`, `o1c_max`, `o1c_soft`, `o1c_sum`, `o1c_add`, and the
 *    token path `o1c_tok_near` / `o1c_tok_merge`, all taken with zero far-field landmarks.
 *
 *  attn_window_gated — the unit-head variant of the dory page ("Dory's token path"):
 *    `dory_prep` (rotate-half RoPE, L2 unit heads, learned query scale, K/V into a
 *    position-indexed ring), `low_key`, `dory_score`, `dory_soft`, `dory_sum`, `dory_gate`.
 *
 * Conventions for every entry point:
 *  - Tensors are contiguous f32 (meta: u32) in DEVICE memory owned by the caller, each base
 *    pointer 16-byte aligned. The library never allocates on these paths.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream). Calls are asynchronous
 *    on that stream and never synchronise; results are ready when the stream reaches them.
 *  - Return 0 on success or a negative WINATTN_E* code; nothing is launched on error except
 *    for WINATTN_ELAUNCH, which reports a failed launch.
 *  - `workspace` is caller-owned device memory of at least the size the matching *_workspace
 *    query returns (0 means the call needs none and NULL may be passed). Its first 64 KiB hold
 *    split counters at a fixed place for every call shape. The plans that combine split
 *    partials inside one launch use them: the single-launch decode kernel's ready flags
 *    (kernel 5, also for one-row attn_window_chunk_far calls, whose far part runs in that
 *    launch), the gated single launch's ready flags (kernel 6) and the last-split merge of
 *    kernels 1 to 4 when WINATTN_TUNE_MERGE_KERNEL selects it; plans that merge in a separate
 *    launch never touch them. They must be zero before the first call that uses the workspace
 *    (a fresh zeroed allocation, or attn_workspace_init), and every call leaves them at zero
 *    again, so one workspace serves calls of any shapes in sequence. Two calls that may run at
 *    the same time must not share a workspace.
 */
#ifndef WINATTN_H
#define WINATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define WINATTN_ABI_VERSION 1

#define WINATTN_OK 0
#define WINATTN_EINVAL (-1)      /* a size, pointer, alignment or constraint is invalid */
#define WINATTN_EWORKSPACE (-2)  /* workspace missing or smaller than the query returned */
#define WINATTN_ELAUNCH (-3)     /* the HIP runtime reported an error at launch */
#define WINATTN_EUNSUPPORTED (-4)

/* Ring metadata of one KV group, four u32 per group, laid out as the o1c page's header comment
 * gives it: entries held, slot of the oldest entry, far-field count (the number of keys that
 * have left the window; read only by the far-field calls), and a per-group window override
 * (0 = the call's default w; `wgf`). */
typedef struct {
    uint32_t len;
    uint32_t head;
    uint32_t far_len;
    uint32_t window;
} attn_ring_meta;

/*
 * attn_window_chunk — out[i][g*hpg+h] = softmax attention of q[i][g*hpg+h] over the keys
 * visible to chunk row i of KV group g (o1c page: `o1c_score` defines the key set).
 *
 * Key set of row i, group g, with wg = meta[g].window ? meta[g].window : w,
 * len0 = meta[g].len, head0 = meta[g].head:
 *   the ns sinks sink_k[g][0..ns), then the last min(wg, len0 + i + 1) entries of the stream
 *   [ring entries 0..len0-1, chunk rows 0..i], where ring entry x (0 = oldest) is slot
 *   (head0 + x) mod wg of ring_k[g] and stream entry len0 + j is chunk row j. The window ends
 *   at and includes the row's own key, so a full ring's oldest entry is not seen by row 0.
 * Scores are scale * <q, k>; the result is sum_j softmax_j * v_j.
 *
 * Arguments (all device pointers):
 *   ring_k, ring_v   [ng][w][d]   ring storage; the slot stride is w even when wg < w
 *   meta             [ng] attn_ring_meta (four u32 per group); read only. Requirements (not
 *                                 checked on the device: see attn_window_check_meta):
 *                                 window <= w, len <= wg, head < wg when len > 0. The kernels
 *                                 clamp out-of-range fields so they never read out of bounds;
 *                                 the result is then unspecified.
 *   sink_k, sink_v   [ng][ns][d]  may be NULL iff ns == 0
 *   q                [rows][nh][d], nh = ng*hpg; heads g*hpg .. g*hpg+hpg-1 read group g
 *   chunk_k, chunk_v [rows][ng][d] the chunk's own keys and values
 *   out              [rows][nh][d] fully overwritten
 *   rows, ng, hpg, w >= 1; ns >= 0; d a multiple of 4, 4 <= d <= 256; scale finite
 * Only `out` and the workspace are written.
 */
int attn_window_chunk(const float* ring_k, const float* ring_v, const attn_ring_meta* meta,
                      const float* sink_k, const float* sink_v, const float* q,
                      const float* chunk_k, const float* chunk_v, float* out, int rows, int ng,
                      int hpg, int d, int w, int ns, float scale, void* workspace,
                      size_t workspace_bytes, void* stream);

/* Workspace bytes attn_window_chunk needs for these sizes (0 if the sizes are invalid). */
size_t attn_window_chunk_workspace(int rows, int ng, int hpg, int d, int w, int ns);

/*
 * attn_window_chunk_noalloc — attn_window_chunk for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid allocation): the
 * same operation, arguments, layouts and result, with no workspace argument. The split
 * partials and split counters live instead in a static device array of
 * WINATTN_NOALLOC_SCRATCH_BYTES that every GPU the library runs on holds for the life of the
 * process (its address is looked up on the first call on a device, which also clears the
 * counters with a fill kernel on `stream`). Nothing is allocated or freed, by this call or the
 * library routines it uses.
 *   - Calls whose plan needs more scratch than WINATTN_NOALLOC_SCRATCH_BYTES (the need is what
 *     attn_window_chunk_workspace reports for the same sizes) return WINATTN_EWORKSPACE and
 *     launch nothing.
 *   - All calls on one GPU share that GPU's array, which keeps the last call's contents: two
 *     calls that may overlap on one GPU (other streams, other threads) race and must not be
 *     made. Calls in sequence on one stream are safe (the counters are left at zero).
 * Returns as attn_window_chunk, plus WINATTN_ELAUNCH if the device array cannot be located.
 */
#define WINATTN_NOALLOC_SCRATCH_BYTES (32u << 20)
int attn_window_chunk_noalloc(const float* ring_k, const float* ring_v, const attn_ring_meta* meta,
                              const float* sink_k, const float* sink_v, const float* q,
                              const float* chunk_k, const float* chunk_v, float* out, int rows,
                              int ng, int hpg, int d, int w, int ns, float scale, void* stream);

/*
 * attn_window_gated — the gated unit-head call for rows at positions pos0 .. pos0+rows-1
 * (dory page). Steps, in this order:
 *  1. For each row and KV head kh: x, y = the halves of yk[row][kh]; c, s = the halves of
 *     rope[row]; u = x*c - y*s, v = y*c + x*s; k' = (u, v) / sqrt(sum u^2 + sum v^2 + eps).
 *     k' goes to ring_k[(pos0+row) % cap][kh] and yv[row][kh] to ring_v[(pos0+row) % cap][kh].
 *     Query head a is rotated and normalised the same way and multiplied by q_scale[a].
 *  2. Row `row` (pos = pos0+row) attends with query head a over positions lo..pos,
 *     lo = pos+1 > window ? pos+1-window : 0, reading slot p % cap of KV head a / (nh/nk),
 *     with scores scale * <q', k'> (`dory_score`, `dory_soft`, `dory_sum`).
 *  3. out[row][a][e] = o[e] / (1 + exp(-gate[row][a*hd+e] * gate_scale[a*hd+e])) (`dory_gate`).
 *
 * Arguments (all device pointers):
 *   yq [rows][nh][hd], yk and yv [rows][nk][hd]   raw heads
 *   rope [rows][hd]        cos of the row's angles in [0, hd/2), sin in [hd/2, hd)
 *   q_scale [nh][hd], gate [rows][nh*hd], gate_scale [nh*hd]
 *   ring_k, ring_v [cap][nk][hd]   read, and written at the rows' slots (step 1)
 *   out [rows][nh][hd]             fully overwritten
 *   rows, cap, window, nk >= 1; pos0 >= 0; nh a multiple of nk; hd a multiple of 8,
 *   8 <= hd <= 256; cap >= window + rows - 1 (so no row's write clobbers a key an earlier
 *   row still needs); eps >= 0.
 * Ring slots that no row reads and no row writes are left untouched.
 * Plans: widths 160, 192, 224 and 256 with at least 16 query vectors (rows * nh / nk) per KV
 * head run in one launch (kernel 6: the rotations where the heads are loaded, the ring write by
 * the workgroups that read the row, split partials folded by each query block's last splits;
 * blocks of 16 query vectors below 64 per KV head, of 64 from there on); its workspace holds the
 * split counters and the partials (none with a single split per block). In the 64-vector form
 * a chunk row's ring key slot may be written by several workgroups of the call, always with the
 * same bytes.
 * Other shapes prepare the unit heads and the ring in a first launch, then run the chunk
 * kernels on the prepared queries (the workspace also holds them) and, with several splits, a
 * merge launch. Every plan writes the same results within the tolerance of f32 rounding.
 */
int attn_window_gated(const float* yq, const float* yk, const float* yv, const float* rope,
                      const float* q_scale, const float* gate, const float* gate_scale,
                      float* ring_k, float* ring_v, float* out, int rows, int pos0, int cap,
                      int window, int nh, int nk, int hd, float scale, float eps,
                      void* workspace, size_t workspace_bytes, void* stream);

/* The state after a chunk, for the next call of a decode loop (o1c page, "A sealed layer's
 * attention for a chunk of rows, on Metal": `o1c_ring_commit` and `o1c_meta`; one-row form
 * `o1c_tok_commit`). Pushes the chunk's K/V rows into each group's ring and advances its meta:
 * row j lands in slot (head + len + j) mod wg (wg = the group's window: meta field 3 if
 * non-zero, else w); if len + rows <= wg, len grows by rows; otherwise len = wg, head moves on by
 * ev = len + rows - wg (mod wg) and the far count (field 2) grows by ev. Head and far count are
 * written only when entries are evicted. A chunk longer than wg leaves only its last wg rows
 * (pushes are sequential; the earlier rows are not written).
 *   ring_k, ring_v  device [ng][w][d] f32, updated in place (only the pushed slots)
 *   meta            device [ng][4] u32, updated in place (same rules as attn_window_chunk)
 *   chunk_k, chunk_v device [rows][ng][d] f32, the rows just attended (read only)
 * Sizes as attn_window_chunk (rows, ng, w >= 1; d % 4 == 0, 4 <= d <= 256); 16-byte aligned
 * float pointers, 4-byte aligned meta. Asynchronous on `stream`, allocates nothing; run it after
 * the chunk's attention call on the same stream (that call reads the slots this one
 * overwrites). Invalid device meta is clamped as in attn_window_chunk. Returns 0,
 * WINATTN_EINVAL (nothing launched) or WINATTN_ELAUNCH. */
int attn_window_commit(float* ring_k, float* ring_v, attn_ring_meta* meta, const float* chunk_k,
                       const float* chunk_v, int rows, int ng, int d, int w, void* stream);

/*
 * attn_window_chunk_far — attn_window_chunk plus the far field: landmark summaries of the keys
 * that have left each group's window (o1c page: `o1c_far_e`, `o1c_land`, `o1c_far`, `o1c_soft`,
 * `o1c_add`; token path `o1c_tok_far`, `o1c_tok_merge`).
 *
 * State, per query head gh = g*hpg + h and landmark b < m:
 *   mz     [nh][2m]    mz[gh][b] = far max mx_b, mz[gh][m+b] = far mass z_b (-inf and 0 while
 *                      the field is empty)
 *   t_hat  [nh][m][d]  far numerator: sum over evicted keys of exp(s - mx_b) V,
 *                      s = scale <q_tilde[gh][b], K>; z_b is the same sum of exp(s - mx_b)
 *   q_tilde [nh][m][d] landmark queries; k_tilde [ng][m][d] landmark keys;
 *   mu     [nh][m][m]  mixing matrix, row a, column b
 * Chunk row j >= j0 = wg - len evicts the group's oldest entry x = j - j0 (ring slot
 * (head + x) mod wg while x < len, else chunk row x - len); with e_b(j) = exp(s_b(j) - mx'_b),
 * mx'_b = max(mx_b, s_b(j) over the chunk's evictions), r_b = exp(mx_b - mx'_b) (1 if the max
 * did not move) and z_b(i) = z_b r_b + sum_{j0<=j<=i} e_b(j), row i of head gh with near scores
 * s over its attn_window_chunk key set takes, when far_len + (evictions up to row i) > 0:
 *   fl_a = scale <q, k_tilde[g][a]>, f = max fl, w_b = sum_a exp(fl_a - f) mu[gh][a][b],
 *   c = max(max s, f + mx'_b), G_b = w_b exp(f + mx'_b - c), F = sum_b G_b z_b(i);
 *   out = (sum exp(s - c) V + sum_b G_b (r_b t_hat_b + sum_{j0<=j<=i} e_b(j) V_ev(j)))
 *         / (sum exp(s - c) + F),
 * and drops the far terms (F and the numerator) when F < 0 or the field is empty.
 *
 * Arguments as attn_window_chunk plus the state above (device pointers, read only here), and
 * m, the landmark count: 1 <= m <= 64. rows <= 64 (the far path works on chunks of at most 64
 * rows; larger chunks or m return WINATTN_EUNSUPPORTED). The workspace is required (see
 * attn_window_chunk_far_workspace) and follows the convention above.
 */
int attn_window_chunk_far(const float* ring_k, const float* ring_v, const attn_ring_meta* meta,
                          const float* sink_k, const float* sink_v, const float* q,
                          const float* chunk_k, const float* chunk_v, const float* k_tilde,
                          const float* q_tilde, const float* mu, const float* mz,
                          const float* t_hat, float* out, int rows, int ng, int hpg, int d, int w,
                          int ns, int m, float scale, void* workspace, size_t workspace_bytes,
                          void* stream);

/* Workspace bytes attn_window_chunk_far needs for these sizes (0 if invalid or unsupported). */
size_t attn_window_chunk_far_workspace(int rows, int ng, int hpg, int d, int w, int ns, int m);

/*
 * attn_window_commit_far — the far state and ring after a chunk (o1c page: `o1c_far_commit`,
 * then `o1c_ring_commit` and `o1c_meta`). For every group with evictions in the chunk and every
 * head gh and landmark b: t_hat_b <- r_b t_hat_b + sum_{j>=j0} e_b(j) V_ev(j), mz[gh][b] <- mx'_b,
 * mz[gh][m+b] <- z_b(rows - 1) (notation of attn_window_chunk_far); groups without evictions
 * keep their state. Then exactly attn_window_commit. mz and t_hat [nh] as above, updated in
 * place; q_tilde read only. Sizes as attn_window_chunk_far with hpg = heads per group (no
 * sinks). Asynchronous on `stream`; allocates nothing and needs no workspace. Run it after the
 * chunk's attention call on the same stream. Returns 0, WINATTN_EINVAL, WINATTN_EUNSUPPORTED
 * (nothing launched) or WINATTN_ELAUNCH.
 */
int attn_window_commit_far(float* ring_k, float* ring_v, attn_ring_meta* meta, const float* chunk_k,
                           const float* chunk_v, const float* q_tilde, float* mz, float* t_hat,
                           int rows, int ng, int hpg, int d, int w, int m, float scale,
                           void* stream);

/*
 * attn_window_gated_far — the gated one-row call with the far field (dory page: `dory_os`,
 * `dory_ol`, `dory_omax`, `dory_ofar`, `dory_osoft`, `dory_osum`, `dory_ogate`). The row's own
 * key and value are already in the ring (pushed by the caller), so query head gh (KV head
 * kh = gh / (nh/nk)) attends over the ns sinks of kh and ring slots 0 .. len-1 of kh, with
 * len = meta[kh].len (storage order is irrelevant: the ring holds exactly the window) and
 * scores scale * <q, K>. When meta[kh].far_len > 0 the landmark part joins: fl_a =
 * scale <q, k_tilde[kh][a]>, f = max fl, u_b = sum_a exp(fl_a - f) mu[gh][a][b] (clamped at 0
 * when rect = 1), c = max(max s, f + mz[gh][b]), G_b = u_b exp(f + mz[gh][b] - c), far mass
 * F = sum_b G_b mz[gh][m+b]; when F >= 0,
 *   out = (sum exp(s - c) V + sum_b G_b t_hat[gh][b]) / (sum exp(s - c) + F),
 * else the far terms are dropped; then out[gh][e] /= 1 + exp(-gate[gh*hd+e] * gate_scale[gh*hd+e]).
 *
 * Arguments (device pointers): q [nh][hd]; ring_k, ring_v [nk][w][hd]; meta [nk][4] u32
 * (fields 0 and 2 are read; len <= w, larger values are clamped to w); sink_k, sink_v
 * [nk][ns][hd] (NULL iff ns == 0); k_tilde [nk][m][hd]; mu [nh][m][m]; mz [nh][2m]; t_hat
 * [nh][m][hd]; gate, gate_scale [nh*hd]; out [nh][hd] fully overwritten. nh a multiple of nk,
 * hd % 4 == 0, 4 <= hd <= 256, w >= 1, ns >= 0, 1 <= m <= 64 (larger: WINATTN_EUNSUPPORTED),
 * rect 0 or 1. Workspace as attn_window_gated_far_workspace returns (always non-zero).
 */
int attn_window_gated_far(const float* q, const float* ring_k, const float* ring_v,
                          const attn_ring_meta* meta, const float* sink_k, const float* sink_v,
                          const float* k_tilde, const float* mu, const float* mz,
                          const float* t_hat, const float* gate, const float* gate_scale,
                          float* out, int nh, int nk, int hd, int w, int ns, int m, float scale,
                          int rect, void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes attn_window_gated_far needs for these sizes (0 if invalid or unsupported). */
size_t attn_window_gated_far_workspace(int nh, int nk, int hd, int w, int ns, int m);

/*
 * attn_encoder — encoder attention over packed variable-length sequences (egemma2 page,
 * "EmbeddingGemma 2 encoder": `eg_flash_body` / `eg_flash64` / `eg_flash64s` for whole
 * sequences with segments [start, len] and K/V heads shared by groups of query heads;
 * `EgAtt` / `eg_softmax` for the symmetric window). Sequence s holds rows start .. start+len-1
 * (segs[2s], segs[2s+1]); the row at position i of its sequence attends with query head h to
 * the rows at positions j of the same sequence with |i - j| <= window (window 0: every
 * position), reading KV head h / (nh/nk), with scores scale * <q, k> and no causal mask:
 *   out[row][h*hd .. h*hd+hd) = sum_j softmax_j(scale <q_i, k_j>) v_j.
 *
 * Arguments (device pointers, f32 rows): q row t at q + t*ldq, head h's hd values at h*hd;
 * k, v rows at t*ldk, t*ldv, KV head kvh at kvh*hd; out rows at t*ldo (only the hd-wide head
 * slices of rows inside some sequence are written). The page's packed q|k|v rows are
 * q = QKV + q_off, k = QKV + k_off, v = QKV + v_off with one row stride. segs: device
 * [nseg][2] u32, disjoint sequences. max_len: an upper bound on every len (rows of a longer
 * sequence past max_len are not written). nh a multiple of nk; hd % 4 == 0, 4 <= hd <= 256;
 * every ld* a multiple of 4 and at least the row's heads
 * (nh*hd for q and out, nk*hd for k and v); pointers 16-byte aligned; window >= 0. nseg == 0
 * or max_len == 0 launches nothing. No workspace; asynchronous on `stream`.
 */
int attn_encoder(const float* q, const float* k, const float* v, float* out,
                 const uint32_t* segs, int nseg, int max_len, int ldq, int ldk, int ldv, int ldo,
                 int nh, int nk, int hd, int window, float scale, void* stream);

/* Workspace bytes attn_window_gated needs for these sizes (0 if the sizes are invalid). */
size_t attn_window_gated_workspace(int rows, int nh, int nk, int hd, int window);

/* Zero `bytes` bytes of device memory at `workspace` on `stream` with a fill kernel. */
int attn_workspace_init(void* workspace, size_t bytes, void* stream);

/* Host-side check of ring metadata in HOST memory against the rules above: 0 if every group is
 * valid, WINATTN_EINVAL otherwise (also for a NULL pointer or ng, w < 1). */
int attn_window_check_meta(const attn_ring_meta* host_meta, int ng, int w);

/* Diagnostics: how attn_window_chunk would run these sizes. kernel = 1 (register-resident
 * split-K kernel, up to 8 query vectors per block, split merge in a second launch), 2 (f32
 * matrix-core kernel on 32x32 tiles, 128 per block, above 256 query vectors per group),
 * 3 (LDS-staged vector-ALU split-K kernel, 16 per block; forced plans only), 4 (f32
 * matrix-core kernel on 16x16 tiles, 64 per block: 9 to 256 query vectors per group, and every
 * width above 8 at d > 128) or 5 (single-launch register kernel streaming the rings in slot
 * order, up to 8 query vectors: every query of a group in one block; the group's last splits
 * merge; it also takes one-row attn_window_chunk_far and attn_window_gated_far calls, with the
 * far part in its launch); query_block = query vectors per workgroup; splits = key splits reserved per query
 * block; keys_per_split = keys each split covers at most. Output pointers may be NULL.
 * Returns 0 or WINATTN_EINVAL. */
int attn_window_chunk_plan(int rows, int ng, int hpg, int d, int w, int ns, int* kernel,
                           int* query_block, int* splits, int* keys_per_split);

/* Self-test of the matrix-core operand layout the wide-chunk kernel relies on (after the
 * fragment-layout probe of the egemma2 page, `eg_fragprobe`): one 32x32x2 f32 product with
 * A[i][0] = i, A[i][1] = 1, B[0][j] = 1, B[1][j] = 64 j, so element (i, j) holds i + 64 j.
 * out: device [64][16] floats; out[lane*16 + r] = accumulator r of lane `lane`. */
int attn_mfma_layout_probe(float* out, void* stream);

/* The same self-test for the 16x16x4 f32 product of kernel 4: A[i][0] = i, A[i][1..3] = 1,
 * B[0][j] = 1, B[1][j] = 64 j, B[2][j] = B[3][j] = 0, so element (i, j) holds i + 64 j.
 * out: device [64][4] floats; out[lane*4 + r] = accumulator r of lane `lane`. */
int attn_mfma16_layout_probe(float* out, void* stream);

/* Measurement aid: the achievable HBM read rate for a buffer of a given size. One launch reads
 * every 16-byte element of src[0 .. bytes) once (coalesced 16-byte loads, eight in flight per
 * thread, one workgroup of 256 threads per 32 KiB) and folds them into per-thread sums; sink
 * (device, 256 floats) is written only if the data holds a NaN. bytes: a positive multiple of
 * 16; src 16-byte aligned. Returns 0, WINATTN_EINVAL or WINATTN_ELAUNCH. */
int attn_read_probe(const void* src, size_t bytes, float* sink, void* stream);

/* Tuning knobs for tests and benchmarks (process-wide, not thread-safe; 0 = automatic).
 * They change the launch plan and therefore the workspace size: query the size after setting
 * them. */
#define WINATTN_TUNE_FORCE_KERNEL 1    /* kernel number as reported by attn_window_chunk_plan;
                                         6: the gated call's single launch where its width
                                         allows (chunk calls then plan as with 0) */
#define WINATTN_TUNE_TILES_PER_SPLIT 2 /* key tiles per split */
#define WINATTN_TUNE_TARGET_BLOCKS 3   /* workgroups the split count aims for (also the gated
                                         single launch's) */
#define WINATTN_TUNE_MERGE_KERNEL 4    /* 1 = splits merge in the last split, 2 = separate launch */
#define WINATTN_TUNE_XCD_MAP 5         /* matrix-core and encoder work order: 1 = round-robin, 2 = groups per XCD */
int attn_tuning_set(int knob, int value);

/* A static, human-readable description of a return code. */
const char* attn_strerror(int code);

/* WINATTN_ABI_VERSION of the built library. */
int attn_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* WINATTN_H */
