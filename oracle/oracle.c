/*
 * CPU oracle for windowed grouped-query attention over a ring buffer.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing on the product path may call, link or load this file:
 * only the tests, the smoke check and the benchmark's CPU-baseline leg use it. It shares no
 * code, header or table with the HIP library.
 *
 * It is the plain definition, written out in double precision with a two-pass softmax and an
 * explicit walk over each row's key list, rounding to f32 only where a value is stored
 * (the output, the ring slots). Sources:
 *
 *  - o1c page ("A sealed layer's attention for a chunk of rows, on Metal", crate cortiq-engine
 *    0.8.79): the layout header comment; `wgf` (per-group window override); `o1c_score` (a row's
 *    window over the ring then the chunk's rows up to its own); `o1c_max`, `o1c_soft`, `o1c_sum`,
 *    `o1c_add` (max, exp, 1/sum, value sum). oracle_window_chunk takes the far-field landmark
 *    terms with zero landmarks, so the far mass and far numerators vanish and the near softmax
 *    is its result.
 *  - dory page ("Dory's token path", crate cortiq-engine 0.8.57): `dory_prep` (rotation, unit
 *    heads, query scale, ring write), `low_key`, `dory_score`, `dory_soft`, `dory_sum`, `dory_gate`;
 *    the one-row far-field form `dory_os` .. `dory_ogate` (oracle_window_gated_far).
 *  - o1c far field and commits (oracle_window_commit, oracle_window_chunk_far,
 *    oracle_window_commit_far): see the comments at those functions.
 *  - egemma2 page (`eg_flash_body`, `eg_softmax`): encoder attention over packed sequences
 *    (oracle_encoder_attention).
 *
 * Readings where the pages leave a step open are listed in the design notes; the ones that
 * matter here: a window of wg keys ends at and includes the row itself; the RoPE table is an
 * input; eps is added to the sum of squares inside the square root; every row's prep and ring
 * write happens before any row attends.
 *
 * Return codes: 0 on success, -1 on invalid arguments or meta.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Per-group window: a non-zero override in meta field 3 replaces the default w (`wgf`). */
static uint32_t group_window(const uint32_t *meta, int g, int w) {
    uint32_t ov = meta[4 * g + 3];
    return ov != 0u ? ov : (uint32_t)w;
}

static int meta_ok(const uint32_t *meta, int ng, int w) {
    for (int g = 0; g < ng; ++g) {
        uint32_t wg = group_window(meta, g, w);
        uint32_t len0 = meta[4 * g], head0 = meta[4 * g + 1];
        if (wg > (uint32_t)w || len0 > wg) return 0;
        if (len0 > 0 && head0 >= wg) return 0;
    }
    return 1;
}

/*
 * Key list of chunk row i in group g, as pointers to K and V rows, in order: the ns sinks,
 * then the window's logical entries oldest to newest. Logical entry x < len0 is ring entry x,
 * stored at slot (head0 + x) mod wg of the group's ring (stride w); x >= len0 is chunk row
 * x - len0. The window is the last min(wg, len0 + i + 1) entries up to and including row i
 * (`o1c_score`). Returns the number of keys.
 */
static int key_list(const float *ring_k, const float *ring_v, const uint32_t *meta,
                    const float *sink_k, const float *sink_v, const float *chunk_k,
                    const float *chunk_v, int ng, int d, int w, int ns, int g, int i,
                    const float **kp, const float **vp) {
    uint32_t wg = group_window(meta, g, w);
    uint32_t len0 = meta[4 * g], head0 = meta[4 * g + 1];
    uint32_t end = len0 + (uint32_t)i + 1u;            /* one past the row's own entry */
    uint32_t win = wg < end ? wg : end;
    int n = 0;
    for (int s = 0; s < ns; ++s) {
        kp[n] = sink_k + ((size_t)g * ns + s) * d;
        vp[n] = sink_v + ((size_t)g * ns + s) * d;
        ++n;
    }
    for (uint32_t x = end - win; x < end; ++x) {
        if (x < len0) {
            size_t slot = (size_t)((head0 + x) % wg);
            kp[n] = ring_k + ((size_t)g * w + slot) * d;
            vp[n] = ring_v + ((size_t)g * w + slot) * d;
        } else {
            size_t row = (size_t)(x - len0);
            kp[n] = chunk_k + (row * ng + g) * d;
            vp[n] = chunk_v + (row * ng + g) * d;
        }
        ++n;
    }
    return n;
}

/*
 * Exact softmax attention of one query over n keys, in double:
 * s_j = scale * <q, K_j>; m = max s_j; p_j = exp(s_j - m); out = sum_j p_j V_j / sum_j p_j.
 * `qd` is the query in double. `wts` (n doubles) receives the normalised weights if non-NULL.
 */
static void attend(const double *qd, const float *const *kp, const float *const *vp, int n,
                   int d, double scale, double *sc, double *acc, double *wts) {
    double m = -INFINITY;
    for (int j = 0; j < n; ++j) {
        double dot = 0.0;
        for (int e = 0; e < d; ++e) dot += qd[e] * (double)kp[j][e];
        sc[j] = scale * dot;
        if (sc[j] > m) m = sc[j];
    }
    double l = 0.0;
    for (int j = 0; j < n; ++j) {
        sc[j] = exp(sc[j] - m);
        l += sc[j];
    }
    for (int e = 0; e < d; ++e) acc[e] = 0.0;
    for (int j = 0; j < n; ++j)
        for (int e = 0; e < d; ++e) acc[e] += sc[j] * (double)vp[j][e];
    for (int e = 0; e < d; ++e) acc[e] /= l;
    if (wts)
        for (int j = 0; j < n; ++j) wts[j] = sc[j] / l;
}

static int chunk_args_ok(const float *ring_k, const float *ring_v, const uint32_t *meta,
                         const float *sink_k, const float *sink_v, const float *q,
                         const float *chunk_k, const float *chunk_v, int rows, int ng, int hpg,
                         int d, int w, int ns) {
    if (rows < 1 || ng < 1 || hpg < 1 || d < 1 || w < 1 || ns < 0) return 0;
    if (!ring_k || !ring_v || !meta || !q || !chunk_k || !chunk_v) return 0;
    if (ns > 0 && (!sink_k || !sink_v)) return 0;
    return meta_ok(meta, ng, w);
}

/* One output vector: chunk row i, query head gh = g*hpg + h (heads of a group are contiguous). */
static void chunk_one(const float *ring_k, const float *ring_v, const uint32_t *meta,
                      const float *sink_k, const float *sink_v, const float *q,
                      const float *chunk_k, const float *chunk_v, int ng, int hpg, int d, int w,
                      int ns, double scale, int i, int gh, float *out_vec, double *wts,
                      int *nkeys) {
    int nh = ng * hpg, g = gh / hpg;
    int cap = ns + w;
    const float **kp = (const float **)malloc(sizeof(float *) * (size_t)cap);
    const float **vp = (const float **)malloc(sizeof(float *) * (size_t)cap);
    double *sc = (double *)malloc(sizeof(double) * (size_t)cap);
    double *acc = (double *)malloc(sizeof(double) * (size_t)d);
    double *qd = (double *)calloc((size_t)d, sizeof(double));
    int n = key_list(ring_k, ring_v, meta, sink_k, sink_v, chunk_k, chunk_v, ng, d, w, ns, g, i,
                     kp, vp);
    const float *qv = q + ((size_t)i * nh + gh) * d;
    for (int e = 0; e < d; ++e) qd[e] = (double)qv[e];
    attend(qd, kp, vp, n, d, scale, sc, acc, wts);
    if (out_vec)
        for (int e = 0; e < d; ++e) out_vec[e] = (float)acc[e];
    if (nkeys) *nkeys = n;
    free(kp); free(vp); free(sc); free(acc); free(qd);
}

/* The full chunk call: out[rows][nh][d]. Parallel over (row, query head). */
int oracle_window_chunk(const float *ring_k, const float *ring_v, const uint32_t *meta,
                        const float *sink_k, const float *sink_v, const float *q,
                        const float *chunk_k, const float *chunk_v, float *out, int rows, int ng,
                        int hpg, int d, int w, int ns, float scale) {
    if (!chunk_args_ok(ring_k, ring_v, meta, sink_k, sink_v, q, chunk_k, chunk_v, rows, ng, hpg,
                       d, w, ns) || !out)
        return -1;
    int nh = ng * hpg;
    long total = (long)rows * nh;
#pragma omp parallel for schedule(dynamic, 1)
    for (long t = 0; t < total; ++t) {
        int i = (int)(t / nh), gh = (int)(t % nh);
        chunk_one(ring_k, ring_v, meta, sink_k, sink_v, q, chunk_k, chunk_v, ng, hpg, d, w, ns,
                  (double)scale, i, gh, out + (size_t)t * d, NULL, NULL);
    }
    return 0;
}

/* Selected outputs only: out_sel[k][d] for (sel_rows[k], sel_heads[k]), k < nsel. */
int oracle_window_chunk_select(const float *ring_k, const float *ring_v, const uint32_t *meta,
                               const float *sink_k, const float *sink_v, const float *q,
                               const float *chunk_k, const float *chunk_v, int rows, int ng,
                               int hpg, int d, int w, int ns, float scale, const int32_t *sel_rows,
                               const int32_t *sel_heads, int nsel, float *out_sel) {
    if (!chunk_args_ok(ring_k, ring_v, meta, sink_k, sink_v, q, chunk_k, chunk_v, rows, ng, hpg,
                       d, w, ns) || !out_sel || nsel < 0 || (nsel > 0 && (!sel_rows || !sel_heads)))
        return -1;
    for (int k = 0; k < nsel; ++k)
        if (sel_rows[k] < 0 || sel_rows[k] >= rows || sel_heads[k] < 0 || sel_heads[k] >= ng * hpg)
            return -1;
#pragma omp parallel for schedule(dynamic, 1)
    for (int k = 0; k < nsel; ++k)
        chunk_one(ring_k, ring_v, meta, sink_k, sink_v, q, chunk_k, chunk_v, ng, hpg, d, w, ns,
                  (double)scale, sel_rows[k], sel_heads[k], out_sel + (size_t)k * d, NULL, NULL);
    return 0;
}

/*
 * The normalised softmax weights of one (row, query head), in key-list order (sinks, then the
 * window oldest to newest). `wts` must hold ns + w doubles. Returns the key count, or -1.
 */
int oracle_window_chunk_weights(const float *ring_k, const float *ring_v, const uint32_t *meta,
                                const float *sink_k, const float *sink_v, const float *q,
                                const float *chunk_k, const float *chunk_v, int rows, int ng,
                                int hpg, int d, int w, int ns, float scale, int row, int gh,
                                double *wts) {
    if (!chunk_args_ok(ring_k, ring_v, meta, sink_k, sink_v, q, chunk_k, chunk_v, rows, ng, hpg,
                       d, w, ns) || !wts || row < 0 || row >= rows || gh < 0 || gh >= ng * hpg)
        return -1;
    int n = 0;
    chunk_one(ring_k, ring_v, meta, sink_k, sink_v, q, chunk_k, chunk_v, ng, hpg, d, w, ns,
              (double)scale, row, gh, NULL, wts, &n);
    return n;
}

/*
 * Rotate-half RoPE and L2 normalisation of one head vector (`dory_prep`): with x, y the two
 * halves of the raw head and c, s the halves of the table row, u = x c - y s, v = y c + x s,
 * inv = 1 / sqrt(sum u^2 + sum v^2 + eps); result (u, v) * inv, in double.
 */
static void rotate_unit(const float *raw, const float *rope_row, int hd, double eps, double *res) {
    int half = hd / 2;
    double ss = 0.0;
    for (int e = 0; e < half; ++e) {
        double x = raw[e], y = raw[half + e];
        double c = rope_row[e], s = rope_row[half + e];
        double u = x * c - y * s, v = y * c + x * s;
        res[e] = u;
        res[half + e] = v;
        ss += u * u + v * v;
    }
    double inv = 1.0 / sqrt(ss + eps);
    for (int e = 0; e < hd; ++e) res[e] *= inv;
}

/*
 * The gated call. First, for every row (position pos0 + row): each KV head's unit key and raw
 * value go to ring slot (pos0 + row) mod cap (rounded to f32 there). Then each query head a of
 * each row attends, with its unit query times the learned scale, over positions
 * [lo, pos] (`low_key`: lo = pos + 1 - window when pos + 1 > window, else 0), reading slot
 * j mod cap of KV head a / (nh / nk). Finally z = o / (1 + exp(-gate * gate_scale)) (`dory_gate`).
 * ring_k / ring_v are updated in place; out is z [rows][nh][hd].
 */
int oracle_window_gated(const float *yq, const float *yk, const float *yv, const float *rope,
                        const float *q_scale, const float *gate, const float *gate_scale,
                        float *ring_k, float *ring_v, float *out, int rows, int pos0, int cap,
                        int window, int nh, int nk, int hd, float scale, float eps) {
    if (rows < 1 || pos0 < 0 || cap < 1 || window < 1 || nh < 1 || nk < 1 || hd < 2 || hd % 2)
        return -1;
    if (nh % nk != 0 || cap < window + rows - 1) return -1;
    if (!yq || !yk || !yv || !rope || !q_scale || !gate || !gate_scale || !ring_k || !ring_v || !out)
        return -1;
    int hpg = nh / nk;
    double *tmp = (double *)malloc(sizeof(double) * (size_t)hd);
    for (int r = 0; r < rows; ++r) {
        size_t slot = (size_t)(((long)pos0 + r) % cap);
        for (int kh = 0; kh < nk; ++kh) {
            rotate_unit(yk + ((size_t)r * nk + kh) * hd, rope + (size_t)r * hd, hd, (double)eps, tmp);
            float *kd = ring_k + (slot * nk + kh) * hd;
            float *vd = ring_v + (slot * nk + kh) * hd;
            const float *vs = yv + ((size_t)r * nk + kh) * hd;
            for (int e = 0; e < hd; ++e) {
                kd[e] = (float)tmp[e];
                vd[e] = vs[e];
            }
        }
    }
    free(tmp);
    long total = (long)rows * nh;
#pragma omp parallel for schedule(dynamic, 1)
    for (long t = 0; t < total; ++t) {
        int r = (int)(t / nh), a = (int)(t % nh);
        int kh = a / hpg;
        long pos = (long)pos0 + r;
        long lo = pos + 1 > window ? pos + 1 - window : 0;
        int n = (int)(pos - lo + 1);
        const float **kp = (const float **)malloc(sizeof(float *) * (size_t)n);
        const float **vp = (const float **)malloc(sizeof(float *) * (size_t)n);
        double *sc = (double *)malloc(sizeof(double) * (size_t)n);
        double *acc = (double *)malloc(sizeof(double) * (size_t)hd);
        double *qd = (double *)malloc(sizeof(double) * (size_t)hd);
        for (int j = 0; j < n; ++j) {
            size_t slot = (size_t)((lo + j) % cap);
            kp[j] = ring_k + (slot * nk + kh) * hd;
            vp[j] = ring_v + (slot * nk + kh) * hd;
        }
        rotate_unit(yq + ((size_t)r * nh + a) * hd, rope + (size_t)r * hd, hd, (double)eps, qd);
        for (int e = 0; e < hd; ++e) qd[e] *= (double)q_scale[(size_t)a * hd + e];
        attend(qd, kp, vp, n, hd, (double)scale, sc, acc, NULL);
        float *z = out + ((size_t)r * nh + a) * hd;
        for (int e = 0; e < hd; ++e) {
            size_t ge = (size_t)a * hd + e;
            double gs = (double)gate[(size_t)r * nh * hd + ge] * (double)gate_scale[ge];
            z[e] = (float)(acc[e] / (1.0 + exp(-gs)));
        }
        free(kp); free(vp); free(sc); free(acc); free(qd);
    }
    return 0;
}

/*
 * The state after a chunk (o1c page: `o1c_ring_commit` writes the chunk's K/V rows into the
 * ring, `o1c_meta` advances length, head and the far count; `o1c_tok_commit` is the one-row
 * form). Written here as its plain definition: the rows are pushed one at a time, oldest first.
 * A push lands in slot (head + len) mod wg; while the ring is not full its length grows,
 * otherwise the oldest entry is evicted: the slot is the head's, the head moves on by one and
 * the far count (meta field 2) grows by one. Reading for a chunk longer than the window: the
 * pushes are sequential, so only the chunk's last wg rows remain.
 * ring_k, ring_v [ng][w][d] and meta [ng][4] are updated in place.
 */
int oracle_window_commit(float *ring_k, float *ring_v, uint32_t *meta, const float *chunk_k,
                         const float *chunk_v, int rows, int ng, int d, int w) {
    if (!ring_k || !ring_v || !meta || !chunk_k || !chunk_v) return -1;
    if (rows < 1 || ng < 1 || d < 1 || w < 1) return -1;
    if (!meta_ok(meta, ng, w)) return -1;
    for (int g = 0; g < ng; ++g) {
        const uint32_t wg = group_window(meta, g, w);
        uint32_t len = meta[4 * g], head = meta[4 * g + 1], far = meta[4 * g + 2];
        if (len == 0) head %= wg;   /* an empty ring's head may be any value */
        int evicted = 0;
        for (int j = 0; j < rows; ++j) {
            const uint32_t slot = (uint32_t)(((uint64_t)head + len) % wg);
            const float *ks = chunk_k + ((size_t)j * ng + g) * d;
            const float *vs = chunk_v + ((size_t)j * ng + g) * d;
            float *kd = ring_k + ((size_t)g * w + slot) * d;
            float *vd = ring_v + ((size_t)g * w + slot) * d;
            memcpy(kd, ks, sizeof(float) * (size_t)d);
            memcpy(vd, vs, sizeof(float) * (size_t)d);
            if (len < wg) {
                len += 1;
            } else {
                head = (head + 1) % wg;
                far += 1;
                evicted = 1;
            }
        }
        meta[4 * g] = len;
        if (evicted) {   /* as `o1c_meta`: the head and far count change only on eviction */
            meta[4 * g + 1] = head;
            meta[4 * g + 2] = far;
        }
    }
    return 0;
}

/*
 * The far field (o1c page: `o1c_far_e`, `o1c_land`, `o1c_far`, `o1c_soft`, `o1c_add`,
 * `o1c_far_commit`; token path `o1c_tok_far`, `o1c_tok_merge`). Keys that have left a group's
 * window are summarised per query head gh by m landmarks: landmark b keeps a far max mx_b and
 * a far mass z_b (mz [gh][2m]: maxima then masses) and a far numerator t_hat_b [d], the sums of
 * exp(s - mx_b) and exp(s - mx_b) V over the evicted keys, s = scale <q_tilde_b, K> with the
 * landmark's own query q_tilde [gh][m][d]. A row's query reads them through landmark keys
 * k_tilde [g][m][d] and a mixing matrix mu [gh][m][m] (row a, column b).
 *
 * Evictions inside the chunk: chunk row j >= j0 = wg - len0 pushes out the oldest entry, the
 * group's logical entry x = j - j0 (ring slot (head0 + x) mod wg while x < len0; reading for a
 * chunk longer than the window: a later entry x >= len0 is chunk row x - len0).
 */

/* Evicted entry of chunk row j (j >= j0): its K and V rows. */
static void evicted_entry(const float *ring_k, const float *ring_v, const float *chunk_k,
                          const float *chunk_v, uint32_t len0, uint32_t head0, uint32_t wg,
                          int ng, int d, int w, int g, uint32_t x, const float **k,
                          const float **v) {
    if (x < len0) {
        const size_t slot = (size_t)(head0 + x) % (size_t)wg;
        *k = ring_k + ((size_t)g * w + slot) * d;
        *v = ring_v + ((size_t)g * w + slot) * d;
    } else {
        size_t row = (size_t)(x - len0);
        *k = chunk_k + (row * ng + g) * d;
        *v = chunk_v + (row * ng + g) * d;
    }
}

/*
 * Eviction scores of one landmark (`o1c_far_e`): for the chunk's evicting rows j in [j0, rows),
 * e[j] = exp(fe_j - mx) with fe_j = scale <q_tilde, K_ev(j)>, mx = max(old max, fe_j), the
 * rescale r = exp(old max - mx) of the old mass and numerator (1 if the max did not move: an
 * empty far field starts at -inf), and z[i] = old mass r + sum_{j0 <= j <= i} e[j], the far mass
 * as of row i. e[j] = 0 for j < j0.
 */
static void far_evict(const float *ring_k, const float *ring_v, const float *chunk_k,
                      const float *chunk_v, uint32_t len0, uint32_t head0, uint32_t wg, int ng,
                      int d, int w, int g, int rows, const float *qt, double m_old, double mass,
                      double scale, double *e, double *z, double *mx_out, double *r_out) {
    const long j0 = (long)wg - (long)len0;
    double mx = m_old;
    for (long j = 0; j < rows; ++j) {
        e[j] = -INFINITY;
        if (j < j0) continue;
        const float *k, *v;
        evicted_entry(ring_k, ring_v, chunk_k, chunk_v, len0, head0, wg, ng, d, w, g,
                      (uint32_t)(j - j0), &k, &v);
        double dot = 0.0;
        for (int c = 0; c < d; ++c) dot += (double)qt[c] * (double)k[c];
        e[j] = scale * dot;
        if (e[j] > mx) mx = e[j];
    }
    const double r = mx == m_old ? 1.0 : exp(m_old - mx);
    double acc = mass * r;
    for (long j = 0; j < rows; ++j) {
        e[j] = j >= j0 ? exp(e[j] - mx) : 0.0;
        acc += e[j];
        z[j] = acc;
    }
    *mx_out = mx;
    *r_out = r;
}

static int far_args_ok(const float *k_tilde, const float *q_tilde, const float *mu,
                       const float *mz, const float *t_hat, int m) {
    return k_tilde && q_tilde && mu && mz && t_hat && m >= 1;
}

/*
 * Chunk attention with the far field: out [rows][nh][d]. Row i of head gh (`o1c_far`,
 * `o1c_soft`, `o1c_add`): the near scores over its sinks and window; if the far field is
 * non-empty as of the row (far_len plus the chunk's evictions up to row i), landmark scores
 * fl_a = scale <q, k_tilde_a>, f = max fl, weights w_b = sum_a exp(fl_a - f) mu[a][b], the
 * common max c = max(near max, f + mx_b), gains g_b = w_b exp(f + mx_b - c), far mass
 * F = sum_b g_b z_b(i); if F < 0 the far part is dropped. Then
 * out = (sum_near exp(s - c) V + sum_b g_b r_b t_hat_b + sum_{j0<=j<=i} (sum_b g_b e_b(j)) V_ev(j))
 *       / (sum_near exp(s - c) + F).
 */
int oracle_window_chunk_far(const float *ring_k, const float *ring_v, const uint32_t *meta,
                            const float *sink_k, const float *sink_v, const float *q,
                            const float *chunk_k, const float *chunk_v, const float *k_tilde,
                            const float *q_tilde, const float *mu, const float *mz,
                            const float *t_hat, float *out, int rows, int ng, int hpg, int d,
                            int w, int ns, int m, float scale) {
    if (!out || !chunk_args_ok(ring_k, ring_v, meta, sink_k, sink_v, q, chunk_k, chunk_v, rows,
                               ng, hpg, d, w, ns))
        return -1;
    if (!far_args_ok(k_tilde, q_tilde, mu, mz, t_hat, m)) return -1;
    const int nh = ng * hpg;
    const double sc = (double)scale;
    int bad = 0;
#pragma omp parallel for collapse(2) schedule(dynamic)
    for (int g = 0; g < ng; ++g) {
        for (int h = 0; h < hpg; ++h) {
            const uint32_t wg = group_window(meta, g, w);
            const uint32_t len0 = meta[4 * g], head0 = meta[4 * g + 1], far0 = meta[4 * g + 2];
            const long j0 = (long)wg - (long)len0;
            const int gh = g * hpg + h;
            const size_t nmax = (size_t)ns + wg;
            const float **kp = malloc(sizeof(*kp) * nmax);
            const float **vp = malloc(sizeof(*vp) * nmax);
            double *s = malloc(sizeof(double) * nmax);
            double *acc = malloc(sizeof(double) * (size_t)d);
            double *qd = malloc(sizeof(double) * (size_t)d);
            double *e = malloc(sizeof(double) * (size_t)m * rows);
            double *z = malloc(sizeof(double) * (size_t)m * rows);
            double *mx = malloc(sizeof(double) * (size_t)m);
            double *r = malloc(sizeof(double) * (size_t)m);
            double *fl = malloc(sizeof(double) * (size_t)m);
            double *wb = malloc(sizeof(double) * (size_t)m);
            double *gb = malloc(sizeof(double) * (size_t)m);
            if (!kp || !vp || !s || !acc || !qd || !e || !z || !mx || !r || !fl || !wb || !gb) {
#pragma omp atomic write
                bad = 1;
            } else {
                for (int b = 0; b < m; ++b)
                    far_evict(ring_k, ring_v, chunk_k, chunk_v, len0, head0, wg, ng, d, w, g,
                              rows, q_tilde + ((size_t)gh * m + b) * d,
                              (double)mz[(size_t)gh * 2 * m + b],
                              (double)mz[(size_t)gh * 2 * m + m + b], sc, e + (size_t)b * rows,
                              z + (size_t)b * rows, &mx[b], &r[b]);
                for (int i = 0; i < rows; ++i) {
                    const float *qrow = q + ((size_t)i * nh + gh) * d;
                    for (int c = 0; c < d; ++c) qd[c] = (double)qrow[c];
                    const int n = key_list(ring_k, ring_v, meta, sink_k, sink_v, chunk_k,
                                           chunk_v, ng, d, w, ns, g, i, kp, vp);
                    double cmax = -INFINITY;
                    for (int j = 0; j < n; ++j) {
                        double dot = 0.0;
                        for (int c = 0; c < d; ++c) dot += qd[c] * (double)kp[j][c];
                        s[j] = sc * dot;
                        if (s[j] > cmax) cmax = s[j];
                    }
                    const long farl = (long)far0 + (i >= j0 ? i - j0 + 1 : 0);
                    double far_den = 0.0;
                    int have = 0;
                    if (farl > 0) {
                        double f = -INFINITY;
                        for (int a = 0; a < m; ++a) {
                            const float *kt = k_tilde + ((size_t)g * m + a) * d;
                            double dot = 0.0;
                            for (int c = 0; c < d; ++c) dot += qd[c] * (double)kt[c];
                            fl[a] = sc * dot;
                            if (fl[a] > f) f = fl[a];
                        }
                        for (int b = 0; b < m; ++b) wb[b] = 0.0;
                        for (int a = 0; a < m; ++a) {
                            const double ea = exp(fl[a] - f);
                            for (int b = 0; b < m; ++b)
                                wb[b] += ea * (double)mu[((size_t)gh * m + a) * m + b];
                        }
                        for (int b = 0; b < m; ++b)
                            if (f + mx[b] > cmax) cmax = f + mx[b];
                        for (int b = 0; b < m; ++b) {
                            gb[b] = wb[b] * exp(f + mx[b] - cmax);
                            far_den += gb[b] * z[(size_t)b * rows + i];
                        }
                        if (far_den >= 0.0) have = 1; else far_den = 0.0;
                    }
                    double den = far_den;
                    for (int c = 0; c < d; ++c) acc[c] = 0.0;
                    for (int j = 0; j < n; ++j) {
                        const double p = exp(s[j] - cmax);
                        den += p;
                        for (int c = 0; c < d; ++c) acc[c] += p * (double)vp[j][c];
                    }
                    if (have) {
                        for (int b = 0; b < m; ++b) {
                            const float *th = t_hat + ((size_t)gh * m + b) * d;
                            for (int c = 0; c < d; ++c) acc[c] += gb[b] * r[b] * (double)th[c];
                        }
                        for (long j = j0 < 0 ? 0 : j0; j <= i; ++j) {
                            double cf = 0.0;
                            for (int b = 0; b < m; ++b) cf += gb[b] * e[(size_t)b * rows + j];
                            const float *kk, *vv;
                            evicted_entry(ring_k, ring_v, chunk_k, chunk_v, len0, head0, wg, ng,
                                          d, w, g, (uint32_t)(j - j0), &kk, &vv);
                            for (int c = 0; c < d; ++c) acc[c] += cf * (double)vv[c];
                        }
                    }
                    if (den < 1e-30) den = 1e-30;
                    float *o = out + ((size_t)i * nh + gh) * d;
                    for (int c = 0; c < d; ++c) o[c] = (float)(acc[c] / den);
                }
            }
            free(kp); free(vp); free(s); free(acc); free(qd); free(e); free(z); free(mx);
            free(r); free(fl); free(wb); free(gb);
        }
    }
    return bad ? -1 : 0;
}

/*
 * The far state after the chunk (`o1c_far_commit`), then the ring commit and meta advance:
 * for every head gh and landmark b with evictions in the chunk, t_hat_b <- t_hat_b r_b +
 * sum_{j >= j0} e_b(j) V_ev(j), far max <- mx_b, far mass <- z_b(rows - 1). mz and t_hat are
 * updated in place; then oracle_window_commit (which also adds the evictions to far_len).
 */
int oracle_window_commit_far(float *ring_k, float *ring_v, uint32_t *meta, const float *chunk_k,
                             const float *chunk_v, const float *q_tilde, float *mz,
                             float *t_hat, int rows, int ng, int hpg, int d, int w, int m,
                             float scale) {
    if (!ring_k || !ring_v || !meta || !chunk_k || !chunk_v || !q_tilde || !mz || !t_hat)
        return -1;
    if (rows < 1 || ng < 1 || hpg < 1 || d < 1 || w < 1 || m < 1) return -1;
    if (!meta_ok(meta, ng, w)) return -1;
    double *e = malloc(sizeof(double) * (size_t)rows);
    double *z = malloc(sizeof(double) * (size_t)rows);
    double *acc = malloc(sizeof(double) * (size_t)d);
    if (!e || !z || !acc) { free(e); free(z); free(acc); return -1; }
    for (int g = 0; g < ng; ++g) {
        const uint32_t wg = group_window(meta, g, w);
        const uint32_t len0 = meta[4 * g], head0 = meta[4 * g + 1];
        const long j0 = (long)wg - (long)len0;
        if (j0 >= rows) continue;   /* nothing evicted */
        for (int h = 0; h < hpg; ++h) {
            const int gh = g * hpg + h;
            for (int b = 0; b < m; ++b) {
                double mx, r;
                float *mzb = mz + (size_t)gh * 2 * m;
                far_evict(ring_k, ring_v, chunk_k, chunk_v, len0, head0, wg, ng, d, w, g, rows,
                          q_tilde + ((size_t)gh * m + b) * d, (double)mzb[b],
                          (double)mzb[m + b], (double)scale, e, z, &mx, &r);
                float *th = t_hat + ((size_t)gh * m + b) * d;
                for (int c = 0; c < d; ++c) acc[c] = (double)th[c] * r;
                for (long j = j0 < 0 ? 0 : j0; j < rows; ++j) {
                    const float *kk, *vv;
                    evicted_entry(ring_k, ring_v, chunk_k, chunk_v, len0, head0, wg, ng, d, w,
                                  g, (uint32_t)(j - j0), &kk, &vv);
                    for (int c = 0; c < d; ++c) acc[c] += e[j] * (double)vv[c];
                }
                for (int c = 0; c < d; ++c) th[c] = (float)acc[c];
                mzb[b] = (float)mx;
                mzb[m + b] = (float)z[rows - 1];
            }
        }
    }
    free(e); free(z); free(acc);
    return oracle_window_commit(ring_k, ring_v, meta, chunk_k, chunk_v, rows, ng, d, w);
}

/*
 * The gated one-row call with the far field (dory page: `dory_os`, `dory_ol`, `dory_omax`,
 * `dory_ofar`, `dory_osoft`, `dory_osum`, `dory_ogate`). The row's own key is already in the
 * ring, so query head gh (KV head kh = gh / hpg) attends over the ns sinks of kh and ring slots
 * 0 .. len-1 of kh (len = meta[kh] field 0; storage order does not matter), with scores
 * s = scale <q, K>. When the far count (meta field 2) is non-zero, the landmark part joins:
 * fl_a = scale <q, k_tilde[kh][a]>, f = max fl, u_b = sum_a exp(fl_a - f) mu[gh][a][b] (clamped
 * at 0 when rect is non-zero), c = max(max s, f + mx_b) with mx_b = mz[gh][b], gains
 * G_b = u_b exp(f + mx_b - c), far mass F = sum_b G_b mz[gh][m + b]; the far terms are kept when
 * F >= 0. Then
 *   out = (sum exp(s - c) V + sum_b G_b t_hat_b) / max(sum exp(s - c) + F, 1e-30)
 *         / (1 + exp(-gate * gate_scale)).
 * Layouts: q [nh][hd]; ring_k, ring_v [nk][w][hd]; sink_k, sink_v [nk][ns][hd]; meta [nk][4];
 * k_tilde [nk][m][hd]; mu [nh][m][m]; mz [nh][2m]; t_hat [nh][m][hd]; gate, gate_scale
 * [nh * hd]; out [nh][hd].
 */
int oracle_window_gated_far(const float *q, const float *ring_k, const float *ring_v,
                            const uint32_t *meta, const float *sink_k, const float *sink_v,
                            const float *k_tilde, const float *mu, const float *mz,
                            const float *t_hat, const float *gate, const float *gate_scale,
                            float *out, int nh, int nk, int hd, int w, int ns, int m, float scale,
                            int rect) {
    if (!q || !ring_k || !ring_v || !meta || !k_tilde || !mu || !mz || !t_hat || !gate ||
        !gate_scale || !out)
        return -1;
    if (nh < 1 || nk < 1 || nh % nk != 0 || hd < 1 || w < 1 || ns < 0 || m < 1) return -1;
    if (ns > 0 && (!sink_k || !sink_v)) return -1;
    for (int kh = 0; kh < nk; ++kh)
        if (meta[4 * kh] > (uint32_t)w) return -1;
    const int hpg = nh / nk;
    const double sc = (double)scale;
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1)
    for (int gh = 0; gh < nh; ++gh) {
        const int kh = gh / hpg;
        const int len = (int)meta[4 * kh], far = (int)meta[4 * kh + 2];
        const int n = ns + len;
        double *s = malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
        double *acc = malloc(sizeof(double) * (size_t)hd);
        double *fl = malloc(sizeof(double) * (size_t)m);
        double *u = malloc(sizeof(double) * (size_t)m);
        double *gb = malloc(sizeof(double) * (size_t)m);
        if (!s || !acc || !fl || !u || !gb) {
#pragma omp atomic write
            bad = 1;
        } else {
            const float *qv = q + (size_t)gh * hd;
            double cmax = -INFINITY;
            for (int j = 0; j < n; ++j) {
                const float *k = j < ns ? sink_k + ((size_t)kh * ns + j) * hd
                                        : ring_k + ((size_t)kh * w + (j - ns)) * hd;
                double dot = 0.0;
                for (int e = 0; e < hd; ++e) dot += (double)qv[e] * (double)k[e];
                s[j] = sc * dot;
                if (s[j] > cmax) cmax = s[j];
            }
            double far_den = 0.0;
            int have = 0;
            if (far > 0) {
                double f = -INFINITY;
                for (int a = 0; a < m; ++a) {
                    const float *kt = k_tilde + ((size_t)kh * m + a) * hd;
                    double dot = 0.0;
                    for (int e = 0; e < hd; ++e) dot += (double)qv[e] * (double)kt[e];
                    fl[a] = sc * dot;
                    if (fl[a] > f) f = fl[a];
                }
                for (int b = 0; b < m; ++b) u[b] = 0.0;
                for (int a = 0; a < m; ++a) {
                    const double ea = exp(fl[a] - f);
                    for (int b = 0; b < m; ++b) u[b] += ea * (double)mu[((size_t)gh * m + a) * m + b];
                }
                if (rect)
                    for (int b = 0; b < m; ++b) if (u[b] < 0.0) u[b] = 0.0;
                const float *mzh = mz + (size_t)gh * 2 * m;
                for (int b = 0; b < m; ++b)
                    if (f + (double)mzh[b] > cmax) cmax = f + (double)mzh[b];
                for (int b = 0; b < m; ++b) {
                    gb[b] = u[b] * exp(f + (double)mzh[b] - cmax);
                    far_den += gb[b] * (double)mzh[m + b];
                }
                have = far_den >= 0.0;   /* a negative far mass drops the far terms */
                if (!have) far_den = 0.0;
            }
            double den = far_den;
            for (int e = 0; e < hd; ++e) acc[e] = 0.0;
            for (int j = 0; j < n; ++j) {
                const float *v = j < ns ? sink_v + ((size_t)kh * ns + j) * hd
                                        : ring_v + ((size_t)kh * w + (j - ns)) * hd;
                const double p = exp(s[j] - cmax);
                den += p;
                for (int e = 0; e < hd; ++e) acc[e] += p * (double)v[e];
            }
            if (have)
                for (int b = 0; b < m; ++b) {
                    const float *th = t_hat + ((size_t)gh * m + b) * hd;
                    for (int e = 0; e < hd; ++e) acc[e] += gb[b] * (double)th[e];
                }
            if (den < 1e-30) den = 1e-30;
            float *z = out + (size_t)gh * hd;
            for (int e = 0; e < hd; ++e) {
                const size_t ge = (size_t)gh * hd + e;
                const double gs = (double)gate[ge] * (double)gate_scale[ge];
                z[e] = (float)(acc[e] / den / (1.0 + exp(-gs)));
            }
        }
        free(s); free(acc); free(fl); free(u); free(gb);
    }
    return bad ? -1 : 0;
}

/*
 * Encoder attention over packed variable-length sequences (egemma2 page: `eg_flash_body`,
 * `eg_flash64`, `eg_flash64s` for whole sequences, `EgAtt` / `eg_softmax` for the symmetric
 * window). Sequence s holds tokens start_s .. start_s + len_s - 1 (segs[2s], segs[2s+1]); the
 * token at position i of its sequence attends, with query head h, to the keys and values of KV
 * head h / (nh / nk) at positions j of the same sequence with |i - j| <= window (window 0: all
 * positions), scores scale <q, k>, no causal mask. Row t of q, k, v, out starts at t * ldq,
 * t * ldk, t * ldv, t * ldo floats; head h's hd values follow at h * hd. Rows of out outside
 * every sequence are not written.
 */
int oracle_encoder_attention(const float *q, const float *k, const float *v, float *out,
                             const uint32_t *segs, int nseg, int ldq, int ldk, int ldv,
                             int ldo, int nh, int nk, int hd, int window, float scale) {
    if (!q || !k || !v || !out || !segs || nseg < 0 || nh < 1 || nk < 1 || nh % nk != 0 ||
        hd < 1 || window < 0)
        return -1;
    if (ldq < nh * hd || ldk < nk * hd || ldv < nk * hd || ldo < nh * hd) return -1;
    const int group = nh / nk;
    long total = 0;
    for (int s = 0; s < nseg; ++s) total += (long)segs[2 * s + 1] * nh;
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 16)
    for (long it = 0; it < total; ++it) {
        /* item -> (sequence, position, head) */
        long rem = it;
        int s = 0;
        while (rem >= (long)segs[2 * s + 1] * nh) {
            rem -= (long)segs[2 * s + 1] * nh;
            ++s;
        }
        const long start = segs[2 * s], len = segs[2 * s + 1];
        const long i = rem / nh;
        const int h = (int)(rem % nh), kvh = h / group;
        long lo = 0, hi = len;
        if (window > 0) {
            lo = i > window ? i - window : 0;
            hi = i + window + 1 < len ? i + window + 1 : len;
        }
        const int n = (int)(hi - lo);
        const float **kp = malloc(sizeof(*kp) * (size_t)n);
        const float **vp = malloc(sizeof(*vp) * (size_t)n);
        double *sc = malloc(sizeof(double) * (size_t)n);
        double *acc = malloc(sizeof(double) * (size_t)hd);
        double *qd = malloc(sizeof(double) * (size_t)hd);
        if (!kp || !vp || !sc || !acc || !qd) {
#pragma omp atomic write
            bad = 1;
        } else {
            for (int j = 0; j < n; ++j) {
                kp[j] = k + (size_t)(start + lo + j) * ldk + (size_t)kvh * hd;
                vp[j] = v + (size_t)(start + lo + j) * ldv + (size_t)kvh * hd;
            }
            const float *qv = q + (size_t)(start + i) * ldq + (size_t)h * hd;
            for (int e = 0; e < hd; ++e) qd[e] = (double)qv[e];
            attend(qd, kp, vp, n, hd, (double)scale, sc, acc, NULL);
            float *o = out + (size_t)(start + i) * ldo + (size_t)h * hd;
            for (int e = 0; e < hd; ++e) o[e] = (float)acc[e];
        }
        free(kp); free(vp); free(sc); free(acc); free(qd);
    }
    return bad ? -1 : 0;
}

/* Threads the parallel loops of this library use (1 when built without OpenMP). */
int oracle_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Host-side meta validation with the same rules the oracle enforces (1 = valid). */
int oracle_meta_ok(const uint32_t *meta, int ng, int w) {
    if (!meta || ng < 1 || w < 1) return 0;
    return meta_ok(meta, ng, w);
}
