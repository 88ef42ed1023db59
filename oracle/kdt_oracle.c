/*
 * kdt_oracle.c -- fp64 CPU oracle for tree-verify MLA-absorb attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU-baseline leg
 * of the benchmark may load this library.  It shares no code, header or constant with
 * the HIP library and includes no HIP header.
 *
 * What it computes (plain definitions, no blocking or reordering):
 *
 *  visibility -- "Validating the Native Engine", section "The Broader Context": the
 *    verify kernel applies visibility masking to the draft tree.  Node i sees itself and
 *    every ancestor on its root-to-node path, nothing else.  Bit j of word j/64 of row
 *    (b,i) is set iff node j lies on that path (LSB-first 64-bit words, W = ceil(N/64)).
 *    A row whose walk meets a parent outside [-1, j-1] is invalid: it is zeroed and
 *    counted.
 *
 *  attention -- "The Capstone Validation", section "Context and Motivation": the target
 *    verifies every drafted continuation in one batched pass, so each node must see
 *    exactly what an ordinary decode of its own path would see.  For row (b,i,h) the key
 *    set is the request's committed cache plus the visible tree nodes; with MLA absorption
 *    ("Validating the Native Engine", section "Input Knowledge Required": MLA's absorbed
 *    attention) every head shares the latent rows:
 *        s_k  = scale * (q_lat . ckv_k + q_rope . krope_k)
 *        out  = sum_k exp(s_k - max s) ckv_k / sum_k exp(s_k - max s)
 *    computed in fp64 over fp64 copies of the inputs.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Returns the number of invalid rows; masks is [B][N][W] with W = ceil(N/64). */
int64_t kdt_oracle_visibility(const int32_t *parents, int64_t B, int64_t N, uint64_t *masks)
{
    const int64_t W = (N + 63) / 64;
    int64_t bad = 0;
    for (int64_t b = 0; b < B; b++) {
        const int32_t *par = parents + b * N;
        for (int64_t i = 0; i < N; i++) {
            uint64_t *row = masks + (b * N + i) * W;
            memset(row, 0, (size_t)W * sizeof(uint64_t));
            int ok = 1;
            int64_t j = i;
            while (j != -1) {
                row[j / 64] |= (uint64_t)1 << (j % 64);
                int64_t p = par[j];
                if (p < -1 || p >= j) { ok = 0; break; }   /* parents must precede children */
                j = p;
            }
            if (!ok) {
                memset(row, 0, (size_t)W * sizeof(uint64_t));
                bad++;
            }
        }
    }
    return bad;
}

/*
 * Attention for selected rows.  All float arrays are fp64 and dense:
 *   q_lat [B*N*H][dc], q_rope [B*N*H][dr], ckv [T][dc], krope [T][dr],
 *   tree_ckv [B*N][dc], tree_krope [B*N][dr], masks [B*N][W], cache_lens [B].
 * rows[r] is a flat row id ((b*N + i)*H + h); nrows < 0 means every row in order.
 * out is [nrows][dc].  scale is the fp32 scale widened to fp64.
 */
void kdt_oracle_attention(const double *q_lat, const double *q_rope, const double *ckv,
                          const double *krope, const double *tree_ckv, const double *tree_krope,
                          const uint64_t *masks, const int32_t *cache_lens, int64_t B, int64_t N,
                          int64_t H, int64_t dc, int64_t dr, double scale, const int64_t *rows,
                          int64_t nrows, double *out, int nthreads)
{
    const int64_t W = (N + 63) / 64;
    int64_t *off = (int64_t *)malloc((size_t)(B + 1) * sizeof(int64_t));
    int64_t maxL = 0;
    off[0] = 0;
    for (int64_t b = 0; b < B; b++) {
        off[b + 1] = off[b] + cache_lens[b];
        if (cache_lens[b] > maxL) maxL = cache_lens[b];
    }
    const int64_t total = nrows < 0 ? B * N * H : nrows;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
#pragma omp parallel
    {
        double *s = (double *)malloc((size_t)(maxL + N + 1) * sizeof(double));
        const double **key = (const double **)malloc((size_t)(maxL + N + 1) * sizeof(double *));
#pragma omp for schedule(dynamic, 16)
        for (int64_t r = 0; r < total; r++) {
            const int64_t row = nrows < 0 ? r : rows[r];
            const int64_t bi = row / H;           /* (b*N + i) */
            const int64_t b = bi / N;
            const double *ql = q_lat + row * dc, *qr = q_rope + row * dr;
            const uint64_t *m = masks + bi * W;
            int64_t nk = 0;
            /* committed cache rows of request b */
            for (int64_t t = off[b]; t < off[b + 1]; t++) {
                double a = 0.0, c = 0.0;
                for (int64_t d = 0; d < dc; d++) a += ql[d] * ckv[t * dc + d];
                for (int64_t d = 0; d < dr; d++) c += qr[d] * krope[t * dr + d];
                s[nk] = scale * (a + c);
                key[nk++] = ckv + t * dc;
            }
            /* tree nodes visible to node i */
            for (int64_t j = 0; j < N; j++) {
                if (!((m[j / 64] >> (j % 64)) & 1u)) continue;
                const double *tl = tree_ckv + (b * N + j) * dc, *tr = tree_krope + (b * N + j) * dr;
                double a = 0.0, c = 0.0;
                for (int64_t d = 0; d < dc; d++) a += ql[d] * tl[d];
                for (int64_t d = 0; d < dr; d++) c += qr[d] * tr[d];
                s[nk] = scale * (a + c);
                key[nk++] = tl;
            }
            double *o = out + r * dc;
            for (int64_t d = 0; d < dc; d++) o[d] = 0.0;
            if (nk == 0) continue;               /* no visible key: output 0 */
            double mx = -INFINITY;
            for (int64_t k = 0; k < nk; k++) if (s[k] > mx) mx = s[k];
            double den = 0.0;
            for (int64_t k = 0; k < nk; k++) {
                const double w = exp(s[k] - mx);
                den += w;
                const double *v = key[k];
                for (int64_t d = 0; d < dc; d++) o[d] += w * v[d];
            }
            for (int64_t d = 0; d < dc; d++) o[d] /= den;
        }
        free(s);
        free(key);
    }
    free(off);
}
