/*
 * svla_oracle.c -- plain fp64 CPU oracle for block-causal ReLU linear attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no code,
 * header, table or helper with the HIP library; it is slow on purpose and
 * written so that each step can be checked against the statement of the
 * method by eye.
 *
 * What it computes, per (batch b, head h), following the statement of the
 * method on the SANA-Video pages:
 *   - Linear attention with a state of fixed size d x d (ICLR 2026 oral talk,
 *     "block KV cache" review: the state has shape D x D whatever the
 *     sequence length).
 *   - The state of block i is the previous block's state plus the current
 *     block's KV contribution (same talk, additive update of the cached
 *     state; abstract, design (2) "Constant-Memory KV cache").
 *   - Bidirectional inside a block, causal across blocks (talk, the
 *     description of the hybrid schedule: autoregressive over blocks,
 *     diffusion inside each block).
 *   - Optional per-block decay g of the carried state (SANA-Video 2.0 pages:
 *     "gated" linear attention layers), S_c = g_c * S_{c-1} + local_c.
 *   - Optional 3D RoPE on the numerator only (talk, architecture section on
 *     the changes made to the linear attention; comfyui-wiki model page,
 *     rotary position embeddings).
 *
 * Readings taken where the pages are silent (all documented in the design
 * notes of the repository):
 *   phi(x) = max(x, 0) on Q and K (never V); z = sum phi(k);
 *   O_i = (R_i phi(q_i))^T S_c / (phi(q_i) . z_c + eps), S[k][v] orientation;
 *   a block sees itself (inclusive state); z decays with the same g as S;
 *   RoPE: dims [0,dt) rotate with the frame index t, [dt,dt+dh) with the grid
 *   row h, [dt+dh,dt+dh+dw) with the grid column w; adjacent pairs
 *   (2m, 2m+1) inside each slice, theta_m = base^(-2m/d_slice), rotation by
 *   +angle, applied after the ReLU; token p of a call sits at frame
 *   t0 + p/(gh*gw), row (p/gw)%gh, column p%gw.
 *
 * Layouts: Q, K, V, O are [B,H,N,d] row-major (d fastest), N = nb*n.
 * S is [B,H,d,d] with S[k][v] (k = key feature, v = value feature), z is
 * [B,H,d], g is [B,H,nb].  All arrays are fp64.
 */
#include <math.h>
#include <stddef.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

typedef struct {
    int dt_dims, dh_dims, dw_dims;
    int grid_h, grid_w;
    int t0;
    double base;
} svlao_rope;

/* Rotate x (d entries, already through the ReLU) for the token at call
 * position p; dims past dt+dh+dw stay as they are. */
static void rope_rotate(const svlao_rope *r, long p, int d, const double *x,
                        double *y)
{
    long hw = (long)r->grid_h * r->grid_w;
    double pos[3];
    int width[3];
    pos[0] = (double)(r->t0 + p / hw);
    pos[1] = (double)((p / r->grid_w) % r->grid_h);
    pos[2] = (double)(p % r->grid_w);
    width[0] = r->dt_dims;
    width[1] = r->dh_dims;
    width[2] = r->dw_dims;
    memcpy(y, x, sizeof(double) * (size_t)d);
    int off = 0;
    for (int a = 0; a < 3; ++a) {
        for (int m = 0; 2 * m + 1 < width[a]; ++m) {
            double theta = pow(r->base, -2.0 * m / (double)width[a]);
            double ang = pos[a] * theta;
            double c = cos(ang), s = sin(ang);
            double x0 = x[off + 2 * m], x1 = x[off + 2 * m + 1];
            y[off + 2 * m] = x0 * c - x1 * s;
            y[off + 2 * m + 1] = x0 * s + x1 * c;
        }
        off += width[a];
    }
}

static double relu(double x) { return x > 0.0 ? x : 0.0; }

/*
 * One (b, h) pair.  Block by block: decay the carried state, add the block's
 * local contribution sum_j R_j phi(k_j) (x) v_j and sum_j phi(k_j), then read
 * every token of the block against the inclusive state.
 */
static void one_head(int nb, int n, int d, const double *Q, const double *K,
                     const double *V, const double *g, const svlao_rope *rope,
                     const double *S0, const double *z0, double eps,
                     double *O, double *S_out, double *z_out,
                     double *S_blocks, double *z_blocks,
                     double *S_local, double *z_local, double *den_out)
{
    size_t dd = (size_t)d * d;
    double *S = calloc(dd, sizeof(double));
    double *z = calloc((size_t)d, sizeof(double));
    double *Sl = calloc(dd, sizeof(double));
    double *zl = calloc((size_t)d, sizeof(double));
    double *a = malloc(sizeof(double) * (size_t)d);
    double *ar = malloc(sizeof(double) * (size_t)d);
    double *p = malloc(sizeof(double) * (size_t)d);
    double *pr = malloc(sizeof(double) * (size_t)d);
    if (S0) memcpy(S, S0, sizeof(double) * dd);
    if (z0) memcpy(z, z0, sizeof(double) * (size_t)d);

    for (int c = 0; c < nb; ++c) {
        /* local contribution of block c */
        memset(Sl, 0, sizeof(double) * dd);
        memset(zl, 0, sizeof(double) * (size_t)d);
        for (int j = 0; j < n; ++j) {
            long t = (long)c * n + j;
            const double *kj = K + t * d;
            const double *vj = V + t * d;
            for (int f = 0; f < d; ++f) a[f] = relu(kj[f]);
            if (rope) rope_rotate(rope, t, d, a, ar);
            else memcpy(ar, a, sizeof(double) * (size_t)d);
            for (int k = 0; k < d; ++k) {
                for (int v = 0; v < d; ++v) Sl[(size_t)k * d + v] += ar[k] * vj[v];
                zl[k] += a[k];
            }
        }
        /* carried state: S_c = g_c * S_{c-1} + local_c (g = 1 when ungated) */
        double gamma = g ? g[c] : 1.0;
        for (size_t e = 0; e < dd; ++e) S[e] = gamma * S[e] + Sl[e];
        for (int k = 0; k < d; ++k) z[k] = gamma * z[k] + zl[k];
        if (S_local) memcpy(S_local + (size_t)c * dd, Sl, sizeof(double) * dd);
        if (z_local) memcpy(z_local + (size_t)c * d, zl, sizeof(double) * (size_t)d);
        if (S_blocks) memcpy(S_blocks + (size_t)c * dd, S, sizeof(double) * dd);
        if (z_blocks) memcpy(z_blocks + (size_t)c * d, z, sizeof(double) * (size_t)d);

        /* read-out of every token of block c against the inclusive state */
        for (int i = 0; i < n; ++i) {
            long t = (long)c * n + i;
            const double *qi = Q + t * d;
            for (int f = 0; f < d; ++f) p[f] = relu(qi[f]);
            if (rope) rope_rotate(rope, t, d, p, pr);
            else memcpy(pr, p, sizeof(double) * (size_t)d);
            double den = eps;
            for (int k = 0; k < d; ++k) den += p[k] * z[k];
            if (den_out) den_out[t] = den;
            for (int v = 0; v < d; ++v) {
                double num = 0.0;
                for (int k = 0; k < d; ++k) num += pr[k] * S[(size_t)k * d + v];
                O[t * d + v] = (den != 0.0) ? num / den : 0.0;
            }
        }
    }
    if (S_out) memcpy(S_out, S, sizeof(double) * dd);
    if (z_out) memcpy(z_out, z, sizeof(double) * (size_t)d);
    free(S); free(z); free(Sl); free(zl); free(a); free(ar); free(p); free(pr);
}

/*
 * Full forward over nb blocks of n tokens for every (b, h).
 *   g        [B,H,nb] decay per block, NULL = ungated (g = 1)
 *   rope     NULL = no rotation
 *   S0, z0   carried state entering block 0, NULL = zero
 *   O        [B,H,N,d] output
 *   S_out, z_out        final state, nullable
 *   S_blocks, z_blocks  inclusive state of every block [B,H,nb,d,d] / [B,H,nb,d], nullable
 *   S_local, z_local    each block's own contribution, same shapes, nullable
 *   den_out  [B,H,N] denominators phi(q).z + eps, nullable
 *   threads  OpenMP threads (<= 0: the runtime's default)
 * Returns the number of threads used, or -1 on bad arguments.
 */
int svlao_forward(int B, int H, int nb, int n, int d,
                  const double *Q, const double *K, const double *V,
                  const double *g, const svlao_rope *rope,
                  const double *S0, const double *z0, double eps,
                  double *O, double *S_out, double *z_out,
                  double *S_blocks, double *z_blocks,
                  double *S_local, double *z_local, double *den_out,
                  int threads)
{
    if (B < 0 || H < 0 || nb < 0 || n < 0 || d <= 0) return -1;
    if (rope) {
        if (rope->dt_dims % 2 || rope->dh_dims % 2 || rope->dw_dims % 2) return -1;
        if (rope->dt_dims + rope->dh_dims + rope->dw_dims > d) return -1;
        if (rope->grid_h <= 0 || rope->grid_w <= 0) return -1;
    }
    long pairs = (long)B * H;
    size_t N = (size_t)nb * n;
    size_t dd = (size_t)d * d;
    int used = 1;
#ifdef _OPENMP
    if (threads <= 0) threads = omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 1) num_threads(threads)
#endif
    for (long bh = 0; bh < pairs; ++bh) {
#ifdef _OPENMP
        if (bh == 0) {
#pragma omp atomic write
            used = omp_get_num_threads();
        }
#endif
        one_head(nb, n, d, Q + bh * N * d, K + bh * N * d, V + bh * N * d,
                 g ? g + bh * nb : NULL, rope,
                 S0 ? S0 + bh * dd : NULL, z0 ? z0 + bh * d : NULL, eps,
                 O + bh * N * d,
                 S_out ? S_out + bh * dd : NULL, z_out ? z_out + bh * d : NULL,
                 S_blocks ? S_blocks + bh * nb * dd : NULL,
                 z_blocks ? z_blocks + bh * nb * d : NULL,
                 S_local ? S_local + bh * nb * dd : NULL,
                 z_local ? z_local + bh * nb * d : NULL,
                 den_out ? den_out + bh * N : NULL);
    }
    (void)threads;
    return used;
}
