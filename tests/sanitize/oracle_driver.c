/* Runs the C oracle (built with AddressSanitizer and UndefinedBehaviorSanitizer)
 * over small inputs that reach every branch: RoPE with all three slices and
 * unrotated dims, a gate, a carried state, every optional output, ragged
 * sizes, a zero denominator, empty calls and rejected arguments.  Any invalid
 * access or undefined operation aborts the process. */
#include <math.h>
#include <stdio.h>
#include <stdlib.h>

typedef struct {
    int dt_dims, dh_dims, dw_dims;
    int grid_h, grid_w;
    int t0;
    double base;
} svlao_rope;

int svlao_forward(int B, int H, int nb, int n, int d, const double *Q, const double *K,
                  const double *V, const double *g, const svlao_rope *rope, const double *S0,
                  const double *z0, double eps, double *O, double *S_out, double *z_out,
                  double *S_blocks, double *z_blocks, double *S_local, double *z_local,
                  double *den_out, int threads);

static unsigned long long state = 88172645463325252ull;
static double urand(void)   /* xorshift64, uniform in [-1, 1) */
{
    state ^= state << 13; state ^= state >> 7; state ^= state << 17;
    return (double)(state >> 11) / 4503599627370496.0 - 1.0;
}

static double *arr(size_t n)
{
    double *p = malloc((n ? n : 1) * sizeof *p);
    for (size_t i = 0; i < n; ++i) p[i] = urand();
    return p;
}

static int run(int B, int H, int nb, int n, int d, int use_rope, int gated, int carried, double eps)
{
    const size_t N = (size_t)nb * n, bh = (size_t)B * H;
    double *Q = arr(bh * N * d), *K = arr(bh * N * d), *V = arr(bh * N * d);
    double *g = gated ? arr(bh * nb) : NULL;
    double *S0 = carried ? arr(bh * d * d) : NULL, *z0 = carried ? arr(bh * d) : NULL;
    if (z0) for (size_t i = 0; i < bh * d; ++i) z0[i] = fabs(z0[i]);
    double *O = arr(bh * N * d), *So = arr(bh * d * d), *zo = arr(bh * d);
    double *Sb = arr(bh * nb * d * d), *zb = arr(bh * nb * d);
    double *Sl = arr(bh * nb * d * d), *zl = arr(bh * nb * d), *den = arr(bh * N);
    svlao_rope r = {d >= 16 ? 4 : 2, d >= 16 ? 4 : 0, d >= 16 ? 4 : 0, 3, 5, 2, 10000.0};
    const int used = svlao_forward(B, H, nb, n, d, Q, K, V, g, use_rope ? &r : NULL, S0, z0, eps,
                                   O, So, zo, Sb, zb, Sl, zl, den, 1);
    int bad = used < 0;
    for (size_t i = 0; i < bh * N * d && !bad; ++i) bad = !isfinite(O[i]);
    free(Q); free(K); free(V); free(g); free(S0); free(z0); free(O); free(So); free(zo);
    free(Sb); free(zb); free(Sl); free(zl); free(den);
    return bad;
}

int main(void)
{
    int fails = 0;
    fails += run(1, 2, 4, 37, 16, 1, 1, 1, 1e-6);
    fails += run(2, 1, 3, 16, 8, 1, 0, 0, 1e-6);
    fails += run(1, 1, 1, 45, 32, 1, 1, 1, 1e-3);
    fails += run(1, 1, 2, 1, 4, 0, 1, 0, 1e-6);
    fails += run(1, 1, 5, 0, 8, 0, 1, 1, 1e-6);      /* blocks without tokens */
    fails += run(0, 3, 2, 4, 8, 0, 0, 0, 1e-6);      /* empty batch */
    /* eps = 0 with every query negative: zero denominators, zero outputs */
    {
        double Q[8 * 4], K[8 * 4], V[8 * 4], O[8 * 4];
        for (int i = 0; i < 32; ++i) { Q[i] = -1.0 - i; K[i] = urand(); V[i] = urand(); }
        fails += svlao_forward(1, 1, 2, 4, 4, Q, K, V, NULL, NULL, NULL, NULL, 0.0, O, NULL, NULL,
                               NULL, NULL, NULL, NULL, NULL, 1) < 0;
        for (int i = 0; i < 32; ++i) fails += O[i] != 0.0;
    }
    /* rejected arguments: odd RoPE dims, dims past d, negative sizes */
    {
        double x[4] = {0, 0, 0, 0};
        svlao_rope odd = {3, 0, 0, 1, 1, 0, 10000.0}, wide = {4, 4, 4, 1, 1, 0, 10000.0};
        fails += svlao_forward(1, 1, 1, 1, 4, x, x, x, NULL, &odd, NULL, NULL, 1e-6, x, NULL, NULL,
                               NULL, NULL, NULL, NULL, NULL, 1) != -1;
        fails += svlao_forward(1, 1, 1, 1, 4, x, x, x, NULL, &wide, NULL, NULL, 1e-6, x, NULL, NULL,
                               NULL, NULL, NULL, NULL, NULL, 1) != -1;
        fails += svlao_forward(-1, 1, 1, 1, 4, x, x, x, NULL, NULL, NULL, NULL, 1e-6, x, NULL, NULL,
                               NULL, NULL, NULL, NULL, NULL, 1) != -1;
    }
    printf("oracle under sanitizers: %s\n", fails ? "FAILED" : "clean");
    return fails != 0;
}
