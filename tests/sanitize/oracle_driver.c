/* Driver for the sanitizer build of the CPU oracle (AddressSanitizer and
 * UndefinedBehaviorSanitizer): MTTKRP on small tensors of order 2 to 5, all
 * modes, full outputs against row subsets (in a scrambled order, with
 * repeats), then a few CP-ALS sweeps, including one whose Cholesky fails.
 * Exit status 0 when every check holds. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

int oracle_mttkrp_rows(const double *X, const int64_t *dims, int order, const double *const *U,
                       int64_t R, int mode, const int64_t *rows, int64_t nrows, double *out,
                       int nthreads);
int oracle_cp_als(const double *X, const int64_t *dims, int order, int64_t R, double *const *U,
                  double *lambda, int iters, double *fit, int nthreads);

static uint64_t st = 99;
static double urand(void)
{
    st = st * 6364136223846793005ull + 1442695040888963407ull;
    return (double)(st >> 11) / 9007199254740992.0;
}

int main(void)
{
    int fails = 0;
    const int64_t shapes[][5] = {{5, 4, 0, 0, 0}, {3, 1, 5, 0, 0}, {4, 3, 2, 5, 0}, {2, 3, 2, 3, 2},
                                 {7, 6, 5, 0, 0}};
    const int orders[] = {2, 3, 4, 5, 3};
    /* ranks no larger than the product of any two other dimensions, so the
       R x R systems of CP-ALS are positive definite */
    const int64_t ranks[] = {3, 2, 4, 3, 6};
    for (int c = 0; c < 5; ++c) {
        const int d = orders[c];
        int64_t N = 1;
        for (int m = 0; m < d; ++m) N *= shapes[c][m];
        const int64_t R = ranks[c];
        double *X = malloc(sizeof(double) * N);
        for (int64_t i = 0; i < N; ++i) X[i] = 2 * urand() - 1;
        double *U[5];
        for (int m = 0; m < d; ++m) {
            U[m] = malloc(sizeof(double) * shapes[c][m] * R);
            for (int64_t i = 0; i < shapes[c][m] * R; ++i) U[m][i] = urand();
        }
        for (int n = 0; n < d; ++n) {
            const int64_t In = shapes[c][n];
            double *full = malloc(sizeof(double) * In * R);
            int64_t *rows = malloc(sizeof(int64_t) * (In + 1));
            double *part = malloc(sizeof(double) * (In + 1) * R);
            const double *Uc[5] = {U[0], U[1], U[2], U[3], U[4]};
            Uc[n] = NULL; /* the target factor is not read */
            if (oracle_mttkrp_rows(X, shapes[c], d, Uc, R, n, NULL, 0, full, 2)) ++fails;
            for (int64_t j = 0; j < In; ++j) rows[j] = (j * 7 + 3) % In;
            rows[In] = In - 1;
            if (oracle_mttkrp_rows(X, shapes[c], d, Uc, R, n, rows, In + 1, part, 2)) ++fails;
            for (int64_t j = 0; j <= In; ++j)
                for (int64_t r = 0; r < R; ++r)
                    if (part[j * R + r] != full[rows[j] * R + r]) ++fails;
            free(full);
            free(rows);
            free(part);
        }
        if (d >= 3) {
            double lam[8], fit[3];
            const int s1 = oracle_cp_als(X, shapes[c], d, R, U, lam, 3, fit, 2);
            if (s1 != 0) {
                printf("case %d: cp_als status %d\n", c, s1);
                ++fails;
            }
            for (int k = 0; k < 3; ++k)
                if (!(fit[k] <= 1.0)) ++fails;
            /* a zero column: the Cholesky of the R x R system fails */
            for (int64_t i = 0; i < shapes[c][0]; ++i) U[0][i * R + 1] = 0.0;
            for (int64_t i = 0; i < shapes[c][1]; ++i) U[1][i * R + 1] = 0.0;
            const int s2 = oracle_cp_als(X, shapes[c], d, R, U, lam, 2, fit, 2);
            if (s2 != -7) {
                printf("case %d: zero-column cp_als status %d\n", c, s2);
                ++fails;
            }
        }
        for (int m = 0; m < d; ++m) free(U[m]);
        free(X);
    }
    printf("oracle driver: %d failed checks\n", fails);
    return fails ? 1 : 0;
}
