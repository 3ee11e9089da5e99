/* The oracle (oracle/gpt2_ref.c) built with AddressSanitizer and
 * UndefinedBehaviorSanitizer by tests/test_native_sanitized.py: a forward,
 * a backward and an AdamW step on small shapes (including one where nothing
 * is a multiple of a tile, and one with padded vocabulary columns).  Exit
 * status 0 when the loss is finite and near ln V; a sanitizer report aborts. */
#include <math.h>
#include <stdio.h>
#include <stdlib.h>

typedef long long i64;
typedef struct ref_model ref_model;
i64 ref_param_tensor(int maxT, int V, int Vp, int L, int NH, int C, int idx, i64 *offset, i64 *count,
                     const char **name);
ref_model *ref_create(int maxT, int V, int Vp, int L, int NH, int C, int B, int T);
void ref_destroy(ref_model *M);
double ref_forward(ref_model *M, const double *params, const int *inputs, const int *targets);
int ref_backward(ref_model *M, const double *params, double *grads);
void ref_adamw(double *params, const double *grads, double *m, double *v, i64 n, double lr, double b1, double b2,
               double eps, double wd, int t);

static unsigned long long rng = 88172645463325252ULL;
static double uni(void) {
    rng ^= rng << 13;
    rng ^= rng >> 7;
    rng ^= rng << 17;
    return (double)(rng >> 11) / 9007199254740992.0;
}

static int run(int maxT, int V, int Vp, int L, int NH, int C, int B, int T) {
    i64 n = ref_param_tensor(maxT, V, Vp, L, NH, C, -1, NULL, NULL, NULL);
    double *p = calloc(n, sizeof(double)), *g = calloc(n, sizeof(double));
    double *m = calloc(n, sizeof(double)), *v = calloc(n, sizeof(double));
    int *in = malloc(sizeof(int) * B * T), *tg = malloc(sizeof(int) * B * T);
    for (i64 i = 0; i < n; i++) p[i] = 0.04 * (uni() - 0.5);
    for (int i = 0; i < B * T; i++) {
        in[i] = (int)(uni() * V) % V;
        tg[i] = (int)(uni() * V) % V;
    }
    ref_model *M = ref_create(maxT, V, Vp, L, NH, C, B, T);
    if (!M) return 1;
    double loss = ref_forward(M, p, in, tg);
    int rc = ref_backward(M, p, g);
    ref_adamw(p, g, m, v, n, 1e-4, 0.9, 0.999, 1e-8, 0.0, 1);
    double loss2 = ref_forward(M, p, in, NULL);
    ref_destroy(M);
    free(p); free(g); free(m); free(v); free(in); free(tg);
    printf("V=%d C=%d T=%d: loss %.6f (ln V %.6f)\n", V, C, T, loss, log((double)V));
    return (rc == 0 && isfinite(loss) && fabs(loss - log((double)V)) < 0.5 && isnan(loss2)) ? 0 : 1;
}

int main(void) {
    int bad = 0;
    bad |= run(64, 65, 128, 2, 4, 64, 2, 16);   /* tiny shape, padded vocabulary */
    bad |= run(24, 36, 36, 1, 3, 48, 3, 20);    /* ragged: nothing a multiple of a tile */
    bad |= run(4, 11, 12, 2, 2, 32, 1, 1);      /* one position */
    return bad;
}
