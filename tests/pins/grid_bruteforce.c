/*
 * Exhaustive pins for the oracle's element rounding and shared-exponent rule.
 *
 * The oracle rounds |y| / 2^E to the nearest E2M1 magnitude by a distance
 * search over the eight grid values.  This program checks it against an
 * independent formulation, IEEE-style rounding to a one-mantissa-bit format:
 *   the binade of m fixes the grid spacing (0.5 below 2, 1 in [2,4), 2 in
 *   [4,8)), m is rounded to an integer multiple of that spacing with rint()
 *   (ties to the even multiple, i.e. the even mantissa), values >= 6 saturate,
 *   and the code is rebuilt from the E2M1 bit layout (2 exponent bits, bias 1,
 *   1 mantissa bit, exponent 0 = subnormal).
 * The shared exponent is checked against the fp32 exponent field read from
 * the bit pattern, plus the property amax / 2^E in [4, 8) when not clamped.
 *
 * Element checks: the fp32 bit patterns at E = 0 (all 2^32 with "full",
 * every 7th otherwise), and, for a set of E values including the clamps,
 * every pattern whose scaled magnitude lies in [2^-4, 2^5) plus all
 * subnormals and zeros.  Shared exponent: every non-negative finite fp32
 * pattern.
 *
 * usage: grid_bruteforce <path to liboracle.so> [threads] [full]
 * Without "full", the all-pattern element sweep visits every 7th pattern (the
 * windowed sweeps stay exhaustive); with "full" it visits all 2^32.
 * Prints one line per check and exits nonzero if any check fails.
 */
#include <dlfcn.h>
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

typedef int (*code_fn_t)(float, int);
typedef int (*e8_fn_t)(float);
static code_fn_t oracle_code;
static e8_fn_t oracle_e8;

static float bits_to_float(uint32_t u)
{
    float f;
    memcpy(&f, &u, 4);
    return f;
}

/* E2M1 code of a representable magnitude v, from the bit layout. */
static int encode_e2m1_magnitude(double v)
{
    if (v == 0.0)
        return 0;
    if (v < 1.0)           /* subnormal: exponent field 0, value = mantissa * 0.5 */
        return 1;          /* only 0.5 exists */
    int e;
    double f = frexp(v, &e); /* v = f * 2^e, f in [0.5, 1) */
    int expfield = e;        /* v in [2^(e-1), 2^e): unbiased exponent e-1, bias 1 */
    int mant = (f == 0.75) ? 1 : 0;
    return (expfield << 1) | mant;
}

static int ref_code(float y, int E)
{
    double m = ldexp(fabs((double)y), -E);
    double q;
    if (m >= 6.0) {
        q = 6.0;
    } else {
        double spacing;
        if (m < 2.0) {
            spacing = 0.5;
        } else {
            int e;
            frexp(m, &e);              /* m in [2^(e-1), 2^e) */
            spacing = ldexp(1.0, e - 2);
        }
        q = rint(m / spacing) * spacing;
    }
    return encode_e2m1_magnitude(q) | ((y < 0.0f) ? 8 : 0);
}

static int ref_e8(uint32_t u)
{
    /* u: bits of a non-negative finite float */
    uint32_t field = u >> 23;
    int E;
    if (u == 0)
        E = -127;
    else if (field == 0)
        E = -127; /* subnormal: floor(log2) <= -127, so E <= -129, clamped */
    else
        E = (int)field - 127 - 2;
    if (E < -127)
        E = -127;
    return E;
}

struct job {
    uint64_t lo, hi; /* pattern range [lo, hi) */
    int mode;        /* 0: element at fixed E over all patterns; 1: element windowed; 2: e8m0 */
    uint64_t stride; /* visit every stride-th pattern (1 = exhaustive) */
    int E;
    uint64_t checked, bad;
    uint32_t first_bad;
};

static int in_window(uint32_t u, int E)
{
    uint32_t field = (u >> 23) & 0xFF;
    if (field == 0xFF)
        return 0;
    if (field == 0)
        return 1; /* zeros and subnormals always */
    int ue = (int)field - 127;    /* |y| in [2^ue, 2^(ue+1)) */
    int me = ue - E;              /* scaled magnitude binade */
    return me >= -4 && me <= 4;
}

static void *worker(void *arg)
{
    struct job *j = (struct job *)arg;
    uint64_t first = j->lo + (j->stride - j->lo % j->stride) % j->stride;
    for (uint64_t p = first; p < j->hi; p += j->stride) {
        uint32_t u = (uint32_t)p;
        if (j->mode == 2) {
            if ((u >> 23) >= 0xFF)
                continue; /* inf / nan patterns */
            float a = bits_to_float(u);
            int E = oracle_e8(a);
            int R = ref_e8(u);
            int bad = (E != R);
            if (!bad && E > -127) {
                double r = ldexp((double)a, -E);
                bad = !(r >= 4.0 && r < 8.0);
            }
            j->checked++;
            if (bad) {
                if (!j->bad)
                    j->first_bad = u;
                j->bad++;
            }
            continue;
        }
        if (((u >> 23) & 0xFF) == 0xFF)
            continue;
        if (j->mode == 1 && !in_window(u, j->E))
            continue;
        float y = bits_to_float(u);
        int a = oracle_code(y, j->E);
        int b = ref_code(y, j->E);
        j->checked++;
        if (a != b) {
            if (!j->bad)
                j->first_bad = u;
            j->bad++;
        }
    }
    return NULL;
}

static int run(int mode, int E, uint64_t lo, uint64_t hi, uint64_t stride, int nth, const char *label)
{
    pthread_t th[64];
    struct job jobs[64];
    uint64_t span = hi - lo;
    for (int t = 0; t < nth; ++t) {
        jobs[t].lo = lo + span * t / nth;
        jobs[t].hi = lo + span * (t + 1) / nth;
        jobs[t].mode = mode;
        jobs[t].E = E;
        jobs[t].stride = stride;
        jobs[t].checked = jobs[t].bad = 0;
        jobs[t].first_bad = 0;
        pthread_create(&th[t], NULL, worker, &jobs[t]);
    }
    uint64_t checked = 0, bad = 0;
    uint32_t first = 0;
    for (int t = 0; t < nth; ++t) {
        pthread_join(th[t], NULL);
        checked += jobs[t].checked;
        if (jobs[t].bad && !bad)
            first = jobs[t].first_bad;
        bad += jobs[t].bad;
    }
    printf("%s E=%d stride=%llu checked=%llu bad=%llu", label, E, (unsigned long long)stride, (unsigned long long)checked, (unsigned long long)bad);
    if (bad)
        printf(" first_bad_bits=0x%08x", first);
    printf("\n");
    fflush(stdout);
    return bad ? 1 : 0;
}

int main(int argc, char **argv)
{
    if (argc < 2) {
        fprintf(stderr, "usage: %s liboracle.so [threads] [full]\n", argv[0]);
        return 2;
    }
    void *h = dlopen(argv[1], RTLD_NOW);
    if (!h) {
        fprintf(stderr, "dlopen: %s\n", dlerror());
        return 2;
    }
    oracle_code = (code_fn_t)dlsym(h, "oracle_fp4_code");
    oracle_e8 = (e8_fn_t)dlsym(h, "oracle_e8m0_exponent");
    if (!oracle_code || !oracle_e8) {
        fprintf(stderr, "missing symbols\n");
        return 2;
    }
    int nth = argc > 2 ? atoi(argv[2]) : 8;
    if (nth < 1)
        nth = 1;
    if (nth > 64)
        nth = 64;
    int fail = 0;
    int full = argc > 3 && strcmp(argv[3], "full") == 0;
    fail |= run(2, 0, 0, 0x80000000ull, 1, nth, "e8m0_all_nonneg");
    fail |= run(0, 0, 0, 0x100000000ull, full ? 1 : 7, nth, "fp4_all_patterns");
    const int Es_full[] = {-127, -126, -125, -124, -100, -3, -1, 0, 1, 2, 3, 60, 100, 124, 125, 126, 127};
    const int Es_quick[] = {-127, -126, -124, 0, 1, 125, 127};
    const int *Es = full ? Es_full : Es_quick;
    unsigned nE = full ? sizeof Es_full / sizeof Es_full[0] : sizeof Es_quick / sizeof Es_quick[0];
    for (unsigned i = 0; i < nE; ++i)
        fail |= run(1, Es[i], 0, 0x100000000ull, 1, nth, "fp4_window");
    printf(fail ? "FAIL\n" : "PASS\n");
    return fail;
}
