/*
 * Oracle for the dual-weight GLU projection -- TEST INFRASTRUCTURE ONLY.
 *
 * Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may
 * load this library.  It shares no code, header, table or helper with the
 * HIP library under glu_mlp_gemv_amd/; the product path never calls it.
 *
 * What it computes (plain definition, evaluated slowly and exactly):
 *
 *   DeepSpeed PR #8602 "HybridEngineRollout graph capture + segment-KI for
 *   Qwen3.5 hybrid", comment "Plan B: Dual-Weight GEMV", the
 *   DualWeightGluGEMV forward: its batched fallback defines the value as
 *   silu(h @ Wg^T) * (h @ Wu^T), with Wg, Wu in the nn.Linear layout
 *   [out_features N, in_features K]; its kernel accumulates both dots in fp32.
 *
 *   DeepSpeed PR #9057 "preserve HF precision boundaries in segKI kernels",
 *   section "Changes": the GLU keeps the intermediate bf16 roundings of a
 *   Hugging Face bf16 forward.  A bf16 HF MLP materialises three bf16
 *   tensors before its output: gate = h@Wg^T, up = h@Wu^T and act =
 *   silu(gate); the output is the bf16 product act*up.
 *
 * For every m in [0,M), j in [0,N):
 *   1. G = sum_k h[m,k]*Wg[j,k] in fp64, in increasing k.  A product of two
 *      bf16 values is exact in fp64; only the additions round (2^-53 each).
 *   2. U likewise with Wu.
 *   3. g = RNE_bf16(G), u = RNE_bf16(U), rounded directly from fp64.
 *   4. s = RNE_bf16( g / (1 + exp(-g)) ), every operation in IEEE fp32, exp
 *      rounded to fp32 from an fp64 evaluation (the correctly rounded fp32
 *      value except in vanishingly rare near-midpoint cases).
 *   5. out = RNE_bf16( fl32(s*u) ): two bf16 tensors multiply in fp32 and
 *      round once to bf16.  s*u is exact in fp32 unless it underflows.
 *
 * A second function, glu_oracle_linear, evaluates one projection of a
 * grouped GEMV: the pages' single/triple/quad GEMV kernels, which PR #9057
 * (commit notes) folds into one grouped_linear(x, weights, glu_epilogue), taken
 * without the GLU epilogue, i.e. n nn.Linear projections of one hidden.  A
 * bf16 nn.Linear output is one bf16 tensor, so
 *   out[m,j] = RNE_bf16( sum_k h[m,k]*W[j,k] ),  the sum in fp64 as in 1.
 *
 * Readings where the pages are silent: the silu formula is x/(1+exp(-x))
 * (the PR #8602 listing never defines its SILU); rounding is to nearest,
 * ties to even, throughout (that listing's _rn conversion); no denormal
 * flushing (PR #9057 removed fast math from the kernel builder).
 *
 * Pins (tests/test_oracle_*.py): exact-rational brute force of every step
 * on tiny inputs, an exhaustive sweep of all 65536 bf16 gate values through
 * steps 4-5 against an independent 50-digit Decimal evaluation, closed
 * forms (silu(0)=0, saturation, overflow, NaN), linearity of steps 1-2 in h,
 * row independence (M=1 vs batched), and torch-CPU cross-checks.
 *
 * Build: gcc -O2 -fopenmp -ffp-contract=off (no fast math) -shared -fPIC.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

#if defined(__FAST_MATH__)
#error "the oracle must not be built with fast math"
#endif

/* ---- bf16 <-> fp64 --------------------------------------------------- */

static double bf16_bits_to_double(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

static uint16_t float_bits_hi(float f)
{
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return (uint16_t)(u >> 16);
}

/*
 * Round an fp64 value to the nearest bf16 (ties to even), in one step.
 * bf16: 1 sign, 8 exponent, 7 fraction bits; normal quantum 2^(e-7) for a
 * value in [2^e, 2^(e+1)); subnormal quantum 2^-133 below 2^-126; largest
 * finite (2 - 2^-7)*2^127.  A value at or beyond the midpoint between the
 * largest finite and 2^128 rounds to infinity (that midpoint's even neighbour
 * is 2^128 itself).
 */
static uint16_t rne_bf16_from_double(double x)
{
    if (isnan(x)) {
        return (uint16_t)(signbit(x) ? 0xFFC0u : 0x7FC0u);
    }
    const uint16_t sign = (uint16_t)(signbit(x) ? 0x8000u : 0u);
    double ax = fabs(x);
    if (ax == 0.0) {
        return sign;
    }
    if (ax >= ldexp(1.0 - ldexp(1.0, -9), 128)) {
        return (uint16_t)(sign | 0x7F80u); /* infinity */
    }
    int e2;
    (void)frexp(ax, &e2);      /* ax = f * 2^e2, f in [0.5, 1) */
    int e = e2 - 1;            /* ax in [2^e, 2^(e+1)) */
    int qexp = (e < -126) ? -133 : e - 7;
    /* ax / 2^qexp is exact; nearbyint uses the default mode: to nearest even */
    double r = ldexp(nearbyint(ldexp(ax, -qexp)), qexp);
    /* r is a bf16 value (possibly 2^(e+1)); the fp32 cast is exact */
    return (uint16_t)(sign | float_bits_hi((float)r));
}

/* ---- fp32 silu, rounded steps ----------------------------------------- */

static float silu_f32(float g)
{
    /* exp in fp64, rounded once to fp32 */
    volatile float e = (float)exp(-(double)g);
    volatile float d = 1.0f + e;  /* fp32 add */
    volatile float s = g / d;     /* fp32 divide */
    return s;
}

/* steps 4 and 5 for one output */
static uint16_t glu_epilogue_one(uint16_t g_bits, uint16_t u_bits)
{
    float g = (float)bf16_bits_to_double(g_bits);
    float u = (float)bf16_bits_to_double(u_bits);
    uint16_t s_bits = rne_bf16_from_double((double)silu_f32(g));
    float s = (float)bf16_bits_to_double(s_bits);
    volatile float p = s * u; /* fp32 multiply */
    return rne_bf16_from_double((double)p);
}

/* ---- exported entry points ------------------------------------------- */

#define ORACLE_OK 0
#define ORACLE_ERR_ARG 1

static void set_threads(int threads)
{
#ifdef _OPENMP
    if (threads > 0) {
        omp_set_num_threads(threads);
    }
#else
    (void)threads;
#endif
}

/*
 * Full dual GLU projection.  Arrays are dense row-major bf16 bit patterns:
 * hidden [M,K], gate_w [N,K], up_w [N,K], out [M,N].  The optional fp64
 * outputs (each [M,N], may be NULL) receive G, U and the absolute sums
 * sum_k |h*Wg|, sum_k |h*Wu| used by the interval check.  threads <= 0
 * keeps the OpenMP default.
 */
int glu_oracle_dual_gemv(const uint16_t* hidden, const uint16_t* gate_w, const uint16_t* up_w,
                         uint16_t* out, int64_t M, int64_t N, int64_t K,
                         double* gate_pre, double* up_pre, double* gate_abs, double* up_abs,
                         int threads)
{
    if (M < 0 || N < 0 || K < 0) {
        return ORACLE_ERR_ARG;
    }
    if (M == 0 || N == 0) {
        return ORACLE_OK;
    }
    if (!out || (K > 0 && (!hidden || !gate_w || !up_w))) {
        return ORACLE_ERR_ARG;
    }
    set_threads(threads);
    const int64_t total = M * N;
#pragma omp parallel for schedule(static)
    for (int64_t idx = 0; idx < total; ++idx) {
        const int64_t m = idx / N;
        const int64_t j = idx % N;
        const uint16_t* hrow = hidden + m * K;
        const uint16_t* grow = gate_w + j * K;
        const uint16_t* urow = up_w + j * K;
        double G = 0.0, U = 0.0, Ga = 0.0, Ua = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            const double hk = bf16_bits_to_double(hrow[k]);
            const double pg = hk * bf16_bits_to_double(grow[k]);
            const double pu = hk * bf16_bits_to_double(urow[k]);
            G += pg;
            U += pu;
            Ga += fabs(pg);
            Ua += fabs(pu);
        }
        const uint16_t g = rne_bf16_from_double(G);
        const uint16_t u = rne_bf16_from_double(U);
        out[idx] = glu_epilogue_one(g, u);
        if (gate_pre) gate_pre[idx] = G;
        if (up_pre) up_pre[idx] = U;
        if (gate_abs) gate_abs[idx] = Ga;
        if (up_abs) up_abs[idx] = Ua;
    }
    return ORACLE_OK;
}

/*
 * One projection: out[m,j] = RNE_bf16(sum_k hidden[m,k] * w[j,k]) with the
 * sum in fp64 in increasing k.  Arrays are dense row-major bf16 bit patterns:
 * hidden [M,K], w [N,K], out [M,N].  The optional fp64 outputs (each [M,N],
 * may be NULL) receive the sum and sum_k |hidden*w| for the interval check.
 */
int glu_oracle_linear(const uint16_t* hidden, const uint16_t* w, uint16_t* out, int64_t M, int64_t N,
                      int64_t K, double* pre, double* abs_sum, int threads)
{
    if (M < 0 || N < 0 || K < 0) {
        return ORACLE_ERR_ARG;
    }
    if (M == 0 || N == 0) {
        return ORACLE_OK;
    }
    if (!out || (K > 0 && (!hidden || !w))) {
        return ORACLE_ERR_ARG;
    }
    set_threads(threads);
    const int64_t total = M * N;
#pragma omp parallel for schedule(static)
    for (int64_t pos = 0; pos < total; ++pos) {
        const uint16_t* hvec = hidden + (pos / N) * K;
        const uint16_t* wrow = w + (pos % N) * K;
        double acc = 0.0, acc_abs = 0.0;
        for (int64_t kk = 0; kk < K; ++kk) {
            const double prod = bf16_bits_to_double(hvec[kk]) * bf16_bits_to_double(wrow[kk]);
            acc += prod;
            acc_abs += fabs(prod);
        }
        out[pos] = rne_bf16_from_double(acc);
        if (pre) pre[pos] = acc;
        if (abs_sum) abs_sum[pos] = acc_abs;
    }
    return ORACLE_OK;
}

/*
 * The same computation for a list of (m, j) output positions only; out and
 * the optional fp64 arrays are indexed by list position [count].
 */
int glu_oracle_dual_gemv_sampled(const uint16_t* hidden, const uint16_t* gate_w,
                                 const uint16_t* up_w, int64_t M, int64_t N, int64_t K,
                                 const int64_t* rows_m, const int64_t* cols_j, int64_t count,
                                 uint16_t* out, double* gate_pre, double* up_pre,
                                 double* gate_abs, double* up_abs, int threads)
{
    if (M < 0 || N < 0 || K < 0 || count < 0) {
        return ORACLE_ERR_ARG;
    }
    if (count == 0) {
        return ORACLE_OK;
    }
    if (!rows_m || !cols_j || !out || (K > 0 && (!hidden || !gate_w || !up_w))) {
        return ORACLE_ERR_ARG;
    }
    for (int64_t i = 0; i < count; ++i) {
        if (rows_m[i] < 0 || rows_m[i] >= M || cols_j[i] < 0 || cols_j[i] >= N) {
            return ORACLE_ERR_ARG;
        }
    }
    set_threads(threads);
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < count; ++i) {
        const uint16_t* hrow = hidden + rows_m[i] * K;
        const uint16_t* grow = gate_w + cols_j[i] * K;
        const uint16_t* urow = up_w + cols_j[i] * K;
        double G = 0.0, U = 0.0, Ga = 0.0, Ua = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            const double hk = bf16_bits_to_double(hrow[k]);
            const double pg = hk * bf16_bits_to_double(grow[k]);
            const double pu = hk * bf16_bits_to_double(urow[k]);
            G += pg;
            U += pu;
            Ga += fabs(pg);
            Ua += fabs(pu);
        }
        out[i] = glu_epilogue_one(rne_bf16_from_double(G), rne_bf16_from_double(U));
        if (gate_pre) gate_pre[i] = G;
        if (up_pre) up_pre[i] = U;
        if (gate_abs) gate_abs[i] = Ga;
        if (up_abs) up_abs[i] = Ua;
    }
    return ORACLE_OK;
}

/* Steps 4-5 alone, elementwise over already-rounded bf16 gate and up values. */
int glu_oracle_epilogue(const uint16_t* g_bits, const uint16_t* u_bits, uint16_t* out, int64_t n)
{
    if (n < 0 || (n > 0 && (!g_bits || !u_bits || !out))) {
        return ORACLE_ERR_ARG;
    }
    for (int64_t i = 0; i < n; ++i) {
        out[i] = glu_epilogue_one(g_bits[i], u_bits[i]);
    }
    return ORACLE_OK;
}

/* Step 4 alone: bf16 silu of bf16 inputs (the act tensor of the HF MLP). */
int glu_oracle_silu_bf16(const uint16_t* g_bits, uint16_t* s_bits, int64_t n)
{
    if (n < 0 || (n > 0 && (!g_bits || !s_bits))) {
        return ORACLE_ERR_ARG;
    }
    for (int64_t i = 0; i < n; ++i) {
        float g = (float)bf16_bits_to_double(g_bits[i]);
        s_bits[i] = rne_bf16_from_double((double)silu_f32(g));
    }
    return ORACLE_OK;
}

/* The rounding of step 3 alone: fp64 values to bf16, ties to even. */
int glu_oracle_round_bf16(const double* x, uint16_t* out, int64_t n)
{
    if (n < 0 || (n > 0 && (!x || !out))) {
        return ORACLE_ERR_ARG;
    }
    for (int64_t i = 0; i < n; ++i) {
        out[i] = rne_bf16_from_double(x[i]);
    }
    return ORACLE_OK;
}

/* Threads OpenMP will use for a parallel region (reported by the benchmark). */
int glu_oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
