/*
 * Reference oracle for the MLA KV prolog -- TEST INFRASTRUCTURE ONLY.
 *
 * This file is the plain, slow, CPU-side definition of what the prolog
 * computes.  It exists so that the HIP library can be checked against it.
 * Only the test-suite, the smoke check and the CPU-baseline leg of the
 * benchmark may load it; the product path never does.  It shares no code,
 * header, table or helper with the HIP library.
 *
 * Source of the method: the page "DeepSeek-V2-Lite-Chat MLA KV Prolog
 * migration guide: PyPTO fused operators and aclgraph" (dpshk.com), section
 * "Background" (the seven-step sequence), section "Source-level principle"
 * (the Stage-1 / Stage-2 data flow: kv_a_proj with the caller-transposed
 * weight, slicing into compressed_kv and k_pe, RMSNorm, kv_b_proj, 3-D
 * reshape and view split into k_nope / value, RoPE, assemble) and section
 * "Precision verification" (RoPE in the standard x*cos + x_rot*sin form,
 * the shapes of the one published case, eps = 1e-6).  The W8A8 variant
 * follows the quantised-weight modes named on the DeepSeek-R1 recipe page
 * (cann-recipes-infer, section "Weight conversion"); the pages fix no
 * quantisation formula, so the scheme implemented here is the plain
 * symmetric per-row / per-column int8 one described at each function.
 *
 * Precision: every arithmetic step runs in IEEE single precision (fp32),
 * round to nearest even, in the plain order of the definition: each sum is
 * one fp32 accumulator running over the contracted index in ascending order
 * (products of two fp16 or two bf16 values are exact in fp32, so only the
 * additions round).  The one exception is the RoPE angle: the frequency
 * theta^(-2i/dr), the angle pos * f and its cosine / sine are evaluated in
 * double and rounded to fp32 before the rotation, because an fp32 angle
 * would be off by up to ~3e-3 rad at positions near 32768.  Built with
 * -ffp-contract=off, so no multiply-add is fused.  The W8A8 quantisation
 * decisions run in the same fp32 operations as the GPU kernels take them.
 *
 * Parity pins: every function here is pinned by the CPU tests against
 * closed forms, invariants, special cases and exact integer brute force
 * (see tests/test_oracle_pins.py).  Two readings are "parity unpinned"
 * beyond the tolerance: the exact intermediate rounding points of a GPU
 * implementation, and end-to-end values at full size (the pages print
 * shapes, not values).
 *
 * Build: gcc -O2 -fno-fast-math -ffp-contract=off -fopenmp -shared -fPIC.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_OK 0
#define ORACLE_BAD_ARG (-1)
#define ORACLE_NOMEM (-2)

/* ------------------------------------------------------------------------ */
/* Storage formats.                                                          */
/* ------------------------------------------------------------------------ */

/*
 * Round a double to the nearest value of a binary floating-point format with
 * `prec` significand bits (implicit bit included) and minimum normal
 * exponent `emin`, ties to even, overflow to infinity.  This is the IEEE-754
 * round-to-nearest-even definition written out: the spacing of representable
 * numbers near x is 2^(max(e, emin) - prec + 1) where 2^e <= |x| < 2^(e+1);
 * x / spacing is exact (power-of-two scaling), and nearbyint() rounds it to
 * the nearest integer, ties to even, under the default rounding mode.
 *   fp16: prec 11, emin -14,  max 65504
 *   bf16: prec 8,  emin -126, max (2 - 2^-7) * 2^127
 */
static double round_format(double x, int prec, int emin, double maxval)
{
    if (x == 0.0 || !isfinite(x)) return x;
    int e2;
    (void)frexp(x, &e2);           /* |x| = m * 2^e2, 0.5 <= m < 1 */
    int e = e2 - 1;                /* 2^e <= |x| < 2^(e+1) */
    if (e < emin) e = emin;        /* subnormal range: fixed spacing */
    double spacing = ldexp(1.0, e - prec + 1);
    double q = nearbyint(x / spacing) * spacing;
    if (fabs(q) > maxval) return copysign(INFINITY, x);
    return q;
}

/* dtype codes: 1 = fp16, 2 = bf16 (same numbering as the library header,
 * restated here so that the two share no file). */
static double round_dtype(double x, int dtype)
{
    if (dtype == 1) return round_format(x, 11, -14, 65504.0);
    if (dtype == 2) return round_format(x, 8, -126, ldexp(255.0, 120));
    return x;
}

int oracle_round_to_dtype(const double* in, double* out, int64_t n, int dtype)
{
    if (!in || !out || n < 0 || (dtype != 1 && dtype != 2)) return ORACLE_BAD_ARG;
    for (int64_t i = 0; i < n; ++i) out[i] = round_dtype(in[i], dtype);
    return ORACLE_OK;
}

/* ------------------------------------------------------------------------ */
/* The seven steps, one function each.                                       */
/* ------------------------------------------------------------------------ */

/* Step 1, kv_a_proj: A[n] = sum_k x[k] * Wa[k, n], with Wa stored [H, N1]
 * row-major (the weight is handed over already transposed, as in the
 * "Source-level principle" section).  One fp32 accumulator per output,
 * running over k in ascending order. */
static void step_kv_a_proj(const float* x, const float* Wa, int64_t H,
                           int64_t N1, float* A)
{
    for (int64_t n = 0; n < N1; ++n) A[n] = 0.0f;
    for (int64_t k = 0; k < H; ++k) {
        const float xk = x[k];
        const float* w = Wa + k * N1;
        for (int64_t n = 0; n < N1; ++n) A[n] += xk * w[n];
    }
}

/* Step 3, RMSNorm over the r latent columns (mean over r only, eps inside
 * the square root, gamma applied after the normalisation):
 *   y[j] = (c[j] * inv) * gamma[j],  inv = 1 / sqrt(sum_j c[j]^2 / r + eps)
 * The sum of squares is one fp32 accumulator, ascending in j. */
static float rms_inv(const float* c, int64_t r, float eps)
{
    float ss = 0.0f;
    for (int64_t j = 0; j < r; ++j) ss += c[j] * c[j];
    return 1.0f / sqrtf(ss / (float)r + eps);
}

/* Step 4, kv_b_proj: B[m] = sum_j y[j] * Wb[j, m], Wb stored [r, N2]; one
 * fp32 accumulator per output, ascending in j. */
static void step_kv_b_proj(const float* y, const float* Wb, int64_t r,
                           int64_t N2, float* B)
{
    for (int64_t m = 0; m < N2; ++m) B[m] = 0.0f;
    for (int64_t j = 0; j < r; ++j) {
        const float yj = y[j];
        const float* w = Wb + j * N2;
        for (int64_t m = 0; m < N2; ++m) B[m] += yj * w[m];
    }
}

/* Step 5, reshape [N2] -> [nh, dn+dv] and split each head's row into its
 * first dn entries (k_nope) and its last dv entries (value). */
static void step_split_heads(const float* B, int64_t nh, int64_t dn,
                             int64_t dv, float* k_nope, float* value)
{
    for (int64_t h = 0; h < nh; ++h) {
        const float* row = B + h * (dn + dv);
        for (int64_t d = 0; d < dn; ++d) k_nope[h * dn + d] = row[d];
        for (int64_t e = 0; e < dv; ++e) value[h * dv + e] = row[dn + e];
    }
}

/* Step 6, RoPE in rotate-half form on the dr rope columns:
 *   for i < dr/2:  f_i = theta^(-2i/dr),  a = pos * f_i
 *   out[i]        = p[i] cos a - p[i + dr/2] sin a
 *   out[i + dr/2] = p[i + dr/2] cos a + p[i] sin a
 * i.e. out = p * cos + rotate_half(p) * sin with rotate_half(p) =
 * (-p[dr/2:], p[:dr/2]).  f_i, a, cos a and sin a in double, rounded to
 * fp32; the rotation itself in fp32. */
static void step_rope(const float* p, int64_t dr, int64_t pos, double theta,
                      float* out)
{
    const int64_t half = dr / 2;
    for (int64_t i = 0; i < half; ++i) {
        const double f = pow(theta, -2.0 * (double)i / (double)dr);
        const double a = (double)pos * f;
        const float cs = (float)cos(a), sn = (float)sin(a);
        const float lo = p[i], hi = p[i + half];
        out[i] = lo * cs - hi * sn;
        out[i + half] = hi * cs + lo * sn;
    }
}

/* ------------------------------------------------------------------------ */
/* fp16 / bf16 path.                                                          */
/* ------------------------------------------------------------------------ */

/*
 * X [T,H], Wa [H, r+dr], gamma [r], Wb [r, nh*(dn+dv)]: the fp16/bf16
 * tensors widened (exactly) to float.  pos [T].  dtype selects the storage
 * format of the normalised latent that kv_b_proj consumes (it is the
 * compressed_kv output, materialised in the model's dtype).
 *
 * Outputs, fp32 values before the final rounding to the output dtype:
 *   k_nope [T, nh, dn], value [T, nh, dv], k_pe [T, dr], ckv [T, r].
 * Any output pointer may be NULL to skip it (k_nope and value together).
 */
int oracle_kv_prolog_fp(int64_t T, int64_t H, int64_t r, int64_t dr,
                        int64_t nh, int64_t dn, int64_t dv,
                        const float* X, const float* Wa, const float* gamma,
                        const float* Wb, const int32_t* pos, double eps,
                        double theta, int dtype, float* k_nope, float* value,
                        float* k_pe, float* ckv, int nthreads)
{
    if (T < 0 || H <= 0 || r <= 0 || dr < 0 || (dr % 2) != 0 || nh <= 0 ||
        dn < 0 || dv < 0)
        return ORACLE_BAD_ARG;
    if (T > 0 && (!X || !Wa || !gamma || !Wb || !pos)) return ORACLE_BAD_ARG;
    if (dtype != 1 && dtype != 2) return ORACLE_BAD_ARG;
    const int64_t N1 = r + dr, N2 = nh * (dn + dv);
    const float epsf = (float)eps;
    int bad = 0;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
#pragma omp parallel
    {
        float* A = (float*)malloc(sizeof(float) * (size_t)N1);
        float* y = (float*)malloc(sizeof(float) * (size_t)r);
        float* B = (float*)malloc(sizeof(float) * (size_t)(N2 > 0 ? N2 : 1));
        if (!A || !y || !B) {
#pragma omp atomic write
            bad = 1;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (int64_t t = 0; t < T; ++t) {
                /* 1. kv_a_proj */
                step_kv_a_proj(X + t * H, Wa, H, N1, A);
                /* 2. split: c = A[0:r], p = A[r:r+dr] */
                const float* c = A;
                const float* p = A + r;
                /* 3. RMSNorm */
                const float inv = rms_inv(c, r, epsf);
                for (int64_t j = 0; j < r; ++j) y[j] = (c[j] * inv) * gamma[j];
                if (ckv)
                    for (int64_t j = 0; j < r; ++j) ckv[t * r + j] = y[j];
                /* kv_b_proj consumes the stored (dtype) latent */
                for (int64_t j = 0; j < r; ++j) y[j] = (float)round_dtype((double)y[j], dtype);
                /* 4. kv_b_proj, 5. reshape + split */
                if (k_nope && value && N2 > 0) {
                    step_kv_b_proj(y, Wb, r, N2, B);
                    step_split_heads(B, nh, dn, dv, k_nope + t * nh * dn,
                                     value + t * nh * dv);
                }
                /* 6. RoPE on the rope columns */
                if (k_pe && dr > 0) step_rope(p, dr, pos[t], theta, k_pe + t * dr);
            }
        }
        free(A);
        free(y);
        free(B);
    }
    return bad ? ORACLE_NOMEM : ORACLE_OK;
}

/* ------------------------------------------------------------------------ */
/* W8A8 path.                                                                 */
/* ------------------------------------------------------------------------ */

/*
 * Symmetric int8 quantisation of one row, decided in IEEE single precision:
 *   amax = max |v|;  inv = 127 / amax  (correctly rounded division);
 *   q    = clamp(rint(v * inv), -127, 127)  (rint: ties to even);
 *   scale = amax / 127.
 * A row of zeros gives q = 0 and scale = 0.
 */
static float quantize_row(const float* v, int64_t n, int8_t* q)
{
    float amax = 0.0f;
    for (int64_t i = 0; i < n; ++i) {
        float a = fabsf(v[i]);
        if (a > amax) amax = a;
    }
    if (amax == 0.0f) {
        for (int64_t i = 0; i < n; ++i) q[i] = 0;
        return 0.0f;
    }
    volatile float inv = 127.0f / amax;
    for (int64_t i = 0; i < n; ++i) {
        volatile float s = v[i] * inv;
        float rq = rintf(s);
        if (rq > 127.0f) rq = 127.0f;
        if (rq < -127.0f) rq = -127.0f;
        q[i] = (int8_t)rq;
    }
    volatile float scale = amax / 127.0f;
    return scale;
}

/*
 * X [T,H] (bf16 widened exactly to float), Wqa [H, r+dr] int8 with
 * per-output-column scales swa [r+dr], gamma [r] (bf16 widened to float),
 * Wqb [r, N2] int8 with per-output-column scales swb [N2], pos [T].
 *
 *   a0  qx, sx       = quantize_row(X[t,:])
 *   a1  acc1[n]      = sum_k qx[k] * Wqa[k,n]            (exact integer)
 *       A[n]         = ((float)acc1[n] * sx) * swa[n]    (fp32, this order)
 *   a2  c = A[0:r], p = A[r:]
 *   a3q z[j]         = c[j] * gamma[j]                   (fp32)
 *       qz, sz       = quantize_row(z)
 *   a4  acc2[m]      = sum_j qz[j] * Wqb[j,m]            (exact integer)
 *   a3  inv_t        = 1 / sqrt(sum_j c[j]^2 / r + eps)  (fp32, ascending j)
 *       ckv[j]       = z[j] * inv_t
 *       B[m]         = (((float)acc2[m] * sz) * inv_t) * swb[m]
 *   a5  split B into k_nope / value;  a6  RoPE on p.
 *
 * Quantising z = c*gamma and applying the per-token RMS factor after the
 * integer product is the same as quantising the normalised latent
 * y = inv_t * z (a positive per-row factor leaves the codes unchanged, up to
 * the rounding of the scaled values), and keeps every integer-deciding step
 * free of reduction order.
 *
 * Outputs are fp32 values before the final rounding to bf16.  Optional
 * exports (each may be NULL): acc1 [T, r+dr], acc2 [T, N2], qx [T,H], sx [T],
 * qz [T,r], sz [T].
 */
int oracle_kv_prolog_w8a8(int64_t T, int64_t H, int64_t r, int64_t dr,
                          int64_t nh, int64_t dn, int64_t dv, const float* X,
                          const int8_t* Wqa, const float* swa,
                          const float* gamma, const int8_t* Wqb,
                          const float* swb, const int32_t* pos, double eps,
                          double theta, float* k_nope, float* value,
                          float* k_pe, float* ckv, int32_t* acc1_out,
                          int32_t* acc2_out, int8_t* qx_out, float* sx_out,
                          int8_t* qz_out, float* sz_out, int nthreads)
{
    if (T < 0 || H <= 0 || r <= 0 || dr < 0 || (dr % 2) != 0 || nh <= 0 ||
        dn < 0 || dv < 0)
        return ORACLE_BAD_ARG;
    if (T > 0 && (!X || !Wqa || !swa || !gamma || !Wqb || !swb || !pos))
        return ORACLE_BAD_ARG;
    const int64_t N1 = r + dr, N2 = nh * (dn + dv);
    const float epsf = (float)eps;
    int bad = 0;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
#pragma omp parallel
    {
        int8_t* qx = (int8_t*)malloc((size_t)H);
        int64_t* acc1 = (int64_t*)malloc(sizeof(int64_t) * (size_t)N1);
        float* A = (float*)malloc(sizeof(float) * (size_t)N1);
        float* z = (float*)malloc(sizeof(float) * (size_t)r);
        int8_t* qz = (int8_t*)malloc((size_t)r);
        int64_t* acc2 = (int64_t*)malloc(sizeof(int64_t) * (size_t)(N2 > 0 ? N2 : 1));
        float* B = (float*)malloc(sizeof(float) * (size_t)(N2 > 0 ? N2 : 1));
        if (!qx || !acc1 || !A || !z || !qz || !acc2 || !B) {
#pragma omp atomic write
            bad = 1;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (int64_t t = 0; t < T; ++t) {
                /* a0: per-token activation quantisation */
                const float sx = quantize_row(X + t * H, H, qx);
                /* a1: integer kv_a_proj, then dequantisation */
                for (int64_t n = 0; n < N1; ++n) acc1[n] = 0;
                for (int64_t k = 0; k < H; ++k) {
                    const int64_t xk = qx[k];
                    const int8_t* w = Wqa + k * N1;
                    for (int64_t n = 0; n < N1; ++n) acc1[n] += xk * (int64_t)w[n];
                }
                for (int64_t n = 0; n < N1; ++n) {
                    volatile float a = (float)(int32_t)acc1[n] * sx;
                    A[n] = a * swa[n];
                }
                /* a2: split */
                const float* c = A;
                const float* p = A + r;
                /* a3q: quantise z = c * gamma per token */
                for (int64_t j = 0; j < r; ++j) z[j] = c[j] * gamma[j];
                const float sz = quantize_row(z, r, qz);
                /* a4: integer kv_b_proj */
                if (N2 > 0) {
                    for (int64_t m = 0; m < N2; ++m) acc2[m] = 0;
                    for (int64_t j = 0; j < r; ++j) {
                        const int64_t qj = qz[j];
                        const int8_t* w = Wqb + j * N2;
                        for (int64_t m = 0; m < N2; ++m) acc2[m] += qj * (int64_t)w[m];
                    }
                }
                /* a3: the RMS factor of c */
                const float inv_t = rms_inv(c, r, epsf);
                if (ckv)
                    for (int64_t j = 0; j < r; ++j) ckv[t * r + j] = z[j] * inv_t;
                if (k_nope && value && N2 > 0) {
                    for (int64_t m = 0; m < N2; ++m)
                        B[m] = (((float)(int32_t)acc2[m] * sz) * inv_t) * swb[m];
                    step_split_heads(B, nh, dn, dv, k_nope + t * nh * dn,
                                     value + t * nh * dv);
                }
                /* a6: RoPE */
                if (k_pe && dr > 0) step_rope(p, dr, pos[t], theta, k_pe + t * dr);
                /* optional exports */
                if (acc1_out)
                    for (int64_t n = 0; n < N1; ++n) acc1_out[t * N1 + n] = (int32_t)acc1[n];
                if (acc2_out)
                    for (int64_t m = 0; m < N2; ++m) acc2_out[t * N2 + m] = (int32_t)acc2[m];
                if (qx_out) memcpy(qx_out + t * H, qx, (size_t)H);
                if (sx_out) sx_out[t] = sx;
                if (qz_out) memcpy(qz_out + t * r, qz, (size_t)r);
                if (sz_out) sz_out[t] = sz;
            }
        }
        free(qx); free(acc1); free(A); free(z); free(qz); free(acc2); free(B);
    }
    return bad ? ORACLE_NOMEM : ORACLE_OK;
}

/* ------------------------------------------------------------------------ */
/* Paged KV-cache append (the step after "assemble").                         */
/* ------------------------------------------------------------------------ */

/*
 * MLA caches the normalised latent and the rotated rope key of every token
 * (the smaller KV cache is the point of the method: migration guide,
 * "Background"); the R1 recipe page names paged attention ("Benchmark") and
 * an int8-cache mode W8A8C8 ("Weight conversion") without a layout or a
 * formula.  The reading implemented here:
 *   - the cache is num_slots slots of (r + dr) values, slot s holding
 *     [compressed_kv row | k_pe row]; a paged cache of blocks of B slots is
 *     the same array with slot = block * B + offset;
 *   - token t goes to slot slots[t]; a slot outside [0, num_slots) means the
 *     token is not cached (for example -1 for a padding token); slots of
 *     different tokens are distinct; slots not mapped keep their contents.
 * fp cache: the values themselves (the prolog's outputs, already in the model
 * dtype), no arithmetic.
 */
int oracle_kv_cache_append(int64_t T, int64_t r, int64_t dr, const double* ckv,
                           const double* kpe, const int64_t* slots, int64_t num_slots,
                           double* cache)
{
    if (T < 0 || r < 0 || dr < 0 || num_slots < 0 || (T > 0 && (!ckv || !kpe || !slots)) ||
        (num_slots > 0 && !cache))
        return ORACLE_BAD_ARG;
    const int64_t W = r + dr;
    for (int64_t t = 0; t < T; ++t) {
        const int64_t s = slots[t];
        if (s < 0 || s >= num_slots) continue;
        for (int64_t j = 0; j < r; ++j) cache[s * W + j] = ckv[t * r + j];
        for (int64_t i = 0; i < dr; ++i) cache[s * W + r + i] = kpe[t * dr + i];
    }
    return ORACLE_OK;
}

/*
 * int8 ("C8") cache: each mapped slot's r + dr values (the model-dtype
 * values, exact in fp32) quantised together by quantize_row above -- the
 * same symmetric per-token scheme as the W8A8 activations -- giving codes
 * [num_slots, r + dr] and one fp32 scale per slot (value ~ code * scale).
 */
int oracle_kv_cache_append_int8(int64_t T, int64_t r, int64_t dr, const float* ckv,
                                const float* kpe, const int64_t* slots, int64_t num_slots,
                                int8_t* cache_q, float* scale)
{
    if (T < 0 || r < 0 || dr < 0 || num_slots < 0 || (T > 0 && (!ckv || !kpe || !slots)) ||
        (num_slots > 0 && (!cache_q || !scale)))
        return ORACLE_BAD_ARG;
    const int64_t W = r + dr;
    float* row = (float*)malloc((size_t)(W > 0 ? W : 1) * sizeof(float));
    if (!row) return ORACLE_NOMEM;
    for (int64_t t = 0; t < T; ++t) {
        const int64_t s = slots[t];
        if (s < 0 || s >= num_slots) continue;
        for (int64_t j = 0; j < r; ++j) row[j] = ckv[t * r + j];
        for (int64_t i = 0; i < dr; ++i) row[r + i] = kpe[t * dr + i];
        scale[s] = quantize_row(row, W, cache_q + s * W);
    }
    free(row);
    return ORACLE_OK;
}

/* ------------------------------------------------------------------------ */
/* Standalone RMSNorm and RoPE (the prolog's steps 3 and 6 as operators).     */
/* ------------------------------------------------------------------------ */

/*
 * The migration guide ships RMSNorm and RoPE as kernels of their own next to
 * the fused prolog (section "Directory layout"; a switch for each in its
 * usage section); what they compute is the prolog's step 3 and step 6 above,
 * applied row by row, in the same fp32 arithmetic:
 *   rms_norm: x [rows, n] -> y[j] = (x[j] * inv) * gamma[j],
 *             inv = 1 / sqrt(sum_j x[j]^2 / n + eps)
 *   rope:     x [T, heads, dr] -> every head row of token t rotated by pos[t]
 * Inputs are the model-dtype values widened (exactly) to float; outputs are
 * fp32, before the final rounding.
 */
int oracle_rms_norm(int64_t rows, int64_t n, const float* x, const float* gamma,
                    double eps, float* y)
{
    if (rows < 0 || n <= 0 || (rows > 0 && (!x || !gamma || !y))) return ORACLE_BAD_ARG;
    for (int64_t t = 0; t < rows; ++t) {
        const float* xr = x + t * n;
        const float inv = rms_inv(xr, n, (float)eps);
        for (int64_t j = 0; j < n; ++j) y[t * n + j] = (xr[j] * inv) * gamma[j];
    }
    return ORACLE_OK;
}

int oracle_rope(int64_t T, int64_t heads, int64_t dr, const float* x, const int32_t* pos,
                double theta, float* y)
{
    if (T < 0 || heads <= 0 || dr <= 0 || (dr % 2) != 0 || (T > 0 && (!x || !pos || !y)))
        return ORACLE_BAD_ARG;
    for (int64_t t = 0; t < T; ++t)
        for (int64_t h = 0; h < heads; ++h) {
            const int64_t off = (t * heads + h) * dr;
            step_rope(x + off, dr, pos[t], theta, y + off);
        }
    return ORACLE_OK;
}

/* Number of threads an OpenMP parallel region of this library uses. */
int oracle_num_threads(int nthreads)
{
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
    return omp_get_max_threads();
#else
    (void)nthreads;
    return 1;
#endif
}
