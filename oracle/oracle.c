/*
 * oracle.c -- plain, slow CPU oracle for the W4A8 block-quantized matmul and
 * the Q4_K fused-dequant matmul.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing in the product path may call, link or
 * load this file; only the tests, the smoke check and the CPU-baseline leg of
 * the benchmark do. It shares no code, header, table or constant generator
 * with the HIP library.
 *
 * Sources (web pages on block-quantized 4-bit weights):
 *   [tract]  tract PR #2432 "WIP: W4A8 (Q4_0 int8-dot) path for block_quant",
 *            section "The kernel" and the pipeline figure: Q4_0 4-bit weights
 *            stored N x K with one scale per 32-weight block, activations
 *            quantized to int8 per block, exact integer dot per block, then a
 *            per-block f32 rescale; output f32.
 *   [mlx]    MLX PR #4802 (mx.qqmm mode="affine"): affine 4-bit weights with
 *            per-group scales and biases, x quantized to int8, an int8 x int8
 *            MMA over the original codes with the per-group scale and bias
 *            applied in the kernel; section "Accuracy" gives the error level.
 *   [cke]    C-Kernel-Engine gemm_kernels_q4k.c source page: Q4_K super-blocks
 *            of 256 weights (4.5 bits/weight, fp16 d and dmin, eight 32-weight
 *            sub-blocks with 6-bit scales and mins), functions gemv_q4_k_ref
 *            (code map, "w = d * q - m"), gemm_q4_k_ref (GEMM = one GEMV per
 *            activation row) and gemm_nt_q4_k (A [M x K], B [N x K], C [M x N]).
 *
 * Precision: integer work is exact; the float results are accumulated in
 * double from exactly-converted terms and rounded once to float. Steps where a
 * float decides an integer code (activation and weight quantization) are taken
 * in float32, the precision of the GPU kernels, so both sides make the same
 * decision. Build without -ffast-math and with -ffp-contract=off.
 *
 * Readings where the pages are silent (each listed in the design notes):
 *   - activation scale xs = amax / 127 in float32, code = clamp(rne(v / xs),
 *     -127, 127) with a correctly rounded float32 quotient; amax == 0 gives
 *     xs = 0 and all codes 0;
 *   - Q4_0 scale d = fp16(mx / -8) from the signed extreme mx, codes
 *     clamp(rne(w / d) + 8, 0, 15), value d * (q - 8);
 *   - affine scale = bf16((max - min) / 15), bias = bf16(min), codes
 *     clamp(rne((w - bias) / scale), 0, 15), value scale * q + bias;
 *   - the affine "bias * sum x" term uses the dequantized activation sum
 *     xs * sum(xq) of the group, so y equals dequant(W) . dequant(X) exactly;
 *   - code layout: block b of row n is 16 bytes at offset 16 b; byte j holds
 *     k = 32 b + j in its low nibble and k = 32 b + 16 + j in its high nibble;
 *   - affine 8-bit ([mlx] lists 4, 6 and 8 bits): wq [N][K], byte k = code k;
 *     affine 6-bit: the low 4 bits of every code in the 4-bit layout above
 *     (N x K/2 bytes), then the high 2 bits as N x K/4 bytes: block b of row n
 *     is 8 bytes at offset 8 b, two little-endian words; word h holds code
 *     32 b + 16 h + c (c = 0..15) in byte c % 4, bits 2 (c / 4) and 2 (c / 4) + 1;
 *     scale = bf16((max - min) / (2^bits - 1)), codes 0 .. 2^bits - 1;
 *   - Q4_K struct {fp16 d; fp16 dmin; u8 scales[12]; u8 qs[128]} with the
 *     sixteen 6-bit fields (sc[0..7], m[0..7]) packed little-endian, field f at
 *     bits [6f, 6f + 6) of the 96-bit string.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define OR_OK 0
#define OR_BAD 1

/* ------------------------------------------------------------------------ */
/* Threads (used only to time the oracle on a host's cores)                  */
/* ------------------------------------------------------------------------ */

/* The products below can split their output columns n over T threads: a
 * static partition into T contiguous ranges, each output computed by exactly
 * one thread with the same arithmetic in the same order as with one thread,
 * so the results are bit-identical for every T (C-Kernel-Engine's kernel
 * rules keep threading out of the kernels; here it sits outside the
 * per-output arithmetic). */
#define OR_MAX_THREADS 256
static int g_threads = 1;

int or_set_threads(int t) {
    g_threads = t < 1 ? 1 : (t > OR_MAX_THREADS ? OR_MAX_THREADS : t);
    return g_threads;
}

struct or_range { void (*fn)(const void*, long, long); const void* ctx; long n0, n1; };

static void* or_range_main(void* p) {
    const struct or_range* r = (const struct or_range*)p;
    r->fn(r->ctx, r->n0, r->n1);
    return NULL;
}

/* fn(ctx, n0, n1) over a partition of [0, n). Returns OR_BAD if a thread
 * could not be started (the work done so far is then incomplete). */
static int for_ranges(long n, void (*fn)(const void*, long, long), const void* ctx) {
    long T = g_threads < n ? g_threads : n;
    if (T <= 1) {
        fn(ctx, 0, n);
        return OR_OK;
    }
    pthread_t th[OR_MAX_THREADS];
    struct or_range r[OR_MAX_THREADS];
    long started = 0;
    int rc = OR_OK;
    for (long t = 0; t < T; ++t) {
        r[t].fn = fn;
        r[t].ctx = ctx;
        r[t].n0 = n * t / T;
        r[t].n1 = n * (t + 1) / T;
        if (pthread_create(&th[t], NULL, or_range_main, &r[t]) != 0) {
            rc = OR_BAD;
            break;
        }
        ++started;
    }
    for (long t = 0; t < started; ++t) pthread_join(th[t], NULL);
    return rc;
}

/* ------------------------------------------------------------------------ */
/* Number formats (IEEE 754 binary16 and bfloat16)                           */
/* ------------------------------------------------------------------------ */

/* binary16 -> float: sign, 5-bit exponent (bias 15), 10-bit fraction; the
 * value is written out from the definition, subnormals included. */
float or_f16_to_f32(uint16_t h) {
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1F;
    int f = h & 0x3FF;
    double v;
    if (e == 0) {
        v = ldexp((double)f, -24);
    } else if (e == 31) {
        v = f ? NAN : INFINITY;
    } else {
        v = ldexp((double)(1024 + f), e - 25);
    }
    return (float)(sign ? -v : v);
}

/* float -> binary16 with round-half-even, subnormals and overflow included. */
uint16_t or_f32_to_f16(float x) {
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    double a = fabs((double)x);
    if (isnan(x)) return (uint16_t)(sign | 0x7E00);
    if (isinf(x)) return (uint16_t)(sign | 0x7C00);
    if (a == 0.0) return sign;
    int e2;
    frexp(a, &e2);             /* a = m * 2^e2, m in [0.5, 1): leading bit 2^(e2-1) */
    int e = e2 - 1;            /* a in [2^e, 2^(e+1)) */
    if (e < -14) {
        /* subnormal range: quantum 2^-24; a * 2^24 is exact in double */
        double m = nearbyint(ldexp(a, 24));
        return (uint16_t)(sign | (uint16_t)m);   /* m == 1024 encodes 2^-14 */
    }
    double m = nearbyint(ldexp(a, 10 - e));      /* in [1024, 2048] */
    if (m == 2048.0) { m = 1024.0; e += 1; }
    if (e > 15) return (uint16_t)(sign | 0x7C00);
    return (uint16_t)(sign | (uint16_t)((e + 15) << 10) | (uint16_t)(m - 1024.0));
}

/* bfloat16 is the upper half of a binary32 pattern. */
float or_bf16_to_f32(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

/* float -> bfloat16 with round-half-even on the discarded 16 bits. */
uint16_t or_f32_to_bf16(float x) {
    uint32_t u;
    memcpy(&u, &x, 4);
    if (isnan(x)) return (uint16_t)((u >> 16) | 0x40);
    uint32_t hi = u >> 16, lo = u & 0xFFFF;
    if (lo > 0x8000 || (lo == 0x8000 && (hi & 1))) hi += 1;
    return (uint16_t)hi;
}

static void or_f16_array_to_f32(const uint16_t* in, float* out, long n) {
    for (long i = 0; i < n; ++i) out[i] = or_f16_to_f32(in[i]);
}
void or_f16_to_f32_array(const uint16_t* in, float* out, long n) { or_f16_array_to_f32(in, out, n); }

void or_f32_to_f16_array(const float* in, uint16_t* out, long n) {
    for (long i = 0; i < n; ++i) out[i] = or_f32_to_f16(in[i]);
}

void or_f32_to_bf16_array(const float* in, uint16_t* out, long n) {
    for (long i = 0; i < n; ++i) out[i] = or_f32_to_bf16(in[i]);
}

/* ------------------------------------------------------------------------ */
/* Activation quantization ([tract] "activation -> int8, per-block";         */
/* [mlx] "x is quantized to int8")                                           */
/* ------------------------------------------------------------------------ */

static float load_x(const void* x, int xdt, long i) {
    if (xdt == 0) return ((const float*)x)[i];
    return or_bf16_to_f32(((const uint16_t*)x)[i]);
}

/* x [M][K] (xdt 0 = float32, 1 = bfloat16 bits) -> xq [M][K] int8,
 * xs [M][K/bs] float32 scale, xsum [M][K/bs] int32 sum of the block's codes. */
int or_quantize_act(int M, int K, int bs, int xdt, const void* x,
                    int8_t* xq, float* xs, int32_t* xsum) {
    if (M < 0 || K <= 0 || bs <= 0 || K % bs != 0) return OR_BAD;
    int nb = K / bs;
    for (long m = 0; m < M; ++m) {
        for (int b = 0; b < nb; ++b) {
            long base = m * (long)K + (long)b * bs;
            float amax = 0.0f;
            for (int j = 0; j < bs; ++j) {
                float a = fabsf(load_x(x, xdt, base + j));
                if (a > amax) amax = a;
            }
            float s = amax / 127.0f;      /* float32, correctly rounded */
            int32_t sum = 0;
            for (int j = 0; j < bs; ++j) {
                int q = 0;
                if (amax != 0.0f) {
                    float r = load_x(x, xdt, base + j) / s;   /* float32 quotient */
                    q = (int)nearbyintf(r);                    /* round half even */
                    if (q > 127) q = 127;
                    if (q < -127) q = -127;
                }
                xq[base + j] = (int8_t)q;
                sum += q;
            }
            xs[m * nb + b] = (amax != 0.0f) ? s : 0.0f;
            xsum[m * nb + b] = sum;
        }
    }
    return OR_OK;
}

/* ------------------------------------------------------------------------ */
/* Weight quantizers (data generation for the tests)                         */
/* ------------------------------------------------------------------------ */

static void put_code(uint8_t* row, int k, int q) {
    /* 32-weight block b = k / 32 occupies bytes [16 b, 16 b + 16);
     * position j < 16 -> low nibble of byte j, j >= 16 -> high nibble of byte j - 16 */
    int b = k / 32, j = k % 32;
    uint8_t* byte = row + 16 * b + (j & 15);
    if (j < 16) *byte = (uint8_t)((*byte & 0xF0) | (q & 0x0F));
    else        *byte = (uint8_t)((*byte & 0x0F) | ((q & 0x0F) << 4));
}

static int get_code(const uint8_t* row, int k) {
    int b = k / 32, j = k % 32;
    uint8_t byte = row[16 * b + (j & 15)];
    return (j < 16) ? (byte & 0x0F) : (byte >> 4);
}

int or_get_code(const uint8_t* wq, int K, int n, int k) {
    return get_code(wq + (long)n * (K / 2), k);
}

/* Code of weight (n, k) at a bit width (4, 6 or 8), per the layouts above. */
static int code_at(const uint8_t* wq, int N, int K, int bits, long n, int k) {
    if (bits == 8) return wq[n * (long)K + k];
    int lo = get_code(wq + n * (long)(K / 2), k);
    if (bits == 4) return lo;
    const uint8_t* hp = wq + (long)N * (K / 2) + n * (long)(K / 4);
    int b = k / 32, j = k % 32, h = j / 16, c = j % 16;
    int hi2 = (hp[8 * b + 4 * h + (c % 4)] >> (2 * (c / 4))) & 3;
    return lo | (hi2 << 4);
}

static void put_code_at(uint8_t* wq, int N, int K, int bits, long n, int k, int q) {
    if (bits == 8) { wq[n * (long)K + k] = (uint8_t)q; return; }
    put_code(wq + n * (long)(K / 2), k, q & 0x0F);
    if (bits == 4) return;
    uint8_t* hp = wq + (long)N * (K / 2) + n * (long)(K / 4);
    int b = k / 32, j = k % 32, h = j / 16, c = j % 16;
    uint8_t* byte = hp + 8 * b + 4 * h + (c % 4);
    int sh = 2 * (c / 4);
    *byte = (uint8_t)((*byte & ~(3 << sh)) | (((q >> 4) & 3) << sh));
}

static int bits_ok(int bits) { return bits == 4 || bits == 6 || bits == 8; }

long or_code_bytes(int N, int K, int bits) {
    if (!bits_ok(bits) || N < 0 || K <= 0 || K % 32 != 0) return -1;
    return (long)N * K * bits / 8;
}

int or_get_code_bits(const uint8_t* wq, int N, int K, int bits, int n, int k) {
    return code_at(wq, N, K, bits, n, k);
}

/* Q4_0 ([tract]: 4-bit codes, N x K, one fp16 scale per 32-block):
 * w [N][K] float32 -> wq [N][K/2], wd [N][K/32] fp16 bits. */
int or_quantize_q4_0(int N, int K, const float* w, uint8_t* wq, uint16_t* wd) {
    if (N < 0 || K <= 0 || K % 32 != 0) return OR_BAD;
    int nb = K / 32;
    for (long n = 0; n < N; ++n) {
        uint8_t* row = wq + n * (K / 2);
        memset(row, 0, (size_t)K / 2);
        for (int b = 0; b < nb; ++b) {
            const float* blk = w + n * (long)K + 32L * b;
            int imax = 0;
            for (int j = 1; j < 32; ++j)
                if (fabsf(blk[j]) > fabsf(blk[imax])) imax = j;
            float mx = blk[imax];
            uint16_t d16 = or_f32_to_f16(mx / -8.0f);
            float df = or_f16_to_f32(d16);
            wd[n * nb + b] = d16;
            for (int j = 0; j < 32; ++j) {
                int q = 8;
                if (df != 0.0f) {
                    q = (int)nearbyintf(blk[j] / df) + 8;
                    if (q < 0) q = 0;
                    if (q > 15) q = 15;
                }
                put_code(row, 32 * b + j, q);
            }
        }
    }
    return OR_OK;
}

/* Affine ([mlx]: per-group scale and bias, codes 0 .. 2^bits - 1, bits 4, 6
 * or 8): w [N][K] bfloat16 bits -> wq (or_code_bytes(N, K, bits) bytes),
 * ws, wb [N][K/g] bfloat16 bits. */
int or_quantize_affine_bits(int N, int K, int g, int bits, const uint16_t* w, uint8_t* wq,
                            uint16_t* ws, uint16_t* wb) {
    if (N < 0 || K <= 0 || g <= 0 || g % 32 != 0 || K % g != 0 || !bits_ok(bits)) return OR_BAD;
    int ng = K / g;
    int qmax = (1 << bits) - 1;
    memset(wq, 0, (size_t)or_code_bytes(N, K, bits));
    for (long n = 0; n < N; ++n) {
        for (int gi = 0; gi < ng; ++gi) {
            const uint16_t* grp = w + n * (long)K + (long)g * gi;
            float mn = or_bf16_to_f32(grp[0]), mx = mn;
            for (int j = 1; j < g; ++j) {
                float v = or_bf16_to_f32(grp[j]);
                if (v < mn) mn = v;
                if (v > mx) mx = v;
            }
            float range = mx - mn;
            uint16_t s16 = or_f32_to_bf16(range / (float)qmax);
            uint16_t b16 = or_f32_to_bf16(mn);
            float sf = or_bf16_to_f32(s16), bf = or_bf16_to_f32(b16);
            ws[n * ng + gi] = s16;
            wb[n * ng + gi] = b16;
            for (int j = 0; j < g; ++j) {
                int q = 0;
                if (sf != 0.0f) {
                    float t = or_bf16_to_f32(grp[j]) - bf;
                    q = (int)nearbyintf(t / sf);
                    if (q < 0) q = 0;
                    if (q > qmax) q = qmax;
                }
                put_code_at(wq, N, K, bits, n, g * gi + j, q);
            }
        }
    }
    return OR_OK;
}

int or_quantize_affine(int N, int K, int g, const uint16_t* w, uint8_t* wq, uint16_t* ws, uint16_t* wb) {
    return or_quantize_affine_bits(N, K, g, 4, w, wq, ws, wb);
}

/* ------------------------------------------------------------------------ */
/* Integer partials and results                                              */
/* ------------------------------------------------------------------------ */

/* Per-block integer dot of row n of the weights with row m of the codes.
 * fmt 0 (Q4_0): sum (q - 8) * xq over the block of bs = 32.
 * fmt 1 (affine): sum q * xq over the group of bs. */
static int32_t block_dot(int N, int K, int bs, int fmt, int bits, const uint8_t* wq, const int8_t* xq,
                         long m, long n, int b) {
    const int8_t* xr = xq + m * (long)K;
    int32_t acc = 0;
    for (int j = 0; j < bs; ++j) {
        int k = b * bs + j;
        int q = code_at(wq, N, K, bits, n, k);
        if (fmt == 0) q -= 8;
        acc += (int32_t)q * (int32_t)xr[k];
    }
    return acc;
}

static int check_fmt_bits(int K, int bs, int fmt, int bits) {
    if (!bits_ok(bits) || (fmt == 0 && bits != 4)) return OR_BAD;
    if (K <= 0 || bs <= 0 || K % bs != 0) return OR_BAD;
    if (fmt == 0 && bs != 32) return OR_BAD;
    if (fmt == 1 && (bs % 32 != 0)) return OR_BAD;
    if (fmt != 0 && fmt != 1) return OR_BAD;
    return OR_OK;
}

static int check_fmt(int K, int bs, int fmt) {
    if (K <= 0 || bs <= 0 || K % bs != 0) return OR_BAD;
    if (fmt == 0 && bs != 32) return OR_BAD;
    if (fmt == 1 && (bs % 32 != 0)) return OR_BAD;
    if (fmt != 0 && fmt != 1) return OR_BAD;
    return OR_OK;
}

/* partials [(m1 - m0)][N][K/bs] int32 for rows m0 <= m < m1 (bits 4, 6, 8; Q4_0 is 4-bit only). */
int or_q4_partials_bits(int M, int K, int N, int bs, int fmt, int bits, const uint8_t* wq,
                        const int8_t* xq, int m0, int m1, int32_t* partials) {
    if (check_fmt_bits(K, bs, fmt, bits) || m0 < 0 || m1 > M || m0 > m1 || N < 0) return OR_BAD;
    int nb = K / bs;
    for (long m = m0; m < m1; ++m)
        for (long n = 0; n < N; ++n)
            for (int b = 0; b < nb; ++b)
                partials[((m - m0) * (long)N + n) * nb + b] = block_dot(N, K, bs, fmt, bits, wq, xq, m, n, b);
    return OR_OK;
}

int or_q4_partials(int M, int K, int N, int bs, int fmt, const uint8_t* wq,
                   const int8_t* xq, int m0, int m1, int32_t* partials) {
    return or_q4_partials_bits(M, K, N, bs, fmt, 4, wq, xq, m0, m1, partials);
}

/* One output y[m][n]:
 *   Q4_0:   sum_b d[n,b] * xs[m,b] * P[m,n,b]
 *   affine: sum_g xs[m,g] * (scale[n,g] * A[m,n,g] + bias[n,g] * xsum[m,g])
 * each term exact in double, summed in block order, rounded once to float. */
static float one_output(int N, int K, int bs, int fmt, int bits, const uint8_t* wq, const uint16_t* wscale,
                        const uint16_t* wbias, const int8_t* xq, const float* xs,
                        const int32_t* xsum, long m, long n) {
    int nb = K / bs;
    double y = 0.0;
    for (int b = 0; b < nb; ++b) {
        int32_t p = block_dot(N, K, bs, fmt, bits, wq, xq, m, n, b);
        double a = (double)xs[m * nb + b];
        if (fmt == 0) {
            double d = (double)or_f16_to_f32(wscale[n * nb + b]);
            y += d * a * (double)p;
        } else {
            double s = (double)or_bf16_to_f32(wscale[n * nb + b]);
            double c = (double)or_bf16_to_f32(wbias[n * nb + b]);
            y += a * (s * (double)p + c * (double)xsum[m * nb + b]);
        }
    }
    return (float)y;
}

struct gemm_ctx {
    int M, K, N, bs, fmt, bits;
    const uint8_t* wq; const uint16_t* ws; const uint16_t* wb;
    const int8_t* xq; const float* xs; const int32_t* xsum; float* y;
};

static void gemm_cols(const void* p, long n0, long n1) {
    const struct gemm_ctx* c = (const struct gemm_ctx*)p;
    for (long m = 0; m < c->M; ++m)
        for (long n = n0; n < n1; ++n)
            c->y[m * (long)c->N + n] =
                one_output(c->N, c->K, c->bs, c->fmt, c->bits, c->wq, c->ws, c->wb, c->xq, c->xs, c->xsum, m, n);
}

/* y [M][N] float32. */
int or_q4_gemm_bits(int M, int K, int N, int bs, int fmt, int bits, const uint8_t* wq,
                    const uint16_t* wscale, const uint16_t* wbias, const int8_t* xq,
                    const float* xs, const int32_t* xsum, float* y) {
    if (check_fmt_bits(K, bs, fmt, bits) || M < 0 || N < 0) return OR_BAD;
    struct gemm_ctx c = {M, K, N, bs, fmt, bits, wq, wscale, wbias, xq, xs, xsum, y};
    return for_ranges(N, gemm_cols, &c);
}

int or_q4_gemm(int M, int K, int N, int bs, int fmt, const uint8_t* wq,
               const uint16_t* wscale, const uint16_t* wbias, const int8_t* xq,
               const float* xs, const int32_t* xsum, float* y) {
    return or_q4_gemm_bits(M, K, N, bs, fmt, 4, wq, wscale, wbias, xq, xs, xsum, y);
}

/* y for the listed (ms[i], ns[i]) only. */
int or_q4_gemm_sample_bits(int M, int K, int N, int bs, int fmt, int bits, const uint8_t* wq,
                           const uint16_t* wscale, const uint16_t* wbias, const int8_t* xq,
                           const float* xs, const int32_t* xsum, int count, const int* ms,
                           const int* ns, float* y) {
    if (check_fmt_bits(K, bs, fmt, bits)) return OR_BAD;
    for (int i = 0; i < count; ++i) {
        if (ms[i] < 0 || ms[i] >= M || ns[i] < 0 || ns[i] >= N) return OR_BAD;
        y[i] = one_output(N, K, bs, fmt, bits, wq, wscale, wbias, xq, xs, xsum, ms[i], ns[i]);
    }
    return OR_OK;
}

int or_q4_gemm_sample(int M, int K, int N, int bs, int fmt, const uint8_t* wq,
                      const uint16_t* wscale, const uint16_t* wbias, const int8_t* xq,
                      const float* xs, const int32_t* xsum, int count, const int* ms,
                      const int* ns, float* y) {
    return or_q4_gemm_sample_bits(M, K, N, bs, fmt, 4, wq, wscale, wbias, xq, xs, xsum, count, ms, ns, y);
}

/* ------------------------------------------------------------------------ */
/* Q4_K ([cke]: 256-weight super-blocks, "w = d * q - m")                     */
/* ------------------------------------------------------------------------ */

#define QK 256
#define Q4K_BYTES 144

/* 6-bit fields f = 0..15 (sc[0..7] then m[0..7]) little-endian in 12 bytes. */
void or_q4k_pack_scales(const uint8_t* sc, const uint8_t* mn, uint8_t* out12) {
    memset(out12, 0, 12);
    for (int f = 0; f < 16; ++f) {
        int v = (f < 8) ? sc[f] : mn[f - 8];
        for (int t = 0; t < 6; ++t) {
            int pos = 6 * f + t;
            if ((v >> t) & 1) out12[pos / 8] |= (uint8_t)(1u << (pos % 8));
        }
    }
}

void or_q4k_unpack_scales(const uint8_t* in12, uint8_t* sc, uint8_t* mn) {
    for (int f = 0; f < 16; ++f) {
        int v = 0;
        for (int t = 0; t < 6; ++t) {
            int pos = 6 * f + t;
            v |= ((in12[pos / 8] >> (pos % 8)) & 1) << t;
        }
        if (f < 8) sc[f] = (uint8_t)v; else mn[f - 8] = (uint8_t)v;
    }
}

/* Code of weight i (0..255) of a super-block, per the gemv_q4_k_ref code map:
 * chunk c = i / 64 uses qs[32 c .. 32 c + 31]; its first 32 weights are the
 * low nibbles (sub-block 2 c), the next 32 the high nibbles (sub-block 2 c + 1). */
static int q4k_code(const uint8_t* qs, int i, int* sub) {
    int c = i / 64, r = i % 64;
    if (r < 32) { *sub = 2 * c; return qs[32 * c + r] & 0x0F; }
    *sub = 2 * c + 1;
    return qs[32 * c + r - 32] >> 4;
}

static void q4k_put_code(uint8_t* qs, int i, int q) {
    int c = i / 64, r = i % 64;
    if (r < 32) qs[32 * c + r] = (uint8_t)((qs[32 * c + r] & 0xF0) | (q & 0x0F));
    else qs[32 * c + r - 32] = (uint8_t)((qs[32 * c + r - 32] & 0x0F) | ((q & 0x0F) << 4));
}

/* Dequantized weight i of one 144-byte block, exact in double. */
static double q4k_weight(const uint8_t* blk, int i) {
    uint16_t d16, dm16;
    memcpy(&d16, blk, 2);
    memcpy(&dm16, blk + 2, 2);
    uint8_t sc[8], mn[8];
    or_q4k_unpack_scales(blk + 4, sc, mn);
    int sub;
    int q = q4k_code(blk + 16, i, &sub);
    double d = (double)or_f16_to_f32(d16), dmin = (double)or_f16_to_f32(dm16);
    return d * (double)sc[sub] * (double)q - dmin * (double)mn[sub];
}

/* Dequantize rows of Q4_K weights to double (for tests). w [N][K]. */
int or_q4k_dequant(int N, int K, const uint8_t* blocks, double* w) {
    if (N < 0 || K <= 0 || K % QK != 0) return OR_BAD;
    int nb = K / QK;
    for (long n = 0; n < N; ++n)
        for (int b = 0; b < nb; ++b) {
            const uint8_t* blk = blocks + (n * nb + b) * (long)Q4K_BYTES;
            for (int i = 0; i < QK; ++i) w[n * (long)K + (long)b * QK + i] = q4k_weight(blk, i);
        }
    return OR_OK;
}

/* Quantizer (data generation): per 32-weight sub-block lo = min(0, min w),
 * hi = max w, a = (hi - lo) / 15, b = -lo; d = fp16(max a / 63),
 * dmin = fp16(max b / 63); sc = rne(a / d), m = rne(b / dmin) clamped to 0..63;
 * q = clamp(rne((w + dmin m) / (d sc)), 0, 15). All steps in float32. */
int or_quantize_q4k(int N, int K, const float* w, uint8_t* blocks) {
    if (N < 0 || K <= 0 || K % QK != 0) return OR_BAD;
    int nb = K / QK;
    for (long n = 0; n < N; ++n)
        for (int b = 0; b < nb; ++b) {
            const float* x = w + n * (long)K + (long)b * QK;
            uint8_t* blk = blocks + (n * nb + b) * (long)Q4K_BYTES;
            float a[8], bb[8], amax = 0.0f, bmax = 0.0f;
            for (int s = 0; s < 8; ++s) {
                float lo = 0.0f, hi = x[32 * s];
                for (int j = 0; j < 32; ++j) {
                    float v = x[32 * s + j];
                    if (v < lo) lo = v;
                    if (v > hi) hi = v;
                }
                a[s] = (hi - lo) / 15.0f;
                bb[s] = -lo;
                if (a[s] > amax) amax = a[s];
                if (bb[s] > bmax) bmax = bb[s];
            }
            uint16_t d16 = or_f32_to_f16(amax / 63.0f);
            uint16_t dm16 = or_f32_to_f16(bmax / 63.0f);
            float d = or_f16_to_f32(d16), dmin = or_f16_to_f32(dm16);
            uint8_t sc[8], mn[8];
            for (int s = 0; s < 8; ++s) {
                int v = 0, u = 0;
                if (d != 0.0f) { v = (int)nearbyintf(a[s] / d); if (v < 0) v = 0; if (v > 63) v = 63; }
                if (dmin != 0.0f) { u = (int)nearbyintf(bb[s] / dmin); if (u < 0) u = 0; if (u > 63) u = 63; }
                sc[s] = (uint8_t)v;
                mn[s] = (uint8_t)u;
            }
            memset(blk, 0, Q4K_BYTES);
            memcpy(blk, &d16, 2);
            memcpy(blk + 2, &dm16, 2);
            or_q4k_pack_scales(sc, mn, blk + 4);
            for (int i = 0; i < QK; ++i) {
                int s = i / 32;                  /* sub-block of weight i (0..7) */
                float ds = d * (float)sc[s];
                float dm = dmin * (float)mn[s];
                int q = 0;
                if (ds != 0.0f) {
                    float t = x[i] + dm;
                    q = (int)nearbyintf(t / ds);
                    if (q < 0) q = 0;
                    if (q > 15) q = 15;
                }
                q4k_put_code(blk + 16, i, q);
            }
        }
    return OR_OK;
}

/* One output: y[m][n] = sum_k w^[n,k] * x[m,k], in double, rounded once. */
static float q4k_one(int K, const uint8_t* blocks, const float* x, long m, long n) {
    int nb = K / QK;
    double y = 0.0;
    for (int b = 0; b < nb; ++b) {
        const uint8_t* blk = blocks + (n * nb + b) * (long)Q4K_BYTES;
        for (int i = 0; i < QK; ++i)
            y += q4k_weight(blk, i) * (double)x[m * (long)K + (long)b * QK + i];
    }
    return (float)y;
}

/* [cke] gemm_q4_k_ref: the GEMM is one GEMV per activation row.
 * x [M][K] float32, blocks [N][K/256] x 144 B, y [M][N]. */
struct q4k_gemm_ctx { int M, K, N; const uint8_t* blocks; const float* x; float* y; };

static void q4k_cols(const void* p, long n0, long n1) {
    const struct q4k_gemm_ctx* c = (const struct q4k_gemm_ctx*)p;
    for (long m = 0; m < c->M; ++m)
        for (long n = n0; n < n1; ++n) c->y[m * (long)c->N + n] = q4k_one(c->K, c->blocks, c->x, m, n);
}

int or_q4k_gemv(int K, int N, const uint8_t* blocks, const float* x, float* y) {
    if (K <= 0 || K % QK != 0 || N < 0) return OR_BAD;
    struct q4k_gemm_ctx c = {1, K, N, blocks, x, y};
    return for_ranges(N, q4k_cols, &c);
}

int or_q4k_gemm(int M, int K, int N, const uint8_t* blocks, const float* x, float* y) {
    if (M < 0 || K <= 0 || K % QK != 0 || N < 0) return OR_BAD;
    struct q4k_gemm_ctx c = {M, K, N, blocks, x, y};
    return for_ranges(N, q4k_cols, &c);
}

int or_q4k_gemm_sample(int M, int K, int N, const uint8_t* blocks, const float* x,
                       int count, const int* ms, const int* ns, float* y) {
    if (K <= 0 || K % QK != 0) return OR_BAD;
    for (int i = 0; i < count; ++i) {
        if (ms[i] < 0 || ms[i] >= M || ns[i] < 0 || ns[i] >= N) return OR_BAD;
        y[i] = q4k_one(K, blocks, x, ms[i], ns[i]);
    }
    return OR_OK;
}

/* ------------------------------------------------------------------------ */
/* Input gradient with frozen weights ([cke] section "Backward Pass:         */
/* Gradient w.r.t. Input": dL/dX = W^T . dL/dY with the weights dequantized  */
/* on the fly and no weight gradient; its batched form is one such product   */
/* per activation row).                                                       */
/* ------------------------------------------------------------------------ */

/* Dequantized Q4_0 or affine weight (n, k), exact in double. */
static double w4_weight(int K, int bs, int fmt, const uint8_t* wq, const uint16_t* wscale,
                        const uint16_t* wbias, long n, int k) {
    int nb = K / bs, b = k / bs;
    int q = get_code(wq + n * (long)(K / 2), k);
    if (fmt == 0) return (double)or_f16_to_f32(wscale[n * nb + b]) * (double)(q - 8);
    return (double)or_bf16_to_f32(wscale[n * nb + b]) * (double)q + (double)or_bf16_to_f32(wbias[n * nb + b]);
}

/* dx[m][k] = sum_n dy[m][n] * w^[n][k]: every term exact in double, summed in
 * n order, rounded once to float. dy [M][N], dx [M][K] float32. The weights
 * are dequantized one row at a time (w_row), each row once. */
static int backward_rows(int M, int K, int N, const float* dy, float* dx,
                         double (*weight)(const void* ctx, long n, int k), const void* ctx) {
    double* acc = (double*)calloc((size_t)M * K + 1, sizeof(double));
    double* w_row = (double*)malloc(((size_t)K + 1) * sizeof(double));
    if (!acc || !w_row) { free(acc); free(w_row); return OR_BAD; }
    for (long n = 0; n < N; ++n) {
        for (int k = 0; k < K; ++k) w_row[k] = weight(ctx, n, k);
        for (long m = 0; m < M; ++m) {
            double g = (double)dy[m * (long)N + n];
            for (int k = 0; k < K; ++k) acc[m * (long)K + k] += g * w_row[k];
        }
    }
    for (long i = 0; i < (long)M * K; ++i) dx[i] = (float)acc[i];
    free(acc);
    free(w_row);
    return OR_OK;
}

struct q4k_ctx { int K; const uint8_t* blocks; };
static double q4k_ctx_weight(const void* c, long n, int k) {
    const struct q4k_ctx* x = (const struct q4k_ctx*)c;
    int nb = x->K / QK;
    return q4k_weight(x->blocks + (n * nb + k / QK) * (long)Q4K_BYTES, k % QK);
}

struct w4_ctx { int K, bs, fmt; const uint8_t* wq; const uint16_t* ws; const uint16_t* wb; };
static double w4_ctx_weight(const void* c, long n, int k) {
    const struct w4_ctx* x = (const struct w4_ctx*)c;
    return w4_weight(x->K, x->bs, x->fmt, x->wq, x->ws, x->wb, n, k);
}

int or_q4k_backward(int M, int K, int N, const uint8_t* blocks, const float* dy, float* dx) {
    if (M < 0 || N < 0 || K <= 0 || K % QK != 0) return OR_BAD;
    struct q4k_ctx c = {K, blocks};
    return backward_rows(M, K, N, dy, dx, q4k_ctx_weight, &c);
}

int or_q4_backward(int M, int K, int N, int bs, int fmt, const uint8_t* wq, const uint16_t* wscale,
                   const uint16_t* wbias, const float* dy, float* dx) {
    if (check_fmt(K, bs, fmt) || M < 0 || N < 0) return OR_BAD;
    struct w4_ctx c = {K, bs, fmt, wq, wscale, wbias};
    return backward_rows(M, K, N, dy, dx, w4_ctx_weight, &c);
}

/* dx for the listed (ms[i], ks[i]) only, same arithmetic. */
static int backward_sample(int M, int K, int N, const float* dy, int count, const int* ms, const int* ks,
                           float* dx, double (*weight)(const void* ctx, long n, int k), const void* ctx) {
    for (int i = 0; i < count; ++i) {
        if (ms[i] < 0 || ms[i] >= M || ks[i] < 0 || ks[i] >= K) return OR_BAD;
        double acc = 0.0;
        for (long n = 0; n < N; ++n) acc += (double)dy[ms[i] * (long)N + n] * weight(ctx, n, ks[i]);
        dx[i] = (float)acc;
    }
    return OR_OK;
}

int or_q4k_backward_sample(int M, int K, int N, const uint8_t* blocks, const float* dy, int count,
                           const int* ms, const int* ks, float* dx) {
    if (K <= 0 || K % QK != 0) return OR_BAD;
    struct q4k_ctx c = {K, blocks};
    return backward_sample(M, K, N, dy, count, ms, ks, dx, q4k_ctx_weight, &c);
}

int or_q4_backward_sample(int M, int K, int N, int bs, int fmt, const uint8_t* wq, const uint16_t* wscale,
                          const uint16_t* wbias, const float* dy, int count, const int* ms, const int* ks,
                          float* dx) {
    if (check_fmt(K, bs, fmt)) return OR_BAD;
    struct w4_ctx c = {K, bs, fmt, wq, wscale, wbias};
    return backward_sample(M, K, N, dy, count, ms, ks, dx, w4_ctx_weight, &c);
}
