/*
 * ecmd_oracle.c -- reference evaluator for elementwise tensor Commands.
 *
 * TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only the test suite, the smoke check
 * and the benchmark's CPU-baseline leg may load this library.  It shares no
 * source, header, table or helper with the GPU library; it is deliberately
 * plain and slow so that a reader can check it against the definitions by eye.
 *
 * What it computes (rocRoller "Design Overview", sections "Command Class",
 * "Operations" and "CommandArgument"): a Command is a list of operations in
 * insertion order.  Each operation gets a tag; later operations name earlier
 * results by tag.  Loads read a tensor argument, scalars read a scalar
 * argument, T_Execute E_ operations (Add, Sub, Mul, Neg and type conversions)
 * combine earlier tags, and stores write a tag's value to an output tensor.
 * Argument values (pointers, strides, scalar bits) arrive at execution time.
 *
 * For every logical index p = (i0, i1, i2, i3) of the common shape, in
 * row-major order, the oracle walks the operations in insertion order, keeps
 * one value per tag (so a shared subexpression is computed once per element),
 * and then performs every store.  A tensor view maps p to element offset
 * i0*s0 + i1*s1 + i2*s2 + i3*s3 (rocRoller "Design Overview", section "Kernel
 * Graph": a dimension has a size and a stride; Flatten gives the row-major
 * contiguous index).
 *
 * Arithmetic rules (readings written out in the design notes):
 *   int32 : two's-complement, every op modulo 2^32 (done in uint32_t).
 *   fp32  : IEEE 754 binary32, round to nearest even, each op rounded on its
 *           own (this file must be compiled with -ffp-contract=off), subnormals
 *           kept (Silk "AMDGPU Backend", section "Code Object Format": the
 *           default execution mode keeps FP32/FP16 denormals, mode 3).
 *   Neg   : IEEE negate, i.e. flip the sign bit (int32: 0 - a mod 2^32).
 *   Abs   : clear the sign bit (int32: |INT_MIN| wraps to INT_MIN).
 *   Compare (EQ NE LT LE GT GE; LTU LEU GTU GEU on int32 as unsigned) gives
 *           int32 1 or 0; binary32 comparisons are IEEE (false with a NaN,
 *           except NE).  Min / Max: signed int32; binary32 ignores a NaN
 *           operand and orders -0 below +0.  Select(c, x, y) = c != 0 ? x : y.
 *   f16->f32 exact; f32->f16 and i32->f16 round to nearest even from the exact
 *   value, overflow to infinity, gradual underflow; i32->f32 round to nearest
 *   even; f32->i32 and f16->i32 truncate toward zero, saturate, NaN -> 0.
 *   f16 and bf16 (bfloat16: binary32's sign and 8-bit exponent with a 7-bit
 *   fraction) are compute types too: Add, Sub and Mul give the exact result
 *   rounded once to the operands' format (nearest even, overflow to infinity,
 *   gradual underflow).  The oracle forms the binary64 result and rounds that;
 *   binary64 carries at least 2p + 2 bits for p = 11 and p = 8, so rounding
 *   twice gives the same value as rounding the exact result once (Figueroa,
 *   "When is double rounding innocuous?", 1995).  Conversions to f16 or bf16
 *   round the exact source value once; bf16->f32 and f16->bf16's source values
 *   are exact in binary64.  Compare, Min, Max, Abs, Neg and Select follow the
 *   binary32 rules on the values.
 *
 * Build: gcc -O2 -ffp-contract=off -fno-fast-math -fPIC -shared -pthread
 */
#include <fenv.h>
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <xmmintrin.h>

#define OR_F16 1
#define OR_F32 2
#define OR_I32 3
#define OR_BF16 4

#define OR_LOAD 1
#define OR_SCALAR 2
#define OR_OP 3

#define OR_ADD 1
#define OR_SUB 2
#define OR_MUL 3
#define OR_NEG 4
#define OR_CVT 5
/* comparisons give int32 1 (true) or 0 (false); *_U compare int32 bit patterns as unsigned */
#define OR_CMP_EQ 6
#define OR_CMP_NE 7
#define OR_CMP_LT 8
#define OR_CMP_LE 9
#define OR_CMP_GT 10
#define OR_CMP_GE 11
#define OR_CMP_LTU 12
#define OR_CMP_LEU 13
#define OR_CMP_GTU 14
#define OR_CMP_GEU 15
#define OR_MIN 16
#define OR_MAX 17
#define OR_ABS 18
#define OR_SELECT 19   /* a != 0 ? b : c */

/* One tag of the Command.  kind = load / scalar / op.  For an op, a, b and c
 * are earlier tags (-1 when the operation has fewer operands; only Select has
 * three).  For a load or scalar, arg is the CommandArgument index it reads. */
typedef struct {
    int32_t kind, dtype, op, a, b, c, arg;
} oracle_node;

/* One store: write tag's value through the view of argument arg. */
typedef struct {
    int32_t tag, arg;
} oracle_store;

/* One CommandArgument value.  Tensors: base pointer and element strides of
 * the view over the 4-D logical shape (a view of rank k < 4 has its sizes
 * right-aligned: strides of the missing leading dimensions are 0).
 * Scalars: bits. */
typedef struct {
    void *ptr;
    int64_t stride[4];
    uint32_t bits;
    int32_t dtype;
} oracle_arg;

/* ------------------------------------------------------------------------ */
/* Bit <-> value helpers.                                                    */

static float f32_from_bits(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t bits_from_f32(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

/* binary16 -> value, from the IEEE 754 definition of the format:
 * exponent field 0 is a subnormal m * 2^-24, field 31 is inf/NaN, otherwise
 * (1024 + m) * 2^(e - 25).  Every binary16 value is exactly a binary32 value. */
uint32_t oracle_f16_to_f32(uint16_t h)
{
    uint32_t sign = (uint32_t)(h >> 15);
    uint32_t e = (uint32_t)((h >> 10) & 0x1f);
    uint32_t m = (uint32_t)(h & 0x3ff);
    double mag;
    if (e == 31) {
        if (m == 0)
            return (sign << 31) | 0x7f800000u;       /* infinity */
        return (sign << 31) | 0x7fc00000u;           /* quiet NaN, payload dropped */
    }
    if (e == 0)
        mag = ldexp((double)m, -24);
    else
        mag = ldexp((double)(1024 + m), (int)e - 25);
    float f = (float)mag;                             /* exact: no rounding happens */
    uint32_t u = bits_from_f32(f);
    return (sign << 31) | u;
}

/* Exact real value (held in a double that represents it exactly) -> binary16,
 * round to nearest, ties to even.  The binary16 grid has spacing 2^-24 below
 * 2^-14 and 2^(k-10) in the binade [2^k, 2^(k+1)); a magnitude that rounds to
 * 2^16 or above is infinity. */
static uint16_t f16_round_from_exact(double v)
{
    if (isnan(v))
        return (uint16_t)((signbit(v) ? 0x8000u : 0u) | 0x7e00u);
    uint16_t sign = signbit(v) ? 0x8000u : 0u;
    double a = fabs(v);
    if (isinf(a))
        return sign | 0x7c00u;
    if (a == 0.0)
        return sign;
    int k;                                /* a = f * 2^k with f in [0.5, 1) */
    frexp(a, &k);
    int binade = k - 1;                   /* a in [2^binade, 2^(binade+1)) */
    int spacing_exp = binade < -14 ? -24 : binade - 10;
    double q = nearbyint(ldexp(a, -spacing_exp));   /* exact scaling, RNE */
    double r = ldexp(q, spacing_exp);
    if (r >= 65536.0)
        return sign | 0x7c00u;
    if (r < ldexp(1.0, -14))              /* subnormal (or zero): field = r / 2^-24 */
        return sign | (uint16_t)q;
    frexp(r, &k);
    int e = k - 1;                        /* r may have moved up one binade */
    uint32_t mant = (uint32_t)(ldexp(r, 10 - e)) - 1024u;
    return sign | (uint16_t)(((uint32_t)(e + 15) << 10) | mant);
}

uint16_t oracle_f32_to_f16(uint32_t bits)
{
    return f16_round_from_exact((double)f32_from_bits(bits));  /* float -> double is exact */
}

/* bfloat16 -> value, from the format's definition: sign bit, 8-bit exponent
 * field with bias 127, 7-bit fraction.  Field 0 is a subnormal m * 2^-133,
 * field 255 is inf/NaN, otherwise (128 + m) * 2^(e - 134).  Every bfloat16
 * value is exactly a binary64 value. */
static double bf16_value(uint16_t h)
{
    int neg = (h >> 15) & 1;
    uint32_t e = (uint32_t)((h >> 7) & 0xff);
    uint32_t m = (uint32_t)(h & 0x7f);
    double mag;
    if (e == 255)
        mag = m == 0 ? INFINITY : NAN;
    else if (e == 0)
        mag = ldexp((double)m, -133);
    else
        mag = ldexp((double)(128 + m), (int)e - 134);
    return neg ? -mag : mag;
}

/* Exact real value (held in a double that represents it exactly, or is the
 * binary64 rounding of it, see the header) -> bfloat16, round to nearest,
 * ties to even.  The grid has spacing 2^-133 below 2^-126 and 2^(k-7) in the
 * binade [2^k, 2^(k+1)); a magnitude that rounds to 2^128 or above is
 * infinity.  NaN gives the quiet NaN of the same sign. */
static uint16_t bf16_round_from_exact(double v)
{
    uint16_t sign = signbit(v) ? 0x8000u : 0u;
    if (isnan(v))
        return sign | 0x7fc0u;
    double a = fabs(v);
    if (isinf(a))
        return sign | 0x7f80u;
    if (a == 0.0)
        return sign;
    int k;
    frexp(a, &k);
    int binade = k - 1;                   /* a in [2^binade, 2^(binade+1)) */
    int unit_exp = binade < -126 ? -133 : binade - 7;   /* grid spacing 2^unit_exp */
    double units = nearbyint(ldexp(a, -unit_exp));     /* a in grid units, to nearest even */
    double rounded = ldexp(units, unit_exp);
    if (rounded >= ldexp(1.0, 128))
        return sign | 0x7f80u;
    if (rounded < ldexp(1.0, -126))       /* subnormal (or zero): field = units of 2^-133 */
        return sign | (uint16_t)units;
    frexp(rounded, &k);
    int e = k - 1;                        /* the rounding may carry into the next binade */
    uint32_t fraction = (uint32_t)(ldexp(rounded, 7 - e)) - 128u;
    return sign | (uint16_t)(((uint32_t)(e + 127) << 7) | fraction);
}

/* binary16 -> value as a double (exact). */
static double f16_value(uint16_t h)
{
    return (double)f32_from_bits(oracle_f16_to_f32(h));
}

/* float -> int32: truncate toward zero, saturate at the int32 range, NaN -> 0. */
static int32_t i32_from_f32_sat(float f)
{
    if (isnan(f))
        return 0;
    if (f >= 2147483648.0f)
        return INT32_MAX;
    if (f < -2147483648.0f)
        return INT32_MIN;
    return (int32_t)truncf(f);
}

/* Value of a binary16 / bfloat16 / binary32 bit pattern as a double (exact). */
static double float_value(int dtype, uint32_t bits)
{
    if (dtype == OR_F16) return f16_value((uint16_t)bits);
    if (dtype == OR_BF16) return bf16_value((uint16_t)bits);
    return (double)f32_from_bits(bits);
}

/* Round an exact value to binary16 / bfloat16. */
static uint32_t round16(int dtype, double v)
{
    return dtype == OR_F16 ? f16_round_from_exact(v) : bf16_round_from_exact(v);
}

uint16_t oracle_f32_to_bf16(uint32_t bits) { return bf16_round_from_exact((double)f32_from_bits(bits)); }
uint32_t oracle_bf16_to_f32(uint16_t h) { return bits_from_f32((float)bf16_value(h)); }

/* Bulk helpers so the exhaustive conversion tests do not pay a call per value. */
void oracle_f32_to_f16_range(uint32_t first, uint64_t count, uint16_t *out)
{
    for (uint64_t k = 0; k < count; ++k)
        out[k] = oracle_f32_to_f16((uint32_t)(first + k));
}

void oracle_f16_to_f32_all(uint32_t *out)
{
    for (uint32_t h = 0; h < 65536; ++h)
        out[h] = oracle_f16_to_f32((uint16_t)h);
}

void oracle_f32_to_bf16_range(uint32_t first, uint64_t count, uint16_t *out)
{
    for (uint64_t k = 0; k < count; ++k)
        out[k] = oracle_f32_to_bf16((uint32_t)(first + k));
}

/* Floating-point environment: returns 0 when MXCSR has FTZ and DAZ clear and
 * round-to-nearest selected, and the C rounding mode is FE_TONEAREST. */
int oracle_check_fpenv(void)
{
    unsigned int csr = _mm_getcsr();
    int bad = 0;
    if (csr & (1u << 15)) bad |= 1;          /* FTZ */
    if (csr & (1u << 6)) bad |= 2;           /* DAZ */
    if (csr & (3u << 13)) bad |= 4;          /* RC != nearest */
    if (fegetround() != FE_TONEAREST) bad |= 8;
    return bad;
}

/* ------------------------------------------------------------------------ */
/* One E_ operation on bit patterns.                                         */

/* binary32 minimum / maximum: a NaN operand is ignored unless both are NaN,
 * and -0 counts as smaller than +0 (IEEE 754-2019 minimumNumber and
 * maximumNumber). */
static double min_number(double x, double y)
{
    if (isnan(x)) return y;
    if (isnan(y)) return x;
    if (x < y) return x;
    if (y < x) return y;
    return signbit(x) ? x : y;          /* equal: pick -0 over +0 */
}

static double max_number(double x, double y)
{
    if (isnan(x)) return y;
    if (isnan(y)) return x;
    if (x > y) return x;
    if (y > x) return y;
    return signbit(x) ? y : x;          /* equal: pick +0 over -0 */
}

static uint32_t compare(int op, int src_dtype, uint32_t a, uint32_t b)
{
    int r;
    if (op >= OR_CMP_LTU) {                     /* unsigned int32 */
        if (op == OR_CMP_LTU) r = a < b;
        else if (op == OR_CMP_LEU) r = a <= b;
        else if (op == OR_CMP_GTU) r = a > b;
        else r = a >= b;
    } else if (src_dtype == OR_I32) {           /* signed int32 */
        int32_t x = (int32_t)a, y = (int32_t)b;
        if (op == OR_CMP_EQ) r = x == y;
        else if (op == OR_CMP_NE) r = x != y;
        else if (op == OR_CMP_LT) r = x < y;
        else if (op == OR_CMP_LE) r = x <= y;
        else if (op == OR_CMP_GT) r = x > y;
        else r = x >= y;
    } else {                                    /* floats: C's IEEE comparisons on the exact values */
        double x = float_value(src_dtype, a), y = float_value(src_dtype, b);
        if (op == OR_CMP_EQ) r = x == y;
        else if (op == OR_CMP_NE) r = x != y;  /* true when either is NaN */
        else if (op == OR_CMP_LT) r = x < y;
        else if (op == OR_CMP_LE) r = x <= y;
        else if (op == OR_CMP_GT) r = x > y;
        else r = x >= y;
    }
    return r ? 1u : 0u;
}

static uint32_t apply_op(int op, int dst_dtype, int src_dtype, uint32_t a, uint32_t b, uint32_t c)
{
    if (op >= OR_CMP_EQ && op <= OR_CMP_GEU)
        return compare(op, src_dtype, a, b);
    if (op == OR_SELECT)
        return a != 0u ? b : c;
    if (op == OR_ABS) {
        if (dst_dtype == OR_I32) return (a & 0x80000000u) ? 0u - a : a;   /* |INT_MIN| wraps to INT_MIN */
        if (dst_dtype == OR_F32) return a & 0x7fffffffu;
        return a & 0x7fffu;                      /* binary16, bfloat16 */
    }
    if (op == OR_MIN || op == OR_MAX) {
        if (dst_dtype == OR_I32) {
            int32_t x = (int32_t)a, y = (int32_t)b;
            return (uint32_t)(op == OR_MIN ? (x < y ? x : y) : (x > y ? x : y));
        }
        /* the result is one of the operands, bits and all */
        double x = float_value(dst_dtype, a), y = float_value(dst_dtype, b);
        double m = op == OR_MIN ? min_number(x, y) : max_number(x, y);
        if (isnan(m)) return b;                  /* both NaN */
        if (m == x && m == y) return signbit(m) == signbit(x) ? a : b;
        return m == x ? a : b;
    }
    if (op == OR_CVT) {
        if (src_dtype == dst_dtype)
            return a;
        if (src_dtype == OR_F16 && dst_dtype == OR_F32)
            return oracle_f16_to_f32((uint16_t)a);
        if (src_dtype == OR_F32 && dst_dtype == OR_F16)
            return oracle_f32_to_f16(a);
        if (src_dtype == OR_I32 && dst_dtype == OR_F32)
            return bits_from_f32((float)(int32_t)a);            /* C: current mode, RNE */
        if (src_dtype == OR_I32 && dst_dtype == OR_F16)
            return f16_round_from_exact((double)(int32_t)a);    /* int32 -> double is exact */
        if (src_dtype == OR_F32 && dst_dtype == OR_I32)
            return (uint32_t)i32_from_f32_sat(f32_from_bits(a));
        if (src_dtype == OR_F16 && dst_dtype == OR_I32)
            return (uint32_t)i32_from_f32_sat(f32_from_bits(oracle_f16_to_f32((uint16_t)a)));
        /* bfloat16: every source value is exact in binary64; round it once */
        if (dst_dtype == OR_BF16)
            return src_dtype == OR_I32 ? bf16_round_from_exact((double)(int32_t)a)
                                       : bf16_round_from_exact(float_value(src_dtype, a));
        if (src_dtype == OR_BF16 && dst_dtype == OR_F16)
            return f16_round_from_exact(bf16_value((uint16_t)a));
        if (src_dtype == OR_BF16 && dst_dtype == OR_F32)
            return bits_from_f32((float)bf16_value((uint16_t)a));   /* exact */
        if (src_dtype == OR_BF16 && dst_dtype == OR_I32)
            return (uint32_t)i32_from_f32_sat((float)bf16_value((uint16_t)a));
        return 0;
    }
    if (op == OR_NEG) {
        if (dst_dtype == OR_I32) return 0u - a;
        if (dst_dtype == OR_F32) return a ^ 0x80000000u;
        return (a ^ 0x8000u) & 0xffffu;          /* binary16, bfloat16 */
    }
    if (dst_dtype == OR_I32) {
        if (op == OR_ADD) return a + b;
        if (op == OR_SUB) return a - b;
        return a * b;                        /* low 32 bits of the product */
    }
    if (dst_dtype == OR_F16 || dst_dtype == OR_BF16) {
        /* binary64 result of the exact operands, rounded once to the format */
        double x = float_value(dst_dtype, a), y = float_value(dst_dtype, b), z;
        if (op == OR_ADD) z = x + y;
        else if (op == OR_SUB) z = x - y;
        else z = x * y;
        return round16(dst_dtype, z);
    }
    /* dst_dtype == OR_F32 */
    float x = f32_from_bits(a), y = f32_from_bits(b), z;
    if (op == OR_ADD) z = x + y;
    else if (op == OR_SUB) z = x - y;
    else z = x * y;
    return bits_from_f32(z);
}

/* ------------------------------------------------------------------------ */
/* Element loop.                                                             */

static int64_t offset_of(const oracle_arg *g, const int64_t idx[4])
{
    return idx[0] * g->stride[0] + idx[1] * g->stride[1] + idx[2] * g->stride[2] + idx[3] * g->stride[3];
}

static uint32_t read_elem(const oracle_arg *g, const int64_t idx[4])
{
    int64_t off = offset_of(g, idx);
    if (g->dtype == OR_F16 || g->dtype == OR_BF16) {
        uint16_t h;
        memcpy(&h, (const char *)g->ptr + off * 2, 2);
        return h;
    }
    uint32_t u;
    memcpy(&u, (const char *)g->ptr + off * 4, 4);
    return u;
}

static void write_elem(const oracle_arg *g, const int64_t idx[4], uint32_t v)
{
    int64_t off = offset_of(g, idx);
    if (g->dtype == OR_F16 || g->dtype == OR_BF16) {
        uint16_t h = (uint16_t)v;
        memcpy((char *)g->ptr + off * 2, &h, 2);
    } else {
        memcpy((char *)g->ptr + off * 4, &v, 4);
    }
}

typedef struct {
    const oracle_node *nodes;
    int n_nodes;
    const oracle_store *stores;
    int n_stores;
    const oracle_arg *args;
    int64_t shape[4];
    int64_t first, last;     /* flat index range [first, last) */
} oracle_job;

static void *run_range(void *vp)
{
    const oracle_job *J = (const oracle_job *)vp;
    uint32_t *val = (uint32_t *)malloc(sizeof(uint32_t) * (size_t)(J->n_nodes > 0 ? J->n_nodes : 1));
    for (int64_t p = J->first; p < J->last; ++p) {
        int64_t idx[4], q = p;                 /* row-major: the last index varies fastest */
        for (int d = 3; d >= 0; --d) {
            idx[d] = q % J->shape[d];
            q /= J->shape[d];
        }
        for (int t = 0; t < J->n_nodes; ++t) {
            const oracle_node *n = &J->nodes[t];
            if (n->kind == OR_LOAD)
                val[t] = read_elem(&J->args[n->arg], idx);
            else if (n->kind == OR_SCALAR)
                val[t] = J->args[n->arg].bits;
            else
                val[t] = apply_op(n->op, n->dtype, J->nodes[n->a].dtype, val[n->a],
                                  n->b >= 0 ? val[n->b] : 0u, n->c >= 0 ? val[n->c] : 0u);
        }
        for (int s = 0; s < J->n_stores; ++s)
            write_elem(&J->args[J->stores[s].arg], idx, val[J->stores[s].tag]);
    }
    free(val);
    return NULL;
}

/* Evaluate the Command over the 4-D logical shape.  The caller (the oracle's
 * Python front end) has already checked tags, dtypes and shapes.  nthreads > 1
 * splits the flat index range into contiguous pieces; the result does not
 * depend on it.  Returns 0, or a nonzero code if the floating-point environment
 * is not IEEE default. */
int oracle_eval(const oracle_node *nodes, int n_nodes, const oracle_store *stores, int n_stores,
                const oracle_arg *args, const int64_t shape[4], int nthreads)
{
    if (oracle_check_fpenv() != 0)
        return -1;
    int64_t total = shape[0] * shape[1] * shape[2] * shape[3];
    if (total <= 0)
        return 0;
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    if ((int64_t)nthreads > total) nthreads = (int)total;
    oracle_job jobs[256];
    pthread_t th[256];
    for (int k = 0; k < nthreads; ++k) {
        jobs[k].nodes = nodes;
        jobs[k].n_nodes = n_nodes;
        jobs[k].stores = stores;
        jobs[k].n_stores = n_stores;
        jobs[k].args = args;
        for (int d = 0; d < 4; ++d) jobs[k].shape[d] = shape[d];
        jobs[k].first = total * k / nthreads;
        jobs[k].last = total * (k + 1) / nthreads;
    }
    if (nthreads == 1) {
        run_range(&jobs[0]);
        return 0;
    }
    for (int k = 0; k < nthreads; ++k)
        pthread_create(&th[k], NULL, run_range, &jobs[k]);
    for (int k = 0; k < nthreads; ++k)
        pthread_join(th[k], NULL);
    return 0;
}

int oracle_sizeof_node(void) { return (int)sizeof(oracle_node); }
int oracle_sizeof_store(void) { return (int)sizeof(oracle_store); }
int oracle_sizeof_arg(void) { return (int)sizeof(oracle_arg); }
