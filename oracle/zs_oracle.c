/*
 * Step oracle: one rank's ZeRO-1/2 optimizer step, one element at a time.
 *
 * TEST INFRASTRUCTURE.  Only the tests, the package smoke check and the
 * benchmark's CPU-baseline leg load this library.  It shares no source,
 * header or table with the HIP library.  Build: plain C, -O2,
 * -ffp-contract=off, no fast-math, no flush-to-zero (oracle/build.py).
 *
 * What it computes, per shard element i (CS336 lecture 8 notes, "ZeRO-1 code
 * example": reduce-scatter the gradient, update only the own slice with the
 * rank-local fp32 moments, all-gather the updated parameters; core concepts:
 * bf16 param + bf16 grad + fp32 master + two fp32 Adam moments; DDP-to-ZeRO
 * blog section 3.3: the optimizer is AdamW):
 *
 *   g   = (G[0][i] + G[1][i] + ... + G[W-1][i]) / W    fp32, left to right,
 *         starting from G[0][i]; the sum is what the reduce-scatter computes
 *         (SUM op of the sketch) and the division turns it into the mean that
 *         the data-parallel prose describes (podcast summary, section "Data
 *         parallelism"; DDP-to-ZeRO blog section 2.1)
 *   m   = b1*m + (1-b1)*g
 *   v   = b2*v + (1-b2)*(g*g)
 *   den = sqrt(v)/sqrt(1-b2^t) + eps
 *   th  = th*(1-lr*wd) - (lr/(1-b1^t))*(m/den)       decoupled weight decay
 *   p   = bf16(th), round to nearest even
 *
 * Each statement is one fp32 operation, rounded once (no contraction).  The
 * per-call constants are computed in double from the float hyper-parameters
 * and rounded to float once.  The step counter t starts at 1.
 *
 * Parity pins: see tests/test_oracle_step.py (W=1 against a library AdamW,
 * the first-step closed form, beta=0 and lr=0 cases, float64 brute force,
 * the all-reduce = reduce-scatter + all-gather reassembly).
 */
#include <stdint.h>
#include <string.h>
#include <math.h>

typedef struct {
    float lr, beta1, beta2, eps, weight_decay;
} oracle_hp;

/* The per-call fp32 constants. out[] = {b1, b2, 1-b1, 1-b2, lr/bc1,
 * sqrt(bc2), 1-lr*wd, eps} with bc_k = 1 - beta_k^t. */
void oracle_constants(const oracle_hp* hp, int64_t t, float* out)
{
    double b1 = (double)hp->beta1;
    double b2 = (double)hp->beta2;
    double lr = (double)hp->lr;
    double wd = (double)hp->weight_decay;
    double bc1 = 1.0 - pow(b1, (double)t);
    double bc2 = 1.0 - pow(b2, (double)t);
    out[0] = (float)b1;
    out[1] = (float)b2;
    out[2] = (float)(1.0 - b1);
    out[3] = (float)(1.0 - b2);
    out[4] = (float)(lr / bc1);
    out[5] = (float)sqrt(bc2);
    out[6] = (float)(1.0 - lr * wd);
    out[7] = (float)hp->eps;
}

static float bf16_bits_to_float(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* fp32 -> bf16, round to nearest, ties to even.  NaN stays a quiet NaN with
 * its sign; finite values that round past the largest bf16 become +-Inf. */
static uint16_t float_to_bf16_rne(float f)
{
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    if ((u & 0x7fffffffu) > 0x7f800000u)          /* NaN */
        return (uint16_t)((u >> 16) | 0x0040u);
    uint32_t lsb = (u >> 16) & 1u;
    return (uint16_t)((u + 0x7fffu + lsb) >> 16);
}

void oracle_bf16_round(const float* in, uint16_t* out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = float_to_bf16_rne(in[i]);
}

/* Mean of the W bf16 gradient values of one element, fp32, fixed order. */
static float reduce_one(int32_t W, const uint16_t* grads, int64_t grad_stride,
                        int64_t i)
{
    float acc = bf16_bits_to_float(grads[i]);
    for (int32_t s = 1; s < W; ++s)
        acc = acc + bf16_bits_to_float(grads[(int64_t)s * grad_stride + i]);
    return acc / (float)W;
}

/* AdamW on one element; c[] from oracle_constants. */
static void adamw_one(float g, float* master, float* m, float* v,
                      uint16_t* p16, const float* c)
{
    float mi = (c[0] * *m) + (c[2] * g);
    float g2 = g * g;
    float vi = (c[1] * *v) + (c[3] * g2);
    float root = sqrtf(vi);
    float den = (root / c[5]) + c[7];
    float upd = mi / den;
    float th = (*master * c[6]) - (c[4] * upd);
    *m = mi;
    *v = vi;
    *master = th;
    if (p16)
        *p16 = float_to_bf16_rne(th);
}

/* Reduce-scatter arithmetic only: out[i] = mean over s of G[s][i]. */
void oracle_reduce_mean(int32_t W, const uint16_t* grads, int64_t grad_stride,
                        int64_t n, float* out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = reduce_one(W, grads, grad_stride, i);
}

/* AdamW only, on an already reduced fp32 gradient. */
void oracle_adamw(int64_t n, const float* grad, float* master, float* m,
                  float* v, uint16_t* param_bf16, const oracle_hp* hp,
                  int64_t t)
{
    float c[8];
    oracle_constants(hp, t, c);
    for (int64_t i = 0; i < n; ++i)
        adamw_one(grad[i], &master[i], &m[i], &v[i],
                  param_bf16 ? &param_bf16[i] : 0, c);
}

/* The whole step over n consecutive shard elements:
 * grads is [W][grad_stride] bf16 bits, element i of slice s at
 * grads[s*grad_stride + i]. */
void oracle_step(int32_t W, const uint16_t* grads, int64_t grad_stride,
                 int64_t n, float* master, float* m, float* v,
                 uint16_t* param_bf16, const oracle_hp* hp, int64_t t)
{
    float c[8];
    oracle_constants(hp, t, c);
    for (int64_t i = 0; i < n; ++i)
        adamw_one(reduce_one(W, grads, grad_stride, i),
                  &master[i], &m[i], &v[i],
                  param_bf16 ? &param_bf16[i] : 0, c);
}

/* Pure-bf16 variant (CS336 lecture 8 notes, "Core concepts" and "Code
 * example: FSDP": training in pure bf16 keeps 12 bytes per parameter, the
 * bf16 parameter, the bf16 gradient and the two fp32 Adam moments; there is
 * no fp32 master copy).  The parameter itself is the bf16 value: the step
 * reads it, applies the same AdamW statements in fp32 and rounds the result
 * back to bf16 (nearest even), so updates below half a bf16 ulp are lost.
 * param is [n] bf16 bits, read and written in place. */
void oracle_step_bf16(int32_t W, const uint16_t* grads, int64_t grad_stride,
                      int64_t n, uint16_t* param, float* m, float* v,
                      const oracle_hp* hp, int64_t t)
{
    float c[8];
    oracle_constants(hp, t, c);
    for (int64_t i = 0; i < n; ++i) {
        float g = reduce_one(W, grads, grad_stride, i);
        float mi = (c[0] * m[i]) + (c[2] * g);
        float g2 = g * g;
        float vi = (c[1] * v[i]) + (c[3] * g2);
        float root = sqrtf(vi);
        float den = (root / c[5]) + c[7];
        float upd = mi / den;
        float th = (bf16_bits_to_float(param[i]) * c[6]) - (c[4] * upd);
        m[i] = mi;
        v[i] = vi;
        param[i] = float_to_bf16_rne(th);
    }
}

/* Gradient accumulation into the local gradient bucket (podcast summary of
 * "Training at thousands of GPUs", sections "Motivation" and the glossary:
 * the global batch is split into micro-batches whose gradients are added up
 * one after another before a single optimizer step; DDP-to-ZeRO blog 3.3:
 * gradient_accumulation_steps).  The k micro-batch bf16 gradients of one
 * element are summed in fp32 in micro-batch order, starting from the first,
 * then divided by k (the mean over the micro-batches) and rounded to bf16
 * to nearest even: that bf16 bucket is what the reduce-scatter sends.
 * grads is [k][stride] bf16 bits; out is [n]. */
void oracle_accumulate(int32_t k, const uint16_t* grads, int64_t stride,
                       int64_t n, uint16_t* out)
{
    for (int64_t i = 0; i < n; ++i) {
        float acc = bf16_bits_to_float(grads[i]);
        for (int32_t j = 1; j < k; ++j)
            acc = acc + bf16_bits_to_float(grads[(int64_t)j * stride + i]);
        out[i] = float_to_bf16_rne(acc / (float)k);
    }
}
