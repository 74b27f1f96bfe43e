/*
 * mmb_oracle.c -- plain CPU reference for the backward pass of a GPT-2
 * linear layer  out = inp . W^T + bias.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may call, link or
 * load this file or the library built from it; only the tests, the smoke
 * check and the benchmark's CPU-baseline leg do.  It shares no code, header,
 * table or helper with the HIP kernels.
 *
 * Source of the method: the llm.c page "dev/cuda/matmul_backward.cu"
 * (CPU reference `matmul_backward_cpu`, cuBLAS launcher `matmul_backward1`,
 * bias kernels `matmul_backward_bias_kernel_naive/_faster`).  The three
 * results have a plain definition, so this file writes that definition out,
 * element by element, in IEEE double:
 *
 *   dinp[r,i]    <- dinp[r,i]    + sum_{o<OC} dout[r,o] * weight[o,i]
 *   dweight[o,i] <- dweight[o,i] + sum_{r<BT} dout[r,o] * inp[r,i]
 *   dbias[o]     <- sum_{r<BT} dout[r,o]          (written, not added)
 *
 * and, for the forward whose gradients these are,
 *
 *   out[r,o]     <- sum_{i<C} inp[r,i] * weight[o,i] (+ bias[o])   (written)
 *
 * plus the stochastic rounding of bf16 gradients and the LayerNorm backward
 * (the adjacent op of the same model) described further down.
 *
 * with r running over the B*T rows.  All tensors are dense row-major:
 * inp [BT,C], dout [BT,OC], weight [OC,C], dinp [BT,C], dweight [OC,C],
 * dbias [OC].  The gradients of dinp and dweight add onto what the buffers
 * already hold (the page's launcher calls its GEMMs with beta = 1 for that
 * reason); dbias is assigned, as in every version on the page.
 *
 * Parallelism (OpenMP) only splits independent output elements: rows of
 * dinp, rows (output channels) of dweight and entries of dbias, as the page's
 * CPU reference does.  Each output element is one sequential double sum, so
 * the result does not depend on the thread count.
 */
#include <stddef.h>
#include <stdint.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Gradient with respect to the input: one dot product of length OC per
 * output element (matmul_backward_cpu, first pass; the dinp GEMM of
 * matmul_backward1). */
void mmb_oracle_dinp(double* dinp, const double* dout, const double* weight,
                     long B, long T, long C, long OC)
{
    const long BT = B * T;
#pragma omp parallel for schedule(static)
    for (long r = 0; r < BT; r++) {
        for (long i = 0; i < C; i++) {
            double s = 0.0;
            for (long o = 0; o < OC; o++)
                s += dout[r * OC + o] * weight[o * C + i];
            dinp[r * C + i] = dinp[r * C + i] + s;
        }
    }
}

/* Gradient with respect to the weight: one dot product of length B*T per
 * output element, over the rows of dout and inp (matmul_backward_cpu,
 * second pass; the dweight GEMM of matmul_backward1). */
void mmb_oracle_dweight(double* dweight, const double* dout, const double* inp,
                        long B, long T, long C, long OC)
{
    const long BT = B * T;
#pragma omp parallel for schedule(static)
    for (long o = 0; o < OC; o++) {
        for (long i = 0; i < C; i++) {
            double s = 0.0;
            for (long r = 0; r < BT; r++)
                s += dout[r * OC + o] * inp[r * C + i];
            dweight[o * C + i] = dweight[o * C + i] + s;
        }
    }
}

/* Gradient with respect to the bias: the sum of each dout column over all
 * B*T rows, assigned to dbias (matmul_backward_bias_kernel_naive). */
void mmb_oracle_dbias(double* dbias, const double* dout, long B, long T, long OC)
{
    const long BT = B * T;
#pragma omp parallel for schedule(static)
    for (long o = 0; o < OC; o++) {
        double s = 0.0;
        for (long r = 0; r < BT; r++)
            s += dout[r * OC + o];
        dbias[o] = s;
    }
}

/* The whole backward pass: dinp and dweight accumulate, dbias (when not
 * NULL) is overwritten (matmul_backward1, including its dbias != NULL test). */
void mmb_oracle_backward(double* dinp, double* dweight, double* dbias,
                         const double* dout, const double* inp, const double* weight,
                         long B, long T, long C, long OC)
{
    mmb_oracle_dinp(dinp, dout, weight, B, T, C, OC);
    mmb_oracle_dweight(dweight, dout, inp, B, T, C, OC);
    if (dbias != NULL)
        mmb_oracle_dbias(dbias, dout, B, T, OC);
}

/* The forward of the same layer, whose gradients the functions above are:
 * out[r,o] = sum_{i<C} inp[r,i] * weight[o,i] (+ bias[o] when bias is not
 * NULL), one dot product of length C per output element.  The page's
 * launcher recalls this product in its comments (one GEMM with the weight
 * transposed, alpha = 1, beta = 0: out is assigned, never accumulated); the
 * bias term is the b of out = inp . W^T + b whose gradient dbias is.
 * out is [BT,OC]. */
void mmb_oracle_forward(double* out, const double* inp, const double* weight,
                        const double* bias, long B, long T, long C, long OC)
{
    const long BT = B * T;
#pragma omp parallel for schedule(static)
    for (long r = 0; r < BT; r++) {
        for (long o = 0; o < OC; o++) {
            double s = 0.0;
            for (long i = 0; i < C; i++)
                s += inp[r * C + i] * weight[o * C + i];
            out[r * OC + o] = bias != NULL ? s + bias[o] : s;
        }
    }
}

/* ---- LayerNorm backward ---------------------------------------------------
 *
 * The llm.c page "dev/cuda/layernorm_backward.cu", CPU reference
 * layernorm_backward_cpu: for every row r of B*T rows of C channels, with
 * the forward's saved mean[r] and rstd[r],
 *   norm_i  = (inp[r,i] - mean[r]) * rstd[r]
 *   dnorm_i = weight[i] * dout[r,i]
 *   a = (1/C) sum_i dnorm_i,   b = (1/C) sum_i dnorm_i * norm_i
 *   dbias[i]   += dout[r,i]
 *   dweight[i] += norm_i * dout[r,i]
 *   dinp[r,i]  += (dnorm_i - a - norm_i * b) * rstd[r]
 * All three outputs accumulate onto their buffers, as on the page.  Rows are
 * independent for dinp (OpenMP over rows); dweight and dbias sum over rows,
 * so they are computed column by column (OpenMP over channels), each one
 * sequential double sum in row order. */
void mmb_oracle_layernorm_backward(double* dinp, double* dweight, double* dbias,
                                   const double* dout, const double* inp, const double* weight,
                                   const double* mean, const double* rstd,
                                   long B, long T, long C)
{
    const long BT = B * T;
#pragma omp parallel for schedule(static)
    for (long r = 0; r < BT; r++) {
        const double* d = dout + r * C;
        const double* x = inp + r * C;
        double a = 0.0, b = 0.0;
        for (long i = 0; i < C; i++) {
            const double norm = (x[i] - mean[r]) * rstd[r];
            const double dnorm = weight[i] * d[i];
            a += dnorm;
            b += dnorm * norm;
        }
        a /= (double)C;
        b /= (double)C;
        for (long i = 0; i < C; i++) {
            const double norm = (x[i] - mean[r]) * rstd[r];
            const double dnorm = weight[i] * d[i];
            dinp[r * C + i] += (dnorm - a - norm * b) * rstd[r];
        }
    }
#pragma omp parallel for schedule(static)
    for (long i = 0; i < C; i++) {
        double sw = 0.0, sb = 0.0;
        for (long r = 0; r < BT; r++) {
            const double norm = (inp[r * C + i] - mean[r]) * rstd[r];
            sb += dout[r * C + i];
            sw += norm * dout[r * C + i];
        }
        dbias[i] += sb;
        dweight[i] += sw;
    }
}

/* ---- stochastic rounding of bf16 gradients ------------------------------
 *
 * The llm.c encoder page writes bf16 parameter gradients with stochastic
 * rounding: the fp32 value  accumulated sum + old value  is rounded up or
 * down to a neighbouring bf16 at random, with a deterministic seed per
 * element, so that the rounding is unbiased and runs repeat bit for bit.
 * The page does not show its hash.  Here the random bits come from
 * Philox-4x64 with 10 rounds (Salmon, Moraes, Dror and Shaw, "Parallel
 * random numbers: as easy as 1, 2, 3", SC 2011), keyed by (seed, tag),
 * tag 1 for dweight and 2 for dbias.  Element (row, col) of a row-major
 * gradient takes the call with counter (row, 2*(col/32) + (col/4)%2, 0, 0)
 * and uses bits 16*(col%4) .. 16*(col%4)+15 of output word (col%32)/8: one
 * call covers 16 elements of a row.  The fp32 value x (the exact result
 * rounded to nearest fp32) becomes the upper half of  bits(x) + r16:  it
 * rounds away from zero exactly when the 16 discarded bits plus r16 carry,
 * i.e. with probability (discarded bits)/65536.  Non-finite values round to
 * nearest. */

/* Philox-4x64-10: ten rounds of two 64x64->128-bit products with the
 * published multipliers, the key bumped by the published Weyl constants
 * between rounds. */
void mmb_oracle_philox4x64_10(const uint64_t ctr[4], const uint64_t key[2], uint64_t out[4])
{
    const uint64_t M0 = 0xD2E7470EE14C6C93ULL, M1 = 0xCA5A826395121157ULL;
    const uint64_t W0 = 0x9E3779B97F4A7C15ULL, W1 = 0xBB67AE8584CAA73BULL;
    uint64_t c0 = ctr[0], c1 = ctr[1], c2 = ctr[2], c3 = ctr[3];
    uint64_t k0 = key[0], k1 = key[1];
    for (int round = 0; round < 10; round++) {
        const unsigned __int128 p0 = (unsigned __int128)M0 * c0;
        const unsigned __int128 p1 = (unsigned __int128)M1 * c2;
        const uint64_t hi0 = (uint64_t)(p0 >> 64), lo0 = (uint64_t)p0;
        const uint64_t hi1 = (uint64_t)(p1 >> 64), lo1 = (uint64_t)p1;
        c0 = hi1 ^ c1 ^ k0;
        c1 = lo1;
        c2 = hi0 ^ c3 ^ k1;
        c3 = lo0;
        k0 += W0;
        k1 += W1;
    }
    out[0] = c0;
    out[1] = c1;
    out[2] = c2;
    out[3] = c3;
}

/* The 16 random bits of element (row, col) of the gradient `tag`. */
uint32_t mmb_oracle_sr_bits(uint64_t seed, uint64_t tag, uint64_t row, uint64_t col)
{
    const uint64_t ctr[4] = {row, 2 * (col / 32) + (col / 4) % 2, 0, 0};
    const uint64_t key[2] = {seed, tag};
    uint64_t w[4];
    mmb_oracle_philox4x64_10(ctr, key, w);
    return (uint32_t)((w[(col % 32) / 8] >> (16 * (col % 4))) & 0xFFFF);
}

/* bf16 bits of x rounded with the random bits r16 (0 <= r16 < 65536). */
uint16_t mmb_oracle_sr_bf16(float x, uint32_t r16)
{
    uint32_t u;
    memcpy(&u, &x, 4);
    if ((u & 0x7F800000u) == 0x7F800000u)
        return (uint16_t)((u >> 16) | ((u & 0x007FFFFFu) ? 0x0040u : 0u));
    return (uint16_t)((u + r16) >> 16);
}

/* out[r*cols + c] = stochastic bf16 rounding of exact[r*cols + c] (each value
 * first rounded to nearest fp32), with the bits of element (r, c) of `tag`. */
void mmb_oracle_round_sr(uint16_t* out, const double* exact, long rows, long cols,
                         uint64_t seed, uint64_t tag)
{
#pragma omp parallel for schedule(static)
    for (long r = 0; r < rows; r++)
        for (long c = 0; c < cols; c++)
            out[r * cols + c] = mmb_oracle_sr_bf16((float)exact[r * cols + c],
                                                   mmb_oracle_sr_bits(seed, tag, (uint64_t)r,
                                                                      (uint64_t)c));
}

/* Number of OpenMP threads a parallel region above would use. */
int mmb_oracle_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
