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

/* Number of OpenMP threads a parallel region above would use. */
int mmb_oracle_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
