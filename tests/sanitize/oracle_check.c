/* The CPU oracle under AddressSanitizer / UndefinedBehaviorSanitizer: every
 * function on buffers allocated to their exact sizes (so any read or write
 * past a tensor is reported), over shapes with one row, one channel and
 * ragged sizes.  Test infrastructure only. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

void mmb_oracle_backward(double* dinp, double* dweight, double* dbias, const double* dout,
                         const double* inp, const double* weight, long B, long T, long C, long OC);
void mmb_oracle_forward(double* out, const double* inp, const double* weight, const double* bias,
                        long B, long T, long C, long OC);
void mmb_oracle_layernorm_backward(double* dinp, double* dweight, double* dbias,
                                   const double* dout, const double* inp, const double* weight,
                                   const double* mean, const double* rstd, long B, long T, long C);
void mmb_oracle_philox4x64_10(const uint64_t ctr[4], const uint64_t key[2], uint64_t out[4]);
uint32_t mmb_oracle_sr_bits(uint64_t seed, uint64_t tag, uint64_t row, uint64_t col);
uint16_t mmb_oracle_sr_bf16(float x, uint32_t r16);
void mmb_oracle_round_sr(uint16_t* out, const double* exact, long rows, long cols, uint64_t seed,
                         uint64_t tag);
int mmb_oracle_threads(void);

static double* vec(long n) {
    double* p = (double*)malloc((size_t)(n > 0 ? n : 1) * sizeof(double));
    for (long i = 0; i < n; ++i) p[i] = (double)((i * 7919) % 17) / 8.0 - 1.0;
    return p;
}

int main(void) {
    const long shapes[][4] = {{1, 1, 1, 1}, {2, 3, 5, 7}, {1, 17, 8, 3}, {3, 5, 33, 17}, {2, 16, 64, 192}};
    for (unsigned s = 0; s < sizeof(shapes) / sizeof(shapes[0]); ++s) {
        const long B = shapes[s][0], T = shapes[s][1], C = shapes[s][2], OC = shapes[s][3];
        const long BT = B * T;
        double *dinp = vec(BT * C), *dweight = vec(OC * C), *dbias = vec(OC);
        double *dout = vec(BT * OC), *inp = vec(BT * C), *weight = vec(OC * C), *out = vec(BT * OC);
        mmb_oracle_backward(dinp, dweight, dbias, dout, inp, weight, B, T, C, OC);
        mmb_oracle_backward(dinp, dweight, NULL, dout, inp, weight, B, T, C, OC);
        mmb_oracle_forward(out, inp, weight, dbias, B, T, C, OC);
        mmb_oracle_forward(out, inp, weight, NULL, B, T, C, OC);
        double *mean = vec(BT), *rstd = vec(BT), *lw = vec(C), *lb = vec(C), *lg = vec(C);
        double* ldout = vec(BT * C);
        mmb_oracle_layernorm_backward(dinp, lw, lb, ldout, inp, lg, mean, rstd, B, T, C);
        free(ldout); free(lg);
        uint16_t* r = (uint16_t*)malloc((size_t)(OC * C) * sizeof(uint16_t));
        mmb_oracle_round_sr(r, dweight, OC, C, 1234, 1);
        free(r); free(mean); free(rstd); free(lw); free(lb);
        free(dinp); free(dweight); free(dbias); free(dout); free(inp); free(weight); free(out);
    }
    uint64_t ctr[4] = {1, 2, 3, 4}, key[2] = {5, 6}, o[4];
    mmb_oracle_philox4x64_10(ctr, key, o);
    unsigned acc = 0;
    for (uint32_t v = 0; v < 70000; v += 997) acc += mmb_oracle_sr_bf16((float)v * 1.37f, v & 0xFFFF);
    acc += mmb_oracle_sr_bits(1, 2, 3, 4) + (unsigned)mmb_oracle_threads();
    printf("ok %u %llu\n", acc, (unsigned long long)o[0]);
    return 0;
}
