/*
 * mmb.h -- C ABI of libmmb.so, the backward pass of a GPT-2 linear layer
 * (out = inp . W^T + bias) on AMD Instinct MI355X (gfx950), and the forward
 * product it is the gradient of (mmb_forward, below).
 *
 * Operation (llm.c page "dev/cuda/matmul_backward.cu": CPU reference
 * matmul_backward_cpu and the cuBLAS launcher matmul_backward1), with
 * BT = B*T rows:
 *
 *   dinp[r,i]    += sum_{o<OC} dout[r,o] * weight[o,i]     r<BT, i<C
 *   dweight[o,i] += sum_{r<BT} dout[r,o] * inp[r,i]        o<OC, i<C
 *   dbias[o]      = sum_{r<BT} dout[r,o]                   o<OC, if dbias != NULL
 *
 * dinp and dweight accumulate onto what the buffers already hold (gradients
 * of a parameter used several times add; the page's launcher runs both GEMMs
 * with beta = 1).  dbias is assigned, as in every version on that page.
 *
 * Layout: every tensor is dense and row-major, as on the page:
 *   inp [BT,C], dout [BT,OC], weight [OC,C], dinp [BT,C], dweight [OC,C],
 *   dbias [OC].
 *
 * dtype (one for all six tensors):
 *   MMB_FP32  IEEE fp32 storage, fp32 products and sums (no reduced-precision
 *             substitute; the page's check turns TF32 off).
 *   MMB_BF16  bfloat16 storage, exact products, fp32 accumulation over the
 *             whole reduction; each output is rounded to bf16 once, to
 *             nearest-even, from  float(old) + fp32 sum  (dinp, dweight) or
 *             the fp32 sum (dbias).
 *
 * Pointers are device pointers (hipMalloc or torch CUDA memory) owned by the
 * caller.  dout, inp, weight are read only; dinp and dweight are read and
 * written; dbias is written only.  Output buffers may not overlap each other
 * or any input (MMB_ERR_ALIAS).  Any alignment and any dims >= 1 are
 * accepted.  Calls take the MFMA path: directly when every streamed tensor is
 * 16-byte aligned and C and OC are multiples of 8 (bf16) or 4 (fp32);
 * otherwise each tensor whose rows are not whole 16-byte vectors (dout when
 * OC is ragged; inp, weight, dinp and dweight when C is) or whose address is
 * not 16-byte aligned is copied into an aligned, zero-padded row pitch in the
 * workspace first, and the outputs among them (dinp, dweight) are copied back
 * after (an extra pass over those tensors).  dbias needs no alignment.  Only
 * C or OC above 2^22, or a pointer not aligned to its element size, take the
 * much slower generic path (one thread per output element).
 *
 * The library owns only a per-(device, stream) workspace (split-K partial
 * sums, tile counters and work lists), allocated on first use, grown on
 * demand and freed by mmb_release().  Work is enqueued asynchronously; launch
 * errors are returned, faults during execution surface at the caller's next
 * synchronisation.  Results are deterministic: the same inputs give the same
 * bits on every run (no floating-point atomics; split-K partials are summed
 * in a fixed order).  Calls on different streams are independent; calls on
 * one stream are ordered by it.
 *
 * Blocking: no entry point but mmb_release waits for the device.  The first
 * call of a shape plans it on the host (up to about 0.1 s); the first call of
 * a plan on a stream allocates that stream's copy of the work list
 * (stream-ordered hipMallocAsync where the device supports memory pools) and
 * copies it from pinned host memory with hipMemcpyAsync; a workspace that is
 * too small is replaced in stream order (hipMallocAsync / hipFreeAsync).
 * Where memory pools are missing, plain hipMalloc is used and replaced
 * buffers are kept until mmb_release.
 *
 * Tuning variables (MMB_SPLITS_DWEIGHT, MMB_SPLITS_DINP, MMB_SPLITS_FWD,
 * MMB_PLAN_MODEL, MMB_PLAN_TRACE, MMB_LN_WORKGROUPS) are read from the
 * environment once, when the library is loaded; later changes to the
 * environment have no effect.  mmb_set_tuning replaces one at run time.
 *
 * All functions return MMB_OK (0) or a negative mmb_status; none of them
 * exits or aborts.
 */
#ifndef MMB_H
#define MMB_H

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MMB_FP32 = 0,
    MMB_BF16 = 1
} mmb_dtype;

typedef enum {
    MMB_OK = 0,
    MMB_ERR_NULL = -1,      /* a required pointer is NULL (only dbias may be)  */
    MMB_ERR_DIM = -2,       /* B, T, C or OC < 1                                */
    MMB_ERR_DTYPE = -3,     /* dtype is not an mmb_dtype                       */
    MMB_ERR_OVERFLOW = -4,  /* B*T >= 2^31                                      */
    MMB_ERR_ALIAS = -5,     /* an output range overlaps another buffer's range */
    MMB_ERR_HIP = -6,       /* a HIP runtime call or kernel launch failed      */
    MMB_ERR_NOMEM = -7,     /* the workspace could not be allocated            */
    MMB_ERR_NAME = -8,      /* mmb_set_tuning: not a tuning variable           */
    MMB_ERR_SCRATCH = -9    /* mmb_backward_noalloc: the call needs more than
                               MMB_NOALLOC_SCRATCH_BYTES of scratch            */
} mmb_status;

/* The backward pass on the calling thread's current device, enqueued on the
 * NULL (default) stream.  Arguments as in the file comment. */
int mmb_backward(void* dinp, void* dweight, void* dbias,
                 const void* dout, const void* inp, const void* weight,
                 int B, int T, int C, int OC, int dtype);

/* As mmb_backward, enqueued on `stream` (a hipStream_t; NULL = default). */
int mmb_backward_stream(void* dinp, void* dweight, void* dbias,
                        const void* dout, const void* inp, const void* weight,
                        int B, int T, int C, int OC, int dtype, void* stream);

/* The bf16 backward pass with stochastic rounding of the parameter
 * gradients (the llm.c encoder page writes its bf16 gradients this way, with
 * a deterministic seed per element).  Tensors, layout, ownership, errors and
 * streams as mmb_backward_stream with dtype MMB_BF16 (there is no dtype
 * argument: fp32 needs no rounding).  dinp is rounded to nearest as in
 * mmb_backward.  dweight[o,i] and dbias[o] take the fp32 value (old + sum for
 * dweight, the sum for dbias) to one of its two bf16 neighbours: with d the
 * 16 bits below the bf16 mantissa and r16 the element's random bits, the
 * result is the upper half of bits(value) + r16, so it moves away from zero
 * with probability d/65536 (unbiased).  r16 comes from Philox-4x64-10
 * (Salmon et al., SC 2011) keyed by (seed, tag), tag 1 for dweight and 2 for
 * dbias: element (row, col) (dbias: row 0, col o) uses bits 16*(col%4) ..
 * 16*(col%4)+15 of word (col%32)/8 of the block with counter
 * (row, 2*(col/32) + (col/4)%2, 0, 0).  The random bits of an element depend
 * only on (seed, tag, row, col), never on the launch plan, and the same seed
 * gives the same output bits on every run of a plan.  The fp32 value being
 * rounded is a sum whose order depends on the split-K plan (and so on the
 * device's CU count and the split overrides): output bits are
 * plan-independent only where those fp32 sums are exact (a different plan may
 * move an element by one bf16 step).  Non-finite values round to nearest. */
int mmb_backward_sr(void* dinp, void* dweight, void* dbias,
                    const void* dout, const void* inp, const void* weight,
                    int B, int T, int C, int OC, unsigned long long seed, void* stream);

/* Scratch that mmb_backward_noalloc holds on each device (128 MiB). */
#define MMB_NOALLOC_SCRATCH_BYTES (128u * 1024u * 1024u)

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): the same
 * backward pass as mmb_backward_stream (same arguments, plan, kernels and
 * result bits), but the split-K counters, the work list and the split
 * partials live in a fixed MMB_NOALLOC_SCRATCH_BYTES device array that each
 * device holds from library load to process end, the work list reaches it
 * through kernel arguments and the counters are cleared by a small fill
 * kernel.  The call makes no hipMalloc, hipFree, pinned allocation or
 * host-to-device copy (the first call of a shape plans it on the host, as
 * mmb_backward_stream does).  Returns MMB_ERR_SCRATCH, without enqueuing
 * anything, when the plan needs more scratch than that (the GPT-2 124M
 * layers at B*T = 8192 or 16384 need at most 115 MiB in fp32 and 48 MiB in
 * bf16).  Every call on a device shares that device's
 * scratch, which keeps the last call's contents: calls that overlap on one
 * device (several streams, or host threads) race and give wrong results;
 * order them on one stream.  Ragged or unaligned tensors (see the file
 * comment) keep their packed copies in the scratch too. */
int mmb_backward_noalloc(void* dinp, void* dweight, void* dbias,
                         const void* dout, const void* inp, const void* weight,
                         int B, int T, int C, int OC, int dtype, void* stream);

/* Host-only validation of an argument set, exactly the checks that
 * mmb_backward performs before touching the GPU.  Makes no HIP call. */
int mmb_check_args(const void* dinp, const void* dweight, const void* dbias,
                   const void* dout, const void* inp, const void* weight,
                   int B, int T, int C, int OC, int dtype);

/* Static English text for a status code (never NULL). */
const char* mmb_strerror(int status);

/* Which kernel path a call with these arguments takes: 1 = MFMA tiles
 * (directly or on packed copies of ragged or unaligned tensors), 0 = generic
 * path, or a negative mmb_status.  Host only, no HIP call. */
int mmb_path(const void* dinp, const void* dweight, const void* dbias,
             const void* dout, const void* inp, const void* weight,
             int B, int T, int C, int OC, int dtype);

/* Host-only view of the work plan the MFMA path would use on a device with
 * `num_cus` compute units (8 XCDs when num_cus >= 128): writes the largest
 * split count of each GEMM's tiles {dweight, dinp} to splits[2] and, when
 * `units` is not NULL, up to max_units launch-ordered work units as 8 ints
 * each {kind (0 = dweight, 1 = dinp), tile_m, tile_n, split, kt0, kt1,
 * splits of this tile, first workspace slot of this tile}: the unit covers
 * K iterations [kt0, kt1) of its output tile.  Returns the number of units,
 * or a negative mmb_status.  Honours the MMB_SPLITS_DWEIGHT / MMB_SPLITS_DINP
 * environment overrides like mmb_backward: one count for every tile of that
 * GEMM, or a comma-separated list whose entry t mod length applies to tile t
 * (row-major tile index).  Makes no HIP call. */
int mmb_plan_units(int B, int T, int C, int OC, int dtype, int has_bias, int num_cus,
                   int* splits, int* units, int max_units);

/* Output-tile shape of the MFMA path for `dtype`: shape[0] rows (M),
 * shape[1] columns (N), shape[2] the K depth of one pipeline stage.
 * Host only.  Returns MMB_OK or MMB_ERR_DTYPE / MMB_ERR_NULL. */
int mmb_tile_shape(int dtype, int* shape);

/* ---- the forward product ------------------------------------------------
 *
 * The forward of the same layer, whose gradients mmb_backward computes
 * (the page's launcher recalls it in its comments: one GEMM with the weight
 * transposed, alpha = 1, beta = 0), plus the bias:
 *
 *   out[r,o] = sum_{i<C} inp[r,i] * weight[o,i] + bias[o]     r<BT, o<OC
 *
 * out [BT,OC] is assigned (its old contents are ignored); bias [OC] may be
 * NULL (no bias term).  inp [BT,C] and weight [OC,C] as for mmb_backward,
 * read only; one dtype for all four tensors, with the same arithmetic: fp32
 * throughout, or bf16 storage with fp32 accumulation and one round to
 * nearest-even of  fp32 sum + bias.  out may not overlap inp, weight or bias
 * (MMB_ERR_ALIAS).  Paths as for mmb_backward: 16-byte aligned out, inp,
 * weight and bias with C and OC multiples of 8 (bf16) or 4 (fp32) take the
 * MFMA tiles directly; ragged or unaligned tensors go through packed copies
 * (inp and weight for ragged C; out and bias for ragged OC; out is copied
 * back); C or OC above 2^22, or a pointer not aligned to its element size,
 * the generic path.  Workspace, errors, determinism and streams as for
 * mmb_backward (the two share the per-(device, stream) workspace). */
int mmb_forward(void* out, const void* inp, const void* weight, const void* bias,
                int B, int T, int C, int OC, int dtype);

/* As mmb_forward, enqueued on `stream` (a hipStream_t; NULL = default). */
int mmb_forward_stream(void* out, const void* inp, const void* weight, const void* bias,
                       int B, int T, int C, int OC, int dtype, void* stream);

/* Host-only validation of a forward argument set (no HIP call). */
int mmb_forward_check_args(const void* out, const void* inp, const void* weight,
                           const void* bias, int B, int T, int C, int OC, int dtype);

/* Which kernel path a forward call takes: 1 = MFMA tiles (directly or on
 * packed copies), 0 = generic, or a negative mmb_status.  Host only. */
int mmb_forward_path(const void* out, const void* inp, const void* weight,
                     const void* bias, int B, int T, int C, int OC, int dtype);

/* Host-only view of the forward work plan, as mmb_plan_units: splits[0]
 * receives the largest split count of the forward's tiles, and each unit is
 * {kind (always 1), tile_m, tile_n, split, kt0, kt1, splits, first slot}
 * with tile_m over the BT rows and tile_n over the OC columns.  Honours
 * MMB_SPLITS_FWD (one count, or a per-tile list) like mmb_forward. */
int mmb_forward_plan_units(int B, int T, int C, int OC, int dtype, int has_bias, int num_cus,
                           int* splits, int* units, int max_units);

/* ---- LayerNorm backward -----------------------------------------------------
 *
 * The op next to the linear layer in a GPT-2 block (llm.c page
 * "dev/cuda/layernorm_backward.cu", CPU reference layernorm_backward_cpu).
 * For every row r < BT = B*T of C channels, with the forward's saved mean[r]
 * and rstd[r] (1/sqrt(biased variance + eps)):
 *
 *   norm_i = (inp[r,i] - mean[r]) * rstd[r],   dnorm_i = weight[i] * dout[r,i]
 *   a = (1/C) sum_i dnorm_i,   b = (1/C) sum_i dnorm_i * norm_i
 *   dinp[r,i]  += (dnorm_i - a - norm_i * b) * rstd[r]
 *   dweight[i] += sum_r norm_i * dout[r,i]
 *   dbias[i]   += sum_r dout[r,i]
 *
 * All three outputs accumulate, as on the page.  Layout: dout, inp, dinp
 * [BT,C] row-major; weight, dweight, dbias [C]; mean, rstd [BT].  One dtype
 * for all eight tensors: MMB_FP32, or MMB_BF16 storage with fp32 arithmetic
 * and one round to nearest-even per output.  Device pointers owned by the
 * caller, all required; outputs may not overlap each other or an input
 * (MMB_ERR_ALIAS).  16-byte aligned dinp, dout, inp and weight with C a
 * multiple of 8 (bf16) / 4 (fp32) and C <= 16384 take the row kernel (one
 * wave per row up to C = 2048, two to eight waves sharing a row above; two
 * launches: rows, then a fixed-order column reduction of the
 * per-workgroup fp32 partials, which live in the library's per-(device,
 * stream) workspace); anything else takes the generic kernels (dinp one
 * wave per row; dweight and dbias as partial sums over bands of rows, reduced
 * the same way).  Results are deterministic.  Errors as for mmb_backward. */
int mmb_layernorm_backward(void* dinp, void* dweight, void* dbias,
                           const void* dout, const void* inp, const void* weight,
                           const void* mean, const void* rstd,
                           int B, int T, int C, int dtype, void* stream);

/* Host-only validation of a LayerNorm-backward argument set (no HIP call). */
int mmb_layernorm_check_args(const void* dinp, const void* dweight, const void* dbias,
                             const void* dout, const void* inp, const void* weight,
                             const void* mean, const void* rstd,
                             int B, int T, int C, int dtype);

/* Which path a LayerNorm-backward call takes: 1 = row kernel, 0 = generic,
 * or a negative mmb_status.  Host only. */
int mmb_layernorm_path(const void* dinp, const void* dweight, const void* dbias,
                       const void* dout, const void* inp, const void* weight,
                       const void* mean, const void* rstd,
                       int B, int T, int C, int dtype);

/* Synchronise every device the library has used, then free its workspaces.
 * The next call allocates again. */
int mmb_release(void);

/* Replace one tuning variable (see the file comment) for the rest of the
 * process, or clear it when value is NULL; the planner's choices for later
 * calls follow (plans already made for other values stay cached).  For
 * tuning sweeps and tests.  Host only.  Returns MMB_OK, MMB_ERR_NULL for a
 * NULL name or MMB_ERR_NAME for a name that is not a tuning variable. */
int mmb_set_tuning(const char* name, const char* value);

#ifdef __cplusplus
}
#endif

#endif /* MMB_H */
