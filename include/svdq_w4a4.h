/*
 * svdq_w4a4.h -- C ABI of the gfx950 (MI355X) quantized-linear library.
 *
 * Two layer types, as listed in the "Supported quantization types" table of
 * the Nunchaku Lite pages (Hugging Face Diffusers quantization docs):
 *
 *   svdq_w4a4  4-bit weights and 4-bit activations with an SVDQ low-rank
 *              correction; precision int4 (group 64) or nvfp4 (group 16).
 *   awq_w4a16  int4 weight-only (AWQ style), group 64, bf16 activations.
 *
 * "NunchakuLiteQuantizationConfig" section of the same pages: every floating
 * point buffer is bfloat16 (compute_dtype), the example uses rank 32, and
 * every quantized target is a linear layer.  The news article on Nunchaku
 * Lite describes the low-rank branch as a 16-bit side path that absorbs the
 * outliers while the rest runs in 4 bits.
 *
 * Conventions for every entry point
 * ---------------------------------
 * - Layer convention is nn.Linear: X [M, K], W [N, K], Y = X W^T + b, Y [M, N].
 * - All tensors are dense, row-major, in device memory, 16-byte aligned.
 *   bf16 = IEEE bfloat16.  The caller owns every buffer; the library never
 *   allocates, frees or synchronizes on the hot path.
 * - Packed 4-bit codes are uint8 [rows, K/2]; the low nibble of byte j holds
 *   column 2j, the high nibble column 2j+1.
 *     int4  codes: sign-magnitude, bit 3 = sign, bits 0..2 = |q| in 0..7.
 *     nvfp4 codes: OCP E2M1 (magnitudes 0, .5, 1, 1.5, 2, 3, 4, 6; bit 3 = sign).
 *     AWQ   codes: unsigned 0..15.
 * - `stream` is a hipStream_t (NULL = the null stream).  Calls enqueue work on
 *   it and return without waiting.
 * - Return value: SVDQ_OK or a negative status.  Validation happens before any
 *   launch; on error nothing is written and svdq_last_error() describes the
 *   failure.  The library never aborts the process.
 */
#ifndef SVDQ_W4A4_H
#define SVDQ_W4A4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum svdq_precision { SVDQ_INT4 = 0, SVDQ_NVFP4 = 1 };

enum svdq_status {
  SVDQ_OK = 0,
  SVDQ_EINVAL = -1,       /* null/misaligned pointer, bad dimension, aliasing  */
  SVDQ_EUNSUPPORTED = -2, /* (precision, group_size) or rank not in the table  */
  SVDQ_EARCH = -3,        /* current device is not gfx950                       */
  SVDQ_EWORKSPACE = -4,   /* workspace smaller than svdq_w4a4_workspace_bytes  */
  SVDQ_EDEVICE = -5       /* HIP runtime error (no device, launch failure)     */
};

/* Bytes of scratch svdq_w4a4_linear needs, each part 256-byte aligned: the
 * operand of the product kernel [M, K] (int4: the codes as fp8 E4M3 bytes,
 * followed by the group scales [M, K/64] as bf16; nvfp4: the dequantized
 * activations e2m1 * dec(s8) as fp16, which is exact); the low-rank
 * activations fp32 [M, rank]; when the 16-row blocks of x would fill at
 * most half of the GPU, the first kernel's low-rank partials fp32 [S, M,
 * rank] of S = 2, 4 or 8 slices of K (added in slice order); and,
 * when the 256 x 192 output tiles would fill at most half of the GPU, the
 * fp32 partial sums [ksplit, M, N] of the product split along K (ksplit <= 8,
 * a function of M, N and K; the splits are added in a fixed order).
 * Returns 0 for arguments svdq_w4a4_linear would reject. */
size_t svdq_w4a4_workspace_bytes(int64_t M, int64_t K, int64_t N, int precision,
                                 int group_size, int rank);

/* SVDQ W4A4 linear ("Supported quantization types": svdq_w4a4 rows).
 *
 *   X_hat = X * (1 / smooth)                       per input channel, fp32
 *   per token and group: int4  s = bf16(amax / 7),  q = rne(X_hat / s)
 *                        nvfp4 s = E4M3(amax / 6),  q = E2M1(X_hat / s)
 *   Y = sum_g (q_x . q_w)_g * s_x * s_w * wtscale
 *       + (X_hat lora_down^T) lora_up^T + bias     -> bf16
 *
 * nvfp4 activation range: the activations carry no tensor scale, so a group
 * with amax <= 6 * 2^-10 (about 5.9e-3) gets scale 0 and zero codes (its
 * residual product is dropped; the low-rank branch keeps it), and a group
 * with amax above 6 * 448 = 2688 saturates.  The smoothing factors set where
 * X_hat falls: a static per-tensor activation scale a is the same as smooth
 * * a, with the weights prepared for that smoothing.
 *
 * x         bf16 [M, K]
 * packed_w  uint8 [N, K/2] weight codes (residual after the low-rank split)
 * wscales   int4: bf16 [N, K/64]; nvfp4: uint8 E4M3 [N, K/16]
 * wtscale   nvfp4 fp32 weight tensor scale; must be 1.0f for int4
 * smooth    bf16 [K], per-channel smoothing divisors (> 0, finite)
 * lora_down bf16 [rank, K] (the K -> rank linear); NULL iff rank == 0
 * lora_up   bf16 [N, rank] (the rank -> N linear); NULL iff rank == 0
 * bias      bf16 [N] or NULL
 * precision SVDQ_INT4 with group_size 64, or SVDQ_NVFP4 with group_size 16
 * rank      0..128, multiple of 16
 * out       bf16 [M, N]; must not overlap x, the weights or the workspace
 * workspace device scratch of at least svdq_w4a4_workspace_bytes(...) bytes,
 *           owned by the caller; its contents on entry do not matter
 * Shapes: M >= 1, K % 128 == 0, 128 <= K <= 16384, N % 64 == 0, N >= 64.
 */
int svdq_w4a4_linear(const void* x, int64_t M, int64_t K, int64_t N,
                     const void* packed_w, const void* wscales, float wtscale,
                     const void* smooth, const void* lora_down, const void* lora_up,
                     const void* bias, int precision, int group_size, int rank,
                     void* out, void* workspace, size_t workspace_bytes, void* stream);

/* svdq_w4a4_linear in two phases, for callers that reuse one quantized input
 * (or time the two kernels apart):
 *   svdq_w4a4_quantize  smoothing, activation quantization and the low-rank
 *                       down projection of x into `workspace`;
 *   svdq_w4a4_gemm      the 4-bit product, group scales, low-rank up
 *                       projection, bias and bf16 store, reading `workspace`.
 * The workspace contents between the two calls are private to the library
 * (not the parity-export formats).  Calling quantize then gemm on one stream
 * gives bit-identical results to svdq_w4a4_linear.  Arguments and rules as
 * for svdq_w4a4_linear; the gemm must use the M, K, precision, group_size and
 * rank of the quantize call that filled the workspace. */
int svdq_w4a4_quantize(const void* x, int64_t M, int64_t K, const void* smooth,
                       const void* lora_down, int precision, int group_size, int rank,
                       void* workspace, size_t workspace_bytes, void* stream);
int svdq_w4a4_gemm(const void* workspace, size_t workspace_bytes, int64_t M, int64_t K,
                   int64_t N, const void* packed_w, const void* wscales, float wtscale,
                   const void* lora_up, const void* bias, int precision, int group_size,
                   int rank, void* out, void* stream);

/* svdq_w4a4_linear for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * It takes no workspace: the scratch (the same parts, in the same layout, as
 * svdq_w4a4_linear's workspace) is a static device array of
 * SVDQ_NOALLOC_SCRATCH_BYTES bytes inside the library, one copy per GPU,
 * held until the process ends.  The call allocates and frees nothing.
 *   - A call whose scratch need (svdq_w4a4_workspace_bytes of its arguments)
 *     exceeds SVDQ_NOALLOC_SCRATCH_BYTES returns SVDQ_EWORKSPACE and writes
 *     nothing; with K = N = 3072 and rank 32 that is M up to 20360 tokens
 *     for int4 and 10699 for nvfp4 (M = 4096 needs 13.5 MB for int4 and
 *     25.7 MB for nvfp4; M = 512 int4, whose product is split along K,
 *     27.4 MB).
 *   - Every call on one GPU shares that GPU's scratch: calls that overlap in
 *     time on one GPU (different streams, or host threads) race and give
 *     undefined results; calls on one stream are ordered and safe.  No part
 *     of the scratch needs to start at zero.
 *   - The first call on a device looks up that device's copy of the array
 *     (hipGetSymbolAddress); later calls only launch.
 * Arguments, results and other rules as for svdq_w4a4_linear, whose output
 * this reproduces bit for bit. */
#define SVDQ_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int svdq_w4a4_linear_noalloc(const void* x, int64_t M, int64_t K, int64_t N,
                             const void* packed_w, const void* wscales, float wtscale,
                             const void* smooth, const void* lora_down, const void* lora_up,
                             const void* bias, int precision, int group_size, int rank,
                             void* out, void* stream);

/* AWQ W4A16 linear ("Supported quantization types": awq_w4a16, int4, group 64).
 *
 *   Y = X ((q - z) * s)^T + bias, fp32 accumulation, bf16 output.
 *
 * x        bf16 [M, K]
 * packed_w uint8 [N, K/2] unsigned codes 0..15
 * wscales  bf16 [N, K/64]
 * wzeros   bf16 [N, K/64] zero-points, integer values 0..15
 * bias     bf16 [N] or NULL
 * out      bf16 [M, N]; must not overlap x or the weights
 * Shapes: M >= 1, K % 128 == 0, 128 <= K <= 16384, N % 64 == 0, N >= 64.
 * group_size must be 64.  Bandwidth-bound for M <= 32 (one weight pass per
 * 32 rows of X).
 */
int awq_w4a16_linear(const void* x, int64_t M, int64_t K, int64_t N,
                     const void* packed_w, const void* wscales, const void* wzeros,
                     const void* bias, int group_size, void* out, void* stream);

/* One svdq_w4a4 layer's device tensors and sizes, with the meaning and rules
 * of the svdq_w4a4_linear arguments of the same names (weights [N, K]).
 * Plain C; the caller owns every buffer it points to. */
typedef struct svdq_w4a4_layer {
  const void* packed_w;   /* uint8 [N, K/2] */
  const void* wscales;    /* int4: bf16 [N, K/64]; nvfp4: uint8 E4M3 [N, K/16] */
  float wtscale;          /* nvfp4 weight tensor scale; 1.0f for int4 */
  const void* smooth;     /* bf16 [K] */
  const void* lora_down;  /* bf16 [rank, K]; NULL iff rank == 0 */
  const void* lora_up;    /* bf16 [N, rank]; NULL iff rank == 0 */
  const void* bias;       /* bf16 [N] or NULL */
  int64_t K, N;
  int precision, group_size, rank;
} svdq_w4a4_layer;

/* Bytes of scratch svdq_w4a4_mlp_gelu needs: the up layer's product operand
 * and low-rank activations (as in svdq_w4a4_workspace_bytes, no split
 * partials) followed by the down layer's linear workspace (its fp16
 * product operand [M, H], fp32 low-rank activations [M, down->rank] and, for
 * small M x N, its split-K partials), then fp32 partial sums of the down
 * layer's low-rank activations per 192-column tile of the up projection
 * [ceil(H / 192), M, down->rank].  Returns 0 for arguments
 * svdq_w4a4_mlp_gelu would reject. */
size_t svdq_w4a4_mlp_workspace_bytes(int64_t M, const svdq_w4a4_layer* up,
                                     const svdq_w4a4_layer* down);

/* GELU MLP, Y = down(GELU(up(X))) with GELU(y) = y/2 (1 + erf(y / sqrt 2)),
 * with the fusion of the "Fused kernels" section of the Nunchaku Lite docs
 * page: the up projection's epilogue applies GELU to its bf16 output and
 * quantizes the result for the down projection itself (the down layer's
 * smoothing, nvfp4 group quantization and low-rank down projection), so the
 * hidden [M, H] bf16 tensor is never written or read back.
 *
 * The values are those of svdq_w4a4_linear(up), a bf16 GELU of its output and
 * svdq_w4a4_linear(down) on that, except that the down layer's low-rank
 * activations are summed per 192-column tile of the up projection and the
 * tiles' sums then added in order (not in the quantize kernel's order), so
 * their last bits may differ from the unfused chain's.  The result is
 * deterministic: the same inputs give the same bits on every call.
 *
 * x      bf16 [M, up->K]; H = up->N must equal down->K
 * up     any svdq_w4a4 layer (int4 or nvfp4)
 * down   an nvfp4 layer (group 16): the epilogue writes the nvfp4 operand
 *        only (an int4 group of 64 would straddle the two waves that hold a
 *        tile's 192 columns), so int4 returns SVDQ_EUNSUPPORTED
 * out    bf16 [M, down->N]; must not overlap x, the weights or the workspace
 * workspace  at least svdq_w4a4_mlp_workspace_bytes(M, up, down) bytes
 * Other rules (shapes, ranks, alignment, errors) as for svdq_w4a4_linear,
 * for each layer.
 */
int svdq_w4a4_mlp_gelu(const void* x, int64_t M, const svdq_w4a4_layer* up,
                       const svdq_w4a4_layer* down, void* out, void* workspace,
                       size_t workspace_bytes, void* stream);

/* Fused QKV projection with RMSNorm and RoPE, the fusion of the "Fused
 * kernels" section of the Nunchaku Lite docs page (the Q, K and V
 * projections merged with RMSNorm and RoPE): one svdq_w4a4 linear whose
 * epilogue normalizes and rotates the q and k heads before they are stored.
 *
 *   h = svdq_w4a4_linear(qkv, x)  (bf16 [M, 3 heads head_dim]: q | k | v,
 *                                  heads of head_dim consecutive columns)
 *   for each token m and q or k head: n = bf16(h / sqrt(mean(h^2) + eps) * w)
 *     with w = q_norm or k_norm; out pair (2i, 2i+1) =
 *     bf16(n_2i cos[m,i] - n_2i+1 sin[m,i], n_2i sin[m,i] + n_2i+1 cos[m,i])
 *   v columns: out = h.
 * The GPU computes the norm and rotation in fp32 (the sum of squares in its
 * own order), so a value can differ from an fp64 evaluation by one bf16 ulp.
 *
 * x       bf16 [M, qkv->K]
 * qkv     an svdq_w4a4 layer with N = 3 * heads * head_dim
 * heads   1..256; head_dim 32, 64 or 128, with heads * head_dim a multiple
 *         of 64 (else SVDQ_EUNSUPPORTED): a tile of the product holds 128
 *         q | k columns, whole heads, so that RMSNorm stays in one workgroup
 * q_norm, k_norm  bf16 [head_dim] RMSNorm weights
 * eps     finite, > 0
 * rope_cos, rope_sin  fp32 [M, head_dim / 2]: the rotation of pair i at token m
 * out     bf16 [M, N]; must not overlap x, the weights, the tables or the
 *         workspace
 * workspace  at least svdq_w4a4_workspace_bytes(M, K, N, precision,
 *         group_size, rank) bytes (the linear's)
 * Pointers 16-byte aligned; other rules as for svdq_w4a4_linear.
 */
int svdq_w4a4_qkv_rmsnorm_rope(const void* x, int64_t M, const svdq_w4a4_layer* qkv, int heads,
                               int head_dim, const void* q_norm, const void* k_norm, float eps,
                               const float* rope_cos, const float* rope_sin, void* out,
                               void* workspace, size_t workspace_bytes, void* stream);

/* Offline weight preparation on the GPU, step by step (what the
 * diffuse-compressor tool the Nunchaku Lite pages name under "Resources" does
 * before a checkpoint is saved), bit-identical to the CPU reference packer.
 * svdq_w4a4_prepare_weight below runs the whole preparation, the low-rank
 * split included; these two calls are its first and last steps on their own.
 *
 * Scratch for both calls: svdq_w4a4_prep_workspace_bytes(K) bytes (0 for an
 * invalid K). */
size_t svdq_w4a4_prep_workspace_bytes(int64_t K);

/* Per-channel smoothing factors for svdq_w4a4 weights:
 *   smooth[k] = bf16_rne(sqrt(max_m |x[m, k]| / max_n |w[n, k]|))
 * with the ratio and the root in fp64 and one rounding to bf16; 1 where the
 * result is not finite or not positive (a zero column of x or of w).
 * x_calib  bf16 [M, K] calibration activations, 1 <= M <= 2^22
 * w        fp32 [N, K] weight, 1 <= N <= 2^22; K as for svdq_w4a4_linear
 * smooth_out  bf16 [K]
 * Pointers 16-byte aligned; the output may not overlap an input. */
int svdq_w4a4_smooth_factors(const void* x_calib, int64_t M, const float* w, int64_t N, int64_t K,
                             void* smooth_out, void* workspace, size_t workspace_bytes,
                             void* stream);

/* Quantize and pack a residual weight R (fp32 [N, K]) for svdq_w4a4_linear:
 *   int4 (group 64):  s = bf16(fl32(amax / 7)), q = rne(fl32(r * fl32(1/s))),
 *                     sign-magnitude nibbles; wscales bf16 [N, K/64];
 *                     *wtscale_out = 1 (wtscale_out may be NULL)
 *   nvfp4 (group 16): t = fl32(amax_R / 2688), s8 = E4M3(fl32(amax / fl32(6 t))),
 *                     S = fl32(dec(s8) t), code = E2M1(fl32(r * fl32(1/S)));
 *                     wscales uint8 E4M3 [N, K/16]; *wtscale_out = t (1 for an
 *                     all-zero R), a device fp32
 * Groups with amax < 2^-100 (or a zero scale) get scale 0 and codes 0.
 * packed_w_out uint8 [N, K/2], low nibble = even column.  Outputs may not
 * overlap each other, R or the workspace; errors as for svdq_w4a4_linear. */
int svdq_w4a4_pack_weight(const float* resid, int64_t N, int64_t K, int precision, int group_size,
                          void* packed_w_out, void* wscales_out, float* wtscale_out,
                          void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of scratch svdq_w4a4_prepare_weight needs for an [N, K] weight with
 * the given rank and oversampling (0 for arguments it would reject): the
 * fp64 matrices of the range finder ([max(N, K), rank + oversample] each,
 * and row-slice partial sums) and the fp32 residual [N, K]. */
size_t svdq_w4a4_prepare_workspace_bytes(int64_t N, int64_t K, int rank, int oversample);

/* Offline preparation of one svdq_w4a4 layer on the GPU, from a weight and
 * calibration activations to every weight-side input of svdq_w4a4_linear --
 * what the diffuse-compressor tool named under "Resources" on the Nunchaku
 * Lite pages does before a checkpoint is saved:
 *   1. smooth = the factors of svdq_w4a4_smooth_factors(x_calib, w);
 *   2. the rank-r split of W_hat = W * smooth (per input channel) by a
 *      randomized range finder with subspace iteration (Halko, Martinsson and
 *      Tropp, "Finding structure with randomness", 2011, Algorithms 4.3 and
 *      4.4): l = rank + oversample Gaussian test vectors drawn from `seed`,
 *      power_iters iterations, each product re-orthonormalized (shifted
 *      CholeskyQR, then two CholeskyQR passes); the SVD of the final l x l
 *      factor runs on the host in fp64 (one-sided Jacobi).  lora_up =
 *      bf16(U_r) [N, rank], lora_down = bf16(Sigma_r V_r^T) [rank, K];
 *   3. the residual R = fl32(W_hat - lora_up lora_down), in fp64 from the bf16
 *      factors with the rank terms added in order, quantized and packed as
 *      svdq_w4a4_pack_weight does.
 * The products run as this library's kernels; the call synchronizes `stream`
 * (small matrices go to and from the host), so it is for offline use.  The
 * same arguments and seed give the same bits.
 *
 * w             fp32 [N, K] weight (device); 1 <= N <= 2^20, K as for the linear
 * x_calib       bf16 [Mc, K] calibration activations (device), 1 <= Mc <= 2^22
 * precision, group_size, rank  as for svdq_w4a4_linear; rank <= min(N, K)
 * oversample    0..32 extra test vectors; power_iters 0..16; seed any value
 * outputs (device): smooth_out bf16 [K]; lora_down_out bf16 [rank, K] and
 *   lora_up_out bf16 [N, rank] (NULL iff rank == 0); packed_w_out uint8
 *   [N, K/2]; wscales_out as for svdq_w4a4_pack_weight; wtscale_out fp32 [1]
 * sigma_out     host double [rank], the estimated leading singular values of
 *               W_hat, or NULL
 * workspace     at least svdq_w4a4_prepare_workspace_bytes(N, K, rank,
 *               oversample) bytes of device memory
 * Outputs may not overlap each other, the inputs or the workspace; errors as
 * for svdq_w4a4_linear (validation before any launch). */
int svdq_w4a4_prepare_weight(const float* w, const void* x_calib, int64_t Mc, int64_t N, int64_t K,
                             int precision, int group_size, int rank, int oversample, int power_iters,
                             uint64_t seed, void* smooth_out, void* lora_down_out, void* lora_up_out,
                             void* packed_w_out, void* wscales_out, float* wtscale_out, double* sigma_out,
                             void* workspace, size_t workspace_bytes, void* stream);

/* Parity export of the fused MLP's GELU: out (bf16 [65536]) receives, for
 * every bf16 bit pattern b, the bits of GELU(h) = h/2 (1 + erf(h / sqrt 2))
 * of the value h with bits b, rounded once to bf16 -- the table the epilogue
 * of svdq_w4a4_mlp_gelu looks its GELU up in. */
int svdq_w4a4_gelu_table(void* out, void* stream);

/* Parity export of the first svdq_w4a4 kernel in its packed-code form:
 * smoothing, activation quantization and the low-rank down projection
 * ("Supported quantization types": the svdq_w4a4 activation formats).  This
 * is the export instantiation of the kernel template the linear runs: the
 * same smoothing, scale and low-rank code, but it writes packed nibbles and
 * scales (its int4 codes are rounded by the fp32 1.5 * 2^23 addition) where
 * the linear writes the product operand (see svdq_w4a4_quantize_operand).
 * codes_out  uint8 [M, K/2]; scales_out bf16 [M, K/64] (int4) or uint8 E4M3
 * [M, K/16] (nvfp4); lora_act_out fp32 [M, rank] (may be NULL iff rank == 0).
 * Arguments as for svdq_w4a4_linear. */
int svdq_w4a4_quantize_act(const void* x, int64_t M, int64_t K, const void* smooth,
                           const void* lora_down, int precision, int group_size, int rank,
                           void* codes_out, void* scales_out, float* lora_act_out,
                           void* stream);

/* Parity export of the first svdq_w4a4 kernel exactly as svdq_w4a4_linear
 * launches it: the product operand the second kernel multiplies, written to
 * caller buffers instead of the workspace ("Supported quantization types":
 * the svdq_w4a4 activation formats).
 *   operand_out    int4: uint8 [M, K], each code q (|q| <= 7) as an OCP fp8
 *                  E4M3 byte, exact (a negative value that rounds to 0 gives
 *                  0x80, -0); nvfp4: IEEE binary16 [M, K], e2m1 * dec(s8)
 *                  (always exact)
 *   scale_out      int4: fp32 [M, K/64], the group scales s (the bf16 values,
 *                  0 for a zero group; the linear keeps their bf16 bits in
 *                  its workspace); must be NULL for nvfp4
 *   lora_act_out   fp32 [M, rank] (NULL iff rank == 0)
 * Other arguments and rules as for svdq_w4a4_quantize_act; no output may
 * overlap x or another output. */
int svdq_w4a4_quantize_operand(const void* x, int64_t M, int64_t K, const void* smooth,
                               const void* lora_down, int precision, int group_size, int rank,
                               void* operand_out, float* scale_out, float* lora_act_out,
                               void* stream);

/* Parity export of the 4-bit product of the second svdq_w4a4 kernel (same
 * operand unpacking and matrix instructions): exact per-group integer dot
 * products P[m, n, g] = sum over group g of q_x * q_w, int32 [M, N, K/G].
 * nvfp4 reports doubled E2M1 codes (integers), i.e. 4 * sum(e2m1_x * e2m1_w).
 * act_codes uint8 [M, K/2], w_codes uint8 [N, K/2]. */
int svdq_w4a4_gemm_partials(const void* act_codes, const void* w_codes, int64_t M,
                            int64_t K, int64_t N, int precision, int group_size,
                            int32_t* partials_out, void* stream);

/* Host-only argument validation, without touching the GPU: the checks
 * svdq_w4a4_linear / awq_w4a16_linear perform, with the device architecture
 * given as a string (for example "gfx950:sramecc+:xnack-").  Returns the
 * status the call would return before launching. */
int svdq_w4a4_check(const void* x, int64_t M, int64_t K, int64_t N, const void* packed_w,
                    const void* wscales, float wtscale, const void* smooth,
                    const void* lora_down, const void* lora_up, const void* bias,
                    int precision, int group_size, int rank, const void* out,
                    const void* workspace, size_t workspace_bytes, const char* arch);
int awq_w4a16_check(const void* x, int64_t M, int64_t K, int64_t N, const void* packed_w,
                    const void* wscales, const void* wzeros, const void* bias,
                    int group_size, const void* out, const char* arch);
int svdq_w4a4_mlp_gelu_check(const void* x, int64_t M, const svdq_w4a4_layer* up,
                             const svdq_w4a4_layer* down, const void* out,
                             const void* workspace, size_t workspace_bytes, const char* arch);
int svdq_w4a4_qkv_rmsnorm_rope_check(const void* x, int64_t M, const svdq_w4a4_layer* qkv,
                                     int heads, int head_dim, const void* q_norm,
                                     const void* k_norm, float eps, const float* rope_cos,
                                     const float* rope_sin, const void* out,
                                     const void* workspace, size_t workspace_bytes,
                                     const char* arch);

/* Message for the last failure on the calling thread ("" if none). */
const char* svdq_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* SVDQ_W4A4_H */
