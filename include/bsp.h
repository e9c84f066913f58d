/*
 * bsp.h -- block-scaled precision linear layers (NVFP4 W4A4, MXFP8 W8A8) for AMD MI355X (gfx950).
 *
 * C ABI of libbsp.so. Every entry point:
 *   - takes plain pointers and sizes; device pointers are HIP device memory owned by the caller
 *     (the library never allocates, frees or keeps any pointer after the call returns);
 *   - validates its arguments on the host before launching anything and returns a bsp_status;
 *     on failure nothing was launched and bsp_last_error() describes the problem;
 *   - enqueues its kernels on the caller's stream (hipStream_t passed as void*; NULL = the null
 *     stream) and returns without synchronising or reading anything back;
 *   - takes scalars that are produced on the device (global scales, alpha) as device pointers, so
 *     a forward pass needs no device-to-host sync (the FastVideo nvfp4_qat_config.py page keeps
 *     the activation global scale as a device-resident constant for this reason).
 *
 * Pages cited (by title, section = the function or class on the page):
 *   [FV-QAT]  FastVideo nvfp4_qat_config.py      [FV-NV]  FastVideo nvfp4_config.py
 *   [SGL]     SGLang nvfp4_online.py             [VLO]    vLLM-Omni mxfp8_config.py
 *
 * Formats: e2m1 = 4-bit float (sign, 2 exponent bits bias 1, 1 mantissa bit; max 6);
 * e4m3 = 8-bit float "fn" (bias 7, max 448, no inf); e8m0 = power-of-two scale 2^(byte-127).
 * bf16 inputs are row-major with a row stride `ld` given in elements (ld >= K).
 */
#ifndef BSP_H
#define BSP_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  BSP_OK = 0,
  BSP_EINVAL = -1,      /* null pointer, negative size, bad enum value                     */
  BSP_ESHAPE = -2,      /* shape rule violated (K % 16, K % 32, GEMM K/N alignment, ld < K) */
  BSP_EDTYPE = -3,      /* unsupported output dtype                                        */
  BSP_EUNSUPPORTED = -4,/* the current device is not gfx950                                */
  BSP_EHIP = -5         /* a HIP runtime call failed (launch error); see bsp_last_error     */
} bsp_status;

typedef enum { BSP_OUT_BF16 = 0, BSP_OUT_F32 = 1 } bsp_out_dtype;

/* Message for the last non-OK status returned on this host thread ("" if none). */
const char* bsp_last_error(void);

/* Library ABI version (major*100 + minor). */
int bsp_version(void);

/* Bytes of the NVFP4 scale buffer for `rows` x `K`: ceil(rows/128)*128 * ceil(K/64)*4.
 * [FV-NV] _nvfp4_quantize: swizzled layouts pad the rows to the 128-row tile and the scales keep
 * the padded rows; the shape kernel gives (rows, (K+15)//16) scale bytes. */
int bsp_nvfp4_sf_bytes(int64_t rows, int64_t K, int64_t* bytes);

/* Weight global scale. [FV-QAT] convert_model_to_fp4: gsf = (448*6) / amax(|W|) with NaN/inf
 * replaced first (NaN -> 0, +-inf -> +-largest finite bf16); [SGL] _quantize_weight_nvfp4: gsf = 1
 * when amax == 0. Writes three device fp32 scalars: amax, gsf = fl32(2688/amax) and
 * inv_gsf = fl32(1/gsf) (the fp32 weight alpha of [FV-NV] convert_model_to_nvfp4).
 * w: device bf16 [rows, K], row stride ld. rows or K may be 0 (then amax = 0, gsf = 1). */
int bsp_nvfp4_global_sf(const void* w_bf16, int64_t rows, int64_t K, int64_t ld,
                        float* gsf_dev, float* inv_gsf_dev, float* amax_dev, void* stream);

/* Every quantizer below encodes nan_to_num of its input: a NaN as +0, +-inf as +-largest finite
 * bf16 (the substitution [FV-QAT], [FV-NV] and [SGL] apply before a weight's amax), so scales and
 * elements always come from finite values.
 *
 * NVFP4 quantize. [FV-NV] _nvfp4_quantize / module docstring: e2m1 values, one e4m3 scale
 * per 16 consecutive K elements under the fp32 global scale *gsf_dev, scales in layout_128x4.
 * Per block: a = max|x|; s = fl32(g*fl32(a*fl32(1/6))); S = e4m3(s) (nearest-even, saturate 448);
 * r = S==0 ? 0 : fl32(g/S); q = e2m1(fl32(x*r)) (nearest-even, saturate 6, sign kept).
 * x: device bf16 [M, K], row stride ld; K % 16 == 0.
 * packed: device uint8 [M, K/2] (row stride K/2); byte j of a row = q[2j] | q[2j+1] << 4.
 * sf: device uint8, bsp_nvfp4_sf_bytes(M, K) bytes, 128x4 layout: byte (r, c) at
 *     ((r/128)*(Kp/4) + c/4)*512 + (r%32)*16 + ((r/32)%4)*4 + c%4 with Kp = ceil(K/64)*4;
 *     rows M..Mp-1 and columns K/16..Kp-1 are written as 0x00 (zero padding, no copy of x).
 * Alignment: packed 4-byte, sf 16-byte (else BSP_EINVAL); x any (16-byte aligned rows with
 * ld % 8 == 0 take 16-byte loads). K % 16 != 0 or ld < K: BSP_ESHAPE. NULL pointers: BSP_EINVAL.
 * M == 0 is a no-op returning BSP_OK. */
int bsp_nvfp4_quantize(const void* x_bf16, int64_t M, int64_t K, int64_t ld, const float* gsf_dev,
                       uint8_t* packed, uint8_t* sf, void* stream);

/* Load-time weight prequantization: the global scale, then the NVFP4 quantize, of W [N, K]
 * ([FV-QAT] convert_model_to_fp4, [FV-NV] convert_model_to_nvfp4). Outputs as for the two calls above (gsf_dev, inv_gsf_dev and
 * amax_dev are all required device fp32 slots; the quantize step reads *gsf_dev on the device, so
 * nothing is synchronised). packed 4-byte and sf 16-byte aligned (else BSP_EINVAL). The caller may
 * free W once the stream has passed this call. */
int bsp_nvfp4_prequantize_weight(const void* w_bf16, int64_t N, int64_t K, int64_t ld,
                                 uint8_t* packed, uint8_t* sf, float* gsf_dev, float* inv_gsf_dev,
                                 float* amax_dev, void* stream);

/* alpha = fl32(1 / fl32(x_gsf * w_gsf)) on the device ([FV-QAT] NVFP4QATQuantizeMethod.apply's
 * order; [FV-NV] NVFP4QuantizeMethod.apply divides its stored fl32(1/w_gsf) by x_gsf instead, which
 * is the same bits when x_gsf = 1.0, the static activation scale, and may differ by one ulp
 * otherwise). NULL pointers: BSP_EINVAL. */
int bsp_nvfp4_alpha(const float* x_gsf_dev, const float* w_gsf_dev, float* alpha_dev, void* stream);

/* mm_fp4: C[m, n] = alpha * sum_k e2m1(A[m,k])*e4m3(SA[m,k/16]) * e2m1(B[n,k])*e4m3(SB[n,k/16]),
 * fp32 accumulation, fp32 alpha from *alpha_dev, result rounded to bf16 (nearest-even) or stored
 * as fp32. [FV-NV] _mm_fp4 / [FV-QAT] apply: the weight is passed as the transposed view of its
 * [N, K/2] packed buffer, i.e. B here is that K-major [N, K/2] buffer.
 * a_packed: device uint8 [M, K/2]; a_sf: 128x4 scales for M rows (bsp_nvfp4_sf_bytes(M, K));
 * b_packed: device uint8 [N, K/2]; b_sf: 128x4 scales for N rows; out: device [M, N] with row
 * stride ldc elements (bf16 or fp32 per out_dtype). Requires K % 64 == 0 and K <= 2^24 (else
 * BSP_ESHAPE); M, N arbitrary >= 0. a_packed, a_sf, b_packed and b_sf 16-byte aligned, no NULL
 * pointer (else BSP_EINVAL); out_dtype other than BSP_OUT_BF16 / BSP_OUT_F32: BSP_EDTYPE. Every
 * finite alpha is applied exactly as fl32(alpha * sum) up to the fp32 accumulation. Scale bytes
 * are read as non-negative e4m3: the sign bit is ignored and the NaN code 0x7F reads as 480 (every
 * quantizer here writes 0x00 .. 0x7E). */
int bsp_mm_fp4(const uint8_t* a_packed, const uint8_t* a_sf, const uint8_t* b_packed,
               const uint8_t* b_sf, const float* alpha_dev, int64_t M, int64_t N, int64_t K,
               void* out, int64_t ldc, int out_dtype, void* stream);

/* MXFP8 quantize. [VLO] DiffusionMXFP8Config: 32 consecutive K elements share one e8m0
 * scale (OCP MX). Es = clamp(floor(log2 amax) - 8, -127, 127); scale byte Es+127 (0x00 for an
 * all-zero group); q = e4m3(fl32(x * 2^-Es)) (nearest-even, saturate 448, sign kept).
 * x: device bf16 [M, K], row stride ld, K % 32 == 0. q: device uint8 [M, K] row-major.
 * sf: device uint8 [M, K/32] row-major (the per-row (rows, ceil(K/32)) uint8 scale shape of
 * [VLO] NPUMxfp8LinearMethod.create_weights). Also used once at load for weights ([VLO]
 * NPUMxfp8OnlineLinearMethod.process_weights_after_loading). q 8-byte aligned (else BSP_EINVAL);
 * K % 32 != 0 or ld < K: BSP_ESHAPE. */
int bsp_mxfp8_quantize(const void* x_bf16, int64_t M, int64_t K, int64_t ld, uint8_t* q,
                       uint8_t* sf, void* stream);

/* mm_mxfp8: C[m, n] = sum_k e4m3(A[m,k])*2^(SA[m,k/32]-127) * e4m3(B[n,k])*2^(SB[n,k/32]-127),
 * fp32 accumulation, bf16 or fp32 output ([VLO] NPUMxfp8LinearMethod._quant_matmul: per-row e8m0
 * scales of both operands, group [1, 1, 32], output in the activation dtype).
 * a: [M, K] e4m3, a_sf [M, K/32]; b: [N, K] e4m3 (K-major weight), b_sf [N, K/32]; out [M, N]
 * row stride ldc. Requires K % 128 == 0; operands 16-byte and scales 4-byte aligned (else
 * BSP_EINVAL). With K % 512 == 0 and both scale matrices 16-byte aligned the kernel fetches the
 * scales in 512-K row blocks (faster, same results). */
int bsp_mm_mxfp8(const uint8_t* a, const uint8_t* a_sf, const uint8_t* b, const uint8_t* b_sf,
                 int64_t M, int64_t N, int64_t K, void* out, int64_t ldc, int out_dtype,
                 void* stream);

/* MXFP4 (mm_fp4 with use_nvfp4=False: [FV-NV] _mm_fp4, "MX-FP4" in its module docstring): e2m1
 * values with one e8m0 scale per 32 K elements (OCP MX rule of [VLO] DiffusionMXFP8Config applied to
 * e2m1: Es = clamp(floor(log2 amax) - 2, -127, 127), byte Es+127, 0x00 for an all-zero group,
 * q = e2m1(fl32(x * 2^-Es)) nearest-even saturating at 6). Scales in the 128x4 layout (as NVFP4,
 * one byte per 32 K): byte (r, c) at ((r/128)*(Kp/4) + c/4)*512 + (r%32)*16 + ((r/32)%4)*4 + c%4,
 * Kp = ceil(K/128)*4; padded rows/columns 0x00. Size: bsp_mxfp4_sf_bytes = ceil(rows/128)*128 * Kp. */
int bsp_mxfp4_sf_bytes(int64_t rows, int64_t K, int64_t* bytes);

/* x: device bf16 [M, K] (row stride ld), K % 32 == 0 -> packed uint8 [M, K/2] (even k in the low
 * nibble), sf (bsp_mxfp4_sf_bytes(M, K) bytes). packed 4-byte and sf 16-byte aligned (else
 * BSP_EINVAL). M == 0 is a no-op. */
int bsp_mxfp4_quantize(const void* x_bf16, int64_t M, int64_t K, int64_t ld, uint8_t* packed,
                       uint8_t* sf, void* stream);

/* C[m, n] = alpha * sum_k e2m1(A)*2^(SA-127) * e2m1(B)*2^(SB-127), fp32 accumulation on gfx950's
 * block-scaled FP4 MFMA; alpha_dev may be NULL (alpha = 1). a: [M, K/2], b: [N, K/2] (K-major
 * weight), scales as above, out [M, N] row stride ldc (bf16 or fp32). Requires K % 128 == 0
 * (else BSP_ESHAPE); operands and scales 16-byte aligned (else BSP_EINVAL). */
int bsp_mm_mxfp4(const uint8_t* a_packed, const uint8_t* a_sf, const uint8_t* b_packed,
                 const uint8_t* b_sf, const float* alpha_dev, int64_t M, int64_t N, int64_t K,
                 void* out, int64_t ldc, int out_dtype, void* stream);

/* GELU (tanh form) on bf16, out of place or in place: y = bf16(gelu(x)) with
 * gelu(x) = 0.5*x*(1 + tanh(z)), z = sqrt(2/pi)*(x + 0.044715*x^3), evaluated in fp32 through the
 * logistic form with t = exp(-2|z|) (no cancellation, no overflow). For |x| in [2^-12, 2^6) the
 * result is the correctly rounded bf16 of gelu(x) (a lookup table computed in exact arithmetic);
 * other inputs take the fp32 evaluation (hardware exp2 and reciprocal, a few fp32 ulps), within
 * one bf16 ulp of exact.
 * It is the activation between fc_in and fc_out of the Wan FFN, both of which are in the NVFP4
 * layer set of [FV-QAT] (DEFAULT_FP4_LAYERS: ffn.fc_in, ffn.fc_out).
 * x, y: device bf16 [n], contiguous, 16-byte aligned. */
int bsp_gelu_tanh_bf16(const void* x, void* y, int64_t n, void* stream);

/* layout_8x4 for small-M activations and the 4over6 weight scale. */

/* Bytes of an NVFP4 scale buffer in layout_8x4: ceil(rows/8)*8 * ceil(K/64)*4. */
int bsp_nvfp4_sf_bytes_8x4(int64_t rows, int64_t K, int64_t* bytes);

/* bsp_nvfp4_quantize with the scales in layout_8x4. [FV-NV] _nvfp4_quantize: for layout_8x4 the
 * row tile is 8 (rows padded to a multiple of 8 instead of 128). Layout: 32-byte tiles of 8 rows x
 * 4 scale columns ordered row-tile-major, byte (r, c) at ((r/8)*(Kp/4) + c/4)*32 + (r%8)*4 + c%4
 * (Kp = ceil(K/64)*4); padded rows M..ceil(M/8)*8-1 and columns K/16..Kp-1 are 0x00.
 * sf: bsp_nvfp4_sf_bytes_8x4(M, K) bytes, 4-byte aligned (else BSP_EINVAL). Everything else as
 * bsp_nvfp4_quantize. */
int bsp_nvfp4_quantize_8x4(const void* x_bf16, int64_t M, int64_t K, int64_t ld, const float* gsf_dev,
                           uint8_t* packed, uint8_t* sf, void* stream);

/* bsp_mm_fp4 with the activation (A) scales in layout_8x4 (as written by bsp_nvfp4_quantize_8x4)
 * and the weight (B) scales in 128x4. [FV-NV] _mm_fp4: use_8x4_sf_layout. a_sf 4-byte aligned;
 * the other buffers as bsp_mm_fp4 (else BSP_EINVAL). */
int bsp_mm_fp4_8x4(const uint8_t* a_packed, const uint8_t* a_sf, const uint8_t* b_packed,
                   const uint8_t* b_sf, const float* alpha_dev, int64_t M, int64_t N, int64_t K,
                   void* out, int64_t ldc, int out_dtype, void* stream);

/* Weight scales of the 4over6 variant. [SGL] _quantize_weight_nvfp4: with the 4over6 switches
 * the largest e4m3 block scale is taken as 256 instead of 448; the decode scale is
 * fl32(amax / 1536) (1 when amax == 0) and the encode scale is its fl32 reciprocal, in that order:
 * gsf = fl32(1 / fl32(amax / 1536)), inv_gsf = fl32(1 / gsf). amax as bsp_nvfp4_global_sf
 * (nan_to_num first). Quantizing W with this gsf keeps every block scale <= 256. */
int bsp_nvfp4_global_sf_4over6(const void* w_bf16, int64_t rows, int64_t K, int64_t ld,
                               float* gsf_dev, float* inv_gsf_dev, float* amax_dev, void* stream);

/* Per-token activation scales. [SGL] NVFP4OnlineConfig.__init__ (per-token
 * activation path): weights keep their static tensor scale while each activation row (token) gets
 * its own fp32 scale at run time. Row m: amax_m = max|x[m, :]|, gsf_rows[m] = fl32(2688/amax_m)
 * (1.0 for an all-zero row: the tensor rule of bsp_nvfp4_global_sf applied to the row), and the row
 * is quantized exactly as bsp_nvfp4_quantize would with gsf = gsf_rows[m]. Outputs as
 * bsp_nvfp4_quantize plus gsf_rows: device fp32 [M] (written); packed 4-byte and sf 16-byte aligned
 * (else BSP_EINVAL). A row's amax is taken after nan_to_num, like the tensor amax. Rows of up to
 * 64*8*32 elements (padded to 64) are read once; longer rows are read twice. */
int bsp_nvfp4_quantize_per_token(const void* x_bf16, int64_t M, int64_t K, int64_t ld,
                                 uint8_t* packed, uint8_t* sf, float* gsf_rows_dev, void* stream);

/* mm_fp4 with per-token activation scales: C[m, n] = alpha_m * sum_k A*SA * B*SB with
 * alpha_m = fl32(1 / fl32(x_gsf_rows[m] * w_gsf)) (the scalar alpha of bsp_nvfp4_alpha, row by row),
 * applied in the epilogue. x_gsf_rows: device fp32 [M] from bsp_nvfp4_quantize_per_token; w_gsf:
 * device fp32 scalar (the weight's encode scale). Everything else as bsp_mm_fp4. */
int bsp_mm_fp4_per_token(const uint8_t* a_packed, const uint8_t* a_sf, const uint8_t* b_packed,
                         const uint8_t* b_sf, const float* x_gsf_rows_dev, const float* w_gsf_dev,
                         int64_t M, int64_t N, int64_t K, void* out, int64_t ldc, int out_dtype,
                         void* stream);

/* Producer-fused quantize of the FFN activation: exactly bsp_nvfp4_quantize applied to
 * bsp_gelu_tanh_bf16(y) (GELU evaluated and rounded to bf16 per element as above, then the NVFP4
 * block quantization of those bf16 values), in one pass over y without writing the bf16 activation.
 * [FV-NV] apply: a producer may hand mm_fp4 an already quantized (packed, scales, global scale)
 * triple instead of bf16 activations; here the producer is the GELU between fc_in and fc_out.
 * Arguments, layouts and errors as bsp_nvfp4_quantize (y: device bf16 [M, K], row stride ld). */
int bsp_nvfp4_quantize_gelu(const void* y_bf16, int64_t M, int64_t K, int64_t ld, const float* gsf_dev,
                            uint8_t* packed, uint8_t* sf, void* stream);

/* Producer-fused quantize of a norm's output. [FV-NV] NVFP4QuantizeMethod.apply: the activation
 * may arrive as a pre-quantized (packed, scales, global scale) triple from a fused norm + quantize
 * producer. The page does not name the norm; the one taken is RMSNorm over K (the norm of the
 * LTX-2 blocks that page quantizes):
 *   y[m, k] = bf16( fl32( fl32(x[m, k] * r_m) * w[k] ) ),  r_m = fl32( 1 / sqrt(ss_m / K + eps) ),
 * ss_m = sum of x[m, :]^2 (no gain multiply when weight_bf16 is NULL). ss_m and r_m are evaluated
 * in fp64 and r_m rounded once to fp32; the products and the bf16 rounding are IEEE fp32,
 * nearest even. y is then within 3 fp32 roundings of the exact RMSNorm.
 * bsp_rmsnorm_bf16 writes y: device bf16 [M, K], row stride ldo (>= K).
 * bsp_nvfp4_quantize_rmsnorm writes bsp_nvfp4_quantize(y, gsf) without storing y: its bytes equal
 * those of the NVFP4 quantize of bsp_rmsnorm_bf16's output. Packed, sf and gsf as in
 * bsp_nvfp4_quantize (padded rows' scales 0x00).
 * x: device bf16 [M, K], row stride ld; weight_bf16: NULL or device bf16 [K]; eps: positive and
 * finite (else BSP_EINVAL); K % 16 == 0 (else BSP_ESHAPE); M == 0 returns BSP_OK; packed 4-byte
 * and sf 16-byte aligned (else BSP_EINVAL). A non-finite value in a row of x makes r_m 0 or NaN,
 * so that row's y is zero or NaN, which the quantize encodes as zero codes. Rows of up to 64*8*32
 * elements (padded to 64) are read from HBM once, longer rows twice. */
int bsp_rmsnorm_bf16(const void* x_bf16, int64_t M, int64_t K, int64_t ld, const void* weight_bf16,
                     float eps, void* out_bf16, int64_t ldo, void* stream);
int bsp_nvfp4_quantize_rmsnorm(const void* x_bf16, int64_t M, int64_t K, int64_t ld,
                               const void* weight_bf16, float eps, const float* gsf_dev,
                               uint8_t* packed, uint8_t* sf, void* stream);

/* The same producer fusion one step earlier, in fc_in's epilogue: the NVFP4 encoding of
 * gelu_tanh(alpha * A . B^T), byte for byte what bsp_nvfp4_quantize_gelu(bsp_mm_fp4(...), out_gsf)
 * writes, without the bf16 product ever reaching memory (it exists only as each GEMM tile's LDS
 * image). [FV-NV] apply (the pre-quantized triple of a producer) with the FFN's fc_in as producer.
 * A, B, their scales, alpha, M, N, K as bsp_mm_fp4; N must be a multiple of 128 (else BSP_ESHAPE).
 * out_gsf_dev: device fp32 global scale of the output. out_packed: device u8 [M, N/2], 4-byte
 * aligned; out_sf: device u8, 128x4 layout over [ceil(M/128)*128, N/16] (bsp_nvfp4_sf_bytes(M, N)
 * bytes), 16-byte aligned, rows M.. zero. NULL pointers or misalignment: BSP_EINVAL. */
int bsp_mm_fp4_gelu_nvfp4(const uint8_t* a_packed, const uint8_t* a_sf, const uint8_t* b_packed,
                          const uint8_t* b_sf, const float* alpha_dev, const float* out_gsf_dev,
                          int64_t M, int64_t N, int64_t K, uint8_t* out_packed, uint8_t* out_sf,
                          void* stream);

/* Fused into the GEMM epilogue -- the linear layer's bias.
 * bsp_mm_fp4_bias: [FV-NV] NVFP4QuantizeMethod.apply adds the bias to mm_fp4's bf16 output
 * (out = out + bias, a bf16 add): C[m, n] = bf16(fl32(bf16(alpha * acc)) + fl32(bias[n])), i.e. the
 * bf16 product of bsp_mm_fp4 plus the bias in fp32, rounded to bf16 again (nearest-even both
 * times); with out_dtype fp32, C = fl32(alpha * acc) + bias[n]. bias_bf16: device bf16 [N],
 * 2-byte aligned, not NULL (else BSP_EINVAL). Other arguments, layouts and errors as bsp_mm_fp4. */
int bsp_mm_fp4_bias(const uint8_t* a_packed, const uint8_t* a_sf, const uint8_t* b_packed,
                    const uint8_t* b_sf, const float* alpha_dev, const void* bias_bf16, int64_t M,
                    int64_t N, int64_t K, void* out, int64_t ldc, int out_dtype, void* stream);

/* bsp_mm_mxfp8_bias: [VLO] NPUMxfp8LinearMethod._quant_matmul converts the bias to fp32 and hands it
 * to the quantized matmul: C[m, n] = round(fl32(acc) + bias[n]) with one rounding to the output
 * dtype (bf16 nearest-even, or none for fp32). bias_f32: device fp32 [N], 4-byte aligned, not NULL
 * (else BSP_EINVAL). Other arguments, layouts and errors as bsp_mm_mxfp8. */
int bsp_mm_mxfp8_bias(const uint8_t* a, const uint8_t* a_sf, const uint8_t* b, const uint8_t* b_sf,
                      const float* bias_f32, int64_t M, int64_t N, int64_t K, void* out, int64_t ldc,
                      int out_dtype, void* stream);

/* bsp_mm_mxfp4_bias: the MXFP4 GEMM with the bias added as in bsp_mm_fp4_bias (the same [FV-NV]
 * apply path, use_nvfp4=False). bias_bf16: device bf16 [N]. Other arguments as bsp_mm_mxfp4. */
int bsp_mm_mxfp4_bias(const uint8_t* a_packed, const uint8_t* a_sf, const uint8_t* b_packed,
                      const uint8_t* b_sf, const float* alpha_dev, const void* bias_bf16, int64_t M,
                      int64_t N, int64_t K, void* out, int64_t ldc, int out_dtype, void* stream);

/* NVFP4 with the packed values in a fragment layout. [FV-NV] _nvfp4_quantize passes a do_shuffle
 * switch to its quantizer: operands pre-arranged for the matrix unit, the arrangement being the
 * library's (the pages always pass False). Here a 32-row tile's 64-element K step is one
 * contiguous 1 KB that a wave reads with one load, lane l = i + 32 h taking row i's elements
 * 32 h .. 32 h + 31 of the step. Same codes and scale bytes as bsp_nvfp4_quantize; only the order
 * of the packed bytes differs, and the scales stay in the 128x4 layout (bsp_nvfp4_sf_bytes).
 * Operand [R, K], K % 64 == 0, Rp = ceil(R/32)*32 rows (rows R..Rp-1 zero):
 *  packed (Rp*K/2 bytes): byte 16 l + c of the fragment at (rt*(K/64) + ks)*1024 holds elements
 *    64 ks + 32 h + 2c, +1 (low nibble first) of row 32 rt + i.
 * bsp_nvfp4_frag_bytes: the packed size (BSP_ESHAPE unless K % 64 == 0; NULL: BSP_EINVAL). */
int bsp_nvfp4_frag_bytes(int64_t rows, int64_t K, int64_t* packed_bytes);

/* bsp_nvfp4_quantize (and bsp_nvfp4_quantize_gelu) writing the packed values in the fragment
 * layout. x: device bf16 [M, K] (row stride ld), K % 64 == 0 (else BSP_ESHAPE); packed
 * (bsp_nvfp4_frag_bytes(M, K) bytes) and sf (128x4, bsp_nvfp4_sf_bytes(M, K) bytes) 16-byte
 * aligned (else BSP_EINVAL); every byte of both, padding included, is written. Other arguments and
 * errors as bsp_nvfp4_quantize. Weights take bsp_nvfp4_global_sf, then bsp_nvfp4_quantize_frag. */
int bsp_nvfp4_quantize_frag(const void* x_bf16, int64_t M, int64_t K, int64_t ld, const float* gsf_dev,
                            uint8_t* packed, uint8_t* sf, void* stream);
int bsp_nvfp4_quantize_gelu_frag(const void* y_bf16, int64_t M, int64_t K, int64_t ld,
                                 const float* gsf_dev, uint8_t* packed, uint8_t* sf, void* stream);

/* Load-time weight prequantization with the packed values in the fragment layout: the global scale
 * (bsp_nvfp4_global_sf), then bsp_nvfp4_quantize_frag, of W [N, K] ([FV-QAT] convert_model_to_fp4,
 * [FV-NV] convert_model_to_nvfp4, with the do_shuffle arrangement above). K % 64 == 0 (else
 * BSP_ESHAPE); packed (bsp_nvfp4_frag_bytes(N, K) bytes) and sf (bsp_nvfp4_sf_bytes(N, K) bytes)
 * 16-byte aligned, no NULL pointer (else BSP_EINVAL); gsf_dev, inv_gsf_dev and amax_dev as for
 * bsp_nvfp4_prequantize_weight. Nothing is synchronised; the caller may free W once the stream has
 * passed this call. */
int bsp_nvfp4_prequantize_weight_frag(const void* w_bf16, int64_t N, int64_t K, int64_t ld,
                                      uint8_t* packed, uint8_t* sf, float* gsf_dev,
                                      float* inv_gsf_dev, float* amax_dev, void* stream);

/* bsp_mm_fp4 on fragment-layout packed operands (scales in 128x4): C = alpha * A . B^T, plus the
 * bias as in bsp_mm_fp4_bias when bias_bf16 (device bf16 [N], 2-byte aligned) is not NULL.
 * a_packed: A [M, K] and b_packed: B [N, K] (K-major weight) in the fragment layout; out [M, N]
 * row stride ldc, bf16 or fp32. The same products as bsp_mm_fp4, summed in another order inside
 * each 64-element step (the output may differ from bsp_mm_fp4's by fp32 rounding). Every scale
 * byte is decoded as e4m3 in full (a set sign bit negates, 0x7F and 0xFF give NaN). Requires
 * K % 64 == 0 and K <= 2^24 (else BSP_ESHAPE); operands and scales 16-byte aligned, no NULL
 * operand, scale or alpha pointer (else BSP_EINVAL); out_dtype as bsp_mm_fp4. */
int bsp_mm_fp4_frag(const uint8_t* a_packed, const uint8_t* a_sf, const uint8_t* b_packed,
                    const uint8_t* b_sf, const float* alpha_dev, const void* bias_bf16, int64_t M,
                    int64_t N, int64_t K, void* out, int64_t ldc, int out_dtype, void* stream);

/* MXFP4 in the MFMA fragment layout. [FV-NV] _nvfp4_quantize passes a do_shuffle switch to its
 * quantizer: operands pre-arranged for the matrix unit, the arrangement being the library's (the
 * pages always pass False). This is that arrangement for gfx950's block-scaled MFMA
 * (v_mfma_scale_f32_32x32x64_f8f6f4): each 64-lane operand fragment is one contiguous 1 KB, so the
 * GEMM loads it straight into registers without staging through LDS. Same element and scale values
 * as bsp_mxfp4_quantize (OCP MX rule above); only the byte order differs. Operand [R, K],
 * K % 256 == 0, Rp = ceil(R/32)*32 rows (rows R..Rp-1 zero: codes 0, scales 0x00):
 *  packed (Rp*K/2 bytes): byte j = 16 l + c of the 1 KB fragment at (rt*(K/64) + ks)*1024, lane
 *    l = i + 32 h, holds elements 2c, 2c+1 (low nibble first) of the 32-element block 2 ks + h of
 *    row 32 rt + i, i.e. elements 64 ks + 32 h + 2c, +1;
 *  scales (Rp*K/32 bytes): byte 4 l + jj of the 256-byte group at (rt*(K/256) + kg)*256 is the
 *    e8m0 scale of row 32 rt + i (l = i + 32 h), block 8 kg + 2 jj + h.
 * Sizes: bsp_mxfp4_frag_bytes (BSP_ESHAPE unless K % 256 == 0). */
int bsp_mxfp4_frag_bytes(int64_t rows, int64_t K, int64_t* packed_bytes, int64_t* sf_bytes);

/* bsp_mxfp4_quantize writing the fragment layout. x: device bf16 [M, K] (row stride ld),
 * K % 256 == 0 (else BSP_ESHAPE) -> packed and sf as above (bsp_mxfp4_frag_bytes(M, K) bytes each),
 * both 16-byte aligned (else BSP_EINVAL); every byte of both, padding rows included, is written.
 * M == 0 is a no-op. */
int bsp_mxfp4_quantize_frag(const void* x_bf16, int64_t M, int64_t K, int64_t ld, uint8_t* packed,
                            uint8_t* sf, void* stream);

/* bsp_mm_mxfp4 on fragment-layout operands: C = alpha * A . B^T (+ bias), alpha_dev may be NULL
 * (alpha = 1), bias_bf16 a device bf16 [N] or NULL (added as in bsp_mm_mxfp4_bias). a: A [M, K] and
 * b: B [N, K] (K-major weight) in the fragment layout, each with its scales; out [M, N] row stride
 * ldc, bf16 or fp32. For the same operand values the output is bit-identical to bsp_mm_mxfp4's (and
 * bsp_mm_mxfp4_bias's). Requires K % 256 == 0 and K <= 2^24 (else BSP_ESHAPE); fragments 16-byte
 * and scales 4-byte aligned, bias 2-byte aligned (else BSP_EINVAL). */
int bsp_mm_mxfp4_frag(const uint8_t* a_packed, const uint8_t* a_sf, const uint8_t* b_packed,
                      const uint8_t* b_sf, const float* alpha_dev, const void* bias_bf16, int64_t M,
                      int64_t N, int64_t K, void* out, int64_t ldc, int out_dtype, void* stream);

/* MXFP8 in the MFMA fragment layout: the arrangement above for e4m3 operands. Operand [R, K],
 * K % 256 == 0, Rp = ceil(R/32)*32 rows (rows R..Rp-1 zero):
 *  q (Rp*K bytes): the 2 KB fragment of row tile rt and K step ks at (rt*(K/64) + ks)*2048 is two
 *    1 KB halves b = 0, 1 (the step's two 32-element blocks); byte 16 l + c of half b, lane
 *    l = i + 32 h, is element 64 ks + 32 b + 16 h + c of row 32 rt + i (so a lane's bytes 0-15 and
 *    16-31 of the 32x32x64 MFMA operand are one 16-byte read from each half);
 *  scales (Rp*K/32 bytes): exactly as the MXFP4 fragment layout.
 * Same element and scale values as bsp_mxfp8_quantize; sizes: bsp_mxfp8_frag_bytes (BSP_ESHAPE
 * unless K % 256 == 0). */
int bsp_mxfp8_frag_bytes(int64_t rows, int64_t K, int64_t* q_bytes, int64_t* sf_bytes);

/* bsp_mxfp8_quantize writing the fragment layout. x: device bf16 [M, K] (row stride ld),
 * K % 256 == 0 (else BSP_ESHAPE) -> q and sf as above (bsp_mxfp8_frag_bytes(M, K) bytes each), both
 * 16-byte aligned (else BSP_EINVAL); every byte of both, padding rows included, is written.
 * M == 0 is a no-op. */
int bsp_mxfp8_quantize_frag(const void* x_bf16, int64_t M, int64_t K, int64_t ld, uint8_t* q,
                            uint8_t* sf, void* stream);

/* bsp_mm_mxfp8 on fragment-layout operands (+ optional fp32 bias [N] added before the one rounding,
 * as bsp_mm_mxfp8_bias; NULL for none). a: A [M, K], b: B [N, K] (K-major weight), each with its
 * scales; out [M, N] row stride ldc, bf16 or fp32. For the same operand values the output is
 * bit-identical to bsp_mm_mxfp8's (and bsp_mm_mxfp8_bias's). Requires K % 256 == 0 and
 * K <= 2^24 (else BSP_ESHAPE); fragments 16-byte, scales and bias 4-byte aligned (else
 * BSP_EINVAL). */
int bsp_mm_mxfp8_frag(const uint8_t* a, const uint8_t* a_sf, const uint8_t* b, const uint8_t* b_sf,
                      const float* bias_f32, int64_t M, int64_t N, int64_t K, void* out,
                      int64_t ldc, int out_dtype, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* BSP_H */
