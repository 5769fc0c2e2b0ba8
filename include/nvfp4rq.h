/*
 * nvfp4rq.h - fused block-Hadamard rotation + NVFP4 activation quantization
 * on AMD Instinct MI355X (gfx950).  C ABI of libnvfp4rq.so.
 *
 * The method (page "A Fused Hadamard + NVFP4 Quantization Kernel in Triton",
 * kanthi.in):
 *   - section 1 "The format, precisely": x ~ q * s_block * s_global with q an
 *     E2M1 code per element, s_block one E4M3 byte per 16 consecutive values,
 *     s_global one fp32 per tensor; the 16-element block is first rotated by
 *     the orthonormal 16x16 Sylvester-Hadamard matrix (entries +-1/4);
 *   - section 2 "The kernel": s_global = rotated global amax / 6 / 448
 *     (1.0 when that is zero); s_block = (block amax / 6) / s_global rounded
 *     to E4M3 and clamped at 448; each rotated value divided by
 *     float(s_block) * s_global (by 1.0 when that product is zero) becomes an
 *     E2M1 code by midpoint compares with ties to the even code, sign in bit
 *     3; two codes per byte, even element in the low nibble;
 *   - section 3 "Bit-exact against a reference": E4M3 rounding is to nearest,
 *     ties to even.
 * The stored layout matches the page "NVFP4 Quantization" (atlas-docs),
 * section "The numeric format": codes [rows, cols/2], scales [rows, cols/16]
 * along K (the column axis).
 *
 * Arithmetic contract (bit-exact, reproducible across launch shapes): every
 * step is binary32 with round-to-nearest-even and gradual underflow; the
 * rotation is the butterfly with strides 1, 2, 4, 8 (pairs (a+b, a-b)) then a
 * multiply by 0.25; s_global = (amax / 6) / 448 and the block value
 * (block_amax / 6) / s_global are each two correctly rounded divisions; the
 * element quotient is one correctly rounded division.  Inputs must be finite
 * with |x| <= 2^123 (so that no sum of 16 values overflows); NaN or Inf input
 * gives unspecified codes, and a NaN shows up in *amax_out as a NaN bit
 * pattern.
 *
 * Common rules for every entry point:
 *   - Pointers marked "device" must be device memory of the current HIP
 *     device (or memory it can access).  The caller owns every buffer; the
 *     library allocates nothing and keeps no state between calls.
 *   - Work is enqueued on `stream` (0 = the null stream), which must belong
 *     to the current HIP device (launch shapes are sized for that device),
 *     and the call returns without waiting for it.  Nothing is read back to
 *     the host.
 *   - Validation happens before anything is enqueued: NVFP4_ERR_NULL,
 *     NVFP4_ERR_SHAPE, NVFP4_ERR_ALIGN and NVFP4_ERR_ARG mean no work was
 *     enqueued and no output was touched.  NVFP4_ERR_HIP means a launch was
 *     rejected by the runtime; earlier launches of the same call may already
 *     be enqueued, so the outputs are then undefined.  Faults inside kernels
 *     surface at the caller's next synchronisation, as usual for HIP.
 *   - Outputs must not overlap the input or each other (NVFP4_ERR_ARG).
 *   - Calls that share an output buffer must be ordered (same stream or
 *     explicit events): the amax word can be an atomic accumulator, and the
 *     fused calls keep pass 1's partial maxima at the head of q_out (of
 *     s_out and q_out for the swizzled layout).
 *   - No C++ exception crosses this interface.
 */
#ifndef NVFP4RQ_H
#define NVFP4RQ_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum nvfp4_status {
    NVFP4_OK = 0,
    NVFP4_ERR_NULL = 1,  /* a required pointer is NULL */
    NVFP4_ERR_SHAPE = 2, /* rows < 0, cols < 0, cols % 16 != 0, or the size overflows */
    NVFP4_ERR_ALIGN = 3, /* a pointer misses the alignment its argument requires */
    NVFP4_ERR_ARG = 4,   /* rotate not 0 or 1, overlapping buffers, or a bad scale */
    NVFP4_ERR_HIP = 5    /* the HIP runtime rejected a launch */
} nvfp4_status;

/*
 * Full path: rotated global amax (pass 1), global scale, then rotate+quantize
 * every block (pass 2).  Page "A Fused Hadamard + NVFP4 Quantization Kernel in
 * Triton", section 2 (quantize and hadamard_nvfp4_kernel), with the global amax
 * computed on the device instead of on the host.
 *
 *   x_bf16      device, bf16 bit patterns, row-major contiguous [rows, cols],
 *               16-byte aligned.  cols % 16 == 0.  May be NULL when
 *               rows * cols == 0.
 *   rows, cols  tensor shape; blocks are 16 consecutive values of a row.
 *   rotate      1: rotate each block by H16 before scaling; 0: no rotation.
 *   q_out       device, rows * cols / 2 bytes, 16-byte aligned: E2M1 codes,
 *               row-major [rows, cols/2], element 2k in the low nibble of
 *               byte k.  May be NULL when rows * cols == 0.  The call first
 *               keeps pass 1's per-workgroup maxima and arrival counters in
 *               its first 4 KiB (for tensors of 512 blocks or more), so its
 *               contents are defined only once
 *               the call has completed on the stream.
 *   s_out       device, rows * cols / 16 bytes, 4-byte aligned: E4M3FN block
 *               scales (0x00..0x7E), row-major [rows, cols/16].  May be NULL
 *               when rows * cols == 0.
 *   gscale_out  device, 1 float, 4-byte aligned: the global scale s_global.
 *   amax_out    device, 1 float, 4-byte aligned: the rotated global amax.
 *               Written by this call (for small tensors it is zeroed and
 *               used as the pass-1 accumulator).
 *   stream      HIP stream.
 * Failure mark: with the maxima at the head of q_out, one quantize
 * workgroup writes the head last, after a wait for every workgroup to have
 * read them.  That wait is bounded (200 ms of device wall clock; it cannot
 * run out while the device runs the grid, only if other work keeps part of
 * the grid from starting that long).  If it runs out, gscale_out and
 * amax_out are NaN and every output of the call (codes and scales too) is
 * invalid; the status is still NVFP4_OK, since nothing is read back.
 * rows * cols == 0 is valid: it writes amax 0 and global scale 1.
 */
nvfp4_status nvfp4_rotquant(const uint16_t *x_bf16, int64_t rows, int64_t cols, int rotate,
                            uint8_t *q_out, uint8_t *s_out, float *gscale_out,
                            float *amax_out, hipStream_t stream);

/* As nvfp4_rotquant for fp32 input (x: device, float [rows, cols], 16-byte
   aligned).  The page's own tests quantize fp32 activations (section 3). */
nvfp4_status nvfp4_rotquant_f32(const float *x, int64_t rows, int64_t cols, int rotate,
                                uint8_t *q_out, uint8_t *s_out, float *gscale_out,
                                float *amax_out, hipStream_t stream);

/*
 * Pass 1 alone: *amax_out = max |y| over the whole tensor, y the rotated
 * blocks (or the values themselves when rotate == 0).  Section 2 of the same
 * page: no block scale can be set until the global scale, and with it the
 * tensor-wide maximum, is known.  Arguments as nvfp4_rotquant.  The buffer is zeroed and
 * then accumulated with one atomic maximum per workgroup.
 */
nvfp4_status nvfp4_rotamax(const uint16_t *x_bf16, int64_t rows, int64_t cols, int rotate,
                           float *amax_out, hipStream_t stream);
nvfp4_status nvfp4_rotamax_f32(const float *x, int64_t rows, int64_t cols, int rotate,
                               float *amax_out, hipStream_t stream);

/*
 * Pass 2 alone: reads an amax from device memory, derives the global scale
 * (amax / 6) / 448, writes it to *gscale_out and quantizes every block.
 * Section 2 of the same page (hadamard_nvfp4_kernel).  With the amax written
 * by nvfp4_rotamax on the same tensor this completes nvfp4_rotquant; with an
 * amax kept from an earlier step it is the single-pass quantizer the page's
 * section 2 notes for production use (one read of x instead of two).  Then
 * block values above 448 are clamped to 448 and quotients beyond 6 take the
 * largest code, exactly as the definition gives.
 *   amax_in  device, 1 float, 4-byte aligned, finite and >= 0.
 * Other arguments as nvfp4_rotquant.
 */
nvfp4_status nvfp4_quant_from_amax(const uint16_t *x_bf16, int64_t rows, int64_t cols,
                                   int rotate, const float *amax_in, uint8_t *q_out,
                                   uint8_t *s_out, float *gscale_out, hipStream_t stream);
nvfp4_status nvfp4_quant_from_amax_f32(const float *x, int64_t rows, int64_t cols, int rotate,
                                       const float *amax_in, uint8_t *q_out, uint8_t *s_out,
                                       float *gscale_out, hipStream_t stream);

/*
 * Dequantize for round-trip checks (section 2, dequantize): each code becomes
 * +-{0, .5, 1, 1.5, 2, 3, 4, 6}[code & 7] times fl(float(s) * gscale), rounded
 * to binary32; when rotate == 1 the block is then multiplied by H16^T = H16
 * with the same binary32 butterfly and the multiply by 0.25.
 *   q       device, rows * cols / 2 bytes, 8-byte aligned (layout of q_out).
 *   s       device, rows * cols / 16 bytes (layout of s_out).
 *   gscale  device, 1 float, 4-byte aligned, > 0 and finite.
 *   y_out   device, float [rows, cols], 16-byte aligned.
 * Pointers other than gscale may be NULL when rows * cols == 0.
 */
nvfp4_status nvfp4_dequant(const uint8_t *q, const uint8_t *s, const float *gscale,
                           int64_t rows, int64_t cols, int rotate, float *y_out,
                           hipStream_t stream);

/*
 * Measurement hook: nvfp4_rotquant (or _f32), with every kernel it launches
 * timed by HIP events that the runtime records at that kernel's own start and
 * end (hipExtLaunchKernel), so that a caller can time each pass of the fused
 * call in place, without the dispatch gap an event between launches adds.
 *   events    npairs * 2 created events (hipEventCreate, or torch events that
 *             have been recorded once); the k-th kernel launched records
 *             events[2k] and events[2k + 1]; kernels past npairs are not
 *             timed.
 *   nkernels  receives the number of kernels launched: 2 (amax pass,
 *             quantize pass) when q_out has room for pass 1's partial maxima,
 *             3 (zeroing, amax, quantize) for small tensors and for inputs of
 *             512 MiB and more, 1 or 2 for empty ones.
 * Results are those of nvfp4_rotquant (nvfp4_rotquant_f32 for the _f32
 * variant).  NVFP4_ERR_NULL when events or nkernels is NULL or npairs < 1.
 */
nvfp4_status nvfp4_rotquant_timed(const uint16_t *x_bf16, int64_t rows, int64_t cols, int rotate,
                                  uint8_t *q_out, uint8_t *s_out, float *gscale_out,
                                  float *amax_out, hipStream_t stream, hipEvent_t *events,
                                  int npairs, int *nkernels);
nvfp4_status nvfp4_rotquant_f32_timed(const float *x, int64_t rows, int64_t cols, int rotate,
                                      uint8_t *q_out, uint8_t *s_out, float *gscale_out,
                                      float *amax_out, hipStream_t stream, hipEvent_t *events,
                                      int npairs, int *nkernels);

/*
 * Block scales in the swizzled tiled layout (page "A Fused Hadamard + NVFP4
 * Quantization Kernel in Triton", section 6: GEMMs read scales tiled, and a
 * production kernel writes that layout itself).  The page does not give the
 * layout; the one used is the tiled layout of the GEMM library documentation
 * it cites for 16-element block scales: the [rows, cols/16] scale matrix S,
 * padded with zero bytes to multiples of 128 rows and 4 columns, cut into
 * 128 x 4 tiles of 512 bytes stored tile-row by tile-row, with
 * S[128*rt + 32*i + j][4*ct + k] (i, k < 4, j < 32) at byte
 * 512*(rt*ceil(cols/64) + ct) + 16*j + 4*i + k.
 *
 * nvfp4_swizzled_scale_bytes: size of that buffer, 512*ceil(rows/128)*
 * ceil(cols/64); -1 for a bad shape or more than 2^32 - 1 blocks.  The
 * quantize calls also need 128 rows of input below 2^31 bytes (cols < 2^23
 * for bf16, < 2^22 for fp32; NVFP4_ERR_SHAPE otherwise).
 * nvfp4_rotquant_swizzled(_f32): nvfp4_rotquant with s_out in this layout
 * (s_out holds nvfp4_swizzled_scale_bytes bytes, 4-byte aligned; padding bytes
 * are written as 0).  Codes, g and amax are as for nvfp4_rotquant.  From 16
 * rows and cols >= 256, the call keeps pass 1's per-workgroup maxima in the
 * first 2 KiB of s_out and its arrival counters in the first 4 bytes of code
 * rows 0..15 of q_out, with the same failure mark; both outputs are then
 * defined only once the call has completed.
 * nvfp4_dequant_swizzled: nvfp4_dequant reading scales in this layout.
 */
int64_t nvfp4_swizzled_scale_bytes(int64_t rows, int64_t cols);
nvfp4_status nvfp4_rotquant_swizzled(const uint16_t *x_bf16, int64_t rows, int64_t cols, int rotate,
                                     uint8_t *q_out, uint8_t *s_out, float *gscale_out,
                                     float *amax_out, hipStream_t stream);
nvfp4_status nvfp4_rotquant_swizzled_f32(const float *x, int64_t rows, int64_t cols, int rotate,
                                         uint8_t *q_out, uint8_t *s_out, float *gscale_out,
                                         float *amax_out, hipStream_t stream);
nvfp4_status nvfp4_dequant_swizzled(const uint8_t *q, const uint8_t *s, const float *gscale,
                                    int64_t rows, int64_t cols, int rotate, float *y_out,
                                    hipStream_t stream);

/*
 * Rotation alone: y = x H16 on every 16-element block (butterfly with strides
 * 1, 2, 4, 8, then * 0.25; the arithmetic of nvfp4_rotquant's rotation), stored
 * as fp32 [rows, cols].  With nvfp4_rotamax_f32 and nvfp4_quant_from_amax_f32
 * (rotate = 0) on y it forms the unfused three-kernel arrangement the page "A
 * Fused Hadamard + NVFP4 Quantization Kernel in Triton" sets against the fused
 * kernel (opening paragraph; "Try this" item 4); those outputs equal
 * nvfp4_rotquant's byte for byte.  H16 / 4 is its own inverse, so the call also
 * undoes a rotation up to rounding.
 *   x      device, [rows, cols], 16-byte aligned, cols % 16 == 0.
 *   y_out  device fp32 [rows, cols], 16-byte aligned, not overlapping x.
 */
nvfp4_status nvfp4_rotate16(const uint16_t *x_bf16, int64_t rows, int64_t cols, float *y_out,
                            hipStream_t stream);
nvfp4_status nvfp4_rotate16_f32(const float *x, int64_t rows, int64_t cols, float *y_out,
                                hipStream_t stream);

/*
 * General block rotation: y = x R on every 16-element block, R a 16 x 16
 * binary32 matrix given by the caller, stored as fp32 [rows, cols].  The page
 * "A Fused Hadamard + NVFP4 Quantization Kernel in Triton" ("Try this" item 3)
 * proposes replacing the Hadamard with a random orthogonal matrix and
 * comparing the error; with nvfp4_rotquant_f32 (rotate = 0) on y and
 * nvfp4_dequant (rotate = 0) followed by this call with R transposed, it runs
 * that study on the GPU.  Arithmetic per output j of a block with inputs
 * x_0 .. x_15: t = fl(x_0 * R[0][j]), then t = fma(x_k, R[k][j], t) for
 * k = 1 .. 15 in that order; the result is t.
 *   x      device, [rows, cols], 16-byte aligned, cols % 16 == 0.
 *   r16    device, 256 floats, row-major (R[k][j] at r16[16 k + j]: row k
 *          multiplies input k), 16-byte aligned; read only, may overlap x.
 *   y_out  device fp32 [rows, cols], 16-byte aligned, overlapping neither x
 *          nor r16.
 * rows * cols == 0 returns NVFP4_OK and launches nothing (r16 must still be
 * non-NULL and aligned).
 */
nvfp4_status nvfp4_rotate_matrix(const uint16_t *x_bf16, int64_t rows, int64_t cols,
                                 const float *r16, float *y_out, hipStream_t stream);
nvfp4_status nvfp4_rotate_matrix_f32(const float *x, int64_t rows, int64_t cols, const float *r16,
                                     float *y_out, hipStream_t stream);

/*
 * MXFP4 variant (page "A Fused Hadamard + NVFP4 Quantization Kernel in
 * Triton", section 1 contrasts NVFP4 with MXFP4: 32-element blocks,
 * power-of-two E8M0 scales; its "Try this" list asks for the error study under
 * MXFP4; the page "Hopper kernel for MXFP4" stores a scale as one byte holding
 * a biased binary exponent, value 2^(byte - 127)).  One pass, no global scale:
 * each 32-element block (each 16-element half rotated by H16 when rotate == 1)
 * gets the scale 2^e with e = ceil(log2(fl(block_amax / 6))) clamped to
 * [-127, 127] (byte 0 for an all-zero block), so the block's largest value
 * maps into (3, 6]; each value becomes the E2M1 code of fl(y / 2^e) with the
 * NVFP4 path's midpoint and sign rules.
 *   x       device, row-major [rows, cols], 16-byte aligned, cols % 32 == 0.
 *   q_out   device, rows * cols / 2 bytes, 16-byte aligned (E2M1 codes, element
 *           2k in the low nibble of byte k).
 *   s_out   device, rows * cols / 32 bytes: E8M0 scale bytes [rows, cols/32].
 * Pointers may be NULL when rows * cols == 0.  Other rules as above.
 */
nvfp4_status mxfp4_rotquant(const uint16_t *x_bf16, int64_t rows, int64_t cols, int rotate,
                            uint8_t *q_out, uint8_t *s_out, hipStream_t stream);
nvfp4_status mxfp4_rotquant_f32(const float *x, int64_t rows, int64_t cols, int rotate,
                                uint8_t *q_out, uint8_t *s_out, hipStream_t stream);

/* MXFP4 dequantize: +-{0,.5,1,1.5,2,3,4,6}[code & 7] * 2^(byte - 127), rounded
   to binary32, then each 16-element half multiplied by H16 (same butterfly and
   * 0.25) when rotate == 1.  q: 16-byte aligned; y_out: float [rows, cols],
   16-byte aligned; cols % 32 == 0. */
nvfp4_status mxfp4_dequant(const uint8_t *q, const uint8_t *s, int64_t rows, int64_t cols,
                           int rotate, float *y_out, hipStream_t stream);

/*
 * Measurement support, not part of the method: the launch sequence of
 * nvfp4_rotquant (or _f32) for the same tensor, with each pass replaced by a
 * twin kernel that has the same grid, wave layout, load and store widths,
 * non-temporal rule and chunk order, and does no arithmetic beyond a bitwise
 * fold of the loaded words.  Timing it gives the ceiling the fused call's
 * byte mix (2 B read, then 2 B read and 0.5625 B written per bf16 element)
 * can reach on the machine at hand.
 *   x, rows, cols, q_out, s_out  as for nvfp4_rotquant; q_out and s_out
 *   receive meaningless bytes.
 * Errors as for nvfp4_rotquant.
 */
nvfp4_status nvfp4_stream_calibrate(const uint16_t *x_bf16, int64_t rows, int64_t cols,
                                    uint8_t *q_out, uint8_t *s_out, hipStream_t stream);
nvfp4_status nvfp4_stream_calibrate_f32(const float *x, int64_t rows, int64_t cols,
                                        uint8_t *q_out, uint8_t *s_out, hipStream_t stream);

/*
 * Measurement support, not part of the method: the same twin kernel launched
 * as a single pass with a workgroup per chunk, the launch shape of
 * nvfp4_quant_from_amax (and of mxfp4_rotquant, whose byte mix differs by
 * 1/32 B per element): 2 B read and 0.5625 B written per bf16 element, with
 * no earlier pass to leave any of the input in the caches.  Timing it gives
 * the ceiling of a single pass.  Arguments, outputs and errors as for
 * nvfp4_stream_calibrate.
 */
nvfp4_status nvfp4_stream_calibrate_single(const uint16_t *x_bf16, int64_t rows, int64_t cols,
                                           uint8_t *q_out, uint8_t *s_out, hipStream_t stream);
nvfp4_status nvfp4_stream_calibrate_single_f32(const float *x, int64_t rows, int64_t cols,
                                               uint8_t *q_out, uint8_t *s_out, hipStream_t stream);

/* Static English text for a status code; never NULL. */
const char *nvfp4_status_string(nvfp4_status status);

#ifdef __cplusplus
}
#endif

#endif /* NVFP4RQ_H */
