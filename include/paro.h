/*
 * paro.h -- C ABI of the MI355X (gfx950) rotated W4A16 linear library (libparo.so).
 *
 * The operation is the runtime hot path of ParoQuant ("ParoQuant: pairwise
 * rotations that survive deployment", hungho77.github.io, and the arXiv
 * abstract of "ParoQuant: Pairwise Rotation Quantization for Efficient
 * Reasoning LLM Inference"):
 *
 *   - K stages of Givens rotations over disjoint channel pairs; for a pair
 *     (i, j) with angle t:  x'_i = cos t * x_i + sin t * x_j,
 *                           x'_j = -sin t * x_i + cos t * x_j
 *     (section "A rotation small enough to execute", the 2x2 equation);
 *     every channel is in exactly one pair of each stage, so the pairs of a
 *     stage are independent;
 *   - channel-wise scaling after the rotations; at runtime the activations are
 *     divided by s, at build time the weights are rotated by the same stages
 *     and multiplied by s ("weight transformations are folded and quantized",
 *     same section), so that transform(x) . W'^T = x . W^T;
 *   - a group-wise asymmetric INT4 weight-only linear (W4A16, group 128 along
 *     the input dimension; section "My reduced-calibration experiment"), one
 *     per layer right after the transform (section "From fake quantization to
 *     a real TensorRT engine").
 *
 * Conventions shared by every call
 *   - Shapes: x is [M][D] row-major float16, W is [N][D] row-major float16,
 *     y = transform(x) . dequant(W')^T is [M][N] row-major.
 *   - Packed weights: qweight is N*D/2 bytes of 4-bit codes, two per byte:
 *     byte t of row n's packed row (t < D/2) holds channel 2t in bits 0..3
 *     and channel 2t+1 in bits 4..7. The rows are stored in blocks of 16 (the
 *     last block holds the N % 16 remaining rows, if any): block b starts at
 *     byte 16*b*D/2 and stores its R_b = min(16, N - 16*b) rows group by group,
 *     so byte t of row n = 16*b + r is at
 *         16*b*D/2 + (t/64)*R_b*64 + r*64 + t%64
 *     (with N % 16 == 0: an array [N/16][D/128][16][64]). The linears read one
 *     group of 16 rows as one contiguous kilobyte. scales float16 [N][D/128];
 *     zeros float16 [N][D/128] holding integers 0..15. Dequantized weight:
 *     (q - z) * scale.
 *   - Quantizer (per row n, group g of 128 channels of the folded weights b,
 *     in float64): scale = fp16_rne(max((max b - min b) / 15, 1e-5));
 *     z = clip(rint(-min b / scale), 0, 15); q = clip(rint(b / scale) + z, 0, 15).
 *   - Every pointer argument named *_dev, x, y, W, qweight, scales, zeros, ws
 *     is a DEVICE pointer on the current HIP device; *_host arguments are host
 *     pointers. Device pointers must be 16-byte aligned.
 *   - The linears read scales and zeros as aligned 32-bit words: when
 *     N * D/128 is odd, the word holding the last element also covers the 2
 *     bytes after the array (never a separate page); they are not used.
 *   - The caller owns every buffer. The library allocates nothing, frees
 *     nothing and keeps no mutable global state; calls are re-entrant. The
 *     one exception is paro_rotated_linear_noalloc's fixed scratch array (see
 *     there), which every GPU the library runs on holds from load to exit.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream) and
 *     is asynchronous, except paro_rotation_prepare, which synchronizes
 *     `stream` once its upload is enqueued.
 *   - Errors: argument and shape checks run on the host before anything is
 *     enqueued and return a status; a failed launch returns PARO_EHIP. Faults
 *     inside a kernel surface at the caller's next synchronization.
 *   - Limits: D even, D % 128 == 0, 128 <= D <= PARO_MAX_D; 0 <= K <=
 *     PARO_MAX_K; M >= 0 and N >= 0 (zero sizes enqueue nothing and succeed).
 */
#ifndef PARO_H
#define PARO_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PARO_GROUP 128
#define PARO_MAX_D 16384
#define PARO_MAX_K 64

typedef enum {
  PARO_OK = 0,
  PARO_EINVAL = 1,     /* null or misaligned pointer, negative size, bad dtype, aliasing */
  PARO_ESHAPE = 2,     /* D odd, D % 128 != 0, D outside [128, PARO_MAX_D], K outside [0, PARO_MAX_K] */
  PARO_EPAIRS = 3,     /* a stage does not pair every channel exactly once */
  PARO_ESCALE = 4,     /* a channel scale is not finite and > 0, or an angle is not finite */
  PARO_EWORKSPACE = 5, /* workspace missing or smaller than paro_workspace_bytes() */
  PARO_EHIP = 6        /* the HIP runtime reported an error (launch or copy) */
} paro_status;

typedef enum { PARO_F16 = 0, PARO_F32 = 1 } paro_dtype; /* element type of y */

/* A prepared transform: plain data, copyable. `dev` points at the caller-owned
 * device descriptor written by paro_rotation_prepare. */
typedef struct {
  int32_t K;
  int32_t D;
  void* dev;
} paro_rotation;

/* Human-readable name of a status code (static string, never NULL). */
const char* paro_status_str(int status);

/* Library version as MAJOR*10000 + MINOR*100 + PATCH. */
int paro_version(void);

/* Bytes of device memory a descriptor for (K, D) needs; 0 if (K, D) is invalid. */
size_t paro_rotation_bytes(int K, int D);

/*
 * paro_rotation_encode -- host-only half of paro_rotation_prepare: validate a
 * transform (same arguments and errors as paro_rotation_prepare) and write its
 * descriptor into the HOST buffer desc_host (desc_bytes >= paro_rotation_bytes).
 * Makes no HIP call. Copying those bytes to 16-byte aligned device memory and
 * setting paro_rotation {K, D, device pointer} is equivalent to
 * paro_rotation_prepare.
 *
 * Descriptor layout (each section starts at a multiple of 256 bytes, in order):
 *   struct { uint32 4i | (4j << 16); float cos; float sin; } rec[K][D/2]   (12 bytes each;
 *          4i and 4j are the channels' byte offsets in a float32 row, < 65536 as D <= 16384)
 *   float  inv_s[D]        float32(1 / s)
 *   float  s[D]
 * Within a stage the pairs are stored in a library-chosen order, and a pair
 * (i, j, cos, sin) may be stored as (j, i, cos, -sin), which is the same
 * rotation; the order is a function of the set of pairs only.
 */
paro_status paro_rotation_encode(int K, int D, const int32_t* pairs_host, const float* theta_host,
                                 const float* scale_host, void* desc_host, size_t desc_bytes);

/*
 * paro_rotation_prepare -- validate a transform and upload its descriptor.
 *
 * Defines the transform of section "A rotation small enough to execute":
 *   pairs_host  int32 [K][D/2][2]: stage k's pairs (i, j); each stage must use
 *               every channel 0..D-1 exactly once (else PARO_EPAIRS);
 *   theta_host  float32 [K][D/2]: one angle per pair per stage (finite);
 *   scale_host  float32 [D]: channel scales s > 0 (finite).
 * cos/sin are evaluated in float64 by the C library and rounded once to
 * float32; 1/s is rounded once to float32. The descriptor (layout above) is copied into
 * desc_dev (desc_bytes >= paro_rotation_bytes(K, D)) on `stream`, which is then
 * synchronized so the host arrays may be released on return. On success *out
 * = {K, D, desc_dev}. Nothing is written to the device on an error.
 */
paro_status paro_rotation_prepare(int K, int D, const int32_t* pairs_host, const float* theta_host,
                                  const float* scale_host, void* desc_dev, size_t desc_bytes,
                                  paro_rotation* out, void* stream);

/*
 * paro_pack_weights -- build-time weight fold and INT4 quantization.
 *
 * For each row of W (float16 [N][D]), in float64 with no fused multiply-add:
 * apply the K stages (stage 1 first, same expressions as the activation side),
 * multiply by s, then quantize each 128-channel group as stated at the top and
 * pack the codes. Writes qweight (N*D/2 bytes, the blocked row order stated at
 * the top), scales [N][D/128], zeros [N][D/128].
 * The outputs are bit-identical to the stated float64 definition
 * ("weight transformations are folded and quantized", section "A rotation
 * small enough to execute"; "real INT4 packing", section "From fake
 * quantization to a real TensorRT engine"). W must not alias the outputs.
 */
paro_status paro_pack_weights(const paro_rotation* r, int N, const void* W, uint8_t* qweight,
                              void* scales, void* zeros, void* stream);

/*
 * paro_rotate -- runtime activation-side transform (section "A rotation small
 * enough to execute": the inverse activation-side transformation runs right
 * before the INT4 linear). xout[m][:] = fp16(G_K...G_1 x[m][:] / s), computed
 * in float32 and rounded once to float16. x and xout are float16 [M][D] and
 * must not overlap.
 */
paro_status paro_rotate(const paro_rotation* r, int M, const void* x, void* xout, void* stream);

/* Workspace bytes that suffice for paro_w4a16_linear / paro_rotated_linear at
 * (M, D, N) with any transform (0 for M <= 0 or an invalid D): M * D * 2 rounded
 * up to 256 for the transformed x, plus, for prefill-shaped calls (M > 16), room
 * for the float32 partial sums [S][M][N] of a GEMM whose reduction over D is
 * split S ways to fill the GPU. Calls whose transform runs inside the decode
 * kernel (see paro_rotated_linear) use none of it and accept ws == NULL. */
size_t paro_workspace_bytes(int M, int D, int N);

/*
 * paro_w4a16_linear -- plain group-wise INT4 weight-only linear (section "From
 * fake quantization to a real TensorRT engine": one group-wise INT4 GEMM per
 * layer): y[m][n] = sum_g scale[n][g] * sum_{k in g} x[m][k] * (q[n][k] - z[n][g]),
 * products of float16 values exact, accumulation in float32, y stored as
 * ydtype (PARO_F16 rounds once). A group whose scale is zero contributes
 * nothing, as the formula says (paro_pack_weights never writes one: its scales
 * are at least fp16(1e-5)); a non-finite scale makes the outputs it reaches
 * non-finite. x float16 [M][D]; y [M][N] must not overlap
 * any input. ws is an optional device buffer: given at least
 * paro_workspace_bytes(M, D, N) bytes (which must not overlap any operand), a
 * prefill-shaped call may split its reduction over D and keep the partial sums
 * there; with less (or NULL) it does not split. The two differ only in float32
 * summation order; each is deterministic.
 */
paro_status paro_w4a16_linear(int M, int D, int N, const void* x, const uint8_t* qweight,
                              const void* scales, const void* zeros, void* y, int ydtype, void* ws,
                              size_t ws_bytes, void* stream);

/*
 * paro_rotated_linear -- the fused runtime path: the activation transform of
 * paro_rotate (float32, rounded once to float16 as the linear's 16-bit
 * operand) immediately followed by the INT4 linear of paro_w4a16_linear, with
 * the weights packed by paro_pack_weights for the same transform. With M <= 16,
 * D <= 4096, K <= 8 and (ceil(M / 4) - 1) * (N * D / 2 + N * D / 32) <= 16 MiB
 * (the transform runs per 4-row unit and every unit reads all the weights), or
 * with M = 1, 4096 < D <= 9216 and K <= 8, the transform runs inside the
 * decode kernel (one launch, no workspace);
 * otherwise a transform kernel writes x' into ws, which must
 * then hold at least paro_workspace_bytes(M, D, N) bytes (else
 * PARO_EWORKSPACE; the rest of it serves the linear as above), and the linear
 * reads it, on `stream`. Arguments as in paro_w4a16_linear, with D = r->D.
 */
paro_status paro_rotated_linear(const paro_rotation* r, int M, int N, const void* x,
                                const uint8_t* qweight, const void* scales, const void* zeros,
                                void* y, int ydtype, void* ws, size_t ws_bytes, void* stream);

/*
 * paro_rotated_linear_noalloc -- paro_rotated_linear for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).
 * Same arguments, results and errors as paro_rotated_linear, without a workspace argument: the
 * call's workspace (paro_workspace_bytes(M, D, N) at most) is a fixed scratch array inside the
 * library, paro_noalloc_max_bytes() = 64 MiB on every GPU the library runs on (held until the
 * process ends). A call whose workspace would exceed it returns PARO_EWORKSPACE before
 * anything is enqueued. The call allocates and frees nothing; its first call on a device looks
 * up that device's scratch address once. Every call on one GPU shares that GPU's scratch, so
 * calls that overlap in time on one GPU (two streams, two host threads) race; calls on one
 * stream are ordered and safe. Nothing in the scratch needs to start at zero.
 */
paro_status paro_rotated_linear_noalloc(const paro_rotation* r, int M, int N, const void* x,
                                        const uint8_t* qweight, const void* scales, const void* zeros,
                                        void* y, int ydtype, void* stream);

/* Bytes of the scratch array paro_rotated_linear_noalloc uses (its largest workspace). */
size_t paro_noalloc_max_bytes(void);

/* One linear of a batch: paro_rotated_linear(rot, ...) when rot != NULL (then D
 * must equal rot->D), else paro_w4a16_linear(M, D, N, ...). Pointers as there. */
typedef struct {
  const paro_rotation* rot;
  int32_t M;
  int32_t D;
  int32_t N;
  const void* x;
  const uint8_t* qweight;
  const void* scales;
  const void* zeros;
  void* y;
} paro_linear_args;

/* Workspace bytes paro_linear_batch needs for these calls (may be 0). */
size_t paro_linear_batch_workspace_bytes(int count, const paro_linear_args* calls);

/*
 * paro_linear_batch -- `count` independent linears of the kind above (a decode
 * step's projections, say), each computing bit for bit what its single call
 * computes, in as few launches as their shapes allow:
 *   - decode-shaped calls (M <= 16) that share D: one decode-kernel launch,
 *     their transforms inside it where the single call runs them there;
 *   - the other rotated calls of up to 256 rows: their transforms as one launch
 *     per D (or as few as the GPU holds at once); the decode-shaped ones among
 *     them (D or K past what the decode kernel runs inside) then run their
 *     linears as one decode launch per D;
 *   - calls of 17..64 rows: one skinny-kernel launch per kernel variant (x word
 *     order, scale layout), their split reductions one launch at the end; other
 *     calls of up to 256 rows that share a GEMM tiling: one grouped launch, its
 *     split reductions one more;
 *   - longer calls one at a time, a rotated one's transform right before its
 *     linear or, with two or more long rotated calls, all their transforms
 *     ahead on the library's second stream, each linear waiting for its own.
 * When the rotated calls have several D, the transforms of every D but the one
 * with the most packed weight bytes run on the library's second stream,
 * concurrently with the rest. The second stream joins `stream` through events:
 * both are created per device on the first batch that needs them, outside any
 * stream capture (a batch whose first use falls inside a capture runs on
 * `stream` alone, with the same kernels and results). Each call uses its own
 * consecutive slice of ws (ws_bytes >= paro_linear_batch_workspace_bytes). The
 * calls may run concurrently, so no call's y may overlap any buffer of another
 * call (PARO_EINVAL); every call is checked as its single call would be before
 * anything is enqueued. The `calls` array is read during the call only (host
 * memory).
 */
paro_status paro_linear_batch(int count, const paro_linear_args* calls, int ydtype, void* ws,
                              size_t ws_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PARO_H */
