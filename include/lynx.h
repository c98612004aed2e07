/*
 * lynx.h - C ABI of the RT-Lynx sparse + LoRA linear layer for AMD MI355X (gfx950).
 *
 * The layer (RT-Lynx page, aitrends.kr, "RT-Lynx: Diffusion Transformers에서
 * GEMM Sparsity를 Activation으로 옮겨 실현하는 방법"; section 방법론, item
 * "핵심 메커니즘", and the two formulas of section 코드 예제):
 *
 *     X~   = X with, in every group of 4 consecutive input channels, only the
 *            two entries of largest |x| kept (Top-K 2:4 activation selection)
 *     s    = ||X||_2 / ||X~||_2 per token (row)      (Norm Compensation)
 *     Y    = s * (X~ W^T) + (X LB^T) LA^T           (= S(X) W^T + X (LA LB)^T)
 *
 * Readings fixed by this library where the page is silent:
 *   - groups are 4 consecutive channels of the reduction axis K, aligned at 0
 *     mod 4; ties in |x| go to the lower channel index; -0 and +0 are equal;
 *   - the page's eps is 0; a row whose X~ is zero (only an all-zero row) has s = 1;
 *   - the LoRA branch takes the dense, unscaled X; no bias.
 *
 * Conventions common to every entry point
 *   - bf16 tensors are passed as uint16_t bit patterns.
 *   - Every tensor pointer is a DEVICE pointer owned by the caller; tensors are
 *     contiguous; X, W, LA, LB, T and Y are row-major, the packed operand is
 *     stored as described below; every pointer must be 16-byte aligned.
 *   - Every call is asynchronous on `stream` (a hipStream_t; NULL = default
 *     stream).  The library never allocates device memory, never synchronizes
 *     (outside the debug mode below) and keeps no per-call state, so calls are
 *     re-entrant; concurrent calls that write the same buffers race, as with
 *     any kernel.
 *   - All arguments are validated before anything is launched.  On an error
 *     the status is returned and no output is written.
 *   - Asynchronous device faults surface at the caller's next synchronization
 *     with the stream, not as a status of the call that queued the work.
 *   - Debug mode: with the environment variable LYNX_DEBUG set to anything but
 *     "" or "0" (read on every call), a call that queued work waits for
 *     `stream` before it returns, and a failure of that wait (a fault of this
 *     call's kernels or of earlier work on the stream) is returned as
 *     LYNX_ERR_DEVICE.  A stream that is being captured into a graph is not
 *     waited for.  It serializes the caller; it is meant for debugging.
 *   - Inputs must be finite; NaN/Inf inputs give unspecified outputs.
 *   - Shape limits: K is a positive multiple of 64; M >= 0 and N >= 0 (0 is a
 *     no-op); R (LoRA rank) is one of 0, 16, 32, 48, 64 (0 = no LoRA branch);
 *     M, N, K <= 2^24; (M + 256) * K, (N + 256) * K and (M + 256) * N are each
 *     below 2^31 (every tensor, padded by one 256-row tile, smaller than 2^31
 *     elements, so that 32-bit byte offsets cover it).
 *   - The current device must be gfx950 (MI350 series); otherwise
 *     LYNX_ERR_UNSUPPORTED_DEVICE.
 *
 * Packed sparse operand (the 2:4 activation in the sparse matrix unit's
 * format, which the page has the sparsifier emit directly).  Per row:
 *   values row, K/2 bf16: the two kept entries of every group, in ascending
 *                channel order, copied bit-exactly from X (unscaled);
 *   meta row, K/8 bytes: a 4-bit code per group, (first kept position) |
 *                (second kept position) << 2, positions 0..3 inside the group,
 *                first < second; group 2j in the low nibble of byte j,
 *                group 2j+1 in the high nibble.
 * Storage order: tiles of 16 rows x 64 channels, the A operand of one
 * v_smfmac_f32_16x16x64_bf16 step, each tile contiguous.  With
 * Mp = M rounded up to a multiple of 16:
 *   values [Mp/16][K/64][16][32] bf16  (Mp * K/2 elements): kept value j of
 *          row m at ((m/16)*(K/64) + j/32)*512 + (m%16)*32 + j%32;
 *   meta   [Mp/16][K/64][16][8] uint8  (Mp * K/8 bytes): meta byte j of row m
 *          at ((m/16)*(K/64) + j/8)*128 + (m%16)*8 + j%8.
 * Rows M..Mp-1 are written as zero values and meta 0x44 (positions 0 and 1).
 * The 8 meta bytes of a row and step, read as four little-endian 16-bit
 * words, are the sparse-index operands of the row's four lane groups.
 *   scale  [M] fp32  : s per row;
 *   T      [M][R] bf16 (row-major): X LB^T, the LoRA down-projection of X.
 */
#ifndef LYNX_H
#define LYNX_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef void* lynx_stream_t; /* a hipStream_t */

typedef enum lynx_status {
    LYNX_OK = 0,
    LYNX_ERR_NULL = 1,               /* a required pointer is NULL */
    LYNX_ERR_SHAPE = 2,              /* a size is outside the limits above */
    LYNX_ERR_ALIGN = 3,              /* a pointer is not 16-byte aligned */
    LYNX_ERR_WORKSPACE = 4,          /* workspace is NULL or too small */
    LYNX_ERR_DEVICE = 5,             /* a HIP call or a kernel launch failed */
    LYNX_ERR_UNSUPPORTED_DEVICE = 6, /* the current device is not gfx950 */
    LYNX_ERR_SCRATCH = 7             /* the problem does not fit the static scratch array
                                        of lynx_linear_sparse_lora_noalloc */
} lynx_status;

/* Human-readable name of a status; never NULL. */
const char* lynx_status_string(lynx_status s);

/* Library version as MAJOR*10000 + MINOR*100 + PATCH. */
int lynx_version(void);

/*
 * Bytes of device workspace lynx_linear_sparse_lora needs for an (M, K, R)
 * problem: the packed operand (values Mp*K bytes, meta Mp*K/8, scale 4M) and
 * T (2MR), each 256-byte aligned.  Returns 0 for invalid sizes.
 */
size_t lynx_workspace_bytes(int64_t M, int64_t K, int64_t R);

/*
 * lynx_sparsify - online activation sparsification and LoRA down-projection.
 * Page: 방법론 "핵심 메커니즘" (Top-K 2:4 selection, S(X) = s X~) and
 * 핵심 기여 (pattern decision, Top-K and compression in one execution path,
 * emitting the sparse-unit layout).  One read of X produces:
 *   values (Mp*K/2 bf16), meta (Mp*K/8 bytes), scale [M] - the packed operand;
 *   T [M][R] = X LB^T (fp32 accumulation, rounded to bf16), if R > 0.
 * Inputs: X [M][K] bf16; LB [R][K] bf16 (NULL iff R == 0); T NULL iff R == 0.
 */
lynx_status lynx_sparsify(const uint16_t* X, const uint16_t* LB,
                          int64_t M, int64_t K, int64_t R,
                          uint16_t* values, uint8_t* meta, float* scale, uint16_t* T,
                          lynx_stream_t stream);

/*
 * lynx_linear_sparse_lora - the whole layer Y = S(X) W^T + X (LA LB)^T.
 * Page: 코드 예제, second formula; 방법론 "CUDA 커널 최적화" (the LoRA output
 * is produced and accumulated on chip inside the sparse GEMM).
 * Runs lynx_sparsify into `workspace`, then the 2:4 sparse-MFMA GEMM whose
 * epilogue adds T LA^T and applies s, with fp32 accumulation and a bf16
 * (round-to-nearest-even) store.
 * Inputs: X [M][K], W [N][K], LA [N][R], LB [R][K] (LA, LB NULL iff R == 0).
 * Output: Y [M][N] bf16.  workspace: >= lynx_workspace_bytes(M, K, R) bytes,
 * 256-byte aligned, contents on entry irrelevant, clobbered.
 */
lynx_status lynx_linear_sparse_lora(const uint16_t* X, const uint16_t* W,
                                    const uint16_t* LA, const uint16_t* LB, uint16_t* Y,
                                    int64_t M, int64_t N, int64_t K, int64_t R,
                                    void* workspace, size_t workspace_bytes,
                                    lynx_stream_t stream);

/*
 * lynx_linear_sparse_lora_noalloc - lynx_linear_sparse_lora without a
 * workspace argument, for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  Same inputs, output, kernels and results as
 * lynx_linear_sparse_lora; the packed operand, s and T go to a static device
 * array of the library (64 MiB per device, LYNX_SCRATCH_BYTES), allocated
 * when the library's code is loaded on a device and held until the process
 * ends.  The call itself allocates nothing, on the device or the host.
 *   - Problems whose lynx_workspace_bytes(M, K, R) exceeds LYNX_SCRATCH_BYTES
 *     return LYNX_ERR_SCRATCH (e.g. M = 4096 fits up to K = 12288 with
 *     R = 64; M = 9216 fits up to K = 6144).
 *   - Every call on a device shares that device's array, which keeps the last
 *     call's contents (each call writes every byte it reads before reading
 *     it).  Calls that overlap on one device - on different streams, or from
 *     different host threads without ordering - race on the array and give
 *     undefined results; calls on one stream are ordered and safe.
 *   - The first call on each device looks up the array's device address
 *     (hipGetSymbolAddress) and keeps it; a failure there returns
 *     LYNX_ERR_DEVICE.
 */
#define LYNX_SCRATCH_BYTES ((size_t)64 << 20)

lynx_status lynx_linear_sparse_lora_noalloc(const uint16_t* X, const uint16_t* W,
                                            const uint16_t* LA, const uint16_t* LB, uint16_t* Y,
                                            int64_t M, int64_t N, int64_t K, int64_t R,
                                            lynx_stream_t stream);

/*
 * lynx_linear_sparse_lora_packed - the GEMM half of the layer on an already
 * packed operand: Y = scale * (X~ W^T) + T LA^T, X~ given by values + meta.
 * Same page passages as lynx_linear_sparse_lora.  Used to time the sparse
 * GEMM apart from the sparsifier.  T and LA NULL iff R == 0.
 */
lynx_status lynx_linear_sparse_lora_packed(const uint16_t* values, const uint8_t* meta,
                                           const float* scale, const uint16_t* T,
                                           const uint16_t* W, const uint16_t* LA, uint16_t* Y,
                                           int64_t M, int64_t N, int64_t K, int64_t R,
                                           lynx_stream_t stream);

/*
 * lynx_linear_dense - the dense layer Y = X W^T, bf16 MFMA, fp32 accumulate,
 * bf16 store: the baseline the page's speedups are quoted against
 * (주요 결과, speed/efficiency item).  No LoRA branch.
 */
lynx_status lynx_linear_dense(const uint16_t* X, const uint16_t* W, uint16_t* Y,
                              int64_t M, int64_t N, int64_t K, lynx_stream_t stream);

/*
 * A sequence of linear layers, each either sparse + LoRA or dense: the
 * block-level driver of selective layer skipping (방법론 "핵심 메커니즘",
 * Selective Layer Skipping; 구현 및 학습 세부: in single-stream blocks some
 * layers, e.g. Out/OUp, are left out of the sparsification).  A skipped
 * layer is the original dense layer Y = X W^T (no LoRA branch, which only
 * corrects the sparse one).
 */
typedef enum lynx_layer_mode {
    LYNX_LAYER_SPARSE_LORA = 0,  /* Y = S(X) W^T + X (LA LB)^T, as lynx_linear_sparse_lora */
    LYNX_LAYER_DENSE = 1         /* Y = X W^T, as lynx_linear_dense; LA, LB, R ignored */
} lynx_layer_mode;

typedef struct lynx_layer {
    const uint16_t* X;   /* [M][K] bf16 */
    const uint16_t* W;   /* [N][K] bf16 */
    const uint16_t* LA;  /* [N][R] bf16, NULL iff R == 0 or the layer is dense */
    const uint16_t* LB;  /* [R][K] bf16, NULL iff R == 0 or the layer is dense */
    uint16_t* Y;         /* [M][N] bf16 output */
    int64_t M, N, K, R;
    int32_t mode;        /* a lynx_layer_mode */
} lynx_layer;

/*
 * Bytes of workspace lynx_linear_sequence needs: the largest
 * lynx_workspace_bytes(M, K, R) over its sparse layers (0 if there are none,
 * or if any layer is invalid).  layers: host array of n descriptors.
 */
size_t lynx_sequence_workspace_bytes(const lynx_layer* layers, int64_t n);

/*
 * Runs the n layers in order on `stream` (host array of n descriptors; every
 * pointer inside is a device pointer).  All layers are validated before any
 * launch; on an error nothing is written and the first failing layer's status
 * is returned.  workspace: >= lynx_sequence_workspace_bytes(layers, n) bytes,
 * 256-byte aligned (NULL allowed when no layer is sparse), shared by the
 * sparse layers one after another, contents on entry irrelevant, clobbered.
 * n == 0 is a no-op.  Layers must not write an input of a later layer unless
 * that order is intended: they run exactly in sequence.
 */
lynx_status lynx_linear_sequence(const lynx_layer* layers, int64_t n, void* workspace,
                                 size_t workspace_bytes, lynx_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* LYNX_H */
