/*
 * flce.h -- fused linear cross-entropy forward and backward on AMD Instinct
 * MI355X (gfx950).
 *
 * The operation is the one defined on the page "Een gefuseerde forward-kernel
 * voor lineaire cross-entropy op Apple-GPU's" (section 1): for hidden states H
 * (N x D) and an output projection W (V x D) the logits are Z = H W^T, and
 * for each token i with target y_i
 *
 *     lse_i  = logsumexp_v Z[i, v]          (natural logarithm)
 *     loss_i = lse_i - Z[i, y_i].
 *
 * The same section observes that only these two per-row statistics are
 * needed, so the library streams vocabulary tiles of Z through the online
 * (running max m, scaled sum s) update of that section and never stores the
 * N x V logits: device memory beyond the caller's buffers is a workspace of
 * (2*C + 1)*N floats, where C (the number of vocabulary chunks per row
 * block) is at most a few hundred.
 *
 * Entry points: the forward (flce_forward, flce_forward_ws, and its two
 * launches flce_partials and flce_merge); its backward (flce_backward: dH and
 * dW from the forward's lse, regenerating the logits); the forward and a
 * frozen head's backward with the head stored quantised (flce_forward_quant,
 * flce_backward_quant); workspace sizes, the tile plan, status text and the
 * version.
 *
 * Conventions for every entry point:
 *   - H, W, targets, loss_out, lse_out, workspace (and, for the backward,
 *     lse, grad_loss, dH and dW; for a quantised head, codes, scales and
 *     biases) are DEVICE pointers owned by the caller. The library never
 *     frees them and keeps none of them after the call returns.
 *   - H is N x D and W is V x D, row-major and dense (row stride D elements),
 *     both of `dtype`. They must be 16-byte aligned and D * sizeof(element)
 *     must be a multiple of 16 (D % 8 == 0 for bf16, D % 4 == 0 for fp32).
 *   - targets is int32[N]; loss_out and lse_out are float32[N]; lse_out may be
 *     NULL when only the loss is wanted.
 *   - A target outside [0, V) is not an error: that row's loss is NaN and its
 *     lse is still written. NaN or Inf inputs propagate to the affected rows.
 *   - stream is a hipStream_t passed as void*; NULL means the default stream.
 *     Work is enqueued on it and the call returns without waiting; results
 *     are valid once the stream has completed.
 *   - Errors are reported only through the returned status (no exceptions,
 *     no abort); on an error status nothing has been enqueued.
 *   - All entry points are thread-safe and reentrant. Concurrent calls may
 *     share H and W but not outputs or a workspace.
 *   - Every entry point except flce_forward enqueues kernel launches only (no
 *     allocation, no memset, no copy), so it can be captured into a HIP graph
 *     and replayed; flce_forward adds a stream-ordered allocation and free of
 *     its workspace.
 *   - Accumulation is fp32 (bf16 x bf16 and fp32 x fp32 products on the
 *     matrix cores); outputs are fp32.
 */
#ifndef FLCE_H
#define FLCE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { FLCE_BF16 = 0, FLCE_FP32 = 1 } flce_dtype_t;

typedef enum {
  FLCE_OK = 0,
  FLCE_ERR_INVALID_ARG = -1, /* null pointer, bad size, misalignment, small workspace */
  FLCE_ERR_UNSUPPORTED = -2, /* unknown dtype, D*elem not a multiple of 16, sizes past int32 */
  FLCE_ERR_HIP = -3,         /* a HIP runtime call or a kernel launch failed */
  FLCE_ERR_OOM = -4,         /* the stream-ordered workspace allocation failed */
  FLCE_ERR_SCRATCH = -5      /* flce_forward_noalloc: the shape needs more than its static scratch */
} flce_status_t;

/* How a shape is split into work. Filled by flce_get_plan (diagnostics). */
typedef struct {
  int32_t tile_vocab;      /* vocabulary rows per tile (BV) */
  int32_t tile_tokens;     /* tokens per tile (BT) */
  int32_t row_blocks;      /* ceil(N / BT) */
  int32_t vocab_tiles;     /* ceil(V / BV) */
  int32_t chunks;          /* C: vocabulary chunks per row block */
  int32_t grid;            /* workgroups of the partials kernel */
  int32_t xcd_rows;        /* row blocks per XCD group */
  int32_t xcd_chunks;      /* chunks per XCD group */
  int32_t threads;         /* threads per workgroup of the partials kernel */
  int32_t lds_bytes;       /* LDS per workgroup */
  size_t workspace_bytes;  /* flce_workspace_bytes for the shape */
} flce_plan_t;

/*
 * Loss and lse for every row: the whole forward (partials, then merge).
 * Gets its workspace with hipMallocAsync on `stream` and releases it with
 * hipFreeAsync on the same stream (FLCE_ERR_OOM if that allocation fails).
 * N == 0 is a no-op returning FLCE_OK.
 */
int flce_forward(const void* H, const void* W, const int32_t* targets,
                 int64_t N, int64_t D, int64_t V, int dtype,
                 float* loss_out, float* lse_out, void* stream);

/* Workspace bytes flce_forward_ws needs for a shape (0 for N == 0, and 0 for
 * an invalid or unsupported shape). */
size_t flce_workspace_bytes(int64_t N, int64_t D, int64_t V, int dtype);

/*
 * As flce_forward, with a caller-provided device workspace of at least
 * flce_workspace_bytes(N, D, V, dtype) bytes, 256-byte aligned
 * (FLCE_ERR_INVALID_ARG otherwise). Allocates nothing.
 */
int flce_forward_ws(const void* H, const void* W, const int32_t* targets,
                    int64_t N, int64_t D, int64_t V, int dtype,
                    float* loss_out, float* lse_out,
                    void* workspace, size_t workspace_bytes, void* stream);

/*
 * As flce_forward, for callers that cannot allocate device memory at all:
 * code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc. It calls no allocator (no hipMalloc, hipMallocAsync, hipFree or
 * allocating library routine) and takes no workspace argument: its
 * workspace is a static 16 MiB device array inside the library, one copy per
 * GPU, held until the process ends (the current device's copy is located on
 * its first call there; `stream` must belong to the current device).
 *   - The shape must need at most 16 MiB of workspace, i.e.
 *     flce_workspace_bytes(N, D, V, dtype) <= 16 << 20 (the production shape
 *     N = 8192, D = 4096, V = 151936 needs 0.56 MB); a larger one returns
 *     FLCE_ERR_SCRATCH and enqueues nothing.
 *   - Every call on one GPU uses that GPU's one array, and nothing in it is
 *     carried from call to call (each call writes every value it reads), so
 *     calls on one GPU must not overlap: two calls in flight at once on
 *     different streams of the same GPU race on the array. Serialize them
 *     (one stream, or events).
 *   - Results are bit-identical to flce_forward_ws for the same inputs (the
 *     same kernels and plan). Other conventions as for flce_forward.
 */
int flce_forward_noalloc(const void* H, const void* W, const int32_t* targets,
                         int64_t N, int64_t D, int64_t V, int dtype,
                         float* loss_out, float* lse_out, void* stream);

/*
 * The first of the two launches of flce_forward_ws, on its own: the fused
 * tile contraction Z_tile = H_blk W_blk^T with the online (m, s) update and
 * the target-logit capture (page section 1, the update equations). Writes,
 * into the workspace, one (m, s) pair per (row, chunk) and the target logit
 * per row. Useful for timing the contraction apart from the merge.
 */
int flce_partials(const void* H, const void* W, const int32_t* targets,
                  int64_t N, int64_t D, int64_t V, int dtype,
                  void* workspace, size_t workspace_bytes, void* stream);

/*
 * The second launch: combines the C partial (m, s) pairs of each row into
 * lse = M + ln(sum_c s_c e^(m_c - M)) with M = max_c m_c (the page's update
 * applied between chunks), and loss = lse - z_y. Reads a workspace filled
 * by flce_partials for the same (N, D, V, dtype) and targets.
 */
int flce_merge(const int32_t* targets, int64_t N, int64_t D, int64_t V, int dtype,
               float* loss_out, float* lse_out,
               const void* workspace, size_t workspace_bytes, void* stream);

/*
 * Backward of the same loss, for an upstream gradient g = grad_loss (one
 * float32 per token; g_i = 1/N for a mean over tokens): the gradients of
 * sum_i g_i loss_i,
 *
 *     dZ_iv = g_i (softmax(Z_i)_v - [v == y_i]),   dH = dZ W,   dW = dZ^T H,
 *
 * by the chain rule on the section 1 definition. As on the page (section 1:
 * the training path keeps the forward's log-sum-exp and regenerates the
 * logits tile by tile for its backward), `lse` is the forward's lse_out for
 * the same H, W and targets, and Z is recomputed, never stored whole.
 *
 *   - dH (N x D) and dW (V x D) are float32 DEVICE outputs, row-major, fully
 *     overwritten (N == 0 writes dW = 0 and reads nothing else); dH must be
 *     16-byte aligned, dW 4-byte aligned.
 *   - A target outside [0, V) matches no vocabulary row: that row contributes
 *     g_i softmax(Z_i), the gradient of its lse alone. Pass g_i = 0 to leave a
 *     row out.
 *   - dZ is rounded to `dtype` before the two products (fp32 accumulation);
 *     the result differs from exact arithmetic by about the unit roundoff of
 *     `dtype` times the sum of the absolute values of each output's terms.
 *   - The vocabulary is processed in slices so that dZ, which is N x V, only
 *     ever exists for one slice: each slice's dZ (transposed; for fp32 also
 *     row-major) stays within 1 GiB whatever N and V are, each slice writes
 *     its own rows of dW, and the slices' contributions to dH are added in
 *     slice order (deterministic). The workspace (flce_backward_workspace_bytes,
 *     256-byte aligned, FLCE_ERR_INVALID_ARG if smaller) holds one slice of W
 *     transposed, H transposed and that dZ (each dimension rounded up to 64
 *     elements); for bf16 shapes whose dH product alone would leave compute
 *     units idle, also S x N x D float32 partial sums of dH (2 <= S <= 16
 *     pieces of a slice's contraction, added in order). No O(N x V) memory:
 *     1.43 GB in all at N = 8192, D = 4096, V = 151936 in bf16, where the
 *     fp32 logits alone would take 4.98 GB. Allocates nothing.
 *   - Other conventions (alignment, D * sizeof(element) % 16 == 0, stream,
 *     status codes) as for the forward.
 */
int flce_backward(const void* H, const void* W, const int32_t* targets,
                  const float* lse, const float* grad_loss,
                  int64_t N, int64_t D, int64_t V, int dtype,
                  float* dH, float* dW,
                  void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes flce_backward needs for a shape (0 for an invalid or
 * unsupported shape). */
size_t flce_backward_workspace_bytes(int64_t N, int64_t D, int64_t V, int dtype);

/*
 * Forward with a quantised output head. The page mentions output heads stored
 * quantised (section 2: its first, chunked prototype handled dense and
 * quantised heads; section 9 leaves the quantised variants of the fused kernel
 * out of scope) but fixes no format. This library takes a groupwise affine
 * one: W (V x D) is given as unsigned integer codes q with one float32 scale
 * and one float32 bias per group of `group` consecutive weights of a row, and
 * the head the forward uses is, weight by weight,
 *
 *     w[v][d] = bf16( fl32( fl32(scale[v][g] * q[v][d]) + bias[v][g] ) ),
 *     g = d / group,  bf16() rounding to nearest even,
 *
 * after which loss and lse are exactly as flce_forward computes them for H
 * and that bf16 W.
 *   - H is bf16, N x D as for flce_forward (16-byte aligned, D % 8 == 0).
 *   - bits is 8 (codes: V x D bytes, row-major) or 4 (V x D/2 bytes: byte b
 *     of a row holds weight 2b in its low nibble and 2b+1 in its high one);
 *     codes 16-byte aligned.
 *   - group: a multiple of 8 that divides D; scales and biases are float32
 *     [V][D / group], 4-byte aligned.
 *   - The vocabulary is dequantised slice by slice (about 256 MB of bf16 at a
 *     time) into the workspace, so device memory stays at the codes plus one
 *     slice; a vocabulary that fits one slice gives the same bits as
 *     flce_forward on the dequantised W.
 *   - workspace: flce_forward_quant_workspace_bytes(N, D, V, bits, group)
 *     bytes, 256-byte aligned (FLCE_ERR_INVALID_ARG if smaller). Allocates
 *     nothing. bits not 4 or 8, or a bad group: FLCE_ERR_UNSUPPORTED. Other
 *     conventions as for flce_forward.
 */
int flce_forward_quant(const void* H, const uint8_t* codes, const float* scales, const float* biases,
                       const int32_t* targets, int64_t N, int64_t D, int64_t V, int bits, int group,
                       float* loss_out, float* lse_out,
                       void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes flce_forward_quant needs (0 for N == 0 or an invalid or
 * unsupported shape). */
size_t flce_forward_quant_workspace_bytes(int64_t N, int64_t D, int64_t V, int bits, int group);

/*
 * Backward of flce_forward_quant for a frozen head: dH (N x D, float32,
 * 16-byte aligned, fully overwritten) of sum_i g_i loss_i, where the loss is
 * the one flce_forward_quant defines and lse is its lse_out for the same
 * inputs. The head (codes, scales, biases) gets no gradient. Computed as
 * flce_backward computes dH for the dequantised bf16 W (dZ rounded to bf16,
 * float32 accumulation), one vocabulary slice at a time (at most the
 * forward's dequantisation slice, and small enough that the slice's dZ stays
 * within 1 GiB): each slice's dH contribution is added into dH in slice order
 * (deterministic); a vocabulary that fits one slice gives the same bits as
 * flce_backward's dH on the dequantised W.
 *   - workspace: flce_backward_quant_workspace_bytes(N, D, V, bits, group)
 *     bytes, 256-byte aligned: one dequantised slice, its transpose and dZ of
 *     all rows for the slice (transposed); for shapes whose dH product would
 *     leave compute units idle, also the partial sums of its split
 *     contraction. Allocates nothing. N == 0 enqueues nothing.
 *   - Format, alignment and status codes as for flce_forward_quant and
 *     flce_backward.
 */
int flce_backward_quant(const void* H, const uint8_t* codes, const float* scales, const float* biases,
                        const int32_t* targets, const float* lse, const float* grad_loss,
                        int64_t N, int64_t D, int64_t V, int bits, int group, float* dH,
                        void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes flce_backward_quant needs (0 for N == 0 or an invalid or
 * unsupported shape). */
size_t flce_backward_quant_workspace_bytes(int64_t N, int64_t D, int64_t V, int bits, int group);

/* Tile plan for a shape; FLCE_ERR_INVALID_ARG/UNSUPPORTED as flce_forward. */
int flce_get_plan(int64_t N, int64_t D, int64_t V, int dtype, flce_plan_t* plan);

/* Static text for a status code; never NULL. */
const char* flce_status_string(int status);

/* Library ABI version (major * 10000 + minor * 100 + patch). */
int flce_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FLCE_H */
