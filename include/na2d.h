/*
 * na2d.h -- C ABI of the fused 2D Neighborhood Attention forward pass for
 * AMD Instinct MI355X (gfx950).
 *
 * The operation is Neighborhood Attention as defined in "Neighborhood
 * Attention Transformer" (CSDN translation of the CVPR 2023 paper, section
 * 3.1, equations 2-4; restated in the qiita article "NAT:
 * スライディングウィンドウアテンションの革新", section "Neighborhood
 * Attention(NA)").  For every pixel (y, x) of an H x W map, every head h and
 * every batch item b:
 *
 *   sy = clamp(y - ksize/2, 0, H - ksize),  sx = clamp(x - ksize/2, 0, W - ksize)
 *   for the ksize*ksize keys (ky, kx) in [sy, sy+ksize) x [sx, sx+ksize):
 *     logit = (q[b,h,y,x,:] . k[b,h,ky,kx,:] + rpb[h, ky-y+ksize-1, kx-x+ksize-1]) / sqrt(d)
 *   out[b,h,y,x,:] = sum over keys of softmax(logit) * v[b,h,ky,kx,:]
 *
 * The window is the per-axis set of the ksize nearest pixels, pushed inward
 * at the borders so every pixel keeps the same span (CSDN page, section 1 and
 * section 3.1; qiita border figure).  The bias is divided by sqrt(d) together
 * with Q.K, as Eq. 4 writes it.  No ksize*ksize attention tensor is written
 * to memory: the logits, the softmax and the weighted sum stay on chip.
 *
 * Conventions shared by every entry point:
 *  - q, k, v, out: device memory, [B, heads, H, W, d] contiguous, d fastest.
 *    q, k, v hold `dtype` elements; out is always float32 (a 16-bit output
 *    could not hold the result to the accuracy the fp32 accumulation gives).
 *  - rpb: device memory, float32 [heads, 2*ksize-1, 2*ksize-1], indexed by the
 *    key-minus-query offset (row, then column) plus ksize-1.  rpb == NULL
 *    means no positional bias.
 *  - All pointers must be 16-byte aligned; out must not overlap q, k, v or rpb.
 *  - The caller owns every buffer.  The library allocates nothing, frees
 *    nothing and never synchronises.  Its only state is a process-wide,
 *    mutex-guarded cache of each kernel's occupancy per device (queried on
 *    first use), so concurrent calls from several threads are safe.
 *  - The call is asynchronous on `stream` (a hipStream_t; NULL = the default
 *    stream).  Arguments are checked on the host before anything is
 *    launched: an invalid call returns a negative status and launches
 *    nothing.  A failed launch returns NA2D_ERR_HIP; na2d_last_error() then
 *    gives the HIP error text for the calling thread.
 *  - Non-finite inputs propagate; they are not checked.
 */
#ifndef NA2D_H
#define NA2D_H

#ifdef __cplusplus
extern "C" {
#endif

/* Element type of q, k and v. */
typedef enum {
    NA2D_F32 = 0,
    NA2D_F16 = 1,
    NA2D_BF16 = 2
} na2d_dtype;

/* Kernel family.  AUTO picks MFMA for 16-bit inputs with d = 32 and
 * 3 <= ksize <= NA2D_MFMA_MAX_KSIZE, the VALU kernel otherwise. */
typedef enum {
    NA2D_ALGO_AUTO = 0,
    NA2D_ALGO_VALU = 1, /* one query per lane, fp32 arithmetic, any dtype       */
    NA2D_ALGO_MFMA = 2  /* query tile x key/value halo in LDS, matrix cores      */
} na2d_algo;

/* Window modes of na_forward_nd. */
typedef enum {
    NA_WINDOW_NA = 0,  /* Neighborhood Attention: the k nearest positions per axis, the
                          window clamped inside the grid (start clamp(i - k/2, 0, L - k)) */
    NA_WINDOW_SASA = 1 /* SASA: the window centred on the query (start i - k/2) over the
                          input zero-padded by k/2: a position outside the grid is a zero
                          key and a zero value, so its logit is bias / sqrt(d) and it
                          takes part in the softmax but adds nothing to the output */
} na_window;

/* Status codes (0 = success). */
enum {
    NA2D_OK = 0,
    NA2D_ERR_NULL = -1,        /* q, k, v or out is NULL                                  */
    NA2D_ERR_SHAPE = -2,       /* B, heads, H, W or d <= 0, or an element count overflows */
    NA2D_ERR_KSIZE = -3,       /* ksize even, < 1, > H or > W                              */
    NA2D_ERR_DTYPE = -4,       /* dtype not one of na2d_dtype                              */
    NA2D_ERR_UNSUPPORTED = -5, /* d or ksize outside what the chosen kernel supports       */
    NA2D_ERR_ALIGN = -6,       /* a pointer is not 16-byte aligned                         */
    NA2D_ERR_ALIAS = -7,       /* out overlaps q, k, v or rpb                              */
    NA2D_ERR_HIP = -8,         /* the HIP runtime reported an error at launch              */
    NA2D_ERR_ALGO = -9,        /* algo not one of na2d_algo                                */
    NA2D_ERR_SCRATCH = -10     /* na2d_backward_noalloc: the problem needs more workspace
                                  than NA2D_NOALLOC_SCRATCH_BYTES                          */
};

/* Largest ksize each kernel family accepts.  d must be 16, 32, 64 or 128 for
 * the VALU kernel and 32 for the MFMA kernel. */
#define NA2D_VALU_MAX_KSIZE 63
#define NA2D_MFMA_MAX_KSIZE 25
/* Largest window of the NA1D matrix-core kernel (d = 32, 16-bit inputs). */
#define NA1D_MFMA_MAX_KSIZE 63
/* Largest window per axis of the streaming matrix-core kernel for 3D windows
 * (d = 32, 16-bit inputs, NA); its 2D windows (kd = 1) go up to
 * NA2D_MFMA_MAX_KSIZE. */
#define NA3D_MFMA_MAX_KSIZE 9
/* Largest window whose backward runs on the matrix cores (d = 32, 16-bit
 * inputs); larger windows, fp32 and other head dims use the VALU kernels. */
#define NA2D_BWD_MFMA_MAX_KSIZE 25

/* Fused NA2D forward (CSDN page, section 3.1, Eq. 2-4), kernel chosen
 * automatically.  Sizes are element counts; see the conventions above. */
int na2d_forward(const void *q, const void *k, const void *v, const float *rpb, float *out,
                 int B, int heads, int H, int W, int d, int ksize, int dtype, void *stream);

/* na2d_forward that also writes, per query, the natural log of the softmax
 * denominator: lse = ln sum_j exp((q.k_j + B_j) / sqrt(d)) over the window
 * ([B, heads, H, W] float32, 16-byte aligned, overlapping nothing else;
 * NULL is NA2D_ERR_NULL).  The training forward: na2d_backward reuses it. */
int na2d_forward_lse(const void *q, const void *k, const void *v, const float *rpb, float *out,
                     float *lse, int B, int heads, int H, int W, int d, int ksize, int dtype,
                     void *stream);

/* The same operation with the kernel family forced by `algo` (na2d_algo).
 * NA2D_ERR_UNSUPPORTED if that family cannot run these sizes or dtype. */
int na2d_forward_ex(const void *q, const void *k, const void *v, const float *rpb, float *out,
                    int B, int heads, int H, int W, int d, int ksize, int dtype, int algo,
                    void *stream);

/* Host-only argument check: the status na2d_forward_ex would return for these
 * arguments before launching, with no HIP call made.  Pointers are only
 * compared, never dereferenced. */
int na2d_check_args(const void *q, const void *k, const void *v, const float *rpb,
                    const float *out, int B, int heads, int H, int W, int d, int ksize,
                    int dtype, int algo);

/* The kernel family AUTO resolves to for these sizes (NA2D_ALGO_VALU or
 * NA2D_ALGO_MFMA), or a negative status if the sizes are invalid. */
int na2d_select_algo(int H, int W, int d, int ksize, int dtype);

/* ------------------------------------------------------------------------
 * Neighborhood Attention over one, two or three axes, and SASA windows.
 *
 * The same Eq. 2-4 on a [B, heads, D, H, W] grid of queries (2D: D = 1;
 * 1D: D = H = 1), with a kd x kh x kw window per query.  NATTEN handles 1D
 * and 2D data (CSDN page, section 3.2) and later 1D to 3D (qiita article,
 * section "NATTEN").  SASA is NA run on an input zero-padded by k/2 (CSDN
 * page, section 3.1 after Eq. 4, and section 3.2); mode NA_WINDOW_SASA
 * computes exactly that without materialising the padding.
 *
 *  - q, k, v, out: [B, heads, D, H, W, d] contiguous, d fastest; out float32.
 *  - rpb: float32 [heads, 2kd-1, 2kh-1, 2kw-1], indexed on every axis by key
 *    position minus query position plus (window - 1); NULL = no bias.
 *  - Windows are odd and >= 1.  NA_WINDOW_NA needs each window <= its axis
 *    length (NA2D_ERR_KSIZE otherwise); SASA windows may exceed the axis.
 *    Windows are at most NA2D_VALU_MAX_KSIZE per axis.
 *  - The other conventions (alignment, aliasing, ownership, streams, errors)
 *    are those of na2d_forward.  A call with D = 1, kd = 1, kh = kw and mode
 *    NA_WINDOW_NA is na2d_forward_ex.
 * ------------------------------------------------------------------------ */

/* General form.  `mode` is an na_window, `algo` an na2d_algo.  The MFMA
 * kernels serve 16-bit inputs with d = 32 in three shapes: square 2D windows
 * (D = 1, kd = 1, kh = kw, 3 <= kh <= NA2D_MFMA_MAX_KSIZE), NA or SASA;
 * NA1D (D = H = 1, kd = kh = 1, 3 <= kw <= NA1D_MFMA_MAX_KSIZE, NA); and any
 * other NA window: 3D windows with every axis at most NA3D_MFMA_MAX_KSIZE,
 * 2D windows (rectangular, or square and wider than 13) up to
 * NA2D_MFMA_MAX_KSIZE.  AUTO picks them wherever they apply. */
int na_forward_nd(const void *q, const void *k, const void *v, const float *rpb, float *out,
                  int B, int heads, int D, int H, int W, int d, int kd, int kh, int kw,
                  int mode, int dtype, int algo, void *stream);

/* The kernel family AUTO resolves to for na_forward_nd with these sizes,
 * windows and mode (NA2D_ALGO_VALU or NA2D_ALGO_MFMA), or a negative status
 * if they are invalid. */
int na_select_algo_nd(int D, int H, int W, int d, int kd, int kh, int kw, int mode, int dtype);

/* Host-only check of na_forward_nd's arguments (no HIP call). */
int na_check_args_nd(const void *q, const void *k, const void *v, const float *rpb,
                     const float *out, int B, int heads, int D, int H, int W, int d, int kd,
                     int kh, int kw, int mode, int dtype, int algo);

/* NA1D over a sequence: q, k, v, out [B, heads, L, d]; rpb [heads, 2k-1]
 * indexed by key minus query plus k-1; window start clamp(i - k/2, 0, L - k). */
int na1d_forward(const void *q, const void *k, const void *v, const float *rpb, float *out,
                 int B, int heads, int L, int d, int ksize, int dtype, void *stream);

/* NA3D over a volume: q, k, v, out [B, heads, D, H, W, d]; rpb
 * [heads, 2k-1, 2k-1, 2k-1] (depth, row, column offsets); a k x k x k window
 * clamped per axis. */
int na3d_forward(const void *q, const void *k, const void *v, const float *rpb, float *out,
                 int B, int heads, int D, int H, int W, int d, int ksize, int dtype,
                 void *stream);

/* SASA on a 2D map: na2d_forward's layouts, but the k x k window is centred
 * on the query over the zero-padded input (mode NA_WINDOW_SASA). */
int sasa2d_forward(const void *q, const void *k, const void *v, const float *rpb, float *out,
                   int B, int heads, int H, int W, int d, int ksize, int dtype, void *stream);

/* ------------------------------------------------------------------------
 * Gradients of the NA2D forward (the training half; NATTEN computes them
 * for QK+B and AV, qiita article, section "NATTEN").
 *
 * For L with dL/dout = dout, writes dq, dk, dv = dL/dq, dL/dk, dL/dv
 * ([B, heads, H, W, d] float32, overwritten) and, when rpb is not NULL,
 * drpb = dL/drpb ([heads, 2k-1, 2k-1] float32, overwritten; it must be NULL
 * when rpb is).  q, k, v, rpb, ksize and dtype are those of the forward call;
 * out is its float32 output and dout is float32 [B, heads, H, W, d].  lse is
 * the per-query log-sum-exp that na2d_forward_lse wrote in the same forward
 * call ([B, heads, H, W] float32), or NULL: with it the backward reuses the
 * forward's softmax statistics instead of recomputing them.
 *
 * `workspace` is caller-owned device memory of na2d_backward_workspace_bytes
 * bytes (16-byte aligned, contents ignored on entry): the first kernel leaves
 * each query's softmax statistics there for the second (8 bytes per query),
 * so no k*k attention tensor is stored, followed by per-tile partial sums of
 * the bias gradient ((2k-1)^2 floats per 8 x 8 query tile).  d must be 16,
 * 32, 64 or 128 and ksize <= NA2D_VALU_MAX_KSIZE.  The gradient of the bias
 * table is summed with float atomics, so its last bits may differ from call
 * to call; everything else is deterministic.
 * No output may overlap an input or another output.  Other conventions as
 * for na2d_forward.
 * ------------------------------------------------------------------------ */
int na2d_backward(const void *q, const void *k, const void *v, const float *rpb,
                  const float *out, const float *lse, const float *dout, float *dq, float *dk,
                  float *dv, float *drpb, void *workspace, int B, int heads, int H, int W, int d,
                  int ksize, int dtype, void *stream);

/* The kernels na2d_backward runs for these sizes (NA2D_ALGO_MFMA: both
 * passes on the matrix cores, for 16-bit inputs, d = 32, ksize <=
 * NA2D_BWD_MFMA_MAX_KSIZE and H * W * 128 < 2^31; NA2D_ALGO_VALU otherwise),
 * or a negative status if the sizes are invalid.  Host only. */
int na2d_backward_select_algo(int H, int W, int d, int ksize, int dtype);

/* Bytes of workspace na2d_backward needs for these sizes and window (0 if
 * they are invalid). */
long long na2d_backward_workspace_bytes(int B, int heads, int H, int W, int ksize);

/* Size of the fixed device array that na2d_backward_noalloc uses as its
 * workspace (64 MiB: NAT-Tiny stage 1 needs 3.7 MB, a 448 x 448 map with four
 * heads 15 MB, eight 128 x 128 maps of four heads at k = 21 59 MB). */
#define NA2D_NOALLOC_SCRATCH_BYTES (64ull << 20)

/* na2d_backward for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * The arguments and results are those of na2d_backward without `workspace`:
 * the workspace is a fixed array of NA2D_NOALLOC_SCRATCH_BYTES in device
 * memory that the library holds on each GPU it runs on until the process
 * ends (its address is looked up on the first call on a device).  The call
 * allocates nothing and calls no allocating routine.  Problems whose
 * workspace (na2d_backward_workspace_bytes) exceeds that size are rejected
 * with NA2D_ERR_SCRATCH before anything is launched.  Every call on one GPU
 * shares that GPU's array and leaves it holding its last contents (nothing
 * in it needs clearing: each call writes every byte it reads), so calls that
 * overlap on one GPU -- on different streams, or from different threads
 * without ordering -- race and give wrong gradients; order them. */
int na2d_backward_noalloc(const void *q, const void *k, const void *v, const float *rpb,
                          const float *out, const float *lse, const float *dout, float *dq,
                          float *dk, float *dv, float *drpb, int B, int heads, int H, int W,
                          int d, int ksize, int dtype, void *stream);

/* Host-only check of na2d_backward's arguments (no HIP call). */
int na2d_backward_check_args(const void *q, const void *k, const void *v, const float *rpb,
                             const float *out, const float *lse, const float *dout,
                             const float *dq, const float *dk, const float *dv,
                             const float *drpb, const void *workspace, int B, int heads, int H,
                             int W, int d, int ksize, int dtype);

/* A memory-rate reference, not part of the attention: reads `elems` fp16
 * values from each of a, b and c and writes out[i] = a[i] + b[i] + c[i] in
 * float32 -- the bytes a fused forward with 16-bit inputs moves for `elems`
 * input elements per tensor, read and written once each, with no attention
 * work.  Pointers are device memory, 16-byte aligned; elems > 0 and a
 * multiple of 8.  Asynchronous on `stream`.  Returns NA2D_OK, or
 * NA2D_ERR_NULL / NA2D_ERR_SHAPE / NA2D_ERR_ALIGN before launching, or
 * NA2D_ERR_HIP. */
int na_stream_reference(const void *a, const void *b, const void *c, float *out, long long elems,
                        void *stream);

/* Static text for a status code. */
const char *na2d_strerror(int status);

/* Detail of the last NA2D_ERR_HIP on the calling thread ("" if none). */
const char *na2d_last_error(void);

/* Library version, major * 10000 + minor * 100 + patch. */
int na2d_version(void);

/* Diagnostic: occupancy queries the library has made in this process.  Each
 * kernel is queried once per device and LDS size, on its first launch; a
 * repeated call with the same sizes adds none. */
long long na2d_occupancy_queries(void);

#ifdef __cplusplus
}
#endif

#endif /* NA2D_H */
