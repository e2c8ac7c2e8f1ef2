/* hfa.h -- C ABI of libhfa.so: exact attention forward on AMD MI355X (gfx950).
 *
 * The operation.  For every batch b and head h, with S = Q K^T * scale,
 *
 *     O   = softmax(S) V                    (row softmax over the keys)
 *     LSE = log(sum_j exp(S[:, j]))         (natural log, per query row)
 *
 * i.e. "Attention(Q,K,V) = softmax(QK^T / sqrt(d_k)) V" as defined on the
 * neuralmasteryai page "Hardware Acceleration & Custom Kernels", section 2
 * ("FlashAttention: SRAM Tiling & Online Softmax"), computed the way that
 * section describes: Q, K and V are cut into row tiles that live on chip, and
 * the softmax is taken by the online normalisation identity (running max and
 * running denominator, with the running output sums rescaled as each key tile
 * arrives), so the N x N score matrix is never written to memory.  The
 * TritonForge page ("Tiled FlashAttention-2" card) states the same property:
 * O(N) memory, no N x N matrix materialised.  The log-sum-exp output is not on
 * the pages; it is the running max plus the log of the running denominator.
 *
 * Precision.  HFA_F32: fp32 in and out.  Q K^T is formed from exact int8
 * slices of each row of Q and K (five slices under a power of two 2^e above
 * the row's largest magnitude) on the int8 matrix cores, accumulated exactly
 * and combined in fp64.  The score error of that route is bounded per pair of
 * rows by |scale| (2^-35 (2^e_k A_q + 2^e_q A_k) + d 2^-40 2^(e_q + e_k)),
 * A = sum_c |x_c| of the row; each workgroup evaluates this bound for every
 * key against its own query rows, and if any key exceeds 2^-22 (rows that mix
 * magnitudes far apart, e.g. outlier channels) the workgroup recomputes its
 * rows with both products on the fp64 matrix cores instead (exact products,
 * fp64 sums), so the int8 route serves only where it is within 2^-22.
 * P V runs on the bf16 matrix cores from exact three-piece bf16 splits of P
 * and V (six of the nine piece products; each dropped one is below 2^-21 of
 * its |p v| term) with fp32 accumulation; exp2 runs in fp32 and the
 * denominator and log-sum-exp are combined in fp64.  HFA_BF16: bf16 in and out, matrix
 * products on bf16 matrix cores with fp32 accumulation, softmax in fp32,
 * P rounded to bf16 (round-to-nearest-even) for P V, O rounded to bf16 once.
 *
 * Input domain.  Q, K, V and scale are finite (NaN or infinite entries give
 * unspecified results).  HFA_BF16 accumulates scores in fp32, so every
 * |scale q.k| must stay within the fp32 range (about 3.4e38).  HFA_F32 forms
 * scores in fp64 and has no such limit; only an LSE whose value exceeds the
 * fp32 range is returned as +inf.
 *
 * Ownership.  The caller owns every buffer; hfa_attn_fwd allocates nothing,
 * keeps no state between calls and never holds an N x N buffer.  All pointers
 * passed to it are device pointers on the current HIP device.  The graph
 * functions at the end create host-side driver objects owned by the returned
 * handle.
 *
 * Errors.  Every argument is validated before any HIP call is made; on a
 * validation error the call returns the status and leaves o and lse
 * untouched.  The launch is asynchronous on `stream`: HFA_OK means the work
 * was enqueued; faults during execution surface at the caller's next
 * synchronisation.  The functions are thread-safe.
 */
#ifndef HFA_H
#define HFA_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* In both enums the two *_RANGE_ entries are not values to pass: they make
 * every 32-bit int a valid value of the type, so that an unknown code passed
 * from C (or any foreign-function caller) is rejected with a status instead
 * of being undefined behaviour in the C++ implementation. */
typedef enum {
  HFA_F32 = 0,  /* fp32 (4-byte IEEE binary32) elements */
  HFA_BF16 = 1, /* bf16 (2-byte, upper half of binary32) elements */
  HFA_DTYPE_RANGE_MIN_ = -2147483647 - 1,
  HFA_DTYPE_RANGE_MAX_ = 2147483647
} hfa_dtype;

typedef enum {
  HFA_OK = 0,
  HFA_ERR_NULL = 1,        /* a required pointer is NULL */
  HFA_ERR_SHAPE = 2,       /* B, H or N < 1, or the problem exceeds the index limits */
  HFA_ERR_UNSUPPORTED = 3, /* head dim d not in {64, 128}, or dtype unknown */
  HFA_ERR_SCALE = 4,       /* scale is NaN or infinite */
  HFA_ERR_ALIGN = 5,       /* q, k, v, o not 16-byte aligned, or lse not 4-byte aligned */
  HFA_ERR_ALIAS = 6,       /* o or lse overlaps q, k, v or each other */
  HFA_ERR_NO_DEVICE = 7,   /* no HIP device is current, or it is not gfx950 */
  HFA_ERR_LAUNCH = 8,      /* the kernel launch itself failed */
  HFA_ERR_EPS = 9,         /* hfa_rmsnorm: eps is not a finite value > 0 */
  HFA_ERR_WORKSPACE = 10,  /* hfa_attn_fwd_split: workspace_bytes below what the split needs */
  HFA_STATUS_RANGE_MIN_ = -2147483647 - 1,
  HFA_STATUS_RANGE_MAX_ = 2147483647
} hfa_status;

/* Attention forward.
 *
 *   q, k, v  device, [B, H, N, d] contiguous row-major, element type `dtype`.
 *            Read only; may alias each other.
 *   o        device, [B, H, N, d] contiguous, element type `dtype`. Written once.
 *   lse      device, [B, H, N] contiguous fp32, natural-log log-sum-exp of the
 *            scaled scores of each query row.  Written once.
 *   B, H, N  batch, heads, sequence length: each >= 1, N * d < 2^31.
 *   d        head dimension: 64 or 128.
 *   scale    multiplier of Q K^T (1/sqrt(d) for the usual attention); any finite
 *            value, 0 included.
 *   dtype    HFA_F32 or HFA_BF16, for q, k, v and o alike.
 *   stream   a hipStream_t, passed as a pointer; NULL selects the null stream.
 *
 * Returns HFA_OK or one of the error codes above. */
hfa_status hfa_attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                        int64_t B, int64_t H, int64_t N, int64_t d, float scale,
                        hfa_dtype dtype, void* stream);

/* Static, NUL-terminated description of a status code (never NULL). */
const char* hfa_status_str(hfa_status s);

/* Query rows owned by one workgroup of the kernel hfa_attn_fwd selects for
 * this shape, i.e. the row-tile height B_r of its tiling (bf16: 256 rows, or
 * 128 where at most 128 workgroups of 256 rows would run, at d = 64, and at
 * d = 128 with N <= 4096; a key split of hfa_attn_fwd_split keeps 256;
 * fp32, d = 64: 256, 128 or 64 rows, whichever needs the fewest rounds of
 * workgroups over the 256 compute units of a gfx950 weighted by its measured
 * time per row; fp32, d = 128: 128 rows when B*H*ceil(N/128) workgroups cover
 * the compute units, else 64); 0 for an unsupported dtype or
 * head dim or a shape with B, H or N below 1.  Needs no device and makes no
 * HIP call. */
int64_t hfa_block_rows(hfa_dtype dtype, int64_t B, int64_t H, int64_t N, int64_t d);

/* Key split for shapes with few query tiles.  When B * H * ceil(N / B_r)
 * row tiles give fewer workgroups than the GPU has compute units, the keys of
 * each head can be cut into `splits` contiguous ranges (whole 64-key tiles),
 * one workgroup per (row tile, range): each range runs the same online
 * normalisation over its keys and leaves a partial result (its normalised
 * output O_s and log-sum-exp L_s, fp32) in the caller's workspace, and a
 * second kernel merges the ranges with the identity of the running update of
 * neuralmasteryai "Hardware Acceleration & Custom Kernels", section 2, step 2,
 * applied to whole ranges: with M = max_s L_s and w_s = exp(L_s - M),
 * O = sum_s w_s O_s / sum_s w_s and LSE = M + log sum_s w_s.  bf16 only.
 *
 * hfa_key_splits: the split hfa_attn_fwd_split takes for splits == 0 (1: none;
 * always 1 for HFA_F32); 0 for invalid arguments.  No device, no HIP call. */
int64_t hfa_key_splits(hfa_dtype dtype, int64_t B, int64_t H, int64_t N, int64_t d);

/* Workspace bytes of hfa_attn_fwd_split.
 *
 * HFA_BF16: the bytes `splits` key ranges need (0: the automatic choice); 0
 * when the call splits nothing.  The requested count is clamped to
 * [1, min(ceil(N / 64), 32)] and every range is non-empty, so the ranges
 * actually used may be fewer.
 *
 * HFA_F32 (no key split; splits 0 or 1): the workspace of the packed path, in
 * which a first kernel formats K and V once per call (the int8 slice planes
 * and exponents of K, the bf16 pieces of V and per-tile key statistics,
 * ceil(N / 64) tiles of 57344 bytes per head at d = 64, ceil(N / 32) tiles of
 * 49152 bytes at d = 128) and the attention kernel copies those tiles into LDS
 * as they are, instead of every workgroup formatting every key tile itself.
 * Results are bit for bit those of hfa_attn_fwd.  splits == 0 asks for the
 * library's choice: the workspace where at least 8 workgroups of a head share
 * each key tile and a head has at least 32 key tiles, 0 bytes (no packing)
 * elsewhere, where the packing pass would not pay for itself; splits == 1
 * gives the packed path's size in any case.
 *
 * -1 for invalid arguments (and for splits > 1 with HFA_F32).  No device, no
 * HIP call. */
int64_t hfa_attn_fwd_workspace_size(hfa_dtype dtype, int64_t B, int64_t H, int64_t N, int64_t d,
                                    int64_t splits);

/* hfa_attn_fwd with an optional key split (bf16) or packed K/V (fp32).
 *
 *   q ... dtype, stream  as for hfa_attn_fwd, validated the same way first.
 *   splits           key ranges per head: 0 = hfa_key_splits' choice, 1 = none
 *                    (a bf16 call is then exactly hfa_attn_fwd), > 1 bf16 only
 *                    (HFA_ERR_UNSUPPORTED for HFA_F32); < 0 is HFA_ERR_SHAPE.
 *   workspace        device memory of at least workspace_bytes >=
 *                    hfa_attn_fwd_workspace_size(dtype, B, H, N, d, splits)
 *                    bytes, 16-byte aligned, overlapping no other argument;
 *                    may be NULL when that size is 0.  Its contents on entry
 *                    do not matter; the call leaves the partial results
 *                    (bf16) or the formatted tiles (fp32) there.  HFA_F32: a
 *                    non-NULL workspace selects the packed path (it must then
 *                    hold hfa_attn_fwd_workspace_size(..., 1) bytes); NULL
 *                    runs hfa_attn_fwd.
 *
 * Errors, before any HIP call: those of hfa_attn_fwd, then HFA_ERR_NULL (no
 * workspace), HFA_ERR_ALIGN, HFA_ERR_WORKSPACE (too small), HFA_ERR_ALIAS.
 * Asynchronous on `stream` (two kernels in stream order, or one); the library
 * allocates nothing.  Calls that share a workspace must not overlap in time. */
hfa_status hfa_attn_fwd_split(const void* q, const void* k, const void* v, void* o, float* lse,
                              int64_t B, int64_t H, int64_t N, int64_t d, float scale, hfa_dtype dtype,
                              int64_t splits, void* workspace, int64_t workspace_bytes, void* stream);

/* hfa_attn_fwd_split for callers that cannot allocate device memory: code
 * under stream or graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  Same arguments and results as hfa_attn_fwd_split without the
 * workspace (HFA_F32 calls take hfa_attn_fwd's path, which needs none): the
 * partial results of a bf16 split go to a scratch array inside the library, of
 * 64 MiB, one per GPU (allocated when the library is loaded on that GPU and
 * held until the process ends); the call itself allocates nothing.  A split
 * whose workspace (hfa_attn_fwd_workspace_size) exceeds 64 MiB is rejected
 * with HFA_ERR_WORKSPACE before any HIP call.  Every call on one GPU shares
 * that GPU's array: calls that overlap in time on one GPU (other streams,
 * other threads) race and must be serialised by the caller.  The array needs
 * no clearing; the last call's partial results stay in it. */
hfa_status hfa_attn_fwd_split_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                                      int64_t B, int64_t H, int64_t N, int64_t d, float scale,
                                      hfa_dtype dtype, int64_t splits, void* stream);

/* Graph replay for launch-bound shapes.  Following the "CUDA Graphs" part
 * of section 4 of the neuralmasteryai page "Hardware Acceleration & Custom
 * Kernels" (per-kernel CPU dispatch costs microseconds; a graph captured once
 * is replayed with one driver call), hfa_attn_fwd_graph_create records
 * `count` identical hfa_attn_fwd calls into a HIP graph and instantiates it.
 *
 *   Arguments q ... dtype are those of hfa_attn_fwd and are validated the same
 *   way, with the same status codes, before any HIP call.  The buffers must
 *   stay allocated while the graph exists; every replay rereads q, k, v and
 *   rewrites o and lse.
 *   count  number of launches recorded, 1 <= count <= 2^20 (else HFA_ERR_SHAPE).
 *   out    receives the graph handle (NULL on failure); HFA_ERR_NULL if NULL.
 *
 * The capture runs on a private stream of default priority that is destroyed
 * before returning; the graph holds host-side driver objects only, no device
 * buffers.  HFA_ERR_LAUNCH if a HIP graph call fails.  The graph belongs to
 * the device current at creation. */
typedef struct hfa_graph_s* hfa_graph;
hfa_status hfa_attn_fwd_graph_create(const void* q, const void* k, const void* v, void* o, float* lse,
                                     int64_t B, int64_t H, int64_t N, int64_t d, float scale,
                                     hfa_dtype dtype, int64_t count, hfa_graph* out);

/* Enqueue one replay of the whole graph on `stream` (a hipStream_t of the
 * graph's device; NULL selects the null stream).  HFA_ERR_NULL for a NULL
 * graph, HFA_ERR_LAUNCH if the launch is refused. */
hfa_status hfa_graph_launch(hfa_graph g, void* stream);

/* Release a graph (NULL is ignored).  No replay of it may still be pending:
 * synchronise its streams first. */
void hfa_graph_destroy(hfa_graph g);

/* Row softmax of an fp32 matrix: y[r, :] = exp(x[r, :] - m_r) / sum_j
 * exp(x[r, j] - m_r), m_r = max_j x[r, j].
 *
 * The stable row softmax of the book chapter "Triton and kernel fusion"
 * (section "Fusion": one read of x and one write of y), for any row width:
 * rows wider than one workgroup holds in registers (more than 65536 columns,
 * 49152 without 16-byte alignment) take the route of that chapter's stretch
 * exercise, a running max and running sum per thread (the online
 * normalisation identity of neuralmasteryai "Hardware Acceleration & Custom
 * Kernels", section 2, step 2); their first 143360 (139264) columns stay on
 * chip between the two passes and the rest of x is read a second time to write
 * y.  Arithmetic is fp32 with hardware exp2.
 *
 *   x, y        device, [rows, cols] contiguous fp32, 4-byte aligned (16-byte
 *               alignment with cols % 4 == 0 takes 16-byte accesses).  y may
 *               be x itself (in place) but must not partly overlap it.
 *   rows, cols  >= 1, rows < 2^31, rows * cols * 4 bytes addressable.
 *   stream      a hipStream_t, passed as a pointer; NULL selects the null stream.
 *
 * Finite inputs give finite outputs; -inf entries get weight 0, NaN and +inf
 * propagate.  Validation precedes any HIP call: HFA_ERR_NULL, HFA_ERR_SHAPE,
 * HFA_ERR_ALIGN, HFA_ERR_ALIAS (partial overlap), HFA_ERR_NO_DEVICE, then
 * HFA_ERR_LAUNCH if the launch fails.  Asynchronous on `stream`; allocates
 * nothing. */
hfa_status hfa_softmax_rows(const float* x, float* y, int64_t rows, int64_t cols, void* stream);

/* Fused residual add + RMS normalisation of each row:
 *
 *     s[r, :] = x[r, :] + residual[r, :]     (s = x when residual is NULL)
 *     y[r, :] = s[r, :] / sqrt(sum_j s[r, j]^2 / cols + eps) * weight[:]
 *
 * The normalisation is the TritonForge page's "Fused RMSNorm" card formula
 * (x / sqrt(sum_i x_i^2 / d + eps) scaled elementwise by gamma); the residual
 * form and the second output s are the book chapter "Triton and kernel
 * fusion", section "Fused residual add + RMSNorm" (x and residual read once,
 * y and s written once).  Each row is held in registers by one group of
 * threads, so rows are limited to 65536 columns, the width up to which that
 * chapter's engine takes the fused kernel.
 *
 * Precision: elements are fp32 or bf16 (dtype applies to every array); the
 * sum is one fp32 add of the upcast operands, the mean square, root and
 * products are fp32, and bf16 outputs are rounded once to nearest even.  y is
 * normalised from the fp32 sum, not from its stored (rounded) copy.
 *
 *   x, residual   device, [rows, cols] contiguous; residual may be NULL.
 *   weight        device, [cols] contiguous (gamma).
 *   y             device, [rows, cols]: the normalised rows.
 *   residual_out  device, [rows, cols]: receives s; required when residual is
 *                 given, ignored otherwise.
 *   rows, cols    rows >= 1, rows < 2^31; 1 <= cols <= 65536.
 *   eps           finite and > 0 (1e-6 is the pages' default).
 *   dtype         HFA_F32 or HFA_BF16.
 *   stream        a hipStream_t, passed as a pointer; NULL selects the null stream.
 *
 * Every pointer must be aligned to the element size (16-byte alignment with
 * cols a multiple of 16 bytes takes 16-byte accesses).  y and residual_out may
 * each be exactly x or residual (in place) but must not partly overlap them,
 * and must overlap neither weight nor each other.  Validation precedes any HIP
 * call: HFA_ERR_NULL, HFA_ERR_UNSUPPORTED, HFA_ERR_SHAPE, HFA_ERR_EPS,
 * HFA_ERR_ALIGN, HFA_ERR_ALIAS, HFA_ERR_NO_DEVICE, then HFA_ERR_LAUNCH if the
 * launch fails.  Asynchronous on `stream`; allocates nothing. */
hfa_status hfa_rmsnorm(const void* x, const void* residual, const void* weight, void* y, void* residual_out,
                       int64_t rows, int64_t cols, float eps, hfa_dtype dtype, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* HFA_H */
