/*
 * msda.h - C ABI of the multi-scale deformable attention sampling core on
 * AMD Instinct MI355X (gfx950).
 *
 * The operation (page "Deformable DETR", section "Multi-scale deformable
 * attention", equation MSDeformAttn, the part between the value projection
 * W'_m and the output projection W_m): for every image n, query q and head m,
 *
 *   out[n,q,m,:] = sum_{l<L} sum_{k<K} attn[n,q,m,l,k] *
 *                  bilinear(value[n, level l, m, :], loc[n,q,m,l,k,:])
 *
 * where bilinear() reads the four pixels around a fractional location (same
 * page, section "Deformable attention module"). Conventions the pages leave
 * open and this library fixes:
 *   - loc is normalised: (0,0) and (1,1) are the outer corners of the image,
 *     loc[...,0] is x (width), loc[...,1] is y (height). The pixel-index
 *     coordinate is x = fmaf(loc_x, W_l, -0.5f), y = fmaf(loc_y, H_l, -0.5f),
 *     so pixel j's centre is at (j+0.5)/W_l.
 *   - zero padding: a corner outside the map reads 0; a sample contributes
 *     only if -1 <= x < W_l and -1 <= y < H_l. A NaN or infinite coordinate
 *     never does: that sample adds nothing and gets zero grad_loc and grad_attn.
 *   - at integer x or y the location gradient is the right-derivative
 *     (x0 = floor(x) everywhere).
 *   - pixel (i, j) of level l is row level_start[l] + i*W_l + j of value.
 *   - attn is applied as given (no softmax, no renormalisation inside).
 *
 * Layouts (dense, row-major, as shaped; device arrays aligned to their element
 * size, loc and grad_loc to 8 bytes since they hold (x, y) pairs):
 *   value          [N, S, M, D]          dtype         device
 *   spatial_shapes [L][2] = (H_l, W_l)   int64         HOST, read during the call
 *   level_start    [L]                   int64         HOST, read during the call
 *   loc            [N, Lq, M, L, K, 2]   float32       device
 *   attn           [N, Lq, M, L, K]      float32       device
 *   out, grad_out  [N, Lq, M, D]         dtype         device
 *   grad_value     [N, S, M, D]          float32       device
 *   grad_loc       [N, Lq, M, L, K, 2]   float32       device
 *   grad_attn      [N, Lq, M, L, K]      float32       device
 *
 * Ownership: the caller owns every buffer. The library allocates nothing,
 * keeps no state and holds no pointer after returning; calls are re-entrant.
 * Outputs must not alias inputs or each other.
 *
 * Asynchrony: work is enqueued on `stream` (0 = the null stream) and the call
 * returns; nothing synchronises. A fault inside a kernel surfaces at the
 * caller's next synchronisation.
 *
 * Errors: every call returns a status and never aborts, throws or prints.
 * All argument checks run before any HIP call, so a status other than
 * MSDA_SUCCESS or MSDA_ERROR_LAUNCH means nothing was enqueued.
 */
#ifndef MSDA_H_
#define MSDA_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum msda_status {
  MSDA_SUCCESS = 0,
  MSDA_ERROR_INVALID_VALUE = 1, /* null pointer, negative or zero size, level outside S */
  MSDA_ERROR_NOT_SUPPORTED = 2, /* L > 16, K > 16, D > 1024, oversized map, unknown dtype */
  MSDA_ERROR_MISALIGNED = 3,    /* a device pointer not aligned to its element size */
  MSDA_ERROR_LAUNCH = 4,        /* a kernel launch failed (HIP error after enqueue) */
  MSDA_ERROR_WORKSPACE = 5,     /* backward workspace missing or too small */
  MSDA_ERROR_SCRATCH = 6        /* problem too large for the static scratch of msda_backward_static */
} msda_status;

typedef enum msda_dtype {
  MSDA_F32 = 0,  /* value / out / grad_out in float32 */
  MSDA_BF16 = 1  /* value / out / grad_out in bfloat16; arithmetic in float32 */
} msda_dtype;

/* Limits of the library. */
#define MSDA_MAX_LEVELS 16
#define MSDA_MAX_POINTS 16
#define MSDA_MAX_CHANNELS 1024

/*
 * Host-only argument check shared by the entry points (no HIP call, usable
 * without a GPU). Sizes: N, Lq >= 0 (zero is a no-op); S, M, D, L, K >= 1.
 * Per level: H_l, W_l >= 1, level_start[l] >= 0 and
 * level_start[l] + H_l*W_l <= S; the levels' row ranges must not overlap
 * (MSDA_ERROR_INVALID_VALUE otherwise) but may leave gaps.
 * Returns MSDA_ERROR_NOT_SUPPORTED for L > 16, K > 16, D > 1024, H_l or W_l
 * >= 2^24, S*M*D or Lq*M*D above 2^28 - 1 elements, Lq*M*L*K above 2^29,
 * or a dtype other than MSDA_F32 / MSDA_BF16.
 */
msda_status msda_validate(const int64_t *spatial_shapes, const int64_t *level_start,
                          int64_t N, int64_t S, int64_t M, int64_t D, int64_t L, int64_t Lq,
                          int64_t K, int dtype);

/*
 * Forward sampling (page "Deformable DETR", section "Multi-scale deformable
 * attention", equation MSDeformAttn inside W_m). Writes every element of out
 * (overwritten, not accumulated). Accumulation is float32 in a fixed order, so
 * repeated calls give bitwise-identical results. With dtype MSDA_BF16, value
 * and out are bfloat16: values are widened exactly and the float32 sum is
 * rounded once to nearest-even on store.
 */
msda_status msda_forward(const void *value, const int64_t *spatial_shapes,
                         const int64_t *level_start, const float *loc, const float *attn,
                         void *out, int64_t N, int64_t S, int64_t M, int64_t D, int64_t L,
                         int64_t Lq, int64_t K, int dtype, hipStream_t stream);

/*
 * Bytes of device workspace msda_backward needs for these sizes (the same
 * checks as msda_validate apply). The workspace holds a counting sort of the
 * samples by the 8x8-pixel tile of the value map they touch: a few counters
 * per tile plus up to four 16-byte entries per sample, about 64*N*Lq*M*L*K
 * bytes.
 */
msda_status msda_backward_workspace_size(const int64_t *spatial_shapes, const int64_t *level_start,
                                         int64_t N, int64_t S, int64_t M, int64_t D, int64_t L,
                                         int64_t Lq, int64_t K, int dtype, size_t *bytes);

/*
 * Backward of msda_forward: gradients of sum(grad_out * out) with respect to
 * value, loc and attn (page "Deformable Attention": the bilinear sampling is
 * differentiable, so gradients reach the sampling offsets; out is linear in
 * attn and in value).
 *   grad_attn[n,q,m,l,k] = <grad_out[n,q,m,:], bilinear sample>
 *   grad_loc [n,q,m,l,k,0] = attn * W_l * <grad_out, d sample / d x>
 *   grad_loc [n,q,m,l,k,1] = attn * H_l * <grad_out, d sample / d y>
 *   grad_value[n, corner row, m, :] += attn * corner weight * grad_out
 * All three outputs are float32 and overwritten (every grad_value row is
 * written, including rows no sample touches). dtype applies to value and
 * grad_out. `workspace` is device memory of at least the size
 * msda_backward_workspace_size reports, 256-byte aligned, owned by the caller
 * and used only while the enqueued work runs (calls that overlap on different
 * streams need separate workspaces); MSDA_ERROR_WORKSPACE if it is missing or
 * too small. grad_loc and grad_attn are deterministic; grad_value sums each
 * pixel's contributions in float32 in an order that can vary between calls.
 */
msda_status msda_backward(const void *value, const int64_t *spatial_shapes,
                          const int64_t *level_start, const float *loc, const float *attn,
                          const void *grad_out, float *grad_value, float *grad_loc,
                          float *grad_attn, int64_t N, int64_t S, int64_t M, int64_t D,
                          int64_t L, int64_t Lq, int64_t K, int dtype, void *workspace,
                          size_t workspace_bytes, hipStream_t stream);

/*
 * msda_backward for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Same arguments, results, determinism and asynchrony as msda_backward, with
 * no workspace argument: the workspace is a static device array of
 * MSDA_STATIC_SCRATCH_BYTES that the library holds on each GPU it runs on
 * until the process ends (its address is looked up once per device, on the
 * first call with that device current). The call allocates and frees
 * nothing. A problem whose msda_backward_workspace_size exceeds
 * MSDA_STATIC_SCRATCH_BYTES returns MSDA_ERROR_SCRATCH before any HIP call
 * (decoder-sized problems fit; an encoder-sized one, about 64 bytes per
 * sample, does not). Every call on one GPU shares that GPU's array and the
 * kernels clear what must start at zero, so consecutive calls need nothing
 * from the caller; calls that overlap on one GPU (two streams or two host
 * threads at once) race on the array and must not be issued.
 */
#define MSDA_STATIC_SCRATCH_BYTES ((size_t)64 << 20)

msda_status msda_backward_static(const void *value, const int64_t *spatial_shapes,
                                 const int64_t *level_start, const float *loc, const float *attn,
                                 const void *grad_out, float *grad_value, float *grad_loc,
                                 float *grad_attn, int64_t N, int64_t S, int64_t M, int64_t D,
                                 int64_t L, int64_t Lq, int64_t K, int dtype, hipStream_t stream);

/*
 * The sampling core with the step in front of it done inside the kernels
 * (page "Deformable DETR", section "Deformable attention module": the
 * sampling offsets and the attention logits are one linear projection of the
 * query, and the logits go through a softmax; section "Multi-scale deformable
 * attention": the softmax is taken jointly over the L*K samples of a head and
 * a sample sits at the reference point plus an offset in pixels of level l;
 * section "Variants", iterative bounding box refinement: with a box as the
 * reference, the offsets are scaled by the box's width and height). Computes
 * msda_forward(value, loc, attn) with
 *   attn[n,q,m,l,k] = softmax over (l, k) of logits[n,q,m,:,:]
 *   ref_dim == 2 (reference points, normalised (x, y)):
 *     loc[...,l,k,0] = ref[n,q,0] + offsets[...,l,k,0] / W_l
 *     loc[...,l,k,1] = ref[n,q,1] + offsets[...,l,k,1] / H_l
 *     (binary32: the quotient and the sum are each rounded once)
 *   ref_dim == 4 (boxes (cx, cy, w, h), normalised):
 *     loc[...,l,k,0] = fmaf(offsets[...,l,k,0], w, cx)
 *     loc[...,l,k,1] = fmaf(offsets[...,l,k,1], h, cy)
 * Layouts: ref [N, Lq, ref_dim] float32, device, 8-byte aligned; offsets
 * [N, Lq, M, L, K, 2] float32 (8-byte aligned); logits [N, Lq, M, L, K]
 * float32; value and out as for msda_forward. The softmax is evaluated in
 * float32 as exp(z - max) / sum; a NaN or infinite logit makes its head's
 * weights NaN. ref_dim other than 2 or 4: MSDA_ERROR_INVALID_VALUE. Other
 * errors, ownership and asynchrony as for msda_forward.
 */
msda_status msda_fused_forward(const void *value, const int64_t *spatial_shapes,
                               const int64_t *level_start, const float *ref, int ref_dim,
                               const float *offsets, const float *logits, void *out, int64_t N,
                               int64_t S, int64_t M, int64_t D, int64_t L, int64_t Lq, int64_t K,
                               int dtype, hipStream_t stream);

/*
 * Backward of msda_fused_forward, by the chain rule through the softmax and
 * the location formula (the rounding of the location is taken to have
 * derivative 1). With grad_attn and grad_loc as msda_backward defines them:
 *   grad_logits[i]  = attn[i] * (grad_attn[i] - sum_j attn[j] * grad_attn[j])
 *                     (j over the L*K samples of the same (n, q, m))
 *   grad_offsets    = grad_loc / (W_l, H_l)             (ref_dim 2)
 *                   = grad_loc * (w, h)                 (ref_dim 4)
 *   grad_ref[n,q,:] = sum over (m, l, k) of grad_loc    (ref_dim 2)
 *                   = [sum grad_loc, sum grad_loc * offsets]  (ref_dim 4:
 *                     d/d(cx, cy), then d/d(w, h))
 * A sample outside the map has zero grad_loc and no term in these sums, so a
 * NaN or infinite offset (which puts its sample outside) leaves every result
 * finite; its weight still takes part in its head's softmax.
 * grad_value [N,S,M,D], grad_offsets [N,Lq,M,L,K,2] (8-byte aligned),
 * grad_logits [N,Lq,M,L,K] and grad_ref [N,Lq,ref_dim] are float32 and
 * overwritten. grad_ref may be NULL (then it is not computed: reference
 * points are often detached between layers). The workspace must hold
 * msda_fused_backward_workspace_size bytes; determinism (all but grad_value
 * are deterministic), errors and asynchrony as for msda_backward.
 */
/*
 * Bytes of device workspace msda_fused_backward needs: the above plus 12 bytes
 * per sample (the locations and weights formed from the raw predictions) and
 * 16 bytes per (image, query, head) (reference-gradient partial sums).
 */
msda_status msda_fused_backward_workspace_size(const int64_t *spatial_shapes,
                                               const int64_t *level_start, int64_t N, int64_t S,
                                               int64_t M, int64_t D, int64_t L, int64_t Lq, int64_t K,
                                               int dtype, size_t *bytes);

msda_status msda_fused_backward(const void *value, const int64_t *spatial_shapes,
                                const int64_t *level_start, const float *ref, int ref_dim,
                                const float *offsets, const float *logits, const void *grad_out,
                                float *grad_value, float *grad_offsets, float *grad_logits,
                                float *grad_ref, int64_t N, int64_t S, int64_t M, int64_t D,
                                int64_t L, int64_t Lq, int64_t K, int dtype, void *workspace,
                                size_t workspace_bytes, hipStream_t stream);

/*
 * Deformable groups (page "Deformable Attention", glossary: heads are gathered
 * into fewer deformable groups that share one set of sampled keys while
 * keeping their own projections). G groups of M/G consecutive heads: group
 * g = m / (M/G) supplies the locations and weights of head m, and each head
 * still reads its own value channels:
 *   out[n,q,m,:] = sum_{l,k} attn[n,q,g,l,k] *
 *                  bilinear(value[n, level l, m, :], loc[n,q,g,l,k,:])
 * Layouts: loc [N, Lq, G, L, K, 2], attn [N, Lq, G, L, K]; value, out,
 * grad_out and grad_value as for msda_forward (M heads of D channels).
 * grad_loc [N, Lq, G, L, K, 2] and grad_attn [N, Lq, G, L, K] sum the
 * per-head gradients over the heads of each group. G must divide M
 * (MSDA_ERROR_INVALID_VALUE otherwise) and (M/G)*D must be within
 * MSDA_MAX_CHANNELS. The heads of a group are consecutive channels of a value
 * or out row, so these calls run the sampling core with G heads of (M/G)*D
 * channels; msda_fused_forward / msda_fused_backward take groups the same way
 * (pass M = G and D = (M/G)*D). Everything else as for msda_forward,
 * msda_backward_workspace_size and msda_backward.
 */
msda_status msda_grouped_forward(const void *value, const int64_t *spatial_shapes,
                                 const int64_t *level_start, const float *loc, const float *attn,
                                 void *out, int64_t N, int64_t S, int64_t M, int64_t D, int64_t L,
                                 int64_t Lq, int64_t K, int64_t G, int dtype, hipStream_t stream);

msda_status msda_grouped_backward_workspace_size(const int64_t *spatial_shapes,
                                                 const int64_t *level_start, int64_t N, int64_t S,
                                                 int64_t M, int64_t D, int64_t L, int64_t Lq,
                                                 int64_t K, int64_t G, int dtype, size_t *bytes);

msda_status msda_grouped_backward(const void *value, const int64_t *spatial_shapes,
                                  const int64_t *level_start, const float *loc, const float *attn,
                                  const void *grad_out, float *grad_value, float *grad_loc,
                                  float *grad_attn, int64_t N, int64_t S, int64_t M, int64_t D,
                                  int64_t L, int64_t Lq, int64_t K, int64_t G, int dtype,
                                  void *workspace, size_t workspace_bytes, hipStream_t stream);

/* Static description of a status code; never NULL. */
const char *msda_status_string(msda_status status);

#ifdef __cplusplus
}
#endif

#endif /* MSDA_H_ */
