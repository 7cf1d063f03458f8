// C-ABI layer of the MSDA sampling core: argument checks, batch splitting and
// kernel dispatch. Every check runs before the first HIP call.
#include "msda.h"

#include <algorithm>

#include "msda_internal.h"

namespace {

bool mul_ok(int64_t a, int64_t b, int64_t *r) { return !__builtin_mul_overflow(a, b, r); }

bool aligned(const void *p, uintptr_t n) { return (reinterpret_cast<uintptr_t>(p) % n) == 0; }

int64_t elem_size(int dtype) { return dtype == MSDA_F32 ? 4 : 2; }

// Images per launch so that the value and grad_out slices of one launch stay
// below the out-of-bounds sentinel of the kernels and its samples keep 32-bit
// indices (with four tile entries per sample).
int64_t images_per_launch(int64_t S, int64_t M, int64_t D, int64_t Lq, int64_t L, int64_t K) {
  const int64_t per_image = std::max(S * M * D, Lq * M * D);
  int64_t n = std::max<int64_t>(1, msda::kMaxSliceElems / per_image);
  const int64_t samples = std::max<int64_t>(1, Lq * M * L * K);
  n = std::min(n, std::max<int64_t>(1, (msda::kMaxSliceSamples / 4) / samples));
  return n;
}

msda::Params base_params(const int64_t *spatial_shapes, const int64_t *level_start, int64_t S,
                         int64_t M, int64_t D, int64_t L, int64_t Lq, int64_t K) {
  msda::Params p{};
  p.S = (int32_t)S;
  p.M = (int32_t)M;
  p.D = (int32_t)D;
  p.L = (int32_t)L;
  p.K = (int32_t)K;
  p.Lq = (int32_t)Lq;
  p.LK = (int32_t)(L * K);
  for (int64_t l = 0; l < L; ++l) {
    p.lv.H[l] = (int32_t)spatial_shapes[2 * l];
    p.lv.W[l] = (int32_t)spatial_shapes[2 * l + 1];
    p.lv.start[l] = (int32_t)level_start[l];
  }
  msda::fill_tiles(p.lv, spatial_shapes, L, &p.TPI);
  return p;
}

bool levels_cover_all_rows(const int64_t *spatial_shapes, int64_t L, int64_t S) {
  int64_t covered = 0;
  for (int64_t l = 0; l < L; ++l) covered += spatial_shapes[2 * l] * spatial_shapes[2 * l + 1];
  return covered == S;  // levels are disjoint (checked), so this means no gap
}

msda_status forward_impl(const void *value, const int64_t *spatial_shapes, const int64_t *level_start,
                         const float *loc, const float *attn, const float *ref, int ref_dim, void *out, int64_t N,
                         int64_t S, int64_t M, int64_t D, int64_t L, int64_t Lq, int64_t K, int dtype,
                         hipStream_t stream) {
  msda_status st = msda_validate(spatial_shapes, level_start, N, S, M, D, L, Lq, K, dtype);
  if (st != MSDA_SUCCESS) return st;
  if (ref_dim != 0 && ref_dim != 2 && ref_dim != 4) return MSDA_ERROR_INVALID_VALUE;
  if (N == 0 || Lq == 0) return MSDA_SUCCESS;
  if (!value || !loc || !attn || !out || (ref_dim && !ref)) return MSDA_ERROR_INVALID_VALUE;
  const int64_t esz = elem_size(dtype);
  if (!aligned(value, esz) || !aligned(out, esz) || !aligned(loc, 8) || !aligned(attn, 4) ||
      (ref_dim && !aligned(ref, 8)))
    return MSDA_ERROR_MISALIGNED;

  const msda::DType dt = dtype == MSDA_F32 ? msda::DType::F32 : msda::DType::BF16;
  const msda::LaunchShape shape = msda::choose_shape(
      (int)D, dt, reinterpret_cast<uintptr_t>(value) | reinterpret_cast<uintptr_t>(out),
      std::min(N, images_per_launch(S, M, D, Lq, L, K)) * Lq * M);
  msda::Params p = base_params(spatial_shapes, level_start, S, M, D, L, Lq, K);
  p.ref_dim = ref_dim;
  const int64_t step = images_per_launch(S, M, D, Lq, L, K);
  for (int64_t n0 = 0; n0 < N; n0 += step) {
    const int64_t nb = std::min(step, N - n0);
    p.N = (int32_t)nb;
    p.pairs = nb * Lq * M;
    p.value_elems = (uint32_t)(nb * S * M * D);
    p.value = static_cast<const char *>(value) + n0 * S * M * D * esz;
    p.loc = loc + n0 * Lq * M * L * K * 2;
    p.attn = attn + n0 * Lq * M * L * K;
    p.ref = ref_dim ? ref + n0 * Lq * ref_dim : nullptr;
    p.out = static_cast<char *>(out) + n0 * Lq * M * D * esz;
    if (msda::launch_forward(p, dt, shape, stream) != hipSuccess) return MSDA_ERROR_LAUNCH;
  }
  return MSDA_SUCCESS;
}

msda_status backward_impl(const void *value, const int64_t *spatial_shapes, const int64_t *level_start,
                          const float *loc, const float *attn, const float *ref, int ref_dim, const void *grad_out,
                          float *grad_value, float *grad_loc, float *grad_attn, float *grad_ref, int64_t N,
                          int64_t S, int64_t M, int64_t D, int64_t L, int64_t Lq, int64_t K, int dtype,
                          void *workspace, size_t workspace_bytes, hipStream_t stream) {
  msda_status st = msda_validate(spatial_shapes, level_start, N, S, M, D, L, Lq, K, dtype);
  if (st != MSDA_SUCCESS) return st;
  if (ref_dim != 0 && ref_dim != 2 && ref_dim != 4) return MSDA_ERROR_INVALID_VALUE;
  if (N == 0) return MSDA_SUCCESS;
  if (!grad_value) return MSDA_ERROR_INVALID_VALUE;
  if (!aligned(grad_value, 4)) return MSDA_ERROR_MISALIGNED;
  const int64_t esz = elem_size(dtype);
  const int64_t step = images_per_launch(S, M, D, Lq, L, K);
  const msda::WorkspaceLayout wl =
      msda::workspace_layout(spatial_shapes, L, std::min(step, N), M, Lq, K, ref_dim != 0);
  if (Lq > 0) {
    if (!value || !loc || !attn || !grad_out || !grad_loc || !grad_attn || (ref_dim && !ref))
      return MSDA_ERROR_INVALID_VALUE;
    if (!aligned(value, esz) || !aligned(grad_out, esz) || !aligned(loc, 8) || !aligned(attn, 4) ||
        !aligned(grad_loc, 8) || !aligned(grad_attn, 4) || (ref_dim && !aligned(ref, 8)) ||
        (grad_ref && !aligned(grad_ref, 4)))
      return MSDA_ERROR_MISALIGNED;
    if (!workspace || workspace_bytes < wl.bytes) return MSDA_ERROR_WORKSPACE;
    if (!aligned(workspace, 256)) return MSDA_ERROR_MISALIGNED;
  }
  // Rows outside every level (or every row when there are no queries) get
  // no tile owner: zero them in full first.
  if (Lq == 0 || !levels_cover_all_rows(spatial_shapes, L, S)) {
    if (msda::launch_zero(grad_value, N * S * M * D, stream) != hipSuccess) return MSDA_ERROR_LAUNCH;
  }
  if (Lq == 0) return MSDA_SUCCESS;

  const msda::DType dt = dtype == MSDA_F32 ? msda::DType::F32 : msda::DType::BF16;
  const msda::LaunchShape shape = msda::choose_shape(
      (int)D, dt, reinterpret_cast<uintptr_t>(value) | reinterpret_cast<uintptr_t>(grad_out),
      std::min(N, step) * Lq * M);
  msda::Params p = base_params(spatial_shapes, level_start, S, M, D, L, Lq, K);
  p.ref_dim = ref_dim;
  char *ws = static_cast<char *>(workspace);
  p.ws.tile_count = reinterpret_cast<uint32_t *>(ws + wl.off_count);
  p.ws.tile_cursor = reinterpret_cast<uint32_t *>(ws + wl.off_cursor);
  p.ws.tile_start = reinterpret_cast<uint32_t *>(ws + wl.off_start);
  p.ws.work_item = reinterpret_cast<uint32_t *>(ws + wl.off_witem);
  p.ws.n_work = reinterpret_cast<uint32_t *>(ws + wl.off_nwork);
  p.ws.split_list = reinterpret_cast<uint32_t *>(ws + wl.off_split);
  p.ws.entries = reinterpret_cast<uint32_t *>(ws + wl.off_entries);
  {
    const uint64_t eb = 16 * (uint64_t)wl.Emax;  // the region the scatter pass writes
    p.ws.entries_bytes = eb <= msda::kEntriesOob ? (uint32_t)eb : 0u;
  }
  p.ws.ref_part = reinterpret_cast<float *>(ws + wl.off_refpart);
  p.ws.floc = reinterpret_cast<float *>(ws + wl.off_floc);
  p.ws.fattn = reinterpret_cast<float *>(ws + wl.off_fattn);
  for (int64_t n0 = 0; n0 < N; n0 += step) {
    const int64_t nb = std::min(step, N - n0);
    p.N = (int32_t)nb;
    p.pairs = nb * Lq * M;
    p.T = (int32_t)(nb * M * p.TPI);
    p.value_elems = (uint32_t)(nb * S * M * D);
    p.value = static_cast<const char *>(value) + n0 * S * M * D * esz;
    p.loc = loc + n0 * Lq * M * L * K * 2;
    p.attn = attn + n0 * Lq * M * L * K;
    p.offsets = ref_dim ? p.loc : nullptr;  // fused inputs: the raw predictions
    p.logits = ref_dim ? p.attn : nullptr;
    p.ref = ref_dim ? ref + n0 * Lq * ref_dim : nullptr;
    p.grad_out = static_cast<const char *>(grad_out) + n0 * Lq * M * D * esz;
    p.grad_value = grad_value + n0 * S * M * D;
    p.grad_loc = grad_loc + n0 * Lq * M * L * K * 2;
    p.grad_attn = grad_attn + n0 * Lq * M * L * K;
    p.grad_ref = (ref_dim && grad_ref) ? grad_ref + n0 * Lq * ref_dim : nullptr;
    if (msda::launch_backward(p, dt, shape, stream) != hipSuccess) return MSDA_ERROR_LAUNCH;
  }
  return MSDA_SUCCESS;
}

}  // namespace

extern "C" {

msda_status msda_validate(const int64_t *spatial_shapes, const int64_t *level_start, int64_t N,
                          int64_t S, int64_t M, int64_t D, int64_t L, int64_t Lq, int64_t K,
                          int dtype) {
  if (dtype != MSDA_F32 && dtype != MSDA_BF16) return MSDA_ERROR_NOT_SUPPORTED;
  if (N < 0 || Lq < 0 || S < 1 || M < 1 || D < 1 || L < 1 || K < 1) return MSDA_ERROR_INVALID_VALUE;
  if (L > MSDA_MAX_LEVELS || K > MSDA_MAX_POINTS || D > MSDA_MAX_CHANNELS) return MSDA_ERROR_NOT_SUPPORTED;
  if (spatial_shapes == nullptr || level_start == nullptr) return MSDA_ERROR_INVALID_VALUE;
  int64_t md, img, qmd;
  if (!mul_ok(M, D, &md) || !mul_ok(S, md, &img) || !mul_ok(Lq, md, &qmd)) return MSDA_ERROR_NOT_SUPPORTED;
  if (img > msda::kMaxSliceElems || qmd > msda::kMaxSliceElems) return MSDA_ERROR_NOT_SUPPORTED;
  for (int64_t l = 0; l < L; ++l) {
    const int64_t H = spatial_shapes[2 * l], W = spatial_shapes[2 * l + 1], s0 = level_start[l];
    if (H < 1 || W < 1 || s0 < 0) return MSDA_ERROR_INVALID_VALUE;
    if (H >= (int64_t(1) << 24) || W >= (int64_t(1) << 24)) return MSDA_ERROR_NOT_SUPPORTED;
    if (H * W > S || s0 > S - H * W) return MSDA_ERROR_INVALID_VALUE;
  }
  // Levels occupy disjoint row ranges of value (each row belongs to at most
  // one level, so every grad_value row has one owner).
  for (int64_t a = 0; a < L; ++a)
    for (int64_t b = a + 1; b < L; ++b) {
      const int64_t a0 = level_start[a], a1 = a0 + spatial_shapes[2 * a] * spatial_shapes[2 * a + 1];
      const int64_t b0 = level_start[b], b1 = b0 + spatial_shapes[2 * b] * spatial_shapes[2 * b + 1];
      if (a0 < b1 && b0 < a1) return MSDA_ERROR_INVALID_VALUE;
    }
  // Whole-tensor element counts must fit int64 (they index loc/attn/out).
  int64_t t;
  if (!mul_ok(N, img, &t) || !mul_ok(N, qmd, &t)) return MSDA_ERROR_NOT_SUPPORTED;
  int64_t pts;
  if (!mul_ok(N, Lq, &pts) || !mul_ok(pts, M * L * K * 2, &t)) return MSDA_ERROR_NOT_SUPPORTED;
  // One image's samples need 32-bit indices in the backward's tile entries.
  if (Lq * M * L * K > msda::kMaxSliceSamples / 4) return MSDA_ERROR_NOT_SUPPORTED;
  return MSDA_SUCCESS;
}

msda_status msda_forward(const void *value, const int64_t *spatial_shapes, const int64_t *level_start,
                         const float *loc, const float *attn, void *out, int64_t N, int64_t S, int64_t M,
                         int64_t D, int64_t L, int64_t Lq, int64_t K, int dtype, hipStream_t stream) {
  return forward_impl(value, spatial_shapes, level_start, loc, attn, nullptr, 0, out, N, S, M, D, L, Lq, K, dtype,
                      stream);
}

msda_status msda_fused_forward(const void *value, const int64_t *spatial_shapes, const int64_t *level_start,
                               const float *ref, int ref_dim, const float *offsets, const float *logits, void *out,
                               int64_t N, int64_t S, int64_t M, int64_t D, int64_t L, int64_t Lq, int64_t K,
                               int dtype, hipStream_t stream) {
  if (ref_dim != 2 && ref_dim != 4) return MSDA_ERROR_INVALID_VALUE;
  return forward_impl(value, spatial_shapes, level_start, offsets, logits, ref, ref_dim, out, N, S, M, D, L, Lq, K,
                      dtype, stream);
}

msda_status msda_backward_workspace_size(const int64_t *spatial_shapes, const int64_t *level_start, int64_t N,
                                         int64_t S, int64_t M, int64_t D, int64_t L, int64_t Lq, int64_t K,
                                         int dtype, size_t *bytes) {
  if (!bytes) return MSDA_ERROR_INVALID_VALUE;
  msda_status st = msda_validate(spatial_shapes, level_start, N, S, M, D, L, Lq, K, dtype);
  if (st != MSDA_SUCCESS) return st;
  const int64_t step = std::min(std::max<int64_t>(N, 1), images_per_launch(S, M, D, Lq, L, K));
  *bytes = msda::workspace_layout(spatial_shapes, L, step, M, Lq, K, false).bytes;
  return MSDA_SUCCESS;
}

msda_status msda_fused_backward_workspace_size(const int64_t *spatial_shapes, const int64_t *level_start, int64_t N,
                                               int64_t S, int64_t M, int64_t D, int64_t L, int64_t Lq, int64_t K,
                                               int dtype, size_t *bytes) {
  if (!bytes) return MSDA_ERROR_INVALID_VALUE;
  msda_status st = msda_validate(spatial_shapes, level_start, N, S, M, D, L, Lq, K, dtype);
  if (st != MSDA_SUCCESS) return st;
  const int64_t step = std::min(std::max<int64_t>(N, 1), images_per_launch(S, M, D, Lq, L, K));
  *bytes = msda::workspace_layout(spatial_shapes, L, step, M, Lq, K, true).bytes;
  return MSDA_SUCCESS;
}

msda_status msda_backward(const void *value, const int64_t *spatial_shapes, const int64_t *level_start,
                          const float *loc, const float *attn, const void *grad_out, float *grad_value,
                          float *grad_loc, float *grad_attn, int64_t N, int64_t S, int64_t M, int64_t D,
                          int64_t L, int64_t Lq, int64_t K, int dtype, void *workspace, size_t workspace_bytes,
                          hipStream_t stream) {
  return backward_impl(value, spatial_shapes, level_start, loc, attn, nullptr, 0, grad_out, grad_value, grad_loc,
                       grad_attn, nullptr, N, S, M, D, L, Lq, K, dtype, workspace, workspace_bytes, stream);
}

msda_status msda_backward_static(const void *value, const int64_t *spatial_shapes, const int64_t *level_start,
                                 const float *loc, const float *attn, const void *grad_out, float *grad_value,
                                 float *grad_loc, float *grad_attn, int64_t N, int64_t S, int64_t M, int64_t D,
                                 int64_t L, int64_t Lq, int64_t K, int dtype, hipStream_t stream) {
  static_assert(msda::kStaticScratchBytes == MSDA_STATIC_SCRATCH_BYTES, "scratch size out of step with msda.h");
  size_t need = 0;
  msda_status st = msda_backward_workspace_size(spatial_shapes, level_start, N, S, M, D, L, Lq, K, dtype, &need);
  if (st != MSDA_SUCCESS) return st;
  if (need > msda::kStaticScratchBytes) return MSDA_ERROR_SCRATCH;
  void *ws = nullptr;
  if (msda::static_scratch(&ws) != hipSuccess) return MSDA_ERROR_LAUNCH;
  return backward_impl(value, spatial_shapes, level_start, loc, attn, nullptr, 0, grad_out, grad_value, grad_loc,
                       grad_attn, nullptr, N, S, M, D, L, Lq, K, dtype, ws, msda::kStaticScratchBytes, stream);
}

msda_status msda_fused_backward(const void *value, const int64_t *spatial_shapes, const int64_t *level_start,
                                const float *ref, int ref_dim, const float *offsets, const float *logits,
                                const void *grad_out, float *grad_value, float *grad_offsets, float *grad_logits,
                                float *grad_ref, int64_t N, int64_t S, int64_t M, int64_t D, int64_t L, int64_t Lq,
                                int64_t K, int dtype, void *workspace, size_t workspace_bytes,
                                hipStream_t stream) {
  if (ref_dim != 2 && ref_dim != 4) return MSDA_ERROR_INVALID_VALUE;
  return backward_impl(value, spatial_shapes, level_start, offsets, logits, ref, ref_dim, grad_out, grad_value,
                       grad_offsets, grad_logits, grad_ref, N, S, M, D, L, Lq, K, dtype, workspace,
                       workspace_bytes, stream);
}

// Deformable groups: the M/G heads of a group are consecutive channels of a
// value row and of an out row, so grouped sampling is the sampling core with G
// heads of (M/G)*D channels each.
static bool group_shape(int64_t M, int64_t D, int64_t G, int64_t *Dg) {
  if (G < 1 || M < 1 || M % G != 0) return false;
  return mul_ok(M / G, D, Dg);
}

msda_status msda_grouped_forward(const void *value, const int64_t *spatial_shapes, const int64_t *level_start,
                                 const float *loc, const float *attn, void *out, int64_t N, int64_t S, int64_t M,
                                 int64_t D, int64_t L, int64_t Lq, int64_t K, int64_t G, int dtype,
                                 hipStream_t stream) {
  int64_t Dg;
  if (!group_shape(M, D, G, &Dg)) return MSDA_ERROR_INVALID_VALUE;
  return forward_impl(value, spatial_shapes, level_start, loc, attn, nullptr, 0, out, N, S, G, Dg, L, Lq, K, dtype,
                      stream);
}

msda_status msda_grouped_backward_workspace_size(const int64_t *spatial_shapes, const int64_t *level_start,
                                                 int64_t N, int64_t S, int64_t M, int64_t D, int64_t L, int64_t Lq,
                                                 int64_t K, int64_t G, int dtype, size_t *bytes) {
  int64_t Dg;
  if (!group_shape(M, D, G, &Dg)) return MSDA_ERROR_INVALID_VALUE;
  return msda_backward_workspace_size(spatial_shapes, level_start, N, S, G, Dg, L, Lq, K, dtype, bytes);
}

msda_status msda_grouped_backward(const void *value, const int64_t *spatial_shapes, const int64_t *level_start,
                                  const float *loc, const float *attn, const void *grad_out, float *grad_value,
                                  float *grad_loc, float *grad_attn, int64_t N, int64_t S, int64_t M, int64_t D,
                                  int64_t L, int64_t Lq, int64_t K, int64_t G, int dtype, void *workspace,
                                  size_t workspace_bytes, hipStream_t stream) {
  int64_t Dg;
  if (!group_shape(M, D, G, &Dg)) return MSDA_ERROR_INVALID_VALUE;
  return backward_impl(value, spatial_shapes, level_start, loc, attn, nullptr, 0, grad_out, grad_value, grad_loc,
                       grad_attn, nullptr, N, S, G, Dg, L, Lq, K, dtype, workspace, workspace_bytes, stream);
}

const char *msda_status_string(msda_status status) {
  switch (status) {
    case MSDA_SUCCESS: return "MSDA_SUCCESS: no error";
    case MSDA_ERROR_INVALID_VALUE: return "MSDA_ERROR_INVALID_VALUE: null pointer, bad size or level outside S";
    case MSDA_ERROR_NOT_SUPPORTED: return "MSDA_ERROR_NOT_SUPPORTED: shape, size or dtype beyond the library's limits";
    case MSDA_ERROR_MISALIGNED: return "MSDA_ERROR_MISALIGNED: a device pointer is not aligned to its element size";
    case MSDA_ERROR_LAUNCH: return "MSDA_ERROR_LAUNCH: a kernel launch failed";
    case MSDA_ERROR_WORKSPACE: return "MSDA_ERROR_WORKSPACE: workspace missing or smaller than msda_backward_workspace_size";
    case MSDA_ERROR_SCRATCH:
      return "MSDA_ERROR_SCRATCH: the problem needs more backward workspace than the static scratch "
             "(MSDA_STATIC_SCRATCH_BYTES = 64 MiB) holds; use msda_backward with a workspace";
  }
  return "MSDA: unknown status";
}

}  // extern "C"
