// gfx950 kernels of the multi-scale deformable attention sampling core.
//
// What is computed: page "Deformable DETR", section "Multi-scale deformable
// attention", equation MSDeformAttn (the attention-weighted sum of bilinear
// samples, per head), and its gradients (page "Deformable Attention": the
// bilinear sampling is differentiable). Conventions are stated in msda.h.
//
// Mapping onto CDNA4. The op is a gather, not a contraction, so there is no
// MFMA here; the roof is HBM bandwidth and the L1/L2 gather rate.
//   * value is [N, S, M, D], channel-contiguous: one bilinear corner of one
//     head is one D*elem-byte segment (128 B for fp32 D=32, 64 B for bf16).
//   * A (n, q, m) "pair" owns D output channels and is served by `lpp` lanes,
//     each holding `vec` contiguous channels (16-byte accesses when possible),
//     so every corner read of a pair is one coalesced segment.
//   * Per workgroup, each sample's coordinate transform, corner offsets and
//     corner weights are computed once (one lane per sample, reading loc and
//     attn coalesced) and staged in LDS as a 32-byte descriptor; every lane
//     of the pair then reads the descriptor with an LDS broadcast.
//   * Corners outside the map carry an offset past the buffer's num_records,
//     so buffer loads return 0 and buffer atomics are dropped by the hardware:
//     zero padding with no branch.
//   * Workgroups are renumbered so that each XCD (own L2) works on one
//     contiguous range of queries, which sample overlapping value rows.
//   * Backward: per sample, the three dot products (grad_attn and the two
//     location gradients) are reduced across the pair's lanes with DPP and
//     written coalesced; grad_value is built per pixel tile from a counting
//     sort of the samples, or with float atomics when samples are sparse
//     (see the backward section).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <mutex>
#include <type_traits>

#include "msda_internal.h"

namespace msda {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kDescCap = 544;             // sample descriptors staged per chunk (16 x 34)
constexpr int kRsrcWord3 = 0x00020000;    // gfx9 buffer resource: raw, 32-bit data format

struct F32 {
  static constexpr int size = 4;
};
struct BF16 {
  static constexpr int size = 2;
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, (int)bytes, kRsrcWord3);
}

// Loads VEC elements of type T at byte offset `off` of buffer `r` and widens
// them to float (bf16 -> f32 is exact: the bits move to the upper half).
template <typename T, int VEC>
__device__ __forceinline__ void load_vals(__amdgpu_buffer_rsrc_t r, uint32_t off, float (&v)[VEC]) {
  constexpr int BYTES = VEC * T::size;
  uint32_t w[(BYTES + 3) / 4];
  if constexpr (BYTES == 16) {
    u32x4 x = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
    w[0] = x.x; w[1] = x.y; w[2] = x.z; w[3] = x.w;
  } else if constexpr (BYTES == 8) {
    u32x2 x = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
    w[0] = x.x; w[1] = x.y;
  } else if constexpr (BYTES == 4) {
    w[0] = __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
  } else {
    static_assert(BYTES == 2, "unsupported access width");
    w[0] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0);
  }
  if constexpr (std::is_same<T, F32>::value) {
#pragma unroll
    for (int i = 0; i < VEC; ++i) v[i] = __uint_as_float(w[i]);
  } else if constexpr (VEC == 1) {
    v[0] = __uint_as_float(w[0] << 16);
  } else {
#pragma unroll
    for (int i = 0; i < VEC / 2; ++i) {
      v[2 * i] = __uint_as_float(w[i] << 16);
      v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
}

// float -> bf16 bits, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint32_t bf16_bits(float f) {
  const uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

template <typename T, int VEC>
__device__ __forceinline__ void store_vals(void *base, int64_t elem, const float (&v)[VEC]) {
  if constexpr (std::is_same<T, F32>::value) {
    float *p = reinterpret_cast<float *>(base) + elem;
    if constexpr (VEC == 4) {
      *reinterpret_cast<float4 *>(p) = make_float4(v[0], v[1], v[2], v[3]);
    } else if constexpr (VEC == 2) {
      *reinterpret_cast<float2 *>(p) = make_float2(v[0], v[1]);
    } else {
      p[0] = v[0];
    }
  } else {
    uint16_t *p = reinterpret_cast<uint16_t *>(base) + elem;
    if constexpr (VEC == 1) {
      p[0] = (uint16_t)bf16_bits(v[0]);
    } else {
      uint32_t w[VEC / 2];
#pragma unroll
      for (int i = 0; i < VEC / 2; ++i) w[i] = bf16_bits(v[2 * i]) | (bf16_bits(v[2 * i + 1]) << 16);
      if constexpr (VEC == 8) {
        *reinterpret_cast<uint4 *>(p) = make_uint4(w[0], w[1], w[2], w[3]);
      } else if constexpr (VEC == 4) {
        *reinterpret_cast<uint2 *>(p) = make_uint2(w[0], w[1]);
      } else {
        *reinterpret_cast<uint32_t *>(p) = w[0];
      }
    }
  }
}

// Hardware dispatches workgroup b to XCD b % 8. Renumber so that XCD x runs
// one contiguous range of logical tiles (a bijection for any grid size).
__device__ __forceinline__ int xcd_remap(int b, int nb) {
  const int q = nb >> 3, r = nb & 7, x = b & 7, i = b >> 3;
  return (x < r ? x * (q + 1) : r * (q + 1) + (x - r) * q) + i;
}

template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, true));
}

// Sum (or maximum) over the `lpp` consecutive lanes of a pair; every lane
// gets the result. (The maximum only keeps exp() in range for the softmax: a
// NaN logit, which fmaxf skips, still turns its head's sum and weights NaN.) Steps: quad xor 1, quad xor 2, mirror within 8, mirror
// within 16, then cross-row exchanges. Each step combines two disjoint
// partial results, so the sum is identical in every lane of the group.
template <int LPP, bool MAX = false>
__device__ __forceinline__ float group_sum(float v, int lpp_rt) {
  const int lpp = LPP > 0 ? LPP : lpp_rt;
  auto op = [](float a, float b) { return MAX ? fmaxf(a, b) : a + b; };
  if (lpp >= 2) v = op(v, dpp_mov<0xB1>(v));   // quad_perm [1,0,3,2]
  if (lpp >= 4) v = op(v, dpp_mov<0x4E>(v));   // quad_perm [2,3,0,1]
  if (lpp >= 8) v = op(v, dpp_mov<0x141>(v));  // row_half_mirror
  if (lpp >= 16) v = op(v, dpp_mov<0x140>(v)); // row_mirror
  if (lpp >= 32) v = op(v, __shfl_xor(v, 16));
  if (lpp >= 64) v = op(v, __shfl_xor(v, 32));
  return v;
}

// Level table into LDS: thread l copies level l's entries (indexed reads of
// the argument block, one per thread, rather than a chain of per-level
// branches).
__device__ __forceinline__ void load_levels(const Params &p, int32_t *sH, int32_t *sW, int32_t *sS) {
  const int tid = threadIdx.x;
  if (tid < kMaxLevels) {
    sH[tid] = p.lv.H[tid];
    sW[tid] = p.lv.W[tid];
    sS[tid] = p.lv.start[tid];
  }
}

// The per-sample geometry shared by both passes: index-space coordinate,
// in-map test, floor corner, fractional parts and the four corner element
// offsets (kOobElem where the corner is outside the map).
struct Sample {
  uint32_t off[4];
  float a, b, A;
  bool inside;
};

// Element offset of (image n, row 0, head m, channel 0) for pair P (32-bit:
// every launch keeps value below 2^28 elements).
__device__ __forceinline__ uint32_t pair_base(const Params &p, uint32_t P) {
  const uint32_t lqm = (uint32_t)p.Lq * (uint32_t)p.M;
  const uint32_t n = P / lqm;
  const uint32_t m = (P - n * lqm) % (uint32_t)p.M;
  return (n * (uint32_t)p.S * (uint32_t)p.M + m) * (uint32_t)p.D;
}

// The (n, q, m) pairs of one workgroup of a per-sample pass: pair g of the
// workgroup is pair base + g * stride. Pair-major order (stride 1) takes ppb
// consecutive pairs; head-major order (stride M) takes ppb consecutive queries
// of one head, so that a workgroup's samples, and with the XCD-aware
// numbering an XCD's, concentrate on one head's value channels.
struct PairRange {
  int64_t base;
  int32_t stride, count;
  __device__ int64_t operator()(int g) const { return base + (int64_t)g * stride; }
};

__device__ __forceinline__ PairRange block_pairs(const Params &p, int lb, int ppb) {
  PairRange r;
  if (p.head_major) {
    const int qblocks = (p.Lq + ppb - 1) / ppb;
    const int nm = lb / qblocks, qb = lb - nm * qblocks;
    const int n = nm / p.M, m = nm - n * p.M;
    const int q0 = qb * ppb;
    r.base = ((int64_t)n * p.Lq + q0) * p.M + m;
    r.stride = p.M;
    r.count = min(ppb, p.Lq - q0);
  } else {
    r.base = (int64_t)lb * ppb;
    r.stride = 1;
    r.count = (int)min((int64_t)ppb, p.pairs - r.base);
  }
  return r;
}

// Exact quotient i / d for 1 <= d <= 256 and i * d <= 2^20 (so any i < 4096)
// with mg = ceil(2^20 / d): the rounding error of mg adds less than i / 2^20
// <= 1/d to i / d, whose fractional part is 0 or at most 1 - 1/d.
__device__ __forceinline__ uint32_t small_div(uint32_t i, uint32_t mg) { return (i * mg) >> 20; }
__device__ __forceinline__ uint32_t small_magic(uint32_t d) { return ((1u << 20) + d - 1) / d; }

// Geometry of a sample at normalised location xy with weight A.
__device__ __forceinline__ Sample sample_geometry(const Params &p, uint32_t base_pair, float2 xy, float A, int l,
                                                  const int32_t *sH, const int32_t *sW,
                                                  const int32_t *sS) {
  const int H = sH[l], W = sW[l], s0 = sS[l];
  float x = fmaf(xy.x, (float)W, -0.5f);
  float y = fmaf(xy.y, (float)H, -0.5f);
  Sample s;
  s.inside = (x >= -1.0f) && (x < (float)W) && (y >= -1.0f) && (y < (float)H);
  x = s.inside ? x : 0.0f;
  y = s.inside ? y : 0.0f;
  const float xf = floorf(x), yf = floorf(y);
  s.a = x - xf;
  s.b = y - yf;
  s.A = s.inside ? A : 0.0f;
  const int x0 = (int)xf, y0 = (int)yf;
  const uint32_t row = (uint32_t)p.M * (uint32_t)p.D;
  const uint32_t base = base_pair + (uint32_t)s0 * row;
  const bool xo0 = x0 >= 0, xo1 = x0 + 1 < W, yo0 = y0 >= 0, yo1 = y0 + 1 < H;
  const bool in = s.inside;
  const uint32_t r00 = base + (uint32_t)(y0 * W + x0) * row;
  const uint32_t rW = (uint32_t)W * row;
  s.off[0] = (in && yo0 && xo0) ? r00 : kOobElem;
  s.off[1] = (in && yo0 && xo1) ? r00 + row : kOobElem;
  s.off[2] = (in && yo1 && xo0) ? r00 + rW : kOobElem;
  s.off[3] = (in && yo1 && xo1) ? r00 + rW + row : kOobElem;
  return s;
}

// ------------------------------------------------- fused inputs (optional)
//
// The step in front of the sampling core, done in the kernels when the caller
// passes raw predictions (page "Deformable DETR", section "Deformable
// attention module": offsets and attention logits come from one linear
// projection of the query and the logits go through a softmax; section
// "Multi-scale deformable attention": the softmax runs jointly over a head's
// L*K samples and the location is the reference point plus an offset in
// level-l pixels; section "Variants": with boxes as references the offsets
// are scaled by the box's width and height). Locations are formed in binary32
// as ref + offset / size (points; quotient and sum each rounded once) or as
// one fmaf(offset, box size, box centre) (boxes).

__device__ __forceinline__ float softmax_weight(float z, float2 st) { return expf(z - st.x) * st.y; }

// Reference point (x, y, 0, 0) or box (cx, cy, w, h) of query row q (image
// and query flattened).
__device__ __forceinline__ float4 load_ref(const Params &p, uint32_t q) {
  const float2 *r = reinterpret_cast<const float2 *>(p.ref + (size_t)q * (size_t)p.ref_dim);
  const float2 c = r[0];
  if (p.ref_dim == 2) return make_float4(c.x, c.y, 0.0f, 0.0f);
  const float2 wh = r[1];
  return make_float4(c.x, c.y, wh.x, wh.y);
}

// Normalised location from the per-sample input v: v itself, or v taken as
// an offset from the reference `rf` (fused inputs).
template <bool FUSE>
__device__ __forceinline__ float2 form_loc(const Params &p, float2 v, int l, float4 rf, const int32_t *sH,
                                           const int32_t *sW) {
  if constexpr (!FUSE) return v;
  if (p.ref_dim == 2) return make_float2(rf.x + v.x / (float)sW[l], rf.y + v.y / (float)sH[l]);
  return make_float2(fmaf(v.x, rf.z, rf.x), fmaf(v.y, rf.w, rf.y));
}

// Softmax statistics (max, 1/sum) of a pair's logits z[0, LK), computed by the
// pair's lpp lanes (lane j takes every lpp-th logit); every lane of the pair
// gets them. Lanes of inactive pairs only join the exchanges.
template <int LPP>
__device__ __forceinline__ float2 pair_softmax_stats(const float *z, bool active, int j, int lpp, int LK) {
  float mx = -INFINITY;
  if (active)
    for (int i = j; i < LK; i += lpp) mx = fmaxf(mx, z[i]);
  mx = group_sum<LPP, true>(mx, lpp);
  float s = 0.0f;
  if (active)
    for (int i = j; i < LK; i += lpp) s += expf(z[i] - mx);
  s = group_sum<LPP>(s, lpp);
  return make_float2(mx, 1.0f / s);
}

// Softmax weight of logit z when the L*K logits of its pair sit in lk
// consecutive lanes aligned to lk (a power of two <= 64, all of them active):
// the maximum and the sum come from lane exchanges, with no memory traffic.
__device__ __forceinline__ float segment_softmax(float z, int lk) {
  const float mx = group_sum<0, true>(z, lk);
  const float e = expf(z - mx);
  return e * (1.0f / group_sum<0>(e, lk));
}

// ---------------------------------------------------------------- forward

struct __align__(16) FDesc {
  uint32_t off[4];  // byte offsets of the corners in value
  float w[4];       // attn * bilinear weight, 0 for corners outside the map
};

// Forward. A workgroup takes kBlock / lpp consecutive (n, q, m) pairs. For
// each chunk of pc points: one thread per sample reads its location and
// weight (with fused inputs: offset and logit, forming both), computes the
// corner offsets and weights and writes the sample's descriptor to LDS; after
// a barrier, the lanes of each pair walk its samples, gathering the four
// corner rows and accumulating into registers. Finally each lane stores its
// channels of out.
template <typename T, int VEC, int NCG, int LPP, bool FUSE>
__global__ __launch_bounds__(kBlock) void fwd_kernel(const Params p) {
  // bf16 rows: three samples' corner loads in flight per lane (measured
  // faster than two despite the lower occupancy); fp32 and the fused variant
  // keep the plain loop, which the compiler schedules two samples at a time
  constexpr int SB = std::is_same<T, BF16>::value && NCG == 1 && !FUSE ? 3 : 1;
  __shared__ FDesc desc[kDescCap];
  __shared__ uint32_t pbase[kBlock];
  __shared__ uint32_t pqry[FUSE ? kBlock : 1];  // query row of each pair
  __shared__ float2 sst[FUSE ? kBlock : 1];   // softmax statistics of each pair
  __shared__ int32_t sH[kMaxLevels], sW[kMaxLevels], sS[kMaxLevels];
  load_levels(p, sH, sW, sS);

  const int tid = threadIdx.x;
  const int lpp = LPP > 0 ? LPP : p.lpp;
  const int ppb = kBlock / lpp;
  // descriptor rows padded by one so that consecutive samples of a pair (the
  // lanes that write them) fall on different LDS banks
  const int dstride = ppb + 1;
  const PairRange pr = block_pairs(p, xcd_remap(blockIdx.x, gridDim.x), ppb);
  const int npairs = pr.count;
  const int g = tid / lpp;
  const int j = tid - g * lpp;
  const bool active = g < npairs;
  if (tid < npairs) pbase[tid] = pair_base(p, (uint32_t)pr(tid));
  if constexpr (FUSE) {
    if (tid < npairs) pqry[tid] = (uint32_t)pr(tid) / (uint32_t)p.M;
    if (!p.seg_softmax) {
      const float2 st = pair_softmax_stats<LPP>(p.attn + (active ? pr(g) * p.LK : 0), active, j, lpp, p.LK);
      if (active && j == 0) sst[g] = st;
    }
  }
  const uint32_t kmg = small_magic((uint32_t)p.K);

  const __amdgpu_buffer_rsrc_t rv = make_rsrc(p.value, p.value_elems * (uint32_t)T::size);
  const int nvec = p.D / VEC;
  uint32_t lane_off[NCG];
#pragma unroll
  for (int cg = 0; cg < NCG; ++cg) {
    const int c = j + cg * lpp;
    // Lanes past the last channel read past the buffer (zeros) and store nothing.
    lane_off[cg] = c < nvec ? (uint32_t)(c * VEC * T::size) : kOobElem * (uint32_t)T::size;
  }
  float acc[NCG][VEC];
#pragma unroll
  for (int cg = 0; cg < NCG; ++cg)
#pragma unroll
    for (int e = 0; e < VEC; ++e) acc[cg][e] = 0.0f;

  for (int pc0 = 0; pc0 < p.LK; pc0 += p.pc) {
    const int pcn = min(p.pc, p.LK - pc0);
    const uint32_t pmg = small_magic((uint32_t)pcn);
    __syncthreads();
    // two samples per thread per round, both samples' loads issued first
    const int total = npairs * pcn;
    for (int i0 = tid; i0 < total; i0 += 2 * kBlock) {
      float2 v[2];
      float z[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int i = i0 + u * kBlock;
        const int gg = (int)small_div((uint32_t)(i < total ? i : 0), pmg);
        const int64_t gi = pr(gg) * p.LK + pc0 + ((i < total ? i : 0) - gg * pcn);
        v[u] = i < total ? *reinterpret_cast<const float2 *>(p.loc + 2 * gi) : make_float2(0.0f, 0.0f);
        z[u] = i < total ? p.attn[gi] : 0.0f;
      }
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int i = i0 + u * kBlock;
        if (i >= total) continue;  // whole pairs of samples drop out together
        const int gg = (int)small_div((uint32_t)i, pmg);
        const int pp = i - gg * pcn;
        const int pt = pc0 + pp;
        const int l = (int)small_div((uint32_t)pt, kmg);
        float2 xy = v[u];
        float A = z[u];
        if constexpr (FUSE) {
          xy = form_loc<true>(p, v[u], l, load_ref(p, pqry[gg]), sH, sW);
          A = p.seg_softmax ? segment_softmax(z[u], p.LK) : softmax_weight(z[u], sst[gg]);
        }
        const Sample s = sample_geometry(p, pbase[gg], xy, A, l, sH, sW, sS);
        FDesc d;
        const float wa[2] = {1.0f - s.a, s.a};
        const float wb[2] = {1.0f - s.b, s.b};
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const bool ok = s.off[c] != kOobElem;
          d.off[c] = s.off[c] * (uint32_t)T::size;
          d.w[c] = ok ? s.A * wb[c >> 1] * wa[c & 1] : 0.0f;
        }
        desc[pp * dstride + gg] = d;
      }
    }
    __syncthreads();
    if (active) {
      int pp = 0;
      if constexpr (SB > 1) {
        // SB samples' corner loads issued together, then their FMAs in
        // sample order (the same sums as the loop below)
        for (; pp + SB <= pcn; pp += SB) {
          FDesc d[SB];
          float v[SB][4][VEC];
#pragma unroll
          for (int sb = 0; sb < SB; ++sb) d[sb] = desc[(pp + sb) * dstride + g];
#pragma unroll
          for (int sb = 0; sb < SB; ++sb)
#pragma unroll
            for (int c = 0; c < 4; ++c) load_vals<T, VEC>(rv, d[sb].off[c] + lane_off[0], v[sb][c]);
#pragma unroll
          for (int sb = 0; sb < SB; ++sb)
#pragma unroll
            for (int c = 0; c < 4; ++c)
#pragma unroll
              for (int e = 0; e < VEC; ++e) acc[0][e] = fmaf(d[sb].w[c], v[sb][c][e], acc[0][e]);
        }
      }
#pragma unroll 2
      for (; pp < pcn; ++pp) {
        const FDesc d = desc[pp * dstride + g];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
#pragma unroll
          for (int cg = 0; cg < NCG; ++cg) {
            float v[VEC];
            load_vals<T, VEC>(rv, d.off[c] + lane_off[cg], v);
#pragma unroll
            for (int e = 0; e < VEC; ++e) acc[cg][e] = fmaf(d.w[c], v[e], acc[cg][e]);
          }
        }
      }
    }
  }
  if (active) {
    const int64_t obase = pr(g) * (int64_t)p.D;
#pragma unroll
    for (int cg = 0; cg < NCG; ++cg) {
      const int c = j + cg * lpp;
      if (c < nvec) store_vals<T, VEC>(p.out, obase + (int64_t)c * VEC, acc[cg]);
    }
  }
}

// --------------------------------------------------------------- backward
//
// The backward runs as a short pipeline on the caller's stream:
//   0. (fused inputs only) fused_inputs_kernel forms every sample's location
//      and weight into the workspace; the passes below read them.
//   Dense launches (many samples per value tile):
//   1. zero_u32_kernel clears the tile counters.
//   2. bin_kernel<count> / scan_kernel / bin_kernel<scatter>: a counting sort
//      of (sample, 8x8-pixel tile) entries, one entry per tile that a sample's
//      in-map corners touch. Workgroups own one (image, head) and a range of
//      queries, so their tile histogram fits in LDS and only nonzero bins reach
//      global memory (integer atomics, a few per workgroup). The scan lists
//      the grad_value work items, crowded (split) tiles first; the scatter
//      launch also clears those tiles.
//   3. grad_value items and the sample gradients, in one launch for the hot
//      shapes (bwd_fused_kernel: items first, then sample blocks) or as
//      bwd_sample_kernel then gv_kernel. A grad_value item owns one tile (or a
//      slice of a crowded one): its entries' corner contributions are
//      bucketed by pixel in LDS, then each thread sums the contributions to
//      the pixel it owns in registers and stores them; float atomics appear
//      only for split tiles. The sample blocks compute grad_attn and grad_loc
//      with the forward's gather, reducing each sample's three dot products
//      across the pair's lanes.
//   Sparse launches (decoder-sized): grad_value is zero-filled and the sample
//   pass adds each corner's contribution with float atomics.
// gfx950 float atomics (global and LDS) sustain a small fraction of the
// integer LDS atomic and plain-store rates, so the dense path accumulates
// grad_value without them.

struct __align__(16) BDesc {
  uint32_t off[4];  // element offsets of the corners (kOobElem outside the map)
  float a, b;       // fractional parts of the index coordinate
  float aw, ah;     // attn * W_l, attn * H_l (chain rule through loc * W - 0.5)
};

constexpr size_t kSampleSmemPlain =
    kDescCap * (sizeof(BDesc) + sizeof(float3) + 4) + 3 * kMaxLevels * 4 + kBlock * 4;
// fused inputs add per pair: sum of A * grad_attn, query row; per staged
// sample: its offset
constexpr size_t kSampleSmemFused = kSampleSmemPlain + kBlock * (4 + 4) + kDescCap * 8;
template <bool FUSE>
constexpr size_t sample_smem() { return FUSE ? kSampleSmemFused : kSampleSmemPlain; }

// grad_attn and grad_loc of the pairs of logical block `block` (of `nblocks`),
// with LDS carved from `smem` (sample_smem<FUSE>() bytes). With p.scatter the
// same pass also adds each sample's grad_value contributions (attn * corner
// weight * grad_out) with float atomics. With fused inputs (loc and attn then
// hold the locations and weights that fused_inputs_kernel formed) grad_attn and
// grad_loc become the logit and offset gradients: through the softmax,
// d/dz_i = A_i (grad_attn_i - sum_j A_j grad_attn_j); through the location,
// d/d offset = grad_loc / size (points) or grad_loc * box size (boxes); and the
// reference gradient is the sum of grad_loc (and of grad_loc * offset for the
// box size) over a query's samples.
template <typename T, int VEC, int NCG, int LPP, bool FUSE>
__device__ __forceinline__ void bwd_sample_body(const Params &p, int block, int nblocks, unsigned char *smem) {
  // two samples' corner loads in flight per lane in the hot shapes (measured:
  // the combined backward kernel 176 -> 167 us; three gain nothing more)
  constexpr int BSB = (LPP > 0 && NCG == 1) ? 2 : 1;
  BDesc *desc = reinterpret_cast<BDesc *>(smem);
  float3 *res = reinterpret_cast<float3 *>(desc + kDescCap);
  float *sA = reinterpret_cast<float *>(res + kDescCap);  // each staged sample's weight
  int32_t *sH = reinterpret_cast<int32_t *>(sA + kDescCap);
  int32_t *sW = sH + kMaxLevels, *sS = sW + kMaxLevels;
  uint32_t *pbase = reinterpret_cast<uint32_t *>(sS + kMaxLevels);
  // fused inputs only
  float2 *soff = reinterpret_cast<float2 *>(smem + kSampleSmemPlain);
  float *ssum = reinterpret_cast<float *>(soff + kDescCap);
  uint32_t *pqry = reinterpret_cast<uint32_t *>(ssum + kBlock);
  load_levels(p, sH, sW, sS);

  const int tid = threadIdx.x;
  const int lpp = LPP > 0 ? LPP : p.lpp;
  const int ppb = kBlock / lpp;
  const int dstride = ppb + 1;  // padded descriptor rows (see fwd_kernel)
  const PairRange pr = block_pairs(p, xcd_remap(block, nblocks), ppb);
  const int npairs = pr.count;
  const int g = tid / lpp;
  const int j = tid - g * lpp;
  const bool active = g < npairs;
  if (tid < npairs) pbase[tid] = pair_base(p, (uint32_t)pr(tid));
  if constexpr (FUSE) {
    if (tid < npairs) pqry[tid] = (uint32_t)pr(tid) / (uint32_t)p.M;
  }
  // the pair's sums over its samples (identical in all its lanes)
  float acc_s = 0.0f, acc_rx = 0.0f, acc_ry = 0.0f, acc_bx = 0.0f, acc_by = 0.0f;
  const uint32_t kmg = small_magic((uint32_t)p.K);

  const __amdgpu_buffer_rsrc_t rv = make_rsrc(p.value, p.value_elems * (uint32_t)T::size);
  const __amdgpu_buffer_rsrc_t ro = make_rsrc(p.grad_out, (uint32_t)(p.pairs * p.D) * (uint32_t)T::size);
  const __amdgpu_buffer_rsrc_t rg = make_rsrc(p.grad_value, p.value_elems * 4u);
  const int nvec = p.D / VEC;
  uint32_t lane_elem[NCG];
  float G[NCG][VEC];
#pragma unroll
  for (int cg = 0; cg < NCG; ++cg) {
    const int c = j + cg * lpp;
    lane_elem[cg] = c < nvec ? (uint32_t)(c * VEC) : kOobElem;
    const uint32_t go = active && c < nvec ? (uint32_t)(pr(g) * p.D + c * VEC) : kOobElem;
    load_vals<T, VEC>(ro, go * (uint32_t)T::size, G[cg]);
  }

  for (int pc0 = 0; pc0 < p.LK; pc0 += p.pc) {
    const int pcn = min(p.pc, p.LK - pc0);
    const uint32_t pmg = small_magic((uint32_t)pcn);
    __syncthreads();
    for (int i = tid; i < npairs * pcn; i += kBlock) {
      const int gg = (int)small_div((uint32_t)i, pmg);
      const int pp = i - gg * pcn;
      const int pt = pc0 + pp;
      const int l = (int)small_div((uint32_t)pt, kmg);
      const int64_t gi = pr(gg) * p.LK + pt;
      const float2 xy = *reinterpret_cast<const float2 *>(p.loc + 2 * gi);
      const float A = p.attn[gi];
      if constexpr (FUSE) {
        if (p.ref_dim == 4) soff[pp * dstride + gg] = *reinterpret_cast<const float2 *>(p.offsets + 2 * gi);
      }
      // the weight itself, in the map or not (the softmax gradient needs it;
      // corners outside the map drop the scatter's atomics)
      sA[pp * dstride + gg] = A;
      const Sample s = sample_geometry(p, pbase[gg], xy, A, l, sH, sW, sS);
      BDesc d;
#pragma unroll
      for (int c = 0; c < 4; ++c) d.off[c] = s.off[c];
      d.a = s.a;
      d.b = s.b;
      d.aw = s.A * (float)sW[l];
      d.ah = s.A * (float)sH[l];
      desc[pp * dstride + gg] = d;
    }
    __syncthreads();
    if (active) {
      for (int pp0 = 0; pp0 < pcn; pp0 += BSB) {
        // BSB samples' corner loads issued together (slots past the chunk
        // repeat its first sample and are not used)
        BDesc dd[BSB];
        float dots[BSB][4];
#pragma unroll
        for (int sb = 0; sb < BSB; ++sb) dd[sb] = desc[(pp0 + sb < pcn ? pp0 + sb : pp0) * dstride + g];
#pragma unroll
        for (int sb = 0; sb < BSB; ++sb)
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            dots[sb][c] = 0.0f;
#pragma unroll
            for (int cg = 0; cg < NCG; ++cg) {
              float v[VEC];
              load_vals<T, VEC>(rv, (dd[sb].off[c] + lane_elem[cg]) * (uint32_t)T::size, v);
#pragma unroll
              for (int e = 0; e < VEC; ++e) dots[sb][c] = fmaf(G[cg][e], v[e], dots[sb][c]);
            }
          }
#pragma unroll
        for (int sb = 0; sb < BSB; ++sb) {
          const int pp = pp0 + sb;
          if (pp >= pcn) break;
          const BDesc &d = dd[sb];
          const float *dot = dots[sb];
          const float a = d.a, b = d.b;
          if (p.scatter) {
            const float A = sA[pp * dstride + g];
            const float wa[2] = {1.0f - a, a}, wb[2] = {1.0f - b, b};
#pragma unroll
            for (int c = 0; c < 4; ++c) {
              const float wc = A * wb[c >> 1] * wa[c & 1];
#pragma unroll
              for (int cg = 0; cg < NCG; ++cg)
#pragma unroll
                for (int e = 0; e < VEC; ++e)
                  __builtin_amdgcn_raw_ptr_buffer_atomic_fadd_f32(
                      wc * G[cg][e], rg, (int)((d.off[c] + lane_elem[cg] + (uint32_t)e) * 4u), 0, 0);
            }
          }
          float ga = (1.0f - b) * ((1.0f - a) * dot[0] + a * dot[1]) + b * ((1.0f - a) * dot[2] + a * dot[3]);
          float gx = (1.0f - b) * (dot[1] - dot[0]) + b * (dot[3] - dot[2]);
          float gy = (1.0f - a) * (dot[2] - dot[0]) + a * (dot[3] - dot[1]);
          ga = group_sum<LPP>(ga, lpp);
          gx = group_sum<LPP>(gx, lpp);
          gy = group_sum<LPP>(gy, lpp);
          const float glx = d.aw * gx, gly = d.ah * gy;
          if (j == 0) res[pp * dstride + g] = make_float3(ga, glx, gly);
          if constexpr (FUSE) {
            acc_s = fmaf(sA[pp * dstride + g], ga, acc_s);
            acc_rx += glx;
            acc_ry += gly;
            if (p.ref_dim == 4) {
              // a sample outside the map (also one whose offset is not
              // finite) has a zero location gradient and no term here,
              // rather than 0 * offset
              const float2 o = soff[pp * dstride + g];
              acc_bx = glx != 0.0f ? fmaf(glx, o.x, acc_bx) : acc_bx;
              acc_by = gly != 0.0f ? fmaf(gly, o.y, acc_by) : acc_by;
            }
          }
        }
      }
      if constexpr (FUSE) {
        if (j == 0) ssum[g] = acc_s;  // the pair's full sum after its last chunk
      }
    }
    __syncthreads();
    for (int i = tid; i < npairs * pcn; i += kBlock) {
      const int gg = (int)small_div((uint32_t)i, pmg);
      const int pp = i - gg * pcn;
      const float3 r = res[pp * dstride + gg];
      const int64_t gi = pr(gg) * p.LK + pc0 + pp;
      float2 gl = make_float2(r.y, r.z);
      float gz = r.x;
      if constexpr (FUSE) {
        // one chunk holds all of the pair's samples: its sum is complete here;
        // otherwise grad_attn is stored and finished below
        if (p.LK <= p.pc) gz = sA[pp * dstride + gg] * (r.x - ssum[gg]);
        if (p.ref_dim == 4) {
          const float4 rf = load_ref(p, pqry[gg]);
          gl = make_float2(r.y * rf.z, r.z * rf.w);
        } else {
          const int l = (int)small_div((uint32_t)(pc0 + pp), kmg);
          gl = make_float2(r.y / (float)sW[l], r.z / (float)sH[l]);
        }
      }
      p.grad_attn[gi] = gz;
      *reinterpret_cast<float2 *>(p.grad_loc + 2 * gi) = gl;
    }
  }
  if constexpr (FUSE) {
    // the pair's share of its query's reference gradient (summed over the
    // query's heads by ref_grad_kernel)
    if (active && j == 0 && p.grad_ref)
      *reinterpret_cast<float4 *>(p.ws.ref_part + 4 * pr(g)) = make_float4(acc_rx, acc_ry, acc_bx, acc_by);
    if (p.LK > p.pc) {
      __syncthreads();
      // grad_logits from the grad_attn values this block stored above
      // (visible to the whole workgroup after the barrier)
      for (int i = tid; i < npairs * p.LK; i += kBlock) {
        const int gg = i / p.LK;
        const int64_t gi = pr(gg) * p.LK + (i - gg * p.LK);
        p.grad_attn[gi] = p.attn[gi] * (p.grad_attn[gi] - ssum[gg]);
      }
    }
  }
}

template <typename T, int VEC, int NCG, int LPP, bool FUSE>
__global__ __launch_bounds__(kBlock) void bwd_sample_kernel(const Params p) {
  __shared__ __align__(16) unsigned char smem[sample_smem<FUSE>()];
  bwd_sample_body<T, VEC, NCG, LPP, FUSE>(p, blockIdx.x, gridDim.x, smem);
}

// ------------------------------------------- fused inputs for the backward
//
// The backward with fused inputs first forms every sample's location and
// weight once (the same arithmetic as the fused forward) into the workspace;
// the binning passes and the sample pass then read them as plain inputs. With
// a power-of-two L*K up to 64, thread s takes sample s and a pair's samples
// are consecutive lanes (softmax from lane exchanges); otherwise thread P
// takes pair P and walks its L*K logits.
__global__ __launch_bounds__(kBlock) void fused_inputs_kernel(const Params p, float *loc_out, float *attn_out) {
  __shared__ int32_t sH[kMaxLevels], sW[kMaxLevels], sS[kMaxLevels];
  load_levels(p, sH, sW, sS);
  __syncthreads();
  const uint32_t LK = (uint32_t)p.LK, K = (uint32_t)p.K;
  if (p.seg_softmax) {
    // samples of one launch have 32-bit indices; L*K is a power of two here
    const uint32_t total = (uint32_t)(p.pairs * p.LK);
    const uint32_t s = blockIdx.x * (uint32_t)kBlock + threadIdx.x;
    const bool ok = s < total;  // whole pairs drop out together
    const uint32_t P = (ok ? s : 0u) >> (31 - __builtin_clz(LK));
    const uint32_t pt = (ok ? s : 0u) & (LK - 1u);
    const int l = (int)small_div(pt, small_magic(K));
    const float2 v = ok ? *reinterpret_cast<const float2 *>(p.offsets + 2 * (size_t)s) : make_float2(0.0f, 0.0f);
    const float z = ok ? p.logits[s] : 0.0f;
    const float A = segment_softmax(z, p.LK);
    if (!ok) return;
    const float2 xy = form_loc<true>(p, v, l, load_ref(p, P / (uint32_t)p.M), sH, sW);
    *reinterpret_cast<float2 *>(loc_out + 2 * (size_t)s) = xy;
    attn_out[s] = A;
    return;
  }
  const int64_t P = (int64_t)blockIdx.x * kBlock + threadIdx.x;
  if (P >= p.pairs) return;
  const float *z = p.logits + P * p.LK;
  float mx = -INFINITY;
  for (int i = 0; i < p.LK; ++i) mx = fmaxf(mx, z[i]);
  float sum = 0.0f;
  for (int i = 0; i < p.LK; ++i) sum += expf(z[i] - mx);
  const float2 st = make_float2(mx, 1.0f / sum);
  const float4 rf = load_ref(p, (uint32_t)(P / p.M));
  for (int i = 0; i < p.LK; ++i) {
    const int64_t s = P * p.LK + i;
    const float2 v = *reinterpret_cast<const float2 *>(p.offsets + 2 * s);
    *reinterpret_cast<float2 *>(loc_out + 2 * s) = form_loc<true>(p, v, (int)((uint32_t)i / K), rf, sH, sW);
    attn_out[s] = softmax_weight(z[i], st);
  }
}

// ------------------------------------------------------ tile binning (sort)

// Corner rows/columns of a sample that lie inside the map, as the index
// coordinate rule of sample_geometry defines them. Returns false when the
// sample contributes nothing.
struct Footprint {
  float x, y;        // index-space coordinate
  int y0, x0;        // floor corner
  bool r0, r1, c0, c1;  // rows y0, y0+1 and columns x0, x0+1 inside the map
};

__device__ __forceinline__ bool sample_footprint(float lx, float ly, int H, int W, Footprint &f) {
  const float x = fmaf(lx, (float)W, -0.5f);
  const float y = fmaf(ly, (float)H, -0.5f);
  const bool inside = (x >= -1.0f) && (x < (float)W) && (y >= -1.0f) && (y < (float)H);
  if (!inside) return false;
  f.x = x;
  f.y = y;
  f.x0 = (int)floorf(x);
  f.y0 = (int)floorf(y);
  f.c0 = f.x0 >= 0;
  f.c1 = f.x0 + 1 < W;
  f.r0 = f.y0 >= 0;
  f.r1 = f.y0 + 1 < H;
  return true;
}

__device__ __forceinline__ void load_tile_levels(const Params &p, int32_t *sH, int32_t *sW, int32_t *sS,
                                                 int32_t *sTW, int32_t *sToff) {
  const int tid = threadIdx.x;
  if (tid < kMaxLevels) {
    sH[tid] = p.lv.H[tid];
    sW[tid] = p.lv.W[tid];
    sS[tid] = p.lv.start[tid];
    sTW[tid] = p.lv.TW[tid];
    sToff[tid] = p.lv.toff[tid];
  }
}

constexpr int kBinCap = 2048;      // LDS tile counters of one (image, head)

// MODE 0 counts entries per tile; MODE 1 writes them in tile-major order as
// 16-byte records {pair, x, y, attn} (x, y: the sample's index-space
// coordinate), so the grad_value pass needs no access to loc or attn.
// Workgroup b covers image n, head m and queries [q0, q0 + qpb); its samples
// are the (q, l, k) of that range, at most 8 per thread. Tiles are numbered
// head-major: ((m * N + n) * TPI) + tile within the (image, head).
__device__ __forceinline__ void zero_split_body(const Params &p, int block, int nblocks, const int32_t *sH,
                                                const int32_t *sW, const int32_t *sS, const int32_t *sTW,
                                                const int32_t *sToff);

// LOCAL: a (image, head)'s tiles fit the LDS histogram (TPI <= kBinCap),
// otherwise every entry goes to the global counters; the two are separate
// instantiations so that neither path's waits fall into the other.
template <int MODE, bool LOCAL>
__global__ __launch_bounds__(kBlock) void bin_kernel(const Params p) {
  __shared__ uint32_t cnt[LOCAL ? kBinCap : 1];
  __shared__ uint32_t gbase[MODE == 1 && LOCAL ? kBinCap : 1];
  __shared__ int32_t sH[kMaxLevels], sW[kMaxLevels], sS[kMaxLevels], sTW[kMaxLevels], sToff[kMaxLevels];
  load_tile_levels(p, sH, sW, sS, sTW, sToff);
  const int tid = threadIdx.x;
  // 8 samples per thread in both passes (measured for the scatter pass: 8
  // beat 4 and 2 despite its register count; the longer per-tile runs also
  // help the grad_value pass)
  constexpr int NS = 8;
  const int qpb = MODE == 0 ? p.qpb0 : p.qpb;
  const int qblocks = (p.Lq + qpb - 1) / qpb;
  const int bin_blocks = p.N * p.M * qblocks;
  if (MODE == 1 && (int)blockIdx.x >= bin_blocks) {
    // the scatter launch carries extra workgroups that clear the split tiles
    __syncthreads();
    zero_split_body(p, (int)blockIdx.x - bin_blocks, (int)gridDim.x - bin_blocks, sH, sW, sS, sTW, sToff);
    return;
  }
  const int nm = blockIdx.x / qblocks;
  const int qb = blockIdx.x - nm * qblocks;
  const int n = nm / p.M, m = nm - n * p.M;
  const int q0 = qb * qpb;
  const int nsamp = (min(p.Lq, q0 + qpb) - q0) * p.LK;
  const uint32_t tbase = ((uint32_t)m * (uint32_t)p.N + (uint32_t)n) * (uint32_t)p.TPI;
  constexpr bool local = LOCAL;
  uint4 *rec_out = reinterpret_cast<uint4 *>(p.ws.entries);
  if (local)
    for (int i = tid; i < p.TPI; i += kBlock) cnt[i] = 0;
  __syncthreads();

  // The thread's samples: all their loads first (one round trip), then
  // the tile walk. Sample i is (query qi = i / LK, point pt = i % LK).
  const uint32_t lkmg = small_magic((uint32_t)p.LK), kmg = small_magic((uint32_t)p.K);
  // fused inputs formed here: the raw offsets and logits are read instead
  // (L*K a power of two <= 64, so a pair's samples are L*K aligned lanes)
  const bool form = MODE == 0 && p.form_inputs != 0;
  float2 xyv[NS];
  float av[NS];
#pragma unroll
  for (int r = 0; r < NS; ++r) {
    const int i = tid + r * kBlock;
    const bool ok = i < nsamp;
    const int qi = (int)small_div((uint32_t)(ok ? i : 0), lkmg);
    const int pt = (ok ? i : 0) - qi * p.LK;
    const int64_t sid = (((int64_t)n * p.Lq + q0 + qi) * p.M + m) * p.LK + pt;
    xyv[r] = ok ? *reinterpret_cast<const float2 *>((form ? p.offsets : p.loc) + 2 * sid) : make_float2(0.0f, 0.0f);
    av[r] = (MODE == 1 || form) && ok ? (form ? p.logits : p.attn)[sid] : 0.0f;
  }
  if (form) {
    // each sample's location and softmax weight, as fused_inputs_kernel forms
    // them (the same functions, the same lane positions within a pair's
    // segment), stored for the passes that follow
#pragma unroll
    for (int r = 0; r < NS; ++r) {
      const int i = tid + r * kBlock;
      const bool ok = i < nsamp;  // whole pairs drop out together
      const float A = segment_softmax(av[r], p.LK);
      if (!ok) continue;
      const int qi = (int)small_div((uint32_t)i, lkmg);
      const int pt = i - qi * p.LK;
      const int l = (int)small_div((uint32_t)pt, kmg);
      const int64_t q = (int64_t)n * p.Lq + q0 + qi;
      const int64_t sid = (q * p.M + m) * p.LK + pt;
      xyv[r] = form_loc<true>(p, xyv[r], l, load_ref(p, (uint32_t)q), sH, sW);
      *reinterpret_cast<float2 *>(p.ws.floc + 2 * sid) = xyv[r];
      p.ws.fattn[sid] = A;
    }
  }
  // Up to four tiles per sample, in fixed slots (dy, dx) so that every array
  // index below is a compile-time constant.
  uint4 rec[NS];
  uint32_t tl[NS][4], rk[NS][4];
  bool has[NS][4];
#pragma unroll
  for (int r = 0; r < NS; ++r) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      has[r][k] = false;
      tl[r][k] = 0;
      rk[r][k] = 0;
    }
    const int i = tid + r * kBlock;
    if (i >= nsamp) continue;
    const int qi = (int)small_div((uint32_t)i, lkmg);
    const int pt = i - qi * p.LK;
    const uint32_t P = (uint32_t)(((int64_t)n * p.Lq + q0 + qi) * p.M + m);
    const int l = (int)small_div((uint32_t)pt, kmg);
    const float2 xy = xyv[r];
    const float A = av[r];
    Footprint f;
    if (!sample_footprint(xy.x, xy.y, sH[l], sW[l], f)) continue;
    if (MODE == 1) rec[r] = make_uint4(P, __float_as_uint(f.x), __float_as_uint(f.y), __float_as_uint(A));
    // tile rows/columns touched by the in-map corners
    const int ya = f.r0 ? f.y0 : f.y0 + 1, yb = f.r1 ? f.y0 + 1 : f.y0;
    const int xa = f.c0 ? f.x0 : f.x0 + 1, xb = f.c1 ? f.x0 + 1 : f.x0;
    const int tya = ya >> 3, tyb = yb >> 3, txa = xa >> 3, txb = xb >> 3;
    const uint32_t lt = (uint32_t)sToff[l];
#pragma unroll
    for (int dy = 0; dy < 2; ++dy) {
#pragma unroll
      for (int dx = 0; dx < 2; ++dx) {
        if ((dy && tyb == tya) || (dx && txb == txa)) continue;
        const int k = dy * 2 + dx;
        const uint32_t t = lt + (uint32_t)((dy ? tyb : tya) * sTW[l] + (dx ? txb : txa));
        tl[r][k] = t;
        has[r][k] = true;
        if (local) {
          rk[r][k] = atomicAdd(&cnt[t], 1u);
        } else if (MODE == 0) {
          atomicAdd(p.ws.tile_count + tbase + t, 1u);
        } else {
          rec_out[atomicAdd(p.ws.tile_cursor + tbase + t, 1u)] = rec[r];
        }
      }
    }
  }
  if (!local) return;
  __syncthreads();
  if constexpr (MODE == 0) {
    for (int i = tid; i < p.TPI; i += kBlock) {
      const uint32_t c = cnt[i];
      if (c) atomicAdd(p.ws.tile_count + tbase + i, c);
    }
  } else {
    // reserve each tile's run once per workgroup, then write the records
    // (every slot's run start read first, unconditionally, so that the reads
    // issue together instead of one wait per record)
    for (int i = tid; i < p.TPI; i += kBlock) {
      const uint32_t c = cnt[i];
      if (c) gbase[i] = atomicAdd(p.ws.tile_cursor + tbase + i, c);
    }
    __syncthreads();
    uint32_t dst[NS][4];
#pragma unroll
    for (int r = 0; r < NS; ++r)
#pragma unroll
      for (int k = 0; k < 4; ++k) dst[r][k] = gbase[has[r][k] ? tl[r][k] : 0u] + rk[r][k];
    if (p.ws.entries_bytes != 0) {
      // buffer stores with 32-bit offsets, issued back to back; an absent
      // slot's offset lies past the entries region (whose size the resource
      // carries), so the hardware drops that store
      const __amdgpu_buffer_rsrc_t rr = make_rsrc(rec_out, p.ws.entries_bytes);
#pragma unroll
      for (int r = 0; r < NS; ++r) {
        const u32x4 d = {rec[r].x, rec[r].y, rec[r].z, rec[r].w};
#pragma unroll
        for (int k = 0; k < 4; ++k)
          __builtin_amdgcn_raw_buffer_store_b128(d, rr, has[r][k] ? dst[r][k] * 16u : kEntriesOob, 0, 0);
      }
    } else {
#pragma unroll
      for (int r = 0; r < NS; ++r)
#pragma unroll
        for (int k = 0; k < 4; ++k)
          if (has[r][k]) rec_out[dst[r][k]] = rec[r];
    }
  }
}

// Exclusive scan of the tile counts (one workgroup of 1024 threads, each
// owning a run of consecutive tiles) and the list of grad_value work items:
// a tile gives ceil(count / kPartEntries) items, at least one (an empty tile's
// item writes its zeros). Tiles with several items are listed, in tile order
// (a third prefix sum gives each its slot), so that they can be zeroed first.
constexpr int kScanSplitCap = 2048;  // split tiles whose items the whole scan workgroup writes

__global__ __launch_bounds__(1024) void scan_kernel(const Params p) {
  __shared__ uint32_t wsum_c[16], wsum_q[16], wsum_s[16], wsum_u[16];
  // split tile i: tile, first entry, entry count, first item (before the
  // list's reversal); filled by the tiles' owners, read by every thread
  __shared__ uint4 ssplit[kScanSplitCap];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int per = (p.T + 1023) / 1024;
  const int t0 = tid * per, t1 = min(p.T, t0 + per);
  auto parts_of = [&](uint32_t c) -> uint32_t {
    return max(1u, (c + kPartEntries - 1) / kPartEntries);
  };
  // per thread, over its run of tiles: entries, work items of split tiles,
  // split tiles, single-item tiles
  uint32_t rc = 0, rq = 0, rs = 0, ru = 0;
  for (int t = t0; t < t1; ++t) {
    const uint32_t c = p.ws.tile_count[t];
    const uint32_t parts = parts_of(c);
    rc += c;
    if (parts > 1) {
      rq += parts;
      ++rs;
    } else {
      ++ru;
    }
  }
  uint32_t ic = rc, iq = rq, is = rs, iu = ru;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t yc = __shfl_up(ic, o), yq = __shfl_up(iq, o), ys = __shfl_up(is, o), yu = __shfl_up(iu, o);
    if (lane >= o) {
      ic += yc;
      iq += yq;
      is += ys;
      iu += yu;
    }
  }
  if (lane == 63) {
    wsum_c[wave] = ic;
    wsum_q[wave] = iq;
    wsum_s[wave] = is;
    wsum_u[wave] = iu;
  }
  __syncthreads();
  uint32_t oc = 0, oq = 0, os = 0, ou = 0, tc = 0, tq = 0, ts = 0, tu = 0;
#pragma unroll
  for (int w = 0; w < 16; ++w) {
    if (w < wave) {
      oc += wsum_c[w];
      oq += wsum_q[w];
      os += wsum_s[w];
      ou += wsum_u[w];
    }
    tc += wsum_c[w];
    tq += wsum_q[w];
    ts += wsum_s[w];
    tu += wsum_u[w];
  }
  uint32_t start = oc + ic - rc, qb = oq + iq - rq, sb = os + is - rs, ub = ou + iu - ru;
  uint4 *items = reinterpret_cast<uint4 *>(p.ws.work_item);
  // Work items: every split tile's items first (the longest work starts
  // first), coarse levels first (tiles in reverse order), then one item per
  // remaining tile, also in reverse tile order. With at most kScanSplitCap
  // split tiles their items are written by the whole workgroup (a crowded
  // tile has tens of items, all of one thread's run otherwise).
  const bool shared_split = ts <= (uint32_t)kScanSplitCap;
  for (int t = t0; t < t1; ++t) {
    const uint32_t c = p.ws.tile_count[t];
    const uint32_t parts = parts_of(c);
    p.ws.tile_start[t] = start;
    p.ws.tile_cursor[t] = start;
    if (parts > 1) {
      if (shared_split) {
        ssplit[sb] = make_uint4((uint32_t)t, start, c, qb);
      } else {
        for (uint32_t k = 0; k < parts; ++k) {
          const uint32_t e0 = start + k * kPartEntries;
          items[tq - 1 - (qb + k)] = make_uint4((uint32_t)t, e0, min(e0 + (uint32_t)kPartEntries, start + c), 1u);
        }
      }
      p.ws.split_list[sb++] = (uint32_t)t;
      qb += parts;
    } else {
      items[tq + tu - 1 - ub] = make_uint4((uint32_t)t, start, start + c, 0u);
      ++ub;
    }
    start += c;
  }
  if (shared_split) {
    __syncthreads();
    // item j of the split group belongs to the last split tile whose first
    // item is <= j (first items ascend with the split index)
    for (uint32_t j = (uint32_t)tid; j < tq; j += 1024u) {
      uint32_t lo = 0, hi = ts - 1;
      while (lo < hi) {
        const uint32_t mid = (lo + hi + 1) >> 1;
        if (ssplit[mid].w <= j) lo = mid; else hi = mid - 1;
      }
      const uint4 sp = ssplit[lo];
      const uint32_t e0 = sp.y + (j - sp.w) * kPartEntries;
      items[tq - 1 - j] = make_uint4(sp.x, e0, min(e0 + (uint32_t)kPartEntries, sp.y + sp.z), 1u);
    }
  }
  if (tid == 0) {
    p.ws.tile_start[p.T] = tc;
    p.ws.tile_count[p.T] = ts;  // number of split tiles
    *p.ws.n_work = tq + tu;
  }
}

__device__ __forceinline__ void decode_tile(const Params &p, uint32_t t, const int32_t *sToff, const int32_t *sTW,
                                            int &n, int &m, int &l, int &ty, int &tx) {
  const int mn = (int)(t / (uint32_t)p.TPI);
  const int r = (int)(t - (uint32_t)mn * (uint32_t)p.TPI);
  m = mn / p.N;
  n = mn - m * p.N;
  l = 0;
  for (int k = 1; k < p.L; ++k)
    if (sToff[k] <= r) l = k;
  const int tl = r - sToff[l];
  ty = tl / sTW[l];
  tx = tl - ty * sTW[l];
}

// Zeroes the pixels of tiles whose entries are split over several work items
// (their partial sums are added with atomics): split tiles i = block,
// block + nblocks, ... of the list the scan wrote.
__device__ __forceinline__ void zero_split_body(const Params &p, int block, int nblocks, const int32_t *sH,
                                                const int32_t *sW, const int32_t *sS, const int32_t *sTW,
                                                const int32_t *sToff) {
  const uint32_t nsplit = p.ws.tile_count[p.T];
  for (uint32_t i = (uint32_t)block; i < nsplit; i += (uint32_t)nblocks) {
    int n, m, l, ty, tx;
    decode_tile(p, p.ws.split_list[i], sToff, sTW, n, m, l, ty, tx);
    for (int k = threadIdx.x; k < kTilePix * p.D; k += kBlock) {
      const int pix = k / p.D, c = k - pix * p.D;
      const int py = ty * kTile + (pix >> 3), px = tx * kTile + (pix & 7);
      if (py < sH[l] && px < sW[l])
        p.grad_value[(((int64_t)n * p.S + sS[l] + py * sW[l] + px) * p.M + m) * p.D + c] = 0.0f;
    }
  }
}

// grad_value of one work item (blockIdx.x, last items first: the list ends
// with the coarse levels' crowded tiles) and one group of up to 64 channels
// (blockIdx.y). The item's entries (at most kPartEntries = 4 per thread) are
// read once; each corner that falls in the tile is bucketed by pixel with LDS
// integer atomics into a (grad_out row, weight) list; then thread (pixel, slice) sums
// its pixel's contributions to CS channels in registers, reading the grad_out
// row slices straight from memory with several loads in flight.
constexpr size_t kGvSmem = 4 * kPartEntries * sizeof(uint2) + (2 * kTilePix + 1) * 4 + 5 * kMaxLevels * 4;

// Sums w * grad_out[pair, channels] over the list entries [jb, je) of one
// pixel into acc, U entries in flight. VECP: 16-byte loads of interleaved
// pieces (channel c0 + (c / VG) * 4 * VG + c % VG, the four threads of a pixel
// covering whole 64-byte segments); otherwise element loads of the cnum
// channels from c0 on. Rows of absent slots (and channels past cnum) read past
// the buffer, which returns zeros; their weight is 0 too.
template <typename T, int CS, bool VECP>
__device__ __forceinline__ void gv_accumulate(const uint2 *lst, uint32_t jb, uint32_t je,
                                              __amdgpu_buffer_rsrc_t ro, uint32_t c0, int cnum,
                                              float (&acc)[CS]) {
  constexpr int VG = 16 / T::size;
  // entries in flight per thread (measured: 8 beats 4 up to 8 channels per
  // thread, most for bf16 rows, one 16-byte load per entry; with 16 channels
  // 8 entries cost occupancy); slots past je read at most 56 bytes beyond the
  // list, inside the tile counters that follow it in LDS
  constexpr int U = CS >= 16 ? 4 : 8;
  static_assert((U - 1) * sizeof(uint2) <= kTilePix * sizeof(uint32_t),
                "the list over-read must stay inside the tile counters");
  for (uint32_t j = jb; j < je; j += U) {
    float g[U][CS];
    float w[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      // read unconditionally (slots past je read the LDS words that follow
      // the list, which the workgroup owns) so the reads issue together; an
      // absent slot is masked bitwise rather than selected, so that the
      // compiler cannot turn its read into a predicated one that waits alone
      const uint32_t keep = j + u < je ? 0xffffffffu : 0u;
      const uint2 r2 = lst[j + u];
      w[u] = __uint_as_float(r2.y & keep);
      const uint32_t base = (r2.x & keep) + (keep ? c0 : kOobElem);
      if constexpr (VECP) {
#pragma unroll
        for (int q = 0; q < CS / VG; ++q)
          load_vals<T, VG>(ro, (base + (uint32_t)(q * 4 * VG)) * (uint32_t)T::size,
                           *reinterpret_cast<float(*)[VG]>(&g[u][q * VG]));
      } else {
#pragma unroll
        for (int c = 0; c < CS; ++c)
          load_vals<T, 1>(ro, (c < cnum ? base + (uint32_t)c : kOobElem) * (uint32_t)T::size,
                          *reinterpret_cast<float(*)[1]>(&g[u][c]));
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int c = 0; c < CS; ++c) acc[c] = fmaf(w[u], g[u][c], acc[c]);
  }
}

template <typename T, int CS>
__device__ __forceinline__ void gv_body(const Params &p, uint32_t bx, int cgroup, unsigned char *smem) {
  constexpr int VG = 16 / T::size;  // elements of one 16-byte grad_out load
  constexpr int kEPT = kPartEntries / kBlock;  // entries per thread
  uint2 *lst = reinterpret_cast<uint2 *>(smem);  // (grad_out row offset, weight bits), pixel-major
  uint32_t *cnt = reinterpret_cast<uint32_t *>(smem + 4 * kPartEntries * sizeof(uint2));
  uint32_t *off = cnt + kTilePix;
  int32_t *sH = reinterpret_cast<int32_t *>(off + kTilePix + 1);
  int32_t *sW = sH + kMaxLevels, *sS = sW + kMaxLevels, *sTW = sS + kMaxLevels, *sToff = sTW + kMaxLevels;
  // the item descriptor and the item count are loaded together (the slot
  // exists for every block of the grid; past n_work it is ignored)
  const uint4 item = reinterpret_cast<const uint4 *>(p.ws.work_item)[bx];
  const uint32_t nwork = *p.ws.n_work;
  if (bx >= nwork) return;
  load_tile_levels(p, sH, sW, sS, sTW, sToff);
  const int tid = threadIdx.x;
  if (tid < kTilePix) cnt[tid] = 0;
  const uint32_t t = item.x, e0 = item.y, e1 = item.z;
  const bool split = item.w != 0;
  const uint4 *recs = reinterpret_cast<const uint4 *>(p.ws.entries);
  uint4 rec[kEPT];
#pragma unroll
  for (int r = 0; r < kEPT; ++r) {
    const uint32_t e = e0 + (uint32_t)(tid + r * kBlock);
    rec[r] = e < e1 ? recs[e] : make_uint4(0xffffffffu, 0, 0, 0);
  }
  __syncthreads();
  int n, m, l, ty, tx;
  decode_tile(p, t, sToff, sTW, n, m, l, ty, tx);
  // the item's tile and level are uniform: scalar registers, so that the
  // per-corner tests below wait on nothing (LDS-loaded values would make the
  // compiler wait for every LDS atomic issued since)
  l = __builtin_amdgcn_readfirstlane(l);
  ty = __builtin_amdgcn_readfirstlane(ty);
  tx = __builtin_amdgcn_readfirstlane(tx);
  const int H = __builtin_amdgcn_readfirstlane(sH[l]), W = __builtin_amdgcn_readfirstlane(sW[l]);

  // corners of this thread's entries that fall in the tile, ranked per pixel
  uint32_t cpix[kEPT][4], crk[kEPT][4];
  float cw[kEPT][4];
  bool cin[kEPT][4];
#pragma unroll
  for (int r = 0; r < kEPT; ++r) {
#pragma unroll
    for (int c = 0; c < 4; ++c) cin[r][c] = false;
    if (rec[r].x == 0xffffffffu) continue;
    const float x = __uint_as_float(rec[r].y), y = __uint_as_float(rec[r].z), A = __uint_as_float(rec[r].w);
    const float xf = floorf(x), yf = floorf(y);
    const float a = x - xf, b = y - yf;
    const int x0 = (int)xf, y0 = (int)yf;
    const float wa[2] = {1.0f - a, a}, wb[2] = {1.0f - b, b};
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int cy = y0 + (c >> 1), cx = x0 + (c & 1);
      if (cy < 0 || cy >= H || cx < 0 || cx >= W || (cy >> 3) != ty || (cx >> 3) != tx) continue;
      cin[r][c] = true;
      cpix[r][c] = (uint32_t)((cy & 7) * kTile + (cx & 7));
      cw[r][c] = A * wb[c >> 1] * wa[c & 1];
      crk[r][c] = atomicAdd(&cnt[cpix[r][c]], 1u);
    }
  }
  __syncthreads();
  if (tid < 64) {
    uint32_t v = cnt[tid];
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const uint32_t y = __shfl_up(v, o);
      if (tid >= o) v += y;
    }
    off[tid + 1] = v;
    if (tid == 0) off[0] = 0;
  }
  __syncthreads();
#pragma unroll
  for (int r = 0; r < kEPT; ++r)
#pragma unroll
    for (int c = 0; c < 4; ++c)
      if (cin[r][c])
        lst[off[cpix[r][c]] + crk[r][c]] = make_uint2(rec[r].x * (uint32_t)p.D, __float_as_uint(cw[r][c]));
  __syncthreads();

  const int c0 = cgroup * kChanGroup;
  const int Dc = min(kChanGroup, p.D - c0);
  const int Cs = (Dc + 3) >> 2;  // channels per thread (<= CS)
  const int pix = tid >> 2, slice = tid & 3;
  const int cbeg = c0 + slice * Cs;               // first channel of this thread
  const int cnum = max(0, min(Cs, Dc - slice * Cs));  // channels it owns
  const bool vec = p.gvec != 0 && Cs == CS && (Cs % VG) == 0;
  // Channel of this thread's accumulator c. With 16-byte loads the four
  // threads of a pixel take interleaved 16-byte pieces of the row, so each
  // load instruction reads whole 64-byte segments; otherwise each thread owns
  // a contiguous run of Cs channels.
  auto chan = [&](int c) { return vec ? c0 + (c / VG) * 4 * VG + slice * VG + (c % VG) : cbeg + c; };
  const __amdgpu_buffer_rsrc_t ro = make_rsrc(p.grad_out, (uint32_t)(p.pairs * p.D) * (uint32_t)T::size);
  float acc[CS];
#pragma unroll
  for (int c = 0; c < CS; ++c) acc[c] = 0.0f;
  const uint32_t jb = off[pix], je = off[pix + 1];
  if constexpr (CS >= VG) {
    if (vec) {
      gv_accumulate<T, CS, true>(lst, jb, je, ro, (uint32_t)(c0 + slice * VG), CS, acc);
    } else {
      gv_accumulate<T, CS, false>(lst, jb, je, ro, (uint32_t)cbeg, cnum, acc);
    }
  } else {
    gv_accumulate<T, CS, false>(lst, jb, je, ro, (uint32_t)cbeg, cnum, acc);
  }

  const int64_t row0 = (int64_t)n * p.S + sS[l];
  if (split) {
    // Partial sums of a split tile: add them channel-contiguously, so that one
    // atomic instruction covers whole 64-byte segments of a pixel's row.
    __syncthreads();
    float *stage = reinterpret_cast<float *>(lst);
    const int DcP = Cs * 4;
#pragma unroll
    for (int c = 0; c < CS; ++c)
      if (c < Cs) stage[pix * DcP + chan(c) - c0] = acc[c];
    __syncthreads();
    for (int i = tid; i < kTilePix * Dc; i += kBlock) {
      const int q = i / Dc, c = i - q * Dc;
      const int py = ty * kTile + (q >> 3), px = tx * kTile + (q & 7);
      if (py < H && px < W)
        atomicAdd(p.grad_value + ((row0 + py * W + px) * p.M + m) * p.D + c0 + c, stage[q * DcP + c]);
    }
    return;
  }
  const int py = ty * kTile + (pix >> 3), px = tx * kTile + (pix & 7);
  if (py >= H || px >= W) return;
  float *dst = p.grad_value + ((row0 + py * W + px) * p.M + m) * p.D;
  if (vec && (reinterpret_cast<uintptr_t>(p.grad_value) & 15u) == 0) {
#pragma unroll
    for (int q = 0; q < CS / 4; ++q)
      *reinterpret_cast<float4 *>(dst + chan(4 * q)) =
          make_float4(acc[4 * q], acc[4 * q + 1], acc[4 * q + 2], acc[4 * q + 3]);
    return;
  }
#pragma unroll
  for (int c = 0; c < CS; ++c)
    if (c < cnum) dst[chan(c)] = acc[c];
}

template <typename T, int CS>
__global__ __launch_bounds__(kBlock) void gv_kernel(const Params p) {
  __shared__ __align__(16) unsigned char smem[kGvSmem];
  gv_body<T, CS>(p, blockIdx.x, blockIdx.y, smem);
}

// The grad_value work items and the sample-gradient blocks in one launch: the
// two are independent, so the sample gradients fill the machine while the
// crowded tiles' items finish. Blocks [0, gv_blocks) are grad_value items
// (one channel group when D <= 64), the rest run bwd_sample_body.
template <typename T, int VEC, int NCG, int LPP, int CS, bool FUSE>
__global__ __launch_bounds__(kBlock) void bwd_fused_kernel(const Params p) {
  constexpr size_t kSmem = kGvSmem > sample_smem<FUSE>() ? kGvSmem : sample_smem<FUSE>();
  __shared__ __align__(16) unsigned char smem[kSmem];
  if ((int)blockIdx.x < p.gv_blocks)
    gv_body<T, CS>(p, blockIdx.x, 0, smem);
  else
    bwd_sample_body<T, VEC, NCG, LPP, FUSE>(p, (int)blockIdx.x - p.gv_blocks, (int)gridDim.x - p.gv_blocks,
                                            smem);
}

// Reference gradient of each query (fused inputs): the sum over its M pairs of
// the per-pair sums that the sample pass left in the workspace, in a fixed
// order. Thread i owns component i % ref_dim of query i / ref_dim.
__global__ __launch_bounds__(kBlock) void ref_grad_kernel(const Params p) {
  const int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x;
  const int64_t nq = p.pairs / p.M;
  if (i >= nq * p.ref_dim) return;
  const int64_t q = i / p.ref_dim;
  const int c = (int)(i - q * p.ref_dim);
  float sum = 0.0f;
  for (int m = 0; m < p.M; ++m) sum += p.ws.ref_part[(q * p.M + m) * 4 + c];
  p.grad_ref[i] = sum;
}

__global__ __launch_bounds__(kBlock) void zero_u32_kernel(uint32_t *ptr, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x;
  if (i < n) ptr[i] = 0u;
}

// ------------------------------------------------------------- zero fill

__global__ __launch_bounds__(kBlock) void zero_kernel(float *ptr, int64_t n) {
  const int64_t i = ((int64_t)blockIdx.x * kBlock + threadIdx.x) * 4;
  if (i + 3 < n) {
    *reinterpret_cast<float4 *>(ptr + i) = make_float4(0.f, 0.f, 0.f, 0.f);
  } else {
    for (int64_t k = i; k < n; ++k) ptr[k] = 0.0f;
  }
}

__global__ __launch_bounds__(kBlock) void zero_kernel_unaligned(float *ptr, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x;
  if (i < n) ptr[i] = 0.0f;
}

// --------------------------------------------------------------- dispatch

using KernelFn = void (*)(Params);

template <typename T, int VEC, bool FUSE>
KernelFn pick(bool fwd, int ncg, int lpp) {
  // Compile-time lane counts for the common 16-byte shapes (fp32 D=32 and
  // bf16 D=32), a runtime lane count otherwise.
  if (ncg == 1 && lpp == 8 && VEC * T::size == 16)
    return fwd ? fwd_kernel<T, VEC, 1, 8, FUSE> : bwd_sample_kernel<T, VEC, 1, 8, FUSE>;
  if (ncg == 1 && lpp == 4 && VEC * T::size == 16)
    return fwd ? fwd_kernel<T, VEC, 1, 4, FUSE> : bwd_sample_kernel<T, VEC, 1, 4, FUSE>;
  switch (ncg) {
    case 1: return fwd ? fwd_kernel<T, VEC, 1, 0, FUSE> : bwd_sample_kernel<T, VEC, 1, 0, FUSE>;
    case 2: return fwd ? fwd_kernel<T, VEC, 2, 0, FUSE> : bwd_sample_kernel<T, VEC, 2, 0, FUSE>;
    case 4: return fwd ? fwd_kernel<T, VEC, 4, 0, FUSE> : bwd_sample_kernel<T, VEC, 4, 0, FUSE>;
    default: break;
  }
  if constexpr (VEC == 1) {
    if (ncg == 8) return fwd ? fwd_kernel<T, 1, 8, 0, FUSE> : bwd_sample_kernel<T, 1, 8, 0, FUSE>;
    if (ncg == 16) return fwd ? fwd_kernel<T, 1, 16, 0, FUSE> : bwd_sample_kernel<T, 1, 16, 0, FUSE>;
  }
  return nullptr;
}

template <bool FUSE>
KernelFn select_t(bool fwd, DType dt, const LaunchShape &s) {
  if (dt == DType::F32) {
    switch (s.vec) {
      case 4: return pick<F32, 4, FUSE>(fwd, s.ncg, s.lpp);
      case 2: return pick<F32, 2, FUSE>(fwd, s.ncg, s.lpp);
      case 1: return pick<F32, 1, FUSE>(fwd, s.ncg, s.lpp);
    }
  } else {
    switch (s.vec) {
      case 8: return pick<BF16, 8, FUSE>(fwd, s.ncg, s.lpp);
      case 4: return pick<BF16, 4, FUSE>(fwd, s.ncg, s.lpp);
      case 2: return pick<BF16, 2, FUSE>(fwd, s.ncg, s.lpp);
      case 1: return pick<BF16, 1, FUSE>(fwd, s.ncg, s.lpp);
    }
  }
  return nullptr;
}

KernelFn select(bool fwd, bool fuse, DType dt, const LaunchShape &s) {
  return fuse ? select_t<true>(fwd, dt, s) : select_t<false>(fwd, dt, s);
}

template <typename T>
KernelFn pick_gv(int cs) {
  switch (cs) {
    case 1: return gv_kernel<T, 1>;
    case 2: return gv_kernel<T, 2>;
    case 4: return gv_kernel<T, 4>;
    case 8: return gv_kernel<T, 8>;
    default: return gv_kernel<T, 16>;
  }
}

hipError_t launch_fn(const void *fn, int64_t blocks, int threads, int gy, Params &p, hipStream_t stream) {
  if (blocks <= 0) return hipSuccess;
  if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
  void *args[] = {&p};
  return hipLaunchKernel(fn, dim3((unsigned)blocks, (unsigned)gy), dim3(threads), args, 0, stream);
}

// Lane mapping and chunking of the per-sample passes (forward and the
// backward's sample gradients). The backward's sample pass takes head-major
// workgroups: its value rows then stay in the L2 of the XCD that works on the
// head (the inputs are warm after the binning passes). The forward, which
// meets value cold, keeps pair-major workgroups, whose XCDs read whole pixel
// rows (all heads) from HBM.
void set_sample_shape(Params &p, const LaunchShape &s, bool backward) {
  p.lpp = s.lpp;
  const int ppb = kBlock / s.lpp;
  p.pc = min(p.LK, max(1, kDescCap / (ppb + 1)));
  const bool pow2 = (p.LK & (p.LK - 1)) == 0;
  p.seg_softmax = p.ref_dim != 0 && pow2 && p.LK <= 64 && p.LK <= p.pc ? 1 : 0;
  p.head_major = backward ? 1 : 0;
}

// Workgroups of a per-sample pass.
int64_t sample_blocks(const Params &p, int ppb) {
  if (p.head_major) return (int64_t)p.N * p.M * ((p.Lq + ppb - 1) / ppb);
  return (p.pairs + ppb - 1) / ppb;
}

hipError_t launch_pairs(bool fwd, const Params &p_in, DType dt, const LaunchShape &s, hipStream_t stream) {
  KernelFn fn = select(fwd, p_in.ref_dim != 0, dt, s);
  if (!fn) return hipErrorInvalidValue;
  Params p = p_in;
  set_sample_shape(p, s, !fwd);
  const int64_t blocks = sample_blocks(p, kBlock / s.lpp);
  return launch_fn(reinterpret_cast<const void *>(fn), blocks, kBlock, 1, p, stream);
}

}  // namespace

LaunchShape choose_shape(int D, DType dt, uintptr_t align_bits, int64_t pairs) {
  LaunchShape s = choose_shape_widest(D, dt, align_bits);
  // Small launches (decoder-sized): spread the pairs over more workgroups by
  // giving each lane fewer channels, until there are ~2 workgroups per CU.
  while (s.vec > 1 && s.ncg == 1 && pairs * s.lpp < 512 * (int64_t)kBlock) {
    const int vec = s.vec / 2, nvec = D / vec;
    int lpp = 1;
    while (lpp < nvec && lpp < 64) lpp *= 2;
    if (lpp * 1 < nvec) break;  // would need several channel groups per lane
    s = LaunchShape{vec, lpp, 1};
  }
  return s;
}

LaunchShape choose_shape_widest(int D, DType dt, uintptr_t align_bits) {
  const int esz = dt == DType::F32 ? 4 : 2;
  // Widest access (16, 8, 4, 2 bytes) that divides a head's channels and the
  // pointers' alignment, while one pair fits in 64 lanes x 4 groups.
  for (int bytes = 16; bytes >= esz; bytes /= 2) {
    const int vec = bytes / esz;
    if (D % vec != 0 || (align_bits % (uintptr_t)bytes) != 0) continue;
    const int nvec = D / vec;
    if (nvec > 64 * 4) continue;
    int lpp = 1;
    while (lpp < nvec && lpp < 64) lpp *= 2;
    int ncg = 1;
    while (ncg * lpp < nvec) ncg *= 2;
    return LaunchShape{vec, lpp, ncg};
  }
  // Single-element lanes with up to 16 channel groups (D <= 1024).
  int ncg = 1;
  while (ncg * 64 < D) ncg *= 2;
  int lpp = 1;
  while (lpp < D && lpp < 64) lpp *= 2;
  return LaunchShape{1, lpp, ncg};
}

void fill_tiles(LevelTable &lv, const int64_t *spatial_shapes, int64_t L, int32_t *TPI) {
  int32_t acc = 0;
  for (int64_t l = 0; l < L; ++l) {
    lv.TH[l] = (int32_t)((spatial_shapes[2 * l] + kTile - 1) / kTile);
    lv.TW[l] = (int32_t)((spatial_shapes[2 * l + 1] + kTile - 1) / kTile);
    lv.toff[l] = acc;
    acc += lv.TH[l] * lv.TW[l];
  }
  *TPI = acc;
}

WorkspaceLayout workspace_layout(const int64_t *spatial_shapes, int64_t L, int64_t nimg, int64_t M, int64_t Lq,
                                 int64_t K, bool fused) {
  int64_t tpi = 0;
  for (int64_t l = 0; l < L; ++l)
    tpi += ((spatial_shapes[2 * l] + kTile - 1) / kTile) * ((spatial_shapes[2 * l + 1] + kTile - 1) / kTile);
  WorkspaceLayout w{};
  w.T = nimg * M * tpi;
  w.Emax = 4 * nimg * Lq * M * L * K;
  // grad_value work items, rounded up to the fused launch's block granularity
  w.Wmax = (w.T + (w.Emax + kPartEntries - 1) / kPartEntries + 7) & ~(int64_t)7;
  auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
  size_t o = 0;
  w.off_count = o;   o = up(o + 4 * (size_t)(w.T + 8));
  w.off_cursor = o;  o = up(o + 4 * (size_t)w.T);
  w.off_start = o;   o = up(o + 4 * (size_t)(w.T + 1));
  w.off_witem = o;   o = up(o + 16 * (size_t)w.Wmax);
  w.off_nwork = o;   o = up(o + 4);
  w.off_split = o;   o = up(o + 4 * (size_t)w.T);
  w.off_entries = o; o = up(o + 16 * (size_t)w.Emax);
  // fused inputs: reference-gradient sums per pair, the formed locations and
  // weights per sample
  w.off_refpart = o; o = up(o + (fused ? 16 * (size_t)(nimg * Lq * M) : 0));
  w.off_floc = o;    o = up(o + (fused ? 8 * (size_t)(nimg * Lq * M * L * K) : 0));
  w.off_fattn = o;   o = up(o + (fused ? 4 * (size_t)(nimg * Lq * M * L * K) : 0));
  w.bytes = o;
  return w;
}

hipError_t launch_forward(const Params &p, DType dt, const LaunchShape &s, hipStream_t stream) {
  return launch_pairs(true, p, dt, s, stream);
}

hipError_t launch_backward(const Params &p_in, DType dt, const LaunchShape &s, hipStream_t stream) {
  Params p = p_in;
  p.qpb = max(1, 2048 / p.LK);
  p.qpb0 = max(1, 2048 / p.LK);
  set_sample_shape(p, s, true);
  const bool fuse = p.ref_dim != 0;
  hipError_t e;
  // Sparse launches (few samples per 8x8 value tile, e.g. decoder queries): a
  // tile sort would cost more than it saves; grad_value is zero-filled and
  // the sample pass adds each corner's contribution with float atomics.
  p.scatter = (int64_t)p.Lq * p.LK < 32 * (int64_t)p.TPI ? 1 : 0;
  // 0. fused inputs: every sample's location and weight, formed once into
  //    the workspace, are the loc and attn of the passes below (formed by
  //    the counting pass itself on the dense route when a pair's L*K samples
  //    fit one lane segment)
  p.form_inputs = fuse && !p.scatter && (p.LK & (p.LK - 1)) == 0 && p.LK <= 64 ? 1 : 0;
  if (fuse && !p.form_inputs) {
    Params q = p;
    q.seg_softmax = (p.LK & (p.LK - 1)) == 0 && p.LK <= 64 ? 1 : 0;
    const int64_t items = q.seg_softmax ? p.pairs * p.LK : p.pairs;
    float *lo = p.ws.floc, *ao = p.ws.fattn;
    void *args[] = {&q, &lo, &ao};
    const int64_t blocks = (items + kBlock - 1) / kBlock;
    if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
    e = hipLaunchKernel(reinterpret_cast<const void *>(fused_inputs_kernel), dim3((unsigned)blocks), dim3(kBlock),
                        args, 0, stream);
    if (e != hipSuccess) return e;
    p.loc = p.ws.floc;
    p.attn = p.ws.fattn;
  }
  if (fuse && p.form_inputs) {
    p.loc = p.ws.floc;  // written by the counting pass, read by the passes after it
    p.attn = p.ws.fattn;
  }
  if (p.scatter) {
    if ((e = launch_zero(p.grad_value, (int64_t)p.N * p.S * p.M * p.D, stream)) != hipSuccess) return e;
    if ((e = launch_pairs(false, p, dt, s, stream)) != hipSuccess) return e;
  } else {
    // 16-byte grad_out loads in the grad_value pass when rows and pointer allow
    p.gvec = (s.vec * (dt == DType::F32 ? 4 : 2)) == 16 ? 1 : 0;
    // 1. tile counters and the split-tile counter
    {
      uint32_t *ptr = p.ws.tile_count;
      int64_t n = p.T + 8;
      void *args[] = {&ptr, &n};
      e = hipLaunchKernel(reinterpret_cast<const void *>(zero_u32_kernel),
                          dim3((unsigned)((n + kBlock - 1) / kBlock)), dim3(kBlock), args, 0, stream);
      if (e != hipSuccess) return e;
    }
    // 2. counting sort of (sample, tile) entries; the scatter launch also clears
    //    the tiles whose grad_value is summed over several work items
    const int64_t bin_blocks = (int64_t)p.N * p.M * ((p.Lq + p.qpb - 1) / p.qpb);
    const int64_t bin0_blocks = (int64_t)p.N * p.M * ((p.Lq + p.qpb0 - 1) / p.qpb0);
    const bool local = p.TPI <= kBinCap;
    const void *bin0 = local ? reinterpret_cast<const void *>(bin_kernel<0, true>)
                             : reinterpret_cast<const void *>(bin_kernel<0, false>);
    const void *bin1 = local ? reinterpret_cast<const void *>(bin_kernel<1, true>)
                             : reinterpret_cast<const void *>(bin_kernel<1, false>);
    if ((e = launch_fn(bin0, bin0_blocks, kBlock, 1, p, stream)) != hipSuccess) return e;
    if ((e = launch_fn(reinterpret_cast<const void *>(scan_kernel), 1, 1024, 1, p, stream)) != hipSuccess) return e;
    if ((e = launch_fn(bin1, bin_blocks + 256, kBlock, 1, p, stream)) != hipSuccess) return e;
    // 3. grad_value per tile, and grad_attn / grad_loc per sample
    const int64_t wmax = p.T + (4 * p.pairs * p.LK + kPartEntries - 1) / kPartEntries;
    const int Dc = min(kChanGroup, p.D);
    const int cs_need = (Dc + 3) / 4;
    int cs = 1;
    while (cs < cs_need) cs *= 2;
    const int groups = (p.D + kChanGroup - 1) / kChanGroup;
    const int ppb = kBlock / s.lpp;
    const int64_t nsample = sample_blocks(p, ppb);
    const bool hot_f32 = dt == DType::F32 && s.vec == 4 && s.lpp == 8 && s.ncg == 1 && cs == 8;
    const bool hot_bf16 = dt == DType::BF16 && s.vec == 8 && s.lpp == 4 && s.ncg == 1 && cs == 8;
    // grad_value blocks rounded to a multiple of 8 so that the sample blocks'
    // XCD-aware renumbering sees the hardware's block % 8 placement
    const int64_t gvb = (wmax + 7) & ~(int64_t)7;
    if ((hot_f32 || hot_bf16) && groups == 1 && gvb + nsample <= 0x7fffffff) {
      p.gv_blocks = (int32_t)gvb;
      const void *fn;
      if (hot_f32)
        fn = fuse ? reinterpret_cast<const void *>(bwd_fused_kernel<F32, 4, 1, 8, 8, true>)
                  : reinterpret_cast<const void *>(bwd_fused_kernel<F32, 4, 1, 8, 8, false>);
      else
        fn = fuse ? reinterpret_cast<const void *>(bwd_fused_kernel<BF16, 8, 1, 4, 8, true>)
                  : reinterpret_cast<const void *>(bwd_fused_kernel<BF16, 8, 1, 4, 8, false>);
      if ((e = launch_fn(fn, gvb + nsample, kBlock, 1, p, stream)) != hipSuccess) return e;
    } else {
      if ((e = launch_pairs(false, p, dt, s, stream)) != hipSuccess) return e;
      KernelFn gv = dt == DType::F32 ? pick_gv<F32>(cs) : pick_gv<BF16>(cs);
      if ((e = launch_fn(reinterpret_cast<const void *>(gv), wmax, kBlock, groups, p, stream)) != hipSuccess)
        return e;
    }
  }
  // 4. reference gradients (fused inputs, when asked for)
  if (fuse && p.grad_ref) {
    const int64_t n = p.pairs / p.M * p.ref_dim;
    return launch_fn(reinterpret_cast<const void *>(ref_grad_kernel), (n + kBlock - 1) / kBlock, kBlock, 1, p, stream);
  }
  return hipSuccess;
}

// ------------------------------------------------- static backward scratch
//
// The workspace of the allocation-free backward entry point: one array per
// GPU the library runs on, held until the process ends. Host code never
// passes the array's name to a kernel (on the host it is only a stand-in for
// the symbol); it looks up the device address once per device with that
// device current and passes that address, like a caller's workspace.
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

hipError_t static_scratch(void **ptr) {
  constexpr int kMaxDevices = 256;
  static std::atomic<void *> addr[kMaxDevices];
  static std::mutex mu;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void *p = addr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    std::lock_guard<std::mutex> lock(mu);
    p = addr[dev].load(std::memory_order_relaxed);
    if (p == nullptr) {
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return e;
      addr[dev].store(p, std::memory_order_release);
    }
  }
  *ptr = p;
  return hipSuccess;
}

hipError_t launch_zero(float *ptr, int64_t n, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  const bool aligned = (reinterpret_cast<uintptr_t>(ptr) & 15u) == 0;
  const int64_t per_block = aligned ? (int64_t)kBlock * 4 : (int64_t)kBlock;
  const int64_t blocks = (n + per_block - 1) / per_block;
  if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
  void *args[] = {&ptr, &n};
  const void *fn = aligned ? reinterpret_cast<const void *>(zero_kernel)
                           : reinterpret_cast<const void *>(zero_kernel_unaligned);
  return hipLaunchKernel(fn, dim3((unsigned)blocks), dim3(kBlock), args, 0, stream);
}

}  // namespace msda
