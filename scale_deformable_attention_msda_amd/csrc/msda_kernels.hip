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
//     attn coalesced) and staged in LDS as a 32/48-byte descriptor; every lane
//     of the pair then reads the descriptor with an LDS broadcast.
//   * Corners outside the map carry an offset past the buffer's num_records,
//     so buffer loads return 0 and buffer atomics are dropped by the hardware:
//     zero padding with no branch.
//   * Workgroups are renumbered so that each XCD (own L2) works on one
//     contiguous range of queries, which sample overlapping value rows.
//   * Backward: per sample, the three dot products (grad_attn and the two
//     location gradients) are reduced across the pair's lanes with DPP; the
//     results are staged in LDS and written coalesced. grad_value receives
//     fp32 buffer atomics.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "msda_internal.h"

namespace msda {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kDescCap = 512;             // sample descriptors staged per chunk
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

// Sum over the `lpp` consecutive lanes of a pair; every lane gets the total.
// Steps: quad xor 1, quad xor 2, mirror within 8, mirror within 16, then
// cross-row exchanges. Each step adds two disjoint partial sums, so the
// result is identical in every lane of the group.
template <int LPP>
__device__ __forceinline__ float group_sum(float v, int lpp_rt) {
  const int lpp = LPP > 0 ? LPP : lpp_rt;
  if (lpp >= 2) v += dpp_mov<0xB1>(v);   // quad_perm [1,0,3,2]
  if (lpp >= 4) v += dpp_mov<0x4E>(v);   // quad_perm [2,3,0,1]
  if (lpp >= 8) v += dpp_mov<0x141>(v);  // row_half_mirror
  if (lpp >= 16) v += dpp_mov<0x140>(v); // row_mirror
  if (lpp >= 32) v += __shfl_xor(v, 16);
  if (lpp >= 64) v += __shfl_xor(v, 32);
  return v;
}

__device__ __forceinline__ void load_levels(const Params &p, int32_t *sH, int32_t *sW, int32_t *sS) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int l = 0; l < kMaxLevels; ++l) {
    if (tid == l) {
      sH[l] = p.lv.H[l];
      sW[l] = p.lv.W[l];
      sS[l] = p.lv.start[l];
    }
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

__device__ __forceinline__ Sample sample_geometry(const Params &p, int64_t P, int pt,
                                                  const int32_t *sH, const int32_t *sW,
                                                  const int32_t *sS) {
  const int64_t gi = P * p.LK + pt;
  const float2 xy = *reinterpret_cast<const float2 *>(p.loc + 2 * gi);
  const float A = p.attn[gi];
  const int l = pt / p.K;
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
  const int m = (int)(P % p.M);
  const int64_t n = P / ((int64_t)p.Lq * p.M);
  const uint32_t row = (uint32_t)p.M * (uint32_t)p.D;
  const uint32_t base = (uint32_t)(((n * p.S + s0) * p.M + m) * p.D);
  const bool xo0 = x0 >= 0, xo1 = x0 + 1 < W, yo0 = y0 >= 0, yo1 = y0 + 1 < H;
  const bool in = s.inside;
  s.off[0] = (in && yo0 && xo0) ? base + (uint32_t)(y0 * W + x0) * row : kOobElem;
  s.off[1] = (in && yo0 && xo1) ? base + (uint32_t)(y0 * W + x0 + 1) * row : kOobElem;
  s.off[2] = (in && yo1 && xo0) ? base + (uint32_t)((y0 + 1) * W + x0) * row : kOobElem;
  s.off[3] = (in && yo1 && xo1) ? base + (uint32_t)((y0 + 1) * W + x0 + 1) * row : kOobElem;
  return s;
}

// ---------------------------------------------------------------- forward

struct __align__(16) FDesc {
  uint32_t off[4];  // byte offsets of the corners in value
  float w[4];       // attn * bilinear weight, 0 for corners outside the map
};

template <typename T, int VEC, int NCG, int LPP>
__global__ __launch_bounds__(kBlock) void fwd_kernel(const Params p) {
  __shared__ FDesc desc[kDescCap];
  __shared__ int32_t sH[kMaxLevels], sW[kMaxLevels], sS[kMaxLevels];
  load_levels(p, sH, sW, sS);

  const int tid = threadIdx.x;
  const int lpp = LPP > 0 ? LPP : p.lpp;
  const int ppb = kBlock / lpp;
  const int64_t P0 = (int64_t)xcd_remap(blockIdx.x, gridDim.x) * ppb;
  const int npairs = (int)min((int64_t)ppb, p.pairs - P0);
  const int g = tid / lpp;
  const int j = tid - g * lpp;
  const bool active = g < npairs;

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
    __syncthreads();
    for (int i = tid; i < npairs * pcn; i += kBlock) {
      const int gg = i / pcn;
      const int pp = i - gg * pcn;
      const Sample s = sample_geometry(p, P0 + gg, pc0 + pp, sH, sW, sS);
      FDesc d;
      const float wa[2] = {1.0f - s.a, s.a};
      const float wb[2] = {1.0f - s.b, s.b};
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const bool ok = s.off[c] != kOobElem;
        d.off[c] = s.off[c] * (uint32_t)T::size;
        d.w[c] = ok ? s.A * wb[c >> 1] * wa[c & 1] : 0.0f;
      }
      desc[pp * ppb + gg] = d;
    }
    __syncthreads();
    if (active) {
#pragma unroll 2
      for (int pp = 0; pp < pcn; ++pp) {
        const FDesc d = desc[pp * ppb + g];
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
    const int64_t obase = (P0 + g) * (int64_t)p.D;
#pragma unroll
    for (int cg = 0; cg < NCG; ++cg) {
      const int c = j + cg * lpp;
      if (c < nvec) store_vals<T, VEC>(p.out, obase + (int64_t)c * VEC, acc[cg]);
    }
  }
}

// --------------------------------------------------------------- backward

struct __align__(16) BDesc {
  uint32_t off[4];  // element offsets of the corners (kOobElem outside the map)
  float w[4];       // attn * bilinear weight
  float a, b;       // fractional parts of the index coordinate
  float aw, ah;     // attn * W_l, attn * H_l (chain rule through loc * W - 0.5)
};

template <typename T, int VEC, int NCG, int LPP>
__global__ __launch_bounds__(kBlock) void bwd_kernel(const Params p) {
  __shared__ BDesc desc[kDescCap];
  __shared__ float3 res[kDescCap];
  __shared__ int32_t sH[kMaxLevels], sW[kMaxLevels], sS[kMaxLevels];
  load_levels(p, sH, sW, sS);

  const int tid = threadIdx.x;
  const int lpp = LPP > 0 ? LPP : p.lpp;
  const int ppb = kBlock / lpp;
  const int64_t P0 = (int64_t)xcd_remap(blockIdx.x, gridDim.x) * ppb;
  const int npairs = (int)min((int64_t)ppb, p.pairs - P0);
  const int g = tid / lpp;
  const int j = tid - g * lpp;
  const bool active = g < npairs;

  const __amdgpu_buffer_rsrc_t rv = make_rsrc(p.value, p.value_elems * (uint32_t)T::size);
  const __amdgpu_buffer_rsrc_t rg = make_rsrc(p.grad_value, p.value_elems * 4u);
  const __amdgpu_buffer_rsrc_t ro = make_rsrc(p.grad_out, (uint32_t)(p.pairs * p.D) * (uint32_t)T::size);
  const int nvec = p.D / VEC;
  uint32_t lane_elem[NCG];
  float G[NCG][VEC];
#pragma unroll
  for (int cg = 0; cg < NCG; ++cg) {
    const int c = j + cg * lpp;
    lane_elem[cg] = c < nvec ? (uint32_t)(c * VEC) : kOobElem;
    const uint32_t go = active && c < nvec ? (uint32_t)((P0 + g) * p.D + c * VEC) : kOobElem;
    load_vals<T, VEC>(ro, go * (uint32_t)T::size, G[cg]);
  }

  for (int pc0 = 0; pc0 < p.LK; pc0 += p.pc) {
    const int pcn = min(p.pc, p.LK - pc0);
    __syncthreads();
    for (int i = tid; i < npairs * pcn; i += kBlock) {
      const int gg = i / pcn;
      const int pp = i - gg * pcn;
      const Sample s = sample_geometry(p, P0 + gg, pc0 + pp, sH, sW, sS);
      const int l = (pc0 + pp) / p.K;
      BDesc d;
      const float wa[2] = {1.0f - s.a, s.a};
      const float wb[2] = {1.0f - s.b, s.b};
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        d.off[c] = s.off[c];
        d.w[c] = s.A * wb[c >> 1] * wa[c & 1];
      }
      d.a = s.a;
      d.b = s.b;
      d.aw = s.A * (float)sW[l];
      d.ah = s.A * (float)sH[l];
      desc[pp * ppb + gg] = d;
    }
    __syncthreads();
    if (active) {
#pragma unroll 2
      for (int pp = 0; pp < pcn; ++pp) {
        const BDesc d = desc[pp * ppb + g];
        float dot[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          dot[c] = 0.0f;
#pragma unroll
          for (int cg = 0; cg < NCG; ++cg) {
            float v[VEC];
            load_vals<T, VEC>(rv, (d.off[c] + lane_elem[cg]) * (uint32_t)T::size, v);
#pragma unroll
            for (int e = 0; e < VEC; ++e) dot[c] = fmaf(G[cg][e], v[e], dot[c]);
          }
        }
        const float a = d.a, b = d.b;
        float ga = (1.0f - b) * ((1.0f - a) * dot[0] + a * dot[1]) + b * ((1.0f - a) * dot[2] + a * dot[3]);
        float gx = (1.0f - b) * (dot[1] - dot[0]) + b * (dot[3] - dot[2]);
        float gy = (1.0f - a) * (dot[2] - dot[0]) + a * (dot[3] - dot[1]);
        ga = group_sum<LPP>(ga, lpp);
        gx = group_sum<LPP>(gx, lpp);
        gy = group_sum<LPP>(gy, lpp);
        if (j == 0) res[pp * ppb + g] = make_float3(ga, d.aw * gx, d.ah * gy);
#pragma unroll
        for (int c = 0; c < 4; ++c) {
#pragma unroll
          for (int cg = 0; cg < NCG; ++cg) {
            const uint32_t ob = (d.off[c] + lane_elem[cg]) * 4u;
#pragma unroll
            for (int e = 0; e < VEC; ++e)
              __builtin_amdgcn_raw_ptr_buffer_atomic_fadd_f32(d.w[c] * G[cg][e], rg, ob + 4u * e, 0, 0);
          }
        }
      }
    }
    __syncthreads();
    for (int i = tid; i < npairs * pcn; i += kBlock) {
      const int gg = i / pcn;
      const int pp = i - gg * pcn;
      const float3 r = res[pp * ppb + gg];
      const int64_t gi = (P0 + gg) * p.LK + pc0 + pp;
      p.grad_attn[gi] = r.x;
      *reinterpret_cast<float2 *>(p.grad_loc + 2 * gi) = make_float2(r.y, r.z);
    }
  }
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

template <typename T, int VEC>
KernelFn pick(bool fwd, int ncg, int lpp) {
  // Compile-time lane counts for the common 16-byte shapes (fp32 D=32 and
  // bf16 D=32), a runtime lane count otherwise.
  if (ncg == 1 && lpp == 8 && VEC * T::size == 16)
    return fwd ? fwd_kernel<T, VEC, 1, 8> : bwd_kernel<T, VEC, 1, 8>;
  if (ncg == 1 && lpp == 4 && VEC * T::size == 16)
    return fwd ? fwd_kernel<T, VEC, 1, 4> : bwd_kernel<T, VEC, 1, 4>;
  switch (ncg) {
    case 1: return fwd ? fwd_kernel<T, VEC, 1, 0> : bwd_kernel<T, VEC, 1, 0>;
    case 2: return fwd ? fwd_kernel<T, VEC, 2, 0> : bwd_kernel<T, VEC, 2, 0>;
    case 4: return fwd ? fwd_kernel<T, VEC, 4, 0> : bwd_kernel<T, VEC, 4, 0>;
    default: break;
  }
  if constexpr (VEC == 1) {
    if (ncg == 8) return fwd ? fwd_kernel<T, 1, 8, 0> : bwd_kernel<T, 1, 8, 0>;
    if (ncg == 16) return fwd ? fwd_kernel<T, 1, 16, 0> : bwd_kernel<T, 1, 16, 0>;
  }
  return nullptr;
}

KernelFn select(bool fwd, DType dt, const LaunchShape &s) {
  if (dt == DType::F32) {
    switch (s.vec) {
      case 4: return pick<F32, 4>(fwd, s.ncg, s.lpp);
      case 2: return pick<F32, 2>(fwd, s.ncg, s.lpp);
      case 1: return pick<F32, 1>(fwd, s.ncg, s.lpp);
    }
  } else {
    switch (s.vec) {
      case 8: return pick<BF16, 8>(fwd, s.ncg, s.lpp);
      case 4: return pick<BF16, 4>(fwd, s.ncg, s.lpp);
      case 2: return pick<BF16, 2>(fwd, s.ncg, s.lpp);
      case 1: return pick<BF16, 1>(fwd, s.ncg, s.lpp);
    }
  }
  return nullptr;
}

hipError_t launch(bool fwd, const Params &p_in, DType dt, const LaunchShape &s, hipStream_t stream) {
  KernelFn fn = select(fwd, dt, s);
  if (!fn) return hipErrorInvalidValue;
  Params p = p_in;
  p.lpp = s.lpp;
  const int ppb = kBlock / s.lpp;
  p.pc = min(p.LK, max(1, kDescCap / ppb));
  const int64_t blocks = (p.pairs + ppb - 1) / ppb;
  if (blocks <= 0) return hipSuccess;
  if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
  void *args[] = {&p};
  return hipLaunchKernel(reinterpret_cast<const void *>(fn), dim3((unsigned)blocks), dim3(kBlock), args, 0,
                         stream);
}

}  // namespace

LaunchShape choose_shape(int D, DType dt, uintptr_t align_bits) {
  const int esz = dt == DType::F32 ? 4 : 2;
  LaunchShape s{1, 1, 1};
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
    s = LaunchShape{vec, lpp, ncg};
    return s;
  }
  // Single-element lanes with up to 16 channel groups (D <= 1024).
  int ncg = 1;
  while (ncg * 64 < D) ncg *= 2;
  int lpp = 1;
  while (lpp < D && lpp < 64) lpp *= 2;
  return LaunchShape{1, lpp, ncg};
}

hipError_t launch_forward(const Params &p, DType dt, const LaunchShape &s, hipStream_t stream) {
  return launch(true, p, dt, s, stream);
}

hipError_t launch_backward(const Params &p, DType dt, const LaunchShape &s, hipStream_t stream) {
  return launch(false, p, dt, s, stream);
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
