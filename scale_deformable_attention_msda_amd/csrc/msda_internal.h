// Internal launch interface between the C-ABI layer (msda_api.cpp) and the
// gfx950 kernels (msda_kernels.hip). Not part of the public ABI.
#pragma once

#include <stdint.h>
#include <hip/hip_runtime_api.h>

namespace msda {

constexpr int kMaxLevels = 16;
constexpr int kBlock = 256;  // threads per workgroup: four wave64s

// Element index that marks a corner (or an idle lane) outside the data. Every
// launch covers value / grad_out slices of fewer elements, so the byte offset
// it turns into lies past the buffer's num_records and the buffer instruction
// returns zero (loads) or is dropped (atomics) in hardware. Two sentinels
// added together (corner + idle lane), times 4 bytes, still fit in 32 bits.
constexpr uint32_t kOobElem = 1u << 28;
constexpr int64_t kMaxSliceElems = (int64_t)kOobElem - 1;

struct LevelTable {
  int32_t H[kMaxLevels];
  int32_t W[kMaxLevels];
  int32_t start[kMaxLevels];
};

// One launch covers images [0, N) of the pointers below (the host offsets the
// pointers when it splits a large batch).
struct Params {
  const void *value;
  const float *loc;
  const float *attn;
  const void *grad_out;  // backward only
  void *out;             // forward output
  float *grad_value;     // backward outputs
  float *grad_loc;
  float *grad_attn;
  int64_t pairs;         // N * Lq * M
  int32_t N, S, M, D, L, K, Lq, LK;
  int32_t lpp;           // lanes per (n, q, m) pair, a power of two <= 64
  int32_t pc;            // points per descriptor chunk
  uint32_t value_elems;  // elements of value in this launch (< kOobElem)
  LevelTable lv;
};

enum class DType { F32 = 0, BF16 = 1 };

struct LaunchShape {
  int vec;   // elements per lane per memory access
  int lpp;   // lanes per pair
  int ncg;   // channel groups per lane
};

// Picks the lane mapping for a channel count, element type and pointer alignment.
LaunchShape choose_shape(int D, DType dt, uintptr_t align_bits);

hipError_t launch_forward(const Params &p, DType dt, const LaunchShape &s, hipStream_t stream);
hipError_t launch_backward(const Params &p, DType dt, const LaunchShape &s, hipStream_t stream);
hipError_t launch_zero(float *ptr, int64_t n, hipStream_t stream);

}  // namespace msda
