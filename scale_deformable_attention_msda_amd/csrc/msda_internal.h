// Internal launch interface between the C-ABI layer (msda_api.cpp) and the
// gfx950 kernels (msda_kernels.hip). Not part of the public ABI.
#pragma once

#include <stddef.h>
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
// Samples (N*Lq*M*L*K) of one launch must have 32-bit indices.
constexpr int64_t kMaxSliceSamples = (int64_t)1 << 31;
// Byte offset that marks an absent sort entry in the scatter pass's buffer
// stores: at or past the end of any entries region whose size is below it
// (a larger region uses plain stores instead).
constexpr uint32_t kEntriesOob = 0xfffffff0u;

// grad_value is produced per 8x8-pixel tile of each (image, head, level).
constexpr int kTile = 8;
constexpr int kTilePix = kTile * kTile;
// Entries (sample, tile) handled by one workgroup of the grad_value pass; a
// tile with more entries is split into several work items whose partial sums
// are combined with float atomics.
constexpr int kPartEntries = 1024;
// Channels handled by one grad_value work item.
constexpr int kChanGroup = 64;

struct LevelTable {
  int32_t H[kMaxLevels];
  int32_t W[kMaxLevels];
  int32_t start[kMaxLevels];
  int32_t TH[kMaxLevels];    // tile rows of the level
  int32_t TW[kMaxLevels];    // tile columns of the level
  int32_t toff[kMaxLevels];  // first tile of the level within one (image, head)
};

// Backward scratch, carved out of the caller's workspace.
struct Workspace {
  uint32_t *tile_count;   // [T+8] entries per tile; [T] counts split tiles
  uint32_t *tile_cursor;  // [T]   fill cursor of the scatter pass
  uint32_t *tile_start;   // [T+1] first entry of each tile
  uint32_t *work_item;    // [4*Wmax] grad_value work items {tile, first entry, end entry, split}
  uint32_t *n_work;       // [1]
  uint32_t *split_list;   // [T] tiles whose entries span several work items
  uint32_t *entries;      // [4*Emax] (sample, tile) entries, tile-major, 16-byte records
  uint32_t entries_bytes; // bytes of the entries region when below kEntriesOob (buffer stores), else 0
  float *ref_part;        // [4*pairs] per-pair sums of the reference gradient (fused inputs)
  float *floc;            // [2*samples] locations formed from the fused inputs
  float *fattn;           // [samples] weights formed from the fused inputs
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
  int32_t TPI;           // tiles per (image, head) over all levels
  int32_t T;             // tiles of the launch: N * M * TPI
  int32_t qpb;           // queries per workgroup of the scatter (binning) pass
  int32_t qpb0;          // queries per workgroup of the counting (binning) pass
  int32_t gvec;          // grad_out rows allow 16-byte loads
  int32_t gv_blocks;     // grad_value blocks of the fused backward launch
  int32_t scatter;       // grad_value zero-filled, then added to with float atomics per sample
                         // (sparse launches: no tile sort)
  int32_t seg_softmax;   // fused inputs: a pair's L*K logits sit in L*K consecutive lanes of
                         // the per-sample passes (L*K a power of two <= 64, one chunk)
  int32_t head_major;    // per-sample passes: a workgroup takes consecutive queries of one head
  int32_t form_inputs;   // fused inputs: the counting pass forms every sample's location and
                         // weight from the raw inputs and stores them in the workspace
  // Fused inputs (ref_dim 2 or 4): loc then holds offsets, attn holds logits,
  // and grad_loc / grad_attn receive the offset and logit gradients.
  // ref_dim 0: loc and attn are the sampling core's own inputs.
  const float *ref;      // [pairs / M, ref_dim] reference points or boxes
  const float *offsets;  // backward with fused inputs: the raw offsets and logits
  const float *logits;   // (loc and attn then point at the formed ones)
  int32_t ref_dim;
  float *grad_ref;       // [pairs / M, ref_dim], may be null
  Workspace ws;
  LevelTable lv;
};

enum class DType { F32 = 0, BF16 = 1 };

struct LaunchShape {
  int vec;   // elements per lane per memory access
  int lpp;   // lanes per pair
  int ncg;   // channel groups per lane
};

// Picks the lane mapping for a channel count, element type, pointer alignment
// and the number of (n, q, m) pairs of the launch.
LaunchShape choose_shape_widest(int D, DType dt, uintptr_t align_bits);
LaunchShape choose_shape(int D, DType dt, uintptr_t align_bits, int64_t pairs);

// Tile table and workspace layout of a launch covering `nimg` images.
struct WorkspaceLayout {
  int64_t T, Wmax, Emax;
  size_t off_count, off_cursor, off_start, off_witem, off_nwork, off_split, off_entries, off_refpart, off_floc,
      off_fattn, bytes;
};
WorkspaceLayout workspace_layout(const int64_t *spatial_shapes, int64_t L, int64_t nimg, int64_t M,
                                 int64_t Lq, int64_t K, bool fused);
void fill_tiles(LevelTable &lv, const int64_t *spatial_shapes, int64_t L, int32_t *TPI);

hipError_t launch_forward(const Params &p, DType dt, const LaunchShape &s, hipStream_t stream);
hipError_t launch_backward(const Params &p, DType dt, const LaunchShape &s, hipStream_t stream);
hipError_t launch_zero(float *ptr, int64_t n, hipStream_t stream);

// Bytes of the per-device static scratch array that the allocation-free
// backward uses as its workspace (MSDA_STATIC_SCRATCH_BYTES in msda.h).
constexpr size_t kStaticScratchBytes = (size_t)64 << 20;
// Device address of the current device's scratch array (looked up once per
// device, then cached).
hipError_t static_scratch(void **ptr);

}  // namespace msda
