// Hardware ceilings of MI355X (gfx950) for the access patterns of the MSDA
// sampling core. Each probe is a kernel that runs a bounded loop over one
// pattern and exits normally; the host times it with HIP events (best of 3)
// and prints one markdown row per probe:
//   * HBM stream copy;
//   * gathers of random 128-byte rows (8 lanes x 16 bytes, one bilinear
//     corner of one fp32 head of 32 channels) from a 16 KB region (served
//     by L1), a 2 MB region (L2), a 64 MB region (Infinity Cache) and a
//     1 GB region (HBM);
//   * LDS reads of random 128-byte rows (8 lanes per row) and of random
//     256-byte row pairs (16 lanes: the two x-neighbouring corners);
//   * LDS float atomics (ds_add_f32) on random 128-byte rows, 4 floats per
//     lane, distinct addresses within an instruction, and the same on one
//     shared row per wave (every lane of a wave on the same 32 addresses);
//   * global float atomics (no return) on random 128-byte rows of a 16 MB
//     and a 256 MB buffer, and a window flush: each workgroup adds a window
//     of consecutive pixel rows of one head (128-byte rows, 1 KB apart)
//     into a value-shaped fp32 map;
//   * staging into LDS of 128-byte rows 1 KB apart (one head's channels of
//     consecutive pixels), with direct global-to-LDS loads and with plain
//     loads plus LDS stores.
// Rates are per second over the whole chip and per CU per clock at the
// 2.4 GHz peak engine clock (256 CUs).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <vector>

#define CHECK(x)                                                                        \
  do {                                                                                  \
    hipError_t e_ = (x);                                                                \
    if (e_ != hipSuccess) {                                                             \
      fprintf(stderr, "%s:%d %s\n", __FILE__, __LINE__, hipGetErrorString(e_));         \
      exit(1);                                                                          \
    }                                                                                   \
  } while (0)

namespace {

constexpr double kClock = 2.4e9;
constexpr int kCUs = 256;

__device__ __forceinline__ uint32_t lcg(uint32_t x) { return x * 1664525u + 1013904223u; }

// Random 128-byte rows of a region of (mask + 1) rows at `buf`: lanes 8g..8g+7
// read row r_g, 16 bytes each; 8 rows in flight per lane.
__global__ __launch_bounds__(256) void gather_rows(const float4 *__restrict__ buf, uint32_t mask, int iters,
                                                   float *sink) {
  const int lane8 = threadIdx.x & 7, grp = threadIdx.x >> 3;
  uint32_t r = lcg(blockIdx.x * 7919u + grp * 131u + 12345u);
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int i = 0; i < iters; ++i) {
    float4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      r = lcg(r);
      const uint32_t row = (r >> 7) & mask;
      v[u] = buf[(size_t)row * 8 + lane8];
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      acc.x += v[u].x;
      acc.y += v[u].y;
      acc.z += v[u].z;
      acc.w += v[u].w;
    }
  }
  if (acc.x + acc.y + acc.z + acc.w == 123.456f) sink[blockIdx.x * 256 + threadIdx.x] = acc.x;
}

// LDS reads of random rows of a 64 KB window (512 rows of 128 B). PAIR: 16
// lanes read rows r and r+1 (256 contiguous bytes).
template <bool PAIR>
__global__ __launch_bounds__(256) void lds_read_rows(int iters, float *sink) {
  __shared__ float4 win[4096 + 8];
  for (int i = threadIdx.x; i < 4096 + 8; i += 256) win[i] = make_float4((float)i, 1.f, 2.f, 3.f);
  __syncthreads();
  const int sub = PAIR ? (threadIdx.x & 15) : (threadIdx.x & 7);
  const int grp = PAIR ? (threadIdx.x >> 4) : (threadIdx.x >> 3);
  uint32_t r = lcg(blockIdx.x * 7919u + grp * 131u + 12345u);
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int i = 0; i < iters; ++i) {
    float4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      r = lcg(r);
      const uint32_t row = (r >> 7) & 511u;
      v[u] = win[row * 8 + sub];
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      acc.x += v[u].x;
      acc.y += v[u].y;
      acc.z += v[u].z;
      acc.w += v[u].w;
    }
  }
  if (acc.x + acc.y + acc.z + acc.w == 123.456f) sink[blockIdx.x * 256 + threadIdx.x] = acc.x;
}

// ds_add_f32 on random rows of a 64 KB window: lanes 8g..8g+7 add to the 32
// floats of row r_g (4 each). SHARED: every group of a wave uses the same row.
template <bool SHARED>
__global__ __launch_bounds__(256) void lds_add_rows(int iters, float *sink) {
  __shared__ float win[16384];
  for (int i = threadIdx.x; i < 16384; i += 256) win[i] = 0.f;
  __syncthreads();
  const int lane8 = threadIdx.x & 7;
  const int grp = SHARED ? (threadIdx.x >> 6) : (threadIdx.x >> 3);
  uint32_t r = lcg(blockIdx.x * 7919u + grp * 131u + 12345u);
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      r = lcg(r);
      const uint32_t row = (r >> 7) & 511u;
      float *p = win + row * 32 + lane8 * 4;
#pragma unroll
      for (int c = 0; c < 4; ++c) atomicAdd(p + c, 1.0f);
    }
  }
  __syncthreads();
  if (win[threadIdx.x] == 123.456f) sink[blockIdx.x * 256 + threadIdx.x] = win[threadIdx.x];
}

// Global float atomics without return on random 128-byte rows: lanes
// 32g..32g+31 add one float each to row r_g.
__global__ __launch_bounds__(256) void global_add_rows(float *buf, uint32_t mask, int iters) {
  const int lane32 = threadIdx.x & 31, grp = threadIdx.x >> 5;
  uint32_t r = lcg(blockIdx.x * 7919u + grp * 131u + 12345u);
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      r = lcg(r);
      const uint32_t row = (r >> 7) & mask;
      unsafeAtomicAdd(buf + (size_t)row * 32 + lane32, 1.0f);
    }
  }
}

// Window flush: workgroup b adds `rows` consecutive pixel rows of head
// b % heads, starting at pixel (b / heads) * step, into a [pixels, heads, 32]
// fp32 map (128-byte rows, heads * 128 bytes apart). Pixels wrap modulo the
// map, so every address stays inside it.
__global__ __launch_bounds__(256) void window_flush(float *map, int pixels, int heads, int rows, int step) {
  const int m = blockIdx.x % heads;
  const int p0 = (blockIdx.x / heads) * step;
  for (int i = threadIdx.x; i < rows * 32; i += 256) {
    const int pr = i >> 5, c = i & 31;
    const int pix = (p0 + pr) % pixels;
    unsafeAtomicAdd(map + ((size_t)pix * heads + m) * 32 + c, 1.0f);
  }
}

// Staging of `rows` 128-byte rows, 1 KB apart in global memory (one head of a
// [pixels, 8, 32] fp32 map), into contiguous LDS, repeated over windows
// iters times. DIRECT: global_load_lds_dwordx4 (data goes straight to LDS);
// otherwise global loads into registers, then ds_write_b128.
template <bool DIRECT>
__global__ __launch_bounds__(256) void stage_rows(const float4 *__restrict__ map, int pixels, int rows, int iters,
                                                  float *sink) {
  // a wave's direct load fills 8 whole rows from its base row r0 (a multiple
  // of 8 below `rows` <= 441), so the window holds 448 rows
  __shared__ float4 win[448 * 8];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int m = blockIdx.x & 7;
  float acc = 0.f;
  for (int it = 0; it < iters; ++it) {
    const int p0 = (int)(((uint32_t)(blockIdx.x * 131 + it * 977) * 2654435761u) % (uint32_t)(pixels - rows));
    // 64 lanes x 16 B = 8 rows per wave instruction
    for (int r0 = wave * 8; r0 < rows; r0 += 32) {
      const int rr = r0 + (lane >> 3);
      const int rrc = rr < rows ? rr : rows - 1;
      const float4 *src = map + ((size_t)(p0 + rrc) * 8 + m) * 8 + (lane & 7);
      if constexpr (DIRECT) {
        __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void *)(win + r0 * 8), 16, 0, 0);
      } else {
        const float4 v = *src;
        if (rr < rows) win[rr * 8 + (lane & 7)] = v;
      }
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    acc += win[(threadIdx.x * 7 + it) % (rows * 8)].x;
    __syncthreads();
  }
  if (acc == 123.456f) sink[blockIdx.x * 256 + threadIdx.x] = acc;
}

__global__ void copy_kernel(const float4 *__restrict__ a, float4 *__restrict__ b, size_t n) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
    b[i] = a[i];
}

__global__ void fill_kernel(float4 *a, size_t n, float v) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
    a[i] = make_float4(v, v, v, v);
}

template <typename F>
float best_ms(F launch, int reps = 3) {
  hipEvent_t a, b;
  CHECK(hipEventCreate(&a));
  CHECK(hipEventCreate(&b));
  launch();  // warm-up
  CHECK(hipDeviceSynchronize());
  float best = 1e30f;
  for (int i = 0; i < reps; ++i) {
    CHECK(hipEventRecord(a));
    launch();
    CHECK(hipEventRecord(b));
    CHECK(hipEventSynchronize(b));
    float ms;
    CHECK(hipEventElapsedTime(&ms, a, b));
    best = std::min(best, ms);
  }
  CHECK(hipEventDestroy(a));
  CHECK(hipEventDestroy(b));
  return best;
}

void row(const char *name, const char *what, double ms, double bytes, double ops, const char *opname) {
  const double s = ms * 1e-3;
  const double perclk = bytes / s / kCUs / kClock;
  printf("| %s | %s | %.3f | %.1f | %.1f | %.3g %s/s |\n", name, what, ms, bytes / s / 1e9, perclk, ops / s,
         opname);
  fflush(stdout);
}

}  // namespace

int main() {
  hipDeviceProp_t prop;
  CHECK(hipGetDeviceProperties(&prop, 0));
  printf("device: %s, %d CUs, clock %d kHz, LDS per workgroup %zu B\n\n", prop.gcnArchName,
         prop.multiProcessorCount, prop.clockRate, prop.sharedMemPerBlock);
  printf("| probe | pattern | best ms | GB/s | B/clk/CU | op rate |\n|---|---|---|---|---|---|\n");
  fflush(stdout);

  float *sink;
  CHECK(hipMalloc(&sink, (size_t)65536 * 256 * 4));

  // HBM copy: 512 MiB read + 512 MiB written (beyond the 256 MB Infinity Cache)
  {
    const size_t n = (size_t)512 << 20 >> 4;
    float4 *a, *b;
    CHECK(hipMalloc(&a, n * 16));
    CHECK(hipMalloc(&b, n * 16));
    fill_kernel<<<4096, 256>>>(a, n, 1.f);
    const float ms = best_ms([&] { copy_kernel<<<8192, 256>>>(a, b, n); });
    row("hbm_copy", "float4 copy, 512 MiB each way", ms, 2.0 * n * 16, 2.0 * n * 16, "B");
    CHECK(hipFree(a));
    CHECK(hipFree(b));
  }

  // random 128-byte row gathers from regions of growing size
  {
    const size_t big_rows = (size_t)1 << 23;  // 1 GiB
    float4 *buf;
    CHECK(hipMalloc(&buf, big_rows * 128));
    fill_kernel<<<8192, 256>>>(buf, big_rows * 8, 1.f);
    struct G {
      const char *name, *what;
      uint32_t mask;
      int iters;
    } gs[] = {{"gather_l1", "random 128 B rows of a 16 KB region", (1u << 7) - 1, 256},
              {"gather_l2", "random 128 B rows of a 2 MB region", (1u << 14) - 1, 96},
              {"gather_mall", "random 128 B rows of a 64 MB region", (1u << 19) - 1, 48},
              {"gather_hbm", "random 128 B rows of a 1 GB region", (1u << 23) - 1, 24}};
    for (const G &g : gs) {
      const int blocks = 4096;
      const float ms = best_ms([&] { gather_rows<<<blocks, 256>>>(buf, g.mask, g.iters, sink); });
      const double rows_read = (double)blocks * 32 * g.iters * 8;
      row(g.name, g.what, ms, rows_read * 128, rows_read, "rows");
    }
    CHECK(hipFree(buf));
  }

  // LDS reads and LDS float atomics (64 KB per workgroup: two per CU)
  {
    const int blocks = 2048, iters = 1024;
    float ms = best_ms([&] { lds_read_rows<false><<<blocks, 256>>>(iters, sink); });
    double n = (double)blocks * 32 * iters * 8;
    row("lds_read_row", "ds_read_b128, random 128 B rows of 64 KB, 8 lanes/row", ms, n * 128, n, "rows");
    ms = best_ms([&] { lds_read_rows<true><<<blocks, 256>>>(iters, sink); });
    n = (double)blocks * 16 * iters * 8;
    row("lds_read_pair", "ds_read_b128, random 256 B row pairs of 64 KB, 16 lanes/pair", ms, n * 256, n,
        "pairs");
    const int aiters = 16;
    ms = best_ms([&] { lds_add_rows<false><<<blocks, 256>>>(aiters, sink); });
    n = (double)blocks * 256 * aiters * 4 * 4;
    row("lds_add_f32", "ds_add_f32, random 128 B rows, distinct addresses", ms, n * 4, n, "adds");
    ms = best_ms([&] { lds_add_rows<true><<<blocks, 256>>>(aiters, sink); });
    row("lds_add_f32_shared", "ds_add_f32, 8 lane groups of a wave on one row", ms, n * 4, n, "adds");
  }

  // global float atomics
  {
    const size_t rows_big = (size_t)1 << 21;  // 256 MB
    float *buf;
    CHECK(hipMalloc(&buf, rows_big * 128));
    CHECK(hipMemset(buf, 0, rows_big * 128));
    const int blocks = 4096, iters = 16;
    double n = (double)blocks * 256 * iters * 4;
    float ms = best_ms([&] { global_add_rows<<<blocks, 256>>>(buf, (1u << 17) - 1, iters); });
    row("global_add_16mb", "global atomic add f32, random 128 B rows of 16 MB", ms, n * 4, n, "adds");
    ms = best_ms([&] { global_add_rows<<<blocks, 256>>>(buf, (1u << 21) - 1, iters); });
    row("global_add_256mb", "global atomic add f32, random 128 B rows of 256 MB", ms, n * 4, n, "adds");
    // window flush into a [22223, 8, 32] map: 5.6 K workgroups of 441 rows
    const int pixels = 22223, heads = 8, rows = 441, wg = 5632;
    ms = best_ms([&] { window_flush<<<wg, 256>>>(buf, pixels, heads, rows, 31); });
    n = (double)wg * rows * 32;
    row("window_flush", "5632 windows of 441 rows (1 KB apart) added to a 22.7 MB map", ms, n * 4, n, "adds");
    CHECK(hipFree(buf));
  }

  // staging into LDS: one head's rows (128 B, 1 KB apart) of a [pixels, 8, 32] map
  {
    const int pixels = 22223 * 4, rows = 441, iters = 16, blocks = 2048;
    float4 *map;
    CHECK(hipMalloc(&map, (size_t)pixels * 1024));
    fill_kernel<<<4096, 256>>>(map, (size_t)pixels * 64, 1.f);
    const double n = (double)blocks * iters * rows;
    float ms = best_ms([&] { stage_rows<true><<<blocks, 256>>>(map, pixels, rows, iters, sink); });
    row("stage_direct", "global_load_lds_dwordx4, 441 rows of 128 B per window", ms, n * 128, n, "rows");
    ms = best_ms([&] { stage_rows<false><<<blocks, 256>>>(map, pixels, rows, iters, sink); });
    row("stage_plain", "global_load_dwordx4 + ds_write_b128, same windows", ms, n * 128, n, "rows");
    CHECK(hipFree(map));
  }
  CHECK(hipFree(sink));
  printf("\nclock for B/clk/CU: %.1f GHz peak engine clock, %d CUs\n", kClock / 1e9, kCUs);
  return 0;
}
