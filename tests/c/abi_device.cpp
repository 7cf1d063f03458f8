// Device-side use of the C ABI with plain HIP (no torch): hipMalloc'd buffers,
// a stream of its own, msda_forward, msda_backward_workspace_size and
// msda_backward, checked against closed forms. On a map whose head m reads the
// same channel vector c_m at every pixel, with weights summing to 1 per
// (query, head) and every sample inside the map, out = c_m; grad_attn =
// <grad_out, c_m>; grad_loc = 0; and <grad_out, out> = <grad_value, value>.
// The two calls are then captured in a HIP graph and replayed (see below).
// Prints one line per check and "OK" at the end; exit status 0 on success.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdio>
#include <vector>

#include "msda.h"

#define HIP_OK(x)                                                              \
  do {                                                                         \
    hipError_t e_ = (x);                                                       \
    if (e_ != hipSuccess) {                                                    \
      std::printf("HIP error %s at %s\n", hipGetErrorString(e_), #x);          \
      return 2;                                                                \
    }                                                                          \
  } while (0)

int main() {
  const int64_t N = 1, M = 2, D = 8, L = 2, K = 3, Lq = 17;
  const int64_t shapes[2][2] = {{6, 10}, {3, 5}};
  const int64_t starts[2] = {0, 60};
  const int64_t S = 75;
  const int64_t P = N * Lq * M * L * K;  // sampled points

  std::vector<float> value(N * S * M * D), loc(2 * P), attn(P), grad_out(N * Lq * M * D);
  auto c = [](int64_t m, int64_t d) { return 0.5f + 0.1f * (float)m + 0.01f * (float)d; };
  for (int64_t s = 0; s < S; ++s)
    for (int64_t m = 0; m < M; ++m)
      for (int64_t d = 0; d < D; ++d) value[(s * M + m) * D + d] = c(m, d);
  // locations in [0.18, 0.82]^2: on both levels (6x10 and 3x5) every corner
  // lies in the map, none past its last row or column; weights (i + 1) / sum
  // over a pair's L*K samples
  unsigned st = 12345u;
  auto rnd = [&st]() {
    st = st * 1664525u + 1013904223u;
    return (float)(st >> 8) / (float)(1u << 24);
  };
  const int64_t LK = L * K;
  const float wsum = (float)(LK * (LK + 1) / 2);
  for (int64_t i = 0; i < P; ++i) {
    loc[2 * i] = 0.18f + 0.64f * rnd();
    loc[2 * i + 1] = 0.18f + 0.64f * rnd();
    attn[i] = (float)(i % LK + 1) / wsum;
  }
  for (int64_t i = 0; i < N * Lq * M * D; ++i) grad_out[i] = 1.0f + 0.001f * (float)(i % 97);

  hipStream_t stream;
  HIP_OK(hipStreamCreate(&stream));
  float *dv, *dl, *da, *dout, *dg, *dgv, *dgl, *dga;
  HIP_OK(hipMalloc(&dv, value.size() * 4));
  HIP_OK(hipMalloc(&dl, loc.size() * 4));
  HIP_OK(hipMalloc(&da, attn.size() * 4));
  HIP_OK(hipMalloc(&dout, grad_out.size() * 4));
  HIP_OK(hipMalloc(&dg, grad_out.size() * 4));
  HIP_OK(hipMalloc(&dgv, value.size() * 4));
  HIP_OK(hipMalloc(&dgl, loc.size() * 4));
  HIP_OK(hipMalloc(&dga, attn.size() * 4));
  HIP_OK(hipMemcpy(dv, value.data(), value.size() * 4, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(dl, loc.data(), loc.size() * 4, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(da, attn.data(), attn.size() * 4, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(dg, grad_out.data(), grad_out.size() * 4, hipMemcpyHostToDevice));

  int fails = 0;
  msda_status s = msda_forward(dv, &shapes[0][0], starts, dl, da, dout, N, S, M, D, L, Lq, K, MSDA_F32, stream);
  std::printf("msda_forward: %s\n", msda_status_string(s));
  fails += s != MSDA_SUCCESS;
  size_t ws_bytes = 0;
  s = msda_backward_workspace_size(&shapes[0][0], starts, N, S, M, D, L, Lq, K, MSDA_F32, &ws_bytes);
  fails += s != MSDA_SUCCESS;
  void *ws = nullptr;
  HIP_OK(hipMalloc(&ws, ws_bytes));
  s = msda_backward(dv, &shapes[0][0], starts, dl, da, dg, dgv, dgl, dga, N, S, M, D, L, Lq, K, MSDA_F32, ws,
                    ws_bytes, stream);
  std::printf("msda_backward: %s\n", msda_status_string(s));
  fails += s != MSDA_SUCCESS;
  HIP_OK(hipStreamSynchronize(stream));

  std::vector<float> out(grad_out.size()), gv(value.size()), gl(loc.size()), ga(attn.size());
  HIP_OK(hipMemcpy(out.data(), dout, out.size() * 4, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(gv.data(), dgv, gv.size() * 4, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(gl.data(), dgl, gl.size() * 4, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(ga.data(), dga, ga.size() * 4, hipMemcpyDeviceToHost));

  double e_out = 0, e_ga = 0, e_gl = 0, lhs = 0, rhs = 0, scale = 0;
  for (int64_t q = 0; q < N * Lq; ++q)
    for (int64_t m = 0; m < M; ++m) {
      double dot = 0;
      for (int64_t d = 0; d < D; ++d) {
        const int64_t i = (q * M + m) * D + d;
        e_out = std::fmax(e_out, std::fabs((double)out[i] - (double)c(m, d)));
        dot += (double)grad_out[i] * (double)c(m, d);
        lhs += (double)grad_out[i] * (double)out[i];
        scale += std::fabs((double)grad_out[i] * (double)out[i]);
      }
      for (int64_t j = 0; j < LK; ++j) {
        const int64_t i = (q * M + m) * LK + j;
        e_ga = std::fmax(e_ga, std::fabs((double)ga[i] - dot));
        e_gl = std::fmax(e_gl, std::fmax(std::fabs((double)gl[2 * i]), std::fabs((double)gl[2 * i + 1])));
      }
    }
  for (size_t i = 0; i < gv.size(); ++i) rhs += (double)gv[i] * (double)value[i];
  const double e_adj = std::fabs(lhs - rhs) / scale;
  std::printf("out vs c_m: %.3e\ngrad_attn vs <G, c_m>: %.3e\ngrad_loc vs 0: %.3e\nadjoint: %.3e\n", e_out, e_ga,
              e_gl, e_adj);
  fails += !(e_out <= 1e-6) + !(e_ga <= 1e-5) + !(e_gl <= 1e-4) + !(e_adj <= 1e-6);

  // The same two calls captured into a HIP graph on this stream and replayed
  // twice; before each replay the outputs are overwritten (eagerly, outside
  // the graph) with NaN bytes. Every replay must reproduce the eager results:
  // out, grad_loc and grad_attn bit for bit, grad_value to 1e-6.
  hipGraph_t graph = nullptr;
  hipGraphExec_t exec = nullptr;
  HIP_OK(hipStreamBeginCapture(stream, hipStreamCaptureModeGlobal));
  msda_status s1 = msda_forward(dv, &shapes[0][0], starts, dl, da, dout, N, S, M, D, L, Lq, K, MSDA_F32, stream);
  msda_status s2 = msda_backward(dv, &shapes[0][0], starts, dl, da, dg, dgv, dgl, dga, N, S, M, D, L, Lq, K,
                                 MSDA_F32, ws, ws_bytes, stream);
  HIP_OK(hipStreamEndCapture(stream, &graph));
  std::printf("captured forward: %s, backward: %s\n", msda_status_string(s1), msda_status_string(s2));
  fails += (s1 != MSDA_SUCCESS) + (s2 != MSDA_SUCCESS);
  HIP_OK(hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0));
  for (int rep = 0; rep < 2; ++rep) {
    HIP_OK(hipMemsetAsync(dout, 0xff, out.size() * 4, stream));
    HIP_OK(hipMemsetAsync(dgv, 0xff, gv.size() * 4, stream));
    HIP_OK(hipMemsetAsync(dgl, 0xff, gl.size() * 4, stream));
    HIP_OK(hipMemsetAsync(dga, 0xff, ga.size() * 4, stream));
    HIP_OK(hipStreamSynchronize(stream));
    HIP_OK(hipGraphLaunch(exec, stream));
    HIP_OK(hipStreamSynchronize(stream));
    std::vector<float> out2(out.size()), gv2(gv.size()), gl2(gl.size()), ga2(ga.size());
    HIP_OK(hipMemcpy(out2.data(), dout, out2.size() * 4, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(gv2.data(), dgv, gv2.size() * 4, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(gl2.data(), dgl, gl2.size() * 4, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(ga2.data(), dga, ga2.size() * 4, hipMemcpyDeviceToHost));
    int diff = 0;
    double e_gv = 0;
    for (size_t i = 0; i < out.size(); ++i) diff += !(out2[i] == out[i]);
    for (size_t i = 0; i < gl.size(); ++i) diff += !(gl2[i] == gl[i]);
    for (size_t i = 0; i < ga.size(); ++i) diff += !(ga2[i] == ga[i]);
    for (size_t i = 0; i < gv.size(); ++i) {
      const double e = std::fabs((double)gv2[i] - (double)gv[i]);
      e_gv = (e == e) ? std::fmax(e_gv, e) : INFINITY;  // NaN left behind counts as a failure
    }
    std::printf("graph replay %d: %d differing out/grad_loc/grad_attn elements, grad_value %.3e\n", rep, diff, e_gv);
    fails += (diff != 0) + !(e_gv <= 1e-6);
  }
  HIP_OK(hipGraphExecDestroy(exec));
  HIP_OK(hipGraphDestroy(graph));

  HIP_OK(hipFree(ws));
  for (float *p : {dv, dl, da, dout, dg, dgv, dgl, dga}) HIP_OK(hipFree(p));
  HIP_OK(hipStreamDestroy(stream));
  std::printf("%s\n", fails ? "FAILED" : "OK");
  return fails ? 1 : 0;
}
