// Router logits of the routed forward: the gate of each token is a linear
// map of its local-branch output over all query heads ("Learning When to
// Attend", section "The Architecture of Conditional Attention": local
// attention first, then one routing decision per token). The local kernel's
// epilogue leaves <router_w[h], o_local[b][h][i]> per (b, h, i); this kernel
// adds the heads in order (deterministic) and the bias:
//   gate[b][i] = bias + sum_h part[b][h][i]
#include "logo_internal.h"

namespace logo {
namespace {

__global__ __launch_bounds__(256) void router_sum_kernel(const float* __restrict__ part,
                                                         float bias, float* __restrict__ gate,
                                                         int Hq, int n, long long positions) {
  const long long t = (long long)blockIdx.x * 256 + threadIdx.x;
  if (t >= positions) return;
  const long long b = t / n;
  const int i = (int)(t % n);
  float g = bias;
  for (int h = 0; h < Hq; ++h) g += part[(b * Hq + h) * n + i];
  gate[t] = g;
}

}  // namespace

hipError_t launch_router_sum(const Dims& d, const float* part, float bias, float* gate,
                             hipStream_t s) {
  const long long positions = (long long)d.B * d.n;
  if (positions == 0) return hipSuccess;
  hipLaunchKernelGGL(router_sum_kernel, dim3((unsigned)((positions + 255) / 256)), dim3(256), 0,
                     s, part, bias, gate, d.Hq, d.n, positions);
  return hipGetLastError();
}

}  // namespace logo
