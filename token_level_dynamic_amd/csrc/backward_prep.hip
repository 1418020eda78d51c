// Row terms of the backward, for both I/O dtypes.
//
// The forward is o_i = o_local_i + [i in S] g_i o_global_i with g_i =
// sigmoid(gate_i) (LoGo abstract: a learned gate activates global attention;
// "Learning When to Attend", "The Architecture of Conditional Attention":
// exact full-context attention for the selected tokens). With the selection
// held fixed, a softmax-attention row with upstream gradient e needs, besides
// its probabilities, the scalar <e, o_row> (the probability-weighted mean of
// <e, v_j>). This file computes those scalars for every row of both
// branches, gathers the selected rows' queries and gated upstream gradients
// into dense arrays for the matrix-core kernels (with each row's lse in log2
// units, as those kernels exponentiate), and the gate gradient
//   dgate_i = g_i (1 - g_i) sum_h <do_{h,i}, o_global_{h,i}>   (i in S), 0 elsewhere.
#include "logo_internal.h"

namespace logo {
namespace {

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  bf16x2 r = __builtin_convertvector((f32x2){a, b}, bf16x2);
  return __builtin_bit_cast(uint32_t, r);
}

// 8 consecutive elements of an I/O-dtype row as float.
template <bool BF16>
__device__ __forceinline__ void load8(const void* base, long long off, float (&x)[8]) {
  if (BF16) {
    const uint4 u = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(base) + off);
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = __uint_as_float(w[i] << 16);
      x[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  } else {
    const float4* f = reinterpret_cast<const float4*>(static_cast<const float*>(base) + off);
    const float4 a = f[0], b = f[1];
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
    x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
  }
}

template <bool BF16>
__device__ __forceinline__ void store8(void* base, long long off, const float (&x)[8]) {
  if (BF16) {
    *reinterpret_cast<uint4*>(static_cast<uint16_t*>(base) + off) =
        make_uint4(pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]), pack_bf16x2(x[4], x[5]),
                   pack_bf16x2(x[6], x[7]));
  } else {
    float4* f = reinterpret_cast<float4*>(static_cast<float*>(base) + off);
    f[0] = make_float4(x[0], x[1], x[2], x[3]);
    f[1] = make_float4(x[4], x[5], x[6], x[7]);
  }
}

// x as stored in the I/O dtype (bf16: round to nearest even), back as float.
template <bool BF16>
__device__ __forceinline__ float round_io(float x) {
  if (!BF16) return x;
  const uint32_t w = pack_bf16x2(x, 0.0f);
  return __uint_as_float(w << 16);
}

__device__ __forceinline__ void load8f(const float* base, long long off, float (&x)[8]) {
  const float4* f = reinterpret_cast<const float4*>(base + off);
  const float4 a = f[0], b = f[1];
  x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
  x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
}

struct PrepParams {
  const void* q;
  const void* o;
  const void* dout;
  const float* gate;
  const int32_t* rank;
  const float* o_ls;
  const float* o_g;
  float* D_l;
  float* D_g;
  const float* lse_l;
  const float* lse_g;
  float* L2_l;
  float* L2_g;
  void* qs;
  void* dog;
  int Hq, n, ksel;
  long long rows;  // B * Hq * n
  View vq, vo;
};

// TPR threads per row, 8 elements each; groups of TPR lanes reduce by xor
// shuffles (TPR divides 64, so a group never straddles a wave).
template <int D, bool BF16>
__global__ __launch_bounds__(256) void bwd_rows_kernel(PrepParams p) {
  constexpr int TPR = D / 8;
  const long long t = (long long)blockIdx.x * 256 + threadIdx.x;
  const long long row = t / TPR;
  const int c = (int)(t % TPR) * 8;
  const bool live = row < p.rows;
  const long long rr = live ? row : 0;
  const int i = (int)(rr % p.n);
  const long long bh = rr / p.n;
  const int b = (int)(bh / p.Hq);
  const int h = (int)(bh % p.Hq);
  const int rk = p.rank[(size_t)b * p.n + i];
  const long long oo = b * p.vo.sb + h * p.vo.sh + (long long)i * p.vo.st + c;
  float dov[8], ol[8];
  load8<BF16>(p.dout, oo, dov);
  if (rk >= 0)
    load8f(p.o_ls, ((long long)bh * p.ksel + rk) * D + c, ol);
  else
    load8<BF16>(p.o, oo, ol);
  float dl = 0.0f, dg = 0.0f;
#pragma unroll
  for (int e = 0; e < 8; ++e) dl = fmaf(dov[e], ol[e], dl);
  // g * dout of a selected row, rounded as the matrix-core kernels will read
  // it, so that its D term and their dP agree (each row's ds then sums to 0)
  float gd[8];
  if (rk >= 0) {
    const float g = 1.0f / (1.0f + expf(-p.gate[(size_t)b * p.n + i]));
#pragma unroll
    for (int e = 0; e < 8; ++e) gd[e] = round_io<BF16>(g * dov[e]);
    float og[8];
    load8f(p.o_g, ((long long)bh * p.ksel + rk) * D + c, og);
#pragma unroll
    for (int e = 0; e < 8; ++e) dg = fmaf(gd[e], og[e], dg);
  }
#pragma unroll
  for (int off = TPR / 2; off >= 1; off >>= 1) {
    dl += __shfl_xor(dl, off, 64);
    dg += __shfl_xor(dg, off, 64);
  }
  if (!live) return;
  if (c == 0) {
    p.D_l[rr] = dl;
    p.L2_l[rr] = p.lse_l[rr] * kLog2e;
  }
  if (rk >= 0) {
    const long long cr = (long long)bh * p.ksel + rk;
    if (c == 0) {
      p.D_g[cr] = dg;
      p.L2_g[cr] = p.lse_g[cr] * kLog2e;
    }
    float qv[8];
    load8<BF16>(p.q, b * p.vq.sb + h * p.vq.sh + (long long)i * p.vq.st + c, qv);
    store8<BF16>(p.qs, cr * D + c, qv);
    store8<BF16>(p.dog, cr * D + c, gd);
  }
}

struct GateParams {
  const void* dout;
  const float* gate;
  const int32_t* rank;
  const float* o_g;
  float* dgate;
  int Hq, n, ksel;
  long long positions;  // B * n
  View vo;
};

// One wave per (b, i); the sum over heads runs in head order (deterministic).
template <int D, bool BF16>
__global__ __launch_bounds__(256) void bwd_dgate_kernel(GateParams p) {
  const long long w = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (w >= p.positions) return;
  const int b = (int)(w / p.n);
  const int i = (int)(w % p.n);
  const int rk = p.rank[w];
  if (rk < 0) {
    if (lane == 0) p.dgate[w] = 0.0f;
    return;
  }
  float acc = 0.0f;
  for (int h = 0; h < p.Hq; ++h) {
    const long long oo = b * p.vo.sb + h * p.vo.sh + (long long)i * p.vo.st;
    const float* og = p.o_g + (((long long)b * p.Hq + h) * p.ksel + rk) * D;
#pragma unroll
    for (int e = lane; e < D; e += 64) {
      const float dv = BF16 ? __uint_as_float((uint32_t)static_cast<const uint16_t*>(p.dout)[oo + e]
                                              << 16)
                            : static_cast<const float*>(p.dout)[oo + e];
      acc = fmaf(dv, og[e], acc);
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) acc += __shfl_xor(acc, off, 64);
  if (lane == 0) {
    const float g = 1.0f / (1.0f + expf(-p.gate[w]));
    p.dgate[w] = g * (1.0f - g) * acc;
  }
}

template <int D, bool BF16>
hipError_t launch_prep_t(const Dims& d, const BwdArgs& a, hipStream_t s) {
  PrepParams pp;
  pp.q = a.q;
  pp.o = a.o;
  pp.dout = a.dout;
  pp.gate = a.gate;
  pp.rank = a.rank;
  pp.o_ls = a.o_ls;
  pp.o_g = a.o_g;
  pp.D_l = a.D_l;
  pp.D_g = a.D_g;
  pp.lse_l = a.lse_l;
  pp.lse_g = a.lse_g;
  pp.L2_l = a.L2_l;
  pp.L2_g = a.L2_g;
  pp.qs = a.qs;
  pp.dog = a.dog;
  pp.Hq = d.Hq;
  pp.n = d.n;
  pp.ksel = d.k;
  pp.rows = (long long)d.B * d.Hq * d.n;
  pp.vq = d.vq;
  pp.vo = d.vo;
  const long long threads = pp.rows * (D / 8);
  hipLaunchKernelGGL((bwd_rows_kernel<D, BF16>), dim3((unsigned)((threads + 255) / 256)),
                     dim3(256), 0, s, pp);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  GateParams gp;
  gp.dout = a.dout;
  gp.gate = a.gate;
  gp.rank = a.rank;
  gp.o_g = a.o_g;
  gp.dgate = a.dgate;
  gp.Hq = d.Hq;
  gp.n = d.n;
  gp.ksel = d.k;
  gp.positions = (long long)d.B * d.n;
  gp.vo = d.vo;
  hipLaunchKernelGGL((bwd_dgate_kernel<D, BF16>), dim3((unsigned)((gp.positions + 3) / 4)),
                     dim3(256), 0, s, gp);
  return hipGetLastError();
}

}  // namespace

BwdWorkspace bwd_workspace(const Dims& d) {
  auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  const size_t es = d.dtype == 1 ? 2 : 4;
  BwdWorkspace w;
  w.D_l = 0;
  w.D_g = up((size_t)d.B * d.Hq * d.n * 4);
  w.L2_l = w.D_g + up((size_t)d.B * d.Hq * d.k * 4);
  w.L2_g = w.L2_l + up((size_t)d.B * d.Hq * d.n * 4);
  w.qs = w.L2_g + up((size_t)d.B * d.Hq * d.k * 4);
  w.dog = w.qs + up((size_t)d.B * d.Hq * d.k * d.d * es);
  w.total = w.dog + up((size_t)d.B * d.Hq * d.k * d.d * es);
  return w;
}

hipError_t launch_bwd_prep(const Dims& d, const BwdArgs& a, hipStream_t s) {
  if (d.B == 0 || d.n == 0) return hipSuccess;
  const bool bf = d.dtype == 1;
  if (d.d == 64) return bf ? launch_prep_t<64, true>(d, a, s) : launch_prep_t<64, false>(d, a, s);
  if (d.d == 128)
    return bf ? launch_prep_t<128, true>(d, a, s) : launch_prep_t<128, false>(d, a, s);
  return hipErrorInvalidValue;
}

}  // namespace logo
