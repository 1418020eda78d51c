// float32 attention kernels for both branches (float32 in, float32 math,
// float32 out; nothing is rounded to a narrower type). Same definitions as
// the bf16 kernels:
//   local  (every query):   softmax over L(i) = [max(0, i-W+1), i]
//   global (selected rows): softmax over G(i) = [0, i]
// ("Local-global attention", attention-mask sketch; "Learning When to
// Attend", "The Architecture of Conditional Attention").
//
// One wave per query row, keys in chunks of 64: lane j scores key j of the
// chunk (a full d-length dot product), the chunk's max and sum come from
// wave reductions, and each lane accumulates the output for its d columns
// (d/64 of them) with the chunk's probabilities broadcast across the wave.
// This path serves float32 problems, which are small; the bf16 path is the
// matrix-core one.
#include "logo_internal.h"

namespace logo {
namespace {

constexpr int kWaves = 4;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInit = -1.0e30f;

struct Params {
  const float* q;
  const float* k;
  const float* v;
  const int32_t* idx;
  const int32_t* rank;
  const float* gate;
  float* out_f32;
  const float* scratch;
  float* out_io;
  int B, Hq, Hkv, n, W, ksel;
  float scale_log2;
  long long rows;  // B * Hq * R
  View vq, vk, vv, vo;  // element strides of q, k, v, o
  float* lse_out;       // optional per-row log-sum-exp (natural log)
  float* og_out;        // optional f32 o_global rows (fused global)
  const float* router_w;  // routed local: [Hq][D]
  float* router_part;     // routed local: [B][Hq][n]
  const int32_t* seg_start;  // packed examples: [n] first token of the example, or NULL
};

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x = fmaxf(x, __shfl_xor(x, off, 64));
  return x;
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off, 64);
  return x;
}

template <int D, bool GLOBAL, int EPI>
__global__ __launch_bounds__(kWaves * 64) void attn_f32_kernel(Params p) {
  __shared__ float qs[kWaves][D];
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const long long row = (long long)blockIdx.x * kWaves + wave;
  if (row >= p.rows) return;  // whole wave leaves; no block barriers below
  const int R = GLOBAL ? p.ksel : p.n;
  const int r = (int)(row % R);
  const int bh = (int)(row / R);
  const int b = bh / p.Hq;
  const int h = bh % p.Hq;
  const int hk = h / (p.Hq / p.Hkv);
  int pos = GLOBAL ? p.idx[(size_t)b * p.ksel + r] : r;
  if (GLOBAL && p.seg_start) pos = min(max(pos, 0), p.n - 1);  // packed: defensive clamp
  const int ss = p.seg_start ? p.seg_start[pos] : 0;  // packed examples: example start
  const int lo = GLOBAL ? ss : max(ss, pos - p.W + 1);
  const int hi = pos;

  const float* qrow = p.q + b * p.vq.sb + h * p.vq.sh + (long long)pos * p.vq.st;
  for (int e = lane; e < D; e += 64) qs[wave][e] = qrow[e];
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

  const float* kg = p.k + b * p.vk.sb + hk * p.vk.sh;
  const float* vg = p.v + b * p.vv.sb + hk * p.vv.sh;

  constexpr int NC = D / 64;  // output columns per lane
  float acc[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) acc[c] = 0.0f;
  float m_run = kNegInit, l_run = 0.0f;

  for (int j0 = lo; j0 <= hi; j0 += 64) {
    const int j = j0 + lane;
    float s = -INFINITY;
    if (j <= hi) {
      const float4* kr = reinterpret_cast<const float4*>(kg + (size_t)j * p.vk.st);
      float dot = 0.0f;
#pragma unroll 8
      for (int e4 = 0; e4 < D / 4; ++e4) {
        float4 kv = kr[e4];
        dot = fmaf(qs[wave][4 * e4 + 0], kv.x, dot);
        dot = fmaf(qs[wave][4 * e4 + 1], kv.y, dot);
        dot = fmaf(qs[wave][4 * e4 + 2], kv.z, dot);
        dot = fmaf(qs[wave][4 * e4 + 3], kv.w, dot);
      }
      s = dot * p.scale_log2;
    }
    const float m_new = fmaxf(m_run, wave_max(s));
    const float alpha = exp2f(m_run - m_new);
    const float pj = exp2f(s - m_new);
    l_run = l_run * alpha + wave_sum(pj);
    m_run = m_new;
#pragma unroll
    for (int c = 0; c < NC; ++c) acc[c] *= alpha;
    const int cnt = min(64, hi - j0 + 1);
    for (int jj = 0; jj < cnt; ++jj) {
      const float pw = __shfl(pj, jj, 64);
      const float* vr = vg + (size_t)(j0 + jj) * p.vv.st;
#pragma unroll
      for (int c = 0; c < NC; ++c) acc[c] = fmaf(pw, vr[lane + 64 * c], acc[c]);
    }
  }

  const float inv = 1.0f / l_run;
  const size_t head_row = (size_t)(b * p.Hq + h);
  if (p.lse_out && lane == 0)
    p.lse_out[head_row * R + (GLOBAL ? r : pos)] = (m_run + log2f(l_run)) * kLn2;
  float* const orow = p.out_io + b * p.vo.sb + h * p.vo.sh + (long long)pos * p.vo.st;
  float sig = 0.0f;
  if (EPI == 3 || EPI == 5) sig = 1.0f / (1.0f + expf(-p.gate[(size_t)b * p.n + pos]));
  float rdot = 0.0f;
  int rk = -1;
  if (EPI == 1) {
    rk = p.rank[(size_t)b * p.n + pos];
    if (rk >= p.ksel) rk = -1;  // never address past the scratch rows
  }
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const int e = lane + 64 * c;
    const float o = acc[c] * inv;
    if (EPI == 0) {
      p.out_f32[(head_row * p.n + pos) * D + e] = o;
    } else if (EPI == 4) {
      p.out_f32[(head_row * p.n + pos) * D + e] = o;
      orow[e] = o;
      rdot = fmaf(o, p.router_w[(size_t)h * D + e], rdot);
    } else if (EPI == 5) {
      orow[e] = p.scratch[(head_row * p.n + pos) * D + e] + sig * o;
    } else if (EPI == 2) {
      p.out_f32[(head_row * p.ksel + r) * D + e] = o;
    } else if (EPI == 1) {
      if (rk >= 0) p.out_f32[(head_row * p.ksel + rk) * D + e] = o;
      else orow[e] = o;
    } else {
      const float l = p.scratch[(head_row * p.ksel + r) * D + e];
      if (p.og_out) p.og_out[(head_row * p.ksel + r) * D + e] = o;
      orow[e] = l + sig * o;
    }
  }
  if (EPI == 4) {
    rdot = wave_sum(rdot);
    if (lane == 0) p.router_part[head_row * p.n + pos] = rdot;
  }
}

template <int D, bool GLOBAL, int EPI>
hipError_t launch_one(const Params& prm, hipStream_t s) {
  const long long blocks = (prm.rows + kWaves - 1) / kWaves;
  hipLaunchKernelGGL((attn_f32_kernel<D, GLOBAL, EPI>), dim3((unsigned)blocks),
                     dim3(kWaves * 64), 0, s, prm);
  return hipGetLastError();
}

template <int D>
hipError_t dispatch_epi(Epi epi, const Params& prm, hipStream_t s) {
  switch (epi) {
    case Epi::LocalAll: return launch_one<D, false, 0>(prm, s);
    case Epi::LocalFused: return launch_one<D, false, 1>(prm, s);
    case Epi::GlobalAll: return launch_one<D, true, 2>(prm, s);
    case Epi::GlobalFused: return launch_one<D, true, 3>(prm, s);
    case Epi::LocalRouted: return launch_one<D, false, 4>(prm, s);
    case Epi::GlobalRouted: return launch_one<D, true, 5>(prm, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_attn_f32(const Dims& d, Epi epi, const AttnArgs& a, hipStream_t s) {
  const bool global =
      epi == Epi::GlobalAll || epi == Epi::GlobalFused || epi == Epi::GlobalRouted;
  const int R = global ? d.k : d.n;
  if (d.B == 0 || R == 0) return hipSuccess;
  Params prm;
  prm.q = static_cast<const float*>(a.q);
  prm.k = static_cast<const float*>(a.k);
  prm.v = static_cast<const float*>(a.v);
  prm.idx = a.idx;
  prm.rank = a.rank;
  prm.gate = a.gate;
  prm.out_f32 = a.out_f32;
  prm.scratch = a.scratch;
  prm.out_io = static_cast<float*>(a.out_io);
  prm.B = d.B;
  prm.Hq = d.Hq;
  prm.Hkv = d.Hkv;
  prm.n = d.n;
  prm.W = d.window;
  prm.ksel = d.k;
  prm.scale_log2 = d.scale * kLog2e;
  prm.rows = (long long)d.B * d.Hq * R;
  prm.vq = d.vq;
  prm.vk = d.vk;
  prm.vv = d.vv;
  prm.vo = d.vo;
  prm.lse_out = a.lse_out;
  prm.og_out = a.og_out;
  prm.router_w = a.router_w;
  prm.router_part = a.router_part;
  prm.seg_start = a.seg_start;
  if (d.d == 64) return dispatch_epi<64>(epi, prm, s);
  if (d.d == 128) return dispatch_epi<128>(epi, prm, s);
  return hipErrorInvalidValue;
}

}  // namespace logo
