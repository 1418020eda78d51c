// float32 backward of both attention branches (SIMT; the float32 I/O path).
//
// Same quantities as the bf16 kernels (backward_bf16.hip): with the
// selection held fixed, a softmax row with upstream gradient e (do_i for
// local rows over L(i) = [max(0, i-W+1), i], g_i do_i for selected rows over
// G(i) = [0, i]; "Local-global attention", attention-mask sketch; "Learning
// When to Attend", "The Architecture of Conditional Attention") gives
//   p_j = exp(scale <q, k_j> - lse),  ds_j = p_j (<e, v_j> - Dr)
//   dq += scale sum_j ds_j k_j,  dk_j += scale ds_j q,  dv_j += p_j e.
//
// bwd_dq_f32_kernel: one wave per query row; lanes take 64 keys at a time
//   for the scores, then one d column each for the dq sum.
// bwd_dkdv_f32_kernel: one wave per key; lanes take 64 reading rows at a
//   time (local rows of its window, then selected rows at or after it, for
//   every query head of the group), then one d column each for the sums.
#include "logo_internal.h"

namespace logo {
namespace {

constexpr int kWaves = 4;

__device__ __forceinline__ float dot_row(const float* a, const float* b_lds, int D) {
  const float4* a4 = reinterpret_cast<const float4*>(a);
  float acc = 0.0f;
  for (int e4 = 0; e4 < D / 4; ++e4) {
    const float4 x = a4[e4];
    acc = fmaf(x.x, b_lds[4 * e4 + 0], acc);
    acc = fmaf(x.y, b_lds[4 * e4 + 1], acc);
    acc = fmaf(x.z, b_lds[4 * e4 + 2], acc);
    acc = fmaf(x.w, b_lds[4 * e4 + 3], acc);
  }
  return acc;
}

struct DqF32Params {
  const float* q;
  const float* k;
  const float* v;
  const float* dout;
  const float* qs;
  const float* dog;
  const int32_t* idx;
  const float* lse;
  const float* Dr;
  float* dq;
  int Hq, Hkv, n, W, ksel;
  float scale;
  long long rows;
  View vq, vk, vv, vo;
};

template <int D, bool GLOBAL>
__global__ __launch_bounds__(256) void bwd_dq_f32_kernel(DqF32Params p) {
  __shared__ float qsh[kWaves][D];
  __shared__ float esh[kWaves][D];
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const long long row = (long long)blockIdx.x * kWaves + wave;
  if (row >= p.rows) return;  // whole wave leaves; no block barriers below
  const int R = GLOBAL ? p.ksel : p.n;
  const int r = (int)(row % R);
  const long long bh = row / R;
  const int b = (int)(bh / p.Hq);
  const int h = (int)(bh % p.Hq);
  const int hk = h / (p.Hq / p.Hkv);
  const int pos = GLOBAL ? p.idx[(size_t)b * p.ksel + r] : r;
  const int lo = GLOBAL ? 0 : max(0, pos - p.W + 1);
  const float* qr = GLOBAL ? p.qs + (bh * p.ksel + r) * D
                           : p.q + b * p.vq.sb + h * p.vq.sh + (long long)pos * p.vq.st;
  const float* er = GLOBAL ? p.dog + (bh * p.ksel + r) * D
                           : p.dout + b * p.vo.sb + h * p.vo.sh + (long long)pos * p.vo.st;
  for (int e = lane; e < D; e += 64) {
    qsh[wave][e] = qr[e];
    esh[wave][e] = er[e];
  }
  __builtin_amdgcn_wave_barrier();
  const float lse = p.lse[bh * R + r];
  const float dr = p.Dr[bh * R + r];
  const float* kg = p.k + b * p.vk.sb + hk * p.vk.sh;
  const float* vg = p.v + b * p.vv.sb + hk * p.vv.sh;
  constexpr int NC = D / 64;
  float acc[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) acc[c] = 0.0f;
  for (int j0 = lo; j0 <= pos; j0 += 64) {
    const int j = j0 + lane;
    float ds = 0.0f;
    if (j <= pos) {
      const float s = dot_row(kg + (long long)j * p.vk.st, qsh[wave], D) * p.scale;
      const float pr = expf(s - lse);
      const float dp = dot_row(vg + (long long)j * p.vv.st, esh[wave], D);
      ds = pr * (dp - dr);
    }
    const int cnt = min(64, pos - j0 + 1);
    for (int jj = 0; jj < cnt; ++jj) {
      const float dsj = __shfl(ds, jj, 64);
      const float* kr = kg + (long long)(j0 + jj) * p.vk.st;
#pragma unroll
      for (int c = 0; c < NC; ++c) acc[c] = fmaf(dsj, kr[lane + 64 * c], acc[c]);
    }
  }
  float* out = p.dq + (bh * p.n + pos) * D;
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const float x = p.scale * acc[c];
    if (GLOBAL) out[lane + 64 * c] += x;
    else out[lane + 64 * c] = x;
  }
}

struct DkdvF32Params {
  const float* q;
  const float* k;
  const float* v;
  const float* dout;
  const float* qs;
  const float* dog;
  const int32_t* idx;
  const float* lse_l;
  const float* lse_g;
  const float* D_l;
  const float* D_g;
  float* dk;
  float* dv;
  int Hq, Hkv, n, W, ksel;
  float scale;
  long long keys;  // B * Hkv * n
  View vq, vk, vv, vo;
};

template <int D>
__global__ __launch_bounds__(256) void bwd_dkdv_f32_kernel(DkdvF32Params p) {
  __shared__ float ksh[kWaves][D];
  __shared__ float vsh[kWaves][D];
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const long long kid = (long long)blockIdx.x * kWaves + wave;
  if (kid >= p.keys) return;  // whole wave leaves; no block barriers below
  const int j = (int)(kid % p.n);
  const long long bk = kid / p.n;
  const int b = (int)(bk / p.Hkv);
  const int hk = (int)(bk % p.Hkv);
  const int G = p.Hq / p.Hkv;
  const float* kr = p.k + b * p.vk.sb + hk * p.vk.sh + (long long)j * p.vk.st;
  const float* vr = p.v + b * p.vv.sb + hk * p.vv.sh + (long long)j * p.vv.st;
  for (int e = lane; e < D; e += 64) {
    ksh[wave][e] = kr[e];
    vsh[wave][e] = vr[e];
  }
  __builtin_amdgcn_wave_barrier();
  constexpr int NC = D / 64;
  float adk[NC], adv[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) adk[c] = adv[c] = 0.0f;

  const int* idx_b = p.idx + (size_t)b * p.ksel;
  int r_start = 0;
  {
    int lo = 0, hi = p.ksel;
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (idx_b[mid] < j) lo = mid + 1;
      else hi = mid;
    }
    r_start = lo;
  }
  const int i_end = min(p.n - 1, j + p.W - 1);
  for (int hl = 0; hl < G; ++hl) {
    const int h = hk * G + hl;
    const long long hb = (long long)b * p.Hq + h;
    // kind 0: local rows j..i_end; kind 1: selected rows r_start..k-1
    for (int kind = 0; kind < 2; ++kind) {
      const int first = kind == 0 ? j : r_start;
      const int last = kind == 0 ? i_end : p.ksel - 1;
      for (int c0 = first; c0 <= last; c0 += 64) {
        const int rr = c0 + lane;
        float pr = 0.0f, ds = 0.0f;
        if (rr <= last) {
          const float* qrow;
          const float* erow;
          float lse, dr;
          if (kind == 0) {
            qrow = p.q + b * p.vq.sb + h * p.vq.sh + (long long)rr * p.vq.st;
            erow = p.dout + b * p.vo.sb + h * p.vo.sh + (long long)rr * p.vo.st;
            lse = p.lse_l[hb * p.n + rr];
            dr = p.D_l[hb * p.n + rr];
          } else {
            qrow = p.qs + (hb * p.ksel + rr) * D;
            erow = p.dog + (hb * p.ksel + rr) * D;
            lse = p.lse_g[hb * p.ksel + rr];
            dr = p.D_g[hb * p.ksel + rr];
          }
          const float s = dot_row(qrow, ksh[wave], D) * p.scale;
          pr = expf(s - lse);
          const float dp = dot_row(erow, vsh[wave], D);
          ds = pr * (dp - dr);
        }
        const int cnt = min(64, last - c0 + 1);
        for (int t = 0; t < cnt; ++t) {
          const float prt = __shfl(pr, t, 64);
          const float dst = __shfl(ds, t, 64);
          const int r2 = c0 + t;
          const float* qrow;
          const float* erow;
          if (kind == 0) {
            qrow = p.q + b * p.vq.sb + h * p.vq.sh + (long long)r2 * p.vq.st;
            erow = p.dout + b * p.vo.sb + h * p.vo.sh + (long long)r2 * p.vo.st;
          } else {
            qrow = p.qs + (hb * p.ksel + r2) * D;
            erow = p.dog + (hb * p.ksel + r2) * D;
          }
#pragma unroll
          for (int c = 0; c < NC; ++c) {
            adv[c] = fmaf(prt, erow[lane + 64 * c], adv[c]);
            adk[c] = fmaf(dst, qrow[lane + 64 * c], adk[c]);
          }
        }
      }
    }
  }
  float* dkr = p.dk + (bk * p.n + j) * D;
  float* dvr = p.dv + (bk * p.n + j) * D;
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    dkr[lane + 64 * c] = p.scale * adk[c];
    dvr[lane + 64 * c] = adv[c];
  }
}

template <int D, bool GLOBAL>
hipError_t dq_f32_t(const Dims& d, const BwdArgs& a, hipStream_t s) {
  const int R = GLOBAL ? d.k : d.n;
  DqF32Params p;
  p.q = static_cast<const float*>(a.q);
  p.k = static_cast<const float*>(a.k);
  p.v = static_cast<const float*>(a.v);
  p.dout = static_cast<const float*>(a.dout);
  p.qs = static_cast<const float*>(a.qs);
  p.dog = static_cast<const float*>(a.dog);
  p.idx = a.idx;
  p.lse = GLOBAL ? a.lse_g : a.lse_l;
  p.Dr = GLOBAL ? a.D_g : a.D_l;
  p.dq = a.dq;
  p.Hq = d.Hq;
  p.Hkv = d.Hkv;
  p.n = d.n;
  p.W = d.window;
  p.ksel = d.k;
  p.scale = d.scale;
  p.rows = (long long)d.B * d.Hq * R;
  p.vq = d.vq;
  p.vk = d.vk;
  p.vv = d.vv;
  p.vo = d.vo;
  if (p.rows == 0) return hipSuccess;
  hipLaunchKernelGGL((bwd_dq_f32_kernel<D, GLOBAL>), dim3((unsigned)((p.rows + 3) / 4)),
                     dim3(256), 0, s, p);
  return hipGetLastError();
}

template <int D>
hipError_t dkdv_f32_t(const Dims& d, const BwdArgs& a, hipStream_t s) {
  DkdvF32Params p;
  p.q = static_cast<const float*>(a.q);
  p.k = static_cast<const float*>(a.k);
  p.v = static_cast<const float*>(a.v);
  p.dout = static_cast<const float*>(a.dout);
  p.qs = static_cast<const float*>(a.qs);
  p.dog = static_cast<const float*>(a.dog);
  p.idx = a.idx;
  p.lse_l = a.lse_l;
  p.lse_g = a.lse_g;
  p.D_l = a.D_l;
  p.D_g = a.D_g;
  p.dk = a.dk;
  p.dv = a.dv;
  p.Hq = d.Hq;
  p.Hkv = d.Hkv;
  p.n = d.n;
  p.W = d.window;
  p.ksel = d.k;
  p.scale = d.scale;
  p.keys = (long long)d.B * d.Hkv * d.n;
  p.vq = d.vq;
  p.vk = d.vk;
  p.vv = d.vv;
  p.vo = d.vo;
  if (p.keys == 0) return hipSuccess;
  hipLaunchKernelGGL((bwd_dkdv_f32_kernel<D>), dim3((unsigned)((p.keys + 3) / 4)), dim3(256), 0,
                     s, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd_dq_f32(const Dims& d, bool global, const BwdArgs& a, hipStream_t s) {
  if (d.B == 0 || d.n == 0) return hipSuccess;
  if (d.d == 64) return global ? dq_f32_t<64, true>(d, a, s) : dq_f32_t<64, false>(d, a, s);
  if (d.d == 128) return global ? dq_f32_t<128, true>(d, a, s) : dq_f32_t<128, false>(d, a, s);
  return hipErrorInvalidValue;
}

hipError_t launch_bwd_dkdv_f32(const Dims& d, const BwdArgs& a, hipStream_t s) {
  if (d.B == 0 || d.n == 0) return hipSuccess;
  if (d.d == 64) return dkdv_f32_t<64>(d, a, s);
  if (d.d == 128) return dkdv_f32_t<128>(d, a, s);
  return hipErrorInvalidValue;
}

}  // namespace logo
