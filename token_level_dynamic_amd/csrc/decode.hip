// Threshold budget controller and the decode step, for both I/O dtypes.
//
// LoGo (abstract): a learned gate activates global attention per token and a
// threshold-based budget controller holds the target global ratio. "Learning
// When to Attend" (section "Empirical Validation and System Optimization"):
// decoding reads the full context only for tokens routed to it.
//
//   controller: sel_b = gate_b > tau_b;  tau_b <- tau_b + eta (sel_b - rho)
//   decode:     query at i = lens_b - 1 over its cache; o = o_local over
//               [max(0, i-W+1), i], plus sigmoid(gate_b) o_global over [0, i]
//               when sel_b
//
// The decode step is bandwidth-bound (each cached key and value is read
// once per step, shared by the Hq/Hkv query heads of its kv head). It is
// split over chunks of kChunk keys: one workgroup per (b, kv head, chunk)
// keeps an online softmax per query head and branch (local: keys of the
// window; global: every key, only when the sequence is selected) and writes
// a partial (max, sum, weighted values); chunks with nothing to do exit at
// once. A reduction kernel merges the partials of each (b, query head).
#include <math.h>

#include "logo_internal.h"

namespace logo {
namespace {

constexpr int kChunk = 2048;      // keys per workgroup
constexpr int kSub = 64;          // keys per wave step (one per lane)
constexpr int kDecWaves = 4;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNeg = -1.0e30f;

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  bf16x2 r = __builtin_convertvector((f32x2){a, b}, bf16x2);
  return __builtin_bit_cast(uint32_t, r);
}

template <bool BF16>
__device__ __forceinline__ float ld_io(const void* base, long long i) {
  if (BF16) return __uint_as_float((uint32_t)static_cast<const uint16_t*>(base)[i] << 16);
  return static_cast<const float*>(base)[i];
}

__device__ __forceinline__ float wmax(float x) {
  for (int off = 32; off >= 1; off >>= 1) x = fmaxf(x, __shfl_xor(x, off, 64));
  return x;
}
__device__ __forceinline__ float wsum(float x) {
  for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off, 64);
  return x;
}

__device__ __forceinline__ int clamp_len(int len, int cap) { return min(max(len, 1), cap); }

__global__ void decode_ctrl_kernel(const float* gate, float* tau, uint8_t* selected, int B,
                                   float rho, float eta) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= B) return;
  const float g = gate[b];
  const float t = tau[b];
  const bool sel = g > t;  // NaN: false
  selected[b] = sel ? 1 : 0;
  tau[b] = t + eta * ((sel ? 1.0f : 0.0f) - rho);
}

struct DecParams {
  const void* q;       // [B][Hq][D]
  const void* kc;      // [B][Hkv][cap][D]
  const void* vc;
  const int32_t* lens;
  const uint8_t* selected;
  float* part;         // [B][Hq][nchunk][2][D + 2]: acc[D], max (log2 units), sum
  int B, Hq, Hkv, cap, W, nchunk;
  float scale_log2;
};

// One workgroup per (b, kv head, chunk); waves take 64-key steps of the chunk
// in turn, lane = key for the scores, lane = d column pair for the values.
template <int D, int G, bool BF16>
__global__ __launch_bounds__(kDecWaves * 64) void decode_partial_kernel(DecParams p) {
  constexpr int NC = D / 64;  // d columns per lane
  __shared__ float qs[G][D];
  __shared__ float pw[kDecWaves][2][G][kSub];  // probabilities of a wave step
  __shared__ float red[kDecWaves][2][G][D + 2];
  const int c = blockIdx.x % p.nchunk;
  const int bk = blockIdx.x / p.nchunk;
  const int b = bk / p.Hkv, hk = bk % p.Hkv;
  const int i = clamp_len(p.lens[b], p.cap) - 1;
  const int lo = max(0, i - p.W + 1);
  const bool sel = p.selected[b] != 0;
  const int c0 = c * kChunk, c1 = min(c0 + kChunk, i + 1);  // keys [c0, c1)
  const bool do_loc = c0 <= i && c1 > lo;
  const bool do_glb = sel && c0 <= i;
  if (!do_loc && !do_glb) return;  // uniform over the workgroup: no barrier is skipped
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  for (int e = tid; e < G * D; e += kDecWaves * 64)
    qs[e / D][e % D] = ld_io<BF16>(p.q, ((long long)b * p.Hq + hk * G + e / D) * D + e % D);
  __syncthreads();
  const long long kvb = ((long long)b * p.Hkv + hk) * p.cap;
  // online state per head and branch (0 local, 1 global)
  float m[2][G], l[2][G], acc[2][G][NC];
#pragma unroll
  for (int br = 0; br < 2; ++br)
#pragma unroll
    for (int g = 0; g < G; ++g) {
      m[br][g] = kNeg;
      l[br][g] = 0.0f;
#pragma unroll
      for (int cc = 0; cc < NC; ++cc) acc[br][g][cc] = 0.0f;
    }
  for (int j0 = c0 + wave * kSub; j0 < c1; j0 += kDecWaves * kSub) {
    const int j = j0 + lane;
    const bool valid = j < c1;
    const bool inwin = valid && j >= lo;
    float s[G];
#pragma unroll
    for (int g = 0; g < G; ++g) s[g] = 0.0f;
    if (valid) {
      const long long kr = (kvb + j) * D;
      for (int e = 0; e < D; e += 8) {
        float kv[8];
        if (BF16) {
          const uint4 u = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(p.kc) + kr + e);
          const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            kv[2 * t] = __uint_as_float(w[t] << 16);
            kv[2 * t + 1] = __uint_as_float(w[t] & 0xffff0000u);
          }
        } else {
          const float4 a = *reinterpret_cast<const float4*>(static_cast<const float*>(p.kc) + kr + e);
          const float4 bq = *reinterpret_cast<const float4*>(static_cast<const float*>(p.kc) + kr + e + 4);
          kv[0] = a.x; kv[1] = a.y; kv[2] = a.z; kv[3] = a.w;
          kv[4] = bq.x; kv[5] = bq.y; kv[6] = bq.z; kv[7] = bq.w;
        }
#pragma unroll
        for (int g = 0; g < G; ++g)
#pragma unroll
          for (int t = 0; t < 8; ++t) s[g] = fmaf(qs[g][e + t], kv[t], s[g]);
      }
    }
    // per head: new maxima, probabilities of this step, rescale
#pragma unroll
    for (int br = 0; br < 2; ++br) {
      if (br == 0 ? !do_loc : !do_glb) continue;
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const bool in = br == 0 ? inwin : valid;
        const float x = in ? s[g] * p.scale_log2 : kNeg;
        const float mn = fmaxf(m[br][g], wmax(x));
        const float alpha = exp2f(m[br][g] - mn);
        const float pr = in ? exp2f(x - mn) : 0.0f;
        l[br][g] = l[br][g] * alpha + wsum(pr);
        m[br][g] = mn;
#pragma unroll
        for (int cc = 0; cc < NC; ++cc) acc[br][g][cc] *= alpha;
        pw[wave][br][g][lane] = pr;
      }
    }
    __builtin_amdgcn_wave_barrier();
    // values: lane owns d columns lane + 64 cc
    const int cnt = min(kSub, c1 - j0);
    for (int jj = 0; jj < cnt; ++jj) {
      const long long vr = (kvb + j0 + jj) * D;
      float vv[NC];
#pragma unroll
      for (int cc = 0; cc < NC; ++cc) vv[cc] = ld_io<BF16>(p.vc, vr + lane + 64 * cc);
#pragma unroll
      for (int br = 0; br < 2; ++br) {
        if (br == 0 ? !do_loc : !do_glb) continue;
#pragma unroll
        for (int g = 0; g < G; ++g) {
          const float pr = pw[wave][br][g][jj];
#pragma unroll
          for (int cc = 0; cc < NC; ++cc) acc[br][g][cc] = fmaf(pr, vv[cc], acc[br][g][cc]);
        }
      }
    }
    __builtin_amdgcn_wave_barrier();
  }
  // merge the four waves' states, then write this chunk's partial
#pragma unroll
  for (int br = 0; br < 2; ++br)
#pragma unroll
    for (int g = 0; g < G; ++g) {
#pragma unroll
      for (int cc = 0; cc < NC; ++cc) red[wave][br][g][lane + 64 * cc] = acc[br][g][cc];
      if (lane == 0) {
        red[wave][br][g][D] = m[br][g];
        red[wave][br][g][D + 1] = l[br][g];
      }
    }
  __syncthreads();
  for (int e = tid; e < 2 * G * D; e += kDecWaves * 64) {
    const int br = e / (G * D), g = (e / D) % G, dd = e % D;
    float mx = kNeg;
    for (int w = 0; w < kDecWaves; ++w) mx = fmaxf(mx, red[w][br][g][D]);
    float a = 0.0f, ls = 0.0f;
    for (int w = 0; w < kDecWaves; ++w) {
      const float f = exp2f(red[w][br][g][D] - mx);
      a = fmaf(f, red[w][br][g][dd], a);
      ls = fmaf(f, red[w][br][g][D + 1], ls);
    }
    float* out = p.part + ((((long long)b * p.Hq + hk * G + g) * p.nchunk + c) * 2 + br) * (D + 2);
    out[dd] = a;
    if (dd == 0) {
      out[D] = mx;
      out[D + 1] = ls;
    }
  }
}

struct RedParams {
  const float* part;
  const int32_t* lens;
  const uint8_t* selected;
  const float* gate;
  void* o;             // [B][Hq][D]
  int B, Hq, cap, W, nchunk;
};

// One wave per (b, query head): merge the chunk partials of each branch in
// chunk order (deterministic) and combine.
template <int D, bool BF16>
__global__ __launch_bounds__(256) void decode_reduce_kernel(RedParams p) {
  constexpr int NC = D / 64;
  const long long w = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (w >= (long long)p.B * p.Hq) return;
  const int b = (int)(w / p.Hq);
  const int i = clamp_len(p.lens[b], p.cap) - 1;
  const int lo = max(0, i - p.W + 1);
  const bool sel = p.selected[b] != 0;
  float out[NC];
#pragma unroll
  for (int cc = 0; cc < NC; ++cc) out[cc] = 0.0f;
  for (int br = 0; br < 2; ++br) {
    if (br == 1 && !sel) break;
    const int cfirst = br == 0 ? lo / kChunk : 0;
    const int clast = i / kChunk;
    float mx = kNeg;
    for (int c = cfirst; c <= clast; ++c)
      mx = fmaxf(mx, p.part[((w * p.nchunk + c) * 2 + br) * (D + 2) + D]);
    float a[NC], ls = 0.0f;
#pragma unroll
    for (int cc = 0; cc < NC; ++cc) a[cc] = 0.0f;
    for (int c = cfirst; c <= clast; ++c) {
      const float* pt = p.part + ((w * p.nchunk + c) * 2 + br) * (D + 2);
      const float f = exp2f(pt[D] - mx);
      ls = fmaf(f, pt[D + 1], ls);
#pragma unroll
      for (int cc = 0; cc < NC; ++cc) a[cc] = fmaf(f, pt[lane + 64 * cc], a[cc]);
    }
    const float wgt = br == 0 ? 1.0f : 1.0f / (1.0f + expf(-p.gate[b]));
#pragma unroll
    for (int cc = 0; cc < NC; ++cc) out[cc] = fmaf(wgt, a[cc] / ls, out[cc]);
  }
#pragma unroll
  for (int cc = 0; cc < NC; ++cc) {
    const long long e = w * D + lane + 64 * cc;
    if (BF16) static_cast<uint16_t*>(p.o)[e] = (uint16_t)(pack_bf16x2(out[cc], 0.0f) & 0xffffu);
    else static_cast<float*>(p.o)[e] = out[cc];
  }
}

// tau_b = the largest logit with mask == 0 (NaN excluded), -inf if none.
__global__ __launch_bounds__(1024) void calibrate_kernel(const float* gate, const uint8_t* mask,
                                                         float* tau, int n) {
  __shared__ float wm[16];
  const int b = blockIdx.x;
  float mx = -INFINITY;
  for (int i = threadIdx.x; i < n; i += 1024) {
    const float g = gate[(size_t)b * n + i];
    if (mask[(size_t)b * n + i] == 0 && !isnan(g)) mx = fmaxf(mx, g);
  }
  mx = wmax(mx);
  if ((threadIdx.x & 63) == 0) wm[threadIdx.x >> 6] = mx;
  __syncthreads();
  if (threadIdx.x == 0) {
    float r = -INFINITY;
    for (int t = 0; t < 16; ++t) r = fmaxf(r, wm[t]);
    tau[b] = r;
  }
}

// mask = gate > tau_b; idx = selected positions ascending, -1 after count.
// One 1024-thread workgroup per sequence: thread t owns a contiguous slice.
__global__ __launch_bounds__(1024) void select_threshold_kernel(const float* gate,
                                                                const float* tau, uint8_t* mask,
                                                                int32_t* idx, int32_t* count,
                                                                int n) {
  __shared__ int sums[1024];
  const int b = blockIdx.x, t = threadIdx.x;
  const float th = tau[b];
  const int per = (n + 1023) / 1024;
  const int i0 = min(n, t * per), i1 = min(n, i0 + per);
  int c = 0;
  for (int i = i0; i < i1; ++i) c += gate[(size_t)b * n + i] > th ? 1 : 0;
  sums[t] = c;
  __syncthreads();
  // inclusive scan (Hillis-Steele) over 1024 slice counts
  for (int off = 1; off < 1024; off <<= 1) {
    const int x = t >= off ? sums[t - off] : 0;
    __syncthreads();
    sums[t] += x;
    __syncthreads();
  }
  int pos = sums[t] - c;
  const int total = sums[1023];
  for (int i = i0; i < i1; ++i) {
    const bool s = gate[(size_t)b * n + i] > th;
    mask[(size_t)b * n + i] = s ? 1 : 0;
    if (s) idx[(size_t)b * n + pos++] = i;
  }
  for (int r = total + t; r < n; r += 1024) idx[(size_t)b * n + r] = -1;
  if (t == 0) count[b] = total;
}

template <int D, int G, bool BF16>
hipError_t decode_t(const DecodeDims& d, const DecodeArgs& a, hipStream_t s) {
  DecParams p;
  p.q = a.q;
  p.kc = a.k_cache;
  p.vc = a.v_cache;
  p.lens = a.lens;
  p.selected = a.selected;
  p.part = a.part;
  p.B = d.B;
  p.Hq = d.Hq;
  p.Hkv = d.Hkv;
  p.cap = d.cap;
  p.W = d.window;
  p.nchunk = (d.cap + kChunk - 1) / kChunk;
  p.scale_log2 = d.scale * kLog2e;
  hipLaunchKernelGGL((decode_partial_kernel<D, G, BF16>),
                     dim3((unsigned)((long long)d.B * d.Hkv * p.nchunk)), dim3(kDecWaves * 64), 0,
                     s, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  RedParams r;
  r.part = a.part;
  r.lens = a.lens;
  r.selected = a.selected;
  r.gate = a.gate;
  r.o = a.o;
  r.B = d.B;
  r.Hq = d.Hq;
  r.cap = d.cap;
  r.W = d.window;
  r.nchunk = p.nchunk;
  hipLaunchKernelGGL((decode_reduce_kernel<D, BF16>),
                     dim3((unsigned)(((long long)d.B * d.Hq + 3) / 4)), dim3(256), 0, s, r);
  return hipGetLastError();
}

template <int D, bool BF16>
hipError_t decode_g(const DecodeDims& d, const DecodeArgs& a, hipStream_t s) {
  switch (d.Hq / d.Hkv) {
    case 1: return decode_t<D, 1, BF16>(d, a, s);
    case 2: return decode_t<D, 2, BF16>(d, a, s);
    case 4: return decode_t<D, 4, BF16>(d, a, s);
    case 7: return decode_t<D, 7, BF16>(d, a, s);
    case 8: return decode_t<D, 8, BF16>(d, a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

bool decode_group_supported(int G) { return G == 1 || G == 2 || G == 4 || G == 7 || G == 8; }

size_t decode_partial_bytes(const DecodeDims& d) {
  const size_t nchunk = (d.cap + kChunk - 1) / kChunk;
  return ((size_t)d.B * d.Hq * nchunk * 2 * (d.d + 2) * sizeof(float) + 255) / 256 * 256;
}

hipError_t launch_decode_ctrl(const DecodeDims& d, const float* gate, float* tau,
                              uint8_t* selected, hipStream_t s) {
  hipLaunchKernelGGL(decode_ctrl_kernel, dim3((d.B + 255) / 256), dim3(256), 0, s, gate, tau,
                     selected, d.B, (float)d.rho, d.eta);
  return hipGetLastError();
}

hipError_t launch_decode(const DecodeDims& d, const DecodeArgs& a, hipStream_t s) {
  const bool bf = d.dtype == 1;
  if (d.d == 64) return bf ? decode_g<64, true>(d, a, s) : decode_g<64, false>(d, a, s);
  if (d.d == 128) return bf ? decode_g<128, true>(d, a, s) : decode_g<128, false>(d, a, s);
  return hipErrorInvalidValue;
}

hipError_t launch_calibrate(const Dims& d, const float* gate, const uint8_t* mask, float* tau,
                            hipStream_t s) {
  if (d.B == 0 || d.n == 0) return hipSuccess;
  hipLaunchKernelGGL(calibrate_kernel, dim3(d.B), dim3(1024), 0, s, gate, mask, tau, d.n);
  return hipGetLastError();
}

hipError_t launch_select_threshold(const Dims& d, const float* gate, const float* tau,
                                   uint8_t* mask, int32_t* idx, int32_t* count, hipStream_t s) {
  if (d.B == 0 || d.n == 0) return hipSuccess;
  hipLaunchKernelGGL(select_threshold_kernel, dim3(d.B), dim3(1024), 0, s, gate, tau, mask, idx,
                     count, d.n);
  return hipGetLastError();
}

}  // namespace logo
