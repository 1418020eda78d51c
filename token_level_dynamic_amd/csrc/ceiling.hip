// Throughput ceilings of one gfx950 compute unit, measured by small
// kernels: the bf16 matrix-core rate, the LDS read rate of the two read
// forms the attention kernels use (16-byte rows and the transposing 8-byte
// read) alone and in those kernels' tile patterns, the exp2 rate,
// matrix-core work with LDS reads beside it, and the HBM streaming read rate. Built into its own
// library (libceiling.so), used only by the benchmark's ceiling mode; the
// attention library does not contain or call it.
//
// Every kernel records, per workgroup, the shader clock (s_memtime) and the
// constant 100 MHz clock (s_memrealtime) at its start and end, so the host
// can turn work per workgroup into work per clock cycle and read the clock
// frequency under load. All LDS addresses are masked into the kernel's own
// array; besides the streaming read of a caller's buffer, nothing is read
// from or written to global memory except one sink value per thread and the
// clock records.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16* lds_v4i16_ptr;

constexpr int kThreads = 256;
constexpr int kLdsChunks = 4096;  // 16-byte chunks: 64 KiB

__device__ __forceinline__ void record(long long* clk, long long t0, long long r0) {
  const long long t1 = __builtin_amdgcn_s_memtime();
  const long long r1 = __builtin_amdgcn_s_memrealtime();
  if (threadIdx.x == 0) {
    long long* c = clk + 4 * blockIdx.x;
    c[0] = t0;
    c[1] = t1;
    c[2] = r0;
    c[3] = r1;
  }
}

// bf16 value with a small magnitude from an integer (finite, nonzero mostly)
__device__ __forceinline__ uint32_t bf16_pair(uint32_t x) {
  const uint32_t a = 0x3c00u + (x % 509u);          // ~[2^-7, 2^-6)
  const uint32_t b = 0xbc00u + ((x * 7u) % 509u);   // negative, same range
  return a | (b << 16);
}

// 4 independent accumulator chains of v_mfma_f32_32x32x16_bf16
__global__ __launch_bounds__(kThreads) void mfma_kernel(float* sink, long long* clk, int iters) {
  const uint32_t t = threadIdx.x + blockIdx.x * kThreads;
  const bf16x8 a = __builtin_bit_cast(
      bf16x8, make_uint4(bf16_pair(t), bf16_pair(t + 1), bf16_pair(t + 2), bf16_pair(t + 3)));
  const bf16x8 b = __builtin_bit_cast(
      bf16x8, make_uint4(bf16_pair(t + 5), bf16_pair(t + 9), bf16_pair(t + 11), bf16_pair(t + 13)));
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  const long long t0 = __builtin_amdgcn_s_memtime();
  const long long r0 = __builtin_amdgcn_s_memrealtime();
#pragma unroll 1
  for (int i = 0; i < iters; ++i) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, a, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, a, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, b, c3, 0, 0, 0);
  }
  record(clk, t0, r0);
  float s = 0.0f;
#pragma unroll
  for (int e = 0; e < 16; ++e) s += c0[e] + c1[e] + c2[e] + c3[e];
  sink[t] = s;
}

// ds_read_b128, consecutive lanes on consecutive 16-byte chunks
__global__ __launch_bounds__(kThreads) void lds_b128_kernel(float* sink, long long* clk,
                                                            int iters) {
  __shared__ uint4 buf[kLdsChunks];
  for (int i = threadIdx.x; i < kLdsChunks; i += kThreads)
    buf[i] = make_uint4(i, 3 * i, 5 * i, 7 * i);
  __syncthreads();
  uint32_t x0 = 0, x1 = 0, x2 = 0, x3 = 0;
  const int base = threadIdx.x;
  const long long t0 = __builtin_amdgcn_s_memtime();
  const long long r0 = __builtin_amdgcn_s_memrealtime();
#pragma unroll 1
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const uint4 v = buf[(base + (i * 8 + u) * kThreads) & (kLdsChunks - 1)];
      x0 ^= v.x;
      x1 ^= v.y;
      x2 ^= v.z;
      x3 ^= v.w;
    }
  }
  record(clk, t0, r0);
  sink[threadIdx.x + blockIdx.x * kThreads] = (float)(x0 ^ x1 ^ x2 ^ x3);
}

// ds_read_b64_tr_b16 in the attention kernels' pattern: within each group of
// 16 lanes, 4 rows of a padded row-major tile (row stride 144 bf16) and 4
// column offsets
__global__ __launch_bounds__(kThreads) void lds_tr_kernel(float* sink, long long* clk, int iters) {
  __shared__ __attribute__((aligned(16))) uint16_t buf[kLdsChunks * 8];
  for (int i = threadIdx.x; i < kLdsChunks * 8; i += kThreads) buf[i] = (uint16_t)(i * 13);
  __syncthreads();
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int row = (lane & 15) >> 2;
  const int col = ((lane >> 4) & 1) * 16 + (lane & 3) * 4 + (lane >> 5) * 32;
  constexpr int kStride = 144;  // bf16 per row: 128 + 16 pad
  constexpr int kRowsMax = (kLdsChunks * 8) / kStride;  // 227 rows fit
  uint32_t x0 = 0, x1 = 0;
  const long long t0 = __builtin_amdgcn_s_memtime();
  const long long r0 = __builtin_amdgcn_s_memrealtime();
#pragma unroll 1
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      // rows (4 u + row + 16 wave) mod 192: below kRowsMax, columns below 128
      const int r = (4 * ((i * 8 + u) & 31) + row + 16 * wave) % 192;
      const v4i16 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_ptr)(buf + r * kStride + col));
      const uint2 w = __builtin_bit_cast(uint2, v);
      x0 ^= w.x;
      x1 ^= w.y;
    }
  }
  static_assert(192 <= kRowsMax, "rows in range");
  record(clk, t0, r0);
  sink[threadIdx.x + blockIdx.x * kThreads] = (float)(x0 ^ x1);
}

// v_exp_f32: 8 independent chains of exp2(fma(x, c, y))
__global__ __launch_bounds__(kThreads) void exp_kernel(float* sink, long long* clk, int iters) {
  float a[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) a[j] = -0.001f * (threadIdx.x + j);
  const long long t0 = __builtin_amdgcn_s_memtime();
  const long long r0 = __builtin_amdgcn_s_memrealtime();
#pragma unroll 1
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int j = 0; j < 8; ++j) a[j] = __builtin_amdgcn_exp2f(fmaf(a[j], -0.5f, -0.25f));
  }
  record(clk, t0, r0);
  float s = 0.0f;
#pragma unroll
  for (int j = 0; j < 8; ++j) s += a[j];
  sink[threadIdx.x + blockIdx.x * kThreads] = s;
}

// Matrix-core products with LDS reads beside them: per 4 products, NR
// ds_read_b128 of 1 KiB per wave (NR = 4 is the attention kernels' ratio of
// LDS bytes to products at 32 query rows per wave, NR = 2 that of 64 rows).
// Four accumulator chains; the reads of one iteration are folded into the
// A operands of the next iteration's products.
template <int NR>
__global__ __launch_bounds__(kThreads) void mfma_lds_kernel(float* sink, long long* clk,
                                                            int iters) {
  __shared__ uint4 buf[kLdsChunks];
  for (int i = threadIdx.x; i < kLdsChunks; i += kThreads)
    buf[i] = make_uint4(bf16_pair(i), bf16_pair(i + 1), bf16_pair(i + 2), bf16_pair(i + 3));
  __syncthreads();
  const uint32_t t = threadIdx.x + blockIdx.x * kThreads;
  const bf16x8 b = __builtin_bit_cast(
      bf16x8, make_uint4(bf16_pair(t + 5), bf16_pair(t + 9), bf16_pair(t + 11), bf16_pair(t + 13)));
  bf16x8 a[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) a[j] = b;
  f32x16 c[4] = {};
  const int base = threadIdx.x;
  const long long t0 = __builtin_amdgcn_s_memtime();
  const long long r0 = __builtin_amdgcn_s_memrealtime();
#pragma unroll 1
  for (int i = 0; i < iters; ++i) {
    uint4 na[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) na[j] = make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      const uint4 v = buf[(base + (i * NR + r) * kThreads) & (kLdsChunks - 1)];
      na[r & 3].x ^= v.x;
      na[r & 3].y ^= v.y;
      na[r & 3].z ^= v.z;
      na[r & 3].w ^= v.w;
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) c[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[j], b, c[j], 0, 0, 0);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (j < NR) a[j] = __builtin_bit_cast(bf16x8, na[j]);
  }
  record(clk, t0, r0);
  float s = 0.0f;
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int e = 0; e < 16; ++e) s += c[j][e];
  sink[t] = s;
}

// The attention kernel's own LDS read patterns over one 64-key tile at
// d = 128, repeated: its V^T fragments (32 ds_read_b64_tr_b16 per wave and
// tile: two 32-key blocks x two 16-key halves x four 32-wide d blocks x two
// 4-key row groups) or its K fragments (16 ds_read_b128: two 32-key blocks x
// eight 16-wide d steps). Layouts: row stride STRIDE bf16 (padded rows), or
// STRIDE = 128 with 16-byte chunk c of row r stored at chunk c ^ swz(r).
template <int STRIDE, int SWZ>
__device__ __forceinline__ int tile_off(int r, int c /* bf16 column */) {
  if (SWZ == 0) return r * STRIDE + c;
  const int ch = c >> 3, f = SWZ == 1 ? 4 * (r & 3) : (r & 15);
  return r * STRIDE + ((ch ^ f) << 3) + (c & 7);
}

template <int STRIDE, int SWZ>
__global__ __launch_bounds__(kThreads) void tile_v_kernel(float* sink, long long* clk, int iters) {
  constexpr int kTile = 64 * STRIDE;
  __shared__ __attribute__((aligned(16))) uint16_t buf[2 * kTile];
  for (int i = threadIdx.x; i < 2 * kTile; i += kThreads) buf[i] = (uint16_t)(i * 13);
  __syncthreads();
  const int lane = threadIdx.x & 63;
  const int half = lane >> 5;
  const int tr_row = (lane & 15) >> 2;
  const int tr_col = ((lane >> 4) & 1) * 16 + (lane & 3) * 4;
  uint32_t x0 = 0, x1 = 0;
  const long long t0 = __builtin_amdgcn_s_memtime();
  const long long r0 = __builtin_amdgcn_s_memrealtime();
#pragma unroll 1
  for (int i = 0; i < iters; ++i) {
    asm volatile("" ::: "memory");
    const uint16_t* tb = buf + (i & 1) * kTile;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
          for (int g = 0; g < 2; ++g) {
            const int r = kb * 32 + hh * 16 + half * 4 + tr_row + 8 * g;  // < 64
            const int c = db * 32 + tr_col;                                // < 128
            const v4i16 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (lds_v4i16_ptr)(tb + tile_off<STRIDE, SWZ>(r, c)));
            const uint2 w = __builtin_bit_cast(uint2, v);
            x0 ^= w.x;
            x1 ^= w.y;
          }
  }
  record(clk, t0, r0);
  sink[threadIdx.x + blockIdx.x * kThreads] = (float)(x0 ^ x1);
}

template <int STRIDE, int SWZ>
__global__ __launch_bounds__(kThreads) void tile_k_kernel(float* sink, long long* clk, int iters) {
  constexpr int kTile = 64 * STRIDE;
  __shared__ __attribute__((aligned(16))) uint16_t buf[2 * kTile];
  for (int i = threadIdx.x; i < 2 * kTile; i += kThreads) buf[i] = (uint16_t)(i * 13);
  __syncthreads();
  const int lane = threadIdx.x & 63;
  const int col = lane & 31, half = lane >> 5;
  uint32_t x0 = 0, x1 = 0, x2 = 0, x3 = 0;
  const long long t0 = __builtin_amdgcn_s_memtime();
  const long long r0 = __builtin_amdgcn_s_memrealtime();
#pragma unroll 1
  for (int i = 0; i < iters; ++i) {
    asm volatile("" ::: "memory");
    const uint16_t* tb = buf + (i & 1) * kTile;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const int r = kb * 32 + col;        // < 64
        const int c = s * 16 + half * 8;    // < 128
        const uint4 v = *reinterpret_cast<const uint4*>(tb + tile_off<STRIDE, SWZ>(r, c));
        x0 ^= v.x;
        x1 ^= v.y;
        x2 ^= v.z;
        x3 ^= v.w;
      }
  }
  record(clk, t0, r0);
  sink[threadIdx.x + blockIdx.x * kThreads] = (float)(x0 ^ x1 ^ x2 ^ x3);
}

// Dependent matrix-core products: NC accumulator chains, each product
// accumulating into the previous one's result (4 products per iteration).
template <int NC>
__global__ __launch_bounds__(kThreads) void mfma_chain_kernel(float* sink, long long* clk,
                                                              int iters) {
  const uint32_t t = threadIdx.x + blockIdx.x * kThreads;
  const bf16x8 a = __builtin_bit_cast(
      bf16x8, make_uint4(bf16_pair(t), bf16_pair(t + 1), bf16_pair(t + 2), bf16_pair(t + 3)));
  const bf16x8 b = __builtin_bit_cast(
      bf16x8, make_uint4(bf16_pair(t + 5), bf16_pair(t + 9), bf16_pair(t + 11), bf16_pair(t + 13)));
  f32x16 c[NC] = {};
  const long long t0 = __builtin_amdgcn_s_memtime();
  const long long r0 = __builtin_amdgcn_s_memrealtime();
#pragma unroll 1
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
      c[j % NC] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(j & 1 ? a : b, j & 2 ? b : a, c[j % NC],
                                                         0, 0, 0);
  }
  record(clk, t0, r0);
  float s = 0.0f;
#pragma unroll
  for (int j = 0; j < NC; ++j)
#pragma unroll
    for (int e = 0; e < 16; ++e) s += c[j][e];
  sink[t] = s;
}

// Matrix-core products with independent vector work beside them in the
// same wave: per 4 products (4 accumulator chains), NV rounds of an FMA and
// an exp2 on each of 4 independent float chains (8 NV VALU instructions, 4 NV
// of them transcendental). MODE 1 / 2 keep only the products / only the
// vector work; MODE 3 runs the products in even waves and the vector work in
// odd ones (two loops chosen once per wave), so the two kinds come from
// different waves (of one SIMD when two workgroups share a CU).
template <int NV, int MODE, bool VACC = false>
__global__ __launch_bounds__(kThreads) void mfma_valu_kernel(float* sink, long long* clk,
                                                             int iters) {
  const uint32_t t = threadIdx.x + blockIdx.x * kThreads;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const bf16x8 a = __builtin_bit_cast(
      bf16x8, make_uint4(bf16_pair(t), bf16_pair(t + 1), bf16_pair(t + 2), bf16_pair(t + 3)));
  const bf16x8 b = __builtin_bit_cast(
      bf16x8, make_uint4(bf16_pair(t + 5), bf16_pair(t + 9), bf16_pair(t + 11), bf16_pair(t + 13)));
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  float x0 = -0.001f * threadIdx.x, x1 = x0 - 0.1f, x2 = x0 - 0.2f, x3 = x0 - 0.3f;
  auto valu_round = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      x0 = __builtin_amdgcn_exp2f(fmaf(x0, -0.5f, -0.25f));
      x1 = __builtin_amdgcn_exp2f(fmaf(x1, -0.5f, -0.25f));
      x2 = __builtin_amdgcn_exp2f(fmaf(x2, -0.5f, -0.25f));
      x3 = __builtin_amdgcn_exp2f(fmaf(x3, -0.5f, -0.25f));
    }
  };
  auto mfma_round = [&]() __attribute__((always_inline)) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, a, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, a, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, b, c3, 0, 0, 0);
    // VACC: keep the accumulators in architectural VGPRs (as in kernels whose
    // vector code reads them) rather than accumulation registers
    if (VACC) asm volatile("" : "+v"(c0), "+v"(c1), "+v"(c2), "+v"(c3));
  };
  const long long t0 = __builtin_amdgcn_s_memtime();
  const long long r0 = __builtin_amdgcn_s_memrealtime();
  if (MODE == 0) {
#pragma unroll 1
    for (int i = 0; i < iters; ++i) {
      mfma_round();
      valu_round();
    }
  } else if (MODE == 1 || (MODE == 3 && (wave & 1) == 0)) {
#pragma unroll 1
    for (int i = 0; i < iters; ++i) mfma_round();
  } else {
#pragma unroll 1
    for (int i = 0; i < iters; ++i) valu_round();
  }
  record(clk, t0, r0);
  float s = x0 + x1 + x2 + x3;
#pragma unroll
  for (int e = 0; e < 16; ++e) s += c0[e] + c1[e] + c2[e] + c3[e];
  sink[t] = s;
}

// Matrix-core products on operands read from LDS that hold pseudo-random
// bf16 values with every mantissa bit in play (magnitudes 2^-4 .. 2^3,
// random signs), 0.5 KiB per product as in the 0.5 KiB case above: the
// power, hence the clock, of products on data like the attention inputs.
__device__ __forceinline__ uint32_t hash32(uint32_t x) {
  x ^= x >> 16; x *= 0x7feb352du; x ^= x >> 15; x *= 0x846ca68bu; x ^= x >> 16;
  return x;
}
__device__ __forceinline__ uint32_t rand_bf16_pair(uint32_t x) {
  const uint32_t h = hash32(x), g = hash32(x ^ 0x9e3779b9u);
  // exponent 123..130 (2^-4 .. 2^3), random sign and 7 mantissa bits
  const uint32_t a = ((h & 1u) << 15) | ((123u + ((h >> 1) & 7u)) << 7) | ((h >> 4) & 0x7fu);
  const uint32_t b = ((g & 1u) << 15) | ((123u + ((g >> 1) & 7u)) << 7) | ((g >> 4) & 0x7fu);
  return a | (b << 16);
}
__global__ __launch_bounds__(kThreads) void mfma_lds_random_kernel(float* sink, long long* clk,
                                                                   int iters) {
  __shared__ uint4 buf[kLdsChunks];
  for (int i = threadIdx.x; i < kLdsChunks; i += kThreads)
    buf[i] = make_uint4(rand_bf16_pair(4 * i), rand_bf16_pair(4 * i + 1),
                        rand_bf16_pair(4 * i + 2), rand_bf16_pair(4 * i + 3));
  __syncthreads();
  const uint32_t t = threadIdx.x + blockIdx.x * kThreads;
  const bf16x8 b = __builtin_bit_cast(
      bf16x8, make_uint4(rand_bf16_pair(7 * t), rand_bf16_pair(7 * t + 1),
                         rand_bf16_pair(7 * t + 2), rand_bf16_pair(7 * t + 3)));
  bf16x8 a[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) a[j] = b;
  f32x16 c[4] = {};
  const int base = threadIdx.x;
  const long long t0 = __builtin_amdgcn_s_memtime();
  const long long r0 = __builtin_amdgcn_s_memrealtime();
#pragma unroll 1
  for (int i = 0; i < iters; i += 4) {
    // fresh operands for two chains per product round, read two rounds ahead
    // (register indices fixed at compile time)
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const uint4 n0 = buf[(base + ((i + u) * 2) * kThreads) & (kLdsChunks - 1)];
      const uint4 n1 = buf[(base + ((i + u) * 2 + 1) * kThreads) & (kLdsChunks - 1)];
#pragma unroll
      for (int j = 0; j < 4; ++j)
        c[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[j], b, c[j], 0, 0, 0);
      a[u] = __builtin_bit_cast(bf16x8, n0);
      a[(u + 2) & 3] = __builtin_bit_cast(bf16x8, n1);
    }
  }
  record(clk, t0, r0);
  float s = 0.0f;
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int e = 0; e < 16; ++e) s += c[j][e];
  sink[t] = s;
}

// HBM read rate: every thread streams 16-byte loads over the buffer in a
// grid-stride loop (indices below n16 only) and folds them into one value.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
__global__ __launch_bounds__(kThreads) void stream_read_kernel(const u32x4* __restrict__ src,
                                                               long long n16, float* sink) {
  uint32_t x = 0;
  const long long stride = (long long)gridDim.x * kThreads;
  for (long long i = blockIdx.x * (long long)kThreads + threadIdx.x; i < n16; i += stride) {
    const u32x4 v = __builtin_nontemporal_load(src + i);
    x ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  sink[threadIdx.x + blockIdx.x * kThreads] = (float)x;
}

// The same stream through the LDS DMA the attention kernels use: each wave
// moves 1 KiB chunks (16 bytes a lane, buffer_load_dwordx4 ... lds) into an
// 8-slot ring of its own, at most 6 in flight, chunks grid-strided over the
// buffer (at most 1 GiB: 32-bit buffer sizes). One value per lane is read
// back at the end so the stores are live.
__global__ __launch_bounds__(kThreads) void stream_lds_kernel(const u32x4* __restrict__ src,
                                                              long long n16, float* sink) {
  __shared__ uint4 ring[kThreads / 64][8][64];
  typedef __attribute__((address_space(3))) void* lds_ptr;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const long long nchunk = n16 / 64;
  const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<u32x4*>(src), (short)0, (int)(nchunk * 1024), 0x00020000);
  const long long stride = (long long)gridDim.x * (kThreads / 64);
  int slot = 0;
  for (long long c = blockIdx.x * (long long)(kThreads / 64) + wave; c < nchunk; c += stride) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_ptr)&ring[wave][slot][0], 16,
                                             (uint32_t)(c * 1024 + lane * 16), 0, 0, 0);
    slot = (slot + 1) & 7;
    __builtin_amdgcn_s_waitcnt(0x0F76);   // vmcnt(6)
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);     // vmcnt(0)
  __syncthreads();
  const uint4 v = ring[wave][0][lane];
  sink[threadIdx.x + blockIdx.x * kThreads] = (float)(v.x ^ v.w);
}

}  // namespace

// Models of a tile loop (512-thread workgroups, one per CU for the LDS it
// takes): the product waves issue, per iteration, NR ds_read_b128 (1 KiB
// each per wave, landing in the A operands of the next iteration's
// products), 4 v_mfma_f32_32x32x16_bf16 and NF FMAs in 4 chains. BOTH:
// all eight waves (two per SIMD) issue, else waves 0-3 only (one per SIMD).
template <int NR, int NF, bool BOTH>
__global__ __launch_bounds__(512) void tile_model_kernel(float* sink, long long* clk, int iters) {
  __shared__ uint4 buf[2 * kLdsChunks];
  for (int i = threadIdx.x; i < 2 * kLdsChunks; i += 512)
    buf[i] = make_uint4(bf16_pair(i), bf16_pair(i + 1), bf16_pair(i + 2), bf16_pair(i + 3));
  __syncthreads();
  const uint32_t t = threadIdx.x + blockIdx.x * 512;
  const int team = __builtin_amdgcn_readfirstlane(threadIdx.x >> 8);
  const bf16x8 b = __builtin_bit_cast(
      bf16x8, make_uint4(bf16_pair(t + 5), bf16_pair(t + 9), bf16_pair(t + 11), bf16_pair(t + 13)));
  bf16x8 a[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) a[j] = b;
  f32x16 c[4] = {};
  float x0 = -0.001f * threadIdx.x, x1 = x0 - 0.1f, x2 = x0 - 0.2f, x3 = x0 - 0.3f;
  const int base = threadIdx.x;
  const long long t0 = __builtin_amdgcn_s_memtime();
  const long long r0 = __builtin_amdgcn_s_memrealtime();
  if (BOTH || team == 0) {
#pragma unroll 1
    for (int i = 0; i < iters; ++i) {
      bf16x8 na[4];
#pragma unroll
      for (int r = 0; r < NR; ++r)
        na[r & 3] = __builtin_bit_cast(bf16x8, buf[(base + (i * NR + r) * 512) & (2 * kLdsChunks - 1)]);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        c[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[j], b, c[j], 0, 0, 0);
#pragma unroll
      for (int f = 0; f < NF; f += 4) {
        x0 = fmaf(x0, 0.999f, 0.25f);
        if (f + 1 < NF) x1 = fmaf(x1, 0.999f, 0.25f);
        if (f + 2 < NF) x2 = fmaf(x2, 0.999f, 0.25f);
        if (f + 3 < NF) x3 = fmaf(x3, 0.999f, 0.25f);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (j < NR) a[j] = na[j];
    }
  }
  __syncthreads();
  record(clk, t0, r0);
  float s = x0 + x1 + x2 + x3;
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int e = 0; e < 16; ++e) s += c[j][e];
  if (s == 1.2345f) sink[t & 255] = s;
}

// Matrix-core and vector work on the two waves that share a SIMD (512-thread
// workgroups: waves w and w + 4 run on one SIMD). MODE 0: all eight waves
// issue products; 1: waves 0-3 issue products, 4-7 nothing; 2: waves 0-3
// products, 4-7 NV rounds of 4 independent FMA chains per iteration; 3: as 2
// with v_exp_f32 chains; 4: waves 0-3 products and the FMA rounds in the same
// wave, 4-7 nothing; 5: as 4 with v_exp_f32; 6: as 2 with v_dot2_f32_bf16
// chains. Per iteration a product wave
// issues 4 v_mfma_f32_32x32x16_bf16 (4 x 32 cycles of one SIMD's matrix core).
template <int MODE, int NV>
__global__ __launch_bounds__(512) void simd_pair_kernel(float* sink, long long* clk, int iters) {
  const uint32_t t = threadIdx.x + blockIdx.x * 512;
  const int team = __builtin_amdgcn_readfirstlane(threadIdx.x >> 8);
  const bf16x8 a = __builtin_bit_cast(
      bf16x8, make_uint4(bf16_pair(t), bf16_pair(t + 1), bf16_pair(t + 2), bf16_pair(t + 3)));
  const bf16x8 b = __builtin_bit_cast(
      bf16x8, make_uint4(bf16_pair(t + 5), bf16_pair(t + 9), bf16_pair(t + 11), bf16_pair(t + 13)));
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  float x0 = -0.001f * threadIdx.x, x1 = x0 - 0.1f, x2 = x0 - 0.2f, x3 = x0 - 0.3f;
  auto fma_round = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      x0 = fmaf(x0, 0.999f, 0.25f);
      x1 = fmaf(x1, 0.999f, 0.25f);
      x2 = fmaf(x2, 0.999f, 0.25f);
      x3 = fmaf(x3, 0.999f, 0.25f);
    }
  };
  auto exp_round = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      x0 = __builtin_amdgcn_exp2f(-x0);
      x1 = __builtin_amdgcn_exp2f(-x1);
      x2 = __builtin_amdgcn_exp2f(-x2);
      x3 = __builtin_amdgcn_exp2f(-x3);
    }
  };
  // v_dot2_f32_bf16 of a packed pair with (1, 1): the attention kernels' row sums
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
  const bf16x2 pr = __builtin_bit_cast(bf16x2, bf16_pair(t + 7));
  auto dot_round = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      x0 = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, x0, false);
      x1 = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, x1, false);
      x2 = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, x2, false);
      x3 = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, x3, false);
    }
  };
  auto mfma_round = [&]() __attribute__((always_inline)) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, a, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, a, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, b, c3, 0, 0, 0);
  };
  const long long t0 = __builtin_amdgcn_s_memtime();
  const long long r0 = __builtin_amdgcn_s_memrealtime();
  const bool products = MODE == 0 || team == 0;
  if (products) {
#pragma unroll 1
    for (int i = 0; i < iters; ++i) {
      mfma_round();
      if (MODE == 4) fma_round();
      if (MODE == 5) exp_round();
    }
  } else if (MODE == 2) {
#pragma unroll 1
    for (int i = 0; i < iters; ++i) fma_round();
  } else if (MODE == 3) {
#pragma unroll 1
    for (int i = 0; i < iters; ++i) exp_round();
  } else if (MODE == 6) {
#pragma unroll 1
    for (int i = 0; i < iters; ++i) dot_round();
  }
  __syncthreads();
  record(clk, t0, r0);
  float s = x0 + x1 + x2 + x3;
#pragma unroll
  for (int e = 0; e < 16; ++e) s += c0[e] + c1[e] + c2[e] + c3[e];
  if (s == 1.2345f) sink[t & 255] = s;
}

// Wave placement: every wave of a 512-thread workgroup writes the SIMD it
// runs on (bits 5:4 of its HW_ID register) to sink[8 * block + wave].
__global__ __launch_bounds__(512) void wave_simd_kernel(float* sink) {
  const int wave = threadIdx.x >> 6;
  const int simd = __builtin_amdgcn_s_getreg((1 << 11) | (4 << 6) | 4);   // hwreg(HW_ID, 4, 2)
  if ((threadIdx.x & 63) == 0) sink[blockIdx.x * 8 + wave] = (float)simd;
}

extern "C" {

// kind: 0 matrix-core products, 1 ds_read_b128, 2 ds_read_b64_tr_b16,
// 3 v_exp_f32, 4/5/6 products with 0.5 / 1 / 2 KiB of LDS reads per product,
// 7/8/9 the V^T read pattern of one tile (row stride 144, 160, or 128 with
// chunk swizzle 4 (r & 3)), 10/11 the K read pattern (stride 136, or 128 with
// chunk swizzle r & 15), 12 streaming reads of src (src_bytes, a multiple of
// 16; iters and clk unused), 13-18 products beside vector work (13: both in
// every wave, 2 FMA+exp2 rounds per product; 14 products only; 15 vector
// only; 16 products in even waves and vector work in odd ones; 17, 18: as
// 13, 16 with 4 rounds), 19 products on full-entropy random operands from
// LDS (0.5 KiB per product), 20/21 products in 1 / 2 dependent accumulator
// chains, 22/23 as 13/14 with the accumulators in architectural VGPRs, 24
// the SIMD of each wave of 512-thread workgroups (sink[8 * block + wave]),
// 25-30 matrix-core and vector work on the two waves that share a SIMD
// (simd_pair_kernel modes 0-5), 31-36 tile-loop models (tile_model_kernel:
// 31 one wave per SIMD, 0.5 KiB LDS + 3.5 FMA per product; 32 two waves per
// SIMD, 1 KiB + 3.5; 33 as 31 without FMAs; 34 as 31 without LDS; 35 as 32
// without FMAs; 36 as 32 without LDS), 37/38 products in waves 0-3 beside 4
// v_dot2_f32_bf16 / 4 FMA per product in waves 4-7 (simd_pair_kernel modes
// 6 and 2), 39 the streaming reads of 12 through the LDS DMA (src_bytes at
// most 1 GiB).
// sink: blocks * 256 floats; clk: blocks * 4
// int64. Returns a hipError_t.
int ceiling_launch(int kind, int blocks, int iters, float* sink, long long* clk,
                   const void* src, long long src_bytes, hipStream_t stream) {
  if (blocks <= 0 || !sink) return (int)hipErrorInvalidValue;
  if (kind == 12 || kind == 39) {
    if (!src || src_bytes <= 0 || src_bytes % 16) return (int)hipErrorInvalidValue;
    if (kind == 39 && src_bytes > (1LL << 30)) return (int)hipErrorInvalidValue;
    if (kind == 12)
      hipLaunchKernelGGL(stream_read_kernel, dim3(blocks), dim3(kThreads), 0, stream,
                         static_cast<const u32x4*>(src), src_bytes / 16, sink);
    else
      hipLaunchKernelGGL(stream_lds_kernel, dim3(blocks), dim3(kThreads), 0, stream,
                         static_cast<const u32x4*>(src), src_bytes / 16, sink);
    return (int)hipGetLastError();
  }
  if (iters <= 0 || !clk) return (int)hipErrorInvalidValue;
  const dim3 g(blocks), b(kThreads);
  switch (kind) {
    case 0: hipLaunchKernelGGL(mfma_kernel, g, b, 0, stream, sink, clk, iters); break;
    case 1: hipLaunchKernelGGL(lds_b128_kernel, g, b, 0, stream, sink, clk, iters); break;
    case 2: hipLaunchKernelGGL(lds_tr_kernel, g, b, 0, stream, sink, clk, iters); break;
    case 3: hipLaunchKernelGGL(exp_kernel, g, b, 0, stream, sink, clk, iters); break;
    case 4: hipLaunchKernelGGL(mfma_lds_kernel<2>, g, b, 0, stream, sink, clk, iters); break;
    case 5: hipLaunchKernelGGL(mfma_lds_kernel<4>, g, b, 0, stream, sink, clk, iters); break;
    case 6: hipLaunchKernelGGL(mfma_lds_kernel<8>, g, b, 0, stream, sink, clk, iters); break;
    case 7: hipLaunchKernelGGL((tile_v_kernel<144, 0>), g, b, 0, stream, sink, clk, iters); break;
    case 8: hipLaunchKernelGGL((tile_v_kernel<160, 0>), g, b, 0, stream, sink, clk, iters); break;
    case 9: hipLaunchKernelGGL((tile_v_kernel<128, 1>), g, b, 0, stream, sink, clk, iters); break;
    case 10: hipLaunchKernelGGL((tile_k_kernel<136, 0>), g, b, 0, stream, sink, clk, iters); break;
    case 11: hipLaunchKernelGGL((tile_k_kernel<128, 2>), g, b, 0, stream, sink, clk, iters); break;
    case 13: hipLaunchKernelGGL((mfma_valu_kernel<2, 0>), g, b, 0, stream, sink, clk, iters); break;
    case 14: hipLaunchKernelGGL((mfma_valu_kernel<2, 1>), g, b, 0, stream, sink, clk, iters); break;
    case 15: hipLaunchKernelGGL((mfma_valu_kernel<2, 2>), g, b, 0, stream, sink, clk, iters); break;
    case 16: hipLaunchKernelGGL((mfma_valu_kernel<2, 3>), g, b, 0, stream, sink, clk, iters); break;
    case 17: hipLaunchKernelGGL((mfma_valu_kernel<4, 0>), g, b, 0, stream, sink, clk, iters); break;
    case 18: hipLaunchKernelGGL((mfma_valu_kernel<4, 3>), g, b, 0, stream, sink, clk, iters); break;
    case 19: hipLaunchKernelGGL(mfma_lds_random_kernel, g, b, 0, stream, sink, clk, iters); break;
    case 20: hipLaunchKernelGGL(mfma_chain_kernel<1>, g, b, 0, stream, sink, clk, iters); break;
    case 22: hipLaunchKernelGGL((mfma_valu_kernel<2, 0, true>), g, b, 0, stream, sink, clk, iters); break;
    case 23: hipLaunchKernelGGL((mfma_valu_kernel<2, 1, true>), g, b, 0, stream, sink, clk, iters); break;
    case 21: hipLaunchKernelGGL(mfma_chain_kernel<2>, g, b, 0, stream, sink, clk, iters); break;
    case 24: hipLaunchKernelGGL(wave_simd_kernel, g, dim3(512), 0, stream, sink); break;
    case 25: hipLaunchKernelGGL((simd_pair_kernel<0, 8>), g, dim3(512), 0, stream, sink, clk, iters); break;
    case 26: hipLaunchKernelGGL((simd_pair_kernel<1, 8>), g, dim3(512), 0, stream, sink, clk, iters); break;
    case 27: hipLaunchKernelGGL((simd_pair_kernel<2, 8>), g, dim3(512), 0, stream, sink, clk, iters); break;
    case 28: hipLaunchKernelGGL((simd_pair_kernel<3, 2>), g, dim3(512), 0, stream, sink, clk, iters); break;
    case 29: hipLaunchKernelGGL((simd_pair_kernel<4, 8>), g, dim3(512), 0, stream, sink, clk, iters); break;
    case 30: hipLaunchKernelGGL((simd_pair_kernel<5, 2>), g, dim3(512), 0, stream, sink, clk, iters); break;
    case 31: hipLaunchKernelGGL((tile_model_kernel<2, 14, false>), g, dim3(512), 0, stream, sink, clk, iters); break;
    case 32: hipLaunchKernelGGL((tile_model_kernel<4, 14, true>), g, dim3(512), 0, stream, sink, clk, iters); break;
    case 33: hipLaunchKernelGGL((tile_model_kernel<2, 0, false>), g, dim3(512), 0, stream, sink, clk, iters); break;
    case 34: hipLaunchKernelGGL((tile_model_kernel<0, 14, false>), g, dim3(512), 0, stream, sink, clk, iters); break;
    case 35: hipLaunchKernelGGL((tile_model_kernel<4, 0, true>), g, dim3(512), 0, stream, sink, clk, iters); break;
    case 36: hipLaunchKernelGGL((tile_model_kernel<0, 14, true>), g, dim3(512), 0, stream, sink, clk, iters); break;
    case 37: hipLaunchKernelGGL((simd_pair_kernel<6, 4>), g, dim3(512), 0, stream, sink, clk, iters); break;
    case 38: hipLaunchKernelGGL((simd_pair_kernel<2, 4>), g, dim3(512), 0, stream, sink, clk, iters); break;
    default: return (int)hipErrorInvalidValue;
  }
  return (int)hipGetLastError();
}

}  // extern "C"
