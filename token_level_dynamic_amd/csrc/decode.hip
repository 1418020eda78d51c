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

// keys per chunk partial: a work item of the stream (and a workgroup of the
// chunked kernel). Larger chunks mean fewer partial stores between the tile
// loads (each delays the next wait) and fewer partials to merge, smaller
// ones a finer balance over the compute units; 1024 measured best.
constexpr int kChunk = 1024;
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

// Wave-wide max / sum without LDS permutes: rotations within each 16-lane
// DPP row, then the row pairs and the wave halves exchanged with
// v_permlane16_swap / v_permlane32_swap; every lane gets the result.
template <int N>  // rotate right by N lanes within each 16-lane row
__device__ __forceinline__ float dpp_ror(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x),
                                                               0x120 + N, 0xf, 0xf, false));
}
#define LOGO_DPP_ROR(x, n) dpp_ror<(n)>(x)
__device__ __forceinline__ float wmax(float x) {
  x = fmaxf(x, LOGO_DPP_ROR(x, 8));
  x = fmaxf(x, LOGO_DPP_ROR(x, 4));
  x = fmaxf(x, LOGO_DPP_ROR(x, 2));
  x = fmaxf(x, LOGO_DPP_ROR(x, 1));
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto c = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return fmaxf(__uint_as_float(c[0]), __uint_as_float(c[1]));
}
__device__ __forceinline__ float wsum(float x) {
  x += LOGO_DPP_ROR(x, 8);
  x += LOGO_DPP_ROR(x, 4);
  x += LOGO_DPP_ROR(x, 2);
  x += LOGO_DPP_ROR(x, 1);
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto c = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return __uint_as_float(c[0]) + __uint_as_float(c[1]);
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
  float* part;         // [B][Hkv][nchunk][2][G][D + 4]: acc[D], max (log2 units), sum, 2 pad
  int B, Hq, Hkv, cap, W, nchunk;
  float scale_log2;
};

// Sum over the 16 lanes of a DPP row (rotations by 8, 4, 2, 1 within the
// row): every lane of the row gets the row's total.
__device__ __forceinline__ float row16_sum(float x) {
  x += LOGO_DPP_ROR(x, 8);
  x += LOGO_DPP_ROR(x, 4);
  x += LOGO_DPP_ROR(x, 2);
  x += LOGO_DPP_ROR(x, 1);
  return x;
}

// EPL consecutive elements of an I/O-dtype row as float (16 B for bf16 x 8,
// 8 B for bf16 x 4, two or one float4 for float32).
template <int EPL, bool BF16>
__device__ __forceinline__ void load_seg(const void* base, long long off, float (&x)[EPL]) {
  if (EPL == 1) {
    x[0] = BF16 ? __uint_as_float((uint32_t)static_cast<const uint16_t*>(base)[off] << 16)
                : static_cast<const float*>(base)[off];
    return;
  }
  if (BF16) {
    const uint16_t* pp = static_cast<const uint16_t*>(base) + off;
    uint32_t w[EPL / 2 > 0 ? EPL / 2 : 1];
    if (EPL == 8) {
      const uint4 u = *reinterpret_cast<const uint4*>(pp);
      w[0] = u.x; w[1] = u.y; w[2 % (EPL / 2)] = u.z; w[3 % (EPL / 2)] = u.w;
    } else {
      const uint2 u = *reinterpret_cast<const uint2*>(pp);
      w[0] = u.x; w[1] = u.y;
    }
#pragma unroll
    for (int t = 0; t < EPL / 2; ++t) {
      x[(2 * t) % EPL] = __uint_as_float(w[t] << 16);
      x[(2 * t + 1) % EPL] = __uint_as_float(w[t] & 0xffff0000u);
    }
  } else {
    const float4* f = reinterpret_cast<const float4*>(static_cast<const float*>(base) + off);
#pragma unroll
    for (int t = 0; t < EPL / 4; ++t) {
      const float4 a = f[t];
      x[(4 * t) % EPL] = a.x;
      x[(4 * t + 1) % EPL] = a.y;
      x[(4 * t + 2) % EPL] = a.z;
      x[(4 * t + 3) % EPL] = a.w;
    }
  }
}

// One workgroup per (b, kv head, chunk); waves take 64-key steps of the chunk
// in turn. Within a step the 16 lanes of each DPP row share one key at a
// time (4 keys per wave instruction): lane (row r, position s) holds
// elements [s*EPL, s*EPL + EPL) of the G queries in registers, loads the same
// slice of the key row (coalesced 16-lane loads), and the row sums its
// partial dot products with DPP rotates. The values use the same key
// assignment, each lane accumulating its EPL output elements. Loads are
// issued kBatch iterations at a time, so each wave keeps kBatch rows of
// 16 lanes in flight.
//
// Each workgroup does one branch of one chunk: the first B*Hkv*nchunk
// workgroups the local branch (chunks that overlap the window), the rest the
// global branch (every chunk of a selected sequence), all in one launch and
// with one set of accumulators (the window's keys are read twice for a
// selected sequence: a few percent more bytes for twice the occupancy).
// Workgroups with nothing to do exit at once.
constexpr int kBatch = 4;

template <int D, int G, bool BF16>
__global__ __launch_bounds__(kDecWaves * 64) void decode_partial_kernel(DecParams p) {
  constexpr int EPL = D / 16;   // elements per lane
  constexpr int NB = 1;
  __shared__ __attribute__((aligned(16))) float qsh[G][D];  // the G queries
  __shared__ float sbuf[kDecWaves][G][kSub];       // scores of a wave step
  __shared__ float pw[kDecWaves][NB][G][kSub];     // probabilities of a wave step
  __shared__ float red[kDecWaves][NB][G][D + 2];
  const int per_kind = p.B * p.Hkv * p.nchunk;
  const bool loc = (int)blockIdx.x < per_kind;  // uniform: local or global branch
  const int wid = loc ? (int)blockIdx.x : (int)blockIdx.x - per_kind;
  const int c = wid % p.nchunk;
  const int bk = wid / p.nchunk;
  const int b = bk / p.Hkv, hk = bk % p.Hkv;
  const int i = clamp_len(p.lens[b], p.cap) - 1;
  const int lo = max(0, i - p.W + 1);
  const bool sel = p.selected[b] != 0;
  const int c0 = c * kChunk, c1 = min(c0 + kChunk, i + 1);  // keys [c0, c1)
  const bool in_win = c0 <= i && c1 > lo;
  // uniform over the workgroup: no barrier is skipped
  if (loc ? !in_win : (!sel || c0 > i)) return;
  const bool act[1] = {true};
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar registers
  const int grp = lane >> 4, seg = lane & 15;
  for (int e = tid; e < G * D; e += kDecWaves * 64) {
    float x[1];
    load_seg<1, BF16>(p.q, ((long long)b * p.Hq + hk * G) * D + e, x);
    qsh[e / D][e % D] = x[0];
  }
  __syncthreads();
  const long long kvb = ((long long)b * p.Hkv + hk) * p.cap;
  float m[NB][G], l[NB][G], acc[NB][G][EPL];
#pragma unroll
  for (int br = 0; br < NB; ++br)
#pragma unroll
    for (int g = 0; g < G; ++g) {
      m[br][g] = kNeg;
      l[br][g] = 0.0f;
#pragma unroll
      for (int t = 0; t < EPL; ++t) acc[br][g][t] = 0.0f;
    }
  for (int j0 = c0 + wave * kSub; j0 < c1; j0 += kDecWaves * kSub) {
    // scores: kSub/4 iterations of 4 keys, loads kBatch iterations ahead
#pragma unroll
    for (int i0 = 0; i0 < kSub / 4; i0 += kBatch) {
      float kv[kBatch][EPL];
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const int j = min(j0 + (i0 + u) * 4 + grp, c1 - 1);  // past the chunk: masked below
        load_seg<EPL, BF16>(p.kc, (kvb + j) * D + seg * EPL, kv[u]);
      }
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const int jl = (i0 + u) * 4 + grp;
#pragma unroll
        for (int g = 0; g < G; ++g) {
          float sg = 0.0f;
          const float* qg = &qsh[g][seg * EPL];
#pragma unroll
          for (int t = 0; t < EPL; ++t) sg = fmaf(qg[t], kv[u][t], sg);
          sg = row16_sum(sg);
          if (seg == 0) sbuf[wave][g][jl] = sg;
        }
      }
    }
    __builtin_amdgcn_wave_barrier();
    // online softmax, lane = key of the step
    const int j = j0 + lane;
    const bool valid = j < c1;
    const bool inwin = valid && j >= lo;
#pragma unroll
    for (int br = 0; br < NB; ++br) {
      if (!act[br]) continue;
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const bool in = loc ? inwin : valid;
        const float x = in ? sbuf[wave][g][lane] * p.scale_log2 : kNeg;
        const float mn = fmaxf(m[br][g], wmax(x));
        const float alpha = exp2f(m[br][g] - mn);
        const float pr = in ? exp2f(x - mn) : 0.0f;
        l[br][g] = l[br][g] * alpha + wsum(pr);
        m[br][g] = mn;
#pragma unroll
        for (int t = 0; t < EPL; ++t) acc[br][g][t] *= alpha;
        pw[wave][br][g][lane] = pr;
      }
    }
    __builtin_amdgcn_wave_barrier();
    // values: same 4-keys-per-instruction assignment
    const int cnt = min(kSub, c1 - j0);
#pragma unroll
    for (int i0 = 0; i0 < kSub / 4; i0 += kBatch) {
      if (i0 * 4 >= cnt) break;  // uniform
      float vv[kBatch][EPL];
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const int jj = min((i0 + u) * 4 + grp, cnt - 1);
        load_seg<EPL, BF16>(p.vc, (kvb + j0 + jj) * D + seg * EPL, vv[u]);
      }
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const int jl = (i0 + u) * 4 + grp;
        const bool live = jl < cnt;
#pragma unroll
        for (int br = 0; br < NB; ++br) {
          if (!act[br]) continue;
#pragma unroll
          for (int g = 0; g < G; ++g) {
            const float pr = live ? pw[wave][br][g][jl] : 0.0f;
#pragma unroll
            for (int t = 0; t < EPL; ++t) acc[br][g][t] = fmaf(pr, vv[u][t], acc[br][g][t]);
          }
        }
      }
    }
    __builtin_amdgcn_wave_barrier();
  }
  // add the four rows' partial sums (same elements, different keys), then
  // merge the four waves' states and write this chunk's partial
#pragma unroll
  for (int br = 0; br < NB; ++br)
#pragma unroll
    for (int g = 0; g < G; ++g) {
#pragma unroll
      for (int t = 0; t < EPL; ++t) {
        float x = acc[br][g][t];
        x += __shfl_xor(x, 16, 64);
        x += __shfl_xor(x, 32, 64);
        if (grp == 0) red[wave][br][g][seg * EPL + t] = x;
      }
      if (lane == 0) {
        red[wave][br][g][D] = m[br][g];
        red[wave][br][g][D + 1] = l[br][g];
      }
    }
  __syncthreads();
  for (int e = tid; e < NB * G * D; e += kDecWaves * 64) {
    const int br = e / (G * D), g = (e / D) % G, dd = e % D;
    if (!act[br]) continue;
    float mx = kNeg;
    for (int w = 0; w < kDecWaves; ++w) mx = fmaxf(mx, red[w][br][g][D]);
    float a = 0.0f, ls = 0.0f;
    for (int w = 0; w < kDecWaves; ++w) {
      const float f = exp2f(red[w][br][g][D] - mx);
      a = fmaf(f, red[w][br][g][dd], a);
      ls = fmaf(f, red[w][br][g][D + 1], ls);
    }
    const int slot = loc ? 0 : 1;  // partial slot: 0 local, 1 global
    float* out =
        p.part + ((((long long)b * p.Hkv + hk) * p.nchunk + c) * 2 + slot) * G * (D + 4) + g * (D + 4);
    out[dd] = a;
    if (dd == 0) {
      out[D] = mx;
      out[D + 1] = ls;
    }
  }
}

// ---- bf16 decode as a persistent stream ------------------------------------
//
// One workgroup per compute unit takes every nwg-th work item, an item
// being (b, branch, kv head, chunk of kChunk keys) with at least one key to
// read: local items cover the chunks that overlap the window, global items
// every chunk of a selected sequence. Items are numbered sequence-major,
// branch, kv head, chunk, so at any moment the workgroups read neighbouring
// chunks of the same caches (HBM serves such a sweep measurably faster than
// as many separate streams). The item numbering (a prefix sum over
// (b, branch) of kv heads x chunks) and each sequence's last position are
// built in LDS at the start, so looking up an item reads no global memory.
//
// K/V tiles of kStKeys keys, with the item's query rows, stream into LDS by
// bounds-checked buffer loads with kStStages buffers, across item
// boundaries: three tiles are always in flight while one is consumed (past
// the end of the range, loads of an empty range keep the count, so every
// wait is the same). Each tile is computed on
// the matrix cores with the kv head's G query heads as 16 columns (columns
// G..15 are zero): S^T = K Q^T (16x16x32 steps), online softmax per column,
// O^T += V^T P^T (16x16x16 steps, V^T from the transposing LDS read). Every
// wave computes the scores and the softmax; wave w accumulates only its
// share of the d blocks, so no cross-wave merge is needed and each wave
// writes its own slice of the item's partial (max, sum, weighted values)
// when the item ends.
constexpr int kStWaves = 4;
constexpr int kStStages = 4;
constexpr int kStKeys = 64;
constexpr int kStCols = 16;      // query heads per kv head the kernel takes
constexpr int kStPlan = 2048;    // plan entries in LDS: 2B + 1, so B <= 1023
constexpr int kStMaxB = (kStPlan - 1) / 2;
constexpr int kWaitLgkm0 = 0xC07F; // s_waitcnt lgkmcnt(0), vmcnt/expcnt untouched
// s_waitcnt immediate for vmcnt(N), expcnt and lgkmcnt untouched (gfx9
// encoding: vmcnt bits 3:0 at 3:0, bits 5:4 at 15:14)
template <int N>
constexpr int vm_wait() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  return 0x0F70 | (N & 15) | ((N >> 4) << 14);
}
constexpr float kLazy = 8.0f;      // log2 headroom before the running max moves

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Tiles are row-major without padding (a K tile then a V tile per stage);
// bank conflicts are avoided by storing 16-byte chunk c of row r at chunk
// c ^ f(r): for K reads (16 consecutive rows, one chunk) f spreads the rows
// over all banks; for the transposing V reads (8 rows, two adjacent chunks)
// f moves whole chunk pairs.
template <int D>
struct StTile {
  static constexpr int kCpr = D / 8;                  // 16-byte chunks per row
  static constexpr int kElems = kStKeys * D;          // one K or V tile
  // the item's query rows, padded to one load per wave (rows past G, and
  // the padding, read as zero)
  static constexpr int qElems = kStCols * D > 2048 ? kStCols * D : 2048;
  static constexpr int kStage = 2 * kElems + qElems;  // K tile, V tile, query rows
  static constexpr int kInstr = kCpr / kStWaves;      // buffer loads per wave per tile
  static constexpr int qInstr = qElems / 512 / kStWaves;  // ... and per query block
  __device__ static int fk(int r) { return D == 128 ? (r & 15) : ((r >> 1) & 7); }
  __device__ static int fv(int r) { return D == 128 ? 2 * (r & 7) : 2 * ((r >> 1) & 3); }
};

struct StParams {
  const uint16_t* q;   // [B][Hq][D] bf16
  const uint16_t* kc;  // [B][Hkv][cap][D]
  const uint16_t* vc;
  const int32_t* lens;
  const uint8_t* selected;
  float* part;         // as DecParams::part
  int B, Hq, Hkv, cap, W, nchunk, nwg;
  float scale_log2;
};

// Wave w issues instructions j = w, w+4, ... (NJ of them) that fill one
// tile: lane l of instruction j moves 16 bytes at byte offset voff[i] of the
// buffer [base, base + nbytes) to LDS byte 1024*j + 16*l of dst; offsets at
// or past nbytes read as zero (nbytes = 0: the whole tile). The resource
// type is device-only, so it is built here and not in the kernel's lambdas.
template <int NJ>
__device__ __forceinline__ void st_issue(const void* base, int nbytes, uint16_t* dst,
                                         const uint32_t* voff, int wave) {
  typedef __attribute__((address_space(3))) void* lds_ptr;
  const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<void*>(base), (short)0, nbytes, 0x00020000);
#pragma unroll
  for (int i = 0; i < NJ; ++i)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_ptr)(dst + (wave + kStWaves * i) * 512),
                                             16, voff[i], 0, 0, 0);
}

// Partial records of one item: the lane stores NB 16-byte blocks at byte
// offsets off[k] of the buffer [base, base + nbytes), then (max, sum, 0, 0)
// at off_ml; offsets at or past nbytes are dropped by the buffer range
// check (lanes with nothing to write).
template <int NB>
__device__ __forceinline__ void st_store(float* base, int nbytes, const f32x4 (&v)[NB],
                                         const int (&off)[NB], int off_ml, float m, float l) {
  typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
  const __amdgpu_buffer_rsrc_t rsrc =
      __builtin_amdgcn_make_buffer_rsrc(base, (short)0, nbytes, 0x00020000);
#pragma unroll
  for (int k = 0; k < NB; ++k)
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v[k]), rsrc, off[k], 0, 0);
  const u32x4 ml = {__float_as_uint(m), __float_as_uint(l), 0u, 0u};
  __builtin_amdgcn_raw_buffer_store_b128(ml, rsrc, off_ml, 0, 0);
}

template <int D>
__global__ __launch_bounds__(kStWaves * 64, 1) void decode_stream_kernel(StParams p) {
  using TL = StTile<D>;
  constexpr int QS = D / 32;            // 32-wide k steps of the scores
  constexpr int DBW = D / 16 / kStWaves;  // 16-wide d blocks per wave
  // one LDS object per stage (K tile, V tile, query rows): the compiler
  // tells the stage being read from the stages whose loads are in flight
  // only when they are distinct objects
  static_assert(kStStages == 4, "the stages are the four LDS objects T0..T3");
  __shared__ __attribute__((aligned(16))) uint16_t T0[TL::kStage];
  __shared__ __attribute__((aligned(16))) uint16_t T1[TL::kStage];
  __shared__ __attribute__((aligned(16))) uint16_t T2[TL::kStage];
  __shared__ __attribute__((aligned(16))) uint16_t T3[TL::kStage];
  __shared__ int plan[kStPlan];     // plan[s]: first item of segment s = 2b + branch
  __shared__ int last[kStMaxB];     // last position (lens - 1) of each sequence
  __shared__ int wtot[kStWaves];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar registers
  const int col = lane & 15, grp = lane >> 4;
  const int G = p.Hq / p.Hkv;
  const int S = 2 * p.B;

  // ---- item numbering -----------------------------------------------------
  {
    constexpr int PER = kStPlan / (kStWaves * 64);
    int cnt[PER], sum = 0;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int s = tid * PER + j;
      int c = 0;
      if (s < S) {
        const int b = s >> 1;
        const int i = clamp_len(p.lens[b], p.cap) - 1;
        if ((s & 1) == 0) {
          last[b] = i;
          c = i / kChunk - max(0, i - p.W + 1) / kChunk + 1;
        } else {
          c = p.selected[b] ? i / kChunk + 1 : 0;
        }
        c *= p.Hkv;
      }
      cnt[j] = c;
      sum += c;
    }
    // inclusive scan of the per-thread sums: within the wave, then across
    int incl = sum;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int y = __shfl_up(incl, off, 64);
      if (lane >= off) incl += y;
    }
    if (lane == 63) wtot[wave] = incl;
    __syncthreads();
    int base = 0;
    for (int w = 0; w < wave; ++w) base += wtot[w];
    int ex = base + incl - sum;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      plan[tid * PER + j] = ex;   // past S: the total
      ex += cnt[j];
    }
    __syncthreads();
  }
  const int N = plan[S];  // S < kStPlan; plan[S] = total items
  const int k0 = blockIdx.x;  // items k0, k0 + nwg, ... below N
  if (k0 >= N) return;

  // An item's description; every field is uniform over the workgroup.
  struct Item {
    int k, s, b, br, hk, c, ks, ke, t, tb;
  };
  auto load_item = [&] __device__ (Item& it, int k) __attribute__((always_inline)) {
    int s = it.s;
    while (__builtin_amdgcn_readfirstlane(plan[s + 1]) <= k) ++s;
    it.k = k;
    it.s = s;
    it.b = s >> 1;
    it.br = s & 1;
    const int i = __builtin_amdgcn_readfirstlane(last[it.b]);
    const int lo = max(0, i - p.W + 1);
    const int cf = it.br == 0 ? lo / kChunk : 0;
    const int nch = i / kChunk - cf + 1;
    const int r = k - __builtin_amdgcn_readfirstlane(plan[s]);
    it.hk = r / nch;
    it.c = cf + r % nch;
    it.ks = max(it.c * kChunk, it.br == 0 ? lo : 0);
    it.ke = min(it.c * kChunk + kChunk, i + 1);
    it.t = it.ks / kStKeys;
    it.tb = (it.ke - 1) / kStKeys;
  };
  auto advance = [&] __device__ (Item& it) __attribute__((always_inline)) {
    // next tile; false when the range is done
    if (it.t < it.tb) {
      ++it.t;
      return true;
    }
    if (it.k + p.nwg >= N) return false;
    load_item(it, it.k + p.nwg);
    return true;
  };

  // ---- tile staging ----------------------------------------------------------
  uint32_t k_voff[TL::kInstr], v_voff[TL::kInstr], q_voff[TL::qInstr];
#pragma unroll
  for (int i = 0; i < TL::kInstr; ++i) {
    const int byte = (wave + kStWaves * i) * 1024 + lane * 16;
    const int r = byte / (2 * D), q = (byte % (2 * D)) / 16;
    k_voff[i] = (uint32_t)(r * 2 * D + (q ^ TL::fk(r)) * 16);
    v_voff[i] = (uint32_t)(r * 2 * D + (q ^ TL::fv(r)) * 16);
  }
#pragma unroll
  for (int i = 0; i < TL::qInstr; ++i) {
    const int byte = (wave + kStWaves * i) * 1024 + lane * 16;
    const int r = byte / (2 * D), q = (byte % (2 * D)) / 16;
    q_voff[i] = (uint32_t)(r * 2 * D + (q ^ TL::fk(r)) * 16);
  }
  // tile t of (b, kv head): keys t*64 .. of the cache; keys past the last
  // position read as zero (the range ends there); `real` false: an empty
  // range (no memory is read) that only keeps the count of loads
  auto issue = [&] __device__ (const Item& it, bool real, uint16_t* dst)
      __attribute__((always_inline)) {
    const int key0 = it.t * kStKeys;
    const int i = __builtin_amdgcn_readfirstlane(last[it.b]);
    const int nbytes = real ? min(i + 1 - key0, kStKeys) * D * 2 : 0;
    const size_t row0 = ((size_t)it.b * p.Hkv + it.hk) * p.cap + key0;
    st_issue<TL::kInstr>(p.kc + row0 * D, nbytes, dst, k_voff, wave);
    st_issue<TL::kInstr>(p.vc + row0 * D, nbytes, dst + TL::kElems, v_voff, wave);
    // the G query rows of (b, kv head); rows G.. read as zero
    st_issue<TL::qInstr>(p.q + ((size_t)it.b * p.Hq + it.hk * G) * D, real ? G * D * 2 : 0,
                         dst + 2 * TL::kElems, q_voff, wave);
  };

  // ---- per-item state ----------------------------------------------------------
  f32x4 acc[DBW];
#pragma unroll
  for (int j = 0; j < DBW; ++j) acc[j] = (f32x4){};
  float m_run = -1.0e30f, l_run = 0.0f;

  typedef short v4i16 __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) v4i16* lds_v4i16_ptr;
  // LDS reads take one integer offset from the stage object itself: a
  // pointer derived through several steps loses the alias information that
  // tells the compiler this stage is not one whose loads are in flight, and
  // every such read then waits for all of them.
  //
  // K fragment (A of 16x16x32): key kb*16 + col, d chunk 4 s + grp
  auto read_k = [&] __device__ (const uint16_t* tb, int kb, int s)
      __attribute__((always_inline)) {
    const int r = kb * 16 + col;
    const int off = r * D + (((4 * s + grp) ^ TL::fk(r)) * 8);
    return __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(tb + off));
  };
  // Q^T fragment (B of 16x16x32): query head `col`, d chunk 4 s + grp
  auto read_q = [&] __device__ (const uint16_t* tb, int s) __attribute__((always_inline)) {
    const int off = 2 * TL::kElems + col * D + (((4 * s + grp) ^ TL::fk(col)) * 8);
    return __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(tb + off));
  };
  // V^T fragment (A of 16x16x16) through the transposing read: within each
  // 16-lane group, source lane s addresses key row 4*grp + s/4 and d columns
  // 16*db + 4*(s%4); the destination lane then holds d = 16*db + col for
  // keys kb*16 + 4*grp + [0, 4)
  auto read_v = [&] __device__ (const uint16_t* tb, int kb, int db)
      __attribute__((always_inline)) {
    const int r = kb * 16 + 4 * grp + (col >> 2);
    const int cc = 2 * db + ((col & 3) >> 1);
    const int off = TL::kElems + r * D + ((cc ^ TL::fv(r)) * 8) + 4 * (col & 1);
    return __builtin_bit_cast(
        bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_ptr)(tb + off)));
  };

  // one tile of the current item: scores of the four 16-key blocks, online
  // softmax per query column, this wave's d blocks of P V
  auto compute = [&] __device__ (const Item& it, const uint16_t* tb)
      __attribute__((always_inline)) {
    const int key0 = it.t * kStKeys;
    const bool full = key0 >= it.ks && key0 + kStKeys <= it.ke;
    bf16x8 qf[QS];
#pragma unroll
    for (int s = 0; s < QS; ++s) qf[s] = read_q(tb, s);
    f32x4 sc[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      bf16x8 kf[QS];
#pragma unroll
      for (int s = 0; s < QS; ++s) kf[s] = read_k(tb, kb, s);
#pragma unroll
      for (int s = 0; s < QS; ++s)
        sc[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[s], qf[s], s ? sc[kb] : (f32x4){},
                                                         0, 0, 0);
    }
    if (!full) {
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int key = key0 + kb * 16 + 4 * grp + e;
          sc[kb][e] = key >= it.ks && key < it.ke ? sc[kb][e] : -INFINITY;
        }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int e = 0; e < 4; ++e) mx = fmaxf(mx, sc[kb][e]);
    // the column's max over its four lanes (col, col+16, col+32, col+48)
    const auto s16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(mx), __float_as_uint(mx),
                                                      false, false);
    mx = fmaxf(__uint_as_float(s16[0]), __uint_as_float(s16[1]));
    const auto s32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx),
                                                      false, false);
    mx = fmaxf(__uint_as_float(s32[0]), __uint_as_float(s32[1])) * p.scale_log2;
    const float m_new = mx > m_run + kLazy ? mx : m_run;
    const float alpha = exp2f(m_run - m_new);
    m_run = m_new;
    l_run *= alpha;
    if (__builtin_amdgcn_ballot_w64(alpha != 1.0f) != 0) {
#pragma unroll
      for (int j = 0; j < DBW; ++j) acc[j] *= alpha;
    }
    // the row sum adds the bf16 values the products use (a dot product with
    // (1, 1)): with the lazy max a probability can reach 2^kLazy, and the
    // sum of the unrounded values would bias o by that weight's rounding
    const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      float pr[4];
#pragma unroll
      for (int e = 0; e < 4; ++e)
        pr[e] = __builtin_amdgcn_exp2f(fmaf(sc[kb][e], p.scale_log2, -m_run));
      const uint32_t p01 = pack_bf16x2(pr[0], pr[1]), p23 = pack_bf16x2(pr[2], pr[3]);
      l_run = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, p01), ones, l_run, false);
      l_run = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, p23), ones, l_run, false);
      const bf16x4 pt = __builtin_bit_cast(bf16x4, make_uint2(p01, p23));
#pragma unroll
      for (int j = 0; j < DBW; ++j)
        acc[j] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(read_v(tb, kb, wave * DBW + j), pt,
                                                           acc[j], 0, 0, 0);
    }
  };
  // the item's partial: this wave's d blocks for query heads < G; wave 0
  // adds the max and the sum
  constexpr int kDrop = 0x40000000;  // past every record group: dropped
  auto flush = [&] __device__ (const Item& it) __attribute__((always_inline)) {
    const auto s16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(l_run),
                                                      __float_as_uint(l_run), false, false);
    float l_tot = __uint_as_float(s16[0]) + __uint_as_float(s16[1]);
    const auto s32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(l_tot),
                                                      __float_as_uint(l_tot), false, false);
    l_tot = __uint_as_float(s32[0]) + __uint_as_float(s32[1]);
    // record group of (b, kv head, chunk, branch): G records of D + 4
    // floats (16-byte aligned)
    float* grp_base = p.part + ((((size_t)it.b * p.Hkv + it.hk) * p.nchunk + it.c) * 2 + it.br) *
                                   G * (D + 4);
    const bool mine = col < G;
    int off[DBW];
#pragma unroll
    for (int j = 0; j < DBW; ++j)
      off[j] = mine ? (col * (D + 4) + (wave * DBW + j) * 16 + 4 * grp) * 4 : kDrop;
    const int off_ml = mine && wave == 0 && grp == 0 ? (col * (D + 4) + D) * 4 : kDrop;
    st_store<DBW>(grp_base, G * (D + 4) * 4, acc, off, off_ml, m_run, l_tot);
#pragma unroll
    for (int j = 0; j < DBW; ++j) acc[j] = (f32x4){};
    m_run = -1.0e30f;
    l_run = 0.0f;
  };

  // ---- the stream ------------------------------------------------------------
  // Tile number q (counted from 0 over this workgroup's items) lives in
  // buffer q % 4; the steps are unrolled four times so every LDS access
  // names its buffer at compile time.
  Item ci, ii;  // the tile being computed, the next tile to issue
  ci.s = 0;
  load_item(ci, k0);
  ii = ci;
  bool more = true;  // ii names a tile not yet issued
  auto put = [&] __device__ (uint16_t* dst) __attribute__((always_inline)) {
    issue(ii, more, dst);
    if (more) more = advance(ii);
  };
  // each tile's loads are followed by one group of (here dropped) stores,
  // as in every step, so the first waits count the same way
  put(T0);
  put(T1);
  put(T2);
  bool live = true;
  auto step = [&] __device__ (const uint16_t* tc, uint16_t* tn) __attribute__((always_inline)) {
    // Three tiles are in flight and loads complete in issue order, so this
    // tile's loads have landed once no more than the two newer tiles' loads
    // are outstanding. Partial stores issued in between only add to the
    // count: the wait may last longer, never too short.
    __builtin_amdgcn_s_waitcnt(vm_wait<2 * (2 * TL::kInstr + TL::qInstr)>());
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
    __builtin_amdgcn_s_barrier();
    put(tn);
    compute(ci, tc);
    if (ci.t == ci.tb) flush(ci);
    live = advance(ci);
  };
#pragma unroll 1
  while (live) {
    step(T0, T3);
    if (live) step(T1, T0);
    if (live) step(T2, T1);
    if (live) step(T3, T2);
  }
  __builtin_amdgcn_s_waitcnt(vm_wait<0>());
}

struct RedParams {
  const float* part;   // as DecParams::part
  const int32_t* lens;
  const uint8_t* selected;
  const float* gate;
  void* o;             // [B][Hq][D]
  int B, Hq, Hkv, cap, W, nchunk;
};

// One workgroup per (b, query head): for each branch the kRedWaves waves
// take every kRedWaves-th chunk partial, kRedBatch of them in flight at a
// time, and keep an online merge (running max, rescaled sum and weighted
// values); the waves' states are then merged through LDS in wave order
// (deterministic) and the branches combined.
constexpr int kRedWaves = 8;
constexpr int kRedBatch = 16;

template <int D, bool BF16>
__global__ __launch_bounds__(kRedWaves * 64) void decode_reduce_kernel(RedParams p) {
  constexpr int NC = D / 64;   // d elements per lane
  __shared__ float wpart[kRedWaves][D + 2];
  const long long w = blockIdx.x;  // b * Hq + h
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int b = (int)(w / p.Hq);
  const int G = p.Hq / p.Hkv;
  const int hk = (int)(w % p.Hq) / G, g = (int)(w % p.Hq) % G;
  const long long row0 = (long long)b * p.Hkv + hk;
  const int i = clamp_len(p.lens[b], p.cap) - 1;
  const int lo = max(0, i - p.W + 1);
  const bool sel = p.selected[b] != 0;
  float out[NC];
#pragma unroll
  for (int cc = 0; cc < NC; ++cc) out[cc] = 0.0f;
  for (int br = 0; br < 2; ++br) {
    if (br == 1 && !sel) break;  // uniform
    const int cfirst = br == 0 ? lo / kChunk : 0;
    const int clast = i / kChunk;
    float m = kNeg, l = 0.0f, a[NC];
#pragma unroll
    for (int cc = 0; cc < NC; ++cc) a[cc] = 0.0f;
    for (int c0 = cfirst + wave; c0 <= clast; c0 += kRedWaves * kRedBatch) {
      float pm[kRedBatch], pl[kRedBatch], pa[kRedBatch][NC];
#pragma unroll
      for (int u = 0; u < kRedBatch; ++u) {
        const int c = c0 + u * kRedWaves;
        const bool ok = c <= clast;
        const float* pt =
            p.part + ((row0 * p.nchunk + (ok ? c : cfirst)) * 2 + br) * G * (D + 4) + g * (D + 4);
        pm[u] = ok ? pt[D] : kNeg;
        pl[u] = ok ? pt[D + 1] : 0.0f;
#pragma unroll
        for (int cc = 0; cc < NC; ++cc) pa[u][cc] = ok ? pt[lane + 64 * cc] : 0.0f;
      }
      float mx = m;
#pragma unroll
      for (int u = 0; u < kRedBatch; ++u) mx = fmaxf(mx, pm[u]);
      const float f0 = exp2f(m - mx);
      l *= f0;
#pragma unroll
      for (int cc = 0; cc < NC; ++cc) a[cc] *= f0;
#pragma unroll
      for (int u = 0; u < kRedBatch; ++u) {
        const float f = exp2f(pm[u] - mx);
        l = fmaf(f, pl[u], l);
#pragma unroll
        for (int cc = 0; cc < NC; ++cc) a[cc] = fmaf(f, pa[u][cc], a[cc]);
      }
      m = mx;
    }
    // merge the waves' states in wave order
#pragma unroll
    for (int cc = 0; cc < NC; ++cc) wpart[wave][lane + 64 * cc] = a[cc];
    if (lane == 0) {
      wpart[wave][D] = m;
      wpart[wave][D + 1] = l;
    }
    __syncthreads();
    if (wave == 0) {
      float mx = kNeg;
      for (int v = 0; v < kRedWaves; ++v) mx = fmaxf(mx, wpart[v][D]);
      float tot = 0.0f, sum[NC];
#pragma unroll
      for (int cc = 0; cc < NC; ++cc) sum[cc] = 0.0f;
      for (int v = 0; v < kRedWaves; ++v) {
        const float f = exp2f(wpart[v][D] - mx);
        tot = fmaf(f, wpart[v][D + 1], tot);
#pragma unroll
        for (int cc = 0; cc < NC; ++cc) sum[cc] = fmaf(f, wpart[v][lane + 64 * cc], sum[cc]);
      }
      const float wgt = br == 0 ? 1.0f : 1.0f / (1.0f + expf(-p.gate[b]));
#pragma unroll
      for (int cc = 0; cc < NC; ++cc) out[cc] = fmaf(wgt, sum[cc] / tot, out[cc]);
    }
    __syncthreads();
  }
  if (wave != 0) return;
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

// compute units of the current device (the stream kernel runs one
// workgroup on each)
int compute_units() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1)
    return 256;
  return n;
}

hipError_t launch_reduce_d(int D, bool bf16, const DecodeDims& d, const DecodeArgs& a, int nchunk,
                           hipStream_t s);

// The chunked kernel: float32 caches, or more sequences than the stream
// kernel's item table holds; G is a template parameter.
template <int D, int G, bool BF16>
hipError_t decode_chunked(const DecodeDims& d, const DecodeArgs& a, hipStream_t s) {
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
  const dim3 grid((unsigned)(2LL * d.B * d.Hkv * p.nchunk));
  hipLaunchKernelGGL((decode_partial_kernel<D, G, BF16>), grid, dim3(kDecWaves * 64), 0, s, p);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_reduce_d(D, BF16, d, a, p.nchunk, s);
}

// The stream kernel: bf16 caches, B <= kStMaxB, any G <= kStCols.
template <int D>
hipError_t decode_stream(const DecodeDims& d, const DecodeArgs& a, hipStream_t s) {
  StParams sp;
  sp.q = static_cast<const uint16_t*>(a.q);
  sp.kc = static_cast<const uint16_t*>(a.k_cache);
  sp.vc = static_cast<const uint16_t*>(a.v_cache);
  sp.lens = a.lens;
  sp.selected = a.selected;
  sp.part = a.part;
  sp.B = d.B;
  sp.Hq = d.Hq;
  sp.Hkv = d.Hkv;
  sp.cap = d.cap;
  sp.W = d.window;
  sp.nchunk = (d.cap + kChunk - 1) / kChunk;
  sp.nwg = compute_units();
  sp.scale_log2 = d.scale * kLog2e;
  hipLaunchKernelGGL((decode_stream_kernel<D>), dim3((unsigned)sp.nwg), dim3(kStWaves * 64), 0,
                     s, sp);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_reduce_d(D, true, d, a, sp.nchunk, s);
}

hipError_t launch_reduce_d(int D, bool bf16, const DecodeDims& d, const DecodeArgs& a, int nchunk,
                           hipStream_t s) {
  RedParams r;
  r.part = a.part;
  r.lens = a.lens;
  r.selected = a.selected;
  r.gate = a.gate;
  r.o = a.o;
  r.B = d.B;
  r.Hq = d.Hq;
  r.Hkv = d.Hkv;
  r.cap = d.cap;
  r.W = d.window;
  r.nchunk = nchunk;
  const dim3 grid((unsigned)((long long)d.B * d.Hq)), block(kRedWaves * 64);
  if (D == 64 && bf16) hipLaunchKernelGGL((decode_reduce_kernel<64, true>), grid, block, 0, s, r);
  else if (D == 64) hipLaunchKernelGGL((decode_reduce_kernel<64, false>), grid, block, 0, s, r);
  else if (bf16) hipLaunchKernelGGL((decode_reduce_kernel<128, true>), grid, block, 0, s, r);
  else hipLaunchKernelGGL((decode_reduce_kernel<128, false>), grid, block, 0, s, r);
  return hipGetLastError();
}

bool stream_path(const DecodeDims& d) {
  return d.dtype == 1 && d.B <= kStMaxB && d.Hq / d.Hkv <= kStCols;
}

template <int D, bool BF16>
hipError_t decode_g(const DecodeDims& d, const DecodeArgs& a, hipStream_t s) {
  if (BF16 && stream_path(d)) return decode_stream<D>(d, a, s);
  switch (d.Hq / d.Hkv) {
    case 1: return decode_chunked<D, 1, BF16>(d, a, s);
    case 2: return decode_chunked<D, 2, BF16>(d, a, s);
    case 4: return decode_chunked<D, 4, BF16>(d, a, s);
    case 7: return decode_chunked<D, 7, BF16>(d, a, s);
    case 8: return decode_chunked<D, 8, BF16>(d, a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

int64_t decode_chunks(int64_t cap) { return (cap + kChunk - 1) / kChunk; }

bool decode_group_supported(const DecodeDims& d) {
  if (stream_path(d)) return true;  // any G up to 16
  const int G = d.Hq / d.Hkv;
  return G == 1 || G == 2 || G == 4 || G == 7 || G == 8;
}

size_t decode_partial_bytes(const DecodeDims& d) {
  const size_t nchunk = (d.cap + kChunk - 1) / kChunk;
  return ((size_t)d.B * d.Hq * nchunk * 2 * (d.d + 4) * sizeof(float) + 255) / 256 * 256;
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
