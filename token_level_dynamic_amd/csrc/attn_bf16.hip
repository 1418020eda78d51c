// bf16 attention kernels for both branches, on CDNA4 matrix cores.
//
//   local  (every query):    softmax over L(i) = [max(0, i-W+1), i]
//     "Local-global attention", attention-mask sketch (causal and
//     within-window); LoGo abstract (every token gets local attention)
//   global (selected rows):  softmax over G(i) = [0, i]
//     "Learning When to Attend", "The Architecture of Conditional
//     Attention" (exact full-context attention for a sparse query subset)
//
// Both are one flash-style kernel: K/V tiles of 64 keys are staged through
// LDS and each wave keeps an online softmax for 32 query rows in registers.
//
// Work unit = (batch b, kv head, block of 32 query rows, one query head of
// the group). A workgroup of 4 waves takes 4 consecutive units of one
// (b, kv head); units run position-block-major, so grouped-query heads
// that read the same keys share a workgroup and its K/V tiles. Local rows
// are consecutive positions; global rows are the selected positions
// gathered through idx (ascending), so every tile of them is dense.
//
// Matrix-core mapping (v_mfma_f32_32x32x16_bf16, one wave):
//   S^T[32 keys x 32 queries] = K_tile(32 x d) * Q^T(d x 32)
//     A = K rows from LDS, B = Q rows held in registers for the whole loop.
//     Accumulator lane l: query l%32, keys kb*32 + j*8 + (l/32)*4 + i for
//     element j*4+i, so a query's 64 scores of a tile live in two lanes
//     (l and l^32): row max and sum need one cross-half exchange.
//   O^T[32 d x 32 queries] += V^T(32 x 16 keys) * P^T(16 keys x 32 queries)
//     B = the probabilities straight from the S^T accumulator (converted to
//     bf16); the contraction order over keys is permuted so each lane's own
//     8 scores form its B operand, and V^T is read from LDS in the same key
//     order. V^T is produced by transposing 4x8 blocks in registers while
//     staging V (global V is [key][d]).
//
// Workgroup order is XCD-aware: workgroup ids are dealt to the 8 XCDs in
// turn, so logical tiles are renumbered so each XCD walks a contiguous
// range of (b, kv head) units and keeps their K/V in its own L2. Global
// tiles of one unit run longest causal prefix first.
#include "logo_internal.h"

namespace logo {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kRows = 32;     // query rows per wave
constexpr int kKeys = 64;     // keys per tile
constexpr int kNumXcd = 8;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegInit = -1.0e30f;

template <int D>
struct Smem {
  static constexpr int kStride = D + 8;        // bf16 per K row (16 B pad)
  static constexpr int vStride = kKeys + 4;    // bf16 per V^T row (8 B pad)
  static constexpr int kElems = kKeys * kStride;
  static constexpr int vElems = D * vStride;
  static constexpr int stage = kElems + vElems;
  static constexpr int bytes = 2 * stage * 2;  // two stages, 2 B each
};

struct Params {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const int32_t* idx;
  const int32_t* rank;
  const float* gate;
  float* out_f32;
  const float* scratch;
  uint16_t* out_io;
  int B, Hq, Hkv, n, W, ksel;
  float scale_log2;     // scale * log2(e)
  int units;            // units per (b, kv head)
  int wg_per_unit;      // workgroups per (b, kv head)
  int total_wg;         // B * Hkv * wg_per_unit
  int per_xcd;          // ceil(total_wg / 8)
};

__device__ __forceinline__ uint16_t f32_to_bf16_bits(float x) {
  bf16x2 r = __builtin_convertvector((f32x2){x, 0.0f}, bf16x2);
  return (uint16_t)(__builtin_bit_cast(uint32_t, r) & 0xffffu);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  bf16x2 r = __builtin_convertvector((f32x2){a, b}, bf16x2);
  return __builtin_bit_cast(uint32_t, r);
}

template <int D, bool GLOBAL, int EPI>
__global__ __launch_bounds__(kThreads, 2) void attn_bf16_kernel(Params p) {
  using SM = Smem<D>;
  extern __shared__ __attribute__((aligned(16))) uint16_t smem[];

  // ---- which tile -------------------------------------------------------
  const int bid = blockIdx.x;
  const int L = (bid % kNumXcd) * p.per_xcd + bid / kNumXcd;
  if (L >= p.total_wg) return;
  const int unit_bh = L / p.wg_per_unit;       // b * Hkv + kv head
  int w = L % p.wg_per_unit;
  if (GLOBAL) w = p.wg_per_unit - 1 - w;        // longest prefix first
  const int b = unit_bh / p.Hkv;
  const int hk = unit_bh % p.Hkv;
  const int G = p.Hq / p.Hkv;
  const int R = GLOBAL ? p.ksel : p.n;          // rows per (b, head)

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int col = lane & 31;   // query row of this lane within the wave
  const int half = lane >> 5;  // which 8-wide k slice / 4-row group

  // Units of this workgroup: w*4 .. w*4+3 (position-block-major).
  const int u_first = w * kWaves;
  const int u_last = min(u_first + kWaves, p.units) - 1;
  const int u = u_first + wave;
  const bool wave_on = u < p.units;
  const int pb = (wave_on ? u : u_last) / G;
  const int h = hk * G + (wave_on ? u : u_last) % G;

  // Row positions of this lane and the wave's / workgroup's key range.
  const int r_lane = pb * kRows + col;
  const bool row_ok = wave_on && r_lane < R;
  int pos;
  if (GLOBAL) {
    pos = (r_lane < R) ? p.idx[(size_t)b * p.ksel + r_lane] : -1;
  } else {
    pos = r_lane;
  }
  const int r_first = pb * kRows;
  const int r_last = min(pb * kRows + kRows, R) - 1;
  // positions of this wave's first and last real rows (ascending in rows)
  int wpos_lo, wpos_hi;
  if (GLOBAL) {
    wpos_lo = p.idx[(size_t)b * p.ksel + r_first];
    wpos_hi = p.idx[(size_t)b * p.ksel + r_last];
  } else {
    wpos_lo = r_first;
    wpos_hi = r_last;
  }
  const int wkey_lo = GLOBAL ? 0 : max(0, wpos_lo - p.W + 1);
  const int wkey_hi = wpos_hi;
  // workgroup range: first unit's first row to last unit's last row
  const int pb_first = u_first / G;
  const int pb_last = u_last / G;
  int gpos_lo, gpos_hi;
  {
    const int rf = pb_first * kRows;
    const int rl = min(pb_last * kRows + kRows, R) - 1;
    if (GLOBAL) {
      gpos_lo = p.idx[(size_t)b * p.ksel + rf];
      gpos_hi = p.idx[(size_t)b * p.ksel + rl];
    } else {
      gpos_lo = rf;
      gpos_hi = rl;
    }
  }
  const int gkey_lo = GLOBAL ? 0 : max(0, gpos_lo - p.W + 1);
  const int gkey_hi = gpos_hi;
  const int t_lo = gkey_lo / kKeys;
  const int t_hi = gkey_hi / kKeys;

  const size_t kv_base = (size_t)(b * p.Hkv + hk) * p.n * D;
  const uint16_t* kg = p.k + kv_base;
  const uint16_t* vg = p.v + kv_base;

  // ---- Q rows into registers -------------------------------------------
  constexpr int QS = D / 16;  // k-steps of 16 along d
  bf16x8 qreg[QS];
  {
    const bool ok = row_ok && pos >= 0;
    const uint16_t* qrow = p.q + ((size_t)(b * p.Hq + h) * p.n + (ok ? pos : 0)) * D;
#pragma unroll
    for (int s = 0; s < QS; ++s) {
      uint4 x = ok ? *reinterpret_cast<const uint4*>(qrow + s * 16 + half * 8)
                   : make_uint4(0, 0, 0, 0);
      qreg[s] = __builtin_bit_cast(bf16x8, x);
    }
  }

  // ---- staging of K / V^T tiles ----------------------------------------
  constexpr int KCH = kKeys * D / 8 / kThreads;   // 16-B K chunks per thread
  constexpr int VBLK = (kKeys / 4) * (D / 8);     // 4x8 V blocks per tile
  uint4 kpre[KCH];
  uint4 vpre[4];
  const bool v_thread = tid < VBLK;
  const int v_dg = tid % (D / 8);
  const int v_kg = tid / (D / 8);

  auto load_tile = [&](int t) {
    const int key0 = t * kKeys;
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      const int c = tid + i * kThreads;
      const int row = c / (D / 8);
      const int c8 = c % (D / 8);
      const int key = key0 + row;
      kpre[i] = key < p.n ? *reinterpret_cast<const uint4*>(kg + (size_t)key * D + c8 * 8)
                          : make_uint4(0, 0, 0, 0);
    }
    if (v_thread) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int key = key0 + v_kg * 4 + r;
        vpre[r] = key < p.n ? *reinterpret_cast<const uint4*>(vg + (size_t)key * D + v_dg * 8)
                            : make_uint4(0, 0, 0, 0);
      }
    }
  };
  auto store_tile = [&](int stage) {
    uint16_t* ks = smem + stage * SM::stage;
    uint16_t* vs = ks + SM::kElems;
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      const int c = tid + i * kThreads;
      const int row = c / (D / 8);
      const int c8 = c % (D / 8);
      *reinterpret_cast<uint4*>(ks + row * SM::kStride + c8 * 8) = kpre[i];
    }
    if (v_thread) {
      // rows r0..r3 (keys), dwords m (d pairs 2m, 2m+1) -> V^T rows d, 4 keys each
      const uint32_t* r0 = reinterpret_cast<const uint32_t*>(&vpre[0]);
      const uint32_t* r1 = reinterpret_cast<const uint32_t*>(&vpre[1]);
      const uint32_t* r2 = reinterpret_cast<const uint32_t*>(&vpre[2]);
      const uint32_t* r3 = reinterpret_cast<const uint32_t*>(&vpre[3]);
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        uint2 even, odd;
        even.x = (r0[m] & 0xffffu) | (r1[m] << 16);
        even.y = (r2[m] & 0xffffu) | (r3[m] << 16);
        odd.x = (r0[m] >> 16) | (r1[m] & 0xffff0000u);
        odd.y = (r2[m] >> 16) | (r3[m] & 0xffff0000u);
        const int d0 = v_dg * 8 + 2 * m;
        *reinterpret_cast<uint2*>(vs + d0 * SM::vStride + v_kg * 4) = even;
        *reinterpret_cast<uint2*>(vs + (d0 + 1) * SM::vStride + v_kg * 4) = odd;
      }
    }
  };

  // ---- online softmax state --------------------------------------------
  constexpr int DB = D / 32;  // 32-wide d blocks of the output
  f32x16 acc_o[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i) acc_o[i] = (f32x16){};
  float m_run = kNegInit;
  float l_run = 0.0f;

  if (t_lo <= t_hi) {
    load_tile(t_lo);
    store_tile(0);
  }
  __syncthreads();

#pragma unroll 1
  for (int t = t_lo; t <= t_hi; ++t) {
    const int stage = (t - t_lo) & 1;
    const bool more = t < t_hi;
    if (more) load_tile(t + 1);

    const int key0 = t * kKeys;
    const bool active = wave_on && key0 <= wkey_hi && key0 + kKeys - 1 >= wkey_lo;
    if (active) {
      const uint16_t* ks = smem + stage * SM::stage;
      const uint16_t* vs = ks + SM::kElems;
      // S^T = K Q^T for two 32-key blocks
      f32x16 sc[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        sc[kb] = (f32x16){};
        const uint16_t* krow = ks + (kb * 32 + col) * SM::kStride + half * 8;
#pragma unroll
        for (int s = 0; s < QS; ++s) {
          bf16x8 a = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(krow + s * 16));
          sc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qreg[s], sc[kb], 0, 0, 0);
        }
      }
      // mask only where some row of this wave sees an invalid key here
      bool full;
      if (GLOBAL) {
        full = key0 + kKeys - 1 <= wpos_lo;
      } else {
        full = key0 >= wpos_hi - p.W + 1 && key0 + kKeys - 1 <= wpos_lo;
      }
      float mx = kNegInit;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          float x = sc[kb][e] * p.scale_log2;
          if (!full) {
            const int key = key0 + kb * 32 + (e >> 2) * 8 + half * 4 + (e & 3);
            bool ok = key <= pos;
            if (!GLOBAL) ok = ok && key >= pos - p.W + 1;
            x = ok ? x : -INFINITY;
          }
          sc[kb][e] = x;
          mx = fmaxf(mx, x);
        }
      }
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      const float m_new = fmaxf(m_run, mx);
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
      float lsum = 0.0f;
      bf16x8 pb16[2][2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        float pv[16];
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          pv[e] = __builtin_amdgcn_exp2f(sc[kb][e] - m_new);
          lsum += pv[e];
        }
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          uint4 packed;
          packed.x = pack_bf16x2(pv[hh * 8 + 0], pv[hh * 8 + 1]);
          packed.y = pack_bf16x2(pv[hh * 8 + 2], pv[hh * 8 + 3]);
          packed.z = pack_bf16x2(pv[hh * 8 + 4], pv[hh * 8 + 5]);
          packed.w = pack_bf16x2(pv[hh * 8 + 6], pv[hh * 8 + 7]);
          pb16[kb][hh] = __builtin_bit_cast(bf16x8, packed);
        }
      }
      l_run = l_run * alpha + lsum;
#pragma unroll
      for (int db = 0; db < DB; ++db) acc_o[db] *= alpha;
      // O^T += V^T P^T, 4 steps of 16 keys
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const uint16_t* vrow = vs + (db * 32 + col) * SM::vStride + half * 4;
#pragma unroll
        for (int st = 0; st < 4; ++st) {
          const int kb = st >> 1, hh = st & 1;
          const int k0 = kb * 32 + hh * 16;
          uint2 lo = *reinterpret_cast<const uint2*>(vrow + k0);
          uint2 hi = *reinterpret_cast<const uint2*>(vrow + k0 + 8);
          uint4 a4 = make_uint4(lo.x, lo.y, hi.x, hi.y);
          acc_o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              __builtin_bit_cast(bf16x8, a4), pb16[kb][hh], acc_o[db], 0, 0, 0);
        }
      }
    }
    if (more) store_tile(stage ^ 1);
    __syncthreads();
  }

  // ---- epilogue ----------------------------------------------------------
  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  if (!row_ok) return;
  const float inv = 1.0f / l_tot;
  const size_t head_row = (size_t)(b * p.Hq + h);
  // EPI: 0 LocalAll, 1 LocalFused, 2 GlobalAll, 3 GlobalFused
  int rk = -1;
  if (EPI == 1) rk = p.rank[(size_t)b * p.n + pos];
  float sig = 0.0f;
  if (EPI == 3) sig = 1.0f / (1.0f + expf(-p.gate[(size_t)b * p.n + pos]));
#pragma unroll
  for (int db = 0; db < DB; ++db) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int d0 = db * 32 + j * 8 + half * 4;
      float4 o4 = make_float4(acc_o[db][j * 4 + 0] * inv, acc_o[db][j * 4 + 1] * inv,
                              acc_o[db][j * 4 + 2] * inv, acc_o[db][j * 4 + 3] * inv);
      if (EPI == 0) {
        *reinterpret_cast<float4*>(p.out_f32 + (head_row * p.n + pos) * D + d0) = o4;
      } else if (EPI == 2) {
        *reinterpret_cast<float4*>(p.out_f32 + (head_row * p.ksel + r_lane) * D + d0) = o4;
      } else if (EPI == 1) {
        if (rk >= 0) {
          *reinterpret_cast<float4*>(p.out_f32 + (head_row * p.ksel + rk) * D + d0) = o4;
        } else {
          uint2 w2 = make_uint2(pack_bf16x2(o4.x, o4.y), pack_bf16x2(o4.z, o4.w));
          *reinterpret_cast<uint2*>(p.out_io + (head_row * p.n + pos) * D + d0) = w2;
        }
      } else {
        const float4 l4 =
            *reinterpret_cast<const float4*>(p.scratch + (head_row * p.ksel + r_lane) * D + d0);
        float4 c4 = make_float4(l4.x + sig * o4.x, l4.y + sig * o4.y, l4.z + sig * o4.z,
                                l4.w + sig * o4.w);
        uint2 w2 = make_uint2(pack_bf16x2(c4.x, c4.y), pack_bf16x2(c4.z, c4.w));
        *reinterpret_cast<uint2*>(p.out_io + (head_row * p.n + pos) * D + d0) = w2;
      }
    }
  }
}

template <int D, bool GLOBAL, int EPI>
hipError_t launch_one(const Params& prm, hipStream_t s) {
  // more than 64 KiB of dynamic LDS must be allowed per kernel (idempotent)
  static const hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void*>(&attn_bf16_kernel<D, GLOBAL, EPI>),
      hipFuncAttributeMaxDynamicSharedMemorySize, Smem<D>::bytes);
  if (attr != hipSuccess) return attr;
  const int grid = prm.per_xcd * kNumXcd;
  hipLaunchKernelGGL((attn_bf16_kernel<D, GLOBAL, EPI>), dim3(grid), dim3(kThreads),
                     Smem<D>::bytes, s, prm);
  return hipGetLastError();
}

template <int D>
hipError_t dispatch_epi(Epi epi, const Params& prm, hipStream_t s) {
  switch (epi) {
    case Epi::LocalAll: return launch_one<D, false, 0>(prm, s);
    case Epi::LocalFused: return launch_one<D, false, 1>(prm, s);
    case Epi::GlobalAll: return launch_one<D, true, 2>(prm, s);
    case Epi::GlobalFused: return launch_one<D, true, 3>(prm, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_attn_bf16(const Dims& d, Epi epi, const AttnArgs& a, hipStream_t s) {
  const bool global = epi == Epi::GlobalAll || epi == Epi::GlobalFused;
  const int R = global ? d.k : d.n;
  if (d.B == 0 || R == 0) return hipSuccess;
  Params prm;
  prm.q = static_cast<const uint16_t*>(a.q);
  prm.k = static_cast<const uint16_t*>(a.k);
  prm.v = static_cast<const uint16_t*>(a.v);
  prm.idx = a.idx;
  prm.rank = a.rank;
  prm.gate = a.gate;
  prm.out_f32 = a.out_f32;
  prm.scratch = a.scratch;
  prm.out_io = static_cast<uint16_t*>(a.out_io);
  prm.B = d.B;
  prm.Hq = d.Hq;
  prm.Hkv = d.Hkv;
  prm.n = d.n;
  prm.W = d.window;
  prm.ksel = d.k;
  prm.scale_log2 = d.scale * kLog2e;
  const int G = d.Hq / d.Hkv;
  const int npb = (R + kRows - 1) / kRows;
  prm.units = npb * G;
  prm.wg_per_unit = (prm.units + kWaves - 1) / kWaves;
  prm.total_wg = d.B * d.Hkv * prm.wg_per_unit;
  prm.per_xcd = (prm.total_wg + kNumXcd - 1) / kNumXcd;
  if (d.d == 64) return dispatch_epi<64>(epi, prm, s);
  if (d.d == 128) return dispatch_epi<128>(epi, prm, s);
  return hipErrorInvalidValue;
}

}  // namespace logo
