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
//     8 scores form its B operand. A = V^T comes from the row-major V tile
//     in LDS through the gfx950 transposing LDS read (ds_read_b64_tr_b16),
//     which hands each lane 4 consecutive keys of its own d column.
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
constexpr float kLazy = 8.0f;  // log2 headroom before the running max moves

template <int D>
struct Smem {
  // Row strides (bf16): K rows 16 B of pad (stride = 4 mod 32 banks) keep
  // the 16-byte operand reads conflict-free; V rows 32 B of pad (stride =
  // 8 mod 32 banks) keep the transposing 8-byte reads conflict-free.
  static constexpr int kStride = D + 8;
  static constexpr int vStride = D + 16;
  static constexpr int kElems = kKeys * kStride;
  static constexpr int vElems = kKeys * vStride;
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
__global__ __launch_bounds__(kThreads, 2)
__attribute__((amdgpu_waves_per_eu(2, 2))) void attn_bf16_kernel(Params p) {
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

  // ---- staging of K / V tiles ------------------------------------------
  // Both are copied row-major in 16-byte chunks through registers. Rows past
  // the end are clamped to the last key: such keys only occur in tiles that
  // are masked per element (they lie after every query), so their scores
  // are discarded and their values are finite. The loads have no branches,
  // so they stay in flight across the tile's matrix work.
  constexpr int KCH = kKeys * D / 8 / kThreads;   // 16-B chunks per thread: 2 or 4
  static_assert(KCH == 2 || KCH == 4, "staging assumes 2 or 4 chunks per thread");
  constexpr int kRowStep = kThreads / (D / 8);    // rows between a thread's chunks
  uint4 kp0, kp1, kp2, kp3, vp0, vp1, vp2, vp3;
  const int st_row0 = tid / (D / 8);
  const int st_col = (tid % (D / 8)) * 8;
  const uint16_t* kg_thread = kg + st_col;
  const uint16_t* vg_thread = vg + st_col;
  uint16_t* ks_thread = smem + st_row0 * SM::kStride + st_col;
  uint16_t* vs_thread = smem + SM::kElems + st_row0 * SM::vStride + st_col;
  const int last_key = p.n - 1;

#define LOGO_ROW(I_) ((size_t)min(key0_ + st_row0 + (I_) * kRowStep, last_key) * D)
#define LOGO_LOAD_TILE(T_)                                                          \
  do {                                                                              \
    const int key0_ = (T_) * kKeys;                                                 \
    kp0 = *reinterpret_cast<const uint4*>(kg_thread + LOGO_ROW(0));                 \
    vp0 = *reinterpret_cast<const uint4*>(vg_thread + LOGO_ROW(0));                 \
    kp1 = *reinterpret_cast<const uint4*>(kg_thread + LOGO_ROW(1));                 \
    vp1 = *reinterpret_cast<const uint4*>(vg_thread + LOGO_ROW(1));                 \
    if constexpr (KCH == 4) {                                                       \
      kp2 = *reinterpret_cast<const uint4*>(kg_thread + LOGO_ROW(2));               \
      vp2 = *reinterpret_cast<const uint4*>(vg_thread + LOGO_ROW(2));               \
      kp3 = *reinterpret_cast<const uint4*>(kg_thread + LOGO_ROW(3));               \
      vp3 = *reinterpret_cast<const uint4*>(vg_thread + LOGO_ROW(3));               \
    }                                                                               \
  } while (0)

#define LOGO_STORE_TILE(STAGE_)                                                     \
  do {                                                                              \
    const int off_ = (STAGE_) * SM::stage;                                          \
    *reinterpret_cast<uint4*>(ks_thread + off_) = kp0;                              \
    *reinterpret_cast<uint4*>(vs_thread + off_) = vp0;                              \
    *reinterpret_cast<uint4*>(ks_thread + off_ + kRowStep * SM::kStride) = kp1;     \
    *reinterpret_cast<uint4*>(vs_thread + off_ + kRowStep * SM::vStride) = vp1;     \
    if constexpr (KCH == 4) {                                                       \
      *reinterpret_cast<uint4*>(ks_thread + off_ + 2 * kRowStep * SM::kStride) = kp2; \
      *reinterpret_cast<uint4*>(vs_thread + off_ + 2 * kRowStep * SM::vStride) = vp2; \
      *reinterpret_cast<uint4*>(ks_thread + off_ + 3 * kRowStep * SM::kStride) = kp3; \
      *reinterpret_cast<uint4*>(vs_thread + off_ + 3 * kRowStep * SM::vStride) = vp3; \
    }                                                                               \
  } while (0)

  // Transposing V reads (ds_read_b64_tr_b16). Within each 16-lane group the
  // instruction gives destination lane 4q+j, element e, the element j of the
  // 8 bytes addressed by source lane 4e+q. Source lane s of group G = l/16
  // therefore addresses key row (s/4) and d columns 16*(G%2) + 4*(s%4): the
  // destination lane then holds 4 consecutive keys for its own d column,
  // d = l % 32 of the 32-wide block, as the MFMA A operand needs.
  const int tr_row = (lane & 15) >> 2;
  const int tr_col = ((lane >> 4) & 1) * 16 + (lane & 3) * 4;

  // ---- online softmax state --------------------------------------------
  constexpr int DB = D / 32;  // 32-wide d blocks of the output
  f32x16 acc_o[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i) acc_o[i] = (f32x16){};
  float m_run = kNegInit;
  float l_run = 0.0f;

  if (t_lo <= t_hi) {
    LOGO_LOAD_TILE(t_lo);
    LOGO_STORE_TILE(0);
  }
  __syncthreads();

#pragma unroll 1
  for (int t = t_lo; t <= t_hi; ++t) {
    const int stage = (t - t_lo) & 1;
    const bool more = t < t_hi;
    // unconditional (rows clamped): a branch here would make the compiler
    // wait for these loads before the tile's matrix work
    LOGO_LOAD_TILE(t + 1);

    const int key0 = t * kKeys;
    const bool active = wave_on && key0 <= wkey_hi && key0 + kKeys - 1 >= wkey_lo;
    if (__builtin_amdgcn_readfirstlane(active)) {  // uniform per wave
      const uint16_t* ks = smem + stage * SM::stage;
      const uint16_t* vs = ks + SM::kElems;
      // S^T = K Q^T for two 32-key blocks; each block's K fragments are all
      // requested from LDS before its MFMA chain starts
      f32x16 sc[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const uint16_t* krow = ks + (kb * 32 + col) * SM::kStride + half * 8;
        bf16x8 kf[QS];
#pragma unroll
        for (int s = 0; s < QS; ++s)
          kf[s] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(krow + s * 16));
        sc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[0], qreg[0], (f32x16){}, 0, 0, 0);
#pragma unroll
        for (int s = 1; s < QS; ++s)
          sc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[s], qreg[s], sc[kb], 0, 0, 0);
      }
      // mask only where some row of this wave sees an invalid key here
      bool full;
      if (GLOBAL) {
        full = key0 + kKeys - 1 <= wpos_lo;
      } else {
        full = key0 >= wpos_hi - p.W + 1 && key0 + kKeys - 1 <= wpos_lo;
      }
      if (!full) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int key = key0 + kb * 32 + (e >> 2) * 8 + half * 4 + (e & 3);
            bool ok = key <= pos;
            if (!GLOBAL) ok = ok && key >= pos - p.W + 1;
            sc[kb][e] = ok ? sc[kb][e] : -INFINITY;
          }
        }
      }
      // raw row max; the scale (> 0) is folded into the exponent below
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int e = 0; e < 16; ++e) mx = fmaxf(mx, sc[kb][e]);
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64)) * p.scale_log2;
      // Lazy rescaling: the running max m_run (log2 units) only moves when a
      // row's new max exceeds it by more than kLazy, so probabilities stay
      // below 2^kLazy and the output is rescaled only on those tiles.
      const bool grow = mx > m_run + kLazy;
      if (__builtin_amdgcn_ballot_w64(grow) != 0) {
        const float m_new = grow ? mx : m_run;
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
        m_run = m_new;
        l_run *= alpha;
#pragma unroll
        for (int db = 0; db < DB; ++db) acc_o[db] *= alpha;
      }
      const float neg_m = -m_run;
      float lsum = 0.0f;
      bf16x8 pb16[2][2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        float pv[16];
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          pv[e] = __builtin_amdgcn_exp2f(fmaf(sc[kb][e], p.scale_log2, neg_m));
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
      l_run += lsum;
      // O^T += V^T P^T, 4 steps of 16 keys per 32-wide d block. Step st
      // covers keys kb*32 + hh*16 + [0, 16); this lane's half supplies keys
      // +4*half+[0,4) and +8+4*half+[0,4), matching its probabilities.
      typedef short v4i16 __attribute__((ext_vector_type(4)));
      typedef __attribute__((address_space(3))) v4i16* lds_v4i16_ptr;
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        bf16x8 vf[4];
#pragma unroll
        for (int st = 0; st < 4; ++st) {
          const int kbase = (st >> 1) * 32 + (st & 1) * 16 + half * 4 + tr_row;
          const uint16_t* a0 = vs + kbase * SM::vStride + db * 32 + tr_col;
          const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_ptr)(a0));
          const v4i16 hi =
              __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_ptr)(a0 + 8 * SM::vStride));
          const uint2 l2 = __builtin_bit_cast(uint2, lo);
          const uint2 h2 = __builtin_bit_cast(uint2, hi);
          vf[st] = __builtin_bit_cast(bf16x8, make_uint4(l2.x, l2.y, h2.x, h2.y));
        }
#pragma unroll
        for (int st = 0; st < 4; ++st)
          acc_o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[st], pb16[st >> 1][st & 1],
                                                              acc_o[db], 0, 0, 0);
      }
    }
    if (more) LOGO_STORE_TILE(stage ^ 1);
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

#undef LOGO_ROW
#undef LOGO_LOAD_TILE
#undef LOGO_STORE_TILE

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
