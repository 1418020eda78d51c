// bf16 backward of both attention branches on CDNA4 matrix cores.
//
// With the selection S held fixed, one softmax-attention row (query q, keys
// k_j and values v_j of its range R, upstream gradient e) contributes
//   p_j  = exp(scale <q, k_j> - lse)             (lse saved by the forward)
//   dv_j += p_j e
//   ds_j  = p_j (<e, v_j> - Dr),  Dr = <e, o_row> (the row prep kernel)
//   dq   += scale sum_j ds_j k_j
//   dk_j += scale ds_j q
// Local rows: e = do_i over L(i) = [max(0, i-W+1), i] ("Local-global
// attention", attention-mask sketch). Selected rows: e = g_i do_i over
// G(i) = [0, i] ("Learning When to Attend", "The Architecture of
// Conditional Attention"; LoGo abstract for the gate).
//
// Two kernels, both on v_mfma_f32_32x32x16_bf16 (A: lane l holds row l%32,
// k = (l/32)*8 + [0,8); B: column l%32, same k; C: column l%32, rows
// (e/4)*8 + (l/32)*4 + e%4 for element e):
//
// bwd_dkdv_kernel: key-stationary. A workgroup owns 128 keys of one
//   (b, kv head) and streams 32-row query tiles through LDS: for each query
//   head of the group, the selected rows at or after its first key, then
//   the local rows that read its keys. Its eight waves form four pairs of
//   32 keys with two roles, one wave of each role per SIMD:
//     producer (K, V rows of its keys in registers as A operands):
//       S^T [32 keys x 32 q] = K Q^T,  dP^T = V dO^T   (B = Q, dO rows)
//       P = exp2(S scale log2e - lse log2e), dS = P (dP - Dr)
//       and hands P, dS over through LDS as bf16 [32 q x 32 keys] tiles;
//     consumer (the dK^T, dV^T accumulators):
//       dV^T [d x keys] += dO^T P,  dK^T [d x keys] += Q^T dS
//       with dO^T, Q^T, P and dS all read by the gfx950 transposing LDS read
//       (ds_read_b64_tr_b16), and issues the workgroup's tile loads.
//   While one wave of a SIMD runs its elementwise work the other's matrix
//   products keep the matrix core busy; one wave alone per SIMD leaves it
//   idle whenever that wave is not issuing products.
//
// bwd_dq_kernel: query-stationary, like the forward: 32 rows per wave with
//   Q and dO rows in registers, K/V tiles of 64 keys through LDS:
//     S^T = K Q^T, dP^T = V dO^T, dS^T = P^T (dP^T - Dr), dQ^T += K^T dS^T.
//   The local launch writes dq for every row; the global launch then adds
//   the selected rows' global part in place (same stream, so ordered).
#include "logo_internal.h"

#include <type_traits>

namespace logo {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16* lds_v4i16_ptr;

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kNumXcd = 8;
constexpr float kLog2e = 1.4426950408889634f;
constexpr int kWaitVm0 = 0x0F70;  // s_waitcnt vmcnt(0), other counters untouched
constexpr uint32_t kPadOff = 0x40000000u;

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  bf16x2 r = __builtin_convertvector((f32x2){a, b}, bf16x2);
  return __builtin_bit_cast(uint32_t, r);
}

__device__ __forceinline__ bf16x8 ld16(const uint16_t* p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(p));
}

// XOR swizzle of a d = 128 tile's 16-byte chunks by the row's low four bits:
// logical chunk c of row r sits in slot c ^ swz16(r). Both the 16-byte row
// reads (16 rows, one chunk) and the transposing reads (4 rows, 4 chunks)
// then cover all 64 banks once; a whole 16-row group shares the pattern.
__device__ __forceinline__ int swz16(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }

// Lane l of instruction j fills LDS slot j*64 + l of a tile whose rows are
// `chunks` 16-byte slots long (the last ones padding). Returns the byte
// offset of that slot's source within a row block of row stride `st2`
// bytes, or an out-of-range offset (reads zero) for padding slots.
__device__ __forceinline__ uint32_t slot_off(int slot, int chunks, int dchunks, int st2) {
  const int row = slot / chunks, c = slot % chunks;
  return c < dchunks ? (uint32_t)(row * st2 + c * 16) : kPadOff;
}

// Issues this wave's share (instructions j = wave, wave+4, ...) of the
// buffer-load-to-LDS instructions that fill a tile of `rows` rows.
// Source: bytes [base, base + nbytes), row r of the tile at byte
// soff + r * st2. Rows past the end read zero (hardware bounds check).
template <int NCH, int CHUNKS, int DCH, bool SWZ = false>
__device__ __forceinline__ void issue_rows(const uint16_t* base, int nbytes, uint16_t* dst,
                                           int soff, int st2, int wave, int lane) {
  typedef __attribute__((address_space(3))) void* lds_ptr;
  const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(base), (short)0, nbytes, 0x00020000);
#pragma unroll
  for (int i = 0; i < (NCH + kWaves - 1) / kWaves; ++i) {
    const int j = wave + kWaves * i;
    // (wave < kWaves: with NCH a multiple of kWaves every wave issues all)
    if (NCH % kWaves == 0 || j < NCH) {
      // SWZ: slot (row, pc) takes the row's logical chunk pc ^ swz16(row)
      // (unpadded rows)
      const int slot = j * 64 + lane, row = slot / CHUNKS, pc = slot % CHUNKS;
      const uint32_t voff = SWZ ? (uint32_t)(row * st2 + ((pc ^ swz16(row)) << 4))
                                : slot_off(slot, CHUNKS, DCH, st2);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_ptr)(dst + j * 512), 16, voff, soff,
                                               0, 0);
    }
  }
}

// Row-load instructions j = part, part + 2, ... (< NQ) of a tile: lane l
// of instruction j fills LDS slot j*64 + l from byte (glb ? voff_g : voff_l)[i]
// + soff of [base, base + nbytes) (out of range: zero). The buffer resource
// is built here, in a device function: its type must not reach the host pass.
template <int NQ, int NI>
__device__ __forceinline__ void issue_part(const uint16_t* base, int nbytes, uint16_t* dst,
                                           const uint32_t (&voff_g)[NI],
                                           const uint32_t (&voff_l)[NI], bool glb, int soff,
                                           int part) {
  typedef __attribute__((address_space(3))) void* lds_ptr;
  const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(base), (short)0, nbytes, 0x00020000);
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    if (part + 2 * i < NQ) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_ptr)(dst + (part + 2 * i) * 512), 16,
                                               glb ? voff_g[i] : voff_l[i], soff, 0, 0);
    }
  }
}

// =========================================================================
// dK / dV
// =========================================================================
constexpr int kQT = 32;    // query rows per tile
constexpr int kKW = 32;    // keys per wave pair
constexpr int kPairs = 4;  // wave pairs per workgroup
constexpr int kKB = kKW * kPairs;  // keys per workgroup
constexpr int kDkdvThreads = 2 * kPairs * 64;

// Q and dO tiles are read two ways: rows as 16-byte operands (producer) and
// 4 rows x 8 bytes at a time by the transposing read (consumer). d = 128:
// unpadded rows whose logical 16-byte chunk c of row r sits in slot
// c ^ swz(r), which spreads both kinds of read over all 64 banks. d = 64:
// 32 B of padding per row (two-way conflicts on both kinds).
template <int D>
struct QTile {
  static constexpr bool kSwz = D == 128;
  static constexpr int kChunks = kSwz ? D / 8 : D / 8 + 2;
  static constexpr int kStride = kChunks * 8;  // elements
  static constexpr int kElems = kQT * kStride;
  static constexpr int kInstr = kQT * kChunks / 64;
  static_assert(kQT * kChunks % 64 == 0, "tile must be whole instructions");
  // depends on r's low four bits only, so whole 16-row groups share it
  __device__ static int swz(int r) { return kSwz ? swz16(r) : 0; }
  // source byte offset (row stride st2 bytes) of LDS slot `slot` of a tile;
  // pad slots read an out-of-range offset (zero)
  __device__ static uint32_t slot_src(int slot, int st2) {
    const int row = slot / kChunks, pc = slot % kChunks;
    return pc < D / 8 ? (uint32_t)(row * st2 + ((pc ^ swz(row)) << 4)) : kPadOff;
  }
};

struct DkdvParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* dout;
  const uint16_t* qs;   // [B][Hq][k][D]
  const uint16_t* dog;  // [B][Hq][k][D]
  const int32_t* idx;
  const float* L2_l;   // lse * log2(e), [B][Hq][n]
  const float* L2_g;   // [B][Hq][k]
  const float* D_l;
  const float* D_g;
  float* dk;
  float* dv;
  int B, Hq, Hkv, n, W, ksel;
  float scale_log2;
  float scale;
  int nkb;       // key blocks per (b, kv head)
  int total_wg;  // B * Hkv * nkb
  int per_xcd;
  View vq, vk, vv, vo;
};

// Per-tile row data (lse, Dr, positions) also arrive by buffer loads into
// LDS: one instruction per array, lanes 0..7 carry the 32 values and the
// others read out of range (zeros), so each array gets a 1 KiB landing slot.
constexpr int kSlot = 256;  // floats per landing slot

// P and dS of one tile, handed from producer to consumer waves: per wave
// pair a [32 query rows][32 keys] bf16 tile of each, rows of 64 bytes whose
// 8-byte chunks are XOR-swizzled by (row / 4) % 8, so the producers' row
// writes and the consumers' transposing reads both cover the banks once.
constexpr int kPsPair = 2 * kQT * kKW;      // P then dS (elements)
constexpr int kPsElems = kPairs * kPsPair;

__device__ __forceinline__ int ps_off(int row, int chunk) {
  return row * kKW + ((chunk ^ ((row >> 2) & 7)) << 2);
}

// The B operand of a dV / dK product from a P or dS tile: key column l % 32,
// rows r0 + {half*4 + [0,4)} and r0 + 8 + {half*4 + [0,4)}, the order of
// the A operand that read_tr gives for the same rows.
__device__ __forceinline__ bf16x8 read_tr_ps(const uint16_t* tile, int r0, int lane) {
  const int rl = r0 + (lane >> 5) * 4 + ((lane & 15) >> 2);
  const int chunk = ((lane >> 4) & 1) * 4 + (lane & 3);
  const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_ptr)(tile + ps_off(rl, chunk)));
  const v4i16 hi =
      __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_ptr)(tile + ps_off(rl + 8, chunk)));
  const uint2 l2 = __builtin_bit_cast(uint2, lo);
  const uint2 h2 = __builtin_bit_cast(uint2, hi);
  return __builtin_bit_cast(bf16x8, make_uint4(l2.x, l2.y, h2.x, h2.y));
}

// 32 consecutive 4-byte values from byte soff of [src, src + nbytes) into
// dst[0..32) (values past nbytes read zero); the rest of the slot gets zeros.
// The buffer resource is built here: its type is device-only and must not
// appear where the host pass compiles a kernel's lambdas.
__device__ __forceinline__ void issue_row_data(const void* src, int nbytes, float* dst, int soff,
                                               int lane) {
  typedef __attribute__((address_space(3))) void* lds_ptr;
  const __amdgpu_buffer_rsrc_t rsrc =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(src), (short)0, nbytes, 0x00020000);
  const uint32_t voff = lane < kQT / 4 ? (uint32_t)lane * 16 : kPadOff;
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_ptr)dst, 16, voff, soff, 0, 0);
}

// Wave pair w owns keys j0 + 32w ... j0 + 32w + 31: producer wave w,
// consumer wave 4 + w. Step u: producers work on tile u, consumers on tile
// u-1 and issue the loads of tile u+1; one barrier per step.
template <int D>
__global__ __launch_bounds__(kDkdvThreads, 1) void bwd_dkdv_kernel(DkdvParams p) {
  using QT = QTile<D>;
  constexpr int QS = D / 16;  // k-steps along d
  constexpr int DB = D / 32;  // 32-wide d blocks
  constexpr int DCH = D / 8;
  constexpr int NQ = QT::kInstr;
  // Three of each buffer (tile u read by producers, u-1 by consumers, u+1
  // landing), each a distinct LDS object so the compiler can tell reads of
  // one from buffer loads still landing in another.
  __shared__ __attribute__((aligned(16))) uint16_t Q0[QT::kElems];
  __shared__ __attribute__((aligned(16))) uint16_t Q1[QT::kElems];
  __shared__ __attribute__((aligned(16))) uint16_t Q2[QT::kElems];
  __shared__ __attribute__((aligned(16))) uint16_t O0[QT::kElems];
  __shared__ __attribute__((aligned(16))) uint16_t O1[QT::kElems];
  __shared__ __attribute__((aligned(16))) uint16_t O2[QT::kElems];
  __shared__ __attribute__((aligned(16))) float R0[3 * kSlot];  // lse | Dr | pos
  __shared__ __attribute__((aligned(16))) float R1[3 * kSlot];
  __shared__ __attribute__((aligned(16))) float R2[3 * kSlot];
  __shared__ __attribute__((aligned(16))) uint16_t PS0[kPsElems];
  __shared__ __attribute__((aligned(16))) uint16_t PS1[kPsElems];
  __shared__ __attribute__((aligned(16))) uint16_t PS2[kPsElems];

  const int bid = blockIdx.x;
  const int L = (bid % kNumXcd) * p.per_xcd + bid / kNumXcd;
  if (L >= p.total_wg) return;
  const int unit = L / p.nkb;      // b * Hkv + kv head
  const int kb = L % p.nkb;        // key blocks of a unit run in order: most work first
  const int b = unit / p.Hkv;
  const int hk = unit % p.Hkv;
  const int G = p.Hq / p.Hkv;
  const int j0 = kb * kKB;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar registers
  const bool producer = wave < kPairs;
  const int pw = wave & (kPairs - 1);  // wave pair
  const int lane = tid & 63;
  const int col = lane & 31;
  const int half = lane >> 5;
  const int key0 = j0 + pw * kKW;  // first key of the wave pair
  const int key = key0 + col;

  // Query tiles: selected rows at or after j0 (T_glb tiles per head of the
  // group), then per head T_loc local tiles (rows j0 ..., every row whose
  // window reaches a key of the block).
  const int i_last = min(p.n - 1, j0 + kKB - 1 + p.W - 1);
  const int T_loc = (i_last - j0) / kQT + 1;
  const int* idx_b = p.idx + (size_t)b * p.ksel;
  int r_start = 0;
  {
    int lo = 0, hi = p.ksel;  // first r with idx_b[r] >= j0
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (idx_b[mid] < j0) lo = mid + 1;
      else hi = mid;
    }
    r_start = __builtin_amdgcn_readfirstlane(lo);
  }
  // Selected-row tiles lie on one grid of 32-row blocks shared by every
  // workgroup of the (b, kv head) and run from the last block backwards,
  // heads innermost: the workgroups of an XCD then read the same tile at
  // about the same time (a unit's gathered rows are larger than one XCD's
  // L2). Rows of the first block before r_start sit before j0: P = 0 there.
  const int rb0 = r_start / kQT;
  const int T_glb = r_start < p.ksel ? (p.ksel + kQT - 1) / kQT - rb0 : 0;
  const int T_gs = G * T_glb;  // selected-row tiles come first
  const int T = T_gs + G * T_loc;

  // Tile loads, issued by the consumer waves (cw = 0..3) one tile per step
  // in tile order. Wave cw loads half the row loads of one matrix (Q for
  // cw 0, 1, dO for cw 2, 3: instructions j = cw % 2, cw % 2 + 2, ...) and
  // one row-data array (lse: cw 1, positions: cw 2, Dr: cw 3). Everything
  // that does not change from tile to tile is set up here once; a cursor
  // walks the tiles (selected-row tiles first, heads innermost, then each
  // head's local tiles) without divisions.
  const int cw = wave - kPairs;
  const bool mat_o = cw >= 2;   // dO rather than Q
  const int part = cw & 1;
  constexpr int NI = (NQ + 1) / 2;  // row-load instructions per wave (at most)
  const View& mv = mat_o ? p.vo : p.vq;
  const uint16_t* lsrc = (mat_o ? p.dout : p.q) + b * mv.sb + (long long)hk * G * mv.sh;
  const long long lhead = mv.sh;                        // elements per head
  const int lbytes = ((p.n - 1) * mv.st + D) * 2;
  const int lst2 = mv.st * 2;
  const long long ghead = (long long)p.ksel * D;
  const uint16_t* gsrc = (mat_o ? p.dog : p.qs) + ((long long)b * p.Hq + hk * G) * ghead;
  const int gbytes = p.ksel * D * 2;
  uint32_t voff_l[NI], voff_g[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int slot = (part + 2 * i) * 64 + lane;
    voff_l[i] = QT::slot_src(slot, lst2);
    voff_g[i] = QT::slot_src(slot, D * 2);
  }
  const float* row_l = (cw == 1 ? p.L2_l : p.D_l) + ((long long)b * p.Hq + hk * G) * p.n;
  const float* row_g = (cw == 1 ? p.L2_g : p.D_g) + ((long long)b * p.Hq + hk * G) * p.ksel;
  struct Cursor {
    int h;     // head within the group
    int r0;    // first row (position, or index into the selected rows)
    int left;  // tiles left in this head's run (local) or this row block (selected)
    bool glb;
  };
  Cursor cur;
  cur.glb = T_gs > 0;
  cur.h = 0;
  cur.r0 = cur.glb ? (rb0 + T_glb - 1) * kQT : j0;
  cur.left = cur.glb ? G : T_loc;
  int glb_blocks = T_glb;  // selected-row blocks not yet finished
  auto advance = [&] __device__ () __attribute__((always_inline)) {
    if (cur.glb) {
      ++cur.h;
      if (--cur.left == 0) {
        cur.h = 0;
        cur.left = G;
        cur.r0 -= kQT;
        if (--glb_blocks == 0) {
          cur.glb = false;
          cur.r0 = j0;
          cur.left = T_loc;
        }
      }
    } else {
      cur.r0 += kQT;
      if (--cur.left == 0) {
        ++cur.h;
        cur.r0 = j0;
        cur.left = T_loc;
      }
    }
  };
  auto issue = [&] __device__ (uint16_t* qdst, uint16_t* odst, float* rdst)
      __attribute__((always_inline)) {
    {
      const uint16_t* src = cur.glb ? gsrc + cur.h * ghead : lsrc + cur.h * lhead;
      issue_part<NQ, NI>(src, cur.glb ? gbytes : lbytes, mat_o ? odst : qdst,
                         voff_g, voff_l, cur.glb, cur.r0 * (cur.glb ? D * 2 : lst2), part);
    }
    if (cw == 2) {
      // positions: the selected rows' from idx, a local tile's written here
      if (cur.glb) {
        issue_row_data(idx_b, p.ksel * 4, rdst + 2 * kSlot, cur.r0 * 4, lane);
      } else if (lane < kQT) {
        reinterpret_cast<int*>(rdst)[2 * kSlot + lane] = cur.r0 + lane;
      }
    } else if (cw != 0) {
      const float* src = cur.glb ? row_g + cur.h * p.ksel : row_l + cur.h * (long long)p.n;
      issue_row_data(src, (cur.glb ? p.ksel : p.n) * 4, rdst + (cw == 1 ? 0 : kSlot),
                     cur.r0 * 4, lane);
    }
    advance();
  };

  // Element offsets of this lane's tile reads: the producer's operand of
  // k-step s (row col, logical chunk 2s + half), the consumer's transposing
  // reads of d block db, rows half*4 + (lane & 15)/4 and 8 more (the second
  // 16-row half adds 16 rows: same swizzle).
  int poff[QS], toff_lo[DB], toff_hi[DB];
#pragma unroll
  for (int s = 0; s < QS; ++s) poff[s] = col * QT::kStride + (((2 * s + half) ^ QT::swz(col)) << 3);
  {
    const int rl = half * 4 + ((lane & 15) >> 2), rh = rl + 8;
    const int tr_col = ((lane >> 4) & 1) * 16 + (lane & 3) * 4;
    const int cc = tr_col >> 3, within = tr_col & 7;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      toff_lo[db] = rl * QT::kStride + (((db * 4 + cc) ^ QT::swz(rl)) << 3) + within;
      toff_hi[db] = rh * QT::kStride + (((db * 4 + cc) ^ QT::swz(rh)) << 3) + within;
    }
  }
  auto read_qt = [&] __device__ (const uint16_t* tile, int hh, int db)
      __attribute__((always_inline)) {
    const uint16_t* g0 = tile + hh * 16 * QT::kStride;
    const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_ptr)(g0 + toff_lo[db]));
    const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_ptr)(g0 + toff_hi[db]));
    const uint2 l2 = __builtin_bit_cast(uint2, lo);
    const uint2 h2 = __builtin_bit_cast(uint2, hi);
    return __builtin_bit_cast(bf16x8, make_uint4(l2.x, l2.y, h2.x, h2.y));
  };

  // Whether some row of tile t reads some key of this wave pair: row pos
  // reads key j iff 0 <= pos - j < wlim, so some j of [key0, key0 + 31] iff
  // 0 <= pos - key0 < wlim + 31. Both waves of the pair skip a tile none of
  // whose rows does (its P and dS are zero). Rows past the end of the list
  // read zero Q and dO rows and add exactly zero either way.
  auto pair_live = [&] __device__ (int t, const float* rc) __attribute__((always_inline)) {
    const uint32_t wlim = t < T_gs ? 0x80000000u : (uint32_t)p.W;
    const int pos = reinterpret_cast<const int*>(rc)[2 * kSlot + col];
    return __builtin_amdgcn_ballot_w64((uint32_t)(pos - key0) < wlim + 31u) != 0;
  };

  bf16x8 kreg[QS], vreg[QS];  // producer: K and V rows of the lane's key
  f32x16 acc_dk[DB], acc_dv[DB];  // consumer: dK^T, dV^T

  // Producer work for tile t: S^T = K Q^T and dP^T = V dO^T (a lane holds
  // one query row, l % 32, and 16 keys), then per element
  // P = exp2(S scale log2e - lse log2e) on the key's range (0 elsewhere)
  // and dS = P (dP - Dr), packed to bf16 and handed over.
  auto produce = [&] __device__ (int t, const uint16_t* qc, const uint16_t* oc, const float* rc,
                                 uint16_t* ps) __attribute__((always_inline)) {
    if (!pair_live(t, rc)) return;
    // key j is read by row pos iff 0 <= pos - j < wlim (window, or any
    // earlier key for selected rows). Rows past the end of the tile's list
    // have zero Q / dO rows and zero row terms, so they add exactly zero.
    const uint32_t wlim = t < T_gs ? 0x80000000u : (uint32_t)p.W;
    f32x16 s_acc = (f32x16){}, p_acc = (f32x16){};
#pragma unroll
    for (int s = 0; s < QS; ++s) {
      s_acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kreg[s], ld16(qc + poff[s]), s_acc, 0, 0,
                                                      0);
      p_acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vreg[s], ld16(oc + poff[s]), p_acc, 0, 0,
                                                      0);
    }
    const float l2 = rc[col];
    const float dr = rc[kSlot + col];
    const int pos = reinterpret_cast<const int*>(rc)[2 * kSlot + col];
    // element e is key kw0 + (e/4)*8 + half*4 + e%4
    const int rel = pos - (key0 + half * 4);
    // Rows are in ascending position (row 0, lane 0's, first; rows past the
    // end of the list read zero everywhere and add zero whatever P is): when
    // row 0 already reads every key of the pair, and for local rows the
    // last row still does, no element needs the range test.
    const int pos0 = __builtin_amdgcn_readfirstlane(pos);
    const bool all_in = pos0 >= key0 + kKW - 1 &&
                        (t < T_gs || pos0 + kQT - 1 - key0 < p.W);
    uint16_t* pt = ps + pw * kPsPair;
    auto body = [&] __device__ (auto masked) __attribute__((always_inline)) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float pv[4], dsv[4];
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const int e = j * 4 + w;
          const float x = __builtin_amdgcn_exp2f(fmaf(s_acc[e], p.scale_log2, -l2));
          if (decltype(masked)::value) {
            const bool ok = (uint32_t)(rel - (j * 8 + w)) < wlim;
            pv[w] = ok ? x : 0.0f;
          } else {
            pv[w] = x;
          }
          dsv[w] = pv[w] * (p_acc[e] - dr);
        }
        const int off = ps_off(col, 2 * j + half);
        *reinterpret_cast<uint2*>(pt + off) =
            make_uint2(pack_bf16x2(pv[0], pv[1]), pack_bf16x2(pv[2], pv[3]));
        *reinterpret_cast<uint2*>(pt + kQT * kKW + off) =
            make_uint2(pack_bf16x2(dsv[0], dsv[1]), pack_bf16x2(dsv[2], dsv[3]));
      }
    };
    if (all_in) {
      body(std::integral_constant<bool, false>());
    } else {
      body(std::integral_constant<bool, true>());
    }
  };

  // Consumer work for a tile: dV^T += dO^T P and dK^T += Q^T dS, contraction
  // rows 0..15 then 16..31.
  auto consume = [&] __device__ (int t, const uint16_t* qc, const uint16_t* oc, const float* rc,
                                 const uint16_t* ps) __attribute__((always_inline)) {
    if (!pair_live(t, rc)) return;
    const uint16_t* pt = ps + pw * kPsPair;
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const bf16x8 pb = read_tr_ps(pt, hh * 16, lane);
      const bf16x8 sb = read_tr_ps(pt + kQT * kKW, hh * 16, lane);
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        acc_dv[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(read_qt(oc, hh, db), pb,
                                                              acc_dv[db], 0, 0, 0);
        acc_dk[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(read_qt(qc, hh, db), sb,
                                                              acc_dk[db], 0, 0, 0);
      }
    }
  };

  // Step u: producers work on tile u, consumers on tile u-1 and issue the
  // loads of tile u+1; buffers named at compile time, three steps per trip.
  // Each role runs its own loop (so the allocator gives the producer's K, V
  // operands and the consumer's accumulators the same registers); both
  // loops pass the same barriers: one before the first step, one per step.
  if (producer) {
    // K and V rows of this lane's key: A operands for the whole kernel.
    const int kk = min(key, p.n - 1);
    const uint16_t* kr = p.k + b * p.vk.sb + hk * p.vk.sh + (long long)kk * p.vk.st + half * 8;
    const uint16_t* vr = p.v + b * p.vv.sb + hk * p.vv.sh + (long long)kk * p.vv.st + half * 8;
#pragma unroll
    for (int s = 0; s < QS; ++s) {
      kreg[s] = ld16(kr + s * 16);
      vreg[s] = ld16(vr + s * 16);
    }
    __syncthreads();
#pragma unroll 1
    for (int u = 0; u <= T; u += 3) {
      if (u < T) produce(u, Q0, O0, R0, PS0);
      __syncthreads();
      if (u + 1 <= T) {
        if (u + 1 < T) produce(u + 1, Q1, O1, R1, PS1);
        __syncthreads();
      }
      if (u + 2 <= T) {
        if (u + 2 < T) produce(u + 2, Q2, O2, R2, PS2);
        __syncthreads();
      }
    }
    return;
  }

#pragma unroll
  for (int i = 0; i < DB; ++i) {
    acc_dk[i] = (f32x16){};
    acc_dv[i] = (f32x16){};
  }
  auto cstep = [&] __device__ (int u, const uint16_t* qp, const uint16_t* op, const float* rp,
                               const uint16_t* psr, uint16_t* qn, uint16_t* on, float* rn)
      __attribute__((always_inline)) {
    if (u + 1 < T) issue(qn, on, rn);
    if (u >= 1) consume(u - 1, qp, op, rp, psr);
    __builtin_amdgcn_s_waitcnt(kWaitVm0);
    __syncthreads();
  };
  issue(Q0, O0, R0);
  __builtin_amdgcn_s_waitcnt(kWaitVm0);
  __syncthreads();
#pragma unroll 1
  for (int u = 0; u <= T; u += 3) {
    cstep(u, Q2, O2, R2, PS2, Q1, O1, R1);
    if (u + 1 <= T) cstep(u + 1, Q0, O0, R0, PS0, Q2, O2, R2);
    if (u + 2 <= T) cstep(u + 2, Q1, O1, R1, PS1, Q0, O0, R0);
  }

  if (key >= p.n) return;
  float* dkr = p.dk + (((long long)b * p.Hkv + hk) * p.n + key) * D;
  float* dvr = p.dv + (((long long)b * p.Hkv + hk) * p.n + key) * D;
#pragma unroll
  for (int db = 0; db < DB; ++db) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int d0 = db * 32 + j * 8 + half * 4;
      *reinterpret_cast<float4*>(dkr + d0) =
          make_float4(acc_dk[db][j * 4] * p.scale, acc_dk[db][j * 4 + 1] * p.scale,
                      acc_dk[db][j * 4 + 2] * p.scale, acc_dk[db][j * 4 + 3] * p.scale);
      *reinterpret_cast<float4*>(dvr + d0) =
          make_float4(acc_dv[db][j * 4], acc_dv[db][j * 4 + 1], acc_dv[db][j * 4 + 2],
                      acc_dv[db][j * 4 + 3]);
    }
  }
}
// =========================================================================
// dQ
// =========================================================================
constexpr int kRows = 32;  // query rows per wave
constexpr int kKeys = 64;  // keys per tile

template <int D>
struct KVTile {
  // K rows are read both as 16-byte operands and transposed. d = 128:
  // unpadded rows, logical 16-byte chunk c of row r in slot c ^ swz(r), which
  // spreads both kinds of read over all 64 banks; d = 64: 32 B of pad
  // (conflict-free transposing reads). V rows only as 16-byte operands: 16 B.
  static constexpr bool kSwz = D == 128;
  static constexpr int kChunks = kSwz ? D / 8 : D / 8 + 2;
  static constexpr int vChunks = D / 8 + 1;
  // depends on r's low four bits only, so whole 16-row groups share it
  __device__ static int swz(int r) { return kSwz ? swz16(r) : 0; }
  static constexpr int kStride = kChunks * 8;
  static constexpr int vStride = vChunks * 8;
  static constexpr int kElems = kKeys * kStride;
  static constexpr int vElems = kKeys * vStride;
  static constexpr int kInstr = kKeys * kChunks / 64;
  static constexpr int vInstr = kKeys * vChunks / 64;
};

struct DqParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* dout;
  const uint16_t* qs;
  const uint16_t* dog;
  const int32_t* idx;
  const float* lse;   // local [B][Hq][n] or global [B][Hq][k]
  const float* Dr;    // same shape as lse
  float* dq;
  int B, Hq, Hkv, n, W, ksel;
  float scale_log2;
  float scale;
  int units;
  int wg_per_unit;
  int total_wg;
  int per_xcd;
  View vq, vk, vv, vo;
};

template <int D, bool GLOBAL>
__global__ __launch_bounds__(kThreads, 2) void bwd_dq_kernel(DqParams p) {
  using KT = KVTile<D>;
  constexpr int QS = D / 16;
  constexpr int DB = D / 32;
  constexpr int DCH = D / 8;
  __shared__ __attribute__((aligned(16))) uint16_t K0[KT::kElems];
  __shared__ __attribute__((aligned(16))) uint16_t K1[KT::kElems];
  __shared__ __attribute__((aligned(16))) uint16_t V0[KT::vElems];
  __shared__ __attribute__((aligned(16))) uint16_t V1[KT::vElems];

  const int bid = blockIdx.x;
  const int L = (bid % kNumXcd) * p.per_xcd + bid / kNumXcd;
  if (L >= p.total_wg) return;
  const int unit_bh = L / p.wg_per_unit;
  int w = L % p.wg_per_unit;
  if (GLOBAL) w = p.wg_per_unit - 1 - w;  // longest prefix first
  const int b = unit_bh / p.Hkv;
  const int hk = unit_bh % p.Hkv;
  const int G = p.Hq / p.Hkv;
  const int R = GLOBAL ? p.ksel : p.n;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar registers
  const int lane = tid & 63;
  const int col = lane & 31;
  const int half = lane >> 5;

  const int u_first = w * kWaves;
  const int u_last = min(u_first + kWaves, p.units) - 1;
  const int u = u_first + wave;
  const bool wave_on = u < p.units;
  const int pb = (wave_on ? u : u_last) / G;
  const int h = hk * G + (wave_on ? u : u_last) % G;
  auto row_pos = [&] __device__ (int r) __attribute__((always_inline)) {
    return GLOBAL ? p.idx[(size_t)b * p.ksel + r] : r;
  };
  const int r_lane = pb * kRows + col;
  const bool row_ok = wave_on && r_lane < R;
  const int pos = r_lane < R ? row_pos(r_lane) : -1;
  const int wpos_lo = row_pos(pb * kRows);
  const int wpos_hi = row_pos(min(pb * kRows + kRows, R) - 1);
  const int wkey_lo = GLOBAL ? 0 : max(0, wpos_lo - p.W + 1);
  const int wkey_hi = wpos_hi;
  const int gpos_lo = row_pos((u_first / G) * kRows);
  const int gpos_hi = row_pos(min((u_last / G) * kRows + kRows, R) - 1);
  const int t_lo = (GLOBAL ? 0 : max(0, gpos_lo - p.W + 1)) / kKeys;
  const int t_hi = gpos_hi / kKeys;

  const long long hb = (long long)b * p.Hq + h;
  // Q and upstream-gradient rows of this lane's query: B operands.
  bf16x8 qreg[QS], oreg[QS];
  float lse2 = 0.0f, dr = 0.0f;
  {
    const int rr = row_ok ? r_lane : 0;
    const uint16_t* qr;
    const uint16_t* orr;
    if (GLOBAL) {
      qr = p.qs + (hb * p.ksel + rr) * D;
      orr = p.dog + (hb * p.ksel + rr) * D;
    } else {
      qr = p.q + b * p.vq.sb + h * p.vq.sh + (long long)rr * p.vq.st;
      orr = p.dout + b * p.vo.sb + h * p.vo.sh + (long long)rr * p.vo.st;
    }
#pragma unroll
    for (int s = 0; s < QS; ++s) {
      qreg[s] = ld16(qr + s * 16 + half * 8);
      oreg[s] = ld16(orr + s * 16 + half * 8);
    }
    lse2 = p.lse[hb * R + rr] * kLog2e;
    dr = p.Dr[hb * R + rr];
  }

  const int k_st2 = p.vk.st * 2, v_st2 = p.vv.st * 2;
  const uint16_t* const kg = p.k + b * p.vk.sb + hk * p.vk.sh;
  const uint16_t* const vg = p.v + b * p.vv.sb + hk * p.vv.sh;
  const int k_bytes = ((p.n - 1) * p.vk.st + D) * 2;
  const int v_bytes = ((p.n - 1) * p.vv.st + D) * 2;
  auto issue_kv = [&] __device__ (int t, uint16_t* kdst, uint16_t* vdst)
      __attribute__((always_inline)) {
    issue_rows<KT::kInstr, KT::kChunks, DCH, KT::kSwz>(kg, k_bytes, kdst, t * kKeys * k_st2,
                                                       k_st2, wave, lane);
    issue_rows<KT::vInstr, KT::vChunks, DCH>(vg, v_bytes, vdst, t * kKeys * v_st2, v_st2, wave,
                                             lane);
  };

  f32x16 acc[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i) acc[i] = (f32x16){};

  auto is_active = [&] __device__ (int t) __attribute__((always_inline)) {
    const int key0 = t * kKeys;
    return wave_on && key0 <= wkey_hi && key0 + kKeys - 1 >= wkey_lo;
  };

  // Element offsets of this lane's K tile reads: the operand of k-step s
  // (row col, logical chunk 2s + half) and the transposing reads of d block
  // db, rows half*4 + (lane & 15)/4 and 8 more; whole 16-row groups added
  // to either keep the swizzle.
  int koff[QS], toff_lo[DB], toff_hi[DB];
#pragma unroll
  for (int s = 0; s < QS; ++s) koff[s] = col * KT::kStride + (((2 * s + half) ^ KT::swz(col)) << 3);
  {
    const int rl = half * 4 + ((lane & 15) >> 2), rh = rl + 8;
    const int tr_col = ((lane >> 4) & 1) * 16 + (lane & 3) * 4;
    const int cc = tr_col >> 3, within = tr_col & 7;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      toff_lo[db] = rl * KT::kStride + (((db * 4 + cc) ^ KT::swz(rl)) << 3) + within;
      toff_hi[db] = rh * KT::kStride + (((db * 4 + cc) ^ KT::swz(rh)) << 3) + within;
    }
  }
  auto read_kt = [&] __device__ (const uint16_t* ks, int r0, int db)
      __attribute__((always_inline)) {
    const uint16_t* g0 = ks + r0 * KT::kStride;
    const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_ptr)(g0 + toff_lo[db]));
    const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_ptr)(g0 + toff_hi[db]));
    const uint2 l2 = __builtin_bit_cast(uint2, lo);
    const uint2 h2 = __builtin_bit_cast(uint2, hi);
    return __builtin_bit_cast(bf16x8, make_uint4(l2.x, l2.y, h2.x, h2.y));
  };

  auto tile = [&] __device__ (int t, const uint16_t* ks, const uint16_t* vs)
      __attribute__((always_inline)) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      // A 32-key block no row of the wave reads (past the last row's
      // position, or below the first row's window) adds exactly zero: skip.
      {
        const int kb0 = t * kKeys + kb * 32;
        if (kb0 > wkey_hi || kb0 + 31 < wkey_lo) continue;
      }
      f32x16 sacc = (f32x16){}, pacc = (f32x16){};
      const uint16_t* kblk = ks + kb * 32 * KT::kStride;
      const uint16_t* vrow = vs + (kb * 32 + col) * KT::vStride + half * 8;
#pragma unroll
      for (int s = 0; s < QS; ++s) {
        sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ld16(kblk + koff[s]), qreg[s], sacc, 0, 0,
                                                       0);
        pacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ld16(vrow + s * 16), oreg[s], pacc, 0, 0,
                                                       0);
      }
      uint32_t dk2[8];
      const int key0 = t * kKeys + kb * 32;
      // Every row of the wave reads every key of the block: no range test
      // (rows past the end compute garbage only for their own dq row, which
      // is never stored).
      const bool all_in = wpos_lo >= key0 + 31 && (GLOBAL || key0 >= wpos_hi - p.W + 1);
      if (all_in) {
#pragma unroll
        for (int e2 = 0; e2 < 8; ++e2) {
          float ds[2];
#pragma unroll
          for (int i = 0; i < 2; ++i) {
            const int e = 2 * e2 + i;
            ds[i] = __builtin_amdgcn_exp2f(fmaf(sacc[e], p.scale_log2, -lse2)) * (pacc[e] - dr);
          }
          dk2[e2] = pack_bf16x2(ds[0], ds[1]);
        }
      } else {
#pragma unroll
        for (int e2 = 0; e2 < 8; ++e2) {
          float ds[2];
#pragma unroll
          for (int i = 0; i < 2; ++i) {
            const int e = 2 * e2 + i;
            const int key = key0 + (e >> 2) * 8 + half * 4 + (e & 3);
            bool ok = row_ok && key <= pos;
            if (!GLOBAL) ok = ok && key >= pos - p.W + 1;
            const float pr =
                ok ? __builtin_amdgcn_exp2f(fmaf(sacc[e], p.scale_log2, -lse2)) : 0.0f;
            ds[i] = pr * (pacc[e] - dr);
          }
          dk2[e2] = pack_bf16x2(ds[0], ds[1]);
        }
      }
#pragma unroll
      for (int db = 0; db < DB; ++db) {
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const bf16x8 sb = __builtin_bit_cast(
              bf16x8, make_uint4(dk2[4 * hh], dk2[4 * hh + 1], dk2[4 * hh + 2], dk2[4 * hh + 3]));
          acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(read_kt(ks, kb * 32 + hh * 16, db),
                                                            sb, acc[db], 0, 0, 0);
        }
      }
    }
  };

  auto step = [&] __device__ (int t, const uint16_t* ks, const uint16_t* vs, uint16_t* kn,
                              uint16_t* vn) __attribute__((always_inline)) {
    if (t + 1 <= t_hi) issue_kv(t + 1, kn, vn);
    if (__builtin_amdgcn_readfirstlane(is_active(t))) tile(t, ks, vs);
    __builtin_amdgcn_s_waitcnt(kWaitVm0);
    __syncthreads();
  };

  {
    issue_kv(t_lo, K0, V0);
    __builtin_amdgcn_s_waitcnt(kWaitVm0);
    __syncthreads();
  }
#pragma unroll 1
  for (int t = t_lo; t <= t_hi; t += 2) {
    step(t, K0, V0, K1, V1);
    if (t + 1 <= t_hi) step(t + 1, K1, V1, K0, V0);
  }

  if (!row_ok) return;
  float* dqr = p.dq + (hb * p.n + pos) * D;
#pragma unroll
  for (int db = 0; db < DB; ++db) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int d0 = db * 32 + j * 8 + half * 4;
      float4 v4 = make_float4(acc[db][j * 4] * p.scale, acc[db][j * 4 + 1] * p.scale,
                              acc[db][j * 4 + 2] * p.scale, acc[db][j * 4 + 3] * p.scale);
      float4* dst = reinterpret_cast<float4*>(dqr + d0);
      if (GLOBAL) {
        const float4 old = *dst;
        v4.x += old.x;
        v4.y += old.y;
        v4.z += old.z;
        v4.w += old.w;
      }
      *dst = v4;
    }
  }
}

template <int D>
hipError_t dkdv_t(const Dims& d, const BwdArgs& a, hipStream_t s) {
  DkdvParams p;
  p.q = static_cast<const uint16_t*>(a.q);
  p.k = static_cast<const uint16_t*>(a.k);
  p.v = static_cast<const uint16_t*>(a.v);
  p.dout = static_cast<const uint16_t*>(a.dout);
  p.qs = static_cast<const uint16_t*>(a.qs);
  p.dog = static_cast<const uint16_t*>(a.dog);
  p.idx = a.idx;
  p.L2_l = a.L2_l;
  p.L2_g = a.L2_g;
  p.D_l = a.D_l;
  p.D_g = a.D_g;
  p.dk = a.dk;
  p.dv = a.dv;
  p.B = d.B;
  p.Hq = d.Hq;
  p.Hkv = d.Hkv;
  p.n = d.n;
  p.W = d.window;
  p.ksel = d.k;
  p.scale = d.scale;
  p.scale_log2 = d.scale * kLog2e;
  p.nkb = (d.n + kKB - 1) / kKB;
  p.total_wg = d.B * d.Hkv * p.nkb;
  p.per_xcd = (p.total_wg + kNumXcd - 1) / kNumXcd;
  p.vq = d.vq;
  p.vk = d.vk;
  p.vv = d.vv;
  p.vo = d.vo;
  hipLaunchKernelGGL((bwd_dkdv_kernel<D>), dim3(p.per_xcd * kNumXcd), dim3(kDkdvThreads), 0,
                     s, p);
  return hipGetLastError();
}

template <int D, bool GLOBAL>
hipError_t dq_t(const Dims& d, const BwdArgs& a, hipStream_t s) {
  const int R = GLOBAL ? d.k : d.n;
  if (R == 0) return hipSuccess;
  DqParams p;
  p.q = static_cast<const uint16_t*>(a.q);
  p.k = static_cast<const uint16_t*>(a.k);
  p.v = static_cast<const uint16_t*>(a.v);
  p.dout = static_cast<const uint16_t*>(a.dout);
  p.qs = static_cast<const uint16_t*>(a.qs);
  p.dog = static_cast<const uint16_t*>(a.dog);
  p.idx = a.idx;
  p.lse = GLOBAL ? a.lse_g : a.lse_l;
  p.Dr = GLOBAL ? a.D_g : a.D_l;
  p.dq = a.dq;
  p.B = d.B;
  p.Hq = d.Hq;
  p.Hkv = d.Hkv;
  p.n = d.n;
  p.W = d.window;
  p.ksel = d.k;
  p.scale = d.scale;
  p.scale_log2 = d.scale * kLog2e;
  const int G = d.Hq / d.Hkv;
  p.units = (R + kRows - 1) / kRows * G;
  p.wg_per_unit = (p.units + kWaves - 1) / kWaves;
  p.total_wg = d.B * d.Hkv * p.wg_per_unit;
  p.per_xcd = (p.total_wg + kNumXcd - 1) / kNumXcd;
  p.vq = d.vq;
  p.vk = d.vk;
  p.vv = d.vv;
  p.vo = d.vo;
  hipLaunchKernelGGL((bwd_dq_kernel<D, GLOBAL>), dim3(p.per_xcd * kNumXcd), dim3(kThreads), 0,
                     s, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd_dkdv_bf16(const Dims& d, const BwdArgs& a, hipStream_t s) {
  if (d.B == 0 || d.n == 0) return hipSuccess;
  if (d.d == 64) return dkdv_t<64>(d, a, s);
  if (d.d == 128) return dkdv_t<128>(d, a, s);
  return hipErrorInvalidValue;
}

hipError_t launch_bwd_dq_bf16(const Dims& d, bool global, const BwdArgs& a, hipStream_t s) {
  if (d.B == 0 || d.n == 0) return hipSuccess;
  if (d.d == 64) return global ? dq_t<64, true>(d, a, s) : dq_t<64, false>(d, a, s);
  if (d.d == 128) return global ? dq_t<128, true>(d, a, s) : dq_t<128, false>(d, a, s);
  return hipErrorInvalidValue;
}

}  // namespace logo
