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
#include <algorithm>

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
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInit = -1.0e30f;
constexpr float kLazy = 8.0f;  // log2 headroom before the running max moves
// s_waitcnt immediate for vmcnt(0) with expcnt/lgkmcnt left alone (gfx9 encoding)
constexpr int kWaitVm0 = 0x0F70;

template <int D>
struct Smem {
  // Tiles are filled by bounds-checked buffer loads that write LDS
  // directly: one instruction moves 64 lanes x 16 B into 1 KiB of
  // consecutive LDS, so a tile of 64 rows is 64 x kChunks 16-byte slots and
  // kChunks instructions fill it.
  // d = 128: unpadded rows; logical chunk c of row r sits in slot c ^ swz(r)
  // of the row, which spreads both the 16-byte K operand reads (16 rows,
  // one chunk) and the transposing V reads (4 rows, 4 chunks, twice) over
  // all 64 banks. d = 64: padded rows (the swizzle measured slower there):
  // K rows carry 16 B of pad (16-byte operand reads conflict-free), V rows
  // 32 B; pad slots read an out-of-range offset (zero).
  static constexpr bool kSwz = D == 128;
  static constexpr int kChunks = kSwz ? D / 8 : D / 8 + 1;
  static constexpr int vChunks = kSwz ? D / 8 : D / 8 + 2;
  static constexpr int kStride = kChunks * 8;
  static constexpr int vStride = vChunks * 8;
  static constexpr int kElems = kKeys * kStride;
  static constexpr int vElems = kKeys * vStride;
  // depends on r's low four bits only, so whole 16-row groups share it
  __device__ static int swz(int r) { return kSwz ? ((r & 3) << 2) | ((r >> 2) & 3) : 0; }
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
  View vq, vk, vv, vo;  // element strides of q, k, v, o
  float* lse_out;       // optional per-row log-sum-exp (natural log)
  float* og_out;        // optional f32 o_global rows (fused global)
  const float* router_w;  // routed local: [Hq][D]
  float* router_part;     // routed local: [B][Hq][n]
  const int32_t* seg_start;  // packed examples: [n] first token of the example, or NULL
  const int32_t* sched_perm; // packed global: workgroup slots by work, heaviest first
                             // (NULL: the last row block first)
  int32_t* sched_count;      // global: per (b, kv head) next rank, zeroed before the
                             // launch; NULL: the static order
  int nsplit;                // fused global: key ranges per row block (1: none)
  float* part;               // nsplit > 1: partials [nsplit][B*Hq][ksel][D + 4]
                             // (unnormalised o, then max and sum)
};

__device__ __forceinline__ uint16_t f32_to_bf16_bits(float x) {
  bf16x2 r = __builtin_convertvector((f32x2){x, 0.0f}, bf16x2);
  return (uint16_t)(__builtin_bit_cast(uint32_t, r) & 0xffffu);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  bf16x2 r = __builtin_convertvector((f32x2){a, b}, bf16x2);
  return __builtin_bit_cast(uint32_t, r);
}

// Wave `wave` issues its share (instructions j = wave, wave+4, ...) of the
// NCH buffer-load-to-LDS instructions that fill one tile: lane l of
// instruction j moves 16 bytes from byte voff[i] + soff of the buffer
// [base, base + nbytes) to LDS byte 1024*j + 16*l of dst. Offsets at or past
// nbytes read as zero (hardware bounds check), so rows past the end of the
// sequence need no clamping. The buffer resource is built here: its type
// is device-only and must not appear where the host pass compiles the
// kernel's signature or lambdas.
template <int NJ, int NCH>
__device__ __forceinline__ void issue_tile(const uint16_t* base, int nbytes, uint16_t* dst,
                                           const uint32_t* voff, int soff, int wave) {
  typedef __attribute__((address_space(3))) void* lds_ptr;
  const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(base), (short)0, nbytes, 0x00020000);
#pragma unroll
  for (int i = 0; i < NJ; ++i) {
    const int j = wave + kWaves * i;
    // (wave < kWaves: with NCH a multiple of kWaves every wave issues NJ)
    if (NCH == NJ * kWaves || j < NCH)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_ptr)(dst + j * 512), 16, voff[i], soff,
                                               0, 0);
  }
}

// One row block of one (b, kv head): up to 4 units (32 rows x one query
// head each, one per wave) that share K/V tiles.
//
// EPI: 0 LocalAll, 1 LocalFused, 2 GlobalAll, 3 GlobalFused, 4 LocalRouted,
// 5 GlobalRouted (see Epi), and the two halves of the single-launch fused
// forward:
//   6 (global rows, gathered through idx): the selected rows' local branch
//     and global branch from one walk over their causal prefix. The walk
//     goes from the diagonal down to key 0 (SEG: to the first token of the
//     lowest example in the block). Keys inside a row's window
//     [i-W+1, i] come first, so after the tile holding the window's lowest
//     key the running output is that row's local output: it is normalised
//     and parked in the scratch rows (this lane's row only). The walk then
//     goes on over the keys below the window with the same running state,
//     which ends as the global output over [0, i]. A tile holding some
//     row's window edge is walked twice with complementary masks (window
//     keys, then the keys below it). Writes o = o_local + sigmoid(g) o_global.
//   7 (unselected rows, gathered through idx = the unselected positions,
//     ksel = their count): the local branch only; writes o.
// SEG: packed examples (p.seg_start set): keys before a row's example start
// are masked (in both of EPI 6's walks) and tile ranges start at the
// example; positions read from idx
// are clamped and ranks beyond the scratch rows ignored, so inconsistent
// example offsets cannot address outside the buffers. Compiled separately so
// the plain path carries none of it.
template <int D, bool GLOBAL, int EPI, bool SEG>
__device__ __forceinline__ void attn_block(const Params& p, int unit_bh, int w, int split,
                                           uint16_t* K0, uint16_t* K1, uint16_t* V0,
                                           uint16_t* V1) {
  using SM = Smem<D>;
  // rows come from a position list (idx) rather than being 0..n-1
  constexpr bool GATHER = GLOBAL || EPI == 7;
  // the walk goes from the diagonal down to key 0
  constexpr bool BACKWARD = EPI == 6;
  const int b = unit_bh / p.Hkv;
  const int hk = unit_bh % p.Hkv;
  const int G = p.Hq / p.Hkv;
  const int R = GATHER ? p.ksel : p.n;          // rows per (b, head)

  const int tid = threadIdx.x;
  // uniform in the wave: what derives from it (rows, heads, key ranges)
  // lives in scalar registers
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
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

  auto row_pos = [&] __device__ (int r) __attribute__((always_inline)) {
    if (!GATHER) return r;
    const int ix = p.idx[(size_t)b * p.ksel + r];
    return SEG ? min(max(ix, 0), p.n - 1) : ix;
  };
  // Row of this lane and the wave's / workgroup's key range.
  const int r_lane = pb * kRows + col;
  const bool row_ok = wave_on && r_lane < R;
  const int pos = r_lane < R ? row_pos(r_lane) : -1;
  const int wpos_lo = row_pos(pb * kRows);                 // rows ascend
  const int wpos_hi = row_pos(min(pb * kRows + kRows, R) - 1);
  // Packed examples: keys before a row's example start are not read; the
  // starts do not decrease along the rows.
  auto seg0 = [&] __device__ (int pos_) __attribute__((always_inline)) {
    return SEG ? p.seg_start[pos_] : 0;
  };
  const int ss = pos >= 0 ? seg0(pos) : 0;
  const int wss_lo = seg0(wpos_lo), wss_hi = seg0(wpos_hi);
  const int wkey_lo = GLOBAL ? wss_lo : max(wss_lo, wpos_lo - p.W + 1);
  const int wkey_hi = wpos_hi;
  const int gpos_lo = row_pos((u_first / G) * kRows);
  const int gpos_hi = row_pos(min((u_last / G) * kRows + kRows, R) - 1);
  const int gss_lo = seg0(gpos_lo);
  int t_lo = (GLOBAL ? gss_lo : max(gss_lo, gpos_lo - p.W + 1)) / kKeys;
  int t_hi = gpos_hi / kKeys;
  if (EPI == 3 && p.nsplit > 1) {
    // this workgroup's share of the block's key tiles (possibly none)
    const int per = (t_hi - t_lo + p.nsplit) / p.nsplit;
    t_lo += split * per;
    t_hi = min(t_hi, t_lo + per - 1);
  }
  // EPI 6: the lowest window key of this lane's row and the wave's range of
  // them (rows ascend, so the first and last rows bound it)
  const int lb = pos - p.W + 1;
  const int wlb_lo = wpos_lo - p.W + 1, wlb_hi = wpos_hi - p.W + 1;

  // This (b, kv head)'s K and V, read through bounds-checked buffer loads:
  // keys past the end read as zero (they only occur in tiles masked per
  // element, after every query of the tile).
  const int k_st = p.vk.st, v_st = p.vv.st;
  const int k_bytes = ((p.n - 1) * k_st + D) * 2;
  const int v_bytes = ((p.n - 1) * v_st + D) * 2;
  const uint16_t* const kg = p.k + b * p.vk.sb + hk * p.vk.sh;
  const uint16_t* const vg = p.v + b * p.vv.sb + hk * p.vv.sh;

  // ---- Q rows into registers -------------------------------------------
  constexpr int QS = D / 16;  // k-steps of 16 along d
  bf16x8 qreg[QS];
  {
    const bool ok = row_ok && pos >= 0;
    const uint16_t* qrow =
        p.q + b * p.vq.sb + h * p.vq.sh + (long long)(ok ? pos : 0) * p.vq.st;
#pragma unroll
    for (int s = 0; s < QS; ++s) {
      uint4 x = ok ? *reinterpret_cast<const uint4*>(qrow + s * 16 + half * 8)
                   : make_uint4(0, 0, 0, 0);
      qreg[s] = __builtin_bit_cast(bf16x8, x);
    }
  }

  // ---- tile staging: buffer loads straight into LDS ----------------------
  // Wave w issues the tile's instructions j = w, w+4, ...; lane l of
  // instruction j fills slot j*64 + l = (row, physical chunk pc), reading
  // the row's logical chunk pc ^ swz(row); pad slots read an out-of-range
  // offset (zero, no fault).
  constexpr int KJ = (SM::kChunks + kWaves - 1) / kWaves;  // instructions per wave
  constexpr int VJ = (SM::vChunks + kWaves - 1) / kWaves;
  constexpr uint32_t kPadOff = 0x40000000u;
  uint32_t k_voff[KJ], v_voff[VJ];
#pragma unroll
  for (int i = 0; i < KJ; ++i) {
    const int slot = (wave + kWaves * i) * 64 + lane;
    const int row = slot / SM::kChunks, pc = slot % SM::kChunks;
    k_voff[i] =
        pc < D / 8 ? (uint32_t)(row * k_st * 2 + (pc ^ SM::swz(row)) * 16) : kPadOff;
  }
#pragma unroll
  for (int i = 0; i < VJ; ++i) {
    const int slot = (wave + kWaves * i) * 64 + lane;
    const int row = slot / SM::vChunks, pc = slot % SM::vChunks;
    v_voff[i] =
        pc < D / 8 ? (uint32_t)(row * v_st * 2 + (pc ^ SM::swz(row)) * 16) : kPadOff;
  }
  auto issue_kv = [&] __device__ (int t, uint16_t* kdst, uint16_t* vdst)
      __attribute__((always_inline)) {
    issue_tile<KJ, SM::kChunks>(kg, k_bytes, kdst, k_voff, t * kKeys * k_st * 2, wave);
    issue_tile<VJ, SM::vChunks>(vg, v_bytes, vdst, v_voff, t * kKeys * v_st * 2, wave);
  };

  // Transposing V reads (ds_read_b64_tr_b16). Within each 16-lane group the
  // instruction gives destination lane 4q+j, element e, the element j of the
  // 8 bytes addressed by source lane 4e+q. Source lane s of group G = l/16
  // therefore addresses key row (s/4) and d columns 16*(G%2) + 4*(s%4): the
  // destination lane then holds 4 consecutive keys for its own d column,
  // d = l % 32 of the 32-wide block, as the MFMA A operand needs.
  const int tr_row = (lane & 15) >> 2;
  const int tr_col = ((lane >> 4) & 1) * 16 + (lane & 3) * 4;
  typedef short v4i16 __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) v4i16* lds_v4i16_ptr;
  constexpr int DB0 = D / 32;
  // Element offsets of this lane's fragment reads within a tile: the K
  // operand of k-step s (row col; rows 32.. add 32 rows: same swizzle), and
  // the transposing V reads of d block db, rows +0 and +8 of the 16-key
  // half (kb and hh add whole 16-row groups: same swizzle)
  constexpr int QS0 = D / 16;
  int koff[QS0], voff_lo[DB0], voff_hi[DB0];
#pragma unroll
  for (int s = 0; s < QS0; ++s)
    koff[s] = col * SM::kStride + (((2 * s + half) ^ SM::swz(col)) * 8);
  {
    const int rl = half * 4 + tr_row, rh = rl + 8;
    const int cc = tr_col >> 3, within = tr_col & 7;
#pragma unroll
    for (int db = 0; db < DB0; ++db) {
      voff_lo[db] = rl * SM::vStride + (((db * 4 + cc) ^ SM::swz(rl)) * 8) + within;
      voff_hi[db] = rh * SM::vStride + (((db * 4 + cc) ^ SM::swz(rh)) * 8) + within;
    }
  }

  // ---- online softmax state ----------------------------------------------
  constexpr int DB = D / 32;  // 32-wide d blocks of the output
  f32x16 acc_o[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i) acc_o[i] = (f32x16){};
  float m_run = kNegInit;   // running row max, log2 units
  float l_run = 0.0f;       // this lane's half of the row sum
  bool snapped = false;     // EPI 6: this lane's local output is parked

  // Mask modes of one tile: the branch's own range (local window or causal
  // prefix), or (EPI 6) the keys below the row's window.
  constexpr int kOwn = 0, kBelow = 1;
  auto is_active = [&] __device__ (int t) __attribute__((always_inline)) {
    const int key0 = t * kKeys;
    return wave_on && key0 <= wkey_hi && key0 + kKeys - 1 >= wkey_lo;
  };
  // every element of the tile is read by every row of the wave (no mask)
  auto is_full = [&] __device__ (int t, int mode) __attribute__((always_inline)) {
    const int key0 = t * kKeys;
    if (SEG && key0 < wss_hi) return false;  // a row's example starts inside or after the tile
    if (EPI == 6 && mode == kBelow) return key0 + kKeys - 1 < wlb_lo;
    if (EPI == 6) return key0 >= wlb_hi && key0 + kKeys - 1 <= wpos_lo;
    if (GLOBAL) return key0 + kKeys - 1 <= wpos_lo;
    return key0 >= wpos_hi - p.W + 1 && key0 + kKeys - 1 <= wpos_lo;
  };
  // V fragment for keys kb*32 + hh*16 + [0,16) of d block db (A operand of
  // O^T += V^T P^T); this lane's half supplies keys +4*half+[0,4) and
  // +8+4*half+[0,4), matching its probabilities.
  auto read_vf = [&] __device__ (const uint16_t* vs, int kb, int hh, int db)
      __attribute__((always_inline)) {
    const uint16_t* g0 = vs + (kb * 32 + hh * 16) * SM::vStride;
    const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_ptr)(g0 + voff_lo[db]));
    const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_ptr)(g0 + voff_hi[db]));
    const uint2 l2 = __builtin_bit_cast(uint2, lo);
    const uint2 h2 = __builtin_bit_cast(uint2, hi);
    return __builtin_bit_cast(bf16x8, make_uint4(l2.x, l2.y, h2.x, h2.y));
  };
  // The running max (log2 units) moves lazily: only when a block's max
  // exceeds it by more than kLazy, so probabilities stay below 2^kLazy and
  // the output is rescaled rarely.
  // two probabilities: exp2, bf16 pack, this lane's sum over the block. The
  // sum adds the rounded values the P V products use (a dot product with
  // (1, 1)), so the output is a weighted mean of V rows with exactly those
  // weights: with a lazy max the largest probability is not 1 but up to
  // 2^kLazy, and its rounding would otherwise bias every element of o by
  // up to 2^-9 of the dominant V row.
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
  auto prob_pair = [&] __device__ (float s0, float s1, float& bsum)
      __attribute__((always_inline)) {
    const float p0 = __builtin_amdgcn_exp2f(fmaf(s0, p.scale_log2, -m_run));
    const float p1 = __builtin_amdgcn_exp2f(fmaf(s1, p.scale_log2, -m_run));
    uint32_t pk = pack_bf16x2(p0, p1);
    bsum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pk), ones, bsum, false);
    // an empty asm that "reads and writes" the result pins the pair where it
    // is written (the optimiser would otherwise cluster all exponentials)
    asm volatile("" : "+v"(pk), "+v"(bsum));
    return pk;
  };
  // After a block's probabilities were made against the running max: the
  // lazy max may only move if some probability exceeds 2^kLazy, which a
  // lane's block sum at or below 2^kLazy excludes; so the block max is
  // computed only when some lane's sum exceeds it. A row without a max yet
  // (m_run = kNegInit) gets infinite probabilities for every unmasked key
  // and so always takes this path; a fully masked block leaves it unset.
  // Then the max moves as before and, where it moved, the probabilities are
  // made again. Returns the accumulator's rescale factor; adds the block to l.
  auto settle = [&] __device__ (f32x16& s, uint32_t* pk, float bsum)
      __attribute__((always_inline)) {
    float alpha = 1.0f;
    if (__builtin_amdgcn_ballot_w64(bsum > 256.0f) != 0) {
      float mx = -INFINITY;
#pragma unroll
      for (int e = 0; e < 16; ++e) mx = fmaxf(mx, s[e]);
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx),
                                                        __float_as_uint(mx), false, false);
      mx = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1])) * p.scale_log2;
      const float m_new = mx > m_run + kLazy ? mx : m_run;
      alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
      l_run *= alpha;
      if (__builtin_amdgcn_ballot_w64(alpha != 1.0f) != 0) {
        bsum = 0.0f;
#pragma unroll
        for (int c = 0; c < 8; ++c) pk[c] = prob_pair(s[2 * c], s[2 * c + 1], bsum);
      }
    }
    l_run += bsum;
    return alpha;
  };
  auto mask_block = [&] __device__ (int key0, f32x16& s, int mode)
      __attribute__((always_inline)) {
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int key = key0 + (e >> 2) * 8 + half * 4 + (e & 3);
      bool ok;
      if (EPI == 6 && mode == kBelow) {
        ok = key < lb;                      // below the window (so also causal)
        if (SEG) ok = ok && key >= ss;
      } else {
        ok = key <= pos;
        if (SEG) ok = ok && key >= ss;
        if (!GLOBAL || EPI == 6) ok = ok && key >= lb;
      }
      s[e] = ok ? s[e] : -INFINITY;
    }
  };
  auto rescale = [&] __device__ (float alpha) __attribute__((always_inline)) {
    if (__builtin_amdgcn_ballot_w64(alpha != 1.0f) != 0) {
#pragma unroll
      for (int db = 0; db < DB; ++db) acc_o[db] *= alpha;
    }
  };

  // One tile of 64 keys as two 32-key blocks (kb), in four phases:
  //   QK(kb0) | QK(kb1) + softmax(kb0) | PV(kb0) + softmax(kb1) | PV(kb1)
  // so half of the MFMAs carry softmax VALU work of the other block in their
  // shadow; the second wave of the SIMD covers the rest.
  auto tile = [&] __device__ (int t, const uint16_t* ks, const uint16_t* vs, int mode)
      __attribute__((always_inline)) {
    const bool full = __builtin_amdgcn_readfirstlane(is_full(t, mode));
    const int key0 = t * kKeys;
    f32x16 sc0, sc1;
    uint32_t pk0[8], pk1[8];   // bf16 probability pairs of blocks 0 and 1
    {
      bf16x8 kf[QS];
#pragma unroll
      for (int s = 0; s < QS; ++s)
        kf[s] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(ks + koff[s]));
      // all eight reads in flight before the first product (otherwise they
      // are issued two at a time, each pair waited for)
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int s = 0; s < QS; ++s)
        sc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[s], qreg[s], s ? sc0 : (f32x16){},
                                                       0, 0, 0);
    }
    bf16x8 kf1[QS];
#pragma unroll
    for (int s = 0; s < QS; ++s)
      kf1[s] = __builtin_bit_cast(bf16x8,
                                  *reinterpret_cast<const uint4*>(ks + 32 * SM::kStride + koff[s]));
    if (!full) mask_block(key0, sc0, mode);
    __builtin_amdgcn_sched_barrier(0);
    // QK(kb1), 8 pairs of block 0 spread over its QS MFMAs
    float bsum0 = 0.0f, bsum1 = 0.0f;
#pragma unroll
    for (int s = 0; s < QS; ++s) {
      sc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf1[s], qreg[s], s ? sc1 : (f32x16){},
                                                     0, 0, 0);
#pragma unroll
      for (int i = 0; i < 8 / QS; ++i) {
        const int c = s * (8 / QS) + i;
        pk0[c] = prob_pair(sc0[2 * c], sc0[2 * c + 1], bsum0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    // V fragments are read one d block ahead of their products (the last
    // reads of PV(kb0) fetch the first of PV(kb1)), so no product waits on
    // the LDS read issued just before it; the first two are read before
    // block 0 settles
    bf16x8 va0 = read_vf(vs, 0, 0, 0), va1 = read_vf(vs, 0, 1, 0);
    rescale(settle(sc0, pk0, bsum0));
    if (!full) mask_block(key0 + 32, sc1, mode);
    __builtin_amdgcn_sched_barrier(0);
    // PV(kb0), 8 pairs of block 1 spread over its 2*DB MFMAs
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const int nkb = db + 1 < DB ? 0 : 1, ndb = db + 1 < DB ? db + 1 : 0;
      const bf16x8 vn0 = read_vf(vs, nkb, 0, ndb);
      const bf16x8 vn1 = read_vf(vs, nkb, 1, ndb);
      acc_o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
          va0, __builtin_bit_cast(bf16x8, make_uint4(pk0[0], pk0[1], pk0[2], pk0[3])), acc_o[db],
          0, 0, 0);
      acc_o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
          va1, __builtin_bit_cast(bf16x8, make_uint4(pk0[4], pk0[5], pk0[6], pk0[7])), acc_o[db],
          0, 0, 0);
#pragma unroll
      for (int i = 0; i < 8 / DB; ++i) {
        const int c = db * (8 / DB) + i;
        pk1[c] = prob_pair(sc1[2 * c], sc1[2 * c + 1], bsum1);
      }
      __builtin_amdgcn_sched_barrier(0);
      va0 = vn0;
      va1 = vn1;
    }
    // block 0's products were made before block 1 moved the max
    rescale(settle(sc1, pk1, bsum1));
    // PV(kb1)
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      bf16x8 vn0 = va0, vn1 = va1;
      if (db + 1 < DB) {
        vn0 = read_vf(vs, 1, 0, db + 1);
        vn1 = read_vf(vs, 1, 1, db + 1);
      }
      acc_o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
          va0, __builtin_bit_cast(bf16x8, make_uint4(pk1[0], pk1[1], pk1[2], pk1[3])), acc_o[db],
          0, 0, 0);
      acc_o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
          va1, __builtin_bit_cast(bf16x8, make_uint4(pk1[4], pk1[5], pk1[6], pk1[7])), acc_o[db],
          0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
      va0 = vn0;
      va1 = vn1;
    }
  };
  // EPI 6: rows whose window's lowest key lies in tile t have now seen
  // exactly their window: park acc / l (float32) in the row's scratch row.
  const size_t head_row = (size_t)(b * p.Hq + h);
  auto park_local = [&] __device__ (int t) __attribute__((always_inline)) {
    const int key0 = t * kKeys;
    const bool here = row_ok && lb >= key0 && lb < key0 + kKeys;
    const auto lsw = __builtin_amdgcn_permlane32_swap(__float_as_uint(l_run),
                                                       __float_as_uint(l_run), false, false);
    const float inv = 1.0f / (__uint_as_float(lsw[0]) + __uint_as_float(lsw[1]));
    if (here) {
      float* const dst = p.out_f32 + (head_row * p.ksel + r_lane) * D;
#pragma unroll
      for (int db = 0; db < DB; ++db) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
          *reinterpret_cast<float4*>(dst + db * 32 + j * 8 + half * 4) =
              make_float4(acc_o[db][j * 4 + 0] * inv, acc_o[db][j * 4 + 1] * inv,
                          acc_o[db][j * 4 + 2] * inv, acc_o[db][j * 4 + 3] * inv);
      }
    }
    snapped = snapped || here;
  };
  auto compute = [&] __device__ (int t, const uint16_t* ks, const uint16_t* vs)
      __attribute__((always_inline)) {
    if (!__builtin_amdgcn_readfirstlane(is_active(t))) return;
    if (EPI != 6) {
      tile(t, ks, vs, kOwn);
      return;
    }
    const int key0 = t * kKeys;
    // window keys of some row in this tile; some row's window edge in it;
    // keys below some row's window in it
    if (key0 + kKeys - 1 >= wlb_lo) {
      tile(t, ks, vs, kOwn);
      if (key0 <= wlb_hi) park_local(t);
    }
    if (key0 < wlb_hi) tile(t, ks, vs, kBelow);
  };

  // ---- main loop: tile i of the walk computes from one buffer pair while
  // tile i+1 lands in the other. The loop is unrolled by two so every LDS
  // access names its buffer at compile time.
  const int nt = t_hi - t_lo + 1;
  auto tile_at = [&] __device__ (int i) __attribute__((always_inline)) {
    return BACKWARD ? t_hi - i : t_lo + i;
  };
  auto step = [&] __device__ (int i, const uint16_t* ks, const uint16_t* vs, uint16_t* kn,
                              uint16_t* vn) __attribute__((always_inline)) {
    if (i + 1 < nt) issue_kv(tile_at(i + 1), kn, vn);
    compute(tile_at(i), ks, vs);
    __builtin_amdgcn_s_waitcnt(kWaitVm0);
    __syncthreads();
  };
  if (nt > 0) {
    issue_kv(tile_at(0), K0, V0);
    __builtin_amdgcn_s_waitcnt(kWaitVm0);
    __syncthreads();
  }
#pragma unroll 1
  for (int i = 0; i < nt; i += 2) {
    step(i, K0, V0, K1, V1);
    if (i + 1 < nt) step(i + 1, K1, V1, K0, V0);
  }

  // ---- epilogue ----------------------------------------------------------
  const auto lsw = __builtin_amdgcn_permlane32_swap(__float_as_uint(l_run),
                                                     __float_as_uint(l_run), false, false);
  const float l_tot = __uint_as_float(lsw[0]) + __uint_as_float(lsw[1]);
  if (EPI == 3 && p.nsplit > 1 && row_ok) {
    // partial of one key range: unnormalised o, running max (log2 units),
    // row sum; a merge kernel combines the ranges and applies the gate
    float* const po =
        p.part + (((size_t)split * p.B * p.Hq + head_row) * p.ksel + r_lane) * (D + 4);
#pragma unroll
    for (int db = 0; db < DB; ++db) {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        *reinterpret_cast<float4*>(po + db * 32 + j * 8 + half * 4) =
            make_float4(acc_o[db][j * 4 + 0], acc_o[db][j * 4 + 1], acc_o[db][j * 4 + 2],
                        acc_o[db][j * 4 + 3]);
    }
    if (half == 0) *reinterpret_cast<float2*>(po + D) = make_float2(m_run, l_tot);
  } else if (row_ok) {
  const float inv = 1.0f / l_tot;
  if (p.lse_out && half == 0)
    p.lse_out[head_row * R + (GLOBAL ? r_lane : pos)] = (m_run + __log2f(l_tot)) * kLn2;
  uint16_t* const orow = p.out_io + b * p.vo.sb + h * p.vo.sh + (long long)pos * p.vo.st;
  int rk = -1;
  if (EPI == 1) {
    rk = p.rank[(size_t)b * p.n + pos];
    if (SEG && rk >= p.ksel) rk = -1;  // never address past the scratch rows
  }
  float sig = 0.0f;
  if (EPI == 3 || EPI == 5 || EPI == 6) sig = 1.0f / (1.0f + expf(-p.gate[(size_t)b * p.n + pos]));
  // Everything the stores combine with is loaded first: the compiler cannot
  // tell these buffers from the outputs, so a load placed after a store
  // would wait for every store before it. EPI 3/5: the row's local output;
  // EPI 6: the parked local output (rows that parked one); EPI 4: the head's
  // router weights, for this lane's half of <router_w[h], o_local row>.
  constexpr bool kPre = EPI == 3 || EPI == 4 || EPI == 5 || EPI == 6;
  float4 pre[kPre ? DB * 4 : 1];
  if (kPre && (EPI != 6 || snapped)) {
    const float* src = EPI == 4 ? p.router_w + (size_t)h * D
                       : EPI == 5 ? p.scratch + (head_row * p.n + pos) * D
                                  : p.scratch + (head_row * p.ksel + r_lane) * D;
#pragma unroll
    for (int k = 0; k < DB * 4; ++k)
      pre[k] = *reinterpret_cast<const float4*>(src + (k >> 2) * 32 + (k & 3) * 8 + half * 4);
  }
  float rdot = 0.0f;
#pragma unroll
  for (int db = 0; db < DB; ++db) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int d0 = db * 32 + j * 8 + half * 4;
      float4 o4 = make_float4(acc_o[db][j * 4 + 0] * inv, acc_o[db][j * 4 + 1] * inv,
                              acc_o[db][j * 4 + 2] * inv, acc_o[db][j * 4 + 3] * inv);
      float4 l4 = pre[kPre ? db * 4 + j : 0];
      if (EPI == 0) {
        *reinterpret_cast<float4*>(p.out_f32 + (head_row * p.n + pos) * D + d0) = o4;
      } else if (EPI == 4) {
        *reinterpret_cast<float4*>(p.out_f32 + (head_row * p.n + pos) * D + d0) = o4;
        uint2 w2 = make_uint2(pack_bf16x2(o4.x, o4.y), pack_bf16x2(o4.z, o4.w));
        *reinterpret_cast<uint2*>(orow + d0) = w2;
        rdot = fmaf(o4.x, l4.x, fmaf(o4.y, l4.y, fmaf(o4.z, l4.z, fmaf(o4.w, l4.w, rdot))));
      } else if (EPI == 5 || EPI == 6) {
        // EPI 6: a row whose window reaches key 0 never parked one: its
        // local output is its global output
        if (EPI == 6 && !snapped) l4 = o4;
        float4 c4 = make_float4(l4.x + sig * o4.x, l4.y + sig * o4.y, l4.z + sig * o4.z,
                                l4.w + sig * o4.w);
        uint2 w2 = make_uint2(pack_bf16x2(c4.x, c4.y), pack_bf16x2(c4.z, c4.w));
        *reinterpret_cast<uint2*>(orow + d0) = w2;
      } else if (EPI == 2) {
        *reinterpret_cast<float4*>(p.out_f32 + (head_row * p.ksel + r_lane) * D + d0) = o4;
      } else if (EPI == 1) {
        if (rk >= 0) {
          *reinterpret_cast<float4*>(p.out_f32 + (head_row * p.ksel + rk) * D + d0) = o4;
        } else {
          uint2 w2 = make_uint2(pack_bf16x2(o4.x, o4.y), pack_bf16x2(o4.z, o4.w));
          *reinterpret_cast<uint2*>(orow + d0) = w2;
        }
      } else if (EPI == 7) {
        uint2 w2 = make_uint2(pack_bf16x2(o4.x, o4.y), pack_bf16x2(o4.z, o4.w));
        *reinterpret_cast<uint2*>(orow + d0) = w2;
      } else {
        if (p.og_out)
          *reinterpret_cast<float4*>(p.og_out + (head_row * p.ksel + r_lane) * D + d0) = o4;
        float4 c4 = make_float4(l4.x + sig * o4.x, l4.y + sig * o4.y, l4.z + sig * o4.z,
                                l4.w + sig * o4.w);
        uint2 w2 = make_uint2(pack_bf16x2(c4.x, c4.y), pack_bf16x2(c4.z, c4.w));
        *reinterpret_cast<uint2*>(orow + d0) = w2;
      }
    }
  }
  if (EPI == 4) {
    // both halves of a query's row are live together (row_ok is per query)
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(rdot), __float_as_uint(rdot),
                                                     false, false);
    if (half == 0)
      p.router_part[head_row * p.n + pos] = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
  }
  }  // row_ok
}

template <int D, bool GLOBAL, int EPI, bool SEG, bool QUEUE>
__global__ __launch_bounds__(kThreads, 2)
__attribute__((amdgpu_waves_per_eu(2, 2))) void attn_bf16_kernel(Params p) {
  using SM = Smem<D>;
  // Four distinct LDS objects, so the compiler can tell that reads of one
  // buffer do not wait on buffer loads still landing in another.
  __shared__ __attribute__((aligned(16))) uint16_t K0[SM::kElems];
  __shared__ __attribute__((aligned(16))) uint16_t K1[SM::kElems];
  __shared__ __attribute__((aligned(16))) uint16_t V0[SM::vElems];
  __shared__ __attribute__((aligned(16))) uint16_t V1[SM::vElems];

  // ---- which tile -------------------------------------------------------
  const int bid = blockIdx.x;
  const int Lx = (bid % kNumXcd) * p.per_xcd + bid / kNumXcd;
  if (Lx >= p.total_wg * p.nsplit) return;
  // split key ranges (fused global branch of a small problem): workgroup
  // Lx takes key range `split` of row block L
  const int split = Lx % p.nsplit;
  const int L = Lx / p.nsplit;
  // Queued global launches (p.sched_count set): each (b, kv head) unit has a
  // queue of its row blocks, heaviest first (the last rows; for packed
  // examples the order the schedule kernel built). A workgroup takes blocks
  // from its home unit's queue (the unit its XCD holds, so K/V stay in that
  // L2) and, once that queue is empty, from the other units' in turn, until
  // every queue is empty: an XCD whose units have less work (a selection
  // that leans late in one sequence and early in another) goes on with
  // the others' remaining blocks instead of idling. An empty queue stays
  // empty, so every block is taken exactly once. Otherwise the workgroup
  // does the one block its index names. Always compiled for the routed and
  // the packed-example global branches; the fused branch has both forms
  // and takes the queue when fewer (b, kv head) units than XCDs make the
  // static order split a unit's blocks over XCDs by index (longest first:
  // one XCD of the pair gets most of the work). With one unit per XCD and a
  // balanced selection the queue measured 3.5 % slower (its codegen and
  // atomics); it saves 2.5 % on the routed branch's router-driven selection
  // and 38 % on a selection as skewed as latest tokens in one sequence,
  // earliest in the other.
  constexpr bool kQueue = GLOBAL && (EPI == 5 || SEG || QUEUE);
  const bool queued = kQueue && p.sched_count != nullptr;
  __shared__ int taken[2];
#pragma unroll 1
  for (int iter = 0;; ++iter) {
    int unit_bh = L / p.wg_per_unit;             // b * Hkv + kv head
    int w = L % p.wg_per_unit;
    if (queued) {
      if (threadIdx.x == 0) {
        const int nu = p.B * p.Hkv;
        int u = unit_bh;
        int r = atomicAdd(p.sched_count + u, 1);
        for (int tries = 1; r >= p.wg_per_unit && tries < nu; ++tries) {
          u = u + 1 < nu ? u + 1 : 0;
          r = atomicAdd(p.sched_count + u, 1);
        }
        taken[0] = u;
        taken[1] = r;
      }
      __syncthreads();
      if (taken[1] >= p.wg_per_unit) return;  // every queue is empty
      unit_bh = taken[0];
      w = p.sched_perm ? p.sched_perm[taken[1]] : p.wg_per_unit - 1 - taken[1];
    } else {
      if (iter > 0) return;
      if (GLOBAL) w = p.wg_per_unit - 1 - w;      // longest prefix first
    }
    attn_block<D, GLOBAL, EPI, SEG>(p, unit_bh, w, split, K0, K1, V0, V1);
    // every wave is done with this block's tiles before the next block's
    // loads reuse the buffers
    if (kQueue) __syncthreads();
  }
}

// Which (b, kv head) units each XCD serves in the single-launch fused
// forward, and how many row-block workgroups of each kind there are. Units
// are pinned to XCDs (their K/V stay in that XCD's L2): with U = 8 m units,
// XCD x serves units x, x + 8, ...; with U = 8 / c, each unit has c XCDs,
// which take its workgroups in turn.
struct FusedPlan {
  int U;        // B * Hkv
  int per;      // U = 8m: m units per XCD; 8 % U == 0: c XCDs per unit
  int gw, lw;   // global / local workgroups per unit
};

// Single-launch fused forward: on each XCD its global row blocks first
// (longest causal prefix first), then its local row blocks, so the short
// local blocks fill the gaps the long global ones leave at the end. The
// global rows (selected) compute their local branch too (EPI 6); the local
// rows are the unselected ones (EPI 7). Nothing depends on anything else
// in the launch. Packed examples (SEG): a row's prefix starts at its
// example's first token, so the global row blocks' work varies widely;
// each global workgroup takes the next of its unit's blocks in the order of
// pg.sched_perm (most keys to stream first) from a counter, so the XCDs
// that share a unit stay balanced.
template <int D, bool SEG>
__global__ __launch_bounds__(kThreads, 2)
__attribute__((amdgpu_waves_per_eu(2, 2))) void attn_bf16_fused_kernel(Params pg, Params pl,
                                                                       FusedPlan plan) {
  using SM = Smem<D>;
  __shared__ __attribute__((aligned(16))) uint16_t K0[SM::kElems];
  __shared__ __attribute__((aligned(16))) uint16_t K1[SM::kElems];
  __shared__ __attribute__((aligned(16))) uint16_t V0[SM::vElems];
  __shared__ __attribute__((aligned(16))) uint16_t V1[SM::vElems];
  const int x = blockIdx.x % kNumXcd;
  const int s = blockIdx.x / kNumXcd;
  int unit, rank, ng;
  if (plan.U >= kNumXcd) {
    // m units on this XCD, their blocks interleaved by rank
    const int m = plan.per;
    ng = m * plan.gw;
    const int sl = s < ng ? s : s - ng;
    if (s >= ng && sl >= m * plan.lw) return;
    unit = x + kNumXcd * (sl % m);
    rank = sl / m;
  } else {
    // this XCD is number j of the c that serve unit x % U
    const int c = plan.per, j = x / plan.U;
    ng = plan.gw > j ? (plan.gw - j + c - 1) / c : 0;
    const int nl = plan.lw > j ? (plan.lw - j + c - 1) / c : 0;
    const int sl = s < ng ? s : s - ng;
    if (s >= ng && sl >= nl) return;
    unit = x % plan.U;
    rank = j + sl * c;
  }
  if (s < ng) {
    int w = plan.gw - 1 - rank;   // longest causal prefix first
    if (SEG) {
      __shared__ int ticket;
      if (threadIdx.x == 0) ticket = atomicAdd(pg.sched_count + unit, 1);
      __syncthreads();
      // exactly plan.gw global workgroups serve a unit; the clamp only
      // keeps a miscount in bounds
      w = pg.sched_perm[min(ticket, plan.gw - 1)];
    }
    attn_block<D, true, 6, SEG>(pg, unit, w, 0, K0, K1, V0, V1);
  } else
    attn_block<D, false, 7, SEG>(pl, unit, rank, 0, K0, K1, V0, V1);
}

// Small problems (the global branch split over key ranges): the split global
// branch (EPI 3, partials) and the local band (EPI 1) in one grid, global
// workgroups first; neither reads the other's results, and a merge kernel
// combines them after. Each part keeps its own XCD-aware order (the global
// part's grid is a multiple of 8, so the local part's workgroups are dealt
// to the XCDs as in a launch of their own).
template <int D>
__global__ __launch_bounds__(kThreads, 2)
__attribute__((amdgpu_waves_per_eu(2, 2))) void attn_bf16_pair_kernel(Params pg, Params pl,
                                                                      int g_grid) {
  using SM = Smem<D>;
  __shared__ __attribute__((aligned(16))) uint16_t K0[SM::kElems];
  __shared__ __attribute__((aligned(16))) uint16_t K1[SM::kElems];
  __shared__ __attribute__((aligned(16))) uint16_t V0[SM::vElems];
  __shared__ __attribute__((aligned(16))) uint16_t V1[SM::vElems];
  const int bid = blockIdx.x;
  if (bid < g_grid) {
    const int Lx = (bid % kNumXcd) * pg.per_xcd + bid / kNumXcd;
    if (Lx >= pg.total_wg * pg.nsplit) return;
    const int split = Lx % pg.nsplit;
    const int L = Lx / pg.nsplit;
    attn_block<D, true, 3, false>(pg, L / pg.wg_per_unit,
                                  pg.wg_per_unit - 1 - L % pg.wg_per_unit, split, K0, K1, V0,
                                  V1);
  } else {
    const int b2 = bid - g_grid;
    const int Lx = (b2 % kNumXcd) * pl.per_xcd + b2 / kNumXcd;
    if (Lx >= pl.total_wg) return;
    attn_block<D, false, 1, false>(pl, Lx / pl.wg_per_unit, Lx % pl.wg_per_unit, 0, K0, K1, V0,
                                   V1);
  }
}

// Work order of the global branch's workgroups over packed examples: the
// keys a workgroup streams (from its first row's example start to its last
// row) estimate its work; slots are bucketed by that estimate (1024 buckets,
// heaviest first; order within a bucket is arbitrary, which changes only
// the timing, never a result) into perm, and the per-unit counters the
// workgroups take ranks from are zeroed. One 1024-thread workgroup.
__global__ __launch_bounds__(1024) void global_sched_kernel(const int32_t* __restrict__ idx,
                                                            const int32_t* __restrict__ seg_start,
                                                            int n, int K, int G, int units,
                                                            int wpu, int n_count,
                                                            int32_t* __restrict__ perm,
                                                            int32_t* __restrict__ count) {
  __shared__ int bins[1024];
  __shared__ int wmax[16];
  const int t = threadIdx.x;
  for (int i = t; i < n_count; i += 1024) count[i] = 0;
  auto work = [&](int w) {
    const int u0 = w * kWaves, u1 = min(u0 + kWaves, units) - 1;
    const int r0 = (u0 / G) * kRows, r1 = min((u1 / G) * kRows + kRows, K) - 1;
    const int p0 = min(max(idx[r0], 0), n - 1), p1 = min(max(idx[r1], 0), n - 1);
    return max(p1 - seg_start[p0] + 1, 1);
  };
  int mx = 1;
  for (int w = t; w < wpu; w += 1024) mx = max(mx, work(w));
  for (int off = 32; off > 0; off >>= 1) mx = max(mx, __shfl_xor(mx, off, 64));
  if ((t & 63) == 0) wmax[t >> 6] = mx;
  bins[t] = 0;
  __syncthreads();
  mx = 1;
  for (int i = 0; i < 16; ++i) mx = max(mx, wmax[i]);
  // bucket 0 = heaviest
  auto bucket = [&](int wk) { return 1023 - (int)((long long)wk * 1023 / mx); };
  for (int w = t; w < wpu; w += 1024) atomicAdd(&bins[bucket(work(w))], 1);
  __syncthreads();
  {  // exclusive scan of the 1024 counts: within each wave, then across
    const int c = bins[t];
    int incl = c;
    for (int off = 1; off < 64; off <<= 1) {
      const int y = __shfl_up(incl, off, 64);
      if ((t & 63) >= off) incl += y;
    }
    if ((t & 63) == 63) wmax[t >> 6] = incl;  // wave totals (the maxima are consumed)
    __syncthreads();
    int base = 0;
    for (int i = 0; i < (t >> 6); ++i) base += wmax[i];
    bins[t] = base + incl - c;
  }
  __syncthreads();
  for (int w = t; w < wpu; w += 1024) perm[atomicAdd(&bins[bucket(work(w))], 1)] = w;
}

__global__ void zero_ints_kernel(int32_t* __restrict__ p, int n) {
  for (int i = threadIdx.x; i < n; i += blockDim.x) p[i] = 0;
}

// Fused global branch split over key ranges: one wave per selected row
// merges the ranges' partials (max m_s and sum l_s in log2 units, o_s
// unnormalised: o = sum_s 2^(m_s - m) o_s / sum_s 2^(m_s - m) l_s, m the
// largest m_s), then writes o_local + sigmoid(gate) o_global as the fused
// epilogue does. Every row has key 0 in the first range, so the sum is
// positive.
template <int D>
__global__ __launch_bounds__(256) void global_merge_kernel(
    const float* __restrict__ part, int nsplit, int B, int Hq, int k, int n,
    const int32_t* __restrict__ idx, const float* __restrict__ gate,
    const float* __restrict__ scratch, uint16_t* __restrict__ out, View vo) {
  constexpr int E = D / 64;  // elements per lane
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const long long rows = (long long)B * Hq * k;
  const long long row = (long long)blockIdx.x * 4 + wave;  // (b * Hq + h) * k + r
  if (row >= rows) return;
  const int head_row = (int)(row / k), r = (int)(row % k);
  const int b = head_row / Hq, h = head_row % Hq;
  const size_t plane = (size_t)rows * (D + 4);
  const float* const p0 = part + (size_t)row * (D + 4);
  float m = -INFINITY;
  for (int s = 0; s < nsplit; ++s) m = fmaxf(m, p0[s * plane + D]);
  float l = 0.0f, acc[E];
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] = 0.0f;
  for (int s = 0; s < nsplit; ++s) {
    const float* const ps = p0 + s * plane;
    const float wgt = __builtin_amdgcn_exp2f(ps[D] - m);
    l = fmaf(ps[D + 1], wgt, l);
#pragma unroll
    for (int e = 0; e < E; ++e) acc[e] = fmaf(ps[lane * E + e], wgt, acc[e]);
  }
  const float inv = 1.0f / l;
  const int pos = idx[(size_t)b * k + r];
  const float sig = 1.0f / (1.0f + expf(-gate[(size_t)b * n + pos]));
  const float* const lrow = scratch + ((size_t)head_row * k + r) * D + lane * E;
  uint16_t* const orow = out + b * vo.sb + h * vo.sh + (long long)pos * vo.st + lane * E;
  if (E == 2) {
    const float c0 = lrow[0] + sig * (acc[0] * inv);
    const float c1 = lrow[1] + sig * (acc[E - 1] * inv);
    *reinterpret_cast<uint32_t*>(orow) = pack_bf16x2(c0, c1);
  } else {
    orow[0] = f32_to_bf16_bits(lrow[0] + sig * (acc[0] * inv));
  }
}

template <int D, bool GLOBAL, int EPI, bool SEG = false, bool QUEUE = false>
hipError_t launch_one(const Params& prm, hipStream_t s) {
  static_assert(GLOBAL == (EPI == 2 || EPI == 3 || EPI == 5), "epilogue of the other branch");
  const int grid = prm.per_xcd * kNumXcd;  // per_xcd counts split workgroups
  hipLaunchKernelGGL((attn_bf16_kernel<D, GLOBAL, EPI, SEG, QUEUE>), dim3(grid), dim3(kThreads), 0, s,
                     prm);
  return hipGetLastError();
}

template <int D>
hipError_t dispatch_epi(Epi epi, const Params& prm, hipStream_t s) {
  if (prm.seg_start) {  // packed examples: the fused forward only
    if (epi == Epi::LocalFused) return launch_one<D, false, 1, true>(prm, s);
    if (epi == Epi::GlobalFused) return launch_one<D, true, 3, true>(prm, s);
    return hipErrorInvalidValue;
  }
  switch (epi) {
    case Epi::LocalAll: return launch_one<D, false, 0>(prm, s);
    case Epi::LocalFused: return launch_one<D, false, 1>(prm, s);
    case Epi::GlobalAll: return launch_one<D, true, 2>(prm, s);
    case Epi::GlobalFused:
      return prm.sched_count ? launch_one<D, true, 3, false, true>(prm, s)
                             : launch_one<D, true, 3>(prm, s);
    case Epi::LocalRouted: return launch_one<D, false, 4>(prm, s);
    case Epi::GlobalRouted: return launch_one<D, true, 5>(prm, s);
  }
  return hipErrorInvalidValue;
}

template <int D>
hipError_t launch_fused(const Params& pg, const Params& pl, const FusedPlan& plan, int grid,
                        hipStream_t s) {
  if (pg.seg_start)
    hipLaunchKernelGGL((attn_bf16_fused_kernel<D, true>), dim3(grid), dim3(kThreads), 0, s, pg,
                       pl, plan);
  else
    hipLaunchKernelGGL((attn_bf16_fused_kernel<D, false>), dim3(grid), dim3(kThreads), 0, s, pg,
                       pl, plan);
  return hipGetLastError();
}

}  // namespace

bool attn_bf16_fused_ok(const Dims& d) {
  if (d.dtype != 1 || d.k <= 0 || (d.d != 64 && d.d != 128)) return false;
  if (attn_bf16_splits(d) > 1) return false;    // small problems split key ranges instead
  const int U = d.B * d.Hkv;
  return U % kNumXcd == 0 || kNumXcd % U == 0;
}

hipError_t launch_attn_bf16_fused(const Dims& d, const AttnArgs& a, const int32_t* nidx,
                                  hipStream_t s) {
  if (d.B == 0 || d.k == 0) return hipSuccess;
  Params pg{};
  pg.q = static_cast<const uint16_t*>(a.q);
  pg.k = static_cast<const uint16_t*>(a.k);
  pg.v = static_cast<const uint16_t*>(a.v);
  pg.idx = a.idx;
  pg.gate = a.gate;
  pg.out_f32 = a.out_f32;          // parked local outputs of the selected rows
  pg.scratch = a.out_f32;
  pg.out_io = static_cast<uint16_t*>(a.out_io);
  pg.B = d.B;
  pg.Hq = d.Hq;
  pg.Hkv = d.Hkv;
  pg.n = d.n;
  pg.W = d.window;
  pg.ksel = d.k;
  pg.scale_log2 = d.scale * kLog2e;
  pg.vq = d.vq;
  pg.vk = d.vk;
  pg.vv = d.vv;
  pg.vo = d.vo;
  pg.nsplit = 1;
  const int G = d.Hq / d.Hkv;
  pg.units = (d.k + kRows - 1) / kRows * G;
  pg.wg_per_unit = (pg.units + kWaves - 1) / kWaves;
  pg.total_wg = d.B * d.Hkv * pg.wg_per_unit;
  pg.seg_start = a.seg_start;
  if (a.seg_start) {
    // packed examples (one stream): the global row blocks' work order
    if (d.B != 1 || !a.sched) return hipErrorInvalidValue;
    int32_t* const perm = a.sched;
    hipLaunchKernelGGL(global_sched_kernel, dim3(1), dim3(1024), 0, s, a.idx, a.seg_start, d.n,
                       d.k, G, pg.units, pg.wg_per_unit, d.B * d.Hkv, perm,
                       a.sched + pg.wg_per_unit);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    pg.sched_perm = perm;
    pg.sched_count = a.sched + pg.wg_per_unit;   // zeroed by the kernel above
  }
  Params pl = pg;
  const int nl = d.n - d.k;          // unselected rows per sequence
  pl.idx = nidx;
  pl.ksel = nl;
  pl.units = (nl + kRows - 1) / kRows * G;
  pl.wg_per_unit = (pl.units + kWaves - 1) / kWaves;
  pl.total_wg = d.B * d.Hkv * pl.wg_per_unit;
  FusedPlan plan;
  plan.U = d.B * d.Hkv;
  plan.gw = pg.wg_per_unit;
  plan.lw = nl > 0 ? pl.wg_per_unit : 0;
  int slots;
  if (plan.U >= kNumXcd) {
    plan.per = plan.U / kNumXcd;
    slots = plan.per * (plan.gw + plan.lw);
  } else {
    plan.per = kNumXcd / plan.U;
    // XCD j = 0 of a unit has the most slots
    slots = (plan.gw + plan.per - 1) / plan.per + (plan.lw + plan.per - 1) / plan.per;
  }
  const int grid = slots * kNumXcd;
  if (d.d == 64) return launch_fused<64>(pg, pl, plan, grid, s);
  if (d.d == 128) return launch_fused<128>(pg, pl, plan, grid, s);
  return hipErrorInvalidValue;
}

int attn_bf16_splits(const Dims& d) {
  // Enough workgroups for two per CU on a 256-CU part, at most 8 ranges and
  // at least 4 key tiles per range; a fixed function of the shape, so the
  // workspace it needs does not depend on the device.
  constexpr long long kTarget = 512;
  if (d.k <= 0) return 1;
  const long long G = d.Hq / d.Hkv;
  const long long units = ((long long)d.k + kRows - 1) / kRows * G;
  const long long total = (long long)d.B * d.Hkv * ((units + kWaves - 1) / kWaves);
  if (total >= kTarget) return 1;
  long long s = (kTarget + total - 1) / total;
  // The paired launch also runs the local band's workgroups (every row).
  // When they and at least two ranges per global row block fit in one
  // round of kTarget workgroups, take the most ranges that still fit: a
  // second round costs more than the longer ranges (4K layer: 8 ranges,
  // 704 workgroups, 0.072 ms; 4 ranges, 480 workgroups, 0.061 ms).
  const long long lunits = ((long long)d.n + kRows - 1) / kRows * G;
  const long long local = (long long)d.B * d.Hkv * ((lunits + kWaves - 1) / kWaves);
  if (local + 2 * total <= kTarget) s = (kTarget - local) / total;
  s = std::min<long long>(s, 8);
  s = std::min<long long>(s, std::max<long long>(1, ((long long)d.n + kKeys - 1) / kKeys / 4));
  return (int)std::max<long long>(s, 1);
}

size_t attn_bf16_split_floats(const Dims& d) {
  const int s = attn_bf16_splits(d);
  return s > 1 ? (size_t)s * d.B * d.Hq * d.k * (d.d + 4) : 0;
}

size_t attn_bf16_sched_ints(const Dims& d, bool packed) {
  const size_t npb = ((size_t)d.k + kRows - 1) / kRows;
  const size_t units = npb * (size_t)(d.Hq / d.Hkv);
  return (packed ? (units + kWaves - 1) / kWaves : 0) + (size_t)d.B * d.Hkv;
}

namespace {

// The launch parameters of one branch (everything but the work queues).
Params branch_params(const Dims& d, Epi epi, const AttnArgs& a) {
  const bool global =
      epi == Epi::GlobalAll || epi == Epi::GlobalFused || epi == Epi::GlobalRouted;
  const int R = global ? d.k : d.n;
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
  prm.vq = d.vq;
  prm.vk = d.vk;
  prm.vv = d.vv;
  prm.vo = d.vo;
  prm.lse_out = a.lse_out;
  prm.og_out = a.og_out;
  prm.router_w = a.router_w;
  prm.router_part = a.router_part;
  prm.seg_start = a.seg_start;
  prm.sched_perm = nullptr;
  prm.sched_count = nullptr;
  // a small fused global branch splits each row block's keys over several
  // workgroups (partials in a.split_part) and merges them after
  prm.nsplit = 1;
  prm.part = nullptr;
  if (epi == Epi::GlobalFused && a.split_part && !a.seg_start && !a.lse_out && !a.og_out) {
    prm.nsplit = attn_bf16_splits(d);
    if (prm.nsplit > 1) prm.part = a.split_part;
    else prm.nsplit = 1;
  }
  prm.per_xcd = (prm.total_wg * prm.nsplit + kNumXcd - 1) / kNumXcd;
  return prm;
}

template <int D>
hipError_t launch_merge(const Dims& d, const AttnArgs& a, const Params& prm, hipStream_t s) {
  const long long rows = (long long)d.B * d.Hq * d.k;
  const dim3 mgrid((unsigned)((rows + 3) / 4));
  hipLaunchKernelGGL(global_merge_kernel<D>, mgrid, dim3(256), 0, s, prm.part, prm.nsplit, d.B,
                     d.Hq, d.k, d.n, a.idx, a.gate, a.scratch, prm.out_io, d.vo);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_bf16(const Dims& d, Epi epi, const AttnArgs& a, hipStream_t s) {
  const bool global =
      epi == Epi::GlobalAll || epi == Epi::GlobalFused || epi == Epi::GlobalRouted;
  const int R = global ? d.k : d.n;
  if (d.B == 0 || R == 0) return hipSuccess;
  Params prm = branch_params(d, epi, a);
  const int G = d.Hq / d.Hkv;
  if (global && a.sched && prm.nsplit == 1) {
    // the queues' counters are zeroed by a kernel on the stream (no memset
    // node, so the sequence can be captured in a graph)
    if (a.seg_start) {
      int32_t* perm = a.sched;
      int32_t* count = a.sched + prm.wg_per_unit;
      hipLaunchKernelGGL(global_sched_kernel, dim3(1), dim3(1024), 0, s, a.idx, a.seg_start,
                         d.n, d.k, G, prm.units, prm.wg_per_unit, d.B * d.Hkv, perm, count);
      prm.sched_perm = perm;
      prm.sched_count = count;
    } else if (epi != Epi::GlobalFused || d.B * d.Hkv < kNumXcd) {
      hipLaunchKernelGGL(zero_ints_kernel, dim3(1), dim3(256), 0, s, a.sched, d.B * d.Hkv);
      prm.sched_count = a.sched;
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipError_t e;
  if (d.d == 64) e = dispatch_epi<64>(epi, prm, s);
  else if (d.d == 128) e = dispatch_epi<128>(epi, prm, s);
  else return hipErrorInvalidValue;
  if (e != hipSuccess || prm.nsplit == 1) return e;
  return d.d == 64 ? launch_merge<64>(d, a, prm, s) : launch_merge<128>(d, a, prm, s);
}

bool attn_bf16_pair_ok(const Dims& d) {
  return d.dtype == 1 && d.k > 0 && (d.d == 64 || d.d == 128) && attn_bf16_splits(d) > 1;
}

hipError_t launch_attn_bf16_pair(const Dims& d, const AttnArgs& a, hipStream_t s) {
  if (d.B == 0 || d.k == 0) return hipSuccess;
  if (!a.split_part || a.seg_start || a.lse_out || a.og_out) return hipErrorInvalidValue;
  const Params pg = branch_params(d, Epi::GlobalFused, a);
  const Params pl = branch_params(d, Epi::LocalFused, a);
  if (pg.nsplit < 2) return hipErrorInvalidValue;
  const int g_grid = pg.per_xcd * kNumXcd;
  const int grid = g_grid + pl.per_xcd * kNumXcd;
  if (d.d == 64)
    hipLaunchKernelGGL(attn_bf16_pair_kernel<64>, dim3(grid), dim3(kThreads), 0, s, pg, pl,
                       g_grid);
  else
    hipLaunchKernelGGL(attn_bf16_pair_kernel<128>, dim3(grid), dim3(kThreads), 0, s, pg, pl,
                       g_grid);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return d.d == 64 ? launch_merge<64>(d, a, pg, s) : launch_merge<128>(d, a, pg, s);
}

}  // namespace logo
