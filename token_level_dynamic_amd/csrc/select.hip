// Budget controller + compaction: per sequence, the k largest gate logits
// (ties to the lower position), written as mask / ascending idx / rank.
//
// Pages: LoGo abstract (a gate and a threshold-based budget controller
// keeping a target global ratio); "Learning When to Attend", section "The
// Architecture of Conditional Attention" (a binary decision per token).
//
// One workgroup of 1024 threads per sequence.
//  1. Threshold: radix select on the order-preserving 32-bit image of each
//     logit (NaN lowest, -0.0 == +0.0), digits of 12, 10 and 10 bits, MSB
//     first, histograms in LDS. It yields T, the k-th largest image, and
//     `need`, how many tokens with image == T are taken (lowest positions).
//  2. Compaction: one pass in position order. A token is selected when its
//     image > T, or == T and fewer than `need` tokens with image == T come
//     before it. Its rank is (#images > T before it) + min(#ties before it,
//     need). Both counts come from one block-wide exclusive scan of a packed
//     (greater, tie) pair per thread, carried across chunks.
#include "logo_internal.h"

namespace logo {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kItems = 8;                 // positions per thread per chunk
constexpr int kChunk = kThreads * kItems; // 8192 < 2^16: packed counts fit
constexpr int kRegChunks = 8;             // sequences of up to 65536 positions are read
                                          // once, into registers (8 x 8 per thread)

__device__ __forceinline__ uint32_t order_image(float x) {
  uint32_t u = __float_as_uint(x);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0u;  // NaN: below -inf (0x007fffff)
  if (u == 0x80000000u) u = 0u;                     // -0.0 -> +0.0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Exclusive scan of one uint32 per thread across the 1024-thread block.
// Returns the exclusive prefix; *total receives the block sum. Uses
// `ws` (kWaves + 1 entries of LDS). Contains three barriers.
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t x, uint32_t* ws,
                                                         uint32_t* total) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  uint32_t incl = x;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    uint32_t y = __shfl_up(incl, off, 64);
    if (lane >= off) incl += y;
  }
  if (lane == 63) ws[wave] = incl;
  __syncthreads();
  if (wave == 0) {
    uint32_t t = lane < kWaves ? ws[lane] : 0u;
    uint32_t ti = t;
#pragma unroll
    for (int off = 1; off < kWaves; off <<= 1) {
      uint32_t y = __shfl_up(ti, off, 64);
      if (lane >= off) ti += y;
    }
    if (lane < kWaves) ws[lane] = ti - t;        // exclusive per wave
    if (lane == kWaves - 1) ws[kWaves] = ti;     // block total
  }
  __syncthreads();
  uint32_t r = ws[wave] + incl - x;
  *total = ws[kWaves];
  __syncthreads();  // every wave has read ws before the next scan rewrites it
  return r;
}

// One workgroup per sequence. Batched rows (SEG == false): row b holds
// gate[b*n .. b*n + n), writes idx[b*k ..] with positions within the row and
// rank = index in the row's list. Packed examples (SEG == true): example e
// is seg[e] = {start, length, k_e, offset}; positions written to idx (at
// idx[offset ..]) are absolute token positions and rank is the index in the
// concatenated list; writes past `idx_cap` are dropped.
// nidx (optional): the positions not selected, ascending (the rows the
// local-only work of a fused forward gathers): batched rows at
// nidx[b*(n-k) ..]; packed examples at nidx[start - offset ..] (the tokens
// before the example less its selected predecessors), absolute positions,
// writes past `nidx_cap` dropped.
template <bool SEG>
__global__ __launch_bounds__(kThreads) void select_kernel(
    const float* __restrict__ gate, int n_rows, int k_rows, uint8_t* __restrict__ mask,
    int32_t* __restrict__ idx, int32_t* __restrict__ rank, const int4* __restrict__ seg,
    int idx_cap, int32_t* __restrict__ nidx, int nidx_cap) {
  __shared__ uint32_t hist[4096];
  __shared__ uint32_t scan_ws[kWaves + 1];
  __shared__ uint32_t s_digit, s_before;

  const int b = blockIdx.x;
  const int t = threadIdx.x;
  int start, n, k, koff;
  if (SEG) {
    const int4 sg = seg[b];
    start = sg.x;
    n = sg.y;
    k = sg.z;
    koff = sg.w;
  } else {
    start = b * n_rows;
    n = n_rows;
    k = k_rows;
    koff = b * k_rows;
  }
  const int pos_add = SEG ? start : 0;    // idx values: absolute or within the row
  const int rank_add = SEG ? koff : 0;    // rank values: into the concatenation or the row
  const float* g = gate + (size_t)start;
  uint8_t* mrow = mask + (size_t)start;
  int32_t* rrow = rank + (size_t)start;
  int32_t* irow = idx ? idx + (size_t)koff : nullptr;
  // unselected tokens before this row / example: its first entry of nidx
  const long long nbase = SEG ? (long long)start - koff : (long long)b * (n_rows - k_rows);
  int32_t* nrow = nidx && nbase >= 0 ? nidx + nbase : nullptr;
  const int icap = SEG ? idx_cap - koff : k;  // entries of irow that may be written
  const long long ncap = SEG ? nidx_cap - nbase : n_rows - k_rows;  // of nrow

  // This thread's positions c * kChunk + t * kItems + j, as order images,
  // read once (every radix pass and the compaction use them); longer
  // sequences stream the logits from memory in each pass instead.
  const bool vec = (n % 4) == 0 && (start % 4) == 0;
  auto load_chunk = [&](int p0, uint32_t* img) {
    if (vec && p0 + kItems <= n) {
      const float4* src = reinterpret_cast<const float4*>(g + p0);
      const float4 a = src[0], c = src[1];
      img[0] = order_image(a.x); img[1] = order_image(a.y);
      img[2] = order_image(a.z); img[3] = order_image(a.w);
      img[4] = order_image(c.x); img[5] = order_image(c.y);
      img[6] = order_image(c.z); img[7] = order_image(c.w);
    } else {
#pragma unroll
      for (int j = 0; j < kItems; ++j) img[j] = (p0 + j < n) ? order_image(g[p0 + j]) : 0u;
    }
  };
  const bool in_regs = n <= kRegChunks * kChunk;
  uint32_t reg[kRegChunks][kItems];
  if (in_regs) {
#pragma unroll
    for (int c = 0; c < kRegChunks; ++c) {
      if (c * kChunk >= n) break;
      load_chunk(c * kChunk + t * kItems, reg[c]);
    }
  }

  uint32_t T;        // threshold image
  uint32_t need;     // ties at T to take
  if (k == 0) {
    T = 0xffffffffu;  // no finite or infinite logit has this image
    need = 0;
  } else {
    uint32_t prefix = 0, pmask = 0, remaining = (uint32_t)k;
#pragma unroll 1
    for (int pass = 0; pass < 3; ++pass) {
      const int bits = pass == 0 ? 12 : 10;
      const int shift = pass == 0 ? 20 : (pass == 1 ? 10 : 0);
      const int nb = 1 << bits;
      for (int i = t; i < nb; i += kThreads) hist[i] = 0;
      __syncthreads();
      if (in_regs) {
#pragma unroll
        for (int c = 0; c < kRegChunks; ++c) {
          if (c * kChunk >= n) break;
#pragma unroll
          for (int j = 0; j < kItems; ++j) {
            const uint32_t u = reg[c][j];
            if (c * kChunk + t * kItems + j < n && (u & pmask) == prefix)
              atomicAdd(&hist[(u >> shift) & (nb - 1)], 1u);
          }
        }
      } else {
        for (int i = t; i < n; i += kThreads) {
          uint32_t u = order_image(g[i]);
          if ((u & pmask) == prefix) atomicAdd(&hist[(u >> shift) & (nb - 1)], 1u);
        }
      }
      __syncthreads();
      // Thread t owns bins_per descending digits starting at nb-1-t*bins_per.
      const int per = nb / kThreads;  // 4 or 1
      uint32_t local = 0;
      for (int j = 0; j < per; ++j) local += hist[nb - 1 - (t * per + j)];
      uint32_t tot;
      uint32_t before = block_exclusive_scan(local, scan_ws, &tot);
      for (int j = 0; j < per; ++j) {
        const int digit = nb - 1 - (t * per + j);
        const uint32_t c = hist[digit];
        if (before < remaining && remaining <= before + c) {
          s_digit = (uint32_t)digit;
          s_before = before;
        }
        before += c;
      }
      __syncthreads();
      remaining -= s_before;
      prefix |= s_digit << shift;
      pmask |= (uint32_t)(nb - 1) << shift;
      __syncthreads();
    }
    T = prefix;
    need = remaining;
  }

  // Compaction in position order.
  uint32_t carry_gt = 0, carry_tie = 0;
  auto compact = [&](int base, const uint32_t* img) {
    const int p0 = base + t * kItems;
    uint32_t ngt = 0, ntie = 0;
#pragma unroll
    for (int j = 0; j < kItems; ++j) {
      const bool in = p0 + j < n;
      ngt += (in && img[j] > T) ? 1u : 0u;
      ntie += (in && img[j] == T) ? 1u : 0u;
    }
    uint32_t tot;
    const uint32_t ex = block_exclusive_scan(ngt | (ntie << 16), scan_ws, &tot);
    uint32_t gt_before = carry_gt + (ex & 0xffffu);
    uint32_t tie_before = carry_tie + (ex >> 16);
    uint8_t mv[kItems];
    int32_t rv[kItems];
#pragma unroll
    for (int j = 0; j < kItems; ++j) {
      const bool gt = img[j] > T;
      const bool tie = img[j] == T;
      const bool sel = gt || (tie && tie_before < need);
      const uint32_t r = gt_before + (tie_before < need ? tie_before : need);
      mv[j] = sel ? 1 : 0;
      rv[j] = sel ? (int32_t)r + rank_add : -1;
      if (sel && p0 + j < n && (int)r < icap) irow[r] = p0 + j + pos_add;
      // unselected: p - r tokens before it are unselected too (r of them are selected)
      if (!sel && nrow && p0 + j < n && p0 + j - (int)r < ncap)
        nrow[p0 + j - (int)r] = p0 + j + pos_add;
      gt_before += gt ? 1u : 0u;
      tie_before += tie ? 1u : 0u;
    }
    if (vec && p0 + kItems <= n) {
      // rows start 4-byte aligned (n % 4 == 0) and p0 % 8 == 0
      uint32_t* md = reinterpret_cast<uint32_t*>(mrow + p0);
      md[0] = mv[0] | (mv[1] << 8) | (mv[2] << 16) | ((uint32_t)mv[3] << 24);
      md[1] = mv[4] | (mv[5] << 8) | (mv[6] << 16) | ((uint32_t)mv[7] << 24);
      int4* rd = reinterpret_cast<int4*>(rrow + p0);
      rd[0] = make_int4(rv[0], rv[1], rv[2], rv[3]);
      rd[1] = make_int4(rv[4], rv[5], rv[6], rv[7]);
    } else {
#pragma unroll
      for (int j = 0; j < kItems; ++j) {
        if (p0 + j < n) {
          mrow[p0 + j] = mv[j];
          rrow[p0 + j] = rv[j];
        }
      }
    }
    carry_gt += tot & 0xffffu;
    carry_tie += tot >> 16;
  };
  if (in_regs) {
#pragma unroll
    for (int c = 0; c < kRegChunks; ++c) {
      if (c * kChunk >= n) break;
      compact(c * kChunk, reg[c]);
    }
  } else {
#pragma unroll 1
    for (int base = 0; base < n; base += kChunk) {
      uint32_t img[kItems];
      load_chunk(base + t * kItems, img);
      compact(base, img);
    }
  }
}

}  // namespace

hipError_t launch_select(const Dims& d, const float* gate, uint8_t* mask,
                         int32_t* idx, int32_t* rank, hipStream_t s, int32_t* nidx) {
  if (d.B == 0 || d.n == 0) return hipSuccess;
  hipLaunchKernelGGL(select_kernel<false>, dim3(d.B), dim3(kThreads), 0, s, gate, d.n, d.k, mask,
                     idx, rank, nullptr, 0, nidx, 0);
  return hipGetLastError();
}

hipError_t launch_select_segments(int n_segments, const int4* seg, const float* gate,
                                  uint8_t* mask, int32_t* idx, int32_t* rank, int idx_cap,
                                  hipStream_t s, int32_t* nidx, int nidx_cap) {
  if (n_segments == 0) return hipSuccess;
  hipLaunchKernelGGL(select_kernel<true>, dim3(n_segments), dim3(kThreads), 0, s, gate, 0, 0,
                     mask, idx, rank, seg, idx_cap, nidx, nidx_cap);
  return hipGetLastError();
}

namespace {

// Per-example table {start, length, k_e = ceil(rho * length), offset of the
// example's selection} from cu_seqlens, and every token's example start.
// One workgroup scans the examples in order (offsets need a prefix sum);
// tokens are filled by every thread.
// Offsets are clamped into [0, T] (each at or after the previous one), so
// inconsistent offsets cannot address outside the token arrays.
__global__ __launch_bounds__(kThreads) void varlen_prep_kernel(const int32_t* __restrict__ cu,
                                                               int E, int T, double rho,
                                                               int4* __restrict__ seg,
                                                               int32_t* __restrict__ seg_start) {
  __shared__ uint32_t scan_ws[kWaves + 1];
  const int t = threadIdx.x;
  uint32_t carry = 0;
  for (int base = 0; base < E; base += kThreads) {
    const int e = base + t;
    int a = 0, len = 0, k = 0;
    if (e < E) {
      a = min(max(cu[e], 0), T);
      len = min(max(cu[e + 1], a), T) - a;
      const double kk = ceil(rho * (double)len);
      k = (int)min(max(kk, 0.0), (double)len);
    }
    uint32_t tot;
    const uint32_t before = block_exclusive_scan((uint32_t)k, scan_ws, &tot);
    if (e < E) seg[e] = make_int4(a, len, k, (int)(carry + before));
    carry += tot;
    for (int e2 = base; e2 < min(base + kThreads, E); ++e2) {
      const int a2 = min(max(cu[e2], 0), T), b2 = min(max(cu[e2 + 1], a2), T);
      for (int i = a2 + t; i < b2; i += kThreads) seg_start[i] = a2;
    }
  }
}

}  // namespace

hipError_t launch_varlen_prep(const int32_t* cu, int E, int T, double rho, int4* seg,
                              int32_t* seg_start, hipStream_t s) {
  if (E == 0) return hipSuccess;
  hipLaunchKernelGGL(varlen_prep_kernel, dim3(1), dim3(kThreads), 0, s, cu, E, T, rho, seg,
                     seg_start);
  return hipGetLastError();
}

}  // namespace logo
