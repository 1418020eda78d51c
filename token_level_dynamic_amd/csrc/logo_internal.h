// Internal interface between the C ABI (abi.cpp) and the HIP kernels.
// gfx950 (CDNA4) only.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace logo {

// Element strides of one [B][H][n][d] tensor view (d stride 1). The host
// has checked that ((n-1) * st + d) elements of one (b, h) fit in 2^31
// bytes, so per-sequence offsets fit 32-bit arithmetic.
struct View {
  long long sb, sh;  // batch, head
  int st;            // token
};

// Validated problem, as the kernels see it.
struct Dims {
  int B, Hq, Hkv, n, d, window;
  int k;          // selected tokens per sequence
  float scale;    // score scale
  int dtype;      // 0 f32, 1 bf16 (for q, k, v, o)
  View vq, vk, vv, vo;  // layouts of the caller's q, k, v and o
};

// What the attention kernels write for each row they finish.
enum class Epi : int {
  LocalAll = 0,    // o_local[b][h][i][:] (f32) for every row
  LocalFused = 1,  // rank[i] >= 0: scratch[b][h][rank][:] (f32); else o (io dtype)
  GlobalAll = 2,   // o_global[b][h][r][:] (f32), r = row in idx
  GlobalFused = 3,  // o = scratch[b][h][r] + sigmoid(gate) * o_global (io dtype)
  LocalRouted = 4,  // o_local[b][h][i][:] (f32) and o (io dtype) for every row, and
                    // router_part[b][h][i] = <router_w[h], o_local row>
  GlobalRouted = 5  // o = scratch[b][h][i] + sigmoid(gate) * o_global (io dtype)
};

struct AttnArgs {
  const void* q;
  const void* k;
  const void* v;
  const int32_t* idx;    // global branch rows [B][k]
  const int32_t* rank;   // fused local: [B][n]
  const float* gate;     // fused global: [B][n]
  float* out_f32;        // o_local / o_global / scratch (fused local)
  const float* scratch;  // fused global: local outputs of selected rows
  void* out_io;          // fused: final output o
  float* lse_out;        // optional: natural-log log-sum-exp of each row's
                         // scaled scores (local [B][Hq][n], global [B][Hq][k])
  float* og_out;         // optional, fused global: o_global [B][Hq][k][d] f32
  const float* router_w; // routed local: [Hq][d] f32
  float* router_part;    // routed local: [B][Hq][n] f32
  const int32_t* seg_start;  // packed examples: first token of each token's
                             // example (keys before it are masked); or NULL
  int32_t* sched;        // bf16 global branch: workspace of attn_bf16_sched_ints()
                         // ints for the workgroup queues (and, for packed examples,
                         // the work order), or NULL for the static order
  float* split_part;     // bf16 fused global branch: attn_bf16_split_floats() floats
                         // for the key-range partials of a small problem, or NULL
                         // (no split)
};

// Everything the backward kernels read and write. q, k, v, o and dout are
// the caller's (views as in Dims; dout has o's strides); lse_*, o_*_sel,
// o_global come from the training forward; the rest is workspace or output.
struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const float* gate;      // [B][n]
  const void* o;          // forward output (io dtype)
  const void* dout;       // upstream gradient of o (io dtype)
  const int32_t* idx;     // [B][k]
  const int32_t* rank;    // [B][n]
  const float* lse_l;     // [B][Hq][n]   natural log
  const float* lse_g;     // [B][Hq][k]
  const float* o_ls;      // [B][Hq][k][d] local output of the selected rows
  const float* o_g;       // [B][Hq][k][d] global output of the selected rows
  float* dq;              // [B][Hq][n][d]
  float* dk;              // [B][Hkv][n][d]
  float* dv;              // [B][Hkv][n][d]
  float* dgate;           // [B][n]
  // workspace
  float* D_l;             // [B][Hq][n]   <do_i, o_local_i>
  float* D_g;             // [B][Hq][k]   g_i <do_i, o_global_i>
  float* L2_l;            // [B][Hq][n]   lse_local * log2(e)
  float* L2_g;            // [B][Hq][k]   lse_global * log2(e)
  void* qs;               // [B][Hq][k][d] io dtype: q of the selected rows
  void* dog;              // [B][Hq][k][d] io dtype: g_i do_i of the selected rows
};

// Backward workspace: offsets (bytes, 256-aligned) of D_l, D_g, L2_l, L2_g,
// qs, dog and the total.
struct BwdWorkspace {
  size_t D_l, D_g, L2_l, L2_g, qs, dog, total;
};
BwdWorkspace bwd_workspace(const Dims& d);

hipError_t launch_bwd_prep(const Dims& d, const BwdArgs& a, hipStream_t s);
hipError_t launch_bwd_dkdv_bf16(const Dims& d, const BwdArgs& a, hipStream_t s);
hipError_t launch_bwd_dq_bf16(const Dims& d, bool global, const BwdArgs& a, hipStream_t s);
hipError_t launch_bwd_dkdv_f32(const Dims& d, const BwdArgs& a, hipStream_t s);
hipError_t launch_bwd_dq_f32(const Dims& d, bool global, const BwdArgs& a, hipStream_t s);

// nidx (optional, [B][n-k]): the unselected positions of each row, ascending.
hipError_t launch_select(const Dims& d, const float* gate, uint8_t* mask,
                         int32_t* idx, int32_t* rank, hipStream_t s, int32_t* nidx = nullptr);

// Packed examples: select per example (see select.hip) and build the
// per-example table and per-token example starts from cu_seqlens. nidx
// (optional, nidx_cap entries): the unselected positions of the stream,
// ascending.
hipError_t launch_select_segments(int n_segments, const int4* seg, const float* gate,
                                  uint8_t* mask, int32_t* idx, int32_t* rank, int idx_cap,
                                  hipStream_t s, int32_t* nidx = nullptr, int nidx_cap = 0);
hipError_t launch_varlen_prep(const int32_t* cu, int E, int T, double rho, int4* seg,
                              int32_t* seg_start, hipStream_t s);

// Ints of workspace the bf16 global branch uses for its workgroup queues
// (one counter per (b, kv head)) and, for packed examples, the work order.
size_t attn_bf16_sched_ints(const Dims& d, bool packed);
// Key ranges the bf16 fused global branch splits each row block into (1: no
// split; more when the problem has fewer than 512 row-block workgroups), and
// the float32 partials that takes: splits * B * Hq * k * (d + 4), or 0.
int attn_bf16_splits(const Dims& d);
// The single-launch fused bf16 forward: selected rows compute both
// branches, unselected rows (nidx [B][n-k], ascending) the local one; a
// kernel of its own writes o. Applies when attn_bf16_fused_ok(d). Packed
// examples (a.seg_start set, B = 1): a.sched holds the work order the
// launch computes first (attn_bf16_sched_ints(d, true) ints).
bool attn_bf16_fused_ok(const Dims& d);
hipError_t launch_attn_bf16_fused(const Dims& d, const AttnArgs& a, const int32_t* nidx,
                                  hipStream_t s);
size_t attn_bf16_split_floats(const Dims& d);
// Problems whose global branch is split over key ranges (attn_bf16_splits(d)
// > 1): the split global branch and the local band in one launch, then the
// merge (a.split_part, a.scratch and a.out_f32 as for the two launches).
bool attn_bf16_pair_ok(const Dims& d);
hipError_t launch_attn_bf16_pair(const Dims& d, const AttnArgs& a, hipStream_t s);
hipError_t launch_attn_bf16(const Dims& d, Epi epi, const AttnArgs& a,
                            hipStream_t s);

hipError_t launch_attn_f32(const Dims& d, Epi epi, const AttnArgs& a,
                           hipStream_t s);

// gate[b][i] = bias + sum_h part[b][h][i] (heads summed in order).
hipError_t launch_router_sum(const Dims& d, const float* part, float bias, float* gate,
                             hipStream_t s);

// ---- threshold controller and decode step --------------------------------
struct DecodeDims {
  int B, Hq, Hkv, cap, d, window;
  double rho;
  float eta;
  float scale;
  int dtype;
};
struct DecodeArgs {
  const void* q;          // [B][Hq][d]
  const void* k_cache;    // [B][Hkv][cap][d]
  const void* v_cache;
  const int32_t* lens;    // [B]
  const float* gate;      // [B]
  const uint8_t* selected;
  float* part;            // workspace: chunk partials
  void* o;                // [B][Hq][d]
};
// query heads per kv head the decode step supports for this problem: up to
// 16 for bf16 caches of at most 1023 sequences, else 1, 2, 4, 7 or 8
bool decode_group_supported(const DecodeDims& d);
// chunk partials per cache of `cap` positions
int64_t decode_chunks(int64_t cap);
size_t decode_partial_bytes(const DecodeDims& d);
hipError_t launch_decode_ctrl(const DecodeDims& d, const float* gate, float* tau,
                              uint8_t* selected, hipStream_t s);
hipError_t launch_decode(const DecodeDims& d, const DecodeArgs& a, hipStream_t s);
hipError_t launch_calibrate(const Dims& d, const float* gate, const uint8_t* mask, float* tau,
                            hipStream_t s);
hipError_t launch_select_threshold(const Dims& d, const float* gate, const float* tau,
                                   uint8_t* mask, int32_t* idx, int32_t* count, hipStream_t s);

hipError_t launch_combine(const Dims& d, const float* o_local,
                          const float* o_global, const int32_t* rank,
                          const float* gate, void* o, hipStream_t s);

}  // namespace logo
