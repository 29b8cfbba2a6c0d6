// Internal definitions shared by the host API and the kernels of libspava.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/spava.h"

namespace spava {

constexpr int kKeyTile = 64;     // keys per LDS tile in the attention kernels
constexpr int kQTile = 256;      // queries per attention workgroup (8 waves x 32)
// Key splits of the row-statistics pass: one wave per (pair, 32 observer rows, split),
// all of about the same cost. The waves resident on a SIMD share its matrix unit, so
// the pass takes about ceil(waves / kScoreWaveSlots) * (split + kScoreWaveOverhead)
// key steps, kScoreWaveSlots = 256 CUs x 4 SIMDs (a fit to timings of split lengths
// 512..2048 at 16384 keys per block). The split length, a multiple of 32 in
// [kScoreSplitMin, kScoreSplitMax], minimises that estimate (ties: the longer). A
// launch with more waves than kScoreWaveSlots (bf16) uses the build capped at two waves
// per SIMD.
constexpr int kScoreSplitMin = 512;
constexpr int kScoreSplitMax = 4096;
constexpr int kScoreWaveSlots = 1024;
constexpr int kScoreWaveOverhead = 32;
// The score pass keeps the float64 logits of the row-statistics pass when one
// (block, KV head) pair's logits fit in kLogitPairBytes; pairs are then processed in
// chunks of at most kLogitChunkBytes of logits. Otherwise the logits are recomputed.
constexpr int64_t kLogitPairBytes = int64_t(512) << 20;
constexpr int64_t kLogitChunkBytes = int64_t(4) << 30;

inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline int64_t round_up(int64_t a, int64_t b) { return cdiv(a, b) * b; }

// Everything the kernels need about one call, derived on the host from spava_shape.
struct Plan {
  int64_t N;
  int H, Hq, Hkv, G, D, A, l, w;
  int nb;           // block length N / H
  int dtype;        // spava_dtype
  double scale;     // logit scale
  int64_t qs_tok, qs_head, kvs_tok, kvs_head, os_tok, os_head;
  int l0, l1;       // rows passed by block 0 and by each block j >= 1
  int Lmax;         // non-local (anchor + passing) rows of the last block
  int Lpad;         // Lmax rounded up to a key tile
  int R;            // observer rows per (block, KV head): G * w
  int split_keys;   // keys per split of the row-statistics pass
  int KS;           // key splits of the row-statistics pass: ceil(nb / split_keys)
  int T;            // query tiles per block
  int loc_tiles;    // key tiles per block
  int sched;        // query-tile dispatch order (ScheduleMode); never changes results
  int obs_query;    // selection observers: 0 = last w queries of each block,
                    // 1 = the w rows of a query block (every key visible)
  int recompute_logits;  // the caller asked for SPAVA_LOGITS_RECOMPUTE
  int store_logits; // 1: the score pass reads stored logits instead of recomputing
  int pair_chunk;   // (block, KV head) pairs per chunk when logits are stored
};

// The selection's key splits and whether it stores its logits (after R is final).
void set_select_layout(Plan* p);

// Dispatch order of the (block, query tile) pairs of the attention grid (the values
// of spava_schedule).
enum ScheduleMode {
  kSchedLongestFirst = SPAVA_SCHED_LONGEST_FIRST,
  kSchedNatural = SPAVA_SCHED_NATURAL,
  kSchedZigZag = SPAVA_SCHED_ZIGZAG
};

// Non-local prefix length of block h: anchor + passing rows of blocks 0..h-1.
__host__ __device__ inline int prefix_len(const Plan& p, int h) {
  return h == 0 ? 0 : p.A + p.l0 + (h - 1) * p.l1;
}

// Source token of prefix row r for KV head g: the anchor rows [0, A), then the passing
// rows of blocks 0, 1, ... in block order (explainer "APB-V: ...", Berechnung: the
// anchor and the aggregated passing blocks). -1 for padding rows past Lmax and for an
// index outside its block's candidates (block j's rows, minus the anchor for j = 0),
// so a bad index reads as a zero row and never out of bounds.
__device__ inline int64_t prefix_source(const Plan& p, const int32_t* idx, int g, int r) {
  if (r < p.A) return r;
  if (r >= p.Lmax) return -1;
  int rr = r - p.A;
  int j, t;
  if (rr < p.l0) {
    j = 0;
    t = rr;
  } else {
    rr -= p.l0;
    j = 1 + rr / p.l1;
    t = rr % p.l1;
  }
  const int64_t src = idx[(static_cast<int64_t>(j) * p.Hkv + g) * p.l + t];
  const int64_t s = static_cast<int64_t>(j) * p.nb;
  const int64_t lo = j == 0 ? s + p.A : s;
  return (src >= lo && src < s + p.nb) ? src : -1;
}

// Workspace carving (byte offsets, 256-byte aligned regions).
struct SelectWs {
  size_t rowstat_part, rowstat, scores, logits, total;
};
struct AttnWs {
  size_t kpre, vpre, vtloc, order, order2, total;
};

// Workspace of the overlapped layer: the selection's and the attention's.
struct OverlapWs {
  size_t select, attn, total;
};

struct QueryWs {
  size_t part_o, part_lse, vtctx, vtq, total;
};

SelectWs select_ws_layout(const Plan& p);
AttnWs attn_ws_layout(const Plan& p);
QueryWs query_ws_layout(const Plan& p, int64_t nq);
OverlapWs overlap_ws_layout(const Plan& p);

// Kernel launchers (defined next to their kernels). They return hipSuccess or the
// launch error.
hipError_t launch_select(const Plan& p, const void* q, const void* k, int32_t* idx,
                         double* scores, char* ws, hipStream_t st);
hipError_t launch_attn_bf16(const Plan& p, const void* q, const void* k, const void* v,
                            const int32_t* idx, void* out, float* lse, char* ws,
                            hipStream_t st);
// The bf16 attention in two launches (the overlapped layer): block 0, which sees no
// passing rows (also gathers the anchor tiles and every block's local V^T), then the
// other blocks (gathers the passing rows first). Together they compute exactly what
// launch_attn_bf16 computes.
hipError_t launch_attn_bf16_block0(const Plan& p, const void* q, const void* k, const void* v,
                                   void* out, float* lse, char* ws, hipStream_t st);
hipError_t launch_attn_bf16_rest(const Plan& p, const void* q, const void* k, const void* v,
                                 const int32_t* idx, void* out, float* lse, char* ws,
                                 hipStream_t st);
hipError_t launch_attn_f32(const Plan& p, const void* q, const void* k, const void* v,
                           const int32_t* idx, void* out, float* lse, char* ws,
                           hipStream_t st);
hipError_t launch_query(const Plan& p, int64_t nq, const void* q_qr, const void* k_qr,
                        const void* v_qr, const void* k, const void* v, void* out, float* lse,
                        char* ws, hipStream_t st);

}  // namespace spava
