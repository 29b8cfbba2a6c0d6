// Approximate attention, bf16 inputs: gather + schedule + MFMA flash attention.
//
// Method (explainer "APB-V: ...", Methodik > Approximativer Attention-Mechanismus >
// Berechnung; abstract of "Spava: ..."): queries of context block h attend to the
// anchor block, the aggregated passing blocks of blocks 0..h-1 and their own causal
// local context. On one GPU all H blocks run in one grid; the pages' load balancing
// ("Systemseitige Optimierungen": ZigZag pairing so every host carries the same
// passing length) becomes a longest-first order of the query tiles.
//
// Kernels:
//   prep       gathers anchor + passing rows of every KV head into a contiguous
//              prefix (K row-major, V transposed into MFMA-ready tiles) and
//              transposes each block's local V into the same tile format;
//   schedule   orders the (block, query tile) pairs (longest first by default);
//   attention  one workgroup = 256 queries x 1 query head = 8 waves x 32 queries
//              (2 waves per SIMD). K/V tiles of 64 keys go through a three-stage
//              LDS ring, loaded two tiles ahead;
//              each tile is one flash step (attn_common.h): S^T = K Q^T and
//              O^T += V^T P^T on v_mfma_f32_32x32x16_bf16 with float32 accumulators
//              and an online softmax in float32 with exp2 and a folded scale.
//
// A launch covers a range of blocks. The overlapped layer (the one-GPU form of the
// pages' overlap of passing-block transfers with compute, "Systemseitige
// Optimierungen") runs block 0, which sees no passing rows, while the selection runs
// on another stream, and the other blocks after it; every query is computed exactly
// as in a launch over all blocks.
#include "attn_common.h"

namespace spava {
namespace {

// Whole anchor tiles: prefix tiles [0, A / 64) hold anchor rows only.
__host__ __device__ inline int anchor_tiles(const Plan& p) { return p.A / BN; }

// Key tiles of work item `pair` (= block * T + query tile): the block's prefix tiles,
// then its local tiles up to the last query of the tile.
__device__ inline int pair_cost(const Plan& p, int pair) {
  const int h = pair / p.T, t = pair % p.T;
  const int loc = min(p.nb, (t + 1) * kQTile);
  return (prefix_len(p, h) + BN - 1) / BN + (loc + BN - 1) / BN;
}

// order[rank] = pair for the pairs [pair0, pair0 + npairs) (whole blocks). Longest
// first: pairs ranked by decreasing key-tile count, ties by pair index. Natural:
// block-major. ZigZag: the range's blocks paired as (first + i, last - i), the pages'
// host pairing, tiles of a pair alternating.
// One 256-pair chunk of the ranking, by one workgroup of 256 threads (cost: LDS).
__device__ inline void schedule_chunk(const Plan& p, int32_t* __restrict__ order, int pair0,
                                      int npairs, int chunk, int* cost) {
  const int P = npairs;
  const int i = chunk * 256 + static_cast<int>(threadIdx.x);   // pair pair0 + i
  const bool valid = i < P;
  int rank = 0;
  if (p.sched == kSchedNatural) {
    rank = i;
  } else if (p.sched == kSchedZigZag) {
    const int nh = P / p.T;
    const int h = i / p.T, t = i % p.T;
    const int mirror = nh - 1 - h;
    const int pr = min(h, mirror);
    rank = (h == mirror) ? pr * 2 * p.T + t : pr * 2 * p.T + 2 * t + (h > mirror ? 1 : 0);
  } else {
    // Rank = number of pairs that come first (higher cost, or equal cost and lower
    // index); the costs of each chunk of 256 pairs are computed once into LDS (slots
    // past P hold -1, which never counts: costs are >= 0) and read 4 at a time.
    const int ci = valid ? pair_cost(p, pair0 + i) : 0;
    for (int j0 = 0; j0 < P; j0 += 256) {
      __syncthreads();
      const int jt = j0 + static_cast<int>(threadIdx.x);
      cost[threadIdx.x] = jt < P ? pair_cost(p, pair0 + jt) : -1;
      __syncthreads();
      const int4* c4 = reinterpret_cast<const int4*>(cost);
#pragma unroll 8
      for (int q4 = 0; q4 < 64; ++q4) {
        const int4 c = c4[q4];
        const int jb = j0 + 4 * q4;
        rank += (c.x > ci) || (c.x == ci && jb < i);
        rank += (c.y > ci) || (c.y == ci && jb + 1 < i);
        rank += (c.z > ci) || (c.z == ci && jb + 2 < i);
        rank += (c.w > ci) || (c.w == ci && jb + 3 < i);
      }
    }
  }
  if (valid) order[rank] = pair0 + i;
}

// grid.x: prefix tiles [t0, t1), then (with_local) H*loc_tiles local V tiles, then
// ceil(npairs / 256) workgroups that rank the work items of the attention launch that
// follows (at grid.y == 0); grid.y: KV head.
template <int D>
__global__ __launch_bounds__(256) void prep_kernel(Plan p, const uint16_t* __restrict__ k,
                                                   const uint16_t* __restrict__ v,
                                                   const int32_t* __restrict__ idx,
                                                   uint16_t* __restrict__ kpre,
                                                   uint16_t* __restrict__ vtpre,
                                                   uint16_t* __restrict__ vtloc, int t0, int t1,
                                                   int with_local, int32_t* __restrict__ order,
                                                   int pair0, int npairs) {
  __shared__ __attribute__((aligned(16))) uint16_t Vs[BN][D + 8];
  __shared__ int64_t src_tok[BN];
  __shared__ __attribute__((aligned(16))) int cost[256];
  const int ngather = (t1 - t0) + (with_local ? p.H * p.loc_tiles : 0);
  if (static_cast<int>(blockIdx.x) >= ngather) {
    if (blockIdx.y == 0) schedule_chunk(p, order, pair0, npairs, blockIdx.x - ngather, cost);
    return;
  }
  const int g = blockIdx.y;
  const int tid = threadIdx.x;
  const int npre_tiles = p.Lpad / BN;
  const bool is_prefix = static_cast<int>(blockIdx.x) < t1 - t0;
  int tile, h = 0;
  if (is_prefix) {
    tile = t0 + blockIdx.x;
  } else {
    const int lt = blockIdx.x - (t1 - t0);
    h = lt / p.loc_tiles;
    tile = lt % p.loc_tiles;
  }
  if (tid < BN) {
    if (is_prefix) {
      src_tok[tid] = prefix_source(p, idx, g, tile * BN + tid);
    } else {
      const int off = tile * BN + tid;
      src_tok[tid] = off < p.nb ? static_cast<int64_t>(h) * p.nb + off : -1;
    }
  }
  __syncthreads();
  constexpr int CPR = D / 8;  // 16-byte chunks per row
  for (int c = tid; c < BN * CPR; c += 256) {
    const int row = c / CPR, col = c % CPR;
    const int64_t tok = src_tok[row];
    const int64_t off = tok * p.kvs_tok + g * p.kvs_head + col * 8;
    uint4 vv = make_uint4(0, 0, 0, 0);
    if (tok >= 0) vv = *reinterpret_cast<const uint4*>(v + off);
    *reinterpret_cast<uint4*>(&Vs[row][col * 8]) = vv;
    if (is_prefix) {
      uint4 kk = make_uint4(0, 0, 0, 0);
      if (tok >= 0) kk = *reinterpret_cast<const uint4*>(k + off);
      *reinterpret_cast<uint4*>(kpre + (static_cast<int64_t>(g) * p.Lpad + tile * BN + row) * D +
                                col * 8) = kk;
    }
  }
  __syncthreads();
  uint16_t* dst;
  if (is_prefix)
    dst = vtpre + (static_cast<int64_t>(g) * npre_tiles + tile) * D * BN;
  else
    dst = vtloc + ((static_cast<int64_t>(g) * p.H + h) * p.loc_tiles + tile) * D * BN;
  store_vt_tile<D>(Vs, dst);
}

// NG = (pairs in `order`) x Hkv work groups of G workgroups (one per query head).
// LSE: write the log-sum-exp (the caller asked for it), which adds the float32 sum of
// the weights to every tile step.
template <int D, bool LSE>
__global__ __launch_bounds__(kThreads) void attn_kernel(
    Plan p, const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ kpre, const uint16_t* __restrict__ vtpre,
    const uint16_t* __restrict__ vtloc, const int32_t* __restrict__ order,
    uint16_t* __restrict__ out, float* __restrict__ lse, int NG, float c_log2) {
  using C = Cfg<D>;
  __shared__ __attribute__((aligned(16))) char smem[3 * C::STAGE];

  // Work item: XCD-aware mapping so the G heads of one KV group run back to back
  // on one XCD (consecutive workgroup ids are spread round-robin over 8 XCDs).
  const int b = blockIdx.x;
  const int xcd = b & 7, slot = b >> 3;
  const int gs = (slot / p.G) * 8 + xcd;
  if (gs >= NG) return;
  const int hl = slot % p.G;
  const int rank = gs / p.Hkv, g = gs % p.Hkv, hq = g * p.G + hl;
  const int pair = order[rank];
  const int h = pair / p.T, t = pair % p.T;

  const int64_t s_h = static_cast<int64_t>(h) * p.nb;
  const int64_t e_h = s_h + p.nb;
  const int64_t q0 = s_h + static_cast<int64_t>(t) * kQTile;
  const int64_t q_end = min(q0 + kQTile, e_h);
  const int L = prefix_len(p, h);
  const int np = (L + BN - 1) / BN;                                  // prefix tiles
  const int nloc = static_cast<int>((q_end - s_h + BN - 1) / BN);   // local tiles
  const int ntiles = np + nloc;

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int lr = lane & 31, lh = lane >> 5;
  const int64_t qw0 = q0 + static_cast<int64_t>(kWaveQ) * w;   // first query of this wave
  const bool wave_active = qw0 < e_h;
  const int64_t qi = qw0 + lr;                                  // this lane's query

  const uint16_t* kpre_g = kpre + static_cast<int64_t>(g) * p.Lpad * D;
  const uint16_t* vtpre_g = vtpre + static_cast<int64_t>(g) * (p.Lpad / BN) * D * BN;
  const uint16_t* vtloc_gh = vtloc + (static_cast<int64_t>(g) * p.H + h) * p.loc_tiles * D * BN;
  const uint16_t* k_g = k + g * p.kvs_head;

  // Tile it: prefix tiles come from the gathered Kpre/Vtpre, local tiles read K in
  // place and V^T from the block's transposed tiles.
  TileDma<D> dma;
  dma.init(p.kvs_tok);
  // Per-workgroup tile bases and K ranges, so issuing a tile is a few scalar adds:
  // full local tiles share one range; only a block's last tile can be partial.
  const uint16_t* kpre0 = kpre_g;
  const uint16_t* vpre0 = vtpre_g;
  const uint16_t* kloc0 = k_g + s_h * p.kvs_tok;
  const int64_t kloc_step = static_cast<int64_t>(BN) * p.kvs_tok;
  const int kbytes_pre = TileDma<D>::k_range(BN, D);
  const int kbytes_loc = TileDma<D>::k_range(BN, p.kvs_tok);
  const int lt_part = (p.nb % BN) != 0 ? p.nb / BN : -1;     // partial local tile
  const int kbytes_part = TileDma<D>::k_range(p.nb % BN, p.kvs_tok);
  auto issue_tile = [&](int it, char* dst) {
    if (it < np) {
      dma.issue(kpre0 + static_cast<int64_t>(it) * BN * D, false, kbytes_pre,
                vpre0 + static_cast<int64_t>(it) * D * BN, dst);
    } else {
      const int lt = it - np;
      dma.issue(kloc0 + lt * kloc_step, true, lt == lt_part ? kbytes_part : kbytes_loc,
                vtloc_gh + static_cast<int64_t>(lt) * D * BN, dst);
    }
  };

  bf16x8 qf[C::DK];
  load_q<D>(q + qi * p.qs_tok + hq * p.qs_head + lh * 8, qi < e_h, qf);
  Flash<D> f;
  f.init();

  // Which tiles need a mask, decided once per wave so the tile loop only compares
  // indices: local tiles from it_diag on touch this wave's causal diagonal
  // (key0 + BN - 1 > qw0, i.e. (it - np) * BN > qw0 - s_h - BN + 1); the last prefix
  // tile (it_edge) is partial when the prefix length is not a multiple of BN; a wave
  // past the block end masks everything.
  const int64_t rel0 = qw0 - s_h;
  const int first_diag = rel0 >= BN - 1 ? static_cast<int>((rel0 - (BN - 1)) / BN) + 1 : 0;
  const int it_diag = np + first_diag;
  const int it_edge = (L % BN) != 0 ? np - 1 : -1;
  const int qrel = static_cast<int>(qi - s_h);   // this lane's query inside the block

  // Three LDS stages, tiles loaded one iteration ahead of their use: while tile it is
  // computed, tile it+1 is complete (its first K fragments go into registers during
  // tile it's P V) and tile it+2 is in flight into the stage tile it-1 used.
  if (ntiles > 0) issue_tile(0, smem);
  if (ntiles > 1) issue_tile(1, smem + C::STAGE);
  wait_tile_loads();
  __syncthreads();
  // Local tiles past this wave's last query are fully masked for it: the wave computes
  // tiles [0, it_end) and only loads its share of the rest, in a second, load-only loop
  // (chosen once per wave: a branch around the tile step inside one loop made the
  // compiler copy the O accumulators on every tile). A wave past the block end only
  // loads.
  const int64_t q_last = min(qw0 + kWaveQ, e_h) - 1;
  const int it_end = wave_active ? min(ntiles, np + static_cast<int>((q_last - s_h) / BN) + 1) : 0;
  int st = 0;   // stage of tile it
  if (it_end > 0) {
    KHead<D> kh;
    kh.read(smem);
    for (int it = 0; it < it_end; ++it) {
      const int st1 = st == 2 ? 0 : st + 1, st2 = st1 == 2 ? 0 : st1 + 1;
      if (it + 2 < ntiles) issue_tile(it + 2, smem + st2 * C::STAGE);
      // Last visible key of a masked tile: the prefix length in the partial prefix
      // tile, the causal diagonal in a local tile.
      const bool diag = it >= it_diag;
      const bool masked = diag || it == it_edge;
      auto lim_of = [&]() {
        int lim = BN - 1;
        if (it == it_edge) lim = L - it * BN - 1;
        if (diag) {
          const int rel = qrel - (it - np) * BN;      // integer select (no floating max)
          lim = rel < 0 ? -1 : rel;
        }
        return lim;
      };
      attend_tile<D, LSE>(kh, smem + st * C::STAGE,
                          it + 1 < ntiles ? smem + st1 * C::STAGE : nullptr, qf, f, masked, lim_of,
                          c_log2);
      wait_tile_loads();   // tile it+2, which the next iteration's P V reads K from
      __syncthreads();
      st = st1;
    }
  }
  for (int it = it_end; it < ntiles; ++it) {
    const int st1 = st == 2 ? 0 : st + 1, st2 = st1 == 2 ? 0 : st1 + 1;
    if (it + 2 < ntiles) issue_tile(it + 2, smem + st2 * C::STAGE);
    wait_tile_loads();
    __syncthreads();
    st = st1;
  }

  // ---- epilogue: normalise, round to bf16, write O and LSE. Each wave stages its 32
  // output rows in LDS (no wave reads a stage after the loop's last barrier) and then
  // stores whole rows, 16 bytes per lane: stored straight from the accumulator layout,
  // every store instruction would write 16 bytes into each of 32 rows (16K tokens:
  // the attention call 3% slower).
  const float ltot_b = flash_rowsum_b<D>(f);   // bf16 weights: normalises O
  constexpr int ORB = 2 * D + 16;              // bytes per staged row (padded)
  static_assert(kWaves * kWaveQ * ORB <= 3 * C::STAGE, "staged rows must fit the stages");
  char* ob = smem + w * (kWaveQ * ORB);
  const float cy = 1.f / ltot_b;
#pragma unroll
  for (int dm = 0; dm < C::DM; ++dm)
#pragma unroll
    for (int grp = 0; grp < 4; ++grp) {
      f32x2 lo = {f.o[dm][grp * 4 + 0] * cy, f.o[dm][grp * 4 + 1] * cy};
      f32x2 hi = {f.o[dm][grp * 4 + 2] * cy, f.o[dm][grp * 4 + 3] * cy};
      bf16x2 blo = __builtin_convertvector(lo, bf16x2);
      bf16x2 bhi = __builtin_convertvector(hi, bf16x2);
      uint2 pk;
      pk.x = __builtin_bit_cast(uint32_t, blo);
      pk.y = __builtin_bit_cast(uint32_t, bhi);
      *reinterpret_cast<uint2*>(ob + lr * ORB + out_dim<D>(dm, grp, lh) * 2) = pk;
    }
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): this wave's rows are in LDS
  __builtin_amdgcn_wave_barrier();
  constexpr int LPR = 2 * D / 16;       // lanes per row
  constexpr int RPS = 64 / LPR;         // rows per store
#pragma unroll
  for (int j = 0; j < kWaveQ / RPS; ++j) {
    const int row = j * RPS + lane / LPR, c16 = lane % LPR;
    const u32x4 v4 = *reinterpret_cast<const u32x4*>(ob + row * ORB + c16 * 16);
    const int64_t qrow = qw0 + row;
    if (qrow < e_h) *reinterpret_cast<u32x4*>(out + qrow * p.os_tok + hq * p.os_head + c16 * 8) = v4;
  }
  if (LSE) {
    const float ltot = flash_rowsum<D>(f);     // float32 weights: the LSE
    if (lh == 0 && qi < e_h)
      lse[static_cast<int64_t>(hq) * p.N + qi] = (f.mrun + log2f(ltot)) * 0.69314718055994531f;
  }
}

struct AttnPtrs {
  uint16_t *kpre, *vtpre, *vtloc;
  int32_t *order, *order2;
};
static AttnPtrs attn_ptrs(const Plan& p, char* ws) {
  const AttnWs w = attn_ws_layout(p);
  return {reinterpret_cast<uint16_t*>(ws + w.kpre), reinterpret_cast<uint16_t*>(ws + w.vpre),
          reinterpret_cast<uint16_t*>(ws + w.vtloc), reinterpret_cast<int32_t*>(ws + w.order),
          reinterpret_cast<int32_t*>(ws + w.order2)};
}

// Gather prefix tiles [t0, t1) (and, with_local, every block's local V^T tiles), and
// rank the work items of blocks [h0, h1) into `order`, in one launch.
template <int D>
void launch_prep(const Plan& p, const uint16_t* k, const uint16_t* v, const int32_t* idx,
                 const AttnPtrs& a, int t0, int t1, bool with_local, int32_t* order, int h0,
                 int h1, hipStream_t st) {
  const int P = (h1 - h0) * p.T;
  const unsigned gx = static_cast<unsigned>((t1 - t0) + (with_local ? p.H * p.loc_tiles : 0) +
                                            cdiv(P, 256));
  if (gx == 0) return;
  hipLaunchKernelGGL(prep_kernel<D>, dim3(gx, p.Hkv), dim3(256), 0, st, p, k, v, idx, a.kpre,
                     a.vtpre, a.vtloc, t0, t1, with_local ? 1 : 0, order, h0 * p.T, P);
}

// Run the attention kernel over the work items of blocks [h0, h1), in `order`.
template <int D>
void launch_attn_blocks(const Plan& p, const uint16_t* q, const uint16_t* k, const AttnPtrs& a,
                        int32_t* order, uint16_t* out, float* lse, int h0, int h1,
                        hipStream_t st) {
  const int P = (h1 - h0) * p.T;
  if (P <= 0) return;
  const int NG = P * p.Hkv;
  const int64_t grid = round_up(NG, 8) * p.G;
  const float c_log2 = static_cast<float>(p.scale * 1.4426950408889634);
  if (lse)
    hipLaunchKernelGGL((attn_kernel<D, true>), dim3(static_cast<unsigned>(grid)), dim3(kThreads),
                       0, st, p, q, k, a.kpre, a.vtpre, a.vtloc, order, out, lse, NG, c_log2);
  else
    hipLaunchKernelGGL((attn_kernel<D, false>), dim3(static_cast<unsigned>(grid)), dim3(kThreads),
                       0, st, p, q, k, a.kpre, a.vtpre, a.vtloc, order, out, lse, NG, c_log2);
}

template <int D>
hipError_t launch_d(const Plan& p, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                    const int32_t* idx, uint16_t* out, float* lse, char* ws, hipStream_t st) {
  const AttnPtrs a = attn_ptrs(p, ws);
  launch_prep<D>(p, k, v, idx, a, 0, p.Lpad / BN, true, a.order, 0, p.H, st);
  launch_attn_blocks<D>(p, q, k, a, a.order, out, lse, 0, p.H, st);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_bf16(const Plan& p, const void* q, const void* k, const void* v,
                            const int32_t* idx, void* out, float* lse, char* ws, hipStream_t st) {
  auto qq = static_cast<const uint16_t*>(q);
  auto kk = static_cast<const uint16_t*>(k);
  auto vv = static_cast<const uint16_t*>(v);
  auto oo = static_cast<uint16_t*>(out);
  if (p.D == 128) return launch_d<128>(p, qq, kk, vv, idx, oo, lse, ws, st);
  return launch_d<64>(p, qq, kk, vv, idx, oo, lse, ws, st);
}

hipError_t launch_attn_bf16_block0(const Plan& p, const void* q, const void* k, const void* v,
                                   void* out, float* lse, char* ws, hipStream_t st) {
  auto qq = static_cast<const uint16_t*>(q);
  auto kk = static_cast<const uint16_t*>(k);
  auto vv = static_cast<const uint16_t*>(v);
  auto oo = static_cast<uint16_t*>(out);
  const AttnPtrs a = attn_ptrs(p, ws);
  // The whole-anchor prefix tiles and every block's local V^T tiles need no indices.
  if (p.D == 128) {
    launch_prep<128>(p, kk, vv, nullptr, a, 0, anchor_tiles(p), true, a.order, 0, 1, st);
    launch_attn_blocks<128>(p, qq, kk, a, a.order, oo, lse, 0, 1, st);
  } else {
    launch_prep<64>(p, kk, vv, nullptr, a, 0, anchor_tiles(p), true, a.order, 0, 1, st);
    launch_attn_blocks<64>(p, qq, kk, a, a.order, oo, lse, 0, 1, st);
  }
  return hipGetLastError();
}

hipError_t launch_attn_bf16_rest(const Plan& p, const void* q, const void* k, const void* v,
                                 const int32_t* idx, void* out, float* lse, char* ws,
                                 hipStream_t st) {
  auto qq = static_cast<const uint16_t*>(q);
  auto kk = static_cast<const uint16_t*>(k);
  auto vv = static_cast<const uint16_t*>(v);
  auto oo = static_cast<uint16_t*>(out);
  const AttnPtrs a = attn_ptrs(p, ws);
  // The prefix tiles from the anchor's ragged last tile on hold passing rows.
  if (p.D == 128) {
    launch_prep<128>(p, kk, vv, idx, a, anchor_tiles(p), p.Lpad / BN, false, a.order2, 1, p.H,
                     st);
    launch_attn_blocks<128>(p, qq, kk, a, a.order2, oo, lse, 1, p.H, st);
  } else {
    launch_prep<64>(p, kk, vv, idx, a, anchor_tiles(p), p.Lpad / BN, false, a.order2, 1, p.H,
                    st);
    launch_attn_blocks<64>(p, qq, kk, a, a.order2, oo, lse, 1, p.H, st);
  }
  return hipGetLastError();
}

}  // namespace spava
