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
//              (2 waves per SIMD). K/V tiles of 64 keys are double-buffered in LDS;
//              each tile is one flash step (attn_common.h): S^T = K Q^T and
//              O^T += V^T P^T on v_mfma_f32_32x32x16_bf16 with float32 accumulators
//              and an online softmax in float32 with exp2 and a folded scale.
//
// Split mode (the one-GPU form of the pages' overlap of passing-block transfers with
// compute, "Systemseitige Optimierungen"): part X attends every query to the whole
// anchor tiles and its local keys, which need no selection, and stores (O, LSE) per
// query; part Y attends to the rest of the prefix (the passing rows, with the
// anchor's ragged last tile) and merges with part X by log-sum-exp. X can run while
// the selection runs on another stream.
#include "attn_common.h"

namespace spava {
namespace {

// Source token of prefix row r (anchor then passing rows of blocks 0, 1, ...) for KV
// head g; -1 for padding rows and for indices outside the block's candidates.
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

// Whole anchor tiles: prefix tiles [0, A / 64) hold anchor rows only.
__host__ __device__ inline int anchor_tiles(const Plan& p) { return p.A / BN; }

// grid.x: prefix tiles [t0, t1), then (with_local) H*loc_tiles local V tiles;
// grid.y: KV head.
template <int D>
__global__ __launch_bounds__(256) void prep_kernel(Plan p, const uint16_t* __restrict__ k,
                                                   const uint16_t* __restrict__ v,
                                                   const int32_t* __restrict__ idx,
                                                   uint16_t* __restrict__ kpre,
                                                   uint16_t* __restrict__ vtpre,
                                                   uint16_t* __restrict__ vtloc, int t0, int t1) {
  __shared__ __attribute__((aligned(16))) uint16_t Vs[BN][D + 8];
  __shared__ int64_t src_tok[BN];
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

// Prefix tiles [pt0, pt1) and whether local tiles follow, for block h in a mode.
struct TileRange {
  int pt0, pt1, local;
};
__device__ inline TileRange tile_range(const Plan& p, int h, int mode) {
  const int npre = (prefix_len(p, h) + BN - 1) / BN;
  const int nax = h >= 1 ? anchor_tiles(p) : 0;
  if (mode == kAttnPartX) return {0, nax, 1};
  if (mode == kAttnPartY) return {nax, npre, 0};
  return {0, npre, 1};
}

__device__ inline int pair_cost(const Plan& p, int pair, int mode) {
  const int h = pair / p.T, t = pair % p.T;
  const int loc = min(p.nb, (t + 1) * kQTile);
  const TileRange tr = tile_range(p, h, mode);
  return (tr.pt1 - tr.pt0) + (tr.local ? (loc + BN - 1) / BN : 0);
}

// order[rank] = pair (pair = block * T + query tile). Longest first: pairs ranked by
// decreasing key-tile count, ties by pair index. Natural: block-major. ZigZag: blocks
// paired as (p, H-1-p), the pages' host pairing, tiles of a pair alternating.
__global__ __launch_bounds__(256) void schedule_kernel(Plan p, int32_t* __restrict__ order,
                                                       int mode) {
  __shared__ __attribute__((aligned(16))) int cost[256];
  const int P = p.H * p.T;
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  const bool valid = i < P;
  int rank = 0;
  if (p.sched == kSchedNatural) {
    rank = i;
  } else if (p.sched == kSchedZigZag) {
    const int h = i / p.T, t = i % p.T;
    const int mirror = p.H - 1 - h;
    const int pr = min(h, mirror);
    rank = (h == mirror) ? pr * 2 * p.T + t : pr * 2 * p.T + 2 * t + (h > mirror ? 1 : 0);
  } else {
    // Rank = number of pairs that come first (higher cost, or equal cost and lower
    // index); the costs of each chunk of 256 pairs are computed once into LDS (slots
    // past P hold -1, which never counts: costs are >= 0) and read 4 at a time.
    const int ci = valid ? pair_cost(p, i, mode) : 0;
    for (int j0 = 0; j0 < P; j0 += 256) {
      __syncthreads();
      const int jt = j0 + static_cast<int>(threadIdx.x);
      cost[threadIdx.x] = jt < P ? pair_cost(p, jt, mode) : -1;
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
  if (valid) order[rank] = i;
}

template <int D, int MODE>
__global__ __launch_bounds__(kThreads) void attn_kernel(
    Plan p, const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ kpre, const uint16_t* __restrict__ vtpre,
    const uint16_t* __restrict__ vtloc, const int32_t* __restrict__ order,
    uint16_t* __restrict__ out, float* __restrict__ lse, int NG, float c_log2,
    float* __restrict__ part_o, float* __restrict__ part_lse) {
  constexpr int mode = MODE;
  using C = Cfg<D>;
  __shared__ __attribute__((aligned(16))) char smem[2 * C::STAGE];

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
  // Part Y of block 0 has nothing to do: part X wrote its final output.
  if (mode == kAttnPartY && h == 0) return;
  const int L = prefix_len(p, h);
  const int npre = (L + BN - 1) / BN;
  const TileRange tr = tile_range(p, h, mode);
  const int np = tr.pt1 - tr.pt0;
  const int nloc = tr.local ? static_cast<int>((q_end - s_h + BN - 1) / BN) : 0;
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
  const uint16_t* kpre0 = kpre_g + static_cast<int64_t>(tr.pt0) * BN * D;
  const uint16_t* vpre0 = vtpre_g + static_cast<int64_t>(tr.pt0) * D * BN;
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
  const int it_diag = tr.local ? np + first_diag : ntiles;
  const int it_edge =
      ((L % BN) != 0 && npre - 1 >= tr.pt0 && npre - 1 < tr.pt1) ? npre - 1 - tr.pt0 : -1;
  const int qrel = static_cast<int>(qi - s_h);   // this lane's query inside the block

  if (ntiles > 0) issue_tile(0, smem);
  wait_tile_loads();
  __syncthreads();

  for (int it = 0; it < ntiles; ++it) {
    if (it + 1 < ntiles) issue_tile(it + 1, smem + ((it + 1) & 1) * C::STAGE);
    // Last visible key of a masked tile: the prefix length in the partial prefix
    // tile, the causal diagonal in a local tile. Tiles past this wave's queries are
    // processed fully masked (lim = -1) rather than branched around, which keeps the
    // O accumulators in place across iterations.
    const bool diag = it >= it_diag;
    const bool masked = diag || it == it_edge || !wave_active;
    int lim = BN - 1;
    if (masked) {
      if (it == it_edge) lim = L - (tr.pt0 + it) * BN - 1;
      if (diag) {
        const int rel = qrel - (it - np) * BN;      // integer select (no floating max)
        lim = rel < 0 ? -1 : rel;
      }
      if (!wave_active) lim = -1;
    }
    const char* ks = smem + (it & 1) * C::STAGE;
    attend_tile<D>(ks, ks + C::KBYTES, qf, f, masked, lim, c_log2);
    wait_tile_loads();
    __syncthreads();
  }

  // ---- epilogue: normalise, round to bf16, write O and LSE
  const float ltot = flash_rowsum<D>(f);
  if (qi < e_h && mode == kAttnPartX && h >= 1) {
    // Part X of a block with a prefix: keep the normalised partial (O, log2-LSE).
    const float inv = 1.f / ltot;
    float* po = part_o + (qi * p.Hq + hq) * D;
#pragma unroll
    for (int dm = 0; dm < C::DM; ++dm)
#pragma unroll
      for (int grp = 0; grp < 4; ++grp) {
        float4 v4;
        v4.x = f.o[dm][grp * 4 + 0] * inv;
        v4.y = f.o[dm][grp * 4 + 1] * inv;
        v4.z = f.o[dm][grp * 4 + 2] * inv;
        v4.w = f.o[dm][grp * 4 + 3] * inv;
        *reinterpret_cast<float4*>(po + out_dim<D>(dm, grp, lh)) = v4;
      }
    if (lh == 0) part_lse[static_cast<int64_t>(hq) * p.N + qi] = f.mrun + log2f(ltot);
  } else if (qi < e_h) {
    // Full output, or part Y merged with part X: O = (wx O_x + wy O_y) / (wx + wy) with
    // w = 2^LSE relative to the larger of the two LSEs.
    float cx = 0.f, cy = 1.f / ltot, lse2 = f.mrun + log2f(ltot);
    const float* po = nullptr;
    if (mode == kAttnPartY) {
      const float lx = part_lse[static_cast<int64_t>(hq) * p.N + qi];
      const float ly = ltot > 0.f ? f.mrun + log2f(ltot) : -INFINITY;
      const float mx = fmaxf(lx, ly);
      const float wx = exp2f(lx - mx), wy = ltot > 0.f ? exp2f(ly - mx) : 0.f;
      const float den = wx + wy;
      cx = wx / den;
      cy = ltot > 0.f ? wy / (ltot * den) : 0.f;
      lse2 = mx + log2f(den);
      po = part_o + (qi * p.Hq + hq) * D;
    }
    uint16_t* op = out + qi * p.os_tok + hq * p.os_head;
#pragma unroll
    for (int dm = 0; dm < C::DM; ++dm)
#pragma unroll
      for (int grp = 0; grp < 4; ++grp) {
        float4 ox = {0.f, 0.f, 0.f, 0.f};
        if (po) ox = *reinterpret_cast<const float4*>(po + out_dim<D>(dm, grp, lh));
        f32x2 lo = {ox.x * cx + f.o[dm][grp * 4 + 0] * cy, ox.y * cx + f.o[dm][grp * 4 + 1] * cy};
        f32x2 hi = {ox.z * cx + f.o[dm][grp * 4 + 2] * cy, ox.w * cx + f.o[dm][grp * 4 + 3] * cy};
        bf16x2 blo = __builtin_convertvector(lo, bf16x2);
        bf16x2 bhi = __builtin_convertvector(hi, bf16x2);
        uint2 pk;
        pk.x = __builtin_bit_cast(uint32_t, blo);
        pk.y = __builtin_bit_cast(uint32_t, bhi);
        *reinterpret_cast<uint2*>(op + out_dim<D>(dm, grp, lh)) = pk;
      }
    if (lse && lh == 0) lse[static_cast<int64_t>(hq) * p.N + qi] = lse2 * 0.69314718055994531f;
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

// Gather prefix tiles [t0, t1) (and, with_local, every block's local V^T tiles).
template <int D>
void launch_prep(const Plan& p, const uint16_t* k, const uint16_t* v, const int32_t* idx,
                 const AttnPtrs& a, int t0, int t1, bool with_local, hipStream_t st) {
  const unsigned gx = static_cast<unsigned>((t1 - t0) + (with_local ? p.H * p.loc_tiles : 0));
  if (gx == 0) return;
  hipLaunchKernelGGL(prep_kernel<D>, dim3(gx, p.Hkv), dim3(256), 0, st, p, k, v, idx, a.kpre,
                     a.vtpre, a.vtloc, t0, t1);
}

// Order the (block, query tile) pairs for `mode` and run the attention kernel.
template <int D>
void launch_attn_mode(const Plan& p, const uint16_t* q, const uint16_t* k, const AttnPtrs& a,
                      int32_t* order, uint16_t* out, float* lse, int mode, float* part_o,
                      float* part_lse, hipStream_t st) {
  const int P = p.H * p.T;
  hipLaunchKernelGGL(schedule_kernel, dim3(static_cast<unsigned>(cdiv(P, 256))), dim3(256), 0, st,
                     p, order, mode);
  const int NG = P * p.Hkv;
  const int64_t grid = round_up(NG, 8) * p.G;
  const float c_log2 = static_cast<float>(p.scale * 1.4426950408889634);
  const dim3 gd(static_cast<unsigned>(grid));
  if (mode == kAttnPartX)
    hipLaunchKernelGGL((attn_kernel<D, kAttnPartX>), gd, dim3(kThreads), 0, st, p, q, k, a.kpre,
                       a.vtpre, a.vtloc, order, out, lse, NG, c_log2, part_o, part_lse);
  else if (mode == kAttnPartY)
    hipLaunchKernelGGL((attn_kernel<D, kAttnPartY>), gd, dim3(kThreads), 0, st, p, q, k, a.kpre,
                       a.vtpre, a.vtloc, order, out, lse, NG, c_log2, part_o, part_lse);
  else
    hipLaunchKernelGGL((attn_kernel<D, kAttnFull>), gd, dim3(kThreads), 0, st, p, q, k, a.kpre,
                       a.vtpre, a.vtloc, order, out, lse, NG, c_log2, part_o, part_lse);
}

template <int D>
hipError_t launch_d(const Plan& p, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                    const int32_t* idx, uint16_t* out, float* lse, char* ws, hipStream_t st) {
  const AttnPtrs a = attn_ptrs(p, ws);
  launch_prep<D>(p, k, v, idx, a, 0, p.Lpad / BN, true, st);
  launch_attn_mode<D>(p, q, k, a, a.order, out, lse, kAttnFull, nullptr, nullptr, st);
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

hipError_t launch_attn_bf16_part_x(const Plan& p, const void* q, const void* k, const void* v,
                                   void* out, float* lse, char* ws, float* part_o,
                                   float* part_lse, hipStream_t st) {
  auto qq = static_cast<const uint16_t*>(q);
  auto kk = static_cast<const uint16_t*>(k);
  auto vv = static_cast<const uint16_t*>(v);
  auto oo = static_cast<uint16_t*>(out);
  const AttnPtrs a = attn_ptrs(p, ws);
  if (p.D == 128) {
    launch_prep<128>(p, kk, vv, nullptr, a, 0, anchor_tiles(p), true, st);
    launch_attn_mode<128>(p, qq, kk, a, a.order, oo, lse, kAttnPartX, part_o, part_lse, st);
  } else {
    launch_prep<64>(p, kk, vv, nullptr, a, 0, anchor_tiles(p), true, st);
    launch_attn_mode<64>(p, qq, kk, a, a.order, oo, lse, kAttnPartX, part_o, part_lse, st);
  }
  return hipGetLastError();
}

hipError_t launch_attn_bf16_gather_passing(const Plan& p, const void* k, const void* v,
                                           const int32_t* idx, char* ws, hipStream_t st) {
  auto kk = static_cast<const uint16_t*>(k);
  auto vv = static_cast<const uint16_t*>(v);
  const AttnPtrs a = attn_ptrs(p, ws);
  if (p.D == 128) launch_prep<128>(p, kk, vv, idx, a, anchor_tiles(p), p.Lpad / BN, false, st);
  else launch_prep<64>(p, kk, vv, idx, a, anchor_tiles(p), p.Lpad / BN, false, st);
  return hipGetLastError();
}

hipError_t launch_attn_bf16_part_y(const Plan& p, const void* q, const void* k, void* out,
                                   float* lse, char* ws, float* part_o, float* part_lse,
                                   hipStream_t st) {
  auto qq = static_cast<const uint16_t*>(q);
  auto kk = static_cast<const uint16_t*>(k);
  auto oo = static_cast<uint16_t*>(out);
  const AttnPtrs a = attn_ptrs(p, ws);
  if (p.D == 128)
    launch_attn_mode<128>(p, qq, kk, a, a.order2, oo, lse, kAttnPartY, part_o, part_lse, st);
  else
    launch_attn_mode<64>(p, qq, kk, a, a.order2, oo, lse, kAttnPartY, part_o, part_lse, st);
  return hipGetLastError();
}

}  // namespace spava
