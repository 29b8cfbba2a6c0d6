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

// grid.x: [0, Lpad/64) prefix tiles, then H*loc_tiles local V tiles; grid.y: KV head.
template <int D>
__global__ __launch_bounds__(256) void prep_kernel(Plan p, const uint16_t* __restrict__ k,
                                                   const uint16_t* __restrict__ v,
                                                   const int32_t* __restrict__ idx,
                                                   uint16_t* __restrict__ kpre,
                                                   uint16_t* __restrict__ vtpre,
                                                   uint16_t* __restrict__ vtloc) {
  __shared__ __attribute__((aligned(16))) uint16_t Vs[BN][D + 8];
  __shared__ int64_t src_tok[BN];
  const int g = blockIdx.y;
  const int tid = threadIdx.x;
  const int npre_tiles = p.Lpad / BN;
  const bool is_prefix = static_cast<int>(blockIdx.x) < npre_tiles;
  int tile, h = 0;
  if (is_prefix) {
    tile = blockIdx.x;
  } else {
    const int lt = blockIdx.x - npre_tiles;
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

__device__ inline int pair_cost(const Plan& p, int pair) {
  const int h = pair / p.T, t = pair % p.T;
  const int loc = min(p.nb, (t + 1) * kQTile);
  return (prefix_len(p, h) + BN - 1) / BN + (loc + BN - 1) / BN;
}

// order[rank] = pair (pair = block * T + query tile). Longest first: pairs ranked by
// decreasing key-tile count, ties by pair index. Natural: block-major. ZigZag: blocks
// paired as (p, H-1-p), the pages' host pairing, tiles of a pair alternating.
__global__ __launch_bounds__(256) void schedule_kernel(Plan p, int32_t* __restrict__ order) {
  const int P = p.H * p.T;
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= P) return;
  int rank = 0;
  if (p.sched == kSchedNatural) {
    rank = i;
  } else if (p.sched == kSchedZigZag) {
    const int h = i / p.T, t = i % p.T;
    const int mirror = p.H - 1 - h;
    const int pr = min(h, mirror);
    rank = (h == mirror) ? pr * 2 * p.T + t : pr * 2 * p.T + 2 * t + (h > mirror ? 1 : 0);
  } else {
    const int ci = pair_cost(p, i);
    for (int j = 0; j < P; ++j) {
      const int cj = pair_cost(p, j);
      rank += (cj > ci) || (cj == ci && j < i);
    }
  }
  order[rank] = i;
}

template <int D>
__global__ __launch_bounds__(kThreads) void attn_kernel(
    Plan p, const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ kpre, const uint16_t* __restrict__ vtpre,
    const uint16_t* __restrict__ vtloc, const int32_t* __restrict__ order,
    uint16_t* __restrict__ out, float* __restrict__ lse, int NG, float c_log2) {
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
  const int L = prefix_len(p, h);
  const int npre = (L + BN - 1) / BN;
  const int nloc = static_cast<int>((q_end - s_h + BN - 1) / BN);
  const int ntiles = npre + nloc;

  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63;
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
  TileStage<D> stage;
  auto load_tile = [&](int it) {
    const bool pre = it < npre;
    const int lt = it - npre;
    const int64_t key0 = s_h + static_cast<int64_t>(lt) * BN;
    const uint16_t* kb = pre ? kpre_g + static_cast<int64_t>(it) * BN * D : k_g + key0 * p.kvs_tok;
    const int64_t krow = pre ? D : p.kvs_tok;
    const int64_t kvalid = pre ? BN : e_h - key0;
    const uint16_t* vb = pre ? vtpre_g + static_cast<int64_t>(it) * D * BN
                             : vtloc_gh + static_cast<int64_t>(lt) * D * BN;
    stage.load(kb, krow, kvalid, vb);
  };

  bf16x8 qf[C::DK];
  load_q<D>(q + qi * p.qs_tok + hq * p.qs_head + lh * 8, qi < e_h, qf);
  Flash<D> f;
  f.init();

  load_tile(0);
  stage.store(smem);
  __syncthreads();

  for (int it = 0; it < ntiles; ++it) {
    if (it + 1 < ntiles) load_tile(it + 1);
    const bool local = it >= npre;
    const int64_t key0 = local ? s_h + static_cast<int64_t>(it - npre) * BN : 0;
    // Last visible key of the tile: the prefix length in the last prefix tile, the
    // causal diagonal in a local tile. Tiles past this wave's queries are processed
    // fully masked (lim = -1) rather than branched around, which keeps the O
    // accumulators in place across iterations.
    int lim = BN - 1;
    if (!local && it == npre - 1 && (L % BN) != 0) lim = L - it * BN - 1;
    if (local && key0 + BN - 1 > qw0) {
      const int64_t rel = qi - key0;               // integer select (no floating max)
      lim = rel < 0 ? -1 : static_cast<int>(rel);
    }
    if (!wave_active) lim = -1;
    const char* ks = smem + (it & 1) * C::STAGE;
    attend_tile<D>(ks, ks + C::KBYTES, qf, f, lim, c_log2);
    if (it + 1 < ntiles) stage.store(smem + ((it + 1) & 1) * C::STAGE);
    __syncthreads();
  }

  // ---- epilogue: normalise, round to bf16, write O and LSE
  const float ltot = flash_rowsum<D>(f);
  if (qi < e_h) {
    const float inv = 1.f / ltot;
    uint16_t* op = out + qi * p.os_tok + hq * p.os_head;
#pragma unroll
    for (int dm = 0; dm < C::DM; ++dm)
#pragma unroll
      for (int grp = 0; grp < 4; ++grp) {
        f32x2 lo = {f.o[dm][grp * 4 + 0] * inv, f.o[dm][grp * 4 + 1] * inv};
        f32x2 hi = {f.o[dm][grp * 4 + 2] * inv, f.o[dm][grp * 4 + 3] * inv};
        bf16x2 blo = __builtin_convertvector(lo, bf16x2);
        bf16x2 bhi = __builtin_convertvector(hi, bf16x2);
        uint2 pk;
        pk.x = __builtin_bit_cast(uint32_t, blo);
        pk.y = __builtin_bit_cast(uint32_t, bhi);
        *reinterpret_cast<uint2*>(op + out_dim<D>(dm, grp, lh)) = pk;
      }
    if (lse && lh == 0)
      lse[static_cast<int64_t>(hq) * p.N + qi] = (f.mrun + log2f(ltot)) * 0.69314718055994531f;
  }
}

template <int D>
hipError_t launch_d(const Plan& p, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                    const int32_t* idx, uint16_t* out, float* lse, char* ws, hipStream_t st) {
  const AttnWs w = attn_ws_layout(p);
  uint16_t* kpre = reinterpret_cast<uint16_t*>(ws + w.kpre);
  uint16_t* vtpre = reinterpret_cast<uint16_t*>(ws + w.vpre);
  uint16_t* vtloc = reinterpret_cast<uint16_t*>(ws + w.vtloc);
  int32_t* order = reinterpret_cast<int32_t*>(ws + w.order);
  const unsigned prep_x = static_cast<unsigned>(p.Lpad / BN + p.H * p.loc_tiles);
  hipLaunchKernelGGL(prep_kernel<D>, dim3(prep_x, p.Hkv), dim3(256), 0, st, p, k, v, idx, kpre,
                     vtpre, vtloc);
  const int P = p.H * p.T;
  hipLaunchKernelGGL(schedule_kernel, dim3(static_cast<unsigned>(cdiv(P, 256))), dim3(256), 0, st,
                     p, order);
  const int NG = P * p.Hkv;
  const int64_t grid = round_up(NG, 8) * p.G;
  const float c_log2 = static_cast<float>(p.scale * 1.4426950408889634);
  hipLaunchKernelGGL(attn_kernel<D>, dim3(static_cast<unsigned>(grid)), dim3(kThreads), 0, st, p, q, k, kpre, vtpre, vtloc, order, out, lse, NG, c_log2);
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

}  // namespace spava
