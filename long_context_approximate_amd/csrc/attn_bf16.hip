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
//   schedule   ranks (block, query tile) pairs by decreasing key-tile count;
//   attention  one workgroup = 256 queries x 1 query head (4 waves x 64 queries).
//              K/V tiles of 64 keys are double-buffered in LDS; S^T = K Q^T and
//              O^T += V^T P^T run on v_mfma_f32_32x32x16_bf16 with float32
//              accumulators; online softmax in float32 with exp2 and a folded scale.
//
// MFMA 32x32x16 operand layout (wave64): lane l supplies row/column (l % 32) of A/B
// and 8 consecutive reduction slots selected by (l / 32); accumulator register r of
// lane l holds row 8*(r/4) + 4*(l/32) + (r%4), column l % 32. Computing S^T (keys x
// queries) leaves each lane with one query and 16 keys per 32-key block, which is
// exactly the B operand P^T of the second product once V^T's key slots are stored
// in the same order; so P never leaves registers.
#include "spava_internal.h"

namespace spava {
namespace {

#ifndef SPAVA_ATTN_QB
#define SPAVA_ATTN_QB 1   // 32-query blocks per wave (1: 8 waves of 32 queries, 2 waves/SIMD)
#endif

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int BN = kKeyTile;                  // 64 keys per tile
constexpr int VROWB = BN * 2 + 16;            // bytes per V^T row in LDS (padded)

template <int D>
struct Cfg {
  static constexpr int KROWB = D * 2 + 16;    // bytes per K row in LDS (padded)
  static constexpr int KBYTES = BN * KROWB;
  static constexpr int VBYTES = D * VROWB;
  static constexpr int STAGE = KBYTES + VBYTES;
  static constexpr int DK = D / 16;           // MFMA steps over the head dim
  static constexpr int DM = D / 32;           // 32-row blocks of O^T
};

// Key offset inside a 16-key chunk for MFMA reduction slot s (an involution).
__host__ __device__ constexpr int slot_key(int s) {
  return 8 * ((s & 7) >> 2) + 4 * (s >> 3) + (s & 3);
}

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
  for (int c = tid; c < D * (BN / 8); c += 256) {
    const int d = c / (BN / 8), sc = c % (BN / 8);   // slots sc*8 .. sc*8+7
    uint16_t vals[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int slot = sc * 8 + e;
      const int key = (slot & ~15) + slot_key(slot & 15);
      vals[e] = Vs[key][d];
    }
    uint4 pk;
    pk.x = vals[0] | (static_cast<uint32_t>(vals[1]) << 16);
    pk.y = vals[2] | (static_cast<uint32_t>(vals[3]) << 16);
    pk.z = vals[4] | (static_cast<uint32_t>(vals[5]) << 16);
    pk.w = vals[6] | (static_cast<uint32_t>(vals[7]) << 16);
    *reinterpret_cast<uint4*>(dst + static_cast<int64_t>(d) * BN + sc * 8) = pk;
  }
}

__device__ inline int pair_cost(const Plan& p, int pair) {
  const int h = pair / p.T, t = pair % p.T;
  const int loc = min(p.nb, (t + 1) * kQTile);
  return (prefix_len(p, h) + BN - 1) / BN + (loc + BN - 1) / BN;
}

// order[rank] = pair, pairs ranked by decreasing cost, ties by pair index.
__global__ __launch_bounds__(256) void schedule_kernel(Plan p, int32_t* __restrict__ order) {
  const int P = p.H * p.T;
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= P) return;
  const int ci = pair_cost(p, i);
  int rank = 0;
  for (int j = 0; j < P; ++j) {
    const int cj = pair_cost(p, j);
    rank += (cj > ci) || (cj == ci && j < i);
  }
  order[rank] = i;
}

// Query tile: NW waves x QB 32-query blocks per wave; BM = NW*32*QB = kQTile.
template <int D, int QB, int NW>
struct Tile {
  static constexpr int THREADS = NW * 64;
  static constexpr int WQ = 32 * QB;             // queries per wave
  static constexpr int KCH = BN * D / 8 / THREADS; // 16-byte K chunks per thread per tile
  static constexpr int VCH = D * BN / 8 / THREADS; // 16-byte V^T chunks per thread per tile
  static_assert(NW * WQ == kQTile, "query tile must match the plan");
  static_assert(KCH >= 1 && VCH >= 1, "tile too small for the workgroup");
};

// Softmax rescale threshold (log2 units): the running reference max is only raised
// when a tile's max exceeds it by more than this, so exp2 values stay <= 2^8 and the
// accumulators are rescaled rarely. The result is exact: numerator and denominator
// share the reference.
constexpr float kRescaleLog2 = 8.0f;

template <int D, int QB, int NW>
__global__ __launch_bounds__(NW * 64) void attn_kernel(
    Plan p, const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ kpre, const uint16_t* __restrict__ vtpre,
    const uint16_t* __restrict__ vtloc, const int32_t* __restrict__ order,
    uint16_t* __restrict__ out, float* __restrict__ lse, int NG, float c_log2) {
  using C = Cfg<D>;
  using TL = Tile<D, QB, NW>;
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
  const int64_t qw0 = q0 + static_cast<int64_t>(TL::WQ) * w;   // first query of this wave
  const int64_t qw_last = qw0 + TL::WQ - 1;
  const bool wave_active = qw0 < e_h;

  // ---- tile loaders (global -> registers -> LDS)
  const uint16_t* kpre_g = kpre + static_cast<int64_t>(g) * p.Lpad * D;
  const uint16_t* vtpre_g = vtpre + static_cast<int64_t>(g) * (p.Lpad / BN) * D * BN;
  const uint16_t* vtloc_gh = vtloc + (static_cast<int64_t>(g) * p.H + h) * p.loc_tiles * D * BN;
  const uint16_t* k_g = k + g * p.kvs_head;

  u32x4 kreg[TL::KCH], vreg[TL::VCH];
  // Branch-free body (only the source pointers depend on the tile kind) so the
  // staging registers stay in VGPRs.
  auto load_tile = [&](int it) {
    const bool pre = it < npre;
    const int lt = it - npre;
    const int64_t key0 = s_h + static_cast<int64_t>(lt) * BN;
    const uint16_t* kb = pre ? kpre_g + static_cast<int64_t>(it) * BN * D : k_g + key0 * p.kvs_tok;
    const int64_t krow = pre ? D : p.kvs_tok;
    const int64_t kvalid = pre ? BN : e_h - key0;
    const uint16_t* vb = pre ? vtpre_g + static_cast<int64_t>(it) * D * BN
                             : vtloc_gh + static_cast<int64_t>(lt) * D * BN;
#pragma unroll
    for (int i = 0; i < TL::KCH; ++i) {
      const int c = tid + TL::THREADS * i;
      const int row = c / (D / 8), col = c % (D / 8);
      kreg[i] = row < kvalid ? *reinterpret_cast<const u32x4*>(kb + row * krow + col * 8)
                             : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int i = 0; i < TL::VCH; ++i)
      vreg[i] = *reinterpret_cast<const u32x4*>(vb + (tid + TL::THREADS * i) * 8);
  };
  auto store_tile = [&](int buf) {
    char* ks = smem + buf * C::STAGE;
    char* vs = ks + C::KBYTES;
#pragma unroll
    for (int i = 0; i < TL::KCH; ++i) {
      const int c = tid + TL::THREADS * i;
      const int row = c / (D / 8), col = c % (D / 8);
      *reinterpret_cast<u32x4*>(ks + row * C::KROWB + col * 16) = kreg[i];
    }
#pragma unroll
    for (int i = 0; i < TL::VCH; ++i) {
      const int c = tid + TL::THREADS * i;
      const int d = c / (BN / 8), col = c % (BN / 8);
      *reinterpret_cast<u32x4*>(vs + d * VROWB + col * 16) = vreg[i];
    }
  };

  // ---- Q fragments (B operand of S^T = K Q^T), kept in registers
  bf16x8 qf[QB][C::DK];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int64_t qi = qw0 + 32 * qb + lr;
    const bool ok = qi < e_h;
    const uint16_t* qp = q + qi * p.qs_tok + hq * p.qs_head + lh * 8;
#pragma unroll
    for (int dk = 0; dk < C::DK; ++dk) {
      u32x4 raw = ok ? *reinterpret_cast<const u32x4*>(qp + dk * 16) : u32x4{0u, 0u, 0u, 0u};
      qf[qb][dk] = __builtin_bit_cast(bf16x8, raw);
    }
  }

  f32x16 o[QB][C::DM];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb)
#pragma unroll
    for (int dm = 0; dm < C::DM; ++dm)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[qb][dm][r] = 0.f;
  float mrun[QB], lsum[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    mrun[qb] = -INFINITY;
    lsum[qb] = 0.f;
  }

  load_tile(0);
  store_tile(0);
  __syncthreads();

  for (int it = 0; it < ntiles; ++it) {
    if (it + 1 < ntiles) load_tile(it + 1);
    const bool local = it >= npre;
    const int lt = it - npre;
    const int64_t key0 = local ? s_h + static_cast<int64_t>(lt) * BN : 0;
    const bool skip = !wave_active || (local && key0 > qw_last);
    if (!skip) {
      const char* ks = smem + (it & 1) * C::STAGE;
      const char* vs = ks + C::KBYTES;
      f32x16 s[QB][2];
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) s[qb][kb][r] = 0.f;
#pragma unroll
      for (int dk = 0; dk < C::DK; ++dk) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(ks + (kb * 32 + lr) * C::KROWB +
                                                            (dk * 16 + lh * 8) * 2);
#pragma unroll
          for (int qb = 0; qb < QB; ++qb)
            s[qb][kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[qb][dk], s[qb][kb], 0, 0, 0);
        }
      }
      // Masks: keys past the prefix length in the last prefix tile; causal on the
      // diagonal local tile.
      const bool pre_tail = !local && it == npre - 1 && (L % BN) != 0;
      const bool diag = local && key0 + BN - 1 > qw0;
      if (pre_tail || diag) {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          const int qrel = static_cast<int>(qw0 + 32 * qb + lr - key0);   // query - key0
          const int lim = pre_tail ? L - it * BN - 1 : qrel;              // last visible kk
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int kk = kb * 32 + 8 * (r >> 2) + 4 * lh + (r & 3);
              if (kk > lim) s[qb][kb][r] = -INFINITY;
            }
        }
      }
      // Online softmax (log2 domain, lazy rescale) and P^T fragments.
      bf16x8 pf[QB][4];
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        float mx = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[qb][kb][r]);
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float mt = mx * c_log2;
        if (__any(mt > mrun[qb] + kRescaleLog2)) {
          const float mnew = fmaxf(mrun[qb], mt);
          const float alpha = __builtin_amdgcn_exp2f(mrun[qb] - (mnew == -INFINITY ? 0.f : mnew));
          mrun[qb] = mnew;
          lsum[qb] *= alpha;
#pragma unroll
          for (int dm = 0; dm < C::DM; ++dm)
#pragma unroll
            for (int r = 0; r < 16; ++r) o[qb][dm][r] *= alpha;
        }
        const float mref = mrun[qb] == -INFINITY ? 0.f : mrun[qb];
        float ps = 0.f;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float pv = __builtin_amdgcn_exp2f(fmaf(s[qb][kb][r], c_log2, -mref));
            s[qb][kb][r] = pv;
            ps += pv;
          }
        lsum[qb] += ps;
#pragma unroll
        for (int kc = 0; kc < 4; ++kc) {
          const int kb = kc >> 1, half = kc & 1;
#pragma unroll
          for (int e2 = 0; e2 < 4; ++e2) {
            f32x2 two = {s[qb][kb][half * 8 + 2 * e2], s[qb][kb][half * 8 + 2 * e2 + 1]};
            bf16x2 cv = __builtin_convertvector(two, bf16x2);
            pf[qb][kc][2 * e2] = cv[0];
            pf[qb][kc][2 * e2 + 1] = cv[1];
          }
        }
      }
      // O^T += V^T P^T
#pragma unroll
      for (int kc = 0; kc < 4; ++kc) {
#pragma unroll
        for (int dm = 0; dm < C::DM; ++dm) {
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(vs + (dm * 32 + lr) * VROWB +
                                                            (kc * 16 + lh * 8) * 2);
#pragma unroll
          for (int qb = 0; qb < QB; ++qb)
            o[qb][dm] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[qb][kc], o[qb][dm], 0, 0, 0);
        }
      }
    }
    if (it + 1 < ntiles) store_tile((it + 1) & 1);
    __syncthreads();
  }

  // ---- epilogue: normalise, round to bf16, write O and LSE
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const float ltot = lsum[qb] + __shfl_xor(lsum[qb], 32);
    const int64_t qi = qw0 + 32 * qb + lr;
    if (qi >= e_h) continue;
    const float inv = 1.f / ltot;
    uint16_t* op = out + qi * p.os_tok + hq * p.os_head;
#pragma unroll
    for (int dm = 0; dm < C::DM; ++dm)
#pragma unroll
      for (int grp = 0; grp < 4; ++grp) {
        f32x2 lo = {o[qb][dm][grp * 4 + 0] * inv, o[qb][dm][grp * 4 + 1] * inv};
        f32x2 hi = {o[qb][dm][grp * 4 + 2] * inv, o[qb][dm][grp * 4 + 3] * inv};
        bf16x2 blo = __builtin_convertvector(lo, bf16x2);
        bf16x2 bhi = __builtin_convertvector(hi, bf16x2);
        uint2 pk;
        pk.x = __builtin_bit_cast(uint32_t, blo);
        pk.y = __builtin_bit_cast(uint32_t, bhi);
        const int d = dm * 32 + 8 * grp + 4 * lh;
        *reinterpret_cast<uint2*>(op + d) = pk;
      }
    if (lse && lh == 0)
      lse[static_cast<int64_t>(hq) * p.N + qi] = (mrun[qb] + log2f(ltot)) * 0.69314718055994531f;
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
  constexpr int QB = SPAVA_ATTN_QB, NW = kQTile / (32 * SPAVA_ATTN_QB);
  hipLaunchKernelGGL((attn_kernel<D, QB, NW>), dim3(static_cast<unsigned>(grid)), dim3(NW * 64), 0,
                     st, p, q, k, kpre, vtpre, vtloc, order, out, lse, NG, c_log2);
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
