// Query block B_qr: per-host partial attention and log-sum-exp merge.
//
// Method (explainer "APB-V: ...", Methodik > Kontext-Splitting: the embeddings are
// split into anchor, query block B_qr and context blocks; Systemseitige
// Optimierungen > fused context + query forward: each host attends the query rows to
// what it holds and the partial results are merged with FlashAttention's log-sum-exp
// outputs). The partial key sets are disjoint — host h's own context block, plus the
// query block's own keys (causal) — so the merge is exact: row i of B_qr sees every
// context key and the query keys [0, i].
//
// Kernels:
//   vt_rows    V^T tiles (MFMA slot order) of the context blocks and of the query keys;
//   partial    bf16: one workgroup = 256 query rows x 1 head x 1 partial (H context
//              blocks + the query block itself), the same flash step as the main
//              attention; f32: 64 query rows per workgroup on the float64 matrix
//              cores, the main float32 attention's step (float32 exponentials);
//   merge      O = sum_h exp(LSE_h - LSE) O_h with LSE = log sum_h exp(LSE_h).
#include "attn_common.h"
#include "attn_f32_step.h"

namespace spava {
namespace {

// V^T tiles of `nsegs` consecutive segments of `nseg` rows of v (KV head = grid.y):
// dst [Hkv][nsegs][tiles_per_seg][D][64]; rows past a segment's end are zero.
// grid (nsegs * tiles_per_seg, Hkv), 256 threads.
template <int D>
__global__ __launch_bounds__(256) void vt_rows_kernel(const uint16_t* __restrict__ v, int64_t nseg,
                                                      int nsegs, int tiles_per_seg,
                                                      int64_t stride_tok, int64_t stride_head,
                                                      uint16_t* __restrict__ dst) {
  __shared__ __attribute__((aligned(16))) uint16_t Vs[BN][D + 8];
  const int g = blockIdx.y;
  const int seg = blockIdx.x / tiles_per_seg, tile = blockIdx.x % tiles_per_seg;
  constexpr int CPR = D / 8;
  for (int c = threadIdx.x; c < BN * CPR; c += 256) {
    const int row = c / CPR, col = c % CPR;
    const int64_t off = static_cast<int64_t>(tile) * BN + row;
    uint4 vv = make_uint4(0, 0, 0, 0);
    if (off < nseg)
      vv = *reinterpret_cast<const uint4*>(v + (seg * nseg + off) * stride_tok + g * stride_head +
                                           col * 8);
    *reinterpret_cast<uint4*>(&Vs[row][col * 8]) = vv;
  }
  __syncthreads();
  store_vt_tile<D>(Vs, dst + ((static_cast<int64_t>(g) * nsegs + seg) * tiles_per_seg + tile) *
                                 D * BN);
}

// One workgroup per (partial, query tile, query head); kThreads threads. Partial
// ph < H: context block ph, every key visible. Partial H: the query block's own keys,
// causal. NG = (H + 1) * qtiles * Hkv groups of G workgroups; the grid is
// round_up(NG, 8) * G workgroups, mapped like the main attention so the G heads of one
// KV group run on one XCD and read each K/V tile through its L2 once.
template <int D>
__global__ __launch_bounds__(kThreads) void query_partial_kernel(
    Plan p, int64_t nq, int qtiles, int NG, const uint16_t* __restrict__ q_qr,
    const uint16_t* __restrict__ k_qr, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ vtctx, const uint16_t* __restrict__ vtq,
    float* __restrict__ part_o, float* __restrict__ part_lse, float c_log2) {
  using C = Cfg<D>;
  __shared__ __attribute__((aligned(16))) char smem[3 * C::STAGE];
  const int b = blockIdx.x;
  const int xcd = b & 7, slot = b >> 3;
  const int gs = (slot / p.G) * 8 + xcd;
  if (gs >= NG) return;
  const int hl = slot % p.G;
  const int g = gs % p.Hkv, hq = g * p.G + hl;
  const int ph = (gs / p.Hkv) / qtiles, qt = (gs / p.Hkv) % qtiles;
  const bool self = ph == p.H;
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int lr = lane & 31, lh = lane >> 5;
  const int64_t q0 = static_cast<int64_t>(qt) * kQTile;
  const int64_t qw0 = q0 + static_cast<int64_t>(kWaveQ) * w;
  const int64_t qi = qw0 + lr;
  const bool wave_active = qw0 < nq;

  const int64_t s = static_cast<int64_t>(ph) * p.nb;   // context block start
  const int qkt = static_cast<int>((nq + BN - 1) / BN);
  const int ntiles = self ? static_cast<int>((min(nq, q0 + kQTile) + BN - 1) / BN) : p.loc_tiles;
  const uint16_t* kbase = self ? k_qr + g * p.kvs_head : k + s * p.kvs_tok + g * p.kvs_head;
  const int64_t nkeys = self ? nq : p.nb;
  const uint16_t* vtbase = self ? vtq + static_cast<int64_t>(g) * qkt * D * BN
                                : vtctx + (static_cast<int64_t>(g) * p.H + ph) * p.loc_tiles * D * BN;

  TileDma<D> dma;
  dma.init(p.kvs_tok);
  auto issue_tile = [&](int it, char* dst) {
    const int64_t key0 = static_cast<int64_t>(it) * BN;
    const int64_t rows = nkeys - key0 < BN ? nkeys - key0 : BN;
    dma.issue(kbase + key0 * p.kvs_tok, true, TileDma<D>::k_range(rows, p.kvs_tok),
              vtbase + static_cast<int64_t>(it) * D * BN, dst);
  };

  bf16x8 qf[C::DK];
  load_q<D>(q_qr + qi * p.qs_tok + hq * p.qs_head + lh * 8, qi < nq, qf);
  Flash<D> f;
  f.init();

  // The main attention's three-stage ring: while tile it is computed, tile it+1 is
  // complete (its first K fragments are read during tile it's P V) and tile it+2 is in
  // flight.
  if (ntiles > 0) issue_tile(0, smem);
  if (ntiles > 1) issue_tile(1, smem + C::STAGE);
  wait_tile_loads();
  __syncthreads();
  int st = 0;   // stage of tile it
  if (!wave_active) {
    // No queries in this wave: it only loads its share of every tile. (Decided once,
    // outside the loop: a branch around the tile step inside it made the compiler copy
    // the O accumulators and the prefetched K fragments on every tile.)
    for (int it = 0; it < ntiles; ++it) {
      const int st1 = st == 2 ? 0 : st + 1, st2 = st1 == 2 ? 0 : st1 + 1;
      if (it + 2 < ntiles) issue_tile(it + 2, smem + st2 * C::STAGE);
      wait_tile_loads();
      __syncthreads();
      st = st1;
    }
  } else {
    KHead<D> kh;
    if (ntiles > 0) kh.read(smem);
    for (int it = 0; it < ntiles; ++it) {
      const int st1 = st == 2 ? 0 : st + 1, st2 = st1 == 2 ? 0 : st1 + 1;
      if (it + 2 < ntiles) issue_tile(it + 2, smem + st2 * C::STAGE);
      const int64_t key0 = static_cast<int64_t>(it) * BN;
      // Hide keys past the segment end; in the query block also keys after the query
      // (tiles past all of the wave's queries run fully masked: limit -1, every weight
      // 0, the state unchanged).
      int64_t lim = nkeys - key0 - 1;
      if (self && qi - key0 < lim) lim = qi - key0;
      if (lim < -1) lim = -1;
      const int lim32 = lim < BN - 1 ? static_cast<int>(lim) : BN - 1;
      attend_tile<D, true>(kh, smem + st * C::STAGE,
                           it + 1 < ntiles ? smem + st1 * C::STAGE : nullptr, qf, f,
                           __any(lim32 < BN - 1) != 0, [=]() { return lim32; }, c_log2);
      wait_tile_loads();   // tile it+2
      __syncthreads();
      st = st1;
    }
  }
  const float ltot = flash_rowsum<D>(f);       // float32 weights: the LSE
  const float ltot_b = flash_rowsum_b<D>(f);   // bf16 weights: normalises O
  if (qi < nq) {
    const float inv = 1.f / ltot_b;
    float* op = part_o + ((static_cast<int64_t>(ph) * nq + qi) * p.Hq + hq) * D;
#pragma unroll
    for (int dm = 0; dm < C::DM; ++dm)
#pragma unroll
      for (int grp = 0; grp < 4; ++grp) {
        const float4 v4 = make_float4(f.o[dm][grp * 4] * inv, f.o[dm][grp * 4 + 1] * inv,
                                      f.o[dm][grp * 4 + 2] * inv, f.o[dm][grp * 4 + 3] * inv);
        *reinterpret_cast<float4*>(op + out_dim<D>(dm, grp, lh)) = v4;
      }
    if (lh == 0)
      part_lse[(static_cast<int64_t>(ph) * p.Hq + hq) * nq + qi] =
          (f.mrun + log2f(ltot)) * 0.69314718055994531f;
  }
}

// float32 inputs on the float64 matrix cores (F64Flash); grid
// ((H + 1) * ceil(nq / 64), Hq), four waves of 16 rows.
template <int D>
__global__ __launch_bounds__(256, 2) void query_partial_f32_kernel(
    Plan p, int64_t nq, int qtiles, const float* __restrict__ q_qr, const float* __restrict__ k_qr,
    const float* __restrict__ v_qr, const float* __restrict__ k, const float* __restrict__ v,
    float* __restrict__ part_o, double* __restrict__ part_lse) {
  __shared__ __attribute__((aligned(16))) F64Tile<D> tile;
  const int ph = blockIdx.x / qtiles, qt = blockIdx.x % qtiles;
  const int hq = blockIdx.y, g = hq / p.G;
  const bool self = ph == p.H;
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t qi = static_cast<int64_t>(qt) * kF64QTile + w * 16 + (lane & 15);
  const bool valid = qi < nq;
  const int64_t q_last = min(static_cast<int64_t>(qt + 1) * kF64QTile, nq) - 1;
  const float* kb = self ? k_qr : k + static_cast<int64_t>(ph) * p.nb * p.kvs_tok;
  const float* vb = self ? v_qr : v + static_cast<int64_t>(ph) * p.nb * p.kvs_tok;
  const int64_t nkeys = self ? q_last + 1 : p.nb;

  F64Flash<D> f;
  f.init(valid ? q_qr + qi * p.qs_tok + hq * p.qs_head : nullptr);
  for (int64_t key0 = 0; key0 < nkeys; key0 += BN) {
    __syncthreads();
    f64_load_tile<D>(tile, kb + key0 * p.kvs_tok + g * p.kvs_head,
                     vb + key0 * p.kvs_tok + g * p.kvs_head, p.kvs_tok,
                     static_cast<int>(min<int64_t>(BN, nkeys - key0)));
    __syncthreads();
    // Visible keys form a prefix of the tile: all present keys of a context block, the
    // query keys up to the row itself.
    int64_t lim = nkeys - 1 - key0;
    if (self) lim = min(lim, qi - key0);
    f.step(tile, valid ? static_cast<int>(min<int64_t>(lim, BN - 1)) : -1, p.scale);
  }
  f.finish();
  if (!valid) return;
  f.store(part_o + ((static_cast<int64_t>(ph) * nq + qi) * p.Hq + hq) * D);
  // The partial's LSE is kept in float64 for the merge weights exp(LSE_h - LSE).
  if ((lane >> 4) == 0) part_lse[(static_cast<int64_t>(ph) * p.Hq + hq) * nq + qi] = f.lse();
}

__device__ inline void store4(uint16_t* dst, float4 v) {
  f32x2 lo = {v.x, v.y}, hi = {v.z, v.w};
  uint2 pk;
  pk.x = __builtin_bit_cast(uint32_t, __builtin_convertvector(lo, bf16x2));
  pk.y = __builtin_bit_cast(uint32_t, __builtin_convertvector(hi, bf16x2));
  *reinterpret_cast<uint2*>(dst) = pk;
}
__device__ inline void store4(float* dst, float4 v) { *reinterpret_cast<float4*>(dst) = v; }

// One thread per (row, head, 4 dims): LSE merge of the H + 1 partials, computed in the
// precision L of the stored partial LSEs (float for bf16 outputs, double for float32).
template <typename T, typename L>
__global__ __launch_bounds__(256) void query_merge_kernel(Plan p, int64_t nq,
                                                          const float* __restrict__ part_o,
                                                          const L* __restrict__ part_lse,
                                                          T* __restrict__ out,
                                                          float* __restrict__ lse) {
  const int64_t t = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int dq = p.D / 4;
  if (t >= nq * p.Hq * dq) return;
  const int d4 = static_cast<int>(t % dq);
  const int64_t rh = t / dq;
  const int hq = static_cast<int>(rh % p.Hq);
  const int64_t qi = rh / p.Hq;
  L m = -INFINITY;
  for (int ph = 0; ph <= p.H; ++ph)
    m = fmax(m, part_lse[(static_cast<int64_t>(ph) * p.Hq + hq) * nq + qi]);
  L ssum = 0;
  for (int ph = 0; ph <= p.H; ++ph)
    ssum += exp(part_lse[(static_cast<int64_t>(ph) * p.Hq + hq) * nq + qi] - m);
  const L total = m + log(ssum);
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int ph = 0; ph <= p.H; ++ph) {
    const float wgt =
        static_cast<float>(exp(part_lse[(static_cast<int64_t>(ph) * p.Hq + hq) * nq + qi] - total));
    const float4 o = *reinterpret_cast<const float4*>(
        part_o + ((static_cast<int64_t>(ph) * nq + qi) * p.Hq + hq) * p.D + d4 * 4);
    acc.x = fmaf(wgt, o.x, acc.x);
    acc.y = fmaf(wgt, o.y, acc.y);
    acc.z = fmaf(wgt, o.z, acc.z);
    acc.w = fmaf(wgt, o.w, acc.w);
  }
  store4(out + qi * p.os_tok + hq * p.os_head + d4 * 4, acc);
  if (lse && d4 == 0) lse[static_cast<int64_t>(hq) * nq + qi] = static_cast<float>(total);
}

template <int D>
hipError_t launch_query_bf16(const Plan& p, int64_t nq, const uint16_t* q_qr, const uint16_t* k_qr,
                             const uint16_t* v_qr, const uint16_t* k, const uint16_t* v,
                             uint16_t* out, float* lse, char* ws, hipStream_t st) {
  const QueryWs w = query_ws_layout(p, nq);
  float* part_o = reinterpret_cast<float*>(ws + w.part_o);
  float* part_lse = reinterpret_cast<float*>(ws + w.part_lse);
  uint16_t* vtctx = reinterpret_cast<uint16_t*>(ws + w.vtctx);
  uint16_t* vtq = reinterpret_cast<uint16_t*>(ws + w.vtq);
  const int qkt = static_cast<int>(cdiv(nq, BN));
  hipLaunchKernelGGL(vt_rows_kernel<D>, dim3(static_cast<unsigned>(p.H * p.loc_tiles), p.Hkv),
                     dim3(256), 0, st, v, static_cast<int64_t>(p.nb), p.H, p.loc_tiles, p.kvs_tok,
                     p.kvs_head, vtctx);
  hipLaunchKernelGGL(vt_rows_kernel<D>, dim3(static_cast<unsigned>(qkt), p.Hkv), dim3(256), 0, st,
                     v_qr, nq, 1, qkt, p.kvs_tok, p.kvs_head, vtq);
  const int qtiles = static_cast<int>(cdiv(nq, kQTile));
  const float c_log2 = static_cast<float>(p.scale * 1.4426950408889634);
  const int NG = (p.H + 1) * qtiles * p.Hkv;
  const int64_t groups = round_up(NG, 8) * p.G;
  hipLaunchKernelGGL(query_partial_kernel<D>, dim3(static_cast<unsigned>(groups)), dim3(kThreads), 0,
                     st, p, nq, qtiles, NG, q_qr, k_qr, k, vtctx, vtq, part_o, part_lse, c_log2);
  const int64_t threads = nq * p.Hq * (p.D / 4);
  const dim3 mgrid(static_cast<unsigned>(cdiv(threads, 256)));
  hipLaunchKernelGGL((query_merge_kernel<uint16_t, float>), mgrid, dim3(256), 0, st, p, nq, part_o,
                     part_lse, out, lse);
  return hipGetLastError();
}

template <int D>
hipError_t launch_query_f32(const Plan& p, int64_t nq, const float* q_qr, const float* k_qr,
                            const float* v_qr, const float* k, const float* v, float* out,
                            float* lse, char* ws, hipStream_t st) {
  const QueryWs w = query_ws_layout(p, nq);
  float* part_o = reinterpret_cast<float*>(ws + w.part_o);
  double* part_lse = reinterpret_cast<double*>(ws + w.part_lse);
  const int qtiles = static_cast<int>(cdiv(nq, kF64QTile));
  hipLaunchKernelGGL(query_partial_f32_kernel<D>,
                     dim3(static_cast<unsigned>((p.H + 1) * qtiles), p.Hq), dim3(256), 0, st, p,
                     nq, qtiles, q_qr, k_qr, v_qr, k, v, part_o, part_lse);
  const int64_t threads = nq * p.Hq * (p.D / 4);
  const dim3 mgrid(static_cast<unsigned>(cdiv(threads, 256)));
  hipLaunchKernelGGL((query_merge_kernel<float, double>), mgrid, dim3(256), 0, st, p, nq, part_o,
                     part_lse, out, lse);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_query(const Plan& p, int64_t nq, const void* q_qr, const void* k_qr,
                        const void* v_qr, const void* k, const void* v, void* out, float* lse,
                        char* ws, hipStream_t st) {
  if (p.dtype == SPAVA_BF16) {
    auto c = [](const void* x) { return static_cast<const uint16_t*>(x); };
    auto o = static_cast<uint16_t*>(out);
    if (p.D == 128)
      return launch_query_bf16<128>(p, nq, c(q_qr), c(k_qr), c(v_qr), c(k), c(v), o, lse, ws, st);
    return launch_query_bf16<64>(p, nq, c(q_qr), c(k_qr), c(v_qr), c(k), c(v), o, lse, ws, st);
  }
  auto c = [](const void* x) { return static_cast<const float*>(x); };
  auto o = static_cast<float*>(out);
  if (p.D == 128)
    return launch_query_f32<128>(p, nq, c(q_qr), c(k_qr), c(v_qr), c(k), c(v), o, lse, ws, st);
  return launch_query_f32<64>(p, nq, c(q_qr), c(k_qr), c(v_qr), c(k), c(v), o, lse, ws, st);
}

}  // namespace spava
