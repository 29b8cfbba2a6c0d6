// Approximate attention, float32 inputs (float64 matrix cores, float64 arithmetic).
//
// Same visible set as the bf16 path (explainer "APB-V: ...", Methodik >
// Approximativer Attention-Mechanismus > Berechnung): anchor + passing rows of the
// earlier blocks, then the block's own causal keys. Float64 arithmetic except the
// float32 exponentials (the tile step of attn_f32_step.h). A workgroup of four waves
// covers 64 consecutive queries of one head and streams 64-key K/V tiles through LDS.
#include "attn_f32_step.h"

namespace spava {
namespace {

constexpr int BN = kKeyTile;

// Contiguous prefix copies Kpre/Vpre [Hkv][Lpad][D]; grid (Lpad/64, Hkv).
template <int D>
__global__ __launch_bounds__(256) void prep_f32_kernel(Plan p, const float* __restrict__ k,
                                                       const float* __restrict__ v,
                                                       const int32_t* __restrict__ idx,
                                                       float* __restrict__ kpre,
                                                       float* __restrict__ vpre) {
  const int g = blockIdx.y;
  const int r0 = blockIdx.x * BN;
  constexpr int CPR = D / 4;
  for (int c = threadIdx.x; c < BN * CPR; c += 256) {
    const int row = c / CPR, col = c % CPR;
    const int64_t tok = prefix_source(p, idx, g, r0 + row);
    float4 kk = make_float4(0, 0, 0, 0), vv = make_float4(0, 0, 0, 0);
    if (tok >= 0) {
      const int64_t off = tok * p.kvs_tok + g * p.kvs_head + col * 4;
      kk = *reinterpret_cast<const float4*>(k + off);
      vv = *reinterpret_cast<const float4*>(v + off);
    }
    const int64_t dst = (static_cast<int64_t>(g) * p.Lpad + r0 + row) * D + col * 4;
    *reinterpret_cast<float4*>(kpre + dst) = kk;
    *reinterpret_cast<float4*>(vpre + dst) = vv;
  }
}

// grid (H * ceil(nb / 64), Hq), block 256: four waves of 16 queries (F64Flash).
template <int D>
__global__ __launch_bounds__(256, 2) void attn_f32_mfma_kernel(
    Plan p, const float* __restrict__ q, const float* __restrict__ k,
    const float* __restrict__ v, const float* __restrict__ kpre,
    const float* __restrict__ vpre, float* __restrict__ out, float* __restrict__ lse) {
  __shared__ __attribute__((aligned(16))) F64Tile<D> tile;
  const int tiles_per_block = (p.nb + kF64QTile - 1) / kF64QTile;
  const int h = blockIdx.x / tiles_per_block, qt = blockIdx.x % tiles_per_block;
  const int hq = blockIdx.y, g = hq / p.G;
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t s_h = static_cast<int64_t>(h) * p.nb, e_h = s_h + p.nb;
  const int64_t qi = s_h + static_cast<int64_t>(qt) * kF64QTile + w * 16 + (lane & 15);
  const bool valid = qi < e_h;
  const int64_t q_last = min(s_h + static_cast<int64_t>(qt + 1) * kF64QTile, e_h) - 1;

  F64Flash<D> f;
  f.init(valid ? q + qi * p.qs_tok + hq * p.qs_head : nullptr);
  const int L = prefix_len(p, h);
  const int npre = (L + BN - 1) / BN;
  const int nloc = static_cast<int>((q_last - s_h) / BN) + 1;
  for (int it = 0; it < npre + nloc; ++it) {
    const bool local = it >= npre;
    const int64_t key0 = local ? s_h + static_cast<int64_t>(it - npre) * BN
                               : static_cast<int64_t>(it) * BN;
    __syncthreads();   // the previous tile is no longer read
    if (local)
      f64_load_tile<D>(tile, k + key0 * p.kvs_tok + g * p.kvs_head,
                       v + key0 * p.kvs_tok + g * p.kvs_head, p.kvs_tok,
                       static_cast<int>(min<int64_t>(BN, e_h - key0)));
    else
      f64_load_tile<D>(tile, kpre + (static_cast<int64_t>(g) * p.Lpad + key0) * D,
                       vpre + (static_cast<int64_t>(g) * p.Lpad + key0) * D, D, BN);
    __syncthreads();
    // Visible keys of the tile form a prefix: the prefix rows below L, or the causal
    // keys up to the query itself; none for a padding row.
    const int64_t lim = local ? qi - key0 : static_cast<int64_t>(L) - key0 - 1;
    f.step(tile, valid ? static_cast<int>(min<int64_t>(lim, BN - 1)) : -1, p.scale);
  }
  f.finish();
  if (!valid) return;
  f.store(out + qi * p.os_tok + hq * p.os_head);
  if (lse && (lane >> 4) == 0) lse[static_cast<int64_t>(hq) * p.N + qi] = static_cast<float>(f.lse());
}

template <int D>
hipError_t launch_f32_d(const Plan& p, const float* q, const float* k, const float* v,
                        const int32_t* idx, float* out, float* lse, char* ws, hipStream_t st) {
  const AttnWs w = attn_ws_layout(p);
  float* kpre = reinterpret_cast<float*>(ws + w.kpre);
  float* vpre = reinterpret_cast<float*>(ws + w.vpre);
  if (p.Lpad > 0)
    hipLaunchKernelGGL(prep_f32_kernel<D>, dim3(p.Lpad / BN, p.Hkv), dim3(256), 0, st, p, k, v,
                       idx, kpre, vpre);
  const unsigned gx = static_cast<unsigned>(p.H * cdiv(p.nb, kF64QTile));
  hipLaunchKernelGGL(attn_f32_mfma_kernel<D>, dim3(gx, p.Hq), dim3(256), 0, st, p, q, k, v,
                     kpre, vpre, out, lse);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_f32(const Plan& p, const void* q, const void* k, const void* v,
                           const int32_t* idx, void* out, float* lse, char* ws, hipStream_t st) {
  auto qq = static_cast<const float*>(q);
  auto kk = static_cast<const float*>(k);
  auto vv = static_cast<const float*>(v);
  auto oo = static_cast<float*>(out);
  if (p.D == 128) return launch_f32_d<128>(p, qq, kk, vv, idx, oo, lse, ws, st);
  return launch_f32_d<64>(p, qq, kk, vv, idx, oo, lse, ws, st);
}

}  // namespace spava
