// Approximate attention, float32 inputs (float64 matrix cores, float64 arithmetic).
//
// Same visible set as the bf16 path (explainer "APB-V: ...", Methodik >
// Approximativer Attention-Mechanismus > Berechnung): anchor + passing rows of the
// earlier blocks, then the block's own causal keys. Float64 arithmetic except the
// float32 exponentials, as in the lane-pair step the query-block partials use
// (attn_f32_step.h). A workgroup of four waves covers 64 consecutive queries of one
// head and streams 64-key K/V tiles through LDS.
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

// float64 matrix cores: v_mfma_f64_16x16x4_f64 (wave64). Lane l supplies row (l % 16)
// of A and column (l % 16) of B at reduction slot l / 16; accumulator element r of
// lane l holds row 4r + l/16, column l % 16.
//
// One wave = 16 queries of one head; a workgroup of four waves covers 64 queries and
// streams 64-key tiles of K and V (float32, widened at each use) through LDS.
//   S^T = K Q^T: A = K (16 keys), B = Q^T (16 queries); lane l holds the head-dim
//        quarter l/16 of its query's q (32 values at d = 128), one MFMA per
//        dimension of the quarter. Element r of lane l's block kb is key
//        16 kb + 4r + l/16 of query l % 16.
//   O^T += V^T P^T: A = V^T (16 head dims), B = P^T; k-step r of key block kb takes
//        the keys 16 kb + 4r + s (slot s = l/16), so lane l's B operand is its own
//        element r: P stays in registers. V^T is stored with the keys of each 16-key
//        block permuted (key 4r + s at slot 4s + r), so a lane's four A operands of a
//        block are one 16-byte LDS read.
// Softmax per tile against the running maximum: logits, maximum, weights' sum and O
// in float64, the weights exp(x - m) evaluated in float32 (as in the lane-pair path).
constexpr int kF64Waves = 4;
constexpr int kF64QTile = kF64Waves * 16;   // queries per workgroup

typedef double f64x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

template <int D>
struct F64Cfg {
  static constexpr int KSTR = D + 4;     // K row stride in LDS (floats)
  static constexpr int VSTR = BN + 4;    // V^T row stride in LDS (floats)
  static constexpr int QD = D / 4;       // head dims per lane (its reduction-slot quarter)
  static constexpr int DB = D / 16;      // 16-row blocks of O^T
};

// V^T column of key `row` of a tile: within each 16-key block, key 4r + s -> slot 4s + r.
__device__ inline int f64_vslot(int row) {
  return (row & ~15) + 4 * (row & 3) + ((row & 15) >> 2);
}

// grid (H * ceil(nb / 64), Hq), block 256.
template <int D>
__global__ __launch_bounds__(256, 2) void attn_f32_mfma_kernel(
    Plan p, const float* __restrict__ q, const float* __restrict__ k,
    const float* __restrict__ v, const float* __restrict__ kpre,
    const float* __restrict__ vpre, float* __restrict__ out, float* __restrict__ lse) {
  using C = F64Cfg<D>;
  __shared__ __attribute__((aligned(16))) float ks[BN * C::KSTR];
  __shared__ __attribute__((aligned(16))) float vts[D * C::VSTR];
  const int tiles_per_block = (p.nb + kF64QTile - 1) / kF64QTile;
  const int h = blockIdx.x / tiles_per_block, qt = blockIdx.x % tiles_per_block;
  const int hq = blockIdx.y, g = hq / p.G;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int lq = lane & 15, lg = lane >> 4;
  const int64_t s_h = static_cast<int64_t>(h) * p.nb, e_h = s_h + p.nb;
  const int64_t qi = s_h + static_cast<int64_t>(qt) * kF64QTile + w * 16 + lq;
  const bool valid = qi < e_h;
  const int64_t q_last = min(s_h + static_cast<int64_t>(qt + 1) * kF64QTile, e_h) - 1;

  float qf[C::QD];
#pragma unroll
  for (int c = 0; c < C::QD / 4; ++c) {
    f32x4 x4 = {0.f, 0.f, 0.f, 0.f};
    if (valid)
      x4 = *reinterpret_cast<const f32x4*>(q + qi * p.qs_tok + hq * p.qs_head + lg * C::QD + 4 * c);
#pragma unroll
    for (int e = 0; e < 4; ++e) qf[4 * c + e] = x4[e];
  }
  f64x4 o[C::DB];
#pragma unroll
  for (int db = 0; db < C::DB; ++db) o[db] = f64x4{0.0, 0.0, 0.0, 0.0};
  double m = -INFINITY, l = 0.0;

  const int L = prefix_len(p, h);
  const int npre = (L + BN - 1) / BN;
  const int nloc = static_cast<int>((q_last - s_h) / BN) + 1;
  for (int it = 0; it < npre + nloc; ++it) {
    const bool local = it >= npre;
    const int64_t key0 = local ? s_h + static_cast<int64_t>(it - npre) * BN
                               : static_cast<int64_t>(it) * BN;
    const int nrows = local ? static_cast<int>(min<int64_t>(BN, e_h - key0)) : BN;
    const float* kb0 = local ? k + key0 * p.kvs_tok + g * p.kvs_head
                             : kpre + (static_cast<int64_t>(g) * p.Lpad + key0) * D;
    const float* vb0 = local ? v + key0 * p.kvs_tok + g * p.kvs_head
                             : vpre + (static_cast<int64_t>(g) * p.Lpad + key0) * D;
    const int64_t rstride = local ? p.kvs_tok : D;
    __syncthreads();   // the previous tile is no longer read
    for (int c = tid; c < BN * (D / 4); c += 256) {
      const int row = c / (D / 4), c4 = c % (D / 4);
      f32x4 kk = {0.f, 0.f, 0.f, 0.f}, vv = {0.f, 0.f, 0.f, 0.f};
      if (row < nrows) {
        kk = *reinterpret_cast<const f32x4*>(kb0 + row * rstride + 4 * c4);
        vv = *reinterpret_cast<const f32x4*>(vb0 + row * rstride + 4 * c4);
      }
      *reinterpret_cast<f32x4*>(&ks[row * C::KSTR + 4 * c4]) = kk;
      const int slot = f64_vslot(row);
#pragma unroll
      for (int e = 0; e < 4; ++e) vts[(4 * c4 + e) * C::VSTR + slot] = vv[e];
    }
    __syncthreads();
    // Keys kk <= lim of the tile are visible to this lane's query: the prefix rows
    // below L, or the causal keys up to the query itself; none for a padding row.
    int64_t lim = local ? qi - key0 : static_cast<int64_t>(L) - key0 - 1;
    if (!valid) lim = -1;
    const int lim32 = static_cast<int>(min<int64_t>(lim, BN - 1));

    f64x4 sacc[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      sacc[kb] = f64x4{0.0, 0.0, 0.0, 0.0};
#pragma unroll
      for (int c = 0; c < C::QD / 4; ++c) {
        const f32x4 kv = *reinterpret_cast<const f32x4*>(&ks[(kb * 16 + lq) * C::KSTR + lg * C::QD + 4 * c]);
#pragma unroll
        for (int e = 0; e < 4; ++e)
          sacc[kb] = __builtin_amdgcn_mfma_f64_16x16x4f64(static_cast<double>(kv[e]),
                                                          static_cast<double>(qf[4 * c + e]),
                                                          sacc[kb], 0, 0, 0);
      }
    }
    // Logits, tile maximum of this lane's query (its keys, then across the four lane
    // groups that hold the query's other keys), running maximum and rescale.
    double mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int kk = kb * 16 + 4 * r + lg;
        const double x = kk <= lim32 ? sacc[kb][r] * p.scale : -INFINITY;
        sacc[kb][r] = x;
        mx = fmax(mx, x);
      }
    mx = fmax(mx, __shfl_xor(mx, 16));
    mx = fmax(mx, __shfl_xor(mx, 32));
    if (mx > m) {
      const double alpha = exp(m - mx);   // m = -inf gives 0
      l *= alpha;
#pragma unroll
      for (int db = 0; db < C::DB; ++db) o[db] *= alpha;
      m = mx;
    }
    const bool none = m == -INFINITY;     // nothing visible yet: every weight is 0
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const double pe =
            none ? 0.0 : static_cast<double>(expf(static_cast<float>(sacc[kb][r] - m)));
        sacc[kb][r] = pe;
        l += pe;
      }
    // O^T += V^T P^T
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const f32x4 vv = *reinterpret_cast<const f32x4*>(&vts[(db * 16 + lq) * C::VSTR + kb * 16 + 4 * lg]);
#pragma unroll
        for (int r = 0; r < 4; ++r)
          o[db] = __builtin_amdgcn_mfma_f64_16x16x4f64(static_cast<double>(vv[r]), sacc[kb][r],
                                                       o[db], 0, 0, 0);
      }
  }
  // The query's weight sum over the four lane groups; element r of block db is head
  // dim 16 db + 4r + lg of query qi.
  l += __shfl_xor(l, 16);
  l += __shfl_xor(l, 32);
  if (!valid) return;
  const double inv = 1.0 / l;
  float* orow = out + qi * p.os_tok + hq * p.os_head;
#pragma unroll
  for (int db = 0; db < C::DB; ++db)
#pragma unroll
    for (int r = 0; r < 4; ++r) orow[16 * db + 4 * r + lg] = static_cast<float>(o[db][r] * inv);
  if (lse && lg == 0) lse[static_cast<int64_t>(hq) * p.N + qi] = static_cast<float>(m + log(l));
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
