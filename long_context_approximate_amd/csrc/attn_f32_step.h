// float32-input attention step on the float64 matrix cores, shared by the main float32
// attention and the query block's float32 partials.
//
// v_mfma_f64_16x16x4_f64 (wave64): lane l supplies row (l % 16) of A and column (l % 16)
// of B at reduction slot l / 16; accumulator element r of lane l holds row 4r + l/16,
// column l % 16.
//
// One wave = 16 queries of one head; a workgroup of four waves covers 64 queries and
// streams 64-key tiles of K and V (float32 in LDS, widened at each use).
//   S^T = K Q^T: A = K (16 keys), B = Q^T (16 queries); lane l holds the head-dim
//        quarter l/16 of its query's q (32 values at d = 128), one MFMA per
//        dimension of the quarter. Element r of lane l's block kb is key
//        16 kb + 4r + l/16 of query l % 16.
//   O^T += V^T P^T: A = V^T (16 head dims), B = P^T; k-step r of key block kb takes
//        the keys 16 kb + 4r + s (slot s = l/16), so lane l's B operand is its own
//        element r: P stays in registers. V^T is stored with the keys of each 16-key
//        block permuted (key 4r + s at slot 4s + r), so a lane's four A operands of a
//        block are one 16-byte LDS read.
// Logits, the running maximum (per tile), the weights' sum and O are float64; only the
// weights exp(x - m) are evaluated in float32 and widened. With float32 arithmetic
// instead, three error sources each reach the 1e-5 bar on heavy-tailed keys (the
// denominator dropping many tiny weights in one direction, the rounding of logits of
// magnitude ~30, float32 O sums over thousands of keys).
#pragma once

#include "spava_internal.h"

namespace spava {

constexpr int kF64Waves = 4;
constexpr int kF64QTile = kF64Waves * 16;   // queries per workgroup
constexpr int kF64Keys = kKeyTile;          // keys per LDS tile

typedef double f64x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

template <int D>
struct F64Cfg {
  static constexpr int KSTR = D + 4;          // K row stride in LDS (floats)
  static constexpr int VSTR = kF64Keys + 4;   // V^T row stride in LDS (floats)
  static constexpr int QD = D / 4;            // head dims per lane (its reduction-slot quarter)
  static constexpr int DB = D / 16;           // 16-row blocks of O^T
};

// V^T column of key `row` of a tile: within each 16-key block, key 4r + s -> slot 4s + r.
__device__ inline int f64_vslot(int row) {
  return (row & ~15) + 4 * (row & 3) + ((row & 15) >> 2);
}

template <int D>
struct F64Tile {
  float k[kF64Keys * F64Cfg<D>::KSTR];
  float vt[D * F64Cfg<D>::VSTR];
};

// Fill the tile with rows [0, nrows) of K and V starting at kb0 / vb0 (row stride
// `rstride` floats; rows past nrows are zeros). All 256 threads of the workgroup call it.
template <int D>
__device__ inline void f64_load_tile(F64Tile<D>& t, const float* kb0, const float* vb0,
                                     int64_t rstride, int nrows) {
  using C = F64Cfg<D>;
  for (int c = threadIdx.x; c < kF64Keys * (D / 4); c += kF64Waves * 64) {
    const int row = c / (D / 4), c4 = c % (D / 4);
    f32x4 kk = {0.f, 0.f, 0.f, 0.f}, vv = {0.f, 0.f, 0.f, 0.f};
    if (row < nrows) {
      kk = *reinterpret_cast<const f32x4*>(kb0 + row * rstride + 4 * c4);
      vv = *reinterpret_cast<const f32x4*>(vb0 + row * rstride + 4 * c4);
    }
    *reinterpret_cast<f32x4*>(&t.k[row * C::KSTR + 4 * c4]) = kk;
    const int slot = f64_vslot(row);
#pragma unroll
    for (int e = 0; e < 4; ++e) t.vt[(4 * c4 + e) * C::VSTR + slot] = vv[e];
  }
}

// One wave's 16 queries; lane l holds query l % 16.
template <int D>
struct F64Flash {
  using C = F64Cfg<D>;
  float qf[C::QD];
  f64x4 o[C::DB];
  double m, l;   // running maximum; this lane's partial weight sum (its keys)

  // qrow: the query's d values, or null for a padding row (zeros).
  __device__ void init(const float* qrow) {
    const int lg = (threadIdx.x & 63) >> 4;
#pragma unroll
    for (int c = 0; c < C::QD / 4; ++c) {
      f32x4 x4 = {0.f, 0.f, 0.f, 0.f};
      if (qrow) x4 = *reinterpret_cast<const f32x4*>(qrow + lg * C::QD + 4 * c);
#pragma unroll
      for (int e = 0; e < 4; ++e) qf[4 * c + e] = x4[e];
    }
#pragma unroll
    for (int db = 0; db < C::DB; ++db) o[db] = f64x4{0.0, 0.0, 0.0, 0.0};
    m = -INFINITY;
    l = 0.0;
  }

  // Keys kk <= lim (< 0: none) of the tile are visible to this lane's query.
  __device__ void step(const F64Tile<D>& t, int lim, double scale) {
    const int lane = threadIdx.x & 63;
    const int lq = lane & 15, lg = lane >> 4;
    f64x4 sacc[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      sacc[kb] = f64x4{0.0, 0.0, 0.0, 0.0};
#pragma unroll
      for (int c = 0; c < C::QD / 4; ++c) {
        const f32x4 kv =
            *reinterpret_cast<const f32x4*>(&t.k[(kb * 16 + lq) * C::KSTR + lg * C::QD + 4 * c]);
#pragma unroll
        for (int e = 0; e < 4; ++e)
          sacc[kb] = __builtin_amdgcn_mfma_f64_16x16x4f64(static_cast<double>(kv[e]),
                                                          static_cast<double>(qf[4 * c + e]),
                                                          sacc[kb], 0, 0, 0);
      }
    }
    // Logits; the tile maximum of this lane's query (its keys, then across the four
    // lane groups that hold the query's other keys); running maximum and rescale.
    double mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const double x = kb * 16 + 4 * r + lg <= lim ? sacc[kb][r] * scale : -INFINITY;
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
        const f32x4 vv =
            *reinterpret_cast<const f32x4*>(&t.vt[(db * 16 + lq) * C::VSTR + kb * 16 + 4 * lg]);
#pragma unroll
        for (int r = 0; r < 4; ++r)
          o[db] = __builtin_amdgcn_mfma_f64_16x16x4f64(static_cast<double>(vv[r]), sacc[kb][r],
                                                       o[db], 0, 0, 0);
      }
  }

  // The query's weight sum over the four lane groups (all lanes of the wave call it).
  __device__ void finish() {
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
  }
  // Write O / l for this lane's query to orow (its d values), rounded to float32:
  // element r of block db is head dim 16 db + 4r + lane/16.
  __device__ void store(float* orow) const {
    const int lg = (threadIdx.x & 63) >> 4;
    const double inv = 1.0 / l;
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
      for (int r = 0; r < 4; ++r) orow[16 * db + 4 * r + lg] = static_cast<float>(o[db][r] * inv);
  }
  __device__ double lse() const { return m + log(l); }
};

}  // namespace spava
