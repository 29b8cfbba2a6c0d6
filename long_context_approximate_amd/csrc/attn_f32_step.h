// float32-input attention step shared by the main float32 attention and the query-block
// float32 partials.
//
// One query row is owned by a lane pair (l, l ^ 32) of a wave: each lane holds half of
// the head dimension of q and of the O numerators. The logits are float64 dot
// products (the two halves combined by a cross-half shuffle, so both lanes hold the
// same value), the running maximum, the softmax denominator and the O numerators are
// float64; only the exponentials are float32. Float32 logits of magnitude ~30 (heavy-
// tailed keys) carry ~1e-5 of rounding into the LSE, and float32 sums over thousands
// of keys random-walk to a similar error in O; this layout avoids both while keeping
// 64 float + 64 double registers per lane at d = 128.
#pragma once

#include "spava_internal.h"

namespace spava {

constexpr int kF32Tile = kKeyTile;   // keys per LDS tile

template <int D>
struct F32Cfg {
  static constexpr int H = D / 2;        // head dims per lane
  static constexpr int ROW = 2 * (H + 1);  // LDS row: two halves, each padded by one
};

// LDS tile: K widened to float64, V as float32; row kk holds key kk, the half of lane
// pair member `half` at offset half * (H + 1) (the pad keeps the halves in different banks).
template <int D>
struct F32Tile {
  double k[kF32Tile][F32Cfg<D>::ROW];
  float v[kF32Tile][F32Cfg<D>::ROW];
};

// Fill the tile with `nrows` rows read by `row_ptr(r)` (a pointer to key r's d values
// of k or v); rows past nrows are zero. All `nthreads` threads of the workgroup call it.
template <int D, typename KPtr, typename VPtr>
__device__ inline void f32_load_tile(F32Tile<D>& t, int nrows, KPtr kptr, VPtr vptr, int nthreads) {
  constexpr int H = F32Cfg<D>::H;
  for (int c = threadIdx.x; c < kF32Tile * D; c += nthreads) {
    const int row = c / D, d = c % D;
    float kv = 0.f, vv = 0.f;
    if (row < nrows) {
      kv = kptr(row)[d];
      vv = vptr(row)[d];
    }
    const int col = (d / H) * (H + 1) + d % H;
    t.k[row][col] = static_cast<double>(kv);
    t.v[row][col] = vv;
  }
}

template <int D>
struct F32Row {
  static constexpr int H = F32Cfg<D>::H;
  float q[H];
  double acc[H];
  double m, l;
  int half;   // which half of the head dims this lane holds (lane >> 5)

  // qrow: the query row's d values (or null for a padding row: zeros).
  __device__ void init(const float* qrow) {
    half = (threadIdx.x & 63) >> 5;
#pragma unroll
    for (int d = 0; d < H; ++d) {
      q[d] = qrow ? qrow[half * H + d] : 0.f;
      acc[d] = 0.0;
    }
    m = -INFINITY;
    l = 0.0;
  }

  // Keys 0..lim of the tile are visible to this row (lim < 0: none). Both lanes of
  // the pair have the same lim, so they stay converged through the shuffle.
  __device__ void step(const F32Tile<D>& t, int lim, double scale) {
    const int off = half * (H + 1);
    const int last = min(lim, kF32Tile - 1);
    for (int kk = 0; kk <= last; ++kk) {
      double dot = 0.0;
#pragma unroll
      for (int d = 0; d < H; ++d) dot = fma(static_cast<double>(q[d]), t.k[kk][off + d], dot);
      dot += __shfl_xor(dot, 32);
      const double x = dot * scale;
      if (x > m) {
        const double alpha = exp(m - x);   // m = -inf gives 0
#pragma unroll
        for (int d = 0; d < H; ++d) acc[d] *= alpha;
        l *= alpha;
        m = x;
      }
      const double pe = static_cast<double>(expf(static_cast<float>(x - m)));
      l += pe;
#pragma unroll
      for (int d = 0; d < H; ++d) acc[d] = fma(pe, static_cast<double>(t.v[kk][off + d]), acc[d]);
    }
  }

  // Write this lane's half of O / l to orow (the row's d values), rounded to float32.
  __device__ void store(float* orow) const {
    const double inv = 1.0 / l;
#pragma unroll
    for (int d = 0; d < H; ++d) orow[half * H + d] = static_cast<float>(acc[d] * inv);
  }
  __device__ double lse() const { return m + log(l); }
};

}  // namespace spava
