// Passing-block selection: float64 window scores and per-(block, KV head) top-l.
//
// Method (explainer "APB-V: ...", Methodik > Approximativer Attention-Mechanismus >
// Passing Blocks): each block forwards its most essential KV rows, ranked by
// query-to-context attention scores. Scoring rule used here: the score of key p of
// block j under KV head g is the mean, over the G query heads of g and the last w
// queries i of block j, of the softmax of scale*<q_i, k_p> over the block's own
// causal keys [s_j, i]. Selection takes the l_j largest, ties to the lower position.
//
// Kernels, in launch order:
// Observers are the last w queries of each block (causal), or, for the query-aware
// variant, the rows of a query block that follows the context (every key visible).
//
//   rowstats  (m, z) = (reference, sum exp(logit - reference)) of every observer row
//             over one key split, the reference within 64 of the row's largest
//             logit; float64 dot products on v_mfma_f64_16x16x4_f64. When the plan
//             stores logits, the scaled float64 logits are written too;
//   merge     combine the key splits of each row into (m, 1/z);
//   colsum    per key: sum over all observer rows of exp(x - m) / z, in one fixed
//             order for every key (so equal keys get bitwise-equal scores), then
//             divide by G*w. It reads the stored logits, or recomputes them with the
//             same products (bitwise the same values either way).
// With stored logits the pairs are processed in chunks (rowstats, merge, colsum per
// chunk) so the logit buffer stays bounded.
//   topl      per (j, g): 8-pass MSB radix select on the float64 bit patterns
//             (scores are >= 0, so unsigned order is numeric order) to find the
//             l_j-th largest score, then an in-order compaction that keeps every
//             larger score and the lowest-positioned equal ones.
//
// fp64 MFMA 16x16x4 lane layout (wave64): lane l supplies row (l % 16) of A and
// column (l % 16) of B at reduction slot l / 16; accumulator register r of lane l
// holds row 4*r + l/16, column l % 16. Each lane therefore owns a contiguous quarter
// of the head dimension of one row and one key (slot l/16 <-> d in [l/16*D/4, +D/4)).
// A wave computes a 32-row x 32-key logit tile per step (2 x 2 MFMA blocks).
#include <algorithm>

#include "spava_internal.h"

// No floating-point contraction in this file: every product and sum is rounded on its
// own, so each kernel instantiation (and the stored-logit and recomputing score
// passes) performs exactly the same operations on the same values.
#pragma clang fp contract(off)

namespace spava {
namespace {

typedef double f64x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWaveRows = 32;   // observer rows per wave tile
constexpr int kWaveKeys = 32;   // keys per wave tile

// One lane's quarter-row of q or k (D/4 consecutive elements), kept as stored bits.
template <typename T, int D>
struct Frag;

template <int D>
struct Frag<uint16_t, D> {
  static constexpr int W = D / 8;  // 32-bit words (2 bf16 each)
  uint32_t w[W];
  __device__ void load(const uint16_t* ptr, bool ok) {
#pragma unroll
    for (int i = 0; i < W / 4; ++i) {
      const u32x4 v = ok ? *reinterpret_cast<const u32x4*>(ptr + 8 * i) : u32x4{0u, 0u, 0u, 0u};
      w[4 * i] = v[0];
      w[4 * i + 1] = v[1];
      w[4 * i + 2] = v[2];
      w[4 * i + 3] = v[3];
    }
  }
  __device__ double at(int s) const {
    const uint32_t x = w[s >> 1];
    const uint32_t b = (s & 1) ? (x & 0xFFFF0000u) : (x << 16);
    return static_cast<double>(__uint_as_float(b));
  }
};

template <int D>
struct Frag<float, D> {
  static constexpr int W = D / 4;
  uint32_t w[W];
  __device__ void load(const float* ptr, bool ok) {
#pragma unroll
    for (int i = 0; i < W / 4; ++i) {
      const u32x4 v = ok ? *reinterpret_cast<const u32x4*>(ptr + 4 * i) : u32x4{0u, 0u, 0u, 0u};
      w[4 * i] = v[0];
      w[4 * i + 1] = v[1];
      w[4 * i + 2] = v[2];
      w[4 * i + 3] = v[3];
    }
  }
  __device__ double at(int s) const { return static_cast<double>(__uint_as_float(w[s])); }
};

// Keep a loop-invariant fragment as stored bits: the empty asm tells the compiler the
// words may change, so the fp64 widening is redone per use instead of hoisted into
// twice the registers (more than two waves per SIMD can hold).
template <typename F>
__device__ inline void opaque(F& f) {
#pragma unroll
  for (int i = 0; i < F::W; ++i) asm volatile("" : "+v"(f.w[i]));
}

// Observer row r of (block j, KV head g): head g*G + r / w and query row e_j - w + r % w
// of q, or row r % w of the query block when the observers are the query block.
__device__ inline int64_t row_token(const Plan& p, int j, int r) {
  return p.obs_query ? (r % p.w) : static_cast<int64_t>(j + 1) * p.nb - p.w + (r % p.w);
}
// Last key position observer row r sees: its own position (causal), or every key of
// the block for query-block observers.
__device__ inline int64_t row_key_limit(const Plan& p, int j, int r) {
  return p.obs_query ? INT64_MAX : row_token(p, j, r);
}
__device__ inline int row_head(const Plan& p, int g, int r) { return g * p.G + r / p.w; }

// 32x32 tile of unscaled logits: acc[rb][kb] holds rows rb*16 + 4*r + l/16 and key
// kb*16 + l%16 of the tile.
template <typename T, int D>
__device__ inline void tile_logits(const Frag<T, D> (&qa)[2], const Frag<T, D> (&kf)[2],
                                   f64x4 (&acc)[2][2]) {
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) acc[rb][kb] = f64x4{0.0, 0.0, 0.0, 0.0};
#pragma unroll
  for (int s = 0; s < D / 4; ++s) {
    const double a0 = qa[0].at(s), a1 = qa[1].at(s);
    const double b0 = kf[0].at(s), b1 = kf[1].at(s);
    acc[0][0] = __builtin_amdgcn_mfma_f64_16x16x4f64(a0, b0, acc[0][0], 0, 0, 0);
    acc[0][1] = __builtin_amdgcn_mfma_f64_16x16x4f64(a0, b1, acc[0][1], 0, 0, 0);
    acc[1][0] = __builtin_amdgcn_mfma_f64_16x16x4f64(a1, b0, acc[1][0], 0, 0, 0);
    acc[1][1] = __builtin_amdgcn_mfma_f64_16x16x4f64(a1, b1, acc[1][1], 0, 0, 0);
  }
}

// Load the lane's A fragments (observer rows r0 + rb*16 + l%16) for (j, g).
template <typename T, int D>
__device__ inline void load_rows(const Plan& p, const T* q, int j, int g, int r0, int col, int kg,
                                 Frag<T, D> (&qa)[2]) {
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    const int r = r0 + rb * 16 + col;
    const bool ok = r < p.R;
    const int rr = ok ? r : 0;
    const T* ptr = q + row_token(p, j, rr) * p.qs_tok + row_head(p, g, rr) * p.qs_head + kg * (D / 4);
    qa[rb].load(ptr, ok);
  }
}

// Load the lane's B fragments (keys key0 + kb*16 + l%16, valid below key_end).
template <typename T, int D>
__device__ inline void load_keys(const Plan& p, const T* k, int g, int64_t key0, int64_t key_end,
                                 int col, int kg, Frag<T, D> (&kf)[2]) {
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    const int64_t key = key0 + kb * 16 + col;
    const bool ok = key < key_end;
    const T* ptr = k + (ok ? key : 0) * p.kvs_tok + g * p.kvs_head + kg * (D / 4);
    kf[kb].load(ptr, ok);
  }
}

// exp(y) in float64 for y <= 709, within 2 ulp; 0 below -745.2 (and for y = -inf).
// Tang's table-driven method: y = (64 n + j) ln2/64 + r with |r| <= ln2/128, so
// exp(y) = 2^n * 2^(j/64) * exp(r); 2^(j/64) comes from a 64-entry table in LDS and
// exp(r) from its degree-5 Taylor polynomial (truncation error below 2^-54, a sixth of
// an ulp of 1). ln2/64 is split into a 36-bit head (exact products k * head for
// |k| < 2^17) and a tail. Branch-free: the argument is clamped to -746 so the
// arithmetic stays finite, and the underflow is a final select, so a run of calls
// issues its table reads together.
constexpr int kExpTab = 64;
__device__ inline void init_exp_table(double* tab) {
  if (threadIdx.x < kExpTab) tab[threadIdx.x] = exp2(static_cast<double>(threadIdx.x) / kExpTab);
  __syncthreads();
}
// The routine without its final underflow select: below -745.2 it returns 0 or a
// subnormal (at most 2^-1074) instead of 0. The row sums use it: a sum that already
// holds a term of at least 1 (the reference's own) is bitwise unchanged by that.
__device__ inline double exp_tab_raw(double y, const double* tab) {
  const double yc = fmax(y, -746.0);
  const double k = rint(yc * 0x1.71547652b82fep+6);         // y * 64 / ln2
  double r = fma(-k, 0x1.62e42fefa0000p-7, yc);             // head of ln2 / 64
  r = fma(-k, 0x1.cf79abc9e3b3ap-46, r);                    // tail
  double a = fma(r, 1.0 / 120.0, 1.0 / 24.0);
  a = fma(r, a, 1.0 / 6.0);
  a = fma(r, a, 0.5);
  a = fma(r, a, 1.0);
  const double er = fma(r, a, 1.0);
  const int ki = static_cast<int>(k);
  return ldexp(tab[ki & (kExpTab - 1)] * er, ki >> 6);
}
__device__ inline double exp_tab(double y, const double* tab) {
  const double yc = fmax(y, -746.0);
  const double v = exp_tab_raw(yc, tab);
  return yc > -745.2 ? v : 0.0;
}

// Row statistics keep a lazy reference instead of the running maximum: the reference is
// raised only when a tile's largest logit exceeds it by more than this margin (the
// first tile, or a far larger logit), so the common path has no rescaling branch.
// Terms exp(x - ref) stay below e^64 and a row's sum below 2^105: no overflow, and the
// relative rounding of a float64 sum does not depend on its scale.
constexpr double kRefMargin = 64.0;

// The stored logits are written once and read once (3.3 GB at 128K tokens, far past
// the caches): both passes use non-temporal accesses so the stream does not evict
// what the caches hold for others.
typedef double f64x2 __attribute__((ext_vector_type(2)));
__device__ inline double2 nt_load2(const double* ptr) {
  const f64x2 v = __builtin_nontemporal_load(reinterpret_cast<const f64x2*>(ptr));
  return make_double2(v[0], v[1]);
}

// Combine two (max, sum) pairs of the same row.
__device__ inline void lse_merge(double& m, double& z, double mo, double zo, const double* tab) {
  const double mn = fmax(m, mo);
  if (mn == -INFINITY) return;  // both empty
  const double a = (m == -INFINITY) ? 0.0 : z * exp_tab(m - mn, tab);
  const double b = (mo == -INFINITY) ? 0.0 : zo * exp_tab(mo - mn, tab);
  z = a + b;
  m = mn;
}

// Stored logits are key-tile major: pair (jg - jg0), then 32-key tile t = (key - s_j)/32,
// then row r, then the key's slot in the tile; a pair holds R * round_up(n_b, 32)
// values. A row-statistics tile (32 rows x 32 keys) is one contiguous 8 KB block, and
// the score pass streams a key tile's rows from one contiguous run.
__device__ inline int64_t logit_pair_len(const Plan& p) {
  return static_cast<int64_t>(p.R) * ((static_cast<int64_t>(p.nb) + 31) & ~int64_t(31));
}
__device__ inline int64_t logit_at(const Plan& p, int r, int64_t kk) {   // kk = key - s_j
  return ((kk >> 5) * p.R + r) * 32 + (kk & 31);
}

// One wave per (jg, 32-row tile, key split) for the pairs [jg0, jg0 + npairs). Waves
// are independent (no barriers). STORE: also write the scaled logits of every visible
// (row, key) to the stored-logit layout above. MINB = 2 caps the registers at two waves
// per SIMD (a few spills), for launches with more waves than SIMDs: the second wave
// hides the first's memory and dependency stalls (the float64 products and the
// vector work of a SIMD do not overlap, so a wave alone leaves the stalls exposed).
template <typename T, int D, bool STORE, int MINB>
__global__ __launch_bounds__(256, MINB) void rowstats_kernel(Plan p, const T* __restrict__ q,
                                                       const T* __restrict__ k,
                                                       double2* __restrict__ part,
                                                       double* __restrict__ logits,
                                                       int row_tiles, int jg0, int npairs) {
  __shared__ double etab[kExpTab];
  init_exp_table(etab);
  const int64_t wid = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  const int64_t total = static_cast<int64_t>(npairs) * row_tiles * p.KS;
  if (wid >= total) return;
  const int split = static_cast<int>(wid % p.KS);
  const int64_t rest = wid / p.KS;
  const int rt = static_cast<int>(rest % row_tiles);
  const int jg = jg0 + static_cast<int>(rest / row_tiles);
  const int j = jg / p.Hkv, g = jg % p.Hkv;
  const int lane = threadIdx.x & 63, col = lane & 15, kg = lane >> 4;
  const int64_t s = static_cast<int64_t>(j) * p.nb;
  const int64_t split_lo = s + static_cast<int64_t>(split) * p.split_keys;
  const int64_t split_hi = min(s + p.nb, split_lo + p.split_keys);
  const int r0 = rt * kWaveRows;
  double* lg = STORE ? logits + static_cast<int64_t>(jg - jg0) * logit_pair_len(p) : nullptr;

  Frag<T, D> qa[2];
  load_rows<T, D>(p, q, j, g, r0, col, kg, qa);
  double m[2][4], z[2][4];
  int qi[2][4];   // last visible key of each row, relative to s (-1: padding row)
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      m[rb][rr] = -INFINITY;
      z[rb][rr] = 0.0;
      const int r = r0 + rb * 16 + 4 * rr + kg;
      qi[rb][rr] =
          r < p.R ? static_cast<int>(min<int64_t>(row_key_limit(p, j, r) - s, p.nb)) : -1;
    }
  // Last key every row of this wave sees (wave-uniform); tiles at or below it, inside
  // the split and without padding rows take the unmasked path.
  int qmin = INT32_MAX;
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) qmin = min(qmin, qi[rb][rr]);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) qmin = min(qmin, __shfl_xor(qmin, off));
  const bool rows_full = r0 + kWaveRows <= p.R;
  Frag<T, D> kf[2];
  load_keys<T, D>(p, k, g, split_lo, split_hi, col, kg, kf);
  for (int64_t key0 = split_lo; key0 < split_hi; key0 += kWaveKeys) {
    opaque(qa[0]);
    opaque(qa[1]);
    f64x4 acc[2][2];
    tile_logits<T, D>(qa, kf, acc);
    // Prefetch the next key tile while this tile's softmax statistics are formed.
    if (key0 + kWaveKeys < split_hi)
      load_keys<T, D>(p, k, g, key0 + kWaveKeys, split_hi, col, kg, kf);
    const bool full = rows_full && key0 + kWaveKeys <= split_hi && key0 + kWaveKeys - 1 <= s + qmin;
    if (full) {
      // Every (row, key) of the tile is visible: the same updates without masks.
      double* tb = STORE ? lg + logit_at(p, r0 + kg, key0 - s) + col : nullptr;
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const double x0 = p.scale * acc[rb][0][rr], x1 = p.scale * acc[rb][1][rr];
          if (STORE) {
            double* row = tb + (rb * 16 + 4 * rr) * 32;   // rows of one tile are 32 apart
            __builtin_nontemporal_store(x0, row);
            __builtin_nontemporal_store(x1, row + 16);
          }
          const double mt = fmax(x0, x1);
          if (mt > m[rb][rr] + kRefMargin) {
            z[rb][rr] =
                (m[rb][rr] == -INFINITY) ? 0.0 : z[rb][rr] * exp_tab(m[rb][rr] - mt, etab);
            m[rb][rr] = mt;
          }
          z[rb][rr] += exp_tab_raw(x0 - m[rb][rr], etab);
          z[rb][rr] += exp_tab_raw(x1 - m[rb][rr], etab);
        }
      continue;
    }
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        double x[2];
        bool vis[2];
        double mt = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const int64_t key = key0 + kb * 16 + col;
          vis[kb] = key < split_hi && key - s <= qi[rb][rr];
          x[kb] = p.scale * acc[rb][kb][rr];
          if (vis[kb]) mt = fmax(mt, x[kb]);
          if (STORE && vis[kb])
            __builtin_nontemporal_store(
                x[kb], lg + logit_at(p, r0 + rb * 16 + 4 * rr + kg, key - s));
        }
        if (mt > m[rb][rr] + kRefMargin) {
          z[rb][rr] = (m[rb][rr] == -INFINITY) ? 0.0 : z[rb][rr] * exp_tab(m[rb][rr] - mt, etab);
          m[rb][rr] = mt;
        }
        // Hidden keys add exp(-inf) = 0 (x - m is never formed with m = -inf for them).
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
          z[rb][rr] += exp_tab(vis[kb] ? x[kb] - m[rb][rr] : -INFINITY, etab);
      }
  }
  // Reduce over the 16 lanes (l % 16) that hold different keys of the same rows.
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
#pragma unroll
      for (int off = 8; off >= 1; off >>= 1) {
        const double mo = __shfl_xor(m[rb][rr], off);
        const double zo = __shfl_xor(z[rb][rr], off);
        lse_merge(m[rb][rr], z[rb][rr], mo, zo, etab);
      }
      const int r = r0 + rb * 16 + 4 * rr + kg;
      if (col == 0 && r < p.R)
        part[(static_cast<int64_t>(jg) * p.KS + split) * p.R + r] =
            make_double2(m[rb][rr], z[rb][rr]);
    }
}

// Rows of the pairs [jg0, jg0 + npairs).
__global__ void merge_kernel(Plan p, const double2* __restrict__ part,
                             double2* __restrict__ rowstat, int jg0, int npairs) {
  __shared__ double etab[kExpTab];
  init_exp_table(etab);
  const int64_t total = static_cast<int64_t>(npairs) * p.R;
  const int64_t t = static_cast<int64_t>(jg0) * p.R + static_cast<int64_t>(blockIdx.x) * blockDim.x +
                    threadIdx.x;
  if (t >= static_cast<int64_t>(jg0) * p.R + total) return;
  const int64_t jg = t / p.R;
  const int r = static_cast<int>(t % p.R);
  double m = -INFINITY, z = 0.0;
  for (int sidx = 0; sidx < p.KS; ++sidx) {
    const double2 pr = part[(jg * p.KS + sidx) * p.R + r];
    lse_merge(m, z, pr.x, pr.y, etab);
  }
  rowstat[t] = make_double2(m, 1.0 / z);   // (reference, 1 / sum)
}

// exp(x - m) / z of one visible (row, key), else 0 (the same code in both score passes).
__device__ inline double prob_term(bool vis, double x, double2 mz, const double* etab) {
  return vis ? exp_tab(x - mz.x, etab) * mz.y : 0.0;
}

// The four lanes col, col+16, col+32, col+48 hold disjoint row sets of the same key;
// add them in a fixed order and write the mean.
__device__ inline void finish_colsum(const Plan& p, const double (&colsum)[2], const int64_t (&key)[2],
                                     int col, int kg, int jg, int64_t s, int64_t e,
                                     double* __restrict__ scores) {
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    const double v0 = __shfl(colsum[kb], col);
    const double v1 = __shfl(colsum[kb], col + 16);
    const double v2 = __shfl(colsum[kb], col + 32);
    const double v3 = __shfl(colsum[kb], col + 48);
    const double sum = ((v0 + v1) + v2) + v3;
    if (kg == 0 && key[kb] < e)
      scores[static_cast<int64_t>(jg) * p.nb + (key[kb] - s)] =
          sum / static_cast<double>(static_cast<int64_t>(p.G) * p.w);
  }
}

// One wave per (jg, 32-key tile); loops over all observer rows in a fixed order and
// recomputes each logit.
template <typename T, int D>
__global__ __launch_bounds__(256) void colsum_kernel(Plan p, const T* __restrict__ q,
                                                     const T* __restrict__ k,
                                                     const double2* __restrict__ rowstat,
                                                     double* __restrict__ scores, int key_tiles) {
  __shared__ double etab[kExpTab];
  init_exp_table(etab);
  const int64_t wid = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  const int64_t total = static_cast<int64_t>(p.H - 1) * p.Hkv * key_tiles;
  if (wid >= total) return;
  const int kt = static_cast<int>(wid % key_tiles);
  const int jg = static_cast<int>(wid / key_tiles);
  const int j = jg / p.Hkv, g = jg % p.Hkv;
  const int lane = threadIdx.x & 63, col = lane & 15, kg = lane >> 4;
  const int64_t s = static_cast<int64_t>(j) * p.nb;
  const int64_t e = s + p.nb;
  const int64_t key0 = s + static_cast<int64_t>(kt) * kWaveKeys;

  Frag<T, D> kf[2];
  load_keys<T, D>(p, k, g, key0, e, col, kg, kf);
  int64_t key[2];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) key[kb] = key0 + kb * 16 + col;
  const double2* st = rowstat + static_cast<int64_t>(jg) * p.R;

  double colsum[2] = {0.0, 0.0};
  Frag<T, D> qa[2];
  load_rows<T, D>(p, q, j, g, 0, col, kg, qa);
  for (int r0 = 0; r0 < p.R; r0 += kWaveRows) {
    opaque(kf[0]);
    opaque(kf[1]);
    f64x4 acc[2][2];
    tile_logits<T, D>(qa, kf, acc);
    // Prefetch the next observer rows while this tile's probabilities are summed.
    if (r0 + kWaveRows < p.R) load_rows<T, D>(p, q, j, g, r0 + kWaveRows, col, kg, qa);
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int r = r0 + rb * 16 + 4 * rr + kg;
        const bool ok = r < p.R;
        const double2 mz = ok ? st[r] : make_double2(0.0, 0.0);
        const int64_t qi = ok ? row_key_limit(p, j, r) : -1;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const double x = p.scale * acc[rb][kb][rr];
          colsum[kb] += prob_term(key[kb] <= qi, x, mz, etab);
        }
      }
  }
  finish_colsum(p, colsum, key, col, kg, jg, s, e, scores);
}

// Same sums for the pairs [jg0, jg0 + npairs), reading the logits rowstats stored:
// the rows, their order and every operation match colsum_kernel, so the scores are
// bitwise the same.
__global__ __launch_bounds__(256) void colsum_stored_kernel(Plan p, const double* __restrict__ logits,
                                                            const double2* __restrict__ rowstat,
                                                            double* __restrict__ scores,
                                                            int key_tiles, int jg0, int npairs) {
  __shared__ double etab[kExpTab];
  init_exp_table(etab);
  const int64_t wid = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  const int64_t total = static_cast<int64_t>(npairs) * key_tiles;
  if (wid >= total) return;
  const int kt = static_cast<int>(wid % key_tiles);
  const int jg = jg0 + static_cast<int>(wid / key_tiles);
  const int j = jg / p.Hkv;
  const int lane = threadIdx.x & 63, col = lane & 15, kg = lane >> 4;
  const int64_t s = static_cast<int64_t>(j) * p.nb;
  const int64_t e = s + p.nb;
  const int64_t key0 = s + static_cast<int64_t>(kt) * kWaveKeys;
  // This lane holds two adjacent keys (one 16-byte load per row when both are
  // visible); the row order of every key's sum is that of colsum_kernel, so the
  // scores are the same. One load instruction covers 4 consecutive rows of the key
  // tile: 1 KB contiguous.
  int64_t key[2];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) key[kb] = key0 + 2 * col + kb;
  const double2* st = rowstat + static_cast<int64_t>(jg) * p.R;
  const double* lg = logits + static_cast<int64_t>(jg - jg0) * logit_pair_len(p);

  // Keys every observer row sees (window rows sit at e - w .. e - 1 and see keys up
  // to their own position; query-block rows see the whole block): row tiles without
  // padding rows then need no visibility test.
  const bool keys_full = p.obs_query ? key0 + kWaveKeys <= e : key0 + kWaveKeys - 1 <= e - p.w;
  double colsum[2] = {0.0, 0.0};
  for (int r0 = 0; r0 < p.R; r0 += kWaveRows) {
    if (keys_full && r0 + kWaveRows <= p.R) {
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const int r = r0 + rb * 16 + 4 * rr + kg;
          const double2 mz = st[r];
          const double2 t = nt_load2(lg + logit_at(p, r, key[0] - s));
          colsum[0] += prob_term(true, t.x, mz, etab);
          colsum[1] += prob_term(true, t.y, mz, etab);
        }
      continue;
    }
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int r = r0 + rb * 16 + 4 * rr + kg;
        const bool ok = r < p.R;
        const double2 mz = ok ? st[r] : make_double2(0.0, 0.0);
        const int64_t qi = ok ? row_key_limit(p, j, r) : -1;
        const bool v0 = key[0] <= qi && key[0] < e;
        const bool v1 = key[1] <= qi && key[1] < e;   // implies v0
        const double* row = lg + logit_at(p, ok ? r : 0, key[0] - s);
        double x0 = 0.0, x1 = 0.0;
        if (v1) {
          const double2 t = nt_load2(row);
          x0 = t.x;
          x1 = t.y;
        } else {
          if (v0) x0 = row[0];
          if (v1) x1 = row[1];
        }
        colsum[0] += prob_term(v0, x0, mz, etab);
        colsum[1] += prob_term(v1, x1, mz, etab);
      }
  }
  finish_colsum(p, colsum, key, col, kg, jg, s, e, scores);
}

// One workgroup per (j, g). 1024 threads = 16 waves of 64.
__global__ __launch_bounds__(1024) void topl_kernel(Plan p, const double* __restrict__ scores,
                                                    int32_t* __restrict__ idx) {
  __shared__ unsigned int hist[256];
  __shared__ unsigned long long s_prefix;
  __shared__ int s_k;
  __shared__ int wave_gt[16], wave_eq[16];
  const int jg = blockIdx.x;
  const int j = jg / p.Hkv;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int c0 = j == 0 ? p.A : 0;                  // first candidate (block-local)
  const int n = p.nb - c0;
  const int lj = j == 0 ? p.l0 : p.l1;
  const int64_t s = static_cast<int64_t>(j) * p.nb;
  const unsigned long long* u =
      reinterpret_cast<const unsigned long long*>(scores + static_cast<int64_t>(jg) * p.nb + c0);
  int32_t* out = idx + static_cast<int64_t>(jg) * p.l;

  for (int t = lj + tid; t < p.l; t += blockDim.x) out[t] = -1;
  if (lj == 0) return;
  if (lj == n) {
    for (int t = tid; t < n; t += blockDim.x) out[t] = static_cast<int32_t>(s + c0 + t);
    return;
  }

  // Radix select: find the exact bit pattern T of the lj-th largest score and how
  // many scores equal to T belong to the selection.
  unsigned long long prefix = 0, mask = 0;
  int krem = lj;
  for (int pass = 0; pass < 8; ++pass) {
    const int shift = 56 - 8 * pass;
    for (int b = tid; b < 256; b += blockDim.x) hist[b] = 0;
    __syncthreads();
    for (int base = 0; base < n; base += blockDim.x) {
      const int t = base + tid;
      const unsigned long long x = t < n ? u[t] : 0ull;
      const bool m = t < n && (x & mask) == prefix;
      const unsigned dg = static_cast<unsigned>(x >> shift) & 0xFFu;
      // Scores share their leading bytes, so a wave's matching lanes usually carry one
      // digit: then a single atomic adds them all.
      const unsigned long long act = __ballot(m);
      if (act != 0ull) {
        const int first = __ffsll(static_cast<long long>(act)) - 1;
        const unsigned d0 = static_cast<unsigned>(__shfl(static_cast<int>(dg), first));
        if (__ballot(m && dg != d0) == 0ull) {
          if (lane == first) atomicAdd(&hist[d0], static_cast<unsigned>(__popcll(act)));
        } else if (m) {
          atomicAdd(&hist[dg], 1u);
        }
      }
    }
    __syncthreads();
    if (wave == 0) {
      // Digits in descending order, four per lane (lane L: 255 - 4L down to 252 - 4L);
      // a prefix sum over the lanes finds where the count from the top reaches krem.
      unsigned c[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) c[i] = hist[255 - 4 * lane - i];
      const int lsum = static_cast<int>(c[0] + c[1] + c[2] + c[3]);
      int incl = lsum;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int v = __shfl_up(incl, off);
        if (lane >= off) incl += v;
      }
      const unsigned long long hit = __ballot(incl >= krem);
      if (lane == __ffsll(static_cast<long long>(hit)) - 1) {
        int cum = incl - lsum;
        int digit = 255 - 4 * lane - 3;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if (cum + static_cast<int>(c[i]) >= krem) {
            digit = 255 - 4 * lane - i;
            break;
          }
          cum += static_cast<int>(c[i]);
        }
        s_prefix = prefix | (static_cast<unsigned long long>(digit) << shift);
        s_k = krem - cum;
      }
    }
    __syncthreads();
    prefix = s_prefix;
    krem = s_k;
    mask |= 0xFFull << shift;
    __syncthreads();
  }
  const unsigned long long thr = prefix;
  const int take_eq = krem;                         // >= 1

  // In-order compaction over candidate positions.
  int gt_before = 0, eq_before = 0;   // counts over earlier chunks
  for (int base = 0; base < n; base += blockDim.x) {
    const int t = base + tid;
    const unsigned long long x = t < n ? u[t] : 0ull;
    const bool gt = t < n && x > thr;
    const bool eq = t < n && x == thr;
    const unsigned long long bgt = __ballot(gt);
    const unsigned long long beq = __ballot(eq);
    const unsigned long long lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    const int gt_in = __popcll(bgt & lt_mask);
    const int eq_in = __popcll(beq & lt_mask);
    if (lane == 0) {
      wave_gt[wave] = __popcll(bgt);
      wave_eq[wave] = __popcll(beq);
    }
    __syncthreads();
    int gt_prev = 0, eq_prev = 0, gt_all = 0, eq_all = 0;
    for (int w2 = 0; w2 < 16; ++w2) {
      if (w2 < wave) {
        gt_prev += wave_gt[w2];
        eq_prev += wave_eq[w2];
      }
      gt_all += wave_gt[w2];
      eq_all += wave_eq[w2];
    }
    // Output slot = larger scores before me + equal scores taken before me.
    const int eq_rank = eq_before + eq_prev + eq_in;
    const int pos = gt_before + gt_prev + gt_in + min(eq_rank, take_eq);
    if (gt || (eq && eq_rank < take_eq)) out[pos] = static_cast<int32_t>(s + c0 + t);
    gt_before += gt_all;
    eq_before += eq_all;
    __syncthreads();
  }
}

}  // namespace

// Row statistics at two waves per SIMD: bf16 inputs, launches with more waves than
// SIMDs. float32 fragments take twice the registers (hundreds of spills at that cap).
template <typename T>
constexpr int kTwoWaves = sizeof(T) == 2 ? 2 : 1;
template <typename T>
static bool two_waves_per_simd(int64_t waves) {
  return sizeof(T) == 2 && waves > kScoreWaveSlots;
}

template <typename T, int D>
static hipError_t launch_select_t(const Plan& p, const T* q, const T* k, int32_t* idx,
                                  double* scores_out, char* ws, hipStream_t st) {
  const SelectWs w = select_ws_layout(p);
  double2* part = reinterpret_cast<double2*>(ws + w.rowstat_part);
  double2* rowstat = reinterpret_cast<double2*>(ws + w.rowstat);
  double* scores = scores_out ? scores_out : reinterpret_cast<double*>(ws + w.scores);
  double* logits = reinterpret_cast<double*>(ws + w.logits);
  const int JG = (p.H - 1) * p.Hkv;
  const int row_tiles = static_cast<int>(cdiv(p.R, kWaveRows));
  const int key_tiles = static_cast<int>(cdiv(p.nb, kWaveKeys));
  if (p.store_logits) {
    for (int jg0 = 0; jg0 < JG; jg0 += p.pair_chunk) {
      const int np = std::min(p.pair_chunk, JG - jg0);
      const int64_t w1 = static_cast<int64_t>(np) * row_tiles * p.KS;
      const dim3 grid(static_cast<unsigned>(cdiv(w1, 4)));
      if (two_waves_per_simd<T>(w1))
        hipLaunchKernelGGL((rowstats_kernel<T, D, true, kTwoWaves<T>>), grid, dim3(256), 0, st, p, q, k, part,
                           logits, row_tiles, jg0, np);
      else
        hipLaunchKernelGGL((rowstats_kernel<T, D, true, 1>), grid, dim3(256), 0, st, p, q, k, part,
                           logits, row_tiles, jg0, np);
      const int64_t rows = static_cast<int64_t>(np) * p.R;
      hipLaunchKernelGGL(merge_kernel, dim3(static_cast<unsigned>(cdiv(rows, 256))), dim3(256), 0,
                         st, p, part, rowstat, jg0, np);
      const int64_t w3 = static_cast<int64_t>(np) * key_tiles;
      hipLaunchKernelGGL(colsum_stored_kernel, dim3(static_cast<unsigned>(cdiv(w3, 4))), dim3(256),
                         0, st, p, logits, rowstat, scores, key_tiles, jg0, np);
    }
  } else {
    const int64_t w1 = static_cast<int64_t>(JG) * row_tiles * p.KS;
    const dim3 grid(static_cast<unsigned>(cdiv(w1, 4)));
    if (two_waves_per_simd<T>(w1))
      hipLaunchKernelGGL((rowstats_kernel<T, D, false, kTwoWaves<T>>), grid, dim3(256), 0, st, p, q, k, part,
                         nullptr, row_tiles, 0, JG);
    else
      hipLaunchKernelGGL((rowstats_kernel<T, D, false, 1>), grid, dim3(256), 0, st, p, q, k, part,
                         nullptr, row_tiles, 0, JG);
    const int64_t rows = static_cast<int64_t>(JG) * p.R;
    hipLaunchKernelGGL(merge_kernel, dim3(static_cast<unsigned>(cdiv(rows, 256))), dim3(256), 0, st,
                       p, part, rowstat, 0, JG);
    const int64_t w3 = static_cast<int64_t>(JG) * key_tiles;
    hipLaunchKernelGGL((colsum_kernel<T, D>), dim3(static_cast<unsigned>(cdiv(w3, 4))), dim3(256),
                       0, st, p, q, k, rowstat, scores, key_tiles);
  }
  if (p.l > 0)
    hipLaunchKernelGGL(topl_kernel, dim3(static_cast<unsigned>(JG)), dim3(1024), 0, st, p, scores,
                       idx);
  return hipGetLastError();
}

hipError_t launch_select(const Plan& p, const void* q, const void* k, int32_t* idx,
                         double* scores, char* ws, hipStream_t st) {
  if (p.dtype == SPAVA_BF16) {
    auto qq = static_cast<const uint16_t*>(q);
    auto kk = static_cast<const uint16_t*>(k);
    if (p.D == 128) return launch_select_t<uint16_t, 128>(p, qq, kk, idx, scores, ws, st);
    return launch_select_t<uint16_t, 64>(p, qq, kk, idx, scores, ws, st);
  }
  auto qq = static_cast<const float*>(q);
  auto kk = static_cast<const float*>(k);
  if (p.D == 128) return launch_select_t<float, 128>(p, qq, kk, idx, scores, ws, st);
  return launch_select_t<float, 64>(p, qq, kk, idx, scores, ws, st);
}

}  // namespace spava
