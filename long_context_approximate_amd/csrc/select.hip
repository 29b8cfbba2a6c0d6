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
//   rowstats  (m, z) = (max logit, sum exp(logit - max)) of every observer row over
//             one key split, register-blocked fp64 dot products staged through LDS;
//   merge     combine the key splits of each row;
//   colsum    per key: sum over all observer rows of exp(x - m) / z, in one fixed
//             order for every key, then divide by G*w;
//   topl      per (j, g): 8-pass MSB radix select on the float64 bit patterns
//             (scores are >= 0, so unsigned order is numeric order) to find the
//             l_j-th largest score, then an in-order compaction that keeps every
//             larger score and the lowest-positioned equal ones.
#include "spava_internal.h"

namespace spava {
namespace {

constexpr int kTile = kScoreTile;  // 64 rows x 64 keys per workgroup
constexpr int kDChunk = 32;        // head-dim slice staged in LDS at a time

__device__ inline double to_f64(uint16_t b) {
  return static_cast<double>(__uint_as_float(static_cast<uint32_t>(b) << 16));
}
__device__ inline double to_f64(float f) { return static_cast<double>(f); }

// Observer row r of (block j, KV head g): head g*G + r / w, query e_j - w + r % w.
struct RowMap {
  __device__ static int64_t token(const Plan& p, int j, int r) {
    return static_cast<int64_t>(j + 1) * p.nb - p.w + (r % p.w);
  }
  __device__ static int head(const Plan& p, int g, int r) { return g * p.G + r / p.w; }
};

// 64x64 tile of logits (unscaled dot products) for rows [r0, r0+64) and keys
// [c0, c0+64) of block j; each thread owns rows tr+16a and keys tk+16b.
template <typename T>
__device__ inline void tile_dots(const Plan& p, const T* q, const T* k, int j, int g, int r0,
                                 int64_t key0, double (*Qs)[kTile + 1], double (*Ks)[kTile + 1],
                                 int64_t* q_off, int64_t* k_tok, double acc[4][4]) {
  const int tid = threadIdx.x, tr = tid >> 4, tk = tid & 15;
  const int64_t e = static_cast<int64_t>(j + 1) * p.nb;
  if (tid < kTile) {
    const int r = r0 + tid;
    q_off[tid] = r < p.R ? RowMap::token(p, j, r) * p.qs_tok + RowMap::head(p, g, r) * p.qs_head
                         : -1;
    const int64_t key = key0 + tid;
    k_tok[tid] = key < e ? key : -1;
  }
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = 0.0;
  for (int dc = 0; dc < p.D / kDChunk; ++dc) {
    __syncthreads();
    {
      // Q rows: gather by precomputed element offsets.
      const int r = tid >> 2, part = tid & 3;
      const int64_t off = q_off[r];
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const int dd = part * 8 + t;
        Qs[dd][r] = off >= 0 ? to_f64(q[off + dc * kDChunk + dd]) : 0.0;
      }
      const int64_t tok = k_tok[r];
      const T* kb = k + g * p.kvs_head;
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const int dd = part * 8 + t;
        Ks[dd][r] = tok >= 0 ? to_f64(kb[tok * p.kvs_tok + dc * kDChunk + dd]) : 0.0;
      }
    }
    __syncthreads();
#pragma unroll 4
    for (int dd = 0; dd < kDChunk; ++dd) {
      double qa[4], kv[4];
#pragma unroll
      for (int a = 0; a < 4; ++a) qa[a] = Qs[dd][tr + 16 * a];
#pragma unroll
      for (int b = 0; b < 4; ++b) kv[b] = Ks[dd][tk + 16 * b];
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) acc[a][b] = fma(qa[a], kv[b], acc[a][b]);
    }
  }
}

// Combine two (max, sum) pairs of the same row.
__device__ inline void lse_merge(double& m, double& z, double mo, double zo) {
  const double mn = fmax(m, mo);
  if (mn == -INFINITY) return;  // both empty
  const double a = (m == -INFINITY) ? 0.0 : z * exp(m - mn);
  const double b = (mo == -INFINITY) ? 0.0 : zo * exp(mo - mn);
  z = a + b;
  m = mn;
}

template <typename T>
__global__ __launch_bounds__(256) void rowstats_kernel(Plan p, const T* __restrict__ q,
                                                       const T* __restrict__ k,
                                                       double2* __restrict__ part) {
  __shared__ double Qs[kDChunk][kTile + 1];
  __shared__ double Ks[kDChunk][kTile + 1];
  __shared__ int64_t q_off[kTile], k_tok[kTile];
  const int r0 = blockIdx.x * kTile;
  const int split = blockIdx.y;
  const int jg = blockIdx.z;
  const int j = jg / p.Hkv, g = jg % p.Hkv;
  const int tid = threadIdx.x, tr = tid >> 4, tk = tid & 15;
  const int64_t s = static_cast<int64_t>(j) * p.nb;
  const int64_t split_lo = s + static_cast<int64_t>(split) * kScoreSplitKeys;
  const int64_t split_hi = min(s + p.nb, split_lo + kScoreSplitKeys);

  double m[4], z[4];
  int64_t qi[4];
#pragma unroll
  for (int a = 0; a < 4; ++a) {
    m[a] = -INFINITY;
    z[a] = 0.0;
    const int r = r0 + tr + 16 * a;
    qi[a] = r < p.R ? RowMap::token(p, j, r) : -1;   // -1: padding row sees nothing
  }
  for (int64_t key0 = split_lo; key0 < split_hi; key0 += kTile) {
    double acc[4][4];
    tile_dots(p, q, k, j, g, r0, key0, Qs, Ks, q_off, k_tok, acc);
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      double x[4];
      bool vis[4];
      double mt = -INFINITY;
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const int64_t key = key0 + tk + 16 * b;
        vis[b] = key < split_hi && key <= qi[a];
        x[b] = p.scale * acc[a][b];
        if (vis[b]) mt = fmax(mt, x[b]);
      }
      if (mt > m[a]) {
        z[a] = (m[a] == -INFINITY) ? 0.0 : z[a] * exp(m[a] - mt);
        m[a] = mt;
      }
#pragma unroll
      for (int b = 0; b < 4; ++b)
        if (vis[b]) z[a] += exp(x[b] - m[a]);
    }
  }
  // Reduce over the 16 lanes (tk) that share each row.
#pragma unroll
  for (int a = 0; a < 4; ++a) {
#pragma unroll
    for (int off = 8; off >= 1; off >>= 1) {
      const double mo = __shfl_xor(m[a], off);
      const double zo = __shfl_xor(z[a], off);
      lse_merge(m[a], z[a], mo, zo);
    }
    const int r = r0 + tr + 16 * a;
    if (tk == 0 && r < p.R)
      part[(static_cast<int64_t>(jg) * p.KS + split) * p.R + r] = make_double2(m[a], z[a]);
  }
}

__global__ void merge_kernel(Plan p, const double2* __restrict__ part,
                             double2* __restrict__ rowstat) {
  const int64_t total = static_cast<int64_t>(p.H - 1) * p.Hkv * p.R;
  const int64_t t = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (t >= total) return;
  const int64_t jg = t / p.R;
  const int r = static_cast<int>(t % p.R);
  double m = -INFINITY, z = 0.0;
  for (int sidx = 0; sidx < p.KS; ++sidx) {
    const double2 pr = part[(jg * p.KS + sidx) * p.R + r];
    lse_merge(m, z, pr.x, pr.y);
  }
  rowstat[t] = make_double2(m, z);
}

template <typename T>
__global__ __launch_bounds__(256) void colsum_kernel(Plan p, const T* __restrict__ q,
                                                     const T* __restrict__ k,
                                                     const double2* __restrict__ rowstat,
                                                     double* __restrict__ scores) {
  __shared__ double Qs[kDChunk][kTile + 1];
  __shared__ double Ks[kDChunk][kTile + 1];
  __shared__ int64_t q_off[kTile], k_tok[kTile];
  __shared__ double red[16][kTile + 1];
  const int kt = blockIdx.x;
  const int jg = blockIdx.y;
  const int j = jg / p.Hkv, g = jg % p.Hkv;
  const int tid = threadIdx.x, tr = tid >> 4, tk = tid & 15;
  const int64_t s = static_cast<int64_t>(j) * p.nb;
  const int64_t key0 = s + static_cast<int64_t>(kt) * kTile;

  double col[4] = {0.0, 0.0, 0.0, 0.0};
  for (int r0 = 0; r0 < p.R; r0 += kTile) {
    double acc[4][4];
    tile_dots(p, q, k, j, g, r0, key0, Qs, Ks, q_off, k_tok, acc);
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const int r = r0 + tr + 16 * a;
      const bool row_ok = r < p.R;
      const int64_t qi = row_ok ? RowMap::token(p, j, r) : -1;
      const double2 st = row_ok ? rowstat[static_cast<int64_t>(jg) * p.R + r] : make_double2(0, 1);
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const int64_t key = key0 + tk + 16 * b;
        const double x = p.scale * acc[a][b];
        const double pi = (row_ok && key <= qi) ? exp(x - st.x) / st.y : 0.0;
        col[b] += pi;
      }
    }
  }
#pragma unroll
  for (int b = 0; b < 4; ++b) red[tr][tk + 16 * b] = col[b];
  __syncthreads();
  if (tid < kTile) {
    const int64_t key = key0 + tid;
    if (key < s + p.nb) {
      double sum = 0.0;
      for (int t = 0; t < 16; ++t) sum += red[t][tid];
      scores[static_cast<int64_t>(jg) * p.nb + (key - s)] =
          sum / static_cast<double>(static_cast<int64_t>(p.G) * p.w);
    }
  }
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
    for (int t = tid; t < n; t += blockDim.x) {
      const unsigned long long x = u[t];
      if ((x & mask) == prefix) atomicAdd(&hist[(x >> shift) & 0xFF], 1u);
    }
    __syncthreads();
    if (tid == 0) {
      int cum = 0;
      int digit = 0;
      for (int d = 255; d >= 0; --d) {
        const int c = static_cast<int>(hist[d]);
        if (cum + c >= krem) {
          digit = d;
          break;
        }
        cum += c;
      }
      s_prefix = prefix | (static_cast<unsigned long long>(digit) << shift);
      s_k = krem - cum;
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

template <typename T>
static hipError_t launch_select_t(const Plan& p, const T* q, const T* k, int32_t* idx,
                                  double* scores_out, char* ws, hipStream_t st) {
  const SelectWs w = select_ws_layout(p);
  double2* part = reinterpret_cast<double2*>(ws + w.rowstat_part);
  double2* rowstat = reinterpret_cast<double2*>(ws + w.rowstat);
  double* scores = scores_out ? scores_out : reinterpret_cast<double*>(ws + w.scores);
  const int JG = (p.H - 1) * p.Hkv;
  dim3 g1(static_cast<unsigned>(cdiv(p.R, kTile)), p.KS, JG);
  hipLaunchKernelGGL(rowstats_kernel<T>, g1, dim3(256), 0, st, p, q, k, part);
  const int64_t rows = static_cast<int64_t>(JG) * p.R;
  hipLaunchKernelGGL(merge_kernel, dim3(static_cast<unsigned>(cdiv(rows, 256))), dim3(256), 0, st,
                     p, part, rowstat);
  dim3 g3(static_cast<unsigned>(cdiv(p.nb, kTile)), JG);
  hipLaunchKernelGGL(colsum_kernel<T>, g3, dim3(256), 0, st, p, q, k, rowstat, scores);
  if (p.l > 0) hipLaunchKernelGGL(topl_kernel, dim3(JG), dim3(1024), 0, st, p, scores, idx);
  return hipGetLastError();
}

hipError_t launch_select(const Plan& p, const void* q, const void* k, int32_t* idx,
                         double* scores, char* ws, hipStream_t st) {
  if (p.dtype == SPAVA_BF16)
    return launch_select_t(p, static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                           idx, scores, ws, st);
  return launch_select_t(p, static_cast<const float*>(q), static_cast<const float*>(k), idx,
                         scores, ws, st);
}

}  // namespace spava
