// Host side of the C ABI declared in include/spava.h: argument checks, planning,
// workspace carving and kernel launches. No device memory is allocated here.
#include <math.h>
#include <stdlib.h>
#include <string.h>

#include <atomic>
#include <initializer_list>
#include <mutex>

#include "spava_internal.h"

namespace spava {

static bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

static size_t region(size_t& cursor, size_t bytes) {
  size_t at = cursor;
  cursor += static_cast<size_t>(round_up(static_cast<int64_t>(bytes), 256));
  return at;
}

// The product of the factors (each in [0, 2^31)) is at most INT32_MAX, so a launch of
// that many work items fits the 32-bit grid size of a dispatch and int indexing.
// Stops at the first partial product above the bound, so nothing overflows.
static bool fits_launch(std::initializer_list<int64_t> factors) {
  int64_t prod = 1;
  for (int64_t f : factors) {
    if (f < 0 || f > INT32_MAX) return false;
    prod *= f;
    if (prod > INT32_MAX) return false;
  }
  return true;
}

// The selection's launches for this plan's observer count R.
static bool select_launches_fit(const Plan& p) {
  const int64_t j = p.H > 1 ? p.H - 1 : 0;
  return fits_launch({j, p.Hkv, cdiv(p.R, 32), p.KS, 64}) &&
         fits_launch({j, p.Hkv, cdiv(p.nb, 32), 64}) && fits_launch({j, p.Hkv, p.R}) &&
         fits_launch({j, p.Hkv, 1024});
}

static spava_status make_plan(const spava_shape* s, Plan* p) {
  if (!s) return SPAVA_ERR_NULL;
  if (s->dtype != SPAVA_BF16 && s->dtype != SPAVA_F32) return SPAVA_ERR_DTYPE;
  if (s->seq_len < 1 || s->num_hosts < 1 || s->seq_len % s->num_hosts != 0) return SPAVA_ERR_SHAPE;
  if (s->num_q_heads < 1 || s->num_kv_heads < 1 || s->num_q_heads % s->num_kv_heads != 0)
    return SPAVA_ERR_SHAPE;
  if (s->head_dim != 64 && s->head_dim != 128) return SPAVA_ERR_SHAPE;
  const int64_t nb = s->seq_len / s->num_hosts;
  if (nb > (int64_t(1) << 30)) return SPAVA_ERR_SHAPE;
  if (s->anchor_len < 0 || s->anchor_len > nb) return SPAVA_ERR_SHAPE;
  if (s->passing_len < 0) return SPAVA_ERR_SHAPE;
  if (s->window < 1 || s->window > nb) return SPAVA_ERR_SHAPE;
  if (!(s->sm_scale == s->sm_scale) || isinf(s->sm_scale)) return SPAVA_ERR_SHAPE;
  if (s->schedule < SPAVA_SCHED_LONGEST_FIRST || s->schedule > SPAVA_SCHED_ZIGZAG)
    return SPAVA_ERR_OPTION;
  if (s->select_logits != SPAVA_LOGITS_AUTO && s->select_logits != SPAVA_LOGITS_RECOMPUTE)
    return SPAVA_ERR_OPTION;
  const int64_t unit = s->dtype == SPAVA_BF16 ? 8 : 4;   // elements per 16 bytes
  const int64_t strides[6] = {s->q_stride_tok, s->q_stride_head, s->kv_stride_tok,
                              s->kv_stride_head, s->o_stride_tok, s->o_stride_head};
  for (int64_t st : strides) {
    if (st < 0) return SPAVA_ERR_SHAPE;
    if (st % unit != 0) return SPAVA_ERR_ALIGN;
  }
  // The attention reads K tiles in place through 32-bit buffer offsets: 63 token rows
  // of stride plus one row of 2 * head_dim bytes must stay below 2^31.
  if (s->kv_stride_tok > (INT32_MAX - 2 * 128) / (2 * (kKeyTile - 1))) return SPAVA_ERR_SHAPE;
  p->N = s->seq_len;
  p->H = s->num_hosts;
  p->Hq = s->num_q_heads;
  p->Hkv = s->num_kv_heads;
  p->G = s->num_q_heads / s->num_kv_heads;
  p->D = s->head_dim;
  p->A = s->anchor_len;
  p->l = s->passing_len;
  p->w = s->window;
  p->nb = static_cast<int>(nb);
  p->dtype = s->dtype;
  p->scale = s->sm_scale > 0 ? s->sm_scale : 1.0 / sqrt(static_cast<double>(s->head_dim));
  p->qs_tok = s->q_stride_tok;
  p->qs_head = s->q_stride_head;
  p->kvs_tok = s->kv_stride_tok;
  p->kvs_head = s->kv_stride_head;
  p->os_tok = s->o_stride_tok;
  p->os_head = s->o_stride_head;
  p->sched = s->schedule;
  p->recompute_logits = s->select_logits == SPAVA_LOGITS_RECOMPUTE ? 1 : 0;
  // Rows each block passes: C_0 excludes the anchor, C_j (j >= 1) is the whole block.
  const int64_t l0 = p->H > 1 ? std::min<int64_t>(p->l, nb - p->A) : 0;
  const int64_t l1 = p->H > 2 ? std::min<int64_t>(p->l, nb) : 0;
  p->l0 = static_cast<int>(l0);
  p->l1 = static_cast<int>(l1);
  const int64_t lmax = p->H > 1 ? p->A + l0 + (p->H - 2) * l1 : 0;
  if (lmax > (int64_t(1) << 30)) return SPAVA_ERR_SHAPE;
  p->Lmax = static_cast<int>(lmax);
  p->Lpad = static_cast<int>(round_up(lmax, kKeyTile));
  const int64_t R = static_cast<int64_t>(p->G) * p->w;
  if (R > (int64_t(1) << 30)) return SPAVA_ERR_SHAPE;
  p->R = static_cast<int>(R);
  p->T = static_cast<int>(cdiv(nb, kQTile));
  p->loc_tiles = static_cast<int>(cdiv(nb, kKeyTile));
  p->obs_query = 0;
  set_select_layout(p);
  // Every launch must fit a 32-bit work-item count and the int arithmetic of its
  // indexing. The attention grid bound also keeps N * Hq below 2^30.
  if (p->Hq > 65535 || p->Hkv > 65535) return SPAVA_ERR_SHAPE;
  if (!fits_launch({p->H, p->T, p->Hkv})) return SPAVA_ERR_SHAPE;
  const int64_t attn_groups = round_up(static_cast<int64_t>(p->H) * p->T * p->Hkv, 8);
  if (!fits_launch({attn_groups, p->G, 512})) return SPAVA_ERR_SHAPE;    // attention
  if (!fits_launch({p->H, p->loc_tiles})) return SPAVA_ERR_SHAPE;
  // The gather launch also carries the workgroups that rank the attention's work items.
  const int64_t prep_groups = p->Lpad / kKeyTile + static_cast<int64_t>(p->H) * p->loc_tiles +
                              cdiv(static_cast<int64_t>(p->H) * p->T, 256);
  if (!fits_launch({prep_groups, p->Hkv, 256})) return SPAVA_ERR_SHAPE;   // gather
  if (!select_launches_fit(*p)) return SPAVA_ERR_SHAPE;
  return SPAVA_OK;
}

// The selection's key split length (see kScoreSplitMin) and whether its score pass
// reads stored logits (SPAVA_LOGITS_RECOMPUTE makes it recompute them: less
// workspace, more time). Scores are bitwise the same either way: the split length
// depends on the pair count of the whole call, not on the chunks.
void set_select_layout(Plan* p) {
  const int64_t jg = static_cast<int64_t>(p->H > 1 ? p->H - 1 : 0) * p->Hkv;
  const int64_t row_tiles = cdiv(p->R, 32);
  // Past 2^31 (pair, row tile) units the launch check rejects the shape anyway; skip
  // the search there so no product below can overflow.
  const bool huge = jg > INT32_MAX || row_tiles > INT32_MAX / std::max<int64_t>(1, jg);
  const int64_t units = std::max<int64_t>(1, huge ? 1 : jg * row_tiles);
  int64_t best_cost = INT64_MAX;
  p->split_keys = kScoreSplitMax;
  for (int split = kScoreSplitMax; !huge && split >= kScoreSplitMin; split -= 32) {
    const int64_t ks = cdiv(p->nb, split);
    const int64_t cost = cdiv(units * ks, kScoreWaveSlots) *
                         (std::min<int64_t>(split, p->nb) + kScoreWaveOverhead);
    if (cost < best_cost) {
      best_cost = cost;
      p->split_keys = split;
    }
  }
  p->KS = static_cast<int>(cdiv(p->nb, p->split_keys));
  const bool recompute = p->recompute_logits != 0;
  // A pair's stored logits: R rows of round_up(nb, 32) values (32-key tiles).
  // R * nbp * 8 <= kLogitPairBytes, tested without forming the (possibly huge) product.
  const int64_t nbp = round_up(p->nb, 32);
  const bool small = p->R <= kLogitPairBytes / (static_cast<int64_t>(sizeof(double)) * nbp);
  const int64_t per_pair =
      small ? static_cast<int64_t>(p->R) * nbp * static_cast<int64_t>(sizeof(double)) : 0;
  p->store_logits = (!recompute && jg > 0 && small) ? 1 : 0;
  p->pair_chunk = p->store_logits
                      ? static_cast<int>(std::max<int64_t>(1, std::min(jg, kLogitChunkBytes / per_pair)))
                      : 0;
}

SelectWs select_ws_layout(const Plan& p) {
  SelectWs w{};
  size_t cur = 0;
  const size_t jg = static_cast<size_t>(p.H > 1 ? p.H - 1 : 0) * p.Hkv;
  w.rowstat_part = region(cur, jg * p.KS * p.R * 2 * sizeof(double));
  w.rowstat = region(cur, jg * p.R * 2 * sizeof(double));
  w.scores = region(cur, jg * p.nb * sizeof(double));
  w.logits = region(cur, p.store_logits ? static_cast<size_t>(p.pair_chunk) * p.R *
                                              round_up(p.nb, 32) * sizeof(double)
                                        : 0);
  w.total = cur;
  return w;
}

AttnWs attn_ws_layout(const Plan& p) {
  AttnWs w{};
  size_t cur = 0;
  const size_t es = p.dtype == SPAVA_BF16 ? 2 : 4;
  w.kpre = region(cur, static_cast<size_t>(p.Hkv) * p.Lpad * p.D * es);
  w.vpre = region(cur, static_cast<size_t>(p.Hkv) * p.Lpad * p.D * es);
  const size_t loc = p.dtype == SPAVA_BF16
                         ? static_cast<size_t>(p.Hkv) * p.H * p.loc_tiles * kKeyTile * p.D * es
                         : 0;
  w.vtloc = region(cur, loc);
  w.order = region(cur, static_cast<size_t>(p.H) * p.T * sizeof(int32_t));
  w.order2 = region(cur, static_cast<size_t>(p.H) * p.T * sizeof(int32_t));
  w.total = cur;
  return w;
}

OverlapWs overlap_ws_layout(const Plan& p) {
  OverlapWs w{};
  size_t cur = 0;
  w.select = region(cur, select_ws_layout(p).total);
  w.attn = region(cur, attn_ws_layout(p).total);
  w.total = cur;
  return w;
}

QueryWs query_ws_layout(const Plan& p, int64_t nq) {
  QueryWs w{};
  size_t cur = 0;
  const size_t parts = static_cast<size_t>(p.H + 1);
  w.part_o = region(cur, parts * nq * p.Hq * p.D * sizeof(float));
  // float32 inputs keep the partial LSEs in float64 (the merge weights need them).
  w.part_lse = region(cur, parts * p.Hq * nq * (p.dtype == SPAVA_BF16 ? sizeof(float) : sizeof(double)));
  const bool bf = p.dtype == SPAVA_BF16;
  w.vtctx = region(cur, bf ? static_cast<size_t>(p.Hkv) * p.H * p.loc_tiles * kKeyTile * p.D * 2 : 0);
  w.vtq = region(cur, bf ? static_cast<size_t>(p.Hkv) * cdiv(nq, kKeyTile) * kKeyTile * p.D * 2 : 0);
  w.total = cur;
  return w;
}

// Scratch of the allocation-free selection (spava_select_passing_noalloc): one copy
// per GPU, held until the process ends. In host code `scratch` is only a stand-in for
// the device array: its device address comes from hipGetSymbolAddress, once per
// device, and only that address is ever handed to a kernel.
static __device__ __align__(256) unsigned char scratch[SPAVA_NOALLOC_SCRATCH_BYTES];

// Device address of `scratch` on the current device (looked up on first use there).
static spava_status scratch_address(char** out) {
  static std::mutex mu;
  static char* addr[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return SPAVA_ERR_HIP;
  if (dev < 0 || dev >= 64) return SPAVA_ERR_DEVICE;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr)
      return SPAVA_ERR_HIP;
    addr[dev] = static_cast<char*>(ptr);
  }
  *out = addr[dev];
  return SPAVA_OK;
}

// gfx950 check, once per device ordinal.
static spava_status check_device() {
  static std::mutex mu;
  static int known[64];  // 0 unknown, 1 ok, 2 bad
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return SPAVA_ERR_HIP;
  if (dev < 0 || dev >= 64) return SPAVA_ERR_DEVICE;
  std::lock_guard<std::mutex> lock(mu);
  if (known[dev] == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return SPAVA_ERR_HIP;
    known[dev] = strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
  }
  return known[dev] == 1 ? SPAVA_OK : SPAVA_ERR_DEVICE;
}

}  // namespace spava

using namespace spava;

extern "C" {

const char* spava_status_string(int status) {
  switch (status) {
    case SPAVA_OK: return "SPAVA_OK";
    case SPAVA_ERR_NULL: return "SPAVA_ERR_NULL: a required pointer is NULL";
    case SPAVA_ERR_SHAPE: return "SPAVA_ERR_SHAPE: sizes violate the shape constraints";
    case SPAVA_ERR_DTYPE: return "SPAVA_ERR_DTYPE: unknown dtype";
    case SPAVA_ERR_ALIGN: return "SPAVA_ERR_ALIGN: pointer or stride not 16-byte aligned";
    case SPAVA_ERR_WORKSPACE: return "SPAVA_ERR_WORKSPACE: workspace too small";
    case SPAVA_ERR_HIP: return "SPAVA_ERR_HIP: HIP runtime call or kernel launch failed";
    case SPAVA_ERR_DEVICE: return "SPAVA_ERR_DEVICE: current device is not gfx950";
    case SPAVA_ERR_OPTION: return "SPAVA_ERR_OPTION: unknown schedule or select_logits value";
    default: return "SPAVA: unknown status";
  }
}

int spava_abi_version(void) { return 2; }

spava_status spava_validate_shape(const spava_shape* shape) {
  Plan p;
  return make_plan(shape, &p);
}

spava_status spava_select_workspace_bytes(const spava_shape* shape, size_t* bytes) {
  if (!bytes) return SPAVA_ERR_NULL;
  Plan p;
  spava_status st = make_plan(shape, &p);
  if (st != SPAVA_OK) return st;
  *bytes = select_ws_layout(p).total;
  return SPAVA_OK;
}

spava_status spava_attn_workspace_bytes(const spava_shape* shape, size_t* bytes) {
  if (!bytes) return SPAVA_ERR_NULL;
  Plan p;
  spava_status st = make_plan(shape, &p);
  if (st != SPAVA_OK) return st;
  *bytes = attn_ws_layout(p).total;
  return SPAVA_OK;
}

spava_status spava_select_passing(const spava_shape* shape, const void* q, const void* k,
                                  int32_t* passing_idx, double* scores_out, void* workspace,
                                  size_t workspace_bytes, void* stream) {
  Plan p;
  spava_status st = make_plan(shape, &p);
  if (st != SPAVA_OK) return st;
  if (!q || !k) return SPAVA_ERR_NULL;
  const bool any = p.H > 1 && p.l > 0;
  if (p.H > 1 && p.l > 0 && !passing_idx) return SPAVA_ERR_NULL;
  if (!aligned16(q) || !aligned16(k)) return SPAVA_ERR_ALIGN;
  if (passing_idx && (reinterpret_cast<uintptr_t>(passing_idx) & 3u)) return SPAVA_ERR_ALIGN;
  if (scores_out && (reinterpret_cast<uintptr_t>(scores_out) & 7u)) return SPAVA_ERR_ALIGN;
  const SelectWs ws = select_ws_layout(p);
  const bool need_ws = p.H > 1 && (any || scores_out);
  if (need_ws) {
    if (!workspace) return SPAVA_ERR_NULL;
    if (!aligned16(workspace)) return SPAVA_ERR_ALIGN;
    if (workspace_bytes < ws.total) return SPAVA_ERR_WORKSPACE;
  }
  if (p.H == 1) return SPAVA_OK;                 // no block passes anything
  if (!any && !scores_out) return SPAVA_OK;      // l == 0: the index array is empty
  st = check_device();
  if (st != SPAVA_OK) return st;
  hipError_t e = launch_select(p, q, k, passing_idx, scores_out, static_cast<char*>(workspace),
                               static_cast<hipStream_t>(stream));
  return e == hipSuccess ? SPAVA_OK : SPAVA_ERR_HIP;
}

spava_status spava_select_passing_noalloc(const spava_shape* shape, const void* q,
                                          const void* k, int32_t* passing_idx,
                                          double* scores_out, void* stream) {
  if (!shape) return SPAVA_ERR_NULL;
  // The same plan as spava_select_passing with the logits recomputed: the scratch then
  // holds only the row statistics and the scores.
  spava_shape s = *shape;
  s.select_logits = SPAVA_LOGITS_RECOMPUTE;
  Plan p;
  spava_status st = make_plan(&s, &p);
  if (st != SPAVA_OK) return st;
  if (!q || !k) return SPAVA_ERR_NULL;
  const bool any = p.H > 1 && p.l > 0;
  if (any && !passing_idx) return SPAVA_ERR_NULL;
  if (!aligned16(q) || !aligned16(k)) return SPAVA_ERR_ALIGN;
  if (passing_idx && (reinterpret_cast<uintptr_t>(passing_idx) & 3u)) return SPAVA_ERR_ALIGN;
  if (scores_out && (reinterpret_cast<uintptr_t>(scores_out) & 7u)) return SPAVA_ERR_ALIGN;
  if (select_ws_layout(p).total > SPAVA_NOALLOC_SCRATCH_BYTES) return SPAVA_ERR_WORKSPACE;
  if (p.H == 1 || (!any && !scores_out)) return SPAVA_OK;
  st = check_device();
  if (st != SPAVA_OK) return st;
  char* ws = nullptr;
  st = scratch_address(&ws);
  if (st != SPAVA_OK) return st;
  hipError_t e = launch_select(p, q, k, passing_idx, scores_out, ws,
                               static_cast<hipStream_t>(stream));
  return e == hipSuccess ? SPAVA_OK : SPAVA_ERR_HIP;
}

spava_status spava_approx_attn_fwd(const spava_shape* shape, const void* q, const void* k,
                                   const void* v, const int32_t* passing_idx, void* out,
                                   float* lse_out, void* workspace, size_t workspace_bytes,
                                   void* stream) {
  Plan p;
  spava_status st = make_plan(shape, &p);
  if (st != SPAVA_OK) return st;
  if (!q || !k || !v || !out) return SPAVA_ERR_NULL;
  if (p.H > 1 && p.l > 0 && !passing_idx) return SPAVA_ERR_NULL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out)) return SPAVA_ERR_ALIGN;
  if (passing_idx && (reinterpret_cast<uintptr_t>(passing_idx) & 3u)) return SPAVA_ERR_ALIGN;
  if (lse_out && (reinterpret_cast<uintptr_t>(lse_out) & 3u)) return SPAVA_ERR_ALIGN;
  const AttnWs ws = attn_ws_layout(p);
  if (!workspace) return SPAVA_ERR_NULL;
  if (!aligned16(workspace)) return SPAVA_ERR_ALIGN;
  if (workspace_bytes < ws.total) return SPAVA_ERR_WORKSPACE;
  st = check_device();
  if (st != SPAVA_OK) return st;
  hipError_t e;
  if (p.dtype == SPAVA_BF16)
    e = launch_attn_bf16(p, q, k, v, passing_idx, out, lse_out, static_cast<char*>(workspace),
                         static_cast<hipStream_t>(stream));
  else
    e = launch_attn_f32(p, q, k, v, passing_idx, out, lse_out, static_cast<char*>(workspace),
                        static_cast<hipStream_t>(stream));
  return e == hipSuccess ? SPAVA_OK : SPAVA_ERR_HIP;
}

// The query block's launches: 1 <= n_query <= 2^30, partial and merge grids in range.
static bool query_launches_fit(const Plan& p, int64_t nq) {
  if (nq < 1 || nq > (int64_t(1) << 30)) return false;
  return fits_launch({static_cast<int64_t>(p.H) + 1, cdiv(nq, kQTile), p.Hkv}) &&
         fits_launch({round_up((static_cast<int64_t>(p.H) + 1) * cdiv(nq, kQTile) * p.Hkv, 8),
                      p.G, 512}) &&
         fits_launch({nq, p.Hq, p.D / 4}) && fits_launch({cdiv(nq, kKeyTile), 256});
}

// Plan of the query-aware selection: observers are the n_query rows of a query block.
static spava_status make_query_select_plan(const spava_shape* shape, int64_t n_query, Plan* p) {
  spava_status st = make_plan(shape, p);
  if (st != SPAVA_OK) return st;
  if (n_query < 1 || n_query * p->G > (int64_t(1) << 30)) return SPAVA_ERR_SHAPE;
  p->w = static_cast<int>(n_query);
  p->R = static_cast<int>(n_query * p->G);
  p->obs_query = 1;
  set_select_layout(p);
  if (!select_launches_fit(*p)) return SPAVA_ERR_SHAPE;
  return SPAVA_OK;
}

spava_status spava_select_query_workspace_bytes(const spava_shape* shape, int64_t n_query,
                                                size_t* bytes) {
  if (!bytes) return SPAVA_ERR_NULL;
  Plan p;
  spava_status st = make_query_select_plan(shape, n_query, &p);
  if (st != SPAVA_OK) return st;
  *bytes = select_ws_layout(p).total;
  return SPAVA_OK;
}

spava_status spava_select_passing_query(const spava_shape* shape, int64_t n_query,
                                        const void* q_qr, const void* k, int32_t* passing_idx,
                                        double* scores_out, void* workspace,
                                        size_t workspace_bytes, void* stream) {
  Plan p;
  spava_status st = make_query_select_plan(shape, n_query, &p);
  if (st != SPAVA_OK) return st;
  if (!q_qr || !k) return SPAVA_ERR_NULL;
  const bool any = p.H > 1 && p.l > 0;
  if (any && !passing_idx) return SPAVA_ERR_NULL;
  if (!aligned16(q_qr) || !aligned16(k)) return SPAVA_ERR_ALIGN;
  if (passing_idx && (reinterpret_cast<uintptr_t>(passing_idx) & 3u)) return SPAVA_ERR_ALIGN;
  if (scores_out && (reinterpret_cast<uintptr_t>(scores_out) & 7u)) return SPAVA_ERR_ALIGN;
  const SelectWs ws = select_ws_layout(p);
  if (p.H > 1 && (any || scores_out)) {
    if (!workspace) return SPAVA_ERR_NULL;
    if (!aligned16(workspace)) return SPAVA_ERR_ALIGN;
    if (workspace_bytes < ws.total) return SPAVA_ERR_WORKSPACE;
  }
  if (p.H == 1 || (!any && !scores_out)) return SPAVA_OK;
  st = check_device();
  if (st != SPAVA_OK) return st;
  hipError_t e = launch_select(p, q_qr, k, passing_idx, scores_out, static_cast<char*>(workspace),
                               static_cast<hipStream_t>(stream));
  return e == hipSuccess ? SPAVA_OK : SPAVA_ERR_HIP;
}

spava_status spava_query_workspace_bytes(const spava_shape* shape, int64_t n_query,
                                         size_t* bytes) {
  if (!bytes) return SPAVA_ERR_NULL;
  Plan p;
  spava_status st = make_plan(shape, &p);
  if (st != SPAVA_OK) return st;
  if (!query_launches_fit(p, n_query)) return SPAVA_ERR_SHAPE;
  *bytes = query_ws_layout(p, n_query).total;
  return SPAVA_OK;
}

spava_status spava_query_attn_fwd(const spava_shape* shape, int64_t n_query, const void* q_qr,
                                  const void* k_qr, const void* v_qr, const void* k,
                                  const void* v, void* out_qr, float* lse_qr, void* workspace,
                                  size_t workspace_bytes, void* stream) {
  Plan p;
  spava_status st = make_plan(shape, &p);
  if (st != SPAVA_OK) return st;
  if (!query_launches_fit(p, n_query)) return SPAVA_ERR_SHAPE;
  if (!q_qr || !k_qr || !v_qr || !k || !v || !out_qr || !workspace) return SPAVA_ERR_NULL;
  if (!aligned16(q_qr) || !aligned16(k_qr) || !aligned16(v_qr) || !aligned16(k) ||
      !aligned16(v) || !aligned16(out_qr) || !aligned16(workspace))
    return SPAVA_ERR_ALIGN;
  if (lse_qr && (reinterpret_cast<uintptr_t>(lse_qr) & 3u)) return SPAVA_ERR_ALIGN;
  if (workspace_bytes < query_ws_layout(p, n_query).total) return SPAVA_ERR_WORKSPACE;
  st = check_device();
  if (st != SPAVA_OK) return st;
  hipError_t e = launch_query(p, n_query, q_qr, k_qr, v_qr, k, v, out_qr, lse_qr,
                              static_cast<char*>(workspace), static_cast<hipStream_t>(stream));
  return e == hipSuccess ? SPAVA_OK : SPAVA_ERR_HIP;
}

spava_status spava_layer_overlap_workspace_bytes(const spava_shape* shape, size_t* bytes) {
  if (!bytes) return SPAVA_ERR_NULL;
  Plan p;
  spava_status st = make_plan(shape, &p);
  if (st != SPAVA_OK) return st;
  *bytes = overlap_ws_layout(p).total;
  return SPAVA_OK;
}

spava_status spava_layer_overlap_fwd(const spava_shape* shape, const void* q, const void* k,
                                     const void* v, int32_t* passing_idx, double* scores_out,
                                     void* out, float* lse_out, void* workspace,
                                     size_t workspace_bytes, void* stream, void* side_stream) {
  Plan p;
  spava_status st = make_plan(shape, &p);
  if (st != SPAVA_OK) return st;
  if (p.dtype != SPAVA_BF16) return SPAVA_ERR_DTYPE;
  if (!q || !k || !v || !out || !workspace) return SPAVA_ERR_NULL;
  const bool any = p.H > 1 && p.l > 0;
  if (any && !passing_idx) return SPAVA_ERR_NULL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) || !aligned16(workspace))
    return SPAVA_ERR_ALIGN;
  if (passing_idx && (reinterpret_cast<uintptr_t>(passing_idx) & 3u)) return SPAVA_ERR_ALIGN;
  if (scores_out && (reinterpret_cast<uintptr_t>(scores_out) & 7u)) return SPAVA_ERR_ALIGN;
  if (lse_out && (reinterpret_cast<uintptr_t>(lse_out) & 3u)) return SPAVA_ERR_ALIGN;
  const OverlapWs w = overlap_ws_layout(p);
  if (workspace_bytes < w.total) return SPAVA_ERR_WORKSPACE;
  st = check_device();
  if (st != SPAVA_OK) return st;
  char* ws = static_cast<char*>(workspace);
  hipStream_t main_st = static_cast<hipStream_t>(stream);
  hipStream_t side_st = static_cast<hipStream_t>(side_stream);
  // Nothing to select: the plain layer on the main stream.
  if (!any) {
    if (p.H > 1 && scores_out &&
        launch_select(p, q, k, passing_idx, scores_out, ws + w.select, main_st) != hipSuccess)
      return SPAVA_ERR_HIP;
    return launch_attn_bf16(p, q, k, v, passing_idx, out, lse_out, ws + w.attn, main_st) ==
                   hipSuccess
               ? SPAVA_OK
               : SPAVA_ERR_HIP;
  }
  // Two events per thread and device, created on first use and kept: this entry
  // records and waits on them within one call, so reusing them across calls (in
  // stream order) is safe, and concurrent callers on other threads have their own.
  struct CallEvents {
    hipEvent_t ev[64][2];
  };
  thread_local CallEvents tev{};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return SPAVA_ERR_HIP;
  if (dev < 0 || dev >= 64) return SPAVA_ERR_DEVICE;
  for (int i = 0; i < 2; ++i)
    if (tev.ev[dev][i] == nullptr &&
        hipEventCreateWithFlags(&tev.ev[dev][i], hipEventDisableTiming) != hipSuccess) {
      tev.ev[dev][i] = nullptr;
      return SPAVA_ERR_HIP;
    }
  hipEvent_t inputs_ready = tev.ev[dev][0], passing_ready = tev.ev[dev][1];
  bool ok = true;
  // Side stream: the selection, once the main stream has reached this call (the inputs
  // are ready there).
  ok = ok && hipEventRecord(inputs_ready, main_st) == hipSuccess;
  ok = ok && hipStreamWaitEvent(side_st, inputs_ready, 0) == hipSuccess;
  ok = ok && launch_select(p, q, k, passing_idx, scores_out, ws + w.select, side_st) == hipSuccess;
  ok = ok && hipEventRecord(passing_ready, side_st) == hipSuccess;
  // Main stream: block 0 meanwhile (no passing rows), then the other blocks.
  ok = ok && launch_attn_bf16_block0(p, q, k, v, out, lse_out, ws + w.attn, main_st) == hipSuccess;
  ok = ok && hipStreamWaitEvent(main_st, passing_ready, 0) == hipSuccess;
  ok = ok && launch_attn_bf16_rest(p, q, k, v, passing_idx, out, lse_out, ws + w.attn, main_st) ==
                 hipSuccess;
  return ok ? SPAVA_OK : SPAVA_ERR_HIP;
}

}  // extern "C"
