// Device pieces shared by the bf16 attention kernels (approximate attention over
// [anchor | passing | local causal] and the query-block partials): LDS tile layout,
// the V^T key-slot order, and one flash-attention step over a 64-key tile.
//
// MFMA 32x32x16 bf16 operand layout (wave64): lane l supplies row/column (l % 32) of
// A/B and 8 consecutive reduction slots selected by (l / 32); accumulator register r
// of lane l holds row 8*(r/4) + 4*(l/32) + (r%4), column l % 32. Computing S^T (keys x
// queries) leaves each lane with one query and 16 keys per 32-key block, which is
// exactly the B operand P^T of the second product once V^T's key slots are stored in
// the same order; so P never leaves registers.
#pragma once

#include "spava_internal.h"

namespace spava {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int BN = kKeyTile;                  // 64 keys per tile
constexpr int VROWB = BN * 2 + 16;            // bytes per V^T row in LDS (padded)
constexpr int kWaves = 8;                     // waves per attention workgroup
constexpr int kThreads = kWaves * 64;
constexpr int kWaveQ = 32;                    // queries per wave
static_assert(kWaves * kWaveQ == kQTile, "query tile must match the plan");

// Softmax reference (log2 units). p = exp2(c*s - ref) is computed against the running
// reference first; only when a lane's partial sum of the tile's bf16 weights leaves
// [0, kSumLimit] (a logit about 8 or more above the reference, or the first unmasked
// tile) is the reference
// raised to the tile maximum, O and the row sum rescaled and the tile recomputed. So
// the per-tile maximum is never needed on the common path. The result is exact:
// numerator and denominator share the reference. Raising the reference to a new
// dominant logit keeps that key's weight at exactly 1, free of bf16 rounding in P;
// for a dominant key below that limit, O's normaliser sums the same bf16 weights the
// product uses (Flash::lsum_b), so the key's rounding cancels.
// kRefInit is finite so that masked scores (-inf) give p = 0 and never NaN.
constexpr float kRefInit = -1.0e30f;
constexpr float kSumLimit = 256.0f;

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

// Write one 64-key V^T tile [D][64] (slot order) to global memory from 64 V rows
// staged in LDS as Vs[row][D + 8]; called by all 256 threads of a workgroup.
template <int D>
__device__ inline void store_vt_tile(const uint16_t (*Vs)[D + 8], uint16_t* dst) {
  for (int c = threadIdx.x; c < D * (BN / 8); c += 256) {
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

typedef __attribute__((address_space(3))) void* lds_ptr_t;
// A generic pointer into __shared__ memory as an LDS-address-space pointer.
__device__ inline lds_ptr_t as_lds(char* ptr) { return (lds_ptr_t)(ptr); }
// One 16-byte-per-lane buffer load into LDS (64 lanes -> 1 KB at dst + 16 * lane).
// A plain function, not a template member: with the builtin called directly from
// the kernel templates, the host pass emitted the launch stub of only one of them.
__device__ inline void load_lds16(__amdgpu_buffer_rsrc_t rsrc, lds_ptr_t dst, uint32_t voffset) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, dst, 16, voffset, 0, 0, 0);
}

// Direct global -> LDS tile loads (buffer_load_dwordx4 with the LDS bit): no
// register staging and no LDS store instructions. A stage (K rows of KROWB bytes,
// then V^T rows of VROWB bytes, each row ending in a 16-byte pad) is a run of
// 16-byte slots; one load writes 64 consecutive slots (1 KB at the wave's LDS
// address + 16 * lane), and each lane fetches the global chunk that belongs in its
// slot. Pad slots, and K rows past the valid count, use offsets beyond the buffer's
// range: the hardware reads nothing for them. Wave w loads K blocks 8r + w and V^T
// blocks 8r + w in full rounds of eight, then at most one of the leftover blocks.
// Completion is tracked by vmcnt: wait_tile_loads() then a barrier publishes a stage.
template <int D>
struct TileDma {
  using C = Cfg<D>;
  static constexpr int KSPR = C::KROWB / 16, VSPR = VROWB / 16;   // slots per row
  static constexpr int KBLK = C::KBYTES / 1024, VBLK = C::VBYTES / 1024;
  static constexpr int KR = KBLK / kWaves, VR = VBLK / kWaves;     // full rounds
  static constexpr int KREM = KBLK % kWaves, VREM = VBLK % kWaves;
  static_assert(C::KBYTES % 1024 == 0 && C::VBYTES % 1024 == 0, "stage must be whole 1 KB blocks");
  static_assert(KREM + VREM <= kWaves, "leftover blocks must fit one round");
  static constexpr uint32_t kOut = 0x7FFFFFF0u;   // past every buffer range
  static constexpr int kRsrcFlags = 0x00020000;   // raw buffer, 32-bit data format
  int wave;                            // this wave's index (wave-uniform)
  uint32_t kpre[KR], kloc[KR];         // byte offsets of K rows: 2D-byte rows, runtime stride
  uint32_t voff[VR];                   // byte offsets into the V^T tile
  uint32_t tpre, tloc;                 // the leftover block's offsets (V^T: both equal)
  int tkind;                           // leftover block: 0 K, 1 V^T, 2 none (wave-uniform)
  int tlds;                            // its LDS offset inside a stage

  __device__ static void k_offsets(int blk, int lane, int64_t krow_loc, uint32_t& pre,
                                   uint32_t& loc) {
    const int sl = blk * 64 + lane, r = sl / KSPR, c = sl % KSPR;
    pre = kOut;
    loc = kOut;
    if (c < D / 8) {
      pre = static_cast<uint32_t>(r * (2 * D) + c * 16);
      loc = static_cast<uint32_t>(r * krow_loc * 2 + c * 16);
    }
  }
  __device__ static uint32_t v_offset(int blk, int lane) {
    const int sl = blk * 64 + lane, r = sl / VSPR, c = sl % VSPR;
    return c < BN / 8 ? static_cast<uint32_t>(r * (2 * BN) + c * 16) : kOut;
  }

  // krow_loc: row stride (elements) of K read in place; (BN - 1) * krow_loc * 2 + 2D
  // must stay below 2^31 (the plan checks this).
  __device__ void init(int64_t krow_loc) {
    wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int r = 0; r < KR; ++r) k_offsets(r * kWaves + wave, lane, krow_loc, kpre[r], kloc[r]);
#pragma unroll
    for (int r = 0; r < VR; ++r) voff[r] = v_offset(r * kWaves + wave, lane);
    tkind = wave < KREM ? 0 : (wave < KREM + VREM ? 1 : 2);
    tpre = kOut;
    tloc = kOut;
    tlds = 0;
    if (tkind == 0) {
      k_offsets(KR * kWaves + wave, lane, krow_loc, tpre, tloc);
      tlds = (KR * kWaves + wave) * 1024;
    } else if (tkind == 1) {
      tpre = tloc = v_offset(VR * kWaves + wave - KREM, lane);
      tlds = C::KBYTES + (VR * kWaves + wave - KREM) * 1024;
    }
  }
  // Bytes of a K tile's buffer range: `rows` rows of `stride` elements, the last one
  // ending after its 2D bytes of data.
  __device__ static int k_range(int64_t rows, int64_t stride) {
    return static_cast<int>((rows - 1) * stride * 2 + 2 * D);
  }
  // kb: first K row of the tile; local: rows use the runtime stride (else 2D bytes
  // per row); kbytes: k_range of the rows present; vb: the V^T tile [D][BN].
  __device__ void issue(const uint16_t* kb, bool local, int kbytes, const uint16_t* vb,
                        char* dst) const {
    const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(kb), static_cast<short>(0), kbytes, kRsrcFlags);
    const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(vb), static_cast<short>(0), D * BN * 2, kRsrcFlags);
#pragma unroll
    for (int r = 0; r < KR; ++r) {
      const uint32_t a = kpre[r], b = kloc[r];
      load_lds16(rk, as_lds(dst + (r * kWaves + wave) * 1024), local ? b : a);
    }
#pragma unroll
    for (int r = 0; r < VR; ++r)
      load_lds16(rv, as_lds(dst + C::KBYTES + (r * kWaves + wave) * 1024), voff[r]);
    const uint32_t ta = tpre, tb = tloc;
    if (tkind == 0)
      load_lds16(rk, as_lds(dst + tlds), local ? tb : ta);
    else if (tkind == 1)
      load_lds16(rv, as_lds(dst + tlds), ta);
  }
};

// Wait for this wave's outstanding global -> LDS tile loads (vmcnt(0); other
// counters left alone). A barrier after it makes the stage visible to every wave.
__device__ inline void wait_tile_loads() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Per-wave flash state for 32 queries: O^T accumulators, running reference max
// (log2 units) and this lane's partial row sums (keys it holds; the partner lane
// l ^ 32 holds the rest of the query's keys): lsum of the float32 weights, which the
// log-sum-exp uses, and lsum_b of the same weights rounded to bf16, exactly as they
// enter the P V product, which normalises O. With one normaliser per side, numerator
// and denominator carry the same rounding: a row dominated by one key whose weight
// sits far from a power of two gets that key's v back, not v times its weight's bf16
// rounding error (up to 2^-8, i.e. 0.018 for |v| = 4.5).
template <int D>
struct Flash {
  f32x16 o[Cfg<D>::DM];
  float mrun, lsum, lsum_b;
  __device__ void init() {
#pragma unroll
    for (int dm = 0; dm < Cfg<D>::DM; ++dm)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[dm][r] = 0.f;
    mrun = kRefInit;
    lsum = 0.f;
    lsum_b = 0.f;
  }
};

// Load this lane's Q fragments (B operand of S^T = K Q^T) for query row qp (a pointer
// to the row's d values, already offset by lh * 8), or zeros.
template <int D>
__device__ inline void load_q(const uint16_t* qp, bool ok, bf16x8 (&qf)[Cfg<D>::DK]) {
#pragma unroll
  for (int dk = 0; dk < Cfg<D>::DK; ++dk) {
    u32x4 raw = ok ? *reinterpret_cast<const u32x4*>(qp + dk * 16) : u32x4{0u, 0u, 0u, 0u};
    qf[dk] = __builtin_bit_cast(bf16x8, raw);
  }
}

// p = exp2(c*s - ref) of this lane's 32 scores, packed to bf16 in the P^T operand
// order; returns the lane's partial sum of the float32 values when SUM (else 0: a
// caller that wants no log-sum-exp needs only the bf16 weights).
template <bool SUM>
__device__ inline float exp_tile(const f32x16 (&s)[2], float ref, float c_log2, bf16x8 (&pf)[4]) {
  // Two chains, each started from its first pair (p >= 0, so this equals 0 + pair).
  float sum0 = 0.f, sum1 = 0.f;
#pragma unroll
  for (int kc = 0; kc < 4; ++kc) {
    const int kb = kc >> 1, half = kc & 1;
#pragma unroll
    for (int e2 = 0; e2 < 4; ++e2) {
      const int r = half * 8 + 2 * e2;
      f32x2 two = {__builtin_amdgcn_exp2f(fmaf(s[kb][r], c_log2, -ref)),
                   __builtin_amdgcn_exp2f(fmaf(s[kb][r + 1], c_log2, -ref))};
      if (SUM) {
        const float pr = two[0] + two[1];
        if (kc & 1) sum1 = (kc == 1 && e2 == 0) ? pr : sum1 + pr;
        else sum0 = (kc == 0 && e2 == 0) ? pr : sum0 + pr;
      }
      const bf16x2 cv = __builtin_convertvector(two, bf16x2);
      pf[kc][2 * e2] = cv[0];
      pf[kc][2 * e2 + 1] = cv[1];
    }
  }
  return sum0 + sum1;
}

// Sum of this lane's 32 bf16 weights of a tile (v_dot2 against (1, 1): the products
// are exact, two accumulation chains). Each dword is copied to a scalar before the
// bit cast: a bit cast applied to a vector subscript directly lost the subscript
// (every call read element 0).
__device__ inline float bf16_tile_sum(const bf16x8 (&pf)[4]) {
  const bf16x2 ones = {static_cast<__bf16>(1.0f), static_cast<__bf16>(1.0f)};
  float s0 = 0.f, s1 = 0.f;
#pragma unroll
  for (int kc = 0; kc < 4; ++kc) {
    const u32x4 w = __builtin_bit_cast(u32x4, pf[kc]);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t word = w[e];
      const bf16x2 pair = __builtin_bit_cast(bf16x2, word);
      if (e & 1) s1 = __builtin_amdgcn_fdot2_f32_bf16(pair, ones, s1, false);
      else s0 = __builtin_amdgcn_fdot2_f32_bf16(pair, ones, s0, false);
    }
  }
  return s0 + s1;
}

// K fragments held ahead of a tile step: those of the first kSteps head-dim steps
// (kSteps of DK, both 32-row key blocks). The loop reads them for tile t+1 from LDS
// during the second half of tile t's P V, so the products of tile t+1 start without
// waiting for LDS; the remaining DK - kSteps steps are read at the start of the step.
// (All DK steps ahead would need 32 more registers than two waves per SIMD allow.)
template <int D>
struct KHead {
  static constexpr int kSteps = Cfg<D>::DK < 4 ? Cfg<D>::DK : 4;
  bf16x8 f[2 * kSteps];
  __device__ void read(const char* ks) {
    using C = Cfg<D>;
    const int lane = threadIdx.x & 63;
    const int lr = lane & 31, lh = lane >> 5;
#pragma unroll
    for (int dk = 0; dk < kSteps; ++dk)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
        f[dk * 2 + kb] = *reinterpret_cast<const bf16x8*>(ks + (kb * 32 + lr) * C::KROWB +
                                                         (dk * 16 + lh * 8) * 2);
  }
};

// One 64-key tile (K rows at ks, V^T at ks + KBYTES) for this wave's 32 queries:
// S^T = K Q^T, then, when `masked` (a wave-uniform flag), hide keys kk > lim() (kk = key
// index inside the tile; lim() >= 63 hides nothing; evaluated only for masked tiles, so
// unmasked ones pay no per-lane limit arithmetic), online softmax in the log2 domain
// against the running reference, then O^T += V^T P^T. kh holds this tile's first K
// fragments on entry; when ks_next is not null it holds the next tile's on return
// (read during the second half of P V). LDS fragments are read in batches ahead of
// their products (the rest of K first; V^T in two halves), so each batch is in flight
// while earlier work runs. LSE: also sum the float32 weights for the log-sum-exp (30
// VALU instructions per tile) and check the reference against that sum; without it the
// check uses the sum of the bf16 weights that O's normaliser needs anyway. The two sums
// differ by the bf16 rounding, so near the limit the variants may raise the reference
// at different tiles; O then differs in rounding only.
template <int D, bool LSE, typename LimFn>
__device__ inline void attend_tile(KHead<D>& kh, const char* ks, const char* ks_next,
                                   const bf16x8 (&qf)[Cfg<D>::DK], Flash<D>& f, bool masked,
                                   LimFn lim_of, float c_log2) {
  using C = Cfg<D>;
  constexpr int KH = KHead<D>::kSteps;
  const int lane = threadIdx.x & 63;
  const int lr = lane & 31, lh = lane >> 5;
  const char* vs = ks + C::KBYTES;
  bf16x8 kr[2 * (C::DK - KH) + 1];
#pragma unroll
  for (int dk = KH; dk < C::DK; ++dk)
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
      kr[(dk - KH) * 2 + kb] = *reinterpret_cast<const bf16x8*>(ks + (kb * 32 + lr) * C::KROWB +
                                                               (dk * 16 + lh * 8) * 2);
  f32x16 s[2];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int r = 0; r < 16; ++r) s[kb][r] = 0.f;
#pragma unroll
  for (int dk = 0; dk < C::DK; ++dk)
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
      s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
          dk < KH ? kh.f[dk * 2 + kb] : kr[(dk - KH) * 2 + kb], qf[dk], s[kb], 0, 0, 0);
  // V^T fragments of key chunks 0-1 now (in flight during the softmax), of chunks 2-3
  // once the first half of the products is issued.
  bf16x8 vf[4 * C::DM];
  auto read_v = [&](int kc) {
#pragma unroll
    for (int dm = 0; dm < C::DM; ++dm)
      vf[kc * C::DM + dm] = *reinterpret_cast<const bf16x8*>(vs + (dm * 32 + lr) * VROWB +
                                                            (kc * 16 + lh * 8) * 2);
  };
  read_v(0);
  read_v(1);
  __builtin_amdgcn_sched_barrier(0);
  if (masked) {
    const int lim = lim_of();
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int kk = kb * 32 + 8 * (r >> 2) + 4 * lh + (r & 3);
        if (kk > lim) s[kb][r] = -INFINITY;
      }
  }
  bf16x8 pf[4];
  float ps = exp_tile<LSE>(s, f.mrun, c_log2, pf);
  float pb = 0.f;
  if (!LSE) pb = bf16_tile_sum(pf);
  if (__any(!((LSE ? ps : pb) <= kSumLimit))) {
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float mnew = fmaxf(f.mrun, mx * c_log2);
    const float alpha = __builtin_amdgcn_exp2f(f.mrun - mnew);
    f.mrun = mnew;
    f.lsum *= alpha;
    f.lsum_b *= alpha;
#pragma unroll
    for (int dm = 0; dm < C::DM; ++dm)
#pragma unroll
      for (int r = 0; r < 16; ++r) f.o[dm][r] *= alpha;
    ps = exp_tile<LSE>(s, mnew, c_log2, pf);
    if (!LSE) pb = bf16_tile_sum(pf);
  }
  if (LSE) {
    f.lsum += ps;
    pb = bf16_tile_sum(pf);
  }
  f.lsum_b += pb;
#pragma unroll
  for (int kc = 0; kc < 2; ++kc)
#pragma unroll
    for (int dm = 0; dm < C::DM; ++dm)
      f.o[dm] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[kc * C::DM + dm], pf[kc], f.o[dm], 0, 0, 0);
  read_v(2);
  read_v(3);
  if (ks_next != nullptr) kh.read(ks_next);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int kc = 2; kc < 4; ++kc)
#pragma unroll
    for (int dm = 0; dm < C::DM; ++dm)
      f.o[dm] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[kc * C::DM + dm], pf[kc], f.o[dm], 0, 0, 0);
}

// Final row sums of this lane's query (both lanes of the pair hold the same value):
// of the float32 weights (for the log-sum-exp) and of the bf16 weights (normalises O).
template <int D>
__device__ inline float flash_rowsum(const Flash<D>& f) {
  return f.lsum + __shfl_xor(f.lsum, 32);
}
template <int D>
__device__ inline float flash_rowsum_b(const Flash<D>& f) {
  return f.lsum_b + __shfl_xor(f.lsum_b, 32);
}

// O[d] for this lane's query is f.o[dm][grp*4 + j] at d = dm*32 + 8*grp + 4*(l/32) + j.
template <int D>
__device__ inline int out_dim(int dm, int grp, int lh) {
  return dm * 32 + 8 * grp + 4 * lh;
}

}  // namespace spava
