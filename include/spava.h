/*
 * spava.h -- C ABI of the Spava / APB-V approximate-attention prefill library for
 * AMD Instinct MI355X (gfx950).
 *
 * The method (arXiv 2601.21444; pages: "Spava: Accelerating Long-Video Understanding
 * via Sequence-Parallelism-aware Approximate Attention", abstract; and the
 * explainer "APB-V: ..." on gist.science, section "Methodik: APB-V" >
 * "Approximativer Attention-Mechanismus"): the token sequence is cut into H
 * contiguous context blocks. Queries of block h attend causally to their own keys,
 * to an anchor block (the first A tokens) and to the passing blocks of all earlier
 * blocks: the l most important key/value rows each earlier block forwards, chosen
 * by query-to-context attention scores. Here all H "hosts" run on one GPU.
 *
 * Two calls make one prefill layer over the context:
 *   spava_select_passing   scores every key of blocks 0..H-2 and picks each
 *                          block's passing rows per KV head;
 *   spava_approx_attn_fwd  gathers anchor + passing rows and runs the attention.
 * A third call attends a query block (the text question after the context) to the
 * whole context exactly, by per-host partials merged with their log-sum-exp:
 *   spava_query_attn_fwd.
 * spava_layer_overlap_fwd does the two calls of a layer at once, overlapping the
 * selection with the part of the attention that needs no passing rows.
 *
 * Two execution choices travel in the shape struct, never in process state: the
 * dispatch order of the attention's query tiles (spava_shape.schedule) and whether
 * the selection keeps or recomputes its float64 logits (spava_shape.select_logits).
 * Neither changes any result. The library reads no environment variable.
 *
 * Conventions shared by every entry point
 *   - All tensor pointers are DEVICE pointers owned by the caller. The library
 *     allocates no device memory: scratch space is the caller's `workspace`, sized
 *     by the matching *_workspace_bytes query. Nothing is retained after a call.
 *   - Calls enqueue work on `stream` (a hipStream_t; NULL = the default stream) and
 *     return without waiting. Results are ready once the stream reaches that point.
 *   - Every argument is checked on the host before anything is enqueued; on any
 *     error nothing is enqueued and the status says why. SPAVA_ERR_HIP reports a
 *     launch failure; a fault inside a kernel surfaces at the caller's next
 *     synchronisation.
 *   - Calls are reentrant. Concurrent calls may share inputs but not outputs or
 *     workspace.
 *   - Inputs must be finite. Batch size is 1; one attention layer per call.
 */
#ifndef SPAVA_H
#define SPAVA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SPAVA_OK = 0,
  SPAVA_ERR_NULL = 1,       /* a required pointer is NULL                           */
  SPAVA_ERR_SHAPE = 2,      /* sizes violate the constraints below                  */
  SPAVA_ERR_DTYPE = 3,      /* unknown dtype                                        */
  SPAVA_ERR_ALIGN = 4,      /* pointer or stride not 16-byte aligned                */
  SPAVA_ERR_WORKSPACE = 5,  /* workspace smaller than the size query returned       */
  SPAVA_ERR_HIP = 6,        /* a HIP runtime call or kernel launch failed           */
  SPAVA_ERR_DEVICE = 7,     /* current device is not gfx950                         */
  SPAVA_ERR_OPTION = 8      /* schedule or select_logits holds an unknown value      */
} spava_status;

typedef enum { SPAVA_BF16 = 0, SPAVA_F32 = 1 } spava_dtype;

/*
 * Dispatch order of the attention's (block, query tile) work items
 * (spava_shape.schedule). Outputs are bitwise the same under every order; only the
 * time differs. The explainer's load balancing ("Systemseitige Optimierungen":
 * ZigZag pairing of hosts h and H-1-h so every host carries the same work) becomes,
 * on one GPU, an order in which the hardware dispatcher takes the longest items first.
 */
typedef enum {
  SPAVA_SCHED_LONGEST_FIRST = 0,  /* decreasing key-tile count, ties by index (default) */
  SPAVA_SCHED_NATURAL = 1,        /* block-major                                        */
  SPAVA_SCHED_ZIGZAG = 2          /* blocks paired (p, H-1-p), tiles of a pair alternating */
} spava_schedule;

/*
 * Where the selection's second pass gets the float64 logits from
 * (spava_shape.select_logits). Scores and indices are bitwise the same either way;
 * the workspace size follows this field.
 */
typedef enum {
  SPAVA_LOGITS_AUTO = 0,       /* keep the first pass's logits when one (block, KV head)
                                  pair's take at most 512 MiB (G * w * n_b * 8 bytes),
                                  in chunks of at most 4 GiB of logits; else recompute
                                  (default)                                             */
  SPAVA_LOGITS_RECOMPUTE = 1   /* always recompute them: less workspace, more time      */
} spava_select_logits;

/*
 * Problem shape and tensor layout.
 *
 * Layout: q is [N, Hq, d]; k and v are [N, Hkv, d]; out is [N, Hq, d]; element
 * (t, h, :) of q starts at q + t*q_stride_tok + h*q_stride_head (strides in
 * ELEMENTS), and the d values are contiguous. k and v share kv_* strides.
 *
 * Constraints (else SPAVA_ERR_SHAPE):
 *   N >= 1, H >= 1, N % H == 0; block length n_b = N / H.      [contiguous blocks]
 *   Hq >= 1, Hkv >= 1, Hq % Hkv == 0; G = Hq / Hkv; query head hq reads KV head
 *   hq / G.
 *   head_dim in {64, 128}.
 *   0 <= anchor_len A <= n_b          (the anchor, tokens [0, A), lies in block 0)
 *   passing_len l >= 0                (block j passes l_j = min(l, |C_j|) rows, where
 *                                      C_0 = [A, n_b) and C_j = block j for j >= 1)
 *   1 <= window w <= n_b              (observer queries: the last w of each block)
 *   sm_scale: logit scale; <= 0 selects 1/sqrt(head_dim).
 *   Offsets are 64-bit; the limits are those of the launches: Hq, Hkv <= 65535 and
 *   every kernel grid below 2^31 work items, which for the attention means
 *   N * Hq < 2^30 (e.g. 16M tokens x 32 heads), and for the selection
 *   (H-1) * Hkv * ceil(G*w/32) * S * 64 < 2^31, S = ceil(n_b / split) key splits of
 *   the row statistics (split between 512 and 4096 keys, chosen per shape).
 *   kv_stride_tok <= 17043519 elements: attention reads K tiles in place through
 *   32-bit buffer offsets (63 token strides plus one row below 2^31 bytes).
 * Alignment (else SPAVA_ERR_ALIGN): tensor pointers 16-byte aligned; strides a
 * multiple of 8 elements (bf16) or 4 elements (f32).
 * Options (else SPAVA_ERR_OPTION): schedule is a spava_schedule, select_logits a
 * spava_select_logits. A zero-initialised struct selects the defaults.
 */
typedef struct {
  int64_t seq_len;          /* N                                  */
  int32_t num_hosts;        /* H (virtual hosts = context blocks) */
  int32_t num_q_heads;      /* Hq                                 */
  int32_t num_kv_heads;     /* Hkv                                */
  int32_t head_dim;         /* d                                  */
  int32_t anchor_len;       /* A                                  */
  int32_t passing_len;      /* l                                  */
  int32_t window;           /* w                                  */
  int32_t dtype;            /* spava_dtype of q, k, v and out     */
  double sm_scale;
  int64_t q_stride_tok, q_stride_head;
  int64_t kv_stride_tok, kv_stride_head;
  int64_t o_stride_tok, o_stride_head;
  int32_t schedule;         /* spava_schedule (0 = longest first) */
  int32_t select_logits;    /* spava_select_logits (0 = auto)     */
} spava_shape;

/* Human-readable name of a status code (static string, never NULL). */
const char* spava_status_string(int status);

/* ABI version of this header: 2 (version 1 had no schedule / select_logits fields). */
int spava_abi_version(void);

/* Host-only check of a shape (no HIP call). SPAVA_OK or the error it would raise. */
spava_status spava_validate_shape(const spava_shape* shape);

/* Bytes of workspace spava_select_passing needs for this shape (host only). */
spava_status spava_select_workspace_bytes(const spava_shape* shape, size_t* bytes);

/* Bytes of workspace spava_approx_attn_fwd needs for this shape (host only). */
spava_status spava_attn_workspace_bytes(const spava_shape* shape, size_t* bytes);

/*
 * Passing-block selection ("Passing Blocks": each block forwards its most
 * essential KV rows, identified by query-to-context attention scores).
 *
 * For every block j in [0, H-2] and KV head g, the score of key p of block j is
 * the mean over the G query heads of group g and the last w queries i of block j
 * of softmax_p(sm_scale * <q_i, k_p>), the softmax taken over the block's own keys
 * [s_j, i] (causal, inclusive). Scores are computed in float64. Block j passes the
 * l_j candidates with the largest scores; equal scores go to the lower position.
 * The last block's selection is never used and is not computed.
 *
 *   q, k         device, dtype per shape, layout above (read only)
 *   passing_idx  device int32 [max(H-1,0), Hkv, l] (written): for each (j, g) the
 *                selected positions (absolute token indices) in ascending order,
 *                then -1 up to l entries
 *   scores_out   device float64 [H-1, Hkv, n_b] (written) or NULL: the score of every
 *                key of block j (index p - j*n_b), anchor keys included
 *   workspace    device, >= spava_select_workspace_bytes bytes (contents scratch)
 * With H == 1 or l == 0 nothing but the -1 fill (if any) is enqueued.
 */
spava_status spava_select_passing(const spava_shape* shape, const void* q, const void* k,
                                  int32_t* passing_idx, double* scores_out,
                                  void* workspace, size_t workspace_bytes, void* stream);

/*
 * Approximate attention ("Berechnung": attention over the anchor, the aggregated
 * passing blocks and the local context).
 *
 * For query position i in block h and query head hq (KV head g = hq / G) the
 * visible keys are: for h >= 1 the anchor [0, A), then the passing rows of blocks
 * 0..h-1 for head g (in block order); then the local keys [h*n_b, i].
 *   out[i, hq, :] = sum_p softmax_p(sm_scale * <q_i, k_p>) v_p over that set
 *   lse_out[hq, i] = log sum_p exp(sm_scale * <q_i, k_p>)   (natural log)
 * bf16 inputs use bf16 matrix cores with float32 accumulation and softmax: the
 * softmax weights enter the P V product rounded to bf16, O is divided by the sum of
 * those rounded weights and lse_out uses the sum of the float32 weights; `out` is
 * rounded to bf16 (nearest even). f32 inputs compute logits, softmax sums and O in
 * float64 (exponentials in float32) and round `out` to float32.
 *
 *   q, k, v      device, dtype per shape (read only)
 *   passing_idx  device int32 [max(H-1,0), Hkv, l] as written by
 *                spava_select_passing (read only). Block j's entries must lie in
 *                block j's candidates; an entry outside them is read as a zero row
 *                (never out of bounds).
 *   out          device [N, Hq, d] via o_* strides, dtype per shape (written)
 *   lse_out      device float32 [Hq, N] (written) or NULL. With NULL (bf16) the
 *                kernel skips the float32 weight sum (3-5% faster); O is the same up
 *                to rounding (the running reference may be raised at another tile).
 *   workspace    device, >= spava_attn_workspace_bytes bytes (contents scratch)
 */
spava_status spava_approx_attn_fwd(const spava_shape* shape, const void* q, const void* k,
                                   const void* v, const int32_t* passing_idx, void* out,
                                   float* lse_out, void* workspace, size_t workspace_bytes,
                                   void* stream);

/* Bytes of workspace spava_select_passing_query needs (host only). */
spava_status spava_select_query_workspace_bytes(const spava_shape* shape, int64_t n_query,
                                                size_t* bytes);

/*
 * Query-aware passing-block selection (a variant of spava_select_passing; explainer
 * "APB-V: ...", Methodik > Passing Blocks: KV rows ranked by query-to-context
 * attention scores). The observers are the n_query rows of the query block q_qr
 * (all G query heads of each KV group) instead of each block's last w queries; the
 * query block follows the whole context, so every key of block j is visible:
 *   score_j,g(p) = mean over hq in g and rows i of q_qr of
 *                  softmax over p' in block j of (sm_scale * <q_qr_i, k_p'>), at p.
 * Selection, output layout, tie rule and errors are those of spava_select_passing;
 * `window` is not used. q_qr is [n_query, Hq, d] with the shape's q strides;
 * 1 <= n_query and n_query * G <= 2^30.
 */
spava_status spava_select_passing_query(const spava_shape* shape, int64_t n_query,
                                        const void* q_qr, const void* k, int32_t* passing_idx,
                                        double* scores_out, void* workspace,
                                        size_t workspace_bytes, void* stream);

/* Bytes of workspace spava_query_attn_fwd needs for n_query query rows (host only). */
spava_status spava_query_workspace_bytes(const spava_shape* shape, int64_t n_query,
                                         size_t* bytes);

/*
 * Query block B_qr (explainer "APB-V: ...", Methodik > Kontext-Splitting: the input is
 * split into anchor, query block and context blocks; Systemseitige Optimierungen >
 * fused context + query forward: each host attends the query rows to what it holds
 * and the partial results are merged with their log-sum-exp).
 *
 * The n_query rows of B_qr follow the N context tokens. Row i attends to every
 * context key [0, N) and to the query keys [0, i]:
 *   out_qr[i, hq, :] = sum_p softmax_p(sm_scale * <q_qr_i, k_p>) v_p over that set
 *   lse_qr[hq, i]    = log sum_p exp(sm_scale * <q_qr_i, k_p>)      (natural log)
 * computed as H + 1 partials over disjoint key sets (each context block, then the
 * query block itself) merged by log-sum-exp, which is exact.
 *
 *   shape        the context's shape; its q/kv/o strides also describe q_qr, k_qr,
 *                v_qr and out_qr. anchor_len, passing_len and window are not used.
 *   n_query      1 <= n_query <= 2^30
 *   q_qr         device [n_query, Hq, d]; k_qr, v_qr device [n_query, Hkv, d]
 *   k, v         device context [N, Hkv, d]
 *   out_qr       device [n_query, Hq, d], dtype per shape (written)
 *   lse_qr       device float32 [Hq, n_query] (written) or NULL
 *   workspace    device, >= spava_query_workspace_bytes bytes (contents scratch)
 */
spava_status spava_query_attn_fwd(const spava_shape* shape, int64_t n_query, const void* q_qr,
                                  const void* k_qr, const void* v_qr, const void* k,
                                  const void* v, void* out_qr, float* lse_qr, void* workspace,
                                  size_t workspace_bytes, void* stream);

/* Bytes of workspace spava_layer_overlap_fwd needs (host only). */
spava_status spava_layer_overlap_workspace_bytes(const spava_shape* shape, size_t* bytes);

/*
 * One prefill layer with the selection overlapped ("Systemseitige Optimierungen" of
 * the explainer "APB-V: ...": passing blocks are transferred while attention computes;
 * on one GPU the transfer is the selection, and the work that needs no passing rows is
 * block 0's attention, whose queries see only their own causal keys).
 *
 * Computes exactly what spava_select_passing followed by spava_approx_attn_fwd
 * compute, bitwise:
 *   on side_stream  the selection (passing_idx, scores_out);
 *   on stream       concurrently, the gather of the anchor tiles and of every block's
 *                   local values and block 0's attention; then, after the side stream,
 *                   the gather of the passing rows and the other blocks' attention.
 *
 *   q, k, v, passing_idx, scores_out, out, lse_out   as in the two calls above
 *   workspace     device, >= spava_layer_overlap_workspace_bytes bytes (the selection's
 *                 and the attention's workspaces)
 *   stream        hipStream_t the call is ordered on; every result is ready once it
 *                 reaches this point
 *   side_stream   a second hipStream_t (NULL = the default stream). It first waits for
 *                 work already enqueued on `stream`, so inputs produced there are safe;
 *                 `stream` waits for it before the blocks that need passing rows. Using
 *                 the same stream twice is correct but overlaps nothing.
 * The call synchronises the two streams with two HIP events that the library creates
 * once per calling thread and device and keeps for the life of the process.
 * bf16 only (SPAVA_ERR_DTYPE for f32). With H == 1 or l == 0 nothing needs selecting
 * and the plain attention runs on `stream`.
 */
spava_status spava_layer_overlap_fwd(const spava_shape* shape, const void* q, const void* k,
                                     const void* v, int32_t* passing_idx, double* scores_out,
                                     void* out, float* lse_out, void* workspace,
                                     size_t workspace_bytes, void* stream, void* side_stream);

/*
 * Allocation-free selection, for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid allocation.
 *
 * Computes exactly what spava_select_passing computes (same kernels; the float64
 * logits are recomputed rather than stored, which gives bitwise the same scores and
 * indices), but takes no workspace: its scratch (row statistics and, when scores_out
 * is NULL, the scores) lives in a fixed array of SPAVA_NOALLOC_SCRATCH_BYTES bytes
 * inside the library, one per GPU, held until the process ends. The array's device
 * address is looked up once per device on the first call there; nothing is allocated
 * or freed, ever.
 *
 *   shape, q, k, passing_idx, scores_out   as in spava_select_passing
 *                                          (shape->select_logits is ignored)
 *   stream   hipStream_t (NULL = the default stream)
 *
 * SPAVA_ERR_WORKSPACE when the shape needs more scratch than the array holds (the
 * selection workspace of the same shape with SPAVA_LOGITS_RECOMPUTE, which
 * spava_select_workspace_bytes reports; 23.4 MiB for 262144 tokens in 16 blocks with
 * 8 KV heads, G = 4 and w = 128). Nothing in the array needs to start at any value:
 * every byte a call reads it first writes. All calls on one GPU share the array, so
 * calls that overlap on one GPU (concurrent streams, or threads) race and must be
 * ordered by the caller; calls on different GPUs do not interact.
 */
#define SPAVA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

spava_status spava_select_passing_noalloc(const spava_shape* shape, const void* q,
                                          const void* k, int32_t* passing_idx,
                                          double* scores_out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SPAVA_H */
