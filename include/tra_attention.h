/*
 * tra_attention.h -- C ABI of the entropy-radius block-sparse spatiotemporal
 * attention library for AMD Instinct MI355X (gfx950).
 *
 * The method (Token Radius Attention for Efficient Video Generation,
 * "2. Methodology" and "The TRA Pipeline"): video tokens on a (T, H, W)
 * latent grid are grouped into blocks of 64 tokens, each an 8 x 8 spatial tile
 * inside one frame (the page's tile-major layout).  A cheap probe measures,
 * per query block, the softmax entropy of block-pooled queries against all
 * block-pooled keys, and maps it to an integer radius (the page's
 * entropy -> budget -> radius chain, reduced to one linear quantiser at block
 * granularity).  Exact softmax attention is then computed for the block's
 * queries over only the key/value blocks whose Chebyshev distance in
 * (frame, tile row, tile column) is within that radius -- dynamic block-sparse
 * attention as described in "AB-Attention speeds up video diffusion
 * transformers up to 2.23x" (first paragraph), with a radius neighbourhood as
 * in "Radial Attention to Accelerate Video Generation" ("The idea behind
 * Radial Attention").
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Tensors q, k, v: DEVICE pointers, bfloat16, contiguous
 *   [heads][T][H][W][head_dim] (batch 1; fold a batch B into heads as B*heads).
 * - out: DEVICE pointer, float32, same layout.  Only real tokens are written.
 * - block must be 64 (8 x 8 tiles).  head_dim must be 64 or 128.
 *   Tiles are counted nby = ceil(H/8), nbx = ceil(W/8) per frame, nb = T*nby*nbx,
 *   block id kb = (t*nby + by)*nbx + bx; tiles on the right/bottom edge may be
 *   partial and their missing cells are not tokens (never keys, no output).
 * - Softmax scale is 1/sqrt(head_dim).
 * - Radii are integers >= 0; TRA_RADIUS_INF passed as both r_min and r_max
 *   selects the dense mode (every key block kept, probe skipped).
 * - V is multiplied on fp16 matrix cores as v 2^e_h, with one power-of-two
 *   exponent e_h per head that puts the head's largest |v| into [2^15, 2^16);
 *   the output is multiplied back by 2^-e_h.  This is exact for every finite
 *   bfloat16 within 2^30 of the head's largest |v| (smaller values round at an
 *   absolute 2^-25 of it), so any finite bfloat16 V is accepted.  Inputs must
 *   be finite.
 * - All work is enqueued on `stream`; no entry point synchronises it (except
 *   the benchmark helpers tra_time_attn and tra_profile_end).  Scratch memory
 *   comes from a library-owned stream-ordered pool (hipMallocAsync semantics)
 *   and is returned to it on `stream` before the call returns; the pool keeps
 *   freed memory for later calls until tra_release_scratch.  tra_probe can
 *   instead take a caller-owned workspace of tra_workspace_bytes bytes.
 * - The caller owns every pointer it passes; the library keeps none after the
 *   call returns.  Calls on different streams are independent.
 * - Argument errors are detected on the host before anything is enqueued and
 *   return a negative status; launch errors return TRA_ERR_HIP.  Faults inside
 *   kernels surface at the caller's next synchronisation, as usual in HIP.
 */
#ifndef TRA_ATTENTION_H
#define TRA_ATTENTION_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define TRA_RADIUS_INF 2147483647

enum tra_status {
    TRA_OK = 0,
    TRA_ERR_INVALID_ARG = -1, /* null pointer, non-positive size, r_min > r_max, negative radius */
    TRA_ERR_UNSUPPORTED = -2, /* block != 64, head_dim not in {64,128}, sizes beyond int32 indexing */
    TRA_ERR_HIP = -3,         /* a HIP call or kernel launch failed */
    TRA_ERR_NOMEM = -4,       /* scratch allocation failed */
    TRA_ERR_TOO_LARGE = -5    /* needs more than the static scratch of tra_probe_static holds */
};

/* Human-readable name of a status code (static string, never NULL). */
const char *tra_status_string(int status);

/* Library ABI version (major*100 + minor). */
int tra_version(void);

/*
 * Tile grid of a (T, H, W) token grid: writes nby, nbx, nb (any may be NULL).
 * Returns TRA_OK, or TRA_ERR_INVALID_ARG / TRA_ERR_UNSUPPORTED for bad sizes.
 */
int tra_grid(int T, int H, int W, int block, int *nby, int *nbx, int *nb);

/*
 * Row stride of the key-block index lists for radii up to r_max:
 * min(2 r_max + 1, T) * min(2 r_max + 1, nby) * min(2 r_max + 1, nbx)
 * (nb for TRA_RADIUS_INF).  Returns a negative status on bad arguments.
 */
int64_t tra_maxcnt(int T, int H, int W, int block, int r_max);

/*
 * The whole layer: probe -> radii -> key-block lists -> block-sparse
 * attention, enqueued on `stream`.
 *   q, k, v   device bf16 [heads][T][H][W][head_dim]
 *   r_min, r_max  0 <= r_min <= r_max, or both TRA_RADIUS_INF (dense mode)
 *   out       device fp32 [heads][T][H][W][head_dim]
 * Equivalent to tra_probe, then tra_mask, then tra_attn on one stream, bit for
 * bit (the fused path reads q, k and v from HBM once for the probe and the
 * key/value tile packing, and builds the attention walks straight from the
 * radii without writing the lists out).
 */
int tra_attention(const void *q, const void *k, const void *v,
                  int T, int H, int W, int heads, int head_dim, int block,
                  int r_min, int r_max, void *out, hipStream_t stream);

/*
 * Bytes of the caller-owned workspace tra_probe takes for these sizes (the
 * fp32 block means of q and k, 256-byte aligned); r_max is checked as for
 * tra_maxcnt.  Returns the size, or a negative status for invalid sizes.
 */
int64_t tra_workspace_bytes(int T, int H, int W, int heads, int head_dim, int block, int r_max);

/*
 * Probe (Token Radius Attention ..., "Insight I" and "The TRA Pipeline:
 * Entropy-to-Budget / Budget-to-Radius"), per (head, query block b):
 *   Qbar_b, Kbar_b = means of q and k over the real tokens of block b (fp32);
 *   s_bc = Qbar_b . Kbar_c / sqrt(head_dim) for all nb key blocks c (fp32);
 *   H_b = entropy of softmax_c(s_bc) in nats, h_norm_b = H_b / ln(nb)
 *         (0 when nb = 1);
 *   radius_b = clamp(r_min + floor(h_norm_b * (r_max - r_min + 1)), r_min, r_max),
 *         the floor taken on the exact product of the stored fp32 h_norm_b
 *         and the integer (r_max - r_min + 1).
 *   q, k      device bf16 [heads][T][H][W][head_dim]
 *   radius    device int32 [heads][nb]   (written)
 *   h_norm    device fp32 [heads][nb]    (written; may be NULL)
 *   ws        device workspace of tra_workspace_bytes(T,H,W,heads,head_dim,block,r_max)
 *             bytes, owned by the caller and overwritten (its content is
 *             meaningless afterwards); NULL takes library scratch instead.  A
 *             workspace must not be used by two calls that may overlap.
 * Dense mode (both radii TRA_RADIUS_INF) fills radius with TRA_RADIUS_INF and
 * h_norm with 0 (ws is not touched).
 */
int tra_probe(const void *q, const void *k, int T, int H, int W, int heads, int head_dim,
              int block, int r_min, int r_max, int32_t *radius, float *h_norm, void *ws,
              hipStream_t stream);

/*
 * tra_probe for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.  Same
 * arguments and results as tra_probe (bit for bit), but the pooled means live
 * in a static device array of tra_static_scratch_bytes() bytes (64 MiB) that
 * every GPU the library runs on holds until the process ends; the call makes
 * no allocation of any kind.  Sizes whose workspace
 * (tra_workspace_bytes) exceeds the array return TRA_ERR_TOO_LARGE before
 * anything is enqueued.  Every call on one GPU shares that GPU's array (its
 * content is left from the last call and nothing in it needs clearing: the
 * probe writes every value it reads), so calls that may overlap on one GPU --
 * on different streams or from different threads without ordering -- race.
 */
int tra_probe_static(const void *q, const void *k, int T, int H, int W, int heads, int head_dim,
                     int block, int r_min, int r_max, int32_t *radius, float *h_norm,
                     hipStream_t stream);
int64_t tra_static_scratch_bytes(void);

/*
 * Key-block lists (Token Radius Attention ..., "The TRA Pipeline: Fused CUDA
 * Kernels": radius comparison and block pruning into a regular block-sparse
 * mask), per (head, query block qb) with r = radius[h][qb] clamped to
 * [0, r_max]:
 *   list = all key blocks kb with max(|t_q - t_k|, |by_q - by_k|, |bx_q - bx_k|) <= r,
 *          in ascending kb order (always contains qb itself).
 *   radius  device int32 [heads][nb]
 *   idx     device int32 [heads][nb][maxcnt], maxcnt = tra_maxcnt(T,H,W,block,r_max);
 *           only the first cnt entries of each row are written
 *   cnt     device int32 [heads][nb]
 * r_max = TRA_RADIUS_INF gives full lists (maxcnt = nb).
 */
int tra_mask(const int32_t *radius, int T, int H, int W, int heads, int block, int r_max,
             int32_t *idx, int32_t *cnt, hipStream_t stream);

/*
 * Block-sparse attention (AB-Attention ..., first paragraph: exact attention
 * on the kept key/value blocks only), per head and real query token i of
 * block qb:
 *   out_i = sum_j softmax_j(q_i . k_j / sqrt(head_dim)) v_j over the real key
 *           tokens j of the blocks idx[h][qb][0 .. cnt[h][qb]).
 *   q, k, v  device bf16 [heads][T][H][W][head_dim]
 *   idx, cnt device int32 lists as produced by tra_mask with row stride maxcnt;
 *           both NULL selects the dense mode (every block, ascending)
 *   out      device fp32 [heads][T][H][W][head_dim]
 * List entries outside [0, nb) are skipped and cnt is clamped to [0, maxcnt];
 * any other entry counts once per occurrence, in any order (a duplicate block
 * enters the softmax twice); a query block whose list keeps no key gets zeros.
 * maxcnt must lie in [1, 2^30] when lists are given.
 * Arithmetic: q.k on bf16 matrix cores with fp32 accumulation; online softmax
 * in fp32; probabilities rounded to fp16 and multiplied with v 2^e_h (the
 * per-head power-of-two scale above) on fp16 matrix cores with fp32
 * accumulation.
 */
int tra_attn(const void *q, const void *k, const void *v, int T, int H, int W, int heads,
             int head_dim, int block, const int32_t *idx, const int32_t *cnt, int64_t maxcnt,
             void *out, hipStream_t stream);

/*
 * Token-level radius policy (Token Radius Attention for Efficient Video
 * Generation, "Insight I", "Insight II" and "The TRA Pipeline":
 * Entropy-to-Budget, Budget-to-Radius, Fused CUDA Kernels), per head:
 *   tra_token_probe (the dense warm-up), per real query token i:
 *     H_i  = entropy (natural log) of softmax_j(q_i . k_j / sqrt(head_dim)) over
 *            every real key token j of the head;
 *     b_i  = tau exp(H_i) keys, clamped to [1, N]  (N = T H W);
 *     r0_i = sqrt(b_i / (pi S(t_i))),  S(t) = sum_{t'=0}^{T-1} exp(-2 gamma |t' - t|):
 *            the base radius whose disks r0_i exp(-gamma |t' - t_i|) over the
 *            T frames have a total area of b_i tokens.
 *     entropy, r0  device fp32 [heads][T][H][W] (written; entropy may be NULL)
 *   tra_token_mask: key block K is kept for query block Q when at least
 *     min_votes real query tokens i of Q have a real key token j of K with
 *     (y_j - y_i)^2 + (x_j - x_i)^2 <= (r0_i exp(-gamma |t_j - t_i|))^2
 *     (a Euclidean disk in every frame); lists ascending.
 *     r0       device fp32 [heads][T][H][W]
 *     idx      device int32 [heads][nb][nb] (row stride nb; first cnt entries written)
 *     cnt      device int32 [heads][nb]
 *     The squared radius is formed in fp32: decisions within rounding of a
 *     lattice distance may differ from exact arithmetic.
 *   tra_token_attention: tra_token_probe, tra_token_mask, then tra_attn with
 *     those lists, on one stream (library scratch, nothing else written).
 * tau > 0 and gamma >= 0 finite; min_votes in [1, 64]; other arguments as for
 * tra_attention.  The warm-up costs a dense Q.K^T pass; the page computes it
 * once and reuses the lists across denoising steps (tra_plan / tra_attn_plan).
 */
int tra_token_probe(const void *q, const void *k, int T, int H, int W, int heads, int head_dim,
                    int block, float tau, float gamma, float *entropy, float *r0,
                    hipStream_t stream);
int tra_token_mask(const float *r0, int T, int H, int W, int heads, int block, float gamma,
                   int min_votes, int32_t *idx, int32_t *cnt, hipStream_t stream);
int tra_token_attention(const void *q, const void *k, const void *v, int T, int H, int W,
                        int heads, int head_dim, int block, float tau, float gamma,
                        int min_votes, void *out, hipStream_t stream);

/*
 * The token policy's warm-up fused into one dense attention pass (Token
 * Radius Attention ..., "The TRA Pipeline: Entropy-to-Budget" and "Fused CUDA
 * Kernels": the entropy comes from the dense warm-up attention itself).  Writes
 * the dense attention output (as tra_attn in dense mode) and, for every real
 * query token, its row's entropy and base radius exactly as tra_token_probe
 * defines them.
 *   out      device fp32 [heads][T][H][W][head_dim]
 *   entropy  device fp32 [heads][T][H][W] (may be NULL)
 *   r0       device fp32 [heads][T][H][W]
 * tau > 0 and gamma >= 0 finite.  A warm-up step is this call then
 * tra_token_mask on r0 (and tra_plan of the lists for the steps that reuse them).
 */
int tra_token_warmup(const void *q, const void *k, const void *v, int T, int H, int W, int heads,
                     int head_dim, int block, float tau, float gamma, void *out, float *entropy,
                     float *r0, hipStream_t stream);

/*
 * Sampling with inclusion-probability weighting (AB-Attention speeds up video
 * diffusion transformers up to 2.23x, second paragraph: key blocks sampled in
 * proportion to importance estimates and reweighted by inverse inclusion
 * probability, so that one pass estimates dense attention), per head and
 * query block Q:
 *   p_QK  = softmax over every key block K of Qbar_Q . Kbar_K / sqrt(head_dim)
 *           (means over real tokens; one query cluster per block);
 *   pi_QK = min(1, m p_QK), pi_QQ = 1 (the own block is always kept);
 *   K is kept iff u[h][Q][K] < pi_QK, with log-weight lw = -ln pi_QK.
 *   tra_sip_mask writes the kept blocks ascending:
 *     u       device fp32 [heads][nb][nb] uniforms in [0, 1) drawn by the caller
 *     m       expected number of blocks drawn per query block (>= 0, finite)
 *     idx, lw device int32 / fp32 [heads][nb][nb] (row stride nb; first cnt written)
 *     cnt     device int32 [heads][nb]
 *     p and pi are formed in fp32: draws within rounding of pi may differ from
 *     exact arithmetic.
 *   tra_attn_weighted is tra_attn with a log-weight per list entry (laid out
 *     like idx): every key of the entry's block enters the softmax with its
 *     logit plus lw, i.e. exp(lw) times in numerator and denominator -- the
 *     self-normalised inverse-inclusion estimate of dense attention when the
 *     lists come from tra_sip_mask.  lw = NULL is tra_attn.
 */
int tra_sip_mask(const void *q, const void *k, const float *u, int T, int H, int W, int heads,
                 int head_dim, int block, float m, int32_t *idx, int32_t *cnt, float *lw,
                 hipStream_t stream);
int tra_attn_weighted(const void *q, const void *k, const void *v, int T, int H, int W, int heads,
                      int head_dim, int block, const int32_t *idx, const int32_t *cnt,
                      const float *lw, int64_t maxcnt, void *out, hipStream_t stream);

/*
 * Plan / execute split with cross-step reuse (Token Radius Attention ...,
 * "The TRA Pipeline: Cross-Step Reuse": the sparsity decided in a warm-up step
 * is reused by the later denoising steps).  tra_plan turns key-block lists into
 * the attention walk -- the pairing of query blocks into work items
 * (neighbours whose list lengths are within a factor of two: vertical ones, or,
 * in a head where a sample of the candidate pairs shows temporal walks at least
 * 5% shorter per list entry, one tile in frames 2p and 2p + 1; the other blocks
 * re-paired by length class, so that long lists share a walk with long ones),
 * the union of each item's two lists, then the work order -- and stores it in a
 * caller-owned device buffer of tra_plan_bytes bytes; tra_attn_plan then runs the attention of new
 * q, k, v along that walk, so later steps skip the list processing.
 * tra_attn(idx, cnt) is tra_plan followed by tra_attn_plan on library scratch.
 *   plan      device buffer, tra_plan_bytes(T,H,W,heads,block,maxcnt) bytes,
 *             owned by the caller; written by tra_plan, read by tra_attn_plan.
 *             Its content is opaque; it is valid for the T, H, W, heads, block
 *             and maxcnt it was made with and must be passed back with exactly
 *             those (anything else is undefined, not detected).
 *   idx, cnt, maxcnt  as for tra_attn (maxcnt in [1, 2^30]; lists as for tra_attn).
 * tra_plan_bytes returns the size, or a negative status for invalid sizes.
 * Plans are written on `stream`; using one on another stream needs the caller's
 * own synchronisation.
 */
int64_t tra_plan_bytes(int T, int H, int W, int heads, int block, int64_t maxcnt);
int tra_plan(const int32_t *idx, const int32_t *cnt, int64_t maxcnt, int T, int H, int W,
             int heads, int block, void *plan, hipStream_t stream);
int tra_attn_plan(const void *q, const void *k, const void *v, int T, int H, int W, int heads,
                  int head_dim, int block, const void *plan, int64_t maxcnt, void *out,
                  hipStream_t stream);

/*
 * The walk plan of the radius mask's lists built straight from the radii, as
 * tra_attention builds it (Token Radius Attention ..., "The TRA Pipeline:
 * Fused CUDA Kernels" -- radius comparison and block pruning -- and
 * "Cross-Step Reuse"): no lists are written; frame by frame, vertical
 * neighbours of equal radius share a work item and the frame's other blocks
 * are paired in (radius descending, tile column, tile row) order, the items
 * listed frame after frame (grids beyond 256 tiles per frame, 1024 frames or
 * 8192 blocks per head take the same rule over the whole head); each item's
 * walk is the union of its two blocks' key boxes.  Every query
 * block meets the same key blocks in the same order as along tra_plan of
 * tra_mask's lists for these radii, so tra_attn_plan along either plan gives
 * the same results.
 *   radius    device int32 [heads][nb]; values are clamped to [0, r_max] as
 *             tra_mask clamps them.  r_max >= 0 (TRA_RADIUS_INF allowed).
 *   plan      device buffer of tra_plan_bytes(T,H,W,heads,block,maxcnt) bytes with
 *             maxcnt = tra_maxcnt(T,H,W,block,r_max); pass that maxcnt to
 *             tra_attn_plan.
 */
int tra_plan_radius(const int32_t *radius, int T, int H, int W, int heads, int block, int r_max,
                    void *plan, hipStream_t stream);

/*
 * Benchmark helper: the attention kernel alone.  Builds the walk plan of the
 * lists (idx, cnt and optional log-weights lw as for tra_attn_weighted; idx =
 * cnt = NULL is the dense mode) and packs k and v, then launches the attention
 * kernel `reps` times back to back on `stream` between one pair of HIP events,
 * waits for the second event and writes the mean milliseconds per launch to
 * *ms.  out holds the attention output (as tra_attn_weighted).  reps in
 * [1, 4096] (each launch gets its own 2 KB of work-claiming counters, zeroed
 * before the timed launches); other values return TRA_ERR_INVALID_ARG.
 * Unlike the other entry points this one synchronises (on its own event).
 */
int tra_time_attn(const void *q, const void *k, const void *v, int T, int H, int W, int heads,
                  int head_dim, int block, const int32_t *idx, const int32_t *cnt,
                  const float *lw, int64_t maxcnt, int reps, void *out, float *ms,
                  hipStream_t stream);
/* The same along a stored plan (tra_plan or tra_plan_radius, with its maxcnt);
 * plan = NULL is the dense mode. */
int tra_time_attn_plan(const void *q, const void *k, const void *v, int T, int H, int W,
                       int heads, int head_dim, int block, const void *plan, int64_t maxcnt,
                       int reps, void *out, float *ms, hipStream_t stream);

/*
 * Returns the current device's pooled scratch memory that no call holds any
 * more to the driver (the pool otherwise keeps it for later calls).  Call it
 * after the streams that used the library have been synchronised.
 */
int tra_release_scratch(void);

/*
 * Optional per-kernel timing, for benchmarks.  Between tra_profile_begin and
 * tra_profile_end every kernel this library enqueues is bracketed by a pair of
 * hipEvents recorded on its own stream (process-wide switch; do not overlap
 * with calls from other threads).  tra_profile_end synchronises those events,
 * writes the summed milliseconds ms[kind] and the launch counts
 * launches[kind] for kind < n (either pointer may be NULL), releases the
 * events and stops recording.  Kinds:
 */
enum tra_kernel_kind {
    TRA_KERNEL_PACK_POOL = 0, /* pooling of q/k and tile packing of k/v */
    TRA_KERNEL_ENTROPY = 1,   /* pooled-logit entropy -> radius */
    TRA_KERNEL_MASK = 2,      /* radius -> key-block lists */
    TRA_KERNEL_ATTN = 3,      /* block-sparse attention */
    TRA_KERNEL_FILL = 4,      /* dense-mode radius fill */
    TRA_KERNEL_ORDER = 5,     /* work order: equal-work XCD ranges, longest class first */
    TRA_KERNEL_UNION = 6,     /* walk of each work item: union of its two lists, or from the radii */
    TRA_KERNEL_TOKEN_ENTROPY = 7, /* per-token entropy and base radius (warm-up) */
    TRA_KERNEL_TOKEN_MASK = 8,    /* token-disk voting lists */
    TRA_KERNEL_SIP = 9,           /* sampled lists with inverse-inclusion weights */
    TRA_KERNEL_VMAX = 10,         /* largest |v| per head (the fp16 scale of V) */
    TRA_KERNEL_PAIR = 11,         /* pair table: which two query blocks share a work item */
    TRA_KERNEL_KINDS = 12
};
int tra_profile_begin(void);
int tra_profile_end(double *ms, int *launches, int n);

#ifdef __cplusplus
}
#endif

#endif /* TRA_ATTENTION_H */
