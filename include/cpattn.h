/*
 * libcpattn -- context-parallel (ring) attention for one rank's share, on
 * AMD Instinct MI355X (gfx950).  Plain C ABI: host or device pointers and
 * sizes only; no HIP, torch or C++ types cross it (streams are void*).
 *
 * The method ("序列与上下文并行", section 上下文并行：注意力本身切分): the
 * sequence is cut into segments, one per rank.  Rank i keeps its own Q
 * segment and meets every rank's K/V segment in ring order j = i, i+1, ...
 * (mod N); each meeting yields a partial attention result that is folded into
 * the running result by online softmax.  Causal work is balanced by a
 * Z-shaped (zigzag) chunk assignment, and every rank knows the global
 * position of each of its tokens (same page, section 工程实践).  Attention
 * itself is softmax(Q K^T / sqrt(D) + mask) V ("Tensor并行与算子拆分",
 * section 注意力的并行化优化).  On one GPU the ranks are index ranges.
 *
 * Conventions shared by every call:
 *  - Tensors are dense, row-major and contiguous.  Per-head data is
 *    [B, H, rows, D] with D fastest; "rank-major" data is [N, B, H, L/N, D].
 *  - Element types: cpa_dtype for Q/K/V; O and lse are always float32.
 *  - Device pointers must be 16-byte aligned (offset tables 8-byte aligned).
 *  - Size limits (CPA_ESHAPE beyond them): B*H <= 65535; at most 2^30 rows
 *    per query or key block; and a matrix-core launch (bf16, D = 64 or 128)
 *    stays under 2^32 work-items: ceil(rows / 128) * B*H * 256 for the
 *    forward and dQ passes, nblk * ceil(key rows / 128) * B*H * 512 for the
 *    dK/dV pass of a ring over nblk blocks.
 *  - Ownership: the caller allocates and frees every buffer; the library
 *    keeps no pointer after a call returns and never allocates device memory.
 *  - Execution: every device call only enqueues work on `stream` (a
 *    hipStream_t, or NULL for the default stream) and returns; nothing
 *    synchronises.  A buffer may be reused once the stream has passed it.
 *  - Errors: every call checks its arguments on the host before any launch
 *    and returns a cpa_status; on failure nothing was enqueued (CPA_EHIP: the
 *    launch itself failed) and cpa_last_error() explains.  No C++ exception
 *    crosses this boundary.
 *  - Thread safety: calls may be made from several host threads; the error
 *    text is per thread.
 */
#ifndef CPATTN_H
#define CPATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  CPA_OK = 0,
  CPA_EINVAL = 1,       /* null pointer, bad rank index, misalignment, bad flag */
  CPA_ESHAPE = 2,       /* sizes that do not fit the method (e.g. L % 2N != 0) */
  CPA_EDTYPE = 3,       /* unknown element type / element size */
  CPA_EUNSUPPORTED = 4, /* valid but not built (head_dim outside {16, 64, 128}) */
  CPA_EHIP = 5          /* the HIP runtime reported an error while launching */
} cpa_status;

typedef enum { CPA_BF16 = 0, CPA_F32 = 1 } cpa_dtype;

/*
 * Zigzag layout (host only; no GPU needed).
 * Z-shaped assignment of "序列与上下文并行" (上下文并行, 工程实践), read as:
 * the L tokens form 2N chunks of C = L/(2N); rank r holds chunk r and chunk
 * 2N-1-r, so every rank gets the same causal work (2N C^2 + C key/query
 * pairs per head).
 *   L    total sequence length, > 0, divisible by 2N
 *   N    number of (virtual) ranks, >= 1
 *   out  host int64 [N, L/N]: out[r*(L/N) + t] = global position of rank r's
 *        t-th local token (chunk r ascending, then chunk 2N-1-r ascending).
 * Returns CPA_ESHAPE for L <= 0 or L % 2N != 0, CPA_EINVAL for N < 1 or a
 * null `out`.
 */
cpa_status cpa_zigzag_layout(int64_t L, int32_t N, int64_t *out);

/*
 * Partial attention of one ring step: Q_i against (K_j, V_j)
 * ("序列与上下文并行", 上下文并行: each step gives a partial result for the
 * local queries).
 *   Q      device [B, H, Lq, D] of `dt`
 *   K, V   device [B, H, Lk, D] of `dt`
 *   q_off  device int64 [Lq], k_off device int64 [Lk]: global token
 *          positions (precondition: strictly increasing; the kernel classifies
 *          whole tiles from their first and last entries)
 *   causal nonzero: key u is visible to query t iff k_off[u] <= q_off[t]
 *   scale  score scale; <= 0 selects 1/sqrt(D)
 *   O      device float32 [B, H, Lq, D]  (written)
 *   lse    device float32 [B, H, Lq]     (written): natural-log sum of
 *          exp(scaled scores) over the visible keys
 * A query with no visible key gets O = 0 and lse = -inf.  D must be 16, 64 or
 * 128 (CPA_EUNSUPPORTED otherwise).  bf16 inputs are multiplied on the
 * matrix cores with float32 accumulation; softmax is float32.
 */
cpa_status cpa_partial(const void *Q, const void *K, const void *V, cpa_dtype dt,
                       int32_t B, int32_t H, int64_t Lq, int64_t Lk, int32_t D,
                       const int64_t *q_off, const int64_t *k_off, int32_t causal,
                       float scale, float *O, float *lse, void *stream);

/*
 * Online-softmax merge, in place ("序列与上下文并行", 上下文并行: partial
 * results are folded together incrementally by online softmax):
 *   lse = ln(e^lse_acc + e^lse_new),
 *   O   = O_acc e^(lse_acc - lse) + O_new e^(lse_new - lse).
 * An empty side (lse = -inf) has weight 0; two empty sides give (0, -inf).
 *   O_acc, lse_acc  device float32 [rows, D] / [rows], read and written
 *   O_new, lse_new  device float32 [rows, D] / [rows], read only
 *   rows            number of query rows (B*H*Lq), >= 0; D in {16, 64, 128}
 */
cpa_status cpa_merge(float *O_acc, float *lse_acc, const float *O_new,
                     const float *lse_new, int64_t rows, int32_t D, void *stream);

/*
 * Workspace bytes cpa_rank_forward needs: one partial (O, lse) in float32,
 * B*H*(L/N)*(D+1)*4 bytes rounded up to 256.  Returns 0 for invalid sizes.
 */
size_t cpa_rank_forward_workspace(int32_t B, int32_t H, int64_t L, int32_t N, int32_t D);

/*
 * Whole ring for virtual rank i ("序列与上下文并行", 上下文并行): for
 * s = 0 .. N-1, j = (i + s) mod N, the partial of Q_i against (K_j, V_j);
 * step 0 writes (O_i, lse_i) directly, later steps go to the workspace and
 * are merged in.  Enqueues N partials and N-1 merges on `stream`.
 *   i, N          rank index 0 <= i < N
 *   Q_i           device [B, H, L/N, D] of `dt` (rank i's tokens, rank order)
 *   K_all, V_all  device rank-major [N, B, H, L/N, D] of `dt`
 *   pos_all       device int64 [N, L/N], e.g. cpa_zigzag_layout's table
 *   O_i, lse_i    device float32 [B, H, L/N, D] / [B, H, L/N] (written)
 *   ws, ws_bytes  device workspace of at least cpa_rank_forward_workspace()
 *                 bytes (CPA_EINVAL if smaller); unused when N == 1
 */
cpa_status cpa_rank_forward(int32_t i, int32_t N, const void *Q_i, const void *K_all,
                            const void *V_all, const int64_t *pos_all, cpa_dtype dt,
                            int32_t B, int32_t H, int64_t L, int32_t D, int32_t causal,
                            float scale, float *O_i, float *lse_i, void *ws,
                            size_t ws_bytes, void *stream);

/*
 * cpa_rank_forward without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  The partial of each ring step goes to a
 * 16 MiB scratch array inside the library, one per GPU, held until the
 * process ends; the rank's rows are worked in slices that fit it (whole heads
 * when a head's partial fits, else row ranges of one head), so no size is
 * refused for its sake.  The call itself allocates nothing.  Arguments,
 * results and errors as for cpa_rank_forward; N == 1 uses no scratch.  Every
 * call on one GPU shares that GPU's scratch: calls that can overlap on one
 * GPU (different streams without ordering) race and must be serialised by
 * the caller.  The scratch is written before it is read in every call, so
 * nothing carries over from one call to the next.
 */
cpa_status cpa_rank_forward_noalloc(int32_t i, int32_t N, const void *Q_i, const void *K_all,
                                    const void *V_all, const int64_t *pos_all, cpa_dtype dt,
                                    int32_t B, int32_t H, int64_t L, int32_t D, int32_t causal,
                                    float scale, float *O_i, float *lse_i, void *stream);

/*
 * Rank i's whole ring in ONE launch: the same result as cpa_rank_forward (up
 * to rounding order), but the kernel walks the N K/V blocks itself and keeps
 * the online-softmax state (O, running max, sums) in registers from one block
 * to the next ("序列与上下文并行", 上下文并行: the partial results are folded
 * incrementally), so no partial O is written and no merge pass runs.  The
 * blocks are visited as j = i+1, i+2, ..., i+N-1, i (mod N): the rank's own
 * block comes last, which keeps the workgroups of a head in step through the
 * other blocks (better L2 reuse); the result does not depend on the order
 * beyond rounding.  Arguments as for cpa_rank_forward, without workspace.
 * bf16 with D = 64 or 128 only (CPA_EUNSUPPORTED otherwise; use
 * cpa_rank_forward for fp32 or D = 16).
 */
cpa_status cpa_rank_forward_fused(int32_t i, int32_t N, const void *Q_i, const void *K_all,
                                  const void *V_all, const int64_t *pos_all, cpa_dtype dt,
                                  int32_t B, int32_t H, int64_t L, int32_t D, int32_t causal,
                                  float scale, float *O_i, float *lse_i, void *stream);

/*
 * The ranks' rings directly on global-order data: cpa_rank_forward_fused for
 * each rank r in [rank_lo, rank_hi), with the zigzag permute folded into the
 * kernel's addressing (rank r's local row u is global row zig(r, u): chunk r
 * for u < C, chunk 2N-1-r after, C = L/(2N)), so Q, K, V are read and O, lse
 * written in global token order without separate permute passes ("序列与上下文
 * 并行", 上下文并行 and 工程实践: the Z-shaped assignment, global positions).
 * A token's position is its global index, so the causal bounds are the
 * zigzag closed form; no position table is taken, and no table can disagree
 * with the addressing.
 *   Q, K, V    device [B, H, L, D] bf16, global order
 *   O, lse     device float32 [B, H, L, D] / [B, H, L]: the selected ranks'
 *              rows are written, the others are left untouched
 *   causal, scale   as for cpa_partial
 * bf16 with D = 64 or 128 and C a multiple of 32 (CPA_EUNSUPPORTED otherwise;
 * use the permute + cpa_rank_forward_fused path).  One launch for all the
 * selected ranks.
 */
cpa_status cpa_share_forward(const void *Q, const void *K, const void *V, cpa_dtype dt, int32_t B,
                             int32_t H, int64_t L, int32_t D, int32_t N, int32_t rank_lo,
                             int32_t rank_hi, int32_t causal, float scale, float *O, float *lse,
                             void *stream);

/*
 * cpa_share_forward with precise weights, for inputs whose V rows differ
 * widely in size.  The softmax weights multiply V in the output sum
 * ("Tensor并行与算子拆分", 注意力的并行化优化); cpa_share_forward rounds them to
 * bf16 first, which bounds O's error by V's largest rows times the bf16
 * rounding.  Here each weight p is split into hi = bf16(p) and
 * lo = bf16(p - hi), both multiply V on the matrix cores, and O is divided
 * by the fp32 sum of the weights: O's error no longer grows with V's scale.
 * The matrix cores do 24 instead of 18 products per tile (D = 128), so the
 * launch takes longer.  Arguments, layout, outputs and errors as for
 * cpa_share_forward.
 */
cpa_status cpa_share_forward_precise(const void *Q, const void *K, const void *V, cpa_dtype dt,
                                     int32_t B, int32_t H, int64_t L, int32_t D, int32_t N,
                                     int32_t rank_lo, int32_t rank_hi, int32_t causal,
                                     float scale, float *O, float *lse, void *stream);

/*
 * Permutation between global order and rank-major zigzag order, for ranks
 * [rank_lo, rank_hi) (the data-pipeline step of "序列与上下文并行", 工程实践:
 * each rank's data must follow the CP layout).
 *   forward (inverse == 0): dst[r - rank_lo, b, h, t, :] = src[b, h, pos_all[r, t], :]
 *   inverse (inverse != 0): dst[b, h, pos_all[r, t], :] = src[r - rank_lo, b, h, t, :]
 *   src, dst     device, elements of `elem_bytes` (2, 4 or 8); row = D elements
 *   B, H, L, D   global shape [B, H, L, D]; D >= 1 (D = 1 for lse)
 *   pos_all      device int64 [N, L/N]; every entry in [0, L)
 *   rank_lo/hi   0 <= rank_lo < rank_hi <= N
 * Rows of dst not named by the selected ranks are left untouched (inverse).
 * A pure copy: bit-exact.  Row bytes D*elem_bytes must be a multiple of 4.
 */
cpa_status cpa_zigzag_permute(const void *src, void *dst, int32_t elem_bytes,
                              int32_t B, int32_t H, int64_t L, int32_t D,
                              const int64_t *pos_all, int32_t N, int32_t rank_lo,
                              int32_t rank_hi, int32_t inverse, void *stream);

/*
 * Backward.  The pages give no backward; context parallelism serves training
 * ("序列与上下文并行", 工程实践: CP is validated by comparing training losses),
 * so the gradients of O = softmax(Q K^T * scale + mask) V are provided.  For
 * an upstream gradient dO, with P = exp(scores - lse) on visible pairs:
 *   delta_t = sum_d dO[t, d] O[t, d],   dS = P * (dO V^T - delta),
 *   dQ = scale dS K,   dK = scale dS^T Q,   dV = P^T dO.
 * Under CP these hold block by block when lse and delta are the query rows'
 * FINAL values (over every key they see), so a ring step needs only the
 * rank's (Q, dO, lse, delta) and the block's (K, V).  Gradients are float32;
 * bf16 inputs use the matrix cores with P and dS rounded to bf16.
 */

/*
 * delta [rows] = sum over d of dO * O, the per-row term of the softmax
 * derivative, computed once per rank before its ring steps.
 *   O      device float32 [rows, D] (the forward's output)
 *   dO     device [rows, D] of `dt`
 *   delta  device float32 [rows] (written)
 * D in {16, 64, 128}.
 */
cpa_status cpa_backward_delta(const float *O, const void *dO, cpa_dtype dt, int64_t rows,
                              int32_t D, float *delta, void *stream);

/*
 * One ring step of the backward: the gradient contributions of Q_i against
 * (K_j, V_j), ADDED into dQ, dK and dV (so steps accumulate).
 *   Q, dO         device [B, H, Lq, D] of `dt`;  K, V device [B, H, Lk, D] of `dt`
 *   lse, delta    device float32 [B, H, Lq]: the query rows' final values
 *                 (a row with lse = -inf contributes nothing)
 *   q_off, k_off, causal, scale   as for cpa_partial
 *   dQ            device float32 [B, H, Lq, D] (read and written)
 *   dK, dV        device float32 [B, H, Lk, D] (read and written)
 * D in {16, 64, 128}; bf16 with D = 64 or 128 runs on the matrix cores.
 */
cpa_status cpa_partial_backward(const void *Q, const void *K, const void *V, const void *dO,
                                const float *lse, const float *delta, cpa_dtype dt, int32_t B,
                                int32_t H, int64_t Lq, int64_t Lk, int32_t D,
                                const int64_t *q_off, const int64_t *k_off, int32_t causal,
                                float scale, float *dQ, float *dK, float *dV, void *stream);

/*
 * Rank i's ring backward: delta_i from (O_i, dO_i), then every K/V block in
 * the forward's fused order.  dQ_i is WRITTEN (all blocks summed); rank i's
 * contributions to every block's gradient are ADDED into dK_all / dV_all
 * (zero them before the first rank; after all N ranks they hold the full
 * dK, dV in rank-major order).  bf16 with D = 64 or 128 takes two launches
 * besides delta (one for dQ over the whole ring, one for every block's dK/dV).
 *   i, N, Q_i, K_all, V_all, pos_all, dt, B, H, L, D, causal, scale
 *                 as for cpa_rank_forward
 *   O_i, lse_i    device float32 [B, H, L/N, D] / [B, H, L/N]: rank i's forward
 *   dO_i          device [B, H, L/N, D] of `dt`
 *   dQ_i          device float32 [B, H, L/N, D] (written)
 *   dK_all, dV_all device float32 rank-major [N, B, H, L/N, D] (read and written)
 *   delta_i       device float32 [B, H, L/N] (written; kept for reuse)
 */
cpa_status cpa_rank_backward(int32_t i, int32_t N, const void *Q_i, const void *K_all,
                             const void *V_all, const int64_t *pos_all, const float *O_i,
                             const void *dO_i, const float *lse_i, cpa_dtype dt, int32_t B,
                             int32_t H, int64_t L, int32_t D, int32_t causal, float scale,
                             float *dQ_i, float *dK_all, float *dV_all, float *delta_i,
                             void *stream);

/*
 * The ranks' ring backward directly on global-order data: cpa_rank_backward
 * for each rank r in [rank_lo, rank_hi), with the zigzag permute folded into
 * the kernels' addressing as in cpa_share_forward (rank r's local row u is
 * global row zig(r, u), and a token's position is its global index), so no
 * tensor is permuted before or after and no position table is taken.
 *   Q, K, V, dO   device [B, H, L, D] bf16, global order
 *   O, lse        device float32 [B, H, L, D] / [B, H, L]: the forward's
 *                 output in global order (cpa_share_forward)
 *   dQ            device float32 [B, H, L, D]: the selected ranks' rows are
 *                 WRITTEN, the others are left untouched
 *   dK, dV        device float32 [B, H, L, D]: the selected ranks'
 *                 contributions are ADDED (zero them first; after all N ranks
 *                 they hold the full dK, dV in global order)
 *   delta         device float32 [B, H, L]: the selected ranks' rows are
 *                 written (workspace, kept for reuse)
 *   causal, scale as for cpa_partial
 * bf16 with D = 64 or 128 and L/(2N) a multiple of 32 (CPA_EUNSUPPORTED
 * otherwise; use the permute + cpa_rank_backward path).  Three launches per
 * rank: delta, the dQ pass and the dK/dV pass.
 */
cpa_status cpa_share_backward(const void *Q, const void *K, const void *V, const float *O,
                              const void *dO, const float *lse, cpa_dtype dt, int32_t B,
                              int32_t H, int64_t L, int32_t D, int32_t N, int32_t rank_lo,
                              int32_t rank_hi, int32_t causal, float scale, float *dQ, float *dK,
                              float *dV, float *delta, void *stream);

/* Pairing of the elements a rotary embedding rotates together. */
typedef enum {
  CPA_ROPE_INTERLEAVED = 0, /* pairs (2k, 2k+1), as the sinusoidal table interleaves sin/cos */
  CPA_ROPE_HALF = 1         /* pairs (k, k + D/2) */
} cpa_rope_pairing;

/*
 * Rotary position embedding at GLOBAL positions ("序列与上下文并行", 工程实践:
 * after the CP split, positions are global, so each rank must know the global
 * offset of its segment).  Frequencies theta_k = base^(-2k/D), k < D/2, the
 * schedule of the sinusoidal table in "Tensor并行与算子拆分" (model code,
 * PositionalEncoding).  Pair k = (a, b) of a row at position p is rotated by
 * phi = p * theta_k:  y_a = x_a cos phi - x_b sin phi,  y_b = x_a sin phi + x_b cos phi.
 * The angle is reduced in float64 before a float32 sin/cos, so it stays
 * accurate at million-token positions; the rotation is float32 and bf16
 * results are rounded to nearest even.
 *   x, y     device [B, H, rows, D] of `dt` (y may equal x: in place)
 *   pos      device int64 [rows]: global position of each row (any order, >= 0)
 *   base     > 1 (10000 in the pages' table)
 *   pairing  cpa_rope_pairing
 * D must be a multiple of 8 in [8, 512] (CPA_EUNSUPPORTED otherwise).
 */
cpa_status cpa_rope(const void *x, void *y, cpa_dtype dt, int32_t B, int32_t H, int64_t rows,
                    int32_t D, const int64_t *pos, double base, int32_t pairing, void *stream);

/*
 * cpa_zigzag_permute (forward) with the rotary embedding folded in: one pass
 * over memory that gathers each rank's rows and rotates each at its global
 * position,
 *   dst[r - rank_lo, b, h, t, :] = rope(src[b, h, pos_all[r, t], :], pos_all[r, t]).
 * Arguments as for cpa_zigzag_permute (src global [B, H, L, D], dst rank-major
 * [rank_hi - rank_lo, B, H, L/N, D], both of `dt`; src and dst must not
 * overlap) and cpa_rope (base, pairing, D).
 */
cpa_status cpa_zigzag_permute_rope(const void *src, void *dst, cpa_dtype dt, int32_t B,
                                   int32_t H, int64_t L, int32_t D, const int64_t *pos_all,
                                   int32_t N, int32_t rank_lo, int32_t rank_hi, double base,
                                   int32_t pairing, void *stream);

/*
 * Check of the precondition on position tables (debug aid).  Under causal
 * masking the attention calls take each block's positions as strictly
 * increasing: with the zigzag
 * layout a rank's positions are its two chunks in ascending order ("序列与
 * 上下文并行", section 上下文并行：注意力本身切分, the Z-shaped assignment), and
 * the kernels classify tiles, and find a row's visible keys, from that order.
 * They do not check it; this call does, for `rows` tables of n positions each
 * (a pos_all table is rows = N, n = L/N; a q_off / k_off table is rows = 1).
 *   off        device int64 [rows, n]
 *   first_bad  device int64 [1], written by the stream: the smallest flat
 *              index i with i % n != 0 and off[i] <= off[i - 1], or rows * n
 *              when every table is strictly increasing (also when it is empty)
 * Two launches (a one-thread fill of first_bad, then the check), no memset;
 * the caller reads first_bad after synchronising the stream.
 */
cpa_status cpa_check_offsets(const int64_t *off, int64_t rows, int64_t n, int64_t *first_bad,
                             void *stream);

/* Text of the last error on the calling thread ("" if none); valid until the
 * thread's next call into the library. */
const char *cpa_last_error(void);

/* Library version, e.g. "libcpattn 0.2.0 gfx950". */
const char *cpa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* CPATTN_H */
