/*
 * wide.h -- C ABI of the masked group-mask layer library (libwide.so).
 *
 * The library executes the routed operators of one transformer layer whose
 * tokens carry binary group masks, as defined in "WIDE: Boosting Adaptive LLM
 * Inference via Token-level Dynamic Width Pruning" (arXiv 2607.28418):
 *   - mask reordering            (section 3.3, Eq. 7; Appendix B, Algorithm 1)
 *   - GEMM-MN, N-axis routing    (Figure 1; Appendix B, Algorithm 2)
 *   - GEMM-K, K-axis routing     (Appendix B, Eq. 21 and Algorithm 3)
 *   - head-group-masked attention (section 3.1, Eq. 2; Appendix B, Algorithm 4)
 * on AMD Instinct MI355X (gfx950).
 *
 * Common conventions
 *   - Every pointer argument is a DEVICE pointer owned by the caller. The
 *     library never allocates, frees or keeps caller memory; its only scratch
 *     is the workspace the caller passes in (decoding attention, the split-K
 *     GEMM paths).
 *   - bf16 tensors are raw IEEE bfloat16 bits (wide_bf16). Matrices are
 *     row-major with the given leading dimension (in elements). Weights are
 *     [out_features][in_features], so every GEMM computes C = A * B^T with
 *     A [M][K] and B [N][K] (section 3.3).
 *   - Masks are uint8, token-major [rows][groups]; any nonzero byte means the
 *     group is active for that token (class 0 of the router, section 3.1,
 *     Eq. 5).
 *   - All work is enqueued on `stream` (a hipStream_t; NULL = default stream)
 *     and is asynchronous. The library never synchronises the stream and never
 *     reads mask-derived values on the host, so the calls can be captured in a
 *     HIP graph (section 3.3 names the device-to-host sync of the naive method
 *     as its first cost).
 *   - Each call returns a wide_status. Arguments are validated on the host
 *     before anything is launched; on an error nothing is launched and no
 *     output is touched.
 *   - Floating-point products accumulate in fp32 on the MFMA units; softmax
 *     runs in fp32.
 */
#ifndef WIDE_H
#define WIDE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef uint16_t wide_bf16;     /* raw bfloat16 bits */
typedef void *wide_stream_t;    /* hipStream_t */

typedef enum {
  WIDE_OK = 0,
  WIDE_ERR_INVALID_ARG = -1,   /* null pointer, bad size, misalignment, aliasing */
  WIDE_ERR_UNSUPPORTED = -2,   /* valid request this library does not implement */
  WIDE_ERR_NO_DEVICE = -3,     /* no usable HIP device */
  WIDE_ERR_LAUNCH = -4,        /* the HIP runtime rejected a kernel launch */
  WIDE_ERR_TOO_LARGE = -5      /* needs more scratch than wide_attn_noalloc's built-in buffer */
} wide_status;

typedef enum { WIDE_DTYPE_BF16 = 0, WIDE_DTYPE_F32 = 1 } wide_dtype;

/*
 * wide_reorder -- mask reordering (section 3.3, Eq. 7; Appendix B,
 * Algorithm 1).
 *
 * For every routing column (b, g), stable-partitions the row indices so that
 * the rows whose mask byte is nonzero come first, in ascending order, followed
 * by the other rows in ascending order. The reordered mask of the page is then
 * implied: it is 1 exactly at the first counts[b][g] positions.
 *
 *   mask   [batch][rows][groups] uint8, nonzero = active.
 *   perm   out, [batch][groups][rows] int32: perm[b][g][j] is the physical row
 *          of logical row j of column (b, g).
 *   counts out, [batch][groups] int32: number of active rows of column (b, g).
 *
 * For the GEMMs the token dimension is flattened (batch = 1, rows = B*T); for
 * attention each sequence keeps its own column (batch = B, rows = Tq). With
 * B = 1 the two coincide and one call serves both.
 * Errors: WIDE_ERR_INVALID_ARG for null pointers, batch/rows/groups < 1, or
 * rows >= 2^31; WIDE_ERR_LAUNCH if the launch fails.
 */
int wide_reorder(const uint8_t *mask, int64_t batch, int64_t rows, int64_t groups,
                 int32_t *perm, int32_t *counts, wide_stream_t stream);

/*
 * wide_gemm_mn -- N-axis routed GEMM, GEMM-MN (Figure 1; Appendix B,
 * Algorithm 2).
 *
 *   C[m][n] = sum_k A[m][k] * B[n][k]   if token m keeps group g = n / G,
 *   C[m][n] is NOT written              otherwise.
 *
 *   A  [M][K] bf16, leading dim lda;  B [N][K] bf16, leading dim ldb.
 *   C  [M][N], leading dim ldc, element type c_dtype (WIDE_DTYPE_BF16: one
 *      round-to-nearest-even of the fp32 sum; WIDE_DTYPE_F32: the fp32 sum).
 *   G  group size; N must be a multiple of G.
 *   perm, counts: the output of wide_reorder(mask, 1, M, N/G, ...). Row tiles
 *      wholly past counts[g] exit at once; rows past it are neither loaded
 *      nor multiplied.
 *   mask [M][N/G]: used only when perm == NULL, which selects the
 *      matrix-vector path for M <= 4 (one decode step needs no reorder).
 * Entries of inactive (token, group) pairs are left untouched: the caller
 * zero-initialises C when it needs zeros there (Algorithm 2 takes a
 * zero-initialised C).
 * Requirements: K % 8 == 0; lda, ldb >= K and multiples of 8; ldc >= N;
 * A, B, C 16-byte aligned; C must not overlap A or B. WIDE_ERR_UNSUPPORTED
 * unless G % 16 == 0, M * lda * 2 < 2^31 (rows are gathered with 32-bit byte
 * offsets) and ldb < 2^22. A group narrower than the output tile (G < 64, or
 * a group size that is not a multiple of the tile width) is covered by tiles
 * of its own whose columns past the group are computed but not stored: still
 * exact, at G / 64 of the tile's MFMA work for G < 64.
 */
int wide_gemm_mn(const wide_bf16 *A, int64_t lda, const wide_bf16 *B, int64_t ldb,
                 void *C, int64_t ldc, int c_dtype, int64_t M, int64_t N, int64_t K,
                 int64_t G, const int32_t *perm, const int32_t *counts,
                 const uint8_t *mask, wide_stream_t stream);

/*
 * wide_gemm_mn_swiglu -- the FFN gate and up projections fused with the
 * activation (section 3.1, Eq. 3, with phi = SiLU):
 *
 *   H[m][n] = SiLU(sum_k A[m][k] Wg[n][k]) * (sum_k A[m][k] Wu[n][k])
 *   for active (m, n / G); other entries are not written.
 *
 * Both products accumulate in fp32; the activation is applied in fp32 and H
 * is rounded once to h_dtype. Wg and Wu are [N][K] with the same leading dim
 * ldb. Arguments and requirements otherwise as wide_gemm_mn.
 */
int wide_gemm_mn_swiglu(const wide_bf16 *A, int64_t lda, const wide_bf16 *Wg,
                        const wide_bf16 *Wu, int64_t ldb, void *H, int64_t ldh,
                        int h_dtype, int64_t M, int64_t N, int64_t K, int64_t G,
                        const int32_t *perm, const int32_t *counts,
                        const uint8_t *mask, wide_stream_t stream);

/*
 * wide_gemm_mn_ws, wide_gemm_mn_swiglu_ws -- wide_gemm_mn and
 * wide_gemm_mn_swiglu (Figure 1; Appendix B, Algorithm 2 and its split-K
 * variant) with a caller-owned workspace. The workgroups then derive the list
 * of active tiles from counts on the device (the host still never reads
 * them), take the tiles in that order, and when the active tiles leave a
 * last round on the compute units at most half full, every tile of that
 * round is split into slices of K computed by separate workgroups; a second
 * kernel sums the slices in slice order, applies the epilogue (SwiGLU for
 * the _swiglu form) and scatters the active rows. The page's split-K variant
 * reduces the slices with atomics; here the order is fixed, so results are
 * bitwise reproducible for a given shape, mask and device.
 *   workspace: device memory of at least wide_gemm_mn_workspace_bytes(M, N,
 *     K, G, swiglu) bytes, 16-byte aligned, overlapping no other argument.
 *     Contents on entry are ignored and overwritten; calls sharing a
 *     workspace must not run at the same time. NULL (or a size of 0 when the
 *     function returns 0) is the plain call. Ignored when perm == NULL.
 * Results: as the plain call; a split tile's fp32 sums are formed as slice 0
 * + slice 1 + ... and may round differently from a single pass over K.
 * Requirements and errors as the plain call; WIDE_ERR_INVALID_ARG when a
 * workspace is given that is smaller than needed, misaligned or overlapping.
 */
int wide_gemm_mn_ws(const wide_bf16 *A, int64_t lda, const wide_bf16 *B, int64_t ldb,
                    void *C, int64_t ldc, int c_dtype, int64_t M, int64_t N, int64_t K,
                    int64_t G, const int32_t *perm, const int32_t *counts,
                    const uint8_t *mask, void *workspace, size_t workspace_bytes,
                    wide_stream_t stream);
int wide_gemm_mn_swiglu_ws(const wide_bf16 *A, int64_t lda, const wide_bf16 *Wg,
                           const wide_bf16 *Wu, int64_t ldb, void *H, int64_t ldh,
                           int h_dtype, int64_t M, int64_t N, int64_t K, int64_t G,
                           const int32_t *perm, const int32_t *counts,
                           const uint8_t *mask, void *workspace, size_t workspace_bytes,
                           wide_stream_t stream);

/* Bytes of device workspace wide_gemm_mn_ws (swiglu = 0) or
 * wide_gemm_mn_swiglu_ws (swiglu = 1) needs on the current device: a small
 * header plus one fp32 output tile (256 or 320 rows) per compute unit (0
 * when K is too short for any split, for sizes out of range, and for the
 * fused SwiGLU over groups of a multiple of 64 but not of 128 features, whose
 * tiles run in the static order, faster there than the scheduled one). */
size_t wide_gemm_mn_workspace_bytes(int64_t M, int64_t N, int64_t K, int64_t G, int swiglu);

/*
 * wide_order_by_pattern -- a row order for GEMM-K (Appendix B, Eq. 21): the
 * stable sort of the token rows by the reflected Gray code rank of their
 * routing pattern over the first min(groups, 8) groups (group 0 the most
 * significant bit). Rows whose masks agree on those groups become adjacent,
 * and since neighbouring Gray codes differ in one group, every group's active
 * rows form few long runs: whole 16-row MFMA fragments then skip a group.
 * The order is a scheduling choice of this library; GEMM-K's result does not
 * depend on it.
 *   mask  [rows][groups] uint8, nonzero = active.
 *   order out, [rows] int32: order[j] is the token row at sorted position j;
 *         rows with equal keys keep ascending order.
 * One workgroup, no scratch memory, nothing read on the host.
 * Errors: WIDE_ERR_INVALID_ARG for null pointers, rows or groups < 1 or
 * >= 2^31, or an order that overlaps the mask.
 */
int wide_order_by_pattern(const uint8_t *mask, int64_t rows, int64_t groups, int32_t *order,
                          wide_stream_t stream);

/*
 * wide_gemm_k -- K-axis routed GEMM, GEMM-K (Appendix B, Eq. 21 and
 * Algorithm 3):
 *
 *   C[m][n] = beta * C[m][n]
 *           + sum_g mask[m][g] * sum_{k in [gG, (g+1)G)} A[m][k] * B[n][k]
 *
 *   A [M][K] bf16 (lda), B [N][K] bf16 (ldb), C [M][N] fp32 (ldc).
 *   mask [M][K/G] uint8. beta is 0 or 1. With beta = 0 every entry of C is
 *   written, exact 0 for rows with no active group.
 *   order: NULL, or a permutation of 0 .. M-1 (wide_order_by_pattern). With
 *     it, and N % 256 == 0, the output tiles cover sorted positions: A rows
 *     are gathered and C rows scattered through the order, a tile runs only
 *     the K-groups some of its rows keep, and a 16-row MFMA fragment none of
 *     whose rows keeps the current group skips its multiply-adds. The result
 *     is the same sum over the same products (the skipped work adds zeros);
 *     only a K-split tile's grouping of partial sums can differ. An entry
 *     outside [0, M) is dropped (its row is left unwritten), never
 *     dereferenced. Ignored for M <= 4 and when N % 256 != 0.
 * The page's Algorithm 3 gives every (sorted row tile of one group, K-group)
 * pair a pipeline and adds each partial into C with atomics; here a tile
 * covers all groups of its rows and keeps C in registers, and the order
 * replaces the per-group sorted rows of wide_reorder, because one order serves
 * every group without moving any partial sum.
 * The A segment of an inactive (row, group) pair is never loaded, and a tile
 * with no active pair only scales its part of C. Summation order is fixed:
 * results are bitwise reproducible run to run.
 * Requirements: K % G == 0; lda, ldb >= K and multiples of 8; ldc >= N and a
 * multiple of 4; 16-byte aligned A, B, C; C must not overlap A, B, mask or
 * order. WIDE_ERR_UNSUPPORTED unless G % 16 == 0, K / G <= 512,
 * N % 128 == 0, lda < 2^22 and ldb < 2^22. When G is not a multiple of 64 a
 * 64-deep stage spans several groups and each 16-byte chunk of an A row is
 * predicated by its own (row, group) bit; the order is then ignored.
 */
int wide_gemm_k(const wide_bf16 *A, int64_t lda, const wide_bf16 *B, int64_t ldb,
                float *C, int64_t ldc, int beta, int64_t M, int64_t N, int64_t K,
                int64_t G, const int32_t *order, const uint8_t *mask, wide_stream_t stream);

/*
 * wide_gemm_k_ws -- wide_gemm_k (the same product, Appendix B, Eq. 21) with a
 * caller-owned workspace. When the 256 x 256 output tiles leave a last round
 * on the device's compute units at most half full, each tile of that round is
 * split into slices of K computed by separate workgroups; the workspace holds
 * the partial tiles of all slices but the last, and a second kernel adds them
 * into C. Shapes whose 256 x 320 tiles fill whole rounds (N a multiple of 320,
 * G of 64) run those tiles instead, with no split, as wide_gemm_k does; so do
 * shapes whose 256 x 192 tiles fill whole rounds where 256 x 256 ones do not.
 *   workspace: device memory of at least wide_gemm_k_workspace_bytes(M, N, K)
 *     bytes, 16-byte aligned, not overlapping A, B, C, mask or order. Its
 *     contents on entry are ignored and overwritten; calls that share a
 *     workspace must not run at the same time (e.g. on two streams). NULL, or
 *     a size of 0 when the plan needs none, is wide_gemm_k.
 * Results: as wide_gemm_k, bitwise reproducible for a given shape and device.
 * A split tile's sum is C = (beta C + last slice) + slice 0 + slice 1 + ...,
 * which rounds differently from wide_gemm_k's single pass over K.
 * Requirements and errors as wide_gemm_k; WIDE_ERR_INVALID_ARG when a
 * workspace is given that is smaller than needed, misaligned or overlapping.
 */
int wide_gemm_k_ws(const wide_bf16 *A, int64_t lda, const wide_bf16 *B, int64_t ldb,
                   float *C, int64_t ldc, int beta, int64_t M, int64_t N, int64_t K,
                   int64_t G, const int32_t *order, const uint8_t *mask, void *workspace,
                   size_t workspace_bytes, wide_stream_t stream);

/* Bytes of device workspace wide_gemm_k_ws needs for an M x N x K product on
 * the current device (0: no tile is split; also 0 for sizes out of range). */
size_t wide_gemm_k_workspace_bytes(int64_t M, int64_t N, int64_t K);

/*
 * wide_gemm_k_grouped -- GEMM-K computed group by group from the reorder
 * (Appendix B, Eq. 21 and Algorithm 3): the same product as wide_gemm_k,
 *
 *   C[m][n] = beta * C[m][n]
 *           + sum_g [m among the first counts[g] rows of perm[g]]
 *                   * sum_{k in [gG, (g+1)G)} A[m][k] * B[n][k],
 *
 * with the rows that keep group g read from wide_reorder's output instead of
 * a mask. Every (group, 256 sorted rows, 256 or 128 features) tile that has
 * rows multiplies them over the group's G columns only, and adds its partial
 * tile into C with fp32 atomic adds at the gathered rows; a tile past
 * counts[g] does nothing. Work and A traffic are those of the active pairs
 * only; the cost is K/G partial writes per output row, which suits large
 * groups (the page's observation that GEMM-K needs G > 128).
 *   A [M][K] bf16 (lda), B [N][K] bf16 (ldb), C [M][N] fp32 (ldc).
 *   perm [K/G][M], counts [K/G]: wide_reorder(mask, 1, M, K/G, ...) of the
 *     [M][K/G] mask. perm entries outside [0, M) are dropped (never
 *     dereferenced); counts are clamped to M.
 *   beta 0: C is zeroed first (rows in no group end at exact 0); 1: added to.
 *   C must be ordinary device memory (hipMalloc, torch): the adds are
 *   device-scope fp32 atomics, which host-coherent memory does not take.
 * Results: the partials of different groups reach an entry of C in no fixed
 * order, so fp32 rounding can differ run to run (the sum is the same up to
 * reassociation of K/G terms).
 * Requirements: K % G == 0; lda, ldb >= K and multiples of 8; ldc >= N and a
 * multiple of 4; 16-byte aligned A, B, C; C must not overlap A, B, perm or
 * counts (WIDE_ERR_INVALID_ARG). WIDE_ERR_UNSUPPORTED unless G % 64 == 0,
 * N % 128 == 0, M * lda * 2 < 2^31 and ldb < 2^22.
 */
int wide_gemm_k_grouped(const wide_bf16 *A, int64_t lda, const wide_bf16 *B, int64_t ldb,
                        float *C, int64_t ldc, int beta, int64_t M, int64_t N, int64_t K,
                        int64_t G, const int32_t *perm, const int32_t *counts,
                        wide_stream_t stream);

/*
 * wide_attn -- head-group-masked causal GQA attention (section 3.1, Eq. 2;
 * Appendix B, Algorithm 4 and its decoding paragraph).
 *
 *   Q [B][Tq][Hq][d], K and V [B][Tk][Hk][d] bf16, contiguous.
 *   O [B][Tq][Hq][d], element type o_dtype (bf16 or fp32).
 * Query head h reads KV head g = h / (Hq/Hk) and is gated by routing group g
 * (the attention group size is (Hq/Hk)*d). For an active (b, t, g) and every
 * head h of group g:
 *   O[b][t][h] = sum_j softmax_j(scale * <Q[b][t][h], K[b][j][g]>) V[b][j][g]
 * over the valid keys j in [jmin, jmax): jmin = leftpad[b] (0 if leftpad is
 * NULL); jmax = t + (Tk - Tq) + 1 if causal (bottom-right aligned), else Tk.
 * A row with no valid key gets O = 0. Rows of inactive groups are not written.
 *   scale: softmax scale; 0 selects 1/sqrt(d).
 *   perm, counts: wide_reorder(mask, B, Tq, Hk, ...) output ([B][Hk][Tq] and
 *     [B][Hk]); required for Tq > 1.
 *   mask [B][Tq][Hk]: used when perm == NULL; then Tq must be 1 (decoding
 *     reads the routing bytes directly; no reorder runs).
 *   workspace: device scratch of at least wide_attn_workspace_bytes(...)
 *     bytes (0 bytes for Tq > 1); may be NULL when that is 0.
 * Requirements: Hq % Hk == 0; Tk >= Tq >= 1; 16-byte aligned Q, K, V, O;
 * O must not overlap Q, K or V. WIDE_ERR_UNSUPPORTED unless d == 128, one
 * sequence's Q and K each span less than 2^31 bytes, and (decoding) Hq/Hk <= 16
 * and Tk <= 262144.
 */
int wide_attn(const wide_bf16 *Q, const wide_bf16 *K, const wide_bf16 *V, void *O,
              int o_dtype, int64_t B, int64_t Tq, int64_t Tk, int64_t Hq, int64_t Hk,
              int64_t d, int causal, float scale, const int32_t *leftpad,
              const int32_t *perm, const int32_t *counts, const uint8_t *mask,
              void *workspace, size_t workspace_bytes, wide_stream_t stream);

/*
 * wide_router -- the bottleneck router of one layer and its routing decision
 * (section 3.1 "Routing Components", Eq. 4 and 5), optionally followed by the
 * mask reordering of wide_reorder, all on the device.
 *
 *   H = X W1^T (fp32), R[m][2g + c] = sum_j H[m][j] * W2[2g + c][j] (fp32,
 *   j in order), mask[m][g] = 1 (the group runs) iff R[m][2g] >= R[m][2g+1]:
 *   class 0 is the argmax, a tie included.
 *
 *   X  [batch * rows][D] bf16, leading dim ldx (ldx >= D, a multiple of 8).
 *   W1 [r][D] bf16, contiguous: the page's W1 (D x r) transposed into this
 *      library's [out][in] convention. r is 16, 32, 48 or 64.
 *   W2 [2 * groups][r] bf16, contiguous: the page's W2 (r x 2 N_G) transposed;
 *      rows 2g and 2g + 1 are the two classes of group g.
 *   mask   out [batch][rows][groups] uint8 (0 or 1), always written.
 *   logits out [batch * rows][2 * groups] fp32, or NULL.
 *   perm, counts: out, or both NULL; when given, the reorder of the mask just
 *      written, as wide_reorder(mask, batch, rows, groups, perm, counts).
 * Requirements: D % 8 == 0; 16-byte aligned X, W1, W2, logits; groups * r <=
 * 16384; (batch * rows) * ldx * 2 < 2^31; outputs overlap no input.
 */
int wide_router(const wide_bf16 *X, int64_t ldx, const wide_bf16 *W1, const wide_bf16 *W2,
                int64_t batch, int64_t rows, int64_t D, int64_t r, int64_t groups,
                uint8_t *mask, float *logits, int32_t *perm, int32_t *counts,
                wide_stream_t stream);

/*
 * wide_attn_grouped -- wide_attn with routing groups finer than the KV heads
 * (the page's sub-GQA granularity, section 3.1: G_attn = (Hq/groups) * d,
 * down to one query head per group). `groups` is a multiple of Hk that
 * divides Hq; query head h is gated by routing group h / (Hq/groups) and
 * still reads KV head h / (Hq/Hk). mask is [B][Tq][groups]; perm and counts
 * are wide_reorder(mask, B, Tq, groups, ...) output ([B][groups][Tq] and
 * [B][groups]). groups = Hk is exactly wide_attn. Other arguments, output
 * rules, requirements and errors as wide_attn; WIDE_ERR_INVALID_ARG when
 * groups is not a multiple of Hk dividing Hq.
 */
int wide_attn_grouped(const wide_bf16 *Q, const wide_bf16 *K, const wide_bf16 *V, void *O,
                      int o_dtype, int64_t B, int64_t Tq, int64_t Tk, int64_t Hq, int64_t Hk,
                      int64_t groups, int64_t d, int causal, float scale,
                      const int32_t *leftpad, const int32_t *perm, const int32_t *counts,
                      const uint8_t *mask, void *workspace, size_t workspace_bytes,
                      wide_stream_t stream);

/*
 * wide_attn_noalloc -- wide_attn for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): the same computation, arguments and results as
 * wide_attn, minus the workspace. Decoding (Tq = 1) keeps its split-KV
 * partials in a scratch array built into the library, 32 MiB per device,
 * held from the first call on a device until the process ends; prefill
 * needs no scratch. Nothing is allocated or freed by the call. The partials
 * a call reads are always written earlier in the same call, so the array
 * needs no clearing, but every call on one device shares it: calls that
 * overlap on one device (two streams) race and must be serialised by the
 * caller.
 * Errors: as wide_attn, plus WIDE_ERR_TOO_LARGE when
 * wide_attn_workspace_bytes(B, Tq, Tk, Hq, Hk, d) exceeds 32 MiB (for
 * decoding: B * Hq * ceil(Tk / 64) > 63550).
 */
int wide_attn_noalloc(const wide_bf16 *Q, const wide_bf16 *K, const wide_bf16 *V, void *O,
                      int o_dtype, int64_t B, int64_t Tq, int64_t Tk, int64_t Hq, int64_t Hk,
                      int64_t d, int causal, float scale, const int32_t *leftpad,
                      const int32_t *perm, const int32_t *counts, const uint8_t *mask,
                      wide_stream_t stream);

/* Bytes of device workspace wide_attn needs for these sizes (0 if none). */
size_t wide_attn_workspace_bytes(int64_t B, int64_t Tq, int64_t Tk, int64_t Hq,
                                 int64_t Hk, int64_t d);

/*
 * wide_mfma_probe -- a measurement, not part of the routed layer: `blocks`
 * workgroups of 4 waves each run `iters` rounds of 8 independent bf16 MFMAs
 * (16 x 16 x 32, 16384 FLOPs each) from register operands, so the elapsed
 * time gives the matrix-core rate the device sustains:
 * blocks * 4 * iters * 8 * 16384 FLOPs. sink: device float [blocks * 4],
 * written (one value per wave). Errors: WIDE_ERR_INVALID_ARG for a null sink,
 * blocks outside [1, 65535] or iters outside [1, 2^24].
 */
int wide_mfma_probe(int64_t blocks, int64_t iters, float *sink, wide_stream_t stream);

/* Static, human-readable text for a wide_status value. */
const char *wide_status_string(int status);

/* ABI version: bumped on any incompatible change of the declarations above. */
int wide_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* WIDE_H */
