/*
 * dg.h - C ABI of libdg: fine-grained-scaled FP8 GEMM for AMD MI355X (gfx950).
 *
 * What is computed (DeepGEMM project introduction, docs.beyondata.com,
 * sections Interfaces, Grouped GEMM (contiguous layout) and Grouped GEMM
 * (masked layout); "Deepseek DeepGEMM technical principles", blog.51cto.com,
 * section "Technical background and core principles"):
 *
 *   D[m][n] = bf16( sum_kb  P_kb[m][n] * (sfa[kb][m] * sfb[n/128][kb]) )
 *   P_kb[m][n] = sum_{k in slice kb} e4m3(A[m][k]) * e4m3(B[n][k])
 *
 * A is [M][K] and B is [N][K] (the "NT" layout: both K-contiguous), both
 * OCP e4m3fn bytes.  Activations carry one fp32 scale per 1x128 tile, weights
 * one per 128x128 block.  Each 128-wide K slice is a low-precision partial
 * product that is scaled and promoted into an fp32 accumulator; the output is
 * bf16 (round to nearest even).
 *
 * Entry points, in the order below: the dense NT GEMM and the two MoE grouped
 * layouts (contiguous, masked); the same with power-of-two (UE8M0) scales;
 * the forms that also quantise their output for the next layer (fp32 or
 * UE8M0 output scales); the K-axis grouped weight-gradient GEMM; the dense
 * GEMM with the NN, TN and TT operand majors (fp32 or UE8M0 scales); the
 * 1x128 and 128x128 quantisers (row-wise, column-wise for M-major
 * activations, fp32 or UE8M0 scales); host utilities.
 *
 * Conventions for every entry point
 *   - All data pointers are DEVICE pointers on the current HIP device; the
 *     caller allocates and owns every buffer (including any workspace).  The
 *     library allocates nothing per call and never synchronises the host.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream); all
 *     work is enqueued on it asynchronously.
 *   - e4m3 = uint8_t (OCP e4m3fn, max 448), bf16 = uint16_t bit patterns.
 *   - Argument errors are detected on the host before anything is launched and
 *     returned as a negative dg_status; nothing is enqueued in that case.
 *     A launch failure returns DG_ERR_HIP.  The text of the last error on the
 *     calling thread is available from dg_get_last_error_string().
 *   - The output must not alias any input.
 *   - m == 0 (or n == 0) is a successful no-op.  k == 0 writes zeros (the
 *     empty sum); then a, b, sfa and sfb are not read and may be NULL.
 *
 * Shape and alignment rules (checked; DG_ERR_* on violation)
 *   - k % 128 == 0 (DG_ERR_UNSUPPORTED_SHAPE); m, n arbitrary >= 0.
 *   - a, b, d, sfa, sfb 16-byte aligned; lda, ldb multiples of 16 (bytes =
 *     elements); ldd a multiple of 8 elements; ld_sfa a multiple of 4 and
 *     >= the rows it covers (DG_ERR_MISALIGNED / DG_ERR_INVALID_VALUE).
 *   - Each operand (per group) stays below 4 GiB, and the output holds fewer
 *     than 2^31 tiles of 64x64 (over all groups of the masked and K-grouped
 *     layouts): DG_ERR_UNSUPPORTED_SHAPE otherwise.
 */
#ifndef DG_H_
#define DG_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  DG_SUCCESS = 0,
  DG_ERR_INVALID_VALUE = -1,    /* null pointer, negative size, bad leading dim */
  DG_ERR_UNSUPPORTED_SHAPE = -2,/* k % 128 != 0, contiguous m_total % 128 != 0, too large */
  DG_ERR_MISALIGNED = -3,       /* pointer or stride not 16-byte aligned */
  DG_ERR_WORKSPACE = -4,        /* workspace smaller than dg_get_workspace_size() */
  DG_ERR_HIP = -5               /* a HIP runtime call or kernel launch failed */
} dg_status;

/* ---------------------------------------------------------------- GEMMs -- */

/*
 * Dense NT GEMM (gemm_fp8_fp8_bf16_nt; project introduction, section
 * Interfaces, "Normal dense GEMM (non-grouped)").
 *   a   [m][lda]  e4m3, row r's K values at a + r*lda
 *   sfa [k/128][ld_sfa] fp32, MN-major ("TMA-aligned and transposed" in the
 *       pages; here ld_sfa = round_up(m, 4), see dg_get_sf_leading_dim)
 *   b   [n][ldb]  e4m3
 *   sfb [ceil(n/128)][k/128] fp32 (the last row block may be partial)
 *   d   [m][ldd]  bf16 output; only columns < n of rows < m are written
 *   workspace: device scratch of at least dg_get_workspace_size(m, n, k, 1)
 *       bytes (may be NULL when that size is 0); zero-filled before its first
 *       use, see dg_get_workspace_size.
 */
int dg_fp8_gemm_nt(const uint8_t* a, const float* sfa, const uint8_t* b, const float* sfb,
                   uint16_t* d, int m, int n, int k, int64_t lda, int64_t ldb, int64_t ldd,
                   int64_t ld_sfa, void* workspace, size_t workspace_bytes, void* stream);

/*
 * dg_fp8_gemm_nt without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  Operands, output, rules and errors are
 * those of dg_fp8_gemm_nt.  The split-K partials and arrival counters live
 * in a scratch array inside the library, one per GPU, of 32 MiB + 32 KiB,
 * held until the process ends; a shape whose configuration needs more
 * (dg_get_workspace_size(m, n, k, 1) > 33587200, e.g. a 4096 x 2816 x 7168
 * GEMM, which divides the K ranges of 256 x 256 tiles) is rejected with
 * DG_ERR_WORKSPACE before anything is enqueued.  Nothing is allocated: the
 * first call on a GPU looks up that GPU's array and enqueues one small kernel
 * on `stream` that clears its counters; every call leaves them at zero.
 * All calls on one GPU share its array, so calls that may run at the same
 * time on one GPU (on different streams, or graphs launched concurrently)
 * race and must be serialised by the caller.
 */
int dg_fp8_gemm_nt_noalloc(const uint8_t* a, const float* sfa, const uint8_t* b, const float* sfb,
                           uint16_t* d, int m, int n, int k, int64_t lda, int64_t ldb, int64_t ldd,
                           int64_t ld_sfa, void* stream);

/*
 * Grouped GEMM, contiguous layout (m_grouped_gemm_fp8_fp8_bf16_nt_contiguous;
 * project introduction, section "Grouped GEMM (contiguous layout)"): the
 * tokens of all experts are concatenated along M; only M is grouped, N and K
 * are shared.
 *   a   [m_total][k] e4m3, sfa [k/128][ld_sfa] fp32 (ld_sfa >= m_total)
 *   b   [num_groups][n][k] e4m3, sfb [num_groups][ceil(n/128)][k/128] fp32
 *   d   [m_total][n] bf16
 *   m_indices [m_total] int32 (device): expert of each row.
 * Rules: m_total % 128 == 0 (each expert segment is aligned to the M block,
 * dg_get_m_alignment_for_contiguous_layout()).  A row whose index is < 0 or
 * >= num_groups is padding and is NOT written.  Within each aligned 128-row
 * block all non-padding rows must name the same expert (precondition; if it is
 * violated, rows whose index differs from the block's largest valid index are
 * left unwritten).  Nothing is read out of bounds for any index value.
 */
int dg_grouped_contiguous(const uint8_t* a, const float* sfa, const uint8_t* b,
                          const float* sfb, uint16_t* d, const int32_t* m_indices,
                          int m_total, int n, int k, int num_groups, int64_t ld_sfa,
                          void* workspace, size_t workspace_bytes, void* stream);

/*
 * Grouped GEMM, masked layout (m_grouped_gemm_fp8_fp8_bf16_nt_masked; project
 * introduction, section "Grouped GEMM (masked layout)"): used when the host
 * does not know how many tokens each expert received (graph-captured decode),
 * so the valid-row counts live on the device and only the valid part is
 * computed.
 *   a   [num_groups][m_max][k] e4m3
 *   sfa [num_groups][k/128][ld_sfa] fp32 (ld_sfa >= m_max)
 *   b   [num_groups][n][k] e4m3, sfb [num_groups][ceil(n/128)][k/128] fp32
 *   d   [num_groups][m_max][n] bf16
 *   masked_m [num_groups] int32 (device): valid rows per group, clamped to
 *       [0, m_max].  Rows >= masked_m[g] of group g are NOT written.
 *   expected_m: host hint of the typical masked_m (used only to pick tile
 *       sizes; any value >= 0 is valid, 0 = unknown).
 */
int dg_grouped_masked(const uint8_t* a, const float* sfa, const uint8_t* b, const float* sfb,
                      uint16_t* d, const int32_t* masked_m, int num_groups, int m_max, int n,
                      int k, int expected_m, int64_t ld_sfa, void* workspace,
                      size_t workspace_bytes, void* stream);

/*
 * The three GEMMs with power-of-two (UE8M0) scales.  The yfxerp.com DeepGEMM
 * article (section 3.1) gives the scale factors of the newer architecture as
 * UE8M0 - an unsigned 8-bit exponent E standing for 2^(E-127) - packed four
 * to a 32-bit word, in place of fp32.  The product is the same formula as
 * above with sfa and sfb replaced by 2^(E-127); since the scales are powers of
 * two the kernel applies them inside the block-scaled matrix instruction
 * instead of on the accumulator.  Scale layouts (bytes, MN-major for both
 * operands, four consecutive rows or column blocks per dword):
 *   sfa [k/128][ld_sfa] uint8 (masked: [num_groups][k/128][ld_sfa]);
 *       ld_sfa >= rows, a multiple of 4 (dg_get_sf_leading_dim)
 *   sfb [num_groups][k/128][ld_sfb] uint8 with
 *       ld_sfb = dg_get_ue8m0_sfb_leading_dim(n) = round_up(ceil(n/128), 4)
 * Everything else (operands, output, workspace, rules, errors) is as for the
 * fp32-scale entry point of the same layout.  Exponent 255 (NaN in E8M0) is
 * outside the contract; the quantisers below never write it.  A tile shape
 * that has no UE8M0 instance (only possible through a forced configuration)
 * returns DG_ERR_UNSUPPORTED_SHAPE.
 */
int dg_fp8_gemm_nt_ue8m0(const uint8_t* a, const uint8_t* sfa, const uint8_t* b,
                         const uint8_t* sfb, uint16_t* d, int m, int n, int k, int64_t lda,
                         int64_t ldb, int64_t ldd, int64_t ld_sfa, void* workspace,
                         size_t workspace_bytes, void* stream);
int dg_grouped_contiguous_ue8m0(const uint8_t* a, const uint8_t* sfa, const uint8_t* b,
                                const uint8_t* sfb, uint16_t* d, const int32_t* m_indices,
                                int m_total, int n, int k, int num_groups, int64_t ld_sfa,
                                void* workspace, size_t workspace_bytes, void* stream);
int dg_grouped_masked_ue8m0(const uint8_t* a, const uint8_t* sfa, const uint8_t* b,
                            const uint8_t* sfb, uint16_t* d, const int32_t* masked_m,
                            int num_groups, int m_max, int n, int k, int expected_m,
                            int64_t ld_sfa, void* workspace, size_t workspace_bytes,
                            void* stream);

/*
 * The three fp32-scale GEMMs with a quantised copy of their output, for the
 * next layer's activations: besides d, every 1x128 tile of the bf16 output
 * (a row's 128-column block) is quantised exactly as dg_quant_1x128 would
 * quantise d, in the GEMM's epilogue instead of a second launch.  The pages
 * leave FP8 casts to the caller and suggest fusing them into the kernel that
 * produces the activations (project introduction, section Interfaces, the
 * notice at its start).
 *   dq  e4m3 [rows][n] (masked: [num_groups][m_max][n]), row stride n
 *   dsf fp32 [n/128][ld_dsf] (masked: [num_groups][n/128][ld_dsf]), MN-major
 *       like sfa; ld_dsf >= rows (m, m_total or m_max), a multiple of 4
 * Rules: n % 128 == 0 (DG_ERR_UNSUPPORTED_SHAPE); dq, dsf 16-byte aligned.
 * Exactly the rows that d receives are written (padding rows of the
 * contiguous layout and rows >= masked_m[g] are left untouched in dq and
 * dsf).  Dense only: the scale padding rows [m, ld_dsf) are written as 0.
 * The tile shapes used are those whose columns are whole 128-column blocks,
 * so the configuration (and the workspace need) may differ from the plain
 * entry point's; dg_get_workspace_size covers both.
 */
int dg_fp8_gemm_nt_qout(const uint8_t* a, const float* sfa, const uint8_t* b, const float* sfb,
                        uint16_t* d, uint8_t* dq, float* dsf, int m, int n, int k, int64_t lda,
                        int64_t ldb, int64_t ldd, int64_t ld_sfa, int64_t ld_dsf, void* workspace,
                        size_t workspace_bytes, void* stream);
int dg_grouped_contiguous_qout(const uint8_t* a, const float* sfa, const uint8_t* b,
                               const float* sfb, uint16_t* d, uint8_t* dq, float* dsf,
                               const int32_t* m_indices, int m_total, int n, int k, int num_groups,
                               int64_t ld_sfa, int64_t ld_dsf, void* workspace,
                               size_t workspace_bytes, void* stream);
int dg_grouped_masked_qout(const uint8_t* a, const float* sfa, const uint8_t* b, const float* sfb,
                           uint16_t* d, uint8_t* dq, float* dsf, const int32_t* masked_m,
                           int num_groups, int m_max, int n, int k, int expected_m, int64_t ld_sfa,
                           int64_t ld_dsf, void* workspace, size_t workspace_bytes, void* stream);

/*
 * The UE8M0 GEMMs with a quantised copy of their output in the same format:
 * input scales as for the *_ue8m0 entry points, and every 1x128 tile of the
 * bf16 output quantised exactly as dg_quant_1x128_ue8m0 would quantise d
 * (E = ceil(log2(amax / 448)) + 127 clamped to [0, 254], q = e4m3(x / 2^(E-127))).
 *   dq  as for the *_qout entry points
 *   dsf uint8 exponents [n/128][ld_dsf] (masked: [num_groups][n/128][ld_dsf])
 * Rules, written rows and scale padding as for the *_qout entry points.
 */
int dg_fp8_gemm_nt_ue8m0_qout(const uint8_t* a, const uint8_t* sfa, const uint8_t* b, const uint8_t* sfb,
                              uint16_t* d, uint8_t* dq, uint8_t* dsf, int m, int n, int k, int64_t lda,
                              int64_t ldb, int64_t ldd, int64_t ld_sfa, int64_t ld_dsf, void* workspace,
                              size_t workspace_bytes, void* stream);
int dg_grouped_contiguous_ue8m0_qout(const uint8_t* a, const uint8_t* sfa, const uint8_t* b,
                                     const uint8_t* sfb, uint16_t* d, uint8_t* dq, uint8_t* dsf,
                                     const int32_t* m_indices, int m_total, int n, int k, int num_groups,
                                     int64_t ld_sfa, int64_t ld_dsf, void* workspace,
                                     size_t workspace_bytes, void* stream);
int dg_grouped_masked_ue8m0_qout(const uint8_t* a, const uint8_t* sfa, const uint8_t* b, const uint8_t* sfb,
                                 uint16_t* d, uint8_t* dq, uint8_t* dsf, const int32_t* masked_m,
                                 int num_groups, int m_max, int n, int k, int expected_m, int64_t ld_sfa,
                                 int64_t ld_dsf, void* workspace, size_t workspace_bytes, void* stream);

/*
 * K-axis grouped GEMM (the weight-gradient GEMM of MoE training): the tokens
 * of all experts are concatenated along K, and group g owns the K range
 * [k_offsets[g], k_offsets[g+1]).  The pages name grouping along K next to
 * grouping along M ("DeepGEMM: efficient BLAS kernel library on GPU",
 * yfxerp.com, section 3.2) and say no more; reading taken here: both operands
 * are activation-like and carry the activation quantiser's 1x128 scales along
 * K, so
 *   D_g[m][n] = bf16( sum_{kb in group g} P_kb[m][n] * (sfa[kb][m] * sfb[kb][n]) ).
 *   a   [m][k] e4m3, sfa [k/128][ld_sfa] fp32 (ld_sfa >= m, a multiple of 4)
 *   b   [n][k] e4m3, sfb [k/128][ld_sfb] fp32 (ld_sfb >= n, a multiple of 4):
 *       one scale per row of B and 128-wide K slice (dg_quant_1x128 of B)
 *   d   [num_groups][m][n] bf16
 *   k_offsets [num_groups + 1] int32 (device): 0 = k_offsets[0] <= ... <=
 *       k_offsets[num_groups] = k, multiples of 128 (precondition; values are
 *       clamped to [0, k] and rounded down to a slice, so nothing is read out
 *       of bounds for any content).  An empty group writes zeros.
 * Rules as for dg_fp8_gemm_nt with lda = ldb = k and ldd = n, plus n % 8 == 0.
 * Needs no workspace (pass NULL, 0).  Data-parallel over (group, M tile,
 * N tile) units.
 */
int dg_k_grouped_nt(const uint8_t* a, const float* sfa, const uint8_t* b, const float* sfb, uint16_t* d,
                    const int32_t* k_offsets, int num_groups, int m, int n, int k, int64_t ld_sfa,
                    int64_t ld_sfb, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Dense GEMM with the other operand majors: NN, TN and TT beside NT ("DeepGEMM:
 * efficient BLAS kernel library on GPU", yfxerp.com, section 3.1, which lists
 * the four layouts without defining them).  Reading taken here: the letters
 * name the operations in D = op(A) * op(B) on row-major storage, NT being
 * D = A * B^T with a [m][k] and b [n][k].  So
 *   NN: a [m][lda] (K-major),  b [k][ldb] (N-major: B(n, kk) at b + kk*ldb + n)
 *   TN: a [k][lda] (M-major: A(r, kk) at a + kk*lda + r), b [k][ldb] (N-major)
 *   TT: a [k][lda] (M-major),  b [n][ldb] (K-major)
 * and in every case D[r][c] = bf16( sum_kb P_kb[r][c] * (sfa[kb][r] * sfb[c/128][kb]) )
 * with the scales in the NT layouts: sfa [k/128][ld_sfa] (one scale per row
 * of the logical A and 128-deep K slice), sfb [ceil(n/128)][k/128] (one per
 * 128x128 block of the logical B).  The codes are the same bytes as for NT,
 * stored transposed: a 1x128 tile along K of an M-major A is a column
 * segment of 128 rows (dg_quant_1x128_mn produces it); a 128x128 weight block
 * is a block either way, so an N-major B can take the codes of
 * dg_quant_128x128 applied to its [k][n] storage with that call's scale
 * matrix transposed (when n % 128 == 0).
 * Rules as for dg_fp8_gemm_nt, except for an M-major A: m % 16 == 0,
 * lda >= m, lda % 16 == 0, k * lda < 2^32; for an N-major B: n % 16 == 0,
 * ldb >= n, ldb % 16 == 0, k * ldb < 2^32.  Workspace as for dg_fp8_gemm_nt
 * (the same tile choice and work division).
 */
int dg_fp8_gemm_nn(const uint8_t* a, const float* sfa, const uint8_t* b, const float* sfb,
                   uint16_t* d, int m, int n, int k, int64_t lda, int64_t ldb, int64_t ldd,
                   int64_t ld_sfa, void* workspace, size_t workspace_bytes, void* stream);
int dg_fp8_gemm_tn(const uint8_t* a, const float* sfa, const uint8_t* b, const float* sfb,
                   uint16_t* d, int m, int n, int k, int64_t lda, int64_t ldb, int64_t ldd,
                   int64_t ld_sfa, void* workspace, size_t workspace_bytes, void* stream);
int dg_fp8_gemm_tt(const uint8_t* a, const float* sfa, const uint8_t* b, const float* sfb,
                   uint16_t* d, int m, int n, int k, int64_t lda, int64_t ldb, int64_t ldd,
                   int64_t ld_sfa, void* workspace, size_t workspace_bytes, void* stream);

/*
 * The same three with UE8M0 scales, the format the pages give for the
 * architecture that has the four layouts (same article, section 3.1): sfa
 * and sfb are exponent bytes in the layouts of dg_fp8_gemm_nt_ue8m0 (sfa
 * [k/128][ld_sfa], sfb [k/128][dg_get_ue8m0_sfb_leading_dim(n)]), the scales
 * again belonging to the logical operands; dg_quant_1x128_mn_ue8m0 quantises
 * an M-major A.  Rules as for the fp32-scale forms.
 */
int dg_fp8_gemm_nn_ue8m0(const uint8_t* a, const uint8_t* sfa, const uint8_t* b, const uint8_t* sfb,
                         uint16_t* d, int m, int n, int k, int64_t lda, int64_t ldb, int64_t ldd,
                         int64_t ld_sfa, void* workspace, size_t workspace_bytes, void* stream);
int dg_fp8_gemm_tn_ue8m0(const uint8_t* a, const uint8_t* sfa, const uint8_t* b, const uint8_t* sfb,
                         uint16_t* d, int m, int n, int k, int64_t lda, int64_t ldb, int64_t ldd,
                         int64_t ld_sfa, void* workspace, size_t workspace_bytes, void* stream);
int dg_fp8_gemm_tt_ue8m0(const uint8_t* a, const uint8_t* sfa, const uint8_t* b, const uint8_t* sfb,
                         uint16_t* d, int m, int n, int k, int64_t lda, int64_t ldb, int64_t ldd,
                         int64_t ld_sfa, void* workspace, size_t workspace_bytes, void* stream);

/* ----------------------------------------------------------- quantisers -- */

/*
 * Activation quantiser, one fp32 scale per 1x128 tile ("Deepseek DeepGEMM
 * technical principles", section "Technical background and core principles";
 * fp32 scales per the yfxerp.com DeepGEMM article, section 3.1).  For each row
 * r and 128-column slice j of x (bf16 widened exactly to fp32):
 *   amax = max |x|,  s = fp32(amax / 448)  (IEEE division, round to nearest),
 *   q = e4m3( fp32(x / s) )  (nearest, ties to even, magnitudes above 448
 *   clamp to 448; an all-zero tile gets s = 0 and signed-zero codes).
 *   x  [num_groups][rows][cols] bf16 (row-major, contiguous)
 *   q  [num_groups][rows][cols] e4m3
 *   sf [num_groups][cols/128][ld_sf] fp32 (MN-major); entries for rows in
 *      [rows, ld_sf) are written as 0.
 * cols % 128 == 0; ld_sf >= rows and a multiple of 4.  num_groups >= 1 (use
 * num_groups > 1 for the masked layout's [G][M_max][K] activations).
 */
int dg_quant_1x128(const uint16_t* x, uint8_t* q, float* sf, int rows, int cols,
                   int64_t ld_sf, int num_groups, void* stream);

/*
 * The same activation quantiser for an M-major matrix (the A operand of the
 * TN and TT GEMMs above): x is stored [rows][cols] = [K][M], and the 1x128
 * tiles run along K, i.e. tile (kb, c) is the column segment
 * x[128 kb .. 128 kb + 127][c].  The result equals dg_quant_1x128 applied to
 * x^T (rows and cols swapped) with its codes stored transposed:
 *   q  [rows][cols] e4m3 (the layout of x)
 *   sf [rows/128][ld_sf] fp32; entries for columns in [cols, ld_sf) are 0.
 * rows % 128 == 0, cols % 8 == 0, ld_sf >= cols and a multiple of 4.
 */
int dg_quant_1x128_mn(const uint16_t* x, uint8_t* q, float* sf, int rows, int cols, int64_t ld_sf,
                      void* stream);

/*
 * Weight quantiser, one fp32 scale per 128x128 block (same sources and the
 * same arithmetic as dg_quant_1x128, with amax over the block; when rows is
 * not a multiple of 128 the last block covers only the valid rows).
 *   w  [num_groups][rows][cols] bf16, q [num_groups][rows][cols] e4m3
 *   sf [num_groups][ceil(rows/128)][cols/128] fp32
 * cols % 128 == 0.
 */
int dg_quant_128x128(const uint16_t* w, uint8_t* q, float* sf, int rows, int cols,
                     int num_groups, void* stream);

/*
 * The two quantisers with UE8M0 scales (scale format: yfxerp.com DeepGEMM
 * article, section 3.1; the pages do not say how the exponent is chosen).
 * Each tile or block takes the smallest power of two not below amax/448:
 *   E = ceil(log2(amax / 448)) + 127 on the exact quotient, clamped to
 *   [0, 254]; an all-zero tile gets E = 0;  s = 2^(E-127);
 *   q = e4m3( fp32(x / s) ) with the same rounding and clamping as above
 *   (x / s only shifts the exponent, so it is exact for normal results).
 * dg_quant_1x128_ue8m0: x, q as dg_quant_1x128;
 *   sf [num_groups][cols/128][ld_sf] uint8, rows [rows, ld_sf) written as 0.
 * dg_quant_128x128_ue8m0: w, q as dg_quant_128x128;
 *   sf [num_groups][cols/128][ld_sfb] uint8 (MN-major, unlike the fp32 weight
 *   scales), ld_sfb = dg_get_ue8m0_sfb_leading_dim(rows), pads written as 0.
 */
int dg_quant_1x128_ue8m0(const uint16_t* x, uint8_t* q, uint8_t* sf, int rows, int cols,
                         int64_t ld_sf, int num_groups, void* stream);
int dg_quant_128x128_ue8m0(const uint16_t* w, uint8_t* q, uint8_t* sf, int rows, int cols,
                           int num_groups, void* stream);
/* dg_quant_1x128_mn with UE8M0 scales: sf [rows/128][ld_sf] uint8, columns
 * [cols, ld_sf) written as 0 (dg_quant_1x128_ue8m0 of x^T, codes transposed). */
int dg_quant_1x128_mn_ue8m0(const uint16_t* x, uint8_t* q, uint8_t* sf, int rows, int cols, int64_t ld_sf,
                            void* stream);

/* -------------------------------------------------------------- utilities -- */

/* Workspace bytes a GEMM of this shape needs (0 when it needs none).  For the
 * masked layout pass m = m_max; for contiguous pass m = m_total.
 * The workspace holds per-tile arrival counters in a region of fixed size at
 * its start (32 KiB, the same for every shape and configuration) and the
 * split-K partial sums after it.  It must be zero-filled once before its
 * first use; every call leaves the counters back at zero, so a workspace can
 * be reused without clearing by later calls of any shape, as long as it is
 * large enough for each.  Calls that run at the same time must not share a
 * workspace.
 * Shapes the GEMMs reject for their tile count (see the shape rules above)
 * report 0. */
size_t dg_get_workspace_size(int m, int n, int k, int num_groups);

/* Number of compute units the persistent kernels are sized to (set_num_sms /
 * get_num_sms; project introduction, section Utility functions).  The default
 * is the device's CU count, or DG_NUM_CUS from the environment.
 * dg_get_num_cus returns a negative dg_status if no device can be queried;
 * dg_set_num_cus accepts 0 .. 4096, 0 restoring the default. */
int dg_get_num_cus(void);
int dg_set_num_cus(int num_cus);

/* Row alignment each expert segment needs in the contiguous layout
 * (get_m_alignment_for_contiguous_layout; section Utility functions): 128. */
int dg_get_m_alignment_for_contiguous_layout(void);

/* Leading dimension of the transposed activation scale matrix for m rows
 * (get_tma_aligned_size; section Utility functions): round_up(m, 4), so that
 * every column starts 16-byte aligned.  Returns -1 for m < 0. */
int64_t dg_get_sf_leading_dim(int m);

/* Leading dimension of the UE8M0 weight-scale matrix for n rows of B:
 * round_up(ceil(n/128), 4) bytes.  Returns -1 for n < 0. */
int64_t dg_get_ue8m0_sfb_leading_dim(int n);

/* Text of the last error on the calling thread ("" if none). */
const char* dg_get_last_error_string(void);

/* Human-readable description of the tile configuration the library would
 * choose for a GEMM (layout 0 = dense, 1 = contiguous, 2 = masked, 3 = K-grouped, plus 8 for
 * the *_qout entry points; m is M, M_total or M_max; expected_m is the masked
 * layout's hint, 0 otherwise),
 * written into buf (NUL-terminated, truncated to len).  Returns DG_SUCCESS or
 * an error for invalid arguments or shapes the GEMMs reject for their tile
 * count.  Pure host logic: needs no device. */
int dg_describe_config(int layout, int m, int n, int k, int num_groups, int expected_m,
                       int num_cus, char* buf, size_t len);

#ifdef __cplusplus
}
#endif

#endif /* DG_H_ */
