/*
 * dg.h - FP8 NT GEMM with fine-grained scaling factors and its M-grouped
 * (MoE) variants, for AMD Instinct MI355X (gfx950).
 *
 * Calls: the dense GEMM and the contiguous, masked and no-padding M-grouped
 * GEMMs (float32 scales, promoted per 128-K block), the same four with
 * power-of-two scales applied by the matrix cores (*_ue8m0), the FP8 x FP4
 * (W4A8) M-grouped GEMMs, and the K-grouped weight-gradient GEMM (float32
 * output, also *_ue8m0). The general contract below holds for all of them;
 * each declaration states what differs.
 *
 * The operation (see the "DeepGEMM for PPU" README, "Interfaces > Notices",
 * "Normal dense GEMMs", "Grouped GEMMs (contiguous layout)" and "Grouped GEMMs
 * (masked layout)"; scale recipe (1, 128, 128) from the "DeepGEMM
 * Compatibility Wrapper (deep-gemm)" page, "0.2.7 Compatibility Additions"):
 *
 *     Ahat[m][k] = e4m3(A[m][k]) * sfa[k/128][m]
 *     Bhat[n][k] = e4m3(B[n][k]) * sfb[n/128][k/128]
 *     D[m][n]    = bf16( sum_k Ahat[m][k] * Bhat[n][k] )
 *
 * NT format only: A is row-major [M][K] (K contiguous) and B is the
 * transposed right-hand side, row-major [N][K]. FP8 is OCP E4M3 (e4m3fn,
 * max 448). Scales are float32. The LHS scales are stored transposed
 * ("M-major") with a 16-byte aligned leading dimension
 * ld_sfa = dg_get_tma_aligned_size(M, 4), i.e. sfa[kb * ld_sfa + m]. D is
 * row-major BF16 [M][N], rounded to nearest even.
 *
 * Accumulation: per 128-wide K block the FP8 products are summed in float32
 * by the matrix cores; each block's partial sum is then multiplied by
 * sfa * sfb and added into a float32 total ("promotion"). Results agree
 * with the exact sum rounded once to BF16 up to float32 summation-order
 * rounding.
 *
 * Ownership: every pointer is caller-owned device memory (HIP). The library
 * allocates nothing, keeps no reference after the call returns, and never
 * reads device memory from the host. Each call enqueues one kernel on
 * `stream` (a hipStream_t; NULL = the null stream) and returns without
 * synchronising; the calls are safe to capture in a HIP graph.
 *
 * Errors: arguments are checked before anything is enqueued; any failure
 * returns a nonzero dg_status and enqueues nothing. Checked: null pointers,
 * non-positive N/K/max_m, negative M/G, K % 128, N % 128, contiguous
 * M % 128, 16-byte alignment of A, B, D and of the scale arrays, and the
 * size limits below. M == 0 (dense, contiguous) and G == 0 are successful
 * no-ops. A failed kernel launch returns DG_ERR_LAUNCH. Faults inside a
 * kernel surface asynchronously at the caller's next synchronisation, as
 * for any HIP kernel. Thread safety: calls may be made from any thread;
 * the only library state is the CU-count setting.
 *
 * Limits: K <= 2^20, N <= 2^20, every operand < 2^40 bytes, num_groups <= 4096
 * for the masked layout, <= 2048 for the no-padding layout and <= 512 for
 * the K-grouped GEMM.
 */
#ifndef DG_H
#define DG_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int dg_status;

#define DG_OK 0
#define DG_ERR_NULL 1         /* a required pointer is NULL                   */
#define DG_ERR_SHAPE 2        /* a size is out of range or not a multiple     */
#define DG_ERR_ALIGN 3        /* a pointer is not 16-byte aligned             */
#define DG_ERR_UNSUPPORTED 4  /* a size beyond the documented limits          */
#define DG_ERR_LAUNCH 5       /* hipLaunchKernel or a HIP query failed        */
#define DG_ERR_DEVICE 6       /* no HIP device, or the device is not gfx950   */

/*
 * Dense FP8 NT GEMM ("DeepGEMM for PPU" README, "Normal dense GEMMs").
 *   a   [m][k]   E4M3                       b   [n][k]   E4M3
 *   sfa [k/128][dg_get_tma_aligned_size(m,4)] float32
 *   sfb [n/128][k/128] float32              d   [m][n]   BF16 (written in full)
 * m >= 0 (any value; ragged M is supported), n % 128 == 0, k % 128 == 0.
 */
dg_status dg_fp8_gemm_nt(const void* a, const float* sfa,
                         const void* b, const float* sfb,
                         void* d,
                         int m, int n, int k, void* stream);

/*
 * M-grouped FP8 NT GEMM, contiguous layout ("DeepGEMM for PPU" README,
 * "Grouped GEMMs (contiguous layout)"; 128-row alignment from the
 * "DeepGEMM Compatibility Wrapper" page, "Contiguous Grouped GEMM
 * Alignment"). Only M is grouped; N and K are shared by every group.
 *   a   [m][k] E4M3, the groups' rows concatenated, each group's segment
 *       starting on a multiple of 128 rows and padded to one
 *   sfa [k/128][dg_get_tma_aligned_size(m,4)] float32
 *   b   [num_groups][n][k] E4M3          sfb [num_groups][n/128][k/128] float32
 *   d   [m][n] BF16
 *   grouped_layout [m] int32 (device): group id of each row, -1 for padding.
 * Row r of d is written iff grouped_layout[r] equals the id g of the first
 * row of the 128-row block that holds r, and 0 <= g < G. Every other row
 * (padding, an id outside [0, G), or an id that differs from its block's
 * first row) is never written and never influences written rows; for
 * layouts whose segments are 128-row aligned, as required, this writes
 * exactly the rows with an id in [0, G). m % 128 == 0.
 */
dg_status dg_m_grouped_fp8_gemm_nt_contiguous(const void* a, const float* sfa,
                                              const void* b, const float* sfb,
                                              void* d, const int32_t* grouped_layout,
                                              int m, int n, int k, int num_groups,
                                              void* stream);

/*
 * M-grouped FP8 NT GEMM, masked layout ("DeepGEMM for PPU" README,
 * "Grouped GEMMs (masked layout)"), for decoding under graph capture where
 * the host does not know how many rows each group holds.
 *   a   [num_groups][max_m][k] E4M3
 *   sfa [num_groups][k/128][dg_get_tma_aligned_size(max_m,4)] float32
 *   b   [num_groups][n][k] E4M3          sfb [num_groups][n/128][k/128] float32
 *   d   [num_groups][max_m][n] BF16
 *   masked_m [num_groups] int32 (device): valid rows of each group, read by
 *       the kernel only, clamped to [0, max_m].
 * Rows m < masked_m[g] of d[g] are written; all other rows are untouched.
 * The launch shape depends only on (num_groups, max_m, n, k) and the CU
 * count, so one captured graph serves any masked_m contents.
 */
dg_status dg_m_grouped_fp8_gemm_nt_masked(const void* a, const float* sfa,
                                          const void* b, const float* sfb,
                                          void* d, const int32_t* masked_m,
                                          int num_groups, int max_m, int n, int k,
                                          void* stream);

/*
 * M-grouped FP8 NT GEMM, no-padding layout ("DeepGEMM for PPU" README,
 * "Grouped GEMMs (nopad layout)"): the groups' rows are concatenated with no
 * alignment padding, and a per-group row count replaces the per-row index.
 *   a   [m][k] E4M3: group 0's rows, then group 1's, ... (any counts)
 *   sfa [k/128][dg_get_tma_aligned_size(m,4)] float32
 *   b   [num_groups][n][k] E4M3          sfb [num_groups][n/128][k/128] float32
 *   d   [m][n] BF16
 *   group_rows [num_groups] int32 (device): rows of each group, read by the
 *       kernel only. A negative count counts as zero.
 * Group g owns rows [s_g, e_g) with s_g = min(sum_{j<g} c_j, m) and
 * e_g = min(s_g + c_g, m), c_j = max(group_rows[j], 0): rows at or past m
 * do not exist, so a group that would reach past them is cut off there.
 * Those rows of d are written; rows at or past min(sum_j c_j, m) are
 * untouched. As for the masked layout the launch shape does not depend on
 * the counts, so one captured graph serves any group_rows contents.
 * m >= 0 (any value).
 */
dg_status dg_m_grouped_fp8_gemm_nt_nopad(const void* a, const float* sfa,
                                         const void* b, const float* sfb,
                                         void* d, const int32_t* group_rows,
                                         int m, int n, int k, int num_groups,
                                         void* stream);

/*
 * The four GEMMs above with power-of-two scales applied by the matrix cores
 * ("DeepGEMM Compatibility Wrapper" page, "0.2.7 Compatibility Additions":
 * UE8M0 scale casting and the packed UE8M0 scale conversion). Arguments,
 * layouts and checks are exactly those of the call without the suffix. The
 * scales are meant to be positive normal powers of two, as a UE8M0 cast at
 * quantisation makes them; each float32 scale s is used as 2^(e - 127),
 * e being its biased exponent field (bits 30..23), which is s itself for
 * such a value (sign and mantissa bits are ignored, as in the packed UE8M0
 * conversion; e = 255 gives NaN). The per-block scales are applied inside
 * the MFMA as E8M0 block scales and the products accumulate in float32 in
 * the MFMA, so there is no separate promotion step.
 */
dg_status dg_fp8_gemm_nt_ue8m0(const void* a, const float* sfa,
                               const void* b, const float* sfb,
                               void* d,
                               int m, int n, int k, void* stream);
dg_status dg_m_grouped_fp8_gemm_nt_contiguous_ue8m0(const void* a, const float* sfa,
                                                    const void* b, const float* sfb,
                                                    void* d, const int32_t* grouped_layout,
                                                    int m, int n, int k, int num_groups,
                                                    void* stream);
dg_status dg_m_grouped_fp8_gemm_nt_masked_ue8m0(const void* a, const float* sfa,
                                                const void* b, const float* sfb,
                                                void* d, const int32_t* masked_m,
                                                int num_groups, int max_m, int n, int k,
                                                void* stream);
dg_status dg_m_grouped_fp8_gemm_nt_nopad_ue8m0(const void* a, const float* sfa,
                                               const void* b, const float* sfb,
                                               void* d, const int32_t* group_rows,
                                               int m, int n, int k, int num_groups,
                                               void* stream);

/*
 * M-grouped FP8 x FP4 (W4A8) NT GEMMs ("DeepGEMM Compatibility Wrapper"
 * page, "0.2.7 Compatibility Additions": FP8 E4M3 A with packed E2M1 FP4 B,
 * LHS scales per 1x128 and RHS scales per 1x32), contiguous and masked
 * layouts. Everything is as for the FP8 calls of the same layout except B
 * and its scales:
 *   b   [num_groups][n][k/2] bytes: OCP E2M1 FP4 values packed two per byte
 *       along K, element 2j in the low nibble of byte j and 2j+1 in the high
 *       one (E2M1: sign bit 3, exponent bits 2..1 with bias 1, mantissa bit 0;
 *       values 0, 0.5, 1, 1.5, 2, 3, 4, 6 and their negatives)
 *   sfb [num_groups][k/32][dg_get_tma_aligned_size(n,4)] float32: one scale
 *       per row n and 32-wide K block, stored transposed like the LHS scales.
 * All scales (sfa and sfb) are read as UE8M0, exactly as by the *_ue8m0
 * calls: 2^(e - 127) with e the float32 exponent field, meant for positive
 * normal powers of two. Products accumulate in float32 inside the MFMA.
 *   D = bf16( sum_k e4m3(A[m][k]) sfa[k/128][m] * e2m1(B[n][k]) sfb[k/32][n] )
 */
dg_status dg_m_grouped_fp8_fp4_gemm_nt_contiguous(const void* a, const float* sfa,
                                                  const void* b, const float* sfb,
                                                  void* d, const int32_t* grouped_layout,
                                                  int m, int n, int k, int num_groups,
                                                  void* stream);
dg_status dg_m_grouped_fp8_fp4_gemm_nt_masked(const void* a, const float* sfa,
                                              const void* b, const float* sfb,
                                              void* d, const int32_t* masked_m,
                                              int num_groups, int max_m, int n, int k,
                                              void* stream);

/*
 * K-grouped FP8 NT GEMM, contiguous K groups: the weight-gradient shape of
 * an MoE layer ("DeepGEMM Compatibility Wrapper" page, "0.2.7 Compatibility
 * Additions": K sizes given on the host, each a multiple of 128, scale recipe
 * (1, 1, 128); per the wrapper's notes, a missing C means D starts from
 * zero, a separate C is the starting value of D, and C given as D itself
 * accumulates into D).
 *   ks  [num_groups] int (HOST memory): K of each group, each >= 0 and a
 *       multiple of 128; K = sum of ks; group g owns K positions
 *       [sum_{j<g} ks[j], sum_{j<=g} ks[j]).
 *   a   [m][K] E4M3                     sfa [K/128][dg_get_tma_aligned_size(m,4)] float32
 *   b   [n][K] E4M3                     sfb [K/128][dg_get_tma_aligned_size(n,4)] float32
 *       (one scale per row and 128-wide K block for both operands)
 *   c   [num_groups][m][n] float32 or NULL; d [num_groups][m][n] float32
 *   d[g][i][j] = (c ? c[g][i][j] : 0)
 *                + sum_{k in group g} e4m3(a[i][k]) sfa[k/128][i] * e4m3(b[j][k]) sfb[k/128][j]
 * c may equal d (accumulation in place); otherwise c and d must not
 * overlap. A group with ks = 0 gets d[g] = c[g] (or zeros). Products
 * accumulate in float32 with a promotion per 128-K block, as for the other
 * GEMMs. num_groups in [1, 512] (an empty ks is rejected), m >= 0 (m == 0 is
 * a no-op), n % 128 == 0, K <= 2^20; c (when given) 16-byte aligned.
 */
dg_status dg_k_grouped_fp8_gemm_nt_contiguous(const void* a, const float* sfa,
                                              const void* b, const float* sfb,
                                              const float* c, float* d,
                                              const int* ks, int num_groups,
                                              int m, int n, void* stream);

/* The K-grouped GEMM with power-of-two scales applied by the matrix cores:
 * arguments and checks as above, every scale read as UE8M0 exactly as by
 * the other *_ue8m0 calls (2^(e - 127), e the float32 exponent field). The
 * per-row scales of both operands become the MFMA's per-lane E8M0 block
 * scales, and the products accumulate in the MFMA: no promotion step. */
dg_status dg_k_grouped_fp8_gemm_nt_contiguous_ue8m0(const void* a, const float* sfa,
                                                    const void* b, const float* sfb,
                                                    const float* c, float* d,
                                                    const int* ks, int num_groups,
                                                    int m, int n, void* stream);

/* Row alignment of each group's segment in the contiguous layout: 128
 * ("DeepGEMM Compatibility Wrapper" page, "Contiguous Grouped GEMM
 * Alignment"; "DeepGEMM for PPU" README, "Utilities"). */
int dg_get_mk_alignment_for_contiguous_layout(void);

/* x rounded up so that x * element_size is a multiple of 16 bytes: the
 * leading dimension of the transposed LHS scales ("DeepGEMM for PPU"
 * README, "Utilities"; "DeepGEMM Compatibility Wrapper" page, "0.2.7
 * Compatibility Additions"). Returns -1 for x < 0 or an element_size that
 * does not divide 16. */
int dg_get_tma_aligned_size(int x, int element_size);

/* Number of compute units the persistent kernels spread over ("DeepGEMM for
 * PPU" README, "Utilities": the maximum SM count to use). Defaults to all
 * CUs of the current device. dg_get_num_cus returns 0 when there is no
 * device. dg_set_num_cus(n) with n <= 0 restores the default; n above the
 * device's CU count is clamped to it. */
int dg_get_num_cus(void);
dg_status dg_set_num_cus(int num_cus);

/* Static description of a status code. */
const char* dg_status_string(dg_status status);

#ifdef __cplusplus
}
#endif

#endif /* DG_H */
