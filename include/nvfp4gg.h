/*
 * nvfp4gg.h -- C ABI of the MI355X (gfx950) NVFP4 block-scaled grouped GEMM.
 *
 * The operation (kernelindex page kernelbot-nvfp4-group-gemm-444497, header
 * comment of its kernel source; page kernelbot-nvfp4-group-gemm-505431,
 * custom_kernel_fallback and apply_scale_factors): for every group i,
 *
 *   C_i[m][n] = sum_k a_i(m,k) * sfa_i(m, k/16) * b_i(n,k) * sfb_i(n, k/16)
 *
 * rounded to fp16 (round-to-nearest-even, overflow to +-inf), accumulated in
 * fp32.  a, b are FP4 E2M1 codes, sfa, sfb are FP8 E4M3 scales, one per 16
 * consecutive K of a row.
 *
 * Memory layouts (all row-major, unpadded):
 *   A_i   M_i x K_i   FP4, two codes per byte, row stride K_i/2 bytes; element
 *                     2j of a row is the low nibble of byte j, element 2j+1 the
 *                     high nibble (page 505431, dequantize_fp4).
 *   B_i   N_i x K_i   same as A_i.
 *   SFA_i M_i x K_i/16 E4M3 bytes, scale of A_i[m][16s .. 16s+15] at [m][s]
 *                     (page 505431, apply_scale_factors: plain [rows, K/16]).
 *   SFB_i N_i x K_i/16 likewise for B_i.
 *   C_i   M_i x N_i   fp16, row stride N_i elements (page 505431, the epilogue
 *                     of group_gemm_kernel_impl addresses C as row * N + col).
 *
 * Ownership: the caller allocates and owns every operand and output.  The
 * size arrays and the pointer arrays are HOST memory, read only during the
 * call; each element pointer is a DEVICE pointer.  C_i is overwritten.
 *
 * Library state: tiles whose K range is split over several workgroups are
 * summed through a device workspace (fp32 partial tiles and one counter per
 * workgroup) that the library allocates with hipMalloc on the first call for
 * a (device, stream) pair, sized for the device's compute units (no launch
 * has more workgroups), and keeps until the process ends: 3 partial tiles of
 * 192 KiB and one int per compute unit (144 MiB and 1 KiB on a 256-CU MI355X).
 * Only that first call allocates (and is not capturable into a HIP graph);
 * every later call on the pair allocates, frees and synchronises nothing.
 * The counters return to zero at the end of every call, so calls on one
 * stream may follow each other with no reset; calls on different streams
 * use different workspaces.
 *
 * Streams: work is enqueued on `stream` (a hipStream_t; NULL is the default
 * stream) and the call returns without synchronising.
 *
 * Errors: every argument is validated before any HIP call.  Return codes:
 *   NVFP4GG_OK            0  success (also when every group is empty)
 *   NVFP4GG_INVALID_ARG  -1  g <= 0, a NULL array, a negative size, K_i not a
 *                            multiple of 16, a NULL or misaligned (16-byte)
 *                            device pointer of a non-empty operand
 *   NVFP4GG_UNSUPPORTED  -2  valid but outside what the kernels handle: a
 *                            non-empty group with K_i % 128 != 0, an operand
 *                            of 2 GiB or more, M_i * N_i >= 2^31, a launch
 *                            whose schedule cost reaches 2^31 units (over
 *                            100 s of GPU work), or a grid of more than 1024
 *                            workgroups (a device with more compute units)
 *   NVFP4GG_HIP_ERROR    -3  a HIP call (launch, first-call workspace allocation) failed
 * nvfp4_group_gemm_last_error() describes the last failure on this thread.
 */
#ifndef NVFP4GG_H
#define NVFP4GG_H

#ifdef __cplusplus
extern "C" {
#endif

#define NVFP4GG_OK 0
#define NVFP4GG_INVALID_ARG (-1)
#define NVFP4GG_UNSUPPORTED (-2)
#define NVFP4GG_HIP_ERROR (-3)

/* Grouped GEMM, one pass over all groups.
 *   g                 number of groups (>= 1; any count, groups are launched
 *                     in batches that fit the kernel-argument block)
 *   M, N, K           host arrays of g sizes; M_i, N_i >= 0 (a group with
 *                     M_i == 0 or N_i == 0 is skipped), K_i >= 0, K_i % 16 == 0
 *                     (K_i == 0 writes zeros to C_i)
 *   A_ptrs .. SFB_ptrs host arrays of g device pointers to the packed operands
 *   C_ptrs            host array of g device pointers to the fp16 outputs
 *   stream            hipStream_t (NULL: default stream)
 */
int nvfp4_group_gemm(int g, const int* M, const int* N, const int* K,
                     const void* const* A_ptrs, const void* const* B_ptrs,
                     const void* const* SFA_ptrs, const void* const* SFB_ptrs,
                     void* const* C_ptrs, void* stream);

/* nvfp4_group_gemm for callers that cannot allocate device memory (code
 * being captured into a HIP graph, tight serving loops, harnesses that
 * forbid hipMalloc): the same arguments, kernels, results and return codes,
 * but the split-tile workspace is a static device array of the library
 * (144 MiB of partial tiles and 1 KiB of counters, the workspace of 256
 * workgroups) instead of the per-stream one, so no call allocates, frees or
 * synchronises.  Each device holds its own copy from the first use of the
 * library on it until the process ends; the first call on a device looks up
 * its address (hipGetSymbolAddress).  Every call first clears the counters
 * with a small kernel on `stream`.  A device with more than 256 compute
 * units is rejected (NVFP4GG_UNSUPPORTED): its launches could need more
 * workspace than the array holds.  All calls on one device share the one
 * array, so calls that overlap on a device (from different streams or
 * threads) race and give wrong results: the caller serialises them. */
int nvfp4_group_gemm_noalloc(int g, const int* M, const int* N, const int* K,
                             const void* const* A_ptrs, const void* const* B_ptrs,
                             const void* const* SFA_ptrs, const void* const* SFB_ptrs,
                             void* const* C_ptrs, void* stream);

/* The same grouped GEMM with SFA_i and SFB_i in the blocked scale layout
 * that the pages' kernels consume (page 482006: to_blocked_gpu in its cuBLAS
 * path, and the scale-factor layout atom of its CuTe kernel, shape
 * ((32,4),(16,4)) with strides ((16,4),(0,1)); page 505431, the scale-factor
 * copy comment block of its kernel).  A scale array of R rows and S = K_i/16
 * scale columns is padded to R' = ceil(R/128)*128 rows and S' = ceil(S/4)*4
 * columns and cut into 128 x 4 atoms of 512 bytes, atoms of one 128-row band
 * consecutive in column order, bands in row order.  Inside an atom, row r
 * (0..127) and column c (0..3) are byte 16*(r%32) + 4*(r/32) + c.  So the
 * scale of row r, column s is byte
 *     512*((r/128)*(S'/4) + s/4) + 16*(r%32) + 4*((r/32)%4) + s%4.
 * SFA_i holds ceil(M_i/128)*128*K_i/16 bytes, SFB_i ceil(N_i/128)*128*K_i/16
 * (K_i % 128 == 0 is required anyway, so S' = S).  Padding bytes are never
 * used in a result.  All other arguments, layouts, ownership, workspace and
 * return codes as nvfp4_group_gemm. */
int nvfp4_group_gemm_blocked(int g, const int* M, const int* N, const int* K,
                             const void* const* A_ptrs, const void* const* B_ptrs,
                             const void* const* SFA_ptrs, const void* const* SFB_ptrs,
                             void* const* C_ptrs, void* stream);

/* The grouped GEMM with a batch of L_i independent products per group, the
 * pages' (M, N, K, L) problem sizes (page 505431, custom_kernel_fallback:
 * C[m,n,l] = sum_k A[m,k,l] B[n,k,l]; page 482006, its CuTe kernel's
 * operand layouts, whose batch stride is the whole M x K, N x K or M x N
 * slice): every operand of group i holds L_i consecutive slices laid out as
 * in nvfp4_group_gemm (A_i: L_i slices of M_i x K_i/2 bytes, SFA_i: L_i of
 * M_i x K_i/16, ..., C_i: L_i of M_i x N_i fp16), slice l of C_i being
 * A_i[l] . B_i[l]^T.  L_i >= 0 (L_i == 0 skips the group).  Every slice must
 * start 16-byte aligned: with L_i > 1 each slice's byte count must be a
 * multiple of 16, else NVFP4GG_UNSUPPORTED.  Otherwise as nvfp4_group_gemm. */
int nvfp4_group_gemm_batched(int g, const int* M, const int* N, const int* K, const int* L,
                             const void* const* A_ptrs, const void* const* B_ptrs,
                             const void* const* SFA_ptrs, const void* const* SFB_ptrs,
                             void* const* C_ptrs, void* stream);

/* The MXFP4 form of the grouped GEMM: the same E2M1 operands A_i, B_i and
 * fp16 output, with one E8M0 scale per 32 consecutive K of a row instead of
 * an E4M3 scale per 16:
 *   C_i[m][n] = sum_k a_i(m,k) * 2^(sfa_i(m, k/32) - 127) * b_i(n,k) * 2^(sfb_i(n, k/32) - 127)
 * rounded to fp16, accumulated in fp32.  The pages name this MX block
 * scaling beside the NVFP4 one (page 505431: the block-scaled MMA kind that
 * covers both and the scale-type field of its instruction descriptor; page
 * 444497, header comment) without defining it; E8M0 is read as in the OCP
 * MX format: an unsigned 8-bit exponent, value 2^(code - 127), code 0xFF NaN.
 *   SFA_i  M_i x K_i/32 E8M0 bytes, row-major, unpadded; SFB_i N_i x K_i/32.
 * It runs on gfx950's block-scaled FP4 MFMA directly, with no
 * dequantisation.  Arguments, ownership, workspace and return codes as
 * nvfp4_group_gemm (K_i % 128 == 0 likewise). */
int mxfp4_group_gemm(int g, const int* M, const int* N, const int* K,
                     const void* const* A_ptrs, const void* const* B_ptrs,
                     const void* const* SFA_ptrs, const void* const* SFB_ptrs,
                     void* const* C_ptrs, void* stream);

/* The dequantisation step alone, with the same device code the GEMM uses:
 * out[r][k] = fp16( e2m1(X[r][k]) * e4m3(SFX[r][k/16]) ) for a rows x K
 * packed FP4 matrix X and its rows x K/16 scales (layouts as A_i, SFA_i
 * above; page 505431, dequantize_fp4 and apply_scale_factors).  out is a
 * device buffer of rows*K fp16, row-major.  The product of an E2M1 and an
 * E4M3 value has at most 6 significant bits and lies within fp16's normal
 * range, so the result is exact.  Same return codes as nvfp4_group_gemm. */
int nvfp4_dequant_f16(int rows, int K, const void* X, const void* SFX,
                      void* out, void* stream);

/* Bound, in polls of about a microsecond, on how long the workgroup that
 * finishes a tile split over several workgroups waits for the others
 * (process-wide; default 2^20).  When all workgroups of a launch run at once,
 * as on an otherwise idle GPU, the wait ends long before.  When it runs out,
 * the tile is finished by the last of the others instead, so results do not
 * depend on it; 0 makes that the rule (the test of that path uses it).
 * Returns NVFP4GG_INVALID_ARG for a negative count. */
int nvfp4_group_gemm_set_wait_limit(int polls);

/* The m-block size, in fragments of 16 rows (1..12), used for every launch
 * (process-wide); 0 (the default) chooses it per launch from the problem
 * sizes.  Results do not depend on it beyond fp32 rounding order (each
 * output is one fp32 sum of exact products in every case); it exists for
 * tuning and so that tests can run every tile shape.  Returns
 * NVFP4GG_INVALID_ARG for a value outside 0..12. */
int nvfp4_group_gemm_set_max_frags(int frags);

/* Thread-local description of the last non-OK return ("" if none). */
const char* nvfp4_group_gemm_last_error(void);

/* ABI version of this header: 7 (2 added nvfp4_group_gemm_blocked, 3
 * mxfp4_group_gemm, 4 nvfp4_group_gemm_set_wait_limit, 5
 * nvfp4_group_gemm_batched, 6 nvfp4_group_gemm_set_max_frags and the
 * workspace that no longer grows, 7 nvfp4_group_gemm_noalloc). */
int nvfp4_group_gemm_version(void);

#ifdef __cplusplus
}
#endif

#endif /* NVFP4GG_H */
