/*
 * fdec_test.h -- test, tuning and measurement controls of libfdec.  Not for production
 * use: nothing here is needed to run the fused path (include/fdec.h), and production
 * callers should not call any of it.
 *
 * Overrides.  The override setters change which GEMV kernel and work split later calls
 * plan.  The values live in process-wide atomics; every compute call reads them once at
 * entry, plans once, checks its workspace against that plan and launches that plan, so a
 * setter racing with a call cannot make the call launch a plan its workspace was not
 * checked for.  The production workspace queries of fdec.h ignore the overrides; the
 * queries below include them.  A call made while an override is active needs a workspace
 * of the size these queries return.
 */
#ifndef FDEC_TEST_H
#define FDEC_TEST_H

#include "fdec.h"

#ifdef __cplusplus
extern "C" {
#endif

/* fdec_set_gemv_split(k): GEMVs of at most 16 rows run the split-K VALU kernel with K
 *   split into about k parts per column tile (0 restores the built-in choice; values
 *   that do not fit the shape are clamped).  Calls with more than 16 rows ignore it:
 *   only the matrix-core kernel takes them.
 * fdec_set_gemv_tiling(waves, cols_per_workgroup): force the column-owning GEMV
 *   kernel's workgroup shape (1..14 dot waves next to the staging waves, 16 waves in
 *   all; each dot wave owns at most 8 columns with K <= 2048, fewer with longer K or with
 *   3..4 rows); (0, 0) restores the built-in choice.  Shapes the kernel cannot take fall
 *   back to it.
 * fdec_test_fail_launches(on): while on, every compute call validates its arguments
 *   and then returns FDEC_ERR_HIP without touching the GPU (exercises the error path
 *   on machines without a GPU). */
FDEC_API void fdec_set_gemv_split(int32_t k);
FDEC_API void fdec_set_gemv_tiling(int32_t waves, int32_t cols_per_workgroup);
FDEC_API void fdec_test_fail_launches(int32_t on);
/* fdec_set_mfma_plan(kernel, tiles, groups_per_wave): the matrix-core kernel GEMVs of
 *   5..16 rows run.  kernel 0: the built-in choice; 1: the row-block kernel (its
 *   activation staged in LDS); 2: the kernel whose waves split K, with `tiles` 16-column
 *   tiles per workgroup (4 or 8) and `groups_per_wave` 128-wide groups per wave (1..4; at
 *   most 2 with the SwiGLU prologue), 0 for either leaving the built-in choice; 3: the
 *   kernel fed by direct-to-LDS loads of every operand (also the pair-mode gate_up of
 *   fdec_w4_gemv_swiglu and of the 16-row layer). */
FDEC_API void fdec_set_mfma_plan(int32_t kernel, int32_t tiles, int32_t groups_per_wave);
/* fdec_set_kmfma_waves(waves): waves per workgroup (6..8) of the kernel whose waves split
 *   K, each wave taking its own groups of the workgroup's K slice; 0 (or any other value)
 *   leaves the built-in choice. */
FDEC_API void fdec_set_kmfma_waves(int32_t waves);

/* Workspace sizes under the overrides active now (equal to the fdec.h queries when none
 * is): fdec_test_gemv_workspace_bytes for fdec_swiglu_w4_gemv / fdec_w4_gemv,
 * fdec_test_mlp_workspace_bytes for fdec_mlp_decode / _chain / _graph_create / _update. */
FDEC_API size_t fdec_test_gemv_workspace_bytes(int32_t M, int32_t K, int32_t N);
/* fdec_test_gemv_kernel(M, K, N, swiglu): the kernel fdec_swiglu_w4_gemv (swiglu != 0) or
 *   fdec_w4_gemv (swiglu == 0) launches for this shape under the current switches:
 *   0 column-owning (VALU), 1 split-K (VALU, with the finish kernel), 2 matrix-core row
 *   blocks, 3 matrix-core with the waves splitting K, 4 matrix-core fed by direct-to-LDS
 *   loads; -1 for a shape the entry points reject.  Host-side planning only: no GPU. */
FDEC_API int32_t fdec_test_gemv_kernel(int32_t M, int32_t K, int32_t N, int32_t swiglu);
FDEC_API size_t fdec_test_mlp_workspace_bytes(int32_t M, int32_t H, int32_t I);

/*
 * Measurement probes (no part of the method; they bound what the GEMV could reach).
 *
 * fdec_test_empty_kernel: one launch of a kernel that does nothing, with `wgs`
 *   workgroups of `threads` threads (1 <= wgs <= 65536, threads a multiple of 64 in
 *   [64, 1024]).  Back-to-back launches of it measure the per-launch floor.
 *
 * fdec_test_read_ceiling: one launch that only reads, in the order the column-owning
 *   GEMV reads, the bytes that GEMV reads, and writes one 4-byte word per workgroup:
 *     - `wgs` workgroups of 1024 threads; workgroup b reads the 16-byte chunks
 *       [b * per_wg, (b + 1) * per_wg) of `stream` (its columns' packed weights,
 *       contiguous), stream16 = wgs * per_wg chunks in all, non-temporal loads;
 *     - every workgroup reads all bcast16 chunks of `bcast0` and of `bcast1` (the
 *       activation inputs g and u);
 *     - for each of `rows` rows of `pieces` (row r at byte offset r * row_bytes), the
 *       16-byte pieces covering bytes [b * piece_bytes, (b + 1) * piece_bytes) of the
 *       row (the group scales of its columns);
 *     - sink[b] = a checksum of what it read (uint32 [wgs]).
 *   Limits: per_wg <= 4096, bcast16 <= 2048, rows * (piece_bytes / 16 + 2) <= 1024,
 *   every range inside its buffer (the caller passes the byte sizes; they are checked),
 *   16-byte aligned pointers and row_bytes % 16 == 0.
 */
FDEC_API int fdec_test_empty_kernel(int32_t wgs, int32_t threads, fdec_stream stream);
FDEC_API int fdec_test_read_ceiling(const void* stream_buf, size_t stream_bytes, int32_t per_wg,
                                    const void* bcast0, const void* bcast1, size_t bcast_bytes,
                                    const void* pieces, size_t pieces_bytes, int32_t rows,
                                    int32_t row_bytes, int32_t piece_bytes, int32_t wgs,
                                    uint32_t* sink, fdec_stream stream);

#ifdef __cplusplus
}
#endif
#endif /* FDEC_TEST_H */
