/*
 * w4a16_internal.h -- entry points of libw4a16.so that force a kernel choice.
 *
 * Not part of the public C ABI (include/w4a16.h): tests and benchmarks use
 * them to run a particular kernel at a shape where the automatic choice would
 * pick another. The result of a forced choice satisfies the same contract as
 * the public call it extends.
 */
#ifndef W4A16_INTERNAL_H
#define W4A16_INTERNAL_H

#include <stddef.h>
#include <stdint.h>

#include "../../include/w4a16.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 *   path   : 0 = automatic, 1 = M == 1 GEMV, 2 = M <= 48 small-batch kernel
 *            (MFMA 16x16x32, one row tile of 16, two past 16 rows, three past
 *            32), 3 = LDS-DMA tile kernel (the only path of the grouped and
 *            batched calls, and of group size 32)
 *   variant: -1 = default for the path; otherwise
 *            path 1: 1 = the half-wave layout (the fallback for slice lengths
 *              with no MFMA tiling), 0 = the MFMA layout where it applies;
 *            path 2: 1 or 2 = the register-streaming kernel with that many
 *              column tiles of 16 per wave (1 only past 32 rows); 3 .. 6 =
 *              the LDS-staged kernel (M <= 16) with stage geometry 0 .. 3
 *              (groups per stage x stages in flight: 8 x 3, 4 x 6, 4 x 5,
 *              4 x 4);
 *            path 3: rows per tile, 48 .. 144 in steps of 16 (80 .. 128 at
 *              group size 32).
 * An unavailable combination returns W4A16_ERR_SHAPE (W4A16_ERR_GROUP_SIZE
 * for group size 32 on a kernel or tile height that takes 128 only).
 */
typedef struct {
  int32_t path;
  int32_t variant;
} w4a16_config;

/* The automatic choice of a plain GEMM (split_k = 0, no config): its path
 * and variant (as above, variant resolved) and split-K. W4A16_OK, or the
 * status the public call would return for these sizes (M = 0 gives
 * W4A16_OK with path 0 and split-K 0: nothing would run). */
w4a16_status w4a16_gemm_auto_config(int64_t M, int64_t N, int64_t K, int32_t group_size,
                                    w4a16_config* cfg_out, int32_t* split_k_out);

size_t w4a16_gemm_workspace_bytes_ex(int64_t M, int64_t N, int64_t K, int32_t group_size,
                                     int32_t split_k, const w4a16_config* cfg);

w4a16_status w4a16_gemm_ex(const uint16_t* x, const uint8_t* w_packed,
                           const uint16_t* scales, uint16_t* y,
                           int64_t M, int64_t N, int64_t K, int32_t group_size,
                           int32_t split_k, float* workspace,
                           size_t workspace_bytes, void* stream,
                           const w4a16_config* cfg);

w4a16_status w4a16_gemm_grouped_ex(const uint16_t* x, const uint8_t* w_packed,
                                   const uint16_t* scales, const int32_t* m_sizes,
                                   uint16_t* y, int32_t G, int64_t M_total,
                                   int64_t N, int64_t K, int32_t group_size,
                                   void* stream, const w4a16_config* cfg);

size_t w4a16_gemm_batched_workspace_bytes_ex(int32_t B, int64_t M, int64_t N, int64_t K,
                                             int32_t group_size, int32_t split_k,
                                             const w4a16_config* cfg);

w4a16_status w4a16_gemm_batched_ex(const uint16_t* x, const uint8_t* w_packed,
                                   const uint16_t* scales, uint16_t* y,
                                   int32_t B, int64_t M, int64_t N, int64_t K,
                                   int32_t group_size, int32_t split_k,
                                   float* workspace, size_t workspace_bytes,
                                   void* stream, const w4a16_config* cfg);

#ifdef __cplusplus
}
#endif

#endif /* W4A16_INTERNAL_H */
