/*
 * w4a16.h -- C ABI of a W4A16 GEMM library for AMD Instinct MI355X (gfx950).
 *
 *   Y[M,N] = X[M,K] . dequant(W)[N,K]^T,   dequant(W)[n,k] = S[n, k/g] * (q[n,k] - 8)
 *
 * X and Y are bf16, W is packed unsigned int4 (two nibbles per byte), S holds
 * one bf16 scale per output row per g-wide K group (group_size g = 128, or 32
 * on the tile kernel), accumulation is fp32 and the output is rounded to bf16
 * (round to nearest even).
 *
 * Sources for the operation (pages by title, section in quotes):
 *  - "Add Triton BF16xINT4 rowwise GEMM for ROCm gfx942/gfx950": Summary (bf16
 *    activation times row-major int4 weight; plain, grouped and batched ops),
 *    Implementation "Fused A-operand dot" (low nibble pairs with even K, high
 *    nibble with odd K), "Split-K without atomics" (fp32 [SPLIT_K,M,N]
 *    workspace, separate reduce kernel, graph-safe), "Native fused grouped
 *    kernel" (one launch over G groups, M_total a host int, row offsets from
 *    an on-device exclusive cumsum of M_sizes, no device-to-host sync).
 *  - "[ROCm][Kernel] W4A16 skinny GEMM: hand-asm kernel for gfx1151": section 1
 *    "Magic-constant bf16 dequant" (a nibble decodes as scale * (n - 8),
 *    symmetric), section 3 "Exact buffer-descriptor sizing" (weight and scale
 *    buffers bounded by their exact byte sizes), "Benchmark results
 *    (per-GEMM)" (the decoder GEMMs quantised with one scale per 32 k).
 *
 * Conventions for every entry point:
 *  - Pointers are DEVICE pointers to caller-owned, contiguous, row-major
 *    memory. bf16 values are passed as their raw 16-bit patterns (uint16_t).
 *    Every tensor pointer must be 16-byte aligned (W4A16_ERR_ALIGN).
 *  - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *  - A call only validates its arguments on the host and enqueues kernels on
 *    `stream`: it allocates nothing, copies nothing between host and device
 *    and never synchronises, so it may be captured in a HIP graph.
 *  - Argument errors are returned synchronously, before anything is
 *    enqueued. A failed launch returns W4A16_ERR_LAUNCH. Faults inside a
 *    kernel surface at the caller's next synchronisation (HIP convention).
 *  - The library keeps no state between calls; calls are reentrant. Calls
 *    that share a workspace must be ordered (same stream) by the caller.
 *  - Size limits: every dimension < 2^31; each of X, the packed W of one
 *    group, S of one group, Y and the workspace must be smaller than 2^32
 *    bytes (W4A16_ERR_SHAPE otherwise).
 */
#ifndef W4A16_H
#define W4A16_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  W4A16_OK = 0,
  W4A16_ERR_NULL = 1,        /* a required pointer is NULL                       */
  W4A16_ERR_SHAPE = 2,       /* a dimension is negative, zero where not allowed,
                                odd K, or a size limit is exceeded               */
  W4A16_ERR_GROUP_SIZE = 3,  /* group_size not 128 or 32, K % 128 != 0, or group
                                size 32 with a kernel that takes 128 only        */
  W4A16_ERR_SPLIT_K = 4,     /* split_k not in {0, 1, 2, 4, 8, 16}               */
  W4A16_ERR_WORKSPACE = 5,   /* workspace NULL or smaller than required          */
  W4A16_ERR_ALIGN = 6,       /* a tensor pointer is not 16-byte aligned          */
  W4A16_ERR_LAUNCH = 7       /* the HIP runtime rejected a kernel launch         */
} w4a16_status;

/* Human-readable name of a status code (static string, never NULL). */
const char* w4a16_status_string(int status);

/*
 * Packs unsigned 4-bit values, one per byte, two per byte:
 *   w_packed[r, j] = (q[r, 2j] & 0xF) | (q[r, 2j+1] & 0xF) << 4
 * (low nibble = even k; "Add Triton BF16xINT4 rowwise GEMM for ROCm
 * gfx942/gfx950", Implementation "Fused A-operand dot"). The high four bits
 * of each q byte are ignored.
 *   q        : [rows, K] uint8, device
 *   w_packed : [rows, K/2] uint8, device, written
 *   rows >= 0 (0 = nothing to do), K >= 2 and even.
 * For the weights of a grouped GEMM pass rows = G * N.
 */
w4a16_status w4a16_pack_int4(const uint8_t* q, uint8_t* w_packed,
                             int64_t rows, int64_t K, void* stream);

/*
 * The split-K factor the library uses for w4a16_gemm with group_size 128
 * when split_k == 0 (auto) at this shape: for the M = 1 GEMV only what its register budget for
 * x needs (at most 64 groups per slice), for the M <= 48 kernel slices
 * only while fewer than half of the compute units have a workgroup, and
 * for the tile kernel the power of
 * two (at most 16) of least estimated time among those that keep tiles x SK
 * within one workgroup per compute unit, counting the fp32 partials and the
 * reduce, chosen together with the tile height (so, unlike the MI350X Triton
 * page's prune of split-K at M >= 512, a tall-K shape with few tiles splits
 * at any M). Returns 0 on invalid dimensions.
 */
int32_t w4a16_gemm_auto_split_k(int64_t M, int64_t N, int64_t K);

/*
 * Bytes of workspace w4a16_gemm needs at this shape and split_k (0 = auto)
 * with group_size 128: SK * M * N * 4 (rounded up to 256) when the effective
 * split factor SK > 1, plus, on the tile kernel (M > 16 where the small-
 * batch kernel does not take the shape), (K/128) *
 * round_up(M, 4) * 4 for the per-row group sums of X. Returns 0 when none is
 * needed and for invalid arguments. w4a16_gemm_workspace_bytes_gs gives it
 * for either group size.
 */
size_t w4a16_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K,
                                  int32_t split_k);

/*
 * Y = X . dequant(W)^T.
 *   x         : [M, K] bf16, device
 *   w_packed  : [N, K/2] uint8 (see w4a16_pack_int4), device
 *   scales    : [N, K/group_size] bf16, row n holds the scales of output
 *               column n, device
 *   y         : [M, N] bf16, device, written (bf16 round-to-nearest-even of
 *               the fp32 accumulator)
 *   M >= 0 (M == 0: returns W4A16_OK, nothing enqueued), N >= 1, K >= 128.
 *   group_size: 128, or 32; K % 128 == 0 either way. Group size 32 always
 *               runs the tile kernel (path 3, configurations 2 to 5), at any
 *               M: the M = 1 and M <= 48 kernels take 128-groups only.
 *   split_k   : 0 = auto, or 1, 2, 4, 8, 16. With SK > 1 the K range is cut
 *               into SK contiguous slices of ceil((K/128)/SK) blocks of 128 k
 *               (trailing slices may be empty); slice s writes its fp32 partial sums to
 *               workspace[s, :, :] with plain stores (an empty slice writes
 *               zeros) and a second kernel sums the slices in order
 *               s = 0..SK-1 in fp32 and rounds once to bf16.
 *   workspace : fp32 device scratch, overwritten; may be NULL when
 *               w4a16_gemm_workspace_bytes_gs is 0. With SK > 1 its first
 *               SK * M * N floats hold the [SK, M, N] partials after the call.
 *   workspace_bytes: its size in bytes (>= w4a16_gemm_workspace_bytes_gs for
 *               this group_size).
 * Rows of Y are written exactly once; no atomics are used, so the result is
 * bitwise reproducible for a given shape and split_k.
 */
w4a16_status w4a16_gemm(const uint16_t* x, const uint8_t* w_packed,
                        const uint16_t* scales, uint16_t* y,
                        int64_t M, int64_t N, int64_t K, int32_t group_size,
                        int32_t split_k, float* workspace,
                        size_t workspace_bytes, void* stream);

/*
 * Bytes of workspace w4a16_gemm_grouped needs with group_size 128: (K/128) *
 * round_up(M_total, 4) * 4 (one fp32 row sum per row and 128-group). Returns
 * 0 for invalid arguments or M_total == 0. w4a16_gemm_grouped_workspace_bytes_gs
 * gives it for either group size.
 */
size_t w4a16_gemm_grouped_workspace_bytes(int32_t G, int64_t M_total, int64_t N, int64_t K);

/*
 * Grouped GEMM in one launch: for each group g with
 *   start_g = sum_{h<g} m_sizes[h]   (computed on the device),
 * rows [start_g, start_g + m_sizes[g]) of Y are those rows of X times
 * dequant(W_g)^T.
 *   x         : [M_total, K] bf16, rows concatenated in group order, device
 *   w_packed  : [G, N, K/2] uint8, device
 *   scales    : [G, N, K/group_size] bf16, device
 *   m_sizes   : [G] int32, DEVICE memory (4-byte aligned), read by the kernel
 *               (never copied to the host). Preconditions, not checked
 *               (checking would need a sync): m_sizes[g] >= 0 and
 *               sum == M_total. If they are broken the kernel still writes
 *               only rows inside [0, M_total) of y and reads only rows inside
 *               x; which rows are then written is unspecified. A group with
 *               m_sizes[g] == 0 contributes nothing.
 *   y         : [M_total, N] bf16, device, written
 *   G >= 1, M_total >= 0 (0: W4A16_OK, nothing enqueued), N >= 1, K >= 128,
 *   group_size 128 or 32 (tile configurations 2 to 5), K % 128 == 0; the
 *   scales of all groups together must be smaller than 2^32 bytes.
 *   workspace : fp32 device scratch of workspace_bytes >= the value of
 *               w4a16_gemm_grouped_workspace_bytes_gs; overwritten.
 * Two kernels are enqueued: a pass over X computing per-row group sums, and
 * the grouped tile kernel. The tile grid is sized from the host value
 * M_total: (ceil(M_total/BM) + G) * ceil(N/BN) workgroups; workgroups past
 * the last tile of the last group exit at once.
 */
w4a16_status w4a16_gemm_grouped(const uint16_t* x, const uint8_t* w_packed,
                                const uint16_t* scales, const int32_t* m_sizes,
                                uint16_t* y, int32_t G, int64_t M_total,
                                int64_t N, int64_t K, int32_t group_size,
                                float* workspace, size_t workspace_bytes,
                                void* stream);

/*
 * Bytes of workspace w4a16_gemm_batched needs at this shape and split_k (0 =
 * auto) with group_size 128: SK * B * M * N * 4 (rounded up to 256) when the
 * effective split factor SK > 1, plus (K/128) * round_up(B * M, 4) * 4 for
 * the per-row group sums of X. Returns 0 for invalid arguments or M == 0.
 * w4a16_gemm_batched_workspace_bytes_gs gives it for either group size.
 */
size_t w4a16_gemm_batched_workspace_bytes(int32_t B, int64_t M, int64_t N, int64_t K,
                                          int32_t split_k);

/*
 * Batched GEMM ("Add Triton BF16xINT4 rowwise GEMM for ROCm gfx942/gfx950",
 * Summary: the batched op beside the plain and grouped ones): B independent
 * problems of the same shape, Y[b] = X[b] . dequant(W[b])^T, in one launch
 * of the tile kernel with split-K ("Split-K without atomics").
 *   x         : [B, M, K] bf16, device
 *   w_packed  : [B, N, K/2] uint8, device
 *   scales    : [B, N, K/group_size] bf16, device
 *   y         : [B, M, N] bf16, device, written
 *   B >= 1, M >= 0 (0: W4A16_OK, nothing enqueued), B * M < 2^31, N >= 1,
 *   K >= 128, group_size 128 or 32 (tile configurations 2 to 5), K % 128 ==
 *   0; the scales of all B problems together must be smaller than 2^32
 *   bytes.
 *   split_k   : 0 (auto: the tile height and split chosen together, as for
 *               w4a16_gemm with B x ceil(M/h) row tiles per column) or 1, 2,
 *               4, 8, 16.
 *   workspace : fp32 device scratch of workspace_bytes >= the value of
 *               w4a16_gemm_batched_workspace_bytes_gs; overwritten.
 * Enqueues the per-row group sums of X, the tile kernel (weight group b =
 * problem b, its rows at b * M), and for SK > 1 the split-K reduce. Every
 * row of Y is written exactly once, no atomics: bitwise reproducible for a
 * given shape and split_k.
 */
w4a16_status w4a16_gemm_batched(const uint16_t* x, const uint8_t* w_packed,
                                const uint16_t* scales, uint16_t* y,
                                int32_t B, int64_t M, int64_t N, int64_t K,
                                int32_t group_size, int32_t split_k,
                                float* workspace, size_t workspace_bytes,
                                void* stream);

/*
 * The reduce step of split-K on its own ("Split-K without atomics"):
 *   y[m, n] = bf16_rne( ((ws[0,m,n] + ws[1,m,n]) + ws[2,m,n]) + ... )
 * summed in fp32 in slice order s = 0..SK-1.
 *   workspace : [SK, M, N] fp32, device, read only
 *   y         : [M, N] bf16, device, written
 *   1 <= split_k <= 64, M >= 0, N >= 0 (either 0: nothing enqueued).
 * w4a16_gemm calls the same kernel after its split-K slices.
 */
w4a16_status w4a16_splitk_reduce(const float* workspace, uint16_t* y,
                                 int32_t split_k, int64_t M, int64_t N,
                                 void* stream);

/*
 * Explicit kernel selection, for tests and benchmarks that must exercise a
 * particular kernel at a shape where the automatic choice would pick another.
 * The result of a forced path still satisfies the same contract.
 *   path   : 0 = automatic, 1 = M == 1 GEMV (at most 64 groups per split-K
 *            slice),
 *            2 = M <= 48 MFMA 16x16x32 small-batch kernel (one row tile of
 *            16, two past 16 rows, three past 32; automatic for M <= 16,
 *            for M <= 32 while ceil(N/32) <= 3 x compute units, for M <= 48
 *            while ceil(N/16) <= compute units), 3 = MFMA tile kernel
 *            (LDS-staged; the only path of the grouped call)
 *   variant: -1 = default for the path; otherwise
 *            path 1: 1000 * layout + layout digits.
 *              layout 2 (default, MFMA diagonal contraction of 16 groups per
 *              instruction): 2000 + 100 * h + 10 * depth + blocks, with
 *              h = 4 * x_staged_in_lds + (waves_per_workgroup / 4 - 1)
 *              (waves 4, 8, 12, 16; x held in registers otherwise),
 *              depth 1..3 = weight blocks in flight per wave, blocks 1..9 =
 *              row blocks per wave (sets the grid), 0 = one workgroup per
 *              compute unit. Combinations that would not fit the register
 *              budget of their occupancy are not built (W4A16_ERR_LAUNCH).
 *              Slice lengths with no MFMA geometry run layout 1 variant 124.
 *              layout 0 (1 KiB weight runs per wave) and layout 1 (one row
 *              per half-wave, x in registers): 100 * nt + 10 * depth + rows,
 *              nt 1 = non-temporal weight loads, depth 1..3 (layout 0) or
 *              1..4 (layout 1) = loads in flight, rows 1..9 = rows or row
 *              blocks per wave;
 *            path 2: 10 * waves_per_workgroup +
 *            column_tiles_per_wave (41, 42, 44, 81, 82, 84; default 81 for
 *            M <= 8, 82 above): waves
 *            take a column block's groups in turn; or the streaming layout
 *            1000 * u + 100 * row_tiles + 10 * units_in_flight + waves / 4,
 *            units of 4 << (u - 1) groups (one workgroup per compute unit,
 *            X of the slice staged in LDS, each wave streaming blocks of
 *            16 * row_tiles weight rows): 1121, 1131, 1122, 1222, 2121,
 *            2122, 3121, 3112, 3131; with more than 32 groups per slice it
 *            runs the default of the first form; path 3: tile
 *            configuration index (0: 128x256 and 1: 128x128 with weights
 *            dequantised into LDS; 2: 128x256 with LDS-DMA staging, 8
 *            waves, 3 LDS stages; 3, 4, 5, 6, 7, 8: the same with 96x256,
 *            112x256, 80x256, 144x256, 64x256 and 48x256 tiles; group_size
 *            32 runs on 2 to 5 only, W4A16_ERR_GROUP_SIZE otherwise). By
 *            default the call picks among 2 to 8 (2 to 5 for group_size 32)
 *            the tile height and split with the least estimated time: the
 *            rounds of one workgroup per compute unit times rows per tile, weighted by
 *            each height's measured per-row rate (the grouped call
 *            estimates ceil(M_total/h) + G/2 row tiles per column).
 * An unavailable combination (e.g. path 1 with M != 1, path 2 with M > 48,
 * with M > 16 and a variant other than 81 or 82, or with M > 32 and a
 * variant other than 81)
 * returns W4A16_ERR_SHAPE; path 1 or 2 with group_size 32 returns
 * W4A16_ERR_GROUP_SIZE.
 */
typedef struct {
  int32_t path;
  int32_t variant;
} w4a16_config;

/* w4a16_gemm_workspace_bytes for the kernel selected by cfg (NULL = auto). */
size_t w4a16_gemm_workspace_bytes_ex(int64_t M, int64_t N, int64_t K,
                                     int32_t split_k, const w4a16_config* cfg);

/* w4a16_gemm with an explicit kernel selection (cfg NULL = automatic). */
w4a16_status w4a16_gemm_ex(const uint16_t* x, const uint8_t* w_packed,
                           const uint16_t* scales, uint16_t* y,
                           int64_t M, int64_t N, int64_t K, int32_t group_size,
                           int32_t split_k, float* workspace,
                           size_t workspace_bytes, void* stream,
                           const w4a16_config* cfg);

/* w4a16_gemm_grouped with an explicit tile configuration (path must be 0 or 3). */
w4a16_status w4a16_gemm_grouped_ex(const uint16_t* x, const uint8_t* w_packed,
                                   const uint16_t* scales, const int32_t* m_sizes,
                                   uint16_t* y, int32_t G, int64_t M_total,
                                   int64_t N, int64_t K, int32_t group_size,
                                   float* workspace, size_t workspace_bytes,
                                   void* stream, const w4a16_config* cfg);

/* w4a16_gemm_batched_workspace_bytes for an explicit tile configuration. */
size_t w4a16_gemm_batched_workspace_bytes_ex(int32_t B, int64_t M, int64_t N, int64_t K,
                                             int32_t split_k, const w4a16_config* cfg);

/*
 * Workspace bytes for either group size (128 or 32; the functions above are
 * these with 128). With group_size 32 the tile kernel runs at every M and its
 * row sums take (K/32) * round_up(rows, 4) * 4 bytes. cfg NULL = automatic.
 * Return 0 for invalid arguments (including a group size the selected kernel
 * does not take) and when no workspace is needed.
 */
size_t w4a16_gemm_workspace_bytes_gs(int64_t M, int64_t N, int64_t K, int32_t group_size,
                                     int32_t split_k, const w4a16_config* cfg);
size_t w4a16_gemm_grouped_workspace_bytes_gs(int32_t G, int64_t M_total, int64_t N, int64_t K,
                                             int32_t group_size);
size_t w4a16_gemm_batched_workspace_bytes_gs(int32_t B, int64_t M, int64_t N, int64_t K,
                                             int32_t group_size, int32_t split_k,
                                             const w4a16_config* cfg);

/* w4a16_gemm_batched with an explicit tile configuration (path must be 0 or 3). */
w4a16_status w4a16_gemm_batched_ex(const uint16_t* x, const uint8_t* w_packed,
                                   const uint16_t* scales, uint16_t* y,
                                   int32_t B, int64_t M, int64_t N, int64_t K,
                                   int32_t group_size, int32_t split_k,
                                   float* workspace, size_t workspace_bytes,
                                   void* stream, const w4a16_config* cfg);

#ifdef __cplusplus
}
#endif

#endif /* W4A16_H */
