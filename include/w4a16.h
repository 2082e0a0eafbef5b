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
 * The split-K factor w4a16_gemm uses at this shape and group size when
 * split_k == 0 (auto): for the M = 1 GEMV only what its register budget for x
 * needs (at most 64 groups per slice), for the M <= 48 kernel slices only
 * while fewer than half of the compute units have a workgroup, and for the
 * tile kernel the power of two (at most 16) of least estimated time among
 * those that keep tiles x SK within one workgroup per compute unit, counting
 * the fp32 partials and the reduce, chosen together with the tile height
 * (so, unlike the MI350X Triton page's prune of split-K at M >= 512, a
 * tall-K shape with few tiles splits at any M). Returns 0 on invalid
 * arguments.
 */
int32_t w4a16_gemm_auto_split_k(int64_t M, int64_t N, int64_t K, int32_t group_size);

/*
 * Bytes of workspace w4a16_gemm uses at this shape and split_k (0 = auto)
 * with group_size 128 (w4a16_gemm_workspace_bytes_gs: either group size):
 *  - SK * M * N * 4, rounded up to 256, for the split-K partials when the
 *    effective split factor SK is above 1 (required);
 *  - plus, on the tile kernel (M > 48, or group size 32 at any M) with a wide
 *    N (at least 32 column tiles of 256 at group 128, 8 at group 32),
 *    (K/group_size) * round_up(M, 4) * 4 for the -136 * row sums of X from a
 *    pre-pass kernel (optional: with less room, or a NULL workspace at SK 1,
 *    the tile kernel forms the row sums itself, which costs more time once
 *    many column tiles repeat them).
 * Returns 0 when no workspace is used and for invalid arguments.
 */
size_t w4a16_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K,
                                  int32_t split_k);
size_t w4a16_gemm_workspace_bytes_gs(int64_t M, int64_t N, int64_t K,
                                     int32_t group_size, int32_t split_k);

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
 *               runs the tile kernel, at any M: the M = 1 and M <= 48 kernels
 *               take 128-groups only.
 *   split_k   : 0 = auto, or 1, 2, 4, 8, 16. With SK > 1 the K range is cut
 *               into SK contiguous slices of ceil((K/128)/SK) blocks of 128 k
 *               (trailing slices may be empty); slice s writes its fp32
 *               partial sums to workspace[s, :, :] with plain stores (an
 *               empty slice writes zeros) and a second kernel sums the slices
 *               in order s = 0..SK-1 in fp32 and rounds once to bf16
 *               ("Add Triton BF16xINT4 rowwise GEMM for ROCm gfx942/gfx950",
 *               Implementation "Split-K without atomics").
 *   workspace : fp32 device scratch, overwritten, or NULL. Required when the
 *               effective SK is above 1: its first SK * M * N floats then hold
 *               the [SK, M, N] partials after the call. Where
 *               w4a16_gemm_workspace_bytes_gs also counts row sums and the
 *               workspace has that room, a pre-pass kernel writes the
 *               -136 * row sums of X after the partials (256-byte aligned)
 *               and the tile kernel reads them; otherwise the tile kernel
 *               forms them itself (same results).
 *   workspace_bytes: its size in bytes (with SK > 1 at least the rounded
 *               partials, else W4A16_ERR_WORKSPACE).
 * Rows of Y are written exactly once; no atomics are used, so the result is
 * bitwise reproducible for a given shape and split_k.
 */
w4a16_status w4a16_gemm(const uint16_t* x, const uint8_t* w_packed,
                        const uint16_t* scales, uint16_t* y,
                        int64_t M, int64_t N, int64_t K, int32_t group_size,
                        int32_t split_k, float* workspace,
                        size_t workspace_bytes, void* stream);

/*
 * w4a16_gemm for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same computation and kernels, with the workspace replaced by a scratch
 * array inside the library, W4A16_NOALLOC_SCRATCH_BYTES bytes per GPU, held
 * from the library's first use on that GPU until the process ends. The call
 * allocates nothing (no hipMalloc, hipFree or allocating library routine).
 *   Arguments as for w4a16_gemm, without workspace and workspace_bytes.
 *   The split-K partials (SK * M * N * 4 bytes, rounded up to 256, when the
 *   effective SK is above 1) must fit the scratch, else W4A16_ERR_WORKSPACE
 *   is returned before anything is enqueued; the pre-pass row sums are used
 *   where they fit beside them (else the tile kernel forms them). Every byte
 *   of scratch a call reads is first written by that call.
 *   All calls on one GPU share its scratch: calls that overlap in time on one
 *   GPU (different streams, or different host threads without ordering) race
 *   and give undefined results; calls ordered on one stream are safe.
 * The kernels are those w4a16_gemm runs with a workspace of
 * w4a16_gemm_workspace_bytes_gs bytes (when that fits the scratch): the same
 * results, bit for bit.
 */
#define W4A16_NOALLOC_SCRATCH_BYTES (16u << 20)
w4a16_status w4a16_gemm_noalloc(const uint16_t* x, const uint8_t* w_packed,
                                const uint16_t* scales, uint16_t* y,
                                int64_t M, int64_t N, int64_t K, int32_t group_size,
                                int32_t split_k, void* stream);

/*
 * Grouped GEMM in one launch ("Add Triton BF16xINT4 rowwise GEMM for ROCm
 * gfx942/gfx950", Implementation "Native fused grouped kernel"): for each
 * group g with
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
 *   group_size 128 or 32, K % 128 == 0; the scales of all groups together
 *   must be smaller than 2^32 bytes.
 * One kernel is enqueued; it needs no workspace. Its grid is sized from the
 * host value M_total: (ceil(M_total/BM) + G) * ceil(N/256) workgroups for a
 * tile height BM chosen on the host; each workgroup counts the real tiles
 * from m_sizes on the device, and those past the last one exit at once.
 */
w4a16_status w4a16_gemm_grouped(const uint16_t* x, const uint8_t* w_packed,
                                const uint16_t* scales, const int32_t* m_sizes,
                                uint16_t* y, int32_t G, int64_t M_total,
                                int64_t N, int64_t K, int32_t group_size,
                                void* stream);

/*
 * Bytes of workspace w4a16_gemm_batched uses at this shape, group size and
 * split_k (0 = auto): SK * B * M * N * 4, rounded up to 256, when the
 * effective split factor SK is above 1 (required), plus the optional
 * pre-pass row sums (K/group_size) * round_up(B * M, 4) * 4 for a wide N, as
 * for w4a16_gemm. Returns 0 when none is used, for invalid arguments or
 * M == 0.
 */
size_t w4a16_gemm_batched_workspace_bytes(int32_t B, int64_t M, int64_t N, int64_t K,
                                          int32_t group_size, int32_t split_k);

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
 *   K >= 128, group_size 128 or 32, K % 128 == 0; the scales of all B
 *   problems together must be smaller than 2^32 bytes.
 *   split_k   : 0 (auto: the tile height and split chosen together, as for
 *               w4a16_gemm with B x ceil(M/h) row tiles per column) or 1, 2,
 *               4, 8, 16.
 *   workspace : fp32 device scratch, overwritten, or NULL when SK is 1
 *               (same layout and rules as for w4a16_gemm).
 * Enqueues the tile kernel (weight group b = problem b, its rows at b * M),
 * preceded by the row-sum pre-pass where the workspace has room for it (as
 * for w4a16_gemm), and, for SK > 1, the split-K reduce. Every row of Y is written exactly
 * once, no atomics: bitwise reproducible for a given shape and split_k.
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

#ifdef __cplusplus
}
#endif

#endif /* W4A16_H */
