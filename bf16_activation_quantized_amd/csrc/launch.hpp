// Host-side launchers of the device kernels (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

namespace w4a16 {

// Raises a kernel's dynamic-LDS limit to `bytes` on the current device, once
// per device: `done` is the caller's per-kernel set of devices already set
// (bit d = device d; a device index past 63 sets it on every call).
inline hipError_t ensure_dyn_lds(const void* fn, int bytes, std::atomic<uint64_t>& done) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) dev = -1;
  const uint64_t bit = (dev >= 0 && dev < 64) ? (uint64_t{1} << dev) : 0;
  if (bit != 0 && (done.load(std::memory_order_acquire) & bit) != 0) return hipSuccess;
  const hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e == hipSuccess && bit != 0) done.fetch_or(bit, std::memory_order_release);
  return e;
}

hipError_t launch_pack_int4(const uint8_t* q, uint8_t* out, uint64_t total_in, hipStream_t stream);
hipError_t launch_splitk_reduce(const float* ws, uint16_t* y, uint64_t mn, int sk, hipStream_t stream);

// M = 1 decode GEMV; gps = 128-groups per split-K slice (<= 64), sk slices;
// ws == nullptr writes bf16 y, else fp32 partials ws[s, 0, :]. The MFMA layout
// where the slice length has a tiling of 16 (row, group) pairs per
// instruction, otherwise (or when forced) the half-wave layout.
hipError_t launch_gemv_m1(const uint16_t* x, const uint8_t* w, const uint16_t* s, uint16_t* y, float* ws,
                          int N, int K, int gps, int sk, bool force_halfwave, hipStream_t stream);

// 1 <= M <= kSkinnyMaxRows decode on MFMA 16x16x32; nt column tiles of 16 per
// wave (1 or 2), 8 waves per workgroup (past 32 rows only nt = 1).
hipError_t launch_skinny(const uint16_t* x, const uint8_t* w, const uint16_t* s, uint16_t* y, float* ws,
                         int M, int N, int K, int gps, int sk, int nt, int waves, hipStream_t stream);

// 1 <= M <= 16 decode with X and the weights staged in LDS by DMA (skinny_lds.hip)
bool skinny_lds_fits(int M, int gps);
hipError_t launch_skinny_lds(const uint16_t* x, const uint8_t* w, const uint16_t* s, uint16_t* y, float* ws, int M,
                             int N, int K, int gps, int sk, int geometry, hipStream_t stream);

// slices of at most this many groups stage their scales in LDS (16 NT x gps x 2
// bytes, at most 32 KiB)
constexpr int kSkinnyMaxScaleGroups = 256;
// rows of the small-batch kernel: 16 per row tile, two or three row tiles
// with 8 waves of 1 or 2 column tiles
constexpr int kSkinnyMaxRows = 48;

// out[g * ld + m] = -136 * sum_{k in group g} x[m, k], groups of gsize = 128 or 32 k
hipError_t launch_rowsum_neg136(const uint16_t* x, float* out, int M, int K, int ld, int gsize,
                                hipStream_t stream);

// LDS-DMA tile GEMM with bm x 256 output tiles (bm = 48 .. 144 rows in steps
// of 16; scale groups of gsize = 128 or 32 k, see tile_rows_ok): plain
// (m_sizes == nullptr, m_uniform == 0, G == 1), grouped (rows per weight group
// in m_sizes on the device) or batched (G weight groups of m_uniform rows
// each). With ws != nullptr (plain and batched) slice s of gridDim.y = sk
// writes fp32 partials ws[s, :, :]. sxn: the -136 * row sums [K/gsize, ld] of
// launch_rowsum_neg136, or nullptr for the kernel to form them itself.
hipError_t launch_tile(const uint16_t* x, const uint8_t* w, const uint16_t* s, const float* sxn, int ld, uint16_t* y,
                       float* ws, const int32_t* m_sizes, int m_uniform, int M_total, int N, int K, int G, int gps,
                       int sk, int bm, int gsize, hipStream_t stream);
// whether the tile kernel is built for bm-row tiles at scale group gsize
bool tile_rows_ok(int bm, int gsize);
constexpr int kTileCols = 256;

}  // namespace w4a16
