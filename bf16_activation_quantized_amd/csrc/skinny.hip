// Small-batch decode, 1 <= M <= 48: Y[M, N] with bf16 MFMA 16x16x32.
//
// X (at most 16 rows) is the 16-row A operand (rows >= M read as zero through
// the exact buffer extent); a column block of 16 * NT output columns is
// the B side, dequantised in registers from the packed weights with the
// magic-constant OR ("[ROCm][Kernel] W4A16 skinny GEMM: hand-asm kernel for
// gfx1151", section 1). The weight operand is bf16(128 + q), exact; the
// "- 136" is applied as -136 * sum(x), obtained by one extra MFMA per step
// against a constant bf16(-136) operand and used as the initial accumulator
// of every column tile in the group. The fp32 group sum is then scaled by the
// bf16 scale of its column once per 128-group.
//
// MFMA 16x16x32 lane mapping: lane l supplies row (l % 16) of A and column
// (l % 16) of B for the k-block (l / 16); since the same k-block index is
// used on both sides, any order of k inside a lane's 8 values is valid as
// long as A and B agree. Lane l reads, for group g, the 16 packed bytes of
// k in [128 g + 32 (l/16), +32): dword j of them feeds MFMA step j, in the
// pair order (0,4,1,5,2,6,3,7); A gets the same 8 x values permuted alike.
// Result: lane l holds rows 4 (l/16) + i (i = 0..3) of column (l % 16).
//
// Work split: a workgroup of WAVES waves owns a column block; its waves take
// the 128-groups of the K-slice round robin and are reduced through LDS at
// the end. A group's X is fetched in whole cache lines (4 rows x 256 bytes
// per instruction) and transposed into the MFMA layout through a per-wave
// LDS tile; the slice's scales of the block's columns are staged in LDS once.
// Fetched in the MFMA layout instead, X (16 rows x 4 pieces spread over 256
// bytes per instruction) and the scales (one line per column) cost more
// address-unit time than the weight stream itself. gridDim.y = SK slices ("Add Triton BF16xINT4 rowwise GEMM for
// ROCm gfx942/gfx950", Implementation "Split-K without atomics": fp32
// partials to ws[s, :, :] with plain stores).
#include <algorithm>

#include "common.hpp"
#include "launch.hpp"

namespace w4a16 {

__device__ __forceinline__ bf16x8 as_bf16x8(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  return __builtin_bit_cast(bf16x8, u32x4{a, b, c, d});
}

// MT: row tiles of 16 (M <= 16 MT); XR: row quads of X loaded per group
// (M <= 4 XR <= 16 MT). The A-operand rows past them are never written in
// the staging tile; they feed only output rows >= M, which are not stored.
template <int NT, int WAVES, bool SLDS, int XR = 4, int MT = 1>
__global__ __launch_bounds__(64 * WAVES) void skinny_kernel(const uint16_t* __restrict__ x,
                                                            const uint8_t* __restrict__ w,
                                                            const uint16_t* __restrict__ s,
                                                            uint16_t* __restrict__ y,
                                                            float* __restrict__ ws,
                                                            int M, int N, int K, int gps) {
  static_assert(XR >= 1 && XR <= 4 * MT && MT >= 1 && MT <= 3, "row quads within the row tiles");
  __shared__ f32x4 red[WAVES > 1 ? (WAVES - 1) : 1][MT][NT][64];
  // per-wave staging of one group of X: [16 MT rows][16 slots of 16 bytes],
  // the piece p of row r in slot p ^ (r & 15) (conflict-free for both access
  // patterns)
  __shared__ u32x4 xst[WAVES][16 * 16 * MT];
  // SLDS: the slice's scales of the workgroup's 16 NT columns, [column][group]
  // (dynamic size 16 NT x gps x 2 bytes), fetched once in whole lines; per
  // group the lanes then read LDS instead of one line per column
  extern __shared__ uint16_t scl[];

  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int col = lane & 15;
  const int kb = lane >> 4;
  const int G = K / kGroup;
  const int slice = blockIdx.y;
  const int g0 = slice * gps;
  const int g1 = min(G, g0 + gps);
  const int nb = blockIdx.x * 16 * NT;
  const int gs = g1 > g0 ? g1 - g0 : 0;

  const __amdgpu_buffer_rsrc_t rx = make_rsrc(x, (uint32_t)M * (uint32_t)K * 2u);
  const __amdgpu_buffer_rsrc_t rw = make_rsrc(w, (uint32_t)((uint64_t)N * (uint32_t)K / 2u));
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(s, (uint32_t)N * (uint32_t)G * 2u);

  // per-lane row bases. X is fetched in whole cache lines: load j of a group
  // covers rows 4 j .. 4 j + 3, lane l reading 16-byte piece l % 16 of row
  // 4 j + l / 16 (a fetch in the MFMA layout would touch 32 partly used lines
  // per instruction); the wave then transposes the group through LDS.
  const uint32_t xrow = (uint32_t)(lane >> 4) * (uint32_t)K * 2u + 16u * (uint32_t)(lane & 15);
  const uint32_t xrow4 = 4u * (uint32_t)K * 2u;
  uint32_t wrow[NT], srow[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const uint32_t n = (uint32_t)(nb + 16 * t + col);
    wrow[t] = n * (uint32_t)(K / 2) + (uint32_t)kb * 16u;
    srow[t] = n * (uint32_t)G * 2u;
  }

  const uint32_t neg136 = 0xC308C308u;   // bf16(-136) pair
  const bf16x8 bneg = as_bf16x8(neg136, neg136, neg136, neg136);

  f32x4 acc[MT][NT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[mt][t] = f32x4{0.f, 0.f, 0.f, 0.f};

  // double-buffered loads: x (4 x 16 B), weights (NT x 16 B), scales (NT).
  // Two named buffer sets, so that no register array is indexed at run time.
  u32x4 xb0[XR], xb1[XR];
  u32x4 wb0[NT], wb1[NT];
  uint16_t sb0[NT], sb1[NT];
  auto issue = [&](u32x4 (&xb)[XR], u32x4 (&wb)[NT], uint16_t (&sb)[NT], int g) {
    const uint32_t xo = xrow + (uint32_t)g * 256u;
#pragma unroll
    for (int j = 0; j < XR; ++j) xb[j] = ld128(rx, xo + xrow4 * (uint32_t)j);
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      wb[t] = ld128(rw, wrow[t] + (uint32_t)g * 64u);
      if constexpr (!SLDS) sb[t] = ld16(rs, srow[t] + (uint32_t)g * 2u);
      else sb[t] = (uint16_t)(16 * t + col) * (uint16_t)gs + (uint16_t)(g - g0);   // LDS index
    }
  };
  auto compute = [&](const u32x4 (&xb)[XR], const u32x4 (&wb)[NT], const uint16_t (&sb)[NT]) {
    u32x4* xw = xst[wave];
    wave_lds_exchange();   // after the previous group's reads of the tile
#pragma unroll
    for (int j = 0; j < XR; ++j) {
      const int r = 4 * j + (lane >> 4), pc = lane & 15;
      xw[16 * r + (pc ^ (r & 15))] = xb[j];
    }
    wave_lds_exchange();   // the pieces read below were written by other lanes
    if constexpr (MT == 1) {
      bf16x8 a[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        // row m = col, piece 4 kb + j: k = 128 g + 32 kb + 8 j + 0..7
        const u32x4 v = xw[16 * col + ((4 * kb + j) ^ col)];
        a[j] = as_bf16x8(__builtin_amdgcn_perm(v.z, v.x, 0x05040100u), __builtin_amdgcn_perm(v.z, v.x, 0x07060302u),
                         __builtin_amdgcn_perm(v.w, v.y, 0x05040100u), __builtin_amdgcn_perm(v.w, v.y, 0x07060302u));
      }
      // -136 * sum of this group's x for the lane's 4 output rows
      f32x4 c0 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < 4; ++j) c0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[j], bneg, c0, 0, 0, 0);
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const u32x4 wv = wb[t];
        const uint32_t wd[4] = {wv.x, wv.y, wv.z, wv.w};
        f32x4 tmp = c0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const bf16x8 b = as_bf16x8(magic_pair_interleaved(wd[j], 0), magic_pair_interleaved(wd[j], 1),
                                     magic_pair_interleaved(wd[j], 2), magic_pair_interleaved(wd[j], 3));
          tmp = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[j], b, tmp, 0, 0, 0);
        }
        const float sc = bf16f(SLDS ? scl[sb[t]] : sb[t]);
        acc[0][t].x = fmaf(sc, tmp.x, acc[0][t].x);
        acc[0][t].y = fmaf(sc, tmp.y, acc[0][t].y);
        acc[0][t].z = fmaf(sc, tmp.z, acc[0][t].z);
        acc[0][t].w = fmaf(sc, tmp.w, acc[0][t].w);
      }
    } else {
      // two row tiles: the weight operands are dequantised once for both
      bf16x8 bw[NT][4];
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const u32x4 wv = wb[t];
        const uint32_t wd[4] = {wv.x, wv.y, wv.z, wv.w};
#pragma unroll
        for (int j = 0; j < 4; ++j)
          bw[t][j] = as_bf16x8(magic_pair_interleaved(wd[j], 0), magic_pair_interleaved(wd[j], 1),
                               magic_pair_interleaved(wd[j], 2), magic_pair_interleaved(wd[j], 3));
      }
      float sc[NT];
#pragma unroll
      for (int t = 0; t < NT; ++t) sc[t] = bf16f(SLDS ? scl[sb[t]] : sb[t]);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        bf16x8 a[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          // row m = 16 mt + col, piece 4 kb + j
          const u32x4 v = xw[16 * (16 * mt + col) + ((4 * kb + j) ^ col)];
          a[j] = as_bf16x8(__builtin_amdgcn_perm(v.z, v.x, 0x05040100u), __builtin_amdgcn_perm(v.z, v.x, 0x07060302u),
                           __builtin_amdgcn_perm(v.w, v.y, 0x05040100u), __builtin_amdgcn_perm(v.w, v.y, 0x07060302u));
        }
        f32x4 c0 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < 4; ++j) c0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[j], bneg, c0, 0, 0, 0);
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          f32x4 tmp = c0;
#pragma unroll
          for (int j = 0; j < 4; ++j) tmp = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[j], bw[t][j], tmp, 0, 0, 0);
          acc[mt][t].x = fmaf(sc[t], tmp.x, acc[mt][t].x);
          acc[mt][t].y = fmaf(sc[t], tmp.y, acc[mt][t].y);
          acc[mt][t].z = fmaf(sc[t], tmp.z, acc[mt][t].z);
          acc[mt][t].w = fmaf(sc[t], tmp.w, acc[mt][t].w);
        }
      }
    }
  };

  int g = g0 + wave;
  if constexpr (SLDS) {
    // scales first (the wait for them then covers nothing else), then the
    // wave's first two groups, then the scales go to LDS
    constexpr int kB = 16;               // loads per batch
    const int per_col = (gs + 63) / 64;  // 64-scale chunks per column
    const int items = (16 * NT / WAVES) * per_col;
    uint16_t sv[kB];
    auto sc_item = [&](int it, int& c, int& gi) {
      c = wave + WAVES * (it / per_col);
      gi = 64 * (it % per_col) + lane;
    };
#pragma unroll
    for (int b = 0; b < kB; ++b) {
      int c, gi;
      sc_item(b, c, gi);
      sv[b] = b < items && gi < gs ? ld16(rs, ((uint32_t)(nb + c) * (uint32_t)G + (uint32_t)(g0 + gi)) * 2u) : 0;
    }
    __builtin_amdgcn_sched_barrier(0);
    if (g < g1) issue(xb0, wb0, sb0, g);
    if (g + WAVES < g1) issue(xb1, wb1, sb1, g + WAVES);
#pragma unroll
    for (int b = 0; b < kB; ++b) {
      int c, gi;
      sc_item(b, c, gi);
      if (b < items && gi < gs) scl[c * gs + gi] = sv[b];
    }
    for (int it0 = kB; it0 < items; it0 += kB) {
#pragma unroll
      for (int b = 0; b < kB; ++b) {
        int c, gi;
        sc_item(it0 + b, c, gi);
        if (it0 + b < items && gi < gs) scl[c * gs + gi] = ld16(rs, ((uint32_t)(nb + c) * (uint32_t)G + (uint32_t)(g0 + gi)) * 2u);
      }
    }
    __syncthreads();
    while (g < g1) {
      compute(xb0, wb0, sb0);
      if (g + 2 * WAVES < g1) issue(xb0, wb0, sb0, g + 2 * WAVES);
      g += WAVES;
      if (g >= g1) break;
      compute(xb1, wb1, sb1);
      if (g + 2 * WAVES < g1) issue(xb1, wb1, sb1, g + 2 * WAVES);
      g += WAVES;
    }
  } else {
    if (g < g1) issue(xb0, wb0, sb0, g);
    while (g < g1) {
      if (g + WAVES < g1) issue(xb1, wb1, sb1, g + WAVES);
      compute(xb0, wb0, sb0);
      g += WAVES;
      if (g >= g1) break;
      if (g + WAVES < g1) issue(xb0, wb0, sb0, g + WAVES);
      compute(xb1, wb1, sb1);
      g += WAVES;
    }
  }

  // cross-wave reduction: waves 1.. park their tiles in LDS, wave 0 sums
  if (WAVES > 1) {
    if (wave > 0) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int t = 0; t < NT; ++t) red[wave - 1][mt][t][lane] = acc[mt][t];
    }
    __syncthreads();
    if (wave != 0) return;
#pragma unroll
    for (int v = 0; v < WAVES - 1; ++v) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          const f32x4 p = red[v][mt][t][lane];
          acc[mt][t].x += p.x;
          acc[mt][t].y += p.y;
          acc[mt][t].z += p.z;
          acc[mt][t].w += p.w;
        }
    }
  }

#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int n = nb + 16 * t + col;
      if (n >= N) continue;
      const float vals[4] = {acc[mt][t].x, acc[mt][t].y, acc[mt][t].z, acc[mt][t].w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = 16 * mt + 4 * kb + i;
        if (m < M) {
          if (ws == nullptr) y[(size_t)m * N + n] = to_bf16(vals[i]);
          else ws[((size_t)slice * M + m) * N + n] = vals[i];
        }
      }
    }
}

template <int NT, int WV, int XR, int MT = 1>
static hipError_t launch_skinny_t(const uint16_t* x, const uint8_t* w, const uint16_t* s, uint16_t* y, float* ws,
                                  int M, int N, int K, int gps, int sk, hipStream_t stream) {
  dim3 grid((N + 16 * NT - 1) / (16 * NT), sk);
  // scales staged in LDS while the slice's scale block stays small
  if (gps <= kSkinnyMaxScaleGroups) {
    const size_t dyn = ((size_t)16 * NT * gps * 2 + 15) & ~(size_t)15;
    static std::atomic<uint64_t> lds_set{0};   // per instantiation and device
    const hipError_t ea = ensure_dyn_lds(reinterpret_cast<const void*>(&skinny_kernel<NT, WV, true, XR, MT>),
                                         16 * NT * kSkinnyMaxScaleGroups * 2, lds_set);
    if (ea != hipSuccess) return ea;
    hipLaunchKernelGGL((skinny_kernel<NT, WV, true, XR, MT>), grid, dim3(64 * WV), dyn, stream, x, w, s, y, ws, M,
                       N, K, gps);
  } else {
    hipLaunchKernelGGL((skinny_kernel<NT, WV, false, XR, MT>), grid, dim3(64 * WV), 0, stream, x, w, s, y, ws, M, N,
                       K, gps);
  }
  return hipGetLastError();
}

hipError_t launch_skinny(const uint16_t* x, const uint8_t* w, const uint16_t* s, uint16_t* y, float* ws,
                         int M, int N, int K, int gps, int sk, int nt, int waves, hipStream_t stream) {
  if (M < 1 || M > kSkinnyMaxRows) return hipErrorInvalidValue;
  // only the row quads of X that hold rows < M are loaded; two row tiles of
  // 16 past 16 rows (8 waves of 1 or 2 column tiles), three past 32 rows (8
  // waves of 1 column tile)
#define W4A16_SKINNY(NTT, WV)                                                                           \
  if (nt == NTT && waves == WV) {                                                                       \
    if (M <= 4) return launch_skinny_t<NTT, WV, 1>(x, w, s, y, ws, M, N, K, gps, sk, stream);          \
    if (M <= 8) return launch_skinny_t<NTT, WV, 2>(x, w, s, y, ws, M, N, K, gps, sk, stream);          \
    if (M <= 12) return launch_skinny_t<NTT, WV, 3>(x, w, s, y, ws, M, N, K, gps, sk, stream);         \
    if (M <= 16) return launch_skinny_t<NTT, WV, 4>(x, w, s, y, ws, M, N, K, gps, sk, stream);         \
    if constexpr (WV == 8 && NTT <= 2) {                                                               \
      if (M <= 24) return launch_skinny_t<NTT, WV, 6, 2>(x, w, s, y, ws, M, N, K, gps, sk, stream);    \
      if (M <= 32) return launch_skinny_t<NTT, WV, 8, 2>(x, w, s, y, ws, M, N, K, gps, sk, stream);    \
      if constexpr (NTT == 1) { /* three row tiles: one column tile fits the registers */               \
        if (M <= 40) return launch_skinny_t<NTT, WV, 10, 3>(x, w, s, y, ws, M, N, K, gps, sk, stream); \
        return launch_skinny_t<NTT, WV, 12, 3>(x, w, s, y, ws, M, N, K, gps, sk, stream);              \
      }                                                                                                 \
    }                                                                                                   \
    return hipErrorInvalidValue;                                                                        \
  }
  W4A16_SKINNY(1, 8)
  W4A16_SKINNY(2, 8)
#undef W4A16_SKINNY
  return hipErrorInvalidValue;
}

}  // namespace w4a16
