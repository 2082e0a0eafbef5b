// Small-batch decode, 1 <= M <= 16: Y[M, N] with bf16 MFMA 16x16x32.
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
// the end. gridDim.y = SK slices ("Add Triton BF16xINT4 rowwise GEMM for
// ROCm gfx942/gfx950", Implementation "Split-K without atomics": fp32
// partials to ws[s, :, :] with plain stores).
#include "common.hpp"
#include "launch.hpp"

namespace w4a16 {

__device__ __forceinline__ bf16x8 as_bf16x8(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  return __builtin_bit_cast(bf16x8, u32x4{a, b, c, d});
}

template <int NT, int WAVES>
__global__ __launch_bounds__(64 * WAVES) void skinny_kernel(const uint16_t* __restrict__ x,
                                                            const uint8_t* __restrict__ w,
                                                            const uint16_t* __restrict__ s,
                                                            uint16_t* __restrict__ y,
                                                            float* __restrict__ ws,
                                                            int M, int N, int K, int gps) {
  __shared__ f32x4 red[WAVES > 1 ? (WAVES - 1) : 1][NT][64];

  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int col = lane & 15;
  const int kb = lane >> 4;
  const int G = K / kGroup;
  const int slice = blockIdx.y;
  const int g0 = slice * gps;
  const int g1 = min(G, g0 + gps);
  const int nb = blockIdx.x * 16 * NT;

  const __amdgpu_buffer_rsrc_t rx = make_rsrc(x, (uint32_t)M * (uint32_t)K * 2u);
  const __amdgpu_buffer_rsrc_t rw = make_rsrc(w, (uint32_t)((uint64_t)N * (uint32_t)K / 2u));
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(s, (uint32_t)N * (uint32_t)G * 2u);

  // per-lane row bases
  const uint32_t xrow = (uint32_t)col * (uint32_t)K * 2u + (uint32_t)kb * 64u;   // row m = col
  uint32_t wrow[NT], srow[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const uint32_t n = (uint32_t)(nb + 16 * t + col);
    wrow[t] = n * (uint32_t)(K / 2) + (uint32_t)kb * 16u;
    srow[t] = n * (uint32_t)G * 2u;
  }

  const uint32_t neg136 = 0xC308C308u;   // bf16(-136) pair
  const bf16x8 bneg = as_bf16x8(neg136, neg136, neg136, neg136);

  f32x4 acc[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};

  // double-buffered loads: x (4 x 16 B), weights (NT x 16 B), scales (NT).
  // Two named buffer sets, so that no register array is indexed at run time.
  u32x4 xb0[4], xb1[4];
  u32x4 wb0[NT], wb1[NT];
  uint16_t sb0[NT], sb1[NT];
  auto issue = [&](u32x4 (&xb)[4], u32x4 (&wb)[NT], uint16_t (&sb)[NT], int g) {
    const uint32_t xo = xrow + (uint32_t)g * 256u;
#pragma unroll
    for (int j = 0; j < 4; ++j) xb[j] = ld128(rx, xo + 16u * j);
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      wb[t] = ld128(rw, wrow[t] + (uint32_t)g * 64u);
      sb[t] = ld16(rs, srow[t] + (uint32_t)g * 2u);
    }
  };
  auto compute = [&](const u32x4 (&xb)[4], const u32x4 (&wb)[NT], const uint16_t (&sb)[NT]) {
    bf16x8 a[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const u32x4 v = xb[j];
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
      const float sc = bf16f(sb[t]);
      acc[t].x = fmaf(sc, tmp.x, acc[t].x);
      acc[t].y = fmaf(sc, tmp.y, acc[t].y);
      acc[t].z = fmaf(sc, tmp.z, acc[t].z);
      acc[t].w = fmaf(sc, tmp.w, acc[t].w);
    }
  };

  int g = g0 + wave;
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

  // cross-wave reduction: waves 1.. park their tiles in LDS, wave 0 sums
  if (WAVES > 1) {
    if (wave > 0) {
#pragma unroll
      for (int t = 0; t < NT; ++t) red[wave - 1][t][lane] = acc[t];
    }
    __syncthreads();
    if (wave != 0) return;
#pragma unroll
    for (int v = 0; v < WAVES - 1; ++v) {
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const f32x4 p = red[v][t][lane];
        acc[t].x += p.x;
        acc[t].y += p.y;
        acc[t].z += p.z;
        acc[t].w += p.w;
      }
    }
  }

#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int n = nb + 16 * t + col;
    if (n >= N) continue;
    const float vals[4] = {acc[t].x, acc[t].y, acc[t].z, acc[t].w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = 4 * kb + i;
      if (m < M) {
        if (ws == nullptr) y[(size_t)m * N + n] = to_bf16(vals[i]);
        else ws[((size_t)slice * M + m) * N + n] = vals[i];
      }
    }
  }
}

hipError_t launch_skinny(const uint16_t* x, const uint8_t* w, const uint16_t* s, uint16_t* y, float* ws,
                         int M, int N, int K, int gps, int sk, int nt, int waves, hipStream_t stream) {
#define W4A16_SKINNY(NTT, WV)                                                                      \
  if (nt == NTT && waves == WV) {                                                                  \
    dim3 grid((N + 16 * NTT - 1) / (16 * NTT), sk);                                                \
    hipLaunchKernelGGL((skinny_kernel<NTT, WV>), grid, dim3(64 * WV), 0, stream, x, w, s, y, ws, M, \
                       N, K, gps);                                                                 \
    return hipGetLastError();                                                                      \
  }
  W4A16_SKINNY(1, 4)
  W4A16_SKINNY(2, 4)
  W4A16_SKINNY(4, 4)
  W4A16_SKINNY(1, 8)
  W4A16_SKINNY(2, 8)
  W4A16_SKINNY(4, 8)
#undef W4A16_SKINNY
  return hipErrorInvalidValue;
}

}  // namespace w4a16
