// Small-batch decode, 1 <= M <= 16, with the operands staged in LDS by DMA.
//
// Same contraction as skinny.hip (MFMA 16x16x32 bf16, X the 16-row A operand,
// the weight columns the B operand as bf16(128 + q) from the magic-constant
// OR of "[ROCm][Kernel] W4A16 skinny GEMM: hand-asm kernel for gfx1151",
// section 1; each 128-group's chain starts from -136 * sum(x), formed by an
// MFMA against a constant bf16(-136) operand, and is scaled once per group),
// organised for the memory system instead of the register file:
//  * a workgroup (8 waves) owns 32 output columns; the K range of its slice is
//    streamed in stages of 8 groups: X [16 rows, 1024 k] (32 KiB) and the
//    packed weights [32 rows, 512 B] (16 KiB) go global -> LDS by buffer loads
//    that write LDS directly, 1 KiB of one X row or 512 B of one weight row
//    per wave instruction (contiguous runs), two stages ahead of the compute;
//  * every X row and weight row is read once per workgroup (the register
//    layout of skinny.hip re-reads X per wave and group and reads 16 weight
//    rows x 64 B per instruction);
//  * 16-byte chunks are XOR-swizzled by row (chunk c of row r in slot
//    c ^ xswz(r & 15)) so that the MFMA operand reads of 16 rows are free of
//    bank conflicts; the DMA lanes fetch the chunk that belongs in their slot;
//  * per stage the 2 column tiles x 8 groups are 16 units, two per wave; a
//    unit is one group of one column tile: 4 MFMA steps whose k order is
//    permuted alike on both sides (lane (r, kb) of step st holds k = 32 kb +
//    8 st + 0..7: one 16-byte LDS read of packed weights serves the 4 steps);
//  * the scales come with each stage (one DMA of the 32-bit words holding the
//    stage's 32 x 8 scales);
//  * the four waves of a column tile are summed through LDS at the end, in
//    wave order.
// gridDim.y = SK slices of the K range ("Add Triton BF16xINT4 rowwise GEMM for
// ROCm gfx942/gfx950", Implementation "Split-K without atomics": fp32 partials
// to ws[s, :, :] with plain stores; an empty slice writes zeros).
#include "common.hpp"
#include "launch.hpp"

namespace w4a16 {

namespace {

constexpr int kSLWaves = 8;
constexpr int kSLCols = 32;                         // output columns per workgroup

// Stage geometry for SG 128-groups per stage (SG = 4 or 8)
template <int SG>
struct SLStage {
  static constexpr int kX = 16 * SG * 256;          // X: 16 rows x SG groups x 256 B
  static constexpr int kW = kSLCols * SG * 64;      // packed W: 32 rows x SG groups x 64 B
  static constexpr int kS = kSLCols * SG * 4;       // scales: the 32-bit word holding each, [32][SG]
  static constexpr int kBytes = kX + kW + kS;
  static constexpr int kXI = 16 * SG * 256 / 1024 / kSLWaves;   // X DMA instructions per wave
  static constexpr int kWI = kSLCols * SG * 64 / 1024 / kSLWaves;   // W DMA instructions per wave
  static constexpr int kSW = kSLCols * SG * 4 / 256;            // waves with a scale DMA instruction
};

__device__ __forceinline__ void sl_dma16(__amdgpu_buffer_rsrc_t r, uint8_t* lds_dst, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds_dst, 16, voff, 0, 0, 0);
}
// the same with the non-temporal hint, for the weights: read once, streamed
// past the caches (16 x 8192 x 8192: 12.36 -> 12.07 us; the tile kernel,
// whose weight columns are re-read by other row tiles from L2, ran 3-17 %
// slower with it)
__device__ __forceinline__ void sl_dma16nt(__amdgpu_buffer_rsrc_t r, uint8_t* lds_dst, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds_dst, 16, voff, 0, 0, 2);
}
__device__ __forceinline__ void sl_dma4(__amdgpu_buffer_rsrc_t r, uint8_t* lds_dst, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds_dst, 4, voff, 0, 0, 0);
}

// s_waitcnt on the vector-memory counter only, then a workgroup barrier
template <int VM>
__device__ __forceinline__ void sl_wait_barrier() {
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(VM) : "memory");
}

// barrier after a wait that leaves `later` stages of PER DMA instructions each
// in flight (later = 0 .. MAXL)
template <int PER, int MAXL>
__device__ __forceinline__ void wait_stages(int later) {
  if constexpr (MAXL >= 4) {
    if (later >= 4) { sl_wait_barrier<4 * PER>(); return; }
  }
  if constexpr (MAXL >= 3) {
    if (later == 3) { sl_wait_barrier<3 * PER>(); return; }
  }
  if constexpr (MAXL >= 2) {
    if (later == 2) { sl_wait_barrier<2 * PER>(); return; }
  }
  if (later == 1) { sl_wait_barrier<PER>(); return; }
  sl_wait_barrier<0>();
}

}  // namespace

template <int SG, int NS>
__global__ __launch_bounds__(64 * kSLWaves) void skinny_lds_kernel(const uint16_t* __restrict__ x,
                                                                   const uint8_t* __restrict__ w,
                                                                   const uint16_t* __restrict__ s,
                                                                   void* __restrict__ out, int M, int N, int K,
                                                                   int gps) {
  using ST = SLStage<SG>;
  static_assert(SG == 4 || SG == 8, "groups per stage");
  static_assert(NS >= 3, "stages");
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int m16 = lane & 15, kb = lane >> 4;
  const uint32_t xs = xswz(m16);   // this lane's row swizzle in both operands
  const int G = K / kGroup;
  const int slice = blockIdx.y;
  const int gb = slice * gps;
  const int ge = min(G, gb + gps);
  const int ng = ge > gb ? ge - gb : 0;
  const int nst = (ng + SG - 1) / SG;
  const int n0 = blockIdx.x * kSLCols;
  const int ncols = min(kSLCols, N - n0);

  const uint32_t KB = (uint32_t)K * 2u;   // bytes per X row
  const uint32_t K2 = (uint32_t)K / 2u;   // bytes per packed weight row
  const __amdgpu_buffer_rsrc_t rx = make_rsrc(x, (uint32_t)M * KB);
  const __amdgpu_buffer_rsrc_t rw = make_rsrc(w + (size_t)n0 * K2, (uint32_t)ncols * K2);
  // scales: the whole tensor, read as the aligned word holding each (columns
  // past N read other scales or zeros and are never stored)
  const __amdgpu_buffer_rsrc_t rs = make_scale_rsrc(s, (uint32_t)N * (uint32_t)G);

  // DMA of stage j (groups gb + SG j ..) into buffer b. X: instruction q =
  // wv + 8 i is row q / (SG / 4), part q % (SG / 4) (64 of the row's 16 SG
  // slots); W: instruction q = wv + 8 i holds 16 / SG rows (4 SG slots each).
  // Groups past the slice read past the buffer extents (zeros). Rows >= M of
  // X and >= N of W lie past their extents too.
  auto issue = [&](int j, int b) {
    uint8_t* base = lds + b * ST::kBytes;
    const int glo = gb + SG * j;
#pragma unroll
    for (int i = 0; i < ST::kXI; ++i) {
      const int q = wv + kSLWaves * i;
      const int row = q / (SG / 4), h = q % (SG / 4);
      const int slot = 64 * h + lane;
      const int c = slot ^ (int)xswz(row);      // chunk held by this slot
      const int g = glo + (c >> 4);
      const uint32_t off = g < ge ? (uint32_t)row * KB + (uint32_t)g * 256u + 16u * (uint32_t)(c & 15) : 0xFFFFFFF0u;
      sl_dma16(rx, base + row * (SG * 256) + h * 1024, off);
    }
#pragma unroll
    for (int i = 0; i < ST::kWI; ++i) {
      const int q = wv + kSLWaves * i;
      const int row = (16 / SG) * q + lane / (4 * SG);
      const int c = (lane % (4 * SG)) ^ (int)xswz(row);
      const int g = glo + (c >> 2);
      const uint32_t off = g < ge ? (uint32_t)row * K2 + (uint32_t)g * 64u + 16u * (uint32_t)(c & 3) : 0xFFFFFFF0u;
      sl_dma16nt(rw, base + ST::kX + q * 1024, off);
    }
    // scales: lane i of instruction t (waves t < SG / 2) fetches the word
    // holding the scale of column (64 t + i) / SG, group (64 t + i) % SG
    if (wv < ST::kSW) {
      const int idx = 64 * wv + lane;
      const int col = idx / SG, g = glo + idx % SG;
      sl_dma4(rs, base + ST::kX + ST::kW + wv * 256, (((uint32_t)(n0 + col) * (uint32_t)G + (uint32_t)g) * 2u) & ~3u);
    }
  };

  const uint32_t magic = vgpr_const(kMagicPair);
  const uint32_t mask = __builtin_amdgcn_readfirstlane(vgpr_const(kNibblePairMask));
  const uint32_t neg136 = vgpr_const(0xC308C308u);   // bf16(-136) pair
  const bf16x8 bneg = __builtin_bit_cast(bf16x8, u32x4{neg136, neg136, neg136, neg136});

  const int ct = wv & 1;                       // the wave's column tile
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};

  // unit (ct, gl) of the stage in buffer b: X rows in A, column tile ct in B
  auto unit = [&](const uint8_t* sb, int gl, int g) {
    bf16x8 a[4];
#pragma unroll
    for (int st = 0; st < 4; ++st)
      a[st] = *reinterpret_cast<const bf16x8*>(sb + m16 * (SG * 256) + 16 * ((16 * gl + 4 * kb + st) ^ xs));
    const int r = 16 * ct + m16;
    const u32x4 pk = *reinterpret_cast<const u32x4*>(sb + ST::kX + r * (SG * 64) + 16 * ((4 * gl + kb) ^ xs));
    const uint32_t sw = *reinterpret_cast<const uint32_t*>(sb + ST::kX + ST::kW + 4 * (r * SG + gl));
    const float sc = __uint_as_float((((uint32_t)(n0 + r) * (uint32_t)G + (uint32_t)g) & 1u) ? (sw & 0xFFFF0000u)
                                                                                               : (sw << 16));
    // -136 * sum of the group's x in every column: the chain's start
    f32x4 t = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int st = 0; st < 4; ++st) t = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[st], bneg, t, 0, 0, 0);
    const uint32_t wd[4] = {pk.x, pk.y, pk.z, pk.w};
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      const uint32_t w0 = wd[st], w4 = w0 >> 4;
      u32x4 o;
      o.x = and_or_sv(__builtin_amdgcn_perm(w4, w0, 0x0C040C00u), mask, magic);
      o.y = and_or_sv(__builtin_amdgcn_perm(w4, w0, 0x0C050C01u), mask, magic);
      o.z = and_or_sv(__builtin_amdgcn_perm(w4, w0, 0x0C060C02u), mask, magic);
      o.w = and_or_sv(__builtin_amdgcn_perm(w4, w0, 0x0C070C03u), mask, magic);
      t = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[st], __builtin_bit_cast(bf16x8, o), t, 0, 0, 0);
    }
    acc.x = fmaf(sc, t.x, acc.x);
    acc.y = fmaf(sc, t.y, acc.y);
    acc.z = fmaf(sc, t.z, acc.z);
    acc.w = fmaf(sc, t.w, acc.w);
  };

  if (nst > 0) {
#pragma unroll
    for (int j = 0; j < NS - 1; ++j)
      if (j < nst) issue(j, j);
    // stage 0 landed (the later ones may still be in flight)
    const int later = min(nst, NS - 1) - 1;
    if (wv < ST::kSW) wait_stages<ST::kXI + ST::kWI + 1, NS - 2>(later);
    else wait_stages<ST::kXI + ST::kWI, NS - 2>(later);
  }
  // NS - 1 stages in flight
  for (int j = 0; j < nst; ++j) {
    const bool ahead = j + NS - 1 < nst;
    if (ahead) issue(j + NS - 1, (j + NS - 1) % NS);
    const uint8_t* sb = lds + (j % NS) * ST::kBytes;
#pragma unroll
    for (int u = 0; u < SG / 4; ++u) {
      const int gl = (wv >> 1) + 4 * u;
      const int g = gb + SG * j + gl;
      if (g < ge) unit(sb, gl, g);   // wave-uniform
    }
    if (j + 1 < nst) {
      // stage j + 1 landed: the DMA issued after it by this wave (stages
      // j + 2 .. j + NS - 1, those that exist) may still be in flight (no
      // other vector-memory operation is issued in this loop); and every wave
      // is done with stage j
      const int later = min(nst - 1, j + NS - 1) - (j + 1);   // stages issued after j + 1
      if (wv < ST::kSW) wait_stages<ST::kXI + ST::kWI + 1, NS - 2>(later);
      else wait_stages<ST::kXI + ST::kWI, NS - 2>(later);
    }
  }

  // ---- the four waves of a column tile: summed in wave order (waves ct,
  // ct + 2, ct + 4, ct + 6), through LDS (the stages are free now)
  __syncthreads();
  f32x4* red = reinterpret_cast<f32x4*>(lds);
  red[wv * 64 + lane] = acc;
  __syncthreads();
  if (wv < 2) {
    f32x4 v = red[wv * 64 + lane];
#pragma unroll
    for (int k = 1; k < 4; ++k) {
      const f32x4 p = red[(wv + 2 * k) * 64 + lane];
      v.x += p.x;
      v.y += p.y;
      v.z += p.z;
      v.w += p.w;
    }
    const int n = n0 + 16 * wv + m16;
    const float vals[4] = {v.x, v.y, v.z, v.w};
    if (n < N) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = 4 * kb + i;
        if (m < M) {
          if (gridDim.y > 1) static_cast<float*>(out)[((size_t)slice * M + m) * N + n] = vals[i];
          else static_cast<uint16_t*>(out)[(size_t)m * N + n] = to_bf16(vals[i]);
        }
      }
    }
  }
}

bool skinny_lds_fits(int M, int gps) { return M >= 1 && M <= 16 && gps >= 1; }

template <int SG, int NS>
static hipError_t launch_sl(const uint16_t* x, const uint8_t* w, const uint16_t* s, void* out, int M, int N, int K,
                            int gps, int sk, hipStream_t stream) {
  constexpr int lds = NS * SLStage<SG>::kBytes;
  static std::atomic<uint64_t> lds_set{0};
  const hipError_t ea = ensure_dyn_lds(reinterpret_cast<const void*>(&skinny_lds_kernel<SG, NS>), lds, lds_set);
  if (ea != hipSuccess) return ea;
  hipLaunchKernelGGL((skinny_lds_kernel<SG, NS>), dim3((N + kSLCols - 1) / kSLCols, sk), dim3(64 * kSLWaves), lds,
                     stream, x, w, s, out, M, N, K, gps);
  return hipGetLastError();
}

hipError_t launch_skinny_lds(const uint16_t* x, const uint8_t* w, const uint16_t* s, uint16_t* y, float* ws, int M,
                             int N, int K, int gps, int sk, int geometry, hipStream_t stream) {
  if (!skinny_lds_fits(M, gps)) return hipErrorInvalidValue;
  void* out = sk > 1 ? static_cast<void*>(ws) : static_cast<void*>(y);
  switch (geometry) {
    case 0: return launch_sl<8, 3>(x, w, s, out, M, N, K, gps, sk, stream);   // 3 x 49 KiB
    case 1: return launch_sl<4, 6>(x, w, s, out, M, N, K, gps, sk, stream);   // 6 x 24.5 KiB
    case 2: return launch_sl<4, 5>(x, w, s, out, M, N, K, gps, sk, stream);
    case 3: return launch_sl<4, 4>(x, w, s, out, M, N, K, gps, sk, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace w4a16
