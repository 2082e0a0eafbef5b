// Prefill (M in the hundreds to thousands) and grouped W4A16 GEMM on bf16
// MFMA 32x32x16, LDS-staged and double-buffered.
//
// Numerics: the weight operand in LDS is bf16(128 + q), exact, produced from
// the packed nibbles with the magic-constant OR ("[ROCm][Kernel] W4A16 skinny
// GEMM: hand-asm kernel for gfx1151", section 1). For every 128-group g the
// MFMA chain of a 32x32 output tile starts from -136 * sum_{k in g} x[m, k]
// (per row, from the row-sum pre-pass below), so after the group's 8 MFMA
// steps it holds sum_k x * (q - 8) in fp32; that is scaled by the bf16 scale
// of the column and added to the fp32 accumulator. No weight is ever rounded.
//
// Structure per workgroup (BM x BN output tile, waves WM x WN, each wave a
// (BM/WM) x (BN/WN) tile of 32x32 sub-tiles), following "Add Triton
// BF16xINT4 rowwise GEMM for ROCm gfx942/gfx950", Implementation ("XCD
// remapping", GROUP_SIZE_M grouping) and section 2 of the hand-asm page
// (prefetch of the next K-tile while the current one is multiplied):
//  * K-tile = 64 k; an X tile [BM, 64] bf16 and a W tile [BN, 64] bf16
//    (dequantised on the way from global to LDS) per stage, two stages;
//  * 16-byte LDS chunks of a 128-byte row are XOR-swizzled by (row & 7);
//  * global loads of K-tile t+1 are issued before the MFMAs of K-tile t;
//  * buffer resources carry exact extents (section 3 of the hand-asm page),
//    so the M tail (rows past M) and the N tail read zeros; stores past the
//    last row are dropped and columns >= N are skipped.
// Grouped ("Native fused grouped kernel" on the MI350X Triton page): the
// grid covers (ceil(M_total/BM) + G) linear M-tiles x N-tiles; each
// workgroup walks M_sizes on the device (exclusive prefix sums, clamped to
// [0, M_total)) to find its group, and surplus workgroups exit at once.
#include "common.hpp"
#include "launch.hpp"
#include "tilemap.hpp"

namespace w4a16 {

// ---------------------------------------------------------------- row sums
// out[g * ld + m] = -136 * sum_{k in group g} x[m, k], fp32, for groups of GS
// = 128 or 32 k. One wave per row; a wave instruction covers 512 consecutive
// k and up to 8 of them are in flight before any is reduced; a group's lanes
// (16 for 128 k, 4 for 32 k) are summed with DPP. Loads past the row read
// zeros (exact buffer extent).
template <int GS>
__global__ __launch_bounds__(256) void rowsum_neg136_kernel(const uint16_t* __restrict__ x,
                                                           float* __restrict__ out, int M, int K,
                                                           int ld) {
  constexpr int U = 8;
  constexpr int LPG = GS / 8;   // lanes per group
  const int lane = threadIdx.x & 63;
  const int m = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (m >= M) return;
  const __amdgpu_buffer_rsrc_t rx = make_rsrc(x + (size_t)m * K, (uint32_t)K * 2u);
  for (int base = 0; base < K; base += 512 * U) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = ld128(rx, (uint32_t)(base + 512 * u + 8 * lane) * 2u);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int k = base + 512 * u + 8 * lane;
      float p = (bf16lo(v[u].x) + bf16hi(v[u].x)) + (bf16lo(v[u].y) + bf16hi(v[u].y)) +
                (bf16lo(v[u].z) + bf16hi(v[u].z)) + (bf16lo(v[u].w) + bf16hi(v[u].w));
      if constexpr (LPG == 16) {
        p = row16_sum(p);
      } else {
        p += dpp_f<0xB1>(p);   // quad_perm [1,0,3,2]
        p += dpp_f<0x4E>(p);   // quad_perm [2,3,0,1]
      }
      if ((lane & (LPG - 1)) == 0 && k < K) out[(size_t)(k / GS) * ld + m] = -136.0f * p;
    }
  }
}

// ---------------------------------------------------------------- tile GEMM
struct TileArgs {
  const uint16_t* x;      // [M_total, K]
  const uint8_t* w;       // [G, N, K/2]
  const uint16_t* s;      // [G, N, K/128]
  const float* sxn;       // [K/128, ld] = -136 * row sums per group
  uint16_t* y;            // [M_total, N]
  float* ws;              // [SK, M_total, N] fp32 split-K partials, or nullptr
  const int32_t* m_sizes; // [G] on device, or nullptr for one group of M_total rows
  int m_uniform;          // batched: rows per weight group (M_sizes not used), else 0
  int M_total, N, K, G, ld;
  int gps;                // 128-groups per split-K slice (gridDim.y slices)
  int mtiles;             // linear M-tiles covered by the grid
  int ntiles;
};

template <int BM, int BN, int WM, int WN>
__global__ __launch_bounds__(64 * WM * WN) void tile_kernel(const TileArgs args) {
  constexpr int NTHR = 64 * WM * WN;
  constexpr int TM = BM / WM, TN = BN / WN;     // wave tile
  constexpr int SM = TM / 32, SN = TN / 32;     // 32x32 sub-tiles per wave
  constexpr int BK = 64;                        // k per K-tile (half a group)
  constexpr int ROWB = BK * 2;                  // bytes per LDS row (128)
  constexpr int LA = BM * (ROWB / 16) / NTHR;   // 16-B X loads per thread per K-tile
  constexpr int LB = BN * 2 / NTHR;             // 16-B packed W loads per thread per K-tile
  static_assert(LA * NTHR == BM * (ROWB / 16), "X tile / threads");
  static_assert(LB * NTHR == BN * 2 && LB >= 1, "W tile / threads");
  static_assert(SM >= 1 && SN >= 1, "wave tile");

  __shared__ __attribute__((aligned(16))) uint8_t lds[2 * (BM + BN) * ROWB];
  uint8_t* const As0 = lds;
  uint8_t* const Bs0 = lds + BM * ROWB;
  uint8_t* const As1 = lds + (BM + BN) * ROWB;
  uint8_t* const Bs1 = As1 + BM * ROWB;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;
  const int Gk = args.K / kGroup;

  // ---- tile id and rows
  int mt_lin, nt;
  int MT = args.mtiles, nblocks = (int)gridDim.x;
  if (args.m_sizes != nullptr) {
    MT = real_mtiles(BM, args.M_total, args.m_sizes, args.G);
    nblocks = MT * args.ntiles;
    if ((int)blockIdx.x >= nblocks) return;
  }
  tile_coords(blockIdx.x, nblocks, MT, args.ntiles, &mt_lin, &nt);
  const TileRows tr = tile_rows(mt_lin, BM, args.M_total, args.m_sizes, args.G, args.m_uniform);
  const int wg = tr.wg, row0 = tr.row0, rows = tr.rows;
  if (rows <= 0) return;
  const int n0 = nt * BN;
  const int ncols = min(BN, args.N - n0);

  const size_t K2 = (size_t)args.K / 2;
  const __amdgpu_buffer_rsrc_t rx = make_rsrc(args.x + (size_t)row0 * args.K, (uint32_t)rows * (uint32_t)args.K * 2u);
  const __amdgpu_buffer_rsrc_t rw =
      make_rsrc(args.w + ((size_t)wg * args.N + n0) * K2, (uint32_t)((size_t)ncols * K2));
  const __amdgpu_buffer_rsrc_t rs =
      make_rsrc(args.s + ((size_t)wg * args.N + n0) * Gk, (uint32_t)ncols * (uint32_t)Gk * 2u);
  const __amdgpu_buffer_rsrc_t rsx =
      make_rsrc(args.sxn + row0, (uint32_t)(((size_t)Gk * args.ld - row0) * 4u));
  const __amdgpu_buffer_rsrc_t ry = make_rsrc(args.y + (size_t)row0 * args.N, (uint32_t)rows * (uint32_t)args.N * 2u);
  const int slice = blockIdx.y;
  const int gb = slice * args.gps;
  const int ge = min(Gk, gb + args.gps);
  const __amdgpu_buffer_rsrc_t rws =
      make_rsrc(args.ws + ((size_t)slice * args.M_total + row0) * args.N, (uint32_t)rows * (uint32_t)args.N * 4u);

  // ---- per-thread staging coordinates
  uint32_t a_goff[LA], a_loff[LA];
#pragma unroll
  for (int i = 0; i < LA; ++i) {
    const int ci = tid + NTHR * i;
    const int r = ci >> 3, c = ci & 7;
    a_goff[i] = (uint32_t)r * (uint32_t)args.K * 2u + (uint32_t)c * 16u;
    a_loff[i] = (uint32_t)(r * ROWB + ((c ^ (r & 7)) << 4));
  }
  uint32_t b_goff[LB];
  int b_row[LB], b_half[LB];
#pragma unroll
  for (int i = 0; i < LB; ++i) {
    const int ci = tid + NTHR * i;
    b_row[i] = ci >> 1;
    b_half[i] = ci & 1;
    b_goff[i] = (uint32_t)b_row[i] * (uint32_t)K2 + (uint32_t)b_half[i] * 16u;
  }

  u32x4 ra[LA], rb[LB];
  auto gload = [&](int kt) {
#pragma unroll
    for (int i = 0; i < LA; ++i) ra[i] = ld128(rx, a_goff[i], (uint32_t)kt * (uint32_t)ROWB);
#pragma unroll
    for (int i = 0; i < LB; ++i) rb[i] = ld128(rw, b_goff[i], (uint32_t)kt * 32u);
  };
  auto lstore = [&](uint8_t* As, uint8_t* Bs) {
#pragma unroll
    for (int i = 0; i < LA; ++i) *reinterpret_cast<u32x4*>(As + a_loff[i]) = ra[i];
#pragma unroll
    for (int i = 0; i < LB; ++i) {
      const int r = b_row[i];
      const uint32_t wd[4] = {rb[i].x, rb[i].y, rb[i].z, rb[i].w};
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const uint32_t w4 = wd[d] >> 4;
        u32x4 o;
        o.x = magic_pair_natural(wd[d], w4, 0);
        o.y = magic_pair_natural(wd[d], w4, 1);
        o.z = magic_pair_natural(wd[d], w4, 2);
        o.w = magic_pair_natural(wd[d], w4, 3);
        const int c = 4 * b_half[i] + d;
        *reinterpret_cast<u32x4*>(Bs + r * ROWB + ((c ^ (r & 7)) << 4)) = o;
      }
    }
  };

  // ---- per-lane MFMA operand coordinates
  const int l32 = lane & 31, lh = lane >> 5;
  uint32_t a_rd[SM], b_rd[SN];
#pragma unroll
  for (int ms = 0; ms < SM; ++ms) a_rd[ms] = (uint32_t)((wm * TM + 32 * ms + l32) * ROWB);
#pragma unroll
  for (int ns = 0; ns < SN; ++ns) b_rd[ns] = (uint32_t)((wn * TN + 32 * ns + l32) * ROWB);
  const int a_sw = (l32 & 7);   // (row & 7) for all rows this lane reads (row = 32*x + l32 + 8*...)

  // init (-136 sum x) and scales of a group
  uint32_t sx_off[SM][4];
#pragma unroll
  for (int ms = 0; ms < SM; ++ms)
#pragma unroll
    for (int j = 0; j < 4; ++j) sx_off[ms][j] = (uint32_t)(wm * TM + 32 * ms + 8 * j + 4 * lh) * 4u;
  uint32_t sc_off[SN];
#pragma unroll
  for (int ns = 0; ns < SN; ++ns) sc_off[ns] = (uint32_t)(wn * TN + 32 * ns + l32) * (uint32_t)Gk * 2u;

  f32x16 init_c[SM], init_n[SM];
  uint16_t sc_c[SN], sc_n[SN];
  auto load_group = [&](f32x16 (&ini)[SM], uint16_t (&sc)[SN], int g) {
    const uint32_t gb = (uint32_t)g * (uint32_t)args.ld * 4u;
#pragma unroll
    for (int ms = 0; ms < SM; ++ms) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        // the group offset is a row offset of the row-sum matrix: it goes into
        // the range-checked vector offset, never the scalar one
        const u32x4 v = ld128(rsx, sx_off[ms][j] + gb);
        ini[ms][4 * j + 0] = __uint_as_float(v.x);
        ini[ms][4 * j + 1] = __uint_as_float(v.y);
        ini[ms][4 * j + 2] = __uint_as_float(v.z);
        ini[ms][4 * j + 3] = __uint_as_float(v.w);
      }
    }
#pragma unroll
    for (int ns = 0; ns < SN; ++ns) sc[ns] = ld16(rs, sc_off[ns], (uint32_t)g * 2u);
  };

  f32x16 acc[SM][SN], tmp[SM][SN];
#pragma unroll
  for (int ms = 0; ms < SM; ++ms)
#pragma unroll
    for (int ns = 0; ns < SN; ++ns)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[ms][ns][e] = 0.0f;

  // one K-tile (4 MFMA steps of 16 k) from LDS; `first` starts the chains
  auto mma_tile = [&](const uint8_t* As, const uint8_t* Bs, bool first) {
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      const int c = 2 * st + lh;
      const uint32_t co = (uint32_t)((c ^ a_sw) << 4);
      bf16x8 a[SM], b[SN];
#pragma unroll
      for (int ms = 0; ms < SM; ++ms) a[ms] = *reinterpret_cast<const bf16x8*>(As + a_rd[ms] + co);
#pragma unroll
      for (int ns = 0; ns < SN; ++ns) b[ns] = *reinterpret_cast<const bf16x8*>(Bs + b_rd[ns] + co);
#pragma unroll
      for (int ms = 0; ms < SM; ++ms)
#pragma unroll
        for (int ns = 0; ns < SN; ++ns)
          tmp[ms][ns] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[ms], b[ns],
                                                               (first && st == 0) ? init_c[ms] : tmp[ms][ns], 0, 0, 0);
    }
  };

  // ---- main loop: one 128-group (two K-tiles) per iteration
  if (gb < ge) {
    gload(2 * gb);
    load_group(init_c, sc_c, gb);
    lstore(As0, Bs0);
    __syncthreads();
  }
  for (int g = gb; g < ge; ++g) {
    gload(2 * g + 1);
    if (g + 1 < ge) load_group(init_n, sc_n, g + 1);
    mma_tile(As0, Bs0, true);
    lstore(As1, Bs1);
    __syncthreads();
    if (g + 1 < ge) gload(2 * g + 2);
    mma_tile(As1, Bs1, false);
#pragma unroll
    for (int ns = 0; ns < SN; ++ns) {
      const float scv = bf16f(sc_c[ns]);
#pragma unroll
      for (int ms = 0; ms < SM; ++ms)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[ms][ns][e] = fmaf(scv, tmp[ms][ns][e], acc[ms][ns][e]);
    }
    if (g + 1 < ge) {
#pragma unroll
      for (int ms = 0; ms < SM; ++ms) init_c[ms] = init_n[ms];
#pragma unroll
      for (int ns = 0; ns < SN; ++ns) sc_c[ns] = sc_n[ns];
      lstore(As0, Bs0);
      __syncthreads();
    }
  }

  // ---- epilogue: fp32 -> bf16 (RNE), lane holds rows 8j + 4*lh + i of column l32
#pragma unroll
  for (int ns = 0; ns < SN; ++ns) {
    const int ncol = wn * TN + 32 * ns + l32;
    if (ncol >= ncols) continue;
#pragma unroll
    for (int ms = 0; ms < SM; ++ms) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = wm * TM + 32 * ms + 8 * j + 4 * lh + i;
          const uint32_t e = (uint32_t)r * (uint32_t)args.N + (uint32_t)(n0 + ncol);
          if (args.ws == nullptr) st16(to_bf16(acc[ms][ns][4 * j + i]), ry, e * 2u);
          else st32(__float_as_uint(acc[ms][ns][4 * j + i]), rws, e * 4u);
        }
      }
    }
  }
}

hipError_t launch_rowsum_neg136(const uint16_t* x, float* out, int M, int K, int ld, int gsize,
                                hipStream_t stream) {
  if (M <= 0) return hipSuccess;
  if (gsize == 128)
    hipLaunchKernelGGL(rowsum_neg136_kernel<128>, dim3((M + 3) / 4), dim3(256), 0, stream, x, out, M, K, ld);
  else if (gsize == 32)
    hipLaunchKernelGGL(rowsum_neg136_kernel<32>, dim3((M + 3) / 4), dim3(256), 0, stream, x, out, M, K, ld);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

template <int BM, int BN, int WM, int WN>
static hipError_t launch_tile_t(const TileArgs& a0, int mtiles_bound, int sk, hipStream_t stream) {
  TileArgs a = a0;
  a.mtiles = mtiles_bound;
  a.ntiles = (a.N + BN - 1) / BN;
  const long long blocks = (long long)a.mtiles * a.ntiles;
  if (blocks <= 0) return hipSuccess;
  if (blocks > 0x7FFFFFFFLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL((tile_kernel<BM, BN, WM, WN>), dim3((unsigned)blocks, sk), dim3(64 * WM * WN), 0, stream, a);
  return hipGetLastError();
}

// Tile configurations (BM x BN):
//   0: 128 x 256, 2 x 4 waves of 64 x 64, weights dequantised into LDS
//   1: 128 x 128, 2 x 2 waves of 64 x 64, weights dequantised into LDS
//   2: 128 x 256, 8 waves of 128 x 32, LDS-DMA staging, 3 stages (prefill.hip)
struct TileCfg { int bm, bn; };
static const TileCfg kTileCfgs[] = {{128, 256}, {128, 128}, {128, 256}, {96, 256}, {112, 256},
                                    {80, 256},  {144, 256}, {64, 256},  {48, 256}};
int tile_num_cfgs() { return (int)(sizeof(kTileCfgs) / sizeof(kTileCfgs[0])); }
int tile_bm(int cfg) { return kTileCfgs[cfg].bm; }
int tile_bn(int cfg) { return kTileCfgs[cfg].bn; }
bool tile_group_ok(int cfg, int gsize) {
  if (cfg < 0 || cfg >= tile_num_cfgs()) return false;
  return gsize == 128 || (gsize == 32 && cfg >= 2 && cfg <= 5);
}

hipError_t launch_tile(const uint16_t* x, const uint8_t* w, const uint16_t* s, const float* sxn, uint16_t* y,
                       float* ws, const int32_t* m_sizes, int m_uniform, int M_total, int N, int K, int G, int ld,
                       int gps, int sk, int cfg, int gsize, hipStream_t stream) {
  if (cfg < 0 || cfg >= tile_num_cfgs()) return hipErrorInvalidValue;
  if (cfg >= 2)   // LDS-DMA kernel: 8 (cfg 2), 6 (3), 7 (4), 5 (5), 9 (6), 4 (7) or 3 (8) row tiles of 16
    return launch_prefill(x, w, s, sxn, y, ws, m_sizes, m_uniform, M_total, N, K, G, ld, gps, sk,
                          kTileCfgs[cfg].bm / 16, gsize, stream);
  if (gsize != 128) return hipErrorInvalidValue;   // configs 0 and 1: 128-groups only
  TileArgs a;
  a.x = x; a.w = w; a.s = s; a.sxn = sxn; a.y = y; a.ws = ws; a.m_sizes = m_sizes; a.m_uniform = m_uniform;
  a.M_total = M_total; a.N = N; a.K = K; a.G = G; a.ld = ld; a.gps = gps;
  a.mtiles = 0; a.ntiles = 0;
  const int bm = tile_bm(cfg);
  const int mt = m_uniform > 0 ? G * ((m_uniform + bm - 1) / bm)
                               : (M_total + bm - 1) / bm + (m_sizes != nullptr ? G : 0);
  switch (cfg) {
    case 0: return launch_tile_t<128, 256, 2, 4>(a, mt, sk, stream);
    case 1: return launch_tile_t<128, 128, 2, 2>(a, mt, sk, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace w4a16
