// Decode GEMV for M = 1: y[n] = sum_k x[k] * s[n, k/128] * (q[n, k] - 8).
//
// Memory-bound: every packed weight byte and scale is read once. Layout of
// the work (the access-pattern lesson of "gfx1151: 61.7% of ... per-token
// byte budget runs KQuantGemmK with 8-12 of 32 lanes idle", section "The
// second half of the mechanism: the access pattern": consecutive lanes read
// consecutive 16-byte pieces, so one wave instruction is two contiguous
// 512-byte bursts):
//  * a half-wave (32 lanes) owns one weight row at a time; lane h reads the
//    16-byte chunks h, h+32, h+64, ... of the row (32 k values each, always
//    inside one 128-group, so one scale per chunk);
//  * x of the K-slice is loaded once per lane into registers, already in the
//    pair order of the magic-constant dequant, with -136 * sum(x) of each
//    chunk precomputed (the "(128 + n) - 136" of "[ROCm][Kernel] W4A16 skinny
//    GEMM: hand-asm kernel for gfx1151", section 1, applied once per chunk);
//  * a ring of D weight rows per half-wave is kept in flight, and the first
//    D rows are requested before x is loaded (the software pipelining of
//    section 2 of the same page);
//  * half-wave h of the grid takes rows h, h + H, h + 2H, ... (H = half-waves
//    in the grid), so neighbouring rows are streamed at the same time by
//    neighbouring half-waves all over the GPU;
//  * per row, the 32 lane partials are summed with a half-wave reduction.
// With split-K (gridDim.y = SK) slice s covers the 128-groups
// [s * gps, min((s + 1) * gps, G)) and writes fp32 partials to ws[s, 0, :].
#include "common.hpp"
#include "launch.hpp"

namespace w4a16 {

template <int CPL, int D, int AUX>
__global__ __launch_bounds__(256) void gemv_m1_kernel(const uint16_t* __restrict__ x,
                                                      const uint8_t* __restrict__ w,
                                                      const uint16_t* __restrict__ s,
                                                      uint16_t* __restrict__ y,
                                                      float* __restrict__ ws,
                                                      int N, int K, int gps) {
  const int lane = threadIdx.x & 63;
  const int hl = lane & 31;             // lane within the half-wave
  const int hw = (int)(blockIdx.x * 8 + (threadIdx.x >> 5));   // global half-wave id
  const int H = (int)(gridDim.x * 8);   // half-waves in the grid
  const int G = K / kGroup;
  const int slice = blockIdx.y;
  const int g0 = slice * gps;
  const int g1 = min(G, g0 + gps);
  const int nchunks = g1 > g0 ? (g1 - g0) * 4 : 0;
  // rows n = hw + r * H: at any moment neighbouring half-waves (across the
  // whole grid) stream neighbouring rows
  const int nrows = hw < N ? (N - 1 - hw) / H + 1 : 0;

  const __amdgpu_buffer_rsrc_t rx = make_rsrc(x, (uint32_t)K * 2u);
  const __amdgpu_buffer_rsrc_t rw = make_rsrc(w, (uint32_t)((uint64_t)N * (uint32_t)K / 2u));
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(s, (uint32_t)N * (uint32_t)G * 2u);

  // ---- weight ring: rows r, r+1, ..., r+D-1 of this half-wave in flight
  u32x4 wbuf[D][CPL];
  uint16_t sbuf[D][CPL];
  auto issue = [&](u32x4 (&wb)[CPL], uint16_t (&sb)[CPL], int r) {
    const int n = hw + r * H;
    const bool live = r < nrows;
    const uint32_t wrow = (uint32_t)n * (uint32_t)(K / 2) + (uint32_t)g0 * 64u;
    const uint32_t srow = ((uint32_t)n * (uint32_t)G + (uint32_t)g0) * 2u;
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
      const int c = hl + 32 * i;
      if (live && c < nchunks) {
        wb[i] = __builtin_amdgcn_raw_buffer_load_b128(rw, wrow + 16u * (uint32_t)c, 0, AUX);
        sb[i] = ld16(rs, srow + 2u * (uint32_t)(c >> 2));
      } else {
        wb[i] = u32x4{0u, 0u, 0u, 0u};
        sb[i] = 0;
      }
    }
  };
#pragma unroll
  for (int j = 0; j < D; ++j) issue(wbuf[j], sbuf[j], j);

  // ---- x of this lane's chunks (after the weight loads are in flight),
  // pair-interleaved, plus -136 * sum per chunk
  uint32_t xp[CPL][16];
  float cinit[CPL];
#pragma unroll
  for (int i = 0; i < CPL; ++i) {
    const int c = hl + 32 * i;
    const bool valid = c < nchunks;
    const uint32_t kb = (uint32_t)(g0 * kGroup + 32 * c) * 2u;
    float sx = 0.0f;
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      u32x4 v = valid ? ld128(rx, kb + 16u * d) : u32x4{0u, 0u, 0u, 0u};
      sx += (bf16lo(v.x) + bf16hi(v.x)) + (bf16lo(v.y) + bf16hi(v.y)) +
            (bf16lo(v.z) + bf16hi(v.z)) + (bf16lo(v.w) + bf16hi(v.w));
      // (x0,x4), (x1,x5), (x2,x6), (x3,x7)
      xp[i][4 * d + 0] = __builtin_amdgcn_perm(v.z, v.x, 0x05040100u);
      xp[i][4 * d + 1] = __builtin_amdgcn_perm(v.z, v.x, 0x07060302u);
      xp[i][4 * d + 2] = __builtin_amdgcn_perm(v.w, v.y, 0x05040100u);
      xp[i][4 * d + 3] = __builtin_amdgcn_perm(v.w, v.y, 0x07060302u);
    }
    cinit[i] = -136.0f * sx;
  }

  auto consume = [&](const u32x4 (&wb)[CPL], const uint16_t (&sb)[CPL], int r) {
    float acc = 0.0f;
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
      float t = cinit[i];
      const uint32_t wd[4] = {wb[i].x, wb[i].y, wb[i].z, wb[i].w};
#pragma unroll
      for (int d = 0; d < 4; ++d) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          t = __builtin_amdgcn_fdot2_f32_bf16(
              as_bf16x2(magic_pair_interleaved(wd[d], j)),
              as_bf16x2(xp[i][4 * d + j]), t, false);
        }
      }
      acc = fmaf(bf16f(sb[i]), t, acc);
    }
    // half-wave reduction (xor offsets stay within 32 lanes)
    acc += __shfl_xor(acc, 16, 32);
    acc += __shfl_xor(acc, 8, 32);
    acc += __shfl_xor(acc, 4, 32);
    acc += __shfl_xor(acc, 2, 32);
    acc += __shfl_xor(acc, 1, 32);
    const int n = hw + r * H;
    if (hl == 0 && r < nrows) {
      if (ws == nullptr) y[n] = to_bf16(acc);
      else ws[(size_t)slice * N + n] = acc;
    }
  };

  // ---- ring: consume row r from slot r % D, refill the slot with row r + D
  for (int r0 = 0; r0 < nrows; r0 += D) {
#pragma unroll
    for (int j = 0; j < D; ++j) {
      if (r0 + j < nrows) {
        consume(wbuf[j], sbuf[j], r0 + j);
        if (r0 + j + D < nrows) issue(wbuf[j], sbuf[j], r0 + j + D);
      }
    }
  }
}

// ---------------------------------------------------------------- flat layout
// Same arithmetic, but the lanes of a wave are laid over a block of R weight
// rows (of this K-slice) so that every wave instruction reads one contiguous
// 1 KiB run: in instruction i lane l takes 16-byte chunk c = 64 i + l of the
// block, i.e. row c / cps, chunk c % cps (cps = chunks per row-slice).
// R = 64 / gcd(cps, 64) rows make the block a whole number I of 1 KiB runs.
// A lane keeps R row partials; the R sums are formed with a wave-wide
// reduce-scatter (exchange halves, then tree) and written by lanes 0, 32, ...
template <int R>
__device__ __forceinline__ void wave_reduce_rows(float (&acc)[R], int lane, float* out_rows) {
  if (R == 4) {
    // offset 32: lanes < 32 keep rows 0,1; lanes >= 32 keep rows 2,3
    const bool hi = lane & 32;
    float k0 = hi ? acc[2] : acc[0], k1 = hi ? acc[3] : acc[1];
    float s0 = hi ? acc[0] : acc[2], s1 = hi ? acc[1] : acc[3];
    k0 += __shfl_xor(s0, 32);
    k1 += __shfl_xor(s1, 32);
    // offset 16: lanes with bit 16 keep the second
    const bool h16 = lane & 16;
    float k = h16 ? k1 : k0, sv = h16 ? k0 : k1;
    k += __shfl_xor(sv, 16);
    k += __shfl_xor(k, 8);
    k += __shfl_xor(k, 4);
    k += __shfl_xor(k, 2);
    k += __shfl_xor(k, 1);
    out_rows[0] = k;   // lane 0: row 0, lane 16: row 1, lane 32: row 2, lane 48: row 3
  } else if (R == 2) {
    const bool hi = lane & 32;
    float k = hi ? acc[1] : acc[0], sv = hi ? acc[0] : acc[1];
    k += __shfl_xor(sv, 32);
    k += __shfl_xor(k, 16);
    k += __shfl_xor(k, 8);
    k += __shfl_xor(k, 4);
    k += __shfl_xor(k, 2);
    k += __shfl_xor(k, 1);
    out_rows[0] = k;   // lane 0: row 0, lane 32: row 1
  } else {
    float k = acc[0];
    k += __shfl_xor(k, 32);
    k += __shfl_xor(k, 16);
    k += __shfl_xor(k, 8);
    k += __shfl_xor(k, 4);
    k += __shfl_xor(k, 2);
    k += __shfl_xor(k, 1);
    out_rows[0] = k;
  }
}

constexpr int kMaxChunks = 256;   // 32-k chunks per row-slice (64 groups)

template <int R, int I, int D, int AUX>
__global__ __launch_bounds__(256) void gemv_flat_kernel(const uint16_t* __restrict__ x,
                                                        const uint8_t* __restrict__ w,
                                                        const uint16_t* __restrict__ s,
                                                        uint16_t* __restrict__ y,
                                                        float* __restrict__ ws,
                                                        int N, int K, int gps) {
  const int lane = threadIdx.x & 63;
  const int wv = (int)(blockIdx.x * 4 + (threadIdx.x >> 6));   // global wave id
  const int W = (int)(gridDim.x * 4);
  const int G = K / kGroup;
  const int slice = blockIdx.y;
  const int g0 = slice * gps;
  const int g1 = min(G, g0 + gps);
  const int cps = g1 > g0 ? (g1 - g0) * 4 : 0;   // chunks per row in this slice
  const int nblk = (N + R - 1) / R;
  // row blocks b = wv + j * W: neighbouring waves stream neighbouring blocks
  const int nb = wv < nblk ? (nblk - 1 - wv) / W + 1 : 0;

  const __amdgpu_buffer_rsrc_t rx = make_rsrc(x, (uint32_t)K * 2u);
  const __amdgpu_buffer_rsrc_t rw = make_rsrc(w, (uint32_t)((uint64_t)N * (uint32_t)K / 2u));
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(s, (uint32_t)N * (uint32_t)G * 2u);
  const uint32_t rowb = (uint32_t)(K / 2);

  // ---- x of the slice, prepared once per workgroup in LDS: each 32-k chunk
  // as 16 dwords in the magic-constant pair order plus -136 * its sum
  __shared__ u32x4 xprep[kMaxChunks * 4];
  __shared__ float cinl[kMaxChunks];
  const int tid = threadIdx.x;
  constexpr int kPrepPer = (kMaxChunks * 4 + 255) / 256;
  u32x4 xv[kPrepPer];
#pragma unroll
  for (int k = 0; k < kPrepPer; ++k) {
    const int p = tid + 256 * k;   // 16-byte piece p = 4 * chunk + d
    xv[k] = p < cps * 4 ? ld128(rx, (uint32_t)(g0 * kGroup) * 2u + 16u * (uint32_t)p) : u32x4{0u, 0u, 0u, 0u};
  }

  // static per-lane mapping, identical for every block
  uint32_t woff[I], soff[I];
  int rib[I], chi[I];
  bool valid[I];
#pragma unroll
  for (int i = 0; i < I; ++i) {
    const int c = 64 * i + lane;
    valid[i] = cps > 0 && c < R * cps;
    const int r = valid[i] ? c / cps : 0;
    const int ch = valid[i] ? c - r * cps : 0;
    rib[i] = r;
    chi[i] = ch;
    woff[i] = (uint32_t)r * rowb + (uint32_t)g0 * 64u + (uint32_t)ch * 16u;
    soff[i] = ((uint32_t)r * (uint32_t)G + (uint32_t)g0 + (uint32_t)(ch >> 2)) * 2u;
  }

  u32x4 wbuf[D][I];
  uint16_t sbuf[D][I];
  auto issue = [&](u32x4 (&wb)[I], uint16_t (&sb)[I], int j) {
    const int b = wv + j * W;
    const bool live = j < nb;
    const uint32_t wbase = (uint32_t)b * (uint32_t)R * rowb;
    const uint32_t sbase = (uint32_t)b * (uint32_t)R * (uint32_t)G * 2u;
#pragma unroll
    for (int i = 0; i < I; ++i) {
      if (live && valid[i]) {
        wb[i] = __builtin_amdgcn_raw_buffer_load_b128(rw, wbase + woff[i], 0, AUX);
        sb[i] = ld16(rs, sbase + soff[i]);
      } else {
        wb[i] = u32x4{0u, 0u, 0u, 0u};
        sb[i] = 0;
      }
    }
  };
#pragma unroll
  for (int j = 0; j < D; ++j) issue(wbuf[j], sbuf[j], j);

  const uint32_t ones = 0x3F803F80u;   // bf16 (1, 1)
#pragma unroll
  for (int k = 0; k < kPrepPer; ++k) {
    const int p = tid + 256 * k;
    if (p < cps * 4) {   // whole quads of a chunk are active together (cps * 4 % 4 == 0)
      const u32x4 v = xv[k];
      u32x4 o;
      o.x = __builtin_amdgcn_perm(v.z, v.x, 0x05040100u);   // (x0, x4)
      o.y = __builtin_amdgcn_perm(v.z, v.x, 0x07060302u);   // (x1, x5)
      o.z = __builtin_amdgcn_perm(v.w, v.y, 0x05040100u);   // (x2, x6)
      o.w = __builtin_amdgcn_perm(v.w, v.y, 0x07060302u);   // (x3, x7)
      xprep[p] = o;
      float sx = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(v.x), as_bf16x2(ones), 0.0f, false);
      sx = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(v.y), as_bf16x2(ones), sx, false);
      sx = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(v.z), as_bf16x2(ones), sx, false);
      sx = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(v.w), as_bf16x2(ones), sx, false);
      sx += __shfl_xor(sx, 1, 4);
      sx += __shfl_xor(sx, 2, 4);
      if ((p & 3) == 0) cinl[p >> 2] = -136.0f * sx;
    }
  }
  __syncthreads();

  const uint32_t magic = vgpr_const(kMagicPair);
  const uint32_t mask = __builtin_amdgcn_readfirstlane(kNibblePairMask);
  uint32_t xp[I][16];
  float cinit[I];
  float rmask[I][R];
#pragma unroll
  for (int i = 0; i < I; ++i) {
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const u32x4 o = valid[i] ? xprep[4 * chi[i] + d] : u32x4{0u, 0u, 0u, 0u};
      xp[i][4 * d + 0] = o.x;
      xp[i][4 * d + 1] = o.y;
      xp[i][4 * d + 2] = o.z;
      xp[i][4 * d + 3] = o.w;
    }
    cinit[i] = valid[i] ? cinl[chi[i]] : 0.0f;
#pragma unroll
    for (int rr = 0; rr < R; ++rr) rmask[i][rr] = (valid[i] && rib[i] == rr) ? 1.0f : 0.0f;
  }

  auto consume = [&](const u32x4 (&wb)[I], const uint16_t (&sb)[I], int j) {
    float acc[R];
#pragma unroll
    for (int rr = 0; rr < R; ++rr) acc[rr] = 0.0f;
#pragma unroll
    for (int i = 0; i < I; ++i) {
      float t = cinit[i];
      const uint32_t wd[4] = {wb[i].x, wb[i].y, wb[i].z, wb[i].w};
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const uint32_t w0 = wd[d], w1 = wd[d] >> 4, w2 = wd[d] >> 8, w3 = wd[d] >> 12;
        t = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(and_or_sv(w0, mask, magic)),
                                           as_bf16x2(xp[i][4 * d + 0]), t, false);
        t = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(and_or_sv(w1, mask, magic)),
                                           as_bf16x2(xp[i][4 * d + 1]), t, false);
        t = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(and_or_sv(w2, mask, magic)),
                                           as_bf16x2(xp[i][4 * d + 2]), t, false);
        t = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(and_or_sv(w3, mask, magic)),
                                           as_bf16x2(xp[i][4 * d + 3]), t, false);
      }
      const float v = bf16f(sb[i]) * t;
#pragma unroll
      for (int rr = 0; rr < R; ++rr) acc[rr] = fmaf(rmask[i][rr], v, acc[rr]);
    }
    float red[1];
    wave_reduce_rows<R>(acc, lane, red);
    const int rr = R == 4 ? (lane >> 4) : (R == 2 ? (lane >> 5) : 0);
    const int n = (wv + j * W) * R + rr;
    if ((lane & (R == 4 ? 15 : (R == 2 ? 31 : 63))) == 0 && j < nb && n < N) {
      if (ws == nullptr) y[n] = to_bf16(red[0]);
      else ws[(size_t)slice * N + n] = red[0];
    }
  };

  for (int j0 = 0; j0 < nb; j0 += D) {
#pragma unroll
    for (int j = 0; j < D; ++j) {
      if (j0 + j < nb) {
        consume(wbuf[j], sbuf[j], j0 + j);
        if (j0 + j + D < nb) issue(wbuf[j], sbuf[j], j0 + j + D);
      }
    }
  }
}

// flat-layout geometry for a slice of `cps` chunks per row; false if it does
// not fit the instantiated shapes (R <= 4 rows, I <= 8 runs of 1 KiB)
static bool flat_geometry(int cps, int* R, int* I) {
  int g = 64, a = cps;
  while (a % 2 == 0 && g > 1) { a /= 2; g /= 2; }   // g = 64 / gcd(cps, 64)
  *R = g;
  *I = g * cps / 64;
  return *R <= 4 && *I >= 1 && *I <= 8;
}

template <int R, int I>
static hipError_t launch_flat_ri(const uint16_t* x, const uint8_t* w, const uint16_t* s, uint16_t* y, float* ws,
                                 int N, int K, int gps, int sk, int depth, int nt, int blocks_per_wave,
                                 hipStream_t stream) {
  const int nblk = (N + R - 1) / R;
  const int waves = (nblk + blocks_per_wave - 1) / blocks_per_wave;
  dim3 grid((waves + 3) / 4, sk);
#define W4A16_FLAT(DD, AA)                                                                           \
  if (depth == DD && nt == AA) {                                                                     \
    hipLaunchKernelGGL((gemv_flat_kernel<R, I, DD, AA * 2>), grid, dim3(256), 0, stream, x, w, s, y, ws, \
                       N, K, gps);                                                                   \
    return hipGetLastError();                                                                        \
  }
  W4A16_FLAT(1, 0)
  W4A16_FLAT(2, 0)
  W4A16_FLAT(3, 0)
  W4A16_FLAT(1, 1)
  W4A16_FLAT(2, 1)
  W4A16_FLAT(3, 1)
#undef W4A16_FLAT
  return hipErrorInvalidValue;
}

static hipError_t launch_flat(const uint16_t* x, const uint8_t* w, const uint16_t* s, uint16_t* y, float* ws,
                              int N, int K, int gps, int sk, int R, int I, int depth, int nt, int bpw,
                              hipStream_t stream) {
#define W4A16_RI(RR, II) \
  if (R == RR && I == II) return launch_flat_ri<RR, II>(x, w, s, y, ws, N, K, gps, sk, depth, nt, bpw, stream);
  W4A16_RI(1, 1) W4A16_RI(1, 2) W4A16_RI(1, 3) W4A16_RI(1, 4) W4A16_RI(1, 5) W4A16_RI(1, 6) W4A16_RI(1, 7)
  W4A16_RI(1, 8)
  W4A16_RI(2, 1) W4A16_RI(2, 3) W4A16_RI(2, 5) W4A16_RI(2, 7)
  W4A16_RI(4, 1) W4A16_RI(4, 3) W4A16_RI(4, 5) W4A16_RI(4, 7)
#undef W4A16_RI
  return hipErrorInvalidValue;
}

template <int CPL>
static hipError_t launch_gemv_cpl(const uint16_t* x, const uint8_t* w, const uint16_t* s, uint16_t* y,
                                  float* ws, int N, int K, int gps, int sk, int variant, hipStream_t stream) {
  // variant: 10 * prefetch depth + rows per half-wave target (1..9); 100 adds
  // the non-temporal cache policy on the weight stream
  const int nt = (variant / 100) % 10;
  const int depth = (variant / 10) % 10;
  const int rows_target = variant % 10 > 0 ? variant % 10 : 1;
  const int halfwaves = (N + rows_target - 1) / rows_target;
  const int blocks = (halfwaves + 7) / 8;
  dim3 grid(blocks > 0 ? blocks : 1, sk);
#define W4A16_GEMV(DD, AA)                                                                          \
  if (depth == DD && nt == AA) {                                                                    \
    hipLaunchKernelGGL((gemv_m1_kernel<CPL, DD, AA * 2>), grid, dim3(256), 0, stream, x, w, s, y, ws, \
                       N, K, gps);                                                                  \
    return hipGetLastError();                                                                       \
  }
  W4A16_GEMV(1, 0)
  W4A16_GEMV(2, 0)
  W4A16_GEMV(3, 0)
  W4A16_GEMV(4, 0)
  W4A16_GEMV(1, 1)
  W4A16_GEMV(2, 1)
  W4A16_GEMV(3, 1)
  W4A16_GEMV(4, 1)
#undef W4A16_GEMV
  return hipErrorInvalidValue;
}

bool gemv_flat_fits(int gps) {
  int R, I;
  return flat_geometry(gps * 4, &R, &I);
}

hipError_t launch_gemv_m1(const uint16_t* x, const uint8_t* w, const uint16_t* s, uint16_t* y,
                          float* ws, int N, int K, int gps, int sk, int variant,
                          hipStream_t stream) {
  // variant: 1000 * layout (0 flat, 1 half-wave) + 100 * non-temporal
  //          + 10 * prefetch depth + blocks (flat) / rows (half-wave) per wave
  const int layout = (variant / 1000) % 10;
  int R = 0, I = 0;
  if (layout == 0 && flat_geometry(gps * 4, &R, &I)) {
    const int nt = (variant / 100) % 10;
    const int depth = (variant / 10) % 10 > 0 ? (variant / 10) % 10 : 2;
    const int bpw = variant % 10 > 0 ? variant % 10 : 4;
    return launch_flat(x, w, s, y, ws, N, K, gps, sk, R, I, depth, nt, bpw, stream);
  }
  const int v = variant % 1000;
  const int cpl = (gps * 4 + 31) / 32;   // chunks per lane in a slice
  switch (cpl) {
    case 1: return launch_gemv_cpl<1>(x, w, s, y, ws, N, K, gps, sk, v, stream);
    case 2: return launch_gemv_cpl<2>(x, w, s, y, ws, N, K, gps, sk, v, stream);
    case 3: return launch_gemv_cpl<3>(x, w, s, y, ws, N, K, gps, sk, v, stream);
    case 4: return launch_gemv_cpl<4>(x, w, s, y, ws, N, K, gps, sk, v, stream);
    case 5: return launch_gemv_cpl<5>(x, w, s, y, ws, N, K, gps, sk, v, stream);
    case 6: return launch_gemv_cpl<6>(x, w, s, y, ws, N, K, gps, sk, v, stream);
    case 7: return launch_gemv_cpl<7>(x, w, s, y, ws, N, K, gps, sk, v, stream);
    case 8: return launch_gemv_cpl<8>(x, w, s, y, ws, N, K, gps, sk, v, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace w4a16
