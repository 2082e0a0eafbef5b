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

#include <algorithm>
#include <atomic>

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
    // half-wave reduction (DPP): the sum lands in lanes 31 and 63
    acc = half32_sum(acc);
    const int n = hw + r * H;
    if (hl == 31 && r < nrows) {
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

// Sum of each of R row partials over the 64 lanes of a wave (DPP, no LDS
// trips), valid in lane 63.
template <int R>
__device__ __forceinline__ void wave_reduce_rows(float (&acc)[R]) {
#pragma unroll
  for (int rr = 0; rr < R; ++rr) acc[rr] = wave64_sum(acc[rr]);
}

constexpr int kMaxChunks = 256;   // 32-k chunks per row-slice (64 groups)

// ---------------------------------------------------------------- MFMA layout
// The default for M = 1. The lanes of a wave are laid over a block of R weight
// rows (of this K-slice) so that every wave instruction reads one contiguous
// 1 KiB run, and the multiply-add runs on the matrix cores.
// In instruction i lane L = m + 16 kb reads the 16 bytes of sub-chunk kb of
// block-group 16 i + m (a block-group is one 128-k group of one row). For the
// 4 dwords j of those bytes a 16x16x32 MFMA takes A[m][.] = the lane's 8
// weights as bf16(128 + q) and B[.][n] = the matching 8 x values of lane
// (n, kb), i.e. of group 16 i + n. D[m][n] then sums W of group m against x
// of group n over the group's 128 k: the diagonal D[m][m] is group m's dot
// product (the other entries are unused). The chain starts from -136 * sum(x)
// of the group; lane (n + 16 q) holds D rows 4q..4q+3 of column n, so the
// diagonal sits in the 16 lanes with n / 4 == q, register n % 4.
// x of the slice is prepared once per workgroup in LDS: 16-byte pieces
// (group g, sub-chunk kb, dword j) in the pair order of the dequant, slot
// (4 kb + j) XOR-swizzled by (g & 15) so that the 16 lanes of a B read (16
// consecutive groups, same slot) hit 16 different bank groups.
template <int R, int I, int D, int WAVES>
__global__ __launch_bounds__(64 * WAVES) void gemv_mfma_kernel(const uint16_t* __restrict__ x,
                                                               const uint8_t* __restrict__ w,
                                                               const uint16_t* __restrict__ s,
                                                               void* __restrict__ out,
                                                               int N, int K, int gps, int bper, int brem) {
  // (13 dwords of arguments: all of them arrive preloaded in SGPRs where the
  // code object asks for kernel-argument preloading, so the first address
  // computations wait on no scalar load)
  constexpr int NTHR = 64 * WAVES;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wq = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave in the workgroup
  const int G = K / kGroup;
  const int slice = blockIdx.y;
  const int g0 = slice * gps;
  const int g1 = min(G, g0 + gps);
  const int Gs = g1 > g0 ? g1 - g0 : 0;        // groups per row in this slice
  // the workgroup owns a contiguous, balanced range of row blocks (bper or,
  // for the first brem workgroups, bper + 1; computed on the host); its waves
  // take them in turn (block b_lo + wq + WAVES * j)
  const int b_lo = (int)blockIdx.x * bper + min((int)blockIdx.x, brem);
  const int nbw = bper + ((int)blockIdx.x < brem ? 1 : 0);
  const int nb = wq < nbw ? (nbw - 1 - wq) / WAVES + 1 : 0;

  const __amdgpu_buffer_rsrc_t rx = make_rsrc(x, (uint32_t)K * 2u);
  const __amdgpu_buffer_rsrc_t rw = make_rsrc(w, (uint32_t)((uint64_t)N * (uint32_t)K / 2u));
  const __amdgpu_buffer_rsrc_t rs = make_scale_rsrc(s, (uint32_t)N * (uint32_t)G);
  const uint32_t rowb = (uint32_t)(K / 2);

  __shared__ u32x4 xlds[kMaxChunks * 4];     // 64 groups x 16 pieces
  __shared__ float clds[16 * I];              // -136 * group sum, per block-group (0 past the slice)

  // ---- x pieces of the slice (issued first: L2 hits, needed before the weights)
  constexpr int kPer = (kMaxChunks * 4 + NTHR - 1) / NTHR;
  u32x4 xv[kPer];
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    const int p = tid + NTHR * k;
    // past the slice the offset is past the extent: the hardware returns 0
    xv[k] = ld128(rx, p < Gs * 16 ? (uint32_t)(g0 * kGroup) * 2u + 16u * (uint32_t)p : 0xFFFFFFF0u);
  }

  // the wave's x requests go out ahead of its first weight request
  __builtin_amdgcn_sched_barrier(0);

  // ---- per-lane offsets of a block's loads (the same for every block; block
  // b adds b * R rows). Lane (m, kb) of instruction i reads sub-chunk kb of
  // block-group gi = 16 i + m, i.e. row gi / Gs, slice group gi % Gs. When the
  // slice is the whole row (no split) the block is one contiguous run and
  // block-group gi sits at 64 gi: a few instructions get the first request
  // out; a slice needs the row / group split (by compares: R <= 4).
  const int m = lane & 15, kb = lane >> 4;
  auto block_group = [&](int gi, int& r, int& gin) {
    r = 0;
    gin = gi;
#pragma unroll
    for (int rr = 1; rr < R; ++rr)
      if (gin >= Gs) { gin -= Gs; ++r; }
  };
  uint32_t woff[I], soff[I];
  if (Gs == G) {
#pragma unroll
    for (int i = 0; i < I; ++i) {
      const uint32_t gi = (uint32_t)(16 * i + m);
      const bool ok = gi < (uint32_t)(R * G);
      woff[i] = ok ? gi * 64u + (uint32_t)kb * 16u : 0xFFFFFFF0u;
      soff[i] = ok ? gi * 2u : 0xFFFFFFF0u;
    }
  } else {
#pragma unroll
    for (int i = 0; i < I; ++i) {
      const int gi = 16 * i + m;
      const bool ok = gi < R * Gs;
      int r, gin;
      block_group(gi, r, gin);
      // invalid lanes read past the extent (zeros); their products are masked by rmask
      woff[i] = ok ? (uint32_t)r * rowb + (uint32_t)(g0 + gin) * 64u + (uint32_t)kb * 16u : 0xFFFFFFF0u;
      soff[i] = ok ? ((uint32_t)r * (uint32_t)G + (uint32_t)(g0 + gin)) * 2u : 0xFFFFFFF0u;
    }
  }

  // ---- weight ring. Every slot is refilled after it is consumed, also past
  // the wave's last block: such loads (and those of rows past N) use an
  // offset past the buffer extent, which the hardware answers with zeros and
  // no memory traffic, so the ring has the same wait counts on every trip.
  u32x4 wbuf[D][I];
  uint32_t sbuf[D][I];
  auto issue = [&](u32x4 (&wb)[I], uint32_t (&sb)[I], int jb) {
    // a dead block (or lane) has base (or offset) 0xFFFFFFF0; the saturating
    // add keeps any sum with it at or above that, past every extent
    const bool live = jb < nb;
    const uint32_t b = (uint32_t)(b_lo + wq + jb * WAVES);
    const uint32_t wbase = live ? b * (uint32_t)R * rowb : 0xFFFFFFF0u;
    const uint32_t sbase = live ? b * (uint32_t)R * (uint32_t)G * 2u : 0xFFFFFFF0u;
#pragma unroll
    for (int i = 0; i < I; ++i) sb[i] = ld32(rs, __builtin_elementwise_add_sat(sbase, soff[i]) & ~3u);
#pragma unroll
    for (int i = 0; i < I; ++i)
      wb[i] = __builtin_amdgcn_raw_buffer_load_b128(rw, __builtin_elementwise_add_sat(wbase, woff[i]), 0, 2);
    // keep one block's loads together, in issue order
    __builtin_amdgcn_sched_barrier(0);
  };
  // D - 1 blocks requested up front (one when D = 1); each step then
  // requests one more block (see the loop at the end)
#pragma unroll
  for (int jb = 0; jb < (D > 1 ? D - 1 : 1); ++jb) issue(wbuf[jb], sbuf[jb], jb);

  // ---- the rest of the per-lane mapping, needed only when a block is consumed
  uint32_t xaddr[I], sshift[I];
  float rmask[I][R];
#pragma unroll
  for (int i = 0; i < I; ++i) {
    const int gi = 16 * i + m;
    const bool ok = gi < R * Gs;
    int r, gin;
    block_group(gi, r, gin);
    if (!ok) r = gin = 0;
    // scales are read as the aligned 32-bit word that holds them (16-bit
    // loads get packed in pairs by the compiler, which ties the wait of one
    // block to the next one's loads); in block 0 the lane's scale is the low
    // half (shift 16 into the bf16 position) when its offset is 4-aligned
    sshift[i] = (soff[i] & 2u) ? 0u : 16u;
    // LDS byte address of piece (gin, kb, j = 0); piece j is at xaddr ^ (16 j)
    xaddr[i] = (uint32_t)gin * 256u + 16u * ((uint32_t)(4 * kb) ^ (uint32_t)(gin & 15));
#pragma unroll
    for (int rr = 0; rr < R; ++rr) rmask[i][rr] = (ok && r == rr) ? 1.0f : 0.0f;
  }
  // one-hot of the diagonal register: lane (n + 16 q) holds D[4q + j][n]
  float onehot[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) onehot[j] = (m == 4 * kb + j) ? 1.0f : 0.0f;

  // ---- prepare x in LDS: pair-interleave, swizzle, per-group -136 * sum
  for (int e = tid; e < 16 * I; e += NTHR) clds[e] = 0.0f;
  __syncthreads();
  const uint32_t ones = vgpr_const(0x3F803F80u);
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    const int p = tid + NTHR * k;               // piece p = 16 g + 4 kb + j
    const u32x4 v = xv[k];                      // zeros past the slice
    u32x4 o;
    o.x = __builtin_amdgcn_perm(v.z, v.x, 0x05040100u);
    o.y = __builtin_amdgcn_perm(v.z, v.x, 0x07060302u);
    o.z = __builtin_amdgcn_perm(v.w, v.y, 0x05040100u);
    o.w = __builtin_amdgcn_perm(v.w, v.y, 0x07060302u);
    const int g = p >> 4, slot = (p & 15) ^ (g & 15);
    if (p < kMaxChunks * 4) xlds[16 * g + slot] = o;
    float sx = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(v.x), as_bf16x2(ones), 0.0f, false);
    sx = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(v.y), as_bf16x2(ones), sx, false);
    sx = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(v.z), as_bf16x2(ones), sx, false);
    sx = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(v.w), as_bf16x2(ones), sx, false);
    // 16 consecutive pieces form one group (p = tid + NTHR k, NTHR % 16 == 0):
    // one DPP row of 16 lanes
    sx = row16_sum(sx);
    if (p < Gs * 16 && (p & 15) == 0) {
#pragma unroll
      for (int r = 0; r < R; ++r)
        if (r * Gs + g < 16 * I) clds[r * Gs + g] = -136.0f * sx;   // per block-group
    }
  }
  __syncthreads();

  const uint32_t magic = vgpr_const(kMagicPair);
  const uint32_t mask = __builtin_amdgcn_readfirstlane(vgpr_const(kNibblePairMask));

  // x in registers: every lane reads its B operands and initial C once from
  // LDS; the empty asm makes them opaque, so the compiler keeps them live
  // across blocks instead of re-reading LDS per block (x re-read from LDS per
  // block ran 12.9 against 11.2 us)
  u32x4 xr[I][4];
  f32x4 cr[I];
#pragma unroll
  for (int i = 0; i < I; ++i) {
    cr[i] = *reinterpret_cast<const f32x4*>(reinterpret_cast<const uint8_t*>(clds) +
                                            4u * (uint32_t)(16 * i + 4 * kb));
#pragma unroll
    for (int j = 0; j < 4; ++j)
      xr[i][j] = *reinterpret_cast<const u32x4*>(reinterpret_cast<const uint8_t*>(xlds) +
                                                 (xaddr[i] ^ (16u * (uint32_t)j)));
  }
#pragma unroll
  for (int i = 0; i < I; ++i) {
    asm volatile("" : "+v"(cr[i]));
#pragma unroll
    for (int j = 0; j < 4; ++j) asm volatile("" : "+v"(xr[i][j]));
  }

  auto consume = [&](const u32x4 (&wb)[I], const uint32_t (&sb)[I], int jb) {
    // block b's scale offsets are block 0's + b * R * G * 2: when R * G is odd
    // and b is odd, every lane's scale sits in the other half of its word
    const uint32_t flip = ((uint32_t)(b_lo + wq + jb * WAVES) & (uint32_t)(R * G) & 1u) << 4;
    float acc[R];
#pragma unroll
    for (int rr = 0; rr < R; ++rr) acc[rr] = 0.0f;
    // instruction group i: B operands (x) and initial C (-136 * sum(x) of
    // block-groups 16 i + 4 q + 0..3, the rows of D in this lane) from the
    // registers above
#pragma unroll
    for (int i = 0; i < I; ++i) {
      f32x4 c = cr[i];
      bf16x8 bq[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) bq[j] = __builtin_bit_cast(bf16x8, xr[i][j]);
      const uint32_t wd[4] = {wb[i].x, wb[i].y, wb[i].z, wb[i].w};
      {
        // two dwords per 64-bit shift
        uint32_t w4[4], w8[4], w12[4];
        shr64_pair<4>(wd[0], wd[1], w4[0], w4[1]);
        shr64_pair<4>(wd[2], wd[3], w4[2], w4[3]);
        shr64_pair<8>(wd[0], wd[1], w8[0], w8[1]);
        shr64_pair<8>(wd[2], wd[3], w8[2], w8[3]);
        shr64_pair<12>(wd[0], wd[1], w12[0], w12[1]);
        shr64_pair<12>(wd[2], wd[3], w12[2], w12[3]);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const bf16x8 a = __builtin_bit_cast(bf16x8, u32x4{(wd[j] & mask) | magic, (w4[j] & mask) | magic,
                                                            (w8[j] & mask) | magic, (w12[j] & mask) | magic});
          c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bq[j], c, 0, 0, 0);
        }
      }
      const float v = (c.x * onehot[0] + c.y * onehot[1]) + (c.z * onehot[2] + c.w * onehot[3]);
      const float sv = __uint_as_float((sb[i] << (sshift[i] ^ flip)) & 0xFFFF0000u) * v;
#pragma unroll
      for (int rr = 0; rr < R; ++rr) acc[rr] = fmaf(rmask[i][rr], sv, acc[rr]);
    }
    wave_reduce_rows<R>(acc);
    if (lane == 63 && jb < nb) {
      // one slice: bf16 y; several: fp32 partials of this slice
      const bool partials = gridDim.y > 1;
#pragma unroll
      for (int rr = 0; rr < R; ++rr) {
        const int n = (b_lo + wq + jb * WAVES) * R + rr;
        if (n < N) {
          if (!partials) static_cast<uint16_t*>(out)[n] = to_bf16(acc[rr]);
          else static_cast<float*>(out)[(size_t)slice * N + n] = acc[rr];
        }
      }
    }
  };

  // Ring of D register sets: block j + D - 1 is requested as soon as block
  // j - 1 is consumed, before block j is waited for and consumed, so a
  // block's consume overlaps the flight of the next D - 1 (with the request
  // after the consume, each block's dequant and MFMAs added to every wave's
  // chain of round trips: D = 2 took 1 x 17408 x 5120 from 9.66 to 9.45 us).
  // Every step issues the same loads (dead blocks read nothing), so the
  // compiler's waits are the same counts on every trip.
  // D = 1 (one register set): the next block is requested after the
  // current one is consumed.
  if constexpr (D == 1) {
    for (int j = 0; j < nb; ++j) {
      consume(wbuf[0], sbuf[0], j);
      issue(wbuf[0], sbuf[0], j + 1);
    }
  } else {
    for (int j0 = 0; j0 < nb; j0 += D) {
#pragma unroll
      for (int u = 0; u < D; ++u) {
        issue(wbuf[(u + D - 1) % D], sbuf[(u + D - 1) % D], j0 + u + D - 1);
        if (j0 + u < nb) consume(wbuf[u], sbuf[u], j0 + u);
      }
    }
  }
}

// MFMA-layout geometry: a block of R rows holds 16 * I groups (R <= 4, I <= 8)
static bool mfma_geometry(int gs, int* R, int* I) {
  int g = 16, a = gs;
  while (a % 2 == 0 && g > 1) { a /= 2; g /= 2; }   // g = 16 / gcd(gs, 16)
  *R = g;
  *I = g * gs / 16;
  return gs > 0 && *R <= 4 && *I >= 1 && *I <= 8;
}

// Compute units of the current device (cached per device).
static int cu_count() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int v = cache[dev].load(std::memory_order_relaxed);
  if (v == 0) {
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0) v = 256;
    cache[dev].store(v, std::memory_order_relaxed);
  }
  return v;
}

// One 8-wave workgroup per compute unit, x held in registers. A ring of two
// weight blocks per wave where the waves average two blocks or more (with
// about one block per wave the ring only adds dead requests: 1 x 6144 x 2560
// 4.78 -> 4.94 us) and a block is under 7 instructions (a second register
// set of 7 spills).
template <int R, int I>
static hipError_t launch_mfma_ri(const uint16_t* x, const uint8_t* w, const uint16_t* s, uint16_t* y, float* ws,
                                 int N, int K, int gps, int sk, hipStream_t stream) {
  constexpr int kWaves = 8;
  const int nblk = (N + R - 1) / R;
  const int gx = std::max(1, std::min(cu_count(), (nblk + kWaves - 1) / kWaves));
  const int bper = nblk / gx, brem = nblk - bper * gx;
  void* out = sk > 1 ? static_cast<void*>(ws) : static_cast<void*>(y);
  if constexpr (I < 7) {
    if (bper >= 2 * kWaves) {
      hipLaunchKernelGGL((gemv_mfma_kernel<R, I, 2, kWaves>), dim3(gx, sk), dim3(64 * kWaves), 0, stream, x, w, s,
                         out, N, K, gps, bper, brem);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((gemv_mfma_kernel<R, I, 1, kWaves>), dim3(gx, sk), dim3(64 * kWaves), 0, stream, x, w, s, out,
                     N, K, gps, bper, brem);
  return hipGetLastError();
}

// Half-wave layout (slices with no MFMA geometry): two rows in flight per
// half-wave, about four rows per half-wave, non-temporal weight loads.
template <int CPL>
static hipError_t launch_halfwave(const uint16_t* x, const uint8_t* w, const uint16_t* s, uint16_t* y, float* ws,
                                  int N, int K, int gps, int sk, hipStream_t stream) {
  constexpr int kRowsPerHalfwave = 4;
  const int halfwaves = (N + kRowsPerHalfwave - 1) / kRowsPerHalfwave;
  const int blocks = (halfwaves + 7) / 8;
  hipLaunchKernelGGL((gemv_m1_kernel<CPL, 2, 2>), dim3(blocks > 0 ? blocks : 1, sk), dim3(256), 0, stream, x, w, s,
                     y, ws, N, K, gps);
  return hipGetLastError();
}

hipError_t launch_gemv_m1(const uint16_t* x, const uint8_t* w, const uint16_t* s, uint16_t* y, float* ws, int N,
                          int K, int gps, int sk, bool force_halfwave, hipStream_t stream) {
  int R = 0, I = 0;
  if (!force_halfwave && mfma_geometry(gps, &R, &I)) {
#define W4A16_RI(RR, II) \
  if (R == RR && I == II) return launch_mfma_ri<RR, II>(x, w, s, y, ws, N, K, gps, sk, stream);
    W4A16_RI(1, 1) W4A16_RI(1, 2) W4A16_RI(1, 3) W4A16_RI(1, 4)
    W4A16_RI(2, 1) W4A16_RI(2, 3) W4A16_RI(2, 5) W4A16_RI(2, 7)
    W4A16_RI(4, 1) W4A16_RI(4, 3) W4A16_RI(4, 5) W4A16_RI(4, 7)
#undef W4A16_RI
  }
  // the half-wave kernel takes every slice of at most 64 groups
  switch ((gps * 4 + 31) / 32) {   // 32-k chunks per lane in a slice
    case 1: return launch_halfwave<1>(x, w, s, y, ws, N, K, gps, sk, stream);
    case 2: return launch_halfwave<2>(x, w, s, y, ws, N, K, gps, sk, stream);
    case 3: return launch_halfwave<3>(x, w, s, y, ws, N, K, gps, sk, stream);
    case 4: return launch_halfwave<4>(x, w, s, y, ws, N, K, gps, sk, stream);
    case 5: return launch_halfwave<5>(x, w, s, y, ws, N, K, gps, sk, stream);
    case 6: return launch_halfwave<6>(x, w, s, y, ws, N, K, gps, sk, stream);
    case 7: return launch_halfwave<7>(x, w, s, y, ws, N, K, gps, sk, stream);
    case 8: return launch_halfwave<8>(x, w, s, y, ws, N, K, gps, sk, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace w4a16
