// Prefill / grouped W4A16 GEMM for gfx950 with LDS-DMA staging and in-register
// dequantisation.
//
// Numerics: the weight operand is bf16(128 + q), exact, from the
// magic-constant OR ("[ROCm][Kernel] W4A16 skinny GEMM: hand-asm kernel for
// gfx1151", section 1); each 128-group's MFMA chain of a 16x16 output tile
// starts from -136 * sum_{k in g} x[m, k], so after the group's 4 MFMA steps it
// holds sum_k x * (q - 8) in fp32, which is scaled by the column's bf16 scale
// and added to the fp32 accumulator. No weight is ever rounded. The row sums
// are formed in the kernel, on the matrix core: an MFMA of the X fragments
// against a constant bf16(-136) operand gives -136 * sum_k x[m, k] in every
// output column; the MS row tiles of a stage are spread over the 8 waves and
// done one group ahead, into the stage's row-sum slots.
//
// Structure (one 512-thread workgroup per (16 MS) x 256 output tile, 8 waves
// of (16 MS) x 32, MS = 3 .. 9; one workgroup per compute unit):
//  * one K-stage = one 128-group: X [16 MS rows, 128 k] bf16 and the packed
//    weights [256 rows, 64 B] (16 KiB, still 4-bit), filled by buffer loads
//    that write LDS directly (no registers, no VALU), issued two groups
//    ahead, and the 16 MS row sums (-136 * sum x) written by the waves one
//    group ahead; three stages in LDS;
//  * each wave reads its 32 columns of packed weights once per group and
//    dequantises them in registers (32 VGPRs of bf16 B operands), then sweeps
//    the MS row tiles of 16: 4 MFMA 16x16x32 steps per (row tile, column
//    tile), one rescale FMA per output element per group. A dequantised
//    fragment serves MS row tiles: with VALU ops issuing only about every 8
//    cycles while the matrix core is busy, dequant + rescale must stay near 2
//    VALU ops per 16-cycle MFMA, which the taller tile (MS = 14) meets;
//  * within a group the MFMA k order is permuted: lane (r, kb) of step st
//    holds k = 32 kb + 8 st + 0..7 for both operands, so one lane's four steps
//    of packed weights are one 16-byte LDS read;
//  * LDS rows are XOR-swizzled in 16-byte chunks (X rows by xswz(row & 15),
//    weights by (row >> 1) & 3): the DMA lanes fetch the chunk that belongs
//    at their LDS slot, and the MFMA operand reads are free of bank
//    conflicts (4 LDS cycles per 16-byte read of a wave; see xswz);
//  * one barrier per group, after an explicit wait for the next group's DMA.
// The M tail and N tail read zeros through the exact buffer extents; stores
// past the last row are dropped and columns >= N are skipped.
#include <type_traits>

#include "common.hpp"
#include "launch.hpp"
#include "tilemap.hpp"

namespace w4a16 {

namespace {

constexpr int kPN = 256;                    // columns per tile (8 waves x 32)
constexpr int kNW = 8;                      // waves per workgroup
constexpr int kWStage = kPN * 64;           // packed W: 256 rows x 128 k / 2

// LDS stage of a tile with MS row tiles of 16 (one 128-k stage): X, packed
// W, the row sums of its 128 / GS scale groups
template <int MS, int GS = 128>
struct Stage {
  static constexpr int kRows = 16 * MS;
  static constexpr int kX = kRows * 256;     // X: rows x 128 k x 2 B
  static constexpr int kW = kWStage;
  static constexpr int kR = kRows * 4 * (128 / GS);   // -136 * row sums, fp32, [128 / GS][rows]
  static constexpr int kBytes = kX + kW + kR;
};

struct PrefillArgs {
  const uint16_t* x;       // [M_total, K]
  const uint8_t* w;        // [G, N, K/2]
  const uint16_t* s;       // [G, N, K/GS]
  const float* sxn;        // [K/GS, ld] -136 * row sums from the pre-pass (RSK false), else unused
  uint16_t* y;             // [M_total, N]
  float* ws;               // [SK, M_total, N] fp32 split-K partials, or nullptr
  const int32_t* m_sizes;  // [G] on device, or nullptr
  int m_uniform;           // batched: rows per weight group (M_sizes not used), else 0
  int M_total, N, K, G, ld;
  int gps;                 // 128-groups per split-K slice
  int mtiles, ntiles;
};

// s_waitcnt with only the vector-memory counter limited (gfx9 encoding:
// vmcnt in bits 3:0 and 15:14, expcnt and lgkmcnt at their maxima), followed
// by a workgroup barrier. The "memory" clobber keeps LDS reads on their side.
template <int VM>
__device__ __forceinline__ void wait_vm_barrier() {
  static_assert(VM >= 0 && VM < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(VM) : "memory");
}

__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, uint8_t* lds_dst, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds_dst, 16, voff, soff, 0, 0);
}

}  // namespace

template <int NSTAGE, int MS, int GS, bool RSK>
__global__ __launch_bounds__(64 * kNW) void prefill_kernel(const PrefillArgs args) {
  static_assert(NSTAGE == 3, "stages: the row sums of group j + 1 are formed while group j + 2 is in flight");
  static_assert(MS >= 2 && MS <= 16, "row tiles");
  static_assert(GS == 128 || GS == 32, "scale group");
  constexpr int NSG = 128 / GS;         // scale groups per 128-k stage
  using ST = Stage<MS, GS>;
  constexpr int BM = ST::kRows;
  constexpr int TN = kPN / kNW;         // columns per wave (32)
  constexpr int SN = TN / 16;           // 16-column MFMA tiles per wave (2)
  constexpr int NQX = 4 * MS;           // X DMA instructions per group (4 rows of 256 B each)
  constexpr int QX = (NQX + kNW - 1) / kNW;   // per wave (block q = wave + 8 i)
  constexpr int QW = 16 / kNW;          // W DMA instructions per wave and group
  constexpr int RL = 4 * MS;            // row-sum DMA lanes (16 B = 4 rows each), RSK false
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int Gk = args.K / kGroup;       // 128-k stages
  const int Gs = args.K / GS;           // scale groups

  int mt, nt;
  int MT = args.mtiles, nblocks = (int)gridDim.x;
  if (args.m_sizes != nullptr) {
    MT = real_mtiles(BM, args.M_total, args.m_sizes, args.G);
    nblocks = MT * args.ntiles;
    if ((int)blockIdx.x >= nblocks) return;
  }
  tile_coords(blockIdx.x, nblocks, MT, args.ntiles, &mt, &nt);
  const TileRows tr = tile_rows(mt, BM, args.M_total, args.m_sizes, args.G, args.m_uniform);
  if (tr.rows <= 0) return;
  const int row0 = tr.row0, rows = tr.rows;
  const int n0 = nt * kPN;
  const int ncols = min(kPN, args.N - n0);

  const uint32_t K2 = (uint32_t)args.K / 2u;
  const uint32_t KB = (uint32_t)args.K * 2u;   // bytes per X row
  const __amdgpu_buffer_rsrc_t rx = make_rsrc(args.x + (size_t)row0 * args.K, (uint32_t)rows * KB);
  const __amdgpu_buffer_rsrc_t rw =
      make_rsrc(args.w + ((size_t)tr.wg * args.N + n0) * K2, (uint32_t)ncols * K2);
  // scales: the whole tensor (word-aligned reads, see make_scale_rsrc); columns
  // past N read other scales or zeros and are never stored
  const __amdgpu_buffer_rsrc_t rs =
      make_scale_rsrc(args.s, (uint32_t)((size_t)args.G * args.N * Gs));
  // row sums of the pre-pass (RSK false): [K/GS, ld] fp32, from this tile's first row
  const __amdgpu_buffer_rsrc_t rsx =
      make_rsrc(RSK ? nullptr : args.sxn + row0, RSK ? 0u : (uint32_t)(((size_t)Gs * args.ld - row0) * 4u));
  const int slice = blockIdx.y;
  const int gb = slice * args.gps;
  const int ge = min(Gk, gb + args.gps);
  const int ng = ge > gb ? ge - gb : 0;

  // ---- DMA lane offsets (constant over groups)
  // X instruction i of wave wv fills LDS block q = wv + 8 i (if q < 4 MS),
  // i.e. tile rows 4 q + (lane >> 4), slot lane & 15; the chunk stored in
  // slot p of row r is p ^ xswz(r & 15), and r & 15 = 4 (q & 3) + (lane >> 4)
  // with q & 3 = wv & 3 for every i: row offset 4 (q & ~3) KB plus xvo().
  // (recomputed from the lane id at each issue: a few VALU ops per group
  // instead of registers held across the main loop)
  auto xvo = [&]() {
    const int r = 4 * (wv & 3) + (lane >> 4), xp = lane & 15;
    return (uint32_t)r * KB + 16u * ((uint32_t)xp ^ xswz(r));
  };
  // W instruction i fills block q = QW wv + i: tile rows 16 q + (lane >> 2),
  // slot lane & 3; the chunk stored in slot p of row r is p ^ ((r >> 1) & 3).
  auto wvo = [&]() {
    const int wr = lane >> 2, wp = lane & 3;
    return (uint32_t)(16 * QW * wv + wr) * K2 + 16u * (uint32_t)(wp ^ ((wr >> 1) & 3));
  };

  // byte offset of a stage, kept in a scalar register: every LDS address of
  // the stage is then one add of it to a loop-invariant lane offset
  auto stage_off = [&](int stage) { return __builtin_amdgcn_readfirstlane((uint32_t)stage * (uint32_t)ST::kBytes); };
  // Row offsets always go into the vector offset, which the hardware range
  // checks against the buffer extent (rows past the tile read zeros); the
  // scalar offset only carries the group's k offset, which stays inside a row.
  auto issue = [&](int g, int stage) {
    uint8_t* base = lds + stage_off(stage);
    // the group is the same in every lane; keeping its offsets scalar avoids
    // a waterfall loop around each load
    const uint32_t gx = __builtin_amdgcn_readfirstlane((uint32_t)g * 256u);
    const uint32_t gw = __builtin_amdgcn_readfirstlane((uint32_t)g * 64u);
    const uint32_t xo = xvo();
#pragma unroll
    for (int i = 0; i < QX; ++i) {
      const int q = wv + kNW * i;   // wave-uniform
      if (NQX % kNW == 0 || q < NQX) dma16(rx, base + 1024 * q, xo + (uint32_t)(4 * (q & ~3)) * KB, gx);
    }
    const uint32_t wo = wvo();
#pragma unroll
    for (int i = 0; i < QW; ++i) dma16(rw, base + ST::kX + 1024 * (QW * wv + i), wo + (uint32_t)i * 16u * K2, gw);
    // RSK false: wave sg < NSG fetches the row sums of scale group sg of the
    // stage, lanes 0 .. RL - 1 four rows each
    if (!RSK && wv < NSG && lane < RL)
      dma16(rsx, base + ST::kX + ST::kW + ST::kRows * 4 * wv,
            (uint32_t)(4 * lane) * 4u + (uint32_t)(NSG * g + wv) * (uint32_t)args.ld * 4u, 0u);
  };

  // ---- scales: GS = 128: the aligned word holding s[n][g] for this lane's
  // SN columns; GS = 32: the stage's four scales s[n][4 g .. 4 g + 3], one
  // 8-byte load (aligned: K / 32 is a multiple of 4)
  const int m16 = lane & 15, kb = lane >> 4;
  using SW = typename std::conditional<GS == 128, uint32_t, u32x2>::type;
  uint32_t soff[SN];
#pragma unroll
  for (int ns = 0; ns < SN; ++ns)
    soff[ns] = (uint32_t)((size_t)tr.wg * args.N + n0 + TN * wv + 16 * ns + m16) * (uint32_t)Gs * 2u;
  // GS = 32: the group's offset goes into the scalar offset (soff is a
  // multiple of 8; a lane whose vector offset is in range holds a real row,
  // and the 8 bytes lie in that row; a lane past the extent reads zeros)
  auto load_scales = [&](SW (&sw)[SN], int g) {
#pragma unroll
    for (int ns = 0; ns < SN; ++ns) {
      if constexpr (GS == 128) sw[ns] = ld32(rs, (soff[ns] + 2u * (uint32_t)g) & ~3u);
      else sw[ns] = ld64(rs, soff[ns], __builtin_amdgcn_readfirstlane(8u * (uint32_t)g));
    }
  };
  // s[n][g] is the high half of its word where soff + 2 g has bit 1 set; the
  // parity of soff is the lane's (the same for its SN columns), that of 2 g
  // flips with g: a byte permute with a per-lane selector, flipped once per
  // group, moves the half into the top of an fp32 (one VALU op per column)
  const uint32_t sel_base = (soff[0] & 2u) ? 0x03020C0Cu : 0x01000C0Cu;
  auto scale_sel = [&](int g) { return sel_base ^ ((g & 1) ? 0x02020000u : 0u); };
  auto scale_of = [&](uint32_t word, uint32_t sel) { return __uint_as_float(__builtin_amdgcn_perm(word, word, sel)); };
  // scale group st (0..3) of a stage's four, GS = 32
  auto scale32 = [](u32x2 w, int st) {
    const uint32_t v = st < 2 ? w.x : w.y;
    return __uint_as_float((st & 1) ? (v & 0xFFFF0000u) : (v << 16));
  };

  // ---- LDS operand offsets within a stage
  // A (X): row 16 ms + m16, logical chunk 4 kb + st, slot chunk ^ xswz(m16)
  // (4 kb + st) ^ x = ((4 kb) ^ x) ^ st: one base register
  const uint32_t aoff0 = (uint32_t)m16 * 256u + 16u * ((uint32_t)(4 * kb) ^ xswz(m16));
  // B (packed W): row TN wv + 16 ns + m16, logical chunk kb
  const uint32_t boff = ST::kX + (uint32_t)(TN * wv + m16) * 64u + 16u * (uint32_t)(kb ^ ((m16 >> 1) & 3));
  // C init: -136 * row sums of rows 16 ms + 4 kb + 0..3
  const uint32_t roff = ST::kX + ST::kW + 16u * (uint32_t)kb;

  const uint32_t magic = vgpr_const(kMagicPair);
  const uint32_t mask = __builtin_amdgcn_readfirstlane(vgpr_const(kNibblePairMask));

  f32x4 acc[MS][SN];
#pragma unroll
  for (int ms = 0; ms < MS; ++ms)
#pragma unroll
    for (int ns = 0; ns < SN; ++ns) acc[ms][ns] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

  SW sc_cur[SN], sc_nxt[SN];

  // GS = 32 operand offsets (natural k order, see below)
  const uint32_t aoffN = (uint32_t)m16 * 256u + 16u * ((uint32_t)kb ^ xswz(m16));
  const uint32_t boffN = ST::kX + (uint32_t)(TN * wv + m16) * 64u + 4u * (uint32_t)kb + 16u * (uint32_t)((m16 >> 1) & 3);
  // ---- -136 * row sums of a landed stage, on the matrix core: MFMA steps of
  // the X fragments against a constant bf16(-136) operand give D[m][n] =
  // -136 * sum_k x[m, k] in every column n, so the lanes of column 0 (lane
  // (0, kb) holds rows 4 kb + 0..3) store the tile's 16 sums. GS = 128: the
  // group's four steps chained (any k order sums the whole group); GS = 32:
  // step st alone is 32-group st (natural k order). Row tile ms of the stage
  // is taken by wave (ms + j) mod 8, so that the extra tile of MS > 8 moves
  // from wave to wave with the group j. Products x * 136 are exact in fp32.
  // The MFMAs are issued at the start of a group's compute and their results
  // stored after its dequantisation, so no wave waits on them.
  constexpr int RSM = (MS + kNW - 1) / kNW;   // row tiles of sums per wave, at most
  const uint32_t neg136 = vgpr_const(0xC308C308u);   // bf16(-136) pair
  const bf16x8 bneg = __builtin_bit_cast(bf16x8, u32x4{neg136, neg136, neg136, neg136});
  auto rs_tile = [&](int j, int i) { return ((wv - j) & (kNW - 1)) + kNW * i; };   // wave-uniform
  auto rs_issue = [&](int stage, int j, f32x4 (&d)[RSM][NSG]) {
    const uint8_t* sb = lds + stage_off(stage);
#pragma unroll
    for (int i = 0; i < RSM; ++i) {
      const int ms = rs_tile(j, i);
      if (ms < MS) {
        if constexpr (GS == 128) {
          d[i][0] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int st = 0; st < 4; ++st) {
            const bf16x8 a =
                *reinterpret_cast<const bf16x8*>(sb + (aoff0 ^ (16u * (uint32_t)st)) + 4096u * (uint32_t)ms);
            d[i][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bneg, d[i][0], 0, 0, 0);
          }
        } else {
#pragma unroll
          for (int st = 0; st < 4; ++st) {
            const bf16x8 a =
                *reinterpret_cast<const bf16x8*>(sb + (aoffN ^ (64u * (uint32_t)st)) + 4096u * (uint32_t)ms);
            d[i][st] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bneg, f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
          }
        }
      }
    }
  };
  auto rs_store = [&](int stage, int j, const f32x4 (&d)[RSM][NSG]) {
    uint8_t* sb = lds + stage_off(stage);
#pragma unroll
    for (int i = 0; i < RSM; ++i) {
      const int ms = rs_tile(j, i);
      if (ms < MS && m16 == 0) {
#pragma unroll
        for (int st = 0; st < NSG; ++st)
          *reinterpret_cast<f32x4*>(sb + roff + (uint32_t)(ST::kRows * 4 * st) + 64u * (uint32_t)ms) = d[i][st];
      }
    }
  };

  // GS = 32: MFMA step st covers scale group st of the stage (natural k
  // order: lane (r, kb) of step st holds k = 32 st + 8 kb + 0..7 for both
  // operands), each step starts from its group's row sums and is rescaled on
  // its own. A: chunk 4 st + kb of the row, slot (4 st + kb) ^ xswz(row) =
  // ((kb ^ xswz(row)) ^ 4 st); B: dword kb of chunk st of the packed row, slot
  // st ^ ((row >> 1) & 3).
  auto compute32 = [&](int stage, int rstage, int j) {
    if constexpr (GS == 32) {
    const uint8_t* sb = lds + stage_off(stage);
    f32x4 rsd[RSM][NSG];
    // row tile ms's operands: the 4 steps' initial C (row sums of the
    // stage's four 32-groups) and A fragments; the next row tile's reads go
    // out before this tile's MFMAs (two register sets)
    f32x4 cq[2][NSG];
    bf16x8 aq[2][4];
    auto read_rows = [&](int ms, f32x4 (&c)[NSG], bf16x8 (&a)[4]) {
#pragma unroll
      for (int st = 0; st < NSG; ++st)
        c[st] = *reinterpret_cast<const f32x4*>(sb + roff + (uint32_t)(ST::kRows * 4 * st) + 64u * (uint32_t)ms);
#pragma unroll
      for (int st = 0; st < 4; ++st)
        a[st] = *reinterpret_cast<const bf16x8*>(sb + (aoffN ^ (64u * (uint32_t)st)) + 4096u * (uint32_t)ms);
    };
    read_rows(0, cq[0], aq[0]);
    if (rstage >= 0) rs_issue(rstage, j, rsd);
    bf16x8 bd[SN][4];
#pragma unroll
    for (int ns = 0; ns < SN; ++ns)
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        const uint32_t w0 = *reinterpret_cast<const uint32_t*>(sb + (boffN ^ (16u * (uint32_t)st)) + 1024u * (uint32_t)ns);
        const uint32_t w4 = w0 >> 4;
        u32x4 o;
        o.x = and_or_sv(__builtin_amdgcn_perm(w4, w0, 0x0C040C00u), mask, magic);
        o.y = and_or_sv(__builtin_amdgcn_perm(w4, w0, 0x0C050C01u), mask, magic);
        o.z = and_or_sv(__builtin_amdgcn_perm(w4, w0, 0x0C060C02u), mask, magic);
        o.w = and_or_sv(__builtin_amdgcn_perm(w4, w0, 0x0C070C03u), mask, magic);
        bd[ns][st] = __builtin_bit_cast(bf16x8, o);
      }
    float scv[SN][4];
#pragma unroll
    for (int ns = 0; ns < SN; ++ns)
#pragma unroll
      for (int st = 0; st < 4; ++st) scv[ns][st] = scale32(sc_cur[ns], st);
    if (rstage >= 0) rs_store(rstage, j, rsd);
    // step st's products are rescaled after the next step's MFMAs are issued
    // (the last step's after the next row tile's first step), so no MFMA
    // result is read right behind its issue; the empty asm pins each rescale
    // there, otherwise all steps' products stay live
    f32x4 t[2][SN];
    auto rescale = [&](const f32x4 (&u)[SN], int ms, int st) {
#pragma unroll
      for (int ns = 0; ns < SN; ++ns) {
        acc[ms][ns].x = fmaf(scv[ns][st], u[ns].x, acc[ms][ns].x);
        acc[ms][ns].y = fmaf(scv[ns][st], u[ns].y, acc[ms][ns].y);
        acc[ms][ns].z = fmaf(scv[ns][st], u[ns].z, acc[ms][ns].z);
        acc[ms][ns].w = fmaf(scv[ns][st], u[ns].w, acc[ms][ns].w);
        asm volatile("" : "+v"(acc[ms][ns]));
      }
    };
#pragma unroll
    for (int ms = 0; ms < MS; ++ms) {
      const int cur = ms & 1;
      if (ms + 1 < MS) read_rows(ms + 1, cq[(ms + 1) & 1], aq[(ms + 1) & 1]);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int st = 0; st < 4; ++st) {
#pragma unroll
        for (int ns = 0; ns < SN; ++ns)
          t[st & 1][ns] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aq[cur][st], bd[ns][st], cq[cur][st], 0, 0, 0);
        if (st > 0) rescale(t[(st - 1) & 1], ms, st - 1);
        else if (ms > 0) rescale(t[1], ms - 1, 3);
      }
    }
    rescale(t[1], MS - 1, 3);
    }
  };

  auto compute = [&](int stage, int g, int rstage, int j) {
    if constexpr (GS == 128) {
    const uint8_t* sb = lds + stage_off(stage);
    f32x4 rsd[RSM][NSG];
    // row tile ms's operands: initial C and the 4 steps' A fragments; the next
    // row tile's reads go out before this tile's MFMAs (two register sets)
    f32x4 cq[2];
    bf16x8 aq[2][4];
    auto read_rows = [&](int ms, f32x4& c0, bf16x8 (&a)[4]) {
      c0 = *reinterpret_cast<const f32x4*>(sb + roff + 64u * (uint32_t)ms);
#pragma unroll
      for (int st = 0; st < 4; ++st)
        a[st] = *reinterpret_cast<const bf16x8*>(sb + (aoff0 ^ (16u * (uint32_t)st)) + 4096u * (uint32_t)ms);
    };
    read_rows(0, cq[0], aq[0]);
    if (rstage >= 0) rs_issue(rstage, j, rsd);
    // dequantise this wave's TN columns x 128 k: bd[ns][st] = 8 bf16 (128 + q)
    bf16x8 bd[SN][4];
#pragma unroll
    for (int ns = 0; ns < SN; ++ns) {
      const u32x4 pk = *reinterpret_cast<const u32x4*>(sb + boff + 1024u * (uint32_t)ns);
      const uint32_t wd[4] = {pk.x, pk.y, pk.z, pk.w};
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        const uint32_t w0 = wd[st], w4 = w0 >> 4;
        u32x4 o;
        o.x = and_or_sv(__builtin_amdgcn_perm(w4, w0, 0x0C040C00u), mask, magic);
        o.y = and_or_sv(__builtin_amdgcn_perm(w4, w0, 0x0C050C01u), mask, magic);
        o.z = and_or_sv(__builtin_amdgcn_perm(w4, w0, 0x0C060C02u), mask, magic);
        o.w = and_or_sv(__builtin_amdgcn_perm(w4, w0, 0x0C070C03u), mask, magic);
        bd[ns][st] = __builtin_bit_cast(bf16x8, o);
      }
    }
    const uint32_t ssel = scale_sel(g);
    float scv[SN];
#pragma unroll
    for (int ns = 0; ns < SN; ++ns) scv[ns] = scale_of(sc_cur[ns], ssel);
    if (rstage >= 0) rs_store(rstage, j, rsd);
#pragma unroll
    for (int ms = 0; ms < MS; ++ms) {
      const int cur = ms & 1;
      if (ms + 1 < MS) read_rows(ms + 1, cq[(ms + 1) & 1], aq[(ms + 1) & 1]);
      __builtin_amdgcn_sched_barrier(0);
      const f32x4 c0 = cq[cur];
      f32x4 t[SN];
#pragma unroll
      for (int ns = 0; ns < SN; ++ns) t[ns] = c0;
#pragma unroll
      for (int st = 0; st < 4; ++st)
#pragma unroll
        for (int ns = 0; ns < SN; ++ns)
          t[ns] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aq[cur][st], bd[ns][st], t[ns], 0, 0, 0);
#pragma unroll
      for (int ns = 0; ns < SN; ++ns) {
        acc[ms][ns].x = fmaf(scv[ns], t[ns].x, acc[ms][ns].x);
        acc[ms][ns].y = fmaf(scv[ns], t[ns].y, acc[ms][ns].y);
        acc[ms][ns].z = fmaf(scv[ns], t[ns].z, acc[ms][ns].z);
        acc[ms][ns].w = fmaf(scv[ns], t[ns].w, acc[ms][ns].w);
      }
    }
      }
  };

  // ---- pipeline: group j + 2 is loaded while group j is computed, and (RSK)
  // the row sums of group j + 1 (landed) are formed during group j's compute
  // (otherwise they arrive with the stage's DMA from the pre-pass). The
  // barrier that ends group j waits for all of this wave's vector-memory
  // operations (vmcnt(0)) and LDS writes: that includes the DMA of group
  // j + 1 and the DMA of group j + 2 issued at the start of group j, which
  // has had a whole group of compute to land, and publishes group j + 1's row
  // sums. A precise count would let group j + 2 stay in flight, but it is only
  // correct while the compiler emits no other vector memory operations
  // (spills count too), so the simple wait is used.
  if (ng > 0) {
    issue(gb, 0);
    if (ng > 1) issue(gb + 1, 1);
    load_scales(sc_cur, gb);
    wait_vm_barrier<0>();
    if constexpr (RSK) {
      f32x4 rsd[RSM][NSG];
      rs_issue(0, 0, rsd);
      rs_store(0, 0, rsd);
      wait_vm_barrier<0>();
    }
  }
  for (int j = 0; j < ng; ++j) {
    const int g = gb + j;
    const bool ahead = j + NSTAGE - 1 < ng;
    if (ahead) issue(g + NSTAGE - 1, (j + NSTAGE - 1) % NSTAGE);
    // GS = 32: every trip loads (the last one reloads its own group's words,
    // unused) and the copy below is unconditional; GS = 128: only trips with
    // a next group. Each form measured 1-2 % faster on its own group size
    // (1322 x {19456, 6144, 2560} x {2560, 2560, 9728} at group 32; 8 x 256 x
    // 2048 x 4096 and 1322 x 6144 x 2560 at group 128).
    if (GS == 32 || j + 1 < ng) load_scales(sc_nxt, j + 1 < ng ? g + 1 : g);
    // RSK: the row sums of group j + 1 (landed) are formed during group j
    const int rstage = RSK && j + 1 < ng ? (j + 1) % NSTAGE : -1;
    if constexpr (GS == 128) compute(j % NSTAGE, g, rstage, j + 1);
    else compute32(j % NSTAGE, rstage, j + 1);
    if (j + 1 < ng) wait_vm_barrier<0>();
    if (GS == 32 || j + 1 < ng) {
#pragma unroll
      for (int ns = 0; ns < SN; ++ns) sc_cur[ns] = sc_nxt[ns];
    }
  }

  // ---- epilogue: lane holds rows 16 ms + 4 kb + i of column TN wv + 16 ns + m16
  const __amdgpu_buffer_rsrc_t ry = make_rsrc(args.y + (size_t)row0 * args.N, (uint32_t)rows * (uint32_t)args.N * 2u);
  const __amdgpu_buffer_rsrc_t rws =
      make_rsrc(args.ws + ((size_t)slice * args.M_total + row0) * args.N, (uint32_t)rows * (uint32_t)args.N * 4u);
  // bf16 output of a full column tile with N % 8 == 0 (16-byte aligned rows
  // of 8 columns): through LDS, so that every lane stores 16 bytes (8
  // columns of one row) with 9x fewer store instructions than 2-byte stores
  // of the 4 rows of one column a lane holds (1322 x 19456 x 2560: 140.5 ->
  // 140.0 us; 8 x 256 x 2048 x 4096 batched: 46.9 -> 46.3 us). The wave's
  // tile goes row-major into its own LDS region (the stages are free once
  // every wave is past its last group), then back out as 16-byte rows.
  if (args.ws == nullptr && ncols == kPN && args.N % 8 == 0) {
    static_assert(kNW * BM * TN * 2 <= NSTAGE * ST::kBytes, "epilogue tile fits the stages' LDS");
    __syncthreads();
    uint8_t* wreg = lds + wv * (BM * TN * 2);
#pragma unroll
    for (int ms = 0; ms < MS; ++ms)
#pragma unroll
      for (int ns = 0; ns < SN; ++ns)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          *reinterpret_cast<uint16_t*>(wreg + (16 * ms + 4 * kb + i) * (TN * 2) + (16 * ns + m16) * 2) =
              to_bf16(acc[ms][ns][i]);
    wave_lds_exchange();   // the rows below were written by other lanes
    // lane: row lane / 4 + 16 t, columns 8 (lane % 4) .. + 7 of the wave's 32;
    // rows past the tile's last are past the buffer extent (dropped)
#pragma unroll
    for (int tt = 0; tt < MS; ++tt) {
      const int r = (lane >> 2) + 16 * tt, c8 = lane & 3;
      const u32x4 v = *reinterpret_cast<const u32x4*>(wreg + r * (TN * 2) + c8 * 16);
      st128(v, ry, ((uint32_t)r * (uint32_t)args.N + (uint32_t)(n0 + TN * wv + 8 * c8)) * 2u);
    }
  } else if (args.ws == nullptr) {
#pragma unroll
    for (int ns = 0; ns < SN; ++ns) {
      const int ncol = TN * wv + 16 * ns + m16;
      if (ncol < ncols) {
#pragma unroll
        for (int ms = 0; ms < MS; ++ms)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const uint32_t e = (uint32_t)(16 * ms + 4 * kb + i) * (uint32_t)args.N + (uint32_t)(n0 + ncol);
            st16(to_bf16(acc[ms][ns][i]), ry, e * 2u);
          }
      }
    }
  } else {
#pragma unroll
    for (int ns = 0; ns < SN; ++ns) {
      const int ncol = TN * wv + 16 * ns + m16;
      if (ncol < ncols) {
#pragma unroll
        for (int ms = 0; ms < MS; ++ms)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const uint32_t e = (uint32_t)(16 * ms + 4 * kb + i) * (uint32_t)args.N + (uint32_t)(n0 + ncol);
            st32(__float_as_uint(acc[ms][ns][i]), rws, e * 4u);
          }
      }
    }
  }
}

// ---------------------------------------------------------------- row-sum pre-pass
// out[g * ld + m] = -136 * sum_{k in group g} x[m, k], fp32, for groups of GS
// = 128 or 32 k: the initial accumulators of the tile kernel's group chains
// when they come from a separate pass (the tile kernel forms them itself
// otherwise). One wave per row; a wave instruction covers 512 consecutive k
// and up to 8 of them are in flight before any is reduced; a group's lanes
// (16 for 128 k, 4 for 32 k) are summed with DPP. Loads past the row read
// zeros (exact buffer extent).
template <int GS>
__global__ __launch_bounds__(256) void rowsum_neg136_kernel(const uint16_t* __restrict__ x,
                                                           float* __restrict__ out, int M, int K, int ld) {
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

hipError_t launch_rowsum_neg136(const uint16_t* x, float* out, int M, int K, int ld, int gsize, hipStream_t stream) {
  if (M <= 0) return hipSuccess;
  if (gsize == 128)
    hipLaunchKernelGGL(rowsum_neg136_kernel<128>, dim3((M + 3) / 4), dim3(256), 0, stream, x, out, M, K, ld);
  else if (gsize == 32)
    hipLaunchKernelGGL(rowsum_neg136_kernel<32>, dim3((M + 3) / 4), dim3(256), 0, stream, x, out, M, K, ld);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

template <int NSTAGE, int MS, int GS, bool RSK>
static hipError_t launch_prefill_rsk(PrefillArgs a, int sk, hipStream_t stream) {
  constexpr int BM = Stage<MS, GS>::kRows;
  const int lds_bytes = NSTAGE * Stage<MS, GS>::kBytes;
  static std::atomic<uint64_t> lds_set{0};   // per instantiation and device
  const hipError_t ea =
      ensure_dyn_lds(reinterpret_cast<const void*>(&prefill_kernel<NSTAGE, MS, GS, RSK>), lds_bytes, lds_set);
  if (ea != hipSuccess) return ea;
  a.mtiles = a.m_uniform > 0 ? a.G * ((a.m_uniform + BM - 1) / BM)
                             : (a.M_total + BM - 1) / BM + (a.m_sizes != nullptr ? a.G : 0);
  a.ntiles = (a.N + kPN - 1) / kPN;
  const long long blocks = (long long)a.mtiles * a.ntiles;
  if (blocks <= 0) return hipSuccess;
  if (blocks > 0x7FFFFFFFLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL((prefill_kernel<NSTAGE, MS, GS, RSK>), dim3((unsigned)blocks, sk), dim3(64 * kNW), lds_bytes,
                     stream, a);
  return hipGetLastError();
}

// row sums formed in the kernel (sxn == nullptr) or taken from the pre-pass
template <int NSTAGE, int MS, int GS = 128>
static hipError_t launch_prefill_t(PrefillArgs a, int sk, hipStream_t stream) {
  if (a.sxn == nullptr) return launch_prefill_rsk<NSTAGE, MS, GS, true>(a, sk, stream);
  return launch_prefill_rsk<NSTAGE, MS, GS, false>(a, sk, stream);
}

// Tile heights: 16 MS rows, MS = 3 .. 9 (48 .. 144 rows) at group 128; at
// group 32 the four row-sum sets per stage leave room for MS = 5 .. 8 only
// (a 144-row tile would not fit three stages in LDS).
bool tile_rows_ok(int bm, int gsize) {
  if (bm % 16 != 0) return false;
  const int ms = bm / 16;
  if (gsize == 128) return ms >= 3 && ms <= 9;
  if (gsize == 32) return ms >= 5 && ms <= 8;
  return false;
}

hipError_t launch_tile(const uint16_t* x, const uint8_t* w, const uint16_t* s, const float* sxn, int ld, uint16_t* y,
                       float* ws, const int32_t* m_sizes, int m_uniform, int M_total, int N, int K, int G, int gps,
                       int sk, int bm, int gsize, hipStream_t stream) {
  if (!tile_rows_ok(bm, gsize)) return hipErrorInvalidValue;
  PrefillArgs a;
  a.x = x; a.w = w; a.s = s; a.sxn = sxn; a.y = y; a.ws = ws; a.m_sizes = m_sizes; a.m_uniform = m_uniform;
  a.M_total = M_total; a.N = N; a.K = K; a.G = G; a.ld = ld; a.gps = gps;
  a.mtiles = 0; a.ntiles = 0;
  if (gsize == 32) {
    switch (bm / 16) {
      case 8: return launch_prefill_t<3, 8, 32>(a, sk, stream);   // 3 x 50.5 KiB stages
      case 7: return launch_prefill_t<3, 7, 32>(a, sk, stream);
      case 6: return launch_prefill_t<3, 6, 32>(a, sk, stream);
      case 5: return launch_prefill_t<3, 5, 32>(a, sk, stream);
      default: return hipErrorInvalidValue;
    }
  }
  switch (bm / 16) {
    case 9: return launch_prefill_t<3, 9>(a, sk, stream);     // 144 x 256 tiles, 3 x 52.6 KiB stages
    case 8: return launch_prefill_t<3, 8>(a, sk, stream);     // 128 x 256 tiles, 3 x 48.5 KiB stages
    case 7: return launch_prefill_t<3, 7>(a, sk, stream);     // 112 x 256 tiles, 3 x 44.4 KiB stages
    case 6: return launch_prefill_t<3, 6>(a, sk, stream);     // 96 x 256 tiles, 3 x 40.4 KiB stages
    case 5: return launch_prefill_t<3, 5>(a, sk, stream);     // 80 x 256 tiles, 3 x 36.3 KiB stages
    case 4: return launch_prefill_t<3, 4>(a, sk, stream);     // 64 x 256 tiles, 3 x 32.3 KiB stages
    case 3: return launch_prefill_t<3, 3>(a, sk, stream);     // 48 x 256 tiles, 3 x 28.2 KiB stages
    default: return hipErrorInvalidValue;
  }
}

}  // namespace w4a16
