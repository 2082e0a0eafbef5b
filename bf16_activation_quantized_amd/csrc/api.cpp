// C-ABI entry points: argument validation on the host (before anything is
// enqueued), path and split-K selection, workspace layout and launches.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <mutex>

#include <stddef.h>
#include <stdint.h>

#include "../../include/w4a16.h"
#include "launch.hpp"
#include "w4a16_internal.h"

namespace {

constexpr int64_t kGroup = 128;       // k per pipeline stage (and the default scale group)
constexpr int32_t kGroupSmall = 32;   // the other scale group size (tile path only)
constexpr int64_t kMaxDim = 0x7FFFFFFFLL;
constexpr uint64_t kMaxBytes = 0xFFFFFFFFULL;   // one buffer resource extent

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
uint64_t round_up(uint64_t v, uint64_t a) { return (v + a - 1) / a * a; }

bool valid_split(int32_t sk) { return sk == 0 || sk == 1 || sk == 2 || sk == 4 || sk == 8 || sk == 16; }

// Which kernel family runs a plain GEMM at this shape.
enum Path { kPathAuto = 0, kPathGemv = 1, kPathSkinny = 2, kPathTile = 3 };

int32_t pow2_at_least(int64_t v) {
  int32_t p = 1;
  while (p < v && p < 16) p <<= 1;
  return p;
}

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Compute units of the current device (cached per device; safe to call from
// several host threads).
int device_cus() {
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

// Small batch: the register-streaming kernel with one column tile of 16 per
// wave up to 8 rows and past 32, two between (8 waves per workgroup; at
// 17408 x 5120 and 8192 x 8192: M = 2-4 7-10 % faster with one tile, M >= 9
// 4-12 % faster with two; past 32 rows the three row tiles leave registers
// for one only). At 9-16 rows the LDS-staged kernel (variant 6: stages of 4
// groups, 4 in flight) instead: over N x K = 8192 x 8192, 17408 x 5120,
// 7168 x 8192, 4096 x 4096, 2560 x 9728, 2048 x 5120 and 896 x 5120 it ran
// 2-18 % faster at M = 16; at M = 8 it lost at four of the seven, at M <= 4
// at five, by up to 33 % (its X stage is read in full whatever M is).
int skinny_default_tiles(int64_t M) {
  if (M > 8 && M <= 16) return 6;
  return M <= 8 || M > 32 ? 1 : 2;
}
constexpr int kSkinnyWaves = 8;

Path auto_path(int64_t M, int64_t N, int64_t K, int32_t sk) {
  const int64_t Gk = K / kGroup;
  if (M == 1) {
    // the GEMV keeps a lane's x in registers: at most 64 groups per slice
    const int64_t s = sk > 0 ? sk : 16;
    return ceil_div(Gk, s) <= 64 ? kPathGemv : kPathSkinny;
  }
  if (M <= 16) return kPathSkinny;
  // two row tiles of 16 (one 8-wave workgroup per compute unit per round):
  // at 17 <= M <= 32 the small-batch kernel ran 6-33 % faster than the tile
  // kernel at 17408 x 5120, 8192 x 8192 and 2560 x 9728 (at most 2.1 rounds
  // of workgroups), 4-12 % slower at 28672 x 8192 (3.5 rounds)
  if (M <= 32 && ceil_div(N, 32) <= 3 * (int64_t)device_cus()) return kPathSkinny;
  // three row tiles (8 waves of one column tile): only while one round of
  // workgroups covers N (4096 x 4096 and 2560 x 9728 at 33-48 rows: 8-35 %
  // faster than the tile kernel; 8192 x 8192, two rounds: 15-30 % slower)
  if (M <= w4a16::kSkinnyMaxRows && ceil_div(N, 16) <= (int64_t)device_cus()) return kPathSkinny;
  return kPathTile;
}

// Cost model of the tile path, in units of one row x one 128-group of work on
// one compute unit at the 128-row tile's rate (≈0.0162 us on MI355X: the
// 144-row tile runs 20 groups in 48.7 us). One workgroup per compute unit:
// a launch takes ceil(tiles x SK / CUs) rounds of (rows / rate) x groups per
// slice. A split adds its fp32 partials, written by the tile kernel and read
// by the reduce (8 x SK x M x N bytes at ≈4 TB/s), the reduce launch (≈1 us)
// and ≈1.5 us per 8 slices (the reduce has the loads of up to 8 slices in
// flight before it adds them, so every 8 slices are one more round trip).
// Splits only where tiles x SK fit one round (a second, mostly idle round of
// slices never pays: at M = 96..384, N x K = 17408 x 5120 doubling past it
// cost 24-52 %). The three split costs and the rates of the 48- to 80-row
// tiles below were fitted to every explicit choice timed at 42 shapes (M
// 64..4096; N x K 896..17408 x 2560..8192): the automatic choice is within
// 1 % of the fastest at 41 of them and 5.6 % at the last (with the partials
// at 5 TB/s, a 2 us launch and no per-8-slices term: 1.7 % on average, 10 %
// at worst, by choosing SK 16 where 8 was faster), and the deep prefill,
// grouped and batched workloads keep their choices.
constexpr double kUnitUs = 0.0162, kReduceBytesPerUs = 4.0e6, kReduceLaunchUs = 1.0, kReduceBatchUs = 1.5;

double tile_cost(int64_t M, int64_t N, int64_t Gk, int64_t tiles, int bm, double rate, int64_t sk, int64_t cus) {
  double c = (double)ceil_div(tiles * sk, cus) * bm / rate * (double)ceil_div(Gk, sk);
  if (sk > 1)
    c += (8.0 * (double)sk * (double)M * (double)N / kReduceBytesPerUs + kReduceLaunchUs +
          (double)ceil_div(sk, 8) * kReduceBatchUs) /
         kUnitUs;
  return c;
}

// The split of least cost for `tiles` tiles of bm rows (rate: per-row rate of
// the height): 1, or a power of two up to 16 (and the group count) whose
// slices fit one round.
int32_t tile_split_rate(int64_t M, int64_t N, int64_t Gk, int64_t tiles, int bm, double rate) {
  const int64_t cus = device_cus();
  int32_t best = 1;
  double best_cost = tile_cost(M, N, Gk, tiles, bm, rate, 1, cus);
  for (int32_t sk = 2; sk <= 16 && sk <= Gk && tiles * sk <= cus; sk <<= 1) {
    const double c = tile_cost(M, N, Gk, tiles, bm, rate, sk, cus);
    if (c < best_cost * (1.0 - 1e-9)) {
      best = sk;
      best_cost = c;
    }
  }
  return best;
}

// Per-row rates of the tile heights, relative to the 128-row tile (shorter
// tiles amortise the per-group dequantisation and barrier over fewer rows;
// at 1322 x 19456 x 2560 on one box: 4 rounds of 128 rows 166 us, 4 of 112
// rows 161 us, 3 of 144 rows 146 us, 5 of 96 rows 176 us; the 80-, 64- and
// 48-row rates fitted with the split costs above).
struct TileCand { int bm; double rate; };
constexpr TileCand kTileCands[] = {{128, 1.0}, {144, 0.96}, {112, 0.91}, {96, 0.907},
                                   {80, 0.80}, {64, 0.66},  {48, 0.58}};

double tile_rate(int bm) {
  for (const TileCand& c : kTileCands)
    if (c.bm == bm) return c.rate;
  return 0.9;
}

int32_t tile_split(int64_t M, int64_t N, int64_t Gk, int64_t tiles, int bm) {
  return tile_split_rate(M, N, Gk, tiles, bm, tile_rate(bm));
}

// Tile height of the least estimated cost, with its own best split when
// split_k is automatic (`split` < 0) or the given one. `tiles(bm)` counts the
// output tiles of a height. Only heights built for the scale group size gs
// are candidates.
template <class T>
int pick_tile_rows(int64_t M, int64_t N, int64_t Gk, T tiles, int64_t split, int32_t gs) {
  const int64_t cus = device_cus();
  int best = 128;
  double best_cost = 0.0;
  for (const TileCand& c : kTileCands) {
    if (!w4a16::tile_rows_ok(c.bm, gs)) continue;
    const int64_t t = tiles(c.bm);
    const int64_t sk = split > 0 ? split : tile_split_rate(M, N, Gk, t, c.bm, c.rate);
    const double cost = tile_cost(M, N, Gk, t, c.bm, c.rate, sk, cus);
    if (best_cost == 0.0 || cost < best_cost * (1.0 - 1e-9)) {
      best = c.bm;
      best_cost = cost;
    }
  }
  return best;
}

int64_t tile_cols(int64_t N) { return ceil_div(N, w4a16::kTileCols); }

// split_k = 0: automatic, chosen with the height; otherwise fixed
int default_tile_rows(int64_t M, int64_t N, int64_t K, int32_t split_k, int32_t gs) {
  const int64_t nt = tile_cols(N), Gk = K / kGroup;
  return pick_tile_rows(
      M, N, Gk, [&](int bm) { return ceil_div(std::max<int64_t>(M, 1), bm) * nt; }, split_k > 0 ? split_k : -1,
      gs);
}

// grouped (no split-K): M_sizes stays on the device, so the tile count is
// estimated as ceil(M_total / bm) + G / 2 per column (each group's partial
// last tile adds half a tile on average; the kernel maps only the real tiles)
int default_grouped_tile_rows(int64_t G, int64_t M_total, int64_t N, int64_t K, int32_t gs) {
  const int64_t nt = tile_cols(N);
  return pick_tile_rows(
      M_total, N, K / kGroup,
      [&](int bm) { return (ceil_div(std::max<int64_t>(M_total, 1), bm) + G / 2) * nt; }, 1, gs);
}

int32_t auto_split(Path path, int64_t M, int64_t N, int64_t K, int bm, int nt) {
  const int64_t Gk = K / kGroup;
  int32_t sk = 1;
  switch (path) {
    case kPathGemv:
      // only what the register budget for x needs (at most 64 groups per
      // slice): a split adds the reduce kernel, and over N x K from 1024 x
      // 8192 to 28672 x 8192 one slice was fastest wherever it fits
      sk = pow2_at_least(ceil_div(Gk, 64));
      break;
    case kPathSkinny: {
      // split only when fewer than half of the compute units have a
      // workgroup, and then as far as one round of workgroups goes: the
      // reduce kernel and the partials cost more than the shorter slices save
      // once the grid is half full (4096 x 4096, 128 workgroups: SK 1 8-16 %
      // faster than 2), while a grid a quarter full or less gains from
      // filling the GPU (M = 16 at 2048 x 5120, 64 workgroups: SK 4 9.3 us,
      // SK 2 10.3; at 896 x 5120, 28 workgroups: SK 8 8.7, SK 4 9.1;
      // 2560 x 9728, 80 workgroups: SK 2 20 % faster than 4)
      const int64_t wgs = ceil_div(N, 16 * (int64_t)nt), cus = device_cus();
      if (2 * wgs < cus)
        while (sk < 16 && 2 * sk <= Gk && wgs * sk * 2 <= cus) sk <<= 1;
      break;
    }
    case kPathTile:
      sk = tile_split(M, N, Gk, ceil_div(M, bm) * tile_cols(N), bm);
      break;
    default:
      break;
  }
  return sk;
}

// Row sums of X on the tile path: the tile kernel forms -136 * sum_k x per
// (row, scale group) itself, on the matrix core, in every column tile; a
// separate pre-pass forms them once, into the workspace. The kernel's own
// sums cost more once many column tiles repeat them (1322 x 19456 x 2560,
// 76 column tiles: 157 against 150.5 us with the pre-pass; N = 2048 and
// 4096 at 1322 rows, 8 and 16 tiles: 1-3 us faster than the pre-pass; at
// group 32 the in-kernel sums take four MFMAs per stage instead of one chain
// and the crossover is lower), so the pre-pass is used from 32 column tiles
// at group 128 and 8 at group 32, when the caller gives the workspace room.
bool tile_prepass(int64_t N, int32_t gs) { return tile_cols(N) * (kGroup / gs) >= 32; }

// bytes of the [K / gs, ld] fp32 row sums of the pre-pass
uint64_t rowsum_bytes(int64_t M, int64_t K, int32_t gs) {
  return (uint64_t)(K / gs) * round_up((uint64_t)M, 4) * 4u;
}

struct Plan {
  Path path;
  int32_t sk;         // effective split-K
  int32_t gps;        // 128-groups per slice
  int variant;        // GEMV: 1 = half-wave layout; small batch: column tiles per wave; tile: rows per tile
  uint64_t ws_split;  // bytes of the [SK, M, N] fp32 partials
  uint64_t ws_sx;     // bytes of the pre-pass row sums (tile path with a wide N), else 0
};

// Group size 32 runs on the tile path only (the GEMV and small-batch kernels
// take one scale per 128 k), whatever M is.
w4a16_status make_plan(int64_t M, int64_t N, int64_t K, int32_t split_k, const w4a16_config* cfg, int32_t gs,
                       Plan* p) {
  const int64_t Gk = K / kGroup;
  Path path = gs == kGroup ? auto_path(M, N, K, split_k) : kPathTile;
  int variant = -1;
  if (cfg != nullptr) {
    if (cfg->path < 0 || cfg->path > 3) return W4A16_ERR_SHAPE;
    if (cfg->path != 0) path = (Path)cfg->path;
    variant = cfg->variant;
  }
  if (path == kPathGemv && M != 1) return W4A16_ERR_SHAPE;
  if (path == kPathSkinny && M > w4a16::kSkinnyMaxRows) return W4A16_ERR_SHAPE;
  if (path != kPathTile && gs != kGroup) return W4A16_ERR_GROUP_SIZE;
  switch (path) {
    case kPathGemv:
      if (variant > 1) return W4A16_ERR_SHAPE;
      if (variant < 0) variant = 0;   // the MFMA layout where it applies
      break;
    case kPathSkinny:
      if (variant <= 0) variant = skinny_default_tiles(M);
      // past 32 rows (three row tiles) one column tile per wave only; variants
      // 3..6: the LDS-staged kernel (M <= 16), stage geometries 0..3
      if (variant > 6 || (M > 32 && variant != 1) || (variant >= 3 && M > 16)) return W4A16_ERR_SHAPE;
      break;
    case kPathTile:
      if (variant <= 0) variant = default_tile_rows(M, N, K, split_k, gs);
      if (!w4a16::tile_rows_ok(variant, kGroup) && !w4a16::tile_rows_ok(variant, kGroupSmall))
        return W4A16_ERR_SHAPE;
      if (!w4a16::tile_rows_ok(variant, gs)) return W4A16_ERR_GROUP_SIZE;
      break;
    default:
      return W4A16_ERR_SHAPE;
  }
  int32_t sk = split_k > 0 ? split_k : auto_split(path, M, N, K, variant, variant >= 3 ? 2 : variant);
  if (sk > Gk && split_k == 0) sk = 1;
  if (path == kPathGemv && ceil_div(Gk, sk) > 64) {
    if (split_k != 0) return W4A16_ERR_SPLIT_K;   // explicit split too small for the GEMV path
    sk = pow2_at_least(ceil_div(Gk, 64));
  }
  p->path = path;
  p->sk = sk;
  p->gps = (int32_t)ceil_div(Gk, sk);
  p->variant = variant;
  p->ws_split = sk > 1 ? (uint64_t)sk * (uint64_t)M * (uint64_t)N * 4u : 0u;
  p->ws_sx = path == kPathTile && tile_prepass(N, gs) ? rowsum_bytes(M, K, gs) : 0u;
  return W4A16_OK;
}

uint64_t plan_bytes(const Plan& p) { return round_up(p.ws_split, 256) + p.ws_sx; }

w4a16_status check_dims(int64_t M, int64_t N, int64_t K, int32_t group_size) {
  if (M < 0 || N < 1 || K < 1 || M > kMaxDim || N > kMaxDim || K > kMaxDim) return W4A16_ERR_SHAPE;
  if ((group_size != kGroup && group_size != kGroupSmall) || K % kGroup != 0) return W4A16_ERR_GROUP_SIZE;
  // buffer extents of one resource
  if ((uint64_t)N * (uint64_t)K / 2u > kMaxBytes) return W4A16_ERR_SHAPE;
  if ((uint64_t)M * (uint64_t)K * 2u > kMaxBytes) return W4A16_ERR_SHAPE;
  if ((uint64_t)M * (uint64_t)N * 4u > kMaxBytes) return W4A16_ERR_SHAPE;
  return W4A16_OK;
}

w4a16_status check_batched(int32_t B, int64_t M, int64_t N, int64_t K, int32_t group_size) {
  if (B < 1 || M < 0) return W4A16_ERR_SHAPE;
  if ((uint64_t)B * (uint64_t)M > (uint64_t)kMaxDim) return W4A16_ERR_SHAPE;
  w4a16_status st = check_dims((int64_t)B * M, N, K, group_size);
  if (st != W4A16_OK) return st;
  // one buffer resource covers the scales of all problems
  if ((uint64_t)B * (uint64_t)N * (uint64_t)(K / group_size) * 2u > kMaxBytes) return W4A16_ERR_SHAPE;
  return W4A16_OK;
}

w4a16_status launched(hipError_t e) { return e == hipSuccess ? W4A16_OK : W4A16_ERR_LAUNCH; }

// Validated plan of a plain GEMM: status, or W4A16_OK with *p filled and
// *empty set when M == 0 (nothing to enqueue).
w4a16_status plan_gemm(const uint16_t* x, const uint8_t* w, const uint16_t* s, uint16_t* y, int64_t M, int64_t N,
                       int64_t K, int32_t group_size, int32_t split_k, const w4a16_config* cfg, Plan* p,
                       bool* empty) {
  *empty = false;
  if (!valid_split(split_k)) return W4A16_ERR_SPLIT_K;
  w4a16_status st = check_dims(M, N, K, group_size);
  if (st != W4A16_OK) return st;
  if (M == 0) {   // empty problem: nothing to read or write
    *empty = true;
    return W4A16_OK;
  }
  if (x == nullptr || w == nullptr || s == nullptr || y == nullptr) return W4A16_ERR_NULL;
  if (!aligned16(x) || !aligned16(w) || !aligned16(s) || !aligned16(y)) return W4A16_ERR_ALIGN;
  st = make_plan(M, N, K, split_k, cfg, group_size, p);
  if (st != W4A16_OK) return st;
  if (p->ws_split > kMaxBytes) return W4A16_ERR_SHAPE;
  return W4A16_OK;
}

// Enqueues a planned GEMM; `partials` holds the [SK, M, N] fp32 slices when
// p.sk > 1 (unused otherwise); `rowsums` (tile path, may be nullptr) the
// pre-pass row sums.
w4a16_status launch_plan(const Plan& p, const uint16_t* x, const uint8_t* w, const uint16_t* s, uint16_t* y,
                         int64_t M, int64_t N, int64_t K, int32_t group_size, float* partials, float* rowsums,
                         hipStream_t strm) {
  float* ws_split = p.sk > 1 ? partials : nullptr;
  const int iM = (int)M, iN = (int)N, iK = (int)K;
  hipError_t e = hipSuccess;
  switch (p.path) {
    case kPathGemv:
      e = w4a16::launch_gemv_m1(x, w, s, y, ws_split, iN, iK, p.gps, p.sk, p.variant == 1, strm);
      break;
    case kPathSkinny:
      if (p.variant >= 3 && w4a16::skinny_lds_fits(iM, p.gps))
        e = w4a16::launch_skinny_lds(x, w, s, y, ws_split, iM, iN, iK, p.gps, p.sk, p.variant - 3, strm);
      else
        e = w4a16::launch_skinny(x, w, s, y, ws_split, iM, iN, iK, p.gps, p.sk, p.variant >= 3 ? 1 : p.variant,
                                 kSkinnyWaves, strm);
      break;
    case kPathTile: {
      const int ld = (int)round_up((uint64_t)M, 4);
      if (rowsums != nullptr) e = w4a16::launch_rowsum_neg136(x, rowsums, iM, iK, ld, group_size, strm);
      if (e == hipSuccess)
        e = w4a16::launch_tile(x, w, s, rowsums, ld, y, ws_split, nullptr, 0, iM, iN, iK, 1, p.gps, p.sk, p.variant,
                               group_size, strm);
      break;
    }
    default:
      return W4A16_ERR_SHAPE;
  }
  if (e != hipSuccess) return W4A16_ERR_LAUNCH;
  if (p.sk > 1) return launched(w4a16::launch_splitk_reduce(ws_split, y, (uint64_t)M * (uint64_t)N, p.sk, strm));
  return W4A16_OK;
}

w4a16_status run_gemm(const uint16_t* x, const uint8_t* w, const uint16_t* s, uint16_t* y, int64_t M, int64_t N,
                      int64_t K, int32_t group_size, int32_t split_k, float* workspace, size_t workspace_bytes,
                      void* stream, const w4a16_config* cfg) {
  Plan p;
  bool empty = false;
  w4a16_status st = plan_gemm(x, w, s, y, M, N, K, group_size, split_k, cfg, &p, &empty);
  if (st != W4A16_OK || empty) return st;
  if (p.ws_split > 0) {
    if (workspace == nullptr) return W4A16_ERR_WORKSPACE;
    if (!aligned16(workspace)) return W4A16_ERR_ALIGN;
    if (workspace_bytes < round_up(p.ws_split, 256)) return W4A16_ERR_WORKSPACE;
  }
  // the pre-pass row sums only where the workspace has room for them too
  float* rowsums = nullptr;
  if (p.ws_sx > 0 && workspace != nullptr && aligned16(workspace) && workspace_bytes >= plan_bytes(p))
    rowsums = reinterpret_cast<float*>(reinterpret_cast<uint8_t*>(workspace) + round_up(p.ws_split, 256));
  return launch_plan(p, x, w, s, y, M, N, K, group_size, workspace, rowsums, reinterpret_cast<hipStream_t>(stream));
}

size_t gemm_workspace_bytes(int64_t M, int64_t N, int64_t K, int32_t group_size, int32_t split_k,
                            const w4a16_config* cfg) {
  if (!valid_split(split_k) || check_dims(M, N, K, group_size) != W4A16_OK || M == 0) return 0;
  Plan p;
  if (make_plan(M, N, K, split_k, cfg, group_size, &p) != W4A16_OK) return 0;
  return (size_t)plan_bytes(p);
}

// Batched: B problems of M rows on the tile kernel (weight group b = problem
// b, its M rows at b * M), tile height and split-K as for one problem of B x
// ceil(M / h) row tiles per column. (M <= 16 problems run the tile kernel too:
// the per-problem scale tensors are not 16-byte aligned in general, which the
// decode kernels require.)
struct BatchedPlan {
  int bm;
  int32_t sk, gps;
  uint64_t ws_split, ws_sx;
};

w4a16_status make_batched_plan(int32_t B, int64_t M, int64_t N, int64_t K, int32_t split_k, const w4a16_config* cfg,
                               int32_t gs, BatchedPlan* p) {
  const int64_t Gk = K / kGroup, nt = tile_cols(N), Mt = (int64_t)B * M;
  int bm = -1;
  if (cfg != nullptr) {
    if (cfg->path != 0 && cfg->path != kPathTile) return W4A16_ERR_SHAPE;
    bm = cfg->variant;
  }
  if (bm <= 0)
    bm = pick_tile_rows(
        Mt, N, Gk, [&](int h) { return (int64_t)B * ceil_div(M, h) * nt; }, split_k > 0 ? split_k : -1, gs);
  if (!w4a16::tile_rows_ok(bm, kGroup) && !w4a16::tile_rows_ok(bm, kGroupSmall)) return W4A16_ERR_SHAPE;
  if (!w4a16::tile_rows_ok(bm, gs)) return W4A16_ERR_GROUP_SIZE;
  const int64_t tiles = (int64_t)B * ceil_div(M, bm) * nt;
  int32_t sk = split_k > 0 ? split_k : tile_split(Mt, N, Gk, tiles, bm);
  if (sk > Gk && split_k == 0) sk = 1;
  p->bm = bm;
  p->sk = sk;
  p->gps = (int32_t)ceil_div(Gk, sk);
  p->ws_split = sk > 1 ? (uint64_t)sk * (uint64_t)Mt * (uint64_t)N * 4u : 0u;
  p->ws_sx = tile_prepass(N, gs) ? rowsum_bytes(Mt, K, gs) : 0u;
  return W4A16_OK;
}

size_t batched_workspace_bytes(int32_t B, int64_t M, int64_t N, int64_t K, int32_t group_size, int32_t split_k,
                               const w4a16_config* cfg) {
  if (!valid_split(split_k) || check_batched(B, M, N, K, group_size) != W4A16_OK || M == 0) return 0;
  BatchedPlan p;
  if (make_batched_plan(B, M, N, K, split_k, cfg, group_size, &p) != W4A16_OK) return 0;
  return (size_t)(round_up(p.ws_split, 256) + p.ws_sx);
}

// ---------------------------------------------------------------- scratch of the no-allocation entry point
// Device scratch for w4a16_gemm_noalloc: the split-K partials and the
// pre-pass row sums live here instead of in a caller's workspace. Each GPU
// holds its own copy (allocated with the library's code object) until the
// process ends. In host code `scratch` names a host-side stand-in, so its
// device address comes from hipGetSymbolAddress, once per device.
constexpr size_t kScratchBytes = (size_t)W4A16_NOALLOC_SCRATCH_BYTES;
__device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The device address of this GPU's scratch (nullptr on failure): looked up
// with the device current, on the first call per device, and kept.
void* scratch_ptr() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    g_scratch_ptr[dev] = p;
  }
  return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

const char* w4a16_status_string(int status) {
  switch (status) {
    case W4A16_OK: return "W4A16_OK";
    case W4A16_ERR_NULL: return "W4A16_ERR_NULL: a required pointer is NULL";
    case W4A16_ERR_SHAPE: return "W4A16_ERR_SHAPE: invalid dimension or size limit exceeded";
    case W4A16_ERR_GROUP_SIZE:
      return "W4A16_ERR_GROUP_SIZE: group_size must be 128 or 32 (32: tile path only) and K a multiple of 128";
    case W4A16_ERR_SPLIT_K: return "W4A16_ERR_SPLIT_K: split_k must be 0, 1, 2, 4, 8 or 16";
    case W4A16_ERR_WORKSPACE: return "W4A16_ERR_WORKSPACE: workspace missing or too small";
    case W4A16_ERR_ALIGN: return "W4A16_ERR_ALIGN: pointers must be 16-byte aligned";
    case W4A16_ERR_LAUNCH: return "W4A16_ERR_LAUNCH: kernel launch failed";
    default: return "W4A16: unknown status";
  }
}

w4a16_status w4a16_pack_int4(const uint8_t* q, uint8_t* w_packed, int64_t rows, int64_t K, void* stream) {
  if (rows < 0 || K < 2 || K % 2 != 0) return W4A16_ERR_SHAPE;
  if (q == nullptr || w_packed == nullptr) return W4A16_ERR_NULL;
  if (!aligned16(q) || !aligned16(w_packed)) return W4A16_ERR_ALIGN;
  if (rows == 0) return W4A16_OK;
  if ((uint64_t)rows > (uint64_t)INT64_MAX / (uint64_t)K) return W4A16_ERR_SHAPE;
  return launched(
      w4a16::launch_pack_int4(q, w_packed, (uint64_t)rows * (uint64_t)K, reinterpret_cast<hipStream_t>(stream)));
}

int32_t w4a16_gemm_auto_split_k(int64_t M, int64_t N, int64_t K, int32_t group_size) {
  if (check_dims(M, N, K, group_size) != W4A16_OK || M == 0) return 0;
  Plan p;
  if (make_plan(M, N, K, 0, nullptr, group_size, &p) != W4A16_OK) return 0;
  return p.sk;
}

w4a16_status w4a16_gemm_auto_config(int64_t M, int64_t N, int64_t K, int32_t group_size, w4a16_config* cfg_out,
                                    int32_t* split_k_out) {
  if (cfg_out == nullptr || split_k_out == nullptr) return W4A16_ERR_NULL;
  cfg_out->path = 0;
  cfg_out->variant = -1;
  *split_k_out = 0;
  const w4a16_status st = check_dims(M, N, K, group_size);
  if (st != W4A16_OK || M == 0) return st;
  Plan p;
  const w4a16_status sp = make_plan(M, N, K, 0, nullptr, group_size, &p);
  if (sp != W4A16_OK) return sp;
  cfg_out->path = (int32_t)p.path;
  cfg_out->variant = p.variant;
  *split_k_out = p.sk;
  return W4A16_OK;
}

size_t w4a16_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K, int32_t split_k) {
  return gemm_workspace_bytes(M, N, K, kGroup, split_k, nullptr);
}

size_t w4a16_gemm_workspace_bytes_gs(int64_t M, int64_t N, int64_t K, int32_t group_size, int32_t split_k) {
  return gemm_workspace_bytes(M, N, K, group_size, split_k, nullptr);
}

size_t w4a16_gemm_workspace_bytes_ex(int64_t M, int64_t N, int64_t K, int32_t group_size, int32_t split_k,
                                     const w4a16_config* cfg) {
  return gemm_workspace_bytes(M, N, K, group_size, split_k, cfg);
}

w4a16_status w4a16_gemm(const uint16_t* x, const uint8_t* w_packed, const uint16_t* scales, uint16_t* y, int64_t M,
                        int64_t N, int64_t K, int32_t group_size, int32_t split_k, float* workspace,
                        size_t workspace_bytes, void* stream) {
  return run_gemm(x, w_packed, scales, y, M, N, K, group_size, split_k, workspace, workspace_bytes, stream, nullptr);
}

w4a16_status w4a16_gemm_noalloc(const uint16_t* x, const uint8_t* w_packed, const uint16_t* scales, uint16_t* y,
                                int64_t M, int64_t N, int64_t K, int32_t group_size, int32_t split_k, void* stream) {
  Plan p;
  bool empty = false;
  w4a16_status st = plan_gemm(x, w_packed, scales, y, M, N, K, group_size, split_k, nullptr, &p, &empty);
  if (st != W4A16_OK || empty) return st;
  // the partials must fit the scratch; the row sums only where they fit too
  // (otherwise the tile kernel forms them), as with a caller's workspace
  if (round_up(p.ws_split, 256) > kScratchBytes) return W4A16_ERR_WORKSPACE;
  float* ws = nullptr;
  if (p.ws_split > 0 || p.ws_sx > 0) {
    ws = reinterpret_cast<float*>(scratch_ptr());
    if (ws == nullptr) return W4A16_ERR_LAUNCH;
  }
  float* rowsums = nullptr;
  if (p.ws_sx > 0 && plan_bytes(p) <= kScratchBytes)
    rowsums = reinterpret_cast<float*>(reinterpret_cast<uint8_t*>(ws) + round_up(p.ws_split, 256));
  return launch_plan(p, x, w_packed, scales, y, M, N, K, group_size, ws, rowsums,
                     reinterpret_cast<hipStream_t>(stream));
}

w4a16_status w4a16_gemm_ex(const uint16_t* x, const uint8_t* w_packed, const uint16_t* scales, uint16_t* y,
                           int64_t M, int64_t N, int64_t K, int32_t group_size, int32_t split_k, float* workspace,
                           size_t workspace_bytes, void* stream, const w4a16_config* cfg) {
  return run_gemm(x, w_packed, scales, y, M, N, K, group_size, split_k, workspace, workspace_bytes, stream, cfg);
}

w4a16_status w4a16_gemm_grouped(const uint16_t* x, const uint8_t* w_packed, const uint16_t* scales,
                                const int32_t* m_sizes, uint16_t* y, int32_t G, int64_t M_total, int64_t N, int64_t K,
                                int32_t group_size, void* stream) {
  return w4a16_gemm_grouped_ex(x, w_packed, scales, m_sizes, y, G, M_total, N, K, group_size, stream, nullptr);
}

w4a16_status w4a16_gemm_grouped_ex(const uint16_t* x, const uint8_t* w_packed, const uint16_t* scales,
                                   const int32_t* m_sizes, uint16_t* y, int32_t G, int64_t M_total, int64_t N,
                                   int64_t K, int32_t group_size, void* stream, const w4a16_config* cfg) {
  if (G < 1 || M_total < 0) return W4A16_ERR_SHAPE;
  w4a16_status st = check_dims(M_total, N, K, group_size);
  if (st != W4A16_OK) return st;
  if ((uint64_t)N * (uint64_t)K / 2u * (uint64_t)G > (uint64_t)INT64_MAX / 2) return W4A16_ERR_SHAPE;
  // one buffer resource covers the scales of all groups
  if ((uint64_t)G * (uint64_t)N * (uint64_t)(K / group_size) * 2u > kMaxBytes) return W4A16_ERR_SHAPE;
  if (M_total == 0) return W4A16_OK;   // empty problem: nothing to read or write
  if (x == nullptr || w_packed == nullptr || scales == nullptr || m_sizes == nullptr || y == nullptr)
    return W4A16_ERR_NULL;
  if (!aligned16(x) || !aligned16(w_packed) || !aligned16(scales) || !aligned16(y)) return W4A16_ERR_ALIGN;
  if (((uintptr_t)m_sizes & 3u) != 0) return W4A16_ERR_ALIGN;
  int bm = -1;
  if (cfg != nullptr) {
    if (cfg->path != 0 && cfg->path != kPathTile) return W4A16_ERR_SHAPE;
    bm = cfg->variant;
  }
  if (bm <= 0) bm = default_grouped_tile_rows(G, M_total, N, K, group_size);
  if (!w4a16::tile_rows_ok(bm, kGroup) && !w4a16::tile_rows_ok(bm, kGroupSmall)) return W4A16_ERR_SHAPE;
  if (!w4a16::tile_rows_ok(bm, group_size)) return W4A16_ERR_GROUP_SIZE;
  const int Gk = (int)(K / kGroup);
  // row sums formed in the kernel: the call takes no workspace
  return launched(w4a16::launch_tile(x, w_packed, scales, nullptr, 0, y, nullptr, m_sizes, 0, (int)M_total, (int)N,
                                     (int)K, G, Gk, 1, bm, group_size, reinterpret_cast<hipStream_t>(stream)));
}

size_t w4a16_gemm_batched_workspace_bytes(int32_t B, int64_t M, int64_t N, int64_t K, int32_t group_size,
                                          int32_t split_k) {
  return batched_workspace_bytes(B, M, N, K, group_size, split_k, nullptr);
}

size_t w4a16_gemm_batched_workspace_bytes_ex(int32_t B, int64_t M, int64_t N, int64_t K, int32_t group_size,
                                             int32_t split_k, const w4a16_config* cfg) {
  return batched_workspace_bytes(B, M, N, K, group_size, split_k, cfg);
}

w4a16_status w4a16_gemm_batched_ex(const uint16_t* x, const uint8_t* w_packed, const uint16_t* scales, uint16_t* y,
                                   int32_t B, int64_t M, int64_t N, int64_t K, int32_t group_size, int32_t split_k,
                                   float* workspace, size_t workspace_bytes, void* stream, const w4a16_config* cfg) {
  if (!valid_split(split_k)) return W4A16_ERR_SPLIT_K;
  w4a16_status st = check_batched(B, M, N, K, group_size);
  if (st != W4A16_OK) return st;
  if (M == 0) return W4A16_OK;   // empty problems: nothing to read or write
  if (x == nullptr || w_packed == nullptr || scales == nullptr || y == nullptr) return W4A16_ERR_NULL;
  if (!aligned16(x) || !aligned16(w_packed) || !aligned16(scales) || !aligned16(y)) return W4A16_ERR_ALIGN;
  BatchedPlan p;
  st = make_batched_plan(B, M, N, K, split_k, cfg, group_size, &p);
  if (st != W4A16_OK) return st;
  if (p.ws_split > kMaxBytes) return W4A16_ERR_SHAPE;
  if (p.ws_split > 0) {
    if (workspace == nullptr) return W4A16_ERR_WORKSPACE;
    if (!aligned16(workspace)) return W4A16_ERR_ALIGN;
    if (workspace_bytes < round_up(p.ws_split, 256)) return W4A16_ERR_WORKSPACE;
  }
  hipStream_t strm = reinterpret_cast<hipStream_t>(stream);
  float* ws_split = p.sk > 1 ? workspace : nullptr;
  const int Mt = (int)((int64_t)B * M);
  const int ld = (int)round_up((uint64_t)Mt, 4);
  float* rowsums = nullptr;
  if (p.ws_sx > 0 && workspace != nullptr && aligned16(workspace) &&
      workspace_bytes >= round_up(p.ws_split, 256) + p.ws_sx)
    rowsums = reinterpret_cast<float*>(reinterpret_cast<uint8_t*>(workspace) + round_up(p.ws_split, 256));
  hipError_t e = hipSuccess;
  if (rowsums != nullptr) e = w4a16::launch_rowsum_neg136(x, rowsums, Mt, (int)K, ld, group_size, strm);
  if (e == hipSuccess)
    e = w4a16::launch_tile(x, w_packed, scales, rowsums, ld, y, ws_split, nullptr, (int)M, Mt, (int)N, (int)K, B,
                           p.gps, p.sk, p.bm, group_size, strm);
  if (e != hipSuccess) return W4A16_ERR_LAUNCH;
  if (p.sk > 1) return launched(w4a16::launch_splitk_reduce(ws_split, y, (uint64_t)Mt * (uint64_t)N, p.sk, strm));
  return W4A16_OK;
}

w4a16_status w4a16_gemm_batched(const uint16_t* x, const uint8_t* w_packed, const uint16_t* scales, uint16_t* y,
                                int32_t B, int64_t M, int64_t N, int64_t K, int32_t group_size, int32_t split_k,
                                float* workspace, size_t workspace_bytes, void* stream) {
  return w4a16_gemm_batched_ex(x, w_packed, scales, y, B, M, N, K, group_size, split_k, workspace, workspace_bytes,
                               stream, nullptr);
}

w4a16_status w4a16_splitk_reduce(const float* workspace, uint16_t* y, int32_t split_k, int64_t M, int64_t N,
                                 void* stream) {
  if (split_k < 1 || split_k > 64 || M < 0 || N < 0) return W4A16_ERR_SHAPE;
  if (M == 0 || N == 0) return W4A16_OK;
  if (workspace == nullptr || y == nullptr) return W4A16_ERR_NULL;
  if (!aligned16(workspace) || !aligned16(y)) return W4A16_ERR_ALIGN;
  if ((uint64_t)M > (uint64_t)INT64_MAX / (uint64_t)N / 64u) return W4A16_ERR_SHAPE;
  return launched(w4a16::launch_splitk_reduce(workspace, y, (uint64_t)M * (uint64_t)N, split_k,
                                              reinterpret_cast<hipStream_t>(stream)));
}

}  // extern "C"
