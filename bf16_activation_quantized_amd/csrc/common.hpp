// Device helpers shared by the W4A16 kernels (gfx950 / CDNA4 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace w4a16 {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int kGroup = 128;            // K elements per scale group
constexpr uint32_t kRsrcWord3 = 0x00020000u;   // raw buffer, 32-bit data format

// ---------------------------------------------------------------- buffers
// A buffer resource with an exact byte extent: loads past `bytes` return 0
// and stores past it are dropped by the hardware, so tails need no guards
// ("[ROCm][Kernel] W4A16 skinny GEMM: hand-asm kernel for gfx1151", section 3
// "Exact buffer-descriptor sizing").
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, kRsrcWord3);
}

// Scales read as the aligned 32-bit word that holds them: the buffer starts
// at the (16-byte aligned) tensor base and its extent is rounded up to a
// multiple of 4. The at most 2 bytes past the tensor lie in the same aligned
// word as its last scale, hence in a mapped page; without the rounding, an
// odd element count would make the word of the last scale partly out of range
// and the hardware would return 0 for all of it.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_scale_rsrc(const uint16_t* s, uint32_t count) {
  return make_rsrc(s, (count * 2u + 3u) & ~3u);
}

__device__ __forceinline__ u32x4 ld128(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff = 0) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
}
__device__ __forceinline__ uint32_t ld32(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff = 0) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0);
}
__device__ __forceinline__ u32x2 ld64(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff = 0) {
  return __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, 0);
}
__device__ __forceinline__ uint16_t ld16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff = 0) {
  return __builtin_amdgcn_raw_buffer_load_b16(r, voff, soff, 0);
}
__device__ __forceinline__ void st128(u32x4 v, __amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff = 0) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, voff, soff, 0);
}
__device__ __forceinline__ void st64(u32x2 v, __amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff = 0) {
  __builtin_amdgcn_raw_buffer_store_b64(v, r, voff, soff, 0);
}
__device__ __forceinline__ void st32(uint32_t v, __amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff = 0) {
  __builtin_amdgcn_raw_buffer_store_b32(v, r, voff, soff, 0);
}
__device__ __forceinline__ void st16(uint16_t v, __amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff = 0) {
  __builtin_amdgcn_raw_buffer_store_b16(v, r, voff, soff, 0);
}

// ---------------------------------------------------------------- LDS
// XOR swizzle of the 16-byte chunks of an LDS operand row, by row & 15: the
// row's low two bits, and its 4-row block j = (row >> 2) & 3 mapped to
// 0, 2, 3, 1. Chunk c of row r sits in slot c ^ xswz(r) (within its aligned
// run of 16 chunks). A wave's 16-byte MFMA fragment read, lane (m, kb) at row
// m and chunk 4 kb + st (or kb + 4 st), then takes the 4 cycles of a
// conflict-free read on gfx950 by the LDS bank-conflict counter, for rows of
// any multiple of 256 B; XOR by row & 7 or by row & 15 measured 2-way
// conflicts (8 cycles). The block map is a permutation whose XOR with the
// identity is one too.
// Lanes of one wave exchanging data through LDS (each lane reads what other
// lanes of its wave wrote): one wave's LDS instructions are executed in
// program order, but the compiler, reasoning per lane, may move a lane's
// reads above writes it can tell go elsewhere (and, across a loop, its next
// writes above its reads). An empty asm with a memory clobber between the two
// sides keeps them in program order.
__device__ __forceinline__ void wave_lds_exchange() { asm volatile("" ::: "memory"); }

__device__ __forceinline__ uint32_t xswz(int r) {
  return (uint32_t)((r & 3) | ((r >> 1) & 4) | ((((r >> 2) ^ (r >> 3)) & 1) << 3));
}

// ---------------------------------------------------------------- bf16
__device__ __forceinline__ float bf16lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16hi(uint32_t v) { return __uint_as_float(v & 0xFFFF0000u); }
__device__ __forceinline__ float bf16f(uint16_t v) { return __uint_as_float((uint32_t)v << 16); }

// A 32-bit word as a bf16 pair. Taken by value on purpose: clang's
// __builtin_bit_cast applied directly to an ext-vector element (v.y) reads the
// vector's first element instead (observed with ROCm 7.2 clang).
__device__ __forceinline__ bf16x2 as_bf16x2(uint32_t u) { return __builtin_bit_cast(bf16x2, u); }

// Two fp32 -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2 r = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, r);
}
__device__ __forceinline__ uint16_t to_bf16(float v) {
  return (uint16_t)(pack_bf16x2(v, 0.0f) & 0xFFFFu);
}

// ---------------------------------------------------------------- dequant
// Magic-constant int4 -> bf16 ("[ROCm][Kernel] W4A16 skinny GEMM ...",
// section 1): a nibble n OR-ed into the low mantissa bits of the bf16 pattern
// 0x4300 (= 128.0, whose ulp is 1) reads as bf16(128 + n), exactly. The
// contraction then sees (128 + n); the "- 136" of the page's (128 + n) - 136
// = n - 8 is applied outside the dot, once per group, as -136 * sum(x).
constexpr uint32_t kMagicPair = 0x43004300u;
constexpr uint32_t kNibblePairMask = 0x000F000Fu;

// Word w holds the nibbles of 8 consecutive k (k0 in bits 0-3 ... k7 in
// bits 28-31). Pair j (0..3) = (bf16(128+q[j]), bf16(128+q[j+4])), i.e. the
// k order inside the 8-block becomes (0,4,1,5,2,6,3,7).
__device__ __forceinline__ uint32_t magic_pair_interleaved(uint32_t w, int j) {
  return ((w >> (4 * j)) & kNibblePairMask) | kMagicPair;
}

// (a & m) | o in one VOP3 instruction. gfx950 VOP3 cannot encode literal
// constants, so the compiler would split a literal-mask and-or into two VOP2
// instructions; here the mask comes from an SGPR and `o` from a VGPR.
__device__ __forceinline__ uint32_t and_or_sv(uint32_t a, uint32_t m_sgpr, uint32_t o_vgpr) {
  uint32_t r;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "s"(m_sgpr), "v"(o_vgpr));
  return r;
}
// An opaque VGPR copy of a constant, so that it stays in one register.
__device__ __forceinline__ uint32_t vgpr_const(uint32_t c) {
  uint32_t r;
  asm volatile("v_mov_b32 %0, %1" : "=v"(r) : "s"(c));
  return r;
}

// Two dwords shifted right by `sh` with one v_lshrrev_b64 (issued at the rate
// of a 32-bit shift on gfx950): bits of `hi` that move into `lo` land in
// positions that the nibble mask clears, so lo >> sh and hi >> sh are both
// usable for the magic-constant unpack. Inline asm keeps the compiler from
// splitting it into two 32-bit shifts.
template <int SH>
__device__ __forceinline__ void shr64_pair(uint32_t lo, uint32_t hi, uint32_t& olo, uint32_t& ohi) {
  const uint64_t v = ((uint64_t)hi << 32) | lo;
  uint64_t r;
  asm("v_lshrrev_b64 %0, %1, %2" : "=v"(r) : "n"(SH), "v"(v));
  olo = (uint32_t)r;
  ohi = (uint32_t)(r >> 32);
}

// Natural k order: pair j (0..3) = (bf16(128+q[2j]), bf16(128+q[2j+1])).
// v_perm puts byte j of w into byte 0 and byte j of (w >> 4) into byte 2.
__device__ __forceinline__ uint32_t magic_pair_natural(uint32_t w, uint32_t w4, int j) {
  // selector: byte0 <- src1.byte j (w), byte2 <- src0.byte j (w4); bytes 1, 3 unused (masked)
  const uint32_t sel = (uint32_t)j | ((uint32_t)(4 + j) << 16) | 0x0C000C00u;
  return (__builtin_amdgcn_perm(w4, w, sel) & kNibblePairMask) | kMagicPair;
}

// ---------------------------------------------------------------- DPP sums
// Cross-lane sums on the VALU with DPP (a few cycles per step) instead of
// ds_bpermute round trips through the LDS unit.
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROW_MASK, 0xF, true));
}
// Sum over each row of 16 lanes; every lane of the row gets the row's sum.
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp_f<0xB1>(v);    // quad_perm [1,0,3,2]
  v += dpp_f<0x4E>(v);    // quad_perm [2,3,0,1]
  v += dpp_f<0x141>(v);   // row_half_mirror
  v += dpp_f<0x140>(v);   // row_mirror
  return v;
}
// Sum over each half-wave (32 lanes): valid in lanes 16..31 and 48..63.
__device__ __forceinline__ float half32_sum(float v) {
  v = row16_sum(v);
  v += dpp_f<0x142, 0xA>(v);   // row_bcast15 into rows 1 and 3
  return v;
}
// Sum over the whole wave: valid in lanes 48..63.
__device__ __forceinline__ float wave64_sum(float v) {
  v = half32_sum(v);
  v += dpp_f<0x143, 0xC>(v);   // row_bcast31 into rows 2 and 3
  return v;
}

// ---------------------------------------------------------------- XCD mapping
// Workgroups are dispatched to the 8 XCDs round robin (blockIdx % 8). Remap so
// that each XCD owns a contiguous run of logical tile ids: neighbouring tiles
// (which share weight columns) then share one XCD's L2 ("Add Triton
// BF16xINT4 rowwise GEMM for ROCm gfx942/gfx950", Implementation "XCD
// remapping").
constexpr int kNumXcd = 8;
__device__ __forceinline__ int xcd_remap(int bid, int nblocks) {
  const int per = (nblocks + kNumXcd - 1) / kNumXcd;
  const int xcd = bid % kNumXcd;
  const int idx = bid / kNumXcd;
  // XCDs with index < rem own `per` tiles, the others `per - 1`
  const int rem = nblocks - (per - 1) * kNumXcd;
  int base;
  if (xcd < rem) base = xcd * per;
  else base = rem * per + (xcd - rem) * (per - 1);
  return base + idx;
}

}  // namespace w4a16
