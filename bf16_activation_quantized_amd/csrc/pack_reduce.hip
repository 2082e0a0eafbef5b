// Element-wise kernels: int4 packing and the split-K reduce.
//
// pack: w_packed[j] = (q[2j] & 0xF) | (q[2j+1] & 0xF) << 4 over the flat
// [rows, K] byte array (K even, so a pair never straddles a row); "Add Triton
// BF16xINT4 rowwise GEMM for ROCm gfx942/gfx950", Implementation "Fused
// A-operand dot" (low nibble = even K).
//
// reduce: y = bf16_rne(sum_s ws[s]) in slice order, fp32; same page,
// "Split-K without atomics".
#include "common.hpp"
#include "launch.hpp"

namespace w4a16 {

// Each thread packs 32 input bytes (two 16-byte loads) into 16 output bytes.
// Bytes b0 (even k) and b1 (odd k) of each input pair become one output byte.
__device__ __forceinline__ uint32_t pack8(uint32_t a, uint32_t b) {
  // a holds k0..k3, b holds k4..k7 (one byte each); output byte i = k(2i) | k(2i+1) << 4
  const uint32_t lo_a = a & 0x000F000Fu;           // k0 at 0, k2 at 16
  const uint32_t hi_a = (a >> 4) & 0x00F000F0u;    // k1 at 4, k3 at 20
  const uint32_t pa = lo_a | hi_a;                 // byte0 = k0|k1<<4, byte2 = k2|k3<<4
  const uint32_t lo_b = b & 0x000F000Fu;
  const uint32_t hi_b = (b >> 4) & 0x00F000F0u;
  const uint32_t pb = lo_b | hi_b;
  // gather bytes 0, 2 of pa and 0, 2 of pb
  return __builtin_amdgcn_perm(pb, pa, 0x06040200u);
}

__global__ __launch_bounds__(256) void pack_int4_kernel(const uint8_t* __restrict__ q,
                                                        uint8_t* __restrict__ out,
                                                        uint64_t total_in) {
  const uint64_t nvec = total_in / 32;
  const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  for (uint64_t v = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; v < nvec; v += stride) {
    const u32x4 a = *reinterpret_cast<const u32x4*>(q + v * 32);
    const u32x4 b = *reinterpret_cast<const u32x4*>(q + v * 32 + 16);
    u32x4 r;
    r.x = pack8(a.x, a.y);
    r.y = pack8(a.z, a.w);
    r.z = pack8(b.x, b.y);
    r.w = pack8(b.z, b.w);
    *reinterpret_cast<u32x4*>(out + v * 16) = r;
  }
  // tail (< 32 input bytes, an even count), handled by the first threads
  const uint64_t done = nvec * 32;
  const uint64_t t = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t < (total_in - done) / 2) {
    const uint64_t i = done + 2 * t;
    out[i / 2] = (uint8_t)((q[i] & 0xF) | ((q[i + 1] & 0xF) << 4));
  }
}

// One thread sums 8 consecutive outputs across the SK slices (two 16-byte
// loads per slice; the loads of up to 8 slices go out before their adds, one
// memory round trip per 8 slices; the adds run in slice order). Against 4
// outputs per thread: 1322 x 2560 at SK 2, 92 -> 88 us for the whole GEMM.
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float* __restrict__ ws,
                                                            uint16_t* __restrict__ y,
                                                            uint64_t mn, int sk) {
  // vector path only when every slice starts 16-byte aligned; the last
  // mn % 8 outputs take the scalar path
  const uint64_t nvec = (mn % 4 == 0) ? mn / 8 : 0;
  const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  for (uint64_t v = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; v < nvec; v += stride) {
    f32x4 a0 = {0.f, 0.f, 0.f, 0.f}, a1 = {0.f, 0.f, 0.f, 0.f};
    for (int s0 = 0; s0 < sk; s0 += 8) {
      f32x4 p0[8], p1[8];
#pragma unroll
      for (int s = 0; s < 8; ++s)
        if (s0 + s < sk) {
          p0[s] = *reinterpret_cast<const f32x4*>(ws + (uint64_t)(s0 + s) * mn + v * 8);
          p1[s] = *reinterpret_cast<const f32x4*>(ws + (uint64_t)(s0 + s) * mn + v * 8 + 4);
        }
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        if (s0 + s < sk) {
          if (s0 + s == 0) {
            a0 = p0[0];
            a1 = p1[0];
          } else {
            a0.x = a0.x + p0[s].x; a0.y = a0.y + p0[s].y; a0.z = a0.z + p0[s].z; a0.w = a0.w + p0[s].w;
            a1.x = a1.x + p1[s].x; a1.y = a1.y + p1[s].y; a1.z = a1.z + p1[s].z; a1.w = a1.w + p1[s].w;
          }
        }
      }
    }
    u32x4 o;
    o.x = pack_bf16x2(a0.x, a0.y);
    o.y = pack_bf16x2(a0.z, a0.w);
    o.z = pack_bf16x2(a1.x, a1.y);
    o.w = pack_bf16x2(a1.z, a1.w);
    *reinterpret_cast<u32x4*>(y + v * 8) = o;
  }
  for (uint64_t i = nvec * 8 + (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < mn; i += stride) {
    float acc = ws[i];
    for (int s = 1; s < sk; ++s) acc = acc + ws[(uint64_t)s * mn + i];
    y[i] = to_bf16(acc);
  }
}

static int grid_for(uint64_t items, int per_block) {
  uint64_t g = (items + per_block - 1) / per_block;
  if (g < 1) g = 1;
  if (g > 65536) g = 65536;
  return (int)g;
}

hipError_t launch_pack_int4(const uint8_t* q, uint8_t* out, uint64_t total_in, hipStream_t stream) {
  hipLaunchKernelGGL(pack_int4_kernel, dim3(grid_for(total_in / 32 + 1, 256)), dim3(256), 0, stream,
                     q, out, total_in);
  return hipGetLastError();
}

hipError_t launch_splitk_reduce(const float* ws, uint16_t* y, uint64_t mn, int sk, hipStream_t stream) {
  hipLaunchKernelGGL(splitk_reduce_kernel, dim3(grid_for((mn % 4 == 0 ? mn / 8 : mn) + 1, 256)), dim3(256), 0, stream,
                     ws, y, mn, sk);
  return hipGetLastError();
}

}  // namespace w4a16
