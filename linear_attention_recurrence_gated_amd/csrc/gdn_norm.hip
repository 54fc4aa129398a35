// Gated RMS output norm to FP16 for gfx950.
//
// Per (token, value head) row of 128 values ("#413 prefill: ...", section "What changes":
// the norm reads the FP32 recurrence output and writes only the FP16 copy):
//     y_j = fp16_rne( o_j * rsqrt(mean(o^2) + eps) * w[h][j] * sigmoid(z_j) )
// The pages print no formula; this is the plain reading of a gated RMS norm with a
// per-value-head weight and a sigmoid gate.
//
// Bound by HBM traffic (read o and z, write y: 1280 bytes per row): each half-wave owns a
// row (16 bytes of o and of z per lane, one coalesced 512-byte load each), the sum of
// squares is reduced inside the half-wave with DPP, and a grid-stride loop keeps two rows
// per half-wave in flight.
#include "gdn_common.h"
#include "gdn_kernels.h"

namespace gdn {
namespace {

constexpr int NT = 256;

__device__ __forceinline__ uint32_t pack_half2(float a, float b) {
  const _Float16 ha = (_Float16)a, hb = (_Float16)b;  // round to nearest even
  return (uint32_t)__builtin_bit_cast(uint16_t, ha) |
         ((uint32_t)__builtin_bit_cast(uint16_t, hb) << 16);
}

__device__ __forceinline__ float sigmoid(float x) { return 1.0f / (1.0f + expf(-x)); }

__device__ __forceinline__ void norm_row(const NormArgs& a, int row, int p,
                                         const float4 ov, const float4 zv) {
  const int h = row % a.n_v_heads;
  const float4 wv = *reinterpret_cast<const float4*>(a.w + h * kDim + 4 * p);
  float ss = ov.x * ov.x + ov.y * ov.y + ov.z * ov.z + ov.w * ov.w;
  ss = half_wave_sum(ss);
  const float rs = 1.0f / sqrtf(ss * (1.0f / kDim) + a.eps);
  uint2 out;
  out.x = pack_half2(ov.x * rs * wv.x * sigmoid(zv.x), ov.y * rs * wv.y * sigmoid(zv.y));
  out.y = pack_half2(ov.z * rs * wv.z * sigmoid(zv.z), ov.w * rs * wv.w * sigmoid(zv.w));
  *reinterpret_cast<uint2*>(a.y + row * kDim + 4 * p) = out;
}

__global__ __launch_bounds__(NT) void out_norm_kernel(NormArgs a) {
  const int p = threadIdx.x & 31;
  const int rows_per_iter = gridDim.x * (NT / 32);
  int row = blockIdx.x * (NT / 32) + (threadIdx.x >> 5);
  // two rows per half-wave per iteration; each half-wave's row is uniform across it
  for (; row + rows_per_iter < a.n_rows; row += 2 * rows_per_iter) {
    const int row2 = row + rows_per_iter;
    const float4 o1 = *reinterpret_cast<const float4*>(a.o + row * kDim + 4 * p);
    const float4 z1 = *reinterpret_cast<const float4*>(a.z + row * kDim + 4 * p);
    const float4 o2 = *reinterpret_cast<const float4*>(a.o + row2 * kDim + 4 * p);
    const float4 z2 = *reinterpret_cast<const float4*>(a.z + row2 * kDim + 4 * p);
    norm_row(a, row, p, o1, z1);
    norm_row(a, row2, p, o2, z2);
  }
  if (row < a.n_rows) {
    const float4 o1 = *reinterpret_cast<const float4*>(a.o + row * kDim + 4 * p);
    const float4 z1 = *reinterpret_cast<const float4*>(a.z + row * kDim + 4 * p);
    norm_row(a, row, p, o1, z1);
  }
}

}  // namespace

hipError_t launch_out_norm(const NormArgs& a, hipStream_t stream) {
  void* args[] = {const_cast<NormArgs*>(&a)};
  const int rows_per_block = NT / 32;
  int nblocks = (a.n_rows + rows_per_block - 1) / rows_per_block;
  const int cap = 256 * 16;  // 16 workgroups per CU, then grid-stride
  if (nblocks > cap) nblocks = cap;
  return hipLaunchKernel(reinterpret_cast<const void*>(&out_norm_kernel), dim3(nblocks),
                         dim3(NT), args, 0, stream);
}

}  // namespace gdn
