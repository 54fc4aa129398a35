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
// squares is reduced inside the half-wave with DPP, and a grid-stride loop issues the
// loads of two rows per half-wave before any arithmetic, with non-temporal (streaming)
// loads and stores since every byte is touched once.
#include "gdn_common.h"
#include "gdn_kernels.h"

namespace gdn {
namespace {

constexpr int NT = 256;

__device__ __forceinline__ void norm_row(const NormArgs& a, int row, int p, const f32x4 ov,
                                         const f32x4 zv) {
  const int h = row % a.n_v_heads;
  const float4 wv = *reinterpret_cast<const float4*>(a.w + h * kDim + 4 * p);
  __builtin_nontemporal_store(gated_rms_row(ov, zv, wv, a.eps),
                              reinterpret_cast<u32x2*>(a.y + row * kDim + 4 * p));
}

// rows per half-wave per iteration, all loaded before any math (measured at T = 32768:
// 1, 2, 3, 4, 6, 8 rows: 391, 382, 390, 397, 428, 464 us; fewer registers per wave leave
// more waves resident to cover the memory latency)
constexpr int ROWS = 2;

__global__ __launch_bounds__(NT) void out_norm_kernel(NormArgs a) {
  const int p = threadIdx.x & 31;
  const int hw = blockIdx.x * (NT / 32) + (threadIdx.x >> 5);  // this half-wave
  const int nhw = gridDim.x * (NT / 32);
  // Rows hw, hw + nhw, hw + 2 nhw, ...; each half-wave's row is uniform across its 32
  // lanes, so the conditions below never split a half-wave.
  for (int row = hw; row < a.n_rows; row += ROWS * nhw) {
    f32x4 ov[ROWS], zv[ROWS];
#pragma unroll
    for (int u = 0; u < ROWS; ++u) {
      const int r = row + u * nhw;
      if (r < a.n_rows) {
        ov[u] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(a.o + r * kDim) + p);
        zv[u] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(a.z + r * kDim) + p);
      }
    }
#pragma unroll
    for (int u = 0; u < ROWS; ++u) {
      const int r = row + u * nhw;
      if (r < a.n_rows) norm_row(a, r, p, ov[u], zv[u]);
    }
  }
}

}  // namespace

hipError_t launch_out_norm(const NormArgs& a, hipStream_t stream) {
  void* args[] = {const_cast<NormArgs*>(&a)};
  const int rows_per_block = (NT / 32) * ROWS;
  int nblocks = (a.n_rows + rows_per_block - 1) / rows_per_block;
  const int cap = 256 * 8;  // 8 workgroups per CU (32 waves), then grid-stride
  if (nblocks > cap) nblocks = cap;
  return hipLaunchKernel(reinterpret_cast<const void*>(&out_norm_kernel), dim3(nblocks),
                         dim3(NT), args, 0, stream);
}

}  // namespace gdn
