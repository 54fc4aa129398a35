// Internal interface between the C-ABI layer (gdn_api.hip) and the kernel launchers.
// Every launcher enqueues on `stream` and returns the hipError_t of the launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace gdn {

constexpr int kDim = 128;          // dk = dv supported by every kernel
constexpr int kMaxGroup = 4;       // value heads per key head supported
constexpr int kChunk = 32;         // tokens per WY chunk
constexpr int kSuperBlock = 2048;  // tokens whose chunk operators are prepared at once
constexpr int kChunksPerSB = kSuperBlock / kChunk;
// Floats per (chunk, value head) in the chunked workspace:
//   [0, 1024)    T * diag(beta), row-major 32x32 (T = (I + A)^-1)
//   [1024, 2048) P, row-major 32x32
//   [2048, 2080) e^{gamma_t}
//   [2080, 2112) e^{gamma_last - gamma_t}
//   [2112]       e^{gamma_last}
//   [2113, 2176) padding (keeps every slot 256-byte aligned)
constexpr int kSlot = 2176;
constexpr int kSlotT = 0, kSlotP = 1024, kSlotEg = 2048, kSlotEb = 2080, kSlotEgl = 2112;

struct SeqArgs {
  const float* q;
  const float* k;
  const float* v;
  const float* g;
  const float* beta;
  const float* s_in;
  float* s_out;
  float* o;
  int T;
  int n_k_heads;
};

struct ChunkArgs {
  const float* q;
  const float* k;
  const float* v;
  const float* g;
  const float* beta;
  const float* s_src;  // state before the super-block
  float* s_dst;        // state after the super-block
  float* o;
  float* ws;
  int t_begin;         // first token of the super-block
  int n_tok;           // tokens in the super-block (1 .. kSuperBlock)
  int n_k_heads;
  int n_v_heads;
};

struct NormArgs {
  const float* o;
  const float* z;
  const float* w;
  uint16_t* y;
  float eps;
  int n_rows;  // T * n_v_heads
  int n_v_heads;
};

struct PreArgs {
  const float* x;        // [T][C], C = (2 n_k_heads + n_v_heads) * 128: q | k | v channels
  const float* conv_w;   // [C][4]
  const float* hist_in;  // [3][C]
  float* hist_out;       // [3][C]
  const float* a;        // [T][n_v_heads] raw gate (NULL: no gate and beta)
  const float* b;        // [T][n_v_heads] raw beta
  const float* A_log;    // [n_v_heads]
  const float* dt_bias;  // [n_v_heads]
  float* q;              // [T][n_k_heads][128]
  float* k;              // [T][n_k_heads][128]
  float* v;              // [T][n_v_heads][128]
  float* g;              // [T][n_v_heads]
  float* beta;           // [T][n_v_heads]
  int activation;        // 0: none, 1: SiLU
  float eps;
  int T;
  int n_k_heads;
  int n_v_heads;
};

// Compute units of the device that `stream` runs on (queried once per device, then cached).
hipError_t device_cu_count(hipStream_t stream, int* cus);

hipError_t launch_seq(const SeqArgs& a, int group, hipStream_t stream);
hipError_t launch_chunk_prep(const ChunkArgs& a, hipStream_t stream);
// Scan of super-block `scan`; if prep_next is not NULL the same launch also forms the
// operators of the next super-block (into prep_next->ws, the other workspace half); if
// norm_prev is not NULL it also runs the output norm of norm_prev->n_rows rows (those of
// the previous super-block, whose o was written by the previous launch).
hipError_t launch_chunk_scan_fused(const ChunkArgs& scan, const ChunkArgs* prep_next,
                                   const NormArgs* norm_prev, hipStream_t stream);
hipError_t launch_out_norm(const NormArgs& a, hipStream_t stream);
// Grid of the pre kernel (one wave per run of tokens of one 128-channel head block, then
// one thread per gate value): false if a wave or workgroup index would not fit in 31 bits.
bool pre_grid(int64_t T, int n_k_heads, int n_v_heads, bool gates, int* conv_blocks,
              int* blocks);
hipError_t launch_pre(const PreArgs& a, hipStream_t stream);

}  // namespace gdn
