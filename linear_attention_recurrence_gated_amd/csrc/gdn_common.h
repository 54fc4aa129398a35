// Device helpers shared by the gfx950 kernels of libgdn: wave64 cross-lane sums, the
// FP32 matrix-core product and the XCD-aware block order.
#pragma once

#include <utility>

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

typedef float f32x4 __attribute__((ext_vector_type(4)));

// DPP move within a row of 16 lanes (gfx9 DPP16 control codes).  Written as update_dpp
// with old = 0 and bound_ctrl so that the compiler fuses the move into the consuming add
// (one v_add_f32_dpp per step).
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, true));
}

constexpr int DPP_XOR1 = 0xB1;          // quad_perm [1,0,3,2]
constexpr int DPP_XOR2 = 0x4E;          // quad_perm [2,3,0,1]
constexpr int DPP_HALF_MIRROR = 0x141;  // lane i <- lane 7-i within each 8 lanes
constexpr int DPP_MIRROR = 0x140;       // lane i <- lane 15-i within each 16 lanes
constexpr int SWIZZLE_XOR16 = 0x401F;   // ds_swizzle bit mode: and 0x1f, or 0, xor 0x10

// Sum over the 32 lanes of each half of the wave; every lane receives its half's sum.
// Four DPP steps reduce inside a row of 16 lanes; ds_swizzle (lane ^ 16 within each 32)
// then adds the other row of the half.  (v_permlane16_swap does this last step on the VALU;
// this compiler's builtin for it uses the first result in place of the second, and written
// as inline assembly with its wait states it made the sequential kernel 14 % slower, which
// issues six of these reductions per token and overlaps the swizzles' latencies.)
// Must be executed by all 32 lanes of the half.
__device__ __forceinline__ float half_wave_sum(float x) {
  x += dpp_mov<DPP_XOR1>(x);
  x += dpp_mov<DPP_XOR2>(x);
  x += dpp_mov<DPP_HALF_MIRROR>(x);
  x += dpp_mov<DPP_MIRROR>(x);
  return x + __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, x),
                                                                   SWIZZLE_XOR16));
}

// Gated RMS norm of one (token, value head) row of 128 values held by a half-wave, 4 per
// lane (lane p of the half holds columns 4p .. 4p+3 of o, z and the head's weight w):
//     y_j = fp16_rne( o_j * rsqrt(mean(o^2) + eps) * w_j * sigmoid(z_j) )
// returned as two packed pairs of binary16 bit patterns.  Every kernel that writes y uses
// this one function, so they agree bit for bit.  The reciprocal square root, 2^x and the
// reciprocal are the hardware's single instructions (each within about 1 FP32 ulp), far
// below half an FP16 ulp; the result is then rounded to FP16 by round-to-nearest-even.
// Must be executed by all 32 lanes of the half.
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_half2_rne(float a, float b) {
  const _Float16 ha = (_Float16)a, hb = (_Float16)b;  // round to nearest even
  return (uint32_t)__builtin_bit_cast(uint16_t, ha) |
         ((uint32_t)__builtin_bit_cast(uint16_t, hb) << 16);
}
__device__ __forceinline__ float sigmoid_hw(float x) {
  // 1 / (1 + e^{-x}) with e^{-x} = 2^{-x log2(e)}
  return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(x * -1.44269504088896341f));
}
__device__ __forceinline__ u32x2 gated_rms_row(const f32x4 ov, const f32x4 zv, const float4 wv,
                                               float eps) {
  float ss = ov.x * ov.x + ov.y * ov.y + ov.z * ov.z + ov.w * ov.w;
  ss = half_wave_sum(ss);
  const float rs = __builtin_amdgcn_rsqf(ss * (1.0f / 128) + eps);
  u32x2 out;
  out.x = pack_half2_rne(ov.x * rs * wv.x * sigmoid_hw(zv.x), ov.y * rs * wv.y * sigmoid_hw(zv.y));
  out.y = pack_half2_rne(ov.z * rs * wv.z * sigmoid_hw(zv.z), ov.w * rs * wv.w * sigmoid_hw(zv.w));
  return out;
}

// D = A * B + C on a 16x16 tile with a K-step of 4 (v_mfma_f32_16x16x4_f32).
// Lane l supplies A[l % 16][l / 16] and B[l / 16][l % 16]; the accumulator holds
// C[4 * (l / 16) + r][l % 16] in register r.
__device__ __forceinline__ f32x4 mfma16x16x4(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// Raw buffer resources: the hardware checks every access against num_records, so a load
// past the end returns 0 and a store past the end is dropped.  Ragged tails therefore need
// no branches, every lane issues the same memory operations, and per-lane offsets are
// 32-bit byte offsets from a base held in scalar registers.
typedef __amdgpu_buffer_rsrc_t buf_rsrc;
constexpr int kBufferDword3 = 0x00020000;  // gfx9 raw buffer: 32-bit data format

__device__ __forceinline__ buf_rsrc make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes,
                                           kBufferDword3);
}
// (the b32 builtins move raw 32-bit words: reinterpret the bits, never convert the value)
__device__ __forceinline__ float buf_load(buf_rsrc r, uint32_t byte_off) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, byte_off, 0, 0));
}
__device__ __forceinline__ f32x4 buf_load4(buf_rsrc r, uint32_t byte_off) {
  return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 0));
}
__device__ __forceinline__ void buf_store(buf_rsrc r, uint32_t byte_off, float v) {
  __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), r, byte_off, 0, 0);
}
__device__ __forceinline__ void buf_store2(buf_rsrc r, uint32_t byte_off, u32x2 v) {
  __builtin_amdgcn_raw_buffer_store_b64(v, r, byte_off, 0, 0);
}
// Non-temporal stores (cache policy `nt`): for results that this kernel does not read
// back, so that they stream out instead of staying dirty in the L2 until the kernel ends.
constexpr int kCacheNT = 2;
__device__ __forceinline__ void buf_store_nt(buf_rsrc r, uint32_t byte_off, float v) {
  __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), r, byte_off, 0, kCacheNT);
}
__device__ __forceinline__ void buf_store2_nt(buf_rsrc r, uint32_t byte_off, u32x2 v) {
  __builtin_amdgcn_raw_buffer_store_b64(v, r, byte_off, 0, kCacheNT);
}

// Direct global -> LDS load (gfx950): lane l's 16 bytes at byte_off (from the descriptor's
// base, checked against its size: out of range reads as 0) land at LDS address
// lds_base + LDS_OFF + 16 l, without passing through registers.  The wave-uniform LDS
// address travels in m0.  Issued as inline assembly so that the compiler does not treat it
// as a pending LDS write (it would then wait for every such load before the next LDS
// read); the caller waits with wait_vm_lgkm0 before the barrier that publishes the data.
// On this GFX9-family target a scalar-ALU write of m0 needs one wait state before an
// LDS-DMA load reads it (the compiler's own lowering of these loads puts an s_nop 0 there,
// and its hazard recogniser does not look inside inline assembly), so the sequence carries
// that s_nop itself; m0 is declared clobbered so the compiler keeps nothing of its own in
// it across the load.  LDS_OFF is an immediate, so an unrolled run of loads keeps one base
// register rather than one per destination.
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) char* lds_cptr;
__device__ __forceinline__ i32x4 make_desc(const void* base, int bytes) {
  const uint64_t a = (uint64_t)base;
  return i32x4{(int)(uint32_t)a, (int)(uint32_t)(a >> 32), bytes > 0 ? bytes : 0, kBufferDword3};
}
__device__ __forceinline__ uint32_t lds_address(const void* p) {
  return (uint32_t)(size_t)(lds_cptr)p;
}
template <int LDS_OFF>
__device__ __forceinline__ void dma16(const i32x4& desc, uint32_t byte_off, uint32_t lds_base) {
  asm volatile("s_add_u32 m0, %0, %1\n\ts_nop 0\n\tbuffer_load_dwordx4 %2, %3, 0 offen lds"
               :: "s"(lds_base), "i"(LDS_OFF), "v"(byte_off), "s"(desc) : "scc", "m0");
}
// Loads I = 0, 1, ... of a run: destination LDS_OFF + 1024 I, per-lane offsets off[I].
template <int LDS_OFF, int... I>
__device__ __forceinline__ void dma16_run(const i32x4& desc, const uint32_t* off, uint32_t lds_base,
                                          std::integer_sequence<int, I...>) {
  (dma16<LDS_OFF + 1024 * I>(desc, off[I], lds_base), ...);
}

// s_waitcnt vmcnt(N) lgkmcnt(0): at most N vector memory operations of this wave remain
// in flight (they complete in issue order) and all its LDS operations are done.
template <int N>
__device__ __forceinline__ void wait_vm_lgkm0() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4));
}

// Workgroup barrier without the implicit waits of __syncthreads (the caller has waited for
// exactly what the other waves will read); the empty asm statements keep the compiler
// from moving memory accesses across it.
__device__ __forceinline__ void barrier_only() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Workgroups are handed to the 8 XCDs round-robin (workgroup b runs on XCD b % 8).  This
// maps a workgroup id to a logical block so that consecutive logical blocks share an XCD
// (and its L2): XCD x receives the logical range [x*n/8, (x+1)*n/8).
__device__ __forceinline__ int xcd_grouped_block(int b, int n) {
  return (n % 8 == 0) ? (b % 8) * (n / 8) + b / 8 : b;
}

}  // namespace gdn
