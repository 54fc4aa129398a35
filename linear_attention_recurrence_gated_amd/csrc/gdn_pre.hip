// The step before the recurrence for gfx950 ("Round 20 Track C Audit: gdn_pre ...",
// section 1: the 4-tap causal conv of gp_conv and the key-head branch of gdn_pre; section
// 2 lists the outputs): per token t and channel c of the projection output x [T][C],
//     u[t][c] = sum_{j<4} w[c][j] xe[t + j][c]    (xe = 3 history rows, then x; tap 3 is
//                                                  the current token)
//     u       = act(u)                              (none, or SiLU u / (1 + e^-u))
//     q = u_q / sqrt(|u_q|^2 + eps) / sqrt(dk),   k = u_k / sqrt(|u_k|^2 + eps),   v = u_v
//     g = -e^{A_log[h]} softplus(a + dt_bias[h]),  beta = 1 / (1 + e^-b)
// and the conv inputs of the last 3 tokens as the history of the next call.  The
// activation, the eps form and the gate formula are this library's readings (the page
// shows the conv and the normalised outputs but prints none of them).
//
// Bound by HBM traffic (each channel of each token is read once and written once), so the
// layout is for streaming: one wave owns one 128-channel block of one head (q or k of a
// key head, v of a value head) for a run of 32 tokens, two channels per lane, so each
// token's block is one coalesced 512-byte load and one 512-byte store.  The three previous
// rows of the conv slide along in registers (a run re-reads only the 3 rows before it).
// Loads go out in batches of 16 tokens, the next batch's while the current one is
// computed, and loads and stores are non-temporal (streamed data that nothing here reads
// again); measured at T = 32768 against the same kernel with batches of 4 tokens, 64-token
// runs and no prefetch: 5.6 against 4.5 TB/s, where a device-to-device copy of the same
// bytes through the framework's copy reaches 5.0.  The q/k normalisation is a wave-wide
// sum (DPP inside each row of 16 lanes and across the rows).  SiLU's sigmoid and the
// normalisation's reciprocal square root use the hardware's single instructions; the gate
// and beta, one thread per value, use the exact exp and log1p.  Extra workgroups
// at the end of the grid form the gate and beta.
#include "gdn_common.h"
#include "gdn_kernels.h"

namespace gdn {
namespace {

constexpr int PRE_NT = 256;    // 4 waves per workgroup
constexpr int PRE_RUN = 32;    // tokens per wave
constexpr int PRE_BATCH = 16;  // tokens whose loads are issued together

typedef float nt_f2 __attribute__((ext_vector_type(2)));  // for the non-temporal builtins

__device__ __forceinline__ float row16_sum(float x) {
  x += dpp_mov<DPP_XOR1>(x);
  x += dpp_mov<DPP_XOR2>(x);
  x += dpp_mov<DPP_HALF_MIRROR>(x);
  x += dpp_mov<DPP_MIRROR>(x);
  return x;
}

constexpr int DPP_ROW_BCAST15 = 0x142;  // row r <- lane 15 of row r - 1 (rows in row_mask)
constexpr int DPP_ROW_BCAST31 = 0x143;  // rows 2, 3 <- lane 31 (rows in row_mask)

// Sum over the 64 lanes as a wave-uniform value, in a fixed order: each 16-lane row sums
// itself, then rows 1 and 3 add rows 0 and 2 and row 3 adds lane 31's value, so lane 63
// holds (s2 + s3) + (s0 + s1).
__device__ __forceinline__ float wave_sum(float x) {
  x = row16_sum(x);
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x),
                                                             DPP_ROW_BCAST15, 0xA, 0xF, false));
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x),
                                                             DPP_ROW_BCAST31, 0xC, 0xF, false));
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 63));
}

// u * sigmoid(u) with the sigmoid from the hardware's 2^x and reciprocal (each within about
// 1 FP32 ulp): far below the tolerance of the step, at a fraction of the exact functions'
// instructions in a kernel that streams its data once.
__device__ __forceinline__ float silu(float u) {
  return u * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(u * -1.44269504088896341f));
}

__device__ __forceinline__ float softplus(float z) {
  return z > 0.f ? z + log1pf(expf(-z)) : log1pf(expf(z));  // log(1 + e^z)
}

// One wave: head block hb (0 .. Hk-1: q of key head hb; Hk .. 2Hk-1: k of key head hb-Hk;
// then v of value head hb-2Hk) for tokens [t0, t1).
__device__ __forceinline__ void conv_run(const PreArgs& a, int hb, int t0, int t1) {
  const int Hk = a.n_k_heads, Hv = a.n_v_heads;
  const int64_t C = (int64_t)(2 * Hk + Hv) * kDim;
  const int p = threadIdx.x & 63;
  const int64_t ch = (int64_t)hb * kDim + 2 * p;  // first of this lane's two channels
  const float4 w0 = *reinterpret_cast<const float4*>(a.conv_w + ch * 4);
  const float4 w1 = *reinterpret_cast<const float4*>(a.conv_w + (ch + 1) * 4);

  // xe row r of this lane's channels: history row r for r < 3, else x row r - 3
  auto xe = [&](int64_t r) {
    const float* src = r < 3 ? a.hist_in + r * C : a.x + (r - 3) * C;
    return *reinterpret_cast<const float2*>(src + ch);
  };
  // the rows before token t0: xe[t0], xe[t0 + 1], xe[t0 + 2]
  float2 h0 = xe(t0), h1 = xe(t0 + 1), h2 = xe(t0 + 2);

  const bool is_q = hb < Hk, is_k = !is_q && hb < 2 * Hk;
  float* out;
  int64_t ostride;
  if (is_q) {
    out = a.q + (int64_t)hb * kDim + 2 * p;
    ostride = (int64_t)Hk * kDim;
  } else if (is_k) {
    out = a.k + (int64_t)(hb - Hk) * kDim + 2 * p;
    ostride = (int64_t)Hk * kDim;
  } else {
    out = a.v + (int64_t)(hb - 2 * Hk) * kDim + 2 * p;
    ostride = (int64_t)Hv * kDim;
  }
  const float qscale = 0.08838834764831845f;  // 1 / sqrt(128), rounded to float

  // Batches of PRE_BATCH tokens, the loads of batch b + 1 in flight while batch b is
  // computed (two register buffers, alternating, so every index is a constant).
  auto load = [&](float2 (&xr)[PRE_BATCH], int tb) {
#pragma unroll
    for (int i = 0; i < PRE_BATCH; ++i)
      if (tb + i < t1) {
        const nt_f2 v = __builtin_nontemporal_load(
            reinterpret_cast<const nt_f2*>(a.x + (int64_t)(tb + i) * C + ch));
        xr[i] = make_float2(v.x, v.y);
      }
  };
  auto compute = [&](const float2 (&xr)[PRE_BATCH], int tb) {
#pragma unroll
    for (int i = 0; i < PRE_BATCH; ++i) {
      if (tb + i < t1) {  // uniform across the wave
        const float2 cur = xr[i];
        float u0 = fmaf(w0.w, cur.x, fmaf(w0.z, h2.x, fmaf(w0.y, h1.x, w0.x * h0.x)));
        float u1 = fmaf(w1.w, cur.y, fmaf(w1.z, h2.y, fmaf(w1.y, h1.y, w1.x * h0.y)));
        if (a.activation) {
          u0 = silu(u0);
          u1 = silu(u1);
        }
        if (is_q || is_k) {
          const float ss = wave_sum(fmaf(u1, u1, u0 * u0));
          float r = __builtin_amdgcn_rsqf(ss + a.eps);  // hardware 1/sqrt, within ~1 ulp
          if (is_q) r *= qscale;
          u0 *= r;
          u1 *= r;
        }
        __builtin_nontemporal_store(nt_f2{u0, u1},
                                    reinterpret_cast<nt_f2*>(out + (int64_t)(tb + i) * ostride));
        h0 = h1;
        h1 = h2;
        h2 = cur;
      }
    }
  };
  float2 xa[PRE_BATCH], xb[PRE_BATCH];
  load(xa, t0);
  for (int tb = t0; tb < t1; tb += 2 * PRE_BATCH) {
    if (tb + PRE_BATCH < t1) load(xb, tb + PRE_BATCH);
    compute(xa, tb);
    if (tb + PRE_BATCH >= t1) break;
    if (tb + 2 * PRE_BATCH < t1) load(xa, tb + 2 * PRE_BATCH);
    compute(xb, tb + PRE_BATCH);
  }
  if (t1 == a.T) {  // the conv inputs of the call's last 3 tokens: xe[T], xe[T+1], xe[T+2]
    *reinterpret_cast<float2*>(a.hist_out + ch) = h0;
    *reinterpret_cast<float2*>(a.hist_out + C + ch) = h1;
    *reinterpret_cast<float2*>(a.hist_out + 2 * C + ch) = h2;
  }
}

__global__ __launch_bounds__(PRE_NT) void pre_kernel(PreArgs a, int conv_blocks) {
  const int b = blockIdx.x;
  if (b < conv_blocks) {
    const int n_hb = 2 * a.n_k_heads + a.n_v_heads;
    const int wave = b * (PRE_NT / 64) + (threadIdx.x >> 6);
    const int runs = (a.T + PRE_RUN - 1) / PRE_RUN;
    if (wave >= runs * n_hb) return;  // whole waves
    // consecutive waves take consecutive head blocks of the same run of tokens
    const int run = wave / n_hb, hb = wave % n_hb;
    const int t0 = run * PRE_RUN;
    conv_run(a, hb, t0, min(a.T, t0 + PRE_RUN));
  } else {
    // gate and beta: one thread per (token, value head)
    const int64_t e = (int64_t)(b - conv_blocks) * PRE_NT + threadIdx.x;
    if (e >= (int64_t)a.T * a.n_v_heads) return;
    const int h = (int)(e % a.n_v_heads);
    a.g[e] = -expf(a.A_log[h]) * softplus(a.a[e] + a.dt_bias[h]);
    a.beta[e] = 1.0f / (1.0f + expf(-a.b[e]));
  }
}

}  // namespace

bool pre_grid(int64_t T, int n_k_heads, int n_v_heads, bool gates, int* conv_blocks,
              int* blocks) {
  constexpr int64_t kMax = (int64_t)1 << 31;
  const int64_t waves = (T + PRE_RUN - 1) / PRE_RUN * (2 * n_k_heads + n_v_heads);
  const int64_t cb = (waves + PRE_NT / 64 - 1) / (PRE_NT / 64);
  const int64_t gb = gates ? (T * n_v_heads + PRE_NT - 1) / PRE_NT : 0;
  if (waves >= kMax || cb + gb >= kMax) return false;
  *conv_blocks = (int)cb;
  *blocks = (int)(cb + gb);
  return true;
}

hipError_t launch_pre(const PreArgs& a, hipStream_t stream) {
  int conv_blocks = 0, blocks = 0;
  if (!pre_grid(a.T, a.n_k_heads, a.n_v_heads, a.a != nullptr, &conv_blocks, &blocks))
    return hipErrorInvalidValue;
  void* args[] = {const_cast<PreArgs*>(&a), &conv_blocks};
  return hipLaunchKernel(reinterpret_cast<const void*>(&pre_kernel), dim3(blocks),
                         dim3(PRE_NT), args, 0, stream);
}

}  // namespace gdn
