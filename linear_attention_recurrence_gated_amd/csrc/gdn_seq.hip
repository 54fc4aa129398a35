// Sequential gated delta rule for gfx950: one token at a time, the state on chip.
//
// Per value head h and token t ("#413 prefill: DeltaNet recurrence with the three value
// heads of a key head in one thread", sections "What changes" and "Exactness"):
//     kv = e^{g} S^T k,   d = beta (v - kv),   S <- e^{g} S + k d^T,   o = S^T q.
// The output sum is taken from the pre-update state: o = e^{g} (S^T q) + d (k.q), which
// is the same quantity and lets the kv sum and the output sum run side by side.
//
// Work split (designed for wave64 and 256 CUs with four SIMDs each, not taken from the
// pages):
//  - one workgroup = one key head x 8 value columns, for all G value heads of that key
//    head (they share every staged tile of q/k rows); 16 key heads x 16 column blocks =
//    256 workgroups, one per CU;
//  - a 64-lane wave holds 2 value columns of one value head, 32 lanes per column (two DPP
//    rows), each lane owning 4 of the 128 key rows (4 floats of state in VGPRs for the
//    whole sequence).  A value head has 4 waves, so a workgroup has 4G waves: for G = 3,
//    12 waves, exactly 3 per SIMD, which keeps every SIMD equally loaded and gives each
//    three independent dependency chains to interleave;
//  - the kv and output sums over the 128 rows are chains of four products per lane, four
//    DPP steps inside each row of 16 lanes, then one exchange between the two rows of a
//    column for both sums at once (v_permlane16_swap trades the kv row sums of the odd rows
//    for the output row sums of the even rows, so after one add the even rows hold the kv
//    sum and the odd rows the output sum, and one DPP row broadcast copies the kv sum to
//    the odd rows): no LDS round trip and no barrier per token;
//  - the inputs of 16 tokens (q/k rows of the key head, the block's v columns, e^{g},
//    beta and k.q) are staged in double-buffered LDS; the next tile's global loads are in
//    flight while the current tile computes; one barrier per 16 tokens.
#include <type_traits>

#include "gdn_common.h"
#include "gdn_kernels.h"

namespace gdn {
namespace {

constexpr int TB = 16;    // tokens per staged tile
constexpr int COLS = 8;   // value columns per workgroup
constexpr int NT = 256;   // threads that stage the q/k rows
constexpr int RPL = 4;    // key rows per lane: 32 lanes per column
template <int G>
constexpr int seq_threads() { return 256 * G; }  // 4 waves per value head
constexpr int NCB = kDim / COLS;  // column blocks per key head

template <int G>
struct SeqSmem {
  float k[2][TB][kDim];
  float q[2][TB][kDim];
  float v[2][TB][G][COLS];
  float2 ab[2][TB][G];  // (e^{g}, beta)
  float kq[2][TB];      // k.q of the key head
  // outputs: [..][1][col] from the odd row of each column (where the output sum lands),
  // [..][0][col] written and never read by the even row, so no lane needs a branch
  float o[2][TB][G][2][COLS];
};

// One thread's share of a tile's inputs, in registers until written to LDS.
struct SeqStage {
  float4 k[2], q[2];
  float4 v;
  float g, b;
};

template <int G>
__device__ __forceinline__ void stage_load(SeqStage& st, const SeqArgs& a, int t0, int kh,
                                           int cb, int tid) {
  const int Hk = a.n_k_heads, Hv = G * a.n_k_heads;
  const int p = tid & 31;
  if (tid < NT) {  // whole waves
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const int t = min(t0 + (tid >> 5) + 8 * m, a.T - 1);  // clamped rows are never used
      const int off = (t * Hk + kh) * kDim + 4 * p;
      st.k[m] = *reinterpret_cast<const float4*>(a.k + off);
      st.q[m] = *reinterpret_cast<const float4*>(a.q + off);
    }
  }
  if (tid < TB * G * 2) {
    const int tt = tid / (2 * G), rem = tid % (2 * G), m = rem >> 1, half = rem & 1;
    const int t = min(t0 + tt, a.T - 1);
    st.v = *reinterpret_cast<const float4*>(a.v + (t * Hv + kh + m * Hk) * kDim + cb * COLS +
                                            4 * half);
  }
  if (tid < TB * G) {
    const int tt = tid / G, m = tid % G;
    const int t = min(t0 + tt, a.T - 1);
    const int off = t * Hv + kh + m * Hk;
    st.g = a.g[off];
    st.b = a.beta[off];
  }
}

template <int G>
__device__ __forceinline__ void stage_store(SeqSmem<G>& sm, int buf, const SeqStage& st,
                                            int tid) {
  const int p = tid & 31;
  if (tid < NT) {  // whole waves
    float part[2];
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const int tt = (tid >> 5) + 8 * m;
      *reinterpret_cast<float4*>(&sm.k[buf][tt][4 * p]) = st.k[m];
      *reinterpret_cast<float4*>(&sm.q[buf][tt][4 * p]) = st.q[m];
      // explicit fused operations: the prologue's copy of this code and the loop's must
      // evaluate k.q alike (left to the compiler, they may be contracted differently)
      part[m] = fmaf(st.k[m].w, st.q[m].w,
                     fmaf(st.k[m].z, st.q[m].z, fmaf(st.k[m].y, st.q[m].y, st.k[m].x * st.q[m].x)));
    }
    // each half-wave holds one token's k and q rows
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const float s = half_wave_sum(part[m]);
      if (p == 0) sm.kq[buf][(tid >> 5) + 8 * m] = s;
    }
  }
  if (tid < TB * G * 2) {
    const int tt = tid / (2 * G), rem = tid % (2 * G), m = rem >> 1, half = rem & 1;
    *reinterpret_cast<float4*>(&sm.v[buf][tt][m][4 * half]) = st.v;
  }
  if (tid < TB * G) {
    const int tt = tid / G, m = tid % G;
    sm.ab[buf][tt][m] = make_float2(expf(st.g), st.b);
  }
}

template <int G>
__device__ __forceinline__ void store_outputs(const SeqSmem<G>& sm, int buf, const SeqArgs& a,
                                              int t0, int kh, int cb, int tid) {
  if (tid < TB * G * 2) {
    const int Hk = a.n_k_heads, Hv = G * a.n_k_heads;
    const int tt = tid / (2 * G), rem = tid % (2 * G), m = rem >> 1, half = rem & 1;
    const int t = t0 + tt;
    if (t < a.T)
      *reinterpret_cast<float4*>(a.o + (t * Hv + kh + m * Hk) * kDim + cb * COLS + 4 * half) =
          *reinterpret_cast<const float4*>(&sm.o[buf][tt][m][1][4 * half]);
  }
}

// Sum over the 16 lanes of each DPP row; every lane receives its row's sum.
__device__ __forceinline__ float row16_sum(float x) {
  x += dpp_mov<DPP_XOR1>(x);
  x += dpp_mov<DPP_XOR2>(x);
  x += dpp_mov<DPP_HALF_MIRROR>(x);
  x += dpp_mov<DPP_MIRROR>(x);
  return x;
}

// v_permlane16_swap_b32 x, y: the odd 16-lane rows of x trade places with the even rows of
// y.  Inline assembly because this compiler's builtin for it returns one of the two
// results for both; the s_nop gives the two wait states the instruction needs after a
// vector-ALU write of its operands (the compiler's own lowering places the same s_nop 1).
__device__ __forceinline__ void permlane16_swap(float& x, float& y) {
  asm volatile("s_nop 1\n\tv_permlane16_swap_b32 %0, %1" : "+v"(x), "+v"(y));
}

// One token of one wave: kc, qc are this token's k and q rows of the lane (already in
// registers); the next token's rows are read into kn, qn while it computes.
template <int G>
__device__ __forceinline__ void token_step(SeqSmem<G>& sm, int buf, int tt, int tn,
                                           const float4* kr, const float4* qr,
                                           const float4& kc, const float4& qc, float4& kn,
                                           float4& qn, float (&S)[RPL], int m, int cl,
                                           int parity) {
  constexpr int ROW4 = kDim / 4;  // float4 per token row
  kn = kr[tn * ROW4];
  qn = qr[tn * ROW4];
  const float2 ab = sm.ab[buf][tt][m];
  const float vv = sm.v[buf][tt][m][cl];
  const float kq = sm.kq[buf][tt];
  // four products per lane, then the 16 lanes of each DPP row
  float pk = fmaf(S[3], kc.w, fmaf(S[2], kc.z, fmaf(S[1], kc.y, S[0] * kc.x)));
  float pq = fmaf(S[3], qc.w, fmaf(S[2], qc.z, fmaf(S[1], qc.y, S[0] * qc.x)));
  pk = row16_sum(pk);
  pq = row16_sum(pq);
  // the two rows of the column: even rows end with S^T k, odd rows with S^T q
  permlane16_swap(pk, pq);  // by row: pk = (pk0, pq0, pk2, pq2), pq = (pk1, pq1, pk3, pq3)
  float skr = pk + pq;             // even rows: S^T k, odd rows: S^T q
  const float esum = ab.x * skr;  // odd rows: e^g S^T q
  // S^T k into the odd rows too (rows 1 and 3 take lane 15 of rows 0 and 2; rows 0 and 2
  // keep theirs), in place: written as assembly with `esum` as an input so that the
  // multiply above is issued first and no copy of the sum is needed (the compiler's own
  // form kept the sum alive past the broadcast and copied it every token).  The s_nop
  // gives the two wait states a DPP read needs after a vector-ALU write of its source.
  asm("s_nop 1\n\tv_mov_b32_dpp %0, %0 row_bcast:15 row_mask:0xa bank_mask:0xf"
      : "+v"(skr)
      : "v"(esum));
  const float d = ab.y * fmaf(-ab.x, skr, vv);  // beta (v - e^g S^T k)
  const float om = fmaf(d, kq, esum);           // odd rows: (e^g S + k d^T)^T q
#pragma unroll
  for (int i = 0; i < RPL; ++i) S[i] = fmaf((&kc.x)[i], d, ab.x * S[i]);
  sm.o[buf][tt][m][parity][cl] = om;  // the odd row's 16 lanes hold the same value
}

template <int G>
__device__ __forceinline__ void compute_tile(SeqSmem<G>& sm, int buf, int ntok, float (&S)[RPL],
                                             int m, int r, int cl) {
  // The k and q rows of the next token are read while this one computes, and every
  // per-token scalar is read before the reductions: no LDS latency waits on the chain.
  const float4* kr = reinterpret_cast<const float4*>(&sm.k[buf][0][RPL * r]);
  const float4* qr = reinterpret_cast<const float4*>(&sm.q[buf][0][RPL * r]);
  const int parity = (threadIdx.x >> 4) & 1;  // odd DPP row of the column: the output sum
  float4 kx[2], qx[2];
  kx[0] = kr[0];
  qx[0] = qr[0];
  if (ntok == TB) {
    // a full tile, unrolled: the two register sets alternate and every LDS offset is an
    // immediate, so no moves or address arithmetic sit between the tokens
#pragma unroll
    for (int tt = 0; tt < TB; ++tt)
      token_step<G>(sm, buf, tt, tt + 1 < TB ? tt + 1 : tt, kr, qr, kx[tt & 1], qx[tt & 1],
                    kx[~tt & 1], qx[~tt & 1], S, m, cl, parity);
  } else {
    for (int tt = 0; tt < ntok; ++tt) {
      token_step<G>(sm, buf, tt, min(tt + 1, ntok - 1), kr, qr, kx[0], qx[0], kx[1], qx[1],
                    S, m, cl, parity);
      kx[0] = kx[1];
      qx[0] = qx[1];
    }
  }
}

template <int G>
__global__ __launch_bounds__(seq_threads<G>()) void seq_kernel(SeqArgs a) {
  __shared__ SeqSmem<G> sm;
  const int L = xcd_grouped_block(blockIdx.x, gridDim.x);
  const int kh = L / NCB, cb = L % NCB;
  const int Hk = a.n_k_heads;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int m = w >> 2;                       // value head of the group
  const int cl = (w & 3) * 2 + (lane >> 5);   // column of this lane in the block
  const int r = lane & 31;                    // owns key rows 4r .. 4r+3
  const int j = cb * COLS + cl;
  const int h = kh + m * Hk;

  float S[RPL];
#pragma unroll
  for (int i = 0; i < RPL; ++i) S[i] = a.s_in[(h * kDim + RPL * r + i) * kDim + j];
  // Wait for the state here: left to the compiler, the wait lands inside the token loop,
  // where it also waits for the next tile's staging loads once per tile.
  __builtin_amdgcn_s_waitcnt(0);

  const int ntiles = (a.T + TB - 1) / TB;
  SeqStage st;
  stage_load<G>(st, a, 0, kh, cb, tid);
  stage_store<G>(sm, 0, st, tid);
  __syncthreads();
  // Tile n computes from LDS buffer n & 1 while tile n + 1 is staged into the other; the
  // loop is unrolled over the two buffers so that every LDS address is a per-lane base
  // plus an immediate (a runtime buffer index costs address arithmetic at every token).
  auto tile = [&](auto bc, int n) {
    constexpr int B = decltype(bc)::value;
    const bool more = n + 1 < ntiles;
    if (more) stage_load<G>(st, a, (n + 1) * TB, kh, cb, tid);
    if (n > 0) store_outputs<G>(sm, B ^ 1, a, (n - 1) * TB, kh, cb, tid);
    compute_tile<G>(sm, B, min(TB, a.T - n * TB), S, m, r, cl);
    if (more) stage_store<G>(sm, B ^ 1, st, tid);
    __syncthreads();
  };
  for (int n = 0; n < ntiles; n += 2) {
    tile(std::integral_constant<int, 0>(), n);
    if (n + 1 >= ntiles) break;
    tile(std::integral_constant<int, 1>(), n + 1);
  }
  store_outputs<G>(sm, (ntiles - 1) & 1, a, (ntiles - 1) * TB, kh, cb, tid);

#pragma unroll
  for (int i = 0; i < RPL; ++i) a.s_out[(h * kDim + RPL * r + i) * kDim + j] = S[i];
}

template <int G>
hipError_t launch_g(const SeqArgs& a, hipStream_t stream) {
  void* args[] = {const_cast<SeqArgs*>(&a)};
  return hipLaunchKernel(reinterpret_cast<const void*>(&seq_kernel<G>),
                         dim3(a.n_k_heads * NCB), dim3(seq_threads<G>()), args, 0, stream);
}

}  // namespace

hipError_t launch_seq(const SeqArgs& a, int group, hipStream_t stream) {
  switch (group) {
    case 1: return launch_g<1>(a, stream);
    case 2: return launch_g<2>(a, stream);
    case 3: return launch_g<3>(a, stream);
    case 4: return launch_g<4>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace gdn
