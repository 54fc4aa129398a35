// Sequential gated delta rule for gfx950: one token at a time, the state on chip.
//
// Per value head h and token t ("#413 prefill: DeltaNet recurrence with the three value
// heads of a key head in one thread", sections "What changes" and "Exactness"):
//     kv = e^{g} S^T k,   d = beta (v - kv),   S <- e^{g} S + k d^T,   o = S^T q.
// The output sum is taken from the pre-update state: o = e^{g} (S^T q) + d (k.q), which
// is the same quantity and lets the kv sum and the output sum run side by side.
//
// Work split (designed for wave64 and 256 CUs, not taken from the pages):
//  - one workgroup = one key head x 8 value columns, for all value heads of that key head
//    (the G heads share every staged tile of q/k rows); 16 key heads x 16 column blocks =
//    256 workgroups, one per CU;
//  - a 64-lane wave holds 4 value columns of one value head; the 16 lanes of a column (one
//    DPP row) each own 8 of the 128 key rows (8 floats of state per lane, in VGPRs for the
//    whole sequence); each value head of the key head has 2 waves, so the SIMDs run
//    several waves whose dependency chains interleave;
//  - the kv and output sums over the 128 rows are two chains of four products per lane,
//    then four DPP steps across the 16 lanes of the row, entirely inside the wave: no LDS
//    round trip, no barrier per token;
//  - the inputs of 16 tokens (q/k rows of the key head, the block's v columns, e^{g},
//    beta and k.q) are staged in double-buffered LDS; the next tile's global loads are in
//    flight while the current tile computes; one barrier per 16 tokens.
#include "gdn_common.h"
#include "gdn_kernels.h"

namespace gdn {
namespace {

constexpr int TB = 16;    // tokens per staged tile
constexpr int COLS = 8;   // value columns per workgroup
constexpr int NT = 256;   // threads that stage the q/k rows
constexpr int RPL = 8;    // key rows per lane: 16 lanes per column
template <int G>
constexpr int seq_threads() { return 128 * (G < 2 ? 2 : G); }  // 2 waves per value head
constexpr int NCB = kDim / COLS;  // column blocks per key head

template <int G>
struct SeqSmem {
  float k[2][TB][kDim];
  float q[2][TB][kDim];
  float v[2][TB][G][COLS];
  float2 ab[2][TB][G];  // (e^{g}, beta)
  float kq[2][TB];      // k.q of the key head
  float o[2][TB][G][COLS];
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
          *reinterpret_cast<const float4*>(&sm.o[buf][tt][m][4 * half]);
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

template <int G>
__device__ __forceinline__ void compute_tile(SeqSmem<G>& sm, int buf, int ntok, float (&S)[RPL],
                                             int m, int r, int cl) {
  // The k and q rows of the next token are read while this one computes, and every
  // per-token scalar is read before the reductions: no LDS latency waits on the chain.
  const float4* kr = reinterpret_cast<const float4*>(&sm.k[buf][0][RPL * r]);
  const float4* qr = reinterpret_cast<const float4*>(&sm.q[buf][0][RPL * r]);
  constexpr int ROW4 = kDim / 4;  // float4 per token row
  float4 k0 = kr[0], k1 = kr[1], q0 = qr[0], q1 = qr[1];
  for (int tt = 0; tt < ntok; ++tt) {
    const int tn = min(tt + 1, ntok - 1);  // the last token of the tile re-reads its own
    const float4 kn0 = kr[tn * ROW4], kn1 = kr[tn * ROW4 + 1];
    const float4 qn0 = qr[tn * ROW4], qn1 = qr[tn * ROW4 + 1];
    const float2 ab = sm.ab[buf][tt][m];
    const float vv = sm.v[buf][tt][m][cl];
    const float kq = sm.kq[buf][tt];
    const float kk[RPL] = {k0.x, k0.y, k0.z, k0.w, k1.x, k1.y, k1.z, k1.w};
    const float qq[RPL] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w};
    // two chains of four products each, then the 16 lanes of the column
    float pk = fmaf(S[3], kk[3], fmaf(S[2], kk[2], fmaf(S[1], kk[1], S[0] * kk[0]))) +
               fmaf(S[7], kk[7], fmaf(S[6], kk[6], fmaf(S[5], kk[5], S[4] * kk[4])));
    float pq = fmaf(S[3], qq[3], fmaf(S[2], qq[2], fmaf(S[1], qq[1], S[0] * qq[0]))) +
               fmaf(S[7], qq[7], fmaf(S[6], qq[6], fmaf(S[5], qq[5], S[4] * qq[4])));
    pk = row16_sum(pk);  // S^T k over the 128 rows of this column
    pq = row16_sum(pq);  // S^T q
    const float d = ab.y * fmaf(-ab.x, pk, vv);  // beta (v - e^g S^T k)
    const float om = fmaf(ab.x, pq, d * kq);     // (e^g S + k d^T)^T q
#pragma unroll
    for (int i = 0; i < RPL; ++i) S[i] = fmaf(kk[i], d, ab.x * S[i]);
    if (r == 0) sm.o[buf][tt][m][cl] = om;
    k0 = kn0; k1 = kn1; q0 = qn0; q1 = qn1;
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
  const bool computes = w < 2 * G;             // (G = 1: waves 2 and 3 only stage)
  const int m = computes ? w >> 1 : 0;         // value head of the group
  const int cl = (w & 1) * 4 + (lane >> 4);    // column of this lane in the block
  const int r = lane & 15;                     // owns key rows 8r .. 8r+7
  const int j = cb * COLS + cl;
  const int h = kh + m * Hk;

  float S[RPL];
#pragma unroll
  for (int i = 0; i < RPL; ++i) S[i] = a.s_in[(h * kDim + RPL * r + i) * kDim + j];

  const int ntiles = (a.T + TB - 1) / TB;
  SeqStage st;
  stage_load<G>(st, a, 0, kh, cb, tid);
  stage_store<G>(sm, 0, st, tid);
  __syncthreads();
  for (int n = 0; n < ntiles; ++n) {
    const int buf = n & 1;
    const bool more = n + 1 < ntiles;
    if (more) stage_load<G>(st, a, (n + 1) * TB, kh, cb, tid);
    if (n > 0) store_outputs<G>(sm, buf ^ 1, a, (n - 1) * TB, kh, cb, tid);
    if (computes) compute_tile<G>(sm, buf, min(TB, a.T - n * TB), S, m, r, cl);
    if (more) stage_store<G>(sm, buf ^ 1, st, tid);
    __syncthreads();
  }
  store_outputs<G>(sm, (ntiles - 1) & 1, a, (ntiles - 1) * TB, kh, cb, tid);

  if (computes) {
#pragma unroll
    for (int i = 0; i < RPL; ++i) a.s_out[(h * kDim + RPL * r + i) * kDim + j] = S[i];
  }
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
