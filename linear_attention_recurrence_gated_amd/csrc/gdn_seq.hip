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
//  - a 64-lane wave holds 2 value columns of one value head; the 32 lanes of a column each
//    own 4 of the 128 key rows (4 floats of state per lane, in VGPRs for the whole
//    sequence); the G value heads of the key head are G groups of 4 waves, so every SIMD
//    runs G waves whose dependency chains interleave;
//  - the kv and output sums over the 128 rows are reduced across the 32 lanes with four
//    DPP steps and one ds_swizzle (lane ^ 16), entirely inside the wave: no LDS array and
//    no barrier per token;
//  - the inputs of 16 tokens (q/k rows of the key head, the block's v columns, e^{g},
//    beta and k.q) are staged in double-buffered LDS; the next tile's global loads are in
//    flight while the current tile computes; one barrier per 16 tokens.
#include "gdn_common.h"
#include "gdn_kernels.h"

namespace gdn {
namespace {

constexpr int TB = 16;    // tokens per staged tile
constexpr int COLS = 8;   // value columns per workgroup
constexpr int NT = 256;   // threads per value head (4 waves); a workgroup has G NT
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

template <int G>
__device__ __forceinline__ void compute_tile(SeqSmem<G>& sm, int buf, int ntok, float (&S)[4],
                                             int m, int r, int cl) {
  // The k and q rows of the next token are read while this one computes, and every
  // per-token scalar is read before the reductions: no LDS latency waits on the chain.
  float4 kk = *reinterpret_cast<const float4*>(&sm.k[buf][0][4 * r]);
  float4 qq = *reinterpret_cast<const float4*>(&sm.q[buf][0][4 * r]);
  for (int tt = 0; tt < ntok; ++tt) {
    const int tn = min(tt + 1, ntok - 1);  // the last token of the tile re-reads its own
    const float4 kn = *reinterpret_cast<const float4*>(&sm.k[buf][tn][4 * r]);
    const float4 qn = *reinterpret_cast<const float4*>(&sm.q[buf][tn][4 * r]);
    const float2 ab = sm.ab[buf][tt][m];
    const float vv = sm.v[buf][tt][m][cl];
    const float kq = sm.kq[buf][tt];
    float pk = fmaf(S[3], kk.w, fmaf(S[2], kk.z, fmaf(S[1], kk.y, S[0] * kk.x)));
    float pq = fmaf(S[3], qq.w, fmaf(S[2], qq.z, fmaf(S[1], qq.y, S[0] * qq.x)));
    pk = half_wave_sum(pk);  // S^T k over the 128 rows of this column
    pq = half_wave_sum(pq);  // S^T q
    const float d = ab.y * fmaf(-ab.x, pk, vv);  // beta (v - e^g S^T k)
    const float om = fmaf(ab.x, pq, d * kq);     // (e^g S + k d^T)^T q
    S[0] = fmaf(kk.x, d, ab.x * S[0]);
    S[1] = fmaf(kk.y, d, ab.x * S[1]);
    S[2] = fmaf(kk.z, d, ab.x * S[2]);
    S[3] = fmaf(kk.w, d, ab.x * S[3]);
    if (r == 0) sm.o[buf][tt][m][cl] = om;
    kk = kn;
    qq = qn;
  }
}

template <int G>
__global__ __launch_bounds__(NT * G) void seq_kernel(SeqArgs a) {
  __shared__ SeqSmem<G> sm;
  const int L = xcd_grouped_block(blockIdx.x, gridDim.x);
  const int kh = L / NCB, cb = L % NCB;
  const int Hk = a.n_k_heads;
  const int tid = threadIdx.x, lane = tid & 63;
  const int m = __builtin_amdgcn_readfirstlane(tid / NT);  // value head of the group
  const int cl = ((tid % NT) >> 6) * 2 + (lane >> 5);    // column of this lane in the block
  const int r = lane & 31;                                // owns key rows 4r .. 4r+3
  const int j = cb * COLS + cl;
  const int h = kh + m * Hk;

  float S[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) S[i] = a.s_in[(h * kDim + 4 * r + i) * kDim + j];

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
    compute_tile<G>(sm, buf, min(TB, a.T - n * TB), S, m, r, cl);
    if (more) stage_store<G>(sm, buf ^ 1, st, tid);
    __syncthreads();
  }
  store_outputs<G>(sm, (ntiles - 1) & 1, a, (ntiles - 1) * TB, kh, cb, tid);

#pragma unroll
  for (int i = 0; i < 4; ++i) a.s_out[(h * kDim + 4 * r + i) * kDim + j] = S[i];
}

template <int G>
hipError_t launch_g(const SeqArgs& a, hipStream_t stream) {
  void* args[] = {const_cast<SeqArgs*>(&a)};
  return hipLaunchKernel(reinterpret_cast<const void*>(&seq_kernel<G>),
                         dim3(a.n_k_heads * NCB), dim3(NT * G), args, 0, stream);
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
