// Chunked (WY-form) gated delta rule for gfx950: a prep kernel that is parallel over the
// chunks of a 2048-token super-block, and a scan kernel that walks those chunks carrying
// the state on chip.
//
// Per chunk of 32 tokens and value head ("#1372 DeltaNet recurrence:
// STRATA_GDN_CHUNKED=1", section "What it does"), with gamma_t the inclusive running sum
// of the log-decay g inside the chunk and S0 the state before the chunk:
//     A[t][i] = beta_t e^{gamma_t - gamma_i} k_t.k_i  (i < t),     T = (I + A)^-1
//     D  = T diag(beta) (V - diag(e^{gamma}) K S0)
//     O  = diag(e^{gamma}) Q S0 + P D,   P[t][i] = e^{gamma_t - gamma_i} q_t.k_i  (i <= t)
//     S' = e^{gamma_last} S0 + K^T diag(e^{gamma_last - gamma}) D
// Every exponent is <= 0 (the gates are negative), so nothing overflows.
//
// gfx950 design (not the pages' kernels):
//  - prep: one workgroup per (chunk, key head).  The Gram products K K^T and Q K^T run on
//    the FP32 matrix cores (v_mfma_f32_16x16x4_f32); gamma is summed in FP64 so that the
//    decay differences keep full FP32 accuracy; T comes from forward substitution with one
//    lane per column.  It writes T diag(beta), P and the decay vectors of the key head's
//    value heads into the caller's workspace.
//  - scan: one workgroup per (value head, 16*CSB value columns), 2*CSB waves.  Each wave
//    owns 64 key rows x 16 value columns of the state as four MFMA accumulator tiles that
//    stay in VGPRs for the whole super-block.  K S0 and Q S0 are accumulated over the
//    wave's 64 rows on the matrix cores (the state registers are the B operand as they
//    are), the two row halves exchange partial sums through LDS (one barrier per chunk),
//    then D = T U, O = e^{gamma} Q S0 + P D and the rank-32 state update K^T D run as
//    further 16x16x4 MFMAs.  K and Q of the next chunk are staged through double-buffered
//    LDS while the current chunk computes.
#include "gdn_common.h"
#include "gdn_kernels.h"

namespace gdn {
namespace {

constexpr int KP = 132;  // LDS row stride (floats) of a staged 32 x 128 K or Q chunk

// ---------------------------------------------------------------------------------------
// prep
// ---------------------------------------------------------------------------------------
constexpr int PREP_NT = 256;

struct PrepSmem {
  float k[kChunk][KP];
  float q[kChunk][KP];
  float gram[2][kChunk][kChunk + 1];  // [0] = K K^T, [1] = Q K^T
  float gs[kMaxGroup][kChunk];
  float bs[kMaxGroup][kChunk];
  double gam[4][kChunk];
  float A[4][kChunk][kChunk];
};

__global__ __launch_bounds__(PREP_NT) void chunk_prep_kernel(ChunkArgs a) {
  __shared__ PrepSmem sm;
  const int c = blockIdx.x, kh = blockIdx.y;
  const int Hk = a.n_k_heads, Hv = a.n_v_heads, G = Hv / Hk;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  const int c0 = c * kChunk;  // first token of the chunk, relative to the super-block

  // 1. K, Q rows of the chunk (zero past the end), g and beta of the value heads.
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const int f = tid + PREP_NT * m, tt = f >> 5, p = f & 31;
    float4 kv = make_float4(0.f, 0.f, 0.f, 0.f), qv = kv;
    if (c0 + tt < a.n_tok) {
      const int off = ((a.t_begin + c0 + tt) * Hk + kh) * kDim + 4 * p;
      kv = *reinterpret_cast<const float4*>(a.k + off);
      qv = *reinterpret_cast<const float4*>(a.q + off);
    }
    *reinterpret_cast<float4*>(&sm.k[tt][4 * p]) = kv;
    *reinterpret_cast<float4*>(&sm.q[tt][4 * p]) = qv;
  }
  if (tid < kChunk * G) {
    const int m = tid >> 5, tt = tid & 31;
    float gv = 0.f, bv = 0.f;
    if (c0 + tt < a.n_tok) {
      const int off = (a.t_begin + c0 + tt) * Hv + kh + m * Hk;
      gv = a.g[off];
      bv = a.beta[off];
    }
    sm.gs[m][tt] = gv;
    sm.bs[m][tt] = bv;
  }
  __syncthreads();

  // 2. Gram tiles on the matrix cores.  Needed: the lower-triangular 16x16 tiles
  //    (0,0), (1,0), (1,1) of K K^T and of Q K^T; wave w takes tiles w and w + 4.
  for (int tile = w; tile < 6; tile += 4) {
    const int mat = tile / 3, sub = tile % 3;
    const int ti = sub == 0 ? 0 : 1, tj = sub == 2 ? 1 : 0;
    const float* X = mat == 0 ? &sm.k[0][0] : &sm.q[0][0];
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < kDim / 16; ++s) {
      const int col = 16 * s + 4 * (l >> 4);
      const f32x4 av = *reinterpret_cast<const f32x4*>(X + (16 * ti + (l & 15)) * KP + col);
      const f32x4 bv = *reinterpret_cast<const f32x4*>(&sm.k[16 * tj + (l & 15)][col]);
#pragma unroll
      for (int r = 0; r < 4; ++r) acc = mfma16x16x4(av[r], bv[r], acc);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r)
      sm.gram[mat][16 * ti + 4 * (l >> 4) + r][16 * tj + (l & 15)] = acc[r];
  }
  __syncthreads();

  // 3. Per value head (wave w handles head m = mb + w).
  for (int mb = 0; mb < G; mb += 4) {
    const int m = mb + w;
    const bool active = m < G;
    const int h = kh + m * Hk;
    float* slot = a.ws + ((size_t)c * Hv + h) * kSlot;
    double gam_l = 0.0;
    if (active) {
      const int t = l & 31;
      for (int s = 0; s < kChunk; ++s)
        if (s <= t) gam_l += (double)sm.gs[m][s];  // inclusive running sum, in FP64
      if (l < kChunk) sm.gam[w][t] = gam_l;
    }
    __syncthreads();
    if (active) {
      const int i = l & 31;
      const double gi = sm.gam[w][i];
#pragma unroll 4
      for (int s = 0; s < kChunk / 2; ++s) {
        const int t = (l >> 5) + 2 * s;
        const float dec = i <= t ? expf((float)(sm.gam[w][t] - gi)) : 0.f;
        // the upper Gram tile (0,1) is never formed: select, never multiply, past the diagonal
        sm.A[w][t][i] = i < t ? sm.bs[m][t] * dec * sm.gram[0][t][i] : 0.f;
        slot[kSlotP + t * kChunk + i] = i <= t ? dec * sm.gram[1][t][i] : 0.f;
      }
      if (l < kChunk) {
        const double glast = sm.gam[w][kChunk - 1];
        slot[kSlotEg + l] = expf((float)gam_l);
        slot[kSlotEb + l] = expf((float)(glast - gam_l));
        if (l == 0) slot[kSlotEgl] = expf((float)glast);
      }
    }
    __syncthreads();
    if (active && l < kChunk) {
      // Column j = l of T = (I + A)^-1 by forward substitution: row t of (I + A) T = I
      // gives T[t][j] = [t == j] - sum_{i < t} A[t][i] T[i][j].
      const int j = l;
      float Tc[kChunk];
#pragma unroll
      for (int t = 0; t < kChunk; ++t) {
        float x = t == j ? 1.f : 0.f;
#pragma unroll
        for (int i = 0; i < t; ++i) x = fmaf(-sm.A[w][t][i], Tc[i], x);
        Tc[t] = x;
      }
      const float bj = sm.bs[m][j];
#pragma unroll
      for (int t = 0; t < kChunk; ++t) slot[kSlotT + t * kChunk + j] = Tc[t] * bj;
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------------------
// scan
// ---------------------------------------------------------------------------------------
template <int CSB>
struct ScanSmem {
  float k[2][kChunk][KP];
  float q[2][kChunk][KP];
  f32x4 x[2][CSB][2][3][64];  // partial-sum exchange: [parity][col slice][row half][tile][lane]
};

// Per-wave operands of one chunk, prefetched from global memory one chunk ahead.
struct ScanOps {
  float v[2][4];  // V[16tt + 4(l/16) + r][col]
  f32x4 T00, T10, T11;  // T diag(beta) blocks, MFMA A-operand order
  f32x4 Pa, Pb;         // P blocks (rh,0) and (1,1) (Pb used by rh = 1 only)
  f32x4 eg[2], eb[2];
  float egl;
};

template <int CSB>
__global__ __launch_bounds__(128 * CSB) void chunk_scan_kernel(ChunkArgs a) {
  constexpr int NT = 128 * CSB;
  constexpr int NCB = kDim / (16 * CSB);       // column blocks per value head
  constexpr int KQ_F4 = 2 * kChunk * 32 / NT;  // float4 of K and Q staged per thread
  __shared__ ScanSmem<CSB> sm;

  const int Hk = a.n_k_heads, Hv = a.n_v_heads, G = Hv / Hk;
  const int L = xcd_grouped_block(blockIdx.x, gridDim.x);
  // logical order: key head, then value head of the group, then column block
  const int kh = L / (G * NCB), m = (L / NCB) % G, cblk = L % NCB;
  const int h = kh + m * Hk;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  const int cs = w >> 1, rh = w & 1;
  const int col = cblk * 16 * CSB + 16 * cs + (l & 15);
  const int lr = 4 * (l >> 4);  // row offset of this lane inside a 16-row MFMA tile
  const int nch = (a.n_tok + kChunk - 1) / kChunk;

  // state: tile rt holds rows 64 rh + 16 rt + lr + r, column col
  f32x4 S[4];
#pragma unroll
  for (int rt = 0; rt < 4; ++rt)
#pragma unroll
    for (int r = 0; r < 4; ++r)
      S[rt][r] = a.s_src[((size_t)h * kDim + 64 * rh + 16 * rt + lr + r) * kDim + col];

  auto load_ops = [&](ScanOps& op, int c) {
    const float* slot = a.ws + ((size_t)c * Hv + h) * kSlot;
    const int c0 = c * kChunk;
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int tk = c0 + 16 * tt + lr + r;
        op.v[tt][r] =
            tk < a.n_tok ? a.v[((size_t)(a.t_begin + tk) * Hv + h) * kDim + col] : 0.f;
      }
    const int arow = (l & 15) * kChunk + lr;
    op.T00 = *reinterpret_cast<const f32x4*>(slot + kSlotT + arow);
    op.T10 = *reinterpret_cast<const f32x4*>(slot + kSlotT + 16 * kChunk + arow);
    op.T11 = *reinterpret_cast<const f32x4*>(slot + kSlotT + 16 * kChunk + 16 + arow);
    op.Pa = *reinterpret_cast<const f32x4*>(slot + kSlotP + 16 * rh * kChunk + arow);
    op.Pb = *reinterpret_cast<const f32x4*>(slot + kSlotP + 16 * kChunk + 16 + arow);
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      op.eg[tt] = *reinterpret_cast<const f32x4*>(slot + kSlotEg + 16 * tt + lr);
      op.eb[tt] = *reinterpret_cast<const f32x4*>(slot + kSlotEb + 16 * tt + lr);
    }
    op.egl = slot[kSlotEgl];
  };

  float4 kst[KQ_F4 / 2], qst[KQ_F4 / 2];
  auto stage_load = [&](int c) {
#pragma unroll
    for (int i = 0; i < KQ_F4 / 2; ++i) {
      const int f = tid + NT * i, tt = f >> 5, p = f & 31;
      const int tk = c * kChunk + tt;
      float4 kv = make_float4(0.f, 0.f, 0.f, 0.f), qv = kv;
      if (tk < a.n_tok) {
        const size_t off = ((size_t)(a.t_begin + tk) * Hk + kh) * kDim + 4 * p;
        kv = *reinterpret_cast<const float4*>(a.k + off);
        qv = *reinterpret_cast<const float4*>(a.q + off);
      }
      kst[i] = kv;
      qst[i] = qv;
    }
  };
  auto stage_store = [&](int buf) {
#pragma unroll
    for (int i = 0; i < KQ_F4 / 2; ++i) {
      const int f = tid + NT * i, tt = f >> 5, p = f & 31;
      *reinterpret_cast<float4*>(&sm.k[buf][tt][4 * p]) = kst[i];
      *reinterpret_cast<float4*>(&sm.q[buf][tt][4 * p]) = qst[i];
    }
  };

  ScanOps cur, nxt;
  stage_load(0);
  stage_store(0);
  if (nch > 1) stage_load(1);
  load_ops(cur, 0);
  __syncthreads();

  for (int c = 0; c < nch; ++c) {
    const int buf = c & 1, par = c & 1;
    // (a) partial K S0 and Q S0 over this wave's 64 rows; K^T operands for the update.
    f32x4 W[2], QS[2];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      W[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
      QS[tt] = W[tt];
    }
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
      const int row = 64 * rh + 16 * rt + lr;
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        const f32x4 ka = *reinterpret_cast<const f32x4*>(&sm.k[buf][16 * tt + (l & 15)][row]);
        const f32x4 qa = *reinterpret_cast<const f32x4*>(&sm.q[buf][16 * tt + (l & 15)][row]);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          W[tt] = mfma16x16x4(ka[r], S[rt][r], W[tt]);
          QS[tt] = mfma16x16x4(qa[r], S[rt][r], QS[tt]);
        }
      }
    }
    float kt[4][2][4];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          kt[rt][tt][r] = sm.k[buf][16 * tt + lr + r][64 * rh + 16 * rt + (l & 15)];

    // (a') stage the next chunk's K/Q into the other LDS buffer (last read in chunk c-1,
    //      before that chunk's barrier), then start loading the one after it.
    if (c + 1 < nch) {
      stage_store(buf ^ 1);
      if (c + 2 < nch) stage_load(c + 2);
      load_ops(nxt, c + 1);
    }

    // (b) exchange partial sums with the other row half of the same columns.
    sm.x[par][cs][rh][0][l] = W[0];
    sm.x[par][cs][rh][1][l] = W[1];
    // (selects, not QS[rh]: a runtime index would push the array out of registers)
    sm.x[par][cs][rh][2][l] = rh ? QS[0] : QS[1];
    __syncthreads();
    W[0] += sm.x[par][cs][1 - rh][0][l];
    W[1] += sm.x[par][cs][1 - rh][1][l];
    const f32x4 QSf = (rh ? QS[1] : QS[0]) + sm.x[par][cs][1 - rh][2][l];

    // (c) U = V - e^{gamma} (K S0), C layout: token 16 tt + lr + r, column col.
    f32x4 U[2];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int r = 0; r < 4; ++r) U[tt][r] = fmaf(-cur.eg[tt][r], W[tt][r], cur.v[tt][r]);

    // (d) D = T diag(beta) U; T is lower triangular, so tile (0,1) is zero.
    f32x4 D[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int r = 0; r < 4; ++r) D[0] = mfma16x16x4(cur.T00[r], U[0][r], D[0]);
#pragma unroll
    for (int r = 0; r < 4; ++r) D[1] = mfma16x16x4(cur.T10[r], U[0][r], D[1]);
#pragma unroll
    for (int r = 0; r < 4; ++r) D[1] = mfma16x16x4(cur.T11[r], U[1][r], D[1]);

    // (e) outputs of token tile rh: O = e^{gamma} Q S0 + P D (P lower triangular).
    f32x4 O = (rh ? cur.eg[1] : cur.eg[0]) * QSf;
#pragma unroll
    for (int r = 0; r < 4; ++r) O = mfma16x16x4(cur.Pa[r], D[0][r], O);
    if (rh == 1) {
#pragma unroll
      for (int r = 0; r < 4; ++r) O = mfma16x16x4(cur.Pb[r], D[1][r], O);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int tk = c * kChunk + 16 * rh + lr + r;
      if (tk < a.n_tok) a.o[((size_t)(a.t_begin + tk) * Hv + h) * kDim + col] = O[r];
    }

    // (f, g) S' = e^{gamma_last} S0 + K^T diag(e^{gamma_last - gamma}) D.
    f32x4 Dh[2];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) Dh[tt] = cur.eb[tt] * D[tt];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
      S[rt] = cur.egl * S[rt];
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int r = 0; r < 4; ++r) S[rt] = mfma16x16x4(kt[rt][tt][r], Dh[tt][r], S[rt]);
    }
    cur = nxt;
  }

#pragma unroll
  for (int rt = 0; rt < 4; ++rt)
#pragma unroll
    for (int r = 0; r < 4; ++r)
      a.s_dst[((size_t)h * kDim + 64 * rh + 16 * rt + lr + r) * kDim + col] = S[rt][r];
}

constexpr int kScanCSB = 2;

}  // namespace

hipError_t launch_chunk_prep(const ChunkArgs& a, hipStream_t stream) {
  void* args[] = {const_cast<ChunkArgs*>(&a)};
  const int nch = (a.n_tok + kChunk - 1) / kChunk;
  return hipLaunchKernel(reinterpret_cast<const void*>(&chunk_prep_kernel),
                         dim3(nch, a.n_k_heads), dim3(PREP_NT), args, 0, stream);
}

hipError_t launch_chunk_scan(const ChunkArgs& a, hipStream_t stream) {
  void* args[] = {const_cast<ChunkArgs*>(&a)};
  const int nblocks = a.n_v_heads * (kDim / (16 * kScanCSB));
  return hipLaunchKernel(reinterpret_cast<const void*>(&chunk_scan_kernel<kScanCSB>),
                         dim3(nblocks), dim3(128 * kScanCSB), args, 0, stream);
}

}  // namespace gdn
