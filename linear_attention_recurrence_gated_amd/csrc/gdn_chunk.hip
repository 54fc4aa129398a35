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

// The operators of chunk c for key head kh and its value heads.  Called by every thread
// of a 256-thread workgroup (it contains barriers); ends with a barrier, so one
// workgroup may process several items in a row.
__device__ __forceinline__ void prep_item(const ChunkArgs& a, int c, int kh, PrepSmem& sm) {
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
#pragma unroll
      for (int s4 = 0; s4 < kChunk / 4; ++s4) {  // inclusive running sum, in FP64
        const float4 g4 = *reinterpret_cast<const float4*>(&sm.gs[m][4 * s4]);
        gam_l += 4 * s4 + 0 <= t ? (double)g4.x : 0.0;
        gam_l += 4 * s4 + 1 <= t ? (double)g4.y : 0.0;
        gam_l += 4 * s4 + 2 <= t ? (double)g4.z : 0.0;
        gam_l += 4 * s4 + 3 <= t ? (double)g4.w : 0.0;
      }
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
      // gives T[t][j] = [t == j] - sum_{i < t} A[t][i] T[i][j].  Each row's sum runs in
      // four independent partial sums (i mod 4), and row t+1 of A is read from LDS (as
      // 16-byte broadcasts) before row t is computed, so neither the FMA chain nor the
      // LDS latency serialises the solve.
      const int j = l;
      float Tc[kChunk];
      f32x4 arow[2][kChunk / 4];
#pragma unroll
      for (int q4 = 0; q4 < kChunk / 4; ++q4)
        arow[0][q4] = *reinterpret_cast<const f32x4*>(&sm.A[w][0][4 * q4]);
#pragma unroll
      for (int t = 0; t < kChunk; ++t) {
        const int cb = t & 1;
        if (t + 1 < kChunk) {
#pragma unroll
          for (int q4 = 0; q4 < kChunk / 4; ++q4)
            if (4 * q4 < t + 1)
              arow[cb ^ 1][q4] = *reinterpret_cast<const f32x4*>(&sm.A[w][t + 1][4 * q4]);
        }
        float part[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < t; ++i) part[i & 3] = fmaf(arow[cb][i >> 2][i & 3], Tc[i], part[i & 3]);
        Tc[t] = (t == j ? 1.f : 0.f) - ((part[0] + part[1]) + (part[2] + part[3]));
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
// One workgroup = one value head x 32 value columns: 4 waves, wave (cs, rh) owning value
// columns 16 cs .. 16 cs + 15 of the workgroup and key rows 64 rh .. 64 rh + 63.  Every
// operand a chunk needs (K and Q rows of the key head, the head's WY slot from the
// workspace and the workgroup's V tile) is staged into LDS once per workgroup with
// coalesced 16-byte loads, one chunk ahead, and read from LDS by the waves; only the
// outputs go straight to memory.
constexpr int SC_NT = 256;  // threads per scan workgroup
constexpr int SC_COLS = 32; // value columns per scan workgroup
constexpr int TPAD = 36;    // LDS row stride of T, P and V^T (floats): conflict-free reads

struct ScanSmem {
  float k[2][kChunk][KP];
  float q[2][kChunk][KP];
  float T[2][kChunk][TPAD];        // T diag(beta)
  float P[2][kChunk][TPAD];
  float vt[2][SC_COLS][TPAD];      // V^T: [column of the workgroup][token]
  float eg[2][kChunk], eb[2][kChunk], egl[2][4];
  f32x4 x[2][2][2][4][64];         // exchange: [parity][col slice][row half][tile][lane]
};

// Global loads of one chunk's operands, held in registers until written to LDS.
struct ScanStage {
  f32x4 k[4], q[4];  // K/Q rows: float4 index tid + 256 i of the 32 x 32 float4 tile
  f32x4 slot[3];     // workspace slot: float4 index tid + 256 i (< 544)
  f32x4 v;           // V: token tid / 8, columns 4 (tid % 8) .. +3
};

// One scan workgroup (block index `b` of `nb` scan workgroups).
__device__ __forceinline__ void scan_block(const ChunkArgs& a, int b, int nb, ScanSmem& sm) {
  constexpr int NCB = kDim / SC_COLS;  // column blocks per value head
  constexpr int SLOT_F4 = kSlot / 4;   // 544

  const int Hk = a.n_k_heads, Hv = a.n_v_heads, G = Hv / Hk;
  const int L = xcd_grouped_block(b, nb);
  // logical order: key head, then value head of the group, then column block
  const int kh = L / (G * NCB), m = (L / NCB) % G, cblk = L % NCB;
  const int h = kh + m * Hk;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  const int cs = w >> 1, rh = w & 1;
  const int colw = 16 * cs + (l & 15);      // column inside the workgroup
  const int col = cblk * SC_COLS + colw;    // value column
  const int lr = 4 * (l >> 4);  // row offset of this lane inside a 16-row MFMA tile
  const int nch = (a.n_tok + kChunk - 1) / kChunk;

  // state: tile rt holds rows 64 rh + 16 rt + lr + r, column col
  f32x4 S[4];
#pragma unroll
  for (int rt = 0; rt < 4; ++rt)
#pragma unroll
    for (int r = 0; r < 4; ++r)
      S[rt][r] = a.s_src[((size_t)h * kDim + 64 * rh + 16 * rt + lr + r) * kDim + col];

  // The super-block's tokens, addressed through bounds-checked buffer resources: reads
  // past its last token return 0 (the zero padding of a partial chunk), writes past it are
  // dropped.  Byte offsets stay far below 2^32 (at most 2048 tokens per super-block).
  const buf_rsrc rs_k = make_rsrc(a.k + (size_t)a.t_begin * Hk * kDim, a.n_tok * Hk * kDim * 4);
  const buf_rsrc rs_q = make_rsrc(a.q + (size_t)a.t_begin * Hk * kDim, a.n_tok * Hk * kDim * 4);
  const buf_rsrc rs_v = make_rsrc(a.v + (size_t)a.t_begin * Hv * kDim, a.n_tok * Hv * kDim * 4);
  const buf_rsrc rs_o = make_rsrc(a.o + (size_t)a.t_begin * Hv * kDim, a.n_tok * Hv * kDim * 4);

  ScanStage st;
  // Global loads for chunk c (the workspace slot is clamped to the last chunk, so loads
  // past the end stay inside the workspace; tokens past the end read as 0).  Every thread
  // issues the same loads in every chunk, so the compiler's wait counts stay exact.
  auto stage_load = [&](int c) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int f = tid + SC_NT * i, tt = f >> 5, p = f & 31;
      const int off = (((c * kChunk + tt) * Hk + kh) * kDim + 4 * p) * 4;
      st.k[i] = buf_load4(rs_k, off);
      st.q[i] = buf_load4(rs_q, off);
    }
    const f32x4* slot =
        reinterpret_cast<const f32x4*>(a.ws + ((size_t)min(c, nch - 1) * Hv + h) * kSlot);
#pragma unroll
    for (int i = 0; i < 3; ++i) st.slot[i] = slot[min(tid + SC_NT * i, SLOT_F4 - 1)];
    st.v = buf_load4(rs_v, (((c * kChunk + (tid >> 3)) * Hv + h) * kDim + cblk * SC_COLS +
                            4 * (tid & 7)) * 4);
  };
  auto stage_store = [&](int b) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int f = tid + SC_NT * i, tt = f >> 5, p = f & 31;
      *reinterpret_cast<f32x4*>(&sm.k[b][tt][4 * p]) = st.k[i];
      *reinterpret_cast<f32x4*>(&sm.q[b][tt][4 * p]) = st.q[i];
    }
    // slot float4 f: T rows (f < 256), P rows (f < 512), then e^gamma, e^(last-gamma), e^last
    *reinterpret_cast<f32x4*>(&sm.T[b][tid >> 3][4 * (tid & 7)]) = st.slot[0];
    *reinterpret_cast<f32x4*>(&sm.P[b][tid >> 3][4 * (tid & 7)]) = st.slot[1];
    if (tid < 8) *reinterpret_cast<f32x4*>(&sm.eg[b][4 * tid]) = st.slot[2];
    else if (tid < 16) *reinterpret_cast<f32x4*>(&sm.eb[b][4 * (tid - 8)]) = st.slot[2];
    else if (tid == 16) *reinterpret_cast<f32x4*>(&sm.egl[b][0]) = st.slot[2];
    const int vt_tok = tid >> 3, vt_col = 4 * (tid & 7);
#pragma unroll
    for (int i = 0; i < 4; ++i) sm.vt[b][vt_col + i][vt_tok] = st.v[i];
  };

  auto chunk_step = [&](int c) {
    const int buf = c & 1;
    // (a) operands of this chunk from LDS (written before the previous chunk's barrier),
    //     then partial K S0 and Q S0 over this wave's 64 rows.
    f32x4 ka[4][2], qa[4][2];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        const int row = 64 * rh + 16 * rt + lr;
        ka[rt][tt] = *reinterpret_cast<const f32x4*>(&sm.k[buf][16 * tt + (l & 15)][row]);
        qa[rt][tt] = *reinterpret_cast<const f32x4*>(&sm.q[buf][16 * tt + (l & 15)][row]);
      }
    float kt[4][2][4];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          kt[rt][tt][r] = sm.k[buf][16 * tt + lr + r][64 * rh + 16 * rt + (l & 15)];
    const int ar = l & 15;
    const f32x4 T00 = *reinterpret_cast<const f32x4*>(&sm.T[buf][ar][lr]);
    const f32x4 T10 = *reinterpret_cast<const f32x4*>(&sm.T[buf][16 + ar][lr]);
    const f32x4 T11 = *reinterpret_cast<const f32x4*>(&sm.T[buf][16 + ar][16 + lr]);
    const f32x4 Pa = *reinterpret_cast<const f32x4*>(&sm.P[buf][16 * rh + ar][lr]);
    const f32x4 Pb = *reinterpret_cast<const f32x4*>(&sm.P[buf][16 + ar][16 + lr]);
    f32x4 eg[2], eb[2], vv[2];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      eg[tt] = *reinterpret_cast<const f32x4*>(&sm.eg[buf][16 * tt + lr]);
      eb[tt] = *reinterpret_cast<const f32x4*>(&sm.eb[buf][16 * tt + lr]);
      vv[tt] = *reinterpret_cast<const f32x4*>(&sm.vt[buf][colw][16 * tt + lr]);
    }
    const float egl = sm.egl[buf][0];

    f32x4 P4[4];  // partial W0, W1, QS0, QS1
#pragma unroll
    for (int i = 0; i < 4; ++i) P4[i] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
          P4[tt] = mfma16x16x4(ka[rt][tt][r], S[rt][r], P4[tt]);
          P4[2 + tt] = mfma16x16x4(qa[rt][tt][r], S[rt][r], P4[2 + tt]);
        }

    // (a') stage chunk c+1 into the other LDS buffer (its last reads were in chunk c-1's
    //      phase (a), before that chunk's barrier), then load chunk c+2.
    stage_store(buf ^ 1);
    stage_load(c + 2);

    // (b) exchange partial sums with the other row half of the same columns; both halves
    //     add the two halves in the same order, so they hold identical sums.
    const int par = c & 1;
    sm.x[par][cs][rh][0][l] = P4[0];
    sm.x[par][cs][rh][1][l] = P4[1];
    sm.x[par][cs][rh][2][l] = rh ? P4[2] : P4[3];  // the other half's output tile
    __syncthreads();
    f32x4 W[2];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) W[tt] = sm.x[par][cs][0][tt][l] + sm.x[par][cs][1][tt][l];
    const f32x4 QSo = sm.x[par][cs][1 - rh][2][l];
    const f32x4 QSf = rh ? (QSo + P4[3]) : (P4[2] + QSo);

    // (c) U = V - e^{gamma} (K S0), C layout: token 16 tt + lr + r, column col.
    f32x4 U[2];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int r = 0; r < 4; ++r) U[tt][r] = fmaf(-eg[tt][r], W[tt][r], vv[tt][r]);

    // (d) D = T diag(beta) U; T is lower triangular, so tile (0,1) is zero.
    f32x4 D[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      D[0] = mfma16x16x4(T00[r], U[0][r], D[0]);
      D[1] = mfma16x16x4(T10[r], U[0][r], D[1]);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) D[1] = mfma16x16x4(T11[r], U[1][r], D[1]);

    // (e) outputs of token tile rh: O = e^{gamma} Q S0 + P D (P lower triangular).
    f32x4 O = (rh ? eg[1] : eg[0]) * QSf;
#pragma unroll
    for (int r = 0; r < 4; ++r) O = mfma16x16x4(Pa[r], D[0][r], O);
    if (rh == 1) {
#pragma unroll
      for (int r = 0; r < 4; ++r) O = mfma16x16x4(Pb[r], D[1][r], O);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {  // dropped by the buffer past the last token
      const int tk = c * kChunk + 16 * rh + lr + r;
      buf_store(rs_o, ((tk * Hv + h) * kDim + col) * 4, O[r]);
    }

    // (f, g) S' = e^{gamma_last} S0 + K^T diag(e^{gamma_last - gamma}) D.
    f32x4 Dh[2];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) Dh[tt] = eb[tt] * D[tt];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) S[rt] = egl * S[rt];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) S[rt] = mfma16x16x4(kt[rt][tt][r], Dh[tt][r], S[rt]);
  };

  stage_load(0);
  stage_store(0);
  stage_load(1);
  __syncthreads();
  for (int c = 0; c < nch; ++c) chunk_step(c);

#pragma unroll
  for (int rt = 0; rt < 4; ++rt)
#pragma unroll
    for (int r = 0; r < 4; ++r)
      a.s_dst[((size_t)h * kDim + 64 * rh + 16 * rt + lr + r) * kDim + col] = S[rt][r];
}

// Prep alone: one workgroup per (chunk, key head) of a super-block.
__global__ __launch_bounds__(PREP_NT, 2) void chunk_prep_kernel(ChunkArgs a) {
  __shared__ PrepSmem sm;
  prep_item(a, blockIdx.x, blockIdx.y, sm);
}

// Scan of super-block n fused with the prep of super-block n+1: workgroups
// [0, n_scan) scan (they are dispatched first and take one CU each), the rest loop over
// the (chunk, key head) items of the next super-block on the CUs the scan leaves idle.
// The two roles touch disjoint halves of the workspace, and the next launch reads what
// this one's prep wrote, so the roles never wait for each other.
struct FusedArgs {
  ChunkArgs scan;
  ChunkArgs prep;
  int n_scan;  // scan workgroups
  int has_prep;
};

union FusedSmem {
  ScanSmem scan;
  PrepSmem prep;
};

__global__ __launch_bounds__(SC_NT) void chunk_fused_kernel(FusedArgs f) {
  static_assert(SC_NT == PREP_NT, "both roles run with the same workgroup size");
  __shared__ FusedSmem sm;
  const int b = blockIdx.x;
  if (b < f.n_scan) {
    scan_block(f.scan, b, f.n_scan, sm.scan);
  } else if (f.has_prep) {
    const int Hk = f.prep.n_k_heads;
    const int items = ((f.prep.n_tok + kChunk - 1) / kChunk) * Hk;
    const int n_prep = gridDim.x - f.n_scan;
    for (int it = b - f.n_scan; it < items; it += n_prep) prep_item(f.prep, it / Hk, it % Hk, sm.prep);
  }
}

}  // namespace

hipError_t launch_chunk_prep(const ChunkArgs& a, hipStream_t stream) {
  void* args[] = {const_cast<ChunkArgs*>(&a)};
  const int nch = (a.n_tok + kChunk - 1) / kChunk;
  return hipLaunchKernel(reinterpret_cast<const void*>(&chunk_prep_kernel),
                         dim3(nch, a.n_k_heads), dim3(PREP_NT), args, 0, stream);
}

hipError_t launch_chunk_scan_fused(const ChunkArgs& scan, const ChunkArgs* prep_next,
                                   hipStream_t stream) {
  FusedArgs f;
  f.scan = scan;
  f.prep = prep_next ? *prep_next : scan;
  f.n_scan = scan.n_v_heads * (kDim / SC_COLS);
  f.has_prep = prep_next != nullptr;
  // the prep workgroups fill the CUs the scan leaves free (at least 32 of them)
  int n_prep = 0;
  if (prep_next) {
    n_prep = kNumCUs - f.n_scan;
    if (n_prep < 32) n_prep = 32;
  }
  void* args[] = {&f};
  return hipLaunchKernel(reinterpret_cast<const void*>(&chunk_fused_kernel),
                         dim3(f.n_scan + n_prep), dim3(SC_NT), args, 0, stream);
}

}  // namespace gdn
