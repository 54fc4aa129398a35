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
//  - scan: one workgroup per (value head, 32 value columns): four compute waves, each
//    owning 64 key rows x 16 value columns of the state as four MFMA accumulator tiles that
//    stay in VGPRs for the whole super-block, a producer wave that copies every chunk's
//    operands into a three-buffer LDS ring with direct loads, and three waves that run the
//    output norm of the previous super-block.  Per chunk, K S0 and Q S0 are accumulated
//    over each wave's 64 rows on the matrix cores (the state registers are the B operand as
//    they are), the two row halves exchange partial sums through LDS at one barrier, then
//    D = T U, O = e^{gamma} Q S0 + P D and the rank-32 state update K^T D run as further
//    16x16x4 MFMAs.
//  - the prep of super-block n+1 runs on the CUs the scan of n leaves free, in the same
//    launch.
//  - results that the launch does not read back (o, y, the final state) are stored
//    non-temporally (measured: 2.226 against 2.243 ms per 32768-token layer).
#include <cstddef>
#include <type_traits>

#include "gdn_common.h"
#include "gdn_kernels.h"

namespace gdn {
namespace {

// ---------------------------------------------------------------------------------------
// prep
// ---------------------------------------------------------------------------------------
constexpr int PREP_NT = 256;

struct PrepSmem {
  float gram[2][kChunk][kChunk + 1];  // [0] = K K^T, [1] = Q K^T
  float gs[kMaxGroup][kChunk];
  float bs[kMaxGroup][kChunk];
  double gam[4][kChunk];
  float A[4][kChunk][kChunk];
};

// The operators of chunk c for key head kh and its value heads.  Called by every thread
// of a group of 256 threads (thread `tid` of the group; it contains workgroup barriers,
// which every group of the workgroup reaches the same number of times per item); ends with
// a barrier, so a group may process several items in a row.
__device__ __forceinline__ void prep_item(const ChunkArgs& a, int c, int kh, PrepSmem& sm, int tid) {
  const int Hk = a.n_k_heads, Hv = a.n_v_heads, G = Hv / Hk;
  const int w = tid >> 6, l = tid & 63;
  const int c0 = c * kChunk;  // first token of the chunk, relative to the super-block

  // 1. g and beta of the value heads (zero past the end).
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
  //    (0,0), (1,0), (1,1) of K K^T and of Q K^T.  The waves split the keys: wave w forms
  //    all six tiles over keys 32 w .. 32 w + 31, from the K and Q rows of the chunk loaded
  //    once, straight from global memory into registers (lane: row l % 16, four keys
  //    4 (l / 16) of each group of 16), through descriptors whose range ends with the
  //    call's last token, so rows past it read as 0.  One round trip to memory per wave;
  //    the four partial tiles are then added in a fixed order, (w0 + w2) + (w1 + w3),
  //    through sm.A, which step 3 only fills afterwards.
  const int nv = min(kChunk, a.n_tok - c0);  // tokens of the chunk (>= 1)
  const size_t row0 = ((size_t)(a.t_begin + c0) * Hk + kh) * kDim;
  const uint32_t rbytes = (uint32_t)(((nv - 1) * Hk + 1) * kDim * 4);
  const buf_rsrc rk = make_rsrc(a.k + row0, rbytes), rq = make_rsrc(a.q + row0, rbytes);
  {
    f32x4 kr[2][2], qr[2][2];  // [row tile][group of 16 keys]
#pragma unroll
    for (int ti = 0; ti < 2; ++ti)
#pragma unroll
      for (int sg = 0; sg < 2; ++sg) {
        const uint32_t off = (uint32_t)((16 * ti + (l & 15)) * Hk * kDim * 4) +
                             16 * (l >> 4) + 64 * (2 * w + sg);
        kr[ti][sg] = buf_load4(rk, off);
        qr[ti][sg] = buf_load4(rq, off);
      }
    f32x4 acc[6];  // K K^T (0,0), (1,0), (1,1), then Q K^T (0,0), (1,0), (1,1)
#pragma unroll
    for (int t = 0; t < 6; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int sg = 0; sg < 2; ++sg)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        acc[0] = mfma16x16x4(kr[0][sg][r], kr[0][sg][r], acc[0]);
        acc[1] = mfma16x16x4(kr[1][sg][r], kr[0][sg][r], acc[1]);
        acc[2] = mfma16x16x4(kr[1][sg][r], kr[1][sg][r], acc[2]);
        acc[3] = mfma16x16x4(qr[0][sg][r], kr[0][sg][r], acc[3]);
        acc[4] = mfma16x16x4(qr[1][sg][r], kr[0][sg][r], acc[4]);
        acc[5] = mfma16x16x4(qr[1][sg][r], kr[1][sg][r], acc[5]);
      }
    f32x4* const part = reinterpret_cast<f32x4*>(&sm.A[0][0][0]);  // [2][6][64]
    if (w >= 2) {
#pragma unroll
      for (int t = 0; t < 6; ++t) part[((w - 2) * 6 + t) * 64 + l] = acc[t];
    }
    __syncthreads();
    if (w < 2) {
#pragma unroll
      for (int t = 0; t < 6; ++t) acc[t] += part[(w * 6 + t) * 64 + l];
      if (w == 1) {
#pragma unroll
        for (int t = 0; t < 6; ++t) part[(6 + t) * 64 + l] = acc[t];
      }
    }
    __syncthreads();
    if (w == 0) {
#pragma unroll
      for (int t = 0; t < 6; ++t) {
        const f32x4 sum = acc[t] + part[(6 + t) * 64 + l];
        const int mat = t / 3, sub = t % 3;
        const int ti = sub == 0 ? 0 : 1, tj = sub == 2 ? 1 : 0;
#pragma unroll
        for (int r = 0; r < 4; ++r)
          sm.gram[mat][16 * ti + 4 * (l >> 4) + r][16 * tj + (l & 15)] = sum[r];
      }
    }
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
// One workgroup = one value head x 32 value columns: 4 compute waves, wave (cs, rh) owning
// value columns 16 cs .. 16 cs + 15 of the workgroup and key rows 64 rh .. 64 rh + 63, and
// a producer wave.  Every operand a chunk needs (K and Q rows of the key head, the head's
// WY slot from the workspace and the workgroup's V tile) is copied by the producer from
// global memory straight into LDS with direct loads (16 bytes per lane, no registers, no
// LDS store instructions), into a ring of three buffers, chunk c + 3 into the buffer of
// chunk c as soon as chunk c's barrier has passed; the compute waves read everything from
// LDS and issue no loads (a direct load holds its wave for as long as the CU's vector
// memory path needs to move its 1 KB), only their output stores.
constexpr int SC_NT = 320;   // threads per scan workgroup: 4 compute waves + 1 producer
constexpr int SC_COLS = 32;  // value columns per scan workgroup
constexpr int SC_RING = 3;   // chunk buffers in LDS

// A direct load fills 64 consecutive 16-byte slots, so the tiles are unpadded; instead the
// 16-byte columns of each row are permuted (XOR with a function of the row) so that the
// reads below hit distinct LDS banks:
//   K, Q  [32 tokens][32 float4]  float4 p of token t at t*32 + (p ^ (t & 15))
//   T, P  [32 rows][8 float4]     float4 c of row i at i*8 + (c ^ sw8(i))
//   V     [32 tokens][8 float4]   float4 c of token t at t*8 + (c ^ swv(t))
//   misc  floats: e^gamma [0, 32), e^{gamma_last - gamma} [32, 64), e^{gamma_last} [64]
__device__ __forceinline__ int sw8(int i) { return (i ^ (i >> 3)) & 7; }
__device__ __forceinline__ int swv(int t) { return ((t >> 2) & 1) << 2; }

constexpr int SC_XCHG = 2 * 2 * 2 * 3 * 64;  // [parity][col slice][row half][tile][lane]

// The ring is laid out array by array (the K tiles of all ring positions, then the Q
// tiles, ...), so that each of a lane's read patterns reaches its tile in every ring
// position from one base register plus an immediate offset below 64 KiB (the reach of an
// LDS instruction's offset field): no address arithmetic inside the chunk loop.
struct ScanSmem {
  f32x4 k[SC_RING][kChunk * 32];
  f32x4 q[SC_RING][kChunk * 32];
  f32x4 T[SC_RING][kChunk * 8];
  f32x4 P[SC_RING][kChunk * 8];
  f32x4 misc[SC_RING][64];
  f32x4 v[SC_RING][kChunk * SC_COLS / 4];
  f32x4 x[SC_XCHG];
};
static_assert(sizeof(ScanSmem) <= 160 * 1024, "LDS of one CU");

// Raw buffer resource over `bytes` bytes from `base`; an empty range for bytes <= 0.
__device__ __forceinline__ buf_rsrc rsrc_range(const float* base, int bytes) {
  return make_rsrc(base, bytes > 0 ? (uint32_t)bytes : 0u);
}

template <int N>
using ic = std::integral_constant<int, N>;

// One wave of a scan workgroup: row half RH (key rows 64 RH .. 64 RH + 63) of column slice
// cs (value columns 16 cs .. 16 cs + 15 of the workgroup's 32).  The row half is a
// template parameter and the chunk loop is unrolled over the three ring buffers, so every
// LDS address is a loop-invariant per-lane base plus a constant, and the per-chunk global
// offsets live in scalar buffer descriptors: the instructions between the matrix products
// are the arithmetic of the method itself.
template <int RH>
__device__ __forceinline__ void scan_wave(const ChunkArgs& a, int h, int kh, int cblk, int cs,
                                          ScanSmem& sm) {
  const int Hv = a.n_v_heads;
  const int l = threadIdx.x & 63;
  const int q4 = l >> 4, lc = l & 15, lr = 4 * q4;
  const int colw = 16 * cs + lc;            // column inside the workgroup
  const int col = cblk * SC_COLS + colw;    // value column
  const int nch = (a.n_tok + kChunk - 1) / kChunk;

  // state: tile rt holds rows 64 RH + 16 rt + lr + r, column col
  f32x4 S[4];
#pragma unroll
  for (int rt = 0; rt < 4; ++rt)
#pragma unroll
    for (int r = 0; r < 4; ++r)
      S[rt][r] = a.s_src[((size_t)h * kDim + 64 * RH + 16 * rt + lr + r) * kDim + col];

  // LDS element indices of this lane's reads, relative to a ring buffer; token tile tt
  // and ring position add constants.
  int ka_i[4];     // f32x4 in k / q: token lc, float4 16 RH + 4 rt + q4 of its row
#pragma unroll
  for (int rt = 0; rt < 4; ++rt) ka_i[rt] = lc * 32 + ((16 * RH + 4 * rt + q4) ^ lc);
  int kt_i[4][4];  // float in k: token lr + r, row 64 RH + 16 rt + lc
#pragma unroll
  for (int rt = 0; rt < 4; ++rt)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = lr + r, row = 64 * RH + 16 * rt + lc;
      kt_i[rt][r] = (t * 32 + ((row >> 2) ^ (t & 15))) * 4 + (row & 3);
    }
  const int t00_i = lc * 8 + (q4 ^ sw8(lc));
  const int t10_i = (16 + lc) * 8 + (q4 ^ sw8(16 + lc));
  const int t11_i = (16 + lc) * 8 + ((4 + q4) ^ sw8(16 + lc));
  // P tiles of this wave's share of P D: row half 0 takes tile (0,0) and steps 0, 1 of
  // tile (1,0); row half 1 steps 2, 3 of tile (1,0) and tile (1,1) (six products each).
  const int pa_i = RH ? t10_i : t00_i;
  const int pb_i = RH ? t11_i : t10_i;
  // float in v: token lr (+ r, + 16 tt), column colw
  const int vv_i = (lr * 8 + ((colw >> 2) ^ ((q4 & 1) << 2))) * 4 + (colw & 3);
  // Exchange area of the column slice, [row half][tile][lane] from here: tiles 0, 1 the
  // partial K S0 of each token tile, tile 2 the part of the other half's output tile.
  const f32x4* const xs = sm.x + cs * 2 * 3 * 64 + l;
  constexpr int XW = 192 * RH, XP = 192 * (1 - RH) + 128;  // this half's tiles, partner's part

  // O stores of token 16 RH + lr + r of a chunk
  uint32_t o_off[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) o_off[r] = (((16 * RH + lr + r) * Hv + h) * kDim + col) * 4;


  // Output tile RH of chunk c - 1: this wave's part plus the other half's, which arrives
  // with the barrier of chunk c.  For c = 0 the range is empty and the stores are dropped.
  auto store_prev_o = [&](const f32x4 own, const f32x4 other, int c) {
    const f32x4 O = own + other;
    const int cp = c > 0 ? c - 1 : 0;
    const buf_rsrc ro = rsrc_range(a.o + (size_t)(a.t_begin + cp * kChunk) * Hv * kDim,
                                   c > 0 ? (a.n_tok - cp * kChunk) * Hv * kDim * 4 : 0);
#pragma unroll
    for (int r = 0; r < 4; ++r) buf_store_nt(ro, o_off[r], O[r]);  // dropped past the end
  };
  f32x4 Oprev = f32x4{0.f, 0.f, 0.f, 0.f};  // this wave's part of the previous output tile

  auto step = [&](auto rbc, int c) {
    constexpr int RB = decltype(rbc)::value;
    const float* kf = reinterpret_cast<const float*>(sm.k[RB]);
    const float* vf = reinterpret_cast<const float*>(sm.v[RB]);

    // (a)+(b) This chunk's operands (published by the previous barrier; the buffer is
    //     reloaded after this chunk's barrier, so everything is read before it) and the
    //     partial K S0 over this wave's 64 rows (the state registers are the B operand as
    //     they are).  The reads go out in the order the products consume them: all K tiles
    //     and the first Q tiles before the first product, the rest in four batches, one
    //     behind the products of each row tile (the other Q tiles with the first K^T tile,
    //     the second K^T tile with the operators T and P, the last two K^T tiles, the
    //     decays and V), so that every batch lands while the matrix core is busy instead
    //     of all of them queueing on the LDS at once after the barrier.  The fences keep
    //     the compiler from merging the batches.
    f32x4 ka[4][2], qa[4][2];
    float kt[4][2][4];
    f32x4 T00, T10, T11, Pa, Pb, eg[2], eb[2], vv[2];
    float egl;
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) ka[rt][tt] = sm.k[RB][ka_i[rt] + 16 * 32 * tt];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) qa[0][tt] = sm.q[RB][ka_i[0] + 16 * 32 * tt];
    __builtin_amdgcn_sched_barrier(0);
    f32x4 Wp[2], Qp[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) Wp[i] = Qp[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    auto w_rt = [&](int rt) {  // row tile rt's share of the partial K S0
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) Wp[tt] = mfma16x16x4(ka[rt][tt][r], S[rt][r], Wp[tt]);
    };
    auto kt_rt = [&](int rt) {  // K^T operands of row tile rt for the state update
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int r = 0; r < 4; ++r) kt[rt][tt][r] = kf[kt_i[rt][r] + 16 * 32 * 4 * tt];
    };
    w_rt(0);
#pragma unroll
    for (int rt = 1; rt < 4; ++rt)
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) qa[rt][tt] = sm.q[RB][ka_i[rt] + 16 * 32 * tt];
    kt_rt(0);
    __builtin_amdgcn_sched_barrier(0);
    w_rt(1);
    kt_rt(1);
    T00 = sm.T[RB][t00_i];
    T10 = sm.T[RB][t10_i];
    T11 = sm.T[RB][t11_i];
    Pa = sm.P[RB][pa_i];
    Pb = sm.P[RB][pb_i];
    __builtin_amdgcn_sched_barrier(0);
    w_rt(2);
    kt_rt(2);
    kt_rt(3);
    __builtin_amdgcn_sched_barrier(0);
    w_rt(3);
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      eg[tt] = sm.misc[RB][4 * tt + q4];
      eb[tt] = sm.misc[RB][8 + 4 * tt + q4];
#pragma unroll
      for (int r = 0; r < 4; ++r) vv[tt][r] = vf[vv_i + 32 * r + 16 * 32 * tt];
    }
    egl = reinterpret_cast<const float*>(sm.misc[RB])[64];
    __builtin_amdgcn_sched_barrier(0);

    //     Then the partial Q S0, whose products cover the exchange: a few before the
    //     partial K S0 is written, the rest after the barrier while it is read back.
    auto qs = [&](int rt, int r) {
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) Qp[tt] = mfma16x16x4(qa[rt][tt][r], S[rt][r], Qp[tt]);
    };
    qs(0, 0);
    qs(0, 1);
    __builtin_amdgcn_sched_barrier(0);

    // (c) Exchange with the other row half of the same columns: the two K S0 partials of
    //     this chunk go out; the other half's part of the previous chunk's output tile
    //     comes in.  (The producer has published chunk c + 1 by the same barrier.)
    f32x4* const xc = const_cast<f32x4*>(xs) + (c & 1) * (SC_XCHG / 2);  // this chunk's
    f32x4* const xn = const_cast<f32x4*>(xs) + (~c & 1) * (SC_XCHG / 2);  // the next one's
    xc[XW] = Wp[0];
    xc[XW + 64] = Wp[1];
    qs(0, 2);
    qs(0, 3);
    __builtin_amdgcn_sched_barrier(0);
    wait_vm_lgkm0<63>();  // LDS writes done; the O stores may still be in flight
    barrier_only();
    __builtin_amdgcn_sched_barrier(0);
    f32x4 Wx[2][2];  // [row half][token tile]
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      Wx[0][tt] = xc[64 * tt];
      Wx[1][tt] = xc[192 + 64 * tt];
    }
    const f32x4 Xprev = xc[XP];
    __builtin_amdgcn_sched_barrier(0);  // the reads go out before the products below
    // Eight Q S0 products go first, covering the latency of those reads; left free, the
    // compiler starts the U arithmetic after one product and the wave waits for the LDS
    // with the matrix pipe nearly idle (measured: 2.207 against 2.225 ms per 32768-token
    // layer; 4, 12 and 16 products first: 2.214, 2.213, 2.210).
#pragma unroll
    for (int r = 0; r < 4; ++r) qs(1, r);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int rt = 2; rt < 4; ++rt)
#pragma unroll
      for (int r = 0; r < 4; ++r) qs(rt, r);
    store_prev_o(Oprev, Xprev, c);
    // Both halves add the two partials in the same order, so they hold identical sums.
    f32x4 W[2];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) W[tt] = Wx[0][tt] + Wx[1][tt];

    // (d) U = V - e^{gamma} (K S0), C layout: token 16 tt + lr + r, column col.
    f32x4 U[2];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int r = 0; r < 4; ++r) U[tt][r] = fmaf(-eg[tt][r], W[tt][r], vv[tt][r]);

    // (e) D = T diag(beta) U; T is lower triangular, so tile (0,1) is zero.
    f32x4 D[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      D[0] = mfma16x16x4(T00[r], U[0][r], D[0]);
      D[1] = mfma16x16x4(T10[r], U[0][r], D[1]);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) D[1] = mfma16x16x4(T11[r], U[1][r], D[1]);

    // (f) Outputs O = e^{gamma} Q S0 + P D (P lower triangular).  Token tile RH is this
    //     wave's; its part here covers its own rows of Q S0, the other half's part (sent
    //     at the next barrier) the rest.
    f32x4 own = eg[RH] * Qp[RH];
    f32x4 other = eg[1 - RH] * Qp[1 - RH];
    if (RH == 0) {
#pragma unroll
      for (int r = 0; r < 4; ++r) own = mfma16x16x4(Pa[r], D[0][r], own);
#pragma unroll
      for (int r = 0; r < 2; ++r) other = mfma16x16x4(Pb[r], D[0][r], other);
    } else {
#pragma unroll
      for (int r = 2; r < 4; ++r) own = mfma16x16x4(Pa[r], D[0][r], own);
#pragma unroll
      for (int r = 0; r < 4; ++r) own = mfma16x16x4(Pb[r], D[1][r], own);
    }
    Oprev = own;
    xn[XW + 128] = other;  // read after the next barrier

    // (g) S' = e^{gamma_last} S0 + K^T diag(e^{gamma_last - gamma}) D.
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
    __builtin_amdgcn_sched_barrier(0);
  };

  barrier_only();  // chunk 0 published by the producer
  for (int c = 0; c < nch; c += SC_RING) {
    step(ic<0>(), c);
    if (c + 1 >= nch) break;
    step(ic<1>(), c + 1);
    if (c + 2 >= nch) break;
    step(ic<2>(), c + 2);
  }
  // The last chunk's output tile: one more barrier brings the other half's part.
  wait_vm_lgkm0<63>();
  barrier_only();
  store_prev_o(Oprev, xs[(nch & 1) * (SC_XCHG / 2) + XP], nch);

  // The state goes out through 32-bit buffer offsets recomputed here from the lane id (not
  // addresses kept from before the loop, which would occupy registers all along it).
  const int lid = __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
  const buf_rsrc rs = make_rsrc(a.s_dst + (size_t)h * kDim * kDim, kDim * kDim * 4);
  const uint32_t s_off = ((64 * RH + 4 * (lid >> 4)) * kDim + cblk * SC_COLS + 16 * cs + (lid & 15)) * 4;
#pragma unroll
  for (int rt = 0; rt < 4; ++rt)
#pragma unroll
    for (int r = 0; r < 4; ++r) buf_store_nt(rs, s_off + (16 * rt + r) * kDim * 4, S[rt][r]);
}

// The producer wave of a scan workgroup: all direct loads of every chunk, and the waits
// that make a chunk's operands complete before the barrier that publishes them.  It meets
// the compute waves at the same barriers (one before the first chunk, one per chunk, one
// after the last).
constexpr int SC_DMA = 45;  // direct loads per chunk: K 16, Q 16, T 4, P 4, decays 1, V 4

__device__ __forceinline__ void scan_producer(const ChunkArgs& a, int h, int kh, int cblk,
                                              ScanSmem& sm) {
  const int Hk = a.n_k_heads, Hv = a.n_v_heads;
  const int l = threadIdx.x & 63;
  const int nch = (a.n_tok + kChunk - 1) / kChunk;

  // Per-lane byte offsets: slot s of a 64-slot slice is lane s % 64, so each lane fetches
  // the source float4 that the permutation of the tile puts there.  K and Q slices
  // relative to the chunk's first token, T / P / decays relative to the workspace slot, V
  // relative to the chunk's first token.
  uint32_t off_kq[16], off_t[4], off_p[4], off_v[4];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int t = (64 * i + l) >> 5, p = (l & 31) ^ (t & 15);
    off_kq[i] = ((t * Hk + kh) * kDim + 4 * p) * 4;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int srow = (64 * i + l) >> 3;
    off_t[i] = (kSlotT + srow * kChunk + 4 * ((l & 7) ^ sw8(srow))) * 4;
    off_p[i] = off_t[i] + (kSlotP - kSlotT) * 4;
    off_v[i] = ((srow * Hv + h) * kDim + cblk * SC_COLS + 4 * ((l & 7) ^ swv(srow))) * 4;
  }
  const uint32_t off_m = (kSlotEg + 4 * min(l, 16)) * 4;  // lanes past 16 repeat lane 16
  const uint32_t lds = lds_address(&sm);

  // Descriptors of chunk c: its tokens onward (an empty range past the end, so the loads
  // return 0) and its workspace slot (clamped to the last chunk).
  auto tok_desc = [&](const float* base, int row_floats, int c) {
    return make_desc(base + (size_t)(a.t_begin + c * kChunk) * row_floats,
                     (a.n_tok - c * kChunk) * row_floats * 4);
  };
  auto issue = [&](auto rbc, int c) {
    constexpr int RB = decltype(rbc)::value;
    const i32x4 dk = tok_desc(a.k, Hk * kDim, c), dq = tok_desc(a.q, Hk * kDim, c);
    const i32x4 dv = tok_desc(a.v, Hv * kDim, c);
    const i32x4 dw = make_desc(a.ws + ((size_t)min(c, nch - 1) * Hv + h) * kSlot, kSlot * 4);
    const auto s16 = std::make_integer_sequence<int, 16>();
    const auto s4 = std::make_integer_sequence<int, 4>();
    dma16_run<offsetof(ScanSmem, k) + RB * sizeof(sm.k[0])>(dk, off_kq, lds, s16);
    dma16_run<offsetof(ScanSmem, q) + RB * sizeof(sm.q[0])>(dq, off_kq, lds, s16);
    dma16_run<offsetof(ScanSmem, T) + RB * sizeof(sm.T[0])>(dw, off_t, lds, s4);
    dma16_run<offsetof(ScanSmem, P) + RB * sizeof(sm.P[0])>(dw, off_p, lds, s4);
    dma16_run<offsetof(ScanSmem, v) + RB * sizeof(sm.v[0])>(dv, off_v, lds, s4);
    dma16<offsetof(ScanSmem, misc) + RB * sizeof(sm.misc[0])>(dw, off_m, lds);
  };
  // At the barrier of chunk c the loads of chunk c + 1 must have landed; those of chunk
  // c + 2 (issued after the previous barrier) may still be in flight.  After it, every
  // compute wave has read chunk c, whose buffer then takes chunk c + 3.
  auto publish = [&]() {
    wait_vm_lgkm0<SC_DMA>();
    barrier_only();
  };
  issue(ic<0>(), 0);
  issue(ic<1>(), 1);
  publish();
  issue(ic<2>(), 2);
  for (int c = 0; c < nch; c += SC_RING) {
    publish();
    issue(ic<0>(), c + 3);
    if (c + 1 >= nch) break;
    publish();
    issue(ic<1>(), c + 4);
    if (c + 2 >= nch) break;
    publish();
    issue(ic<2>(), c + 5);
  }
  barrier_only();  // the compute waves' last exchange
  // Loads past the last chunk (never read) must land before the workgroup's LDS is
  // released.
  wait_vm_lgkm0<0>();
}

// One scan workgroup (block index `b` of `nb` scan workgroups).
__device__ __forceinline__ void scan_block(const ChunkArgs& a, int b, int nb, ScanSmem& sm) {
  constexpr int NCB = kDim / SC_COLS;  // column blocks per value head
  const int Hk = a.n_k_heads, G = a.n_v_heads / Hk;
  const int L = xcd_grouped_block(b, nb);
  // logical order: key head, then value head of the group, then column block
  const int kh = L / (G * NCB), m = (L / NCB) % G, cblk = L % NCB;
  const int h = kh + m * Hk;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (w == 4)
    scan_producer(a, h, kh, cblk, sm);
  else if (w & 1)
    scan_wave<1>(a, h, kh, cblk, w >> 1, sm);
  else
    scan_wave<0>(a, h, kh, cblk, w >> 1, sm);
}

// Prep alone: one workgroup per (chunk, key head) of a super-block.
__global__ __launch_bounds__(PREP_NT, 4) void chunk_prep_kernel(ChunkArgs a) {
  __shared__ PrepSmem sm;
  prep_item(a, blockIdx.x, blockIdx.y, sm, threadIdx.x);
}

// Scan of super-block n fused with the prep of super-block n+1: workgroups
// [0, n_scan) scan (they are dispatched first and take one CU each), the rest loop over
// the (chunk, key head) items of the next super-block on the CUs the scan leaves idle.
// The two roles touch disjoint halves of the workspace, and the next launch reads what
// this one's prep wrote, so the roles never wait for each other.
struct FusedArgs {
  ChunkArgs scan;
  ChunkArgs prep;
  NormArgs norm;
  int n_scan;  // scan workgroups
  int has_prep;
  int has_norm;
};

// The output norm of the previous super-block, run by the three waves of each scan
// workgroup that the scan leaves free (they share the SIMDs with the compute waves, whose
// issue their vector instructions delay, so the role keeps its arithmetic to the row's).
// They take part in exactly the scan's barriers (one before the first chunk, one per
// chunk, one after the last), doing a slice of rows between barriers: half-wave `worker`
// of `nworkers` owns rows worker + j * nworkers, j = 0 .. 127
// (n_scan * 6 * 128 >= 2048 * n_v_heads rows), and handles j = c and j = c + 64 between
// the barriers of chunks c - 1 and c, with the loads of the next slice issued before the
// arithmetic of this one.  Slices left over (nch < 64) run before the final barrier.
__device__ __forceinline__ void norm_role(const NormArgs& n, int worker, int nworkers, int nch) {
  const int p = threadIdx.x & 31;
  const uint32_t bytes = (uint32_t)n.n_rows * kDim * 4;
  const buf_rsrc ro = make_rsrc(n.o, bytes), rz = make_rsrc(n.z, bytes);
  const buf_rsrc ry = make_rsrc(n.y, bytes / 2);
  // Every row of this worker belongs to one value head: rows are worker + j * nworkers
  // and nworkers (6 half-waves x 4 scan workgroups per value head) is a multiple of the
  // head count (checked at launch), so the head's weight row is loaded once (measured:
  // 2.174 against 2.197 ms per 32768-token layer with a load and a modulo per row).
  const int hw = worker % n.n_v_heads;
  const f32x4 wrow = buf_load4(make_rsrc(n.w, (uint32_t)n.n_v_heads * kDim * 4),
                               ((uint32_t)hw * kDim + 4 * p) * 4);
  const float4 wv = float4{wrow[0], wrow[1], wrow[2], wrow[3]};
  f32x4 ov[2][2], zv[2][2];  // [buffer][row of the slice]
  auto row_of = [&](int j) { return worker + j * nworkers; };
  // Buffer indices are compile-time constants throughout, and the loops have no early
  // exit: loaded values in flight never meet a branch join, at which the compiler would
  // have to wait for them.
  auto load = [&](auto bc, int c) {  // rows past the end read as 0
    constexpr int B = decltype(bc)::value;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int r = row_of(c + kChunksPerSB * i);
      const uint32_t off = ((uint32_t)r * kDim + 4 * p) * 4;
      ov[B][i] = buf_load4(ro, off);
      zv[B][i] = buf_load4(rz, off);
    }
  };
  auto finish = [&](auto bc, int c) {
    constexpr int B = decltype(bc)::value;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int r = row_of(c + kChunksPerSB * i);
      if (r < n.n_rows)  // whole half-waves: the two halves of a wave may differ
        buf_store2_nt(ry, ((uint32_t)r * kDim + 4 * p) * 2,
                      gated_rms_row(ov[B][i], zv[B][i], wv, n.eps));
    }
  };
  // Slices j .. 63 after the chunks (no barriers), the loads of slice j already in buffer B.
  auto tail = [&](auto bc, int j) {
    if constexpr (decltype(bc)::value == 1) {
      load(ic<0>(), j + 1);
      finish(ic<1>(), j);
      ++j;
    }
    for (; j < kChunksPerSB; j += 2) {
      load(ic<1>(), j + 1);
      finish(ic<0>(), j);
      load(ic<0>(), j + 2);
      finish(ic<1>(), j + 1);
    }
  };
  load(ic<0>(), 0);
  barrier_only();
  int c = 0;
  for (; c + 1 < nch; c += 2) {
    load(ic<1>(), c + 1);
    finish(ic<0>(), c);
    barrier_only();
    load(ic<0>(), c + 2);
    finish(ic<1>(), c + 1);
    barrier_only();
  }
  if (c < nch) {  // an odd chunk count: one more chunk, then the rest from buffer 1
    load(ic<1>(), c + 1);
    finish(ic<0>(), c);
    barrier_only();
    tail(ic<1>(), c + 1);
  } else {
    tail(ic<0>(), c);
  }
  barrier_only();  // the compute waves' last exchange
}

union FusedSmem {
  ScanSmem scan;
  PrepSmem prep[2];  // one per group of 4 waves
};

// Workgroups of 512 threads (8 waves, two per SIMD).  A scan workgroup uses 4 compute waves
// and the producer (the other 3 end at once); a prep workgroup runs two independent streams
// of items, waves 0-3 and 4-7, each with its own LDS area (a wave that has ended no longer
// takes part in barriers, so a stream that runs out of items simply ends).
constexpr int FUSED_NT = 512;
static_assert(FUSED_NT >= SC_NT && FUSED_NT == 2 * PREP_NT, "roles of the fused workgroup");

__global__ __launch_bounds__(FUSED_NT) void chunk_fused_kernel(FusedArgs f) {
  __shared__ FusedSmem sm;
  const int b = blockIdx.x;
  if (b < f.n_scan) {
    if (threadIdx.x < SC_NT) {
      scan_block(f.scan, b, f.n_scan, sm.scan);
    } else if (f.has_norm) {
      const int per_wg = (FUSED_NT - SC_NT) / 32;  // norm half-waves per scan workgroup
      norm_role(f.norm, b * per_wg + (threadIdx.x - SC_NT) / 32, f.n_scan * per_wg,
                (f.scan.n_tok + kChunk - 1) / kChunk);
    }
  } else if (f.has_prep) {
    const int Hk = f.prep.n_k_heads;
    const int items = ((f.prep.n_tok + kChunk - 1) / kChunk) * Hk;
    const int n_streams = 2 * ((int)gridDim.x - f.n_scan);
    const int g = __builtin_amdgcn_readfirstlane(threadIdx.x / PREP_NT);
    for (int it = 2 * (b - f.n_scan) + g; it < items; it += n_streams)
      prep_item(f.prep, it / Hk, it % Hk, sm.prep[g], threadIdx.x - g * PREP_NT);
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
                                   const NormArgs* norm_prev, hipStream_t stream) {
  FusedArgs f;
  f.scan = scan;
  f.prep = prep_next ? *prep_next : scan;
  f.norm = norm_prev ? *norm_prev : NormArgs{};
  f.has_norm = norm_prev != nullptr;
  f.n_scan = scan.n_v_heads * (kDim / SC_COLS);
  f.has_prep = prep_next != nullptr;
  // the norm role gives each half-wave rows of a single value head (norm_role)
  if (norm_prev && (f.n_scan * ((FUSED_NT - SC_NT) / 32)) % norm_prev->n_v_heads != 0)
    return hipErrorInvalidValue;
  // the prep workgroups fill the CUs the scan leaves free (at least 32 of them)
  int n_prep = 0;
  if (prep_next) {
    int cus = 0;
    if (const hipError_t e = device_cu_count(stream, &cus)) return e;
    n_prep = cus - f.n_scan;
    if (n_prep < 32) n_prep = 32;
  }
  void* args[] = {&f};
  return hipLaunchKernel(reinterpret_cast<const void*>(&chunk_fused_kernel),
                         dim3(f.n_scan + n_prep), dim3(FUSED_NT), args, 0, stream);
}

}  // namespace gdn
