// kda_twopass.hip -- chunked (64-token) prefill in two passes on MFMA (gfx950).
//
// Chunk algebra.  Unrolling the gated delta rule (GLM-5.3-Flash model notes,
// Glm5NextTextLinearAttention snippet) over one chunk of C = 64 tokens from the
// entry state S (dk x dv), with G_i = sum_{s<=i} log_g_s per key channel,
// gamma = G_63, Xk = beta K exp(G), Xv = beta V:
//   A[i,j]   = beta_i sum_c k_ic k_jc exp(G_ic - G_jc)     (j < i)
//   T        = (I + A)^-1,  W = T Xk,  U = T Xv
//   Delta    = U - W S                                  (per-token beta (v - S^T k))
//   Aqk[i,j] = sum_c q_ic k_jc exp(G_ic - G_jc)            (j <= i)
//   O        = scale (Q exp(G) S + Aqk Delta) = Qs S + As Delta
//              with Qs = scale Q exp(G), As = scale Aqk
//   S_next   = exp(gamma) S + (K exp(gamma - G))^T Delta
// (the output reads the state after each token's update).
//
// Pass 1 (prep_kernel) depends on nothing but the chunk's own inputs, so it
// runs over every (chunk, head) at once: it forms A, Aqk, T and writes the
// fp16 operands W, Qs, K exp(gamma - G), U, As plus exp(gamma) to a workspace
// slot.  Pass 2 (scan_kernel) is the only serial part: per (unit, 32-column
// value tile) it walks the unit's chunks with the fp32 state in MFMA
// accumulators, three 64x128x32-class products per chunk (W S and Qs S share
// the state operand; K^T Delta updates the state) and As Delta, which reads
// the Delta tile the state update reads, with the slot operands of the next
// two chunks in flight while one chunk is processed.  Its eight waves split
// the roles: four form Delta (the serial chain), four form the outputs, all
// eight update 16 state rows each.  scan4_kernel is the four-wave form (each
// wave both roles for one 16-token block, two workgroups per CU), taken when
// there are more tiles than CUs.  Outputs leave as whole 128-byte rows (fp32)
// with the nontemporal policy; the slot is written likewise where its pieces
// form whole lines per instruction.
//
// Decay factors without overflow (pass 1).  The chunk is cut into four
// 16-token blocks.  With R_I = G before block I's first token:
//   Kl = k exp(G - R_I) <= |k|, Ql = q exp(G - R_I), Kr = k exp(R_{I+1} - G) <= |k|
// come from prefix / suffix products of exp(log_g) inside a block.
// Off-diagonal tiles (I > J) pair Kl_I exp(R_I - R_{J+1}) with Kr_J: every
// factor is <= 1 for any gate.  Diagonal tiles use the block's midpoint M_I:
// Kl_I exp(R_I - M_I) against Kr_I exp(M_I - R_{I+1}), factors bounded by
// exp(HALF_SPAN_MAX).  exp(G) = Kl-side factor times exp(R_I) <= 1 and
// exp(gamma - G) = Kr-side factor times exp(gamma - R_{I+1}) <= 1.
//
// Strong decays.  The midpoint factors of the diagonal tiles grow like the
// decay over half a block; beyond HALF_SPAN_MAX in any channel the chunk's
// diagonal tiles are built instead by a binary tree of token pairs whose
// factors are all <= 1 (diag_tree below), so no gate, however strong, leaves
// the MFMA path.
//
// Fast-path guard.  A chunk is evaluated token by token in exact fp32 (in
// pass 2) instead when its inputs could overflow an fp16 operand, a diagonal
// block of A exceeds 1 in magnitude, any fp16 intermediate (T, W, U, Qs, As,
// Delta) would exceed F16_SAFE, or the entry state exceeds S_MAX.
//
// Arithmetic: fp16 MFMA operands (formed in fp32 from the bf16 inputs and
// rounded once; the guard keeps them inside fp16's range), fp32
// accumulation and state; outputs fp32, or rounded once to bf16.  With L a strictly lower 16x16 diagonal
// block of A (L^16 = 0), (I + L)^-1 = (I - L)(I + L^2)(I + L^4)(I + L^8); the
// off-diagonal blocks of T follow by block forward substitution,
// T_IJ = -T_II sum_{J<=K<I} A_IK T_KJ.
//
// Fragment algebra of the 16x16x16 MFMA (lane = 16 lg + lc): the A operand
// holds X[lc][4lg+e] ("fragA(X)"), the B operand and the result hold
// X[4lg+e][lc] ("fragB(X)").  Hence fragB(XY) = mfma(fragA(X), fragB(Y)) and
// fragA(XY) = mfma(fragB(Y), fragA(X)).
#include <cstdlib>
#include <cstring>
#include <mutex>

#include "kda_common.h"
#include "kda_fallback.h"
#include "kda_launch.h"

namespace kda {
namespace {

constexpr int C = 64;        // chunk length
constexpr int D = 128;       // head dim (dk = dv)
constexpr int DVT = 32;      // value columns per scan workgroup
constexpr int NTILE = D / DVT;
constexpr int NTP = 512;     // threads per prep workgroup: eight waves, two workgroups per CU
constexpr int LDK = D + 8;   // fp16 row stride of [64][128] LDS arrays
constexpr int LDX = C + 4;   // fp16 row stride of [128][64] LDS arrays
constexpr int LDT = C + 8;   // fp16 row stride of the Delta^T tile
constexpr float HALF_SPAN_MAX = 6.0f;           // max decay (e-folds) over half a block
constexpr unsigned short QK_MAX_BITS = 0x4280;  // bf16 bits of 64.0: |q|, |k| bound
constexpr unsigned short V_MAX_BITS = 0x4580;   // bf16 bits of 4096.0: |v| bound
constexpr float BETA_MAX = 1.0f;                // |beta| bound
constexpr float S_MAX = 2048.0f;                // |S| bound of the fast path
constexpr float F16_SAFE = 16384.0f;            // bound of every fp16 intermediate

// Workspace slot of one (chunk, head), bytes.
// -W, Qs, As and (K exp(gamma - G))^T are stored in the order the scan's
// lanes read them, so every scan load instruction covers 1 KiB of whole lines:
//   NW, QS: [I 4][ks 4][lane 64][j 8] = X[16I+lc][32ks+8lg+j]
//   AS:     [I 4][ks 2][lane 64][j 8] = As[16I+lc][32ks+8lg+j]  (zero above the diagonal;
//           the all-zero pieces (I 0|1, ks 1) are left unwritten)
//   KDT:    [r 8][ks 2][lane 64][j 8] = Kd^T[16r+lc][32ks+8lg+j]
constexpr size_t OFF_NW = 0;        // -W          64 x 128  fp16
constexpr size_t OFF_QS = 16384;    // Qs          64 x 128  fp16
constexpr size_t OFF_KDT = 32768;   // Kd^T        128 x 64  fp16
constexpr size_t OFF_UP = 49152;    // U  by scan lane: [I][tile][b][lane][e] = U[16I+lc][32tile+16b+4lg+e]
constexpr size_t OFF_AS = 65536;    // As          64 x 64   fp16
constexpr size_t OFF_GAM = 73728;   // exp(gamma)  [128] fp32
constexpr size_t OFF_FLAG = 74240;  // per prep wave "not on the fast path" [8] bytes
constexpr size_t SLOT_BYTES = 74752;

// position of fragA(X_IJ) (lane holds X[16I+lc][16J+4lg+e]) in a [I][ks][lane][j] field of
// 64 x (16 nks) fp16: k-step J/2, lane (lg' = 2(J&1) + lg/2, lc), position 4(lg&1)
__device__ __forceinline__ int frag_pos(int I, int J, int nks, int lane) {
  const int lc = lane & 15, lg = lane >> 4;
  return ((I * nks + (J >> 1)) * 64 + 16 * (2 * (J & 1) + (lg >> 1)) + lc) * 8 + 4 * (lg & 1);
}

// LDS fragment slots of pass 1 (one f16x4 per lane each).
constexpr int S_TD = 0;    // fragA(T_II)               4
constexpr int S_AO = 4;    // fragA(A_IJ), I > J        6
constexpr int S_TO = 10;   // fragA(T_IJ), I > J        6
constexpr int NFRAG = 16;

__device__ __forceinline__ constexpr int tile10(int I, int J) { return (I * (I + 1)) / 2 + J; }  // J <= I
__device__ __forceinline__ constexpr int pair6(int I, int J) { return (I * (I - 1)) / 2 + J; }   // J < I

struct PrepArgs {
  const bf16_t* q;
  const bf16_t* k;
  const bf16_t* v;
  const float* log_g;
  const float* beta;
  const int32_t* cu_seqlens;  // null: dense
  const int32_t* cstart;      // packed: first chunk slot of each document
  const int32_t* table;       // packed: document of each chunk slot (-1: none)
  unsigned char* ws;          // chunk slots
  int T;                      // dense tokens per sequence
  int H;
  int nchd;                   // dense chunks per sequence
  float scale;
};

constexpr float L2_EPS = 1e-6f;  // eps inside the root of the q / k L2 normalisation

struct __align__(16) PrepSmem {
  union {
    struct {
      f16 Kl[C][LDK];      // k exp(G - R_blk)
      f16 Kr[C][LDK];      // k exp(R_blk_end - G)
    } a;                   // until the products are done
    struct {
      f16 XkT[D][LDX];     // (beta k exp(G))^T
      f16 XvT[D][LDX];     // (beta v)^T
    } x;                   // from then on
  } u;
  f16 Ql[C][LDK];          // q exp(G - R_blk)
  float tot[4][D];         // per-block products of exp(log_g)
  f16 fDl[4][D];           // exp(R_I - M_I)
  f16 fDr[4][D];           // exp(M_I - R_{I+1})
  float beta[C];
  float2 nrm[2][C];        // per channel half: (k.k, q.q) of each row (L2 normalisation)
  int strong[8];           // per stage-A wave: a half block decays beyond HALF_SPAN_MAX
  f16x4 frag[NFRAG][64];
};

// fp16 factor row exp(R_I - R_{J+1}) for the off-diagonal pair (I, J), channels kc..kc+7
// (only the non-adjacent pairs (2,0), (3,0), (3,1) need one).
__device__ __forceinline__ f16x8 off_factor(const PrepSmem& sm, int I, int J, int kc) {
  const float4 a0 = *reinterpret_cast<const float4*>(&sm.tot[J + 1][kc]);
  const float4 a1 = *reinterpret_cast<const float4*>(&sm.tot[J + 1][kc + 4]);
  float f[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
  if (I - J == 3) {
    const float4 b0 = *reinterpret_cast<const float4*>(&sm.tot[2][kc]);
    const float4 b1 = *reinterpret_cast<const float4*>(&sm.tot[2][kc + 4]);
    f[0] *= b0.x; f[1] *= b0.y; f[2] *= b0.z; f[3] *= b0.w;
    f[4] *= b1.x; f[5] *= b1.y; f[6] *= b1.z; f[7] *= b1.w;
  }
  f16x8 r;
#pragma unroll
  for (int c = 0; c < 8; ++c) r[c] = (f16)f[c];
  return r;
}

// Column J of T below the diagonal, into the fragment slots.  tbJ =
// fragB(T_JJ).  Returns "an entry is too large".
template <int J>
__device__ __forceinline__ bool t_column(PrepSmem& sm, f16x4 tbJ, int lane) {
  bool bad = false;
  f16x4 tb[4];  // fragB(T_KJ)
  tb[J] = tbJ;
#pragma unroll
  for (int I = J + 1; I < 4; ++I) {
    f32x4 r = zero4();  // fragB(R), R = sum_K A_IK T_KJ
#pragma unroll
    for (int K = J; K < I; ++K) r = mfma16(sm.frag[S_AO + pair6(I, K)][lane], tb[K], r);
    const f16x4 rh = h4(r);
    const f16x4 tiA = sm.frag[S_TD + I][lane];
    const f32x4 ta = mfma16(rh, tiA, zero4());   // fragA(T_II R)
    const f32x4 tbb = mfma16(tiA, rh, zero4());  // fragB(T_II R)
    f16x4 sa, sb;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      bad |= !(fabsf(ta[e]) <= F16_SAFE);
      sa[e] = (f16)(-ta[e]);
      sb[e] = (f16)(-tbb[e]);
    }
    sm.frag[S_TO + pair6(I, J)][lane] = sa;
    tb[I] = sb;
  }
  return bad;
}

// x from lane (lane - SH) / (lane + SH) of the same 16-lane row (DPP row
// shift); lanes whose source lies outside the row keep `fill`.  A DPP read
// from a lane outside EXEC also returns `fill`, so the shift must run in every
// lane: the empty asm pins it ahead of the caller's select, which the compiler
// would otherwise turn into an EXEC-masked branch around the shift.
template <int SH>
__device__ __forceinline__ float row_shr(float x, float fill) {
  float y = __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, fill),
                                                                  __builtin_bit_cast(int, x), 0x110 + SH, 0xf, 0xf,
                                                                  false));
  asm volatile("" : "+v"(y));
  return y;
}
template <int SH>
__device__ __forceinline__ float row_shl(float x, float fill) {
  float y = __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, fill),
                                                                  __builtin_bit_cast(int, x), 0x100 + SH, 0xf, 0xf,
                                                                  false));
  asm volatile("" : "+v"(y));
  return y;
}

// The value of x in lane (lane ^ 8), within the same 16-lane row (a DPP row
// rotation by 8).  x is taken as a scalar: a bit cast of a vector element in
// place can read the vector's first element instead.
__device__ __forceinline__ float row_ror8(float x) {
  float y = __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x128, 0xf, 0xf,
                                                                  false));
  asm volatile("" : "+v"(y));
  return y;
}

// Cache policy of the scans' output stores: nontemporal (the NT bit of the
// buffer instruction's aux field).  The outputs are never read back, and
// whole-line streaming stores leave L2 to the slot lines the other tiles of a
// unit still read.
constexpr int OUT_AUX = 2;

// The fp32 outputs of a 16-token x 32-column block stored as whole 128-byte
// rows.  Lane (lc, lg) holds o[b][e] = O[row lc][col 16b + 4lg + e]; lanes lc
// and lc ^ 8 swap one half (a DPP rotation by 8 within the 16-lane row), so the
// first store writes rows 0..7 and the second rows 8..15, each instruction
// eight whole rows.  off0: byte offset of the block's row 0, column 0; rs: row
// stride in bytes.  Every lane of the wave must take part (DPP).
__device__ __forceinline__ void store_rows_f32(const f32x4 (&o)[2], __amdgpu_buffer_rsrc_t r, uint32_t off0,
                                               uint32_t rs, int lc, int lg) {
  const bool lo = lc < 8;
  const f32x4 x = lo ? o[1] : o[0];
  f32x4 y;
#pragma unroll
  for (int e = 0; e < 4; ++e) y[e] = row_ror8(x[e]);
  const f32x4 pa = lo ? o[0] : y, pb = lo ? y : o[1];
  const uint32_t off = off0 + static_cast<uint32_t>(lc & 7) * rs + static_cast<uint32_t>(16 * (lc >> 3) + 4 * lg) * 4u;
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(i32x4, pa), r, static_cast<int>(off), 0, OUT_AUX);
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(i32x4, pb), r, static_cast<int>(off + 8 * rs), 0, OUT_AUX);
}

struct DiagTiles {
  f32x4 a;  // fragA of sum_c k_t k_s exp(G_t - G_s), s < t (rows t = lc)
  f32x4 b;  // the same in fragB (rows t = 4lg+e)
  f32x4 q;  // fragA of sum_c q_t k_s exp(G_t - G_s), s <= t
};

// One level of the pair tree: tiles of 2HF tokens, t in the upper and s in
// the lower half of one tile.  P(t) = gates from the start of t's half through
// t, S(s) = gates after s to the end of s's half; exp(G_t - G_s) = P(t) S(s).
// Products along the tokens are segmented scans across the 16 lanes of the
// row (lane lc = token).
template <int HF>
__device__ __forceinline__ void tree_level(const float (&a)[8], const float (&kf)[8], const float (&qf)[8], int lc,
                                           int lg, DiagTiles& r) {
  const int pos = lc & (HF - 1);
  const bool upper = ((lc / HF) & 1) != 0;
  f16x8 L, Lq, R;
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    // every shift is taken in all lanes first (see row_shr), then selected
    float P = a[c], Si = a[c];
    if (HF >= 2) {
      const float up = row_shr<1>(P, 1.f), dn = row_shl<1>(Si, 1.f);
      P *= pos >= 1 ? up : 1.f;
      Si *= pos + 1 < HF ? dn : 1.f;
    }
    if (HF >= 4) {
      const float up = row_shr<2>(P, 1.f), dn = row_shl<2>(Si, 1.f);
      P *= pos >= 2 ? up : 1.f;
      Si *= pos + 2 < HF ? dn : 1.f;
    }
    if (HF >= 8) {
      const float up = row_shr<4>(P, 1.f), dn = row_shl<4>(Si, 1.f);
      P *= pos >= 4 ? up : 1.f;
      Si *= pos + 4 < HF ? dn : 1.f;
    }
    float S = 1.f;  // exclusive of s
    if (HF >= 2) {
      const float nx = row_shl<1>(Si, 1.f);
      S = pos + 1 < HF ? nx : 1.f;
    }
    L[c] = (f16)(upper ? kf[c] * P : 0.f);
    Lq[c] = (f16)(upper ? qf[c] * P : 0.f);
    R[c] = (f16)(upper ? 0.f : kf[c] * S);
  }
  const f32x4 ta = mfma32(R, L, zero4());   // (t = lc, s = 4lg+e)
  const f32x4 tb = mfma32(L, R, zero4());   // (t = 4lg+e, s = lc)
  const f32x4 tq = mfma32(R, Lq, zero4());  // (t = lc, s = 4lg+e)
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    if ((lc ^ (4 * lg + e)) < 2 * HF) {  // t and s in one tile of this level
      r.a[e] += ta[e];
      r.b[e] += tb[e];
      r.q[e] += tq[e];
    }
  }
}

// The diagonal tiles of block I (tokens 16I .. 16I+15 of the chunk starting at
// token tok0, nv of them valid) for chunks with strong decays: every pair
// s < t of the block belongs to exactly one level (the tile of 2HF tokens, HF
// = 8, 4, 2, 1, that has t in its upper and s in its lower half), and every
// operand is an input times products of gates <= 1, so nothing overflows for
// any gate (-inf included) and small values only lose what is negligible.
// k, q and log_g are read again here (rows past nv read zeros: identity
// tokens); ik, iq scale k and q (the L2 normalisation, else 1).
__device__ __noinline__ DiagTiles diag_tree(const bf16_t* qg, const bf16_t* kg, const float* lgg, size_t tok0,
                                            int nv, int H, int h, int I, float ik, float iq) {
  const int lane = threadIdx.x & 63, lc = lane & 15, lg = lane >> 4;
  const uint32_t rs = static_cast<uint32_t>(H * D);
  const size_t base = (tok0 * H + h) * D;
  const uint32_t nrow = static_cast<uint32_t>(nv);
  const __amdgpu_buffer_rsrc_t rg = buffer_rsrc(lgg + base, nrow * rs * 4u);
  const __amdgpu_buffer_rsrc_t rk = buffer_rsrc(kg + base, nrow * rs * 2u);
  const __amdgpu_buffer_rsrc_t rq = buffer_rsrc(qg + base, nrow * rs * 2u);
  DiagTiles r{zero4(), zero4(), zero4()};
  float qk = 0.f;
#pragma unroll 1
  for (int ks = 0; ks < 4; ++ks) {
    const uint32_t off = static_cast<uint32_t>(16 * I + lc) * rs + static_cast<uint32_t>(32 * ks + 8 * lg);
    const float4 g0 = __builtin_bit_cast(float4, buffer_load16(rg, off * 4u));
    const float4 g1 = __builtin_bit_cast(float4, buffer_load16(rg, off * 4u + 16u));
    const uint4 kw = buffer_load16(rk, off * 2u), qw = buffer_load16(rq, off * 2u);
    const float gv[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
    const uint32_t kk[4] = {kw.x, kw.y, kw.z, kw.w}, qq[4] = {qw.x, qw.y, qw.z, qw.w};
    float a[8], kf[8], qf[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      a[c] = exp_fast(gv[c]);
      kf[c] = ((c & 1) ? bf16_hi(kk[c >> 1]) : bf16_lo(kk[c >> 1])) * ik;
      qf[c] = ((c & 1) ? bf16_hi(qq[c >> 1]) : bf16_lo(qq[c >> 1])) * iq;
      qk += qf[c] * kf[c];
    }
    tree_level<8>(a, kf, qf, lc, lg, r);
    tree_level<4>(a, kf, qf, lc, lg, r);
    tree_level<2>(a, kf, qf, lc, lg, r);
    tree_level<1>(a, kf, qf, lc, lg, r);
  }
  // the pairs t = s of Aqk: q_t . k_t, summed over the four channel groups
  qk += __shfl_xor(qk, 16, 64);
  qk += __shfl_xor(qk, 32, 64);
#pragma unroll
  for (int e = 0; e < 4; ++e) r.q[e] += (4 * lg + e) == lc ? qk : 0.f;
  return r;
}

template <bool L2>
__global__ void __launch_bounds__(NTP) __attribute__((amdgpu_waves_per_eu(4))) prep_kernel(PrepArgs p) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  PrepSmem& sm = *reinterpret_cast<PrepSmem*>(smem_raw);

  const int H = p.H;
  const int cs = blockIdx.x / H;
  const int h = blockIdx.x - cs * H;
  size_t tok_begin;
  int ntok, ck;
  if (p.table) {
    const int doc = p.table[cs];
    if (doc < 0) return;
    ck = cs - p.cstart[doc];
    tok_begin = p.cu_seqlens[doc];
    ntok = p.cu_seqlens[doc + 1] - p.cu_seqlens[doc];
  } else {
    const int doc = cs / p.nchd;
    ck = cs - doc * p.nchd;
    tok_begin = static_cast<size_t>(doc) * p.T;
    ntok = p.T;
  }
  const int nv = min(C, ntok - ck * C);
  const size_t tok0 = tok_begin + static_cast<size_t>(ck) * C;
  unsigned char* slot = p.ws + (static_cast<size_t>(cs) * H + h) * SLOT_BYTES;

  const int tid = threadIdx.x, lane = tid & 63, lc = lane & 15, lg = lane >> 4;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index 0..7, uniform (SGPR)
  // stage A: wave w covers block IA = w/2 (rows 16IA .. 16IA+15) and channel
  // half w%2; lane (qt, oct) = (lane%8, lane/8) owns rows r0 = 16IA+2qt, r0+1
  // and channels c8 .. c8+7.  The eight row pairs of a channel octet are eight
  // adjacent lanes, so products over them are DPP row shifts.
  const int IA = w >> 1;
  const int qt = lane & 7;
  const int oct = lane >> 3;
  const int c8 = 64 * (w & 1) + 8 * oct;
  const int r0 = 16 * IA + 2 * qt;
  const float lim_lo = __expf(-HALF_SPAN_MAX);
  bool bad = false;
  bool strong = false;  // a half block of this thread's channels decays beyond HALF_SPAN_MAX

  // ---------------- phase 1: loads and stage A (this thread: 2 rows x 8 channels)
  float4 g[2][2];
  uint4 kr[2], qr[2], vr[2];
  float bt[2];
  {
    // range-checked loads over the chunk's nv valid rows: rows past a
    // document's end read zeros, i.e. identity tokens (k = 0, beta = 0, log_g = 0)
    const uint32_t rs = static_cast<uint32_t>(H * D);  // row stride, elements
    const size_t base = (tok0 * H + h) * D;
    const uint32_t nrow = static_cast<uint32_t>(nv);
    const __amdgpu_buffer_rsrc_t rg = buffer_rsrc(p.log_g + base, nrow * rs * 4u);
    const __amdgpu_buffer_rsrc_t rk = buffer_rsrc(p.k + base, nrow * rs * 2u);
    const __amdgpu_buffer_rsrc_t rq = buffer_rsrc(p.q + base, nrow * rs * 2u);
    const __amdgpu_buffer_rsrc_t rv = buffer_rsrc(p.v + base, nrow * rs * 2u);
    const __amdgpu_buffer_rsrc_t rb = buffer_rsrc(p.beta + tok0 * H + h, nrow * static_cast<uint32_t>(H) * 4u);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const uint32_t row = static_cast<uint32_t>(r0 + j);
      const uint32_t off = row * rs + static_cast<uint32_t>(c8);
      g[j][0] = __builtin_bit_cast(float4, buffer_load16(rg, off * 4u));
      g[j][1] = __builtin_bit_cast(float4, buffer_load16(rg, off * 4u + 16u));
      kr[j] = buffer_load16(rk, off * 2u);
      qr[j] = buffer_load16(rq, off * 2u);
      vr[j] = buffer_load16(rv, off * 2u);
      bt[j] = buffer_load_f32(rb, row * static_cast<uint32_t>(H) * 4u);
    }
  }
  {
    u16x2 mk = {0, 0}, mv = {0, 0};
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const uint32_t kw[4] = {kr[j].x, kr[j].y, kr[j].z, kr[j].w};
      const uint32_t qw[4] = {qr[j].x, qr[j].y, qr[j].z, qr[j].w};
      const uint32_t vw[4] = {vr[j].x, vr[j].y, vr[j].z, vr[j].w};
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        mk = __builtin_elementwise_max(mk, __builtin_bit_cast(u16x2, kw[x] & 0x7fff7fffu));
        mk = __builtin_elementwise_max(mk, __builtin_bit_cast(u16x2, qw[x] & 0x7fff7fffu));
        mv = __builtin_elementwise_max(mv, __builtin_bit_cast(u16x2, vw[x] & 0x7fff7fffu));
      }
      bad |= !(fabsf(bt[j]) <= BETA_MAX);
    }
    // normalised q and k rows are at most 1 in magnitude: only v is bounded then
    if (!L2) bad |= mk[0] > QK_MAX_BITS || mk[1] > QK_MAX_BITS;
    bad |= mv[0] > V_MAX_BITS || mv[1] > V_MAX_BITS;
  }
  // L2 normalisation: 1/|k| and 1/|q| of rows r0, r0+1.  A row's channels sit
  // in the eight oct lanes of this wave and of its partner wave w^1 (the other
  // channel half): a shuffle reduction, then one exchange through LDS.
  float ikr[2] = {1.f, 1.f}, iqr[2] = {1.f, 1.f};
  if (L2) {
    float kk[2], qq[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const uint32_t kw[4] = {kr[j].x, kr[j].y, kr[j].z, kr[j].w};
      const uint32_t qw[4] = {qr[j].x, qr[j].y, qr[j].z, qr[j].w};
      float a = 0.f, b = 0.f;
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        const float k0 = bf16_lo(kw[x]), k1 = bf16_hi(kw[x]), q0 = bf16_lo(qw[x]), q1 = bf16_hi(qw[x]);
        a += k0 * k0 + k1 * k1;
        b += q0 * q0 + q1 * q1;
      }
#pragma unroll
      for (int o = 8; o < 64; o <<= 1) {  // over the eight channel octets
        a += __shfl_xor(a, o, 64);
        b += __shfl_xor(b, o, 64);
      }
      kk[j] = a;
      qq[j] = b;
    }
    if (oct == 0) {
#pragma unroll
      for (int j = 0; j < 2; ++j) sm.nrm[w & 1][r0 + j] = make_float2(kk[j], qq[j]);
    }
    lds_barrier();
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const float2 o = sm.nrm[(w & 1) ^ 1][r0 + j];
      ikr[j] = __frsqrt_rn(kk[j] + o.x + L2_EPS);
      iqr[j] = __frsqrt_rn(qq[j] + o.y + L2_EPS);
    }
  }
  f16x8 hl[2], hr[2], xv[2];  // k exp(G - R), k exp(R' - G), beta v of rows r0, r0+1
  {
    // two passes of four channels keep the live registers down
#pragma unroll
    for (int hc = 0; hc < 2; ++hc) {
      float tot4[4];
      f16x4 fdl4, fdr4, hq4[2];
#pragma unroll
      for (int cc = 0; cc < 4; ++cc) {
        const int c = 4 * hc + cc;
        const float4 ga = g[0][hc], gb4 = g[1][hc];
        const float a0 = exp_fast(cc == 0 ? ga.x : cc == 1 ? ga.y : cc == 2 ? ga.z : ga.w);
        const float a1 = exp_fast(cc == 0 ? gb4.x : cc == 1 ? gb4.y : cc == 2 ? gb4.z : gb4.w);
        const float pr = a0 * a1;
        // inclusive prefix (x) and suffix (y) products over the block's eight
        // row pairs (lanes qt = 0..7 of this octet; every shift is taken in
        // all lanes first, then selected)
        float x = pr, y = pr, t;
        t = row_shr<1>(x, 1.f); x = qt >= 1 ? x * t : x;
        t = row_shr<2>(x, 1.f); x = qt >= 2 ? x * t : x;
        t = row_shr<4>(x, 1.f); x = qt >= 4 ? x * t : x;
        t = row_shl<1>(y, 1.f); y = qt <= 6 ? y * t : y;
        t = row_shl<2>(y, 1.f); y = qt <= 5 ? y * t : y;
        t = row_shl<4>(y, 1.f); y = qt <= 3 ? y * t : y;
        const float xe = row_shr<1>(x, 1.f), ye = row_shl<1>(y, 1.f);
        const float E = qt >= 1 ? xe : 1.f;  // over the row pairs before this lane's
        const float F = qt <= 6 ? ye : 1.f;  // over the row pairs after it
        // broadcasts from row pairs 3 and 4 of this octet: swizzle bit masks
        // (lane & 0x18) | 3 and | 4, immediates instead of address registers
        const float dl = __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, x), 0x78));
        const float dr = __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, y), 0x98));
        const float Pv[2] = {E * a0, E * pr};
        const float Sv[2] = {a1 * F, F};
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const uint32_t kw = c < 2 ? kr[j].x : c < 4 ? kr[j].y : c < 6 ? kr[j].z : kr[j].w;
          const uint32_t qw = c < 2 ? qr[j].x : c < 4 ? qr[j].y : c < 6 ? qr[j].z : qr[j].w;
          const uint32_t vw = c < 2 ? vr[j].x : c < 4 ? vr[j].y : c < 6 ? vr[j].z : vr[j].w;
          const float kv = ((c & 1) ? bf16_hi(kw) : bf16_lo(kw)) * ikr[j];
          const float qv = ((c & 1) ? bf16_hi(qw) : bf16_lo(qw)) * iqr[j];
          const float vv = (c & 1) ? bf16_hi(vw) : bf16_lo(vw);
          hl[j][c] = (f16)(kv * Pv[j]);
          hq4[j][cc] = (f16)(qv * Pv[j]);
          hr[j][c] = (f16)(kv * Sv[j]);
          xv[j][c] = (f16)(bt[j] * vv);
        }
        strong |= (dl < lim_lo) | (dr < lim_lo);
        bad |= (dl != dl) | (dr != dr);
        tot4[cc] = dl * dr;
        // the reciprocals only feed fp16 factors: the hardware estimate is enough
        fdl4[cc] = (f16)__builtin_amdgcn_rcpf(fmaxf(dl, lim_lo));
        fdr4[cc] = (f16)__builtin_amdgcn_rcpf(fmaxf(dr, lim_lo));
      }
      const int cb = c8 + 4 * hc;
      if (qt == 0) {
        *reinterpret_cast<float4*>(&sm.tot[IA][cb]) = make_float4(tot4[0], tot4[1], tot4[2], tot4[3]);
        *reinterpret_cast<f16x4*>(&sm.fDl[IA][cb]) = fdl4;
        *reinterpret_cast<f16x4*>(&sm.fDr[IA][cb]) = fdr4;
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) *reinterpret_cast<f16x4*>(&sm.Ql[r0 + j][cb]) = hq4[j];
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      *reinterpret_cast<f16x8*>(&sm.u.a.Kl[r0 + j][c8]) = hl[j];
      *reinterpret_cast<f16x8*>(&sm.u.a.Kr[r0 + j][c8]) = hr[j];
    }
    if ((w & 1) == 0 && oct == 0) *reinterpret_cast<float2*>(&sm.beta[r0]) = make_float2(bt[0], bt[1]);
    const bool any_strong = __builtin_amdgcn_ballot_w64(strong) != 0;
    if (lane == 0) sm.strong[w] = any_strong;
  }
  // the checks so far as a wave mask now: a per-lane flag evaluated at the
  // end would keep their inputs live through the products
  const uint64_t bad_a = __builtin_amdgcn_ballot_w64(bad);
  asm volatile("" ::"s"(bad_a));
  bad = false;
  lds_barrier();
  // workgroup-uniform: the diagonal tiles of this chunk come from the pair tree
  const bool tree = (sm.strong[0] | sm.strong[1] | sm.strong[2] | sm.strong[3] | sm.strong[4] | sm.strong[5] |
                     sm.strong[6] | sm.strong[7]) != 0;

  // ---------------- phase 2: K exp(gamma - G) out, Xk, products
  {
    f16* kdt = reinterpret_cast<f16*>(slot + OFF_KDT);
    // Kd^T[dk][tok] for dk = c8+c, tok = r0, r0+1: row block dk/16, k-step
    // tok/32 = IA/2, lane (lg = tok%32/8, lc = dk%16), positions tok%8 .. +1
    const int lgk = 2 * (IA & 1) + (qt >> 2);
#pragma unroll
    for (int hc = 0; hc < 2; ++hc) {
      const int cb = c8 + 4 * hc;
      float4 T[4];
#pragma unroll
      for (int I = 0; I < 4; ++I) T[I] = *reinterpret_cast<const float4*>(&sm.tot[I][cb]);
      float gam[4];
#pragma unroll
      for (int cc = 0; cc < 4; ++cc) {
        const int c = 4 * hc + cc;
        const float t0 = cc == 0 ? T[0].x : cc == 1 ? T[0].y : cc == 2 ? T[0].z : T[0].w;
        const float t1 = cc == 0 ? T[1].x : cc == 1 ? T[1].y : cc == 2 ? T[1].z : T[1].w;
        const float t2 = cc == 0 ? T[2].x : cc == 1 ? T[2].y : cc == 2 ? T[2].z : T[2].w;
        const float t3 = cc == 0 ? T[3].x : cc == 1 ? T[3].y : cc == 2 ? T[3].z : T[3].w;
        const float e1 = t0, e2 = e1 * t1, e3 = e2 * t2;
        const float fr = IA == 0 ? 1.f : IA == 1 ? e1 : IA == 2 ? e2 : e3;      // exp(R_IA)
        const float gd = IA == 0 ? t1 * t2 * t3 : IA == 1 ? t2 * t3             // exp(gamma - R_{IA+1})
                       : IA == 2 ? t3 : 1.f;
        gam[cc] = e3 * t3;
        const int dk = c8 + c;
        f16x2 kd;
        kd[0] = (f16)((float)hr[0][c] * gd);
        kd[1] = (f16)((float)hr[1][c] * gd);
        *reinterpret_cast<f16x2*>(kdt + (((dk >> 4) * 2 + (IA >> 1)) * 64 + 16 * lgk + (dk & 15)) * 8 + 2 * (qt & 3)) = kd;
        // Xk = beta k exp(G) = beta Kl exp(R_IA), kept in registers until the
        // products have released Kl / Kr
#pragma unroll
        for (int j = 0; j < 2; ++j) hl[j][c] = (f16)((float)hl[j][c] * bt[j] * fr);
      }
      if (IA == 0 && qt == 0)
        *reinterpret_cast<float4*>(reinterpret_cast<float*>(slot + OFF_GAM) + cb) = make_float4(gam[0], gam[1], gam[2], gam[3]);
    }
    // materialise Xk here: sunk below the products, its factors would stay live there
#pragma unroll
    for (int j = 0; j < 2; ++j) asm volatile("" : "+v"(hl[j]));
  }
  f16x4 tbd;  // fragB(T_ww), waves 0-3
  int item0 = 0, nitem = 0;
  if (w < 4) {
    // diagonal block I = w of A in both layouts, and its inverse
    const int I = w;
    f32x4 accA = zero4(), accB = zero4();
    if (tree) {
      float ik = 1.f, iq = 1.f;
      if (L2) {
        const float2 n0 = sm.nrm[0][16 * I + lc], n1 = sm.nrm[1][16 * I + lc];
        ik = __frsqrt_rn(n0.x + n1.x + L2_EPS);
        iq = __frsqrt_rn(n0.y + n1.y + L2_EPS);
      }
      const DiagTiles dt = diag_tree(p.q, p.k, p.log_g, tok0, nv, H, h, I, ik, iq);
      accA = dt.a;
      accB = dt.b;
      // Aqk_II (the item list skips it on this path)
      float amax = 0.f;
      f16x4 res;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float x = (4 * lg + e) <= lc ? p.scale * dt.q[e] : 0.f;
        amax = fmaxf(amax, fabsf(x));
        res[e] = (f16)x;
      }
      bad |= !(amax <= F16_SAFE);
      __builtin_nontemporal_store(res, reinterpret_cast<f16x4*>(reinterpret_cast<f16*>(slot + OFF_AS) +
                                                                frag_pos(I, I, 2, lane)));
    } else {
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const int kc = 32 * ks + 8 * lg;
        const f16x8 ls = ld8(&sm.u.a.Kl[16 * I + lc][kc]) * ld8(&sm.fDl[I][kc]);
        const f16x8 rs = ld8(&sm.u.a.Kr[16 * I + lc][kc]) * ld8(&sm.fDr[I][kc]);
        accA = mfma32(rs, ls, accA);  // fragA: rows 16I+lc, cols 16I+4lg+e
        accB = mfma32(ls, rs, accB);  // fragB: rows 16I+4lg+e, cols 16I+lc
      }
    }
    f16x4 a, b;
    const float bA = sm.beta[16 * I + lc];
    const float4 bB4 = *reinterpret_cast<const float4*>(&sm.beta[16 * I + 4 * lg]);
    const float bB[4] = {bB4.x, bB4.y, bB4.z, bB4.w};
    float lmax = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float la = (4 * lg + e) < lc ? bA * accA[e] : 0.f;
      const float lb = lc < (4 * lg + e) ? bB[e] * accB[e] : 0.f;
      lmax = fmaxf(lmax, fabsf(la));
      a[e] = (f16)la;
      b[e] = (f16)lb;
    }
    bad |= !(lmax <= 1.0f);
    // (I + L)^-1 = (I - L)(I + L^2)(I + L^4)(I + L^8), in both layouts
    const f16x4 b2 = h4(mfma16(a, b, zero4()));
    const f16x4 a2 = h4(mfma16(b, a, zero4()));
    const f16x4 b4 = h4(mfma16(a2, b2, zero4()));
    const f16x4 a4 = h4(mfma16(b2, a2, zero4()));
    const f16x4 b8 = h4(mfma16(a4, b4, zero4()));
    const f16x4 a8 = h4(mfma16(b4, a4, zero4()));
    f32x4 ta, tb;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float id = lc == 4 * lg + e ? 1.f : 0.f;
      ta[e] = id - (float)a[e];
      tb[e] = id - (float)b[e];
    }
    ta = mfma16(b2, h4(ta), ta);
    ta = mfma16(b4, h4(ta), ta);
    ta = mfma16(b8, h4(ta), ta);
    tb = mfma16(a2, h4(tb), tb);
    tb = mfma16(a4, h4(tb), tb);
    tb = mfma16(a8, h4(tb), tb);
    float tmax = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) tmax = fmaxf(tmax, fabsf(ta[e]));
    bad |= !(tmax <= F16_SAFE);
    sm.frag[S_TD + I][lane] = h4(ta);
    tbd = h4(tb);
    item0 = 12 + w;  // one of the last four tiles (Aqk row block 3)
    nitem = 1;
  } else {
    item0 = 3 * (w - 4);  // three of the first twelve tiles
    nitem = 3;
  }
  // the sixteen remaining tiles: A_IJ (I > J) and Aqk_IJ (J <= I)
#pragma unroll 1
  for (int m = 0; m < nitem; ++m) {
    const int item = item0 + m;
    const bool isq = item >= 6;
    int I, J;
    if (!isq) {  // pairs (1,0) (2,0) (2,1) (3,0) (3,1) (3,2)
      I = item >= 3 ? 3 : item >= 1 ? 2 : 1;
      J = item - pair6(I, 0);
    } else {
      const int t = item - 6;
      I = t >= 6 ? 3 : t >= 3 ? 2 : t >= 1 ? 1 : 0;
      J = t - tile10(I, 0);
      if (tree && I == J) continue;  // the diagonal waves wrote it (wave-uniform)
    }
    const f16(*L)[LDK] = isq ? sm.Ql : sm.u.a.Kl;
    f32x4 acc = zero4();
    f16x8 l[4], r[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int kc = 32 * ks + 8 * lg;
      l[ks] = ld8(&L[16 * I + lc][kc]);
      r[ks] = ld8(&sm.u.a.Kr[16 * J + lc][kc]);
    }
    if (I == J) {
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const int kc = 32 * ks + 8 * lg;
        l[ks] = l[ks] * ld8(&sm.fDl[I][kc]);
        r[ks] = r[ks] * ld8(&sm.fDr[I][kc]);
      }
    } else if (I - J >= 2) {
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) l[ks] = l[ks] * off_factor(sm, I, J, 32 * ks + 8 * lg);
    }
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) acc = mfma32(r[ks], l[ks], acc);  // fragA: rows 16I+lc, cols 16J+4lg+e
    f16x4 res;
    if (!isq) {
      const float bA = sm.beta[16 * I + lc];
#pragma unroll
      for (int e = 0; e < 4; ++e) res[e] = (f16)(bA * acc[e]);
      sm.frag[S_AO + pair6(I, J)][lane] = res;
    } else {  // As = scale Aqk, straight to the slot
      float amax = 0.f;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float x = (16 * J + 4 * lg + e) <= (16 * I + lc) ? p.scale * acc[e] : 0.f;
        amax = fmaxf(amax, fabsf(x));
        res[e] = (f16)x;
      }
      bad |= !(amax <= F16_SAFE);
      __builtin_nontemporal_store(res, reinterpret_cast<f16x4*>(reinterpret_cast<f16*>(slot + OFF_AS) +
                                                                frag_pos(I, J, 2, lane)));
    }
  }
  lds_barrier();

  // ---------------- phase 3: Xk^T, Xv^T into LDS; waves 0-3: column w of T;
  // waves 0-5: one of the six zero tiles of As above the diagonal
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    f16x2 xk2, xv2;
    xk2[0] = hl[0][c]; xk2[1] = hl[1][c];
    xv2[0] = xv[0][c]; xv2[1] = xv[1][c];
    *reinterpret_cast<f16x2*>(&sm.u.x.XkT[c8 + c][r0]) = xk2;
    *reinterpret_cast<f16x2*>(&sm.u.x.XvT[c8 + c][r0]) = xv2;
  }
  // As above its diagonal: tiles (0,1) and (2,3) share their 32-token
  // fragments with nonzero tiles and are written as zeros; the fragments of
  // row blocks 0 and 1 over tokens 32..63 are all zero, never written, and
  // never read by the scans
  if (w < 2) {
    const int zi = 2 * w, zj = zi + 1;
    f16x4 z;
#pragma unroll
    for (int e = 0; e < 4; ++e) z[e] = (f16)0.f;
    __builtin_nontemporal_store(z, reinterpret_cast<f16x4*>(reinterpret_cast<f16*>(slot + OFF_AS) +
                                                          frag_pos(zi, zj, 2, lane)));
  }
  switch (w) {
    case 0: bad |= t_column<0>(sm, tbd, lane); break;
    case 1: bad |= t_column<1>(sm, tbd, lane); break;
    case 2: bad |= t_column<2>(sm, tbd, lane); break;
    case 3: bad |= t_column<3>(sm, tbd, lane); break;
    default: break;
  }
  lds_barrier();

  // ---------------- phase 4: W, U, Qs for value / key columns 16w .. 16w+15
  {
    f16* nw = reinterpret_cast<f16*>(slot + OFF_NW);
    f16* qs = reinterpret_cast<f16*>(slot + OFF_QS);
    f16* up = reinterpret_cast<f16*>(slot + OFF_UP);
    float omax = 0.f;
    const int n = w;
    f16x4 xk[4], xvv[4];
#pragma unroll
    for (int J = 0; J < 4; ++J) {
      xk[J] = ld4(&sm.u.x.XkT[16 * n + lc][16 * J + 4 * lg]);
      xvv[J] = ld4(&sm.u.x.XvT[16 * n + lc][16 * J + 4 * lg]);
    }
    // exp(R_I) of columns 16n+4lg .. +3
    const float4 e0 = *reinterpret_cast<const float4*>(&sm.tot[0][16 * n + 4 * lg]);
    const float4 e1 = *reinterpret_cast<const float4*>(&sm.tot[1][16 * n + 4 * lg]);
    const float4 e2 = *reinterpret_cast<const float4*>(&sm.tot[2][16 * n + 4 * lg]);
    const float R1[4] = {e0.x, e0.y, e0.z, e0.w};
    const float R2[4] = {R1[0] * e1.x, R1[1] * e1.y, R1[2] * e1.z, R1[3] * e1.w};
    const float R3[4] = {R2[0] * e2.x, R2[1] * e2.y, R2[2] * e2.z, R2[3] * e2.w};
#pragma unroll
    for (int I = 0; I < 4; ++I) {
      f32x4 aW = zero4(), aU = zero4(), aQ;  // aQ: Qs^T [col 4lg+e][tok lc]
      const f16x4 ql = ld4(&sm.Ql[16 * I + lc][16 * n + 4 * lg]);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float rI = I == 0 ? 1.f : I == 1 ? R1[e] : I == 2 ? R2[e] : R3[e];
        aQ[e] = p.scale * (float)ql[e] * rI;
      }
#pragma unroll
      for (int J = 0; J <= I; ++J) {
        const f16x4 tf = I == J ? sm.frag[S_TD + I][lane] : sm.frag[S_TO + pair6(I, J)][lane];
        aW = mfma16(xk[J], tf, aW);   // W^T     [col 4lg+e][tok lc]
        aU = mfma16(xvv[J], tf, aU);  // U^T     [col 4lg+e][tok lc]
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        omax = fmaxf(omax, fmaxf(fmaxf(fabsf(aW[e]), fabsf(aU[e])), fabsf(aQ[e])));
        aW[e] = -aW[e];
      }
      // X[tok 16I+lc][col 16n+4lg+e]: block I, k-step n/2, lane
      // (lg' = 2(n&1) + lg/2, lc), position 4(lg&1)+e
      const int rowoff = ((I * 4 + (n >> 1)) * 64 + 16 * (2 * (n & 1) + (lg >> 1)) + lc) * 8 + 4 * (lg & 1);
      // whole 128-byte lines per instruction (512 contiguous bytes), stored
      // nontemporally: the scan reads them long after this kernel
      __builtin_nontemporal_store(h4(aW), reinterpret_cast<f16x4*>(nw + rowoff));
      __builtin_nontemporal_store(h4(aQ), reinterpret_cast<f16x4*>(qs + rowoff));
      // U in the order one scan lane consumes it (same lane here): this
      // wave's 16 columns are half b = n & 1 of tile n / 2, 512 contiguous
      // bytes, stored like W and Qs
      const int laneoff = (((I * NTILE + (n >> 1)) * 2 + (n & 1)) * 64 + lane) * 4;
      __builtin_nontemporal_store(h4(aU), reinterpret_cast<f16x4*>(up + laneoff));
    }
    bad |= !(omax <= F16_SAFE);
  }
  // one "not on the fast path" byte per wave
  const bool any = (__builtin_amdgcn_ballot_w64(bad) | bad_a) != 0;
  if (lane == 0) slot[OFF_FLAG + w] = any ? 1 : 0;
}

// ---------------------------------------------------------------------------
// Pass 2: the serial state scan.

// U of token block I, column tile `tile`, as one scan lane holds it: [b][e] =
// U[16I+lc][32tile+16b+4lg+e], its two halves 512 bytes apart in the slot.
__device__ __forceinline__ f16x8 ld_up(const unsigned char* sl, int I, int tile, int lane) {
  const f16* up = reinterpret_cast<const f16*>(sl + OFF_UP) + ((I * NTILE + tile) * 2 * 64 + lane) * 4;
  const f16x4 lo = *reinterpret_cast<const f16x4*>(up), hi = *reinterpret_cast<const f16x4*>(up + 64 * 4);
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

struct ScanArgs {
  const bf16_t* q;
  const bf16_t* k;
  const bf16_t* v;
  const float* log_g;
  const float* beta;
  const float* init_state;
  float* final_state;
  const int32_t* cu_seqlens;  // null: dense
  const int32_t* cstart;      // packed: first chunk slot of each document
  const int32_t* order;       // null: identity document order
  const unsigned char* ws;    // chunk slots
  void* out;                  // fp32, or bf16 when out_bf16
  bool out_bf16;
  bool l2;                    // q / k rows L2-normalised (the fallback normalises its own)
  int num_docs;
  int T;
  int H;
  int nchd;
  int n_slots;                // chunk slots per head in the workspace
  float scale;
};

constexpr int NTS = 512;  // scan threads: 8 waves

struct __align__(16) ScanSmem {
  f16 ST[DVT][LDK];   // S^T (fp16) [value col][key row]
  f16 DT[DVT][LDT];   // Delta^T    [value col][token]
  f16 DTX[DVT][LDT];  // where the output waves' copy of that store lands (never read)
  fb::Stage<8> fb;
  int sbp[8];         // per wave: state beyond the fast-path bound
  int dbp[8];         // per wave: Delta beyond the fp16 bound (output waves: unused)
};

// Slot operands of one chunk as one scan thread uses them.  Waves 0-3 form
// Delta rows 16w.. (m = -W rows); waves 4-7 form output rows 16(w-4)..
// (m = Qs rows, then As rows against Delta); every wave updates key rows
// 16w.. .  Both kinds run the same instruction stream (transposed products
// [col][token]); only their operands and the targets of their stores differ,
// and each kind skips the one load it has no use for (a wave-uniform branch).
struct Pre {
  f16x8 m[4];       // -W or Qs row 16I+lc, key cols 32ks+8lg ..
  f16x8 u;          // U of this lane, [b][e] (Delta waves)
  f16x8 kd[2];      // Kd^T row 16w+lc, tokens 32ks+8lg ..
  f16x8 as[2];      // As row 16I+lc, tokens 32ks+8lg .. (output waves)
  float4 gam;       // exp(gamma) of key rows 16w+4lg ..
  int2 flag;        // the eight per-wave bytes of the prep kernel
};

struct State2 {
  f32x4 s0, s1;
};

// The token-by-token evaluation of one chunk, out of line: its scattered
// loads and waits stay out of the scan loop's wait-count bookkeeping.
__device__ __noinline__ State2 scan_fallback(fb::Stage<8>& st, State2 in, const fb::Args fa, size_t tok_begin,
                                             int ntok, int k, int h, int col0) {
  f32x4 s[1][2] = {{in.s0, in.s1}};
  fb::eval_chunk<8>(st, s, fa, tok_begin, ntok, k, h, col0);
  return State2{s[0][0], s[0][1]};
}

__global__ void __launch_bounds__(NTS, 1) scan_kernel(ScanArgs p) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  ScanSmem& sm = *reinterpret_cast<ScanSmem*>(smem_raw);

  const int num_units = p.num_docs * p.H;
  const int grp = blockIdx.x / (8 * NTILE);
  const int rem = blockIdx.x - grp * 8 * NTILE;
  const int tile = rem / 8;
  const int u = grp * 8 + (rem & 7);  // rank of the unit (longest documents first)
  if (u >= num_units) return;
  const int H = p.H;
  const int rank = u / H;
  const int h = u - rank * H;
  const int doc = p.order ? p.order[rank] : rank;
  const int col0 = tile * DVT;
  size_t tok_begin;
  int ntok, cbase;
  if (p.cu_seqlens) {
    tok_begin = p.cu_seqlens[doc];
    ntok = p.cu_seqlens[doc + 1] - p.cu_seqlens[doc];
    cbase = p.cstart[doc];
  } else {
    tok_begin = static_cast<size_t>(doc) * p.T;
    ntok = p.T;
    cbase = doc * p.nchd;
  }
  const int nch = (ntok + C - 1) / C;
  if (cbase + nch > p.n_slots) return;  // malformed cu_seqlens: never read past the workspace
  const size_t unit_state = (static_cast<size_t>(doc) * H + h) * D * D;
  const unsigned char* slot0 = p.ws + (static_cast<size_t>(cbase) * H + h) * SLOT_BYTES;
  const size_t slot_stride = static_cast<size_t>(H) * SLOT_BYTES;

  const int tid = threadIdx.x, lane = tid & 63, lc = lane & 15, lg = lane >> 4;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, uniform (SGPR)
  const bool is_o = w >= 4;     // output wave (else Delta wave)
  const int I = w & 3;          // token block of the Delta / output rows

  // Loads of chunk k's operands, in three groups: the flag (used first), the
  // Delta / output operands (phase A) and the state-update operands (phase B).
  auto slot_of = [&](int k) { return slot0 + static_cast<size_t>(k) * slot_stride; };
  auto load_flag = [&](int k, Pre& r) { r.flag = *reinterpret_cast<const int2*>(slot_of(k) + OFF_FLAG); };
  auto load_a = [&](int k, Pre& r) {
    const unsigned char* sl = slot_of(k);
    const f16* mp = reinterpret_cast<const f16*>(sl + (is_o ? OFF_QS : OFF_NW)) + (I * 4 * 64 + lane) * 8;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) r.m[ks] = ld8(mp + ks * 64 * 8);
    if (!is_o) r.u = ld_up(sl, I, tile, lane);
    else r.u = f16x8{};
  };
  auto load_b = [&](int k, Pre& r) {
    const unsigned char* sl = slot_of(k);
    const f16* kd = reinterpret_cast<const f16*>(sl + OFF_KDT) + (w * 2 * 64 + lane) * 8;
    const f16* as = reinterpret_cast<const f16*>(sl + OFF_AS) + (I * 2 * 64 + lane) * 8;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) r.kd[ks] = ld8(kd + ks * 64 * 8);
    if (is_o) {
      r.as[0] = ld8(as);
      r.as[1] = I >= 2 ? ld8(as + 64 * 8) : f16x8{};  // row blocks 0, 1: zero past token 31
    } else {
      r.as[0] = r.as[1] = f16x8{};
    }
    r.gam = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(sl + OFF_GAM) + 16 * w + 4 * lg);
  };
  auto load = [&](int k, Pre& r) {
    load_flag(k, r);
    load_a(k, r);
    load_b(k, r);
    __builtin_amdgcn_sched_barrier(0);
  };

  // s[0][b][e] = S[16w+4lg+e][col0+16b+lc]
  auto write_st = [&](f32x4 (&s)[1][2]) {
    bool big = false;
#pragma unroll
    for (int b = 0; b < 2; ++b) {
#pragma unroll
      for (int e = 0; e < 4; ++e) big |= !(fabsf(s[0][b][e]) <= S_MAX);
      *reinterpret_cast<f16x4*>(&sm.ST[16 * b + lc][16 * w + 4 * lg]) = h4(s[0][b]);
    }
    const bool any = __builtin_amdgcn_ballot_w64(big) != 0;
    if (lane == 0) sm.sbp[w] = any;
  };

  f32x4 s[1][2];
#pragma unroll
  for (int b = 0; b < 2; ++b)
#pragma unroll
    for (int e = 0; e < 4; ++e)
      s[0][b][e] = p.init_state ? p.init_state[unit_state + (16 * w + 4 * lg + e) * D + col0 + 16 * b + lc] : 0.f;
  write_st(s);
  const fb::Args fa{p.q, p.k, p.v, p.log_g, p.beta, p.out, H, p.scale, p.out_bf16, p.l2};

  // One chunk: consume cur (chunk k); each group of cur's registers is
  // refilled with chunk k+2 right after its last use (clamped to the last
  // chunk, so every step issues the same loads), which gives each load
  // almost two steps to arrive without a third register buffer.
  auto step = [&](int k, Pre& cur) {
    const int kn = min(k + 2, nch - 1);
    const size_t tok0 = tok_begin + static_cast<size_t>(k) * C;
    const int nv = min(C, ntok - k * C);
    lds_barrier();  // ST of the entry state is complete
    const int pflag = __builtin_amdgcn_readfirstlane(cur.flag.x | cur.flag.y);
    // the load groups stay in program order (flag, phase A, phase B operands,
    // chunk after chunk), so the wait before each use counts exactly the
    // loads issued after it
    __builtin_amdgcn_sched_barrier(0);
    load_flag(kn, cur);
    __builtin_amdgcn_sched_barrier(0);
    const bool sbig = (sm.sbp[0] | sm.sbp[1] | sm.sbp[2] | sm.sbp[3] | sm.sbp[4] | sm.sbp[5] | sm.sbp[6] |
                       sm.sbp[7]) != 0;

    // ---- phase A: Delta^T = U^T + S^T (-W)^T (waves 0-3, into DT) and the
    // first part of O^T, S^T Qs^T (waves 4-7, kept), one instruction stream
    f16x8 sf[4][2];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int b = 0; b < 2; ++b) sf[ks][b] = ld8(&sm.ST[16 * b + lc][32 * ks + 8 * lg]);
    f16* dt = is_o ? &sm.DTX[0][0] : &sm.DT[0][0];
    bool dbig = false;
    f32x4 oacc[2];
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      f32x4 acc;
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[e] = is_o ? 0.f : (float)cur.u[4 * b + e];
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) acc = mfma32(sf[ks][b], cur.m[ks], acc);  // [col 4lg+e][tok lc]
      oacc[b] = acc;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        dbig |= !(fabsf(acc[e]) <= F16_SAFE);
        dt[(16 * b + 4 * lg + e) * LDT + 16 * I + lc] = (f16)acc[e];
      }
    }
    {
      const bool any = __builtin_amdgcn_ballot_w64(dbig) != 0;
      if (lane == 0) sm.dbp[w] = any;
    }
    __builtin_amdgcn_sched_barrier(0);
    load_a(kn, cur);
    __builtin_amdgcn_sched_barrier(0);
    lds_barrier();

    // ---- phase B: S = exp(gamma) S + Kd^T Delta (all waves, key rows 16w..),
    // then O^T += Delta^T As^T (waves 4-7, to out)
    const bool fbk = pflag != 0 || sbig || (sm.dbp[0] | sm.dbp[1] | sm.dbp[2] | sm.dbp[3]) != 0;
    if (!fbk) {  // workgroup-uniform
      f16x8 dB[2][2];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int b = 0; b < 2; ++b) dB[ks][b] = ld8(&sm.DT[16 * b + lc][32 * ks + 8 * lg]);
      const float gg[4] = {cur.gam.x, cur.gam.y, cur.gam.z, cur.gam.w};
#pragma unroll
      for (int b = 0; b < 2; ++b) {
#pragma unroll
        for (int e = 0; e < 4; ++e) s[0][b][e] *= gg[e];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) s[0][b] = mfma32(cur.kd[ks], dB[ks][b], s[0][b]);
      }
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) oacc[b] = mfma32(dB[ks][b], cur.as[ks], oacc[b]);  // [col 4lg+e][tok lc]
      __builtin_amdgcn_sched_barrier(0);
      load_b(kn, cur);
      __builtin_amdgcn_sched_barrier(0);
      write_st(s);
      // output rows past the document's end fall outside the resource; the
      // Delta waves' copy of the store gets an empty resource (dropped)
      const uint32_t osz = p.out_bf16 ? 2u : 4u;
      const __amdgpu_buffer_rsrc_t orsrc = buffer_rsrc(
          static_cast<unsigned char*>(p.out) + ((tok0 * H + h) * D + col0) * osz,
          is_o ? static_cast<uint32_t>(((nv - 1) * H * D + DVT)) * osz : 0u);
      if (p.out_bf16) {  // kernel-argument branch: uniform
        const uint32_t ooff = static_cast<uint32_t>((16 * I + lc) * H * D + 4 * lg) * osz;
#pragma unroll
        for (int b = 0; b < 2; ++b) buffer_store8_bf16(oacc[b], orsrc, ooff + 32 * b);
      } else {
        store_rows_f32(oacc, orsrc, static_cast<uint32_t>(16 * I * H * D) * 4u, static_cast<uint32_t>(H * D) * 4u,
                       lc, lg);
      }
    } else {
      // token by token from the entry state; writes this chunk's outputs
      __syncthreads();
      const State2 r = scan_fallback(sm.fb, State2{s[0][0], s[0][1]}, fa, tok_begin, ntok, k, h, col0);
      s[0][0] = r.s0;
      s[0][1] = r.s1;
      __syncthreads();
      __builtin_amdgcn_sched_barrier(0);
      load_b(kn, cur);
      __builtin_amdgcn_sched_barrier(0);
      write_st(s);
    }
  };

  // two operand buffers, even and odd chunks; the main loop body has no
  // branch around a step
  if (nch > 0) {  // workgroup-uniform
    Pre b0, b1;
    load(0, b0);
    load(min(1, nch - 1), b1);
    int k = 0;
    for (; k + 2 <= nch; k += 2) {
      step(k, b0);
      step(k + 1, b1);
    }
    if (k < nch) step(k, b0);
  }

  if (p.final_state) {
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        p.final_state[unit_state + (16 * w + 4 * lg + e) * D + col0 + 16 * b + lc] = s[0][b][e];
  }
}

// ---------------------------------------------------------------------------
// Pass 2, four-wave form: the same 32-column tiles as scan_kernel, with each
// wave forming both Delta and the outputs of token block I = w (one read of
// the staged state serves both products) and updating key rows 32w .. 32w+31.
// At about half of scan_kernel's registers per lane, two workgroups share a
// CU, so when there are more tiles than CUs two units' serial chains
// interleave on every CU and hide each other's waits.
constexpr int NT4 = 256;  // four-wave scan threads

struct __align__(16) Scan4Smem {
  f16 ST[DVT][LDK];   // S^T (fp16) [value col][key row]
  f16 DT[DVT][LDT];   // Delta^T    [value col][token]
  fb::Stage<4> fb;
  int sbp[4];         // per wave: state beyond the fast-path bound
  int dbp[4];         // per wave: Delta beyond the fp16 bound
};

// Slot operands of one chunk as one four-wave scan thread uses them.
struct Pre4 {
  f16x8 mw[4];      // -W row 16w+lc, key cols 32ks+8lg ..
  f16x8 mq[4];      // Qs row 16w+lc, key cols 32ks+8lg ..
  f16x8 u;          // U of this lane, [b][e]
  f16x8 kd[2][2];   // Kd^T rows 32w+16a+lc, tokens 32ks+8lg ..
  f16x8 as[2];      // As row 16w+lc, tokens 32ks+8lg ..
  float4 gam[2];    // exp(gamma) of key rows 32w+16a+4lg ..
  int2 flag;
};

struct WaveState4 {
  f32x4 s[2][2];
};

// The token-by-token evaluation of one chunk, out of line (see scan_fallback).
__device__ __noinline__ WaveState4 scan4_fallback(fb::Stage<4>& st, WaveState4 in, const fb::Args fa,
                                                  size_t tok_begin, int ntok, int k, int h, int col0) {
  fb::eval_chunk<4>(st, in.s, fa, tok_begin, ntok, k, h, col0);
  return in;
}

__global__ void __launch_bounds__(NT4, 2) scan4_kernel(ScanArgs p) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  Scan4Smem& sm = *reinterpret_cast<Scan4Smem*>(smem_raw);

  const int num_units = p.num_docs * p.H;
  const int grp = blockIdx.x / (8 * NTILE);
  const int rem = blockIdx.x - grp * 8 * NTILE;
  const int tile = rem / 8;
  const int u = grp * 8 + (rem & 7);  // rank of the unit (longest documents first)
  if (u >= num_units) return;
  const int H = p.H;
  const int rank = u / H;
  const int h = u - rank * H;
  const int doc = p.order ? p.order[rank] : rank;
  const int col0 = tile * DVT;
  size_t tok_begin;
  int ntok, cbase;
  if (p.cu_seqlens) {
    tok_begin = p.cu_seqlens[doc];
    ntok = p.cu_seqlens[doc + 1] - p.cu_seqlens[doc];
    cbase = p.cstart[doc];
  } else {
    tok_begin = static_cast<size_t>(doc) * p.T;
    ntok = p.T;
    cbase = doc * p.nchd;
  }
  const int nch = (ntok + C - 1) / C;
  if (cbase + nch > p.n_slots) return;  // malformed cu_seqlens: never read past the workspace
  const size_t unit_state = (static_cast<size_t>(doc) * H + h) * D * D;
  const unsigned char* slot0 = p.ws + (static_cast<size_t>(cbase) * H + h) * SLOT_BYTES;
  const size_t slot_stride = static_cast<size_t>(H) * SLOT_BYTES;

  const int tid = threadIdx.x, lane = tid & 63, lc = lane & 15, lg = lane >> 4;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index = token block, uniform (SGPR)

  auto slot_of = [&](int k) { return slot0 + static_cast<size_t>(k) * slot_stride; };
  auto load_flag = [&](int k, Pre4& r) { r.flag = *reinterpret_cast<const int2*>(slot_of(k) + OFF_FLAG); };
  auto load_a = [&](int k, Pre4& r) {
    const unsigned char* sl = slot_of(k);
    const f16* nw = reinterpret_cast<const f16*>(sl + OFF_NW) + (w * 4 * 64 + lane) * 8;
    const f16* qs = reinterpret_cast<const f16*>(sl + OFF_QS) + (w * 4 * 64 + lane) * 8;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      r.mw[ks] = ld8(nw + ks * 64 * 8);
      r.mq[ks] = ld8(qs + ks * 64 * 8);
    }
    r.u = ld_up(sl, w, tile, lane);
  };
  auto load_b = [&](int k, Pre4& r) {
    const unsigned char* sl = slot_of(k);
#pragma unroll
    for (int a = 0; a < 2; ++a) {
      const f16* kd = reinterpret_cast<const f16*>(sl + OFF_KDT) + ((2 * w + a) * 2 * 64 + lane) * 8;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) r.kd[a][ks] = ld8(kd + ks * 64 * 8);
      r.gam[a] = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(sl + OFF_GAM) + 32 * w + 16 * a +
                                                  4 * lg);
    }
    const f16* as = reinterpret_cast<const f16*>(sl + OFF_AS) + (w * 2 * 64 + lane) * 8;
    r.as[0] = ld8(as);
    r.as[1] = w >= 2 ? ld8(as + 64 * 8) : f16x8{};  // row blocks 0, 1: zero past token 31
  };
  auto load = [&](int k, Pre4& r) {
    load_flag(k, r);
    load_a(k, r);
    load_b(k, r);
    __builtin_amdgcn_sched_barrier(0);
  };

  // s[a][b][e] = S[32w+16a+4lg+e][col0+16b+lc]
  auto write_st = [&](f32x4 (&s)[2][2]) {
    bool big = false;
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int b = 0; b < 2; ++b) {
#pragma unroll
        for (int e = 0; e < 4; ++e) big |= !(fabsf(s[a][b][e]) <= S_MAX);
        *reinterpret_cast<f16x4*>(&sm.ST[16 * b + lc][32 * w + 16 * a + 4 * lg]) = h4(s[a][b]);
      }
    const bool any = __builtin_amdgcn_ballot_w64(big) != 0;
    if (lane == 0) sm.sbp[w] = any;
  };

  f32x4 s[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        s[a][b][e] = p.init_state
                         ? p.init_state[unit_state + (32 * w + 16 * a + 4 * lg + e) * D + col0 + 16 * b + lc]
                         : 0.f;
  write_st(s);
  const fb::Args fa{p.q, p.k, p.v, p.log_g, p.beta, p.out, H, p.scale, p.out_bf16, p.l2};

  // One chunk, as in scan_kernel: cur holds chunk k; each group of its
  // registers is refilled with chunk k+1 right after its last use (one
  // buffer: the other workgroup on the CU covers the wait).
  auto step = [&](int k, Pre4& cur) {
    const int kn = min(k + 1, nch - 1);
    const size_t tok0 = tok_begin + static_cast<size_t>(k) * C;
    const int nv = min(C, ntok - k * C);
    lds_barrier();  // ST of the entry state is complete
    const int pflag = __builtin_amdgcn_readfirstlane(cur.flag.x | cur.flag.y);
    __builtin_amdgcn_sched_barrier(0);
    load_flag(kn, cur);
    __builtin_amdgcn_sched_barrier(0);
    const bool sbig = (sm.sbp[0] | sm.sbp[1] | sm.sbp[2] | sm.sbp[3]) != 0;

    // ---- phase A: Delta^T = U^T + S^T (-W)^T (into DT) and the first part of
    // O^T, S^T Qs^T, for token block w, from one read of the staged state
    f16x8 sf[4][2];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int b = 0; b < 2; ++b) sf[ks][b] = ld8(&sm.ST[16 * b + lc][32 * ks + 8 * lg]);
    bool dbig = false;
    f32x4 oacc[2];
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      f32x4 acc;
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[e] = (float)cur.u[4 * b + e];
      f32x4 o = zero4();
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        acc = mfma32(sf[ks][b], cur.mw[ks], acc);  // [col 4lg+e][tok lc]
        o = mfma32(sf[ks][b], cur.mq[ks], o);
      }
      oacc[b] = o;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        dbig |= !(fabsf(acc[e]) <= F16_SAFE);
        sm.DT[16 * b + 4 * lg + e][16 * w + lc] = (f16)acc[e];
      }
    }
    {
      const bool any = __builtin_amdgcn_ballot_w64(dbig) != 0;
      if (lane == 0) sm.dbp[w] = any;
    }
    __builtin_amdgcn_sched_barrier(0);
    load_a(kn, cur);
    __builtin_amdgcn_sched_barrier(0);
    lds_barrier();

    // ---- phase B: S = exp(gamma) S + Kd^T Delta (key rows 32w..), then
    // O^T += Delta^T As^T (to out)
    const bool fbk = pflag != 0 || sbig || (sm.dbp[0] | sm.dbp[1] | sm.dbp[2] | sm.dbp[3]) != 0;
    if (!fbk) {  // workgroup-uniform
      f16x8 dB[2][2];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int b = 0; b < 2; ++b) dB[ks][b] = ld8(&sm.DT[16 * b + lc][32 * ks + 8 * lg]);
#pragma unroll
      for (int a = 0; a < 2; ++a) {
        const float gg[4] = {cur.gam[a].x, cur.gam[a].y, cur.gam[a].z, cur.gam[a].w};
#pragma unroll
        for (int b = 0; b < 2; ++b) {
#pragma unroll
          for (int e = 0; e < 4; ++e) s[a][b][e] *= gg[e];
#pragma unroll
          for (int ks = 0; ks < 2; ++ks) s[a][b] = mfma32(cur.kd[a][ks], dB[ks][b], s[a][b]);
        }
      }
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) oacc[b] = mfma32(dB[ks][b], cur.as[ks], oacc[b]);  // [col 4lg+e][tok lc]
      __builtin_amdgcn_sched_barrier(0);
      load_b(kn, cur);
      __builtin_amdgcn_sched_barrier(0);
      write_st(s);
      // output rows past the document's end fall outside the resource
      const uint32_t osz = p.out_bf16 ? 2u : 4u;
      const __amdgpu_buffer_rsrc_t orsrc =
          buffer_rsrc(static_cast<unsigned char*>(p.out) + ((tok0 * H + h) * D + col0) * osz,
                      static_cast<uint32_t>(((nv - 1) * H * D + DVT)) * osz);
      if (p.out_bf16) {  // kernel-argument branch: uniform
        const uint32_t ooff = static_cast<uint32_t>((16 * w + lc) * H * D + 4 * lg) * osz;
#pragma unroll
        for (int b = 0; b < 2; ++b) buffer_store8_bf16(oacc[b], orsrc, ooff + 32 * b);
      } else {
        store_rows_f32(oacc, orsrc, static_cast<uint32_t>(16 * w * H * D) * 4u, static_cast<uint32_t>(H * D) * 4u,
                       lc, lg);
      }
    } else {
      // token by token from the entry state; writes this chunk's outputs
      __syncthreads();
      WaveState4 r;
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b) r.s[a][b] = s[a][b];
      r = scan4_fallback(sm.fb, r, fa, tok_begin, ntok, k, h, col0);
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b) s[a][b] = r.s[a][b];
      __syncthreads();
      __builtin_amdgcn_sched_barrier(0);
      load_b(kn, cur);
      __builtin_amdgcn_sched_barrier(0);
      write_st(s);
    }
  };

  if (nch > 0) {  // workgroup-uniform
    Pre4 b0;
    load(0, b0);
    for (int k = 0; k < nch; ++k) step(k, b0);
  }

  if (p.final_state) {
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          p.final_state[unit_state + (32 * w + 16 * a + 4 * lg + e) * D + col0 + 16 * b + lc] = s[a][b][e];
  }
}

// ---------------------------------------------------------------------------
// Packed problems: the document map, one workgroup.
//  - cstart[d] = sum over earlier documents of ceil(len / 64); cstart[n] = total;
//  - table[slot] = document owning the slot (a binary search of cstart per
//    slot), -1 for unused slots up to n_slots;
//  - with do_order (n <= MAX_ORDER_DOCS): order[rank] = document, longest
//    first (ties by index), from a bitonic sort of (length descending, index)
//    keys in LDS over the next power of two >= n.
constexpr int MAX_ORDER_DOCS = 16384;

__global__ void __launch_bounds__(1024) doc_map_kernel(const int32_t* __restrict__ cu, int n, int n_slots,
                                                       int32_t* __restrict__ cstart, int32_t* __restrict__ table,
                                                       int32_t* __restrict__ order, int do_order) {
  __shared__ int wsum[16];
  __shared__ uint64_t key[MAX_ORDER_DOCS];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  int carry = 0;
  for (int base = 0; base < n; base += 1024) {
    const int d = base + tid;
    const int len = d < n ? max(cu[d + 1] - cu[d], 0) : 0;
    const int nc = (len + C - 1) / C;
    int x = nc;  // inclusive scan within the wave
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(x, o, 64);
      x += lane >= o ? y : 0;
    }
    if (lane == 63) wsum[wv] = x;
    __syncthreads();
    int woff = 0, total = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      woff += i < wv ? wsum[i] : 0;
      total += wsum[i];
    }
    if (d < n) cstart[d] = carry + woff + x - nc;
    carry += total;
    __syncthreads();
  }
  if (tid == 0) cstart[n] = carry;
  __syncthreads();  // cstart complete (global writes of this workgroup)
  for (int c = tid; c < n_slots; c += 1024) {
    int doc = -1;
    if (c < carry) {  // the last document whose first slot is <= c (empty documents own none)
      int lo = 0, hi = n;  // cstart[lo] <= c < cstart[hi]
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (cstart[mid] <= c) lo = mid; else hi = mid;
      }
      doc = lo;
    }
    table[c] = doc;
  }
  if (!do_order) return;  // kernel argument: uniform
  int m = 1;
  while (m < n) m <<= 1;
  for (int i = tid; i < m; i += 1024) {
    // ascending keys = longest first, then lower index; padding sorts last
    const uint32_t len = i < n ? static_cast<uint32_t>(max(cu[i + 1] - cu[i], 0)) : 0u;
    key[i] = i < n ? (static_cast<uint64_t>(0x7fffffffu - len) << 32) | static_cast<uint32_t>(i) : ~uint64_t(0);
  }
  __syncthreads();
  for (int size = 2; size <= m; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int i = tid; i < m; i += 1024) {
        const int j = i ^ stride;
        if (j > i) {
          const bool up = (i & size) == 0;
          const uint64_t x = key[i], y = key[j];
          if ((x > y) == up) {
            key[i] = y;
            key[j] = x;
          }
        }
      }
      __syncthreads();
    }
  }
  for (int r = tid; r < n; r += 1024) order[r] = static_cast<int32_t>(key[r] & 0xffffffffu);
}

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

// Chunk slots per head: dense B ceil(T/64); packed ceil(T/64) + N (each
// document adds at most one partial chunk).
int64_t n_slots_of(int num_seqs, int seq_len, bool packed) {
  const int64_t nchd = (static_cast<int64_t>(seq_len) + C - 1) / C;
  return packed ? nchd + num_seqs : nchd * num_seqs;
}

struct WsLayout {
  int32_t* cstart;
  int32_t* table;
  int32_t* order;
  unsigned char* slots;
  size_t bytes;
};

WsLayout ws_layout(void* base, int num_seqs, int seq_len, int H, bool packed) {
  WsLayout l{};
  unsigned char* b = static_cast<unsigned char*>(base);
  size_t off = 0;
  const int64_t ns = n_slots_of(num_seqs, seq_len, packed);
  if (packed) {
    l.cstart = reinterpret_cast<int32_t*>(b + off);
    off += align256(static_cast<size_t>(num_seqs + 1) * 4);
    l.table = reinterpret_cast<int32_t*>(b + off);
    off += align256(static_cast<size_t>(ns) * 4);
    l.order = reinterpret_cast<int32_t*>(b + off);
    off += align256(static_cast<size_t>(num_seqs) * 4);
  }
  l.slots = b + off;
  off += static_cast<size_t>(ns) * H * SLOT_BYTES;
  l.bytes = off;
  return l;
}

}  // namespace

size_t twopass_workspace_bytes(int num_seqs, int seq_len, int num_heads, bool packed) {
  return ws_layout(nullptr, num_seqs, seq_len, num_heads, packed).bytes;
}

bool twopass_supported(const ChunkLaunch& a) {
  const int64_t blocks = n_slots_of(a.num_seqs, a.seq_len, a.cu_seqlens != nullptr) * a.num_heads;
  // the prep kernel's range-checked loads span one chunk's rows of log_g in
  // 32-bit byte offsets: C * H * D * 4 bytes
  const bool offsets_fit = int64_t(C) * a.num_heads * D * 4 <= int64_t(UINT32_MAX);
  return a.bf16 && a.d == D && blocks < (int64_t(1) << 31) && offsets_fit;
}

// The kernels' LDS limits are raised once per device (the attribute is per
// device); a mutex keeps concurrent first calls from different host threads
// apart.
static hipError_t prepare_device() {
  constexpr int MAX_DEV = 64;
  static std::mutex lock;
  static bool ready[MAX_DEV] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= MAX_DEV) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> g(lock);
  if (!ready[dev]) {
    const struct {
      const void* fn;
      size_t bytes;
    } k[] = {{reinterpret_cast<const void*>(prep_kernel<false>), sizeof(PrepSmem)},
             {reinterpret_cast<const void*>(prep_kernel<true>), sizeof(PrepSmem)},
             {reinterpret_cast<const void*>(scan_kernel), sizeof(ScanSmem)},
             {reinterpret_cast<const void*>(scan4_kernel), sizeof(Scan4Smem)}};
    for (const auto& x : k) {
      e = hipFuncSetAttribute(x.fn, hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(x.bytes));
      if (e != hipSuccess) return e;
    }
    ready[dev] = true;
  }
  return hipSuccess;
}

// Scan form: four 32-column tiles per (sequence or document, head); the
// four-wave form, two workgroups per CU, when there are more tiles than CUs,
// else the eight-wave form, whose steps are shorter.  KDA_PREFILL_PATH=tile8
// or =tile4 forces a form (a test and diagnosis switch).
enum class ScanForm { Tile8, Tile4 };
constexpr int64_t TILE4_MIN_TILES = 257;

ScanForm scan_form(const ChunkLaunch& a) {
  const char* e = std::getenv("KDA_PREFILL_PATH");
  if (e && std::strcmp(e, "tile8") == 0) return ScanForm::Tile8;
  if (e && std::strcmp(e, "tile4") == 0) return ScanForm::Tile4;
  const int64_t tiles = static_cast<int64_t>(a.num_seqs) * a.num_heads * NTILE;
  return tiles >= TILE4_MIN_TILES ? ScanForm::Tile4 : ScanForm::Tile8;
}

hipError_t launch_chunk_twopass(const ChunkLaunch& a, hipStream_t stream) {
  {
    const hipError_t e = prepare_device();
    if (e != hipSuccess) return e;
  }
  const bool packed = a.cu_seqlens != nullptr;
  const WsLayout l = ws_layout(a.workspace, a.num_seqs, a.seq_len, a.num_heads, packed);
  const int64_t ns = n_slots_of(a.num_seqs, a.seq_len, packed);
  const int nchd = (a.seq_len + C - 1) / C;
  if (packed) {
    const int do_order = a.num_seqs > 1 && a.num_seqs <= MAX_ORDER_DOCS;
    hipLaunchKernelGGL(doc_map_kernel, dim3(1), dim3(1024), 0, stream, a.cu_seqlens, a.num_seqs,
                       static_cast<int>(ns), l.cstart, l.table, l.order, do_order);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (ns > 0) {
    PrepArgs pp{};
    pp.q = static_cast<const bf16_t*>(a.q);
    pp.k = static_cast<const bf16_t*>(a.k);
    pp.v = static_cast<const bf16_t*>(a.v);
    pp.log_g = a.log_g;
    pp.beta = a.beta;
    pp.cu_seqlens = a.cu_seqlens;
    pp.cstart = packed ? l.cstart : nullptr;
    pp.table = packed ? l.table : nullptr;
    pp.ws = l.slots;
    pp.T = a.seq_len;
    pp.H = a.num_heads;
    pp.nchd = nchd;
    pp.scale = a.scale;
    if (a.l2)
      hipLaunchKernelGGL(prep_kernel<true>, dim3(static_cast<unsigned>(ns * a.num_heads)), dim3(NTP),
                         sizeof(PrepSmem), stream, pp);
    else
      hipLaunchKernelGGL(prep_kernel<false>, dim3(static_cast<unsigned>(ns * a.num_heads)), dim3(NTP),
                         sizeof(PrepSmem), stream, pp);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  ScanArgs sp{};
  sp.q = static_cast<const bf16_t*>(a.q);
  sp.k = static_cast<const bf16_t*>(a.k);
  sp.v = static_cast<const bf16_t*>(a.v);
  sp.log_g = a.log_g;
  sp.beta = a.beta;
  sp.init_state = a.init_state;
  sp.final_state = a.final_state;
  sp.cu_seqlens = a.cu_seqlens;
  sp.cstart = packed ? l.cstart : nullptr;
  sp.order = (packed && a.num_seqs > 1 && a.num_seqs <= MAX_ORDER_DOCS) ? l.order : nullptr;
  sp.ws = l.slots;
  sp.out = a.out;
  sp.out_bf16 = a.out_bf16;
  sp.l2 = a.l2;
  sp.num_docs = a.num_seqs;
  sp.T = a.seq_len;
  sp.H = a.num_heads;
  sp.nchd = nchd;
  sp.n_slots = static_cast<int>(ns);
  sp.scale = a.scale;
  const unsigned units = static_cast<unsigned>(a.num_seqs) * static_cast<unsigned>(a.num_heads);
  const ScanForm form = scan_form(a);
  const unsigned blocks = ((units + 7) / 8) * 8 * NTILE;
  if (form == ScanForm::Tile4)
    hipLaunchKernelGGL(scan4_kernel, dim3(blocks), dim3(NT4), sizeof(Scan4Smem), stream, sp);
  else
    hipLaunchKernelGGL(scan_kernel, dim3(blocks), dim3(NTS), sizeof(ScanSmem), stream, sp);
  return hipGetLastError();
}

}  // namespace kda
