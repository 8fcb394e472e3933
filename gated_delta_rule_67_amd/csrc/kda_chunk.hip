// kda_chunk.hip -- chunked (64-token) prefill of the KDA recurrence on MFMA (gfx950).
//
// Chunk algebra.  Unrolling the gated delta rule (GLM-5.3-Flash model notes,
// Glm5NextTextLinearAttention snippet) over one chunk of C = 64 tokens from the
// entry state S (dk x dv), with G_i = sum_{s<=i} log_g_s per key channel and
// gamma = G_63:
//   A[i,j]   = beta_i sum_c k_ic k_jc exp(G_ic - G_jc)   (j < i)
//   X        = beta * (V - (K exp(G)) S)
//   Delta    = (I + A)^-1 X
//   Aqk[i,j] = sum_c q_ic k_jc exp(G_ic - G_jc)          (j <= i)
//   O        = scale ((Q exp(G)) S + Aqk Delta)
//   S_next   = exp(gamma) S + (K exp(gamma - G))^T Delta
// (the output reads the state after each token's update).
//
// Work split.  One workgroup owns one (unit, 32-column value tile); a unit's
// four tiles run as four workgroups placed on one XCD so that they share the
// unit's q/k/log_g rows in that XCD's L2 (value columns never interact).  Its
// four waves are software-pipelined over chunks: in each of the three phases
// per chunk a wave does producer work for chunk k+1 (gate products and
// decay-scaled operands, the 64x64 products A and Aqk, the inverses of the
// four 16x16 diagonal blocks of (I + A)) and consumer work for chunk k
// (everything that needs the state: (K exp G) S and (Q exp G) S, Delta by
// blocked forward substitution, the outputs and the state update), so VALU
// gate work overlaps MFMA chains inside one wave.  The fp32 state tile
// S[128][32] stays in MFMA accumulator registers for the whole unit; global
// loads of chunk k+2 are issued a full chunk before use; three LDS-only
// barriers separate the phases.
//
// Decay factors without overflow.  The chunk is cut into four 16-token blocks.
// With R_I = G before block I's first token:
//   Kl = k exp(G - R_I) <= |k|, Ql = q exp(G - R_I), Kr = k exp(R_{I+1} - G) <= |k|
// come from prefix / suffix products of exp(log_g) inside a block (thread
// local).  Off-diagonal tiles (I > J) pair Kl_I exp(R_I - R_{J+1}) with Kr_J:
// every factor is <= 1 for any gate.  Diagonal tiles use the block's midpoint
// M_I as reference: Kl_I exp(R_I - M_I) against Kr_I exp(M_I - R_{I+1}); these
// factors are >= 1, bounded by exp(HALF_SPAN_MAX).  A chunk whose half-block
// decay exceeds the bound, whose inputs could overflow an fp16 operand, or
// whose diagonal blocks of A exceed 1 in magnitude, is evaluated token by
// token (exact fp32) inside this kernel instead.
//
// Arithmetic: fp16 MFMA operands (formed in fp32 from the bf16 inputs,
// rounded once, kept inside fp16's range by the guard), fp32
// accumulation, state and outputs.  With L a strictly lower 16x16 diagonal
// block of A (|L| <= 1, L^16 = 0), (I + L)^-1 = (I - L)(I + L^2)(I + L^4)(I + L^8)
// is formed with 16x16x16 MFMAs.  Products whose result feeds another MFMA
// as its A operand are computed transposed (C = B^T A^T), so the result
// already sits in the A-operand lane layout and is stored fragment-major.
#include "kda_common.h"
#include "kda_fallback.h"
#include "kda_launch.h"

namespace kda {
namespace {

constexpr int C = 64;        // chunk length
constexpr int D = 128;       // head dim (dk = dv)
constexpr int DVT = 32;      // value columns per workgroup
constexpr int NTILE = D / DVT;
constexpr int NT = 256;      // threads: 4 waves, each with a producer and a consumer part
constexpr int LDK = D + 8;   // fp16 row stride of [64][128] matrices
constexpr int LDT = C + 8;   // fp16 row stride of [*][64] matrices
constexpr int LDV = DVT + 8; // fp16 row stride of the value tile
constexpr float HALF_SPAN_MAX = 6.0f;   // max decay (e-folds) over half a block
constexpr unsigned short QK_MAX_BITS = 0x4280;  // bf16 bits of 64.0: |q|, |k| bound
constexpr float V_MAX = 4096.0f;        // |v| bound of the fast path
constexpr float S_MAX = 2048.0f;        // |S| bound of the fast path
constexpr float BETA_MAX = 1.0f;        // |beta| bound of the fast path

// fragment slots per chunk buffer: 0-3 diagonal inverses T_II, 4-9 A_IJ
// (I > J), 10-19 Aqk lower tiles; each slot holds one f16x4 per lane.
constexpr int SLOT_A = 4, SLOT_Q = 10, NSLOT = 20;

struct ChunkArgs {
  const bf16_t* q;
  const bf16_t* k;
  const bf16_t* v;
  const float* log_g;
  const float* beta;
  const float* init_state;
  float* final_state;
  const int32_t* cu_seqlens;  // null: dense
  const int32_t* order;       // null: identity document order
  float* out;
  int num_docs;
  int T;                      // dense tokens per sequence
  int H;
  float scale;
};


// Kr and KdT are dead while a chunk is evaluated token by token, so the
// fallback's staging area overlays them.
struct KrKd {
  f16 Kr[C][LDK];          // k exp(R_blk_end - G)   (producer only)
  f16 KdT[D][LDT];         // (k exp(gamma - G))^T   [channel][token]
};

struct __align__(16) Smem {
  f16 Kl[2][C][LDK];       // k exp(G - R_blk), by chunk parity
  f16 Ql[2][C][LDK];       // q exp(G - R_blk), by chunk parity
  union {
    KrKd kk;
    fb::Stage<4> fb;
  } u;
  f16 V[2][C][LDV];        // value tile (fp16), by chunk parity
  float beta[2][C];
  float tot[4][D];         // per-block products of exp(log_g)   (producer only)
  f16 fDl[4][D];           // exp(R_I - M_I)                     (producer only)
  f16 fDr[4][D];           // exp(M_I - R_{I+1})                 (producer only)
  f16 fOff[3][D];          // exp(R_I - R_{J+1}) for (2,0), (3,0), (3,1)
  f16 fR[2][4][D];         // exp(R_I), by chunk parity
  float fGam[2][D];        // exp(gamma), by chunk parity
  f16x4 frag[2][NSLOT][64];
  f16 ST[DVT][LDK];        // S^T (fp16) for the consumers' products
  f16 DT[DVT][LDT];        // Delta^T
  int fbp[2][4];           // producer waves: chunk cannot take the fast path
  int sbp[4];              // consumer waves: state beyond the fast-path bound
};
static_assert(sizeof(fb::Stage<4>) <= sizeof(KrKd), "fallback staging does not fit");

// Whether the chunk in buffer buf must be evaluated token by token: a
// producer wave flagged it, or the state left the fast path's range.
__device__ __forceinline__ bool fast_path_blocked(const Smem& sm, int buf) {
  return (sm.fbp[buf][0] | sm.fbp[buf][1] | sm.fbp[buf][2] | sm.fbp[buf][3] |
          sm.sbp[0] | sm.sbp[1] | sm.sbp[2] | sm.sbp[3]) != 0;
}

__device__ __forceinline__ int tile10(int I, int J) { return (I * (I + 1)) / 2 + J; }  // J <= I
__device__ __forceinline__ int pair6(int I, int J) { return (I * (I - 1)) / 2 + J; }   // J < I


// Raw inputs of one chunk as one producer thread loads them (16-byte loads):
// rows 16*blk + 4*qt + j (j < 4) of channels 8*oct .. 8*oct+7, plus 8 values
// of the value tile and one beta.
struct Raw {
  float4 g[4][2];
  uint4 k[4];
  uint4 q[4];
  uint4 v;
  float beta;
};

// What a producer thread carries from stage A to the end of the chunk's products.
struct Prod {
  bool bad;
};

__global__ void __launch_bounds__(NT, 1) chunk_kernel(ChunkArgs p) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  Smem& sm = *reinterpret_cast<Smem*>(smem_raw);

  const int num_units = p.num_docs * p.H;
  const int grp = blockIdx.x / (8 * NTILE);
  const int rem = blockIdx.x - grp * 8 * NTILE;
  const int tile = rem / 8;
  const int u = grp * 8 + (rem & 7);  // rank of the unit (longest documents first)
  if (u >= num_units) return;
  const int rank = u / p.H;
  const int h = u - rank * p.H;
  const int doc = p.order ? p.order[rank] : rank;
  const int col0 = tile * DVT;
  const int H = p.H;
  size_t tok_begin;
  int ntok;
  if (p.cu_seqlens) {
    tok_begin = p.cu_seqlens[doc];
    ntok = p.cu_seqlens[doc + 1] - p.cu_seqlens[doc];
  } else {
    tok_begin = static_cast<size_t>(doc) * p.T;
    ntok = p.T;
  }
  const int nch = (ntok + C - 1) / C;
  const size_t unit_state = (static_cast<size_t>(doc) * H + h) * D * D;

  const int tid = threadIdx.x, lane = tid & 63, lc = lane & 15, lg = lane >> 4;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, uniform (SGPR)
  const int pw = w;  // producer role: token block; consumer role: state rows 32w..
  const int oct = lane & 15;     // producer: channels 8*oct .. 8*oct+7
  const int qt = lane >> 4;      // producer: rows 4*qt .. 4*qt+3 of block pw
  const int c8 = 8 * oct;
  const float lim_lo = __expf(-HALF_SPAN_MAX);

  // ---------------- producer helpers
  auto load_raw = [&](int ck, Raw& r) {
    const int nv = min(C, ntok - ck * C);
    const size_t tok0 = tok_begin + static_cast<size_t>(ck) * C;
    // uniform bases; per-lane 32-bit offsets (64 rows x H x D fits easily)
    const float* gb = p.log_g + (tok0 * H + h) * D;
    const bf16_t* kb = p.k + (tok0 * H + h) * D;
    const bf16_t* qb = p.q + (tok0 * H + h) * D;
    const int rs = H * D;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const unsigned off = static_cast<unsigned>(min(16 * pw + 4 * qt + j, nv - 1) * rs + c8);
      r.g[j][0] = *reinterpret_cast<const float4*>(gb + off);
      r.g[j][1] = *reinterpret_cast<const float4*>(gb + off + 4u);
      r.k[j] = *reinterpret_cast<const uint4*>(kb + off);
      r.q[j] = *reinterpret_cast<const uint4*>(qb + off);
    }
    const int vr = tid >> 2, vc = (tid & 3) * 8;
    const bf16_t* vb = p.v + (tok0 * H + h) * D + col0;
    r.v = *reinterpret_cast<const uint4*>(vb + static_cast<unsigned>(min(vr, nv - 1) * rs + vc));
    const float* bb = p.beta + tok0 * H + h;
    r.beta = bb[static_cast<unsigned>(min(tid & (C - 1), nv - 1) * H)];
  };

  // stage A of chunk ck into buffer buf: exp(log_g), its products over the
  // 16-token block (prefix and suffix; the four 4-token quarters of a block
  // sit in lanes oct, oct+16, oct+32, oct+48), the decay-scaled operands Kl,
  // Ql, Kr, the block totals and diagonal-tile factors, the value tile and beta.
  auto stage_a = [&](int ck, int buf, Raw& r, Prod& o) {
    const int nv = min(C, ntok - ck * C);
    bool bad = false;
    u16x2 mk = {0, 0};
    // padding rows (past the document's end) become identity tokens:
    // k = q = 0, log_g = 0
    const int nrow = nv - (16 * pw + 4 * qt);  // rows of this lane's quarter inside the chunk
    if (nv < C) {  // workgroup-uniform: only a document's last chunk has padding rows
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const bool pad = j >= nrow;
        r.k[j].x = pad ? 0u : r.k[j].x; r.k[j].y = pad ? 0u : r.k[j].y;
        r.k[j].z = pad ? 0u : r.k[j].z; r.k[j].w = pad ? 0u : r.k[j].w;
        r.q[j].x = pad ? 0u : r.q[j].x; r.q[j].y = pad ? 0u : r.q[j].y;
        r.q[j].z = pad ? 0u : r.q[j].z; r.q[j].w = pad ? 0u : r.q[j].w;
#pragma unroll
        for (int x = 0; x < 2; ++x) r.g[j][x] = pad ? make_float4(0.f, 0.f, 0.f, 0.f) : r.g[j][x];
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t kw[4] = {r.k[j].x, r.k[j].y, r.k[j].z, r.k[j].w};
      const uint32_t qw[4] = {r.q[j].x, r.q[j].y, r.q[j].z, r.q[j].w};
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        mk = __builtin_elementwise_max(mk, __builtin_bit_cast(u16x2, kw[x] & 0x7fff7fffu));
        mk = __builtin_elementwise_max(mk, __builtin_bit_cast(u16x2, qw[x] & 0x7fff7fffu));
      }
    }
    bad |= mk[0] > QK_MAX_BITS || mk[1] > QK_MAX_BITS;
    // Per channel: P = exp(G - R_blk), S = exp(R_blk_end - G) on this lane's 4
    // rows, folded straight into the fp16 operand rows.
    f16x8 hl[4], hq[4], hr[4];
    float tot8[8];
    f16x8 fdl8, fdr8;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      float a[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float4 g4 = r.g[j][c >> 2];
        const int cc = c & 3;
        const float gv = cc == 0 ? g4.x : cc == 1 ? g4.y : cc == 2 ? g4.z : g4.w;
        a[j] = exp_fast(gv);
      }
      const float p1 = a[0] * a[1], p2 = p1 * a[2], p3 = p2 * a[3];  // inside the quarter
      const float s1 = a[2] * a[3], s0 = a[1] * s1;
      const float t0 = __shfl(p3, oct, 64), t1 = __shfl(p3, oct + 16, 64);
      const float t2 = __shfl(p3, oct + 32, 64), t3 = __shfl(p3, oct + 48, 64);
      // exclusive products over the quarters before / after this lane's
      const float E = (qt >= 1 ? t0 : 1.f) * (qt >= 2 ? t1 : 1.f) * (qt >= 3 ? t2 : 1.f);
      const float F = (qt <= 2 ? t3 : 1.f) * (qt <= 1 ? t2 : 1.f) * (qt <= 0 ? t1 : 1.f);
      const float Pv[4] = {E * a[0], E * p1, E * p2, E * p3};
      const float Sv[4] = {s0 * F, s1 * F, a[3] * F, F};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t kw = c < 2 ? r.k[j].x : c < 4 ? r.k[j].y : c < 6 ? r.k[j].z : r.k[j].w;
        const uint32_t qw = c < 2 ? r.q[j].x : c < 4 ? r.q[j].y : c < 6 ? r.q[j].z : r.q[j].w;
        const float kv = (c & 1) ? bf16_hi(kw) : bf16_lo(kw);
        const float qv = (c & 1) ? bf16_hi(qw) : bf16_lo(qw);
        hl[j][c] = (f16)(kv * Pv[j]);
        hq[j][c] = (f16)(qv * Pv[j]);
        hr[j][c] = (f16)(kv * Sv[j]);
      }
      const float dl = t0 * t1, dr = t2 * t3;  // over the first / second half of the block
      bad |= (dl < lim_lo) | (dr < lim_lo) | (dl != dl) | (dr != dr);
      tot8[c] = dl * dr;
      fdl8[c] = (f16)(1.f / fmaxf(dl, lim_lo));
      fdr8[c] = (f16)(1.f / fmaxf(dr, lim_lo));
    }
    // the four quarter lanes of a channel octet write identical values
    *reinterpret_cast<float4*>(&sm.tot[pw][c8]) = make_float4(tot8[0], tot8[1], tot8[2], tot8[3]);
    *reinterpret_cast<float4*>(&sm.tot[pw][c8 + 4]) = make_float4(tot8[4], tot8[5], tot8[6], tot8[7]);
    *reinterpret_cast<f16x8*>(&sm.fDl[pw][c8]) = fdl8;
    *reinterpret_cast<f16x8*>(&sm.fDr[pw][c8]) = fdr8;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int row = 16 * pw + 4 * qt + j;
      *reinterpret_cast<f16x8*>(&sm.Kl[buf][row][c8]) = hl[j];
      *reinterpret_cast<f16x8*>(&sm.Ql[buf][row][c8]) = hq[j];
      *reinterpret_cast<f16x8*>(&sm.u.kk.Kr[row][c8]) = hr[j];
    }
    {
      const int vr = tid >> 2;
      const uint4 x = r.v;
      float vv[8] = {bf16_lo(x.x), bf16_hi(x.x), bf16_lo(x.y), bf16_hi(x.y),
                     bf16_lo(x.z), bf16_hi(x.z), bf16_lo(x.w), bf16_hi(x.w)};
      f16x8 vh;
      float vmax = 0.f;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        vv[j] = vr < nv ? vv[j] : 0.f;
        vmax = fmaxf(vmax, fabsf(vv[j]));
        vh[j] = (f16)vv[j];
      }
      bad |= !(vmax <= V_MAX);
      *reinterpret_cast<f16x8*>(&sm.V[buf][vr][(tid & 3) * 8]) = vh;
      const float bv = (tid & (C - 1)) < nv ? r.beta : 0.f;
      sm.beta[buf][tid & (C - 1)] = bv;  // the four waves write identical values
      bad |= !(fabsf(bv) <= BETA_MAX);
    }
    o.bad = bad;
  };

  // factors from the block totals; the KdT values of this chunk into kd[]:
  // kd[c] holds rows 16*pw+4*qt .. +3 of channel c8+c.
  auto factors = [&](int buf, f16x4 (&kd)[8]) {
    float T[4][8];
#pragma unroll
    for (int I = 0; I < 4; ++I) {
      const float4 a = *reinterpret_cast<const float4*>(&sm.tot[I][c8]);
      const float4 b = *reinterpret_cast<const float4*>(&sm.tot[I][c8 + 4]);
      T[I][0] = a.x; T[I][1] = a.y; T[I][2] = a.z; T[I][3] = a.w;
      T[I][4] = b.x; T[I][5] = b.y; T[I][6] = b.z; T[I][7] = b.w;
    }
    float gd[8], gam[8];
    f16x8 r1, r2, r3, o20, o30, o31;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      // exp(gamma - R_{pw+1}): product of the totals of the later blocks
      gd[c] = pw == 0 ? T[1][c] * T[2][c] * T[3][c] : pw == 1 ? T[2][c] * T[3][c] : pw == 2 ? T[3][c] : 1.f;
      const float e1 = T[0][c], e2 = e1 * T[1][c], e3 = e2 * T[2][c];
      r1[c] = (f16)e1;  r2[c] = (f16)e2;  r3[c] = (f16)e3;
      gam[c] = e3 * T[3][c];
      o20[c] = (f16)T[1][c];
      o30[c] = (f16)(T[1][c] * T[2][c]);
      o31[c] = (f16)T[2][c];
    }
    // every lane of every wave writes the same values: no branch in this phase
    const f16 one = (f16)1.f;
    *reinterpret_cast<f16x8*>(&sm.fR[buf][0][c8]) = f16x8{one, one, one, one, one, one, one, one};
    *reinterpret_cast<f16x8*>(&sm.fR[buf][1][c8]) = r1;
    *reinterpret_cast<f16x8*>(&sm.fR[buf][2][c8]) = r2;
    *reinterpret_cast<f16x8*>(&sm.fR[buf][3][c8]) = r3;
    *reinterpret_cast<float4*>(&sm.fGam[buf][c8]) = make_float4(gam[0], gam[1], gam[2], gam[3]);
    *reinterpret_cast<float4*>(&sm.fGam[buf][c8 + 4]) = make_float4(gam[4], gam[5], gam[6], gam[7]);
    *reinterpret_cast<f16x8*>(&sm.fOff[0][c8]) = o20;  // (2,0)
    *reinterpret_cast<f16x8*>(&sm.fOff[1][c8]) = o30;  // (3,0)
    *reinterpret_cast<f16x8*>(&sm.fOff[2][c8]) = o31;  // (3,1)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const f16x8 kr = ld8(&sm.u.kk.Kr[16 * pw + 4 * qt + j][c8]);
#pragma unroll
      for (int c = 0; c < 8; ++c) kd[c][j] = (f16)((float)kr[c] * gd[c]);
    }
  };

  auto write_kdt = [&](const f16x4 (&kd)[8]) {
#pragma unroll
    for (int c = 0; c < 8; ++c)
      *reinterpret_cast<f16x4*>(&sm.u.kk.KdT[c8 + c][16 * pw + 4 * qt]) = kd[c];
  };

  // A, Aqk and the diagonal-block inverses of one chunk into frag[buf].
  auto products = [&](int buf, bool bad_in) {
    bool bad = bad_in;
    // diagonal block I = pw: A-layout (swapped product) and B-layout
    {
      const int I = pw;
      f32x4 accA = zero4(), accB = zero4();
      f16x8 l[4], r[4], fl[4], fr[4];
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const int kc = 32 * ks + 8 * lg;
        l[ks] = ld8(&sm.Kl[buf][16 * I + lc][kc]);
        r[ks] = ld8(&sm.u.kk.Kr[16 * I + lc][kc]);
        fl[ks] = ld8(&sm.fDl[I][kc]);
        fr[ks] = ld8(&sm.fDr[I][kc]);
      }
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const f16x8 ls = l[ks] * fl[ks], rs = r[ks] * fr[ks];
        accA = mfma32(rs, ls, accA);  // A layout: rows 16I+lc, cols 16I+4lg+e
        accB = mfma32(ls, rs, accB);  // B layout: rows 16I+4lg+e, cols 16I+lc
      }
      f16x4 a, b;
      const float bA = sm.beta[buf][16 * I + lc];
      const float4 bB4 = *reinterpret_cast<const float4*>(&sm.beta[buf][16 * I + 4 * lg]);
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
      // (I + L)^-1 = (I - L)(I + L^2)(I + L^4)(I + L^8), L strictly lower
      const f16x4 b2 = h4(mfma16(a, b, zero4()));
      const f16x4 a2 = h4(mfma16(b, a, zero4()));
      const f16x4 b4 = h4(mfma16(a2, b2, zero4()));
      const f16x4 a4 = h4(mfma16(b2, a2, zero4()));
      const f16x4 b8 = h4(mfma16(a4, b4, zero4()));
      f32x4 t;
#pragma unroll
      for (int e = 0; e < 4; ++e) t[e] = (lc == 4 * lg + e ? 1.f : 0.f) - (float)a[e];
      t = mfma16(b2, h4(t), t);
      t = mfma16(b4, h4(t), t);
      t = mfma16(b8, h4(t), t);
      sm.frag[buf][I][lane] = h4(t);
    }
    // four of the sixteen remaining tiles: A_IJ (I > J) and Aqk_IJ (J <= I)
#pragma unroll 1
    for (int m = 0; m < 4; ++m) {
      const int item = pw + 4 * m;
      const bool isq = item >= 6;
      int I, J;
      if (!isq) {
        // pairs (1,0) (2,0) (2,1) (3,0) (3,1) (3,2)
        I = item >= 3 ? 3 : item >= 1 ? 2 : 1;
        J = item - pair6(I, 0);
      } else {
        const int t = item - 6;
        I = t >= 6 ? 3 : t >= 3 ? 2 : t >= 1 ? 1 : 0;
        J = t - tile10(I, 0);
      }
      const f16(*L)[LDK] = isq ? sm.Ql[buf] : sm.Kl[buf];
      const int off = (I == 2 && J == 0) ? 0 : (I == 3 && J == 0) ? 1 : (I == 3 && J == 1) ? 2 : -1;
      f32x4 acc = zero4();
      f16x8 l[4], r[4], fl[4], fr[4];
      // factor rows (an all-ones row is never needed: no scaling then)
      const f16* flp = I == J ? &sm.fDl[I][0] : off >= 0 ? &sm.fOff[off][0] : nullptr;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const int kc = 32 * ks + 8 * lg;
        l[ks] = ld8(&L[16 * I + lc][kc]);
        r[ks] = ld8(&sm.u.kk.Kr[16 * J + lc][kc]);
        if (flp) fl[ks] = ld8(flp + kc);
        if (I == J) fr[ks] = ld8(&sm.fDr[I][kc]);
      }
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const f16x8 ls = flp ? l[ks] * fl[ks] : l[ks];
        const f16x8 rs = I == J ? r[ks] * fr[ks] : r[ks];
        acc = mfma32(rs, ls, acc);  // A layout: rows 16I+lc, cols 16J+4lg+e
      }
      f16x4 res;
      if (!isq) {
        const float bA = sm.beta[buf][16 * I + lc];
#pragma unroll
        for (int e = 0; e < 4; ++e) res[e] = (f16)(bA * acc[e]);
        sm.frag[buf][SLOT_A + pair6(I, J)][lane] = res;
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) res[e] = (f16)((16 * J + 4 * lg + e) <= (16 * I + lc) ? acc[e] : 0.f);
        sm.frag[buf][SLOT_Q + tile10(I, J)][lane] = res;
      }
    }
    return bad;
  };

  // ---------------- consumer state: s[a][b][e] = S[32cw+16a+4lg+e][col0+16b+lc]
  const int cw = pw;
  const int nb = cw & 1;          // consumer value-column tile (16 columns)
  const bool is_z = cw >= 2;      // waves 2,3: Z and outputs; waves 0,1: X and Delta

  auto write_st = [&](f32x4 (&s)[2][2]) {
    bool big = false;
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int b = 0; b < 2; ++b) {
#pragma unroll
        for (int e = 0; e < 4; ++e) big |= !(fabsf(s[a][b][e]) <= S_MAX);
        *reinterpret_cast<f16x4*>(&sm.ST[16 * b + lc][32 * cw + 16 * a + 4 * lg]) = h4(s[a][b]);
      }
    const bool any = __builtin_amdgcn_ballot_w64(big) != 0;
    if (lane == 0) sm.sbp[cw] = any;
  };


  // ---------------- state and prologue
  f32x4 s[2][2];   // s[a][b][e] = S[32cw+16a+4lg+e][col0+16b+lc]
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        s[a][b][e] = p.init_state ? p.init_state[unit_state + (32 * cw + 16 * a + 4 * lg + e) * D + col0 + 16 * b + lc]
                                  : 0.f;
  write_st(s);
  Raw raw;
  Prod pr;
  f16x4 kd[8];
  if (nch > 0) {
    load_raw(0, raw);
    stage_a(0, 0, raw, pr);
    if (nch > 1) load_raw(1, raw);
    lds_barrier();
    factors(0, kd);
    lds_barrier();
    {
      const bool bad = products(0, pr.bad);
      const bool any = __builtin_amdgcn_ballot_w64(bad) != 0;
      if (lane == 0) sm.fbp[0][pw] = any;
    }
    lds_barrier();
  }

  // ---------------- one chunk: consumer work on chunk k, producer work on
  // chunk k+1 (when `produce`).  The consumer part runs the fast path's
  // products for every chunk; for a chunk flagged for token-by-token
  // evaluation it skips the state update, and the fallback then recomputes
  // the chunk's outputs over the ones written here.
  auto chunk_step = [&](int k, bool produce) {
    const int buf = k & 1, nbuf = buf ^ 1;
    const bool fbk = fast_path_blocked(sm, buf);
    const size_t tok0 = tok_begin + static_cast<size_t>(k) * C;
    const int nv = min(C, ntok - k * C);
    f32x4 yz[4];

    // ---- phase 1: producer stage A of chunk k+1; consumer Y / Z of chunk k
    if (produce) {
      write_kdt(kd);
      stage_a(k + 1, nbuf, raw, pr);
    } else {
      write_kdt(kd);
    }
    {
      // Y = (Kl exp R_I) S (waves 0,1) or Z = (Ql exp R_I) S (waves 2,3)
      const f16(*L)[LDK] = is_z ? sm.Ql[buf] : sm.Kl[buf];
      f16x8 sf[4];
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) sf[ks] = ld8(&sm.ST[16 * nb + lc][32 * ks + 8 * lg]);
#pragma unroll
      for (int I = 0; I < 4; ++I) {
        f16x8 a[4], f[4];
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          const int kc = 32 * ks + 8 * lg;
          a[ks] = ld8(&L[16 * I + lc][kc]);
          f[ks] = ld8(&sm.fR[buf][I][kc]);
        }
        f32x4 acc = zero4();
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) acc = mfma32(a[ks] * f[ks], sf[ks], acc);
        yz[I] = acc;
      }
      if (!is_z) {  // X = beta (V - Y)
#pragma unroll
        for (int I = 0; I < 4; ++I) {
          const float4 b4 = *reinterpret_cast<const float4*>(&sm.beta[buf][16 * I + 4 * lg]);
          const float bt[4] = {b4.x, b4.y, b4.z, b4.w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int i = 16 * I + 4 * lg + e;
            yz[I][e] = bt[e] * ((float)sm.V[buf][i][16 * nb + lc] - yz[I][e]);
          }
        }
      }
    }
    lds_barrier();

    // ---- phase 2: producer factors of chunk k+1 and loads of chunk k+2;
    // consumer Delta_I = T_II (X_I - sum_{J<I} A_IJ Delta_J)  (waves 0,1)
    if (produce) {
      factors(nbuf, kd);
      load_raw(min(k + 2, nch - 1), raw);
    }
    if (!is_z) {
      f16x4 dh[4];
#pragma unroll
      for (int I = 0; I < 4; ++I) {
        f32x4 r = yz[I];
#pragma unroll
        for (int J = 0; J < I; ++J) r = mfma16(-sm.frag[buf][SLOT_A + pair6(I, J)][lane], dh[J], r);
        dh[I] = h4(mfma16(sm.frag[buf][I][lane], h4(r), zero4()));
        *reinterpret_cast<f16x4*>(&sm.DT[16 * nb + lc][16 * I + 4 * lg]) = dh[I];
      }
    }
    lds_barrier();

    // ---- phase 3: producer products of chunk k+1; consumer O = scale (Z + Aqk Delta)
    // (waves 2,3) and S = exp(gamma) S + Kd^T Delta (all waves)
    if (produce) {
      const bool bad = products(nbuf, pr.bad);
      const bool any = __builtin_amdgcn_ballot_w64(bad) != 0;
      if (lane == 0) sm.fbp[nbuf][pw] = any;
    }
    if (is_z) {
#pragma unroll
      for (int I = 0; I < 4; ++I) {
        f32x4 o = yz[I];
#pragma unroll
        for (int J = 0; J <= I; ++J)
          o = mfma16(sm.frag[buf][SLOT_Q + tile10(I, J)][lane], ld4(&sm.DT[16 * nb + lc][16 * J + 4 * lg]), o);
        float* ob = p.out + (tok0 * H + h) * D + col0 + 16 * nb + lc;
        if (nv == C) {
#pragma unroll
          for (int e = 0; e < 4; ++e) ob[static_cast<unsigned>((16 * I + 4 * lg + e) * H * D)] = p.scale * o[e];
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int i = 16 * I + 4 * lg + e;
            if (i < nv) ob[static_cast<unsigned>(i * H * D)] = p.scale * o[e];
          }
        }
      }
    }
    if (!fbk) {  // workgroup-uniform; a chunk taken token by token keeps its entry state
#pragma unroll
    for (int a = 0; a < 2; ++a) {
      const float4 g4 = *reinterpret_cast<const float4*>(&sm.fGam[buf][32 * cw + 16 * a + 4 * lg]);
      const float gg[4] = {g4.x, g4.y, g4.z, g4.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        s[a][0][e] *= gg[e];
        s[a][1][e] *= gg[e];
      }
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int J = 0; J < 4; ++J)
          s[a][b] = mfma16(ld4(&sm.u.kk.KdT[32 * cw + 16 * a + lc][16 * J + 4 * lg]),
                           ld4(&sm.DT[16 * b + lc][16 * J + 4 * lg]), s[a][b]);
    }
    write_st(s);
    }
    lds_barrier();

    if (fbk) {  // workgroup-uniform
      const fb::Args fa{p.q, p.k, p.v, p.log_g, p.beta, p.out, p.H, p.scale};
      fb::eval_chunk<4>(sm.u.fb, s, fa, tok_begin, ntok, k, h, col0);
      write_st(s);
      lds_barrier();
    }
  };

  for (int k = 0; k + 1 < nch; ++k) chunk_step(k, true);
  if (nch > 0) chunk_step(nch - 1, false);

  if (p.final_state) {
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          p.final_state[unit_state + (32 * cw + 16 * a + 4 * lg + e) * D + col0 + 16 * b + lc] = s[a][b][e];
  }
}

}  // namespace

size_t chunk_workspace_bytes(int n_docs, bool packed) {
  if (!packed || n_docs <= 0) return 0;
  return ((static_cast<size_t>(n_docs) * sizeof(int32_t) + 255) / 256) * 256;
}

bool chunk_mfma_supported(const ChunkLaunch& a) { return a.bf16 && a.d == D; }

hipError_t launch_chunk_mfma(const ChunkLaunch& a, hipStream_t stream) {
  {  // the kernel's LDS limit is raised once per device (the attribute is per device)
    constexpr int MAX_DEV = 64;
    static bool ready[MAX_DEV] = {};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= MAX_DEV) return hipErrorInvalidDevice;
    if (!ready[dev]) {
      e = hipFuncSetAttribute(reinterpret_cast<const void*>(chunk_kernel), hipFuncAttributeMaxDynamicSharedMemorySize,
                              static_cast<int>(sizeof(Smem)));
      if (e != hipSuccess) return e;
      ready[dev] = true;
    }
  }
  ChunkArgs p{};
  p.q = static_cast<const bf16_t*>(a.q);
  p.k = static_cast<const bf16_t*>(a.k);
  p.v = static_cast<const bf16_t*>(a.v);
  p.log_g = a.log_g;
  p.beta = a.beta;
  p.init_state = a.init_state;
  p.final_state = a.final_state;
  p.cu_seqlens = a.cu_seqlens;
  p.order = nullptr;
  p.out = static_cast<float*>(a.out);
  p.num_docs = a.num_seqs;
  p.T = a.seq_len;
  p.H = a.num_heads;
  p.scale = a.scale;
  if (a.cu_seqlens && a.num_seqs > 1 && a.num_seqs <= 4096 && a.workspace) {
    int32_t* order = static_cast<int32_t*>(a.workspace);
    const hipError_t e = launch_doc_order(a.cu_seqlens, a.num_seqs, order, stream);
    if (e != hipSuccess) return e;
    p.order = order;
  }
  const unsigned units = static_cast<unsigned>(a.num_seqs) * static_cast<unsigned>(a.num_heads);
  const unsigned blocks = ((units + 7) / 8) * 8 * NTILE;
  hipLaunchKernelGGL(chunk_kernel, dim3(blocks), dim3(NT), sizeof(Smem), stream, p);
  return hipGetLastError();
}

}  // namespace kda
