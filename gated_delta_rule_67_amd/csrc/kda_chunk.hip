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
// One workgroup (4 waves) owns one (unit, 32-column value tile) and walks the
// unit's chunks in order with its fp32 state tile S[128][32] resident in MFMA
// accumulator registers.  Value columns are independent, so a unit's 4 tiles
// run as 4 workgroups (placed on one XCD so they share q/k/log_g in its L2).
//
// Decay factors without overflow.  The chunk is cut into four 16-token blocks.
// For block I with reference R_I = G at its first token's predecessor:
//   Kl = k exp(G - R_I) <= |k|, Ql = q exp(G - R_I), Kr = k exp(R_{I+1} - G) <= |k|
// come from prefix / suffix products of exp(log_g) inside the block (thread
// local).  Off-diagonal tiles (I > J) of A and Aqk use Kl_I * exp(R_I - R_{J+1})
// against Kr_J: every factor is <= 1 for any gate.  Diagonal tiles use a
// mid-block reference M_I (after the block's 8th token): Kl_I * exp(R_I - M_I)
// against Kr_I * exp(M_I - R_{I+1}); these factors are >= 1 and are bounded by
// exp(HALF_SPAN_MAX).  A chunk whose half-block decay exceeds that bound, or
// whose inputs could overflow the fp16 MFMA operands, is evaluated token by
// token (exact fp32) instead, inside this kernel.
//
// Arithmetic: fp16 MFMA operands (bf16 q/k/v convert exactly), fp32
// accumulation, fp32 state and outputs.  (I + A)^-1 is applied by blocked
// forward substitution: the four 16x16 diagonal blocks are inverted in fp32 on
// the VALU, then Delta_I = T_II (X_I - sum_{J<I} A_IJ Delta_J) chains 16x16x16
// MFMAs whose C-layout outputs are directly the next B operands.
#include "kda_common.h"
#include "kda_launch.h"

namespace kda {
namespace {

typedef _Float16 f16;
typedef f16 f16x2 __attribute__((ext_vector_type(2)));
typedef f16 f16x4 __attribute__((ext_vector_type(4)));
typedef f16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int C = 64;        // chunk length
constexpr int D = 128;       // head dim (dk = dv)
constexpr int DVT = 32;      // value columns per workgroup
constexpr int NTILE = D / DVT;
constexpr int NT = 256;      // threads (4 waves)
constexpr int LDK = D + 8;   // fp16 row stride of [64][128] matrices
constexpr int LDT = C + 8;   // fp16 row stride of [*][64] matrices
constexpr int LDA = C + 4;   // fp32 row stride of A
constexpr int LDV = DVT + 4; // fp32 row stride of V
constexpr float HALF_SPAN_MAX = 6.0f;   // max decay (in e-folds) over half a block
constexpr float QK_MAX = 64.0f;         // |q|, |k| bound of the fast path
constexpr float V_MAX = 4096.0f;        // |v| bound of the fast path
constexpr float S_MAX = 2048.0f;        // |S| bound of the fast path
constexpr float BETA_MAX = 2.0f;        // |beta| bound of the fast path
constexpr int FB_TG = 16;               // tokens staged per pass in the fallback

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

struct __align__(16) Smem {
  f16 Kl[C][LDK];       // k exp(G - R_blk)            (also fallback staging)
  f16 Ql[C][LDK];       // q exp(G - R_blk)
  f16 Kr[C][LDK];       // k exp(R_blk_end - G)
  f16 KdT[D][LDT];      // (k exp(gamma - G))^T        [channel][token]
  f16 ST[DVT][LDK];     // S^T in fp16                 [value col][channel]
  float A32[C][LDA];    // beta_i * P, strictly lower (fp32, diagonal inverses read it)
  f16 Ah[C][LDT];       // same in fp16 (off-diagonal blocks feed the substitution)
  f16 Aqk[C][LDT];      // q k decay products, lower incl. diagonal
  f16 Td[4][16][20];    // inverses of the four diagonal blocks of (I + A)
  f16 DT[DVT][LDT];     // Delta^T                     [value col][token]
  float V[C][LDV];      // value tile of the chunk (fp32)
  float beta[C];
  float tot[4][D];      // per-block products of exp(log_g)
  f16 fR[4][D];         // exp(R_I)
  f16 fOff[6][D];       // exp(R_I - R_{J+1}), I > J
  f16 fDl[4][D];        // exp(R_I - M_I)
  f16 fDr[4][D];        // exp(M_I - R_{I+1})
  float fGam[D];        // exp(gamma)
  float red[2][4][DVT][2];  // fallback column reductions
  float kq[FB_TG];
};

// Fallback staging aliases the fast-path operand buffers.
struct FbStage {
  float a[FB_TG][D];
  float k[FB_TG][D];
  float q[FB_TG][D];
};
static_assert(sizeof(FbStage) <= 3 * sizeof(f16) * C * LDK, "fallback staging does not fit");

__device__ __forceinline__ f32x4 mfma32(f16x8 a, f16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16(f16x4 a, f16x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f16x8 ld8(const f16* p) { return *reinterpret_cast<const f16x8*>(p); }
__device__ __forceinline__ f16x4 ld4(const f16* p) { return *reinterpret_cast<const f16x4*>(p); }
__device__ __forceinline__ f16x4 to_h4(f32x4 x) {
  f16x4 r;
  r[0] = (f16)x[0]; r[1] = (f16)x[1]; r[2] = (f16)x[2]; r[3] = (f16)x[3];
  return r;
}

// (I, J) of the ten lower 16x16 tiles of a 64x64 matrix, and the index of the
// off-diagonal pair in fOff.
__device__ __forceinline__ void tile_ij(int t, int& I, int& J) {
  // 0:(0,0) 1:(1,0) 2:(1,1) 3:(2,0) 4:(2,1) 5:(2,2) 6:(3,0) 7:(3,1) 8:(3,2) 9:(3,3)
  I = t >= 6 ? 3 : t >= 3 ? 2 : t >= 1 ? 1 : 0;
  J = t - (I * (I + 1)) / 2;
}
__device__ __forceinline__ int off_pair(int I, int J) { return (I * (I - 1)) / 2 + J; }  // I > J

__global__ void __launch_bounds__(NT) doc_order_kernel(const int32_t* __restrict__ cu, int n,
                                                       int32_t* __restrict__ order) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const int li = cu[i + 1] - cu[i];
  int rank = 0;
  for (int j = 0; j < n; ++j) {
    const int lj = cu[j + 1] - cu[j];
    rank += (lj > li) || (lj == li && j < i);
  }
  order[rank] = i;
}

// Token-by-token evaluation of one chunk (exact fp32), on the state held in
// MFMA C layout: s[a][b][e] = S[32w + 16a + 4(l/16) + e][16b + (l%16)].
__device__ void chunk_fallback(Smem& sm, f32x4 (&s)[2][2], const ChunkArgs& p, size_t tok0, int nv,
                               int h, int col0) {
  FbStage& st = *reinterpret_cast<FbStage*>(&sm.Kl[0][0]);
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, lc = lane & 15, lg = lane >> 4;
  const int H = p.H;
  for (int t0 = 0; t0 < nv; t0 += FB_TG) {
    const int tg = min(FB_TG, nv - t0);
    __syncthreads();
    {
      constexpr int PER = FB_TG * D / NT;  // elements per thread per pass
      float la[PER], lk[PER], lq[PER];
#pragma unroll
      for (int u = 0; u < PER; ++u) {
        const int idx = tid + u * NT, r = min(idx / D, tg - 1), c = idx % D;
        const size_t row = (tok0 + t0 + r) * H + h;
        la[u] = p.log_g[row * D + c];
        lk[u] = to_f32(p.k[row * D + c]);
        lq[u] = to_f32(p.q[row * D + c]);
      }
#pragma unroll
      for (int u = 0; u < PER; ++u) {
        const int idx = tid + u * NT, r = idx / D, c = idx % D;
        st.a[r][c] = exp_fast(la[u]);
        st.k[r][c] = lk[u];
        st.q[r][c] = lq[u];
      }
    }
    __syncthreads();
    {  // kq[r] = k_r . q_r : 16 lanes per token, 8 channels each
      const int r = tid >> 4, c0 = (tid & 15) * 8;
      float acc = 0.f;
      if (r < tg) {
#pragma unroll
        for (int c = 0; c < 8; ++c) acc += st.k[r][c0 + c] * st.q[r][c0 + c];
      }
#pragma unroll
      for (int off = 1; off < 16; off <<= 1) acc += __shfl_xor(acc, off);
      if ((tid & 15) == 0 && r < tg) sm.kq[r] = acc;
    }
    __syncthreads();
    for (int r = 0; r < tg; ++r) {
      const int par = (t0 + r) & 1;
      float pa[2] = {0.f, 0.f}, pb[2] = {0.f, 0.f};
#pragma unroll
      for (int a = 0; a < 2; ++a) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int c = 32 * w + 16 * a + 4 * lg + e;
          const float al = st.a[r][c], kc = st.k[r][c], qc = st.q[r][c];
#pragma unroll
          for (int b = 0; b < 2; ++b) {
            s[a][b][e] *= al;
            pa[b] += s[a][b][e] * kc;
            pb[b] += s[a][b][e] * qc;
          }
        }
      }
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        pa[b] += __shfl_xor(pa[b], 16); pa[b] += __shfl_xor(pa[b], 32);
        pb[b] += __shfl_xor(pb[b], 16); pb[b] += __shfl_xor(pb[b], 32);
      }
      if (lg == 0) {
#pragma unroll
        for (int b = 0; b < 2; ++b) {
          sm.red[par][w][16 * b + lc][0] = pa[b];
          sm.red[par][w][16 * b + lc][1] = pb[b];
        }
      }
      __syncthreads();
      const float bt = sm.beta[t0 + r], kq = sm.kq[r];
      float dl[2];
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        const int n = 16 * b + lc;
        float A = 0.f, B = 0.f;
#pragma unroll
        for (int ww = 0; ww < 4; ++ww) {
          A += sm.red[par][ww][n][0];
          B += sm.red[par][ww][n][1];
        }
        dl[b] = bt * (sm.V[t0 + r][n] - A);
        if (w == 0 && lg == 0)
          p.out[((tok0 + t0 + r) * H + h) * D + col0 + n] = p.scale * (B + dl[b] * kq);
      }
#pragma unroll
      for (int a = 0; a < 2; ++a) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float kc = st.k[r][32 * w + 16 * a + 4 * lg + e];
#pragma unroll
          for (int b = 0; b < 2; ++b) s[a][b][e] += kc * dl[b];
        }
      }
    }
  }
}

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
  size_t tok_begin;
  int ntok;
  if (p.cu_seqlens) {
    tok_begin = p.cu_seqlens[doc];
    ntok = p.cu_seqlens[doc + 1] - p.cu_seqlens[doc];
  } else {
    tok_begin = static_cast<size_t>(doc) * p.T;
    ntok = p.T;
  }
  const int H = p.H;
  const size_t unit_state = (static_cast<size_t>(doc) * H + h) * D * D;

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, lc = lane & 15, lg = lane >> 4;

  // Zero the never-written upper parts once: Aqk above the diagonal blocks and
  // the diagonal-block inverses' upper triangles are read as zeros.
  for (int idx = tid; idx < C * LDT; idx += NT) {
    (&sm.Aqk[0][0])[idx] = (f16)0.f;
    (&sm.Ah[0][0])[idx] = (f16)0.f;
  }

  // ---- initial state in C layout: s[a][b][e] = S[32w+16a+4lg+e][col0+16b+lc]
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
  bool s_big = false;
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b) {
#pragma unroll
      for (int e = 0; e < 4; ++e) s_big |= !(fabsf(s[a][b][e]) <= S_MAX);
      *reinterpret_cast<f16x4*>(&sm.ST[16 * b + lc][32 * w + 16 * a + 4 * lg]) = to_h4(s[a][b]);
    }

  const int cp = tid & 63;     // channel pair: channels 2cp, 2cp+1
  const int c0 = 2 * cp;
  const int blk = w;           // token block of this thread in stage A
  const float lim_lo = __expf(-HALF_SPAN_MAX);

  for (int cs = 0; cs < ntok; cs += C) {
    const int nv = min(C, ntok - cs);  // valid rows of this chunk
    const size_t tok0 = tok_begin + cs;

    // ---------------- stage A: loads, gate products, base operands
    float P[16][2], Sf[16][2];
    uint32_t kk[16], qq[16];
    bool bad = s_big;
    {
      // Loads are issued unconditionally (rows past the end of the document
      // re-read its last row) so that all of them are in flight at once; the
      // padding rows are then replaced by identity tokens (k = q = v = 0,
      // log_g = 0, beta = 0).
      float2 lgv[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int r = min(16 * blk + i, nv - 1);
        const size_t row = (tok0 + r) * H + h;
        lgv[i] = *reinterpret_cast<const float2*>(p.log_g + row * D + c0);
        kk[i] = *reinterpret_cast<const uint32_t*>(p.k + row * D + c0);
        qq[i] = *reinterpret_cast<const uint32_t*>(p.q + row * D + c0);
      }
      const int vr = tid >> 2, vc = (tid & 3) * 8;  // V: 64 rows x 4 threads x 8 columns
      const uint4 vraw =
          *reinterpret_cast<const uint4*>(p.v + ((tok0 + min(vr, nv - 1)) * H + h) * D + col0 + vc);
      const float braw = p.beta[(tok0 + min(tid & (C - 1), nv - 1)) * H + h];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        if (16 * blk + i >= nv) {
          lgv[i] = make_float2(0.f, 0.f);
          kk[i] = 0u;
          qq[i] = 0u;
        }
      }
      if (tid < C) {
        const float bv = tid < nv ? braw : 0.f;
        sm.beta[tid] = bv;
        bad |= !(fabsf(bv) <= BETA_MAX);
      }
      {
        float vv[8] = {bf16_lo(vraw.x), bf16_hi(vraw.x), bf16_lo(vraw.y), bf16_hi(vraw.y),
                       bf16_lo(vraw.z), bf16_hi(vraw.z), bf16_lo(vraw.w), bf16_hi(vraw.w)};
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          if (vr >= nv) vv[j] = 0.f;
          sm.V[vr][vc + j] = vv[j];
          bad |= !(fabsf(vv[j]) <= V_MAX);
        }
      }
      float al[16][2];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        al[i][0] = exp_fast(lgv[i].x);
        al[i][1] = exp_fast(lgv[i].y);
      }
#pragma unroll
      for (int ch = 0; ch < 2; ++ch) {
        float pr = 1.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) { pr *= al[i][ch]; P[i][ch] = pr; }
        float sf = 1.f;
#pragma unroll
        for (int i = 15; i >= 0; --i) { Sf[i][ch] = sf; sf *= al[i][ch]; }
        sm.tot[blk][c0 + ch] = P[15][ch];
        // diagonal-tile factors around the mid-block reference
        const float dl = P[7][ch], dr = Sf[7][ch];
        bad |= !(dl >= lim_lo) || !(dr >= lim_lo);
        sm.fDl[blk][c0 + ch] = (f16)(1.f / fmaxf(dl, lim_lo));
        sm.fDr[blk][c0 + ch] = (f16)(1.f / fmaxf(dr, lim_lo));
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int r = 16 * blk + i;
        const float k0 = bf16_lo(kk[i]), k1 = bf16_hi(kk[i]);
        const float q0 = bf16_lo(qq[i]), q1 = bf16_hi(qq[i]);
        bad |= !(fabsf(k0) <= QK_MAX) || !(fabsf(k1) <= QK_MAX) || !(fabsf(q0) <= QK_MAX) ||
               !(fabsf(q1) <= QK_MAX);
        f16x2 hk, hq, hr;
        hk[0] = (f16)(k0 * P[i][0]); hk[1] = (f16)(k1 * P[i][1]);
        hq[0] = (f16)(q0 * P[i][0]); hq[1] = (f16)(q1 * P[i][1]);
        hr[0] = (f16)(k0 * Sf[i][0]); hr[1] = (f16)(k1 * Sf[i][1]);
        *reinterpret_cast<f16x2*>(&sm.Kl[r][c0]) = hk;
        *reinterpret_cast<f16x2*>(&sm.Ql[r][c0]) = hq;
        *reinterpret_cast<f16x2*>(&sm.Kr[r][c0]) = hr;
      }
    }
    const bool fallback = __syncthreads_or(bad);  // also publishes tot/fDl/fDr/V/beta

    if (fallback) {
      chunk_fallback(sm, s, p, tok0, nv, h, col0);
    } else {
      // ---------------- factors from the block totals; Kd^T
      {
        float Qt[4][2];
#pragma unroll
        for (int I = 0; I < 4; ++I) { Qt[I][0] = sm.tot[I][c0]; Qt[I][1] = sm.tot[I][c0 + 1]; }
#pragma unroll
        for (int ch = 0; ch < 2; ++ch) {
          const int c = c0 + ch;
          // e^{gamma - R_{blk+1}}: product of the totals of the later blocks
          float gd = 1.f;
#pragma unroll
          for (int I = 3; I > 0; --I)
            if (I > blk) gd *= Qt[I][ch];
          f16 col[16];
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const float kv = ch == 0 ? bf16_lo(kk[i]) : bf16_hi(kk[i]);
            col[i] = (f16)(kv * Sf[i][ch] * gd);
          }
          *reinterpret_cast<f16x8*>(&sm.KdT[c][16 * blk]) =
              f16x8{col[0], col[1], col[2], col[3], col[4], col[5], col[6], col[7]};
          *reinterpret_cast<f16x8*>(&sm.KdT[c][16 * blk + 8]) =
              f16x8{col[8], col[9], col[10], col[11], col[12], col[13], col[14], col[15]};
          if (blk == 0) {
            float r = 1.f;
#pragma unroll
            for (int I = 0; I < 4; ++I) { sm.fR[I][c] = (f16)r; r *= Qt[I][ch]; }
            sm.fGam[c] = r;
            sm.fOff[off_pair(1, 0)][c] = (f16)1.f;
            sm.fOff[off_pair(2, 0)][c] = (f16)Qt[1][ch];
            sm.fOff[off_pair(2, 1)][c] = (f16)1.f;
            sm.fOff[off_pair(3, 0)][c] = (f16)(Qt[1][ch] * Qt[2][ch]);
            sm.fOff[off_pair(3, 1)][c] = (f16)Qt[2][ch];
            sm.fOff[off_pair(3, 2)][c] = (f16)1.f;
          }
        }
      }
      __syncthreads();

      // ---------------- (a)/(b): A = Kl Kr^T and Aqk = Ql Kr^T, lower tiles
      for (int t = w; t < 20; t += 4) {
        int I, J;
        tile_ij(t % 10, I, J);
        const bool isq = t >= 10;
        const f16(*L)[LDK] = isq ? sm.Ql : sm.Kl;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          const int kc = 32 * ks + 8 * lg;
          f16x8 af = ld8(&L[16 * I + lc][kc]);
          f16x8 bf = ld8(&sm.Kr[16 * J + lc][kc]);
          if (I == J) {
            af = af * ld8(&sm.fDl[I][kc]);
            bf = bf * ld8(&sm.fDr[I][kc]);
          } else if (I > J + 1) {
            af = af * ld8(&sm.fOff[off_pair(I, J)][kc]);
          }
          acc = mfma32(af, bf, acc);
        }
        const int j = 16 * J + lc;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int i = 16 * I + 4 * lg + e;
          if (isq) {
            sm.Aqk[i][j] = (f16)(j <= i ? acc[e] : 0.f);
          } else {
            const float a = j < i ? sm.beta[i] * acc[e] : 0.f;
            sm.A32[i][j] = a;
            sm.Ah[i][j] = (f16)a;
          }
        }
      }

      // ---------------- (c)/(d): Y = Kg S (waves 0,1) and Z = Qg S (waves 2,3)
      // Kg = Kl exp(R_I) row block by row block; B operand S^T from LDS.
      const int nb = w & 1;           // value-column tile of 16 handled by this wave
      const bool is_z = w >= 2;
      f32x4 yz[4];
      {
        const f16(*L)[LDK] = is_z ? sm.Ql : sm.Kl;
#pragma unroll
        for (int I = 0; I < 4; ++I) {
          f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int ks = 0; ks < 4; ++ks) {
            const int kc = 32 * ks + 8 * lg;
            const f16x8 af = ld8(&L[16 * I + lc][kc]) * ld8(&sm.fR[I][kc]);
            const f16x8 bf = ld8(&sm.ST[16 * nb + lc][kc]);
            acc = mfma32(af, bf, acc);
          }
          yz[I] = acc;
        }
      }
      // X = beta (V - Y) on waves 0,1 (C layout rows 16I+4lg+e, column 16nb+lc)
      if (!is_z) {
#pragma unroll
        for (int I = 0; I < 4; ++I)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int i = 16 * I + 4 * lg + e;
            yz[I][e] = sm.beta[i] * (sm.V[i][16 * nb + lc] - yz[I][e]);
          }
      }
      __syncthreads();  // A32 / Ah / Aqk complete

      // ---------------- inverses of the diagonal blocks of (I + A), fp32 VALU
      {
        const int I = w;
        float x[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) x[i] = (i == lc) ? 1.f : 0.f;
#pragma unroll
        for (int j = 0; j < 16; ++j) {
#pragma unroll
          for (int i = j + 1; i < 16; ++i) x[i] -= sm.A32[16 * I + i][16 * I + j] * x[j];
        }
        if (lg == 0) {
#pragma unroll
          for (int i = 0; i < 16; ++i) sm.Td[I][i][lc] = (f16)x[i];
        }
      }
      __syncthreads();

      // ---------------- Delta by blocked forward substitution (waves 0,1)
      if (!is_z) {
        f16x4 dh[4];
#pragma unroll
        for (int I = 0; I < 4; ++I) {
          f32x4 r = yz[I];
#pragma unroll
          for (int J = 0; J < I; ++J) {
            const f16x4 a = -ld4(&sm.Ah[16 * I + lc][16 * J + 4 * lg]);
            r = mfma16(a, dh[J], r);
          }
          f32x4 z = {0.f, 0.f, 0.f, 0.f};
          const f32x4 d = mfma16(ld4(&sm.Td[I][lc][4 * lg]), to_h4(r), z);
          dh[I] = to_h4(d);
          *reinterpret_cast<f16x4*>(&sm.DT[16 * nb + lc][16 * I + 4 * lg]) = dh[I];
        }
      }
      __syncthreads();

      // ---------------- O = scale (Z + Aqk Delta) (waves 2,3)
      if (is_z) {
#pragma unroll
        for (int I = 0; I < 4; ++I) {
          f32x4 o = yz[I];
#pragma unroll
          for (int J = 0; J <= I; ++J)
            o = mfma16(ld4(&sm.Aqk[16 * I + lc][16 * J + 4 * lg]), ld4(&sm.DT[16 * nb + lc][16 * J + 4 * lg]), o);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int i = 16 * I + 4 * lg + e;
            if (i < nv) p.out[((tok0 + i) * H + h) * D + col0 + 16 * nb + lc] = p.scale * o[e];
          }
        }
      }

      // ---------------- S = exp(gamma) S + Kd^T Delta (all waves)
#pragma unroll
      for (int a = 0; a < 2; ++a) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float g = sm.fGam[32 * w + 16 * a + 4 * lg + e];
          s[a][0][e] *= g;
          s[a][1][e] *= g;
        }
#pragma unroll
        for (int b = 0; b < 2; ++b) {
#pragma unroll
          for (int J = 0; J < 4; ++J)
            s[a][b] = mfma16(ld4(&sm.KdT[32 * w + 16 * a + lc][16 * J + 4 * lg]),
                             ld4(&sm.DT[16 * b + lc][16 * J + 4 * lg]), s[a][b]);
        }
      }
    }

    // ---------------- S^T (fp16) for the next chunk; magnitude guard
    __syncthreads();  // everyone is done reading ST / DT / staging of this chunk
    s_big = false;
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int b = 0; b < 2; ++b) {
#pragma unroll
        for (int e = 0; e < 4; ++e) s_big |= !(fabsf(s[a][b][e]) <= S_MAX);
        *reinterpret_cast<f16x4*>(&sm.ST[16 * b + lc][32 * w + 16 * a + 4 * lg]) = to_h4(s[a][b]);
      }
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

}  // namespace

size_t chunk_workspace_bytes(int n_docs, bool packed) {
  if (!packed || n_docs <= 0) return 0;
  return ((static_cast<size_t>(n_docs) * sizeof(int32_t) + 255) / 256) * 256;
}

bool chunk_mfma_supported(const ChunkLaunch& a) { return a.bf16 && a.d == D; }

hipError_t launch_chunk_mfma(const ChunkLaunch& a, hipStream_t stream) {
  static bool attr_set = false;
  if (!attr_set) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(chunk_kernel),
                                             hipFuncAttributeMaxDynamicSharedMemorySize,
                                             static_cast<int>(sizeof(Smem)));
    if (e != hipSuccess) return e;
    attr_set = true;
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
  if (a.cu_seqlens && a.num_seqs > 1 && a.num_seqs <= 4096 && a.doc_order) {
    const int n = a.num_seqs;
    hipLaunchKernelGGL(doc_order_kernel, dim3((n + NT - 1) / NT), dim3(NT), 0, stream, a.cu_seqlens, n,
                       a.doc_order);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    p.order = a.doc_order;
  }
  const unsigned units = static_cast<unsigned>(a.num_seqs) * static_cast<unsigned>(a.num_heads);
  const unsigned blocks = ((units + 7) / 8) * 8 * NTILE;
  hipLaunchKernelGGL(chunk_kernel, dim3(blocks), dim3(NT), sizeof(Smem), stream, p);
  return hipGetLastError();
}

}  // namespace kda
