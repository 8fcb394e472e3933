// kda_backward.hip -- reverse mode of the chunked KDA prefill (gfx950).
//
// The loss L = sum(d_out * out) + sum(d_final * final_state) is differentiated
// through the gated delta rule (NeMo glm5_next.layers: `_torch_recurrent_kda`
// is the differentiable reference; the KDA parameters are trained under FSDP).
// Everything is fp32: operands, MFMA (v_mfma_f32_16x16x4_f32) and state.
//
// Chunk form (64 tokens, one unit = (sequence or document, head)).  Inside a
// chunk with entry state S, b_t = prod_{u<=t} alpha_u (alpha = exp(log_g), per
// key channel), r(t,s) = prod_{s<u<=t} alpha_u:
//
//   Akk[t,s] = sum_i k_t k_s r(t,s) (s < t),  Aqk[t,s] = sum_i q_t k_s r(t,s) (s <= t)
//   T = (I + diag(beta) Akk)^-1,  W = T diag(beta) (K*b),  U = T diag(beta) V
//   Delta = U - W S,  O = scale((Q*b) S + Aqk Delta),  S' = b_C S + Kd^T Delta
//   with Kd_t = k_t r(C-1, t).
//
// Reverse mode, per chunk, given dO and the exit-state gradient dS':
//   dDelta = scale Aqk^T dO + Kd dS'          dR = T^T dDelta
//   dS     = b_C dS' + scale (Q*b)^T dO - W^T dDelta
//   dv = beta dR,   dbeta = rowsum(dR * (V - (K*b) S)) + rowsum(dA * Akk)
//   dA = -tril(dR Delta^T, -1),  dAqk = scale tril(dO Delta^T)
//   d(K*b) = -beta dR S^T,  d(Q*b) = scale dO S^T,  dKd = Delta dS'^T
// and the decay-weighted pairs pass gradients to q, k and the cumulative log
// decays G (dG_t gets +x_t dx_t through the later index of a pair and -y_s dy_s
// through the earlier one); log_g gets the reverse cumulative sum of dG.
//
// Pair products without overflow for any gate (-inf included): the lower
// triangle of a chunk is split by a binary tree.  At level l (l = 0..5) the
// tiles are 64 >> l tokens wide; a pair (t, s) belongs to level l when t is in
// the upper half and s in the lower half of the same level-l tile.  Then
// r(t,s) = F_l(t) F_l(s) with F_l(t) = product of alpha from the first token
// of t's half to t (upper half) or from t+1 to the last token of the half
// (lower half).  Every factor is a product of gates <= 1, so the MFMA operands
// x_t F_l(t) and y_s F_l(s) are bounded by the inputs.  Pairs t = s have r = 1.
//
// Kernels, in launch order (slots are chunks, one workgroup per (slot, head)
// or per (unit, value-column tile)):
//   bwd_prep      per chunk: Akk, Aqk, T, W, U, Kd, scale*(Q*b), b_C
//   bwd_fscan     per unit, serially over its chunks: entry states S, Delta
//   bwd_rscan     per unit, backwards: exit-state gradients dS', dDelta, dS0
//   bwd_gstate    per chunk: dv, dbeta, dAqk, dA and the state-side parts of
//                 dq, dk and dG (staged in the dq, dk, dlog_g outputs)
//   bwd_gpairs    per chunk: the pair terms, then dlog_g = reverse cumsum(dG)
#include <algorithm>

#include "kda_common.h"
#include "kda_launch.h"

namespace kda {
namespace {

constexpr int C = 64;    // tokens per chunk
constexpr int NT = 256;  // threads per workgroup: 4 waves

__device__ __forceinline__ f32x4 mma(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const float* log_g;
  const float* beta;
  const float* init_state;  // [N, H, D, D] or null (zeros)
  const int32_t* cu;        // packed: [N+1] token offsets; dense: null
  const int32_t* cstart;    // packed: [N+1] first chunk slot of each document
  const int32_t* table;     // packed: [n_slots] document of each slot, -1 unused
  const float* d_out;       // [tokens, H, D]
  const float* d_final;     // [N, H, D, D] or null (zeros)
  float* dq;
  float* dk;
  float* dv;
  float* dlog_g;
  float* dbeta;
  float* d_init;  // [N, H, D, D] or null (not written)
  // workspace, one entry per (slot, head), index slot * H + h
  float* S_in;  // D x D   entry state of the chunk
  float* dSo;   // D x D   gradient of the chunk's exit state
  float* Wm;    // C x D
  float* Um;    // C x D
  float* Kd;    // C x D
  float* Qs;    // C x D   scale * q_t * b_t
  float* Dl;    // C x D   Delta
  float* dDl;   // C x D   dDelta
  float* As;    // C x C   scale * Aqk
  float* Tm;    // C x C
  float* Ab;    // C x C   Akk (strictly lower, beta not applied)
  float* dAq;   // C x C   dL/dAqk
  float* dAb;   // C x C   dL/dAkk
  float* eg;    // D       b_C
  int N;
  int T;
  int H;
  int cps;  // dense: chunks per sequence
  float scale;
};

struct Loc {
  int n;
  int64_t tok0;
  int count;
};

// Chunk slot c -> (document, first token, tokens in the chunk).
__device__ __forceinline__ bool locate(const BwdArgs& a, int c, Loc& L) {
  if (a.cu == nullptr) {
    if (a.cps == 0) return false;
    L.n = c / a.cps;
    if (L.n >= a.N) return false;
    const int j = c - L.n * a.cps;
    L.tok0 = static_cast<int64_t>(L.n) * a.T + static_cast<int64_t>(j) * C;
    L.count = min(C, a.T - j * C);
    return L.count > 0;
  }
  const int n = a.table[c];
  if (n < 0) return false;
  const int j = c - a.cstart[n];
  L.n = n;
  L.tok0 = static_cast<int64_t>(a.cu[n]) + static_cast<int64_t>(j) * C;
  L.count = min(C, a.cu[n + 1] - a.cu[n] - j * C);
  return L.count > 0;
}

// Chunk slots of unit document n: [first, first + count).
__device__ __forceinline__ void unit_chunks(const BwdArgs& a, int n, int& first, int& count) {
  if (a.cu == nullptr) {
    first = n * a.cps;
    count = a.cps;
  } else {
    first = a.cstart[n];
    count = a.cstart[n + 1] - first;
  }
}

// C rows of a [tokens, H, D] tensor into LDS (row stride LD), rows >= count zero.
// (The staging helpers run a compile-time number of iterations so that all of
// a thread's loads are in flight before its LDS stores.)
template <int D, int LD, typename In, int NTH = NT>
__device__ __forceinline__ void load_rows(float* dst, const In* src, int64_t tok0, int count, int H, int h) {
  constexpr int G = D / 4, N = C * G, IT = (N + NTH - 1) / NTH;
  float4 x[IT];
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int idx = it * NTH + threadIdx.x, t = idx / G, g4 = idx - t * G;
    x[it] = make_float4(0.f, 0.f, 0.f, 0.f);
    if (idx < N && t < count) x[it] = load4(src + ((tok0 + t) * H + h) * D + 4 * g4);
  }
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int idx = it * NTH + threadIdx.x, t = idx / G, g4 = idx - t * G;
    if (idx < N) *reinterpret_cast<float4*>(dst + t * LD + 4 * g4) = x[it];
  }
}

// A dense rows x cols fp32 matrix (contiguous) into LDS with row stride LD.
template <int ROWS, int COLS, int LD, int NTH = NT>
__device__ __forceinline__ void load_mat(float* dst, const float* src) {
  constexpr int G = COLS / 4, N = ROWS * G, IT = (N + NTH - 1) / NTH;
  float4 x[IT];
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int idx = it * NTH + threadIdx.x;
    if (idx < N) x[it] = load4(src + idx * 4);
  }
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int idx = it * NTH + threadIdx.x, t = idx / G, g4 = idx - t * G;
    if (idx < N) *reinterpret_cast<float4*>(dst + t * LD + 4 * g4) = x[it];
  }
}

// Columns [c0, c0 + COLS) of a dense rows x LDG matrix into LDS (stride LD).
template <int ROWS, int COLS, int LD>
__device__ __forceinline__ void load_cols(float* dst, const float* src, int ldg, int c0) {
  constexpr int G = COLS / 4, N = ROWS * G, IT = (N + NT - 1) / NT;
  float4 x[IT];
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int idx = it * NT + threadIdx.x, t = idx / G, g4 = idx - t * G;
    if (idx < N) x[it] = load4(src + static_cast<int64_t>(t) * ldg + c0 + 4 * g4);
  }
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int idx = it * NT + threadIdx.x, t = idx / G, g4 = idx - t * G;
    if (idx < N) *reinterpret_cast<float4*>(dst + t * LD + 4 * g4) = x[it];
  }
}

template <int ROWS, int COLS, int LD>
__device__ __forceinline__ void store_cols(float* dst, int ldg, int c0, const float* src) {
  constexpr int G = COLS / 4;
  for (int idx = threadIdx.x; idx < ROWS * G; idx += NT) {
    const int t = idx / G, g4 = idx - t * G;
    *reinterpret_cast<float4*>(dst + static_cast<int64_t>(t) * ldg + c0 + 4 * g4) =
        *reinterpret_cast<const float4*>(src + t * LD + 4 * g4);
  }
}

// Gates of one channel over 32 tokens [base, base + 32) of the chunk (1 past
// the document end).
template <int D>
__device__ __forceinline__ void load_alpha(float (&al)[32], const float* log_g, int64_t tok0, int count, int H, int h,
                                           int i, int base) {
#pragma unroll
  for (int u = 0; u < 32; ++u) {
    const int t = base + u;
    al[u] = t < count ? exp_fast(log_g[((tok0 + t) * H + h) * D + i]) : 1.f;
  }
}

// Level-l factors F_l(t) of one channel for tokens [base, base + 32), written
// to sF[t * LD + i] (see the header).
template <int L, int LD>
__device__ __forceinline__ void level_factors(const float (&al)[32], int base, int i, float* sF) {
  constexpr int HH = 32 >> L;  // half size
#pragma unroll
  for (int b0 = 0; b0 < 32; b0 += HH) {
    const bool upper = ((base + b0) & HH) != 0;
    if (upper) {
      float p = 1.f;
#pragma unroll
      for (int u = 0; u < HH; ++u) {
        p *= al[b0 + u];
        sF[(base + b0 + u) * LD + i] = p;
      }
    } else {
      float p = 1.f;
#pragma unroll
      for (int u = HH - 1; u >= 0; --u) {
        sF[(base + b0 + u) * LD + i] = p;
        p *= al[b0 + u];
      }
    }
  }
}

// Pair (t, s) is taken at level l.
__device__ __forceinline__ bool at_level(int l, int t, int s) {
  const int hh = 32 >> l;
  return ((t ^ s) < 2 * hh) && (t & hh) && !(s & hh);
}

__device__ __forceinline__ f32x4 zero4f() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// ---------------------------------------------------------------------------
// bwd_prep: per (chunk, head).
template <int D>
struct PrepL {
  static constexpr int LD = D + 4, LM = C + 4;
  static constexpr int CD = C * LD, CM = C * LM;
  static constexpr int R0 = 0;                          // K, later V
  static constexpr int R1 = R0 + CD;                    // Q, later K*b
  static constexpr int R2 = R1 + CD;                    // F, later Akk | Aqk
  static constexpr int R3 = R2 + (CD > 2 * CM ? CD : 2 * CM);  // T
  static constexpr int R4 = R3 + CM;                    // 4 x 16 x 17 wave scratch
  static constexpr int RB = R4 + 4 * 16 * 17;           // beta [C]
  static constexpr int RT = RB + C;                     // block totals [2][D]
  static constexpr int FLOATS = RT + 2 * D;
  static constexpr size_t BYTES = sizeof(float) * FLOATS;
};

template <int D, typename In>
__global__ void __launch_bounds__(NT) bwd_prep(BwdArgs a) {
  using P = PrepL<D>;
  constexpr int LD = P::LD, LM = P::LM;
  extern __shared__ __align__(16) float sm[];
  float* sK = sm + P::R0;
  float* sQ = sm + P::R1;
  float* sF = sm + P::R2;
  float* sAb = sm + P::R2;
  float* sAq = sm + P::R2 + P::CM;
  float* sT = sm + P::R3;
  float* sBeta = sm + P::RB;
  float* sTot = sm + P::RT;

  const int slot = blockIdx.x / a.H, h = blockIdx.x - slot * a.H;
  Loc L;
  if (!locate(a, slot, L)) return;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, r = lane & 15, kq = lane >> 4;
  const size_t sh = static_cast<size_t>(slot) * a.H + h;
  const In* q = static_cast<const In*>(a.q);
  const In* k = static_cast<const In*>(a.k);
  const In* v = static_cast<const In*>(a.v);

  load_rows<D, LD>(sK, k, L.tok0, L.count, a.H, h);
  load_rows<D, LD>(sQ, q, L.tok0, L.count, a.H, h);
  if (tid < C) sBeta[tid] = tid < L.count ? a.beta[(L.tok0 + tid) * a.H + h] : 0.f;
  // gates of channel ci over half ph of the chunk
  const int ci = tid % D, ph = tid / D;
  const bool chan = ph < 2;
  float al[32];
  if (chan) load_alpha<D>(al, a.log_g, L.tok0, L.count, a.H, h, ci, 32 * ph);

  f32x4 ab_d = zero4f(), aq_d = zero4f(), ab_0 = zero4f(), aq_0 = zero4f(), ab_1 = zero4f(), aq_1 = zero4f();
  // product of one 16 x 16 tile (I, J) with factors
  auto pair_tile = [&](int I, int J, f32x4& accK, f32x4& accQ) {
#pragma unroll 4
    for (int k0 = 0; k0 < D; k0 += 4) {
      const int kk = k0 + kq;
      const int ts = (16 * J + r) * LD + kk, tt = (16 * I + r) * LD + kk;
      const float ys = sK[ts] * sF[ts];
      const float ft = sF[tt];
      accK = mma(sK[tt] * ft, ys, accK);
      accQ = mma(sQ[tt] * ft, ys, accQ);
    }
  };
#pragma unroll
  for (int l = 0; l < 6; ++l) {
    __syncthreads();  // previous level done with sF; inputs loaded
    if (chan) {
      switch (l) {
        case 0: level_factors<0, LD>(al, 32 * ph, ci, sF); break;
        case 1: level_factors<1, LD>(al, 32 * ph, ci, sF); break;
        case 2: level_factors<2, LD>(al, 32 * ph, ci, sF); break;
        case 3: level_factors<3, LD>(al, 32 * ph, ci, sF); break;
        case 4: level_factors<4, LD>(al, 32 * ph, ci, sF); break;
        default: level_factors<5, LD>(al, 32 * ph, ci, sF); break;
      }
    }
    __syncthreads();
    if (l == 0) {
      pair_tile(2 + (w >> 1), w & 1, ab_0, aq_0);
    } else if (l == 1) {
      if (w < 2) pair_tile(w == 0 ? 1 : 3, w == 0 ? 0 : 2, ab_1, aq_1);
    } else {
      f32x4 tk = zero4f(), tq = zero4f();
      pair_tile(w, w, tk, tq);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const bool ok = at_level(l, 16 * w + 4 * kq + j, 16 * w + r);
        ab_d[j] += ok ? tk[j] : 0.f;
        aq_d[j] += ok ? tq[j] : 0.f;
      }
    }
  }
  // diagonal of Aqk: r(t, t) = 1
  {
    f32x4 tq = zero4f();
#pragma unroll 4
    for (int k0 = 0; k0 < D; k0 += 4) {
      const int kk = k0 + kq;
      tq = mma(sQ[(16 * w + r) * LD + kk], sK[(16 * w + r) * LD + kk], tq);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) aq_d[j] += (4 * kq + j == r) ? tq[j] : 0.f;
  }
  __syncthreads();  // everyone done with sF
  for (int idx = tid; idx < 2 * P::CM; idx += NT) sAb[idx] = 0.f;
  __syncthreads();
  auto put = [&](float* M, int I, int J, const f32x4& x) {
#pragma unroll
    for (int j = 0; j < 4; ++j) M[(16 * I + 4 * kq + j) * LM + 16 * J + r] = x[j];
  };
  put(sAb, w, w, ab_d);
  put(sAq, w, w, aq_d);
  put(sAb, 2 + (w >> 1), w & 1, ab_0);
  put(sAq, 2 + (w >> 1), w & 1, aq_0);
  if (w < 2) {
    put(sAb, w == 0 ? 1 : 3, w == 0 ? 0 : 2, ab_1);
    put(sAq, w == 0 ? 1 : 3, w == 0 ? 0 : 2, aq_1);
  }
  // block totals of the two halves for the cumulative decays
  if (chan) {
    float p = 1.f;
#pragma unroll
    for (int u = 0; u < 32; ++u) p *= al[u];
    sTot[ph * D + ci] = p;
  }
  __syncthreads();
  // Akk and scale * Aqk to the workspace
  for (int idx = tid; idx < C * C; idx += NT) {
    const int t = idx / C, s = idx - t * C;
    a.Ab[sh * C * C + idx] = sAb[t * LM + s];
    a.As[sh * C * C + idx] = a.scale * sAq[t * LM + s];
  }
  // per channel: b_t (prefix), Qs = scale q b, K*b (in place of Q), Kd = k r(C-1, t), b_C
  if (chan) {
    float b = ph == 1 ? sTot[ci] : 1.f;
#pragma unroll
    for (int u = 0; u < 32; ++u) {
      const int t = 32 * ph + u;
      b *= al[u];
      const float qv = sQ[t * LD + ci];
      a.Qs[(sh * C + t) * D + ci] = a.scale * qv * b;
      sQ[t * LD + ci] = sK[t * LD + ci] * b;
    }
    if (ph == 1) a.eg[sh * D + ci] = b;
    float rr = ph == 0 ? sTot[D + ci] : 1.f;
#pragma unroll
    for (int u = 31; u >= 0; --u) {
      const int t = 32 * ph + u;
      a.Kd[(sh * C + t) * D + ci] = sK[t * LD + ci] * rr;
      rr *= al[u];
    }
  }
  for (int idx = tid; idx < P::CM; idx += NT) sT[idx] = 0.f;
  __syncthreads();  // K no longer needed; T zeroed
  load_rows<D, LD>(sK, v, L.tok0, L.count, a.H, h);  // V
  // T = (I + diag(beta) Akk)^-1: diagonal 16 x 16 blocks by forward substitution
  if (tid < 64) {
    const int I = tid >> 4, c = tid & 15;
    float x[16];
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      float acc = (t == c) ? 1.f : 0.f;
      const float bt = sBeta[16 * I + t];
#pragma unroll
      for (int s = 0; s < t; ++s) acc -= bt * sAb[(16 * I + t) * LM + 16 * I + s] * x[s];
      x[t] = acc;
      sT[(16 * I + t) * LM + 16 * I + c] = acc;
    }
  }
  // off-diagonal blocks: T_IJ = -T_II sum_{J <= K < I} A_IK T_KJ
  float* scr = sm + P::R4 + w * 16 * 17;
  for (int I = 1; I < 4; ++I) {
    __syncthreads();
    if (w < I) {
      const int J = w;
      f32x4 x = zero4f();
      const float bI = sBeta[16 * I + r];
      for (int Kb = J; Kb < I; ++Kb) {
#pragma unroll
        for (int k0 = 0; k0 < 16; k0 += 4) {
          const int kk = k0 + kq;
          x = mma(bI * sAb[(16 * I + r) * LM + 16 * Kb + kk], sT[(16 * Kb + kk) * LM + 16 * J + r], x);
        }
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) scr[(4 * kq + j) * 17 + r] = x[j];
    }
    __syncthreads();
    if (w < I) {
      const int J = w;
      f32x4 y = zero4f();
#pragma unroll
      for (int k0 = 0; k0 < 16; k0 += 4) {
        const int kk = k0 + kq;
        y = mma(sT[(16 * I + r) * LM + 16 * I + kk], scr[kk * 17 + r], y);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) sT[(16 * I + 4 * kq + j) * LM + 16 * J + r] = -y[j];
    }
  }
  __syncthreads();
  for (int idx = tid; idx < C * C; idx += NT) {
    const int t = idx / C, s = idx - t * C;
    a.Tm[sh * C * C + idx] = sT[t * LM + s];
  }
  // W = T diag(beta) (K*b), U = T diag(beta) V; T is lower triangular
  const int kend = 16 * (w + 1);
  for (int ct = 0; ct < D / 16; ++ct) {
    f32x4 accW = zero4f(), accU = zero4f();
    for (int k0 = 0; k0 < kend; k0 += 4) {
      const int s = k0 + kq;
      const float tv = sT[(16 * w + r) * LM + s];
      const float bs = sBeta[s];
      accW = mma(tv, bs * sQ[s * LD + 16 * ct + r], accW);
      accU = mma(tv, bs * sK[s * LD + 16 * ct + r], accU);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int t = 16 * w + 4 * kq + j;
      a.Wm[(sh * C + t) * D + 16 * ct + r] = accW[j];
      a.Um[(sh * C + t) * D + 16 * ct + r] = accU[j];
    }
  }
}

// ---------------------------------------------------------------------------
// bwd_fscan: per (unit, value-column tile), serially over the unit's chunks.
template <int D>
struct ScanL {
  static constexpr int DVT = D < 32 ? D : 32;
  static constexpr int NTILE = D / DVT;
  static constexpr int LD = D + 4, LV = DVT + 4, LM = C + 4;
  // forward: state tile, W, Kd, U tile, Delta tile, b_C
  static constexpr int FS = 0, FW = FS + D * LV, FK = FW + C * LD, FU = FK + C * LD, FX = FU + C * LV,
                       FG = FX + C * LV, F_FLOATS = FG + D;
  // reverse: dS tile, Kd, Qs, W, dO tile, dDelta tile, b_C, As
  static constexpr int RS = 0, RK = RS + D * LV, RQ = RK + C * LD, RW = RQ + C * LD, RO = RW + C * LD,
                       RX = RO + C * LV, RG = RX + C * LV, RM = RG + D, R_FLOATS = RM + C * LM;
};

template <int D>
__global__ void __launch_bounds__(NT) bwd_fscan(BwdArgs a) {
  using P = ScanL<D>;
  constexpr int DVT = P::DVT, LD = P::LD, LV = P::LV;
  extern __shared__ __align__(16) float sm[];
  float* sS = sm + P::FS;
  float* sW = sm + P::FW;
  float* sKd = sm + P::FK;
  float* sU = sm + P::FU;
  float* sX = sm + P::FX;
  float* sG = sm + P::FG;

  const int unit = blockIdx.x / P::NTILE, tile = blockIdx.x - unit * P::NTILE;
  const int n = unit / a.H, h = unit - n * a.H;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, r = lane & 15, kq = lane >> 4;
  const int c0 = tile * DVT;
  int first, nch;
  unit_chunks(a, n, first, nch);

  // entry state of the first chunk
  for (int idx = tid; idx < D * DVT; idx += NT) {
    const int i = idx / DVT, j = idx - i * DVT;
    sS[i * LV + j] = a.init_state ? a.init_state[(static_cast<size_t>(n) * a.H + h) * D * D + i * D + c0 + j] : 0.f;
  }
  for (int c = 0; c < nch; ++c) {
    const size_t sh = static_cast<size_t>(first + c) * a.H + h;
    __syncthreads();  // previous chunk done with every buffer
    load_mat<C, D, LD>(sW, a.Wm + sh * C * D);
    load_mat<C, D, LD>(sKd, a.Kd + sh * C * D);
    load_cols<C, DVT, LV>(sU, a.Um + sh * C * D, D, c0);
    for (int i = tid; i < D; i += NT) sG[i] = a.eg[sh * D + i];
    store_cols<D, DVT, LV>(a.S_in + sh * D * D, D, c0, sS);
    __syncthreads();
    // Delta = U - W S
    for (int tq = w; tq < 4 * (DVT / 16); tq += 4) {
      const int tb = tq % 4, cb = tq / 4;
      f32x4 acc = zero4f();
#pragma unroll 4
      for (int k0 = 0; k0 < D; k0 += 4) {
        const int kk = k0 + kq;
        acc = mma(sW[(16 * tb + r) * LD + kk], sS[kk * LV + 16 * cb + r], acc);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int t = 16 * tb + 4 * kq + j, col = 16 * cb + r;
        const float dl = sU[t * LV + col] - acc[j];
        sX[t * LV + col] = dl;
        a.Dl[(sh * C + t) * D + c0 + col] = dl;
      }
    }
    __syncthreads();
    // S = b_C S + Kd^T Delta
    for (int tq = w; tq < (D / 16) * (DVT / 16); tq += 4) {
      const int ib = tq % (D / 16), cb = tq / (D / 16);
      f32x4 acc = zero4f();
#pragma unroll 4
      for (int k0 = 0; k0 < C; k0 += 4) {
        const int s = k0 + kq;
        acc = mma(sKd[s * LD + 16 * ib + r], sX[s * LV + 16 * cb + r], acc);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int i = 16 * ib + 4 * kq + j, col = 16 * cb + r;
        sS[i * LV + col] = sG[i] * sS[i * LV + col] + acc[j];
      }
    }
  }
}

// bwd_rscan: per (unit, value-column tile), backwards over the unit's chunks.
template <int D>
__global__ void __launch_bounds__(NT) bwd_rscan(BwdArgs a) {
  using P = ScanL<D>;
  constexpr int DVT = P::DVT, LD = P::LD, LV = P::LV, LM = P::LM;
  extern __shared__ __align__(16) float sm[];
  float* sS = sm + P::RS;  // dS tile
  float* sKd = sm + P::RK;
  float* sQs = sm + P::RQ;
  float* sW = sm + P::RW;
  float* sO = sm + P::RO;  // dO tile
  float* sX = sm + P::RX;  // dDelta tile
  float* sG = sm + P::RG;
  float* sAs = sm + P::RM;

  const int unit = blockIdx.x / P::NTILE, tile = blockIdx.x - unit * P::NTILE;
  const int n = unit / a.H, h = unit - n * a.H;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, r = lane & 15, kq = lane >> 4;
  const int c0 = tile * DVT;
  int first, nch;
  unit_chunks(a, n, first, nch);
  const size_t uo = (static_cast<size_t>(n) * a.H + h) * D * D;

  for (int idx = tid; idx < D * DVT; idx += NT) {
    const int i = idx / DVT, j = idx - i * DVT;
    sS[i * LV + j] = a.d_final ? a.d_final[uo + i * D + c0 + j] : 0.f;
  }
  for (int c = nch - 1; c >= 0; --c) {
    const int slot = first + c;
    const size_t sh = static_cast<size_t>(slot) * a.H + h;
    Loc L;
    locate(a, slot, L);
    __syncthreads();
    load_mat<C, C, LM>(sAs, a.As + sh * C * C);
    load_mat<C, D, LD>(sKd, a.Kd + sh * C * D);
    load_mat<C, D, LD>(sQs, a.Qs + sh * C * D);
    load_mat<C, D, LD>(sW, a.Wm + sh * C * D);
    for (int idx = tid; idx < C * (DVT / 4); idx += NT) {
      const int t = idx / (DVT / 4), g4 = idx - t * (DVT / 4);
      float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
      if (t < L.count) x = load4(a.d_out + ((L.tok0 + t) * a.H + h) * D + c0 + 4 * g4);
      *reinterpret_cast<float4*>(sO + t * LV + 4 * g4) = x;
    }
    for (int i = tid; i < D; i += NT) sG[i] = a.eg[sh * D + i];
    store_cols<D, DVT, LV>(a.dSo + sh * D * D, D, c0, sS);
    __syncthreads();
    // dDelta = As^T dO + Kd dS
    for (int tq = w; tq < 4 * (DVT / 16); tq += 4) {
      const int tb = tq % 4, cb = tq / 4;
      f32x4 acc = zero4f();
#pragma unroll 4
      for (int k0 = 0; k0 < C; k0 += 4) {
        const int s = k0 + kq;
        acc = mma(sAs[s * LM + 16 * tb + r], sO[s * LV + 16 * cb + r], acc);
      }
#pragma unroll 4
      for (int k0 = 0; k0 < D; k0 += 4) {
        const int kk = k0 + kq;
        acc = mma(sKd[(16 * tb + r) * LD + kk], sS[kk * LV + 16 * cb + r], acc);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int t = 16 * tb + 4 * kq + j, col = 16 * cb + r;
        sX[t * LV + col] = acc[j];
        a.dDl[(sh * C + t) * D + c0 + col] = acc[j];
      }
    }
    __syncthreads();
    // dS = b_C dS + Qs^T dO - W^T dDelta
    for (int tq = w; tq < (D / 16) * (DVT / 16); tq += 4) {
      const int ib = tq % (D / 16), cb = tq / (D / 16);
      f32x4 acc = zero4f();
#pragma unroll 4
      for (int k0 = 0; k0 < C; k0 += 4) {
        const int t = k0 + kq;
        acc = mma(sQs[t * LD + 16 * ib + r], sO[t * LV + 16 * cb + r], acc);
        acc = mma(-sW[t * LD + 16 * ib + r], sX[t * LV + 16 * cb + r], acc);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int i = 16 * ib + 4 * kq + j, col = 16 * cb + r;
        sS[i * LV + col] = sG[i] * sS[i * LV + col] + acc[j];
      }
    }
  }
  __syncthreads();
  if (a.d_init) store_cols<D, DVT, LV>(a.d_init + uo, D, c0, sS);
}

// ---------------------------------------------------------------------------
// bwd_gstate: per (chunk, head).  Wave w owns rows [16w, 16w + 16) of every
// C x D result.
template <int D>
struct GsL {
  static constexpr int LD = D + 4, LM = C + 4;
  static constexpr int RS = 0;                 // r(C-1, t) (staging), S, Delta (rows), dS'
  static constexpr int RX = RS + (D > C ? D : C) * LD;  // dDelta, Kb, dO
  static constexpr int RR = RX + C * LD;       // b (staging), dR, Delta
  static constexpr int RT = RR + C * LD;       // T
  static constexpr int RB = RT + C * LM;       // beta [C]
  static constexpr int RE = RB + C;            // b_C [D]
  static constexpr int RY = RE + D;            // dgamma [D]
  static constexpr int RW = RY + D;            // per-wave column sums [4][D]
  static constexpr int RQ = RW + 4 * D;        // dbeta rows [C]
  static constexpr int FLOATS = RQ + C;
  static constexpr size_t BYTES = sizeof(float) * FLOATS;
};

template <int D, typename In>
__global__ void __launch_bounds__(NT) bwd_gstate(BwdArgs a) {
  using P = GsL<D>;
  constexpr int LD = P::LD, LM = P::LM, NCT = D / 16;
  extern __shared__ __align__(16) float sm[];
  float* sS = sm + P::RS;
  float* sX = sm + P::RX;
  float* sR = sm + P::RR;
  float* sT = sm + P::RT;
  float* sBeta = sm + P::RB;
  float* sEg = sm + P::RE;
  float* sGam = sm + P::RY;
  float* sCol = sm + P::RW;
  float* sDb = sm + P::RQ;

  const int slot = blockIdx.x / a.H, h = blockIdx.x - slot * a.H;
  Loc L;
  if (!locate(a, slot, L)) return;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, r = lane & 15, kq = lane >> 4;
  const size_t sh = static_cast<size_t>(slot) * a.H + h;
  const In* q = static_cast<const In*>(a.q);
  const In* k = static_cast<const In*>(a.k);
  const In* v = static_cast<const In*>(a.v);
  const int H = a.H;
  auto row = [&](int t) { return (L.tok0 + t) * H + h; };

  if (tid < C) {
    sBeta[tid] = tid < L.count ? a.beta[row(tid)] : 0.f;
    sDb[tid] = 0.f;
  }
  load_mat<C, C, LM>(sT, a.Tm + sh * C * C);
  load_mat<C, D, LD>(sX, a.dDl + sh * C * D);
  load_rows<D, LD>(sR, a.log_g, L.tok0, L.count, H, h);  // log_g rows (0 past the end)
  __syncthreads();
  // per channel: b_t into sR, r(C-1, t) into sS (staging), b_C into sEg
  for (int i = tid; i < D; i += NT) {
    float rr = 1.f;
    for (int t = C - 1; t >= 0; --t) {
      sS[t * LD + i] = rr;
      rr *= exp_fast(sR[t * LD + i]);
    }
    float b = 1.f;
    for (int t = 0; t < C; ++t) {
      b *= exp_fast(sR[t * LD + i]);
      sR[t * LD + i] = b;
    }
    sEg[i] = b;
  }
  __syncthreads();
  float bb[NCT][4], rc[NCT][4], kv[NCT][4];
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int t = 16 * w + 4 * kq + j, i = 16 * ct + r;
      bb[ct][j] = sR[t * LD + i];
      rc[ct][j] = sS[t * LD + i];
      kv[ct][j] = t < L.count ? to_f32(k[row(t) * D + i]) : 0.f;
    }
  __syncthreads();
  // dR = T^T dDelta -> sR;  dv = beta dR
  for (int ct = 0; ct < NCT; ++ct) {
    f32x4 acc = zero4f();
    for (int k0 = 16 * w; k0 < C; k0 += 4) {
      const int s = k0 + kq;
      acc = mma(sT[s * LM + 16 * w + r], sX[s * LD + 16 * ct + r], acc);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int t = 16 * w + 4 * kq + j, i = 16 * ct + r;
      sR[t * LD + i] = acc[j];
      if (t < L.count) a.dv[row(t) * D + i] = sBeta[t] * acc[j];
    }
  }
  __syncthreads();
  // S into sS; K*b into sX
  load_mat<D, D, LD>(sS, a.S_in + sh * D * D);
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
    for (int j = 0; j < 4; ++j) sX[(16 * w + 4 * kq + j) * LD + 16 * ct + r] = kv[ct][j] * bb[ct][j];
  __syncthreads();
  float dq_[NCT][4], dk_[NCT][4], dg_[NCT][4];
  float dbr[4] = {0.f, 0.f, 0.f, 0.f};
  // V - (K*b) S against dR: the R part of dbeta
  for (int ct = 0; ct < NCT; ++ct) {
    f32x4 acc = zero4f();
#pragma unroll 4
    for (int k0 = 0; k0 < D; k0 += 4) {
      const int kk = k0 + kq;
      acc = mma(sX[(16 * w + r) * LD + kk], sS[kk * LD + 16 * ct + r], acc);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int t = 16 * w + 4 * kq + j, jj = 16 * ct + r;
      const float vv = t < L.count ? to_f32(v[row(t) * D + jj]) : 0.f;
      dbr[j] += sR[t * LD + jj] * (vv - acc[j]);
    }
  }
  // d(K*b) = -beta dR S^T
  for (int ct = 0; ct < NCT; ++ct) {
    f32x4 acc = zero4f();
#pragma unroll 4
    for (int k0 = 0; k0 < D; k0 += 4) {
      const int jj = k0 + kq;
      acc = mma(sR[(16 * w + r) * LD + jj], sS[(16 * ct + r) * LD + jj], acc);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int t = 16 * w + 4 * kq + j;
      const float dkb = -sBeta[t] * acc[j];
      dk_[ct][j] = dkb * bb[ct][j];
      dg_[ct][j] = dkb * kv[ct][j] * bb[ct][j];
    }
  }
  __syncthreads();  // done with K*b
  load_rows<D, LD>(sX, a.d_out, L.tok0, L.count, H, h);
  __syncthreads();
  // d(Q*b) = scale dO S^T
  for (int ct = 0; ct < NCT; ++ct) {
    f32x4 acc = zero4f();
#pragma unroll 4
    for (int k0 = 0; k0 < D; k0 += 4) {
      const int jj = k0 + kq;
      acc = mma(sX[(16 * w + r) * LD + jj], sS[(16 * ct + r) * LD + jj], acc);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int t = 16 * w + 4 * kq + j, i = 16 * ct + r;
      const float dqb = a.scale * acc[j];
      const float qv = t < L.count ? to_f32(q[row(t) * D + i]) : 0.f;
      dq_[ct][j] = dqb * bb[ct][j];
      dg_[ct][j] += dqb * qv * bb[ct][j];
    }
  }
  // b_C sum_j dS'[i, j] S[i, j]: D / 4 consecutive threads per row, coalesced
  {
    constexpr int G = D / 4, N = D * G, IT = (N + NT - 1) / NT;
    static_assert(G <= 64 && NT % G == 0 && (N >= NT || N % 64 == 0), "row groups must stay inside a wave");
    float4 x[IT];
#pragma unroll
    for (int it = 0; it < IT; ++it)
      if (it * NT + tid < N) x[it] = load4(a.dSo + sh * D * D + static_cast<size_t>(it * NT + tid) * 4);
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      const int idx = it * NT + tid, i = idx / G, jj = 4 * (idx - i * G);
      if (idx >= N) continue;  // whole waves
      const float* sr = sS + i * LD + jj;
      float acc = x[it].x * sr[0] + x[it].y * sr[1] + x[it].z * sr[2] + x[it].w * sr[3];
#pragma unroll
      for (int o = 1; o < G; o <<= 1) acc += __shfl_xor(acc, o, 64);
      if ((tid & (G - 1)) == 0) sGam[i] = sEg[i] * acc;
    }
  }
  __syncthreads();  // done with S
  load_mat<C, D, LD>(sS, a.Dl + sh * C * D);  // Delta, rows
  __syncthreads();
  // dAqk = scale tril(dO Delta^T), dA = -tril(dR Delta^T, -1)
  for (int sb = 0; sb < 4; ++sb) {
    f32x4 aq = zero4f(), aa = zero4f();
    if (sb <= w) {
#pragma unroll 4
      for (int k0 = 0; k0 < D; k0 += 4) {
        const int jj = k0 + kq;
        const float dl = sS[(16 * sb + r) * LD + jj];
        aq = mma(sX[(16 * w + r) * LD + jj], dl, aq);
        aa = mma(sR[(16 * w + r) * LD + jj], dl, aa);
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int t = 16 * w + 4 * kq + j, s = 16 * sb + r;
      const float gq = s <= t ? a.scale * aq[j] : 0.f;
      const float ga = s < t ? -aa[j] : 0.f;
      dbr[j] += ga * a.Ab[sh * C * C + t * C + s];
      a.dAq[sh * C * C + t * C + s] = gq;
      a.dAb[sh * C * C + t * C + s] = sBeta[t] * ga;
    }
  }
  // rows of dbeta: reduce over the 16 lanes sharing kq
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    float x = dbr[j];
    x += __shfl_xor(x, 1, 64);
    x += __shfl_xor(x, 2, 64);
    x += __shfl_xor(x, 4, 64);
    x += __shfl_xor(x, 8, 64);
    if (r == 0) sDb[16 * w + 4 * kq + j] = x;
  }
  __syncthreads();  // done with Delta rows (sS) and dR (sR)
  load_mat<C, D, LD>(sR, a.Dl + sh * C * D);   // Delta
  load_mat<D, D, LD>(sS, a.dSo + sh * D * D);  // dS'
  __syncthreads();
  // dKd = Delta dS'^T
  float colp[NCT];
  for (int ct = 0; ct < NCT; ++ct) {
    f32x4 acc = zero4f();
#pragma unroll 4
    for (int k0 = 0; k0 < D; k0 += 4) {
      const int jj = k0 + kq;
      acc = mma(sR[(16 * w + r) * LD + jj], sS[(16 * ct + r) * LD + jj], acc);
    }
    float cs = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float kd = kv[ct][j] * rc[ct][j];
      dk_[ct][j] += acc[j] * rc[ct][j];
      dg_[ct][j] -= acc[j] * kd;
      cs += acc[j] * kd;
    }
    cs += __shfl_xor(cs, 16, 64);
    cs += __shfl_xor(cs, 32, 64);
    colp[ct] = cs;
  }
  if (kq == 0)
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) sCol[w * D + 16 * ct + r] = colp[ct];
  __syncthreads();
  // dgamma joins dG at the chunk's last token; write the staged parts
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int t = 16 * w + 4 * kq + j, i = 16 * ct + r;
      if (t >= L.count) continue;
      float g = dg_[ct][j];
      if (t == L.count - 1) g += sGam[i] + sCol[i] + sCol[D + i] + sCol[2 * D + i] + sCol[3 * D + i];
      a.dq[row(t) * D + i] = dq_[ct][j];
      a.dk[row(t) * D + i] = dk_[ct][j];
      a.dlog_g[row(t) * D + i] = g;
    }
  if (tid < L.count) a.dbeta[row(tid)] = sDb[tid];
}

// ---------------------------------------------------------------------------
// bwd_gpairs: per (chunk, head): pair terms of Aqk and Akk, then dlog_g.
template <int D>
struct GpL {
  static constexpr int LD = D + 4, LM = C + 4;
  static constexpr int RQ = 0;
  static constexpr int RK = RQ + C * LD;
  static constexpr int RF = RK + C * LD;  // F, later dG
  static constexpr int RA = RF + C * LD;  // dAqk
  static constexpr int RB = RA + C * LM;  // dAkk
  static constexpr int FLOATS = RB + C * LM;
  static constexpr size_t BYTES = sizeof(float) * FLOATS;
};

constexpr int NTG = 512;  // bwd_gpairs: 8 waves, two per token block

template <int D, typename In>
__global__ void __launch_bounds__(NTG) bwd_gpairs(BwdArgs a) {
  using P = GpL<D>;
  constexpr int LD = P::LD, LM = P::LM, NCT = D / 16;
  // wave wv: token block w = wv & 3, channel tiles [ch * NCTW, ch * NCTW + NCTW)
  constexpr int NCTW = NCT >= 2 ? NCT / 2 : 1;
  extern __shared__ __align__(16) float sm[];
  float* sQ = sm + P::RQ;
  float* sK = sm + P::RK;
  float* sF = sm + P::RF;
  float* sdAq = sm + P::RA;
  float* sdAb = sm + P::RB;

  const int slot = blockIdx.x / a.H, h = blockIdx.x - slot * a.H;
  Loc L;
  if (!locate(a, slot, L)) return;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, w = wv & 3, r = lane & 15, kq = lane >> 4;
  const int ctb = (wv >> 2) * NCTW;
  const bool active = ctb < NCT;
  const size_t sh = static_cast<size_t>(slot) * a.H + h;
  const int H = a.H;
  auto row = [&](int t) { return (L.tok0 + t) * H + h; };

  load_rows<D, LD, In, NTG>(sQ, static_cast<const In*>(a.q), L.tok0, L.count, H, h);
  load_rows<D, LD, In, NTG>(sK, static_cast<const In*>(a.k), L.tok0, L.count, H, h);
  load_mat<C, C, LM, NTG>(sdAq, a.dAq + sh * C * C);
  load_mat<C, C, LM, NTG>(sdAb, a.dAb + sh * C * C);
  const int ci = tid % D, ph = tid / D;
  const bool chan = ph < 2;
  float al[32];
  if (chan) load_alpha<D>(al, a.log_g, L.tok0, L.count, H, h, ci, 32 * ph);

  float dq_[NCTW][4], dk_[NCTW][4], dg_[NCTW][4];
#pragma unroll
  for (int ct = 0; ct < NCTW; ++ct)
#pragma unroll
    for (int j = 0; j < 4; ++j) dq_[ct][j] = dk_[ct][j] = dg_[ct][j] = 0.f;

  // rows of block w against the partner range [p0, p0 + plen) at level l:
  // dX (w in the upper half) or dY (w in the lower half)
  auto level_terms = [&](int l, bool upper_rows, int p0, int plen) {
#pragma unroll
    for (int ct = 0; ct < NCTW; ++ct) {
      const int i0 = 16 * (ctb + ct);
      if (upper_rows) {
        f32x4 xq = zero4f(), xk = zero4f();
        for (int k0 = 0; k0 < plen; k0 += 4) {
          const int s = p0 + k0 + kq, t = 16 * w + r;
          const bool ok = at_level(l, t, s);
          const float ys = sK[s * LD + i0 + r] * sF[s * LD + i0 + r];
          xq = mma(ok ? sdAq[t * LM + s] : 0.f, ys, xq);
          xk = mma(ok ? sdAb[t * LM + s] : 0.f, ys, xk);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int t = 16 * w + 4 * kq + j, i = i0 + r;
          const float ft = sF[t * LD + i];
          const float gq = ft * xq[j], gk = ft * xk[j];
          dq_[ct][j] += gq;
          dk_[ct][j] += gk;
          dg_[ct][j] += sQ[t * LD + i] * gq + sK[t * LD + i] * gk;
        }
      } else {
        f32x4 y = zero4f();
        for (int k0 = 0; k0 < plen; k0 += 4) {
          const int t = p0 + k0 + kq, s = 16 * w + r;
          const bool ok = at_level(l, t, s);
          const float ft = sF[t * LD + i0 + r];
          y = mma(ok ? sdAq[t * LM + s] : 0.f, sQ[t * LD + i0 + r] * ft, y);
          y = mma(ok ? sdAb[t * LM + s] : 0.f, sK[t * LD + i0 + r] * ft, y);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int s = 16 * w + 4 * kq + j, i = i0 + r;
          const float gy = sF[s * LD + i] * y[j];
          dk_[ct][j] += gy;
          dg_[ct][j] -= sK[s * LD + i] * gy;
        }
      }
    }
  };
#pragma unroll
  for (int l = 0; l < 6; ++l) {
    __syncthreads();
    if (chan) {
      switch (l) {
        case 0: level_factors<0, LD>(al, 32 * ph, ci, sF); break;
        case 1: level_factors<1, LD>(al, 32 * ph, ci, sF); break;
        case 2: level_factors<2, LD>(al, 32 * ph, ci, sF); break;
        case 3: level_factors<3, LD>(al, 32 * ph, ci, sF); break;
        case 4: level_factors<4, LD>(al, 32 * ph, ci, sF); break;
        default: level_factors<5, LD>(al, 32 * ph, ci, sF); break;
      }
    }
    __syncthreads();
    if (!active) continue;
    if (l == 0) {
      if (w >= 2) level_terms(0, true, 0, 32);
      else level_terms(0, false, 32, 32);
    } else if (l == 1) {
      if (w & 1) level_terms(1, true, 16 * (w - 1), 16);
      else level_terms(1, false, 16 * (w + 1), 16);
    } else {
      level_terms(l, true, 16 * w, 16);
      level_terms(l, false, 16 * w, 16);
    }
  }
  // pairs t = s (r = 1): Aqk only
#pragma unroll
  for (int ct = 0; ct < NCTW; ++ct)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int t = 16 * w + 4 * kq + j, i = 16 * (ctb + ct) + r;
      const float d = sdAq[t * LM + t];
      dq_[ct][j] += d * sK[t * LD + i];
      dk_[ct][j] += d * sQ[t * LD + i];
    }
  __syncthreads();  // done with F
  // add the state-side parts staged by bwd_gstate; dG into sF for the cumsum
#pragma unroll
  for (int ct = 0; ct < NCTW; ++ct)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int t = 16 * w + 4 * kq + j, i = 16 * (ctb + ct) + r;
      if (!active) continue;
      float g = 0.f;
      if (t < L.count) {
        const int64_t o = row(t) * D + i;
        a.dq[o] += dq_[ct][j];
        a.dk[o] += dk_[ct][j];
        g = a.dlog_g[o] + dg_[ct][j];
      }
      sF[t * LD + i] = g;
    }
  __syncthreads();
  for (int i = tid; i < D; i += NTG) {
    float acc = 0.f;
    for (int t = C - 1; t >= 0; --t) {
      acc += sF[t * LD + i];
      if (t < L.count) a.dlog_g[row(t) * D + i] = acc;
    }
  }
}

// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(1024) bwd_chunk_map(const int32_t* __restrict__ cu, int n, int n_slots,
                                                      int32_t* __restrict__ cstart, int32_t* __restrict__ table) {
  __shared__ int wsum[16];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  int carry = 0;
  for (int base = 0; base < n; base += 1024) {
    const int d = base + tid;
    const int len = d < n ? max(cu[d + 1] - cu[d], 0) : 0;
    const int nc = (len + C - 1) / C;
    int x = nc;
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
  __syncthreads();
  for (int d = tid; d < n; d += 1024) {
    const int b = cstart[d], e = min(cstart[d + 1], n_slots);
    for (int c = b; c < e; ++c) table[c] = d;
  }
  for (int c = max(carry, 0) + tid; c < n_slots; c += 1024) table[c] = -1;
}

size_t al256(size_t x) { return (x + 255) / 256 * 256; }

int64_t bwd_slots(int num_seqs, int seq_len, bool packed) {
  const int64_t nchd = (static_cast<int64_t>(seq_len) + C - 1) / C;
  return packed ? nchd + num_seqs : nchd * num_seqs;
}

struct BwdWs {
  int32_t* cstart;
  int32_t* table;
  float* f[14];
  size_t bytes;
};

// Workspace: packed map, then the per-(slot, head) arrays in BwdArgs order.
BwdWs bwd_ws(void* base, int num_seqs, int seq_len, int H, int D, bool packed) {
  BwdWs l{};
  unsigned char* b = static_cast<unsigned char*>(base);
  size_t off = 0;
  const int64_t ns = bwd_slots(num_seqs, seq_len, packed);
  if (packed) {
    l.cstart = reinterpret_cast<int32_t*>(b + off);
    off += al256(static_cast<size_t>(num_seqs + 1) * 4);
    l.table = reinterpret_cast<int32_t*>(b + off);
    off += al256(static_cast<size_t>(ns) * 4);
  }
  const size_t sh = static_cast<size_t>(ns) * H;
  const size_t per[14] = {size_t(D) * D, size_t(D) * D, size_t(C) * D, size_t(C) * D, size_t(C) * D,
                          size_t(C) * D, size_t(C) * D, size_t(C) * D, size_t(C) * C, size_t(C) * C,
                          size_t(C) * C, size_t(C) * C, size_t(C) * C, size_t(D)};
  for (int i = 0; i < 14; ++i) {
    l.f[i] = reinterpret_cast<float*>(b + off);
    off += al256(sh * per[i] * 4);
  }
  l.bytes = off;
  return l;
}

template <int D, typename In>
hipError_t set_lds_d() {
  hipError_t e;
  e = hipFuncSetAttribute(reinterpret_cast<const void*>(bwd_prep<D, In>), hipFuncAttributeMaxDynamicSharedMemorySize,
                          static_cast<int>(PrepL<D>::BYTES));
  if (e != hipSuccess) return e;
  e = hipFuncSetAttribute(reinterpret_cast<const void*>(bwd_gstate<D, In>),
                          hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(GsL<D>::BYTES));
  if (e != hipSuccess) return e;
  e = hipFuncSetAttribute(reinterpret_cast<const void*>(bwd_gpairs<D, In>),
                          hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(GpL<D>::BYTES));
  if (e != hipSuccess) return e;
  e = hipFuncSetAttribute(reinterpret_cast<const void*>(bwd_fscan<D>), hipFuncAttributeMaxDynamicSharedMemorySize,
                          static_cast<int>(sizeof(float) * ScanL<D>::F_FLOATS));
  if (e != hipSuccess) return e;
  return hipFuncSetAttribute(reinterpret_cast<const void*>(bwd_rscan<D>),
                             hipFuncAttributeMaxDynamicSharedMemorySize,
                             static_cast<int>(sizeof(float) * ScanL<D>::R_FLOATS));
}

// LDS limits are raised once per device for every instantiation.
hipError_t bwd_prepare_device() {
  constexpr int MAX_DEV = 64;
  static bool ready[MAX_DEV] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= MAX_DEV) return hipErrorInvalidDevice;
  if (ready[dev]) return hipSuccess;
  if ((e = set_lds_d<16, float>()) != hipSuccess) return e;
  if ((e = set_lds_d<32, float>()) != hipSuccess) return e;
  if ((e = set_lds_d<64, float>()) != hipSuccess) return e;
  if ((e = set_lds_d<128, float>()) != hipSuccess) return e;
  if ((e = set_lds_d<16, bf16_t>()) != hipSuccess) return e;
  if ((e = set_lds_d<32, bf16_t>()) != hipSuccess) return e;
  if ((e = set_lds_d<64, bf16_t>()) != hipSuccess) return e;
  if ((e = set_lds_d<128, bf16_t>()) != hipSuccess) return e;
  ready[dev] = true;
  return hipSuccess;
}

template <int D, typename In>
hipError_t run_bwd(const BwdArgs& a, int64_t ns, hipStream_t stream) {
  const unsigned chunk_blocks = static_cast<unsigned>(ns * a.H);
  const unsigned unit_blocks = static_cast<unsigned>(a.N) * a.H * ScanL<D>::NTILE;
  hipError_t e;
  if (chunk_blocks > 0) {
    hipLaunchKernelGGL((bwd_prep<D, In>), dim3(chunk_blocks), dim3(NT), PrepL<D>::BYTES, stream, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if (unit_blocks > 0) {
    hipLaunchKernelGGL((bwd_fscan<D>), dim3(unit_blocks), dim3(NT), sizeof(float) * ScanL<D>::F_FLOATS, stream, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL((bwd_rscan<D>), dim3(unit_blocks), dim3(NT), sizeof(float) * ScanL<D>::R_FLOATS, stream, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if (chunk_blocks > 0) {
    hipLaunchKernelGGL((bwd_gstate<D, In>), dim3(chunk_blocks), dim3(NT), GsL<D>::BYTES, stream, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL((bwd_gpairs<D, In>), dim3(chunk_blocks), dim3(NTG), GpL<D>::BYTES, stream, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace

size_t bwd_workspace_bytes(int num_seqs, int seq_len, int num_heads, int d, bool packed) {
  return bwd_ws(nullptr, num_seqs, seq_len, num_heads, d, packed).bytes;
}

bool bwd_supported(const BwdLaunch& a) {
  const bool packed = a.cu_seqlens != nullptr;
  const int64_t blocks = bwd_slots(a.num_seqs, a.seq_len, packed) * a.num_heads;
  return (a.d == 16 || a.d == 32 || a.d == 64 || a.d == 128) && blocks < (int64_t(1) << 31) &&
         int64_t(a.num_seqs) * a.num_heads * 4 < (int64_t(1) << 31);
}

hipError_t launch_chunk_bwd(const BwdLaunch& s, hipStream_t stream) {
  hipError_t e = bwd_prepare_device();
  if (e != hipSuccess) return e;
  const bool packed = s.cu_seqlens != nullptr;
  const BwdWs l = bwd_ws(s.workspace, s.num_seqs, s.seq_len, s.num_heads, s.d, packed);
  const int64_t ns = bwd_slots(s.num_seqs, s.seq_len, packed);
  BwdArgs a{};
  a.q = s.q; a.k = s.k; a.v = s.v; a.log_g = s.log_g; a.beta = s.beta; a.init_state = s.init_state;
  a.cu = s.cu_seqlens;
  a.cstart = packed ? l.cstart : nullptr;
  a.table = packed ? l.table : nullptr;
  a.d_out = s.d_out; a.d_final = s.d_final;
  a.dq = s.dq; a.dk = s.dk; a.dv = s.dv; a.dlog_g = s.dlog_g; a.dbeta = s.dbeta; a.d_init = s.d_init;
  a.S_in = l.f[0]; a.dSo = l.f[1]; a.Wm = l.f[2]; a.Um = l.f[3]; a.Kd = l.f[4]; a.Qs = l.f[5];
  a.Dl = l.f[6]; a.dDl = l.f[7]; a.As = l.f[8]; a.Tm = l.f[9]; a.Ab = l.f[10]; a.dAq = l.f[11];
  a.dAb = l.f[12]; a.eg = l.f[13];
  a.N = s.num_seqs; a.T = s.seq_len; a.H = s.num_heads;
  a.cps = packed ? 0 : static_cast<int>((static_cast<int64_t>(s.seq_len) + C - 1) / C);
  a.scale = s.scale;
  if (packed) {
    hipLaunchKernelGGL(bwd_chunk_map, dim3(1), dim3(1024), 0, stream, s.cu_seqlens, s.num_seqs,
                       static_cast<int>(ns), l.cstart, l.table);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  switch (s.d) {
    case 16: return s.bf16 ? run_bwd<16, bf16_t>(a, ns, stream) : run_bwd<16, float>(a, ns, stream);
    case 32: return s.bf16 ? run_bwd<32, bf16_t>(a, ns, stream) : run_bwd<32, float>(a, ns, stream);
    case 64: return s.bf16 ? run_bwd<64, bf16_t>(a, ns, stream) : run_bwd<64, float>(a, ns, stream);
    case 128: return s.bf16 ? run_bwd<128, bf16_t>(a, ns, stream) : run_bwd<128, float>(a, ns, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace kda
