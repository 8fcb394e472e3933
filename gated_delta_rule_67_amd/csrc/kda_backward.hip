// kda_backward.hip -- reverse mode of the chunked KDA prefill (gfx950).
//
// The loss L = sum(d_out * out) + sum(d_final * final_state) is differentiated
// through the gated delta rule (NeMo glm5_next.layers: `_torch_recurrent_kda`
// is the differentiable reference; the KDA parameters are trained under FSDP).
// Arithmetic: fp32 operands, MFMA (v_mfma_f32_16x16x4_f32) and state; for bf16
// inputs the two scans and bwd_gstate form their products from split-bf16
// operands (three bf16 MFMAs per product, about 16 bits of precision per term)
// with the state and every stored intermediate kept in fp32.
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
// bwd_gpairs sums levels 3-5 (pairs inside an aligned 8-token group) per
// channel with r(t, s) as a running product of gates instead.
//
// Kernels, in launch order (slots are chunks, one workgroup per (slot, head)
// or per (unit, value-column tile)):
//   bwd_prep      per chunk: Akk, Aqk, T, W, U, Kd, scale*(Q*b), b_C
//   bwd_fscan     per unit, serially over its chunks: entry states S, Delta
//                 (bwd_fscan3 with split-bf16 products)
//   bwd_rscan     per unit, backwards: exit-state gradients dS', dDelta, dS0
//                 (bwd_rscan3 with split-bf16 products)
//   bwd_gstate    per chunk: dv, dbeta, dAqk, dA and the state-side parts of
//                 dq, dk and dG (staged in the dq, dk, dlog_g outputs)
//   bwd_gpairs    per (chunk, 64 channels): the pair terms, then
//                 dlog_g = reverse cumsum(dG)
#include <algorithm>
#include <type_traits>

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
  float* QsT;   // D x C   (scale * q_t * b_t)^T
  float* Dl;    // C x D   Delta
  float* dDl;   // D x C   dDelta^T
  float* AsT;   // C x C   (scale * Aqk)^T
  float* Tm;    // C x C   T^T
  float* Ab;    // C x C   Akk (strictly lower, beta not applied)
  float* dAq;   // C x C   dL/dAqk
  float* dAb;   // C x C   dL/dAkk
  float* eg;    // D       b_C
  float* WT;    // D x C   W^T
  float* KdT;   // D x C   Kd^T
  int N;
  int T;
  int H;
  int cps;      // dense: chunks per sequence
  int n_slots;  // chunk slots per head
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
// a thread's loads are in flight before its LDS stores.  Their loads are
// unconditional, from an index clamped into range, and out-of-range values
// are replaced afterwards: a load under a branch waits for its data before
// the next one issues.  count >= 1.)
template <int D, int LD, typename In, int NTH = NT>
__device__ __forceinline__ void load_rows(float* dst, const In* src, int64_t tok0, int count, int H, int h) {
  constexpr int G = D / 4, N = C * G, IT = (N + NTH - 1) / NTH;
  float4 x[IT];
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int idx = it * NTH + threadIdx.x, t = idx / G, g4 = idx - t * G;
    const float4 y = load4(src + ((tok0 + min(t, count - 1)) * H + h) * D + 4 * g4);
    x[it] = t < count ? y : make_float4(0.f, 0.f, 0.f, 0.f);
  }
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int idx = it * NTH + threadIdx.x, t = idx / G, g4 = idx - t * G;
    if (idx < N) *reinterpret_cast<float4*>(dst + t * LD + 4 * g4) = x[it];
  }
}

// C rows of a [tokens, H, D] tensor transposed into LDS: dst[i * LDT + t],
// rows >= count zero.
template <int D, int LDT, typename In, int NTH = NT>
__device__ __forceinline__ void load_rows_t(float* dst, const In* src, int64_t tok0, int count, int H, int h) {
  constexpr int G = D / 4, N = C * G, IT = (N + NTH - 1) / NTH;
  float4 x[IT];
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int idx = it * NTH + threadIdx.x, t = idx / G, g4 = idx - t * G;
    const float4 y = load4(src + ((tok0 + min(t, count - 1)) * H + h) * D + 4 * g4);
    x[it] = t < count ? y : make_float4(0.f, 0.f, 0.f, 0.f);
  }
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int idx = it * NTH + threadIdx.x, t = idx / G, c = 4 * (idx - t * G);
    if (idx < N) {
      dst[(c + 0) * LDT + t] = x[it].x;
      dst[(c + 1) * LDT + t] = x[it].y;
      dst[(c + 2) * LDT + t] = x[it].z;
      dst[(c + 3) * LDT + t] = x[it].w;
    }
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
    x[it] = load4(src + min(idx, N - 1) * 4);
  }
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int idx = it * NTH + threadIdx.x, t = idx / G, g4 = idx - t * G;
    if (idx < N) *reinterpret_cast<float4*>(dst + t * LD + 4 * g4) = x[it];
  }
}

// Gates of one channel over 32 tokens [base, base + 32) of the chunk (1 past
// the document end).
template <int D>
__device__ __forceinline__ void load_alpha(float (&al)[32], const float* log_g, int64_t tok0, int count, int H, int h,
                                           int i, int base) {
  float lg[32];
#pragma unroll
  for (int u = 0; u < 32; ++u) lg[u] = log_g[((tok0 + min(base + u, count - 1)) * H + h) * D + i];
  __builtin_amdgcn_sched_barrier(0);  // all 32 loads in flight before the first use
#pragma unroll
  for (int u = 0; u < 32; ++u) al[u] = base + u < count ? exp_fast(lg[u]) : 1.f;
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
__device__ __forceinline__ float ld1f(const float* p) { return *p; }
__device__ __forceinline__ float ld1f(const bf16_t* p) { return to_f32(*p); }

// Split-bf16 operands (bf16 inputs).  An fp32 value x is held as hi + lo, two
// bf16 values (round to nearest even twice: |x - hi - lo| <= 2^-16 |x|), and a
// product as three bf16 MFMAs, hi*hi + hi*lo + lo*hi.
// bf16 inputs (2e-2 bar) run the scans on split-bf16 products; fp32 inputs
// keep fp32 products.  The split kernels contract in 32-wide blocks.
template <int D, typename In>
constexpr bool split_scans() {
  return sizeof(In) == 2 && D % 32 == 0;
}

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ f32x4 mfma_bf(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));

// Two fp32 values rounded to nearest even as packed bf16 (one
// v_cvt_pk_bf16_f32), and back.
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  bf16x2v r;
  r[0] = static_cast<__bf16>(a);
  r[1] = static_cast<__bf16>(b);
  return __builtin_bit_cast(uint32_t, r);
}
__device__ __forceinline__ float bf16_lo_f(uint32_t p) { return __uint_as_float(p << 16); }
__device__ __forceinline__ float bf16_hi_f(uint32_t p) { return __uint_as_float(p & 0xffff0000u); }

// hi and lo halves of a pair of values, packed: hi = bf16(x), lo = bf16(x - hi)
__device__ __forceinline__ void split_pair(float x0, float x1, uint32_t& hi, uint32_t& lo) {
  hi = pack_bf16(x0, x1);
  lo = pack_bf16(x0 - bf16_lo_f(hi), x1 - bf16_hi_f(hi));
}
__device__ __forceinline__ void put_split(uint16_t* hi, uint16_t* lo, float x) {
  uint32_t h, l;
  split_pair(x, 0.f, h, l);
  *hi = static_cast<uint16_t>(h);
  *lo = static_cast<uint16_t>(l);
}
// four consecutive values
__device__ __forceinline__ void put_split4(uint16_t* hi, uint16_t* lo, float4 x) {
  uint32_t h01, l01, h23, l23;
  split_pair(x.x, x.y, h01, l01);
  split_pair(x.z, x.w, h23, l23);
  *reinterpret_cast<uint2*>(hi) = make_uint2(h01, h23);
  *reinterpret_cast<uint2*>(lo) = make_uint2(l01, l23);
}

// ---------------------------------------------------------------------------
// bwd_prep: per (chunk, head).
template <typename In>
constexpr int prep_threads() {
  return sizeof(In) == 2 ? 256 : 512;
}

template <int D, typename In>
struct PrepL {
  // bf16 inputs: K, Q and V^T stay bf16 in LDS and the regions overlap more
  // ((K*b)^T over K and Q, V^T over Akk, T over Aqk): about 75 KB for d = 128,
  // two 4-wave workgroups per CU, so one's load and store phases overlap the
  // other's products.  fp32 inputs: fp32 rows, one 8-wave workgroup per CU.
  static constexpr bool COMPACT = sizeof(In) == 2;
  static constexpr int NTH = prep_threads<In>();
  static constexpr int LD = D + 4, LM = C + 4;
  static constexpr int LDK = COMPACT ? D + 8 : D + 4;  // K, Q row stride (elements)
  static constexpr int LMV = C + 4;                     // V^T row stride (elements)
  static constexpr int CD = C * LD, CM = C * LM;
  static constexpr int KQF = COMPACT ? C * LDK / 2 : (CD > D * LM ? CD : D * LM);  // floats per K or Q region
  static constexpr int R0 = 0;                          // K rows (fp32 layout: later V^T)
  static constexpr int R1 = R0 + KQF;                   // Q rows (fp32 layout: later (K*b)^T)
  static constexpr int R2 = R1 + KQF;                   // F, later Akk | Aqk
  static constexpr int R3 = R2 + (CD > 2 * CM ? CD : 2 * CM);  // T (fp32 layout)
  static constexpr int R4 = R3 + (COMPACT ? 0 : CM);    // 4 x 16 x 17 wave scratch
  static constexpr int RB = R4 + 4 * 16 * 17;           // beta [C]
  static constexpr int RT = RB + C;                     // block totals [2][D]
  static constexpr int FLOATS = RT + 2 * D;
  static constexpr size_t BYTES = sizeof(float) * FLOATS;
  static_assert(!COMPACT || 2 * KQF >= D * LM, "(K*b)^T fits over K and Q");
  static_assert(!COMPACT || D * LMV / 2 <= CM, "V^T fits over Akk");
};

// C rows of a [tokens, H, D] bf16 tensor copied into LDS as bf16 (row stride
// LDK), rows >= count zero.
template <int D, int LDK, int NTH>
__device__ __forceinline__ void load_rows_raw(bf16_t* dst, const bf16_t* src, int64_t tok0, int count, int H, int h) {
  constexpr int G = D / 4, N = C * G, IT = (N + NTH - 1) / NTH;
  uint2 x[IT];
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int idx = it * NTH + threadIdx.x, t = idx / G, g4 = idx - t * G;
    const uint2 y = *reinterpret_cast<const uint2*>(src + ((tok0 + min(t, count - 1)) * H + h) * D + 4 * g4);
    x[it] = t < count ? y : make_uint2(0u, 0u);
  }
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int idx = it * NTH + threadIdx.x, t = idx / G, g4 = idx - t * G;
    if (idx < N) *reinterpret_cast<uint2*>(dst + t * LDK + 4 * g4) = x[it];
  }
}

template <int D, typename In>
__global__ void __launch_bounds__(prep_threads<In>()) bwd_prep(BwdArgs a) {
  using P = PrepL<D, In>;
  constexpr int LD = P::LD, LM = P::LM, LDK = P::LDK, NTH = P::NTH;
  using KQ = std::conditional_t<P::COMPACT, In, float>;  // element type of K, Q, V^T in LDS
  extern __shared__ __align__(16) float sm[];
  KQ* sK = reinterpret_cast<KQ*>(sm + P::R0);
  KQ* sQ = reinterpret_cast<KQ*>(sm + P::R1);
  float* sF = sm + P::R2;
  float* sAb = sm + P::R2;
  float* sAq = sm + P::R2 + P::CM;
  float* sT = P::COMPACT ? sAq : sm + P::R3;
  float* sBeta = sm + P::RB;
  float* sTot = sm + P::RT;

  const int slot = blockIdx.x / a.H, h = blockIdx.x - slot * a.H;
  Loc L;
  if (!locate(a, slot, L)) return;
  // wave wv: 16-token block w, and half hf of the channels (pair tiles) or of
  // the column tiles (W, U)
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, w = wv & 3, hf = wv >> 2, r = lane & 15, kq = lane >> 4;
  constexpr int KH = (NTH == 512 && D >= 32) ? D / 2 : D;  // channels per half
  const bool khalf = hf * KH < D;
  const size_t sh = static_cast<size_t>(slot) * a.H + h;
  const In* q = static_cast<const In*>(a.q);
  const In* k = static_cast<const In*>(a.k);
  const In* v = static_cast<const In*>(a.v);

  if constexpr (P::COMPACT) {
    load_rows_raw<D, LDK, NTH>(sK, k, L.tok0, L.count, a.H, h);
    load_rows_raw<D, LDK, NTH>(sQ, q, L.tok0, L.count, a.H, h);
  } else {
    load_rows<D, LD, In, NTH>(sK, k, L.tok0, L.count, a.H, h);
    load_rows<D, LD, In, NTH>(sQ, q, L.tok0, L.count, a.H, h);
  }
  if (tid < C) {
    const float bv = a.beta[(L.tok0 + min(tid, L.count - 1)) * a.H + h];
    sBeta[tid] = tid < L.count ? bv : 0.f;
  }
  // gates of channel ci over half ph of the chunk
  const int ci = tid % D, ph = tid / D;
  const bool chan = ph < 2;
  float al[32];
  if (chan) load_alpha<D>(al, a.log_g, L.tok0, L.count, a.H, h, ci, 32 * ph);

  f32x4 ab_d = zero4f(), aq_d = zero4f(), ab_0 = zero4f(), aq_0 = zero4f(), ab_1 = zero4f(), aq_1 = zero4f();
  // product of one 16 x 16 tile (I, J) with factors; channels read as float4
  // (k = k0 + 4 kq + m for the m-th MFMA, the same order on both sides)
  auto pair_tile = [&](int I, int J, f32x4& accK, f32x4& accQ) {
    const int tt = (16 * I + r) * LD + 4 * kq, ts = (16 * J + r) * LD + 4 * kq;
    const int ttk = (16 * I + r) * LDK + 4 * kq, tsk = (16 * J + r) * LDK + 4 * kq;
    for (int k0 = hf * KH; k0 < hf * KH + KH; k0 += 16) {
      const float4 ft = *reinterpret_cast<const float4*>(sF + tt + k0);
      const float4 kt = load4(sK + ttk + k0);
      const float4 qt = load4(sQ + ttk + k0);
      const float4 fs = *reinterpret_cast<const float4*>(sF + ts + k0);
      const float4 ks = load4(sK + tsk + k0);
      accK = mma(kt.x * ft.x, ks.x * fs.x, accK);
      accQ = mma(qt.x * ft.x, ks.x * fs.x, accQ);
      accK = mma(kt.y * ft.y, ks.y * fs.y, accK);
      accQ = mma(qt.y * ft.y, ks.y * fs.y, accQ);
      accK = mma(kt.z * ft.z, ks.z * fs.z, accK);
      accQ = mma(qt.z * ft.z, ks.z * fs.z, accQ);
      accK = mma(kt.w * ft.w, ks.w * fs.w, accK);
      accQ = mma(qt.w * ft.w, ks.w * fs.w, accQ);
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
    if (!khalf) continue;
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
  if (khalf) {
    f32x4 tq = zero4f();
    const int tt = (16 * w + r) * LDK + 4 * kq;
    for (int k0 = hf * KH; k0 < hf * KH + KH; k0 += 16) {
      const float4 qt = load4(sQ + tt + k0);
      const float4 kt = load4(sK + tt + k0);
      tq = mma(qt.x, kt.x, tq);
      tq = mma(qt.y, kt.y, tq);
      tq = mma(qt.z, kt.z, tq);
      tq = mma(qt.w, kt.w, tq);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) aq_d[j] += (4 * kq + j == r) ? tq[j] : 0.f;
  }
  __syncthreads();  // everyone done with sF
  for (int idx = tid; idx < 2 * P::CM; idx += NTH) sAb[idx] = 0.f;
  __syncthreads();
  // the two channel halves of every tile: the first half's waves store, the
  // second half's add
  auto put = [&](float* M, int I, int J, const f32x4& x) {
#pragma unroll
    for (int j = 0; j < 4; ++j) M[(16 * I + 4 * kq + j) * LM + 16 * J + r] += x[j];
  };
  for (int pass = 0; pass < 2; ++pass) {
    if (pass == 1) __syncthreads();
    if (hf != pass || !khalf) continue;
    put(sAb, w, w, ab_d);
    put(sAq, w, w, aq_d);
    put(sAb, 2 + (w >> 1), w & 1, ab_0);
    put(sAq, 2 + (w >> 1), w & 1, aq_0);
    if (w < 2) {
      put(sAb, w == 0 ? 1 : 3, w == 0 ? 0 : 2, ab_1);
      put(sAq, w == 0 ? 1 : 3, w == 0 ? 0 : 2, aq_1);
    }
  }
  // block totals of the two halves for the cumulative decays
  if (chan) {
    float p = 1.f;
#pragma unroll
    for (int u = 0; u < 32; ++u) p *= al[u];
    sTot[ph * D + ci] = p;
  }
  __syncthreads();
  // Akk and (scale * Aqk)^T to the workspace
  for (int idx = tid; idx < C * C; idx += NTH) {
    const int t = idx / C, s = idx - t * C;
    // whole lines per instruction, read only by later kernels: nontemporal
    __builtin_nontemporal_store(sAb[t * LM + s], a.Ab + sh * C * C + idx);
    __builtin_nontemporal_store(a.scale * sAq[s * LM + t], a.AsT + sh * C * C + idx);
  }
  // per channel: b_t (prefix), Qs = scale q b, K*b (kept), Kd = k r(C-1, t), b_C
  // (the transposed rows QsT and KdT of channel ci are 32 consecutive floats
  // of this thread: written as float4)
  float kb[32];
  if (chan) {
    float b = ph == 1 ? sTot[ci] : 1.f;
    float* qst = a.QsT + (sh * D + ci) * C + 32 * ph;
    float x4[4];
#pragma unroll
    for (int u = 0; u < 32; ++u) {
      const int t = 32 * ph + u;
      b *= al[u];
      const float qv = ld1f(sQ + t * LDK + ci);
      x4[u & 3] = a.scale * qv * b;
      if ((u & 3) == 3) *reinterpret_cast<float4*>(qst + u - 3) = make_float4(x4[0], x4[1], x4[2], x4[3]);
      kb[u] = ld1f(sK + t * LDK + ci) * b;
    }
    if (ph == 1) a.eg[sh * D + ci] = b;
    float rr = ph == 0 ? sTot[D + ci] : 1.f;
    float* kdt = a.KdT + (sh * D + ci) * C + 32 * ph;
#pragma unroll
    for (int u = 31; u >= 0; --u) {
      const int t = 32 * ph + u;
      const float kd = ld1f(sK + t * LDK + ci) * rr;
      x4[u & 3] = kd;
      __builtin_nontemporal_store(kd, a.Kd + (sh * C + t) * D + ci);
      if ((u & 3) == 0) *reinterpret_cast<float4*>(kdt + u) = make_float4(x4[0], x4[1], x4[2], x4[3]);
      rr *= al[u];
    }
  }
  if constexpr (P::COMPACT) __syncthreads();  // T lies over Aqk: the (scale Aqk)^T writes are done
  for (int idx = tid; idx < P::CM; idx += NTH) sT[idx] = 0.f;
  __syncthreads();  // K and Q no longer needed; T zeroed
  float* sKbT = P::COMPACT ? sm + P::R0 : reinterpret_cast<float*>(sQ);  // (K*b)^T [i][t]
  KQ* sVT = P::COMPACT ? reinterpret_cast<KQ*>(sAb) : sK;                // V^T [i][t]
  if (chan) {
#pragma unroll
    for (int u = 0; u < 32; u += 4)
      *reinterpret_cast<float4*>(sKbT + ci * LM + 32 * ph + u) = make_float4(kb[u], kb[u + 1], kb[u + 2], kb[u + 3]);
  }
  // V^T: the fp32 layout stages it now; the compact one loads V into
  // registers and writes it over Akk once the solve below is done with Akk
  constexpr int VG = D / 4, VN = C * VG, VIT = (VN + NTH - 1) / NTH;
  uint2 vx[P::COMPACT ? VIT : 1];
  if constexpr (P::COMPACT) {
#pragma unroll
    for (int it = 0; it < VIT; ++it) {
      const int idx = it * NTH + tid, t = idx / VG, g4 = idx - t * VG;
      const uint2 y = *reinterpret_cast<const uint2*>(v + ((L.tok0 + min(t, L.count - 1)) * a.H + h) * D + 4 * g4);
      vx[it] = t < L.count ? y : make_uint2(0u, 0u);
    }
  } else {
    load_rows_t<D, LM, In, NTH>(sVT, v, L.tok0, L.count, a.H, h);
  }
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
  float* scr = sm + P::R4 + w * 16 * 17;  // (waves wv < 4 only)
  for (int I = 1; I < 4; ++I) {
    __syncthreads();
    if (wv < I) {
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
    if (wv < I) {
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
  for (int idx = tid; idx < C * C; idx += NTH) {
    const int t = idx / C, s = idx - t * C;
    __builtin_nontemporal_store(sT[s * LM + t], a.Tm + sh * C * C + idx);  // T^T
  }
  if constexpr (P::COMPACT) {  // V^T over Akk (the solve is done with it)
    uint16_t* vt = reinterpret_cast<uint16_t*>(sVT);
#pragma unroll
    for (int it = 0; it < VIT; ++it) {
      const int idx = it * NTH + tid, t = idx / VG, c = 4 * (idx - t * VG);
      if (idx >= VN) continue;
      vt[(c + 0) * P::LMV + t] = static_cast<uint16_t>(vx[it].x);
      vt[(c + 1) * P::LMV + t] = static_cast<uint16_t>(vx[it].x >> 16);
      vt[(c + 2) * P::LMV + t] = static_cast<uint16_t>(vx[it].y);
      vt[(c + 3) * P::LMV + t] = static_cast<uint16_t>(vx[it].y >> 16);
    }
    __syncthreads();
  }
  // W = T diag(beta) (K*b), U = T diag(beta) V; T is lower triangular, so
  // rows [16w, 16w + 16) contract over s < 16 (w + 1)
  constexpr int NCT = D / 16, NCTP = (NTH == 512 && NCT >= 2) ? NCT / 2 : NCT;
  constexpr bool PAIRED = NTH == 256 && NCT >= 2;  // 4 waves: paired row blocks, half the column tiles each
  constexpr int NCW = PAIRED ? NCT / 2 : NCTP;     // column tiles per wave
  constexpr int NB = NCW < 4 ? NCW : 4;
  // rows [16 rb, 16 rb + 16) of W and U, column tiles [c0, c0 + NB)
  auto wu_block = [&](int rb, int c0) {
    const int kend = 16 * (rb + 1);
    f32x4 accW[NB], accU[NB];
#pragma unroll
    for (int n = 0; n < NB; ++n) accW[n] = accU[n] = zero4f();
    for (int k0 = 0; k0 < kend; k0 += 16) {
      const float4 tv = *reinterpret_cast<const float4*>(sT + (16 * rb + r) * LM + k0 + 4 * kq);
      const float4 bs = *reinterpret_cast<const float4*>(sBeta + k0 + 4 * kq);
      const float4 av = make_float4(tv.x * bs.x, tv.y * bs.y, tv.z * bs.z, tv.w * bs.w);
      float4 bw[NB], bu[NB];
#pragma unroll
      for (int n = 0; n < NB; ++n) {
        bw[n] = *reinterpret_cast<const float4*>(sKbT + (16 * (c0 + n) + r) * LM + k0 + 4 * kq);
        bu[n] = load4(sVT + (16 * (c0 + n) + r) * P::LMV + k0 + 4 * kq);
      }
#pragma unroll
      for (int n = 0; n < NB; ++n) {
        accW[n] = mma(av.x, bw[n].x, accW[n]);
        accU[n] = mma(av.x, bu[n].x, accU[n]);
      }
#pragma unroll
      for (int n = 0; n < NB; ++n) {
        accW[n] = mma(av.y, bw[n].y, accW[n]);
        accU[n] = mma(av.y, bu[n].y, accU[n]);
      }
#pragma unroll
      for (int n = 0; n < NB; ++n) {
        accW[n] = mma(av.z, bw[n].z, accW[n]);
        accU[n] = mma(av.z, bu[n].z, accU[n]);
      }
#pragma unroll
      for (int n = 0; n < NB; ++n) {
        accW[n] = mma(av.w, bw[n].w, accW[n]);
        accU[n] = mma(av.w, bu[n].w, accU[n]);
      }
    }
#pragma unroll
    for (int n = 0; n < NB; ++n) {
      const int i = 16 * (c0 + n) + r;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int t = 16 * rb + 4 * kq + j;
        a.Wm[(sh * C + t) * D + i] = accW[n][j];
        a.Um[(sh * C + t) * D + i] = accU[n][j];
      }
      *reinterpret_cast<float4*>(a.WT + (sh * D + i) * C + 16 * rb + 4 * kq) =
          make_float4(accW[n][0], accW[n][1], accW[n][2], accW[n][3]);
    }
  };
  if constexpr (!PAIRED) {
    // 8 waves: block w, the column tiles of half hf (D = 16: one tile, first half)
#pragma unroll
    for (int cc = 0; cc < NCTP; cc += NB) {
      const int c0 = hf * NCTP + cc;
      if (c0 < NCT) wu_block(w, c0);
    }
  } else {
    // 4 waves: block I costs I + 1 steps of 16, so waves pair blocks {0, 3}
    // and {1, 2} and split the column tiles, 5 steps each
    const int rb0 = w < 2 ? 0 : 1;
#pragma unroll
    for (int e = 0; e < 2; ++e)
#pragma unroll
      for (int cc = 0; cc < NCW; cc += NB) wu_block(e == 0 ? rb0 : 3 - rb0, (w & 1) * NCW + cc);
  }
}

// ---------------------------------------------------------------------------
// Scans: per (unit, 32-column value tile), serially over the unit's chunks.
// The state (or state-gradient) tile lives in LDS transposed, [column][i], so
// that every product reads both operands along the contraction index; the
// next chunk's operands are loaded into registers while the current chunk is
// computed.
template <int D>
struct ScanL {
  static constexpr int DVT = D < 32 ? D : 32;
  static constexpr int NTILE = D / DVT;
  static constexpr int NBC = DVT / 16;  // 16-column blocks per tile
  static constexpr int LD = D + 4, LM = C + 4, LV = DVT + 4;
  // forward: S^T tile, W rows, Kd^T rows, U tile, Delta^T tile, b_C
  static constexpr int FS = 0, FW = FS + DVT * LD, FK = FW + C * LD, FU = FK + D * LM, FX = FU + C * LV,
                       FG = FX + DVT * LM, F_FLOATS = FG + D;
  // reverse: dS^T tile, As^T rows, Kd rows, Qs^T rows, W^T rows, dO^T tile, dDelta^T tile, b_C
  static constexpr int RS = 0, RA = RS + DVT * LD, RK = RA + C * LM, RQ = RK + C * LD, RW = RQ + D * LM,
                       RO = RW + D * LM, RX = RO + DVT * LM, RG = RX + DVT * LM, R_FLOATS = RG + D;
};

// Registers holding one ROWS x COLS block of a row-major global matrix
// (leading dimension ldg, first column c0) on its way to LDS: the loads are
// issued early and the block is written to LDS after the work they overlap.
template <int ROWS, int COLS, int NTH = NT>
struct Staged {
  static constexpr int G = COLS / 4, N = ROWS * G, IT = (N + NTH - 1) / NTH;
  float4 x[IT];
  // (the scans' next-chunk prefetch; these branches do not hold the scan
  // loop, whose loads have a whole step to arrive)
  __device__ __forceinline__ void load(const float* src, int ldg, int c0, int valid_rows = ROWS) {
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      const int idx = it * NTH + threadIdx.x, t = idx / G, g4 = idx - t * G;
      x[it] = make_float4(0.f, 0.f, 0.f, 0.f);
      if (idx < N && t < valid_rows) x[it] = load4(src + static_cast<int64_t>(t) * ldg + c0 + 4 * g4);
    }
  }
  // rows of tokens of a [tokens, H, D] tensor (rows >= valid_rows zero)
  __device__ __forceinline__ void load_tokens(const float* src, int64_t tok0, int H, int h, int D, int c0,
                                              int valid_rows) {
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      const int idx = it * NTH + threadIdx.x, t = idx / G, g4 = idx - t * G;
      x[it] = make_float4(0.f, 0.f, 0.f, 0.f);
      if (idx < N && t < valid_rows) x[it] = load4(src + ((tok0 + t) * H + h) * D + c0 + 4 * g4);
    }
  }
  // The same without branches: unconditional loads from a row clamped into
  // range (valid_rows >= 1), rows >= valid_rows replaced by zeros afterwards.
  __device__ __forceinline__ void load_all(const float* src, int ldg, int c0) {
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      const int idx = it * NTH + threadIdx.x, t = idx / G, g4 = idx - t * G;
      x[it] = load4(src + static_cast<int64_t>(min(t, ROWS - 1)) * ldg + c0 + 4 * g4);
    }
  }
  __device__ __forceinline__ void load_tokens_all(const float* src, int64_t tok0, int H, int h, int D, int c0,
                                                  int valid_rows) {
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      const int idx = it * NTH + threadIdx.x, t = idx / G, g4 = idx - t * G;
      const float4 y = load4(src + ((tok0 + min(t, valid_rows - 1)) * H + h) * D + c0 + 4 * g4);
      x[it] = t < valid_rows ? y : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  }
  __device__ __forceinline__ void store(float* dst, int ld) const {
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      const int idx = it * NTH + threadIdx.x, t = idx / G, g4 = idx - t * G;
      if (idx < N) *reinterpret_cast<float4*>(dst + t * ld + 4 * g4) = x[it];
    }
  }
  __device__ __forceinline__ void store_t(float* dst, int ldt) const {
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      const int idx = it * NTH + threadIdx.x, t = idx / G, c = 4 * (idx - t * G);
      if (idx < N) {
        dst[(c + 0) * ldt + t] = x[it].x;
        dst[(c + 1) * ldt + t] = x[it].y;
        dst[(c + 2) * ldt + t] = x[it].z;
        dst[(c + 3) * ldt + t] = x[it].w;
      }
    }
  }
};

// A D x DVT tile kept transposed in LDS (tT[col * LD + i]) to or from the
// row-major D x D global matrix g at columns [c0, c0 + DVT).
template <int D, int DVT, int LD, int NTH = NT>
__device__ __forceinline__ void tile_to_global(float* g, int c0, const float* tT) {
  constexpr int G = DVT / 4;
  for (int idx = threadIdx.x; idx < D * G; idx += NTH) {
    const int i = idx / G, c = 4 * (idx - i * G);
    *reinterpret_cast<float4*>(g + static_cast<size_t>(i) * D + c0 + c) =
        make_float4(tT[c * LD + i], tT[(c + 1) * LD + i], tT[(c + 2) * LD + i], tT[(c + 3) * LD + i]);
  }
}
template <int D, int DVT, int LD, int NTH = NT>
__device__ __forceinline__ void tile_from_global(float* tT, const float* g, int c0) {
  constexpr int G = DVT / 4;
  for (int idx = threadIdx.x; idx < D * G; idx += NTH) {
    const int i = idx / G, c = 4 * (idx - i * G);
    const float4 x = g ? load4(g + static_cast<size_t>(i) * D + c0 + c) : make_float4(0.f, 0.f, 0.f, 0.f);
    tT[c * LD + i] = x.x;
    tT[(c + 1) * LD + i] = x.y;
    tT[(c + 2) * LD + i] = x.z;
    tT[(c + 3) * LD + i] = x.w;
  }
}

template <int NB>
__device__ __forceinline__ void mm_kc(f32x4 (&acc)[NB], const float* A, int lda, const float* Bt, int ldb, int k_lo,
                                      int k_hi);

// Block -> (unit, value tile): the NTILE tiles of a unit are 8 blocks apart,
// so they run on one XCD and the chunk operands they all read (W, Kd, ...)
// come from HBM once into that XCD's L2.
__device__ __forceinline__ void scan_block(int& unit, int& tile, int ntile) {
  const int b = blockIdx.x, grp = b / (8 * ntile), rem = b - grp * 8 * ntile;
  tile = rem / 8;
  unit = grp * 8 + (rem & 7);
}

constexpr int NSC = 512;  // scan threads: 8 waves

// bwd_fscan: entry state of every chunk, and Delta = U - W S.
template <int D>
__global__ void __launch_bounds__(NSC) bwd_fscan(BwdArgs a) {
  using P = ScanL<D>;
  constexpr int DVT = P::DVT, NBC = P::NBC, LD = P::LD, LM = P::LM, LV = P::LV;
  extern __shared__ __align__(16) float sm[];
  float* sST = sm + P::FS;
  float* sW = sm + P::FW;
  float* sKT = sm + P::FK;
  float* sU = sm + P::FU;
  float* sXT = sm + P::FX;
  float* sG = sm + P::FG;

  int unit, tile;
  scan_block(unit, tile, P::NTILE);
  if (unit >= a.N * a.H) return;
  const int n = unit / a.H, h = unit - n * a.H;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, r = lane & 15, kq = lane >> 4;
  const int c0 = tile * DVT;
  int first, nch;
  unit_chunks(a, n, first, nch);

  tile_from_global<D, DVT, LD, NSC>(
      sST, a.init_state ? a.init_state + (static_cast<size_t>(n) * a.H + h) * D * D : nullptr, c0);
  Staged<C, D, NSC> pW;
  Staged<D, C, NSC> pK;
  Staged<C, DVT, NSC> pU;
  Staged<1, D, NSC> pG;
  auto fetch = [&](int c) {
    const size_t sh = static_cast<size_t>(first + c) * a.H + h;
    pW.load(a.Wm + sh * C * D, D, 0);
    pK.load(a.KdT + sh * D * C, C, 0);
    pU.load(a.Um + sh * C * D, D, c0);
    pG.load(a.eg + sh * D, D, 0);
  };
  if (nch > 0) fetch(0);
  for (int c = 0; c < nch; ++c) {
    const size_t sh = static_cast<size_t>(first + c) * a.H + h;
    __syncthreads();  // the previous chunk is done with every buffer
    pW.store(sW, LD);
    pK.store(sKT, LM);
    pU.store(sU, LV);
    pG.store(sG, D);
    if (c + 1 < nch) fetch(c + 1);
    tile_to_global<D, DVT, LD, NSC>(a.S_in + sh * D * D, c0, sST);
    __syncthreads();
    // Delta = U - W S: wave w, rows [16 (w & 3), +16), columns [16 (w >> 2), +16)
    if (w < 4 * NBC) {
      const int I = w & 3, nb = w >> 2;
      f32x4 acc[1] = {zero4f()};
      mm_kc<1>(acc, sW + 16 * I * LD, LD, sST + 16 * nb * LD, LD, 0, D);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int t = 16 * I + 4 * kq + j, col = 16 * nb + r;
        const float dl = sU[t * LV + col] - acc[0][j];
        sXT[col * LM + t] = dl;
        a.Dl[(sh * C + t) * D + c0 + col] = dl;
      }
    }
    __syncthreads();
    // S = b_C S + Kd^T Delta
    for (int ib = w; ib < D / 16; ib += 8) {
      f32x4 acc[NBC];
#pragma unroll
      for (int nb = 0; nb < NBC; ++nb) acc[nb] = zero4f();
      mm_kc<NBC>(acc, sKT + 16 * ib * LM, LM, sXT, LM, 0, C);
#pragma unroll
      for (int nb = 0; nb < NBC; ++nb)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int i = 16 * ib + 4 * kq + j, col = 16 * nb + r;
          sST[col * LD + i] = sG[i] * sST[col * LD + i] + acc[nb][j];
        }
    }
  }
}

// ---------------------------------------------------------------------------
// Scans with split-bf16 products (bf16 inputs): about 16 bits of precision per
// product term at 16 times the matrix rate of fp32.  The state itself stays
// fp32; its split copy is refreshed after each update.
// acc[n] += A[16 rows][k] * Bt[16 rows + 16 n][k] over k in [k_lo, k_hi), both
// operands split (hi, lo arrays of bf16 bits, row strides lda, ldb in
// elements); lane (r, g) feeds k = k0 + 8 g + j of each 32-wide block.
template <int NB>
__device__ __forceinline__ void mm3(f32x4 (&acc)[NB], const uint16_t* Ah, const uint16_t* Al, int lda,
                                    const uint16_t* Bh, const uint16_t* Bl, int ldb, int k_lo, int k_hi) {
  const int lane = threadIdx.x & 63, r = lane & 15, g = lane >> 4;
  const int ao = r * lda + 8 * g, bo = r * ldb + 8 * g;
  f32x4 cross[NB];
#pragma unroll
  for (int n = 0; n < NB; ++n) cross[n] = zero4f();
  for (int k0 = k_lo; k0 < k_hi; k0 += 32) {
    const bf16x8 ah = *reinterpret_cast<const bf16x8*>(Ah + ao + k0);
    const bf16x8 al = *reinterpret_cast<const bf16x8*>(Al + ao + k0);
#pragma unroll
    for (int n = 0; n < NB; ++n) {
      const bf16x8 bh = *reinterpret_cast<const bf16x8*>(Bh + 16 * n * ldb + bo + k0);
      const bf16x8 bl = *reinterpret_cast<const bf16x8*>(Bl + 16 * n * ldb + bo + k0);
      acc[n] = mfma_bf(ah, bh, acc[n]);
      cross[n] = mfma_bf(ah, bl, cross[n]);
      cross[n] = mfma_bf(al, bh, cross[n]);
    }
  }
#pragma unroll
  for (int n = 0; n < NB; ++n) acc[n] += cross[n];
}

// Split layout of the forward scan (bytes): S^T fp32 and split, W rows split,
// Kd^T rows split, U tile fp32, Delta^T split, b_C.
template <int D>
struct ScanLS {
  using B = ScanL<D>;
  static constexpr int DVT = B::DVT, LD = B::LD, LV = B::LV;
  static constexpr int LDH = D + 8, LMH = C + 8;  // bf16 row strides
  static constexpr size_t SST = 0;
  static constexpr size_t SSH = SST + sizeof(float) * DVT * LD;
  static constexpr size_t SSL = SSH + 2 * DVT * LDH;
  static constexpr size_t SWH = SSL + 2 * DVT * LDH;
  static constexpr size_t SWL = SWH + 2 * C * LDH;
  static constexpr size_t SKH = SWL + 2 * C * LDH;
  static constexpr size_t SKL = SKH + 2 * D * LMH;
  static constexpr size_t SU = SKL + 2 * D * LMH;
  static constexpr size_t SXH = SU + sizeof(float) * C * LV;
  static constexpr size_t SXL = SXH + 2 * DVT * LMH;
  static constexpr size_t SG = SXL + 2 * DVT * LMH;
  static constexpr size_t BYTES = SG + sizeof(float) * D;
};

// Registers of a staged block written split (rows of ld elements).
template <int ROWS, int COLS, int NTH>
__device__ __forceinline__ void store_split(const Staged<ROWS, COLS, NTH>& s, uint16_t* hi, uint16_t* lo, int ld) {
  constexpr int G = COLS / 4;
#pragma unroll
  for (int it = 0; it < Staged<ROWS, COLS, NTH>::IT; ++it) {
    const int idx = it * NTH + threadIdx.x, t = idx / G, g4 = idx - t * G;
    if (idx < Staged<ROWS, COLS, NTH>::N) put_split4(hi + t * ld + 4 * g4, lo + t * ld + 4 * g4, s.x[it]);
  }
}

// Row-major LDS operands of bwd_gstate, fp32 rows (SP = false) or split rows
// (SP = true): a row of K values holds its K hi bf16 then its K lo bf16 in
// the same row stride (K + 4 floats), so either layout fits the same region.
__device__ __forceinline__ float bf2f(uint16_t b) { return __uint_as_float(static_cast<uint32_t>(b) << 16); }

template <bool SP>
__device__ __forceinline__ float ld_el(const float* base, int row, int ld, int K, int col) {
  if constexpr (SP) {
    const uint16_t* p = reinterpret_cast<const uint16_t*>(base) + 2 * row * ld;
    return bf2f(p[col]) + bf2f(p[K + col]);
  } else {
    return base[row * ld + col];
  }
}
template <bool SP>
__device__ __forceinline__ void st_el(float* base, int row, int ld, int K, int col, float v) {
  if constexpr (SP) {
    uint16_t* p = reinterpret_cast<uint16_t*>(base) + 2 * row * ld;
    put_split(p + col, p + K + col, v);
  } else {
    base[row * ld + col] = v;
  }
}
// acc[n] += A rows x Bt rows over k in [k_lo, k_hi) (rows of K values, strides in floats)
template <bool SP, int NB>
__device__ __forceinline__ void mm_any(f32x4 (&acc)[NB], const float* A, int lda, const float* Bt, int ldb, int K,
                                       int k_lo, int k_hi) {
  if constexpr (SP) {
    const uint16_t* a16 = reinterpret_cast<const uint16_t*>(A);
    const uint16_t* b16 = reinterpret_cast<const uint16_t*>(Bt);
    mm3<NB>(acc, a16, a16 + K, 2 * lda, b16, b16 + K, 2 * ldb, k_lo, k_hi);
  } else {
    mm_kc<NB>(acc, A, lda, Bt, ldb, k_lo, k_hi);
  }
}
template <bool SP, int ROWS, int COLS, int NTH>
__device__ __forceinline__ void stage_store(const Staged<ROWS, COLS, NTH>& st, float* dst, int ld) {
  if constexpr (SP) {
    uint16_t* d16 = reinterpret_cast<uint16_t*>(dst);
    store_split(st, d16, d16 + COLS, 2 * ld);
  } else {
    st.store(dst, ld);
  }
}
// bwd_fscan with split-bf16 products: entry state of every chunk, Delta = U - W S.
template <int D>
__global__ void __launch_bounds__(NSC) bwd_fscan3(BwdArgs a) {
  using P = ScanLS<D>;
  constexpr int DVT = P::DVT, NBC = DVT / 16, LD = P::LD, LV = P::LV, LDH = P::LDH, LMH = P::LMH;
  constexpr int LM = ScanL<D>::LM;
  extern __shared__ __align__(16) unsigned char smb[];
  float* sST = reinterpret_cast<float*>(smb + P::SST);
  uint16_t* sSh = reinterpret_cast<uint16_t*>(smb + P::SSH);
  uint16_t* sSl = reinterpret_cast<uint16_t*>(smb + P::SSL);
  uint16_t* sWh = reinterpret_cast<uint16_t*>(smb + P::SWH);
  uint16_t* sWl = reinterpret_cast<uint16_t*>(smb + P::SWL);
  uint16_t* sKh = reinterpret_cast<uint16_t*>(smb + P::SKH);
  uint16_t* sKl = reinterpret_cast<uint16_t*>(smb + P::SKL);
  float* sU = reinterpret_cast<float*>(smb + P::SU);
  uint16_t* sXh = reinterpret_cast<uint16_t*>(smb + P::SXH);
  uint16_t* sXl = reinterpret_cast<uint16_t*>(smb + P::SXL);
  float* sG = reinterpret_cast<float*>(smb + P::SG);

  int unit, tile;
  scan_block(unit, tile, ScanL<D>::NTILE);
  if (unit >= a.N * a.H) return;
  const int n = unit / a.H, h = unit - n * a.H;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, r = lane & 15, kq = lane >> 4;
  const int c0 = tile * DVT;
  int first, nch;
  unit_chunks(a, n, first, nch);

  tile_from_global<D, DVT, LD, NSC>(
      sST, a.init_state ? a.init_state + (static_cast<size_t>(n) * a.H + h) * D * D : nullptr, c0);
  __syncthreads();
  for (int idx = tid; idx < DVT * D; idx += NSC) {
    const int col = idx / D, i = idx - col * D;
    put_split(sSh + col * LDH + i, sSl + col * LDH + i, sST[col * LD + i]);
  }
  // W and Kd^T arrive fp32 and are split as they are staged
  Staged<C, D, NSC> pW;
  Staged<D, C, NSC> pK;
  Staged<C, DVT, NSC> pU;
  Staged<1, D, NSC> pG;
  auto fetch = [&](int c) {
    const size_t sh = static_cast<size_t>(first + c) * a.H + h;
    pW.load(a.Wm + sh * C * D, D, 0);
    pK.load(a.KdT + sh * D * C, C, 0);
    pU.load(a.Um + sh * C * D, D, c0);
    pG.load(a.eg + sh * D, D, 0);
  };
  if (nch > 0) fetch(0);
  for (int c = 0; c < nch; ++c) {
    const size_t sh = static_cast<size_t>(first + c) * a.H + h;
    __syncthreads();  // the previous chunk is done with every buffer
    store_split(pW, sWh, sWl, LDH);
    store_split(pK, sKh, sKl, LMH);
    pU.store(sU, LV);
    pG.store(sG, D);
    if (c + 1 < nch) fetch(c + 1);
    tile_to_global<D, DVT, LD, NSC>(a.S_in + sh * D * D, c0, sST);
    __syncthreads();
    // Delta = U - W S: wave w, rows [16 (w & 3), +16), columns [16 (w >> 2), +16)
    if (w < 4 * NBC) {
      const int I = w & 3, nb = w >> 2;
      f32x4 acc[1] = {zero4f()};
      mm3<1>(acc, sWh + 16 * I * LDH, sWl + 16 * I * LDH, LDH, sSh + 16 * nb * LDH, sSl + 16 * nb * LDH, LDH, 0, D);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int t = 16 * I + 4 * kq + j, col = 16 * nb + r;
        const float dl = sU[t * LV + col] - acc[0][j];
        put_split(sXh + col * LMH + t, sXl + col * LMH + t, dl);
        a.Dl[(sh * C + t) * D + c0 + col] = dl;
      }
    }
    __syncthreads();
    // S = b_C S + Kd^T Delta (fp32 state; its split copy refreshed)
    for (int ib = w; ib < D / 16; ib += 8) {
      f32x4 acc[NBC];
#pragma unroll
      for (int nb = 0; nb < NBC; ++nb) acc[nb] = zero4f();
      mm3<NBC>(acc, sKh + 16 * ib * LMH, sKl + 16 * ib * LMH, LMH, sXh, sXl, LMH, 0, C);
#pragma unroll
      for (int nb = 0; nb < NBC; ++nb)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int i = 16 * ib + 4 * kq + j, col = 16 * nb + r;
          const float v = sG[i] * sST[col * LD + i] + acc[nb][j];
          sST[col * LD + i] = v;
          put_split(sSh + col * LDH + i, sSl + col * LDH + i, v);
        }
    }
  }
  (void)LM;
}

// Split layout of the reverse scan (bytes): dS^T split (the fp32 dS tile is
// held in registers), As^T rows, Kd rows, Qs^T rows, W^T rows, dO^T and
// dDelta^T tiles, all split; b_C.
template <int D>
struct ScanLR {
  static constexpr int DVT = ScanL<D>::DVT;
  static constexpr int LDH = D + 8, LMH = C + 8;  // bf16 row strides
  static constexpr size_t SSH = 0;
  static constexpr size_t SSL = SSH + 2 * DVT * LDH;
  static constexpr size_t SAH = SSL + 2 * DVT * LDH;
  static constexpr size_t SAL = SAH + 2 * C * LMH;
  static constexpr size_t SKH = SAL + 2 * C * LMH;
  static constexpr size_t SKL = SKH + 2 * C * LDH;
  static constexpr size_t SQH = SKL + 2 * C * LDH;
  static constexpr size_t SQL = SQH + 2 * D * LMH;
  static constexpr size_t SWH = SQL + 2 * D * LMH;
  static constexpr size_t SWL = SWH + 2 * D * LMH;
  static constexpr size_t SOH = SWL + 2 * D * LMH;
  static constexpr size_t SOL = SOH + 2 * DVT * LMH;
  static constexpr size_t SXH = SOL + 2 * DVT * LMH;
  static constexpr size_t SXL = SXH + 2 * DVT * LMH;
  static constexpr size_t SG = SXL + 2 * DVT * LMH;
  static constexpr size_t BYTES = SG + sizeof(float) * D;
  static_assert(BYTES <= 160 * 1024, "fits one CU's LDS");
};

// bwd_rscan with split-bf16 products: backwards over the unit's chunks,
// dDelta and the exit-state gradient of every chunk, and dS0.  Wave w owns
// the dS elements (16 w + 4 kq + j, 16 nb + r) of the tile in registers.
template <int D>
__global__ void __launch_bounds__(NSC) bwd_rscan3(BwdArgs a) {
  using P = ScanLR<D>;
  constexpr int DVT = P::DVT, NBC = DVT / 16, LDH = P::LDH, LMH = P::LMH;
  extern __shared__ __align__(16) unsigned char smb[];
  uint16_t* sSh = reinterpret_cast<uint16_t*>(smb + P::SSH);
  uint16_t* sSl = reinterpret_cast<uint16_t*>(smb + P::SSL);
  uint16_t* sAh = reinterpret_cast<uint16_t*>(smb + P::SAH);
  uint16_t* sAl = reinterpret_cast<uint16_t*>(smb + P::SAL);
  uint16_t* sKh = reinterpret_cast<uint16_t*>(smb + P::SKH);
  uint16_t* sKl = reinterpret_cast<uint16_t*>(smb + P::SKL);
  uint16_t* sQh = reinterpret_cast<uint16_t*>(smb + P::SQH);
  uint16_t* sQl = reinterpret_cast<uint16_t*>(smb + P::SQL);
  uint16_t* sWh = reinterpret_cast<uint16_t*>(smb + P::SWH);
  uint16_t* sWl = reinterpret_cast<uint16_t*>(smb + P::SWL);
  uint16_t* sOh = reinterpret_cast<uint16_t*>(smb + P::SOH);
  uint16_t* sOl = reinterpret_cast<uint16_t*>(smb + P::SOL);
  uint16_t* sXh = reinterpret_cast<uint16_t*>(smb + P::SXH);
  uint16_t* sXl = reinterpret_cast<uint16_t*>(smb + P::SXL);
  float* sG = reinterpret_cast<float*>(smb + P::SG);

  int unit, tile;
  scan_block(unit, tile, ScanL<D>::NTILE);
  if (unit >= a.N * a.H) return;
  const int n = unit / a.H, h = unit - n * a.H;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, r = lane & 15, kq = lane >> 4;
  const int c0 = tile * DVT;
  int first, nch;
  unit_chunks(a, n, first, nch);
  const size_t uo = (static_cast<size_t>(n) * a.H + h) * D * D;
  const bool owner = w < D / 16;  // this wave holds rows [16 w, 16 w + 16) of dS

  // dS tile in registers: ds[nb][j] = dS[16 w + 4 kq + j][c0 + 16 nb + r]
  float ds[NBC][4];
#pragma unroll
  for (int nb = 0; nb < NBC; ++nb)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int i = 16 * w + 4 * kq + j, col = 16 * nb + r;
      ds[nb][j] = (owner && a.d_final) ? a.d_final[uo + static_cast<size_t>(i) * D + c0 + col] : 0.f;
      if (owner) put_split(sSh + col * LDH + i, sSl + col * LDH + i, ds[nb][j]);
    }
  // the operands arrive fp32 and are split as they are staged
  Staged<C, C, NSC> pA;
  Staged<C, D, NSC> pK;
  Staged<D, C, NSC> pQ;
  Staged<D, C, NSC> pW;
  Staged<C, DVT, NSC> pO;
  Staged<1, D, NSC> pG;
  auto fetch = [&](int c) {
    const int slot = first + c;
    const size_t sh = static_cast<size_t>(slot) * a.H + h;
    Loc L;
    locate(a, slot, L);
    pA.load(a.AsT + sh * C * C, C, 0);
    pK.load(a.Kd + sh * C * D, D, 0);
    pQ.load(a.QsT + sh * D * C, C, 0);
    pW.load(a.WT + sh * D * C, C, 0);
    pO.load_tokens(a.d_out, L.tok0, a.H, h, D, c0, L.count);
    pG.load(a.eg + sh * D, D, 0);
  };
  if (nch > 0) fetch(nch - 1);
  for (int c = nch - 1; c >= 0; --c) {
    const size_t sh = static_cast<size_t>(first + c) * a.H + h;
    __syncthreads();
    store_split(pA, sAh, sAl, LMH);
    store_split(pK, sKh, sKl, LDH);
    store_split(pQ, sQh, sQl, LMH);
    store_split(pW, sWh, sWl, LMH);
    {  // dO^T tile, split
      constexpr int G = DVT / 4;
#pragma unroll
      for (int it = 0; it < decltype(pO)::IT; ++it) {
        const int idx = it * NSC + tid, t = idx / G, cc = 4 * (idx - t * G);
        if (idx >= decltype(pO)::N) continue;
        put_split(sOh + (cc + 0) * LMH + t, sOl + (cc + 0) * LMH + t, pO.x[it].x);
        put_split(sOh + (cc + 1) * LMH + t, sOl + (cc + 1) * LMH + t, pO.x[it].y);
        put_split(sOh + (cc + 2) * LMH + t, sOl + (cc + 2) * LMH + t, pO.x[it].z);
        put_split(sOh + (cc + 3) * LMH + t, sOl + (cc + 3) * LMH + t, pO.x[it].w);
      }
    }
    pG.store(sG, D);
    if (c > 0) fetch(c - 1);
    // the exit-state gradient of chunk c
    if (owner) {
#pragma unroll
      for (int nb = 0; nb < NBC; ++nb)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          a.dSo[sh * D * D + static_cast<size_t>(16 * w + 4 * kq + j) * D + c0 + 16 * nb + r] = ds[nb][j];
    }
    __syncthreads();
    // dDelta = As^T dO + Kd dS: wave w, rows [16 (w & 3), +16), columns [16 (w >> 2), +16)
    if (w < 4 * NBC) {
      const int I = w & 3, nb = w >> 2;
      f32x4 acc[1] = {zero4f()};
      mm3<1>(acc, sAh + 16 * I * LMH, sAl + 16 * I * LMH, LMH, sOh + 16 * nb * LMH, sOl + 16 * nb * LMH, LMH, 0, C);
      mm3<1>(acc, sKh + 16 * I * LDH, sKl + 16 * I * LDH, LDH, sSh + 16 * nb * LDH, sSl + 16 * nb * LDH, LDH, 0, D);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int t = 16 * I + 4 * kq + j, col = 16 * nb + r;
        put_split(sXh + col * LMH + t, sXl + col * LMH + t, acc[0][j]);
      }
      *reinterpret_cast<float4*>(a.dDl + (sh * D + c0 + 16 * nb + r) * C + 16 * I + 4 * kq) =
          make_float4(acc[0][0], acc[0][1], acc[0][2], acc[0][3]);  // dDelta^T
    }
    __syncthreads();
    // dS = b_C dS + Qs^T dO - W^T dDelta (fp32 in registers; split copy refreshed)
    if (owner) {
      f32x4 acc[NBC], neg[NBC];
#pragma unroll
      for (int nb = 0; nb < NBC; ++nb) acc[nb] = neg[nb] = zero4f();
      mm3<NBC>(acc, sQh + 16 * w * LMH, sQl + 16 * w * LMH, LMH, sOh, sOl, LMH, 0, C);
      mm3<NBC>(neg, sWh + 16 * w * LMH, sWl + 16 * w * LMH, LMH, sXh, sXl, LMH, 0, C);
#pragma unroll
      for (int nb = 0; nb < NBC; ++nb)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int i = 16 * w + 4 * kq + j, col = 16 * nb + r;
          ds[nb][j] = sG[i] * ds[nb][j] + acc[nb][j] - neg[nb][j];
          put_split(sSh + col * LDH + i, sSl + col * LDH + i, ds[nb][j]);
        }
    }
  }
  if (a.d_init && owner) {
#pragma unroll
    for (int nb = 0; nb < NBC; ++nb)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        a.d_init[uo + static_cast<size_t>(16 * w + 4 * kq + j) * D + c0 + 16 * nb + r] = ds[nb][j];
  }
}

// bwd_rscan: backwards over the unit's chunks; dDelta and the exit-state
// gradient of every chunk, and the gradient of the initial state.
template <int D>
__global__ void __launch_bounds__(NSC) bwd_rscan(BwdArgs a) {
  using P = ScanL<D>;
  constexpr int DVT = P::DVT, NBC = P::NBC, LD = P::LD, LM = P::LM;
  extern __shared__ __align__(16) float sm[];
  float* sST = sm + P::RS;  // dS^T tile
  float* sAT = sm + P::RA;
  float* sKd = sm + P::RK;
  float* sQT = sm + P::RQ;
  float* sWT = sm + P::RW;
  float* sOT = sm + P::RO;  // dO^T tile
  float* sXT = sm + P::RX;  // dDelta^T tile
  float* sG = sm + P::RG;

  int unit, tile;
  scan_block(unit, tile, P::NTILE);
  if (unit >= a.N * a.H) return;
  const int n = unit / a.H, h = unit - n * a.H;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, r = lane & 15, kq = lane >> 4;
  const int c0 = tile * DVT;
  int first, nch;
  unit_chunks(a, n, first, nch);
  const size_t uo = (static_cast<size_t>(n) * a.H + h) * D * D;

  tile_from_global<D, DVT, LD, NSC>(sST, a.d_final ? a.d_final + uo : nullptr, c0);
  Staged<C, C, NSC> pA;
  Staged<C, D, NSC> pK;
  Staged<D, C, NSC> pQ;
  Staged<D, C, NSC> pW;
  Staged<C, DVT, NSC> pO;
  Staged<1, D, NSC> pG;
  auto fetch = [&](int c) {
    const int slot = first + c;
    const size_t sh = static_cast<size_t>(slot) * a.H + h;
    Loc L;
    locate(a, slot, L);
    pA.load(a.AsT + sh * C * C, C, 0);
    pK.load(a.Kd + sh * C * D, D, 0);
    pQ.load(a.QsT + sh * D * C, C, 0);
    pW.load(a.WT + sh * D * C, C, 0);
    pO.load_tokens(a.d_out, L.tok0, a.H, h, D, c0, L.count);
    pG.load(a.eg + sh * D, D, 0);
  };
  if (nch > 0) fetch(nch - 1);
  for (int c = nch - 1; c >= 0; --c) {
    const size_t sh = static_cast<size_t>(first + c) * a.H + h;
    __syncthreads();
    pA.store(sAT, LM);
    pK.store(sKd, LD);
    pQ.store(sQT, LM);
    pW.store(sWT, LM);
    pO.store_t(sOT, LM);
    pG.store(sG, D);
    if (c > 0) fetch(c - 1);
    tile_to_global<D, DVT, LD, NSC>(a.dSo + sh * D * D, c0, sST);
    __syncthreads();
    // dDelta = As^T dO + Kd dS: wave w, rows [16 (w & 3), +16), columns [16 (w >> 2), +16)
    if (w < 4 * NBC) {
      const int I = w & 3, nb = w >> 2;
      f32x4 acc[1] = {zero4f()};
      mm_kc<1>(acc, sAT + 16 * I * LM, LM, sOT + 16 * nb * LM, LM, 0, C);
      mm_kc<1>(acc, sKd + 16 * I * LD, LD, sST + 16 * nb * LD, LD, 0, D);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int t = 16 * I + 4 * kq + j, col = 16 * nb + r;
        sXT[col * LM + t] = acc[0][j];
      }
      *reinterpret_cast<float4*>(a.dDl + (sh * D + c0 + 16 * nb + r) * C + 16 * I + 4 * kq) =
          make_float4(acc[0][0], acc[0][1], acc[0][2], acc[0][3]);  // dDelta^T
    }
    __syncthreads();
    // dS = b_C dS + Qs^T dO - W^T dDelta
    for (int ib = w; ib < D / 16; ib += 8) {
      f32x4 acc[NBC], neg[NBC];
#pragma unroll
      for (int nb = 0; nb < NBC; ++nb) acc[nb] = neg[nb] = zero4f();
      mm_kc<NBC>(acc, sQT + 16 * ib * LM, LM, sOT, LM, 0, C);
      mm_kc<NBC>(neg, sWT + 16 * ib * LM, LM, sXT, LM, 0, C);
#pragma unroll
      for (int nb = 0; nb < NBC; ++nb)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int i = 16 * ib + 4 * kq + j, col = 16 * nb + r;
          sST[col * LD + i] = sG[i] * sST[col * LD + i] + acc[nb][j] - neg[nb][j];
        }
    }
  }
  __syncthreads();
  if (a.d_init) tile_to_global<D, DVT, LD, NSC>(a.d_init + uo, c0, sST);
}

// ---------------------------------------------------------------------------
// Tile products with both operands contiguous along the contraction index k
// (rows of A, rows of Bt): lane (r, kq) reads one float4 per 16-wide k block
// and feeds it to four MFMAs, k = k0 + 4 kq + m for the m-th.  The order of k
// inside a block is the same permutation for A and B, so the sum is unchanged.
// acc[n] += A[16 rows from A][k] * Bt[16 rows from Bt + 16 n ldb][k], k in [k_lo, k_hi).
template <int NB>
__device__ __forceinline__ void mm_kc(f32x4 (&acc)[NB], const float* A, int lda, const float* Bt, int ldb, int k_lo,
                                      int k_hi) {
  const int lane = threadIdx.x & 63, r = lane & 15, kq = lane >> 4;
  const float* ar = A + r * lda + 4 * kq;
  const float* br = Bt + r * ldb + 4 * kq;
  for (int k0 = k_lo; k0 < k_hi; k0 += 16) {
    const float4 a = *reinterpret_cast<const float4*>(ar + k0);
    float4 b[NB];
#pragma unroll
    for (int n = 0; n < NB; ++n) b[n] = *reinterpret_cast<const float4*>(br + 16 * n * ldb + k0);
#pragma unroll
    for (int n = 0; n < NB; ++n) acc[n] = mma(a.x, b[n].x, acc[n]);
#pragma unroll
    for (int n = 0; n < NB; ++n) acc[n] = mma(a.y, b[n].y, acc[n]);
#pragma unroll
    for (int n = 0; n < NB; ++n) acc[n] = mma(a.z, b[n].z, acc[n]);
#pragma unroll
    for (int n = 0; n < NB; ++n) acc[n] = mma(a.w, b[n].w, acc[n]);
  }
}

// A dense ROWS x COLS fp32 matrix into LDS rows (stride LD floats), fp32 or split.
template <bool SP, int ROWS, int COLS, int LD, int NTH>
__device__ __forceinline__ void load_mat_any(float* dst, const float* src) {
  if constexpr (SP) {
    Staged<ROWS, COLS, NTH> st;
    st.load_all(src, COLS, 0);
    uint16_t* d16 = reinterpret_cast<uint16_t*>(dst);
    store_split(st, d16, d16 + COLS, 2 * LD);
  } else {
    load_mat<ROWS, COLS, LD, NTH>(dst, src);
  }
}

// ---------------------------------------------------------------------------
// bwd_gstate: per (chunk, head).  Wave w owns rows [16w, 16w + 16) of every
// C x D result.
template <int D>
struct GsL {
  static constexpr int LD = D + 4, LM = C + 4;
  static constexpr int BIG = (D > C ? D : C) * LD;
  static constexpr int MID = (C * LD > D * LM ? C * LD : D * LM);
  static constexpr int RS = 0;                 // r(C-1, t) (staging), S, Delta (rows)
  static constexpr int RX = RS + BIG;          // dDelta^T (D x LM), dO; then dS' over RX and RR
  static constexpr int RR = RX + MID;          // log_g, b (staging), dR
  static constexpr int RT = RR + C * LD;       // T^T
  static constexpr int RB = RT + C * LM;       // beta [C]
  static constexpr int RE = RB + C;            // b_C [D]
  static constexpr int RY = RE + D;            // dgamma [D]
  static constexpr int RW = RY + D;            // per-wave column sums [4][D]
  static constexpr int RQ = RW + 4 * D;        // dbeta rows, two halves [2][C]
  static constexpr int FLOATS = RQ + 2 * C;
  static constexpr size_t BYTES = sizeof(float) * FLOATS;
};

constexpr int NTS = 512;  // bwd_gstate: 8 waves, two per token block

template <int D, typename In>
__global__ void __launch_bounds__(NTS) bwd_gstate(BwdArgs a) {
  using P = GsL<D>;
  constexpr int LD = P::LD, LM = P::LM, NCT = D / 16;
  // wave wv: token block w = wv & 3, channel tiles [ctb, ctb + NCTH)
  constexpr int NCTH = NCT >= 2 ? NCT / 2 : 1, NB = NCTH < 4 ? NCTH : 4;
  // bf16 inputs: the product operands (T^T, dDelta^T, dR, S, dO, Delta, dS')
  // are held split in LDS, rows of the same stride
  constexpr bool SP = split_scans<D, In>();
  extern __shared__ __align__(16) float sm[];
  float* sS = sm + P::RS;
  float* sX = sm + P::RX;
  float* sR = sm + P::RR;
  float* sT = sm + P::RT;
  float* sBeta = sm + P::RB;
  float* sEg = sm + P::RE;
  float* sGam = sm + P::RY;
  float* sCol = sm + P::RW;
  float* sDb = sm + P::RQ;  // [2][C]: the two halves of each row's dbeta

  const int slot = blockIdx.x / a.H, h = blockIdx.x - slot * a.H;
  Loc L;
  if (!locate(a, slot, L)) return;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, w = wv & 3, half = wv >> 2;
  const int r = lane & 15, kq = lane >> 4;
  const int ctb = half * NCTH;
  const bool active = ctb < NCT;
  const size_t sh = static_cast<size_t>(slot) * a.H + h;
  const In* q = static_cast<const In*>(a.q);
  const In* k = static_cast<const In*>(a.k);
  const In* v = static_cast<const In*>(a.v);
  const int H = a.H;
  auto row = [&](int t) { return (L.tok0 + t) * H + h; };

  if (tid < C) {
    const float bv = a.beta[row(min(tid, L.count - 1))];
    sBeta[tid] = tid < L.count ? bv : 0.f;
  }
  if (tid < 2 * C) sDb[tid] = 0.f;
  load_mat_any<SP, C, C, LM, NTS>(sT, a.Tm + sh * C * C);   // T^T
  load_mat_any<SP, D, C, LM, NTS>(sX, a.dDl + sh * D * C);  // dDelta^T
  load_rows<D, LD, float, NTS>(sR, a.log_g, L.tok0, L.count, H, h);  // log_g rows (0 past the end)
  __syncthreads();
  // the entry state and dO are loaded now and written to LDS after dR
  Staged<D, D, NTS> stS;
  stS.load_all(a.S_in + sh * D * D, D, 0);
  Staged<C, D, NTS> stO;
  stO.load_tokens_all(a.d_out, L.tok0, H, h, D, 0, L.count);
  // per channel: b_t into sR, r(C-1, t) into sS (staging), b_C into sEg
  for (int i = tid; i < D; i += NTS) {
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
  float bb[NCTH][4], rc[NCTH][4], kv[NCTH][4];
#pragma unroll
  for (int c = 0; c < NCTH; ++c)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int t = 16 * w + 4 * kq + j, i = 16 * (ctb + c) + r;
      bb[c][j] = active ? sR[t * LD + i] : 0.f;
      rc[c][j] = active ? sS[t * LD + i] : 0.f;
      const float kx = to_f32(k[row(min(t, L.count - 1)) * D + min(i, D - 1)]);
      kv[c][j] = active && t < L.count ? kx : 0.f;
    }
  __syncthreads();
  // dR = T^T dDelta -> sR;  dv = beta dR.  (T^T)[t][s] = 0 for s < t.
  if (active) {
#pragma unroll
    for (int c0 = 0; c0 < NCTH; c0 += NB) {
      f32x4 acc[NB];
#pragma unroll
      for (int n = 0; n < NB; ++n) acc[n] = zero4f();
      mm_any<SP, NB>(acc, sT + 16 * w * LM, LM, sX + 16 * (ctb + c0) * LM, LM, C, SP ? 32 * (w >> 1) : 16 * w, C);
#pragma unroll
      for (int n = 0; n < NB; ++n)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int t = 16 * w + 4 * kq + j, i = 16 * (ctb + c0 + n) + r;
          st_el<SP>(sR, t, LD, D, i, acc[n][j]);
          if (t < L.count) a.dv[row(t) * D + i] = sBeta[t] * acc[n][j];
        }
    }
  }
  stage_store<SP>(stS, sS, LD);
  __syncthreads();  // dR and S in place; dDelta^T no longer needed
  stage_store<SP>(stO, sX, LD);  // dO
  Staged<D, D, NTS> stD;  // dS', for the row sums against S
  stD.load_all(a.dSo + sh * D * D, D, 0);
  float dq_[NCTH][4], dk_[NCTH][4], dg_[NCTH][4];
  float dbr[4] = {0.f, 0.f, 0.f, 0.f};
  // X = dR S^T: d(K*b) = -beta X, and the R part of dbeta,
  // dR_t . (v_t - (K*b)_t S) = dR_t . v_t - (K*b)_t . X_t
  if (active) {
#pragma unroll
    for (int c0 = 0; c0 < NCTH; c0 += NB) {
      f32x4 acc[NB];
#pragma unroll
      for (int n = 0; n < NB; ++n) acc[n] = zero4f();
      mm_any<SP, NB>(acc, sR + 16 * w * LD, LD, sS + 16 * (ctb + c0) * LD, LD, D, 0, D);
#pragma unroll
      for (int n = 0; n < NB; ++n)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int c = c0 + n, t = 16 * w + 4 * kq + j, i = 16 * (ctb + c) + r;
          const float kb = kv[c][j] * bb[c][j];
          const float vx = to_f32(v[row(min(t, L.count - 1)) * D + i]);
          const float vv = t < L.count ? vx : 0.f;
          dbr[j] += ld_el<SP>(sR, t, LD, D, i) * vv - kb * acc[n][j];
          const float dkb = -sBeta[t] * acc[n][j];
          dk_[c][j] = dkb * bb[c][j];
          dg_[c][j] = dkb * kb;
        }
    }
  }
  __syncthreads();  // dO in place
  Staged<C, D, NTS> stL;  // Delta rows
  stL.load_all(a.Dl + sh * C * D, D, 0);
  // Y = dO S^T: d(Q*b) = scale Y
  if (active) {
#pragma unroll
    for (int c0 = 0; c0 < NCTH; c0 += NB) {
      f32x4 acc[NB];
#pragma unroll
      for (int n = 0; n < NB; ++n) acc[n] = zero4f();
      mm_any<SP, NB>(acc, sX + 16 * w * LD, LD, sS + 16 * (ctb + c0) * LD, LD, D, 0, D);
#pragma unroll
      for (int n = 0; n < NB; ++n)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int c = c0 + n, t = 16 * w + 4 * kq + j, i = 16 * (ctb + c) + r;
          const float dqb = a.scale * acc[n][j];
          const float qx = to_f32(q[row(min(t, L.count - 1)) * D + i]);
          const float qv = t < L.count ? qx : 0.f;
          dq_[c][j] = dqb * bb[c][j];
          dg_[c][j] += dqb * qv * bb[c][j];
        }
    }
  }
  // b_C sum_j dS'[i, j] S[i, j]: D / 4 consecutive threads per row, coalesced
  {
    constexpr int G = D / 4, N = D * G, IT = (N + NTS - 1) / NTS;
    static_assert(G <= 64 && NTS % G == 0 && (N >= NTS || N % 64 == 0), "row groups must stay inside a wave");
    static_assert(decltype(stD)::IT == IT, "same thread mapping as the staged dS'");
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      const int idx = it * NTS + tid, i = idx / G, jj = 4 * (idx - i * G);
      if (idx >= N) continue;  // whole waves
      const float4 xd = stD.x[it];
      float acc = xd.x * ld_el<SP>(sS, i, LD, D, jj) + xd.y * ld_el<SP>(sS, i, LD, D, jj + 1) +
                  xd.z * ld_el<SP>(sS, i, LD, D, jj + 2) + xd.w * ld_el<SP>(sS, i, LD, D, jj + 3);
#pragma unroll
      for (int o = 1; o < G; o <<= 1) acc += __shfl_xor(acc, o, 64);
      if ((tid & (G - 1)) == 0) sGam[i] = sEg[i] * acc;
    }
  }
  __syncthreads();  // done with S
  stage_store<SP>(stL, sS, LD);  // Delta, rows
  __syncthreads();
  stD.load_all(a.dSo + sh * D * D, D, 0);  // dS' again (L2), for Z
  // dAqk = scale tril(dO Delta^T), dA = -tril(dR Delta^T, -1); this wave's
  // two s blocks [2 half, 2 half + 2)
  {
    f32x4 aq[2], aa[2];
    float akk[2][4];
#pragma unroll
    for (int n = 0; n < 2; ++n)
#pragma unroll
      for (int j = 0; j < 4; ++j) akk[n][j] = a.Ab[sh * C * C + (16 * w + 4 * kq + j) * C + 16 * (2 * half + n) + r];
#pragma unroll
    for (int n = 0; n < 2; ++n) aq[n] = aa[n] = zero4f();
    mm_any<SP, 2>(aq, sX + 16 * w * LD, LD, sS + 32 * half * LD, LD, D, 0, D);
    mm_any<SP, 2>(aa, sR + 16 * w * LD, LD, sS + 32 * half * LD, LD, D, 0, D);
#pragma unroll
    for (int n = 0; n < 2; ++n)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int t = 16 * w + 4 * kq + j, s = 16 * (2 * half + n) + r;
        const float gq = s <= t ? a.scale * aq[n][j] : 0.f;
        const float ga = s < t ? -aa[n][j] : 0.f;
        dbr[j] += ga * akk[n][j];
        a.dAq[sh * C * C + t * C + s] = gq;
        a.dAb[sh * C * C + t * C + s] = sBeta[t] * ga;
      }
  }
  // rows of dbeta: reduce over the 16 lanes sharing kq; one half per wave pair
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    float x = dbr[j];
    x += __shfl_xor(x, 1, 64);
    x += __shfl_xor(x, 2, 64);
    x += __shfl_xor(x, 4, 64);
    x += __shfl_xor(x, 8, 64);
    if (r == 0) sDb[half * C + 16 * w + 4 * kq + j] = x;
  }
  __syncthreads();  // done with dO (sX) and dR (sR); Delta rows stay in sS
  static_assert(D * LD <= P::MID + C * LD, "dS' fits over the dO and dR regions");
  stage_store<SP>(stD, sX, LD);  // dS'
  __syncthreads();
  // Z = Delta dS'^T: dKd = Z
  float colp[NCTH];
  if (active) {
#pragma unroll
    for (int c0 = 0; c0 < NCTH; c0 += NB) {
      f32x4 acc[NB];
#pragma unroll
      for (int n = 0; n < NB; ++n) acc[n] = zero4f();
      mm_any<SP, NB>(acc, sS + 16 * w * LD, LD, sX + 16 * (ctb + c0) * LD, LD, D, 0, D);
#pragma unroll
      for (int n = 0; n < NB; ++n) {
        const int c = c0 + n;
        float cs = 0.f;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float kd = kv[c][j] * rc[c][j];
          dk_[c][j] += acc[n][j] * rc[c][j];
          dg_[c][j] -= acc[n][j] * kd;
          cs += acc[n][j] * kd;
        }
        cs += __shfl_xor(cs, 16, 64);
        cs += __shfl_xor(cs, 32, 64);
        colp[c] = cs;
      }
    }
    if (kq == 0)
#pragma unroll
      for (int c = 0; c < NCTH; ++c) sCol[w * D + 16 * (ctb + c) + r] = colp[c];
  }
  __syncthreads();
  // dgamma joins dG at the chunk's last token; the staged parts go through
  // LDS (the operand regions are free now) and out as whole rows
  float* oq = sm + P::RS;
  float* ok = sm + P::RX;
  float* og = sm + P::RR;
  if (active) {
#pragma unroll
    for (int c = 0; c < NCTH; ++c)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int t = 16 * w + 4 * kq + j, i = 16 * (ctb + c) + r;
        float g = dg_[c][j];
        if (t == L.count - 1) g += sGam[i] + sCol[i] + sCol[D + i] + sCol[2 * D + i] + sCol[3 * D + i];
        oq[t * LD + i] = dq_[c][j];
        ok[t * LD + i] = dk_[c][j];
        og[t * LD + i] = g;
      }
  }
  __syncthreads();
  for (int idx = tid; idx < C * (D / 4); idx += NTS) {
    const int t = idx / (D / 4), c4 = 4 * (idx - t * (D / 4));
    if (t >= L.count) continue;
    const int64_t o = row(t) * D + c4;
    // whole rows, read back only by bwd_gpairs: nontemporal
    __builtin_nontemporal_store(*reinterpret_cast<const f32x4*>(oq + t * LD + c4), reinterpret_cast<f32x4*>(a.dq + o));
    __builtin_nontemporal_store(*reinterpret_cast<const f32x4*>(ok + t * LD + c4), reinterpret_cast<f32x4*>(a.dk + o));
    __builtin_nontemporal_store(*reinterpret_cast<const f32x4*>(og + t * LD + c4),
                                reinterpret_cast<f32x4*>(a.dlog_g + o));
  }
  if (tid < L.count) a.dbeta[row(tid)] = sDb[tid] + sDb[C + tid];
}

// ---------------------------------------------------------------------------
// bwd_gpairs: per (chunk, head, group of up to 64 channels): pair terms of Aqk
// and Akk, then dlog_g.  Every term is per channel, so a chunk's channels split
// over NSPL workgroups; that keeps a workgroup's LDS under half of a CU's and
// lets two of them share a CU, one streaming while the other computes.  Q, K
// and the level factors are kept transposed ([channel][token]) so that the
// pair products read them along the contracted token index; bf16 inputs stay
// bf16 in LDS.
template <int D, typename In>
struct GpL {
  static constexpr int CW = D < 64 ? D : 64;  // channels per workgroup
  static constexpr int NSPL = D / CW;         // workgroups per (chunk, head)
  static constexpr int LM = C + 4;
  static constexpr size_t QKB = sizeof(In) * CW * LM;
  static constexpr size_t OQ = 0;                                 // Q^T  [CW][LM] In
  static constexpr size_t OK = OQ + QKB;                          // K^T  [CW][LM] In
  static constexpr size_t OF = OK + QKB;                          // F^T, later dG^T [CW][LM]
  static constexpr size_t OA = OF + sizeof(float) * CW * LM;      // dAqk [C][LM]
  static constexpr size_t OB = OA + sizeof(float) * C * LM;       // dAkk [C][LM]
  static constexpr size_t OS = OB + sizeof(float) * C * LM;       // per-segment totals [8][CW]
  static constexpr size_t BYTES = OS + sizeof(float) * 8 * CW;
};

constexpr int NTG = 512;  // bwd_gpairs: 8 waves, two per token block

// Channels [c0, c0 + CW) of C rows of a [tokens, H, D] tensor, transposed into
// LDS as the input type: dst[c * LDT + t], rows >= count zero.
template <int D, int CW, int LDT, typename In>
__device__ __forceinline__ void load_cols_t(In* dst, const In* src, int64_t tok0, int count, int H, int h, int c0) {
  constexpr int G = CW / 4, N = C * G, IT = (N + NTG - 1) / NTG;
  uint2 xb[IT];   // bf16: 4 raw values
  float4 xf[IT];  // fp32
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int idx = it * NTG + threadIdx.x, t = idx / G, g4 = idx - t * G;
    const In* p = src + ((tok0 + min(t, count - 1)) * H + h) * D + c0 + 4 * g4;
    if constexpr (sizeof(In) == 2) {
      const uint2 y = *reinterpret_cast<const uint2*>(p);
      xb[it] = t < count ? y : make_uint2(0u, 0u);
    } else {
      const float4 y = *reinterpret_cast<const float4*>(p);
      xf[it] = t < count ? y : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  }
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int idx = it * NTG + threadIdx.x, t = idx / G, c = 4 * (idx - t * G);
    if (idx >= N) continue;
    if constexpr (sizeof(In) == 2) {
      uint16_t* d = reinterpret_cast<uint16_t*>(dst);
      d[(c + 0) * LDT + t] = static_cast<uint16_t>(xb[it].x);
      d[(c + 1) * LDT + t] = static_cast<uint16_t>(xb[it].x >> 16);
      d[(c + 2) * LDT + t] = static_cast<uint16_t>(xb[it].y);
      d[(c + 3) * LDT + t] = static_cast<uint16_t>(xb[it].y >> 16);
    } else {
      dst[(c + 0) * LDT + t] = xf[it].x;
      dst[(c + 1) * LDT + t] = xf[it].y;
      dst[(c + 2) * LDT + t] = xf[it].z;
      dst[(c + 3) * LDT + t] = xf[it].w;
    }
  }
}


// Level-l factors of one channel for the 8 tokens [8 seg, 8 seg + 8): al are
// their gates, segtot[s] the product of the gates of segment s (LDS, this
// channel, stride CW).  A half of 8 or more tokens spans whole segments: its
// factors are a product inside the segment times the totals of the segments
// before it (upper half) or after it (lower half) within the half.
template <int L, int CW>
__device__ __forceinline__ void level_factors8(const float (&al)[8], int seg, const float* segtot, float (&f)[8]) {
  constexpr int HH = 32 >> L;
  if constexpr (HH >= 8) {
    constexpr int NS = HH / 8;            // segments per half
    const int s0 = seg & ~(NS - 1);       // first segment of the half
    const bool upper = ((8 * seg) & HH) != 0;
    if (upper) {
      float p = 1.f;
      for (int s = s0; s < seg; ++s) p *= segtot[s * CW];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        p *= al[u];
        f[u] = p;
      }
    } else {
      float p = 1.f;
      for (int s = seg + 1; s < s0 + NS; ++s) p *= segtot[s * CW];
#pragma unroll
      for (int u = 7; u >= 0; --u) {
        f[u] = p;
        p *= al[u];
      }
    }
  } else {
#pragma unroll
    for (int b0 = 0; b0 < 8; b0 += HH) {
      const bool upper = ((b0 & HH) != 0);  // 8 seg is a multiple of 2 HH
      if (upper) {
        float p = 1.f;
#pragma unroll
        for (int u = 0; u < HH; ++u) {
          p *= al[b0 + u];
          f[b0 + u] = p;
        }
      } else {
        float p = 1.f;
#pragma unroll
        for (int u = HH - 1; u >= 0; --u) {
          f[b0 + u] = p;
          p *= al[b0 + u];
        }
      }
    }
  }
}

template <int D, typename In>
__global__ void __launch_bounds__(NTG, 2) bwd_gpairs(BwdArgs a) {
  using P = GpL<D, In>;
  constexpr int CW = P::CW, NSPL = P::NSPL, LM = P::LM, NCT = CW / 16;
  // wave wv: token block w = wv & 3, channel tiles [ctb, ctb + NCTW)
  constexpr int NCTW = NCT >= 2 ? NCT / 2 : 1;
  extern __shared__ __align__(16) unsigned char gsm[];
  In* sQT = reinterpret_cast<In*>(gsm + P::OQ);
  In* sKT = reinterpret_cast<In*>(gsm + P::OK);
  float* sFT = reinterpret_cast<float*>(gsm + P::OF);
  float* sdAq = reinterpret_cast<float*>(gsm + P::OA);
  float* sdAb = reinterpret_cast<float*>(gsm + P::OB);
  float* sSeg = reinterpret_cast<float*>(gsm + P::OS);

  // the NSPL channel groups of a (chunk, head) are 8 blocks apart (one XCD,
  // one L2 for the shared dA tiles)
  const int b = blockIdx.x;
  const int grp = b / (8 * NSPL), rem = b - grp * 8 * NSPL;
  const int part = rem / 8;
  const int sh_idx = grp * 8 + (rem & 7);
  const int slot = sh_idx / a.H, h = sh_idx - slot * a.H;
  if (slot >= a.n_slots) return;
  Loc L;
  if (!locate(a, slot, L)) return;
  const int c0 = part * CW;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, w = wv & 3, r = lane & 15, kq = lane >> 4;
  const int ctb = (wv >> 2) * NCTW;
  const bool active = ctb < NCT;
  const size_t sh = static_cast<size_t>(slot) * a.H + h;
  const int H = a.H;
  auto row = [&](int t) { return (L.tok0 + t) * H + h; };

  load_cols_t<D, CW, LM, In>(sQT, static_cast<const In*>(a.q), L.tok0, L.count, H, h, c0);
  load_cols_t<D, CW, LM, In>(sKT, static_cast<const In*>(a.k), L.tok0, L.count, H, h, c0);
  load_mat<C, C, LM, NTG>(sdAq, a.dAq + sh * C * C);
  load_mat<C, C, LM, NTG>(sdAb, a.dAb + sh * C * C);
  // factor threads: channel fi, tokens [8 seg, 8 seg + 8)
  const int fi = tid % CW, seg = tid / CW;
  const bool fthr = seg < 8;
  float al[8], lg[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) lg[u] = a.log_g[row(min(8 * seg + u, L.count - 1)) * D + c0 + fi];
  __builtin_amdgcn_sched_barrier(0);  // all 8 loads in flight before the first use
#pragma unroll
  for (int u = 0; u < 8; ++u) al[u] = (fthr && 8 * seg + u < L.count) ? exp_fast(lg[u]) : 1.f;
  if (fthr) {
    float p = 1.f;
#pragma unroll
    for (int u = 0; u < 8; ++u) p *= al[u];
    sSeg[seg * CW + fi] = p;
  }

  float dq_[NCTW][4], dk_[NCTW][4], dg_[NCTW][4];
#pragma unroll
  for (int ct = 0; ct < NCTW; ++ct)
#pragma unroll
    for (int j = 0; j < 4; ++j) dq_[ct][j] = dk_[ct][j] = dg_[ct][j] = 0.f;

  // rows of block w against the partner tokens [p0, p0 + plen) at level l:
  // dX (block w in the upper half) or dY (block w in the lower half)
  auto level_terms = [&](int l, bool upper_rows, int p0, int plen) {
#pragma unroll
    for (int ct = 0; ct < NCTW; ++ct) {
      const int i0 = 16 * (ctb + ct);
      const In* bk = sKT + (i0 + r) * LM + 4 * kq;
      const In* bq = sQT + (i0 + r) * LM + 4 * kq;
      const float* bf = sFT + (i0 + r) * LM + 4 * kq;
      if (upper_rows) {
        const int t = 16 * w + r;
        f32x4 xq = zero4f(), xk = zero4f();
        for (int k0 = p0; k0 < p0 + plen; k0 += 16) {
          const int s0 = k0 + 4 * kq;
          const float4 aq = *reinterpret_cast<const float4*>(sdAq + t * LM + s0);
          const float4 ab = *reinterpret_cast<const float4*>(sdAb + t * LM + s0);
          const float4 kk = load4(bk + k0);
          const float4 ff = *reinterpret_cast<const float4*>(bf + k0);
          const bool m0 = at_level(l, t, s0), m1 = at_level(l, t, s0 + 1), m2 = at_level(l, t, s0 + 2),
                     m3 = at_level(l, t, s0 + 3);
          xq = mma(m0 ? aq.x : 0.f, kk.x * ff.x, xq);
          xk = mma(m0 ? ab.x : 0.f, kk.x * ff.x, xk);
          xq = mma(m1 ? aq.y : 0.f, kk.y * ff.y, xq);
          xk = mma(m1 ? ab.y : 0.f, kk.y * ff.y, xk);
          xq = mma(m2 ? aq.z : 0.f, kk.z * ff.z, xq);
          xk = mma(m2 ? ab.z : 0.f, kk.z * ff.z, xk);
          xq = mma(m3 ? aq.w : 0.f, kk.w * ff.w, xq);
          xk = mma(m3 ? ab.w : 0.f, kk.w * ff.w, xk);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int to = 16 * w + 4 * kq + j, i = i0 + r;
          const float ft = sFT[i * LM + to];
          const float gq = ft * xq[j], gk = ft * xk[j];
          dq_[ct][j] += gq;
          dk_[ct][j] += gk;
          dg_[ct][j] += ld1f(sQT + i * LM + to) * gq + ld1f(sKT + i * LM + to) * gk;
        }
      } else {
        const int s = 16 * w + r;
        f32x4 y1 = zero4f(), y2 = zero4f();
        for (int k0 = p0; k0 < p0 + plen; k0 += 16) {
          const int t0 = k0 + 4 * kq;
          const float4 qq = load4(bq + k0);
          const float4 kk = load4(bk + k0);
          const float4 ff = *reinterpret_cast<const float4*>(bf + k0);
          float aq[4], ab[4];
#pragma unroll
          for (int m = 0; m < 4; ++m) {
            const bool ok = at_level(l, t0 + m, s);
            aq[m] = ok ? sdAq[(t0 + m) * LM + s] : 0.f;
            ab[m] = ok ? sdAb[(t0 + m) * LM + s] : 0.f;
          }
          y1 = mma(aq[0], qq.x * ff.x, y1);
          y2 = mma(ab[0], kk.x * ff.x, y2);
          y1 = mma(aq[1], qq.y * ff.y, y1);
          y2 = mma(ab[1], kk.y * ff.y, y2);
          y1 = mma(aq[2], qq.z * ff.z, y1);
          y2 = mma(ab[2], kk.z * ff.z, y2);
          y1 = mma(aq[3], qq.w * ff.w, y1);
          y2 = mma(ab[3], kk.w * ff.w, y2);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int so = 16 * w + 4 * kq + j, i = i0 + r;
          const float gy = sFT[i * LM + so] * (y1[j] + y2[j]);
          dk_[ct][j] += gy;
          dg_[ct][j] -= ld1f(sKT + i * LM + so) * gy;
        }
      }
    }
  };
  // levels 0-2 (pairs across 32-, 16- and 8-token halves) as MFMA tile
  // products; levels 3-5 (pairs inside an aligned 8-token group) below
#pragma unroll
  for (int l = 0; l < 3; ++l) {
    __syncthreads();  // segment totals written; previous level's factors read
    if (fthr) {
      float f[8];
      switch (l) {
        case 0: level_factors8<0, CW>(al, seg, sSeg + fi, f); break;
        case 1: level_factors8<1, CW>(al, seg, sSeg + fi, f); break;
        default: level_factors8<2, CW>(al, seg, sSeg + fi, f); break;
      }
      float* dst = sFT + fi * LM + 8 * seg;
      *reinterpret_cast<float4*>(dst) = make_float4(f[0], f[1], f[2], f[3]);
      *reinterpret_cast<float4*>(dst + 4) = make_float4(f[4], f[5], f[6], f[7]);
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
      level_terms(2, true, 16 * w, 16);
      level_terms(2, false, 16 * w, 16);
    }
  }
  // Pairs t > s inside the 8-token group [8 seg, 8 seg + 8), per channel fi:
  // r(t, s) is a running product of the gates, so each pair costs a few
  // fused multiply-adds on the vector units instead of a masked MFMA level.
  //   a = dAqk r, b = dAkk r:  dq_t += a k_s, dk_t += b k_s,
  //   c = a q_t + b k_t: dk_s += c,  u = k_s c: dG_t += u, dG_s -= u
  float pq[8], pk[8], pg[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) pq[u] = pk[u] = pg[u] = 0.f;
  if (fthr) {
    float kx[8], qx[8];
    {
      const float4 k0 = load4(sKT + fi * LM + 8 * seg), k1 = load4(sKT + fi * LM + 8 * seg + 4);
      const float4 q0 = load4(sQT + fi * LM + 8 * seg), q1 = load4(sQT + fi * LM + 8 * seg + 4);
      kx[0] = k0.x; kx[1] = k0.y; kx[2] = k0.z; kx[3] = k0.w; kx[4] = k1.x; kx[5] = k1.y; kx[6] = k1.z; kx[7] = k1.w;
      qx[0] = q0.x; qx[1] = q0.y; qx[2] = q0.z; qx[3] = q0.w; qx[4] = q1.x; qx[5] = q1.y; qx[6] = q1.z; qx[7] = q1.w;
    }
    const float* aq = sdAq + 8 * seg * LM + 8 * seg;  // aq[t * LM + s]: dAqk of the group's pair (t, s)
    const float* ab = sdAb + 8 * seg * LM + 8 * seg;
#pragma unroll
    for (int s0 = 0; s0 < 7; ++s0) {
      float rr = 1.f;
#pragma unroll
      for (int t0 = s0 + 1; t0 < 8; ++t0) {
        rr *= al[t0];
        const float av = aq[t0 * LM + s0] * rr, bv = ab[t0 * LM + s0] * rr;
        pq[t0] += av * kx[s0];
        pk[t0] += bv * kx[s0];
        const float cv = av * qx[t0] + bv * kx[t0];
        pk[s0] += cv;
        const float uv = kx[s0] * cv;
        pg[t0] += uv;
        pg[s0] -= uv;
      }
    }
  }
  // pairs t = s (r = 1): Aqk only
#pragma unroll
  for (int ct = 0; ct < NCTW; ++ct)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int t = 16 * w + 4 * kq + j, i = 16 * (ctb + ct) + r;
      const float d = sdAq[t * LM + t];
      dq_[ct][j] += d * ld1f(sKT + i * LM + t);
      dk_[ct][j] += d * ld1f(sQT + i * LM + t);
    }
  __syncthreads();  // done with Q^T, K^T, F^T and the dA tiles
  // Sums in [token][channel] rows (stride LO): dq over the dAqk tile, dk over
  // the dAkk tile, dG over Q^T, K^T and F^T; first the in-group terms, then
  // the MFMA lanes' terms, then the state-side parts staged by bwd_gstate,
  // read and written as whole rows.
  constexpr int LO = CW + 4;
  float* oq = sdAq;
  float* ok = sdAb;
  float* og = reinterpret_cast<float*>(gsm + P::OQ);
  static_assert(C * LO * sizeof(float) <= P::OA - P::OQ, "dG rows fit over Q^T, K^T and F^T");
  if (fthr) {
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int t = 8 * seg + u;
      oq[t * LO + fi] = pq[u];
      ok[t * LO + fi] = pk[u];
      og[t * LO + fi] = pg[u];
    }
  }
  __syncthreads();
  if (active) {
#pragma unroll
    for (int ct = 0; ct < NCTW; ++ct)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int t = 16 * w + 4 * kq + j, i = 16 * (ctb + ct) + r;
        oq[t * LO + i] += dq_[ct][j];
        ok[t * LO + i] += dk_[ct][j];
        og[t * LO + i] += dg_[ct][j];
      }
  }
  __syncthreads();
  for (int idx = tid; idx < C * (CW / 4); idx += NTG) {
    const int t = idx / (CW / 4), c4 = 4 * (idx - t * (CW / 4));
    const int64_t o = row(min(t, L.count - 1)) * D + c0 + c4;
    const float4 xq = *reinterpret_cast<const float4*>(a.dq + o), xk = *reinterpret_cast<const float4*>(a.dk + o);
    const float4 xg = *reinterpret_cast<const float4*>(a.dlog_g + o);
    float4* pgq = reinterpret_cast<float4*>(og + t * LO + c4);
    if (t < L.count) {
      const float4 yq = *reinterpret_cast<const float4*>(oq + t * LO + c4);
      const float4 yk = *reinterpret_cast<const float4*>(ok + t * LO + c4);
      const float4 yg = *pgq;
      // the final gradients, whole rows: nontemporal
      __builtin_nontemporal_store(f32x4{xq.x + yq.x, xq.y + yq.y, xq.z + yq.z, xq.w + yq.w},
                                  reinterpret_cast<f32x4*>(a.dq + o));
      __builtin_nontemporal_store(f32x4{xk.x + yk.x, xk.y + yk.y, xk.z + yk.z, xk.w + yk.w},
                                  reinterpret_cast<f32x4*>(a.dk + o));
      *pgq = make_float4(xg.x + yg.x, xg.y + yg.y, xg.z + yg.z, xg.w + yg.w);
    } else {
      *pgq = make_float4(0.f, 0.f, 0.f, 0.f);
    }
  }
  __syncthreads();
  // dlog_g = reverse cumulative sum of dG over the chunk: each factor thread
  // sums its 8 tokens, then adds the totals of the segments after its own
  float g[8];
  if (fthr) {
#pragma unroll
    for (int u = 0; u < 8; ++u) g[u] = og[(8 * seg + u) * LO + fi];
#pragma unroll
    for (int u = 6; u >= 0; --u) g[u] += g[u + 1];
    sSeg[seg * CW + fi] = g[0];
  }
  __syncthreads();
  if (fthr) {
    float off = 0.f;
    for (int s = seg + 1; s < 8; ++s) off += sSeg[s * CW + fi];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int t = 8 * seg + u;
      if (t < L.count) a.dlog_g[row(t) * D + c0 + fi] = g[u] + off;
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
  float* f[16];
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
  const size_t per[16] = {size_t(D) * D, size_t(D) * D, size_t(C) * D, size_t(C) * D, size_t(C) * D,
                          size_t(C) * D, size_t(C) * D, size_t(C) * D, size_t(C) * C, size_t(C) * C,
                          size_t(C) * C, size_t(C) * C, size_t(C) * C, size_t(D), size_t(C) * D, size_t(C) * D};
  for (int i = 0; i < 16; ++i) {
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
                          static_cast<int>(PrepL<D, In>::BYTES));
  if (e != hipSuccess) return e;
  e = hipFuncSetAttribute(reinterpret_cast<const void*>(bwd_gstate<D, In>),
                          hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(GsL<D>::BYTES));
  if (e != hipSuccess) return e;
  e = hipFuncSetAttribute(reinterpret_cast<const void*>(bwd_gpairs<D, In>),
                          hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(GpL<D, In>::BYTES));
  if (e != hipSuccess) return e;
  e = hipFuncSetAttribute(reinterpret_cast<const void*>(bwd_fscan<D>), hipFuncAttributeMaxDynamicSharedMemorySize,
                          static_cast<int>(sizeof(float) * ScanL<D>::F_FLOATS));
  if (e != hipSuccess) return e;
  if constexpr (split_scans<D, In>()) {
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(bwd_fscan3<D>), hipFuncAttributeMaxDynamicSharedMemorySize,
                            static_cast<int>(ScanLS<D>::BYTES));
    if (e != hipSuccess) return e;
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(bwd_rscan3<D>), hipFuncAttributeMaxDynamicSharedMemorySize,
                            static_cast<int>(ScanLR<D>::BYTES));
    if (e != hipSuccess) return e;
  }
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
  const unsigned unit_blocks = static_cast<unsigned>((static_cast<int64_t>(a.N) * a.H + 7) / 8 * 8) * ScanL<D>::NTILE;
  hipError_t e;
  if (chunk_blocks > 0) {
    using PP = PrepL<D, In>;
    hipLaunchKernelGGL((bwd_prep<D, In>), dim3(chunk_blocks), dim3(PP::NTH), PP::BYTES, stream, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if (unit_blocks > 0) {
    if constexpr (split_scans<D, In>())
      hipLaunchKernelGGL((bwd_fscan3<D>), dim3(unit_blocks), dim3(NSC), ScanLS<D>::BYTES, stream, a);
    else
      hipLaunchKernelGGL((bwd_fscan<D>), dim3(unit_blocks), dim3(NSC), sizeof(float) * ScanL<D>::F_FLOATS, stream, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if constexpr (split_scans<D, In>())
      hipLaunchKernelGGL((bwd_rscan3<D>), dim3(unit_blocks), dim3(NSC), ScanLR<D>::BYTES, stream, a);
    else
      hipLaunchKernelGGL((bwd_rscan<D>), dim3(unit_blocks), dim3(NSC), sizeof(float) * ScanL<D>::R_FLOATS, stream, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if (chunk_blocks > 0) {
    hipLaunchKernelGGL((bwd_gstate<D, In>), dim3(chunk_blocks), dim3(NTS), GsL<D>::BYTES, stream, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    using P = GpL<D, In>;
    const unsigned pair_blocks = (chunk_blocks + 7) / 8 * 8 * P::NSPL;
    hipLaunchKernelGGL((bwd_gpairs<D, In>), dim3(pair_blocks), dim3(NTG), P::BYTES, stream, a);
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
  // bwd_gpairs runs up to two workgroups per (slot, head), rounded up to 16
  return (a.d == 16 || a.d == 32 || a.d == 64 || a.d == 128) && (blocks + 16) * 2 < (int64_t(1) << 31) &&
         (int64_t(a.num_seqs) * a.num_heads + 8) * 4 < (int64_t(1) << 31);
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
  a.S_in = l.f[0]; a.dSo = l.f[1]; a.Wm = l.f[2]; a.Um = l.f[3]; a.Kd = l.f[4]; a.QsT = l.f[5];
  a.Dl = l.f[6]; a.dDl = l.f[7]; a.AsT = l.f[8]; a.Tm = l.f[9]; a.Ab = l.f[10]; a.dAq = l.f[11];
  a.dAb = l.f[12]; a.eg = l.f[13]; a.WT = l.f[14]; a.KdT = l.f[15];
  a.N = s.num_seqs; a.T = s.seq_len; a.H = s.num_heads;
  a.cps = packed ? 0 : static_cast<int>((static_cast<int64_t>(s.seq_len) + C - 1) / C);
  a.n_slots = static_cast<int>(ns);
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
