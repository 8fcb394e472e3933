// kda_recurrent.hip -- token-recurrent evaluation of the KDA recurrence (gfx950).
//
// Serves decode and multi-row verify (kda_step), prefill with fp32 q/k/v, and
// any prefill problem the chunked MFMA kernel does not take.  Each workgroup
// owns one (unit, value-column tile): unit = (sequence or packed document n,
// head h), tile = DVT consecutive value columns of the fp32 state S[D][D].
// Value columns never interact (the read-back sums over the key axis only),
// so the tiles of a unit run independently.
//
// The state tile is loaded once (16-byte loads), kept in registers for all of
// the unit's tokens and stored once.  Per token, following the gated delta
// rule of the GLM-5.3-Flash model notes (Glm5NextTextLinearAttention snippet):
//   S' = Diag(exp(log_g_t)) S                   decay of the key axis (rows)
//   a  = S'^T k_t,  b = S'^T q_t,  kq = k_t.q_t     one pass over S'
//   delta = beta_t (v_t - a)
//   S  = S' + k_t delta^T
//   o_t = scale S^T q_t = scale (b + delta kq)     read from the updated state
//
// Thread layout: thread t owns 4 consecutive columns (one float4 per row) of
// RP consecutive rows; CL = DVT/4 column lanes, RG = NT/CL row groups.  The
// reduction over rows is a wave shuffle across the row groups of a wave plus
// one LDS exchange across waves.
//
// With the q / k L2 normalisation (L2 = true) the same pass also sums k.k and
// q.q; with ik = 1/sqrt(k.k + eps) and iq likewise, the normalised rows give
// a = ik S'^T k, b = iq S'^T q, kq = ik iq k.q and the update S' + (ik k) delta^T,
// so the raw rows are never rescaled in memory.
#include "kda_common.h"
#include "kda_launch.h"

namespace kda {
namespace {

template <int D, int DVT>
struct RecCfg {
  // threads per workgroup: a whole 64 KiB state streams best with 512 threads
  static constexpr int NT = (D * DVT / 4) >= 4096 ? 512 : (D * DVT / 4) >= 1024 ? 256 : 64;
  static constexpr int CL = DVT / 4;                            // column lanes
  static constexpr int RG = NT / CL;                            // row groups
  static constexpr int RP = D / RG;                             // rows per thread
  static constexpr int NW = NT / 64;                            // waves
  static constexpr int NTILE = D / DVT;                         // column tiles per unit
  static constexpr int TG = 16;                                 // tokens staged per pass
  static_assert(RP >= 1 && RG * RP == D && CL * RG == NT && CL <= 64, "bad recurrent tiling");
};

struct RecArgs {
  const void* q;
  const void* k;
  const void* v;
  const float* log_g;
  const float* beta;
  const float* init_state;    // [N, H, D, D] or null (zeros)
  float* final_state;         // [N, H, D, D] or null; may equal init_state
  const int32_t* cu_seqlens;  // [N+1] or null (dense)
  void* out;                  // fp32, or bf16 when out_bf16
  float* deltas;              // per-token delta [.., H, dv] or null
  bool out_bf16;
  int num_units;              // N * H
  int T;                      // dense: tokens per sequence
  int H;
  float scale;
};

constexpr float L2_EPS = 1e-6f;  // eps inside the root of the q / k L2 normalisation

template <int D, int DVT, typename In, bool L2>
__global__ void __launch_bounds__((RecCfg<D, DVT>::NT)) recurrent_kernel(RecArgs a) {
  using C = RecCfg<D, DVT>;
  constexpr int CL = C::CL, RP = C::RP, NT = C::NT, NW = C::NW, TG = C::TG, NTILE = C::NTILE;
  constexpr int NR = L2 ? 11 : 9;  // reduced values per column lane: a[4], b[4], kq (+ kk, qq)

  __shared__ float s_k[TG][D];
  __shared__ float s_q[TG][D];
  __shared__ float s_a[TG][D];  // exp(log_g)
  __shared__ float s_beta[TG];
  __shared__ float s_red[2][NW][CL][NR];

  // blockIdx -> (unit, tile): the NTILE tiles of a unit sit 8 blocks apart so
  // they land on the same XCD (blocks are dealt to the 8 XCDs round-robin) and
  // share that XCD's L2 for the unit's q/k/log_g rows.
  int unit, tile;
  if (NTILE == 1) {
    unit = blockIdx.x;
    tile = 0;
  } else {
    const int grp = blockIdx.x / (8 * NTILE);
    const int rem = blockIdx.x - grp * 8 * NTILE;
    tile = rem / 8;
    unit = grp * 8 + (rem & 7);
  }
  if (unit >= a.num_units) return;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int cl = tid % CL;
  const int g = tid / CL;
  const int n = unit / a.H;
  const int h = unit - n * a.H;
  const int col = tile * DVT + 4 * cl;  // first of this thread's 4 value columns

  int tok0, ntok;
  if (a.cu_seqlens) {
    tok0 = a.cu_seqlens[n];
    ntok = a.cu_seqlens[n + 1] - tok0;
  } else {
    tok0 = n * a.T;
    ntok = a.T;
  }
  const In* q = static_cast<const In*>(a.q);
  const In* k = static_cast<const In*>(a.k);
  const In* v = static_cast<const In*>(a.v);
  const int H = a.H;

  // the state streams through once: nontemporal loads and stores
  float4 s[RP];
  if (a.init_state) {
    const float* S0 = a.init_state + static_cast<size_t>(unit) * D * D;
#pragma unroll
    for (int p = 0; p < RP; ++p) s[p] = load4_stream(S0 + (g * RP + p) * D + col);
  } else {
#pragma unroll
    for (int p = 0; p < RP; ++p) s[p] = make_float4(0.f, 0.f, 0.f, 0.f);
  }

  for (int t0 = 0; t0 < ntok; t0 += TG) {
    const int tg = min(TG, ntok - t0);
    __syncthreads();  // the previous pass is done with the staging buffers
    for (int idx = tid; idx < tg * D; idx += NT) {
      const int tt = idx / D, i = idx - tt * D;
      const size_t row = static_cast<size_t>(tok0 + t0 + tt) * H + h;
      s_k[tt][i] = to_f32(k[row * D + i]);
      s_q[tt][i] = to_f32(q[row * D + i]);
      s_a[tt][i] = exp_fast(a.log_g[row * D + i]);
    }
    if (tid < tg) s_beta[tid] = a.beta[static_cast<size_t>(tok0 + t0 + tid) * H + h];
    __syncthreads();

    for (int tt = 0; tt < tg; ++tt) {
      const size_t row = static_cast<size_t>(tok0 + t0 + tt) * H + h;
      const float4 vv = load4(v + row * D + col);
      const int par = (t0 + tt) & 1;
      float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
      float b0 = 0.f, b1 = 0.f, b2 = 0.f, b3 = 0.f, kq = 0.f, kk = 0.f, qq = 0.f;
#pragma unroll
      for (int p = 0; p < RP; ++p) {
        const int r = g * RP + p;
        const float al = s_a[tt][r], kr = s_k[tt][r], qr = s_q[tt][r];
        s[p].x *= al; s[p].y *= al; s[p].z *= al; s[p].w *= al;
        a0 += s[p].x * kr; a1 += s[p].y * kr; a2 += s[p].z * kr; a3 += s[p].w * kr;
        b0 += s[p].x * qr; b1 += s[p].y * qr; b2 += s[p].z * qr; b3 += s[p].w * qr;
        kq += kr * qr;
        if (L2) {
          kk += kr * kr;
          qq += qr * qr;
        }
      }
#pragma unroll
      for (int off = CL; off < 64; off <<= 1) {  // row groups within the wave
        a0 += __shfl_xor(a0, off); a1 += __shfl_xor(a1, off);
        a2 += __shfl_xor(a2, off); a3 += __shfl_xor(a3, off);
        b0 += __shfl_xor(b0, off); b1 += __shfl_xor(b1, off);
        b2 += __shfl_xor(b2, off); b3 += __shfl_xor(b3, off);
        kq += __shfl_xor(kq, off);
        if (L2) {
          kk += __shfl_xor(kk, off);
          qq += __shfl_xor(qq, off);
        }
      }
      if (lane < CL) {
        float* r = s_red[par][wave][cl];
        r[0] = a0; r[1] = a1; r[2] = a2; r[3] = a3;
        r[4] = b0; r[5] = b1; r[6] = b2; r[7] = b3; r[8] = kq;
        if (L2) {
          r[9] = kk;
          r[10] = qq;
        }
      }
      __syncthreads();
      float A[4] = {0.f, 0.f, 0.f, 0.f}, B[4] = {0.f, 0.f, 0.f, 0.f}, KQ = 0.f, KK = 0.f, QQ = 0.f;
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        const float* r = s_red[par][w][cl];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          A[c] += r[c];
          B[c] += r[4 + c];
        }
        KQ += r[8];
        if (L2) {
          KK += r[9];
          QQ += r[10];
        }
      }
      float ik = 1.f;  // 1 / |k_t| (normalised rows), else 1
      if (L2) {
        ik = __frsqrt_rn(KK + L2_EPS);
        const float iq = __frsqrt_rn(QQ + L2_EPS);
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          A[c] *= ik;
          B[c] *= iq;
        }
        KQ *= ik * iq;
      }
      const float bt = s_beta[tt];
      const float vj[4] = {vv.x, vv.y, vv.z, vv.w};
      float dl[4], o[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        dl[c] = bt * (vj[c] - A[c]);
        o[c] = a.scale * (B[c] + dl[c] * KQ);
      }
      if (g == 0) {
        if (a.out_bf16)
          store_out4(static_cast<bf16_t*>(a.out) + row * D + col, o[0], o[1], o[2], o[3]);
        else
          store_out4(static_cast<float*>(a.out) + row * D + col, o[0], o[1], o[2], o[3]);
        if (a.deltas) *reinterpret_cast<float4*>(a.deltas + row * D + col) = make_float4(dl[0], dl[1], dl[2], dl[3]);
      }
#pragma unroll
      for (int p = 0; p < RP; ++p) {
        const float kr = s_k[tt][g * RP + p] * ik;
        s[p].x += kr * dl[0]; s[p].y += kr * dl[1]; s[p].z += kr * dl[2]; s[p].w += kr * dl[3];
      }
    }
  }

  if (a.final_state) {
    float* S1 = a.final_state + static_cast<size_t>(unit) * D * D;
#pragma unroll
    for (int p = 0; p < RP; ++p) store4_stream(S1 + (g * RP + p) * D + col, s[p]);
  }
}


// Commit of accepted rows: sequence n's state advances by its first accept[n]
// rows with the delta of each row already known (saved by the rows pass), so
// each row is only the state update of the recurrence above,
// S' = Diag(exp(log_g_t)) S + k_t delta_t^T, in the same order of operations.
// Nothing is reduced; the tile streams in and out once.
struct CommitArgs {
  const void* k;
  const float* log_g;
  const float* deltas;
  const int32_t* accept;
  float* state;
  int num_units;  // N * H
  int n_tok;
  int H;
};

template <int D, int DVT, typename In, bool L2>
__global__ void __launch_bounds__((RecCfg<D, DVT>::NT)) commit_kernel(CommitArgs a) {
  using C = RecCfg<D, DVT>;
  constexpr int CL = C::CL, RP = C::RP, NT = C::NT, TG = C::TG, NTILE = C::NTILE;
  __shared__ float s_k[TG][D];
  __shared__ float s_a[TG][D];
  __shared__ float s_ik[TG];  // 1 / |k_t| of the normalised rows

  int unit, tile;
  if (NTILE == 1) {
    unit = blockIdx.x;
    tile = 0;
  } else {
    const int grp = blockIdx.x / (8 * NTILE);
    const int rem = blockIdx.x - grp * 8 * NTILE;
    tile = rem / 8;
    unit = grp * 8 + (rem & 7);
  }
  if (unit >= a.num_units) return;
  const int n = unit / a.H;
  const int h = unit - n * a.H;
  const int m = min(max(a.accept[n], 0), a.n_tok);
  if (m == 0) return;  // nothing accepted: the state stays as it is

  const int tid = threadIdx.x;
  const int cl = tid % CL;
  const int g = tid / CL;
  const int col = tile * DVT + 4 * cl;
  const int H = a.H;
  const In* k = static_cast<const In*>(a.k);
  float* S = a.state + static_cast<size_t>(unit) * D * D;

  float4 s[RP];
#pragma unroll
  for (int p = 0; p < RP; ++p) s[p] = load4_stream(S + (g * RP + p) * D + col);

  for (int t0 = 0; t0 < m; t0 += TG) {
    const int tg = min(TG, m - t0);
    __syncthreads();  // the previous pass is done with the staging buffers
    for (int idx = tid; idx < tg * D; idx += NT) {
      const int tt = idx / D, i = idx - tt * D;
      const size_t row = (static_cast<size_t>(n) * a.n_tok + t0 + tt) * H + h;
      s_k[tt][i] = to_f32(k[row * D + i]);
      s_a[tt][i] = exp_fast(a.log_g[row * D + i]);
    }
    __syncthreads();
    if (L2) {  // 16 lanes per staged row, D/16 channels each
      for (int idx = tid; idx < TG * 16; idx += NT) {
        const int tt = idx >> 4, part = idx & 15;
        float ss = 0.f;
#pragma unroll
        for (int c = 0; c < D / 16; ++c) {
          const float x = s_k[tt][part * (D / 16) + c];
          ss += x * x;
        }
#pragma unroll
        for (int o = 1; o < 16; o <<= 1) ss += __shfl_xor(ss, o);
        if (part == 0) s_ik[tt] = __frsqrt_rn(ss + L2_EPS);
      }
      __syncthreads();
    }
    for (int tt = 0; tt < tg; ++tt) {
      const size_t row = (static_cast<size_t>(n) * a.n_tok + t0 + tt) * H + h;
      const float4 dl = load4(a.deltas + row * D + col);
      const float ik = L2 ? s_ik[tt] : 1.f;
#pragma unroll
      for (int p = 0; p < RP; ++p) {
        const int r = g * RP + p;
        const float al = s_a[tt][r], kr = s_k[tt][r] * ik;
        s[p].x *= al; s[p].y *= al; s[p].z *= al; s[p].w *= al;
        s[p].x += kr * dl.x; s[p].y += kr * dl.y; s[p].z += kr * dl.z; s[p].w += kr * dl.w;
      }
    }
  }
#pragma unroll
  for (int p = 0; p < RP; ++p) store4_stream(S + (g * RP + p) * D + col, s[p]);
}

template <int D, typename In>
hipError_t launch_commit_d(const CommitArgs& a, bool l2, hipStream_t stream) {
  using C = RecCfg<D, D>;  // whole states: nothing is reduced, the tile only streams
  if (l2)
    hipLaunchKernelGGL((commit_kernel<D, D, In, true>), dim3(static_cast<unsigned>(a.num_units)), dim3(C::NT), 0,
                       stream, a);
  else
    hipLaunchKernelGGL((commit_kernel<D, D, In, false>), dim3(static_cast<unsigned>(a.num_units)), dim3(C::NT), 0,
                       stream, a);
  return hipGetLastError();
}

template <int D, int DVT, typename In>
hipError_t launch_rec(const RecArgs& a, bool l2, hipStream_t stream) {
  using C = RecCfg<D, DVT>;
  unsigned blocks = static_cast<unsigned>(a.num_units);
  if (C::NTILE > 1) blocks = ((blocks + 7) / 8) * 8 * C::NTILE;
  if (l2)
    hipLaunchKernelGGL((recurrent_kernel<D, DVT, In, true>), dim3(blocks), dim3(C::NT), 0, stream, a);
  else
    hipLaunchKernelGGL((recurrent_kernel<D, DVT, In, false>), dim3(blocks), dim3(C::NT), 0, stream, a);
  return hipGetLastError();
}

// Pick the value-column tile: split a unit when there are too few units to
// give every CU several workgroups, or when each unit carries several tokens
// (per-token reductions then dominate, and half-width tiles halve them).  A
// single-token unit (decode) keeps whole 64 KiB tiles, which stream best.
template <typename In>
hipError_t launch_rec_d(int d, const RecArgs& a, bool l2, hipStream_t stream) {
  const bool few = a.num_units < 1024;
  const bool multi = a.cu_seqlens != nullptr || a.T > 1;
  switch (d) {
    case 16: return launch_rec<16, 16, In>(a, l2, stream);
    case 32: return launch_rec<32, 32, In>(a, l2, stream);
    case 64: return few ? launch_rec<64, 32, In>(a, l2, stream) : launch_rec<64, 64, In>(a, l2, stream);
    case 128:
      if (a.num_units < 256) return launch_rec<128, 32, In>(a, l2, stream);
      return (few || multi) ? launch_rec<128, 64, In>(a, l2, stream) : launch_rec<128, 128, In>(a, l2, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_recurrent(const RecArgs& a, int d, bool bf16, bool l2, hipStream_t stream) {
  if (a.num_units == 0) return hipSuccess;
  return bf16 ? launch_rec_d<bf16_t>(d, a, l2, stream) : launch_rec_d<float>(d, a, l2, stream);
}

}  // namespace

hipError_t launch_step(const StepLaunch& s, hipStream_t stream) {
  if (s.n_tok == 0) return hipSuccess;
  RecArgs a{};
  a.q = s.q; a.k = s.k; a.v = s.v; a.log_g = s.log_g; a.beta = s.beta;
  a.init_state = s.state;
  // in place: every workgroup reads its tile before writing it; speculative
  // rows leave the state as it was
  a.final_state = s.keep_state ? nullptr : s.state;
  a.cu_seqlens = nullptr;
  a.out = s.out;
  a.out_bf16 = s.out_bf16;
  a.deltas = s.deltas;
  a.num_units = s.num_seqs * s.num_heads;
  a.T = s.n_tok;
  a.H = s.num_heads;
  a.scale = s.scale;
  return launch_recurrent(a, s.d, s.bf16, s.l2, stream);
}

hipError_t launch_commit(const CommitLaunch& c, hipStream_t stream) {
  if (c.num_seqs == 0) return hipSuccess;
  CommitArgs a{};
  a.k = c.k; a.log_g = c.log_g; a.deltas = c.deltas; a.accept = c.accept; a.state = c.state;
  a.num_units = c.num_seqs * c.num_heads;
  a.n_tok = c.n_tok;
  a.H = c.num_heads;
  const bool l2 = c.l2;
  switch (c.d) {
    case 16: return c.bf16 ? launch_commit_d<16, bf16_t>(a, l2, stream) : launch_commit_d<16, float>(a, l2, stream);
    case 32: return c.bf16 ? launch_commit_d<32, bf16_t>(a, l2, stream) : launch_commit_d<32, float>(a, l2, stream);
    case 64: return c.bf16 ? launch_commit_d<64, bf16_t>(a, l2, stream) : launch_commit_d<64, float>(a, l2, stream);
    case 128:
      return c.bf16 ? launch_commit_d<128, bf16_t>(a, l2, stream) : launch_commit_d<128, float>(a, l2, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_chunk_recurrent(const ChunkLaunch& c, hipStream_t stream) {
  RecArgs a{};
  a.q = c.q; a.k = c.k; a.v = c.v; a.log_g = c.log_g; a.beta = c.beta;
  a.init_state = c.init_state;
  a.final_state = c.final_state;
  a.cu_seqlens = c.cu_seqlens;
  a.out = c.out;
  a.out_bf16 = c.out_bf16;
  a.num_units = c.num_seqs * c.num_heads;
  a.T = c.seq_len;
  a.H = c.num_heads;
  a.scale = c.scale;
  return launch_recurrent(a, c.d, c.bf16, c.l2, stream);
}

}  // namespace kda
