// kda_fallback.h -- exact fp32 token-by-token evaluation of one 64-token chunk
// on a 32-column state tile, for the chunks the MFMA fast path cannot take.
//
// The tile lives in MFMA accumulator layout across the NWAVE waves of the
// workgroup, each owning NA = 8 / NWAVE blocks of 16 key rows:
// s[a][b][e] = S[16 NA w + 16a + 4lg + e][col0 + 16b + lc] (w = wave,
// lane = 16lg + lc).  Per token (GLM-5.3-Flash model notes,
// Glm5NextTextLinearAttention snippet): decay the key rows, read back S^T k,
// form delta = beta (v - S^T k), add k delta^T; the output is read from the
// updated state through S_new^T q = S_decayed^T q + delta (k . q).
// With the q / k L2 normalisation the staged k and q rows are divided by
// sqrt(sum of squares + eps) before the walk.  Outputs are fp32, or rounded
// once to bf16.
#pragma once

#include "kda_common.h"

namespace kda {
namespace fb {

constexpr int C = 64;     // chunk length
constexpr int D = 128;    // head dim
constexpr int DVT = 32;   // state columns per workgroup
constexpr int TG = 16;    // tokens staged per pass

template <int NWAVE>
struct Stage {
  float a[TG][D];
  float k[TG][D];
  float q[TG][D];
  float v[TG][DVT];
  float beta[TG];
  float kq[TG];
  float ik[TG];   // 1/|k| and 1/|q| of the staged rows (L2 normalisation)
  float iq[TG];
  float red[2][NWAVE][DVT][2];
};

struct Args {
  const bf16_t* q;
  const bf16_t* k;
  const bf16_t* v;
  const float* log_g;
  const float* beta;
  void* out;       // fp32, or bf16 when out_bf16
  int H;
  float scale;
  bool out_bf16;
  bool l2;         // L2-normalise the q and k rows
};

// Chunk ck of the document whose tokens start at tok_begin (ntok tokens), head
// h, state columns col0 .. col0+31.  Writes the chunk's outputs to p.out and
// advances s.  The NWAVE waves of the workgroup run it together (it
// synchronises the whole workgroup internally, so every thread of the
// workgroup must call it the same number of times).
template <int NWAVE>
__device__ __forceinline__ void eval_chunk(Stage<NWAVE>& st, f32x4 (&s)[8 / NWAVE][2], const Args& p,
                                           size_t tok_begin, int ntok, int ck, int h, int col0) {
  constexpr int NT = 64 * NWAVE;
  constexpr int NA = 8 / NWAVE;
  const int tid = static_cast<int>(threadIdx.x), lane = tid & 63, lc = lane & 15, lg = lane >> 4;
  const int cw = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, uniform (SGPR)
  const int H = p.H;
  const int nv = min(C, ntok - ck * C);
  const size_t tok0 = tok_begin + static_cast<size_t>(ck) * C;
  for (int t0 = 0; t0 < nv; t0 += TG) {
    const int tg = min(TG, nv - t0);
    lds_barrier();
    {
      constexpr int PER = TG * D / NT;
      static_assert(TG * D % NT == 0 && TG * DVT % NT == 0, "fallback staging split");
      float la[PER], lk[PER], lq[PER];
#pragma unroll
      for (int x = 0; x < PER; ++x) {
        const int idx = tid + x * NT, r = min(idx / D, tg - 1), c = idx % D;
        const size_t row = (tok0 + t0 + r) * H + h;
        la[x] = p.log_g[row * D + c];
        lk[x] = to_f32(p.k[row * D + c]);
        lq[x] = to_f32(p.q[row * D + c]);
      }
      constexpr int PV = TG * DVT / NT;
      float vv[PV];
#pragma unroll
      for (int x = 0; x < PV; ++x) {
        const int idx = tid + x * NT, vr = idx / DVT, vcol = idx % DVT;
        vv[x] = to_f32(p.v[((tok0 + t0 + min(vr, tg - 1)) * H + h) * D + col0 + vcol]);
      }
      const float bb = p.beta[(tok0 + t0 + min(tid & (TG - 1), tg - 1)) * H + h];
#pragma unroll
      for (int x = 0; x < PER; ++x) {
        const int idx = tid + x * NT, r = idx / D, c = idx % D;
        st.a[r][c] = exp_fast(la[x]);
        st.k[r][c] = lk[x];
        st.q[r][c] = lq[x];
      }
#pragma unroll
      for (int x = 0; x < PV; ++x) {
        const int idx = tid + x * NT;
        st.v[idx / DVT][idx % DVT] = vv[x];
      }
      if (tid < TG) st.beta[tid] = bb;
    }
    lds_barrier();
    {  // kq[r] = k_r . q_r (and k.k, q.q): 16 lanes per token, 8 channels each
      if (tid < 16 * TG) {
        const int r = tid >> 4, cc = (tid & 15) * 8;
        float acc = 0.f, kk = 0.f, qq = 0.f;
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          acc += st.k[r][cc + c] * st.q[r][cc + c];
          kk += st.k[r][cc + c] * st.k[r][cc + c];
          qq += st.q[r][cc + c] * st.q[r][cc + c];
        }
#pragma unroll
        for (int o = 1; o < 16; o <<= 1) {
          acc += __shfl_xor(acc, o);
          kk += __shfl_xor(kk, o);
          qq += __shfl_xor(qq, o);
        }
        const float ik = p.l2 ? __frsqrt_rn(kk + 1e-6f) : 1.f;
        const float iq = p.l2 ? __frsqrt_rn(qq + 1e-6f) : 1.f;
        if ((tid & 15) == 0) {
          st.kq[r] = acc * ik * iq;
          st.ik[r] = ik;
          st.iq[r] = iq;
        }
      }
    }
    lds_barrier();
    if (p.l2) {  // the staged rows normalised in place
      constexpr int PER = TG * D / NT;
#pragma unroll
      for (int x = 0; x < PER; ++x) {
        const int idx = tid + x * NT, r = idx / D, c = idx % D;
        st.k[r][c] *= st.ik[r];
        st.q[r][c] *= st.iq[r];
      }
      lds_barrier();
    }
    for (int r = 0; r < tg; ++r) {
      const int par = (t0 + r) & 1;
      {
        float pa[2] = {0.f, 0.f}, pb[2] = {0.f, 0.f};
#pragma unroll
        for (int a = 0; a < NA; ++a)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int c = 16 * NA * cw + 16 * a + 4 * lg + e;
            const float al = st.a[r][c], kc = st.k[r][c], qc = st.q[r][c];
#pragma unroll
            for (int b = 0; b < 2; ++b) {
              s[a][b][e] *= al;
              pa[b] += s[a][b][e] * kc;
              pb[b] += s[a][b][e] * qc;
            }
          }
#pragma unroll
        for (int b = 0; b < 2; ++b) {
          pa[b] += __shfl_xor(pa[b], 16);
          pa[b] += __shfl_xor(pa[b], 32);
          pb[b] += __shfl_xor(pb[b], 16);
          pb[b] += __shfl_xor(pb[b], 32);
        }
        if (lg == 0) {
#pragma unroll
          for (int b = 0; b < 2; ++b) {
            st.red[par][cw][16 * b + lc][0] = pa[b];
            st.red[par][cw][16 * b + lc][1] = pb[b];
          }
        }
      }
      lds_barrier();
      {
        const float bt = st.beta[r], kq = st.kq[r];
        float dl[2];
#pragma unroll
        for (int b = 0; b < 2; ++b) {
          const int n = 16 * b + lc;
          float A = 0.f, B = 0.f;
#pragma unroll
          for (int x = 0; x < NWAVE; ++x) {
            A += st.red[par][x][n][0];
            B += st.red[par][x][n][1];
          }
          dl[b] = bt * (st.v[r][n] - A);
          if (cw == 0 && lg == 0) {
            const float o = p.scale * (B + dl[b] * kq);
            const size_t oi = ((tok0 + t0 + r) * H + h) * D + col0 + n;
            if (p.out_bf16)
              reinterpret_cast<__bf16*>(p.out)[oi] = static_cast<__bf16>(o);
            else
              static_cast<float*>(p.out)[oi] = o;
          }
        }
#pragma unroll
        for (int a = 0; a < NA; ++a)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float kc = st.k[r][16 * NA * cw + 16 * a + 4 * lg + e];
#pragma unroll
            for (int b = 0; b < 2; ++b) s[a][b][e] += kc * dl[b];
          }
      }
    }
  }
}

}  // namespace fb
}  // namespace kda
