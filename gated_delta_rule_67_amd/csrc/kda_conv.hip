// kda_conv.hip -- short causal depthwise convolution feeding q, k and v (gfx950).
//
// NeMo glm5_next.layers, `_TorchShortConvolution`: a depthwise causal Conv1d
// over [batch, sequence, channels] that resets at packed boundaries; its width
// K is the config's linear_conv_kernel_dim.  For a document n, channel c and
// token t of n (counted from the document start):
//
//     y[t, c] = act( sum_{j<K} w[c, j] * xe[t - (K-1) + j, c] )
//
// where xe is the document's inputs preceded by its K-1 cached inputs
// (init_cache[n, c, :], oldest first, or zeros).  The cache after the
// document, final_cache[n, c, :], is the last K-1 entries of xe: the state a
// following call (decode) continues from.  act is the identity or SiLU.
//
// HBM-bound: one read of x and one write of y per element, plus a K-1 token
// halo per run.  One thread owns 8 channels (one 16-byte bf16 access per
// token) over a run of R tokens and keeps the K-1 previous inputs in
// registers; the run's tokens are loaded 8 at a time so that their loads are
// in flight together.
#include <algorithm>

#include "kda_common.h"
#include "kda_launch.h"
#include "kda_vec8.h"

namespace kda {
namespace {

constexpr int R = 32;      // tokens per thread
constexpr int NTC = 256;   // threads per workgroup
constexpr int UNR = 8;     // tokens loaded together

struct ConvArgs {
  const void* x;
  const float* w;            // [Cn, K]
  const int32_t* cu;         // packed [N+1], or null (dense)
  const float* init_cache;   // [N, Cn, K-1] or null (zeros)
  float* final_cache;        // [N, Cn, K-1] or null
  void* out;
  int64_t total;             // tokens in x
  int N;                     // sequences (dense) or documents (packed)
  int T;                     // dense: tokens per sequence
  int Cn;
  int act;                   // 0 identity, 1 SiLU
};

// document containing token t: [ds, de)
__device__ __forceinline__ void doc_of(const ConvArgs& a, int64_t t, int& n, int64_t& ds, int64_t& de) {
  if (a.cu == nullptr) {
    n = static_cast<int>(t / a.T);
    ds = static_cast<int64_t>(n) * a.T;
    de = ds + a.T;
    return;
  }
  int lo = 0, hi = a.N;  // last n with cu[n] <= t; then cu[n+1] > t
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (a.cu[mid] <= t) lo = mid;
    else hi = mid;
  }
  n = lo;
  ds = a.cu[n];
  de = a.cu[n + 1];
}

__device__ __forceinline__ int64_t doc_end(const ConvArgs& a, int n) {
  return a.cu ? static_cast<int64_t>(a.cu[n + 1]) : static_cast<int64_t>(n + 1) * a.T;
}

template <int K, typename In>
__global__ void __launch_bounds__(NTC) conv_kernel(ConvArgs a) {
  constexpr int M = K - 1, CH = 8;
  const int c = CH * (blockIdx.x * NTC + threadIdx.x);
  if (c >= a.Cn) return;
  const int64_t t0 = static_cast<int64_t>(blockIdx.y) * R;
  const int64_t t1 = min(t0 + R, a.total);
  if (t0 >= t1) return;
  const In* x = static_cast<const In*>(a.x);
  In* y = static_cast<In*>(a.out);
  const int Cn = a.Cn;

  float wr[CH][K];
#pragma unroll
  for (int ch = 0; ch < CH; ++ch)
#pragma unroll
    for (int j = 0; j < K; ++j) wr[ch][j] = a.w[(c + ch) * K + j];

  int n;
  int64_t ds, de;
  doc_of(a, t0, n, ds, de);
  float win[M > 0 ? M : 1][CH];
  // the window of token t of document n: the M inputs before it, from the
  // document itself or (before its start) from its cache
  auto fill = [&](int64_t t) {
#pragma unroll
    for (int m = 0; m < M; ++m) {
      const int64_t tau = t - M + m;
      if (tau >= ds) {
        load8f(x + tau * Cn + c, win[m]);
      } else if (a.init_cache) {
        const int p = static_cast<int>(tau - ds) + M;
        const float* cc = a.init_cache + (static_cast<size_t>(n) * Cn + c) * M + p;
#pragma unroll
        for (int ch = 0; ch < CH; ++ch) win[m][ch] = cc[ch * M];
      } else {
#pragma unroll
        for (int ch = 0; ch < CH; ++ch) win[m][ch] = 0.f;
      }
    }
  };
  fill(t0);
  // the run in segments that stay inside one document; the window is
  // refilled only between segments, so the token loop issues no loads but
  // the next tokens' own
  int64_t t = t0;
  while (true) {
    const int64_t te = min(t1, de);
    for (int64_t tb = t; tb < te; tb += UNR) {
      // unconditional loads (past te they repeat token te-1 and go unused):
      // a load under a branch would wait for its data before the next issues
      float xv[UNR][CH];
#pragma unroll
      for (int u = 0; u < UNR; ++u) load8f(x + min(tb + u, te - 1) * Cn + c, xv[u]);
#pragma unroll
      for (int u = 0; u < UNR; ++u) {
        if (tb + u >= te) break;
        float o[CH];
#pragma unroll
        for (int ch = 0; ch < CH; ++ch) {
          float acc = wr[ch][M] * xv[u][ch];
#pragma unroll
          for (int m = 0; m < M; ++m) acc += wr[ch][m] * win[m][ch];
          if (a.act == 1) acc = acc / (1.f + exp_fast(-acc));
          o[ch] = acc;
        }
        store8f(y + (tb + u) * Cn + c, o);
#pragma unroll
        for (int m = 0; m + 1 < M; ++m)
#pragma unroll
          for (int ch = 0; ch < CH; ++ch) win[m][ch] = win[m + 1][ch];
        if constexpr (M > 0) {
#pragma unroll
          for (int ch = 0; ch < CH; ++ch) win[M - 1][ch] = xv[u][ch];
        }
      }
    }
    if (te == de && a.final_cache) {  // the document ends in this run
      float* fc = a.final_cache + (static_cast<size_t>(n) * Cn + c) * M;
#pragma unroll
      for (int ch = 0; ch < CH; ++ch)
#pragma unroll
        for (int m = 0; m < M; ++m) fc[ch * M + m] = win[m][ch];
    }
    if (te >= t1) break;
    t = te;  // the next non-empty document starts at t
    do {
      ++n;
      ds = de;
      de = doc_end(a, n);
    } while (t >= de);
    fill(t);
  }
}

// Documents without tokens: their final cache is their initial cache.
__global__ void __launch_bounds__(NTC) conv_empty_kernel(ConvArgs a, int M) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * NTC + threadIdx.x;  // (document, channel)
  if (i >= static_cast<int64_t>(a.N) * a.Cn) return;
  const int n = static_cast<int>(i / a.Cn);
  const int64_t len = a.cu ? static_cast<int64_t>(a.cu[n + 1]) - a.cu[n] : a.T;
  if (len != 0) return;
  for (int m = 0; m < M; ++m) a.final_cache[i * M + m] = a.init_cache ? a.init_cache[i * M + m] : 0.f;
}

template <int K, typename In>
hipError_t launch_k(const ConvArgs& a, hipStream_t stream) {
  const dim3 grid(static_cast<unsigned>((a.Cn / 8 + NTC - 1) / NTC), static_cast<unsigned>((a.total + R - 1) / R));
  hipLaunchKernelGGL((conv_kernel<K, In>), grid, dim3(NTC), 0, stream, a);
  return hipGetLastError();
}

template <typename In>
hipError_t launch_in(int K, const ConvArgs& a, hipStream_t stream) {
  switch (K) {
    case 1: return launch_k<1, In>(a, stream);
    case 2: return launch_k<2, In>(a, stream);
    case 3: return launch_k<3, In>(a, stream);
    case 4: return launch_k<4, In>(a, stream);
    case 5: return launch_k<5, In>(a, stream);
    case 6: return launch_k<6, In>(a, stream);
    case 7: return launch_k<7, In>(a, stream);
    case 8: return launch_k<8, In>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_short_conv(const ConvLaunch& s, hipStream_t stream) {
  ConvArgs a{};
  a.x = s.x;
  a.w = s.weight;
  a.cu = s.cu_seqlens;
  a.init_cache = s.init_cache;
  a.final_cache = s.final_cache;
  a.out = s.out;
  a.N = s.num_seqs;
  a.T = s.seq_len;
  a.total = s.cu_seqlens ? static_cast<int64_t>(s.seq_len) : static_cast<int64_t>(s.num_seqs) * s.seq_len;
  a.Cn = s.channels;
  a.act = s.activation;
  if (a.total > 0) {
    const hipError_t e = s.bf16 ? launch_in<bf16_t>(s.kernel_size, a, stream) : launch_in<float>(s.kernel_size, a, stream);
    if (e != hipSuccess) return e;
  }
  // documents without tokens: packed ones, or every sequence of a dense T = 0
  if (s.final_cache && s.kernel_size > 1 && a.N > 0 && (s.cu_seqlens != nullptr || s.seq_len == 0)) {
    const int64_t items = static_cast<int64_t>(a.N) * a.Cn;
    hipLaunchKernelGGL(conv_empty_kernel, dim3(static_cast<unsigned>((items + NTC - 1) / NTC)), dim3(NTC), 0, stream, a,
                       s.kernel_size - 1);
    return hipGetLastError();
  }
  return hipSuccess;
}

}  // namespace kda
