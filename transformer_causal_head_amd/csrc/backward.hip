// Backward pass of prefill attention: dQ, dK, dV from the forward's inputs,
// its output O, the output gradient dO and the stored log-sum-exp.
//
// The weights are recomputed from the LSE instead of being stored (the
// textbook's FlashAttention section: on the backward pass the weight matrix
// is recomputed block by block).  With P_ij = exp(s_ij - LSE_i),
// s_ij = scale * q_i . k_j, and the softmax Jacobian p_i (delta_ij - p_j)
// (textbook, "Почему делить на корень из d_h"):
//     dV_j += P_ij dO_i
//     dP_ij = dO_i . v_j
//     dS_ij = P_ij (dP_ij - Delta_i),   Delta_i = sum_j P_ij dP_ij = dO_i . O_i
//     dQ_i  = scale * sum_j dS_ij k_j
//     dK_j += scale * sum_i dS_ij q_i
// summed over the query heads that share a K/V head (GQA/MQA).
//
// This file holds the Delta reduction and the general row kernels (one
// wavefront per dQ row or per dK/dV row, any head size up to 256, fp32 or
// bf16).  They are exact in fp32 arithmetic but not tuned; the bf16 MFMA
// kernels live in backward_bf16.hip.

#include <math.h>

#include "common.h"
#include "kernels.h"

namespace attn {

namespace {

struct BwdParams {
  const void* Q;
  const void* K;
  const void* V;
  const void* O;
  const void* dO;
  const float* LSE;
  float* delta;
  float* lse2;    // delta pass output (may be null): LSE * log2(e), +inf where LSE = -inf
  const uint64_t* kbits;  // key-padding mask (one bit per key, kwords words per sequence) or null
  int kwords;
  void* dQ;
  void* dK;
  void* dV;
  int B, Nq, Nkv, S, Dh;
  int causal, window;
  float scale;
};

// Delta_i = dO_i . O_i, one wavefront per (b, h, i) row.  With p.lse2 it
// also stores the row's LSE in log2 units for the MFMA kernels, with a row
// that saw no key (LSE = -inf, possible under a key-padding mask) mapped to
// +inf, so that the weights recomputed from it, 2^(s c - lse2), are 0 there
// instead of 2^(+inf).
template <typename T>
__global__ __launch_bounds__(256) void delta_kernel(BwdParams p) {
  const int lane = threadIdx.x & 63;
  const long long row = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= (long long)p.B * p.Nq * p.S) return;
  const T* O = static_cast<const T*>(p.O) + (size_t)row * p.Dh;
  const T* dO = static_cast<const T*>(p.dO) + (size_t)row * p.Dh;
  float acc = 0.f;
  for (int d = lane; d < p.Dh; d += 64) acc = __builtin_fmaf(to_float(O[d]), to_float(dO[d]), acc);
  acc = wave_sum(acc);
  if (lane == 0) {
    p.delta[row] = acc;
    if (p.lse2 != nullptr) {
      const float l = p.LSE[row];
      p.lse2[row] = l == -INFINITY ? INFINITY : l * kLog2e;
    }
  }
}

// key j of sequence b not hidden by the key-padding mask
__device__ __forceinline__ bool key_kept(const BwdParams& p, int b, int j) {
  return p.kbits == nullptr || ((p.kbits[(size_t)b * p.kwords + (j >> 6)] >> (j & 63)) & 1);
}

// visible keys of query i: [lo, hi)
__device__ __forceinline__ void key_range(const BwdParams& p, int i, int& lo, int& hi) {
  hi = p.causal ? i + 1 : p.S;
  lo = (p.causal && p.window > 0) ? max(0, i - p.window + 1) : 0;
}

// dQ row (b, h, i): loop over its visible keys.
template <typename T>
__global__ __launch_bounds__(256) void dq_rows_kernel(BwdParams p) {
  const int lane = threadIdx.x & 63;
  const long long row = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= (long long)p.B * p.Nq * p.S) return;
  const int i = (int)(row % p.S);
  const long long bh = row / p.S;
  const int h = (int)(bh % p.Nq);
  const int b = (int)(bh / p.Nq);
  const int g = h / (p.Nq / p.Nkv);
  const size_t qoff = (size_t)row * p.Dh;
  const size_t kvoff = ((size_t)b * p.Nkv + g) * (size_t)p.S * p.Dh;
  const T* Q = static_cast<const T*>(p.Q);
  const T* K = static_cast<const T*>(p.K);
  const T* V = static_cast<const T*>(p.V);
  const T* dO = static_cast<const T*>(p.dO);

  float q[4], go[4], acc[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int d = lane + 64 * u;
    q[u] = d < p.Dh ? to_float(Q[qoff + d]) : 0.f;
    go[u] = d < p.Dh ? to_float(dO[qoff + d]) : 0.f;
    acc[u] = 0.f;
  }
  const float lse = p.LSE[row];
  const float dlt = p.delta[row];
  int lo, hi;
  key_range(p, i, lo, hi);
  // a row that saw no key (LSE = -inf) has O = 0 and passes no gradient
  if (lse == -INFINITY) hi = lo;
  for (int j = lo; j < hi; ++j) {
    if (!key_kept(p, b, j)) continue;
    const size_t r = kvoff + (size_t)j * p.Dh;
    float sq = 0.f, sv = 0.f;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int d = lane + 64 * u;
      if (d < p.Dh) {
        sq = __builtin_fmaf(q[u], to_float(K[r + d]), sq);
        sv = __builtin_fmaf(go[u], to_float(V[r + d]), sv);
      }
    }
    sq = wave_sum(sq);
    sv = wave_sum(sv);
    const float pij = expf(sq * p.scale - lse);
    const float ds = pij * (sv - dlt);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int d = lane + 64 * u;
      if (d < p.Dh) acc[u] = __builtin_fmaf(ds, to_float(K[r + d]), acc[u]);
    }
  }
  T* dQ = static_cast<T*>(p.dQ);
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int d = lane + 64 * u;
    if (d < p.Dh) dQ[qoff + d] = from_float<T>(acc[u] * p.scale);
  }
}

// dK, dV row (b, g, j): loop over the query heads of group g and the queries
// that see key j.
template <typename T>
__global__ __launch_bounds__(256) void dkv_rows_kernel(BwdParams p) {
  const int lane = threadIdx.x & 63;
  const long long row = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= (long long)p.B * p.Nkv * p.S) return;
  const int j = (int)(row % p.S);
  const long long bg = row / p.S;
  const int g = (int)(bg % p.Nkv);
  const int b = (int)(bg / p.Nkv);
  const int G = p.Nq / p.Nkv;
  const size_t kvoff = (size_t)row * p.Dh;
  const T* Q = static_cast<const T*>(p.Q);
  const T* K = static_cast<const T*>(p.K);
  const T* V = static_cast<const T*>(p.V);
  const T* dO = static_cast<const T*>(p.dO);

  float k[4], v[4], dk[4], dv[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int d = lane + 64 * u;
    k[u] = d < p.Dh ? to_float(K[kvoff + d]) : 0.f;
    v[u] = d < p.Dh ? to_float(V[kvoff + d]) : 0.f;
    dk[u] = 0.f;
    dv[u] = 0.f;
  }
  // queries that see key j: i >= j (causal), i - j < window; none if the key
  // is padding
  const int i_lo = p.causal ? j : 0;
  const int i_hi = !key_kept(p, b, j) ? i_lo
                   : (p.causal && p.window > 0) ? min(p.S, j + p.window) : p.S;
  for (int hh = 0; hh < G; ++hh) {
    const int h = g * G + hh;
    const size_t qrow0 = ((size_t)b * p.Nq + h) * p.S;
    for (int i = i_lo; i < i_hi; ++i) {
      const size_t r = (qrow0 + i) * p.Dh;
      float sq = 0.f, sv = 0.f;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int d = lane + 64 * u;
        if (d < p.Dh) {
          sq = __builtin_fmaf(to_float(Q[r + d]), k[u], sq);
          sv = __builtin_fmaf(to_float(dO[r + d]), v[u], sv);
        }
      }
      sq = wave_sum(sq);
      sv = wave_sum(sv);
      const float pij = expf(sq * p.scale - p.LSE[qrow0 + i]);
      const float ds = pij * (sv - p.delta[qrow0 + i]);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int d = lane + 64 * u;
        if (d < p.Dh) {
          dv[u] = __builtin_fmaf(pij, to_float(dO[r + d]), dv[u]);
          dk[u] = __builtin_fmaf(ds, to_float(Q[r + d]), dk[u]);
        }
      }
    }
  }
  T* dK = static_cast<T*>(p.dK);
  T* dV = static_cast<T*>(p.dV);
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int d = lane + 64 * u;
    if (d < p.Dh) {
      dK[kvoff + d] = from_float<T>(dk[u] * p.scale);
      dV[kvoff + d] = from_float<T>(dv[u]);
    }
  }
}

template <typename T>
hipError_t launch_general(const BwdParams& p, hipStream_t stream) {
  const long long qrows = (long long)p.B * p.Nq * p.S;
  const long long kvrows = (long long)p.B * p.Nkv * p.S;
  if ((qrows + 3) / 4 > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(delta_kernel<T>, dim3((unsigned)((qrows + 3) / 4)), dim3(256), 0, stream, p);
  hipLaunchKernelGGL(dq_rows_kernel<T>, dim3((unsigned)((qrows + 3) / 4)), dim3(256), 0, stream, p);
  hipLaunchKernelGGL(dkv_rows_kernel<T>, dim3((unsigned)((kvrows + 3) / 4)), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

// Delta, then the rows' LSE in log2 units (the MFMA kernels read both)
size_t backward_workspace(int B, int Nq, int S) { return 2 * (size_t)B * Nq * S * sizeof(float); }

hipError_t launch_backward_delta(const void* O, const void* dO, const float* LSE, float* delta,
                                 float* lse2, long long rows, int Dh, int is_bf16,
                                 hipStream_t stream) {
  BwdParams p{};
  p.O = O;
  p.dO = dO;
  p.LSE = LSE;
  p.delta = delta;
  p.lse2 = lse2;
  p.B = 1;
  p.Nq = 1;
  p.S = (int)rows;
  p.Dh = Dh;
  if ((rows + 3) / 4 > 0x7fffffffLL || rows > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  if (is_bf16)
    hipLaunchKernelGGL(delta_kernel<__bf16>, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL(delta_kernel<float>, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_backward_general(const void* Q, const void* K, const void* V, const void* O,
                                   const void* dO, const float* LSE, void* dQ, void* dK, void* dV,
                                   int B, int Nq, int Nkv, int S, int Dh, int causal, int window,
                                   float scale, void* ws, int is_bf16, const uint64_t* kbits,
                                   hipStream_t stream) {
  BwdParams p{};
  p.Q = Q;
  p.K = K;
  p.V = V;
  p.O = O;
  p.dO = dO;
  p.LSE = LSE;
  p.delta = static_cast<float*>(ws);
  p.dQ = dQ;
  p.dK = dK;
  p.dV = dV;
  p.B = B;
  p.Nq = Nq;
  p.Nkv = Nkv;
  p.S = S;
  p.Dh = Dh;
  p.causal = causal;
  p.window = window;
  p.scale = scale;
  p.kbits = kbits;
  p.kwords = key_mask_words(S);
  return is_bf16 ? launch_general<__bf16>(p, stream) : launch_general<float>(p, stream);
}

}  // namespace attn
