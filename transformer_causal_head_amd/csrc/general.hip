// General attention row kernel: one wavefront computes one output row with a
// streaming (running max, running sum) softmax.  It covers fp32 inputs, head
// sizes other than 128, and decode shapes the MFMA kernels do not take.  It
// is correct for every supported shape but not tuned: each key costs a
// wavefront-wide dot-product reduction.
//
// Definition followed: softmax(q K^T * scale + M) V for one query row
// (textbook attention chapter, "Scaled dot-product attention"), with the
// causal / window visibility of sections "Маскирование" and "Скользящее окно"
// (visible iff j <= i and i - j < window).  Query row i of a head sits at
// position i in a plain prefill, and at position n - S + i when S rows are
// the newest tokens of a cache of n keys (chunked prefill; a decode step is
// the case S = 1, whose query sees every cached key -- section
// "Prefill и decode").

#include <math.h>

#include "common.h"
#include "kernels.h"

namespace attn {

namespace {

struct RowParams {
  const void* Q;
  const void* K;
  const void* V;
  void* O;
  float* LSE;
  int B, Nq, Nkv, S, Dh, kv_rows;  // S: query rows per head
  const int32_t* lens;              // keys per sequence in a cache, or null
  const uint64_t* kbits;            // key-padding mask bits (kwords per sequence), or null
  int kwords;
  int causal, window;
  float scale;
  long long n_rows;
  RopeQ rope;  // query rotation at load (RoPE); table == nullptr: none
};

template <typename T>
__global__ __launch_bounds__(256) void rows_kernel(RowParams p) {
  const int lane = threadIdx.x & 63;
  const long long row = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= p.n_rows) return;

  const T* Q = static_cast<const T*>(p.Q);
  const T* K = static_cast<const T*>(p.K);
  const T* V = static_cast<const T*>(p.V);
  T* O = static_cast<T*>(p.O);
  const int G = p.Nq / p.Nkv;

  // row (b, h, i); n keys; query position pos; visible keys [lo, hi)
  const int i = (int)(row % p.S);
  const long long bh = row / p.S;
  const int h = (int)(bh % p.Nq);
  const int b = (int)(bh / p.Nq);
  const int n = p.lens ? max(0, min(p.lens[b], p.kv_rows)) : p.S;
  const int pos = p.lens ? n - p.S + i : i;
  const int hi = p.causal ? min(pos + 1, n) : n;
  const int lo = (p.causal && p.window > 0) ? max(0, pos - p.window + 1) : 0;
  const int g = h / G;
  const size_t qoff = (size_t)row * p.Dh;
  const size_t kvoff = ((size_t)b * p.Nkv + g) * (size_t)p.kv_rows * p.Dh;

  float q[4], o[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int d = lane + 64 * u;
    q[u] = d < p.Dh ? to_float(Q[qoff + d]) : 0.f;
    o[u] = 0.f;
  }
  if (p.rope.table != nullptr) {
    // RoPE at load: element d pairs with d ^ 1 (pairs layout) or d +- Dh/2
    // (halves); the partner is read again from Q, the rotated value rounded
    // to the input type as a separate rotation pass would store it
    const int half = p.Dh / 2;
    const int rpos = p.rope.positions ? p.rope.positions[(size_t)b * p.S + i]
                   : p.rope.start ? p.rope.start[b] + i
                   : (p.S == 1 && p.lens ? n - 1 : pos);
    const float* cs = p.rope.table + (size_t)min(max(rpos, 0), p.rope.P - 1) * p.Dh;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int d = lane + 64 * u;
      if (d < p.Dh) {
        const bool first = p.rope.style == 0 ? (d & 1) == 0 : d < half;
        const int e = p.rope.style == 0 ? (d ^ 1) : (first ? d + half : d - half);
        const int m = p.rope.style == 0 ? d / 2 : (first ? d : d - half);
        const float c = cs[m], s = cs[half + m];
        const float x = q[u], y = to_float(Q[qoff + e]);
        const float r = first ? __builtin_fmaf(x, c, -y * s) : __builtin_fmaf(y, s, x * c);
        q[u] = to_float(from_float<T>(r));
      }
    }
  }
  float m = -INFINITY, l = 0.f;
  const uint64_t* kw = p.kbits ? p.kbits + (size_t)b * p.kwords : nullptr;
  for (int j = lo; j < hi; ++j) {
    if (kw && !((kw[j >> 6] >> (j & 63)) & 1)) continue;  // padding key (uniform branch)
    const size_t r = kvoff + (size_t)j * p.Dh;
    float part = 0.f;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int d = lane + 64 * u;
      if (d < p.Dh) part = __builtin_fmaf(q[u], to_float(K[r + d]), part);
    }
    const float s = wave_sum(part) * p.scale;
    const float m_new = fmaxf(m, s);
    const float alpha = expf(m - m_new);  // m = -inf on the first key -> 0
    const float e = expf(s - m_new);
    l = l * alpha + e;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int d = lane + 64 * u;
      const float v = d < p.Dh ? to_float(V[r + d]) : 0.f;
      o[u] = __builtin_fmaf(e, v, o[u] * alpha);
    }
    m = m_new;
  }
  // no visible key leaves l = 0: the row becomes 0/0 = NaN (decode length
  // below 1), or O = 0 and LSE = -inf when a key-padding mask hid every key
  const float inv = (kw && l == 0.f) ? 0.f : 1.f / l;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int d = lane + 64 * u;
    if (d < p.Dh) O[qoff + d] = from_float<T>(o[u] * inv);
  }
  if (p.LSE != nullptr && lane == 0) p.LSE[row] = m + logf(l);
}

}  // namespace

hipError_t launch_rows_general(const void* Q, const void* K, const void* V, void* O,
                               float* LSE, int B, int Nq, int Nkv, int S, int Dh,
                               int kv_rows, const int32_t* lens, const uint64_t* kbits,
                               int causal, int window, float scale, int is_bf16,
                               hipStream_t stream, const RopeQ* rope) {
  RowParams p;
  p.Q = Q;
  p.K = K;
  p.V = V;
  p.O = O;
  p.LSE = LSE;
  p.B = B;
  p.Nq = Nq;
  p.Nkv = Nkv;
  p.S = S;
  p.Dh = Dh;
  p.kv_rows = kv_rows;
  p.lens = lens;
  p.kbits = kbits;
  p.kwords = key_mask_words(kv_rows);
  p.causal = causal;
  p.window = window;
  p.scale = scale;
  p.n_rows = (long long)B * Nq * S;
  p.rope = rope ? *rope : RopeQ{nullptr, 0, nullptr, nullptr, 0};
  const long long nblocks = (p.n_rows + 3) / 4;
  if (nblocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  if (is_bf16)
    hipLaunchKernelGGL(rows_kernel<__bf16>, dim3((unsigned)nblocks), dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL(rows_kernel<float>, dim3((unsigned)nblocks), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace attn
