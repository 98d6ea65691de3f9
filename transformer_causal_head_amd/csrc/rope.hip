// Rotary position embedding (RoPE) of queries and keys, and the KV-cache
// append that rotates the keys on their way into the cache.
//
// The textbook's attention chapter ("Как в attention попадает позиция", and
// step 4 of "Прямой проход по шагам") rotates q and k by a position-dependent
// angle so that their dot product depends only on the offset i - j; V is not
// rotated, and K is stored in the cache after the rotation (the layer-cache
// section), so a key is rotated once, when it is appended.  The formula is
// RoFormer's (Su et al., which the page cites): pair m of a head vector is
// turned by p * theta_m, theta_m = base^(-2m/Dh), as (a, b) ->
// (a cos - b sin, a sin + b cos).  Pairs are (x[2m], x[2m+1]) in the "pairs"
// layout (RoFormer's) or (x[m], x[m + Dh/2]) in the "half" layout
// (GPT-NeoX, LLaMA checkpoints in the Hugging Face format).
//
// The angles come from a [P, Dh] fp32 table (cos in columns 0 .. Dh/2 - 1,
// sin in Dh/2 .. Dh - 1) built once per (P, Dh, base) in double precision
// and rounded once to fp32, so that the rotation's accuracy does not depend
// on how large the position is.  The rotation itself is fp32 (two fmas per
// element) and rounds to the tensor's element type once.
//
// Both rotating kernels are streaming, HBM-bound copies: each thread turns
// PP pairs of one row (16-byte vector loads when the row allows it), and rows
// are enumerated with the head index fastest, so the heads of one token read
// the same table row back to back (it stays in L2).

#include <math.h>

#include "common.h"
#include "kernels.h"


namespace attn {

namespace {

__global__ __launch_bounds__(256) void rope_table_kernel(float* table, int P, int Dh, double base) {
  const int half = Dh / 2;
  const long long idx = (long long)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (long long)P * half) return;
  const int p = (int)(idx / half);
  const int m = (int)(idx % half);
  const double theta = pow(base, -2.0 * m / Dh);
  double s, c;
  sincos((double)p * theta, &s, &c);
  table[(size_t)p * Dh + m] = (float)c;
  table[(size_t)p * Dh + half + m] = (float)s;
}

// N consecutive elements (N * sizeof(T) bytes, 16-byte aligned when VEC) widened to fp32
template <typename T, int N, bool VEC, bool NT = false>
__device__ __forceinline__ void load_row(const T* src, float (&dst)[N]) {
  if constexpr (VEC) {
    constexpr int E = 16 / sizeof(T);
    static_assert(N % E == 0, "whole 16-byte chunks");
#pragma unroll
    for (int c = 0; c < N / E; ++c) {
      const u32x4* a = reinterpret_cast<const u32x4*>(src) + c;
      const u32x4 w = NT ? __builtin_nontemporal_load(a) : *a;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        if constexpr (sizeof(T) == 2)
          dst[c * E + e] = (e & 1) ? bf16_hi(w[e / 2]) : bf16_lo(w[e / 2]);
        else
          dst[c * E + e] = __uint_as_float(w[e]);
      }
    }
  } else {
#pragma unroll
    for (int e = 0; e < N; ++e) dst[e] = to_float(src[e]);
  }
}

template <typename T, int N, bool VEC, bool NT = false>
__device__ __forceinline__ void store_row(T* dst, const float (&src)[N]) {
  if constexpr (VEC) {
    constexpr int E = 16 / sizeof(T);
#pragma unroll
    for (int c = 0; c < N / E; ++c) {
      u32x4 w;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if constexpr (sizeof(T) == 2)
          w[e] = pack_bf16x2(src[c * E + 2 * e], src[c * E + 2 * e + 1]);
        else
          w[e] = __float_as_uint(src[c * E + e]);
      }
      if constexpr (NT)
        __builtin_nontemporal_store(w, reinterpret_cast<u32x4*>(dst) + c);
      else
        reinterpret_cast<u32x4*>(dst)[c] = w;
    }
  } else {
#pragma unroll
    for (int e = 0; e < N; ++e) dst[e] = from_float<T>(src[e]);
  }
}

// Rotate thread j's PP pairs of one row (tpr threads per row): x -> y (y may
// be x), with the cos / sin row cs of its position.
template <typename T, int PP, int STYLE, bool VEC>
__device__ __forceinline__ void rotate_pairs(const T* x, T* y, const float* cs, int half, int j,
                                             int tpr) {
  // rows of X / Y (read once, written once) bypass the caches' retention with
  // non-temporal accesses; the table rows, reread by every head, do not
  constexpr bool NTX = VEC;
  if constexpr (STYLE == 0 && VEC) {
    // pairs layout, 16-byte vectors: a chunk of E elements holds CP whole
    // pairs; thread j takes chunks j, j + tpr, ..., so that every load
    // instruction of the wavefront reads consecutive chunks of a row
    constexpr int E = 16 / sizeof(T);
    constexpr int CP = E / 2;
#pragma unroll
    for (int u = 0; u < PP / CP; ++u) {
      const int ch = j + u * tpr;
      float v[E], c[CP], s[CP];
      load_row<T, E, true, NTX>(x + ch * E, v);
      load_row<float, CP, CP % 4 == 0>(cs + ch * CP, c);
      load_row<float, CP, CP % 4 == 0>(cs + half + ch * CP, s);
#pragma unroll
      for (int k = 0; k < CP; ++k) {
        const float a = v[2 * k], b = v[2 * k + 1];
        v[2 * k] = __builtin_fmaf(a, c[k], -b * s[k]);
        v[2 * k + 1] = __builtin_fmaf(a, s[k], b * c[k]);
      }
      store_row<T, E, true, NTX>(y + ch * E, v);
    }
    return;
  }
  const int m0 = j * PP;
  float c[PP], s[PP];
  load_row<float, PP, VEC>(cs + m0, c);
  load_row<float, PP, VEC>(cs + half + m0, s);
  if constexpr (STYLE == 0) {  // pairs (x[2m], x[2m+1]): 2 * PP consecutive elements
    float v[2 * PP];
    load_row<T, 2 * PP, VEC, NTX>(x + 2 * m0, v);
#pragma unroll
    for (int k = 0; k < PP; ++k) {
      const float a = v[2 * k], b = v[2 * k + 1];
      v[2 * k] = __builtin_fmaf(a, c[k], -b * s[k]);
      v[2 * k + 1] = __builtin_fmaf(a, s[k], b * c[k]);
    }
    store_row<T, 2 * PP, VEC, NTX>(y + 2 * m0, v);
  } else {  // halves (x[m], x[m + half])
    float va[PP], vb[PP];
    load_row<T, PP, VEC, NTX>(x + m0, va);
    load_row<T, PP, VEC, NTX>(x + half + m0, vb);
#pragma unroll
    for (int k = 0; k < PP; ++k) {
      const float a = va[k], b = vb[k];
      va[k] = __builtin_fmaf(a, c[k], -b * s[k]);
      vb[k] = __builtin_fmaf(a, s[k], b * c[k]);
    }
    store_row<T, PP, VEC, NTX>(y + m0, va);
    store_row<T, PP, VEC, NTX>(y + half + m0, vb);
  }
}

__device__ __forceinline__ int clamp_pos(int p, int P) { return min(max(p, 0), P - 1); }

struct RopeParams {
  const void* X;
  void* Y;
  const int32_t* positions;  // [B, S] or null
  const int32_t* start;      // [B] (position of row 0) or null (0)
  const float* table;
  int P, B, H, S, Dh;
  long long n_rows;  // B * S * H
};

// thread -> (row, pair group); rows (b, s, h) with h fastest
template <typename T, int PP, int STYLE, bool VEC>
__global__ __launch_bounds__(256) void rope_kernel(RopeParams p) {
  const int half = p.Dh / 2;
  const int tpr = half / PP;
  const long long t = (long long)blockIdx.x * 256 + threadIdx.x;
  const long long item = t / tpr;
  if (item >= p.n_rows) return;
  const int j = (int)(t % tpr);
  const int h = (int)(item % p.H);
  const long long bs = item / p.H;
  const int s = (int)(bs % p.S);
  const int b = (int)(bs / p.S);
  const int pos = p.positions ? p.positions[(size_t)b * p.S + s] : (p.start ? p.start[b] : 0) + s;
  const float* cs = p.table + (size_t)clamp_pos(pos, p.P) * p.Dh;
  const size_t row = (((size_t)b * p.H + h) * p.S + s) * p.Dh;
  rotate_pairs<T, PP, STYLE, VEC>(static_cast<const T*>(p.X) + row, static_cast<T*>(p.Y) + row,
                                  cs, half, j, tpr);
}

struct AppendRopeParams {
  const void* Knew;
  const void* Vnew;
  void* Kc;
  void* Vc;
  const int32_t* pos;        // [B] slot / position of each sequence's first new row
  const int32_t* positions;  // [B, Snew] rotation positions, or null (pos[b] + i)
  const float* table;
  int P, B, Nkv, Snew, Tcap, Dh, rolling;
  int first;                 // first new row written (rolling appends longer than Tcap)
  long long n_rows;          // B * (Snew - first) * Nkv
};

// K rows rotated into the cache, V rows copied; same thread map as rope_kernel
template <typename T, int PP, int STYLE, bool VEC>
__global__ __launch_bounds__(256) void kv_append_rope_kernel(AppendRopeParams p) {
  const int half = p.Dh / 2;
  const int tpr = half / PP;
  const long long t = (long long)blockIdx.x * 256 + threadIdx.x;
  const long long item = t / tpr;
  if (item >= p.n_rows) return;
  const int j = (int)(t % tpr);
  const int rows = p.Snew - p.first;
  const int g = (int)(item % p.Nkv);
  const long long bi = item / p.Nkv;
  const int i = p.first + (int)(bi % rows);
  const int b = (int)(bi / rows);
  const long long p0 = p.pos[b];
  if (p0 < 0) return;
  long long slot = p0 + i;
  if (p.rolling) {
    slot %= p.Tcap;
  } else if (slot >= p.Tcap) {
    return;
  }
  const long long rp = p.positions ? (long long)p.positions[(size_t)b * p.Snew + i] : p0 + i;
  const int rpos = (int)min(max(rp, 0LL), (long long)p.P - 1);
  const size_t src = (((size_t)b * p.Nkv + g) * p.Snew + i) * p.Dh;
  const size_t dst = (((size_t)b * p.Nkv + g) * p.Tcap + (size_t)slot) * p.Dh;
  rotate_pairs<T, PP, STYLE, VEC>(static_cast<const T*>(p.Knew) + src, static_cast<T*>(p.Kc) + dst,
                                  p.table + (size_t)rpos * p.Dh, half, j, tpr);
  // V: this thread's share of the row (2 * PP elements), unchanged; with
  // vectors, thread j copies chunks j, j + tpr, ... as in the pairs layout
  const T* vs = static_cast<const T*>(p.Vnew) + src;
  T* vd = static_cast<T*>(p.Vc) + dst;
  if constexpr (VEC) {
    constexpr int E = 16 / sizeof(T);
#pragma unroll
    for (int u = 0; u < 2 * PP / E; ++u) {
      const int ch = j + u * tpr;
      float v[E];
      load_row<T, E, true>(vs + ch * E, v);
      store_row<T, E, true>(vd + ch * E, v);
    }
  } else {
    float v[2 * PP];
    load_row<T, 2 * PP, false>(vs + 2 * j * PP, v);
    store_row<T, 2 * PP, false>(vd + 2 * j * PP, v);
  }
}

// pairs per thread: 8 with 16-byte vectors when every segment a thread
// touches is 16-byte aligned (head size a multiple of 16, aligned buffers),
// else 1 with element accesses
bool vec_ok(int Dh, uintptr_t align) { return Dh % 16 == 0 && align % 16 == 0; }

hipError_t grid_for(long long n_rows, int Dh, bool vec, unsigned& blocks) {
  const long long threads = n_rows * (Dh / 2 / (vec ? 8 : 1));
  const long long nb = (threads + 255) / 256;
  if (nb > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  blocks = (unsigned)nb;
  return hipSuccess;
}

template <typename T, int STYLE>
hipError_t rope_typed(const RopeParams& p, bool vec, hipStream_t stream) {
  unsigned blocks;
  if (grid_for(p.n_rows, p.Dh, vec, blocks) != hipSuccess) return hipErrorInvalidConfiguration;
  if (blocks == 0) return hipSuccess;
  if (vec)
    hipLaunchKernelGGL((rope_kernel<T, 8, STYLE, true>), dim3(blocks), dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL((rope_kernel<T, 1, STYLE, false>), dim3(blocks), dim3(256), 0, stream, p);
  return hipGetLastError();
}

template <typename T, int STYLE>
hipError_t append_typed(const AppendRopeParams& p, bool vec, hipStream_t stream) {
  unsigned blocks;
  if (grid_for(p.n_rows, p.Dh, vec, blocks) != hipSuccess) return hipErrorInvalidConfiguration;
  if (blocks == 0) return hipSuccess;
  if (vec)
    hipLaunchKernelGGL((kv_append_rope_kernel<T, 8, STYLE, true>), dim3(blocks), dim3(256), 0,
                       stream, p);
  else
    hipLaunchKernelGGL((kv_append_rope_kernel<T, 1, STYLE, false>), dim3(blocks), dim3(256), 0,
                       stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_rope_table(float* table, int P, int Dh, double base, hipStream_t stream) {
  const long long n = (long long)P * (Dh / 2);
  const long long blocks = (n + 255) / 256;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(rope_table_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, table, P, Dh,
                     base);
  return hipGetLastError();
}

hipError_t launch_rope(const void* X, void* Y, const int32_t* positions, const int32_t* start,
                       const float* table, int P, int B, int H, int S, int Dh, int style,
                       int elem_bytes, hipStream_t stream) {
  RopeParams p;
  p.X = X;
  p.Y = Y;
  p.positions = positions;
  p.start = start;
  p.table = table;
  p.P = P;
  p.B = B;
  p.H = H;
  p.S = S;
  p.Dh = Dh;
  p.n_rows = (long long)B * S * H;
  const bool vec = vec_ok(Dh, (uintptr_t)X | (uintptr_t)Y | (uintptr_t)table);
  if (elem_bytes == 2)
    return style ? rope_typed<__bf16, 1>(p, vec, stream) : rope_typed<__bf16, 0>(p, vec, stream);
  return style ? rope_typed<float, 1>(p, vec, stream) : rope_typed<float, 0>(p, vec, stream);
}

hipError_t launch_kv_append_rope(const void* Knew, const void* Vnew, void* Kc, void* Vc,
                                 const int32_t* pos, const int32_t* positions, const float* table,
                                 int P, int B, int Nkv, int Snew, int Dh, int Tcap, int rolling,
                                 int style, int elem_bytes, hipStream_t stream) {
  AppendRopeParams p;
  p.Knew = Knew;
  p.Vnew = Vnew;
  p.Kc = Kc;
  p.Vc = Vc;
  p.pos = pos;
  p.positions = positions;
  p.table = table;
  p.P = P;
  p.B = B;
  p.Nkv = Nkv;
  p.Snew = Snew;
  p.Tcap = Tcap;
  p.Dh = Dh;
  p.rolling = rolling;
  p.first = (rolling && Snew > Tcap) ? Snew - Tcap : 0;
  p.n_rows = (long long)B * (Snew - p.first) * Nkv;
  const bool vec = vec_ok(Dh, (uintptr_t)Knew | (uintptr_t)Vnew | (uintptr_t)Kc | (uintptr_t)Vc |
                                  (uintptr_t)table);
  if (elem_bytes == 2)
    return style ? append_typed<__bf16, 1>(p, vec, stream) : append_typed<__bf16, 0>(p, vec, stream);
  return style ? append_typed<float, 1>(p, vec, stream) : append_typed<float, 0>(p, vec, stream);
}

}  // namespace attn
