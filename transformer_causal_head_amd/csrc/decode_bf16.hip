// KV-cache decode step, bf16 cache, head size 128, split over the key axis.
//
// The step is one query row per sequence against its cached keys (textbook
// attention chapter, "KV-кэш" and "Prefill и decode": a 1 x t score row;
// decode is bound by reading the cache).  The key axis of every (sequence,
// K/V head) is cut into chunks of kDecodeChunk keys; each chunk yields a
// partial (running max m, running sum l, unnormalised output o) for the G
// query heads that share the K/V head, and a second kernel merges the
// partials with the same rescaling identity the online softmax uses
// (the Chinese post's Flash Attention section: rescale by exp(m_old - m_new)).
//
// gfx950 design
//   * Chunks past a sequence's length exit at once, so the work follows the
//     ragged lengths and fills the chip (thousands of workgroups).
//   * K rows stream straight from HBM into MFMA B operands
//     (v_mfma_f32_16x16x32_bf16, query heads on the M axis); every K byte is
//     read once per K/V head and shared by its G query heads.
//   * The probabilities go through a per-wave LDS slot and the PV update is
//     a VALU FMA stream over 16-byte V loads (8 head-dims per lane, 4 keys
//     per wavefront instruction), so V is read row-major and coalesced.
//   * Rows at or beyond the length are never read: loads clamp to the last
//     valid row and those keys get probability 0.

#include "common.h"
#include "kernels.h"

namespace attn {

namespace {

constexpr int D = 128;
constexpr int CH = kDecodeChunk;   // keys per workgroup
constexpr int WKEYS = CH / 4;      // keys per wave
constexpr int STEP = 64;           // keys per inner step

struct DecParams {
  const __bf16* q;
  const __bf16* K;
  const __bf16* V;
  const int32_t* lens;
  __bf16* O;
  float* LSE;
  float* ws_o;    // [B, Nkv, n_chunks, G, D] unnormalised partial outputs
  float* ws_ml;   // [B, Nkv, n_chunks, G, 2]  (m in log2 units, l)
  int B, Nq, Nkv, Tcap, n_chunks;
  float c;        // scale * log2(e)
};

__device__ __forceinline__ void wave_sync_lds() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <int G>
__global__ __launch_bounds__(256) void decode_partial_kernel(DecParams p) {
  static_assert(G >= 1 && G <= 8, "query heads per K/V head");
  __shared__ float pbuf[4][STEP][G];
  __shared__ float abuf[4][G];
  __shared__ float ob[4][G][D];
  __shared__ float mlb[4][G][2];

  const int chunk = blockIdx.x;
  const int g = blockIdx.y;
  const int b = blockIdx.z;
  const int n = min(p.lens[b], p.Tcap);
  if (chunk * CH >= n) return;

  const int tid = threadIdx.x;
  const int w = tid >> 6;
  const int lane = tid & 63;
  const int l16 = lane & 15;
  const int grp = lane >> 4;

  const size_t kv_base = ((size_t)b * p.Nkv + g) * (size_t)p.Tcap * D;

  // A operand: q[head = l16][d = 32*ks + 8*grp + i], zero rows past G
  bf16x8 qa[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    if (l16 < G) {
      const __bf16* src = p.q + ((size_t)b * p.Nq + (size_t)g * G + l16) * D + ks * 32 + grp * 8;
      qa[ks] = *reinterpret_cast<const bf16x8*>(src);
    } else {
      qa[ks] = bf16x8{};
    }
  }

  // running stats of head hh = 4*grp + r (valid for hh < G), replicated over
  // the 16 lanes of the group
  float m_run[4], l_run[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    m_run[r] = -INFINITY;
    l_run[r] = 0.f;
  }
  float o[G][8];
#pragma unroll
  for (int hh = 0; hh < G; ++hh)
#pragma unroll
    for (int e = 0; e < 8; ++e) o[hh][e] = 0.f;

  const int wk0 = chunk * CH + w * WKEYS;
  for (int s = 0; s < WKEYS / STEP; ++s) {
    const int k0 = wk0 + s * STEP;
    if (k0 >= n) break;

    // scores S[head][key] for 4 groups of 16 keys
    f32x4 acc[4];
#pragma unroll
    for (int kg = 0; kg < 4; ++kg) {
      const int key = min(k0 + kg * 16 + l16, n - 1);
      const __bf16* src = p.K + kv_base + (size_t)key * D + grp * 8;
      acc[kg] = f32x4{};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        bf16x8 kb = *reinterpret_cast<const bf16x8*>(src + ks * 32);
        acc[kg] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[ks], kb, acc[kg], 0, 0, 0);
      }
    }
    // acc[kg][r] at lane (grp, l16): head 4*grp + r, key k0 + 16*kg + l16
#pragma unroll
    for (int kg = 0; kg < 4; ++kg)
      if (k0 + kg * 16 + l16 >= n) acc[kg] = f32x4{-INFINITY, -INFINITY, -INFINITY, -INFINITY};

#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float mx = fmaxf(fmaxf(acc[0][r], acc[1][r]), fmaxf(acc[2][r], acc[3][r]));
#pragma unroll
      for (int off = 8; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off, 64));
      const float m_new = fmaxf(m_run[r], mx * p.c);
      const float alpha = exp2_fast(m_run[r] - m_new);  // k0 < n: m_new is finite
      m_run[r] = m_new;
      float rs = 0.f;
#pragma unroll
      for (int kg = 0; kg < 4; ++kg) {
        const float e = exp2_fast(__builtin_fmaf(acc[kg][r], p.c, -m_new));
        acc[kg][r] = e;
        rs += e;
      }
      l_run[r] = l_run[r] * alpha + rs;
      const int hh = grp * 4 + r;
      if (hh < G) {
#pragma unroll
        for (int kg = 0; kg < 4; ++kg) pbuf[w][kg * 16 + l16][hh] = acc[kg][r];
        if (l16 == 0) abuf[w][hh] = alpha;
      }
    }
    wave_sync_lds();

    // PV: lane (grp, l16) takes keys k0 + 4*t + grp and head-dims 8*l16 .. +7
    float al[G];
#pragma unroll
    for (int hh = 0; hh < G; ++hh) al[hh] = abuf[w][hh];
#pragma unroll
    for (int hh = 0; hh < G; ++hh)
#pragma unroll
      for (int e = 0; e < 8; ++e) o[hh][e] *= al[hh];
#pragma unroll 4
    for (int t = 0; t < STEP / 4; ++t) {
      const int kl = t * 4 + grp;
      const int key = min(k0 + kl, n - 1);
      const u32x4 vv = *reinterpret_cast<const u32x4*>(p.V + kv_base + (size_t)key * D + l16 * 8);
      float vf[8];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        vf[2 * j] = bf16_lo(vv[j]);
        vf[2 * j + 1] = bf16_hi(vv[j]);
      }
#pragma unroll
      for (int hh = 0; hh < G; ++hh) {
        const float pr = pbuf[w][kl][hh];
#pragma unroll
        for (int e = 0; e < 8; ++e) o[hh][e] = __builtin_fmaf(pr, vf[e], o[hh][e]);
      }
    }
    wave_sync_lds();
  }

  // reduce the wave: o over the 4 key subsets, l over the 16 lanes of a group
#pragma unroll
  for (int hh = 0; hh < G; ++hh)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float v = o[hh][e];
      v += __shfl_xor(v, 16, 64);
      v += __shfl_xor(v, 32, 64);
      o[hh][e] = v;
    }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    float v = l_run[r];
#pragma unroll
    for (int off = 8; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
    l_run[r] = v;
  }
  if (grp == 0) {
#pragma unroll
    for (int hh = 0; hh < G; ++hh)
#pragma unroll
      for (int e = 0; e < 8; ++e) ob[w][hh][l16 * 8 + e] = o[hh][e];
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int hh = grp * 4 + r;
    if (hh < G && l16 == 0) {
      mlb[w][hh][0] = m_run[r];
      mlb[w][hh][1] = l_run[r];
    }
  }
  __syncthreads();

  // combine the 4 waves and write the chunk's partial
  const size_t part = (((size_t)b * p.Nkv + g) * p.n_chunks + chunk) * G;
  for (int idx = tid; idx < G * D; idx += 256) {
    const int hh = idx / D;
    const int d = idx % D;
    float M = -INFINITY;
#pragma unroll
    for (int ww = 0; ww < 4; ++ww) M = fmaxf(M, mlb[ww][hh][0]);
    float acc_o = 0.f, acc_l = 0.f;
#pragma unroll
    for (int ww = 0; ww < 4; ++ww) {
      const float f = exp2_fast(mlb[ww][hh][0] - M);  // idle wave: m = -inf -> 0
      acc_o = __builtin_fmaf(f, ob[ww][hh][d], acc_o);
      acc_l = __builtin_fmaf(f, mlb[ww][hh][1], acc_l);
    }
    p.ws_o[(part + hh) * D + d] = acc_o;
    if (d == 0) {
      p.ws_ml[(part + hh) * 2 + 0] = M;
      p.ws_ml[(part + hh) * 2 + 1] = acc_l;
    }
  }
}

// One wavefront per (sequence, query head): merge the chunk partials.
__global__ __launch_bounds__(256) void decode_merge_kernel(DecParams p) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= p.B * p.Nq) return;
  const int b = row / p.Nq;
  const int h = row % p.Nq;
  const int G = p.Nq / p.Nkv;
  const int g = h / G;
  const int hh = h % G;
  const int n = min(p.lens[b], p.Tcap);
  const int nc = n > 0 ? (n + CH - 1) / CH : 0;

  float M = -INFINITY;
  for (int c = 0; c < nc; ++c) {
    const size_t part = (((size_t)b * p.Nkv + g) * p.n_chunks + c) * G + hh;
    M = fmaxf(M, p.ws_ml[part * 2]);
  }
  float L = 0.f, o0 = 0.f, o1 = 0.f;
  for (int c = 0; c < nc; ++c) {
    const size_t part = (((size_t)b * p.Nkv + g) * p.n_chunks + c) * G + hh;
    const float f = exp2_fast(p.ws_ml[part * 2] - M);
    L = __builtin_fmaf(f, p.ws_ml[part * 2 + 1], L);
    const f32x2 ov = *reinterpret_cast<const f32x2*>(p.ws_o + part * D + lane * 2);
    o0 = __builtin_fmaf(f, ov[0], o0);
    o1 = __builtin_fmaf(f, ov[1], o1);
  }
  const float inv = 1.f / L;  // n < 1 leaves L = 0: NaN row
  *reinterpret_cast<uint32_t*>(p.O + (size_t)row * D + lane * 2) = pack_bf16x2(o0 * inv, o1 * inv);
  if (p.LSE != nullptr && lane == 0) p.LSE[row] = (M + __log2f(L)) * kLn2;
}

}  // namespace

bool decode_bf16_d128_supported(int Nq, int Nkv) {
  const int G = Nq / Nkv;
  return G == 1 || G == 2 || G == 4 || G == 8;
}

size_t decode_bf16_d128_workspace(int B, int Nq, int Nkv, int Tcap) {
  const size_t n_chunks = ((size_t)Tcap + CH - 1) / CH;
  const size_t parts = (size_t)B * Nq * n_chunks;  // B * Nkv * n_chunks * G
  return parts * D * sizeof(float) + parts * 2 * sizeof(float);
}

hipError_t launch_decode_bf16_d128(const void* q, const void* Kc, const void* Vc,
                                   const int32_t* lens, void* O, float* LSE, int B, int Nq,
                                   int Nkv, int Tcap, void* ws, hipStream_t stream) {
  DecParams p;
  p.q = static_cast<const __bf16*>(q);
  p.K = static_cast<const __bf16*>(Kc);
  p.V = static_cast<const __bf16*>(Vc);
  p.lens = lens;
  p.O = static_cast<__bf16*>(O);
  p.LSE = LSE;
  p.B = B;
  p.Nq = Nq;
  p.Nkv = Nkv;
  p.Tcap = Tcap;
  p.n_chunks = (Tcap + CH - 1) / CH;
  const size_t parts = (size_t)B * Nq * p.n_chunks;
  p.ws_o = static_cast<float*>(ws);
  p.ws_ml = p.ws_o + parts * D;
  p.c = kLog2e / sqrtf((float)D);
  const dim3 grid(p.n_chunks, Nkv, B);
  switch (Nq / Nkv) {
    case 1: hipLaunchKernelGGL(decode_partial_kernel<1>, grid, dim3(256), 0, stream, p); break;
    case 2: hipLaunchKernelGGL(decode_partial_kernel<2>, grid, dim3(256), 0, stream, p); break;
    case 4: hipLaunchKernelGGL(decode_partial_kernel<4>, grid, dim3(256), 0, stream, p); break;
    case 8: hipLaunchKernelGGL(decode_partial_kernel<8>, grid, dim3(256), 0, stream, p); break;
    default: return hipErrorInvalidValue;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int rows = B * Nq;
  hipLaunchKernelGGL(decode_merge_kernel, dim3((rows + 3) / 4), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace attn
