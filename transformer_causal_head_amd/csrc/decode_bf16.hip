// KV-cache decode step, bf16 cache, head size 128, split over the key axis.
//
// The step is one query row per sequence against its cached keys (textbook
// attention chapter, "KV-кэш" and "Prefill и decode": a 1 x t score row;
// decode is bound by reading the cache).  With a window the query sees only
// the last `window` keys (section "Скользящее окно", i - j < window); chunks
// wholly before that range do nothing.  The key axis of every (sequence,
// K/V head) is cut into chunks; each chunk yields a partial (running max m,
// running sum l, unnormalised output o) for the G query heads that share the
// K/V head, and a second kernel merges the partials with the same rescaling
// identity the online softmax uses (the Chinese post's Flash Attention
// section: rescale by exp(m_old - m_new)).
//
// gfx950 design
//   * One wavefront per (sequence, K/V head, chunk); chunks past a sequence's
//     length exit at once, so the work follows the ragged lengths.
//   * The chunk length is chosen on the host: as long as the grid still has
//     thousands of work items (long chunks mean fewer partials and longer
//     sequential streams), and never a power of two: chunks whose starts sit
//     on 128 KB multiples made concurrently running waves collide in the
//     memory system and cost ~10% of the bandwidth.
//   * The chunk streams in steps of 32 keys.  K and V rows are both copied
//     HBM -> LDS by the DMA path (global_load_lds_dwordx4) with the
//     non-temporal hint: each copy instruction moves 4 whole 256-byte rows,
//     i.e. 1 KB of contiguous memory, and nothing is staged in VGPRs.
//     Loading K straight into MFMA operand registers instead touches 16 rows
//     x 64 bytes per instruction and tops out ~12% lower.
//   * Two LDS stages per tensor; the copies for step s + 2 are issued as soon
//     as step s has read its stage, so two steps (32 KB) stay in flight per
//     wave.  The step loop is unrolled by two so every stage is a distinct LDS
//     object and every wait count is a compile-time constant.
//   * Both products run on v_mfma_f32_16x16x32_bf16 in the transposed form of
//     the prefill kernel: S^T = K q^T (keys on M, the G query heads on N), and
//     O^T = V^T P^T, whose B operand is the S^T accumulator layout.  K is read
//     from LDS in operand layout (a row-XOR swizzle keeps the 16-row reads
//     conflict free); V is transposed on its way out by ds_read_b64_tr_b16.
//   * Every K and V byte is read once per K/V head and shared by its G query
//     heads.  Rows at or past the length are never used: copy addresses clamp
//     to the last valid row and those keys get probability 0.

#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace attn {

namespace {

constexpr int D = 128;
constexpr int STEP = 32;             // keys per pipeline step
constexpr int STAGE = STEP * D * 2;  // bytes of K (or V) per step
constexpr float TAU = 8.f;
constexpr int kNonTemporal = 2;      // cache-policy bit of the copy instructions

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) char lds_char;
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) const i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) const bf16x8 lds_bf16x8;

struct DecParams {
  const __bf16* q;
  const __bf16* K;
  const __bf16* V;
  const int32_t* lens;
  __bf16* O;
  float* LSE;
  float* ws_o;    // [B, Nkv, n_slots, G, D] unnormalised partial outputs
  float* ws_ml;   // [B, Nkv, n_slots, G, 2]  (m in log2 units, l)
  int B, Nq, Nkv, G, Tcap;
  int n_slots;    // chunks that can hold visible keys, per (sequence, K/V head)
  int ch;         // keys per chunk (a multiple of STEP)
  int window;     // > 0: only keys lens[b] - window .. lens[b] - 1 are visible
  float c;        // scale * log2(e)
};

// 16-byte chunk c of V row r sits at chunk position c ^ vswz(r) (keeps the
// transposing reads conflict free); chunk c of K row r at c ^ (r & 15) (the
// operand reads take one chunk of 16 consecutive rows).
__device__ __forceinline__ int vswz(int r) { return ((r << 1) & 14) | ((r >> 3) & 1); }
__device__ __forceinline__ int kswz(int r) { return r & 15; }

// Rows [k0, k0+32) of one head -> one LDS stage: 8 copies of 4 whole rows,
// lane i of a copy lands at byte 16*i of its 1 KB piece.  Rows past `last`
// are clamped to it.
template <bool IS_K>
__device__ __forceinline__ void load_rows(const __bf16* head, int k0, int last, lds_char* stage,
                                          int lane) {
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int r = j * 4 + (lane >> 4);
    const int c = (lane & 15) ^ (IS_K ? kswz(r) : vswz(r));
    const int row = min(k0 + r, last);
    __builtin_amdgcn_global_load_lds(head + (size_t)row * D + c * 8,
                                     (lds_void*)(stage + j * 1024), 16, 0, kNonTemporal);
  }
}

// s_waitcnt vmcnt(N) with the other counters left alone (gfx9 encoding:
// vmcnt bits [3:0] and [15:14], expcnt [6:4] = 7, lgkmcnt [11:8] = 15)
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt(((N >> 4) << 14) | 0x0F70 | (N & 15));
}

__global__ __launch_bounds__(64) void decode_partial_kernel(DecParams p) {
  // four separate LDS objects, so the compiler can tell that a copy into one
  // stage never aliases the reads of another
  __shared__ __attribute__((aligned(1024))) char k0s[STAGE];
  __shared__ __attribute__((aligned(1024))) char k1s[STAGE];
  __shared__ __attribute__((aligned(1024))) char v0s[STAGE];
  __shared__ __attribute__((aligned(1024))) char v1s[STAGE];

  lds_char* const K0 = (lds_char*)k0s;
  lds_char* const K1 = (lds_char*)k1s;
  lds_char* const V0 = (lds_char*)v0s;
  lds_char* const V1 = (lds_char*)v1s;

  const int g = blockIdx.y;
  const int b = blockIdx.z;
  const int n = min(p.lens[b], p.Tcap);
  const int lo = p.window > 0 ? max(0, n - p.window) : 0;  // first visible key
  // workgroup x takes the x-th chunk from the one holding key lo
  const int chunk = lo / p.ch + blockIdx.x;
  const int c0 = chunk * p.ch;
  if (c0 >= n) return;
  const int s0 = lo > c0 ? (lo - c0) / STEP : 0;  // first step holding a visible key
  const int nsteps = (min(p.ch, n - c0) + STEP - 1) / STEP;
  const int last = min(n, c0 + p.ch) - 1;

  const int lane = threadIdx.x;
  const int l16 = lane & 15;
  const int grp = lane >> 4;
  const int G = p.G;

  const size_t kvh = ((size_t)b * p.Nkv + g) * (size_t)p.Tcap * D;
  const __bf16* Kh = p.K + kvh;
  const __bf16* Vh = p.V + kvh;

  // q^T operand: lane (grp, l16) holds q[head g*G + l16][32*ks + 8*grp + i]
  bf16x8 qf[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    if (l16 < G) {
      const __bf16* src = p.q + ((size_t)b * p.Nq + (size_t)g * G + l16) * D + ks * 32 + grp * 8;
      qf[ks] = *reinterpret_cast<const bf16x8*>(src);
    } else {
      qf[ks] = bf16x8{};
    }
  }

  // copies in flight, oldest first: q, then K(0), V(0), K(1), V(1).  A step's
  // copies are 16 vector-memory instructions, so vmcnt(16) before step s means
  // step s has landed while step s + 1 is still in flight.  Copies are issued
  // for two steps past the chunk's end too (all rows clamp to its last row
  // and mostly hit L2), so that count holds on every path and the compiler
  // adds no full drain of its own.
  load_rows<true>(Kh, c0 + s0 * STEP, last, K0, lane);
  load_rows<false>(Vh, c0 + s0 * STEP, last, V0, lane);
  load_rows<true>(Kh, c0 + (s0 + 1) * STEP, last, K1, lane);
  load_rows<false>(Vh, c0 + (s0 + 1) * STEP, last, V1, lane);

  // transposing-read offsets: A operand of O^T += V^T P^T, d = 16*db + l16,
  // keys 4*grp + i (first read) and 16 + 4*grp + i (second read)
  int voff[2][8];
  {
    const int ip = l16 >> 2, u = l16 & 3;
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      const int r = 16 * hf + 4 * grp + ip;
#pragma unroll
      for (int db = 0; db < 8; ++db)
        voff[hf][db] = r * 256 + (((2 * db + (u >> 1)) ^ vswz(r)) << 4) + (u & 1) * 8;
    }
  }
  // K operand offsets: row 16*kb + l16, 16-byte chunk 4*ks + grp
  int koff[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) koff[ks] = l16 * 256 + (((4 * ks + grp) ^ kswz(l16)) << 4);

  f32x4 o[8];
#pragma unroll
  for (int db = 0; db < 8; ++db) o[db] = f32x4{};
  float m_run = -INFINITY, l_run = 0.f;

  auto step = [&](int s, const lds_char* kst, const lds_char* vst) {
    const int k0 = c0 + s * STEP;
    // S^T = K q^T; accumulator register r of block kb: key k0 + 16*kb + 4*grp + r,
    // query column l16
    f32x4 sc[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      sc[kb] = f32x4{};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const bf16x8 a = *(lds_bf16x8*)(kst + kb * 4096 + koff[ks]);
        sc[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qf[ks], sc[kb], 0, 0, 0);
      }
    }
    if (k0 + STEP > n || k0 < lo) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int key = k0 + kb * 16 + grp * 4 + r;
          if (key >= n || key < lo) sc[kb][r] = -INFINITY;
        }
    }
    float mx = fmaxf(fmaxf(fmaxf(sc[0][0], sc[0][1]), fmaxf(sc[0][2], sc[0][3])),
                     fmaxf(fmaxf(sc[1][0], sc[1][1]), fmaxf(sc[1][2], sc[1][3])));
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float m_cand = mx * p.c;  // every step run holds a visible key: finite
    if (__builtin_amdgcn_ballot_w64(m_cand > m_run + TAU)) {
      const float m_new = fmaxf(m_run, m_cand);
      const float alpha = exp2_fast(m_run - m_new);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < 8; ++db) o[db] *= alpha;
    }
    float rs = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float e = exp2_fast(__builtin_fmaf(sc[kb][r], p.c, -m_run));
        sc[kb][r] = e;
        rs += e;
      }
    l_run += rs;
    u32x4 pk;
    pk[0] = pack_bf16x2(sc[0][0], sc[0][1]);
    pk[1] = pack_bf16x2(sc[0][2], sc[0][3]);
    pk[2] = pack_bf16x2(sc[1][0], sc[1][1]);
    pk[3] = pack_bf16x2(sc[1][2], sc[1][3]);
    const bf16x8 pf = __builtin_bit_cast(bf16x8, pk);
#pragma unroll
    for (int db = 0; db < 8; ++db) {
      const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) i16x4*)(vst + voff[0][db]));
      const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) i16x4*)(vst + voff[1][db]));
      const bf16x8 a = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      o[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pf, o[db], 0, 0, 0);
    }
  };

  // Steps in pairs from s0: the first of a pair uses stage 0, the second stage
  // 1.  Before step s the copies of steps s and s + 1 are outstanding; once
  // step s has read its stage, the copies of step s + 2 go into it.
  for (int s = s0; s < nsteps; s += 2) {
    wait_vm<16>();
    step(s, K0, V0);
    load_rows<true>(Kh, c0 + (s + 2) * STEP, last, K0, lane);
    load_rows<false>(Vh, c0 + (s + 2) * STEP, last, V0, lane);
    wait_vm<16>();
    if (s + 1 < nsteps) step(s + 1, K1, V1);
    load_rows<true>(Kh, c0 + (s + 3) * STEP, last, K1, lane);
    load_rows<false>(Vh, c0 + (s + 3) * STEP, last, V1, lane);
  }
  wait_vm<0>();  // no copy may still target LDS when the wave ends

  // partial of this chunk: O^T register r of block db is d = 16*db + 4*grp + r
  // of query column l16
  l_run += __shfl_xor(l_run, 16, 64);
  l_run += __shfl_xor(l_run, 32, 64);
  if (l16 < G) {
    const size_t part = (((size_t)b * p.Nkv + g) * p.n_slots + blockIdx.x) * G + l16;
    float* dst = p.ws_o + part * D + 4 * grp;
#pragma unroll
    for (int db = 0; db < 8; ++db) *reinterpret_cast<f32x4*>(dst + 16 * db) = o[db];
    if (grp == 0) {
      p.ws_ml[part * 2 + 0] = m_run;
      p.ws_ml[part * 2 + 1] = l_run;
    }
  }
}

// One wavefront per (sequence, query head): merge the chunk partials.  Lanes
// first read the chunks' (m, l) side by side and reduce them across the
// wavefront; then each lane accumulates two head-dims over the chunks, with
// the chunk weights broadcast from the lane that computed them.
__global__ __launch_bounds__(256) void decode_merge_kernel(DecParams p) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= p.B * p.Nq) return;
  const int b = row / p.Nq;
  const int h = row % p.Nq;
  const int G = p.G;
  const int g = h / G;
  const int hh = h % G;
  const int n = min(p.lens[b], p.Tcap);
  const int nc = n > 0 ? (n + p.ch - 1) / p.ch : 0;
  // partial slot x holds chunk c_lo + x; chunks c_lo .. nc-1 wrote one
  const int c_lo = p.window > 0 ? max(0, n - p.window) / p.ch : 0;
  const size_t part0 = ((size_t)b * p.Nkv + g) * p.n_slots * G + hh;  // slot x: part0 + x*G

  float M = -INFINITY;
  const int ns = max(0, nc - c_lo);  // slots written
  for (int x = lane; x < ns; x += 64) M = fmaxf(M, p.ws_ml[(part0 + (size_t)x * G) * 2]);
  M = wave_max(M);
  float L = 0.f, o0 = 0.f, o1 = 0.f;
  for (int cb = 0; cb < ns; cb += 64) {
    // lane j of this batch holds slot cb + j's weight
    float wgt = 0.f;
    if (cb + lane < ns) {
      const size_t part = part0 + (size_t)(cb + lane) * G;
      wgt = exp2_fast(p.ws_ml[part * 2] - M);
      L = __builtin_fmaf(wgt, p.ws_ml[part * 2 + 1], L);
    }
    const int cnt = min(64, ns - cb);
    int j = 0;
    for (; j + 4 <= cnt; j += 4) {
      f32x2 ov[4];
      float wj[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        ov[u] = *reinterpret_cast<const f32x2*>(p.ws_o + (part0 + (size_t)(cb + j + u) * G) * D + lane * 2);
        wj[u] = __shfl(wgt, j + u, 64);
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        o0 = __builtin_fmaf(wj[u], ov[u][0], o0);
        o1 = __builtin_fmaf(wj[u], ov[u][1], o1);
      }
    }
    for (; j < cnt; ++j) {
      const f32x2 ov = *reinterpret_cast<const f32x2*>(p.ws_o + (part0 + (size_t)(cb + j) * G) * D + lane * 2);
      const float wj = __shfl(wgt, j, 64);
      o0 = __builtin_fmaf(wj, ov[0], o0);
      o1 = __builtin_fmaf(wj, ov[1], o1);
    }
  }
  L = wave_sum(L);
  const float inv = 1.f / L;  // n < 1 leaves L = 0: NaN row
  *reinterpret_cast<uint32_t*>(p.O + (size_t)row * D + lane * 2) = pack_bf16x2(o0 * inv, o1 * inv);
  if (p.LSE != nullptr && lane == 0) p.LSE[row] = (M + __log2f(L)) * kLn2;
}

}  // namespace

bool decode_bf16_d128_supported(int Nq, int Nkv) { return Nq / Nkv <= 16; }

// Keys per chunk: the longest candidate that still gives the grid at least
// 2048 (sequence, K/V head, chunk) items when every sequence has L visible
// keys (L = Tcap, or the window when it is shorter).  The candidates are
// multiples of 32 keys, none a power of two.
int decode_bf16_d128_chunk(int B, int Nkv, int L) {
  static const int kChunks[] = {1792, 1152, 896, 640, 384, 224, 160, 96};
  const long long heads = (long long)B * Nkv;
  for (int ch : kChunks)
    if (heads * ((L + ch - 1) / ch) >= 2048) return ch;
  return kChunks[sizeof(kChunks) / sizeof(kChunks[0]) - 1];
}

namespace {
// visible keys at most, chunk length, and partial slots per (sequence, K/V head)
struct DecodePlan {
  int ch, n_slots;
};
DecodePlan decode_plan(int B, int Nkv, int Tcap, int window) {
  const int L = (window > 0 && window < Tcap) ? window : Tcap;
  DecodePlan d;
  d.ch = decode_bf16_d128_chunk(B, Nkv, L);
  const int all = (Tcap + d.ch - 1) / d.ch;
  // a window of L keys starting anywhere touches at most ceil(L / ch) + 1 chunks
  d.n_slots = L < Tcap ? std::min(all, (L + d.ch - 1) / d.ch + 1) : all;
  return d;
}
}  // namespace

size_t decode_bf16_d128_workspace(int B, int Nq, int Nkv, int Tcap, int window) {
  const DecodePlan d = decode_plan(B, Nkv, Tcap, window);
  const size_t parts = (size_t)B * Nq * d.n_slots;  // B * Nkv * n_slots * G
  return parts * D * sizeof(float) + parts * 2 * sizeof(float);
}

hipError_t launch_decode_bf16_d128(const void* q, const void* Kc, const void* Vc,
                                   const int32_t* lens, void* O, float* LSE, int B, int Nq,
                                   int Nkv, int Tcap, int window, float scale, void* ws,
                                   hipStream_t stream) {
  const DecodePlan d = decode_plan(B, Nkv, Tcap, window);
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
  p.G = Nq / Nkv;
  p.Tcap = Tcap;
  p.ch = d.ch;
  p.n_slots = d.n_slots;
  const size_t parts = (size_t)B * Nq * p.n_slots;
  p.ws_o = static_cast<float*>(ws);
  p.ws_ml = p.ws_o + parts * D;
  p.window = window;
  p.c = kLog2e * scale;
  if (Nkv > 65535 || B > 65535) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(decode_partial_kernel, dim3(p.n_slots, Nkv, B), dim3(64), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int rows = B * Nq;
  hipLaunchKernelGGL(decode_merge_kernel, dim3((rows + 3) / 4), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace attn
