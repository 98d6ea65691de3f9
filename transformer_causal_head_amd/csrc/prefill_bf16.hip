// Fused causal / sliding-window / grouped-query attention prefill, bf16 in,
// fp32 accumulate, head size 128, on gfx950 MFMA (v_mfma_f32_32x32x16_bf16).
//
// Method: the textbook's formula softmax(Q K^T * scale + M) V (attention
// chapter, "Scaled dot-product attention"), computed tile by tile with the
// running row maximum and running sum of exponentials that the Chinese
// multi-head attention post describes under "Flash Attention" (rescale the
// old accumulator when a new maximum appears), so the S x S score matrix is
// never written to memory.  Tiles that the causal mask or the window hide
// entirely are never loaded or computed (the textbook's cost remark: the
// explicit form computes the masked half anyway; the window makes useful work
// O(T W d)).
//
// gfx950 design
//   * Scores are computed transposed, S^T = K Q^T: the key index runs along
//     MFMA rows (A operand from LDS), the query index along columns (B
//     operand, Q kept in VGPRs for the whole kernel).  A lane then owns one
//     query column, so the row max and row sum of the softmax are in-register
//     reductions plus one exchange between the two 32-lane halves.
//   * The S^T accumulator layout is exactly the B-operand layout the PV
//     product needs (O^T = V^T P^T), so P goes from fp32 accumulator to bf16
//     operand with one v_cvt_pk_bf16_f32 per pair and no lane exchange.
//   * V is stored transposed in LDS with its keys permuted inside each group
//     of 16 so that each lane's 8 keys of the V^T operand are one 16-byte
//     LDS read.
//   * One workgroup = 4 waves sharing each K/V tile: for grouped-query
//     attention the waves take different query heads of the same K/V head, so
//     a K/V tile is fetched once per group; for MHA they take consecutive
//     query blocks of one head.
//   * Workgroups are ordered longest-key-range first (causal work grows with
//     the query position); with a multiple of 8 (batch, K/V head, head-group)
//     combinations, all workgroups of one K/V head land on the same XCD and
//     share its L2.

#include "common.h"
#include "kernels.h"

namespace attn {

namespace {

constexpr int D = 128;        // head size
constexpr int NW = 4;         // waves per workgroup
constexpr int BN = 64;        // keys per K/V tile
constexpr int KSTR = D + 8;   // K tile row stride (bf16), 16-byte pad
constexpr int VSTR = BN + 8;  // V^T tile row stride (bf16), 16-byte pad

struct Params {
  const __bf16* Q;
  const __bf16* K;
  const __bf16* V;
  __bf16* O;
  float* LSE;
  int B, Nq, Nkv, S;
  int causal, window;
  float c;        // scale * log2(e)
  int G;          // query heads per K/V head
  int hp;         // heads of one group per workgroup
  int qspan;      // queries per workgroup
  int n_qtiles;
  int n_hsub;     // G / hp
};

// Position of key k (0..BN-1) inside a V^T row: bits 2 and 3 swapped, which
// puts the 8 keys one lane feeds to a 16-key MFMA step next to each other.
__device__ __forceinline__ int vt_pos(int k) {
  return (k & ~12) | ((k & 4) << 1) | ((k & 8) >> 1);
}

template <int QB>
__global__ __launch_bounds__(NW * 64) void prefill_kernel(Params p) {
  constexpr int QW = 32 * QB;  // queries per wave
  __shared__ __attribute__((aligned(16))) __bf16 Ks[BN * KSTR];
  __shared__ __attribute__((aligned(16))) __bf16 Vt[D * VSTR];

  const int tid = threadIdx.x;
  const int w = tid >> 6;
  const int lane = tid & 63;
  const int ln = lane & 31;
  const int hl = lane >> 5;

  // workgroup -> (q tile, batch, K/V head, head subgroup); heavy tiles first
  const int inner = p.B * p.Nkv * p.n_hsub;
  const int bid = blockIdx.x;
  const int qt = p.causal ? (p.n_qtiles - 1 - bid / inner) : (bid / inner);
  int rest = bid % inner;
  const int hsub = rest % p.n_hsub;
  rest /= p.n_hsub;
  const int g = rest % p.Nkv;
  const int b = rest / p.Nkv;

  const int head = g * p.G + hsub * p.hp + (w % p.hp);
  const int qa = qt * p.qspan + (w / p.hp) * QW;  // first query of this wave
  const int q0 = qt * p.qspan;
  const int q1 = min(p.S, q0 + p.qspan);
  const int wq1 = min(p.S, qa + QW);
  const bool wave_live = qa < p.S;

  const size_t kv_base = ((size_t)b * p.Nkv + g) * (size_t)p.S * D;
  const size_t q_base = ((size_t)b * p.Nq + head) * (size_t)p.S * D;

  // Q^T operand fragments: query column ln of block qb, d = 16*ks + 8*hl + i
  bf16x8 qf[QB][8];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    int qrow = min(qa + qb * 32 + ln, p.S - 1);
    const bf16x8* src = reinterpret_cast<const bf16x8*>(p.Q + q_base + (size_t)qrow * D + hl * 8);
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) qf[qb][ks] = src[ks * 2];
  }

  f32x16 oacc[QB][4];
  float m_run[QB], l_run[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    m_run[qb] = -INFINITY;
    l_run[qb] = 0.f;
#pragma unroll
    for (int db = 0; db < 4; ++db) oacc[qb][db] = f32x16{};
  }

  // key range of the workgroup
  const int hi = p.causal ? q1 : p.S;
  const int lo = (p.causal && p.window > 0) ? max(0, q0 - p.window + 1) : 0;
  const int t_lo = lo / BN;
  const int t_hi = (hi + BN - 1) / BN;

  // tile loader mapping: thread -> keys 4*kg..4*kg+3, d = 8*dc..8*dc+7
  const int kg = tid >> 4;
  const int dc = tid & 15;

  for (int t = t_lo; t < t_hi; ++t) {
    const int k0 = t * BN;
    __syncthreads();
    {
      u32x4 kv[4], vv[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        int key = k0 + kg * 4 + c;
        if (key < p.S) {
          size_t off = kv_base + (size_t)key * D + dc * 8;
          kv[c] = *reinterpret_cast<const u32x4*>(p.K + off);
          vv[c] = *reinterpret_cast<const u32x4*>(p.V + off);
        } else {
          kv[c] = u32x4{0, 0, 0, 0};
          vv[c] = u32x4{0, 0, 0, 0};
        }
      }
#pragma unroll
      for (int c = 0; c < 4; ++c)
        *reinterpret_cast<u32x4*>(&Ks[(kg * 4 + c) * KSTR + dc * 8]) = kv[c];
      const int kpos = vt_pos(kg * 4);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int j = e >> 1;
        uint32_t w01, w23;
        if (e & 1) {
          w01 = (vv[0][j] >> 16) | (vv[1][j] & 0xffff0000u);
          w23 = (vv[2][j] >> 16) | (vv[3][j] & 0xffff0000u);
        } else {
          w01 = (vv[0][j] & 0xffffu) | (vv[1][j] << 16);
          w23 = (vv[2][j] & 0xffffu) | (vv[3][j] << 16);
        }
        *reinterpret_cast<u32x2*>(&Vt[(dc * 8 + e) * VSTR + kpos]) = u32x2{w01, w23};
      }
    }
    __syncthreads();

    // does this wave see any (query, key) pair of the tile?
    bool live = wave_live;
    if (p.causal) live = live && (k0 <= wq1 - 1);
    if (p.window > 0) live = live && (k0 + BN - 1 >= qa - p.window + 1);
    if (!live) continue;
    bool need_mask = (k0 + BN > p.S);
    if (p.causal) need_mask = need_mask || (k0 + BN - 1 > qa);
    if (p.window > 0) need_mask = need_mask || (wq1 - 1 - k0 >= p.window);

    // S^T = K Q^T for the tile
    f32x16 sacc[QB][BN / 32];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int kb = 0; kb < BN / 32; ++kb) sacc[qb][kb] = f32x16{};
#pragma unroll
    for (int kb = 0; kb < BN / 32; ++kb) {
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        bf16x8 a = *reinterpret_cast<const bf16x8*>(&Ks[(kb * 32 + ln) * KSTR + ks * 16 + hl * 8]);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
          sacc[qb][kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[qb][ks], sacc[qb][kb], 0, 0, 0);
      }
    }

    // mask: accumulator register r of key block kb holds key
    // k0 + 32*kb + 8*(r/4) + 4*hl + (r%4) for query column ln
    if (need_mask) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        const int qi = qa + qb * 32 + ln;
#pragma unroll
        for (int kb = 0; kb < BN / 32; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int kj = k0 + kb * 32 + (r >> 2) * 8 + hl * 4 + (r & 3);
            bool ok = kj < p.S;
            if (p.causal) ok = ok && (kj <= qi);
            if (p.window > 0) ok = ok && (qi - kj < p.window);
            if (!ok) sacc[qb][kb][r] = -INFINITY;
          }
      }
    }

    // online softmax per query column, then P^T operand fragments
    bf16x8 pf[QB][BN / 16];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < BN / 32; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[qb][kb][r]);
      mx = fmaxf(mx, swap_halves(mx));
      const float m_new = fmaxf(m_run[qb], mx * p.c);
      const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
      const float alpha = exp2_fast(m_run[qb] - m_use);
      m_run[qb] = m_new;
      float rs = 0.f;
#pragma unroll
      for (int kb = 0; kb < BN / 32; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float e = exp2_fast(__builtin_fmaf(sacc[qb][kb][r], p.c, -m_use));
          sacc[qb][kb][r] = e;
          rs += e;
        }
      l_run[qb] = l_run[qb] * alpha + rs;
#pragma unroll
      for (int db = 0; db < 4; ++db) oacc[qb][db] *= alpha;
#pragma unroll
      for (int kb = 0; kb < BN / 32; ++kb)
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          u32x4 pk;
#pragma unroll
          for (int j = 0; j < 4; ++j)
            pk[j] = pack_bf16x2(sacc[qb][kb][kk * 8 + 2 * j], sacc[qb][kb][kk * 8 + 2 * j + 1]);
          pf[qb][kb * 2 + kk] = __builtin_bit_cast(bf16x8, pk);
        }
    }

    // O^T += V^T P^T
#pragma unroll
    for (int ks = 0; ks < BN / 16; ++ks) {
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        bf16x8 a = *reinterpret_cast<const bf16x8*>(&Vt[(db * 32 + ln) * VSTR + ks * 16 + hl * 8]);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
          oacc[qb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[qb][ks], oacc[qb][db], 0, 0, 0);
      }
    }
  }

  if (!wave_live) return;
  // epilogue: O = O_acc / l, LSE = (m + log2 l) * ln 2
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int qi = qa + qb * 32 + ln;
    const float l_tot = l_run[qb] + swap_halves(l_run[qb]);
    if (qi >= p.S) continue;
    const float inv = 1.f / l_tot;
    __bf16* orow = p.O + q_base + (size_t)qi * D;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4) {
        const int d0 = db * 32 + a4 * 8 + hl * 4;
        u32x2 st;
        st[0] = pack_bf16x2(oacc[qb][db][a4 * 4 + 0] * inv, oacc[qb][db][a4 * 4 + 1] * inv);
        st[1] = pack_bf16x2(oacc[qb][db][a4 * 4 + 2] * inv, oacc[qb][db][a4 * 4 + 3] * inv);
        *reinterpret_cast<u32x2*>(orow + d0) = st;
      }
    if (p.LSE != nullptr && hl == 0)
      p.LSE[((size_t)b * p.Nq + head) * p.S + qi] = (m_run[qb] + __log2f(l_tot)) * kLn2;
  }
}

}  // namespace

hipError_t launch_prefill_bf16_d128(const void* Q, const void* K, const void* V, void* O,
                                    float* LSE, int B, int Nq, int Nkv, int S, int causal,
                                    int window, float scale, hipStream_t stream) {
  constexpr int QB = 2;
  Params p;
  p.Q = static_cast<const __bf16*>(Q);
  p.K = static_cast<const __bf16*>(K);
  p.V = static_cast<const __bf16*>(V);
  p.O = static_cast<__bf16*>(O);
  p.LSE = LSE;
  p.B = B;
  p.Nq = Nq;
  p.Nkv = Nkv;
  p.S = S;
  p.causal = causal;
  p.window = window;
  p.c = scale * kLog2e;
  p.G = Nq / Nkv;
  p.hp = (p.G % 4 == 0) ? 4 : (p.G % 2 == 0) ? 2 : 1;
  p.n_hsub = p.G / p.hp;
  p.qspan = (NW / p.hp) * 32 * QB;
  p.n_qtiles = (S + p.qspan - 1) / p.qspan;
  const long long nblocks = (long long)p.n_qtiles * B * Nkv * p.n_hsub;
  if (nblocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(prefill_kernel<QB>, dim3((unsigned)nblocks), dim3(NW * 64), 0, stream, p);
  return hipGetLastError();
}

}  // namespace attn
