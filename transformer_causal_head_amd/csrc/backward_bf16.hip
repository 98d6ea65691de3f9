// Backward pass of prefill attention on bf16 MFMA (head size 64, 128 or 256).
// Same mathematics as the general row kernels in backward.hip (the
// weights recomputed from the stored LSE, the softmax Jacobian p (delta - p)
// of the textbook's "Почему делить на корень из d_h"), split into two kernels
// so that every gradient has a single owner and no float atomics are needed
// (the results are bitwise reproducible):
//
//   dq_kernel  -- one wavefront per 32 query rows of one head, streaming the
//                 K/V tiles of its key range like the forward pass:
//                   S^T  = K Q^T     (A: K tile rows,  B: Q in VGPRs)
//                   dP^T = V dO^T    (A: V tile rows,  B: dO in VGPRs)
//                   dS^T = P^T (dP^T - Delta),  P^T = exp2(S^T c - LSE log2 e)
//                 (LSE log2 e comes from the Delta pass, +inf for a row that
//                 saw no key under a key-padding mask, so its weights are 0)
//                   dQ^T += K^T dS^T (A: K tile read transposed, B: dS^T)
//   dkv_kernel -- (head sizes 64 and 256; head size 128 uses dkv_pipe_kernel
//                 below, which puts dV and dK on different wavefronts; at 256
//                 one wavefront per SIMD holds the K and V fragments and both
//                 accumulators, 512 registers with a few spilled)
//                 one wavefront per 32 keys of one K/V head, streaming the Q and
//                 dO tiles of every query head of its group over the queries
//                 that see those keys:
//                   S  = Q K^T       (A: Q tile rows,  B: K in VGPRs)
//                   dP = dO V^T      (A: dO tile rows, B: V in VGPRs)
//                   dV^T += dO^T P   (A: dO tile read transposed, B: P)
//                   dK^T += Q^T dS   (A: Q tile read transposed,  B: dS)
//
// In both, the 32x32 score accumulator is used directly (rounded to bf16) as
// the B operand of the product that contracts over its rows; the transposing
// LDS reads deliver the A operand in the matching row order.  Tiles are
// copied HBM -> LDS by buffer DMA, two stages, with the swizzle of tiles.h.

#include "common.h"
#include "kernels.h"
#include "tiles.h"


namespace attn {

namespace {

struct BwdMfmaParams {
  const __bf16* Q;
  const __bf16* K;
  const __bf16* V;
  const __bf16* dO;
  const float* lse2;   // the rows' LSE in log2 units, +inf for a row that saw no key
  const float* delta;
  const uint64_t* kbits;  // key-padding mask (kwords words per sequence) or null
  int kwords;
  __bf16* dQ;
  __bf16* dK;
  __bf16* dV;
  int B, Nq, Nkv, S;
  int causal, window;
  float c;       // scale * log2(e)
  float scale;
  int G;         // query heads per K/V head
  // dq_kernel grid
  int hp, qspan, n_qtiles, n_hsub;
};

// Mask of one 32x32 accumulator: rows (r/4)*8 + hl*4 + r%4 of the block,
// column ln.  Visible iff key <= query (causal), query - key < window, and
// both below S.
__device__ __forceinline__ bool visible(const BwdMfmaParams& p, int q, int k) {
  bool ok = q < p.S && k < p.S;
  if (p.causal) ok = ok && k <= q;
  if (p.window > 0) ok = ok && q - k < p.window;
  return ok;
}

// ---------------------------------------------------------------------------
// dQ: one wavefront = 32 query rows of one head; workgroup as in the forward
// KM: a key-padding mask is given (p.kbits); without it the kernels are
// compiled as if it did not exist.
template <int D, int NW, bool KM>
__global__ __launch_bounds__(NW * 64) void dq_kernel(BwdMfmaParams p) {
  using geo = Geo<D>;
  constexpr int KS = geo::KS;
  constexpr int DB = geo::DB;
  __shared__ __attribute__((aligned(1024))) char k0s[geo::TILE];
  __shared__ __attribute__((aligned(1024))) char k1s[geo::TILE];
  __shared__ __attribute__((aligned(1024))) char v0s[geo::TILE];
  __shared__ __attribute__((aligned(1024))) char v1s[geo::TILE];

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int ln = lane & 31;
  const int hl = lane >> 5;

  const int inner = p.B * p.Nkv * p.n_hsub;
  const int bid = blockIdx.x;
  const int qt = p.causal ? (p.n_qtiles - 1 - bid / inner) : (bid / inner);
  int rest = bid % inner;
  const int hsub = rest % p.n_hsub;
  rest /= p.n_hsub;
  const int g = rest % p.Nkv;
  const int b = rest / p.Nkv;

  const int head = g * p.G + hsub * p.hp + (w % p.hp);
  const int qa = qt * p.qspan + (w / p.hp) * 32;  // first query row of this wave
  const int q0 = qt * p.qspan;
  const int q1 = min(p.S, q0 + p.qspan);
  const int wq1 = min(p.S, qa + 32);
  const bool wave_live = qa < p.S;

  const size_t kv_base = ((size_t)b * p.Nkv + g) * (size_t)p.S * D;
  const HeadRef Kh = head_ref<D>(p.K + kv_base, p.S);
  const HeadRef Vh = head_ref<D>(p.V + kv_base, p.S);
  const size_t q_row0 = ((size_t)b * p.Nq + head) * (size_t)p.S;

  const int hi_key = p.causal ? q1 : p.S;
  const int lo_key = (p.causal && p.window > 0) ? max(0, q0 - p.window + 1) : 0;
  const int t_lo = lo_key / BN;
  const int nt = (hi_key + BN - 1) / BN - t_lo;

  load_tile<D, NW>(Kh, t_lo * BN, k0s, w, lane);
  load_tile<D, NW>(Vh, t_lo * BN, v0s, w, lane);

  // Q and dO as B operands: query column ln, head dims 16*ks + 8*hl + i
  const int qi = min(qa + ln, p.S - 1);
  bf16x8 qf[KS], df[KS];
  {
    const bf16x8* qs = reinterpret_cast<const bf16x8*>(p.Q + (q_row0 + qi) * D + hl * 8);
    const bf16x8* ds = reinterpret_cast<const bf16x8*>(p.dO + (q_row0 + qi) * D + hl * 8);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      qf[ks] = qs[ks * 2];
      df[ks] = ds[ks * 2];
    }
  }
  const float lse2 = p.lse2[q_row0 + qi];
  const float dlt = p.delta[q_row0 + qi];
  const uint64_t* const kr = KM ? p.kbits + (size_t)b * p.kwords : nullptr;

  int roff[KS];
  row_operand_offsets<D>(ln, hl, roff);
  int troff[2][DB];
  tr_operand_offsets<D>(lane, troff);

  f32x16 dq[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) dq[db] = f32x16{};

  // tiles with any visible pair for this wave, and with only visible pairs
  auto fdiv = [](int a) { return a >= 0 ? a / BN : -((-a + BN - 1) / BN); };
  int tl_lo = p.window > 0 ? fdiv(qa - p.window + 1) : -1;
  int tl_hi = p.causal ? fdiv(wq1 - 1) : (p.S - 1) / BN;
  if (!wave_live) tl_hi = tl_lo - 1;
  int tf_lo = p.window > 0 ? -fdiv(-(wq1 - p.window)) : 0;
  int tf_hi = fdiv(p.S - BN);
  if (p.causal) tf_hi = min(tf_hi, fdiv(qa - (BN - 1)));
  tl_lo = __builtin_amdgcn_readfirstlane(tl_lo);
  tl_hi = __builtin_amdgcn_readfirstlane(tl_hi);
  tf_lo = __builtin_amdgcn_readfirstlane(tf_lo);
  tf_hi = __builtin_amdgcn_readfirstlane(tf_hi);

  // tile i reads stage (Kt, Vt) and copies tile i + 1 into the other stage;
  // the loop below passes the stages as fixed LDS objects so that the
  // compiler can tell the copies in flight from the tile being read
  auto step = [&](int i, const char* Kt, const char* Vt, char* Kn, char* Vn) {
    const int t = t_lo + i;
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this tile's copies have landed
    __syncthreads();
    if (i + 1 < nt) {
      load_tile<D, NW>(Kh, (t + 1) * BN, Kn, w, lane);
      load_tile<D, NW>(Vh, (t + 1) * BN, Vn, w, lane);
    }
    if (t < tl_lo || t > tl_hi) return;
    // key-padding flags of the tile's 64 keys (one mask word); a tile of
    // padding only contributes nothing
    const uint64_t kword = KM ? kr[t] : ~0ull;
    if (KM && kword == 0) return;
    const bool need_mask = t < tf_lo || t > tf_hi || (KM && kword != ~0ull);
    const int k0 = t * BN;
    if constexpr (D == 256) {
      // At head size 256 (one wave per SIMD) S and dP of both 32-key halves
      // come first, so that the weights of half 0 can run beside the products
      // of half 1 and those of half 1 beside dQ of half 0 (the backward at
      // 16384 tokens 1-3 % faster).  With two waves per SIMD the other wave
      // fills those gaps already (head size 128 unchanged, 64 4 % slower).
      f32x16 s2[2], dp2[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        s2[kb] = f32x16{};
        dp2[kb] = f32x16{};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const bf16x8 ka = *reinterpret_cast<const bf16x8*>(Kt + kb * 32 * geo::RB + roff[ks]);
          s2[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[ks], s2[kb], 0, 0, 0);
        }
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const bf16x8 va = *reinterpret_cast<const bf16x8*>(Vt + kb * 32 * geo::RB + roff[ks]);
          dp2[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, df[ks], dp2[kb], 0, 0, 0);
        }
      }
      bf16x8 dsf2[2][2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        // register r: key k0 + 32*kb + 8*(r/4) + 4*hl + r%4, query qa + ln
        if (need_mask) {
          const uint32_t kwl = (uint32_t)(kword >> (kb * 32)) >> (hl * 4);
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = k0 + kb * 32 + (r >> 2) * 8 + hl * 4 + (r & 3);
            bool hide = !visible(p, qa + ln, key);
            if (KM) hide = hide || !((kwl >> ((r >> 2) * 8 + (r & 3))) & 1);
            if (hide) s2[kb][r] = -INFINITY;
          }
        }
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          u32x4 pk;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int r0 = kk * 8 + 2 * j;
            const float p0 = exp2_fast(__builtin_fmaf(s2[kb][r0], p.c, -lse2));
            const float p1 = exp2_fast(__builtin_fmaf(s2[kb][r0 + 1], p.c, -lse2));
            pk[j] = pack_bf16x2(p0 * (dp2[kb][r0] - dlt), p1 * (dp2[kb][r0 + 1] - dlt));
          }
          dsf2[kb][kk] = __builtin_bit_cast(bf16x8, pk);
        }
      }
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
#pragma unroll
          for (int db = 0; db < DB; ++db) {
            const bf16x8 a = read_tr_operand<D>(Kt, kb * 2 + kk, troff, db);
            dq[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, dsf2[kb][kk], dq[db], 0, 0, 0);
          }
    } else {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const bf16x8 ka = *reinterpret_cast<const bf16x8*>(Kt + kb * 32 * geo::RB + roff[ks]);
          s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[ks], s, 0, 0, 0);
        }
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const bf16x8 va = *reinterpret_cast<const bf16x8*>(Vt + kb * 32 * geo::RB + roff[ks]);
          dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, df[ks], dp, 0, 0, 0);
        }
        // register r: key k0 + 32*kb + 8*(r/4) + 4*hl + r%4, query qa + ln
        if (need_mask) {
          // this lane's flags: register r holds key k0 + 32*kb + 8*(r/4) + 4*hl + r%4
          const uint32_t kwl = (uint32_t)(kword >> (kb * 32)) >> (hl * 4);
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = k0 + kb * 32 + (r >> 2) * 8 + hl * 4 + (r & 3);
            bool hide = !visible(p, qa + ln, key);
            if (KM) hide = hide || !((kwl >> ((r >> 2) * 8 + (r & 3))) & 1);
            if (hide) s[r] = -INFINITY;
          }
        }
        bf16x8 dsf[2];
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          u32x4 pk;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int r0 = kk * 8 + 2 * j;
            const float p0 = exp2_fast(__builtin_fmaf(s[r0], p.c, -lse2));
            const float p1 = exp2_fast(__builtin_fmaf(s[r0 + 1], p.c, -lse2));
            pk[j] = pack_bf16x2(p0 * (dp[r0] - dlt), p1 * (dp[r0 + 1] - dlt));
          }
          dsf[kk] = __builtin_bit_cast(bf16x8, pk);
        }
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
#pragma unroll
          for (int db = 0; db < DB; ++db) {
            const bf16x8 a = read_tr_operand<D>(Kt, kb * 2 + kk, troff, db);
            dq[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, dsf[kk], dq[db], 0, 0, 0);
          }
      }
    }
  };
  int i = 0;
  for (; i + 1 < nt; i += 2) {
    step(i, k0s, v0s, k1s, v1s);
    step(i + 1, k1s, v1s, k0s, v0s);
  }
  if (i < nt) step(i, k0s, v0s, k1s, v1s);
  __builtin_amdgcn_s_waitcnt(0x0F70);  // no copy may still target LDS when the wave ends

  if (!wave_live || qa + ln >= p.S) return;
  __bf16* row = p.dQ + (q_row0 + qa + ln) * D;
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int a4 = 0; a4 < 4; ++a4) {
      const int d0 = db * 32 + a4 * 8 + hl * 4;
      u32x2 st;
      st[0] = pack_bf16x2(dq[db][a4 * 4 + 0] * p.scale, dq[db][a4 * 4 + 1] * p.scale);
      st[1] = pack_bf16x2(dq[db][a4 * 4 + 2] * p.scale, dq[db][a4 * 4 + 3] * p.scale);
      *reinterpret_cast<u32x2*>(row + d0) = st;
    }
}

// ---------------------------------------------------------------------------
// dK, dV: one wavefront = 32 keys of one K/V head; workgroup = NW waves of
// consecutive keys; loops over (query head of the group, query tile).
template <int D, int NW, bool KM>
__global__ __launch_bounds__(NW * 64) void dkv_kernel(BwdMfmaParams p) {
  using geo = Geo<D>;
  constexpr int KS = geo::KS;
  constexpr int DB = geo::DB;
  constexpr int KB = NW * 32;  // keys per workgroup
  __shared__ __attribute__((aligned(1024))) char q0s[geo::TILE];
  __shared__ __attribute__((aligned(1024))) char q1s[geo::TILE];
  __shared__ __attribute__((aligned(1024))) char o0s[geo::TILE];
  __shared__ __attribute__((aligned(1024))) char o1s[geo::TILE];
  // LSE and Delta of the tile's 64 query rows, next to the Q / dO tile
  __shared__ __attribute__((aligned(256))) float a0s[2 * BN];
  __shared__ __attribute__((aligned(256))) float a1s[2 * BN];

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int ln = lane & 31;
  const int hl = lane >> 5;

  const int n_kb = (p.S + KB - 1) / KB;
  const int kt = blockIdx.x % n_kb;  // key blocks in ascending order: heaviest first
  const int bg = blockIdx.x / n_kb;
  const int g = bg % p.Nkv;
  const int b = bg / p.Nkv;

  const int k0 = kt * KB;
  const int k1 = min(p.S, k0 + KB);
  const int kw0 = k0 + w * 32;          // this wave's first key
  const int kw1 = min(p.S, kw0 + 32);
  const bool wave_live = kw0 < p.S;
  const size_t kv_row0 = ((size_t)b * p.Nkv + g) * (size_t)p.S;

  // query range of the workgroup: queries that see any of its keys
  const int qlo = p.causal ? k0 : 0;
  const int qhi = (p.causal && p.window > 0) ? min(p.S, k1 - 1 + p.window) : p.S;
  const int t_lo = qlo / BN;
  const int n_qt = (qhi + BN - 1) / BN - t_lo;  // query tiles per head
  const int n_items = p.G * max(n_qt, 0);

  // copies of item `item` (query head hh of the group, query tile q0): the Q
  // and dO tiles, and 64 LSE (wave 0) and 64 Delta (wave 1) values, which
  // read as zero past the last row like the tile rows
  auto issue = [&](int item, char* qdst, char* odst, float* adst) {
    const int hh = item / n_qt;
    const int q0 = (t_lo + item % n_qt) * BN;
    const size_t row0 = ((size_t)b * p.Nq + (size_t)g * p.G + hh) * (size_t)p.S;
    load_tile<D, NW>(head_ref<D>(p.Q + row0 * D, p.S), q0, qdst, w, lane);
    load_tile<D, NW>(head_ref<D>(p.dO + row0 * D, p.S), q0, odst, w, lane);
    if (w < 2) {
      const float* src = (w == 0 ? p.lse2 : p.delta) + row0;
      const __amdgpu_buffer_rsrc_t rs =
          __builtin_amdgcn_make_buffer_rsrc((void*)src, (short)0, p.S * 4, 0x00020000);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(adst + w * BN), 4, (q0 + lane) * 4,
                                               0, 0, 0);
    }
  };
  if (n_items > 0) issue(0, q0s, o0s, a0s);

  // key-padding flag of this lane's key; a wave whose 32 keys are all
  // padding has no gradient to form
  bool key_ok = true, any_key = true, all_keys = true;
  const int kj = min(kw0 + ln, p.S - 1);
  if constexpr (KM) {
    key_ok = (p.kbits[(size_t)b * p.kwords + (kj >> 6)] >> (kj & 63)) & 1;
    const uint64_t key_bal = __builtin_amdgcn_ballot_w64(key_ok);
    any_key = __builtin_amdgcn_readfirstlane(key_bal != 0);
    all_keys = __builtin_amdgcn_readfirstlane(key_bal == ~0ull);
  }

  // K and V as B operands: key column ln, head dims 16*ks + 8*hl + i
  bf16x8 kf[KS], vf[KS];
  {
    const bf16x8* ks_ = reinterpret_cast<const bf16x8*>(p.K + (kv_row0 + kj) * D + hl * 8);
    const bf16x8* vs_ = reinterpret_cast<const bf16x8*>(p.V + (kv_row0 + kj) * D + hl * 8);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      kf[ks] = ks_[ks * 2];
      vf[ks] = vs_[ks * 2];
    }
  }

  int roff[KS];
  row_operand_offsets<D>(ln, hl, roff);
  int troff[2][DB];
  tr_operand_offsets<D>(lane, troff);

  f32x16 dk[DB], dv[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    dk[db] = f32x16{};
    dv[db] = f32x16{};
  }

  // item `it` reads stage (Qt, Ot, At) and copies item it + 1 into the other
  // stage (fixed LDS objects, as in dq_kernel)
  auto item = [&](int it, const char* Qt, const char* Ot, const float* At, char* Qn, char* On,
                  float* An) {
    const int q0 = (t_lo + it % n_qt) * BN;
    __builtin_amdgcn_s_waitcnt(0x0F70);
    __syncthreads();
    if (it + 1 < n_items) issue(it + 1, Qn, On, An);
    // does this wave see any (query, key) pair of the tile?  all of them?
    bool live = wave_live && q0 < p.S && any_key;
    if (p.causal) live = live && q0 + BN - 1 >= kw0;
    if (p.window > 0) live = live && q0 - (kw1 - 1) < p.window;
    if (!live) return;
    bool full = q0 + BN <= p.S && kw1 - kw0 == 32 && all_keys;
    if (p.causal) full = full && q0 >= kw1 - 1;
    if (p.window > 0) full = full && q0 + BN - 1 - kw0 < p.window;

#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const bf16x8 qa = *reinterpret_cast<const bf16x8*>(Qt + mb * 32 * geo::RB + roff[ks]);
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa, kf[ks], s, 0, 0, 0);
      }
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const bf16x8 oa = *reinterpret_cast<const bf16x8*>(Ot + mb * 32 * geo::RB + roff[ks]);
        dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(oa, vf[ks], dp, 0, 0, 0);
      }
      // register r: query q0 + 32*mb + 8*(r/4) + 4*hl + r%4, key kw0 + ln;
      // the LSE and Delta of those rows are 4 consecutive floats per r/4
      if (!full) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int q = q0 + mb * 32 + (r >> 2) * 8 + hl * 4 + (r & 3);
          if (!visible(p, q, kw0 + ln) || (KM && !key_ok)) s[r] = -INFINITY;
        }
      }
      bf16x8 pf[2], sf[2];
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        u32x4 pp, ss;
        f32x4 l4[2], d4[2];
#pragma unroll
        for (int a = 0; a < 2; ++a) {
          l4[a] = *reinterpret_cast<const f32x4*>(At + mb * 32 + (2 * kk + a) * 8 + hl * 4);
          d4[a] = *reinterpret_cast<const f32x4*>(At + BN + mb * 32 + (2 * kk + a) * 8 + hl * 4);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int r0 = kk * 8 + 2 * j;
          const f32x4 lv = l4[j >> 1], dv4 = d4[j >> 1];
          const int u = (2 * j) & 3;
          const float p0 = exp2_fast(__builtin_fmaf(s[r0], p.c, -lv[u]));
          const float p1 = exp2_fast(__builtin_fmaf(s[r0 + 1], p.c, -lv[u + 1]));
          pp[j] = pack_bf16x2(p0, p1);
          ss[j] = pack_bf16x2(p0 * (dp[r0] - dv4[u]), p1 * (dp[r0 + 1] - dv4[u + 1]));
        }
        pf[kk] = __builtin_bit_cast(bf16x8, pp);
        sf[kk] = __builtin_bit_cast(bf16x8, ss);
      }
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const bf16x8 oa = read_tr_operand<D>(Ot, mb * 2 + kk, troff, db);
          dv[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(oa, pf[kk], dv[db], 0, 0, 0);
          const bf16x8 qa = read_tr_operand<D>(Qt, mb * 2 + kk, troff, db);
          dk[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa, sf[kk], dk[db], 0, 0, 0);
        }
    }
  };
  int it = 0;
  for (; it + 1 < n_items; it += 2) {
    item(it, q0s, o0s, a0s, q1s, o1s, a1s);
    item(it + 1, q1s, o1s, a1s, q0s, o0s, a0s);
  }
  if (it < n_items) item(it, q0s, o0s, a0s, q1s, o1s, a1s);
  __builtin_amdgcn_s_waitcnt(0x0F70);

  if (!wave_live || kw0 + ln >= p.S) return;
  __bf16* krow = p.dK + (kv_row0 + kw0 + ln) * D;
  __bf16* vrow = p.dV + (kv_row0 + kw0 + ln) * D;
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int a4 = 0; a4 < 4; ++a4) {
      const int d0 = db * 32 + a4 * 8 + hl * 4;
      u32x2 sk, sv;
      sk[0] = pack_bf16x2(dk[db][a4 * 4 + 0] * p.scale, dk[db][a4 * 4 + 1] * p.scale);
      sk[1] = pack_bf16x2(dk[db][a4 * 4 + 2] * p.scale, dk[db][a4 * 4 + 3] * p.scale);
      sv[0] = pack_bf16x2(dv[db][a4 * 4 + 0], dv[db][a4 * 4 + 1]);
      sv[1] = pack_bf16x2(dv[db][a4 * 4 + 2], dv[db][a4 * 4 + 3]);
      *reinterpret_cast<u32x2*>(krow + d0) = sk;
      *reinterpret_cast<u32x2*>(vrow + d0) = sv;
    }
}

// dK, dV on two wavefronts per 32 keys, skewed by one item: a workgroup of 8
// waves holds 128 keys of one K/V head and runs the (query head, 64-query
// tile) items of its group in order.  In round `it`:
//   waves 0-3 (dV) compute S = Q K^T and P for item it, store P (fp32, in
//              their accumulator layout) to LDS and accumulate dV^T += dO^T P;
//   waves 4-7 (dK) compute dP = dO V^T for item it and keep it in registers,
//              then form dS = P (dP - Delta) for item it - 1 from the P the dV
//              waves stored in the previous round, and accumulate
//              dK^T += Q^T dS.
// One barrier per round orders everything: it publishes the previous round's
// P and frees the stages the next copies overwrite.  Q and Delta live for
// three rounds (item it - 1 on the dK side, it, and it + 1 being copied), dO,
// LSE and P for two.  Each role issues the copies of the stages it reads
// transposed (dV: dO and LSE; dK: Q and Delta) and runs its own loop unrolled
// by that stage count, so every transposing read names a fixed LDS object and
// the compiler keeps the copies in flight across it.  Same products and
// roundings as the other forms: the results are bit for bit theirs.
template <int D, bool KM>
__global__ __launch_bounds__(512) void dkv_pipe_kernel(BwdMfmaParams p) {
  using geo = Geo<D>;
  constexpr int NR = 4;  // waves per role
  constexpr int KS = geo::KS;
  constexpr int DB = geo::DB;
  constexpr int KB = 128;  // keys per workgroup
  constexpr int PW = 2 * 4 * 64;  // f32x4 of P per wave pair: [32-query block][register group][lane]
  __shared__ __attribute__((aligned(1024))) char q0s[geo::TILE];
  __shared__ __attribute__((aligned(1024))) char q1s[geo::TILE];
  __shared__ __attribute__((aligned(1024))) char q2s[geo::TILE];
  __shared__ __attribute__((aligned(1024))) char o0s[geo::TILE];
  __shared__ __attribute__((aligned(1024))) char o1s[geo::TILE];
  __shared__ __attribute__((aligned(256))) float l0s[BN];
  __shared__ __attribute__((aligned(256))) float l1s[BN];
  __shared__ __attribute__((aligned(256))) float d0s[BN];
  __shared__ __attribute__((aligned(256))) float d1s[BN];
  __shared__ __attribute__((aligned(256))) float d2s[BN];
  __shared__ __attribute__((aligned(16))) f32x4 p0s[NR * PW];
  __shared__ __attribute__((aligned(16))) f32x4 p1s[NR * PW];

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool krole = w >= NR;  // wave-uniform: dK (true) or dV
  const int wl = w & (NR - 1);  // index within the role; waves w and w + 4 share keys
  const int lane = tid & 63;
  const int ln = lane & 31;
  const int hl = lane >> 5;

  const int n_kb = (p.S + KB - 1) / KB;
  const int kt = blockIdx.x % n_kb;
  const int bg = blockIdx.x / n_kb;
  const int g = bg % p.Nkv;
  const int b = bg / p.Nkv;

  const int k0 = kt * KB;
  const int k1 = min(p.S, k0 + KB);
  const int kw0 = k0 + wl * 32;  // this wave's first key
  const int kw1 = min(p.S, kw0 + 32);
  const bool wave_live = kw0 < p.S;
  const size_t kv_row0 = ((size_t)b * p.Nkv + g) * (size_t)p.S;

  const int qlo = p.causal ? k0 : 0;
  const int qhi = (p.causal && p.window > 0) ? min(p.S, k1 - 1 + p.window) : p.S;
  const int t_lo = qlo / BN;
  const int n_qt = (qhi + BN - 1) / BN - t_lo;
  const int n_items = p.G * max(n_qt, 0);

  auto item_q0 = [&](int it) { return (t_lo + it % n_qt) * BN; };
  auto item_row0 = [&](int it) {
    return ((size_t)b * p.Nq + (size_t)g * p.G + it / n_qt) * (size_t)p.S;
  };
  // one 4-byte DMA per lane: 64 values of an fp32 row vector (LSE or Delta)
  auto load_vec = [&](const float* src, int q0, float* dst) {
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc((void*)src, (short)0, p.S * 4, 0x00020000);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)dst, 4, (q0 + lane) * 4, 0, 0, 0);
  };
  auto issue_v = [&](int it, char* odst, float* ldst) {  // dV waves: dO and LSE
    const size_t row0 = item_row0(it);
    const int q0 = item_q0(it);
    load_tile<D, NR>(head_ref<D>(p.dO + row0 * D, p.S), q0, odst, wl, lane);
    if (wl == 0) load_vec(p.lse2 + row0, q0, ldst);
  };
  auto issue_k = [&](int it, char* qdst, float* ddst) {  // dK waves: Q and Delta
    const size_t row0 = item_row0(it);
    const int q0 = item_q0(it);
    load_tile<D, NR>(head_ref<D>(p.Q + row0 * D, p.S), q0, qdst, wl, lane);
    if (wl == 0) load_vec(p.delta + row0, q0, ddst);
  };
  // does the wave pair see any (query, key) pair of item it?  all of them?
  // key-padding flag of this lane's key (waves w and w + 4 share keys)
  bool key_ok = true, any_key = true, all_keys = true;
  const int kj = min(kw0 + ln, p.S - 1);
  if constexpr (KM) {
    key_ok = (p.kbits[(size_t)b * p.kwords + (kj >> 6)] >> (kj & 63)) & 1;
    const uint64_t key_bal = __builtin_amdgcn_ballot_w64(key_ok);
    any_key = __builtin_amdgcn_readfirstlane(key_bal != 0);
    all_keys = __builtin_amdgcn_readfirstlane(key_bal == ~0ull);
  }
  auto live_of = [&](int it) {
    if (it >= n_items) return false;
    const int q0 = item_q0(it);
    bool live = wave_live && q0 < p.S && any_key;
    if (p.causal) live = live && q0 + BN - 1 >= kw0;
    if (p.window > 0) live = live && q0 - (kw1 - 1) < p.window;
    return live;
  };
  auto full_of = [&](int it) {
    const int q0 = item_q0(it);
    bool full = q0 + BN <= p.S && kw1 - kw0 == 32 && all_keys;
    if (p.causal) full = full && q0 >= kw1 - 1;
    if (p.window > 0) full = full && q0 + BN - 1 - kw0 < p.window;
    return full;
  };
  auto qstage = [&](int k) -> const char* { return k == 0 ? q0s : (k == 1 ? q1s : q2s); };

  // K fragments (dV waves, for S) or V fragments (dK waves, for dP) as B
  // operands: key column ln, head dims 16*ks + 8*hl + i
  bf16x8 bf[KS];
  {
    const bf16x8* src =
        reinterpret_cast<const bf16x8*>((krole ? p.V : p.K) + (kv_row0 + kj) * D + hl * 8);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) bf[ks] = src[ks * 2];
  }
  int roff[KS];
  row_operand_offsets<D>(ln, hl, roff);
  int troff[2][DB];
  tr_operand_offsets<D>(lane, troff);

  f32x16 acc[DB];  // dV (waves 0-3) or dK / scale (waves 4-7)
#pragma unroll
  for (int db = 0; db < DB; ++db) acc[db] = f32x16{};

  if (n_items > 0) {
    if (krole)
      issue_k(0, q0s, d0s);
    else
      issue_v(0, o0s, l0s);
  }

  if (!krole) {
    // round it: item it; dO, LSE and P in stage it % 2, Q in stage it % 3
    auto v_round = [&](int it, const char* Ot, const float* Lt, f32x4* Pt, char* On, float* Ln) {
      __builtin_amdgcn_s_waitcnt(0x0F70);
      __syncthreads();
      if (!live_of(it)) {
        if (it + 1 < n_items) issue_v(it + 1, On, Ln);
        return;
      }
      const int q0 = item_q0(it);
      const bool full = full_of(it);
      const char* Qt = qstage(it % 3);
      f32x4* const pw = Pt + wl * PW + lane;
      bf16x8 pf[2][2];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        f32x16 s = f32x16{};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const bf16x8 qa = *reinterpret_cast<const bf16x8*>(Qt + mb * 32 * geo::RB + roff[ks]);
          s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa, bf[ks], s, 0, 0, 0);
        }
        // register r: query q0 + 32*mb + 8*(r/4) + 4*hl + r%4, key kw0 + ln
        if (!full) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int q = q0 + mb * 32 + (r >> 2) * 8 + hl * 4 + (r & 3);
            if (!visible(p, q, kw0 + ln) || (KM && !key_ok)) s[r] = -INFINITY;
          }
        }
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          const f32x4 l4 = *reinterpret_cast<const f32x4*>(Lt + mb * 32 + a * 8 + hl * 4);
          f32x4 e;
#pragma unroll
          for (int u = 0; u < 4; ++u)
            e[u] = exp2_fast(__builtin_fmaf(s[a * 4 + u], p.c, -l4[u]));
          pw[(mb * 4 + a) * 64] = e;
          u32x4& dst = *reinterpret_cast<u32x4*>(&pf[mb][a >> 1]);
          dst[(a & 1) * 2 + 0] = pack_bf16x2(e[0], e[1]);
          dst[(a & 1) * 2 + 1] = pack_bf16x2(e[2], e[3]);
        }
      }
      // the next item's copies go out after the reads of the Q stage, which
      // is picked at run time (the compiler would otherwise wait for the
      // copies before those reads) and before the transposing reads of dO
      if (it + 1 < n_items) issue_v(it + 1, On, Ln);
      // dV^T += dO^T P
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
#pragma unroll
          for (int db = 0; db < DB; ++db) {
            const bf16x8 oa = read_tr_operand<D>(Ot, mb * 2 + kk, troff, db);
            acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(oa, pf[mb][kk], acc[db], 0, 0, 0);
          }
    };
    int it = 0;
    for (; it + 1 < n_items; it += 2) {
      v_round(it, o0s, l0s, p0s, o1s, l1s);
      v_round(it + 1, o1s, l1s, p1s, o0s, l0s);
    }
    if (it < n_items) v_round(it, o0s, l0s, p0s, o1s, l1s);
    // the dK waves' last round (the dS and dK of the last item)
    __builtin_amdgcn_s_waitcnt(0x0F70);
    __syncthreads();
  } else {
    f32x16 dp_prev[2] = {f32x16{}, f32x16{}};
    bool live_prev = false;
    // round it (0 .. n_items): dP of item it (dO in stage it % 2); dS and dK
    // of item it - 1 (Q and Delta in stage (it - 1) % 3, P in stage (it - 1) % 2)
    auto k_round = [&](int it, const char* Qp, const float* Dp, char* Qn, float* Dn) {
      __builtin_amdgcn_s_waitcnt(0x0F70);
      __syncthreads();
      const bool live = live_of(it);
      f32x16 dp[2];
      if (live) {
        const char* Ot = (it & 1) ? o1s : o0s;
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
          dp[mb] = f32x16{};
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) {
            const bf16x8 oa = *reinterpret_cast<const bf16x8*>(Ot + mb * 32 * geo::RB + roff[ks]);
            dp[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(oa, bf[ks], dp[mb], 0, 0, 0);
          }
        }
      }
      // dS of item it - 1 from the P stored in the previous round
      bf16x8 sf[2][2];
      if (live_prev) {
        const f32x4* const pr = ((it & 1) ? p0s : p1s) + wl * PW + lane;
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
          for (int a = 0; a < 4; ++a) {
            const f32x4 e = pr[(mb * 4 + a) * 64];
            const f32x4 d4 = *reinterpret_cast<const f32x4*>(Dp + mb * 32 + a * 8 + hl * 4);
            u32x4& dst = *reinterpret_cast<u32x4*>(&sf[mb][a >> 1]);
            dst[(a & 1) * 2 + 0] = pack_bf16x2(e[0] * (dp_prev[mb][a * 4 + 0] - d4[0]),
                                               e[1] * (dp_prev[mb][a * 4 + 1] - d4[1]));
            dst[(a & 1) * 2 + 1] = pack_bf16x2(e[2] * (dp_prev[mb][a * 4 + 2] - d4[2]),
                                               e[3] * (dp_prev[mb][a * 4 + 3] - d4[3]));
          }
      }
      // the next item's copies go out after the reads of the dO and P stages,
      // which are picked at run time, and before the transposing reads of Q
      if (it + 1 < n_items) issue_k(it + 1, Qn, Dn);
      if (live_prev) {
        // dK^T += Q^T dS
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
          for (int kk = 0; kk < 2; ++kk)
#pragma unroll
            for (int db = 0; db < DB; ++db) {
              const bf16x8 qa = read_tr_operand<D>(Qp, mb * 2 + kk, troff, db);
              acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa, sf[mb][kk], acc[db], 0, 0, 0);
            }
      }
      if (live) {
        dp_prev[0] = dp[0];
        dp_prev[1] = dp[1];
      }
      live_prev = live;
    };
    for (int it = 0;; it += 3) {
      if (it > n_items) break;
      k_round(it, q2s, d2s, q1s, d1s);
      if (it + 1 > n_items) break;
      k_round(it + 1, q0s, d0s, q2s, d2s);
      if (it + 2 > n_items) break;
      k_round(it + 2, q1s, d1s, q0s, d0s);
    }
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);

  if (!wave_live || kw0 + ln >= p.S) return;
  __bf16* row = (krole ? p.dK : p.dV) + (kv_row0 + kw0 + ln) * D;
  const float f = krole ? p.scale : 1.f;
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int a4 = 0; a4 < 4; ++a4) {
      const int d0 = db * 32 + a4 * 8 + hl * 4;
      u32x2 st;
      st[0] = pack_bf16x2(acc[db][a4 * 4 + 0] * f, acc[db][a4 * 4 + 1] * f);
      st[1] = pack_bf16x2(acc[db][a4 * 4 + 2] * f, acc[db][a4 * 4 + 3] * f);
      *reinterpret_cast<u32x2*>(row + d0) = st;
    }
}

template <int D, bool KM>
hipError_t launch_bwd(BwdMfmaParams p, hipStream_t stream) {
  constexpr int NWQ = D == 256 ? 4 : 8;  // dQ waves per workgroup (256: 404 registers, one per SIMD)
  constexpr int NWK = 4;                 // dK/dV waves per workgroup (one per SIMD)
  if ((long long)p.S * D * 2 > 0x7fffffffLL) return hipErrorInvalidValue;
  p.hp = (p.G % 4 == 0 && NWQ % 4 == 0) ? 4 : (p.G % 2 == 0) ? 2 : 1;
  p.n_hsub = p.G / p.hp;
  p.qspan = (NWQ / p.hp) * 32;
  p.n_qtiles = (p.S + p.qspan - 1) / p.qspan;
  const long long nq = (long long)p.n_qtiles * p.B * p.Nkv * p.n_hsub;
  // dK / dV: at head size 128 on two wavefronts per 32 keys with the weights
  // passed through LDS (dkv_pipe_kernel), at head size 64 on one wavefront per
  // 32 keys (dkv_kernel)
  constexpr bool pair = D == 128;
  const long long nk = pair ? (long long)((p.S + 127) / 128) * p.B * p.Nkv
                            : (long long)((p.S + NWK * 32 - 1) / (NWK * 32)) * p.B * p.Nkv;
  if (nq > 0x7fffffffLL || nk > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((dq_kernel<D, NWQ, KM>), dim3((unsigned)nq), dim3(NWQ * 64), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if constexpr (pair)
    hipLaunchKernelGGL((dkv_pipe_kernel<D, KM>), dim3((unsigned)nk), dim3(512), 0, stream, p);
  else
    hipLaunchKernelGGL((dkv_kernel<D, NWK, KM>), dim3((unsigned)nk), dim3(NWK * 64), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

bool backward_bf16_supported(int Dh) { return Dh == 64 || Dh == 128 || Dh == 256; }

hipError_t launch_backward_bf16(const void* Q, const void* K, const void* V, const void* O,
                                const void* dO, const float* LSE, void* dQ, void* dK, void* dV,
                                int B, int Nq, int Nkv, int S, int Dh, int causal, int window,
                                float scale, void* ws, const uint64_t* kbits, hipStream_t stream) {
  const long long rows = (long long)B * Nq * S;
  float* const delta = static_cast<float*>(ws);
  hipError_t e = launch_backward_delta(O, dO, LSE, delta, delta + rows, rows, Dh, 1, stream);
  if (e != hipSuccess) return e;
  BwdMfmaParams p;
  p.Q = static_cast<const __bf16*>(Q);
  p.K = static_cast<const __bf16*>(K);
  p.V = static_cast<const __bf16*>(V);
  p.dO = static_cast<const __bf16*>(dO);
  p.lse2 = delta + rows;
  p.delta = delta;
  p.kbits = kbits;
  p.kwords = key_mask_words(S);
  p.dQ = static_cast<__bf16*>(dQ);
  p.dK = static_cast<__bf16*>(dK);
  p.dV = static_cast<__bf16*>(dV);
  p.B = B;
  p.Nq = Nq;
  p.Nkv = Nkv;
  p.S = S;
  p.causal = causal;
  p.window = window;
  p.c = scale * kLog2e;
  p.scale = scale;
  p.G = Nq / Nkv;
  switch (Dh) {
    case 64: return kbits ? launch_bwd<64, true>(p, stream) : launch_bwd<64, false>(p, stream);
    case 128: return kbits ? launch_bwd<128, true>(p, stream) : launch_bwd<128, false>(p, stream);
    case 256: return kbits ? launch_bwd<256, true>(p, stream) : launch_bwd<256, false>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace attn
