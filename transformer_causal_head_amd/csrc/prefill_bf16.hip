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
//   * Scores are computed transposed, S^T = K Q^T: keys run along MFMA rows
//     (A operand, from LDS), queries along columns (B operand, Q held in VGPRs
//     for the whole kernel).  A lane owns one query column, so the softmax row
//     max and row sum are in-register reductions plus one v_permlane32_swap.
//   * The S^T accumulator layout is exactly the B-operand layout of the PV
//     product O^T = V^T P^T, so P goes from fp32 accumulator to bf16 operand
//     with v_cvt_pk_bf16_f32 and no lane exchange.
//   * K and V tiles (64 keys x 256 B) are copied HBM -> LDS by the buffer DMA
//     path (buffer_load_dwordx4 ... lds): no VGPR staging, one offset per lane,
//     rows past the sequence read as zero (buffer range check), double-
//     buffered and issued one tile ahead, so the copy overlaps the math.  Rows are stored
//     with a GF(2)-linear 16-byte-chunk swizzle that keeps both the 16-byte K
//     reads and the transposing V reads free of bank conflicts.
//   * V stays row-major in LDS; ds_read_b64_tr_b16 transposes it on the way
//     into the V^T operand.
//   * Software pipeline by one tile: the iteration for tile t computes S(t+1)
//     = K(t+1) Q^T, the exponentials of S(t), O += V(t)^T P(t), and the mask
//     and running maximum of S(t+1).  On interior tiles the two MFMA blocks
//     each form one basic block with the VALU work that does not depend on
//     them (the exponentials of t beside QK^T of t+1, the row maxima of t+1
//     beside PV of t), interleaved by scheduling groups, so a wave's own VALU
//     work issues between its MFMAs.  Boundary tiles keep the steps apart and
//     raise the wave's issue priority while it issues its QK^T block.
//   * Lazy rescale: the running maximum moves only when a new score exceeds it
//     by more than TAU (log2 units).  Exponentials stay <= 2^TAU, and the
//     accumulator is rescaled only on those rare moves.  The final O / l and
//     the LSE are unchanged (both use the same reference maximum).
//   * One workgroup = 8 waves (2 per SIMD) of 32 queries sharing every K/V
//     tile: for grouped-query
//     attention the waves take different query heads of one K/V head, so a
//     K/V tile is fetched once per group; for MHA they take consecutive query
//     blocks of one head.
//   * Workgroups run longest-key-range first; with a multiple of 8 (batch,
//     K/V head, head-group) combinations all workgroups of one K/V head land
//     on the same XCD and share its L2.

#include <mutex>
#include <unordered_map>

#include "common.h"
#include "kernels.h"
#include "tiles.h"

namespace attn {

namespace {

constexpr int QB = 1;  // 32-query blocks per wave
constexpr float TAU = 8.f;

// waves per workgroup: two per SIMD while the registers allow it
template <int D>
constexpr int waves_for() { return D == 128 ? 8 : 4; }

struct Params {
  const __bf16* Q;
  const __bf16* K;
  const __bf16* V;
  __bf16* O;
  float* LSE;
  const int32_t* lens;  // keys per sequence in a cache (chunked prefill), or null
  const uint64_t* kbits;  // key-padding mask, one bit per key (kwords words per sequence)
  int kwords;
  int B, Nq, Nkv, S;    // S: query rows per head
  int kv_rows;          // rows per K/V head in memory (S, or the cache capacity)
  int causal, window;
  float c;        // scale * log2(e)
  int G;          // query heads per K/V head
  int hp;         // heads of one group per workgroup
  int qspan;      // queries per workgroup
  int n_qtiles;
  int n_hsub;     // G / hp
  // 0: a workgroup's query blocks are consecutive (qspan rows from qt *
  // qspan).  1: they are strided, block qt + k * n_qtiles for k = 0 ..
  // NW / hp - 1, so that every workgroup of a causal prefill holds early and
  // late queries alike (used when the whole grid runs in one round).
  int strided;
  // query rotation at load (RoPE), table == nullptr: none
  RopeQ rope;
  // causal one-round grids of 4-wave workgroups (two per CU): the first half
  // of the grid takes the query tiles heaviest first, the second half
  // lightest first, so that the two workgroups a CU receives together stream
  // about the same number of key tiles in total
  int zigzag;
  // Work items [0, n_static) go to workgroup blockIdx.x; the rest are drawn at
  // run time from the counters at `queues` (8 per-XCD draw counters, then the
  // count of workgroups done drawing) by the workgroups from n_static on.
  // queues == nullptr: every workgroup takes item blockIdx.x.
  unsigned* queues;
  int n_items, n_static;
};

// The tail of a multi-round grid, drawn at run time.  The dispatcher hands
// workgroup i to XCD i % 8, so every XCD receives the same share of the grid,
// and the XCDs do not run at the same speed.  Queue x holds the tail items
// that XCD x would have received (n_static + x, + 8, ...), heaviest first.  A
// workgroup draws from its own XCD's queue while it lasts (that XCD's L2
// holds the K/V heads of those items) and then from the others', so an XCD
// that runs ahead takes over the last items of a slower one.  Returns the
// item, or -1 once every queue is empty.  The workgroup that draws last
// clears the counters for the next launch that uses them.
__device__ int draw_item(const Params& p) {
  const int x = __builtin_amdgcn_s_getreg(6164) & 7;  // HW_REG_XCC_ID
  const int n = p.n_items - p.n_static;
  int item = -1;
  for (int k = 0; k < 8 && item < 0; ++k) {
    const int q = (x + k) & 7;
    const unsigned j = atomicAdd(p.queues + q, 1u);
    if (j < (unsigned)((n - q + 7) / 8)) item = p.n_static + (int)j * 8 + q;
  }
  // the draws above have returned before the count below is raised
  __asm__ volatile("" ::: "memory");
  if (atomicAdd(p.queues + 8, 1u) == gridDim.x - (unsigned)p.n_static - 1u)
    for (int k = 0; k < 9; ++k) atomicExch(p.queues + k, 0u);
  return item;
}

template <int D, int QB_>
__device__ __forceinline__ void qk_tile(const char* Kt, const int (&koff)[Geo<D>::KS],
                                        const bf16x8 (&qf)[QB_][Geo<D>::KS],
                                        f32x16 (&s)[QB_][2]) {
  constexpr int KS = Geo<D>::KS;
  // raised issue priority while this wave issues its QK^T block: the wave
  // that reaches the matrix core first finishes its block first and moves on
  // to softmax VALU work while the other wave on the SIMD takes the matrix core
  __builtin_amdgcn_s_setprio(1);
#pragma unroll
  for (int qb = 0; qb < QB_; ++qb)
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) s[qb][kb] = f32x16{};
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(Kt + kb * 32 * Geo<D>::RB + koff[ks]);
#pragma unroll
      for (int qb = 0; qb < QB_; ++qb)
        s[qb][kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[qb][ks], s[qb][kb], 0, 0, 0);
    }
  // LDS read-ahead: the K fragments run six reads ahead of their MFMAs (the
  // compiler's own schedule keeps one or two)
  if (QB_ == 1) {
    __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);  // 6 LDS reads
#pragma unroll
    for (int k = 0; k < 2 * KS - 6; ++k) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // 1 MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // 1 LDS read
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 6, 0);
  }
  __builtin_amdgcn_s_setprio(0);
}

template <int D, int QB_>
__device__ __forceinline__ void pv_tile(const char* Vt, const int (&voff)[2][Geo<D>::DB],
                                        const bf16x8 (&pf)[QB_][4],
                                        f32x16 (&o)[QB_][Geo<D>::DB]) {
  constexpr int DB = Geo<D>::DB;
#pragma unroll
  for (int kk = 0; kk < 4; ++kk)
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) i16x4*)(Vt + kk * 16 * Geo<D>::RB + voff[0][db]));
      const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) i16x4*)(Vt + kk * 16 * Geo<D>::RB + voff[1][db]));
      const bf16x8 a = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
      for (int qb = 0; qb < QB_; ++qb)
        o[qb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[qb][kk], o[qb][db], 0, 0, 0);
    }
  // the V^T fragments run four MFMAs ahead of their products
  if (QB_ == 1) {
    __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);  // 8 transposing reads
#pragma unroll
    for (int k = 0; k < 4 * DB - 4; ++k) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // 1 MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // 2 reads
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
  }
}

// The two products without scheduling constraints of their own: the fused
// interior step interleaves them with softmax VALU work.
template <int D, int QB_>
__device__ __forceinline__ void qk_body(const char* Kt, const int (&koff)[Geo<D>::KS],
                                        const bf16x8 (&qf)[QB_][Geo<D>::KS],
                                        f32x16 (&s)[QB_][2]) {
  constexpr int KS = Geo<D>::KS;
#pragma unroll
  for (int qb = 0; qb < QB_; ++qb)
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) s[qb][kb] = f32x16{};
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(Kt + kb * 32 * Geo<D>::RB + koff[ks]);
#pragma unroll
      for (int qb = 0; qb < QB_; ++qb)
        s[qb][kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[qb][ks], s[qb][kb], 0, 0, 0);
    }
}

template <int D, int QB_>
__device__ __forceinline__ void pv_body(const char* Vt, const int (&voff)[2][Geo<D>::DB],
                                        const bf16x8 (&pf)[QB_][4],
                                        f32x16 (&o)[QB_][Geo<D>::DB]) {
  constexpr int DB = Geo<D>::DB;
#pragma unroll
  for (int kk = 0; kk < 4; ++kk)
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const bf16x8 a = read_tr_operand<D>(Vt, kk, voff, db);
#pragma unroll
      for (int qb = 0; qb < QB_; ++qb)
        o[qb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[qb][kk], o[qb][db], 0, 0, 0);
    }
}

// KM: a key-padding mask is given (p.kbits); without it the kernel is
// compiled exactly as if the mask did not exist.
// SK (head size 128, 8 waves, no key mask): the workgroup's key range is split
// in two.  Waves 0-3 take the first half of its key tiles and waves 4-7 the
// second, each with its own LDS stages, for the same 128 query rows (wave w
// and w + 4 share theirs); at the end waves 4-7 hand their running maximum,
// sum and unnormalised output to waves 0-3 through LDS, which merge them by
// the same rescaling identity the online softmax uses.  Used when the grid
// runs in one round: a causal prefill is as long as its heaviest workgroup,
// and the split halves the serial key walk of the heavy query tiles.
template <int D, int NW, bool KM, bool SK = false>
// Head size 128 also runs as 4 waves (one per SIMD) with two workgroups per CU
// (at most 256 registers per lane), for grids that would fill the chip only
// once with 8-wave workgroups.  Head size 64 always runs as 4 waves with three
// workgroups per CU (at most 168 registers; two with a key-padding mask, whose
// extra registers would spill at that bound).
__global__ __launch_bounds__(NW * 64, (D == 128 && NW == 4) ? 2 : ((D == 64 && NW == 4) ? (KM ? 2 : 3) : 1)) void prefill_kernel(Params p) {
  static_assert(!SK || (D == 128 && NW == 8 && !KM), "key split: head size 128, 8 waves, no mask");
  using geo = Geo<D>;
  constexpr int TILE = geo::TILE;
  constexpr int KS = geo::KS;
  constexpr int DB = geo::DB;
  constexpr int QW = 32 * QB;  // queries per wave
  // interior tiles take the fused step (see fused_step) at head size 128
  // without a key mask; the other forms keep every step apart
  constexpr bool FUSED = QB == 1 && D == 128 && !KM;
  // four separate LDS objects, so the compiler can tell that the DMA copies
  // into one stage never alias reads of another (with a key split, each holds
  // one stage per half)
  constexpr int NH = SK ? 2 : 1;
  __shared__ __attribute__((aligned(1024))) char k0s[NH * TILE];
  __shared__ __attribute__((aligned(1024))) char k1s[NH * TILE];
  __shared__ __attribute__((aligned(1024))) char v0s[NH * TILE];
  __shared__ __attribute__((aligned(1024))) char v1s[NH * TILE];

  const int tid = threadIdx.x;
  __shared__ int s_item;
  int bid = blockIdx.x;
  if (p.queues != nullptr && bid >= p.n_static) {
    if (tid == 0) s_item = draw_item(p);
    __syncthreads();
    bid = s_item;
    if (bid < 0) return;  // a spare workgroup that found every queue empty
  }
  const int w_all = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int half = SK ? (w_all >> 2) : 0;  // key half (SK)
  const int w = SK ? (w_all & 3) : w_all;  // query wave; copying wave of its half
  constexpr int NWQ = SK ? 4 : NW;         // query waves (and copying waves per stage)
  const int lane = tid & 63;
  const int ln = lane & 31;
  const int hl = lane >> 5;

  // workgroup -> (q tile, batch, K/V head, head subgroup); heavy tiles first
  const int inner = p.B * p.Nkv * p.n_hsub;
  const int qidx = bid / inner;
  const int qt = !p.causal ? qidx
                 : (p.zigzag && qidx >= p.n_qtiles / 2) ? qidx - p.n_qtiles / 2
                                                        : p.n_qtiles - 1 - qidx;
  int rest = bid % inner;
  const int hsub = rest % p.n_hsub;
  rest /= p.n_hsub;
  const int g = rest % p.Nkv;
  const int b = rest / p.Nkv;

  // Keys of this sequence and the absolute position of query row 0: a plain
  // prefill has S keys and starts at 0; a chunk of S queries against a cache
  // of lens[b] keys sits at the cache's end (positions lens[b] - S ..).
  const int n_keys = p.lens ? max(0, min(p.lens[b], p.kv_rows)) : p.S;
  const int q_off = p.lens ? n_keys - p.S : 0;

  const int head = g * p.G + hsub * p.hp + (w % p.hp);
  const int nblk = NWQ / p.hp;  // query blocks of QW rows per workgroup
  // first query row of this wave (and its position); the workgroup's rows
  // span [q0, q1)
  const int qa_row = p.strided ? (qt + (w / p.hp) * p.n_qtiles) * QW
                               : qt * p.qspan + (w / p.hp) * QW;
  const int qa = q_off + qa_row;
  const int q0 = q_off + (p.strided ? qt * QW : qt * p.qspan);
  const int q1 = q_off + min(p.S, p.strided ? (qt + (nblk - 1) * p.n_qtiles + 1) * QW
                                            : qt * p.qspan + p.qspan);
  const int wq1 = q_off + min(p.S, qa_row + QW);
  const bool wave_live = qa_row < p.S;

  const size_t kv_base = ((size_t)b * p.Nkv + g) * (size_t)p.kv_rows * D;
  const HeadRef Kh = head_ref<D>(p.K + kv_base, n_keys);
  const HeadRef Vh = head_ref<D>(p.V + kv_base, n_keys);
  const size_t q_base = ((size_t)b * p.Nq + head) * (size_t)p.S * D;

  // key range of the workgroup
  const int hi_key = p.causal ? q1 : n_keys;
  const int lo_key = (p.causal && p.window > 0) ? max(0, q0 - p.window + 1) : 0;
  int t_lo = lo_key / BN;
  int t_end = (hi_key + BN - 1) / BN;  // one past the last tile
  if constexpr (KM) {
    // drop the leading and trailing tiles that hold padding keys only (a
    // left- or right-padded batch), so they are neither copied nor waited
    // for: each lane tests one tile's mask word, the ballot gives the ends
    const uint64_t* kr = p.kbits + (size_t)b * p.kwords;
    while (t_lo < t_end) {
      const int t = t_lo + lane;
      const uint64_t bal = __builtin_amdgcn_ballot_w64(t < t_end && kr[t] != 0);
      if (bal) {
        t_lo += __builtin_ctzll(bal);
        break;
      }
      t_lo = min(t_lo + 64, t_end);
    }
    while (t_end > t_lo) {
      const int t = t_end - 1 - lane;
      const uint64_t bal = __builtin_amdgcn_ballot_w64(t >= t_lo && kr[t] != 0);
      if (bal) {
        t_end -= __builtin_ctzll(bal);
        break;
      }
      t_end = max(t_end - 64, t_lo);
    }
    t_lo = __builtin_amdgcn_readfirstlane(t_lo);
    t_end = __builtin_amdgcn_readfirstlane(t_end);
  }
  const int nt = t_end - t_lo;
  // Every wave runs n_it iterations (one barrier each).  Its half of the
  // workgroup copies and computes the nt_h tiles from t_base: all nt tiles,
  // or with a key split the first ceil(nt/2) (waves 0-3) or the rest (4-7).
  const int n_it = SK ? (nt + 1) / 2 : nt;
  const int t_base = t_lo + half * n_it;
  const int nt_h = SK ? (half ? nt - n_it : n_it) : nt;

  char* const K0 = k0s + half * TILE;
  char* const K1 = k1s + half * TILE;
  char* const V0 = v0s + half * TILE;
  char* const V1 = v1s + half * TILE;

  // start the copies first, they overlap the set-up below
  if (nt_h > 0) {
    load_tile<D, NWQ>(Kh, t_base * BN, K0, w, lane);
    load_tile<D, NWQ>(Vh, t_base * BN, V0, w, lane);
  }
  if (nt_h > 1) load_tile<D, NWQ>(Kh, (t_base + 1) * BN, K1, w, lane);

  // Q^T operand fragments: query column ln of block qb, d = 16*ks + 8*hl + i
  bf16x8 qf[QB][KS];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int qrow = min(qa_row + qb * 32 + ln, p.S - 1);
    const bf16x8* src = reinterpret_cast<const bf16x8*>(p.Q + q_base + (size_t)qrow * D + hl * 8);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[qb][ks] = src[ks * 2];
  }
  if (p.rope.table != nullptr) {
    // RoPE at load: this lane holds elements 16*ks + 8*hl + i of its query
    // row; a pair (2m, 2m+1) sits inside one fragment, a pair (m, m + D/2)
    // in fragments ks and ks + KS/2 of the same lane
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const int qrow = min(qa_row + qb * 32 + ln, p.S - 1);
      const int pos = p.rope.positions ? p.rope.positions[(size_t)b * p.S + qrow]
                                       : (p.rope.start ? p.rope.start[b] : q_off) + qrow;
      const float* cs = p.rope.table + (size_t)min(max(pos, 0), p.rope.P - 1) * D;
      if (p.rope.style == 0) {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const f32x4 c = *reinterpret_cast<const f32x4*>(cs + 8 * ks + 4 * hl);
          const f32x4 s = *reinterpret_cast<const f32x4*>(cs + D / 2 + 8 * ks + 4 * hl);
          bf16x8 x = qf[qb][ks];
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const float a = (float)x[2 * k], bb = (float)x[2 * k + 1];
            x[2 * k] = (__bf16)__builtin_fmaf(a, c[k], -bb * s[k]);
            x[2 * k + 1] = (__bf16)__builtin_fmaf(a, s[k], bb * c[k]);
          }
          qf[qb][ks] = x;
        }
      } else {
#pragma unroll
        for (int ks = 0; ks < KS / 2; ++ks) {
          const f32x4 c0 = *reinterpret_cast<const f32x4*>(cs + 16 * ks + 8 * hl);
          const f32x4 c1 = *reinterpret_cast<const f32x4*>(cs + 16 * ks + 8 * hl + 4);
          const f32x4 s0 = *reinterpret_cast<const f32x4*>(cs + D / 2 + 16 * ks + 8 * hl);
          const f32x4 s1 = *reinterpret_cast<const f32x4*>(cs + D / 2 + 16 * ks + 8 * hl + 4);
          bf16x8 x = qf[qb][ks], y = qf[qb][ks + KS / 2];
#pragma unroll
          for (int k = 0; k < 8; ++k) {
            const float c = k < 4 ? c0[k] : c1[k - 4], s = k < 4 ? s0[k] : s1[k - 4];
            const float a = (float)x[k], bb = (float)y[k];
            x[k] = (__bf16)__builtin_fmaf(a, c, -bb * s);
            y[k] = (__bf16)__builtin_fmaf(a, s, bb * c);
          }
          qf[qb][ks] = x;
          qf[qb][ks + KS / 2] = y;
        }
      }
    }
  }

  // LDS byte offsets inside a tile
  int koff[KS];  // K operand: row ln (+32*kb), chunk 2*ks + hl
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) koff[ks] = ln * geo::RB + (((2 * ks + hl) ^ swz<D>(ln)) << 4);
  int voff[2][DB];  // V^T operand through the transposing read
  {
    const int gq = lane >> 4, j = lane & 15;
    const int h = gq >> 1, dpart = gq & 1, ip = j >> 2, u = j & 3;
#pragma unroll
    for (int ih = 0; ih < 2; ++ih) {
      const int r = 8 * ih + 4 * h + ip;
#pragma unroll
      for (int db = 0; db < DB; ++db)
        voff[ih][db] = r * geo::RB + (((4 * db + 2 * dpart + (u >> 1)) ^ swz<D>(r)) << 4) + (u & 1) * 8;
    }
  }

  f32x16 oacc[QB][DB];
  float m_run[QB], l_run[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    m_run[qb] = -INFINITY;
    l_run[qb] = 0.f;
#pragma unroll
    for (int db = 0; db < DB; ++db) oacc[qb][db] = f32x16{};
  }

  // Tile ranges of this wave, as wave-uniform integers: tiles [tl_lo, tl_hi]
  // hold at least one visible (query, key) pair; tiles [tf_lo, tf_hi] hold
  // only visible pairs (no mask needed).  floor division by BN = 64.
  auto fdiv = [](int a) { return a >= 0 ? a / BN : -((-a + BN - 1) / BN); };
  int tl_lo = p.window > 0 ? fdiv(qa - p.window + 1) : -1;
  int tl_hi = p.causal ? fdiv(wq1 - 1) : fdiv(n_keys - 1);
  if (!wave_live) tl_hi = tl_lo - 1;
  int tf_lo = p.window > 0 ? -fdiv(-(wq1 - p.window)) : 0;  // ceil((wq1 - window) / 64)
  int tf_hi = fdiv(n_keys - BN);
  if (p.causal) tf_hi = min(tf_hi, fdiv(qa - (BN - 1)));
  tl_lo = __builtin_amdgcn_readfirstlane(tl_lo);
  tl_hi = __builtin_amdgcn_readfirstlane(tl_hi);
  tf_lo = __builtin_amdgcn_readfirstlane(tf_lo);
  tf_hi = __builtin_amdgcn_readfirstlane(tf_hi);
  // key-padding flags of the tiles.  Lane j holds the mask word of tile
  // kw_base + j; two ballots over those words give, one bit per tile, "holds
  // a real key" (kw_key) and "holds padding" (kw_pad), so the per-tile tests
  // are scalar bit tests.  The window is refilled between runs of KW_RUN
  // tiles, outside the loop that streams the tiles: a load inside it would
  // make the copies of the next tiles wait.  A run of KW_RUN tiles asks about
  // tiles up to one past its last, which the 64-tile window covers.
  uint64_t kw_lane = 0, kw_key = ~0ull, kw_pad = 0;
  int kw_base = t_lo;
  auto refill = [&](int base) {
    kw_base = base;
    const int t = base + lane;
    kw_lane = t < t_end ? p.kbits[(size_t)b * p.kwords + t] : 0;
    kw_key = __builtin_amdgcn_ballot_w64(kw_lane != 0);
    kw_pad = __builtin_amdgcn_ballot_w64(kw_lane != ~0ull);
  };
  if constexpr (KM) refill(t_lo);
  constexpr int KW_RUN = 62;  // even: the two-stage loop below keeps its parity
  auto key_word = [&](int t) -> uint64_t {  // the word itself (boundary tiles only)
    if constexpr (!KM) {
      return ~0ull;
    } else {
      const int j = t - kw_base;
      const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)kw_lane, j);
      const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)(kw_lane >> 32), j);
      return ((uint64_t)hi << 32) | lo;
    }
  };
  // does this wave see any (query, key) pair of tile t?  (a tile of padding
  // keys only is skipped like one the causal mask hides)
  auto live = [&](int t) {
    return t >= tl_lo && t <= tl_hi && (!KM || ((kw_key >> (t - kw_base)) & 1));
  };

  // --- pieces of the per-tile softmax ---
  auto masked = [&](int t) {
    return t < tf_lo || t > tf_hi || (KM && ((kw_pad >> (t - kw_base)) & 1));
  };
  // Visible keys of this lane's query qi form one interval [lo_i, hi_i]
  // (causal: hi_i = qi; window: lo_i = qi - window + 1; keys < S), so a
  // boundary tile's mask is two compares per score.
  int key_lo[QB], key_hi[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int qi = qa + qb * 32 + ln;
    key_hi[qb] = p.causal ? min(qi, n_keys - 1) : n_keys - 1;
    key_lo[qb] = p.window > 0 ? qi - p.window + 1 : 0;
  }
  auto mask_tile = [&](int t, f32x16 (&s)[QB][2]) {
    const int k0 = t * BN + hl * 4;
    // this lane's key flags: bit o of kl is key k0 + o
    const uint64_t kl = key_word(t) >> (hl * 4);
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      // key of register r in block kb: k0 + 32*kb + 8*(r/4) + (r%4)
      const int hi = key_hi[qb] - k0, lo = key_lo[qb] - k0;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int o = kb * 32 + (r >> 2) * 8 + (r & 3);
          bool hide = o > hi || o < lo;
          if (KM) hide = hide || !((kl >> o) & 1);
          if (hide) s[qb][kb][r] = -INFINITY;
        }
    }
  };
  // running max over the tile's (masked) scores; rescale O and l when it
  // moves by more than TAU
  auto max_rescale = [&](f32x16 (&s)[QB][2]) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[qb][kb][r]);
      const float m_cand = xhalf_max(mx) * p.c;
      if (__builtin_amdgcn_ballot_w64(m_cand > m_run[qb] + TAU)) {
        const float m_new = fmaxf(m_run[qb], m_cand);
        const float alpha = exp2_fast(m_run[qb] - (m_new == -INFINITY ? 0.f : m_new));
        m_run[qb] = m_new;
        l_run[qb] *= alpha;
#pragma unroll
        for (int db = 0; db < DB; ++db) oacc[qb][db] *= alpha;
      }
    }
  };
  // P = exp2(S*c - m) rounded to bf16, l += row sum
  auto exp_part = [&](f32x16 (&s)[QB][2], bf16x8 (&pf)[QB][4]) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const float m_use = m_run[qb] == -INFINITY ? 0.f : m_run[qb];
      float rs = 0.f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          u32x4 pk;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const float e0 = exp2_fast(__builtin_fmaf(s[qb][kb][kk * 8 + 2 * j], p.c, -m_use));
            const float e1 = exp2_fast(__builtin_fmaf(s[qb][kb][kk * 8 + 2 * j + 1], p.c, -m_use));
            rs += e0;
            rs += e1;
            pk[j] = pack_bf16x2(e0, e1);
          }
          pf[qb][kb * 2 + kk] = __builtin_bit_cast(bf16x8, pk);
        }
      l_run[qb] += rs;
    }
  };
  // O^T += V^T P^T
  auto exp_pv = [&](f32x16 (&s)[QB][2], const char* Vt) {
    bf16x8 pf[QB][4];
    exp_part(s, pf);
    pv_tile<D, QB>(Vt, voff, pf, oacc);
  };
  // the row maxima of a tile (log2 units), and whether any exceeds the
  // running maximum by more than TAU; apply_max then moves the maximum and
  // rescales (the same arithmetic as max_rescale, split in two)
  auto find_max = [&](f32x16 (&s)[QB][2], float (&m_cand)[QB]) {
    bool any = false;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[qb][kb][r]);
      m_cand[qb] = xhalf_max(mx) * p.c;
      any = any || __builtin_amdgcn_ballot_w64(m_cand[qb] > m_run[qb] + TAU) != 0;
    }
    return any;
  };
  auto apply_max = [&](const float (&m_cand)[QB]) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const float m_new = fmaxf(m_run[qb], m_cand[qb]);
      const float alpha = exp2_fast(m_run[qb] - (m_new == -INFINITY ? 0.f : m_new));
      m_run[qb] = m_new;
      l_run[qb] *= alpha;
#pragma unroll
      for (int db = 0; db < DB; ++db) oacc[qb][db] *= alpha;
    }
  };
  // One interior step in two phases, each a single basic block: the QK^T
  // block of tile t+1 on the matrix cores while the VALU forms P(t) (four
  // VALU instructions per MFMA, the K fragments six reads ahead); then the PV
  // block of tile t while the VALU finds the row maxima of tile t+1 (two per
  // MFMA, the V^T fragments four MFMAs ahead).  The rare rescale comes last.
  // The same operations in the same order as the separate steps, so the
  // results are bit-identical.
  auto fused_step = [&](const char* Kt, const char* Vt, f32x16 (&sc)[QB][2], f32x16 (&sn)[QB][2]) {
    bf16x8 pf[QB][4];
    qk_body<D, QB>(Kt, koff, qf, sn);
    exp_part(sc, pf);
    __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);  // 6 LDS reads
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // 1 MFMA
      __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);  // 4 VALU
      if (k < 10) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // 1 LDS read
    }
    __builtin_amdgcn_sched_barrier(0);
    pv_body<D, QB>(Vt, voff, pf, oacc);
    float m_cand[QB];
    const bool need = find_max(sn, m_cand);
    __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);  // 8 transposing reads
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // 1 MFMA
      __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);  // 2 VALU
      if (k < 12) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // 2 reads
    }
    __builtin_amdgcn_sched_barrier(0);
    if (need) apply_max(m_cand);
  };




  // The pipelined loop: iteration i (tile t = t_lo + i) holds S(t) in
  // registers; K(t+1) and V(t) are in LDS, and the copies of K(t+2) and
  // V(t+1) are issued at its top.  The iteration computes S(t+1) (QK^T), P(t)
  // (exponentials, row sums) and O += V(t)^T P(t).  With the fused step, S(t)
  // arrives masked and with its running maximum applied, and the iteration
  // ends with the mask and maximum of tile t+1 (the fused step pairs them
  // with the PV block).  Without it the mask and maximum of tile t come first,
  // right after S(t+1) is issued: they need only S(t), so the VALU runs them
  // while the matrix cores work on S(t+1).  Placing them after PV(t) instead
  // (as the fused form must) made one-wave-per-SIMD head size 256 16 % slower
  // and head size 64 and key-padded prefill 2-3 % slower.
  f32x16 sa[QB][2], sb[QB][2];
  wait_dma();
  __syncthreads();
  if (nt_h > 0 && live(t_base)) {
    qk_tile<D, QB>(K0, koff, qf, sa);
    if constexpr (FUSED) {
      if (masked(t_base)) mask_tile(t_base, sa);
      max_rescale(sa);
    }
  }
  auto iteration = [&](int i, f32x16 (&s_cur)[QB][2], f32x16 (&s_next)[QB][2], bool fused) {
    const int t = t_base + i;
    char* const Kcur = (i & 1) ? K1 : K0;   // holds K(t), free after the barrier
    char* const Knext = (i & 1) ? K0 : K1;  // holds K(t+1)
    char* const Vcur = (i & 1) ? V1 : V0;   // holds V(t)
    char* const Vnext = (i & 1) ? V0 : V1;  // gets V(t+1)
    wait_dma();
    __syncthreads();
    if (i + 2 < nt_h) load_tile<D, NWQ>(Kh, (t + 2) * BN, Kcur, w, lane);
    if (i + 1 < nt_h) load_tile<D, NWQ>(Vh, (t + 1) * BN, Vnext, w, lane);
    if (fused) {
      fused_step(Knext, Vcur, s_cur, s_next);
    } else {
      const bool nx = i + 1 < nt_h && live(t + 1);
      if (nx) qk_tile<D, QB>(Knext, koff, qf, s_next);
      if constexpr (FUSED) {
        if (i < nt_h && live(t)) exp_pv(s_cur, Vcur);
        if (nx) {
          if (masked(t + 1)) mask_tile(t + 1, s_next);
          max_rescale(s_next);
        }
      } else {
        if (i < nt_h && live(t)) {
          if (masked(t)) mask_tile(t, s_cur);
          max_rescale(s_cur);
          exp_pv(s_cur, Vcur);
        }
      }
    }
  };

  // The loop runs in pairs of iterations, so that stages and score buffers
  // alternate with a static pattern.
  int i = 0;
  if constexpr (KM) {
    for (int c = 0; c < nt; c += KW_RUN) {
      if (c > 0) refill(t_lo + c);
      const int c_end = min(nt, c + KW_RUN);
      for (; i + 1 < c_end; i += 2) {
        iteration(i, sa, sb, false);
        iteration(i + 1, sb, sa, false);
      }
    }
  } else {
    // This wave's fused iterations: tile t live, tile t+1 live and unmasked,
    // i.e. t in [max(tl_lo, tf_lo - 1), min(tl_hi, tf_hi - 1)].  They run in a
    // loop of their own (one loop body holding both step forms would not fit
    // the registers), from the first even iteration of the range; every loop
    // runs one barrier per iteration, so the waves stay in step.
    const int f_lo = max(tl_lo, tf_lo - 1) - t_base;
    const int f_hi = min(min(tl_hi, tf_hi - 1) - t_base, nt_h - 2);
    const int fa = (max(f_lo, 0) + 1) & ~1;
    const int npairs = (FUSED && f_hi >= fa) ? (f_hi - fa + 1) / 2 : 0;
    const int a_end = npairs > 0 ? fa : 0;
    for (; i < a_end; i += 2) {
      iteration(i, sa, sb, false);
      iteration(i + 1, sb, sa, false);
    }
    for (int q = 0; q < npairs; ++q, i += 2) {
      iteration(i, sa, sb, true);
      iteration(i + 1, sb, sa, true);
    }
    for (; i + 1 < n_it; i += 2) {
      iteration(i, sa, sb, false);
      iteration(i + 1, sb, sa, false);
    }
  }
  if (i < n_it) iteration(i, sa, sb, false);

  if constexpr (SK) {
    // merge the two key halves: every copy has landed and every stage read
    // once all waves pass this barrier (the last iteration issues none)
    __syncthreads();
    // wave w + 4's unnormalised output (64 values per lane) at value-major
    // float offsets in k0s (query waves 0, 1) or k1s (2, 3); its (m, l) in v0s
    float* xo = reinterpret_cast<float*>((w < 2 ? k0s : k1s) + (w & 1) * TILE);
    float* xml = reinterpret_cast<float*>(v0s) + w * 128;
    if (half) {
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) xo[(db * 16 + r) * 64 + lane] = oacc[0][db][r];
      xml[lane] = m_run[0];
      xml[64 + lane] = l_run[0];
    }
    __syncthreads();
    if (half) return;
    const float mb = xml[lane], lb = xml[64 + lane];
    const float M = fmaxf(m_run[0], mb);
    const float Mu = M == -INFINITY ? 0.f : M;
    const float ra = exp2_fast(m_run[0] - Mu), rb = exp2_fast(mb - Mu);
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        oacc[0][db][r] = __builtin_fmaf(rb, xo[(db * 16 + r) * 64 + lane], oacc[0][db][r] * ra);
    l_run[0] = __builtin_fmaf(rb, lb, l_run[0] * ra);
    m_run[0] = M;
  }

  // Epilogue through LDS (head size 128, and head size 64 with a key mask):
  // each live wave stages its 32 output rows in LDS in the tiles' swizzled
  // layout, so that it stores them as whole 16-byte chunks of consecutive
  // rows instead of 8-byte pieces of 32 rows at a time.  Without a key split
  // every wave is done with the stages once all pass a barrier, and wave w
  // takes half w % 2 of stage w / 2; with one, each query wave reuses its own
  // merge buffer, which no other wave reads.  The unmasked head-size-64 form
  // would spill at its register bound with it, and at head size 256 (one
  // workgroup per CU) the barrier costs more than the wider stores gain.
  if constexpr (QB == 1 && (D == 128 || (D == 64 && KM))) {
    char* ob;
    if constexpr (SK) {
      ob = (w < 2 ? k0s : k1s) + (w & 1) * TILE;
    } else {
      __syncthreads();
      char* const stage = w_all < 2 ? k0s : w_all < 4 ? k1s : w_all < 6 ? v0s : v1s;
      ob = stage + (w_all & 1) * (TILE / 2);
    }
    if (!wave_live) return;
    const float l_tot = xhalf_sum(l_run[0]);
    const float inv = (KM && l_tot == 0.f) ? 0.f : 1.f / l_tot;
    const int zr = swz<D>(ln);
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4) {
        u32x2 st;
        st[0] = pack_bf16x2(oacc[0][db][a4 * 4 + 0] * inv, oacc[0][db][a4 * 4 + 1] * inv);
        st[1] = pack_bf16x2(oacc[0][db][a4 * 4 + 2] * inv, oacc[0][db][a4 * 4 + 3] * inv);
        *reinterpret_cast<u32x2*>(ob + ln * geo::RB + (((db * 4 + a4) ^ zr) << 4) + hl * 8) = st;
      }
    constexpr int RPI = 1024 / geo::RB;  // rows per 16-byte-per-lane instruction
#pragma unroll
    for (int i = 0; i < 32 / RPI; ++i) {
      const int r = i * RPI + lane / geo::NC, c = lane % geo::NC;
      const u32x4 v = *reinterpret_cast<const u32x4*>(ob + r * geo::RB + ((c ^ swz<D>(r)) << 4));
      if (qa_row + r < p.S) *reinterpret_cast<u32x4*>(p.O + q_base + (size_t)(qa_row + r) * D + c * 8) = v;
    }
    const int qi = qa_row + ln;
    if (p.LSE != nullptr && hl == 0 && qi < p.S)
      p.LSE[((size_t)b * p.Nq + head) * p.S + qi] = (m_run[0] + __log2f(l_tot)) * kLn2;
    return;
  }
  if (!wave_live) return;
  // epilogue: O = O_acc / l, LSE = (m + log2 l) * ln 2
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int qi = qa_row + qb * 32 + ln;  // query row
    const float l_tot = xhalf_sum(l_run[qb]);
    if (qi >= p.S) continue;
    // with a key-padding mask a row may see no key at all: O = 0, LSE = -inf
    const float inv = (KM && l_tot == 0.f) ? 0.f : 1.f / l_tot;
    __bf16* orow = p.O + q_base + (size_t)qi * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
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

// Counters of the run-time drawn grid tails: kQueueSets sets of 16 words on
// each device that runs the library (9 used; the rest keep sets on separate
// 64-byte lines), one set per stream that launches such grids.  Kernels of
// one stream run one after another and the last drawing workgroup of each
// launch clears its set, so a set never has two users at once.
// hipStreamDestroy waits for the stream's work, so a stream created later at
// the same handle cannot overlap a launch of the old one.  Launches into the
// per-thread default stream (one handle, several streams), into a stream
// being captured into a graph (a replay could overlap any launch), into a
// stream of another device, and from streams beyond the last set take the
// fixed order instead.
constexpr int kQueueSets = 256;
static __device__ __align__(256) unsigned prefill_queues[kQueueSets * 16];

namespace {
constexpr int kQueueDevices = 64;
constexpr int kSpareGroups = 512;  // extra workgroups of a drawn grid: 64 per XCD

std::mutex queue_mu;
unsigned* queue_base[kQueueDevices];  // device address of prefill_queues
std::unordered_map<hipStream_t, int> queue_set[kQueueDevices];

// The counter set of `stream` on device dev, or null for the fixed order.
unsigned* stream_queues(int dev, hipStream_t stream) {
  if (dev < 0 || dev >= kQueueDevices || stream == hipStreamPerThread) return nullptr;
  hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(stream, &cap) != hipSuccess || cap != hipStreamCaptureStatusNone)
    return nullptr;
  int sdev = -1;
  if (hipStreamGetDevice(stream, &sdev) != hipSuccess || sdev != dev) return nullptr;
  std::lock_guard<std::mutex> lock(queue_mu);
  if (queue_base[dev] == nullptr) {
    void* a = nullptr;
    if (hipGetSymbolAddress(&a, HIP_SYMBOL(prefill_queues)) != hipSuccess) return nullptr;
    queue_base[dev] = static_cast<unsigned*>(a);
  }
  auto& sets = queue_set[dev];
  auto it = sets.find(stream);
  if (it == sets.end()) {
    if (sets.size() >= (size_t)kQueueSets) return nullptr;
    it = sets.emplace(stream, (int)sets.size()).first;
  }
  return queue_base[dev] + 16 * it->second;
}

template <int D>
hipError_t launch_prefill(const void* Q, const void* K, const void* V, void* O, float* LSE,
                          int B, int Nq, int Nkv, int S, int kv_rows, const int32_t* lens,
                          const uint64_t* kbits, int causal, int window, float scale,
                          hipStream_t stream, const RopeQ* rope) {
  constexpr int NW = waves_for<D>();
  // one head of K (or V) is addressed through a 31-bit buffer range
  if ((long long)kv_rows * D * 2 > 0x7fffffffLL || (long long)S * D * 2 > 0x7fffffffLL)
    return hipErrorInvalidValue;
  Params p;
  p.Q = static_cast<const __bf16*>(Q);
  p.K = static_cast<const __bf16*>(K);
  p.V = static_cast<const __bf16*>(V);
  p.O = static_cast<__bf16*>(O);
  p.LSE = LSE;
  p.lens = lens;
  p.kbits = kbits;
  p.kwords = key_mask_words(kv_rows);
  p.B = B;
  p.Nq = Nq;
  p.Nkv = Nkv;
  p.S = S;
  p.kv_rows = kv_rows;
  p.causal = causal;
  p.window = window;
  p.c = scale * kLog2e;
  p.G = Nq / Nkv;
  p.rope = rope ? *rope : RopeQ{nullptr, 0, nullptr, nullptr, 0};
  int dev = 0, n_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    n_cu = 0;
  // query blocks per workgroup and the grid for nw waves per workgroup
  auto geometry = [&](int nw) {
    p.hp = (p.G % 4 == 0 && nw % 4 == 0) ? 4 : (p.G % 2 == 0) ? 2 : 1;
    p.n_hsub = p.G / p.hp;
    p.qspan = (nw / p.hp) * 32 * QB;
    p.n_qtiles = (S + p.qspan - 1) / p.qspan;
    return (long long)p.n_qtiles * B * Nkv * p.n_hsub;
  };
  long long nblocks = geometry(NW);
  // A plain prefill whose grid of 8-wave workgroups fills the chip at most
  // once runs as 4-wave workgroups, two per CU: twice the workgroups, and the
  // two on a CU do not wait at each other's barriers, so one's softmax
  // overlaps the other's matrix work.  Each wave computes the same rows
  // either way.  (A chunk against a long cache stays on 8 waves: there the
  // second copy of every K/V tile per CU costs more than the overlap gains.)
  const bool small = D == 128 && NW == 8 && lens == nullptr && n_cu > 0 &&
                     nblocks <= n_cu;
  if (small) nblocks = geometry(4);
  // A causal one-round grid without a key mask whose heads hold at least 4096
  // keys splits each workgroup's key range between two sets of four waves
  // instead (SK form: the grid of the 4-wave form, 8 waves per workgroup, so
  // it runs in two rounds).  The split halves the serial key walk of the
  // heaviest workgroups; on shorter heads the second round's start-up costs
  // more than that saves.
  const bool split = small && causal && kbits == nullptr && S >= 4096;
  if (nblocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  // A causal prefill whose grid runs in one round lasts as long as its
  // heaviest workgroup: with consecutive query blocks the last tile of a head
  // sees n_qtiles times the keys of the first.  Strided blocks give every
  // workgroup the same mix (a window keeps them consecutive: strided blocks
  // would make each workgroup stream most of the sequence).  The 4-wave
  // form is faster with consecutive blocks.
  p.strided = !small && causal && window == 0 && lens == nullptr && p.n_qtiles > 1 &&
              nblocks <= n_cu;
  p.zigzag = small && !split && causal && (p.n_qtiles % 2 == 0);
  // A causal prefill without a window whose grid runs four or more rounds
  // draws its last quarter of items at run time.  Those are the lightest
  // query tiles (short key prefixes), so an XCD that takes one over from
  // another fetches little that its L2 does not hold.  With a window, a
  // cache or no mask the items cost about the same, each stolen one streams
  // its whole key range from HBM, and the drawn tail measured 1 % slower on
  // the GQA window workload.  On grids under four rounds one atomic per
  // drawing workgroup costs more than the balance gains.
  p.queues = nullptr;
  p.n_items = p.n_static = (int)nblocks;
  if (!small && causal && window == 0 && lens == nullptr && n_cu > 0 && nblocks >= 4LL * n_cu &&
      nblocks + kSpareGroups <= 0x7fffffffLL) {
    p.queues = stream_queues(dev, stream);
    if (p.queues) {
      p.n_static = (p.n_items - p.n_items / 4) & ~7;  // a multiple of 8: XCDs keep their items
      nblocks += kSpareGroups;
    }
  }
  if constexpr (D == 128 && NW == 8) {
    if (split) {
      hipLaunchKernelGGL((prefill_kernel<D, 8, false, true>), dim3((unsigned)nblocks), dim3(512), 0,
                         stream, p);
      return hipGetLastError();
    }
    if (small) {
      if (kbits)
        hipLaunchKernelGGL((prefill_kernel<D, 4, true>), dim3((unsigned)nblocks), dim3(256), 0,
                           stream, p);
      else
        hipLaunchKernelGGL((prefill_kernel<D, 4, false>), dim3((unsigned)nblocks), dim3(256), 0,
                           stream, p);
      return hipGetLastError();
    }
  }
  if (kbits) {
    hipLaunchKernelGGL((prefill_kernel<D, NW, true>), dim3((unsigned)nblocks), dim3(NW * 64), 0,
                       stream, p);
  } else {
    hipLaunchKernelGGL((prefill_kernel<D, NW, false>), dim3((unsigned)nblocks), dim3(NW * 64), 0,
                       stream, p);
  }
  return hipGetLastError();
}

}  // namespace

bool prefill_bf16_supported(int Dh) { return Dh == 64 || Dh == 128 || Dh == 256; }

hipError_t launch_prefill_bf16(const void* Q, const void* K, const void* V, void* O, float* LSE,
                               int B, int Nq, int Nkv, int S, int Dh, int kv_rows,
                               const int32_t* lens, const uint64_t* kbits, int causal, int window,
                               float scale, hipStream_t stream, const RopeQ* rope) {
  switch (Dh) {
    case 64:
      return launch_prefill<64>(Q, K, V, O, LSE, B, Nq, Nkv, S, kv_rows, lens, kbits, causal,
                                window, scale, stream, rope);
    case 128:
      return launch_prefill<128>(Q, K, V, O, LSE, B, Nq, Nkv, S, kv_rows, lens, kbits, causal,
                                 window, scale, stream, rope);
    case 256:
      return launch_prefill<256>(Q, K, V, O, LSE, B, Nq, Nkv, S, kv_rows, lens, kbits, causal,
                                 window, scale, stream, rope);
    default:
      return hipErrorInvalidValue;
  }
}

}  // namespace attn
