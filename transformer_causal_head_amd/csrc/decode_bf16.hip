// KV-cache decode step, bf16 cache, head size 64, 128 or 256, split over the
// key axis.
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
//     the prefill kernel: S^T = K q^T (keys on M, up to 16 query heads on N),
//     and O^T = V^T P^T, whose B operand is the S^T accumulator layout.  K is
//     read from LDS in operand layout and V is transposed on its way out by
//     ds_read_b64_tr_b16; row-XOR swizzles keep both conflict free.  More than
//     16 query heads per K/V head (up to 32: MQA) take a second N block that
//     reuses every K and V fragment.
//   * Even split (at most 64 sequences, grids of at least 512 chunk items):
//     the visible steps of all (sequence, K/V head) pairs are laid end to end
//     and cut into ranges, one per wavefront of a fixed grid of 1024 (four per
//     CU; 512 with 16 or more query heads per K/V head), weighted by XCD
//     parity.  Per-sequence chunks leave a grid of mixed-length items (every
//     sequence's last chunk is short, sequences end at different chunks) that
//     the dispatcher spreads unevenly when they all run at once; equal ranges
//     finish together.  A range crossing a (sequence, K/V head) boundary
//     writes one partial per piece, piece (segment s, wavefront w) to slot
//     s + w, so the merge finds a segment's pieces in one contiguous run.
//   * Every K and V byte is read once per K/V head and shared by its G query
//     heads.  Rows at or past the length are never used: copy addresses clamp
//     to the last valid row and those keys get probability 0.

#include <algorithm>
#include <mutex>

#include "common.h"
#include "kernels.h"

namespace attn {

namespace {

constexpr int STEP = 32;             // keys per pipeline step
constexpr float TAU = 8.f;
constexpr int kNonTemporal = 2;      // cache-policy bit of the copy instructions
// even split: wavefronts of the partial grid -- four per CU, all resident at
// once (more would leave a second round for the rest); two per CU with 16 or
// more query heads per K/V head, whose steps carry twice the matrix work and
// whose partials cost G (Dh + 2) floats per piece
constexpr int kEvenWaves = 1024;
constexpr int kEvenWavesWide = 512;
// even split: range weights of the wavefronts on even and odd XCDs.  The
// dispatcher hands wavefront w to XCD w % 8, and streaming decode runs 7-10 %
// slower on the odd XCDs, so their ranges are shorter (64 : 55).
constexpr long long kWeightEven = 64, kWeightOdd = 55;
// merge: partial outputs a wavefront requests at a time
constexpr int kMergeBatch = 16;
// shortest chunk (and shortest even-split range): 640 keys, 224 with 16 or
// more query heads per K/V head -- shorter ones cost more in partials to
// write and merge than their extra parallelism gains
constexpr int kFloorKeys = 640;
constexpr int kFloorKeysWide = 224;
// even split with a key-padding mask: the 32-key flag words of a piece's steps
// are copied into LDS when the piece starts (4 KB per wavefront), so a piece
// spans at most kMaskWords - 2 steps; the host takes the even split only when
// every range fits
constexpr int kMaskWords = 1024;

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) char lds_char;
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) const bf16x8 lds_bf16x8;

// Geometry for head size D: a row is RB = 2*D bytes (NC 16-byte chunks); a
// step's rows fill STAGE bytes = NPIECE copies of 1 KB (RP rows each); QK^T
// takes KS 32-wide slices of the head, PV yields DB 16-wide output blocks.
template <int D>
struct DGeo {
  static constexpr int RB = 2 * D;
  static constexpr int NC = D / 8;
  static constexpr int STAGE = STEP * RB;
  static constexpr int NPIECE = STAGE / 1024;
  static constexpr int RP = 1024 / RB;
  static constexpr int KS = D / 32;
  static constexpr int DB = D / 16;
};

struct DecParams {
  const __bf16* q;
  const __bf16* K;
  const __bf16* V;
  const int32_t* lens;
  const uint64_t* kbits;  // key-padding mask, one bit per cache slot (kwords words per sequence)
  int kwords;
  // decode with append: the new token's K and V rows ([B, Nkv, D]) go to
  // cache row slot[b]; the chunk holding that row reads them from here
  const __bf16* knew;
  const __bf16* vnew;
  const int32_t* slot;
  __bf16* Kw;  // the caches, written
  __bf16* Vw;
  __bf16* O;
  float* LSE;
  float* ws_o;    // [B, Nkv, n_slots, G, D] unnormalised partial outputs
  float* ws_ml;   // [B, Nkv, n_slots, G, 2]  (m in log2 units, l)
  int* ws_seg;    // even split: [B, Nkv, 2] first and last range of each segment
  int B, Nq, Nkv, G, Tcap;
  int n_slots;    // chunks that can hold visible keys, per (sequence, K/V head)
  int ch;         // keys per chunk (a multiple of STEP)
  int window;     // > 0: only keys lens[b] - window .. lens[b] - 1 are visible
  int mw;         // merge: wavefronts per (sequence, query head) row, 1 to 16
  int ev_nw;      // even split: wavefronts of the partial grid (0: one per chunk)
  int ev_min;     // even split: fewest steps per wavefront range
  float c;        // scale * log2(e)
  RopeQ rope;     // query rotation at load (RoPE); table == nullptr: none
};

// 16-byte chunk c of K row r sits at chunk position c ^ kswz(r) (the operand
// reads take one chunk of 16 consecutive rows), of V row r at c ^ vswz(r)
// (keeps the transposing reads conflict free).  GF(2)-linear in the row bits,
// checked exhaustively against both read patterns under 32 and 64 banks.
template <int D>
__device__ __forceinline__ int kswz(int r) {
  if constexpr (D == 64) return (r & 7) ^ ((r >> 3) & 1);
  else return r & 15;
}
template <int D>
__device__ __forceinline__ int vswz(int r) {
  if constexpr (D == 64) return ((r & 1) << 1) ^ (((r >> 1) & 1) << 2) ^ (((r >> 2) & 1) << 1);
  else return ((r << 1) & 14) | ((r >> 3) & 1);
}

// Even split: lane j < B describes sequence j -- its visible length n, first
// visible key lo, and ns, the steps of 32 keys that hold visible keys (step
// indices lo/32 .. (n-1)/32) -- and incl is the inclusive prefix sum of ns
// over the lanes.  Segment (b, g) covers global steps Nkv*(incl_b - ns_b) +
// g*ns_b onwards; tot is the total, nwe the wavefronts in use (ranges of at
// least p.ev_min steps, at most p.ev_nw of them).  Both kernels compute it the
// same way from the lengths, so they agree on every range.
struct EvenTable {
  int n, lo, ns, incl, nwe;
  long long tot;
};
__device__ __forceinline__ EvenTable even_table(const DecParams& p, int lane) {
  EvenTable t = {0, 0, 0, 0, 1, 0};
  if (lane < p.B) {
    t.n = max(0, min(p.lens[lane], p.Tcap));
    t.lo = p.window > 0 ? max(0, t.n - p.window) : 0;
    t.ns = t.n > 0 ? (t.n - 1) / STEP - t.lo / STEP + 1 : 0;
  }
  int v = t.ns;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int u = __shfl_up(v, o, 64);
    if (lane >= o) v += u;
  }
  t.incl = v;
  t.tot = (long long)__shfl(v, 63, 64) * p.Nkv;
  t.nwe = (int)max(1LL, min((long long)p.ev_nw, t.tot / p.ev_min));
  return t;
}
// weight of wavefronts 0 .. w-1 (even w on even XCDs, odd w on odd ones)
__device__ __forceinline__ long long range_weight(int w) {
  return kWeightEven * ((w + 1) >> 1) + kWeightOdd * (w >> 1);
}
// first global step of wavefront w's range (w = nwe: the total)
__device__ __forceinline__ long long range_start(const EvenTable& t, int w) {
  return t.tot * range_weight(w) / range_weight(t.nwe);
}

// Rows [k0, k0+32) of one head -> one LDS stage: NPIECE copies of RP whole
// rows, lane i of a copy landing at byte 16*i of its 1 KB piece.  Rows past
// `last` are clamped to it.
template <int D, bool IS_K>
__device__ __forceinline__ void load_rows(const __bf16* head, int k0, int last, lds_char* stage,
                                          int lane) {
  using g = DGeo<D>;
#pragma unroll
  for (int j = 0; j < g::NPIECE; ++j) {
    const int r = j * g::RP + lane / g::NC;
    const int c = (lane % g::NC) ^ (IS_K ? kswz<D>(r) : vswz<D>(r));
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

// NB blocks of 16 query heads per K/V head (G <= 16 * NB).  KM: a key-padding
// mask is given (p.kbits); without it the kernel is compiled as if it did not
// exist.  APP: the new token's K and V rows are appended in the same launch.
// RQ: the queries are rotated at load (RoPE, p.rope).  EV: even split (the
// grid is p.ev_nw wavefronts, each taking one range of the steps of all
// (sequence, K/V head) pairs laid end to end); chunk mode otherwise.
template <int D, int NB, bool KM, bool APP = false, bool RQ = false, bool EV = false>
__global__ __launch_bounds__(64) void decode_partial_kernel(DecParams p) {
  using geo = DGeo<D>;
  constexpr int STAGE = geo::STAGE;
  constexpr int KS = geo::KS;
  constexpr int DB = geo::DB;
  constexpr int PER_STEP = 2 * geo::NPIECE;  // copy instructions per step (K and V)
  // four separate LDS objects, so the compiler can tell that a copy into one
  // stage never aliases the reads of another
  __shared__ __attribute__((aligned(1024))) char k0s[STAGE];
  __shared__ __attribute__((aligned(1024))) char k1s[STAGE];
  __shared__ __attribute__((aligned(1024))) char v0s[STAGE];
  __shared__ __attribute__((aligned(1024))) char v1s[STAGE];
  // even split with a key mask: flag word of step s at kwl[s - kw_base]
  __shared__ __attribute__((aligned(16))) uint32_t kwl[(KM && EV) ? kMaskWords : 1];
  int kw_base = 0;

  lds_char* const K0 = (lds_char*)k0s;
  lds_char* const K1 = (lds_char*)k1s;
  lds_char* const V0 = (lds_char*)v0s;
  lds_char* const V1 = (lds_char*)v1s;

  const int lane = threadIdx.x & 63;
  // The work item: steps s0 .. nsteps-1 of 32 keys from key c0 of (sequence b,
  // K/V head g), keys lo .. n-1 visible, rows clamped to `last`; its partial
  // goes to slot `slot` (G rows of the workspace from slot * G).
  int b, g, n, lo, c0, s0 = 0, nsteps = 0, last = 0;
  size_t slot;
  EvenTable tab;
  long long ev_a = 0, ev_e = 0;  // even split: this wavefront's global steps still to run
  int ev_w = 0;
  // append: lane l < NC holds 16 bytes of the new K row, NC <= l < 2 NC of the
  // new V row (loaded before any copy, so the copy waits cover it).  One
  // `writer` wavefront per (sequence, K/V head) -- chunk 0, or the wavefront
  // whose range starts the segment -- writes them to cache row slot[b]; the
  // work item that holds that row (if the query sees it) copies the cache as
  // usual and then overwrites that row of its LDS stage with them, so no
  // wavefront uses the row being written.
  constexpr int NCH = D / 8;
  u32x4 new_row = {};
  int alt_row = -1;
  bool writer = false;
  // the new rows of (b, g); the item's keys run from k_lo to k_hi
  auto load_new = [&](int k_lo, int k_hi) {
    if constexpr (APP) {
      const size_t nrow = ((size_t)b * p.Nkv + g) * D;
      if (lane < NCH)
        new_row = *reinterpret_cast<const u32x4*>(p.knew + nrow + lane * 8);
      else if (lane < 2 * NCH)
        new_row = *reinterpret_cast<const u32x4*>(p.vnew + nrow + (lane - NCH) * 8);
      const int sl = p.slot[b];
      alt_row = sl >= max(lo, k_lo) && sl < min(n, k_hi) ? sl : -1;
    }
  };
  auto write_new_row = [&]() {
    if constexpr (APP) {
      const int sl = p.slot[b];
      if (writer && sl >= 0 && sl < p.Tcap && lane < 2 * NCH) {
        __bf16* dst = (lane < NCH ? p.Kw : p.Vw) + (((size_t)b * p.Nkv + g) * p.Tcap + sl) * D;
        *reinterpret_cast<u32x4*>(dst + (lane % NCH) * 8) = new_row;
      }
    }
  };

  // even split: take the segment (b, g) from its step s_in to the end of the
  // segment or of this wavefront's range
  auto enter = [&](int s_in) {
    n = __builtin_amdgcn_readlane(tab.n, b);
    lo = __builtin_amdgcn_readlane(tab.lo, b);
    const int ns_b = __builtin_amdgcn_readlane(tab.ns, b);
    const int cnt = (int)min((long long)(ns_b - s_in), ev_e - ev_a);
    c0 = 0;
    s0 = lo / STEP + s_in;
    nsteps = s0 + cnt;
    // rows past the piece clamp to its last row: the copies issued past its
    // end then re-read one row instead of the next wavefront's keys
    last = min(n, nsteps * STEP) - 1;
    slot = (size_t)b * p.Nkv + g + ev_w;
    ev_a += cnt;
    writer = s_in == 0;
    // the merge reads which ranges hold the segment's first and last steps
    if (lane == 0) {
      int* seg = p.ws_seg + 2 * ((size_t)b * p.Nkv + g);
      if (s_in == 0) seg[0] = ev_w;
      if (s_in + cnt == ns_b) seg[1] = ev_w;
    }
    load_new(s0 * STEP, nsteps * STEP);
    if constexpr (KM) {
      // flag words of steps s0 .. nsteps-1 (two per 64-bit mask word, starting
      // at an even step), 64 lanes x 4 bytes per copy; words past the
      // sequence's mask read as zero
      kw_base = s0 & ~1;
      const int nw = min(nsteps - kw_base, kMaskWords);
      const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
          (void*)(p.kbits + (size_t)b * p.kwords), (short)0, p.kwords * 8, 0x00020000);
      for (int i = 0; i < nw; i += 64)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(kwl + i), 4, (kw_base + i + lane) * 4, 0,
                                                 0, 0);
    }
  };
  if constexpr (EV) {
    tab = even_table(p, lane);
    ev_w = blockIdx.x;
    if constexpr (APP) {
      // a sequence with no visible key has no range: wavefront 0 writes its
      // new rows (nothing reads them in this launch)
      if (ev_w == 0) {
        for (uint64_t zb = __builtin_amdgcn_ballot_w64(lane < p.B && tab.ns == 0); zb; zb &= zb - 1) {
          const int bz = __builtin_ctzll(zb);
          const int sl = p.slot[bz];
          if (sl < 0 || sl >= p.Tcap) continue;
          for (int gz = 0; gz < p.Nkv; ++gz) {
            if (lane < 2 * NCH) {
              const size_t head = (size_t)bz * p.Nkv + gz;
              const u32x4 v = *reinterpret_cast<const u32x4*>((lane < NCH ? p.knew : p.vnew) +
                                                              head * D + (lane % NCH) * 8);
              __bf16* dst = (lane < NCH ? p.Kw : p.Vw) + (head * p.Tcap + sl) * D;
              *reinterpret_cast<u32x4*>(dst + (lane % NCH) * 8) = v;
            }
          }
        }
      }
    }
    if (ev_w >= tab.nwe) return;
    ev_a = range_start(tab, ev_w);
    ev_e = range_start(tab, ev_w + 1);
    if (ev_a >= ev_e) return;
    // the segment holding step ev_a: sequence b is the first whose steps end
    // past it (every lane at or past B holds the total)
    b = __builtin_popcountll(__builtin_amdgcn_ballot_w64((long long)tab.incl * p.Nkv <= ev_a));
    const int ns_b = __builtin_amdgcn_readlane(tab.ns, b);
    const long long off = ev_a - (long long)(__builtin_amdgcn_readlane(tab.incl, b) - ns_b) * p.Nkv;
    g = (int)(off / ns_b);
    enter((int)(off - (long long)g * ns_b));
  } else {
    g = blockIdx.y;
    b = blockIdx.z;
    n = min(p.lens[b], p.Tcap);
    lo = p.window > 0 ? max(0, n - p.window) : 0;  // first visible key
    // workgroup x takes the x-th chunk from the one holding key lo
    c0 = (lo / p.ch + blockIdx.x) * p.ch;
    slot = ((size_t)b * p.Nkv + g) * p.n_slots + blockIdx.x;
    writer = blockIdx.x == 0;
    load_new(c0, c0 + p.ch);
    if (c0 >= n) {
      write_new_row();
      return;
    }
    s0 = lo > c0 ? (lo - c0) / STEP : 0;  // first step holding a visible key
    nsteps = (min(p.ch, n - c0) + STEP - 1) / STEP;
    last = min(n, c0 + p.ch) - 1;
  }

  // key-padding flags: lane j holds the 32 flags of step s_flags + j (a chunk
  // has at most 64 steps), read in the loop with v_readlane
  const int s_flags = s0;
  uint32_t kw_lane = 0;
  if constexpr (KM && !EV) {
    // drop the leading and trailing steps whose 32 keys are all padding, so
    // they are neither copied nor waited for; the ballot gives the ends
    const int s = s0 + lane;
    if (s < nsteps) {
      const int k = c0 + s * STEP;
      kw_lane = (uint32_t)(p.kbits[(size_t)b * p.kwords + (k >> 6)] >> (k & 32));
    }
    const uint64_t bal = __builtin_amdgcn_ballot_w64(kw_lane != 0);
    if (bal == 0) {
      nsteps = s0;  // padding only: no step runs, the partial stays empty
    } else {
      nsteps = s0 + 64 - __builtin_clzll(bal);
      s0 += __builtin_ctzll(bal);
    }
    s0 = __builtin_amdgcn_readfirstlane(s0);
    nsteps = __builtin_amdgcn_readfirstlane(nsteps);
  }
  const int l16 = lane & 15;
  const int grp = lane >> 4;
  const int G = p.G;
  // chunk mode runs this body once; the even split once per segment piece
  for (;;) {

    const size_t kvh = ((size_t)b * p.Nkv + g) * (size_t)p.Tcap * D;
    const __bf16* Kh = p.K + kvh;
    const __bf16* Vh = p.V + kvh;

    // q^T operand: lane (grp, l16) of block nb holds
    // q[head g*G + 16*nb + l16][32*ks + 8*grp + i]
    bf16x8 qf[NB][KS];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int hh = 16 * nb + l16;
        if (hh < G) {
          const __bf16* src = p.q + ((size_t)b * p.Nq + (size_t)g * G + hh) * D + ks * 32 + grp * 8;
          qf[nb][ks] = *reinterpret_cast<const bf16x8*>(src);
        } else {
          qf[nb][ks] = bf16x8{};
        }
      }

    // RoPE: the angle row of the query's position is loaded with q, before
    // the cache copies; the rotation itself waits until those are issued
    constexpr int NCS = RQ ? KS : 1;  // f32x4 cos and sin vectors per lane
    f32x4 rc[NCS], rs[NCS];
    if constexpr (RQ) {
      const int pos = p.rope.positions ? p.rope.positions[b] : p.lens[b] - 1;
      const float* cs = p.rope.table + (size_t)min(max(pos, 0), p.rope.P - 1) * D;
      // pairs layout: elements 32*ks + 8*grp + i use angles 16*ks + 4*grp + i/2;
      // halves: elements 32*ks + 8*grp + i (ks < KS/2) use angles 32*ks + 8*grp + i
#pragma unroll
      for (int u = 0; u < NCS; ++u) {
        const int m = p.rope.style == 0 ? 16 * u + 4 * grp : 32 * (u >> 1) + 8 * grp + 4 * (u & 1);
        rc[u] = *reinterpret_cast<const f32x4*>(cs + m);
        rs[u] = *reinterpret_cast<const f32x4*>(cs + D / 2 + m);
      }
    }
    // copies in flight, oldest first: q, then K(0), V(0), K(1), V(1).  A step's
    // copies are PER_STEP vector-memory instructions, so vmcnt(PER_STEP) before
    // step s means step s has landed while step s + 1 is still in flight.
    // Copies are issued for two steps past the chunk's end too (all rows clamp
    // to its last row and mostly hit L2), so that count holds on every path and
    // the compiler adds no full drain of its own.
    load_rows<D, true>(Kh, c0 + s0 * STEP, last, K0, lane);
    load_rows<D, false>(Vh, c0 + s0 * STEP, last, V0, lane);
    load_rows<D, true>(Kh, c0 + (s0 + 1) * STEP, last, K1, lane);
    load_rows<D, false>(Vh, c0 + (s0 + 1) * STEP, last, V1, lane);
    if constexpr (RQ) {
      // RoPE at load: lane (grp, l16) holds elements 32*ks + 8*grp + i of its
      // query head's row; a pair (2m, 2m+1) sits inside one fragment, a pair
      // (m, m + D/2) in fragments ks and ks + KS/2 of the same lane
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        if (p.rope.style == 0) {
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) {
            bf16x8 x = qf[nb][ks];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
              const float c = rc[ks][k], sn = rs[ks][k];
              const float a = (float)x[2 * k], bb = (float)x[2 * k + 1];
              x[2 * k] = (__bf16)__builtin_fmaf(a, c, -bb * sn);
              x[2 * k + 1] = (__bf16)__builtin_fmaf(a, sn, bb * c);
            }
            qf[nb][ks] = x;
          }
        } else {
#pragma unroll
          for (int ks = 0; ks < KS / 2; ++ks) {
            bf16x8 x = qf[nb][ks], y = qf[nb][ks + KS / 2];
#pragma unroll
            for (int k = 0; k < 8; ++k) {
              const float c = rc[2 * ks + (k >> 2)][k & 3], sn = rs[2 * ks + (k >> 2)][k & 3];
              const float a = (float)x[k], bb = (float)y[k];
              x[k] = (__bf16)__builtin_fmaf(a, c, -bb * sn);
              y[k] = (__bf16)__builtin_fmaf(a, sn, bb * c);
            }
            qf[nb][ks] = x;
            qf[nb][ks + KS / 2] = y;
          }
        }
      }
    }

    // transposing-read offsets: A operand of O^T += V^T P^T, d = 16*db + l16,
    // keys 4*grp + i (first read) and 16 + 4*grp + i (second read)
    int voff[2][DB];
    {
      const int ip = l16 >> 2, u = l16 & 3;
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        const int r = 16 * hf + 4 * grp + ip;
#pragma unroll
        for (int db = 0; db < DB; ++db)
          voff[hf][db] = r * geo::RB + (((2 * db + (u >> 1)) ^ vswz<D>(r)) << 4) + (u & 1) * 8;
      }
    }
    // K operand offsets: row 16*kb + l16, 16-byte chunk 4*ks + grp (the K
    // swizzle does not depend on row bit 4, so one offset serves both kb)
    int koff[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      koff[ks] = l16 * geo::RB + (((4 * ks + grp) ^ kswz<D>(l16)) << 4);

    f32x4 o[NB][DB];
    float m_run[NB], l_run[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      m_run[nb] = -INFINITY;
      l_run[nb] = 0.f;
#pragma unroll
      for (int db = 0; db < DB; ++db) o[nb][db] = f32x4{};
    }

    // Where the registers allow (Dh x query-head blocks <= 256), a step stops
    // once its K and V^T operands are in registers; its softmax and PV
    // products run in finish_pv(), after the copies that refill its stage have
    // been issued: they read only registers, so the copies need not queue
    // behind them (and a wave keeps more bytes in flight).
    constexpr bool EARLY_V = D * NB <= 256;
    bf16x8 va[EARLY_V ? DB : 1];
    bf16x8 pf[NB];
    // S^T = K q^T of the current step; accumulator register r of block kb:
    // key k0 + 16*kb + 4*grp + r, query column l16 of head block nb
    f32x4 sc[NB][2];
    bool pv_pending = false;
    int pend_k0 = 0;
    uint32_t pend_kw = ~0u;
    // hide keys outside [lo, n) (and padding), fold the step into the running
    // (m, l, o) and leave P^T in pf
    auto softmax = [&](int k0, uint32_t kw) {
      if (k0 + STEP > n || k0 < lo || (KM && kw != ~0u)) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int key = k0 + kb * 16 + grp * 4 + r;
            bool hide = key >= n || key < lo;
            if (KM) hide = hide || !((kw >> (kb * 16 + grp * 4 + r)) & 1);
            if (hide) {
#pragma unroll
              for (int nb = 0; nb < NB; ++nb) sc[nb][kb][r] = -INFINITY;
            }
          }
      }
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        f32x4 (&t)[2] = sc[nb];
        float mx = fmaxf(fmaxf(fmaxf(t[0][0], t[0][1]), fmaxf(t[0][2], t[0][3])),
                         fmaxf(fmaxf(t[1][0], t[1][1]), fmaxf(t[1][2], t[1][3])));
        mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
        mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
        // every step run holds a visible key unless a key-padding mask hides it
        const float m_cand = mx * p.c;
        if (__builtin_amdgcn_ballot_w64(m_cand > m_run[nb] + TAU)) {
          const float m_new = fmaxf(m_run[nb], m_cand);
          const float alpha = exp2_fast(m_run[nb] - m_new);
          m_run[nb] = m_new;
          l_run[nb] *= alpha;
#pragma unroll
          for (int db = 0; db < DB; ++db) o[nb][db] *= alpha;
        }
        const float m_use = (KM && m_run[nb] == -INFINITY) ? 0.f : m_run[nb];
        float rs = 0.f;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float e = exp2_fast(__builtin_fmaf(t[kb][r], p.c, -m_use));
            t[kb][r] = e;
            rs += e;
          }
        l_run[nb] += rs;
        u32x4 pk;
        pk[0] = pack_bf16x2(t[0][0], t[0][1]);
        pk[1] = pack_bf16x2(t[0][2], t[0][3]);
        pk[2] = pack_bf16x2(t[1][0], t[1][1]);
        pk[3] = pack_bf16x2(t[1][2], t[1][3]);
        pf[nb] = __builtin_bit_cast(bf16x8, pk);
      }
    };
    auto finish_pv = [&]() {
      if constexpr (EARLY_V) {
        if (pv_pending) {
          softmax(pend_k0, pend_kw);
#pragma unroll
          for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
              o[nb][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va[db], pf[nb], o[nb][db], 0, 0, 0);
          pv_pending = false;
        }
      }
    };
    auto step = [&](int s, const lds_char* kst, const lds_char* vst) {
      const int k0 = c0 + s * STEP;
      // flags of keys k0 .. k0 + 31 (k0 is a multiple of 32); a step of padding
      // keys only changes nothing
      uint32_t kw = ~0u;
      if constexpr (KM) {
        if constexpr (EV)
          kw = __builtin_amdgcn_readfirstlane(kwl[min(s - kw_base, kMaskWords - 1)]);
        else
          kw = __builtin_amdgcn_readlane(kw_lane, s - s_flags);
        if (kw == 0) return;
      }
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) sc[nb][kb] = f32x4{};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const bf16x8 a = *(lds_bf16x8*)(kst + kb * 16 * geo::RB + koff[ks]);
#pragma unroll
          for (int nb = 0; nb < NB; ++nb)
            sc[nb][kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qf[nb][ks], sc[nb][kb], 0, 0, 0);
        }
      }
      auto read_v = [&](int db) {
        const i16x4 lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) i16x4*)(vst + voff[0][db]));
        const i16x4 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) i16x4*)(vst + voff[1][db]));
        return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7));
      };
      if constexpr (EARLY_V) {
#pragma unroll
        for (int db = 0; db < DB; ++db) va[db] = read_v(db);
        pend_k0 = k0;
        pend_kw = kw;
        pv_pending = true;  // softmax and products run in finish_pv()
      } else {
        softmax(k0, kw);
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const bf16x8 a = read_v(db);
#pragma unroll
          for (int nb = 0; nb < NB; ++nb)
            o[nb][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pf[nb], o[nb][db], 0, 0, 0);
        }
      }
    };

    // Steps in pairs from s0: the first of a pair uses stage 0, the second stage
    // 1.  Before step s the copies of steps s and s + 1 are outstanding; once
    // step s has read its stage, the copies of step s + 2 go into it.
    // APP: after step s's copies have landed, put the new row into its stage.
    // When the new row is the chunk's last row, the stage rows after it were
    // copied from that same cache row (copies clamp to `last`), i.e. from the
    // bytes workgroup 0 is overwriting: they get the new row too.  Their
    // weights are 0, but 0 times a stale NaN or Inf would still be NaN.
    auto substitute = [&](int s, lds_char* kst, lds_char* vst) {
      if constexpr (APP) {
        const int r = alt_row - (c0 + s * STEP);
        const int l = lane;
        if (r >= 0 && r < STEP && l < 2 * NCH) {  // r is wave-uniform
          const bool isk = l < NCH;
          const int c = isk ? l : l - NCH;
          const int r_end = alt_row == last ? STEP : r + 1;
          typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
          for (int rr = r; rr < r_end; ++rr) {
            const int off = (rr / geo::RP) * 1024 +
                            ((rr % geo::RP) * NCH + (c ^ (isk ? kswz<D>(rr) : vswz<D>(rr)))) * 16;
            *(lds_u32x4*)((isk ? kst : vst) + off) = new_row;
          }
        }
        // the step's operand reads use other pointer types: keep them after the store
        __asm__ __volatile__("" ::: "memory");
      }
    };

    // The loop starts with the copies of step s + 2, not with a read of stage
    // 0: entered at such a read, the loop merges the states of its entry and
    // its back edge there, and the compiler can no longer tell which copies may
    // still target stage 0; it then drains every copy in flight.
    if (s0 < nsteps) {
      wait_vm<PER_STEP>();
      substitute(s0, K0, V0);
      step(s0, K0, V0);
      for (int s = s0;; s += 2) {
        wait_lds_reads();  // step s has read stage 0
        load_rows<D, true>(Kh, c0 + (s + 2) * STEP, last, K0, lane);
        load_rows<D, false>(Vh, c0 + (s + 2) * STEP, last, V0, lane);
        finish_pv();
        wait_vm<PER_STEP>();
        if (s + 1 >= nsteps) break;
        substitute(s + 1, K1, V1);
        step(s + 1, K1, V1);
        wait_lds_reads();  // step s + 1 has read stage 1
        load_rows<D, true>(Kh, c0 + (s + 3) * STEP, last, K1, lane);
        load_rows<D, false>(Vh, c0 + (s + 3) * STEP, last, V1, lane);
        finish_pv();
        wait_vm<PER_STEP>();
        if (s + 2 >= nsteps) break;
        substitute(s + 2, K0, V0);
        step(s + 2, K0, V0);
      }
    }
    wait_vm<0>();  // no copy may still target LDS when the wave ends
    write_new_row();

    // partial of this chunk: O^T register r of block db is d = 16*db + 4*grp + r
    // of query column l16
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      float l_tot = l_run[nb];
      l_tot += __shfl_xor(l_tot, 16, 64);
      l_tot += __shfl_xor(l_tot, 32, 64);
      const int hh = 16 * nb + l16;
      if (hh < G) {
        const size_t part = slot * G + hh;
        float* dst = p.ws_o + part * D + 4 * grp;
#pragma unroll
        for (int db = 0; db < DB; ++db) *reinterpret_cast<f32x4*>(dst + 16 * db) = o[nb][db];
        if (grp == 0) {
          p.ws_ml[part * 2 + 0] = m_run[nb];
          p.ws_ml[part * 2 + 1] = l_tot;
        }
      }
    }
    if constexpr (!EV) {
      break;
    } else {
      if (ev_a >= ev_e) break;
      // next segment: the next K/V head, else the next sequence with steps
      if (++g == p.Nkv) {
        g = 0;
        b = __builtin_ctzll(__builtin_amdgcn_ballot_w64(lane > b && tab.ns > 0));
      }
      enter(0);
    }
  }  // segments
}

// Merge the chunk partials of one (sequence, query head) row: slot x holds a
// chunk's running max m_x (log2 units), its sum l_x and its unnormalised output
// o_x; the row's output is sum_x 2^(m_x - M) o_x / sum_x 2^(m_x - M) l_x with
// M = max_x m_x, and its LSE is (M + log2 of the denominator) ln 2.
//
// p.mw wavefronts share a row (1 to 16; blockDim.x = 64 * max(4, p.mw)), each
// folding a contiguous run of slots under its own running max; the row's first
// wavefront then folds the wavefronts' results, rescaled to the common max,
// from LDS, in wavefront order.  The kernel is latency-bound (a row's partials
// are a few KB): a wavefront requests sixteen partial outputs at a time, the
// first sixteen together with their (m, l), before the weights are known.
//
// EV: the partials of the even split; segment (b, g) holds the pieces of the
// wavefronts whose ranges meet its steps, wavefront w's piece at slot
// b*Nkv + g + w.
template <int D, bool KM, bool EV = false>
__global__ __launch_bounds__(1024) void decode_merge_kernel(DecParams p) {
  constexpr int PL = D / 64;  // head-dims per lane
  typedef float fvec __attribute__((ext_vector_type(PL)));
  __shared__ fvec s_acc[16][64];
  __shared__ float s_m[16], s_l[16];
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int mw = p.mw;
  const int row = blockIdx.x * ((int)(blockDim.x >> 6) / mw) + wv / mw;
  const int part = wv % mw;
  const bool valid = row < p.B * p.Nq;
  const int G = p.G;
  int ns = 0;  // slots written for this row
  size_t part0 = 0;
  if (valid) {
    const int b = row / p.Nq;
    const int h = row % p.Nq;
    if constexpr (EV) {
      // a segment with visible keys was taken by ranges wf .. wl, which the
      // partial kernel recorded.  The record is read together with the
      // length, not after it (one memory round trip fewer); a segment without
      // visible keys has no record, and its stale words are not used.
      const int2 fl =*reinterpret_cast<const int2*>(p.ws_seg + 2 * ((size_t)b * p.Nkv + h / G));
      const int n = max(0, min(p.lens[b], p.Tcap));
      if (n > 0) {
        ns = fl.y - fl.x + 1;
        part0 = ((size_t)b * p.Nkv + h / G + fl.x) * G + h % G;  // slot x: part0 + x*G
      }
    } else {
      const int n = min(p.lens[b], p.Tcap);
      const int nc = n > 0 ? (n + p.ch - 1) / p.ch : 0;
      // partial slot x holds chunk c_lo + x; chunks c_lo .. nc-1 wrote one
      const int c_lo = p.window > 0 ? max(0, n - p.window) / p.ch : 0;
      ns = max(0, nc - c_lo);
      part0 = ((size_t)b * p.Nkv + h / G) * p.n_slots * G + h % G;  // slot x: part0 + x*G
    }
  }
  const int x0 = part * ns / mw, x1 = (part + 1) * ns / mw;  // this wavefront's slots

  float Mw = -INFINITY;  // running max of the slots folded so far
  float Ll = 0.f;        // this lane's share of the weighted l sum
  fvec acc = {};
  auto load_o = [&](int x) { return *reinterpret_cast<const fvec*>(p.ws_o + (part0 + (size_t)x * G) * D + lane * PL); };
  for (int cb = x0; cb < x1; cb += 64) {
    const int cnt = min(64, x1 - cb);
    // lane j holds slot cb + j's (m, l); lanes past the run hold a zero weight
    float m = -INFINITY, l = 0.f;
    if (lane < cnt) {
      const float2 v = *reinterpret_cast<const float2*>(p.ws_ml + (part0 + (size_t)(cb + lane) * G) * 2);
      m = v.x;
      l = v.y;
    }
    fvec ov[kMergeBatch];
#pragma unroll
    for (int u = 0; u < kMergeBatch; ++u) ov[u] = u < cnt ? load_o(cb + u) : fvec{};
    const float Mn = fmaxf(Mw, wave_max(m));
    // every slot so far may hold padding only (M = -inf): weights 0, not NaN
    const float Mu = Mn == -INFINITY ? 0.f : Mn;
    const float r = exp2_fast(Mw - Mu);
    acc = acc * r;
    const float wgt = exp2_fast(m - Mu);
    Ll = __builtin_fmaf(wgt, l, Ll * r);
    Mw = Mn;
#pragma unroll
    for (int u = 0; u < kMergeBatch; ++u) {
      const float wu = __shfl(wgt, u, 64);
#pragma unroll
      for (int e = 0; e < PL; ++e) acc[e] = __builtin_fmaf(wu, ov[u][e], acc[e]);
    }
    for (int j = kMergeBatch; j < cnt; j += kMergeBatch) {
#pragma unroll
      for (int u = 0; u < kMergeBatch; ++u) ov[u] = j + u < cnt ? load_o(cb + j + u) : fvec{};
#pragma unroll
      for (int u = 0; u < kMergeBatch; ++u) {
        const float wu = __shfl(wgt, j + u, 64);
#pragma unroll
        for (int e = 0; e < PL; ++e) acc[e] = __builtin_fmaf(wu, ov[u][e], acc[e]);
      }
    }
  }
  float M = Mw;
  float L = wave_sum(Ll);
  if (mw > 1) {
    s_acc[wv][lane] = acc;
    if (lane == 0) {
      s_m[wv] = Mw;
      s_l[wv] = L;
    }
    __syncthreads();
    if (part != 0) return;
    for (int w = 1; w < mw; ++w) M = fmaxf(M, s_m[wv + w]);
    const float Mu = M == -INFINITY ? 0.f : M;
    const float r0 = exp2_fast(Mw - Mu);
    acc = acc * r0;
    L *= r0;
    for (int w = 1; w < mw; ++w) {
      const float r = exp2_fast(s_m[wv + w] - Mu);
      const fvec o = s_acc[wv + w][lane];
#pragma unroll
      for (int e = 0; e < PL; ++e) acc[e] = __builtin_fmaf(r, o[e], acc[e]);
      L = __builtin_fmaf(r, s_l[wv + w], L);
    }
  }
  if (!valid) return;
  // no slot (n < 1) leaves L = 0: a NaN row, or O = 0 and LSE = -inf with a key-padding mask
  const float inv = (KM && L == 0.f) ? 0.f : 1.f / L;
  __bf16* dst = p.O + (size_t)row * D + lane * PL;
#pragma unroll
  for (int e = 0; e < PL; ++e) dst[e] = (__bf16)(acc[e] * inv);
  if (p.LSE != nullptr && lane == 0) p.LSE[row] = (M + __log2f(L)) * kLn2;
}

}  // namespace

bool decode_bf16_supported(int Nq, int Nkv, int Dh) {
  return (Dh == 64 || Dh == 128 || Dh == 256) && Nq / Nkv <= 32;
}

// Keys per chunk: the longest candidate that still gives the grid at least
// 2048 (sequence, K/V head, chunk) items -- 1024 for 16 or more query heads
// per K/V head -- when every sequence has L visible keys (L = Tcap, or the
// window when it is shorter).  The candidates are multiples of 32 keys, none
// a power of two.
int decode_bf16_chunk(int B, int Nkv, int L, int G) {
  // at most 64 steps per chunk: the key-padding trim tests one step per lane
  static const int kChunks[] = {1792, 1152, 896, 640, 384, 224, 160, 96};
  static_assert(1792 <= 64 * STEP, "a chunk must fit one wavefront of steps");
  // each chunk writes G x (Dh + 2) fp32 partials that the merge reads back;
  // with 16 or more query heads per K/V head that is several percent of a
  // short chunk's K/V bytes, so those groups take half the item count
  const long long min_items = G >= 16 ? 1024 : 2048;
  // ... but never shorter than 640 keys (224 with 16 or more query heads per
  // K/V head): at small batches the item count would otherwise ask for
  // chunks of a few steps, whose partials cost more to write and merge than
  // the extra items gain (one sequence of 32768 tokens: 60 us at 96-key
  // chunks, 30 us at 640)
  const int floor_ch = G >= 16 ? kFloorKeysWide : kFloorKeys;
  const long long heads = (long long)B * Nkv;
  for (int ch : kChunks)
    if (ch <= floor_ch || heads * ((L + ch - 1) / ch) >= min_items) return ch;
  return floor_ch;
}


namespace {
// partial slots one merge wavefront folds at most: one round of requests
// (12 slots in rounds of eight were 1-2 % slower on the batched decode, 4 in
// rounds of four 6-8 % slower)
constexpr int kMergeSlots = 16;
// merge: enough wavefronts per row that each folds at most kMergeSlots slots
int merge_waves(long long slots) {
  int mw = 1;
  while (mw < 16 && (slots + mw - 1) / mw > kMergeSlots) mw *= 2;
  return mw;
}
// chunk length and partial slots per (sequence, K/V head); whether the even
// split may serve the shape (without a key-padding mask or an append), its
// merge wavefronts per row, and the workspace slots (G rows each) both need
struct DecodePlan {
  int ch, n_slots, mw;
  bool ev;
  int ev_mw;
  long long slots;
};
DecodePlan decode_plan(int B, int Nq, int Nkv, int Dh, int Tcap, int window) {
  const int L = (window > 0 && window < Tcap) ? window : Tcap;
  DecodePlan d;
  d.ch = decode_bf16_chunk(B, Nkv, L, Nq / Nkv);
  const int all = (Tcap + d.ch - 1) / d.ch;
  // a window of L keys starting anywhere touches at most ceil(L / ch) + 1 chunks
  d.n_slots = L < Tcap ? std::min(all, (L + d.ch - 1) / d.ch + 1) : all;
  d.mw = merge_waves(d.n_slots);
  d.slots = (long long)B * Nkv * d.n_slots;
  // the even split takes up to 64 sequences (one lane each in its table) and
  // grids of at least kEvenWaves / 2 chunk items: below that every chunk runs
  // at once anyway, and the table each wavefront builds first (a dependent
  // load of the lengths before its first copy) costs more than the balance
  // gains (one sequence of 32768 keys, 8 K/V heads: 31 us against 28).  At
  // head size 256 only the plain form with one block of query heads fits the
  // registers (see launch_decode_bf16).
  d.ev = B <= 64 && d.slots >= kEvenWaves / 2 && (Dh <= 128 || Nq / Nkv <= 16);
  // the even split's merge folds runs of about as many pieces as the chunk
  // mode's (a row's share of the grid is the same); longer runs just loop
  d.ev_mw = d.mw;
  if (d.ev) d.slots = std::max(d.slots, (long long)B * Nkv + kEvenWaves);
  return d;
}

template <int D, int NB, bool KM, bool APP = false, bool RQ = false, bool EV = false>
hipError_t launch_decode_km(const DecParams& p, hipStream_t stream) {
  const dim3 grid = EV ? dim3(p.ev_nw) : dim3(p.n_slots, p.Nkv, p.B);
  hipLaunchKernelGGL((decode_partial_kernel<D, NB, KM, APP, RQ, EV>), grid, dim3(64), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int rows = p.B * p.Nq;
  const int wpb = p.mw < 4 ? 4 : p.mw;  // wavefronts per block
  const int rpb = wpb / p.mw;           // rows per block
  hipLaunchKernelGGL((decode_merge_kernel<D, KM, EV>), dim3((rows + rpb - 1) / rpb), dim3(64 * wpb),
                     0, stream, p);
  return hipGetLastError();
}
template <int D, int NB>
hipError_t launch_decode(const DecParams& p, hipStream_t stream) {
  if (p.knew) {  // append (no key mask)
    if constexpr (D <= 128) {
      if (p.ev_nw) return launch_decode_km<D, NB, false, true, false, true>(p, stream);
    }
    return launch_decode_km<D, NB, false, true>(p, stream);
  }
  if (p.kbits) {
    if constexpr (D <= 128) {
      if (p.ev_nw)
        return p.rope.table ? launch_decode_km<D, NB, true, false, true, true>(p, stream)
                            : launch_decode_km<D, NB, true, false, false, true>(p, stream);
    }
    return p.rope.table ? launch_decode_km<D, NB, true, false, true>(p, stream)
                        : launch_decode_km<D, NB, true>(p, stream);
  }
  if constexpr (D <= 128) {
    if (p.ev_nw)
      return p.rope.table ? launch_decode_km<D, NB, false, false, true, true>(p, stream)
                          : launch_decode_km<D, NB, false, false, false, true>(p, stream);
  } else if constexpr (NB == 1) {
    if (p.ev_nw) return launch_decode_km<D, NB, false, false, false, true>(p, stream);
  }
  return p.rope.table ? launch_decode_km<D, NB, false, false, true>(p, stream)
                      : launch_decode_km<D, NB, false>(p, stream);
}
}  // namespace

size_t decode_bf16_workspace(int B, int Nq, int Nkv, int Dh, int Tcap, int window) {
  const DecodePlan d = decode_plan(B, Nq, Nkv, Dh, Tcap, window);
  const size_t parts = (size_t)d.slots * (Nq / Nkv);
  return parts * Dh * sizeof(float) + parts * 2 * sizeof(float) +
         (d.ev ? (size_t)B * Nkv * 2 * sizeof(int) : 0);
}

hipError_t launch_decode_bf16(const void* q, const void* Kc, const void* Vc, const int32_t* lens,
                              void* O, float* LSE, int B, int Nq, int Nkv, int Dh, int Tcap,
                              int window, float scale, const uint64_t* kbits, void* ws,
                              hipStream_t stream, const void* knew, const void* vnew,
                              const int32_t* slot, const RopeQ* rope) {
  const DecodePlan d = decode_plan(B, Nq, Nkv, Dh, Tcap, window);
  DecParams p;
  p.knew = static_cast<const __bf16*>(knew);
  p.vnew = static_cast<const __bf16*>(vnew);
  p.slot = slot;
  p.Kw = static_cast<__bf16*>(const_cast<void*>(Kc));
  p.Vw = static_cast<__bf16*>(const_cast<void*>(Vc));
  p.q = static_cast<const __bf16*>(q);
  p.K = static_cast<const __bf16*>(Kc);
  p.V = static_cast<const __bf16*>(Vc);
  p.lens = lens;
  p.kbits = kbits;
  p.kwords = key_mask_words(Tcap);
  p.O = static_cast<__bf16*>(O);
  p.LSE = LSE;
  p.B = B;
  p.Nq = Nq;
  p.Nkv = Nkv;
  p.G = Nq / Nkv;
  p.Tcap = Tcap;
  p.ch = d.ch;
  p.n_slots = d.n_slots;
  // the even split at head size 256 only in its plain form (the rotating and
  // appending forms spill there); with a key mask at head sizes up to 128, when
  // every wavefront's range fits the flag words a wavefront holds in LDS (a
  // range is at most tot * 64 / C(W) + 1 steps, tot counting every step of
  // every (sequence, K/V head) pair up to the visible span)
  bool ev = d.ev && (Dh <= 128 || (rope == nullptr && knew == nullptr && kbits == nullptr));
  if (ev && kbits != nullptr) {
    const int nw = Nq / Nkv >= 16 ? kEvenWavesWide : kEvenWaves;
    const int L = (window > 0 && window < Tcap) ? window : Tcap;
    const long long tot = (long long)B * Nkv * ((L + STEP - 1) / STEP + 1);
    const long long cw = kWeightEven * ((nw + 1) / 2) + kWeightOdd * (nw / 2);
    ev = tot * kWeightEven / cw + 3 <= kMaskWords - 2;
  }
  p.ev_nw = ev ? (p.G >= 16 ? kEvenWavesWide : kEvenWaves) : 0;
  p.ev_min = (p.G >= 16 ? kFloorKeysWide : kFloorKeys) / STEP;
  p.mw = ev ? d.ev_mw : d.mw;
  const size_t parts = (size_t)d.slots * (Nq / Nkv);
  p.ws_o = static_cast<float*>(ws);
  p.ws_ml = p.ws_o + parts * Dh;
  p.ws_seg = reinterpret_cast<int*>(p.ws_ml + parts * 2);
  p.window = window;
  p.c = kLog2e * scale;
  p.rope = rope ? *rope : RopeQ{nullptr, 0, nullptr, nullptr, 0};
  if (Nkv > 65535 || B > 65535) return hipErrorInvalidConfiguration;
  const bool two = p.G > 16;
  switch (Dh) {
    case 64: return two ? launch_decode<64, 2>(p, stream) : launch_decode<64, 1>(p, stream);
    case 128: return two ? launch_decode<128, 2>(p, stream) : launch_decode<128, 1>(p, stream);
    case 256: return two ? launch_decode<256, 2>(p, stream) : launch_decode<256, 1>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

// Scratch of the allocation-free decode (attn_decode_noalloc): the split-K
// partials live in this fixed array instead of a caller's workspace.  Each
// device that loads the library holds its own copy until the process ends.
// In host code `scratch` only names the symbol; its device address is looked
// up once per device (with that device current) and kept in scratch_ptr.
static __device__ __align__(256) char scratch[kDecodeScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
void* scratch_ptr[kMaxDevices];
}  // namespace

hipError_t decode_scratch(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    scratch_ptr[dev] = p;
  }
  *ptr = scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace attn
