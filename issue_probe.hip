// Issue probe: how the matrix cores, the vector ALU and LDS operand reads of
// one compute unit share their time on gfx950.  Measurement tooling of the
// benchmark, not part of the attention library: `python bench.py
// --build-probe` compiles it into _build/libissue_probe.so, and `python
// bench.py --issue-probe` runs it.
//
// Every wave runs `iters` rounds of 32 slots.  A slot holds, depending on the
// mode:
//   MFMA   one v_mfma_f32_32x32x16_bf16 (four independent accumulators), with
//          its A operand from registers, or (LDS) from a 16-byte ds_read of a
//          16 KB LDS tile, one read per `reuse` products;
//   VALU   `nv` vector instructions: pairs of v_fma_f32 + v_exp_f32 on eight
//          independent chains (nv even), or nv v_fma_f32 alone (exp off).
// Waves can mix both in one instruction stream (interleaved by the compiler's
// scheduling barriers: 1 MFMA, then the slot's VALU work), or split them: in
// `split` mode the waves of the lower half of the workgroup issue only the
// MFMA work and the upper half only the VALU work, so that each SIMD holds
// one wave of each kind.  The results are folded into one store per lane so
// that nothing is dropped.
#include <hip/hip_runtime.h>
#include <stddef.h>

typedef __bf16 pb_bf16x8 __attribute__((ext_vector_type(8)));
typedef float pb_f32x16 __attribute__((ext_vector_type(16)));

template <bool DO_MFMA, bool DO_VALU, bool LDS, int REUSE, bool EXP, int NV>
__device__ __forceinline__ void probe_body(int iters, float* out, char* tile) {
  const int lane = threadIdx.x & 63;
  constexpr bool mf = DO_MFMA;
  constexpr bool va = DO_VALU;
  constexpr int NOPS = EXP ? NV / 2 : NV;  // chain steps per slot
  // operands: small values so nothing overflows
  pb_bf16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(0.001f * (float)((lane + i) & 7));
    b[i] = (__bf16)(0.001f * (float)((lane * 3 + i) & 7));
  }
  if (LDS) {
    for (int i = threadIdx.x; i < 16384 / 16; i += blockDim.x)
      reinterpret_cast<pb_bf16x8*>(tile)[i] = a;
    __syncthreads();
  }
  pb_f32x16 acc[4] = {};
  float v[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = 0.25f + 0.01f * (float)(lane & 7) + 0.02f * i;
  const float c0 = -0.75f, c1 = 0.125f;
  // ds_read offsets: 16 rows of 1 KB, lane's 16 bytes, rotating through the tile
  int off = lane * 16;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 32; ++j) {
      if (mf) {
        pb_bf16x8 aa = a;
        if (LDS && (j % REUSE) == 0) {
          aa = *reinterpret_cast<const pb_bf16x8*>(tile + ((off + j * 1024) & 16383));
          a = aa;
        }
        acc[j & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(LDS ? a : aa, b, acc[j & 3], 0, 0, 0);
      }
      if (va) {
        // consecutive steps go to different chains, so none waits on its own result
#pragma unroll
        for (int k = 0; k < NOPS; ++k) {
          const int ch = (j * NOPS + k) & 7;
          float t = __builtin_fmaf(v[ch], c0, c1);
          v[ch] = EXP ? __builtin_amdgcn_exp2f(t) : t;
        }
      }
      if (DO_MFMA && DO_VALU) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // 1 MFMA
        if (LDS) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // LDS read
        __builtin_amdgcn_sched_group_barrier(0x002, NV, 0);  // the slot's VALU
      }
    }
    off += 16;
  }
  float r = 0.f;
#pragma unroll
  for (int q = 0; q < 4; ++q)
#pragma unroll
    for (int i = 0; i < 16; ++i) r += acc[q][i];
#pragma unroll
  for (int i = 0; i < 8; ++i) r += v[i];
  out[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = r;
}

// LDS read bandwidth: every wave streams `iters` rounds of 32 reads of one
// type from a 16 KB tile -- 16-byte row reads (ds_read_b128) or transposing
// 8-byte reads (ds_read_b64_tr_b16) -- with (MFMA) one matrix product per
// read pair of the transposing kind, the PV product's pattern.
template <bool TR, bool WITH_MFMA>
__global__ __launch_bounds__(512) void lds_probe_kernel(int iters, float* out) {
  __shared__ __attribute__((aligned(1024))) char tile[16384];
  typedef short pb_i16x4 __attribute__((ext_vector_type(4)));
  const int lane = threadIdx.x & 63;
  for (int i = threadIdx.x; i < 16384 / 4; i += blockDim.x)
    reinterpret_cast<float*>(tile)[i] = 0.001f * (float)(i & 15);
  __syncthreads();
  pb_bf16x8 b;
#pragma unroll
  for (int i = 0; i < 8; ++i) b[i] = (__bf16)(0.001f * (float)((lane * 3 + i) & 7));
  pb_f32x16 acc[4] = {};
  typedef unsigned pb_u32x4 __attribute__((ext_vector_type(4)));
  unsigned fold = 0;
  int off = lane * 16;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 32; ++j) {
      pb_bf16x8 a;
      if (TR) {
        // two transposing reads (rows 4*(lane/16) + i, 8 bytes at column lane % 16)
        const int base = ((lane >> 4) * 4 * 256 + (((lane & 15) * 8 + (lane >> 4) * 32) & 255) +
                          j * 512 + it * 16) & 16383;
        const pb_i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) pb_i16x4*)(tile + base));
        const pb_i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) pb_i16x4*)(tile + ((base + 4096) & 16383)));
        a = __builtin_bit_cast(pb_bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      } else {
        a = *reinterpret_cast<const pb_bf16x8*>(tile + ((off + j * 1024) & 16383));
      }
      if (WITH_MFMA) acc[j & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[j & 3], 0, 0, 0);
      else fold ^= __builtin_bit_cast(pb_u32x4, a).x;  // one cheap op per read
    }
    off += 16;
  }
  float r = 0.f;
#pragma unroll
  for (int q = 0; q < 4; ++q)
#pragma unroll
    for (int i = 0; i < 16; ++i) r += acc[q][i];
  r += (float)(fold & 1u);
  out[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = r;
}

// kind 4: ds_read_b128 only; 5: ds_read_b64_tr_b16 pairs only; 6: tr pairs + MFMA
extern "C" int lds_probe(int kind, int waves, int blocks, int iters, float* out, void* stream) {
  if (!out || waves < 1 || waves > 8 || blocks < 1 || iters < 1) return -1;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const dim3 grid(blocks), block(64 * waves);
  if (kind == 4) hipLaunchKernelGGL((lds_probe_kernel<false, false>), grid, block, 0, s, iters, out);
  else if (kind == 5) hipLaunchKernelGGL((lds_probe_kernel<true, false>), grid, block, 0, s, iters, out);
  else if (kind == 6) hipLaunchKernelGGL((lds_probe_kernel<true, true>), grid, block, 0, s, iters, out);
  else return -1;
  return hipGetLastError() == hipSuccess ? 0 : -5;
}

template <bool DO_MFMA, bool DO_VALU, bool LDS, int REUSE, bool EXP, int NV>
__global__ __launch_bounds__(512) void probe_kernel(int iters, float* out, int split) {
  __shared__ __attribute__((aligned(1024))) char tile[16384];
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nw = blockDim.x >> 6;
  if (DO_MFMA && DO_VALU && split) {
    // the lower half of the waves issue MFMA work only, the upper half VALU work
    // only (waves are placed on the SIMDs round-robin, so each SIMD gets one of each)
    if (w < nw / 2) probe_body<true, false, LDS, REUSE, EXP, NV>(iters, out, tile);
    else probe_body<false, true, LDS, REUSE, EXP, NV>(iters, out, tile);
  } else {
    probe_body<DO_MFMA, DO_VALU, LDS, REUSE, EXP, NV>(iters, out, tile);
  }
}

// kind: 0 MFMA only, 1 VALU only, 2 both in one stream, 3 both split over waves
// lds: A operand from LDS with one read per `reuse` (1 or 2) products
// nv: VALU instructions per slot (0, 2, 4, 6, 8); exp: v_exp_f32 in the VALU work
// Returns 0, -1 on an unsupported combination, -5 if the launch failed.
extern "C" int issue_probe(int kind, int waves, int blocks, int iters, int lds, int reuse, int exp,
                           int nv, float* out, void* stream) {
  if (!out || waves < 1 || waves > 8 || blocks < 1 || iters < 1) return -1;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const dim3 grid(blocks), block(64 * waves);
  const int split = kind == 3;
  const bool m = kind == 0 || kind >= 2, v = kind >= 1;
#define PROBE(M, V, L, R, E, N) \
  hipLaunchKernelGGL((probe_kernel<M, V, L, R, E, N>), grid, block, 0, s, iters, out, split)
  if (m && !v) {
    if (!lds) PROBE(true, false, false, 1, false, 0);
    else if (reuse == 1) PROBE(true, false, true, 1, false, 0);
    else if (reuse == 2) PROBE(true, false, true, 2, false, 0);
    else return -1;
  } else if (!m && v) {
    if (exp && nv == 2) PROBE(false, true, false, 1, true, 2);
    else if (exp && nv == 4) PROBE(false, true, false, 1, true, 4);
    else if (exp && nv == 8) PROBE(false, true, false, 1, true, 8);
    else if (!exp && nv == 4) PROBE(false, true, false, 1, false, 4);
    else if (!exp && nv == 8) PROBE(false, true, false, 1, false, 8);
    else return -1;
  } else {
    // both: register or LDS operands (reuse 1), with exp+fma or fma work
    if (!lds && exp && nv == 2) PROBE(true, true, false, 1, true, 2);
    else if (!lds && exp && nv == 4) PROBE(true, true, false, 1, true, 4);
    else if (!lds && exp && nv == 8) PROBE(true, true, false, 1, true, 8);
    else if (!lds && !exp && nv == 4) PROBE(true, true, false, 1, false, 4);
    else if (!lds && !exp && nv == 8) PROBE(true, true, false, 1, false, 8);
    else if (lds && exp && nv == 4) PROBE(true, true, true, 1, true, 4);
    else if (lds && !exp && nv == 4) PROBE(true, true, true, 1, false, 4);
    else return -1;
  }
#undef PROBE
  return hipGetLastError() == hipSuccess ? 0 : -5;
}
