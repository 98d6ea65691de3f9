// KV-cache append: copy the new tokens' K and V rows into the caches.
//
// The textbook's step-by-step forward pass (attention chapter,
// "Прямой проход по шагам") concatenates the new K and V after the cached
// ones, so token position p goes to cache row p.  Its sliding-window section
// ("Скользящее окно") keeps only the last positions -- Mistral's rolling
// buffer cache -- which here means position p goes to row p mod Tcap.
//
// One wavefront per (new row, K/V head, sequence) copies that row of K and of
// V with the widest load the row length and the buffers' alignment allow.
// When a rolling append is longer than the buffer only its last Tcap rows
// are written (each to its own slot, so no two lanes race on a row); a
// linear append's rows that would land outside [0, Tcap) are dropped.

#include "common.h"
#include "kernels.h"

namespace attn {

namespace {

struct AppendParams {
  const char* Knew;
  const char* Vnew;
  char* Kc;
  char* Vc;
  const int32_t* pos;
  int Nkv, Snew, Tcap, rolling;
  int row_bytes;  // Dh * element size
  int first;      // first new row to write (rolling appends longer than Tcap)
};

template <typename U>
__global__ __launch_bounds__(64) void kv_append_kernel(AppendParams p) {
  const int i = p.first + blockIdx.x;
  const int g = blockIdx.y;
  const int b = blockIdx.z;
  const long long p0 = p.pos[b];
  if (p0 < 0) return;
  long long slot = p0 + i;
  if (p.rolling) {
    slot %= p.Tcap;
  } else if (slot >= p.Tcap) {
    return;
  }
  const size_t src = (((size_t)b * p.Nkv + g) * p.Snew + i) * (size_t)p.row_bytes;
  const size_t dst = (((size_t)b * p.Nkv + g) * p.Tcap + (size_t)slot) * (size_t)p.row_bytes;
  const int n = p.row_bytes / (int)sizeof(U);
  for (int e = threadIdx.x; e < n; e += 64) {
    reinterpret_cast<U*>(p.Kc + dst)[e] = reinterpret_cast<const U*>(p.Knew + src)[e];
    reinterpret_cast<U*>(p.Vc + dst)[e] = reinterpret_cast<const U*>(p.Vnew + src)[e];
  }
}

}  // namespace

hipError_t launch_kv_append(const void* Knew, const void* Vnew, void* Kc, void* Vc,
                            const int32_t* pos, int B, int Nkv, int Snew, int Dh, int Tcap,
                            int rolling, int elem_bytes, hipStream_t stream) {
  AppendParams p;
  p.Knew = static_cast<const char*>(Knew);
  p.Vnew = static_cast<const char*>(Vnew);
  p.Kc = static_cast<char*>(Kc);
  p.Vc = static_cast<char*>(Vc);
  p.pos = pos;
  p.Nkv = Nkv;
  p.Snew = Snew;
  p.Tcap = Tcap;
  p.rolling = rolling;
  p.row_bytes = Dh * elem_bytes;
  p.first = (rolling && Snew > Tcap) ? Snew - Tcap : 0;
  const int rows = Snew - p.first;
  if (Nkv > 65535 || B > 65535) return hipErrorInvalidConfiguration;
  // widest unit dividing the row length and every buffer's alignment
  uintptr_t align = (uintptr_t)Knew | (uintptr_t)Vnew | (uintptr_t)Kc | (uintptr_t)Vc |
                    (uintptr_t)p.row_bytes;
  const dim3 grid(rows, Nkv, B);
  if (align % 16 == 0)
    hipLaunchKernelGGL(kv_append_kernel<u32x4>, grid, dim3(64), 0, stream, p);
  else if (align % 4 == 0)
    hipLaunchKernelGGL(kv_append_kernel<uint32_t>, grid, dim3(64), 0, stream, p);
  else
    hipLaunchKernelGGL(kv_append_kernel<uint16_t>, grid, dim3(64), 0, stream, p);
  return hipGetLastError();
}

}  // namespace attn
