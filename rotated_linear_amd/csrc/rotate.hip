// Runtime activation-side transform: K stages of disjoint-pair Givens rotations,
// then division by the channel scales ("ParoQuant: pairwise rotations that
// survive deployment", section "A rotation small enough to execute").
//
// One workgroup of 512 threads transforms R rows held in LDS as float32 for all
// K stages (rotation_core.h). Stage parameters stream through a register ring
// issued before the rows are even loaded; 1/s is applied on the way out with one
// float32 -> float16 rounding. With PERM the output keeps every 8-channel word in
// the order the INT4 decode of the linear kernels produces ([0,4,1,5,2,6,3,7]),
// which is how paro_rotated_linear hands its workspace to them.
#include "rotation_core.h"

namespace paro {
namespace {

constexpr int kRotThreads = 512;

template <int R, int PPT, int PD, bool EXACT, bool PERM>
__global__ __launch_bounds__(kRotThreads) void rotate_rows_kernel(const uint16_t* __restrict__ x,
                                                                   uint16_t* __restrict__ xout, int M, int D,
                                                                   int K, const PairRec* __restrict__ recs,
                                                                   const float* __restrict__ inv_s) {
  extern __shared__ __attribute__((aligned(16))) float lds[];  // [D][R]
  const int tid = threadIdx.x;
  const int row0 = blockIdx.x * R;
  const int P = D / 2;
  const int words = D / 8;  // 16-byte words per row
  const int total = words * R;

  StageRing<kRotThreads, PPT, PD, EXACT> ring;
  if (K > 0) ring_prime(ring, K, P, tid, recs);

  // rows -> LDS, four 16-byte loads in flight per thread per batch
  for (int base = 0; base < total; base += 4 * kRotThreads) {
    uint4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      int e = base + tid + u * kRotThreads;
      e = e < total ? e : total - 1;
      const int r = e / words, w = e - r * words;
      int row = row0 + r;
      row = row < M ? row : M - 1;
      v[u] = *reinterpret_cast<const uint4*>(x + size_t(row) * D + size_t(w) * 8);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int e = base + tid + u * kRotThreads;
      if (e < total) {
        const int r = e / words, w = e - r * words;
        const _Float16* h = reinterpret_cast<const _Float16*>(&v[u]);
#pragma unroll
        for (int t = 0; t < 8; ++t) lds[(w * 8 + t) * R + r] = static_cast<float>(h[t]);
      }
    }
  }
  __syncthreads();
  if (K > 0) ring_run<R>(ring, lds, K, P, tid, recs);

  for (int e = tid; e < total; e += kRotThreads) {
    const int r = e / words, w = e - r * words;
    const int row = row0 + r;
    if (row >= M) continue;
    _Float16 h[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int c = w * 8 + u;
      h[PERM ? nib_slot(u) : u] = static_cast<_Float16>(lds[c * R + r] * inv_s[c]);
    }
    *reinterpret_cast<uint4*>(xout + size_t(row) * D + size_t(w) * 8) = *reinterpret_cast<const uint4*>(h);
  }
}

template <int R, int PPT, int PD, bool EXACT, bool PERM>
hipError_t launch_rows(const DevRot& Rt, int M, const uint16_t* x, uint16_t* xout, hipStream_t st) {
  const size_t lds = size_t(Rt.D) * R * sizeof(float);
  if (lds > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&rotate_rows_kernel<R, PPT, PD, EXACT, PERM>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, int(lds));
    if (e != hipSuccess) return e;
  }
  const int blocks = (M + R - 1) / R;
  hipLaunchKernelGGL((rotate_rows_kernel<R, PPT, PD, EXACT, PERM>), dim3(blocks), dim3(kRotThreads), lds, st, x,
                     xout, M, Rt.D, Rt.K, Rt.rec, Rt.inv_s);
  return hipGetLastError();
}

template <int R, int PPT, int PD, bool PERM>
hipError_t launch_exact(const DevRot& Rt, int M, const uint16_t* x, uint16_t* xout, hipStream_t st) {
  if (Rt.D / 2 == PPT * kRotThreads) return launch_rows<R, PPT, PD, true, PERM>(Rt, M, x, xout, st);
  return launch_rows<R, PPT, PD, false, PERM>(Rt, M, x, xout, st);
}

template <int R, bool PERM>
hipError_t launch_ppt(const DevRot& Rt, int M, const uint16_t* x, uint16_t* xout, hipStream_t st) {
  const int ppt = (Rt.D / 2 + kRotThreads - 1) / kRotThreads;  // pairs per thread per stage
  if (ppt <= 1) return launch_exact<R, 1, 8, PERM>(Rt, M, x, xout, st);
  if (ppt <= 2) return launch_exact<R, 2, 8, PERM>(Rt, M, x, xout, st);
  if (ppt <= 3) return launch_exact<R, 3, 8, PERM>(Rt, M, x, xout, st);
  if (ppt <= 4) return launch_exact<R, 4, 4, PERM>(Rt, M, x, xout, st);
  if (ppt <= 6) return launch_exact<R, 6, 4, PERM>(Rt, M, x, xout, st);
  if (ppt <= 9) return launch_exact<R, 9, 2, PERM>(Rt, M, x, xout, st);
  if (ppt <= 12) return launch_exact<R, 12, 2, PERM>(Rt, M, x, xout, st);
  return launch_exact<R, 16, 2, PERM>(Rt, M, x, xout, st);
}

template <bool PERM>
hipError_t launch_r(const DevRot& R, int M, const uint16_t* x, uint16_t* xout, hipStream_t st) {
  // Rows per workgroup: amortize the stage parameters over several rows once there are
  // enough rows to keep >= 512 workgroups, within 80 KB of LDS (two workgroups per CU).
  const size_t row_bytes = size_t(R.D) * 4;
  if (M >= 4 * 512 && 4 * row_bytes <= 80 * 1024) return launch_ppt<4, PERM>(R, M, x, xout, st);
  if (M >= 2 * 512 && 2 * row_bytes <= 80 * 1024) return launch_ppt<2, PERM>(R, M, x, xout, st);
  return launch_ppt<1, PERM>(R, M, x, xout, st);
}

}  // namespace

hipError_t launch_rotate(const DevRot& R, int M, const uint16_t* x, uint16_t* xout, bool nibble_order,
                         hipStream_t st) {
  if (R.D / 2 > 16 * kRotThreads) return hipErrorInvalidValue;
  return nibble_order ? launch_r<true>(R, M, x, xout, st) : launch_r<false>(R, M, x, xout, st);
}

}  // namespace paro
