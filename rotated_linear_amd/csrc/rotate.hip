// Runtime activation-side transform: K stages of disjoint-pair Givens rotations,
// then division by the channel scales ("ParoQuant: pairwise rotations that
// survive deployment", section "A rotation small enough to execute").
//
// One workgroup transforms R rows. The rows live in LDS as float32 for all K
// stages, interleaved by channel (lds[c][r]), so one LDS access moves a pair's
// element for all R rows. Each thread owns pairs p = tid, tid + NT, ...; the
// pairs of a stage touch disjoint channels, so a stage is one pass with no
// write conflicts and one barrier. The pair list and (cos, sin) of stage k+1
// are fetched into registers while stage k computes. 1/s is applied on the
// way out, with one float32 -> float16 rounding.
#include "paro_internal.h"

namespace paro {
namespace {

template <int R>
struct RowVec {
  using T = float __attribute__((ext_vector_type(R)));
};
template <>
struct RowVec<1> {
  using T = float;
};

constexpr int kRotThreads = 512;
constexpr int kMaxPairsPerThread = PARO_MAX_D / 2 / kRotThreads;  // 16

template <int R>
__global__ __launch_bounds__(kRotThreads) void rotate_rows_kernel(const uint16_t* __restrict__ x,
                                                                   uint16_t* __restrict__ xout, int M, int D,
                                                                   int K, const uint32_t* __restrict__ pairs,
                                                                   const float2* __restrict__ cs,
                                                                   const float* __restrict__ inv_s) {
  using V = typename RowVec<R>::T;
  extern __shared__ float lds[];  // [D][R]
  V* rows = reinterpret_cast<V*>(lds);
  const int tid = threadIdx.x;
  const int row0 = blockIdx.x * R;
  const int chunks = D / 8;  // 8 halves = 16 bytes per global access

  for (int e = tid; e < chunks * R; e += kRotThreads) {
    const int r = e / chunks, c8 = e - r * chunks;
    const int row = row0 + r;
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    if (row < M) v = *reinterpret_cast<const uint4*>(x + size_t(row) * D + c8 * 8);
    const _Float16* h = reinterpret_cast<const _Float16*>(&v);
#pragma unroll
    for (int t = 0; t < 8; ++t) lds[(c8 * 8 + t) * R + r] = static_cast<float>(h[t]);
  }

  const int P = D / 2;
  const int npp = (P - tid + kRotThreads - 1) / kRotThreads;  // pairs this thread owns per stage
  uint32_t ij[kMaxPairsPerThread];
  float2 t[kMaxPairsPerThread];
  if (K > 0) {
#pragma unroll
    for (int q = 0; q < kMaxPairsPerThread; ++q)
      if (q < npp) {
        ij[q] = pairs[tid + q * kRotThreads];
        t[q] = cs[tid + q * kRotThreads];
      }
  }
  __syncthreads();

  for (int k = 0; k < K; ++k) {
    uint32_t nij[kMaxPairsPerThread];
    float2 nt[kMaxPairsPerThread];
    const bool more = k + 1 < K;
#pragma unroll
    for (int q = 0; q < kMaxPairsPerThread; ++q)
      if (more && q < npp) {
        nij[q] = pairs[size_t(k + 1) * P + tid + q * kRotThreads];
        nt[q] = cs[size_t(k + 1) * P + tid + q * kRotThreads];
      }
#pragma unroll
    for (int q = 0; q < kMaxPairsPerThread; ++q)
      if (q < npp) {
        const int i = int(ij[q] & 0xFFFFu), j = int(ij[q] >> 16);
        const float c = t[q].x, s = t[q].y;
        const V vi = rows[i], vj = rows[j];
        rows[i] = c * vi + s * vj;
        rows[j] = c * vj - s * vi;
      }
    __syncthreads();
    if (more) {
#pragma unroll
      for (int q = 0; q < kMaxPairsPerThread; ++q)
        if (q < npp) {
          ij[q] = nij[q];
          t[q] = nt[q];
        }
    }
  }

  for (int e = tid; e < chunks * R; e += kRotThreads) {
    const int r = e / chunks, c8 = e - r * chunks;
    const int row = row0 + r;
    if (row >= M) continue;
    _Float16 h[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int c = c8 * 8 + u;
      h[u] = static_cast<_Float16>(lds[c * R + r] * inv_s[c]);
    }
    *reinterpret_cast<uint4*>(xout + size_t(row) * D + c8 * 8) = *reinterpret_cast<const uint4*>(h);
  }
}

template <int R>
hipError_t launch_rows(const DevRot& Rt, int M, const uint16_t* x, uint16_t* xout, hipStream_t st) {
  const size_t lds = size_t(Rt.D) * R * sizeof(float);
  if (lds > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&rotate_rows_kernel<R>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, int(lds));
    if (e != hipSuccess) return e;
  }
  const int blocks = (M + R - 1) / R;
  hipLaunchKernelGGL(rotate_rows_kernel<R>, dim3(blocks), dim3(kRotThreads), lds, st, x, xout, M, Rt.D, Rt.K,
                     Rt.pairs, Rt.cs, Rt.inv_s);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_rotate(const DevRot& R, int M, const uint16_t* x, uint16_t* xout, hipStream_t st) {
  // Rows per workgroup: as many as keep the LDS image within 80 KB (two workgroups per CU),
  // but no more than the batch has.
  const size_t row_bytes = size_t(R.D) * 4;
  if (M >= 4 && 4 * row_bytes <= 80 * 1024) return launch_rows<4>(R, M, x, xout, st);
  if (M >= 2 && 2 * row_bytes <= 80 * 1024) return launch_rows<2>(R, M, x, xout, st);
  return launch_rows<1>(R, M, x, xout, st);
}

}  // namespace paro
