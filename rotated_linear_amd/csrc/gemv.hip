// Decode-shaped W4A16 linear (small M): y[m][n] = sum_g scale[n][g] *
// sum_{k in g} x[m][k] * (q[n][k] - z[n][g]), optionally with the activation
// transform fused in front ("ParoQuant: pairwise rotations that survive
// deployment", section "A rotation small enough to execute": the inverse
// activation-side transform runs immediately before the packed INT4 linear).
//
// HBM-bound design for gfx950:
//   * a team of 16 lanes streams RPT weight rows; lane l of a team owns the
//     16-byte chunks l, l+16, ... of each row (32 channels = a quarter group),
//     so a team reads 256 contiguous bytes per row per step (coalesced);
//   * PF chunk-steps of weights (and their scale / zero) are kept in flight per
//     lane in a register ring; in the fused kernel the first PF steps are issued
//     before the transform runs, so the K dependent LDS stages overlap the
//     first HBM round trips;
//   * nibbles become float16 with one AND-OR against the 0x6400 exponent
//     pattern (low nibbles -> 1024 + q, high nibbles -> 1024 + 16 q), then the
//     zero-point is subtracted exactly in float16 ((1024 + q) - (1024 + z) =
//     q - z) and v_dot2_f32_f16 accumulates x * (q - z) in float32; the
//     high-nibble partial sum is scaled by 1/16 (exact) and the group scale is
//     applied in float32 once per 32 channels;
//   * x (or the transformed x, rounded once to float16) sits in LDS with each
//     8-channel word permuted to [0,4,2,6,1,5,3,7], the order the AND-OR
//     decode yields;
//   * the 16 lanes of a team combine their partial sums with xor shuffles.
#include "paro_internal.h"

namespace paro {
namespace {

typedef _Float16 h2 __attribute__((ext_vector_type(2)));

template <int R>
struct RowVec {
  using T = float __attribute__((ext_vector_type(R)));
};
template <>
struct RowVec<1> {
  using T = float;
};

template <int R>
__device__ inline float lane_of(const typename RowVec<R>::T& v, int r) {
  if constexpr (R == 1) {
    return v;
  } else {
    return v[r];
  }
}

constexpr int kThreads = 256;
constexpr int kTeam = 16;
constexpr int kTeams = kThreads / kTeam;
constexpr int kPF = 4;  // chunk-steps in flight per lane

// slot of channel offset e (0..7) inside its permuted 8-channel word
__device__ inline int perm_slot(int e) { return ((e & 1) << 2) | ((e >> 2) & 1) | (e & 2); }

__device__ inline h2 as_h2(uint32_t v) { return __builtin_bit_cast(h2, v); }

template <int MR, bool FUSED, int RPT>
__global__ __launch_bounds__(kThreads) void gemv_kernel(int M, int D, int N, int K, const uint16_t* __restrict__ x,
                                                         const uint8_t* __restrict__ qweight,
                                                         const uint16_t* __restrict__ scales,
                                                         const uint16_t* __restrict__ zeros, void* __restrict__ y,
                                                         int ydtype, const uint32_t* __restrict__ pairs,
                                                         const float2* __restrict__ cs,
                                                         const float* __restrict__ inv_s) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  _Float16* xs = reinterpret_cast<_Float16*>(smem);  // [MR][D], permuted words
  const int tid = threadIdx.x;
  const int team = tid / kTeam, tl = tid % kTeam;
  const int n0 = (blockIdx.x * kTeams + team) * RPT;
  const int CPR = D / 32;  // 16-byte chunks per weight row
  const int G = D / PARO_GROUP;
  const int S = (CPR + kTeam - 1) / kTeam;

  // ---- weight prefetch ring (issued first so the fused transform hides under it)
  uint4 wbuf[kPF][RPT];
  uint32_t szbuf[kPF][RPT];  // scale bits | zero bits << 16
  auto issue = [&](int slot_s, uint4 (&wb)[RPT], uint32_t (&sz)[RPT]) {
    const int c = tl + kTeam * slot_s;
#pragma unroll
    for (int rr = 0; rr < RPT; ++rr) {
      const int n = n0 + rr;
      if (slot_s < S && c < CPR && n < N) {
        wb[rr] = *reinterpret_cast<const uint4*>(qweight + size_t(n) * (D / 2) + size_t(c) * 16);
        const size_t gi = size_t(n) * G + (c >> 2);
        sz[rr] = uint32_t(scales[gi]) | (uint32_t(zeros[gi]) << 16);
      } else {
        wb[rr] = make_uint4(0u, 0u, 0u, 0u);
        sz[rr] = 0u;
      }
    }
  };
#pragma unroll
  for (int q = 0; q < kPF; ++q) issue(q, wbuf[q], szbuf[q]);

  // ---- activations into LDS (transformed when FUSED)
  const int words = D / 8;
  if constexpr (FUSED) {
    using V = typename RowVec<MR>::T;
    float* rot = reinterpret_cast<float*>(smem + size_t(MR) * D * 2);  // [D][MR]
    V* rows = reinterpret_cast<V*>(rot);
    for (int e = tid; e < words * MR; e += kThreads) {
      const int m = e / words, w = e - m * words;
      uint4 v = make_uint4(0u, 0u, 0u, 0u);
      if (m < M) v = *reinterpret_cast<const uint4*>(x + size_t(m) * D + w * 8);
      const _Float16* h = reinterpret_cast<const _Float16*>(&v);
#pragma unroll
      for (int u = 0; u < 8; ++u) rot[(w * 8 + u) * MR + m] = static_cast<float>(h[u]);
    }
    __syncthreads();
    const int P = D / 2;
    for (int k = 0; k < K; ++k) {
      for (int p = tid; p < P; p += kThreads) {
        const uint32_t ij = pairs[size_t(k) * P + p];
        const float2 t = cs[size_t(k) * P + p];
        const int i = int(ij & 0xFFFFu), j = int(ij >> 16);
        const V vi = rows[i], vj = rows[j];
        rows[i] = t.x * vi + t.y * vj;
        rows[j] = t.x * vj - t.y * vi;
      }
      __syncthreads();
    }
    for (int e = tid; e < words * MR; e += kThreads) {
      const int m = e / words, w = e - m * words;
      _Float16 h[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int c = w * 8 + u;
        h[perm_slot(u)] = static_cast<_Float16>(rot[c * MR + m] * inv_s[c]);
      }
      *reinterpret_cast<uint4*>(xs + size_t(m) * D + w * 8) = *reinterpret_cast<const uint4*>(h);
    }
  } else {
    for (int e = tid; e < words * MR; e += kThreads) {
      const int m = e / words, w = e - m * words;
      uint4 v = make_uint4(0u, 0u, 0u, 0u);
      if (m < M) v = *reinterpret_cast<const uint4*>(x + size_t(m) * D + w * 8);
      const _Float16* h = reinterpret_cast<const _Float16*>(&v);
      _Float16 o[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) o[perm_slot(u)] = h[u];
      *reinterpret_cast<uint4*>(xs + size_t(m) * D + w * 8) = *reinterpret_cast<const uint4*>(o);
    }
  }
  __syncthreads();

  // ---- stream the weights
  float acc[MR][RPT];
#pragma unroll
  for (int m = 0; m < MR; ++m)
#pragma unroll
    for (int rr = 0; rr < RPT; ++rr) acc[m][rr] = 0.f;

  for (int s0 = 0; s0 < S; s0 += kPF) {
#pragma unroll
    for (int q = 0; q < kPF; ++q) {
      const int s = s0 + q;
      const int c = tl + kTeam * s;
      if (s < S && c < CPR) {
        uint4 xv[MR][4];
#pragma unroll
        for (int m = 0; m < MR; ++m)
#pragma unroll
          for (int w = 0; w < 4; ++w)
            xv[m][w] = *reinterpret_cast<const uint4*>(xs + size_t(m) * D + size_t(c) * 32 + w * 8);
#pragma unroll
        for (int rr = 0; rr < RPT; ++rr) {
          const uint32_t sz = szbuf[q][rr];
          const float sc = static_cast<float>(__builtin_bit_cast(_Float16, uint16_t(sz & 0xFFFFu)));
          const _Float16 z = __builtin_bit_cast(_Float16, uint16_t(sz >> 16));
          const _Float16 zl = static_cast<_Float16>(1024.0f) + z;
          const _Float16 zh = static_cast<_Float16>(1024.0f) + static_cast<_Float16>(16.0f) * z;
          const h2 zl2 = {zl, zl}, zh2 = {zh, zh};
          float al[MR], ah[MR];
#pragma unroll
          for (int m = 0; m < MR; ++m) al[m] = ah[m] = 0.f;
          const uint32_t wv[4] = {wbuf[q][rr].x, wbuf[q][rr].y, wbuf[q][rr].z, wbuf[q][rr].w};
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            const uint32_t u = wv[w], u8 = u >> 8;
            const h2 lo0 = as_h2((u & 0x000F000Fu) | 0x64006400u) - zl2;   // ch 0, 4
            const h2 hi0 = as_h2((u & 0x00F000F0u) | 0x64006400u) - zh2;   // ch 1, 5 (x16)
            const h2 lo1 = as_h2((u8 & 0x000F000Fu) | 0x64006400u) - zl2;  // ch 2, 6
            const h2 hi1 = as_h2((u8 & 0x00F000F0u) | 0x64006400u) - zh2;  // ch 3, 7 (x16)
#pragma unroll
            for (int m = 0; m < MR; ++m) {
              const uint4 xw = xv[m][w];  // (x0,x4) (x2,x6) (x1,x5) (x3,x7)
              al[m] = __builtin_amdgcn_fdot2(lo0, as_h2(xw.x), al[m], false);
              al[m] = __builtin_amdgcn_fdot2(lo1, as_h2(xw.y), al[m], false);
              ah[m] = __builtin_amdgcn_fdot2(hi0, as_h2(xw.z), ah[m], false);
              ah[m] = __builtin_amdgcn_fdot2(hi1, as_h2(xw.w), ah[m], false);
            }
          }
#pragma unroll
          for (int m = 0; m < MR; ++m) acc[m][rr] += sc * (al[m] + 0.0625f * ah[m]);
        }
      }
      issue(s + kPF, wbuf[q], szbuf[q]);
    }
  }

  // ---- team reduction and store
#pragma unroll
  for (int m = 0; m < MR; ++m)
#pragma unroll
    for (int rr = 0; rr < RPT; ++rr) {
      float v = acc[m][rr];
      v += __shfl_xor(v, 8);
      v += __shfl_xor(v, 4);
      v += __shfl_xor(v, 2);
      v += __shfl_xor(v, 1);
      acc[m][rr] = v;
    }
#pragma unroll
  for (int m = 0; m < MR; ++m)
#pragma unroll
    for (int rr = 0; rr < RPT; ++rr) {
      const int idx = m * RPT + rr;
      const int n = n0 + rr;
      if ((idx % kTeam) == tl && m < M && n < N) {
        if (ydtype == PARO_F32)
          static_cast<float*>(y)[size_t(m) * N + n] = acc[m][rr];
        else
          static_cast<_Float16*>(y)[size_t(m) * N + n] = static_cast<_Float16>(acc[m][rr]);
      }
    }
}

template <int MR, bool FUSED, int RPT>
hipError_t launch_cfg(const DevRot* rot, int M, int D, int N, const uint16_t* x, const uint8_t* qweight,
                      const uint16_t* scales, const uint16_t* zeros, void* y, int ydtype, hipStream_t st) {
  const size_t lds = size_t(MR) * D * 2 + (FUSED ? size_t(MR) * D * 4 : 0);
  if (lds > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&gemv_kernel<MR, FUSED, RPT>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, int(lds));
    if (e != hipSuccess) return e;
  }
  const int rows_per_block = kTeams * RPT;
  const int blocks = (N + rows_per_block - 1) / rows_per_block;
  hipLaunchKernelGGL((gemv_kernel<MR, FUSED, RPT>), dim3(blocks), dim3(kThreads), lds, st, M, D, N,
                     rot ? rot->K : 0, x, qweight, scales, zeros, y, ydtype, rot ? rot->pairs : nullptr,
                     rot ? rot->cs : nullptr, rot ? rot->inv_s : nullptr);
  return hipGetLastError();
}

template <int MR, bool FUSED>
hipError_t launch_rpt(const DevRot* rot, int M, int D, int N, const uint16_t* x, const uint8_t* qweight,
                      const uint16_t* scales, const uint16_t* zeros, void* y, int ydtype, hipStream_t st) {
  // rows per team: enough workgroups to cover the 256 CUs before growing per-lane work
  if (N >= 4 * kTeams * 256) return launch_cfg<MR, FUSED, 4>(rot, M, D, N, x, qweight, scales, zeros, y, ydtype, st);
  if (N >= 2 * kTeams * 256) return launch_cfg<MR, FUSED, 2>(rot, M, D, N, x, qweight, scales, zeros, y, ydtype, st);
  return launch_cfg<MR, FUSED, 1>(rot, M, D, N, x, qweight, scales, zeros, y, ydtype, st);
}

template <bool FUSED>
hipError_t launch_mr(const DevRot* rot, int M, int D, int N, const uint16_t* x, const uint8_t* qweight,
                     const uint16_t* scales, const uint16_t* zeros, void* y, int ydtype, hipStream_t st) {
  if (M == 1) return launch_rpt<1, FUSED>(rot, M, D, N, x, qweight, scales, zeros, y, ydtype, st);
  if (M == 2) return launch_rpt<2, FUSED>(rot, M, D, N, x, qweight, scales, zeros, y, ydtype, st);
  return launch_rpt<4, FUSED>(rot, M, D, N, x, qweight, scales, zeros, y, ydtype, st);
}

}  // namespace

hipError_t launch_gemv(const DevRot* rot, int M, int D, int N, const uint16_t* x, const uint8_t* qweight,
                       const uint16_t* scales, const uint16_t* zeros, void* y, int ydtype, hipStream_t st) {
  if (M < 1 || M > 4) return hipErrorInvalidValue;
  if (rot) return launch_mr<true>(rot, M, D, N, x, qweight, scales, zeros, y, ydtype, st);
  return launch_mr<false>(nullptr, M, D, N, x, qweight, scales, zeros, y, ydtype, st);
}

}  // namespace paro
