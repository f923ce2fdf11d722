// Runtime activation-side transform: K stages of disjoint-pair Givens rotations,
// then division by the channel scales ("ParoQuant: pairwise rotations that
// survive deployment", section "A rotation small enough to execute").
//
// One workgroup of 512 threads holds R rows in LDS as float32, interleaved by
// channel (lds[c * R + r]: one R-wide vector per channel, so a stage moves a pair
// of channels for all R rows with two vector reads and two vector writes), runs
// the K stages (rotation_core.h) and writes fp16(rows * (1/s)). Workgroups are
// persistent over blocks of R rows. Stage parameters stream through a register
// ring issued before the block's rows are loaded.
//
// LDS banks (32 on gfx950): inside a stage, the host's pair order keeps the channels
// of 8 (16, 32) consecutive lanes distinct modulo 8 (16, 32), so the R = 4 (2, 1)
// vector accesses are conflict-free. Rows move between global memory and LDS two
// adjacent channels per lane (4-byte accesses, every load of a block in flight at
// once), so a wave's vector accesses cover consecutive channels.
//
// With PERM the output keeps every 8-channel word in the order the INT4 decode of
// the linear kernels produces ([0,4,1,5,2,6,3,7]), which is how
// paro_rotated_linear hands its workspace to them.
#include <algorithm>

#include "rotation_core.h"

namespace paro {
namespace {

constexpr int kRotThreads = 512;
constexpr size_t kRotLds = 160 * 1024;
constexpr int kCUs = 256;

template <int R, int PPT, int PD, bool EXACT, bool PERM>
__global__ __launch_bounds__(kRotThreads) void rotate_rows_kernel(const uint16_t* __restrict__ x,
                                                                   uint16_t* __restrict__ xout, int M, int D,
                                                                   int K, const PairRec* recs,
                                                                   const float* __restrict__ inv_s) {
  extern __shared__ __attribute__((aligned(16))) float lds[];  // [D][R]
  const int tid = threadIdx.x;
  const int P = D / 2;
  const int nblk = (M + R - 1) / R;

  for (int blk = blockIdx.x; blk < nblk; blk += gridDim.x) {
    const int row0 = blk * R;
    StageRing<kRotThreads, PPT, PD, EXACT> ring;
    if (K > 0) ring_prime(ring, K, P, tid, recs);

    // rows -> LDS: lane = two adjacent channels (one 4-byte load per row, all of the thread's
    // loads in flight at once); a wave writes 128 consecutive channel vectors
    using V = typename RowVec<R>::T;
    V* rows = reinterpret_cast<V*>(lds);
    uintptr_t xb = reinterpret_cast<uintptr_t>(x);
    asm volatile("" : "+s"(xb));  // as for 1/s below: addresses formed where the loads issue
    const uint32_t* xr[R];
#pragma unroll
    for (int r = 0; r < R; ++r)
      xr[r] = reinterpret_cast<const uint32_t*>(reinterpret_cast<const uint16_t*>(xb) + size_t(min(row0 + r, M - 1)) * D);
    {
      uint32_t hv[PPT][R];  // channel pair cp = tid + u * NT: channels 2 cp (low half), 2 cp + 1
#pragma unroll
      for (int u = 0; u < PPT; ++u) {
        const int cp = min(tid + u * kRotThreads, P - 1);
#pragma unroll
        for (int r = 0; r < R; ++r) hv[u][r] = xr[r][cp];
      }
#pragma unroll
      for (int u = 0; u < PPT; ++u) {
        const int cp = tid + u * kRotThreads;
        if (cp < P) {
          float f0[R], f1[R];
#pragma unroll
          for (int r = 0; r < R; ++r) {
            f0[r] = static_cast<float>(__builtin_bit_cast(_Float16, uint16_t(hv[u][r])));
            f1[r] = static_cast<float>(__builtin_bit_cast(_Float16, uint16_t(hv[u][r] >> 16)));
          }
          rows[2 * cp] = *reinterpret_cast<const V*>(f0);
          rows[2 * cp + 1] = *reinterpret_cast<const V*>(f1);
        }
      }
    }
    __syncthreads();
    if (K > 0) ring_run<R>(ring, lds, K, P, tid, recs);  // ends with a barrier

    // LDS -> fp16(rows * (1/s)), rows below M only; lane = channel pair as above. The thread's
    // 1/s values are loaded together first (one memory round trip per block).
    {
      // the base is made opaque per block so the loads' addresses are formed here, not hoisted
      // out of the block loop and kept live (or spilled) across the stages
      uintptr_t isb = reinterpret_cast<uintptr_t>(inv_s), ob = reinterpret_cast<uintptr_t>(xout);
      asm volatile("" : "+s"(isb), "+s"(ob));
      float2 isv[PPT];
#pragma unroll
      for (int u = 0; u < PPT; ++u) isv[u] = reinterpret_cast<const float2*>(isb)[min(tid + u * kRotThreads, P - 1)];
#pragma unroll
      for (int u = 0; u < PPT; ++u) {
        const int cp = tid + u * kRotThreads;
        if (cp < P) {
          const V v0 = rows[2 * cp], v1 = rows[2 * cp + 1];
          const float* f0 = reinterpret_cast<const float*>(&v0);
          const float* f1 = reinterpret_cast<const float*>(&v1);
          const int c = 2 * cp;
#pragma unroll
          for (int r = 0; r < R; ++r) {
            if (row0 + r < M) {
              const uint16_t h0 = __builtin_bit_cast(uint16_t, static_cast<_Float16>(f0[r] * isv[u].x));
              const uint16_t h1 = __builtin_bit_cast(uint16_t, static_cast<_Float16>(f1[r] * isv[u].y));
              uint16_t* out = reinterpret_cast<uint16_t*>(ob) + size_t(row0 + r) * D;
              if constexpr (PERM) {  // channels c, c + 1 sit apart in the decode order
                out[(c & ~7) | nib_slot(c & 7)] = h0;
                out[(c & ~7) | nib_slot((c + 1) & 7)] = h1;
              } else {
                reinterpret_cast<uint32_t*>(out)[cp] = uint32_t(h0) | (uint32_t(h1) << 16);
              }
            }
          }
        }
      }
    }
    __syncthreads();  // the next block overwrites the rows
  }
}

template <int R, int PPT, int PD, bool EXACT, bool PERM>
hipError_t launch_rows(const DevRot& Rt, int M, const uint16_t* x, uint16_t* xout, hipStream_t st) {
  const size_t lds = size_t(Rt.D) * R * sizeof(float);
  const void* fn = reinterpret_cast<const void*>(&rotate_rows_kernel<R, PPT, PD, EXACT, PERM>);
  if (lds > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, int(lds));
    if (e != hipSuccess) return e;
  }
  const long nblk = (M + R - 1) / R;
  const long per_cu = std::max<long>(1, long(kRotLds / lds));  // workgroups one CU holds at once
  const int grid = int(std::min<long>(nblk, per_cu * kCUs));
  hipLaunchKernelGGL((rotate_rows_kernel<R, PPT, PD, EXACT, PERM>), dim3(grid), dim3(kRotThreads), lds, st, x,
                     xout, M, Rt.D, Rt.K, Rt.rec, Rt.inv_s);
  return hipGetLastError();
}

template <int R, int PPT, int PD, bool PERM>
hipError_t launch_exact(const DevRot& Rt, int M, const uint16_t* x, uint16_t* xout, hipStream_t st) {
  if (Rt.D / 2 == PPT * kRotThreads) return launch_rows<R, PPT, PD, true, PERM>(Rt, M, x, xout, st);
  return launch_rows<R, PPT, PD, false, PERM>(Rt, M, x, xout, st);
}

// Pairs per thread per stage (PPT) and its ring depth; R rows take PPT up to kMaxPpt<R>
// (beyond it the float32 rows and the records outgrow the registers).
template <int R>
constexpr int kMaxPpt = R == 4 ? 9 : 16;

template <int R, bool PERM>
hipError_t launch_ppt(const DevRot& Rt, int M, const uint16_t* x, uint16_t* xout, hipStream_t st) {
  const int ppt = (Rt.D / 2 + kRotThreads - 1) / kRotThreads;
  if (ppt <= 1) return launch_exact<R, 1, 8, PERM>(Rt, M, x, xout, st);
  if (ppt <= 2) return launch_exact<R, 2, 8, PERM>(Rt, M, x, xout, st);
  if (ppt <= 3) return launch_exact<R, 3, 4, PERM>(Rt, M, x, xout, st);
  if (ppt <= 4) return launch_exact<R, 4, 4, PERM>(Rt, M, x, xout, st);
  if (ppt <= 6) return launch_exact<R, 6, 2, PERM>(Rt, M, x, xout, st);
  if (ppt <= 9) return launch_exact<R, 9, 2, PERM>(Rt, M, x, xout, st);
  if constexpr (kMaxPpt<R> >= 12)
    if (ppt <= 12) return launch_exact<R, 12, 2, PERM>(Rt, M, x, xout, st);
  if constexpr (kMaxPpt<R> >= 14)
    if (ppt <= 14) return launch_exact<R, 14, 1, PERM>(Rt, M, x, xout, st);
  if constexpr (kMaxPpt<R> >= 16) return launch_exact<R, 16, 1, PERM>(Rt, M, x, xout, st);
  return hipErrorInvalidValue;
}

template <bool PERM>
hipError_t launch_r(const DevRot& R, int M, const uint16_t* x, uint16_t* xout, hipStream_t st) {
  // Rows per workgroup: a stage's parameters are read once per block, so larger blocks
  // save their traffic once there are enough rows to give every CU a block.
  const size_t row_bytes = size_t(R.D) * 4;
  const int ppt = (R.D / 2 + kRotThreads - 1) / kRotThreads;
  if (M >= 4 * kCUs && 4 * row_bytes <= kRotLds && ppt <= kMaxPpt<4>) return launch_ppt<4, PERM>(R, M, x, xout, st);
  if (M >= 2 * kCUs && 2 * row_bytes <= kRotLds && ppt <= kMaxPpt<2>) return launch_ppt<2, PERM>(R, M, x, xout, st);
  return launch_ppt<1, PERM>(R, M, x, xout, st);
}

}  // namespace

hipError_t launch_rotate(const DevRot& R, int M, const uint16_t* x, uint16_t* xout, bool nibble_order,
                         hipStream_t st) {
  if (R.D / 2 > 16 * kRotThreads) return hipErrorInvalidValue;
  return nibble_order ? launch_r<true>(R, M, x, xout, st) : launch_r<false>(R, M, x, xout, st);
}

}  // namespace paro
