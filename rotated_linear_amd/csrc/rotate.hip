// Runtime activation-side transform: K stages of disjoint-pair Givens rotations,
// then division by the channel scales ("ParoQuant: pairwise rotations that
// survive deployment", section "A rotation small enough to execute").
//
// One workgroup of NT (512) threads holds R rows in LDS as float32, interleaved by
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

constexpr size_t kRotLds = 160 * 1024;
constexpr int kCUs = 256;

template <int NT, int R, int PPT, int PD, bool EXACT, bool PERM>
__global__ __launch_bounds__(NT) void rotate_rows_kernel(const uint16_t* __restrict__ x,
                                                                   uint16_t* __restrict__ xout, int M, int D,
                                                                   int K, const PairRec* recs,
                                                                   const float* __restrict__ inv_s) {
  extern __shared__ __attribute__((aligned(16))) float lds[];  // [D][R]
  const int tid = threadIdx.x;
  const int P = D / 2;
  const int nblk = (M + R - 1) / R;

  for (int blk = blockIdx.x; blk < nblk; blk += gridDim.x) {
    const int row0 = blk * R;
    StageRing<NT, PPT, PD, EXACT> ring;
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
        const int cp = min(tid + u * NT, P - 1);
#pragma unroll
        for (int r = 0; r < R; ++r) hv[u][r] = xr[r][cp];
      }
#pragma unroll
      for (int u = 0; u < PPT; ++u) {
        const int cp = tid + u * NT;
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

    // LDS -> fp16(rows * (1/s)), rows below M only, one 32-bit word per row per lane: the
    // adjacent channels (2j, 2j + 1), or with PERM channels (e, e + 4) of 8-channel chunk c8
    // (j = 4 c8 + e), which sit side by side in the decode order. The thread's 1/s values are
    // loaded together first (one memory round trip per block).
    {
      // the bases are made opaque per block so the loads' addresses are formed here, not hoisted
      // out of the block loop and kept live (or spilled) across the stages
      uintptr_t isb = reinterpret_cast<uintptr_t>(inv_s), ob = reinterpret_cast<uintptr_t>(xout);
      asm volatile("" : "+s"(isb), "+s"(ob));
      const float* isp = reinterpret_cast<const float*>(isb);
      float isa[PPT], isc[PPT];
#pragma unroll
      for (int u = 0; u < PPT; ++u) {
        const int j = min(tid + u * NT, P - 1);
        const int ca = PERM ? 8 * (j >> 2) + (j & 3) : 2 * j, cb = PERM ? ca + 4 : ca + 1;
        isa[u] = isp[ca];
        isc[u] = isp[cb];
      }
#pragma unroll
      for (int u = 0; u < PPT; ++u) {
        const int j = tid + u * NT;
        if (j < P) {
          const int ca = PERM ? 8 * (j >> 2) + (j & 3) : 2 * j, cb = PERM ? ca + 4 : ca + 1;
          const V va = rows[ca], vb = rows[cb];
          const float* fa = reinterpret_cast<const float*>(&va);
          const float* fb = reinterpret_cast<const float*>(&vb);
#pragma unroll
          for (int r = 0; r < R; ++r) {
            if (row0 + r < M) {
              const uint32_t lo = __builtin_bit_cast(uint16_t, static_cast<_Float16>(fa[r] * isa[u]));
              const uint32_t hi = __builtin_bit_cast(uint16_t, static_cast<_Float16>(fb[r] * isc[u]));
              reinterpret_cast<uint32_t*>(reinterpret_cast<uint16_t*>(ob) + size_t(row0 + r) * D)[j] = lo | (hi << 16);
            }
          }
        }
      }
    }
    __syncthreads();  // the next block overwrites the rows
  }
}

template <int NT, int R, int PPT, int PD, bool EXACT, bool PERM>
hipError_t launch_rows(const DevRot& Rt, int M, const uint16_t* x, uint16_t* xout, hipStream_t st) {
  const size_t lds = size_t(Rt.D) * R * sizeof(float);
  const void* fn = reinterpret_cast<const void*>(&rotate_rows_kernel<NT, R, PPT, PD, EXACT, PERM>);
  if (lds > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, int(lds));
    if (e != hipSuccess) return e;
  }
  const long nblk = (M + R - 1) / R;
  const long per_cu = std::max<long>(1, long(kRotLds / lds));  // workgroups one CU holds at once
  const int grid = int(std::min<long>(nblk, per_cu * kCUs));
  hipLaunchKernelGGL((rotate_rows_kernel<NT, R, PPT, PD, EXACT, PERM>), dim3(grid), dim3(NT), lds, st, x, xout, M,
                     Rt.D, Rt.K, Rt.rec, Rt.inv_s);
  return hipGetLastError();
}

template <int NT, int R, int PPT, int PD, bool PERM>
hipError_t launch_exact(const DevRot& Rt, int M, const uint16_t* x, uint16_t* xout, hipStream_t st) {
  if (Rt.D / 2 == PPT * NT) return launch_rows<NT, R, PPT, PD, true, PERM>(Rt, M, x, xout, st);
  return launch_rows<NT, R, PPT, PD, false, PERM>(Rt, M, x, xout, st);
}

// Threads, pairs per thread per stage (PPT) and ring depth by row width (the ring is shallower
// for wide rows, whose records and row vectors take more registers).
template <int R, bool PERM>
hipError_t launch_ppt(const DevRot& Rt, int M, const uint16_t* x, uint16_t* xout, hipStream_t st) {
  const int P = Rt.D / 2;
  if (P <= 512) return launch_exact<512, R, 1, 8, PERM>(Rt, M, x, xout, st);
  if (P <= 1024) return launch_exact<512, R, 2, 8, PERM>(Rt, M, x, xout, st);
  if (P <= 1536) return launch_exact<512, R, 3, 4, PERM>(Rt, M, x, xout, st);
  if (P <= 2048) return launch_exact<512, R, 4, 4, PERM>(Rt, M, x, xout, st);
  if (P <= 3072) return launch_exact<512, R, 6, 2, PERM>(Rt, M, x, xout, st);
  if (P <= 4608) return launch_exact<512, R, 9, 2, PERM>(Rt, M, x, xout, st);
  if constexpr (R <= 2) {  // wider rows (D > 9216) never take 4 rows per workgroup
    if (P <= 6144) return launch_exact<512, R, 12, 2, PERM>(Rt, M, x, xout, st);
    if (P <= 7168) return launch_exact<512, R, 14, 1, PERM>(Rt, M, x, xout, st);
    return launch_exact<512, R, 16, 1, PERM>(Rt, M, x, xout, st);
  }
  return hipErrorInvalidValue;
}

template <bool PERM>
hipError_t launch_r(const DevRot& R, int M, const uint16_t* x, uint16_t* xout, hipStream_t st) {
  // Rows per workgroup: a stage's parameters are read once per block, so larger blocks
  // save their traffic once there are enough rows to give every CU a block.
  const size_t row_bytes = size_t(R.D) * 4;
  if (M >= 4 * kCUs && 4 * row_bytes <= kRotLds && R.D <= 9216) return launch_ppt<4, PERM>(R, M, x, xout, st);
  if (M >= 2 * kCUs && 2 * row_bytes <= kRotLds) return launch_ppt<2, PERM>(R, M, x, xout, st);
  return launch_ppt<1, PERM>(R, M, x, xout, st);
}

}  // namespace

hipError_t launch_rotate(const DevRot& R, int M, const uint16_t* x, uint16_t* xout, bool nibble_order,
                         hipStream_t st) {
  if (R.D / 2 > 8 * 1024) return hipErrorInvalidValue;
  return nibble_order ? launch_r<true>(R, M, x, xout, st) : launch_r<false>(R, M, x, xout, st);
}

}  // namespace paro
