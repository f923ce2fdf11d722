// Prefill-shaped W4A16 linear on the gfx950 matrix cores.
//
// y[m][n] = sum_g scale[n][g] * sum_{k in g} x[m][k] * (q[n][k] - z[n][g])
// (group-wise INT4 GEMM, "ParoQuant: pairwise rotations that survive
// deployment", section "From fake quantization to a real TensorRT engine";
// group size 128, section "My reduced-calibration experiment").
//
// Design:
//   * the K loop walks one 128-channel quantization group at a time;
//   * the group's A tile (x or the transformed x, float16) and the group's
//     dequantized B tile are staged in LDS. B holds the exact integers (q - z)
//     as float16 (nibble -> 1024 + q by an AND-OR with the 0x6400 exponent
//     pattern, minus 1024 + z, both exact), so v_mfma_f32_16x16x32_f16 forms
//     exact products summed in float32;
//   * the per-(n, group) scale is applied in float32 after the group's MFMAs
//     (acc += scale * acc_group), never folded into float16 weights;
//   * the AND-OR decode of a 32-bit word yields channels in the order
//     [0,4,1,5,2,6,3,7]; the A tile is written to LDS with every 8-channel
//     word permuted the same way, so A and B agree on the reduction order;
//   * the next group's global loads are issued before the current group's
//     MFMAs (register double buffering).
#include "paro_internal.h"

namespace paro {
namespace {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef float f4 __attribute__((ext_vector_type(4)));

constexpr int BK = PARO_GROUP;   // one group per K step
constexpr int LDA = BK + 8;      // LDS row stride in halves (16-byte pad)

__device__ inline uint32_t dq2(uint32_t u, uint32_t zz) {
  // (1024 + q) - (1024 + z) for the two nibbles selected by 0x000F000F
  const h2 v = __builtin_bit_cast(h2, (u & 0x000F000Fu) | 0x64006400u) - __builtin_bit_cast(h2, zz);
  return __builtin_bit_cast(uint32_t, v);
}

template <int BM, int BN, int WM, int WN>
struct Cfg {
  static constexpr int kWaves = WM * WN;
  static constexpr int kThreads = 64 * kWaves;
  static constexpr int TM = BM / WM / 16;  // 16x16 tiles per wave along M
  static constexpr int TN = BN / WN / 16;  // along N
  static constexpr int A_VEC = BM * BK / 8 / kThreads;  // 16-byte A loads per thread per group
  static constexpr int B_VEC = BN * BK / 32 / kThreads;  // 16-byte qweight loads per thread per group
  static constexpr size_t kLds = size_t(BM + BN) * LDA * 2 + BN * 4;
  static_assert(BM * BK / 8 % kThreads == 0, "A tile split");
  static_assert(BN * BK / 32 % kThreads == 0 || B_VEC == 0, "B tile split");
};

template <int BM, int BN, int WM, int WN>
__global__ __launch_bounds__(64 * WM * WN) void gemm_kernel(
    int M, int D, int N, const uint16_t* __restrict__ x, const uint8_t* __restrict__ qweight,
    const uint16_t* __restrict__ scales, const uint16_t* __restrict__ zeros, void* __restrict__ y, int ydtype) {
  using C = Cfg<BM, BN, WM, WN>;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  _Float16* As = reinterpret_cast<_Float16*>(smem);  // [BM][LDA]
  _Float16* Bs = As + BM * LDA;                       // [BN][LDA]
  float* Ss = reinterpret_cast<float*>(Bs + BN * LDA);  // [BN]

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;
  const int m0 = blockIdx.y * BM, n0 = blockIdx.x * BN;
  const int G = D / BK;

  // per-thread staging registers
  uint4 areg[C::A_VEC];
  uint4 breg[C::B_VEC > 0 ? C::B_VEC : 1];
  uint32_t zreg[C::B_VEC > 0 ? C::B_VEC : 1];
  float sreg[C::B_VEC > 0 ? C::B_VEC : 1];

  auto load_group = [&](int g) {
#pragma unroll
    for (int i = 0; i < C::A_VEC; ++i) {
      const int idx = tid + i * C::kThreads;
      const int r = idx / (BK / 8), w = idx % (BK / 8);
      const int m = m0 + r;
      areg[i] = m < M ? *reinterpret_cast<const uint4*>(x + size_t(m) * D + size_t(g) * BK + w * 8)
                      : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int i = 0; i < C::B_VEC; ++i) {
      const int idx = tid + i * C::kThreads;
      const int r = idx / (BK / 32), w = idx % (BK / 32);
      const int n = n0 + r;
      if (n < N) {
        breg[i] = *reinterpret_cast<const uint4*>(qweight + size_t(n) * (D / 2) + size_t(g) * (BK / 2) + w * 16);
        const _Float16 z = __builtin_bit_cast(_Float16, zeros[size_t(n) * G + g]);
        const _Float16 zz = static_cast<_Float16>(1024.0f) + z;
        zreg[i] = uint32_t(__builtin_bit_cast(uint16_t, zz)) * 0x10001u;
        sreg[i] = static_cast<float>(__builtin_bit_cast(_Float16, scales[size_t(n) * G + g]));
      } else {
        breg[i] = make_uint4(0u, 0u, 0u, 0u);
        zreg[i] = 0x64006400u;
        sreg[i] = 0.f;
      }
    }
  };

  auto store_group = [&]() {
#pragma unroll
    for (int i = 0; i < C::A_VEC; ++i) {
      const int idx = tid + i * C::kThreads;
      const int r = idx / (BK / 8), w = idx % (BK / 8);
      const h8 v = __builtin_bit_cast(h8, areg[i]);
      const h8 p = __builtin_shufflevector(v, v, 0, 4, 1, 5, 2, 6, 3, 7);
      *reinterpret_cast<h8*>(As + r * LDA + w * 8) = p;
    }
#pragma unroll
    for (int i = 0; i < C::B_VEC; ++i) {
      const int idx = tid + i * C::kThreads;
      const int r = idx / (BK / 32), w = idx % (BK / 32);
      const uint32_t wv[4] = {breg[i].x, breg[i].y, breg[i].z, breg[i].w};
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const uint32_t u = wv[t];
        uint4 o;
        o.x = dq2(u, zreg[i]);        // ch 0, 4
        o.y = dq2(u >> 4, zreg[i]);   // ch 1, 5
        o.z = dq2(u >> 8, zreg[i]);   // ch 2, 6
        o.w = dq2(u >> 12, zreg[i]);  // ch 3, 7
        *reinterpret_cast<uint4*>(Bs + r * LDA + w * 32 + t * 8) = o;
      }
      if (w == 0) Ss[r] = sreg[i];
    }
  };

  f4 acc[C::TM][C::TN];
  f4 accg[C::TM][C::TN];
#pragma unroll
  for (int i = 0; i < C::TM; ++i)
#pragma unroll
    for (int j = 0; j < C::TN; ++j) acc[i][j] = f4{0.f, 0.f, 0.f, 0.f};

  const int lrow = lane & 15, lk = (lane >> 4) * 8;
  load_group(0);
  for (int g = 0; g < G; ++g) {
    __syncthreads();
    store_group();
    __syncthreads();
    if (g + 1 < G) load_group(g + 1);
#pragma unroll
    for (int i = 0; i < C::TM; ++i)
#pragma unroll
      for (int j = 0; j < C::TN; ++j) accg[i][j] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < BK; kk += 32) {
      h8 af[C::TM], bf[C::TN];
#pragma unroll
      for (int i = 0; i < C::TM; ++i)
        af[i] = *reinterpret_cast<const h8*>(As + (wm * C::TM * 16 + i * 16 + lrow) * LDA + kk + lk);
#pragma unroll
      for (int j = 0; j < C::TN; ++j)
        bf[j] = *reinterpret_cast<const h8*>(Bs + (wn * C::TN * 16 + j * 16 + lrow) * LDA + kk + lk);
#pragma unroll
      for (int i = 0; i < C::TM; ++i)
#pragma unroll
        for (int j = 0; j < C::TN; ++j)
          accg[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[i], bf[j], accg[i][j], 0, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < C::TN; ++j) {
      const float sc = Ss[wn * C::TN * 16 + j * 16 + lrow];
#pragma unroll
      for (int i = 0; i < C::TM; ++i) acc[i][j] += sc * accg[i][j];
    }
  }

  // C tile layout of v_mfma_f32_16x16x32_f16: lane holds column (lane & 15),
  // rows 4 * (lane >> 4) + r, r = 0..3.
#pragma unroll
  for (int i = 0; i < C::TM; ++i)
#pragma unroll
    for (int j = 0; j < C::TN; ++j) {
      const int n = n0 + wn * C::TN * 16 + j * 16 + lrow;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = m0 + wm * C::TM * 16 + i * 16 + (lane >> 4) * 4 + r;
        if (m < M && n < N) {
          if (ydtype == PARO_F32)
            static_cast<float*>(y)[size_t(m) * N + n] = acc[i][j][r];
          else
            static_cast<_Float16*>(y)[size_t(m) * N + n] = static_cast<_Float16>(acc[i][j][r]);
        }
      }
    }
}

template <int BM, int BN, int WM, int WN>
hipError_t launch_cfg(int M, int D, int N, const uint16_t* x, const uint8_t* qweight, const uint16_t* scales,
                      const uint16_t* zeros, void* y, int ydtype, hipStream_t st) {
  using C = Cfg<BM, BN, WM, WN>;
  if (C::kLds > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&gemm_kernel<BM, BN, WM, WN>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, int(C::kLds));
    if (e != hipSuccess) return e;
  }
  dim3 grid((N + BN - 1) / BN, (M + BM - 1) / BM);
  hipLaunchKernelGGL((gemm_kernel<BM, BN, WM, WN>), grid, dim3(C::kThreads), C::kLds, st, M, D, N, x, qweight,
                     scales, zeros, y, ydtype);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm(int M, int D, int N, const uint16_t* x, const uint8_t* qweight, const uint16_t* scales,
                       const uint16_t* zeros, void* y, int ydtype, hipStream_t st) {
  if (M <= 16) return launch_cfg<16, 64, 1, 4>(M, D, N, x, qweight, scales, zeros, y, ydtype, st);
  if (M <= 64) return launch_cfg<64, 64, 2, 2>(M, D, N, x, qweight, scales, zeros, y, ydtype, st);
  return launch_cfg<128, 128, 2, 2>(M, D, N, x, qweight, scales, zeros, y, ydtype, st);
}

}  // namespace paro
