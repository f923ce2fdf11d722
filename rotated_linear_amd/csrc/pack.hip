// Build-time weight fold + group-wise asymmetric INT4 quantization + nibble packing.
//
// One workgroup per weight row. The row is rotated in float64 in LDS by the K
// stages (the 2x2 Givens equation of "ParoQuant: pairwise rotations that
// survive deployment", section "A rotation small enough to execute"),
// multiplied by the channel scales ("weight transformations are folded and
// quantized", same section), then every 128-channel group is quantized to
// 4-bit codes with a float16 scale and an integer zero-point.
//
// This file is compiled with -ffp-contract=off: each product and each sum is
// rounded on its own, so the result is bit-identical to the float64 definition
// (products c*b_i and s*b_j, then one add or subtract). Division and rint are
// the IEEE float64 operations; float64 -> float16 is rounded once, by hand,
// rather than through float32 (which could round twice).
#include "paro_internal.h"

namespace paro {
namespace {

constexpr int kPackThreads = 256;

// float64 -> float16 bits, round to nearest, ties to even; handles subnormals.
__device__ inline uint16_t f64_to_f16_bits(double v) {
  const uint64_t b = __builtin_bit_cast(uint64_t, v);
  const uint16_t sign = uint16_t((b >> 48) & 0x8000u);
  const uint64_t a = b & 0x7FFFFFFFFFFFFFFFull;
  if (a >= 0x7FF0000000000000ull) return sign | (a > 0x7FF0000000000000ull ? 0x7E00 : 0x7C00);
  const int e = int(a >> 52) - 1023;
  if (e < -26) return sign;  // below half the smallest subnormal (2^-25): rounds to zero
  const uint64_t mant = (a & ((1ull << 52) - 1)) | (1ull << 52);  // e >= -26 implies a normal double
  int shift;       // bits of `mant` dropped
  int out_exp;     // biased float16 exponent field of the unrounded result
  if (e >= -14) {  // normal float16 range
    if (e > 15) return sign | 0x7C00;
    shift = 42;
    out_exp = e + 15;
  } else {  // subnormal float16: unit 2^-24
    shift = 42 + (-14 - e);
    out_exp = 0;
  }
  uint64_t m = mant >> shift;
  const uint64_t rem = mant & ((1ull << shift) - 1);
  const uint64_t half = 1ull << (shift - 1);
  if (rem > half || (rem == half && (m & 1))) ++m;
  uint32_t bits;
  if (out_exp == 0) {
    bits = uint32_t(m);  // may carry into the smallest normal: encoding stays correct
  } else {
    // m holds 11 bits with the implicit one; a carry to 2^11 bumps the exponent
    if (m == (1ull << 11)) {
      m >>= 1;
      ++out_exp;
    }
    if (out_exp >= 31) return sign | 0x7C00;
    bits = (uint32_t(out_exp) << 10) | uint32_t(m & 0x3FF);
  }
  return sign | uint16_t(bits);
}

__device__ inline double f16_bits_to_f64(uint16_t h) {
  return static_cast<double>(static_cast<float>(__builtin_bit_cast(_Float16, h)));
}

__global__ __launch_bounds__(kPackThreads) void pack_rows_kernel(int N, int D, int K, const uint16_t* __restrict__ W,
                                                                  const PairRec* __restrict__ recs,
                                                                  const float* __restrict__ s,
                                                                  uint8_t* __restrict__ qweight,
                                                                  uint16_t* __restrict__ scales,
                                                                  uint16_t* __restrict__ zeros) {
  extern __shared__ double brow[];  // [D]
  const int n = blockIdx.x;
  const int tid = threadIdx.x;
  const uint16_t* w = W + size_t(n) * D;
  for (int c = tid; c < D; c += kPackThreads)
    brow[c] = f16_bits_to_f64(w[c]);
  __syncthreads();

  const int P = D / 2;
  for (int k = 0; k < K; ++k) {
    for (int p = tid; p < P; p += kPackThreads) {
      const PairRec r = recs[size_t(k) * P + p];
      const int i = int((r.ij & 0xFFFFu) >> 2), j = int(r.ij >> 18);  // the fields are 4 i and 4 j
      const double c = r.c, sn = r.s;
      const double bi = brow[i], bj = brow[j];
      brow[i] = c * bi + sn * bj;
      brow[j] = c * bj - sn * bi;
    }
    __syncthreads();
  }
  for (int c = tid; c < D; c += kPackThreads) brow[c] = brow[c] * static_cast<double>(s[c]);
  __syncthreads();

  const int lane = tid & 63, wave = tid >> 6;
  const int G = D / PARO_GROUP;
  // the row's group 0 and group stride in the blocked qweight layout (paro_internal.h)
  uint8_t* const qrow = qweight + qw_row_offset<size_t>(size_t(n), size_t(D));
  const size_t qstride = qw_group_stride<size_t>(size_t(n), size_t(N));
  for (int g = wave; g < G; g += kPackThreads / 64) {
    const double v0 = brow[g * PARO_GROUP + 2 * lane];
    const double v1 = brow[g * PARO_GROUP + 2 * lane + 1];
    double lo = v0 < v1 ? v0 : v1;
    double hi = v0 < v1 ? v1 : v0;
    for (int off = 32; off >= 1; off >>= 1) {
      const double olo = __shfl_xor(lo, off);
      const double ohi = __shfl_xor(hi, off);
      lo = olo < lo ? olo : lo;
      hi = ohi > hi ? ohi : hi;
    }
    double step = (hi - lo) / 15.0;
    if (step < 1e-5) step = 1e-5;
    const uint16_t s16 = f64_to_f16_bits(step);
    const double sc = f16_bits_to_f64(s16);
    double z = __builtin_rint(-lo / sc);
    z = z < 0.0 ? 0.0 : (z > 15.0 ? 15.0 : z);
    z = z + 0.0;  // canonical +0
    double q0 = __builtin_rint(v0 / sc) + z;
    double q1 = __builtin_rint(v1 / sc) + z;
    q0 = q0 < 0.0 ? 0.0 : (q0 > 15.0 ? 15.0 : q0);
    q1 = q1 < 0.0 ? 0.0 : (q1 > 15.0 ? 15.0 : q1);
    qrow[size_t(g) * qstride + lane] = uint8_t(int(q0) | (int(q1) << 4));
    if (lane == 0) {
      scales[size_t(n) * G + g] = s16;
      zeros[size_t(n) * G + g] = f64_to_f16_bits(z);
    }
  }
}

}  // namespace

hipError_t launch_pack(const DevRot& R, int N, const uint16_t* W, uint8_t* qweight, uint16_t* scales,
                       uint16_t* zeros, hipStream_t st) {
  const size_t lds = size_t(R.D) * sizeof(double);
  if (lds > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&pack_rows_kernel),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, int(lds));
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(pack_rows_kernel, dim3(N), dim3(kPackThreads), lds, st, N, R.D, R.K, W, R.rec, R.s,
                     qweight, scales, zeros);
  return hipGetLastError();
}

}  // namespace paro
