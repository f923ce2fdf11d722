// Internal declarations shared by the host API and the kernel translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "paro.h"

namespace paro {

inline size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

// Device descriptor of a prepared transform. Four sections, each 256-byte aligned:
//   pairs  uint32 [K][D/2]   i | (j << 16)
//   cs     float2 [K][D/2]   (cos, sin) rounded once to float32
//   inv_s  float  [D]        1/s rounded once to float32 (activation side)
//   s      float  [D]        s (weight side)
struct DescLayout {
  size_t pairs_off, cs_off, inv_s_off, s_off, total;
};

inline DescLayout desc_layout(int K, int D) {
  DescLayout L;
  const size_t P = size_t(K) * size_t(D / 2);
  L.pairs_off = 0;
  L.cs_off = align256(P * 4);
  L.inv_s_off = L.cs_off + align256(P * 8);
  L.s_off = L.inv_s_off + align256(size_t(D) * 4);
  L.total = L.s_off + align256(size_t(D) * 4);
  return L;
}

struct DevRot {
  int K, D;
  const uint32_t* pairs;
  const float2* cs;
  const float* inv_s;
  const float* s;
};

inline DevRot dev_rot(const paro_rotation& r) {
  const DescLayout L = desc_layout(r.K, r.D);
  const char* base = static_cast<const char*>(r.dev);
  return DevRot{r.K, r.D, reinterpret_cast<const uint32_t*>(base + L.pairs_off),
                reinterpret_cast<const float2*>(base + L.cs_off),
                reinterpret_cast<const float*>(base + L.inv_s_off),
                reinterpret_cast<const float*>(base + L.s_off)};
}

// Largest M the single-kernel decode path (transform fused into the GEMV) takes.
constexpr int kFusedMaxM = 4;
// Largest M the GEMV path takes; above it the MFMA GEMM runs.
constexpr int kGemvMaxM = 4;

// Whether paro_rotated_linear runs its transform inside the decode kernel.
bool fused_decode_ok(int M, int D);

// Kernel launchers (each returns the launch's hipError_t).
hipError_t launch_pack(const DevRot& R, int N, const uint16_t* W, uint8_t* qweight, uint16_t* scales,
                       uint16_t* zeros, hipStream_t st);
hipError_t launch_rotate(const DevRot& R, int M, const uint16_t* x, uint16_t* xout, hipStream_t st);
// rot == nullptr: plain linear on x. Otherwise x is transformed inside the kernel.
hipError_t launch_gemv(const DevRot* rot, int M, int D, int N, const uint16_t* x, const uint8_t* qweight,
                       const uint16_t* scales, const uint16_t* zeros, void* y, int ydtype, hipStream_t st);
hipError_t launch_gemm(int M, int D, int N, const uint16_t* x, const uint8_t* qweight, const uint16_t* scales,
                       const uint16_t* zeros, void* y, int ydtype, hipStream_t st);

}  // namespace paro
