// Internal declarations shared by the host API and the kernel translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <vector>

#include "paro.h"

namespace paro {

inline size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

// Device descriptor of a prepared transform. Three sections, each 256-byte aligned:
//   rec    PairRec [K][D/2]  {i | (j << 16), cos, sin} (12 bytes: one 3-dword load per pair)
//   inv_s  float   [D]       1/s rounded once to float32 (activation side)
//   s      float   [D]       s (weight side)
struct PairRec {
  uint32_t ij;
  float c, s;
};
static_assert(sizeof(PairRec) == 12, "PairRec must stay 12 bytes");

struct DescLayout {
  size_t rec_off, inv_s_off, s_off, total;
};

inline DescLayout desc_layout(int K, int D) {
  DescLayout L;
  const size_t P = size_t(K) * size_t(D / 2);
  L.rec_off = 0;
  L.inv_s_off = align256(P * sizeof(PairRec));
  L.s_off = L.inv_s_off + align256(size_t(D) * 4);
  L.total = L.s_off + align256(size_t(D) * 4);
  return L;
}

struct DevRot {
  int K, D;
  const PairRec* rec;
  const float* inv_s;
  const float* s;
};

inline DevRot dev_rot(const paro_rotation& r) {
  const DescLayout L = desc_layout(r.K, r.D);
  const char* base = static_cast<const char*>(r.dev);
  return DevRot{r.K, r.D, reinterpret_cast<const PairRec*>(base + L.rec_off),
                reinterpret_cast<const float*>(base + L.inv_s_off), reinterpret_cast<const float*>(base + L.s_off)};
}

// One Givens pair of a stage with its float32 (cos, sin).
struct StagePair {
  int i, j;
  float c, s;
};

// Reorder one stage's pairs (and orient them, negating sin on a swap) so that every
// aligned run of q = 64, 32, 16, 8 consecutive pairs has distinct first channels mod q
// and distinct second channels mod q. Returns false if D % 128 != 0 or sizes mismatch.
bool schedule_stage(int D, std::vector<StagePair>& pairs);

// Largest M the single-kernel decode path (transform fused into the decode kernel) takes.
constexpr int kFusedMaxM = 4;
// Largest M the decode kernel takes; above it the tiled MFMA GEMM runs.
constexpr int kDecodeMaxM = 16;
// LDS budget of one decode workgroup.
constexpr size_t kDecodeMaxLds = 144 * 1024;

// Whether paro_rotated_linear runs its transform inside the decode kernel.
bool fused_decode_ok(int M, int D, int N);
// Whether the (plain) decode kernel takes this shape.
bool decode_ok(int M, int D, int N);

// LDS bytes of a decode workgroup.
size_t decode_lds_bytes(bool fused, int M, int D, int N);

// Kernel launchers (each returns the launch's hipError_t).
hipError_t launch_pack(const DevRot& R, int N, const uint16_t* W, uint8_t* qweight, uint16_t* scales,
                       uint16_t* zeros, hipStream_t st);
// nibble_order: write each 8-channel word as [0,4,1,5,2,6,3,7] (the decode kernel's A order).
hipError_t launch_rotate(const DevRot& R, int M, const uint16_t* x, uint16_t* xout, bool nibble_order,
                         hipStream_t st);
// rot == nullptr: plain linear on x (x_nibble_order tells its word order). Otherwise x is
// transformed inside the kernel (M <= 4).
hipError_t launch_decode(const DevRot* rot, int M, int D, int N, const uint16_t* x, bool x_nibble_order,
                         const uint8_t* qweight, const uint16_t* scales, const uint16_t* zeros, void* y, int ydtype,
                         hipStream_t st);
hipError_t launch_gemm(int M, int D, int N, const uint16_t* x, const uint8_t* qweight, const uint16_t* scales,
                       const uint16_t* zeros, void* y, int ydtype, hipStream_t st);

}  // namespace paro
