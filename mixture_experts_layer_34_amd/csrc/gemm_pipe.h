// Pieces shared by the pipelined grouped GEMMs (bf16 and MXFP8): LDS
// swizzles, the wait-and-barrier primitives of the direct-to-LDS pipeline,
// scalar-cache loads of the device-side schedule tables, and the tile raster.
#pragma once
#include "mok_device.h"
#include "mok_internal.h"

namespace mok {

// K-contiguous stage layout: physical 16-byte chunk of logical chunk c in
// row r, for rows of BK = 32 (64 bytes, 4 chunks) or 64 (128 bytes, 8
// chunks).  Sixteen consecutive rows read at one logical chunk hit 16
// distinct 16-byte bank groups (64 banks), and any 8 consecutive rows hit 8
// distinct ones (32 banks).
template <int BK>
__device__ __forceinline__ int swz_k(int r, int c) {
  if constexpr (BK == 32) return c ^ (((r >> 1) ^ (r >> 2)) & 3);
  else return c ^ ((r ^ (r >> 3)) & 7);
}
// M/N-contiguous stage layout: physical 64-byte chunk of logical chunk c in
// the row of k = r.  A transposing read touches rows k..k+3 at one chunk:
// they land in four distinct 64-byte bank groups.
__device__ __forceinline__ int swz_mn(int r, int c) { return c ^ (r & 3); }

// Wait until at most N of this wave's vector memory operations are
// outstanding and its LDS reads have returned, then meet the workgroup.  The
// LDS wait is also issued through the builtin so that the compiler's own
// counter model knows the reads have returned (it does not look inside asm).
constexpr int kWaitLgkm0 = 0xC07F;  // s_waitcnt lgkmcnt(0), vmcnt and expcnt not waited on
template <int N>
__device__ __forceinline__ void vm_wait_barrier() {
  __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Two consecutive int32 at a wave-uniform address through the scalar cache
// (p[1] is read only when valid1): no vector-memory counter is touched, so
// the copies in flight are not waited for.
__device__ __forceinline__ void sload_pair(const int32_t* p, bool valid1, int32_t& v0, int32_t& v1) {
  const int32_t* p1 = valid1 ? p + 1 : p;
  asm volatile("s_load_dword %0, %2, 0x0\n\ts_load_dword %1, %3, 0x0\n\ts_waitcnt lgkmcnt(0)"
               : "=s"(v0), "=s"(v1)
               : "s"(p), "s"(p1)
               : "memory");
}

__device__ __forceinline__ i32x4_t sload4(const int32_t* p) {  // p 16-byte aligned
  i32x4_t v;
  asm volatile("s_load_dwordx4 %0, %1, 0x0\n\ts_waitcnt lgkmcnt(0)" : "=s"(v) : "s"(p) : "memory");
  return v;
}
__device__ __forceinline__ int32_t sload(const int32_t* p) {
  int32_t v;
  asm volatile("s_load_dword %0, %1, 0x0\n\ts_waitcnt lgkmcnt(0)" : "=s"(v) : "s"(p) : "memory");
  return v;
}

// Block until this wave has at most `later` stages of D copies outstanding
// (later <= MAXL), then meet the workgroup.
template <int D, int MAXL>
__device__ __forceinline__ void wait_stages(int later) {
  if (MAXL >= 4 && later >= 4) vm_wait_barrier<(MAXL >= 4 ? 4 : 0) * D>();
  else if (MAXL >= 3 && later >= 3) vm_wait_barrier<(MAXL >= 3 ? 3 : 0) * D>();
  else if (MAXL >= 2 && later >= 2) vm_wait_barrier<(MAXL >= 2 ? 2 : 0) * D>();
  else if (later >= 1) vm_wait_barrier<D>();
  else vm_wait_barrier<0>();
}

struct TileCoord {
  int e_loc, row0, row_end, m0, n0, z;
};

// Grouped raster inside one expert: groups of GM m-tiles, n-tiles outer and
// m-tiles inner within a group, so that a run of consecutive tiles forms a
// GM x (run / GM) block that reuses both operands.  The weight-gradient
// GEMMs measure best with GM = 2, the row GEMMs with 4.
template <int GM = 4>
__device__ __forceinline__ void tile_mn(int local, int mt, int ntn, int& m, int& n) {
  const int g = local / (GM * ntn);
  const int gm0 = g * GM;
  const int gsz = mt - gm0 < GM ? mt - gm0 : GM;
  const int rem = local - g * GM * ntn;
  n = rem / gsz;
  m = gm0 + rem % gsz;
}

// The tile coordinates are wave-uniform; say so, so that addresses and
// buffer resources live in scalar registers.
__device__ __forceinline__ TileCoord uniform(TileCoord c) {
  c.e_loc = __builtin_amdgcn_readfirstlane(c.e_loc);
  c.row0 = __builtin_amdgcn_readfirstlane(c.row0);
  c.row_end = __builtin_amdgcn_readfirstlane(c.row_end);
  c.m0 = __builtin_amdgcn_readfirstlane(c.m0);
  c.n0 = __builtin_amdgcn_readfirstlane(c.n0);
  c.z = __builtin_amdgcn_readfirstlane(c.z);
  return c;
}

}  // namespace mok
