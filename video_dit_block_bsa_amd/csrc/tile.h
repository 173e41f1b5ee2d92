// Tile helpers shared by the forward and backward attention kernels of
// libbsa.so: block and slot addressing in latent order, kernel arguments with
// the magic numbers for dividing block ids, buffer resources and a fence-free
// workgroup barrier.
#pragma once

#include "common.h"

namespace bsa {

__device__ __forceinline__ int swap23(int m) {
  return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1);
}

// Kernel arguments. Block ids are split into (bt, bh, bw) with multiply-high
// division by magic numbers (exact for the ranges the host checks), so the
// per-key-block address math stays on the scalar unit.
struct AttnArgs {
  Geom g;
  int stride;
  int q_begin;        // first query block of the launch (the others are skipped)
  int nq8;            // query blocks of the launch per head, rounded up to a multiple of 8
  uint32_t mag_nw;    // floor(2^32 / nW) + 1, or 0 when nW = 1 (see div_magic)
  uint32_t mag_nhw;   // floor(2^32 / (nH*nW)) + 1, or 0 when nH*nW = 1
  uint32_t mag_nwk;   // the same for the key-block grid
  uint32_t mag_nhwk;
  int unit_shift;     // log2 of the 128-key units per key block (key blocks of 256+ tokens)
  int lcwk, lchk;     // log2 of the key chunk's w and h extents
  int lcw, lch;       // the same for the query chunk
  float c_log2;       // scale * log2(e)
  int x0;             // id of the launch's first workgroup among all of the call's (a multiple of 8)
};

// x / d with m = magic(d): the high half of x * m, exact for the ranges the
// host checks. A divisor of 1 (whose magic would not fit in 32 bits) is
// encoded as m = 0 and handled only when kGeneral is set: the host launches
// the general kernels (the kPartial instantiations) for any grid with a
// block count of 1 along w or in a frame.
template <bool kGeneral>
__device__ __forceinline__ int div_magic(int x, uint32_t m) {
  if constexpr (kGeneral) return m ? (int)__umulhi((uint32_t)x, m) : x;
  return (int)__umulhi((uint32_t)x, m);
}

inline uint32_t magic(int d) {
  return d == 1 ? 0u : (uint32_t)(0x100000000ull / (uint64_t)d + 1);
}

// Latent-order token of the first slot of block i.
template <bool kGeneral = false>
__device__ __forceinline__ int block_origin(const AttnArgs& a, int i) {
  const Geom& g = a.g;
  const int bt = div_magic<kGeneral>(i, a.mag_nhw);
  const int rem = i - bt * g.nH * g.nW;
  const int bh = div_magic<kGeneral>(rem, a.mag_nw);
  const int bw = rem - bh * g.nW;
  return ((bt * g.ct) * g.H + bh * g.ch) * g.W + bw * g.cw;
}

// Offset (in tokens) of slot j inside its block.
__device__ __forceinline__ int slot_offset(const Geom& g, int j) {
  const int iw = j % g.cw;
  const int r2 = j / g.cw;
  return ((r2 / g.ch) * g.H + r2 % g.ch) * g.W + iw;
}

// The same two for key blocks (key chunk and key-block grid).
template <bool kGeneral = false>
__device__ __forceinline__ int key_block_origin(const AttnArgs& a, int i) {
  const Geom& g = a.g;
  const int bt = div_magic<kGeneral>(i, a.mag_nhwk);
  const int rem = i - bt * g.nHk * g.nWk;
  const int bh = div_magic<kGeneral>(rem, a.mag_nwk);
  const int bw = rem - bh * g.nWk;
  return ((bt * g.ctk) * g.H + bh * g.chk) * g.W + bw * g.cwk;
}

__device__ __forceinline__ int key_slot_offset(const Geom& g, int j) {
  const int iw = j % g.cwk;
  const int r2 = j / g.cwk;
  return ((r2 / g.chk) * g.H + r2 % g.chk) * g.W + iw;
}

// Extents along t, h and w of key block i's box that lie inside the grid
// (the chunk's own extents except for a partial block at the far edge).
struct Extent {
  int t, h, w;
};
template <bool kGeneral = false>
__device__ __forceinline__ Extent key_block_extent(const AttnArgs& a, int i) {
  const Geom& g = a.g;
  const int bt = div_magic<kGeneral>(i, a.mag_nhwk);
  const int rem = i - bt * g.nHk * g.nWk;
  const int bh = div_magic<kGeneral>(rem, a.mag_nwk);
  const int bw = rem - bh * g.nWk;
  return {min(g.ctk, g.T - bt * g.ctk), min(g.chk, g.H - bh * g.chk), min(g.cwk, g.W - bw * g.cwk)};
}

// The same for query block i (query chunk).
template <bool kGeneral = false>
__device__ __forceinline__ Extent block_extent(const AttnArgs& a, int i) {
  const Geom& g = a.g;
  const int bt = div_magic<kGeneral>(i, a.mag_nhw);
  const int rem = i - bt * g.nH * g.nW;
  const int bh = div_magic<kGeneral>(rem, a.mag_nw);
  const int bw = rem - bh * g.nW;
  return {min(g.ct, g.T - bt * g.ct), min(g.ch, g.H - bh * g.ch), min(g.cw, g.W - bw * g.cw)};
}

__device__ __forceinline__ bool slot_inside(const AttnArgs& a, const Extent& e, int j) {
  return (j & (a.g.cw - 1)) < e.w && ((j >> a.lcw) & (a.g.ch - 1)) < e.h && (j >> (a.lcw + a.lch)) < e.t;
}

// Whether slot j of a key block with extents e lies inside the grid (key
// chunk sides are powers of two).
__device__ __forceinline__ bool key_slot_inside(const AttnArgs& a, const Extent& e, int j) {
  return (j & (a.g.cwk - 1)) < e.w && ((j >> a.lcwk) & (a.g.chk - 1)) < e.h &&
         (j >> (a.lcwk + a.lchk)) < e.t;
}

typedef __attribute__((address_space(3))) void lds_void;
typedef short short4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) short4_t lds_short4;

// Word 3 of a raw buffer resource on gfx9-class GPUs: 32-bit data format.
constexpr int kBufferWord3 = 0x00020000;

// Joins the workgroup without a memory fence: a fence would also wait for
// the tile loads still in flight into other slots. Callers wait for their
// own loads with s_waitcnt first; the empty asm statements keep the compiler
// from moving LDS accesses across the barrier.
__device__ __forceinline__ void workgroup_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Kernel arguments for a problem with index rows of `stride` entries.
inline AttnArgs make_attn_args(const Geom& g, int stride, int q_begin = 0) {
  AttnArgs a;
  a.g = g;
  a.stride = stride;
  a.q_begin = q_begin;
  a.nq8 = (g.nb - q_begin + 7) / 8 * 8;
  a.x0 = 0;
  a.mag_nw = magic(g.nW);
  a.mag_nhw = magic(g.nH * g.nW);
  a.mag_nwk = magic(g.nWk);
  a.mag_nhwk = magic(g.nHk * g.nWk);
  a.unit_shift = 0;
  for (int m = g.nk / 128; m > 1; m >>= 1) ++a.unit_shift;
  a.lcwk = 0;
  for (int m = g.cwk; m > 1; m >>= 1) ++a.lcwk;
  a.lchk = 0;
  for (int m = g.chk; m > 1; m >>= 1) ++a.lchk;
  a.lcw = 0;
  for (int m = g.cw; m > 1; m >>= 1) ++a.lcw;
  a.lch = 0;
  for (int m = g.ch; m > 1; m >>= 1) ++a.lch;
  a.c_log2 = g.scale * 1.4426950408889634f;
  return a;
}

}  // namespace bsa
