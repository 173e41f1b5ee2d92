// Internal definitions shared by the HIP kernels of libbsa.so (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bsa {

constexpr int kHeadDim = 128;   // d
constexpr int kBlockTokens = 128;  // ct*ch*cw
constexpr int kThreads = 256;   // four wave64 per workgroup

typedef uint16_t bf16_bits;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Geometry of one problem as the kernels see it.
struct Geom {
  int bh;           // batch * heads
  int S;            // tokens per (batch, head)
  int T, H, W;      // latent grid
  int ct, ch, cw;   // chunk shape
  int nH, nW;       // blocks along h and w
  int nb;           // query blocks per (batch, head)
  int nq;           // tokens per query block (64 or 128)
  int cond_blocks;  // leading condition query blocks (0 = no block-causal mask)
  float scale;      // softmax scale
  // Key blocks: the grid cut with the key chunk (the query chunk unless the
  // problem gives a separate one).
  int ctk, chk, cwk;
  int nHk, nWk;
  int nbk;           // key blocks per (batch, head)
  int nk;            // tokens per key block
  int cond_kblocks;  // leading condition key blocks
  // Nonzero when a chunk does not divide the grid: block counts are then
  // ceilings and the last block along a cut axis holds only the tokens of
  // its box that lie inside the grid.
  int partial;
};

// Latent-order token of slot j (0..127) of block i: blocks run in
// [nT, nH, nW] order and the slots of a block in [t, h, w] order.
__device__ __forceinline__ int block_token(const Geom& g, int i, int j) {
  const int bw = i % g.nW;
  const int rest = i / g.nW;
  const int bh = rest % g.nH;
  const int bt = rest / g.nH;
  const int iw = j % g.cw;
  const int r2 = j / g.cw;
  const int ih = r2 % g.ch;
  const int it = r2 / g.ch;
  return ((bt * g.ct + it) * g.H + bh * g.ch + ih) * g.W + bw * g.cw + iw;
}

// Latent-order token of slot j (0 .. nk-1) of key block i.
__device__ __forceinline__ int key_block_token(const Geom& g, int i, int j) {
  const int bw = i % g.nWk;
  const int rest = i / g.nWk;
  const int bh = rest % g.nHk;
  const int bt = rest / g.nHk;
  const int iw = j % g.cwk;
  const int r2 = j / g.cwk;
  const int ih = r2 % g.chk;
  const int it = r2 / g.chk;
  return ((bt * g.ctk + it) * g.H + bh * g.chk + ih) * g.W + bw * g.cwk + iw;
}

// Whether slot j (0 .. nq-1) of query block i lies inside the grid.
__device__ __forceinline__ bool block_slot_valid(const Geom& g, int i, int j) {
  const int bw = i % g.nW;
  const int rest = i / g.nW;
  const int bh = rest % g.nH;
  const int bt = rest / g.nH;
  const int r2 = j / g.cw;
  return bt * g.ct + r2 / g.ch < g.T && bh * g.ch + r2 % g.ch < g.H && bw * g.cw + j % g.cw < g.W;
}

// Whether slot j (0 .. nk-1) of key block i lies inside the grid.
__device__ __forceinline__ bool key_slot_valid(const Geom& g, int i, int j) {
  const int bw = i % g.nWk;
  const int rest = i / g.nWk;
  const int bh = rest % g.nHk;
  const int bt = rest / g.nHk;
  const int r2 = j / g.cwk;
  return bt * g.ctk + r2 / g.chk < g.T && bh * g.chk + r2 % g.chk < g.H &&
         bw * g.cwk + j % g.cwk < g.W;
}

// Whether a problem needs the general kernel instantiations: partial
// blocks, or a block count of 1 along w or within a frame (the fast ones
// divide block ids by magic numbers that need a divisor of 2 or more).
inline bool needs_general(const Geom& g) {
  return g.partial || g.nW == 1 || g.nH * g.nW == 1 || g.nWk == 1 || g.nHk * g.nWk == 1;
}

// Number of leading key blocks query block i may select (block-causal:
// condition query blocks see the condition key blocks only).
__device__ __forceinline__ int allowed_key_blocks(const Geom& g, int i) {
  return (g.cond_blocks > 0 && i < g.cond_blocks) ? g.cond_kblocks : g.nbk;
}

// The same count in query-chunk blocks (the dense kernel walks all allowed
// keys in blocks of the query chunk).
__device__ __forceinline__ int allowed_blocks(const Geom& g, int i) {
  return (g.cond_blocks > 0 && i < g.cond_blocks) ? g.cond_blocks : g.nb;
}

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

}  // namespace bsa
