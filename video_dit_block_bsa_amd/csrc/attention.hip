// Block-restricted flash attention ("Sparse attention computation" of the
// LongCat-Video deep dive, section "Block Sparse Attention": softmax over the
// keys of the selected blocks only) and its dense baseline, for gfx950.
//
// Work decomposition
//   One workgroup (4 x wave64) per (batch*head, query block of 128 tokens),
//   two workgroups per CU; wave w owns queries 32w .. 32w+31 of the block.
//   The workgroup walks the query block's key-block list in units of 128
//   keys; K and V tiles are staged in LDS as [token][channel] rows, in half
//   tiles of 64 keys. (Query blocks of 64 tokens and key blocks of other
//   sizes are described at the kernel.)
//
// Math per key block and wave (bf16 MFMA 32x32x16, fp32 accumulate)
//   S^T = K Q^T     4 key sub-tiles x 8 channel steps = 32 MFMA. Q^T stays in
//                   registers for the whole loop (B operand); K rows come from
//                   LDS (A operand).
//   online softmax  each lane owns one query (C column) and holds 64 of its
//                   128 scores; the row max needs one exchange with lane^32.
//                   exp2 with scale*log2(e) folded in.
//   O^T += V^T P^T  4 channel sub-tiles x 8 key steps = 32 MFMA; P^T is taken
//                   straight from the S^T accumulators (converted to bf16).
//                   The V^T operand is read from the [key][channel] V tile
//                   with gfx950's transposing LDS read (ds_read_b64_tr_b16),
//                   two 4-key reads per fragment, so V needs no repacked copy.
//   For the P^T registers to line up with natural key order, the K rows are
//   read with bits 2 and 3 of the row index swapped: the accumulator of row m
//   then holds key swap23(m), and the 8 values a lane contributes to one
//   16-key MFMA step are consecutive keys.
//
// Tiles reach LDS with direct-to-LDS buffer loads (buffer_load_dwordx4 ...
// lds), no VGPR staging, through a ring of five half-tile slots described at
// the kernel. LDS rows are unpadded; XOR swizzles on 16-byte chunks keep the
// operand reads free of bank conflicts. The epilogue divides by the softmax
// sum and writes O in latent order.
//
// Workgroup order is XCD-aware: MI355X dispatches consecutive workgroups
// round-robin over its 8 XCDs, so the id is remapped to give each XCD a
// contiguous run of query blocks of the same head, while all XCDs work on the
// same head at a time (its K/V, 110 MB at 215K tokens, stay resident in the
// 256 MB Infinity Cache).
#include <type_traits>

#include "launch.h"
#include "tile.h"

namespace bsa {

// Softmax rescaling is lazy: the running max m (log2 units) is only moved
// when a tile's max exceeds it by more than this, so most tiles skip the
// O *= alpha pass. Probabilities stay <= 2^8, well inside fp32 and bf16.
constexpr float kRescaleSlack = 8.0f;

// Half tiles live in LDS as 64 rows of 256 bytes (16 chunks of 16 bytes)
// with no padding. Chunk c of row r is stored at chunk c ^ swz(r), where
// swz(r) is swap23 of the row's low four bits. The MFMA operand reads of a
// wave touch rows swap23(n) + const with the same logical chunk, which this
// spreads over all 16 chunk positions: conflict-free. Each direct-to-LDS load
// writes 64 lanes x 16 bytes = 4 whole rows, so lane L of a load writes
// physical chunk L % 16 of row base + L / 16 and fetches the logical chunk
// that lands there.
__device__ __forceinline__ int swz(int row) { return swap23(row & 15); }

// V tiles are read four rows at a time (transposing reads); spreading rows
// r..r+3 over the four 64-byte slots of a 256-byte row keeps them apart.
__device__ __forceinline__ int swzv(int row) { return 4 * (row & 3); }

constexpr int kHalfRows = kBlockTokens / 2;            // key rows per half tile
constexpr int kSlots = 5;                               // half-tile ring per workgroup

// Tiles stream through a ring of five 16 KB half-tile slots in the order
// K_0 lo, K_0 hi, V_0 lo, V_0 hi, K_1 lo, ... (lo = key rows 0..63). Phase p
// (S^T and softmax of key block p/2 for even p, P V for odd p) reads half
// tiles 2p and 2p+1 and, once every wave is past the barrier that opens it,
// refills the two slots phase p-1 read with half tiles 2p+3 and 2p+4. Each
// load is thus issued two phases before it is read, with three half tiles
// (48 KB) in flight per workgroup. Slot of half tile n is n mod 5; every
// slot is its own LDS object, and the phase loop is unrolled over the ten
// phases after which the assignment repeats, so that each read names its
// slot at compile time and never waits on loads into the other slots.
//
// With kLse the kernel also writes each query's softmax log-normaliser
// (natural log, -inf for a query block with no key blocks), which the
// backward pass uses to recompute the probabilities.
//
// Key blocks may be cut with their own chunk ("Implementation details and
// design trade-offs": key blocks of 64 to 1024 tokens). The loop always
// walks units of 128 keys, staged as two half tiles:
//   kKeyMode 0: a key block is one unit (128 tokens);
//   kKeyMode 1: a key block of 128 * 2^unit_shift tokens is that many units,
//               unit u holding its slots 128u .. 128u+127;
//   kKeyMode 2: key blocks of 64 tokens, two per unit (lower and upper half);
//               when the count is odd the last unit's upper half repeats the
//               lower one and its scores are set to -inf.
// A unit's slot offsets are those of its first slot plus those of its slot
// index (power-of-two chunk sides make the offset linear in the index bits).
//
// kPartial (a chunk that does not divide the grid: "3D block partitioning"
// counts blocks with ceilings, so the last block along a cut axis holds only
// the tokens of its box inside the grid): a query slot outside the grid
// computes on the block's slot 0 and is never written; the scores of key
// slots outside the grid are set to -inf; a tile row outside the grid fetches
// row 0 of its block, so every load stays inside the tensor. Grids the chunks
// divide use the instantiation without any of this.
//
// kSplit serves query blocks of 64 tokens: wave w takes queries 32(w%2) ..
// +31 and key half w/2 (keys 0..63 or 64..127) of every unit, keeps its own
// running max and sum over its keys, and the two key halves of a query meet
// in LDS after the loop (O = (O_a 2^(m_a-m) + O_b 2^(m_b-m)) / (l_a 2^(m_a-m)
// + l_b 2^(m_b-m)), m = max(m_a, m_b)). Every wave then issues half the MFMAs
// of a unit, and the key half is a template constant inside the loop (two
// copies), so each read still names its slot.
//
// kUnion also serves query blocks of 64 tokens (128-token key blocks, grids
// the chunks divide): one workgroup takes the two blocks at t-rows r0 + 2m
// and r0 + 2m + 1 of the same (h, w) column (r0: the launch's first row),
// whose 128 slots form one box of twice the chunk's depth (slot j >= 64 is
// slot j - 64 of the second block, by the linearity of the slot offsets);
// after an odd number of rows the last one has no partner, and waves 2, 3
// then read the first block's slot 0, own no unit and write nothing. It
// walks the union of the two key lists, merged by a two-cursor walk, and
// stages each key block once; waves 0, 1 (first block) and 2, 3 (second
// block) skip the products of a unit their block did not select. Neighbouring
// blocks select mostly the same keys, so the tiles gathered per query drop
// by a quarter on smooth inputs while the MFMA work stays that of the blocks'
// own lists. The walk visits every list entry once whatever the lists'
// order; ascending lists make it share the most. A wave's arithmetic depends
// only on its own block's list, walked in that list's order, so a block gets
// the same bits whichever block it is paired with.
template <bool kDense, bool kLse, int kKeyMode, bool kSplit, bool kPartial, bool kUnion = false>
__global__ __launch_bounds__(kThreads, 2) void attn_kernel(
    AttnArgs a, const bf16_bits* __restrict__ qp, const bf16_bits* __restrict__ kp,
    const bf16_bits* __restrict__ vp, const int32_t* __restrict__ idx,
    const int32_t* __restrict__ cntp, bf16_bits* __restrict__ op, float* __restrict__ lsep) {
  __shared__ __attribute__((aligned(1024))) bf16_bits slot0[kHalfRows * kHeadDim];
  __shared__ __attribute__((aligned(1024))) bf16_bits slot1[kHalfRows * kHeadDim];
  __shared__ __attribute__((aligned(1024))) bf16_bits slot2[kHalfRows * kHeadDim];
  __shared__ __attribute__((aligned(1024))) bf16_bits slot3[kHalfRows * kHeadDim];
  __shared__ __attribute__((aligned(1024))) bf16_bits slot4[kHalfRows * kHeadDim];
  auto slot_ptr = [&](auto sc) -> bf16_bits* {
    constexpr int sl = decltype(sc)::value;
    if constexpr (sl == 0) return slot0;
    else if constexpr (sl == 1) return slot1;
    else if constexpr (sl == 2) return slot2;
    else if constexpr (sl == 3) return slot3;
    else return slot4;
  };
  const Geom& g = a.g;

  // XCD-aware remap: hardware id x runs on XCD x % 8; give XCD c the query
  // blocks [c*chunk, (c+1)*chunk) of the current head. A call split into
  // workgroup ranges numbers its workgroups across the launches (x0 is a
  // multiple of 8, so x % 8 is still the XCD).
  const int x = blockIdx.x + a.x0;
  const int pair = x / a.nq8;
  const int r = x - pair * a.nq8;
  const int chunk = a.nq8 >> 3;
  const int nhw = g.nH * g.nW;  // query blocks per t-row
  // kUnion: x indexes pairs; pair p = m nhw + c holds block q_begin + 2m nhw
  // + c and, if it exists, the block one t-row after it.
  const int qi = (kUnion ? 0 : a.q_begin) + (r & 7) * chunk + (r >> 3);
  const int qb = kUnion ? a.q_begin + qi + div_magic<false>(qi, a.mag_nhw) * nhw : qi;
  if (qb >= g.nb) return;
  const bool has_b = kUnion && qb + nhw < g.nb;  // the pair's second block exists

  const int t = threadIdx.x;
  const int lane = t & 63;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6);
  const int n = lane & 31;
  const int gs = lane >> 5;
  const int qh = kSplit ? (w & 1) : w;  // 32-query slice of the block
  const int kh = kSplit ? (w >> 1) : 0; // key half (split mode)
  const size_t hoff = (size_t)pair * g.S * kHeadDim;
  // K and V of this (batch, head) as buffer resources: a tile load takes one
  // 32-bit lane offset, and anything past the head reads as zero.
  const uint32_t head_bytes = (uint32_t)g.S * (kHeadDim * 2);
  const __amdgpu_buffer_rsrc_t krs =
      __builtin_amdgcn_make_buffer_rsrc((void*)(kp + hoff), (short)0, head_bytes, kBufferWord3);
  const __amdgpu_buffer_rsrc_t vrs =
      __builtin_amdgcn_make_buffer_rsrc((void*)(vp + hoff), (short)0, head_bytes, kBufferWord3);

  // A query slot of a partial block that lies outside the grid, or one of
  // the missing second block of a lone last row (kUnion), reads slot 0 of the
  // (first) block instead, and its row is never written.
  const bool q_inside =
      kUnion ? (w < 2 || has_b) : !kPartial || block_slot_valid(g, qb, 32 * qh + n);
  const int qtok = block_origin<kPartial>(a, qb) + (q_inside ? slot_offset(g, 32 * qh + n) : 0);
  bf16x8 qf[8];
#pragma unroll
  for (int s = 0; s < 8; ++s)
    qf[s] = __builtin_bit_cast(
        bf16x8, *reinterpret_cast<const u32x4*>(qp + hoff + (size_t)qtok * kHeadDim + 16 * s + 8 * gs));
  // Q must be in registers before the first tile load is issued: a later
  // wait for Q would also wait for every tile load in flight.
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)

  // This wave stages rows 16w .. 16w+15 of each half tile: 4 loads of 4
  // rows, load i covering rows 16w + 4i .. +3 (lane L: row 16w + 4i + L/16,
  // physical chunk L%16). The chunk sides are powers of two, so a slot's
  // token offset is linear in the bits of its index: the offset of row
  // 16w + 4i + r is that of 16w + r plus the (uniform) offset of slot 4i, and
  // the upper half tile is the lower one shifted by the offset of slot 64.
  // The swizzles depend on the row's low four bits 4i + r: for K the logical
  // chunk is (L%16) ^ r ^ 4*sb(i), with sb swapping the two bits of i; for V
  // it is (L%16) ^ 4r. So one lane offset k0 serves every load: load i of K
  // uses k0 ^ 64*sb(i), every load of V uses k0 ^ 80r, and the rest is scalar.
  const int r_lane = lane >> 4;
  const uint32_t k0 = (uint32_t)key_slot_offset(g, 16 * w + r_lane) * (kHeadDim * 2) +
                      (uint32_t)(((lane & 15) ^ r_lane) << 4);
  const uint32_t vx = 80u * (uint32_t)r_lane;  // ((L%16) ^ 4r) ^ ((L%16) ^ r), in bytes
  const uint32_t half_off = (uint32_t)key_slot_offset(g, kHalfRows) * (kHeadDim * 2);

  int count, count_b = 0;
  const int32_t* list = nullptr;
  const int32_t* list_b = nullptr;  // kUnion: the second block's list
  if (kDense) {
    count = allowed_blocks(g, qb);
  } else {
    list = idx + ((size_t)pair * g.nb + qb) * a.stride;
    count = min(max(cntp[(size_t)pair * g.nb + qb], 0), a.stride);
    if (kUnion && has_b) {
      list_b = list + (size_t)nhw * a.stride;
      count_b = min(max(cntp[(size_t)pair * g.nb + qb + nhw], 0), a.stride);
    }
  }
  // Next usable position of list l (c entries) at or after `from` (ids
  // outside [0, Nk) are skipped).
  auto next_valid_in = [&](const int32_t* l, int c, int from) {
    if (kDense) return from;
    while (from < c) {
      const int kb = l[from];
      if (kb >= 0 && kb < g.nbk) break;
      ++from;
    }
    return from;
  };
  auto next_valid = [&](int from) { return next_valid_in(list, count, from); };
  auto kb_at = [&](int pos) { return kDense ? pos : list[pos]; };
  // Unit cursor: (position, unit within the key block) for kKeyMode 0 and 1,
  // (position of the lower block, position of the upper block) for kKeyMode 2.
  // The unit exists while .a < count. kUnion: (position in the first list,
  // position in the second, the unit's key block = the smaller of the two
  // entries, bit 0 / bit 1 set when it is the first / second list's entry);
  // the unit exists while either position is inside its list.
  struct Cursor {
    int a, b, kb, m;
  };
  auto union_unit = [&](int pa, int pb) -> Cursor {
    const int ka = pa < count ? list[pa] : 0x7fffffff;
    const int kb = pb < count_b ? list_b[pb] : 0x7fffffff;
    const int k = min(ka, kb);
    return {pa, pb, k, (ka == k ? 1 : 0) | (kb == k ? 2 : 0)};
  };
  auto live = [&](const Cursor& c) { return kUnion ? (c.a < count || c.b < count_b) : c.a < count; };
  auto first_unit = [&]() -> Cursor {
    if constexpr (kUnion) return union_unit(next_valid(0), next_valid_in(list_b, count_b, 0));
    const int p = next_valid(0);
    return {p, kKeyMode == 2 ? next_valid(p + 1) : 0, 0, 0};
  };
  auto next_unit = [&](Cursor c) -> Cursor {
    if constexpr (kUnion) {
      return union_unit((c.m & 1) ? next_valid(c.a + 1) : c.a,
                        (c.m & 2) ? next_valid_in(list_b, count_b, c.b + 1) : c.b);
    } else if constexpr (kKeyMode == 1) {
      if (c.b + 1 < (1 << a.unit_shift)) return {c.a, c.b + 1, 0, 0};
      return {next_valid(c.a + 1), 0, 0, 0};
    } else if constexpr (kKeyMode == 2) {
      const int p = next_valid(c.b + 1);
      return {p, next_valid(p + 1), 0, 0};
    } else {
      return {next_valid(c.a + 1), 0, 0, 0};
    }
  };
  // Byte offset of the first slot of half h (0: keys 0..63, 1: keys 64..127)
  // of a unit.
  auto unit_base = [&](Cursor c, int h) -> uint32_t {
    if constexpr (kKeyMode == 2) {
      const int p = (h != 0 && c.b < count) ? c.b : c.a;
      return (uint32_t)key_block_origin<kPartial>(a, kb_at(p)) * (kHeadDim * 2);
    } else if constexpr (kKeyMode == 1) {
      return (uint32_t)(key_block_origin<kPartial>(a, kb_at(c.a)) +
                        key_slot_offset(g, c.b * kBlockTokens)) * (kHeadDim * 2) +
             h * half_off;
    } else {
      return (uint32_t)key_block_origin<kPartial>(a, kUnion ? c.kb : kb_at(c.a)) * (kHeadDim * 2) +
             h * half_off;
    }
  };
  // Half tile e (0: K lo, 1: K hi, 2: V lo, 3: V hi) of a unit into a slot.
  // A row of a partial key block that lies outside the grid fetches row 0 of
  // the block instead (inside the grid, so every address stays inside the
  // tensor; its scores are masked, so the finite values it brings are
  // multiplied by probability 0).
  auto load_half = [&](Cursor c, int e, bf16_bits* dst_slot) {
    const uint32_t base = unit_base(c, e & 1);
    char* dst = reinterpret_cast<char*>(dst_slot) + 16 * w * 256;
    bool cut = false;
    Extent ex = {0, 0, 0};
    int jbase = 0;  // slot of row 0 of this half tile in its key block
    if constexpr (kPartial) {
      int kb;
      if constexpr (kKeyMode == 2) {
        kb = kb_at(((e & 1) && c.b < count) ? c.b : c.a);
      } else {
        kb = kb_at(c.a);
        jbase = (kKeyMode == 1 ? c.b * kBlockTokens : 0) + kHalfRows * (e & 1);
      }
      ex = key_block_extent<kPartial>(a, kb);
      cut = ex.t != g.ctk || ex.h != g.chk || ex.w != g.cwk;
    }
    // Bit x: row 16w + x of the half tile lies inside the grid (scalar work,
    // only for a cut block).
    uint32_t inside = 0xffffu;
    if (cut) {
      inside = 0u;
      for (int x = 0; x < 16; ++x)
        if (key_slot_inside(a, ex, jbase + 16 * w + x)) inside |= 1u << x;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      constexpr uint32_t sb64[4] = {0, 128, 64, 192};  // 64 * (i with its two bits swapped)
      const uint32_t row_s = (uint32_t)key_slot_offset(g, 4 * i) * (kHeadDim * 2);
      uint32_t voff = e < 2 ? (k0 ^ sb64[i]) : (k0 ^ vx);
      uint32_t soff = base + row_s;
      if (cut) {
        const bool in = ((inside >> (4 * i + (lane >> 4))) & 1u) != 0u;
        voff = in ? voff + row_s : (uint32_t)(lane & 15) * 16u;
        soff = base;
      }
      __builtin_amdgcn_raw_ptr_buffer_load_lds(e < 2 ? krs : vrs, (lds_void*)(dst + i * 1024), 16,
                                               voff, soff, 0, 0);
    }
  };

  f32x16 oacc[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) oacc[u] = f32x16{};
  float m2 = -INFINITY;  // running max of score * c_log2
  float l_part = 0.f;    // this lane's share of the softmax denominator
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
  // K operand reads: lane n reads row swap23(n) of a 32-row sub-tile at
  // logical chunk 2s + gs, stored at chunk (2s + gs) ^ (n & 15). In bytes that
  // is ka0 ^ 32s (the XOR only touches bits 5..7, which ka0 keeps for it).
  const int cx = n & 15;
  const int ka0 = swap23(n) * 256 + ((cx >> 1) << 5) + ((gs ^ (cx & 1)) << 4);
  // Transposing V reads: in each group of 16 lanes, lane j points at key
  // 16s + 8gs + (j%16)/4 (+4 for the second read) and channels
  // 32u + 16*((lane/16)%2) + 4*(j%4) .. +3; lane i then receives channel
  // 32u + (lane%32) of those four keys. Chunk c of V row r sits at c ^ swzv(r),
  // which in bytes is va0 ^ 64u for channel sub-tile u.
  int va0;
  {
    const int jj = lane & 15;
    const int q = jj >> 2;
    const int c0 = 2 * ((lane >> 4) & 1) + ((jj & 3) >> 1);
    va0 = (8 * gs + q) * 256 + 64 * q + 16 * c0 + 8 * (jj & 1);
  }

  // Units: cur (the unit of the current phase) and nxt (the one after it,
  // not live past the last). KH is the key half in split mode.
  auto run = [&](auto khc) {
  constexpr int KH = decltype(khc)::value;
  constexpr int kT = kSplit ? 2 : 4;  // 32-key sub-tiles of S per wave
  Cursor cur = first_unit();
  if (live(cur)) {
    Cursor nxt = next_unit(cur);
    // Half tiles 0, 1, 2 (K_0 lo, K_0 hi, V_0 lo) into slots 0, 1, 2.
    load_half(cur, 0, slot0);
    load_half(cur, 1, slot1);
    load_half(cur, 2, slot2);
    bf16x8 pf[8];

    // Phase with index pm = p mod 10 (its slots are fixed at compile time).
    // Returns false when the last block's P V phase is done.
    auto phase = [&](auto pmc) -> bool {
      constexpr int pm = decltype(pmc)::value;
      constexpr bool is_s = (pm % 2) == 0;
      constexpr int sa = (2 * pm) % kSlots, sb = (2 * pm + 1) % kSlots;
      constexpr int sc = (2 * pm + 3) % kSlots, sd = (2 * pm + 4) % kSlots;
      // Every phase issues exactly two half tiles (past the last block they
      // repeat the current one and are never read), so at the start of phase
      // p the loads in flight are always half tiles 2p, 2p+1, 2p+2: a fixed
      // vmcnt lets the last of them stay in flight.
      __builtin_amdgcn_s_waitcnt(0x0074);  // vmcnt(4) lgkmcnt(0)
      workgroup_barrier();
      // Refill the slots of the previous phase with half tiles 2p+3, 2p+4:
      // V_j hi and K_{j+1} lo in an S phase, K_{j+1} hi and V_{j+1} lo in a
      // P V phase.
      const Cursor un = live(nxt) ? nxt : cur;
      if constexpr (is_s) {
        load_half(cur, 3, slot_ptr(std::integral_constant<int, sc>{}));
        load_half(un, 0, slot_ptr(std::integral_constant<int, sd>{}));
      } else {
        load_half(un, 1, slot_ptr(std::integral_constant<int, sc>{}));
        load_half(un, 2, slot_ptr(std::integral_constant<int, sd>{}));
      }
      const char* lo = reinterpret_cast<const char*>(slot_ptr(std::integral_constant<int, sa>{}));
      const char* hi = reinterpret_cast<const char*>(slot_ptr(std::integral_constant<int, sb>{}));
      // kUnion: whether this wave's block selected the unit's key block.
      const bool own = !kUnion || ((cur.m >> (w >> 1)) & 1) != 0;
      if constexpr (is_s) {
        if (!own) return true;
        // S^T = K Q^T for this wave's 32 queries and all 128 keys, channel
        // steps outermost (four independent accumulators between dependent
        // MFMAs).
        f32x16 sacc[kT];
#pragma unroll
        for (int tt = 0; tt < kT; ++tt) sacc[tt] = f32x16{};
#pragma unroll
        for (int s = 0; s < 8; ++s) {
#pragma unroll
          for (int tt = 0; tt < kT; ++tt) {
            const char* kt = kSplit ? (KH ? hi : lo) : (tt < 2 ? lo : hi);
            const bf16x8 af =
                *reinterpret_cast<const bf16x8*>(kt + 32 * (tt & 1) * 256 + (ka0 ^ (32 * s)));
            sacc[tt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, qf[s], sacc[tt], 0, 0, 0);
          }
        }
        if constexpr (kKeyMode == 2) {
          // A lone last 64-token key block: its unit has no upper half.
          if ((!kSplit || KH == 1) && cur.b >= count) {
#pragma unroll
            for (int tt = kT - 2; tt < kT; ++tt)
#pragma unroll
              for (int i = 0; i < 16; ++i) sacc[tt][i] = -INFINITY;
          }
        }
        if constexpr (kPartial) {
          // Keys of a partial block that lie outside the grid get -inf.
          // Half h of the unit (keys 64h .. 64h+63) holds slots base .. +63
          // of key block kb; accumulator value i of this wave's sub-tile tl
          // of that half is key 32 tl + 16 (i/8) + 8 gs + i%8 of the half.
          auto mask_half = [&](int h, int kb, int base) {
            const Extent e = key_block_extent<kPartial>(a, kb);
            if (e.t == g.ctk && e.h == g.chk && e.w == g.cwk) return;
            // The lane's offset passes through an empty asm so that nothing
            // derived from it is hoisted out of the loop (64 live registers).
            int lb = base + 8 * gs;
            asm volatile("" : "+v"(lb));
#pragma unroll
            for (int tl = 0; tl < 2; ++tl) {
              const int tt = kSplit ? tl : 2 * h + tl;
#pragma unroll
              for (int i = 0; i < 16; ++i) {
                const int j = lb + 32 * tl + 16 * (i >> 3) + (i & 7);
                if (!key_slot_inside(a, e, j)) sacc[tt][i] = -INFINITY;
              }
            }
          };
          if constexpr (kKeyMode == 2) {
            if (!kSplit || KH == 0) mask_half(0, kb_at(cur.a), 0);
            if ((!kSplit || KH == 1) && cur.b < count) mask_half(1, kb_at(cur.b), 0);
          } else {
            const int base = kKeyMode == 1 ? cur.b * kBlockTokens : 0;
            if (!kSplit || KH == 0) mask_half(0, kb_at(cur.a), base);
            if (!kSplit || KH == 1) mask_half(1, kb_at(cur.a), base + kHalfRows);
          }
        }
        // Online softmax for this lane's query (both lane halves agree on m2).
        float mx = -INFINITY;
#pragma unroll
        for (int tt = 0; tt < kT; ++tt)
#pragma unroll
          for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sacc[tt][i]);
        mx = fmaxf(mx, __shfl_xor(mx, 32)) * a.c_log2;
        const bool grow = mx > m2 + kRescaleSlack;
        if (__ballot(grow) != 0ull) {
          const float m_new = grow ? mx : m2;
          const float alpha = __builtin_amdgcn_exp2f(m2 - m_new);
          m2 = m_new;
          l_part *= alpha;
#pragma unroll
          for (int u = 0; u < 4; ++u) oacc[u] *= alpha;
        }
        // A wave may have seen only masked keys so far (m2 still -inf: the
        // empty half of a lone 64-token key block in split mode, or a unit
        // outside the grid): its probabilities are then exp2(-inf - 0) = 0.
        const float msub = ((kSplit || kPartial) && m2 == -INFINITY) ? 0.f : m2;
#pragma unroll
        for (int tt = 0; tt < kT; ++tt) {
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            u32x4 packed;
#pragma unroll
            for (int j2 = 0; j2 < 4; ++j2) {
              const f32x2 pr = {
                  __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[tt][8 * h + 2 * j2], a.c_log2, -msub)),
                  __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[tt][8 * h + 2 * j2 + 1], a.c_log2, -msub))};
              const bf16x2 pb = __builtin_convertvector(pr, bf16x2);
              l_part = __builtin_amdgcn_fdot2_f32_bf16(pb, ones, l_part, false);
              packed[j2] = __builtin_bit_cast(uint32_t, pb);
            }
            pf[2 * tt + h] = __builtin_bit_cast(bf16x8, packed);
          }
        }
        return true;
      } else {
        // O^T += V^T P^T; the V^T operand of channel sub-tile u for key step
        // s is two transposing reads of four keys each. The two halves are
        // separate loops so that every read names one slot (through a select
        // of two slots the compiler would wait for all tile loads in flight).
        auto pv_half = [&](const char* vhalf, int s0) {
#pragma unroll
          for (int s = 0; s < 4; ++s) {
#pragma unroll
            for (int u = 0; u < 4; ++u) {
              const char* p0 = vhalf + (va0 ^ (64 * u)) + s * 16 * 256;
              const short4_t vlo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4*)(p0));
              const short4_t vhi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4*)(p0 + 4 * 256));
              const bf16x8 af = __builtin_bit_cast(
                  bf16x8, u32x4{__builtin_bit_cast(u32x2, vlo)[0], __builtin_bit_cast(u32x2, vlo)[1],
                                __builtin_bit_cast(u32x2, vhi)[0], __builtin_bit_cast(u32x2, vhi)[1]});
              oacc[u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, pf[s0 + s], oacc[u], 0, 0, 0);
            }
          }
        };
        if constexpr (kSplit) {
          pv_half(KH ? hi : lo, 0);
        } else if (own) {
          pv_half(lo, 0);
          pv_half(hi, 4);
        }
        if (!live(nxt)) return false;
        cur = nxt;
        nxt = next_unit(cur);
        return true;
      }
    };
    using std::integral_constant;
    while (phase(integral_constant<int, 0>{}) && phase(integral_constant<int, 1>{}) &&
           phase(integral_constant<int, 2>{}) && phase(integral_constant<int, 3>{}) &&
           phase(integral_constant<int, 4>{}) && phase(integral_constant<int, 5>{}) &&
           phase(integral_constant<int, 6>{}) && phase(integral_constant<int, 7>{}) &&
           phase(integral_constant<int, 8>{}) && phase(integral_constant<int, 9>{})) {
    }
    // The trailing loads are never read, but must land before the workgroup
    // gives its LDS to the next one (or to the merge below).
    __builtin_amdgcn_s_waitcnt(0x0070);
  }
  };
  if constexpr (kSplit) {
    if (kh == 0)
      run(std::integral_constant<int, 0>{});
    else
      run(std::integral_constant<int, 1>{});
  } else {
    run(std::integral_constant<int, 0>{});
  }

  float l = l_part + __shfl_xor(l_part, 32);
  if constexpr (kSplit) {
    // The key halves of each query meet: waves 2, 3 leave O, m and l in LDS
    // (the ring is idle now), waves 0, 1 merge them and write the output.
    __syncthreads();
    float* ob = reinterpret_cast<float*>(qh == 0 ? slot0 : slot1);  // 64 values x 64 lanes
    float* mb = reinterpret_cast<float*>(slot2) + qh * 128;
    if (kh == 1) {
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int i = 0; i < 16; ++i) ob[(u * 16 + i) * 64 + lane] = oacc[u][i];
      mb[lane] = m2;
      mb[64 + lane] = l;
    }
    __syncthreads();
    if (kh == 1) return;
    const float m_b = mb[lane], l_b = mb[64 + lane];
    const float m = fmaxf(m2, m_b);
    const float fa = (m2 == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m2 - m);
    const float fb = (m_b == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m_b - m);
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int i = 0; i < 16; ++i) oacc[u][i] = oacc[u][i] * fa + ob[(u * 16 + i) * 64 + lane] * fb;
    l = l * fa + l_b * fb;
    m2 = m;
  }
  const float inv = (l > 0.f) ? 1.0f / l : 0.f;
  if (!q_inside) return;
  if constexpr (kLse) {
    // sum_j exp(scale * q.k_j) = 2^m2 * l, so lse = (m2 + log2 l) * ln 2.
    if (gs == 0)
      lsep[(size_t)pair * g.S + qtok] = (l > 0.f) ? (m2 + log2f(l)) * 0.6931471805599453f : -INFINITY;
  }
  bf16_bits* orow = op + hoff + (size_t)qtok * kHeadDim;
  // Accumulator value i of sub-tile u is channel 32u + 8(i/4) + 4gs + i%4.
#pragma unroll
  for (int u = 0; u < 4; ++u) {
#pragma unroll
    for (int a4 = 0; a4 < 4; ++a4) {
      const f32x2 lo = {oacc[u][4 * a4 + 0] * inv, oacc[u][4 * a4 + 1] * inv};
      const f32x2 hi = {oacc[u][4 * a4 + 2] * inv, oacc[u][4 * a4 + 3] * inv};
      const u32x2 packed = {__builtin_bit_cast(uint32_t, __builtin_convertvector(lo, bf16x2)),
                            __builtin_bit_cast(uint32_t, __builtin_convertvector(hi, bf16x2))};
      *reinterpret_cast<u32x2*>(orow + 32 * u + 8 * a4 + 4 * gs) = packed;
    }
  }
}

namespace {

// 64-token query blocks with 128-token key blocks go in t-adjacent pairs
// (kUnion), counted from the launch's first t-row, on grids the chunks divide.
bool pairs_query_blocks(const Geom& g, int q_begin) {
  return g.nq != kBlockTokens && g.nk == kBlockTokens && !needs_general(g) &&
         q_begin % (g.nH * g.nW) == 0;
}

// A sparse call goes out as launches of at most this many workgroups: 15
// full rounds of the chip (256 compute units holding two workgroups each),
// so every launch but the last ends without a partly filled round, and the
// clock, which climbs over the launches of a step under this load, gets
// several launch boundaries. Measured against launches of 8 heads at 215K
// tokens (53,760 workgroups), each box against itself: 0.5-2 % less time per
// step on three boxes; at 720p (23,040 workgroups, one launch before) 0.8 %.
// Ranges of 21 rounds measured the same, ranges of 5-10 rounds and of 35
// rounds slower.
constexpr unsigned kLaunchWorkgroups = 15 * 512;

hipError_t launch_attention_heads(const Geom& g, const bf16_bits* q, const bf16_bits* k,
                                  const bf16_bits* v, const int32_t* idx, const int32_t* cnt,
                                  int stride, bool dense, bf16_bits* o, float* lse, int q_begin,
                                  hipStream_t stream) {
  if (q_begin >= g.nb) return hipSuccess;
  dim3 grid((unsigned)((size_t)g.bh * ((g.nb - q_begin + 7) / 8 * 8)));
  const bool split = g.nq != kBlockTokens;
  // Grids the chunks divide (with more than one block along w and within a
  // frame) run kernels compiled without the general code, which would
  // otherwise cost them registers and time.
  bool part = needs_general(g);
  if (dense) {
    // Dense attention walks all allowed keys in blocks of the query chunk.
    // Its result does not depend on the block shape, so 64-token chunks run
    // as boxes of twice their depth when those tile the grid and the
    // condition frames (half the key traffic per query).
    Geom gd = g;
    const int rows = g.nb / (g.nH * g.nW);
    if (split && !g.partial && q_begin == 0 && rows % 2 == 0 &&
        (g.cond_blocks / (g.nH * g.nW)) % 2 == 0) {
      gd.ct = 2 * g.ct;
      gd.nq = kBlockTokens;
      gd.nb = g.nb / 2;
      gd.cond_blocks = g.cond_blocks / 2;
      grid = dim3((unsigned)((size_t)g.bh * ((gd.nb + 7) / 8 * 8)));
    }
    const bool split_d = gd.nq != kBlockTokens;
    gd.ctk = gd.ct;
    gd.chk = gd.ch;
    gd.cwk = gd.cw;
    gd.nHk = gd.nH;
    gd.nWk = gd.nW;
    gd.nbk = gd.nb;
    gd.nk = gd.nq;
    gd.cond_kblocks = gd.cond_blocks;
    const AttnArgs a = make_attn_args(gd, 1, q_begin);
    part = needs_general(gd);
#define BSA_LAUNCH_DENSE(MODE, SPLIT, PART)                                                          \
  hipLaunchKernelGGL((attn_kernel<true, false, MODE, SPLIT, PART>), grid, dim3(kThreads), 0, stream, \
                     a, q, k, v, idx, cnt, o, nullptr)
    if (split_d) {
      if (part) BSA_LAUNCH_DENSE(2, true, true);
      else BSA_LAUNCH_DENSE(2, true, false);
    } else {
      if (part) BSA_LAUNCH_DENSE(0, false, true);
      else BSA_LAUNCH_DENSE(0, false, false);
    }
#undef BSA_LAUNCH_DENSE
    return hipGetLastError();
  }
  AttnArgs a = make_attn_args(g, stride, q_begin);
  const int mode = g.nk == 64 ? 2 : g.nk > kBlockTokens ? 1 : 0;
  const int nhw = g.nH * g.nW;
  if (pairs_query_blocks(g, q_begin)) {
    const int pairs = ((g.nb - q_begin) / nhw + 1) / 2 * nhw;
    a.nq8 = (pairs + 7) / 8 * 8;
    const unsigned total = (unsigned)((size_t)g.bh * a.nq8);
    for (unsigned x0 = 0; x0 < total; x0 += kLaunchWorkgroups) {
      a.x0 = (int)x0;
      const dim3 range(total - x0 < kLaunchWorkgroups ? total - x0 : kLaunchWorkgroups);
      if (lse)
        hipLaunchKernelGGL((attn_kernel<false, true, 0, false, false, true>), range, dim3(kThreads), 0,
                           stream, a, q, k, v, idx, cnt, o, lse);
      else
        hipLaunchKernelGGL((attn_kernel<false, false, 0, false, false, true>), range, dim3(kThreads),
                           0, stream, a, q, k, v, idx, cnt, o, lse);
      const hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
  }
#define BSA_LAUNCH_ATTN(LSE, MODE, SPLIT)                                                      \
  if (part)                                                                                     \
    hipLaunchKernelGGL((attn_kernel<false, LSE, MODE, SPLIT, true>), range, dim3(kThreads), 0,  \
                       stream, a, q, k, v, idx, cnt, o, lse);                                   \
  else                                                                                          \
    hipLaunchKernelGGL((attn_kernel<false, LSE, MODE, SPLIT, false>), range, dim3(kThreads), 0, \
                       stream, a, q, k, v, idx, cnt, o, lse)
#define BSA_LAUNCH_ATTN_MODES(LSE, SPLIT)                \
  if (mode == 0) { BSA_LAUNCH_ATTN(LSE, 0, SPLIT); }     \
  else if (mode == 1) { BSA_LAUNCH_ATTN(LSE, 1, SPLIT); } \
  else { BSA_LAUNCH_ATTN(LSE, 2, SPLIT); }
  for (unsigned x0 = 0; x0 < grid.x; x0 += kLaunchWorkgroups) {
    a.x0 = (int)x0;
    const dim3 range(grid.x - x0 < kLaunchWorkgroups ? grid.x - x0 : kLaunchWorkgroups);
    if (lse) {
      if (split) { BSA_LAUNCH_ATTN_MODES(true, true); }
      else { BSA_LAUNCH_ATTN_MODES(true, false); }
    } else {
      if (split) { BSA_LAUNCH_ATTN_MODES(false, true); }
      else { BSA_LAUNCH_ATTN_MODES(false, false); }
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
#undef BSA_LAUNCH_ATTN_MODES
#undef BSA_LAUNCH_ATTN
  return hipSuccess;
}

}  // namespace

// Sparse calls split themselves into workgroup ranges (above). Dense calls
// of more than 32,768 workgroups go out as launches of 8 (batch, head) pairs
// each: measured at 215K tokens (53,760 workgroups as one launch), each box
// against itself, the sparse kernel in 8-head launches took 45.9-47.7 ms
// against 47.9-48.4 ms on three boxes, with the clock climbing from 1.4 to
// 1.7 GHz over the launches of a step. Every workgroup's work is the same in
// any split, so outputs do not change.
hipError_t launch_attention(const Geom& g, const bf16_bits* q, const bf16_bits* k,
                            const bf16_bits* v, const int32_t* idx, const int32_t* cnt,
                            int stride, bool dense, bf16_bits* o, float* lse, int q_begin,
                            hipStream_t stream) {
  constexpr int kGroupHeads = 8;
  if (!dense || (size_t)g.bh * g.nb <= 32768 || g.bh <= kGroupHeads)
    return launch_attention_heads(g, q, k, v, idx, cnt, stride, dense, o, lse, q_begin, stream);
  for (int h0 = 0; h0 < g.bh; h0 += kGroupHeads) {
    Geom gh = g;
    gh.bh = g.bh - h0 < kGroupHeads ? g.bh - h0 : kGroupHeads;
    const size_t toff = (size_t)h0 * g.S * kHeadDim;
    const size_t roff = (size_t)h0 * g.nb;  // list rows of the group's first pair
    const hipError_t e = launch_attention_heads(
        gh, q + toff, k + toff, v + toff, dense ? idx : idx + roff * stride, dense ? cnt : cnt + roff,
        stride, dense, o + toff, lse ? lse + (size_t)h0 * g.S : nullptr, q_begin, stream);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace bsa
