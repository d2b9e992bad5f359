// Paged decode attention for gfx950: split-context partition kernel plus a
// log-sum-exp reduce across partitions.
//
// [L] "Paged Attention: OS-Inspired Memory Management for KV Caches",
//     "How PagedAttention works", step 4: walk the block table, load each
//     block's keys and values, attend exactly as over contiguous memory.
// [B] "What is PagedAttention and how does it manage KV cache?",
//     "How PagedAttention works": two-level indirection (table -> block,
//     tokens contiguous inside the block) keeps the loads coalesced.
//
// Work decomposition. One workgroup per (sequence s, KV head g, context
// partition p). A partition is P consecutive tokens, P a multiple of 16; the
// work unit is 16 tokens of one KV head (a 4 KiB K tile and a 4 KiB V tile),
// so a block of B tokens is B / 16 units and a partition may start inside a
// block. With B = 8 a unit spans two blocks: its first 8 tokens come from
// one 2 KiB tile, the other 8 from the next block's. The workgroup's waves take the partition's units round-robin.
// Inside a wave, lane = 16 * r + c: DPP row r (0..3) holds tokens 4i + r of
// the unit (i = 0..3) and lane c of the row holds dims 8c .. 8c+7, so each
// 16-byte load of a row reads 256 contiguous bytes and a wave-wide load reads
// 1 KiB of the contiguous 4 KiB tile.
//
// q.K: 4 dot2 per lane, then a sum over the 16 lanes of the DPP row (four
// DPP adds). Softmax: every lane keeps an online (max, sum) for the tokens of
// its row, in the log2 domain (scores are pre-multiplied by scale * log2 e,
// exponentials are exp2). P.V: fp32 FMA of p with the fp16 V row chunk. At the
// end the 4 rows of a wave merge by cross-row shuffles, the 4 waves merge in
// LDS; a single-partition sequence writes fp16 output directly, otherwise the
// partition's (max, sum) in fp32 and its normalised result acc[D] / sum in
// fp16 go to the workspace for the reduce kernel (fp16 rows: half the bytes
// of fp32 sums, measured 0.6 % faster per call on the batch-128 chat
// workload, where scattered partial writes amid the read stream are dear).
//
// Exact masking: tokens at or past L only occur in a sequence's last block;
// that block takes a masked path that selects (never multiplies) so NaN or
// Inf in unused slots cannot reach the result. Arithmetic order depends only
// on logical positions, so physical ids never change an output bit.
#include "decode_even.h"
#include "pa_debug.h"
#include "pa_internal.h"

namespace pa {
namespace {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr float kNegBig = -1.0e30f;   // "no token yet" running max; exp2 of it is 0

__device__ __forceinline__ float dpp_row_sum(float x) {
  // quad_perm [1,0,3,2], quad_perm [2,3,0,1], row_half_mirror, row_mirror:
  // after the four steps every lane of the 16-lane row holds the row's sum.
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0xB1,
                                                             0xF, 0xF, false));
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x4E,
                                                             0xF, 0xF, false));
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x141,
                                                             0xF, 0xF, false));
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x140,
                                                             0xF, 0xF, false));
  return x;
}

// Element values are passed by value before the bit cast: a bit cast applied
// directly to an ext-vector element expression (a.y) reads element x.
__device__ __forceinline__ half2_t as_h2(uint32_t u) { return __builtin_bit_cast(half2_t, u); }

__device__ __forceinline__ float dot8(const u32x4& a, const u32x4& b) {
  float s = 0.f;
  s = __builtin_amdgcn_fdot2(as_h2(a.x), as_h2(b.x), s, false);
  s = __builtin_amdgcn_fdot2(as_h2(a.y), as_h2(b.y), s, false);
  s = __builtin_amdgcn_fdot2(as_h2(a.z), as_h2(b.z), s, false);
  s = __builtin_amdgcn_fdot2(as_h2(a.w), as_h2(b.w), s, false);
  return s;
}

__device__ __forceinline__ float lo_f(uint32_t u) {
  return (float)__builtin_bit_cast(half2_t, u).x;
}
__device__ __forceinline__ float hi_f(uint32_t u) {
  return (float)__builtin_bit_cast(half2_t, u).y;
}

// acc[0..7] += p * v (8 fp16 values in a uint4), fp32 FMA
__device__ __forceinline__ void fma8(float* acc, float p, const u32x4& v) {
  acc[0] = __builtin_fmaf(p, lo_f(v.x), acc[0]);
  acc[1] = __builtin_fmaf(p, hi_f(v.x), acc[1]);
  acc[2] = __builtin_fmaf(p, lo_f(v.y), acc[2]);
  acc[3] = __builtin_fmaf(p, hi_f(v.y), acc[3]);
  acc[4] = __builtin_fmaf(p, lo_f(v.z), acc[4]);
  acc[5] = __builtin_fmaf(p, hi_f(v.z), acc[5]);
  acc[6] = __builtin_fmaf(p, lo_f(v.w), acc[6]);
  acc[7] = __builtin_fmaf(p, hi_f(v.w), acc[7]);
}

// One pipelined work unit is 16 tokens of one KV head: a 4 KiB K tile and a
// 4 KiB V tile at D = 128. A block of B = 32 tokens is two units, so the
// register footprint does not grow with B.
constexpr int kUnit = 16;

struct Tile {
  u32x4 k[4];   // row r of the wave holds tokens 4i + r of the unit
  u32x4 v[4];
};

// Tile loads go through a buffer resource built on the unit's tile base
// (wave-uniform, so it lives in scalar registers); each lane supplies its
// byte offset within the row group (vector offset) and the row group's
// offset rides in the scalar offset. The resource's range `nbytes` is checked
// by the hardware against the lane's offset: out-of-range lanes get zeros
// and touch no memory. A range of 0 therefore turns the load into a no-op
// that still counts as issued (the loop's wait counts stay uniform), and a
// range of 256 * valid_tokens never drops a valid token's row (a valid
// token t = 4i + r has vector offset below 256 (r + 1) <= 256 * valid). Every
// offset lies inside the unit's 4 KiB tile either way. Word 3 is the
// raw-buffer format for the gfx9 family; cache policy bit 1 is the
// non-temporal hint.
constexpr int kUnitBytes = kUnit * kHeadDim * 2;
constexpr int kRsrcWord3 = 0x00020000;

template <bool NT>
__device__ __forceinline__ void load_tile(Tile& t, const _Float16* kb, const _Float16* vb,
                                          int nbytes, unsigned lane_byte_off) {
  const __amdgpu_buffer_rsrc_t rk =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<_Float16*>(kb), 0, nbytes, kRsrcWord3);
  const __amdgpu_buffer_rsrc_t rv =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<_Float16*>(vb), 0, nbytes, kRsrcWord3);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int so = i * (4 * kHeadDim * 2);   // row i of the tile: scalar offset
    t.k[i] = __builtin_amdgcn_raw_buffer_load_b128(rk, lane_byte_off, so, NT ? 2 : 0);
    t.v[i] = __builtin_amdgcn_raw_buffer_load_b128(rv, lane_byte_off, so, NT ? 2 : 0);
  }
}

// B = 8: row groups 0-1 (tokens 0-7) from the first block's tile, 2-3 (tokens
// 8-15) from the second's, each with its own range (an empty second range
// leaves a block the sequence does not have untouched).
template <bool NT>
__device__ __forceinline__ void load_tile_split(Tile& t, const _Float16* kb0, const _Float16* vb0,
                                                int nbytes0, const _Float16* kb1,
                                                const _Float16* vb1, int nbytes1,
                                                unsigned lane_byte_off) {
  const __amdgpu_buffer_rsrc_t rk0 =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<_Float16*>(kb0), 0, nbytes0, kRsrcWord3);
  const __amdgpu_buffer_rsrc_t rv0 =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<_Float16*>(vb0), 0, nbytes0, kRsrcWord3);
  const __amdgpu_buffer_rsrc_t rk1 =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<_Float16*>(kb1), 0, nbytes1, kRsrcWord3);
  const __amdgpu_buffer_rsrc_t rv1 =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<_Float16*>(vb1), 0, nbytes1, kRsrcWord3);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int so = (i & 1) * (4 * kHeadDim * 2);
    t.k[i] = __builtin_amdgcn_raw_buffer_load_b128(i < 2 ? rk0 : rk1, lane_byte_off, so, NT ? 2 : 0);
    t.v[i] = __builtin_amdgcn_raw_buffer_load_b128(i < 2 ? rv0 : rv1, lane_byte_off, so, NT ? 2 : 0);
  }
}

// Online-softmax update of one lane's state for the unit in `t`.
// tok_base = logical position of the unit's token 0 for this lane's row
// (unit start + r); with MASK, tokens at or past `L` are excluded by
// selection.
template <int G, bool MASK>
__device__ __forceinline__ void process_tile(const Tile& t, const u32x4 (&q)[G], float (&m)[G],
                                             float (&l)[G], float (&acc)[G][8], float scale_log2,
                                             int tok_base, int L) {
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float sc[4];
    float mx = m[h];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      sc[i] = dpp_row_sum(dot8(q[h], t.k[i])) * scale_log2;
      if (MASK) {
        const bool valid = (tok_base + 4 * i) < L;
        sc[i] = valid ? sc[i] : kNegBig;
      }
      mx = __builtin_fmaxf(mx, sc[i]);
    }
    const float alpha = __builtin_amdgcn_exp2f(m[h] - mx);
    m[h] = mx;
    float lsum = l[h] * alpha;
#pragma unroll
    for (int d = 0; d < 8; ++d) acc[h][d] *= alpha;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float p = __builtin_amdgcn_exp2f(sc[i] - mx);
      if (MASK) {
        const bool valid = (tok_base + 4 * i) < L;
        if (valid) {
          lsum += p;
          fma8(acc[h], p, t.v[i]);
        }
      } else {
        lsum += p;
        fma8(acc[h], p, t.v[i]);
      }
    }
    l[h] = lsum;
  }
}

// Merge state (mo, lo, acco) into (m, l, acc).
__device__ __forceinline__ void merge_state(float& m, float& l, float* acc, float mo, float lo,
                                            const float* acco) {
  const float mx = __builtin_fmaxf(m, mo);
  const float a = __builtin_amdgcn_exp2f(m - mx);
  const float b = __builtin_amdgcn_exp2f(mo - mx);
  m = mx;
  l = l * a + lo * b;
#pragma unroll
  for (int d = 0; d < 8; ++d) acc[d] = acc[d] * a + acco[d] * b;
}

// Tokens [tok0, tok0 + len) of sequence s (clamped length L) and KV head g
// (len > 0): piece p of the nparts pieces the sequence's walk is cut into.
// With one piece the result is the output; otherwise the piece's maximum and
// sum (fp32) and its normalised result (fp16) go to partial row p.
// G query heads share KV head g. The workgroup's waves are split into NH =
// G / HPW head groups (wave w serves heads HPW * (w % NH) ... of the group)
// and NU = NW / NH unit subsets (wave w walks units w / NH, + NU, ...), so a
// wave holds the state of at most HPW heads whatever G is. When NH > 1 each
// K/V tile is loaded by NH waves of the same workgroup: the repeats are
// served by the caches, HBM traffic is unchanged.
template <int BT, int G, int HPW, int NW, int DEPTH, bool NT>
__device__ __forceinline__ void vec_piece(const DecodeArgs& a, int s, int g, int L, int tok0,
                                          int len, int nparts, int p) {
  s = __builtin_amdgcn_readfirstlane(s);
  g = __builtin_amdgcn_readfirstlane(g);
  L = __builtin_amdgcn_readfirstlane(L);
  tok0 = __builtin_amdgcn_readfirstlane(tok0);
  len = __builtin_amdgcn_readfirstlane(len);
  nparts = __builtin_amdgcn_readfirstlane(nparts);
  p = __builtin_amdgcn_readfirstlane(p);
  constexpr int D = kHeadDim;
  constexpr int NH = G / HPW;           // head groups
  constexpr int NU = NW / NH;           // unit subsets
  static_assert(BT == 8 || BT % kUnit == 0, "block size must be 8 or a multiple of 16");
  constexpr bool kSplit = BT == 8;      // a unit spans two blocks
  const int B = BT > 0 ? BT : a.B;      // BT = 0: block size known at run time only
  const int UPB = kSplit ? 1 : B / kUnit;   // units per block (B >= 16)
  static_assert(DEPTH == 1 || DEPTH == 2, "prefetch depth 1 or 2");
  static_assert(G % HPW == 0 && NW % NH == 0, "waves must cover the head groups");
  __shared__ float s_acc[NW][HPW][D];
  __shared__ float s_ml[NW][HPW][2];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = lane >> 4;
  const int c = lane & 15;
  const int hgrp = wave % NH;
  const int usub = wave / NH;
  const int hq0 = g * G;
  const int64_t n_out = (int64_t)a.S * a.Hq * D;   // elements of out and of the query
  (void)n_out;
  const int nunits = (len + kUnit - 1) / kUnit;
  const int n_full = len / kUnit;        // units with every slot valid
  // tok0 is a multiple of 16, not necessarily of B: the piece may start
  // inside a block. U0 is its first unit counted from the sequence start.
  const int U0 = tok0 / kUnit;
  // blocks holding the piece's tokens (B = 8: two per unit, the last
  // possibly absent when the final unit ends within its first half)
  const int blk0 = kSplit ? 2 * U0 : U0 / UPB;
  const int nblk = kSplit ? (len + 7) / 8 : (U0 + nunits - 1) / UPB - blk0 + 1;

  const int hw0 = hq0 + hgrp * HPW;      // this wave's first query head
  u32x4 q[HPW];
#pragma unroll
  for (int h = 0; h < HPW; ++h) {
    const int64_t qo = ((int64_t)s * a.Hq + hw0 + h) * D + 8 * c;
    q[h] = PA_IN_BOUNDS(kBsQuery, qo >= 0 && qo + 8 <= n_out)
               ? *reinterpret_cast<const u32x4*>(a.q + qo)
               : u32x4{0, 0, 0, 0};
  }
  float m[HPW], l[HPW], acc[HPW][8];
#pragma unroll
  for (int h = 0; h < HPW; ++h) {
    m[h] = kNegBig;
    l[h] = 0.f;
#pragma unroll
    for (int d = 0; d < 8; ++d) acc[h][d] = 0.f;
  }

  const int32_t* trow = a.tables + (int64_t)s * a.MB + blk0;
  const unsigned lane_off = (r * D + 8 * c) * 2u;   // bytes
  const int64_t pool_elems = (int64_t)a.NB * a.Hkv * B * D;
  (void)pool_elems;

  // Blocks are walked in chunks of 64: one lane holds one table entry of the
  // chunk and v_readlane hands the wave its entry, so no table access sits
  // inside the pipelined loop (a partition of at most 64 blocks, the default,
  // is a single chunk). Wave w takes the chunk's units w, w + NW, ... and
  // issues the loads of the units DEPTH steps ahead before computing the
  // current one. The load instructions are unconditional (past the wave's
  // last unit they are no-ops with an empty range) so that the compiler's
  // wait counts stay partial. Only the partition's final unit can be
  // partial; its loads fetch only the valid tokens and it takes the masked
  // update. A table entry outside the pool is clamped to block 0 (no access
  // leaves the pool; the result for such input is unspecified).
  for (int cb = 0; cb < nblk; cb += 64) {
    const int ce = cb + 64 < nblk ? cb + 64 : nblk;
    const int tbl = cb + lane < ce && PA_IN_BOUNDS(kBsTable, (int64_t)s * a.MB + blk0 + cb + lane <
                                                              (int64_t)a.S * a.MB)
                        ? trow[cb + lane]
                        : -1;
    // the partition's units (counted from its start) whose block is in [cb, ce)
    const int ub0 = kSplit ? cb / 2 : (blk0 + cb) * UPB - U0;
    const int ue0 = kSplit ? (ce + 1) / 2 : (blk0 + ce) * UPB - U0;
    const int ub = ub0 > 0 ? ub0 : 0;
    const int ue = ue0 < nunits ? ue0 : nunits;
    auto locate = [&](int u) -> int64_t {
      const int au = U0 + u;
      const int bi = au / UPB;
      const int phys = __builtin_amdgcn_readlane(tbl, bi - blk0 - cb);
      const int safe = (unsigned)phys < (unsigned)a.NB ? phys : 0;
      return (((int64_t)safe * a.Hkv + g) * B + (au - bi * UPB) * kUnit) * D;
    };
    // B = 8: tile base of block j (0, 1) of unit u. The chunk's 64 entries
    // hold whole units (units start at even block indices), so both lanes
    // read here are in the chunk; an entry past the partition's blocks is -1
    // and is clamped to block 0, with an empty range.
    auto locate_half = [&](int u, int j) -> int64_t {
      const int phys = __builtin_amdgcn_readlane(tbl, 2 * u + j - cb);
      const int safe = (unsigned)phys < (unsigned)a.NB ? phys : 0;
      return ((int64_t)safe * a.Hkv + g) * B * D;
    };
    // Loads unit u, or issues a no-op load when u is past the wave's last unit.
    auto fetch = [&](Tile& t, int u) {
      const bool live = u < ue;
      const int uu = live ? u : ue - 1;
      if constexpr (kSplit) {
        const int valid = len - uu * kUnit;
        const int64_t b0 = locate_half(uu, 0);
        const int64_t b1 = locate_half(uu, 1);
        const int v0 = valid < 8 ? valid : 8;
        const int v1 = valid - 8 < 0 ? 0 : (valid - 8 > 8 ? 8 : valid - 8);
        int n0 = live ? v0 * (kHeadDim * 2) : 0;
        int n1 = live ? v1 * (kHeadDim * 2) : 0;
        // each half tile (8 rows) inside the pool
        if (!PA_IN_BOUNDS(kBsPool, b0 >= 0 && b0 + 8 * kHeadDim <= pool_elems)) n0 = 0;
        if (!PA_IN_BOUNDS(kBsPool, b1 >= 0 && b1 + 8 * kHeadDim <= pool_elems)) n1 = 0;
        load_tile_split<NT>(t, a.k_pool + b0, a.v_pool + b0, n0, a.k_pool + b1, a.v_pool + b1, n1,
                            lane_off);
      } else {
        const int64_t base = locate(uu);
        const int valid = len - uu * kUnit;
        int nbytes = !live ? 0 : (valid >= kUnit ? kUnitBytes : valid * (kHeadDim * 2));
        // the unit's whole tile (16 rows) inside the pool
        if (!PA_IN_BOUNDS(kBsPool, base >= 0 && base + kUnit * kHeadDim <= pool_elems)) nbytes = 0;
        load_tile<NT>(t, a.k_pool + base, a.v_pool + base, nbytes, lane_off);
      }
    };
    auto step = [&](const Tile& t, int u) {
      if (u < n_full) {
        process_tile<HPW, false>(t, q, m, l, acc, a.scale_log2, 0, 0);
      } else {
        process_tile<HPW, true>(t, q, m, l, acc, a.scale_log2, tok0 + u * kUnit + r, L);
      }
    };
    int u = ub + usub;
    if (u >= ue) continue;
    if (DEPTH == 1) {
      Tile t0, t1;
      fetch(t0, u);
      while (true) {
        int un = u + NU;
        fetch(t1, un);
        step(t0, u);
        if (un >= ue) break;
        u = un;
        un = u + NU;
        fetch(t0, un);
        step(t1, u);
        if (un >= ue) break;
        u = un;
      }
    } else {
      Tile t0, t1, t2;
      fetch(t0, u);
      int un = u + NU;
      fetch(t1, un);
      while (true) {
        un = u + 2 * NU;
        fetch(t2, un);
        step(t0, u);
        u += NU;
        if (u >= ue) break;
        un = u + 2 * NU;
        fetch(t0, un);
        step(t1, u);
        u += NU;
        if (u >= ue) break;
        un = u + 2 * NU;
        fetch(t1, un);
        step(t2, u);
        u += NU;
        if (u >= ue) break;
      }
    }
  }

  // merge the four rows of the wave (lanes c, c+16, c+32, c+48)
#pragma unroll
  for (int h = 0; h < HPW; ++h) {
#pragma unroll
    for (int x = 16; x <= 32; x *= 2) {
      const float mo = __shfl_xor(m[h], x);
      const float lo = __shfl_xor(l[h], x);
      float ao[8];
#pragma unroll
      for (int d = 0; d < 8; ++d) ao[d] = __shfl_xor(acc[h][d], x);
      merge_state(m[h], l[h], acc[h], mo, lo, ao);
    }
  }
  if (r == 0) {
#pragma unroll
    for (int h = 0; h < HPW; ++h) {
#pragma unroll
      for (int d = 0; d < 8; ++d) s_acc[wave][h][8 * c + d] = acc[h][d];
      if (c == 0) {
        s_ml[wave][h][0] = m[h];
        s_ml[wave][h][1] = l[h];
      }
    }
  }
  __syncthreads();

  // combine the unit subsets: thread e handles output element (h, d); the
  // waves serving head h are hg + NH * k, k < NU, with hg = h / HPW
  for (int e = threadIdx.x; e < G * D; e += NW * 64) {
    const int h = e / D;
    const int d = e % D;
    const int hg = h / HPW;
    const int hh = h % HPW;
    float mx = s_ml[hg][hh][0];
#pragma unroll
    for (int k = 1; k < NU; ++k) mx = __builtin_fmaxf(mx, s_ml[hg + NH * k][hh][0]);
    float lsum = 0.f, num = 0.f;
#pragma unroll
    for (int k = 0; k < NU; ++k) {
      const int w = hg + NH * k;
      const float f = __builtin_amdgcn_exp2f(s_ml[w][hh][0] - mx);
      lsum += f * s_ml[w][hh][1];
      num += f * s_acc[w][hh][d];
    }
    const int hq = hq0 + h;
    if (nparts == 1) {
      const float o = lsum > 0.f ? num / lsum : 0.f;
      const int64_t oi = ((int64_t)s * a.Hq + hq) * D + d;
      if (PA_IN_BOUNDS(kBsOut, oi >= 0 && oi < n_out)) a.out[oi] = (_Float16)o;
    } else {
      const int64_t row = ((int64_t)s * a.Hq + hq) * a.Pmax + p;
      if (PA_IN_BOUNDS(kBsPartial, row >= 0 && row < (int64_t)a.S * a.Hq * a.Pmax)) {
        reinterpret_cast<_Float16*>(a.part_acc)[row * D + d] = (_Float16)(lsum > 0.f ? num / lsum : 0.f);
        if (d == 0) {
          a.part_ml[row * 2] = mx;
          a.part_ml[row * 2 + 1] = lsum;
        }
      }
    }
  }
}

// One workgroup per (partition, sequence, KV head), partitions of a.P tokens.
// blockIdx -> (p, s, g) with g fastest: consecutive workgroups go to
// consecutive XCDs, so every workgroup of one KV head lands on the same XCD
// when Hkv is a multiple of 8 (shared prefix blocks stay in one L2).
template <int BT, int G, int HPW, int NW, int DEPTH, bool NT>
__global__ __launch_bounds__(NW * 64)
__attribute__((amdgpu_waves_per_eu(PA_DECODE_MIN_WAVES_PER_EU)))
void decode_partition_kernel(const DecodeArgs a) {
  constexpr int D = kHeadDim;
  const int B = BT > 0 ? BT : a.B;
  int id = blockIdx.x;
  const int g = id % a.Hkv;
  id /= a.Hkv;
  const int s = id % a.S;
  const int p = id / a.S;
  int L = PA_IN_BOUNDS(kBsLength, s < a.S) ? a.lens[s] : 0;
  L = L < 0 ? 0 : L;
  L = L > a.MB * B ? a.MB * B : L;
  L = L > a.Pmax * a.P ? a.Pmax * a.P : L;
  const int tok0 = p * a.P;
  const int hq0 = g * G;
  const int64_t n_out = (int64_t)a.S * a.Hq * D;
  (void)n_out;
  if (tok0 >= L) {
    if (p == 0) {  // empty sequence: zero output
      for (int e = threadIdx.x; e < G * D; e += NW * 64) {
        const int64_t o = ((int64_t)s * a.Hq + hq0 + e / D) * D + (e % D);
        if (PA_IN_BOUNDS(kBsOut, o >= 0 && o < n_out)) a.out[o] = (_Float16)0.f;
      }
    }
    return;
  }
  const int nparts = (L + a.P - 1) / a.P;
  const int len = (tok0 + a.P < L ? tok0 + a.P : L) - tok0;
  vec_piece<BT, G, HPW, NW, DEPTH, NT>(a, s, g, L, tok0, len, nparts, p);
}

// Equal-work split of the whole batch (decode_even.h), one or two query heads
// per KV head.
template <int BT, int G, int HPW, int NW, int DEPTH, bool NT>
__global__ __launch_bounds__(NW * 64)
__attribute__((amdgpu_waves_per_eu(PA_DECODE_MIN_WAVES_PER_EU)))
void decode_vec_even_kernel(const DecodeArgs a) {
  constexpr int D = kHeadDim;
  even_split_walk<NW * 64>(
      a, BT > 0 ? BT : a.B,
      [&](int s, int g, int L, int tok0, int len, int nparts, int p) {
        vec_piece<BT, G, HPW, NW, DEPTH, NT>(a, s, g, L, tok0, len, nparts, p);
      },
      [&](int s) {
        const int64_t n_out = (int64_t)a.S * a.Hq * D;
        (void)n_out;
        for (int e = threadIdx.x; e < a.Hkv * G * D; e += NW * 64) {
          const int64_t o = (int64_t)s * a.Hq * D + e;
          if (PA_IN_BOUNDS(kBsOut, o >= 0 && o < n_out)) a.out[o] = (_Float16)0.f;
        }
      });
}

// One wave per (s, hq): out = sum_p 2^(m_p - M) l_p o_p / sum_p 2^(m_p - M) l_p
// (o_p the piece's normalised result, l_p its sum) over the sequence's pieces (its partitions, or the counts the even split
// recorded). Sequences of one piece were finished by the partition kernel.
__global__ __launch_bounds__(64) void decode_reduce_kernel(const DecodeArgs a, int B_MB) {
  constexpr int D = kHeadDim;
  const int hq = blockIdx.x % a.Hq;
  const int s = blockIdx.x / a.Hq;
  int L = PA_IN_BOUNDS(kBsLength, s < a.S) ? a.lens[s] : 0;
  L = L < 0 ? 0 : L;
  L = L > B_MB ? B_MB : L;
  const int pc = s * a.Hkv + hq / (a.Hq / a.Hkv);
  int np = a.part_np ? (PA_IN_BOUNDS(kBsPartial, pc < a.S * a.Hkv) ? a.part_np[pc] : 0)
                     : (L + a.P - 1) / a.P;
  np = np > a.Pmax ? a.Pmax : np;
  if (np <= 1) return;
  const int64_t row0 = ((int64_t)s * a.Hq + hq) * a.Pmax;
  if (!PA_IN_BOUNDS(kBsPartial, row0 >= 0 && row0 + np <= (int64_t)a.S * a.Hq * a.Pmax)) return;
  // one pass, rescaling to the running maximum: the loads of all pieces are
  // independent of the arithmetic and go out together
  float mx = kNegBig, den = 0.f, n0 = 0.f, n1 = 0.f;
  const int d = 2 * threadIdx.x;
#pragma unroll 4
  for (int p = 0; p < np; ++p) {
    const float mp = a.part_ml[(row0 + p) * 2];
    const float lp = a.part_ml[(row0 + p) * 2 + 1];
    // the piece's normalised result in fp16: scale back by its sum
    const _Float16* hv = reinterpret_cast<const _Float16*>(a.part_acc) + (row0 + p) * D + d;
    const float2 v = float2{(float)hv[0] * lp, (float)hv[1] * lp};
    const float mn = __builtin_fmaxf(mx, mp);
    const float fo = __builtin_amdgcn_exp2f(mx - mn);
    const float fp = __builtin_amdgcn_exp2f(mp - mn);
    den = den * fo + fp * lp;
    n0 = n0 * fo + fp * v.x;
    n1 = n1 * fo + fp * v.y;
    mx = mn;
  }
  const int64_t oi = ((int64_t)s * a.Hq + hq) * D + d;
  if (!PA_IN_BOUNDS(kBsOut, oi >= 0 && oi + 2 <= (int64_t)a.S * a.Hq * D)) return;
  _Float16* o = a.out + oi;
  o[0] = (_Float16)(den > 0.f ? n0 / den : 0.f);
  o[1] = (_Float16)(den > 0.f ? n1 / den : 0.f);
}

template <int BT, int G>
hipError_t launch_partition(const DecodeArgs& a, hipStream_t stream) {
  constexpr int HPW = G < kDecodeHeadsPerWave ? G : kDecodeHeadsPerWave;
  constexpr int NH = G / HPW;
  constexpr int NW = decode_waves(G) > NH ? decode_waves(G) : NH;
  if (a.part_np) {
    auto kernel = decode_vec_even_kernel<BT, G, HPW, NW, kDecodeDepth, kDecodeNontemporal>;
    // one head per KV head: two workgroups per CU (one wave per SIMD) measured
    // 2 % faster on the chat lengths than all eight resident ones; two heads:
    // as many as are resident (no count measured better)
    const int64_t grid = even_split_grid(a, kernel, NW * 64, G == 1 ? 2 : 1 << 20);
    if (grid <= 0) return hipErrorInvalidValue;
    kernel<<<(unsigned)grid, NW * 64, 0, stream>>>(a);
    return hipGetLastError();
  }
  const int64_t grid = (int64_t)a.Pmax * a.S * a.Hkv;
  if constexpr (G <= 2) {
    if (grid <= kSmallLaunchWorkgroups) {
      decode_partition_kernel<BT, G, HPW, 2 * NW, kDecodeDepth, kDecodeNontemporal>
          <<<(unsigned)grid, 2 * NW * 64, 0, stream>>>(a);
      return hipGetLastError();
    }
  }
  decode_partition_kernel<BT, G, HPW, NW, kDecodeDepth, kDecodeNontemporal>
      <<<(unsigned)grid, NW * 64, 0, stream>>>(a);
  return hipGetLastError();
}

template <int BT>
hipError_t launch_partition_g(const DecodeArgs& a, int G, hipStream_t stream) {
  switch (G) {
    case 1: return launch_partition<BT, 1>(a, stream);
    case 2: return launch_partition<BT, 2>(a, stream);
    // groups of 4 and 8 on the matrix cores
    case 4: return launch_decode_mfma(a, BT > 0 ? BT : a.B, 4, stream);
    case 8: return launch_decode_mfma(a, BT > 0 ? BT : a.B, 8, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

PA_BOUNDS_COLLECTOR(bounds_take_decode)

hipError_t launch_decode(const DecodeArgs& a, int B, int G, hipStream_t stream) {
  hipError_t e;
  switch (B) {   // the common block sizes are compile-time specialisations
    case 8: e = launch_partition_g<8>(a, G, stream); break;
    case 16: e = launch_partition_g<16>(a, G, stream); break;
    case 32: e = launch_partition_g<32>(a, G, stream); break;
    default: e = launch_partition_g<0>(a, G, stream); break;
  }
  if (e != hipSuccess || a.Pmax <= 1) return e;
  const int64_t grid = (int64_t)a.S * a.Hq;
  decode_reduce_kernel<<<(unsigned)grid, 64, 0, stream>>>(a, a.MB * B);
  return hipGetLastError();
}

}  // namespace pa
