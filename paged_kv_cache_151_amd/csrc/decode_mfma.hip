// Grouped-query decode on the matrix cores, for groups of 4 and 8 query heads.
//
// [L] "Paged Attention: OS-Inspired Memory Management for KV Caches",
//     "How PagedAttention works", step 4: walk the block table, load each
//     block's keys and values, attend exactly as over contiguous memory.
//
// With 8 query heads per KV head every loaded K/V tile meets 8 queries, and
// the vector path's arithmetic (dot products, row sums, P.V per head) becomes
// the bound; with 4 it is close to it. Here the G heads are the rows of a
// 16-row matrix tile (rows G-15 are zero queries whose results are discarded)
// and each 16-token unit costs four score products and eight value products:
//   scores   S^T = K Q^T (v_mfma_f32_16x16x32_f16, lane l = 16 kq + m): the A
//            operand is key token m, dims 32c + 8kq .. +7, loaded from the
//            pool straight into registers; the B operand is query head m, the
//            same dims, held in registers; lane l receives S for head m and
//            tokens 4kq + r of the unit.
//   output   O^T = V^T P^T per 16-dim tile n (v_mfma_f32_16x16x16_f16): the B
//            operand is P as the score product left it (head m, tokens
//            4kq .. 4kq + 3); the A operand, V for the same tokens at dim
//            16n + m, comes from the unit's V tile staged in LDS by one
//            transposing read (ds_read_b64_tr_b16: in each 16-lane group, lane
//            i receives 16-bit word i % 4 from the address of lane 4e + i / 4
//            as its element e). Lane l ends with O[head m][dims 16n + 4kq + r].
// Each head's softmax state lives in the four lanes of its row (m, kq = 0..3);
// rescaling is lazy, as in the prefill kernel: the running maximum is raised,
// and the accumulators rescaled, only when some head's new scores exceed it
// by 2^8, decided on lane maxima (a head exceeds the bound exactly when one of
// its lanes does).
//
// Everything else is the partition kernel's: one workgroup per (partition,
// sequence, KV head) in the same order, the same length clamping and empty
// sequence, block-table chunks of 64 entries handed out by v_readlane, units
// dealt round-robin to the waves and fetched one unit ahead with empty-range
// no-op loads past a wave's last unit, the same cross-wave merge, and the
// same partial rows: a piece's normalised result in fp16 (the reduce kernel
// scales it back by the piece's sum). Scattered writes amid the read stream
// cost far more than their share of the bandwidth: with eight heads per
// piece, fp32 rows took about 4 % of a call on the chat lengths. V tiles go to a per-wave LDS double
// buffer by buffer loads that write LDS directly; piece c of V row r sits at
// c ^ 2 (r % 8), which keeps the transposing reads free of bank conflicts.
#include "decode_even.h"
#include "pa_debug.h"
#include "pa_internal.h"

namespace pa {
namespace {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef short s4 __attribute__((ext_vector_type(4)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) unsigned char lds_u8;
typedef __attribute__((address_space(3))) s4 lds_s4;

constexpr float kNegBigG = -1.0e30f;      // "no token yet"; exp2 of it is 0
constexpr float kSlackG = 8.0f;           // lazy rescaling slack, log2 units
constexpr int kRowBytesG = kHeadDim * 2;  // one token row of one KV head
constexpr int kTileBytesG = kDecodeUnit * kRowBytesG;
constexpr int kRsrcWord3G = 0x00020000;   // raw buffer, gfx9 family

// lgkmcnt(0): every LDS read this wave issued has returned its data.
#define PA_G_WAIT_LDS() __builtin_amdgcn_s_waitcnt(0xC07F)
// vmcnt(0): every vector memory operation of this wave has completed.
#define PA_G_WAIT_VM0() __builtin_amdgcn_s_waitcnt(0x0F70)

template <int S>
struct Stage {
  static constexpr int value = S;
};

// Waves per workgroup and units fetched ahead of the one being computed
// (compile-time tuning parameters).
#ifndef PA_MFMA_WAVES
#define PA_MFMA_WAVES 4
#endif
#ifndef PA_MFMA_DEPTH
#define PA_MFMA_DEPTH 1
#endif

// 16-byte buffer loads of each lane into LDS (lane i's bytes at dst + 16 i;
// lanes past the resource's range write zeros), plain and non-temporal.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, lds_u8* dst, unsigned voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)dst, 16, voff,
                                           0, 0, 0);
}
__device__ __forceinline__ void dma16_nt(__amdgpu_buffer_rsrc_t r, lds_u8* dst, unsigned voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)dst, 16, voff,
                                           0, 0, 2);
}

// Tokens [tok0, tok0 + len) of sequence s and KV head g (len > 0): piece p of
// the nparts pieces the sequence's walk is cut into. With one piece the
// result is the output; otherwise the piece's (maximum, sum, accumulators)
// go to partial row p for the reduce kernel.
template <int BT, int G, int NW, int DEPTH, bool NT>
__device__ __forceinline__ void attend_piece(const DecodeArgs& a, int s, int g, int tok0, int len,
                                             int nparts, int p) {
  // the piece is the same for every lane: keep its description in scalar
  // registers (integer division and loads after stores leave it in vector ones)
  s = __builtin_amdgcn_readfirstlane(s);
  g = __builtin_amdgcn_readfirstlane(g);
  tok0 = __builtin_amdgcn_readfirstlane(tok0);
  len = __builtin_amdgcn_readfirstlane(len);
  nparts = __builtin_amdgcn_readfirstlane(nparts);
  p = __builtin_amdgcn_readfirstlane(p);
  static_assert(G == 4 || G == 8, "groups of 4 or 8 query heads");
  static_assert(DEPTH == 1 || DEPTH == 2, "prefetch depth 1 or 2");
  constexpr int D = kHeadDim;
  constexpr int U = kDecodeUnit;
  static_assert(BT == 0 || BT == 8 || BT % U == 0, "block size 8 or a multiple of 16");
  constexpr bool kSplit = BT == 8;      // a unit spans two blocks
  const int B = BT > 0 ? BT : a.B;
  const int UPB = kSplit ? 1 : B / U;   // units per block (B >= 16)
  // per-wave V tile buffers, one array per stage (the compiler tracks loads
  // into LDS per array and waits only where a read meets its stage); after
  // the walk each wave's tile of stage 0 holds its G x D accumulators for the
  // cross-wave merge (G * D * 4 bytes fit one 4 KiB tile)
  static_assert(G * D * 4 <= kTileBytesG, "accumulators fit a wave's tile");
  __shared__ __attribute__((aligned(16))) unsigned char s_v0[NW * kTileBytesG];
  __shared__ __attribute__((aligned(16))) unsigned char s_v1[NW * kTileBytesG];
  __shared__ __attribute__((aligned(16))) unsigned char s_v2[DEPTH == 2 ? NW * kTileBytesG : 16];
  __shared__ float s_ml[NW][G][2];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int m = lane & 15;
  const int kq = lane >> 4;
  const int hq0 = g * G;
  const int64_t n_out = (int64_t)a.S * a.Hq * D;               // elements of out and of the query
  const int64_t pool_elems = (int64_t)a.NB * a.Hkv * B * D;    // elements of each pool
  (void)n_out;
  (void)pool_elems;
  const int nunits = (len + U - 1) / U;
  const int U0 = tok0 / U;
  const int blk0 = kSplit ? 2 * U0 : U0 / UPB;
  const int nblk = kSplit ? (len + 7) / 8 : (U0 + nunits - 1) / UPB - blk0 + 1;

  // The lazy maximum below is taken on unscaled scores, which keeps their
  // order only for a scale >= 0. A negative scale is applied as |scale| to the
  // negated queries instead: flipping the fp16 sign bits is exact, so every
  // score changes sign exactly and scale * score is unchanged.
  const bool neg_scale = a.scale_log2 < 0.f;
  const float sl2 = neg_scale ? -a.scale_log2 : a.scale_log2;
  const unsigned qflip = neg_scale ? 0x80008000u : 0u;

  // query heads as B operands: slice c holds dims 32c + 8kq .. +7 of head m
  h8 qf[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int64_t qo = ((int64_t)s * a.Hq + hq0 + m) * D + 32 * c + 8 * kq;
    const u32x4 raw = m < G && PA_IN_BOUNDS(kBsQuery, qo >= 0 && qo + 8 <= n_out)
                          ? *reinterpret_cast<const u32x4*>(a.q + qo)
                          : u32x4{0, 0, 0, 0};
    qf[c] = __builtin_bit_cast(h8, raw ^ qflip);
  }
  f4 o[8];
#pragma unroll
  for (int n = 0; n < 8; ++n) o[n] = f4{0.f, 0.f, 0.f, 0.f};
  float mrow = kNegBigG, lsum = 0.f;

  // K operand: token m, dims 32c + 8kq (c in the scalar offset)
  const unsigned k_off = (unsigned)(m * kRowBytesG + 16 * kq);
  // B = 8: rows 0-7 come from the unit's first block, rows 8-15 from its
  // second, through per-lane addresses (element offset inside the block)
  const int k_elt8 = (m & 7) * D + 8 * kq;
  // V into LDS: lane 16kq + m of row group i writes piece slot m of row
  // 4i + kq, so it loads the global piece the swizzle places there
  unsigned v_dma[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = 4 * i + kq;
    v_dma[i] = (unsigned)(r * kRowBytesG + ((m ^ ((r & 7) << 1)) << 4));
  }
  // transposing read of tile n: lane 4e + q of group kq reads row 4kq + e,
  // dims 16n + 4q .. +3
  const int te = (lane & 15) >> 2, tq = lane & 3;
  const int vr = 4 * kq + te;
  int v_rd[8];
#pragma unroll
  for (int n = 0; n < 8; ++n) {
    const int piece = 2 * n + (tq >> 1);
    v_rd[n] = vr * kRowBytesG + ((piece ^ ((vr & 7) << 1)) << 4) + (tq & 1) * 8;
  }
  const int wbase = wave * kTileBytesG;

  const int32_t* trow = a.tables + (int64_t)s * a.MB + blk0;
  for (int cb = 0; cb < nblk; cb += 64) {
    const int ce = cb + 64 < nblk ? cb + 64 : nblk;
    const int tbl = cb + lane < ce && PA_IN_BOUNDS(kBsTable, (int64_t)s * a.MB + blk0 + cb + lane <
                                                              (int64_t)a.S * a.MB)
                        ? trow[cb + lane]
                        : -1;
    const int ub0 = kSplit ? cb / 2 : (blk0 + cb) * UPB - U0;
    const int ue0 = kSplit ? (ce + 1) / 2 : (blk0 + ce) * UPB - U0;
    const int ub = ub0 > 0 ? ub0 : 0;
    const int ue = ue0 < nunits ? ue0 : nunits;
    auto locate = [&](int u) -> int64_t {
      const int au = U0 + u;
      const int bi = au / UPB;
      const int phys = __builtin_amdgcn_readlane(tbl, bi - blk0 - cb);
      const int safe = (unsigned)phys < (unsigned)a.NB ? phys : 0;
      return (((int64_t)safe * a.Hkv + g) * B + (au - bi * UPB) * U) * D;
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
    // K of unit u into ka, V into the wave's buffer of this stage; past the
    // wave's last unit the loads have an empty range (zeros, no memory read)
    auto fetch = [&](h8 (&ka)[4], int u, auto stage) {
      const bool live = u < ue;
      const int uu = live ? u : ue - 1;
      const int valid = len - uu * U;
      __amdgpu_buffer_rsrc_t rk, rv, rv1;
      if constexpr (kSplit) {
        const int64_t b0 = locate_half(uu, 0);
        const int64_t b1 = locate_half(uu, 1);
        const int v0 = valid < 8 ? valid : 8;
        const int v1 = valid - 8 < 0 ? 0 : (valid - 8 > 8 ? 8 : valid - 8);
        // each half tile (8 rows) inside the pool
        const bool in0 = PA_IN_BOUNDS(kBsPool, b0 >= 0 && b0 + 8 * D <= pool_elems);
        const bool in1 = PA_IN_BOUNDS(kBsPool, b1 >= 0 && b1 + 8 * D <= pool_elems);
        const int n0 = live && in0 ? v0 * kRowBytesG : 0;
        const int n1 = live && in1 ? v1 * kRowBytesG : 0;
        rv = __builtin_amdgcn_make_buffer_rsrc(const_cast<_Float16*>(a.v_pool + b0), 0, n0, kRsrcWord3G);
        rv1 = __builtin_amdgcn_make_buffer_rsrc(const_cast<_Float16*>(a.v_pool + b1), 0, n1, kRsrcWord3G);
        // K rows past the valid tokens are read from their (clamped, in-pool)
        // block but never used: their scores are masked by selection
        if (live && (m < 8 ? in0 : in1)) {
          const u32x4* kr = reinterpret_cast<const u32x4*>(a.k_pool + (m < 8 ? b0 : b1) + k_elt8);
#pragma unroll
          for (int c = 0; c < 4; ++c)
            ka[c] = __builtin_bit_cast(h8, NT ? __builtin_nontemporal_load(kr + 4 * c) : kr[4 * c]);
        } else {
#pragma unroll
          for (int c = 0; c < 4; ++c) ka[c] = h8{};
        }
      } else {
        const int64_t base = locate(uu);
        int nbytes = !live ? 0 : (valid >= U ? kTileBytesG : valid * kRowBytesG);
        // the unit's whole tile (16 rows) inside the pool
        if (!PA_IN_BOUNDS(kBsPool, base >= 0 && base + U * D <= pool_elems)) nbytes = 0;
        rk = __builtin_amdgcn_make_buffer_rsrc(const_cast<_Float16*>(a.k_pool + base), 0, nbytes, kRsrcWord3G);
        rv = __builtin_amdgcn_make_buffer_rsrc(const_cast<_Float16*>(a.v_pool + base), 0, nbytes, kRsrcWord3G);
        rv1 = rv;
#pragma unroll
        for (int c = 0; c < 4; ++c)
          ka[c] = __builtin_bit_cast(
              h8, __builtin_amdgcn_raw_buffer_load_b128(rk, k_off, 64 * c, NT ? 2 : 0));
      }
      // the wave last read this stage two units ago: its reads must have
      // returned before the buffer is refilled
      __builtin_amdgcn_sched_barrier(0);
      PA_G_WAIT_LDS();
      constexpr int st = decltype(stage)::value;
      lds_u8* vb = (st == 0 ? (lds_u8*)s_v0 : st == 1 ? (lds_u8*)s_v1 : (lds_u8*)s_v2) + wbase;
      // row groups 0-1 hold rows 0-7, groups 2-3 rows 8-15 (the second block at B = 8)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bool second = kSplit && i >= 2;
        const __amdgpu_buffer_rsrc_t r = second ? rv1 : rv;
        const unsigned off = second ? v_dma[i] - 8 * kRowBytesG : v_dma[i];
        if (NT) dma16_nt(r, vb + i * 1024, off);
        else dma16(r, vb + i * 1024, off);
      }
    };
    auto step = [&](const h8 (&ka)[4], int u, auto stage) {
      constexpr int st = decltype(stage)::value;
      const lds_u8* vb = (st == 0 ? (lds_u8*)s_v0 : st == 1 ? (lds_u8*)s_v1 : (lds_u8*)s_v2) + wbase;
      f4 sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < 4; ++c) sc = __builtin_amdgcn_mfma_f32_16x16x32_f16(ka[c], qf[c], sc, 0, 0, 0);
      const int valid = len - u * U;
      bool vis[4];
      float mx = kNegBigG;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        vis[r] = 4 * kq + r < valid;
        mx = __builtin_fmaxf(mx, vis[r] ? sc[r] : kNegBigG);
      }
      const float mloc = mx > 0.5f * kNegBigG ? mx * sl2 : kNegBigG;
      if (__builtin_amdgcn_ballot_w64(mloc > mrow + kSlackG)) {
        mx = __builtin_fmaxf(mx, __shfl_xor(mx, 16));
        mx = __builtin_fmaxf(mx, __shfl_xor(mx, 32));
        const float mcand = mx > 0.5f * kNegBigG ? mx * sl2 : kNegBigG;
        const float mnew = __builtin_fmaxf(mrow, mcand);
        const float alpha = __builtin_amdgcn_exp2f(mrow - mnew);
        mrow = mnew;
        lsum *= alpha;
#pragma unroll
        for (int n = 0; n < 8; ++n) o[n] *= alpha;
      }
      h4 pb;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float pr = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[r], sl2, -mrow));
        pr = vis[r] ? pr : 0.f;
        lsum += pr;
        pb[r] = (_Float16)pr;
      }
#pragma unroll
      for (int n = 0; n < 8; ++n) {
        const s4 raw = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4*)(vb + v_rd[n]));
        o[n] = __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(h4, raw), pb, o[n], 0, 0, 0);
      }
    };
    int u = ub + wave;
    if (u >= ue) continue;
    if constexpr (DEPTH == 1) {
      h8 k0[4], k1[4];
      fetch(k0, u, Stage<0>{});
      while (true) {
        int un = u + NW;
        fetch(k1, un, Stage<1>{});
        step(k0, u, Stage<0>{});
        if (un >= ue) break;
        u = un;
        un = u + NW;
        fetch(k0, un, Stage<0>{});
        step(k1, u, Stage<1>{});
        if (un >= ue) break;
        u = un;
      }
    } else {
      // unit j of the wave uses register set and stage j % 3
      h8 k0[4], k1[4], k2[4];
      fetch(k0, u, Stage<0>{});
      fetch(k1, u + NW, Stage<1>{});
      while (true) {
        fetch(k2, u + 2 * NW, Stage<2>{});
        step(k0, u, Stage<0>{});
        u += NW;
        if (u >= ue) break;
        fetch(k0, u + 2 * NW, Stage<0>{});
        step(k1, u, Stage<1>{});
        u += NW;
        if (u >= ue) break;
        fetch(k1, u + 2 * NW, Stage<1>{});
        step(k2, u, Stage<2>{});
        u += NW;
        if (u >= ue) break;
      }
    }
    // the last fetch was a no-op into a stage: let it land before the next
    // chunk's first load writes that stage
    PA_G_WAIT_VM0();
  }
  PA_G_WAIT_VM0();   // no load into LDS outlives the wave

  // the four lanes of a head hold its sum in parts and the same maximum; the
  // wave's accumulators go to its own tile of stage 0, which no other wave
  // touches (its loads into LDS have landed, its reads have returned)
  float lt = lsum + __shfl_xor(lsum, 16);
  lt += __shfl_xor(lt, 32);
  PA_G_WAIT_LDS();
  float* acc_w = reinterpret_cast<float*>(s_v0 + wbase);
  if (m < G) {
    if (kq == 0) {
      s_ml[wave][m][0] = mrow;
      s_ml[wave][m][1] = lt;
    }
#pragma unroll
    for (int n = 0; n < 8; ++n) {
#pragma unroll
      for (int r = 0; r < 4; ++r) acc_w[m * D + 16 * n + 4 * kq + r] = o[n][r];
    }
  }
  __syncthreads();

  // combine the waves: thread e handles output element (head h, dim d)
  for (int e = threadIdx.x; e < G * D; e += NW * 64) {
    const int h = e / D;
    const int d = e % D;
    float mx = s_ml[0][h][0];
#pragma unroll
    for (int w = 1; w < NW; ++w) mx = __builtin_fmaxf(mx, s_ml[w][h][0]);
    float den = 0.f, num = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float f = __builtin_amdgcn_exp2f(s_ml[w][h][0] - mx);
      den += f * s_ml[w][h][1];
      num += f * reinterpret_cast<const float*>(s_v0 + w * kTileBytesG)[h * D + d];
    }
    const int hq = hq0 + h;
    if (nparts == 1) {
      const float ov = den > 0.f ? num / den : 0.f;
      const int64_t oi = ((int64_t)s * a.Hq + hq) * D + d;
      if (PA_IN_BOUNDS(kBsOut, oi >= 0 && oi < n_out)) a.out[oi] = (_Float16)ov;
    } else {
      const int64_t row = ((int64_t)s * a.Hq + hq) * a.Pmax + p;
      if (PA_IN_BOUNDS(kBsPartial, p >= 0 && p < a.Pmax && row < (int64_t)a.S * a.Hq * a.Pmax)) {
        reinterpret_cast<_Float16*>(a.part_acc)[row * D + d] = (_Float16)(den > 0.f ? num / den : 0.f);
        if (d == 0) {
          a.part_ml[row * 2] = mx;
          a.part_ml[row * 2 + 1] = den;
        }
      }
    }
  }
}

// Clamped context length of sequence s: within the table and the launch.
__device__ __forceinline__ int clamped_len(const DecodeArgs& a, int s, int B, int cap) {
  int L = PA_IN_BOUNDS(kBsLength, s >= 0 && s < a.S) ? a.lens[s] : 0;
  L = L < 0 ? 0 : L;
  L = L > a.MB * B ? a.MB * B : L;
  return L > cap ? cap : L;
}

// Zero output of every query head of KV head g of sequence s (empty sequence).
template <int G, int NW>
__device__ __forceinline__ void zero_heads(const DecodeArgs& a, int s, int g) {
  for (int e = threadIdx.x; e < G * kHeadDim; e += NW * 64) {
    const int64_t oi = ((int64_t)s * a.Hq + g * G + e / kHeadDim) * kHeadDim + (e % kHeadDim);
    if (PA_IN_BOUNDS(kBsOut, oi >= 0 && oi < (int64_t)a.S * a.Hq * kHeadDim)) a.out[oi] = (_Float16)0.f;
  }
}

// One workgroup per (partition, sequence, KV head), partitions of a.P tokens.
template <int BT, int G, int NW, int DEPTH, bool NT>
__global__ __launch_bounds__(NW * 64) void decode_mfma_kernel(const DecodeArgs a) {
  const int B = BT > 0 ? BT : a.B;
  int id = blockIdx.x;
  const int g = id % a.Hkv;
  id /= a.Hkv;
  const int s = id % a.S;
  const int p = id / a.S;
  const int L = clamped_len(a, s, B, a.Pmax * a.P);
  const int tok0 = p * a.P;
  if (tok0 >= L) {
    if (p == 0) zero_heads<G, NW>(a, s, g);
    return;
  }
  const int nparts = (L + a.P - 1) / a.P;
  const int len = (tok0 + a.P < L ? tok0 + a.P : L) - tok0;
  attend_piece<BT, G, NW, DEPTH, NT>(a, s, g, tok0, len, nparts, p);
}

// Equal-work split of the whole batch (the walk and its reasons are in
// decode_even.h). Four waves per SIMD are asked for explicitly: left to itself
// the compiler keeps the walk's state in 151 VGPRs and three waves per SIMD;
// at 127 it needs no spills.
template <int BT, int G, int NW, int DEPTH, bool NT>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(4, 4)))
void decode_mfma_even_kernel(const DecodeArgs a) {
  even_split_walk<NW * 64>(
      a, BT > 0 ? BT : a.B,
      [&](int s, int g, int /*L*/, int tok0, int len, int nparts, int p) {
        attend_piece<BT, G, NW, DEPTH, NT>(a, s, g, tok0, len, nparts, p);
      },
      [&](int s) {
        for (int g = 0; g < a.Hkv; ++g) zero_heads<G, NW>(a, s, g);
      });
}

template <int BT, int G>
hipError_t launch_bt(const DecodeArgs& a, hipStream_t stream) {
  constexpr int NW = PA_MFMA_WAVES;
  if (a.part_np) {
    auto kernel = decode_mfma_even_kernel<BT, G, NW, PA_MFMA_DEPTH, kDecodeNontemporal>;
    // two workgroups per CU: 0.7 % faster for groups of 8 on the chat lengths
    // than the four resident ones, groups of 4 within noise
    const int64_t grid = even_split_grid(a, kernel, NW * 64, 2);
    if (grid <= 0) return hipErrorInvalidValue;
    kernel<<<(unsigned)grid, NW * 64, 0, stream>>>(a);
    return hipGetLastError();
  }
  const int64_t grid = (int64_t)a.Pmax * a.S * a.Hkv;
  decode_mfma_kernel<BT, G, NW, PA_MFMA_DEPTH, kDecodeNontemporal>
      <<<(unsigned)grid, NW * 64, 0, stream>>>(a);
  return hipGetLastError();
}

template <int G>
hipError_t launch_g(const DecodeArgs& a, int B, hipStream_t stream) {
  switch (B) {
    case 8: return launch_bt<8, G>(a, stream);
    case 16: return launch_bt<16, G>(a, stream);
    case 32: return launch_bt<32, G>(a, stream);
    default: return launch_bt<0, G>(a, stream);
  }
}

}  // namespace

PA_BOUNDS_COLLECTOR(bounds_take_decode_mfma)

hipError_t launch_decode_mfma(const DecodeArgs& a, int B, int G, hipStream_t stream) {
  switch (G) {
    case 4: return launch_g<4>(a, B, stream);
    case 8: return launch_g<8>(a, B, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pa
