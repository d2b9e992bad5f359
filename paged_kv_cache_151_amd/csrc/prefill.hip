// Paged prefill attention for gfx950: many new query tokens per sequence,
// causal, keys and values read through the block table, dense tiles on MFMA.
//
// [L] "Paged Attention: OS-Inspired Memory Management for KV Caches",
//     "How PagedAttention works", step 1 (the prompt is stored in the blocks
//     the manager hands out) and step 4 (attention walks the table as if the
//     tokens were contiguous); "Memory sharing across requests" (a prompt may
//     start with blocks that other requests already filled).
//
// Problem. Sequence s has L tokens in the cache, the last n of them new (rows
// query_start[s] .. query_start[s+1]-1 of the packed query). New token j sits
// at position L - n + j and attends over positions 0 .. L - n + j.
//
// Work decomposition. A wave owns 16 * QT query rows of one query head. A
// workgroup is NW waves over one KV head g: NW query heads of g with the same
// rows when the group has at least NW heads, otherwise NW / G row tiles of
// each of the G heads. Keys and values are taken KC tokens at a time (a chunk
// of KC / 16 units, each a contiguous 4 KiB tile of the pool per KV head). The
// workgroup loads each chunk once, two chunks ahead of the one being computed,
// with buffer loads that write straight into LDS (no staging registers, no
// separate store step), into one of three LDS stages; the waves read their
// matrix operands from there. Defaults (QT = 2, NW = 4, KC = 32, three LDS
// stages) are set in prefill_internal.h.
//
// Instruction budget. A wave issues at most one instruction per turn on its
// SIMD, so every scalar or vector instruction around the 16 matrix products of
// a 32-key step costs issue slots the products need. Each wave loads one pool
// (K or V) of half the units of every chunk, with per-lane offsets that never
// change: per chunk it computes those units' base addresses and valid lengths. The
// block table is read with a vector load (scalar loads share their wait
// counter with LDS reads, so every operand wait would also wait for them),
// and chunks that every row of the workgroup sees in full run through a loop
// with a single code path (no masking, no per-wave skip, no join that makes
// the compiler copy the accumulators).
//
// Matrix products (v_mfma_f32_16x16x32_f16; lane l = 16 kq + m):
//   scores   S^T = K Q^T per unit: the A operand is key token m, dims
//            32c + 8kq .. +7 (one 16-byte LDS read), the B operand the query
//            rows held in registers; lane l receives S for query row m and
//            tokens 4kq + r of the unit.
//   output   O^T = V^T P^T per 32 keys: the B operand is P exactly as the score
//            product left it (query m; tokens 4kq + r of two units), the A
//            operand V for the same 8 tokens at dim 16n + m, gathered from the
//            row-major V tile by two transposing LDS reads (ds_read_b64_tr_b16:
//            in each 16-lane group, lane i receives 16-bit word i % 4 from the
//            address of lane 4e + i / 4 as its element e). Lane l ends with
//            O[row m][dims 16n + 4kq + r].
// Every per-row softmax quantity (running max, sum, rescale factor) lives in
// the lanes of that row, so the only cross-lane steps are the row-max
// exchanges when a row's running maximum must be raised (rare) and the final
// sum.
//
// LDS layout: a chunk is KC token rows of 256 bytes for K and for V, each row
// split into 16 pieces of 16 bytes. Piece c of row r is stored at position
// c ^ (r % 16) for K and c ^ 2 (r % 8) for V, which spreads the operand reads
// of a wave over all banks.
//
// Masking: keys and values past the sequence's L tokens are fetched as zeros
// by the buffer range check (so NaN or Inf in unused slots never enters a
// product); causal exclusions select the score to "no token" and p to 0.
#include "pa_debug.h"
#include "prefill_internal.h"

namespace pa {
namespace {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef short s4 __attribute__((ext_vector_type(4)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

constexpr float kNegBig = -1.0e30f;
// Lazy rescaling slack in log2 units: softmax weights stay at most 2^kSlack.
#ifndef PA_PREFILL_SLACK
#define PA_PREFILL_SLACK 8.0f
#endif
constexpr float kSlack = PA_PREFILL_SLACK;
constexpr int kUnitTok = 16;
constexpr int kRowBytes = kHeadDim * 2;    // one token row of one KV head
constexpr int kRsrcWord3 = 0x00020000;     // raw buffer, gfx9 family


typedef __attribute__((address_space(3))) unsigned char lds_u8;
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
typedef __attribute__((address_space(3))) s4 lds_s4;

// byte offset of 16-byte piece c of token row r in a K (or V) stage
__device__ __forceinline__ int k_pos(int r, int c) { return r * kRowBytes + ((c ^ (r & 15)) << 4); }
__device__ __forceinline__ int v_pos(int r, int c) {
  return r * kRowBytes + ((c ^ ((r & 7) << 1)) << 4);
}

template <bool V>
struct Flag {
  static constexpr bool value = V;
};

template <int S>
struct Stage {
  static constexpr int value = S;
};

// 16-byte buffer load of each lane into LDS: lane i's bytes land at dst + 16 i
// (lanes past the resource's range write zeros). Plain cache policy: the row
// blocks of one sequence and KV head read the same chunks side by side on one
// XCD, and its L2 serves the repeats (the non-temporal hint measured 3 %
// slower). Kept out of the kernel template: the host pass must not see the
// LDS pointer argument inside it.
__device__ __forceinline__ void load_lds16(__amdgpu_buffer_rsrc_t r, lds_u8* dst, unsigned voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)dst, 16, voff,
                                           0, 0, 0);
}

// vmcnt(n): wait until at most n vector memory operations of this wave are
// outstanding (gfx9 encoding; lgkmcnt and expcnt left at their maximum).
#define PA_WAIT_VM(n) __builtin_amdgcn_s_waitcnt(((n) & 15) | (((n) >> 4) << 14) | 0x0F70)
// lgkmcnt(0): every LDS read this wave issued has returned its data (vmcnt and
// expcnt left at their maximum).
#define PA_WAIT_LDS() __builtin_amdgcn_s_waitcnt(0xC07F)

// Three waves per SIMD with one row tile (at most 168 VGPRs; it fits in about
// 150); two row tiles fit in about 235 VGPRs, two waves per SIMD.
template <int BT, int G, int QT, int NW, int KC, int NST>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(QT == 1 ? 3 : 2)))
void prefill_kernel(const PrefillArgs a) {
  constexpr int D = kHeadDim;
  constexpr int HW = G < NW ? G : NW;      // query heads in a workgroup
  constexpr int RW = NW / HW;              // row tiles per head in a workgroup
  constexpr int QR = 16 * QT;              // query rows per wave
  constexpr int QB = RW * QR;              // query rows per workgroup
  constexpr int NHG = G / HW;              // workgroups per KV head and row block
  constexpr int NTH = NW * 64;             // threads
  constexpr int NU = KC / kUnitTok;        // 16-token units per chunk
  constexpr int NKS = KC / 32;             // 32-token steps of the value product
  constexpr int NPC = 32 * KC;             // 16-byte pieces per chunk (K and V)
  constexpr int NP = NPC / NTH;            // pieces per thread and chunk
  constexpr int kStageBytes = KC * kRowBytes;
  static_assert(G == 1 || G == 2 || G == 4 || G == 8, "group size");
  static_assert(NW == 4, "the load layout assumes four waves");
  static_assert(KC == 32 || KC == 64, "keys per step");
  static_assert(NP * NTH == NPC, "whole load instructions per chunk");
  static_assert(NST == 3 || NST == 4, "three or four LDS stages");
  // One array per stage, always indexed at compile time: the compiler tracks
  // loads into LDS per array and waits only where a read meets its stage.
  __shared__ __attribute__((aligned(16))) unsigned char s_k0[kStageBytes];
  __shared__ __attribute__((aligned(16))) unsigned char s_v0[kStageBytes];
  __shared__ __attribute__((aligned(16))) unsigned char s_k1[kStageBytes];
  __shared__ __attribute__((aligned(16))) unsigned char s_v1[kStageBytes];
  __shared__ __attribute__((aligned(16))) unsigned char s_k2[kStageBytes];
  __shared__ __attribute__((aligned(16))) unsigned char s_v2[kStageBytes];
  __shared__ __attribute__((aligned(16))) unsigned char s_k3[NST == 4 ? kStageBytes : 16];
  __shared__ __attribute__((aligned(16))) unsigned char s_v3[NST == 4 ? kStageBytes : 16];
  auto kst = [&](int st) -> lds_u8* {
    return st == 0 ? (lds_u8*)s_k0 : st == 1 ? (lds_u8*)s_k1 : st == 2 ? (lds_u8*)s_k2 : (lds_u8*)s_k3;
  };
  auto vst = [&](int st) -> lds_u8* {
    return st == 0 ? (lds_u8*)s_v0 : st == 1 ? (lds_u8*)s_v1 : st == 2 ? (lds_u8*)s_v2 : (lds_u8*)s_v3;
  };
  const int B = BT > 0 ? BT : a.B;
  // B = 8: a 16-token unit spans two blocks (two half tiles of 2 KiB), so it
  // takes two table entries and two buffer resources.
  constexpr bool kSplit = BT == 8;
  constexpr int NE = kSplit ? 2 : 1;       // table entries per unit
  const int UPB = kSplit ? 1 : B / kUnitTok;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int m = lane & 15;
  const int kq = lane >> 4;

  // Work order. Workgroups are dealt to the 8 XCDs round-robin by blockIdx,
  // so XCD x runs work items x * per_xcd, x * per_xcd + 1, ... in order. The
  // list is ordered (g, s, hg, rank) with the row-block rank fastest: the
  // row blocks of one (sequence, KV head) run side by side on one XCD and
  // read its keys and values from that XCD's L2, and each XCD gets a
  // contiguous range of KV heads across all sequences (balanced when Hkv is
  // a multiple of 8). Rank 0 is a sequence's last row block (the most keys).
  const int64_t bid = blockIdx.x;
  int64_t id = (bid % 8) * a.per_xcd + bid / 8;
  if (id >= a.n_work) return;
  const int rank = (int)(id % a.n_rank);
  id /= a.n_rank;
  const int hg = (int)(id % NHG);
  id /= NHG;
  const int s = (int)(id % a.S);
  const int g = (int)(id / a.S);

  const bool s_ok = PA_IN_BOUNDS(kBsLength, s >= 0 && s < a.S);
  const int qs0 = s_ok ? a.qstart[s] : 0;
  const int qs1 = s_ok ? a.qstart[s + 1] : 0;
  if (qs0 < 0 || qs1 > a.T || qs1 <= qs0) return;
  const int n = qs1 - qs0;
  const int nqb = (n + QB - 1) / QB;
  if (rank >= nqb) return;                 // whole workgroup, before any barrier
  const int qb = nqb - 1 - rank;
  int L = s_ok ? a.lens[s] : 0;
  L = L < 0 ? 0 : L;
  L = L > a.MB * B ? a.MB * B : L;
  const int base_pos = L - n;
  const int64_t n_rows = (int64_t)a.T * a.Hq * D;            // elements of the query and out
  const int64_t pool_bytes = (int64_t)a.NB * a.Hkv * B * kRowBytes;
  (void)n_rows;
  (void)pool_bytes;              // row j sits at position base_pos + j

  // keys the workgroup walks: [0, kend_wg), as far as its last row sees
  const int jl_wg = (qb * QB + QB < n ? qb * QB + QB : n) - 1;
  int kend_wg = base_pos + jl_wg + 1;
  kend_wg = kend_wg > L ? L : kend_wg;
  kend_wg = kend_wg < 0 ? 0 : kend_wg;
  const int nchunk_wg = (kend_wg + KC - 1) / KC;
  const int nblk = (kend_wg + B - 1) / B;
  // Chunks that every row of the workgroup sees in full (keys before the
  // position of its first row), rounded down to whole turns of the stages:
  // these run through a loop with a single code path.
  int nall = base_pos + qb * QB + 1 > 0 ? (base_pos + qb * QB + 1) / KC : 0;
  nall = nall > nchunk_wg ? nchunk_wg : nall;
  const int nfast = nall - nall % NST;

  // this wave's rows and the chunks it computes
  const int hq = g * G + hg * HW + wave % HW;
  const int j0 = qb * QB + (wave / HW) * QR;
  const bool wave_rows = j0 < n;
  const int jl = (j0 + QR < n ? j0 + QR : n) - 1;
  int kend = base_pos + jl + 1;
  kend = kend > L ? L : kend;
  kend = kend < 0 ? 0 : kend;
  const int nchunk = wave_rows ? (kend + KC - 1) / KC : 0;

  // The lazy maximum below is taken on unscaled scores, which keeps their
  // order only for a scale >= 0. A negative scale is applied as |scale| to the
  // negated queries instead: flipping the fp16 sign bits is exact, so every
  // score changes sign exactly and scale * score is unchanged.
  const bool neg_scale = a.scale_log2 < 0.f;
  const float sl2 = neg_scale ? -a.scale_log2 : a.scale_log2;
  const unsigned qflip = neg_scale ? 0x80008000u : 0u;

  // query rows as B operands
  h8 qf[QT][4];
  int pos[QT];
#pragma unroll
  for (int t = 0; t < QT; ++t) {
    const int j = j0 + 16 * t + m;
    const bool ok = j < n;
    pos[t] = base_pos + j;
    const int64_t qo = ((int64_t)(qs0 + (ok ? j : 0)) * a.Hq + hq) * D + 8 * kq;
    const _Float16* qrow = a.q + qo;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const u32x4 raw = ok && PA_IN_BOUNDS(kBsQuery, qo >= 0 && qo + 32 * c + 8 <= n_rows)
                            ? *reinterpret_cast<const u32x4*>(qrow + 32 * c)
                            : u32x4{0, 0, 0, 0};
      qf[t][c] = __builtin_bit_cast(h8, raw ^ qflip);
    }
  }

  float mrow[QT], lsum[QT];
  f4 o[QT][8];
#pragma unroll
  for (int t = 0; t < QT; ++t) {
    mrow[t] = kNegBig;
    lsum[t] = 0.f;
#pragma unroll
    for (int nn = 0; nn < 8; ++nn) o[t][nn] = f4{0.f, 0.f, 0.f, 0.f};
  }

  // Physical blocks come from the table by a vector load per chunk (lane u
  // reads unit u's entry, range-checked to the workgroup's nblk entries; no
  // LDS wait ever waits for a table read, as it would for scalar loads, which
  // share the LDS counter). Each chunk's entries are loaded a whole turn of
  // the pipeline before its chunk loads, into one of NST registers, so that
  // the wait for a chunk's data always covers them. Entries outside the pool
  // are clamped to block 0.
  const bool table_ok = PA_IN_BOUNDS(kBsTable, nblk <= a.MB);
  const __amdgpu_buffer_rsrc_t trs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<int32_t*>(a.tables + (int64_t)s * a.MB), 0, table_ok ? nblk * 4 : 0, kRsrcWord3);
  auto table_load = [&](int chunk) -> int {
    if constexpr (kSplit) {   // lane 2u + h reads the block of half h of unit u
      const int e = 2 * NU * chunk + (lane < 2 * NU ? lane : 0);
      return __builtin_amdgcn_raw_buffer_load_b32(trs, (unsigned)e * 4u, 0, 0);
    }
    const int U = NU * chunk + (lane < NU ? lane : 0);
    return __builtin_amdgcn_raw_buffer_load_b32(trs, (unsigned)(U / UPB) * 4u, 0, 0);
  };

  // Loads into LDS. Wave w loads pool w / 2 (K, then V) of each chunk, units
  // (w % 2) * NU / 2 .. + NU / 2 - 1, four row groups (4 token rows) per
  // unit: one buffer resource per unit and wave. Lane 16 kq + m of row group
  // i writes LDS piece slot m of row r = 4i + kq of the unit, so it loads the
  // global piece that the swizzle places there (m ^ swizzle(r)): four fixed
  // offsets into a unit for the whole kernel. Lanes past a unit's valid
  // tokens fall outside the resource's range and write zeros.
  static_assert(NW == 4 && NU % 2 == 0, "one pool and half the units per wave");
  constexpr int UW = NU / 2;                      // units per wave and chunk
  const bool w_is_v = wave >= 2;
  const int w_u0 = (wave & 1) * UW;
  unsigned voff[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = 4 * i + kq;
    const int piece = w_is_v ? (m ^ ((r & 7) << 1)) : (m ^ (r & 15));
    voff[i] = (unsigned)(r * kRowBytes + (piece << 4));
  }
  const uint32_t blk_bytes = (uint32_t)a.Hkv * (uint32_t)B * kRowBytes;   // one block, all heads
  const unsigned char* pg = (const unsigned char*)(w_is_v ? a.v_pool : a.k_pool) + (size_t)g * B * kRowBytes;
  const int w_lds = w_u0 * kUnitTok * kRowBytes;
  auto load_chunk = [&](int c, int st, const int (&ph)[NE * NU]) {
#pragma unroll
    for (int j = 0; j < UW; ++j) {
      const int U = NU * c + w_u0 + j;
      // one resource and offset per row group (rows 4i .. 4i + 3 of the unit)
      __amdgpu_buffer_rsrc_t rs[4];
      unsigned vo[4];
      if constexpr (kSplit) {
        // half h holds unit tokens 8h .. 8h + 7: row groups 2h and 2h + 1
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int t0 = U * kUnitTok + 8 * h;
          const int valid = L - t0 < 8 ? L - t0 : 8;
          int nbytes = t0 < kend_wg ? valid * kRowBytes : 0;
          const int phys = ph[2 * (w_u0 + j) + h];
          const uint32_t safe = (unsigned)phys < (unsigned)a.NB ? (uint32_t)phys : 0u;
          // the half tile (8 rows) inside the pool
          if (!PA_IN_BOUNDS(kBsPool, (int64_t)g * B * kRowBytes + (int64_t)safe * blk_bytes +
                                             8 * kRowBytes <= pool_bytes))
            nbytes = 0;
          const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
              const_cast<unsigned char*>(pg + (uint64_t)safe * blk_bytes), 0, nbytes, kRsrcWord3);
          rs[2 * h] = r;
          rs[2 * h + 1] = r;
          vo[2 * h] = voff[2 * h] - h * 8 * kRowBytes;
          vo[2 * h + 1] = voff[2 * h + 1] - h * 8 * kRowBytes;
        }
      } else {
        const int valid = L - U * kUnitTok < kUnitTok ? L - U * kUnitTok : kUnitTok;
        int nbytes = U * kUnitTok < kend_wg ? valid * kRowBytes : 0;
        const int phys = ph[w_u0 + j];
        const uint32_t safe = (unsigned)phys < (unsigned)a.NB ? (uint32_t)phys : 0u;
        const uint64_t off = (uint64_t)safe * blk_bytes + (uint32_t)((U % UPB) * kUnitTok * kRowBytes);
        // the unit's whole tile (16 rows) inside the pool
        if (!PA_IN_BOUNDS(kBsPool, (int64_t)g * B * kRowBytes + (int64_t)off + kUnitTok * kRowBytes <=
                                       pool_bytes))
          nbytes = 0;
        const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<unsigned char*>(pg + off), 0, nbytes, kRsrcWord3);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          rs[i] = r;
          vo[i] = voff[i];
        }
      }
      // The branch is uniform; each side names its LDS array at compile time.
      // (With the array chosen at run time the compiler cannot tell which
      // stage a load writes and waits for every load before any LDS read.)
      if (w_is_v) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          lds_u8* dst = vst(st) + w_lds + (j * kUnitTok + 4 * i) * kRowBytes;
          load_lds16(rs[i], dst, vo[i]);
        }
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          lds_u8* dst = kst(st) + w_lds + (j * kUnitTok + 4 * i) * kRowBytes;
          load_lds16(rs[i], dst, vo[i]);
        }
      }
    }
  };

  // Operand reads, per lane:
  //   K, unit u, dim block cc: row 16u + m, piece 4cc + kq;
  //   V, product nn: rows 4kq + m/4 (unit 0) and 16 + 4kq + m/4 (unit 1),
  //   dims 16nn + 4 (m % 4) .. +3, i.e. half (m % 2) of piece 2nn + (m % 4) / 2.
  const int v_row = 4 * kq + (m >> 2);
  auto compute = [&](int st, int c, auto masked_flag) {
    constexpr bool masked = decltype(masked_flag)::value;
    const lds_u8* kb = kst(st);
    const lds_u8* vb = vst(st);
    h8 ka[NU][4];
#pragma unroll
    for (int u = 0; u < NU; ++u) {
#pragma unroll
      for (int cc = 0; cc < 4; ++cc)
        ka[u][cc] = __builtin_bit_cast(h8, *(const lds_u32x4*)(kb + k_pos(16 * u + m, 4 * cc + kq)));
    }
    h8 va[NKS][8];
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
#pragma unroll
      for (int nn = 0; nn < 8; ++nn) {
        const int off = v_pos(32 * ks + v_row, 2 * nn + ((m & 3) >> 1)) + (m & 1) * 8;
        const s4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4*)(vb + off));
        const s4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4*)(vb + off + 16 * kRowBytes));
        const u32x2 l2 = __builtin_bit_cast(u32x2, lo);
        const u32x2 h2 = __builtin_bit_cast(u32x2, hi);
        va[ks][nn] = __builtin_bit_cast(h8, u32x4{l2.x, l2.y, h2.x, h2.y});
      }
    }
#pragma unroll
    for (int t = 0; t < QT; ++t) {
      f4 sc[NU];
#pragma unroll
      for (int u = 0; u < NU; ++u) {
        f4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int cc = 0; cc < 4; ++cc)
          acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(ka[u][cc], qf[t][cc], acc, 0, 0, 0);
        sc[u] = acc;
      }
      // Raw scores; the maximum is taken before scaling (sl2 >= 0, so the
      // order is kept) and p = 2^(sl2 * s - m) is one fused multiply-add and
      // one exp2 per score.
      float x[4 * NU];
      bool vis[4 * NU];
      float mx = kNegBig;
#pragma unroll
      for (int j = 0; j < 4 * NU; ++j) {
        const float v = sc[j / 4][j % 4];
        vis[j] = !masked || c * KC + 16 * (j / 4) + 4 * kq + (j % 4) <= pos[t];
        x[j] = v;
        mx = __builtin_fmaxf(mx, vis[j] ? v : kNegBig);
      }
      // Running maximum m (log2 domain, scaled). Lazy rescaling: m is raised,
      // and the accumulators rescaled, only when some row of the wave would
      // otherwise see p above 2^kSlack; until then p <= 2^kSlack, well inside
      // fp16's range. The result is the same softmax: the final division uses
      // the same m for numerator and denominator. A row's maximum exceeds the
      // bound exactly when one of its lanes' maxima does, so the decision is
      // taken on each lane's own maximum; the row maxima are exchanged across
      // lanes only when some row must be raised.
      const float mloc = mx > 0.5f * kNegBig ? mx * sl2 : kNegBig;
      if (__builtin_amdgcn_ballot_w64(mloc > mrow[t] + kSlack)) {
        mx = __builtin_fmaxf(mx, __shfl_xor(mx, 16));
        mx = __builtin_fmaxf(mx, __shfl_xor(mx, 32));
        const float mcand = mx > 0.5f * kNegBig ? mx * sl2 : kNegBig;
        const float mnew = __builtin_fmaxf(mrow[t], mcand);
        const float alpha = __builtin_amdgcn_exp2f(mrow[t] - mnew);
        mrow[t] = mnew;
        lsum[t] *= alpha;
#pragma unroll
        for (int nn = 0; nn < 8; ++nn) o[t][nn] *= alpha;
      }
      float ls = lsum[t];
      h8 pb[NKS];
#pragma unroll
      for (int j = 0; j < 4 * NU; ++j) {
        float p = __builtin_amdgcn_exp2f(__builtin_fmaf(x[j], sl2, -mrow[t]));
        p = vis[j] ? p : 0.f;
        ls += p;
        pb[j / 8][j % 8] = (_Float16)p;
      }
      lsum[t] = ls;
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
#pragma unroll
        for (int nn = 0; nn < 8; ++nn)
          o[t][nn] = __builtin_amdgcn_mfma_f32_16x16x32_f16(va[ks][nn], pb[ks], o[t][nn], 0, 0, 0);
      }
    }
  };

  // Pipeline over NST LDS stages: chunk k goes to stage k % NST. Iteration
  // c: wait until this wave's LDS reads have returned their data and its
  // loads of chunk c are done (the loads of chunks c + 1 .. c + NST - 2 may
  // still be in flight), barrier (every wave's part of chunk c is in LDS, and
  // no wave still reads the stage of chunk c - 1), read chunk c + NST - 1's
  // entries, start the table read for chunk c + 2 NST - 1 and the loads of
  // chunk c + NST - 1 into the stage chunk c - 1 used, compute chunk c.
  // The LDS wait is explicit: the barrier instruction does not wait for
  // outstanding reads, and the compiler is free to schedule the value products
  // of chunk c - 1, with the waits for their operand reads, below the barrier;
  // the scheduling fence keeps those reads above the wait. Without it a wave
  // could still be reading a stage when another wave's loads refill it.
  // Both loops are unrolled NST times so that every stage index is a
  // compile-time constant. The first runs the chunks every row sees in full
  // (all waves, no mask); the second the rest, where a wave masks the keys
  // beyond its rows (one masked code path: a second, unmasked copy there
  // costs the registers of a third wave per SIMD) and skips chunks past them.
  // Every wave runs the same iterations (barriers). Past the last chunk the
  // loads have an empty range: no memory is read, the stage is filled with
  // zeros.
  if (nchunk_wg > 0) {
    int ph[NE * NU];
    int tvr[NST];   // table entries of chunk x live in tvr[x % NST]
    auto entries = [&](int tv) {
#pragma unroll
      for (int u = 0; u < NE * NU; ++u) ph[u] = __builtin_amdgcn_readlane(tv, u);
    };
    // The explicit wait at the top of each iteration counts loads in issue
    // order, so the scheduling fences keep that order: table reads of chunks
    // 0 .. NST - 1, then per chunk x < NST - 1 the table read of chunk
    // x + NST and the loads of chunk x.
#pragma unroll
    for (int x = 0; x < NST; ++x) tvr[x] = table_load(x);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int x = 0; x + 1 < NST; ++x) {
      entries(tvr[x]);
      tvr[x] = table_load(x + NST);
      __builtin_amdgcn_sched_barrier(0);
      load_chunk(x, x, ph);
      __builtin_amdgcn_sched_barrier(0);
    }
    // Iteration c (stage st = c % NST). Issue order per iteration: the table
    // read of chunk c + 2 NST - 1, then the loads of chunk c + NST - 1. At the
    // top, the loads issued after chunk c's are NST - 2 such pairs.
    auto turn = [&](int c, auto st_flag, auto masked_flag) {
      constexpr int st = decltype(st_flag)::value;
      constexpr int nx = (st + NST - 1) % NST;
      __builtin_amdgcn_sched_barrier(0);
      PA_WAIT_LDS();
      PA_WAIT_VM((NST - 2) * (NP + 1));
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_sched_barrier(0);
      entries(tvr[nx]);
      tvr[nx] = table_load(c + 2 * NST - 1);
      __builtin_amdgcn_sched_barrier(0);
      load_chunk(c + NST - 1, nx, ph);
      if constexpr (decltype(masked_flag)::value) {
        if (c < nchunk) compute(st, c, Flag<true>{});
      } else {
        compute(st, c, Flag<false>{});   // every row sees chunk c in full
      }
    };
    int c = 0;
    for (; c < nfast; c += NST) {
      turn(c, Stage<0>{}, Flag<false>{});
      turn(c + 1, Stage<1>{}, Flag<false>{});
      turn(c + 2, Stage<2>{}, Flag<false>{});
      if constexpr (NST == 4) turn(c + 3, Stage<3>{}, Flag<false>{});
    }
    while (c < nchunk_wg) {
      turn(c, Stage<0>{}, Flag<true>{});
      if (++c >= nchunk_wg) break;
      turn(c, Stage<1>{}, Flag<true>{});
      if (++c >= nchunk_wg) break;
      turn(c, Stage<2>{}, Flag<true>{});
      if (++c >= nchunk_wg) break;
      if constexpr (NST == 4) {
        turn(c, Stage<3>{}, Flag<true>{});
        if (++c >= nchunk_wg) break;
      }
    }
    PA_WAIT_VM(0);   // no load into LDS outlives the workgroup
  }

  // normalise and store: lane holds row m, dims 16nn + 4kq + r
#pragma unroll
  for (int t = 0; t < QT; ++t) {
    float lt = lsum[t];
    lt += __shfl_xor(lt, 16);
    lt += __shfl_xor(lt, 32);
    const int j = j0 + 16 * t + m;
    if (j >= n) continue;
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    const int64_t oo = ((int64_t)(qs0 + j) * a.Hq + hq) * D + 4 * kq;
    if (!PA_IN_BOUNDS(kBsOut, oo >= 0 && oo + 16 * 7 + 4 <= n_rows)) continue;
    _Float16* orow = a.out + oo;
#pragma unroll
    for (int nn = 0; nn < 8; ++nn) {
      typedef _Float16 h4 __attribute__((ext_vector_type(4)));
      h4 ov;
#pragma unroll
      for (int r = 0; r < 4; ++r) ov[r] = (_Float16)(o[t][nn][r] * inv);
      *reinterpret_cast<u32x2*>(orow + 16 * nn) = __builtin_bit_cast(u32x2, ov);
    }
  }
}

template <int BT, int G>
hipError_t launch_g(const PrefillArgs& a, int64_t grid, hipStream_t stream) {
  prefill_kernel<BT, G, prefill_row_tiles(G), kPrefillWaves, kPrefillChunk, kPrefillStages>
      <<<(unsigned)grid, kPrefillWaves * 64, 0, stream>>>(a);
  return hipGetLastError();
}

template <int BT>
hipError_t launch_bt(const PrefillArgs& a, int G, int64_t grid, hipStream_t stream) {
  switch (G) {
    case 1: return launch_g<BT, 1>(a, grid, stream);
    case 2: return launch_g<BT, 2>(a, grid, stream);
    case 4: return launch_g<BT, 4>(a, grid, stream);
    case 8: return launch_g<BT, 8>(a, grid, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

PA_BOUNDS_COLLECTOR(bounds_take_prefill)

int prefill_rows_per_workgroup(int G) {
  const int hw = G < kPrefillWaves ? G : kPrefillWaves;
  return (kPrefillWaves / hw) * 16 * prefill_row_tiles(G);
}

int64_t prefill_work_items(int G, int S, int Hkv, int max_query_len) {
  const int QB = prefill_rows_per_workgroup(G);
  const int nhg = G > kPrefillWaves ? G / kPrefillWaves : 1;
  return (int64_t)((max_query_len + QB - 1) / QB) * S * nhg * Hkv;
}

hipError_t launch_prefill(const PrefillArgs& a, int B, int G, int max_query_len,
                          hipStream_t stream) {
  const int QB = prefill_rows_per_workgroup(G);
  PrefillArgs b = a;
  b.n_rank = (max_query_len + QB - 1) / QB;
  b.n_work = prefill_work_items(G, a.S, a.Hkv, max_query_len);
  b.per_xcd = (b.n_work + 7) / 8;
  const int64_t grid = 8 * b.per_xcd;
  if (b.n_work == 0) return hipSuccess;
  switch (B) {
    case 8: return launch_bt<8>(b, G, grid, stream);
    case 16: return launch_bt<16>(b, G, grid, stream);
    case 32: return launch_bt<32>(b, G, grid, stream);
    default: return launch_bt<0>(b, G, grid, stream);
  }
}

}  // namespace pa
