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
// workgroup is 4 waves over one KV head g: 4 query heads of g with the same
// rows when the group has at least 4 heads, otherwise 4 / G row tiles of each
// of the G heads; all 4 waves walk the same tokens, so a K/V tile fetched by
// one is served to the others from the CU's cache. Tokens are taken 32 at a
// time (a chunk: two 16-token units of one KV head, each a contiguous 4 KiB
// tile in the pool).
//
// Matrix products (v_mfma_f32_16x16x32_f16; lane l = 16 kq + m):
//   scores   S^T = K Q^T per unit: the A operand is the key tile itself (lane
//            holds token m, dims 32c + 8kq .. +7, one 16-byte load from the
//            pool), the B operand the query rows held in registers; lane l
//            receives S for query row m and tokens 4kq + r.
//   output   O^T = V^T P^T per chunk: the B operand is P exactly as the score
//            product left it (query m, the lane's 8 tokens), the A operand
//            carries V for the same 8 tokens at one output dimension. The 16
//            dimensions of product n are 8m' + n (m' the A row), so lane l
//            loads dims 8m .. 8m+7 of its 8 tokens with 16-byte loads and
//            regroups them in registers: no LDS transpose. Lane l ends with
//            O[row m][dims 32kq + 8r + n].
// Every per-row softmax quantity (running max, sum, rescale factor) lives in
// the lanes of that row, so the only cross-lane steps are the two row-max
// exchanges per chunk and the final sum.
//
// Masking: keys and values past the sequence's L tokens are fetched as zeros
// by the buffer range check (so NaN or Inf in unused slots never enters a
// product); causal exclusions select the score to "no token" and p to 0.
#include "prefill_internal.h"

namespace pa {
namespace {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr float kNegBig = -1.0e30f;
// Lazy rescaling slack in log2 units: softmax weights stay at most 2^kSlack.
#ifndef PA_PREFILL_SLACK
#define PA_PREFILL_SLACK 8.0f
#endif
constexpr float kSlack = PA_PREFILL_SLACK;
constexpr int kChunk = 32;                 // tokens per loop step (two 16-token units)
constexpr int kUnitTok = 16;
constexpr int kRowBytes = kHeadDim * 2;    // one token row of one KV head
constexpr int kRsrcWord3 = 0x00020000;     // raw buffer, gfx9 family

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const _Float16* base, int nbytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<_Float16*>(base), 0, nbytes, kRsrcWord3);
}

// Registers of one chunk: k[u][c] = key token m of unit u, dims 32c + 8kq ..;
// v[j] = value row of token tok(8kq + j) at dims 8m .. 8m+7, where the lane's
// token j is 16 (j / 4) + 4kq + (j % 4) of the chunk.
struct Chunk {
  u32x4 k[2][4];
  u32x4 v[8];
};

template <int BT, int G, int QT, bool NT>
__global__ __launch_bounds__(256) void prefill_kernel(const PrefillArgs a) {
  constexpr int D = kHeadDim;
  constexpr int HW = G < 4 ? G : 4;        // query heads in a workgroup
  constexpr int RW = 4 / HW;               // row tiles per head in a workgroup
  constexpr int QR = 16 * QT;              // query rows per wave
  constexpr int QB = RW * QR;              // query rows per workgroup
  constexpr int NHG = G / HW;              // workgroups per KV head and row block
  static_assert(G == 1 || G == 2 || G == 4 || G == 8, "group size");
  const int B = BT > 0 ? BT : a.B;
  const int UPB = B / kUnitTok;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
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

  const int qs0 = a.qstart[s];
  const int qs1 = a.qstart[s + 1];
  if (qs0 < 0 || qs1 > a.T || qs1 <= qs0) return;
  const int n = qs1 - qs0;
  const int nqb = (n + QB - 1) / QB;
  if (rank >= nqb) return;
  const int qb = nqb - 1 - rank;
  int L = a.lens[s];
  L = L < 0 ? 0 : L;
  L = L > a.MB * B ? a.MB * B : L;
  const int hq = g * G + hg * HW + wave % HW;
  const int j0 = qb * QB + (wave / HW) * QR;
  if (j0 >= n) return;                     // no barriers below: waves are independent
  const int base_pos = L - n;              // row j sits at position base_pos + j

  // query rows as B operands
  h8 qf[QT][4];
  int pos[QT];
#pragma unroll
  for (int t = 0; t < QT; ++t) {
    const int j = j0 + 16 * t + m;
    const bool ok = j < n;
    pos[t] = base_pos + j;
    const _Float16* qrow = a.q + ((int64_t)(qs0 + (ok ? j : 0)) * a.Hq + hq) * D + 8 * kq;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const u32x4 raw = ok ? *reinterpret_cast<const u32x4*>(qrow + 32 * c) : u32x4{0, 0, 0, 0};
      qf[t][c] = __builtin_bit_cast(h8, raw);
    }
  }

  const int jl = (j0 + QR < n ? j0 + QR : n) - 1;   // last valid row of the wave
  int kend = base_pos + jl + 1;                      // keys [0, kend) can be visible
  kend = kend > L ? L : kend;
  kend = kend < 0 ? 0 : kend;
  const int nchunk = (kend + kChunk - 1) / kChunk;
  // chunks whose every key is visible to every row of the wave
  int nfull = base_pos + j0 + 1 >= 0 ? (base_pos + j0 + 1) / kChunk : 0;
  nfull = nfull > nchunk ? nchunk : nfull;

  float mrow[QT], lsum[QT];
  f4 o[QT][8];
#pragma unroll
  for (int t = 0; t < QT; ++t) {
    mrow[t] = kNegBig;
    lsum[t] = 0.f;
#pragma unroll
    for (int nn = 0; nn < 8; ++nn) o[t][nn] = f4{0.f, 0.f, 0.f, 0.f};
  }

  // Physical blocks come from the table through scalar loads (the index is
  // wave-uniform): they are counted apart from the vector loads, so waiting
  // for a table entry never waits for the K/V tiles in flight. The entries
  // of chunk c + 1 are requested while chunk c - 1 is still being fetched
  // and computed. Entries outside the pool are clamped to block 0.
  typedef const __attribute__((address_space(4))) int32_t* const_i32;
  const const_i32 trow = (const_i32)(a.tables + (int64_t)s * a.MB);
  const int nblk = (kend + B - 1) / B;
  // physical block of unit U, or -1 when U holds no visible key
  auto table_entry = [&](int U) -> int {
    const int bi = U / UPB;
    return U * kUnitTok < kend && bi < nblk ? trow[bi] : -1;
  };
  auto unit_base = [&](int U, int phys, int& nbytes) -> int64_t {
    const int tok = U * kUnitTok;
    if (phys < 0) {                        // past the visible keys: no-op load
      nbytes = 0;
      return 0;
    }
    const int valid = L - tok < kUnitTok ? L - tok : kUnitTok;
    nbytes = valid * kRowBytes;
    const int bi = U / UPB;
    const int safe = (unsigned)phys < (unsigned)a.NB ? phys : 0;
    return (((int64_t)safe * a.Hkv + g) * B + (U - bi * UPB) * kUnitTok) * D;
  };
  // Byte offsets inside a unit's 4 KiB tile. The token of every load sits in
  // the vector offset, which the range check always covers, so a token at or
  // past L reads as zero whether or not the scalar offset is checked too.
  const unsigned k_voff = m * kRowBytes + kq * 16;       // token m, dims 8kq (+32c via soffset)
  const unsigned v_voff = kq * 4 * kRowBytes + m * 16;   // token 4kq, dims 8m
  auto fetch = [&](Chunk& ch, int c, const int (&ph)[2]) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      int nbytes;
      const int64_t base = unit_base(2 * c + u, ph[u], nbytes);
      const __amdgpu_buffer_rsrc_t rk = rsrc(a.k_pool + base, nbytes);
      const __amdgpu_buffer_rsrc_t rv = rsrc(a.v_pool + base, nbytes);
#pragma unroll
      for (int cc = 0; cc < 4; ++cc)
        ch.k[u][cc] = __builtin_amdgcn_raw_buffer_load_b128(rk, k_voff, cc * 64, NT ? 2 : 0);
#pragma unroll
      for (int r = 0; r < 4; ++r)
        ch.v[4 * u + r] =
            __builtin_amdgcn_raw_buffer_load_b128(rv, v_voff + r * kRowBytes, 0, NT ? 2 : 0);
    }
  };

  auto compute = [&](const Chunk& ch, int c, bool masked) {
    // V^T operands: product nn takes dim 8m + nn of the lane's 8 tokens
    h8 va[8];
    {
      h8 vr[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) vr[j] = __builtin_bit_cast(h8, ch.v[j]);
#pragma unroll
      for (int nn = 0; nn < 8; ++nn) {
#pragma unroll
        for (int j = 0; j < 8; ++j) va[nn][j] = vr[j][nn];
      }
    }
#pragma unroll
    for (int t = 0; t < QT; ++t) {
      f4 sc[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        f4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int cc = 0; cc < 4; ++cc)
          acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(h8, ch.k[u][cc]),
                                                       qf[t][cc], acc, 0, 0, 0);
        sc[u] = acc;
      }
      // Raw scores; the maximum is taken before scaling (the scale is
      // positive, so the order is the same) and p = 2^(scale_log2 * s - m)
      // is one fused multiply-add and one exp2 per score.
      float x[8];
      bool vis[8];
      float mx = kNegBig;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float v = sc[j / 4][j % 4];
        vis[j] = !masked || c * kChunk + 16 * (j / 4) + 4 * kq + (j % 4) <= pos[t];
        x[j] = v;
        mx = __builtin_fmaxf(mx, vis[j] ? v : kNegBig);
      }
      mx = __builtin_fmaxf(mx, __shfl_xor(mx, 16));
      mx = __builtin_fmaxf(mx, __shfl_xor(mx, 32));
      // Running maximum m (log2 domain, scaled). Lazy rescaling: m is raised,
      // and the accumulators rescaled, only when some row of the wave would
      // otherwise see p above 2^kSlack; until then p <= 2^kSlack, exactly
      // representable in fp16's range. The result is the same softmax: the
      // final division uses the same m for numerator and denominator.
      const float mcand = mx > 0.5f * kNegBig ? mx * a.scale_log2 : kNegBig;
      const bool raise = mcand > mrow[t] + kSlack;
      if (__builtin_amdgcn_ballot_w64(raise)) {
        const float mnew = __builtin_fmaxf(mrow[t], mcand);
        const float alpha = __builtin_amdgcn_exp2f(mrow[t] - mnew);
        mrow[t] = mnew;
        lsum[t] *= alpha;
#pragma unroll
        for (int nn = 0; nn < 8; ++nn) o[t][nn] *= alpha;
      }
      float ls = lsum[t];
      h8 pb;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        float p = __builtin_amdgcn_exp2f(__builtin_fmaf(x[j], a.scale_log2, -mrow[t]));
        p = vis[j] ? p : 0.f;
        ls += p;
        pb[j] = (_Float16)p;
      }
      lsum[t] = ls;
#pragma unroll
      for (int nn = 0; nn < 8; ++nn)
        o[t][nn] = __builtin_amdgcn_mfma_f32_16x16x32_f16(va[nn], pb, o[t][nn], 0, 0, 0);
    }
  };

  if (nchunk > 0) {
    Chunk b0, b1;
    int ph[2] = {table_entry(0), table_entry(1)};
    fetch(b0, 0, ph);
    ph[0] = table_entry(2);
    ph[1] = table_entry(3);
    int c = 0;
    while (true) {
      fetch(b1, c + 1, ph);
      ph[0] = table_entry(2 * c + 4);
      ph[1] = table_entry(2 * c + 5);
      compute(b0, c, c >= nfull);
      if (++c >= nchunk) break;
      fetch(b0, c + 1, ph);
      ph[0] = table_entry(2 * c + 4);
      ph[1] = table_entry(2 * c + 5);
      compute(b1, c, c >= nfull);
      if (++c >= nchunk) break;
    }
  }

  // normalise and store: lane holds row m, dims 32kq + 8r + nn
#pragma unroll
  for (int t = 0; t < QT; ++t) {
    float lt = lsum[t];
    lt += __shfl_xor(lt, 16);
    lt += __shfl_xor(lt, 32);
    const int j = j0 + 16 * t + m;
    if (j >= n) continue;
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    _Float16* orow = a.out + ((int64_t)(qs0 + j) * a.Hq + hq) * D + 32 * kq;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      h8 ov;
#pragma unroll
      for (int nn = 0; nn < 8; ++nn) ov[nn] = (_Float16)(o[t][nn][r] * inv);
      *reinterpret_cast<u32x4*>(orow + 8 * r) = __builtin_bit_cast(u32x4, ov);
    }
  }
}

template <int BT, int G>
hipError_t launch_g(const PrefillArgs& a, int64_t grid, hipStream_t stream) {
  prefill_kernel<BT, G, kPrefillRowTiles, kDecodeNontemporal><<<(unsigned)grid, 256, 0, stream>>>(a);
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

int prefill_rows_per_workgroup(int G) {
  const int hw = G < 4 ? G : 4;
  return (4 / hw) * 16 * kPrefillRowTiles;
}

hipError_t launch_prefill(const PrefillArgs& a, int B, int G, int max_query_len,
                          hipStream_t stream) {
  const int QB = prefill_rows_per_workgroup(G);
  const int nhg = G > 4 ? G / 4 : 1;
  PrefillArgs b = a;
  b.n_rank = (max_query_len + QB - 1) / QB;
  b.n_work = (int64_t)b.n_rank * a.S * nhg * a.Hkv;
  b.per_xcd = (b.n_work + 7) / 8;
  const int64_t grid = 8 * b.per_xcd;
  if (b.n_work == 0) return hipSuccess;
  switch (B) {
    case 16: return launch_bt<16>(b, G, grid, stream);
    case 32: return launch_bt<32>(b, G, grid, stream);
    default: return launch_bt<0>(b, G, grid, stream);
  }
}

}  // namespace pa
