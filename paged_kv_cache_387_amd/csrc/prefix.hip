// Shared-prefix attention pass for gfx950 (CDNA4).
//
// Sequences forked from one parent share the physical blocks of their common
// beginning (reference counts and copy-on-write: "KVcache-learning",
// fairy2021.github.io, s05 and s08; block sharing between requests, "KV Cache
// and PagedAttention (vllm-musa)", 7yue.com, section 2).  Attention over such
// a prefix is the same for every sharer except for the query, so instead of
// each sequence streaming the prefix on its own, one pass reads each prefix
// tile once per (group, kv head) and applies it to all the group's queries:
//   for every member s and query head h of kv head kvh, over prefix tokens t
//     m, l, o = max, sum and weighted V of the (base-2) scores scale*q[s][h].K_t
// The result is written as partial (normalized o, log-sum-exp) in the same
// format as the decode kernel's split-K partials, and the log-sum-exp merge
// combines it with the sequence's own suffix partials: softmax over the
// concatenation equals the merge of softmaxes over the pieces.
//
// Work decomposition.  A group of n sequences has n*G query columns per kv
// head (G query heads per kv head).  One workgroup (4 waves) takes CW = 16*C
// columns and one partition of the prefix; wave w takes the partition's tiles
// w, w+4, ...  Per 16-token tile a wave computes, for each of its C chunks of
// 16 columns, the 16x16 score tile S^T = K q (MFMA, K as loaded is the A
// operand), the online softmax per column, and O^T += V^T P^T (MFMA); the K and
// V operands (and their widening from int8 / E4M3) are prepared once per tile
// and reused by the C chunks, so the MFMA work per byte loaded is C times that
// of decode.  The waves' states are combined through LDS at the end.  Tiles
// are read with ordinary loads: the workgroups of the other column blocks read
// the same tiles at about the same time from L2.
#include "attn_common.h"

namespace pkv {
namespace {

// Wait until at most N vector-memory operations of the wave are outstanding
// (loads complete in issue order), and keep the compiler from moving memory
// accesses across the wait.  Loads straight into LDS are not tracked by the
// compiler's own wait counts, so the ring below waits for them explicitly.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
  asm volatile("" ::: "memory");
}

__device__ __forceinline__ void load16_to_lds(const uint8_t *src, u4 *lds_row) {
  __builtin_amdgcn_global_load_lds(
      (const __attribute__((address_space(1))) void *)src,
      (__attribute__((address_space(3))) void *)lds_row, 16, 0, 0);
}

// 16-byte LDS read at byte address `addr` + OFF (an LDS offset).  Issued as
// inline assembly: the compiler would otherwise wait for every load in flight
// into LDS before any LDS read (it cannot tell the ring's slots apart).  The
// caller waits with lds_wait before using the value.
template <int OFF>
__device__ __forceinline__ u4 lds_read16(uint32_t addr) {
  u4 x;
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(x) : "v"(addr), "i"(OFF));
  return x;
}
__device__ __forceinline__ void lds_wait() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }
// Makes later uses of x depend on the preceding lds_wait.
__device__ __forceinline__ void after_wait(u4 &x) { asm volatile("" : "+v"(x)); }

template <int I, int N, int STRIDE>
__device__ __forceinline__ void lds_read_row(uint32_t addr, u4 *out) {
  if constexpr (I < N) {
    out[I] = lds_read16<I * STRIDE>(addr);
    lds_read_row<I + 1, N, STRIDE>(addr, out);
  }
}

// Tiles in flight per wave (LDS ring slots): 2*NL KiB each.
template <int KV> struct PrefixRing { static constexpr int NR = 4; };
template <> struct PrefixRing<PKV_F32> { static constexpr int NR = 2; };
template <> struct PrefixRing<PKV_I8> { static constexpr int NR = 6; };
template <> struct PrefixRing<PKV_E4M3> { static constexpr int NR = 6; };

template <int KV, int D, int BS, int C>
__global__ __launch_bounds__(64 * kWaves, 1) void prefix_kernel(PrefixParams p) {
  constexpr int EB = Kv<KV>::EB;
  constexpr bool QUANT = (KV == PKV_I8 || KV == PKV_E4M3);
  constexpr int SLICE = BS * D * EB;
  constexpr int TPB = BS >= kTile ? BS / kTile : 1;
  constexpr bool SPLIT = BS < kTile;
  constexpr int TB = SPLIT ? BS : kTile;
  constexpr int NL = D * EB / 64;
  constexpr int NACC = D / 16;
  constexpr int E = 4 / EB;
  constexpr int NR = PrefixRing<KV>::NR;  // tiles in flight per wave
  constexpr int LPT = 2 * NL + (QUANT ? 2 : 0);   // vector-memory loads per tile
  constexpr int CW = 16 * C;
  static_assert(BS == 8 || BS == 16 || BS == 32, "block size");
  static_assert((NR - 1) * LPT < 64, "wait count");

  // Per wave, NR slots of one tile each: K loads 0..NL-1, then V loads, each
  // 64 lanes x 16 bytes as the lanes read them.  After the tile loop the same
  // memory holds the accumulators of the wave combine.
  __shared__ u4 lds_ring[kWaves][NR][2 * NL][64];
  static_assert(sizeof(lds_ring) >= sizeof(f4) * C * NACC * 64, "combine space");
  f4(*lds_acc)[NACC][64] = reinterpret_cast<f4(*)[NACC][64]>(&lds_ring[0][0][0][0]);
  __shared__ float lds_m[kWaves][CW];
  __shared__ float lds_l[kWaves][CW];

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = lane & 15;
  const int g = lane >> 4;

  // Workgroup -> (unit = (group, kv head), column block, partition).  Unit u
  // runs on die u % kXcds; the column blocks of one partition are adjacent
  // slots of that die, so they read the same tiles at about the same time.
  const int bid = blockIdx.x;
  const int die_slot = bid / kXcds;
  const int ugroups = unit_groups(p.num_units);
  const int per_part = ugroups * p.col_blocks;
  const int part = die_slot / per_part;
  const int rem = die_slot - part * per_part;
  const int cb = rem / ugroups;
  const int u = (rem - cb * ugroups) * kXcds + bid % kXcds;
  if (u >= p.num_units || part >= p.num_pparts) return;
  const int grp = u / p.num_kv_heads;
  const int kvh = u - grp * p.num_kv_heads;
  const int G = p.group;
  const int H = p.num_heads;

  int off = p.offsets[grp];
  int end = p.offsets[grp + 1];
  off = off < 0 ? 0 : (off > p.num_members ? p.num_members : off);
  end = end < off ? off : (end > p.num_members ? p.num_members : end);
  const int ncols = (end - off) * G;
  const int c0 = cb * CW;
  if (c0 >= ncols) return;

  int plen = p.prefix_lens[grp];
  plen = plen < 0 ? 0 : (plen > p.max_prefix_blocks * BS ? p.max_prefix_blocks * BS : plen);
  const int ntile = plen / kTile;
  const int first = part * p.pp_tiles;
  if (first >= ntile) return;
  const int last = min(first + p.pp_tiles, ntile);
  const int nt_part = last - first;
  const int nt_w = nt_part > w ? (nt_part - w + kWaves - 1) / kWaves : 0;
  const int32_t *trow = p.tables + (size_t)grp * p.max_prefix_blocks;

  auto load_tv = [&](int c, int *tvb) {
    const int tile = first + w + (c + lane) * kWaves;
    const int lim = p.max_prefix_blocks;
    int e = SPLIT ? 2 * tile : tile / TPB;
    e = e < lim ? e : lim - 1;
    if constexpr (SPLIT) {
      const int e2 = 2 * tile + 1 < lim ? 2 * tile + 1 : e;
      *tvb = trow[e2];
    }
    return trow[e];
  };
  int tvb_next = 0;
  int tv_next = load_tv(0, &tvb_next);

  // Query columns: column c0 + 16*ch + r is head kvh*G + (c % G) of member
  // c / G.  Columns past the group hold member 0's query and are not stored.
  int col_seq[C], col_head[C];
  bool col_ok[C];
#pragma unroll
  for (int ch = 0; ch < C; ++ch) {
    const int c = c0 + 16 * ch + r;
    col_ok[ch] = c < ncols;
    const int cc = col_ok[ch] ? c : 0;
    int sq = p.members[off + cc / G];
    col_ok[ch] = col_ok[ch] && (unsigned)sq < (unsigned)p.num_seqs;
    col_seq[ch] = (unsigned)sq < (unsigned)p.num_seqs ? sq : 0;
    col_head[ch] = kvh * G + cc % G;
  }
  float qf32[C][NL][4];
  h8 qf16[C][NL][QUANT ? 2 : 1];
#pragma unroll
  for (int ch = 0; ch < C; ++ch) {
    const size_t qrow = ((size_t)col_seq[ch] * H + col_head[ch]) * D;
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      if constexpr (KV == PKV_F32) {
        const float *qp = reinterpret_cast<const float *>(p.q) + qrow + (4 * i + g) * 4;
        const u4 raw = load16(reinterpret_cast<const uint8_t *>(qp));
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) qf32[ch][i][jj] = as_f32(raw[jj]);
      } else if constexpr (KV == PKV_F16) {
        const _Float16 *qp = reinterpret_cast<const _Float16 *>(p.q) + qrow + (4 * i + g) * 8;
        qf16[ch][i][0] = __builtin_bit_cast(h8, load16(reinterpret_cast<const uint8_t *>(qp)));
      } else {
        const _Float16 *qp = reinterpret_cast<const _Float16 *>(p.q) + qrow + (4 * i + g) * 16;
        qf16[ch][i][0] = __builtin_bit_cast(h8, load16(reinterpret_cast<const uint8_t *>(qp)));
        qf16[ch][i][QUANT ? 1 : 0] =
            __builtin_bit_cast(h8, load16(reinterpret_cast<const uint8_t *>(qp + 8)));
      }
    }
  }
  // int8: 1152 * (sum of the column's q), taken out of the biased scores
  float qbias[C];
#pragma unroll
  for (int ch = 0; ch < C; ++ch) {
    qbias[ch] = 0.0f;
    if constexpr (KV == PKV_I8) {
      float qs = 0.0f;
#pragma unroll
      for (int i = 0; i < NL; ++i)
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int e = 0; e < 8; ++e) qs += (float)qf16[ch][i][h][e];
      qbias[ch] = kI8Bias * row_sum4(qs);
    }
  }

  float m[C], l[C];
  f4 acc[C][NACC];
  f4 accp[C];
#pragma unroll
  for (int ch = 0; ch < C; ++ch) {
    m[ch] = -INFINITY;
    l[ch] = 0.0f;
    accp[ch] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int a = 0; a < NACC; ++a) acc[ch][a] = f4{0.f, 0.f, 0.f, 0.f};
  }

  const size_t kv_head_off = (size_t)kvh * SLICE;
  const size_t block_stride = (size_t)p.num_kv_heads * SLICE;
  // Headroom (base-2 units) a column's maximum may rise before the running
  // state is rescaled.  Quantized V folds its scale (and the factor 64) into
  // the fp16 weights, which must stay below fp16's maximum: 4 * 64 * s_v.
  constexpr float kTau = QUANT ? 2.0f : 8.0f;
  bool fresh = true;     // no tile consumed yet (wave-uniform)

  struct Tile {
    u4 k[NL];
    u4 v[NL];
    u2 ks, vs;
    bool ok;
  };
  struct Slot {   // what of a tile in flight lives in registers
    u2 ks, vs;
    bool ok;
  };

  // Loads of prefix tile `tile` (table entries: lane j of tv / tvb) into ring
  // slot `slot`, with the addressing of the decode kernel (all prefix tiles
  // are full): K and V straight into LDS, the scales into registers.
  auto issue = [&](int tv, int tvb, int j, int tile, int slot, Slot &t) {
    int pa = __builtin_amdgcn_readlane(tv, j);
    int pb = SPLIT ? __builtin_amdgcn_readlane(tvb, j) : pa;
    t.ok = (unsigned)pa < (unsigned)p.num_blocks && (unsigned)pb < (unsigned)p.num_blocks;
    pa = t.ok ? pa : 0;
    pb = t.ok ? pb : 0;
    const int tq = SPLIT ? 0 : tile % TPB;
    const size_t tile_off = (size_t)tq * (TB * D * EB);
    const int pk = SPLIT && r >= 8 ? pb : pa;
    const int pv = SPLIT && g >= 2 ? pb : pa;
    const int tk = SPLIT ? (r & 7) : r;
    const int tv0 = SPLIT ? 4 * (g & 1) : 4 * g;
    const uint8_t *kb = p.k_cache + (size_t)pk * block_stride + kv_head_off + tile_off;
    const uint8_t *vb = p.v_cache + (size_t)pv * block_stride + kv_head_off + tile_off;
#pragma unroll
    for (int i = 0; i < NL; ++i)
      load16_to_lds(kb + (size_t)((4 * i + g) * TB + tk) * 16, &lds_ring[w][slot][i][0]);
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      if constexpr (EB == 1)
        load16_to_lds(vb + (size_t)((16 * i + r) * (TB / 4) + tv0 / 4) * 16,
                      &lds_ring[w][slot][NL + i][0]);
      else
        load16_to_lds(vb + (size_t)((16 * i + r) * TB + tv0) * 4, &lds_ring[w][slot][NL + i][0]);
    }
    if constexpr (QUANT) {
      const size_t so = ((size_t)pv * p.num_kv_heads + kvh) * BS + tq * kTile + tv0;
      t.ks = *reinterpret_cast<const u2 *>(p.k_scale + so);
      t.vs = *reinterpret_cast<const u2 *>(p.v_scale + so);
    }
  };

  auto consume = [&](int slot, const Slot &sl) {
    if (!sl.ok) return;  // table entry outside the pool: tile skipped
    Tile t;
    const uint32_t base = (uint32_t)(size_t)(
        (__attribute__((address_space(3))) const u4 *)&lds_ring[w][slot][0][lane]);
    u4 kv[2 * NL];
    lds_read_row<0, 2 * NL, 1024>(base, kv);
    lds_wait();
#pragma unroll
    for (int i = 0; i < 2 * NL; ++i) after_wait(kv[i]);
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      t.k[i] = kv[i];
      t.v[i] = kv[NL + i];
    }
    t.ks = sl.ks;
    t.vs = sl.vs;
    // Operands shared by the C chunks.
    h8 kq[NL][2];        // widened K codes (quantized)
    h4 vh[NL][4];        // V^T operands: [i][0..1] fp16, [i][e] widened codes
    float ksf[4], vsf[4];
    if constexpr (QUANT) {
#pragma unroll
      for (int i = 0; i < NL; ++i) codes16_to_h8<KV>(t.k[i], kq[i][0], kq[i][1]);
#pragma unroll
      for (int i = 0; i < NL; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) vh[i][e] = codes4_to_h4<KV>(t.v[i][e]);
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        ksf[v] = (float)as_h2(t.ks[v >> 1])[v & 1];
        vsf[v] = (float)as_h2(t.vs[v >> 1])[v & 1] * kPvBoost;
      }
    } else if constexpr (KV == PKV_F16) {
#pragma unroll
      for (int i = 0; i < NL; ++i) {
        const uint32_t lo01 = __builtin_amdgcn_perm(t.v[i][1], t.v[i][0], 0x05040100u);
        const uint32_t lo23 = __builtin_amdgcn_perm(t.v[i][3], t.v[i][2], 0x05040100u);
        const uint32_t hi01 = __builtin_amdgcn_perm(t.v[i][1], t.v[i][0], 0x07060302u);
        const uint32_t hi23 = __builtin_amdgcn_perm(t.v[i][3], t.v[i][2], 0x07060302u);
        vh[i][0] = __builtin_bit_cast(h4, u2{lo01, lo23});
        vh[i][1] = __builtin_bit_cast(h4, u2{hi01, hi23});
      }
    }
    // q.K of every chunk: C independent accumulator chains
    f4 sc[C];
#pragma unroll
    for (int ch = 0; ch < C; ++ch) sc[ch] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < NL; ++i) {
#pragma unroll
      for (int ch = 0; ch < C; ++ch) {
        if constexpr (KV == PKV_F32) {
#pragma unroll
          for (int jj = 0; jj < 4; ++jj)
            sc[ch] = __builtin_amdgcn_mfma_f32_16x16x4f32(as_f32(t.k[i][jj]), qf32[ch][i][jj],
                                                          sc[ch], 0, 0, 0);
        } else if constexpr (KV == PKV_F16) {
          sc[ch] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(h8, t.k[i]),
                                                          qf16[ch][i][0], sc[ch], 0, 0, 0);
        } else {
          sc[ch] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kq[i][0], qf16[ch][i][0], sc[ch], 0,
                                                          0, 0);
          sc[ch] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kq[i][1], qf16[ch][i][QUANT ? 1 : 0],
                                                          sc[ch], 0, 0, 0);
        }
      }
    }
    // base-2 scores (the K scale is per token: the same for every chunk)
    float coef[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) coef[v] = QUANT ? p.qk_scale * ksf[v] : p.qk_scale;
    float x[C][4], mn[C];
    bool over = false;
#pragma unroll
    for (int ch = 0; ch < C; ++ch) {
#pragma unroll
      for (int v = 0; v < 4; ++v)
        x[ch][v] = (KV == PKV_I8 ? sc[ch][v] - qbias[ch] : sc[ch][v]) * coef[v];
      const float bm = row_max4(fmaxf(fmaxf(x[ch][0], x[ch][1]), fmaxf(x[ch][2], x[ch][3])));
      mn[ch] = fmaxf(m[ch], bm);
      over = over || mn[ch] > m[ch] + kTau;
    }
    // Running maxima: set by the first tile; afterwards moved (and the
    // accumulators rescaled) only when some column's maximum rose by more
    // than kTau, so the weights exp2(x - m) stay below 2^kTau.
    if (fresh) {
#pragma unroll
      for (int ch = 0; ch < C; ++ch) m[ch] = mn[ch];
      fresh = false;
    } else if (__builtin_amdgcn_ballot_w64(over) != 0) {
#pragma unroll
      for (int ch = 0; ch < C; ++ch) {
        const float alpha = fast_exp2(m[ch] - mn[ch]);
        l[ch] *= alpha;
#pragma unroll
        for (int a = 0; a < NACC; ++a) acc[ch][a] *= alpha;
        if constexpr (KV == PKV_I8) accp[ch] *= alpha;
        m[ch] = mn[ch];
      }
    }
#pragma unroll
    for (int ch = 0; ch < C; ++ch) {
      float pr[4];
#pragma unroll
      for (int v = 0; v < 4; ++v) pr[v] = fast_exp2(x[ch][v] - m[ch]);
      l[ch] += (pr[0] + pr[1]) + (pr[2] + pr[3]);
      if constexpr (KV == PKV_F32) {
#pragma unroll
        for (int i = 0; i < NL; ++i)
#pragma unroll
          for (int jj = 0; jj < 4; ++jj)
            acc[ch][i] = __builtin_amdgcn_mfma_f32_16x16x4f32(as_f32(t.v[i][jj]), pr[jj],
                                                              acc[ch][i], 0, 0, 0);
      } else if constexpr (KV == PKV_F16) {
        const h4 pb = h4{(_Float16)pr[0], (_Float16)pr[1], (_Float16)pr[2], (_Float16)pr[3]};
#pragma unroll
        for (int i = 0; i < NL; ++i) {
          acc[ch][2 * i] =
              __builtin_amdgcn_mfma_f32_16x16x16f16(vh[i][0], pb, acc[ch][2 * i], 0, 0, 0);
          acc[ch][2 * i + 1] =
              __builtin_amdgcn_mfma_f32_16x16x16f16(vh[i][1], pb, acc[ch][2 * i + 1], 0, 0, 0);
        }
      } else {
        float ps[4];
#pragma unroll
        for (int v = 0; v < 4; ++v) ps[v] = pr[v] * vsf[v];
        const h4 pb = h4{(_Float16)ps[0], (_Float16)ps[1], (_Float16)ps[2], (_Float16)ps[3]};
        if constexpr (KV == PKV_I8) {
          const h4 ones = h4{(_Float16)1.0f, (_Float16)1.0f, (_Float16)1.0f, (_Float16)1.0f};
          accp[ch] = __builtin_amdgcn_mfma_f32_16x16x16f16(ones, pb, accp[ch], 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < NL; ++i)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            acc[ch][4 * i + e] =
                __builtin_amdgcn_mfma_f32_16x16x16f16(vh[i][e], pb, acc[ch][4 * i + e], 0, 0, 0);
      }
    }
  };

  // Tile loop: a ring of NR LDS slots per wave, in chunks of 64 tiles (one
  // table entry per lane).  In the steady state the slot consumed next is the
  // oldest of NR tiles in flight: (NR - 1) * LPT loads were issued after its
  // own.  The drain at the end of a chunk waits for everything.
  for (int cc = 0; cc < nt_w; cc += 64) {
    const int nc = min(64, nt_w - cc);
    const int tv = tv_next, tvb = tvb_next;
    const int t0 = first + w + cc * kWaves;
    Slot ring[NR];
#pragma unroll
    for (int j = 0; j < NR; ++j) {
      const int jj = j < nc ? j : nc - 1;
      issue(tv, tvb, jj, t0 + jj * kWaves, j, ring[j]);
    }
    int k0 = 0;
    for (; k0 + 2 * NR <= nc; k0 += NR) {
#pragma unroll
      for (int j = 0; j < NR; ++j) {
        wait_vmcnt<(NR - 1) * LPT>();
        consume(j, ring[j]);
        asm volatile("" ::: "memory");   // the slot's reads before its refill
        issue(tv, tvb, k0 + j + NR, t0 + (k0 + j + NR) * kWaves, j, ring[j]);
      }
    }
#pragma unroll
    for (int j = 0; j < NR; ++j) {
      if (k0 + j < nc) {
        wait_vmcnt<0>();
        consume(j, ring[j]);
      }
      asm volatile("" ::: "memory");
      if (k0 + j + NR < nc) issue(tv, tvb, k0 + j + NR, t0 + (k0 + j + NR) * kWaves, j, ring[j]);
    }
#pragma unroll
    for (int j = 0; j < NR; ++j)
      if (k0 + NR + j < nc) {
        wait_vmcnt<0>();
        consume(j, ring[j]);
      }
    wait_vmcnt<0>();
    if (cc + 64 < nt_w) tv_next = load_tv(cc + 64, &tvb_next);
  }

  // ---- combine the waves: running maxima and sums through LDS, then the
  // accumulators one wave after the other; the last wave writes the partials.
#pragma unroll
  for (int ch = 0; ch < C; ++ch) {
    if constexpr (KV == PKV_I8) {
#pragma unroll
      for (int a = 0; a < NACC; ++a) acc[ch][a] -= kI8Bias * accp[ch];
    }
    l[ch] = row_sum4(l[ch]);
    if (g == 0) {
      lds_m[w][16 * ch + r] = m[ch];
      lds_l[w][16 * ch + r] = l[ch];
    }
  }
  __syncthreads();
  float Mx[C], den[C];
#pragma unroll
  for (int ch = 0; ch < C; ++ch) {
    float M = lds_m[0][16 * ch + r];
#pragma unroll
    for (int ww = 1; ww < kWaves; ++ww) M = fmaxf(M, lds_m[ww][16 * ch + r]);
    float z = 0.0f;
#pragma unroll
    for (int ww = 0; ww < kWaves; ++ww) {
      const float mw = lds_m[ww][16 * ch + r];
      z += mw == -INFINITY ? 0.0f : exp2f(mw - M) * lds_l[ww][16 * ch + r];
    }
    Mx[ch] = M;
    den[ch] = z;
    const float f = m[ch] == -INFINITY ? 0.0f : exp2f(m[ch] - M);
#pragma unroll
    for (int a = 0; a < NACC; ++a) acc[ch][a] *= f;
  }
#pragma unroll
  for (int st = 0; st < kWaves - 1; ++st) {
    if (w == st) {
#pragma unroll
      for (int ch = 0; ch < C; ++ch)
#pragma unroll
        for (int a = 0; a < NACC; ++a)
          lds_acc[ch][a][lane] = st == 0 ? acc[ch][a] : acc[ch][a] + lds_acc[ch][a][lane];
    }
    __syncthreads();
  }
  if (w != kWaves - 1) return;
#pragma unroll
  for (int ch = 0; ch < C; ++ch) {
    if (!col_ok[ch]) continue;
    const size_t row =
        ((size_t)col_seq[ch] * H + col_head[ch]) * p.ws_stride + p.ws_pre + part;
    float inv = 1.0f / den[ch];
    if constexpr (QUANT) inv *= (1.0f / kPvBoost);
    float *dst = p.ws_o + row * D;
    // acc[ch][E*i + e][v] is output element E*(16i + 4g + v) + e: for each i
    // the lane holds 4E consecutive elements.
#pragma unroll
    for (int i = 0; i < NACC / E; ++i) {
      float vals[4 * E];
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const f4 a = acc[ch][E * i + e] + lds_acc[ch][E * i + e][lane];
#pragma unroll
        for (int v = 0; v < 4; ++v) vals[E * v + e] = a[v] * inv;
      }
#pragma unroll
      for (int k = 0; k < E; ++k)
        *reinterpret_cast<f4 *>(dst + E * (16 * i + 4 * g) + 4 * k) =
            f4{vals[4 * k], vals[4 * k + 1], vals[4 * k + 2], vals[4 * k + 3]};
    }
    if (g == 0) p.ws_lse[row] = Mx[ch] + log2f(den[ch]);
  }
}

template <int KV, int D, int BS>
hipError_t launch_prefix_typed(const PrefixParams &p, hipStream_t stream) {
  constexpr int C = KV == PKV_F32 ? 2 : 4;
  hipLaunchKernelGGL((prefix_kernel<KV, D, BS, C>), dim3((unsigned)prefix_grid(p)),
                     dim3(64 * kWaves), 0, stream, p);
  return hipGetLastError();
}

template <int KV, int D>
hipError_t launch_prefix_bs(const PrefixParams &p, int block_size, hipStream_t stream) {
  switch (block_size) {
    case 8: return launch_prefix_typed<KV, D, 8>(p, stream);
    case 32: return launch_prefix_typed<KV, D, 32>(p, stream);
    default: return launch_prefix_typed<KV, D, 16>(p, stream);
  }
}

template <int KV>
hipError_t launch_prefix_d(const PrefixParams &p, int head_dim, int block_size,
                           hipStream_t stream) {
  return head_dim == 64 ? launch_prefix_bs<KV, 64>(p, block_size, stream)
                        : launch_prefix_bs<KV, 128>(p, block_size, stream);
}

}  // namespace

hipError_t launch_prefix(const PrefixParams &p, int cache_dtype, int head_dim, int block_size,
                         hipStream_t stream) {
  switch (cache_dtype) {
    case PKV_F32: return launch_prefix_d<PKV_F32>(p, head_dim, block_size, stream);
    case PKV_F16: return launch_prefix_d<PKV_F16>(p, head_dim, block_size, stream);
    case PKV_I8: return launch_prefix_d<PKV_I8>(p, head_dim, block_size, stream);
    default: return launch_prefix_d<PKV_E4M3>(p, head_dim, block_size, stream);
  }
}

}  // namespace pkv
