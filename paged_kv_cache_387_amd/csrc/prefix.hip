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
// head (G query heads per kv head).  One workgroup (4 waves) takes a block of
// the group's columns and one partition of the prefix; the waves split the
// partition's tokens, every wave applies its tokens to all the block's
// columns, and the waves' states are combined through LDS at the end.  fp16,
// int8 and E4M3 caches run on 32x32x16 MFMAs (prefix32_kernel below); fp32
// caches, which have no such MFMA, on 16x16x4 f32 MFMAs (prefix_kernel).  The
// K and V operands of a tile are prepared once and reused by every column, so
// the MFMA work per byte loaded is the column count times that of decode.
#include "attn_common.h"
#include "lds_ring.h"

namespace pkv {
namespace {

typedef float f16v __attribute__((ext_vector_type(16)));

// ---------------------------------------------------------------------------
// fp32 caches: 16x16 MFMA blocks (fp32 operands have no 32x32x16 form).
template <int D, int BS, int C>
__global__ __launch_bounds__(64 * kWaves, 1) void prefix_kernel(PrefixParams p) {
  constexpr int EB = 4;
  constexpr int SLICE = BS * D * EB;
  constexpr int TPB = BS >= kTile ? BS / kTile : 1;
  constexpr bool SPLIT = BS < kTile;
  constexpr int TB = SPLIT ? BS : kTile;
  constexpr int NL = D * EB / 64;
  constexpr int NACC = D / 16;
  constexpr int NR = 2;                   // tiles in flight per wave (LDS ring slots)
  constexpr int LPT = 2 * NL;             // vector-memory loads per tile
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
#pragma unroll
  for (int ch = 0; ch < C; ++ch) {
    const size_t qrow = ((size_t)col_seq[ch] * H + col_head[ch]) * D;
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      const float *qp = reinterpret_cast<const float *>(p.q) + qrow + (4 * i + g) * 4;
      const u4 raw = load16(reinterpret_cast<const uint8_t *>(qp));
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) qf32[ch][i][jj] = as_f32(raw[jj]);
    }
  }

  float m[C], l[C];
  f4 acc[C][NACC];
#pragma unroll
  for (int ch = 0; ch < C; ++ch) {
    m[ch] = -INFINITY;
    l[ch] = 0.0f;
#pragma unroll
    for (int a = 0; a < NACC; ++a) acc[ch][a] = f4{0.f, 0.f, 0.f, 0.f};
  }

  const size_t kv_head_off = (size_t)kvh * SLICE;
  const size_t block_stride = (size_t)p.num_kv_heads * SLICE;
  // Headroom (base-2 units) a column's maximum may rise before the running
  // state is rescaled: the fp32 weights exp2(x - m) then stay below 2^8.
  constexpr float kTau = 8.0f;
  bool fresh = true;     // no tile consumed yet (wave-uniform)

  // Loads of prefix tile `tile` (table entries: lane j of tv / tvb) into ring
  // slot `slot`, with the addressing of the decode kernel (all prefix tiles
  // are full): K and V straight into LDS.  Returns whether both table entries
  // are in the pool.
  auto issue = [&](int tv, int tvb, int j, int tile, int slot) {
    int pa = __builtin_amdgcn_readlane(tv, j);
    int pb = SPLIT ? __builtin_amdgcn_readlane(tvb, j) : pa;
    const bool ok = (unsigned)pa < (unsigned)p.num_blocks && (unsigned)pb < (unsigned)p.num_blocks;
    pa = ok ? pa : 0;
    pb = ok ? pb : 0;
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
    for (int i = 0; i < NL; ++i)
      load16_to_lds(vb + (size_t)((16 * i + r) * TB + tv0) * 4, &lds_ring[w][slot][NL + i][0]);
    return ok;
  };

  auto consume = [&](int slot, bool ok) {
    if (!ok) return;  // table entry outside the pool: tile skipped
    const uint32_t base = (uint32_t)(size_t)(
        (__attribute__((address_space(3))) const u4 *)&lds_ring[w][slot][0][lane]);
    u4 kv[2 * NL];
    lds_read_row<0, 2 * NL, 1024>(base, kv);
    lds_wait();
#pragma unroll
    for (int i = 0; i < 2 * NL; ++i) after_wait(kv[i]);
    // q.K of every chunk: C independent accumulator chains
    f4 sc[C];
#pragma unroll
    for (int ch = 0; ch < C; ++ch) sc[ch] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < NL; ++i)
#pragma unroll
      for (int ch = 0; ch < C; ++ch)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)
          sc[ch] = __builtin_amdgcn_mfma_f32_16x16x4f32(as_f32(kv[i][jj]), qf32[ch][i][jj],
                                                        sc[ch], 0, 0, 0);
    float x[C][4], mn[C];
    bool over = false;
#pragma unroll
    for (int ch = 0; ch < C; ++ch) {
#pragma unroll
      for (int v = 0; v < 4; ++v) x[ch][v] = sc[ch][v] * p.qk_scale;
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
        m[ch] = mn[ch];
      }
    }
#pragma unroll
    for (int ch = 0; ch < C; ++ch) {
      float pr[4];
#pragma unroll
      for (int v = 0; v < 4; ++v) pr[v] = fast_exp2(x[ch][v] - m[ch]);
      l[ch] += (pr[0] + pr[1]) + (pr[2] + pr[3]);
#pragma unroll
      for (int i = 0; i < NL; ++i)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)
          acc[ch][i] = __builtin_amdgcn_mfma_f32_16x16x4f32(as_f32(kv[NL + i][jj]), pr[jj],
                                                            acc[ch][i], 0, 0, 0);
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
    bool ring[NR];
#pragma unroll
    for (int j = 0; j < NR; ++j) {
      const int jj = j < nc ? j : nc - 1;
      ring[j] = issue(tv, tvb, jj, t0 + jj * kWaves, j);
    }
    int k0 = 0;
    for (; k0 + 2 * NR <= nc; k0 += NR) {
#pragma unroll
      for (int j = 0; j < NR; ++j) {
        wait_vmcnt<(NR - 1) * LPT>();
        consume(j, ring[j]);
        asm volatile("" ::: "memory");   // the slot's reads before its refill
        ring[j] = issue(tv, tvb, k0 + j + NR, t0 + (k0 + j + NR) * kWaves, j);
      }
    }
#pragma unroll
    for (int j = 0; j < NR; ++j) {
      if (k0 + j < nc) {
        wait_vmcnt<0>();
        consume(j, ring[j]);
      }
      asm volatile("" ::: "memory");
      if (k0 + j + NR < nc) ring[j] = issue(tv, tvb, k0 + j + NR, t0 + (k0 + j + NR) * kWaves, j);
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
    const float inv = 1.0f / den[ch];
    float *dst = p.ws_o + row * D;
    // acc[ch][i][v] is output element 16i + 4g + v
#pragma unroll
    for (int i = 0; i < NACC; ++i)
      *reinterpret_cast<f4 *>(dst + 16 * i + 4 * g) = (acc[ch][i] + lds_acc[ch][i][lane]) * inv;
    if (g == 0) p.ws_lse[row] = Mx[ch] + log2f(den[ch]);
  }
}

// ---------------------------------------------------------------------------
// 2- and 1-byte caches: 32x32 MFMA blocks.
//
// A wave takes 32-token steps (two 16-token tiles) of the partition, steps
// w, w+4, ... (waves split the tokens; all four hold the workgroup's 64 query
// columns as two blocks of 32).  Per step and column block:
//   S^T[32 tokens][32 columns] = K q      D/16 MFMAs 32x32x16 (k = 16 dims)
//   online softmax per column
//   O^T[D][32] += V^T P^T                 2 x D/32 MFMAs (k = 16 tokens)
// Layouts of v_mfma_f32_32x32x16_f16, lane l = 32h + n: A row l%32 and
// B column l%32 hold k = 8h .. 8h+7; D holds column n, rows 8j + 4h + v
// (j, v = 0..3) in element 4j + v.  Hence:
//   q.K: lane (n, h) gives token n's K and column n's q for dims 16kk + 8h ..
//        (1-byte K: columns of 16 codes are split over the MFMA pair 2c, 2c+1:
//        lane h loads code column 2c + h, its low 8 codes go to MFMA 2c and the
//        high 8 to 2c + 1, and q follows the same order);
//   P.V: the scores of lane (n, h) are tokens 8j + 4h + v; MFMA kc (tokens
//        16kc .. 16kc+15) takes elements 8kc .. 8kc+7 as its k slots, i.e.
//        tokens 16kc + 4h + 0..3 and 16kc + 8 + 4h + 0..3 -- the V operand of
//        lane (m, h) reads exactly those tokens: two 16-byte groups of V.
//        2-byte V: group = 4 tokens x dims (2c, 2c+1), c = 32G + m: one MFMA
//        for the even dims and one for the odd dims of each G.  1-byte V:
//        group = 4 tokens x dims 4m .. 4m+3: one MFMA per dim offset e.
// K, V (and quantized-cache scales) go straight into a per-wave LDS ring.
// MODE kModeShared: units are (group, kv head), columns the members' query
// heads, the whole prefix visible, partials out.  MODE kModePrefill: units
// are (sequence, kv head), columns its query tokens' heads with causal
// limits; `out` (of type OUT) is written directly when there is one
// partition, else partials.
template <int KV, int D, int BS, int MODE, int OUT>
__global__ __launch_bounds__(64 * kWaves, 1) void prefix32_kernel(PrefixParams p) {
  constexpr int EB = Kv<KV>::EB;
  constexpr bool QUANT = EB == 1;
  static_assert(KV == PKV_F16 || QUANT, "2- and 1-byte caches");
  constexpr int SLICE = BS * D * EB;
  constexpr bool SPLIT = BS < kTile;
  constexpr int TB = SPLIT ? BS : kTile;       // tokens of a stored tile
  constexpr int TPS = BS >= 32 ? 1 : 32 / BS;  // table entries per 32-token step
  constexpr int NKK = D / 16;                  // q.K MFMAs per block
  constexpr int KLD = QUANT ? NKK / 2 : NKK;   // 16-byte K loads per lane and step
  constexpr int NG = QUANT ? 1 : D / 64;       // 2-byte V: groups of 32 column pairs
  constexpr int VLD = QUANT ? 4 : 4 * NG;      // 16-byte V loads per lane and step
  constexpr int NT = QUANT ? 4 : 2 * NG;       // output tiles (32 rows) per column block
  constexpr int NB2 = 2;                       // column blocks of 32 per wave
  constexpr int CW = 32 * NB2;
  constexpr int NR = QUANT ? 4 : 2;            // LDS ring depth (steps in flight)
  constexpr int LPS = KLD + VLD + (QUANT ? 1 : 0);
  static_assert((NR - 1) * LPS < 64, "wait count");

  // The ring (per wave: NR slots of KLD + VLD rows of 64 lanes x 16 bytes);
  // after the tile loop the same memory holds every wave's accumulators.
  constexpr size_t kRingBytes = sizeof(u4) * kWaves * NR * (KLD + VLD) * 64;
  constexpr size_t kAccBytes = sizeof(f16v) * kWaves * NB2 * NT * 64;
  __shared__ u4 lds_raw[(kRingBytes > kAccBytes ? kRingBytes : kAccBytes) / sizeof(u4)];
  u4(*lds_ring)[NR][KLD + VLD][64] = reinterpret_cast<u4(*)[NR][KLD + VLD][64]>(&lds_raw[0]);
  f16v(*lds_acc)[NB2][NT][64] = reinterpret_cast<f16v(*)[NB2][NT][64]>(&lds_raw[0]);
  __shared__ uint32_t lds_sc[kWaves][NR][64];   // quantized: K then V scales of the step
  __shared__ float lds_m[kWaves][CW];
  __shared__ float lds_l[kWaves][CW];

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 31;
  const int h = lane >> 5;

  const int bid = blockIdx.x;
  const int die_slot = bid / kXcds;
  const int ugroups = unit_groups(p.num_units);
  const int per_part = ugroups * p.col_blocks;
  const int part = die_slot / per_part;
  const int rem = die_slot - part * per_part;
  const int cb = rem / ugroups;
  const int u = (rem - cb * ugroups) * kXcds + bid % kXcds;
  if (u >= p.num_units || part >= p.num_pparts) return;
  const int grp = u / p.num_kv_heads;         // group, or sequence
  const int kvh = u - grp * p.num_kv_heads;
  const int G = p.group;
  const int H = p.num_heads;
  constexpr bool PREFILL = MODE == kModePrefill;

  // columns (and, prefill, the tokens of data and the causal limits)
  int off, end, ltok;
  const int32_t *trow;
  int tlim;
  if constexpr (PREFILL) {
    off = p.query_offsets[grp];
    end = p.query_offsets[grp + 1];
    off = off < 0 ? 0 : (off > p.num_query_tokens ? p.num_query_tokens : off);
    end = end < off ? off : (end > p.num_query_tokens ? p.num_query_tokens : end);
    ltok = p.seq_lens[grp];
    ltok = ltok < 0 ? 0 : (ltok > p.max_blocks * BS ? p.max_blocks * BS : ltok);
    if (end - off > ltok) end = off + ltok;   // queries are the sequence's last tokens
    trow = p.block_tables + (size_t)grp * p.max_blocks;
    tlim = p.max_blocks;
  } else {
    off = p.offsets[grp];
    end = p.offsets[grp + 1];
    off = off < 0 ? 0 : (off > p.num_members ? p.num_members : off);
    end = end < off ? off : (end > p.num_members ? p.num_members : end);
    int plen = p.prefix_lens[grp];
    plen = plen < 0 ? 0 : (plen > p.max_prefix_blocks * BS ? p.max_prefix_blocks * BS : plen);
    ltok = plen / kTile * kTile;
    trow = p.tables + (size_t)grp * p.max_prefix_blocks;
    tlim = p.max_prefix_blocks;
  }
  const int nq = end - off;
  const int ncols = nq * G;
  const int c0 = cb * CW;
  if (c0 >= ncols) return;
  // Prefill: query i (column c, i = c / G) sees tokens < ltok - nq + i + 1.
  // The workgroup's columns span limits lim_lo .. lim_hi; tokens at or past
  // lim_hi are never needed.
  const int lim_lo = PREFILL ? ltok - nq + c0 / G + 1 : ltok;
  const int lim_hi = PREFILL ? ltok - nq + min(nq - 1, (c0 + CW - 1) / G) + 1 : ltok;
  const int ntile = (lim_hi + kTile - 1) / kTile;
  const int first = part * p.pp_tiles;        // even: pp_tiles is a multiple of 8
  if (first >= ntile) return;
  const int last = min(first + p.pp_tiles, ntile);
  const int nsteps = (last - first + 1) / 2;  // the last may hold one tile
  const int ns_w = nsteps > w ? (nsteps - w + kWaves - 1) / kWaves : 0;
  // The column blocks of one partition read the same tiles: each starts its
  // walk at a different step, so that they do not request the same lines of
  // the same L2 channels at the same time (walks of up to 64 steps).
  const int rot = ns_w > 0 && ns_w <= 64 ? (cb * 5) % ns_w : 0;
  auto walk = [&](int k) { return rot ? (k + rot < ns_w ? k + rot : k + rot - ns_w) : k; };

  // Table entries of step c + lane of this wave (TPS per step), clamped.
  auto load_tv = [&](int c, int *tv) {
    const int step = w + walk(c + lane < ns_w ? c + lane : 0) * kWaves;
    const int e0 = (first / 2 + step) * TPS;
#pragma unroll
    for (int e = 0; e < TPS; ++e) tv[e] = trow[e0 + e < tlim ? e0 + e : tlim - 1];
  };
  int tv_next[TPS];
  load_tv(0, tv_next);

  // Query columns: column c0 + 32*nb + n is head kvh*G + (c % G) of member
  // c / G (shared prefix), or of query row off + c / G (prefill); col_seq is
  // the row of q (and of the output).  Columns past the end repeat column 0.
  int col_seq[NB2], col_head[NB2], col_lim[NB2];
  bool col_ok[NB2];
#pragma unroll
  for (int nb = 0; nb < NB2; ++nb) {
    const int c = c0 + 32 * nb + n;
    col_ok[nb] = c < ncols;
    const int cc = col_ok[nb] ? c : 0;
    if constexpr (PREFILL) {
      col_seq[nb] = off + cc / G;
      col_lim[nb] = ltok - nq + cc / G + 1;
    } else {
      const int sq = p.members[off + cc / G];
      col_ok[nb] = col_ok[nb] && (unsigned)sq < (unsigned)p.num_seqs;
      col_seq[nb] = (unsigned)sq < (unsigned)p.num_seqs ? sq : 0;
      col_lim[nb] = ltok;
    }
    col_head[nb] = kvh * G + cc % G;
  }
  // B operands: q dims of MFMA kk for lane half h (see the K order above)
  h8 qf[NB2][NKK];
#pragma unroll
  for (int nb = 0; nb < NB2; ++nb) {
    const _Float16 *qr = reinterpret_cast<const _Float16 *>(p.q) +
                         ((size_t)col_seq[nb] * H + col_head[nb]) * D;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      const int d0 = QUANT ? 16 * (2 * (kk / 2) + h) + 8 * (kk % 2) : 16 * kk + 8 * h;
      qf[nb][kk] = __builtin_bit_cast(h8, load16(reinterpret_cast<const uint8_t *>(qr + d0)));
    }
  }
  float m[NB2], l[NB2];
  f16v acc[NB2][NT];
  float psum[NB2];   // int8: sum of the fp16 weights P' of this lane's rows
#pragma unroll
  for (int nb = 0; nb < NB2; ++nb) {
    m[nb] = -INFINITY;
    l[nb] = 0.0f;
    psum[nb] = 0.0f;
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[nb][t] = f16v{};
  }
  // Headroom (base-2 units) a column's maximum may rise before the running
  // state is rescaled: the weights exp2(x - m) stay below kWMax = 2^kTau
  // (with the rounding of fast_exp2).  Quantized V folds its scale times the
  // wave's boost into the fp16 weights (lower_boost keeps them below fp16's
  // largest value); a smaller headroom there keeps the boost high.
  constexpr float kTau = QUANT ? 2.0f : 8.0f;
  constexpr float kWMax = QUANT ? 4.0f * 1.0001f : 256.0f * 1.0001f;
  bool fresh = true;
  float vboost = kVBoost0;                      // quantized V: the wave's boost
  float vlim = kFoldMax / (kWMax * kVBoost0);   // and the largest scale it admits

  const size_t kv_head_off = (size_t)kvh * SLICE;
  const size_t block_stride = (size_t)p.num_kv_heads * SLICE;

  struct Slot {
    bool ok;
    bool half;   // the step holds one tile only
    int t0;      // first token of the step
  };

  // Block (and tile within the block) of token tt (0..31) of a step whose
  // table entries are e[0..TPS-1]; *row receives its row in the stored tile.
  auto locate = [&](const int *e, int tt, int *row, size_t *tile_off) {
    if constexpr (BS == 32) {
      *row = tt & 15;
      *tile_off = (size_t)(tt >> 4) * (TB * D * EB);
      return e[0];
    } else if constexpr (BS == 16) {
      *row = tt & 15;
      *tile_off = 0;
      return e[tt >> 4];
    } else {
      *row = tt & 7;
      *tile_off = 0;
      return e[tt >> 3];
    }
  };

  auto issue = [&](const int *tv, int j, int step_tile, int slot, Slot &sl) {
    // entries past the data (padding) are replaced by the step's first,
    // whose data is read in their place; a missing second tile is read from
    // the first
    sl.half = step_tile + 1 >= last;
    sl.t0 = step_tile * kTile;
    const int left = ltok - sl.t0;   // tokens of data from the step's start
    int used = BS >= 32 ? 1 : (left + BS - 1) / BS;
    used = used < 1 ? 1 : (used > TPS ? TPS : used);
    int e[TPS];
    bool ok = true;
#pragma unroll
    for (int k = 0; k < TPS; ++k) {
      e[k] = __builtin_amdgcn_readlane(tv[k < used ? k : 0], j);
      ok = ok && (unsigned)e[k] < (unsigned)p.num_blocks;
    }
    sl.ok = ok;
#pragma unroll
    for (int k = 0; k < TPS; ++k) e[k] = ok ? e[k] : 0;
    // a missing second tile is read from the first (its weights are zero)
    const int tmask = sl.half ? 15 : 31;
    // K: token n
    {
      int row;
      size_t toff;
      const int b = locate(e, n & tmask, &row, &toff);
      const uint8_t *kb = p.k_cache + (size_t)b * block_stride + kv_head_off + toff;
#pragma unroll
      for (int k = 0; k < KLD; ++k)
        load16_to_lds(kb + (size_t)(((2 * k + h) * TB + row) * 16), &lds_ring[w][slot][k][0]);
    }
    // V: tile kc, token quads 4h and 8 + 4h
#pragma unroll
    for (int kc = 0; kc < 2; ++kc) {
#pragma unroll
      for (int qd = 0; qd < 2; ++qd) {
        int row;
        size_t toff;
        const int tt = ((16 * kc) & tmask) + 8 * qd + 4 * h;
        const int b = locate(e, tt, &row, &toff);
        const uint8_t *vb = p.v_cache + (size_t)b * block_stride + kv_head_off + toff;
        if constexpr (QUANT) {
          const int grp4 = (D == 128) ? n : (n & 15);   // dims 4*grp4 .. +3
          load16_to_lds(vb + (size_t)((grp4 * (TB / 4) + row / 4) * 16),
                        &lds_ring[w][slot][KLD + 2 * kc + qd][0]);
        } else {
#pragma unroll
          for (int gg = 0; gg < NG; ++gg)
            load16_to_lds(vb + (size_t)(((32 * gg + n) * TB + row) * 4),
                          &lds_ring[w][slot][KLD + (kc * NG + gg) * 2 + qd][0]);
        }
      }
    }
    if constexpr (QUANT) {
      // lane: K (lanes 0-15 of each half) or V (16-31) scales of tokens 2i, 2i+1
      const int i = n & 15;
      int row;
      size_t toff;
      const int b = locate(e, (2 * i) & tmask, &row, &toff);
      const int tile_in_block = (int)(toff / (TB * D * EB));
      const uint16_t *sc = (n < 16 ? p.k_scale : p.v_scale) +
                           ((size_t)b * p.num_kv_heads + kvh) * BS + tile_in_block * kTile + row;
      __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void *)sc,
                                       (__attribute__((address_space(3))) void *)&lds_sc[w][slot][0],
                                       4, 0, 0);
    }
  };

  auto consume = [&](int slot, const Slot &sl) {
    if (!sl.ok) return;   // a table entry outside the pool: step skipped
    const uint32_t base = (uint32_t)(size_t)(
        (__attribute__((address_space(3))) const u4 *)&lds_ring[w][slot][0][lane]);
    u4 raw[KLD + VLD];
    lds_read_row<0, KLD + VLD, 1024>(base, raw);
    u2 ksw[4], vsw[4];
    if constexpr (QUANT) {
      // scales of this lane's tokens 8j + 4h + 0..3: words 4j + 2h, +1
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const uint32_t a = (uint32_t)(size_t)(
            (__attribute__((address_space(3))) const uint32_t *)&lds_sc[w][slot][4 * jj + 2 * h]);
        asm volatile("ds_read_b64 %0, %1" : "=v"(ksw[jj]) : "v"(a));
        asm volatile("ds_read_b64 %0, %1 offset:64" : "=v"(vsw[jj]) : "v"(a));
      }
    }
    lds_wait();
#pragma unroll
    for (int i = 0; i < KLD + VLD; ++i) after_wait(raw[i]);
    float ksf[16], vsf[16];
    if constexpr (QUANT) {
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        asm volatile("" : "+v"(ksw[jj]));
        asm volatile("" : "+v"(vsw[jj]));
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          ksf[4 * jj + v] = (float)as_h2(ksw[jj][v >> 1])[v & 1];
          vsf[4 * jj + v] = (float)as_h2(vsw[jj][v >> 1])[v & 1];
        }
      }
    }
    // A operands
    h8 ka[NKK];
    if constexpr (QUANT) {
#pragma unroll
      for (int k = 0; k < KLD; ++k) k_codes16<KV>(raw[k], ka[2 * k], ka[2 * k + 1]);
    } else {
#pragma unroll
      for (int k = 0; k < KLD; ++k) ka[k] = __builtin_bit_cast(h8, raw[k]);
    }
    h8 va[2][NT];   // [kc][output tile]
#pragma unroll
    for (int kc = 0; kc < 2; ++kc) {
      if constexpr (QUANT) {
        const u4 a = raw[KLD + 2 * kc], b = raw[KLD + 2 * kc + 1];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const h4 lo = codes4_to_h4<KV>(a[e]), hi = codes4_to_h4<KV>(b[e]);
          va[kc][e] = h8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        }
      } else {
#pragma unroll
        for (int gg = 0; gg < NG; ++gg) {
          const u4 a = raw[KLD + (kc * NG + gg) * 2], b = raw[KLD + (kc * NG + gg) * 2 + 1];
          const u4 ev = u4{__builtin_amdgcn_perm(a[1], a[0], 0x05040100u),
                           __builtin_amdgcn_perm(a[3], a[2], 0x05040100u),
                           __builtin_amdgcn_perm(b[1], b[0], 0x05040100u),
                           __builtin_amdgcn_perm(b[3], b[2], 0x05040100u)};
          const u4 od = u4{__builtin_amdgcn_perm(a[1], a[0], 0x07060302u),
                           __builtin_amdgcn_perm(a[3], a[2], 0x07060302u),
                           __builtin_amdgcn_perm(b[1], b[0], 0x07060302u),
                           __builtin_amdgcn_perm(b[3], b[2], 0x07060302u)};
          va[kc][2 * gg] = __builtin_bit_cast(h8, ev);
          va[kc][2 * gg + 1] = __builtin_bit_cast(h8, od);
        }
      }
    }
    // Prefill: steps that reach a causal limit or the end of the data mask
    // per element (token t0 + 8j + 4h + v of element 4j + v): scores of
    // tokens at or past the column's limit, and V (and its scales) of tokens
    // past the data, which may be unwritten slots.
    const bool edge = PREFILL && sl.t0 + 32 > lim_lo;
    if (edge) {
#pragma unroll
      for (int kc = 0; kc < 2; ++kc)
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int tok = sl.t0 + 16 * kc + (i < 4 ? 4 * h + i : 8 + 4 * h + (i - 4));
          if (tok >= ltok) {
#pragma unroll
            for (int t = 0; t < NT; ++t) va[kc][t][i] = (_Float16)0.0f;
          }
        }
      if constexpr (QUANT) {
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (sl.t0 + 8 * (i / 4) + 4 * h + (i % 4) >= ltok) vsf[i] = 0.0f;
      }
    }
    if constexpr (QUANT) {
      // A V scale above what the wave's boost admits for weights up to
      // 2^kTau (never one of an fp16 value at the initial boost of an E4M3
      // cache): lower the boost first.  Lane (n, h) holds the scales of the
      // step's tokens 8j + 4h + v, the same for every n.
      float smax = 0.0f;
#pragma unroll
      for (int i = 0; i < 16; ++i) smax = fmaxf(smax, fabsf(vsf[i]));
      if (__builtin_expect(__builtin_amdgcn_ballot_w64(smax > vlim) != 0, 0)) {
        const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(smax),
                                                        __float_as_uint(smax), false, false);
        const float sw = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
        const float nbst = lower_boost(vboost, sw, kWMax);
        const float f = nbst / vboost;
#pragma unroll
        for (int nb = 0; nb < NB2; ++nb) {
#pragma unroll
          for (int t = 0; t < NT; ++t) acc[nb][t] *= f;
          if constexpr (KV == PKV_I8) psum[nb] *= f;
        }
        vboost = nbst;
        vlim = kFoldMax / (kWMax * nbst);
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) vsf[i] *= vboost;
    }
    // Scores.  Base-2 score x = k * s (fp16 cache: k = qk_scale for every
    // token, so the block maximum is taken on the raw s and the scale is
    // applied inside the exponent's fma; quantized caches: the per-token K
    // scale makes x explicit).
    float x[NB2][16], mn[NB2];
    uint32_t dead[NB2];   // bit i: element i takes no part (masked token)
    bool over = false;
    const float ks = p.qk_scale;
    const bool masked = edge || sl.half;   // wave-uniform
    // the column blocks' accumulation chains interleaved, so that consecutive
    // MFMAs do not wait on each other
    f16v scs[NB2];
#pragma unroll
    for (int nb = 0; nb < NB2; ++nb) scs[nb] = f16v{};
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk)
#pragma unroll
      for (int nb = 0; nb < NB2; ++nb)
        scs[nb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ka[kk], qf[nb][kk], scs[nb], 0, 0, 0);
#pragma unroll
    for (int nb = 0; nb < NB2; ++nb) {
      f16v &sc = scs[nb];
      // masked elements: rows 16..31 (elements 8..15) of a half step belong
      // to the missing tile; prefill edge steps mask tokens at or past the
      // column's causal limit.  They are left out of the maximum, and their
      // weights are zeroed below.
      dead[nb] = sl.half ? 0xFF00u : 0u;
      if (edge) {
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (sl.t0 + 8 * (i / 4) + 4 * h + (i % 4) >= col_lim[nb]) dead[nb] |= 1u << i;
      }
      float bm;
      if constexpr (QUANT) {
        bm = -INFINITY;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          x[nb][i] = sc[i] * ks * ksf[i];
          if (!masked || !((dead[nb] >> i) & 1u)) bm = fmaxf(bm, x[nb][i]);
        }
      } else {
#pragma unroll
        for (int i = 0; i < 16; ++i) x[nb][i] = sc[i];
        // wave-uniform: the largest score, or the smallest (negative scale);
        // with every element masked e stays infinite and bm is -inf (or NaN
        // for a zero scale, which the maximum below ignores)
        float e = ks >= 0.0f ? -INFINITY : INFINITY;
        if (ks >= 0.0f) {
#pragma unroll
          for (int i = 0; i < 16; ++i)
            if (!masked || !((dead[nb] >> i) & 1u)) e = fmaxf(e, sc[i]);
        } else {
#pragma unroll
          for (int i = 0; i < 16; ++i)
            if (!masked || !((dead[nb] >> i) & 1u)) e = fminf(e, sc[i]);
        }
        bm = e * ks;
      }
      const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(bm), __float_as_uint(bm),
                                                      false, false);
      bm = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
      mn[nb] = fmaxf(m[nb], bm);
      over = over || mn[nb] > m[nb] + kTau;
    }
    if (fresh) {
#pragma unroll
      for (int nb = 0; nb < NB2; ++nb) m[nb] = mn[nb];
      fresh = false;
    } else if (__builtin_amdgcn_ballot_w64(over) != 0) {
#pragma unroll
      for (int nb = 0; nb < NB2; ++nb) {
        const float alpha = fast_exp2(m[nb] - mn[nb]);
        l[nb] *= alpha;
#pragma unroll
        for (int t = 0; t < NT; ++t) acc[nb][t] *= alpha;
        if constexpr (KV == PKV_I8) psum[nb] *= alpha;
        m[nb] = mn[nb];
      }
    }
#pragma unroll
    for (int nb = 0; nb < NB2; ++nb) {
      float pr[16];
#pragma unroll
      for (int i = 0; i < 16; ++i)
        pr[i] = QUANT ? fast_exp2(x[nb][i] - m[nb]) : fast_exp2(fmaf(x[nb][i], ks, -m[nb]));
      if (masked) {
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if ((dead[nb] >> i) & 1u) pr[i] = 0.0f;
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        l[nb] += pr[i];
        if constexpr (QUANT) pr[i] *= vsf[i];
      }
#pragma unroll
      for (int kc = 0; kc < 2; ++kc) {
        const h8 pb = h8{(_Float16)pr[8 * kc], (_Float16)pr[8 * kc + 1], (_Float16)pr[8 * kc + 2],
                         (_Float16)pr[8 * kc + 3], (_Float16)pr[8 * kc + 4],
                         (_Float16)pr[8 * kc + 5], (_Float16)pr[8 * kc + 6],
                         (_Float16)pr[8 * kc + 7]};
        if constexpr (KV == PKV_I8) {   // the weights exactly as the MFMA sees them
#pragma unroll
          for (int i = 0; i < 8; ++i) psum[nb] += (float)pb[i];
        }
#pragma unroll
        for (int t = 0; t < NT; ++t)
          acc[nb][t] = __builtin_amdgcn_mfma_f32_32x32x16_f16(va[kc][t], pb, acc[nb][t], 0, 0, 0);
      }
    }
  };

  for (int cc = 0; cc < ns_w; cc += 64) {
    const int nc = min(64, ns_w - cc);
    int tv[TPS];
#pragma unroll
    for (int k = 0; k < TPS; ++k) tv[k] = tv_next[k];
    auto step_tile = [&](int j) { return first + 2 * (w + walk(cc + j) * kWaves); };
    Slot ring[NR];
#pragma unroll
    for (int j = 0; j < NR; ++j) {
      const int jj = j < nc ? j : nc - 1;
      issue(tv, jj, step_tile(jj), j, ring[j]);
    }
    int k0 = 0;
    for (; k0 + 2 * NR <= nc; k0 += NR) {
#pragma unroll
      for (int j = 0; j < NR; ++j) {
        wait_vmcnt<(NR - 1) * LPS>();
        consume(j, ring[j]);
        asm volatile("" ::: "memory");
        issue(tv, k0 + j + NR, step_tile(k0 + j + NR), j, ring[j]);
      }
    }
#pragma unroll
    for (int j = 0; j < NR; ++j) {
      if (k0 + j < nc) {
        wait_vmcnt<0>();
        consume(j, ring[j]);
      }
      asm volatile("" ::: "memory");
      if (k0 + j + NR < nc) issue(tv, k0 + j + NR, step_tile(k0 + j + NR), j, ring[j]);
    }
#pragma unroll
    for (int j = 0; j < NR; ++j)
      if (k0 + NR + j < nc) {
        wait_vmcnt<0>();
        consume(j, ring[j]);
      }
    wait_vmcnt<0>();
    if (cc + 64 < ns_w) load_tv(cc + 64, tv_next);
  }

  // ---- combine the waves: maxima and sums, then the accumulators ----
#pragma unroll
  for (int nb = 0; nb < NB2; ++nb) {
    if constexpr (KV == PKV_I8) {   // biased codes: subtract 1152 * (column's sum of P')
      const auto ps = __builtin_amdgcn_permlane32_swap(__float_as_uint(psum[nb]),
                                                       __float_as_uint(psum[nb]), false, false);
      const float bias = kI8Bias * (__uint_as_float(ps[0]) + __uint_as_float(ps[1]));
#pragma unroll
      for (int t = 0; t < NT; ++t) acc[nb][t] -= bias;
    }
    const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(l[nb]),
                                                    __float_as_uint(l[nb]), false, false);
    l[nb] = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    if (h == 0) {
      lds_m[w][32 * nb + n] = m[nb];
      lds_l[w][32 * nb + n] = l[nb];
    }
  }
  __syncthreads();
  float Mx[NB2], den[NB2];
#pragma unroll
  for (int nb = 0; nb < NB2; ++nb) {
    const int col = 32 * nb + n;
    float M = lds_m[0][col];
#pragma unroll
    for (int ww = 1; ww < kWaves; ++ww) M = fmaxf(M, lds_m[ww][col]);
    float z = 0.0f;
#pragma unroll
    for (int ww = 0; ww < kWaves; ++ww) {
      const float mw = lds_m[ww][col];
      z += mw == -INFINITY ? 0.0f : exp2f(mw - M) * lds_l[ww][col];
    }
    Mx[nb] = M;
    den[nb] = z;
    float f = m[nb] == -INFINITY ? 0.0f : exp2f(m[nb] - M);
    if constexpr (QUANT) f *= 1.0f / vboost;   // undo the wave's V-scale boost
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[nb][t] *= f;
  }
  // every wave's scaled accumulators to LDS, then wave w reduces and writes
  // the output rows 8w + 4h .. 8w + 4h + 3 of every tile (elements 4w .. 4w+3)
#pragma unroll
  for (int nb = 0; nb < NB2; ++nb)
#pragma unroll
    for (int t = 0; t < NT; ++t) lds_acc[w][nb][t][lane] = acc[nb][t];
  __syncthreads();
  const int jj = w;          // row group of this wave
  const int r0 = 8 * jj + 4 * h;
#pragma unroll
  for (int nb = 0; nb < NB2; ++nb) {
    if (!col_ok[nb]) continue;
    // prefill with a single partition writes the output row itself
    const bool direct = PREFILL && p.num_pparts == 1;
    const size_t orow = (size_t)col_seq[nb] * H + col_head[nb];
    const size_t row = orow * p.ws_stride + p.ws_pre + part;
    const float inv = 1.0f / den[nb];
    float *dst = direct ? nullptr : p.ws_o + row * D;
    f4 o[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      f4 a = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ww = 0; ww < kWaves; ++ww) {
        const float *src = reinterpret_cast<const float *>(&lds_acc[ww][nb][t][lane]) + 4 * jj;
        a += *reinterpret_cast<const f4 *>(src);
      }
      o[t] = a * inv;
    }
    // element 4j + v of tile t is row 8j + 4h + v:
    //   2-byte V, t = 2G + parity: dim 2(32G + row) + parity
    //   1-byte V, t = e:           dim 4 row + e
    // 4 consecutive output elements at element offset e0 of the row
    auto put4 = [&](int e0, f4 v) {
      if (direct) {
        if constexpr (OUT == PKV_F32)
          *reinterpret_cast<f4 *>(reinterpret_cast<float *>(p.out) + orow * D + e0) = v;
        else
          *reinterpret_cast<h4 *>(reinterpret_cast<_Float16 *>(p.out) + orow * D + e0) =
              h4{to_f16_out(v[0]), to_f16_out(v[1]), to_f16_out(v[2]), to_f16_out(v[3])};
      } else {
        *reinterpret_cast<f4 *>(dst + e0) = v;
      }
    };
    if constexpr (QUANT) {
      if (!(D == 64 && r0 >= 16)) {   // rows past the 16 dim groups of D = 64
#pragma unroll
        for (int v = 0; v < 4; ++v) put4(4 * (r0 + v), f4{o[0][v], o[1][v], o[2][v], o[3][v]});
      }
    } else {
#pragma unroll
      for (int gg = 0; gg < NG; ++gg) {
        const int e0 = 2 * (32 * gg + r0);
        put4(e0, f4{o[2 * gg][0], o[2 * gg + 1][0], o[2 * gg][1], o[2 * gg + 1][1]});
        put4(e0 + 4, f4{o[2 * gg][2], o[2 * gg + 1][2], o[2 * gg][3], o[2 * gg + 1][3]});
      }
    }
    if (!direct && w == 0 && h == 0) p.ws_lse[row] = Mx[nb] + log2f(den[nb]);
  }
}

template <int KV, int D, int BS>
hipError_t launch_prefix_typed(const PrefixParams &p, hipStream_t stream) {
  if constexpr (KV == PKV_F32)
    hipLaunchKernelGGL((prefix_kernel<D, BS, 2>), dim3((unsigned)prefix_grid(p)),
                       dim3(64 * kWaves), 0, stream, p);
  else
    hipLaunchKernelGGL((prefix32_kernel<KV, D, BS, kModeShared, PKV_F32>),
                       dim3((unsigned)prefix_grid(p)), dim3(64 * kWaves), 0, stream, p);
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

// Merge of prefill partials (several partitions): a thread owns 4 elements of
// one (query row, head) row; the row's sequence is found by bisection over
// query_offsets, and its partitions are those that start below its causal
// limit.  One pass over the partials with a running (max, sum, weighted sum).
template <int D, int OUT>
__global__ __launch_bounds__(256) void prefill_merge_kernel(PrefixParams p) {
  constexpr int TPH = D / 4;
  constexpr int RPW = 256 / TPH;
  const int t = threadIdx.x;
  const int rl = t / TPH, dv = t % TPH;
  const int row = blockIdx.x * RPW + rl;
  if (row >= p.num_query_tokens * p.num_heads) return;
  const int qr = row / p.num_heads;
  int lo = 0, hi = p.num_seqs;   // the last sequence whose first query row is <= qr
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (p.query_offsets[mid] <= qr) lo = mid; else hi = mid;
  }
  const int s = lo;
  int off = p.query_offsets[s], end = p.query_offsets[s + 1];
  off = off < 0 ? 0 : (off > p.num_query_tokens ? p.num_query_tokens : off);
  end = end < off ? off : (end > p.num_query_tokens ? p.num_query_tokens : end);
  int L = p.seq_lens[s];
  L = L < 0 ? 0 : (L > p.max_blocks * p.block_size ? p.max_blocks * p.block_size : L);
  if (end - off > L) end = off + L;
  const int i = qr - off;
  if (i < 0 || i >= end - off) return;   // not a query row of s (the pass wrote nothing)
  const int lim = L - (end - off) + i + 1;
  const int np = ((lim + kTile - 1) / kTile + p.pp_tiles - 1) / p.pp_tiles;
  const size_t base = (size_t)row * p.ws_stride;
  const f4 *o = reinterpret_cast<const f4 *>(p.ws_o + base * D) + dv;
  float m = -INFINITY, z = 0.0f;
  f4 acc = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
  for (int q = 0; q < np; ++q) {
    const float lq = p.ws_lse[base + q];
    const f4 oq = o[(size_t)q * (D / 4)];
    const float mn = fmaxf(m, lq);
    const float a = exp2f(m - mn), b = exp2f(lq - mn);
    acc = acc * a + oq * b;
    z = z * a + b;
    m = mn;
  }
  const f4 r = acc * (1.0f / z);
  const size_t oi = (size_t)row * D + 4 * dv;
  if constexpr (OUT == PKV_F32)
    *reinterpret_cast<f4 *>(reinterpret_cast<float *>(p.out) + oi) = r;
  else
    *reinterpret_cast<h4 *>(reinterpret_cast<_Float16 *>(p.out) + oi) =
        h4{to_f16_out(r[0]), to_f16_out(r[1]), to_f16_out(r[2]), to_f16_out(r[3])};
}

template <int KV, int D, int BS, int OUT>
hipError_t launch_prefill_typed(const PrefixParams &p, hipStream_t stream) {
  hipLaunchKernelGGL((prefix32_kernel<KV, D, BS, kModePrefill, OUT>),
                     dim3((unsigned)prefix_grid(p)), dim3(64 * kWaves), 0, stream, p);
  return hipGetLastError();
}

template <int KV, int D, int OUT>
hipError_t launch_prefill_bs(const PrefixParams &p, int block_size, hipStream_t stream) {
  switch (block_size) {
    case 8: return launch_prefill_typed<KV, D, 8, OUT>(p, stream);
    case 32: return launch_prefill_typed<KV, D, 32, OUT>(p, stream);
    default: return launch_prefill_typed<KV, D, 16, OUT>(p, stream);
  }
}

template <int KV, int OUT>
hipError_t launch_prefill_d(const PrefixParams &p, int head_dim, int block_size,
                            hipStream_t stream) {
  return head_dim == 64 ? launch_prefill_bs<KV, 64, OUT>(p, block_size, stream)
                        : launch_prefill_bs<KV, 128, OUT>(p, block_size, stream);
}

template <int KV>
hipError_t launch_prefill_o(const PrefixParams &p, int out_dtype, int head_dim, int block_size,
                            hipStream_t stream) {
  return out_dtype == PKV_F32 ? launch_prefill_d<KV, PKV_F32>(p, head_dim, block_size, stream)
                              : launch_prefill_d<KV, PKV_F16>(p, head_dim, block_size, stream);
}

template <int D, int OUT>
hipError_t launch_prefill_merge_typed(const PrefixParams &p, hipStream_t stream) {
  constexpr int RPW = 256 / (D / 4);
  const int rows = p.num_query_tokens * p.num_heads;
  hipLaunchKernelGGL((prefill_merge_kernel<D, OUT>), dim3((rows + RPW - 1) / RPW), dim3(256), 0,
                     stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill(const PrefixParams &p, int cache_dtype, int out_dtype, int head_dim,
                          int block_size, hipStream_t stream) {
  hipError_t err;
  switch (cache_dtype) {
    case PKV_F16:
      err = launch_pipe(p, true, out_dtype, head_dim, block_size, 1, stream);
      break;
    case PKV_I8: err = launch_prefill_o<PKV_I8>(p, out_dtype, head_dim, block_size, stream); break;
    default: err = launch_prefill_o<PKV_E4M3>(p, out_dtype, head_dim, block_size, stream); break;
  }
  if (err != hipSuccess || p.num_pparts <= 1) return err;
  if (out_dtype == PKV_F32)
    return head_dim == 64 ? launch_prefill_merge_typed<64, PKV_F32>(p, stream)
                          : launch_prefill_merge_typed<128, PKV_F32>(p, stream);
  return head_dim == 64 ? launch_prefill_merge_typed<64, PKV_F16>(p, stream)
                        : launch_prefill_merge_typed<128, PKV_F16>(p, stream);
}

hipError_t launch_prefix(const PrefixParams &p, int cache_dtype, int head_dim, int block_size,
                         hipStream_t stream) {
  switch (cache_dtype) {
    case PKV_F32: return launch_prefix_d<PKV_F32>(p, head_dim, block_size, stream);
    case PKV_F16: return launch_pipe(p, false, PKV_F32, head_dim, block_size, 2, stream);
    case PKV_I8: return launch_prefix_d<PKV_I8>(p, head_dim, block_size, stream);
    default: return launch_prefix_d<PKV_E4M3>(p, head_dim, block_size, stream);
  }
}

}  // namespace pkv
