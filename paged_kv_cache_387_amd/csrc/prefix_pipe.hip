// Multi-query attention pass over the paged cache for fp16 caches on gfx950,
// with the matrix cores and the vector ALUs working at the same time.
//
// It computes what prefix32_kernel (prefix.hip) computes, for units with many
// query columns: a (sequence, kv head) of a chunked prefill, whose columns are
// its query tokens times the G query heads of the kv head, each attending
// causally over the sequence's cached tokens ("KVcache-learning",
// fairy2021.github.io, s01 attention and s04: a new token sees the cache and
// the new tokens before it); or a (group, kv head) of a shared prefix, whose
// columns are the members' query heads (s05 and s08: forked sequences share
// their common blocks).  Per column, online softmax over 32-token steps: the
// running maximum m, the sum l of the weights exp2(x - m) and the weighted V
// sum; out = o / l, or the partial (o / l, m + log2 l) for a merge by
// log-sum-exp ("LLM inference: vLLM PagedAttention", jsqmd.com, section 4.1).
//
// Work decomposition.  A workgroup of four waves takes 64 * CG query columns of
// one unit and one partition of its tokens; the waves form TG = 4 / CG token
// groups of CG waves.  A token group walks every TG-th 32-token step of the
// partition, and its CG waves take 64 columns each.  They load each step once,
// between them (each wave CG-th of the step's 16-byte rows, straight into LDS),
// into a ring of NR steps that all of them then read: a step's K and V cross
// from L2 once per token group, not once per wave, and the ring is deep enough
// to keep several steps in flight.  With two token groups the pair of waves
// holding the same columns combines its states at the end.
//
// Per wave and step, with the 32x32x16 f16 MFMA (lane l = 32h + n: A row and
// B column l % 32, k = 8h .. 8h+7; D column n, rows 8j + 4h + v in element
// 4j + v), the same operand layouts as prefix32_kernel:
//   S^T[32 tokens][32 columns] = K q      D/16 MFMAs per column block
//   O^T[D][32 columns] += V^T P^T         2 * D/32 MFMAs per column block
// The walk is a two-stage pipeline: while step k's softmax (vector ALU work)
// runs, step k+1's q.K MFMAs are already in the matrix core; step k's P.V
// MFMAs follow.  The running maximum moves only when a column's maximum rises
// by more than 8 (base 2), which keeps the rescale of the accumulators out of
// the common path.
#include "attn_common.h"
#include "lds_ring.h"

namespace pkv {
namespace {

typedef float f16v __attribute__((ext_vector_type(16)));

template <int V>
struct IC {
  static constexpr int value = V;
};

template <int D, int BS, int MODE, int OUT, int TG>
__global__ __launch_bounds__(64 * kWaves, 1) void pipe32_kernel(PrefixParams p) {
  constexpr int CG = kWaves / TG;              // waves of one token group
  constexpr int TB = BS < kTile ? BS : kTile;  // tokens of a stored tile
  constexpr int TPS = BS >= 32 ? 1 : 32 / BS;  // table entries per 32-token step
  constexpr int NKK = D / 16;                  // q.K MFMAs per column block = K rows
  constexpr int NG = D / 64;                   // groups of 32 V column pairs
  constexpr int VLD = 4 * NG;                  // V rows of a step
  constexpr int NT = 2 * NG;                   // output tiles (32 rows) per column block
  constexpr int LPS = NKK + VLD;               // 16-byte rows (x 64 lanes) of a step
  constexpr int LPW = LPS / CG;                // of them loaded by each wave
  constexpr int NR = 4;                        // ring depth (steps)
  constexpr int NB2 = 2;                       // column blocks of 32 per wave
  constexpr int CW = 32 * NB2;                 // columns per wave
  constexpr int EB = 2;
  constexpr bool PREFILL = MODE == kModePrefill;
  static_assert(kWaves == 4 && (TG == 1 || TG == 2), "waves");
  static_assert(LPS % CG == 0 && NKK % CG == 0, "row split");
  static_assert(4 * LPW < 64, "wait count");
  static_assert(NKK + VLD <= 16 && VLD < 16, "LDS read counts");

  // The ring: per token group, NR steps of LPS rows of 64 lanes x 16 bytes,
  // each lane's 16 bytes as the lane reads them.  With two token groups the
  // same memory then holds group 1's accumulators for the combine.
  constexpr int kRingU4 = TG * NR * LPS * 64;
  constexpr int kAccU4 = TG > 1 ? CG * NB2 * NT * 4 * 64 : 0;
  __shared__ u4 lds_raw[kRingU4 > kAccU4 ? kRingU4 : kAccU4];
  __shared__ float lds_m[TG > 1 ? CG * CW : 1];
  __shared__ float lds_l[TG > 1 ? CG * CW : 1];

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int cgi = w % CG;
  const int tgi = w / CG;
  const int n = lane & 31;
  const int h = lane >> 5;

  // Workgroup -> (unit, column block, partition); unit u runs on die u % kXcds.
  const int bid = blockIdx.x;
  const int die_slot = bid / kXcds;
  const int ugroups = unit_groups(p.num_units);
  const int per_part = ugroups * p.col_blocks;
  const int part = die_slot / per_part;
  const int rem = die_slot - part * per_part;
  const int cb = rem / ugroups;
  const int u = (rem - cb * ugroups) * kXcds + bid % kXcds;
  if (u >= p.num_units || part >= p.num_pparts) return;
  const int grp = u / p.num_kv_heads;   // group, or sequence
  const int kvh = u - grp * p.num_kv_heads;
  const int G = p.group;
  const int H = p.num_heads;

  int off, end, ltok, tlim;
  const int32_t *trow;
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
  const int c0 = cb * (CW * CG);
  if (c0 >= ncols) return;
  // Prefill: query i (column c, i = c / G) sees tokens < ltok - nq + i + 1;
  // tokens at or past the workgroup's largest limit are never needed.
  const int lim_hi = PREFILL ? ltok - nq + min(nq - 1, (c0 + CW * CG - 1) / G) + 1 : ltok;
  const int ntile = (lim_hi + kTile - 1) / kTile;
  const int first = part * p.pp_tiles;   // even: pp_tiles is a multiple of 8
  if (first >= ntile) return;
  const int last = min(first + p.pp_tiles, ntile);
  const int nsteps = (last - first + 1) / 2;   // the last may hold one tile
  const int ns_g = nsteps > tgi ? (nsteps - tgi + TG - 1) / TG : 0;   // steps of this group
  const int ns_max = (nsteps + TG - 1) / TG;                           // of group 0

  // This wave's columns wc0 .. wc0 + 63: column wc0 + 32 nb + n is head
  // kvh*G + (c % G) of member / query row c / G.  A wave past the columns
  // still loads its share of every step and meets every barrier.
  const int wc0 = c0 + CW * cgi;
  const bool idle = wc0 >= ncols;
  const int wlim_lo = PREFILL ? ltok - nq + (idle ? 0 : wc0 / G) + 1 : ltok;
  int col_seq[NB2], col_head[NB2], col_lim[NB2];
  bool col_ok[NB2];
#pragma unroll
  for (int nb = 0; nb < NB2; ++nb) {
    const int c = wc0 + 32 * nb + n;
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
  // The base-2 score is x = ks * (q.k).  A negative scale is folded into q
  // (an exact fp16 negation), so that the step's largest x is ks times the
  // largest dot product.
  const float ks = fabsf(p.qk_scale);
  const uint32_t qneg = p.qk_scale < 0.0f ? 0x80008000u : 0u;
  // q is requested here and moved into place after the ring's first steps
  // are requested, so that the two round trips overlap.
  u4 qraw[NB2][NKK];
  h8 qf[NB2][NKK];
#pragma unroll
  for (int nb = 0; nb < NB2; ++nb) {
    const _Float16 *qr = reinterpret_cast<const _Float16 *>(p.q) +
                         ((size_t)col_seq[nb] * H + col_head[nb]) * D;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk)
      qraw[nb][kk] = load16(reinterpret_cast<const uint8_t *>(qr + 16 * kk + 8 * h));
  }

  float m[NB2], l[NB2];
  f16v acc[NB2][NT];
#pragma unroll
  for (int nb = 0; nb < NB2; ++nb) {
    m[nb] = -INFINITY;
    l[nb] = 0.0f;
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[nb][t] = f16v{};
  }
  // Headroom (base 2) a column's maximum may rise before the state is
  // rescaled: the weights stay below 2^8 (and fp16 holds them).
  constexpr float kTau = 8.0f;
  bool fresh = true;

  const size_t kv_head_off = (size_t)kvh * (BS * D * EB);
  const size_t block_stride = (size_t)p.num_kv_heads * (BS * D * EB);
  u4(*ring)[LPS][64] = reinterpret_cast<u4(*)[LPS][64]>(&lds_raw[0]) + tgi * NR;

  // Table entries of the group's step k (TPS of them, clamped to the row),
  // read with scalar loads: the row is never written during the pass.  They
  // are read one issue ahead (unconditionally, so that no register value is
  // merged from two paths), which hides their latency under a step and keeps
  // them out of the vector-memory count the ring's waits rely on.
  const __attribute__((address_space(4))) int32_t *trow_s =
      (const __attribute__((address_space(4))) int32_t *)trow;
  auto entries = [&](int k, int *e) {
    const int gs = tgi + TG * k;
    const int e0 = (first / 2 + gs) * TPS;
#pragma unroll
    for (int q = 0; q < TPS; ++q) e[q] = trow_s[e0 + q < tlim ? e0 + q : tlim - 1];
  };
  int ent[TPS];   // entries of the next step to issue

  // Block (and tile within it) of token tt (0..31) of a step whose table
  // entries are e[]; *row receives the token's row in the stored tile.
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
  // The rows i = cgi, cgi + CG, ... of a step (i is wave-uniform): K rows
  // (i < NKK: token n, dims 8(2i + h) ..) and V rows (token quads 8qd + 4h
  // of tile kc, column pairs 32gg + n), the layouts of prefix32_kernel.
  auto issue_rows = [&](const int *e, int tmask, int slot) {
#pragma unroll
    for (int ii = 0; ii < LPW; ++ii) {
      const int i = ii * CG + cgi;
      int row;
      size_t toff;
      if (ii < NKK / CG) {
        const int b = locate(e, n & tmask, &row, &toff);
        const uint8_t *kb = p.k_cache + (size_t)b * block_stride + kv_head_off + toff;
        load16_to_lds(kb + (size_t)(((2 * i + h) * TB + row) * 16), &ring[slot][i][0]);
      } else {
        const int iv = i - NKK;
        const int kc = iv / (2 * NG), gg = (iv / 2) % NG, qd = iv % 2;
        const int b = locate(e, ((16 * kc) & tmask) + 8 * qd + 4 * h, &row, &toff);
        const uint8_t *vb = p.v_cache + (size_t)b * block_stride + kv_head_off + toff;
        load16_to_lds(vb + (size_t)(((32 * gg + n) * TB + row) * 4), &ring[slot][i][0]);
      }
    }
  };
  // This wave's rows of the group's step k into ring slot `slot`.  Entries
  // past the data (padding) are replaced by the step's first; a missing
  // second tile is read from the first (its weights are zero).
  auto issue = [&](int k, int slot, const int *ek) {
    const int st = first + 2 * (tgi + TG * k);
    const bool half = st + 1 >= last;
    const int left = ltok - st * kTile;
    int used = BS >= 32 ? 1 : (left + BS - 1) / BS;
    used = used < 1 ? 1 : (used > TPS ? TPS : used);
    // an entry outside the pool reads block 0 instead (its numbers are
    // unspecified; no access leaves the pool)
    int e[TPS];
#pragma unroll
    for (int q = 0; q < TPS; ++q) {
      e[q] = ek[q < used ? q : 0];
      e[q] = (unsigned)e[q] < (unsigned)p.num_blocks ? e[q] : 0;
    }
    const int tmask = half ? 15 : 31;
    issue_rows(e, tmask, slot);
  };

  auto ring_addr = [&](int slot) {
    return (uint32_t)(size_t)(
        (__attribute__((address_space(3))) const u4 *)&ring[slot][0][lane]);
  };
  // S^T blocks of a step from its K rows: two interleaved accumulation
  // chains, so that consecutive MFMAs do not wait on each other.
  auto qk = [&](const u4 *kr, f16v *s) {
#pragma unroll
    for (int nb = 0; nb < NB2; ++nb) s[nb] = f16v{};
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk)
#pragma unroll
      for (int nb = 0; nb < NB2; ++nb)
        s[nb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(h8, kr[kk]),
                                                       qf[nb][kk], s[nb], 0, 0, 0);
  };
  // Weights of a step (dot products s, first token t0) as the fp16 P^T
  // operands, with the running state moved first where a column's maximum
  // rose by more than kTau.  MASKED: element 4j + v (token t0 + 8j + 4h + v)
  // takes no part when it lies in a missing second tile (half) or, prefill,
  // at or past the column's causal limit.
  auto softmax = [&](auto masked_c, const f16v *s, int t0, bool half, h8 (*pb)[2]) {
    constexpr bool MASKED = decltype(masked_c)::value;
    uint32_t dead[NB2];
    float mn[NB2];
    bool over = false;
#pragma unroll
    for (int nb = 0; nb < NB2; ++nb) {
      dead[nb] = 0u;
      if constexpr (MASKED) {
        dead[nb] = half ? 0xFF00u : 0u;
        if constexpr (PREFILL) {
#pragma unroll
          for (int i = 0; i < 16; ++i)
            if (t0 + 8 * (i / 4) + 4 * h + (i % 4) >= col_lim[nb]) dead[nb] |= 1u << i;
        }
      }
      float e = -INFINITY;
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (!MASKED || !((dead[nb] >> i) & 1u)) e = fmaxf(e, s[nb][i]);
      float bm = e * ks;   // every element masked: -inf (NaN for a zero scale: ignored)
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
        const float alpha = mn[nb] == m[nb] ? 1.0f : fast_exp2(m[nb] - mn[nb]);
        l[nb] *= alpha;
#pragma unroll
        for (int t = 0; t < NT; ++t) acc[nb][t] *= alpha;
        m[nb] = mn[nb];
      }
    }
#pragma unroll
    for (int nb = 0; nb < NB2; ++nb) {
      float pr[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) pr[i] = fast_exp2(fmaf(s[nb][i], ks, -m[nb]));
      if constexpr (MASKED) {
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if ((dead[nb] >> i) & 1u) pr[i] = 0.0f;
      }
      float ps[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) ps[j] = (pr[4 * j] + pr[4 * j + 1]) + (pr[4 * j + 2] + pr[4 * j + 3]);
      l[nb] += (ps[0] + ps[1]) + (ps[2] + ps[3]);
#pragma unroll
      for (int kc = 0; kc < 2; ++kc)
        pb[nb][kc] = h8{(_Float16)pr[8 * kc], (_Float16)pr[8 * kc + 1], (_Float16)pr[8 * kc + 2],
                        (_Float16)pr[8 * kc + 3], (_Float16)pr[8 * kc + 4],
                        (_Float16)pr[8 * kc + 5], (_Float16)pr[8 * kc + 6],
                        (_Float16)pr[8 * kc + 7]};
    }
  };
  // O^T += V^T P^T from a step's V rows.  ZERO: V of tokens at or past the
  // data's end is zeroed (unwritten slots may hold NaN).
  auto pv = [&](auto zero_c, const u4 *vr, h8 (*pb)[2], int t0) {
    constexpr bool ZERO = decltype(zero_c)::value;
    h8 va[2][NT];
#pragma unroll
    for (int kc = 0; kc < 2; ++kc)
#pragma unroll
      for (int gg = 0; gg < NG; ++gg) {
        const u4 a = vr[(kc * NG + gg) * 2], b = vr[(kc * NG + gg) * 2 + 1];
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
    if constexpr (ZERO) {
#pragma unroll
      for (int kc = 0; kc < 2; ++kc)
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int tok = t0 + 16 * kc + (i < 4 ? 4 * h + i : 8 + 4 * h + (i - 4));
          if (tok >= ltok) {
#pragma unroll
            for (int t = 0; t < NT; ++t) va[kc][t][i] = (_Float16)0.0f;
          }
        }
    }
#pragma unroll
    for (int kc = 0; kc < 2; ++kc)
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int nb = 0; nb < NB2; ++nb)
          acc[nb][t] = __builtin_amdgcn_mfma_f32_32x32x16_f16(va[kc][t], pb[nb][kc], acc[nb][t],
                                                              0, 0, 0);
  };
  auto barrier = [&]() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };

  // ---- the walk.  Ring slot of step k: k % NR.  Iteration k waits for
  // step k+1's rows, meets the group at a barrier (every wave has then
  // finished iteration k-1, so slot (k-1) % NR is free, and every wave's rows
  // of step k+1 are in LDS), issues step k+NR-1 into the freed slot (in the
  // pipelined loop after step k+1's q.K MFMAs, which keeps the load
  // instructions off the head of the step), then computes step k's softmax
  // and P.V and step k+1's q.K.  The prologue issues steps 0 .. NR-2 and
  // each pipelined iteration one step, whether or not they exist, so that
  // there the loads behind step k+1 are always one step's; the masked tail
  // issues only real steps and counts them exactly.  Every wave runs ns_max
  // iterations, so that the barriers match.
  // Waits for a step whose rows have `after` later steps' rows issued behind
  // them (loads complete in issue order; table loads issued since only make
  // the wait longer).  The count must not exceed what was really issued
  // after the step, so near the end of a walk it is smaller.
  auto wait_step = [&](int after) {
    static_assert(NR - 2 <= 4, "wait cases");
    switch (after) {
      case 0: wait_vmcnt<0>(); break;
      case 1: wait_vmcnt<LPW>(); break;
      case 2: wait_vmcnt<2 * LPW>(); break;
      case 3: wait_vmcnt<3 * LPW>(); break;
      default: wait_vmcnt<4 * LPW>(); break;
    }
  };
  // The prologue issues its NR - 1 steps unconditionally: a step past the
  // walk reloads an in-pool block into a slot no step reads.
#pragma unroll
  for (int j = 0; j < NR - 1; ++j) {
    entries(j, ent);
    issue(j, j, ent);
  }
  entries(NR - 1, ent);
  // Every q load is issued before the first move: each move is a scheduling
  // barrier, and a load after one would wait for the load before it.
#pragma unroll
  for (int nb = 0; nb < NB2; ++nb)
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      u4 r = qraw[nb][kk] ^ u4{qneg, qneg, qneg, qneg};
      // q stays in accumulation registers (the MFMAs read their B operand
      // from there), leaving the vector registers to the walk's working set
      asm volatile("" : "+a"(r));
      qf[nb][kk] = __builtin_bit_cast(h8, r);
    }
  wait_vmcnt<(NR - 2) * LPW>();
  barrier();
  f16v S[NB2];
  if (!idle && ns_g > 0) {
    u4 kr[NKK];
    lds_read_row<0, NKK, 1024>(ring_addr(0), kr);
    lds_wait();
#pragma unroll
    for (int i = 0; i < NKK; ++i) after_wait(kr[i]);
    qk(kr, S);
  }
  auto advance = [&](int k, int slot) {
    const int fslot = slot == 0 ? NR - 1 : slot - 1;   // slot of step k-1, refilled now
    if (k + 1 < ns_g) wait_step(min(NR - 3, ns_g - 2 - k));
    barrier();
    if (k + NR - 1 < ns_g) issue(k + NR - 1, fslot, ent);
  };
  // Steps 0 .. nfast-1 have a next step and no masks: the last steps of a
  // walk are the only ones that can hold a missing second tile (the last) or,
  // prefill, tokens at or past a column's causal limit (limits only grow
  // with the column, and the walk's tokens with the step).
  int nfast = 0;
  if (!idle) {
    while (nfast + 1 < ns_g) {
      const int st = first + 2 * (tgi + TG * nfast);
      if (st + 1 >= last || (PREFILL && st * kTile + 32 > wlim_lo)) break;
      ++nfast;
    }
  }
  // One pipelined step: softmax and P.V of step k (scores si), q.K of step
  // k+1 (into so); one basic block apart from the rare rescale.  The next
  // step's K rows arrive under the softmax, this step's V rows under the
  // next step's q.K MFMAs.
  auto fast_step = [&](int k, int slot, f16v *si, f16v *so) {
    const int nslot = slot + 1 == NR ? 0 : slot + 1;
    const int t0 = (first + 2 * (tgi + TG * k)) * kTile;
    // the prologue issues NR - 1 steps and every pipelined iteration one,
    // whether or not they exist: one step's loads are always behind step
    // k+1's here
    wait_vmcnt<(NR - 3) * LPW>();
    barrier();
    u4 kr[NKK], vr[VLD];
    lds_read_row<0, NKK, 1024>(ring_addr(nslot), kr);
    h8 pb[NB2][2];
    softmax(IC<0>{}, si, t0, false, pb);
    lds_wait();
#pragma unroll
    for (int i = 0; i < NKK; ++i) after_wait(kr[i]);
    lds_read_row<0, VLD, 1024>(ring_addr(slot) + NKK * 1024, vr);
    qk(kr, so);
    {
      // Unconditional, so that no branch splits the step's instructions
      // (the exponentials then interleave with the q.K MFMAs): past the
      // walk's end it reloads a clamped, in-pool block into the slot just
      // freed, which no step reads again.  Loads issued after the step a
      // wait is for only lengthen that wait.
      const int fslot = slot == 0 ? NR - 1 : slot - 1;
      issue(k + NR - 1, fslot, ent);
    }
    lds_wait();
#pragma unroll
    for (int i = 0; i < VLD; ++i) after_wait(vr[i]);
    // Scalar and LDS loads share one wait counter: the next entries are
    // requested after the wait for the V rows, so that the next wait on that
    // counter (the next step's K rows) is a step away.
    entries(k + NR, ent);
    pv(IC<0>{}, vr, pb, t0);
    return nslot;
  };
  int k = 0, slot = 0;
  f16v S2[NB2];
  // four steps per iteration (two where fewer are left): the scores
  // alternate between S and S2, and the loop's fixed costs spread further
  for (; k + 4 <= nfast; k += 4) {
    slot = fast_step(k, slot, S, S2);
    slot = fast_step(k + 1, slot, S2, S);
    slot = fast_step(k + 2, slot, S, S2);
    slot = fast_step(k + 3, slot, S2, S);
  }
  for (; k + 2 <= nfast; k += 2) {
    slot = fast_step(k, slot, S, S2);
    slot = fast_step(k + 1, slot, S2, S);
  }
  if (k < nfast) {
    slot = fast_step(k, slot, S, S2);
#pragma unroll
    for (int nb = 0; nb < NB2; ++nb) S[nb] = S2[nb];
    ++k;
  }
  // The rest, one step after the other, with the masks: the last step, steps
  // with a missing second tile or (prefill) past a column's causal limit or
  // the data.  Idle waves only load and meet the barriers.
  for (; k < ns_max; ++k) {
    const int nslot = slot + 1 == NR ? 0 : slot + 1;
    advance(k, slot);
    if (!idle && k < ns_g) {
      const int st = first + 2 * (tgi + TG * k);
      const int t0 = st * kTile;
      u4 vr[VLD];
      lds_read_row<0, VLD, 1024>(ring_addr(slot) + NKK * 1024, vr);
      h8 pb[NB2][2];
      softmax(IC<1>{}, S, t0, st + 1 >= last, pb);
      lds_wait();
#pragma unroll
      for (int i = 0; i < VLD; ++i) after_wait(vr[i]);
      pv(IC<1>{}, vr, pb, t0);
      if (k + 1 < ns_g) {
        u4 kr[NKK];
        lds_read_row<0, NKK, 1024>(ring_addr(nslot), kr);
        lds_wait();
#pragma unroll
        for (int i = 0; i < NKK; ++i) after_wait(kr[i]);
        qk(kr, S);
      }
    }
    entries(k + NR, ent);   // after this step's LDS waits (see the pipelined step)
    slot = nslot;
  }

  // ---- results: l over the lane halves; with two token groups, group 1's
  // state is folded into group 0's through LDS.
#pragma unroll
  for (int nb = 0; nb < NB2; ++nb) {
    const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(l[nb]),
                                                    __float_as_uint(l[nb]), false, false);
    l[nb] = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  }
  if constexpr (TG > 1) {
    // [column group][block][tile][piece][lane]: a lane's 16-byte pieces
    // next to its neighbours', free of bank conflicts
    f4(*lds_acc)[NB2][NT][4][64] = reinterpret_cast<f4(*)[NB2][NT][4][64]>(&lds_raw[0]);
    barrier();   // every wave is done with the ring
    if (tgi == 1 && !idle) {
#pragma unroll
      for (int nb = 0; nb < NB2; ++nb) {
        if (h == 0) {
          lds_m[cgi * CW + 32 * nb + n] = m[nb];
          lds_l[cgi * CW + 32 * nb + n] = l[nb];
        }
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
          for (int q = 0; q < 4; ++q)
            lds_acc[cgi][nb][t][q][lane] = f4{acc[nb][t][4 * q], acc[nb][t][4 * q + 1],
                                              acc[nb][t][4 * q + 2], acc[nb][t][4 * q + 3]};
      }
    }
    __syncthreads();
    if (tgi == 1 || idle) return;
#pragma unroll
    for (int nb = 0; nb < NB2; ++nb) {
      const float m1 = lds_m[cgi * CW + 32 * nb + n];
      const float l1 = lds_l[cgi * CW + 32 * nb + n];
      const float M = fmaxf(m[nb], m1);
      const float f0 = m[nb] == -INFINITY ? 0.0f : exp2f(m[nb] - M);
      const float f1 = m1 == -INFINITY ? 0.0f : exp2f(m1 - M);
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const f4 *o = &lds_acc[cgi][nb][t][0][lane];
        const f16v other = f16v{o[0][0], o[0][1], o[0][2], o[0][3], o[64][0], o[64][1],
                                o[64][2], o[64][3], o[128][0], o[128][1], o[128][2],
                                o[128][3], o[192][0], o[192][1], o[192][2], o[192][3]};
        acc[nb][t] = acc[nb][t] * f0 + other * f1;
      }
      l[nb] = l[nb] * f0 + l1 * f1;
      m[nb] = M;
    }
  } else {
    if (idle) return;
  }

  // ---- output: lane (n, h) holds, for column n, dims 2(32gg + 8j + 4h + v) + par
  // in element 4j + v of tile 2gg + par: 8 consecutive dims per (gg, j).
  const bool direct = PREFILL && p.num_pparts == 1;
#pragma unroll
  for (int nb = 0; nb < NB2; ++nb) {
    if (!col_ok[nb]) continue;
    const size_t orow = (size_t)col_seq[nb] * H + col_head[nb];
    const size_t row = orow * p.ws_stride + p.ws_pre + part;
    const float inv = 1.0f / l[nb];
#pragma unroll
    for (int gg = 0; gg < NG; ++gg)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const f16v &ev = acc[nb][2 * gg];
        const f16v &od = acc[nb][2 * gg + 1];
        const int d0 = 2 * (32 * gg + 8 * j + 4 * h);
        const f4 lo = f4{ev[4 * j], od[4 * j], ev[4 * j + 1], od[4 * j + 1]} * inv;
        const f4 hi = f4{ev[4 * j + 2], od[4 * j + 2], ev[4 * j + 3], od[4 * j + 3]} * inv;
        if (direct) {
          if constexpr (OUT == PKV_F32) {
            float *o = reinterpret_cast<float *>(p.out) + orow * D + d0;
            *reinterpret_cast<f4 *>(o) = lo;
            *reinterpret_cast<f4 *>(o + 4) = hi;
          } else {
            _Float16 *o = reinterpret_cast<_Float16 *>(p.out) + orow * D + d0;
            *reinterpret_cast<h8 *>(o) =
                h8{to_f16_out(lo[0]), to_f16_out(lo[1]), to_f16_out(lo[2]), to_f16_out(lo[3]),
                   to_f16_out(hi[0]), to_f16_out(hi[1]), to_f16_out(hi[2]), to_f16_out(hi[3])};
          }
        } else {
          float *o = p.ws_o + row * D + d0;
          *reinterpret_cast<f4 *>(o) = lo;
          *reinterpret_cast<f4 *>(o + 4) = hi;
        }
      }
    if (!direct && h == 0) p.ws_lse[row] = m[nb] + log2f(l[nb]);
  }
}

template <int D, int BS, int MODE, int OUT>
hipError_t pipe_typed(const PrefixParams &p, int tg, hipStream_t stream) {
  if (tg == 2)
    hipLaunchKernelGGL((pipe32_kernel<D, BS, MODE, OUT, 2>), dim3((unsigned)prefix_grid(p)),
                       dim3(64 * kWaves), 0, stream, p);
  else
    hipLaunchKernelGGL((pipe32_kernel<D, BS, MODE, OUT, 1>), dim3((unsigned)prefix_grid(p)),
                       dim3(64 * kWaves), 0, stream, p);
  return hipGetLastError();
}

template <int D, int MODE, int OUT>
hipError_t pipe_bs(const PrefixParams &p, int block_size, int tg, hipStream_t stream) {
  switch (block_size) {
    case 8: return pipe_typed<D, 8, MODE, OUT>(p, tg, stream);
    case 32: return pipe_typed<D, 32, MODE, OUT>(p, tg, stream);
    default: return pipe_typed<D, 16, MODE, OUT>(p, tg, stream);
  }
}

}  // namespace

hipError_t launch_pipe(const PrefixParams &p, bool prefill, int out_dtype, int head_dim,
                       int block_size, int token_groups, hipStream_t stream) {
  if (!prefill)
    return head_dim == 64
               ? pipe_bs<64, kModeShared, PKV_F32>(p, block_size, token_groups, stream)
               : pipe_bs<128, kModeShared, PKV_F32>(p, block_size, token_groups, stream);
  if (out_dtype == PKV_F32)
    return head_dim == 64
               ? pipe_bs<64, kModePrefill, PKV_F32>(p, block_size, token_groups, stream)
               : pipe_bs<128, kModePrefill, PKV_F32>(p, block_size, token_groups, stream);
  return head_dim == 64
             ? pipe_bs<64, kModePrefill, PKV_F16>(p, block_size, token_groups, stream)
             : pipe_bs<128, kModePrefill, PKV_F16>(p, block_size, token_groups, stream);
}

}  // namespace pkv
