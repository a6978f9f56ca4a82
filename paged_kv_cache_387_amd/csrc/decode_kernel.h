// PagedAttention decode for gfx950 (CDNA4).
//
// What is computed: for each sequence s and query head h (kv head h / G),
//   out[s][h] = softmax_t(scale * q[s][h] . K_t) V_t  over the cached tokens
// t < seq_len, with K/V reached through the block table (logical block t/16 ->
// physical block; "KV Cache and PagedAttention (vllm-musa)", 7yue.com,
// section 5; "KVcache-learning", fairy2021.github.io, s01 and s05).  Long
// sequences are split into pieces whose partial results are merged with a
// log-sum-exp reduction ("partial accumulate, then merge" of paged_attention_v2,
// "vLLM PagedAttention deep dive", jsqmd.com, section 4.1).
//
// Work decomposition: a unit is one (sequence, kv head); a workgroup is 4
// wavefronts.  Three walks share the per-tile code below:
//  * kWalkSplit: one workgroup per (unit, partition).  Wave w takes tiles
//    first+w, first+w+4, ... of the partition; at the end the four wave states
//    are combined through LDS into the output row (or the partition's partial).
//  * kWalkRuns: one workgroup per (unit, run of consecutive partitions whose
//    size is a multiple of 4 tiles): the waves interleave the run's tiles as
//    in the split walk, every wave ends each partition at the same step, and
//    the four states of a finished partition are combined through LDS into
//    its partial, which waits in LDS until the run's last load is issued.
//  * kWalkStream: the batch's tiles, in (sequence, kv head, tile) order, are
//    dealt to the grid's waves in equal shares of whole blocks (each
//    workgroup first scans seq_lens for the share boundaries).  A wave walks
//    the pieces of the units its share covers, tile by tile, ending each piece
//    itself: a unit wholly inside one share is written directly, the other
//    pieces leave partials for the merge.  Every wave streams the same number
//    of bytes however ragged the lengths are.
// For one 16-token tile a wave computes
//   S^T[t][h] = K[t] . q[h]      one 16x16 MFMA tile: rows = the tile's 16
//                                 tokens, columns = the G <= 16 query heads of
//                                 the GQA group (columns >= G have q = 0)
//   online softmax per column (running max m, partial sum l, fp32, base 2)
//   O^T[d][h] += V^T[d][t] P^T[t][h]   MFMA tiles of 16 head_dim rows
// The MFMA accumulator layout puts column h = lane % 16 and rows
// 4*(lane/16)+v (v = 0..3) in lane `lane`; the same registers are the P^T
// operand of the P.V MFMA (k index = token), so scores never move between
// lanes except for two cross-row reductions (max over the 16 tokens).
//
// Pool layout (see include/pkv.h): a (block, kv head) tile of K stores each
// token's vector as 16-byte columns, token-minor: 16-byte load number i of lane
// (r = lane%16, g = lane/16) reads column 4i+g of token r at byte (64i+lane)*16
// -- one contiguous 1 KiB per wave instruction.  V of 2- and 4-byte elements
// stores 4-byte columns, token-minor: load i of lane (r, g) reads tokens
// 4g..4g+3 of column 16i+r at byte (16i+r)*64 + 16g.  V of 1-byte elements
// stores 16-byte groups (4 elements x 4 tokens): load i of lane (r, g) reads
// group (16i+r, g) at byte ((16i+r)*4 + g)*16, whose word e holds element
// 4(16i+r)+e of tokens 4g..4g+3 -- an MFMA operand as it stands.  Again 1 KiB
// contiguous per instruction.
//
// Data types: fp32 KV uses 16x16x4 f32 MFMAs; fp16 KV uses 16x16x32 f16 (q.K)
// and 16x16x16 f16 (P.V); int8 / E4M3 codes are widened exactly to fp16 (int8
// by a byte permute under an fp16 exponent, E4M3 by the gfx950 fp8
// conversion) and use the fp16 MFMAs, the K scale multiplies the scores and
// the V scale is folded into P (P' = p * s_v * b in fp16, b a power-of-two
// boost that keeps P' out of fp16's subnormal range and below its largest
// value; see lower_boost).
#pragma once

#include "attn_common.h"

namespace pkv {
namespace {
// Tiles of K/V (and scales) one wavefront keeps in flight: the ring of
// prefetched blocks is NB deep.  Registers per tile: 2 * NL * 4 (+4 scales).
#ifndef PKV_PREFETCH_F32
#define PKV_PREFETCH_F32 2
#endif
#ifndef PKV_PREFETCH_F16
#define PKV_PREFETCH_F16 3
#endif
#ifndef PKV_PREFETCH_Q8
#define PKV_PREFETCH_Q8 4
#endif
// Workgroups per compute unit the register budget is sized for (one wave per
// SIMD each, so also waves per SIMD).
#ifndef PKV_OCCUPANCY_F16
#define PKV_OCCUPANCY_F16 2
#endif
#ifndef PKV_OCCUPANCY_Q8
#define PKV_OCCUPANCY_Q8 2
#endif
template <int KV> struct Prefetch {
  static constexpr int NB = PKV_PREFETCH_F16;
  static constexpr int OCC = PKV_OCCUPANCY_F16;
};
template <> struct Prefetch<PKV_F32> {
  static constexpr int NB = PKV_PREFETCH_F32;
  static constexpr int OCC = 2;
};
template <> struct Prefetch<PKV_I8> {
  static constexpr int NB = PKV_PREFETCH_Q8;
  static constexpr int OCC = PKV_OCCUPANCY_Q8;
};
template <> struct Prefetch<PKV_E4M3> {
  static constexpr int NB = PKV_PREFETCH_Q8;
  static constexpr int OCC = PKV_OCCUPANCY_Q8;
};

// Four consecutive output elements (idx a multiple of 4).
template <int OUT>
__device__ __forceinline__ void store_out4(void *out, size_t idx, f4 v) {
  if constexpr (OUT == PKV_F32)
    *reinterpret_cast<f4 *>(reinterpret_cast<float *>(out) + idx) = v;
  else
    *reinterpret_cast<h4 *>(reinterpret_cast<_Float16 *>(out) + idx) =
        h4{to_f16_out(v[0]), to_f16_out(v[1]), to_f16_out(v[2]), to_f16_out(v[3])};
}

// Issue priority by progress (runs walk).  The waves on a compute unit
// compete for instruction issue and the hardware favours older waves, so
// waves with equal work drift apart; in the runs walk the four waves of a
// workgroup meet at a barrier at every partition end, where the ones ahead
// wait for the one behind.  A wave lowers its priority (s_setprio, the
// in-kernel wave priority) as it works through its tiles: 3 for the first
// quarter, then 2, 1 and 0, so the one that is behind wins issue.  Measured
// on C3 (512-token partitions): 183 -> 176 us; no gain elsewhere.
template <bool ON> struct PrioSteps {
  int q1, q2, q3;   // steps at which the priority drops
  __device__ __forceinline__ explicit PrioSteps(int total)
      : q1(total / 4), q2(total / 2), q3(total - total / 4) {
    if constexpr (ON) __builtin_amdgcn_s_setprio(3);
  }
  __device__ __forceinline__ void at(int k) const {
    if constexpr (ON) {
      if (k == q1) __builtin_amdgcn_s_setprio(2);
      else if (k == q2) __builtin_amdgcn_s_setprio(1);
      else if (k == q3) __builtin_amdgcn_s_setprio(0);
    }
  }
};

// 64-bit lane shift (the stream walk's scan of sequence lengths).
__device__ __forceinline__ int64_t shfl_up64(int64_t x, int d) {
  const int lo = __shfl_up((int)(uint32_t)x, d, 64);
  const int hi = __shfl_up((int)(x >> 32), d, 64);
  return (int64_t)(((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo);
}

// WALK: kWalkSplit, kWalkRuns or kWalkStream (see above).  SRC < 0: decode
// only.  SRC = PKV_F16 / PKV_F32: fused decode step, the new token's K/V (of
// that type) is written first (see DecodeParams).  BS = block size (8, 16 or
// 32 tokens).  The kernel works on 16-token tiles (the MFMA row count): a
// 32-token block is two tiles stored one after the other, a 16-token tile
// spans two 8-token blocks.
template <int KV, int D, int OUT, int SRC, int BS, int WALK>
__global__ __launch_bounds__(64 * kDecodeWaves, Prefetch<KV>::OCC) void decode_kernel(DecodeParams p) {
  constexpr int EB = Kv<KV>::EB;
  constexpr bool QUANT = (KV == PKV_I8 || KV == PKV_E4M3);
  constexpr int SLICE = BS * D * EB;          // bytes of one (block, kv head) slice
  constexpr int TPB = BS >= kTile ? BS / kTile : 1;   // tiles per block
  constexpr bool SPLIT = BS < kTile;          // a tile spans two blocks
  constexpr int TB = SPLIT ? BS : kTile;      // tokens of a tile within one block
  constexpr int NL = D * EB / 64;             // 16-byte loads per lane per K (and V) tile
  constexpr int NACC = D / 16;                // 16x16 output tiles
  constexpr int E = 4 / EB;                   // head_dim elements per V word
  constexpr int LDS_ROW = D + 4;
  constexpr int NB = Prefetch<KV>::NB;
  constexpr bool WAVE = WALK == kWalkStream;  // waves walk and end their pieces alone
  constexpr int TS = WAVE ? 1 : kDecodeWaves; // tile stride of a wave's walk
  static_assert(BS == 8 || BS == 16 || BS == 32, "block size");
  static_assert(WALK == kWalkSplit || WALK == kWalkRuns || WALK == kWalkStream, "walk");

  // the split and runs walks' combine of the four wave states (a token size
  // otherwise), and the runs walk's finished partials of the run's earlier
  // partitions: [partition][head][D + 4] (the output row, then its
  // log-sum-exp)
  __shared__ __attribute__((aligned(16)))
      float lds_o[WAVE ? 1 : kDecodeWaves][WAVE ? 1 : kMaxGroup][WAVE ? 4 : LDS_ROW];
  __shared__ float lds_m[WAVE ? 1 : kDecodeWaves][WAVE ? 1 : kMaxGroup];
  __shared__ float lds_l[WAVE ? 1 : kDecodeWaves][WAVE ? 1 : kMaxGroup];
  __shared__ __attribute__((aligned(16))) float lds_stage[WALK == kWalkRuns ? stage_floats(D) : 1];
  // the fused step's staged new token (stored K, V rows and scales): one area
  // per wave in the stream walk, where each wave may hold a tail tile
  constexpr int NEWB = SRC >= 0 ? D * EB : 16;
  constexpr int NEWW = WALK == kWalkStream ? kDecodeWaves : 1;
  __shared__ __attribute__((aligned(16))) uint8_t lds_new_all[NEWW][2][NEWB];
  __shared__ uint16_t lds_new_sc_all[NEWW][2];

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform
  const int r = lane & 15;
  const int g = lane >> 4;
  const int bid = blockIdx.x;
  const int G = p.group;
  const int H = p.num_heads;
  const int Hkv = p.num_kv_heads;
  const int cap_tokens = p.max_blocks * BS;
  uint8_t (*lds_new)[NEWB] = lds_new_all[WALK == kWalkStream ? w : 0];
  uint16_t *lds_new_sc = lds_new_sc_all[WALK == kWalkStream ? w : 0];
  // Tiles one unit of a sequence of `len` tokens spans in the stream walk's
  // order: whole blocks (a 32-token block counts two tiles even when only its
  // first holds tokens), so that every share boundary is a block boundary.
  auto span_of = [&](int len) {
    len = len < 0 ? 0 : (len > cap_tokens ? cap_tokens : len);
    return TPB > 1 ? (len + BS - 1) / BS * TPB : (len + kTile - 1) / kTile;
  };

  // ---- the stream walk: where this wave's share starts ----
  // Each workgroup scans the spans of all sequences (thread t sums a
  // contiguous slice; wave scans, then the four wave totals), derives the
  // share (the same in every workgroup) and finds the sequence that holds the
  // first tile of each of its four waves.
  int64_t sg = 0, sg_end = 0;   // this wave's share [sg, sg_end) of the batch's tiles
  int64_t sc = 0;               // tiles (per kv head) of the sequences before ss
  int64_t share = 1;
  int ss = 0, sspan = 0;        // the sequence holding tile sg, and its span
  int wave_id = 0;
  if constexpr (WALK == kWalkStream) {
    __shared__ int64_t lds_tot[kDecodeWaves];
    __shared__ int64_t lds_c[kDecodeWaves];
    __shared__ int lds_s[kDecodeWaves];
    const int S = p.num_seqs;
    constexpr int NT = 64 * kDecodeWaves;
    const int per = (S + NT - 1) / NT;
    const int s_lo = min(S, (int)threadIdx.x * per), s_hi = min(S, s_lo + per);
    int64_t mine = 0;
    for (int s = s_lo; s < s_hi; ++s) mine += span_of(p.seq_lens[s]);
    int64_t inc = mine;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int64_t v = shfl_up64(inc, o);
      if (lane >= o) inc += v;
    }
    if (lane == 63) lds_tot[w] = inc;
    if (threadIdx.x < kDecodeWaves) lds_s[threadIdx.x] = -1;
    __syncthreads();
    int64_t before = 0, total = 0;
#pragma unroll
    for (int i = 0; i < kDecodeWaves; ++i) {
      const int64_t t = lds_tot[i];
      before += i < w ? t : 0;
      total += t;
    }
    const int64_t T = total * Hkv;   // tiles of the batch
    int64_t nw = (T + p.min_share - 1) / p.min_share;
    nw = nw < p.stream_waves ? nw : p.stream_waves;
    nw = nw < 1 ? 1 : nw;
    share = (T + nw - 1) / nw;
    share = (share + TPB - 1) / TPB * TPB;
    share = share < 1 ? 1 : share;
    int64_t c = before + inc - mine;   // spans of the sequences before s_lo
    const int64_t g0 = (int64_t)bid * kDecodeWaves * share;
    for (int s = s_lo; s < s_hi; ++s) {
      const int sp = span_of(p.seq_lens[s]);
#pragma unroll
      for (int i = 0; i < kDecodeWaves; ++i) {
        const int64_t gs = g0 + i * share;
        if (Hkv * c <= gs && gs < Hkv * (c + sp)) {
          lds_s[i] = s;
          lds_c[i] = c;
        }
      }
      c += sp;
    }
    __syncthreads();
    wave_id = bid * kDecodeWaves + w;
    sg = g0 + w * share;
    sg_end = sg + share < T ? sg + share : T;
    ss = __builtin_amdgcn_readfirstlane(lds_s[w]);
    if (ss < 0) return;                   // a share beyond the batch: nothing to do
    sc = lds_c[w];
    sspan = span_of(p.seq_lens[ss]);
  }

  // out needs only element alignment; vector stores when it allows them
  const bool out_vec =
      (reinterpret_cast<uintptr_t>(p.out) & (OUT == PKV_F32 ? 15u : 7u)) == 0;

  // ---- wave walks: finished outputs wait in LDS for the wave's last load ----
  // A wave's loads and stores complete in order, so a store issued among the
  // walk's loads makes the next wait for a tile a wait for the store as
  // well.  A wave's outputs other than its last (a partition of a run, a
  // piece of a share) therefore go to its LDS slots (KST of them; a full set
  // is stored on the spot) and are stored after its last load.  Lane (r, g)
  // stages its NACC quads of head r (see emit) in quad-major order, each quad
  // of the 64 lanes one contiguous 1 KiB.
  constexpr int KST = 2;
  __shared__ __attribute__((aligned(16)))
      f4 lds_st[WAVE ? kDecodeWaves : 1][WAVE ? KST : 1][WAVE ? NACC : 1][WAVE ? 64 : 1];
  __shared__ float lds_st_lse[WAVE ? kDecodeWaves : 1][WAVE ? KST : 1][kMaxGroup];
  struct Staged {
    size_t base;        // direct: element offset of the unit's head-0 row in `out`;
                        // partial: row of head 0
    size_t rstride;     // partial: rows between consecutive heads
    int direct;         // rows of `out` (else partial rows of the workspace)
    int info_u;         // stream walk: the unit whose record to store (-1: none)
    int info_fw, info_n;
  };
  __shared__ Staged lds_st_dst[WAVE ? kDecodeWaves : 1][WAVE ? KST : 1];   // where each goes
  int nst = 0;
  // Stores one output (quads q[c] of lane (r, g), head r's log-sum-exp lse)
  // where `d` says; lanes r >= G hold no head.
  auto store_output = [&](const Staged &d, const f4 *q, float lse) __attribute__((always_inline)) {
    if (r < G) {
#pragma unroll
      for (int c = 0; c < NACC; ++c) {
        const int i = c / E, j = c % E;
        const int d0 = E * (16 * i + 4 * g) + 4 * j;
        if (d.direct) {
          const size_t idx = d.base + (size_t)r * D + d0;
          if (out_vec) {
            store_out4<OUT>(p.out, idx, q[c]);
          } else {
#pragma unroll
            for (int k = 0; k < 4; ++k) store_out<OUT>(p.out, idx + k, q[c][k]);
          }
        } else {
          *reinterpret_cast<f4 *>(p.ws_o + (d.base + r * d.rstride) * D + d0) = q[c];
        }
      }
      if (!d.direct && g == 0) p.ws_lse[d.base + r * d.rstride] = lse;
    }
    if (d.info_u >= 0 && lane == 0) {
      p.ws_info[2 * d.info_u] = d.info_fw;
      p.ws_info[2 * d.info_u + 1] = d.info_n;
    }
  };
  auto flush_staged = [&]() __attribute__((always_inline)) {
    if constexpr (WAVE) {
      for (int k = 0; k < nst; ++k) {
        f4 q[NACC];
#pragma unroll
        for (int c = 0; c < NACC; ++c) q[c] = lds_st[w][k][c][lane];
        const Staged d = lds_st_dst[w][k];
        store_output(d, q, lds_st_lse[w][k][r]);
      }
      nst = 0;
    }
  };

  // ---- one pass per piece of a unit (a stream share may hold several) ----
  for (;;) {
  int s, kvh;
  int first, last;        // the tiles [first, last) of the workgroup (split) or wave
  int part0 = 0;          // split / runs: first partition of the workgroup
  int piece_end = 0;      // stream: the piece's end in span tiles
  bool piece_head = true, piece_tail = true;   // stream: the piece starts / ends its unit
  if constexpr (WALK == kWalkStream) {
    if (sg >= sg_end || ss >= p.num_seqs) {
      flush_staged();
      break;
    }
    const int64_t off = sg - Hkv * sc;
    kvh = (int)(off / sspan);
    const int a = (int)(off - (int64_t)kvh * sspan);
    const int64_t rem = sg_end - sg;
    piece_end = rem < sspan - a ? a + (int)rem : sspan;
    s = ss;
    first = a;
    last = piece_end;
    piece_head = a == 0;
    piece_tail = piece_end == sspan;
  } else {
    // Workgroup -> (unit, partition or run).  Workgroups are dealt to the dies
    // round robin, so unit u runs on die u % kXcds (with 8 kv heads: one kv
    // head per die, whose L2 then serves the blocks that sequences share).
    // Ids go partition-major: workgroups resident together work on the same
    // region of their sequences, so a shared prefix is read while it is still
    // cached.  The unit-group count is odd (unit_groups), so the partitions
    // of one unit land on different compute units.
    const int die_slot = bid / kXcds;
    const int ugroups = unit_groups(p.num_units);
    const int run = die_slot / ugroups;
    const int u = (die_slot % ugroups) * kXcds + bid % kXcds;
    if (u >= p.num_units) return;
    s = u / Hkv;
    kvh = u - s * Hkv;
    // A run of several partitions needs partitions of whole wave rounds (every
    // wave then ends each partition but the last at the same step) and room
    // for its staged partials; the host only sets up such runs.
    const int rp = WALK == kWalkRuns ? p.run_parts : 1;
    if (WALK == kWalkRuns && (rp < 1 || p.part_tiles % kDecodeWaves != 0 ||
                              (rp - 1) * G * (D + 4) > stage_floats(D)))
      return;
    part0 = run * rp;
    first = part0 * p.part_tiles;
    last = 0;   // set once the length is known
  }
  const int32_t *trow = p.block_tables + (size_t)s * p.max_blocks;
  // the wave's first tile
  int wfirst = WAVE ? first : first + w;

  // Table entries of this wave's walk steps c0 + lane (one per lane; readlane
  // picks entry j): the tile's block (the first of its two blocks when SPLIT;
  // tvb holds the second).  Entries are clamped to `lim` blocks.
  auto load_tv = [&](int c0, int lim, int *tvb) {
    const int tile = wfirst + (c0 + lane) * TS;
    int e = SPLIT ? 2 * tile : tile / TPB;
    e = e < lim ? e : lim - 1;
    if constexpr (SPLIT) {
      const int e2 = 2 * tile + 1 < lim ? 2 * tile + 1 : e;
      *tvb = trow[e2];
    }
    return trow[e];
  };

  // The piece's first loads are all issued before any is waited for, the
  // ones needed first first (a wave's loads complete in order, so waiting for
  // one leaves the later ones in flight; the empty asm statements keep the
  // compiler from reordering them): the sequence length and, in the fused
  // step, the copy source (read without a branch: any readable word stands in
  // for a null cow_src); then the table entries of the wave's first 64 tiles
  // (clamped to the row), the q fragment (B operand of the q.K MFMAs, column
  // r = head kvh*G+r; columns r >= G repeat head kvh*G and their results are
  // never stored) and, in the fused step, the unit's new token (every wave
  // loads it, only the one with the tail tile uses it: the same loads on
  // every path keep the waits exact).
  const int L_raw = p.seq_lens[s];
  int cow_raw = -1;
  if constexpr (SRC >= 0) cow_raw = *(p.cow_src ? p.cow_src + s : p.seq_lens + s);
  asm volatile("" ::: "memory");
  int tvb_next = 0;
  int tv_next = load_tv(0, p.max_blocks, &tvb_next);
  const size_t qrow = ((size_t)s * H + kvh * G + (r < G ? r : 0)) * D;
  float qf32[NL][4];
  h8 qf16[NL][QUANT ? 2 : 1];
#pragma unroll
  for (int i = 0; i < NL; ++i) {
    if constexpr (KV == PKV_F32) {
      const float *qp = reinterpret_cast<const float *>(p.q) + qrow + (4 * i + g) * 4;
      const u4 raw = load16(reinterpret_cast<const uint8_t *>(qp));
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) qf32[i][jj] = as_f32(raw[jj]);
    } else if constexpr (KV == PKV_F16) {
      const _Float16 *qp = reinterpret_cast<const _Float16 *>(p.q) + qrow + (4 * i + g) * 8;
      qf16[i][0] = __builtin_bit_cast(h8, load16(reinterpret_cast<const uint8_t *>(qp)));
    } else {
      const _Float16 *qp = reinterpret_cast<const _Float16 *>(p.q) + qrow + (4 * i + g) * 16;
      qf16[i][0] = __builtin_bit_cast(h8, load16(reinterpret_cast<const uint8_t *>(qp)));
      qf16[i][QUANT ? 1 : 0] =
          __builtin_bit_cast(h8, load16(reinterpret_cast<const uint8_t *>(qp + 8)));
    }
  }

  TokenRaw<SRC >= 0 ? SRC : PKV_F16, D> new_raw;
  if constexpr (SRC >= 0) {
    constexpr size_t esz = SRC == PKV_F32 ? 4 : 2;
    const size_t row = ((size_t)s * Hkv + kvh) * D * esz;
    load_token_raw<SRC, D>(static_cast<const uint8_t *>(p.key_new) + row,
                           static_cast<const uint8_t *>(p.value_new) + row, new_raw, lane);
  }
  asm volatile("" ::: "memory");

  // fused step: the block to copy into the tail block, if any
  const int cow_req = SRC >= 0 && p.cow_src ? cow_raw : -1;
  int L = L_raw;
  L = L < 0 ? 0 : (L > cap_tokens ? cap_tokens : L);
  const int nblk = (L + BS - 1) / BS;                 // blocks in use
  const int ntile = (L + kTile - 1) / kTile;          // tiles in use
  const int nparts_s = WALK == kWalkStream ? 1 : (ntile + p.part_tiles - 1) / p.part_tiles;
  const int npre = prefix_parts_of(p, s);   // shared-prefix partials (merged later)
  if constexpr (WALK == kWalkStream) {
    last = last < ntile ? last : ntile;       // a block's second tile past the length
  } else {
    if (first >= ntile) {
      if (first == 0 && npre == 0) {  // empty sequence: zero output rows
        for (int e = threadIdx.x; e < G * D; e += 64 * kDecodeWaves)
          store_out<OUT>(p.out, ((size_t)s * H + kvh * G + e / D) * D + e % D, 0.0f);
      }
      return;
    }
    const int rp = WALK == kWalkRuns ? p.run_parts : 1;
    last = min(first + rp * p.part_tiles, ntile);
  }
  // The wave's tiles: wfirst + k * TS, k < nt_w.
  int nt_w;
  if constexpr (WAVE) {
    nt_w = last - first;
  } else {
    const int nt_part = last - first;
    nt_w = nt_part > w ? (nt_part - w + kDecodeWaves - 1) / kDecodeWaves : 0;
  }
  // Runs: the partitions of the run.  Every one but the last is full, and
  // with part_tiles a multiple of the wave count each wave walks exactly
  // tpw = part_tiles / kDecodeWaves of its tiles: partition j of the run ends
  // for every wave after its step (j + 1) * tpw - 1.
  const int nparts_run = WALK == kWalkRuns ? (last - first + p.part_tiles - 1) / p.part_tiles : 1;
  const int tpw = p.part_tiles / kDecodeWaves;
  const int wlast = WAVE ? wfirst + nt_w : last;   // end of the wave's tiles (wave walks)

  // ---- fused step: the new token, written behind ----
  // The piece that holds a sequence's tail tile also stores the new token at
  // position L - 1, after giving the tail block the contents of block
  // cow_src[s] when that names another block.  Nothing waits for these stores:
  //  * the tail block's tiles are read from the copy source, whose bytes the
  //    copy reproduces;
  //  * the wave that consumes the tail tile (the last tile of its walk) keeps
  //    the token's stored form in LDS and puts it in place of slot L - 1 of
  //    the loaded tile;
  //  * that wave stores the token and does the copy after its tiles, merging
  //    the new token into the chunks it copies, so where the copy and the
  //    token's own stores meet they write equal bytes and their order does
  //    not matter.  (Stores issued among the walk's loads would make every
  //    later wait for a load a wait for all memory operations.)
  // Pieces and partitions are whole blocks, so the tail block lies within the
  // piece of its tail tile.  Other sequences may read the copy source
  // concurrently; nothing else writes these bytes.
  const int tail_tile = ntile - 1;
  const int tail_blk = nblk - 1;
  const int new_row = (L - 1) % kTile;   // row of the new token in the tail tile
  const int new_slot = (L - 1) % BS;     // its slot in the tail block
  // The first loads of K/V depend on nothing here but cow_src[s] (read with
  // seq_lens); the tail block's own table entry is taken from the table
  // entries of the chunk of steps that holds the tail tile, and the new
  // token's bits, loaded with the piece's first loads, are first used after
  // the ring's loads are issued.
  const bool tail_here = SRC >= 0 && tail_tile >= (WAVE ? wfirst : first) &&
                         tail_tile < (WAVE ? wlast : last);
  const int cow_from = tail_here && (unsigned)cow_req < (unsigned)p.num_blocks ? cow_req : -1;
  const bool step_wave = tail_here && (WAVE || w == (tail_tile - first) % kDecodeWaves);
  bool tail_ok = false;                  // the tail block's table entry is in the pool
  int tail_phys = 0;
  size_t tail_slice = 0, tail_sc = 0;
  // The tail tile's step in the wave's walk: its chunk (c0) and entry j in it.
  const int tail_step = step_wave ? (tail_tile - wfirst) / TS : -1;
  const int tail_c0 = tail_step >= 0 ? tail_step / 64 * 64 : -1;
  // At the start of the tail tile's chunk, right after the ring's first loads:
  // encode the new token and keep its row-order bytes in LDS.  The tail
  // block's entry is lane j of the chunk's entries (tvb: the second block of
  // a SPLIT tile).  (A tail entry outside the pool writes nothing; its tile
  // is skipped.)
  auto step_write = [&](int tv, int tvb, int j) {
    if constexpr (SRC >= 0) {
      constexpr int PER = D / 64;
      tail_phys = SPLIT && tail_blk == 2 * tail_tile + 1 ? __builtin_amdgcn_readlane(tvb, j)
                                                          : __builtin_amdgcn_readlane(tv, j);
      tail_ok = (unsigned)tail_phys < (unsigned)p.num_blocks;
      if (!tail_ok) return;
      tail_slice = ((size_t)tail_phys * Hkv + kvh) * SLICE;
      tail_sc = ((size_t)tail_phys * Hkv + kvh) * BS;
      // first use of the token's bits: here, not hoisted above the ring's
      // loads (which would wait for the token and then issue the ring)
      TokenRaw<SRC, D> raw = new_raw;
#pragma unroll
      for (int which = 0; which < 2; ++which)
#pragma unroll
        for (int k = 0; k < TokenRaw<SRC, D>::RW; ++k) asm volatile("" : "+v"(raw.w[which][k]));
      float new_x[2][D / 64];
      token_from_raw<SRC, D>(raw, new_x);
      const TokenCodes<D> tc = encode_token<KV, D>(new_x);
#pragma unroll
      for (int which = 0; which < 2; ++which)
#pragma unroll
        for (int k = 0; k < PER; ++k) {
          uint8_t *dst = &lds_new[which][(lane * PER + k) * EB];
          if constexpr (EB == 4) *reinterpret_cast<uint32_t *>(dst) = tc.c[which][k];
          else if constexpr (EB == 2) *reinterpret_cast<uint16_t *>(dst) = (uint16_t)tc.c[which][k];
          else *dst = (uint8_t)tc.c[which][k];
        }
      if (lane == 0) {
        lds_new_sc[0] = tc.sc[0];
        lds_new_sc[1] = tc.sc[1];
      }
    }
  };
  // After the wave's tiles: the new token's stores (from the staged row), and
  // the copy.  Issued after the last load of the walk, so no wait for a load
  // ever has a store before it, and nothing waits for these stores.
  auto step_store = [&]() {
    if constexpr (SRC >= 0) {
      constexpr int PER = D / 64;
      TokenCodes<D> tc;
#pragma unroll
      for (int which = 0; which < 2; ++which)
#pragma unroll
        for (int k = 0; k < PER; ++k) {
          const uint8_t *src = &lds_new[which][(lane * PER + k) * EB];
          if constexpr (EB == 4) tc.c[which][k] = *reinterpret_cast<const uint32_t *>(src);
          else if constexpr (EB == 2) tc.c[which][k] = *reinterpret_cast<const uint16_t *>(src);
          else tc.c[which][k] = *src;
        }
      tc.sc[0] = lds_new_sc[0];
      tc.sc[1] = lds_new_sc[1];
      store_token<KV, D, BS>(tc, p.k_cache_w + tail_slice, p.v_cache_w + tail_slice,
                             QUANT ? p.k_scale_w + tail_sc + new_slot : nullptr,
                             QUANT ? p.v_scale_w + tail_sc + new_slot : nullptr, new_slot, lane);
    }
  };
  // The copy (its registers are free after the tiles).
  auto cow_copy = [&]() {
    if constexpr (SRC >= 0) {
      // copy the slice 16 bytes at a time; chunks that hold bytes of slot
      // new_slot take them from the staged row
      const size_t sslice = ((size_t)cow_from * Hkv + kvh) * SLICE;
      constexpr int CHUNKS = SLICE / 16;
      constexpr int TILE_CH = TB * D * EB / 16;   // chunks per stored tile
      constexpr int ROUND = 4;                    // chunks per lane in flight
      for (int q0 = 0; q0 < CHUNKS; q0 += 64 * ROUND) {
        u4 ck[ROUND], cv[ROUND];
#pragma unroll
        for (int k = 0; k < ROUND; ++k) {
          const int q = q0 + 64 * k + lane;
          if (q < CHUNKS) {
            ck[k] = *reinterpret_cast<const u4 *>(p.k_cache_w + sslice + 16 * (size_t)q);
            cv[k] = *reinterpret_cast<const u4 *>(p.v_cache_w + sslice + 16 * (size_t)q);
          }
        }
#pragma unroll
        for (int k = 0; k < ROUND; ++k) {
          const int q = q0 + 64 * k + lane;
          if (q >= CHUNKS) continue;
          const int tb = q / TILE_CH, tq = q % TILE_CH;   // stored tile, chunk in it
          // K chunk: 16-byte column tq / TB of token tb*TB + tq % TB
          if (tb * TB + tq % TB == new_slot)
            ck[k] = *reinterpret_cast<const u4 *>(&lds_new[0][16 * (tq / TB)]);
          if constexpr (EB == 1) {
            // V chunk: elements 4c .. 4c+3 of tokens tb*TB + 4u .. +3
            const int c = tq / (TB / 4), u = tq % (TB / 4);
            const int v0 = new_slot - (tb * TB + 4 * u);
            if ((unsigned)v0 < 4u) {
              const uint32_t nw = *reinterpret_cast<const uint32_t *>(&lds_new[1][4 * c]);
#pragma unroll
              for (int e = 0; e < 4; ++e)
                cv[k][e] = (cv[k][e] & ~(0xFFu << (8 * v0))) | (((nw >> (8 * e)) & 0xFFu) << (8 * v0));
            }
          } else {
            // V chunk: 4-byte column c of tokens tb*TB + u0 .. +3
            const int c = (4 * tq) / TB, u0 = (4 * tq) % TB;
            const int v0 = new_slot - (tb * TB + u0);
            if ((unsigned)v0 < 4u) {
              const uint32_t nw = *reinterpret_cast<const uint32_t *>(&lds_new[1][4 * c]);
#pragma unroll
              for (int e = 0; e < 4; ++e) cv[k][e] = e == v0 ? nw : cv[k][e];
            }
          }
          *reinterpret_cast<u4 *>(p.k_cache_w + tail_slice + 16 * (size_t)q) = ck[k];
          *reinterpret_cast<u4 *>(p.v_cache_w + tail_slice + 16 * (size_t)q) = cv[k];
        }
      }
      if constexpr (QUANT) {
        const size_t ssc = ((size_t)cow_from * Hkv + kvh) * BS;
        if (lane < BS) {
          const uint16_t ksc = lane == new_slot ? lds_new_sc[0] : p.k_scale_w[ssc + lane];
          const uint16_t vsc = lane == new_slot ? lds_new_sc[1] : p.v_scale_w[ssc + lane];
          p.k_scale_w[tail_sc + lane] = ksc;
          p.v_scale_w[tail_sc + lane] = vsc;
        }
      }
    }
  };

  // ---- per-wave running state ----
  float m = -INFINITY;   // running max of column r (base-2 scaled scores)
  float l = 0.0f;        // partial sum of this lane's 4 rows
  f4 acc[NACC];
#pragma unroll
  for (int a = 0; a < NACC; ++a) acc[a] = f4{0.f, 0.f, 0.f, 0.f};
  f4 accp = f4{0.f, 0.f, 0.f, 0.f};   // int8: sum_t P'_t of column r (every row)
  float vboost = kVBoost0;             // quantized V: the wave's boost b and the
  float vlim = kFoldMax / kVBoost0;    // largest V scale it admits (weights <= 1)

  const size_t kv_head_off = (size_t)kvh * SLICE;
  const size_t block_stride = (size_t)Hkv * SLICE;

  struct Tile {
    u4 k[NL];
    u4 v[NL];
    u2 ks, vs;   // fp16 scales of tokens 4g..4g+3 (quantized only)
    bool ok;
  };

  // Start the loads of tile `tile` (absolute), whose table entries are lane j
  // of tv (and tvb).  Lane (r, g) reads token r of the tile for K and tokens
  // 4g..4g+3 for V and the scales; with SPLIT, tokens 0-7 come from the first
  // block and 8-15 from the second.
  auto issue = [&](int tv, int tvb, int j, int tile, Tile &t) {
    int pa = __builtin_amdgcn_readlane(tv, j);
    if (SRC >= 0 && cow_from >= 0 && (SPLIT ? 2 * tile : tile / TPB) == tail_blk &&
        (unsigned)pa < (unsigned)p.num_blocks)
      pa = cow_from;
    // with SPLIT, a second block past the sequence's end (its tokens are all
    // masked) is read from the first block instead
    int pb = SPLIT && 2 * tile + 1 < nblk ? __builtin_amdgcn_readlane(tvb, j) : pa;
    if (SRC >= 0 && SPLIT && cow_from >= 0 && 2 * tile + 1 == tail_blk &&
        (unsigned)pb < (unsigned)p.num_blocks)
      pb = cow_from;
    t.ok = (unsigned)pa < (unsigned)p.num_blocks && (unsigned)pb < (unsigned)p.num_blocks;
    pa = t.ok ? pa : 0;
    pb = t.ok ? pb : 0;
    // Slices are runs of TB-token tiles (TB = 8 when SPLIT, else 16; a
    // 32-token block holds two): this tile's bytes start at tile_off.
    const int tq = SPLIT ? 0 : tile % TPB;               // tile within its block
    const size_t tile_off = (size_t)tq * (TB * D * EB);
    const int pk = SPLIT && r >= 8 ? pb : pa;            // block of this lane's K token
    const int pv = SPLIT && g >= 2 ? pb : pa;            // block of this lane's V tokens
    const int tk = SPLIT ? (r & 7) : r;                  // K token within its tile
    const int tv0 = SPLIT ? 4 * (g & 1) : 4 * g;         // first V token within its tile
    const uint8_t *kb = p.k_cache + (size_t)pk * block_stride + kv_head_off + tile_off;
    const uint8_t *vb = p.v_cache + (size_t)pv * block_stride + kv_head_off + tile_off;
#pragma unroll
    for (int i = 0; i < NL; ++i)
      t.k[i] = load16_stream(kb + (size_t)((4 * i + g) * TB + tk) * 16);
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      if constexpr (EB == 1)
        t.v[i] = load16_stream(vb + (size_t)((16 * i + r) * (TB / 4) + tv0 / 4) * 16);
      else
        t.v[i] = load16_stream(vb + (size_t)((16 * i + r) * TB + tv0) * 4);
    }
    if constexpr (QUANT) {
      const size_t so = ((size_t)pv * Hkv + kvh) * BS + tq * kTile + tv0;
      t.ks = *reinterpret_cast<const u2 *>(p.k_scale + so);
      t.vs = *reinterpret_cast<const u2 *>(p.v_scale + so);
    }
  };

  // Fold tile `tile` (its data already loaded) into the running state.
  auto consume = [&](int tile, Tile &t) {
    if constexpr (SRC >= 0) {
      // the tail tile: slot L - 1 takes the new token as staged in LDS
      if (step_wave && tile == tail_tile) {
        if (r == new_row) {
#pragma unroll
          for (int i = 0; i < NL; ++i) t.k[i] = *reinterpret_cast<const u4 *>(&lds_new[0][16 * (4 * i + g)]);
        }
        const int v0 = new_row - 4 * g;   // word (2- and 4-byte V) or byte (1-byte V)
        if ((unsigned)v0 < 4u) {
#pragma unroll
          for (int i = 0; i < NL; ++i) {
            const uint32_t nw = *reinterpret_cast<const uint32_t *>(&lds_new[1][4 * (16 * i + r)]);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              if constexpr (EB == 1)
                t.v[i][e] = (t.v[i][e] & ~(0xFFu << (8 * v0))) | (((nw >> (8 * e)) & 0xFFu) << (8 * v0));
              else
                t.v[i][e] = e == v0 ? nw : t.v[i][e];
            }
          }
          if constexpr (QUANT) {
            const uint32_t sh = 16 * (v0 & 1), keep = ~(0xFFFFu << sh);
            const uint32_t nk = (uint32_t)lds_new_sc[0] << sh, nv = (uint32_t)lds_new_sc[1] << sh;
            if (v0 < 2) {
              t.ks[0] = (t.ks[0] & keep) | nk;
              t.vs[0] = (t.vs[0] & keep) | nv;
            } else {
              t.ks[1] = (t.ks[1] & keep) | nk;
              t.vs[1] = (t.vs[1] & keep) | nv;
            }
          }
        }
      }
    }
    // q.K for the tile: S^T[token 4g+v][head r] in sc[v]
    f4 sc = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      if constexpr (KV == PKV_F32) {
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)
          sc = __builtin_amdgcn_mfma_f32_16x16x4f32(as_f32(t.k[i][jj]), qf32[i][jj], sc, 0, 0,
                                                    0);
      } else if constexpr (KV == PKV_F16) {
        sc = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(h8, t.k[i]), qf16[i][0],
                                                    sc, 0, 0, 0);
      } else {
        h8 lo, hi;
        k_codes16<KV>(t.k[i], lo, hi);
        sc = __builtin_amdgcn_mfma_f32_16x16x32_f16(lo, qf16[i][0], sc, 0, 0, 0);
        sc = __builtin_amdgcn_mfma_f32_16x16x32_f16(hi, qf16[i][QUANT ? 1 : 0], sc, 0, 0, 0);
      }
    }
    if (!t.ok) return;  // table entry outside the pool: tile skipped
    const int tok0 = tile * kTile + 4 * g;
    float x[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      x[v] = sc[v] * p.qk_scale;
      if constexpr (QUANT) x[v] *= (float)as_h2(t.ks[v >> 1])[v & 1];
    }
    u4 vw[NL];
#pragma unroll
    for (int i = 0; i < NL; ++i) vw[i] = t.v[i];
    u2 vs = t.vs;
    // Only a sequence's last tile can be partial (uniform per wave).  Its
    // unwritten slots may hold anything, NaN included: their scores become
    // -inf and their V words (and V scales) zero.
    if (__builtin_expect((tile + 1) * kTile > L, 0)) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const bool valid = tok0 + v < L;
        x[v] = valid ? x[v] : -INFINITY;
        if constexpr (!QUANT) {   // word v holds token 4g+v
#pragma unroll
          for (int i = 0; i < NL; ++i) vw[i][v] = valid ? vw[i][v] : 0u;
        }
      }
      if constexpr (QUANT) {      // byte v of every word holds token 4g+v
        uint32_t keep = 0u;
#pragma unroll
        for (int v = 0; v < 4; ++v) keep |= (tok0 + v < L ? 0xFFu : 0u) << (8 * v);
#pragma unroll
        for (int i = 0; i < NL; ++i)
#pragma unroll
          for (int e = 0; e < 4; ++e) vw[i][e] &= keep;
        const uint32_t keep0 = (tok0 + 0 < L ? 0xFFFFu : 0u) | (tok0 + 1 < L ? 0xFFFF0000u : 0u);
        const uint32_t keep1 = (tok0 + 2 < L ? 0xFFFFu : 0u) | (tok0 + 3 < L ? 0xFFFF0000u : 0u);
        vs = u2{vs[0] & keep0, vs[1] & keep1};
      }
    }
    float bm = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
    bm = fmaxf(bm, xor16(bm));
    bm = fmaxf(bm, xor32(bm));
    const float mn = fmaxf(m, bm);
    // Rescale only when some column's running max rose (m = -inf before the
    // first tile, so the first tile always rescales: alpha = 0).
    if (__builtin_amdgcn_ballot_w64(mn > m) != 0) {
      const float alpha = exp2f(m - mn);
      l *= alpha;
#pragma unroll
      for (int a = 0; a < NACC; ++a) acc[a] *= alpha;
      if constexpr (KV == PKV_I8) accp *= alpha;
      m = mn;
    }
    float pr[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) pr[v] = exp2f(x[v] - m);
    l += (pr[0] + pr[1]) + (pr[2] + pr[3]);

    // P.V: the lane's pr[v] is P^T[token 4g+v][head r], the B operand as is.
    if constexpr (KV == PKV_F32) {
#pragma unroll
      for (int i = 0; i < NL; ++i)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)
          acc[i] = __builtin_amdgcn_mfma_f32_16x16x4f32(as_f32(vw[i][jj]), pr[jj], acc[i], 0,
                                                        0, 0);
    } else if constexpr (KV == PKV_F16) {
      const h4 pb = h4{(_Float16)pr[0], (_Float16)pr[1], (_Float16)pr[2], (_Float16)pr[3]};
#pragma unroll
      for (int i = 0; i < NL; ++i) {
        // word v = token 4g+v, halves (dim 2c, dim 2c+1) of column c = 16i + r
        const uint32_t lo01 = __builtin_amdgcn_perm(vw[i][1], vw[i][0], 0x05040100u);
        const uint32_t lo23 = __builtin_amdgcn_perm(vw[i][3], vw[i][2], 0x05040100u);
        const uint32_t hi01 = __builtin_amdgcn_perm(vw[i][1], vw[i][0], 0x07060302u);
        const uint32_t hi23 = __builtin_amdgcn_perm(vw[i][3], vw[i][2], 0x07060302u);
        acc[2 * i] = __builtin_amdgcn_mfma_f32_16x16x16f16(
            __builtin_bit_cast(h4, u2{lo01, lo23}), pb, acc[2 * i], 0, 0, 0);
        acc[2 * i + 1] = __builtin_amdgcn_mfma_f32_16x16x16f16(
            __builtin_bit_cast(h4, u2{hi01, hi23}), pb, acc[2 * i + 1], 0, 0, 0);
      }
    } else {
      float sv[4];
#pragma unroll
      for (int v = 0; v < 4; ++v) sv[v] = (float)as_h2(vs[v >> 1])[v & 1];
      // A V scale above what the wave's boost admits (never one of an fp16
      // value): lower the boost first.  Lanes of one row group g hold the
      // same tokens' scales.
      const float smax = fmaxf(fmaxf(fabsf(sv[0]), fabsf(sv[1])), fmaxf(fabsf(sv[2]), fabsf(sv[3])));
      if (__builtin_expect(__builtin_amdgcn_ballot_w64(smax > vlim) != 0, 0)) {
        float sw = fmaxf(smax, xor16(smax));
        sw = fmaxf(sw, xor32(sw));
        const float nb = lower_boost(vboost, sw, 1.0f);
        const float f = nb / vboost;
#pragma unroll
        for (int a = 0; a < NACC; ++a) acc[a] *= f;
        if constexpr (KV == PKV_I8) accp *= f;
        vboost = nb;
        vlim = kFoldMax / nb;
      }
      float ps[4];
#pragma unroll
      for (int v = 0; v < 4; ++v) ps[v] = pr[v] * sv[v] * vboost;
      const h4 pb = h4{(_Float16)ps[0], (_Float16)ps[1], (_Float16)ps[2], (_Float16)ps[3]};
      if constexpr (KV == PKV_I8) {
        const h4 ones = h4{(_Float16)1.0f, (_Float16)1.0f, (_Float16)1.0f, (_Float16)1.0f};
        accp = __builtin_amdgcn_mfma_f32_16x16x16f16(ones, pb, accp, 0, 0, 0);
      }
      // word e of load i: element 4(16i+r)+e of tokens 4g..4g+3 (1-byte V layout)
#pragma unroll
      for (int i = 0; i < NL; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          acc[4 * i + e] = __builtin_amdgcn_mfma_f32_16x16x16f16(codes4_to_h4<KV>(vw[i][e]), pb,
                                                                 acc[4 * i + e], 0, 0, 0);
    }
  };

  // The accumulators as true sums of weight times value: the int8 bias taken
  // out and the wave's V-scale boost undone (a power of two: exact).
  auto unbias = [&]() __attribute__((always_inline)) {
    if constexpr (KV == PKV_I8) {
#pragma unroll
      for (int a = 0; a < NACC; ++a) acc[a] -= kI8Bias * accp;
    }
    if constexpr (QUANT) {
      const float ib = 1.0f / vboost;
#pragma unroll
      for (int a = 0; a < NACC; ++a) acc[a] *= ib;
    }
  };

  // ---- wave walks: a wave ends its piece (or partition) alone ----
  // Lane (r, g) holds head r's elements E*(16i + 4g + v) + e in acc[E*i + e][v]:
  // for each i the 4E consecutive elements from E*(16i + 4g), the E quads
  // c = E*i + j (j < E).  The normalized row goes to `out` (direct) or, with
  // its base-2 log-sum-exp m + log2(l), to partial row row0 + r * rstride of
  // the workspace: at once for the wave's last output, else through an LDS
  // slot.  Then the state restarts.
  auto emit = [&](bool direct, size_t row0, size_t rstride, bool last_out, int info_u, int info_fw,
                  int info_n) __attribute__((always_inline)) {
    unbias();
    float lt = l + xor16(l);
    lt += xor32(lt);
    const float inv = lt > 0.0f ? 1.0f / lt : 0.0f;
    f4 q[NACC];
#pragma unroll
    for (int i = 0; i < NACC / E; ++i) {
      float vals[4 * E];
#pragma unroll
      for (int v = 0; v < 4; ++v)
#pragma unroll
        for (int e = 0; e < E; ++e) vals[v * E + e] = acc[E * i + e][v] * inv;
#pragma unroll
      for (int j = 0; j < E; ++j)
        q[E * i + j] = f4{vals[4 * j], vals[4 * j + 1], vals[4 * j + 2], vals[4 * j + 3]};
    }
    const float lse = m + log2f(lt);
    const Staged d{direct ? ((size_t)s * H + kvh * G) * D : row0, rstride, direct ? 1 : 0, info_u,
                   info_fw, info_n};
    if (last_out) {
      store_output(d, q, lse);
    } else {
      if (nst == KST) flush_staged();
#pragma unroll
      for (int c = 0; c < NACC; ++c) lds_st[w][nst][c][lane] = q[c];
      if (g == 0) lds_st_lse[w][nst][r] = lse;
      if (lane == 0) lds_st_dst[w][nst] = d;
      ++nst;
    }
    m = -INFINITY;
    l = 0.0f;
#pragma unroll
    for (int a = 0; a < NACC; ++a) acc[a] = f4{0.f, 0.f, 0.f, 0.f};
    accp = f4{0.f, 0.f, 0.f, 0.f};
    vboost = kVBoost0;
    vlim = kFoldMax / kVBoost0;
  };
  // ---- split and runs walks: the four wave states through LDS ----
  // The waves' states go to LDS (the barrier waits for LDS only: loads and
  // the fused step's stores may be in flight), and combine() merges the four
  // of element quad (head hh, dims d0..d0+3) into the normalized output and
  // its base-2 log-sum-exp (M + log2 den).
  auto publish = [&]() __attribute__((always_inline)) {
    unbias();
    float lt = l + xor16(l);
    lt += xor32(lt);
    if (g == 0) {
      lds_m[w][r] = m;
      lds_l[w][r] = lt;
    }
    if (r < G) {   // columns r >= G repeat head 0 and are never read
#pragma unroll
      for (int a = 0; a < NACC; ++a) {
        const int i = a / E, e = a % E;
#pragma unroll
        for (int v = 0; v < 4; ++v) lds_o[w][r][E * (16 * i + 4 * g + v) + e] = acc[a][v];
      }
    }
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  };
  auto combine = [&](int hh, int d0, f4 &o, float &M, float &den) __attribute__((always_inline)) {
    M = lds_m[0][hh];
#pragma unroll
    for (int ww = 1; ww < kDecodeWaves; ++ww) M = fmaxf(M, lds_m[ww][hh]);
    f4 num = f4{0.f, 0.f, 0.f, 0.f};
    den = 0.f;
#pragma unroll
    for (int ww = 0; ww < kDecodeWaves; ++ww) {
      const float c = exp2f(lds_m[ww][hh] - M);
      num += c * *reinterpret_cast<const f4 *>(&lds_o[ww][hh][d0]);
      den += c * lds_l[ww][hh];
    }
    o = num / den;
  };
  // Runs: a partition other than the run's last ends.  Its partial goes to
  // lds_stage (thread t keeps element quads t, t + 64 * kDecodeWaves, ... and
  // stores them itself after the walk), and the state restarts.  All waves
  // reach this at the same step; the second barrier frees lds_o for the next.
  int flush_at = WALK == kWalkRuns && nparts_run > 1 ? tpw - 1 : -1;   // step that ends
  int staged = 0;                                                      // partition `staged`
  auto end_step = [&](int k) __attribute__((always_inline)) {
    if constexpr (WALK != kWalkRuns) return;
    if (__builtin_expect(k != flush_at, 1)) return;
    publish();
    for (int qd = threadIdx.x; qd < G * D / 4; qd += 64 * kDecodeWaves) {
      const int hh = 4 * qd / D, d0 = 4 * qd % D;
      f4 o;
      float M, den;
      combine(hh, d0, o, M, den);
      float *row = lds_stage + (staged * G + hh) * (D + 4);
      *reinterpret_cast<f4 *>(row + d0) = o;
      if (d0 == 0) row[D] = M + log2f(den);
    }
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    m = -INFINITY;
    l = 0.0f;
#pragma unroll
    for (int a = 0; a < NACC; ++a) acc[a] = f4{0.f, 0.f, 0.f, 0.f};
    accp = f4{0.f, 0.f, 0.f, 0.f};
    ++staged;
    flush_at = staged < nparts_run - 1 ? flush_at + tpw : -1;
  };

  const PrioSteps<WALK == kWalkRuns> prio(nt_w);
  // ---- tile loop: a ring of NB tiles, each refilled right after use ----
  // The wave's tiles are walked in chunks of up to 64 (one table entry per
  // lane).  Within a chunk the steady-state rounds issue every load
  // unconditionally, so the compiler's wait counts stay exact and NB - 1
  // tiles remain in flight while one is consumed; only the last round of a
  // chunk guards its loads.
  for (int c0 = 0; c0 < nt_w; c0 += 64) {
    const int nc = min(64, nt_w - c0);
    const int tv = tv_next, tvb = tvb_next;
    const int t0 = wfirst + c0 * TS;   // tile of chunk entry 0
    Tile ring[NB];
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const int jj = j < nc ? j : nc - 1;
      issue(tv, tvb, jj, t0 + jj * TS, ring[j]);
    }
    if (c0 == tail_c0) step_write(tv, tvb, tail_step - c0);   // the ring's loads are in flight
    int k0 = 0;
    for (; k0 + 2 * NB <= nc; k0 += NB) {
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        consume(t0 + (k0 + j) * TS, ring[j]);
        issue(tv, tvb, k0 + j + NB, t0 + (k0 + j + NB) * TS, ring[j]);
        end_step(c0 + k0 + j);
        prio.at(c0 + k0 + j);
      }
    }
    // last round: the ring holds entries k0 .. k0+NB-1 (those < nc), at most
    // NB - 1 further entries remain to be loaded
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      if (k0 + j < nc) consume(t0 + (k0 + j) * TS, ring[j]);
      if (k0 + j + NB < nc) issue(tv, tvb, k0 + j + NB, t0 + (k0 + j + NB) * TS, ring[j]);
      if (k0 + j < nc) {
        end_step(c0 + k0 + j);
        prio.at(c0 + k0 + j);
      }
    }
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      if (k0 + NB + j < nc) {
        consume(t0 + (k0 + NB + j) * TS, ring[j]);
        end_step(c0 + k0 + NB + j);
        prio.at(c0 + k0 + NB + j);
      }
    }
    if (c0 + 64 < nt_w) tv_next = load_tv(c0 + 64, p.max_blocks, &tvb_next);
  }

  if (SRC >= 0 && step_wave && tail_ok) {
    step_store();
    if (cow_from >= 0 && cow_from != tail_phys) cow_copy();
  }

  if constexpr (WALK == kWalkStream) {
    // The piece's output: direct when it is the whole unit, else a partial in
    // slot 2 * wave + 1 (a unit's first piece, which continues in the next
    // share) or 2 * wave (a piece that began in an earlier share).  The first
    // piece also records the unit's first wave and piece count for the merge.
    const int u = s * Hkv + kvh;
    const bool direct = piece_head && piece_tail;
    const int slot = 2 * wave_id + (piece_head ? 1 : 0);
    const int64_t last_wave = (sg + sspan - 1) / share;   // sg: the unit's first tile
    const bool last_out = sg + (piece_end - first) >= sg_end;
    emit(direct, (size_t)slot * G, 1, last_out, piece_head ? u : -1, wave_id,
         (int)(last_wave - wave_id + 1));
    // past the piece; after a sequence's last kv head, on to the next
    // sequence that has tiles
    sg += piece_end - first;
    if (piece_tail && kvh == Hkv - 1) {
      do {
        sc += sspan;
        ++ss;
        sspan = ss < p.num_seqs ? span_of(p.seq_lens[ss]) : 1;
      } while (sspan == 0);
    }
    continue;
  } else {
    // ---- the run's last partition (the split walk's only one) ----
    publish();
    const bool direct = nparts_s == 1 && npre == 0;
    const int part = part0 + nparts_run - 1;
    for (int qd = threadIdx.x; qd < G * D / 4; qd += 64 * kDecodeWaves) {
      const int hh = 4 * qd / D, d0 = 4 * qd % D;
      f4 o;
      float M, den;
      combine(hh, d0, o, M, den);
      const int h = kvh * G + hh;
      if (direct) {
        const size_t idx = ((size_t)s * H + h) * D + d0;
        if (out_vec) {
          store_out4<OUT>(p.out, idx, o);
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i) store_out<OUT>(p.out, idx + i, o[i]);
        }
      } else {
        const size_t row = ((size_t)s * H + h) * p.ws_stride + part;
        *reinterpret_cast<f4 *>(p.ws_o + row * D + d0) = o;
        if (d0 == 0) p.ws_lse[row] = M + log2f(den);
      }
    }
    // the staged partials of the run's earlier partitions (each thread stores
    // the elements it staged)
    if constexpr (WALK == kWalkRuns)
    for (int j = 0; j < nparts_run - 1; ++j) {
      for (int qd = threadIdx.x; qd < G * D / 4; qd += 64 * kDecodeWaves) {
        const int hh = 4 * qd / D, d0 = 4 * qd % D;
        const float *src = lds_stage + (j * G + hh) * (D + 4);
        const size_t row = ((size_t)s * H + kvh * G + hh) * p.ws_stride + part0 + j;
        *reinterpret_cast<f4 *>(p.ws_o + row * D + d0) = *reinterpret_cast<const f4 *>(src + d0);
        if (d0 == 0) p.ws_lse[row] = src[D];
      }
    }
    return;
  }
  }   // pieces
}

}  // namespace
}  // namespace pkv
