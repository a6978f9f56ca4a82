// PagedAttention decode for gfx950 (CDNA4): launches, and the log-sum-exp
// merge of split sequences.  The decode kernel itself (decode_kernel.h) is
// built here for the split walk (a workgroup per partition); the runs and
// stream walks are built in decode_runs.hip and decode_stream.hip.
#include "decode_kernel.h"

namespace pkv {
namespace {

// Log-sum-exp merge of the partials of sequences that used more than one
// partition or stream piece (and of a sequence's suffix partials with its
// shared-prefix partials).  After the stream walk it also writes the zero rows
// of empty sequences, which no wave visits.  A thread owns 4 output elements
// of one (sequence, head) row and
// folds the partials q = qg, qg + QG, ... into a running (max, sum, weighted
// sum) -- one pass, no separate maximum; the QG groups of a row are then
// combined through LDS.  A workgroup of kMergeThreads holds 256 / (D/4 * QG)
// rows.
constexpr int kMergeThreads = 256;

template <int D, int OUT, int QG>
__global__ __launch_bounds__(kMergeThreads) void merge_kernel(DecodeParams p) {
  constexpr int TPH = D / 4;                       // threads per row and partial group
  constexpr int RPW = kMergeThreads / (TPH * QG);  // rows per workgroup
  static_assert(RPW >= 1, "partial groups");
  __shared__ f4 red_o[QG > 1 ? kMergeThreads : 1];
  __shared__ float red_m[QG > 1 ? kMergeThreads : 1];
  __shared__ float red_z[QG > 1 ? kMergeThreads : 1];
  const int t = threadIdx.x;
  const int rl = t / (TPH * QG);
  const int qg = (t / TPH) % QG;
  const int dv = t % TPH;
  const int row = blockIdx.x * RPW + rl;           // s * H + h
  const bool live_row = row < p.num_seqs * p.num_heads;
  const bool stream = p.walk == kWalkStream;
  int np = 0, npre = 0, fw = 0, hh = 0;
  bool zero_row = false;
  // The row's records are requested together, not one after the other.
  if (live_row) {
    const int s = row / p.num_heads;
    if (stream) {
      // a unit's pieces: slots 2 * fw + 1 (its first piece), then 2 * (fw + j);
      // the record (one 8-byte word: the workspace and the record's offset in
      // it are 256-byte aligned) is read with the length (it is stale for an
      // empty sequence)
      const int h = row - s * p.num_heads;
      hh = h % p.group;
      const int u = s * p.num_kv_heads + h / p.group;
      const int L = p.seq_lens[s];
      const int2 rec = *reinterpret_cast<const int2 *>(p.ws_info + 2 * u);
      fw = rec.x;
      zero_row = L <= 0;
      const bool none = zero_row | (fw < 0) | (fw >= p.stream_waves);
      np = none ? 0 : rec.y;
      np = np < p.stream_waves - fw ? np : p.stream_waves - fw;
    } else {
      int L = p.seq_lens[s];
      const int g = p.seq_group != nullptr ? p.seq_group[s] : -1;
      L = L < 0 ? 0 : (L > p.max_blocks * p.block_size ? p.max_blocks * p.block_size : L);
      const int ntile = (L + kTile - 1) / kTile;
      np = (ntile + p.part_tiles - 1) / p.part_tiles;
      npre = prefix_parts_of_group(p, g);
    }
  }
  // rows with one partition (or piece) and no prefix were written by the
  // decode kernel
  const bool merge = live_row && (np > 1 || npre > 0 || zero_row);
  const int nq = zero_row ? 0 : np + npre;
  float m = -INFINITY, z = 0.0f;
  f4 acc = f4{0.f, 0.f, 0.f, 0.f};
  if (merge) {
    const size_t base = (size_t)row * p.ws_stride;
    const f4 *o = reinterpret_cast<const f4 *>(p.ws_o) + dv;
    // kChunk partials at a time, their loads issued together (a guard per
    // partial would make each load wait for the one before): a slot past the
    // row's last partial reads that partial again and its term is dropped.
    constexpr int kChunk = 8;
    for (int q0 = qg; q0 < nq; q0 += kChunk * QG) {
      float lq[kChunk];
      f4 oq[kChunk];
#pragma unroll
      for (int j = 0; j < kChunk; ++j) {
        const int q = min(q0 + j * QG, nq - 1);
        const size_t fi = stream ? (size_t)(2 * (fw + q) + (q == 0 ? 1 : 0)) * p.group + hh
                                 : base + (q < np ? q : p.ws_pre + (q - np));
        lq[j] = p.ws_lse[fi];
        oq[j] = o[fi * (D / 4)];
      }
#pragma unroll
      for (int j = 0; j < kChunk; ++j) {
        if (q0 + j * QG < nq) {
          const float mn = fmaxf(m, lq[j]);
          const float a = exp2f(m - mn), b = exp2f(lq[j] - mn);
          acc = acc * a + oq[j] * b;
          z = z * a + b;
          m = mn;
        }
      }
    }
  }
  if constexpr (QG > 1) {
    red_o[t] = acc;
    red_m[t] = m;
    red_z[t] = z;
    __syncthreads();
    if (qg != 0) return;
    float M = m;
#pragma unroll
    for (int i = 1; i < QG; ++i) M = fmaxf(M, red_m[t + i * TPH]);
    acc = f4{0.f, 0.f, 0.f, 0.f};
    z = 0.0f;
#pragma unroll
    for (int i = 0; i < QG; ++i) {
      const float mi = red_m[t + i * TPH];
      const float c = mi == -INFINITY ? 0.0f : exp2f(mi - M);
      acc += red_o[t + i * TPH] * c;
      z += red_z[t + i * TPH] * c;
    }
  }
  if (!merge) return;
  const f4 r = zero_row ? f4{0.f, 0.f, 0.f, 0.f} : acc * (1.0f / z);
  const size_t oi = (size_t)row * D + 4 * dv;
  // out needs only element alignment; vector stores when it allows them
  if ((reinterpret_cast<uintptr_t>(p.out) & (OUT == PKV_F32 ? 15u : 7u)) == 0) {
    store_out4<OUT>(p.out, oi, r);
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) store_out<OUT>(p.out, oi + i, r[i]);
  }
}

// Partial groups per row for up to `nq` partials per row (at most 8 partials
// per thread when the row has room for more groups).
inline int merge_groups(int nq, int head_dim) {
  const int max_groups = kMergeThreads / (head_dim / 4);
  int g = 1;
  while (g < max_groups && g * 8 < nq) g *= 2;
  return g;
}

template <int D, int OUT, int QG>
hipError_t launch_merge_g(const DecodeParams &p, hipStream_t stream) {
  constexpr int RPW = kMergeThreads / (D / 4 * QG);
  const int rows = p.num_seqs * p.num_heads;
  hipLaunchKernelGGL((merge_kernel<D, OUT, QG>), dim3((rows + RPW - 1) / RPW),
                     dim3(kMergeThreads), 0, stream, p);
  return hipGetLastError();
}

template <int D, int OUT>
hipError_t launch_merge_d(const DecodeParams &p, hipStream_t stream) {
  switch (merge_groups(p.ws_stride, D)) {
    case 1: return launch_merge_g<D, OUT, 1>(p, stream);
    case 2: return launch_merge_g<D, OUT, 2>(p, stream);
    case 4: return launch_merge_g<D, OUT, 4>(p, stream);
    case 8: return launch_merge_g<D, OUT, 8>(p, stream);
    default:
      if constexpr (D == 64) return launch_merge_g<D, OUT, 16>(p, stream);
      else return launch_merge_g<D, OUT, 8>(p, stream);
  }
}

template <int KV, int D, int OUT, int SRC, int BS>
hipError_t launch_typed(const DecodeParams &p, hipStream_t stream) {
  hipError_t err;
  if (p.walk == kWalkRuns) {
    err = launch_decode_runs(p, KV, SRC >= 0, OUT, D, stream);
  } else if (p.walk == kWalkStream) {
    err = launch_decode_stream(p, KV, SRC >= 0, OUT, D, stream);
  } else {
    const int64_t grid = decode_grid(p.num_units, p.num_runs);
    hipLaunchKernelGGL((decode_kernel<KV, D, OUT, SRC, BS, kWalkSplit>), dim3((unsigned)grid),
                       dim3(64 * kDecodeWaves), 0, stream, p);
    err = hipGetLastError();
  }
  // with shared prefixes the caller launches the merge after the prefix pass
  if (err != hipSuccess || p.seq_group) return err;
  if (p.walk != kWalkStream && p.num_parts <= 1) return err;
  return launch_merge_d<D, OUT>(p, stream);
}

template <int KV, int D, int OUT, int SRC>
hipError_t launch_bs(const DecodeParams &p, hipStream_t stream) {
  switch (p.block_size) {
    case 8: return launch_typed<KV, D, OUT, SRC, 8>(p, stream);
    case 32: return launch_typed<KV, D, OUT, SRC, 32>(p, stream);
    default: return launch_typed<KV, D, OUT, SRC, 16>(p, stream);
  }
}

template <int KV, int D, int SRC>
hipError_t launch_out(const DecodeParams &p, int out_dtype, hipStream_t stream) {
  return out_dtype == PKV_F32 ? launch_bs<KV, D, PKV_F32, SRC>(p, stream)
                              : launch_bs<KV, D, PKV_F16, SRC>(p, stream);
}

template <int KV, int SRC>
hipError_t launch_d(const DecodeParams &p, int out_dtype, int head_dim, hipStream_t stream) {
  return head_dim == 64 ? launch_out<KV, 64, SRC>(p, out_dtype, stream)
                        : launch_out<KV, 128, SRC>(p, out_dtype, stream);
}

}  // namespace

hipError_t launch_merge(const DecodeParams &p, int out_dtype, int head_dim, hipStream_t stream) {
  if (head_dim == 64)
    return out_dtype == PKV_F32 ? launch_merge_d<64, PKV_F32>(p, stream)
                                : launch_merge_d<64, PKV_F16>(p, stream);
  return out_dtype == PKV_F32 ? launch_merge_d<128, PKV_F32>(p, stream)
                              : launch_merge_d<128, PKV_F16>(p, stream);
}

hipError_t launch_decode(const DecodeParams &p, int cache_dtype, int out_dtype, int head_dim,
                         hipStream_t stream) {
  switch (cache_dtype) {
    case PKV_F32: return launch_d<PKV_F32, -1>(p, out_dtype, head_dim, stream);
    case PKV_F16: return launch_d<PKV_F16, -1>(p, out_dtype, head_dim, stream);
    case PKV_I8: return launch_d<PKV_I8, -1>(p, out_dtype, head_dim, stream);
    default: return launch_d<PKV_E4M3, -1>(p, out_dtype, head_dim, stream);
  }
}

// New tokens are fp32 for an fp32 cache and fp16 otherwise (checked by the caller).
hipError_t launch_decode_step(const DecodeParams &p, int cache_dtype, int src_dtype,
                              int out_dtype, int head_dim, hipStream_t stream) {
  (void)src_dtype;
  switch (cache_dtype) {
    case PKV_F32: return launch_d<PKV_F32, PKV_F32>(p, out_dtype, head_dim, stream);
    case PKV_F16: return launch_d<PKV_F16, PKV_F16>(p, out_dtype, head_dim, stream);
    case PKV_I8: return launch_d<PKV_I8, PKV_F16>(p, out_dtype, head_dim, stream);
    default: return launch_d<PKV_E4M3, PKV_F16>(p, out_dtype, head_dim, stream);
  }
}

}  // namespace pkv
