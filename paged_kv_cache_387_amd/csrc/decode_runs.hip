// PagedAttention decode for gfx950: the kernel of decode_kernel.h built for
// the runs walk (a workgroup walks a run of consecutive partitions, each
// ending in its own partial).  A translation unit of its own keeps the
// builds in parallel and the one-partition kernels in decode.hip free of the
// partition-end code.
#include "decode_kernel.h"

namespace pkv {
namespace {

template <int KV, int D, int OUT, int SRC, int BS>
hipError_t runs_typed(const DecodeParams &p, hipStream_t stream) {
  const int64_t grid = decode_grid(p.num_units, p.num_runs);
  hipLaunchKernelGGL((decode_kernel<KV, D, OUT, SRC, BS, kWalkRuns>), dim3((unsigned)grid),
                     dim3(64 * kDecodeWaves), 0, stream, p);
  return hipGetLastError();
}

template <int KV, int D, int OUT, int SRC>
hipError_t runs_bs(const DecodeParams &p, hipStream_t stream) {
  switch (p.block_size) {
    case 8: return runs_typed<KV, D, OUT, SRC, 8>(p, stream);
    case 32: return runs_typed<KV, D, OUT, SRC, 32>(p, stream);
    default: return runs_typed<KV, D, OUT, SRC, 16>(p, stream);
  }
}

template <int KV, int SRC>
hipError_t runs_d(const DecodeParams &p, int out_dtype, int head_dim, hipStream_t stream) {
  if (head_dim == 64)
    return out_dtype == PKV_F32 ? runs_bs<KV, 64, PKV_F32, SRC>(p, stream)
                                : runs_bs<KV, 64, PKV_F16, SRC>(p, stream);
  return out_dtype == PKV_F32 ? runs_bs<KV, 128, PKV_F32, SRC>(p, stream)
                              : runs_bs<KV, 128, PKV_F16, SRC>(p, stream);
}

}  // namespace

// The step's new tokens are fp32 for an fp32 cache and fp16 otherwise, as in
// launch_decode_step.
hipError_t launch_decode_runs(const DecodeParams &p, int cache_dtype, bool step, int out_dtype,
                              int head_dim, hipStream_t stream) {
  switch (cache_dtype) {
    case PKV_F32:
      return step ? runs_d<PKV_F32, PKV_F32>(p, out_dtype, head_dim, stream)
                  : runs_d<PKV_F32, -1>(p, out_dtype, head_dim, stream);
    case PKV_F16:
      return step ? runs_d<PKV_F16, PKV_F16>(p, out_dtype, head_dim, stream)
                  : runs_d<PKV_F16, -1>(p, out_dtype, head_dim, stream);
    case PKV_I8:
      return step ? runs_d<PKV_I8, PKV_F16>(p, out_dtype, head_dim, stream)
                  : runs_d<PKV_I8, -1>(p, out_dtype, head_dim, stream);
    default:
      return step ? runs_d<PKV_E4M3, PKV_F16>(p, out_dtype, head_dim, stream)
                  : runs_d<PKV_E4M3, -1>(p, out_dtype, head_dim, stream);
  }
}

}  // namespace pkv
