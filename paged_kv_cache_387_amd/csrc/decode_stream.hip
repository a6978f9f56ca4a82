// PagedAttention decode for gfx950: the kernel of decode_kernel.h built for
// the stream walk (the batch's tiles dealt to the grid's waves in equal
// shares).  A translation unit of its own keeps the builds in parallel.
#include "decode_kernel.h"

namespace pkv {
namespace {

template <int KV, int D, int OUT, int SRC, int BS>
hipError_t stream_typed(const DecodeParams &p, hipStream_t stream) {
  const int64_t grid = p.stream_waves / kDecodeWaves;
  hipLaunchKernelGGL((decode_kernel<KV, D, OUT, SRC, BS, kWalkStream>), dim3((unsigned)grid),
                     dim3(64 * kDecodeWaves), 0, stream, p);
  return hipGetLastError();
}

template <int KV, int D, int OUT, int SRC>
hipError_t stream_bs(const DecodeParams &p, hipStream_t stream) {
  switch (p.block_size) {
    case 8: return stream_typed<KV, D, OUT, SRC, 8>(p, stream);
    case 32: return stream_typed<KV, D, OUT, SRC, 32>(p, stream);
    default: return stream_typed<KV, D, OUT, SRC, 16>(p, stream);
  }
}

template <int KV, int SRC>
hipError_t stream_d(const DecodeParams &p, int out_dtype, int head_dim, hipStream_t stream) {
  if (head_dim == 64)
    return out_dtype == PKV_F32 ? stream_bs<KV, 64, PKV_F32, SRC>(p, stream)
                                : stream_bs<KV, 64, PKV_F16, SRC>(p, stream);
  return out_dtype == PKV_F32 ? stream_bs<KV, 128, PKV_F32, SRC>(p, stream)
                              : stream_bs<KV, 128, PKV_F16, SRC>(p, stream);
}

}  // namespace

// The step's new tokens are fp32 for an fp32 cache and fp16 otherwise, as in
// launch_decode_step.
hipError_t launch_decode_stream(const DecodeParams &p, int cache_dtype, bool step, int out_dtype,
                                int head_dim, hipStream_t stream) {
  switch (cache_dtype) {
    case PKV_F32:
      return step ? stream_d<PKV_F32, PKV_F32>(p, out_dtype, head_dim, stream)
                  : stream_d<PKV_F32, -1>(p, out_dtype, head_dim, stream);
    case PKV_F16:
      return step ? stream_d<PKV_F16, PKV_F16>(p, out_dtype, head_dim, stream)
                  : stream_d<PKV_F16, -1>(p, out_dtype, head_dim, stream);
    case PKV_I8:
      return step ? stream_d<PKV_I8, PKV_F16>(p, out_dtype, head_dim, stream)
                  : stream_d<PKV_I8, -1>(p, out_dtype, head_dim, stream);
    default:
      return step ? stream_d<PKV_E4M3, PKV_F16>(p, out_dtype, head_dim, stream)
                  : stream_d<PKV_E4M3, -1>(p, out_dtype, head_dim, stream);
  }
}

}  // namespace pkv
