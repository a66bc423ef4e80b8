// calib.hip -- measured ceilings of the running device, reported beside the
// published peaks.  The matrix-unit loop: every wave runs kChains
// independent chains of the prefill's main product shape (16x16x32 fp16 in,
// fp32 accumulate) for n_iter rounds; nothing but the MFMAs sits in the loop,
// so the launch time over the flops is the rate the matrix units sustain.
// The streaming pass: every 16-byte piece of a buffer read and written back
// in place with nontemporal accesses, the decode step's traffic pattern
// (each state read once and written once) without its arithmetic.
#include "common.h"
#include "launch.h"

namespace gdn {

namespace {

constexpr int kChains = 8;
constexpr int kLoopThreads = 256;

__global__ __launch_bounds__(kLoopThreads) void mfma_loop_kernel(int n_iter, float* out) {
  const int lane = threadIdx.x & 63;
  half8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = static_cast<_Float16>(static_cast<float>((lane + i) & 7) * 0.125f);
    b[i] = static_cast<_Float16>(static_cast<float>((lane * 3 + i) & 7) * -0.0625f);
  }
  floatx4 acc[kChains];
#pragma unroll
  for (int c = 0; c < kChains; ++c) acc[c] = floatx4{0.f, 0.f, 0.f, 0.f};
  for (int it = 0; it < n_iter; ++it) {
#pragma unroll
    for (int c = 0; c < kChains; ++c) acc[c] = mfma32(a, b, acc[c]);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kChains; ++c) s += acc[c][0] + acc[c][1] + acc[c][2] + acc[c][3];
  if (lane == 0) out[(blockIdx.x * kLoopThreads + threadIdx.x) >> 6] = s;
}

// x ^= key over n16 16-byte pieces, grid-stride (key = 0 leaves the data as
// it was; as a run-time value it keeps both accesses)
typedef unsigned int u32x4v __attribute__((ext_vector_type(4)));
__global__ __launch_bounds__(256) void stream_inplace_kernel(u32x4v* buf, int64_t n16, uint32_t key) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * 256;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < n16; i += stride) {
    const u32x4v v = __builtin_nontemporal_load(buf + i);
    __builtin_nontemporal_store(v ^ key, buf + i);
  }
}

}  // namespace

hipError_t launch_stream_inplace(void* buf, int64_t bytes, int n_blocks, hipStream_t stream) {
  hipLaunchKernelGGL(stream_inplace_kernel, dim3(n_blocks), dim3(256), 0, stream, static_cast<u32x4v*>(buf),
                     bytes / 16, 0u);
  return hipGetLastError();
}

double mfma_loop_flops(int n_iter, int n_blocks) {
  return static_cast<double>(n_blocks) * (kLoopThreads / 64) * n_iter * kChains * (2.0 * 16 * 16 * 32);
}

int mfma_loop_waves(int n_blocks) { return n_blocks * (kLoopThreads / 64); }

hipError_t launch_mfma_loop(int n_iter, int n_blocks, float* out, hipStream_t stream) {
  hipLaunchKernelGGL(mfma_loop_kernel, dim3(n_blocks), dim3(kLoopThreads), 0, stream, n_iter, out);
  return hipGetLastError();
}

}  // namespace gdn
