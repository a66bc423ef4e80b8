// rmsnorm.hip -- gated RMSNorm after the rule (the "gated RMS-norm" of the
// "Delta-rule layers" row of the model card's Architecture table):
//     out_i = o_i / sqrt(mean_j o_j^2 + eps) * w_i * z_i * sigmoid(z_i)
// per (row, value head) over the 128 value channels, w shared by all heads.
//
// Mapping: 16 lanes per (row, head); a lane owns 8 channels (two float4 of o,
// one 16-byte load of z).  The sum of squares is a 16-lane DPP reduction.
// Grid-stride over (row, head) pairs; the stride is a multiple of 16 lanes, so
// a head's lanes always take the same branch.
#include "common.h"
#include "launch.h"

namespace gdn {

namespace {

constexpr int kThreads = 256;

template <bool kBf16Out>
__global__ __launch_bounds__(kThreads) void gated_rmsnorm_kernel(
    const float* __restrict__ o, const uint16_t* __restrict__ z, int64_t zs,
    const float* __restrict__ w, void* __restrict__ out, int64_t n_heads_total, int Hv,
    float eps) {
  const int p = threadIdx.x & 15;
  float wr[8];
  {
    const float4 a = reinterpret_cast<const float4*>(w)[2 * p];
    const float4 b = reinterpret_cast<const float4*>(w)[2 * p + 1];
    wr[0] = a.x; wr[1] = a.y; wr[2] = a.z; wr[3] = a.w;
    wr[4] = b.x; wr[5] = b.y; wr[6] = b.z; wr[7] = b.w;
  }
  const int64_t stride = static_cast<int64_t>(gridDim.x) * (kThreads / 16);
  for (int64_t hr = static_cast<int64_t>(blockIdx.x) * (kThreads / 16) + (threadIdx.x >> 4);
       hr < n_heads_total; hr += stride) {
    const int64_t row = hr / Hv;
    const int hh = static_cast<int>(hr - row * Hv);
    const float4* op = reinterpret_cast<const float4*>(o + hr * 128 + 8 * p);
    const float4 a = op[0], b = op[1];
    float x[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
    float zf[8];
    bf16x8_to_f32(*reinterpret_cast<const uint4*>(z + row * zs + hh * 128 + 8 * p), zf);
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) ss = fmaf(x[i], x[i], ss);
    ss = sum16(ss);
    const float inv = 1.f / sqrtf(ss * (1.f / 128.f) + eps);
    float r[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float gate = zf[i] / (1.f + expf(-zf[i]));
      r[i] = x[i] * inv * wr[i] * gate;
    }
    if (kBf16Out) {
      *reinterpret_cast<uint4*>(static_cast<uint16_t*>(out) + hr * 128 + 8 * p) = f32_to_bf16x8(r);
    } else {
      float4* dst = reinterpret_cast<float4*>(static_cast<float*>(out) + hr * 128 + 8 * p);
      dst[0] = make_float4(r[0], r[1], r[2], r[3]);
      dst[1] = make_float4(r[4], r[5], r[6], r[7]);
    }
  }
}

}  // namespace

hipError_t launch_gated_rmsnorm(const float* o, const uint16_t* z, int64_t zs, const float* w,
                                void* out, bool out_bf16, int64_t rows, int Hv, float eps,
                                hipStream_t stream) {
  const int64_t heads = rows * Hv;
  if (heads == 0) return hipSuccess;
  const int64_t per_block = kThreads / 16;
  int64_t blocks = (heads + per_block - 1) / per_block;
  if (blocks > 256 * 64) blocks = 256 * 64;  // grid-stride beyond ~16K blocks
  if (out_bf16)
    hipLaunchKernelGGL(gated_rmsnorm_kernel<true>, dim3(static_cast<unsigned>(blocks)),
                       dim3(kThreads), 0, stream, o, z, zs, w, out, heads, Hv, eps);
  else
    hipLaunchKernelGGL(gated_rmsnorm_kernel<false>, dim3(static_cast<unsigned>(blocks)),
                       dim3(kThreads), 0, stream, o, z, zs, w, out, heads, Hv, eps);
  return hipGetLastError();
}

}  // namespace gdn
