// rmsnorm.hip -- gated RMSNorm after the rule (the "gated RMS-norm" of the
// "Delta-rule layers" row of the model card's Architecture table):
//     out_i = o_i / sqrt(mean_j o_j^2 + eps) * w_i * z_i * sigmoid(z_i)
// per (row, value head) over the 128 value channels, w shared by all heads.
//
// Mapping: 16 lanes per (row, head); lane p owns channels 4p .. 4p+3 and
// 64 + 4p .. 64 + 4p + 3, so every load and store instruction covers whole
// contiguous runs (256 B of o per head and instruction).  The sum of squares is
// a 16-lane DPP reduction.  One (row, head) per 16 lanes, no loop.
#include "common.h"
#include "launch.h"

namespace gdn {

namespace {

constexpr int kThreads = 256;

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float float2v __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(float2v{a, b}, bf16x2));
}

template <bool kBf16Out>
__global__ __launch_bounds__(kThreads) void gated_rmsnorm_kernel(
    const float* __restrict__ o, const uint16_t* __restrict__ z, int64_t zs,
    const float* __restrict__ w, void* __restrict__ out, int64_t n_heads_total, int Hv,
    float eps) {
  const int p = threadIdx.x & 15;
  const int64_t hr = static_cast<int64_t>(blockIdx.x) * (kThreads / 16) + (threadIdx.x >> 4);
  if (hr >= n_heads_total) return;       // whole 16-lane groups
  const int64_t row = hr / Hv;
  const int hh = static_cast<int>(hr - row * Hv);
  const float* oh = o + hr * 128;
  const uint16_t* zh = z + row * zs + hh * 128;
  float x[8], zf[8], wr[8];
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    const int c = 64 * half + 4 * p;
    const floatx4 a = __builtin_nontemporal_load(reinterpret_cast<const floatx4*>(oh + c));
    const uint2 zb = *reinterpret_cast<const uint2*>(zh + c);
    const float4 wv = *reinterpret_cast<const float4*>(w + c);
    x[4 * half + 0] = a[0]; x[4 * half + 1] = a[1]; x[4 * half + 2] = a[2]; x[4 * half + 3] = a[3];
    zf[4 * half + 0] = __uint_as_float(zb.x << 16);
    zf[4 * half + 1] = __uint_as_float(zb.x & 0xffff0000u);
    zf[4 * half + 2] = __uint_as_float(zb.y << 16);
    zf[4 * half + 3] = __uint_as_float(zb.y & 0xffff0000u);
    wr[4 * half + 0] = wv.x; wr[4 * half + 1] = wv.y; wr[4 * half + 2] = wv.z; wr[4 * half + 3] = wv.w;
  }
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) ss = fmaf(x[i], x[i], ss);
  ss = sum16(ss);
  const float inv = rsqrtf(ss * (1.f / 128.f) + eps);
  float r[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    // SiLU gate with the hardware exp2 and reciprocal (about 1 ulp each)
    const float gate = zf[i] * __builtin_amdgcn_rcpf(1.f + __expf(-zf[i]));
    r[i] = x[i] * inv * wr[i] * gate;
  }
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    const int c = 64 * half + 4 * p;
    if (kBf16Out) {
      const uint2 v = {pack_bf16x2(r[4 * half], r[4 * half + 1]), pack_bf16x2(r[4 * half + 2], r[4 * half + 3])};
      *reinterpret_cast<uint2*>(static_cast<uint16_t*>(out) + hr * 128 + c) = v;
    } else {
      __builtin_nontemporal_store(floatx4{r[4 * half], r[4 * half + 1], r[4 * half + 2], r[4 * half + 3]},
                                  reinterpret_cast<floatx4*>(static_cast<float*>(out) + hr * 128 + c));
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
  const int64_t blocks = (heads + per_block - 1) / per_block;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
  if (out_bf16)
    hipLaunchKernelGGL(gated_rmsnorm_kernel<true>, dim3(static_cast<unsigned>(blocks)),
                       dim3(kThreads), 0, stream, o, z, zs, w, out, heads, Hv, eps);
  else
    hipLaunchKernelGGL(gated_rmsnorm_kernel<false>, dim3(static_cast<unsigned>(blocks)),
                       dim3(kThreads), 0, stream, o, z, zs, w, out, heads, Hv, eps);
  return hipGetLastError();
}

}  // namespace gdn
