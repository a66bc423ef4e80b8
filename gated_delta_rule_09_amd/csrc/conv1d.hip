// conv1d.hip -- causal depthwise conv (kernel 4) + SiLU + per-head L2 norm of
// the projected q|k|v channels, with the per-sequence conv state.
//
// The "causal conv (kernel 4) in front" of the "Delta-rule layers" row of the
// model card's Architecture table:
//     y[t][c] = silu(sum_{i<4} w[c][i] x[t-3+i][c] + bias[c]),
// history before a sequence start read from that sequence's conv state (oldest
// first) or zero; then y / sqrt(sum y^2 + eps) over each of the first
// n_l2 heads of 128 channels (the q and k heads).  fp32 math, bf16 out.
//
// Mapping: a thread owns 8 adjacent channels (one 16-byte load per token) and a
// run of consecutive tokens (8 for prefill, 1 for a decode batch of one token
// per sequence), loading every input row of the run before any arithmetic and
// keeping the 3-token history in registers, so x is read once (plus a 3-token
// halo per run).  16 lanes cover one 128-channel head, so the L2 sum is a
// 16-lane DPP reduction.  A work-group spans 2048 channels.  Sequence
// boundaries come from cu_seqlens (binary search at the start of the run, then
// a forward walk).  The new conv state is written by a second kernel after all
// reads of the old one are done.
#include "common.h"
#include "launch.h"

namespace gdn {

namespace {

constexpr int kThreads = 256;
constexpr int kChPerThread = 8;
constexpr int kChPerBlock = kThreads * kChPerThread;

// Sequence bounds of sequence n: explicit cu, or equal pieces of length seq_len.
struct Seqs {
  const int32_t* cu;
  int n_seqs;
  int seq_len;
  __device__ int start(int n) const { return cu ? cu[n] : n * seq_len; }
  __device__ int end(int n) const { return cu ? cu[n + 1] : (n + 1) * seq_len; }
  // Sequence that contains token t (t < T_total): largest n with start(n) <= t
  // and end(n) > t.
  __device__ int find(int t) const {
    if (!cu) return t / seq_len;
    int lo = 0, hi = n_seqs - 1;  // answer in [lo, hi]
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (cu[mid] <= t) lo = mid; else hi = mid - 1;
    }
    return lo;
  }
};

// The conv state of sequence n, channels c0 .. c0+7: 24 bf16 (channel-major,
// three taps oldest first) in three 16-byte loads; tap j of channel i goes to
// st[j][i].  Zero without a conv state.
__device__ __forceinline__ void load_state(const uint16_t* conv_state, int n, int C, int c0,
                                           float (&st)[3][8]) {
  if (!conv_state) {
#pragma unroll
    for (int j = 0; j < 3; ++j)
#pragma unroll
      for (int i = 0; i < 8; ++i) st[j][i] = 0.f;
    return;
  }
  const uint4* base = reinterpret_cast<const uint4*>(conv_state + (static_cast<int64_t>(n) * C + c0) * 3);
  float f[24];
  bf16x8_to_f32(base[0], f);
  bf16x8_to_f32(base[1], f + 8);
  bf16x8_to_f32(base[2], f + 16);
#pragma unroll
  for (int j = 0; j < 3; ++j)
#pragma unroll
    for (int i = 0; i < 8; ++i) st[j][i] = f[3 * i + j];
}

// x / (1 + e^-x) with the hardware exp2 and reciprocal (about 1 ulp each;
// the result is rounded to bf16)
__device__ __forceinline__ float silu(float x) {
  return x * __builtin_amdgcn_rcpf(1.f + __expf(-x));
}

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// Eight floats to eight bf16, round to nearest even (v_cvt_pk_bf16_f32).
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float float2v __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint4 pack_bf16x8(const float* f) {
  uint32_t w[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    w[i] = __builtin_bit_cast(uint32_t, __builtin_convertvector(float2v{f[2 * i], f[2 * i + 1]}, bf16x2));
  return uint4{w[0], w[1], w[2], w[3]};
}

// A thread owns 8 adjacent channels and kTile consecutive tokens.  All kTile + 3
// input rows it needs are loaded before any arithmetic, so their latencies
// overlap; the 3-token history moves through registers.
template <int kTile>
__global__ __launch_bounds__(kThreads) void conv1d_kernel(
    const uint16_t* __restrict__ x, int64_t xs, const uint16_t* __restrict__ w,
    const float* __restrict__ bias, uint16_t* __restrict__ y, int64_t ys,
    const uint16_t* __restrict__ conv_state, Seqs seqs, int T_total, int C, int n_l2_ch,
    float l2_eps) {
  // Lanes past C stay to the end (zero inputs, no stores): the L2 sum is a
  // 16-lane DPP reduction.
  const int c0 = (blockIdx.y * kThreads + threadIdx.x) * kChPerThread;
  const bool active = c0 < C;
  const int t0 = blockIdx.x * kTile;
  const int t1 = min(t0 + kTile, T_total);

  // rows t0 - 3 .. t1 - 1 (row j = token t0 - 3 + j); rows outside [0, T) are zero
  uint4 raw[kTile + 3];
#pragma unroll
  for (int j = 0; j < kTile + 3; ++j) {
    const int t = t0 - 3 + j;
    raw[j] = (active && t >= 0 && t < t1) ? *reinterpret_cast<const uint4*>(x + static_cast<int64_t>(t) * xs + c0)
                                          : uint4{0u, 0u, 0u, 0u};
  }

  float wt[8][4], bs[8];
  {
    const uint4* wp = reinterpret_cast<const uint4*>(w + static_cast<int64_t>(c0) * 4);
    float f[32];
#pragma unroll
    for (int q = 0; q < 4; ++q) bf16x8_to_f32(active ? wp[q] : uint4{0u, 0u, 0u, 0u}, f + 8 * q);
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) wt[i][j] = f[i * 4 + j];
#pragma unroll
    for (int i = 0; i < 8; ++i) bs[i] = (bias && active) ? bias[c0 + i] : 0.f;
  }
  const bool l2 = c0 < n_l2_ch;          // uniform over the 16 lanes of a head

  // history h[0] = x[t-3], h[1] = x[t-2], h[2] = x[t-1] of the current token
  float hist[3][8];
  int n = seqs.find(t0);
  int s = seqs.start(n);
  int e = seqs.end(n);
  {
    float st[3][8];
    if (t0 - 3 < s) load_state(active ? conv_state : nullptr, n, C, c0, st);
#pragma unroll
    for (int b = 1; b <= 3; ++b) {
      const int pos = t0 - b;
      if (pos >= s) {
        bf16x8_to_f32(raw[3 - b], hist[3 - b]);
      } else {
        // state tap 3 - (s - pos), chosen by selects so that st stays in registers
        const int tap = 3 - (s - pos);
#pragma unroll
        for (int i = 0; i < 8; ++i) hist[3 - b][i] = tap == 0 ? st[0][i] : (tap == 1 ? st[1][i] : st[2][i]);
      }
    }
  }

#pragma unroll
  for (int j = 0; j < kTile; ++j) {
    const int t = t0 + j;
    if (t >= t1) break;
    if (t >= e) {
      // next non-empty sequence starts exactly at t
      do { ++n; } while (seqs.end(n) <= t);
      s = seqs.start(n);
      e = seqs.end(n);
      load_state(active ? conv_state : nullptr, n, C, c0, hist);
    }
    float cur[8], out[8];
    bf16x8_to_f32(raw[j + 3], cur);
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float acc = fmaf(wt[i][0], hist[0][i], bs[i]);
      acc = fmaf(wt[i][1], hist[1][i], acc);
      acc = fmaf(wt[i][2], hist[2][i], acc);
      acc = fmaf(wt[i][3], cur[i], acc);
      out[i] = silu(acc);
      ss = fmaf(out[i], out[i], ss);
    }
    ss = sum16(ss);
    if (l2) {
      const float inv = rsqrtf(ss + l2_eps);
#pragma unroll
      for (int i = 0; i < 8; ++i) out[i] *= inv;
    }
    if (active) {   // y is written once and read by another kernel: streamed (nontemporal)
      const uint4 pk = pack_bf16x8(out);
      __builtin_nontemporal_store(u32x4{pk.x, pk.y, pk.z, pk.w},
                                  reinterpret_cast<u32x4*>(y + static_cast<int64_t>(t) * ys + c0));
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      hist[0][i] = hist[1][i];
      hist[1][i] = hist[2][i];
      hist[2][i] = cur[i];
    }
  }
}

// New conv state: the last 3 inputs of (old state ++ sequence), per sequence
// and 8-channel group.  Runs after conv1d_kernel on the same stream.
__global__ __launch_bounds__(kThreads) void conv_state_kernel(
    const uint16_t* __restrict__ x, int64_t xs, uint16_t* __restrict__ conv_state, Seqs seqs,
    int C, const int32_t* __restrict__ slots, int n_slots) {
  const int groups = C / kChPerThread;
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
  if (idx >= static_cast<int64_t>(seqs.n_seqs) * groups) return;
  const int n = static_cast<int>(idx / groups);
  const int c0 = static_cast<int>(idx - static_cast<int64_t>(n) * groups) * kChPerThread;
  const int s = seqs.start(n);
  const int len = seqs.end(n) - s;
  if (len == 0) return;
  const int64_t row = slots ? slots[n] : n;     // the conv state row of sequence n
  if (slots && static_cast<uint64_t>(row) >= static_cast<uint64_t>(n_slots)) return;   // outside the pool
  uint16_t* st = conv_state + (row * C + c0) * 3;
  uint16_t old[24];
#pragma unroll
  for (int i = 0; i < 3; ++i) {
    const uint4 p = reinterpret_cast<const uint4*>(st)[i];
    old[8 * i + 0] = p.x & 0xffff; old[8 * i + 1] = p.x >> 16;
    old[8 * i + 2] = p.y & 0xffff; old[8 * i + 3] = p.y >> 16;
    old[8 * i + 4] = p.z & 0xffff; old[8 * i + 5] = p.z >> 16;
    old[8 * i + 6] = p.w & 0xffff; old[8 * i + 7] = p.w >> 16;
  }
  uint16_t nw[24];
#pragma unroll
  for (int j = 0; j < 3; ++j) {          // new slot j holds relative position len-3+j
    const int rel = len - 3 + j;
    if (rel >= 0) {
      const uint4 p = *reinterpret_cast<const uint4*>(x + static_cast<int64_t>(s + rel) * xs + c0);
      const uint16_t v8[8] = {static_cast<uint16_t>(p.x & 0xffff), static_cast<uint16_t>(p.x >> 16),
                              static_cast<uint16_t>(p.y & 0xffff), static_cast<uint16_t>(p.y >> 16),
                              static_cast<uint16_t>(p.z & 0xffff), static_cast<uint16_t>(p.z >> 16),
                              static_cast<uint16_t>(p.w & 0xffff), static_cast<uint16_t>(p.w >> 16)};
#pragma unroll
      for (int i = 0; i < 8; ++i) nw[i * 3 + j] = v8[i];
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) nw[i * 3 + j] = old[i * 3 + (3 + rel)];
    }
  }
#pragma unroll
  for (int i = 0; i < 3; ++i) {
    uint4 p;
    p.x = nw[8 * i + 0] | (static_cast<uint32_t>(nw[8 * i + 1]) << 16);
    p.y = nw[8 * i + 2] | (static_cast<uint32_t>(nw[8 * i + 3]) << 16);
    p.z = nw[8 * i + 4] | (static_cast<uint32_t>(nw[8 * i + 5]) << 16);
    p.w = nw[8 * i + 6] | (static_cast<uint32_t>(nw[8 * i + 7]) << 16);
    reinterpret_cast<uint4*>(st)[i] = p;
  }
}

}  // namespace

hipError_t launch_conv1d(const uint16_t* x, int64_t xs, const uint16_t* w, const float* bias,
                         uint16_t* y, int64_t ys, uint16_t* conv_state, const int32_t* cu,
                         int n_seqs, int T_total, int C, int n_l2_channels, float l2_eps,
                         hipStream_t stream) {
  Seqs seqs{cu, n_seqs, (cu || n_seqs == 0) ? 0 : T_total / n_seqs};
  if (T_total > 0) {
    // one token per sequence (a decode batch): one token per thread
    const bool batch = n_seqs >= T_total;
    const int tile = batch ? 1 : 8;
    const dim3 grid((T_total + tile - 1) / tile, (C + kChPerBlock - 1) / kChPerBlock);
    if (batch)
      hipLaunchKernelGGL(conv1d_kernel<1>, grid, dim3(kThreads), 0, stream, x, xs, w, bias, y, ys,
                         conv_state, seqs, T_total, C, n_l2_channels, l2_eps);
    else
      hipLaunchKernelGGL(conv1d_kernel<8>, grid, dim3(kThreads), 0, stream, x, xs, w, bias, y, ys,
                         conv_state, seqs, T_total, C, n_l2_channels, l2_eps);
    const hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  return launch_conv_state(x, xs, conv_state, cu, n_seqs, T_total, C, stream);
}

hipError_t launch_conv_state(const uint16_t* x, int64_t xs, uint16_t* conv_state,
                             const int32_t* cu, int n_seqs, int T_total, int C,
                             hipStream_t stream, const int32_t* slots, int n_slots) {
  if (!conv_state || n_seqs <= 0) return hipSuccess;
  Seqs seqs{cu, n_seqs, cu ? 0 : T_total / n_seqs};
  const int64_t work = static_cast<int64_t>(n_seqs) * (C / kChPerThread);
  const dim3 grid(static_cast<unsigned>((work + kThreads - 1) / kThreads));
  hipLaunchKernelGGL(conv_state_kernel, grid, dim3(kThreads), 0, stream, x, xs, conv_state, seqs, C,
                     slots, n_slots);
  return hipGetLastError();
}

}  // namespace gdn
