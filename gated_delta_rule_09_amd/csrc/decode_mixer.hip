// decode_mixer.hip -- one decode step of the whole token mixer in one kernel:
// the causal conv (kernel 4) + SiLU of the new token's q|k|v channels with the
// conv state shifted in place, the L2 norm of q and k, the rule with the fp32
// state updated in place, and the gated RMSNorm of o (the "Delta-rule layers"
// row of the model card's Architecture table: conv in front, gated RMS-norm
// after, fp32 recurrent state).
//
// Per (sequence n, key head kh) with its value heads h = kh * G + j:
//   y_c    = silu(sum_i w[c][i] x_{t-3+i}[c] + bias[c]) over the key head's q
//            and k channels and the value heads' v channels (history from the
//            conv state, oldest first; the state becomes (x_{t-2}, x_{t-1}, x_t))
//   q, k   = y / sqrt(sum y^2 + l2_eps) per 128-channel head; q, k, v rounded
//            to bf16, as the separate conv call stores them
//   S_h   <- a S_h + b (v_h - a S_h k) k^T,  o_h = scale * S_h q   (a = exp(g))
//   out_h  = o_h / sqrt(mean(o_h^2) + norm_eps) * w * z_h * sigmoid(z_h)
// with g, b given per (n, h), or formed from the projections a, b as the
// prefill's gate preparation does: g = -exp(A_log) softplus(a + dt_bias),
// b = sigmoid(b_proj) (the kGated instances).
//
// Mapping: one 1024-thread work-group per (n, kh), so the conv channels and
// the states it updates belong to it alone and the in-place updates race with
// nothing.  The conv inputs are loaded first, then the first head's state
// rows, so the state traffic overlaps the conv and L2 phases and the conv does
// not wait behind it (loads return in order).  Sixteen lanes per state row,
// two rows per thread and head; the heads go one after another, the next
// head's rows loaded as soon as the current head's are updated.  That keeps
// the kernel under 64 VGPRs, so two work-groups (32 waves) share a CU and one
// streams its state while the other runs its conv and norm phases; holding
// all G heads at once, or eight lanes per row, needs more registers, one
// work-group per CU, and measured 4-7 % slower.  Both dot products of a row
// use the old row, as in the one-token decode kernel.  Wave j computes head
// j's norm.
#include "common.h"
#include "launch.h"

namespace gdn {

namespace {

constexpr int kD = 128;
constexpr int kThreads = 1024;
constexpr int kLpr = 16;                      // lanes per state row
constexpr int kCpl = kD / (4 * kLpr);         // float4 chunks per lane and row
constexpr int kRowStep = kThreads / kLpr;     // rows between a thread's rows
constexpr int kRows = kD / kRowStep;          // rows per thread and head

struct MixerParams {
  const uint16_t* x; int64_t xs;
  const uint16_t* conv_w; const float* conv_bias;
  uint16_t* conv_state;
  const float* g; const float* beta;
  // gates from the per-head projections instead (ga != nullptr):
  // g = -exp(A_log) softplus(a + dt_bias), beta = sigmoid(b)
  const uint16_t* ga; const uint16_t* gb; int64_t gas, gbs;
  const float* A_log; const float* dt_bias;
  const uint16_t* z; int64_t zs;
  const float* norm_w;
  float* state; const int32_t* slots; int n_slots;
  void* out; int out_bf16;
  int Hk, Hv;
  float scale, l2_eps, norm_eps;
};

__device__ __forceinline__ float silu(float x) { return x * __builtin_amdgcn_rcpf(1.f + __expf(-x)); }

__device__ __forceinline__ float round_bf16(float x) {
  return bf16_to_f32(f32_to_bf16(x));
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) x += __shfl_xor(x, d, 64);
  return x;
}

// Channel of local conv channel c of key head kh: q's 128, k's 128, then the
// G value heads' channels.
__device__ __forceinline__ int channel(int c, int kh, int Hk, int G) {
  return c < kD ? kh * kD + c
       : c < 2 * kD ? Hk * kD + kh * kD + (c - kD)
                    : 2 * Hk * kD + kh * G * kD + (c - 2 * kD);
}

// kGated: the gates come from the projections (p.ga, p.gb, p.A_log, p.dt_bias).
template <int G, bool kGated>
__global__ __launch_bounds__(kThreads) void decode_mixer_kernel(MixerParams p) {
  __shared__ float qk[2][kD];
  __shared__ float vv[G][kD];
  __shared__ float ob[G][kD];

  const int n = blockIdx.x / p.Hk;
  const int kh = blockIdx.x - n * p.Hk;
  const int tid = threadIdx.x;
  const int w = tid >> 6;
  const int lane = tid & 63;
  const int pl = tid & (kLpr - 1);
  const int rg = tid / kLpr;
  const int slot = p.slots ? p.slots[n] : n;
  // a slot outside the pool (say -1 for a padding row) names no state or conv
  // window: the work-group leaves both pools and its output rows untouched
  if (p.slots && static_cast<unsigned>(slot) >= static_cast<unsigned>(p.n_slots)) return;
  const int C = (2 * p.Hk + p.Hv) * kD;

  // ---- the conv inputs of this thread's (at most two) channels -------------
  // Issued before the state rows: loads return in order, so the conv can start
  // while the state is still streaming in.
  constexpr int kCh = (2 + G) * kD;
  constexpr int kPer = (kCh + kThreads - 1) / kThreads;
  float bias[kPer];
  uint16_t wt[kPer][4], hb[kPer][4];           // weights; x_{t-3}, x_{t-2}, x_{t-1}, x_t
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    // straight-line loads (a thread past the last channel reloads it and
    // discards the values), so nothing waits on them before the state loads
    const int c = min(tid + i * kThreads, kCh - 1);
    const int ch = channel(c, kh, p.Hk, G);
    const uint16_t* cs = p.conv_state + (static_cast<int64_t>(slot) * C + ch) * 3;
    const uint16_t* wc = p.conv_w + static_cast<int64_t>(ch) * 4;
    hb[i][0] = cs[0];
    hb[i][1] = cs[1];
    hb[i][2] = cs[2];
    hb[i][3] = p.x[static_cast<int64_t>(n) * p.xs + ch];
    bias[i] = p.conv_bias ? p.conv_bias[ch] : 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) wt[i][e] = wc[e];
  }

  // ---- the first head's state rows ----------------------------------------
  floatx4 s[kRows][kCpl];
  auto load_head = [&](int j, floatx4 (&d)[kRows][kCpl]) {
    const float* S = p.state + (static_cast<int64_t>(slot) * p.Hv + kh * G + j) * (kD * kD);
#pragma unroll
    for (int r = 0; r < kRows; ++r)
#pragma unroll
      for (int c = 0; c < kCpl; ++c)
        d[r][c] = __builtin_nontemporal_load(
            reinterpret_cast<const floatx4*>(S + (rg + kRowStep * r) * kD + 4 * (pl + kLpr * c)));
  };
  load_head(0, s);

  // ---- conv + SiLU of the q, k and v channels, conv state shifted ----------
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int c = tid + i * kThreads;
    if (c < kCh) {
      const int ch = channel(c, kh, p.Hk, G);
      uint16_t* cs = p.conv_state + (static_cast<int64_t>(slot) * C + ch) * 3;
      float acc = bias[i];
#pragma unroll
      for (int e = 0; e < 4; ++e) acc = fmaf(bf16_to_f32(wt[i][e]), bf16_to_f32(hb[i][e]), acc);
      const float y = silu(acc);
      if (c < 2 * kD) qk[c / kD][c % kD] = y;
      else vv[(c - 2 * kD) / kD][(c - 2 * kD) % kD] = round_bf16(y);
      cs[0] = hb[i][1];
      cs[1] = hb[i][2];
      cs[2] = hb[i][3];
    }
  }
  __syncthreads();

  // ---- L2 norm of q (wave 0) and k (wave 1), then rounded to bf16 -----------
  if (w < 2) {
    const float a0 = qk[w][lane], a1 = qk[w][lane + 64];
    const float inv = rsqrtf(wave_sum(a0 * a0 + a1 * a1) + p.l2_eps);
    qk[w][lane] = round_bf16(a0 * inv);
    qk[w][lane + 64] = round_bf16(a1 * inv);
  }
  __syncthreads();

  // ---- the rule, head by head (as decode_step_kernel) ----------------------
  float kk[4 * kCpl], qq[4 * kCpl];
#pragma unroll
  for (int c = 0; c < kCpl; ++c)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      kk[4 * c + i] = qk[1][4 * (pl + kLpr * c) + i];
      qq[4 * c + i] = qk[0][4 * (pl + kLpr * c) + i];
    }
  float kq = 0.f;
#pragma unroll
  for (int j = 0; j < 4 * kCpl; ++j) kq += kk[j] * qq[j];
  kq = sum16(kq);
#pragma unroll
  for (int j = 0; j < G; ++j) {
    const int h = kh * G + j;
    float* S = p.state + (static_cast<int64_t>(slot) * p.Hv + h) * (kD * kD);
    float a, b;
    if (kGated) {
      // softplus(x) = max(x, 0) + log1p(e^-|x|), as the prefill's gate preparation
      const float x = bf16_to_f32(p.ga[static_cast<int64_t>(n) * p.gas + h]) + p.dt_bias[h];
      const float sp = fmaxf(x, 0.f) + log1pf(expf(-fabsf(x)));
      a = expf(-expf(p.A_log[h]) * sp);
      b = 1.f / (1.f + expf(-bf16_to_f32(p.gb[static_cast<int64_t>(n) * p.gbs + h])));
    } else {
      a = expf(p.g[static_cast<int64_t>(n) * p.Hv + h]);
      b = p.beta[static_cast<int64_t>(n) * p.Hv + h];
    }
#pragma unroll
    for (int r = 0; r < kRows; ++r) {
      const int row = rg + kRowStep * r;
      float sk = 0.f, sq = 0.f;
#pragma unroll
      for (int c = 0; c < kCpl; ++c) {
        sk += s[r][c][0] * kk[4 * c] + s[r][c][1] * kk[4 * c + 1] + s[r][c][2] * kk[4 * c + 2] +
              s[r][c][3] * kk[4 * c + 3];
        sq += s[r][c][0] * qq[4 * c] + s[r][c][1] * qq[4 * c + 1] + s[r][c][2] * qq[4 * c + 2] +
              s[r][c][3] * qq[4 * c + 3];
      }
      sk = sum16(sk);
      sq = sum16(sq);
      const float u = b * (vv[j][row] - a * sk);
#pragma unroll
      for (int c = 0; c < kCpl; ++c) {
        floatx4 t;
#pragma unroll
        for (int i = 0; i < 4; ++i) t[i] = a * s[r][c][i] + u * kk[4 * c + i];
        __builtin_nontemporal_store(t, reinterpret_cast<floatx4*>(S + row * kD + 4 * (pl + kLpr * c)));
      }
      if (pl == 0) ob[j][row] = p.scale * (a * sq + u * kq);
    }
    if (j + 1 < G) load_head(j + 1, s);      // the next head's rows stream in
  }
  __syncthreads();

  // ---- gated RMSNorm: wave j, head j, two channels per lane -----------------
  if (w < G) {
    const int h = kh * G + w;
    const float o0 = ob[w][lane], o1 = ob[w][lane + 64];
    const float inv = rsqrtf(wave_sum(o0 * o0 + o1 * o1) * (1.f / kD) + p.norm_eps);
    const uint16_t* zh = p.z + static_cast<int64_t>(n) * p.zs + h * kD;
    const float z0 = bf16_to_f32(zh[lane]), z1 = bf16_to_f32(zh[lane + 64]);
    const float r0 = o0 * inv * p.norm_w[lane] * silu(z0);
    const float r1 = o1 * inv * p.norm_w[lane + 64] * silu(z1);
    const int64_t e = (static_cast<int64_t>(n) * p.Hv + h) * kD;
    if (p.out_bf16) {
      static_cast<uint16_t*>(p.out)[e + lane] = f32_to_bf16(r0);
      static_cast<uint16_t*>(p.out)[e + lane + 64] = f32_to_bf16(r1);
    } else {
      static_cast<float*>(p.out)[e + lane] = r0;
      static_cast<float*>(p.out)[e + lane + 64] = r1;
    }
  }
}

}  // namespace

hipError_t launch_decode_mixer(const uint16_t* x, int64_t xs, const uint16_t* conv_w,
                               const float* conv_bias, uint16_t* conv_state,
                               const GateInputs& gates, const uint16_t* z, int64_t zs,
                               const float* norm_w, float* state, const int32_t* state_slot,
                               int n_slots, void* out, bool out_bf16, int n_seqs, int Hk, int Hv,
                               float scale,
                               float l2_eps, float norm_eps, hipStream_t stream) {
  if (n_seqs == 0) return hipSuccess;
  MixerParams mp;
  mp.x = x; mp.xs = xs; mp.conv_w = conv_w; mp.conv_bias = conv_bias; mp.conv_state = conv_state;
  mp.g = gates.g; mp.beta = gates.beta; mp.ga = gates.a; mp.gb = gates.b;
  mp.gas = gates.a_stride; mp.gbs = gates.b_stride; mp.A_log = gates.A_log; mp.dt_bias = gates.dt_bias;
  mp.z = z; mp.zs = zs; mp.norm_w = norm_w;
  mp.state = state; mp.slots = state_slot; mp.n_slots = n_slots;
  mp.out = out; mp.out_bf16 = out_bf16 ? 1 : 0;
  mp.Hk = Hk; mp.Hv = Hv; mp.scale = scale; mp.l2_eps = l2_eps; mp.norm_eps = norm_eps;
  const dim3 grid(static_cast<unsigned>(n_seqs) * static_cast<unsigned>(Hk));
  const bool gated = gates.a != nullptr;
  switch ((Hv / Hk) * 2 + (gated ? 1 : 0)) {
    case 2: hipLaunchKernelGGL((decode_mixer_kernel<1, false>), grid, dim3(kThreads), 0, stream, mp); break;
    case 3: hipLaunchKernelGGL((decode_mixer_kernel<1, true>), grid, dim3(kThreads), 0, stream, mp); break;
    case 4: hipLaunchKernelGGL((decode_mixer_kernel<2, false>), grid, dim3(kThreads), 0, stream, mp); break;
    case 5: hipLaunchKernelGGL((decode_mixer_kernel<2, true>), grid, dim3(kThreads), 0, stream, mp); break;
    case 6: hipLaunchKernelGGL((decode_mixer_kernel<3, false>), grid, dim3(kThreads), 0, stream, mp); break;
    case 7: hipLaunchKernelGGL((decode_mixer_kernel<3, true>), grid, dim3(kThreads), 0, stream, mp); break;
    case 8: hipLaunchKernelGGL((decode_mixer_kernel<4, false>), grid, dim3(kThreads), 0, stream, mp); break;
    case 9: hipLaunchKernelGGL((decode_mixer_kernel<4, true>), grid, dim3(kThreads), 0, stream, mp); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace gdn
