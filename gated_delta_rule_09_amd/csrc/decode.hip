// decode.hip -- one-token step of the gated delta rule with the fp32 state
// updated in place.
//
// Per (sequence n, value head h), with a = exp(g), b = beta and S the 128x128
// fp32 state (row i = value channel):
//     S <- a S + b (v - a S k) k^T,      o = scale * S q
// Row i of the new state is a*S_i + u_i k^T with u_i = b (v_i - a S_i.k), and
// o_i = scale * (a S_i.q + u_i (k.q)), so both dot products come from the OLD
// row and the state is read once and written once (the rule of the
// "Delta-rule layers" row of the model card's Architecture table, T = 1).
//
// Mapping: one work-group per (n, h).  Eight consecutive lanes share a state
// row; lane p of the eight holds the float4 columns p, p+8, p+16, p+24 of that
// row, so every wave-wide load reads eight whole 128-byte row pieces.  With
// kTh threads, thread t owns rows t/8 + i * kTh/8.  Row dot products are
// reduced inside the 8-lane group with DPP.
#include "common.h"
#include "launch.h"

namespace gdn {

namespace {

constexpr int kD = 128;

// kTh threads per work-group, eight lanes per state row: a thread's rows are
// kTh / 8 apart and it holds kD / (kTh / 8) of them.
template <int kTh> constexpr int row_step() { return kTh / 8; }
template <int kTh> constexpr int rows_per_thread() { return kD / (kTh / 8); }
// One token: 1024 threads, one row each, 56 VGPRs, so two work-groups (32
// waves) share a CU; at 256 sequences x 48 heads this streams the state 6 %
// faster than 512 threads with two rows each.  Several tokens: the per-token
// q/k registers grow with kT, and 512 threads with two rows each are faster
// from two tokens on (and do not spill up to eight).
constexpr int kStepThreads = 1024;
constexpr int kTokThreads = 512;

template <int kTh, bool kSlots>
__global__ __launch_bounds__(kTh) void decode_step_kernel(
    const uint16_t* __restrict__ q, int64_t q_stride, const uint16_t* __restrict__ k,
    int64_t k_stride, const uint16_t* __restrict__ v, int64_t v_stride,
    const float* __restrict__ g, const float* __restrict__ beta, float* __restrict__ state,
    const int32_t* __restrict__ slots, int n_slots, float* __restrict__ o, int Hk, int Hv,
    float scale) {
  const int n = blockIdx.x / Hv;
  const int h = blockIdx.x - n * Hv;
  const int kh = h / (Hv / Hk);
  constexpr int kRowStep = row_step<kTh>();
  constexpr int kRows = rows_per_thread<kTh>();
  const int tid = threadIdx.x;
  const int p = tid & 7;
  const int rg = tid >> 3;
  const int slot = kSlots ? slots[n] : n;
  // a slot outside the pool (say -1 for a padding row) names no state: the
  // work-group leaves the pool and its output rows untouched
  if (kSlots && static_cast<unsigned>(slot) >= static_cast<unsigned>(n_slots)) return;
  float* S = state + (static_cast<int64_t>(slot) * Hv + h) * (kD * kD);

  // Stream the thread's rows first so all its state bytes are in flight.
  floatx4 s[kRows][4];
#pragma unroll
  for (int r = 0; r < kRows; ++r)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      s[r][j] = __builtin_nontemporal_load(
          reinterpret_cast<const floatx4*>(S + (rg + kRowStep * r) * kD + 4 * (p + 8 * j)));

  const uint16_t* kp = k + n * k_stride + kh * kD;
  const uint16_t* qp = q + n * q_stride + kh * kD;
  float kk[16], qq[16];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint2 kb = *reinterpret_cast<const uint2*>(kp + 4 * (p + 8 * j));
    const uint2 qb = *reinterpret_cast<const uint2*>(qp + 4 * (p + 8 * j));
    kk[4 * j + 0] = __uint_as_float(kb.x << 16);
    kk[4 * j + 1] = __uint_as_float(kb.x & 0xffff0000u);
    kk[4 * j + 2] = __uint_as_float(kb.y << 16);
    kk[4 * j + 3] = __uint_as_float(kb.y & 0xffff0000u);
    qq[4 * j + 0] = __uint_as_float(qb.x << 16);
    qq[4 * j + 1] = __uint_as_float(qb.x & 0xffff0000u);
    qq[4 * j + 2] = __uint_as_float(qb.y << 16);
    qq[4 * j + 3] = __uint_as_float(qb.y & 0xffff0000u);
  }
  float kq = 0.f;
#pragma unroll
  for (int j = 0; j < 16; ++j) kq += kk[j] * qq[j];
  kq = sum8(kq);

  const float a = expf(g[static_cast<int64_t>(n) * Hv + h]);
  const float b = beta[static_cast<int64_t>(n) * Hv + h];
  const uint16_t* vp = v + n * v_stride + h * kD;
  float* op = o + (static_cast<int64_t>(n) * Hv + h) * kD;

#pragma unroll
  for (int r = 0; r < kRows; ++r) {
    const int row = rg + kRowStep * r;
    float sk = 0.f, sq = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      sk += s[r][j][0] * kk[4 * j] + s[r][j][1] * kk[4 * j + 1] + s[r][j][2] * kk[4 * j + 2] +
            s[r][j][3] * kk[4 * j + 3];
      sq += s[r][j][0] * qq[4 * j] + s[r][j][1] * qq[4 * j + 1] + s[r][j][2] * qq[4 * j + 2] +
            s[r][j][3] * qq[4 * j + 3];
    }
    sk = sum8(sk);
    sq = sum8(sq);
    const float vi = bf16_to_f32(vp[row]);
    const float u = b * (vi - a * sk);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      floatx4 t;
#pragma unroll
      for (int i = 0; i < 4; ++i) t[i] = a * s[r][j][i] + u * kk[4 * j + i];
      __builtin_nontemporal_store(t, reinterpret_cast<floatx4*>(S + row * kD + 4 * (p + 8 * j)));
    }
    if (p == 0) op[row] = scale * (a * sq + u * kq);
  }
}

// kT consecutive tokens of each sequence in one pass over the state: the
// thread's rows stay in registers while the tokens are applied in order, each
// with the arithmetic above (both dot products from the row before that
// token), so kT tokens cost one read and one write of the state.  Token t of
// sequence n is row n * kT + t of q, k, v, g, beta and o.
template <int kT, int kTh, bool kSlots>
__global__ __launch_bounds__(kTh) void decode_tokens_kernel(
    const uint16_t* __restrict__ q, int64_t q_stride, const uint16_t* __restrict__ k,
    int64_t k_stride, const uint16_t* __restrict__ v, int64_t v_stride,
    const float* __restrict__ g, const float* __restrict__ beta, float* __restrict__ state,
    const int32_t* __restrict__ slots, int n_slots, float* __restrict__ o, int Hk, int Hv,
    float scale) {
  const int n = blockIdx.x / Hv;
  const int h = blockIdx.x - n * Hv;
  const int kh = h / (Hv / Hk);
  constexpr int kRowStep = row_step<kTh>();
  constexpr int kRows = rows_per_thread<kTh>();
  const int tid = threadIdx.x;
  const int p = tid & 7;
  const int rg = tid >> 3;
  const int slot = kSlots ? slots[n] : n;
  // a slot outside the pool (say -1 for a padding row) names no state: the
  // work-group leaves the pool and its output rows untouched
  if (kSlots && static_cast<unsigned>(slot) >= static_cast<unsigned>(n_slots)) return;
  float* S = state + (static_cast<int64_t>(slot) * Hv + h) * (kD * kD);

  // From two tokens on, every token's k and q rows of this key head are staged
  // in LDS (loaded before the state rows, so the staging waits on them
  // alone) and read back when the token is applied: held in registers
  // instead, they cost 16 VGPRs per token and at four tokens leave one
  // work-group per CU (338 against 257 us at 256 sequences x 4 tokens).
  constexpr bool kStage = kT >= 2;
  __shared__ uint2 kq_lds[kStage ? kT : 1][2][32];
  if (kStage && tid < kT * 64) {
    const int t = tid >> 6, which = (tid >> 5) & 1, idx = tid & 31;
    const int64_t row = static_cast<int64_t>(n) * kT + t;
    const uint16_t* src = which ? q + row * q_stride : k + row * k_stride;
    kq_lds[t][which][idx] = *reinterpret_cast<const uint2*>(src + kh * kD + 4 * idx);
  }
  // and every token's v row of this head (held in registers, the v entries
  // of eight tokens alone kept the kernel above 128 VGPRs: 448 against
  // 343 us at 256 sequences x 8 tokens)
  constexpr bool kStageV = kStage;
  __shared__ uint2 v_lds[kStageV ? kT : 1][32];
  if (kStageV && tid < kT * 32) {
    const int t = tid >> 5, idx = tid & 31;
    const int64_t row = static_cast<int64_t>(n) * kT + t;
    v_lds[t][idx] = *reinterpret_cast<const uint2*>(v + row * v_stride + h * kD + 4 * idx);
  }
  floatx4 s[kRows][4];
#pragma unroll
  for (int r = 0; r < kRows; ++r)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      s[r][j] = __builtin_nontemporal_load(
          reinterpret_cast<const floatx4*>(S + (rg + kRowStep * r) * kD + 4 * (p + 8 * j)));

  // every token's g, beta and the thread's v entries (and, without the LDS
  // staging, k and q: this lane's 16 channels as bf16 pairs), all issued
  // before the arithmetic
  uint2 kb[kStage ? 1 : kT][4], qb[kStage ? 1 : kT][4];
  float gt[kT], bt[kT], vt[kStageV ? 1 : kT][kRows];
#pragma unroll
  for (int t = 0; t < kT; ++t) {
    const int64_t row = static_cast<int64_t>(n) * kT + t;
    if constexpr (!kStage) {
      const uint16_t* kp = k + row * k_stride + kh * kD;
      const uint16_t* qp = q + row * q_stride + kh * kD;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        kb[t][j] = *reinterpret_cast<const uint2*>(kp + 4 * (p + 8 * j));
        qb[t][j] = *reinterpret_cast<const uint2*>(qp + 4 * (p + 8 * j));
      }
    }
    gt[t] = g[row * Hv + h];
    bt[t] = beta[row * Hv + h];
#pragma unroll
    for (int r = 0; r < kRows; ++r)
      if constexpr (!kStageV) vt[t][r] = bf16_to_f32(v[row * v_stride + h * kD + rg + kRowStep * r]);
  }
  if (kStage || kStageV) __syncthreads();

#pragma unroll
  for (int t = 0; t < kT; ++t) {
    float kk[16], qq[16];
    const int tt = kStage ? 0 : t;
    if constexpr (kStage) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        kb[0][j] = kq_lds[t][0][p + 8 * j];
        qb[0][j] = kq_lds[t][1][p + 8 * j];
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      kk[4 * j + 0] = __uint_as_float(kb[tt][j].x << 16);
      kk[4 * j + 1] = __uint_as_float(kb[tt][j].x & 0xffff0000u);
      kk[4 * j + 2] = __uint_as_float(kb[tt][j].y << 16);
      kk[4 * j + 3] = __uint_as_float(kb[tt][j].y & 0xffff0000u);
      qq[4 * j + 0] = __uint_as_float(qb[tt][j].x << 16);
      qq[4 * j + 1] = __uint_as_float(qb[tt][j].x & 0xffff0000u);
      qq[4 * j + 2] = __uint_as_float(qb[tt][j].y << 16);
      qq[4 * j + 3] = __uint_as_float(qb[tt][j].y & 0xffff0000u);
    }
    float kq = 0.f;
#pragma unroll
    for (int j = 0; j < 16; ++j) kq += kk[j] * qq[j];
    kq = sum8(kq);
    const float a = expf(gt[t]);
    const float b = bt[t];
    float* op = o + ((static_cast<int64_t>(n) * kT + t) * Hv + h) * kD;
#pragma unroll
    for (int r = 0; r < kRows; ++r) {
      const int row = rg + kRowStep * r;
      float sk = 0.f, sq = 0.f;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        sk += s[r][j][0] * kk[4 * j] + s[r][j][1] * kk[4 * j + 1] + s[r][j][2] * kk[4 * j + 2] +
              s[r][j][3] * kk[4 * j + 3];
        sq += s[r][j][0] * qq[4 * j] + s[r][j][1] * qq[4 * j + 1] + s[r][j][2] * qq[4 * j + 2] +
              s[r][j][3] * qq[4 * j + 3];
      }
      sk = sum8(sk);
      sq = sum8(sq);
      float vv;
      if constexpr (kStageV) vv = bf16_to_f32(reinterpret_cast<const uint16_t*>(v_lds[t])[row]);
      else vv = vt[t][r];
      const float u = b * (vv - a * sk);
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) s[r][j][i] = a * s[r][j][i] + u * kk[4 * j + i];
      if (p == 0) op[row] = scale * (a * sq + u * kq);
    }
  }
#pragma unroll
  for (int r = 0; r < kRows; ++r)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      __builtin_nontemporal_store(s[r][j], reinterpret_cast<floatx4*>(S + (rg + kRowStep * r) * kD + 4 * (p + 8 * j)));
}

template <int kT>
void launch_tokens(dim3 grid, hipStream_t stream, const uint16_t* q, int64_t q_stride,
                   const uint16_t* k, int64_t k_stride, const uint16_t* v, int64_t v_stride,
                   const float* g, const float* beta, float* state, const int32_t* state_slot,
                   int n_slots, float* o, int Hk, int Hv, float scale) {
  if (state_slot)
    hipLaunchKernelGGL((decode_tokens_kernel<kT, kTokThreads, true>), grid, dim3(kTokThreads), 0, stream, q, q_stride, k,
                       k_stride, v, v_stride, g, beta, state, state_slot, n_slots, o, Hk, Hv, scale);
  else
    hipLaunchKernelGGL((decode_tokens_kernel<kT, kTokThreads, false>), grid, dim3(kTokThreads), 0, stream, q, q_stride, k,
                       k_stride, v, v_stride, g, beta, state, state_slot, n_slots, o, Hk, Hv, scale);
}

}  // namespace

hipError_t launch_decode_tokens(const uint16_t* q, int64_t q_stride, const uint16_t* k,
                                int64_t k_stride, const uint16_t* v, int64_t v_stride,
                                const float* g, const float* beta, float* state,
                                const int32_t* state_slot, int n_slots, float* o, int n_seqs,
                                int n_tokens, int Hk, int Hv, float scale, hipStream_t stream) {
  if (n_seqs == 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>(n_seqs) * static_cast<unsigned>(Hv));
  switch (n_tokens) {
    case 1: launch_tokens<1>(grid, stream, q, q_stride, k, k_stride, v, v_stride, g, beta, state, state_slot, n_slots, o, Hk, Hv, scale); break;
    case 2: launch_tokens<2>(grid, stream, q, q_stride, k, k_stride, v, v_stride, g, beta, state, state_slot, n_slots, o, Hk, Hv, scale); break;
    case 3: launch_tokens<3>(grid, stream, q, q_stride, k, k_stride, v, v_stride, g, beta, state, state_slot, n_slots, o, Hk, Hv, scale); break;
    case 4: launch_tokens<4>(grid, stream, q, q_stride, k, k_stride, v, v_stride, g, beta, state, state_slot, n_slots, o, Hk, Hv, scale); break;
    case 5: launch_tokens<5>(grid, stream, q, q_stride, k, k_stride, v, v_stride, g, beta, state, state_slot, n_slots, o, Hk, Hv, scale); break;
    case 6: launch_tokens<6>(grid, stream, q, q_stride, k, k_stride, v, v_stride, g, beta, state, state_slot, n_slots, o, Hk, Hv, scale); break;
    case 7: launch_tokens<7>(grid, stream, q, q_stride, k, k_stride, v, v_stride, g, beta, state, state_slot, n_slots, o, Hk, Hv, scale); break;
    case 8: launch_tokens<8>(grid, stream, q, q_stride, k, k_stride, v, v_stride, g, beta, state, state_slot, n_slots, o, Hk, Hv, scale); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_decode_step(const uint16_t* q, int64_t q_stride, const uint16_t* k,
                              int64_t k_stride, const uint16_t* v, int64_t v_stride,
                              const float* g, const float* beta, float* state,
                              const int32_t* state_slot, int n_slots, float* o, int n_seqs,
                              int Hk, int Hv, float scale, hipStream_t stream) {
  if (n_seqs == 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>(n_seqs) * static_cast<unsigned>(Hv));
  if (state_slot)
    hipLaunchKernelGGL((decode_step_kernel<kStepThreads, true>), grid, dim3(kStepThreads), 0, stream, q, q_stride, k,
                       k_stride, v, v_stride, g, beta, state, state_slot, n_slots, o, Hk, Hv, scale);
  else
    hipLaunchKernelGGL((decode_step_kernel<kStepThreads, false>), grid, dim3(kStepThreads), 0, stream, q, q_stride, k,
                       k_stride, v, v_stride, g, beta, state, state_slot, n_slots, o, Hk, Hv, scale);
  return hipGetLastError();
}

}  // namespace gdn
