// backward.hip -- backward of the gated delta rule: the derivatives of
//     L = sum(dO * O) + sum(dS_T * S_T)
// with respect to q, k, v, g, beta and the initial state, for the rule of the
// "Delta-rule layers" row of the model card's Architecture table,
//     S <- a S + b (v - a S k) k^T,   o = scale S q,   a = exp(g).
//
// A plain per-token design, separate from the inference kernels:
// backward_fwd_kernel runs the recurrence and records the state before every
// token (T x Hv x 64 KB of workspace); backward_rev_kernel walks the tokens
// in reverse with D = dL/dS in registers and takes the chain rule through one
// token's operations (S_prev read back from the record):
//     p = a S_prev k,  u = b (v - p),  S = a S_prev + u k^T
//     D  += scale do q^T                dq_h += scale S^T do
//     du  = D k                         dk_h += D^T u
//     dv  = b du                        dbeta = (v - p) . du
//     dSh = D - b du k^T                dk_h += a S_prev^T (-b du)
//     dg  = a <S_prev, dSh>             D    = a dSh
// and backward_sum_kernel adds the value heads' dq_h, dk_h into their key
// head's dq, dk.  Both per-token kernels use one 1024-thread work-group per
// (sequence, value head) with the decode step's layout: eight lanes per
// state row, lane p holding the float4 columns p, p+8, p+16, p+24.  The
// column sums over the 128 rows (dq_h, dk_h) go through lane shuffles inside
// each wave, then LDS across the 16 waves.
#include "common.h"
#include "launch.h"

namespace gdn {

namespace {

constexpr int kD = 128;
constexpr int kTh = 1024;
constexpr int kWaves = kTh / 64;

struct BwdParams {
  const uint16_t* q; const uint16_t* k; const uint16_t* v;
  int64_t qs, ks, vs;
  const float* g; const float* beta;
  const float* h0;            // initial states or nullptr (zeros)
  const float* d_o;           // [T, Hv, 128]
  const float* dhT;           // gradient of the final states or nullptr
  const int32_t* cu;          // nullptr: equal lengths seq_len
  float* dump;                // [T, Hv, 128, 128]: the state before each token
  float* dq_part; float* dk_part;   // [T, Hv, 128] per value head
  float* dv; float* dg; float* dbeta; float* dh0;
  int n_seqs, seq_len, Hk, Hv;
  float scale;
};

__device__ __forceinline__ void seq_range(const BwdParams& p, int n, int& s0, int& s1) {
  if (p.cu) { s0 = p.cu[n]; s1 = p.cu[n + 1]; }
  else { s0 = n * p.seq_len; s1 = s0 + p.seq_len; }
}

// a if the lane's mask m is all ones, b if it is zero; a bitwise blend of two
// loaded values, so that the compiler cannot turn a choice between two
// register arrays into an indexed (scratch) access
__device__ __forceinline__ float blend(unsigned m, float a, float b) {
  return __uint_as_float((__float_as_uint(a) & m) | (__float_as_uint(b) & ~m));
}

__global__ __launch_bounds__(kTh) void backward_fwd_kernel(BwdParams p) {
  const int n = blockIdx.x / p.Hv;
  const int h = blockIdx.x - n * p.Hv;
  const int kh = h / (p.Hv / p.Hk);
  const int tid = threadIdx.x;
  const int lp = tid & 7;
  const int row = tid >> 3;
  int s0, s1;
  seq_range(p, n, s0, s1);
  float s[16];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    floatx4 x = {0.f, 0.f, 0.f, 0.f};
    if (p.h0) x = *reinterpret_cast<const floatx4*>(p.h0 + ((static_cast<int64_t>(n) * p.Hv + h) * kD + row) * kD + 4 * (lp + 8 * j));
#pragma unroll
    for (int i = 0; i < 4; ++i) s[4 * j + i] = x[i];
  }
  // the next token's k row share, gates and v element are in flight while
  // the current token is applied
  uint2 kn[4] = {};
  float gn = 0.f, bn = 0.f;
  uint16_t vn = 0;
  auto fetch = [&](int t) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
      kn[j] = *reinterpret_cast<const uint2*>(p.k + static_cast<int64_t>(t) * p.ks + kh * kD + 4 * (lp + 8 * j));
    gn = p.g[static_cast<int64_t>(t) * p.Hv + h];
    bn = p.beta[static_cast<int64_t>(t) * p.Hv + h];
    vn = p.v[static_cast<int64_t>(t) * p.vs + h * kD + row];
  };
  if (s1 > s0) fetch(s0);
  for (int t = s0; t < s1; ++t) {
    float* dst = p.dump + ((static_cast<int64_t>(t) * p.Hv + h) * kD + row) * kD;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      __builtin_nontemporal_store(floatx4{s[4 * j], s[4 * j + 1], s[4 * j + 2], s[4 * j + 3]},
                                  reinterpret_cast<floatx4*>(dst + 4 * (lp + 8 * j)));
    float kk[16];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      kk[4 * j + 0] = __uint_as_float(kn[j].x << 16);
      kk[4 * j + 1] = __uint_as_float(kn[j].x & 0xffff0000u);
      kk[4 * j + 2] = __uint_as_float(kn[j].y << 16);
      kk[4 * j + 3] = __uint_as_float(kn[j].y & 0xffff0000u);
    }
    const float a = expf(gn);
    const float b = bn;
    const float vv = bf16_to_f32(vn);
    if (t + 1 < s1) fetch(t + 1);
    float sk = 0.f;
#pragma unroll
    for (int e = 0; e < 16; ++e) sk = fmaf(s[e], kk[e], sk);
    sk = sum8(sk);
    const float u = b * (vv - a * sk);
#pragma unroll
    for (int e = 0; e < 16; ++e) s[e] = fmaf(a, s[e], u * kk[e]);
  }
}

// What one lane of the reverse walk reads for one token; the next token's
// copy is in flight while the current one is processed.  k and q, shared by
// all rows, travel through a double-buffered LDS stage instead.
struct RevToken {
  floatx4 s[4];     // this lane's 16 columns of the recorded state row
  float g, beta, dout;
  uint16_t v;
};

__device__ __forceinline__ void rev_load(const BwdParams& p, int t, int h, int kh, int row, int lp,
                                         RevToken& x) {
  const int64_t th = static_cast<int64_t>(t) * p.Hv + h;
  const float* src = p.dump + (th * kD + row) * kD;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    x.s[j] = __builtin_nontemporal_load(reinterpret_cast<const floatx4*>(src + 4 * (lp + 8 * j)));
  }
  x.g = p.g[th];
  x.beta = p.beta[th];
  x.dout = p.d_o[th * kD + row];
  x.v = p.v[static_cast<int64_t>(t) * p.vs + h * kD + row];
}

// wave 0's share of a token's k (lanes 0..31) and q (lanes 32..63): 4 bf16
__device__ __forceinline__ uint2 kq_load(const BwdParams& p, int t, int kh, int lane) {
  const uint16_t* base = lane < 32 ? p.k + static_cast<int64_t>(t) * p.ks
                                   : p.q + static_cast<int64_t>(t) * p.qs;
  return *reinterpret_cast<const uint2*>(base + kh * kD + 4 * (lane & 31));
}

__device__ __forceinline__ void kq_store(float (*buf)[kD], int lane, uint2 b) {
  *reinterpret_cast<floatx4*>(&buf[lane >> 5][4 * (lane & 31)]) =
      floatx4{__uint_as_float(b.x << 16), __uint_as_float(b.x & 0xffff0000u),
              __uint_as_float(b.y << 16), __uint_as_float(b.y & 0xffff0000u)};
}

__global__ __launch_bounds__(kTh) void backward_rev_kernel(BwdParams p) {
  // All three are double-buffered by token parity, so one barrier per token
  // suffices: a buffer written by token t (before its barrier) is next written
  // by token t - 2, after every thread has passed token t - 1's barrier, which
  // each reader of token t's copy reaches only after its reads.
  __shared__ __align__(16) float part[2][kWaves][2][kD];   // per-wave column sums: dq_h, dk_h
  __shared__ float spart[2][kWaves][2];      // per-wave sums: <S_prev, dSh>, dbeta
  __shared__ __align__(16) float kq[2][2][kD];             // k, q of a token
  const int n = blockIdx.x / p.Hv;
  const int h = blockIdx.x - n * p.Hv;
  const int kh = h / (p.Hv / p.Hk);
  const int tid = threadIdx.x;
  const int lp = tid & 7;
  const int row = tid >> 3;
  const int w = tid >> 6;
  const int lane = tid & 63;
  int s0, s1;
  seq_range(p, n, s0, s1);
  float D[16];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    floatx4 x = {0.f, 0.f, 0.f, 0.f};
    if (p.dhT) x = *reinterpret_cast<const floatx4*>(p.dhT + ((static_cast<int64_t>(n) * p.Hv + h) * kD + row) * kD + 4 * (lp + 8 * j));
#pragma unroll
    for (int i = 0; i < 4; ++i) D[4 * j + i] = x[i];
  }
  RevToken nxt;
  if (s1 > s0) {
    rev_load(p, s1 - 1, h, kh, row, lp, nxt);
    if (w == 0) kq_store(kq[(s1 - 1) & 1], lane, kq_load(p, s1 - 1, kh, lane));
  }
  __syncthreads();
  for (int t = s1 - 1; t >= s0; --t) {
    const int64_t th = static_cast<int64_t>(t) * p.Hv + h;
    const RevToken cur = nxt;
    uint2 kq_next = {0u, 0u};
    if (t > s0) {   // the next token's inputs are in flight during this one
      rev_load(p, t - 1, h, kh, row, lp, nxt);
      if (w == 0) kq_next = kq_load(p, t - 1, kh, lane);
    }
    float Sp[16], kk[16], qq[16];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const floatx4 kx = *reinterpret_cast<const floatx4*>(&kq[t & 1][0][4 * (lp + 8 * j)]);
      const floatx4 qx = *reinterpret_cast<const floatx4*>(&kq[t & 1][1][4 * (lp + 8 * j)]);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        Sp[4 * j + i] = cur.s[j][i];
        kk[4 * j + i] = kx[i];
        qq[4 * j + i] = qx[i];
      }
    }
    const float a = expf(cur.g);
    const float b = cur.beta;
    const float vv = bf16_to_f32(cur.v);
    const float dout = cur.dout;
    // the forward step, recomputed
    float sk = 0.f;
#pragma unroll
    for (int e = 0; e < 16; ++e) sk = fmaf(Sp[e], kk[e], sk);
    sk = sum8(sk);
    const float pk = a * sk;
    const float u = b * (vv - pk);
    // o = scale S q
    float cq[16], ck[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      D[e] = fmaf(p.scale * dout, qq[e], D[e]);
      cq[e] = p.scale * dout * fmaf(a, Sp[e], u * kk[e]);
    }
    // S = Sh + u k^T
    float du = 0.f;
#pragma unroll
    for (int e = 0; e < 16; ++e) du = fmaf(D[e], kk[e], du);
    du = sum8(du);
    const float dp = -b * du;
    float gdot = 0.f;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      ck[e] = fmaf(D[e], u, a * Sp[e] * dp);
      const float dsh = fmaf(dp, kk[e], D[e]);
      gdot = fmaf(Sp[e], dsh, gdot);
      D[e] = a * dsh;
    }
    if (lp == 0) p.dv[th * kD + row] = b * du;
    float bdot = lp == 0 ? (vv - pk) * du : 0.f;
    // Column sums over the wave's eight rows (lanes lp, lp + 8, ..., lp + 56)
    // by a butterfly reduce-scatter over lane bits 5, 4, 3: each exchange
    // sends half of the remaining values to the partner lane and keeps the
    // other half, so lane (b5 b4 b3, lp) ends with the four sums of values
    // j = 16 b5 + 8 b4 + 4 b3 + i (j < 16: cq[j], else ck[j - 16]), i.e. the
    // float4 of columns 4 (lp + 8 (2 b4 + b3)) .. + 3 of dq_h (b5 = 0) or
    // dk_h (b5 = 1).  16 + 8 permutes and a DPP step instead of 96 permutes.
    const unsigned m5 = (lane & 32) ? ~0u : 0u, m4 = (lane & 16) ? ~0u : 0u, m3 = (lane & 8) ? ~0u : 0u;
    float y[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) y[i] = __shfl_xor(blend(m5, cq[i], ck[i]), 32, 64);
#pragma unroll
    for (int i = 0; i < 16; ++i) y[i] += blend(m5, ck[i], cq[i]);
    float z[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) z[i] = __shfl_xor(blend(m4, y[i], y[8 + i]), 16, 64);
#pragma unroll
    for (int i = 0; i < 8; ++i) z[i] += blend(m4, y[8 + i], y[i]);
    floatx4 r;
#pragma unroll
    for (int i = 0; i < 4; ++i)   // DPP row_ror:8 reads lane ^ 8 inside each row of 16
      r[i] = blend(m3, z[4 + i], z[i]) + dpp<0x128>(blend(m3, z[i], z[4 + i]));
    *reinterpret_cast<floatx4*>(&part[t & 1][w][(lane >> 5) & 1][4 * (lp + 8 * ((lane >> 3) & 3))]) = r;
    // <S_prev, dSh> and dbeta over the wave: the eight lanes of a row by DPP,
    // then the eight rows
    gdot = sum8(gdot);
    bdot = sum8(bdot);
    gdot += dpp<0x128>(gdot);
    bdot += dpp<0x128>(bdot);
    gdot += __shfl_xor(gdot, 16, 64);
    bdot += __shfl_xor(bdot, 16, 64);
    gdot += __shfl_xor(gdot, 32, 64);
    bdot += __shfl_xor(bdot, 32, 64);
    if (lane == 0) {
      spart[t & 1][w][0] = gdot;
      spart[t & 1][w][1] = bdot;
    }
    // buffer (t - 1) & 1 was last read by token t + 1, before its barrier
    if (w == 0 && t > s0) kq_store(kq[(t - 1) & 1], lane, kq_next);
    __syncthreads();
    if (tid < 2 * kD) {
      const int which = tid >> 7, c = tid & (kD - 1);
      float acc = 0.f;
#pragma unroll
      for (int ww = 0; ww < kWaves; ++ww) acc += part[t & 1][ww][which][c];
      (which ? p.dk_part : p.dq_part)[th * kD + c] = acc;
    } else if (tid == 2 * kD) {
      float gs = 0.f, bs = 0.f;
#pragma unroll
      for (int ww = 0; ww < kWaves; ++ww) {
        gs += spart[t & 1][ww][0];
        bs += spart[t & 1][ww][1];
      }
      p.dg[th] = a * gs;
      p.dbeta[th] = bs;
    }
  }
  if (p.dh0) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
      *reinterpret_cast<floatx4*>(p.dh0 + ((static_cast<int64_t>(n) * p.Hv + h) * kD + row) * kD + 4 * (lp + 8 * j)) =
          floatx4{D[4 * j], D[4 * j + 1], D[4 * j + 2], D[4 * j + 3]};
  }
}

// dq, dk of key head kh = the sum of its value heads' parts
__global__ __launch_bounds__(256) void backward_sum_kernel(const float* __restrict__ dq_part,
                                                           const float* __restrict__ dk_part,
                                                           float* __restrict__ dq, float* __restrict__ dk,
                                                           int64_t n_elem, int Hk, int Hv) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= n_elem) return;                       // n_elem = T * Hk * 128
  const int c = static_cast<int>(i % kD);
  const int64_t tk = i / kD;
  const int kh = static_cast<int>(tk % Hk);
  const int64_t t = tk / Hk;
  const int G = Hv / Hk;
  float aq = 0.f, ak = 0.f;
  for (int j = 0; j < G; ++j) {
    const int64_t src = (t * Hv + kh * G + j) * kD + c;
    aq += dq_part[src];
    ak += dk_part[src];
  }
  dq[i] = aq;
  dk[i] = ak;
}

}  // namespace

size_t backward_workspace_bytes(int T_total, int Hv) {
  const size_t dump = static_cast<size_t>(T_total) * Hv * kD * kD * sizeof(float);
  const size_t parts = 2 * static_cast<size_t>(T_total) * Hv * kD * sizeof(float);
  return dump + parts;
}

hipError_t launch_backward(const uint16_t* q, int64_t qs, const uint16_t* k, int64_t ks,
                           const uint16_t* v, int64_t vs, const float* g, const float* beta,
                           const float* h0, const float* d_o, const float* dhT, const int32_t* cu,
                           int n_seqs, int T_total, int Hk, int Hv, float scale, float* dq,
                           float* dk, float* dv, float* dg, float* dbeta, float* dh0,
                           void* workspace, hipStream_t stream) {
  if (n_seqs == 0) return hipSuccess;
  BwdParams p;
  p.q = q; p.k = k; p.v = v; p.qs = qs; p.ks = ks; p.vs = vs; p.g = g; p.beta = beta;
  p.h0 = h0; p.d_o = d_o; p.dhT = dhT; p.cu = cu;
  float* ws = static_cast<float*>(workspace);
  p.dump = ws;
  p.dq_part = ws + static_cast<size_t>(T_total) * Hv * kD * kD;
  p.dk_part = p.dq_part + static_cast<size_t>(T_total) * Hv * kD;
  p.dv = dv; p.dg = dg; p.dbeta = dbeta; p.dh0 = dh0;
  p.n_seqs = n_seqs; p.seq_len = cu ? 0 : T_total / n_seqs; p.Hk = Hk; p.Hv = Hv; p.scale = scale;
  const dim3 grid(static_cast<unsigned>(n_seqs) * static_cast<unsigned>(Hv));
  hipLaunchKernelGGL(backward_fwd_kernel, grid, dim3(kTh), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(backward_rev_kernel, grid, dim3(kTh), 0, stream, p);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t n_elem = static_cast<int64_t>(T_total) * Hk * kD;
  if (n_elem > 0) {
    hipLaunchKernelGGL(backward_sum_kernel, dim3(static_cast<unsigned>((n_elem + 255) / 256)), dim3(256), 0,
                       stream, p.dq_part, p.dk_part, dq, dk, n_elem, Hk, Hv);
    e = hipGetLastError();
  }
  return e;
}

}  // namespace gdn
