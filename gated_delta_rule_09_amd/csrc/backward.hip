// backward.hip -- backward of the gated delta rule: the derivatives of
//     L = sum(dO * O) + sum(dS_T * S_T)
// with respect to q, k, v, g, beta and the initial state, for the rule of the
// "Delta-rule layers" row of the model card's Architecture table,
//     S <- a S + b (v - a S k) k^T,   o = scale S q,   a = exp(g).
//
// A per-token design with checkpoints, separate from the inference kernels.
// backward_fwd_kernel runs the recurrence and records the state before every
// kSeg-th token of each sequence (the segment starts).  backward_rev_kernel
// walks the segments of a sequence in reverse with D = dL/dS in registers: it
// stages a segment's k, q, v, dO and gates in LDS, and for each of its tokens,
// last first, rebuilds the state before that token from the segment's
// checkpoint (up to kSeg - 1 forward steps, cheap next to a 64 KB record read)
// and takes the chain rule through the token's operations:
//     p = a S_prev k,  u = b (v - p),  S = a S_prev + u k^T
//     D  += scale do q^T                dq_h += scale S^T do
//     du  = D k                         dk_h += D^T u
//     dv  = b du                        dbeta = (v - p) . du
//     dSh = D - b du k^T                dk_h += a S_prev^T (-b du)
//     dg  = a <S_prev, dSh>             D    = a dSh
// backward_sum_kernel then adds the value heads' dq_h, dk_h into their key
// head's dq, dk.  The state's rows (value channels) evolve independently and
// meet only in dq, dk, dg and dbeta, which are sums over rows: both per-token
// kernels give each work-group one group of kRows rows of one (sequence, value
// head), 128, 64 or 32 rows (1024, 512 or 256 threads; fewer rows when the
// batch has too few (sequence, head) pairs to fill the GPU), in the decode
// step's layout: eight lanes per state row, lane p holding the float4 columns
// p, p+8, p+16, p+24.  Row groups write partial sums, added up at the end.
#include "common.h"
#include "launch.h"

namespace gdn {

namespace {

constexpr int kD = 128;
// Tokens per checkpoint segment: 4 balances the checkpoint traffic against
// the rebuild steps (1.5 per token on average).  Measured at 8 x 1024 tokens:
// 9.3 ms per call with 4, 10.0 ms with 8, 12.9 ms with a checkpoint per token.
constexpr int kSeg = 4;

struct BwdParams {
  const uint16_t* q; const uint16_t* k; const uint16_t* v;
  int64_t qs, ks, vs;
  const float* g; const float* beta;
  const float* h0;            // initial states or nullptr (zeros)
  const float* d_o;           // [T, Hv, 128]
  const float* dhT;           // gradient of the final states or nullptr
  const int32_t* cu;          // nullptr: equal lengths seq_len
  float* ckpt;                // [T / kSeg + n_seqs, Hv, 128, 128]: states at segment starts
  float* dq_part; float* dk_part;   // [T, Hv, R, 128] per (value head, row group)
  float* dg_part; float* dbeta_part; // [T, Hv, R]
  float* dv; float* dh0;
  int n_seqs, seq_len, Hk, Hv;
  int R;                      // row groups per (sequence, value head)
  float scale;
};

__device__ __forceinline__ void seq_range(const BwdParams& p, int n, int& s0, int& s1) {
  if (p.cu) { s0 = p.cu[n]; s1 = p.cu[n + 1]; }
  else { s0 = n * p.seq_len; s1 = s0 + p.seq_len; }
}

// Record slot of the checkpoint at token t (a segment start) of sequence n:
// t / kSeg + n grows by one per segment inside a sequence and jumps by at
// least one between sequences, so slots are distinct and below T / kSeg + N.
__device__ __forceinline__ int64_t ckpt_row(const BwdParams& p, int t, int n, int h, int row) {
  return ((static_cast<int64_t>(t / kSeg + n) * p.Hv + h) * kD + row) * kD;
}

// a where the lane's bit of the wave-wide mask m is set, else b: one
// v_cndmask_b32.  Written as asm so that the compiler cannot turn a choice
// between two register arrays into an indexed (scratch) access.
__device__ __forceinline__ float lane_select(uint64_t m, float a, float b) {
  float r;
  asm("v_cndmask_b32_e64 %0, %1, %2, %3" : "=v"(r) : "v"(b), "v"(a), "s"(m));
  return r;
}
// lanes whose index has bit 5, 4 or 3 set
constexpr uint64_t kLaneBit5 = 0xFFFFFFFF00000000ull;
constexpr uint64_t kLaneBit4 = 0xFFFF0000FFFF0000ull;
constexpr uint64_t kLaneBit3 = 0xFF00FF00FF00FF00ull;

// The record kernel's inputs for kFwdTok tokens, staged in LDS by the whole
// work-group, double-buffered.
constexpr int kFwdTok = 8;
template <int kRows>
struct FwdStage {
  float k[kFwdTok][kD], v[kFwdTok][kRows];
  float a[kFwdTok], beta[kFwdTok];
};

// (sequence, value head, row group) of a block of either per-token kernel
struct RowGroup {
  int n, h, kh, rg;
};
__device__ __forceinline__ RowGroup row_group(const BwdParams& p) {
  RowGroup r;
  const int unit = blockIdx.x / p.R;
  r.rg = blockIdx.x - unit * p.R;
  r.n = unit / p.Hv;
  r.h = unit - r.n * p.Hv;
  r.kh = r.h / (p.Hv / p.Hk);
  return r;
}

template <int kRows>
__global__ __launch_bounds__(8 * kRows) void backward_fwd_kernel(BwdParams p) {
  constexpr int kThr = 8 * kRows;
  constexpr int kK = kFwdTok * kD / kThr;   // k elements staged per thread
  static_assert(kK * kThr == kFwdTok * kD && kFwdTok * kRows == kThr, "staging layout");
  __shared__ __align__(16) FwdStage<kRows> stage[2];
  const RowGroup G = row_group(p);
  const int n = G.n, h = G.h, kh = G.kh;
  const int tid = threadIdx.x;
  const int lp = tid & 7;
  const int lrow = tid >> 3;
  const int row = G.rg * kRows + lrow;
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
  // k element m of thread tid: e = tid + m kThr, token e / 128, channel e % 128;
  // v element: token tid / kRows, row tid % kRows of the group; gates: tid < 8
  uint16_t lk[kK] = {}, lv = 0;
  float lg = 0.f, lb = 0.f;
  auto fetch = [&](int b0) {
#pragma unroll
    for (int m = 0; m < kK; ++m) {
      const int e = tid + m * kThr;
      const int64_t t = b0 + (e >> 7);
      if (t < s1) lk[m] = p.k[t * p.ks + kh * kD + (e & (kD - 1))];
    }
    const int64_t tv = b0 + tid / kRows;
    if (tv < s1) lv = p.v[tv * p.vs + h * kD + G.rg * kRows + tid % kRows];
    if (tid < kFwdTok && b0 + tid < s1) {
      lg = p.g[static_cast<int64_t>(b0 + tid) * p.Hv + h];
      lb = p.beta[static_cast<int64_t>(b0 + tid) * p.Hv + h];
    }
  };
  auto put = [&](FwdStage<kRows>& st) {
#pragma unroll
    for (int m = 0; m < kK; ++m) {
      const int e = tid + m * kThr;
      st.k[e >> 7][e & (kD - 1)] = bf16_to_f32(lk[m]);
    }
    st.v[tid / kRows][tid % kRows] = bf16_to_f32(lv);
    if (tid < kFwdTok) {
      st.a[tid] = expf(lg);
      st.beta[tid] = lb;
    }
  };
  if (s1 > s0) {
    fetch(s0);
    put(stage[0]);
  }
  __syncthreads();
  int buf = 0;
  for (int b0 = s0; b0 < s1; b0 += kFwdTok, buf ^= 1) {
    const FwdStage<kRows>& st = stage[buf];
    const bool more = b0 + kFwdTok < s1;
    if (more) fetch(b0 + kFwdTok);   // in flight during this batch
    const int nb = min(kFwdTok, s1 - b0);
    for (int i = 0; i < nb; ++i) {
      const int t = b0 + i;
      if ((t - s0) % kSeg == 0) {
        float* dst = p.ckpt + ckpt_row(p, t, n, h, row);
#pragma unroll
        for (int j = 0; j < 4; ++j)
          __builtin_nontemporal_store(floatx4{s[4 * j], s[4 * j + 1], s[4 * j + 2], s[4 * j + 3]},
                                      reinterpret_cast<floatx4*>(dst + 4 * (lp + 8 * j)));
      }
      float kk[16];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const floatx4 kx = *reinterpret_cast<const floatx4*>(&st.k[i][4 * (lp + 8 * j)]);
#pragma unroll
        for (int e = 0; e < 4; ++e) kk[4 * j + e] = kx[e];
      }
      const float a = st.a[i];
      float sk = 0.f;
#pragma unroll
      for (int e = 0; e < 16; ++e) sk = fmaf(s[e], kk[e], sk);
      sk = sum8(sk);
      const float u = st.beta[i] * (st.v[i][lrow] - a * sk);
#pragma unroll
      for (int e = 0; e < 16; ++e) s[e] = fmaf(a, s[e], u * kk[e]);
    }
    // the other buffer was last read in the previous batch, which every
    // thread finished before the barrier that ended it
    if (more) put(stage[buf ^ 1]);
    __syncthreads();
  }
}

// A segment's inputs in LDS: token i of the segment, channel c (k, q) or row
// r of the work-group's group (v, dO).
template <int kRows>
struct SegStage {
  float k[kSeg][kD], q[kSeg][kD], v[kSeg][kRows], d_o[kSeg][kRows];
  float a[kSeg], beta[kSeg];
};

// What one thread loads of a segment: k and q element m at e = tid + m kThr
// (token e / 128, channel e % 128) while e < kSeg * 128, the v and dO element
// at token tid / kRows, row tid % kRows while tid < kSeg * kRows, the gates of
// token tid while tid < kSeg.
template <int kRows>
struct SegLoad {
  static constexpr int kThr = 8 * kRows;
  static constexpr int kKQ = (kSeg * kD + kThr - 1) / kThr;
  uint16_t k[kKQ], q[kKQ], v;
  float d_o, g, beta;
};

template <int kRows>
__device__ __forceinline__ void seg_load(const BwdParams& p, int c0, int len, const RowGroup& G, int tid,
                                         SegLoad<kRows>& x) {
  constexpr int kThr = 8 * kRows;
  // per-lane addresses are formed afresh on each call (the empty asm hides
  // tid's provenance) instead of being held in registers across the walk
  asm volatile("" : "+v"(tid));
#pragma unroll
  for (int m = 0; m < SegLoad<kRows>::kKQ; ++m) {
    const int e = tid + m * kThr;
    if (e < len * kD) {
      const int64_t t = c0 + (e >> 7);
      x.k[m] = p.k[t * p.ks + G.kh * kD + (e & (kD - 1))];
      x.q[m] = p.q[t * p.qs + G.kh * kD + (e & (kD - 1))];
    }
  }
  if (tid < len * kRows) {
    const int64_t t = c0 + tid / kRows;
    const int r = G.rg * kRows + tid % kRows;
    x.v = p.v[t * p.vs + G.h * kD + r];
    x.d_o = p.d_o[(t * p.Hv + G.h) * kD + r];
  }
  if (tid < len) {
    const int64_t t = c0 + tid;
    x.g = p.g[t * p.Hv + G.h];
    x.beta = p.beta[t * p.Hv + G.h];
  }
}

template <int kRows>
__device__ __forceinline__ void seg_store(SegStage<kRows>& st, int len, int tid, const SegLoad<kRows>& x) {
  constexpr int kThr = 8 * kRows;
#pragma unroll
  for (int m = 0; m < SegLoad<kRows>::kKQ; ++m) {
    const int e = tid + m * kThr;
    if (e < len * kD) {
      st.k[e >> 7][e & (kD - 1)] = bf16_to_f32(x.k[m]);
      st.q[e >> 7][e & (kD - 1)] = bf16_to_f32(x.q[m]);
    }
  }
  if (tid < len * kRows) {
    st.v[tid / kRows][tid % kRows] = bf16_to_f32(x.v);
    st.d_o[tid / kRows][tid % kRows] = x.d_o;
  }
  if (tid < len) {
    st.a[tid] = expf(x.g);
    st.beta[tid] = x.beta;
  }
}

__device__ __forceinline__ void ckpt_load(const BwdParams& p, int c0, int n, int h, int row, int lp,
                                          float (&x)[16]) {
  const float* src = p.ckpt + ckpt_row(p, c0, n, h, row);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const floatx4 y = __builtin_nontemporal_load(reinterpret_cast<const floatx4*>(src + 4 * (lp + 8 * j)));
#pragma unroll
    for (int i = 0; i < 4; ++i) x[4 * j + i] = y[i];
  }
}

template <int kRows>
__global__ __launch_bounds__(8 * kRows, 4) void backward_rev_kernel(BwdParams p) {
  constexpr int kThr = 8 * kRows;
  constexpr int kWaves = kThr / 64;
  static_assert(kThr >= 2 * kD, "one thread per (column, dq or dk) in the final sums");
  // part and spart are double-buffered by token parity, so one barrier per
  // token suffices: a buffer written by one token (before its barrier) is
  // next written two tokens later, after every thread has passed the barrier
  // in between, which each reader reaches only after its reads.  The segment
  // stage is double-buffered by segment parity on the same argument.
  __shared__ __align__(16) float part[2][kWaves][2][kD];   // per-wave column sums: dq_h, dk_h
  __shared__ float spart[2][kWaves][2];                    // per-wave sums: <S_prev, dSh>, dbeta
  __shared__ __align__(16) SegStage<kRows> stage[2];
  // The state before the current segment's first token: lane tid's 16 values
  // as four float4 at [j][tid].  Each lane reads back only what it wrote, so
  // no barrier guards it.
  __shared__ __align__(16) floatx4 ckpt_lds[4][kThr];
  const RowGroup G = row_group(p);
  const int n = G.n, h = G.h;
  const int tid = threadIdx.x;
  const int lp = tid & 7;
  const int lrow = tid >> 3;
  const int row = G.rg * kRows + lrow;
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
  const int n_seg = (s1 - s0 + kSeg - 1) / kSeg;
  if (n_seg > 0) {
    const int c0 = s0 + (n_seg - 1) * kSeg;
    SegLoad<kRows> x;
    float cn[16];
    seg_load<kRows>(p, c0, s1 - c0, G, tid, x);
    ckpt_load(p, c0, n, h, row, lp, cn);
    seg_store<kRows>(stage[(n_seg - 1) & 1], s1 - c0, tid, x);
#pragma unroll
    for (int j = 0; j < 4; ++j) ckpt_lds[j][tid] = floatx4{cn[4 * j], cn[4 * j + 1], cn[4 * j + 2], cn[4 * j + 3]};
  }
  __syncthreads();
  int tpar = 0;   // parity of the token count processed so far (selects part, spart)
  for (int sg = n_seg - 1; sg >= 0; --sg) {
    const int c0 = s0 + sg * kSeg;
    const int len = min(kSeg, s1 - c0);
    const SegStage<kRows>& st = stage[sg & 1];
    // the previous segment's inputs are in flight during this segment
    SegLoad<kRows> xn = {};
    if (sg > 0) seg_load<kRows>(p, c0 - kSeg, kSeg, G, tid, xn);
    for (int ti = len - 1; ti >= 0; --ti) {
      const int t = c0 + ti;
      const int64_t th = static_cast<int64_t>(t) * p.Hv + h;
      // the state before token t, from the checkpoint
      float Sp[16];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const floatx4 x = ckpt_lds[j][tid];
#pragma unroll
        for (int i = 0; i < 4; ++i) Sp[4 * j + i] = x[i];
      }
#pragma unroll
      for (int j = 0; j < kSeg - 1; ++j) {
        if (j >= ti) break;   // uniform over the work-group
        float kj[16];
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const floatx4 kx = *reinterpret_cast<const floatx4*>(&st.k[j][4 * (lp + 8 * jj)]);
#pragma unroll
          for (int ii = 0; ii < 4; ++ii) kj[4 * jj + ii] = kx[ii];
        }
        const float aj = st.a[j];
        float sk = 0.f;
#pragma unroll
        for (int e = 0; e < 16; ++e) sk = fmaf(Sp[e], kj[e], sk);
        sk = sum8(sk);
        const float uj = st.beta[j] * (st.v[j][lrow] - aj * sk);
#pragma unroll
        for (int e = 0; e < 16; ++e) Sp[e] = fmaf(aj, Sp[e], uj * kj[e]);
      }
      float kk[16];
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const floatx4 kx = *reinterpret_cast<const floatx4*>(&st.k[ti][4 * (lp + 8 * jj)]);
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) kk[4 * jj + ii] = kx[ii];
      }
      const float a = st.a[ti];
      const float b = st.beta[ti];
      const float vv = st.v[ti][lrow];
      const float dout = st.d_o[ti][lrow];
      // the forward step, recomputed
      float sk = 0.f;
#pragma unroll
      for (int e = 0; e < 16; ++e) sk = fmaf(Sp[e], kk[e], sk);
      sk = sum8(sk);
      const float pk = a * sk;
      const float u = b * (vv - pk);
      // o = scale S q: D += scale dout q^T (q read from the stage as used)
      const float sd = p.scale * dout;
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const floatx4 qx = *reinterpret_cast<const floatx4*>(&st.q[ti][4 * (lp + 8 * jj)]);
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) D[4 * jj + ii] = fmaf(sd, qx[ii], D[4 * jj + ii]);
      }
      // S = Sh + u k^T
      float du = 0.f;
#pragma unroll
      for (int e = 0; e < 16; ++e) du = fmaf(D[e], kk[e], du);
      du = sum8(du);
      const float dp = -b * du;
      float gdot = 0.f;
      float cq[16], ck[16];
      const float adp = a * dp, sda = sd * a, sdu = sd * u;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        ck[e] = fmaf(D[e], u, adp * Sp[e]);
        const float dsh = fmaf(dp, kk[e], D[e]);
        gdot = fmaf(Sp[e], dsh, gdot);
        D[e] = a * dsh;
        cq[e] = fmaf(sda, Sp[e], sdu * kk[e]);   // scale dout S (the state after the token)
      }
      // the segment's first token (processed last) loads the previous
      // segment's checkpoint; it replaces this one in ckpt_lds (already read
      // by this token) before the barrier
      float cn[16];
      if (ti == 0 && sg > 0) ckpt_load(p, c0 - kSeg, n, h, row, lp, cn);
      if (lp == 0) p.dv[th * kD + row] = b * du;
      float bdot = lp == 0 ? (vv - pk) * du : 0.f;
      // Column sums over the wave's eight rows (lanes lp, lp + 8, ..., lp + 56)
      // by a butterfly reduce-scatter over lane bits 5, 4, 3: each exchange
      // sends half of the remaining values to the partner lane and keeps the
      // other half, so lane (b5 b4 b3, lp) ends with the four sums of values
      // j = 16 b5 + 8 b4 + 4 b3 + i (j < 16: cq[j], else ck[j - 16]), i.e. the
      // float4 of columns 4 (lp + 8 (2 b4 + b3)) .. + 3 of dq_h (b5 = 0) or
      // dk_h (b5 = 1).  16 + 8 permutes and a DPP step instead of 96 permutes.
      float y[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) y[i] = __shfl_xor(lane_select(kLaneBit5, cq[i], ck[i]), 32, 64);
#pragma unroll
      for (int i = 0; i < 16; ++i) y[i] += lane_select(kLaneBit5, ck[i], cq[i]);
      float z[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) z[i] = __shfl_xor(lane_select(kLaneBit4, y[i], y[8 + i]), 16, 64);
#pragma unroll
      for (int i = 0; i < 8; ++i) z[i] += lane_select(kLaneBit4, y[8 + i], y[i]);
      floatx4 r;
#pragma unroll
      for (int i = 0; i < 4; ++i)   // DPP row_ror:8 reads lane ^ 8 inside each row of 16
        r[i] = lane_select(kLaneBit3, z[4 + i], z[i]) + dpp<0x128>(lane_select(kLaneBit3, z[i], z[4 + i]));
      *reinterpret_cast<floatx4*>(&part[tpar][w][(lane >> 5) & 1][4 * (lp + 8 * ((lane >> 3) & 3))]) = r;
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
        spart[tpar][w][0] = gdot;
        spart[tpar][w][1] = bdot;
      }
      // the previous segment's inputs into the other stage buffer, last read
      // by the segment before this one, ahead of its final barrier
      if (ti == 0 && sg > 0) {
        seg_store<kRows>(stage[(sg - 1) & 1], kSeg, tid, xn);
#pragma unroll
        for (int j = 0; j < 4; ++j)
          ckpt_lds[j][tid] = floatx4{cn[4 * j], cn[4 * j + 1], cn[4 * j + 2], cn[4 * j + 3]};
      }
      __syncthreads();
      const int64_t thr = th * p.R + G.rg;   // (token, value head, row group)
      if (tid < 2 * kD) {
        const int which = tid >> 7, c = tid & (kD - 1);
        float acc = 0.f;
#pragma unroll
        for (int ww = 0; ww < kWaves; ++ww) acc += part[tpar][ww][which][c];
        (which ? p.dk_part : p.dq_part)[thr * kD + c] = acc;
      }
      if (tid == kThr - 1) {
        float gs = 0.f, bs = 0.f;
#pragma unroll
        for (int ww = 0; ww < kWaves; ++ww) {
          gs += spart[tpar][ww][0];
          bs += spart[tpar][ww][1];
        }
        p.dg_part[thr] = a * gs;
        p.dbeta_part[thr] = bs;
      }
      tpar ^= 1;
    }
  }
  if (p.dh0) {
    // the lane's offset is formed afresh here (the empty asm hides tid's
    // provenance) rather than kept live in registers across the token loops
    int tid2 = tid;
    asm volatile("" : "+v"(tid2));
    float* dst = p.dh0 + ((static_cast<int64_t>(n) * p.Hv + h) * kD + G.rg * kRows + (tid2 >> 3)) * kD;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      *reinterpret_cast<floatx4*>(dst + 4 * ((tid2 & 7) + 8 * j)) =
          floatx4{D[4 * j], D[4 * j + 1], D[4 * j + 2], D[4 * j + 3]};
  }
}

// dq, dk of key head kh = the sum of its value heads' and row groups' parts
__global__ __launch_bounds__(256) void backward_sum_kernel(const float* __restrict__ dq_part,
                                                           const float* __restrict__ dk_part,
                                                           float* __restrict__ dq, float* __restrict__ dk,
                                                           int64_t n_elem, int Hk, int Hv, int R) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= n_elem) return;                       // n_elem = T * Hk * 128
  const int c = static_cast<int>(i % kD);
  const int64_t tk = i / kD;
  const int kh = static_cast<int>(tk % Hk);
  const int64_t t = tk / Hk;
  const int parts = (Hv / Hk) * R;               // consecutive in the part arrays
  float aq = 0.f, ak = 0.f;
  for (int j = 0; j < parts; ++j) {
    const int64_t src = ((t * Hv + static_cast<int64_t>(kh) * (Hv / Hk)) * R + j) * kD + c;
    aq += dq_part[src];
    ak += dk_part[src];
  }
  dq[i] = aq;
  dk[i] = ak;
}

// dg, dbeta of (token, value head) = the sum of its row groups' parts
__global__ __launch_bounds__(256) void backward_gate_sum_kernel(const float* __restrict__ dg_part,
                                                                const float* __restrict__ db_part,
                                                                float* __restrict__ dg, float* __restrict__ dbeta,
                                                                int64_t n_elem, int R) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= n_elem) return;                       // n_elem = T * Hv
  float g = 0.f, b = 0.f;
  for (int r = 0; r < R; ++r) {
    g += dg_part[i * R + r];
    b += db_part[i * R + r];
  }
  dg[i] = g;
  dbeta[i] = b;
}

// Row groups per (sequence, value head): enough work-groups to fill the CUs
// (one 1024-thread, two 512-thread or four 256-thread work-groups fit on one).
int row_groups(int n_seqs, int Hv) {
  const int64_t units = static_cast<int64_t>(n_seqs) * Hv;
  if (units <= 128) return 4;
  // measured (medians of 9 calls, 8,192 tokens at 48 heads): 2 groups as fast
  // as 1 at 768 pairs and faster at 384, 1,536 and 3,072; 4 only below 129
  if (units <= 3072) return 2;
  return 1;
}

// checkpoint slots: below T_total / kSeg + n_seqs (ckpt_row)
size_t ckpt_floats(int n_seqs, int T_total, int Hv) {
  return (static_cast<size_t>(T_total / kSeg) + n_seqs) * Hv * kD * kD;
}

template <int kRows>
hipError_t launch_rows(const BwdParams& p, unsigned grid, hipStream_t stream) {
  hipLaunchKernelGGL(backward_fwd_kernel<kRows>, dim3(grid), dim3(8 * kRows), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(backward_rev_kernel<kRows>, dim3(grid), dim3(8 * kRows), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

size_t backward_workspace_bytes(int n_seqs, int T_total, int Hv) {
  const size_t R = row_groups(n_seqs, Hv);
  const size_t parts = 2 * static_cast<size_t>(T_total) * Hv * R * (kD + 1);
  return (ckpt_floats(n_seqs, T_total, Hv) + parts) * sizeof(float);
}

hipError_t launch_backward(const uint16_t* q, int64_t qs, const uint16_t* k, int64_t ks,
                           const uint16_t* v, int64_t vs, const float* g, const float* beta,
                           const float* h0, const float* d_o, const float* dhT, const int32_t* cu,
                           int n_seqs, int T_total, int Hk, int Hv, float scale, float* dq,
                           float* dk, float* dv, float* dg, float* dbeta, float* dh0,
                           void* workspace, hipStream_t stream) {
  if (n_seqs == 0) return hipSuccess;
  const int R = row_groups(n_seqs, Hv);
  BwdParams p;
  p.q = q; p.k = k; p.v = v; p.qs = qs; p.ks = ks; p.vs = vs; p.g = g; p.beta = beta;
  p.h0 = h0; p.d_o = d_o; p.dhT = dhT; p.cu = cu;
  float* ws = static_cast<float*>(workspace);
  const size_t tp = static_cast<size_t>(T_total) * Hv * R;   // (token, value head, row group)
  p.ckpt = ws;
  p.dq_part = ws + ckpt_floats(n_seqs, T_total, Hv);
  p.dk_part = p.dq_part + tp * kD;
  p.dg_part = p.dk_part + tp * kD;
  p.dbeta_part = p.dg_part + tp;
  p.dv = dv; p.dh0 = dh0;
  p.n_seqs = n_seqs; p.seq_len = cu ? 0 : T_total / n_seqs; p.Hk = Hk; p.Hv = Hv; p.scale = scale;
  p.R = R;
  const unsigned grid = static_cast<unsigned>(n_seqs) * static_cast<unsigned>(Hv) * static_cast<unsigned>(R);
  hipError_t e = R == 4 ? launch_rows<32>(p, grid, stream)
               : R == 2 ? launch_rows<64>(p, grid, stream)
                        : launch_rows<128>(p, grid, stream);
  if (e != hipSuccess) return e;
  const int64_t n_elem = static_cast<int64_t>(T_total) * Hk * kD;
  if (n_elem > 0) {
    hipLaunchKernelGGL(backward_sum_kernel, dim3(static_cast<unsigned>((n_elem + 255) / 256)), dim3(256), 0,
                       stream, p.dq_part, p.dk_part, dq, dk, n_elem, Hk, Hv, R);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t n_gate = static_cast<int64_t>(T_total) * Hv;
    hipLaunchKernelGGL(backward_gate_sum_kernel, dim3(static_cast<unsigned>((n_gate + 255) / 256)), dim3(256), 0,
                       stream, p.dg_part, p.dbeta_part, dg, dbeta, n_gate, R);
    e = hipGetLastError();
  }
  return e;
}

}  // namespace gdn
