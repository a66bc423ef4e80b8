// backward_chunk.hip -- chunked backward of the gated delta rule: the
// derivatives of
//     L = sum(dO * O) + sum(dS_T * S_T)
// with respect to q, k, v, g, beta and the initial state, for the rule of the
// "Delta-rule layers" row of the model card's Architecture table,
//     S <- a S + b (v - a S k) k^T,   o = scale S q,   a = exp(g),
// taken through the chunk-parallel (WY) form of the same rule that the
// prefill evaluates (chunks of 64 tokens).  Per chunk, with G the running sum
// of g inside the chunk, gamma = exp(G), M_ij = exp(G_i - G_j) (j <= i),
// D_i = exp(G_last - G_i), A = strictly lower (b_i M_ij k_i.k_j), T = (I + A)^-1:
//     E = V - gamma K S0^T,  U = T (b E),  O = scale (gamma Q S0^T + (M o Q K^T) U),
//     S_C = gamma_last S0 + U^T D K.
// Its chain rule, with dS_C the gradient of the chunk's final state:
//     dU = scale P^T dO + D K dS_C^T,   dR = T^T dU,   dv = b dR,
//     dS0 = gamma_last dS_C + scale (gamma Q)^T-weighted dO - (b gamma K)-weighted dR
//     dA = -dR U^T,  dP = scale dO U^T,
//     dq = scale gamma dO S0 + (dP o M) K,
//     dk = (dP o M)^T Q + D U dS_C - gamma b dR S0 + W K + W^T K,  W = b o dA o M,
//     dbeta_i = dR_i . E_i + sum_j dA_ij M_ij k_i.k_j,
// and the gradient of the log-decays through every gamma, M and D they enter,
// collected per token as dG_i = q_i . dq_i + k_i . (W K - W^T K - (dP o M)^T Q
// - gamma b dR S0 - D U dS_C)_i (+ gamma_last <dS_C, S0> + sum_m k_m . (D U dS_C)_m
// on the last token), then dg = the suffix sum of dG over the chunk.
//
// Six launches:
//   cb_fill/cb_table   chunk slots -> sequence (slot = first token / 64 + sequence)
//   cb_prep            per (chunk, key head): Q K^T, K K^T (fp32 MFMA), then per
//                      value head one 64 x 64 matrix X: A below the four
//                      diagonal 16 x 16 blocks, inside them the blocks of
//                      T_II = (I + A_II)^-1 (forward substitution, one column
//                      per lane; unit diagonal), P_ii on the diagonal and
//                      P_ji above it.  The chains solve with (I + A) blockwise.
//   cb_fwd, cb_bwd     per (sequence, value head, 64 channels): the state chain
//                      forwards, recording S0, U, E of every chunk, and beside
//                      it on the library's second stream the gradient chain
//                      backwards (it needs none of those), recording dS_C and
//                      dR, writing dv and dh0
//   cb_grad            per (chunk, key head): dq, dk (summed over the value
//                      heads in registers), dg, dbeta
// The large contractions run on the bf16 matrix units with fp32 operands
// split into bf16 hi + lo parts (about 2^-17 relative error per product,
// fp32's exponent range): in the chains K S0^T, K dS^T and the state (and
// state-gradient) updates, whose K and Q operands are bf16 already (two
// products each), and every product of the gradient pass (three each where
// both operands are fp32).  Q K^T and K K^T take the bf16 inputs as they
// stand (exact products).  Only the chains' triangular solves and P^T dO run
// on v_mfma_f32_16x16x4_f32.  Either way the gradients keep their accuracy
// at any scale of dO.  In the chains every
// 64-token x 16-channel intermediate stays in the accumulator layout (lane l:
// rows 4 (l / 16) + r, column l % 16) and enters the next product as its B
// operand directly; the A operand then takes its k columns in the same order.
#include <mutex>

#include "common.h"
#include "launch.h"

namespace gdn {

namespace {

constexpr int kD = 128;
constexpr int kC = 64;
constexpr int kKS = 136;          // bf16 row stride of staged K / Q rows (272 bytes)
constexpr int kXS = 68;           // fp32 row stride of staged X (272 bytes)

struct CbParams {
  const uint16_t* q; const uint16_t* k; const uint16_t* v;
  int64_t qs, ks, vs;
  const float* g; const float* beta;
  const float* h0; const float* d_o; const float* dhT;
  const int32_t* cu;          // nullptr: equal lengths seq_len
  int n_seqs, seq_len, Hk, Hv, group, n_slots;
  float scale;
  int32_t* slot_seq;          // [n_slots]: sequence of the chunk in the slot, -1 for none
  float* X;                   // [n_slots][Hv][64][64]: A, T_II, P (see cb_prep)
  float* S0;                  // [n_slots][Hv][128][128]: state before the chunk, [dv][dk]
  float* dSC;                 // [n_slots][Hv][128][128]: dL/dS after the chunk
  float* U; float* E; float* dR;   // [n_slots][Hv][64][128]
  float* dq; float* dk; float* dv; float* dg; float* dbeta; float* dh0;
  // part 0: every chunk.  Parts 1 and 2: the chunks of each sequence from
  // mid = nc / 2 on, and those before it.  The gradient chain's part 1 leaves
  // the state gradient after chunk mid - 1 in that chunk's dSC slot, where
  // part 2 takes it up; the gradient pass of a part does that part's chunks.
  int part;
};

__device__ __forceinline__ floatx4 mfma4(float a, float b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float bf(uint16_t x) { return bf16_to_f32(x); }

// Products on the bf16 matrix units with fp32-like accuracy: each fp32 operand
// x is split as x = hi + lo, hi = x rounded to bf16 (nearest even), lo = the
// remainder x - hi (exact in fp32) rounded to bf16, and a b is taken as
// hi_a hi_b + hi_a lo_b + lo_a hi_b: the dropped lo_a lo_b and lo's rounding
// leave a relative error of about 2^-17 per product, with fp32's exponent
// range (the split needs no scaling at any magnitude of the data).
typedef __bf16 bf16x8v __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
typedef float float2v __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pk_bf16(float a, float b) {   // nearest even
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(float2v{a, b}, bf16x2v));
}
__device__ __forceinline__ void split8(const float (&x)[8], bf16x8v& hi, bf16x8v& lo) {
  uint32_t h[4], l[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    h[j] = pk_bf16(x[2 * j], x[2 * j + 1]);
    const float ra = x[2 * j] - __uint_as_float(h[j] << 16);
    const float rb = x[2 * j + 1] - __uint_as_float(h[j] & 0xffff0000u);
    l[j] = pk_bf16(ra, rb);
  }
  hi = __builtin_bit_cast(bf16x8v, uint4{h[0], h[1], h[2], h[3]});
  lo = __builtin_bit_cast(bf16x8v, uint4{l[0], l[1], l[2], l[3]});
}
// acc += a b over k = 32 (16 x 16 x 32: lane l gives A[l % 16][8 (l / 16) + j]
// and B[8 (l / 16) + j][l % 16]; the result keeps the 16 x 16 x 4 layout)
__device__ __forceinline__ floatx4 mfma_split(const bf16x8v ah, const bf16x8v al, const bf16x8v bh,
                                              const bf16x8v bl, floatx4 acc) {
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bh, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bl, acc, 0, 0, 0);
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, bh, acc, 0, 0, 0);
}

typedef short short4v __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) short4v lds_short4;

// Split-bf16 operands of the chains' 16 x 16 x 32 products.  The reduction
// index of slot (lane group g, element e) is kappa(g, e) = 4 g + e for e < 4
// and 16 + 4 g + (e - 4) otherwise, so that two vertically adjacent
// accumulator tiles (rows 4 g + r of tile a, then of tile b) are a B operand
// over those 32 rows as they stand.  K and Q are bf16 already: as A operands
// they need no split, and a product takes two passes (a hi', a lo').
__device__ __forceinline__ void split_pair(const floatx4 a, const floatx4 b, bf16x8v& hi, bf16x8v& lo) {
  const float x[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  split8(x, hi, lo);
}
// row `row` of a staged matrix, reduction indices c0 + kappa(g4, e)
__device__ __forceinline__ bf16x8v row8(const uint16_t (*rows)[kKS], int row, int c0, int g4) {
  const uint2 a = *reinterpret_cast<const uint2*>(&rows[row][c0 + 4 * g4]);
  const uint2 b = *reinterpret_cast<const uint2*>(&rows[row][c0 + 16 + 4 * g4]);
  return __builtin_bit_cast(bf16x8v, uint4{a.x, a.y, b.x, b.y});
}
// column c0 + (lane % 16) of a staged matrix, rows r0 + kappa(lane / 16, e):
// two transposing reads
__device__ __forceinline__ bf16x8v col8(const uint16_t (*rows)[kKS], int r0, int c0) {
  const int j = threadIdx.x & 15;
  const int g4 = (threadIdx.x >> 4) & 3;
  const short4v a = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_short4*)(&rows[r0 + 4 * g4 + (j >> 2)][c0 + 4 * (j & 3)]));
  const short4v b = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_short4*)(&rows[r0 + 16 + 4 * g4 + (j >> 2)][c0 + 4 * (j & 3)]));
  const uint2 ua = __builtin_bit_cast(uint2, a), ub = __builtin_bit_cast(uint2, b);
  return __builtin_bit_cast(bf16x8v, uint4{ua.x, ua.y, ub.x, ub.y});
}
__device__ __forceinline__ floatx4 mfma_bf(const bf16x8v a, const bf16x8v b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ void cb_seq(const CbParams& p, int n, int& s0, int& s1) {
  if (p.cu) { s0 = p.cu[n]; s1 = p.cu[n + 1]; }
  else { s0 = n * p.seq_len; s1 = s0 + p.seq_len; }
}

// Slot of chunk c of sequence n (first token s0): s0 / 64 + c + n grows by
// one per chunk of a sequence and by at least one from a sequence's last chunk
// to the next sequence's first, so slots are distinct and below T / 64 + N.
__device__ __forceinline__ int cb_slot(int s0, int c, int n) { return (s0 >> 6) + c + n; }

struct SlotChunk { int n, t0, len; };
__device__ __forceinline__ bool slot_chunk(const CbParams& p, int slot, SlotChunk& sc) {
  const int n = p.slot_seq[slot];
  if (n < 0) return false;
  int s0, s1;
  cb_seq(p, n, s0, s1);
  sc.n = n;
  sc.t0 = s0 + kC * (slot - n - (s0 >> 6));
  sc.len = min(kC, s1 - sc.t0);
  return true;
}

// inclusive prefix sum over the 64 lanes, in lane order
__device__ __forceinline__ float wave_prefix_sum(float x, int lane = threadIdx.x & 63) {
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const float y = __shfl_up(x, d, 64);
    if (lane >= d) x += y;
  }
  return x;
}

// sum over the 64 lanes: DPP inside the four rows of 16, then across them
__device__ __forceinline__ float wave_sum(float x) {
  x = sum16(x);
  x += __shfl_xor(x, 16, 64);
  x += __shfl_xor(x, 32, 64);
  return x;
}

// Gates of one chunk and value head, lane i = token i of the chunk (g and
// beta are 0 past its end, so G_63 = G_last and the padded tokens drop out).
struct Gates { float G, gam, dec, bet; };
__device__ __forceinline__ Gates chunk_gates(const CbParams& p, int t0, int len, int h) {
  const int i = threadIdx.x & 63;
  const bool ok = i < len;
  const int64_t gi_at = static_cast<int64_t>(t0 + min(i, len - 1)) * p.Hv + h;
  const float gv = p.g[gi_at], bv = p.beta[gi_at];   // unconditional loads: no branch, no wait
  const float gi = ok ? gv : 0.f;
  Gates r;
  r.bet = ok ? bv : 0.f;
  r.G = wave_prefix_sum(gi);
  const float GL = __shfl(r.G, 63, 64);
  r.gam = expf(r.G);
  r.dec = expf(GL - r.G);
  return r;
}

// Stage the chunk's 64 rows of bf16 K (or Q) of key head kh into LDS rows of
// kKS halves, zero past the end; kThr threads, each 8192 / kThr halves of a row
// (rows 16-byte aligned: the entry point checks the pointers and strides).
template <int kThr>
__device__ __forceinline__ void stage_rows(const uint16_t* src, int64_t stride, int t0, int len, int kh,
                                           uint16_t (*dst)[kKS]) {
  constexpr int kPer = kC * kD / kThr;          // halves per thread: 32 (256 thr) or 16 (512)
  constexpr int kRowThr = kD / kPer;            // threads per row
  const int tid = threadIdx.x;
  const int row = tid / kRowThr;
  // piece j of a thread: channels 8 (tid % kRowThr + kRowThr j) .. + 7, so
  // that the threads of a row read contiguous bytes in each load
  const int c0 = (tid % kRowThr) * 8;
  const bool ok = row < len;
  const uint16_t* s = src + static_cast<int64_t>(t0 + min(row, len - 1)) * stride + kh * kD + c0;
#pragma unroll
  for (int j = 0; j < kPer / 8; ++j) {
    const uint4 y = *reinterpret_cast<const uint4*>(s + 8 * kRowThr * j);
    const uint4 x = ok ? y : make_uint4(0, 0, 0, 0);
    *reinterpret_cast<uint4*>(&dst[row][c0 + 8 * kRowThr * j]) = x;
  }
}

// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void cb_fill_kernel(int32_t* __restrict__ slot_seq, int n) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) slot_seq[i] = -1;
}

__global__ __launch_bounds__(256) void cb_table_kernel(CbParams p) {
  const int n = blockIdx.x * 256 + threadIdx.x;
  if (n >= p.n_seqs) return;
  int s0, s1;
  cb_seq(p, n, s0, s1);
  const int nc = (s1 - s0 + kC - 1) / kC;
  for (int c = 0; c < nc; ++c) p.slot_seq[cb_slot(s0, c, n)] = n;
}

// ---------------------------------------------------------------------------
// cb_prep: one work-group (4 waves) per (chunk slot, key head).
constexpr int kSS = 65;           // fp32 row stride of Q K^T, K K^T
struct PrepLds {
  uint16_t q[kC][kKS], k[kC][kKS];
  float qkt[kC][kSS];
  float kkt[kC][kSS];
};

__device__ __forceinline__ float lane_value(float x, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), lane));
}

__global__ __launch_bounds__(256) void cb_prep_kernel(CbParams p) {
  __shared__ __align__(16) PrepLds sm;
  const int slot = blockIdx.x / p.Hk;
  const int kh = blockIdx.x - slot * p.Hk;
  SlotChunk sc;
  if (!slot_chunk(p, slot, sc)) return;
  const int tid = threadIdx.x;
  const int w = tid >> 6;
  const int lane = tid & 63;
  const int m = lane & 15;
  const int g4 = lane >> 4;

  stage_rows<256>(p.q, p.qs, sc.t0, sc.len, kh, sm.q);
  stage_rows<256>(p.k, p.ks, sc.t0, sc.len, kh, sm.k);
  __syncthreads();
  // Q K^T and K K^T on and below the diagonal: 2 x 10 blocks of 16 x 16
  for (int job = w; job < 20; job += 4) {
    const int kind = job / 10;
    const int b = job - 10 * kind;
    const int ib = b < 1 ? 0 : b < 3 ? 1 : b < 6 ? 2 : 3;
    const int jb = b - ib * (ib + 1) / 2;
    const uint16_t (*A)[kKS] = kind ? sm.k : sm.q;
    floatx4 acc = {0.f, 0.f, 0.f, 0.f};
    // bf16 operands as they stand (their products are exact in fp32), 32 of
    // the reduction a step
#pragma unroll
    for (int kp = 0; kp < kD / 32; ++kp)
      acc = mfma_bf(row8(A, ib * 16 + m, 32 * kp, g4), row8(sm.k, jb * 16 + m, 32 * kp, g4), acc);
    float (*dst)[kSS] = kind ? sm.kkt : sm.qkt;
#pragma unroll
    for (int r = 0; r < 4; ++r) dst[ib * 16 + 4 * g4 + r][jb * 16 + m] = acc[r];
  }
  __syncthreads();

  for (int hv = w; hv < p.group; hv += 4) {
    // the lane index from an opaque copy: its 64 per-row comparisons below
    // are then made row by row instead of hoisted out of this loop
    int lane_v = lane;
    asm volatile("" : "+v"(lane_v));
    const int lane = lane_v;
    const int h = kh * p.group + hv;
    const Gates gt = chunk_gates(p, sc.t0, sc.len, h);
    // The diagonal 16 x 16 blocks of T = (I + A)^-1, T_II = (I + A_II)^-1, by
    // forward substitution: lane 16 I + c holds column c of T_II (t[ii] = row
    // ii), A_ij = b_i M_ij k_i.k_j (j < i) comes from the lane of column j in
    // the same 16-lane group:  T_ic = delta_ic - sum_{j<i} A_ij T_jc.
    const int blk = lane >> 4;
    const int c = lane & 15;
    float t[16];
#pragma unroll
    for (int ii = 0; ii < 16; ++ii) {
      const int i = 16 * blk + ii;
      const float Gi = __shfl(gt.G, i, 64);
      const float bi = __shfl(gt.bet, i, 64);
      const float a = c < ii ? bi * expf(Gi - gt.G) * sm.kkt[i][lane] : 0.f;
      float acc = c == ii ? 1.f : 0.f;
#pragma unroll
      for (int jj = 0; jj < ii; ++jj) acc = fmaf(-__shfl(a, 16 * blk + jj, 64), t[jj], acc);
      t[ii] = acc;
    }
    // X row i, lane = column j: A_ij below the diagonal blocks, T_II inside
    // them (below the diagonal), P_ii on the diagonal, P_ji = M_ji q_j.k_i above
    float* Xh = p.X + (static_cast<int64_t>(slot) * p.Hv + h) * (kC * kC);
#pragma unroll
    for (int i = 0; i < kC; ++i) {
      const float Gi = lane_value(gt.G, i);
      const float bi = lane_value(gt.bet, i);
      const float e = expf(lane < i ? Gi - gt.G : gt.G - Gi);
      Xh[i * kC + lane] = lane < (i & ~15) ? bi * e * sm.kkt[i][lane]
                        : lane < i          ? t[i & 15]
                                            : e * sm.qkt[lane][i];
      __builtin_amdgcn_sched_barrier(0);
    }
  }
}

// ---------------------------------------------------------------------------
// The chains' per-chunk inputs in LDS, and their prefetch: the next chunk's
// K (and Q) rows, its X and its gates are loaded into registers while the
// current chunk computes, and written to LDS after it.
// LDS added to each chain work-group when the two chains' work-groups fit
// the CUs one each: the dispatcher would otherwise put two on a CU (their
// LDS and registers allow it), and the two chains, each a sequence of
// dependent products, then share the CU's SIMDs (one sequence of 8192 tokens:
// 1.97 ms against 1.66 ms with the pad)
constexpr size_t kChainPad = 32 * 1024;
struct ChainLds {
  uint16_t k[kC][kKS];
  uint16_t q[kC][kKS];
  float x[kC][kXS];
  float gam[kC], dec[kC], bet[kC];
};

template <bool kWithQ>
struct ChainNext {
  uint4 k[4];
  uint4 q[kWithQ ? 4 : 1];
  floatx4 x[4];
  float g, b;                 // lane i: token i's g and beta
  int len;                    // tokens of the chunk: rows and gates past it are zeroed in chain_put
};

template <bool kWithQ>
__device__ __forceinline__ void chain_load(const CbParams& p, int t0, int len, int h, int kh,
                                           int64_t sh, ChainNext<kWithQ>& f,
                                           int tid = threadIdx.x) {
  const int lane = tid & 63;
  // K / Q: 32 halves, X: 16 floats per thread, in pieces of 16 bytes: piece
  // j at halves 8 (tid % 4) + 32 j (X: floats 4 (tid % 4) + 16 j), so that
  // the 4 threads of a row read contiguous bytes in each load
  const int row = tid >> 2;
  const bool ok = row < len;
  const int64_t t = t0 + min(row, len - 1);   // rows past the end load the last, then zero
  const uint16_t* sk = p.k + t * p.ks + kh * kD + (tid & 3) * 8;
#pragma unroll
  for (int j = 0; j < 4; ++j) f.k[j] = *reinterpret_cast<const uint4*>(sk + 32 * j);
  if (kWithQ) {
    const uint16_t* sq = p.q + t * p.qs + kh * kD + (tid & 3) * 8;
#pragma unroll
    for (int j = 0; j < 4; ++j) f.q[j] = *reinterpret_cast<const uint4*>(sq + 32 * j);
  }
  (void)ok;
  f.len = len;
  const float* sx = p.X + sh * (kC * kC) + row * kC + (tid & 3) * 4;
#pragma unroll
  for (int j = 0; j < 4; ++j) f.x[j] = *reinterpret_cast<const floatx4*>(sx + 16 * j);
  const int64_t gi_at = static_cast<int64_t>(t0 + min(lane, len - 1)) * p.Hv + h;
  f.g = p.g[gi_at];
  f.b = p.beta[gi_at];
}

template <bool kWithQ>
// (the rows and gates past the chunk's end, loaded from its last token, are
// zeroed here rather than at the load, where the choice would wait for them)
__device__ __forceinline__ void chain_put(const ChainNext<kWithQ>& f, ChainLds& sm,
                                          int tid = threadIdx.x) {
  const int row = tid >> 2;
  const uint32_t keep = row < f.len ? 0xffffffffu : 0u;   // a value mask, not a choice of objects
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint4 kv = f.k[j];
    *reinterpret_cast<uint4*>(&sm.k[row][(tid & 3) * 8 + 32 * j]) =
        make_uint4(kv.x & keep, kv.y & keep, kv.z & keep, kv.w & keep);
    if (kWithQ) {
      const uint4 qv = f.q[j];
      *reinterpret_cast<uint4*>(&sm.q[row][(tid & 3) * 8 + 32 * j]) =
          make_uint4(qv.x & keep, qv.y & keep, qv.z & keep, qv.w & keep);
    }
    *reinterpret_cast<floatx4*>(&sm.x[row][(tid & 3) * 4 + 16 * j]) = f.x[j];
  }
  if ((tid >> 6) == 0) {
    const int lane = tid & 63;
    const bool gok = lane < f.len;
    const float G = wave_prefix_sum(gok ? f.g : 0.f, lane);
    const float GL = __shfl(G, 63, 64);
    sm.gam[lane] = expf(G);
    sm.dec[lane] = expf(GL - G);
    sm.bet[lane] = gok ? f.b : 0.f;
  }
}

// ---------------------------------------------------------------------------
// cb_fwd: one work-group (4 waves) per (sequence, value head, 64 channels);
// wave w carries channels 16 (4 half + w) .. + 15 of S^T in 8 accumulators
// (s[db][r] = S^T[16 db + 4 (lane / 16) + r][channel 16 tile + lane % 16]).


__device__ __forceinline__ void fwd_chain(const CbParams& p, ChainLds& sm, int block) {
  const int unit = block >> 1;
  const int half = block & 1;
  const int n = unit / p.Hv;
  const int h = unit - n * p.Hv;
  const int kh = h / p.group;
  const int tid = threadIdx.x;
  const int w = tid >> 6;
  const int lane = tid & 63;
  const int m = lane & 15;
  const int g4 = lane >> 4;
  const int ch = (4 * half + w) * 16 + m;
  int s0, s1;
  cb_seq(p, n, s0, s1);
  const int nc = (s1 - s0 + kC - 1) / kC;

  floatx4 s[8];
  const int64_t hrow = ((static_cast<int64_t>(n) * p.Hv + h) * kD + ch) * kD + 4 * g4;
#pragma unroll
  for (int db = 0; db < 8; ++db)
    s[db] = p.h0 ? *reinterpret_cast<const floatx4*>(p.h0 + hrow + 16 * db) : floatx4{0.f, 0.f, 0.f, 0.f};

  ChainNext<false> nx;
  if (nc > 0) {
    chain_load(p, s0, min(kC, s1 - s0), h, kh, static_cast<int64_t>(cb_slot(s0, 0, n)) * p.Hv + h, nx);
    chain_put(nx, sm);
  }
  __syncthreads();
  for (int c = 0; c < nc; ++c) {
    // the thread id again from an opaque copy: the prefetch's and LDS writes'
    // lane arithmetic is then redone per chunk, not held in registers
    int tid_c = tid;
    asm volatile("" : "+v"(tid_c));
    const int t0 = s0 + kC * c;
    const int len = min(kC, s1 - t0);
    const int slot = cb_slot(s0, c, n);
    const int64_t sh = static_cast<int64_t>(slot) * p.Hv + h;
    // this chunk's V (used after Z), then the next chunk's inputs
    float vv[4][4];
#pragma unroll
    for (int tb = 0; tb < 4; ++tb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int tok = tb * 16 + 4 * g4 + r;
        vv[tb][r] = bf(p.v[static_cast<int64_t>(t0 + min(tok, len - 1)) * p.vs + h * kD + ch]);
      }
    if (c + 1 < nc)
      chain_load(p, t0 + kC, min(kC, s1 - t0 - kC), h, kh, static_cast<int64_t>(slot + 1) * p.Hv + h, nx, tid_c);

    // the state before the chunk
    float* S0 = p.S0 + (sh * kD + ch) * kD + 4 * g4;
#pragma unroll
    for (int db = 0; db < 8; ++db) *reinterpret_cast<floatx4*>(S0 + 16 * db) = s[db];

    // Z = K S0^T (tokens x channels): split-bf16, 32 state rows a step
    floatx4 z[4];
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) z[tb] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kp = 0; kp < 4; ++kp) {
      bf16x8v bh, bl;
      split_pair(s[2 * kp], s[2 * kp + 1], bh, bl);
#pragma unroll
      for (int tb = 0; tb < 4; ++tb) {
        const bf16x8v ka = row8(sm.k, tb * 16 + m, 32 * kp, g4);
        z[tb] = mfma_bf(ka, bh, z[tb]);
        z[tb] = mfma_bf(ka, bl, z[tb]);
      }
    }
    // E = V - gamma Z, R = b E  (token tb*16 + 4 g4 + r, channel ch)
    float* Eh = p.E + sh * (kC * kD) + ch;
    floatx4 R[4];
#pragma unroll
    for (int tb = 0; tb < 4; ++tb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int tok = tb * 16 + 4 * g4 + r;
        // V past the chunk's end (loaded from its last token) counts as zero
        const float e = (tok < len ? vv[tb][r] : 0.f) - sm.gam[tok] * z[tb][r];
        Eh[tok * kD] = e;
        R[tb][r] = sm.bet[tok] * e;
      }
    // U = (I + A)^-1 R blockwise: U_I = T_II (R_I - sum_{J<I} A_IJ U_J)
    float* Uh = p.U + sh * (kC * kD) + ch;
    floatx4 U[4], DU[4];
#pragma unroll
    for (int ib = 0; ib < 4; ++ib) {
      const int i = ib * 16 + m;
      floatx4 y = R[ib];
#pragma unroll
      for (int jb = 0; jb < ib; ++jb) {
        const floatx4 xr = *reinterpret_cast<const floatx4*>(&sm.x[i][jb * 16 + 4 * g4]);
#pragma unroll
        for (int r = 0; r < 4; ++r) y = mfma4(-xr[r], U[jb][r], y);
      }
      const int j0 = ib * 16 + 4 * g4;
      const floatx4 xr = *reinterpret_cast<const floatx4*>(&sm.x[i][j0]);
      floatx4 u = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int r = 0; r < 4; ++r) u = mfma4(j0 + r < i ? xr[r] : j0 + r == i ? 1.f : 0.f, y[r], u);
      U[ib] = u;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int tok = ib * 16 + 4 * g4 + r;
        Uh[tok * kD] = u[r];
        DU[ib][r] = sm.dec[tok] * u[r];
      }
    }
    // S^T <- gamma_last S^T + K^T (D U): split-bf16, 32 tokens a step
    const float gl = sm.gam[kC - 1];
    bf16x8v duh[2], dul[2];
#pragma unroll
    for (int kp = 0; kp < 2; ++kp) split_pair(DU[2 * kp], DU[2 * kp + 1], duh[kp], dul[kp]);
#pragma unroll
    for (int db = 0; db < 8; ++db) {
      floatx4 acc = s[db] * gl;
#pragma unroll
      for (int kp = 0; kp < 2; ++kp) {
        const bf16x8v kt = col8(sm.k, 32 * kp, db * 16);
        acc = mfma_bf(kt, duh[kp], acc);
        acc = mfma_bf(kt, dul[kp], acc);
      }
      s[db] = acc;
    }
    __syncthreads();   // every wave is done with this chunk's LDS
    if (c + 1 < nc) {
      chain_put(nx, sm, tid_c);
      __syncthreads();
    }
  }
}

// ---------------------------------------------------------------------------
// cb_bwd: the gradient chain, chunks in reverse; wave layout as cb_fwd, with
// ds[db][r] = dS^T[16 db + 4 (lane / 16) + r][channel].
__device__ __forceinline__ void bwd_chain(const CbParams& p, ChainLds& sm, int block) {
  const int unit = block >> 1;
  const int half = block & 1;
  const int n = unit / p.Hv;
  const int h = unit - n * p.Hv;
  const int kh = h / p.group;
  const int tid = threadIdx.x;
  const int w = tid >> 6;
  const int lane = tid & 63;
  const int m = lane & 15;
  const int g4 = lane >> 4;
  const int ch = (4 * half + w) * 16 + m;
  int s0, s1;
  cb_seq(p, n, s0, s1);
  const int nc = (s1 - s0 + kC - 1) / kC;
  const int mid = nc / 2;
  const int c_top = p.part == 2 ? mid : nc;     // chunks c_top - 1 .. c_lo
  const int c_lo = p.part == 1 ? mid : 0;
  if (p.part == 2 && c_top == 0) return;        // no lower part (the whole work-group)

  floatx4 ds[8];
  if (c_top == nc) {
    const int64_t hrow = ((static_cast<int64_t>(n) * p.Hv + h) * kD + ch) * kD + 4 * g4;
#pragma unroll
    for (int db = 0; db < 8; ++db)
      ds[db] = p.dhT ? *reinterpret_cast<const floatx4*>(p.dhT + hrow + 16 * db) : floatx4{0.f, 0.f, 0.f, 0.f};
  } else {
    // left by the part above in the slot of chunk c_top - 1
    const int64_t sh = static_cast<int64_t>(cb_slot(s0, c_top - 1, n)) * p.Hv + h;
    const float* src = p.dSC + (sh * kD + ch) * kD + 4 * g4;
#pragma unroll
    for (int db = 0; db < 8; ++db) ds[db] = *reinterpret_cast<const floatx4*>(src + 16 * db);
  }

  ChainNext<true> nx;
  if (c_top > c_lo) {
    const int tl = s0 + kC * (c_top - 1);
    chain_load(p, tl, min(kC, s1 - tl), h, kh, static_cast<int64_t>(cb_slot(s0, c_top - 1, n)) * p.Hv + h, nx);
    chain_put(nx, sm);
  }
  __syncthreads();
  for (int c = c_top - 1; c >= c_lo; --c) {
    int tid_c = tid;
    asm volatile("" : "+v"(tid_c));
    const int t0 = s0 + kC * c;
    const int len = min(kC, s1 - t0);
    const int slot = cb_slot(s0, c, n);
    const int64_t sh = static_cast<int64_t>(slot) * p.Hv + h;
    // dO of the chunk in the accumulator layout (token tb*16 + 4 g4 + r)
    floatx4 dO[4];
#pragma unroll
    for (int tb = 0; tb < 4; ++tb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int tok = tb * 16 + 4 * g4 + r;
        dO[tb][r] = p.d_o[(static_cast<int64_t>(t0 + min(tok, len - 1)) * p.Hv + h) * kD + ch];
      }
    // the previous chunk's inputs, written to LDS after this one
    if (c > c_lo) chain_load(p, t0 - kC, kC, h, kh, static_cast<int64_t>(slot - 1) * p.Hv + h, nx, tid_c);

    // the gradient of the state after the chunk
    float* dSC = p.dSC + (sh * kD + ch) * kD + 4 * g4;
#pragma unroll
    for (int db = 0; db < 8; ++db) *reinterpret_cast<floatx4*>(dSC + 16 * db) = ds[db];

    // Z = K dS^T: split-bf16, 32 state rows a step
    floatx4 z[4];
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) z[tb] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kp = 0; kp < 4; ++kp) {
      bf16x8v bh, bl;
      split_pair(ds[2 * kp], ds[2 * kp + 1], bh, bl);
#pragma unroll
      for (int tb = 0; tb < 4; ++tb) {
        const bf16x8v ka = row8(sm.k, tb * 16 + m, 32 * kp, g4);
        z[tb] = mfma_bf(ka, bh, z[tb]);
        z[tb] = mfma_bf(ka, bl, z[tb]);
      }
    }
    // dU = scale P^T dO + D Z;  (P^T)_ij = P_ji = X_ij for j > i, X_ii on the diagonal
    floatx4 dU[4];
#pragma unroll
    for (int ib = 0; ib < 4; ++ib) {
      const int i = ib * 16 + m;
      floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int jb = ib; jb < 4; ++jb) {
        const int j0 = jb * 16 + 4 * g4;
        const floatx4 xr = *reinterpret_cast<const floatx4*>(&sm.x[i][j0]);
#pragma unroll
        for (int r = 0; r < 4; ++r) acc = mfma4(j0 + r >= i ? xr[r] : 0.f, dO[jb][r], acc);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) dU[ib][r] = p.scale * acc[r] + sm.dec[ib * 16 + 4 * g4 + r] * z[ib][r];
    }
    // dR = (I + A)^-T dU blockwise, last block first:
    //   dR_I = T_II^T (dU_I - sum_{J>I} A_JI^T dR_J)
    float* dRh = p.dR + sh * (kC * kD) + ch;
    floatx4 dR[4];
#pragma unroll
    for (int ib = 3; ib >= 0; --ib) {
      const int i = ib * 16 + m;
      floatx4 y = dU[ib];
#pragma unroll
      for (int jb = ib + 1; jb < 4; ++jb)
#pragma unroll
        for (int r = 0; r < 4; ++r) y = mfma4(-sm.x[jb * 16 + 4 * g4 + r][i], dR[jb][r], y);
      floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int j = ib * 16 + 4 * g4 + r;
        acc = mfma4(j > i ? sm.x[j][i] : j == i ? 1.f : 0.f, y[r], acc);
      }
      dR[ib] = acc;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int tok = ib * 16 + 4 * g4 + r;
        dRh[tok * kD] = acc[r];
        if (tok < len) p.dv[(static_cast<int64_t>(t0 + tok) * p.Hv + h) * kD + ch] = sm.bet[tok] * acc[r];
      }
    }
    // dS^T <- gamma_last dS^T + Q^T (scale gamma dO) - K^T (b gamma dR):
    // dO and dR scaled in place (not needed again)
#pragma unroll
    for (int jb = 0; jb < 4; ++jb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int tok = jb * 16 + 4 * g4 + r;
        dO[jb][r] *= p.scale * sm.gam[tok];
        dR[jb][r] *= -sm.bet[tok] * sm.gam[tok];
      }
    // split-bf16, 32 tokens a step (the step's split operands, then every
    // row block of dS^T)
    const float gl = sm.gam[kC - 1];
#pragma unroll
    for (int db = 0; db < 8; ++db) ds[db] *= gl;
#pragma unroll
    for (int kp = 0; kp < 2; ++kp) {
      bf16x8v doh, dol, drh, drl;
      split_pair(dO[2 * kp], dO[2 * kp + 1], doh, dol);
      split_pair(dR[2 * kp], dR[2 * kp + 1], drh, drl);
#pragma unroll
      for (int db = 0; db < 8; ++db) {
        const bf16x8v qt = col8(sm.q, 32 * kp, db * 16);
        const bf16x8v kt = col8(sm.k, 32 * kp, db * 16);
        ds[db] = mfma_bf(qt, doh, ds[db]);
        ds[db] = mfma_bf(qt, dol, ds[db]);
        ds[db] = mfma_bf(kt, drh, ds[db]);
        ds[db] = mfma_bf(kt, drl, ds[db]);
      }
    }
    __syncthreads();   // every wave is done with this chunk's LDS
    if (c > c_lo) {
      chain_put(nx, sm, tid_c);
      __syncthreads();
    }
  }
  // the row offset again from an opaque thread id, not held through the loop
  int tid_e = tid;
  asm volatile("" : "+v"(tid_e));
  const int ch_e = (4 * half + (tid_e >> 6)) * 16 + (tid_e & 15);
  if (c_lo > 0) {
    // the gradient of the state after chunk c_lo - 1, for the part below
    const int64_t sh = static_cast<int64_t>(cb_slot(s0, c_lo - 1, n)) * p.Hv + h;
    float* dst = p.dSC + (sh * kD + ch_e) * kD + 4 * ((tid_e >> 4) & 3);
#pragma unroll
    for (int db = 0; db < 8; ++db) *reinterpret_cast<floatx4*>(dst + 16 * db) = ds[db];
  } else if (p.dh0) {
    const int64_t hrow_e = ((static_cast<int64_t>(n) * p.Hv + h) * kD + ch_e) * kD + 4 * ((tid_e >> 4) & 3);
#pragma unroll
    for (int db = 0; db < 8; ++db) *reinterpret_cast<floatx4*>(p.dh0 + hrow_e + 16 * db) = ds[db];
  }
}

static_assert(2 * (sizeof(ChainLds) + kChainPad) > 160 * 1024 && sizeof(ChainLds) + kChainPad <= 160 * 1024,
              "a padded chain work-group fits a CU, two do not");

__global__ __launch_bounds__(256, 2) void cb_fwd_kernel(CbParams p) {
  __shared__ __align__(16) ChainLds sm;
  fwd_chain(p, sm, blockIdx.x);
}

__global__ __launch_bounds__(256, 2) void cb_bwd_kernel(CbParams p) {
  __shared__ __align__(16) ChainLds sm;
  bwd_chain(p, sm, blockIdx.x);
}

// ---------------------------------------------------------------------------
// cb_grad: one work-group (8 waves) per (chunk slot, key head).  Wave w owns
// columns 16 w .. 16 w + 15 of the 64 x 128 results (dq, dk and their parts),
// and a share of the 64 x 64 products dP = scale dO U^T, dA = -dR U^T.
// Every wave needs all of dO, U and dR as A operands: they are split into
// bf16 hi + lo parts once, when staged, and so are dP o M and W, when the
// waves that form them store them.
struct GradLds {
  uint16_t q[kC][kKS], k[kC][kKS];
  union {
    uint16_t in[3][2][kC][kKS];    // dO, U, dR: [array][hi, lo][token][channel]
    uint16_t mid[2][2][kC][kKS];   // dP o M, W: [matrix][hi, lo][i][j], blocks above the diagonal unwritten
  } u;
  float G[kC], gam[kC], dec[kC], bet[kC];
  float part_q[kC][8], part_y[kC][8], part_s[kC][8];
  float part_b[kC][4];
  float dbe[kC];
  float dss[8];
};

// 8 contiguous bf16 of a staged row (one 16-byte read), reduction slot j of
// lane group g4 = channel c0 + j
__device__ __forceinline__ bf16x8v row8c(const uint16_t (*rows)[kKS], int row, int c0) {
  // 24-bit multiply: a 32-bit one is selected as a 64-bit multiply-add whose
  // unused high input may be a register a load in flight still targets
  const uint32_t off = __umul24(static_cast<uint32_t>(row), kKS * 2u) + 2u * static_cast<uint32_t>(c0);
  return __builtin_bit_cast(bf16x8v, *reinterpret_cast<const uint4*>(reinterpret_cast<const char*>(rows) + off));
}
// keep elements 0..3 (reduction slots of the first 16-row block), or 4..7
__device__ __forceinline__ bf16x8v first4(const bf16x8v v) {
  uint4 u = __builtin_bit_cast(uint4, v);
  u.z = u.w = 0u;
  return __builtin_bit_cast(bf16x8v, u);
}
__device__ __forceinline__ bf16x8v last4(const bf16x8v v) {
  uint4 u = __builtin_bit_cast(uint4, v);
  u.x = u.y = 0u;
  return __builtin_bit_cast(bf16x8v, u);
}

__global__ __launch_bounds__(512) void cb_grad_kernel(CbParams p) {
  __shared__ __align__(16) GradLds sm;
  const int slot = blockIdx.x / p.Hk;
  const int kh = blockIdx.x - slot * p.Hk;
  SlotChunk sc;
  if (!slot_chunk(p, slot, sc)) return;
  if (p.part) {
    // this part's chunks only: from the sequence's mid = nc / 2 on (1), before it (2)
    int s0, s1;
    cb_seq(p, sc.n, s0, s1);
    const int c = (sc.t0 - s0) / kC;
    if ((p.part == 1) != (c >= ((s1 - s0 + kC - 1) / kC) / 2)) return;
  }
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform: scalar branches on it
  const int lane = tid & 63;
  const int m = lane & 15;
  const int g4 = lane >> 4;
  const int d = w * 16 + m;            // this lane's column of the 64 x 128 results

  stage_rows<512>(p.q, p.qs, sc.t0, sc.len, kh, sm.q);
  stage_rows<512>(p.k, p.ks, sc.t0, sc.len, kh, sm.k);
  __syncthreads();
  // dq and dk summed over the value heads in registers
  floatx4 dq_tot[4], dk_tot[4];
#pragma unroll
  for (int tb = 0; tb < 4; ++tb) dq_tot[tb] = dk_tot[tb] = floatx4{0.f, 0.f, 0.f, 0.f};

  for (int hv = 0; hv < p.group; ++hv) {
    // the lane indices again from an opaque copy of the thread id: the address
    // arithmetic of every phase below is then redone per value head rather
    // than hoisted out of the loop, where it would hold registers throughout
    int tid_v = tid;
    asm volatile("" : "+v"(tid_v));
    const int lane = tid_v & 63;
    const int m = lane & 15;
    const int g4 = lane >> 4;
    const int d = w * 16 + m;
    const int h = kh * p.group + hv;
    const int64_t sh = static_cast<int64_t>(slot) * p.Hv + h;
    const float* S0 = p.S0 + sh * (kD * kD) + d;
    const float* dSC = p.dSC + sh * (kD * kD) + d;
    // every load of the value head issued up front, so that their latencies
    // overlap: this thread's dO, U, dR row pieces, the E rows of its dbeta
    // share (rows 8 w .. + 7), and its B operands of the products with S0 and
    // dS_C (rows 32 ks + 8 g4 .. + 7, column d), which arrive while the
    // products of the staged rows alone (dbeta's dR . E, dP and dA) run
    // the gates first: their loads then precede the others, whose waits
    // they do not join
    if (w == 0) {
      const Gates gt = chunk_gates(p, sc.t0, sc.len, h);
      sm.G[lane] = gt.G; sm.gam[lane] = gt.gam; sm.dec[lane] = gt.dec; sm.bet[lane] = gt.bet;
    }
    // thread -> row tid / 8 and channels 32 j + 4 (tid % 8) .. + 3, j = 0..3:
    // the 8 threads of a row read 128 contiguous bytes per load
    const int srow = tid_v >> 3;
    const int sc0 = (tid_v & 7) * 4;
    const bool srow_ok = srow < sc.len;
    float xo[16], xu[16], xr[16];
    {
      const float* so = p.d_o + (static_cast<int64_t>(sc.t0 + min(srow, sc.len - 1)) * p.Hv + h) * kD + sc0;
      const float* su = p.U + (sh * kC + srow) * kD + sc0;
      const float* sr = p.dR + (sh * kC + srow) * kD + sc0;
      // grad_o is only 4-byte aligned; rows past the chunk's end read the last
      // row (in bounds) and are zeroed after the load
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) xo[4 * j + e] = so[32 * j + e];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const floatx4 a = *reinterpret_cast<const floatx4*>(su + 32 * j);
        const floatx4 b = *reinterpret_cast<const floatx4*>(sr + 32 * j);
#pragma unroll
        for (int e = 0; e < 4; ++e) { xu[4 * j + e] = a[e]; xr[4 * j + e] = b[e]; }
      }
    }
    // (the scheduler may not move work across these points: every load is
    // issued, in this order, before any of them is waited for)
    __builtin_amdgcn_sched_barrier(0);
    float e0[8], e1[8];
    {
      const float* Eh = p.E + (sh * kC + 8 * w) * kD + lane;
#pragma unroll
      for (int rr = 0; rr < 8; ++rr) {
        e0[rr] = Eh[rr * kD];
        e1[rr] = Eh[rr * kD + 64];
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    float b1[4][8], b2[4][8];
#pragma unroll
    for (int ks = 0; ks < kD / 32; ++ks)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        b1[ks][j] = S0[(32 * ks + 8 * g4 + j) * kD];
        b2[ks][j] = dSC[(32 * ks + 8 * g4 + j) * kD];
      }
    __builtin_amdgcn_sched_barrier(0);
    {  // split and stage
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        float x = xo[j];
        asm volatile("" : "+v"(x));   // the load stays unconditional
        xo[j] = srow_ok ? x : 0.f;
      }
      const float* src[3] = {xo, xu, xr};
#pragma unroll
      for (int a = 0; a < 3; ++a)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float* x = src[a] + 4 * j;
          const uint32_t h0 = pk_bf16(x[0], x[1]), h1 = pk_bf16(x[2], x[3]);
          const uint32_t l0 = pk_bf16(x[0] - __uint_as_float(h0 << 16), x[1] - __uint_as_float(h0 & 0xffff0000u));
          const uint32_t l1 = pk_bf16(x[2] - __uint_as_float(h1 << 16), x[3] - __uint_as_float(h1 & 0xffff0000u));
          *reinterpret_cast<uint2*>(&sm.u.in[a][0][srow][sc0 + 32 * j]) = make_uint2(h0, h1);
          *reinterpret_cast<uint2*>(&sm.u.in[a][1][srow][sc0 + 32 * j]) = make_uint2(l0, l1);
        }
    }
    __syncthreads();

    // dbeta's first part: dR_i . E_i, rows 8 w .. 8 w + 7 (dR as hi + lo)
#pragma unroll
    for (int rr = 0; rr < 8; ++rr) {
      const int i = 8 * w + rr;
      const float r0 = bf(sm.u.in[2][0][i][lane]) + bf(sm.u.in[2][1][i][lane]);
      const float r1 = bf(sm.u.in[2][0][i][lane + 64]) + bf(sm.u.in[2][1][i][lane + 64]);
      const float x = wave_sum(r0 * e0[rr] + r1 * e1[rr]);
      if (lane == 0) sm.dbe[i] = x;
    }
    // dP o M and W = b o dA o M on and below the diagonal: wave w takes the
    // 16 x 16 blocks w and w + 8 of the ten (both products share U^T), held in
    // registers until the staged rows are no longer read
    floatx4 resP[2], resW[2];
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      const int b = w + 8 * s2;
      resP[s2] = resW[s2] = floatx4{0.f, 0.f, 0.f, 0.f};
      if (b >= 10) break;
      const int ib = b < 1 ? 0 : b < 3 ? 1 : b < 6 ? 2 : 3;
      const int jb = b - ib * (ib + 1) / 2;
      floatx4 accP = {0.f, 0.f, 0.f, 0.f}, accA = {0.f, 0.f, 0.f, 0.f};
      // split-bf16 over 32 value channels a step (channels 32 ks + 8 g4 + e)
#pragma unroll
      for (int ks = 0; ks < kD / 32; ++ks) {
        const int c0 = 32 * ks + 8 * g4;
        const bf16x8v bh = row8c(sm.u.in[1][0], jb * 16 + m, c0), bl = row8c(sm.u.in[1][1], jb * 16 + m, c0);
        accP = mfma_split(row8c(sm.u.in[0][0], ib * 16 + m, c0), row8c(sm.u.in[0][1], ib * 16 + m, c0), bh, bl, accP);
        accA = mfma_split(row8c(sm.u.in[2][0], ib * 16 + m, c0), row8c(sm.u.in[2][1], ib * 16 + m, c0), bh, bl, accA);
      }
      // the block of K K^T (bf16 operands as they stand: exact products)
      floatx4 kkt = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kp = 0; kp < kD / 32; ++kp)
        kkt = mfma_bf(row8(sm.k, ib * 16 + m, 32 * kp, g4), row8(sm.k, jb * 16 + m, 32 * kp, g4), kkt);
      const int j = jb * 16 + m;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = ib * 16 + 4 * g4 + r;
        const float Mij = j <= i ? expf(sm.G[i] - sm.G[j]) : 0.f;
        const float dA = j < i ? -accA[r] : 0.f;
        resP[s2][r] = p.scale * accP[r] * Mij;
        resW[s2][r] = sm.bet[i] * dA * Mij;
        const float pb = sum16(dA * Mij * kkt[r]);
        if (m == 0) sm.part_b[i][jb] = pb;
      }
    }
    // (kept after the products above: they need none of the loads below)
    __builtin_amdgcn_sched_barrier(0);
    // products with S0 and dS_C (B operands straight from the workspace):
    //   dq_h  = (scale gamma dO) S0,  X1 = (-gamma b dR) S0,  dKS = (D U) dS_C
    floatx4 dqh[4], x1[4], dks[4];
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) dqh[tb] = x1[tb] = dks[tb] = floatx4{0.f, 0.f, 0.f, 0.f};
    float dss = 0.f;
    // split-bf16 products over k-steps of 32 value channels: lane (m, g4)
    // takes channels c = 32 ks + 8 g4 + j.  The per-token scales are applied
    // to the sums afterwards.
#pragma unroll
    for (int ks = 0; ks < kD / 32; ++ks) {
#pragma unroll
      for (int j = 0; j < 8; ++j) dss = fmaf(b1[ks][j], b2[ks][j], dss);
      bf16x8v b1h, b1l, b2h, b2l;
      split8(b1[ks], b1h, b1l);
      split8(b2[ks], b2h, b2l);
      const int c0 = 32 * ks + 8 * g4;
#pragma unroll
      for (int tb = 0; tb < 4; ++tb) {
        const int i = tb * 16 + m;
        dqh[tb] = mfma_split(row8c(sm.u.in[0][0], i, c0), row8c(sm.u.in[0][1], i, c0), b1h, b1l, dqh[tb]);
        x1[tb] = mfma_split(row8c(sm.u.in[2][0], i, c0), row8c(sm.u.in[2][1], i, c0), b1h, b1l, x1[tb]);
        dks[tb] = mfma_split(row8c(sm.u.in[1][0], i, c0), row8c(sm.u.in[1][1], i, c0), b2h, b2l, dks[tb]);
      }
    }
#pragma unroll
    for (int tb = 0; tb < 4; ++tb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = tb * 16 + 4 * g4 + r;
        dqh[tb][r] *= p.scale * sm.gam[i];
        x1[tb][r] *= -sm.gam[i] * sm.bet[i];
        dks[tb][r] *= sm.dec[i];
      }
    dss = wave_sum(dss);
    if (lane == 0) sm.dss[w] = dss;
    // k . dKS per token now, and dKS into dk: it is not needed again
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = tb * 16 + 4 * g4 + r;
        const float ps = sum16(bf(sm.k[i][d]) * dks[tb][r]);
        if (m == 0) sm.part_s[i][w] = ps;
      }
      dk_tot[tb] += dks[tb];
    }
    __syncthreads();   // staged rows no longer read: their space takes dP o M and W

#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      const int b = w + 8 * s2;
      if (b >= 10) break;
      const int ib = b < 1 ? 0 : b < 3 ? 1 : b < 6 ? 2 : 3;
      const int jb = b - ib * (ib + 1) / 2;
#pragma unroll
      for (int r = 0; r < 4; r += 2) {
        const int i = ib * 16 + 4 * g4 + r, j = jb * 16 + m;
        const uint32_t ph = pk_bf16(resP[s2][r], resP[s2][r + 1]);
        const uint32_t pl = pk_bf16(resP[s2][r] - __uint_as_float(ph << 16),
                                    resP[s2][r + 1] - __uint_as_float(ph & 0xffff0000u));
        const uint32_t wh = pk_bf16(resW[s2][r], resW[s2][r + 1]);
        const uint32_t wl = pk_bf16(resW[s2][r] - __uint_as_float(wh << 16),
                                    resW[s2][r + 1] - __uint_as_float(wh & 0xffff0000u));
        sm.u.mid[0][0][i][j] = static_cast<uint16_t>(ph); sm.u.mid[0][0][i + 1][j] = static_cast<uint16_t>(ph >> 16);
        sm.u.mid[0][1][i][j] = static_cast<uint16_t>(pl); sm.u.mid[0][1][i + 1][j] = static_cast<uint16_t>(pl >> 16);
        sm.u.mid[1][0][i][j] = static_cast<uint16_t>(wh); sm.u.mid[1][0][i + 1][j] = static_cast<uint16_t>(wh >> 16);
        sm.u.mid[1][1][i][j] = static_cast<uint16_t>(wl); sm.u.mid[1][1][i + 1][j] = static_cast<uint16_t>(wl >> 16);
      }
    }
    __syncthreads();

    // per token block: dq_h += (dP o M) K;  X1 += W K;  X2 = W^T K + (dP o M)^T Q;
    // then the block's dot products for dG (q . dq_h, k . (X1 - X2); k . dKS is
    // subtracted in the sum below) and its share of dq, dk
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) {
      floatx4 x2 = {0.f, 0.f, 0.f, 0.f};
      const int i = tb * 16 + m;
      // reduction over tokens 32 kp + kappa(lane / 16, e) (two 16-token
      // blocks a step), every operand bf16 (K, Q as they stand; dP o M and W
      // as hi + lo): the half of a step outside the blocks a product covers
      // (left unwritten in LDS) enters as zeros
#pragma unroll
      for (int kp = 0; 2 * kp <= tb; ++kp) {             // blocks 0 .. tb
        const bool upper_half = 2 * kp + 1 <= tb;
        const bf16x8v kt = col8(sm.k, 32 * kp, w * 16);
        bf16x8v ph = row8(sm.u.mid[0][0], i, 32 * kp, g4), pl = row8(sm.u.mid[0][1], i, 32 * kp, g4);
        bf16x8v wh = row8(sm.u.mid[1][0], i, 32 * kp, g4), wl = row8(sm.u.mid[1][1], i, 32 * kp, g4);
        if (!upper_half) { ph = first4(ph); pl = first4(pl); wh = first4(wh); wl = first4(wl); }
        dqh[tb] = mfma_bf(ph, kt, dqh[tb]);
        dqh[tb] = mfma_bf(pl, kt, dqh[tb]);
        x1[tb] = mfma_bf(wh, kt, x1[tb]);
        x1[tb] = mfma_bf(wl, kt, x1[tb]);
      }
#pragma unroll
      for (int kp = tb / 2; kp < 2; ++kp) {              // blocks tb .. 3
        const bool lower_half = 2 * kp >= tb;
        const bf16x8v kt = col8(sm.k, 32 * kp, w * 16);
        const bf16x8v qt = col8(sm.q, 32 * kp, w * 16);
        bf16x8v wh = col8(sm.u.mid[1][0], 32 * kp, tb * 16), wl = col8(sm.u.mid[1][1], 32 * kp, tb * 16);
        bf16x8v ph = col8(sm.u.mid[0][0], 32 * kp, tb * 16), pl = col8(sm.u.mid[0][1], 32 * kp, tb * 16);
        if (!lower_half) { ph = last4(ph); pl = last4(pl); wh = last4(wh); wl = last4(wl); }
        x2 = mfma_bf(wh, kt, x2);
        x2 = mfma_bf(wl, kt, x2);
        x2 = mfma_bf(ph, qt, x2);
        x2 = mfma_bf(pl, qt, x2);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = tb * 16 + 4 * g4 + r;
        const float pq = sum16(bf(sm.q[t][d]) * dqh[tb][r]);
        const float py = sum16(bf(sm.k[t][d]) * (x1[tb][r] - x2[r]));
        if (m == 0) { sm.part_q[t][w] = pq; sm.part_y[t][w] = py; }
      }
      dq_tot[tb] += dqh[tb];
      dk_tot[tb] += x1[tb] + x2;
    }
    __syncthreads();

    if (w == 0) {
      const int i = lane;
      float dG = 0.f, ks = 0.f, dssT = 0.f;
#pragma unroll
      for (int ww = 0; ww < 8; ++ww) {
        dG += sm.part_q[i][ww] + sm.part_y[i][ww] - sm.part_s[i][ww];
        ks += sm.part_s[i][ww];
        dssT += sm.dss[ww];
      }
      ks = wave_sum(ks);
      if (i == kC - 1) dG += sm.gam[kC - 1] * dssT + ks;
      // dg_i = sum over i' >= i of dG_i'
      const float tot = wave_sum(dG);
      const float dg = tot - wave_prefix_sum(dG) + dG;
      float db = sm.dbe[i];
      for (int jb = 0; jb <= (i >> 4); ++jb) db += sm.part_b[i][jb];
      if (i < sc.len) {
        const int64_t o = static_cast<int64_t>(sc.t0 + i) * p.Hv + h;
        p.dg[o] = dg;
        p.dbeta[o] = db;
      }
    }
    __syncthreads();   // before the next value head's staging
  }

#pragma unroll
  for (int tb = 0; tb < 4; ++tb)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = tb * 16 + 4 * g4 + r;
      if (i < sc.len) {
        const int64_t o = (static_cast<int64_t>(sc.t0 + i) * p.Hk + kh) * kD + d;
        p.dq[o] = dq_tot[tb][r];
        p.dk[o] = dk_tot[tb][r];
      }
    }
}

}  // namespace

size_t chunked_backward_workspace_bytes(int n_seqs, int T_total, int Hv) {
  const size_t slots = static_cast<size_t>(T_total) / kC + static_cast<size_t>(n_seqs);
  auto up = [](size_t b) { return (b + 255) & ~static_cast<size_t>(255); };
  const size_t sh = slots * static_cast<size_t>(Hv);
  return up(slots * 4) + up(sh * kC * kC * 4) + 2 * up(sh * kD * kD * 4) + 3 * up(sh * kC * kD * 4);
}

hipError_t launch_backward_chunked(const uint16_t* q, int64_t qs, const uint16_t* k, int64_t ks,
                                   const uint16_t* v, int64_t vs, const float* g, const float* beta,
                                   const float* h0, const float* d_o, const float* dhT,
                                   const int32_t* cu, int n_seqs, int T_total, int Hk, int Hv,
                                   float scale, float* dq, float* dk, float* dv, float* dg,
                                   float* dbeta, float* dh0, void* workspace, hipStream_t stream) {
  if (n_seqs == 0) return hipSuccess;
  CbParams p;
  p.q = q; p.k = k; p.v = v; p.qs = qs; p.ks = ks; p.vs = vs; p.g = g; p.beta = beta;
  p.h0 = h0; p.d_o = d_o; p.dhT = dhT; p.cu = cu;
  p.n_seqs = n_seqs; p.seq_len = cu ? 0 : T_total / n_seqs; p.Hk = Hk; p.Hv = Hv;
  p.group = Hv / Hk; p.scale = scale;
  const int n_slots = T_total / kC + n_seqs;
  p.n_slots = n_slots;
  auto up = [](size_t b) { return (b + 255) & ~static_cast<size_t>(255); };
  const size_t sh = static_cast<size_t>(n_slots) * Hv;
  unsigned char* base = static_cast<unsigned char*>(workspace);
  p.slot_seq = reinterpret_cast<int32_t*>(base); base += up(static_cast<size_t>(n_slots) * 4);
  p.X = reinterpret_cast<float*>(base); base += up(sh * kC * kC * 4);
  p.S0 = reinterpret_cast<float*>(base); base += up(sh * kD * kD * 4);
  p.dSC = reinterpret_cast<float*>(base); base += up(sh * kD * kD * 4);
  p.U = reinterpret_cast<float*>(base); base += up(sh * kC * kD * 4);
  p.E = reinterpret_cast<float*>(base); base += up(sh * kC * kD * 4);
  p.dR = reinterpret_cast<float*>(base);
  p.dq = dq; p.dk = dk; p.dv = dv; p.dg = dg; p.dbeta = dbeta; p.dh0 = dh0;
  p.part = 0;

  const unsigned chains = static_cast<unsigned>(n_seqs) * static_cast<unsigned>(Hv) * 2u;
  const bool chains_fit = 4 * n_seqs * Hv <= compute_units();
  const size_t pad = chains_fit ? kChainPad : 0;
  if (T_total > 0) {
    hipLaunchKernelGGL(cb_fill_kernel, dim3((n_slots + 255) / 256), dim3(256), 0, stream, p.slot_seq, n_slots);
    hipLaunchKernelGGL(cb_table_kernel, dim3((n_seqs + 255) / 256), dim3(256), 0, stream, p);
    const unsigned per_chunk = static_cast<unsigned>(n_slots) * static_cast<unsigned>(Hk);
    hipLaunchKernelGGL(cb_prep_kernel, dim3(per_chunk), dim3(256), 0, stream, p);
    // the gradient chain needs none of the state chain's records: it runs on
    // the library's second stream beside it; the gradient pass waits for both
    Overlap* ov = overlap_of_current_device();
    if (ov) {
      std::lock_guard<std::mutex> lock(ov->mu);
      hipError_t e = hipEventRecord(ov->start, stream);
      if (e == hipSuccess) e = hipStreamWaitEvent(ov->side, ov->start, 0);
      if (e != hipSuccess) return e;
      // Long sequences whose chains leave compute units idle: the gradient
      // chain in two parts, and the gradient pass over the upper half of each
      // sequence's chunks (done by the first part and by the state chain,
      // which ends first) runs beside the second part.
      if (T_total / n_seqs >= 32 * kC && chains_fit) {
        CbParams ph = p, pl = p;
        ph.part = 1;
        pl.part = 2;
        hipLaunchKernelGGL(cb_bwd_kernel, dim3(chains), dim3(256), pad, ov->side, ph);
        e = hipGetLastError();
        if (e == hipSuccess) e = hipEventRecord(ov->done[0], ov->side);
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(cb_bwd_kernel, dim3(chains), dim3(256), pad, ov->side, pl);
        e = hipGetLastError();
        if (e == hipSuccess) e = hipEventRecord(ov->done[1], ov->side);
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(cb_fwd_kernel, dim3(chains), dim3(256), pad, stream, p);
        e = hipGetLastError();
        if (e == hipSuccess) e = hipStreamWaitEvent(stream, ov->done[0], 0);
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(cb_grad_kernel, dim3(per_chunk), dim3(512), 0, stream, ph);
        e = hipGetLastError();
        if (e == hipSuccess) e = hipStreamWaitEvent(stream, ov->done[1], 0);
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(cb_grad_kernel, dim3(per_chunk), dim3(512), 0, stream, pl);
        return hipGetLastError();
      }
      hipLaunchKernelGGL(cb_bwd_kernel, dim3(chains), dim3(256), pad, ov->side, p);
      hipLaunchKernelGGL(cb_fwd_kernel, dim3(chains), dim3(256), pad, stream, p);
      e = hipGetLastError();
      if (e == hipSuccess) e = hipEventRecord(ov->done[0], ov->side);
      if (e == hipSuccess) e = hipStreamWaitEvent(stream, ov->done[0], 0);
      if (e != hipSuccess) return e;
    } else {
      hipLaunchKernelGGL(cb_fwd_kernel, dim3(chains), dim3(256), pad, stream, p);
      hipLaunchKernelGGL(cb_bwd_kernel, dim3(chains), dim3(256), pad, stream, p);
    }
    hipLaunchKernelGGL(cb_grad_kernel, dim3(per_chunk), dim3(512), 0, stream, p);
  } else if (dh0) {
    hipLaunchKernelGGL(cb_bwd_kernel, dim3(chains), dim3(256), pad, stream, p);
  }
  return hipGetLastError();
}

}  // namespace gdn
