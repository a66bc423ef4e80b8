// chunk.hip -- chunked prefill of the gated delta rule on gfx950.
//
// The rule (the "Delta-rule layers" row of the model card's Architecture
// table: 16 key heads shared by 48 value heads, head dim 128, fp32 state),
// per value head with S the dv x dk state:
//     S_t = S_{t-1} a_t (I - b_t k_t k_t^T) + b_t v_t k_t^T,  o_t = scale S_t q_t
// is computed exactly (up to rounding) in chunks of 64 tokens with the WY / UT
// form.  Inside a chunk with G = inclusive cumsum of g, gamma = exp(G),
// E_ij = exp(G_i - G_j), and S0 the state entering the chunk:
//     A   = strict_lower(diag(b) E * K K^T)
//     U   = (I + A)^-1 (diag(b) V - diag(b gamma) K S0^T)
//     O   = scale (diag(gamma) Q S0^T + lower(E * Q K^T) U)
//     S_L = gamma_L S0 + U^T diag(exp(G_L - G)) K
// (unroll S_i = a_i S_{i-1} + u_i k_i^T with u_i = b_i (v_i - a_i S_{i-1} k_i)
// inside the chunk; every exponent used is <= 0 for g <= 0).
//
// Two kernels, run back to back on the caller's stream:
//
//   prep (fully parallel over every chunk x key head): everything that does not
//   depend on the state.  K and Q are converted to fp16 once (K as rows, Q in
//   MFMA fragment order); the 20 lower 16x16 tiles of K K^T and Q K^T are
//   formed once per key head on fp16 MFMA (exact products of bf16 inputs); for
//   each of the key head's value heads the decay tables, -A, the inverses
//   T_bb = (I + A_bb)^-1 of the four diagonal 16x16 blocks (fp32 forward
//   substitution) and P = scale E * Q K^T are written, also in fragment order.
//   Chunks come from the varlen chunk table, so they restart at every sequence
//   start.
//
//   scan (one work-group per sequence x value head x quarter of the value
//   channels): the sequential part.  A state wave carries the 32 x 128 slice
//   of S^T for the work-group's 32 value channels in registers across all
//   chunks and per chunk runs W = K S0^T (B operand straight from the S^T
//   registers), R = b V - b gamma W, U by blockwise forward substitution
//   (U_i = T_ii (R_i - sum_{j<i} A_ij U_j)) and S^T <- gamma_L S^T + K^T (D U),
//   in phases that each issue the LDS reads of the next phase.  It leaves the
//   fp16 S0 and U in LDS; an output wave forms O = scale (gamma Q S0^T + P U)
//   from them a chunk later and stores it.  Two loader waves copy the next
//   chunk's fragments and V tile into LDS (global_load_lds, one chunk ahead),
//   so the state wave never issues a global memory instruction inside the loop.
//
// Only the fp32-valued operands are rounded to fp16 (S0, U, T_ii, A, P);
// accumulation is fp32 throughout.  The per-chunk state never leaves the
// registers, and fragment reads are lane-contiguous 16-byte LDS loads.
// Work-groups that share a key head get block ids on the same XCD (L2).
#include <algorithm>
#include <atomic>
#include <mutex>
#include <type_traits>

#include "common.h"
#include "launch.h"

namespace gdn {

namespace {

constexpr int kC = 64;            // chunk length
constexpr int kD = 128;           // head dim (dk = dv)
constexpr int kThreads = 256;    // prep work-group
// Scan work-group (kTiles 16-channel tiles of one value head: 32 or 64 value
// channels): state waves, output waves, and two loader waves that copy the
// next chunk into LDS.
constexpr int kScanLoaderWaves = 2;
constexpr int kLoaderThreads = 64 * kScanLoaderWaves;
template <int kOutWaves, int kStateWaves>
constexpr int scan_threads(bool conv = false) {   // conv: two conv waves too
  return 64 * (kStateWaves + kOutWaves + kScanLoaderWaves + (conv ? 2 : 0));
}

// ---- fragment layout in the workspace -------------------------------------
// An A32 fragment of a 16 x 32 block holds, for lane l (row l % 16, group
// g = l / 16), the 8 halves at columns kappa(g, e) (see common.h): 16 bytes per
// lane, lanes in order, 1 KB.  An A16 fragment (16 x 16) holds 4 halves at
// columns 4g .. 4g+3: 8 bytes per lane, 512 B.
constexpr int kFrag = 1024;
constexpr int kFrag16 = 512;
// Per (chunk, key head): K as fp16 rows (row = token, 272 bytes: the padding
// spreads the rows over the LDS banks), then the 16 Q fragments (tb*4+kb).
// Within each 32-column block of a row the eight runs of four columns are
// stored in the order 0 4 1 5 2 6 3 7, so that the 16 bytes at block offset
// 16 m are the columns kappa(m, 0..7): a K fragment is one 16-byte LDS load
// per lane, and K^T fragments come from gfx950's transposing LDS load over the
// rows (any order of the four-column runs works for it).
constexpr int kKRowBytes = 272;
constexpr int kOffQ = kC * kKRowBytes;                // 17408
constexpr int kKQBytes = kOffQ + 16 * kFrag;          // 33792
// Per (chunk, value head):
constexpr int kOffP = 0;                              // 6 A32: (0,0)(1,0)(2,0)(2,1)(3,0)(3,1)
constexpr int kOffT = kOffP + 6 * kFrag;              // 4 A16: T_bb
constexpr int kOffAn10 = kOffT + 4 * kFrag16;         // A16: -A rows 16..31, cols 0..15
constexpr int kOffAn2 = kOffAn10 + kFrag16;           // A32: -A rows 32..47, cols 0..31
constexpr int kOffAn3 = kOffAn2 + kFrag;              // A32: -A rows 48..63, cols 0..31
constexpr int kOffAn32 = kOffAn3 + kFrag;             // A16: -A rows 48..63, cols 32..47
constexpr int kOffDecay = kOffAn32 + kFrag16;         // 4 x 64 floats: b, b gamma, scale gamma, exp(G_L - G)
constexpr int kOffGL = kOffDecay + 4 * 256;           // gamma_L
constexpr int kVBytes = kOffGL + 256;                 // 12544
// Per chunk the scan stages what the state waves read in LDS: [K rows |
// value-head blob from T_bb on | V tile], where the V tile is this
// work-group's value channels of the chunk's 64 tokens, row-major bf16
// (2 kDv bytes per token).  The output waves load their Q and P fragments
// from global memory into registers.
constexpr int kVBStaged = kVBytes - kOffT;                                      // 6400
constexpr int kStageVB = kOffQ;                                                 // 17408
constexpr int kStageV = kStageVB + kVBStaged;                                   // 23808
constexpr int kKPieces = kOffQ / 16;                                            // 1088
constexpr int kVBPieces = kVBStaged / 16;                                       // 400
// Per chunk the state waves leave the fp16 S0 (as B operands, tile t, block
// kb at fragment 4 t + kb) and U (fragments kU0 + 2 t, kU0 + 1 + 2 t) for the
// output waves.
template <int kTiles>
struct ScanShape {
  static constexpr int kDv = 16 * kTiles;                         // value channels per work-group
  static constexpr int kParts = kD / kDv;                         // work-groups per value head
  static constexpr int kVTileBytes = kC * kDv * 2;                // 4096 / 8192
  static constexpr int kStageBytes = kStageV + kVTileBytes;       // 27904 / 32000
  static constexpr int kStagePieces = kStageBytes / 16;
  static constexpr int kStageRounds = (kStagePieces + kLoaderThreads - 1) / kLoaderThreads;
  static constexpr int kVPiecesPerRow = kDv / 8;
  static constexpr int kU0 = 4 * kTiles;
  static constexpr int kXBytes = 6 * kTiles * kFrag;              // 12 / 24 KB
  // conv front (kConvV): each loader wave copies the pre-conv rows of its
  // half of the chunk, 3 rows of history first, and a conv wave forms that
  // half of the V tile from them
  static constexpr int kRawRows = kC / 2 + 3;                     // 35
  static constexpr int kRawBytes = kRawRows * kDv * 2;            // 2240 / 4480
  static constexpr int kRawPieces = kRawBytes / 16;
  static constexpr int kRawRounds = (kRawPieces + 63) / 64;
  static constexpr int kConvTok = kDv / 16;                       // tokens per loader lane
  static constexpr int kKVBRounds = (kKPieces + kVBPieces + kLoaderThreads - 1) / kLoaderThreads;
  static_assert(kStagePieces == kKPieces + kVBPieces + kVTileBytes / 16, "stage = K rows + value blob + V tile");
  static_assert(kStageBytes % 16 == 0, "stage size");
};

// The overlapped prefill: segments of kSegChunks chunks for sequences of at
// least kSegMinChunks chunks, when the scan leaves kSegMinIdleCUs or more
// compute units idle.  kScanLdsPad (kScanLdsPad4) bytes of LDS added to each
// 32-channel (64-channel) scan work-group leave its compute unit too little
// for a prep work-group, so the preps run on the idle units and take nothing
// from the scan's memory pipe.
constexpr int kSegChunks = 256;
constexpr int kSegMinChunks = 2 * kSegChunks;
constexpr int kSegMinIdleCUs = 32;
constexpr int kScanLdsPad = 48 * 1024;      // beside the 32-channel form
constexpr int kScanLdsPad4 = 16 * 1024;     // beside the 64-channel form
static_assert(kOffT % 16 == 0 && kOffQ % 16 == 0, "staged parts are whole pieces");

// ---- prep kernel LDS -------------------------------------------------------
constexpr int kKS = kD + 8;       // K, Q rows (halves)
constexpr int kTS = 16 + 8;       // T_bb rows (halves)
constexpr int kHeadBatch = 3;     // value heads prepared together

// K and Q are only needed until the K rows, Q fragments and Gram tiles are
// formed; their space is then reused for the diagonal blocks of A and the
// inverses T_bb of a batch of up to kHeadBatch value heads.
struct PrepKQ {
  _Float16 K[kC * kKS];
  _Float16 Q[kC * kKS];
};
struct PrepHeads {
  float Ad[kHeadBatch][4 * 16 * 16];
  _Float16 T[kHeadBatch][4 * 16 * kTS];
};
struct __align__(16) PrepSmem {
  union {
    PrepKQ kq;
    PrepHeads vh;
  } u;
  float G[kHeadBatch][kC];
  float bet[kHeadBatch][kC];
};

typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
typedef float float2v __attribute__((ext_vector_type(2)));
// two floats to packed bf16, round to nearest even (v_cvt_pk_bf16_f32)
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(float2v{a, b}, bf16x2v));
}

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

struct PrepParams {
  const uint16_t* q; const uint16_t* k;
  int64_t qs, ks;
  const float* g; const float* beta;
  // gates from the per-head projections instead of g, beta (when ga != nullptr):
  // g = -exp(A_log) softplus(a + dt_bias), beta = sigmoid(b)
  const uint16_t* ga; const uint16_t* gb;
  int64_t gas, gbs;
  const float* A_log; const float* dt_bias;
  // conv front (kConv): q and k come from the causal conv + SiLU + L2 of the
  // pre-conv rows x [T, C] (v is formed by the scan kernel from the same rows)
  const uint16_t* x; int64_t xs;
  const uint16_t* conv_w; const float* conv_bias; const uint16_t* conv_state;
  const int32_t* conv_slots;  // nullptr: sequence n uses conv_state row n
  int conv_n_slots;           // rows of the conv-state pool (with conv_slots)
  float l2_eps;
  const int32_t* cu;          // nullptr: equal lengths seq_len
  const int32_t* chunk_off;   // varlen chunk map (device)
  const int32_t* chunk_tab;
  unsigned char* kq;          // [max_chunks][Hk][kKQBytes]
  unsigned char* vb;          // [max_chunks][Hv][kVBytes]
  int n_seqs, seq_len, Hk, Hv, group;
  // equal lengths: this launch prepares chunks seg_c0 .. seg_c0 + seg_nc - 1
  // of every sequence (seg_nc = 0: all of them)
  int seg_c0, seg_nc;
  float scale;
};

__device__ __forceinline__ half8 lds_a32(const _Float16* base, int stride, int row, int kb,
                                         int grp) {
  const _Float16* p = base + row * stride + kb + 4 * grp;
  return cat8(*reinterpret_cast<const half4*>(p), *reinterpret_cast<const half4*>(p + 16));
}

__device__ __forceinline__ half4 lds_a16(const _Float16* base, int stride, int row, int kb,
                                         int grp) {
  return *reinterpret_cast<const half4*>(base + row * stride + kb + 4 * grp);
}

// Workspace writes of the prep are streamed past the caches (nontemporal): the
// scan reads them long after they would have been evicted, and keeping them
// out of L2 left the prefill launch 2 % faster.
__device__ __forceinline__ void put16(unsigned char* dst, const half8 v) {
  __builtin_nontemporal_store(v, reinterpret_cast<half8*>(dst));
}
__device__ __forceinline__ void put8(unsigned char* dst, const half4 v) {
  __builtin_nontemporal_store(v, reinterpret_cast<half4*>(dst));
}

// Gram tiles of a wave, in the transposed orientation C' = X_j Y_b^T, so
// that lane (col, grp) holds (Y X^T)[16 b + col][16 j + 4 grp + e], e = 0..3:
// the four values an MFMA A-operand fragment (row 16 b + col, columns
// 16 j + 4 grp ..) takes.  Tile k of wave W: Q K^T (isq) or K K^T, block row b,
// block column j.  The waves' lists complete whole fragments:
//   wave 0: P (0,0) (1,0) (1,1) (2,2), A (0,0)
//   wave 1: P (2,0) (2,1) (3,0) (3,1), A (1,1)
//   wave 2: P (3,2) (3,3), A (1,0) (3,2) (2,2)
//   wave 3: A (2,0) (2,1) (3,0) (3,1) (3,3)
struct GramTile { bool isq; int b, j; };
__host__ __device__ constexpr GramTile gram_tile(int W, int k) {
  constexpr GramTile t[4][5] = {
      {{true, 0, 0}, {true, 1, 0}, {true, 1, 1}, {true, 2, 2}, {false, 0, 0}},
      {{true, 2, 0}, {true, 2, 1}, {true, 3, 0}, {true, 3, 1}, {false, 1, 1}},
      {{true, 3, 2}, {true, 3, 3}, {false, 1, 0}, {false, 3, 2}, {false, 2, 2}},
      {{false, 2, 0}, {false, 2, 1}, {false, 3, 0}, {false, 3, 1}, {false, 3, 3}}};
  return t[W][k];
}

// Wave W's share of the elementwise step, for head vh of the batch (G, bet in
// LDS), with E_il = exp(G_i - G_l), i = 16 b + col, l = 16 j + 4 grp + e:
//   Q K^T:                  P  = scale * lower(E * Q K^T)  -> P fragments (global)
//   K K^T, off-diagonal:   -A  = -(b E * K K^T)            -> -A fragments (global)
//   K K^T, diagonal:        A  = strict_lower(b E * K K^T) -> Ad (fp32, LDS)
// P fragment f covers block row tb, columns 32 kb .. +31: (0,0)(1,0)(2,0)(2,1)(3,0)(3,1).
template <int W>
__device__ __forceinline__ void prep_elementwise(PrepSmem& sm, const floatx4 (&gram)[5], int vh,
                                                 unsigned char* vb, int lane, int col, int grp,
                                                 float scale) {
  half4 v[5];
#pragma unroll
  for (int k = 0; k < 5; ++k) {
    constexpr GramTile dummy = gram_tile(W, 0);
    (void)dummy;
    const GramTile t = gram_tile(W, k);
    const int i = 16 * t.b + col;
    const float Gi = sm.G[vh][i];
    const floatx4 Gl = *reinterpret_cast<const floatx4*>(&sm.G[vh][16 * t.j + 4 * grp]);
    if (t.isq) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float x = scale * __expf(Gi - Gl[e]) * gram[k][e];
        v[k][e] = static_cast<_Float16>((t.b > t.j || 4 * grp + e <= col) ? x : 0.f);
      }
    } else {
      const float bi = sm.bet[vh][i];
      floatx4 a;
#pragma unroll
      for (int e = 0; e < 4; ++e) a[e] = bi * __expf(Gi - Gl[e]) * gram[k][e];
      if (t.b == t.j) {
#pragma unroll
        for (int e = 0; e < 4; ++e) a[e] = (4 * grp + e < col) ? a[e] : 0.f;
        *reinterpret_cast<floatx4*>(&sm.u.vh.Ad[vh][(t.b * 16 + col) * 16 + 4 * grp]) = a;
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) v[k][e] = static_cast<_Float16>(-a[e]);
      }
    }
  }
  const half4 z4 = {0, 0, 0, 0};
  if (W == 0) {
    put16(vb + kOffP + 0 * kFrag + lane * 16, cat8(v[0], z4));
    put16(vb + kOffP + 1 * kFrag + lane * 16, cat8(v[1], v[2]));
    put16(vb + kOffP + 3 * kFrag + lane * 16, cat8(v[3], z4));
  } else if (W == 1) {
    put16(vb + kOffP + 2 * kFrag + lane * 16, cat8(v[0], v[1]));
    put16(vb + kOffP + 4 * kFrag + lane * 16, cat8(v[2], v[3]));
  } else if (W == 2) {
    put16(vb + kOffP + 5 * kFrag + lane * 16, cat8(v[0], v[1]));
    put8(vb + kOffAn10 + lane * 8, v[2]);
    put8(vb + kOffAn32 + lane * 8, v[3]);
  } else {
    put16(vb + kOffAn2 + lane * 16, cat8(v[0], v[1]));
    put16(vb + kOffAn3 + lane * 16, cat8(v[2], v[3]));
  }
}

// x / (1 + e^-x) with the hardware exp2 and reciprocal, as the conv front
// of conv1d.hip computes it
__device__ __forceinline__ float conv_silu(float x) {
  return x * __builtin_amdgcn_rcpf(1.f + __expf(-x));
}

// Conv front of one task: chunk rows r0 .. r0 + 3 of the 8 channels ch0 ..
// ch0 + 7 of x.  y = silu(sum_i w[c][i] x[t - 3 + i][c] + bias[c]), history
// before the sequence start s0 from the conv state of sequence `seq` (oldest
// first) or zero, then, with `l2`, y / sqrt(sum y^2 + eps) over the 128
// channels that the 16 lanes of this DPP row hold.  The operations and their
// order are those of conv1d_kernel, so every value equals the one the
// separate conv call stores (bf16, round to nearest even).
struct ConvRows {
  uint4 raw[7];     // x rows r0 - 3 .. r0 + 3 (zero before s0 and at or past len)
  uint4 wq[4];      // 4 taps of each of the 8 channels
};

__device__ __forceinline__ void conv_rows_load(const PrepParams& p, ConvRows& cr, int ch0, int t0,
                                               int r0, int len, int s0) {
#pragma unroll
  for (int j = 0; j < 7; ++j) {
    const int rr = r0 - 3 + j;
    const int t = t0 + rr;
    cr.raw[j] = (rr < len && t >= s0)
                    ? *reinterpret_cast<const uint4*>(p.x + static_cast<int64_t>(t) * p.xs + ch0)
                    : uint4{0u, 0u, 0u, 0u};
  }
  const uint4* wp = reinterpret_cast<const uint4*>(p.conv_w + static_cast<int64_t>(ch0) * 4);
#pragma unroll
  for (int q = 0; q < 4; ++q) cr.wq[q] = wp[q];
}

__device__ __forceinline__ void conv_rows(const PrepParams& p, const ConvRows& cr, int ch0, int t0,
                                          int r0, int s0, int seq, int C, bool l2,
                                          float (&out)[4][8]) {
  float xin[7][8];
#pragma unroll
  for (int k = 0; k < 7; ++k) bf16x8_to_f32(cr.raw[k], xin[k]);
  const int64_t row = p.conv_slots ? p.conv_slots[seq] : seq;
  // a slot outside the pool reads no history (zeros)
  const bool has_row = !p.conv_slots || static_cast<uint64_t>(row) < static_cast<uint64_t>(p.conv_n_slots);
  if (t0 + r0 - 3 < s0 && p.conv_state && has_row) {
    // Rows before the sequence start: chunks start at s0 + 64 i and tasks at
    // multiples of 4, so this is the sequence's first chunk, r0 = 0, and input
    // rows 0, 1, 2 are the tokens s0 - 3, s0 - 2, s0 - 1: state taps 0, 1, 2.
    float st[24];
    const uint4* sp = reinterpret_cast<const uint4*>(p.conv_state + (row * C + ch0) * 3);
    bf16x8_to_f32(sp[0], st);
    bf16x8_to_f32(sp[1], st + 8);
    bf16x8_to_f32(sp[2], st + 16);
#pragma unroll
    for (int k = 0; k < 3; ++k)
#pragma unroll
      for (int i = 0; i < 8; ++i) xin[k][i] = st[3 * i + k];
  }
  float wt[32];
#pragma unroll
  for (int q = 0; q < 4; ++q) bf16x8_to_f32(cr.wq[q], wt + 8 * q);
  float bias[8];
  if (p.conv_bias) {
    const float4 b0 = *reinterpret_cast<const float4*>(p.conv_bias + ch0);
    const float4 b1 = *reinterpret_cast<const float4*>(p.conv_bias + ch0 + 4);
    bias[0] = b0.x; bias[1] = b0.y; bias[2] = b0.z; bias[3] = b0.w;
    bias[4] = b1.x; bias[5] = b1.y; bias[6] = b1.z; bias[7] = b1.w;
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) bias[i] = 0.f;
  }
#pragma unroll
  for (int jj = 0; jj < 4; ++jj) {
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float acc = fmaf(wt[4 * i], xin[jj][i], bias[i]);
      acc = fmaf(wt[4 * i + 1], xin[jj + 1][i], acc);
      acc = fmaf(wt[4 * i + 2], xin[jj + 2][i], acc);
      acc = fmaf(wt[4 * i + 3], xin[jj + 3][i], acc);
      out[jj][i] = conv_silu(acc);
      ss = fmaf(out[jj][i], out[jj][i], ss);
    }
    if (l2) {
      ss = sum16(ss);
      const float inv = rsqrtf(ss + p.l2_eps);
#pragma unroll
      for (int i = 0; i < 8; ++i) out[jj][i] *= inv;
    }
    // round to bf16 as the stored conv output is
#pragma unroll
    for (int i = 0; i < 8; i += 2) {
      const uint32_t b = pack_bf16x2(out[jj][i], out[jj][i + 1]);
      out[jj][i] = __uint_as_float(b << 16);
      out[jj][i + 1] = __uint_as_float(b & 0xffff0000u);
    }
  }
}

// kGated: the gates come from the projections (p.ga, p.gb, p.A_log, p.dt_bias).
// kConv: q and k come from the conv front over p.x.
template <bool kGated, bool kConv>
__global__ __launch_bounds__(kThreads, 3) void chunk_prep_kernel(PrepParams p) {
  __shared__ PrepSmem sm;
  const int kh = blockIdx.x;
  int c = blockIdx.y;     // chunk (index into the blob arrays)
  int t0, len, seq, s0;
  if (p.cu) {
    if (c >= p.chunk_off[p.n_seqs]) return;
    seq = kConv ? p.chunk_tab[3 * c] : 0;
    t0 = p.chunk_tab[3 * c + 1];
    len = p.chunk_tab[3 * c + 2];
    s0 = kConv ? p.cu[seq] : 0;
  } else {
    const int nc = (p.seq_len + kC - 1) / kC;
    const int snc = p.seg_nc ? p.seg_nc : nc;
    seq = c / snc;
    const int i = p.seg_c0 + (c - seq * snc);
    c = seq * nc + i;
    s0 = seq * p.seq_len;
    t0 = s0 + i * kC;
    len = min(kC, p.seq_len - i * kC);
  }
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
  const int lane = tid & 63;
  const int col = lane & 15;
  const int grp = lane >> 4;

  // g and beta of value head vh, one token per lane
  // The gate inputs of value head vh, lane = token (tokens past the end read
  // the last one): loaded here, turned into g, beta (zero past the end) by
  // finish_gb where they are first needed, since a choice on a freshly
  // loaded value makes the wave wait for it on the spot.
  auto load_gb = [&](int vh, float& gv, float& bv) {
    const int64_t t = t0 + min(lane, len - 1);
    const int h = kh * p.group + vh;
    if (kGated) {
      gv = bf16_to_f32(p.ga[t * p.gas + h]);
      bv = bf16_to_f32(p.gb[t * p.gbs + h]);
    } else {
      gv = p.g[t * p.Hv + h];
      bv = p.beta[t * p.Hv + h];
    }
  };
  auto finish_gb = [&](int vh, float& gv, float& bv) {
    const bool valid = lane < len;
    if (kGated) {
      // softplus(x) = max(x, 0) + log1p(e^-|x|), with the accurate libm forms
      const int h = kh * p.group + vh;
      const float x = gv + p.dt_bias[h];
      const float sp = fmaxf(x, 0.f) + log1pf(expf(-fabsf(x)));
      gv = valid ? -expf(p.A_log[h]) * sp : 0.f;
      bv = valid ? 1.f / (1.f + expf(-bv)) : 0.f;
    } else {
      gv = valid ? gv : 0.f;
      bv = valid ? bv : 0.f;
    }
  };
  // decay tables of value head vb0 + w (wave w, lane = token): G = inclusive
  // cumsum of g, then b, b gamma, scale gamma, exp(G_L - G) and gamma_L
  auto decay = [&](int vb0, float gv, float bv) {
    const int h = kh * p.group + vb0 + w;
    unsigned char* vb = p.vb + (static_cast<int64_t>(c) * p.Hv + h) * kVBytes;
    float G = gv;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const float up = __shfl_up(G, d, 64);
      if (lane >= d) G += up;
    }
    const float Glast = __shfl(G, 63, 64);
    const float gam = __expf(G);
    sm.G[w][lane] = G;
    sm.bet[w][lane] = bv;
    float* dec = reinterpret_cast<float*>(vb + kOffDecay);
    __builtin_nontemporal_store(bv, &dec[lane]);
    __builtin_nontemporal_store(bv * gam, &dec[64 + lane]);
    __builtin_nontemporal_store(p.scale * gam, &dec[128 + lane]);
    __builtin_nontemporal_store(__expf(Glast - G), &dec[192 + lane]);
    if (lane == 0) *reinterpret_cast<float*>(vb + kOffGL) = __expf(Glast);
  };

  // ---- K, Q loads (64 rows x 16 pieces of 8 channels), issued first --------
  float gv = 0.f, bv = 0.f;
  const int nb0 = min(kHeadBatch, p.group);
  if (w < nb0) load_gb(w, gv, bv);
  const int C = (2 * p.Hk + p.Hv) * kD;        // channels of x (kConv)
  const int r0 = (tid >> 4) * 4;                 // kConv task: rows r0 .. r0 + 3
  const int g8 = (tid & 15) * 8;                 //   and channels g8 .. g8 + 7 of a head
  if (kConv) {
    // K then Q: load the task's rows, conv, L2, bf16 rounding, fp16 into LDS
    ConvRows cr;
    conv_rows_load(p, cr, p.Hk * kD + kh * kD + g8, t0, r0, len, s0);
    // the first batch's decay tables while the x loads are in flight
    if (w < nb0) {
      finish_gb(w, gv, bv);
      decay(0, gv, bv);
    }
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      if (m == 1) conv_rows_load(p, cr, kh * kD + g8, t0, r0, len, s0);
      float y[4][8];
      conv_rows(p, cr, m == 0 ? p.Hk * kD + kh * kD + g8 : kh * kD + g8, t0, r0, s0, seq, C, true, y);
      _Float16* dst = m == 0 ? sm.u.kq.K : sm.u.kq.Q;
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int r = r0 + jj;
        half8 hv;
#pragma unroll
        for (int i = 0; i < 8; ++i) hv[i] = static_cast<_Float16>(r < len ? y[jj][i] : 0.f);
        *reinterpret_cast<half8*>(&dst[r * kKS + g8]) = hv;
      }
    }
  } else {
    uint4 kraw[4], qraw[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int piece = tid + kThreads * j;
      const int rr = min(piece >> 4, len - 1);
      const int c8 = (piece & 15) * 8;
      // q and k are read once: streamed (nontemporal)
      const u32x4 kt = __builtin_nontemporal_load(
          reinterpret_cast<const u32x4*>(p.k + static_cast<int64_t>(t0 + rr) * p.ks + kh * kD + c8));
      const u32x4 qt = __builtin_nontemporal_load(
          reinterpret_cast<const u32x4*>(p.q + static_cast<int64_t>(t0 + rr) * p.qs + kh * kD + c8));
      kraw[j] = uint4{kt[0], kt[1], kt[2], kt[3]};
      qraw[j] = uint4{qt[0], qt[1], qt[2], qt[3]};
    }
    // the first batch's decay tables while the K, Q loads are in flight
    if (w < nb0) {
      finish_gb(w, gv, bv);
      decay(0, gv, bv);
    }
    // K, Q -> LDS (fp16), rows past the chunk end zeroed
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int piece = tid + kThreads * j;
      const int r = piece >> 4;
      const int c8 = (piece & 15) * 8;
      float fk[8], fq[8];
      bf16x8_to_f32(kraw[j], fk);
      bf16x8_to_f32(qraw[j], fq);
      half8 hk, hq;
      const bool ok = r < len;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        hk[i] = static_cast<_Float16>(ok ? fk[i] : 0.f);
        hq[i] = static_cast<_Float16>(ok ? fq[i] : 0.f);
      }
      *reinterpret_cast<half8*>(&sm.u.kq.K[r * kKS + c8]) = hk;
      *reinterpret_cast<half8*>(&sm.u.kq.Q[r * kKS + c8]) = hq;
    }
  }
  lds_barrier();

  // ---- K rows and Q fragments (written once per chunk and key head) --------
  unsigned char* kq = p.kq + (static_cast<int64_t>(c) * p.Hk + kh) * kKQBytes;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int piece = tid + kThreads * j;       // 64 rows x 4 blocks x 4 runs of 16 bytes
    const int r = piece >> 4;
    const int kb = (piece >> 2) & 3, m = piece & 3;
    put16(kq + r * kKRowBytes + kb * 64 + m * 16, lds_a32(sm.u.kq.K, kKS, r, 32 * kb, m));
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int f = w * 4 + j;
    put16(kq + kOffQ + f * kFrag + lane * 16,
          lds_a32(sm.u.kq.Q, kKS, 16 * (f >> 2) + col, 32 * (f & 3), grp));
  }

  // ---- this wave's five Gram tiles, transposed orientation ------------------
  floatx4 gram[5];
  auto gram_tiles = [&](auto w_c) {
    constexpr int W = decltype(w_c)::value;
#pragma unroll
    for (int k = 0; k < 5; ++k) {
      const GramTile t = gram_tile(W, k);
      const _Float16* Y = t.isq ? sm.u.kq.Q : sm.u.kq.K;
      floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < kD; kb += 32)
        acc = mfma32(lds_a32(sm.u.kq.K, kKS, 16 * t.j + col, kb, grp), lds_a32(Y, kKS, 16 * t.b + col, kb, grp), acc);
      gram[k] = acc;
    }
  };
  switch (w) {
    case 0: gram_tiles(std::integral_constant<int, 0>{}); break;
    case 1: gram_tiles(std::integral_constant<int, 1>{}); break;
    case 2: gram_tiles(std::integral_constant<int, 2>{}); break;
    default: gram_tiles(std::integral_constant<int, 3>{}); break;
  }
  lds_barrier();   // K and Q are no longer read: their space becomes the heads'

  // ---- the key head's value heads, up to kHeadBatch at a time --------------
  for (int vb0 = 0; vb0 < p.group; vb0 += kHeadBatch) {
    const int nb = min(kHeadBatch, p.group - vb0);
    if (vb0 > 0) {
      if (w < nb) {
        load_gb(vb0 + w, gv, bv);
        finish_gb(vb0 + w, gv, bv);
        decay(vb0, gv, bv);
      }
      lds_barrier();   // G, bet of the batch ready
    }

    // P and -A fragments of every head of the batch from this wave's Gram
    // tiles; A's diagonal blocks to LDS
    for (int vh = 0; vh < nb; ++vh) {
      unsigned char* vb = p.vb + (static_cast<int64_t>(c) * p.Hv + kh * p.group + vb0 + vh) * kVBytes;
      switch (w) {
        case 0: prep_elementwise<0>(sm, gram, vh, vb, lane, col, grp, p.scale); break;
        case 1: prep_elementwise<1>(sm, gram, vh, vb, lane, col, grp, p.scale); break;
        case 2: prep_elementwise<2>(sm, gram, vh, vb, lane, col, grp, p.scale); break;
        default: prep_elementwise<3>(sm, gram, vh, vb, lane, col, grp, p.scale); break;
      }
    }
    lds_barrier();   // A_diag of the batch ready

    if (w < nb) {
      // T_bb = (I + A_bb)^-1 of head vb0 + w by forward substitution: lane =
      // 16 blk + column, all four diagonal blocks at once.  Right-looking:
      // once t_j is known it leaves every later row, each row still
      // subtracting its terms in order j = 0, 1, ...
      const int h = kh * p.group + vb0 + w;
      unsigned char* vb = p.vb + (static_cast<int64_t>(c) * p.Hv + h) * kVBytes;
      const int blk = lane >> 4;
      const float* Ab = sm.u.vh.Ad[w] + blk * 256;
      float tt[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) tt[i] = (i == col) ? 1.f : 0.f;
#pragma unroll
      for (int j = 0; j < 16; ++j)
#pragma unroll
        for (int i = j + 1; i < 16; ++i) tt[i] = fmaf(-Ab[i * 16 + j], tt[j], tt[i]);
      _Float16* Tw = sm.u.vh.T[w];
#pragma unroll
      for (int i = 0; i < 16; ++i) Tw[(blk * 16 + i) * kTS + col] = static_cast<_Float16>(tt[i]);
      // T fragments (same-wave LDS write then read: in order within the wave)
#pragma unroll
      for (int bb = 0; bb < 4; ++bb) put8(vb + kOffT + bb * kFrag16 + lane * 8, lds_a16(Tw, kTS, bb * 16 + col, 0, grp));
    }
    if (vb0 + kHeadBatch < p.group) lds_barrier();   // before the next batch overwrites
  }
}

// ---- scan kernel ------------------------------------------------------------

struct ScanParams {
  const uint16_t* v;
  int64_t vs;
  void* o;                    // fp32, or bf16 when o_bf16
  int o_bf16;
  const float* h0; float* hT;
  const int32_t* slots;       // nullptr: sequence n uses state n of h0 / hT
  int n_slots;                // states in the pool (with slots)
  const int32_t* cu;          // nullptr: equal lengths seq_len
  const int32_t* order;       // longest-first schedule (varlen)
  const int32_t* chunk_off;   // first chunk of each sequence (varlen)
  const unsigned char* kq;
  const unsigned char* vb;
  int n_seqs, seq_len, Hk, Hv, group;
  int n_chain_groups;         // n_seqs * Hk
  // equal lengths: this launch runs chunks c_base .. c_base + c_count - 1 of
  // every sequence, from state h0 to state hT (c_base = 0 and c_count >= the
  // chunks of a sequence: all of it)
  int c_base, c_count;
  // conv front (kConvV): v = silu(causal conv of the pre-conv rows), with v
  // pointing at the first v column of x and vs its row stride; conv_w [C, 4]
  // bf16 and conv_bias [C] (or nullptr) of the C = conv_C channels of x,
  // whose value channels start at conv_v0; history before a sequence from
  // conv_state [rows, C, 3] (row conv_slots[n], or n) or zeros
  const uint16_t* conv_w; const float* conv_bias; const uint16_t* conv_state;
  const int32_t* conv_slots;
  int conv_n_slots, conv_C, conv_v0;
};

// Two stage buffers (the chunk being computed, the one being copied in) and
// two sets of the S0 / U fragments passed from the state wave to the output
// wave.
template <int kTiles, bool kConvV>
struct __align__(16) ScanSmem {
  unsigned char buf[2][ScanShape<kTiles>::kStageBytes];
  unsigned char xbuf[2][ScanShape<kTiles>::kXBytes];
};
// with the conv front also the pre-conv rows, [chunk parity][loader wave]
template <int kTiles>
struct __align__(16) ScanSmem<kTiles, true> {
  unsigned char buf[2][ScanShape<kTiles>::kStageBytes];
  unsigned char xbuf[2][ScanShape<kTiles>::kXBytes];
  unsigned char raw[2][2][ScanShape<kTiles>::kRawBytes];
};

typedef short short4v __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) short4v lds_short4;

// gfx950 transposing LDS load (ds_read_b64_tr_b16).  Within each group of 16
// lanes, lane j reads the four 16-bit values at its own address a_j; lane i of
// the group then receives a_{4e + i/4}[i % 4] for e = 0..3.  If lane j points
// at row r0 + j/4, column c0 + 4 (j % 4) of a row-major 16-bit matrix, lane i
// receives column c0 + i of rows r0 .. r0 + 3: a column slice, as an MFMA
// operand needs it.
__device__ __forceinline__ half4 lds_read_tr(const unsigned char* p) {
  return __builtin_bit_cast(half4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4*)(p)));
}

// <2, 2, 2>: 32 channels, one state wave per tile, two output waves; the
// form for work-groups that fit the CUs one each (shortest chunk period).
// <1, 1, 2>: one state and one output wave, two work-groups per CU (LDS and
// 256 VGPRs per wave allow it).  <2, 2, 4>: 64 channels, two tiles per state
// wave, one work-group per CU: a CU moves the chunk's shared K rows, Q and P
// fragments and blob once for twice the channels.
// kTouchV: the L2 prefetch also touches the work-group's own V rows of chunk
// c + 2.  Worth it when every work-group of the launch is resident (the chunk
// period is then the latency of the stage copy); with more work-groups than
// CUs the extra requests cost more than they save.
// kConvV: v is the conv front's output, formed here from the pre-conv rows
// (p.v, p.vs point into x), so it never goes to HBM: the loader waves also
// copy those rows into LDS a chunk ahead, and two more waves (conv waves)
// turn them into the V tile.  On the loader waves themselves the conv held
// up the copies (T = 8192: 212 us against 179 us for the scan).
template <int kOutWaves, int kStateWaves, int kTiles = 2, bool kTouchV = true, bool kConvV = false>
__global__ __launch_bounds__((scan_threads<kOutWaves, kStateWaves>(kConvV)), kOutWaves == 1 ? 2 : 1) void chunk_scan_kernel(ScanParams p) {
  using Sh = ScanShape<kTiles>;
  constexpr int kParts = Sh::kParts;
  constexpr int kDvPerWg = Sh::kDv;
  constexpr int kScanComputeWaves = kStateWaves + kOutWaves;
  static_assert(kTiles % kStateWaves == 0, "tiles split evenly over the state waves");
  __shared__ ScanSmem<kTiles, kConvV> sm;

  // ---- block id -> (sequence rank, value head, value quarter) --------------
  // Chains sharing a key head (group * kParts of them) get block ids that are
  // congruent mod 8, i.e. land on the same XCD and share fragments through L2.
  const int members = p.group * kParts;
  const int bid = blockIdx.x;
  const int xcd = bid & 7;
  const int slot = bid >> 3;
  const int member = slot % members;
  const int gi = 8 * (slot / members) + xcd;
  if (gi >= p.n_chain_groups) return;
  const int rank = gi / p.Hk;
  const int kh = gi - rank * p.Hk;
  const int h = kh * p.group + member / kParts;
  const int part = member % kParts;
  const int n = p.order ? p.order[rank] : rank;
  const int sn = p.slots ? p.slots[n] : n;    // state of sequence n
  // a slot outside the pool (say -1 for padding) names no state: the whole
  // work-group skips the sequence (no state read or written, o not written)
  if (p.slots && static_cast<unsigned>(sn) >= static_cast<unsigned>(p.n_slots)) return;

  const int tid = threadIdx.x;
  const int w = tid >> 6;
  const int lane = tid & 63;
  const bool compute = w < kScanComputeWaves;

  int seq_start, seq_len, chunk0;
  if (p.cu) {
    seq_start = p.cu[n];
    seq_len = p.cu[n + 1] - seq_start;
    chunk0 = p.chunk_off[n];
  } else {
    seq_start = n * p.seq_len + p.c_base * kC;
    seq_len = min(p.seq_len - p.c_base * kC, p.c_count * kC);
    chunk0 = n * ((p.seq_len + kC - 1) / kC) + p.c_base;
  }
  const int n_chunks = (seq_len + kC - 1) / kC;

  if (!compute) {
    // ---- loader waves: copy the stage of chunk ci + 1 into LDS while the
    // compute waves work on chunk ci ---------------------------------------------
    const int lt = tid - 64 * kScanComputeWaves;          // 0 .. kLoaderThreads - 1
    const int lw = w - kScanComputeWaves;
    const unsigned char* kq_head = p.kq + static_cast<int64_t>(kh) * kKQBytes;
    const unsigned char* vb_head = p.vb + static_cast<int64_t>(h) * kVBytes;
    const int64_t kq_step = static_cast<int64_t>(p.Hk) * kKQBytes;
    const int64_t vb_step = static_cast<int64_t>(p.Hv) * kVBytes;
    const uint16_t* v_head = p.v + h * kD + part * kDvPerWg;

    // Piece i of the stage is its byte 16 i: the K rows, the value-head blob
    // from T_bb on, then the V tile (token i / kVPiecesPerRow, channels
    // 8 (i % kVPiecesPerRow) .. +7 of this work-group's kDv).  With the conv
    // front the copy stops before the V tile.
    constexpr int kRounds = kConvV ? Sh::kKVBRounds : Sh::kStageRounds;
    auto stage = [&](int ci) {
      const int cb = chunk0 + ci;
      const unsigned char* kqb = kq_head + cb * kq_step;
      const unsigned char* vbb = vb_head + cb * vb_step;
      unsigned char* dst = sm.buf[ci & 1];
      const int len = min(kC, seq_len - ci * kC);
      const uint16_t* vrow0 = v_head + static_cast<int64_t>(seq_start + ci * kC) * p.vs;
#pragma unroll
      for (int j = 0; j < kRounds; ++j) {
        const int q = kLoaderThreads * j + lt;
        unsigned char* d = dst + (kLoaderThreads * j + 64 * lw) * 16;
        if (q < kKPieces) {
          lds_dma16(kqb + q * 16, d);
        } else if (q < kKPieces + kVBPieces) {
          lds_dma16(vbb + kOffT + (q - kKPieces) * 16, d);
        } else if (!kConvV && q < Sh::kStagePieces) {
          const int vp = q - kKPieces - kVBPieces;
          const int r = min(vp / Sh::kVPiecesPerRow, len - 1);   // rows past the end re-read the last
          lds_dma16(vrow0 + static_cast<int64_t>(r) * p.vs + (vp % Sh::kVPiecesPerRow) * 8, d);
        }
      }
    };
    if constexpr (!kConvV) {
      // Per chunk: the copies of chunk ci + 1.
      if (n_chunks > 0) stage(0);
      for (int ci = 0; ci < n_chunks; ++ci) {
        dma_barrier();
        if (ci + 1 < n_chunks) stage(ci + 1);
      }
    } else {
      // Conv front.  Loader wave `half` copies the pre-conv rows of tokens
      // 32 half - 3 .. 32 half + 31 of a chunk into raw[chunk & 1][half] two
      // chunks ahead (row rr is token 32 half - 3 + rr); conv wave `half`
      // forms tokens 32 half .. 32 half + 31 of the V tile from them a chunk
      // ahead: its lane (cg, tok0) channels 8 cg .. +7 of tokens tok0 ..
      // tok0 + kConvTok - 1 of that half, from rows tok0 .. tok0 + kConvTok
      // + 2.  Tokens before the sequence take the conv state (or zeros); rows
      // past its end re-read the last.  The operations and their order are
      // those of conv1d_kernel: v equals what the separate conv call stores.
      const int half = lw & 1;      // waves lw = 0, 1 copy, lw = 2, 3 convert
      const int true_start = p.cu ? seq_start : n * p.seq_len;
      const int seq_end = seq_start + seq_len;
      const int cg = lane % Sh::kVPiecesPerRow;
      const int tok0 = Sh::kConvTok * (lane / Sh::kVPiecesPerRow);
      const int ch = p.conv_v0 + h * kD + part * kDvPerWg + 8 * cg;    // channel of x
      float wt[32];
      {
        const uint4* wp = reinterpret_cast<const uint4*>(p.conv_w + static_cast<int64_t>(ch) * 4);
#pragma unroll
        for (int q = 0; q < 4; ++q) bf16x8_to_f32(wp[q], wt + 8 * q);
      }
      float bias[8];
      if (p.conv_bias) {
        const float4 b0 = *reinterpret_cast<const float4*>(p.conv_bias + ch);
        const float4 b1 = *reinterpret_cast<const float4*>(p.conv_bias + ch + 4);
        bias[0] = b0.x; bias[1] = b0.y; bias[2] = b0.z; bias[3] = b0.w;
        bias[4] = b1.x; bias[5] = b1.y; bias[6] = b1.z; bias[7] = b1.w;
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) bias[i] = 0.f;
      }
      auto raw_copy = [&](int ci) {
        const int tb = seq_start + ci * kC + 32 * half - 3;     // token of row 0
        unsigned char* dst = sm.raw[ci & 1][half];
#pragma unroll
        for (int j = 0; j < Sh::kRawRounds; ++j) {
          const int q = 64 * j + lane;
          if (q < Sh::kRawPieces) {
            const int t = min(max(tb + q / Sh::kVPiecesPerRow, true_start), seq_end - 1);
            lds_dma16(v_head + static_cast<int64_t>(t) * p.vs + (q % Sh::kVPiecesPerRow) * 8, dst + j * 1024);
          }
        }
      };
      // v of chunk ci into its stage buffer; `first`: the sequence's first
      // chunk, whose rows before token 0 are the history
      auto conv_tile = [&](int ci, bool first) {
        const unsigned char* src = sm.raw[ci & 1][half] + tok0 * (kDvPerWg * 2) + cg * 16;
        float xin[Sh::kConvTok + 3][8];
#pragma unroll
        for (int j = 0; j < Sh::kConvTok + 3; ++j)
          bf16x8_to_f32(*reinterpret_cast<const uint4*>(src + j * (kDvPerWg * 2)), xin[j]);
        if (first && half == 0 && tok0 < 3) {
          float st[24];
          const int64_t row = p.conv_slots ? p.conv_slots[n] : n;
          // a slot outside the pool reads no history (zeros)
          const bool has_row = p.conv_state &&
              (!p.conv_slots || static_cast<uint64_t>(row) < static_cast<uint64_t>(p.conv_n_slots));
          if (has_row) {
            const uint4* sp = reinterpret_cast<const uint4*>(p.conv_state + (row * p.conv_C + ch) * 3);
            bf16x8_to_f32(sp[0], st);
            bf16x8_to_f32(sp[1], st + 8);
            bf16x8_to_f32(sp[2], st + 16);
          } else {
#pragma unroll
            for (int i = 0; i < 24; ++i) st[i] = 0.f;
          }
          // rows 0, 1, 2 are the tokens 3, 2, 1 before the start: taps 0, 1, 2
#pragma unroll
          for (int j = 0; j < 3; ++j)
            if (tok0 + j < 3)
#pragma unroll
              for (int i = 0; i < 8; ++i) xin[j][i] = st[3 * i + tok0 + j];
        }
        unsigned char* dst = sm.buf[ci & 1] + kStageV + (32 * half + tok0) * (kDvPerWg * 2) + cg * 16;
#pragma unroll
        for (int jj = 0; jj < Sh::kConvTok; ++jj) {
          float y[8];
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            float acc = fmaf(wt[4 * i], xin[jj][i], bias[i]);
            acc = fmaf(wt[4 * i + 1], xin[jj + 1][i], acc);
            acc = fmaf(wt[4 * i + 2], xin[jj + 2][i], acc);
            acc = fmaf(wt[4 * i + 3], xin[jj + 3][i], acc);
            y[i] = conv_silu(acc);
          }
          *reinterpret_cast<u32x4*>(dst + jj * (kDvPerWg * 2)) =
              u32x4{pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3]),
                    pack_bf16x2(y[4], y[5]), pack_bf16x2(y[6], y[7])};
        }
      };
      // One extra barrier before the per-chunk ones: chunk 0's rows in LDS.
      // Per chunk ci, the loader waves copy the stage of ci + 1 and the rows
      // of ci + 2 (into the raw buffer of ci, converted a period ago), the
      // conv waves form v of ci + 1 from its rows (copied a period ago).
      if (lw < 2) {
        if (n_chunks > 0) {
          raw_copy(0);
          stage(0);
          if (n_chunks > 1) raw_copy(1);
        }
        dma_barrier();                     // rows of chunk 0 in LDS
        for (int ci = 0; ci < n_chunks; ++ci) {
          dma_barrier();
          if (ci + 1 < n_chunks) {
            stage(ci + 1);
            if (ci + 2 < n_chunks) raw_copy(ci + 2);
          }
        }
      } else {
        lds_barrier();
        if (n_chunks > 0) conv_tile(0, p.cu || p.c_base == 0);
        for (int ci = 0; ci < n_chunks; ++ci) {
          dma_barrier();
          if (ci + 1 < n_chunks) conv_tile(ci + 1, false);
        }
      }
    }
    lds_barrier();                         // the compute waves' last two barriers
    lds_barrier();
    return;
  }

  // L2 prefetch, two chunks ahead, issued by the output wave: its misses
  // then hold up no copy (a wave's loads complete in order).  The `members`
  // work-groups of a key head share its K/Q blob and the blobs of its value
  // heads; member m pulls lines 64 m .. 64 m + 63 of that data (with 64-channel
  // work-groups also the lines 64 members further on), and each work-group
  // its own V rows with kTouchV.  One dword per 128-byte line; the
  // values go to `sink`, stored only under a condition that never holds.
  const int kq_lines = kKQBytes / 128;
  const int vb_lines = p.group * kVBytes / 128;
  auto touch = [&](int ci) -> uint32_t {
    const int cb = chunk0 + ci;
    auto line = [&](int L) {
      L = min(L, kq_lines + vb_lines - 1);
      return L < kq_lines ? p.kq + (static_cast<int64_t>(cb) * p.Hk + kh) * kKQBytes + L * 128
                          : p.vb + (static_cast<int64_t>(cb) * p.Hv + kh * p.group) * kVBytes + (L - kq_lines) * 128;
    };
    const int r = min(lane, min(kC, seq_len - ci * kC) - 1);
    const unsigned char* b = reinterpret_cast<const unsigned char*>(
        p.v + h * kD + part * kDvPerWg + static_cast<int64_t>(seq_start + ci * kC + r) * p.vs);
    uint32_t x = *reinterpret_cast<const uint32_t*>(line(member * 64 + lane));
    if (kTouchV) x ^= *reinterpret_cast<const uint32_t*>(b);
    if (kTiles > 2) x ^= *reinterpret_cast<const uint32_t*>(line((member + members) * 64 + lane));
    return x;
  };

  // ---- compute waves ---------------------------------------------------------
  // Wave 0 carries the state of this work-group's 32 value channels (two
  // 16-channel tiles) from chunk to chunk: W = K S0^T, U, S <- gamma_L S +
  // U^T D K.  Wave 1 forms the outputs a chunk behind it: O = scale (gamma Q
  // S0^T + P U), from the fp16 S0 and U that wave 0 leaves in LDS.  K, K^T
  // and Q fragments are thus read from LDS once per chunk, and the dependent
  // chain from one chunk's state to the next holds no output products.
  const int col = lane & 15;
  const int grp = lane >> 4;
  if constexpr (kConvV) lds_barrier();     // the conv waves' first barrier

  // State wave(s): kStateWaves waves share the work-group's two tiles; wave
  // sw carries tiles t0 .. t0 + NT - 1.
  auto state_wave = [&](auto nt_c, const int t0) {
    constexpr int NT = decltype(nt_c)::value;
    // state tiles: S^T rows (dk) 16 dt + 4 grp + e, column (dv) 16 t + col
    floatx4 sT[NT][8];
    const int64_t sbase0 = ((static_cast<int64_t>(sn) * p.Hv + h) * kD + part * kDvPerWg + col) * kD;
    if (p.h0) {
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) {
          const float4 v = *reinterpret_cast<const float4*>(p.h0 + sbase0 + 16 * (t0 + t) * kD + 16 * dt + 4 * grp);
          sT[t][dt][0] = v.x; sT[t][dt][1] = v.y; sT[t][dt][2] = v.z; sT[t][dt][3] = v.w;
        }
    } else {
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) sT[t][dt] = floatx4{0.f, 0.f, 0.f, 0.f};
    }
    // Nothing may be pending at the loop header: the compiler's wait insertion
    // would otherwise keep a vmcnt(0) inside the loop.
    __builtin_amdgcn_s_waitcnt(0);

    for (int ci = 0; ci < n_chunks; ++ci) {
      const unsigned char* B = sm.buf[ci & 1];
      // VB + kOffX is item X of the value-head blob (staged from T_bb on)
      const unsigned char* VB = B + kStageVB - kOffT;
      unsigned char* X = sm.xbuf[ci & 1];
      // K A-fragment (rows 16 tb .. +15 = tokens, 32 dk columns of block kb):
      // the columns kappa(grp, e) are stored together
      auto kfrag = [&](int tb, int kb) {
        return *reinterpret_cast<const half8*>(B + (16 * tb + col) * kKRowBytes + kb * 64 + grp * 16);
      };
      // K^T A-fragment (rows 16 dt .. +15 = dk, 32 tokens of block kb): two
      // transposing loads over token rows 32 kb + 4 grp .. and 32 kb + 16 + 4 grp ..;
      // lane col reads the run of dk columns 16 dt + 4 (col & 3) .. +3, stored at
      // run slot 2 (col & 3) + (dt & 1) of 32-column block dt / 2
      auto ktfrag = [&](int dt, int kb) {
        const unsigned char* r = B + (32 * kb + 4 * grp + (col >> 2)) * kKRowBytes + (dt >> 1) * 64 +
                                 (2 * (col & 3) + (dt & 1)) * 8;
        return cat8(lds_read_tr(r), lds_read_tr(r + 16 * kKRowBytes));
      };
      auto frag16 = [&](int off) { return *reinterpret_cast<const half4*>(VB + off + lane * 8); };
      auto vfrag = [&](int off) { return *reinterpret_cast<const half8*>(VB + off + lane * 16); };
      auto table = [&](int tab, int tb) {
        return *reinterpret_cast<const floatx4*>(VB + kOffDecay + tab * 256 + (16 * tb + 4 * grp) * 4);
      };
      // V of tokens 16 tb + 4 grp + e, channel 16 t + col: a transposing load
      // over the row-major bf16 V tile
      const unsigned char* vtile = B + kStageV;
      auto vcol = [&](int t, int tb) {
        return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_short4*)(vtile + (16 * tb + 4 * grp + (col >> 2)) * (2 * kDvPerWg) + 32 * t + 8 * (col & 3)));
      };

      // The chunk runs in phases separated by scheduling fences; each phase
      // issues the LDS reads of the next one, so read latency hides behind the
      // products of the current phase.
      lds_barrier();                       // this chunk's stage is in LDS

      // phase 0: K fragments; B operands of S0^T straight from registers, also
      // left in LDS for the output wave
      half8 fk[16];
#pragma unroll
      for (int tb = 0; tb < 4; ++tb)
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) fk[tb * 4 + kb] = kfrag(tb, kb);
      half8 sB[NT][4];
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
          sB[t][kb] = to_half8(sT[t][2 * kb], sT[t][2 * kb + 1]);
          *reinterpret_cast<half8*>(X + (4 * (t0 + t) + kb) * kFrag + lane * 16) = sB[t][kb];
        }
      __builtin_amdgcn_sched_barrier(0);

      // phase 1: V, tables | W = K S0^T by token block, so that the solve
      // below can start on block 0 while later blocks are still in the MFMA
      // pipe (no fence between the two phases); gamma_L S^T in VALU meanwhile
      short4v vr[NT][4];
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) vr[t][tb] = vcol(t0 + t, tb);
      floatx4 bt[4], bg[4];
#pragma unroll
      for (int tb = 0; tb < 4; ++tb) {
        bt[tb] = table(0, tb);
        bg[tb] = table(1, tb);
      }
      floatx4 W[NT][4];
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) W[t][tb] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int tb = 0; tb < 4; ++tb)
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int t = 0; t < NT; ++t) W[t][tb] = mfma32(fk[tb * 4 + kb], sB[t][kb], W[t][tb]);
      // gamma_L S^T, while the products run (S0 has been read as sB)
      {
        const float gl = *reinterpret_cast<const float*>(VB + kOffGL);
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
          for (int dt = 0; dt < 8; ++dt)
#pragma unroll
            for (int e = 0; e < 4; ++e) sT[t][dt][e] *= gl;
      }

      // then T_bb, -A, K^T fragments | R = b V - b gamma W, U by blockwise
      // forward substitution (rows = tokens 16 tb + 4 grp + e, column 16 t +
      // col), the two tiles' dependent chains interleaved
      half4 tT[4];
#pragma unroll
      for (int b = 0; b < 4; ++b) tT[b] = frag16(kOffT + b * kFrag16);
      const half4 an10 = frag16(kOffAn10);
      const half8 an2 = vfrag(kOffAn2);
      const half8 an3 = vfrag(kOffAn3);
      const half4 an32 = frag16(kOffAn32);
      half8 ft[16];
#pragma unroll
      for (int dt = 0; dt < 8; ++dt)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) ft[2 * dt + kb] = ktfrag(dt, kb);
      floatx4 R[NT][4];
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int tb = 0; tb < 4; ++tb)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            R[t][tb][e] = bt[tb][e] * bf16_to_f32(static_cast<uint16_t>(vr[t][tb][e])) - bg[tb][e] * W[t][tb][e];
      const floatx4 z4 = {0.f, 0.f, 0.f, 0.f};
      floatx4 U[NT][4];
      half8 u01[NT], u23[NT];
#pragma unroll
      for (int t = 0; t < NT; ++t) U[t][0] = mfma16(tT[0], to_half4(R[t][0]), z4);
      floatx4 rhs[NT];
#pragma unroll
      for (int t = 0; t < NT; ++t) rhs[t] = mfma16(an10, to_half4(U[t][0]), R[t][1]);
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        U[t][1] = mfma16(tT[1], to_half4(rhs[t]), z4);
        u01[t] = to_half8(U[t][0], U[t][1]);
      }
#pragma unroll
      for (int t = 0; t < NT; ++t) rhs[t] = mfma32(an2, u01[t], R[t][2]);
#pragma unroll
      for (int t = 0; t < NT; ++t) U[t][2] = mfma16(tT[2], to_half4(rhs[t]), z4);
      // The last block row's two products meet in a VALU add: a 16x16x32
      // result taken straight as the accumulator of a 16x16x16 product has
      // been observed to read stale values.
#pragma unroll
      for (int t = 0; t < NT; ++t) rhs[t] = mfma32(an3, u01[t], R[t][3]);
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const floatx4 r2 = mfma16(an32, to_half4(U[t][2]), z4);
#pragma unroll
        for (int e = 0; e < 4; ++e) rhs[t][e] += r2[e];
      }
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        U[t][3] = mfma16(tT[3], to_half4(rhs[t]), z4);
        u23[t] = to_half8(U[t][2], U[t][3]);
      }
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        *reinterpret_cast<half8*>(X + (Sh::kU0 + 2 * (t0 + t)) * kFrag + lane * 16) = u01[t];
        *reinterpret_cast<half8*>(X + (Sh::kU0 + 1 + 2 * (t0 + t)) * kFrag + lane * 16) = u23[t];
      }
      __builtin_amdgcn_sched_barrier(0);

      // phase 2: S^T <- (gamma_L S^T) + K^T (D U)
      floatx4 dl[4];
#pragma unroll
      for (int tb = 0; tb < 4; ++tb) dl[tb] = table(3, tb);
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        floatx4 DU[4];
#pragma unroll
        for (int tb = 0; tb < 4; ++tb)
#pragma unroll
          for (int e = 0; e < 4; ++e) DU[tb][e] = dl[tb][e] * U[t][tb][e];
        const half8 d01 = to_half8(DU[0], DU[1]);
        const half8 d23 = to_half8(DU[2], DU[3]);
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) {
          floatx4 s = sT[t][dt];
          s = mfma32(ft[2 * dt], d01, s);
          s = mfma32(ft[2 * dt + 1], d23, s);
          sT[t][dt] = s;
        }
      }
    }
    lds_barrier();                         // S0, U of the last chunk written
    lds_barrier();

    if (p.hT) {
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int dt = 0; dt < 8; ++dt)
          *reinterpret_cast<float4*>(p.hT + sbase0 + 16 * (t0 + t) * kD + 16 * dt + 4 * grp) =
              make_float4(sT[t][dt][0], sT[t][dt][1], sT[t][dt][2], sT[t][dt][3]);
    }
  };
  if (w < kStateWaves) {
    constexpr int kNT = kTiles / kStateWaves;
    state_wave(std::integral_constant<int, kNT>{}, w * kNT);
    return;
  }

  // ---- output waves: O of chunk ci - 1 during chunk ci -----------------------
  // Output wave ow forms token blocks tb0 .. tb0 + ntb - 1 of O^T =
  // scale gamma^T (S0 Q^T) + U^T P^T (rows = value channels 4 grp + e of tile
  // t, column = token 16 tb + col; the P fragments serve as B operands).  Its
  // Q and P fragments and per-token scales of chunk ci come from global
  // memory (L2, prefetched) straight into registers, a chunk before their use.
  const int64_t o_rs = static_cast<int64_t>(p.Hv) * kD;   // o row stride (floats)
  auto output_wave = [&](auto ow_c) {
    constexpr int ow = decltype(ow_c)::value;
    constexpr int ntb = 4 / kOutWaves;
    constexpr int tb0 = ntb * ow;
    // P fragments in the blob: (0,0)(1,0)(2,0)(2,1)(3,0)(3,1); token block tb
    // uses fragment tb (tb < 2) or 2 tb - 2 and 2 tb - 1
    constexpr int p0 = tb0 < 2 ? tb0 : 2 * tb0 - 2;
    constexpr int tbl = tb0 + ntb - 1;
    constexpr int np = (tbl < 2 ? tbl : 2 * tbl - 1) - p0 + 1;
    constexpr bool need_u23 = tbl >= 2;
    half8 fq[4 * ntb], fp[np];
    float sgl[ntb];                        // scale gamma of token 16 (tb0 + i) + col
    auto load_q = [&](int ci) {
      const int cb = chunk0 + ci;
      const unsigned char* Qb = p.kq + (static_cast<int64_t>(cb) * p.Hk + kh) * kKQBytes + kOffQ;
      const unsigned char* VB = p.vb + (static_cast<int64_t>(cb) * p.Hv + h) * kVBytes;
#pragma unroll
      for (int f = 0; f < 4 * ntb; ++f) fq[f] = *reinterpret_cast<const half8*>(Qb + (4 * tb0 + f) * kFrag + lane * 16);
#pragma unroll
      for (int f = 0; f < np; ++f) fp[f] = *reinterpret_cast<const half8*>(VB + kOffP + (p0 + f) * kFrag + lane * 16);
#pragma unroll
      for (int i = 0; i < ntb; ++i)
        sgl[i] = *reinterpret_cast<const float*>(VB + kOffDecay + 2 * 256 + (16 * (tb0 + i) + col) * 4);
    };
    auto output = [&](int ci) {
      const unsigned char* X = sm.xbuf[ci & 1];
      half8 sB[kTiles][4], u[kTiles][2];
#pragma unroll
      for (int t = 0; t < kTiles; ++t) {
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) sB[t][kb] = *reinterpret_cast<const half8*>(X + (4 * t + kb) * kFrag + lane * 16);
#pragma unroll
        for (int j = 0; j < (need_u23 ? 2 : 1); ++j)
          u[t][j] = *reinterpret_cast<const half8*>(X + (Sh::kU0 + 2 * t + j) * kFrag + lane * 16);
      }
      const int len = min(kC, seq_len - ci * kC);
      const int64_t oe = static_cast<int64_t>(seq_start + ci * kC) * o_rs + h * kD + part * kDvPerWg + 4 * grp;
#pragma unroll
      for (int t = 0; t < kTiles; ++t)
#pragma unroll
        for (int i = 0; i < ntb; ++i) {
          const int tb = tb0 + i;
          floatx4 qs = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int kb = 0; kb < 4; ++kb) qs = mfma32(sB[t][kb], fq[4 * i + kb], qs);
          floatx4 O;
#pragma unroll
          for (int e = 0; e < 4; ++e) O[e] = sgl[i] * qs[e];
          if (tb < 2) {
            O = mfma32(u[t][0], fp[tb - p0], O);
          } else {
            O = mfma32(u[t][0], fp[2 * tb - 2 - p0], O);
            O = mfma32(u[t][need_u23 ? 1 : 0], fp[2 * tb - 1 - p0], O);
          }
          if (16 * tb + col < len) {
            const int64_t e = oe + (16 * tb + col) * o_rs + 16 * t;
            if (p.o_bf16)   // round to nearest even (v_cvt_pk_bf16_f32)
              *reinterpret_cast<uint2*>(static_cast<uint16_t*>(p.o) + e) = uint2{pack_bf16x2(O[0], O[1]), pack_bf16x2(O[2], O[3])};
            else
              *reinterpret_cast<floatx4*>(static_cast<float*>(p.o) + e) = O;
          }
        }
    };
    uint32_t sink = 0, tv = 0, tv_prev = 0;
    constexpr bool prefetcher = ow == kOutWaves - 1;
    if (prefetcher && n_chunks > 0) tv = touch(min(1, n_chunks - 1));
    for (int ci = 0; ci < n_chunks; ++ci) {
      lds_barrier();                       // stage ci in LDS; S0, U of chunk ci - 1 written
      if (prefetcher) {
        sink ^= tv_prev;                   // issued two chunks ago
        tv_prev = tv;
        tv = touch(min(ci + 2, n_chunks - 1));
      }
      if (ci > 0) output(ci - 1);
      load_q(ci);
    }
    sink ^= tv_prev ^ tv;
    if (sink == 0x9e3779b9u && p.n_seqs < 0) static_cast<float*>(p.o)[0] = 0.f;   // keeps the prefetch loads
    lds_barrier();                         // S0, U of the last chunk written
    if (n_chunks > 0) output(n_chunks - 1);
    lds_barrier();
  };
  if (kOutWaves == 1 || w == kStateWaves) output_wave(std::integral_constant<int, 0>{});
  else output_wave(std::integral_constant<int, kOutWaves - 1>{});
}

static_assert(sizeof(ScanSmem<2, true>) + kScanLdsPad <= 160 * 1024, "padded scan work-group fits a CU");
static_assert(sizeof(ScanSmem<2, false>) + kScanLdsPad + sizeof(PrepSmem) > 160 * 1024,
              "no prep work-group fits beside a padded scan work-group");
static_assert(sizeof(ScanSmem<4, true>) + kScanLdsPad4 <= 160 * 1024, "padded 64-channel work-group fits a CU");
static_assert(sizeof(ScanSmem<4, false>) + kScanLdsPad4 + sizeof(PrepSmem) > 160 * 1024,
              "no prep work-group fits beside a padded 64-channel scan work-group");

hipError_t launch_prep(const PrepParams& pp, dim3 grid, bool conv, hipStream_t stream) {
  if (conv) {
    if (pp.ga)
      hipLaunchKernelGGL((chunk_prep_kernel<true, true>), grid, dim3(kThreads), 0, stream, pp);
    else
      hipLaunchKernelGGL((chunk_prep_kernel<false, true>), grid, dim3(kThreads), 0, stream, pp);
  } else {
    if (pp.ga)
      hipLaunchKernelGGL((chunk_prep_kernel<true, false>), grid, dim3(kThreads), 0, stream, pp);
    else
      hipLaunchKernelGGL((chunk_prep_kernel<false, false>), grid, dim3(kThreads), 0, stream, pp);
  }
  return hipGetLastError();
}

// One scan launch: the 32- (kTiles = 2) or 64-channel form, with the conv
// front or without, `lds` bytes of LDS added.
template <int kTiles, bool kTouchV>
hipError_t launch_scan(const ScanParams& sp, int blocks, size_t lds, bool conv, hipStream_t stream) {
  if (conv)
    hipLaunchKernelGGL((chunk_scan_kernel<2, 2, kTiles, kTouchV, true>), dim3(blocks),
                       dim3(scan_threads<2, 2>(true)), lds, stream, sp);
  else
    hipLaunchKernelGGL((chunk_scan_kernel<2, 2, kTiles, kTouchV, false>), dim3(blocks),
                       dim3(scan_threads<2, 2>()), lds, stream, sp);
  return hipGetLastError();
}

}  // namespace

// Compute units of the current device, looked up once per device (calls from
// several host threads may race to fill an entry; they store the same value).
int compute_units() {
  static std::atomic<int> cached[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cached[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cached[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

Overlap* overlap_of_current_device() {
  static Overlap ov[64];
  static std::once_flag once[64];
  static bool ok[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
  std::call_once(once[dev], [&] {
    Overlap& o = ov[dev];
    bool good = hipStreamCreateWithFlags(&o.side, hipStreamNonBlocking) == hipSuccess &&
                hipEventCreateWithFlags(&o.start, hipEventDisableTiming) == hipSuccess;
    for (int i = 0; i < 2 && good; ++i)
      good = hipEventCreateWithFlags(&o.done[i], hipEventDisableTiming) == hipSuccess;
    ok[dev] = good;
  });
  return ok[dev] ? &ov[dev] : nullptr;
}

ChunkWorkspace chunk_workspace_layout(int n_seqs, int T_total, int Hk, int Hv) {
  auto up = [](size_t b) { return (b + 255) & ~static_cast<size_t>(255); };
  ChunkWorkspace ws;
  ws.max_chunks = static_cast<size_t>(T_total) / kC + static_cast<size_t>(n_seqs);
  ws.order_off = 0;
  ws.chunk_off_off = up(sizeof(int32_t) * static_cast<size_t>(n_seqs));
  ws.chunk_tab_off = ws.chunk_off_off + up(sizeof(int32_t) * (static_cast<size_t>(n_seqs) + 1));
  ws.kq_off = ws.chunk_tab_off + up(sizeof(int32_t) * 3 * ws.max_chunks);
  ws.v_off = ws.kq_off + up(ws.max_chunks * static_cast<size_t>(Hk) * kKQBytes);
  ws.carry_off = ws.v_off + up(ws.max_chunks * static_cast<size_t>(Hv) * kVBytes);
  const bool carry = n_seqs > 0 && T_total / n_seqs >= kSegMinChunks * kC;
  ws.total = ws.carry_off + (carry ? static_cast<size_t>(n_seqs) * Hv * kD * kD * sizeof(float) : 0);
  return ws;
}

hipError_t launch_chunk_fwd(const uint16_t* q, int64_t qs, const uint16_t* k, int64_t ks,
                            const uint16_t* v, int64_t vs, const GateInputs& gates,
                            void* o, bool o_bf16, const float* h0, float* hT,
                            const int32_t* state_slot, int n_slots, const int32_t* cu,
                            int n_seqs, int T_total, int Hk, int Hv, float scale,
                            void* workspace, hipStream_t stream, const ConvFront* conv) {
  if (n_seqs == 0) return hipSuccess;
  const ChunkWorkspace ws = chunk_workspace_layout(n_seqs, T_total, Hk, Hv);
  unsigned char* base = static_cast<unsigned char*>(workspace);
  int32_t* order = reinterpret_cast<int32_t*>(base + ws.order_off);
  int32_t* chunk_off = reinterpret_cast<int32_t*>(base + ws.chunk_off_off);
  int32_t* chunk_tab = reinterpret_cast<int32_t*>(base + ws.chunk_tab_off);
  const int seq_len = cu ? 0 : T_total / n_seqs;
  const int nc = cu ? 0 : (seq_len + kC - 1) / kC;    // chunks per sequence (equal lengths)
  int n_chunk_slots;   // grid of the prep kernel
  if (cu) {
    const hipError_t e = launch_chunk_map(cu, n_seqs, T_total, order, chunk_off, chunk_tab, stream);
    if (e != hipSuccess) return e;
    n_chunk_slots = static_cast<int>(ws.max_chunks);
  } else {
    n_chunk_slots = n_seqs * nc;
  }
  PrepParams pp{};
  pp.q = q; pp.k = k; pp.qs = qs; pp.ks = ks; pp.g = gates.g; pp.beta = gates.beta;
  pp.ga = gates.a; pp.gb = gates.b; pp.gas = gates.a_stride; pp.gbs = gates.b_stride;
  pp.A_log = gates.A_log; pp.dt_bias = gates.dt_bias;
  if (conv) {
    pp.x = conv->x; pp.xs = conv->xs; pp.conv_w = conv->w; pp.conv_bias = conv->bias;
    pp.conv_state = conv->state; pp.conv_slots = conv->slots; pp.conv_n_slots = conv->n_slots;
    pp.l2_eps = conv->l2_eps;
  }
  pp.cu = cu; pp.chunk_off = chunk_off; pp.chunk_tab = chunk_tab;
  pp.kq = base + ws.kq_off; pp.vb = base + ws.v_off;
  pp.n_seqs = n_seqs; pp.seq_len = seq_len; pp.Hk = Hk; pp.Hv = Hv; pp.group = Hv / Hk;
  pp.scale = scale;

  ScanParams sp{};
  if (conv) {
    // the scan forms v from x's value columns
    sp.conv_v0 = 2 * Hk * kD;
    sp.conv_C = (2 * Hk + Hv) * kD;
    v = conv->x + sp.conv_v0;
    vs = conv->xs;
    sp.conv_w = conv->w; sp.conv_bias = conv->bias; sp.conv_state = conv->state;
    sp.conv_slots = conv->slots; sp.conv_n_slots = conv->n_slots;
  }
  sp.v = v; sp.vs = vs; sp.o = o; sp.o_bf16 = o_bf16 ? 1 : 0; sp.h0 = h0; sp.hT = hT;
  sp.slots = state_slot;
  sp.n_slots = n_slots;
  sp.cu = cu; sp.order = cu ? order : nullptr; sp.chunk_off = chunk_off;
  sp.kq = base + ws.kq_off; sp.vb = base + ws.v_off;
  sp.n_seqs = n_seqs; sp.seq_len = seq_len; sp.Hk = Hk; sp.Hv = Hv; sp.group = Hv / Hk;
  sp.n_chain_groups = n_seqs * Hk;
  sp.c_base = 0; sp.c_count = nc;
  // work-groups of the 32- and 64-channel forms (the block map rounds the
  // (sequence, key head) groups up to a multiple of the 8 XCDs)
  const int blocks = ((sp.n_chain_groups + 7) / 8) * 8 * sp.group * ScanShape<2>::kParts;
  const int blocks4 = ((sp.n_chain_groups + 7) / 8) * 8 * sp.group * ScanShape<4>::kParts;
  const int cus = compute_units();

  // Long equal-length sequences whose scan leaves compute units idle (in the
  // 32-channel form, else in the 64-channel form): the prep of segment i + 1
  // runs on a second stream, on those idle units, while the scan works
  // through segment i.
  const bool seg32 = blocks + kSegMinIdleCUs <= cus;
  const bool seg64 = !seg32 && blocks4 + kSegMinIdleCUs <= cus;
  if (!cu && !state_slot && T_total > 0 && nc >= kSegMinChunks && (seg32 || seg64) &&
      ws.total > ws.carry_off) {
    Overlap* ov = overlap_of_current_device();
    if (ov) {
      std::lock_guard<std::mutex> lock(ov->mu);
      float* carry = reinterpret_cast<float*>(base + ws.carry_off);
      const int n_seg = (nc + kSegChunks - 1) / kSegChunks;
      auto prep_seg = [&](int s, hipStream_t st) {
        pp.seg_c0 = s * kSegChunks;
        pp.seg_nc = std::min(kSegChunks, nc - pp.seg_c0);
        return launch_prep(pp, dim3(Hk, n_seqs * pp.seg_nc), conv != nullptr, st);
      };
      hipError_t e = prep_seg(0, stream);
      if (e == hipSuccess) e = hipEventRecord(ov->start, stream);
      if (e == hipSuccess) e = hipStreamWaitEvent(ov->side, ov->start, 0);
      for (int s = 0; s < n_seg && e == hipSuccess; ++s) {
        if (s + 1 < n_seg) {
          // done[(s + 1) & 1] was last waited on (enqueued) in step s - 1
          e = prep_seg(s + 1, ov->side);
          if (e == hipSuccess) e = hipEventRecord(ov->done[(s + 1) & 1], ov->side);
          if (e != hipSuccess) break;
        }
        if (s > 0) e = hipStreamWaitEvent(stream, ov->done[s & 1], 0);
        if (e != hipSuccess) break;
        sp.c_base = s * kSegChunks;
        sp.c_count = kSegChunks;
        sp.h0 = s == 0 ? h0 : carry;
        sp.hT = s + 1 == n_seg ? hT : carry;
        e = seg32 ? launch_scan<2, true>(sp, blocks, kScanLdsPad, conv != nullptr, stream)
                  : launch_scan<4, true>(sp, blocks4, kScanLdsPad4, conv != nullptr, stream);
      }
      return e;
    }
  }

  if (T_total > 0 && n_chunk_slots > 0) {
    pp.seg_c0 = 0;
    pp.seg_nc = 0;
    const hipError_t e = launch_prep(pp, dim3(Hk, n_chunk_slots), conv != nullptr, stream);
    if (e != hipSuccess) return e;
  }
  if (blocks <= cus) return launch_scan<2, true>(sp, blocks, 0, conv != nullptr, stream);
  // more work-groups than CUs: the 64-channel form, half as many; no V
  // touch once even those outnumber the CUs
  if (blocks4 <= cus) return launch_scan<4, true>(sp, blocks4, 0, conv != nullptr, stream);
  return launch_scan<4, false>(sp, blocks4, 0, conv != nullptr, stream);
}

}  // namespace gdn
