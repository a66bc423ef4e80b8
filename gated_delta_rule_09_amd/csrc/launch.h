// launch.h -- host-side launchers of the gfx950 kernels (internal to libgdn).
// Arguments are validated by the C ABI layer before any of these is called.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <mutex>

namespace gdn {

hipError_t launch_decode_step(const uint16_t* q, int64_t q_stride, const uint16_t* k,
                              int64_t k_stride, const uint16_t* v, int64_t v_stride,
                              const float* g, const float* beta, float* state,
                              const int32_t* state_slot, int n_slots, float* o, int n_seqs,
                              int Hk, int Hv, float scale, hipStream_t stream);

hipError_t launch_decode_tokens(const uint16_t* q, int64_t q_stride, const uint16_t* k,
                                int64_t k_stride, const uint16_t* v, int64_t v_stride,
                                const float* g, const float* beta, float* state,
                                const int32_t* state_slot, int n_slots, float* o, int n_seqs,
                                int n_tokens, int Hk, int Hv, float scale, hipStream_t stream);

hipError_t launch_conv1d(const uint16_t* x, int64_t xs, const uint16_t* w, const float* bias,
                         uint16_t* y, int64_t ys, uint16_t* conv_state, const int32_t* cu,
                         int n_seqs, int T_total, int C, int n_l2_channels, float l2_eps,
                         hipStream_t stream);

hipError_t launch_gated_rmsnorm(const float* o, const uint16_t* z, int64_t zs, const float* w,
                                void* out, bool out_bf16, int64_t rows, int Hv, float eps,
                                hipStream_t stream);

// The library's second stream and its events, one set per device, made on
// first use (with that device current) and kept until the process ends; the
// overlapped prefill and the backward run work on it beside the caller's
// stream.  The lock keeps one call's records and waits together.  nullptr if
// they could not be made.
struct Overlap {
  std::mutex mu;
  hipStream_t side = nullptr;
  hipEvent_t start = nullptr;
  hipEvent_t done[2] = {};
};
Overlap* overlap_of_current_device();

// Compute units of the current device (256 if the query fails).
int compute_units();

// Workspace of the chunked prefill (each piece 256-byte aligned):
//   order [n_seqs] | chunk_off [n_seqs+1] | chunk_tab [max_chunks][3]
//   | K rows + Q fragments [max_chunks][Hk] | per-value-head fragments [max_chunks][Hv]
struct ChunkWorkspace {
  size_t max_chunks, order_off, chunk_off_off, chunk_tab_off, kq_off, v_off, carry_off, total;
};
// Long sequences (T_total / n_seqs >= 32768) also get the state carried from
// one segment of the overlapped prefill to the next, [n_seqs, Hv, 128, 128]
// fp32 at carry_off.
ChunkWorkspace chunk_workspace_layout(int n_seqs, int T_total, int Hk, int Hv);

hipError_t launch_chunk_map(const int32_t* cu, int n_seqs, int T_total, int32_t* order,
                            int32_t* chunk_off, int32_t* chunk_tab, hipStream_t stream);

// The gates of the prefill: g, beta [T, Hv] fp32 as given, or (a != nullptr)
// formed in the prep kernel from the bf16 projections a, b [T, Hv] (token
// strides a_stride, b_stride) and the per-head A_log, dt_bias.
struct GateInputs {
  const float* g = nullptr;
  const float* beta = nullptr;
  const uint16_t* a = nullptr;
  int64_t a_stride = 0;
  const uint16_t* b = nullptr;
  int64_t b_stride = 0;
  const float* A_log = nullptr;
  const float* dt_bias = nullptr;
};

// One decode step of the whole mixer (decode_mixer.hip), gates given or from
// the projections.
hipError_t launch_decode_mixer(const uint16_t* x, int64_t xs, const uint16_t* conv_w,
                               const float* conv_bias, uint16_t* conv_state,
                               const GateInputs& gates, const uint16_t* z, int64_t zs,
                               const float* norm_w, float* state, const int32_t* state_slot,
                               int n_slots, void* out, bool out_bf16, int n_seqs, int Hk, int Hv,
                               float scale,
                               float l2_eps, float norm_eps, hipStream_t stream);

// The conv front of the fused mixer prefill: the prep kernel computes q, k
// (conv + SiLU + L2, bf16-rounded) and v (conv + SiLU, bf16, into the
// workspace for the scan) from the pre-conv rows x [T, (2 Hk + Hv) 128], with
// the same arithmetic as launch_conv1d.  The conv state is only read; the
// caller shifts it afterwards (launch_conv_state).
struct ConvFront {
  const uint16_t* x = nullptr;
  int64_t xs = 0;
  const uint16_t* w = nullptr;
  const float* bias = nullptr;
  const uint16_t* state = nullptr;
  const int32_t* slots = nullptr;   // nullptr: sequence n uses conv state row n
  int n_slots = 0;                  // rows of the conv-state pool (with slots)
  float l2_eps = 1e-6f;
};

// state_slot != nullptr: sequence n reads h0[state_slot[n]] and writes
// hT[state_slot[n]] (h0 == hT: a state pool of n_slots rows updated in place);
// a sequence whose slot lies outside [0, n_slots) is skipped.
hipError_t launch_chunk_fwd(const uint16_t* q, int64_t qs, const uint16_t* k, int64_t ks,
                            const uint16_t* v, int64_t vs, const GateInputs& gates,
                            void* o, bool o_bf16, const float* h0, float* hT,
                            const int32_t* state_slot, int n_slots, const int32_t* cu,
                            int n_seqs, int T_total, int Hk, int Hv, float scale,
                            void* workspace, hipStream_t stream,
                            const ConvFront* conv = nullptr);

// The new conv state [n_seqs, C, 3] (last three inputs of old state ++
// sequence), after every read of the old one.  With slots, sequence n updates
// row slots[n] of a pool of n_slots rows (none if the slot is outside it).
hipError_t launch_conv_state(const uint16_t* x, int64_t xs, uint16_t* conv_state,
                             const int32_t* cu, int n_seqs, int T_total, int C,
                             hipStream_t stream, const int32_t* slots = nullptr,
                             int n_slots = 0);

// The chunked backward (backward_chunk.hip): per chunk slot (T / 64 + n_seqs
// of them) and value head a 64 x 64 matrix (T and P), the state before and the
// state gradient after the chunk, and U, E, dR.
size_t chunked_backward_workspace_bytes(int n_seqs, int T_total, int Hv);
hipError_t launch_backward_chunked(const uint16_t* q, int64_t qs, const uint16_t* k, int64_t ks,
                                   const uint16_t* v, int64_t vs, const float* g, const float* beta,
                                   const float* h0, const float* d_o, const float* dhT,
                                   const int32_t* cu, int n_seqs, int T_total, int Hk, int Hv,
                                   float scale, float* dq, float* dk, float* dv, float* dg,
                                   float* dbeta, float* dh0, void* workspace, hipStream_t stream);

// Dense MFMA loop (calib.hip): n_blocks work-groups of 4 waves, each wave
// n_iter rounds of 8 independent 16x16x32 fp16 products; one float per wave
// to out (mfma_loop_waves(n_blocks) of them).
double mfma_loop_flops(int n_iter, int n_blocks);
int mfma_loop_waves(int n_blocks);
hipError_t launch_mfma_loop(int n_iter, int n_blocks, float* out, hipStream_t stream);
// Streaming pass (calib.hip): every 16-byte piece of buf read and written back
// unchanged, nontemporally, by n_blocks work-groups of 256 threads.
hipError_t launch_stream_inplace(void* buf, int64_t bytes, int n_blocks, hipStream_t stream);

}  // namespace gdn
