// launch.h -- host-side launchers of the gfx950 kernels (internal to libgdn).
// Arguments are validated by the C ABI layer before any of these is called.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace gdn {

hipError_t launch_decode_step(const uint16_t* q, int64_t q_stride, const uint16_t* k,
                              int64_t k_stride, const uint16_t* v, int64_t v_stride,
                              const float* g, const float* beta, float* state,
                              const int32_t* state_slot, float* o, int n_seqs, int Hk, int Hv,
                              float scale, hipStream_t stream);

hipError_t launch_decode_tokens(const uint16_t* q, int64_t q_stride, const uint16_t* k,
                                int64_t k_stride, const uint16_t* v, int64_t v_stride,
                                const float* g, const float* beta, float* state,
                                const int32_t* state_slot, float* o, int n_seqs, int n_tokens,
                                int Hk, int Hv, float scale, hipStream_t stream);

hipError_t launch_decode_mixer(const uint16_t* x, int64_t xs, const uint16_t* conv_w,
                               const float* conv_bias, uint16_t* conv_state, const float* g,
                               const float* beta, const uint16_t* z, int64_t zs,
                               const float* norm_w, float* state, const int32_t* state_slot,
                               void* out, bool out_bf16, int n_seqs, int Hk, int Hv, float scale,
                               float l2_eps, float norm_eps, hipStream_t stream);

hipError_t launch_conv1d(const uint16_t* x, int64_t xs, const uint16_t* w, const float* bias,
                         uint16_t* y, int64_t ys, uint16_t* conv_state, const int32_t* cu,
                         int n_seqs, int T_total, int C, int n_l2_channels, float l2_eps,
                         hipStream_t stream);

hipError_t launch_gated_rmsnorm(const float* o, const uint16_t* z, int64_t zs, const float* w,
                                void* out, bool out_bf16, int64_t rows, int Hv, float eps,
                                hipStream_t stream);

// Workspace of the chunked prefill (each piece 256-byte aligned):
//   order [n_seqs] | chunk_off [n_seqs+1] | chunk_tab [max_chunks][3]
//   | K rows + Q fragments [max_chunks][Hk] | per-value-head fragments [max_chunks][Hv]
struct ChunkWorkspace {
  size_t max_chunks, order_off, chunk_off_off, chunk_tab_off, kq_off, v_off, total;
};
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

// state_slot != nullptr: sequence n reads h0[state_slot[n]] and writes
// hT[state_slot[n]] (h0 == hT: a state pool updated in place).
hipError_t launch_chunk_fwd(const uint16_t* q, int64_t qs, const uint16_t* k, int64_t ks,
                            const uint16_t* v, int64_t vs, const GateInputs& gates,
                            void* o, bool o_bf16, const float* h0, float* hT,
                            const int32_t* state_slot, const int32_t* cu,
                            int n_seqs, int T_total, int Hk, int Hv, float scale,
                            void* workspace, hipStream_t stream);

}  // namespace gdn
