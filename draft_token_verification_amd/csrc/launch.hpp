// launch.hpp -- host-side launchers of the libspecverify kernels. Internal:
// the C ABI in api.hip validates arguments and then calls these.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sv {

// top2_margin may be null (no margin output). With a workspace of at least
// greedy_workspace_bytes(B, K, V) bytes (8-byte aligned) each sequence's rows
// are split over several workgroups; otherwise one workgroup per sequence.
hipError_t launch_greedy(const void* target, bool bf16, int B, int K, int V, const int32_t* tokens,
                         const int32_t* lens, int32_t* n_accepted, int32_t* next_token, float* top2_margin,
                         void* workspace, size_t workspace_bytes, hipStream_t stream);

// 0 when one workgroup per sequence is used regardless (short rows); the size
// covers fp32 and bf16 rows alike.
size_t greedy_workspace_bytes(int B, int K, int V);

hipError_t launch_accept(const float* p, const float* q, int B, int K, int V, const int32_t* tokens,
                         const int32_t* lens, const float* uniforms, int32_t* n_accepted, int32_t* next_token,
                         hipStream_t stream);

// With a workspace of at least accept_logits_workspace_bytes(B, K, V) bytes
// (8-byte aligned), each sequence is split over several workgroups; otherwise
// one workgroup per sequence.
// draft_lse (may be null): the draft rows' log-normalisers at the temperature,
// [B, K]; given, the draft rows are read only at the rejected position.
hipError_t launch_accept_logits(const void* zt, const void* zd, bool bf16, int B, int K, int V, float temperature,
                                const float* draft_lse, const int32_t* tokens, const int32_t* lens,
                                const float* uniforms, int32_t* n_accepted, int32_t* next_token, void* workspace,
                                size_t workspace_bytes, hipStream_t stream);

// 0 when one workgroup per sequence is used regardless (short rows).
size_t accept_logits_workspace_bytes(int B, int K, int V);

// Fill `words` exchange slots with the empty marker, on `stream`.
hipError_t launch_fill_empty(unsigned long long* slots, int64_t words, hipStream_t stream);

hipError_t launch_warp(const void* logits, bool bf16, int B, int R, int V, const int32_t* lens, int extra_rows,
                       float temperature, float* probs, void* workspace, size_t workspace_bytes, hipStream_t stream);

hipError_t launch_warp_filtered(const void* logits, bool bf16, int B, int R, int V, const int32_t* lens,
                                int extra_rows, float temperature, const int32_t* top_k, const float* top_p,
                                float* probs, hipStream_t stream);

// The penalty stage: workspace bytes for B sequences with histories of up to
// `cap` tokens (hash tables of the committed histories), and the launcher
// (seq may be null: no committed history; tokens may be null: no draft prefix).
size_t penalty_workspace_bytes(int B, int cap);
hipError_t launch_penalties(const void* logits, bool bf16, int B, int R, int V, const int32_t* lens, int extra_rows,
                            const int32_t* seq, const int32_t* seq_len, int cap, const int32_t* tokens, int K,
                            const float* theta, const float* presence, const float* frequency, float* out,
                            void* workspace, hipStream_t stream);

// Draft-length gate parameters as the kernels take them (by value).
struct GateCosts {
    double draft_ms, verify_base_ms, verify_slope_ms, plain_ms, margin;
    int min_draft;
    double margin_threshold;
};

hipError_t launch_gate_update(double* hits, double* trials, int B, int NB, int K, const int32_t* lens,
                              const int32_t* n_accepted, const int32_t* buckets, double decay, hipStream_t stream);

hipError_t launch_gate_choose(const double* hits, const double* trials, int B, int NB, int K, const int32_t* buckets,
                              const float* top2_margin, const GateCosts& g, int32_t* next_lens, hipStream_t stream);

hipError_t launch_commit(int32_t* seq, int32_t* seq_len, int32_t* done, int B, int cap, const int32_t* tokens, int K,
                         const int32_t* n_accepted, const int32_t* next_token, const int32_t* limit, int eos,
                         hipStream_t stream);

// Workspace the cooperative warp path needs (0: that path does not apply to V).
size_t warp_workspace_bytes(int B, int R, int V);

// The device array that serves as the warp's workspace for callers that cannot
// allocate (SV_NOALLOC_SCRATCH_BYTES bytes), and its address on the current
// device (looked up once per device).
constexpr size_t kStaticScratchBytes = size_t(1) << 20;
hipError_t static_scratch(void** ptr);

// Polls a cooperative warp workgroup makes before it recomputes its row alone
// (applies to launches made after the call, on every device).
void set_wait_limit(int tries);
int get_wait_limit();

// Rows the split greedy verify reads ahead of its decision (applies to
// launches made after the call, on every device).
void set_greedy_lookahead(int rows);

}  // namespace sv
