// commit.hip -- append one verify round's output to each sequence on the
// device: the accepted draft prefix t_0 .. t_{n-1} followed by next_token
// (spec-verify card, "Usage": keep draft_tokens[:n_accepted], append
// next_token), so a draft/verify loop keeps its token buffers in HBM and never
// copies them to the host between rounds.
//
// One wavefront per sequence; lane j handles committed tokens j and j + 64
// (at most n + 1 <= 65 of them).
// A sequence stops at its length limit (or the buffer's capacity) and, when
// eos >= 0, right after the first committed eos token; a finished sequence
// is never appended to again.
#include "common.hpp"
#include "launch.hpp"

namespace sv {
namespace {

__global__ __launch_bounds__(kWave) void commit_kernel(int32_t* __restrict__ seq, int32_t* __restrict__ seq_len,
                                                       int32_t* __restrict__ done, int cap,
                                                       const int32_t* __restrict__ tokens, int K,
                                                       const int32_t* __restrict__ n_accepted,
                                                       const int32_t* __restrict__ next_token,
                                                       const int32_t* __restrict__ limit, int eos) {
    const int b = blockIdx.x, j = threadIdx.x;
    if (done[b]) return;
    const int len0 = seq_len[b];
    const int len = len0 < 0 ? 0 : len0;  // a negative length (caller error) cannot index before the row
    int lim = limit ? limit[b] : cap;
    lim = lim > cap ? cap : lim;
    const int na = n_accepted[b];
    const int n = na < 0 ? 0 : (na > K ? K : na);
    // committed token j (0 <= j <= n <= 64): lane j holds j, lane 0 also holds 64
    const int nx = next_token[b];
    const int c0 = j < n ? tokens[(int64_t)b * K + j] : nx;
    const int c1 = j + kWave < n ? tokens[(int64_t)b * K + j + kWave] : nx;
    const uint64_t hit0 = __ballot(eos >= 0 && j <= n && c0 == eos);
    const uint64_t hit1 = __ballot(eos >= 0 && j + kWave <= n && c1 == eos);
    const int first = hit0 ? __builtin_ctzll(hit0) : (hit1 ? kWave + __builtin_ctzll(hit1) : -1);
    const int count_eos = first >= 0 ? first + 1 : n + 1;
    int room = lim - len;
    room = room < 0 ? 0 : room;
    const int count = count_eos < room ? count_eos : room;
    if (j < count) seq[(int64_t)b * cap + len + j] = c0;
    if (j + kWave < count) seq[(int64_t)b * cap + len + j + kWave] = c1;
    if (j == 0) {
        seq_len[b] = len + count;
        done[b] = (len + count >= lim) || (first >= 0 && count_eos <= room);
    }
}

}  // namespace

hipError_t launch_commit(int32_t* seq, int32_t* seq_len, int32_t* done, int B, int cap, const int32_t* tokens, int K,
                         const int32_t* n_accepted, const int32_t* next_token, const int32_t* limit, int eos,
                         hipStream_t stream) {
    hipLaunchKernelGGL(commit_kernel, dim3(B), dim3(kWave), 0, stream, seq, seq_len, done, cap, tokens, K, n_accepted,
                       next_token, limit, eos);
    return hipGetLastError();
}

}  // namespace sv
