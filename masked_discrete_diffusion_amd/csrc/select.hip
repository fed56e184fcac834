// Unmasking after a step (page 3, section 3.2): with a pre-generated order
// every decoded position is unmasked; in semi-autoregressive text decoding the
// most confident positions of the block are unmasked (ties: lower position)
// and the rest stay masked.  One block per sequence; the rank of a candidate
// is the number of candidates that beat it.
#include "common.hpp"
#include "kernels.hpp"

namespace mdm {

namespace {

constexpr int kMaxCand = 1024;

__global__ __launch_bounds__(1024) void k_select(Geometry g, SelectArgs a) {
  __shared__ float conf[kMaxCand];
  __shared__ int pos[kMaxCand];
  __shared__ int sel[kMaxCand];
  const int b = blockIdx.x;
  const int i = threadIdx.x;
  const int n = a.n_cand;
  int p = 0, tok = 0;
  if (i < n) {
    p = a.cand_pos[(int64_t)b * a.cand_stride + i];
    tok = a.token[(int64_t)b * n + i];
    pos[i] = p;
    conf[i] = a.conf ? a.conf[(int64_t)b * n + i] : 0.f;
  }
  __syncthreads();
  int out_idx = i;
  bool chosen = true;
  if (a.by_conf && i < n) {
    const float ci = conf[i];
    int rank = 0;
    for (int j = 0; j < n; ++j) {
      const float cj = conf[j];
      rank += (cj > ci || (cj == ci && pos[j] < p)) ? 1 : 0;
    }
    chosen = rank < a.n_select;
    sel[i] = chosen ? 1 : 0;
  }
  __syncthreads();
  if (i >= n) return;
  if (a.by_conf) {
    int before = 0;
    for (int j = 0; j < n; ++j) before += (sel[j] == (chosen ? 1 : 0) && pos[j] < p) ? 1 : 0;
    out_idx = before;
  }
  if (chosen) {
    a.out_tok[(int64_t)b * a.n_select + out_idx] = tok;
    a.out_pos[(int64_t)b * a.n_select + out_idx] = p;
    if (a.seq_tokens) {
      if (p >= 0 && p < g.seq_len) a.seq_tokens[(int64_t)b * g.seq_len + p] = tok;
      else flag_error(a.err, kErrPos);
    }
  } else if (a.rem_pos) {
    a.rem_pos[(int64_t)b * (n - a.n_select) + out_idx] = p;
  }
}

}  // namespace

hipError_t launch_select(const Geometry& g, const SelectArgs& a, hipStream_t s) {
  if (a.n_cand <= 0) return hipSuccess;
  const int threads = ((a.n_cand + 63) / 64) * 64;
  hipLaunchKernelGGL(k_select, dim3(g.B), dim3(threads), 0, s, g, a);
  return hipGetLastError();
}

}  // namespace mdm
