// The forward pass over row chunks under a logits budget (GLM-5.3 KV/indexer
// cache article, SGLang logits budget: over the budget the query rows are cut
// into pieces, each scored and ranked on its own, and the pieces' results put
// together).  Rows are independent, so a chunk is an ordinary launch over
// rows [a, a + n) once query_start_loc is expressed in the chunk's rows.
#include "dsa_common.h"
#include "dsa_launch.h"

namespace dsa {

// out[i] = clamp(qsl[i] - a, 0, n), i = 0..R: requests that end before the
// chunk become empty at 0, those that start after it empty at n.
__global__ __launch_bounds__(256) void rebase_qsl_kernel(
    const int32_t* __restrict__ qsl, int R, int64_t a, int64_t n,
    int32_t* __restrict__ out) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i > R) return;
  const int64_t v = (int64_t)qsl[i] - a;
  out[i] = (int32_t)(v < 0 ? 0 : (v > n ? n : v));
}

hipError_t launch_forward_chunked(const ChunkedForwardArgs& c,
                                  hipStream_t stream) {
  const ForwardArgs& f = c.f;
  const int64_t T = f.lg.T;
  if (T <= 0) return hipSuccess;
  hipError_t e = launch_quantize_q(f.q_bf16, T * f.lg.H, f.q8, f.q_scale,
                                   stream);
  if (e != hipSuccess) return e;
  const LogitsPlan plan = logits_plan(T, f.lg.R);
  const int64_t H = f.lg.H;
  for (int64_t a = 0; a < T; a += c.rows) {
    const int64_t n = std::min<int64_t>(c.rows, T - a);
    hipLaunchKernelGGL(rebase_qsl_kernel, dim3((unsigned)((f.lg.R + 256) / 256)),
                       dim3(256), 0, stream, f.lg.qsl, f.lg.R, a, n,
                       c.qsl_chunk);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    LogitsArgs lg = f.lg;
    lg.q8 = f.lg.q8 + a * H * kHeadDim;
    lg.q_scale = f.lg.q_scale + a * H;
    lg.weights = f.lg.weights + a * H;
    lg.qsl = c.qsl_chunk;
    lg.positions = f.lg.positions + a;
    lg.T = n;
    if ((e = launch_logits(lg, stream, plan)) != hipSuccess) return e;
    TopkArgs tk = f.tk;
    tk.positions = f.tk.positions + a;
    tk.T = n;
    tk.out = f.tk.out + a * f.tk.out_ld;
    if ((e = launch_topk(tk, stream)) != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace dsa
