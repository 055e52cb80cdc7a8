// Captured forward passes: library calls recorded once into a HIP graph and
// replayed with one launch.
//
// "W4A4 CUDA Kernel for Voice Clone", section 4: per-kernel launch overhead
// dominates small decode-size calls, so the pages capture the forward step
// into a graph; since a graph bakes in its shapes, they pre-capture one graph
// per bucket of the packed length at start-up and, per request, pad to the
// nearest bucket, copy the data into the bucket's buffers and replay.
//
// w4a4_graph_begin / w4a4_graph_end capture whatever library calls the
// caller enqueues on a stream in between (a whole step of many layers, say);
// w4a4_layer_graph_create captures one layer (activation pass + GEMM) on a
// private stream.  None of the library's kernels uses a memset or an
// allocation, so a captured graph holds kernel nodes only.
#include <hip/hip_runtime.h>

#include <new>

#include "w4a4.h"

struct w4a4_graph {
  hipGraph_t graph = nullptr;
  hipGraphExec_t exec = nullptr;
};

namespace {

int hip_err(hipError_t e) { return e == hipSuccess ? W4A4_OK : W4A4_ERR_HIP; }

// End the capture on s and instantiate it; `pending` is an error that
// happened while capturing (the capture is ended and discarded then).
int finish_capture(hipStream_t s, int pending, w4a4_graph** out) {
  hipGraph_t graph = nullptr;
  const hipError_t e = hipStreamEndCapture(s, &graph);   // always ends the capture
  int st = pending != W4A4_OK ? pending : hip_err(e);
  hipGraphExec_t exec = nullptr;
  if (st == W4A4_OK) st = hip_err(hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0));
  w4a4_graph* g = st == W4A4_OK ? new (std::nothrow) w4a4_graph : nullptr;
  if (st == W4A4_OK && !g) st = W4A4_ERR_HIP;
  if (st != W4A4_OK) {
    if (exec) (void)hipGraphExecDestroy(exec);
    if (graph) (void)hipGraphDestroy(graph);
    return st;
  }
  g->graph = graph;
  g->exec = exec;
  *out = g;
  return W4A4_OK;
}

}  // namespace

extern "C" {

int w4a4_graph_begin(void* stream) {
  if (!stream) return W4A4_ERR_NULL;   // the legacy default stream cannot be captured
  return hip_err(hipStreamBeginCapture(reinterpret_cast<hipStream_t>(stream), hipStreamCaptureModeThreadLocal));
}

int w4a4_graph_end(void* stream, w4a4_graph** out) {
  if (!stream) return W4A4_ERR_NULL;
  if (!out) {   // still end the capture so that the stream is usable again
    hipGraph_t graph = nullptr;
    if (hipStreamEndCapture(reinterpret_cast<hipStream_t>(stream), &graph) == hipSuccess && graph)
      (void)hipGraphDestroy(graph);
    return W4A4_ERR_NULL;
  }
  *out = nullptr;
  return finish_capture(reinterpret_cast<hipStream_t>(stream), W4A4_OK, out);
}

int w4a4_layer_graph_create(int64_t M, int64_t N, int64_t K, int32_t R, const uint16_t* x,
                            int64_t ldx, const uint16_t* gamma, double eps, const void* wblob,
                            void* act, uint16_t* y, int64_t ldy, w4a4_graph** out) {
  if (!out) return W4A4_ERR_NULL;
  *out = nullptr;
  if (M <= 0) return W4A4_ERR_SHAPE;   // an empty bucket has nothing to capture
  int st = w4a4_query_variant(M, N, K, R);   // shape rules, checked before any capture
  if (st < 0) return -st;
  // The calls' own argument checks run inside the capture, before they
  // enqueue anything; an error ends the capture and is returned.  A private
  // stream (default priority) keeps the capture away from the caller's work.
  hipStream_t cs = nullptr;
  if (hipStreamCreateWithFlags(&cs, hipStreamNonBlocking) != hipSuccess) return W4A4_ERR_HIP;
  st = hip_err(hipStreamBeginCapture(cs, hipStreamCaptureModeThreadLocal));
  if (st == W4A4_OK) {
    int q = gamma ? w4a4_quantize_act_rmsnorm(M, K, R, x, ldx, gamma, eps, wblob, act, cs)
                  : w4a4_quantize_act(M, K, R, x, ldx, wblob, act, cs);
    int l = q == W4A4_OK ? w4a4_linear(M, N, K, R, act, wblob, y, ldy, cs) : W4A4_OK;
    st = finish_capture(cs, q != W4A4_OK ? q : l, out);
  }
  (void)hipStreamDestroy(cs);
  return st;
}

int w4a4_graph_launch(w4a4_graph* g, void* stream) {
  if (!g || !g->exec) return W4A4_ERR_NULL;
  return hip_err(hipGraphLaunch(g->exec, reinterpret_cast<hipStream_t>(stream)));
}

int w4a4_graph_destroy(w4a4_graph* g) {
  if (!g) return W4A4_OK;
  int st = W4A4_OK;
  if (g->exec && hipGraphExecDestroy(g->exec) != hipSuccess) st = W4A4_ERR_HIP;
  if (g->graph && hipGraphDestroy(g->graph) != hipSuccess) st = W4A4_ERR_HIP;
  delete g;
  return st;
}

}  // extern "C"
